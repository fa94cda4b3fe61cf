"""GPU parity at the edges of the supported shapes, against the fp64 oracle.

- ragged sizes: h, I and E not multiples of any tile or wave, a shared expert
  narrower than the routed ones;
- top-k at its extremes (k = 1, k = E), and the largest expert count and
  top-k (E = 1024, k = 32);
- the widest h and I (16384; 8192 with fp32 activations);
- routing without renormalisation;
- caller routing that drops slots or repeats an expert within a row;
- shared-expert route chunks with a ragged last chunk;
- calls in flight on two streams with their own workspaces;
- the largest steps: N = 1024, and the limit N = 4096, also with E = 1024
  and k = 32 at once.

Same tolerances as the workload tests: logits 1e-3 per row, indices exact
beyond a 1e-3 margin, weights 1e-5, outputs 2e-2 (fp32, bf16, FP8) or 5e-2
(MXFP4)."""
import sys

import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
from tests import harness as H

pytestmark = pytest.mark.gpu

OUT_TOL = {"f32": 2e-2, "bf16": 2e-2, "fp8_b128": 2e-2, "mxfp4": 5e-2}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _x_rows(li, n):
    """n token rows: the layer's own 256, then further seeded batches."""
    parts = [li.x]
    b = 0
    while sum(p.shape[0] for p in parts) < n:
        parts.append(ms.fresh_x(li, 500 + b))
        b += 1
    return torch.cat(parts, 0)[:n].contiguous()


def _check(dl, n, x):
    """Run the layer on n rows; compare logits, routing and every output row
    (near-tie rows where the GPU picked other experts at its own picks, with
    the oracle's weights of those picks)."""
    spec = dl.spec
    got = H.run_layer(dl, n, x=x)
    torch.cuda.synchronize()
    g = {k: v.float().cpu().numpy() for k, v in got.items()}
    lg = oracle.router_logits(spec, x[:n], dl.li.router)
    for t in range(n):
        e = H.rel_err(g["logits"][t], lg[t])
        assert e <= 1e-3, f"row {t}: logits rel err {e}"
    idx, w = oracle.topk(spec, lg, dl.li.bias)
    ref = {"logits": lg, "keys": oracle.keys(spec, lg, dl.li.bias), "idx": idx, "w": w}
    ties = H.check_routing(spec, ref, g["idx"].astype(np.int64), g["w"])
    idx_o, w_o, alt = H.outputs_routing(spec, ref, g["idx"], g["w"])
    out_ref = oracle.experts(dl.li, n, idx_o, w_o, x=x[:n])
    err = H.rel_err(g["out"], out_ref)
    _say(f"    N={n} rows={n} near_ties={len(ties)} other_picks={len(alt)} out_rel_err={err:.3e}")
    assert err <= OUT_TOL[spec.expert_dtype], err


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8_b128", "mxfp4"])
def test_ragged_shapes(fmt):
    """h 96, I 160, shared expert 96 wide, 13 experts, top-3: no dimension is a
    multiple of a tile, a wave or a scale block; N spans both router regimes."""
    _say(f"[ragged] {fmt}")
    act = "f32" if fmt == "f32" else "bf16"
    spec = ms.SPECS["qwen3_next"].with_(hidden=96, num_experts=13, top_k=3, inter=160,
                                        shared_inter=96, act_dtype=act, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=7, device="cuda")
    dl = H.device_layer(li, max_n=33)
    for n in (1, 3, 7, 33):
        _check(dl, n, li.x)


@pytest.mark.parametrize("k", [1, 8])
@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_topk_extremes(k, scoring):
    """k = 1 (every weight is routed_scaling) and k = E (every expert picked)."""
    _say(f"[k extremes] k={k} {scoring}")
    spec = ms.SPECS["qwen3_next"].with_(hidden=256, num_experts=8, top_k=k, inter=128,
                                        shared_inter=0, scoring=scoring, routed_scaling=1.5,
                                        corr_bias=scoring == "sigmoid")
    li = ms.make_layer(spec, seed=11, device="cuda")
    dl = H.device_layer(li, max_n=16)
    for n in (1, 4, 16):
        _check(dl, n, li.x)


def test_large_step():
    """N = 1024 rows: many router token tiles, compaction over several route
    tiles, experts with dozens of routes on the MFMA path."""
    _say("[large N]")
    spec = ms.SPECS["qwen3_30b_a3b"].with_(hidden=256, num_experts=64, top_k=8, inter=128)
    li = ms.make_layer(spec, seed=13, device="cuda")
    n = 1024
    x = _x_rows(li, n)
    dl = H.device_layer(li, max_n=n)
    _check(dl, n, x)


def test_largest_step():
    """N = 4096, the ABI's limit, on a small fp32 layer."""
    _say("[max N]")
    spec = ms.SPECS["tiny"].with_(hidden=64, num_experts=16, top_k=4, inter=64)
    li = ms.make_layer(spec, seed=17, device="cuda")
    n = 4096
    x = _x_rows(li, n)
    dl = H.device_layer(li, max_n=n)
    _check(dl, n, x)


@pytest.mark.parametrize("shared", [0, 96])
def test_dropped_routes(shared):
    """Caller routing with expert ids outside [0, E): such a route adds nothing,
    as a route of weight 0 would.  Some routes dropped, then every route
    dropped (the output is the shared expert alone, or zeros), at a size of
    each compaction form (one wave, one workgroup, every top-k workgroup at
    300 rows: 19 groups of 16 rows, the last ragged); the workspace is reused
    across the calls."""
    _say(f"[dropped routes] shared={shared}")
    spec = ms.SPECS["qwen3_next"].with_(hidden=96, num_experts=13, top_k=3, inter=160,
                                        shared_inter=shared, expert_dtype="bf16")
    li = ms.make_layer(spec, seed=19, device="cuda")
    li = ms.with_x(li, _x_rows(li, 300))
    dl = H.device_layer(li, max_n=300)
    rng = np.random.default_rng(5)
    for n, frac in ((33, 0.3), (3, 0.5), (300, 0.3), (33, 1.0), (300, 1.0), (3, 1.0), (7, 0.0),
                    (300, 0.0)):
        idx = np.stack([rng.permutation(spec.num_experts)[:spec.top_k] for _ in range(n)])
        w = rng.uniform(0.05, 1.0, size=(n, spec.top_k))
        drop = rng.uniform(size=idx.shape) < frac
        bad = np.where(rng.uniform(size=idx.shape) < 0.5, -1, spec.num_experts)
        got = H.run_experts(dl, n, np.where(drop, bad, idx), w.astype(np.float32))
        torch.cuda.synchronize()
        ref_idx = np.where(drop, 0, idx)
        ref_w = np.where(drop, 0.0, w.astype(np.float32).astype(np.float64))
        ref = oracle.experts(li, n, ref_idx, ref_w, x=li.x[:n])
        g = got.float().cpu().numpy()
        if shared == 0 and frac == 1.0:
            assert not g.any(), "every route dropped: the output must be zeros"
            continue
        err = H.rel_err(g, ref)
        _say(f"    N={n} dropped={int(drop.sum())} out_rel_err={err:.3e}")
        assert err <= OUT_TOL["bf16"], err


@pytest.mark.parametrize("n", [129, 300, 2000])
def test_concentrated_routes(n):
    """Caller routing at a step that compacts in every top-k workgroup: every
    row picks the same 3 of 13 experts in its own order, and one row in five
    repeats an expert in two slots (as a hash table row may), so each expert
    holds hundreds of routes spread over all 16-row groups."""
    _say(f"[concentrated routes] N={n}")
    spec = ms.SPECS["qwen3_next"].with_(hidden=96, num_experts=13, top_k=3, inter=160,
                                        shared_inter=64, expert_dtype="bf16")
    li = ms.make_layer(spec, seed=23, device="cuda")
    x = _x_rows(li, n)
    li = ms.with_x(li, x)
    dl = H.device_layer(li, max_n=n)
    rng = np.random.default_rng(7)
    idx = np.stack([rng.permutation([2, 7, 11]) for _ in range(n)])
    rep = rng.uniform(size=n) < 0.2
    idx[rep, 1] = idx[rep, 0]
    w = rng.uniform(0.05, 1.0, size=(n, spec.top_k)).astype(np.float32)
    got = H.run_experts(dl, n, idx, w)
    torch.cuda.synchronize()
    ref = oracle.experts(li, n, idx, w.astype(np.float64), x=li.x[:n])
    err = H.rel_err(got.float().cpu().numpy(), ref)
    _say(f"    out_rel_err={err:.3e}")
    assert err <= OUT_TOL["bf16"], err


@pytest.mark.parametrize("fmt,h,inter,sh", [("bf16", 2144, 512, 256), ("fp8_b128", 2176, 512, 256),
                                            ("mxfp4", 2144, 512, 512)])
def test_many_tiles_beside_mfma(fmt, h, inter, sh):
    """128 experts, top-8, 64 rows: a down pass of 34 64-row tiles per expert
    in the kernel that mixes the MFMA and VALU paths; h is not a multiple of
    the tile (bf16, MXFP4), so every expert ends in a partial tile."""
    _say(f"[many tiles] {fmt} h={h}")
    spec = ms.SPECS["qwen3_30b_a3b"].with_(hidden=h, num_experts=128, top_k=8, inter=inter,
                                           shared_inter=sh, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=23, device="cuda")
    n = 64
    x = _x_rows(li, n)
    dl = H.device_layer(li, max_n=n)
    _check(dl, n, x)


@pytest.mark.parametrize("fmt,h,inter", [("bf16", 512, 512), ("fp8_b128", 512, 512),
                                         ("mxfp4", 512, 512), ("fp8_b128", 640, 512),
                                         ("mxfp4", 704, 512), ("bf16", 96, 512),
                                         ("bf16", 512, 384), ("fp8_b128", 512, 384),
                                         ("mxfp4", 512, 384)])
def test_grouped_gemm_steps(fmt, h, inter):
    """512 rows over 64 experts, top-8: experts average 64 routes, so every
    expert takes route groups of 64 (the grouped-GEMM form of the MFMA path);
    route counts straddle 64, so groups come full, partial and more than one
    per expert, and the shared expert has 8 groups.  The form's items are 256
    gate+up rows and 512 down rows (two or four 128-row tiles): h = 640 ends
    the down matrices in an item of one 128-row FP8 scale block, 704 and 96
    in items of partial 128-row tiles; inter = 384 ends gate+up in an item of
    one 128-row tile (the FP8 item's second scale block past the matrix), and
    MXFP4 then takes its down pass beside the MFMA path no longer (K = 384)."""
    _say(f"[grouped gemm] {fmt} h={h} inter={inter}")
    spec = ms.SPECS["qwen3_next"].with_(hidden=h, num_experts=64, top_k=8, inter=inter,
                                        shared_inter=512, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=31, device="cuda")
    n = 512
    x = _x_rows(li, n)
    dl = H.device_layer(li, max_n=n)
    _check(dl, n, x)


def test_grouped_gemm_verify_shape():
    """The MXFP4 verify layer at 1024 rows: 32 routes per expert on average."""
    _say("[grouped gemm] verify_mxfp4 N=1024")
    li = ms.make_layer("verify_mxfp4", seed=0, device="cuda")
    n = 1024
    x = _x_rows(li, n)
    dl = H.device_layer(li, max_n=n)
    _check(dl, n, x)


@pytest.mark.parametrize("fmt,n", [("bf16", 100), ("fp8_b128", 100), ("mxfp4", 100),
                                   ("fp8_b128", 600), ("mxfp4", 600)])
def test_shared_expert_route_chunks(fmt, n):
    """Beside the MFMA path the shared expert's rows come in chunks of one
    route group, each its own item: 16 routes (N = 100, a last chunk of 4),
    or 64 in the grouped-GEMM form (N = 600, a last chunk of 24)."""
    _say(f"[shared chunks] {fmt} N={n}")
    spec = ms.SPECS["qwen3_next"].with_(hidden=512, num_experts=64, top_k=8, inter=512,
                                        shared_inter=512, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=37, device="cuda")
    x = _x_rows(li, n)
    dl = H.device_layer(li, max_n=n)
    _check(dl, n, x)


@pytest.mark.parametrize("fmt", ["bf16", "fp8_b128", "mxfp4"])
def test_largest_expert_count_and_top_k(fmt):
    """E = 1024 experts and k = 32, the largest the library takes, with a
    shared expert: one row holds 33 slots in the one-row down + blend; two rows
    make 64 routes, the most the one-wave compaction takes; three rows go
    to the workgroup compaction; five rows to the MFMA router and its top-k
    kernel, all at the widest top-k (16 keys per lane)."""
    _say(f"[E=1024, k=32] {fmt}")
    spec = ms.SPECS["qwen3_next"].with_(hidden=256, num_experts=1024, top_k=32, inter=128,
                                        shared_inter=128, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=41, device="cuda")
    dl = H.device_layer(li, max_n=5)
    for n in (1, 2, 3, 5):
        _check(dl, n, li.x)


# (format, h, I = shared I, rows): the widest shapes the library takes
WIDE = [
    ("bf16", 16384, 128, (1, 4, 6)),     # router: 8 chunks per lane (VALU), MFMA router above 4
    ("mxfp4", 16384, 512, (1, 6)),       # gate+up over K = 16384 in 512-column segments
    ("fp8_b128", 256, 16384, (1, 4, 20)),  # down pass over K = 16384, MFMA at 20 rows
    ("f32", 8192, 64, (1, 4, 6)),        # fp32 activations at their widest h
]


@pytest.mark.parametrize("fmt,h,inter,ns", WIDE)
def test_widest_shapes(fmt, h, inter, ns):
    _say(f"[wide] {fmt} h={h} I={inter}")
    act = "f32" if fmt == "f32" else "bf16"
    spec = ms.SPECS["qwen3_next"].with_(hidden=h, num_experts=8, top_k=2, inter=inter,
                                        shared_inter=0 if fmt == "f32" else inter,
                                        act_dtype=act, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=43, device="cuda")
    dl = H.device_layer(li, max_n=max(ns))
    for n in ns:
        _check(dl, n, li.x)


@pytest.mark.parametrize("scoring,rsf", [("softmax", 1.0), ("sigmoid", 2.5)])
@pytest.mark.parametrize("E", [64, 300])
def test_routing_without_renormalisation(scoring, rsf, E):
    """norm_topk off: softmax weights keep the denominator over all E experts
    (E = 300 leaves 5 keys on some lanes and 4 on others), sigmoid weights
    stay σ(logit); both times rsf.  N = 1 and 4 take the router with the fused
    top-k, N = 16 the top-k kernel."""
    _say(f"[no renorm] {scoring} E={E}")
    spec = ms.SPECS["qwen3_next"].with_(hidden=256, num_experts=E, top_k=6, inter=128,
                                        shared_inter=0, scoring=scoring, norm_topk=False,
                                        routed_scaling=rsf, corr_bias=scoring == "sigmoid")
    li = ms.make_layer(spec, seed=47, device="cuda")
    dl = H.device_layer(li, max_n=16)
    for n in (1, 4, 16):
        _check(dl, n, li.x)


def test_two_streams_with_their_own_workspaces():
    """Calls in flight at once on two streams, each with its own workspace,
    give the bits each gives alone: a four-row step (the router with the fused
    top-k, VALU experts) beside a 64-row one (MFMA router, top-k kernel, MFMA
    experts and a shared expert), launched alternately so their kernels overlap."""
    _say("[two streams]")
    spec = ms.SPECS["qwen3_next"].with_(hidden=512, num_experts=64, top_k=8, inter=512,
                                        shared_inter=512)
    li = ms.make_layer(spec, seed=53, device="cuda")
    xa = li.x[:4].contiguous()
    xb = _x_rows(li, 64)
    da, db = H.device_layer(li, max_n=64), H.device_layer(li, max_n=64)
    ref_a, ref_b = H.run_layer(da, 4, x=xa), H.run_layer(db, 64, x=xb)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        outs = []
        for _ in range(4):
            with torch.cuda.stream(sb):
                ob = H.run_layer(db, 64, x=xb, stream=sb)
            with torch.cuda.stream(sa):
                oa = H.run_layer(da, 4, x=xa, stream=sa)
            outs.append((oa, ob))
        torch.cuda.synchronize()
        for oa, ob in outs:
            for key in ref_a:
                assert torch.equal(oa[key], ref_a[key]), ("4 rows", key)
                assert torch.equal(ob[key], ref_b[key]), ("64 rows", key)


@pytest.mark.parametrize("fmt", ["bf16", "fp8_b128", "mxfp4"])
def test_caller_routing_with_repeats(fmt):
    """Caller routing that names an expert more than once in a row (ids drawn
    with replacement) and drops some slots: every repeat is a route of its
    own.  N = 3 (VALU experts), 48 (MFMA beside the VALU path) and 600 (the
    grouped-GEMM form), with a shared expert; every row against the oracle."""
    _say(f"[repeats] {fmt}")
    spec = ms.SPECS["qwen3_next"].with_(hidden=512, num_experts=16, top_k=6, inter=512,
                                        shared_inter=512, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=59, device="cuda")
    dl = H.device_layer(li, max_n=600)
    x = _x_rows(li, 600)
    rng = np.random.default_rng(61)
    for n in (3, 48, 600):
        idx = rng.integers(0, spec.num_experts, size=(n, spec.top_k))
        assert any(len(set(r)) < spec.top_k for r in idx.tolist()), "no row repeats an expert"
        w = rng.uniform(0.05, 1.0, size=(n, spec.top_k)).astype(np.float32)
        drop = rng.uniform(size=idx.shape) < 0.1
        got = H.run_experts(dl, n, np.where(drop, -1, idx), w, x=x)
        torch.cuda.synchronize()
        ref = oracle.experts(li, n, np.where(drop, 0, idx),
                             np.where(drop, 0.0, w.astype(np.float64)), x=x[:n])
        err = H.rel_err(got.float().cpu().numpy(), ref)
        _say(f"    N={n} rows={n} out_rel_err={err:.3e}")
        assert err <= OUT_TOL[fmt], err


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_largest_step_with_the_most_routes(fmt):
    """Every limit at once: N = 4096 rows, E = 1024 experts, k = 32, so 131,072
    routes through the workgroup compaction and the grouped-GEMM form (about
    128 routes per expert), with a shared expert; routing and output of every
    row checked."""
    _say(f"[max N, E, k] {fmt}")
    spec = ms.SPECS["qwen3_next"].with_(hidden=512, num_experts=1024, top_k=32, inter=512,
                                        shared_inter=512, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=67, device="cuda")
    n = 4096
    x = _x_rows(li, n)
    dl = H.device_layer(li, max_n=n)
    _check(dl, n, x)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8_b128", "mxfp4"])
def test_zero_experts(fmt):
    """A router 12 + 4 wide: 12 real experts and 4 zero-computation experts,
    top-5, with a shared expert (fp32: without).  The layer under its own
    routing at N = 1 (the one-row down + blend, the general compaction), 3
    (VALU router and experts) and 20 (MFMA router, experts beside the MFMA
    path); then caller routing through moe_experts_forward that repeats ids,
    picks zero experts and drops ids outside [0, E + Z)."""
    _say(f"[zero experts] {fmt}")
    act = "f32" if fmt == "f32" else "bf16"
    spec = ms.SPECS["qwen3_next"].with_(hidden=512, num_experts=12, zero_experts=4, top_k=5,
                                        inter=512, shared_inter=0 if fmt == "f32" else 512,
                                        act_dtype=act, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=71, device="cuda")
    dl = H.device_layer(li, max_n=48)
    x = _x_rows(li, 48)
    for n in (1, 3, 20):
        _check(dl, n, x)
    rng = np.random.default_rng(73)
    for n in (1, 4, 48):
        idx = rng.integers(0, 16, size=(n, 5))
        idx[0, :2] = [13, 12]  # zero experts in the first row whatever the draw
        drop = rng.uniform(size=idx.shape) < 0.1
        drop[0] = False
        w = rng.uniform(0.05, 1.0, size=(n, 5)).astype(np.float32)
        got = H.run_experts(dl, n, np.where(drop, 99, idx), w, x=x)
        torch.cuda.synchronize()
        ref = oracle.experts(li, n, np.where(drop, 0, idx),
                             np.where(drop, 0.0, w.astype(np.float64)), x=x[:n])
        err = H.rel_err(got.float().cpu().numpy(), ref)
        _say(f"    caller routing N={n} zero picks={int((idx >= 12).sum())} out_rel_err={err:.3e}")
        assert err <= OUT_TOL[fmt], err
