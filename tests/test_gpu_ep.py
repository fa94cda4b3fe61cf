"""The expert-parallel split of the layer (design for several GPUs), checked on
one GPU: S ranks each hold E/S experts and route every row with the same
router; each computes only its own routes (routes to other ranks' experts
are dropped: their ids fall outside the rank's [0, E/S)), without the shared
expert; the shared expert is added once.  The sum of the S partial outputs and
the shared-only output must match the whole layer from the fp64 oracle, to the
output tolerance.  This is the kernel half of the forward pass the pages
shard by experts, with an all-reduce of the partial [N, h] outputs between
the ranks (the summation here stands in for it)."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import mixture_experts_decode_wave_amd as mw
import moe_synth as ms
import oracle
from tests import harness as H

pytestmark = pytest.mark.gpu

OUT_TOL = {"bf16": 2e-2, "fp8_b128": 2e-2, "mxfp4": 5e-2}


@pytest.mark.parametrize("fmt", ["bf16", "fp8_b128", "mxfp4"])
@pytest.mark.parametrize("ranks", [2, 8])
def test_expert_parallel_partials(fmt, ranks):
    print(f"[ep partials] {fmt} ranks={ranks}", flush=True)
    spec = ms.SPECS["qwen3_next"].with_(hidden=1024, num_experts=64, top_k=8, inter=512,
                                        shared_inter=512, expert_dtype=fmt)
    li = ms.make_layer(spec, seed=29, device="cuda")
    n = 16
    x = li.x[:n].contiguous()
    ref = oracle.layer_forward(li, n)
    idx = ref["idx"].astype(np.int32)
    w = ref["w"].astype(np.float32)
    E, El = spec.num_experts, spec.num_experts // ranks
    total = torch.zeros(n, spec.hidden, dtype=torch.float32, device="cuda")
    g, u, d = li.gate, li.up, li.down
    sl = lambda t, e0: None if t is None else t[e0:e0 + El]
    for r in range(ranks):
        e0 = r * El
        cfg_r = H.cfg_of(spec.with_(num_experts=El, shared_inter=0))
        tables_r = mw.ExpertTables.from_stacked(sl(g.w, e0), sl(u.w, e0), sl(d.w, e0),
                                                sl(g.s, e0), sl(u.s, e0), sl(d.s, e0))
        ws_r = mw.alloc_workspace(cfg_r, n, "cuda")
        idx_r = np.where((idx >= e0) & (idx < e0 + El), idx - e0, -1).astype(np.int32)
        out_r = torch.empty(n, spec.hidden, dtype=x.dtype, device="cuda")
        mw.moe_experts_forward(cfg_r, x, tables_r, None,
                               torch.as_tensor(idx_r, device="cuda"),
                               torch.as_tensor(w, device="cuda"), out_r, ws_r)
        total += out_r.float()
    # the shared expert, once: every routed id dropped
    dl = H.device_layer(li, max_n=n)
    sh_out = H.run_experts(dl, n, np.full_like(idx, -1), w)
    total += sh_out.float()
    torch.cuda.synchronize()
    err = H.rel_err(total.cpu().numpy(), ref["out"])
    print(f"    sum of {ranks} partials + shared: out_rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL[fmt], err


def _rank_tables(li, e0, El):
    g, u, d = li.gate, li.up, li.down
    sl = lambda t: None if t is None else t[e0:e0 + El]
    return mw.ExpertTables.from_stacked(sl(g.w), sl(u.w), sl(d.w), sl(g.s), sl(u.s), sl(d.s))


@pytest.mark.parametrize("fmt,gated", [("bf16", False), ("fp8_b128", True), ("mxfp4", False)])
@pytest.mark.parametrize("ranks", [2, 8])
def test_partials_then_shared_combine(fmt, gated, ranks):
    """The library's own expert-parallel calls: each rank's fp32 partial
    (moe_experts_forward_partial, shared expert left out), their sum in rank
    order (standing in for the all-reduce), then the shared expert once, gated
    or not, with one rounding (moe_shared_combine)."""
    print(f"[ep combine] {fmt} gated={gated} ranks={ranks}", flush=True)
    spec = ms.SPECS["qwen3_next"].with_(hidden=1024, num_experts=64, top_k=8, inter=512,
                                        shared_inter=512, expert_dtype=fmt, shared_gate=gated)
    li = ms.make_layer(spec, seed=31, device="cuda")
    El = spec.num_experts // ranks
    cfg_r = H.cfg_of(spec.with_(num_experts=El))  # its shared expert is left out
    ws_r = [mw.alloc_workspace(cfg_r, 16, "cuda") for _ in range(ranks)]
    tables_r = [_rank_tables(li, r * El, El) for r in range(ranks)]
    dl = H.device_layer(li, max_n=16)
    routed_only = dataclasses.replace(li, spec=spec.with_(shared_inter=0), sh_gate=None,
                                      sh_up=None, sh_down=None, sgate=None)
    for n in (1, 16):  # one row: the partial and the combine take the two-kernel form
        x = li.x[:n].contiguous()
        ref = oracle.layer_forward(li, n)
        idx = ref["idx"].astype(np.int32)
        w_dev = torch.as_tensor(ref["w"].astype(np.float32), device="cuda")
        total = torch.zeros(n, spec.hidden, dtype=torch.float32, device="cuda")
        keep, parts = [], []
        for r in range(ranks):
            e0 = r * El
            idx_r = torch.as_tensor(np.where((idx >= e0) & (idx < e0 + El), idx - e0, -1)
                                    .astype(np.int32), device="cuda")
            part = torch.empty(n, spec.hidden, dtype=torch.float32, device="cuda")
            mw.moe_experts_forward_partial(cfg_r, x, tables_r[r], idx_r, w_dev, part, ws_r[r])
            keep.append(idx_r)
            parts.append(part)
            total += part
        out = torch.empty(n, spec.hidden, dtype=x.dtype, device="cuda")
        mw.moe_shared_combine(dl.cfg, x, dl.shared, total, out, dl.ws)
        torch.cuda.synchronize()
        # every partial on its own: the oracle's sum over that rank's routes
        # (a rank without routes gives zeros)
        for r, part in enumerate(parts):
            local = (idx >= r * El) & (idx < (r + 1) * El)
            ref_p = oracle.experts(routed_only, n, np.where(local, idx, 0),
                                   np.where(local, ref["w"], 0.0), x=x)
            err_p = H.rel_err(part.cpu().numpy(), ref_p)
            assert err_p <= OUT_TOL[fmt], (n, r, err_p)
        err = H.rel_err(out.float().cpu().numpy(), ref["out"])
        print(f"    N={n} out_rel_err={err:.3e}", flush=True)
        assert err <= OUT_TOL[fmt], err


@pytest.mark.parametrize("fmt,shared,gated", [("bf16", 512, False), ("fp8_b128", 512, True),
                                              ("mxfp4", 0, False)])
def test_one_rank_partial_and_combine_is_experts_forward(fmt, shared, gated):
    """One rank holding every expert: the fp32 partial then the combine give
    the bits of moe_experts_forward under the same routing (2 rows, 16 and
    48: VALU and MFMA forms), with a shared expert (gated or not) or none."""
    print(f"[ep one rank] {fmt} shared={shared} gated={gated}", flush=True)
    spec = ms.SPECS["qwen3_next"].with_(hidden=512, num_experts=16, top_k=4, inter=512,
                                        shared_inter=shared, expert_dtype=fmt,
                                        shared_gate=gated and shared > 0)
    li = ms.make_layer(spec, seed=37, device="cuda")
    dl = H.device_layer(li, max_n=48)
    for n in (2, 16, 48):
        x = li.x[:n].contiguous()
        routed = H.run_route(dl, n, x=x)
        whole = H.run_experts(dl, n, routed["idx"], routed["w"], x=x)
        part = torch.empty(n, spec.hidden, dtype=torch.float32, device="cuda")
        mw.moe_experts_forward_partial(dl.cfg, x, dl.tables, routed["idx"], routed["w"], part,
                                       dl.ws)
        out = torch.empty_like(whole)
        mw.moe_shared_combine(dl.cfg, x, dl.shared, part, out, dl.ws)
        torch.cuda.synchronize()
        assert torch.equal(out, whole), n


def test_partial_and_combine_replay_from_a_graph():
    """The two calls captured into one HIP graph replay bit-identical to
    eager, with other eager work between the replays."""
    print("[ep graph]", flush=True)
    spec = ms.SPECS["qwen3_next"].with_(hidden=512, num_experts=16, top_k=4, inter=512,
                                        shared_inter=512, expert_dtype="fp8_b128",
                                        shared_gate=True)
    li = ms.make_layer(spec, seed=43, device="cuda")
    dl = H.device_layer(li, max_n=32)
    n = 32
    x = li.x[:n].contiguous()
    routed = H.run_route(dl, n, x=x)
    idx, w = routed["idx"].clone(), routed["w"].clone()
    part = torch.empty(n, spec.hidden, dtype=torch.float32, device="cuda")
    out = torch.empty(n, spec.hidden, dtype=x.dtype, device="cuda")

    def step(stream=None):
        mw.moe_experts_forward_partial(dl.cfg, x, dl.tables, idx, w, part, dl.ws, stream=stream)
        mw.moe_shared_combine(dl.cfg, x, dl.shared, part, out, dl.ws, stream=stream)

    step()
    torch.cuda.synchronize()
    ref_part, ref_out = part.clone(), out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(stream=s)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(stream=torch.cuda.current_stream())
    for _ in range(3):
        part.zero_()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(part, ref_part)
        assert torch.equal(out, ref_out)
        H.run_layer(dl, n, x=x.flip(0).contiguous())  # other eager work on the same workspace
        torch.cuda.synchronize()


def test_combine_after_a_pre_expert_norm():
    """With a pre-expert RMSNorm the experts read the normed rows and the
    shared-expert gate the layer's own input: the partial and the combine take
    the normed rows as x and the input as gate_x, and give the layer with that
    norm from the oracle (routing on the input itself).  A gate read from the
    normed rows instead is 0.078 off at 16 rows by the oracle's own account,
    well outside the tolerance."""
    print("[ep pre-norm]", flush=True)
    spec = ms.SPECS["qwen3_next"].with_(hidden=1024, num_experts=32, top_k=6, inter=512,
                                        shared_inter=512, expert_dtype="fp8_b128",
                                        shared_gate=True)
    li = ms.make_layer(spec, seed=71, device="cuda")
    _, ew = ms.make_norms(spec, 0, "cuda")
    eps = ms.NORM_EPS
    dl = H.device_layer(li, max_n=16)
    for n in (1, 16):
        x = li.x[:n].contiguous()
        ref = oracle.layer_forward(li, n, norms=(None, ew, eps))
        xe = oracle.rms_norm(spec, x, ew, eps).to("cuda").contiguous()
        idx = torch.as_tensor(ref["idx"].astype(np.int32), device="cuda")
        w = torch.as_tensor(ref["w"].astype(np.float32), device="cuda")
        part = torch.empty(n, spec.hidden, dtype=torch.float32, device="cuda")
        mw.moe_experts_forward_partial(dl.cfg, xe, dl.tables, idx, w, part, dl.ws)
        out = torch.empty(n, spec.hidden, dtype=x.dtype, device="cuda")
        mw.moe_shared_combine(dl.cfg, xe, dl.shared, part, out, dl.ws, gate_x=x)
        torch.cuda.synchronize()
        err = H.rel_err(out.float().cpu().numpy(), ref["out"])
        print(f"    N={n} out_rel_err={err:.3e}", flush=True)
        assert err <= OUT_TOL["fp8_b128"], err
