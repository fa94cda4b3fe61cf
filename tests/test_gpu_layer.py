"""GPU parity of libmoewave.so against the fp64 oracle, through the C ABI.

Tolerances (per workload): router logits max|d|/max|ref| <= 1e-3 per row;
routing indices exact where the oracle's k-th / (k+1)-th key margin exceeds
1e-3 (near ties: any valid pick); weights within 1e-5 relative; outputs
max|err|/max|ref| <= 2e-2 (fp32, bf16, FP8 experts) or 5e-2 (MXFP4)."""
import sys

import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
from tests import harness as H
from tests.constructed import identity_layer

pytestmark = pytest.mark.gpu

OUT_TOL = {"f32": 2e-2, "bf16": 2e-2, "fp8_b128": 2e-2, "mxfp4": 5e-2}
WORKLOADS = [(name, n) for name, spec in ms.SPECS.items() for n in spec.ns]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_LAYERS = {}
_ORACLE = {}


def _layer(name):
    if name not in _LAYERS:
        _say(f"[gen] {name}")
        li = ms.make_layer(name, seed=0, device="cuda")
        _LAYERS[name] = H.device_layer(li, max_n=256)
        torch.cuda.synchronize()
    return _LAYERS[name]


@pytest.fixture(scope="module", autouse=True)
def _free_layers():
    yield
    _LAYERS.clear()
    _ORACLE.clear()
    torch.cuda.empty_cache()


def _oracle_route(dl, n):
    li = dl.li
    lg = oracle.router_logits(li.spec, li.x[:n], li.router)
    idx, w = oracle.topk(li.spec, lg, li.bias)
    return {"logits": lg, "keys": oracle.keys(li.spec, lg, li.bias), "idx": idx, "w": w}


def _oracle(dl, n):
    """The oracle's routing of the first n rows and its output [n, h] for
    every row under that routing (computed once per workload and N)."""
    key = (dl.spec.name, n)
    if key not in _ORACLE:
        ref = _oracle_route(dl, n)
        _say(f"    oracle: {n} rows")
        out = oracle.experts(dl.li, n, ref["idx"], ref["w"], x=dl.li.x[:n])
        _ORACLE[key] = (ref, out)
    return _ORACLE[key]


def _check_logits(got, ref):
    for t in range(ref.shape[0]):
        e = H.rel_err(got[t], ref[t])
        assert e <= 1e-3, f"row {t}: logits rel err {e}"


@pytest.mark.parametrize("name,n", WORKLOADS)
def test_layer_matches_oracle(name, n):
    """The whole [N, h] output, every row: under the oracle's routing where
    the GPU picked the same experts, and at the GPU's own picks (weighted by
    the oracle) on near-tie rows where it picked others."""
    _say(f"[layer] {name} N={n}")
    dl = _layer(name)
    spec = dl.spec
    got = H.run_layer(dl, n)
    torch.cuda.synchronize()
    g = {k: v.float().cpu().numpy() for k, v in got.items()}
    ref, out_ref = _oracle(dl, n)
    _check_logits(g["logits"], ref["logits"])
    ties = H.check_routing(spec, ref, g["idx"].astype(np.int64), g["w"])
    idx_o, w_o, alt = H.outputs_routing(spec, ref, g["idx"], g["w"])
    if alt:
        out_ref = out_ref.copy()
        out_ref[alt] = oracle.experts(dl.li, len(alt), idx_o[alt], w_o[alt],
                                      x=dl.li.x[:n][torch.tensor(alt, device=dl.li.x.device)])
    err = H.rel_err(g["out"], out_ref)
    worst = int(np.argmax(np.max(np.abs(g["out"] - out_ref), axis=1)))
    _say(f"    rows={n} near_ties={len(ties)} other_picks={len(alt)} out_rel_err={err:.3e} "
         f"(worst row {worst})")
    assert err <= OUT_TOL[spec.expert_dtype], err


@pytest.mark.parametrize("name,n", WORKLOADS)
def test_experts_with_oracle_routing(name, n):
    """moe_experts_forward under the oracle's own routing, every row."""
    _say(f"[experts] {name} N={n}")
    dl = _layer(name)
    spec = dl.spec
    ref, out_ref = _oracle(dl, n)
    out = H.run_experts(dl, n, ref["idx"], ref["w"].astype(np.float32))
    torch.cuda.synchronize()
    err = H.rel_err(out.float().cpu().numpy(), out_ref)
    _say(f"    rows={n} out_rel_err={err:.3e}")
    assert err <= OUT_TOL[spec.expert_dtype], err


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8_b128", "mxfp4"])
@pytest.mark.parametrize("scoring,rsf,shared", [("softmax", 1.0, False), ("sigmoid", 2.5, True)])
def test_identity_experts_reproduce_input(fmt, scoring, rsf, shared):
    _say(f"[identity] {fmt} {scoring}")
    act = "f32" if fmt == "f32" else "bf16"
    li = identity_layer(fmt, h=128, E=8, k=3, scoring=scoring, rsf=rsf, shared=shared, act=act,
                        device="cuda")
    dl = H.device_layer(li, max_n=16)
    for n in (1, 5, 16):
        got = H.run_layer(dl, n)
        torch.cuda.synchronize()
        x = li.x[:n].double().cpu().numpy()
        want = (rsf + (1.0 if shared else 0.0)) * x
        err = H.rel_err(got["out"].double().cpu().numpy(), want)
        assert err <= 1e-2, (n, err)


@pytest.mark.parametrize("fmt", ["bf16", "fp8_b128", "mxfp4"])
def test_identity_experts_on_the_mfma_path(fmt):
    """Steps of more than 4 rows with K a multiple of 512 take the MFMA path
    for every expert of two or more routes (MXFP4 also stages its scales)."""
    _say(f"[identity mfma] {fmt}")
    li = identity_layer(fmt, h=512, E=8, k=3, scoring="sigmoid", rsf=2.5, shared=True,
                        device="cuda")
    dl = H.device_layer(li, max_n=48)
    for n in (6, 48):
        got = H.run_layer(dl, n)
        torch.cuda.synchronize()
        want = 3.5 * li.x[:n].double().cpu().numpy()
        err = H.rel_err(got["out"].double().cpu().numpy(), want)
        assert err <= 1e-2, (n, err)


def test_shared_expert_sigmoid_gate():
    li = identity_layer("fp8_b128", h=128, E=8, k=2, shared=True, zero_routed_down=True,
                        sgate=True, device="cuda")
    dl = H.device_layer(li, max_n=8)
    got = H.run_layer(dl, 8)
    torch.cuda.synchronize()
    x = li.x[:8].double().cpu().numpy()
    g = 1.0 / (1.0 + np.exp(-(x @ li.sgate.double().cpu().numpy())))
    assert H.rel_err(got["out"].double().cpu().numpy(), g[:, None] * x) <= 1e-2


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_equal_logits_pick_lowest_ids(scoring):
    spec = ms.SPECS["qwen3_next"].with_(hidden=256, num_experts=64, top_k=6, inter=128,
                                        shared_inter=0, scoring=scoring,
                                        corr_bias=scoring == "sigmoid")
    li = ms.make_layer(spec, seed=3, device="cuda")
    li.router[:] = li.router[0:1].clone()   # every expert row equal -> equal logits
    if li.bias is not None:
        li.bias.zero_()
    dl = H.device_layer(li, max_n=8)
    got = H.run_route(dl, 8)
    torch.cuda.synchronize()
    idx = got["idx"].cpu().numpy()
    w = got["w"].cpu().numpy()
    assert (idx == np.arange(6)[None, :]).all(), idx
    assert np.allclose(w, 1 / 6, rtol=1e-6)


def test_runs_are_bitwise_reproducible_and_batch_invariant():
    """Same inputs -> same bits.  A row's logits and routing do not depend on
    the other rows while N stays within one router regime (N <= 4: VALU GEMV
    router; N > 4: K-split MFMA router); for N <= 4 its output does not
    either (every expert product on the VALU path).  Above 4 rows an expert
    of two or more routes runs on MFMA, so output bits may depend on which
    other rows share a row's experts.  Across regimes rows agree to rounding."""
    dl = _layer("qwen3_next")
    a = H.run_layer(dl, 16)
    b = H.run_layer(dl, 16)
    four = H.run_layer(dl, 4)
    eight = H.run_layer(dl, 8)
    one = [H.run_layer(dl, 1, x=dl.li.x[t:t + 1]) for t in (0, 2, 3)]
    torch.cuda.synchronize()
    for key in ("out", "logits", "idx", "w"):
        assert torch.equal(a[key], b[key]), key
    for r, t in zip(one, (0, 2, 3)):
        for key in ("out", "logits", "idx", "w"):
            assert torch.equal(r[key][0], four[key][t]), (key, t)
    for key in ("logits", "idx", "w"):
        assert torch.equal(eight[key], a[key][:8]), key
    assert H.rel_err(a["logits"][:4].cpu().numpy(), four["logits"].cpu().numpy()) < 1e-5
    assert H.rel_err(a["out"][:4].float().cpu().numpy(), four["out"].float().cpu().numpy()) < 1e-2


@pytest.mark.parametrize("name,n", [("qwen3_30b_a3b", 4), ("qwen3_next_gated", 1),
                                    ("verify_mxfp4", 256)])
def test_graph_capture_replays_match_eager(name, n):
    """A captured step replays bit-identical to eager, with other eager work
    between the replays: the VALU path (N = 4), the one-row down + blend with a
    gated shared expert (N = 1), the MFMA path with chained MXFP4 loads."""
    _say(f"[graph] {name} N={n}")
    dl = _layer(name)
    x = dl.li.x[:n].clone()
    eager = H.run_layer(dl, n, x=x)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        H.run_layer(dl, n, x=x, stream=s)   # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = H.run_layer(dl, n, x=x, stream=torch.cuda.current_stream())
    for _ in range(3):
        for v in got.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), k
        H.run_layer(dl, n, x=dl.li.x[:n].flip(0).contiguous())  # other eager work between replays
        torch.cuda.synchronize()
