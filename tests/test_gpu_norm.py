"""moe_layer_forward_norm against the fp64 oracle: the layer with its router
pre-norm and its pre-expert norm (forward.rs: the router input and the
pre_expert_norm step), each alone and both together, the shared-expert gate
on the layer's own input.  Tolerances as for the plain layer: logits 1e-3 per
row, indices exact beyond a 1e-3 margin, weights 1e-5, outputs 2e-2 (5e-2
MXFP4)."""
import numpy as np
import pytest
import torch

import mixture_experts_decode_wave_amd as mw
import moe_synth as ms
import oracle
from tests import harness as H

pytestmark = pytest.mark.gpu

OUT_TOL = {"f32": 2e-2, "bf16": 2e-2, "fp8_b128": 2e-2, "mxfp4": 5e-2}
CASES = [("tiny", 1), ("qwen3_30b_a3b", 4), ("qwen3_next_gated", 1), ("qwen3_next_gated", 16),
         ("deepseek_v3", 1), ("zero_experts_384", 4)]
_LAYERS = {}


def _layer(name):
    if name not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        li = ms.make_layer(name, seed=0, device="cuda")
        _LAYERS[name] = (H.device_layer(li, max_n=16), ms.make_norms(li.spec, 0, "cuda"))
    return _LAYERS[name]


@pytest.mark.parametrize("which", ["both", "router", "expert"])
@pytest.mark.parametrize("name,n", CASES)
def test_layer_with_pre_norms_matches_oracle(name, n, which):
    print(f"[pre-norms] {name} N={n} {which}", flush=True)
    dl, (rw, ew) = _layer(name)
    spec = dl.spec
    rw = rw if which in ("both", "router") else None
    ew = ew if which in ("both", "expert") else None
    eps = ms.NORM_EPS
    x = dl.li.x[:n].contiguous()
    out = torch.empty(n, spec.hidden, dtype=x.dtype, device="cuda")
    logits = torch.empty(n, spec.router_width, dtype=torch.float32, device="cuda")
    idx = torch.empty(n, spec.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(n, spec.top_k, dtype=torch.float32, device="cuda")
    mw.moe_layer_forward_norm(dl.cfg, x, rw, ew, eps, dl.li.router, dl.li.bias, dl.tables,
                              dl.shared, out, dl.ws, logits=logits, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    g = {"logits": logits.cpu().numpy(), "idx": idx.cpu().numpy().astype(np.int64),
         "w": w.cpu().numpy(), "out": out.float().cpu().numpy()}
    xr = x if rw is None else oracle.rms_norm(spec, x, rw, eps)
    xe = x if ew is None else oracle.rms_norm(spec, x, ew, eps)
    lg = oracle.router_logits(spec, xr, dl.li.router)
    for t in range(n):
        e = H.rel_err(g["logits"][t], lg[t])
        assert e <= 1e-3, f"row {t}: logits rel err {e}"
    ridx, rwt = oracle.topk(spec, lg, dl.li.bias)
    ref = {"logits": lg, "keys": oracle.keys(spec, lg, dl.li.bias), "idx": ridx, "w": rwt}
    H.check_routing(spec, ref, g["idx"], g["w"])
    idx_o, w_o, alt = H.outputs_routing(spec, ref, g["idx"], g["w"])
    out_ref = oracle.experts(dl.li, n, idx_o, w_o, x=xe.cpu(), gate_x=x.cpu())
    err = H.rel_err(g["out"], out_ref)
    print(f"    rows={n} other_picks={len(alt)} out_rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL[spec.expert_dtype], err


def test_no_norm_weights_is_the_plain_layer():
    """Both weights NULL: the same bits as moe_layer_forward."""
    dl, _ = _layer("qwen3_next_gated")
    spec = dl.spec
    n = 4
    a = H.run_layer(dl, n)
    x = dl.li.x[:n].contiguous()
    out = torch.empty(n, spec.hidden, dtype=x.dtype, device="cuda")
    mw.moe_layer_forward_norm(dl.cfg, x, None, None, 0.0, dl.li.router, dl.li.bias, dl.tables,
                              dl.shared, out, dl.ws)
    torch.cuda.synchronize()
    assert torch.equal(out, a["out"])


# Shapes where the router computes the norms itself with few workgroups and
# long rows, so that a workgroup's share of the experts' normed rows is more
# than one pair per thread (E = 4: one router workgroup; h = 8192: 1024
# chunks a row), and a ragged row count.
WIDE = [("bf16", 8192, 4, 4), ("bf16", 2048, 4, 3), ("f32", 4096, 8, 2), ("fp8_b128", 8192, 8, 4)]


@pytest.mark.parametrize("fmt,h,E,n", WIDE)
def test_pre_norms_few_router_workgroups(fmt, h, E, n):
    print(f"[pre-norms wide] {fmt} h={h} E={E} N={n}", flush=True)
    act = "f32" if fmt == "f32" else "bf16"
    spec = ms.SPECS["tiny"].with_(hidden=h, num_experts=E, top_k=2, inter=128, act_dtype=act,
                                  expert_dtype=fmt, shared_inter=128)
    li = ms.make_layer(spec, seed=3, device="cuda")
    dl = H.device_layer(li, max_n=n)
    rw, ew = ms.make_norms(spec, 1, "cuda")
    x = li.x[:n].contiguous()
    out = torch.empty(n, h, dtype=x.dtype, device="cuda")
    logits = torch.empty(n, spec.router_width, dtype=torch.float32, device="cuda")
    idx = torch.empty(n, spec.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(n, spec.top_k, dtype=torch.float32, device="cuda")
    mw.moe_layer_forward_norm(dl.cfg, x, rw, ew, ms.NORM_EPS, li.router, li.bias, dl.tables,
                              dl.shared, out, dl.ws, logits=logits, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    xr = oracle.rms_norm(spec, x, rw, ms.NORM_EPS)
    xe = oracle.rms_norm(spec, x, ew, ms.NORM_EPS)
    lg = oracle.router_logits(spec, xr, li.router)
    g_lg = logits.cpu().numpy()
    for t in range(n):
        assert H.rel_err(g_lg[t], lg[t]) <= 1e-3
    ridx, rwt = oracle.topk(spec, lg, li.bias)
    ref = {"logits": lg, "keys": oracle.keys(spec, lg, li.bias), "idx": ridx, "w": rwt}
    g_idx = idx.cpu().numpy().astype(np.int64)
    H.check_routing(spec, ref, g_idx, w.cpu().numpy())
    idx_o, w_o, _ = H.outputs_routing(spec, ref, g_idx, w.cpu().numpy())
    out_ref = oracle.experts(li, n, idx_o, w_o, x=xe.cpu(), gate_x=x.cpu())
    err = H.rel_err(out.float().cpu().numpy(), out_ref)
    print(f"    out_rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL[spec.expert_dtype], err
