"""moe_layer_forward_static, the entry point for callers that cannot
allocate (its workspace is the library's static per-GPU scratch), against
moe_layer_forward on a caller's workspace: the same kernels, so the same bits
of out, logits, idx and w.  Two calls in a row on each layer, the second with
fewer rows, so the second runs on scratch the first left behind; a
configuration beyond the scratch is refused."""
import sys

import pytest
import torch

import mixture_experts_decode_wave_amd as mw
import moe_synth as ms
from mixture_experts_decode_wave_amd.layer import device_layer, run_layer

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _static(dl, n, with_outputs=True):
    spec = dl.spec
    x = dl.li.x[:n].contiguous()
    out = torch.empty(n, spec.hidden, dtype=x.dtype, device=x.device)
    res = {"out": out}
    kw = {}
    if with_outputs:
        res["logits"] = kw["logits"] = torch.empty(n, spec.router_width, dtype=torch.float32,
                                                   device=x.device)
        res["idx"] = kw["topk_idx"] = torch.empty(n, spec.top_k, dtype=torch.int32,
                                                  device=x.device)
        res["w"] = kw["topk_w"] = torch.empty(n, spec.top_k, dtype=torch.float32,
                                              device=x.device)
    mw.moe_layer_forward_static(dl.cfg, x, dl.li.router, dl.li.bias, dl.tables, dl.shared, out,
                                **kw)
    return res


@pytest.mark.parametrize("name,n1,n2", [("verify_mxfp4", 256, 5), ("qwen3_next_gated", 16, 1),
                                        ("deepseek_v3", 4, 1)])
def test_static_scratch_matches_the_workspace_entry_point(name, n1, n2):
    _say(f"[static scratch] {name} N={n1} then N={n2}")
    li = ms.make_layer(name, seed=0, device="cuda")
    dl = device_layer(li, max_n=n1)
    assert mw.workspace_size(dl.cfg, n1) <= mw.STATIC_SCRATCH_BYTES
    for n in (n1, n2):
        ref = run_layer(dl, n)
        got = _static(dl, n)
        torch.cuda.synchronize()
        for key in ("out", "logits", "idx", "w"):
            assert torch.equal(got[key], ref[key]), (name, n, key)
        lean = _static(dl, n, with_outputs=False)  # routing kept in the scratch
        torch.cuda.synchronize()
        assert torch.equal(lean["out"], ref["out"]), (name, n, "out without optional outputs")


def test_static_scratch_refuses_a_larger_workspace():
    spec = ms.SPECS["qwen3_next"].with_(hidden=4096, num_experts=256, top_k=8, inter=1536,
                                        shared_inter=1536, expert_dtype="mxfp4")
    li = ms.make_layer(spec.with_(num_experts=8), seed=0, device="cuda")
    dl = device_layer(li, max_n=1)
    cfg = mw.make_cfg(4096, 256, 8, 1536, 1536, "softmax", True, 1.0, "bf16", "mxfp4")
    n = 1024
    assert mw.workspace_size(cfg, n) > mw.STATIC_SCRATCH_BYTES
    x = torch.zeros(n, 4096, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(mw.MoeError) as e:
        mw.moe_layer_forward_static(cfg, x, li.router, None, dl.tables, dl.shared, out)
    assert e.value.code == -6 and "static scratch holds" in str(e.value)
