"""The expert-parallel split of the layer (design for several GPUs), checked on
one GPU: S ranks each hold E/S experts and route every row with the same
router; each computes only its own routes (routes to other ranks' experts
are dropped: their ids fall outside the rank's [0, E/S)), without the shared
expert; the shared expert is added once.  The sum of the S partial outputs and
the shared-only output must match the whole layer from the fp64 oracle, to the
output tolerance.  This is the kernel half of the forward pass the pages
shard by experts, with an all-reduce of the partial [N, h] outputs between
the ranks (the summation here stands in for it)."""
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
