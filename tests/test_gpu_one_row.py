"""One-row steps: the down pass and the blend run as one kernel where the
down pass streams at most 26 MB.  Checked against the fp64 oracle under
caller routings with a repeated expert and dropped slots (ids -1 and E),
with and without a gated shared expert, in every weight format, at both
lane widths of a weight row (16 and 64 lanes) and with a last workgroup of
fewer output columns; and bitwise against the two-kernel form, which the
same row takes inside a two-row step under top-k routing."""
import sys

import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
from tests import harness as H

pytestmark = pytest.mark.gpu

OUT_TOL = {"f32": 2e-2, "bf16": 2e-2, "fp8_b128": 2e-2, "mxfp4": 5e-2}

# (format, h, I = shared I, shared expert): h / 512 output columns per
# workgroup, h not a multiple of that; I / (elements per 16-byte chunk) >= 128
# gives 64 lanes per weight row, else 16
CASES = [
    ("f32", 1600, 512, False),       # 128 chunks: 64 lanes
    ("f32", 1600, 160, True),        # 40 chunks: 16 lanes
    ("bf16", 1600, 1024, True),      # 64 lanes
    ("bf16", 1600, 160, False),      # 16 lanes
    ("fp8_b128", 1664, 2048, True),  # 64 lanes
    ("fp8_b128", 1664, 512, True),   # 16 lanes
    ("mxfp4", 1600, 4096, False),    # 64 lanes
    ("mxfp4", 1600, 1536, True),     # 16 lanes
]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _layer(fmt, h, inter, shared, gated=False, seed=23):
    act = "f32" if fmt == "f32" else "bf16"
    spec = ms.SPECS["qwen3_next"].with_(hidden=h, num_experts=13, top_k=3, inter=inter,
                                        shared_inter=inter if shared else 0, act_dtype=act,
                                        expert_dtype=fmt, shared_gate=gated and shared)
    li = ms.make_layer(spec, seed=seed, device="cuda")
    return spec, li, H.device_layer(li, max_n=2)


@pytest.mark.parametrize("fmt,h,inter,shared", CASES)
def test_one_row_matches_oracle(fmt, h, inter, shared):
    _say(f"[one row] {fmt} h={h} I={inter} shared={shared}")
    spec, li, dl = _layer(fmt, h, inter, shared, gated=shared)
    E = spec.num_experts
    routings = [
        ([4, 9, 1], [0.5, 0.3, 0.2]),      # distinct experts
        ([7, 7, 2], [0.4, 0.35, 0.25]),    # a repeated expert
        ([3, -1, 11], [0.6, 0.9, 0.4]),    # a slot dropped (id -1)
        ([E, 5, E], [0.2, 0.7, 0.1]),      # two slots dropped (id E)
        ([-1, E, -1], [0.3, 0.3, 0.4]),    # every slot dropped
    ]
    for idx, w in routings:
        idx = np.array([idx], dtype=np.int64)
        w = np.array([w], dtype=np.float32)
        got = H.run_experts(dl, 1, idx, w)
        torch.cuda.synchronize()
        g = got.float().cpu().numpy()
        drop = (idx < 0) | (idx >= E)
        ref = oracle.experts(li, 1, np.where(drop, 0, idx),
                             np.where(drop, 0.0, w.astype(np.float64)), x=li.x[:1])
        if drop.all() and not shared:
            assert not g.any(), "every slot dropped: the output must be zeros"
            continue
        err = H.rel_err(g, ref)
        _say(f"    idx={idx[0].tolist()} out_rel_err={err:.3e}")
        assert err <= OUT_TOL[fmt], err


@pytest.mark.parametrize("fmt,h,inter,shared", CASES)
def test_one_row_is_bitwise_the_two_kernel_form(fmt, h, inter, shared):
    """Top-k routing: row t alone (one kernel) and row t inside a two-row
    step (the down pass, then the blend) give the same bits."""
    _say(f"[one row, bitwise] {fmt} h={h} I={inter} shared={shared}")
    spec, li, dl = _layer(fmt, h, inter, shared, gated=shared)
    two = H.run_layer(dl, 2)
    ones = [H.run_layer(dl, 1, x=li.x[t:t + 1]) for t in (0, 1)]
    torch.cuda.synchronize()
    for t, one in enumerate(ones):
        for key in ("logits", "idx", "w", "out"):
            assert torch.equal(one[key][0], two[key][t]), (key, t)
