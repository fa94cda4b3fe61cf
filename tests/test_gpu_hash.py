"""moe_layer_forward_hash against the fp64 oracle: hash routing (forward.rs,
the hash-routing branch of the top-k step) on synthetic token-to-expert
tables.  The picks are table entries, so they must match exactly; weights to
1e-5, logits to 1e-3 per row, outputs to 2e-2 (5e-2 MXFP4)."""
import numpy as np
import pytest
import torch

import mixture_experts_decode_wave_amd as mw
import moe_synth as ms
import oracle
from tests import harness as H

pytestmark = pytest.mark.gpu

OUT_TOL = {"f32": 2e-2, "bf16": 2e-2, "fp8_b128": 2e-2, "mxfp4": 5e-2}
VOCAB = 1000


def _run(dl, n, tok, tab):
    spec = dl.spec
    x = dl.li.x[:n].contiguous() if n <= dl.li.x.shape[0] else None
    out = torch.empty(n, spec.hidden, dtype=x.dtype, device="cuda")
    logits = torch.empty(n, spec.num_experts, dtype=torch.float32, device="cuda")
    idx = torch.empty(n, spec.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(n, spec.top_k, dtype=torch.float32, device="cuda")
    mw.moe_layer_forward_hash(dl.cfg, x, tok, tab, dl.li.router, dl.tables, dl.shared, out,
                              dl.ws, logits=logits, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    return x, {"logits": logits.cpu().numpy(), "idx": idx.cpu().numpy(), "w": w.cpu().numpy(),
               "out": out.float().cpu().numpy()}


def _compare(dl, n, x, g, tok, tab, rows=None):
    spec = dl.spec
    lg = oracle.router_logits(spec, x, dl.li.router)
    for t in range(n):
        assert H.rel_err(g["logits"][t], lg[t]) <= 1e-3, t
    idx, w = oracle.hash_route(spec, lg, tab.cpu().numpy(), tok.cpu().numpy())
    assert np.array_equal(g["idx"], idx)
    assert np.allclose(g["w"], w, rtol=1e-5, atol=1e-7)
    rows = list(range(n)) if rows is None else rows
    sel = torch.tensor(rows)
    keep = np.where((idx[rows] >= 0) & (idx[rows] < spec.num_experts), idx[rows], 0)
    wk = np.where((idx[rows] >= 0) & (idx[rows] < spec.num_experts), w[rows], 0.0)
    ref = oracle.experts(dl.li, len(rows), keep, wk, x=x.cpu()[sel])
    err = H.rel_err(g["out"][rows], ref)
    print(f"    N={n} out_rel_err={err:.3e}", flush=True)
    assert err <= OUT_TOL[spec.expert_dtype], err


@pytest.mark.parametrize("name,n", [("deepseek_v3", 1), ("deepseek_v3", 4), ("deepseek_v3", 16),
                                    ("qwen3_30b_a3b", 4), ("tiny", 1)])
def test_hash_routed_layer_matches_oracle(name, n):
    print(f"[hash] {name} N={n}", flush=True)
    li = ms.make_layer(name, seed=0, device="cuda")
    dl = H.device_layer(li, max_n=16)
    tab = ms.make_hash_table(li.spec, VOCAB, 0, "cuda")
    tok = ms.make_token_ids(n, VOCAB, 3, "cuda")
    x, g = _run(dl, n, tok, tab)
    _compare(dl, n, x, g, tok, tab)


def test_hash_table_entries_and_tokens_out_of_range():
    """Entries outside [0, E) are dropped and the rest renormalise; a token
    outside the table drops its row (its output is the shared expert alone)."""
    spec = ms.SPECS["qwen3_next"].with_(hidden=256, num_experts=16, top_k=4, inter=128,
                                        shared_inter=128)
    li = ms.make_layer(spec, seed=5, device="cuda")
    dl = H.device_layer(li, max_n=8)
    tab = ms.make_hash_table(spec, 20, 1).clone()
    tab[3, 1] = 16
    tab[4, 0] = -1
    tab[4, 2] = 99
    tab = tab.cuda()
    tok = torch.tensor([3, 4, 20, -2, 0, 5, 7, 3], dtype=torch.int32, device="cuda")
    x, g = _run(dl, 8, tok, tab)
    _compare(dl, 8, x, g, tok, tab)
