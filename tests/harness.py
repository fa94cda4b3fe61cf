"""The comparisons the parity tests make between the HIP library and the
fp64 oracle.  No arithmetic of the layer lives here: the device side runs in
libmoewave.so (set up through mixture_experts_decode_wave_amd.layer), the
reference side in oracle/."""
from __future__ import annotations

import numpy as np

import oracle
from mixture_experts_decode_wave_amd.layer import (DeviceLayer, cfg_of, device_layer,  # noqa: F401
                                                   run_experts, run_layer, run_route)


# ------------------------------------------------------------------ comparisons

def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (the output tolerance measure)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def near_tie_alternatives(keys_row: np.ndarray, k: int, eps: float):
    """Index sets a top-k may validly return when keys within eps of the
    k-th largest key are treated as tied: every expert whose key beats the
    k-th key by more than eps is in; the remaining slots go to any of the
    experts within eps of it.  Returns (must, optional, n_free)."""
    order = np.argsort(-keys_row, kind="stable")
    kth = keys_row[order[k - 1]]
    must = [int(e) for e in order if keys_row[e] > kth + eps]
    band = [int(e) for e in order if abs(keys_row[e] - kth) <= eps]
    return must, band, k - len(must)


def check_routing(spec, ref: dict, got_idx: np.ndarray, got_w: np.ndarray, eps: float = 1e-3):
    """Routing parity under the margin rule.  Rows whose oracle margin between
    the k-th and (k+1)-th key exceeds eps must pick the oracle's index set
    exactly, in the oracle's slot order wherever adjacent keys differ by more
    than eps, with weights within 1e-5 relative.  Other rows must pick a valid
    set (see near_tie_alternatives).  Returns the list of near-tie rows."""
    k = spec.top_k
    keys = ref["keys"]
    ties = []
    for t in range(got_idx.shape[0]):
        kr = keys[t]
        srt = np.sort(kr)[::-1]
        margin = srt[k - 1] - srt[k] if k < len(kr) else np.inf
        gi, gw = got_idx[t], got_w[t]
        assert len(set(gi.tolist())) == k, f"row {t}: repeated experts {gi}"
        assert gi.min() >= 0 and gi.max() < spec.router_width, f"row {t}: id out of range {gi}"
        if margin > eps:
            ri = ref["idx"][t]
            assert set(gi.tolist()) == set(ri.tolist()), f"row {t}: {gi} vs oracle {ri}"
            rk = kr[ri]
            for j in range(k):
                sep_prev = j == 0 or rk[j - 1] - rk[j] > eps
                sep_next = j == k - 1 or rk[j] - rk[j + 1] > eps
                if sep_prev and sep_next:
                    assert gi[j] == ri[j], f"row {t} slot {j}: {gi} vs oracle {ri}"
            wmap = dict(zip(ri.tolist(), ref["w"][t].tolist()))
            for e, wv in zip(gi.tolist(), gw.tolist()):
                assert abs(wv - wmap[e]) <= 1e-5 * abs(wmap[e]) + 1e-7, \
                    f"row {t} expert {e}: w {wv} vs {wmap[e]}"
        else:
            ties.append(t)
            must, band, nfree = near_tie_alternatives(kr, k, eps)
            gs = set(gi.tolist())
            assert set(must) <= gs, f"row {t}: misses a clear winner"
            assert gs - set(must) <= set(band) and len(gs - set(must)) == nfree
    return ties


def assert_sorted_desc(keys_row: np.ndarray, idx_row: np.ndarray, eps: float = 1e-3):
    kk = keys_row[idx_row]
    assert np.all(kk[:-1] >= kk[1:] - eps)


def outputs_routing(spec, ref: dict, got_idx: np.ndarray, got_w: np.ndarray):
    """The routing under which the oracle evaluates the outputs, row by row.

    Where the GPU picked the oracle's own index set, the oracle's picks and
    weights (check_routing has compared the weights).  On a near-tie row where
    the GPU picked a different valid set (the pages' batched and per-row
    routers may also pick differently there), the GPU's picks, weighted by the
    oracle from its fp64 logits (oracle.route_weights): the GPU's weights must
    match those to 1e-5 relative, and that row's output is then compared at
    the GPU's picks.  Returns (idx, w, alt), alt listing the rows of the
    second kind."""
    k = spec.top_k
    idx = np.array(ref["idx"], dtype=np.int32, copy=True)
    w = np.array(ref["w"], dtype=np.float64, copy=True)
    gi = np.asarray(got_idx).astype(np.int32).reshape(-1, k)
    alt = [t for t in range(gi.shape[0]) if set(gi[t].tolist()) != set(idx[t].tolist())]
    if alt:
        wa = oracle.route_weights(spec, np.asarray(ref["logits"])[alt], gi[alt])
        for i, t in enumerate(alt):
            gw = np.asarray(got_w[t], dtype=np.float64)
            assert np.all(np.abs(gw - wa[i]) <= 1e-5 * np.abs(wa[i]) + 1e-7), \
                f"row {t}: near-tie weights {gw} vs oracle at the same picks {wa[i]}"
            idx[t] = gi[t]
            w[t] = wa[i]
    return idx, w, alt
