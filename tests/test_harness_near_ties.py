"""The parity tests' near-tie handling, on the CPU: where a GPU picks a
different valid set on a near-tie row, the output is compared at the GPU's
picks with the oracle's weights of those picks, and the GPU's weights must
match those weights.  Checked here with a constructed near tie and stand-in
GPU results, so the path is exercised even when the GPU happens to pick the
oracle's set on every row."""
import numpy as np
import pytest

import moe_synth as ms
import oracle
from tests import harness as H


def _near_tie_ref():
    spec = ms.SPECS["tiny"].with_(num_experts=6, top_k=2)
    lg = np.array([[2.0, 1.0, 1.0 + 4e-4, -1.0, 0.0, -2.0],    # experts 1 and 2 nearly tie
                   [3.0, -1.0, 0.5, 2.0, -0.5, 0.0]])           # a clear row
    idx, w = oracle.topk(spec, lg)
    return spec, {"logits": lg, "keys": oracle.keys(spec, lg), "idx": idx, "w": w}


def test_other_valid_picks_are_weighted_by_the_oracle():
    spec, ref = _near_tie_ref()
    assert ref["idx"][0].tolist() == [0, 2]
    got_idx = np.array([[0, 1], ref["idx"][1].tolist()])           # the near-tie alternative
    got_w = np.vstack([oracle.route_weights(spec, ref["logits"][:1], [[0, 1]]),
                       ref["w"][1:]]).astype(np.float32)
    ties = H.check_routing(spec, ref, got_idx, got_w)
    assert ties == [0]
    idx, w, alt = H.outputs_routing(spec, ref, got_idx, got_w)
    assert alt == [0]
    assert idx[0].tolist() == [0, 1] and idx[1].tolist() == ref["idx"][1].tolist()
    s = np.exp(ref["logits"][0][[0, 1]])
    assert np.allclose(w[0], s / s.sum(), rtol=1e-13)
    assert np.array_equal(w[1], ref["w"][1])


def test_wrong_weights_at_other_picks_fail():
    spec, ref = _near_tie_ref()
    got_idx = np.array([[0, 1], ref["idx"][1].tolist()])
    got_w = np.vstack([ref["w"][:1], ref["w"][1:]]).astype(np.float32)  # the oracle's picks' weights
    with pytest.raises(AssertionError):
        H.outputs_routing(spec, ref, got_idx, got_w)


def test_a_clear_row_must_match_the_oracle():
    spec, ref = _near_tie_ref()
    got_idx = np.array([ref["idx"][0].tolist(), [0, 2]])           # row 1 is not a near tie
    with pytest.raises(AssertionError):
        H.check_routing(spec, ref, got_idx, ref["w"].astype(np.float32))
