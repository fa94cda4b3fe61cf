"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
published format tables (OCP FP8 / MX specs), torch's own float8 decoders,
BLAS products, brute-force top-k, closed forms of softmax / sigmoid weights,
and constructed experts whose output is known exactly (identity-like experts,
shared-only layers)."""
import itertools
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

import moe_synth as ms
import oracle
from tests.constructed import identity_layer as _identity_layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b = line.split()
                rows.append((a, float(b)))
    return rows


def _same(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        np.nan_to_num(a), np.nan_to_num(b)) and np.array_equal(np.signbit(a[~np.isnan(a)]),
                                                                np.signbit(b[~np.isnan(b)]))


# ---------------------------------------------------------------- decoders

def test_fp8_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(oracle.decode_fp8_e4m3(codes), ref)


def test_fp8_e4m3_spec_points():
    for code, val in _golden("ocp_e4m3_points.txt"):
        got = oracle.decode_fp8_e4m3([int(code, 16)])[0]
        assert _same([got], [val]), (code, got, val)


def test_e8m0_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[125] == 0.25


def test_e2m1_spec_table():
    table = _golden("ocp_e2m1.txt")
    got = oracle.decode_e2m1([int(c) for c, _ in table])
    assert _same(got, [v for _, v in table])


def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(0)
    bits = np.concatenate([rng.integers(0, 1 << 16, 4000), [0, 0x8000, 0x7F80, 0xFF80, 0x0001]])
    bits = bits.astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(oracle.decode_bf16(bits), ref)


# ---------------------------------------------------------------- dequant layouts

def test_tiled_storage_positions():
    """The storage layout of expert weights (16-row x 64-byte tiles), checked
    at positions worked out by hand from its definition: a 32 x 24 fp32
    matrix (96-byte rows: one full tile column and one of 32 bytes)."""
    M = torch.arange(32 * 24, dtype=torch.float32).reshape(32, 24)  # M[r, c] = 24 r + c
    flat = ms.tile_16x64(M).reshape(-1)
    # (row, col) -> fp32 slot in the stored bytes
    for (r, c), slot in {(0, 0): 0, (0, 15): 15, (1, 0): 16, (15, 15): 255, (0, 16): 256,
                         (1, 16): 264, (15, 23): 383, (16, 0): 384, (17, 20): 652,
                         (31, 23): 767}.items():
        assert flat[slot].item() == 24 * r + c, (r, c, slot)
    # the oracle reads the same positions
    got = oracle.dequant("f32", 32, 24, ms.tile_16x64(M))
    assert np.array_equal(got, M.double().numpy())


def test_fp8_b128_dequant_block_layout():
    # ragged: 304 x 416 has partial 128-blocks at the bottom and right, and its
    # 416-byte rows end in a tile column 32 bytes wide (416 = 6 x 64 + 32)
    g = torch.Generator().manual_seed(1)
    w = torch.randn(304, 416, generator=g) * torch.linspace(0.1, 10, 416)
    codes, s = ms.quant_fp8_b128(w)
    assert s.shape == (3, 4)
    # independent expansion of the row-major codes: torch's e4m3 decoder times
    # the block scale repeated
    q = codes.view(torch.float8_e4m3fn).to(torch.float64)
    sfull = s.to(torch.float64).repeat_interleave(128, 0).repeat_interleave(128, 1)[:304, :416]
    ref = (q * sfull).numpy()
    stored, s2 = ms.encode(w, "fp8_b128")
    assert torch.equal(s2, s)
    got = oracle.dequant("fp8_b128", 304, 416, stored, s2)
    assert np.array_equal(got, ref)
    # and the round trip stays within e4m3 rounding of the original
    err = np.abs(got - w.double().numpy())
    bound = np.maximum(np.abs(w.double().numpy()) * 2.0 ** -4, sfull.numpy() * 2.0 ** -10)
    assert np.all(err <= bound + 1e-12)


def test_mxfp4_dequant_nibble_and_scale_layout():
    g = torch.Generator().manual_seed(2)
    w = torch.randn(48, 96, generator=g) * torch.linspace(0.01, 50, 96)
    packed, E = ms.quant_mxfp4(w)
    assert packed.shape == (48, 48) and E.shape == (48, 3)
    table = np.array([v for _, v in _golden("ocp_e2m1.txt")])
    p = packed.numpy()
    nib = np.empty((48, 96), dtype=np.int64)
    nib[:, 0::2] = p & 15
    nib[:, 1::2] = p >> 4
    ref = table[nib] * np.ldexp(1.0, np.repeat(E.numpy().astype(np.int64) - 127, 32, axis=1))
    stored, E2 = ms.encode(w, "mxfp4")  # 48-byte rows: one tile column narrower than 64
    assert torch.equal(E2, E)
    got = oracle.dequant("mxfp4", 48, 96, stored, E2)
    assert np.array_equal(got, ref)
    # the round trip stays within half an e2m1 step of the scaled value
    scale = np.ldexp(1.0, np.repeat(E.numpy().astype(np.int64) - 127, 32, axis=1))
    v = w.double().numpy() / scale
    assert np.all(np.abs(got / scale - np.clip(v, -6, 6)) <= np.where(np.abs(v) < 2, 0.25, 1.0) + 1e-12)


def test_bf16_and_f32_dequant_are_plain():
    g = torch.Generator().manual_seed(3)
    w = torch.randn(32, 40, generator=g)
    assert np.array_equal(oracle.dequant("f32", 32, 40, ms.encode(w, "f32")[0]),
                          w.double().numpy())
    wb = w.to(torch.bfloat16)
    assert np.array_equal(oracle.dequant("bf16", 32, 40, ms.encode(w, "bf16")[0]),
                          wb.double().numpy())


# ---------------------------------------------------------------- router

@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_router_logits_match_blas(act):
    spec = ms.SPECS["tiny"].with_(act_dtype=act, hidden=96, num_experts=13)
    g = torch.Generator().manual_seed(4)
    dt = ms.act_torch_dtype(act)
    x = torch.randn(7, 96, generator=g).to(dt)
    W = torch.randn(13, 96, generator=g).to(dt)
    ref = x.double().numpy() @ W.double().numpy().T
    got = oracle.router_logits(spec, x, W)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- top-k

def _brute_rank(keys):
    """rank of each expert: how many keys beat it (larger, or equal at a lower index)."""
    E = len(keys)
    return np.array([sum(1 for f in range(E) if keys[f] > keys[e] or (keys[f] == keys[e] and f < e))
                     for e in range(E)])


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("coarse", [False, True])
def test_topk_matches_brute_force(scoring, coarse):
    rng = np.random.default_rng(5 + coarse)
    E = 12
    for k in range(1, E + 1):
        spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=k, scoring=scoring)
        lg = rng.normal(size=(6, E))
        if coarse:  # many exact ties
            lg = np.round(lg * 2) / 2
        bias = None
        if scoring == "sigmoid":
            bias = torch.tensor(rng.uniform(-0.1, 0.1, E), dtype=torch.float32)
            if coarse:
                bias = torch.zeros(E)
        idx, _ = oracle.topk(spec, lg, bias)
        keys = oracle.keys(spec, lg, bias)
        for t in range(6):
            if scoring == "sigmoid":
                kb = expit(lg[t]) + (0 if bias is None else bias.double().numpy())
                assert np.array_equal(keys[t], kb)
            rank = _brute_rank(keys[t])
            want = np.argsort(rank)[:k]
            assert list(idx[t]) == list(want), (k, t)


def test_topk_set_maximises_key_sum():
    rng = np.random.default_rng(6)
    E = 9
    for k in (1, 3, 5):
        spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=k)
        lg = rng.normal(size=(4, E))
        idx, _ = oracle.topk(spec, lg)
        for t in range(4):
            best = max(itertools.combinations(range(E), k), key=lambda s: sum(lg[t][list(s)]))
            assert set(idx[t]) == set(best)


def test_topk_ties_go_to_lowest_index():
    spec = ms.SPECS["tiny"].with_(num_experts=8, top_k=3)
    lg = np.array([[0.5, 1.0, 0.5, 1.0, 1.0, -2.0, 1.0, 0.0]])
    idx, w = oracle.topk(spec, lg)
    assert list(idx[0]) == [1, 3, 4]
    assert np.allclose(w[0], [1 / 3] * 3)
    lg = np.array([[-0.0, 0.0, -1.0, -1.0, -1.0, -1.0, -1.0, -1.0]])
    idx, _ = oracle.topk(spec, lg)
    assert list(idx[0]) == [0, 1, 2]


# ---------------------------------------------------------------- weights

def test_weights_closed_forms():
    rng = np.random.default_rng(7)
    E = 10
    lg = rng.normal(size=(5, E)) * 2
    # k = 2, softmax, norm: w0 = sigmoid(l0 - l1)
    spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=2)
    idx, w = oracle.topk(spec, lg)
    for t in range(5):
        l0, l1 = lg[t][idx[t]]
        assert math.isclose(w[t][0], expit(l0 - l1), rel_tol=1e-13)
        assert math.isclose(w[t][1], expit(l1 - l0), rel_tol=1e-13)
    # k = E, softmax, norm: the full softmax
    spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=E)
    idx, w = oracle.topk(spec, lg)
    for t in range(5):
        assert np.allclose(w[t], softmax(lg[t])[idx[t]], rtol=1e-13)
    # softmax without norm: softmax over all E, sliced
    spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=3, norm_topk=False)
    idx, w = oracle.topk(spec, lg)
    for t in range(5):
        assert np.allclose(w[t], softmax(lg[t])[idx[t]], rtol=1e-13)
    # sigmoid without norm, rsf: sigmoid of the logit times rsf
    spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=3, scoring="sigmoid", norm_topk=False,
                                  routed_scaling=2.5)
    idx, w = oracle.topk(spec, lg)
    for t in range(5):
        assert np.allclose(w[t], 2.5 * expit(lg[t][idx[t]]), rtol=1e-13)


@pytest.mark.parametrize("scoring,rsf", [("softmax", 1.0), ("sigmoid", 2.5), ("softmax", 0.5)])
def test_weights_sum_to_rsf_under_norm(scoring, rsf):
    rng = np.random.default_rng(8)
    E, k = 64, 6
    spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=k, scoring=scoring, routed_scaling=rsf)
    lg = rng.normal(size=(20, E)) * 3
    bias = torch.tensor(rng.uniform(-0.1, 0.1, E), dtype=torch.float32) if scoring == "sigmoid" else None
    idx, w = oracle.topk(spec, lg, bias)
    assert np.allclose(w.sum(1), rsf, rtol=1e-13)
    assert np.all(w > 0)
    for t in range(20):
        assert len(set(idx[t])) == k and idx[t].min() >= 0 and idx[t].max() < E


def test_bias_selects_but_does_not_weight():
    E, k = 6, 2
    spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=k, scoring="sigmoid")
    lg = np.array([[2.0, 1.5, 1.0, -3.0, 0.0, 0.5]])
    bias = torch.tensor([0, 0, 0, 5.0, 0, 0], dtype=torch.float32)
    idx, w = oracle.topk(spec, lg, bias)
    assert list(idx[0]) == [3, 0]  # sigma(-3)+5 beats sigma(2)
    s = expit(np.array([-3.0, 2.0]))
    assert np.allclose(w[0], s / s.sum(), rtol=1e-13)


def test_route_weights_at_picks_that_are_not_the_top_k():
    """Weights of arbitrary picks (a near-tie pick of another router need not
    be this oracle's top-k): closed forms at random non-top picks."""
    rng = np.random.default_rng(9)
    E = 11
    lg = rng.normal(size=(6, E)) * 2
    for t in range(6):
        a, b = rng.choice(E, 2, replace=False)
        # k = 2, softmax, norm: w_a = sigmoid(l_a - l_b), whatever the ranks
        spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=2)
        w = oracle.route_weights(spec, lg[t:t + 1], [[a, b]])[0]
        assert math.isclose(w[0], expit(lg[t][a] - lg[t][b]), rel_tol=1e-13)
        assert math.isclose(w[1], expit(lg[t][b] - lg[t][a]), rel_tol=1e-13)
        picks = rng.choice(E, 4, replace=False)
        # softmax without norm: the softmax over all E at the picks, times rsf
        spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=4, norm_topk=False,
                                      routed_scaling=0.5)
        w = oracle.route_weights(spec, lg[t:t + 1], [picks])[0]
        assert np.allclose(w, 0.5 * softmax(lg[t])[picks], rtol=1e-13)
        # sigmoid, norm, rsf: sigmoid at the picks, renormalised, times rsf
        spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=4, scoring="sigmoid",
                                      routed_scaling=2.5)
        w = oracle.route_weights(spec, lg[t:t + 1], [picks])[0]
        s = expit(lg[t][picks])
        assert np.allclose(w, 2.5 * s / s.sum(), rtol=1e-13)
        assert math.isclose(w.sum(), 2.5, rel_tol=1e-13)
    # at its own picks they are the top-k's weights
    for scoring in ("softmax", "sigmoid"):
        spec = ms.SPECS["tiny"].with_(num_experts=E, top_k=3, scoring=scoring)
        idx, w = oracle.topk(spec, lg)
        assert np.array_equal(oracle.route_weights(spec, lg, idx), w)
    with pytest.raises(ValueError):
        oracle.route_weights(ms.SPECS["tiny"].with_(num_experts=E, top_k=2), lg[:1], [[0, E]])


# ---------------------------------------------------------------- experts

@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8_b128", "mxfp4"])
@pytest.mark.parametrize("scoring,rsf", [("softmax", 1.0), ("sigmoid", 2.5)])
def test_identity_experts_reproduce_input(fmt, scoring, rsf):
    li = _identity_layer(fmt, scoring=scoring, rsf=rsf)
    N = 5
    r = oracle.layer_forward(li, N)
    x = li.x[:N].double().numpy()
    assert np.allclose(r["out"], rsf * x, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", ["bf16", "fp8_b128"])
def test_shared_only_with_sigmoid_gate(fmt):
    li = _identity_layer(fmt, shared=True, zero_routed_down=True, sgate=True)
    N = 4
    r = oracle.layer_forward(li, N)
    x = li.x[:N].double().numpy()
    g = expit(x @ li.sgate.double().numpy())
    assert np.allclose(r["out"], g[:, None] * x, rtol=1e-12, atol=1e-12)


def test_routed_plus_shared_identity():
    li = _identity_layer("fp8_b128", shared=True, scoring="sigmoid", rsf=2.5)
    N = 3
    r = oracle.layer_forward(li, N)
    x = li.x[:N].double().numpy()
    assert np.allclose(r["out"], 3.5 * x, rtol=1e-12, atol=1e-12)


def test_blend_pairs_each_weight_with_its_expert():
    # expert e scales its output by 2^e: out = sum_j w_j 2^idx_j x
    li = _identity_layer("bf16", E=6, k=3)
    h = li.spec.hidden
    for e in range(6):
        li.down.w[e].mul_(2.0 ** e)   # powers of two stay exact in bf16
    N = 6
    r = oracle.layer_forward(li, N)
    x = li.x[:N].double().numpy()
    fac = (r["w"] * (2.0 ** r["idx"])).sum(1)
    assert np.allclose(r["out"], fac[:, None] * x, rtol=1e-12, atol=1e-12)
    assert h == 64


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8_b128", "mxfp4"])
def test_single_expert_layer_is_a_dense_swiglu_mlp(fmt):
    h, I = 64, 96
    spec = ms.SPECS["tiny"].with_(hidden=h, num_experts=1, top_k=1, inter=I, expert_dtype=fmt,
                                  act_dtype="bf16")
    li = ms.make_layer(spec, seed=12)
    N = 3
    r = oracle.layer_forward(li, N)
    Wg = oracle.dequant(fmt, I, h, li.gate.w[0], None if li.gate.s is None else li.gate.s[0])
    Wu = oracle.dequant(fmt, I, h, li.up.w[0], None if li.up.s is None else li.up.s[0])
    Wd = oracle.dequant(fmt, h, I, li.down.w[0], None if li.down.s is None else li.down.s[0])
    x = li.x[:N].double().numpy()
    g, u = x @ Wg.T, x @ Wu.T
    ref = (g * expit(g) * u) @ Wd.T
    assert np.allclose(r["w"], 1.0)
    assert np.allclose(r["out"], ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- zero experts

def _zero_spec(E=3, Z=2, k=2, h=64, I=96, shared=0, rsf=1.0, scoring="softmax"):
    return ms.SPECS["tiny"].with_(hidden=h, num_experts=E, zero_experts=Z, top_k=k, inter=I,
                                  shared_inter=shared, expert_dtype="bf16", act_dtype="bf16",
                                  routed_scaling=rsf, scoring=scoring)


def test_zero_experts_widen_the_router():
    spec = _zero_spec(E=3, Z=5)
    li = ms.make_layer(spec, seed=21)
    assert tuple(li.router.shape) == (8, 64)
    lg = oracle.router_logits(spec, li.x[:4], li.router)
    assert lg.shape == (4, 8)
    x, W = li.x[:4].double().numpy(), li.router.double().numpy()
    assert np.allclose(lg, x @ W.T, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("rsf,shared", [(1.0, 0), (2.5, 0), (1.0, 32)])
def test_all_zero_expert_picks_pass_the_input_through(rsf, shared):
    """Every pick a zero-computation expert, weights renormalised: out = rsf x
    (+ the shared expert, which zero experts leave alone)."""
    spec = _zero_spec(E=3, Z=4, k=3, rsf=rsf, shared=shared)
    li = ms.make_layer(spec, seed=22)
    N = 4
    lg = np.random.default_rng(3).normal(size=(N, 7))
    lg[:, 3:] += 20.0  # the zero experts' keys dominate
    idx, w = oracle.topk(spec, lg)
    assert (idx >= 3).all() and np.allclose(w.sum(1), rsf, rtol=1e-13)
    out = oracle.experts(li, N, idx, w)
    want = rsf * li.x[:N].double().numpy()
    if shared:
        only_shared = oracle.experts(li, N, np.full((N, 3), 3), np.zeros((N, 3)))
        want = want + only_shared
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)


def test_one_real_and_one_zero_expert_closed_form():
    """k = 2 picks, a real expert a and a zero expert b: out = w_a y_a(x) + w_b x
    with w_a = sigmoid(l_a - l_b), y_a a dense SwiGLU of the decoded weights."""
    h, I = 64, 96
    spec = _zero_spec(E=3, Z=2, k=2, h=h, I=I)
    li = ms.make_layer(spec, seed=23)
    N = 3
    lg = np.random.default_rng(4).normal(size=(N, 5))
    lg[:, 1] += 30.0   # real expert 1
    lg[:, 4] += 29.0   # zero expert 4 (slot 1)
    idx, w = oracle.topk(spec, lg)
    assert (idx == [[1, 4]] * N).all()
    assert np.allclose(w[:, 0], expit(lg[:, 1] - lg[:, 4]), rtol=1e-13)
    out = oracle.experts(li, N, idx, w)
    Wg = oracle.dequant("bf16", I, h, li.gate.w[1])
    Wu = oracle.dequant("bf16", I, h, li.up.w[1])
    Wd = oracle.dequant("bf16", h, I, li.down.w[1])
    x = li.x[:N].double().numpy()
    g, u = x @ Wg.T, x @ Wu.T
    ref = w[:, :1] * ((g * expit(g) * u) @ Wd.T) + w[:, 1:] * x
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_zero_experts_share_the_softmax_without_norm():
    """Without renormalisation a real pick's weight is its softmax over all
    E + Z router columns, zero experts included."""
    spec = _zero_spec(E=4, Z=4, k=3).with_(norm_topk=False)
    lg = np.random.default_rng(5).normal(size=(5, 8)) * 2
    idx, w = oracle.topk(spec, lg)
    for t in range(5):
        assert np.allclose(w[t], softmax(lg[t])[idx[t]], rtol=1e-13)


def test_routed_sum_matches_per_route_mlp():
    spec = ms.SPECS["qwen3_next"].with_(hidden=256, num_experts=16, top_k=4, inter=128,
                                        shared_inter=128)
    li = ms.make_layer(spec, seed=13)
    N = 3
    r = oracle.layer_forward(li, N)
    x = li.x[:N].double().numpy()
    dq = lambda m, e, R, Cc: oracle.dequant("fp8_b128", R, Cc, m.w[e], m.s[e])
    for t in range(N):
        acc = np.zeros(256)
        for j in range(4):
            e = r["idx"][t, j]
            Wg, Wu, Wd = dq(li.gate, e, 128, 256), dq(li.up, e, 128, 256), dq(li.down, e, 256, 128)
            g, u = Wg @ x[t], Wu @ x[t]
            acc += r["w"][t, j] * (Wd @ (g * expit(g) * u))
        Wg, Wu, Wd = dq(li.sh_gate, 0, 128, 256), dq(li.sh_up, 0, 128, 256), dq(li.sh_down, 0, 256, 128)
        g, u = Wg @ x[t], Wu @ x[t]
        acc += Wd @ (g * expit(g) * u)
        assert np.allclose(r["out"][t], acc, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------ pre-norms

@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_rms_norm_matches_torch(act):
    """The oracle's RMSNorm against torch.nn.functional.rms_norm in float64 on
    the same stored values (a library routine)."""
    spec = ms.SPECS["qwen3_30b_a3b"].with_(hidden=320, act_dtype=act)
    adt = ms.act_torch_dtype(act)
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(6, 320, generator=g) * 3.0).to(adt)
    w = (1.0 + 0.1 * torch.randn(320, generator=g)).to(adt)
    got = oracle.rms_norm64(spec, x, w, 1e-6)
    want = torch.nn.functional.rms_norm(x.double(), (320,), weight=w.double(), eps=1e-6).numpy()
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_rms_norm_constant_rows():
    """A row of one value c with unit weights normalises to c / sqrt(c^2 + eps)."""
    spec = ms.SPECS["qwen3_30b_a3b"].with_(hidden=64)
    for c, eps in ((0.75, 1e-6), (-3.0, 1e-6), (2.0, 0.5)):
        x = torch.full((2, 64), c, dtype=torch.bfloat16)
        w = torch.ones(64, dtype=torch.bfloat16)
        got = oracle.rms_norm64(spec, x, w, eps)
        assert np.allclose(got, c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)


def test_round_bf16_matches_torch_and_ties_to_even():
    """Rounding to bfloat16: bit-exact with torch's float32 -> bfloat16 on
    float32 values, and halfway cases go to the even neighbour."""
    g = torch.Generator().manual_seed(5)
    v = torch.randn(4096, generator=g) * torch.exp(torch.randn(4096, generator=g) * 4)
    want = v.to(torch.bfloat16).float().numpy()
    got = oracle.round_bf16(v.double().numpy())
    assert np.array_equal(got, want)
    half = 2.0 ** -8  # half a bfloat16 step just above 1
    ties = np.array([1 + half, 1 + 3 * half, -(1 + half), 2 * (1 + 3 * half), 1 + half * 1.0001])
    assert np.array_equal(oracle.round_bf16(ties),
                          np.array([1.0, 1 + 4 * half, -1.0, 2 * (1 + 4 * half), 1 + 2 * half],
                                   dtype=np.float32))


def test_pre_norms_route_on_the_router_norm_and_gate_on_the_raw_input():
    """The layer with pre-norms: with a router norm of constant weight a > 0
    the router's rows are a * rmsnorm(x) (rounded) and the logits scale with
    them, so the picks are those of routing on rmsnorm(x) alone; the shared
    gate reads x itself, so an expert norm on a shared-only layer changes the
    shared expert's input but not its gate."""
    li = _identity_layer("bf16", h=64, E=4, k=2, shared=True, zero_routed_down=True, sgate=True)
    spec = li.spec
    n = 4
    x = li.x[:n]
    ones = torch.ones(spec.hidden, dtype=torch.bfloat16)
    base = oracle.layer_forward(li, n, norms=(ones, None, 1e-6))
    twice = oracle.layer_forward(li, n, norms=(2 * ones, None, 1e-6))
    assert np.array_equal(base["idx"], twice["idx"])
    assert np.allclose(twice["logits"], 2 * base["logits"], rtol=1e-12, atol=0)
    # shared-only (routed down weights are zero): out = g(x) * y_sh(rmsnorm(x))
    with_en = oracle.layer_forward(li, n, norms=(None, ones, 1e-6))
    xe = oracle.rms_norm(spec, x, ones, 1e-6)
    y_sh = oracle.experts(li, n, base["idx"], base["w"], x=xe, gate_x=x)
    assert np.allclose(with_en["out"], y_sh, rtol=1e-12, atol=1e-12)
    xd = x.double().numpy()
    g = expit(xd @ li.sgate.double().numpy())
    # the constructed shared expert maps v to v * v[0] (its up rows read v[0]):
    # out_t = g(x_t) * v_t * v_t[0] with v = rmsnorm(x)
    v = xe.double().numpy()
    assert np.allclose(with_en["out"], g[:, None] * v * v[:, :1], rtol=1e-9, atol=1e-9)


# ------------------------------------------------------------------ hash routing

def _hash_spec(k=4, norm=True, rsf=1.0):
    return ms.SPECS["deepseek_v3"].with_(num_experts=16, top_k=k, norm_topk=norm,
                                         routed_scaling=rsf)


def test_hash_route_scores_are_sqrt_softplus():
    """Without renormalisation each weight is sqrt(log(1 + e^z)) of its expert's
    logit (numpy logaddexp, a library routine), over a wide range of z."""
    spec = _hash_spec(k=4, norm=False)
    z = np.array([[-40.0, -3.0, -0.5, 0.0, 0.25, 2.0, 17.0, 60.0] * 2])
    tab = np.array([[0, 5, 6, 7], [1, 2, 3, 4]], dtype=np.int32)
    for row in range(2):
        idx, w = oracle.hash_route(spec, z, tab, [row])
        assert np.array_equal(idx[0], tab[row])
        want = np.sqrt(np.logaddexp(0.0, z[0, tab[row]]))
        assert np.allclose(w[0], want, rtol=1e-14, atol=0)


def test_hash_route_normalises_to_routed_scaling():
    spec = _hash_spec(k=4, norm=True, rsf=2.5)
    rng = np.random.default_rng(1)
    z = rng.normal(size=(6, 16)) * 3
    tab = np.stack([rng.permutation(16)[:4] for _ in range(10)]).astype(np.int32)
    idx, w = oracle.hash_route(spec, z, tab, rng.integers(0, 10, size=6))
    assert np.allclose(w.sum(1), 2.5, rtol=1e-14)
    assert (w > 0).all()
    # two experts in closed form: w0 = r0 / (r0 + r1), r = sqrt(softplus(z))
    spec2 = _hash_spec(k=2, norm=True)
    idx, w = oracle.hash_route(spec2, z[:1], np.array([[3, 9]], dtype=np.int32), [0])
    r = np.sqrt(np.log1p(np.exp(z[0, [3, 9]])))
    assert np.allclose(w[0], r / r.sum(), rtol=1e-14)


def test_hash_route_drops_entries_and_tokens_out_of_range():
    """An expert id outside [0, E) gets weight 0 and the others renormalise
    among themselves; a token id outside the table drops its whole row."""
    spec = _hash_spec(k=3, norm=True)
    z = np.linspace(-2, 2, 16)[None, :].repeat(2, 0)
    tab = np.array([[2, 16, 5], [1, -1, 7]], dtype=np.int32)
    idx, w = oracle.hash_route(spec, z, tab, [0, 2])
    r = np.sqrt(np.log1p(np.exp(z[0, [2, 5]])))
    assert np.allclose(w[0], [r[0] / r.sum(), 0.0, r[1] / r.sum()], rtol=1e-14)
    assert np.array_equal(idx[1], [-1, -1, -1]) and not w[1].any()
