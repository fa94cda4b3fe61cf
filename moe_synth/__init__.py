"""Seeded synthetic inputs for the MoE decode layer.

This module only draws random numbers and stores them in the weight formats the
layer reads (fp32, bf16, FP8-e4m3 with fp32 128x128 block scales, MXFP4 with
e8m0 scales per 32 elements).  It holds none of the layer's arithmetic: no
router product, no scoring, no expert MLP and no decoding of the stored codes.
Both the fp64 oracle and the HIP library are fed from the same bytes made here.

The five workloads follow the layer shapes the pages' MoE decode serves
(forward.rs / forward_token_major.rs config fields: hidden_size,
moe_intermediate_size, shared_expert_intermediate_size, num_experts,
num_experts_per_tok, norm_topk_prob, routed_scaling_factor):

* ``tiny``          h256,  E8,   k2,  I128,  fp32,        softmax+norm
* ``qwen3_30b_a3b`` h2048, E128, k8,  I768,  bf16,        softmax+norm
* ``qwen3_next``    h2048, E512, k10, I512,  fp8 b128,    softmax+norm, shared 512
* ``deepseek_v3``   h7168, E256, k8,  I2048, fp8 b128,    sigmoid+bias, norm, rsf 2.5, shared 2048
* ``verify_mxfp4``  h4096, E256, k8,  I1536, MXFP4,       softmax+norm, shared 1536
* ``zero_experts_384`` h2048, E256 + 128 zero experts (a 384-wide router), k8, I768,
                    bf16, softmax+norm

Distributions: x ~ N(0,1); router rows ~ N(0, (m/sqrt(h))^2) with m = 2 for
qwen3_30b_a3b (logits ~ N(0,2)) and 1 otherwise; gate/up ~ N(0, 1/h),
down ~ N(0, 1/I) (fan-in scaling) before quantisation; correction bias
~ U(-0.1, 0.1) fp32.  x is drawn once as 256 rows and a step of N rows takes
the first N, so every N of a workload shares its rows.

Random draws use torch generators seeded per (workload, tensor kind, expert).
The values depend on the device the draw runs on (CPU and GPU generators
differ), which is harmless: each comparison feeds both sides the same bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

X_ROWS = 256

# tensor kinds for seeding
_K_X, _K_ROUTER, _K_BIAS, _K_GATE, _K_UP, _K_DOWN, _K_SGATE = range(7)
_SHARED_ID = 1 << 20


@dataclass(frozen=True)
class LayerSpec:
    name: str
    index: int                 # 1-based workload number, part of every seed
    hidden: int
    num_experts: int
    top_k: int
    inter: int
    shared_inter: int          # 0 = no shared expert
    scoring: str               # "softmax" | "sigmoid"
    norm_topk: bool
    routed_scaling: float
    act_dtype: str             # "f32" | "bf16"   (x, router, out)
    expert_dtype: str          # "f32" | "bf16" | "fp8_b128" | "mxfp4"
    router_std_mult: float = 1.0
    corr_bias: bool = False
    shared_gate: bool = False  # sigmoid gate vector on the shared expert
    ns: tuple = (1,)
    zero_experts: int = 0      # zero-computation experts: router columns E .. E+Z-1

    def with_(self, **kw) -> "LayerSpec":
        return replace(self, **kw)

    @property
    def router_width(self) -> int:
        """Router rows (= logits per token row): E real experts, then Z zero experts."""
        return self.num_experts + self.zero_experts


SPECS = {
    "tiny": LayerSpec("tiny", 1, 256, 8, 2, 128, 0, "softmax", True, 1.0,
                      "f32", "f32", ns=(1,)),
    "qwen3_30b_a3b": LayerSpec("qwen3_30b_a3b", 2, 2048, 128, 8, 768, 0, "softmax",
                               True, 1.0, "bf16", "bf16", router_std_mult=2.0,
                               ns=(1, 4)),
    "qwen3_next": LayerSpec("qwen3_next", 3, 2048, 512, 10, 512, 512, "softmax",
                            True, 1.0, "bf16", "fp8_b128", ns=(1, 4, 16)),
    "deepseek_v3": LayerSpec("deepseek_v3", 4, 7168, 256, 8, 2048, 2048, "sigmoid",
                             True, 2.5, "bf16", "fp8_b128", corr_bias=True,
                             ns=(1, 16, 64)),
    "verify_mxfp4": LayerSpec("verify_mxfp4", 5, 4096, 256, 8, 1536, 1536, "softmax",
                              True, 1.0, "bf16", "mxfp4", ns=(256,)),
    # the Qwen3-Next-shaped layer with a sigmoid gate on its shared expert (the
    # same weights as qwen3_next, plus the gate vector)
    "qwen3_next_gated": LayerSpec("qwen3_next_gated", 3, 2048, 512, 10, 512, 512, "softmax",
                                  True, 1.0, "bf16", "fp8_b128", shared_gate=True,
                                  ns=(1, 4, 16)),
    # a router 384 wide over 256 real experts and 128 zero-computation experts
    # (the zero-expert MoE the forward_token_major.rs page refuses to route)
    "zero_experts_384": LayerSpec("zero_experts_384", 6, 2048, 256, 8, 768, 0, "softmax",
                                  True, 1.0, "bf16", "bf16", zero_experts=128, ns=(1, 4, 16)),
}


def _seed(spec_index: int, base: int, kind: int, expert: int) -> int:
    # distinct, stable 63-bit seeds per tensor
    s = (base * 1_000_003 + spec_index) * 1_000_033 + kind
    s = s * 2_000_003 + expert
    return s & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std, device, seed):
    return torch.randn(shape, generator=_gen(device, seed), device=device,
                       dtype=torch.float32) * std


# --------------------------------------------------------------------------
# storage encodings (generator side only; decoding belongs to each consumer)
# --------------------------------------------------------------------------

def quant_fp8_b128(w: torch.Tensor):
    """fp32 [R, C] -> (e4m3fn codes u8 [R, C], fp32 scales [ceil(R/128), ceil(C/128)]).

    Per 128x128 block: s = amax / 448 (1 for an all-zero block),
    code = round-to-nearest-even(w / s) clamped to +-448 (OCP E4M3 'fn')."""
    R, C = w.shape
    br, bc = -(-R // 128), -(-C // 128)
    wp = torch.zeros(br * 128, bc * 128, dtype=torch.float32, device=w.device)
    wp[:R, :C] = w
    blk = wp.view(br, 128, bc, 128)
    amax = blk.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / s[:, None, :, None]).clamp_(-448.0, 448.0)
    q = q.view(br * 128, bc * 128)[:R, :C].contiguous()
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s.contiguous()


_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e2m1_codes(v: torch.Tensor) -> torch.Tensor:
    """Round |v| (already scaled, any size) to the e2m1 grid {0,.5,1,1.5,2,3,4,6}
    with ties to the even code and saturation at 6; returns 4-bit codes
    (sign in bit 3)."""
    a = v.abs().clamp(max=6.0)
    mids = torch.tensor(_E2M1_MIDS, dtype=torch.float32, device=v.device)
    i = torch.bucketize(a, mids, right=False)          # mids[i-1] < a <= mids[i]
    tie = (i < 7) & (a == mids[i.clamp(max=6)])
    i = torch.where(tie & (i % 2 == 1), i + 1, i)
    sign = (v < 0) | ((v == 0) & torch.signbit(v))
    return (i | (sign.to(torch.int64) << 3)).to(torch.uint8)


def quant_mxfp4(w: torch.Tensor):
    """fp32 [R, C] (C % 32 == 0) -> (packed u8 [R, C/2], e8m0 scales u8 [R, C/32]).

    OCP MX v1.0: per 32 consecutive elements of a row the shared exponent is
    floor(log2(amax)) - 2 (emax of e2m1), biased by 127 and clamped to [0, 254]
    (127 for an all-zero block); each element is w / 2^(E-127) rounded to e2m1
    (ties to even, saturating).  Element 2i sits in the low nibble of byte i."""
    R, C = w.shape
    assert C % 32 == 0
    blk = w.view(R, C // 32, 32)
    amax = blk.abs().amax(dim=-1)
    e = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax))))
    E = torch.where(amax > 0, e - 2 + 127, torch.full_like(e, 127.0)).clamp_(0, 254)
    scale = torch.exp2(E - 127.0)
    codes = _e2m1_codes(blk / scale[..., None]).view(R, C)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
    return packed, E.to(torch.uint8).contiguous()


def tile_16x64(t: torch.Tensor) -> torch.Tensor:
    """The storage layout of every expert matrix: a row-major [R, C'] tensor
    (R % 16 == 0, rows of rb bytes, rb % 16 == 0) rearranged, byte for byte,
    into tiles of 16 rows x 64 bytes.  Row group g (rows 16 g .. 16 g + 15) is
    16 rb contiguous bytes: tile column t holds bytes [64 t, 64 t + 64) of the
    group's 16 rows, row after row, tile columns in order; when rb % 64 != 0
    the last tile column is 16 rows x (rb % 64) bytes.  Shape and dtype are
    kept; only the order of the bytes changes."""
    R = t.shape[0]
    b = t.contiguous().view(torch.uint8).reshape(R, -1)
    rb = b.shape[1]
    assert R % 16 == 0 and rb % 16 == 0, (R, rb)
    full, rem = divmod(rb, 64)
    g = b.reshape(R // 16, 16, rb)
    parts = []
    if full:
        parts.append(g[:, :, :64 * full].reshape(R // 16, 16, full, 64).permute(0, 2, 1, 3)
                     .reshape(R // 16, full * 1024))
    if rem:
        parts.append(g[:, :, 64 * full:].reshape(R // 16, 16 * rem))
    out = torch.cat(parts, 1).reshape(R, rb).contiguous()
    return out.view(t.dtype).reshape(t.shape)


def encode_rowmajor(w: torch.Tensor, fmt: str):
    """fp32 [R, C] -> (weight codes in plain row-major order, scales or None)."""
    if fmt == "f32":
        return w.contiguous(), None
    if fmt == "bf16":
        return w.to(torch.bfloat16).contiguous(), None
    if fmt == "fp8_b128":
        return quant_fp8_b128(w)
    if fmt == "mxfp4":
        return quant_mxfp4(w)
    raise ValueError(fmt)


def encode(w: torch.Tensor, fmt: str):
    """fp32 [R, C] -> (stored weight tensor in the tiled layout, stored scale
    tensor or None).  Scales stay row-major."""
    codes, scales = encode_rowmajor(w, fmt)
    return tile_16x64(codes), scales


def stored_shape(fmt: str, rows: int, cols: int):
    """(weight shape, weight dtype, scale shape or None, scale dtype or None);
    the weight bytes are in the tiled layout of tile_16x64."""
    if fmt == "f32":
        return (rows, cols), torch.float32, None, None
    if fmt == "bf16":
        return (rows, cols), torch.bfloat16, None, None
    if fmt == "fp8_b128":
        return (rows, cols), torch.uint8, (-(-rows // 128), -(-cols // 128)), torch.float32
    if fmt == "mxfp4":
        return (rows, cols // 2), torch.uint8, (rows, cols // 32), torch.uint8
    raise ValueError(fmt)


def act_torch_dtype(act: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[act]


# --------------------------------------------------------------------------
# a whole layer
# --------------------------------------------------------------------------

@dataclass
class Matrix:
    """E stacked matrices of one kind in storage format: w [E, ...], s [E, ...] or None."""
    w: torch.Tensor
    s: Optional[torch.Tensor]


@dataclass
class LayerInputs:
    spec: LayerSpec
    x: torch.Tensor                   # [X_ROWS, h] act dtype
    router: torch.Tensor              # [E + Z, h] act dtype (Z zero experts)
    bias: Optional[torch.Tensor]      # [E + Z] fp32
    gate: Matrix                      # [E, I, h]
    up: Matrix                        # [E, I, h]
    down: Matrix                      # [E, h, I]
    sh_gate: Optional[Matrix] = None  # [1, I_s, h]
    sh_up: Optional[Matrix] = None
    sh_down: Optional[Matrix] = None  # [1, h, I_s]
    sgate: Optional[torch.Tensor] = None  # [h] act dtype
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def device(self):
        return self.x.device


def _stack(fmt, E, rows, cols, device):
    ws, wdt, ss, sdt = stored_shape(fmt, rows, cols)
    w = torch.empty((E,) + ws, dtype=wdt, device=device)
    s = torch.empty((E,) + ss, dtype=sdt, device=device) if ss is not None else None
    return Matrix(w, s)


def _fill(m: Matrix, e: int, fmt: str, dense: torch.Tensor):
    w, s = encode(dense, fmt)
    m.w[e].copy_(w)
    if m.s is not None:
        m.s[e].copy_(s)


def make_layer(spec: LayerSpec | str, seed: int = 0, device="cpu",
               gate_fn=None) -> LayerInputs:
    """Draw every tensor of one layer on ``device``.

    ``gate_fn(kind, e, rows, cols, device)`` may return a dense fp32 matrix to
    use instead of a random draw (kind in "gate"/"up"/"down"/"sh_gate"/...);
    tests use it to plant constructed experts."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    h, E, I, Is = spec.hidden, spec.num_experts, spec.inter, spec.shared_inter
    adt = act_torch_dtype(spec.act_dtype)
    fmt = spec.expert_dtype
    si = spec.index

    x = _randn((X_ROWS, h), 1.0, device, _seed(si, seed, _K_X, 0)).to(adt)
    EW = spec.router_width
    router = _randn((EW, h), spec.router_std_mult / math.sqrt(h), device,
                    _seed(si, seed, _K_ROUTER, 0)).to(adt)
    bias = None
    if spec.corr_bias:
        g = _gen(device, _seed(si, seed, _K_BIAS, 0))
        bias = (torch.rand(EW, generator=g, device=device, dtype=torch.float32) * 0.2 - 0.1)

    def dense(kind_name, kind, e, rows, cols, fan_in):
        if gate_fn is not None:
            d = gate_fn(kind_name, e, rows, cols, device)
            if d is not None:
                return d.to(device=device, dtype=torch.float32)
        return _randn((rows, cols), 1.0 / math.sqrt(fan_in), device, _seed(si, seed, kind, e))

    gate, up, down = _stack(fmt, E, I, h, device), _stack(fmt, E, I, h, device), _stack(fmt, E, h, I, device)
    for e in range(E):
        _fill(gate, e, fmt, dense("gate", _K_GATE, e, I, h, h))
        _fill(up, e, fmt, dense("up", _K_UP, e, I, h, h))
        _fill(down, e, fmt, dense("down", _K_DOWN, e, h, I, I))
    li = LayerInputs(spec, x, router, bias, gate, up, down, seed=seed)
    if Is > 0:
        li.sh_gate, li.sh_up, li.sh_down = (_stack(fmt, 1, Is, h, device), _stack(fmt, 1, Is, h, device),
                                            _stack(fmt, 1, h, Is, device))
        _fill(li.sh_gate, 0, fmt, dense("sh_gate", _K_GATE, _SHARED_ID, Is, h, h))
        _fill(li.sh_up, 0, fmt, dense("sh_up", _K_UP, _SHARED_ID, Is, h, h))
        _fill(li.sh_down, 0, fmt, dense("sh_down", _K_DOWN, _SHARED_ID, h, Is, Is))
    if spec.shared_gate:
        li.sgate = _randn((h,), 1.0 / math.sqrt(h), device, _seed(si, seed, _K_SGATE, 0)).to(adt)
    return li


def with_x(li: LayerInputs, x: torch.Tensor) -> LayerInputs:
    """Same weights, other token rows."""
    return replace(li, x=x)


# RMSNorm epsilon of the pre-norms (the Qwen3 and DeepSeek-V3 layers use 1e-6)
NORM_EPS = 1e-6
_K_RNORM, _K_ENORM = 7, 8


def make_norms(spec: LayerSpec, seed: int = 0, device="cpu"):
    """Weights of the router pre-norm and of the pre-expert norm, [h] each in
    the activation dtype: 1 + N(0, 0.1^2), as trained RMSNorm weights sit near 1."""
    adt = act_torch_dtype(spec.act_dtype)
    return tuple((1.0 + _randn((spec.hidden,), 0.1, device, _seed(spec.index, seed, k, 0))).to(adt)
                 for k in (_K_RNORM, _K_ENORM))


def make_hash_table(spec: LayerSpec, vocab: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """A static token-to-experts table for hash routing: [vocab, k] int32,
    each row k distinct experts drawn uniformly."""
    g = torch.Generator().manual_seed(_seed(spec.index, seed, 9, 0))
    keys = torch.rand(vocab, spec.num_experts, generator=g)
    return keys.argsort(dim=1)[:, :spec.top_k].to(torch.int32).contiguous().to(device)


def make_token_ids(n: int, vocab: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """n token ids drawn uniformly from [0, vocab), int32."""
    g = torch.Generator().manual_seed(_seed(0, seed, 10, n))
    return torch.randint(0, vocab, (n,), generator=g, dtype=torch.int32).to(device)


def fresh_x(li: LayerInputs, seed: int) -> torch.Tensor:
    """Another [X_ROWS, h] batch of tokens for the same layer."""
    adt = act_torch_dtype(li.spec.act_dtype)
    return _randn((X_ROWS, li.spec.hidden), 1.0, li.device,
                  _seed(li.spec.index, seed, _K_X, 1)).to(adt)


def to_device(li: LayerInputs, device) -> LayerInputs:
    def mv(m):
        if m is None:
            return None
        return Matrix(m.w.to(device), None if m.s is None else m.s.to(device))
    return LayerInputs(li.spec, li.x.to(device), li.router.to(device),
                       None if li.bias is None else li.bias.to(device),
                       mv(li.gate), mv(li.up), mv(li.down), mv(li.sh_gate), mv(li.sh_up),
                       mv(li.sh_down), None if li.sgate is None else li.sgate.to(device),
                       seed=li.seed)


def expert_bytes(spec: LayerSpec, inter: Optional[int] = None) -> int:
    """Stored bytes (weights + scales) of one expert's gate, up and down."""
    I = spec.inter if inter is None else inter
    tot = 0
    for rows, cols in ((I, spec.hidden), (I, spec.hidden), (spec.hidden, I)):
        ws, wdt, ss, sdt = stored_shape(spec.expert_dtype, rows, cols)
        tot += math.prod(ws) * torch.tensor([], dtype=wdt).element_size()
        if ss is not None:
            tot += math.prod(ss) * torch.tensor([], dtype=sdt).element_size()
    return tot


def gate_up_bytes(spec: LayerSpec, inter: Optional[int] = None) -> int:
    I = spec.inter if inter is None else inter
    tot = 0
    for rows, cols in ((I, spec.hidden), (I, spec.hidden)):
        ws, wdt, ss, sdt = stored_shape(spec.expert_dtype, rows, cols)
        tot += math.prod(ws) * torch.tensor([], dtype=wdt).element_size()
        if ss is not None:
            tot += math.prod(ss) * torch.tensor([], dtype=sdt).element_size()
    return tot
