"""fp64 CPU oracle of the MoE decode layer (ctypes wrapper around moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users.  The HIP library never imports, links or
calls it, and it never imports the HIP library.

The C file computes the layer as the forward.rs / forward_token_major.rs pages
describe it (router gate product, scored top-k, expert gate+up, act(gate)*up,
down, weighted-sum blend with an optional sigmoid-gated shared expert), in
double precision from the exact stored input bytes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

FMT = {"f32": 0, "bf16": 1, "fp8_b128": 2, "mxfp4": 3}
SCORING = {"softmax": 0, "sigmoid": 1}


def build() -> str:
    """Compile moe_oracle.c with gcc (OpenMP over the output elements of each product)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-Wno-unused-parameter", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Cfg(C.Structure):
    _fields_ = [("hidden", C.c_int), ("num_experts", C.c_int), ("top_k", C.c_int),
                ("inter", C.c_int), ("shared_inter", C.c_int), ("scoring", C.c_int),
                ("norm_topk", C.c_int), ("routed_scaling", C.c_double),
                ("act_fmt", C.c_int), ("expert_fmt", C.c_int), ("zero_experts", C.c_int)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        vp, ip, dp = C.c_void_p, C.c_int, C.POINTER(C.c_double)
        L.orc_bf16.restype = C.c_double
        L.orc_bf16.argtypes = [C.c_uint16]
        for n in ("orc_fp8_e4m3", "orc_e2m1", "orc_e8m0"):
            getattr(L, n).restype = C.c_double
            getattr(L, n).argtypes = [C.c_uint8]
        L.orc_dequant.argtypes = [ip, ip, ip, vp, vp, vp]
        L.orc_router_logits.argtypes = [ip, ip, ip, ip, vp, vp, vp]
        L.orc_keys.argtypes = [ip, ip, vp, vp, vp]
        L.orc_topk_row.argtypes = [ip, ip, ip, ip, C.c_double, vp, vp, vp, vp]
        L.orc_route_weights.argtypes = [ip, ip, ip, ip, C.c_double, vp, vp, vp]
        L.orc_expert_mlp.argtypes = [ip, ip, ip, vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_experts.argtypes = [vp, ip, vp] + [vp] * 6 + [vp] * 6 + [vp, vp, vp, vp, vp, ip]
        L.orc_rmsnorm.argtypes = [ip, ip, ip, vp, vp, C.c_double, vp]
        L.orc_hash_route_row.argtypes = [ip, ip, ip, C.c_double, vp, vp, vp]
        L.orc_max_threads.restype = ip
        _lib = L
    return _lib


def max_threads() -> int:
    return lib().orc_max_threads()


# ------------------------------------------------------------------ helpers

def _cpu(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(t))
    return t.detach().to("cpu").contiguous()


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def cfg_of(spec) -> _Cfg:
    return _Cfg(spec.hidden, spec.num_experts, spec.top_k, spec.inter, spec.shared_inter,
                SCORING[spec.scoring], int(spec.norm_topk), float(spec.routed_scaling),
                FMT[spec.act_dtype], FMT[spec.expert_dtype], _zero(spec))


def _zero(spec) -> int:
    return int(getattr(spec, "zero_experts", 0))


def _width(spec) -> int:
    """Router rows: the E real experts, then the Z zero-computation experts."""
    return spec.num_experts + _zero(spec)


# ------------------------------------------------------------------ decoders

def decode_bf16(bits) -> np.ndarray:
    return np.array([lib().orc_bf16(int(b)) for b in np.asarray(bits).ravel()])


def decode_fp8_e4m3(codes) -> np.ndarray:
    return np.array([lib().orc_fp8_e4m3(int(b)) for b in np.asarray(codes).ravel()])


def decode_e2m1(nibbles) -> np.ndarray:
    return np.array([lib().orc_e2m1(int(b)) for b in np.asarray(nibbles).ravel()])


def decode_e8m0(codes) -> np.ndarray:
    return np.array([lib().orc_e8m0(int(b)) for b in np.asarray(codes).ravel()])


def dequant(fmt: str, rows: int, cols: int, w, s=None) -> np.ndarray:
    """Stored [rows, cols] matrix (+ scales) -> float64 [rows, cols]."""
    w, s = _cpu(w), _cpu(s)
    out = np.empty((rows, cols), dtype=np.float64)
    rc = lib().orc_dequant(FMT[fmt], rows, cols, _ptr(w), _ptr(s), out.ctypes.data)
    if rc:
        raise ValueError("orc_dequant failed")
    return out


# ------------------------------------------------------------------ router

def router_logits(spec, x, router_w) -> np.ndarray:
    x, router_w = _cpu(x), _cpu(router_w)
    N = x.shape[0]
    out = np.empty((N, _width(spec)), dtype=np.float64)
    lib().orc_router_logits(FMT[spec.act_dtype], N, spec.hidden, _width(spec),
                            _ptr(x), _ptr(router_w), out.ctypes.data)
    return out


def keys(spec, logits: np.ndarray, bias=None) -> np.ndarray:
    """Selection keys, row by row ([N, E] float64)."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    b = _cpu(bias)
    out = np.empty_like(logits)
    for t in range(logits.shape[0]):
        lib().orc_keys(_width(spec), SCORING[spec.scoring],
                       logits[t].ctypes.data, _ptr(b), out[t].ctypes.data)
    return out


def topk(spec, logits: np.ndarray, bias=None):
    """(idx [N,k] int32, w [N,k] float64) from float64 logits [N,E]."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    b = _cpu(bias)
    N, k = logits.shape[0], spec.top_k
    idx = np.empty((N, k), dtype=np.int32)
    w = np.empty((N, k), dtype=np.float64)
    for t in range(N):
        rc = lib().orc_topk_row(_width(spec), k, SCORING[spec.scoring], int(spec.norm_topk),
                                float(spec.routed_scaling), logits[t].ctypes.data, _ptr(b),
                                idx[t].ctypes.data, w[t].ctypes.data)
        if rc:
            raise ValueError("orc_topk_row failed")
    return idx, w


def route_weights(spec, logits: np.ndarray, idx) -> np.ndarray:
    """Routing weights [N,k] float64 of the given picks idx [N,k] (which need
    not be the oracle's own top-k: a near-tie pick of another router is
    weighted as the scoring defines it)."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32).reshape(logits.shape[0], -1))
    N, k = idx.shape
    w = np.empty((N, k), dtype=np.float64)
    for t in range(N):
        rc = lib().orc_route_weights(logits.shape[1], k, SCORING[spec.scoring],
                                     int(spec.norm_topk), float(spec.routed_scaling),
                                     logits[t].ctypes.data, idx[t].ctypes.data, w[t].ctypes.data)
        if rc:
            raise ValueError(f"orc_route_weights failed on row {t}")
    return w


def hash_route(spec, logits: np.ndarray, tid2eid, token_ids):
    """Hash routing: (idx [N,k] int32, w [N,k] float64) for float64 logits
    [N,E], a [V, k] expert table and N token ids.  A token id outside
    [0, V) drops all of its row's routes (idx -1, w 0)."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    tab = np.ascontiguousarray(np.asarray(tid2eid, dtype=np.int32))
    tok = np.asarray(token_ids, dtype=np.int64).ravel()
    N, k = logits.shape[0], spec.top_k
    idx = np.full((N, k), -1, dtype=np.int32)
    w = np.zeros((N, k), dtype=np.float64)
    for t in range(N):
        if not 0 <= tok[t] < tab.shape[0]:
            continue
        idx[t] = tab[tok[t]]
        rc = lib().orc_hash_route_row(spec.num_experts, k, int(spec.norm_topk),
                                      float(spec.routed_scaling), logits[t].ctypes.data,
                                      idx[t].ctypes.data, w[t].ctypes.data)
        if rc:
            raise ValueError("orc_hash_route_row failed")
    return idx, w


# ------------------------------------------------------------------ experts

def expert_mlp(fmt: str, h: int, inter: int, v, wg, sg, wu, su, wd, sd) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    t = [_cpu(a) for a in (wg, sg, wu, su, wd, sd)]
    y = np.empty(h, dtype=np.float64)
    lib().orc_expert_mlp(FMT[fmt], h, inter, v.ctypes.data, *[_ptr(a) for a in t], y.ctypes.data)
    return y


class _HostExperts:
    """Host copies of the experts a routing touches, as C pointer tables."""

    def __init__(self, li, expert_ids):
        E = li.spec.num_experts
        self.keep = []
        self.tabs = {n: (C.c_void_p * E)() for n in ("g", "gs", "u", "us", "d", "ds")}
        for e in sorted(set(int(v) for v in expert_ids)):
            if not 0 <= e < E:  # a zero-computation expert has no tables
                continue
            for n, m in (("g", li.gate), ("u", li.up), ("d", li.down)):
                w = _cpu(m.w[e])
                self.keep.append(w)
                self.tabs[n][e] = w.data_ptr()
                if m.s is not None:
                    s = _cpu(m.s[e])
                    self.keep.append(s)
                    self.tabs[n + "s"][e] = s.data_ptr()
        self.sh = [None] * 6
        if li.sh_gate is not None:
            for i, m in enumerate((li.sh_gate, li.sh_up, li.sh_down)):
                w = _cpu(m.w[0])
                self.keep.append(w)
                self.sh[2 * i] = w
                if m.s is not None:
                    s = _cpu(m.s[0])
                    self.keep.append(s)
                    self.sh[2 * i + 1] = s
        self.sgate = _cpu(li.sgate)

    def args(self, has_scales):
        t = self.tabs
        tab = [t["g"], t["gs"] if has_scales else None, t["u"], t["us"] if has_scales else None,
               t["d"], t["ds"] if has_scales else None]
        return [C.cast(a, C.c_void_p) if a is not None else None for a in tab] + \
            [_ptr(a) for a in self.sh] + [_ptr(self.sgate)]


def experts(li, N: int, idx, w, nthreads: int = 0, x=None, gate_x=None) -> np.ndarray:
    """out [N, h] float64 for the first N rows of x under routing (idx, w);
    gate_x: the rows the shared-expert gate reads (default x)."""
    spec = li.spec
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32).reshape(N, spec.top_k))
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float64).reshape(N, spec.top_k))
    xs = _cpu((li.x if x is None else x)[:N])
    gx = None if gate_x is None else _cpu(gate_x[:N])
    hx = _HostExperts(li, idx.ravel())
    out = np.empty((N, spec.hidden), dtype=np.float64)
    cfg = cfg_of(spec)
    rc = lib().orc_experts(C.byref(cfg), N, _ptr(xs), *hx.args(li.gate.s is not None),
                           _ptr(gx), idx.ctypes.data, w.ctypes.data, out.ctypes.data, nthreads)
    if rc:
        raise ValueError(f"orc_experts failed ({rc})")
    return out


# ------------------------------------------------------------------ pre-norms

def round_bf16(v) -> np.ndarray:
    """float64 values -> the nearest bfloat16 values, ties to even (as float32).

    bfloat16 keeps 8 significant bits: with v = m 2^e (0.5 <= |m| < 1), the
    result is round_half_even(m 2^8) 2^(e-8).  Normal range only (the layer's
    activations never come near 2^-126 or 2^128)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8).astype(np.float32)


def round_act(spec, v) -> torch.Tensor:
    """float64 values -> a tensor in the layer's activation dtype (the normed
    rows are handed on in that dtype, as a separate norm step would store them)."""
    if spec.act_dtype == "f32":
        return torch.from_numpy(np.asarray(v, dtype=np.float64).astype(np.float32))
    return torch.from_numpy(round_bf16(v)).to(torch.bfloat16)


def rms_norm64(spec, x, w, eps: float) -> np.ndarray:
    """Unrounded RMSNorm of the rows of x with weights w (both act dtype), float64."""
    xs, ws = _cpu(x), _cpu(w)
    N, h = xs.shape
    out = np.empty((N, h), dtype=np.float64)
    rc = lib().orc_rmsnorm(FMT[spec.act_dtype], N, h, _ptr(xs), _ptr(ws), float(eps),
                           out.ctypes.data)
    if rc:
        raise ValueError(f"orc_rmsnorm failed ({rc})")
    return out


def rms_norm(spec, x, w, eps: float) -> torch.Tensor:
    """RMSNorm of the rows of x, rounded to the activation dtype (CPU tensor)."""
    return round_act(spec, rms_norm64(spec, x, w, eps))


def layer_forward(li, N: int, nthreads: int = 0, x=None, norms=None) -> dict:
    """The whole layer on the first N rows: logits, keys, idx, w and out (float64).

    norms: None, or (router_norm_w, expert_norm_w, eps) with either weight
    vector None: the router reads rmsnorm(x) with the first, the routed and
    shared experts read rmsnorm(x) with the second, and the shared-expert
    gate reads x itself."""
    spec = li.spec
    xs = _cpu((li.x if x is None else x)[:N])
    xr = xe = xs
    if norms is not None:
        rw, ew, eps = norms
        if rw is not None:
            xr = rms_norm(spec, xs, rw, eps)
        if ew is not None:
            xe = rms_norm(spec, xs, ew, eps)
    lg = router_logits(spec, xr, li.router)
    idx, w = topk(spec, lg, li.bias)
    out = experts(li, N, idx, w, nthreads=nthreads, x=xe, gate_x=xs)
    return {"logits": lg, "keys": keys(spec, lg, li.bias), "idx": idx, "w": w, "out": out}
