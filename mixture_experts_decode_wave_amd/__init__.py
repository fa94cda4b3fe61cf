"""Python binding of libmoewave.so, the gfx950 MoE decode-layer library.

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the layer runs in the library's kernels.
The names mirror the C ABI in include/moe_wave.h (moe_route,
moe_experts_forward, moe_layer_forward, moe_workspace_size, ...).  When the
library is missing this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoewave.so")

ABI_VERSION = 5  # the C ABI these bindings declare (MOE_ABI_VERSION)
MOE_OK = 0
MOE_LAYER_EVENTS = 6
STATIC_SCRATCH_BYTES = 64 << 20  # MOE_STATIC_SCRATCH_BYTES
DT = {"f32": 0, "bf16": 1, "fp8_b128": 2, "mxfp4": 3}
SCORING = {"softmax": 0, "sigmoid": 1}


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


class moe_cfg(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("num_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("shared_inter", C.c_int32), ("scoring", C.c_int32),
                ("norm_topk", C.c_int32), ("routed_scaling", C.c_float),
                ("act_dtype", C.c_int32), ("expert_dtype", C.c_int32),
                ("zero_experts", C.c_int32)]


class moe_expert_tables(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("gate", "up", "down", "gate_scale", "up_scale",
                                            "down_scale")]


class moe_shared_expert(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("gate", "up", "down", "gate_scale", "up_scale",
                                            "down_scale", "gate_vec")]


_lib = None


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build() or "
                               "python mixture_experts_decode_wave_amd/build.py)")
        L = C.CDLL(LIB_PATH)
        vp, i32, cfgp = C.c_void_p, C.c_int32, C.POINTER(moe_cfg)
        L.moe_workspace_size.restype = C.c_size_t
        L.moe_workspace_size.argtypes = [cfgp, i32]
        L.moe_route.restype = C.c_int
        L.moe_route.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.moe_experts_forward.restype = C.c_int
        L.moe_experts_forward.argtypes = [cfgp, i32, vp, C.POINTER(moe_expert_tables),
                                          C.POINTER(moe_shared_expert), vp, vp, vp, vp,
                                          C.c_size_t, vp]
        L.moe_experts_forward_partial.restype = C.c_int
        L.moe_experts_forward_partial.argtypes = [cfgp, i32, vp, C.POINTER(moe_expert_tables),
                                                  vp, vp, vp, vp, C.c_size_t, vp]
        L.moe_shared_combine.restype = C.c_int
        L.moe_shared_combine.argtypes = [cfgp, i32, vp, vp, C.POINTER(moe_shared_expert), vp,
                                         vp, vp, C.c_size_t, vp]
        L.moe_layer_forward.restype = C.c_int
        L.moe_layer_forward.argtypes = [cfgp, i32, vp, vp, vp, C.POINTER(moe_expert_tables),
                                        C.POINTER(moe_shared_expert), vp, vp, vp, vp, vp,
                                        C.c_size_t, vp, vp]
        L.moe_layer_forward_static.restype = C.c_int
        L.moe_layer_forward_static.argtypes = [cfgp, i32, vp, vp, vp,
                                               C.POINTER(moe_expert_tables),
                                               C.POINTER(moe_shared_expert), vp, vp, vp, vp, vp,
                                               vp]
        L.moe_layer_forward_norm.restype = C.c_int
        L.moe_layer_forward_norm.argtypes = [cfgp, i32, vp, vp, vp, C.c_float, vp, vp,
                                             C.POINTER(moe_expert_tables),
                                             C.POINTER(moe_shared_expert), vp, vp, vp, vp, vp,
                                             C.c_size_t, vp, vp]
        L.moe_layer_forward_hash.restype = C.c_int
        L.moe_layer_forward_hash.argtypes = [cfgp, i32, vp, vp, vp, i32, vp,
                                             C.POINTER(moe_expert_tables),
                                             C.POINTER(moe_shared_expert), vp, vp, vp, vp, vp,
                                             C.c_size_t, vp, vp]
        L.moe_probe_stream_read.restype = C.c_int
        L.moe_probe_stream_read.argtypes = [vp, C.c_size_t, vp, i32, vp, vp, vp]
        L.moe_strerror.restype = C.c_char_p
        L.moe_strerror.argtypes = [C.c_int]
        L.moe_last_error.restype = C.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_abi_version.restype = C.c_int
        L.moe_abi_version.argtypes = []
        if L.moe_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has C ABI version {L.moe_abi_version()}, these "
                               f"bindings declare {ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def _check(rc: int):
    if rc != MOE_OK:
        L = lib()
        raise MoeError(rc, f"{L.moe_strerror(rc).decode()}: {L.moe_last_error().decode()}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return C.c_void_p(int(stream))


def make_cfg(hidden: int, num_experts: int, top_k: int, inter: int, shared_inter: int = 0,
             scoring: str = "softmax", norm_topk: bool = True, routed_scaling: float = 1.0,
             act_dtype: str = "bf16", expert_dtype: str = "bf16",
             zero_experts: int = 0) -> moe_cfg:
    return moe_cfg(hidden, num_experts, top_k, inter, shared_inter, SCORING[scoring],
                   int(bool(norm_topk)), float(routed_scaling), DT[act_dtype], DT[expert_dtype],
                   int(zero_experts))


class ExpertTables:
    """Device pointer tables of E routed experts (the moe_expert_tables struct)."""

    def __init__(self, gate: Sequence[int], up: Sequence[int], down: Sequence[int],
                 gate_scale=None, up_scale=None, down_scale=None, device="cuda", keep=()):
        def tab(ptrs):
            if ptrs is None:
                return None
            return torch.tensor([int(p) for p in ptrs], dtype=torch.int64, device=device)
        self.tabs = [tab(t) for t in (gate, up, down, gate_scale, up_scale, down_scale)]
        self.keep = list(keep)
        self.struct = moe_expert_tables(*[None if t is None else t.data_ptr() for t in self.tabs])

    @classmethod
    def from_stacked(cls, gate: torch.Tensor, up: torch.Tensor, down: torch.Tensor,
                     gate_scale=None, up_scale=None, down_scale=None) -> "ExpertTables":
        """Tables over [E, ...] stacked device tensors (one expert per leading index)."""
        def ptrs(t):
            if t is None:
                return None
            stride = t.stride(0) * t.element_size()
            return [t.data_ptr() + e * stride for e in range(t.shape[0])]
        return cls(ptrs(gate), ptrs(up), ptrs(down), ptrs(gate_scale), ptrs(up_scale),
                   ptrs(down_scale), device=gate.device,
                   keep=[gate, up, down, gate_scale, up_scale, down_scale])


class SharedExpert:
    """The moe_shared_expert struct over device tensors."""

    def __init__(self, gate, up, down, gate_scale=None, up_scale=None, down_scale=None,
                 gate_vec=None):
        self.keep = [gate, up, down, gate_scale, up_scale, down_scale, gate_vec]
        self.struct = moe_shared_expert(*[None if t is None else t.data_ptr() for t in self.keep])


def abi_version() -> int:
    return lib().moe_abi_version()


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def workspace_size(cfg: moe_cfg, n_rows: int) -> int:
    return int(lib().moe_workspace_size(C.byref(cfg), n_rows))


def alloc_workspace(cfg: moe_cfg, n_rows: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (the library needs it zeroed once; calls keep it so)."""
    n = workspace_size(cfg, n_rows)
    if n == 0:
        raise MoeError(-2, "invalid configuration for a workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_route(cfg, x, router_w, corr_bias, topk_idx, topk_w, ws, logits=None, stream=None):
    n = x.shape[0]
    _check(lib().moe_route(C.byref(cfg), n, _p(x), _p(router_w), _p(corr_bias), _p(logits),
                           _p(topk_idx), _p(topk_w), _p(ws), ws.numel(), _stream(stream)))


def moe_experts_forward(cfg, x, experts: ExpertTables, shared: Optional[SharedExpert],
                        topk_idx, topk_w, out, ws, stream=None):
    n = x.shape[0]
    _check(lib().moe_experts_forward(C.byref(cfg), n, _p(x), C.byref(experts.struct),
                                     None if shared is None else C.byref(shared.struct),
                                     _p(topk_idx), _p(topk_w), _p(out), _p(ws), ws.numel(),
                                     _stream(stream)))


def moe_experts_forward_partial(cfg, x, experts: ExpertTables, topk_idx, topk_w, partial, ws,
                                stream=None):
    """One expert-parallel rank's routed experts into an fp32 partial [N, h]."""
    n = x.shape[0]
    _check(lib().moe_experts_forward_partial(C.byref(cfg), n, _p(x), C.byref(experts.struct),
                                             _p(topk_idx), _p(topk_w), _p(partial), _p(ws),
                                             ws.numel(), _stream(stream)))


def moe_shared_combine(cfg, x, shared: Optional[SharedExpert], partial_sum, out, ws,
                       gate_x=None, stream=None):
    """out = partial_sum + g * shared(x), rounded once to the act dtype; the
    shared-expert gate reads gate_x (None: x)."""
    n = x.shape[0]
    _check(lib().moe_shared_combine(C.byref(cfg), n, _p(x), _p(gate_x),
                                    None if shared is None else C.byref(shared.struct),
                                    _p(partial_sum), _p(out), _p(ws), ws.numel(),
                                    _stream(stream)))


def moe_layer_forward(cfg, x, router_w, corr_bias, experts: ExpertTables,
                      shared: Optional[SharedExpert], out, ws, logits=None, topk_idx=None,
                      topk_w=None, stream=None, stage_events=None):
    """stage_events: None or a ctypes array of MOE_LAYER_EVENTS hipEvent_t handles."""
    n = x.shape[0]
    _check(lib().moe_layer_forward(C.byref(cfg), n, _p(x), _p(router_w), _p(corr_bias),
                                   C.byref(experts.struct),
                                   None if shared is None else C.byref(shared.struct),
                                   _p(out), _p(logits), _p(topk_idx), _p(topk_w), _p(ws),
                                   ws.numel(), _stream(stream), stage_events))


def moe_layer_forward_static(cfg, x, router_w, corr_bias, experts: ExpertTables,
                             shared: Optional[SharedExpert], out, logits=None, topk_idx=None,
                             topk_w=None, stream=None, stage_events=None):
    """moe_layer_forward on the library's static per-GPU workspace (no
    workspace argument; calls that overlap on one GPU race)."""
    n = x.shape[0]
    _check(lib().moe_layer_forward_static(C.byref(cfg), n, _p(x), _p(router_w), _p(corr_bias),
                                          C.byref(experts.struct),
                                          None if shared is None else C.byref(shared.struct),
                                          _p(out), _p(logits), _p(topk_idx), _p(topk_w),
                                          _stream(stream), stage_events))


def moe_layer_forward_norm(cfg, x, router_norm_w, expert_norm_w, eps, router_w, corr_bias,
                           experts: ExpertTables, shared: Optional[SharedExpert], out, ws,
                           logits=None, topk_idx=None, topk_w=None, stream=None,
                           stage_events=None):
    """moe_layer_forward with the layer's pre-norms (either weight may be None)."""
    n = x.shape[0]
    _check(lib().moe_layer_forward_norm(C.byref(cfg), n, _p(x), _p(router_norm_w),
                                        _p(expert_norm_w), float(eps), _p(router_w),
                                        _p(corr_bias), C.byref(experts.struct),
                                        None if shared is None else C.byref(shared.struct),
                                        _p(out), _p(logits), _p(topk_idx), _p(topk_w), _p(ws),
                                        ws.numel(), _stream(stream), stage_events))


def moe_layer_forward_hash(cfg, x, token_ids, tid2eid, router_w, experts: ExpertTables,
                           shared: Optional[SharedExpert], out, ws, logits=None, topk_idx=None,
                           topk_w=None, stream=None, stage_events=None):
    """moe_layer_forward with hash routing (token_ids [N], tid2eid [vocab, k], int32)."""
    n = x.shape[0]
    _check(lib().moe_layer_forward_hash(C.byref(cfg), n, _p(x), _p(token_ids), _p(tid2eid),
                                        int(tid2eid.shape[0]), _p(router_w),
                                        C.byref(experts.struct),
                                        None if shared is None else C.byref(shared.struct),
                                        _p(out), _p(logits), _p(topk_idx), _p(topk_w), _p(ws),
                                        ws.numel(), _stream(stream), stage_events))


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, grid: int = 2048, stream=None,
                      ev0=None, ev1=None):
    """One read-only pass over buf (zero-filled device tensor) by the
    library's streaming-read probe kernel (a measurement aid, not a step of
    the layer); sink: int32 device tensor of grid * 256 entries."""
    _check(lib().moe_probe_stream_read(_p(buf), buf.numel() * buf.element_size(), _p(sink),
                                       grid, _stream(stream), ev0, ev1))
