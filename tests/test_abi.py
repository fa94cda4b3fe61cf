"""CPU checks of the C ABI: the library loads, exports what include/moe_wave.h
declares, sizes workspaces, and rejects bad arguments with the named status
codes before touching a GPU."""
import ctypes as C
import os
import re

import pytest

import mixture_experts_decode_wave_amd as mw
import moe_synth as ms
from tests.harness import cfg_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_wave.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def _codes():
    src = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define (MOE_E\w+|MOE_OK) \(?(-?\d+)\)?", src)}


CODES = _codes()


def test_library_exports_every_declared_symbol():
    L = mw.lib()
    names = _declared()
    assert {"moe_route", "moe_experts_forward", "moe_layer_forward", "moe_layer_forward_norm",
            "moe_layer_forward_hash",
            "moe_workspace_size", "moe_strerror", "moe_last_error",
            "moe_abi_version", "moe_experts_forward_partial", "moe_shared_combine",
            "moe_probe_stream_read"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert mw.abi_version() == mw.ABI_VERSION == 5


def test_strerror_names_every_code():
    for name, code in CODES.items():
        s = mw.strerror(code)
        assert s and s != "unknown status", name
    assert mw.strerror(12345) == "unknown status"


@pytest.mark.parametrize("name", list(ms.SPECS))
def test_workspace_size_of_every_workload(name):
    spec = ms.SPECS[name]
    cfg = cfg_of(spec)
    for n in spec.ns:
        sz = mw.workspace_size(cfg, n)
        nk = n * spec.top_k
        # at least act + y in fp32
        assert sz >= nk * (spec.inter + spec.hidden) * 4
        assert sz % 256 == 0


def _bad(**kw):
    spec = ms.SPECS["qwen3_next"]
    cfg = cfg_of(spec)
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg


@pytest.mark.parametrize("field,value", [
    ("num_experts", 0), ("num_experts", 2048), ("top_k", 0), ("top_k", 33), ("hidden", 100),
    ("inter", 0), ("shared_inter", 48), ("scoring", 7), ("act_dtype", 5), ("expert_dtype", 9),
    ("norm_topk", 2), ("zero_experts", -1), ("zero_experts", 513)])
def test_workspace_size_zero_for_invalid_cfg(field, value):
    assert mw.workspace_size(_bad(**{field: value}), 4) == 0


def test_hidden_limits_per_activation_dtype():
    """The router holds at most 8 16-byte chunks of a quarter row per lane:
    h up to 16384 with bf16 activations, up to 8192 with fp32 ones."""
    f32 = cfg_of(ms.SPECS["tiny"])
    assert f32.act_dtype == mw.DT["f32"]
    for h, ok in [(8192, True), (8224, False), (16384, False)]:
        f32.hidden = h
        assert (mw.workspace_size(f32, 4) > 0) == ok, h
    bf = cfg_of(ms.SPECS["qwen3_next"])
    for h, ok in [(16384, True), (16416, False)]:
        bf.hidden = h
        assert (mw.workspace_size(bf, 4) > 0) == ok, h


def test_workspace_size_rejects_bad_rows():
    cfg = cfg_of(ms.SPECS["tiny"])
    assert mw.workspace_size(cfg, 0) == 0
    assert mw.workspace_size(cfg, 4097) == 0
    assert mw.workspace_size(cfg, 4096) > 0


def _call_route(cfg, n=4, x=256, w=512, idx=1024, tw=2048, ws=4096, ws_bytes=1 << 40, bias=None):
    L = mw.lib()
    return L.moe_route(C.byref(cfg), n, x, w, bias, None, idx, tw, ws, ws_bytes, None)


def test_route_argument_errors():
    cfg = cfg_of(ms.SPECS["qwen3_next"])
    assert _call_route(cfg, x=None) == CODES["MOE_EINVAL_NULL"]
    assert _call_route(cfg, idx=None) == CODES["MOE_EINVAL_NULL"]
    assert _call_route(cfg, ws=None) == CODES["MOE_EINVAL_NULL"]
    assert _call_route(cfg, ws=4096 + 8) == CODES["MOE_EINVAL_ALIGN"]
    assert _call_route(cfg, x=256 + 2) == CODES["MOE_EINVAL_ALIGN"]
    assert _call_route(cfg, ws_bytes=100) == CODES["MOE_EWORKSPACE"]
    assert "ws_bytes=100 < required" in mw.lib().moe_last_error().decode()
    assert _call_route(cfg, n=0) == CODES["MOE_EINVAL_SHAPE"]
    # a correction bias needs sigmoid scoring
    assert _call_route(cfg, bias=C.c_void_p(8192)) == CODES["MOE_EINVAL_DTYPE"]
    assert _call_route(_bad(top_k=600)) == CODES["MOE_EINVAL_TOPK"]
    assert _call_route(_bad(act_dtype=0)) == CODES["MOE_EINVAL_DTYPE"]
    assert "unsupported dtypes" in mw.lib().moe_last_error().decode()


def test_experts_argument_errors():
    L = mw.lib()
    spec = ms.SPECS["qwen3_next"]
    cfg = cfg_of(spec)
    tabs = mw.moe_expert_tables(4096, 4096, 4096, 4096, 4096, 4096)
    sh = mw.moe_shared_expert(4096, 4096, 4096, 4096, 4096, 4096, None)

    def call(tables=tabs, shared=sh, out=8192, cfg=cfg):
        return L.moe_experts_forward(C.byref(cfg), 4, 256, C.byref(tables),
                                     None if shared is None else C.byref(shared), 512, 1024, out,
                                     4096, 1 << 40, None)

    assert call(out=None) == CODES["MOE_EINVAL_NULL"]
    assert call(shared=None) == CODES["MOE_EINVAL_NULL"]  # shared_inter > 0 needs it
    no_scale = mw.moe_expert_tables(4096, 4096, 4096, None, None, None)
    assert call(tables=no_scale) == CODES["MOE_EINVAL_NULL"]
    assert call(out=8192 + 4) == CODES["MOE_EINVAL_ALIGN"]


def test_expert_parallel_argument_errors():
    """moe_experts_forward_partial and moe_shared_combine check their pointers
    on the host and enqueue nothing when a check fails."""
    L = mw.lib()
    cfg = cfg_of(ms.SPECS["qwen3_next"])
    tabs = mw.moe_expert_tables(4096, 4096, 4096, 4096, 4096, 4096)
    sh = mw.moe_shared_expert(4096, 4096, 4096, 4096, 4096, 4096, None)

    def part(idx=512, partial=8192, tables=tabs):
        return L.moe_experts_forward_partial(C.byref(cfg), 4, 256, C.byref(tables), idx, 1024,
                                             partial, 4096, 1 << 40, None)

    assert part(partial=None) == CODES["MOE_EINVAL_NULL"]
    assert part(idx=None) == CODES["MOE_EINVAL_NULL"]
    assert part(partial=8192 + 4) == CODES["MOE_EINVAL_ALIGN"]
    no_scale = mw.moe_expert_tables(4096, 4096, 4096, None, None, None)
    assert part(tables=no_scale) == CODES["MOE_EINVAL_NULL"]

    def comb(shared=sh, psum=8192, out=16384, c=cfg, gx=None):
        return L.moe_shared_combine(C.byref(c), 4, 256, gx,
                                    None if shared is None else C.byref(shared), psum, out,
                                    4096, 1 << 40, None)

    assert comb(shared=None) == CODES["MOE_EINVAL_NULL"]  # shared_inter > 0 needs it
    assert comb(psum=None) == CODES["MOE_EINVAL_NULL"]
    assert comb(out=None) == CODES["MOE_EINVAL_NULL"]
    assert comb(psum=8192 + 4) == CODES["MOE_EINVAL_ALIGN"]
    assert comb(gx=8192 + 8) == CODES["MOE_EINVAL_ALIGN"]
    assert comb(c=_bad(top_k=0)) == CODES["MOE_EINVAL_TOPK"]


def test_layer_norm_argument_errors():
    """moe_layer_forward_norm checks eps and the norm weights' alignment on the
    host, before anything is enqueued."""
    L = mw.lib()
    spec = ms.SPECS["qwen3_next"]
    cfg = cfg_of(spec)
    tabs = mw.moe_expert_tables(4096, 4096, 4096, 4096, 4096, 4096)
    sh = mw.moe_shared_expert(4096, 4096, 4096, 4096, 4096, 4096, None)

    def call(rw=8192, ew=8192, eps=1e-6):
        return L.moe_layer_forward_norm(C.byref(cfg), 4, 256, rw, ew, eps, 512, None,
                                        C.byref(tabs), C.byref(sh), 8192, None, None, None,
                                        4096, 1 << 40, None, None)

    assert call(eps=-1.0) == CODES["MOE_EINVAL_SHAPE"]
    assert call(eps=float("nan")) == CODES["MOE_EINVAL_SHAPE"]
    assert call(eps=2.0) == CODES["MOE_EINVAL_SHAPE"]
    assert call(rw=8194) == CODES["MOE_EINVAL_ALIGN"]
    assert call(rw=None, ew=8200) == CODES["MOE_EINVAL_ALIGN"]
    # no norm weights: eps is not looked at (the call then reaches the device)
    import torch
    if not torch.cuda.is_available():
        assert call(rw=None, ew=None, eps=-1.0) == CODES["MOE_EHIP"]


def test_layer_hash_argument_errors():
    L = mw.lib()
    spec = ms.SPECS["deepseek_v3"]
    cfg = cfg_of(spec)
    tabs = mw.moe_expert_tables(4096, 4096, 4096, 4096, 4096, 4096)
    sh = mw.moe_shared_expert(4096, 4096, 4096, 4096, 4096, 4096, None)

    def call(tok=8192, tab=8192, vocab=100):
        return L.moe_layer_forward_hash(C.byref(cfg), 4, 256, tok, tab, vocab, 512,
                                        C.byref(tabs), C.byref(sh), 8192, None, None, None,
                                        4096, 1 << 40, None, None)

    assert call(tok=None) == CODES["MOE_EINVAL_NULL"]
    assert call(tab=None) == CODES["MOE_EINVAL_NULL"]
    assert call(tab=8194) == CODES["MOE_EINVAL_ALIGN"]
    assert call(vocab=0) == CODES["MOE_EINVAL_SHAPE"]


def test_no_device_reports_hip_error():
    """With valid arguments and no GPU the first launch fails: MOE_EHIP, not a crash."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    cfg = cfg_of(ms.SPECS["tiny"])
    rc = _call_route(cfg)
    assert rc == CODES["MOE_EHIP"]
    assert mw.lib().moe_last_error().decode()


def test_stream_probe_argument_errors():
    L = mw.lib()
    assert L.moe_probe_stream_read(None, 1024, 4096, 8, None, None, None) == CODES["MOE_EINVAL_NULL"]
    assert L.moe_probe_stream_read(4096, 1024, None, 8, None, None, None) == CODES["MOE_EINVAL_NULL"]
    assert L.moe_probe_stream_read(4104, 1024, 4096, 8, None, None, None) == CODES["MOE_EINVAL_ALIGN"]
    assert L.moe_probe_stream_read(4096, 1000, 4096, 8, None, None, None) == CODES["MOE_EINVAL_ALIGN"]
    assert L.moe_probe_stream_read(4096, 1024, 4096, 0, None, None, None) == CODES["MOE_EINVAL_SHAPE"]


def test_static_entry_point_checks_before_any_hip_call():
    """moe_layer_forward_static refuses a NULL cfg and a configuration whose
    workspace exceeds its static scratch before it touches the device."""
    L = mw.lib()
    assert L.moe_layer_forward_static(None, 1, 256, 512, None, None, None, 1024, None, None,
                                      None, None, None) == CODES["MOE_EINVAL_NULL"]
    cfg = mw.make_cfg(4096, 256, 8, 1536, 1536, "softmax", True, 1.0, "bf16", "mxfp4")
    assert mw.workspace_size(cfg, 1024) > mw.STATIC_SCRATCH_BYTES
    assert L.moe_layer_forward_static(C.byref(cfg), 1024, 256, 512, None, None, None, 1024, None,
                                      None, None, None, None) == CODES["MOE_EWORKSPACE"]
    assert "static scratch holds" in L.moe_last_error().decode()


def test_zero_expert_limits():
    """Zero experts widen the router: E + Z <= 1024, top_k <= min(E + Z, 32)
    (so k may exceed the real experts); the logits and router partials in the
    workspace grow with E + Z."""
    cfg = cfg_of(ms.SPECS["zero_experts_384"])
    assert (cfg.num_experts, cfg.zero_experts) == (256, 128)
    with_z = mw.workspace_size(cfg, 16)
    cfg.zero_experts = 768
    assert mw.workspace_size(cfg, 16) > with_z
    cfg.zero_experts = 769
    assert mw.workspace_size(cfg, 16) == 0
    small = cfg_of(ms.SPECS["tiny"].with_(num_experts=4, zero_experts=4, top_k=6))
    assert mw.workspace_size(small, 4) > 0
    small.top_k = 9
    assert mw.workspace_size(small, 4) == 0


def test_zero_experts_refused_where_not_supported():
    """The expert-parallel calls and hash routing take no zero experts; the
    refusal comes before any HIP call."""
    L = mw.lib()
    cfg = cfg_of(ms.SPECS["zero_experts_384"])
    tabs = mw.moe_expert_tables(4096, 4096, 4096, 4096, 4096, 4096)
    rc = L.moe_experts_forward_partial(C.byref(cfg), 4, 256, C.byref(tabs), 1024, 2048, 8192,
                                       4096, 1 << 40, None)
    assert rc == CODES["MOE_EINVAL_SHAPE"] and "zero experts" in L.moe_last_error().decode()
    rc = L.moe_shared_combine(C.byref(cfg), 4, 256, None, None, 8192, 4096 * 4, 4096, 1 << 40,
                              None)
    assert rc == CODES["MOE_EINVAL_SHAPE"] and "zero experts" in L.moe_last_error().decode()
    rc = L.moe_layer_forward_hash(C.byref(cfg), 4, 256, 1024, 2048, 10, 512, C.byref(tabs), None,
                                  8192, None, None, None, 4096, 1 << 40, None, None)
    assert rc == CODES["MOE_EINVAL_SHAPE"] and "zero experts" in L.moe_last_error().decode()
