"""ctypes binding of libolmo3attn (C ABI in include/olmo3_attn.h).

Argument marshalling only: shapes are read off the tensors, device pointers
and the current HIP stream are passed through, and a non-zero status is
raised as ``Olmo3Error``.  Every step of the computation runs in the HIP
library; there is no fallback, and a missing library is an error.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from . import LAYER_FULL, LAYER_SLIDING  # noqa: F401  (re-exported)

# OLMO3_ATTN_LIB selects another build of the library (the host-sanitized
# one that the ABI tests run under AddressSanitizer and UBSan).
LIB_PATH = os.environ.get("OLMO3_ATTN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libolmo3attn.so")

ABI_VERSION = 11  # OLMO3_ABI_VERSION of include/olmo3_attn.h
DTYPE_BF16, DTYPE_F32, DTYPE_BF16_E4M3 = 0, 1, 2
MODE_PREFILL, MODE_DECODE = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_HIP, ERR_WORKSPACE = range(6)

# Every symbol include/olmo3_attn.h declares.
EXPORTS = (
    "olmo3_layer_type", "olmo3_workspace_bytes", "olmo3_kv_append", "olmo3_attn_prefill",
    "olmo3_attn_decode", "olmo3_status_string", "olmo3_abi_version",
    "olmo3_probe_prefill_visits", "olmo3_probe_prefill_order", "olmo3_probe_decode_reads",
    "olmo3_attn_prefill_phases",
    "olmo3_attn_decode_phases", "olmo3_attn_prefill_ragged", "olmo3_attn_decode_ragged",
    "olmo3_kv_append_e4m3", "olmo3_attn_prefill_e4m3", "olmo3_attn_decode_e4m3",
    "olmo3_attn_decode_e4m3_phases", "olmo3_attn_decode_ragged_e4m3",
    "olmo3_attn_prefill_ragged_e4m3", "olmo3_attn_decode_noalloc",
)
# Size of the library's per-device scratch array that olmo3_attn_decode_noalloc
# uses in place of a workspace (OLMO3_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 << 20
PHASE_PROLOGUE, PHASE_ATTENTION, PHASE_MERGE = 1, 2, 4
PHASES_ALL = PHASE_PROLOGUE | PHASE_ATTENTION | PHASE_MERGE


class RopeStruct(ctypes.Structure):
    """Mirror of ``olmo3_rope``."""

    _fields_ = [
        ("theta", ctypes.c_double),
        ("yarn", ctypes.c_int32),
        ("factor", ctypes.c_double),
        ("orig_ctx", ctypes.c_int64),
        ("beta_fast", ctypes.c_double),
        ("beta_slow", ctypes.c_double),
        ("attn_factor", ctypes.c_double),
    ]


@dataclass(frozen=True)
class Rope:
    """RoPE / YaRN settings; YaRN (when on) applies to full layers only."""

    theta: float = 500000.0
    yarn: bool = False
    factor: float = 8.0
    orig_ctx: int = 8192
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    attn_factor: float = 0.0

    def to_c(self) -> RopeStruct:
        return RopeStruct(self.theta, int(bool(self.yarn)), self.factor, int(self.orig_ctx),
                          self.beta_fast, self.beta_slow, self.attn_factor)


class Olmo3Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None
_i, _i64, _f, _p, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        L.olmo3_layer_type.argtypes = [_i, _i]
        L.olmo3_layer_type.restype = _i
        L.olmo3_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _i64]
        L.olmo3_workspace_bytes.restype = _sz
        L.olmo3_kv_append.argtypes = [_i, _i, _i, _i, _i, _i, ctypes.POINTER(RopeStruct), _f, _i64,
                                      _i, _p, _p, _p, _p, _p, _i64, _p]
        L.olmo3_kv_append.restype = _i
        L.olmo3_attn_prefill.argtypes = [_i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(RopeStruct), _f,
                                         _i64, _i, _p, _p, _p, _p, _p, _p, _p, _i64, _p, _p, _sz, _p]
        L.olmo3_attn_prefill.restype = _i
        L.olmo3_attn_decode.argtypes = [_i, _i, _i, _i, _i, _i, ctypes.POINTER(RopeStruct), _f, _i64,
                                        _i, _p, _p, _p, _p, _p, _p, _p, _i64, _p, _p, _sz, _p]
        L.olmo3_attn_decode.restype = _i
        L.olmo3_attn_decode_noalloc.argtypes = L.olmo3_attn_decode.argtypes[:19] + [_p]
        L.olmo3_attn_decode_noalloc.restype = _i
        L.olmo3_attn_prefill_phases.argtypes = [_i] + L.olmo3_attn_prefill.argtypes
        L.olmo3_attn_prefill_phases.restype = _i
        L.olmo3_attn_decode_phases.argtypes = [_i] + L.olmo3_attn_decode.argtypes
        L.olmo3_attn_decode_phases.restype = _i
        L.olmo3_attn_prefill_ragged.argtypes = [_i, _i, _i, _i64, _i, _i, _i, _i, _i,
                                                ctypes.POINTER(RopeStruct), _f, _p, _p, _i, _p, _p,
                                                _p, _p, _p, _p, _p, _i64, _p, _p, _sz, _p]
        L.olmo3_attn_prefill_ragged.restype = _i
        L.olmo3_attn_decode_ragged.argtypes = [_i, _i, _i, _i, _i, _i, ctypes.POINTER(RopeStruct),
                                               _f, _p, _i64, _i, _p, _p, _p, _p, _p, _p, _p, _i64,
                                               _p, _p, _sz, _p]
        L.olmo3_attn_decode_ragged.restype = _i
        R = ctypes.POINTER(RopeStruct)
        L.olmo3_kv_append_e4m3.argtypes = [_i, _i, _i, _i, _i, _i, R, _f, _i64, _p, _p, _p, _p, _p,
                                           _f, _f, _i64, _p]
        L.olmo3_kv_append_e4m3.restype = _i
        L.olmo3_attn_prefill_e4m3.argtypes = [_i, _i, _i, _i, _i, _i, _i, R, _f, _i64, _p, _p,
                                              _p, _p, _p, _p, _p, _f, _f, _i64, _p, _p, _sz, _p]
        L.olmo3_attn_prefill_e4m3.restype = _i
        L.olmo3_attn_decode_e4m3.argtypes = [_i, _i, _i, _i, _i, _i, R, _f, _i64, _p, _p, _p, _p,
                                             _p, _p, _p, _f, _f, _i64, _p, _p, _sz, _p]
        L.olmo3_attn_decode_e4m3.restype = _i
        L.olmo3_attn_decode_e4m3_phases.argtypes = [_i] + L.olmo3_attn_decode_e4m3.argtypes
        L.olmo3_attn_decode_e4m3_phases.restype = _i
        L.olmo3_attn_decode_ragged_e4m3.argtypes = [_i, _i, _i, _i, _i, _i, R, _f, _p, _i64, _p,
                                                    _p, _p, _p, _p, _p, _p, _f, _f, _i64, _p, _p,
                                                    _sz, _p]
        L.olmo3_attn_decode_ragged_e4m3.restype = _i
        L.olmo3_attn_prefill_ragged_e4m3.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, R, _f, _p,
                                                     _p, _p, _p, _p, _p, _p, _p, _f, _f, _i64, _p,
                                                     _p, _sz, _p]
        L.olmo3_attn_prefill_ragged_e4m3.restype = _i
        L.olmo3_status_string.argtypes = [_i]
        L.olmo3_status_string.restype = ctypes.c_char_p
        L.olmo3_abi_version.argtypes = []
        L.olmo3_abi_version.restype = _i
        L.olmo3_probe_prefill_visits.argtypes = [_i, _i64, _i, _i, _i, _p, _p]
        L.olmo3_probe_prefill_visits.restype = _i
        L.olmo3_probe_prefill_order.argtypes = [_i, _i, _i, _i, _i, _i, _i64, _i, _p, _i64]
        L.olmo3_probe_prefill_order.restype = _i
        L.olmo3_probe_decode_reads.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i64, _i64, _p, _p]
        L.olmo3_probe_decode_reads.restype = _i
        if L.olmo3_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.olmo3_abi_version()}, the binding "
                               f"expects {ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().olmo3_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise Olmo3Error(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32")


def _ptr(t: torch.Tensor | None, name: str, dtype=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def olmo3_layer_type(layer: int, n_layers: int) -> int:
    return lib().olmo3_layer_type(int(layer), int(n_layers))


def olmo3_abi_version() -> int:
    return lib().olmo3_abi_version()


def olmo3_workspace_bytes(mode: int, B: int, T: int, H: int, G: int, d: int, layer_type: int,
                          dtype: int, cache_capacity: int) -> int:
    return lib().olmo3_workspace_bytes(mode, B, T, H, G, d, layer_type, dtype, cache_capacity)


def _cache_dims(k_cache: torch.Tensor):
    if k_cache.dim() != 4:
        raise ValueError("caches are [B, G, capacity, d]")
    B, G, cap, d = k_cache.shape
    return B, G, cap, d


def olmo3_kv_append(k_pre, v, k_gain, k_cache, v_cache, *, window: int, layer_type: int,
                    rope: Rope, eps: float = 1e-6, pos_offset: int = 0, stream=None) -> None:
    """Append k_pre/v [B, T, G*d] at positions pos_offset.. to the cache."""
    B, G, cap, d = _cache_dims(k_cache)
    T = k_pre.shape[1]
    dt = k_pre.dtype
    r = rope.to_c()
    st = lib().olmo3_kv_append(B, T, G, d, window, layer_type, ctypes.byref(r), eps, pos_offset,
                               _dtype_code(k_pre), _ptr(k_pre, "k_pre", dt), _ptr(v, "v", dt),
                               _ptr(k_gain, "k_gain", dt), _ptr(k_cache, "k_cache", dt),
                               _ptr(v_cache, "v_cache", dt), cap, _stream(stream, k_pre.device))
    _check(st, "olmo3_kv_append")


def olmo3_attn_prefill(q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out, workspace, *,
                       window: int, layer_type: int, rope: Rope, eps: float = 1e-6,
                       pos_offset: int = 0, stream=None, phases: int | None = None) -> None:
    """Prefill: q_pre [B, T, H*d], k_pre/v [B, T, G*d] -> out [B, T, H*d].
    ``phases`` (bit set of PHASE_*) selects olmo3_attn_prefill_phases."""
    B, G, cap, d = _cache_dims(k_cache)
    T = q_pre.shape[1]
    H = q_pre.shape[2] // d
    dt = q_pre.dtype
    r = rope.to_c()
    args = (B, T, H, G, d, window, layer_type, ctypes.byref(r), eps, pos_offset, _dtype_code(q_pre),
            _ptr(q_pre, "q_pre", dt), _ptr(k_pre, "k_pre", dt), _ptr(v, "v", dt),
            _ptr(q_gain, "q_gain", dt), _ptr(k_gain, "k_gain", dt), _ptr(k_cache, "k_cache", dt),
            _ptr(v_cache, "v_cache", dt), cap, _ptr(out, "out", dt), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream, q_pre.device))
    if phases is None:
        _check(lib().olmo3_attn_prefill(*args), "olmo3_attn_prefill")
    else:
        _check(lib().olmo3_attn_prefill_phases(phases, *args), "olmo3_attn_prefill_phases")


def olmo3_attn_decode(q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out, workspace, *,
                      window: int, layer_type: int, rope: Rope, pos: int, eps: float = 1e-6,
                      stream=None, phases: int | None = None) -> None:
    """Decode one token per sequence at position ``pos``: q_pre [B, H*d],
    k_pre/v [B, G*d] -> out [B, H*d].  ``phases`` selects
    olmo3_attn_decode_phases."""
    B, G, cap, d = _cache_dims(k_cache)
    H = q_pre.shape[-1] // d
    dt = q_pre.dtype
    r = rope.to_c()
    args = (B, H, G, d, window, layer_type, ctypes.byref(r), eps, pos, _dtype_code(q_pre),
            _ptr(q_pre, "q_pre", dt), _ptr(k_pre, "k_pre", dt), _ptr(v, "v", dt),
            _ptr(q_gain, "q_gain", dt), _ptr(k_gain, "k_gain", dt), _ptr(k_cache, "k_cache", dt),
            _ptr(v_cache, "v_cache", dt), cap, _ptr(out, "out", dt), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream, q_pre.device))
    if phases is None:
        _check(lib().olmo3_attn_decode(*args), "olmo3_attn_decode")
    else:
        _check(lib().olmo3_attn_decode_phases(phases, *args), "olmo3_attn_decode_phases")


def olmo3_attn_decode_noalloc(q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out, *,
                              window: int, layer_type: int, rope: Rope, pos: int,
                              eps: float = 1e-6, stream=None) -> None:
    """olmo3_attn_decode without a workspace: the library's per-device
    scratch array (NOALLOC_SCRATCH_BYTES) stands in for it, and the call
    allocates nothing.  Calls on one device must not overlap in time."""
    B, G, cap, d = _cache_dims(k_cache)
    H = q_pre.shape[-1] // d
    dt = q_pre.dtype
    r = rope.to_c()
    _check(lib().olmo3_attn_decode_noalloc(
        B, H, G, d, window, layer_type, ctypes.byref(r), eps, pos, _dtype_code(q_pre),
        _ptr(q_pre, "q_pre", dt), _ptr(k_pre, "k_pre", dt), _ptr(v, "v", dt),
        _ptr(q_gain, "q_gain", dt), _ptr(k_gain, "k_gain", dt), _ptr(k_cache, "k_cache", dt),
        _ptr(v_cache, "v_cache", dt), cap, _ptr(out, "out", dt), _stream(stream, q_pre.device)),
        "olmo3_attn_decode_noalloc")


def _i32(t: torch.Tensor | None, name: str, n: int) -> int:
    if t is None:
        return 0
    if t.dtype != torch.int32 or t.numel() != n:
        raise ValueError(f"{name} must be an int32 device tensor of {n} elements")
    return _ptr(t, name)


def olmo3_attn_prefill_ragged(q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out, workspace,
                              cu_seqlens, pos_offsets, *, max_len: int, max_end: int, window: int,
                              layer_type: int, rope: Rope, eps: float = 1e-6, stream=None) -> None:
    """Packed prefill of B sequences: q_pre [N, H*d], k_pre/v [N, G*d] ->
    out [N, H*d]; sequence b owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1
    (int32 device tensors: cu_seqlens [B+1], pos_offsets [B] or None) and
    uses cache k_cache[b] / v_cache[b]."""
    B, G, cap, d = _cache_dims(k_cache)
    N = q_pre.shape[0]
    H = q_pre.shape[-1] // d
    dt = q_pre.dtype
    r = rope.to_c()
    st = lib().olmo3_attn_prefill_ragged(
        B, N, max_len, max_end, H, G, d, window, layer_type, ctypes.byref(r), eps,
        _i32(cu_seqlens, "cu_seqlens", B + 1), _i32(pos_offsets, "pos_offsets", B),
        _dtype_code(q_pre), _ptr(q_pre, "q_pre", dt), _ptr(k_pre, "k_pre", dt), _ptr(v, "v", dt),
        _ptr(q_gain, "q_gain", dt), _ptr(k_gain, "k_gain", dt), _ptr(k_cache, "k_cache", dt),
        _ptr(v_cache, "v_cache", dt), cap, _ptr(out, "out", dt), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream, q_pre.device))
    _check(st, "olmo3_attn_prefill_ragged")


def olmo3_attn_decode_ragged(q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out, workspace,
                             positions, *, max_pos: int, window: int, layer_type: int, rope: Rope,
                             eps: float = 1e-6, stream=None) -> None:
    """Decode one token per sequence at its own position (int32 device
    tensor positions [B], each <= max_pos): q_pre [B, H*d], k_pre/v [B, G*d]
    -> out [B, H*d]."""
    B, G, cap, d = _cache_dims(k_cache)
    H = q_pre.shape[-1] // d
    dt = q_pre.dtype
    r = rope.to_c()
    st = lib().olmo3_attn_decode_ragged(
        B, H, G, d, window, layer_type, ctypes.byref(r), eps, _i32(positions, "positions", B),
        max_pos, _dtype_code(q_pre), _ptr(q_pre, "q_pre", dt), _ptr(k_pre, "k_pre", dt),
        _ptr(v, "v", dt), _ptr(q_gain, "q_gain", dt), _ptr(k_gain, "k_gain", dt),
        _ptr(k_cache, "k_cache", dt), _ptr(v_cache, "v_cache", dt), cap, _ptr(out, "out", dt),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream, q_pre.device))
    _check(st, "olmo3_attn_decode_ragged")


def _e4m3_caches(k_cache, v_cache):
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != torch.uint8:
            raise TypeError(f"{name} must hold e4m3 codes as torch.uint8")
    return _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache")


def olmo3_kv_append_e4m3(k_pre, v, k_gain, k_cache, v_cache, *, k_scale: float, v_scale: float,
                         window: int, layer_type: int, rope: Rope, eps: float = 1e-6,
                         pos_offset: int = 0, stream=None) -> None:
    """Append k_pre/v [B, T, G*d] (bf16) to e4m3 caches [B, G, capacity, d] (uint8)."""
    B, G, cap, d = _cache_dims(k_cache)
    T = k_pre.shape[1]
    dt = torch.bfloat16
    kc, vc = _e4m3_caches(k_cache, v_cache)
    r = rope.to_c()
    st = lib().olmo3_kv_append_e4m3(B, T, G, d, window, layer_type, ctypes.byref(r), eps,
                                    pos_offset, _ptr(k_pre, "k_pre", dt), _ptr(v, "v", dt),
                                    _ptr(k_gain, "k_gain", dt), kc, vc, k_scale, v_scale, cap,
                                    _stream(stream, k_pre.device))
    _check(st, "olmo3_kv_append_e4m3")


def olmo3_attn_prefill_e4m3(q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out, workspace, *,
                            k_scale: float, v_scale: float, window: int, layer_type: int,
                            rope: Rope, eps: float = 1e-6, pos_offset: int = 0,
                            stream=None) -> None:
    """Prefill of positions pos_offset..pos_offset+T-1 into e4m3 caches (uint8)."""
    B, G, cap, d = _cache_dims(k_cache)
    T = q_pre.shape[1]
    H = q_pre.shape[2] // d
    dt = torch.bfloat16
    kc, vc = _e4m3_caches(k_cache, v_cache)
    r = rope.to_c()
    st = lib().olmo3_attn_prefill_e4m3(
        B, T, H, G, d, window, layer_type, ctypes.byref(r), eps, pos_offset,
        _ptr(q_pre, "q_pre", dt), _ptr(k_pre, "k_pre", dt), _ptr(v, "v", dt),
        _ptr(q_gain, "q_gain", dt), _ptr(k_gain, "k_gain", dt), kc, vc, k_scale, v_scale, cap,
        _ptr(out, "out", dt),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream, q_pre.device))
    _check(st, "olmo3_attn_prefill_e4m3")


def olmo3_attn_decode_e4m3(q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out, workspace, *,
                           k_scale: float, v_scale: float, window: int, layer_type: int,
                           rope: Rope, pos: int, eps: float = 1e-6, stream=None,
                           phases: int | None = None) -> None:
    """Decode against e4m3 caches (uint8): q_pre [B, H*d], k_pre/v [B, G*d]
    -> out [B, H*d].  ``phases`` selects olmo3_attn_decode_e4m3_phases."""
    B, G, cap, d = _cache_dims(k_cache)
    H = q_pre.shape[-1] // d
    dt = torch.bfloat16
    kc, vc = _e4m3_caches(k_cache, v_cache)
    r = rope.to_c()
    args = (B, H, G, d, window, layer_type, ctypes.byref(r), eps, pos, _ptr(q_pre, "q_pre", dt),
            _ptr(k_pre, "k_pre", dt), _ptr(v, "v", dt), _ptr(q_gain, "q_gain", dt),
            _ptr(k_gain, "k_gain", dt), kc, vc, k_scale, v_scale, cap, _ptr(out, "out", dt),
            _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream, q_pre.device))
    if phases is None:
        _check(lib().olmo3_attn_decode_e4m3(*args), "olmo3_attn_decode_e4m3")
    else:
        _check(lib().olmo3_attn_decode_e4m3_phases(phases, *args), "olmo3_attn_decode_e4m3_phases")


def olmo3_attn_prefill_ragged_e4m3(q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out,
                                   workspace, cu_seqlens, *, k_scale: float, v_scale: float,
                                   max_len: int, window: int, layer_type: int, rope: Rope,
                                   eps: float = 1e-6, stream=None) -> None:
    """First chunks of B prompts packed row after row (q_pre [n_tokens, H*d],
    k_pre/v [n_tokens, G*d], cu_seqlens int32 [B+1]) into e4m3 caches
    [B, G, capacity, d] (uint8); out [n_tokens, H*d]."""
    B, G, cap, d = _cache_dims(k_cache)
    n_tokens = q_pre.shape[0]
    H = q_pre.shape[-1] // d
    dt = torch.bfloat16
    kc, vc = _e4m3_caches(k_cache, v_cache)
    r = rope.to_c()
    st = lib().olmo3_attn_prefill_ragged_e4m3(
        B, n_tokens, max_len, H, G, d, window, layer_type, ctypes.byref(r), eps,
        _i32(cu_seqlens, "cu_seqlens", B + 1), _ptr(q_pre, "q_pre", dt), _ptr(k_pre, "k_pre", dt),
        _ptr(v, "v", dt), _ptr(q_gain, "q_gain", dt), _ptr(k_gain, "k_gain", dt), kc, vc, k_scale,
        v_scale, cap, _ptr(out, "out", dt), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream, q_pre.device))
    _check(st, "olmo3_attn_prefill_ragged_e4m3")


def olmo3_attn_decode_ragged_e4m3(q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out,
                                  workspace, positions, *, k_scale: float, v_scale: float,
                                  max_pos: int, window: int, layer_type: int, rope: Rope,
                                  eps: float = 1e-6, stream=None) -> None:
    """Decode one token per sequence at its own position (int32 device tensor
    positions [B], each <= max_pos) against e4m3 caches (uint8)."""
    B, G, cap, d = _cache_dims(k_cache)
    H = q_pre.shape[-1] // d
    dt = torch.bfloat16
    kc, vc = _e4m3_caches(k_cache, v_cache)
    r = rope.to_c()
    st = lib().olmo3_attn_decode_ragged_e4m3(
        B, H, G, d, window, layer_type, ctypes.byref(r), eps, _i32(positions, "positions", B),
        max_pos, _ptr(q_pre, "q_pre", dt), _ptr(k_pre, "k_pre", dt), _ptr(v, "v", dt),
        _ptr(q_gain, "q_gain", dt), _ptr(k_gain, "k_gain", dt), kc, vc, k_scale, v_scale, cap,
        _ptr(out, "out", dt), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream, q_pre.device))
    _check(st, "olmo3_attn_decode_ragged_e4m3")


def workspace(mode: int, B: int, T: int, H: int, G: int, d: int, layer_type: int,
              dtype: torch.dtype, cache_capacity: int, device) -> torch.Tensor:
    """Device byte buffer of the size ``olmo3_workspace_bytes`` asks for."""
    code = dtype if isinstance(dtype, int) else (DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32)
    n = olmo3_workspace_bytes(mode, B, T, H, G, d, layer_type, code, cache_capacity)
    if n == 0:
        raise Olmo3Error(ERR_INVALID_ARG, "olmo3_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def olmo3_probe_prefill_visits(T: int, window: int, layer_type: int, pos_offset: int = 0,
                               kv_splits: int = 1, device="cuda") -> torch.Tensor:
    """[T, pos_offset + T] uint8 table: how many times the prefill kernel
    (with kv_splits workgroups per query block) accumulates each (query, key
    position) pair, for queries at pos_offset .. pos_offset + T - 1."""
    visit = torch.empty((T, pos_offset + T), dtype=torch.uint8, device=device)
    st = lib().olmo3_probe_prefill_visits(T, pos_offset, window, layer_type, kv_splits,
                                          _ptr(visit, "visit"), _stream(None, visit.device))
    _check(st, "olmo3_probe_prefill_visits")
    return visit


def olmo3_probe_prefill_order(B: int, T: int, H: int, G: int, window: int, layer_type: int,
                              pos_offset: int = 0, kv_splits: int = 1) -> torch.Tensor:
    """[n, 4] int32 CPU tensor: the (sequence, head, query block, key split)
    each workgroup of the d = 128 prefill kernel takes, in workgroup order."""
    n = -(-T // 128) * H * B * kv_splits
    work = torch.zeros((n, 4), dtype=torch.int32)
    st = lib().olmo3_probe_prefill_order(B, T, H, G, window, layer_type, pos_offset, kv_splits,
                                         work.data_ptr(), work.numel())
    _check(st, "olmo3_probe_prefill_order")
    return work


def olmo3_probe_decode_reads(B: int, H: int, G: int, d: int, window: int, layer_type: int,
                             pos: int, cache_capacity: int, dtype: int = DTYPE_BF16,
                             device="cuda") -> torch.Tensor:
    """[cache_capacity] int32 count of reads per slot by the decode kernel that
    serves these arguments (dtype: DTYPE_BF16 or DTYPE_BF16_E4M3)."""
    count = torch.empty(cache_capacity, dtype=torch.int32, device=device)
    st = lib().olmo3_probe_decode_reads(B, H, G, d, window, layer_type, dtype, pos, cache_capacity,
                                        _ptr(count, "count"), _stream(None, count.device))
    _check(st, "olmo3_probe_decode_reads")
    return count
