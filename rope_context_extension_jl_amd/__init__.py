"""Python binding of libbifocal (dynamic bifocal RoPE attention, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libbifocal.so, reached through its C ABI (include/bifocal.h).
PyTorch supplies device memory and the current HIP stream. There is no CPU
fallback: without the built library, or given CPU tensors, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "LIB_PATH", "BifocalError", "lib", "group_size", "tile_class", "prefill_tile_shape",
    "status_string", "rope_apply", "prefill_workspace_size", "bifocal_prefill",
    "decode_workspace_size", "bifocal_decode", "debug_tile_classes", "ie_ratio_view",
    "prefill_cached_workspace_size", "bifocal_prefill_cached",
    "decode_batch_workspace_size", "bifocal_decode_batch",
    "decode_workspace", "decode_batch_workspace",
    "calib_stream_read", "calib_mfma_bf16", "MODES", "REMAPS", "prefill_flags",
    "FLAG_Q_RANGE", "FLAG_K_RANGE",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbifocal.so")
JL_BF16, JL_FP32 = 0, 1
MODES = {"fused": 0, "ie": 1, "plain": 2}
# Remote map, OR-ed into the mode code: floor(x / G) (aliasing) or the real
# x / G (continuous frequency interpolation, JL_REMAP_CONTINUOUS).
REMAPS = {"floor": 0, "continuous": 16}


def _mode_code(mode: str, remap: str) -> int:
    return MODES[mode] | REMAPS[remap]

_c_i64, _c_int, _c_dbl, _c_flt, _c_p, _c_sz = (ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                              ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t)

_SIGS = {
    "jl_group_size": (_c_i64, [_c_i64, _c_i64]),
    "jl_tile_class": (_c_int, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64]),
    "jl_prefill_tile_shape": (_c_int, [_c_int, _c_int, ctypes.POINTER(_c_int),
                                       ctypes.POINTER(_c_int)]),
    "jl_rope_apply": (_c_int, [_c_p, _c_i64, _c_int, _c_int, _c_p, _c_int, _c_i64, _c_dbl, _c_int,
                               _c_p]),
    "jl_prefill_workspace_size": (_c_sz, [_c_i64, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "jl_prefill_ie_ratio_offset": (_c_sz, [_c_i64, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "jl_bifocal_prefill": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_i64,
                                    _c_int, _c_int, _c_int, _c_i64, _c_i64, _c_dbl, _c_flt,
                                    _c_int, _c_int, _c_p, _c_sz, _c_p]),
    "jl_bifocal_prefill_timed": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int,
                                          _c_i64, _c_int, _c_int, _c_int, _c_i64, _c_i64, _c_dbl,
                                          _c_flt, _c_int, _c_int, _c_p, _c_sz, _c_p, _c_p, _c_p]),
    "jl_prefill_cached_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_int, _c_int, _c_int,
                                                 _c_int]),
    "jl_bifocal_prefill_cached": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                           _c_int, _c_int, _c_int, _c_i64, _c_i64, _c_dbl, _c_flt,
                                           _c_int, _c_int, _c_p, _c_sz, _c_p]),
    "jl_bifocal_prefill_cached_timed": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64,
                                                 _c_i64, _c_int, _c_int, _c_int, _c_i64, _c_i64,
                                                 _c_dbl, _c_flt, _c_int, _c_int, _c_p, _c_sz,
                                                 _c_p, _c_p, _c_p]),
    "jl_decode_workspace_size": (_c_sz, [_c_i64, _c_int, _c_int]),
    "jl_bifocal_decode": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_int, _c_int,
                                   _c_int, _c_i64, _c_i64, _c_dbl, _c_flt, _c_int, _c_int, _c_int,
                                   _c_p, _c_sz, _c_p]),
    "jl_bifocal_decode_timed": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_int,
                                         _c_int, _c_int, _c_i64, _c_i64, _c_dbl, _c_flt, _c_int,
                                         _c_int, _c_int, _c_p, _c_sz, _c_p, _c_p, _c_p]),
    "jl_bifocal_decode_noalloc": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_int,
                                           _c_int, _c_int, _c_i64, _c_i64, _c_dbl, _c_flt, _c_int,
                                           _c_int, _c_int, _c_p]),
    "jl_decode_batch_workspace_size": (_c_sz, [_c_int, _c_i64, _c_int, _c_int]),
    "jl_bifocal_decode_batch": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_i64,
                                         _c_i64, _c_int, _c_int, _c_int, _c_i64, _c_i64, _c_dbl,
                                         _c_flt, _c_int, _c_int, _c_int, _c_p, _c_sz, _c_p]),
    "jl_bifocal_decode_batch_timed": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int,
                                               _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_i64,
                                               _c_i64, _c_dbl, _c_flt, _c_int, _c_int, _c_int,
                                               _c_p, _c_sz, _c_p, _c_p, _c_p]),
    "jl_prefill_flags": (_c_int, [_c_p, ctypes.POINTER(ctypes.c_uint32), _c_p]),
    "jl_debug_tile_classes": (_c_int, [_c_i64, _c_i64, _c_p, _c_p]),
    "jl_calib_stream_read": (_c_int, [_c_p, _c_sz, _c_p, _c_int, _c_p]),
    "jl_calib_stream_read_ex": (_c_int, [_c_p, _c_sz, _c_p, _c_int, _c_int, _c_p]),
    "jl_calib_mfma_bf16": (_c_int, [_c_p, _c_int, _c_int, _c_p]),
    "jl_status_string": (ctypes.c_char_p, [_c_int]),
    "jl_last_hip_error": (_c_int, []),
}

_lib = None


class BifocalError(RuntimeError):
    """A libbifocal call returned a negative status."""

    def __init__(self, fn: str, status: int):
        msg = status_string(status)
        if status == -3:
            msg += f" (hipError_t {lib().jl_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libbifocal.so (built in-tree by build.py). Raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libbifocal.so not built at {LIB_PATH}; run "
                              "`python -m rope_context_extension_jl_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().jl_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status < 0:
        raise BifocalError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return JL_BF16
    if t.dtype == torch.float32:
        return JL_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dev(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libbifocal has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _want(t: Optional[torch.Tensor], name: str, shape, dtype, device=None) -> None:
    """Raise ValueError unless t (when given) has this shape, dtype and device.
    The C ABI sees bare pointers, so a mismatch it cannot detect (a float32
    key tensor beside bfloat16 queries, an int64 cu_seqlens) is caught here,
    before anything is launched."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _ws_bytes(workspace: torch.Tensor, device) -> int:
    """Byte size of a workspace tensor of any dtype; it must sit on the call's
    device (the C ABI sees a bare pointer and a byte count)."""
    if workspace.device != device:
        raise ValueError(f"workspace must be on {device}, got {workspace.device}")
    return workspace.numel() * workspace.element_size()


def _want_cu(cu: Optional[torch.Tensor], name: str, device) -> int:
    """Number of sequences described by an int32 [B + 1] prefix-offset tensor."""
    if cu is None:
        return 1
    if cu.dim() != 1 or cu.numel() < 2:
        raise ValueError(f"{name} must be a 1-D tensor of B + 1 >= 2 offsets")
    _want(cu, name, (cu.numel(),), torch.int32, device)
    return cu.numel() - 1


def _want_rank(t: torch.Tensor, name: str, rank: int) -> None:
    if t.dim() != rank:
        raise ValueError(f"{name} must have {rank} dimensions, got shape {tuple(t.shape)}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _events(events):
    """(begin, end) torch.cuda.Event pair -> raw hipEvent_t handles (or NULLs)."""
    if events is None:
        return None, None
    out = []
    for ev in events:
        if ev.cuda_event == 0:  # torch creates the HIP event lazily on first record
            ev.record()
        out.append(ctypes.c_void_p(ev.cuda_event))
    return tuple(out)


# ---------------------------------------------------------------- host-only calls
def group_size(L: int, w_pre: int) -> int:
    g = lib().jl_group_size(int(L), int(w_pre))
    _check("jl_group_size", g)
    return int(g)


def tile_class(q0: int, q1: int, k0: int, k1: int, w0: int) -> int:
    c = lib().jl_tile_class(int(q0), int(q1), int(k0), int(k1), int(w0))
    _check("jl_tile_class", c)
    return int(c)


def prefill_tile_shape(dtype=torch.bfloat16, d: int = 128):
    bm, bn = _c_int(), _c_int()
    code = JL_BF16 if dtype == torch.bfloat16 else JL_FP32
    _check("jl_prefill_tile_shape", lib().jl_prefill_tile_shape(code, d, ctypes.byref(bm),
                                                                ctypes.byref(bn)))
    return bm.value, bn.value


def prefill_workspace_size(T, B, Hq, Hkv, d, dtype=torch.bfloat16, mode="fused") -> int:
    code = JL_BF16 if dtype == torch.bfloat16 else JL_FP32
    n = lib().jl_prefill_workspace_size(int(T), int(B), int(Hq), int(Hkv), int(d), code,
                                        MODES[mode])
    if n == 0 and T > 0:
        raise ValueError("invalid prefill shape")
    return int(n)


def prefill_cached_workspace_size(q_off, Tq, Hq, Hkv, d, mode="fused") -> int:
    return int(lib().jl_prefill_cached_workspace_size(int(q_off), int(Tq), int(Hq), int(Hkv),
                                                      int(d), MODES[mode]))


def decode_workspace_size(capacity, Hq, d) -> int:
    return int(lib().jl_decode_workspace_size(int(capacity), int(Hq), int(d)))


def decode_workspace(capacity, Hq, d, device="cuda") -> torch.Tensor:
    """A decode workspace for jl_bifocal_decode (any contents)."""
    return torch.empty(max(decode_workspace_size(capacity, Hq, d), 16), dtype=torch.uint8,
                       device=device)


def decode_batch_workspace(B, max_keys, Hq, d, device="cuda") -> torch.Tensor:
    """A decode workspace for jl_bifocal_decode_batch (any contents)."""
    return torch.empty(max(decode_batch_workspace_size(B, max_keys, Hq, d), 16),
                       dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- device calls
def rope_apply(x: torch.Tensor, theta: float, cu_seqlens: Optional[torch.Tensor] = None,
               pos_offset: int = 0) -> torch.Tensor:
    """In place: x[t, h, :] <- RoPE(x[t, h, :], position of t). x: [T, H, d]."""
    _want_rank(x, "x", 3)
    T, H, d = x.shape
    _dtype_code(x)
    B = _want_cu(cu_seqlens, "cu_seqlens", x.device)
    st = lib().jl_rope_apply(_dev(x, "x"), T, H, d, _dev(cu_seqlens, "cu_seqlens"), B,
                             int(pos_offset), float(theta), _dtype_code(x), _stream(x.device))
    _check("jl_rope_apply", st)
    return x


def bifocal_prefill(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, w0: int, w_pre: int,
                    theta: float, scale: float = 0.0, mode: str = "fused",
                    cu_seqlens: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, kcache_out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                    events=None, remap: str = "floor"):
    """Causal bifocal attention; xq/xk/v are RAW [T, H, d]. Returns (o, lse).
    events: optional (begin, end) torch.cuda.Event pair, recorded around the
    attention kernels only (jl_bifocal_prefill_timed). remap: "floor" or
    "continuous" (remote positions x / G as real numbers)."""
    _want_rank(xq, "xq", 3)
    _want_rank(xk, "xk", 3)
    T, Hq, d = xq.shape
    Hkv = xk.shape[1]
    _dtype_code(xq)
    dv = xq.device
    _want(xk, "xk", (T, Hkv, d), xq.dtype, dv)
    _want(v, "v", (T, Hkv, d), xq.dtype, dv)
    _want(out, "out", (T, Hq, d), xq.dtype, dv)
    _want(lse, "lse", (Hq, T), torch.float32, dv)
    _want(kcache_out, "kcache_out", (T, Hkv, d), xq.dtype, dv)
    B = _want_cu(cu_seqlens, "cu_seqlens", dv)
    if out is None:
        out = torch.empty_like(xq)
    if lse is None and want_lse:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=xq.device)
    need = prefill_workspace_size(T, B, Hq, Hkv, d, xq.dtype, mode)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xq.device)
    ws_n = _ws_bytes(workspace, dv)
    st = lib().jl_bifocal_prefill_timed(
        _dev(xq, "xq"), _dev(xk, "xk"), _dev(v, "v"), _dev(out, "out"), _dev(lse, "lse"),
        _dev(kcache_out, "kcache_out"), _dev(cu_seqlens, "cu_seqlens"), B, T, Hq, Hkv, d,
        int(w0), int(w_pre), float(theta), float(scale), _dtype_code(xq), _mode_code(mode, remap),
        _dev(workspace, "workspace"), ws_n, _stream(xq.device), *_events(events))
    _check("jl_bifocal_prefill", st)
    return out, lse


FLAG_Q_RANGE, FLAG_K_RANGE = 1, 2


def prefill_flags(workspace: torch.Tensor) -> int:
    """Range flags (FLAG_Q_RANGE | FLAG_K_RANGE) the last prefill left in
    `workspace`; waits for the current stream (jl_prefill_flags)."""
    out = ctypes.c_uint32(0)
    _check("jl_prefill_flags", lib().jl_prefill_flags(_dev(workspace, "workspace"),
                                                       ctypes.byref(out),
                                                       _stream(workspace.device)))
    return int(out.value)


def ie_ratio_view(workspace: torch.Tensor, T, B, Hq, Hkv, d, dtype=torch.bfloat16):
    """[Hq, T] float32 view of the Eq. 7 cancellation ratios an IE prefill left
    in `workspace`."""
    code = JL_BF16 if dtype == torch.bfloat16 else JL_FP32
    off = int(lib().jl_prefill_ie_ratio_offset(T, B, Hq, Hkv, d, code))
    return workspace[off: off + Hq * T * 4].view(torch.float32).view(Hq, T)


def bifocal_prefill_cached(xq: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                           q_off: int, w0: int, w_pre: int, theta: float, scale: float = 0.0,
                           mode: str = "fused", out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                           events=None, remap: str = "floor"):
    """Chunked prefill: RAW queries xq [Tq, Hq, d] at positions q_off .. q_off+Tq-1
    against the absolute cache [capacity, Hkv, d] (rows up to q_off+Tq-1 filled).
    Returns (o [Tq, Hq, d], lse [Hq, Tq])."""
    _want_rank(xq, "xq", 3)
    _want_rank(kcache, "kcache", 3)
    Tq, Hq, d = xq.shape
    C, Hkv, _ = kcache.shape
    _dtype_code(xq)
    dv = xq.device
    _want(kcache, "kcache", (C, Hkv, d), xq.dtype, dv)
    _want(vcache, "vcache", (C, Hkv, d), xq.dtype, dv)
    _want(out, "out", (Tq, Hq, d), xq.dtype, dv)
    _want(lse, "lse", (Hq, Tq), torch.float32, dv)
    if out is None:
        out = torch.empty_like(xq)
    if lse is None and want_lse:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=xq.device)
    if workspace is None:
        need = prefill_cached_workspace_size(q_off, Tq, Hq, Hkv, d, mode)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xq.device)
    ws_n = _ws_bytes(workspace, dv)
    st = lib().jl_bifocal_prefill_cached_timed(
        _dev(xq, "xq"), _dev(kcache, "kcache"), _dev(vcache, "vcache"), _dev(out, "out"),
        _dev(lse, "lse"), int(q_off), Tq, C, Hq, Hkv, d, int(w0), int(w_pre), float(theta),
        float(scale), _dtype_code(xq), _mode_code(mode, remap), _dev(workspace, "workspace"),
        ws_n, _stream(xq.device), *_events(events))
    _check("jl_bifocal_prefill_cached", st)
    return out, lse


def bifocal_decode(xq: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor, pos: int,
                   w0: int, w_pre: int, theta: float, scale: float = 0.0, mode: str = "fused",
                   num_splits: int = 0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   want_lse: bool = True, events=None, remap: str = "floor"):
    """One decode step at `pos` with a RAW query xq [Hq, d] against the absolute
    cache [capacity, Hkv, d]. Returns (o [Hq, d], lse [Hq])."""
    _want_rank(xq, "xq", 2)
    _want_rank(kcache, "kcache", 3)
    Hq, d = xq.shape
    C, Hkv, _ = kcache.shape
    _dtype_code(xq)
    dv = xq.device
    _want(kcache, "kcache", (C, Hkv, d), xq.dtype, dv)
    _want(vcache, "vcache", (C, Hkv, d), xq.dtype, dv)
    _want(out, "out", (Hq, d), xq.dtype, dv)
    _want(lse, "lse", (Hq,), torch.float32, dv)
    if out is None:
        out = torch.empty_like(xq)
    if lse is None and want_lse:
        lse = torch.empty((Hq,), dtype=torch.float32, device=xq.device)
    if workspace is None:
        workspace = decode_workspace(C, Hq, d, xq.device)
    ws_n = _ws_bytes(workspace, dv)
    st = lib().jl_bifocal_decode_timed(
        _dev(xq, "xq"), _dev(kcache, "kcache"), _dev(vcache, "vcache"), _dev(out, "out"),
        _dev(lse, "lse"), int(pos), C, Hq, Hkv, d, int(w0), int(w_pre), float(theta),
        float(scale), _dtype_code(xq), _mode_code(mode, remap), int(num_splits),
        _dev(workspace, "workspace"),
        ws_n, _stream(xq.device), *_events(events))
    _check("jl_bifocal_decode", st)
    return out, lse


def decode_batch_workspace_size(B, max_keys, Hq, d) -> int:
    return int(lib().jl_decode_batch_workspace_size(int(B), int(max_keys), int(Hq), int(d)))


def bifocal_decode_batch(xq: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                         positions: torch.Tensor, cache_starts: torch.Tensor, max_keys: int,
                         w0: int, w_pre: int, theta: float, scale: float = 0.0,
                         mode: str = "fused", num_splits: int = 0,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                         events=None, remap: str = "floor"):
    """One decode step for B sequences: RAW queries xq [B, Hq, d]; sequence b's
    keys 0 .. positions[b] are rows cache_starts[b] + k of the shared cache
    [rows, Hkv, d]. positions / cache_starts: device int32 [B]; max_keys: a
    host bound on positions[b] + 1. Returns (o [B, Hq, d], lse [B, Hq])."""
    _want_rank(xq, "xq", 3)
    _want_rank(kcache, "kcache", 3)
    B, Hq, d = xq.shape
    C, Hkv, _ = kcache.shape
    _dtype_code(xq)
    dv = xq.device
    _want(kcache, "kcache", (C, Hkv, d), xq.dtype, dv)
    _want(vcache, "vcache", (C, Hkv, d), xq.dtype, dv)
    _want(out, "out", (B, Hq, d), xq.dtype, dv)
    _want(lse, "lse", (B, Hq), torch.float32, dv)
    for t, name in ((positions, "positions"), (cache_starts, "cache_starts")):
        if t.dtype != torch.int32 or t.numel() != B or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor of {B} entries")
        if t.device != dv:
            raise ValueError(f"{name} must be on {dv}, got {t.device}")
    if out is None:
        out = torch.empty_like(xq)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=xq.device)
    if workspace is None:
        workspace = decode_batch_workspace(B, max_keys, Hq, d, xq.device)
    ws_n = _ws_bytes(workspace, dv)
    st = lib().jl_bifocal_decode_batch_timed(
        _dev(xq, "xq"), _dev(kcache, "kcache"), _dev(vcache, "vcache"), _dev(out, "out"),
        _dev(lse, "lse"), _dev(positions, "positions"), _dev(cache_starts, "cache_starts"), B,
        int(max_keys), C, Hq, Hkv, d, int(w0), int(w_pre), float(theta), float(scale),
        _dtype_code(xq), _mode_code(mode, remap), int(num_splits), _dev(workspace, "workspace"),
        ws_n, _stream(xq.device), *_events(events))
    _check("jl_bifocal_decode_batch", st)
    return out, lse


def debug_tile_classes(L: int, w0: int, device="cuda") -> torch.Tensor:
    """Device-side tile classes of a length-L sequence, [ceil(L/BM), ceil(L/BN)] int8."""
    bm, bn = prefill_tile_shape(torch.bfloat16, 128)
    out = torch.empty(((L + bm - 1) // bm, (L + bn - 1) // bn), dtype=torch.int8, device=device)
    _check("jl_debug_tile_classes", lib().jl_debug_tile_classes(int(L), int(w0), _dev(out, "out"),
                                                                _stream(out.device)))
    return out


def calib_stream_read(buf: torch.Tensor, events=None, blocks: int = 2048,
                      variant: int = 0) -> None:
    """One streaming read of `buf` (device) by calibration kernel `variant`
    (0 grid-stride, 1 nontemporal chunks, 2 direct-to-LDS chunks); the
    optional (begin, end) events bracket it on the current stream."""
    sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    s = torch.cuda.current_stream(buf.device)
    if events is not None:
        events[0].record(s)
    _check("jl_calib_stream_read_ex", lib().jl_calib_stream_read_ex(
        _dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(sink, "sink"), int(blocks),
        int(variant), _stream(buf.device)))
    if events is not None:
        events[1].record(s)


def calib_mfma_bf16(blocks: int, iters: int, events=None, device="cuda") -> float:
    """Runs the MFMA calibration kernel; returns its FLOP count."""
    sink = torch.empty(int(blocks) * 256, dtype=torch.float32, device=device)
    if events is not None:
        events[0].record(torch.cuda.current_stream(sink.device))
    _check("jl_calib_mfma_bf16", lib().jl_calib_mfma_bf16(_dev(sink, "sink"), int(blocks),
                                                          int(iters), _stream(sink.device)))
    if events is not None:
        events[1].record(torch.cuda.current_stream(sink.device))
    return 4.0 * 32768.0 * 4 * int(blocks) * int(iters)
