"""Python binding of libtkv.so: the C ABI of include/tkv.h, same names.

Argument marshalling only.  Tensors (torch) are passed by ``data_ptr()``; host
per-sequence lengths are plain Python/NumPy integer sequences; streams are
torch streams or raw handles.  Every call raises :class:`TkvError` on a
negative status.  The library must exist: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtkv.so")

TKV_OK = 0
TKV_ERR_ARG = -1
TKV_ERR_CAPACITY = -2
TKV_ERR_STATE = -3
TKV_ERR_HIP = -4
TKV_BF16 = 0
TKV_F32 = 1
# the TKV_ABI_VERSION of include/tkv.h these structures and signatures follow
ABI_VERSION = 4

EXPORTED = (
    "tkv_abi_version", "tkv_last_error", "tkv_append", "tkv_decode_workspace_bytes",
    "tkv_decode_step", "tkv_decode_step_noalloc", "tkv_append_decode_step",
    "tkv_decode_step_window",
    "tkv_decode_step_streamed", "tkv_decode_step_t2",
    "tkv_append_decode_step_t2", "tkv_update_scores", "tkv_assign_tiers",
    "tkv_compact_workspace_bytes", "tkv_compact", "tkv_quantize_t2",
    "tkv_t2_update_workspace_bytes", "tkv_t2_update", "tkv_gather_t1", "tkv_t0_capacity",
    "tkv_compact_host_t1_workspace_bytes", "tkv_compact_host_t1_scratch_bytes",
    "tkv_compact_host_t1", "tkv_read_probe", "tkv_timing_enable",
    "tkv_timing_select", "tkv_timing_reset", "tkv_timing_read",
)


class TkvError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where} failed with status {status}: {msg}")
        self.status = status


class tkv_model(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("alpha_scratch", ctypes.c_int32),
                ("t0_caps", ctypes.c_void_p), ("t1_caps", ctypes.c_void_p)]


class tkv_policy(ctypes.Structure):
    _fields_ = [("prompt_len", ctypes.c_int32), ("num_sinks", ctypes.c_int32),
                ("recent_window", ctypes.c_int32), ("frac_t1", ctypes.c_float),
                ("frac_t2", ctypes.c_float), ("frac_t3", ctypes.c_float),
                ("delta", ctypes.c_int32)]


class tkv_t2_pool(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("t2_pos", ctypes.c_void_p), ("t2_len", ctypes.c_void_p),
                ("cap2", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Open libtkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m tiered_kv_cache_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(_LIB_PATH)
    sig = {
        "tkv_abi_version": (_I, []),
        "tkv_last_error": (ctypes.c_char_p, []),
        "tkv_append": (_I, [ctypes.POINTER(tkv_model), _I, _P, _P, _P, _P, _I, _P, _P, _P,
                            _P, _P, _I, _P]),
        "tkv_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(tkv_model), _I, _I,
                                                         _I, _I]),
        "tkv_decode_step": (_I, [ctypes.POINTER(tkv_model), _I, _I, _I, _P, _P, _P, _P, _I,
                                 _P, _P, _P, _I, _P, _P, _I, _P, _P, _P, _I, _P,
                                 ctypes.c_size_t, _P]),
        "tkv_decode_step_noalloc": (_I, [ctypes.POINTER(tkv_model), _I, _I, _I, _P, _P, _P, _P,
                                         _I, _P, _P, _P, _I, _P, _P, _I, _P, _P, _P, _I, _P]),
        "tkv_append_decode_step": (_I, [ctypes.POINTER(tkv_model), _I, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _I, _P, _P, _P, _I, _P, _P, _I, _P, _P, _P,
                                        _I, _P, ctypes.c_size_t, _P]),
        "tkv_decode_step_window": (_I, [ctypes.POINTER(tkv_model), _I, _I, _I, _P, _P, _P, _P,
                                        _I, _P, _P, _I, _P, _P, _I, _P, _P, _P, _I, _P,
                                        ctypes.c_size_t, _P]),
        "tkv_decode_step_streamed": (_I, [ctypes.POINTER(tkv_model), _I, _P, _P, _P, _P, _I,
                                          _P, _P, _I, _P, _I, _P, _P, _I, _P, _P, _P, _I, _P,
                                          ctypes.c_size_t, _P, _P, _P, _P,
                                          ctypes.POINTER(ctypes.c_int64)]),
        "tkv_decode_step_t2": (_I, [ctypes.POINTER(tkv_model), _I, _I, _I, _P, _P, _P, _P, _I,
                                    _P, _P, _P, _I, ctypes.POINTER(tkv_t2_pool), _P, _P, _I,
                                    _P, _P, _P, _I, _P, ctypes.c_size_t, _P]),
        "tkv_append_decode_step_t2": (_I, [ctypes.POINTER(tkv_model), _I, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _I, _P, _P, _P, _I,
                                           ctypes.POINTER(tkv_t2_pool), _P, _P, _I, _P, _P, _P,
                                           _I, _P, ctypes.c_size_t, _P]),
        "tkv_t2_update_workspace_bytes": (ctypes.c_size_t, [_I, _I]),
        "tkv_t2_update": (_I, [ctypes.POINTER(tkv_model), _I, _P, _I, _P, _P, _P, _P, _P, _P,
                               _P, _I, _P, _P, _P, _P, _I, _I, _P, _P, ctypes.c_size_t, _P]),
        "tkv_update_scores": (_I, [ctypes.POINTER(tkv_model), _I, _I, _I, _P, _I, _P, _P, _I,
                                   _P, _P, _I, _P, _I, _P]),
        "tkv_assign_tiers": (_I, [_I, _P, _I, _P, ctypes.POINTER(tkv_policy), _P, _P, _P, _P]),
        "tkv_compact_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(tkv_model), _I, _I,
                                                          _I, _I]),
        "tkv_compact": (_I, [ctypes.POINTER(tkv_model), _I, _P, _I, _P, _P, _P, _P, _P, _P,
                             _I, _P, _P, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P,
                             ctypes.c_size_t, _P]),
        "tkv_quantize_t2": (_I, [ctypes.POINTER(tkv_model), _I, _P, _P, _I, _P, _P, _I, _P,
                                 _P, _I, _I, _P, _P, _P]),
        "tkv_gather_t1": (_I, [ctypes.POINTER(tkv_model), _P, _P, _I, _P, _I, _P, _I, _P, _P,
                               _P]),
        "tkv_t0_capacity": (_I, [ctypes.POINTER(tkv_policy), _I, _I]),
        "tkv_compact_host_t1_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(tkv_model),
                                                                  _I, _I, _I, _I]),
        "tkv_compact_host_t1_scratch_bytes": (ctypes.c_size_t, [ctypes.POINTER(tkv_model), _I,
                                                                _I, _I]),
        "tkv_compact_host_t1": (_I, [ctypes.POINTER(tkv_model), _I, _P, _I, _P, _P, _P, _P, _P,
                                     _P, _I, _P, _P, _I, _P, _P, _P, _P, _P, _I, _P, _P, _P,
                                     _P, _P, ctypes.c_size_t, _P, ctypes.c_size_t,
                                     ctypes.POINTER(ctypes.c_int64), _P]),
        "tkv_read_probe": (_I, [_P, ctypes.c_size_t, _I, _P, _P]),
        "tkv_timing_enable": (_I, [_I]),
        "tkv_timing_select": (_I, [ctypes.c_char_p]),
        "tkv_timing_reset": (_I, []),
        "tkv_timing_read": (_I, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    found = L.tkv_abi_version()
    if found != ABI_VERSION:
        raise ImportError(f"{_LIB_PATH} has ABI version {found}, this binding expects "
                          f"{ABI_VERSION}: rebuild it with `python -m tiered_kv_cache_amd.build`")
    _lib = L
    return L


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot pass {type(x)} as a pointer")


class _HostInts:
    """Keeps a contiguous int32 copy alive for the duration of a call."""

    def __init__(self, seq):
        self.arr = None if seq is None else np.ascontiguousarray(np.asarray(seq, dtype=np.int32))

    @property
    def ptr(self):
        return None if self.arr is None else self.arr.ctypes.data


def _stream(s) -> Optional[int]:
    if s is None:
        try:
            import torch
            return torch.cuda.current_stream().cuda_stream
        except Exception:
            return None
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    raise TypeError("stream must be a torch stream or a raw handle")


def _event(e) -> Optional[int]:
    if e is None or isinstance(e, int):
        return e
    if hasattr(e, "cuda_event"):
        return e.cuda_event
    raise TypeError("event must be a torch event or a raw handle")


def _check(status: int, where: str) -> None:
    if status != TKV_OK:
        msg = lib().tkv_last_error()
        raise TkvError(status, where, msg.decode() if msg else "")


def make_model(layers: int, q_heads: int, kv_heads: int, head_dim: int, kv_dtype: int,
               softmax_scale: float = 0.0, alpha_scratch: bool = False,
               t0_caps=None, t1_caps=None) -> tkv_model:
    """t0_caps / t1_caps: per-sequence pool capacities (sequences of int, or None); the
    model keeps its own int32 copies alive (set_caps replaces them)."""
    m = tkv_model(layers, q_heads, kv_heads, head_dim, kv_dtype, softmax_scale,
                  1 if alpha_scratch else 0, None, None)
    set_caps(m, t0_caps, t1_caps)
    return m


def set_caps(m: tkv_model, t0_caps=None, t1_caps=None) -> None:
    """Per-sequence pool capacities of a model (None: the calls' cap0 / cap1 for all)."""
    m._caps = [None if c is None else np.ascontiguousarray(np.asarray(c, dtype=np.int32))
               for c in (t0_caps, t1_caps)]
    m.t0_caps = None if m._caps[0] is None else m._caps[0].ctypes.data
    m.t1_caps = None if m._caps[1] is None else m._caps[1].ctypes.data


def make_policy(prompt: int, sinks: int, recent: int, f1: float, f2: float, f3: float,
                delta: int) -> tkv_policy:
    return tkv_policy(prompt, sinks, recent, f1, f2, f3, delta)


# --------------------------------------------------------------------------
# the ABI, one function per entry point
# --------------------------------------------------------------------------
def tkv_abi_version() -> int:
    return lib().tkv_abi_version()


def tkv_append(model, batch, k_new, v_new, k_t0, v_t0, cap0, t0_len, t0_pos, position,
               scores=None, tier=None, max_ctx=0, stream=None) -> None:
    a, b = _HostInts(t0_len), _HostInts(position)
    _check(lib().tkv_append(ctypes.byref(model), batch, _ptr(k_new), _ptr(v_new), _ptr(k_t0),
                            _ptr(v_t0), cap0, a.ptr, _ptr(t0_pos), b.ptr, _ptr(scores),
                            _ptr(tier), max_ctx, _stream(stream)), "tkv_append")


def tkv_decode_workspace_bytes(model, batch, n_layers, cap0, cap1) -> int:
    return lib().tkv_decode_workspace_bytes(ctypes.byref(model), batch, n_layers, cap0, cap1)


def tkv_decode_step(model, batch, layer_begin, layer_end, q, k_t0, v_t0, t0_len, cap0, k_t1,
                    v_t1, t1_len, cap1, out, alpha, alpha_stride, t0_pos=None, t1_pos=None,
                    scores=None, max_ctx=0, workspace=None, workspace_bytes=0,
                    stream=None) -> None:
    a, b = _HostInts(t0_len), _HostInts(t1_len)
    _check(lib().tkv_decode_step(ctypes.byref(model), batch, layer_begin, layer_end, _ptr(q),
                                 _ptr(k_t0), _ptr(v_t0), a.ptr, cap0, _ptr(k_t1), _ptr(v_t1),
                                 b.ptr, cap1, _ptr(out), _ptr(alpha), alpha_stride,
                                 _ptr(t0_pos), _ptr(t1_pos), _ptr(scores), max_ctx,
                                 _ptr(workspace), workspace_bytes, _stream(stream)),
           "tkv_decode_step")


def tkv_decode_step_noalloc(model, batch, layer_begin, layer_end, q, k_t0, v_t0, t0_len, cap0,
                            k_t1, v_t1, t1_len, cap1, out, alpha, alpha_stride, t0_pos=None,
                            t1_pos=None, scores=None, max_ctx=0, stream=None) -> None:
    a, b = _HostInts(t0_len), _HostInts(t1_len)
    _check(lib().tkv_decode_step_noalloc(ctypes.byref(model), batch, layer_begin, layer_end,
                                         _ptr(q), _ptr(k_t0), _ptr(v_t0), a.ptr, cap0,
                                         _ptr(k_t1), _ptr(v_t1), b.ptr, cap1, _ptr(out),
                                         _ptr(alpha), alpha_stride, _ptr(t0_pos), _ptr(t1_pos),
                                         _ptr(scores), max_ctx, _stream(stream)),
           "tkv_decode_step_noalloc")


def tkv_append_decode_step(model, batch, k_new, v_new, position, tier, q, k_t0, v_t0, t0_len,
                           cap0, k_t1, v_t1, t1_len, cap1, out, alpha, alpha_stride, t0_pos,
                           t1_pos=None, scores=None, max_ctx=0, workspace=None,
                           workspace_bytes=0, stream=None) -> None:
    a, b, p = _HostInts(t0_len), _HostInts(t1_len), _HostInts(position)
    _check(lib().tkv_append_decode_step(ctypes.byref(model), batch, _ptr(k_new), _ptr(v_new),
                                        p.ptr, _ptr(tier), _ptr(q), _ptr(k_t0), _ptr(v_t0),
                                        a.ptr, cap0, _ptr(k_t1), _ptr(v_t1), b.ptr, cap1,
                                        _ptr(out), _ptr(alpha), alpha_stride, _ptr(t0_pos),
                                        _ptr(t1_pos), _ptr(scores), max_ctx, _ptr(workspace),
                                        workspace_bytes, _stream(stream)),
           "tkv_append_decode_step")


def tkv_decode_step_window(model, batch, layer_begin, layer_end, q, k_t0, v_t0, t0_len, cap0,
                           t1_win, t1_len, cap1, out, alpha, alpha_stride, t0_pos=None,
                           t1_pos=None, scores=None, max_ctx=0, workspace=None,
                           workspace_bytes=0, stream=None) -> None:
    a, b = _HostInts(t0_len), _HostInts(t1_len)
    _check(lib().tkv_decode_step_window(ctypes.byref(model), batch, layer_begin, layer_end,
                                        _ptr(q), _ptr(k_t0), _ptr(v_t0), a.ptr, cap0,
                                        _ptr(t1_win), b.ptr, cap1, _ptr(out), _ptr(alpha),
                                        alpha_stride, _ptr(t0_pos), _ptr(t1_pos), _ptr(scores),
                                        max_ctx, _ptr(workspace), workspace_bytes,
                                        _stream(stream)), "tkv_decode_step_window")


def tkv_decode_step_streamed(model, batch, q, k_t0, v_t0, t0_len, cap0, host_t1, t1_len, cap1,
                             win, chunk_layers, out, alpha, alpha_stride, t0_pos, t1_pos,
                             scores, max_ctx, workspace, workspace_bytes, stream, side_stream,
                             events, side_stream2=None) -> int:
    """Returns the bytes queued host -> device."""
    a, b = _HostInts(t0_len), _HostInts(t1_len)
    ev = (ctypes.c_void_p * 4)(*[_event(e) for e in events])
    link = ctypes.c_int64()
    _check(lib().tkv_decode_step_streamed(ctypes.byref(model), batch, _ptr(q), _ptr(k_t0),
                                          _ptr(v_t0), a.ptr, cap0, _ptr(host_t1), b.ptr, cap1,
                                          _ptr(win), chunk_layers, _ptr(out), _ptr(alpha),
                                          alpha_stride, _ptr(t0_pos), _ptr(t1_pos),
                                          _ptr(scores), max_ctx, _ptr(workspace),
                                          workspace_bytes, _stream(stream),
                                          _stream(side_stream),
                                          None if side_stream2 is None else _stream(side_stream2),
                                          ev, ctypes.byref(link)),
           "tkv_decode_step_streamed")
    return link.value


class T2Pool:
    """A tkv_t2_pool with the host length array it points to kept alive."""

    def __init__(self, k_codes, v_codes, k_scale, v_scale, t2_pos, t2_len, cap2):
        self._len = _HostInts(t2_len)
        self.struct = tkv_t2_pool(_ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale),
                                  _ptr(t2_pos), self._len.ptr, cap2)


def tkv_decode_step_t2(model, batch, layer_begin, layer_end, q, k_t0, v_t0, t0_len, cap0, k_t1,
                       v_t1, t1_len, cap1, t2: Optional[T2Pool], out, alpha, alpha_stride,
                       t0_pos=None, t1_pos=None, scores=None, max_ctx=0, workspace=None,
                       workspace_bytes=0, stream=None) -> None:
    a, b = _HostInts(t0_len), _HostInts(t1_len)
    _check(lib().tkv_decode_step_t2(ctypes.byref(model), batch, layer_begin, layer_end, _ptr(q),
                                    _ptr(k_t0), _ptr(v_t0), a.ptr, cap0, _ptr(k_t1), _ptr(v_t1),
                                    b.ptr, cap1, None if t2 is None else ctypes.byref(t2.struct),
                                    _ptr(out), _ptr(alpha), alpha_stride, _ptr(t0_pos),
                                    _ptr(t1_pos), _ptr(scores), max_ctx, _ptr(workspace),
                                    workspace_bytes, _stream(stream)), "tkv_decode_step_t2")


def tkv_append_decode_step_t2(model, batch, k_new, v_new, position, tier, q, k_t0, v_t0, t0_len,
                              cap0, k_t1, v_t1, t1_len, cap1, t2: Optional[T2Pool], out, alpha,
                              alpha_stride, t0_pos, t1_pos=None, scores=None, max_ctx=0,
                              workspace=None, workspace_bytes=0, stream=None) -> None:
    a, b, p = _HostInts(t0_len), _HostInts(t1_len), _HostInts(position)
    _check(lib().tkv_append_decode_step_t2(
        ctypes.byref(model), batch, _ptr(k_new), _ptr(v_new), p.ptr, _ptr(tier), _ptr(q),
        _ptr(k_t0), _ptr(v_t0), a.ptr, cap0, _ptr(k_t1), _ptr(v_t1), b.ptr, cap1,
        None if t2 is None else ctypes.byref(t2.struct), _ptr(out), _ptr(alpha), alpha_stride,
        _ptr(t0_pos), _ptr(t1_pos), _ptr(scores), max_ctx, _ptr(workspace), workspace_bytes,
        _stream(stream)), "tkv_append_decode_step_t2")


def tkv_t2_update_workspace_bytes(batch, cap2) -> int:
    return lib().tkv_t2_update_workspace_bytes(batch, cap2)


def tkv_t2_update(model, batch, ctx_len, max_ctx, tier_next, k_codes, v_codes, k_scale,
                  v_scale, t2_pos, t2_len, cap2, new_pos, new_codes, new_scales, n_new,
                  n_new_stride, max_rows, new_t2_len, workspace, workspace_bytes,
                  stream=None) -> None:
    a, b = _HostInts(ctx_len), _HostInts(t2_len)
    _check(lib().tkv_t2_update(ctypes.byref(model), batch, a.ptr, max_ctx, _ptr(tier_next),
                               _ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale),
                               _ptr(t2_pos), b.ptr, cap2, _ptr(new_pos), _ptr(new_codes),
                               _ptr(new_scales), _ptr(n_new), n_new_stride, max_rows,
                               _ptr(new_t2_len), _ptr(workspace), workspace_bytes,
                               _stream(stream)), "tkv_t2_update")


def tkv_update_scores(model, batch, layer_begin, layer_end, alpha, alpha_stride, t0_pos,
                      t0_len, cap0, t1_pos, t1_len, cap1, scores, max_ctx, stream=None) -> None:
    a, b = _HostInts(t0_len), _HostInts(t1_len)
    _check(lib().tkv_update_scores(ctypes.byref(model), batch, layer_begin, layer_end,
                                   _ptr(alpha), alpha_stride, _ptr(t0_pos), a.ptr, cap0,
                                   _ptr(t1_pos), b.ptr, cap1, _ptr(scores), max_ctx,
                                   _stream(stream)), "tkv_update_scores")


def tkv_assign_tiers(batch, ctx_len, max_ctx, scores, policy, tier_prev, tier_next, counts,
                     stream=None) -> None:
    a = _HostInts(ctx_len)
    _check(lib().tkv_assign_tiers(batch, a.ptr, max_ctx, _ptr(scores), ctypes.byref(policy),
                                  _ptr(tier_prev), _ptr(tier_next), _ptr(counts),
                                  _stream(stream)), "tkv_assign_tiers")


def tkv_compact_workspace_bytes(model, batch, max_ctx, cap0, cap1) -> int:
    return lib().tkv_compact_workspace_bytes(ctypes.byref(model), batch, max_ctx, cap0, cap1)


def tkv_compact(model, batch, ctx_len, max_ctx, tier_prev, tier_next, k_t0, v_t0, t0_pos,
                t0_len, cap0, k_t1, v_t1, t1_pos, t1_len, cap1, t2_src, t2_pos, t2_cap,
                t2_codes, t2_scales, new_lens, workspace, workspace_bytes, stream=None) -> None:
    a, b, c = _HostInts(ctx_len), _HostInts(t0_len), _HostInts(t1_len)
    _check(lib().tkv_compact(ctypes.byref(model), batch, a.ptr, max_ctx, _ptr(tier_prev),
                             _ptr(tier_next), _ptr(k_t0), _ptr(v_t0), _ptr(t0_pos), b.ptr,
                             cap0, _ptr(k_t1), _ptr(v_t1), _ptr(t1_pos), c.ptr, cap1,
                             _ptr(t2_src), _ptr(t2_pos), t2_cap, _ptr(t2_codes),
                             _ptr(t2_scales), _ptr(new_lens), _ptr(workspace), workspace_bytes,
                             _stream(stream)), "tkv_compact")


def tkv_quantize_t2(model, batch, k_t0, v_t0, cap0, k_t1, v_t1, cap1, src, n_rows,
                    n_rows_stride, max_rows, codes, scales, stream=None) -> None:
    _check(lib().tkv_quantize_t2(ctypes.byref(model), batch, _ptr(k_t0), _ptr(v_t0), cap0,
                                 _ptr(k_t1), _ptr(v_t1), cap1, _ptr(src), _ptr(n_rows),
                                 n_rows_stride, max_rows, _ptr(codes), _ptr(scales),
                                 _stream(stream)), "tkv_quantize_t2")


def tkv_gather_t1(model, host_k, host_v, max_ctx, positions, n_t1, staging, cap1, dev_t1=None,
                  side_stream=None, ready=None) -> None:
    p = _HostInts(positions)
    _check(lib().tkv_gather_t1(ctypes.byref(model), _ptr(host_k), _ptr(host_v), max_ctx, p.ptr,
                               n_t1, _ptr(staging), cap1, _ptr(dev_t1), _stream(side_stream),
                               _event(ready)), "tkv_gather_t1")


def tkv_t0_capacity(policy, n_from, n_to) -> int:
    cap = lib().tkv_t0_capacity(ctypes.byref(policy), n_from, n_to)
    if cap < 0:
        raise TkvError(cap, "tkv_t0_capacity", "bad policy or range")
    return cap


def tkv_compact_host_t1_workspace_bytes(model, batch, max_ctx, cap0, cap1) -> int:
    return lib().tkv_compact_host_t1_workspace_bytes(ctypes.byref(model), batch, max_ctx, cap0,
                                                     cap1)


def tkv_compact_host_t1_scratch_bytes(model, batch, max_ctx, cap1) -> int:
    return lib().tkv_compact_host_t1_scratch_bytes(ctypes.byref(model), batch, max_ctx, cap1)


def tkv_compact_host_t1(model, batch, ctx_len, max_ctx, tier_prev, tier_next, k_t0, v_t0, t0_pos,
                        t0_len, cap0, t1_pos, t1_len, cap1, store_k, store_v, t1_host, t2_src,
                        t2_pos, t2_cap, t2_codes, t2_scales, new_lens, workspace,
                        workspace_bytes, host_scratch, host_scratch_bytes, stream=None):
    """Returns (new lengths [B][4] as a NumPy array, bytes that crossed the host link)."""
    a, b, c = _HostInts(ctx_len), _HostInts(t0_len), _HostInts(t1_len)
    lens = np.zeros((batch, 4), dtype=np.int32)
    link = ctypes.c_int64()
    _check(lib().tkv_compact_host_t1(ctypes.byref(model), batch, a.ptr, max_ctx, _ptr(tier_prev),
                                     _ptr(tier_next), _ptr(k_t0), _ptr(v_t0), _ptr(t0_pos), b.ptr,
                                     cap0, _ptr(t1_pos), c.ptr, cap1, _ptr(store_k),
                                     _ptr(store_v), _ptr(t1_host), _ptr(t2_src), _ptr(t2_pos),
                                     t2_cap, _ptr(t2_codes), _ptr(t2_scales), _ptr(new_lens),
                                     lens.ctypes.data, _ptr(workspace), workspace_bytes,
                                     _ptr(host_scratch), host_scratch_bytes, ctypes.byref(link),
                                     _stream(stream)), "tkv_compact_host_t1")
    return lens, link.value


def tkv_read_probe(buf, nbytes, waves, sink, stream=None) -> None:
    _check(lib().tkv_read_probe(_ptr(buf), nbytes, waves, _ptr(sink), _stream(stream)),
           "tkv_read_probe")


def tkv_timing_enable(enable: bool) -> None:
    _check(lib().tkv_timing_enable(1 if enable else 0), "tkv_timing_enable")


def tkv_timing_select(kernels=None) -> None:
    """Time only the named kernels (an iterable of names, or None for every kernel)."""
    arg = None if kernels is None else ",".join(kernels).encode()
    _check(lib().tkv_timing_select(arg), "tkv_timing_select")


def tkv_timing_reset() -> None:
    _check(lib().tkv_timing_reset(), "tkv_timing_reset")


def tkv_timing_read(kernel: str):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().tkv_timing_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)),
           "tkv_timing_read")
    return ms.value, n.value
