"""Thin ctypes binding of librwkv7_wkv.so (argument marshalling only).

Function names match the C ABI in include/rwkv7_wkv.h. Each takes torch tensors
(device memory owned by the caller) or None, passes their addresses, sizes and
dtype to the library, launches on the current torch stream unless a stream is
given, and raises RuntimeError with the library's message on a non-zero status.
Every step of the computation runs in the HIP kernels; there is no fallback:
if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librwkv7_wkv.so")

RWKV7_OK = 0
RWKV7_DTYPE_F32 = 0
RWKV7_DTYPE_BF16 = 1
RWKV7_STATE_F32 = 0
RWKV7_STATE_BF16 = 1
RWKV7_STATE_F16 = 2
RWKV7_ALGO_AUTO = 0
RWKV7_ALGO_SEQUENTIAL = 1
RWKV7_ALGO_CHUNKED = 2
RWKV7_ALGO_CHUNKED_SPLIT = 3

EXPORTED = ("rwkv7_wkv_prefill", "rwkv7_wkv_step", "rwkv7_wkv_step_q", "rwkv7_wkv_prefill_ex",
            "rwkv7_tmix_prefill", "rwkv7_tmix_prefill_ex", "rwkv7_tmix_step", "rwkv7_wkv_backward",
            "rwkv7_stack_forward", "rwkv7_wkv_strerror")

_lib = None
_lock = threading.Lock()


class Rwkv7Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("rwkv7 status %d: %s" % (status, msg))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises OSError if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise OSError("HIP library %s is missing: run `python -m linear_rnn_amd.build`" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            sig = [vp] * 9 + [i64] * 4 + [ci]
            for name in ("rwkv7_wkv_prefill", "rwkv7_wkv_step"):
                f = getattr(L, name)
                f.restype = ci
                f.argtypes = sig + [vp]
            L.rwkv7_wkv_step_q.restype = ci
            L.rwkv7_wkv_step_q.argtypes = sig + [ci, vp]
            L.rwkv7_wkv_prefill_ex.restype = ci
            L.rwkv7_wkv_prefill_ex.argtypes = sig + [ci, vp]
            for name in ("rwkv7_tmix_prefill", "rwkv7_tmix_step"):
                f = getattr(L, name)
                f.restype = ci
                f.argtypes = [vp] * 11 + [i64] * 4 + [ci, vp]
            L.rwkv7_tmix_prefill_ex.restype = ci
            L.rwkv7_tmix_prefill_ex.argtypes = [vp] * 11 + [i64] * 4 + [ci, ci, vp]
            L.rwkv7_wkv_backward.restype = ci
            L.rwkv7_wkv_backward.argtypes = [vp] * 16 + [i64] * 4 + [ci, vp]
            L.rwkv7_stack_forward.restype = ci
            L.rwkv7_stack_forward.argtypes = [vp] * 5 + [i64] * 5 + [ci, vp]
            L.rwkv7_wkv_strerror.restype = ctypes.c_char_p
            L.rwkv7_wkv_strerror.argtypes = [ci]
            _lib = L
    return _lib


def rwkv7_wkv_strerror(status: int) -> str:
    return lib().rwkv7_wkv_strerror(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t or None
    return t.data_ptr() or None


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return RWKV7_DTYPE_BF16
    if t.dtype == torch.float32:
        return RWKV7_DTYPE_F32
    return -1


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _args(r, w, k, v, a, b, state_in, y, state_out):
    B, T, H, N = r.shape
    return [_ptr(x) for x in (r, w, k, v, a, b, state_in, y, state_out)] + [B, T, H, N, _dtype_code(r)]


def _check(status: int):
    if status != RWKV7_OK:
        raise Rwkv7Error(status, rwkv7_wkv_strerror(status))


def rwkv7_wkv_prefill(r, w, k, v, a, b, state_in, y, state_out, stream=None):
    """Whole-sequence prefill. Tensors as in include/rwkv7_wkv.h ([B,T,H,64] inputs, float32 y and state)."""
    _check(lib().rwkv7_wkv_prefill(*_args(r, w, k, v, a, b, state_in, y, state_out), _stream(stream)))


def rwkv7_wkv_step(r, w, k, v, a, b, state_in, y, state_out, stream=None):
    """Single-token step (T == 1); state_out may be state_in for an in-place update."""
    _check(lib().rwkv7_wkv_step(*_args(r, w, k, v, a, b, state_in, y, state_out), _stream(stream)))


def _state_code(*states) -> int:
    import torch
    codes = {torch.float32: RWKV7_STATE_F32, torch.bfloat16: RWKV7_STATE_BF16, torch.float16: RWKV7_STATE_F16}
    found = {codes.get(s.dtype, -1) for s in states if s is not None}
    if len(found) > 1:
        raise ValueError("state_in and state_out must share one dtype")
    return found.pop() if found else RWKV7_STATE_F32


def rwkv7_wkv_step_q(r, w, k, v, a, b, state_in, y, state_out, state_dtype=None, stream=None):
    """Single-token step with a float32, bfloat16 or float16 stored state (RWKV7_STATE_*).

    The state format is taken from the state tensors' dtype unless `state_dtype` is given.
    """
    sd = _state_code(state_in, state_out) if state_dtype is None else int(state_dtype)
    _check(lib().rwkv7_wkv_step_q(*_args(r, w, k, v, a, b, state_in, y, state_out), sd, _stream(stream)))


def rwkv7_wkv_prefill_ex(r, w, k, v, a, b, state_in, y, state_out, algo=RWKV7_ALGO_AUTO, stream=None):
    """Prefill with an explicit algorithm (RWKV7_ALGO_*)."""
    _check(lib().rwkv7_wkv_prefill_ex(*_args(r, w, k, v, a, b, state_in, y, state_out), int(algo),
                                      _stream(stream)))


def wkv7(r, w, k, v, a, b, state_in=None, algo=RWKV7_ALGO_AUTO, want_state=True, stream=None):
    """Allocate y ([B,T,H,64] float32) and the final state, run the prefill, return (y, state_out)."""
    import torch
    B, T, H, N = r.shape
    y = torch.empty((B, T, H, N), dtype=torch.float32, device=r.device)
    s_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device) if want_state else None
    rwkv7_wkv_prefill_ex(r, w, k, v, a, b, state_in, y, s_out, algo=algo, stream=stream)
    return y, s_out


def _tmix_args(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out):
    B, T, H, N = r.shape
    return [_ptr(x) for x in (r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out)] + \
        [B, T, H, N, _dtype_code(r)]


def rwkv7_tmix_prefill(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, stream=None):
    """Fused time-mix prefill: prologue (decay, normalised removal key, slots), recurrence, ln_x."""
    _check(lib().rwkv7_tmix_prefill(*_tmix_args(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out),
                                    _stream(stream)))


def rwkv7_tmix_prefill_ex(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, algo=RWKV7_ALGO_AUTO,
                          stream=None):
    """Fused time-mix prefill with an explicit algorithm (RWKV7_ALGO_AUTO / _SEQUENTIAL / _CHUNKED_SPLIT)."""
    _check(lib().rwkv7_tmix_prefill_ex(*_tmix_args(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out),
                                       int(algo), _stream(stream)))


def rwkv7_tmix_step(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, stream=None):
    """Fused time-mix single-token step (T == 1); state_out may be state_in."""
    _check(lib().rwkv7_tmix_step(*_tmix_args(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out),
                                 _stream(stream)))


def tmix(r, w_raw, k, v, kk, a_lr, ln_w=None, ln_b=None, state_in=None, want_state=True, algo=RWKV7_ALGO_AUTO,
         stream=None):
    """Allocate out ([B,T,H,64] float32) and the final state, run the fused prefill, return (out, state_out)."""
    import torch
    B, T, H, N = r.shape
    out = torch.empty((B, T, H, N), dtype=torch.float32, device=r.device)
    s_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device) if want_state else None
    rwkv7_tmix_prefill_ex(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, s_out, algo=algo, stream=stream)
    return out, s_out


def rwkv7_wkv_backward(r, w, k, v, a, b, state_in, dy, dstate_out, dr, dw, dk, dv, da, db, dstate_in,
                       stream=None):
    """Gradients of the recurrence: dr..db ([B,T,H,64] float32) and dstate_in ([B,H,64,64] float32 or None)."""
    B, T, H, N = r.shape
    args = [_ptr(x) for x in (r, w, k, v, a, b, state_in, dy, dstate_out, dr, dw, dk, dv, da, db, dstate_in)]
    _check(lib().rwkv7_wkv_backward(*args, B, T, H, N, _dtype_code(r), _stream(stream)))


def wkv7_backward(r, w, k, v, a, b, dy, state_in=None, dstate_out=None, want_dstate=True, stream=None):
    """Allocate the gradients, run the backward, return dict dr, dw, dk, dv, da, db, dstate_in."""
    import torch
    B, T, H, N = r.shape
    out = {n: torch.empty((B, T, H, N), dtype=torch.float32, device=r.device)
           for n in ("dr", "dw", "dk", "dv", "da", "db")}
    out["dstate_in"] = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device) if want_dstate else None
    rwkv7_wkv_backward(r, w, k, v, a, b, state_in, dy, dstate_out, *(out[n] for n in
                       ("dr", "dw", "dk", "dv", "da", "db", "dstate_in")), stream=stream)
    return out


def rwkv7_stack_forward(w_in, w_out, vecs, x, states, stream=None):
    """L time-mix layers over the residual stream x ([B,T,D] float32, in place) with per-layer states
    ([L,B,H,64,64] float32, in place). w_in [L,D,5D] and w_out [L,D,D] in float32 or bfloat16."""
    L, B, H, N = states.shape[0], states.shape[1], states.shape[2], states.shape[3]
    T = x.shape[1]
    _check(lib().rwkv7_stack_forward(_ptr(w_in), _ptr(w_out), _ptr(vecs), _ptr(x), _ptr(states), L, B, T, H, N,
                                     _dtype_code(w_in), _stream(stream)))
