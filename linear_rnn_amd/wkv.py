"""Thin ctypes binding of librwkv7_wkv.so (argument marshalling only).

Function names match the C ABI in include/rwkv7_wkv.h. Each takes torch tensors
(device memory owned by the caller) or None, passes their addresses, sizes and
dtype to the library, launches on the current torch stream unless a stream is
given, and raises RuntimeError with the library's message on a non-zero status.
Before the call it checks every tensor against the sizes the call takes (shape,
one input dtype, contiguity, 16-byte alignment, one HIP device) and raises
ValueError on a mismatch: the C ABI receives bare pointers and cannot.
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
RWKV7_ERR_SCRATCH = -9
RWKV7_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = ("rwkv7_wkv_prefill", "rwkv7_wkv_step", "rwkv7_wkv_step_q", "rwkv7_wkv_prefill_ex",
            "rwkv7_tmix_prefill", "rwkv7_tmix_prefill_ex", "rwkv7_tmix_step", "rwkv7_wkv_backward",
            "rwkv7_wkv_backward_ex",
            "rwkv7_stack_forward", "rwkv7_wkv_prefill_algo", "rwkv7_wkv_prefill_noalloc",
            "rwkv7_wkv_strerror")

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
            for name in ("rwkv7_wkv_prefill", "rwkv7_wkv_step", "rwkv7_wkv_prefill_noalloc"):
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
            L.rwkv7_wkv_backward_ex.restype = ci
            L.rwkv7_wkv_backward_ex.argtypes = [vp] * 16 + [i64] * 4 + [ci, ci, vp]
            L.rwkv7_stack_forward.restype = ci
            L.rwkv7_stack_forward.argtypes = [vp] * 5 + [i64] * 5 + [ci, vp]
            L.rwkv7_wkv_prefill_algo.restype = ci
            L.rwkv7_wkv_prefill_algo.argtypes = [i64] * 4 + [ci]
            L.rwkv7_wkv_strerror.restype = ctypes.c_char_p
            L.rwkv7_wkv_strerror.argtypes = [ci]
            _lib = L
    return _lib


def rwkv7_wkv_prefill_algo(B: int, T: int, H: int, N: int = 64, dtype: int = RWKV7_DTYPE_BF16) -> int:
    """The RWKV7_ALGO_* value that rwkv7_wkv_prefill runs for this shape and dtype (raises on invalid sizes)."""
    st = lib().rwkv7_wkv_prefill_algo(int(B), int(T), int(H), int(N), int(dtype))
    _check(min(st, 0))
    return st


def rwkv7_wkv_strerror(status: int) -> str:
    return lib().rwkv7_wkv_strerror(int(status)).decode()


def _ptr(t):
    return None if t is None else (t.data_ptr() or None)


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


# ---- argument checks. The C ABI sees raw pointers and cannot check a buffer's size,
# layout or device, so every tensor is checked here against the sizes the call takes
# from r (or the state / residual stream) before the library is called. Shapes,
# dtypes, contiguity and alignment are checked first and the device last, so each
# mistake is named even for host tensors.

def _expect(t, name, shape, dtypes, like, optional=False):
    """Raise unless t is a contiguous, 16-byte aligned tensor of this shape and dtype on like's device."""
    import torch
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, not %s" % (name, type(t).__name__))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, " or ".join(str(d) for d in dtypes)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (row-major), got strides %s" % (name, tuple(t.stride())))
    if t.numel() and t.data_ptr() % 16:
        raise ValueError("%s must be 16-byte aligned" % name)
    if t.device != like.device:
        raise ValueError("%s is on %s, the other tensors on %s" % (name, t.device, like.device))


def _on_gpu(like, stream):
    """The tensors must be device memory of the device the kernels launch on."""
    import torch
    if like.device.type != "cuda":
        raise ValueError("tensors must be on a HIP device (torch 'cuda'), got %s" % like.device)
    if stream is None and like.device.index != torch.cuda.current_device():
        raise ValueError("tensors are on %s but the current device is cuda:%d; pass a stream of that device or "
                         "select it" % (like.device, torch.cuda.current_device()))


def _input_dtypes():
    import torch
    return (torch.bfloat16, torch.float32)


def _f32():
    import torch
    return (torch.float32,)


def _args(r, w, k, v, a, b, state_in, y, state_out, stream=None, state_dtypes=None):
    """Checked arguments of the prefill / step entry points (pointers, sizes, input dtype code)."""
    import torch
    if not isinstance(r, torch.Tensor) or r.dim() != 4:
        raise ValueError("r must be a [B, T, H, N] tensor")
    B, T, H, N = r.shape
    _expect(r, "r", r.shape, _input_dtypes(), r)
    for name, t in zip("wkvab", (w, k, v, a, b)):
        _expect(t, name, r.shape, (r.dtype,), r)
    _expect(y, "y", (B, T, H, N), _f32(), r)
    sd = state_dtypes or _f32()
    _expect(state_in, "state_in", (B, H, N, N), sd, r, optional=True)
    _expect(state_out, "state_out", (B, H, N, N), sd, r, optional=True)
    _on_gpu(r, stream)
    return [_ptr(x) for x in (r, w, k, v, a, b, state_in, y, state_out)] + [B, T, H, N, _dtype_code(r)]


def _check(status: int):
    if status != RWKV7_OK:
        raise Rwkv7Error(status, rwkv7_wkv_strerror(status))


def rwkv7_wkv_prefill(r, w, k, v, a, b, state_in, y, state_out, stream=None):
    """Whole-sequence prefill. Tensors as in include/rwkv7_wkv.h ([B,T,H,64] inputs, float32 y and state)."""
    args = _args(r, w, k, v, a, b, state_in, y, state_out, stream)
    _check(lib().rwkv7_wkv_prefill(*args, _stream(stream)))


def rwkv7_wkv_prefill_noalloc(r, w, k, v, a, b, state_in, y, state_out, stream=None):
    """The split chunked prefill with its records in the library's static device array (allocates nothing;
    bfloat16 inputs; calls on one device must not overlap)."""
    args = _args(r, w, k, v, a, b, state_in, y, state_out, stream)
    _check(lib().rwkv7_wkv_prefill_noalloc(*args, _stream(stream)))


def rwkv7_wkv_step(r, w, k, v, a, b, state_in, y, state_out, stream=None):
    """Single-token step (T == 1); state_out may be state_in for an in-place update."""
    args = _args(r, w, k, v, a, b, state_in, y, state_out, stream)
    _check(lib().rwkv7_wkv_step(*args, _stream(stream)))


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
    import torch
    sd = _state_code(state_in, state_out) if state_dtype is None else int(state_dtype)
    tdt = {RWKV7_STATE_F32: torch.float32, RWKV7_STATE_BF16: torch.bfloat16, RWKV7_STATE_F16: torch.float16}
    if sd not in tdt:
        raise ValueError("state_dtype must be one of RWKV7_STATE_F32 / _BF16 / _F16")
    args = _args(r, w, k, v, a, b, state_in, y, state_out, stream, state_dtypes=(tdt[sd],))
    _check(lib().rwkv7_wkv_step_q(*args, sd, _stream(stream)))


def rwkv7_wkv_prefill_ex(r, w, k, v, a, b, state_in, y, state_out, algo=RWKV7_ALGO_AUTO, stream=None):
    """Prefill with an explicit algorithm (RWKV7_ALGO_*)."""
    args = _args(r, w, k, v, a, b, state_in, y, state_out, stream)
    _check(lib().rwkv7_wkv_prefill_ex(*args, int(algo), _stream(stream)))


def wkv7(r, w, k, v, a, b, state_in=None, algo=RWKV7_ALGO_AUTO, want_state=True, stream=None):
    """Allocate y ([B,T,H,64] float32) and the final state, run the prefill, return (y, state_out)."""
    import torch
    B, T, H, N = r.shape
    y = torch.empty((B, T, H, N), dtype=torch.float32, device=r.device)
    s_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device) if want_state else None
    rwkv7_wkv_prefill_ex(r, w, k, v, a, b, state_in, y, s_out, algo=algo, stream=stream)
    return y, s_out


def _tmix_args(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, stream=None):
    import torch
    if not isinstance(r, torch.Tensor) or r.dim() != 4:
        raise ValueError("r must be a [B, T, H, N] tensor")
    B, T, H, N = r.shape
    _expect(r, "r", r.shape, _input_dtypes(), r)
    for name, t in (("k", k), ("v", v), ("kk", kk), ("a_lr", a_lr)):
        _expect(t, name, r.shape, (r.dtype,), r)
    _expect(w_raw, "w_raw", r.shape, _f32(), r)
    _expect(ln_w, "ln_w", (H * N,), _f32(), r, optional=True)
    _expect(ln_b, "ln_b", (H * N,), _f32(), r, optional=True)
    _expect(state_in, "state_in", (B, H, N, N), _f32(), r, optional=True)
    _expect(out, "out", (B, T, H, N), _f32(), r)
    _expect(state_out, "state_out", (B, H, N, N), _f32(), r, optional=True)
    _on_gpu(r, stream)
    return [_ptr(x) for x in (r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out)] + \
        [B, T, H, N, _dtype_code(r)]


def rwkv7_tmix_prefill(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, stream=None):
    """Fused time-mix prefill: prologue (decay, normalised removal key, slots), recurrence, ln_x."""
    args = _tmix_args(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, stream)
    _check(lib().rwkv7_tmix_prefill(*args, _stream(stream)))


def rwkv7_tmix_prefill_ex(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, algo=RWKV7_ALGO_AUTO,
                          stream=None):
    """Fused time-mix prefill with an explicit algorithm (RWKV7_ALGO_AUTO / _SEQUENTIAL / _CHUNKED /
    _CHUNKED_SPLIT)."""
    args = _tmix_args(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, stream)
    _check(lib().rwkv7_tmix_prefill_ex(*args, int(algo), _stream(stream)))


def rwkv7_tmix_step(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, stream=None):
    """Fused time-mix single-token step (T == 1); state_out may be state_in."""
    args = _tmix_args(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, stream)
    _check(lib().rwkv7_tmix_step(*args, _stream(stream)))


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
    rwkv7_wkv_backward_ex(r, w, k, v, a, b, state_in, dy, dstate_out, dr, dw, dk, dv, da, db, dstate_in,
                          RWKV7_ALGO_AUTO, stream)


def rwkv7_wkv_backward_ex(r, w, k, v, a, b, state_in, dy, dstate_out, dr, dw, dk, dv, da, db, dstate_in,
                          algo=RWKV7_ALGO_AUTO, stream=None):
    """rwkv7_wkv_backward with an explicit algorithm (RWKV7_ALGO_AUTO / _SEQUENTIAL / _CHUNKED)."""
    import torch
    if not isinstance(r, torch.Tensor) or r.dim() != 4:
        raise ValueError("r must be a [B, T, H, N] tensor")
    B, T, H, N = r.shape
    _expect(r, "r", r.shape, _input_dtypes(), r)
    for name, t in zip("wkvab", (w, k, v, a, b)):
        _expect(t, name, r.shape, (r.dtype,), r)
    _expect(state_in, "state_in", (B, H, N, N), _f32(), r, optional=True)
    _expect(dy, "dy", (B, T, H, N), _f32(), r)
    _expect(dstate_out, "dstate_out", (B, H, N, N), _f32(), r, optional=True)
    for name, t in zip(("dr", "dw", "dk", "dv", "da", "db"), (dr, dw, dk, dv, da, db)):
        _expect(t, name, (B, T, H, N), _f32(), r)
    _expect(dstate_in, "dstate_in", (B, H, N, N), _f32(), r, optional=True)
    _on_gpu(r, stream)
    args = [_ptr(x) for x in (r, w, k, v, a, b, state_in, dy, dstate_out, dr, dw, dk, dv, da, db, dstate_in)]
    _check(lib().rwkv7_wkv_backward_ex(*args, B, T, H, N, _dtype_code(r), int(algo), _stream(stream)))


def wkv7_backward(r, w, k, v, a, b, dy, state_in=None, dstate_out=None, want_dstate=True, stream=None,
                  algo=RWKV7_ALGO_AUTO):
    """Allocate the gradients, run the backward, return dict dr, dw, dk, dv, da, db, dstate_in."""
    import torch
    B, T, H, N = r.shape
    out = {n: torch.empty((B, T, H, N), dtype=torch.float32, device=r.device)
           for n in ("dr", "dw", "dk", "dv", "da", "db")}
    out["dstate_in"] = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device) if want_dstate else None
    rwkv7_wkv_backward_ex(r, w, k, v, a, b, state_in, dy, dstate_out, *(out[n] for n in
                          ("dr", "dw", "dk", "dv", "da", "db", "dstate_in")), algo=algo, stream=stream)
    return out


def rwkv7_stack_forward(w_in, w_out, vecs, x, states, stream=None):
    """L time-mix layers over the residual stream x ([B,T,D] float32, in place) with per-layer states
    ([L,B,H,64,64] float32, in place). w_in [L,D,5D] and w_out [L,D,D] in float32 or bfloat16."""
    import torch
    if not isinstance(states, torch.Tensor) or states.dim() != 5:
        raise ValueError("states must be an [L, B, H, N, N] tensor")
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [B, T, D] tensor")
    L, B, H, N = states.shape[0], states.shape[1], states.shape[2], states.shape[3]
    T, D = x.shape[1], H * N
    _expect(states, "states", (L, B, H, N, N), _f32(), states)
    _expect(x, "x", (B, T, D), _f32(), states)
    _expect(w_in, "w_in", (L, D, 5 * D), _input_dtypes(), states)
    _expect(w_out, "w_out", (L, D, D), (w_in.dtype,), states)
    _expect(vecs, "vecs", (L, 5, D), _f32(), states)
    _on_gpu(states, stream)
    args = [_ptr(w_in), _ptr(w_out), _ptr(vecs), _ptr(x), _ptr(states), L, B, T, H, N, _dtype_code(w_in)]
    _check(lib().rwkv7_stack_forward(*args, _stream(stream)))
