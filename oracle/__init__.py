"""Float64 CPU oracle for the RWKV-7 WKV recurrence.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
benchmark's CPU-baseline leg. The GPU library never imports or links it, and it
imports nothing from the GPU package.

The arithmetic lives in ``wkv7_oracle.c`` (plain C, double precision, compiled
with ``-O2 -ffp-contract=off``). This module compiles it with gcc and calls it
through ctypes. What it computes, per (batch, head), with the state S indexed
[value i, key j]::

    S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T,    y_t = S_t r_t

following the RWKV-7 G0 7.2B notes (lshu.cn/news/198401), section 7.1 (state
decayed by w, plus state*a*b, plus v k^T, then read out with r) and section
3.3 (a zero-initialised float32 [H, N, N] state per layer).

Pins (tests/test_oracle_pins.py, all CPU): brute-force matrix products on tiny
T, the closed forms for a = 0 and for w = 1 with a = 0, an exact rational run,
delta-rule retrieval, the memoryless case, linearity and row equivariance.

``tmix`` adds the operator's prologue (decay exp(-exp(w_raw)), normalised removal
key, kernel slots) and epilogue (ln_x GroupNorm) around the recurrence, in numpy
float64; tests/test_oracle_tmix.py pins those pieces to closed forms and to
torch's normalize and group_norm.

``stack_forward`` runs L time-mix layers over a residual stream (projections in numpy float64,
the operator above), rounding at the points that the model's precision fixes (read from the G0
notes' half-precision model and the README's fp32 note; see its docstring), or nowhere ("f64");
tests/test_oracle_stack.py pins it to the GPT/RNN-mode equivalence and to a composition of torch's
own softplus, sigmoid and matmul.

``wkv7_backward`` runs the C reverse-mode derivatives of the recurrence (every
forward state kept, tokens walked backwards); tests/test_oracle_backward.py pins
it to torch float64 autograd of a plain token loop, to finite differences and
to a closed form, and plants mistakes that the pins must catch.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv7_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_wkv7.so")
_lock = threading.Lock()
_lib = None

IN_F32, IN_BF16, IN_F64, IN_F16 = 0, 1, 2, 3
STATE_FORMATS = {"bf16": IN_BF16, "f16": IN_F16}  # 16-bit stored-state encodings (raw uint16 bits)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle_wkv7.so``."""
    global _lib
    with _lock:
        if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            tmp = _LIB_PATH + ".tmp%d" % os.getpid()
            cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC",
                   "-pthread", _SRC, "-o", tmp, "-lm"]
            subprocess.run(cmd, check=True)
            os.replace(tmp, _LIB_PATH)
            _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        with _lock:
            lib = ctypes.CDLL(_LIB_PATH)
            f = lib.wkv7_oracle_f64
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int64] * 4 + [ctypes.c_int] * 3
            fb = lib.wkv7_oracle_bwd_f64
            fb.restype = ctypes.c_int
            fb.argtypes = [ctypes.c_void_p] * 16 + [ctypes.c_int64] * 4 + [ctypes.c_int] * 3
            for name in ("wkv7_oracle_round16", "wkv7_oracle_widen16"):
                g = getattr(lib, name)
                g.restype = ctypes.c_int
                g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
            _lib = lib
    return _lib


def _in_dtype(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return IN_F32
    if x.dtype == np.uint16:  # raw bfloat16 bits
        return IN_BF16
    if x.dtype == np.float64:
        return IN_F64
    raise TypeError("oracle inputs must be float32, float64 or uint16 (bfloat16 bits), got %s" % x.dtype)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def wkv7(r, w, k, v, a, b, state_in=None, nthreads: int | None = None, want_state: bool = True,
         state_format: str | None = None):
    """Run the float64 recurrence.

    r, w, k, v, a, b: arrays of shape [B, T, H, N], all float32, all float64 or
    all uint16 holding bfloat16 bits. state_in: None (zero state) or an array
    [B, H, N, N] of float32 or float64, or of uint16 encodings in
    `state_format` ("bf16" or "f16"), widened exactly. Returns (y [B,T,H,N]
    float64, state_out [B,H,N,N] float64 or None).
    """
    lib = _load()
    ins = [np.ascontiguousarray(x) for x in (r, w, k, v, a, b)]
    shape = ins[0].shape
    if len(shape) != 4 or any(x.shape != shape for x in ins):
        raise ValueError("r,w,k,v,a,b must share one [B,T,H,N] shape")
    dt = _in_dtype(ins[0])
    if any(_in_dtype(x) != dt for x in ins):
        raise TypeError("r,w,k,v,a,b must share one dtype")
    B, T, H, N = shape
    s_in = None
    st_dt = IN_F64
    if state_in is not None:
        s_in = np.ascontiguousarray(state_in)
        if s_in.shape != (B, H, N, N):
            raise ValueError("state_in must be [B,H,N,N]")
        if s_in.dtype == np.float32:
            st_dt = IN_F32
        elif s_in.dtype == np.float64:
            st_dt = IN_F64
        elif s_in.dtype == np.uint16 and state_format in STATE_FORMATS:
            st_dt = STATE_FORMATS[state_format]
        else:
            raise TypeError("state_in must be float32, float64, or uint16 with state_format 'bf16' or 'f16'")
    y = np.empty((B, T, H, N), dtype=np.float64)
    s_out = np.empty((B, H, N, N), dtype=np.float64) if want_state else None
    p = lambda x: None if x is None else x.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    rc = lib.wkv7_oracle_f64(*(p(x) for x in ins), p(s_in), p(y), p(s_out), B, T, H, N, dt, st_dt,
                             int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle failed with status %d" % rc)
    return y, s_out


def round16(x, fmt: str) -> np.ndarray:
    """Round float64 values to a 16-bit state format ("bf16" or "f16"), ties to even; return the uint16 bits."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    if lib.wkv7_oracle_round16(x.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p), x.size,
                               STATE_FORMATS[fmt]) != 0:
        raise RuntimeError("round16 failed")
    return out


def widen16(bits, fmt: str) -> np.ndarray:
    """Widen 16-bit state encodings ("bf16" or "f16") exactly to float64."""
    lib = _load()
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    if lib.wkv7_oracle_widen16(bits.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p),
                               bits.size, STATE_FORMATS[fmt]) != 0:
        raise RuntimeError("widen16 failed")
    return out


def step_q(r, w, k, v, a, b, state_bits, fmt: str, nthreads: int | None = None):
    """One call of the step with a 16-bit stored state: widen the state, run the
    float64 recurrence over the given tokens, read y from the unrounded state,
    and round the new state to `fmt`. state_bits None means a zero state.
    Returns (y float64, new state bits uint16)."""
    y, s = wkv7(r, w, k, v, a, b, state_in=state_bits, nthreads=nthreads, state_format=fmt)
    return y, round16(s, fmt)


# ---------------------------------------------------------------------------------------------
# The time-mix operator with its prologue and epilogue (RWKV-7 G0 7.2B notes, lshu.cn/news/198401,
# section 7.1, "x070 architecture, the two core operators"): the decay enters as w = exp(-exp(w_raw));
# the removal key kk is L2-normalised per head (F.normalize); the kernel slots are a = -kk and
# b = kk * a_lr (a_lr the in-context learning rate); the recurrence output goes through ln_x, a
# GroupNorm with one group per head and eps = 64e-5.

GROUP_NORM_EPS = 64e-5
NORMALIZE_EPS = 1e-12  # F.normalize divides by max(|x|_2, eps)


def _widen_any(x) -> np.ndarray:
    """Exact float64 value of float32, float64 or raw bfloat16 (uint16) inputs."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError("inputs must be float32, float64 or uint16 (bfloat16 bits), got %s" % x.dtype)


def tmix_prologue(w_raw, kk, a_lr):
    """Float64 decay and kernel slots from the raw inputs (arrays [..., N]).

    w = exp(-exp(w_raw)); kk_hat = kk / max(|kk|_2, 1e-12) over the last (head) axis;
    a = -kk_hat; b = kk_hat * a_lr. Returns (w, a, b).
    """
    u = _widen_any(w_raw)
    w = np.exp(-np.exp(u))
    kk64 = _widen_any(kk)
    nrm = np.sqrt(np.sum(kk64 * kk64, axis=-1, keepdims=True))
    kk_hat = kk64 / np.maximum(nrm, NORMALIZE_EPS)
    return w, -kk_hat, kk_hat * _widen_any(a_lr)


def group_norm(y, ln_w=None, ln_b=None, eps: float = GROUP_NORM_EPS):
    """ln_x on y [B, T, H, N]: per (b, t, h), subtract the mean over N, divide by the square root of
    the (population) variance plus eps, then scale by ln_w and shift by ln_b (per channel, [H*N];
    None means 1 and 0)."""
    y = np.asarray(y, dtype=np.float64)
    H, N = y.shape[-2:]
    mu = np.mean(y, axis=-1, keepdims=True)
    d = y - mu
    var = np.mean(d * d, axis=-1, keepdims=True)
    out = d / np.sqrt(var + eps)
    if ln_w is not None:
        out = out * _widen_any(ln_w).reshape(H, N)
    if ln_b is not None:
        out = out + _widen_any(ln_b).reshape(H, N)
    return out


def tmix(r, w_raw, k, v, kk, a_lr, ln_w=None, ln_b=None, state_in=None, nthreads: int | None = None):
    """The fused operator in float64: prologue, recurrence, ln_x.

    r, k, v, kk, a_lr: [B, T, H, N] float32 or bfloat16 bits; w_raw: [B, T, H, N] float32;
    ln_w, ln_b: [H * N] float32 or None. Returns (out [B,T,H,N] float64, state_out float64).
    """
    w, a, b = tmix_prologue(w_raw, kk, a_lr)
    y, s = wkv7(_widen_any(r), w, _widen_any(k), _widen_any(v), a, b, state_in=state_in, nthreads=nthreads)
    return group_norm(y, ln_w, ln_b), s


def wkv7_backward(r, w, k, v, a, b, dy, state_in=None, dstate_out=None, nthreads: int | None = None):
    """Reverse-mode derivatives of the recurrence in float64 (training, G0 notes section 7.2).

    Inputs as for wkv7 (one dtype for r..b; state_in float32/float64 or None); dy [B,T,H,N] and
    dstate_out [B,H,N,N] (or None: zero) are the gradients of a loss with respect to y and the final
    state. Returns dict with dr, dw, dk, dv, da, db ([B,T,H,N] float64) and dstate_in ([B,H,N,N]).
    """
    lib = _load()
    ins = [np.ascontiguousarray(x) for x in (r, w, k, v, a, b)]
    shape = ins[0].shape
    if len(shape) != 4 or any(x.shape != shape for x in ins):
        raise ValueError("r,w,k,v,a,b must share one [B,T,H,N] shape")
    dt = _in_dtype(ins[0])
    if any(_in_dtype(x) != dt for x in ins):
        raise TypeError("r,w,k,v,a,b must share one dtype")
    B, T, H, N = shape
    s_in, st_dt = None, IN_F64
    if state_in is not None:
        s_in = np.ascontiguousarray(state_in)
        st_dt = {np.dtype(np.float32): IN_F32, np.dtype(np.float64): IN_F64}[s_in.dtype]
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    dso = None if dstate_out is None else np.ascontiguousarray(dstate_out, dtype=np.float64)
    out = {n: np.empty(shape, dtype=np.float64) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    out["dstate_in"] = np.empty((B, H, N, N), dtype=np.float64)
    p = lambda x: None if x is None else x.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    rc = lib.wkv7_oracle_bwd_f64(*(p(x) for x in ins), p(s_in), p(dy), p(dso),
                                 *(p(out[n]) for n in ("dr", "dw", "dk", "dv", "da", "db", "dstate_in")),
                                 B, T, H, N, dt, st_dt, int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle backward failed with status %d" % rc)
    return out


# ---------------------------------------------------------------------------------------------
# A stack of L time-mix layers over a residual stream (RWKV-7 G0 7.2B notes, section 3.2: the hybrid
# mode takes the prompt through the model in parallel, then steps token by token with per-layer
# state; section 7.1 for the parameterisation: the decay is soft-clamped by a softplus to at most
# -0.5 before exp(-exp(.)), the in-context learning rate is a sigmoid, the removal key is the key
# scaled per channel, normalised inside the operator).


def _as_dtype(x64, dtype: str):
    """float64 values -> the array the GPU hands on: float32 (round to nearest even), or for "bf16"
    float32 then bfloat16 (each round to nearest even) as raw uint16 bits."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    return round16(x32.astype(np.float64), "bf16")


def _softplus(z):
    return np.logaddexp(0.0, z)


def stack_forward(w_in, w_out, vecs, x, states, dtype: str = "f32", nthreads: int | None = None):
    """L layers in float64. x [B, T, D] float32, states [L, B, H, N, N] (float32 or float64),
    w_in [L, D, 5D] / w_out [L, D, D] float32 or bfloat16 bits, vecs [L, 5, D] float32 (w0, a0, k_k,
    ln_w, ln_b). Per layer: P = q(x) W_in (blocks r|k|v|w|a); w_raw = -softplus(-(w0 + P_w)) - 0.5;
    kk = P_k * k_k; a_lr = sigmoid(a0 + P_a); the operator on r, k, v, kk, a_lr with ln_x; x += q(o) W_out.

    `dtype` is the model's precision and fixes the rounding points, read from the RWKV-7 G0 7.2B
    notes (lshu.cn/news/198401) sections 3.2-3.4 (a model runs in one dtype, half on that page:
    weights and the activations that enter a product are in it; w0 and the [H, N, N] state stay
    float32) and the README's fp32 note (oa0.com/c/1004164: the state and w stay float32, kv is
    converted to float32), with the residual stream float32 as the stack's ABI takes it:
      "f32"  every product's output and every operator input rounded to float32 (the float32 model);
      "bf16" x and o rounded to bfloat16 where they enter a product, P rounded to float32 (a float32
             accumulation), w_raw float32 (the decay input stays float32), r, k, v, kk, a_lr rounded
             to bfloat16 (the operator takes the model's dtype);
      "f64"  no rounding anywhere (the same weights, exact arithmetic to float64): the reference
             against which a model's own rounding is measured.
    Returns (x float64, states float64).
    """
    x = np.asarray(x, dtype=np.float64).copy()
    st = np.asarray(states, dtype=np.float64).copy()
    L, B, H, N = st.shape[:4]
    T, D = x.shape[1], x.shape[2]
    M = B * T
    Wi, Wo, V = _widen_any(w_in), _widen_any(w_out), _widen_any(vecs)
    q = (lambda a: _widen_any(_as_dtype(a, "bf16"))) if dtype == "bf16" else (lambda a: a)
    f32 = (lambda a: a) if dtype == "f64" else (lambda a: a.astype(np.float32).astype(np.float64))
    for l in range(L):
        P = f32(q(x).reshape(M, D) @ Wi[l])
        pr, pk, pv, pw, pa = (P[:, i * D:(i + 1) * D] for i in range(5))
        w_raw = f32(-_softplus(-(V[l, 0] + pw)) - 0.5)
        kk = pk * V[l, 2]
        a_lr = 1.0 / (1.0 + np.exp(-(V[l, 1] + pa)))
        shp = (B, T, H, N)
        ops = [(t if dtype == "f64" else _as_dtype(t, dtype)).reshape(shp) for t in (pr, pk, pv, kk, a_lr)]
        out, s = tmix(ops[0], w_raw.reshape(shp), ops[1], ops[2], ops[3], ops[4], vecs[l, 3], vecs[l, 4],
                      state_in=st[l], nthreads=nthreads)
        st[l] = s
        x = x + (q(out.reshape(M, D)) @ Wo[l]).reshape(B, T, D)
    return x, st
