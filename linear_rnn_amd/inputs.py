"""Seeded synthetic inputs for the WKV-7 recurrence (shared by the GPU tests and the CPU oracle).

This module holds only random-number generation and dtype casting: none of the
recurrence's arithmetic. It imports nothing else from this package, so the
oracle side and the GPU side can both use it without sharing any computation.

Distributions (per (batch, token, head), head size N = 64), chosen to mirror how
an RWKV-7 time-mix layer feeds its WKV operator (RWKV-7 G0 7.2B notes,
lshu.cn/news/198401, section 7.1: decay = exp(-exp(.)), the in-context learning
rate is a sigmoid, the removal key is an L2-normalised key, and the kernel slots
are a = -kk, b = kk * a_lr):

  r, v        ~ N(0, 1)
  k (slot k)  ~ N(0, 1) / 8
  kk          = g / |g|, g ~ N(0, 1)^64         (unit removal key)
  a_lr        = sigmoid(N(0, 1))                (or U(0,1) with 1% forced to 0 and 1% to 1)
  w           = exp(-exp(u)), u ~ U(lo, hi)     (decay multiplier in (0, 1])
  a (slot a)  = -kk,   b (slot b) = kk * a_lr
  state_in    ~ N(0, 0.1^2) float32, or None (zero state)

Everything is drawn in float64 and cast once: to float32 (round to nearest even)
or to bfloat16 (float64 -> float32 -> bfloat16, each round to nearest even).
bfloat16 tensors are returned as uint16 arrays of raw bits, so both sides read
identical bits.

Seeding: numpy PCG64. Each tensor gets one child of SeedSequence(seed); each
tensor is filled in fixed slabs of rows, each slab from its own grandchild, so
the result does not depend on how many threads fill it.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

HEAD_SIZE = 64
_SLAB_ROWS = 1 << 12  # rows of 64 elements per independently seeded slab


@dataclass(frozen=True)
class WkvConfig:
    """One workload shape: batch B, tokens T, heads H, head size N, input dtype."""
    name: str
    B: int
    T: int
    H: int
    dtype: str  # "f32" or "bf16"
    state_in: bool
    u_lo: float = -5.0
    u_hi: float = -0.5
    a_uniform: bool = False  # a_lr ~ U(0,1) with forced exact 0s and 1s
    steps: int = 1  # decode configs: number of consecutive single-token steps
    seed: int = 7000
    N: int = HEAD_SIZE

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H * self.steps


# The five workloads. Head counts follow the RWKV-7 model shapes named on the
# pages (0.1B L12-D768 -> H=12; L24-D1024 -> H=16; 1.5B D2048 -> H=32;
# 7B-class D4096 -> H=64), each with head size 64.
CONFIGS = {
    cfg.name: cfg
    for cfg in (
        WkvConfig("tiny-prefill-f32", B=1, T=64, H=2, dtype="f32", state_in=False, seed=7000),
        WkvConfig("L12-D768-prefill", B=8, T=4096, H=12, dtype="bf16", state_in=True, seed=7001),
        WkvConfig("L24-D1024-prefill-resume", B=16, T=4096, H=16, dtype="bf16", state_in=True, seed=7002),
        WkvConfig("D2048-decode", B=512, T=1, H=32, dtype="bf16", state_in=True, steps=256, seed=7003),
        WkvConfig("D4096-long-prefill", B=4, T=16384, H=64, dtype="bf16", state_in=True,
                  u_lo=-8.0, u_hi=-0.1, a_uniform=True, seed=7004),
    )
}

TENSORS = ("r", "w", "k", "v", "a", "b")


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    return x.astype(np.float32)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the raw bits as uint16."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _cast(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = f64_to_f32(x64)
    return x32 if dtype == "f32" else f32_to_bf16_bits(x32)


def _fill_rows(seq: np.random.SeedSequence, rows: int, draw) -> list:
    """Split `rows` rows into fixed slabs, each drawn by `draw(gen, n)` from its own seed."""
    n_slabs = max(1, -(-rows // _SLAB_ROWS))
    kids = seq.spawn(n_slabs)
    jobs = []
    for s in range(n_slabs):
        lo = s * _SLAB_ROWS
        n = min(_SLAB_ROWS, rows - lo)
        jobs.append((kids[s], lo, n))
    return jobs


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(cfg: WkvConfig, step: int | None = None, B: int | None = None, T: int | None = None,
                H: int | None = None, seed: int | None = None, with_state: bool | None = None) -> dict:
    """Draw r, w, k, v, a, b ([B, T, H, N]) and state_in ([B, H, N, N] float32 or None).

    `step` selects an independent per-step stream (decode workloads). B, T, H and
    seed override the config's values (smaller parity cases with the same
    distributions).
    """
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    H = cfg.H if H is None else H
    N = cfg.N
    seed = cfg.seed if seed is None else seed
    with_state = cfg.state_in if with_state is None else with_state
    root = np.random.SeedSequence([seed] if step is None else [seed, step])
    ss_r, ss_w, ss_k, ss_v, ss_kk, ss_alr, ss_state = root.spawn(7)
    rows = B * T * H
    out_dt = np.float32 if cfg.dtype == "f32" else np.uint16
    res = {name: np.empty((rows, N), dtype=out_dt) for name in TENSORS}

    def normal_rows(scale):
        def draw(g, n):
            return g.standard_normal((n, N)) * scale
        return draw

    def decay_rows(g, n):
        u = g.uniform(cfg.u_lo, cfg.u_hi, size=(n, N))
        return np.exp(-np.exp(u))

    def kk_rows(g, n):
        x = g.standard_normal((n, N))
        return x / np.sqrt(np.sum(x * x, axis=1, keepdims=True))

    def alr_rows(g, n):
        if cfg.a_uniform:
            x = g.uniform(0.0, 1.0, size=(n, N))
            pick = g.uniform(0.0, 1.0, size=(n, N))
            x[pick < 0.01] = 0.0
            x[(pick >= 0.01) & (pick < 0.02)] = 1.0
            return x
        return 1.0 / (1.0 + np.exp(-g.standard_normal((n, N))))

    tasks = []
    for name, ss, draw in (("r", ss_r, normal_rows(1.0)), ("v", ss_v, normal_rows(1.0)),
                           ("k", ss_k, normal_rows(1.0 / 8.0)), ("w", ss_w, decay_rows)):
        for kid, lo, n in _fill_rows(ss, rows, draw):
            tasks.append((name, kid, lo, n, draw))

    def run_simple(task):
        name, kid, lo, n, draw = task
        res[name][lo:lo + n] = _cast(draw(np.random.Generator(np.random.PCG64(kid)), n), cfg.dtype)

    kk_jobs = _fill_rows(ss_kk, rows, None)
    alr_jobs = _fill_rows(ss_alr, rows, None)

    def run_ab(idx):
        kid_kk, lo, n = kk_jobs[idx]
        kid_alr = alr_jobs[idx][0]
        kk = kk_rows(np.random.Generator(np.random.PCG64(kid_kk)), n)
        alr = alr_rows(np.random.Generator(np.random.PCG64(kid_alr)), n)
        res["a"][lo:lo + n] = _cast(-kk, cfg.dtype)
        res["b"][lo:lo + n] = _cast(kk * alr, cfg.dtype)

    nthr = _threads()
    if rows * N >= (1 << 18) and nthr > 1:
        with _cf.ThreadPoolExecutor(nthr) as ex:
            list(ex.map(run_simple, tasks))
            list(ex.map(run_ab, range(len(kk_jobs))))
    else:
        for t in tasks:
            run_simple(t)
        for i in range(len(kk_jobs)):
            run_ab(i)

    out = {name: res[name].reshape(B, T, H, N) for name in TENSORS}
    if with_state:
        g = np.random.Generator(np.random.PCG64(ss_state))
        out["state_in"] = (g.standard_normal((B, H, N, N)) * 0.1).astype(np.float32)
    else:
        out["state_in"] = None
    return out


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 view of an input array (float32, or uint16 bfloat16 bits)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def make_tmix_inputs(cfg: WkvConfig, step: int | None = None, B: int | None = None, T: int | None = None,
                     H: int | None = None, seed: int | None = None, with_state: bool | None = None) -> dict:
    """Raw inputs of the time-mix operator with its prologue and epilogue, [B, T, H, N] each.

    r, v ~ N(0, 1) and k ~ N(0, 1) / 8 in the config's dtype; w_raw = u ~ U(u_lo, u_hi) in float32
    (the decay is exp(-exp(w_raw))); kk ~ N(0, 1)^64, not normalised, in the config's dtype; a_lr as
    for make_inputs; ln_w ~ U(0.2, 1) and ln_b ~ N(0, 0.05^2) per channel ([H * N] float32);
    state_in ~ N(0, 0.1^2) float32 or None. Seeded from SeedSequence([seed, 1]) (per step:
    [seed, 1, step]), a stream of its own.
    """
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    H = cfg.H if H is None else H
    N = cfg.N
    seed = cfg.seed if seed is None else seed
    with_state = cfg.state_in if with_state is None else with_state
    root = np.random.SeedSequence([seed, 1] if step is None else [seed, 1, step])
    kids = root.spawn(10)
    shape = (B, T, H, N)
    gen = [np.random.Generator(np.random.PCG64(k)) for k in kids]
    out = {
        "r": _cast(gen[0].standard_normal(shape), cfg.dtype),
        "k": _cast(gen[1].standard_normal(shape) / 8.0, cfg.dtype),
        "v": _cast(gen[2].standard_normal(shape), cfg.dtype),
        "w_raw": f64_to_f32(gen[3].uniform(cfg.u_lo, cfg.u_hi, size=shape)),
        "kk": _cast(gen[4].standard_normal(shape), cfg.dtype),
    }
    if cfg.a_uniform:
        x = gen[5].uniform(0.0, 1.0, size=shape)
        pick = gen[6].uniform(0.0, 1.0, size=shape)
        x[pick < 0.01] = 0.0
        x[(pick >= 0.01) & (pick < 0.02)] = 1.0
    else:
        x = 1.0 / (1.0 + np.exp(-gen[5].standard_normal(shape)))
    out["a_lr"] = _cast(x, cfg.dtype)
    out["ln_w"] = f64_to_f32(gen[7].uniform(0.2, 1.0, size=H * N))
    out["ln_b"] = f64_to_f32(gen[8].standard_normal(H * N) * 0.05)
    out["state_in"] = (gen[9].standard_normal((B, H, N, N)) * 0.1).astype(np.float32) if with_state else None
    return out


def make_cotangents(B: int, T: int, H: int, seed: int, with_dstate: bool = True, N: int = HEAD_SIZE) -> dict:
    """Seeded gradients flowing into the backward: dy ~ N(0, 1) [B, T, H, N] float32 and
    dstate_out ~ N(0, 0.1^2) [B, H, N, N] float32 (or None). Seeded from SeedSequence([seed, 2])."""
    g_dy, g_ds = (np.random.Generator(np.random.PCG64(k)) for k in np.random.SeedSequence([seed, 2]).spawn(2))
    dy = g_dy.standard_normal((B, T, H, N)).astype(np.float32)
    ds = (g_ds.standard_normal((B, H, N, N)) * 0.1).astype(np.float32) if with_dstate else None
    return {"dy": dy, "dstate_out": ds}


def make_stack_inputs(L: int, B: int, T: int, H: int, dtype: str, seed: int, with_state: bool = True,
                      N: int = HEAD_SIZE) -> dict:
    """Synthetic weights and activations for a stack of L time-mix layers (D = H * N).

    x ~ N(0, 1) [B, T, D] float32 (the residual stream); w_in ~ N(0, 1/D) [L, D, 5D] and
    w_out ~ N(0, 0.25/D) [L, D, D] in `dtype` ("f32", or "bf16" as raw uint16 bits); vecs [L, 5, D]
    float32: w0 ~ U(-5, -1) (decay bias: with unit projections the decays fall mostly in
    0.9-0.999), a0 ~ N(0, 1) (in-context learning rate bias), k_k ~ U(0.5, 1.5) (removal-key scale),
    ln_w ~ U(0.2, 1), ln_b ~ N(0, 0.05^2); states ~ N(0, 0.1^2) [L, B, H, N, N] float32, or zeros.
    Seeded from SeedSequence([seed, 3]).
    """
    D = H * N
    g = [np.random.Generator(np.random.PCG64(k)) for k in np.random.SeedSequence([seed, 3]).spawn(9)]
    vecs = np.empty((L, 5, D), dtype=np.float64)
    vecs[:, 0] = g[3].uniform(-5.0, -1.0, size=(L, D))
    vecs[:, 1] = g[4].standard_normal((L, D))
    vecs[:, 2] = g[5].uniform(0.5, 1.5, size=(L, D))
    vecs[:, 3] = g[6].uniform(0.2, 1.0, size=(L, D))
    vecs[:, 4] = g[7].standard_normal((L, D)) * 0.05
    states = (g[8].standard_normal((L, B, H, N, N)) * 0.1).astype(np.float32) if with_state \
        else np.zeros((L, B, H, N, N), dtype=np.float32)
    return {
        "x": f64_to_f32(g[0].standard_normal((B, T, D))),
        "w_in": _cast(g[1].standard_normal((L, D, 5 * D)) / np.sqrt(D), dtype),
        "w_out": _cast(g[2].standard_normal((L, D, D)) * (0.5 / np.sqrt(D)), dtype),
        "vecs": f64_to_f32(vecs),
        "states": states,
    }
