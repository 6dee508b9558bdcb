"""Pins of the oracle's backward (reverse-mode derivatives of the recurrence), CPU only.

The backward is pinned to torch's float64 autograd of a plain token loop of the forward
formula (RWKV-7 G0 7.2B notes, section 7.1: S_t = S_{t-1} (diag(w) + a b^T) + v k^T, y = S_t r)
and to central finite differences of the oracle's forward; planted mistakes in a copy of
its C source must fail a pin.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "wkv7_oracle.c")
GRADS = ("dr", "dw", "dk", "dv", "da", "db", "dstate_in")


def random_case(seed, B=1, T=5, H=2, N=64):
    rng = np.random.default_rng(seed)
    x = {n: rng.standard_normal((B, T, H, N)) for n in "rvk"}
    x["k"] = x["k"] / 8
    x["w"] = np.exp(-np.exp(rng.uniform(-5, -0.5, (B, T, H, N))))
    kk = rng.standard_normal((B, T, H, N))
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    alr = rng.uniform(0, 1, (B, T, H, N))
    x["a"], x["b"] = -kk, kk * alr
    x["state_in"] = rng.standard_normal((B, H, N, N)) * 0.1
    dy = rng.standard_normal((B, T, H, N))
    ds = rng.standard_normal((B, H, N, N)) * 0.1
    return x, dy, ds


def torch_grads(x, dy, ds):
    t = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True) for n in ("r", "w", "k", "v", "a", "b",
                                                                              "state_in")}
    S = t["state_in"]
    T = dy.shape[1]
    ys = []
    for i in range(T):
        w, a, b = t["w"][:, i], t["a"][:, i], t["b"][:, i]
        M = torch.diag_embed(w) + a.unsqueeze(-1) * b.unsqueeze(-2)  # [B,H,N,N]
        S = S @ M + t["v"][:, i].unsqueeze(-1) * t["k"][:, i].unsqueeze(-2)
        ys.append((S @ t["r"][:, i].unsqueeze(-1)).squeeze(-1))
    y = torch.stack(ys, 1)
    loss = (y * torch.from_numpy(dy)).sum() + (S * torch.from_numpy(ds)).sum()
    loss.backward()
    return {"d" + n if n != "state_in" else "dstate_in": t[n].grad.numpy() for n in t}


def rel(x, ref):
    m = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / m) if m > 0 else float(np.max(np.abs(x)))


def pin_autograd(orc, seed=1, **shape):
    x, dy, ds = random_case(seed, **shape)
    g = orc.wkv7_backward(*(x[n] for n in "rwkvab"), dy, x["state_in"], ds)
    ref = torch_grads(x, dy, ds)
    return max(rel(g[n], ref[n]) for n in GRADS)


def pin_finite_differences(orc, seed=2, per_input=6, h=1e-5):
    x, dy, ds = random_case(seed, T=4)
    g = orc.wkv7_backward(*(x[n] for n in "rwkvab"), dy, x["state_in"], ds)
    rng = np.random.default_rng(seed)

    def loss(xx):
        y, s = orc.wkv7(*(xx[n] for n in "rwkvab"), state_in=xx["state_in"])
        return float(np.sum(y * dy) + np.sum(s * ds))

    worst = 0.0
    for n in ("r", "w", "k", "v", "a", "b", "state_in"):
        gname = "dstate_in" if n == "state_in" else "d" + n
        scale = np.max(np.abs(g[gname])) + 1e-30
        for _ in range(per_input):
            idx = tuple(int(rng.integers(s)) for s in x[n].shape)
            xp = {m: a.copy() for m, a in x.items()}
            xm = {m: a.copy() for m, a in x.items()}
            xp[n][idx] += h
            xm[n][idx] -= h
            fd = (loss(xp) - loss(xm)) / (2 * h)
            worst = max(worst, abs(fd - g[gname][idx]) / scale)
    return worst


def test_backward_matches_torch_autograd():
    assert pin_autograd(oracle) < 1e-12
    assert pin_autograd(oracle, seed=3, B=2, T=3, H=1) < 1e-12


def test_backward_matches_finite_differences():
    assert pin_finite_differences(oracle) < 1e-7


def test_backward_zero_tokens_passes_state_gradient():
    x, dy, ds = random_case(5, T=1)
    g = oracle.wkv7_backward(*(x[n][:, :0] for n in "rwkvab"), dy[:, :0], x["state_in"], ds)
    assert np.array_equal(g["dstate_in"], ds)


def test_backward_linear_attention_closed_form():
    """w = 1, a = 0 and no final-state gradient: y_s = sum_{t<=s} (r_s . k_t) v_t + S0 r_s, so
    dv_t = sum_{s>=t} (r_s . k_t) dy_s and dr_s = sum_{t<=s} (v_t . dy_s) k_t + S0^T dy_s."""
    x, dy, _ = random_case(6, T=6, H=1)
    x["w"] = np.ones_like(x["w"])
    x["a"] = np.zeros_like(x["a"])
    g = oracle.wkv7_backward(*(x[n] for n in "rwkvab"), dy, x["state_in"], None)
    r, k, v, d, S0 = x["r"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], dy[0, :, 0], x["state_in"][0, 0]
    causal = np.tril(r @ k.T)  # [s, t]
    dv = causal.T @ d
    dr = np.tril(d @ v.T) @ k + d @ S0
    assert rel(g["dv"][0, :, 0], dv) < 1e-13 and rel(g["dr"][0, :, 0], dr) < 1e-13


MUTANTS = [
    ("dy_transposed", "G[i * N + j] += dyv[i] * r[j];", "G[i * N + j] += dyv[j] * r[i];"),
    ("drop_lowrank_back", "G[i * N + j] * w[j] + gb[i] * a[j];", "G[i * N + j] * w[j];"),
    ("lowrank_back_swapped", "G[i * N + j] * w[j] + gb[i] * a[j];", "G[i * N + j] * w[j] + gb[i] * b[j];"),
    ("dr_old_state", "s_dr += Sc[i * N + j] * dyv[i];", "s_dr += Sp[i * N + j] * dyv[i];"),
    ("dw_new_state", "s_dw += Sp[i * N + j] * G[i * N + j];", "s_dw += Sc[i * N + j] * G[i * N + j];"),
    ("da_uses_sa", "s_da += Sp[i * N + j] * gb[i];", "s_da += Sp[i * N + j] * sa[i];"),
    ("db_uses_gb", "s_db += G[i * N + j] * sa[i];", "s_db += G[i * N + j] * gb[i];"),
    ("dk_uses_k", "s_dk += G[i * N + j] * v[i];", "s_dk += G[i * N + j] * k[i];"),
    ("dv_uses_v", "s_dv += G[i * N + j] * k[j];", "s_dv += G[i * N + j] * v[j];"),
]


class _Mutant:
    def __init__(self, so):
        lib = ctypes.CDLL(so)
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
        self._lib = lib

    def _bound(self, fn, *a, **kw):
        saved = oracle._lib
        oracle._lib = self._lib
        try:
            return fn(*a, **kw)
        finally:
            oracle._lib = saved

    def wkv7(self, *a, **kw):
        return self._bound(oracle.wkv7, *a, **kw)

    def wkv7_backward(self, *a, **kw):
        return self._bound(oracle.wkv7_backward, *a, **kw)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, old
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC", "-pthread", str(c), "-o",
                    str(so), "-lm"], check=True)
    m = _Mutant(str(so))
    with np.errstate(all="ignore"):
        worst = max(pin_autograd(m), pin_finite_differences(m))
    assert not (worst < 1e-6), (name, worst)
