"""Pins of the oracle's time-mix prologue and epilogue (CPU only).

The operator with its prologue and epilogue follows RWKV-7 G0 7.2B notes
(lshu.cn/news/198401), section 7.1: decay exp(-exp(w_raw)), an L2-normalised removal key
kk_hat (F.normalize), kernel slots a = -kk_hat and b = kk_hat * a_lr, and ln_x, a GroupNorm
with one group per head and eps 64e-5. Each piece is pinned to closed forms or to an
independent library routine (torch's normalize and group_norm); the recurrence in the middle
is pinned by test_oracle_pins.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from linear_rnn_amd.inputs import CONFIGS, make_tmix_inputs


def test_decay_closed_forms():
    u = np.array([math.log(math.log(2.0)), math.log(math.log(4.0)), -np.inf, np.inf, 0.0])
    w, _, _ = oracle.tmix_prologue(u, np.ones(5), np.ones(5))
    assert abs(w[0] - 0.5) < 1e-15 and abs(w[1] - 0.25) < 1e-15
    assert w[2] == 1.0 and w[3] == 0.0
    assert abs(w[4] - math.exp(-1.0)) < 1e-15  # exp(-exp(0)) = 1/e


def test_normalised_key_and_slots():
    rng = np.random.default_rng(3)
    kk = rng.standard_normal((5, 7, 64)) * 3.0
    alr = rng.uniform(0, 1, (5, 7, 64))
    _, a, b = oracle.tmix_prologue(np.zeros_like(kk), kk, alr)
    ref = torch.nn.functional.normalize(torch.from_numpy(kk), dim=-1).numpy()
    assert np.max(np.abs(-a - ref)) < 1e-15
    assert np.max(np.abs(b - ref * alr)) < 1e-15
    assert np.max(np.abs(np.sum(a * a, axis=-1) - 1.0)) < 1e-14
    # a zero key stays zero (division by max(|x|, 1e-12)), with no NaN
    _, a0, b0 = oracle.tmix_prologue(np.zeros(64), np.zeros(64), np.ones(64))
    assert np.all(a0 == 0.0) and np.all(b0 == 0.0)


@pytest.mark.parametrize("affine", [False, True])
def test_group_norm_vs_torch(affine):
    rng = np.random.default_rng(5)
    B, T, H, N = 2, 9, 3, 64
    y = rng.standard_normal((B, T, H, N)) * rng.uniform(0.01, 10, (B, T, H, 1)) + rng.standard_normal((B, T, H, 1))
    lw = rng.uniform(0.2, 1.0, H * N) if affine else None
    lb = rng.standard_normal(H * N) * 0.1 if affine else None
    got = oracle.group_norm(y, lw, lb)
    ref = torch.nn.functional.group_norm(torch.from_numpy(y.reshape(B * T, H * N)), H,
                                         None if lw is None else torch.from_numpy(lw),
                                         None if lb is None else torch.from_numpy(lb), eps=64e-5)
    assert np.max(np.abs(got - ref.numpy().reshape(B, T, H, N))) < 1e-12


def test_delta_rule_through_the_operator():
    """w_raw = -inf (w = 1), a_lr = 1, k = r = the normalised removal key: the state maps
    kk_hat to v_t, so the recurrence output is v_t and the operator returns ln_x(v)."""
    rng = np.random.default_rng(11)
    B, T, H, N = 1, 24, 2, 64
    g = rng.standard_normal((B, T, H, N))
    kk = g / np.linalg.norm(g, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, N))
    lw = rng.uniform(0.2, 1.0, H * N)
    lb = rng.standard_normal(H * N) * 0.05
    s0 = rng.standard_normal((B, H, N, N)) * 0.3
    out, _ = oracle.tmix(kk, np.full((B, T, H, N), -np.inf), kk, v, kk * 7.0, np.ones((B, T, H, N)), lw, lb, s0)
    ref = torch.nn.functional.group_norm(torch.from_numpy(v.reshape(B * T, H * N)), H, torch.from_numpy(lw),
                                         torch.from_numpy(lb), eps=64e-5).numpy().reshape(B, T, H, N)
    assert np.max(np.abs(out - ref)) < 1e-9


def test_operator_against_library_composition():
    """Prologue and epilogue from torch's own exp, normalize and group_norm around the pinned
    recurrence give the same result as the operator."""
    x = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=1, T=40, H=3, seed=21)
    out, s = oracle.tmix(x["r"], x["w_raw"], x["k"], x["v"], x["kk"], x["a_lr"], x["ln_w"], x["ln_b"],
                         x["state_in"])
    wid = oracle._widen_any
    u = torch.from_numpy(wid(x["w_raw"]))
    w = torch.exp(-torch.exp(u)).numpy()
    kh = torch.nn.functional.normalize(torch.from_numpy(wid(x["kk"])), dim=-1).numpy()
    y, s_ref = oracle.wkv7(wid(x["r"]), w, wid(x["k"]), wid(x["v"]), -kh, kh * wid(x["a_lr"]), x["state_in"])
    B, T, H, N = y.shape
    ref = torch.nn.functional.group_norm(torch.from_numpy(y.reshape(B * T, H * N)), H,
                                         torch.from_numpy(wid(x["ln_w"])), torch.from_numpy(wid(x["ln_b"])),
                                         eps=64e-5).numpy().reshape(B, T, H, N)
    assert np.max(np.abs(out - ref)) < 1e-10
    assert np.array_equal(s, s_ref)


def test_tmix_inputs_are_seeded_and_shaped():
    a = make_tmix_inputs(CONFIGS["tiny-prefill-f32"], seed=3)
    b = make_tmix_inputs(CONFIGS["tiny-prefill-f32"], seed=3)
    for n in ("r", "w_raw", "k", "v", "kk", "a_lr", "ln_w", "ln_b"):
        assert np.array_equal(a[n], b[n])
    assert a["w_raw"].dtype == np.float32 and a["ln_w"].shape == (2 * 64,)
    x = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=1, T=3, H=2)
    assert x["r"].dtype == np.uint16 and x["w_raw"].dtype == np.float32 and x["state_in"].shape == (1, 2, 64, 64)
