"""Pins of the oracle's multi-layer stack (CPU only).

The stack's glue (projections, soft clamp, sigmoid, per-channel key scale, residual) is pinned to a
composition written with torch's own softplus, sigmoid, matmul and dtype casts around the pinned
operator; the GPT/RNN-mode equivalence (one call over T tokens equals T calls of one token with the
per-layer states carried; RWKV-7 G0 7.2B notes, section 3.2) pins the state hand-off between calls.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_amd.inputs import bf16_bits_to_f32, make_stack_inputs


def run(z, dtype, x=None, states=None):
    return oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"] if x is None else x,
                                z["states"] if states is None else states, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prompt_then_steps_equals_one_pass(dtype):
    z = make_stack_inputs(3, 2, 11, 2, dtype, seed=5)
    x_all, s_all = run(z, dtype)
    x0, s = run(z, dtype, x=z["x"][:, :6])
    xs = [x0]
    for t in range(6, 11):
        xt, s = run(z, dtype, x=z["x"][:, t:t + 1], states=s)
        xs.append(xt)
    assert np.max(np.abs(np.concatenate(xs, axis=1) - x_all)) <= 1e-12 * np.max(np.abs(x_all))
    assert np.max(np.abs(s - s_all)) <= 1e-12 * np.max(np.abs(s_all))


def _torch_layer(x, z, l, dtype, state):
    """One layer written with torch's own functions (float64), around the pinned operator."""
    def q(t):  # the GPU's rounding of activations before a projection
        return t.to(torch.float32).to(torch.bfloat16).to(torch.float64) if dtype == "bf16" else t

    def op_in(t):  # operator inputs in the weights' dtype, as numpy arrays the operator takes
        t32 = t.to(torch.float32)
        if dtype == "f32":
            return t32.numpy()
        return t32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def widen(a):
        return torch.from_numpy(bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16
                                else a.astype(np.float64))

    wi, wo = widen(z["w_in"][l]), widen(z["w_out"][l])
    v = torch.from_numpy(z["vecs"][l].astype(np.float64))
    B, T, D = x.shape
    H = D // 64
    P = (q(x).reshape(B * T, D) @ wi).to(torch.float32).to(torch.float64)
    pr, pk, pv, pw, pa = P.split(D, dim=1)
    w_raw = (-torch.nn.functional.softplus(-(v[0] + pw)) - 0.5).to(torch.float32).numpy()
    kk = pk * v[2]
    a_lr = torch.sigmoid(v[1] + pa)
    shp = (B, T, H, 64)
    out, s = oracle.tmix(op_in(pr).reshape(shp), w_raw.reshape(shp), op_in(pk).reshape(shp),
                         op_in(pv).reshape(shp), op_in(kk).reshape(shp), op_in(a_lr).reshape(shp),
                         z["vecs"][l, 3], z["vecs"][l, 4], state_in=state)
    x = x + (q(torch.from_numpy(out).reshape(B * T, D)) @ wo).reshape(B, T, D)
    return x, s


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layers_against_torch_composition(dtype):
    z = make_stack_inputs(2, 2, 7, 2, dtype, seed=9)
    xo, so = run(z, dtype)
    x = torch.from_numpy(z["x"].astype(np.float64))
    for l in range(2):
        x, s = _torch_layer(x, z, l, dtype, z["states"][l])
        assert np.max(np.abs(s - so[l])) <= 1e-12 * np.max(np.abs(so[l]))
    assert np.max(np.abs(x.numpy() - xo)) <= 1e-12 * np.max(np.abs(xo))


def test_soft_clamp_and_rate_ranges():
    """w_raw <= -0.5 (so every decay is below exp(-exp(-0.5))) and a_lr in (0, 1), by construction."""
    z = make_stack_inputs(1, 1, 5, 1, "f32", seed=2)
    z["vecs"][0, 0] = np.linspace(-40, 40, 64)
    out_big, _ = run(z, "f32")
    assert np.all(np.isfinite(out_big))
    zz = np.linspace(-40, 40, 1001)
    w_raw = -oracle._softplus(-zz) - 0.5
    assert np.all(w_raw <= -0.5) and abs(w_raw[-1] + 0.5) < 1e-15 and abs(w_raw[0] - (zz[0] - 0.5)) < 1e-12


def test_zero_output_projection_leaves_x():
    z = make_stack_inputs(2, 1, 6, 2, "f32", seed=4)
    z["w_out"][:] = 0
    x, s = run(z, "f32")
    assert np.array_equal(x, z["x"].astype(np.float64))
    # with equal weights both layers see the same input, so from equal states they reach equal states
    z["w_in"][1], z["vecs"][1], z["states"][1] = z["w_in"][0], z["vecs"][0], z["states"][0]
    _, s = run(z, "f32")
    assert np.array_equal(s[0], s[1])


def test_batch_permutation_equivariance():
    z = make_stack_inputs(2, 3, 5, 2, "bf16", seed=6)
    x, s = run(z, "bf16")
    perm = [2, 0, 1]
    xp, sp = run(z, "bf16", x=z["x"][perm], states=z["states"][:, perm])
    assert np.max(np.abs(xp - x[perm])) <= 1e-12 * np.max(np.abs(x))
    assert np.max(np.abs(sp - s[:, perm])) <= 1e-12 * np.max(np.abs(s))
