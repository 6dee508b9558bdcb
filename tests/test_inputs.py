"""Seeded generators and fixed facts about shapes (CPU only)."""
import json
import os

import numpy as np
import pytest

from linear_rnn_amd.inputs import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_deterministic_and_seed_sensitive():
    a = make_inputs(CONFIGS["tiny-prefill-f32"])
    b = make_inputs(CONFIGS["tiny-prefill-f32"])
    c = make_inputs(CONFIGS["tiny-prefill-f32"], seed=1)
    for n in "rwkvab":
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])


def test_shapes_and_dtypes():
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=33, H=3)
    for n in "rwkvab":
        assert x[n].shape == (2, 33, 3, 64) and x[n].dtype == np.uint16
    assert x["state_in"].shape == (2, 3, 64, 64) and x["state_in"].dtype == np.float32
    x0 = make_inputs(CONFIGS["tiny-prefill-f32"])
    assert x0["r"].dtype == np.float32 and x0["state_in"] is None


def test_distributions():
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=512, H=4)
    f = {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in "rwkvab"}
    assert abs(f["r"].std() - 1.0) < 0.02 and abs(f["k"].std() - 0.125) < 0.003
    assert f["w"].min() >= np.exp(-np.exp(-0.5)) - 1e-2 and f["w"].max() <= 1.0
    kk = -f["a"]
    norms = np.linalg.norm(kk, axis=-1)
    assert np.all(np.abs(norms - 1.0) < 2e-2)  # unit before the bfloat16 cast
    alr = f["b"] / np.where(kk == 0, 1, kk)
    assert np.all((alr[kk != 0] > -1e-2) & (alr[kk != 0] < 1.01))


def test_long_context_decay_and_forced_learning_rates():
    cfg = CONFIGS["D4096-long-prefill"]
    x = make_inputs(cfg, B=1, T=256, H=8)
    w = bf16_bits_to_f32(x["w"])
    assert w.min() >= np.float32(np.exp(-np.exp(-0.1))) - 1e-2
    frac_one = np.mean(w == 1.0)
    assert 0.15 < frac_one < 0.30, frac_one  # near-1 decays that round to exactly 1 in bfloat16
    b = bf16_bits_to_f32(x["b"])
    assert np.mean(b == 0) > 0.009  # forced a_lr = 0


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # ties to even
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_state_size_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "state_size.json")))
    D, L, N = g["D"], g["L"], g["head_size"]
    H = D // N
    per_layer = H * N * N  # one [H, N, N] state per layer, as laid out by the library
    assert per_layer == g["wkv_state_per_layer"] == 64 * D
    assert L * (2 * D + per_layer) == g["state_params_total"]
