"""Pins of the oracle's 16-bit stored-state support (reduced-precision decode state).

The oracle widens bfloat16 / binary16 state encodings exactly and rounds float64
states to them, to nearest with ties to even. These CPU tests hold both against
rules that share no code with the oracle: numpy's float16 conversions, the input
module's float32 -> bfloat16 rounding, and exact rational nearest-neighbour checks.
"""
import numpy as np
import pytest

import oracle
from linear_rnn_amd.inputs import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs
from tests import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle


def test_widen16_all_encodings(orc):
    assert pins.pin_widen16(orc) == 0.0


def test_round16_rules(orc):
    assert pins.pin_round16(orc) == 0.0


def test_ties_go_to_even(orc):
    # 1 + 2^-8 lies halfway between bfloat16 1 and 1 + 2^-7; 1 + 3*2^-8 between 1 + 2^-7 and 1 + 2^-6
    assert orc.round16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]), "bf16").tolist() == [0x3F80, 0x3F82]
    # binary16: 1 + 2^-11 halfway between 1 and 1 + 2^-10
    assert orc.round16(np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11]), "f16").tolist() == [0x3C00, 0x3C02]


def test_overflow_and_subnormals(orc):
    got = orc.round16(np.array([65504.0, 65519.0, 65520.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0001]), "f16")
    assert got.tolist() == [0x7BFF, 0x7BFF, 0x7C00, 0x0001, 0x0000, 0x0001]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_identity_token_keeps_a_representable_state(orc, fmt):
    """w = 1, a = b = v = k = 0: the step must hand back the stored state bit for bit."""
    rng = np.random.default_rng(5)
    s = rng.standard_normal((1, 2, 64, 64)) * 0.3
    bits = orc.round16(s, fmt)
    z = np.zeros((1, 1, 2, 64), dtype=np.float32)
    ones = np.ones_like(z)
    y, out = orc.step_q(z, ones, z, z, z, z, bits, fmt)
    assert np.array_equal(out, bits)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_step_q_is_f64_step_then_rounding(orc, fmt):
    """A stored-state step equals the float64 step from the widened state, rounded once."""
    cfg = CONFIGS["D2048-decode"]
    x = make_inputs(cfg, B=2, H=3, step=0)
    bits = orc.round16(x["state_in"].astype(np.float64), fmt)
    y, out = orc.step_q(*(x[n] for n in "rwkvab"), bits, fmt)
    y2, s2 = orc.wkv7(*(x[n] for n in "rwkvab"), state_in=orc.widen16(bits, fmt))
    assert np.array_equal(y, y2)
    assert np.array_equal(out, orc.round16(s2, fmt))
    # and the rounding error of the stored state is within half a unit in the last place
    err = np.abs(orc.widen16(out, fmt) - s2)
    ulp = {"bf16": 2.0 ** -7, "f16": 2.0 ** -10}[fmt]
    assert np.all(err <= 0.5 * ulp * np.exp2(np.floor(np.log2(np.maximum(np.abs(s2), 2.0 ** -14)))) + 2.0 ** -24)


def test_bf16_rounding_agrees_with_input_module_on_state_values(orc):
    rng = np.random.default_rng(9)
    s = (rng.standard_normal(5000) * 0.1).astype(np.float32)
    assert np.array_equal(orc.round16(s.astype(np.float64), "bf16"), f32_to_bf16_bits(s))
    assert np.array_equal(orc.widen16(f32_to_bf16_bits(s), "bf16"), bf16_bits_to_f32(f32_to_bf16_bits(s)))
