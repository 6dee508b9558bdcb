"""The float64 oracle against what the mathematics fixes (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import pins

TOL = 1e-12  # float64 arithmetic against float64 constructions of the same exact result


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle


def test_brute_force_matrix_products(orc):
    assert pins.pin_brute_force(orc) < TOL


@pytest.mark.parametrize("T", [1, 2, 5])
def test_brute_force_tiny_T(orc, T):
    assert pins.pin_brute_force(orc, seed=10 + T, B=1, T=T, H=2) < TOL


@pytest.mark.parametrize("zero", ["a", "b"])
def test_low_rank_off_is_decayed_linear_attention(orc, zero):
    assert pins.pin_decayed_linear_attention(orc, zero=zero) < TOL


def test_w1_a0_is_plain_linear_attention(orc):
    assert pins.pin_plain_linear_attention(orc) < TOL


def test_delta_rule_retrieval(orc):
    assert pins.pin_delta_rule_retrieval(orc) < 1e-12


def test_memoryless(orc):
    assert pins.pin_memoryless(orc) < TOL


def test_linearity_in_v_and_state(orc):
    assert pins.pin_linearity(orc) < TOL


def test_permutation_equivariance(orc):
    assert pins.pin_permutations(orc) < TOL


def test_split_resume(orc):
    assert pins.pin_split_resume(orc) == 0.0


def test_zero_state_default(orc):
    x = pins.rand_inputs(np.random.default_rng(9), 1, 5, 2)
    y0, s0 = pins.call(orc, dict(x, state_in=np.zeros_like(x["state_in"])))
    y1, s1 = pins.call(orc, dict(x, state_in=None))
    assert np.array_equal(y0, y1) and np.array_equal(s0, s1)


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_exact_rational_run(orc, dtype):
    """Dyadic inputs: the oracle must equal exact rational arithmetic bit for bit, in every
    input encoding, and every intermediate must fit float32 exactly (the same inputs are the
    GPU's bit-exact case)."""
    x = pins.dyadic_inputs(seed=11, T=4)
    ye, se, bits = pins.exact_fraction_run(x)
    assert bits <= 24, bits
    xin = x if dtype == "f64" else pins.cast_inputs(x, dtype)
    y, s = pins.call(orc, xin)
    assert np.array_equal(y, ye) and np.array_equal(s, se)
    # every exact result is a float32 value
    assert np.array_equal(ye.astype(np.float32).astype(np.float64), ye)
    assert np.array_equal(se.astype(np.float32).astype(np.float64), se)


def test_bf16_widening_known_bits(orc):
    """bfloat16 encodings from the format's definition (sign, 8-bit exponent, 7-bit fraction)."""
    one = np.full((1, 1, 1, 64), 0x3F80, dtype=np.uint16)      # 1.0
    half = np.full((1, 1, 1, 64), 0x3F00, dtype=np.uint16)     # 0.5
    m_three_q = np.full((1, 1, 1, 64), 0xBF40, dtype=np.uint16)  # -0.75
    zero = np.zeros((1, 1, 1, 64), dtype=np.uint16)
    # S_1 = v k^T with v = -0.75, k = 0.5; y = S_1 r with r = 1 -> each y_i = 64 * (-0.375)
    y, s = orc.wkv7(one, one, half, m_three_q, zero, zero)
    assert np.all(y == -24.0) and np.all(s == -0.375)


def test_threads_do_not_change_result(orc):
    x = pins.rand_inputs(np.random.default_rng(12), 3, 6, 5)
    y1, s1 = pins.call(orc, x, nthreads=1)
    y2, s2 = pins.call(orc, x, nthreads=7)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_bad_arguments_raise(orc):
    x = pins.rand_inputs(np.random.default_rng(13), 1, 2, 1)
    with pytest.raises(ValueError):
        orc.wkv7(x["r"], x["w"], x["k"][:, :1], x["v"], x["a"], x["b"])
    with pytest.raises(TypeError):
        orc.wkv7(*(x[n].astype(np.int32) for n in "rwkvab"))
