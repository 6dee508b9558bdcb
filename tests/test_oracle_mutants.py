"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check the pins catch each.

Every mutant is a one-expression edit of oracle/wkv7_oracle.c, compiled to a temporary
library; at least one pin must then report a deviation far above float64 rounding.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "wkv7_oracle.c")

# (name, original text, replacement)
MUTANTS = [
    ("drop_ab_term", "+ sa * b[j]", ""),
    ("ab_sign_flip", "+ sa * b[j]", "- sa * b[j]"),
    ("drop_vk_term", "+ v[i] * k[j]", ""),
    ("swap_v_k", "v[i] * k[j]", "k[i] * v[j]"),
    ("decay_rows_not_columns", "Si[j] * w[j]", "Si[j] * w[i]"),
    ("decay_complement", "Si[j] * w[j]", "Si[j] * (1.0 - w[j])"),
    ("swap_a_b", "sa += Si[j] * a[j]", "sa += Si[j] * b[j]"),
    ("sa_wrong_index", "sa += Si[j] * a[j]", "sa += Si[j] * a[i]"),
    ("readout_with_k", "yi += Si[j] * r[j]", "yi += Si[j] * k[j]"),
    ("readout_before_update", "yi += Si[j] * r[j]", "yi += ((Si[j] - sa * b[j] - v[i] * k[j]) / w[j]) * r[j]"),
    ("transposed_state_in", "unit * N * N + i * N + j", "unit * N * N + j * N + i"),
    ("previous_token_k", "k[j] = widen(J->k, J->in_dtype, base + j);",
     "k[j] = widen(J->k, J->in_dtype, (t ? base - (size_t)(H * N) : base) + j);"),
    ("bf16_shift", "<< 16;", "<< 15;"),
    ("round_half_away", "rint(x / quantum)", "round(x / quantum)"),
    ("round_toward_zero", "rint(x / quantum)", "trunc(x / quantum)"),
    ("f16_subnormal_floor", "round_to_format(x[i], 11, -14, 65504.0)", "round_to_format(x[i], 11, -15, 65504.0)"),
    ("f16_precision", "round_to_format(x[i], 11, -14, 65504.0)", "round_to_format(x[i], 10, -14, 65504.0)"),
    ("f16_no_overflow", "fabs(r) > maxv ?", "fabs(r) > 2 * maxv ?"),
    ("f16_widen_bias", "e - 25);", "e - 24);"),
    ("f16_encode_bias", "(lead + 15) << 10", "(lead + 14) << 10"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "anchor %r not found in the oracle source" % old
    mut = src.replace(old, new)
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(mut)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC", "-pthread", str(c),
                    "-o", str(so), "-lm"], check=True)
    return str(so)


class _MutantOracle:
    """Same call surface as the oracle module, bound to a mutant library."""

    def __init__(self, so_path):
        lib = ctypes.CDLL(so_path)
        f = lib.wkv7_oracle_f64
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int64] * 4 + [ctypes.c_int] * 3
        for name in ("wkv7_oracle_round16", "wkv7_oracle_widen16"):
            g = getattr(lib, name)
            g.restype = ctypes.c_int
            g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
        self._lib = lib

    def _bound(self, fn, *args, **kw):
        saved = oracle._lib
        oracle._lib = self._lib
        try:
            return fn(*args, **kw)
        finally:
            oracle._lib = saved

    def wkv7(self, *args, **kw):
        return self._bound(oracle.wkv7, *args, **kw)

    def round16(self, *args, **kw):
        return self._bound(oracle.round16, *args, **kw)

    def widen16(self, *args, **kw):
        return self._bound(oracle.widen16, *args, **kw)


def _all_pins(orc):
    res = {
        "brute_force": pins.pin_brute_force(orc),
        "decayed_la_a0": pins.pin_decayed_linear_attention(orc, zero="a"),
        "decayed_la_b0": pins.pin_decayed_linear_attention(orc, zero="b"),
        "plain_la": pins.pin_plain_linear_attention(orc),
        "delta_rule": pins.pin_delta_rule_retrieval(orc),
        "memoryless": pins.pin_memoryless(orc),
        "linearity": pins.pin_linearity(orc),
        "permutations": pins.pin_permutations(orc),
    }
    # exact run in bf16 encoding exercises the input widening
    x = pins.dyadic_inputs(seed=11, T=3)
    ye, se, _ = pins.exact_fraction_run(x)
    y, s = pins.call(orc, pins.cast_inputs(x, "bf16"))
    res["exact_bf16"] = max(pins.rel(y, ye), pins.rel(s, se))
    res["widen16"] = pins.pin_widen16(orc)
    res["round16"] = pins.pin_round16(orc)
    return res


def test_unmutated_oracle_passes_all_pins():
    oracle.build(force=False)
    res = _all_pins(oracle)
    assert max(res.values()) < 1e-12, res


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    orc = _MutantOracle(_build_mutant(tmp_path, name, old, new))
    with np.errstate(all="ignore"):
        res = _all_pins(orc)
    caught = {k: v for k, v in res.items() if not (v < 1e-6)}
    assert caught, "mutant %s passed every pin: %s" % (name, res)
