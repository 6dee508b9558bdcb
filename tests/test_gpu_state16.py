"""GPU parity of the single-token step with a 16-bit stored state (rwkv7_wkv_step_q).

Bars, derived from the arithmetic:
  - y of one step: the kernel computes the token in float32 from the exactly widened
    state, like the oracle does in float64, so y agrees to float32 rounding
    (<= 1e-5, well inside the 2e-3 bar for bfloat16 inputs).
  - the stored state of one step: both sides round the same token result to the
    16-bit format, the kernel from float32 and the oracle from float64; they can
    differ only where the two straddle a rounding boundary, so an element is within
    one encoding step, unless the sum S w + sa b + v k cancels to far below the
    state's scale, where the float32 error of the unrounded value (a few 2^-24 of
    the terms) spans several 16-bit units: there the difference stays below
    2^-16 max|S| (a 64x margin over that error). Differing elements are rare (<= 1%).
  - 256 in-place steps: each side rounds its own trajectory, so the rare one-step
    differences are carried along and decay; the final states agree within 4 units
    in the last place of the largest element, and y within 2e-3.
The drift of a 16-bit stored state from the float32-state trajectory (what the
README's fp32 note warns about) is measured and only bounded loosely.
"""
import numpy as np
import pytest

import oracle
from linear_rnn_amd import wkv
from linear_rnn_amd.inputs import CONFIGS, make_inputs
from tests.gpu_util import TOL_BF16, rel, sample_units, say, to_dev

pytestmark = pytest.mark.gpu
FMTS = {"bf16": (wkv.RWKV7_STATE_BF16, 2.0 ** -8), "f16": (wkv.RWKV7_STATE_F16, 2.0 ** -11)}


@pytest.fixture(scope="module")
def torch():
    import torch as t
    wkv.lib()
    oracle.build(force=False)
    return t


def tdtype(torch, fmt):
    return {"bf16": torch.bfloat16, "f16": torch.float16}[fmt]


def bits_to_dev(torch, bits, fmt):
    return torch.from_numpy(bits.view(np.int16)).cuda().view(tdtype(torch, fmt))


def dev_to_bits(t):
    import torch as tt
    return t.contiguous().view(tt.int16).cpu().numpy().view(np.uint16)


def ordinal(bits):
    """Encodings mapped to a line on which neighbouring values differ by 1 (+0 and -0 both 0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_state_bits(got_bits, ref_bits, fmt):
    """Assert the one-step stored-state bar; return (largest encoding gap, fraction that differ)."""
    gap = np.abs(ordinal(got_bits) - ordinal(ref_bits))
    frac = float(np.mean(gap != 0))
    g = oracle.widen16(got_bits, fmt)
    r = oracle.widen16(ref_bits, fmt)
    smax = float(np.max(np.abs(r)))
    far = gap > 1
    worst = float(np.max(np.abs(g - r)[far])) / smax if far.any() else 0.0
    say("state bits: max gap", int(gap.max()), "frac differing", frac, "elements > 1 step:", int(far.sum()),
        "their worst |diff|/max|S|", worst, "at |S|/max|S| <=", float(np.max(np.abs(r)[far])) / smax if far.any()
        else 0.0)
    assert worst <= 2.0 ** -16 and frac <= 0.01, (int(gap.max()), worst, frac)
    return int(gap.max()), frac


def step_q(d, state_in, y, state_out):
    wkv.rwkv7_wkv_step_q(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], state_in, y, state_out)


def test_f32_state_code_is_the_plain_step(torch):
    say("step_q with float32 state vs step")
    x = make_inputs(CONFIGS["D2048-decode"], B=6, H=7, step=0)
    d = to_dev(x)
    y1 = torch.empty((6, 1, 7, 64), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    s1 = torch.empty_like(d["state_in"])
    s2 = torch.empty_like(s1)
    wkv.rwkv7_wkv_step(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"], y1, s1)
    step_q(d, d["state_in"], y2, s2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("B,H", [(512, 32), (3, 5), (1, 1)])
def test_one_step_vs_oracle(torch, fmt, B, H):
    say("step_q one step", fmt, B, H)
    x = make_inputs(CONFIGS["D2048-decode"], B=B, H=H, step=0)
    bits = oracle.round16(x["state_in"].astype(np.float64), fmt)
    d = to_dev(x)
    s_in = bits_to_dev(torch, bits, fmt)
    s_out = torch.empty_like(s_in)
    y = torch.empty((B, 1, H, 64), dtype=torch.float32, device="cuda")
    step_q(d, s_in, y, s_out)
    torch.cuda.synchronize()
    yr, sr_bits = oracle.step_q(*(x[n] for n in "rwkvab"), bits, fmt)
    ey = rel(y.cpu().numpy(), yr)
    say("step_q one step y error", fmt, B, H, ey)
    assert ey <= TOL_BF16 and ey <= 1e-5, ey
    check_state_bits(dev_to_bits(s_out), sr_bits, fmt)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_null_state_in_and_in_place(torch, fmt):
    say("step_q NULL state_in, then in place", fmt)
    x = make_inputs(CONFIGS["D2048-decode"], B=4, H=6, step=1, with_state=False)
    d = to_dev(x)
    st = torch.empty((4, 6, 64, 64), dtype=tdtype(torch, fmt), device="cuda")
    y = torch.empty((4, 1, 6, 64), dtype=torch.float32, device="cuda")
    step_q(d, None, y, st)  # from zeros
    step_q(d, st, y, st)  # again, in place
    torch.cuda.synchronize()
    _, b1 = oracle.step_q(*(x[n] for n in "rwkvab"), None, fmt)
    yr, b2 = oracle.step_q(*(x[n] for n in "rwkvab"), b1, fmt)
    check_state_bits(dev_to_bits(st), b2, fmt)
    assert rel(y.cpu().numpy(), yr) <= 1e-5


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_d2048_decode_256_steps(torch, fmt):
    """256 in-place steps at B=512, H=32 against the oracle's own 16-bit trajectory on 64
    sampled heads, and against the float32-state kernel (drift of the reduced state)."""
    cfg = CONFIGS["D2048-decode"]
    say("step_q D2048-decode, 256 steps", fmt)
    code, ulp = FMTS[fmt]
    units = sample_units(cfg.B, cfg.H, 64, seed=5)
    bs = np.array([u[0] for u in units])
    hs = np.array([u[1] for u in units])
    x0 = make_inputs(cfg, step=0)
    bits0 = oracle.round16(x0["state_in"].astype(np.float64), fmt)
    sq = bits_to_dev(torch, bits0, fmt)
    s32 = torch.from_numpy(oracle.widen16(bits0, fmt).astype(np.float32)).cuda()  # same start, float32 carry
    y = torch.empty((cfg.B, 1, cfg.H, 64), dtype=torch.float32, device="cuda")
    y32 = torch.empty_like(y)
    ref_bits = np.ascontiguousarray(bits0[bs, hs][:, None])  # [U,1,64,64] as U heads of one batch row
    got_y, ref_y, y_f32 = [], [], []
    for step in range(cfg.steps):
        x = x0 if step == 0 else make_inputs(cfg, step=step, with_state=False)
        d = to_dev(x)
        step_q(d, sq, y, sq)
        wkv.rwkv7_wkv_step(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], s32, y32, s32)
        sub = {n: np.ascontiguousarray(x[n][bs, :, hs, :][:, :, None, :]) for n in "rwkvab"}
        yr, ref_bits = oracle.step_q(*(sub[n] for n in "rwkvab"), ref_bits, fmt)
        ref_y.append(yr[:, 0, 0, :])
        got_y.append(y[bs, 0, hs, :].cpu().numpy())
        y_f32.append(y32[bs, 0, hs, :].cpu().numpy())
    torch.cuda.synchronize()
    got_s = oracle.widen16(dev_to_bits(sq)[bs, hs], fmt)
    ref_s = oracle.widen16(ref_bits[:, 0], fmt)
    es = float(np.max(np.abs(got_s - ref_s)))
    smax = float(np.max(np.abs(ref_s)))
    ey = rel(np.stack(got_y), np.stack(ref_y))
    # drift from the float32-state trajectory (same inputs, same kernel arithmetic)
    drift_s = rel(got_s, s32.cpu().numpy()[bs, hs])
    drift_y = rel(np.stack(got_y), np.stack(y_f32))
    say("step_q 256 steps", fmt, "state gap/ulp(max)", es / (ulp * smax), "y", ey, "drift from f32 state: s",
        drift_s, "y", drift_y)
    assert es <= 4 * ulp * smax, (es, smax)
    assert ey <= TOL_BF16, ey
    assert drift_s <= {"bf16": 0.1, "f16": 0.02}[fmt] and drift_y <= {"bf16": 0.1, "f16": 0.02}[fmt]
