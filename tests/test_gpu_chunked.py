"""GPU parity of the chunked (MFMA) prefill against the float64 oracle and the sequential kernel.

Every test runs both chunked variants: the fused one (one workgroup per head) and the split
one (chunk-parallel prep kernel, per-head scan kernel)."""
import numpy as np
import pytest

import oracle
from linear_rnn_amd import wkv
from linear_rnn_amd.inputs import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs
from tests.gpu_util import TOL_BF16, oracle_units, rel, sample_units, say, to_dev

pytestmark = pytest.mark.gpu
SEQ = wkv.RWKV7_ALGO_SEQUENTIAL
VARIANTS = {"fused": wkv.RWKV7_ALGO_CHUNKED, "split": wkv.RWKV7_ALGO_CHUNKED_SPLIT}


@pytest.fixture(params=sorted(VARIANTS), scope="module")
def CH(request):
    return VARIANTS[request.param]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    wkv.lib()
    oracle.build(force=False)
    return t


def run(torch, d, algo, state=True):
    y, s = wkv.wkv7(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"] if state else None, algo=algo)
    torch.cuda.synchronize()
    return y.cpu().numpy(), s.cpu().numpy()


# 13, 14 and 15 chunks straddle the split scan loop's unroll of 14 (twice its 7-slot ring); 9, 10, 11,
# 20 and 21 chunks straddle one and two turns of the fused kernel's 10-slot ring (161 and 321 tokens
# end in a one-token chunk)
@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (1, 15, 2), (2, 16, 3), (1, 17, 2), (2, 33, 3), (3, 100, 5),
                                   (1, 144, 2), (1, 160, 3), (1, 161, 2), (1, 208, 2), (1, 224, 2),
                                   (1, 240, 2), (1, 320, 2), (2, 321, 3), (2, 1000, 12)])
def test_ragged_vs_oracle(torch, CH, B, T, H):
    say("algo", CH, "chunked ragged", B, T, H)
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=B, T=T, H=H, seed=200 + T)
    y, s = run(torch, to_dev(x), CH)
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y, yr) <= TOL_BF16 and rel(s, sr) <= TOL_BF16, (rel(y, yr), rel(s, sr))


# At least as many heads as compute units: the fused kernel stages y as whole token rows
# (one chunk late) instead of per-wave tiles; ragged ends, 1-token last chunks, more heads than CUs
@pytest.mark.parametrize("B,T,H", [(16, 33, 16), (4, 161, 64), (20, 17, 16)])
def test_ragged_many_heads_vs_oracle(torch, CH, B, T, H):
    say("algo", CH, "chunked ragged, many heads", B, T, H)
    x = make_inputs(CONFIGS["L24-D1024-prefill-resume"], B=B, T=T, H=H, seed=300 + T)
    y, s = run(torch, to_dev(x), CH)
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y, yr) <= TOL_BF16 and rel(s, sr) <= TOL_BF16, (rel(y, yr), rel(s, sr))


# Fewer heads than compute units but more than half of them (129 to 255 on 256 CUs): per-wave y
# tiles, ragged ends, a 1-token last chunk
@pytest.mark.parametrize("B,T,H", [(3, 40, 50), (1, 161, 200), (1, 33, 129)])
def test_ragged_mid_heads_vs_oracle(torch, CH, B, T, H):
    say("algo", CH, "chunked ragged, mid heads", B, T, H)
    x = make_inputs(CONFIGS["L24-D1024-prefill-resume"], B=B, T=T, H=H, seed=400 + T)
    y, s = run(torch, to_dev(x), CH)
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y, yr) <= TOL_BF16 and rel(s, sr) <= TOL_BF16, (rel(y, yr), rel(s, sr))


def test_zero_initial_state(torch, CH):
    say("algo", CH, "chunked, state_in NULL")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=77, H=4, seed=3)
    y, s = run(torch, to_dev(x), CH, state=False)
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=None)
    assert rel(y, yr) <= TOL_BF16 and rel(s, sr) <= TOL_BF16


def test_f32_inputs_are_refused(torch, CH):
    """The chunked algorithm takes bfloat16 inputs only; float32 inputs stay on the sequential kernel."""
    say("algo", CH, "chunked, f32 inputs refused")
    x = make_inputs(CONFIGS["tiny-prefill-f32"])
    with pytest.raises(wkv.Rwkv7Error) as ei:
        run(torch, to_dev(x), CH)
    assert ei.value.status == -7


def test_l12_d768_full(torch, CH):
    cfg = CONFIGS["L12-D768-prefill"]
    say("algo", CH, "chunked L12-D768 full", cfg)
    x = make_inputs(cfg)
    y, s = run(torch, to_dev(x), CH)
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    e = (rel(y, yr), rel(s, sr))
    say("L12-D768 chunked errors", e)
    assert e[0] <= TOL_BF16 and e[1] <= TOL_BF16, e


def test_l24_d1024_full_and_resume(torch, CH):
    """One pass and 4 x 1024-token segments with the state carried, each against the oracle."""
    cfg = CONFIGS["L24-D1024-prefill-resume"]
    say("algo", CH, "chunked L24-D1024 full + resume", cfg)
    x = make_inputs(cfg)
    d = to_dev(x)
    y1, s1 = run(torch, d, CH)
    st = d["state_in"].clone()
    ys = []
    for i in range(4):
        sl = {n: d[n][:, 1024 * i:1024 * (i + 1)].contiguous() for n in "rwkvab"}
        yy = torch.empty(sl["r"].shape, dtype=torch.float32, device="cuda")
        wkv.rwkv7_wkv_prefill_ex(sl["r"], sl["w"], sl["k"], sl["v"], sl["a"], sl["b"], st, yy, st, algo=CH)
        ys.append(yy)
    torch.cuda.synchronize()
    y4 = torch.cat(ys, 1).cpu().numpy()
    s4 = st.cpu().numpy()
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    e = (rel(y1, yr), rel(s1, sr), rel(y4, yr), rel(s4, sr))
    say("L24-D1024 chunked errors (one pass y, s; resumed y, s)", e)
    assert max(e) <= TOL_BF16, e
    # segments are chunk-aligned, so the resumed run repeats the one-pass arithmetic exactly
    assert np.array_equal(y4, y1) and np.array_equal(s4, s1)
    # no state_out: a sequence of several slabs carries its state through a workspace copy instead
    yn, _ = wkv.wkv7(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"], algo=CH, want_state=False)
    torch.cuda.synchronize()
    assert np.array_equal(yn.cpu().numpy(), y1)


def test_unaligned_resume(torch, CH):
    say("algo", CH, "chunked unaligned resume")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=300, H=3, seed=11)
    d = to_dev(x)
    st = d["state_in"].clone()
    ys = []
    for lo, hi in ((0, 37), (37, 38), (38, 200), (200, 300)):
        sl = {n: d[n][:, lo:hi].contiguous() for n in "rwkvab"}
        yy = torch.empty(sl["r"].shape, dtype=torch.float32, device="cuda")
        wkv.rwkv7_wkv_prefill_ex(sl["r"], sl["w"], sl["k"], sl["v"], sl["a"], sl["b"], st, yy, st, algo=CH)
        ys.append(yy)
    torch.cuda.synchronize()
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    e = (rel(torch.cat(ys, 1).cpu().numpy(), yr), rel(st.cpu().numpy(), sr))
    assert max(e) <= TOL_BF16, e


def test_d4096_long_sampled_heads_and_vs_sequential(torch, CH):
    cfg = CONFIGS["D4096-long-prefill"]
    say("algo", CH, "chunked D4096-long full, 16 sampled heads + sequential comparison", cfg)
    x = make_inputs(cfg)
    d = to_dev(x)
    y, s = wkv.wkv7(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"], algo=CH)
    ys, ss = wkv.wkv7(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"], algo=SEQ)
    torch.cuda.synchronize()
    # whole-tensor agreement with the float32 sequential kernel (itself ~1e-6 from the oracle)
    dy = (torch.max(torch.abs(y - ys)) / torch.max(torch.abs(ys))).item()
    ds = (torch.max(torch.abs(s - ss)) / torch.max(torch.abs(ss))).item()
    say("D4096-long chunked vs sequential", dy, ds)
    assert dy <= TOL_BF16 and ds <= TOL_BF16, (dy, ds)
    units = sample_units(cfg.B, cfg.H, 16, seed=4)
    ref = oracle_units(x, units)
    yg = np.stack([y[b, :, h].cpu().numpy() for (b, h) in units])
    sg = np.stack([s[b, h].cpu().numpy() for (b, h) in units])
    yr = np.stack([ref[u][0] for u in units])
    sr = np.stack([ref[u][1] for u in units])
    e = (rel(yg, yr), rel(sg, sr))
    say("D4096-long chunked vs oracle (sampled)", e)
    assert max(e) <= TOL_BF16, e


def test_extreme_decays(torch, CH):
    """w in {0, 1e-6, 1e-2, 0.5, 1}: below 2^-15 the chunked form clamps, which moves a decayed
    term by at most 2^-15 of its size."""
    say("algo", CH, "chunked extreme decays")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=90, H=3, seed=17)
    rng = np.random.default_rng(17)
    choices = np.array([0.0, 1e-6, 1e-2, 0.5, 1.0], dtype=np.float32)
    x["w"] = f32_to_bf16_bits(choices[rng.integers(0, 5, size=x["w"].shape)])
    y, s = run(torch, to_dev(x), CH)
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y, yr) <= TOL_BF16 and rel(s, sr) <= TOL_BF16, (rel(y, yr), rel(s, sr))


def test_delta_rule_retrieval(torch, CH):
    """w = 1, a = -kk, b = kk, k = r = kk (unit): y_t = v_t."""
    say("algo", CH, "chunked delta rule")
    rng = np.random.default_rng(23)
    B, T, H = 1, 64, 2
    kk = rng.standard_normal((B, T, H, 64))
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, 64))
    x = {n: f32_to_bf16_bits(a.astype(np.float32)) for n, a in
         dict(r=kk, k=kk, a=-kk, b=kk, w=np.ones_like(kk), v=v).items()}
    x["state_in"] = (rng.standard_normal((B, H, 64, 64)) * 0.3).astype(np.float32)
    y, _ = run(torch, to_dev(x), CH)
    yr, _ = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y, yr) <= TOL_BF16
    # against v itself, up to the bfloat16 rounding of the keys (|kk|^2 != 1 exactly)
    assert rel(y, bf16_bits_to_f32(x["v"])) <= 2e-2


def test_deterministic(torch, CH):
    say("algo", CH, "chunked determinism")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=300, H=6, seed=8)
    d = to_dev(x)
    y1, s1 = run(torch, d, CH)
    y2, s2 = run(torch, d, CH)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_auto_uses_chunked_for_bf16(torch):
    say("auto dispatch")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=1, T=40, H=2, seed=4)
    d = to_dev(x)
    y_auto = torch.empty((1, 40, 2, 64), dtype=torch.float32, device="cuda")
    wkv.rwkv7_wkv_prefill(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"], y_auto, None)
    y_ch, _ = run(torch, d, wkv.RWKV7_ALGO_CHUNKED_SPLIT)
    torch.cuda.synchronize()
    assert np.array_equal(y_auto.cpu().numpy(), y_ch)
