"""GPU parity of the sequential prefill and the single-token step against the float64 oracle."""
import numpy as np
import pytest

import oracle
from linear_rnn_amd import wkv
from linear_rnn_amd.inputs import CONFIGS, make_inputs
from tests import pins
from tests.gpu_util import TOL_BF16, TOL_F32, oracle_units, rel, sample_units, say, to_dev

pytestmark = pytest.mark.gpu
SEQ = wkv.RWKV7_ALGO_SEQUENTIAL


@pytest.fixture(scope="module")
def torch():
    import torch as t
    wkv.lib()  # loud failure if the HIP library is missing
    oracle.build(force=False)
    return t


def run_prefill(torch, d, algo=SEQ):
    y, s = wkv.wkv7(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"], algo=algo)
    torch.cuda.synchronize()
    return y.cpu().numpy(), s.cpu().numpy()


def test_tiny_f32(torch):
    say("tiny f32 prefill, sequential")
    x = make_inputs(CONFIGS["tiny-prefill-f32"])
    y, s = run_prefill(torch, to_dev(x))
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y, yr) <= TOL_F32 and rel(s, sr) <= TOL_F32, (rel(y, yr), rel(s, sr))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_exact_dyadic_bit_for_bit(torch, dtype):
    """Inputs whose recurrence is exact in float32 (pinned against rationals on the CPU):
    the GPU must reproduce the exact result bit for bit, in prefill and in steps."""
    say("exact dyadic", dtype)
    x = pins.cast_inputs(pins.dyadic_inputs(seed=11, B=2, T=4, H=3), dtype)
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    d = to_dev(x)
    y, s = run_prefill(torch, d)
    assert np.array_equal(y.astype(np.float64), yr) and np.array_equal(s.astype(np.float64), sr)
    # the same sequence as T single-token steps, state updated in place
    st = d["state_in"].clone()
    ys = []
    for t in range(4):
        yt = torch.empty((2, 1, 3, 64), dtype=torch.float32, device="cuda")
        sl = {n: d[n][:, t:t + 1].contiguous() for n in "rwkvab"}
        wkv.rwkv7_wkv_step(sl["r"], sl["w"], sl["k"], sl["v"], sl["a"], sl["b"], st, yt, st)
        ys.append(yt)
    torch.cuda.synchronize()
    assert np.array_equal(torch.cat(ys, 1).cpu().numpy().astype(np.float64), yr)
    assert np.array_equal(st.cpu().numpy().astype(np.float64), sr)


@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (2, 31, 3), (1, 33, 2), (3, 100, 5), (1, 1000, 12)])
def test_ragged_bf16_sequential(torch, B, T, H):
    say("ragged bf16 sequential", B, T, H)
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=B, T=T, H=H, seed=100 + T)
    y, s = run_prefill(torch, to_dev(x))
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y, yr) <= 1e-5 and rel(s, sr) <= 1e-5, (rel(y, yr), rel(s, sr))


def test_many_heads_path(torch):
    """B*H >= 2048 selects the one-head-per-workgroup tiling."""
    say("many heads sequential")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=64, T=20, H=32, seed=5)
    y, s = run_prefill(torch, to_dev(x))
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y, yr) <= 1e-5 and rel(s, sr) <= 1e-5


def test_l12_d768_full(torch):
    cfg = CONFIGS["L12-D768-prefill"]
    say("L12-D768 full, sequential", cfg)
    x = make_inputs(cfg)
    y, s = run_prefill(torch, to_dev(x))
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y, yr) <= TOL_BF16 and rel(s, sr) <= TOL_BF16
    assert rel(y, yr) <= 1e-5 and rel(s, sr) <= 1e-5  # what the fp32 recurrence actually achieves


def test_l24_d1024_split_resume_bit_identical(torch):
    """4 segments of 1024 tokens with the state carried equal one pass, bit for bit."""
    cfg = CONFIGS["L24-D1024-prefill-resume"]
    say("L24-D1024 split/resume, sequential", cfg)
    x = make_inputs(cfg)
    d = to_dev(x)
    y1, s1 = run_prefill(torch, d)
    st = d["state_in"].clone()
    ys = []
    for i in range(4):
        sl = {n: d[n][:, 1024 * i:1024 * (i + 1)].contiguous() for n in "rwkvab"}
        yy = torch.empty_like(sl["r"], dtype=torch.float32)
        wkv.rwkv7_wkv_prefill_ex(sl["r"], sl["w"], sl["k"], sl["v"], sl["a"], sl["b"], st, yy, st, algo=SEQ)
        ys.append(yy)
    torch.cuda.synchronize()
    assert np.array_equal(torch.cat(ys, 1).cpu().numpy(), y1)
    assert np.array_equal(st.cpu().numpy(), s1)
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert rel(y1, yr) <= TOL_BF16 and rel(s1, sr) <= TOL_BF16, (rel(y1, yr), rel(s1, sr))


def test_d2048_decode_steps(torch):
    """256 in-place steps at B=512, H=32; oracle on 64 sampled heads over all steps."""
    cfg = CONFIGS["D2048-decode"]
    say("D2048-decode decode, 256 steps", cfg)
    units = sample_units(cfg.B, cfg.H, 64, seed=3)
    x0 = make_inputs(cfg, step=0)
    state = torch.from_numpy(x0["state_in"]).cuda()
    s_units = {u: x0["state_in"][u[0], u[1]].copy() for u in units}
    y = torch.empty((cfg.B, 1, cfg.H, 64), dtype=torch.float32, device="cuda")
    worst_y = 0.0
    bs = np.array([u[0] for u in units])
    hs = np.array([u[1] for u in units])
    ref_y_all, got_y_all = [], []
    for step in range(cfg.steps):
        x = x0 if step == 0 else make_inputs(cfg, step=step, with_state=False)
        d = to_dev(x)
        wkv.rwkv7_wkv_step(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], state, y, state)
        sub = {n: np.ascontiguousarray(x[n][bs, :, hs, :][:, :, None, :]) for n in "rwkvab"}
        s_in = np.stack([s_units[u] for u in units])[:, None]
        yr, sr = oracle.wkv7(*(sub[n] for n in "rwkvab"), state_in=s_in)
        for i, u in enumerate(units):
            s_units[u] = sr[i, 0]
        ref_y_all.append(yr[:, 0, 0, :])
        got_y_all.append(y[bs, 0, hs, :].cpu().numpy())
    torch.cuda.synchronize()
    worst_y = rel(np.stack(got_y_all), np.stack(ref_y_all))
    st = state.cpu().numpy()
    worst_s = rel(np.stack([st[u] for u in units]), np.stack([s_units[u] for u in units]))
    assert worst_y <= TOL_BF16 and worst_s <= TOL_BF16, (worst_y, worst_s)
    assert worst_y <= 1e-5 and worst_s <= 1e-5, (worst_y, worst_s)


def test_large_state_step_streams_the_same_bits(torch):
    """A float32 state above the last-level cache's size (B=640, H=32: 320 MiB) takes the step with
    non-temporal state accesses. Its results equal, bit for bit, the same heads stepped in a small
    batch (plain accesses), and match the oracle on sampled heads; three in-place steps."""
    cfg = CONFIGS["D2048-decode"]
    B, H = 640, 32
    say("large-state step (320 MiB float32 state), 3 steps", B, H)
    units = sample_units(B, H, 8, seed=5)
    bsel = sorted({u[0] for u in units})
    xs = [make_inputs(cfg, B=B, H=H, step=s, with_state=(s == 0)) for s in range(3)]
    state = torch.from_numpy(xs[0]["state_in"]).cuda()
    small = torch.from_numpy(np.ascontiguousarray(xs[0]["state_in"][bsel])).cuda()
    y = torch.empty((B, 1, H, 64), dtype=torch.float32, device="cuda")
    ys = torch.empty((len(bsel), 1, H, 64), dtype=torch.float32, device="cuda")
    s_ref = {u: xs[0]["state_in"][u[0], u[1]].copy() for u in units}
    for x in xs:
        d = to_dev(x)
        wkv.rwkv7_wkv_step(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], state, y, state)
        ds = {n: d[n][bsel].contiguous() for n in "rwkvab"}
        wkv.rwkv7_wkv_step(ds["r"], ds["w"], ds["k"], ds["v"], ds["a"], ds["b"], small, ys, small)
        torch.cuda.synchronize()
        assert torch.equal(y[bsel], ys)
        for (b, h) in units:
            sub = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in "rwkvab"}
            yr, sr = oracle.wkv7(*(sub[n] for n in "rwkvab"), state_in=s_ref[(b, h)][None, None])
            s_ref[(b, h)] = sr[0, 0]
            assert rel(y[b, 0, h].cpu().numpy(), yr[0, 0, 0]) <= 1e-5
    assert torch.equal(state[bsel], small)
    st = state.cpu().numpy()
    assert max(rel(st[b, h], s_ref[(b, h)]) for (b, h) in units) <= 1e-5


def test_prefill_equals_steps_bit_identical(torch):
    say("prefill vs steps")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=3, T=50, H=4, seed=9)
    d = to_dev(x)
    y1, s1 = run_prefill(torch, d)
    st = d["state_in"].clone()
    ys = []
    for t in range(50):
        sl = {n: d[n][:, t:t + 1].contiguous() for n in "rwkvab"}
        yt = torch.empty((3, 1, 4, 64), dtype=torch.float32, device="cuda")
        wkv.rwkv7_wkv_step(sl["r"], sl["w"], sl["k"], sl["v"], sl["a"], sl["b"], st, yt, st)
        ys.append(yt)
    torch.cuda.synchronize()
    assert np.array_equal(torch.cat(ys, 1).cpu().numpy(), y1)
    assert np.array_equal(st.cpu().numpy(), s1)


def test_d4096_long_sampled_heads(torch):
    cfg = CONFIGS["D4096-long-prefill"]
    say("D4096-long full, sequential, 16 sampled heads", cfg)
    x = make_inputs(cfg)
    units = sample_units(cfg.B, cfg.H, 16, seed=4)
    d = to_dev(x)
    y, s = wkv.wkv7(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"], algo=SEQ)
    torch.cuda.synchronize()
    ref = oracle_units(x, units)
    yg = np.stack([y[b, :, h].cpu().numpy() for (b, h) in units])
    sg = np.stack([s[b, h].cpu().numpy() for (b, h) in units])
    yr = np.stack([ref[u][0] for u in units])
    sr = np.stack([ref[u][1] for u in units])
    assert rel(yg, yr) <= TOL_BF16 and rel(sg, sr) <= TOL_BF16, (rel(yg, yr), rel(sg, sr))


def test_invariants_on_gpu(torch):
    """Delta-rule retrieval (y = v) and the memoryless case, through the float32 kernel."""
    say("invariants")
    rng = np.random.default_rng(21)
    B, T, H = 2, 40, 3
    kk = rng.standard_normal((B, T, H, 64))
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, 64))
    x = {n: a.astype(np.float32) for n, a in
         dict(r=kk, k=kk, a=-kk, b=kk, w=np.ones_like(kk), v=v).items()}
    x["state_in"] = (rng.standard_normal((B, H, 64, 64)) * 0.3).astype(np.float32)
    y, _ = run_prefill(torch, to_dev(x))
    assert rel(y, x["v"]) <= 1e-5
    x2 = dict(x, w=np.zeros_like(x["w"]), a=np.zeros_like(x["a"]))
    y2, _ = run_prefill(torch, to_dev(x2))
    expect = x["v"].astype(np.float64) * np.sum(x["k"].astype(np.float64) * x["r"], axis=-1, keepdims=True)
    assert rel(y2, expect) <= 1e-5


def test_null_state_in_and_out(torch):
    say("null state in/out")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=17, H=3, seed=3)
    d = to_dev(x)
    y = torch.empty((2, 17, 3, 64), dtype=torch.float32, device="cuda")
    wkv.rwkv7_wkv_prefill_ex(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], None, y, None, algo=SEQ)
    torch.cuda.synchronize()
    yr, _ = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=None)
    assert rel(y.cpu().numpy(), yr) <= 1e-5


def test_empty_sequence_copies_state(torch):
    say("T == 0")
    s_in = torch.randn(2, 3, 64, 64, device="cuda")
    s_out = torch.full_like(s_in, 7.0)
    e = torch.empty((2, 0, 3, 64), device="cuda", dtype=torch.bfloat16)
    y = torch.empty((2, 0, 3, 64), device="cuda")
    wkv.rwkv7_wkv_prefill(e, e, e, e, e, e, s_in, y, s_out)
    torch.cuda.synchronize()
    assert torch.equal(s_in, s_out)
    wkv.rwkv7_wkv_prefill(e, e, e, e, e, e, None, y, s_out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(s_out).item() == 0


def test_deterministic(torch):
    say("determinism")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=300, H=6, seed=8)
    d = to_dev(x)
    y1, s1 = run_prefill(torch, d)
    y2, s2 = run_prefill(torch, d)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)
