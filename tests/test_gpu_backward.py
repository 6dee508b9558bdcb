"""GPU parity of the backward (reverse-mode derivatives of the recurrence) against the float64 oracle.

Both algorithms: the checkpointed token-by-token reverse pass (float32 throughout, every dtype) and
the chunked one on MFMA (bfloat16 inputs; float16 operands inside a chunk, so the bfloat16 bar
applies, within the documented decay domain)."""
import numpy as np
import pytest

import oracle
from linear_rnn_amd import wkv
from linear_rnn_amd.inputs import CONFIGS, f32_to_bf16_bits, make_cotangents, make_inputs
from tests.gpu_util import TOL_BF16, TOL_F32, rel, sample_units, say, to_dev

pytestmark = pytest.mark.gpu
GRADS = ("dr", "dw", "dk", "dv", "da", "db")
SEQ, CHK = wkv.RWKV7_ALGO_SEQUENTIAL, wkv.RWKV7_ALGO_CHUNKED


@pytest.fixture(scope="module")
def torch():
    import torch as t
    wkv.lib()
    oracle.build(force=False)
    return t


def run(torch, x, ct, state=True, dstate=True, algo=wkv.RWKV7_ALGO_AUTO):
    d = to_dev(x)
    dy = torch.from_numpy(ct["dy"]).cuda()
    ds = torch.from_numpy(ct["dstate_out"]).cuda() if dstate and ct["dstate_out"] is not None else None
    g = wkv.wkv7_backward(*(d[n] for n in "rwkvab"), dy, d["state_in"] if state else None, ds, algo=algo)
    torch.cuda.synchronize()
    return {n: v.cpu().numpy() for n, v in g.items()}


def ref(x, ct, state=True, dstate=True):
    return oracle.wkv7_backward(*(x[n] for n in "rwkvab"), ct["dy"], state_in=x["state_in"] if state else None,
                                dstate_out=ct["dstate_out"] if dstate else None)


def errors(g, r):
    return {n: rel(g[n], r[n]) for n in GRADS + ("dstate_in",)}


def test_f32_tiny(torch):
    say("backward f32 tiny")
    x = make_inputs(CONFIGS["tiny-prefill-f32"])
    ct = make_cotangents(1, 64, 2, seed=1, with_dstate=False)
    e = errors(run(torch, x, ct, dstate=False), ref(x, ct, dstate=False))
    say("backward f32 tiny errors", e)
    assert max(e.values()) <= TOL_F32, e


@pytest.mark.parametrize("T", [1, 7, 8, 9, 15, 16, 17, 33, 100])
def test_f32_ragged_with_states(torch, T):
    """Every segment and sub-block tail, with state_in and dstate_out."""
    say("backward f32 T", T)
    x = make_inputs(CONFIGS["tiny-prefill-f32"], B=2, T=T, H=3, seed=500 + T, with_state=True)
    ct = make_cotangents(2, T, 3, seed=T)
    e = errors(run(torch, x, ct), ref(x, ct))
    assert max(e.values()) <= TOL_F32, e


@pytest.mark.parametrize("algo", [SEQ, CHK])
@pytest.mark.parametrize("B,T,H", [(1, 5, 1), (2, 64, 3), (3, 250, 4)])
def test_bf16(torch, B, T, H, algo):
    say("backward bf16", B, T, H, "algo", algo)
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=B, T=T, H=H, seed=600 + T)
    ct = make_cotangents(B, T, H, seed=T + 1)
    e = errors(run(torch, x, ct, algo=algo), ref(x, ct))
    say("backward bf16 errors", e)
    assert max(e.values()) <= TOL_BF16, e


@pytest.mark.parametrize("T", [1, 9, 15, 16, 17, 33, 100, 161])
def test_chunked_ragged_with_states(torch, T):
    """Every ragged tail of the last chunk, fewer chunks than the chain's prep waves and more
    than its ring (161 tokens: 11 chunks), with state_in and dstate_out."""
    say("backward chunked T", T)
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=T, H=3, seed=700 + T, with_state=True)
    ct = make_cotangents(2, T, 3, seed=T + 7)
    e = errors(run(torch, x, ct, algo=CHK), ref(x, ct))
    say("backward chunked errors", e)
    assert max(e.values()) <= TOL_BF16, e
    # without state_in and dstate_out
    e = errors(run(torch, x, ct, state=False, dstate=False, algo=CHK), ref(x, ct, state=False, dstate=False))
    assert max(e.values()) <= TOL_BF16, e


def test_chunked_decay_domain(torch):
    """Decays at the edge of the chunked domain (products of eight consecutive decays above 2^-15):
    w in {0.3, 0.55, 0.99, 1}, exact zero a / b rows, long-context slots."""
    say("backward chunked decay domain")
    x = make_inputs(CONFIGS["D4096-long-prefill"], B=1, T=70, H=3, seed=22)
    rng = np.random.default_rng(22)
    choices = np.array([0.3, 0.55, 0.99, 1.0], dtype=np.float32)
    x["w"] = f32_to_bf16_bits(choices[rng.integers(0, 4, size=x["w"].shape)])
    x["a"][0, 10:14] = 0
    x["b"][0, 30:33] = 0
    ct = make_cotangents(1, 70, 3, seed=22)
    e = errors(run(torch, x, ct, algo=CHK), ref(x, ct))
    say("backward chunked domain errors", e)
    assert max(e.values()) <= TOL_BF16, e


def test_auto_picks_chunked_for_bf16_and_sequential_for_f32(torch):
    say("backward AUTO")
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=1, T=50, H=2, seed=41)
    ct = make_cotangents(1, 50, 2, seed=41)
    ga, gc = run(torch, x, ct), run(torch, x, ct, algo=CHK)
    assert all(np.array_equal(ga[n], gc[n]) for n in ga)
    x = make_inputs(CONFIGS["tiny-prefill-f32"], B=1, T=50, H=2, seed=42, with_state=True)
    ga, gs = run(torch, x, ct), run(torch, x, ct, algo=SEQ)
    assert all(np.array_equal(ga[n], gs[n]) for n in ga)


def test_chunked_refuses_f32(torch):
    x = make_inputs(CONFIGS["tiny-prefill-f32"], B=1, T=20, H=1, seed=43)
    ct = make_cotangents(1, 20, 1, seed=43)
    with pytest.raises(RuntimeError):
        run(torch, x, ct, algo=CHK)


@pytest.mark.parametrize("algo", [SEQ, CHK])
def test_many_heads_single_row_block(torch, algo):
    """More than 128 heads: one workgroup per head (no row split), all rows' column sums in LDS."""
    say("backward 140 heads", algo)
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=21, H=70, seed=77)
    ct = make_cotangents(2, 21, 70, seed=77)
    e = errors(run(torch, x, ct, algo=algo), ref(x, ct))
    assert max(e.values()) <= TOL_BF16, e
    x = make_inputs(CONFIGS["tiny-prefill-f32"], B=2, T=13, H=70, seed=78, with_state=True)
    ct = make_cotangents(2, 13, 70, seed=78)
    e = errors(run(torch, x, ct), ref(x, ct))
    assert max(e.values()) <= TOL_F32, e


def test_zero_token_passes_state_gradient(torch):
    say("backward T == 0")
    x = make_inputs(CONFIGS["tiny-prefill-f32"], B=2, T=0, H=2, seed=3, with_state=True)
    ct = make_cotangents(2, 0, 2, seed=3)
    g = run(torch, x, ct)
    assert np.array_equal(g["dstate_in"], ct["dstate_out"])
    assert all(g[n].shape == (2, 0, 2, 64) for n in GRADS)
    g = run(torch, x, ct, dstate=False)
    assert not np.any(g["dstate_in"])


@pytest.mark.parametrize("algo", [SEQ, CHK])
def test_dstate_in_place_bf16(torch, algo):
    """dstate_in may be the dstate_out buffer itself (the chain reads it before it writes)."""
    say("backward bf16 dstate in place", algo)
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=1, T=40, H=2, seed=9, with_state=True)
    ct = make_cotangents(1, 40, 2, seed=9)
    d = to_dev(x)
    dy = torch.from_numpy(ct["dy"]).cuda()
    ds = torch.from_numpy(ct["dstate_out"]).cuda()
    outs = [torch.empty((1, 40, 2, 64), dtype=torch.float32, device="cuda") for _ in GRADS]
    wkv.rwkv7_wkv_backward_ex(*(d[n] for n in "rwkvab"), d["state_in"], dy, ds, *outs, ds, algo=algo)
    torch.cuda.synchronize()
    r = ref(x, ct)
    assert rel(ds.cpu().numpy(), r["dstate_in"]) <= TOL_BF16
    assert max(rel(o.cpu().numpy(), r[n]) for o, n in zip(outs, GRADS)) <= TOL_BF16


def test_dstate_in_place(torch):
    """dstate_in may be the dstate_out buffer itself."""
    say("backward dstate in place")
    x = make_inputs(CONFIGS["tiny-prefill-f32"], B=1, T=40, H=2, seed=8, with_state=True)
    ct = make_cotangents(1, 40, 2, seed=8)
    d = to_dev(x)
    dy = torch.from_numpy(ct["dy"]).cuda()
    ds = torch.from_numpy(ct["dstate_out"]).cuda()
    outs = [torch.empty((1, 40, 2, 64), dtype=torch.float32, device="cuda") for _ in GRADS]
    wkv.rwkv7_wkv_backward(*(d[n] for n in "rwkvab"), d["state_in"], dy, ds, *outs, ds)
    torch.cuda.synchronize()
    r = ref(x, ct)
    assert rel(ds.cpu().numpy(), r["dstate_in"]) <= TOL_F32
    assert max(rel(o.cpu().numpy(), r[n]) for o, n in zip(outs, GRADS)) <= TOL_F32


def test_extreme_decays_and_slots(torch):
    """w in {0, tiny, 1}, exact zero a/b rows and a_lr of exactly 0 or 1 (the token-by-token
    algorithm: decays this small are outside the chunked domain)."""
    say("backward extreme decays")
    x = make_inputs(CONFIGS["D4096-long-prefill"], B=1, T=70, H=3, seed=21)
    rng = np.random.default_rng(21)
    choices = np.array([0.0, 1e-6, 0.5, 1.0], dtype=np.float32)
    x["w"] = f32_to_bf16_bits(choices[rng.integers(0, 4, size=x["w"].shape)])
    x["a"][0, 10:14] = 0
    x["b"][0, 30:33] = 0
    ct = make_cotangents(1, 70, 3, seed=21)
    e = errors(run(torch, x, ct, algo=SEQ), ref(x, ct))
    assert max(e.values()) <= TOL_BF16, e


@pytest.mark.parametrize("algo", [SEQ, CHK])
def test_repeat_is_deterministic(torch, algo):
    say("backward determinism", algo)
    x = make_inputs(CONFIGS["L12-D768-prefill"], B=2, T=90, H=4, seed=31)
    ct = make_cotangents(2, 90, 4, seed=31)
    g1, g2 = run(torch, x, ct, algo=algo), run(torch, x, ct, algo=algo)
    assert all(np.array_equal(g1[n], g2[n]) for n in g1)


@pytest.mark.parametrize("name,algo", [("L12-D768-prefill", SEQ), ("L12-D768-prefill", CHK),
                                       ("L24-D1024-prefill-resume", CHK)])
def test_full_size_sampled(torch, name, algo):
    """Full layer shapes (bfloat16) against the oracle on sampled heads: the 0.1B-model prefill
    (B=8, T=4096, H=12) and, chunked, the 256-head L24-D1024 one (B=16, T=4096, H=16)."""
    cfg = CONFIGS[name]
    say("backward full size", cfg.name, "algo", algo)
    x = make_inputs(cfg)
    ct = make_cotangents(cfg.B, cfg.T, cfg.H, seed=cfg.seed)
    g = run(torch, x, ct, algo=algo)
    units = sample_units(cfg.B, cfg.H, 6, seed=5)
    worst = {}
    for (b, h) in units:
        sl = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in "rwkvab"}
        s_in = np.ascontiguousarray(x["state_in"][b:b + 1, h:h + 1])
        r = oracle.wkv7_backward(*(sl[n] for n in "rwkvab"), np.ascontiguousarray(ct["dy"][b:b + 1, :, h:h + 1]),
                                 state_in=s_in, dstate_out=np.ascontiguousarray(ct["dstate_out"][b:b + 1, h:h + 1]))
        for n in GRADS:
            worst[n] = max(worst.get(n, 0.0), rel(g[n][b:b + 1, :, h:h + 1], r[n]))
        worst["dstate_in"] = max(worst.get("dstate_in", 0.0), rel(g["dstate_in"][b:b + 1, h:h + 1], r["dstate_in"]))
    say("backward full size errors", worst)
    assert max(worst.values()) <= TOL_BF16, worst
    if algo == CHK and name == "L12-D768-prefill":
        # a second call at full size is bit-identical (the chunk pairs' LDS hand-off, at scale)
        g2 = run(torch, x, ct, algo=algo)
        assert all(np.array_equal(g[n], g2[n]) for n in g), [n for n in g if not np.array_equal(g[n], g2[n])]
