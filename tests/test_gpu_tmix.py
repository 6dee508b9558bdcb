"""GPU parity of the fused time-mix operator (prologue, recurrence, ln_x) against the float64 oracle."""
import numpy as np
import pytest

import oracle
from linear_rnn_amd import wkv
from linear_rnn_amd.inputs import CONFIGS, make_tmix_inputs
from tests.gpu_util import TOL_BF16, TOL_F32, rel, sample_units, say

pytestmark = pytest.mark.gpu
NAMES = ("r", "w_raw", "k", "v", "kk", "a_lr")


@pytest.fixture(scope="module")
def torch():
    import torch as t
    wkv.lib()
    oracle.build(force=False)
    return t


def dev(torch, x):
    out = {}
    for n, a in x.items():
        if a is None:
            out[n] = None
        elif a.dtype == np.uint16:
            out[n] = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            out[n] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return out


def run(torch, d, state=True, affine=True):
    o, s = wkv.tmix(*(d[n] for n in NAMES), d["ln_w"] if affine else None, d["ln_b"] if affine else None,
                    d["state_in"] if state else None)
    torch.cuda.synchronize()
    return o.cpu().numpy(), s.cpu().numpy()


def ref(x, state=True, affine=True):
    return oracle.tmix(*(x[n] for n in NAMES), x["ln_w"] if affine else None, x["ln_b"] if affine else None,
                       x["state_in"] if state else None)


def test_f32_tiny(torch):
    say("tmix f32 tiny")
    x = make_tmix_inputs(CONFIGS["tiny-prefill-f32"])
    o, s = run(torch, dev(torch, x), state=False)
    orf, srf = ref(x, state=False)
    e = (rel(o, orf), rel(s, srf))
    say("tmix f32 errors", e)
    assert max(e) <= TOL_F32, e


@pytest.mark.parametrize("B,T,H", [(1, 1, 2), (2, 37, 3), (3, 100, 5), (1, 300, 12)])
def test_bf16_ragged(torch, B, T, H):
    say("tmix bf16", B, T, H)
    x = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=B, T=T, H=H, seed=400 + T)
    o, s = run(torch, dev(torch, x))
    orf, srf = ref(x)
    e = (rel(o, orf), rel(s, srf))
    assert max(e) <= TOL_BF16, e


def test_identity_affine_and_zero_key(torch):
    """ln_w / ln_b NULL mean weight 1 and bias 0; an all-zero removal key row gives a = b = 0."""
    say("tmix NULL affine, zero kk rows")
    x = make_tmix_inputs(CONFIGS["tiny-prefill-f32"], T=40, seed=9)
    x["kk"][0, 5:9] = 0.0
    o, s = run(torch, dev(torch, x), affine=False)
    orf, srf = ref(x, affine=False)
    assert np.all(np.isfinite(o))
    assert max(rel(o, orf), rel(s, srf)) <= TOL_F32


def test_extreme_decays(torch):
    """w_raw = -inf (w = 1), very large (w = 0) and ordinary values mixed."""
    say("tmix extreme decays")
    x = make_tmix_inputs(CONFIGS["tiny-prefill-f32"], T=50, seed=12, with_state=True)
    rng = np.random.default_rng(12)
    pick = rng.integers(0, 4, size=x["w_raw"].shape)
    x["w_raw"] = np.where(pick == 0, -np.inf, np.where(pick == 1, 30.0, x["w_raw"])).astype(np.float32)
    o, s = run(torch, dev(torch, x))
    orf, srf = ref(x)
    assert max(rel(o, orf), rel(s, srf)) <= TOL_F32


def test_steps_equal_prefill(torch):
    """T single-token steps reproduce a prefill over the T tokens bit for bit."""
    say("tmix steps == prefill")
    x = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=2, T=21, H=3, seed=31)
    d = dev(torch, x)
    o1, s1 = run(torch, d)
    st = d["state_in"].clone()
    outs = []
    for t in range(21):
        sl = {n: d[n][:, t:t + 1].contiguous() for n in NAMES}
        o = torch.empty((2, 1, 3, 64), dtype=torch.float32, device="cuda")
        wkv.rwkv7_tmix_step(*(sl[n] for n in NAMES), d["ln_w"], d["ln_b"], st, o, st)
        outs.append(o)
    torch.cuda.synchronize()
    assert np.array_equal(torch.cat(outs, 1).cpu().numpy(), o1)
    assert np.array_equal(st.cpu().numpy(), s1)


def test_decode_shape_sampled(torch):
    """One fused step at the D2048 decode shape (B=512, H=32), sampled heads against the oracle."""
    cfg = CONFIGS["D2048-decode"]
    say("tmix decode shape", cfg)
    x = make_tmix_inputs(cfg, step=0)
    d = dev(torch, x)
    out = torch.empty((cfg.B, 1, cfg.H, 64), dtype=torch.float32, device="cuda")
    st = d["state_in"].clone()
    wkv.rwkv7_tmix_step(*(d[n] for n in NAMES), d["ln_w"], d["ln_b"], st, out, st)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    s = st.cpu().numpy()
    for (b, h) in sample_units(cfg.B, cfg.H, 24, seed=3):
        xs = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in NAMES}
        xs["ln_w"] = np.ascontiguousarray(x["ln_w"][h * 64:(h + 1) * 64])
        xs["ln_b"] = np.ascontiguousarray(x["ln_b"][h * 64:(h + 1) * 64])
        xs["state_in"] = np.ascontiguousarray(x["state_in"][b:b + 1, h:h + 1])
        orf, srf = ref(xs)
        e = (rel(o[b, :, h], orf[0, :, 0]), rel(s[b, h], srf[0, 0]))
        assert max(e) <= TOL_BF16, ((b, h), e)


# ---- the chunked prefill of the fused operator (bfloat16 inputs): one kernel per head
# (RWKV7_ALGO_CHUNKED) and split prep / scan kernels (RWKV7_ALGO_CHUNKED_SPLIT)

CH_VARIANTS = {"fused": wkv.RWKV7_ALGO_CHUNKED, "split": wkv.RWKV7_ALGO_CHUNKED_SPLIT}


@pytest.fixture(params=sorted(CH_VARIANTS), scope="module")
def CH(request):
    return CH_VARIANTS[request.param]


def run_ch(torch, d, state=True, affine=True, algo=None):
    o, s = wkv.tmix(*(d[n] for n in NAMES), d["ln_w"] if affine else None, d["ln_b"] if affine else None,
                    d["state_in"] if state else None, algo=algo)
    torch.cuda.synchronize()
    return o.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("B,T,H", [(1, 2, 1), (1, 17, 2), (2, 37, 3), (3, 100, 5), (1, 300, 12), (2, 1000, 4)])
def test_chunked_vs_oracle(torch, CH, B, T, H):
    say("tmix chunked", CH, B, T, H)
    x = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=B, T=T, H=H, seed=500 + T)
    o, s = run_ch(torch, dev(torch, x), algo=CH)
    orf, srf = ref(x)
    e = (rel(o, orf), rel(s, srf))
    say("tmix chunked errors", e)
    assert max(e) <= TOL_BF16, e


def test_chunked_zero_state_null_affine_zero_key(torch, CH):
    """state_in NULL, ln_w / ln_b NULL, and all-zero removal-key rows (a = b = 0) on the chunked path."""
    say("tmix chunked, NULL state and affine, zero kk rows", CH)
    x = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=2, T=70, H=3, seed=41)
    x["kk"][1, 20:36] = 0
    o, s = run_ch(torch, dev(torch, x), state=False, affine=False, algo=CH)
    orf, srf = ref(x, state=False, affine=False)
    assert np.all(np.isfinite(o))
    assert max(rel(o, orf), rel(s, srf)) <= TOL_BF16


def test_chunked_state_in_place_and_sequential_agree(torch, CH):
    """state_out == state_in on the chunked path; the chunked and the token-by-token prefill agree to the
    bfloat16 tolerance."""
    say("tmix chunked in place vs sequential", CH)
    x = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=2, T=333, H=4, seed=43)
    d = dev(torch, x)
    st = d["state_in"].clone()
    out = torch.empty((2, 333, 4, 64), dtype=torch.float32, device="cuda")
    wkv.rwkv7_tmix_prefill_ex(*(d[n] for n in NAMES), d["ln_w"], d["ln_b"], st, out, st, algo=CH)
    o_seq, s_seq = run_ch(torch, d, algo=wkv.RWKV7_ALGO_SEQUENTIAL)
    torch.cuda.synchronize()
    o_ch, s_ch = out.cpu().numpy(), st.cpu().numpy()
    assert max(rel(o_ch, o_seq), rel(s_ch, s_seq)) <= TOL_BF16
    orf, srf = ref(x)
    assert max(rel(o_ch, orf), rel(s_ch, srf)) <= TOL_BF16


def test_chunked_extreme_decays(torch, CH):
    """w_raw = -inf (w = 1), 30 (w = 0, which the chunked path clamps to 2^-15) and ordinary values."""
    say("tmix chunked extreme decays", CH)
    x = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=1, T=90, H=2, seed=45, with_state=True)
    rng = np.random.default_rng(45)
    pick = rng.integers(0, 4, size=x["w_raw"].shape)
    x["w_raw"] = np.where(pick == 0, -np.inf, np.where(pick == 1, 30.0, x["w_raw"])).astype(np.float32)
    o, s = run_ch(torch, dev(torch, x), algo=CH)
    orf, srf = ref(x)
    assert max(rel(o, orf), rel(s, srf)) <= TOL_BF16


def test_chunked_refuses_f32_and_unknown_algos(torch):
    x = make_tmix_inputs(CONFIGS["tiny-prefill-f32"], T=8, seed=2)
    d = dev(torch, x)
    for algo in CH_VARIANTS.values():
        with pytest.raises(wkv.Rwkv7Error) as ei:
            run_ch(torch, d, algo=algo)
        assert ei.value.status == -7
    xb = make_tmix_inputs(CONFIGS["L12-D768-prefill"], B=1, T=8, H=1, seed=2)
    for algo in (9, -1):
        with pytest.raises(wkv.Rwkv7Error) as ei:
            run_ch(torch, dev(torch, xb), algo=algo)
        assert ei.value.status == -7
