"""The allocation-free prefill (rwkv7_wkv_prefill_noalloc) against the entry point it is a variant
of (rwkv7_wkv_prefill_ex with the split chunked algorithm, whose records live in an allocated
workspace), through the C ABI: two calls in a row, the second with a smaller input; and a call
whose sequence needs several slabs of the static array, with and without state_out."""
import numpy as np
import pytest

import oracle
from linear_rnn_amd import wkv
from linear_rnn_amd.inputs import CONFIGS, make_inputs
from tests.gpu_util import TOL_BF16, rel, say, to_dev

pytestmark = pytest.mark.gpu
SPLIT = wkv.RWKV7_ALGO_CHUNKED_SPLIT


@pytest.fixture(scope="module")
def torch():
    import torch as t
    wkv.lib()
    return t


def both(torch, d, with_state_out=True):
    """(y, state) of the no-allocation call and of the workspace call on the same inputs."""
    B, T, H, N = d["r"].shape
    out = []
    for fn in ("noalloc", "ex"):
        y = torch.full((B, T, H, N), float("nan"), dtype=torch.float32, device="cuda")
        so = torch.full((B, H, N, N), float("nan"), dtype=torch.float32, device="cuda") if with_state_out else None
        args = (d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state_in"], y, so)
        if fn == "noalloc":
            wkv.rwkv7_wkv_prefill_noalloc(*args)
        else:
            wkv.rwkv7_wkv_prefill_ex(*args, algo=SPLIT)
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), None if so is None else so.cpu().numpy()))
    return out


def test_two_calls_in_a_row_second_smaller(torch):
    cfg = CONFIGS["L12-D768-prefill"]
    xs = [make_inputs(cfg, B=3, T=777, H=5, seed=71), make_inputs(cfg, B=1, T=45, H=2, seed=72)]
    for i, x in enumerate(xs):
        say("noalloc call", i, x["r"].shape)
        (yn, sn), (ye, se) = both(torch, to_dev(x))
        assert np.all(np.isfinite(yn)) and np.all(np.isfinite(sn))
        e = (rel(yn, ye), rel(sn, se))
        say("noalloc vs workspace", e, "identical" if np.array_equal(yn, ye) and np.array_equal(sn, se) else "")
        assert max(e) <= TOL_BF16, e
    # the smaller call also against the float64 oracle
    x = xs[1]
    yr, sr = oracle.wkv7(*(x[n] for n in "rwkvab"), state_in=x["state_in"])
    assert max(rel(yn, yr), rel(sn, sr)) <= TOL_BF16


@pytest.mark.parametrize("with_state_out", [True, False])
def test_several_slabs(torch, with_state_out):
    """256 heads: a slab of the 64 MiB array holds 27 chunks, so 1,000 tokens (63 chunks) take three
    slabs; without state_out the carried state also lives in the array."""
    cfg = CONFIGS["L12-D768-prefill"]
    x = make_inputs(cfg, B=4, T=1000, H=64, seed=73)
    say("noalloc several slabs, state_out", with_state_out)
    (yn, sn), (ye, se) = both(torch, to_dev(x), with_state_out)
    assert np.all(np.isfinite(yn))
    assert rel(yn, ye) <= TOL_BF16
    if with_state_out:
        assert rel(sn, se) <= TOL_BF16
