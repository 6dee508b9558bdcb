"""GPU parity of the multi-layer stack (hybrid prompt-then-steps mode) against the float64 oracle."""
import numpy as np
import pytest

import oracle
from linear_rnn_amd import wkv
from linear_rnn_amd.inputs import make_stack_inputs
from tests.gpu_util import TOL_F32, rel, say

pytestmark = pytest.mark.gpu
# bfloat16 weights: x, o and the operator inputs are rounded to bfloat16 on both sides at the same
# points; a float32 sum that lands within float32 rounding of a bfloat16 tie rounds the other way on
# one side, moving that element by one bfloat16 unit (2^-8 relative), and such differences add up
# over layers. The bar is four units of 2^-8 of the tensor's largest magnitude.
TOL_STACK_BF16 = 4 * 2.0 ** -8


@pytest.fixture(scope="module")
def torch():
    import torch as t
    wkv.lib()
    oracle.build(force=False)
    return t


def dev(torch, z):
    out = {}
    for n, a in z.items():
        if a.dtype == np.uint16:
            out[n] = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            out[n] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return out


def gpu_run(torch, d, x=None, states=None):
    x = (d["x"] if x is None else x).clone()
    s = (d["states"] if states is None else states).clone()
    wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], x, s)
    torch.cuda.synchronize()
    return x, s


@pytest.mark.parametrize("dtype,L,B,T,H", [("f32", 3, 2, 37, 2), ("f32", 1, 1, 1, 1), ("bf16", 3, 2, 37, 2),
                                           ("bf16", 2, 3, 70, 3)])
def test_stack_vs_oracle(torch, dtype, L, B, T, H):
    say("stack", dtype, L, B, T, H)
    z = make_stack_inputs(L, B, T, H, dtype, seed=100 + T)
    x, s = gpu_run(torch, dev(torch, z))
    xr, sr = oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"], z["states"], dtype)
    e = (rel(x.cpu().numpy(), xr), rel(s.cpu().numpy(), sr))
    say("stack errors", e)
    assert max(e) <= (TOL_F32 if dtype == "f32" else TOL_STACK_BF16), e


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prompt_then_steps(torch, dtype):
    """GPT mode then RNN mode: a 24-token prompt, then 8 single-token calls, against one 32-token call
    (GPU) and against the oracle."""
    say("stack prompt then steps", dtype)
    z = make_stack_inputs(3, 2, 32, 2, dtype, seed=7)
    d = dev(torch, z)
    x_all, s_all = gpu_run(torch, d)
    x0, s = gpu_run(torch, d, x=d["x"][:, :24].contiguous())
    xs = [x0]
    for t in range(24, 32):
        xt, s = gpu_run(torch, d, x=d["x"][:, t:t + 1].contiguous(), states=s)
        xs.append(xt)
    xcat = torch.cat(xs, dim=1).cpu().numpy()
    tol = TOL_F32 if dtype == "f32" else TOL_STACK_BF16
    assert rel(xcat, x_all.cpu().numpy()) <= tol and rel(s.cpu().numpy(), s_all.cpu().numpy()) <= tol
    xr, sr = oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"], z["states"], dtype)
    assert rel(xcat, xr) <= tol and rel(s.cpu().numpy(), sr) <= tol


def test_twelve_layers_model_width(torch):
    """The 0.1B shape's width and depth (L=12, D=768, H=12), bfloat16 weights."""
    say("stack L12-D768")
    z = make_stack_inputs(12, 2, 20, 12, "bf16", seed=12, with_state=False)
    x, s = gpu_run(torch, dev(torch, z))
    xr, sr = oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"], z["states"], "bf16")
    e = (rel(x.cpu().numpy(), xr), rel(s.cpu().numpy(), sr))
    say("stack L12 errors", e)
    assert max(e) <= TOL_STACK_BF16, e


def test_empty_and_zero_layers(torch):
    z = make_stack_inputs(2, 2, 0, 2, "f32", seed=1)
    d = dev(torch, z)
    x, s = gpu_run(torch, d)
    assert np.array_equal(s.cpu().numpy(), z["states"])


def test_step_in_a_hip_graph(torch):
    """A 3-layer single-token step captured in a HIP graph (after a warm-up call, so the workspace and
    the rocBLAS handle exist) and replayed several times, with eager calls in between, equals the
    same steps run eagerly."""
    say("stack step graph")
    z = make_stack_inputs(3, 4, 1, 2, "bf16", seed=21)
    d = dev(torch, z)
    xs = [torch.randn((4, 1, 128), dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(i))
          for i in range(4)]
    # eager reference: four consecutive steps
    s_ref = d["states"].clone()
    outs_ref = []
    for x in xs:
        xx = x.clone()
        wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], xx, s_ref)
        outs_ref.append(xx)
    torch.cuda.synchronize()
    # graph: static input / state buffers
    x_buf = torch.zeros((4, 1, 128), dtype=torch.float32, device="cuda")
    s_buf = d["states"].clone()
    s_warm = d["states"].clone()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        # warm-up on the capture stream: the workspace and the rocBLAS handle are per stream
        wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], x_buf.clone(), s_warm)
        st.synchronize()
        with torch.cuda.graph(g, stream=st):
            wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], x_buf, s_buf)
    torch.cuda.synchronize()
    s_buf.copy_(d["states"])
    for i, x in enumerate(xs):
        x_buf.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x_buf, outs_ref[i]), i
        # unrelated eager work between replays
        tmp = torch.empty_like(x_buf)
        wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], tmp.copy_(x), s_warm)
        torch.cuda.synchronize()
    assert torch.equal(s_buf, s_ref)


def test_graph_survives_workspace_growth(torch):
    """A step captured in a graph keeps working after a larger eager call on the same stream has grown
    the per-stream workspace: the buffer the graph holds is retired, not freed."""
    say("stack step graph, then a larger eager prompt on the capture stream, then replays")
    z = make_stack_inputs(2, 4, 1, 2, "bf16", seed=23)
    d = dev(torch, z)
    xs = [torch.randn((4, 1, 128), dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(i))
          for i in range(3)]
    s_ref = d["states"].clone()
    outs_ref = []
    for x in xs:
        xx = x.clone()
        wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], xx, s_ref)
        outs_ref.append(xx)
    torch.cuda.synchronize()
    x_buf = torch.zeros((4, 1, 128), dtype=torch.float32, device="cuda")
    s_buf = d["states"].clone()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], x_buf.clone(), d["states"].clone())
        st.synchronize()
        with torch.cuda.graph(g, stream=st):
            wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], x_buf, s_buf)
        # a 300-token prompt (chunked operator, far larger intermediates) on the capture stream
        zp = make_stack_inputs(2, 4, 300, 2, "bf16", seed=24, with_state=False)
        xp = torch.from_numpy(zp["x"]).cuda()
        sp = torch.zeros_like(d["states"])
        wkv.rwkv7_stack_forward(d["w_in"], d["w_out"], d["vecs"], xp, sp)
        st.synchronize()
    torch.cuda.synchronize()
    assert torch.isfinite(xp).all()
    s_buf.copy_(d["states"])
    for i, x in enumerate(xs):
        x_buf.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x_buf, outs_ref[i]), i
    assert torch.equal(s_buf, s_ref)
