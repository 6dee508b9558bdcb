"""GPU parity of the multi-layer stack (hybrid prompt-then-steps mode) against the float64 oracle.

float32 weights: the whole stack against the oracle's float32 model, 1e-5.

bfloat16 weights: the model rounds x and o to bfloat16 where they enter a projection and the
operator's inputs to bfloat16 (the oracle's "bf16" reading). Two implementations of that model
differ wherever a value lands on the other side of a bfloat16 rounding boundary (one unit, 2^-8 of
that element), and every later layer re-rounds, so a difference that is harmless in one layer is
amplified by the layers after it (measured on these synthetic weights: the gap between the bfloat16
model and the same model in exact arithmetic grows from 3e-3 at one layer to 5e-2 at twelve). So the
bfloat16 stack is checked per layer, which isolates each layer's own error: every layer of the GPU
stack, fed the GPU's own input to that layer, must match the oracle's layer on that same input to the
operator's bar (2e-3, tests.gpu_util.TOL_BF16); the multi-layer call must equal that chain of
one-layer calls bit for bit; and end to end the GPU result must be as close to the exact-arithmetic
model (the oracle's "f64") as the oracle's own bfloat16 model is, within a factor of 2.
"""
import numpy as np
import pytest

import oracle
from linear_rnn_amd import wkv
from linear_rnn_amd.inputs import make_stack_inputs
from tests.gpu_util import TOL_BF16, TOL_F32, rel, say

pytestmark = pytest.mark.gpu


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


def layerwise(torch, z, d):
    """Each layer of the GPU stack as a one-layer call on the GPU's own input to it, against the
    oracle's layer on that same input. Returns (worst per-layer error, GPU x, GPU states)."""
    L = z["states"].shape[0]
    x = d["x"].clone()
    states = d["states"].clone()
    worst = 0.0
    for l in range(L):
        x_in = x.cpu().numpy()
        s_in = states[l:l + 1].cpu().numpy()
        s_l = states[l:l + 1]  # a view: updated in place
        wkv.rwkv7_stack_forward(d["w_in"][l:l + 1], d["w_out"][l:l + 1], d["vecs"][l:l + 1], x, s_l)
        torch.cuda.synchronize()
        xr, sr = oracle.stack_forward(z["w_in"][l:l + 1], z["w_out"][l:l + 1], z["vecs"][l:l + 1], x_in, s_in,
                                      "bf16")
        e = max(rel(x.cpu().numpy(), xr), rel(s_l.cpu().numpy(), sr))
        worst = max(worst, e)
    return worst, x, states


@pytest.mark.parametrize("L,B,T,H", [(3, 2, 37, 2), (1, 1, 1, 1)])
def test_stack_f32_vs_oracle(torch, L, B, T, H):
    say("stack f32", L, B, T, H)
    z = make_stack_inputs(L, B, T, H, "f32", seed=100 + T)
    x, s = gpu_run(torch, dev(torch, z))
    xr, sr = oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"], z["states"], "f32")
    e = (rel(x.cpu().numpy(), xr), rel(s.cpu().numpy(), sr))
    say("stack errors", e)
    assert max(e) <= TOL_F32, e


# T = 37 and 70 take the chunked operator (a bfloat16 call of 32 tokens or more), T = 20 and 1 the
# token-by-token one
@pytest.mark.parametrize("L,B,T,H", [(3, 2, 37, 2), (2, 3, 70, 3), (3, 2, 20, 2), (2, 1, 1, 1)])
def test_stack_bf16_layerwise(torch, L, B, T, H):
    say("stack bf16 layerwise", L, B, T, H)
    z = make_stack_inputs(L, B, T, H, "bf16", seed=100 + T)
    d = dev(torch, z)
    worst, xl, sl = layerwise(torch, z, d)
    say("stack bf16 worst per-layer error", worst)
    assert worst <= TOL_BF16, worst
    # the multi-layer call runs exactly that chain of one-layer calls
    x, s = gpu_run(torch, d)
    assert torch.equal(x, xl) and torch.equal(s, sl)


@pytest.mark.parametrize("L,B,T,H", [(3, 2, 37, 2), (2, 3, 70, 3)])
def test_stack_bf16_vs_exact_model(torch, L, B, T, H):
    """End to end against the model in exact arithmetic: no further from it than the oracle's own
    bfloat16 model is (factor 2)."""
    say("stack bf16 vs exact", L, B, T, H)
    z = make_stack_inputs(L, B, T, H, "bf16", seed=100 + T)
    x, s = gpu_run(torch, dev(torch, z))
    xe, se = oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"], z["states"], "f64")
    xb, sb = oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"], z["states"], "bf16")
    gap = max(rel(xb, xe), rel(sb, se))
    e = max(rel(x.cpu().numpy(), xe), rel(s.cpu().numpy(), se))
    say("stack bf16: GPU vs exact %.2e, oracle bf16 vs exact %.2e" % (e, gap))
    assert e <= 2 * gap, (e, gap)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prompt_then_steps(torch, dtype):
    """GPT mode then RNN mode: a 24-token prompt, then 8 single-token calls, against one 32-token call
    (GPU) and against the oracle. With bfloat16 weights the two runs take different operator paths
    (24 tokens and single tokens run token by token, 32 tokens chunked), so they are compared as two
    runs of the bfloat16 model: each no further from the exact-arithmetic model than the oracle's
    bfloat16 model is (factor 2)."""
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
    s = s.cpu().numpy()
    if dtype == "f32":
        assert rel(xcat, x_all.cpu().numpy()) <= TOL_F32 and rel(s, s_all.cpu().numpy()) <= TOL_F32
        xr, sr = oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"], z["states"], dtype)
        assert rel(xcat, xr) <= TOL_F32 and rel(s, sr) <= TOL_F32
        return
    xe, se = oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"], z["states"], "f64")
    xb, sb = oracle.stack_forward(z["w_in"], z["w_out"], z["vecs"], z["x"], z["states"], "bf16")
    gap = max(rel(xb, xe), rel(sb, se))
    for xx, ss in ((xcat, s), (x_all.cpu().numpy(), s_all.cpu().numpy())):
        assert max(rel(xx, xe), rel(ss, se)) <= 2 * gap


def test_twelve_layers_model_width(torch):
    """The 0.1B shape's width and depth (L=12, D=768, H=12), bfloat16 weights, layer by layer."""
    say("stack L12-D768")
    z = make_stack_inputs(12, 2, 20, 12, "bf16", seed=12, with_state=False)
    d = dev(torch, z)
    worst, xl, sl = layerwise(torch, z, d)
    say("stack L12 worst per-layer error", worst)
    assert worst <= TOL_BF16, worst
    x, s = gpu_run(torch, d)
    assert torch.equal(x, xl) and torch.equal(s, sl)


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
