"""The Python binding checks every tensor before it calls the library (no GPU needed).

The C ABI receives bare pointers and cannot see a buffer's size, layout or device, so a
short output, a strided input or a mixed input dtype must be refused in the binding,
before any library call. The library loader is replaced by one that fails the test if
it is reached."""
import pytest
import torch

from linear_rnn_amd import wkv

B, T, H, N = 2, 5, 3, 64


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def forbidden():
        raise AssertionError("the library was called before the arguments were checked")
    monkeypatch.setattr(wkv, "lib", forbidden)


def inputs(dtype=torch.bfloat16):
    return [torch.zeros((B, T, H, N), dtype=dtype) for _ in range(6)]


def good():
    x = inputs()
    return x + [torch.zeros((B, H, N, N)), torch.zeros((B, T, H, N)), torch.zeros((B, H, N, N))]


def test_short_y_is_refused():
    a = good()
    a[7] = torch.zeros((B, T - 1, H, N))
    with pytest.raises(ValueError, match="y has shape"):
        wkv.rwkv7_wkv_prefill(*a)


def test_strided_input_is_refused():
    a = good()
    a[2] = torch.zeros((B, T, H, 2 * N), dtype=torch.bfloat16)[..., ::2]
    with pytest.raises(ValueError, match="k must be contiguous"):
        wkv.rwkv7_wkv_prefill_ex(*a)


def test_mixed_dtype_w_is_refused():
    a = good()
    a[1] = torch.zeros((B, T, H, N), dtype=torch.float32)
    with pytest.raises(ValueError, match="w has dtype"):
        wkv.rwkv7_wkv_prefill(*a)


def test_state_shape_and_dtype_are_checked():
    a = good()
    a[6] = torch.zeros((B, H, N, N - 1))
    with pytest.raises(ValueError, match="state_in has shape"):
        wkv.rwkv7_wkv_prefill(*a)
    a = good()
    a[8] = torch.zeros((B, H, N, N), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="state_out has dtype"):
        wkv.rwkv7_wkv_prefill(*a)


def test_step_q_state_dtype_follows_the_state():
    x = [torch.zeros((B, 1, H, N), dtype=torch.bfloat16) for _ in range(6)]
    s16 = torch.zeros((B, H, N, N), dtype=torch.float16)
    y = torch.zeros((B, 1, H, N))
    with pytest.raises(ValueError, match="state_in has dtype"):
        wkv.rwkv7_wkv_step_q(*x, s16, y, s16, state_dtype=wkv.RWKV7_STATE_BF16)


def test_host_tensors_are_refused_last():
    """Correct sizes on the host: refused for the device, by name."""
    with pytest.raises(ValueError, match="HIP device"):
        wkv.rwkv7_wkv_prefill(*good())


def test_tmix_checks():
    r, k, v, kk, alr = (torch.zeros((B, T, H, N), dtype=torch.bfloat16) for _ in range(5))
    w_raw = torch.zeros((B, T, H, N))
    out = torch.zeros((B, T, H, N))
    with pytest.raises(ValueError, match="ln_w has shape"):
        wkv.rwkv7_tmix_prefill(r, w_raw, k, v, kk, alr, torch.zeros(H * N - 1), None, None, out, None)
    with pytest.raises(ValueError, match="w_raw has dtype"):
        wkv.rwkv7_tmix_prefill(r, w_raw.bfloat16(), k, v, kk, alr, None, None, None, out, None)
    with pytest.raises(ValueError, match="out has shape"):
        wkv.rwkv7_tmix_step(r, w_raw, k, v, kk, alr, None, None, None, out[:, :1], None)


def test_backward_checks():
    x = inputs()
    dy = torch.zeros((B, T, H, N))
    grads = [torch.zeros((B, T, H, N)) for _ in range(6)]
    grads[4] = torch.zeros((B, T, H, N + 1))
    with pytest.raises(ValueError, match="da has shape"):
        wkv.rwkv7_wkv_backward(*x, None, dy, None, *grads, None)
    grads[4] = torch.zeros((B, T, H, N))
    with pytest.raises(ValueError, match="dy has dtype"):
        wkv.rwkv7_wkv_backward(*x, None, dy.bfloat16(), None, *grads, None)


def test_stack_checks():
    L, D = 2, H * N
    states = torch.zeros((L, B, H, N, N))
    x = torch.zeros((B, T, D))
    w_in = torch.zeros((L, D, 5 * D), dtype=torch.bfloat16)
    w_out = torch.zeros((L, D, D), dtype=torch.bfloat16)
    vecs = torch.zeros((L, 5, D))
    with pytest.raises(ValueError, match="x has shape"):
        wkv.rwkv7_stack_forward(w_in, w_out, vecs, torch.zeros((B + 1, T, D)), states)
    with pytest.raises(ValueError, match="w_out has dtype"):
        wkv.rwkv7_stack_forward(w_in, w_out.float(), vecs, x, states)
    with pytest.raises(ValueError, match="HIP device"):
        wkv.rwkv7_stack_forward(w_in, w_out, vecs, x, states)
