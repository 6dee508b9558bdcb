"""The C ABI library loads, exports every declared symbol and rejects bad arguments (CPU only).

Every call here fails validation or has no work, so no HIP call is made.
"""
import ctypes
import os
import re
import subprocess

import pytest

from linear_rnn_amd import wkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rwkv7_wkv.h")

F32, BF16 = wkv.RWKV7_DTYPE_F32, wkv.RWKV7_DTYPE_BF16
OK, E_NULL, E_SHAPE, E_HEAD, E_DTYPE, E_ALIGN, E_ALIAS, E_ALGO = 0, -1, -2, -3, -4, -5, -6, -7


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(rwkv7_\w+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(wkv.LIB_PATH):
        pytest.skip("HIP library not built")
    return wkv.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(wkv.EXPORTED), names
    out = subprocess.run(["nm", "-D", "--defined-only", wkv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (rwkv7_\w+)", out))
    assert set(names) <= exported, (names, exported)


def test_strerror_never_null(L):
    for code in range(-12, 3):
        assert isinstance(wkv.rwkv7_wkv_strerror(code), str) and wkv.rwkv7_wkv_strerror(code)


# Fake device addresses: distinct, 16-byte aligned, far apart. Never dereferenced,
# because every call below is rejected or has no work.
BASE = 1 << 40
GAP = 1 << 34


def ptrs(n=9):
    return [BASE + i * GAP for i in range(n)]


def call(L, fn="rwkv7_wkv_prefill", p=None, B=2, T=3, H=4, N=64, dtype=BF16, algo=None, sdtype=None):
    p = ptrs() if p is None else p
    args = list(p) + [B, T, H, N, dtype]
    if fn == "rwkv7_wkv_prefill_ex":
        args.append(algo)
    if fn == "rwkv7_wkv_step_q":
        args.append(sdtype)
    args.append(None)
    return getattr(L, fn)(*args)


def test_bad_dtype(L):
    assert call(L, dtype=7) == E_DTYPE


@pytest.mark.parametrize("B,T,H", [(-1, 3, 4), (2, -1, 4), (2, 3, -4), (1 << 30, 1, 1 << 10), (1, 1 << 60, 1)])
def test_bad_shape(L, B, T, H):
    assert call(L, B=B, T=T, H=H) == E_SHAPE


@pytest.mark.parametrize("N", [0, 32, 63, 65, 128])
def test_head_size_must_be_64(L, N):
    assert call(L, N=N) == E_HEAD


@pytest.mark.parametrize("idx", range(8))
def test_null_required_pointer(L, idx):
    if idx == 6:  # state_in may be NULL
        return
    p = ptrs()
    p[idx] = None
    assert call(L, p=p) == E_NULL


@pytest.mark.parametrize("idx", range(9))
def test_misaligned_pointer(L, idx):
    p = ptrs()
    p[idx] += 4
    assert call(L, p=p) == E_ALIGN


def test_output_overlapping_input(L):
    p = ptrs()
    p[7] = p[2] + 64  # y inside k
    assert call(L, p=p) == E_ALIAS
    p = ptrs()
    p[8] = p[0]  # state_out on r
    assert call(L, p=p) == E_ALIAS
    p = ptrs()
    p[8] = p[7] + 256  # state_out inside y
    assert call(L, p=p) == E_ALIAS
    p = ptrs()
    p[8] = p[6] + 1024  # partial overlap of state_out and state_in
    assert call(L, p=p) == E_ALIAS
    p = ptrs()
    p[7] = p[6]  # y on state_in
    assert call(L, p=p) == E_ALIAS


def test_adjacent_buffers_are_not_alias(L):
    # y directly after k: touching but not overlapping; use B*H == 0 so nothing launches
    p = ptrs()
    assert call(L, p=p, B=0) == OK


def test_step_requires_one_token(L):
    assert call(L, fn="rwkv7_wkv_step", T=2) == E_SHAPE
    assert call(L, fn="rwkv7_wkv_step", T=0) == E_SHAPE


@pytest.mark.parametrize("algo", [-1, 4, 99])
def test_unknown_algo(L, algo):
    assert call(L, fn="rwkv7_wkv_prefill_ex", algo=algo) == E_ALGO


def test_empty_work_is_ok_without_device(L):
    assert call(L, B=0) == OK
    assert call(L, H=0) == OK
    p = ptrs()
    p[8] = None  # T == 0 with no state_out: nothing to do
    assert call(L, p=p, T=0) == OK
    p = ptrs()
    p[8] = p[6]  # T == 0, state_out == state_in: nothing to copy
    assert call(L, p=p, T=0) == OK
    # zero-element tensors may be NULL
    p = [None] * 9
    assert call(L, p=p, B=0) == OK


def test_binding_error_message(L):
    with pytest.raises(wkv.Rwkv7Error) as ei:
        wkv._check(E_HEAD)
    assert "64" in str(ei.value) and ei.value.status == E_HEAD


@pytest.mark.parametrize("sdtype", [-1, 3, 7])
def test_step_q_rejects_unknown_state_dtype(L, sdtype):
    assert call(L, fn="rwkv7_wkv_step_q", T=1, sdtype=sdtype) == E_DTYPE


@pytest.mark.parametrize("sdtype", [wkv.RWKV7_STATE_F32, wkv.RWKV7_STATE_BF16, wkv.RWKV7_STATE_F16])
def test_step_q_validation(L, sdtype):
    assert call(L, fn="rwkv7_wkv_step_q", T=2, sdtype=sdtype) == E_SHAPE
    assert call(L, fn="rwkv7_wkv_step_q", T=1, N=32, sdtype=sdtype) == E_HEAD
    assert call(L, fn="rwkv7_wkv_step_q", T=1, B=0, sdtype=sdtype) == OK
    p = ptrs()
    p[6] += 8  # 8-byte aligned state_in
    assert call(L, fn="rwkv7_wkv_step_q", p=p, T=1, sdtype=sdtype) == E_ALIGN


def test_step_q_alias_uses_16_bit_state_size(L):
    """state_out starting half-way into a 16-bit state_in overlaps it (rejected before any launch)."""
    B, H = 2, 4
    st16 = B * H * 64 * 64 * 2
    p = ptrs()
    p[8] = p[6] + st16 // 2
    assert call(L, fn="rwkv7_wkv_step_q", p=p, T=1, B=B, H=H, sdtype=wkv.RWKV7_STATE_BF16) == E_ALIAS
    p[8] = p[6] + st16 - 16
    assert call(L, fn="rwkv7_wkv_step_q", p=p, T=1, B=B, H=H, sdtype=wkv.RWKV7_STATE_F16) == E_ALIAS


def test_chunked_refuses_f32_inputs_before_any_launch(L):
    assert call(L, fn="rwkv7_wkv_prefill_ex", dtype=F32, algo=wkv.RWKV7_ALGO_CHUNKED) == E_ALGO
    assert call(L, fn="rwkv7_wkv_prefill_ex", dtype=F32, algo=wkv.RWKV7_ALGO_CHUNKED_SPLIT) == E_ALGO


# ---- the fused time-mix entry points: r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out

def tcall(L, fn="rwkv7_tmix_prefill", p=None, B=2, T=3, H=4, N=64, dtype=BF16):
    p = ptrs(11) if p is None else p
    return getattr(L, fn)(*(list(p) + [B, T, H, N, dtype, None]))


def test_tmix_validation(L):
    assert tcall(L, dtype=5) == E_DTYPE
    assert tcall(L, N=32) == E_HEAD
    assert tcall(L, B=-1) == E_SHAPE
    assert tcall(L, fn="rwkv7_tmix_step", T=2) == E_SHAPE
    for i in (0, 1, 2, 3, 4, 5, 9):  # r, w_raw, k, v, kk, a_lr, out are required
        p = ptrs(11)
        p[i] = None
        assert tcall(L, p=p) == E_NULL, i
    for i in range(11):
        p = ptrs(11)
        p[i] += 4
        assert tcall(L, p=p) == E_ALIGN, i


def test_tmix_aliasing(L):
    p = ptrs(11)
    p[9] = p[4]  # out over kk
    assert tcall(L, p=p) == E_ALIAS
    p = ptrs(11)
    p[10] = p[1]  # state_out over w_raw
    assert tcall(L, p=p) == E_ALIAS
    p = ptrs(11)
    p[9] = p[6]  # out over ln_w
    assert tcall(L, p=p) == E_ALIAS
    p = ptrs(11)
    p[10] = p[8]  # state_out == state_in is allowed; with no work nothing launches
    assert tcall(L, p=p, B=0) == OK


def test_tmix_prefill_ex_algorithms(L):
    """AUTO and SEQUENTIAL, or CHUNKED / CHUNKED_SPLIT with bfloat16 inputs; everything else is refused
    before any launch."""
    def xcall(algo, dtype=BF16, B=2):
        return L.rwkv7_tmix_prefill_ex(*(list(ptrs(11)) + [B, 3, 4, 64, dtype, algo, None]))
    assert xcall(wkv.RWKV7_ALGO_CHUNKED_SPLIT, dtype=F32) == E_ALGO
    assert xcall(wkv.RWKV7_ALGO_CHUNKED, dtype=F32) == E_ALGO
    for algo in (4, -1):
        assert xcall(algo) == E_ALGO, algo
    for algo in (wkv.RWKV7_ALGO_AUTO, wkv.RWKV7_ALGO_SEQUENTIAL, wkv.RWKV7_ALGO_CHUNKED,
                 wkv.RWKV7_ALGO_CHUNKED_SPLIT):
        assert xcall(algo, B=0) == OK, algo
    assert xcall(wkv.RWKV7_ALGO_AUTO, dtype=7) == E_DTYPE


def test_tmix_empty(L):
    assert tcall(L, B=0) == OK and tcall(L, H=0) == OK
    p = ptrs(11)
    p[6] = p[7] = None  # ln_w / ln_b optional
    assert tcall(L, p=p, B=0) == OK


# ---- the backward: r, w, k, v, a, b, state_in, dy, dstate_out, dr, dw, dk, dv, da, db, dstate_in

def bcall(L, p=None, B=2, T=3, H=4, N=64, dtype=BF16):
    p = ptrs(16) if p is None else p
    return L.rwkv7_wkv_backward(*(list(p) + [B, T, H, N, dtype, None]))


def test_backward_validation(L):
    assert bcall(L, dtype=3) == E_DTYPE
    assert bcall(L, N=128) == E_HEAD
    assert bcall(L, T=-2) == E_SHAPE
    for i in (0, 1, 2, 3, 4, 5, 7, 9, 10, 11, 12, 13, 14):  # inputs, dy and the six gradients are required
        p = ptrs(16)
        p[i] = None
        assert bcall(L, p=p) == E_NULL, i
    for i in range(16):
        p = ptrs(16)
        p[i] += 8
        assert bcall(L, p=p) == E_ALIGN, i


def test_backward_aliasing(L):
    for d in range(9, 16):  # each output over each input
        for s in range(9):
            p = ptrs(16)
            p[d] = p[s]
            if d == 15 and s == 8:
                continue  # dstate_in == dstate_out is allowed
            assert bcall(L, p=p) == E_ALIAS, (d, s)
    p = ptrs(16)
    p[12] = p[10] + 256  # dv inside dw
    assert bcall(L, p=p) == E_ALIAS
    p = ptrs(16)
    p[15] = p[8] + 1024  # partial overlap of dstate_in and dstate_out
    assert bcall(L, p=p) == E_ALIAS
    p = ptrs(16)
    p[15] = p[8]
    assert bcall(L, p=p, B=0) == OK


def test_backward_empty(L):
    assert bcall(L, B=0) == OK and bcall(L, H=0) == OK
    p = ptrs(16)
    p[6] = p[8] = p[15] = None  # optional states, T == 0: nothing to copy
    assert bcall(L, p=p, T=0) == OK
    assert bcall(L, p=[None] * 16, B=0) == OK


# ---- the layer stack: w_in, w_out, vecs, x, states

def scall(L_, p=None, n_layers=2, B=2, T=3, H=4, N=64, dtype=BF16):
    p = ptrs(5) if p is None else p
    return L_.rwkv7_stack_forward(*(list(p) + [n_layers, B, T, H, N, dtype, None]))


def test_stack_validation(L):
    assert scall(L, dtype=9) == E_DTYPE
    assert scall(L, N=16) == E_HEAD
    assert scall(L, n_layers=-1) == E_SHAPE
    assert scall(L, B=1 << 16, T=1 << 16) == E_SHAPE  # B*T rows beyond the GEMM library's 32-bit sizes
    for i in range(5):
        p = ptrs(5)
        p[i] = None
        assert scall(L, p=p) == E_NULL, i
        p = ptrs(5)
        p[i] += 4
        assert scall(L, p=p) == E_ALIGN, i
    p = ptrs(5)
    p[3] = p[0]  # x over w_in
    assert scall(L, p=p) == E_ALIAS
    p = ptrs(5)
    p[4] = p[3] + 64  # states inside x
    assert scall(L, p=p) == E_ALIAS
    assert scall(L, n_layers=0) == OK and scall(L, T=0) == OK and scall(L, p=[None] * 5, B=0) == OK


# ---- the allocation-free prefill: refusals happen before any HIP call

def test_noalloc_refusals(L):
    def nc(p=None, B=2, T=3, H=4, dtype=BF16):
        p = ptrs() if p is None else p
        return L.rwkv7_wkv_prefill_noalloc(*(list(p) + [B, T, H, 64, dtype, None]))
    assert nc(dtype=F32) == E_ALGO               # bfloat16 inputs only, as the split algorithm
    assert nc(dtype=7) == E_DTYPE
    assert nc(B=0) == OK and nc(H=0) == OK      # no work
    # one chunk of records (9,472 bytes) per head must fit the 64 MiB array
    cap = wkv.RWKV7_NOALLOC_SCRATCH_BYTES
    too_many = cap // 9472 + 1
    assert nc(B=too_many, H=1) == wkv.RWKV7_ERR_SCRATCH
    # without state_out the carried state (16 KiB per head) must fit as well
    p = ptrs()
    p[8] = None
    heads = cap // (9472 + 16384) + 1
    assert nc(p=p, B=heads, H=1) == wkv.RWKV7_ERR_SCRATCH
    # the ordinary argument checks come first
    p = ptrs()
    p[7] = None
    assert nc(p=p) == E_NULL
    assert "static scratch" in wkv.rwkv7_wkv_strerror(wkv.RWKV7_ERR_SCRATCH)


def _device_cus():
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.get_device_properties(0).multi_processor_count
    except Exception:
        pass
    return 256  # the library's assumption when no device can be queried


@pytest.mark.parametrize("B,T,H", [(8, 4096, 12), (8, 1024, 12), (4, 16384, 64), (16, 4096, 16), (16, 1024, 16),
                                   (1, 4096, 8), (8, 2720, 12), (8, 2736, 12), (16, 288, 16), (16, 304, 16),
                                   (1, 16, 1)])
def test_auto_prefill_rule(L, B, T, H):
    """AUTO: float32 and over-limit bfloat16 calls run sequentially; bfloat16 runs the one-kernel chunked
    prefill once B*H >= CUs * (0.3 + 12.8 / ceil(T / 16)), else the split one."""
    cus = _device_cus()
    nc = -(-T // 16)
    want = wkv.RWKV7_ALGO_CHUNKED if B * H * nc * 10 >= cus * (3 * nc + 128) else wkv.RWKV7_ALGO_CHUNKED_SPLIT
    assert wkv.rwkv7_wkv_prefill_algo(B, T, H) == want
    assert wkv.rwkv7_wkv_prefill_algo(B, T, H, dtype=wkv.RWKV7_DTYPE_F32) == wkv.RWKV7_ALGO_SEQUENTIAL


def test_auto_prefill_rule_at_256_cus(L):
    if _device_cus() != 256:
        pytest.skip("the fixed points below are for a 256-CU device")
    # the prompt shapes the rule was measured on
    assert wkv.rwkv7_wkv_prefill_algo(8, 1024, 12) == wkv.RWKV7_ALGO_CHUNKED_SPLIT
    assert wkv.rwkv7_wkv_prefill_algo(8, 4096, 12) == wkv.RWKV7_ALGO_CHUNKED
    assert wkv.rwkv7_wkv_prefill_algo(4, 16384, 64) == wkv.RWKV7_ALGO_CHUNKED
    # 32-bit element offsets inside a sequence: T*H*64 must stay below 2^31
    assert wkv.rwkv7_wkv_prefill_algo(1, 1 << 22, 8) == wkv.RWKV7_ALGO_SEQUENTIAL
    assert wkv.rwkv7_wkv_prefill_algo(1, (1 << 22) - 16, 8) != wkv.RWKV7_ALGO_SEQUENTIAL
