"""Independent checks ("pins") of the float64 oracle, written from the mathematics.

Each function returns the worst relative deviation between the oracle and a
construction that does not share the oracle's loop structure. The tests in
test_oracle_pins.py assert on them, and test_oracle_mutants.py re-runs them on
deliberately broken copies of the oracle to show that each plausible mistake is
caught by at least one pin.

Recurrence being pinned (per batch and head; S is [value i, key j]):
    S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T,  y_t = S_t r_t
(RWKV-7 G0 7.2B notes, lshu.cn/news/198401, section 7.1; zero initial state per
section 3.3 of the same page).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from linear_rnn_amd.inputs import f32_to_bf16_bits, widen

N = 64


def rel(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.max(np.abs(ref)) if ref.size else 0.0
    d = np.max(np.abs(x - ref)) if ref.size else 0.0
    return float(d / m) if m > 0 else float(d)


def rand_inputs(rng, B, T, H, n=N, decay=(0.3, 1.0)):
    """Generic float64 inputs of moderate size (not the workload distributions)."""
    g = lambda *s: rng.standard_normal(s)  # noqa: E731
    return dict(
        r=g(B, T, H, n), k=g(B, T, H, n) / 4, v=g(B, T, H, n),
        a=g(B, T, H, n) / 8, b=g(B, T, H, n) / 8,
        w=rng.uniform(decay[0], decay[1], size=(B, T, H, n)),
        state_in=g(B, H, n, n) * 0.3,
    )


def call(orc, x, **kw):
    return orc.wkv7(x["r"], x["w"], x["k"], x["v"], x["a"], x["b"], state_in=x.get("state_in"), **kw)


# ---------------------------------------------------------------- brute force
def brute_force(x):
    """Explicit transition matrices M_t = diag(w_t) + a_t b_t^T and matrix products."""
    r, w, k, v, a, b = (widen(x[n]) if x[n].dtype != np.float64 else x[n] for n in "rwkvab")
    B, T, H, n = r.shape
    s0 = x.get("state_in")
    y = np.zeros((B, T, H, n))
    sT = np.zeros((B, H, n, n))
    for bb in range(B):
        for hh in range(H):
            S = np.zeros((n, n)) if s0 is None else np.array(s0[bb, hh], dtype=np.float64)
            for t in range(T):
                M = np.diag(w[bb, t, hh]) + np.outer(a[bb, t, hh], b[bb, t, hh])
                S = S @ M + np.outer(v[bb, t, hh], k[bb, t, hh])
                y[bb, t, hh] = S @ r[bb, t, hh]
            sT[bb, hh] = S
    return y, sT


def pin_brute_force(orc, seed=1, B=2, T=7, H=3):
    x = rand_inputs(np.random.default_rng(seed), B, T, H)
    y, s = call(orc, x)
    yb, sb = brute_force(x)
    return max(rel(y, yb), rel(s, sb))


# ---------------------------------------------------------------- closed forms
def decayed_linear_attention(x):
    """a = 0 (or b = 0): S_t = S_0 diag(prod_{u<=t} w_u) + sum_{s<=t} v_s (k_s * prod_{u=s+1..t} w_u)^T."""
    r, w, k, v = (x[n] for n in "rwkv")
    B, T, H, n = r.shape
    s0 = x["state_in"]
    y = np.zeros((B, T, H, n))
    sT = np.zeros((B, H, n, n))
    for bb in range(B):
        for hh in range(H):
            for t in range(T):
                S = s0[bb, hh] * np.prod(w[bb, :t + 1, hh], axis=0)[None, :]
                for s in range(t + 1):
                    dec = np.prod(w[bb, s + 1:t + 1, hh], axis=0) if s < t else np.ones(n)
                    S = S + np.outer(v[bb, s, hh], k[bb, s, hh] * dec)
                y[bb, t, hh] = S @ r[bb, t, hh]
                if t == T - 1:
                    sT[bb, hh] = S
    return y, sT


def pin_decayed_linear_attention(orc, seed=2, zero="a", B=1, T=12, H=2):
    x = rand_inputs(np.random.default_rng(seed), B, T, H)
    x[zero] = np.zeros_like(x[zero])
    y, s = call(orc, x)
    yc, sc = decayed_linear_attention(x)
    return max(rel(y, yc), rel(s, sc))


def pin_plain_linear_attention(orc, seed=3, B=2, T=40, H=2):
    """w = 1, a = 0: Y = tril(R K^T) V + R S_0^T and S_T = S_0 + V^T K (matrix products only)."""
    x = rand_inputs(np.random.default_rng(seed), B, T, H)
    x["w"] = np.ones_like(x["w"])
    x["a"] = np.zeros_like(x["a"])
    y, s = call(orc, x)
    worst = 0.0
    for bb in range(B):
        for hh in range(H):
            R, K, V = (x[n][bb, :, hh, :] for n in "rkv")
            S0 = x["state_in"][bb, hh]
            Y = np.tril(R @ K.T) @ V + R @ S0.T
            ST = S0 + V.T @ K
            worst = max(worst, rel(y[bb, :, hh, :], Y), rel(s[bb, hh], ST))
    return worst


def pin_delta_rule_retrieval(orc, seed=4, B=1, T=20, H=2):
    """w = 1, a_lr = 1, k = r = kk, a = -kk, b = kk with |kk| = 1: y_t = v_t exactly.

    S_t kk = S_{t-1}(I - kk kk^T) kk + v_t (kk . kk) = v_t: each token's key is
    overwritten with its value (the test-time-training reading of the delta rule,
    wiki.swarma.org RWKV page, "Delta Rule"; RWKV-LM README, oa0.com/c/1004164,
    introduction: the state does an in-context gradient step per token).
    """
    rng = np.random.default_rng(seed)
    x = rand_inputs(rng, B, T, H)
    kk = rng.standard_normal((B, T, H, N))
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    x.update(w=np.ones_like(kk), k=kk, r=kk, a=-kk, b=kk.copy())
    y, _ = call(orc, x)
    return rel(y, x["v"])


def pin_memoryless(orc, seed=5, B=1, T=9, H=2):
    """w = 0, a = 0: y_t = v_t (k_t . r_t), S_T = v_T k_T^T (readout sees this token's write)."""
    x = rand_inputs(np.random.default_rng(seed), B, T, H)
    x["w"] = np.zeros_like(x["w"])
    x["a"] = np.zeros_like(x["a"])
    y, s = call(orc, x)
    yc = x["v"] * np.sum(x["k"] * x["r"], axis=-1, keepdims=True)
    sc = np.einsum("bhi,bhj->bhij", x["v"][:, -1], x["k"][:, -1])
    return max(rel(y, yc), rel(s, sc))


def pin_linearity(orc, seed=6, B=1, T=10, H=2):
    """y and S_T are jointly linear in (v, S_0) for fixed r, w, k, a, b."""
    rng = np.random.default_rng(seed)
    x1 = rand_inputs(rng, B, T, H)
    x2 = dict(x1)
    x2["v"] = rng.standard_normal(x1["v"].shape)
    x2["state_in"] = rng.standard_normal(x1["state_in"].shape) * 0.3
    x3 = dict(x1)
    x3["v"] = 2.0 * x1["v"] - 3.0 * x2["v"]
    x3["state_in"] = 2.0 * x1["state_in"] - 3.0 * x2["state_in"]
    y1, s1 = call(orc, x1)
    y2, s2 = call(orc, x2)
    y3, s3 = call(orc, x3)
    x0 = dict(x1)
    x0["v"] = np.zeros_like(x1["v"])
    x0["state_in"] = np.zeros_like(x1["state_in"])
    y0, s0 = call(orc, x0)
    zero = max(np.max(np.abs(y0)), np.max(np.abs(s0)))
    return max(rel(y3, 2 * y1 - 3 * y2), rel(s3, 2 * s1 - 3 * s2), zero)


def pin_permutations(orc, seed=7, B=1, T=8, H=2):
    """Permuting value rows permutes y and S_T rows; permuting key columns leaves y alone."""
    rng = np.random.default_rng(seed)
    x = rand_inputs(rng, B, T, H)
    y, s = call(orc, x)
    p = rng.permutation(N)
    xv = dict(x)
    xv["v"] = x["v"][..., p]
    xv["state_in"] = x["state_in"][:, :, p, :]
    yv, sv = call(orc, xv)
    q = rng.permutation(N)
    xk = {n: x[n][..., q] for n in "rwkab"}
    xk["v"] = x["v"]
    xk["state_in"] = x["state_in"][:, :, :, q]
    yk, sk = call(orc, xk)
    return max(rel(yv, y[..., p]), rel(sv, s[:, :, p, :]), rel(yk, y), rel(sk, s[:, :, :, q]))


def pin_split_resume(orc, seed=8, B=2, T=30, H=2):
    """One pass equals a pass over the first part followed by a pass resumed from its state
    (RWKV-LM README, oa0.com/c/1004164, "RWKV introduction": forward(tokens, state) continues
    a sequence and gives the same result as one call)."""
    x = rand_inputs(np.random.default_rng(seed), B, T, H)
    y, s = call(orc, x)
    c = 11
    xa = {n: x[n][:, :c] for n in "rwkvab"}
    xa["state_in"] = x["state_in"]
    ya, sa = call(orc, xa)
    xb = {n: x[n][:, c:] for n in "rwkvab"}
    xb["state_in"] = sa
    yb, sb = call(orc, xb)
    return max(rel(np.concatenate([ya, yb], axis=1), y), rel(sb, s))


# ---------------------------------------------------------------- exact rationals
def dyadic_inputs(seed, B=1, T=4, H=2, n=N, nnz_ab=4):
    """Inputs whose float32 and bfloat16 encodings are exact and whose whole recurrence is
    exact in binary floating point: r, k, v in {-1, -1/2, 0, 1/2, 1}, w in {1/2, 3/4, 1},
    a and b with at most `nnz_ab` non-zeros in {-1, -1/2, 1/2, 1}, S_0 in {-1/2, -1/4, 0, 1/4, 1/2}."""
    rng = np.random.default_rng(seed)
    vals = np.array([-1.0, -0.5, 0.0, 0.5, 1.0])
    x = {n_: rng.choice(vals, size=(B, T, H, n)) for n_ in "rkv"}
    x["w"] = rng.choice(np.array([0.5, 0.75, 1.0]), size=(B, T, H, n))
    for n_ in "ab":
        z = np.zeros((B, T, H, n))
        for bb in range(B):
            for t in range(T):
                for hh in range(H):
                    idx = rng.choice(n, size=nnz_ab, replace=False)
                    z[bb, t, hh, idx] = rng.choice(np.array([-1.0, -0.5, 0.5, 1.0]), size=nnz_ab)
        x[n_] = z
    x["state_in"] = rng.choice(np.array([-0.5, -0.25, 0.0, 0.25, 0.5]), size=(B, H, n, n))
    return x


def exact_fraction_run(x):
    """Pure-Python rational arithmetic; also returns the largest binary magnitude needed.

    `bits` is max over every dot product / update of log2(sum |terms| * 2^d), where 2^d is
    the least common denominator of its terms: if bits <= 24, every partial sum, in any
    order and with or without fused multiply-add, is exact in float32.
    """
    F = Fraction
    r, w, k, v, a, b = ([[[[F(float(e)) for e in row] for row in hh] for hh in tt] for tt in x[n]] for n in "rwkvab")
    B, T, H, n = x["r"].shape
    y = np.zeros((B, T, H, n))
    sT = np.zeros((B, H, n, n))
    maxbits = 0.0

    def need(terms):
        nonlocal maxbits
        den = 1
        tot = F(0)
        for tm in terms:
            den = max(den, tm.denominator)
            tot += abs(tm)
        if tot:
            maxbits = max(maxbits, float(np.log2(float(tot * den))))

    for bb in range(B):
        for hh in range(H):
            S = [[F(float(x["state_in"][bb, hh, i, j])) for j in range(n)] for i in range(n)]
            for t in range(T):
                rr, ww, kk, vv, aa, bv = (q[bb][t][hh] for q in (r, w, k, v, a, b))
                for i in range(n):
                    terms = [S[i][j] * aa[j] for j in range(n)]
                    need(terms)
                    sa = sum(terms, F(0))
                    for j in range(n):
                        parts = [S[i][j] * ww[j], sa * bv[j], vv[i] * kk[j]]
                        need(parts)
                        S[i][j] = parts[0] + parts[1] + parts[2]
                    terms = [S[i][j] * rr[j] for j in range(n)]
                    need(terms)
                    y[bb, t, hh, i] = float(sum(terms, F(0)))
            for i in range(n):
                for j in range(n):
                    sT[bb, hh, i, j] = float(S[i][j])
    return y, sT, maxbits


def cast_inputs(x, dtype):
    """float64 dict -> float32 or bfloat16-bit dict (the state stays float32)."""
    out = {}
    for n_ in "rwkvab":
        x32 = x[n_].astype(np.float32)
        out[n_] = x32 if dtype == "f32" else f32_to_bf16_bits(x32)
    out["state_in"] = x["state_in"].astype(np.float32)
    return out


# ---- 16-bit stored-state encodings (reduced-precision decode state)

def _f16_table():
    """Every finite binary16 value, as float64, from numpy's own decoding."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    return bits, vals


def pin_widen16(orc) -> float:
    """Fraction of the 65536 encodings (each format) that the oracle widens differently
    from numpy's float16 decoding and from the input module's bfloat16 decoding."""
    from linear_rnn_amd.inputs import bf16_bits_to_f32
    bits, f16 = _f16_table()
    with np.errstate(invalid="ignore"):
        bf = bf16_bits_to_f32(bits).astype(np.float64)
    bad = 0
    for fmt, ref in (("f16", f16), ("bf16", bf)):
        got = orc.widen16(bits, fmt)
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        same &= (np.signbit(got) == np.signbit(ref)) | np.isnan(ref)  # a NaN's sign carries nothing
        bad += int((~same).sum())
    return bad / (2 << 16)


def round16_cases(seed=31, n=20000):
    """Doubles that exercise 16-bit rounding: log-uniform magnitudes over both
    formats' normal, subnormal and overflow ranges, random signs, and exact
    midpoints between neighbouring binary16 values (ties)."""
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.uniform(-30, 17, n))
    x = mag * rng.choice([-1.0, 1.0], n)
    _, f16 = _f16_table()
    fin = np.unique(f16[np.isfinite(f16)])
    mids = (fin[:-1] + fin[1:]) / 2  # exact in float64
    pick = rng.choice(len(mids), 4000, replace=False)
    edges = np.array([65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26,
                      2.0 ** -14, (1 - 2.0 ** -11) * 2.0 ** -14, 0.0, -0.0])
    return np.concatenate([x, mids[pick], edges, -edges])


def pin_round16(orc, seed=31) -> float:
    """Fraction of cases where the oracle's rounding disagrees with an independent rule.

    binary16: numpy's float64 -> float16 conversion (round to nearest, ties to
    even, with subnormals and overflow to infinity).
    bfloat16: for float32-exact inputs, the input module's float32 -> bfloat16
    rounding; for arbitrary doubles, exact rational comparison with the two
    neighbouring bfloat16 values (nearest wins, ties go to the even encoding).
    """
    from linear_rnn_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    x = round16_cases(seed)
    with np.errstate(over="ignore"):
        ref16 = x.astype(np.float16).view(np.uint16)
    bad = int((orc.round16(x, "f16") != ref16).sum())
    # bfloat16 on float32-exact values
    rng = np.random.default_rng(seed + 1)
    f32 = (np.exp2(rng.uniform(-140, 127, 20000)) * rng.choice([-1.0, 1.0], 20000)).astype(np.float32)
    f32 = np.concatenate([f32, bf16_bits_to_f32(np.arange(0, 0x7f80, 7, dtype=np.uint16)) * np.float32(1 + 2 ** -8)])
    bad += int((orc.round16(f32.astype(np.float64), "bf16") != f32_to_bf16_bits(f32)).sum())
    # bfloat16 on doubles that are not float32 values: exact nearest-neighbour check
    d = np.exp2(rng.uniform(-130, 120, 600)) * (1 + rng.uniform(0, 2.0 ** -30, 600))
    got = orc.round16(d, "bf16")
    for xi, gi in zip(d, got):
        cands = [int(gi) - 1, int(gi), int(gi) + 1]
        vals = {c: Fraction(float(bf16_bits_to_f32(np.array([c], dtype=np.uint16))[0])) for c in cands
                if 0 <= c < 0x7f80}
        xf = Fraction(float(xi))
        best = min(abs(xf - v) for v in vals.values())
        winners = [c for c, v in vals.items() if abs(xf - v) == best]
        ok = int(gi) in winners and (len(winners) == 1 or int(gi) % 2 == 0)
        bad += 0 if ok else 1
    return bad / (len(x) + len(f32) + len(d))
