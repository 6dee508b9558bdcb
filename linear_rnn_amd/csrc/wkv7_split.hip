// Chunked WKV-7 prefill in two kernels, so that the chunk-parallel half of the
// work uses the whole chip whatever the number of heads.
//
// Recurrence (RWKV-7 G0 7.2B notes, lshu.cn/news/198401, section 7.1), per head:
//   S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T,   y_t = S_t r_t.
//
// Chunk form (derived; WY / "DPLR" style). Tokens t = 0..15 of a chunk, state S0
// at its start, gamma_t = sum_{u<=t} log w_u per key column j:
//   U[t]  = S_{t-1} a_t                       (the "state*a" term, a row over values i)
//   U     = A' S0^T + G_u V,   Y = R' S0^T + G_y V,
//   S_C^T = diag(e^{gamma_15}) S0^T + B- U + K- V
// with
//   A^[t] = a_t e^{gamma_{t-1}},  R^[t] = r_t e^{gamma_t},
//   B-[s] = b_s e^{gamma_15 - gamma_s},  K-[s] = k_s e^{gamma_15 - gamma_s},
//   L_ab[t][s] = sum_j a_t,j b_s,j e^{gamma_{t-1} - gamma_s}  (s <  t), L_ak likewise with k,
//   L_rb[t][s] = sum_j r_t,j b_s,j e^{gamma_t - gamma_s}      (s <= t), L_rk likewise with k,
//   T = (I - L_ab)^{-1},  M_r = L_rb T,
//   A' = T A^,  R' = R^ + M_r A^,  G_u = T L_ak,  G_y = M_r L_ak + L_rk.
// Everything except S0 and V is a function of the chunk's own r, w, k, a, b.
//
// Kernel 1 (prep) runs one wave per (head, chunk), all chunks in parallel. It
// computes the decay factors, the four Grams (bfloat16 hi/lo MFMA), T and M_r (float32
// back substitution) and the products above, and writes a 9,472-byte record per
// chunk: A', R', G_u, G_y, B-, K- as float16 MFMA fragments in the exact register
// layout that kernel 2 consumes, plus e^{gamma_15} in float32.
//
// Kernel 2 (scan) carries the float32 state through the chunks. A head's 64
// value rows are independent, so it is split over two workgroups; each has two
// compute waves (16 value rows each, one SIMD each) that advance the state with
// ten 16x16x32 MFMAs per chunk, and one loader wave that streams the records and
// the needed v columns straight into a six-slot LDS ring (global-to-LDS loads),
// five chunks ahead. One LDS barrier per chunk.
//
// Every dependent MFMA chain keeps one instruction shape: chains that mixed
// 16x16x32 and 16x16x16 f16 products gave wrong results on gfx950 (in whichever
// product the register allocation placed last), the same chains in one shape
// are exact.
//
// A long sequence is processed in slabs of chunks (prep of a slab, then its
// scan), so the record buffer stays a bounded workspace; the scan of slab s+1
// starts from the state that slab s stored.
//
// Numerics. Decay factors are running products of w (clamped below at 2^-15):
// factors that multiply the state are <= 1, and the Gram factors pass through
// the decay at token 7, so no factor exceeds w_min^-8. The Grams are products of
// bfloat16 hi/lo halves (hi*hi + hi*lo + lo*hi, about 2^-16 relative, with the
// float32 range) with float32 accumulation; T and M_r are float32; A', R', G_u, G_y,
// B-, K-, the state operand and U are rounded once to float16 as MFMA operands
// (float32 accumulation), so magnitudes must stay below 2^15. The carried state
// is float32 throughout.
//
// MFMA layouts (gfx950, wave64; l = lane, li = l % 16, g = l / 16):
//   16x16x16 f16      : A[m=li][k=4g+e],   B[k=4g+e][n=li]   (e = 0..3)
//   16x16x32 f16/bf16 : A[m=li][k=8g+e],   B[k=8g+e][n=li]   (e = 0..7)
//   all          : D[m=4g+e][n=li]
// A D result is unchanged a B operand with K = 16, and a product with the
// identity as B turns an A-layout tile into the D layout (a transpose).
// Contractions may permute their K index freely as long as both operands use
// the same permutation: the 64-key contractions below take key 16kt + 4g + e for
// (step, lane group, element), matching the state tiles' D layout.
#include <cstdlib>
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

#include "wkv7_device.hpp"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 16;   // tokens per chunk
constexpr float kWMin = 0x1p-15f;

// Record of one (head, chunk): nine 1 KiB fragment blocks (16 bytes per lane),
// then e^{gamma_15} for the 64 key columns.
enum { kRecA0 = 0, kRecA1 = 1, kRecR0 = 2, kRecR1 = 3, kRecG = 4, kRecBK = 5, kRecBlocks = 9 };
constexpr int kRecD = kRecBlocks * 1024;
constexpr int kRecBytes = kRecD + kN * 4;  // 9472

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 mfma16(half4 a, half4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half4 to_h4(f32x4 x) {
  return half4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}
__device__ __forceinline__ half8 cat8(half4 lo, half4 hi) {
  return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}


// bfloat16 bits (low 16 bits of the argument) widened to float32, exactly
__device__ __forceinline__ float bfw(uint32_t raw16) { return __uint_as_float(raw16 << 16); }
// element e (0..3) of four bfloat16 packed in a uint2
__device__ __forceinline__ float bf4(uint2 q, int e) {
  const uint32_t u = e < 2 ? q.x : q.y;
  return (e & 1) ? __uint_as_float(u & 0xffff0000u) : __uint_as_float(u << 16);
}

template <class V>
__device__ __forceinline__ V ld_off(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const V*>(static_cast<const char*>(base) + byte_off);
}
template <class V>
__device__ __forceinline__ void st_off(void* base, uint32_t byte_off, V v) {
  *reinterpret_cast<V*>(static_cast<char*>(base) + byte_off) = v;
}

// ============================================================================ kernel 1: prep

// Inputs of the prep. The plain recurrence takes r, w, k, a, b (bfloat16). The fused
// time-mix operator takes r, k (bfloat16), w_raw (float32) in place of w, and kk,
// a_lr in place of a, b; the prep then forms w = exp(-exp(w_raw)), the unit key
// kk^ = kk / max(|kk|, 1e-12) over the head's 64 channels, a = -kk^ and b = kk^ a_lr.
constexpr int kPrepPlain = 0, kPrepTmix = 1;
struct PrepParams {
  const uint16_t* r;
  const uint16_t* w;   // plain: the decay
  const float* w_raw;  // time-mix: the decay's log-log form
  const uint16_t* k;
  const uint16_t* a;   // plain: a; time-mix: kk
  const uint16_t* b;   // plain: b; time-mix: a_lr
  unsigned char* rec;  // [unit][chunk of slab][kRecBytes]
  int32_t T, H;
  int32_t c0;     // first chunk of the slab
  int32_t nc;     // chunks in the slab
  int32_t items;  // B * H * nc
};

constexpr int kPrepWaves = 4;
constexpr int kFacRow = kN + 4;  // padded float row: token-layout reads of one row spread over the banks
// Factor rows (float32, [row][key]), written in the key layout (lane = key j):
//   E  row t + 1 = e^{gamma_t},            t = -1..15
//   Gq row t + 1 = e^{gamma_t - gamma_7},  t = -1..15
// Fk_t = e^{gamma_7 - gamma_t} = 1 / Gq_t and e^{gamma_15 - gamma_t} = Gq_15 Fk_t are
// formed where they are used.
constexpr int kRowE = 0, kRowG = 17, kFacRows = 34;
constexpr int kPrepLdsPerWave = kFacRows * kFacRow * 4;  // 9,248 bytes
// After the factors are consumed the same wave area holds L_ab ([t][s], float32), the
// right-hand sides of the solve (the identity, then L_rb, [32][16] float32) and the
// rows of T and M_r (float16).
constexpr int kLabOff = 0, kRhsOff = 16 * 16, kTmOffBytes = 3 * 16 * 16 * 4;
static_assert(kTmOffBytes + 2 * 16 * 16 * 2 <= kPrepLdsPerWave, "solve area");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// x = hi + lo with both halves bfloat16 (round to nearest even): 16 significant bits and
// the float32 exponent range, which the Gram operands need (factors up to w_min^-8).
__device__ __forceinline__ void split_bf16(float x, bf16x8& hi, bf16x8& lo, int i) {
  const __bf16 h = (__bf16)x;
  hi[i] = h;
  lo[i] = (__bf16)(x - (float)h);
}
__device__ __forceinline__ f32x4 mfma_bf(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4 lds4(const float* p) { return *reinterpret_cast<const float4*>(p); }
// An ordering point for the values in x and for memory: the compiler computes x
// before it and issues no later memory access ahead of it.
__device__ __forceinline__ void pin16(float (&x)[16]) {
  asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]),
               "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]), "+v"(x[14]), "+v"(x[15])
               :
               : "memory");
}
__device__ __forceinline__ float el(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

template <int MODE>
// three waves per SIMD: the register budget of four spills
__global__ __launch_bounds__(64 * kPrepWaves) __attribute__((amdgpu_waves_per_eu(3))) void wkv7_prep_kernel(PrepParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int item = (int)blockIdx.x * kPrepWaves + wave;
  if (item >= p.items) return;  // wave-uniform; this kernel has no workgroup barrier
  float* fac = reinterpret_cast<float*>(smem_raw + wave * kPrepLdsPerWave);

  // item = (b * nc + chunk) * H + h: neighbouring waves read neighbouring heads of one token block
  const int h = item % p.H;
  const int rest = item / p.H;
  const int cl = rest % p.nc;
  const int bb = rest / p.nc;
  const int unit = bb * p.H + h;
  const int t0 = (p.c0 + cl) * kC;
  const int nt = min(kC, p.T - t0);  // live tokens, >= 1
  const int64_t base = ((int64_t)bb * p.T + t0) * p.H * kN + (int64_t)h * kN;  // element offset of token t0
  const uint32_t tstride = (uint32_t)p.H * kN;                                // elements between tokens
  unsigned char* rec = p.rec + ((int64_t)unit * p.nc + cl) * kRecBytes;

  // ---- raw r, a, b, k in the token layout: lane (t = li, g) holds keys 16kt + 4g .. 4g+3.
  // Past-the-end tokens read token nt-1 and become identity tokens (r = k = a = b = 0, w = 1).
  const int tl = min(li, nt - 1);
  const bool live = li < nt;
  uint2 rr[4], ar[4], br[4], kr[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const uint32_t off = (uint32_t)(tl * tstride + 16 * kt + 4 * g) * 2u;
    rr[kt] = ld_off<uint2>(p.r + base, off);
    ar[kt] = ld_off<uint2>(p.a + base, off);
    br[kt] = ld_off<uint2>(p.b + base, off);
    kr[kt] = ld_off<uint2>(p.k + base, off);
  }
  // ---- w in the key layout: lane = key j, all 16 tokens
  float wc[kC];
#pragma unroll
  for (int t = 0; t < kC; ++t) {
    const int tt = min(t, nt - 1);
    float x;
    if constexpr (MODE == kPrepTmix)
      x = expf(-expf(ld_off<float>(p.w_raw + base, (uint32_t)(tt * tstride + lane) * 4u)));
    else
      x = bfw(ld_off<uint16_t>(p.w + base, (uint32_t)(tt * tstride + lane) * 2u));
    wc[t] = x < kWMin ? kWMin : x;  // clamp (a NaN passes through)
  }
  // The last chunk of a sequence may run past its end: its tokens t >= nt become
  // identity tokens (w = 1, r = k = a = b = 0). The branch is the same for the whole wave.
  if (nt < kC) {
    const uint2 z2 = make_uint2(0u, 0u);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      rr[kt] = live ? rr[kt] : z2;
      ar[kt] = live ? ar[kt] : z2;
      br[kt] = live ? br[kt] : z2;
      kr[kt] = live ? kr[kt] : z2;
    }
#pragma unroll
    for (int t = 0; t < kC; ++t) wc[t] = t < nt ? wc[t] : 1.f;
  }

  // ---- decay factors (lane = j): running products from token 0 (E) and outward from
  // token 7 (Gq), so no factor exceeds w_min^-8
  {
    const int j = lane;
    float e = 1.f, gu = 1.f, gd = 1.f;
    fac[kRowE * kFacRow + j] = 1.f;        // E_{-1}
    fac[(kRowG + 8) * kFacRow + j] = 1.f;  // Gq_7
#pragma unroll
    for (int q = 0; q < kC; ++q) {
      e *= wc[q];
      fac[(kRowE + q + 1) * kFacRow + j] = e;  // E_q
      if (q < 8) {
        gu *= wc[8 + q];  // Gq_t, t = 8 + q: times w_t
        fac[(kRowG + 9 + q) * kFacRow + j] = gu;
        gd *= __builtin_amdgcn_rcpf(wc[7 - q]);  // Gq_t, t = 6 - q: divided by w_{t+1}
        fac[(kRowG + 7 - q) * kFacRow + j] = gd;
      }
    }
    st_off<float>(rec, (uint32_t)(kRecD + 4 * j), e);  // e^{gamma_15}
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the rows are in LDS before other lanes read them
  __builtin_amdgcn_wave_barrier();

  // ---- token layout: operands, the four Grams and B-, K- (stored at once). Key 16kt + 4g + e
  // of the lane's token. Each Gram contracts 64 keys on 16x16x32 bfloat16 MFMAs as
  // hi*hi + hi*lo + lo*hi of the operands' bfloat16 halves (relative error about 2^-16),
  // two key blocks per product: K index 8g + 4(kt % 2) + e. The Grams land in the D layout:
  // lane (s = li, g) holds t = 4g + e; L_rk is formed transposed (operands swapped).
  // Identity as a B operand: B[k = 4g+e][n = li] = (4g + e == li).
  half4 eye;
#pragma unroll
  for (int e = 0; e < 4; ++e) eye[e] = (_Float16)(4 * g + e == li ? 1.f : 0.f);
  const uint32_t lo = (uint32_t)lane * 16u;  // record blocks: 16 bytes per lane
  half4 Ahat[4];
  f32x4 Rhat[4];
  f32x4 Lab = zero4(), Lak = zero4(), Lrb = zero4(), LrkT = zero4();
  // time-mix: 1 / max(|kk|, 1e-12) of this lane's token (its 64 channels are spread over
  // the four lanes li, li + 16, li + 32, li + 48)
  float inv = 1.f;
  if constexpr (MODE == kPrepTmix) {
    float n2 = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = bf4(ar[kt], e);
        n2 = fmaf(x, x, n2);
      }
    n2 += __shfl_xor(n2, 16);
    n2 += __shfl_xor(n2, 32);
    inv = 1.f / fmaxf(sqrtf(n2), 1e-12f);
  }
  bf16x8 ahH, ahL, rhH, rhL, bhH, bhL, khH, khL;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int col = 16 * kt + 4 * g;
    const float4 em1 = lds4(&fac[(kRowE + li) * kFacRow + col]);
    const float4 e0 = lds4(&fac[(kRowE + li + 1) * kFacRow + col]);
    const float4 gqm1 = lds4(&fac[(kRowG + li) * kFacRow + col]);
    const float4 gq = lds4(&fac[(kRowG + li + 1) * kFacRow + col]);
    const float4 g15 = lds4(&fac[(kRowG + 16) * kFacRow + col]);
    const uint2 ra = ar[kt], rv2 = rr[kt], rb = br[kt], rk = kr[kt];
    half4 bbar, kbar;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float av = bf4(ra, e), bv = bf4(rb, e);
      const float rv = bf4(rv2, e), kv = bf4(rk, e);
      if constexpr (MODE == kPrepTmix) {  // a = -kk^, b = kk^ a_lr
        const float kh1 = av * inv;
        av = -kh1;
        bv = kh1 * bv;
      }
      const float f = __builtin_amdgcn_rcpf(el(gq, e));  // e^{gamma_7 - gamma_t}
      const float suf = el(g15, e) * f;  // e^{gamma_15 - gamma_t}
      const int q8 = 4 * (kt & 1) + e;
      split_bf16(av * el(gqm1, e), ahH, ahL, q8);
      split_bf16(rv * el(gq, e), rhH, rhL, q8);
      split_bf16(bv * f, bhH, bhL, q8);
      split_bf16(kv * f, khH, khL, q8);
      Ahat[kt][e] = (_Float16)(av * el(em1, e));
      Rhat[kt][e] = rv * el(e0, e);
      bbar[e] = (_Float16)(bv * suf);
      kbar[e] = (_Float16)(kv * suf);
    }
    const half4 BT = to_h4(mfma16(bbar, eye, zero4()));  // lane (j = li, g): B-[4g+e][16kt + li]
    const half4 KT = to_h4(mfma16(kbar, eye, zero4()));
    st_off<half8>(rec, (kRecBK + kt) * 1024 + lo, cat8(BT, KT));
    if (kt & 1) {
      Lab = mfma_bf(ahH, bhH, Lab);
      Lak = mfma_bf(ahH, khH, Lak);
      Lrb = mfma_bf(rhH, bhH, Lrb);
      LrkT = mfma_bf(khH, rhH, LrkT);
      Lab = mfma_bf(ahH, bhL, Lab);
      Lak = mfma_bf(ahH, khL, Lak);
      Lrb = mfma_bf(rhH, bhL, Lrb);
      LrkT = mfma_bf(khH, rhL, LrkT);
      Lab = mfma_bf(ahL, bhH, Lab);
      Lak = mfma_bf(ahL, khH, Lak);
      Lrb = mfma_bf(rhL, bhH, Lrb);
      LrkT = mfma_bf(khL, rhH, LrkT);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = 4 * g + e;            // row of Lab, Lak, Lrb; column li is s
    Lab[e] = li < t ? Lab[e] : 0.f;     // strictly lower
    Lak[e] = li < t ? Lak[e] : 0.f;
    Lrb[e] = li <= t ? Lrb[e] : 0.f;    // lower with the diagonal
    LrkT[e] = t <= li ? LrkT[e] : 0.f;  // element (s = 4g+e, t = li) of L_rk^T
  }

  // ---- rows of T = (I - L_ab)^{-1} (lanes 0-15) and M_r = L_rb T (lanes 16-31):
  // x (I - L_ab) = rhs, solved right-looking: once x[s2] is final it is folded into
  // every x[s], s < s2. The factor rows are no longer read, so their area is reused;
  // the row of L_ab for the next step is read while the current one is applied.
  float* lab = fac + kLabOff;
  float* rhs = fac + kRhsOff;
  __builtin_amdgcn_s_waitcnt(0xc07f);  // every factor read of this wave has completed
  asm volatile("" ::: "memory");
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lab[(4 * g + e) * 16 + li] = Lab[e];
    rhs[(4 * g + e) * 16 + li] = 4 * g + e == li ? 1.f : 0.f;  // identity: the rows of T
    rhs[(16 + 4 * g + e) * 16 + li] = Lrb[e];                 // L_rb: the rows of M_r
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  const int row = li;
  float x[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = lds4(&rhs[((g & 1) * 16 + row) * 16 + 4 * q]);  // lanes 32-63 repeat lanes 0-31
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * q + e] = el(v, e);
  }
  float4 cur[4], nxt[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) cur[q] = lds4(&lab[(kC - 1) * 16 + 4 * q]);
#pragma unroll
  for (int s2 = kC - 1; s2 >= 1; --s2) {
    if (s2 > 1) {
#pragma unroll
      for (int q = 0; q < (s2 + 2) / 4; ++q) nxt[q] = lds4(&lab[(s2 - 1) * 16 + 4 * q]);
    }
#pragma unroll
    for (int s = 0; s < s2; ++s) x[s] = fmaf(x[s2], el(cur[s / 4], s % 4), x[s]);
    pin16(x);  // this step's updates before the next row's reads: one row in flight, not all
#pragma unroll
    for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
  }
  _Float16* tm = reinterpret_cast<_Float16*>(reinterpret_cast<unsigned char*>(fac) + kTmOffBytes);
  if (g < 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<half4*>(&tm[(g * 16 + row) * 16 + 4 * q]) =
          half4{(_Float16)x[4 * q], (_Float16)x[4 * q + 1], (_Float16)x[4 * q + 2], (_Float16)x[4 * q + 3]};
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  const half4 tB = *reinterpret_cast<const half4*>(&tm[li * 16 + 4 * g]);         // T[t = li][4g..]: T^T as B
  const half4 mB = *reinterpret_cast<const half4*>(&tm[(16 + li) * 16 + 4 * g]);  // M_r^T as B

  // ---- products, stored per block. L_rk^T is added on the vector unit.
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
    half4 ApT[2], RpT[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kt = 2 * kp + u;
      const half4 AT = to_h4(mfma16(Ahat[kt], eye, zero4()));  // lane (j = li, g): A^[4g+e][16kt + li]
      ApT[u] = to_h4(mfma16(AT, tB, zero4()));                 // lane (t = li, g): A'[t][16kt + 4g + e]
      RpT[u] = to_h4(mfma16(AT, mB, Rhat[kt]));                // R'[t][16kt + 4g + e]
    }
    st_off<half8>(rec, (kRecA0 + kp) * 1024 + lo, cat8(ApT[0], ApT[1]));
    st_off<half8>(rec, (kRecR0 + kp) * 1024 + lo, cat8(RpT[0], RpT[1]));
  }
  const half4 LakH = to_h4(Lak);  // as an A operand: L_ak^T (M = s', K = s)
  const half4 GuT = to_h4(mfma16(LakH, tB, zero4()));         // lane (t = li, g): G_u[t][4g + e]
  const half4 GyT = to_h4(mfma16(LakH, mB, zero4()) + LrkT);  // G_y[t][4g + e]
  st_off<half8>(rec, kRecG * 1024 + lo, cat8(GuT, GyT));
}

// ============================================================================ kernel 2: scan

struct ScanParams {
  const unsigned char* rec;  // records of the slab [unit][chunk of slab][kRecBytes]
  const uint16_t* v;
  float* y;
  const float* s_src;  // state at the slab start, or null for zeros
  float* s_dst;        // state at the slab end, or null
  int32_t T, H;
  int32_t c0, nc;
};

// A head's 64 value rows are independent: four compute waves of 16 rows each, two
// per workgroup (one workgroup per CU keeps every compute wave on a SIMD of its
// own). A third wave streams the workgroup's chunks straight into an LDS ring with
// global-to-LDS loads (no register staging), kDist chunks ahead of the reads; the
// compute waves issue no global loads, so nothing they wait on is behind a load.
// One barrier per chunk.
constexpr int kScanWaves = 2;  // compute waves per workgroup
constexpr int kWgPerHead = 4 / kScanWaves;
constexpr int kDist = 5;                          // chunks in flight ahead of the one read next
// ring slots: the chunk being read, the kDist in flight and one spare, so that a slot is
// reloaded only once the compute waves have used what they read from it (no wait on
// outstanding LDS reads at the barrier)
constexpr int kSlots = kDist + 2;
constexpr int kVCols = 16 * kScanWaves;           // value columns of v this workgroup needs
constexpr int kVBytes = kC * kVCols * 2;          // bfloat16, [token][kVCols]: 1 KiB
constexpr int kSlotBytes = kRecBytes + kVBytes;   // 10,496
// y staging: two chunks (by parity) of [token][kVCols] float32, so that a workgroup's y rows
// leave in whole 128-byte lines rather than one 64-byte half per compute wave
constexpr int kYStageBytes = kC * kVCols * 4;  // 2 KiB
constexpr int kScanLds = kSlots * kSlotBytes + 2 * kYStageBytes;  // 77,568: two workgroups fit a compute unit
constexpr int kLoads = kRecBlocks + 2;  // loads per lane per chunk: record blocks, e^gamma, v
constexpr int kScanThreads = 64 * (kScanWaves + 1);
// the load counter holds at most 63 outstanding operations: never more are in flight
static_assert(kDist * kLoads < 64, "load counter");
static_assert(kVBytes == 64 * 16 && kRecBlocks == 9, "one 16-byte piece of v per lane");

__device__ __forceinline__ f32x4 mfma32(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Global-to-LDS load: lane l's BYTES land at LDS address lds + BYTES * l (lds
// wave-uniform, in M0). Written as assembly so that the compiler, which cannot
// tell which later LDS reads these loads feed, inserts no wait of its own; every
// wait on them is an explicit vm_wait.
template <int BYTES>
__device__ __forceinline__ void to_lds(const void* g, uint32_t lds) {
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory");
}
// Every lane of a row of 16 reads lane K of that row (DPP row broadcast).
template <int K>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + K, 0xf, 0xf, false));
}
// Waits until at most N of this wave's vector-memory operations are outstanding
// (they complete in issue order), and orders every later memory access after it.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__global__ __launch_bounds__(kScanThreads) void wkv7_scan_kernel(ScanParams p) {
  extern __shared__ __align__(16) unsigned char ring[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  // consecutive logical ids (the workgroups of one head) run on one XCD and share its L2
  const int lid = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  const int unit = lid / kWgPerHead, part = lid % kWgPerHead;
  const int bb = unit / p.H, hh = unit % p.H;
  const int nc = p.nc;
  const uint32_t tstride = (uint32_t)p.H * kN;
  const int rb = kScanWaves * part + wave;  // a compute wave's value rows: 16 rb .. 16 rb + 15
  const unsigned char* recs = p.rec + (int64_t)unit * nc * kRecBytes;
  const int64_t seq_base =
      ((int64_t)bb * p.T + (int64_t)p.c0 * kC) * p.H * kN + (int64_t)hh * kN + kVCols * part;
  const uint16_t* vbase = p.v + seq_base;  // this workgroup's value columns
  float* ybase = p.y + seq_base;  // this workgroup's value columns of y
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));

  // ---- loader wave: chunk x (clamped to the last one: past the end the loads repeat it)
  // into slot x % kSlots: the record as it is (nine 1 KiB blocks, then e^{gamma_15}),
  // then v [token][kVCols] (lane l: token l / 4, eight columns). Tokens past the end of
  // the sequence repeat the last one; their coefficients in the record are zero.
  // Chunk x + kDist reuses the slot of chunk x + kDist - kSlots = x - 2: the compute
  // waves used what they read from it in the step of chunk x - 2, before the barrier
  // that precedes the loads of chunk x + kDist.
  if (wave == kScanWaves) {
    auto issue = [&](int x) {
      const int xc = min(x, nc - 1);
      const uint32_t slot = ring_lds + (uint32_t)((x % kSlots) * kSlotBytes);
      const unsigned char* src = recs + (int64_t)xc * kRecBytes;
#pragma unroll
      for (int b = 0; b < kRecBlocks; ++b) to_lds<16>(src + b * 1024 + lane * 16, slot + b * 1024);
      to_lds<4>(src + kRecD + lane * 4, slot + kRecD);
      const int nt = min(kC, p.T - (p.c0 + xc) * kC);
      const int t = min(lane >> 2, nt - 1);
      to_lds<16>(vbase + ((int64_t)(xc * kC + t) * tstride + 8 * (lane & 3)), slot + kRecBytes);
    };
    // once chunk c + kDist is issued, chunk c + 1 has landed when at most the loads of
    // kDist - 1 chunks are outstanding (they complete in issue order)
#pragma unroll
    for (int x = 0; x < kDist; ++x) issue(x);
    vm_wait<(kDist - 1) * kLoads>();
    asm volatile("s_barrier" ::: "memory");  // chunk 0
    for (int c = 0; c < nc; ++c) {
      issue(c + kDist);
      vm_wait<(kDist - 1) * kLoads>();
      asm volatile("s_barrier" ::: "memory");  // chunk c + 1
    }
    asm volatile("s_barrier" ::: "memory");  // the last chunk's y is staged
    vm_wait<0>();  // every load has landed before the wave ends
    return;
  }

  // element e of St[kt] = S[i = 16 rb + li][j = 16kt + 4g + e]
  f32x4 St[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) St[kt] = zero4();
  if (p.s_src) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float4 s = *reinterpret_cast<const float4*>(p.s_src + ((int64_t)unit * kN + 16 * rb + li) * kN +
                                                        16 * kt + 4 * g);
      St[kt] = f32x4{s.x, s.y, s.z, s.w};
    }
  }
  // vmcnt(0) as a builtin, so the compiler's own wait counting knows the state has landed
  // (it would otherwise wait for it at the first use, behind the first chunks' loads)
  __builtin_amdgcn_s_waitcnt(0x0f70);

  // fragments of one chunk, read from its ring slot one iteration ahead
  struct Frag {
    half8 a0, a1, r0, r1, gl, bk[4];
    float dv;  // e^{gamma_15} of key 16 (li / 4) + 4g + li % 4: lane 4kt + e of row g holds the
               // decay that every lane of the row needs as its (kt, e) element
    uint32_t v[4];  // V[t = 4g + e][i = 16 rb + li], raw bfloat16 bits (widened when used)
  };
  const uint32_t lo = (uint32_t)lane * 16u;
  // the loop below is unrolled by the ring size, so every slot index is a constant and
  // every LDS address a fixed offset from the lane's base
  auto read = [&](auto slot_index, Frag& f) {
    const unsigned char* slot = ring + decltype(slot_index)::value * kSlotBytes;
    // in the order of use (the next chunk's first products take v and G)
    const uint16_t* vr = reinterpret_cast<const uint16_t*>(slot + kRecBytes);  // [token][kVCols]
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[e] = vr[(4 * g + e) * kVCols + 16 * wave + li];
    f.gl = *reinterpret_cast<const half8*>(slot + kRecG * 1024 + lo);
    f.a0 = *reinterpret_cast<const half8*>(slot + kRecA0 * 1024 + lo);
    f.r0 = *reinterpret_cast<const half8*>(slot + kRecR0 * 1024 + lo);
    f.a1 = *reinterpret_cast<const half8*>(slot + kRecA1 * 1024 + lo);
    f.r1 = *reinterpret_cast<const half8*>(slot + kRecR1 * 1024 + lo);
    f.dv = *reinterpret_cast<const float*>(slot + kRecD + (16 * (li >> 2) + 4 * g + (li & 3)) * 4);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) f.bk[kt] = *reinterpret_cast<const half8*>(slot + (kRecBK + kt) * 1024 + lo);
  };
  const half4 hz = half4{(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
  // y of chunk c goes through LDS: each compute wave stages its 16 columns (lane: token li,
  // columns 16 wave + 4g .. + 3), and after the next barrier wave q stores tokens 8q .. 8q + 7
  // of all kVCols columns, eight lanes (128 contiguous bytes) per token; tokens past the end
  // of the sequence are not stored
  unsigned char* ystage = ring + kSlots * kSlotBytes;
  auto stage_y = [&](auto par, const f32x4& yv) {
    *reinterpret_cast<f32x4*>(ystage + decltype(par)::value * kYStageBytes + (li * kVCols + 16 * wave + 4 * g) * 4) = yv;
  };
  auto flush_y = [&](auto par, int c) {
    const int tt = 8 * wave + (lane >> 3), cc = 4 * (lane & 7);
    const f32x4 v =
        *reinterpret_cast<const f32x4*>(ystage + decltype(par)::value * kYStageBytes + (tt * kVCols + cc) * 4);
    const int nt = min(kC, p.T - (p.c0 + c) * kC);
    const uint32_t off = (uint32_t)(((c * kC + tt) * tstride + cc) * 4u);
    if (nt == kC)  // the same for the whole wave: a whole chunk stores with no lane masked
      st_off<float4>(ybase, off, make_float4(v[0], v[1], v[2], v[3]));
    else if (tt < nt)
      st_off<float4>(ybase, off, make_float4(v[0], v[1], v[2], v[3]));
  };
  // One chunk. Its y is staged at the end, after the state update is issued, when the
  // products that made it have long completed.
  auto step = [&](auto par, const Frag& f) {
    half4 vB;
#pragma unroll
    for (int e = 0; e < 4; ++e) vB[e] = (_Float16)bfw(f.v[e]);
    // K = 32 products (16x16x32 only: every dependent chain keeps one MFMA shape).
    //   U = A' S0^T + G_u V and Y = R' S0^T + G_y V: two key halves, then the
    //   G V term (the record's G block holds G_u | G_y, so a B operand of V | 0
    //   or 0 | V selects one of them);
    //   S^T <- diag(e^{gamma_15}) S^T + [B- | K-] [U ; V] per key tile.
    // the G V terms first: they do not depend on the state, so they need not wait for
    // the previous chunk's update. Y is formed transposed (operands swapped: the state
    // and V fragments serve as A operands, R' and G as B operands, from the same
    // registers), so a lane holds four consecutive value rows of one token for its store.
    f32x4 u = mfma32(f.gl, cat8(vB, hz), zero4());
    f32x4 yv = mfma32(cat8(hz, vB), f.gl, zero4());
    const half8 sB0 = cat8(to_h4(St[0]), to_h4(St[1]));
    const half8 sB1 = cat8(to_h4(St[2]), to_h4(St[3]));
    u = mfma32(f.a0, sB0, u);
    yv = mfma32(sB0, f.r0, yv);
    u = mfma32(f.a1, sB1, u);
    yv = mfma32(sB1, f.r1, yv);
    const half8 uv = cat8(to_h4(u), vB);
    // the decays by row broadcasts (one 4-byte LDS read per lane instead of four 16-byte ones)
    St[0][0] *= row_bcast<0>(f.dv);
    St[0][1] *= row_bcast<1>(f.dv);
    St[0][2] *= row_bcast<2>(f.dv);
    St[0][3] *= row_bcast<3>(f.dv);
    St[0] = mfma32(f.bk[0], uv, St[0]);
    St[1][0] *= row_bcast<4>(f.dv);
    St[1][1] *= row_bcast<5>(f.dv);
    St[1][2] *= row_bcast<6>(f.dv);
    St[1][3] *= row_bcast<7>(f.dv);
    St[1] = mfma32(f.bk[1], uv, St[1]);
    St[2][0] *= row_bcast<8>(f.dv);
    St[2][1] *= row_bcast<9>(f.dv);
    St[2][2] *= row_bcast<10>(f.dv);
    St[2][3] *= row_bcast<11>(f.dv);
    St[2] = mfma32(f.bk[2], uv, St[2]);
    St[3][0] *= row_bcast<12>(f.dv);
    St[3][1] *= row_bcast<13>(f.dv);
    St[3][2] *= row_bcast<14>(f.dv);
    St[3][3] *= row_bcast<15>(f.dv);
    St[3] = mfma32(f.bk[3], uv, St[3]);
    stage_y(par, yv);
  };

  // ---- compute waves. After barrier m they read chunk m and run the step of chunk
  // m - 1, which uses the reads of the iteration before: by barrier m + 1 every read of
  // chunk m - 1 has completed (its values were used), and the loader reloads that
  // chunk's slot only after barrier m + 1 (the ring has a spare slot), so the barrier
  // waits for no LDS read. The loop body has no branch around the reads: a read past
  // the last chunk reads a slot that holds a repeat of it and is never used. (A read on
  // one side of a branch only would make the compiler's wait at the join cover the
  // next chunk's reads too.)
  // the staged y of the previous chunk must be in LDS before the barrier; this also waits for
  // the next chunk's reads, issued a step earlier
  auto sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  };
  Frag fr[2];
  // chunk c + j sits in slot j % kSlots (c is a multiple of the unroll, itself a multiple
  // of the ring size); the two register sets alternate, so the unroll is also even
  constexpr int kUnroll = kSlots % 2 == 0 ? kSlots : 2 * kSlots;
  int c = 0;
  // chunk c + J: barrier, read of the next chunk, y of the chunk before, step; true after
  // the last chunk
  auto chunk = [&](auto J) {
    constexpr int j = decltype(J)::value;
    sync();
    read(std::integral_constant<int, (j + 1) % kSlots>{}, fr[(j + 1) % 2]);
    if (c + j > 0) flush_y(std::integral_constant<int, (j + 1) % 2>{}, c + j - 1);
    step(std::integral_constant<int, j % 2>{}, fr[j % 2]);
    return c + j + 1 >= nc;
  };
  // chunks c .. c + kUnroll - 1, every slot index a constant; true after the last chunk
  auto unrolled = [&](auto self, auto J) -> bool {
    constexpr int j = decltype(J)::value;
    if constexpr (j == kUnroll) {
      return false;
    } else {
      if (chunk(J)) return true;
      return self(self, std::integral_constant<int, j + 1>{});
    }
  };
  sync();  // chunk 0
  read(std::integral_constant<int, 0>{}, fr[0]);
  for (;; c += kUnroll)
    if (unrolled(unrolled, std::integral_constant<int, 0>{})) break;
  sync();  // the last chunk's y is staged (the loader waits at this barrier too)
  if ((nc - 1) % 2 == 0)
    flush_y(std::integral_constant<int, 0>{}, nc - 1);
  else
    flush_y(std::integral_constant<int, 1>{}, nc - 1);

  if (p.s_dst) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      *reinterpret_cast<float4*>(p.s_dst + ((int64_t)unit * kN + 16 * rb + li) * kN + 16 * kt + 4 * g) =
          make_float4(St[kt][0], St[kt][1], St[kt][2], St[kt][3]);
  }
}

// ============================================================================ host side

// Device workspace (records of the chunked split prefill, checkpoints of the
// backward) cached per (device, stream):
// calls on one stream run in order, so they can share it; calls on different
// streams get different buffers. Grown on demand, never shrunk.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::tuple<int, uintptr_t, int>, Workspace> g_ws;


// Record-buffer budget per slab: the scan of a slab reads what its prep wrote
// just before, so a slab about the size of the 256 MB last-level (MALL) cache
// is mostly read back from it; fewer, larger slabs also spend less on launches
// and on the prep's last, partly filled round of waves (measured: one 233 MB
// slab beats three of 78 MB for the 96-head, 4096-token workload).
size_t slab_budget_bytes() {
  static const size_t mb = [] {
    const char* s = std::getenv("RWKV7_SPLIT_SLAB_MB");
    const long v = s ? std::atol(s) : 0;
    return v > 0 ? (size_t)v : (size_t)256;
  }();
  return mb << 20;
}

}  // namespace

hipError_t device_workspace(hipStream_t stream, size_t bytes, void** out, int slot) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace& ws = g_ws[std::make_tuple(dev, reinterpret_cast<uintptr_t>(stream), slot)];
  if (ws.bytes < bytes) {
    if (ws.ptr) {
      // work already queued on this stream may still use the old buffer
      e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return e;
      e = hipFree(ws.ptr);
      if (e != hipSuccess) return e;
      ws.ptr = nullptr;
      ws.bytes = 0;
    }
    e = hipMalloc(&ws.ptr, bytes);
    if (e != hipSuccess) {
      ws.ptr = nullptr;
      return e;
    }
    ws.bytes = bytes;
  }
  *out = ws.ptr;
  return hipSuccess;
}


namespace {

// Resident prep waves on this device: workgroups per compute unit (the prep's
// register footprint decides) times its waves times the compute units.
int64_t prep_waves_resident() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&wkv7_prep_kernel<kPrepPlain>),
                                                   64 * kPrepWaves, kPrepWaves * kPrepLdsPerWave) != hipSuccess ||
      per_cu <= 0)
    per_cu = 2;
  return (int64_t)cus * per_cu * kPrepWaves;
}

}  // namespace

namespace {

// One chunked pass: the prep (in the given input mode) and the scan, slab by slab.
struct SplitJob {
  PrepParams in;  // input pointers (and T, H); the rest is filled per slab
  int mode;
  const uint16_t* v;
  float* y;
  const float* s_in;
  float* s_out;
  int64_t B, T, H;
  hipStream_t stream;
};

hipError_t run_split(const SplitJob& j) {
  const int64_t units = j.B * j.H;
  const int64_t nch = (j.T + kC - 1) / kC;
  // In-sequence offsets are 32-bit: T * H * 64 elements must stay below 2^31.
  if (j.T * j.H * kN >= (int64_t(1) << 31)) return hipErrorNotSupported;
  const int64_t per_chunk = units * kRecBytes;
  int64_t slab = (int64_t)(slab_budget_bytes() / (size_t)per_chunk);
  slab = slab < 1 ? 1 : slab;
  if (slab < nch) {
    // Every prep item takes about the same time, so a slab whose items fill
    // whole rounds of resident waves leaves no round running nearly empty.
    const int64_t W = prep_waves_resident();
    const int64_t rounds = units * slab / W;
    if (rounds >= 1) slab = rounds * W / units > 0 ? rounds * W / units : 1;
  } else {
    slab = nch;
  }
  const int64_t nslab = (nch + slab - 1) / slab;
  if (units * slab > (int64_t(1) << 30)) return hipErrorNotSupported;
  const bool tmp_state = nslab > 1 && j.s_out == nullptr;
  const size_t rec_bytes = (size_t)(units * slab * kRecBytes);
  const size_t bytes = rec_bytes + (tmp_state ? (size_t)units * kN * kN * 4 : 0);
  void* ws = nullptr;
  hipError_t e = device_workspace(j.stream, bytes, &ws, kWorkspaceChunks);
  if (e != hipSuccess) return e;
  unsigned char* rec = static_cast<unsigned char*>(ws);
  float* carry = tmp_state ? reinterpret_cast<float*>(rec + rec_bytes) : j.s_out;

  const void* prep_fn = j.mode == kPrepTmix ? reinterpret_cast<const void*>(&wkv7_prep_kernel<kPrepTmix>)
                                            : reinterpret_cast<const void*>(&wkv7_prep_kernel<kPrepPlain>);
  const void* scan_fn = reinterpret_cast<const void*>(&wkv7_scan_kernel);
  const int prep_lds = kPrepWaves * kPrepLdsPerWave;
  const int scan_lds = kScanLds;
  static const hipError_t a0 = hipFuncSetAttribute(reinterpret_cast<const void*>(&wkv7_prep_kernel<kPrepPlain>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, prep_lds);
  static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&wkv7_prep_kernel<kPrepTmix>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, prep_lds);
  static const hipError_t a2 = hipFuncSetAttribute(scan_fn, hipFuncAttributeMaxDynamicSharedMemorySize, scan_lds);
  if (a0 != hipSuccess) return a0;
  if (a1 != hipSuccess) return a1;
  if (a2 != hipSuccess) return a2;

  for (int64_t s = 0; s < nslab; ++s) {
    const int64_t c0 = s * slab;
    const int64_t ncs = (nch - c0 < slab) ? nch - c0 : slab;
    PrepParams pp = j.in;
    pp.rec = rec;
    pp.T = (int32_t)j.T;
    pp.H = (int32_t)j.H;
    pp.c0 = (int32_t)c0;
    pp.nc = (int32_t)ncs;
    pp.items = (int32_t)(units * ncs);
    void* pargs[] = {&pp};
    const uint32_t pblocks = (uint32_t)((units * ncs + kPrepWaves - 1) / kPrepWaves);
    e = hipLaunchKernel(prep_fn, dim3(pblocks), dim3(64 * kPrepWaves), pargs, prep_lds, j.stream);
    if (e != hipSuccess) return e;
    ScanParams sp{rec,
                  j.v,
                  j.y,
                  s == 0 ? j.s_in : carry,
                  s == nslab - 1 ? j.s_out : carry,
                  (int32_t)j.T,
                  (int32_t)j.H,
                  (int32_t)c0,
                  (int32_t)ncs};
    void* sargs[] = {&sp};
    e = hipLaunchKernel(scan_fn, dim3((uint32_t)(units * kWgPerHead)), dim3(kScanThreads), sargs, scan_lds,
                        j.stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Sum over the 64 lanes of a wave (every lane ends with the same bits).
__device__ __forceinline__ float wave_sum64(float x) {
  x = row16_sum(x);
  x = x + __shfl_xor(x, 16);
  x = x + __shfl_xor(x, 32);
  return x;
}

// ln_x in place on y [rows, 64] (a row is one token of one head): a GroupNorm with
// one group per head, mean and population variance over the 64 channels, then the
// per-channel affine. One wave per row, lane = channel.
constexpr float kGroupNormEps = 64e-5f;
__global__ __launch_bounds__(256) void tmix_ln_kernel(float* y, const float* ln_w, const float* ln_b, int64_t rows,
                                                      int32_t H) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const int h = (int)(row % H);
  float* yr = y + row * kN;
  const float v = yr[lane];
  const float mu = wave_sum64(v) * (1.f / kN);
  const float d = v - mu;
  const float var = wave_sum64(d * d) * (1.f / kN);
  const float o = d * (1.f / sqrtf(var + kGroupNormEps));
  const float gw = ln_w ? ln_w[h * kN + lane] : 1.f;
  const float gb = ln_b ? ln_b[h * kN + lane] : 0.f;
  yr[lane] = fmaf(o, gw, gb);
}

}  // namespace

hipError_t launch_chunked_split(const WkvCall& c) {
  if (c.dtype != 1) return hipErrorNotSupported;  // bfloat16 inputs only
  PrepParams in{};
  in.r = static_cast<const uint16_t*>(c.in[0]);
  in.w = static_cast<const uint16_t*>(c.in[1]);
  in.k = static_cast<const uint16_t*>(c.in[2]);
  in.a = static_cast<const uint16_t*>(c.in[4]);
  in.b = static_cast<const uint16_t*>(c.in[5]);
  SplitJob j{in, kPrepPlain, static_cast<const uint16_t*>(c.in[3]), c.y, static_cast<const float*>(c.s_in),
             static_cast<float*>(c.s_out), c.B, c.T, c.H, c.stream};
  return run_split(j);
}

hipError_t launch_tmix_chunked(const TmixCall& c) {
  if (c.dtype != 1) return hipErrorNotSupported;  // bfloat16 inputs only
  const TmixParams& t = c.p;
  PrepParams in{};
  in.r = static_cast<const uint16_t*>(t.r);
  in.w_raw = t.w_raw;
  in.k = static_cast<const uint16_t*>(t.k);
  in.a = static_cast<const uint16_t*>(t.kk);
  in.b = static_cast<const uint16_t*>(t.a_lr);
  // the scan writes y into out; ln_x then normalises it in place
  SplitJob j{in, kPrepTmix, static_cast<const uint16_t*>(t.v), t.out, t.s_in, t.s_out, c.B, t.T, c.H, c.stream};
  hipError_t e = run_split(j);
  if (e != hipSuccess) return e;
  const int64_t rows = c.B * t.T * c.H;
  float* out = t.out;
  const float* lw = t.ln_w;
  const float* lb = t.ln_b;
  int64_t nrows = rows;
  int32_t h32 = (int32_t)c.H;
  void* args[] = {&out, &lw, &lb, &nrows, &h32};
  return hipLaunchKernel(reinterpret_cast<const void*>(&tmix_ln_kernel), dim3((uint32_t)((rows + 3) / 4)),
                         dim3(256), args, 0, c.stream);
}

}  // namespace rwkv7
