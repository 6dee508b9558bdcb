// Chunk algebra of the chunked WKV-7 prefill, shared by the split kernels
// (prep and scan as two launches, records in device memory) and the fused kernel
// (both roles in one workgroup per head, records in an LDS ring).
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
// Everything except S0 and V is a function of the chunk's own r, w, k, a, b: the
// "prep" of a chunk forms it as one record; the "scan" carries the state through
// the records in order.
//
// Numerics. Decay factors are running products of w (clamped below at 2^-15).
// The Gram factors pass through the decay at token 7 (Gq_t = e^{gamma_t - gamma_7}),
// so no factor exceeds w_min^-8; e^{gamma_t} = Gq_t e^{gamma_7} (e^{gamma_7} >= 2^-120
// is a normal float). The Grams are products of bfloat16 hi/lo halves (hi*hi + hi*lo +
// lo*hi, about 2^-16 relative, with the float32 range) with float32 accumulation (float32
// 16x16x4 products measured slower: the prep then holds the matrix pipe that its SIMD's
// scan wave needs); T and M_r are float32; A', R', G_u, G_y, B-, K-, the state operand and U are rounded once to
// float16 as MFMA operands (float32 accumulation), so magnitudes must stay below 2^15.
// The carried state is float32 throughout.
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
//
// One MFMA instruction per dependent chain. When an MFMA takes the result of the
// MFMA just before it as its accumulator (the same registers), the compiler issues it
// with no wait in between, whatever the two instructions are; chains of one
// instruction are exact that way, but chains that mixed 16x16x32 and 16x16x16 f16
// products gave wrong values on gfx950 in the product placed second. The wrappers
// below therefore come in three families, each with its own operand types and its
// own accumulator type (Acc<family>): Mma16 (16x16x16 f16, half4 operands: the
// prep's transposes and 16-token products), MmaBF (16x16x32 bf16, bf16x8 operands:
// the prep's Grams) and Mma32 (16x16x32 f16, half8 operands: the scan). A result of
// one family can reach another family's product only through an explicit .v (as a
// converted operand, or after a vector-unit addition), never as its accumulator by
// accident.
#pragma once

#include "wkv7_device.hpp"

namespace rwkv7 {
namespace chunk {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kC = 16;  // tokens per chunk
constexpr float kWMin = 0x1p-15f;

// Record of one (head, chunk): nine 1 KiB fragment blocks (16 bytes per lane),
// then e^{gamma_15} for the 64 key columns.
enum { kRecA0 = 0, kRecA1 = 1, kRecR0 = 2, kRecR1 = 3, kRecG = 4, kRecBK = 5, kRecBlocks = 9 };
constexpr int kRecD = kRecBlocks * 1024;
constexpr int kRecBytes = kRecD + kN * 4;  // 9472

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
// A 16x16 float32 accumulator tile of one MFMA family, in the D layout (element e of
// lane (li, g) is row 4g + e, column li).
enum { kFam16 = 0, kFamBF = 1, kFam32 = 2 };
template <int FAMILY>
struct Acc {
  f32x4 v;
};
// 16x16x16 f16 family (the prep's transposes and 16-token products)
struct Mma16 {
  typedef Acc<kFam16> acc;
  __device__ static __forceinline__ acc zero() { return acc{zero4()}; }
  __device__ static __forceinline__ acc mma(half4 a, half4 b, acc c) {
    return acc{__builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c.v, 0, 0, 0)};
  }
};
// 16x16x32 f16 family (the scan)
struct Mma32 {
  typedef Acc<kFam32> acc;
  __device__ static __forceinline__ acc zero() { return acc{zero4()}; }
  __device__ static __forceinline__ acc mma(half8 a, half8 b, acc c) {
    return acc{__builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c.v, 0, 0, 0)};
  }
};
// 16x16x32 bf16 family (the prep's Grams, as products of bfloat16 hi / lo halves)
struct MmaBF {
  typedef Acc<kFamBF> acc;
  __device__ static __forceinline__ acc zero() { return acc{zero4()}; }
  __device__ static __forceinline__ acc mma(bf16x8 a, bf16x8 b, acc c) {
    return acc{__builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c.v, 0, 0, 0)};
  }
};
__device__ __forceinline__ half4 to_h4(f32x4 x) {
  return half4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}
template <int F>
__device__ __forceinline__ half4 to_h4(const Acc<F>& x) {
  return to_h4(x.v);
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
__device__ __forceinline__ float4 lds4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float el(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// ============================================================================ prep

// Inputs of the prep. The plain recurrence takes r, w, k, a, b (bfloat16). The fused
// time-mix operator takes r, k (bfloat16), w_raw (float32) in place of w, and kk,
// a_lr in place of a, b; the prep then forms w = exp(-exp(w_raw)), the unit key
// kk^ = kk / max(|kk|, 1e-12) over the head's 64 channels, a = -kk^ and b = kk^ a_lr.
constexpr int kPrepPlain = 0, kPrepTmix = 1;
struct PrepIn {
  const uint16_t* r;
  const uint16_t* w;   // plain: the decay
  const float* w_raw;  // time-mix: the decay's log-log form
  const uint16_t* k;
  const uint16_t* a;   // plain: a; time-mix: kk
  const uint16_t* b;   // plain: b; time-mix: a_lr
  int32_t T, H;
};

constexpr int kFacRow = kN + 4;  // padded float row: token-layout reads of one row spread over the banks
// Factor rows (float32, [row][key]), written in the key layout (lane = key j):
//   row t + 1 = Gq_t = e^{gamma_t - gamma_7},  t = -1..15;   row kRowE7 = e^{gamma_7}.
// e^{gamma_t} = Gq_t e^{gamma_7}, e^{gamma_7 - gamma_t} = 1 / Gq_t and
// e^{gamma_15 - gamma_t} = Gq_15 / Gq_t are formed where they are used.
constexpr int kRowE7 = 17, kFacRows = 18;
constexpr int kFacBytes = kFacRows * kFacRow * 4;  // 4,896 bytes
// After the factors are consumed the same area holds L_ab ([t][s], float32), the
// right-hand sides of the solve (the identity, then L_rb, [32][16] float32) and the
// rows of T and M_r (float16).
constexpr int kLabOff = 0, kRhsOff = 16 * 16, kTmOffBytes = 3 * 16 * 16 * 4;
constexpr int kPrepScratch = kFacBytes > kTmOffBytes + 2 * 16 * 16 * 2 ? kFacBytes : kTmOffBytes + 2 * 16 * 16 * 2;
// In the fused kernel the scratch sits at the start of the chunk's own record slot:
// it must end before the first record block that the prep writes while the factors
// are still read (B- and K-, and e^{gamma_15}), and the products that overwrite it
// are written only after T and M_r have been read into registers.
static_assert(kPrepScratch <= kRecBK * 1024, "prep scratch overlaps the B-/K- blocks");

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// x = hi + lo with both halves bfloat16 (round to nearest even): 16 significant bits and
// the float32 exponent range, which the Gram operands need (factors up to w_min^-8).
// Two values at a time (elements i, i + 1 of the operands): one packed conversion for
// both high halves, the exact widening of each (a shift, a mask), the two remainders,
// one packed conversion for both low halves.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, bf16x8& hi, bf16x8& lo, int i) {
  const bf16x2 h = __builtin_convertvector(f32x2{x0, x1}, bf16x2);
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const f32x2 r{x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u)};
  const bf16x2 l = __builtin_convertvector(r, bf16x2);
  hi[i] = h[0];
  hi[i + 1] = h[1];
  lo[i] = l[0];
  lo[i + 1] = l[1];
}
// An ordering point for the values in x and for memory: the compiler computes x
// before it and issues no later memory access ahead of it.
__device__ __forceinline__ void pin16(float (&x)[16]) {
  asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]),
               "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]), "+v"(x[14]), "+v"(x[15])
               :
               : "memory");
}

// Loads of streamed input (read once per pass, each load instruction covering whole 128-byte
// lines): the non-temporal hint keeps them from displacing cached data. Measured on the
// one-kernel prefill with r, a, b, k and then w loaded this way: D4096-long 0.966 -> 0.938 ->
// 0.924 ms, L24-D1024 0.279 -> 0.251 -> 0.245 ms, L12-D768 0.215 -> 0.194 -> 0.191 ms. (The scan
// waves' v and y, each line shared by the four scan waves, lost with the hint.)
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const u4v q = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
  return make_uint4(q[0], q[1], q[2], q[3]);
}

// the same for one bfloat16 (a whole 128-byte token row per load instruction)
__device__ __forceinline__ uint32_t ld_stream2(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

// Raw inputs of one (head, chunk) in registers. Token layout for r, a, b, k: lane
// (t = li, g) holds keys 16kt + 4g .. + 3 of token t; key layout for w: lane = key j,
// all 16 tokens. Past-the-end tokens read token nt - 1 (masked in prep_compute).
struct PrepRaw {
  uint2 rr[4], ar[4], br[4], kr[4];
  uint32_t wr[kC];  // plain: bfloat16 bits; time-mix: float32 bits of w_raw
  int nt;           // live tokens, 1..16
};

// Issues the loads of chunk (bb, h, first token t0). base: element offset of token t0.
template <int MODE>
__device__ __forceinline__ void prep_load(const PrepIn& p, int64_t base, int nt, PrepRaw& x) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
  const uint32_t tstride = (uint32_t)p.H * kN;  // elements between tokens
  const int tl = min(li, nt - 1);
  x.nt = nt;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const uint32_t off = (uint32_t)(tl * tstride + 16 * kt + 4 * g) * 2u;
    x.rr[kt] = ld_off<uint2>(p.r + base, off);
    x.ar[kt] = ld_off<uint2>(p.a + base, off);
    x.br[kt] = ld_off<uint2>(p.b + base, off);
    x.kr[kt] = ld_off<uint2>(p.k + base, off);
  }
#pragma unroll
  for (int t = 0; t < kC; ++t) {
    const int tt = min(t, nt - 1);
    if constexpr (MODE == kPrepTmix)
      x.wr[t] = __float_as_uint(ld_off<float>(p.w_raw + base, (uint32_t)(tt * tstride + lane) * 4u));
    else
      x.wr[t] = ld_stream2(reinterpret_cast<const char*>(p.w + base) + (uint32_t)(tt * tstride + lane) * 2u);
  }
}

// Row-coalesced loading of r, a, b, k: lane l loads the 16-byte piece l % 8 (keys
// 8 (l % 8) .. + 7) of token l / 8 + 8 h of each tensor, so the 16 lanes of a
// quarter-wave read two whole 128-byte token rows instead of one 8-byte piece of
// 16 rows. The pieces then pass through LDS (prep_rows_to_raw) into the token layout.
// w is loaded in the key layout as by prep_load (whole rows already).
struct PrepRows {
  uint4 q[4][2];  // r, a, b, k; h = 0, 1
  uint4 wq[2];    // w (bfloat16) in the same form, when the caller takes w with the rows
};
constexpr int kStageRow = 144;             // bytes per staged token row (128 + 16: 16-byte aligned, and rows
                                           // 8 apart share banks, so the token-layout reads conflict 2-way)
constexpr int kStageT = kC * kStageRow;    // one tensor: 2,304 bytes
constexpr int kStageBytes = 4 * kStageT;   // 9,216 bytes
static_assert(kStageBytes <= kRecD, "staged rows end before e^gamma_15");

// Which of r, a, b, k a caller needs (bit q of a row mask: r = 1, a = 2, b = 4, k = 8).
// A form of the prep that never reads a tensor skips its loads and staging; its
// registers then hold zeros.
enum : unsigned { kRowR = 1u, kRowA = 2u, kRowB = 4u, kRowK = 8u, kRowsAll = 15u };

// r, a, b, k rows of chunk (base, nt)
// W: also w (plain bfloat16 form), so that its latency passes with the rows'.
template <unsigned ROWS = kRowsAll, bool W = false>
__device__ __forceinline__ void prep_load_rows(const PrepIn& p, int64_t base, int nt, PrepRows& rows) {
  const int lane = threadIdx.x & 63;
  const uint32_t tstride = (uint32_t)p.H * kN;
  const uint16_t* src[4] = {p.r, p.a, p.b, p.k};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tok = min((lane >> 3) + 8 * h, nt - 1);
    const uint32_t off = (uint32_t)(tok * tstride + 8 * (lane & 7)) * 2u;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      rows.q[q][h] =
          (ROWS >> q) & 1u ? ld_stream16(reinterpret_cast<const char*>(src[q] + base) + off) : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (W) rows.wq[h] = ld_stream16(reinterpret_cast<const char*>(p.w + base) + off);
  }
}
// w of chunk (base, nt) in the key layout
template <int MODE>
__device__ __forceinline__ void prep_load_w(const PrepIn& p, int64_t base, int nt, PrepRaw& x) {
  const int lane = threadIdx.x & 63;
  const uint32_t tstride = (uint32_t)p.H * kN;
  x.nt = nt;
#pragma unroll
  for (int t = 0; t < kC; ++t) {
    const int tt = min(t, nt - 1);
    if constexpr (MODE == kPrepTmix)
      x.wr[t] = __float_as_uint(ld_off<float>(p.w_raw + base, (uint32_t)(tt * tstride + lane) * 4u));
    else
      x.wr[t] = ld_stream2(reinterpret_cast<const char*>(p.w + base) + (uint32_t)(tt * tstride + lane) * 2u);
  }
}

// Writes the loaded rows to stage (kStageBytes of this wave's LDS) and reads them back
// in the token layout of PrepRaw.
template <unsigned ROWS = kRowsAll, bool W = false>
__device__ __forceinline__ void prep_rows_to_raw(const PrepRows& rows, unsigned char* stage, PrepRaw& x) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if ((ROWS >> q) & 1u)
        st_off<uint4>(stage, (uint32_t)(q * kStageT + ((lane >> 3) + 8 * h) * kStageRow + 16 * (lane & 7)),
                      rows.q[q][h]);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): every piece is in LDS before other lanes read it
  __builtin_amdgcn_wave_barrier();
  const uint2 z2 = make_uint2(0u, 0u);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const uint32_t off = (uint32_t)(li * kStageRow + 32 * kt + 8 * g);
    x.rr[kt] = ROWS & kRowR ? ld_off<uint2>(stage, 0 * kStageT + off) : z2;
    x.ar[kt] = ROWS & kRowA ? ld_off<uint2>(stage, 1 * kStageT + off) : z2;
    x.br[kt] = ROWS & kRowB ? ld_off<uint2>(stage, 2 * kStageT + off) : z2;
    x.kr[kt] = ROWS & kRowK ? ld_off<uint2>(stage, 3 * kStageT + off) : z2;
  }
  // every read has returned before the stage is overwritten
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
  if constexpr (W) {
    // w through the first tensor's stage, read back in the key layout (lane = key)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      st_off<uint4>(stage, (uint32_t)(((lane >> 3) + 8 * h) * kStageRow + 16 * (lane & 7)), rows.wq[h]);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < kC; ++t) x.wr[t] = ld_off<uint16_t>(stage, (uint32_t)(t * kStageRow + 2 * lane));
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
  }
}

// What the first phase of a chunk's prep hands to the second: the four Grams in the D
// layout, A^ (float16) and R^ (float32) in the token layout, and the identity operand.
struct PrepMid {
  MmaBF::acc Lab, Lak, Lrb, LrkT;
  half4 Ahat[4];
  f32x4 Rhat[4];
  half4 eye;
};

// The prep of one chunk from its raw inputs, in two phases (prep_grams, then
// prep_finish; prep_compute runs both), so that a caller can issue the loads of its
// next chunk in between. fac: kPrepScratch bytes of this wave's LDS. rec: the chunk's
// record (device memory or LDS); written as nine 1 KiB blocks, 16 bytes per lane, plus
// e^{gamma_15}. rec may hold fac at its start (see above).
//
// The decay factor rows of a chunk into fac (kFacBytes), e^{gamma_15} (64 floats) at
// e15; tokens past the end of the sequence become identity tokens in x.
template <int MODE>
__device__ __forceinline__ void prep_factors(PrepRaw& x, float* fac, unsigned char* e15) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int nt = x.nt;
  const bool live = li < nt;

  float wc[kC];
#pragma unroll
  for (int t = 0; t < kC; ++t) {
    float w;
    if constexpr (MODE == kPrepTmix)
      w = expf(-expf(__uint_as_float(x.wr[t])));
    else
      w = bfw(x.wr[t]);
    wc[t] = fmaxf(w, kWMin);  // clamp (a NaN decay becomes w_min)
  }
  // The last chunk of a sequence may run past its end: its tokens t >= nt become
  // identity tokens (w = 1, r = k = a = b = 0). The branch is the same for the whole wave.
  if (nt < kC) {
    const uint2 z2 = make_uint2(0u, 0u);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      x.rr[kt] = live ? x.rr[kt] : z2;
      x.ar[kt] = live ? x.ar[kt] : z2;
      x.br[kt] = live ? x.br[kt] : z2;
      x.kr[kt] = live ? x.kr[kt] : z2;
    }
#pragma unroll
    for (int t = 0; t < kC; ++t) wc[t] = t < nt ? wc[t] : 1.f;
  }

  // ---- decay factors (lane = j): Gq outward from token 7, so no factor exceeds
  // w_min^-8, and the plain running product for e^{gamma_7} and e^{gamma_15}
  {
    const int j = lane;
    float e = 1.f, gu = 1.f, gd = 1.f;
    fac[8 * kFacRow + j] = 1.f;  // Gq_7
#pragma unroll
    for (int q = 0; q < kC; ++q) {
      e *= wc[q];
      if (q == 7) fac[kRowE7 * kFacRow + j] = e;
      if (q < 8) {
        gu *= wc[8 + q];  // Gq_t, t = 8 + q: times w_t
        fac[(9 + q) * kFacRow + j] = gu;
        gd *= __builtin_amdgcn_rcpf(wc[7 - q]);  // Gq_t, t = 6 - q: divided by w_{t+1}
        fac[(7 - q) * kFacRow + j] = gd;
      }
    }
    st_off<float>(e15, (uint32_t)(4 * j), e);  // e^{gamma_15}
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the rows are in LDS before other lanes read them
  __builtin_amdgcn_wave_barrier();
}

// Phase 1: decay factors, operands, the four Grams; B-, K- and e^{gamma_15} stored.
// Y = false: a record for carrying the state alone (no readout): L_rb and L_rk are not
// formed (zero), so neither is anything of R' and G_y.
template <int MODE, bool Y = true>
__device__ __forceinline__ void prep_grams(PrepRaw& x, float* fac, unsigned char* rec, PrepMid& m) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
  prep_factors<MODE>(x, fac, rec + kRecD);

  // ---- token layout: operands, the four Grams and B-, K- (stored at once). Key 16kt + 4g + e
  // of the lane's token. Each Gram contracts 64 keys on 16x16x32 bfloat16 MFMAs as
  // hi*hi + hi*lo + lo*hi of the operands' bfloat16 halves (relative error about 2^-16),
  // two key blocks per product: K index 8g + 4(kt % 2) + e. The Grams land in the D layout:
  // lane (s = li, g) holds t = 4g + e; L_rk is formed transposed (operands swapped).
  // Identity as a B operand: B[k = 4g+e][n = li] = (4g + e == li).
  half4& eye = m.eye;
#pragma unroll
  for (int e = 0; e < 4; ++e) eye[e] = (_Float16)(4 * g + e == li ? 1.f : 0.f);
  const uint32_t lo = (uint32_t)lane * 16u;  // record blocks: 16 bytes per lane
  half4 (&Ahat)[4] = m.Ahat;
  f32x4 (&Rhat)[4] = m.Rhat;
  MmaBF::acc& Lab = m.Lab;
  MmaBF::acc& Lak = m.Lak;
  MmaBF::acc& Lrb = m.Lrb;
  MmaBF::acc& LrkT = m.LrkT;
  Lab = Lak = Lrb = LrkT = MmaBF::zero();
  bf16x8 ahH, ahL, rhH, rhL, bhH, bhL, khH, khL;
  // time-mix: 1 / max(|kk|, 1e-12) of this lane's token (its 64 channels are spread over
  // the four lanes li, li + 16, li + 32, li + 48)
  float inv = 1.f;
  if constexpr (MODE == kPrepTmix) {
    float n2 = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = bf4(x.ar[kt], e);
        n2 = fmaf(v, v, n2);
      }
    n2 += __shfl_xor(n2, 16);
    n2 += __shfl_xor(n2, 32);
    inv = 1.f / fmaxf(sqrtf(n2), 1e-12f);
  }
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int col = 16 * kt + 4 * g;
    const float4 gqm1 = lds4(&fac[li * kFacRow + col]);      // Gq_{t-1}
    const float4 gq = lds4(&fac[(li + 1) * kFacRow + col]);  // Gq_t
    const float4 g15 = lds4(&fac[16 * kFacRow + col]);       // Gq_15
    const float4 e7 = lds4(&fac[kRowE7 * kFacRow + col]);    // e^{gamma_7}
    const uint2 ra = x.ar[kt], rv2 = x.rr[kt], rb = x.br[kt], rk = x.kr[kt];
    half4 bbar, kbar;
    float ag[4], rg[4], bg[4], kg[4];
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
      // Gram operands: a and r scaled to token 7 from below, b and k from above
      ag[e] = av * el(gqm1, e);
      rg[e] = rv * el(gq, e);
      bg[e] = bv * f;
      kg[e] = kv * f;
      Ahat[kt][e] = (_Float16)(ag[e] * el(e7, e));  // a e^{gamma_{t-1}}
      Rhat[kt][e] = rg[e] * el(e7, e);              // r e^{gamma_t}
      bbar[e] = (_Float16)(bg[e] * el(g15, e));     // b e^{gamma_15 - gamma_t}
      kbar[e] = (_Float16)(kg[e] * el(g15, e));
    }
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const int q8 = 4 * (kt & 1) + e;
      split_bf16x2(ag[e], ag[e + 1], ahH, ahL, q8);
      split_bf16x2(rg[e], rg[e + 1], rhH, rhL, q8);
      split_bf16x2(bg[e], bg[e + 1], bhH, bhL, q8);
      split_bf16x2(kg[e], kg[e + 1], khH, khL, q8);
    }
    const half4 BT = to_h4(Mma16::mma(bbar, eye, Mma16::zero()));  // lane (j = li, g): B-[4g+e][16kt + li]
    const half4 KT = to_h4(Mma16::mma(kbar, eye, Mma16::zero()));
    st_off<half8>(rec, (kRecBK + kt) * 1024 + lo, cat8(BT, KT));
    if (kt & 1) {
      Lab = MmaBF::mma(ahH, bhH, Lab);
      Lak = MmaBF::mma(ahH, khH, Lak);
      if constexpr (Y) Lrb = MmaBF::mma(rhH, bhH, Lrb);
      if constexpr (Y) LrkT = MmaBF::mma(khH, rhH, LrkT);
      Lab = MmaBF::mma(ahH, bhL, Lab);
      Lak = MmaBF::mma(ahH, khL, Lak);
      if constexpr (Y) Lrb = MmaBF::mma(rhH, bhL, Lrb);
      if constexpr (Y) LrkT = MmaBF::mma(khH, rhL, LrkT);
      Lab = MmaBF::mma(ahL, bhH, Lab);
      Lak = MmaBF::mma(ahL, khH, Lak);
      if constexpr (Y) Lrb = MmaBF::mma(rhL, bhH, Lrb);
      if constexpr (Y) LrkT = MmaBF::mma(khL, rhH, LrkT);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = 4 * g + e;            // row of Lab, Lak, Lrb; column li is s
    Lab.v[e] = li < t ? Lab.v[e] : 0.f;     // strictly lower
    Lak.v[e] = li < t ? Lak.v[e] : 0.f;
    Lrb.v[e] = li <= t ? Lrb.v[e] : 0.f;    // lower with the diagonal
    LrkT.v[e] = t <= li ? LrkT.v[e] : 0.f;  // element (s = 4g+e, t = li) of L_rk^T
  }
}

// T = (I - L_ab)^{-1} and M_r = L_rb T of a chunk, by float32 back substitution in fac
// (the factor rows are no longer read). Returns them as float16 fragments: lane (li, g)
// holds T[li][4g + e] in tB and M_r[li][4g + e] in mB (T^T and M_r^T as B operands, T
// and M_r as A operands). Every LDS access of the solve has completed on return.
struct TmFrags {
  half4 tB, mB;
};
__device__ __forceinline__ TmFrags prep_solve(const MmaBF::acc Lab, const MmaBF::acc Lrb, float* fac) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;

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
    lab[(4 * g + e) * 16 + li] = Lab.v[e];
    rhs[(4 * g + e) * 16 + li] = 4 * g + e == li ? 1.f : 0.f;  // identity: the rows of T
    rhs[(16 + 4 * g + e) * 16 + li] = Lrb.v[e];               // L_rb: the rows of M_r
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  const int row = li;
  float xs[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = lds4(&rhs[((g & 1) * 16 + row) * 16 + 4 * q]);  // lanes 32-63 repeat lanes 0-31
#pragma unroll
    for (int e = 0; e < 4; ++e) xs[4 * q + e] = el(v, e);
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
    for (int s = 0; s < s2; ++s) xs[s] = fmaf(xs[s2], el(cur[s / 4], s % 4), xs[s]);
    pin16(xs);  // this step's updates before the next row's reads: one row in flight, not all
#pragma unroll
    for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
  }
  _Float16* tm = reinterpret_cast<_Float16*>(reinterpret_cast<unsigned char*>(fac) + kTmOffBytes);
  if (g < 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<half4*>(&tm[(g * 16 + row) * 16 + 4 * q]) =
          half4{(_Float16)xs[4 * q], (_Float16)xs[4 * q + 1], (_Float16)xs[4 * q + 2], (_Float16)xs[4 * q + 3]};
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  const half4 tB = *reinterpret_cast<const half4*>(&tm[li * 16 + 4 * g]);         // T[t = li][4g..]: T^T as B
  const half4 mB = *reinterpret_cast<const half4*>(&tm[(16 + li) * 16 + 4 * g]);  // M_r^T as B
  // T and M_r are in registers before any product overwrites the scratch (when the
  // scratch is the record's own start)
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
  return TmFrags{tB, mB};
}

// Phase 2: T, M_r and the products A', R', G_u, G_y, stored (Y = false: A' and G_u;
// G_y stored as zeros, R' not stored).
template <bool Y = true>
__device__ __forceinline__ void prep_finish(const PrepMid& m, float* fac, unsigned char* rec) {
  const int lane = threadIdx.x & 63;
  const uint32_t lo = (uint32_t)lane * 16u;
  const half4 eye = m.eye;
  const MmaBF::acc Lak = m.Lak, LrkT = m.LrkT;
  const TmFrags tm = prep_solve(m.Lab, m.Lrb, fac);
  const half4 tB = tm.tB, mB = tm.mB;

  // ---- products, stored per block. L_rk^T is added on the vector unit (a 16x16x32
  // Gram result is not fed to a 16x16x16 product as its accumulator). R^ comes from the
  // vector unit, so it may start a 16x16x16 chain.
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
    half4 ApT[2], RpT[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kt = 2 * kp + u;
      const half4 AT = to_h4(Mma16::mma(m.Ahat[kt], eye, Mma16::zero()));  // lane (j = li, g): A^[4g+e][16kt + li]
      ApT[u] = to_h4(Mma16::mma(AT, tB, Mma16::zero()));                   // lane (t = li, g): A'[t][16kt + 4g + e]
      if constexpr (Y) RpT[u] = to_h4(Mma16::mma(AT, mB, Mma16::acc{m.Rhat[kt]}));  // R'[t][16kt + 4g + e]
    }
    st_off<half8>(rec, (kRecA0 + kp) * 1024 + lo, cat8(ApT[0], ApT[1]));
    if constexpr (Y) st_off<half8>(rec, (kRecR0 + kp) * 1024 + lo, cat8(RpT[0], RpT[1]));
  }
  const half4 LakH = to_h4(Lak);  // as an A operand: L_ak^T (M = s', K = s)
  const half4 GuT = to_h4(Mma16::mma(LakH, tB, Mma16::zero()));          // lane (t = li, g): G_u[t][4g + e]
  half4 GyT = half4{(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
  if constexpr (Y) GyT = to_h4(Mma16::mma(LakH, mB, Mma16::zero()).v + LrkT.v);  // G_y[t][4g + e]
  st_off<half8>(rec, kRecG * 1024 + lo, cat8(GuT, GyT));
}

template <int MODE>
__device__ __forceinline__ void prep_compute(PrepRaw& x, float* fac, unsigned char* rec) {
  PrepMid m;
  prep_grams<MODE>(x, fac, rec, m);
  prep_finish(m, fac, rec);
}

// ============================================================================ scan

// Fragments of one chunk as a scan wave consumes them.
struct Frag {
  half8 a0, a1, r0, r1, gl, bk[4];
  float dv;       // e^{gamma_15} of key 16 (li / 4) + 4g + li % 4: lane 4kt + e of row g holds the
                  // decay that every lane of the row needs as its (kt, e) element
  uint32_t v[4];  // V[t = 4g + e][i = the wave's row li], raw bfloat16 bits (widened when used)
};

// Reads v of a chunk from LDS into f.v. vrow: [token][vcols] bfloat16, at this wave's
// first value column.
__device__ __forceinline__ void read_v(const uint16_t* vrow, int vcols, Frag& f) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) f.v[e] = vrow[(4 * g + e) * vcols + li];
}
// Reads a chunk's record fragments (not v) from its record in LDS.
__device__ __forceinline__ void read_frag(const unsigned char* slot, Frag& f) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
  const uint32_t lo = (uint32_t)lane * 16u;
  // in the order of use (the next chunk's first products take v and G)
  f.gl = *reinterpret_cast<const half8*>(slot + kRecG * 1024 + lo);
  f.a0 = *reinterpret_cast<const half8*>(slot + kRecA0 * 1024 + lo);
  f.r0 = *reinterpret_cast<const half8*>(slot + kRecR0 * 1024 + lo);
  f.a1 = *reinterpret_cast<const half8*>(slot + kRecA1 * 1024 + lo);
  f.r1 = *reinterpret_cast<const half8*>(slot + kRecR1 * 1024 + lo);
  f.dv = *reinterpret_cast<const float*>(slot + kRecD + (16 * (li >> 2) + 4 * g + (li & 3)) * 4);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) f.bk[kt] = *reinterpret_cast<const half8*>(slot + (kRecBK + kt) * 1024 + lo);
}

// Every lane of a row of 16 reads lane K of that row (DPP row broadcast).
template <int K>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + K, 0xf, 0xf, false));
}

// One chunk of the scan for 16 value rows. St: the state in the D layout, element e of
// St[kt] = S[i = row li][j = 16kt + 4g + e]. Returns Y transposed: lane (t = li, g) holds
// y[t][i = 4g + e] of the wave's 16 rows.
//   U = A' S0^T + G_u V and Y = R' S0^T + G_y V: two key halves, then the G V term
//   (the record's G block holds G_u | G_y, so a B operand of V | 0 or 0 | V selects one
//   of them); S^T <- diag(e^{gamma_15}) S^T + [B- | K-] [U ; V] per key tile.
// Every product is 16x16x32 f16 (one shape for the whole dependent chain). The G V terms
// come first: they do not depend on the state, so they need not wait for the previous
// chunk's update. Y is formed transposed (operands swapped: the state and V fragments
// serve as A operands, R' and G as B operands, from the same registers).
// Y = false skips the readout (the state alone is carried; zero is returned).
template <bool Y = true>
__device__ __forceinline__ f32x4 scan_step(Mma32::acc (&St)[4], const Frag& f) {
  const half4 hz = half4{(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
  half4 vB;
#pragma unroll
  for (int e = 0; e < 4; ++e) vB[e] = (_Float16)bfw(f.v[e]);
  Mma32::acc u = Mma32::mma(f.gl, cat8(vB, hz), Mma32::zero());
  Mma32::acc yv = Mma32::zero();
  if constexpr (Y) yv = Mma32::mma(cat8(hz, vB), f.gl, yv);
  const half8 sB0 = cat8(to_h4(St[0]), to_h4(St[1]));
  const half8 sB1 = cat8(to_h4(St[2]), to_h4(St[3]));
  u = Mma32::mma(f.a0, sB0, u);
  if constexpr (Y) yv = Mma32::mma(sB0, f.r0, yv);
  u = Mma32::mma(f.a1, sB1, u);
  if constexpr (Y) yv = Mma32::mma(sB1, f.r1, yv);
  const half8 uv = cat8(to_h4(u), vB);
  // the decays by row broadcasts (one 4-byte LDS read per lane instead of four 16-byte ones)
  St[0].v[0] *= row_bcast<0>(f.dv);
  St[0].v[1] *= row_bcast<1>(f.dv);
  St[0].v[2] *= row_bcast<2>(f.dv);
  St[0].v[3] *= row_bcast<3>(f.dv);
  St[0] = Mma32::mma(f.bk[0], uv, St[0]);
  St[1].v[0] *= row_bcast<4>(f.dv);
  St[1].v[1] *= row_bcast<5>(f.dv);
  St[1].v[2] *= row_bcast<6>(f.dv);
  St[1].v[3] *= row_bcast<7>(f.dv);
  St[1] = Mma32::mma(f.bk[1], uv, St[1]);
  St[2].v[0] *= row_bcast<8>(f.dv);
  St[2].v[1] *= row_bcast<9>(f.dv);
  St[2].v[2] *= row_bcast<10>(f.dv);
  St[2].v[3] *= row_bcast<11>(f.dv);
  St[2] = Mma32::mma(f.bk[2], uv, St[2]);
  St[3].v[0] *= row_bcast<12>(f.dv);
  St[3].v[1] *= row_bcast<13>(f.dv);
  St[3].v[2] *= row_bcast<14>(f.dv);
  St[3].v[3] *= row_bcast<15>(f.dv);
  St[3] = Mma32::mma(f.bk[3], uv, St[3]);
  return yv.v;
}

// ====================================================================== checkpoints
// A 64x64 state (or state gradient) in float16, [row i][key j], stored in the order
// in which MFMA fragments read it: row-major over rows, and within a row the 64 keys
// as [kp][g][h][e] with key = 16 (2 kp + h) + 4 g + e. Lane (li, g) of a wave that owns
// rows i0 .. i0 + 15 (element e of tile kt holding key 16 kt + 4 g + e of row i0 + li)
// writes and reads its 8 keys of each kp as one 16-byte piece.
constexpr int kCkHalves = kN * kN;  // 8 KiB per state
__device__ __forceinline__ uint32_t ck_off(int row, int kp, int g) { return (uint32_t)(row * kN + kp * 32 + g * 8); }
template <int F>
__device__ __forceinline__ void ck_store(_Float16* dst, int i0, const Acc<F> (&tile)[4]) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kp = 0; kp < 2; ++kp)
    *reinterpret_cast<half8*>(dst + ck_off(i0 + li, kp, g)) = cat8(to_h4(tile[2 * kp]), to_h4(tile[2 * kp + 1]));
}

}  // namespace chunk
}  // namespace rwkv7
