// Chunked reverse-mode derivatives of the WKV-7 recurrence, on MFMA. Training runs
// the wkv7 operator (RWKV-7 G0 7.2B notes, lshu.cn/news/198401, section 7.2); the
// pages give only its forward formula (section 7.1), so what follows differentiates
// the chunk form of the forward (the algebra of wkv7_chunk_ops.hpp).
//
// Per chunk of 16 tokens, with the chunk's start state S0 and G = dL/dS at the chunk's
// end, and U = T (A^ S0^T + L_ak V) the chunk's S_{t-1} a_t (value rows as columns):
//   dU = L_rb^T dY + B- G^T              dX = T^T dU
//   dL/dS0 (the G of the previous chunk's end):  G0^T = diag(e^{gamma_15}) G^T + R^^T dY + A^^T dX
// and the input gradients of the chunk follow from dY, dX, U, V, S0 and G (kernel 3).
// The decay's gradient uses the invariance of the recurrence under a shift of the
// cumulative log decay gamma: the result depends on gamma only through r e^{gamma_t},
// a e^{gamma_{t-1}}, b e^{-gamma_t}, k e^{-gamma_t} and the chunk's end state
// S_end = S0 e^{gamma_15} + ..., so with the input gradients dr, da, db, dk,
//   dgamma_t = r_t dr_t - b_t db_t - k_t dk_t + a_{t+1} da_{t+1}   (t < 15, within the chunk)
//   dgamma_15 also gets sum_i S_end[i,j] G[i,j]
//   dlog w_u = sum_{t >= u} dgamma_t (within the chunk),   dw = dlog w / w.
//
// Three kernels:
//   1. the one-kernel chunked prefill in its checkpoint form stores the float16 state at
//      every chunk start (wkv7_fused.hpp);
//   2. the chain, one workgroup per head: prep waves rebuild each chunk's chain record
//      (B-, L_rb^T, T^T, [R^^T | A^^T], e^{gamma_15}) into an LDS ring, last chunk
//      first; scan waves carry G in float32 back through the chunks, store each chunk's
//      end G (float16) and finally dL/dS_0.
//   1 and 2 need only the inputs and dY, so one launch (wkv7_bpass_kernel) runs both,
//   a workgroup per head for each;
//   3. wkv7_bgrad_kernel, one wave per (head, chunk) over the whole chip, forms the
//      chunk's input gradients from its inputs, dY, S0 and end G.
#include <cstdint>

#include "wkv7_chunk_ops.hpp"
#include "wkv7_fused.hpp"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

using namespace chunk;

// ============================================================================ chain

// Chain record of one chunk: eleven 1 KiB fragment blocks (16 bytes per lane), then
// e^{gamma_15} for the 64 keys. Blocks 0-1 are written after the solve (they overlap
// the prep's scratch); the others while the factors are still read, past the scratch.
enum { kCbLrb = 0, kCbTt = 1, kCbBb0 = 5, kCbBb1 = 6, kCbRa = 7, kCbBlocks = 11 };
constexpr int kCbG = kCbBlocks * 1024;
constexpr int kCbBytes = kCbG + kN * 4;  // 11,520
static_assert(kPrepScratch <= kCbBb0 * 1024, "prep scratch overlaps the blocks written during the Gram phase");
static_assert(kStageBytes <= kCbG, "staged rows end before e^gamma_15");

// What the chain waves read of a record.
struct CFrag {
  half8 bb0, bb1;  // B- as A operands: lane (tau = li, g), keys of key pair 0 / 1 (K order of the G tiles)
  half8 lrb;       // L_rb^T as an A operand (m = tau, k = t), K half 2 zero
  half8 tt;        // T^T as an A operand (m = t, k = tau), K half 2 zero
  half8 ra[4];     // per key tile: [R^^T | A^^T] (m = key, k = t of dY | t of dX)
  float dv;        // e^{gamma_15} of key 16 (li / 4) + 4g + li % 4 (spread by row broadcasts)
};

__device__ __forceinline__ void read_cfrag(const unsigned char* slot, CFrag& f) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
  const uint32_t lo = (uint32_t)lane * 16u;
  f.bb0 = *reinterpret_cast<const half8*>(slot + kCbBb0 * 1024 + lo);
  f.bb1 = *reinterpret_cast<const half8*>(slot + kCbBb1 * 1024 + lo);
  f.lrb = *reinterpret_cast<const half8*>(slot + kCbLrb * 1024 + lo);
  f.tt = *reinterpret_cast<const half8*>(slot + kCbTt * 1024 + lo);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) f.ra[kt] = *reinterpret_cast<const half8*>(slot + (kCbRa + kt) * 1024 + lo);
  f.dv = *reinterpret_cast<const float*>(slot + kCbG + (16 * (li >> 2) + 4 * g + (li & 3)) * 4);
}

// The chain record of a chunk from its raw inputs (bfloat16 r, w, a, b), built in the
// record's own slot: fac (the factor rows, then the solve) at its start.
__device__ __forceinline__ void chain_prep(PrepRaw& x, unsigned char* rec) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
  const uint32_t lo = (uint32_t)lane * 16u;
  float* fac = reinterpret_cast<float*>(rec);
  prep_factors<kPrepPlain>(x, fac, rec + kCbG);
  half4 eye;
#pragma unroll
  for (int e = 0; e < 4; ++e) eye[e] = (_Float16)(4 * g + e == li ? 1.f : 0.f);
  const half4 hz = half4{(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
  MmaBF::acc Lab = MmaBF::zero(), Lrb = MmaBF::zero();
  bf16x8 ahH, ahL, rhH, rhL, bhH, bhL;
  half4 bbar[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int col = 16 * kt + 4 * g;
    const float4 gqm1 = lds4(&fac[li * kFacRow + col]);      // Gq_{t-1}
    const float4 gq = lds4(&fac[(li + 1) * kFacRow + col]);  // Gq_t
    const float4 g15 = lds4(&fac[16 * kFacRow + col]);       // Gq_15
    const float4 e7 = lds4(&fac[kRowE7 * kFacRow + col]);    // e^{gamma_7}
    half4 ahat, rhat;
    float ag[4], rg[4], bg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float av = bf4(x.ar[kt], e), bv = bf4(x.br[kt], e), rv = bf4(x.rr[kt], e);
      ag[e] = av * el(gqm1, e);                                // a e^{gamma_{t-1} - gamma_7}
      rg[e] = rv * el(gq, e);                                  // r e^{gamma_t - gamma_7}
      bg[e] = bv * __builtin_amdgcn_rcpf(el(gq, e));           // b e^{gamma_7 - gamma_t}
      ahat[e] = (_Float16)(ag[e] * el(e7, e));                 // A^ = a e^{gamma_{t-1}}
      rhat[e] = (_Float16)(rg[e] * el(e7, e));                 // R^ = r e^{gamma_t}
      bbar[kt][e] = (_Float16)(bg[e] * el(g15, e));            // B- = b e^{gamma_15 - gamma_t}
    }
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const int q8 = 4 * (kt & 1) + e;
      split_bf16x2(ag[e], ag[e + 1], ahH, ahL, q8);
      split_bf16x2(rg[e], rg[e + 1], rhH, rhL, q8);
      split_bf16x2(bg[e], bg[e + 1], bhH, bhL, q8);
    }
    // [R^^T | A^^T] of key tile kt: lane (key 16kt + li, g) holds tokens 4g + e
    const half4 RT = to_h4(Mma16::mma(rhat, eye, Mma16::zero()));
    const half4 AT = to_h4(Mma16::mma(ahat, eye, Mma16::zero()));
    st_off<half8>(rec, (kCbRa + kt) * 1024 + lo, cat8(RT, AT));
    if (kt & 1) {
      st_off<half8>(rec, (kCbBb0 + (kt >> 1)) * 1024 + lo, cat8(bbar[kt - 1], bbar[kt]));
      Lab = MmaBF::mma(ahH, bhH, Lab);
      Lrb = MmaBF::mma(rhH, bhH, Lrb);
      Lab = MmaBF::mma(ahH, bhL, Lab);
      Lrb = MmaBF::mma(rhH, bhL, Lrb);
      Lab = MmaBF::mma(ahL, bhH, Lab);
      Lrb = MmaBF::mma(rhL, bhH, Lrb);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = 4 * g + e;          // row of Lab and Lrb; column li is s
    Lab.v[e] = li < t ? Lab.v[e] : 0.f;   // strictly lower
    Lrb.v[e] = li <= t ? Lrb.v[e] : 0.f;  // lower with the diagonal
  }
  const TmFrags tm = prep_solve(Lab, Lrb, fac);
  // T^T as an A operand: the transpose of T's rows (lane (li, g) holds T[li][4g + e])
  const half4 TT = to_h4(Mma16::mma(tm.tB, eye, Mma16::zero()));
  st_off<half8>(rec, kCbTt * 1024 + lo, cat8(TT, hz));
  st_off<half8>(rec, kCbLrb * 1024 + lo, cat8(to_h4(Lrb), hz));  // lane (tau = li, g): L_rb[4g + e][tau]
}

// The chain's workgroup has the shape of the one-kernel prefill's (fused::kScanW scan
// waves, fused::kPrepW prep waves, the same hand-off and bounded waits), with a ring of
// chain records.
using fused::kScanW;
using fused::kPrepW;
using fused::kRing;
using fused::kThreads;
using fused::post;
using fused::wait_all_at_least;
using fused::wait_at_least;
constexpr int kCtrlOff = kRing * kCbBytes;
constexpr int kLds = kCtrlOff + 4 * (kRing + kScanW);
static_assert(kLds <= 160 * 1024, "LDS per compute unit");

struct ChainParams {
  PrepIn in;           // r, w, k, a, b (bfloat16), T, H
  const float* dy;     // [B, T, H, 64]
  const float* ds_out; // [B, H, 64, 64] or null (zero)
  float* ds_in;        // [B, H, 64, 64] or null
  _Float16* gend;      // [B*H][nc] float16 G at every chunk's end (fragment order)
  int32_t nc;
};

// Chunks are taken last first: step q handles chunk nc - 1 - q. The hand-off is that
// of the one-kernel prefill (wkv7_fused.hip): ready[slot] = the last step whose record
// is complete there, consumed[w] = the steps whose fragments scan wave w holds; the
// smallest unfinished step never waits on a later one, and every wait is bounded.
__device__ __forceinline__ void chain_body(const ChainParams& p, unsigned char* ring, int unit) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int H = p.in.H, T = p.in.T, nc = p.nc;
  const int bb = unit / H, hh = unit % H;
  const uint32_t tstride = (uint32_t)H * kN;
  const int64_t seq_base = (int64_t)bb * T * H * kN + (int64_t)hh * kN;
  int* ready = reinterpret_cast<int*>(ring + kCtrlOff);
  int* consumed = ready + kRing;
  if (threadIdx.x < kRing) ready[threadIdx.x] = -1;
  if (threadIdx.x < kScanW) consumed[threadIdx.x] = 0;
  __syncthreads();
  auto slot_of = [&](int q) { return ring + (q % kRing) * kCbBytes; };

  if (wave >= kScanW) {
    // ---------------------------------------------------------------- prep waves
    const int q0 = wave - kScanW;
    if (q0 >= nc) return;
    const int last = q0 + (nc - 1 - q0) / kPrepW * kPrepW;
    auto nt_of = [&](int q) { return min(kC, T - (nc - 1 - q) * kC); };
    auto base_of = [&](int q) { return seq_base + (int64_t)(nc - 1 - q) * kC * tstride; };
    auto item = [&](int& q, PrepRows& cur, PrepRows& nxt) {
      unsigned char* rec = slot_of(q);
      PrepRaw x;
      prep_load_w<kPrepPlain>(p.in, base_of(q), nt_of(q), x);
      wait_all_at_least(consumed, q - kRing + 1);
      prep_rows_to_raw(cur, rec, x);
      const int qn = min(q + kPrepW, last);
      prep_load_rows(p.in, base_of(qn), nt_of(qn), nxt);
      chain_prep(x, rec);
      post(&ready[q % kRing], q);
      q += kPrepW;
      return q < nc;
    };
    PrepRows ra, rb;
    prep_load_rows(p.in, base_of(q0), nt_of(q0), ra);
    int q = q0;
    while (item(q, ra, rb) && item(q, rb, ra)) {
    }
    return;
  }

  // ------------------------------------------------------------------ chain waves
  __builtin_amdgcn_s_setprio(2);
  const int w = wave;
  Mma32::acc Gt[4];  // element e of Gt[kt] = G[i = 16 w + li][j = 16 kt + 4 g + e]
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) Gt[kt] = Mma32::zero();
  if (p.ds_out) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float4 s = *reinterpret_cast<const float4*>(p.ds_out + ((int64_t)unit * kN + 16 * w + li) * kN +
                                                        16 * kt + 4 * g);
      Gt[kt] = Mma32::acc{f32x4{s.x, s.y, s.z, s.w}};
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  const half4 hz = half4{(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
  // dY of step q for this wave: dY[t = 4g + e][i = 16 w + li]; tokens past the end read
  // the last token (their record coefficients are zero)
  const float* dybase = p.dy + seq_base + 16 * w + li;
  auto load_dy = [&](int q, float (&d)[4]) {
    const int c = nc - 1 - q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = min(c * kC + 4 * g + e, T - 1);
      d[e] = dybase[(int64_t)t * tstride];
    }
  };
  CFrag fa, fb;
  float da_[4], db_[4];
  load_dy(0, da_);
  load_dy(min(1, nc - 1), db_);
  wait_at_least(&ready[0], 0);
  read_cfrag(slot_of(0), fa);
  int q = 0;
  auto body = [&](CFrag& cur, CFrag& nxt, float (&dcur)[4]) {
    const int qn = min(q + 1, nc - 1);
    wait_at_least(&ready[qn % kRing], qn);
    read_cfrag(slot_of(qn), nxt);
    const int c = nc - 1 - q;
    ck_store(p.gend + ((int64_t)unit * nc + c) * kCkHalves, 16 * w, Gt);  // G at the end of chunk c
    half4 dyh;
#pragma unroll
    for (int e = 0; e < 4; ++e) dyh[e] = (_Float16)dcur[e];
    // P = B- G^T, then dU = L_rb^T dY + P (one accumulator chain), dX = T^T dU
    Mma32::acc du = Mma32::mma(cur.bb0, cat8(to_h4(Gt[0]), to_h4(Gt[1])), Mma32::zero());
    du = Mma32::mma(cur.bb1, cat8(to_h4(Gt[2]), to_h4(Gt[3])), du);
    du = Mma32::mma(cur.lrb, cat8(dyh, hz), du);
    const Mma32::acc dx = Mma32::mma(cur.tt, cat8(to_h4(du), hz), Mma32::zero());
    const half8 bop = cat8(dyh, to_h4(dx));  // [dY ; dX] as a B operand (k = t, n = i)
    Gt[0].v[0] *= row_bcast<0>(cur.dv);
    Gt[0].v[1] *= row_bcast<1>(cur.dv);
    Gt[0].v[2] *= row_bcast<2>(cur.dv);
    Gt[0].v[3] *= row_bcast<3>(cur.dv);
    Gt[0] = Mma32::mma(cur.ra[0], bop, Gt[0]);
    Gt[1].v[0] *= row_bcast<4>(cur.dv);
    Gt[1].v[1] *= row_bcast<5>(cur.dv);
    Gt[1].v[2] *= row_bcast<6>(cur.dv);
    Gt[1].v[3] *= row_bcast<7>(cur.dv);
    Gt[1] = Mma32::mma(cur.ra[1], bop, Gt[1]);
    Gt[2].v[0] *= row_bcast<8>(cur.dv);
    Gt[2].v[1] *= row_bcast<9>(cur.dv);
    Gt[2].v[2] *= row_bcast<10>(cur.dv);
    Gt[2].v[3] *= row_bcast<11>(cur.dv);
    Gt[2] = Mma32::mma(cur.ra[2], bop, Gt[2]);
    Gt[3].v[0] *= row_bcast<12>(cur.dv);
    Gt[3].v[1] *= row_bcast<13>(cur.dv);
    Gt[3].v[2] *= row_bcast<14>(cur.dv);
    Gt[3].v[3] *= row_bcast<15>(cur.dv);
    Gt[3] = Mma32::mma(cur.ra[3], bop, Gt[3]);
    load_dy(min(q + 2, nc - 1), dcur);
    post(&consumed[w], qn + 1);
    ++q;
    return q < nc;
  };
  while (body(fa, fb, da_) && body(fb, fa, db_)) {
  }
  if (p.ds_in) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      *reinterpret_cast<float4*>(p.ds_in + ((int64_t)unit * kN + 16 * w + li) * kN + 16 * kt + 4 * g) =
          make_float4(Gt[kt].v[0], Gt[kt].v[1], Gt[kt].v[2], Gt[kt].v[3]);
  }
}

// The two passes that need only the inputs, in one launch: workgroups [0, units) run the
// checkpoint form of the one-kernel prefill, workgroups [units, 2 units) the chain, so
// the two run side by side when there are fewer heads than compute units.
constexpr int kPassLds = fused::kLds > kLds ? fused::kLds : kLds;
__global__ __launch_bounds__(kThreads) void wkv7_bpass_kernel(fused::FusedParams fp, ChainParams cp, int32_t units) {
  extern __shared__ __align__(16) unsigned char ring[];
  if ((int)blockIdx.x < units)
    fused::fused_body<kPrepPlain, true>(fp, ring, blockIdx.x);
  else
    chain_body(cp, ring, blockIdx.x - units);
}

hipError_t launch_pass(const fused::FusedParams& fp, const ChainParams& cp, int64_t units, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&wkv7_bpass_kernel);
  static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kPassLds);
  if (attr != hipSuccess) return attr;
  fused::FusedParams f = fp;
  ChainParams q = cp;
  int32_t u = (int32_t)units;
  void* args[] = {&f, &q, &u};
  return hipLaunchKernel(fn, dim3((uint32_t)(2 * units)), dim3(kThreads), args, kPassLds, stream);
}

// ============================================================================ gradients

// One wave per (head, chunk). Fragment conventions (16x16 tiles; lane (li, g)):
//   "row vector" X[li][4g + e] (A operand of X, B operand of X^T; the token layout when
//   li is a token), "column vector" X[4g + e][li] (the D layout; B operand of X).
// An identity product turns one into the other (tr16). A product with its operands
// swapped returns the transposed result (the same registers serve as A and B), so
// key-space results land in the token layout: lane (t = li, g), keys 16 kt + 4 g + e.
// Contractions over the 64 value rows take row 16 (2 rp + h) + 4 g + e for
// (rp, h = element / 4, e), two 16-row tiles per 16x16x32 product.
constexpr int kGW = 4;  // waves (items) per workgroup
// Per wave: the row staging area (later the scaled operands' column vectors, four
// tensors x four key tiles x 8 bytes per lane), the factor rows, the solve's scratch,
// a 64-float key exchange.
constexpr int kGOpnd = 0;
constexpr int kGFac = kStageBytes;
constexpr int kGScr = kGFac + kFacBytes;
constexpr int kGEx = kGScr + 4096;
constexpr int kGWaveLds = kGEx + kN * 4;  // 18,464 bytes
static_assert(16 * 512 <= kStageBytes, "operand columns fit the staging area");
static_assert(kGScr % 16 == 0 && kGEx % 16 == 0 && kGWaveLds % 16 == 0, "16-byte aligned areas");

struct GradParams {
  PrepIn in;             // r, w, k, a, b (bfloat16), T, H
  const uint16_t* v;
  const float* dy;
  const _Float16* s0;    // [units][nc] chunk start states (fragment order)
  const _Float16* gend;  // [units][nc] gradients at chunk ends (fragment order)
  float* grad[6];        // dr, dw, dk, dv, da, db
  int64_t items;         // units * nc
  int32_t nc;
};

__device__ __forceinline__ half4 tr16(half4 x, half4 eye) { return to_h4(Mma16::mma(x, eye, Mma16::zero())); }
__device__ __forceinline__ half4 lo4(half8 x) { return half4{x[0], x[1], x[2], x[3]}; }
__device__ __forceinline__ half4 hi4(half8 x) { return half4{x[4], x[5], x[6], x[7]}; }
__device__ __forceinline__ half4 f2h(float4 v) {
  return half4{(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
}
__device__ __forceinline__ half4 b2h(uint2 q) {
  return half4{(_Float16)bf4(q, 0), (_Float16)bf4(q, 1), (_Float16)bf4(q, 2), (_Float16)bf4(q, 3)};
}
// Row (16-lane) data movement by DPP: lane li of a row reads lane li + N of the same row
// (zero past its end), or lane (li + N) mod 16.
template <int N>
__device__ __forceinline__ float row_shl(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xf, 0xf, true));
}
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, true));
}
// sum over the row, in every lane of it
__device__ __forceinline__ float row_sum16(float x) {
  x += row_ror<1>(x);
  x += row_ror<2>(x);
  x += row_ror<4>(x);
  x += row_ror<8>(x);
  return x;
}
// sum over lanes li .. 15 of the row
__device__ __forceinline__ float row_suffix16(float x) {
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  x += row_shl<8>(x);
  return x;
}

__global__ __launch_bounds__(64 * kGW, 2) void wkv7_bgrad_kernel(GradParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int64_t item = (int64_t)blockIdx.x * kGW + wave;
  if (item >= p.items) return;
  const int nc = p.nc;
  const int unit = (int)(item / nc), c = (int)(item % nc);
  const int H = p.in.H, T = p.in.T;
  const int bb = unit / H, hh = unit % H;
  const uint32_t tstride = (uint32_t)H * kN;
  const int64_t base = (int64_t)bb * T * H * kN + (int64_t)hh * kN + (int64_t)c * kC * tstride;
  const int nt = min(kC, T - c * kC);
  unsigned char* wl = lds + wave * kGWaveLds;
  float* fac = reinterpret_cast<float*>(wl + kGFac);
  float* scr = reinterpret_cast<float*>(wl + kGScr);
  float* ex = reinterpret_cast<float*>(wl + kGEx);
  unsigned char* opnd = wl + kGOpnd;  // column vectors of a-, r-, b-, k- (slot q * 4 + kt)
  auto opnd_off = [&](int q, int kt) { return (uint32_t)((q * 4 + kt) * 512 + lane * 8); };
  const half4 hz = half4{(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
  half4 eye;
#pragma unroll
  for (int e = 0; e < 4; ++e) eye[e] = (_Float16)(4 * g + e == li ? 1.f : 0.f);

  // ---- loads: the chunk's rows, its v and dY as row vectors (lane t = li; t past the end
  // reads the last token), its start state and end gradient
  PrepRows rows;
  prep_load_rows(p.in, base, nt, rows);
  PrepRaw x;
  prep_load_w<kPrepPlain>(p.in, base, nt, x);
  const int tl = min(li, nt - 1);
  half4 vh[4], dyh[4];  // lane (t = li, g): V[t][16 rt + 4g + e], dY[t][16 rt + 4g + e]
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    vh[rt] = b2h(ld_off<uint2>(p.v + base, (uint32_t)(tl * tstride + 16 * rt + 4 * g) * 2u));
    dyh[rt] = f2h(ld_off<float4>(p.dy + base, (uint32_t)(tl * tstride + 16 * rt + 4 * g) * 4u));
  }
  const _Float16* s0p = p.s0 + item * kCkHalves;
  const _Float16* gp = p.gend + item * kCkHalves;
  prep_rows_to_raw(rows, wl, x);
  prep_factors<kPrepPlain>(x, fac, reinterpret_cast<unsigned char*>(ex));

  // ---- chunk prep: scaled operands (token layout) and their column vectors, the Grams
  half4 AT[4];                           // A^ as column vectors
  half4 bbar[4], kbar[4];                // B-, K- row vectors (lane tau = li)
  MmaBF::acc Lab = MmaBF::zero(), Lak = MmaBF::zero(), Lrb = MmaBF::zero(), Lrk = MmaBF::zero();
  {
    bf16x8 ahH, ahL, rhH, rhL, bhH, bhL, khH, khL;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int col = 16 * kt + 4 * g;
      const float4 gqm1 = lds4(&fac[li * kFacRow + col]);
      const float4 gq = lds4(&fac[(li + 1) * kFacRow + col]);
      const float4 g15 = lds4(&fac[16 * kFacRow + col]);
      const float4 e7 = lds4(&fac[kRowE7 * kFacRow + col]);
      float ag[4], rg[4], bg[4], kg[4];
      half4 ah, agh, rgh, bgh, kgh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float av = bf4(x.ar[kt], e), bv = bf4(x.br[kt], e), rv = bf4(x.rr[kt], e), kv = bf4(x.kr[kt], e);
        const float f = __builtin_amdgcn_rcpf(el(gq, e));
        ag[e] = av * el(gqm1, e);
        rg[e] = rv * el(gq, e);
        bg[e] = bv * f;
        kg[e] = kv * f;
        ah[e] = (_Float16)(ag[e] * el(e7, e));
        bbar[kt][e] = (_Float16)(bg[e] * el(g15, e));
        kbar[kt][e] = (_Float16)(kg[e] * el(g15, e));
        agh[e] = (_Float16)ag[e];
        rgh[e] = (_Float16)rg[e];
        bgh[e] = (_Float16)bg[e];
        kgh[e] = (_Float16)kg[e];
      }
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int q8 = 4 * (kt & 1) + e;
        split_bf16x2(ag[e], ag[e + 1], ahH, ahL, q8);
        split_bf16x2(rg[e], rg[e + 1], rhH, rhL, q8);
        split_bf16x2(bg[e], bg[e + 1], bhH, bhL, q8);
        split_bf16x2(kg[e], kg[e + 1], khH, khL, q8);
      }
      // lane (key 16 kt + li, g): X[t = 4g + e][key], into the (consumed) staging area
      st_off<half4>(opnd, opnd_off(0, kt), tr16(agh, eye));
      st_off<half4>(opnd, opnd_off(1, kt), tr16(rgh, eye));
      st_off<half4>(opnd, opnd_off(2, kt), tr16(bgh, eye));
      st_off<half4>(opnd, opnd_off(3, kt), tr16(kgh, eye));
      AT[kt] = tr16(ah, eye);
      if (kt & 1) {
        Lab = MmaBF::mma(ahH, bhH, Lab);
        Lak = MmaBF::mma(ahH, khH, Lak);
        Lrb = MmaBF::mma(rhH, bhH, Lrb);
        Lrk = MmaBF::mma(rhH, khH, Lrk);
        Lab = MmaBF::mma(ahH, bhL, Lab);
        Lak = MmaBF::mma(ahH, khL, Lak);
        Lrb = MmaBF::mma(rhH, bhL, Lrb);
        Lrk = MmaBF::mma(rhH, khL, Lrk);
        Lab = MmaBF::mma(ahL, bhH, Lab);
        Lak = MmaBF::mma(ahL, khH, Lak);
        Lrb = MmaBF::mma(rhL, bhH, Lrb);
        Lrk = MmaBF::mma(rhL, khH, Lrk);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {  // column vectors: lane (s = li, g) holds L[t = 4g + e][s]
    const int t = 4 * g + e;
    Lab.v[e] = li < t ? Lab.v[e] : 0.f;
    Lak.v[e] = li < t ? Lak.v[e] : 0.f;
    Lrb.v[e] = li <= t ? Lrb.v[e] : 0.f;
    Lrk.v[e] = li <= t ? Lrk.v[e] : 0.f;
  }
  const TmFrags tmf = prep_solve(Lab, Lrb, scr);
  const half4 tB = tmf.tB;                      // T row vectors
  const half8 ttA = cat8(tr16(tB, eye), hz);    // T^T as an A operand
  const half4 lakC = to_h4(Lak), lrbC = to_h4(Lrb), lrkC = to_h4(Lrk);  // L^T as A operands
  const half8 guA = cat8(to_h4(Mma16::mma(lakC, tB, Mma16::zero())), hz);  // lane t: G_u[t][4g + e]
  half8 apA[2];  // A' = T A^ as A operands over the key pairs
  {
    half4 ap[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) ap[kt] = to_h4(Mma16::mma(AT[kt], tB, Mma16::zero()));
    apA[0] = cat8(ap[0], ap[1]);
    apA[1] = cat8(ap[2], ap[3]);
  }
  const half8 bbA[2] = {cat8(bbar[0], bbar[1]), cat8(bbar[2], bbar[3])};
  const half8 kbA[2] = {cat8(kbar[0], kbar[1]), cat8(kbar[2], kbar[3])};

  // ---- value-row quantities per 16-row tile rt (column vectors, lane = value row):
  // U = A' S0^T + G_u V, dU = L_rb^T dY + B- G^T, dX = T^T dU; dV written from here
  half4 uR[4], dxR[4];  // U, dX as row vectors (lane tau / t = li)
  float* dvp = p.grad[3] + base;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    half8 sr[2], gr[2];  // lane (row 16 rt + li, g): the keys of key pair kp
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      sr[kp] = *reinterpret_cast<const half8*>(s0p + ck_off(16 * rt + li, kp, g));
      gr[kp] = *reinterpret_cast<const half8*>(gp + ck_off(16 * rt + li, kp, g));
    }
    const half4 vC = tr16(vh[rt], eye);    // lane (row 16 rt + li, g): V[tau = 4g + e][row]
    const half4 dyC = tr16(dyh[rt], eye);  // dY[t = 4g + e][row]
    Mma32::acc u = Mma32::mma(guA, cat8(vC, hz), Mma32::zero());
    u = Mma32::mma(apA[0], sr[0], u);
    u = Mma32::mma(apA[1], sr[1], u);
    Mma32::acc du = Mma32::mma(cat8(lrbC, hz), cat8(dyC, hz), Mma32::zero());
    du = Mma32::mma(bbA[0], gr[0], du);
    du = Mma32::mma(bbA[1], gr[1], du);
    const half4 dxC = to_h4(Mma32::mma(ttA, cat8(to_h4(du), hz), Mma32::zero()));
    uR[rt] = tr16(to_h4(u), eye);  // lane (tau = li, g): U[tau][row 16 rt + 4g + e]
    dxR[rt] = tr16(dxC, eye);
    // dV^T = [dY ; dX]^T [L_rk | L_ak] + G K-^T (operands swapped): lane (tau = li, g)
    // holds dV[tau][row 16 rt + 4g + e]
    Mma32::acc dv = Mma32::mma(cat8(dyC, dxC), cat8(lrkC, lakC), Mma32::zero());
    dv = Mma32::mma(gr[0], kbA[0], dv);
    dv = Mma32::mma(gr[1], kbA[1], dv);
    if (li < nt)
      st_off<float4>(dvp, (uint32_t)(li * tstride + 16 * rt + 4 * g) * 4u,
                     make_float4(dv.v[0], dv.v[1], dv.v[2], dv.v[3]));
    __builtin_amdgcn_sched_barrier(0);  // one row tile at a time: bounded register pressure
  }
  // row vectors over the 64 rows as 16x16x32 operands (row perm)
  const half8 dyA[2] = {cat8(dyh[0], dyh[1]), cat8(dyh[2], dyh[3])};
  const half8 vA[2] = {cat8(vh[0], vh[1]), cat8(vh[2], vh[3])};
  const half8 uA[2] = {cat8(uR[0], uR[1]), cat8(uR[2], uR[3])};
  const half8 dxA[2] = {cat8(dxR[0], dxR[1]), cat8(dxR[2], dxR[3])};

  // ---- the four C x C Gram gradients, as row vectors (lane t: dL[t][tau = 4g + e]) and
  // their transposes (lane tau: dL[t = 4g + e][tau])
  half4 dLrb, dLrk, dLab, dLak;
  {
    Mma32::acc a = Mma32::mma(uA[0], dyA[0], Mma32::zero());
    a = Mma32::mma(uA[1], dyA[1], a);
    Mma32::acc b = Mma32::mma(vA[0], dyA[0], Mma32::zero());
    b = Mma32::mma(vA[1], dyA[1], b);
    Mma32::acc cc = Mma32::mma(uA[0], dxA[0], Mma32::zero());
    cc = Mma32::mma(uA[1], dxA[1], cc);
    Mma32::acc d = Mma32::mma(vA[0], dxA[0], Mma32::zero());
    d = Mma32::mma(vA[1], dxA[1], d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tau = 4 * g + e;
      dLrb[e] = (_Float16)(tau <= li ? a.v[e] : 0.f);
      dLrk[e] = (_Float16)(tau <= li ? b.v[e] : 0.f);
      dLab[e] = (_Float16)(tau < li ? cc.v[e] : 0.f);
      dLak[e] = (_Float16)(tau < li ? d.v[e] : 0.f);
    }
  }
  const half8 rbk = cat8(dLrb, dLrk), abk = cat8(dLab, dLak);
  const half8 abT = cat8(tr16(dLab, eye), tr16(dLrb, eye)), akT = cat8(tr16(dLak, eye), tr16(dLrk, eye));

  // ---- per key tile: the key-space products (token layout), the end term, the decay's
  // gradient, and the stores
  float* drp = p.grad[0] + base;
  float* dwp = p.grad[1] + base;
  float* dkp = p.grad[2] + base;
  float* dap = p.grad[4] + base;
  float* dbp = p.grad[5] + base;
  // the pieces a key tile reads from memory: its 16 x 16 blocks of S0 and G (row vectors,
  // 8 bytes per lane and row tile) and the raw r, a, b, k (token layout; zero past the end
  // of the sequence); loaded one key tile ahead
  struct KtIn {
    half4 s[4], g[4];
    uint2 r, a, b, k;
  };
  auto kt_load = [&](int kt, KtIn& q) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const uint32_t o = ck_off(16 * rt + li, kt >> 1, g) + 4 * (kt & 1);
      q.s[rt] = *reinterpret_cast<const half4*>(s0p + o);
      q.g[rt] = *reinterpret_cast<const half4*>(gp + o);
    }
    const uint32_t ro = (uint32_t)(tl * tstride + 16 * kt + 4 * g) * 2u;
    const uint2 z2 = make_uint2(0u, 0u);
    q.r = li < nt ? ld_off<uint2>(p.in.r + base, ro) : z2;
    q.a = li < nt ? ld_off<uint2>(p.in.a + base, ro) : z2;
    q.b = li < nt ? ld_off<uint2>(p.in.b + base, ro) : z2;
    q.k = li < nt ? ld_off<uint2>(p.in.k + base, ro) : z2;
  };
  KtIn kin[2];
  kt_load(0, kin[0]);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const KtIn& cur = kin[kt & 1];
    if (kt < 3) kt_load(kt + 1, kin[(kt + 1) & 1]);
    // S0 and G tiles of key tile kt as column vectors over the rows (lane key 16 kt + li)
    half8 sC[2], gC[2];
#pragma unroll
    for (int rp = 0; rp < 2; ++rp) {
      sC[rp] = cat8(tr16(cur.s[2 * rp], eye), tr16(cur.s[2 * rp + 1], eye));
      gC[rp] = cat8(tr16(cur.g[2 * rp], eye), tr16(cur.g[2 * rp + 1], eye));
    }
    // sum over rows of S0 G for key 16 kt + li, times e^{gamma_15}, to the exchange
    {
      float acc = 0.f;
#pragma unroll
      for (int rp = 0; rp < 2; ++rp)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)sC[rp][e], (float)gC[rp][e], acc);
      acc += __shfl_xor(acc, 16);
      acc += __shfl_xor(acc, 32);
      const int j = 16 * kt + li;
      if (g == 0) ex[j] = acc * fac[16 * kFacRow + j] * fac[kRowE7 * kFacRow + j];
    }
    Mma32::acc ys = Mma32::mma(sC[0], dyA[0], Mma32::zero());  // (dY S0)[t][keys]
    ys = Mma32::mma(sC[1], dyA[1], ys);
    Mma32::acc xs = Mma32::mma(sC[0], dxA[0], Mma32::zero());  // (dX S0)
    xs = Mma32::mma(sC[1], dxA[1], xs);
    Mma32::acc ug = Mma32::mma(gC[0], uA[0], Mma32::zero());   // (U G)[tau][keys]
    ug = Mma32::mma(gC[1], uA[1], ug);
    Mma32::acc vg = Mma32::mma(gC[0], vA[0], Mma32::zero());   // (V G)
    vg = Mma32::mma(gC[1], vA[1], vg);
    const half8 bk = cat8(ld_off<half4>(opnd, opnd_off(2, kt)), ld_off<half4>(opnd, opnd_off(3, kt)));
    const half8 ar = cat8(ld_off<half4>(opnd, opnd_off(0, kt)), ld_off<half4>(opnd, opnd_off(1, kt)));
    const Mma32::acc pr = Mma32::mma(bk, rbk, Mma32::zero());  // dL_rb b- + dL_rk k- (scaled operands)
    const Mma32::acc pa = Mma32::mma(bk, abk, Mma32::zero());  // dL_ab b- + dL_ak k-
    const Mma32::acc pb = Mma32::mma(ar, abT, Mma32::zero());  // dL_ab^T a- + dL_rb^T r-
    const Mma32::acc pk = Mma32::mma(ar, akT, Mma32::zero());  // dL_ak^T a- + dL_rk^T r-
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    const int col = 16 * kt + 4 * g;
    const float4 gqm1 = lds4(&fac[li * kFacRow + col]);
    const float4 gq = lds4(&fac[(li + 1) * kFacRow + col]);
    const float4 g15 = lds4(&fac[16 * kFacRow + col]);
    const float4 e7 = lds4(&fac[kRowE7 * kFacRow + col]);
    const float4 e1 = lds4(&ex[col]);
    float dr[4], da[4], db[4], dk[4], dg[4], hv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float q = el(gq, e), qm = el(gqm1, e), E7 = el(e7, e), iq = __builtin_amdgcn_rcpf(q);
      dr[e] = q * E7 * ys.v[e] + q * pr.v[e];
      da[e] = qm * E7 * xs.v[e] + qm * pa.v[e];
      db[e] = iq * pb.v[e] + el(g15, e) * iq * ug.v[e];
      dk[e] = iq * pk.v[e] + el(g15, e) * iq * vg.v[e];
      hv[e] = (float)bbar[kt][e] * ug.v[e] + (float)kbar[kt][e] * vg.v[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float an = row_shl<1>(bf4(cur.a, e) * da[e]);  // a_{t+1} da_{t+1} (zero at t = 15)
      dg[e] = bf4(cur.r, e) * dr[e] - bf4(cur.b, e) * db[e] - bf4(cur.k, e) * dk[e] + an;
      const float tot = row_sum16(hv[e]) + el(e1, e);  // the chunk end's share, for every token
      // dw = dlog w / w, 1 / w = Gq_{t-1} / Gq_t
      dg[e] = (row_suffix16(dg[e]) + tot) * el(gqm1, e) * __builtin_amdgcn_rcpf(el(gq, e));
    }
    if (li < nt) {
      const uint32_t o = (uint32_t)(li * tstride + col) * 4u;
      st_off<float4>(drp, o, make_float4(dr[0], dr[1], dr[2], dr[3]));
      st_off<float4>(dwp, o, make_float4(dg[0], dg[1], dg[2], dg[3]));
      st_off<float4>(dkp, o, make_float4(dk[0], dk[1], dk[2], dk[3]));
      st_off<float4>(dap, o, make_float4(da[0], da[1], da[2], da[3]));
      st_off<float4>(dbp, o, make_float4(db[0], db[1], db[2], db[3]));
    }
    __builtin_amdgcn_sched_barrier(0);  // one key tile at a time
  }
}

hipError_t launch_grad(const GradParams& gp, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&wkv7_bgrad_kernel);
  const int lds = kGW * kGWaveLds;
  GradParams q = gp;
  void* args[] = {&q};
  return hipLaunchKernel(fn, dim3((uint32_t)((gp.items + kGW - 1) / kGW)), dim3(64 * kGW), args, lds, stream);
}

}  // namespace

hipError_t launch_backward_chunked(const BwdCall& c) {
  if (c.dtype != 1 || c.T * c.H * kN >= (int64_t(1) << 31)) return hipErrorNotSupported;
  const int64_t units = c.B * c.H;
  const int64_t nc = (c.T + kC - 1) / kC;
  const size_t ck_bytes = (size_t)(units * nc) * kCkHalves * sizeof(_Float16);
  void* ws = nullptr;
  hipError_t e = device_workspace(c.stream, 2 * ck_bytes, &ws);
  if (e != hipSuccess) return e;
  _Float16* s0 = static_cast<_Float16*>(ws);
  _Float16* gend = reinterpret_cast<_Float16*>(static_cast<char*>(ws) + ck_bytes);
  // 1. the chunk start states and 2. the chain of state gradients, side by side
  fused::FusedParams fp{};
  fp.in.r = static_cast<const uint16_t*>(c.in[0]);
  fp.in.w = static_cast<const uint16_t*>(c.in[1]);
  fp.in.k = static_cast<const uint16_t*>(c.in[2]);
  fp.in.a = static_cast<const uint16_t*>(c.in[4]);
  fp.in.b = static_cast<const uint16_t*>(c.in[5]);
  fp.in.T = (int32_t)c.T;
  fp.in.H = (int32_t)c.H;
  fp.v = static_cast<const uint16_t*>(c.in[3]);
  fp.s_in = c.s_in;
  fp.ck = s0;
  fp.nc = (int32_t)nc;
  ChainParams cp{};
  cp.in.r = static_cast<const uint16_t*>(c.in[0]);
  cp.in.w = static_cast<const uint16_t*>(c.in[1]);
  cp.in.k = static_cast<const uint16_t*>(c.in[2]);
  cp.in.a = static_cast<const uint16_t*>(c.in[4]);
  cp.in.b = static_cast<const uint16_t*>(c.in[5]);
  cp.in.T = (int32_t)c.T;
  cp.in.H = (int32_t)c.H;
  cp.dy = c.dy;
  cp.ds_out = c.ds_out;
  cp.ds_in = c.ds_in;
  cp.gend = gend;
  cp.nc = (int32_t)nc;
  e = launch_pass(fp, cp, units, c.stream);
  if (e != hipSuccess) return e;
  // 3. the input gradients, one wave per (head, chunk)
  GradParams gp{};
  gp.in = cp.in;
  gp.v = static_cast<const uint16_t*>(c.in[3]);
  gp.dy = c.dy;
  gp.s0 = s0;
  gp.gend = gend;
  for (int i = 0; i < 6; ++i) gp.grad[i] = c.grad[i];
  gp.items = units * nc;
  gp.nc = (int32_t)nc;
  return launch_grad(gp, c.stream);
}

}  // namespace rwkv7
