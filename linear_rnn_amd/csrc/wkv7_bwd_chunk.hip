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
//      the start of every even chunk (wkv7_fused.hpp);
//   2. the chain, one workgroup per head: prep waves rebuild each chunk's chain record
//      (B-, L_rb^T, T^T, [R^^T | A^^T], e^{gamma_15}) into an LDS ring, last chunk
//      first; scan waves carry G in float32 back through the chunks, store the end G
//      (float16) of every odd chunk and of the last one, and finally dL/dS_0.
//   1 and 2 need only the inputs and dY, so one launch (wkv7_bpass_kernel) runs both,
//   a workgroup per head for each;
//   3. wkv7_bgrad_kernel, one wave per (head, chunk) over the whole chip, forms the
//      chunk's input gradients from its inputs, dY, S0 and end G; the two waves of a
//      chunk pair rebuild the odd chunk's S0 and the even chunk's G from what is stored
//      (one more chunk step each way), which halves the float16 arrays.
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
  _Float16* gend;      // [B*H][(nc + 1) / 2] float16 G at the end of every odd chunk c and of the
                       // last one, at index c / 2 (fragment order)
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
    constexpr unsigned kRows = kRowR | kRowA | kRowB;  // the chain needs no k
    const int last = q0 + (nc - 1 - q0) / kPrepW * kPrepW;
    auto nt_of = [&](int q) { return min(kC, T - (nc - 1 - q) * kC); };
    auto base_of = [&](int q) { return seq_base + (int64_t)(nc - 1 - q) * kC * tstride; };
    auto item = [&](int& q, PrepRows& cur, PrepRows& nxt) {
      unsigned char* rec = slot_of(q);
      PrepRaw x;
      prep_load_w<kPrepPlain>(p.in, base_of(q), nt_of(q), x);
      wait_all_at_least(consumed, q - kRing + 1);
      prep_rows_to_raw<kRows>(cur, rec, x);
      const int qn = min(q + kPrepW, last);
      prep_load_rows<kRows>(p.in, base_of(qn), nt_of(qn), nxt);
      chain_prep(x, rec);
      post(&ready[q % kRing], q);
      q += kPrepW;
      return q < nc;
    };
    PrepRows ra, rb;
    prep_load_rows<kRows>(p.in, base_of(q0), nt_of(q0), ra);
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
    if ((c & 1) || c == nc - 1)  // G at the end of chunk c
      ck_store(p.gend + ((int64_t)unit * ((nc + 1) >> 1) + (c >> 1)) * kCkHalves, 16 * w, Gt);
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
// The contractions over the 64 value rows accumulate one 16-row tile at a time
// (16x16x16 products), while that tile's U, dX, S0 and G are in registers.
constexpr int kGW = 2;  // waves per workgroup: one chunk pair (wave 0 the even chunk, wave 1 the odd)
// Per wave: the chunk's staged r, a, b, k rows (kept for the whole item), the factor
// rows, the solve's scratch, a 64-float key exchange, and the 64x64 float16 state (or
// gradient) handed to the other wave of the pair.
constexpr int kGStage = 0;
constexpr int kGFac = kStageBytes;
constexpr int kGScr = kGFac + kFacBytes;
constexpr int kGEx = kGScr + 4096;
constexpr int kGX = kGEx + kN * 4;
constexpr int kGWaveLds = kGX + kCkHalves * 2;  // 26,656 bytes
static_assert(kGScr % 16 == 0 && kGX % 16 == 0 && kGWaveLds % 16 == 0, "16-byte aligned areas");
static_assert(3 * kGW * kGWaveLds <= 160 * 1024, "three workgroups per compute unit");

struct GradParams {
  PrepIn in;             // r, w, k, a, b (bfloat16), T, H
  const uint16_t* v;
  const float* dy;
  const _Float16* s0;    // [units][np] start states of the even chunks (fragment order)
  const _Float16* gend;  // [units][np] gradients at the ends of the odd chunks and the last one
  float* grad[6];        // dr, dw, dk, dv, da, db
  int64_t pairs;         // units * np, np = (nc + 1) / 2
  int32_t nc;
};

// The handed-over state: row-major rows of 128 bytes; the 16-byte piece (kp, g) of row i
// sits at piece (4 kp + g) ^ (i & 7), so that the 16 rows of a row-vector access spread
// over the banks.
__device__ __forceinline__ uint32_t xt_off(int row, int kp, int g) {
  return (uint32_t)(row * 128 + 16 * ((4 * kp + g) ^ (row & 7)));
}
// Workgroup barrier for the LDS hand-off: this wave's LDS accesses have completed, global
// ones stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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

// The work of one wave: chunk c of head unit, the odd (ODD) or even chunk of its pair.
template <bool ODD>
__device__ __forceinline__ void grad_item(const GradParams& p, unsigned char* lds, int wave, int unit, int c) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
  const int nc = p.nc, np = (nc + 1) >> 1;
  const int H = p.in.H, T = p.in.T;
  const int bb = unit / H, hh = unit % H;
  const uint32_t tstride = (uint32_t)H * kN;
  const int64_t base = (int64_t)bb * T * H * kN + (int64_t)hh * kN + (int64_t)c * kC * tstride;
  const int nt = min(kC, T - c * kC);
  unsigned char* wl = lds + wave * kGWaveLds;
  unsigned char* stage = wl + kGStage;
  float* fac = reinterpret_cast<float*>(wl + kGFac);
  float* scr = reinterpret_cast<float*>(wl + kGScr);
  float* ex = reinterpret_cast<float*>(wl + kGEx);
  const half4 hz = half4{(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
  half4 eye;
#pragma unroll
  for (int e = 0; e < 4; ++e) eye[e] = (_Float16)(4 * g + e == li ? 1.f : 0.f);

  // ---- loads: the chunk's rows, its v and dY as row vectors (lane t = li; t past the end
  // reads the last token)
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
  prep_rows_to_raw(rows, stage, x);  // the staged rows stay in LDS for the end
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) asm volatile("" : "+v"(vh[rt]), "+v"(dyh[rt]));  // held as float16
  const int64_t slot = ((int64_t)unit * np + (c >> 1)) * kCkHalves;
  const _Float16* s0p = p.s0 + slot;    // even chunks
  const _Float16* gp = p.gend + slot;   // odd chunks and the last one
  const bool g_mem = ODD || c == nc - 1;
  unsigned char* xown = wl + kGX;
  const unsigned char* xpeer = lds + (wave ^ 1) * kGWaveLds + kGX;
  prep_factors<kPrepPlain>(x, fac, reinterpret_cast<unsigned char*>(ex));

  // ---- chunk prep: the Grams (column vectors: lane (s = li, g) holds L[t = 4g + e][s]),
  // A^ column vectors, B-, K- row vectors
  half4 AT[4], RT[4], bbar[4], kbar[4];  // RT: R^ column vectors (odd chunk only)
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
      half4 ah, rh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float av = bf4(x.ar[kt], e), bv = bf4(x.br[kt], e), rv = bf4(x.rr[kt], e), kv = bf4(x.kr[kt], e);
        const float f = __builtin_amdgcn_rcpf(el(gq, e));
        ag[e] = av * el(gqm1, e);
        rg[e] = rv * el(gq, e);
        bg[e] = bv * f;
        kg[e] = kv * f;
        ah[e] = (_Float16)(ag[e] * el(e7, e));  // A^ = a e^{gamma_{t-1}}
        rh[e] = (_Float16)(rg[e] * el(e7, e));  // R^ = r e^{gamma_t}
        bbar[kt][e] = (_Float16)(bg[e] * el(g15, e));
        kbar[kt][e] = (_Float16)(kg[e] * el(g15, e));
      }
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int q8 = 4 * (kt & 1) + e;
        split_bf16x2(ag[e], ag[e + 1], ahH, ahL, q8);
        split_bf16x2(rg[e], rg[e + 1], rhH, rhL, q8);
        split_bf16x2(bg[e], bg[e + 1], bhH, bhL, q8);
        split_bf16x2(kg[e], kg[e + 1], khH, khL, q8);
      }
      AT[kt] = tr16(ah, eye);
      if constexpr (ODD) RT[kt] = tr16(rh, eye);
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
  for (int e = 0; e < 4; ++e) {
    const int t = 4 * g + e;
    Lab.v[e] = li < t ? Lab.v[e] : 0.f;
    Lak.v[e] = li < t ? Lak.v[e] : 0.f;
    Lrb.v[e] = li <= t ? Lrb.v[e] : 0.f;
    Lrk.v[e] = li <= t ? Lrk.v[e] : 0.f;
  }
  const TmFrags tmf = prep_solve(Lab, Lrb, scr);
  half8 owns[4][2];  // the stored G (odd) or S0 (even) of every row tile, in flight during the solve's tail
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
      owns[rt][kp] = *reinterpret_cast<const half8*>((ODD ? gp : s0p) + ck_off(16 * rt + li, kp, g));
  const half4 tB = tmf.tB;                    // T row vectors
  const half8 ttA = cat8(tr16(tB, eye), hz);  // T^T as an A operand
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
  // B- and K- row vectors (A operands over the key pairs) wait in the solve's scratch,
  // free from here on: four 16-byte pieces per lane, read back in every row tile
  unsigned char* bk_l = reinterpret_cast<unsigned char*>(scr);
  st_off<half8>(bk_l, (uint32_t)lane * 16u, cat8(bbar[0], bbar[1]));
  st_off<half8>(bk_l, 1024u + (uint32_t)lane * 16u, cat8(bbar[2], bbar[3]));
  st_off<half8>(bk_l, 2048u + (uint32_t)lane * 16u, cat8(kbar[0], kbar[1]));
  st_off<half8>(bk_l, 3072u + (uint32_t)lane * 16u, cat8(kbar[2], kbar[3]));

  // U = A' S0^T + G_u V and dU = L_rb^T dY + B- G^T, dX = T^T dU of row tile rt (column
  // vectors, lane = value row)
  auto form_u = [&](const half8 (&sr)[2], half4 vC) {
    Mma32::acc u = Mma32::mma(guA, cat8(vC, hz), Mma32::zero());
    u = Mma32::mma(apA[0], sr[0], u);
    return Mma32::mma(apA[1], sr[1], u);
  };
  auto form_dx = [&](const half8 (&gr)[2], half4 dyC) {
    Mma32::acc du = Mma32::mma(cat8(lrbC, hz), cat8(dyC, hz), Mma32::zero());
    du = Mma32::mma(ld_off<half8>(bk_l, (uint32_t)lane * 16u), gr[0], du);
    du = Mma32::mma(ld_off<half8>(bk_l, 1024u + (uint32_t)lane * 16u), gr[1], du);
    return to_h4(Mma32::mma(ttA, cat8(to_h4(du), hz), Mma32::zero()));
  };
  auto ld_ck = [&](const _Float16* src, int rt, half8 (&dst)[2]) {
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) dst[kp] = *reinterpret_cast<const half8*>(src + ck_off(16 * rt + li, kp, g));
  };

  // ---- for the other wave of the pair, per 16-row tile rt and key tile kt = 2 kp + h:
  // the odd chunk's G0 = e^{gamma_15} G + [R^^T | A^^T] [dY ; dX] (the even chunk's end
  // gradient), the even chunk's S_end = e^{gamma_15} S0 + [B-^T | K-^T] [U ; V] (the odd
  // chunk's start state)
  half8 xop[4];   // per key tile: [R^^T | A^^T] (odd) or [B-^T | K-^T] (even) as an A operand
  float4 e15[4];  // e^{gamma_15} of keys 16 kt + 4g + e
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    if constexpr (ODD)
      xop[kt] = cat8(RT[kt], AT[kt]);
    else
      xop[kt] = cat8(tr16(bbar[kt], eye), tr16(kbar[kt], eye));
    const float4 g15 = lds4(&fac[16 * kFacRow + 16 * kt + 4 * g]);
    const float4 e7 = lds4(&fac[kRowE7 * kFacRow + 16 * kt + 4 * g]);
    e15[kt] = make_float4(g15.x * e7.x, g15.y * e7.y, g15.z * e7.z, g15.w * e7.w);
  }
  half4 kept[4];  // U (even) or dX (odd) of each row tile, for the row tiles below
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int row = 16 * rt + li;
    const half8 (&own)[2] = owns[rt];
    half4 pC, qC;  // [dY ; dX] or [U ; V] as a B operand
    if constexpr (ODD) {
      pC = tr16(dyh[rt], eye);
      qC = form_dx(own, pC);
      kept[rt] = qC;
    } else {
      qC = tr16(vh[rt], eye);
      pC = to_h4(form_u(own, qC));
      kept[rt] = pC;
    }
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      half4 t2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kt = 2 * kp + h;
        Mma32::acc o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o.v[e] = (float)own[kp][4 * h + e] * el(e15[kt], e);
        o = Mma32::mma(xop[kt], cat8(pC, qC), o);
        t2[h] = to_h4(o);
      }
      st_off<half8>(xown, xt_off(row, kp, g), cat8(t2[0], t2[1]));
    }
  }
  lds_barrier();  // both waves' states are in LDS

  // ---- per 16-row tile rt: U, dU, dX, dV (stored), and this tile's share of every
  // contraction over the rows: (dY S0), (dX S0), (U G), (V G) per key tile in the token
  // layout, the four C x C Gram gradients, and sum_i S0 G
  Mma16::acc ys[4], xs[4], ug[4], vg[4];
  Mma16::acc dLrb = Mma16::zero(), dLrk = Mma16::zero(), dLab = Mma16::zero(), dLak = Mma16::zero();
  float endp[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    ys[kt] = xs[kt] = ug[kt] = vg[kt] = Mma16::zero();
    endp[kt] = 0.f;
  }
  float* dvp = p.grad[3] + base;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int row = 16 * rt + li;
    half8 sr[2], gr[2];  // lane (row 16 rt + li, g): the keys of key pair kp (row vectors)
    if constexpr (ODD) {
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) sr[kp] = ld_off<half8>(xpeer, xt_off(row, kp, g));
      ld_ck(gp, rt, gr);
    } else {
      ld_ck(s0p, rt, sr);
      if (g_mem) {
        ld_ck(gp, rt, gr);  // the last chunk, alone in its pair
      } else {
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) gr[kp] = ld_off<half8>(xpeer, xt_off(row, kp, g));
      }
    }
    const half4 vC = tr16(vh[rt], eye);    // lane (row 16 rt + li, g): V[tau = 4g + e][row]
    const half4 dyC = tr16(dyh[rt], eye);  // dY[t = 4g + e][row]
    const half4 uC = ODD ? to_h4(form_u(sr, vC)) : kept[rt];
    const half4 dxC = ODD ? kept[rt] : form_dx(gr, dyC);
    const half4 uR = tr16(uC, eye);  // lane (tau = li, g): U[tau][row 16 rt + 4g + e]
    const half4 dxR = tr16(dxC, eye);      // lane (t = li, g): dX[t][row 16 rt + 4g + e]
    // dV^T = [dY ; dX]^T [L_rk | L_ak] + G K-^T (operands swapped): lane (tau = li, g)
    // holds dV[tau][row 16 rt + 4g + e]
    Mma32::acc dv = Mma32::mma(cat8(dyC, dxC), cat8(lrkC, lakC), Mma32::zero());
    dv = Mma32::mma(gr[0], ld_off<half8>(bk_l, 2048u + (uint32_t)lane * 16u), dv);
    dv = Mma32::mma(gr[1], ld_off<half8>(bk_l, 3072u + (uint32_t)lane * 16u), dv);
    if (li < nt)
      st_off<float4>(dvp, (uint32_t)(li * tstride + 16 * rt + 4 * g) * 4u,
                     make_float4(dv.v[0], dv.v[1], dv.v[2], dv.v[3]));
    // Gram gradients, as row vectors over tau (lane t): dL[t][tau] = sum_rows X[t] Y[tau]
    dLrb = Mma16::mma(uR, dyh[rt], dLrb);
    dLrk = Mma16::mma(vh[rt], dyh[rt], dLrk);
    dLab = Mma16::mma(uR, dxR, dLab);
    dLak = Mma16::mma(vh[rt], dxR, dLak);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      // this row tile of S0 and G, key tile kt, as column vectors over its rows (lane key)
      const half4 sC = tr16((kt & 1) ? hi4(sr[kt >> 1]) : lo4(sr[kt >> 1]), eye);
      const half4 gC = tr16((kt & 1) ? hi4(gr[kt >> 1]) : lo4(gr[kt >> 1]), eye);
      ys[kt] = Mma16::mma(sC, dyh[rt], ys[kt]);  // (dY S0)[t][key]
      xs[kt] = Mma16::mma(sC, dxR, xs[kt]);      // (dX S0)[t][key]
      ug[kt] = Mma16::mma(gC, uR, ug[kt]);       // (U G)[tau][key]
      vg[kt] = Mma16::mma(gC, vh[rt], vg[kt]);   // (V G)[tau][key]
#pragma unroll
      for (int e = 0; e < 4; ++e) endp[kt] = fmaf((float)sC[e], (float)gC[e], endp[kt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);  // one row tile at a time (the accumulators stay live)
  }
  // the Gram gradients masked (dL_rb, dL_rk: tau <= t; dL_ab, dL_ak: tau < t), as A operands
  // over tau (lane t) and, transposed, over t (lane tau)
  half4 hrb, hrk, hab, hak;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int tau = 4 * g + e;
    hrb[e] = (_Float16)(tau <= li ? dLrb.v[e] : 0.f);
    hrk[e] = (_Float16)(tau <= li ? dLrk.v[e] : 0.f);
    hab[e] = (_Float16)(tau < li ? dLab.v[e] : 0.f);
    hak[e] = (_Float16)(tau < li ? dLak.v[e] : 0.f);
  }
  const half8 rbk = cat8(hrb, hrk), abk = cat8(hab, hak);
  const half8 abT = cat8(tr16(hab, eye), tr16(hrb, eye)), akT = cat8(tr16(hak, eye), tr16(hrk, eye));
  // sum over the rows of S0 G, times e^{gamma_15}, to the key exchange (lane key 16 kt + li)
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    float acc = endp[kt];
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    const int j = 16 * kt + li;
    if (g == 0) ex[j] = acc * fac[16 * kFacRow + j] * fac[kRowE7 * kFacRow + j];
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();

  // ---- per key tile, in the token layout (lane t = li, keys 16 kt + 4g + e): the scaled
  // operands again (from the staged rows), the Gram-gradient products, the input gradients,
  // the decay's gradient, and the stores
  float* drp = p.grad[0] + base;
  float* dwp = p.grad[1] + base;
  float* dkp = p.grad[2] + base;
  float* dap = p.grad[4] + base;
  float* dbp = p.grad[5] + base;
  const bool live = li < nt;
  const uint2 z2 = make_uint2(0u, 0u);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int col = 16 * kt + 4 * g;
    const uint32_t so = (uint32_t)(li * kStageRow + 32 * kt + 8 * g);
    const uint2 rq = live ? ld_off<uint2>(stage, 0 * kStageT + so) : z2;
    const uint2 aq = live ? ld_off<uint2>(stage, 1 * kStageT + so) : z2;
    const uint2 bq = live ? ld_off<uint2>(stage, 2 * kStageT + so) : z2;
    const uint2 kq = live ? ld_off<uint2>(stage, 3 * kStageT + so) : z2;
    const float4 gqm1 = lds4(&fac[li * kFacRow + col]);
    const float4 gq = lds4(&fac[(li + 1) * kFacRow + col]);
    const float4 g15 = lds4(&fac[16 * kFacRow + col]);
    const float4 e7 = lds4(&fac[kRowE7 * kFacRow + col]);
    const float4 e1 = lds4(&ex[col]);
    half4 agh, rgh, bgh, kgh;
    float bs[4], ks[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float f = __builtin_amdgcn_rcpf(el(gq, e));
      const float bg = bf4(bq, e) * f, kg = bf4(kq, e) * f;
      agh[e] = (_Float16)(bf4(aq, e) * el(gqm1, e));
      rgh[e] = (_Float16)(bf4(rq, e) * el(gq, e));
      bgh[e] = (_Float16)bg;
      kgh[e] = (_Float16)kg;
      bs[e] = bg * el(g15, e);  // B- and K- of this token
      ks[e] = kg * el(g15, e);
    }
    // column vectors of the scaled operands: lane (key 16 kt + li, g) holds X[t = 4g + e][key]
    const half8 bk = cat8(tr16(bgh, eye), tr16(kgh, eye)), ar = cat8(tr16(agh, eye), tr16(rgh, eye));
    const Mma32::acc pr = Mma32::mma(bk, rbk, Mma32::zero());  // dL_rb b- + dL_rk k- (scaled operands)
    const Mma32::acc pa = Mma32::mma(bk, abk, Mma32::zero());  // dL_ab b- + dL_ak k-
    const Mma32::acc pb = Mma32::mma(ar, abT, Mma32::zero());  // dL_ab^T a- + dL_rb^T r-
    const Mma32::acc pk = Mma32::mma(ar, akT, Mma32::zero());  // dL_ak^T a- + dL_rk^T r-
    float dr[4], da[4], db[4], dk[4], dg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float q = el(gq, e), qm = el(gqm1, e), E7 = el(e7, e), iq = __builtin_amdgcn_rcpf(q);
      dr[e] = q * E7 * ys[kt].v[e] + q * pr.v[e];
      da[e] = qm * E7 * xs[kt].v[e] + qm * pa.v[e];
      db[e] = iq * pb.v[e] + el(g15, e) * iq * ug[kt].v[e];
      dk[e] = iq * pk.v[e] + el(g15, e) * iq * vg[kt].v[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float an = row_shl<1>(bf4(aq, e) * da[e]);  // a_{t+1} da_{t+1} (zero at t = 15)
      dg[e] = bf4(rq, e) * dr[e] - bf4(bq, e) * db[e] - bf4(kq, e) * dk[e] + an;
      // the chunk end's share, for every token: e^{gamma_15} sum_i S0 G + sum_tau (B- dB- + K- dK-)
      const float tot = row_sum16(bs[e] * ug[kt].v[e] + ks[e] * vg[kt].v[e]) + el(e1, e);
      // dw = dlog w / w, 1 / w = Gq_{t-1} / Gq_t
      dg[e] = (row_suffix16(dg[e]) + tot) * el(gqm1, e) * __builtin_amdgcn_rcpf(el(gq, e));
    }
    if (live) {
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

// One workgroup per chunk pair (2j, 2j + 1) of a head, one wave per chunk. Only the even
// chunk's S0 and the odd chunk's G are stored: before its row tiles, the even chunk's wave
// forms its end state S_end = S0 e^{gamma_15} + U^T B- + V^T K- (the odd chunk's S0) and
// the odd chunk's wave its start gradient G0 = G e^{gamma_15} + R^^T dY + A^^T dX (the even
// chunk's end G), each into LDS for the other.
__global__ __launch_bounds__(64 * kGW, 2) void wkv7_bgrad_kernel(GradParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nc = p.nc, np = (nc + 1) >> 1;
  const bool odd = wave & 1;
  const int64_t pair = blockIdx.x;
  const int unit = (int)(pair / np);
  const int c = 2 * (int)(pair % np) + (odd ? 1 : 0);
  if (pair >= p.pairs || c >= nc) {  // the odd half of a last pair of one chunk: meets the one barrier
    lds_barrier();
    return;
  }
  if (odd)
    grad_item<true>(p, lds, wave, unit, c);
  else
    grad_item<false>(p, lds, wave, unit, c);
}

hipError_t launch_grad(const GradParams& gp, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&wkv7_bgrad_kernel);
  const int lds = kGW * kGWaveLds;
  GradParams q = gp;
  void* args[] = {&q};
  return hipLaunchKernel(fn, dim3((uint32_t)gp.pairs), dim3(64 * kGW), args, lds, stream);
}

}  // namespace

hipError_t launch_backward_chunked(const BwdCall& c) {
  if (c.dtype != 1 || c.T * c.H * kN >= (int64_t(1) << 31)) return hipErrorNotSupported;
  const int64_t units = c.B * c.H;
  const int64_t nc = (c.T + kC - 1) / kC;
  // the start states of the even chunks and the end gradients of the odd ones (and the last)
  const size_t ck_bytes = (size_t)(units * ((nc + 1) / 2)) * kCkHalves * sizeof(_Float16);
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
  gp.pairs = units * ((nc + 1) / 2);
  gp.nc = (int32_t)nc;
  return launch_grad(gp, c.stream);
}

}  // namespace rwkv7
