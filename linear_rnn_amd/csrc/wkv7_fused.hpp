// The one-kernel chunked prefill's workgroup: one head per workgroup (see
// wkv7_fused.hip for the design). fused_body is the whole workgroup's work, so that
// other kernels can host it (the backward runs its checkpoint form beside another role).
#pragma once
#include <cstdint>

#include "wkv7_chunk_ops.hpp"

namespace rwkv7 {
namespace fused {

using namespace chunk;

constexpr int kScanW = 4;                    // scan waves (16 value rows each)
constexpr int kPrepW = 8;                    // prep waves (one chunk each at a time)
constexpr int kRing = 10;                    // record slots
constexpr int kSlot = kRecBytes;             // 9,472 bytes (a scan wave loads its v itself)
// y leaves the scan waves in one of two ways (ROWS below):
// - staged as whole token rows, [chunk parity][token][64 values] float32 (rows padded to 272
//   bytes against bank conflicts), each scan wave storing four whole 256-byte rows per chunk one
//   chunk later; a progress word per scan wave counts the chunks it has staged;
// - through a tile of each wave's own, [token][16 values] float32 with 80-byte rows, so that its
//   stores cover 4 tokens per quarter-wave instead of 16 (no wait on the other scan waves).
constexpr int kYRowF = kN + 4;               // floats per staged row
constexpr int kYOff = kRing * kSlot;
constexpr int kYBytes = 2 * kC * kYRowF * 4;  // 8,704 bytes
constexpr int kYRow = 80;
constexpr int kYTile = kC * kYRow;           // 1,280 bytes per scan wave
constexpr int kYTileOff = kYOff + kYBytes;
constexpr int kCtrlOff = kYTileOff + kScanW * kYTile;  // ready[kRing], consumed[kScanW], y_done[kScanW]
constexpr int kLds = kCtrlOff + 4 * (kRing + 2 * kScanW);
constexpr float kLnEps = 64e-5f;  // the GroupNorm eps of ln_x
constexpr int kThreads = 64 * (kScanW + kPrepW);
constexpr int kSpinMax = 1 << 20;            // polls of 100-200 cycles: well over any legitimate wait
static_assert(kRing >= 3, "the scan reads one chunk ahead");
static_assert(kLds <= 160 * 1024, "LDS per compute unit");
static_assert(kRecBytes % 16 == 0 && kSlot % 16 == 0, "16-byte record blocks");

struct FusedParams {
  PrepIn in;  // r, w (or w_raw), k, a (or kk), b (or a_lr), T, H
  const uint16_t* v;
  float* y;
  const float* s_in;  // may be null (zero state)
  float* s_out;       // may be null
  _Float16* ck;       // checkpoint form only: the state at the start of every even chunk c, at
                      // index c / 2 of (nc + 1) / 2 per sequence (kCkHalves each)
  int32_t nc;         // chunks per sequence
  const float* ln_w;  // time-mix form: ln_x's affine per (head, channel), may be null (1)
  const float* ln_b;  // may be null (0)
};

__device__ __forceinline__ int lds_peek(const int* p) {
  return __builtin_amdgcn_readfirstlane(__atomic_load_n(p, __ATOMIC_RELAXED));
}
// Waits until *flag >= target, then orders every later memory access after the wait.
__device__ __forceinline__ void wait_at_least(const int* flag, int target) {
#pragma clang loop unroll(disable)
  for (int n = 0; n < kSpinMax; ++n) {
    if (lds_peek(flag) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}
// Waits until every one of the kScanW words at flags is >= target.
__device__ __forceinline__ void wait_all_at_least(const int* flags, int target) {
#pragma clang loop unroll(disable)
  for (int n = 0; n < kSpinMax; ++n) {
    int m = lds_peek(flags);
#pragma unroll
    for (int w = 1; w < kScanW; ++w) m = min(m, lds_peek(flags + w));
    if (m >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}
// Publishes value once every earlier LDS access of this wave has completed.
__device__ __forceinline__ void post(int* flag, int value) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __atomic_store_n(flag, value, __ATOMIC_RELAXED);
}

// CK: the checkpoint form used by the backward. It stores, for every chunk, the
// float16 state the chunk's products start from (ck_store) and writes no y.
// ROWS: y staged as whole token rows (the time-mix form always: ln_x needs a token's 64
// outputs together); otherwise through each scan wave's own tile. Measured on the plain form:
// rows 0.920 -> 0.910 ms at D4096-long and 0.245 -> 0.237 ms at L24-D1024 (256 heads), but
// 0.193 -> 0.200 ms at L12-D768 (96 heads), where each scan wave's extra steps per chunk cost.
template <int MODE, bool CK, bool ROWS = true>
__device__ __forceinline__ void fused_body(const FusedParams& p, unsigned char* ring, int unit) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int H = p.in.H, T = p.in.T, nc = p.nc;
  const int bb = unit / H, hh = unit % H;
  const uint32_t tstride = (uint32_t)H * kN;  // elements between tokens
  const int64_t seq_base = (int64_t)bb * T * H * kN + (int64_t)hh * kN;  // element offset of (bb, 0, hh, 0)
  int* ready = reinterpret_cast<int*>(ring + kCtrlOff);
  int* consumed = ready + kRing;
  int* y_done = consumed + kScanW;
  if (threadIdx.x < kRing) ready[threadIdx.x] = -1;
  if (threadIdx.x < kScanW) consumed[threadIdx.x] = 0;
  if (threadIdx.x < kScanW) y_done[threadIdx.x] = 0;
  __syncthreads();

  if (wave >= kScanW) {
    // ---------------------------------------------------------------- prep waves
    // The wave's chunks are c0, c0 + kPrepW, ... Two sets of row registers alternate: the
    // r, a, b, k rows of the next chunk are loaded between the two phases of the current
    // chunk's prep, so their latency passes during its solve and products and the next
    // slot wait (w, a fifth of the prep's input bytes, is loaded when the chunk starts; the
    // scan waves load v themselves). Past the wave's last chunk the loads repeat its last
    // chunk (unconditional, no branch).
    const int c0 = wave - kScanW;
    if (c0 >= nc) return;
    constexpr unsigned kRows = CK ? kRowA | kRowB | kRowK : kRowsAll;  // no readout, no r
    // the checkpoint form takes w with the rows (measured: backward 0.571 -> 0.560 ms at 96
    // heads; the prefill measured no gain at 96 heads and a 1% loss at 256)
    constexpr bool kW = CK && MODE == kPrepPlain;
    const int last = c0 + (nc - 1 - c0) / kPrepW * kPrepW;  // this wave's last chunk
    auto nt_of = [&](int c) { return min(kC, T - c * kC); };
    auto base_of = [&](int c) { return seq_base + (int64_t)c * kC * tstride; };
    // one chunk; returns false after the wave's last chunk
    auto item = [&](int& c, PrepRows& cur, PrepRows& nxt) {
      const int slot = c % kRing;
      unsigned char* rec = ring + slot * kSlot;
      const int nt = nt_of(c);
      const int64_t base = base_of(c);
      PrepRaw x;
      x.nt = nt;
      if constexpr (!kW) prep_load_w<MODE>(p.in, base, nt, x);
      wait_all_at_least(consumed, c - kRing + 1);  // the slot's previous chunk has been read
      prep_rows_to_raw<kRows, kW>(cur, rec, x);    // the slot's start stages the rows
      PrepMid m;
      prep_grams<MODE, !CK>(x, reinterpret_cast<float*>(rec), rec, m);
      const int cn = min(c + kPrepW, last);
      prep_load_rows<kRows, kW>(p.in, base_of(cn), nt_of(cn), nxt);
      prep_finish<!CK>(m, reinterpret_cast<float*>(rec), rec);
      post(&ready[slot], c);
      c += kPrepW;
      return c < nc;
    };
    PrepRows ra, rb;
    prep_load_rows<kRows, kW>(p.in, base_of(c0), nt_of(c0), ra);
    int c = c0;
    while (item(c, ra, rb) && item(c, rb, ra)) {
    }
    return;
  }

  // ------------------------------------------------------------------ scan waves
  __builtin_amdgcn_s_setprio(2);  // the chain of the state, ahead of the prep's work on this SIMD
  const int w = wave;
  Mma32::acc St[4];  // element e of St[kt] = S[i = 16 w + li][j = 16 kt + 4 g + e]
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) St[kt] = Mma32::zero();
  if (p.s_in) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float4 s = *reinterpret_cast<const float4*>(p.s_in + ((int64_t)unit * kN + 16 * w + li) * kN +
                                                        16 * kt + 4 * g);
      St[kt] = Mma32::acc{f32x4{s.x, s.y, s.z, s.w}};
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the state has landed
  // row stores: lane l writes token 4 w + l / 16 of a chunk, values 4 (l % 16) .. + 3;
  // tile stores: lane l writes token l / 4, values 16 w + 4 (l % 4) .. + 3
  constexpr bool kRows = ROWS || (MODE == kPrepTmix && !CK);
  float* ybase = kRows ? p.y + seq_base + 4 * (lane & 15) : p.y + seq_base + 16 * w + 4 * (lane & 3);
  float* ystage = reinterpret_cast<float*>(ring + kYOff);
  unsigned char* ytile = ring + kYTileOff + w * kYTile;
  auto slot_of = [&](int c) { return ring + (c % kRing) * kSlot; };
  // v of chunk c for this wave: V[t = 4g + e][i = 16 w + li], raw bfloat16 bits (a
  // quarter-wave reads 32 contiguous bytes of one token row); tokens past the end read
  // the last token (their record coefficients are zero)
  const uint16_t* vbase = p.v + seq_base + 16 * w + li;
  auto load_v = [&](int c, uint32_t (&vr)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = min(c * kC + 4 * g + e, T - 1);
      vr[e] = vbase[(int64_t)t * tstride];
    }
  };
  // y of chunk c: each scan wave writes its 16 values of every token into the staged rows of
  // buffer c % 2 and posts; one chunk later, once all four have posted, wave w stores tokens
  // 4w .. 4w + 3 whole (16 lanes per token, one DPP row). A wave writes buffer c % 2 only after
  // every wave has posted chunk c - 1, so every read of chunk c - 2's rows has completed.
  // Time-mix form: ln_x (mean, then the population variance of the centred values, then the
  // affine) on the whole row before the store, by two row sums.
  constexpr bool kLn = MODE == kPrepTmix && !CK;
  float ln_g[4] = {1.f, 1.f, 1.f, 1.f}, ln_o[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kLn) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ch = hh * kN + 4 * (lane & 15) + e;
      if (p.ln_w) ln_g[e] = p.ln_w[ch];
      if (p.ln_b) ln_o[e] = p.ln_b[ch];
    }
  }
  auto stage_y = [&](const f32x4 yv, int cy) {
    st_off<float4>(ystage, (uint32_t)((((cy & 1) * kC + li) * kYRowF + 16 * w + 4 * g) * 4),
                   make_float4(yv[0], yv[1], yv[2], yv[3]));
    post(&y_done[w], cy + 1);
  };
  // the tile's previous reads completed before this wave's previous post (its wait covers every
  // LDS access of the wave)
  auto tile_y = [&](const f32x4 yv, int cy) {
    st_off<float4>(ytile, (uint32_t)(li * kYRow + 16 * g), make_float4(yv[0], yv[1], yv[2], yv[3]));
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    const float4 yq = ld_off<float4>(ytile, (uint32_t)((lane >> 2) * kYRow + 16 * (lane & 3)));
    const int t = cy * kC + (lane >> 2);
    if (t < T) *reinterpret_cast<float4*>(ybase + (int64_t)t * tstride) = yq;
  };
  auto flush_y = [&](int cy) {
    wait_all_at_least(y_done, cy + 1);
    const int tt = 4 * w + (lane >> 4);
    float4 q = ld_off<float4>(ystage, (uint32_t)((((cy & 1) * kC + tt) * kYRowF + 4 * (lane & 15)) * 4));
    if constexpr (kLn) {
      const float mu = row16_sum((q.x + q.y) + (q.z + q.w)) * (1.f / kN);
      const float d0 = q.x - mu, d1 = q.y - mu, d2 = q.z - mu, d3 = q.w - mu;
      const float var = row16_sum(fmaf(d0, d0, fmaf(d1, d1, fmaf(d2, d2, d3 * d3)))) * (1.f / kN);
      const float inv = 1.f / sqrtf(var + kLnEps);
      q = make_float4(fmaf(d0 * inv, ln_g[0], ln_o[0]), fmaf(d1 * inv, ln_g[1], ln_o[1]),
                      fmaf(d2 * inv, ln_g[2], ln_o[2]), fmaf(d3 * inv, ln_g[3], ln_o[3]));
    }
    const int t = cy * kC + tt;
    if (t < T) *reinterpret_cast<float4*>(ybase + (int64_t)t * tstride) = q;
  };
  Frag fa, fb;
  uint32_t va[4], vb[4];  // v two chunks ahead: the set of chunk c is reloaded with chunk c + 2
  load_v(0, va);
  load_v(min(1, nc - 1), vb);
  wait_at_least(&ready[0], 0);
  read_frag(slot_of(0), fa);
  int c = 0;
  // One chunk: the next chunk's fragments are read (its slot waited for) before this
  // chunk's products are issued. Past the last chunk the reads repeat the last chunk, so
  // they are unconditional (a read inside a branch would make the compiler wait for it at
  // the join). Returns false after the last chunk.
  auto body = [&](Frag& cur, Frag& nxt, uint32_t (&vc)[4]) {
    const int cn = min(c + 1, nc - 1);
    wait_at_least(&ready[cn % kRing], cn);
    read_frag(slot_of(cn), nxt);
#pragma unroll
    for (int e = 0; e < 4; ++e) cur.v[e] = vc[e];
    if constexpr (CK) {
      if (!(c & 1)) ck_store(p.ck + ((int64_t)unit * ((nc + 1) >> 1) + (c >> 1)) * kCkHalves, 16 * w, St);
    }
    const f32x4 yv = scan_step<!CK>(St, cur);
    load_v(min(c + 2, nc - 1), vc);
    if constexpr (!CK && kRows) {
      if (c > 0) flush_y(c - 1);  // the previous chunk, which every wave has staged
      stage_y(yv, c);
    } else if constexpr (!CK) {
      tile_y(yv, c);
    }
    post(&consumed[w], cn + 1);  // every fragment up to chunk cn is in registers
    ++c;
    return c < nc;
  };
  while (body(fa, fb, va) && body(fb, fa, vb)) {
  }
  if constexpr (!CK && kRows) flush_y(nc - 1);
  if (p.s_out) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      *reinterpret_cast<float4*>(p.s_out + ((int64_t)unit * kN + 16 * w + li) * kN + 16 * kt + 4 * g) =
          make_float4(St[kt].v[0], St[kt].v[1], St[kt].v[2], St[kt].v[3]);
  }
}

}  // namespace fused
}  // namespace rwkv7
