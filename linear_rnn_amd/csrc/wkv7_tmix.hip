// The WKV-7 time-mix operator with its prologue and epilogue fused around the
// recurrence (RWKV-7 G0 7.2B notes, lshu.cn/news/198401, section 7.1, "x070
// architecture, the two core operators"):
//
//   prologue  w = exp(-exp(w_raw))                       (decay, from float32 w_raw)
//             kk_hat = kk / max(|kk|_2, 1e-12)           (per head, as F.normalize)
//             a = -kk_hat,  b = kk_hat * a_lr            (the kernel's two slots)
//   recurrence S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T,  y_t = S_t r_t
//   epilogue  out = (y - mean) / sqrt(var + 64e-5) * ln_w + ln_b
//             (ln_x: a GroupNorm with one group per head; mean and population
//              variance over the head's 64 channels of one token)
//
// One workgroup owns one head (WAVES waves of 64/WAVES value rows, the lane
// layout and the per-token update of the sequential kernel), so a head's 64
// outputs of a token are all in the workgroup and the GroupNorm never leaves LDS.
// Blocks of TB tokens are staged through LDS: the raw inputs of block n+1 are in
// flight in registers while block n runs three passes (passes 1 and 3 give each
// wave every WAVES-th token):
//   1. prologue, lane = key column: decay, the row's squared norm by a wave
//      reduction, the two slots, written back over the raw values;
//   2. the recurrence, token by token, y into LDS;
//   3. epilogue, lane = channel: mean and variance by wave reductions, affine,
//      one coalesced 256-byte store per token.
// The float32 decay is rounded once per element, as the pages keep it; prefill
// and the single-token step run the same per-row arithmetic (only the number of
// rows a wave holds differs), so T steps reproduce a prefill over T tokens bit
// for bit.
#include "rwkv7_wkv.h"
#include "wkv7_device.hpp"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

constexpr float kGroupNormEps = 64e-5f;
constexpr float kNormalizeEps = 1e-12f;

// Sum over the 64 lanes of a wave; every lane ends with the same bits (each
// step adds a pair of partial sums that both partners hold).
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x = x + __shfl_xor(x, 16);
  x = x + __shfl_xor(x, 32);
  return x;
}

template <bool BF16>
struct TmixIn {
  static constexpr int kEpv = BF16 ? 8 : 4;  // elements per 16-byte load
  static constexpr int kEsz = BF16 ? 2 : 4;
  __device__ static void store(float* dst, const uint4 q) {
    if constexpr (BF16) {
      reinterpret_cast<float4*>(dst)[0] = make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
      reinterpret_cast<float4*>(dst)[1] = make_float4(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w));
    } else {
      *reinterpret_cast<uint4*>(dst) = q;
    }
  }
};

template <bool BF16, int TB, int WAVES>
__global__ __launch_bounds__(kWave* WAVES) void wkv7_tmix_kernel(TmixParams p) {
  constexpr int kWaves = WAVES;
  constexpr int kThreads = kWave * kWaves;
  constexpr int kRpw = kN / kWaves;  // value rows per wave
  constexpr int kMr = kRpw / 4;      // rows per lane
  using In = TmixIn<BF16>;
  constexpr int kEpv = In::kEpv;
  constexpr int kSeg = kN / kEpv;       // 16-byte loads per token row of an input
  constexpr int kSegW = kN / 4;         // 16-byte loads per token row of float32 w_raw
  // staged tensors, in LDS slot order: r, w_raw -> w, k, kk -> a, a_lr -> b, then v
  constexpr int kNq = (TB * kSeg + kThreads - 1) / kThreads;
  constexpr int kNqW = (TB * kSegW + kThreads - 1) / kThreads;

  __shared__ __align__(16) float kv_lds[TB][5][kN];
  __shared__ __align__(16) float v_lds[TB][kN];
  __shared__ __align__(16) float y_lds[TB][kN];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c = lane & 15;
  const int ri = lane >> 4;

  const int64_t unit = xcd_swizzle(blockIdx.x, gridDim.x);
  const int64_t bb = unit / p.H;
  const int64_t hh = unit % p.H;
  const int64_t T = p.T;
  const int64_t tok_stride = (int64_t)p.H * kN;
  const int64_t seq_base = (bb * T * p.H + hh) * kN;  // element offset of token 0
  const int row0 = wave * kRpw;

  // inputs in dtype, by staging slot (slot 1 is w_raw, float32 for every dtype)
  const char* src[6] = {static_cast<const char*>(p.r), nullptr, static_cast<const char*>(p.k),
                        static_cast<const char*>(p.kk), static_cast<const char*>(p.a_lr),
                        static_cast<const char*>(p.v)};
  const char* wsrc = reinterpret_cast<const char*>(p.w_raw);

  float4 S[kMr];
#pragma unroll
  for (int m = 0; m < kMr; ++m) {
    const int row = row0 + 4 * m + ri;
    S[m] = p.s_in ? *reinterpret_cast<const float4*>(p.s_in + (unit * kN + row) * kN + 4 * c)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  uint4 stg[6][kNq];
  uint4 stw[kNqW];
  // For a prefill every lane loads and stores unconditionally (pieces past the
  // end repeat the last piece, tokens at or past T repeat token T-1), so no
  // divergent branch sits around the loads: such branches make the compiler wait
  // for each new prefetch before issuing the next. The single-token step (TB = 1,
  // no loop) loads only the pieces that exist.
  auto issue = [&](int64_t t0) {
#pragma unroll
    for (int x = 0; x < 6; ++x) {
      if (x == 1) continue;
#pragma unroll
      for (int q = 0; q < kNq; ++q) {
        if constexpr (TB == 1) {
          const int e = tid + kThreads * q;
          if (e < kSeg) stg[x][q] = *reinterpret_cast<const uint4*>(src[x] + (seq_base + t0 * tok_stride + e * kEpv) * In::kEsz);
        } else {
          const int e = min(tid + kThreads * q, TB * kSeg - 1);
          const int tok = e / kSeg, seg = e % kSeg;
          const int64_t t = min(t0 + tok, T - 1);
          stg[x][q] = *reinterpret_cast<const uint4*>(src[x] + (seq_base + t * tok_stride + seg * kEpv) * In::kEsz);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kNqW; ++q) {
      if constexpr (TB == 1) {
        const int e = tid + kThreads * q;
        if (e < kSegW) stw[q] = *reinterpret_cast<const uint4*>(wsrc + (seq_base + t0 * tok_stride + e * 4) * 4);
      } else {
        const int e = min(tid + kThreads * q, TB * kSegW - 1);
        const int tok = e / kSegW, seg = e % kSegW;
        const int64_t t = min(t0 + tok, T - 1);
        stw[q] = *reinterpret_cast<const uint4*>(wsrc + (seq_base + t * tok_stride + seg * 4) * 4);
      }
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int x = 0; x < 6; ++x) {
      if (x == 1) continue;
#pragma unroll
      for (int q = 0; q < kNq; ++q) {
        const int e = TB == 1 ? tid + kThreads * q : min(tid + kThreads * q, TB * kSeg - 1);
        const int tok = e / kSeg, seg = e % kSeg;
        if (TB > 1 || e < kSeg) In::store(x < 5 ? &kv_lds[tok][x][seg * kEpv] : &v_lds[tok][seg * kEpv], stg[x][q]);
      }
    }
#pragma unroll
    for (int q = 0; q < kNqW; ++q) {
      const int e = TB == 1 ? tid + kThreads * q : min(tid + kThreads * q, TB * kSegW - 1);
      const int tok = e / kSegW, seg = e % kSegW;
      if (TB > 1 || e < kSegW) *reinterpret_cast<uint4*>(&kv_lds[tok][1][seg * 4]) = stw[q];
    }
  };

  const float* lnw = p.ln_w ? p.ln_w + hh * kN : nullptr;
  const float* lnb = p.ln_b ? p.ln_b + hh * kN : nullptr;
  const float gw = lnw ? lnw[lane] : 1.f;  // lane = channel in the epilogue
  const float gb = lnb ? lnb[lane] : 0.f;

  if (T > 0) issue(0);
  // The state and the first block's loads complete here, together, so the loop
  // below never waits for them (a loop-carried value that may still be in flight
  // makes the compiler wait for every outstanding load, prefetches included, at
  // each block). The single-token step runs one block, so it lets the state load
  // overlap the prologue instead.
  if constexpr (TB > 1) __builtin_amdgcn_s_waitcnt(0x0f70);
  for (int64_t t0 = 0; t0 < T; t0 += TB) {
    const int ntok = (T - t0 < TB) ? (int)(T - t0) : TB;
    __syncthreads();  // every wave is done with the previous block's LDS
    commit();
    __syncthreads();
    if (t0 + TB < T) issue(t0 + TB);  // in flight while this block is computed

    // ---- 1. prologue (lane = key column j)
    for (int tt = wave; tt < ntok; tt += kWaves) {
      const float u = kv_lds[tt][1][lane];
      const float kk = kv_lds[tt][3][lane];
      const float alr = kv_lds[tt][4][lane];
      const float n2 = wave_sum(kk * kk);
      const float kh = kk * (1.f / fmaxf(sqrtf(n2), kNormalizeEps));
      kv_lds[tt][1][lane] = expf(-expf(u));
      kv_lds[tt][3][lane] = -kh;
      kv_lds[tt][4][lane] = kh * alr;
    }
    __syncthreads();

    // ---- 2. recurrence (a whole block: the next token's LDS reads are in flight during this one)
    auto load_tok = [&](int tt, float4& r4, float4& w4, float4& k4, float4& a4, float4& b4, float (&vm)[kMr]) {
      r4 = *reinterpret_cast<const float4*>(&kv_lds[tt][0][4 * c]);
      w4 = *reinterpret_cast<const float4*>(&kv_lds[tt][1][4 * c]);
      k4 = *reinterpret_cast<const float4*>(&kv_lds[tt][2][4 * c]);
      a4 = *reinterpret_cast<const float4*>(&kv_lds[tt][3][4 * c]);
      b4 = *reinterpret_cast<const float4*>(&kv_lds[tt][4][4 * c]);
#pragma unroll
      for (int m = 0; m < kMr; ++m) vm[m] = v_lds[tt][row0 + 4 * m + ri];
    };
    if (TB > 1 && ntok == TB) {
      float4 r4, w4, k4, a4, b4, r4n, w4n, k4n, a4n, b4n;
      float vm[kMr], vmn[kMr];
      load_tok(0, r4, w4, k4, a4, b4, vm);
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        if (tt + 1 < TB) load_tok(tt + 1, r4n, w4n, k4n, a4n, b4n, vmn);
        const float yo = token_update<kMr>(S, r4, w4, k4, a4, b4, vm, c);
        if (c < kMr) y_lds[tt][row0 + 4 * c + ri] = yo;
        if (tt + 1 < TB) {
          r4 = r4n, w4 = w4n, k4 = k4n, a4 = a4n, b4 = b4n;
#pragma unroll
          for (int m = 0; m < kMr; ++m) vm[m] = vmn[m];
        }
      }
    } else {
      for (int tt = 0; tt < ntok; ++tt) {
        float4 r4, w4, k4, a4, b4;
        float vm[kMr];
        load_tok(tt, r4, w4, k4, a4, b4, vm);
        const float yo = token_update<kMr>(S, r4, w4, k4, a4, b4, vm, c);
        if (c < kMr) y_lds[tt][row0 + 4 * c + ri] = yo;
      }
    }
    __syncthreads();

    // ---- 3. epilogue (lane = channel i)
    for (int tt = wave; tt < ntok; tt += kWaves) {
      const float y = y_lds[tt][lane];
      const float mu = wave_sum(y) * (1.f / kN);
      const float d = y - mu;
      const float var = wave_sum(d * d) * (1.f / kN);
      const float o = d * (1.f / sqrtf(var + kGroupNormEps));
      p.out[seq_base + (t0 + tt) * tok_stride + lane] = fmaf(o, gw, gb);
    }
  }

  if (p.s_out) {
#pragma unroll
    for (int m = 0; m < kMr; ++m) {
      const int row = row0 + 4 * m + ri;
      *reinterpret_cast<float4*>(p.s_out + (unit * kN + row) * kN + 4 * c) = S[m];
    }
  }
}

template <bool BF16, int TB, int WAVES>
hipError_t launch_cfg(const TmixCall& c) {
  TmixParams p = c.p;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&wkv7_tmix_kernel<BF16, TB, WAVES>),
                         dim3((uint32_t)(c.B * c.H)), dim3(kWave * WAVES), args, 0, c.stream);
}

}  // namespace

hipError_t launch_tmix(const TmixCall& c) {
  if (c.dtype == 1 && c.p.T > 1) {
    if (c.algo == RWKV7_ALGO_CHUNKED_SPLIT) return launch_tmix_chunked(c);
    if (c.algo == RWKV7_ALGO_CHUNKED) return launch_tmix_fused(c);
  }
  // the single-token step: one token per block, four waves of 16 rows (bound by HBM);
  // a prefill: sixteen-token blocks, eight waves of 8 rows (two per SIMD, to hide the
  // per-token dependency chain)
  if (c.dtype == 1) return c.p.T == 1 ? launch_cfg<true, 1, 4>(c) : launch_cfg<true, 16, 8>(c);
  return c.p.T == 1 ? launch_cfg<false, 1, 4>(c) : launch_cfg<false, 16, 8>(c);
}

}  // namespace rwkv7
