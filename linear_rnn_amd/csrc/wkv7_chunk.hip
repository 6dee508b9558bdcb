// Chunked WKV-7 prefill: the recurrence rewritten per 16-token chunk so that the
// intra-chunk work becomes small dense contractions on MFMA, with the 64x64
// state carried from chunk to chunk in float32 accumulators.
//
// Recurrence (RWKV-7 G0 7.2B notes, lshu.cn/news/198401, section 7.1), per head:
//   S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T,   y_t = S_t r_t.
//
// Chunk form (derived; WY / "DPLR" style). Tokens t = 0..15 of a chunk, state
// S0 at its start, gamma_t = sum_{u<=t} log w_u (per key column j):
//   U[t]   = S_{t-1} a_t  (row vector over values i; the "state*a" term)
//   U      = A^ S0^T + L_ab U + L_ak V        A^[t] = a_t e^{gamma_{t-1}}
//   Y      = R^ S0^T + L_rb U + L_rk V        R^[t] = r_t e^{gamma_t}
//   S_C^T  = diag(e^{gamma_15}) S0^T + B- U + K- V,
//            B-[j][s] = b_s,j e^{gamma_15 - gamma_s},  K- likewise with k
// with the 16x16 lower-triangular Grams
//   L_ab[t][s] = sum_j a_t,j b_s,j e^{gamma_{t-1} - gamma_s}   (s <  t)
//   L_ak[t][s] = sum_j a_t,j k_s,j e^{gamma_{t-1} - gamma_s}   (s <  t)
//   L_rb[t][s] = sum_j r_t,j b_s,j e^{gamma_t - gamma_s}       (s <= t)
//   L_rk[t][s] = sum_j r_t,j k_s,j e^{gamma_t - gamma_s}       (s <= t).
// Eliminating U with T = (I - L_ab)^{-1} and M_r = L_rb T:
//   U = (T A^) S0^T + (T L_ak) V,   Y = (R^ + M_r A^) S0^T + (M_r L_ak + L_rk) V.
// Everything in parentheses depends only on the chunk's inputs; only three small
// MFMA stages (U, Y and the update) touch the state.
//
// Software pipeline. One workgroup (8 waves, two per SIMD) owns one head. In
// loop iteration i, between two barriers, the waves work on six chunks at once:
//   waves 0-3  S: state phase of chunk i (wave = 16-value block)
//              P: fused products of chunk i+1 (wave = 16-key tile)
//              staging of chunk i+5's six inputs from HBM into LDS
//   wave 4     F: decay factors of chunk i+4;  A^, R^ fragments of chunk i+3
//   wave 5     B: rows of T and M_r of chunk i+2; B-, K-, V fragments of chunk i+3
//   waves 6,7  G: Grams of chunk i+3 (keys 0-31 and 32-63 as two partial sums)
// Each stage reads what an earlier iteration wrote into LDS rings deep enough
// for it, so one barrier per iteration suffices. Only the staging waves issue
// global loads: every other role works from LDS, so no wave ever has a load in
// flight into registers that another role's code also uses (the compiler's
// wait-count insertion cannot tell the roles apart and would otherwise make
// the staging waves wait for their own earlier stores). Within a stage, all LDS
// reads are issued before its first LDS write, so each stage pays about one
// LDS round trip rather than one per fragment.
//
// Numerics. Decay factors are running products of w: every factor that
// multiplies the state is <= 1. Each Gram factors e^{gamma_x - gamma_y} through
// the decay at token 7 of its chunk, so no factor exceeds w_min^-8; w is clamped
// below at 2^-15 (which moves a decayed term by at most 2^-15 of its size),
// keeping every factor inside the float32 / bfloat16 exponent range. Grams
// accumulate bfloat16 hi+lo splits of both operands (~2^-16 relative); T and M_r
// come from float32 back substitution; the other operands are rounded once to
// float16. Operands must stay inside the float16 range (|x| < 2^15), which
// RWKV-7 activations and states do.
//
// MFMA layouts (gfx950, wave64; l = lane, li = l % 16, g = l / 16):
//   16x16x16 f16  : A[m=li][k=4g+e], B[k=4g+e][n=li], D[m=4g+e][n=li], e = 0..3
//   16x16x32 bf16 : A[m=li][k=8g+e], B[k=8g+e][n=li], e = 0..7
// A result D (M x N) in registers is unchanged a B operand for K = M, so every
// product is oriented so that results feed the next MFMA from registers or from
// a per-lane LDS "fragment" slot, with no transposition.
#include <type_traits>

#include "wkv7_device.hpp"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 16;        // tokens per chunk
constexpr int kMid = 7;       // reference token of the Gram factorisation
constexpr float kWMin = 0x1p-15f;
constexpr int kNP = kN + 4;   // padded row of float [token][column] arrays
constexpr int kThreads = 512;

__device__ __forceinline__ f32x4 mfma16(half4 a, half4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half4 to_h4(f32x4 x) {
  return half4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}
__device__ __forceinline__ half4 to_h4(float a, float b, float c, float d) {
  return half4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
}
__device__ __forceinline__ f32x4 to_f4(half4 h) {
  return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }


// hi + lo bfloat16 split of 8 floats: hi keeps the top 16 bits (truncation), lo
// is the rounded remainder, so x = hi + lo to ~2^-17 relative.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t u = __float_as_uint(x[e]);
    const float h = __uint_as_float(u & 0xffff0000u);
    hi[e] = __builtin_bit_cast(__bf16, (uint16_t)(u >> 16));
    lo[e] = (__bf16)(x[e] - h);
  }
}

// Load / store at a 32-bit byte offset from a wave-uniform base, so the
// compiler can use the scalar-base addressing form (no 64-bit VALU math).
template <class V>
__device__ __forceinline__ V ld_off(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const V*>(static_cast<const char*>(base) + byte_off);
}
template <class V>
__device__ __forceinline__ void st_off(void* base, uint32_t byte_off, V v) {
  *reinterpret_cast<V*>(static_cast<char*>(base) + byte_off) = v;
}

// Input element storage in LDS: raw bfloat16 bits or float.
template <bool BF16>
struct In;
template <>
struct In<true> {
  using T = uint16_t;
  static constexpr int kRow = kN + 8;  // 144-byte rows: 16-byte reads by row index are conflict free
  __device__ static float get(const T* p) { return __uint_as_float((uint32_t)*p << 16); }
  __device__ static float widen(uint32_t raw) { return __uint_as_float(raw << 16); }
  __device__ static void get8(const T* p, float* out) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    out[0] = bf16_lo(q.x); out[1] = bf16_hi(q.x); out[2] = bf16_lo(q.y); out[3] = bf16_hi(q.y);
    out[4] = bf16_lo(q.z); out[5] = bf16_hi(q.z); out[6] = bf16_lo(q.w); out[7] = bf16_hi(q.w);
  }
  __device__ static void get4(const T* p, float* out) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    out[0] = bf16_lo(q.x); out[1] = bf16_hi(q.x); out[2] = bf16_lo(q.y); out[3] = bf16_hi(q.y);
  }
};
template <>
struct In<false> {
  using T = float;
  [[maybe_unused]] static constexpr int kRow = kN + 4;  // (the float32 path is not launched)
  __device__ static float get(const T* p) { return *p; }
  __device__ static float widen(uint32_t raw) { return __uint_as_float(raw); }
  __device__ static void get8(const T* p, float* out) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
  __device__ static void get4(const T* p, float* out) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  }
};

struct ChunkParams {
  const void* in[6];  // r, w, k, v, a, b
  const float* s_in;
  float* y;
  float* s_out;
  int32_t T;
  int32_t H;
};

// Tensors staged through LDS, in slot order.
enum { kR = 0, kK = 1, kV = 2, kA = 3, kB = 4, kW = 5, kStaged = 6 };
constexpr int kSrc[kStaged] = {0, 2, 3, 4, 5, 1};  // index into ChunkParams::in
constexpr int kRing = 3;  // input slots: chunks i+3 (fragments, Grams), i+4 (factors), i+5 (being filled)
enum { kFacE = 0, kFacS = 1, kFacG = 2, kFacF = 3 };
enum { kLab = 0, kLak = 1, kLrb = 2, kLrk = 3 };

template <bool BF16>
struct Pipe {
  using IT = typename In<BF16>::T;
  IT X[kRing][kStaged][kC][In<BF16>::kRow];  // raw inputs, slot = chunk % kRing
  float fac[2][4][kC + 1][kNP];           // E (row t+1 = e^{gamma_t}, row 0 = 1), Suf, G (row t+1 = e^{gamma_t-gamma_7}), F
  float gp[2][2][4][kC][kC];              // Gram partial sums (key halves) [t][s]
  float lk[2][2][kC][kC];                 // summed L_ak^T [s][t] and L_rk [t][s]
  _Float16 tm[2][2][kC][kC];              // rows of T and of M_r
  half4 oa[3][2][4][kWave];               // A^ A-fragments, R^ seeds, per key tile
  half4 ob[4][3][4][kWave];               // B- and K- A-fragments (key tiles), V B-fragments (value blocks)
  float gam[4][kN];                       // e^{gamma_15}
  half4 ff[2][2][4][kWave];               // (T A^) and (R^ + M_r A^) A-fragments, per key tile
  half4 fl[2][2][kWave];                  // (T L_ak) and (M_r L_ak + L_rk) A-fragments
};

template <bool BF16>
__global__ __launch_bounds__(kThreads) void wkv7_chunk_kernel(ChunkParams p) {
  using IO = In<BF16>;
  using IT = typename IO::T;
  constexpr int kEpv = 16 / sizeof(IT);                 // elements per 16-byte load
  constexpr int kSeg = kN / kEpv;                        // loads per token row
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Pipe<BF16>& sm = *reinterpret_cast<Pipe<BF16>*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15;
  const int g = lane >> 4;

  const int unit = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  const int bb = unit / p.H, hh = unit % p.H;
  const int T = p.T;
  const int tok_stride = p.H * kN;  // elements between consecutive tokens
  const int64_t seq_base = ((int64_t)bb * T * p.H + hh) * kN;
  const int nch = (T + kC - 1) / kC;
  // Per-head bases (uniform); every in-head offset below fits in 32 bits.
  float* yout = p.y + seq_base;
  const bool state_wave = wave < 4;

  // ---- state S^T (waves 0-3): element e of St[kt] is S[i = 16 wave + li][j = 16 kt + 4 g + e]
  f32x4 St[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) St[kt] = zero4();
  if (state_wave && p.s_in) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float4 q = *reinterpret_cast<const float4*>(p.s_in + ((int64_t)unit * kN + 16 * wave + li) * kN +
                                                        16 * kt + 4 * g);
      St[kt] = f32x4{q.x, q.y, q.z, q.w};
    }
  }
  // Complete the state loads here, once: otherwise the loop's wait counts must
  // allow for them on every iteration and end up waiting for unrelated stores.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- staging (global -> registers at the top of an iteration, -> LDS at its
  // end; past-the-end tokens are clamped to T-1 and stored as zeros, and the
  // factor stage turns them into identity tokens: w = 1, everything else 0).
  // State wave w loads all of tensor w and a quarter of tensors 4 and 5, so
  // every load instruction has a wave-uniform base.
  constexpr int kPerTensor = kC * kSeg;            // 16-byte loads per tensor per chunk
  constexpr int kOwn = kPerTensor / kWave;         // own-tensor loads per lane (2 or 4)
  constexpr int kQuarter = kPerTensor / 4;         // loads of tensor 4 (and of 5) per wave (32 or 64)
  constexpr int kShr = 2 * kQuarter / kWave;       // shared loads per lane (1 or 2)
  constexpr uint32_t kEsz = sizeof(IT);
  uint4 stg[kOwn + kShr];
  auto stage_slot = [&](int q, int& x, int& tok, int& seg) {
    int e;
    if (q < kOwn) {
      e = lane + kWave * q;
      x = wave;
    } else {
      const int e2 = lane + kWave * (q - kOwn);  // 0 .. 2 * kQuarter - 1
      x = 4 + e2 / kQuarter;
      e = kQuarter * wave + e2 % kQuarter;
    }
    tok = e / kSeg;
    seg = e % kSeg;
  };
  auto issue_stage = [&](int c) {
#pragma unroll
    for (int q = 0; q < kOwn + kShr; ++q) {
      int x, tok, seg;
      stage_slot(q, x, tok, seg);
      const int t = min(c * kC + tok, T - 1);
      const void* base;
      if (q < kOwn) {  // own tensor: pick the wave's pointer (uniform)
        const void* b1 = static_cast<const IT*>(p.in[kSrc[1]]) + seq_base;
        const void* b2 = static_cast<const IT*>(p.in[kSrc[2]]) + seq_base;
        const void* b3 = static_cast<const IT*>(p.in[kSrc[3]]) + seq_base;
        const void* b0 = static_cast<const IT*>(p.in[kSrc[0]]) + seq_base;
        base = wave == 1 ? b1 : wave == 2 ? b2 : wave == 3 ? b3 : b0;
      } else {  // tensor 4 or 5: uniform per instruction when kQuarter is a multiple of the wave
        const void* b4 = static_cast<const IT*>(p.in[kSrc[4]]) + seq_base;
        const void* b5 = static_cast<const IT*>(p.in[kSrc[5]]) + seq_base;
        base = x == 4 ? b4 : b5;
      }
      stg[q] = ld_off<uint4>(base, (uint32_t)(t * tok_stride + seg * kEpv) * kEsz);
    }
  };
  auto commit_stage = [&](int c) {
    const bool tail = (c + 1) * kC > T;  // uniform: only the last chunk has dead tokens
#pragma unroll
    for (int q = 0; q < kOwn + kShr; ++q) {
      int x, tok, seg;
      stage_slot(q, x, tok, seg);
      uint4 v = stg[q];
      if (tail) {  // component-wise select (a whole-vector select is lowered through scratch memory)
        const bool live = c * kC + tok < T;
        v.x = live ? v.x : 0u;
        v.y = live ? v.y : 0u;
        v.z = live ? v.z : 0u;
        v.w = live ? v.w : 0u;
      }
      *reinterpret_cast<uint4*>(&sm.X[c % kRing][x][tok][seg * kEpv]) = v;
    }
  };

  // y of chunk ychunk: yout4[e] = y[t = 4g + e][i = 16 wave + li]. The state phase
  // leaves it in registers and the next iteration stores it right after issuing
  // its staging loads: loads and stores share one wait counter, so stores issued
  // late in an iteration would hold up the commit's wait (or the next loads).
  f32x4 yout4 = zero4();
  int ychunk = -1;
  auto store_y = [&]() {
    if (ychunk >= 0) {
      const int t0 = ychunk * kC + 4 * g;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t0 + e < T) st_off<float>(yout, (uint32_t)((t0 + e) * tok_stride + 16 * wave + li) * 4u, yout4[e]);
      ychunk = -1;
    }
  };

  for (int it = -5; it < nch; ++it) {
    const int cX = it + 5, cF = it + 4, cG = it + 3, cB = it + 2, cP = it + 1, cS = it;
    const bool doF = cF >= 0 && cF < nch, doG = cG >= 0 && cG < nch, doB = cB >= 0 && cB < nch;
    const bool doP = cP >= 0 && cP < nch, doS = cS >= 0, doX = cX < nch;

    if (state_wave) {
      issue_stage(cX);  // unconditional (clamped), committed at the end of this iteration
      store_y();

      // ================= P: fused products of chunk cP (wave = key tile; wave 0 also the 16x16 ones)
      if (doP) {
        const int kt = wave;
        const int os = cP % 3, ts = cP & 1;
        const half4 aT = sm.oa[os][0][kt][lane];                                     // A^ (M = key, K = t')
        const half4 tB = *reinterpret_cast<const half4*>(&sm.tm[ts][0][li][4 * g]);  // T^T as B: T[t = li][4g..]
        const half4 mB = *reinterpret_cast<const half4*>(&sm.tm[ts][1][li][4 * g]);
        sm.ff[ts][0][kt][lane] = to_h4(mfma16(aT, tB, zero4()));                           // (T A^)^T
        sm.ff[ts][1][kt][lane] = to_h4(mfma16(aT, mB, to_f4(sm.oa[os][1][kt][lane])));     // (R^ + M_r A^)^T
        if (wave == 0) {
          const float4 la = *reinterpret_cast<const float4*>(&sm.lk[ts][0][li][4 * g]);  // L_ak^T as A
          const half4 laA = to_h4(la.x, la.y, la.z, la.w);
          sm.fl[ts][0][lane] = to_h4(mfma16(laA, tB, zero4()));
          const float4 lrk = *reinterpret_cast<const float4*>(&sm.lk[ts][1][li][4 * g]);  // L_rk^T seed
          sm.fl[ts][1][lane] = to_h4(mfma16(laA, mB, f32x4{lrk.x, lrk.y, lrk.z, lrk.w}));
        }
      }

      // ================= S: state phase of chunk cS (wave = value block)
      if (doS) {
        const int fs = cS & 1, os = cS & 3;
        half4 sB[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sB[kt] = to_h4(St[kt]);
        const half4 vB = sm.ob[os][2][wave][lane];
        f32x4 u = zero4(), yv = zero4();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          u = mfma16(sm.ff[fs][0][kt][lane], sB[kt], u);
          yv = mfma16(sm.ff[fs][1][kt][lane], sB[kt], yv);
        }
        u = mfma16(sm.fl[fs][0][lane], vB, u);
        yv = mfma16(sm.fl[fs][1][lane], vB, yv);
        const half4 uB = to_h4(u);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const float4 gm = *reinterpret_cast<const float4*>(&sm.gam[os][16 * kt + 4 * g]);
          St[kt][0] *= gm.x;
          St[kt][1] *= gm.y;
          St[kt][2] *= gm.z;
          St[kt][3] *= gm.w;
          St[kt] = mfma16(sm.ob[os][0][kt][lane], uB, St[kt]);
          St[kt] = mfma16(sm.ob[os][1][kt][lane], vB, St[kt]);
        }
        yout4 = yv;  // stored at the top of the next iteration
        ychunk = cS;
      }

      if (doX) commit_stage(cX);
    } else if (wave == 4) {
      // ================= F: decay factors of chunk cF (lane = key column j)
      if (doF) {
        const IT* wrow = &sm.X[cF % kRing][kW][0][lane];
        IT wr[kC];
#pragma unroll
        for (int t = 0; t < kC; ++t) wr[t] = wrow[t * In<BF16>::kRow];
        float wc[kC], rc[kC];
#pragma unroll
        for (int t = 0; t < kC; ++t) {
          float x = IO::widen(wr[t]);
          x = x < kWMin ? kWMin : x;                 // clamp (a NaN passes through)
          wc[t] = cF * kC + t < T ? x : 1.f;         // identity token past the end
          rc[t] = __builtin_amdgcn_rcpf(wc[t]);
        }
        // Six running products, advanced together so their latencies overlap:
        //   E row t+1 = e^{gamma_t} (prefix), S row t = e^{gamma_15 - gamma_t} (suffix),
        //   G row t+1 = e^{gamma_t - gamma_7}, F row s = e^{gamma_7 - gamma_s}.
        float(*f)[kC + 1][kNP] = sm.fac[cF & 1];
        const int j = lane;
        float e = 1.f, sf = 1.f, gu = 1.f, gd = 1.f, fd = 1.f, fu = 1.f;
        f[kFacE][0][j] = 1.f;
        f[kFacS][kC - 1][j] = 1.f;
        f[kFacG][kMid + 1][j] = 1.f;
        f[kFacF][kMid][j] = 1.f;
#pragma unroll
        for (int q = 0; q < kC; ++q) {
          e *= wc[q];
          f[kFacE][q + 1][j] = e;
          if (q < kC - 1) {  // S row kC-2-q
            sf *= wc[kC - 1 - q];
            f[kFacS][kC - 2 - q][j] = sf;
          }
          if (q < kC - 1 - kMid) {  // G rows kMid+2 .. kC: token t = kMid+1+q
            gu *= wc[kMid + 1 + q];
            f[kFacG][kMid + 2 + q][j] = gu;
          }
          if (q <= kMid) {  // G rows kMid .. 0: token t = kMid-1-q, factor 1 / w_{t+1}
            gd *= rc[kMid - q];
            f[kFacG][kMid - q][j] = gd;
          }
          if (q < kMid) {  // F rows kMid-1 .. 0: s = kMid-1-q, factor w_{s+1}
            fd *= wc[kMid - q];
            f[kFacF][kMid - 1 - q][j] = fd;
          }
          if (q < kC - 1 - kMid) {  // F rows kMid+1 .. kC-1: s = kMid+1+q, factor 1 / w_s
            fu *= rc[kMid + 1 + q];
            f[kFacF][kMid + 1 + q][j] = fu;
          }
        }
      }
      // ================= A^ A-fragments (M = key, K = token) and R^ seeds (D layout) of chunk cG,
      // key tiles 2h and 2h+1 for h = 0, 1
      // (each half reads all it needs before its fragment writes)
      if (doG) {
        for (int h = 0; h < 2; ++h) {
          const int xs = cG % kRing, os = cG % 3;
          const float(*fE)[kNP] = sm.fac[cG & 1][kFacE];
          IT araw[2][4];
          float ea[2][4], rv[2][4];
          float4 er[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int kt = 2 * h + u;
            const int j = 16 * kt + li;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              araw[u][e] = sm.X[xs][kA][4 * g + e][j];
              ea[u][e] = fE[4 * g + e][j];
            }
            IO::get4(&sm.X[xs][kR][li][16 * kt + 4 * g], rv[u]);
            er[u] = *reinterpret_cast<const float4*>(&fE[li + 1][16 * kt + 4 * g]);
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int kt = 2 * h + u;
            sm.oa[os][0][kt][lane] = to_h4(IO::widen(araw[u][0]) * ea[u][0], IO::widen(araw[u][1]) * ea[u][1],
                                           IO::widen(araw[u][2]) * ea[u][2], IO::widen(araw[u][3]) * ea[u][3]);
            sm.oa[os][1][kt][lane] =
                to_h4(rv[u][0] * er[u].x, rv[u][1] * er[u].y, rv[u][2] * er[u].z, rv[u][3] * er[u].w);
          }
        }
      }
    } else if (wave == 5) {
      // ================= B: rows of T = (I - L_ab)^{-1} (lanes 0-15) and M_r = L_rb T (lanes 16-31), chunk cB
      // Back substitution for x (I - L_ab) = rhs: x[s] = rhs[s] + sum_{s' > s} x[s'] L_ab[s'][s],
      // right-looking: once x[s'] is final it is folded into every x[s], s < s'. The wave
      // first sums the Gram partials; L_ak and L_rk go on to the fused products.
      if (doB) {
        const int ps = cB & 1;
        float(*lab)[kC] = sm.gp[ps][0][kLab];
        {
          const int idx = lane * 4;  // 64 lanes x 4 = the 256 entries of each 16x16 matrix
          const int r = idx / kC, c = idx % kC;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            float4 a = *reinterpret_cast<const float4*>(&sm.gp[ps][0][m][r][c]);
            const float4 b = *reinterpret_cast<const float4*>(&sm.gp[ps][1][m][r][c]);
            a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
            if (m == kLab || m == kLrb) {
              *reinterpret_cast<float4*>(&sm.gp[ps][0][m][r][c]) = a;  // in place, [t][s]
            } else if (m == kLrk) {
              *reinterpret_cast<float4*>(&sm.lk[ps][1][r][c]) = a;  // L_rk [t][s]
            } else {
              // L_ak^T [s][t]: element (t = r, s = c + q) goes to [c + q][r]
              sm.lk[ps][0][c + 0][r] = a.x;
              sm.lk[ps][0][c + 1][r] = a.y;
              sm.lk[ps][0][c + 2][r] = a.z;
              sm.lk[ps][0][c + 3][r] = a.w;
            }
          }
        }
        // this wave's sums must be in LDS before its lanes read each other's
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        const bool isT = g == 0;
        const int row = li;
        float x[kC];
#pragma unroll
        for (int s = 0; s < kC; ++s) x[s] = isT ? (s == row ? 1.f : 0.f) : sm.gp[ps][0][kLrb][row][s];
#pragma unroll
        for (int s2 = kC - 1; s2 >= 1; --s2) {
          float lrow[kC];
#pragma unroll
          for (int q = 0; q < (s2 + 3) / 4; ++q)
            *reinterpret_cast<float4*>(&lrow[4 * q]) = *reinterpret_cast<const float4*>(&lab[s2][4 * q]);
#pragma unroll
          for (int s = 0; s < s2; ++s) x[s] = fmaf(x[s2], lrow[s], x[s]);
        }
        if (g < 2) {
          _Float16* dst = &sm.tm[cB & 1][g][row][0];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<half4*>(dst + 4 * q) = to_h4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
        }
      }
      // ================= B- and K- A-fragments (M = key, K = token), V B-fragments, gamma_15 of chunk cG
      if (doG) {
        const int xs = cG % kRing, os = cG & 3;
        const float(*fS)[kNP] = sm.fac[cG & 1][kFacS];
        // every LDS read of the stage first, then the arithmetic and the fragment writes
        IT braw[4][4], kraw[4][4], vraw[4][4];
        float suf[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int j = 16 * kt + li;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 4 * g + e;
            suf[kt][e] = fS[t][j];
            braw[kt][e] = sm.X[xs][kB][t][j];
            kraw[kt][e] = sm.X[xs][kK][t][j];
            vraw[kt][e] = sm.X[xs][kV][t][j];  // value index i = j
          }
        }
        const float g15 = sm.fac[cG & 1][kFacE][kC][lane];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          float bv[4], kv[4], vv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bv[e] = IO::widen(braw[kt][e]) * suf[kt][e];
            kv[e] = IO::widen(kraw[kt][e]) * suf[kt][e];
            vv[e] = IO::widen(vraw[kt][e]);
          }
          sm.ob[os][0][kt][lane] = to_h4(bv[0], bv[1], bv[2], bv[3]);
          sm.ob[os][1][kt][lane] = to_h4(kv[0], kv[1], kv[2], kv[3]);
          sm.ob[os][2][kt][lane] = to_h4(vv[0], vv[1], vv[2], vv[3]);
        }
        sm.gam[os][lane] = g15;
      }
    } else {
      // ================= G: Gram partial sums of chunk cG over keys 32h..32h+31 (h = wave - 6)
      if (doG) {
        const int h = wave - 6;
        const int xs = cG % kRing;
        const float(*fG)[kNP] = sm.fac[cG & 1][kFacG];
        const float(*fF)[kNP] = sm.fac[cG & 1][kFacF];
        const int j0 = 32 * h + 8 * g;
        float av[8], rv[8], bv[8], kv[8];
        IO::get8(&sm.X[xs][kA][li][j0], av);
        IO::get8(&sm.X[xs][kR][li][j0], rv);
        IO::get8(&sm.X[xs][kB][li][j0], bv);
        IO::get8(&sm.X[xs][kK][li][j0], kv);
        float gprev[8], gcur[8], fs[8];
        *reinterpret_cast<float4*>(&gprev[0]) = *reinterpret_cast<const float4*>(&fG[li][j0]);
        *reinterpret_cast<float4*>(&gprev[4]) = *reinterpret_cast<const float4*>(&fG[li][j0 + 4]);
        *reinterpret_cast<float4*>(&gcur[0]) = *reinterpret_cast<const float4*>(&fG[li + 1][j0]);
        *reinterpret_cast<float4*>(&gcur[4]) = *reinterpret_cast<const float4*>(&fG[li + 1][j0 + 4]);
        *reinterpret_cast<float4*>(&fs[0]) = *reinterpret_cast<const float4*>(&fF[li][j0]);
        *reinterpret_cast<float4*>(&fs[4]) = *reinterpret_cast<const float4*>(&fF[li][j0 + 4]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          av[e] *= gprev[e];  // query a_t e^{gamma_{t-1} - gamma_7}
          rv[e] *= gcur[e];   // query r_t e^{gamma_t - gamma_7}
          bv[e] *= fs[e];     // key   b_s e^{gamma_7 - gamma_s}
          kv[e] *= fs[e];     // key   k_s e^{gamma_7 - gamma_s}
        }
        bf16x8 ah, al, rh, rl, bh, bl, kh, kl;
        split8(av, ah, al);
        split8(rv, rh, rl);
        split8(bv, bh, bl);
        split8(kv, kh, kl);
        f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
        acc[kLab] = mfma_bf16(ah, bh, acc[kLab]);
        acc[kLak] = mfma_bf16(ah, kh, acc[kLak]);
        acc[kLrb] = mfma_bf16(rh, bh, acc[kLrb]);
        acc[kLrk] = mfma_bf16(rh, kh, acc[kLrk]);
        acc[kLab] = mfma_bf16(ah, bl, acc[kLab]);
        acc[kLak] = mfma_bf16(ah, kl, acc[kLak]);
        acc[kLrb] = mfma_bf16(rh, bl, acc[kLrb]);
        acc[kLrk] = mfma_bf16(rh, kl, acc[kLrk]);
        acc[kLab] = mfma_bf16(al, bh, acc[kLab]);
        acc[kLak] = mfma_bf16(al, kh, acc[kLak]);
        acc[kLrb] = mfma_bf16(rl, bh, acc[kLrb]);
        acc[kLrk] = mfma_bf16(rl, kh, acc[kLrk]);
        // acc[m][e] = L_m[t = 4g + e][s = li]; strictly (ab, ak) or weakly (rb, rk) lower
        float(*dst)[kC][kC] = sm.gp[cG & 1][h];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 4 * g + e;
            const bool keep = (m == kLab || m == kLak) ? (li < t) : (li <= t);
            dst[m][t][li] = keep ? acc[m][e] : 0.f;
          }
        }
      }
    }
    lds_barrier();
  }

  if (state_wave) store_y();
  if (state_wave && p.s_out) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      *reinterpret_cast<float4*>(p.s_out + ((int64_t)unit * kN + 16 * wave + li) * kN + 16 * kt + 4 * g) =
          make_float4(St[kt][0], St[kt][1], St[kt][2], St[kt][3]);
  }
}

template <bool BF16>
hipError_t launch_chunk_dtype(const WkvCall& c) {
  static_assert(sizeof(Pipe<BF16>) <= 160 * 1024, "LDS budget");
  // In-head offsets are 32-bit: T * H * 64 elements must stay below 2^31.
  if (c.T * c.H * kN >= (int64_t(1) << 31)) return hipErrorNotSupported;
  const void* fn = reinterpret_cast<const void*>(&wkv7_chunk_kernel<BF16>);
  const int bytes = (int)sizeof(Pipe<BF16>);
  // Opt in to more than 64 KiB of LDS once per process (the attribute is per function).
  static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (attr != hipSuccess) return attr;
  ChunkParams p{{c.in[0], c.in[1], c.in[2], c.in[3], c.in[4], c.in[5]}, static_cast<const float*>(c.s_in), c.y,
                static_cast<float*>(c.s_out), (int32_t)c.T, (int32_t)c.H};
  void* args[] = {&p};
  return hipLaunchKernel(fn, dim3((uint32_t)(c.B * c.H)), dim3(kThreads), args, bytes, c.stream);
}

}  // namespace

hipError_t launch_chunked(const WkvCall& c) {
  // bfloat16 inputs only: float32 inputs keep float32 accuracy on the sequential
  // kernel, and their six staged input slots would not fit the LDS ring.
  return c.dtype == 1 ? launch_chunk_dtype<true>(c) : hipErrorNotSupported;
}

}  // namespace rwkv7
