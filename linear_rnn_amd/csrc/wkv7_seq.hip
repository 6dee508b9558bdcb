// Sequential WKV-7 kernel: the recurrence token by token with the 64x64 float32
// state held in VGPRs. Serves the whole-sequence prefill for float32 inputs and
// the batched single-token step (RNN mode).
//
// Per token and head (RWKV-7 G0 7.2B notes, lshu.cn/news/198401, section 7.1):
//   sa_i = sum_j S_ij a_j,  S_ij <- S_ij w_j + sa_i b_j + v_i k_j,  y_i = sum_j S_ij r_j.
//
// Work decomposition. The value rows of S evolve independently (row i needs
// only its own state row, v_i and the shared key-space vectors r, w, k, a, b),
// so a head's 64 rows are split over WAVES*RPW-row workgroups. Inside a wave,
// lane = 16*ri + c holds columns 4c..4c+3 of the RPW/4 rows {4m + ri}; the two
// row dot products (S a and S r) are a 4-term in-lane partial followed by a
// 16-lane DPP butterfly, which leaves the identical sum in every lane of the row.
// State loads and stores are float4 per lane and cover 1 KiB contiguous per
// wave instruction.
//
// Inputs are staged through LDS in blocks of TB tokens: the whole workgroup
// issues coalesced 16-byte loads for block n+1 into registers while it computes
// block n from LDS, where the inputs sit widened to float32.
//
// Arithmetic order is fixed (explicit fmaf, built with -ffp-contract=off) and
// does not depend on RPW, WAVES or TB, so prefill and step give identical bits.
//
// Stored state. The state in HBM is float32, or for the single-token step
// optionally a 16-bit format (bfloat16 or float16): the state-size formula of
// the RWKV-8 ROSA note (trdm.cn/news/547794, "why states are worth quantising")
// scales with the bits per state element Q, and Q = 16 halves the bytes the
// HBM-bound step moves. The kernel widens the stored state exactly, runs the
// token in float32 as above, and rounds the new state to nearest-even only
// when storing it; y is read from the unrounded float32 state.
#include <type_traits>

#include "wkv7_device.hpp"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

struct SeqParams {
  const void* r;
  const void* w;
  const void* k;
  const void* v;
  const void* a;
  const void* b;
  const void* s_in;
  float* y;
  void* s_out;
  int64_t T;
  int32_t H;
};

template <bool BF16>
struct InTraits;
template <>
struct InTraits<true> {
  static constexpr int kEpv = 8;  // elements per 16-byte load
  // Widen 8 bfloat16 values to float32 and write them as two float4.
  __device__ static void store(float* dst, const uint4 q) {
    float4 lo = make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
    float4 hi = make_float4(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w));
    reinterpret_cast<float4*>(dst)[0] = lo;
    reinterpret_cast<float4*>(dst)[1] = hi;
  }
};
template <>
struct InTraits<false> {
  static constexpr int kEpv = 4;
  __device__ static void store(float* dst, const uint4 q) {
    *reinterpret_cast<uint4*>(dst) = q;
  }
};

// Stored-state element formats (RWKV7_STATE_* codes).
enum { kStF32 = 0, kStBF16 = 1, kStF16 = 2 };

// State traffic of a step, streamed once per call. With NT the loads and stores carry the
// non-temporal hint, so a state larger than the last-level cache does not displace
// everything else from it on every step (measured: 1 GiB float32 state 400 -> 368 us per
// step; a 128 MiB bfloat16 state 57 -> 49 us). A state that fits the cache is read back
// from it by the next step, and plain accesses keep that (256 MiB float32: 78 us plain
// against 91 us non-temporal).
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ld_state16(const void* p) {
  if constexpr (NT) {
    const u32x4v q = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
    return make_uint4(q[0], q[1], q[2], q[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ void st_state16(void* p, uint4 o) {
  if constexpr (NT)
    __builtin_nontemporal_store(u32x4v{o.x, o.y, o.z, o.w}, reinterpret_cast<u32x4v*>(p));
  else
    *reinterpret_cast<uint4*>(p) = o;
}

// Four consecutive state elements of one row: load widened, store rounded.
template <int SQ>
struct StateIO;
template <>
struct StateIO<kStF32> {
  template <bool NT = false>
  __device__ static float4 load4(const void* base, int64_t idx) {
    const uint4 q = ld_state16<NT>(static_cast<const float*>(base) + idx);
    return make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z), __uint_as_float(q.w));
  }
  template <bool NT = false>
  __device__ static void store4(void* base, int64_t idx, float4 s) {
    st_state16<NT>(static_cast<float*>(base) + idx,
                   make_uint4(__float_as_uint(s.x), __float_as_uint(s.y), __float_as_uint(s.z), __float_as_uint(s.w)));
  }
};
template <>
struct StateIO<kStBF16> {
  template <bool NT = false>
  __device__ static float4 load4(const void* base, int64_t idx) {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
  }
  __device__ static uint32_t pack(float lo, float hi) {  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
  }
  template <bool NT = false>
  __device__ static void store4(void* base, int64_t idx, float4 s) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = make_uint2(pack(s.x, s.y), pack(s.z, s.w));
  }
};
template <>
struct StateIO<kStF16> {
  template <bool NT = false>
  __device__ static float4 load4(const void* base, int64_t idx) {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return make_float4((float)__builtin_bit_cast(_Float16, (uint16_t)(q.x & 0xffffu)),
                       (float)__builtin_bit_cast(_Float16, (uint16_t)(q.x >> 16)),
                       (float)__builtin_bit_cast(_Float16, (uint16_t)(q.y & 0xffffu)),
                       (float)__builtin_bit_cast(_Float16, (uint16_t)(q.y >> 16)));
  }
  __device__ static uint32_t pack(float lo, float hi) {  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
  }
  template <bool NT = false>
  __device__ static void store4(void* base, int64_t idx, float4 s) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = make_uint2(pack(s.x, s.y), pack(s.z, s.w));
  }
};

template <bool BF16, int WAVES, int RPW, int TB, int SQ, bool NT = false>
__global__ __launch_bounds__(kWave* WAVES) void wkv7_seq_kernel(SeqParams p) {
  using Tr = InTraits<BF16>;
  using St = StateIO<SQ>;
  constexpr int kThreads = kWave * WAVES;
  constexpr int kRpb = WAVES * RPW;     // rows per workgroup
  constexpr int kNrb = kN / kRpb;       // workgroups per head
  constexpr int kMr = RPW / 4;          // rows per lane
  constexpr int kEpv = Tr::kEpv;
  constexpr int kKseg = kN / kEpv;      // 16-byte segments per key-space vector
  constexpr int kVseg = kRpb / kEpv;    // 16-byte segments of this workgroup's v rows
  constexpr int kEsz = BF16 ? 2 : 4;
  constexpr int kNqk = (TB * kKseg + kThreads - 1) / kThreads;
  constexpr int kNqv = (TB * kVseg + kThreads - 1) / kThreads;
  static_assert(kN % kRpb == 0 && RPW % 4 == 0 && kRpb % kEpv == 0, "bad tiling");

  // [token][r, w, k, a, b][column] and [token][row of this workgroup]
  __shared__ __align__(16) float kv_lds[TB][5][kN];
  __shared__ __align__(16) float v_lds[TB][kRpb];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c = lane & 15;
  const int ri = lane >> 4;

  const uint32_t logical = xcd_swizzle(blockIdx.x, gridDim.x);
  const int64_t unit = logical / kNrb;
  const int rb = logical % kNrb;
  const int64_t bb = unit / p.H;
  const int64_t hh = unit % p.H;
  const int64_t T = p.T;
  const int64_t tok_stride = (int64_t)p.H * kN;           // elements between tokens
  const int64_t seq_base = (bb * T * p.H + hh) * kN;      // element offset of token 0
  const int row_wg = rb * kRpb;                           // first row of this workgroup
  const int row0 = row_wg + wave * RPW;                   // first row of this wave

  const char* src[5] = {static_cast<const char*>(p.r), static_cast<const char*>(p.w),
                        static_cast<const char*>(p.k), static_cast<const char*>(p.a),
                        static_cast<const char*>(p.b)};
  const char* vsrc = static_cast<const char*>(p.v);

  // ---- state in
  float4 S[kMr];
#pragma unroll
  for (int m = 0; m < kMr; ++m) {
    const int row = row0 + 4 * m + ri;
    if (p.s_in)
      S[m] = St::template load4<NT>(p.s_in, (unit * kN + row) * kN + 4 * c);
    else
      S[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  uint4 stk[5][kNqk];
  uint4 stv[kNqv];
  // A prefill (TB > 1) loads and stores unconditionally: pieces past the end
  // repeat the last piece and tokens at or past T repeat token T-1, so no
  // divergent branch surrounds the loads (such branches make the compiler wait
  // for each new prefetch before it issues the next). The single-token step
  // (TB = 1, one block) loads only the pieces that exist.
  auto issue = [&](int64_t t0) {
#pragma unroll
    for (int x = 0; x < 5; ++x) {
#pragma unroll
      for (int q = 0; q < kNqk; ++q) {
        const int e0 = tid + kThreads * q;
        const int e = TB > 1 ? min(e0, TB * kKseg - 1) : e0;
        const int tok = e / kKseg, seg = e % kKseg;
        const int64_t t = TB > 1 ? min(t0 + tok, T - 1) : t0 + tok;
        if (TB > 1 || (e < TB * kKseg && t < T)) {
          const int64_t off = seq_base + t * tok_stride + seg * kEpv;
          stk[x][q] = *reinterpret_cast<const uint4*>(src[x] + off * kEsz);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kNqv; ++q) {
      const int e0 = tid + kThreads * q;
      const int e = TB > 1 ? min(e0, TB * kVseg - 1) : e0;
      const int tok = e / kVseg, seg = e % kVseg;
      const int64_t t = TB > 1 ? min(t0 + tok, T - 1) : t0 + tok;
      if (TB > 1 || (e < TB * kVseg && t < T)) {
        const int64_t off = seq_base + t * tok_stride + row_wg + seg * kEpv;
        stv[q] = *reinterpret_cast<const uint4*>(vsrc + off * kEsz);
      }
    }
  };
  auto commit = [&](int64_t t0) {
#pragma unroll
    for (int x = 0; x < 5; ++x) {
#pragma unroll
      for (int q = 0; q < kNqk; ++q) {
        const int e0 = tid + kThreads * q;
        const int e = TB > 1 ? min(e0, TB * kKseg - 1) : e0;
        const int tok = e / kKseg, seg = e % kKseg;
        if (TB > 1 || (e < TB * kKseg && t0 + tok < T)) Tr::store(&kv_lds[tok][x][seg * kEpv], stk[x][q]);
      }
    }
#pragma unroll
    for (int q = 0; q < kNqv; ++q) {
      const int e0 = tid + kThreads * q;
      const int e = TB > 1 ? min(e0, TB * kVseg - 1) : e0;
      const int tok = e / kVseg, seg = e % kVseg;
      if (TB > 1 || (e < TB * kVseg && t0 + tok < T)) Tr::store(&v_lds[tok][seg * kEpv], stv[q]);
    }
  };
  auto load_tok = [&](int tt, float4& r4, float4& w4, float4& k4, float4& a4, float4& b4, float (&vm)[kMr]) {
    r4 = *reinterpret_cast<const float4*>(&kv_lds[tt][0][4 * c]);
    w4 = *reinterpret_cast<const float4*>(&kv_lds[tt][1][4 * c]);
    k4 = *reinterpret_cast<const float4*>(&kv_lds[tt][2][4 * c]);
    a4 = *reinterpret_cast<const float4*>(&kv_lds[tt][3][4 * c]);
    b4 = *reinterpret_cast<const float4*>(&kv_lds[tt][4][4 * c]);
#pragma unroll
    for (int m = 0; m < kMr; ++m) vm[m] = v_lds[tt][wave * RPW + 4 * m + ri];
  };

  if (T > 0) issue(0);
  // A prefill's state and first block complete here, together, so the block loop
  // never waits for them (a loop-carried value that may still be in flight makes
  // the compiler wait for every outstanding load, prefetches included).
  if constexpr (TB > 1) __builtin_amdgcn_s_waitcnt(0x0f70);
  for (int64_t t0 = 0; t0 < T; t0 += TB) {
    __syncthreads();  // every wave is done reading the previous block
    commit(t0);
    __syncthreads();
    if (t0 + TB < T) issue(t0 + TB);  // in flight while this block is computed
    const int ntok = (T - t0 < TB) ? (int)(T - t0) : TB;
    if (TB > 1 && ntok == TB) {  // a whole block: the next token's LDS reads are in flight during this one
      float4 r4, w4, k4, a4, b4, r4n, w4n, k4n, a4n, b4n;
      float vm[kMr], vmn[kMr];
      load_tok(0, r4, w4, k4, a4, b4, vm);
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        if (tt + 1 < TB) load_tok(tt + 1, r4n, w4n, k4n, a4n, b4n, vmn);
        const float yo = token_update<kMr>(S, r4, w4, k4, a4, b4, vm, c);
        // lane c < RPW/4 writes row 4c + ri: the wave's RPW rows are contiguous.
        if (c < kMr) p.y[seq_base + (t0 + tt) * tok_stride + row0 + 4 * c + ri] = yo;
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
        if (c < kMr) p.y[seq_base + (t0 + tt) * tok_stride + row0 + 4 * c + ri] = yo;
      }
    }
  }

  // ---- state out
  if (p.s_out) {
#pragma unroll
    for (int m = 0; m < kMr; ++m) {
      const int row = row0 + 4 * m + ri;
      St::template store4<NT>(p.s_out, (unit * kN + row) * kN + 4 * c, S[m]);
    }
  }
}

// Single-token step with a 16-bit stored state (the float32 step uses the
// prefill kernel above), persistent and software-pipelined. A workgroup is four
// independent waves; wave q owns value rows 16q..16q+15 of one head, and lane
// 8*r8 + c8 holds columns 8c8..8c8+7 of rows 16q + r8 and 16q + r8 + 8, so every
// state and input access of a lane is one 16-byte load or store (with the
// prefill kernel's layout a 16-bit state row piece is only 8 bytes). Row sums
// are an 8-term in-lane chain and an 8-lane DPP butterfly (lane i with 7 - i,
// then i ^ 2, then i ^ 1), which leaves the same bits in every lane of the
// group; the operation order differs from the float32 kernels, so the float32
// intermediate state can differ from theirs by rounding before it is rounded to
// 16 bits. Workgroup g walks heads g, g + G, g + 2G, ...: while it computes one
// head, the raw bits of the next (state rows, the eight columns of r, w, k, a, b,
// v at its two rows) are already in flight into a second register set, and the
// two sets alternate, so no loop-carried copy forces an early wait. No LDS, no
// barriers.
__device__ __forceinline__ float row8_sum(float x) {
  x = x + dpp_f32<0x141>(x);  // row_half_mirror: lane i <-> 7 - i in each group of 8
  x = x + dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x = x + dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  return x;
}

template <int SQ>
__device__ __forceinline__ float widen16(uint32_t h) {
  if constexpr (SQ == kStBF16) return __uint_as_float(h << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <bool BF16, int SQ>
struct StepRaw {
  uint4 s[2];                                                       // 8 state elements of two rows
  typename std::conditional<BF16, uint4, float4>::type r[BF16 ? 1 : 2], w[BF16 ? 1 : 2], k[BF16 ? 1 : 2],
      a[BF16 ? 1 : 2], b[BF16 ? 1 : 2];
  typename std::conditional<BF16, uint16_t, float>::type v[2];
};

template <bool BF16, int SQ, bool NT>
__global__ __launch_bounds__(4 * kWave) void wkv7_step_kernel(SeqParams p, int64_t units) {
  using St = StateIO<SQ>;
  using Raw = StepRaw<BF16, SQ>;
  constexpr int kNv = BF16 ? 1 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int q = threadIdx.x >> 6;
  const int c8 = lane & 7;
  const int r8 = lane >> 3;
  const int row_a = 16 * q + r8;  // rows row_a and row_a + 8
  const int64_t G = gridDim.x;
  const int64_t g = xcd_swizzle(blockIdx.x, gridDim.x);
  using IV = typename std::conditional<BF16, uint4, float4>::type;
  using IS = typename std::conditional<BF16, uint16_t, float>::type;

  auto load = [&](Raw& x, int64_t u) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
      x.s[m] = p.s_in ? ld_state16<NT>(static_cast<const uint16_t*>(p.s_in) + (u * kN + row_a + 8 * m) * kN + 8 * c8)
                      : make_uint4(0u, 0u, 0u, 0u);
    const int64_t ib = u * kN + 8 * c8;
#pragma unroll
    for (int h = 0; h < kNv; ++h) {
      x.r[h] = reinterpret_cast<const IV*>(static_cast<const IS*>(p.r) + ib)[h];
      x.w[h] = reinterpret_cast<const IV*>(static_cast<const IS*>(p.w) + ib)[h];
      x.k[h] = reinterpret_cast<const IV*>(static_cast<const IS*>(p.k) + ib)[h];
      x.a[h] = reinterpret_cast<const IV*>(static_cast<const IS*>(p.a) + ib)[h];
      x.b[h] = reinterpret_cast<const IV*>(static_cast<const IS*>(p.b) + ib)[h];
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) x.v[m] = static_cast<const IS*>(p.v)[u * kN + row_a + 8 * m];
  };
  auto widen8 = [&](const IV* src, float (&o)[8]) {
    if constexpr (BF16) {
      const uint4 qv = src[0];
      o[0] = bf16_lo(qv.x), o[1] = bf16_hi(qv.x), o[2] = bf16_lo(qv.y), o[3] = bf16_hi(qv.y);
      o[4] = bf16_lo(qv.z), o[5] = bf16_hi(qv.z), o[6] = bf16_lo(qv.w), o[7] = bf16_hi(qv.w);
    } else {
      o[0] = src[0].x, o[1] = src[0].y, o[2] = src[0].z, o[3] = src[0].w;
      o[4] = src[1].x, o[5] = src[1].y, o[6] = src[1].z, o[7] = src[1].w;
    }
  };
  auto compute = [&](const Raw& x, int64_t u) {
    float S[2][8];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t wds[4] = {x.s[m].x, x.s[m].y, x.s[m].z, x.s[m].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[m][2 * e] = widen16<SQ>(wds[e] & 0xffffu);
        S[m][2 * e + 1] = widen16<SQ>(wds[e] >> 16);
      }
    }
    float r[8], w[8], k[8], a[8], b[8];
    widen8(x.r, r), widen8(x.w, w), widen8(x.k, k), widen8(x.a, a), widen8(x.b, b);
    float vm[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if constexpr (BF16) vm[m] = __uint_as_float((uint32_t)x.v[m] << 16);
      else vm[m] = x.v[m];
    }
    float sa[2], yp[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float t = S[m][0] * a[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) t = fmaf(S[m][j], a[j], t);
      sa[m] = t;
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) sa[m] = row8_sum(sa[m]);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) S[m][j] = fmaf(S[m][j], w[j], fmaf(sa[m], b[j], vm[m] * k[j]));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float t = S[m][0] * r[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) t = fmaf(S[m][j], r[j], t);
      yp[m] = t;
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) yp[m] = row8_sum(yp[m]);
    if (c8 < 2) p.y[u * kN + row_a + 8 * c8] = c8 == 0 ? yp[0] : yp[1];
    if (p.s_out) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint4 o;
        o.x = St::pack(S[m][0], S[m][1]);
        o.y = St::pack(S[m][2], S[m][3]);
        o.z = St::pack(S[m][4], S[m][5]);
        o.w = St::pack(S[m][6], S[m][7]);
        st_state16<NT>(static_cast<uint16_t*>(p.s_out) + (u * kN + row_a + 8 * m) * kN + 8 * c8, o);
      }
    }
  };

  Raw A, B;
  int64_t u = g;
  if (u < units) load(A, u);
  while (u < units) {
    if (u + G < units) load(B, u + G);
    compute(A, u);
    u += G;
    if (u >= units) break;
    if (u + G < units) load(A, u + G);
    compute(B, u);
    u += G;
  }
}

__global__ void state_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <bool BF16, int WAVES, int RPW, int TB, int SQ = kStF32, bool NT = false>
hipError_t launch_seq_cfg(const WkvCall& c) {
  SeqParams p{c.in[0], c.in[1], c.in[2], c.in[3], c.in[4], c.in[5], c.s_in, c.y, c.s_out, c.T, (int32_t)c.H};
  constexpr int kNrb = kN / (WAVES * RPW);
  const int64_t blocks = c.B * c.H * kNrb;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&wkv7_seq_kernel<BF16, WAVES, RPW, TB, SQ, NT>),
                         dim3((uint32_t)blocks), dim3(kWave * WAVES), args, 0, c.stream);
}

// Stored-state size from which a step streams its state with non-temporal accesses: the
// measured crossovers on MI355X (256 MB last-level cache) lie between 256 and 320 MiB for a
// float32 state and between 64 and 128 MiB for a 16-bit one.
constexpr int64_t kNtStateF32 = int64_t(288) << 20;
constexpr int64_t kNtState16 = int64_t(96) << 20;

// Measured on the D2048 step (B=512, H=32): 8192 workgroups (two heads each)
// beat both one workgroup per head and fully resident grids for 16-bit states.
constexpr int64_t kStepGrid = 8192;

template <bool BF16, int SQ>
hipError_t launch_step(const WkvCall& c) {
  SeqParams p{c.in[0], c.in[1], c.in[2], c.in[3], c.in[4], c.in[5], c.s_in, c.y, c.s_out, c.T, (int32_t)c.H};
  int64_t units = c.B * c.H;
  // Persistent grid: enough four-wave workgroups to keep every SIMD of the
  // 256 CUs busy with several waves, each walking heads with a stride of the grid.
  const int64_t grid = units < kStepGrid ? units : kStepGrid;
  void* args[] = {&p, &units};
  const bool nt = units * kN * kN * 2 > kNtState16;
  const void* fn = nt ? reinterpret_cast<const void*>(&wkv7_step_kernel<BF16, SQ, true>)
                      : reinterpret_cast<const void*>(&wkv7_step_kernel<BF16, SQ, false>);
  return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(4 * kWave), args, 0, c.stream);
}

template <bool BF16>
hipError_t launch_seq_dtype(const WkvCall& c, bool decode_shape) {
  if (decode_shape) {
    // 16-bit stored state: the persistent step kernel. Float32 state: the
    // workgroup-per-head tiling of the prefill kernel, the faster of the two
    // for 16 KiB state rows (78 us against 87 us per D2048 step).
    if (c.sdtype == kStBF16) return launch_step<BF16, kStBF16>(c);
    if (c.sdtype == kStF16) return launch_step<BF16, kStF16>(c);
    if (c.B * c.H * kN * kN * 4 > kNtStateF32) return launch_seq_cfg<BF16, 4, 16, 1, kStF32, true>(c);
    return launch_seq_cfg<BF16, 4, 16, 1>(c);
  }
  if (c.sdtype != kStF32) return hipErrorNotSupported;
  // Prefill: the token loop is serial, so spread each head's rows over more
  // waves when there are few heads.
  const int64_t units = c.B * c.H;
  if (units >= 2048) return launch_seq_cfg<BF16, 4, 16, 16>(c);
  return launch_seq_cfg<BF16, 4, 4, 32>(c);
}

}  // namespace

hipError_t launch_sequential(const WkvCall& c, bool decode_shape) {
  return c.dtype == 1 ? launch_seq_dtype<true>(c, decode_shape) : launch_seq_dtype<false>(c, decode_shape);
}

hipError_t launch_state_copy(const float* s_in, float* s_out, int64_t units, hipStream_t stream) {
  const int64_t n4 = units * kN * kN / 4;
  const int threads = 256;
  const int64_t blocks = (n4 + threads - 1) / threads;
  const float4* src = reinterpret_cast<const float4*>(s_in);
  float4* dst = reinterpret_cast<float4*>(s_out);
  void* args[] = {&src, &dst, const_cast<int64_t*>(&n4)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&state_copy_kernel), dim3((uint32_t)blocks),
                         dim3(threads), args, 0, stream);
}

}  // namespace rwkv7
