// Reverse-mode derivatives of the WKV-7 recurrence. Training the model runs the
// wkv7 operator inside the training scripts (RWKV-7 G0 7.2B notes,
// lshu.cn/news/198401, section 7.2), which needs its derivatives; the pages give
// only the forward formula (section 7.1), so the rules below are its reverse-mode
// differentiation. Forward, per head and token:
//   sa = S_{t-1} a,   S_t = S_{t-1} diag(w) + sa b^T + v k^T,   y = S_t r.
// With G = dL/dS_t (the gradient flowing back from later tokens, seeded by
// dL/dS_T), one token taken in reverse is
//   G  += dy r^T                          (y's contribution)
//   dr_j = sum_i S_t[i,j] dy_i            dk_j = sum_i G[i,j] v_i
//   dw_j = sum_i S_{t-1}[i,j] G[i,j]      dv_i = sum_j G[i,j] k_j
//   gb_i = sum_j G[i,j] b_j               da_j = sum_i S_{t-1}[i,j] gb_i
//   db_j = sum_i G[i,j] sa_i              G   <- G diag(w) + gb a^T
// and after token 0, G is dL/dS_0.
//
// Two kernels, each one workgroup per head, WAVES waves of 64/WAVES value rows,
// with the lane layout of the sequential forward (lane = 16*ri + c holds columns
// 4c..4c+3 of rows {4m + ri} of its wave):
//   1. wkv7_ckpt_kernel runs the recurrence forward and stores the state at the
//      start of every kSeg-token segment (a float32 checkpoint per segment in
//      the workspace), with the forward kernels' arithmetic, bit for bit.
//   2. wkv7_bwd_kernel walks the segments from the last to the first. For each
//      kSub-token sub-block (the last one first) it rebuilds, from the
//      segment's checkpoint, the kSub + 1 states the sub-block touches into
//      registers, then takes the sub-block's tokens in reverse.
// Row sums (dv, gb, and sa in the rebuild) are in-lane partials plus the 16-lane
// DPP butterfly. Column sums (dr, dk, dw, da, db) are in-lane over the lane's
// rows, then reduce-scattered over the wave's four lane rows with two
// permlane swaps (lane l with l^32, then l with l^16), which leaves the wave's
// sum for column 4c + ri in lane (c, ri); the waves' partials meet in LDS and
// are summed in a fixed order when the sub-block ends, so results do not depend
// on scheduling. Inputs of a segment are staged through LDS, widened to float32,
// while the next (earlier) segment's inputs and checkpoint are in flight in
// registers. Gradients are float32.
#include "wkv7_device.hpp"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

constexpr int kSub = 8;              // tokens whose states sit in registers at once
constexpr int kSubs = 2;             // sub-blocks per checkpoint segment
constexpr int kSeg = kSub * kSubs;   // tokens between stored checkpoints
constexpr int kSlots = 7;            // staged per token: r, w, k, v, a, b (dtype), dy (float32)
constexpr int kDy = 6;
enum { kR = 0, kW = 1, kK = 2, kV = 3, kA = 4, kB = 5 };
// column-gradient slots, in the order of the partial buffers
enum { kGr = 0, kGk = 1, kGw = 2, kGa = 3, kGb = 4, kNcol = 5 };

struct BwdParams {
  const void* in[6];  // r, w, k, v, a, b: [B, T, H, 64] in dtype
  const float* s_in;  // [B, H, 64, 64] or null (zero)
  const float* dy;    // [B, T, H, 64]
  const float* ds_out;  // [B, H, 64, 64] or null (zero)
  float* grad[6];       // dr, dw, dk, dv, da, db: [B, T, H, 64]
  float* ds_in;         // [B, H, 64, 64] or null
  float* ck;            // checkpoints [B*H][nseg][64][64]
  int64_t T;
  int32_t H;
  int32_t nseg;
};

// Stages tokens [t0, t0 + kSeg) of the tensors selected by MASK (bits over
// r, w, k, v, a, b, dy) into lds[token][slot][64] as float32: issue() starts the
// 16-byte global loads into registers, commit() widens and stores them.
// Tokens at or past T are neither loaded nor stored.
template <bool BF16, int THREADS, unsigned MASK>
struct SegLoader {
  static constexpr int kEpv = BF16 ? 8 : 4;  // dtype elements per 16-byte load
  static constexpr int kEsz = BF16 ? 2 : 4;
  static constexpr int kPin = kN / kEpv;     // 16-byte pieces per token row of an input
  static constexpr int kNin = __builtin_popcount(MASK & 0x3f);
  static constexpr int kPer = kSeg * kPin;   // pieces per input tensor and segment
  static constexpr int kQin = (kNin * kPer + THREADS - 1) / THREADS;
  static constexpr bool kWithDy = (MASK >> kDy) & 1;
  static constexpr int kQdy = kWithDy ? (kSeg * 16 + THREADS - 1) / THREADS : 0;

  uint4 qin[kQin];
  uint4 qdy[kQdy > 0 ? kQdy : 1];

  // slot of the n-th selected input
  __device__ static int slot_of(int n) {
    int s = 0;
#pragma unroll
    for (int x = 0; x < 6; ++x)
      if ((MASK >> x) & 1) {
        if (n == 0) s = x;
        --n;
      }
    return s;
  }

  __device__ void issue(const BwdParams& p, int64_t seq_base, int64_t tok_stride, int64_t t0, int tid) {
#pragma unroll
    for (int q = 0; q < kQin; ++q) {
      const int e = tid + THREADS * q;
      const int n = e / kPer, rem = e % kPer;
      const int tok = rem / kPin, piece = rem % kPin;
      if (e < kNin * kPer && t0 + tok < p.T) {
        const int slot = slot_of(n);
        const char* src = nullptr;
#pragma unroll
        for (int x = 0; x < 6; ++x)
          if (slot == x) src = static_cast<const char*>(p.in[x]);  // constant indices keep p in SGPRs
        qin[q] = *reinterpret_cast<const uint4*>(src + (seq_base + (t0 + tok) * tok_stride + piece * kEpv) * kEsz);
      }
    }
#pragma unroll
    for (int q = 0; q < kQdy; ++q) {
      const int e = tid + THREADS * q;
      const int tok = e / 16, piece = e % 16;
      if (e < kSeg * 16 && t0 + tok < p.T)
        qdy[q] = *reinterpret_cast<const uint4*>(p.dy + seq_base + (t0 + tok) * tok_stride + piece * 4);
    }
  }

  __device__ void commit(float (*lds)[kSlots][kN], int64_t T, int64_t t0, int tid) const {
#pragma unroll
    for (int q = 0; q < kQin; ++q) {
      const int e = tid + THREADS * q;
      const int n = e / kPer, rem = e % kPer;
      const int tok = rem / kPin, piece = rem % kPin;
      if (e < kNin * kPer && t0 + tok < T) {
        float* dst = &lds[tok][slot_of(n)][piece * kEpv];
        const uint4 v = qin[q];
        if constexpr (BF16) {
          reinterpret_cast<float4*>(dst)[0] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
          reinterpret_cast<float4*>(dst)[1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
        } else {
          *reinterpret_cast<uint4*>(dst) = v;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kQdy; ++q) {
      const int e = tid + THREADS * q;
      const int tok = e / 16, piece = e % 16;
      if (e < kSeg * 16 && t0 + tok < T) *reinterpret_cast<uint4*>(&lds[tok][kDy][piece * 4]) = qdy[q];
    }
  }
};

__device__ __forceinline__ float dot4(const float4 s, const float4 x) {
  return fmaf(s.w, x.w, fmaf(s.z, x.z, fmaf(s.y, x.y, s.x * x.x)));
}

// One forward token for the lane's MR rows (the forward kernels' operation
// order): returns nothing, leaves sa (the row sums S_{t-1} a) in sa[].
template <int MR>
__device__ __forceinline__ void fwd_token(float4 (&S)[MR], float (&sa)[MR], const float4 w4, const float4 k4,
                                          const float4 a4, const float4 b4, const float (&vm)[MR]) {
#pragma unroll
  for (int m = 0; m < MR; ++m) sa[m] = dot4(S[m], a4);
#pragma unroll
  for (int m = 0; m < MR; ++m) sa[m] = row16_sum(sa[m]);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    S[m].x = fmaf(S[m].x, w4.x, fmaf(sa[m], b4.x, vm[m] * k4.x));
    S[m].y = fmaf(S[m].y, w4.y, fmaf(sa[m], b4.y, vm[m] * k4.y));
    S[m].z = fmaf(S[m].z, w4.z, fmaf(sa[m], b4.z, vm[m] * k4.z));
    S[m].w = fmaf(S[m].w, w4.w, fmaf(sa[m], b4.w, vm[m] * k4.w));
  }
}

// x + (the value lane l^32 holds), keeping column p in lanes 0..31 and column
// p + 2 in lanes 32..63: one swap of (lo, hi) = (X[p], X[p+2]) between the wave
// halves, then a sum of the two registers.
__device__ __forceinline__ float swap32_sum(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same between lane rows 0<->1 and 2<->3 (lanes l and l^16): even rows keep
// `even`, odd rows keep `odd`.
__device__ __forceinline__ float swap16_sum(float even, float odd) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(even), __float_as_uint(odd), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Column sums of the wave: X[x][cc] holds the lane's partial for column 4c + cc;
// returns, for each x, the sum over the wave's 64 rows of column 4c + ri.
__device__ __forceinline__ void column_reduce(const float (&X)[kNcol][4], float (&out)[kNcol]) {
#pragma unroll
  for (int x = 0; x < kNcol; ++x) {
    const float y0 = swap32_sum(X[x][0], X[x][2]);  // columns 0 | 2
    const float y1 = swap32_sum(X[x][1], X[x][3]);  // columns 1 | 3
    out[x] = swap16_sum(y0, y1);                    // columns 0, 1 | 2, 3
  }
}

// ---------------------------------------------------------------- checkpoint forward

template <bool BF16, int WAVES>
__global__ __launch_bounds__(kWave* WAVES) void wkv7_ckpt_kernel(BwdParams p) {
  constexpr int kThreads = kWave * WAVES;
  constexpr int kRpw = kN / WAVES;
  constexpr int kMr = kRpw / 4;
  using Ld = SegLoader<BF16, kThreads, (1u << kW) | (1u << kK) | (1u << kV) | (1u << kA) | (1u << kB)>;
  __shared__ __align__(16) float lds[kSeg][kSlots][kN];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c = lane & 15;
  const int ri = lane >> 4;
  const int64_t unit = xcd_swizzle(blockIdx.x, gridDim.x);
  const int64_t bb = unit / p.H, hh = unit % p.H;
  const int64_t T = p.T;
  const int64_t tok_stride = (int64_t)p.H * kN;
  const int64_t seq_base = (bb * T * p.H + hh) * kN;
  const int row0 = wave * kRpw;

  float4 S[kMr];
#pragma unroll
  for (int m = 0; m < kMr; ++m) {
    const int row = row0 + 4 * m + ri;
    S[m] = p.s_in ? *reinterpret_cast<const float4*>(p.s_in + (unit * kN + row) * kN + 4 * c)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  Ld ld;
  ld.issue(p, seq_base, tok_stride, 0, tid);
  for (int seg = 0; seg < p.nseg; ++seg) {
    const int64_t t0 = (int64_t)seg * kSeg;
    const int n = (T - t0 < kSeg) ? (int)(T - t0) : kSeg;
    float* ck = p.ck + (unit * p.nseg + seg) * (int64_t)(kN * kN);
#pragma unroll
    for (int m = 0; m < kMr; ++m)
      *reinterpret_cast<float4*>(ck + (row0 + 4 * m + ri) * kN + 4 * c) = S[m];
    __syncthreads();  // every wave is done with the previous segment's LDS
    ld.commit(lds, T, t0, tid);
    __syncthreads();
    if (seg + 1 < p.nseg) ld.issue(p, seq_base, tok_stride, t0 + kSeg, tid);
    for (int j = 0; j < n; ++j) {
      const float4 w4 = *reinterpret_cast<const float4*>(&lds[j][kW][4 * c]);
      const float4 k4 = *reinterpret_cast<const float4*>(&lds[j][kK][4 * c]);
      const float4 a4 = *reinterpret_cast<const float4*>(&lds[j][kA][4 * c]);
      const float4 b4 = *reinterpret_cast<const float4*>(&lds[j][kB][4 * c]);
      float vm[kMr], sa[kMr];
#pragma unroll
      for (int m = 0; m < kMr; ++m) vm[m] = lds[j][kV][row0 + 4 * m + ri];
      fwd_token<kMr>(S, sa, w4, k4, a4, b4, vm);
    }
  }
}

// ---------------------------------------------------------------- reverse pass

template <bool BF16, int WAVES>
__global__ __launch_bounds__(kWave* WAVES) void wkv7_bwd_kernel(BwdParams p) {
  constexpr int kThreads = kWave * WAVES;
  constexpr int kRpw = kN / WAVES;
  constexpr int kMr = kRpw / 4;
  using Ld = SegLoader<BF16, kThreads, 0x7fu>;
  __shared__ __align__(16) float lds[kSeg][kSlots][kN];
  __shared__ __align__(16) float part[kSub][kNcol][WAVES][kN];  // per-wave column sums
  __shared__ __align__(16) float dv_lds[kSub][kN];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c = lane & 15;
  const int ri = lane >> 4;
  const int64_t unit = xcd_swizzle(blockIdx.x, gridDim.x);
  const int64_t bb = unit / p.H, hh = unit % p.H;
  const int64_t T = p.T;
  const int64_t tok_stride = (int64_t)p.H * kN;
  const int64_t seq_base = (bb * T * p.H + hh) * kN;
  const int row0 = wave * kRpw;

  float4 G[kMr];
#pragma unroll
  for (int m = 0; m < kMr; ++m) {
    const int row = row0 + 4 * m + ri;
    G[m] = p.ds_out ? *reinterpret_cast<const float4*>(p.ds_out + (unit * kN + row) * kN + 4 * c)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  const float* ck_base = p.ck + unit * p.nseg * (int64_t)(kN * kN);
  Ld ld;
  float4 ckq[kMr];
  auto issue = [&](int seg) {
    ld.issue(p, seq_base, tok_stride, (int64_t)seg * kSeg, tid);
    const float* ck = ck_base + (int64_t)seg * (kN * kN);
#pragma unroll
    for (int m = 0; m < kMr; ++m) ckq[m] = *reinterpret_cast<const float4*>(ck + (row0 + 4 * m + ri) * kN + 4 * c);
  };

  issue(p.nseg - 1);
  for (int seg = p.nseg - 1; seg >= 0; --seg) {
    const int64_t t0 = (int64_t)seg * kSeg;
    const int n = (T - t0 < kSeg) ? (int)(T - t0) : kSeg;
    __syncthreads();  // every wave is done with the previous segment's inputs
    ld.commit(lds, T, t0, tid);
    float4 Sck[kMr];
#pragma unroll
    for (int m = 0; m < kMr; ++m) Sck[m] = ckq[m];
    __syncthreads();
    if (seg > 0) issue(seg - 1);

    for (int sb = (n - 1) / kSub; sb >= 0; --sb) {
      const int j0 = sb * kSub;                             // first token of the sub-block in the segment
      const int cnt = (n - j0 < kSub) ? n - j0 : kSub;      // its tokens
      // the state before token j0 of the segment
      float4 Sv[kSub + 1][kMr];
#pragma unroll
      for (int m = 0; m < kMr; ++m) Sv[0][m] = Sck[m];
      for (int j = 0; j < j0; ++j) {
        const float4 w4 = *reinterpret_cast<const float4*>(&lds[j][kW][4 * c]);
        const float4 k4 = *reinterpret_cast<const float4*>(&lds[j][kK][4 * c]);
        const float4 a4 = *reinterpret_cast<const float4*>(&lds[j][kA][4 * c]);
        const float4 b4 = *reinterpret_cast<const float4*>(&lds[j][kB][4 * c]);
        float vm[kMr], sa[kMr];
#pragma unroll
        for (int m = 0; m < kMr; ++m) vm[m] = lds[j][kV][row0 + 4 * m + ri];
        fwd_token<kMr>(Sv[0], sa, w4, k4, a4, b4, vm);
      }
      // rebuild the sub-block's states: Sv[u] is the state before token j0 + u
      float sav[kSub][kMr];
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        if (u < cnt) {
          const int j = j0 + u;
          const float4 w4 = *reinterpret_cast<const float4*>(&lds[j][kW][4 * c]);
          const float4 k4 = *reinterpret_cast<const float4*>(&lds[j][kK][4 * c]);
          const float4 a4 = *reinterpret_cast<const float4*>(&lds[j][kA][4 * c]);
          const float4 b4 = *reinterpret_cast<const float4*>(&lds[j][kB][4 * c]);
          float vm[kMr];
#pragma unroll
          for (int m = 0; m < kMr; ++m) vm[m] = lds[j][kV][row0 + 4 * m + ri];
#pragma unroll
          for (int m = 0; m < kMr; ++m) Sv[u + 1][m] = Sv[u][m];
          fwd_token<kMr>(Sv[u + 1], sav[u], w4, k4, a4, b4, vm);
        }
      }
      // the sub-block's tokens in reverse
#pragma unroll
      for (int u = kSub - 1; u >= 0; --u) {
        if (u < cnt) {
          const int j = j0 + u;
          const float4 r4 = *reinterpret_cast<const float4*>(&lds[j][kR][4 * c]);
          const float4 w4 = *reinterpret_cast<const float4*>(&lds[j][kW][4 * c]);
          const float4 k4 = *reinterpret_cast<const float4*>(&lds[j][kK][4 * c]);
          const float4 a4 = *reinterpret_cast<const float4*>(&lds[j][kA][4 * c]);
          const float4 b4 = *reinterpret_cast<const float4*>(&lds[j][kB][4 * c]);
          float vm[kMr], dym[kMr];
#pragma unroll
          for (int m = 0; m < kMr; ++m) {
            vm[m] = lds[j][kV][row0 + 4 * m + ri];
            dym[m] = lds[j][kDy][row0 + 4 * m + ri];
          }
          const float4(&Sp)[kMr] = Sv[u];
          const float4(&Sc)[kMr] = Sv[u + 1];
          // G += dy r^T
#pragma unroll
          for (int m = 0; m < kMr; ++m) {
            G[m].x = fmaf(dym[m], r4.x, G[m].x);
            G[m].y = fmaf(dym[m], r4.y, G[m].y);
            G[m].z = fmaf(dym[m], r4.z, G[m].z);
            G[m].w = fmaf(dym[m], r4.w, G[m].w);
          }
          // row sums: dv = G k, gb = G b
          float dvr[kMr], gb[kMr];
#pragma unroll
          for (int m = 0; m < kMr; ++m) {
            dvr[m] = dot4(G[m], k4);
            gb[m] = dot4(G[m], b4);
          }
#pragma unroll
          for (int m = 0; m < kMr; ++m) {
            dvr[m] = row16_sum(dvr[m]);
            gb[m] = row16_sum(gb[m]);
          }
          // column partials over the lane's rows
          float X[kNcol][4];
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
            for (int x = 0; x < kNcol; ++x) X[x][cc] = 0.f;
          }
#pragma unroll
          for (int m = 0; m < kMr; ++m) {
            const float sc[4] = {Sc[m].x, Sc[m].y, Sc[m].z, Sc[m].w};
            const float sp[4] = {Sp[m].x, Sp[m].y, Sp[m].z, Sp[m].w};
            const float gg[4] = {G[m].x, G[m].y, G[m].z, G[m].w};
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
              X[kGr][cc] = fmaf(sc[cc], dym[m], X[kGr][cc]);
              X[kGk][cc] = fmaf(gg[cc], vm[m], X[kGk][cc]);
              X[kGw][cc] = fmaf(sp[cc], gg[cc], X[kGw][cc]);
              X[kGa][cc] = fmaf(sp[cc], gb[m], X[kGa][cc]);
              X[kGb][cc] = fmaf(gg[cc], sav[u][m], X[kGb][cc]);
            }
          }
          float colsum[kNcol];
          column_reduce(X, colsum);
#pragma unroll
          for (int x = 0; x < kNcol; ++x) part[u][x][wave][4 * c + ri] = colsum[x];
          float dvo = dvr[0];
#pragma unroll
          for (int m = 1; m < kMr; ++m) dvo = (c == m) ? dvr[m] : dvo;
          if (c < kMr) dv_lds[u][row0 + 4 * c + ri] = dvo;
          // G <- G diag(w) + gb a^T
#pragma unroll
          for (int m = 0; m < kMr; ++m) {
            G[m].x = fmaf(G[m].x, w4.x, gb[m] * a4.x);
            G[m].y = fmaf(G[m].y, w4.y, gb[m] * a4.y);
            G[m].z = fmaf(G[m].z, w4.z, gb[m] * a4.z);
            G[m].w = fmaf(G[m].w, w4.w, gb[m] * a4.w);
          }
        }
      }
      __syncthreads();
      // sum the waves' partials in wave order and write the sub-block's gradients
      const int64_t tbase = seq_base + (t0 + j0) * tok_stride;
      for (int e = tid; e < cnt * kNcol * kN; e += kThreads) {
        const int u = e / (kNcol * kN), x = (e / kN) % kNcol, col = e % kN;
        float s = part[u][x][0][col];
#pragma unroll
        for (int wv = 1; wv < WAVES; ++wv) s += part[u][x][wv][col];
        // partial slots -> gradient tensors dr, dk, dw, da, db
        float* dst = x == kGr ? p.grad[0] : x == kGk ? p.grad[2] : x == kGw ? p.grad[1] : x == kGa ? p.grad[4] : p.grad[5];
        dst[tbase + u * tok_stride + col] = s;
      }
      for (int e = tid; e < cnt * kN; e += kThreads) {
        const int u = e / kN, col = e % kN;
        p.grad[3][tbase + u * tok_stride + col] = dv_lds[u][col];
      }
      __syncthreads();  // the partial buffers are free again
    }
  }

  if (p.ds_in) {
#pragma unroll
    for (int m = 0; m < kMr; ++m) {
      const int row = row0 + 4 * m + ri;
      *reinterpret_cast<float4*>(p.ds_in + (unit * kN + row) * kN + 4 * c) = G[m];
    }
  }
}

template <bool BF16, int WAVES>
hipError_t launch_cfg(BwdParams p, int64_t units, hipStream_t stream) {
  void* args[] = {&p};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&wkv7_ckpt_kernel<BF16, WAVES>),
                                 dim3((uint32_t)units), dim3(kWave * WAVES), args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&wkv7_bwd_kernel<BF16, WAVES>), dim3((uint32_t)units),
                         dim3(kWave * WAVES), args, 0, stream);
}

}  // namespace

hipError_t launch_backward(const BwdCall& c) {
  const int64_t units = c.B * c.H;
  const int64_t nseg = (c.T + kSeg - 1) / kSeg;
  if (nseg > INT32_MAX) return hipErrorNotSupported;
  void* ws = nullptr;
  hipError_t e = device_workspace(c.stream, (size_t)(units * nseg) * kN * kN * sizeof(float), &ws);
  if (e != hipSuccess) return e;
  BwdParams p{};
  for (int i = 0; i < 6; ++i) p.in[i] = c.in[i];
  p.s_in = c.s_in;
  p.dy = c.dy;
  p.ds_out = c.ds_out;
  for (int i = 0; i < 6; ++i) p.grad[i] = c.grad[i];
  p.ds_in = c.ds_in;
  p.ck = static_cast<float*>(ws);
  p.T = c.T;
  p.H = (int32_t)c.H;
  p.nseg = (int32_t)nseg;
  return c.dtype == 1 ? launch_cfg<true, 8>(p, units, c.stream) : launch_cfg<false, 8>(p, units, c.stream);
}

}  // namespace rwkv7
