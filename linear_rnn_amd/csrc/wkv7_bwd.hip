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
// The value rows of S (and of G) evolve independently: row i of the update needs
// only its own row, v_i, dy_i and the key-space vectors. So a head's 64 rows are
// split over NRB workgroups of WAVES waves, with the lane layout of the
// sequential forward (lane = 16*ri + c holds columns 4c..4c+3 of rows {4m + ri}
// of its wave). Only the column gradients couple rows; with two row blocks per
// head, block 0 writes its column sums to the gradients and block 1 to a
// workspace copy that a third kernel adds in (a sum of two terms, whatever the
// order, so results stay deterministic). Splitting pays when heads are few.
//   1. wkv7_ckpt_kernel runs the recurrence forward and stores the state at the
//      start of every kSeg-token segment (a float32 checkpoint per segment in
//      the workspace), with the forward kernels' arithmetic, bit for bit.
//   2. wkv7_bwd_kernel walks the segments from the last to the first. For each
//      kSub-token sub-block (the last one first) it rebuilds, from the
//      segment's checkpoint, the kSub + 1 states the sub-block touches into
//      registers, then takes the sub-block's tokens in reverse.
//   3. wkv7_colsum_kernel (two row blocks only) adds block 1's column sums.
// Row sums (dv, gb, and sa in the rebuild) are in-lane partials plus the 16-lane
// DPP butterfly. Column sums (dr, dk, dw, da, db) are in-lane over the lane's
// rows, then reduce-scattered over the wave's four lane rows with two
// permlane swaps (lane l with l^32, then l with l^16), which leaves the wave's
// sum for column 4c + ri in lane (c, ri); the waves' partials meet in LDS and
// are summed in a fixed order when the sub-block ends, so results do not depend
// on scheduling. Inputs of a segment are staged through LDS, widened to float32,
// while the next (earlier) segment's inputs and checkpoint are in flight in
// registers. Gradients are float32.
#include <type_traits>

#include "wkv7_device.hpp"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

constexpr int kSub = 8;              // tokens whose states sit in registers at once
constexpr int kSubs = 1;             // sub-blocks per checkpoint segment
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
  float* col1;          // column sums of row block 1: [5][B, T, H, 64] (dr, dw, dk, da, db), or null
  int64_t elems;        // B * T * H * 64
  int64_t T;
  int32_t H;
  int32_t nseg;
};

// Stages tokens [t0, t0 + TOK) of the tensors selected by MASK (bits over
// r, w, k, v, a, b, dy) into lds[token][slot][64] as float32: issue() starts the
// 16-byte global loads into registers, commit() widens and stores them.
template <bool BF16, int THREADS, unsigned MASK, int TOK = kSeg>
struct SegLoader {
  static constexpr int kEpv = BF16 ? 8 : 4;  // dtype elements per 16-byte load
  static constexpr int kEsz = BF16 ? 2 : 4;
  static constexpr int kPin = kN / kEpv;     // 16-byte pieces per token row of an input
  static constexpr int kNin = __builtin_popcount(MASK & 0x3f);
  static constexpr int kPer = TOK * kPin;    // pieces per input tensor and batch
  static constexpr int kQin = (kNin * kPer + THREADS - 1) / THREADS;
  static constexpr bool kWithDy = (MASK >> kDy) & 1;
  static constexpr int kQdy = kWithDy ? (TOK * 16 + THREADS - 1) / THREADS : 0;

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

  // Every lane loads and stores unconditionally: pieces past the end repeat the
  // last piece and tokens at or past T repeat token T-1 (T >= 1), so the code
  // has no divergent branches around the loads, which would make the compiler
  // serialise them with waits.
  __device__ void issue(const BwdParams& p, int64_t seq_base, int64_t tok_stride, int64_t t0, int tid) {
#pragma unroll
    for (int q = 0; q < kQin; ++q) {
      const int e = min(tid + THREADS * q, kNin * kPer - 1);
      const int n = e / kPer, rem = e % kPer;
      const int tok = rem / kPin, piece = rem % kPin;
      const int64_t t = min(t0 + tok, p.T - 1);
      const int slot = slot_of(n);
      const char* src = static_cast<const char*>(p.in[0]);
#pragma unroll
      for (int x = 1; x < 6; ++x)
        if (slot == x) src = static_cast<const char*>(p.in[x]);  // constant indices keep p in SGPRs
      qin[q] = *reinterpret_cast<const uint4*>(src + (seq_base + t * tok_stride + piece * kEpv) * kEsz);
    }
#pragma unroll
    for (int q = 0; q < kQdy; ++q) {
      const int e = min(tid + THREADS * q, TOK * 16 - 1);
      const int tok = e / 16, piece = e % 16;
      const int64_t t = min(t0 + tok, p.T - 1);
      qdy[q] = *reinterpret_cast<const uint4*>(p.dy + seq_base + t * tok_stride + piece * 4);
    }
  }

  __device__ void commit(float (*lds)[kSlots][kN], int tid) const {
#pragma unroll
    for (int q = 0; q < kQin; ++q) {
      const int e = min(tid + THREADS * q, kNin * kPer - 1);
      const int n = e / kPer, rem = e % kPer;
      const int tok = rem / kPin, piece = rem % kPin;
      float* dst = &lds[tok][slot_of(n)][piece * kEpv];
      const uint4 v = qin[q];
      if constexpr (BF16) {
        reinterpret_cast<float4*>(dst)[0] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
        reinterpret_cast<float4*>(dst)[1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
      } else {
        *reinterpret_cast<uint4*>(dst) = v;
      }
    }
#pragma unroll
    for (int q = 0; q < kQdy; ++q) {
      const int e = min(tid + THREADS * q, TOK * 16 - 1);
      const int tok = e / 16, piece = e % 16;
      *reinterpret_cast<uint4*>(&lds[tok][kDy][piece * 4]) = qdy[q];
    }
  }
};

// Wait for every outstanding global load of this wave (s_waitcnt vmcnt(0)).
// Placed after a loop's initial state load: otherwise the loop-carried state
// looks possibly in flight at the loop header, and the compiler waits for all
// loads (the prefetch of the next batch included) at every iteration.
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

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

// The key-space vectors at the lane's four columns, and v and dy at its rows.
template <int MR>
struct TokIn {
  float4 r4, w4, k4, a4, b4;
  float vm[MR], dym[MR];
};

// Read token j of the staged segment; rowl = the lane's first row (row0 + ri).
// BWD adds r and dy, which only the reverse step reads.
template <int MR, bool BWD>
__device__ __forceinline__ void load_tok(const float (*lds)[kSlots][kN], int j, int c, int rowl, TokIn<MR>& t) {
  if constexpr (BWD) t.r4 = *reinterpret_cast<const float4*>(&lds[j][kR][4 * c]);
  t.w4 = *reinterpret_cast<const float4*>(&lds[j][kW][4 * c]);
  t.k4 = *reinterpret_cast<const float4*>(&lds[j][kK][4 * c]);
  t.a4 = *reinterpret_cast<const float4*>(&lds[j][kA][4 * c]);
  t.b4 = *reinterpret_cast<const float4*>(&lds[j][kB][4 * c]);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    t.vm[m] = lds[j][kV][rowl + 4 * m];
    if constexpr (BWD) t.dym[m] = lds[j][kDy][rowl + 4 * m];
  }
}

// ---------------------------------------------------------------- checkpoint forward

// Inputs are staged kCkBatch tokens at a time (several checkpoint segments), so
// that the global loads for the next batch have a whole batch of compute to
// arrive in.
constexpr int kCkBatch = 4 * kSeg;

template <bool BF16, int WAVES, int NRB>
__global__ __launch_bounds__(kWave* WAVES) void wkv7_ckpt_kernel(BwdParams p) {
  constexpr int kThreads = kWave * WAVES;
  constexpr int kRpw = kN / (NRB * WAVES);
  constexpr int kMr = kRpw / 4;
  static_assert(kRpw % 4 == 0, "bad tiling");
  using Ld = SegLoader<BF16, kThreads, (1u << kW) | (1u << kK) | (1u << kV) | (1u << kA) | (1u << kB), kCkBatch>;
  __shared__ __align__(16) float lds[kCkBatch][kSlots][kN];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c = lane & 15;
  const int ri = lane >> 4;
  const uint32_t logical = xcd_swizzle(blockIdx.x, gridDim.x);  // a head's row blocks share an XCD
  const int64_t unit = logical / NRB;
  const int rb = logical % NRB;
  const int64_t bb = unit / p.H, hh = unit % p.H;
  const int64_t T = p.T;
  const int64_t tok_stride = (int64_t)p.H * kN;
  const int64_t seq_base = (bb * T * p.H + hh) * kN;
  const int row0 = (rb * WAVES + wave) * kRpw;
  const int rowl = row0 + ri;

  float4 S[kMr];
#pragma unroll
  for (int m = 0; m < kMr; ++m)
    S[m] = p.s_in ? *reinterpret_cast<const float4*>(p.s_in + (unit * kN + rowl + 4 * m) * kN + 4 * c)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  vm_wait_all();

  Ld ld;
  ld.issue(p, seq_base, tok_stride, 0, tid);
  for (int64_t tb = 0; tb < T; tb += kCkBatch) {
    __syncthreads();  // every wave is done with the previous batch's LDS
    ld.commit(lds, tid);
    __syncthreads();
    if (tb + kCkBatch < T) ld.issue(p, seq_base, tok_stride, tb + kCkBatch, tid);
    // The batch's checkpoints are kept in registers and stored after its last
    // token, so the token loop holds no global stores (a store in it makes the
    // compiler wait for the in-flight input loads before entering it).
    float4 ckr[kCkBatch / kSeg][kMr];
#pragma unroll
    for (int q = 0; q < kCkBatch / kSeg; ++q) {
      const int js = q * kSeg;
      if (tb + js < T) {
        const int n = (T - tb - js < kSeg) ? (int)(T - tb - js) : kSeg;
#pragma unroll
        for (int m = 0; m < kMr; ++m) ckr[q][m] = S[m];
        float sa[kMr];
        if (n == kSeg) {  // whole segment: the next token's reads are in flight during this one
          TokIn<kMr> cur, nxt;
          load_tok<kMr, false>(lds, js, c, rowl, cur);
#pragma unroll
          for (int j = 0; j < kSeg; ++j) {
            if (j + 1 < kSeg) load_tok<kMr, false>(lds, js + j + 1, c, rowl, nxt);
            fwd_token<kMr>(S, sa, cur.w4, cur.k4, cur.a4, cur.b4, cur.vm);
            if (j + 1 < kSeg) cur = nxt;
          }
        } else {
          for (int j = 0; j < n; ++j) {
            TokIn<kMr> cur;
            load_tok<kMr, false>(lds, js + j, c, rowl, cur);
            fwd_token<kMr>(S, sa, cur.w4, cur.k4, cur.a4, cur.b4, cur.vm);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kCkBatch / kSeg; ++q) {
      if (tb + q * kSeg < T) {
        float* ck = p.ck + (unit * p.nseg + (tb + q * kSeg) / kSeg) * (int64_t)(kN * kN);
#pragma unroll
        for (int m = 0; m < kMr; ++m) *reinterpret_cast<float4*>(ck + (rowl + 4 * m) * kN + 4 * c) = ckr[q][m];
      }
    }
  }
}

// ---------------------------------------------------------------- reverse pass

template <bool BF16, int WAVES, int NRB>
__global__ __launch_bounds__(kWave* WAVES) void wkv7_bwd_kernel(BwdParams p) {
  constexpr int kThreads = kWave * WAVES;
  constexpr int kRpb = kN / NRB;  // rows per workgroup
  constexpr int kRpw = kRpb / WAVES;
  constexpr int kMr = kRpw / 4;
  static_assert(kRpw % 4 == 0, "bad tiling");
  using Ld = SegLoader<BF16, kThreads, 0x7fu>;
  __shared__ __align__(16) float lds[kSeg][kSlots][kN];
  __shared__ __align__(16) float part[kSub][kNcol][WAVES][kN];  // per-wave column sums
  __shared__ __align__(16) float dv_lds[kSub][kRpb];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c = lane & 15;
  const int ri = lane >> 4;
  const uint32_t logical = xcd_swizzle(blockIdx.x, gridDim.x);
  const int64_t unit = logical / NRB;
  const int rb = logical % NRB;
  const int64_t bb = unit / p.H, hh = unit % p.H;
  const int64_t T = p.T;
  const int64_t tok_stride = (int64_t)p.H * kN;
  const int64_t seq_base = (bb * T * p.H + hh) * kN;
  const int rbase = rb * kRpb;             // first row of this workgroup
  const int row0 = rbase + wave * kRpw;    // first row of this wave
  const int rowl = row0 + ri;              // the lane's first row
  // column sums of this row block go to the gradients (block 0) or to the workspace copy (block 1)
  float* colout[kNcol];
  colout[kGr] = rb == 0 ? p.grad[0] : p.col1 + 0 * p.elems;
  colout[kGw] = rb == 0 ? p.grad[1] : p.col1 + 1 * p.elems;
  colout[kGk] = rb == 0 ? p.grad[2] : p.col1 + 2 * p.elems;
  colout[kGa] = rb == 0 ? p.grad[4] : p.col1 + 3 * p.elems;
  colout[kGb] = rb == 0 ? p.grad[5] : p.col1 + 4 * p.elems;

  float4 G[kMr];
#pragma unroll
  for (int m = 0; m < kMr; ++m)
    G[m] = p.ds_out ? *reinterpret_cast<const float4*>(p.ds_out + (unit * kN + rowl + 4 * m) * kN + 4 * c)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  vm_wait_all();

  const float* ck_base = p.ck + unit * p.nseg * (int64_t)(kN * kN);
  Ld ld;
  float4 ckq[kMr];
  auto issue = [&](int seg) {
    ld.issue(p, seq_base, tok_stride, (int64_t)seg * kSeg, tid);
    const float* ck = ck_base + (int64_t)seg * (kN * kN);
#pragma unroll
    for (int m = 0; m < kMr; ++m) ckq[m] = *reinterpret_cast<const float4*>(ck + (rowl + 4 * m) * kN + 4 * c);
  };

  // One token in reverse: G (dL/dS_t from later tokens) takes y's contribution,
  // the token's gradients are formed, and G moves to dL/dS_{t-1}.
  auto bwd_token = [&](int u, const TokIn<kMr>& t, const float4(&Sp)[kMr], const float4(&Sc)[kMr],
                       const float(&sa)[kMr]) {
    // G += dy r^T
#pragma unroll
    for (int m = 0; m < kMr; ++m) {
      G[m].x = fmaf(t.dym[m], t.r4.x, G[m].x);
      G[m].y = fmaf(t.dym[m], t.r4.y, G[m].y);
      G[m].z = fmaf(t.dym[m], t.r4.z, G[m].z);
      G[m].w = fmaf(t.dym[m], t.r4.w, G[m].w);
    }
    // row sums: dv = G k, gb = G b
    float dvr[kMr], gb[kMr];
#pragma unroll
    for (int m = 0; m < kMr; ++m) {
      dvr[m] = dot4(G[m], t.k4);
      gb[m] = dot4(G[m], t.b4);
    }
#pragma unroll
    for (int m = 0; m < kMr; ++m) {
      dvr[m] = row16_sum(dvr[m]);
      gb[m] = row16_sum(gb[m]);
    }
    // column partials over the lane's rows
    float X[kNcol][4];
#pragma unroll
    for (int m = 0; m < kMr; ++m) {
      const float sc[4] = {Sc[m].x, Sc[m].y, Sc[m].z, Sc[m].w};
      const float sp[4] = {Sp[m].x, Sp[m].y, Sp[m].z, Sp[m].w};
      const float gg[4] = {G[m].x, G[m].y, G[m].z, G[m].w};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        X[kGr][cc] = m == 0 ? sc[cc] * t.dym[m] : fmaf(sc[cc], t.dym[m], X[kGr][cc]);
        X[kGk][cc] = m == 0 ? gg[cc] * t.vm[m] : fmaf(gg[cc], t.vm[m], X[kGk][cc]);
        X[kGw][cc] = m == 0 ? sp[cc] * gg[cc] : fmaf(sp[cc], gg[cc], X[kGw][cc]);
        X[kGa][cc] = m == 0 ? sp[cc] * gb[m] : fmaf(sp[cc], gb[m], X[kGa][cc]);
        X[kGb][cc] = m == 0 ? gg[cc] * sa[m] : fmaf(gg[cc], sa[m], X[kGb][cc]);
      }
    }
    float colsum[kNcol];
    column_reduce(X, colsum);
#pragma unroll
    for (int x = 0; x < kNcol; ++x) part[u][x][wave][4 * c + ri] = colsum[x];
    float dvo = dvr[0];
#pragma unroll
    for (int m = 1; m < kMr; ++m) dvo = (c == m) ? dvr[m] : dvo;
    if (c < kMr) dv_lds[u][row0 - rbase + 4 * c + ri] = dvo;
    // G <- G diag(w) + gb a^T
#pragma unroll
    for (int m = 0; m < kMr; ++m) {
      G[m].x = fmaf(G[m].x, t.w4.x, gb[m] * t.a4.x);
      G[m].y = fmaf(G[m].y, t.w4.y, gb[m] * t.a4.y);
      G[m].z = fmaf(G[m].z, t.w4.z, gb[m] * t.a4.z);
      G[m].w = fmaf(G[m].w, t.w4.w, gb[m] * t.a4.w);
    }
  };

  // Tokens j0 .. j0+cnt-1 of the staged segment, whose first state is S0. A
  // whole sub-block (FULL) runs without per-token guards, with each token's LDS
  // reads issued during the previous token.
  auto sub_block = [&](auto full, int j0, int cnt, const float4(&S0)[kMr]) {
    constexpr bool kFull = decltype(full)::value;
    float4 Sv[kSub + 1][kMr];  // Sv[u] = the state before token j0 + u
#pragma unroll
    for (int m = 0; m < kMr; ++m) Sv[0][m] = S0[m];
    float sav[kSub][kMr];
    TokIn<kMr> cur, nxt;
    load_tok<kMr, false>(lds, j0, c, rowl, cur);
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      if (kFull || u < cnt) {
        if (u + 1 < kSub && (kFull || u + 1 < cnt)) load_tok<kMr, false>(lds, j0 + u + 1, c, rowl, nxt);
#pragma unroll
        for (int m = 0; m < kMr; ++m) Sv[u + 1][m] = Sv[u][m];
        fwd_token<kMr>(Sv[u + 1], sav[u], cur.w4, cur.k4, cur.a4, cur.b4, cur.vm);
        if (u + 1 < kSub) cur = nxt;
      }
    }
    load_tok<kMr, true>(lds, j0 + (kFull ? kSub : cnt) - 1, c, rowl, cur);
#pragma unroll
    for (int u = kSub - 1; u >= 0; --u) {
      if (kFull || u < cnt) {
        if (u > 0) load_tok<kMr, true>(lds, j0 + u - 1, c, rowl, nxt);
        bwd_token(u, cur, Sv[u], Sv[u + 1], sav[u]);
        if (u > 0) cur = nxt;
      }
    }
  };

  issue(p.nseg - 1);
  for (int seg = p.nseg - 1; seg >= 0; --seg) {
    const int64_t t0 = (int64_t)seg * kSeg;
    const int n = (T - t0 < kSeg) ? (int)(T - t0) : kSeg;
    __syncthreads();  // every wave is done with the previous segment's inputs
    ld.commit(lds, tid);
    float4 Sck[kMr];
#pragma unroll
    for (int m = 0; m < kMr; ++m) Sck[m] = ckq[m];
    __syncthreads();
    if (seg > 0) issue(seg - 1);

    for (int sb = (n - 1) / kSub; sb >= 0; --sb) {
      const int j0 = sb * kSub;                          // first token of the sub-block in the segment
      const int cnt = (n - j0 < kSub) ? n - j0 : kSub;   // its tokens
      // the state before token j0 of the segment
      float4 S0[kMr];
#pragma unroll
      for (int m = 0; m < kMr; ++m) S0[m] = Sck[m];
      for (int j = 0; j < j0; ++j) {
        TokIn<kMr> t;
        load_tok<kMr, false>(lds, j, c, rowl, t);
        float sa[kMr];
        fwd_token<kMr>(S0, sa, t.w4, t.k4, t.a4, t.b4, t.vm);
      }
      if (cnt == kSub)
        sub_block(std::true_type{}, j0, kSub, S0);
      else
        sub_block(std::false_type{}, j0, cnt, S0);
      __syncthreads();
      // sum the waves' partials in wave order and write the sub-block's gradients
      const int64_t tbase = seq_base + (t0 + j0) * tok_stride;
      for (int e = tid; e < cnt * kNcol * kN; e += kThreads) {
        const int u = e / (kNcol * kN), x = (e / kN) % kNcol, col = e % kN;
        float s = part[u][x][0][col];
#pragma unroll
        for (int wv = 1; wv < WAVES; ++wv) s += part[u][x][wv][col];
        float* dst = colout[0];
#pragma unroll
        for (int y = 1; y < kNcol; ++y) dst = x == y ? colout[y] : dst;
        dst[tbase + u * tok_stride + col] = s;
      }
      for (int e = tid; e < cnt * kRpb; e += kThreads) {
        const int u = e / kRpb, row = e % kRpb;
        p.grad[3][tbase + u * tok_stride + rbase + row] = dv_lds[u][row];
      }
      __syncthreads();  // the partial buffers are free again
    }
  }

  if (p.ds_in) {
#pragma unroll
    for (int m = 0; m < kMr; ++m)
      *reinterpret_cast<float4*>(p.ds_in + (unit * kN + rowl + 4 * m) * kN + 4 * c) = G[m];
  }
}

// grad[0,1,2,4,5] += the five column sums of row block 1 (float4 per thread).
__global__ __launch_bounds__(256) void wkv7_colsum_kernel(BwdParams p) {
  const int64_t n4 = p.elems / 4;
  const float4* src = reinterpret_cast<const float4*>(p.col1);
  float4* dst[kNcol] = {reinterpret_cast<float4*>(p.grad[0]), reinterpret_cast<float4*>(p.grad[1]),
                        reinterpret_cast<float4*>(p.grad[2]), reinterpret_cast<float4*>(p.grad[4]),
                        reinterpret_cast<float4*>(p.grad[5])};
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
#pragma unroll
    for (int x = 0; x < kNcol; ++x) {
      const float4 a = dst[x][i], b = src[x * n4 + i];
      dst[x][i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    }
  }
}

template <bool BF16, int CK_WAVES, int CK_NRB, int WAVES, int NRB>
hipError_t launch_cfg(BwdParams p, int64_t units, hipStream_t stream) {
  void* args[] = {&p};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&wkv7_ckpt_kernel<BF16, CK_WAVES, CK_NRB>),
                                 dim3((uint32_t)(units * CK_NRB)), dim3(kWave * CK_WAVES), args, 0, stream);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&wkv7_bwd_kernel<BF16, WAVES, NRB>),
                      dim3((uint32_t)(units * NRB)), dim3(kWave * WAVES), args, 0, stream);
  if (e != hipSuccess || NRB == 1) return e;
  const int64_t n4 = p.elems / 4;
  int64_t blocks = (n4 + 255) / 256;
  blocks = blocks > 8192 ? 8192 : blocks;
  return hipLaunchKernel(reinterpret_cast<const void*>(&wkv7_colsum_kernel), dim3((uint32_t)blocks), dim3(256),
                         args, 0, stream);
}

}  // namespace

hipError_t launch_backward(const BwdCall& c) {
  const int64_t units = c.B * c.H;
  const int64_t nseg = (c.T + kSeg - 1) / kSeg;
  if (nseg > INT32_MAX) return hipErrorNotSupported;
  // Two row blocks per head while that still fits the chip's 256 compute units.
  const bool split = units <= 128;
  const int64_t elems = units * c.T * kN;
  const size_t ck_bytes = (size_t)(units * nseg) * kN * kN * sizeof(float);
  const size_t col_bytes = split ? (size_t)elems * kNcol * sizeof(float) : 0;
  void* ws = nullptr;
  hipError_t e = device_workspace(c.stream, ck_bytes + col_bytes, &ws);
  if (e != hipSuccess) return e;
  BwdParams p{};
  for (int i = 0; i < 6; ++i) p.in[i] = c.in[i];
  p.s_in = c.s_in;
  p.dy = c.dy;
  p.ds_out = c.ds_out;
  for (int i = 0; i < 6; ++i) p.grad[i] = c.grad[i];
  p.ds_in = c.ds_in;
  p.ck = static_cast<float*>(ws);
  p.col1 = split ? reinterpret_cast<float*>(static_cast<char*>(ws) + ck_bytes) : nullptr;
  p.elems = elems;
  p.T = c.T;
  p.H = (int32_t)c.H;
  p.nseg = (int32_t)nseg;
  // checkpoint forward: 8 waves of 4 rows, two row blocks per head; reverse pass:
  // 8 waves of 4 rows (two row blocks) or of 8 rows (one row block)
  if (c.dtype == 1)
    return split ? launch_cfg<true, 8, 2, 8, 2>(p, units, c.stream) : launch_cfg<true, 8, 2, 8, 1>(p, units, c.stream);
  return split ? launch_cfg<false, 8, 2, 8, 2>(p, units, c.stream) : launch_cfg<false, 8, 2, 8, 1>(p, units, c.stream);
}

}  // namespace rwkv7
