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
#include <vector>

#include "wkv7_chunk_ops.hpp"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

using namespace chunk;

// ============================================================================ kernel 1: prep

struct PrepParams {
  PrepIn in;
  unsigned char* rec;  // [unit][chunk of slab][kRecBytes]
  int32_t c0;     // first chunk of the slab
  int32_t nc;     // chunks in the slab
  int32_t items;  // B * H * nc
};

constexpr int kPrepWaves = 4;

template <int MODE>
// three waves per SIMD: the register budget of four spills
__global__ __launch_bounds__(64 * kPrepWaves) __attribute__((amdgpu_waves_per_eu(3))) void wkv7_prep_kernel(PrepParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = (int)blockIdx.x * kPrepWaves + wave;
  if (item >= p.items) return;  // wave-uniform; this kernel has no workgroup barrier
  float* fac = reinterpret_cast<float*>(smem_raw + wave * kPrepScratch);

  // item = (b * nc + chunk) * H + h: neighbouring waves read neighbouring heads of one token block
  const int H = p.in.H;
  const int h = item % H;
  const int rest = item / H;
  const int cl = rest % p.nc;
  const int bb = rest / p.nc;
  const int unit = bb * H + h;
  const int t0 = (p.c0 + cl) * kC;
  const int nt = min(kC, p.in.T - t0);  // live tokens, >= 1
  const int64_t base = ((int64_t)bb * p.in.T + t0) * H * kN + (int64_t)h * kN;  // element offset of token t0
  unsigned char* rec = p.rec + ((int64_t)unit * p.nc + cl) * kRecBytes;
  PrepRaw x;
  prep_load<MODE>(p.in, base, nt, x);
  prep_compute<MODE>(x, fac, rec);
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
  const float* ln_w;  // time-mix form: ln_x's affine per (head, channel), may be null (1)
  const float* ln_b;  // may be null (0)
};

// A head's 64 value rows are independent: four compute waves of 16 rows each, two
// per workgroup for the plain recurrence (one workgroup per CU keeps every compute wave on
// a SIMD of its own), all four in one workgroup for the time-mix form, so that a token's
// 64 outputs meet in one workgroup for ln_x. A further wave streams the workgroup's chunks
// straight into an LDS ring with global-to-LDS loads (no register staging), kDist chunks
// ahead of the reads; the compute waves issue no global loads, so nothing they wait on is
// behind a load. One barrier per chunk.
constexpr int kDist = 5;  // chunks in flight ahead of the one read next
// ring slots: the chunk being read, the kDist in flight and one spare, so that a slot is
// reloaded only once the compute waves have used what they read from it (no wait on
// outstanding LDS reads at the barrier)
constexpr int kSlots = kDist + 2;
template <int WAVES>
struct ScanCfg {
  static constexpr int kWgPerHead = 4 / WAVES;
  static constexpr int kVCols = 16 * WAVES;           // value columns of v this workgroup needs
  static constexpr int kVBytes = kC * kVCols * 2;     // bfloat16, [token][kVCols]: 1 or 2 KiB
  static constexpr int kVLoads = kVBytes / 1024;      // one 16-byte piece per lane each
  static constexpr int kSlotBytes = kRecBytes + kVBytes;  // 10,496 / 11,520
  // y staging: two chunks (by parity) of [token][kVCols] float32, so that a workgroup's y
  // rows leave in whole 128-byte lines rather than one 64-byte half per compute wave
  static constexpr int kYStageBytes = kC * kVCols * 4;
  static constexpr int kLds = kSlots * kSlotBytes + 2 * kYStageBytes;  // 77,568 (two per CU) / 88,832
  static constexpr int kLoads = kRecBlocks + 1 + kVLoads;  // loads per lane per chunk: blocks, e^gamma, v
  static constexpr int kThreads = 64 * (WAVES + 1);
  // the load counter holds at most 63 outstanding operations: never more are in flight
  static_assert(kDist * kLoads < 64, "load counter");
  static_assert(kRecBlocks == 9 && kVBytes % 1024 == 0, "whole-wave pieces of v");
};
constexpr float kLnEps = 64e-5f;  // the GroupNorm eps of ln_x

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
// Waits until at most N of this wave's vector-memory operations are outstanding
// (they complete in issue order), and orders every later memory access after it.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// WAVES compute waves per workgroup; LN: ln_x on y before it is stored (WAVES == 4).
template <int WAVES, bool LN>
__global__ __launch_bounds__(64 * (WAVES + 1)) void wkv7_scan_kernel(ScanParams p) {
  using Cfg = ScanCfg<WAVES>;
  static_assert(!LN || WAVES == 4, "ln_x needs a token's 64 outputs in one workgroup");
  constexpr int kScanWaves = WAVES, kWgPerHead = Cfg::kWgPerHead, kVCols = Cfg::kVCols;
  constexpr int kSlotBytes = Cfg::kSlotBytes, kYStageBytes = Cfg::kYStageBytes, kLoads = Cfg::kLoads;
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
  // then v [token][kVCols] (16-byte pieces of eight columns, in token order). Tokens past the end of
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
      constexpr int ppt = kVCols / 8;  // pieces per token
#pragma unroll
      for (int h = 0; h < Cfg::kVLoads; ++h) {
        const int t = min(lane / ppt + h * (64 / ppt), nt - 1);
        to_lds<16>(vbase + ((int64_t)(xc * kC + t) * tstride + 8 * (lane % ppt)), slot + kRecBytes + 1024 * h);
      }
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
  Mma32::acc St[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) St[kt] = Mma32::zero();
  if (p.s_src) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const float4 s = *reinterpret_cast<const float4*>(p.s_src + ((int64_t)unit * kN + 16 * rb + li) * kN +
                                                        16 * kt + 4 * g);
      St[kt] = Mma32::acc{f32x4{s.x, s.y, s.z, s.w}};
    }
  }
  // vmcnt(0) as a builtin, so the compiler's own wait counting knows the state has landed
  // (it would otherwise wait for it at the first use, behind the first chunks' loads)
  __builtin_amdgcn_s_waitcnt(0x0f70);

  // fragments of one chunk, read from its ring slot one iteration ahead. The loop below
  // is unrolled by the ring size, so every slot index is a constant and every LDS
  // address a fixed offset from the lane's base.
  auto read = [&](auto slot_index, Frag& f) {
    const unsigned char* slot = ring + decltype(slot_index)::value * kSlotBytes;
    read_v(reinterpret_cast<const uint16_t*>(slot + kRecBytes) + 16 * wave, kVCols, f);
    read_frag(slot, f);
  };
  // y of chunk c goes through LDS: each compute wave stages its 16 columns (lane: token li,
  // columns 16 wave + 4g .. + 3), and after the next barrier wave q stores its 16 / WAVES
  // tokens of all kVCols columns, kVCols / 4 lanes (whole 128-byte lines) per token; tokens
  // past the end of the sequence are not stored. LN: those kVCols / 4 = 16 lanes are one DPP
  // row holding a token's 64 outputs, so ln_x (mean, then the population variance of the
  // centred values, then the affine) is two row sums before the store.
  constexpr int lpt = kVCols / 4;  // lanes per token in the store
  const int cc = 4 * (lane % lpt);
  float ln_g[4] = {1.f, 1.f, 1.f, 1.f}, ln_o[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (LN) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (p.ln_w) ln_g[e] = p.ln_w[hh * kN + cc + e];
      if (p.ln_b) ln_o[e] = p.ln_b[hh * kN + cc + e];
    }
  }
  unsigned char* ystage = ring + kSlots * kSlotBytes;
  auto stage_y = [&](auto par, const f32x4& yv) {
    *reinterpret_cast<f32x4*>(ystage + decltype(par)::value * kYStageBytes + (li * kVCols + 16 * wave + 4 * g) * 4) = yv;
  };
  auto flush_y = [&](auto par, int c) {
    const int tt = (kC / kScanWaves) * wave + lane / lpt;
    f32x4 v = *reinterpret_cast<const f32x4*>(ystage + decltype(par)::value * kYStageBytes + (tt * kVCols + cc) * 4);
    if constexpr (LN) {
      const float mu = row16_sum((v[0] + v[1]) + (v[2] + v[3])) * (1.f / kN);
      float d[4], q = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d[e] = v[e] - mu;
        q = fmaf(d[e], d[e], q);
      }
      const float inv = 1.f / sqrtf(row16_sum(q) * (1.f / kN) + kLnEps);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(d[e] * inv, ln_g[e], ln_o[e]);
    }
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
    const f32x4 yv = scan_step(St, f);
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
          make_float4(St[kt].v[0], St[kt].v[1], St[kt].v[2], St[kt].v[3]);
  }
}

// ============================================================================ host side

// Device workspace (records of the chunked split prefill, checkpoints of the
// backward, the layer stack's intermediates) cached per (device, stream): calls on
// one stream run in order, so they can share it; calls on different streams get
// different buffers. A buffer that a larger call replaces is retired, not freed: a
// HIP graph captured earlier on that stream may still hold its address, so it stays
// allocated until the process ends. Growth is at least geometric (x2), so retired
// buffers add at most the size of the live one.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::tuple<int, uintptr_t, int>, Workspace> g_ws;
std::vector<void*> g_ws_retired;  // never freed (see above)


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
    // growing allocates, which a stream under graph capture cannot record: such a call
    // must be preceded by an eager call of at least its size on the same stream
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    const size_t grow = ws.bytes > bytes / 2 ? 2 * ws.bytes : bytes;
    void* p = nullptr;
    e = hipMalloc(&p, grow);
    if (e != hipSuccess) return e;
    if (ws.ptr) g_ws_retired.push_back(ws.ptr);
    ws.ptr = p;
    ws.bytes = grow;
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
                                                   64 * kPrepWaves, kPrepWaves * kPrepScratch) != hipSuccess ||
      per_cu <= 0)
    per_cu = 2;
  return (int64_t)cus * per_cu * kPrepWaves;
}

}  // namespace

namespace {

// One chunked pass: the prep (in the given input mode) and the scan, slab by slab.
struct SplitJob {
  PrepIn in;  // input pointers (T and H are filled in from the call)
  int mode;   // kPrepTmix: the time-mix form, with ln_x applied before y is stored
  const uint16_t* v;
  float* y;
  const float* s_in;
  float* s_out;
  int64_t B, T, H;
  hipStream_t stream;
  const float* ln_w = nullptr;
  const float* ln_b = nullptr;
};

// One chunked pass, slab by slab. With fixed == nullptr the records live in the
// per-(device, stream) workspace and a slab's records fit slab_budget_bytes(); otherwise
// the records (and, when state_out is null, the state carried between slabs) live in
// fixed, cap bytes of device memory, which must hold one chunk of records for every
// head (hipErrorInvalidValue before any launch otherwise).
hipError_t run_split(const SplitJob& j, unsigned char* fixed = nullptr, size_t cap = 0) {
  const int64_t units = j.B * j.H;
  const int64_t nch = (j.T + kC - 1) / kC;
  // In-sequence offsets are 32-bit: T * H * 64 elements must stay below 2^31.
  if (j.T * j.H * kN >= (int64_t(1) << 31)) return hipErrorNotSupported;
  const int64_t per_chunk = units * kRecBytes;
  const size_t carry_bytes = (size_t)units * kN * kN * 4;
  size_t budget = slab_budget_bytes();
  if (fixed) {
    const size_t reserve = j.s_out ? 0 : carry_bytes;
    if (cap < reserve + (size_t)per_chunk) return hipErrorInvalidValue;
    budget = cap - reserve;
  }
  int64_t slab = (int64_t)(budget / (size_t)per_chunk);
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
  const size_t bytes = rec_bytes + (tmp_state ? carry_bytes : 0);
  void* ws = fixed;
  hipError_t e = hipSuccess;
  if (fixed) {
    if (bytes > cap) return hipErrorInvalidValue;
  } else {
    e = device_workspace(j.stream, bytes, &ws, kWorkspaceChunks);
    if (e != hipSuccess) return e;
  }
  unsigned char* rec = static_cast<unsigned char*>(ws);
  float* carry = tmp_state ? reinterpret_cast<float*>(rec + rec_bytes) : j.s_out;

  const void* prep_fn = j.mode == kPrepTmix ? reinterpret_cast<const void*>(&wkv7_prep_kernel<kPrepTmix>)
                                            : reinterpret_cast<const void*>(&wkv7_prep_kernel<kPrepPlain>);
  const bool tmix = j.mode == kPrepTmix;
  const void* scan_plain = reinterpret_cast<const void*>(&wkv7_scan_kernel<2, false>);
  const void* scan_ln = reinterpret_cast<const void*>(&wkv7_scan_kernel<4, true>);
  const void* scan_fn = tmix ? scan_ln : scan_plain;
  const int prep_lds = kPrepWaves * kPrepScratch;
  const int scan_lds = tmix ? ScanCfg<4>::kLds : ScanCfg<2>::kLds;
  const int scan_threads = tmix ? ScanCfg<4>::kThreads : ScanCfg<2>::kThreads;
  const int64_t scan_blocks = units * (tmix ? ScanCfg<4>::kWgPerHead : ScanCfg<2>::kWgPerHead);
  static const hipError_t a0 = hipFuncSetAttribute(reinterpret_cast<const void*>(&wkv7_prep_kernel<kPrepPlain>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, prep_lds);
  static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&wkv7_prep_kernel<kPrepTmix>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, prep_lds);
  static const hipError_t a2 =
      hipFuncSetAttribute(scan_plain, hipFuncAttributeMaxDynamicSharedMemorySize, ScanCfg<2>::kLds);
  static const hipError_t a3 = hipFuncSetAttribute(scan_ln, hipFuncAttributeMaxDynamicSharedMemorySize, ScanCfg<4>::kLds);
  if (a0 != hipSuccess) return a0;
  if (a1 != hipSuccess) return a1;
  if (a2 != hipSuccess) return a2;
  if (a3 != hipSuccess) return a3;

  for (int64_t s = 0; s < nslab; ++s) {
    const int64_t c0 = s * slab;
    const int64_t ncs = (nch - c0 < slab) ? nch - c0 : slab;
    PrepParams pp{};
    pp.in = j.in;
    pp.in.T = (int32_t)j.T;
    pp.in.H = (int32_t)j.H;
    pp.rec = rec;
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
                  (int32_t)ncs,
                  j.ln_w,
                  j.ln_b};
    void* sargs[] = {&sp};
    e = hipLaunchKernel(scan_fn, dim3((uint32_t)scan_blocks), dim3(scan_threads), sargs, scan_lds, j.stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_chunked_split(const WkvCall& c) {
  if (c.dtype != 1) return hipErrorNotSupported;  // bfloat16 inputs only
  PrepIn in{};
  in.r = static_cast<const uint16_t*>(c.in[0]);
  in.w = static_cast<const uint16_t*>(c.in[1]);
  in.k = static_cast<const uint16_t*>(c.in[2]);
  in.a = static_cast<const uint16_t*>(c.in[4]);
  in.b = static_cast<const uint16_t*>(c.in[5]);
  SplitJob j{in, kPrepPlain, static_cast<const uint16_t*>(c.in[3]), c.y, static_cast<const float*>(c.s_in),
             static_cast<float*>(c.s_out), c.B, c.T, c.H, c.stream};
  return run_split(j);
}

// ---------------------------------------------------------------------------- no-allocation variant
// The chunk records of rwkv7_wkv_prefill_noalloc live in this array, one copy per
// device (the runtime provides it when it loads this code object). Host code never
// passes the array's name to a kernel: on the host the name is a stand-in, not a
// device address. Each device's address is looked up once, with that device current,
// and only that address reaches kernels.
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_addr[kMaxScratchDevices];  // per device, null until looked up

hipError_t scratch_address(unsigned char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_chunked_split_noalloc(const WkvCall& c) {
  if (c.dtype != 1) return hipErrorNotSupported;  // bfloat16 inputs only
  unsigned char* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  PrepIn in{};
  in.r = static_cast<const uint16_t*>(c.in[0]);
  in.w = static_cast<const uint16_t*>(c.in[1]);
  in.k = static_cast<const uint16_t*>(c.in[2]);
  in.a = static_cast<const uint16_t*>(c.in[4]);
  in.b = static_cast<const uint16_t*>(c.in[5]);
  SplitJob j{in, kPrepPlain, static_cast<const uint16_t*>(c.in[3]), c.y, static_cast<const float*>(c.s_in),
             static_cast<float*>(c.s_out), c.B, c.T, c.H, c.stream};
  return run_split(j, ws, kNoallocScratchBytes);
}

size_t noalloc_scratch_need(int64_t units, bool state_out) {
  return (size_t)units * kRecBytes + (state_out ? 0 : (size_t)units * kN * kN * 4);
}

hipError_t launch_tmix_chunked(const TmixCall& c) {
  if (c.dtype != 1) return hipErrorNotSupported;  // bfloat16 inputs only
  const TmixParams& t = c.p;
  PrepIn in{};
  in.r = static_cast<const uint16_t*>(t.r);
  in.w_raw = t.w_raw;
  in.k = static_cast<const uint16_t*>(t.k);
  in.a = static_cast<const uint16_t*>(t.kk);
  in.b = static_cast<const uint16_t*>(t.a_lr);
  // the scan applies ln_x to y before it stores it into out
  SplitJob j{in, kPrepTmix, static_cast<const uint16_t*>(t.v), t.out, t.s_in, t.s_out, c.B, t.T, c.H, c.stream,
             t.ln_w, t.ln_b};
  return run_split(j);
}

}  // namespace rwkv7
