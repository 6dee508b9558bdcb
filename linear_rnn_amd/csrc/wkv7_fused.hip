// Chunked WKV-7 prefill in one kernel: one workgroup per head, whose prep waves
// form the chunk records (the chunk algebra of wkv7_chunk_ops.hpp) into an LDS
// ring and whose scan waves carry the float32 state through them in order. No
// record leaves the compute unit, so the kernel moves only the algorithmic bytes:
// the six inputs once, y once, the state in and out.
//
// Roles (12 waves, three per SIMD):
//   waves 0-3   scan: wave w owns value rows 16w .. 16w + 15 of the state (float32, in
//               MFMA accumulators); per chunk ten 16x16x32 MFMAs and one 16-byte y
//               store per lane (RWKV-7 G0 7.2B notes, lshu.cn/news/198401, section
//               7.1: y is read out with r after the update).
//   waves 4-11  prep: wave p takes chunks p, p + 8, p + 16, ...; it loads the chunk's
//               r, w, k, a, b, waits for its ring slot to be free,
//               forms the record in the slot (its factor and solve scratch lives at the
//               slot's start) and marks the slot ready.
// Hand-off through LDS words, no workgroup barrier after the first: ready[slot] holds
// the last chunk whose record is complete in that slot (written after the writer's
// LDS stores have completed), consumed[w] the number of chunks whose fragments scan
// wave w has read into registers. A prep wave reuses the slot of chunk c - kRing once
// every consumed[w] > c - kRing. The smallest unfinished chunk never waits on a later
// one, so the hand-off cannot deadlock; every wait is also bounded (kSpinMax polls),
// so a wave never spins forever even if the protocol were broken.
#include <cstdint>

#include "wkv7_fused.hpp"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

using namespace chunk;
using namespace fused;

template <int MODE, bool CK = false, bool ROWS = true>
__global__ __launch_bounds__(kThreads) void wkv7_fused_kernel(FusedParams p) {
  extern __shared__ __align__(16) unsigned char ring[];
  fused_body<MODE, CK, ROWS>(p, ring, blockIdx.x);
}

template <int MODE, bool CK = false, bool ROWS = true>
hipError_t launch_fused(const FusedParams& fp, int64_t units, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&wkv7_fused_kernel<MODE, CK, ROWS>);
  static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (attr != hipSuccess) return attr;
  FusedParams q = fp;
  void* args[] = {&q};
  return hipLaunchKernel(fn, dim3((uint32_t)units), dim3(kThreads), args, kLds, stream);
}

// Compute units of the current device (256 if the query fails).
int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

// Offsets inside a sequence are 32-bit element counts (T * H * 64 below 2^31).
bool fused_domain(int64_t T, int64_t H) { return T * H * kN < (int64_t(1) << 31); }


}  // namespace

hipError_t launch_chunked(const WkvCall& c) {
  // bfloat16 inputs only: float32 inputs keep float32 accuracy on the sequential kernel
  if (c.dtype != 1 || !fused_domain(c.T, c.H)) return hipErrorNotSupported;
  FusedParams fp{};
  fp.in.r = static_cast<const uint16_t*>(c.in[0]);
  fp.in.w = static_cast<const uint16_t*>(c.in[1]);
  fp.in.k = static_cast<const uint16_t*>(c.in[2]);
  fp.in.a = static_cast<const uint16_t*>(c.in[4]);
  fp.in.b = static_cast<const uint16_t*>(c.in[5]);
  fp.in.T = (int32_t)c.T;
  fp.in.H = (int32_t)c.H;
  fp.v = static_cast<const uint16_t*>(c.in[3]);
  fp.y = c.y;
  fp.s_in = static_cast<const float*>(c.s_in);
  fp.s_out = static_cast<float*>(c.s_out);
  fp.nc = (int32_t)((c.T + kC - 1) / kC);
  // y as whole token rows when the heads fill the chip, else through each scan wave's tile
  const int64_t units = c.B * c.H;
  if (units >= cu_count()) return launch_fused<kPrepPlain, false, true>(fp, units, c.stream);
  return launch_fused<kPrepPlain, false, false>(fp, units, c.stream);
}

hipError_t launch_tmix_fused(const TmixCall& c) {
  const TmixParams& t = c.p;
  if (c.dtype != 1 || !fused_domain(t.T, c.H)) return hipErrorNotSupported;
  FusedParams fp{};
  fp.in.r = static_cast<const uint16_t*>(t.r);
  fp.in.w_raw = t.w_raw;
  fp.in.k = static_cast<const uint16_t*>(t.k);
  fp.in.a = static_cast<const uint16_t*>(t.kk);
  fp.in.b = static_cast<const uint16_t*>(t.a_lr);
  fp.in.T = (int32_t)t.T;
  fp.in.H = (int32_t)c.H;
  fp.v = static_cast<const uint16_t*>(t.v);
  fp.y = t.out;
  fp.s_in = t.s_in;
  fp.s_out = t.s_out;
  fp.nc = (int32_t)((t.T + kC - 1) / kC);
  fp.ln_w = t.ln_w;  // ln_x is applied by the scan waves before y is stored
  fp.ln_b = t.ln_b;
  return launch_fused<kPrepTmix>(fp, c.B * c.H, c.stream);
}

}  // namespace rwkv7
