// A stack of L time-mix layers over a residual stream: the hybrid "fast" mode
// of RWKV-7 inference (RWKV-7 G0 7.2B notes, lshu.cn/news/198401, section 3.2:
// the prompt goes through the model in one parallel pass, then tokens are
// generated one at a time with a fixed-size state per layer, section 3.3). One
// call takes T tokens through every layer; T = 1 is a generation step. Each
// layer keeps its own 64x64 float32 WKV state per head, carried in and out.
//
// Per layer l, with x the [M = B*T, D = H*64] float32 residual stream and the
// time-mix parameterisation of section 7.1 (decay soft-clamped by a softplus and
// applied as exp(-exp(.)); the in-context learning rate a sigmoid; the removal
// key the key scaled per channel and L2-normalised per head; ln_x a GroupNorm):
//   P     = x W_in[l]                       [M, 5D]: column blocks r | k | v | w | a
//   w_raw = -softplus(-(w0 + P_w)) - 0.5    float32
//   kk    = P_k * k_k;  a_lr = sigmoid(a0 + P_a)
//   o     = ln_x(wkv7(r, w, k, v, a = -kk^, b = kk^ a_lr))   (the fused operator)
//   x    += o W_out[l]
// Token shift, the channel mix, the output gate and the low-rank projections of
// the full model are not part of this stack.
//
// Kernels per layer: a cast of x to the weights' dtype (bfloat16 only), the
// input projection (rocBLAS GEMM, float32 accumulation and output), the
// activation kernel below, the fused time-mix kernel (one workgroup per head),
// a cast of o, and the output projection accumulated into x by the GEMM
// (beta = 1). Intermediates live in the per-(device, stream) workspace. A
// bfloat16 prompt of 32 tokens or more runs the time-mix operator as a chunked
// prefill (its own workspace); shorter calls run it token by token.
#include <rocblas/rocblas.h>

#include <map>
#include <mutex>
#include <utility>

#include "wkv7_device.hpp"
#include "rwkv7_wkv.h"
#include "wkv7_internal.hpp"

namespace rwkv7 {
namespace {

__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// dst (bfloat16) <- src (float32), four elements per thread.
__global__ __launch_bounds__(256) void stack_cast_kernel(const float* src, uint16_t* dst, int64_t n4) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    reinterpret_cast<uint2*>(dst)[i] = make_uint2(bf16_pack(v.x, v.y), bf16_pack(v.z, v.w));
  }
}

struct ActParams {
  const float* P;     // [M, 5D]
  const float* vecs;  // this layer's [5, D]: w0, a0, k_k, ln_w, ln_b
  void* r;
  void* k;
  void* v;
  float* w_raw;
  void* kk;
  void* a_lr;
  int64_t M;
  int32_t D;
};

// softplus(z) = log(1 + e^z), without overflow for large z.
__device__ __forceinline__ float softplus(float z) { return z > 20.f ? z : log1pf(expf(z)); }

template <bool BF16>
__device__ __forceinline__ void put(void* base, int64_t i, float x) {
  if constexpr (BF16)
    static_cast<uint16_t*>(base)[i] = __builtin_bit_cast(uint16_t, (__bf16)x);
  else
    static_cast<float*>(base)[i] = x;
}

// One thread per (row, channel): the operator's inputs from the projection.
template <bool BF16>
__global__ __launch_bounds__(256) void stack_act_kernel(ActParams p) {
  const int64_t n = p.M * p.D;
  const int D = p.D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / D;
    const int c = (int)(i - m * D);
    const float* row = p.P + m * 5 * (int64_t)D;
    const float pk = row[D + c];
    put<BF16>(p.r, i, row[c]);
    put<BF16>(p.k, i, pk);
    put<BF16>(p.v, i, row[2 * D + c]);
    p.w_raw[i] = -softplus(-(p.vecs[c] + row[3 * D + c])) - 0.5f;
    put<BF16>(p.kk, i, pk * p.vecs[2 * D + c]);
    put<BF16>(p.a_lr, i, 1.f / (1.f + expf(-(p.vecs[D + c] + row[4 * D + c]))));
  }
}

// rocBLAS handles, one per (device, stream), used under the lock.
std::mutex g_blas_mu;
std::map<std::pair<int, uintptr_t>, rocblas_handle> g_blas;

hipError_t blas_handle(hipStream_t stream, rocblas_handle* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto key = std::make_pair(dev, reinterpret_cast<uintptr_t>(stream));
  auto it = g_blas.find(key);
  if (it == g_blas.end()) {
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return hipErrorUnknown;
    if (rocblas_set_stream(h, stream) != rocblas_status_success) {
      rocblas_destroy_handle(h);
      return hipErrorUnknown;
    }
    it = g_blas.emplace(key, h).first;
  }
  *out = it->second;
  return hipSuccess;
}

// Row-major Y[M, N] = X[M, K] W[K, N] + beta Y, float32 accumulation and output. In
// rocBLAS's column-major terms this is Y^T = W^T X^T with the same buffers.
hipError_t gemm(rocblas_handle h, bool bf16, const void* X, const void* W, float* Y, int64_t M, int64_t K, int64_t N,
                float beta) {
  const float alpha = 1.f;
  const rocblas_datatype ab = bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const rocblas_status st = rocblas_gemm_ex(
      h, rocblas_operation_none, rocblas_operation_none, (rocblas_int)N, (rocblas_int)M, (rocblas_int)K, &alpha, W, ab,
      (rocblas_int)N, X, ab, (rocblas_int)K, &beta, Y, rocblas_datatype_f32_r, (rocblas_int)N, Y,
      rocblas_datatype_f32_r, (rocblas_int)N, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? hipSuccess : hipErrorUnknown;
}

// bfloat16 prompts of at least this many tokens run the time-mix operator as a
// chunked prefill (shorter ones and single-token calls run it token by token)
constexpr int64_t kChunkedPromptMin = 32;

uint32_t grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (uint32_t)(b > 16384 ? 16384 : (b < 1 ? 1 : b));
}

}  // namespace

hipError_t launch_stack(const StackCall& c) {
  const bool bf16 = c.dtype == 1;
  const int64_t esz = bf16 ? 2 : 4;
  const int64_t D = c.H * kN;
  const int64_t M = c.B * c.T;
  const int64_t MD = M * D;
  // workspace: P [M,5D] f32 | r k v kk a_lr (dtype) | w_raw f32 | o f32 | x and o in dtype (bf16 only)
  const size_t bP = (size_t)MD * 5 * 4, bIn = (size_t)MD * esz, bF = (size_t)MD * 4;
  const size_t need = bP + 5 * bIn + 2 * bF + (bf16 ? 2 * bIn : 0);
  void* ws = nullptr;
  hipError_t e = device_workspace(c.stream, need, &ws);
  if (e != hipSuccess) return e;
  char* q = static_cast<char*>(ws);
  float* P = reinterpret_cast<float*>(q);
  q += bP;
  void* in[5];  // r, k, v, kk, a_lr
  for (int i = 0; i < 5; ++i, q += bIn) in[i] = q;
  float* w_raw = reinterpret_cast<float*>(q);
  q += bF;
  float* o = reinterpret_cast<float*>(q);
  q += bF;
  uint16_t* xq = bf16 ? reinterpret_cast<uint16_t*>(q) : nullptr;
  uint16_t* oq = bf16 ? reinterpret_cast<uint16_t*>(q + bIn) : nullptr;

  std::lock_guard<std::mutex> lk(g_blas_mu);
  rocblas_handle h = nullptr;
  e = blas_handle(c.stream, &h);
  if (e != hipSuccess) return e;
  const uint32_t g4 = grid_for(MD / 4), g1 = grid_for(MD);
  for (int64_t l = 0; l < c.L; ++l) {
    const char* w_in = static_cast<const char*>(c.w_in) + (size_t)l * D * 5 * D * esz;
    const char* w_out = static_cast<const char*>(c.w_out) + (size_t)l * D * D * esz;
    const float* vecs = c.vecs + l * 5 * D;
    float* state = c.states + l * c.B * c.H * kN * kN;
    const void* xin = c.x;
    if (bf16) {
      const float* src = c.x;
      int64_t n4 = MD / 4;
      void* args[] = {&src, &xq, &n4};
      e = hipLaunchKernel(reinterpret_cast<const void*>(&stack_cast_kernel), dim3(g4), dim3(256), args, 0, c.stream);
      if (e != hipSuccess) return e;
      xin = xq;
    }
    e = gemm(h, bf16, xin, w_in, P, M, D, 5 * D, 0.f);
    if (e != hipSuccess) return e;
    ActParams ap{P, vecs, in[0], in[1], in[2], w_raw, in[3], in[4], M, (int32_t)D};
    void* aargs[] = {&ap};
    e = hipLaunchKernel(bf16 ? reinterpret_cast<const void*>(&stack_act_kernel<true>)
                             : reinterpret_cast<const void*>(&stack_act_kernel<false>),
                        dim3(g1), dim3(256), aargs, 0, c.stream);
    if (e != hipSuccess) return e;
    TmixCall tc{{in[0], w_raw, in[1], in[2], in[3], in[4], vecs + 3 * D, vecs + 4 * D, state, o, state, c.T,
                 (int32_t)c.H},
                c.B, c.H, c.dtype, c.stream};
    tc.algo = bf16 && c.T >= kChunkedPromptMin ? auto_prefill_algo(c.B, c.T, c.H, c.dtype) : RWKV7_ALGO_SEQUENTIAL;
    e = launch_tmix(tc);
    if (e != hipSuccess) return e;
    const void* oin = o;
    if (bf16) {
      const float* src = o;
      int64_t n4 = MD / 4;
      void* args[] = {&src, &oq, &n4};
      e = hipLaunchKernel(reinterpret_cast<const void*>(&stack_cast_kernel), dim3(g4), dim3(256), args, 0, c.stream);
      if (e != hipSuccess) return e;
      oin = oq;
    }
    e = gemm(h, bf16, oin, w_out, c.x, M, D, D, 1.f);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rwkv7
