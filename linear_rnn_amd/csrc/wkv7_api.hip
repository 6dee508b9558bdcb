// C ABI of the WKV-7 library: argument validation and kernel dispatch.
// Every check runs before the first HIP call, so invalid calls are rejected
// without touching the device.
#include <stdint.h>

#include <atomic>

#include "rwkv7_wkv.h"
#include "wkv7_internal.hpp"

namespace rwkv7 {

int auto_prefill_algo(int64_t B, int64_t T, int64_t H, int dtype) {
  // the chunked kernels use 32-bit element offsets inside a sequence
  if (dtype != RWKV7_DTYPE_BF16 || T * H * 64 >= (int64_t(1) << 31)) return RWKV7_ALGO_SEQUENTIAL;
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    cus = cached[dev].load(std::memory_order_relaxed);
    if (cus == 0 && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
      cached[dev].store(cus, std::memory_order_relaxed);
  }
  if (cus <= 0) cus = 256;
  // measured on MI355X (256 CUs), up to one head per CU: the one-kernel prefill takes about 16 us
  // to fill and drain its pipeline plus 0.79 us per chunk; the split one 0.43 us per chunk of scan
  // plus 1.2 us*CUs per chunk and head of prep (4.8 ns on 256 CUs). The one-kernel form wins when
  // B*H >= CUs * (0.3 + 12.8 / chunks): 96 heads from about 2,700 tokens, 128 from 1,024, 256 from about 290.
  const int64_t nc = (T + 15) / 16;
  return B * H * nc * 10 >= (int64_t)cus * (3 * nc + 128) ? RWKV7_ALGO_CHUNKED : RWKV7_ALGO_CHUNKED_SPLIT;
}

}  // namespace rwkv7

namespace {

using rwkv7::WkvCall;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  bool empty() const { return hi <= lo; }
};

bool overlap(Range x, Range y) { return !x.empty() && !y.empty() && x.lo < y.hi && y.lo < x.hi; }

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, p ? lo + (uintptr_t)bytes : lo};
}

int validate(const void* const in[6], const void* s_in, const float* y, const void* s_out, int64_t B,
             int64_t T, int64_t H, int64_t N, int dtype, int sdtype) {
  if (dtype != RWKV7_DTYPE_F32 && dtype != RWKV7_DTYPE_BF16) return RWKV7_ERR_DTYPE;
  if (sdtype != RWKV7_STATE_F32 && sdtype != RWKV7_STATE_BF16 && sdtype != RWKV7_STATE_F16)
    return RWKV7_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0) return RWKV7_ERR_SHAPE;
  if (N != RWKV7_HEAD_SIZE) return RWKV7_ERR_HEAD_SIZE;
  // Size limits: workgroup counts up to B*H*16 must fit a 31-bit grid, and every
  // byte offset must fit in int64 with room to spare.
  int64_t units = 0, tok_heads = 0, elems = 0;
  if (__builtin_mul_overflow(B, H, &units) || units > (int64_t(1) << 26)) return RWKV7_ERR_SHAPE;
  if (__builtin_mul_overflow(units, T, &tok_heads) || __builtin_mul_overflow(tok_heads, int64_t(64), &elems) ||
      elems > (int64_t(1) << 58))
    return RWKV7_ERR_SHAPE;

  const int64_t esz = dtype == RWKV7_DTYPE_BF16 ? 2 : 4;
  const int64_t in_bytes = elems * esz;
  const int64_t y_bytes = elems * 4;
  const int64_t st_bytes = units * 64 * 64 * (sdtype == RWKV7_STATE_F32 ? 4 : 2);

  if (elems > 0) {
    for (int i = 0; i < 6; ++i)
      if (!in[i]) return RWKV7_ERR_NULL;
    if (!y) return RWKV7_ERR_NULL;
  }
  const void* ptrs[9] = {in[0], in[1], in[2], in[3], in[4], in[5], s_in, y, s_out};
  for (const void* q : ptrs)
    if (q && (reinterpret_cast<uintptr_t>(q) & 15u)) return RWKV7_ERR_ALIGN;

  const Range ry = range_of(y, y_bytes);
  const Range rsi = range_of(s_in, st_bytes);
  const Range rso = range_of(s_out, st_bytes);
  for (int i = 0; i < 6; ++i) {
    const Range ri = range_of(in[i], in_bytes);
    if (overlap(ry, ri) || overlap(rso, ri)) return RWKV7_ERR_ALIAS;
  }
  if (overlap(ry, rsi) || overlap(ry, rso)) return RWKV7_ERR_ALIAS;
  if (s_out && s_in && s_out != s_in && overlap(rso, rsi)) return RWKV7_ERR_ALIAS;
  return RWKV7_OK;
}

int run(const void* r, const void* w, const void* k, const void* v, const void* a, const void* b,
        const void* state_in, float* y, void* state_out, int64_t B, int64_t T, int64_t H, int64_t N,
        int dtype, int sdtype, int algo, bool step, void* stream) {
  const void* in[6] = {r, w, k, v, a, b};
  if (algo < RWKV7_ALGO_AUTO || algo > RWKV7_ALGO_CHUNKED_SPLIT) return RWKV7_ERR_ALGO;
  const int st = validate(in, state_in, y, state_out, B, T, H, N, dtype, sdtype);
  if (st != RWKV7_OK) return st;
  if (step && T != 1) return RWKV7_ERR_SHAPE;

  WkvCall c{{r, w, k, v, a, b}, state_in, y, state_out, B, T, H, dtype, sdtype, static_cast<hipStream_t>(stream)};
  if (B * H == 0) return RWKV7_OK;
  hipError_t e = hipSuccess;
  if (T == 0) {  // prefill only, float32 state
    if (state_out && state_out != state_in)
      e = rwkv7::launch_state_copy(static_cast<const float*>(state_in), static_cast<float*>(state_out), B * H,
                                   c.stream);
    return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
  }
  if (step) {
    e = rwkv7::launch_sequential(c, /*decode_shape=*/true);
  } else {
    if (algo == RWKV7_ALGO_AUTO) algo = rwkv7::auto_prefill_algo(B, T, H, dtype);
    e = algo == RWKV7_ALGO_CHUNKED         ? rwkv7::launch_chunked(c)
        : algo == RWKV7_ALGO_CHUNKED_SPLIT ? rwkv7::launch_chunked_split(c)
                                           : rwkv7::launch_sequential(c, false);
  }
  if (e == hipErrorNotSupported) return RWKV7_ERR_ALGO;
  return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
}

int validate_tmix(const void* const in[5], const float* w_raw, const float* ln_w, const float* ln_b,
                  const float* s_in, const float* out, const float* s_out, int64_t B, int64_t T, int64_t H, int64_t N,
                  int dtype) {
  if (dtype != RWKV7_DTYPE_F32 && dtype != RWKV7_DTYPE_BF16) return RWKV7_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0) return RWKV7_ERR_SHAPE;
  if (N != RWKV7_HEAD_SIZE) return RWKV7_ERR_HEAD_SIZE;
  int64_t units = 0, tok_heads = 0, elems = 0;
  if (__builtin_mul_overflow(B, H, &units) || units > (int64_t(1) << 26)) return RWKV7_ERR_SHAPE;
  if (__builtin_mul_overflow(units, T, &tok_heads) || __builtin_mul_overflow(tok_heads, int64_t(64), &elems) ||
      elems > (int64_t(1) << 58))
    return RWKV7_ERR_SHAPE;
  const int64_t in_bytes = elems * (dtype == RWKV7_DTYPE_BF16 ? 2 : 4);
  const int64_t f32_bytes = elems * 4;
  const int64_t st_bytes = units * 64 * 64 * 4;
  const int64_t ln_bytes = H * 64 * 4;
  if (elems > 0) {
    for (int i = 0; i < 5; ++i)
      if (!in[i]) return RWKV7_ERR_NULL;
    if (!w_raw || !out) return RWKV7_ERR_NULL;
  }
  const void* ptrs[11] = {in[0], in[1], in[2], in[3], in[4], w_raw, ln_w, ln_b, s_in, out, s_out};
  for (const void* q : ptrs)
    if (q && (reinterpret_cast<uintptr_t>(q) & 15u)) return RWKV7_ERR_ALIGN;
  const Range ro = range_of(out, f32_bytes);
  const Range rso = range_of(s_out, st_bytes);
  const Range rsi = range_of(s_in, st_bytes);
  const Range srcs[8] = {range_of(in[0], in_bytes), range_of(in[1], in_bytes), range_of(in[2], in_bytes),
                         range_of(in[3], in_bytes), range_of(in[4], in_bytes), range_of(w_raw, f32_bytes),
                         range_of(ln_w, ln_bytes), range_of(ln_b, ln_bytes)};
  for (const Range& ri : srcs)
    if (overlap(ro, ri) || overlap(rso, ri)) return RWKV7_ERR_ALIAS;
  if (overlap(ro, rsi) || overlap(ro, rso)) return RWKV7_ERR_ALIAS;
  if (s_out && s_in && s_out != s_in && overlap(rso, rsi)) return RWKV7_ERR_ALIAS;
  return RWKV7_OK;
}

int run_tmix(const void* r, const float* w_raw, const void* k, const void* v, const void* kk, const void* a_lr,
             const float* ln_w, const float* ln_b, const float* state_in, float* out, float* state_out, int64_t B,
             int64_t T, int64_t H, int64_t N, int dtype, int algo, bool step, void* stream) {
  const void* in[5] = {r, k, v, kk, a_lr};
  const int st = validate_tmix(in, w_raw, ln_w, ln_b, state_in, out, state_out, B, T, H, N, dtype);
  if (st != RWKV7_OK) return st;
  if (step && T != 1) return RWKV7_ERR_SHAPE;
  // the token-by-token kernel (AUTO keeps the bit-exact match with T single steps), or
  // the chunked prefill for bfloat16 inputs
  if (algo < RWKV7_ALGO_AUTO || algo > RWKV7_ALGO_CHUNKED_SPLIT) return RWKV7_ERR_ALGO;
  if ((algo == RWKV7_ALGO_CHUNKED || algo == RWKV7_ALGO_CHUNKED_SPLIT) && dtype != RWKV7_DTYPE_BF16)
    return RWKV7_ERR_ALGO;
  if (B * H == 0) return RWKV7_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (T == 0) {
    if (state_out && state_out != state_in) e = rwkv7::launch_state_copy(state_in, state_out, B * H, s);
    return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
  }
  rwkv7::TmixCall c{{r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, T, (int32_t)H}, B, H, dtype, s};
  c.algo = algo;
  e = rwkv7::launch_tmix(c);
  if (e == hipErrorNotSupported) return RWKV7_ERR_ALGO;
  return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
}

int validate_backward(const void* const in[6], const float* s_in, const float* dy, const float* ds_out,
                      float* const grad[6], const float* ds_in, int64_t B, int64_t T, int64_t H, int64_t N,
                      int dtype) {
  if (dtype != RWKV7_DTYPE_F32 && dtype != RWKV7_DTYPE_BF16) return RWKV7_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0) return RWKV7_ERR_SHAPE;
  if (N != RWKV7_HEAD_SIZE) return RWKV7_ERR_HEAD_SIZE;
  int64_t units = 0, tok_heads = 0, elems = 0;
  if (__builtin_mul_overflow(B, H, &units) || units > (int64_t(1) << 26)) return RWKV7_ERR_SHAPE;
  if (__builtin_mul_overflow(units, T, &tok_heads) || __builtin_mul_overflow(tok_heads, int64_t(64), &elems) ||
      elems > (int64_t(1) << 58))
    return RWKV7_ERR_SHAPE;
  const int64_t in_bytes = elems * (dtype == RWKV7_DTYPE_BF16 ? 2 : 4);
  const int64_t f32_bytes = elems * 4;
  const int64_t st_bytes = units * 64 * 64 * 4;
  if (elems > 0) {
    for (int i = 0; i < 6; ++i)
      if (!in[i] || !grad[i]) return RWKV7_ERR_NULL;
    if (!dy) return RWKV7_ERR_NULL;
  }
  const void* ptrs[16] = {in[0],   in[1],   in[2],   in[3],   in[4],   in[5],   s_in,    dy,
                          ds_out,  grad[0], grad[1], grad[2], grad[3], grad[4], grad[5], ds_in};
  for (const void* q : ptrs)
    if (q && (reinterpret_cast<uintptr_t>(q) & 15u)) return RWKV7_ERR_ALIGN;
  Range src[9];
  for (int i = 0; i < 6; ++i) src[i] = range_of(in[i], in_bytes);
  src[6] = range_of(s_in, st_bytes);
  src[7] = range_of(dy, f32_bytes);
  src[8] = range_of(ds_out, st_bytes);
  Range dst[7];
  for (int i = 0; i < 6; ++i) dst[i] = range_of(grad[i], f32_bytes);
  dst[6] = range_of(ds_in, st_bytes);
  for (int d = 0; d < 7; ++d) {
    for (int i = 0; i < 9; ++i) {
      if (d == 6 && i == 8 && ds_in == ds_out) continue;  // dstate in place
      if (overlap(dst[d], src[i])) return RWKV7_ERR_ALIAS;
    }
    for (int e = d + 1; e < 7; ++e)
      if (overlap(dst[d], dst[e])) return RWKV7_ERR_ALIAS;
  }
  return RWKV7_OK;
}

int validate_stack(const void* w_in, const void* w_out, const float* vecs, const float* x, const float* states,
                   int64_t L, int64_t B, int64_t T, int64_t H, int64_t N, int dtype) {
  if (dtype != RWKV7_DTYPE_F32 && dtype != RWKV7_DTYPE_BF16) return RWKV7_ERR_DTYPE;
  if (L < 0 || B < 0 || T < 0 || H < 0) return RWKV7_ERR_SHAPE;
  if (N != RWKV7_HEAD_SIZE) return RWKV7_ERR_HEAD_SIZE;
  // The projections' sizes must fit the GEMM library's 32-bit arguments: rows B*T and
  // columns 5*D below 2^31; the tensors' byte sizes must fit int64 with room.
  int64_t units = 0, M = 0, MD = 0, st = 0;
  if (__builtin_mul_overflow(B, H, &units) || units > (int64_t(1) << 26)) return RWKV7_ERR_SHAPE;
  if (H > (int64_t(1) << 20) || L > (int64_t(1) << 20)) return RWKV7_ERR_SHAPE;
  if (__builtin_mul_overflow(B, T, &M) || M >= (int64_t(1) << 31)) return RWKV7_ERR_SHAPE;
  const int64_t D = H * 64;
  if (__builtin_mul_overflow(M, D, &MD) || MD > (int64_t(1) << 40)) return RWKV7_ERR_SHAPE;
  if (__builtin_mul_overflow(units * 64 * 64, L, &st) || st > (int64_t(1) << 40)) return RWKV7_ERR_SHAPE;
  const int64_t esz = dtype == RWKV7_DTYPE_BF16 ? 2 : 4;
  if (L * D * D * 5 * esz > (int64_t(1) << 50)) return RWKV7_ERR_SHAPE;
  const bool work = L > 0 && MD > 0;
  if (work && (!w_in || !w_out || !vecs || !x || !states)) return RWKV7_ERR_NULL;
  const void* ptrs[5] = {w_in, w_out, vecs, x, states};
  for (const void* q : ptrs)
    if (q && (reinterpret_cast<uintptr_t>(q) & 15u)) return RWKV7_ERR_ALIGN;
  const Range rx = range_of(x, MD * 4), rs = range_of(states, st * 4);
  const Range srcs[3] = {range_of(w_in, L * D * 5 * D * esz), range_of(w_out, L * D * D * esz),
                         range_of(vecs, L * 5 * D * 4)};
  for (const Range& r : srcs)
    if (overlap(rx, r) || overlap(rs, r)) return RWKV7_ERR_ALIAS;
  if (overlap(rx, rs)) return RWKV7_ERR_ALIAS;
  return RWKV7_OK;
}

}  // namespace

extern "C" {

int rwkv7_stack_forward(const void* w_in, const void* w_out, const float* vecs, float* x, float* states, int64_t L,
                        int64_t B, int64_t T, int64_t H, int64_t N, int dtype, void* stream) {
  const int st = validate_stack(w_in, w_out, vecs, x, states, L, B, T, H, N, dtype);
  if (st != RWKV7_OK) return st;
  if (L == 0 || B * T * H == 0) return RWKV7_OK;
  rwkv7::StackCall c{w_in, w_out, vecs, x, states, L, B, T, H, dtype, static_cast<hipStream_t>(stream)};
  const hipError_t e = rwkv7::launch_stack(c);
  return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
}

int rwkv7_wkv_backward(const void* r, const void* w, const void* k, const void* v, const void* a, const void* b,
                       const float* state_in, const float* dy, const float* dstate_out, float* dr, float* dw,
                       float* dk, float* dv, float* da, float* db, float* dstate_in, int64_t B, int64_t T,
                       int64_t H, int64_t N, int dtype, void* stream) {
  return rwkv7_wkv_backward_ex(r, w, k, v, a, b, state_in, dy, dstate_out, dr, dw, dk, dv, da, db, dstate_in, B, T,
                               H, N, dtype, RWKV7_ALGO_AUTO, stream);
}

int rwkv7_wkv_backward_ex(const void* r, const void* w, const void* k, const void* v, const void* a,
                          const void* b, const float* state_in, const float* dy, const float* dstate_out, float* dr,
                          float* dw, float* dk, float* dv, float* da, float* db, float* dstate_in, int64_t B,
                          int64_t T, int64_t H, int64_t N, int dtype, int algo, void* stream) {
  const void* in[6] = {r, w, k, v, a, b};
  float* const grad[6] = {dr, dw, dk, dv, da, db};
  const int st = validate_backward(in, state_in, dy, dstate_out, grad, dstate_in, B, T, H, N, dtype);
  if (st != RWKV7_OK) return st;
  if (algo != RWKV7_ALGO_AUTO && algo != RWKV7_ALGO_SEQUENTIAL && algo != RWKV7_ALGO_CHUNKED) return RWKV7_ERR_ALGO;
  if (algo == RWKV7_ALGO_CHUNKED && (dtype != RWKV7_DTYPE_BF16 || T * H * 64 >= (int64_t(1) << 31)))
    return RWKV7_ERR_ALGO;
  if (B * H == 0) return RWKV7_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (T == 0) {  // no tokens: the state gradient passes through
    if (dstate_in && dstate_in != dstate_out) e = rwkv7::launch_state_copy(dstate_out, dstate_in, B * H, s);
    return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
  }
  rwkv7::BwdCall c{{r, w, k, v, a, b}, state_in, dy, dstate_out, {dr, dw, dk, dv, da, db}, dstate_in, B, T, H,
                   dtype, s};
  // AUTO: the chunked backward for bfloat16 inputs inside its domain (as the prefill's AUTO),
  // the float32 token-by-token one otherwise
  if (algo == RWKV7_ALGO_AUTO && dtype == RWKV7_DTYPE_BF16 && T * H * 64 < (int64_t(1) << 31))
    algo = RWKV7_ALGO_CHUNKED;
  if (algo == RWKV7_ALGO_CHUNKED) {
    e = rwkv7::launch_backward_chunked(c);
    if (e == hipErrorNotSupported) return RWKV7_ERR_ALGO;
    return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
  }
  e = rwkv7::launch_backward(c);
  if (e == hipErrorNotSupported) return RWKV7_ERR_SHAPE;
  return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
}

int rwkv7_tmix_prefill(const void* r, const float* w_raw, const void* k, const void* v, const void* kk,
                       const void* a_lr, const float* ln_w, const float* ln_b, const float* state_in, float* out,
                       float* state_out, int64_t B, int64_t T, int64_t H, int64_t N, int dtype, void* stream) {
  return run_tmix(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, B, T, H, N, dtype, RWKV7_ALGO_AUTO,
                  false, stream);
}

int rwkv7_tmix_prefill_ex(const void* r, const float* w_raw, const void* k, const void* v, const void* kk,
                          const void* a_lr, const float* ln_w, const float* ln_b, const float* state_in, float* out,
                          float* state_out, int64_t B, int64_t T, int64_t H, int64_t N, int dtype, int algo,
                          void* stream) {
  return run_tmix(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, B, T, H, N, dtype, algo, false,
                  stream);
}

int rwkv7_tmix_step(const void* r, const float* w_raw, const void* k, const void* v, const void* kk,
                    const void* a_lr, const float* ln_w, const float* ln_b, const float* state_in, float* out,
                    float* state_out, int64_t B, int64_t T, int64_t H, int64_t N, int dtype, void* stream) {
  return run_tmix(r, w_raw, k, v, kk, a_lr, ln_w, ln_b, state_in, out, state_out, B, T, H, N, dtype, RWKV7_ALGO_AUTO,
                  true, stream);
}


int rwkv7_wkv_prefill(const void* r, const void* w, const void* k, const void* v, const void* a, const void* b,
                      const float* state_in, float* y, float* state_out, int64_t B, int64_t T, int64_t H,
                      int64_t N, int dtype, void* stream) {
  return run(r, w, k, v, a, b, state_in, y, state_out, B, T, H, N, dtype, RWKV7_STATE_F32, RWKV7_ALGO_AUTO, false,
             stream);
}

int rwkv7_wkv_step(const void* r, const void* w, const void* k, const void* v, const void* a, const void* b,
                   const float* state_in, float* y, float* state_out, int64_t B, int64_t T, int64_t H, int64_t N,
                   int dtype, void* stream) {
  return run(r, w, k, v, a, b, state_in, y, state_out, B, T, H, N, dtype, RWKV7_STATE_F32, RWKV7_ALGO_SEQUENTIAL,
             true, stream);
}

int rwkv7_wkv_step_q(const void* r, const void* w, const void* k, const void* v, const void* a, const void* b,
                     const void* state_in, float* y, void* state_out, int64_t B, int64_t T, int64_t H, int64_t N,
                     int dtype, int state_dtype, void* stream) {
  return run(r, w, k, v, a, b, state_in, y, state_out, B, T, H, N, dtype, state_dtype, RWKV7_ALGO_SEQUENTIAL, true,
             stream);
}

int rwkv7_wkv_prefill_ex(const void* r, const void* w, const void* k, const void* v, const void* a,
                         const void* b, const float* state_in, float* y, float* state_out, int64_t B, int64_t T,
                         int64_t H, int64_t N, int dtype, int algo, void* stream) {
  return run(r, w, k, v, a, b, state_in, y, state_out, B, T, H, N, dtype, RWKV7_STATE_F32, algo, false, stream);
}

int rwkv7_wkv_prefill_noalloc(const void* r, const void* w, const void* k, const void* v, const void* a,
                              const void* b, const float* state_in, float* y, float* state_out, int64_t B, int64_t T,
                              int64_t H, int64_t N, int dtype, void* stream) {
  const void* in[6] = {r, w, k, v, a, b};
  const int st = validate(in, state_in, y, state_out, B, T, H, N, dtype, RWKV7_STATE_F32);
  if (st != RWKV7_OK) return st;
  if (dtype != RWKV7_DTYPE_BF16) return RWKV7_ERR_ALGO;
  if (B * H == 0) return RWKV7_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    const hipError_t e = state_out && state_out != state_in ? rwkv7::launch_state_copy(state_in, state_out, B * H, s)
                                                            : hipSuccess;
    return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
  }
  if (T * H * 64 >= (int64_t(1) << 31)) return RWKV7_ERR_ALGO;
  if (rwkv7::noalloc_scratch_need(B * H, state_out != nullptr) > rwkv7::kNoallocScratchBytes)
    return RWKV7_ERR_SCRATCH;
  WkvCall c{{r, w, k, v, a, b}, state_in, y, state_out, B, T, H, dtype, RWKV7_STATE_F32, s};
  const hipError_t e = rwkv7::launch_chunked_split_noalloc(c);
  if (e == hipErrorInvalidValue) return RWKV7_ERR_SCRATCH;
  if (e == hipErrorNotSupported) return RWKV7_ERR_ALGO;
  return e == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
}

int rwkv7_wkv_prefill_algo(int64_t B, int64_t T, int64_t H, int64_t N, int dtype) {
  if (dtype != RWKV7_DTYPE_F32 && dtype != RWKV7_DTYPE_BF16) return RWKV7_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0) return RWKV7_ERR_SHAPE;
  if (N != RWKV7_HEAD_SIZE) return RWKV7_ERR_HEAD_SIZE;
  int64_t units = 0, tok_heads = 0, elems = 0;
  if (__builtin_mul_overflow(B, H, &units) || units > (int64_t(1) << 26)) return RWKV7_ERR_SHAPE;
  if (__builtin_mul_overflow(units, T, &tok_heads) || __builtin_mul_overflow(tok_heads, int64_t(64), &elems) ||
      elems > (int64_t(1) << 58))
    return RWKV7_ERR_SHAPE;
  return rwkv7::auto_prefill_algo(B, T, H, dtype);
}

const char* rwkv7_wkv_strerror(int status) {
  switch (status) {
    case RWKV7_OK: return "success";
    case RWKV7_ERR_NULL: return "a required pointer is NULL";
    case RWKV7_ERR_SHAPE: return "invalid shape (negative B/T/H, T != 1 for a step, or sizes too large)";
    case RWKV7_ERR_HEAD_SIZE: return "head size N must be 64";
    case RWKV7_ERR_DTYPE: return "unknown input or state dtype";
    case RWKV7_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case RWKV7_ERR_ALIAS: return "outputs overlap inputs or each other";
    case RWKV7_ERR_ALGO: return "unknown or unsupported algorithm for these arguments";
    case RWKV7_ERR_HIP: return "HIP runtime error";
    case RWKV7_ERR_SCRATCH: return "the call needs more than the static scratch array of rwkv7_wkv_prefill_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
