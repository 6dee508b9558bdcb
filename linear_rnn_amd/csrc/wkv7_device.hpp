// Device-side helpers shared by the WKV-7 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rwkv7 {

constexpr int kN = 64;       // head size (fixed by the model family)
constexpr int kWave = 64;    // CDNA wavefront width
constexpr uint32_t kXcds = 8;  // MI355X accelerator complex dies, each with its own L2

// bfloat16 is the upper half of a binary32 word: widening is a shift, exact.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// DPP lane exchange inside a 16-lane row. CTRL is a gfx9 DPP control code.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row with a butterfly whose partner maps are
// lane^8 (row_ror:8), lane^7 within each half (row_half_mirror), lane^2 and
// lane^1 (quad_perm). Each step adds a pair of values that both partners hold,
// and float addition commutes, so every lane of the row ends with the same bits.
__device__ __forceinline__ float row16_sum(float x) {
  x = x + dpp_f32<0x128>(x);  // row_ror:8
  x = x + dpp_f32<0x141>(x);  // row_half_mirror
  x = x + dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x = x + dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  return x;
}

// Workgroup barrier for data exchanged through LDS only: wait for this wave's
// LDS operations, then s_barrier. Unlike __syncthreads() it does not wait for
// outstanding global loads, so prefetches stay in flight across the barrier
// (their consumers wait on them through the usual register dependencies).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The dispatcher deals consecutive workgroup ids to the XCDs round-robin.
// Renumber so that each run of nblocks/8 consecutive logical ids executes on a
// single XCD; workgroups that read the same data then share one L2. Ids in the
// tail (nblocks % 8) keep their number. Bijective on [0, nblocks).
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t bid, uint32_t nblocks) {
  const uint32_t per = nblocks / kXcds;
  if (bid >= per * kXcds) return bid;
  return (bid % kXcds) * per + bid / kXcds;
}

// One token for the MR rows a lane holds (4 columns each): sa = S a (4 in-lane
// terms, then the 16-lane butterfly), S <- S diag(w) + sa b^T + v k^T, y = S r.
// Returns y of row 4c + ri when c < MR (the lane's output slot); both kernels
// call this, which keeps prefill and step bit-identical.
template <int MR>
__device__ __forceinline__ float token_update(float4 (&S)[MR], const float4 r4, const float4 w4, const float4 k4,
                                              const float4 a4, const float4 b4, const float (&vm)[MR], int c) {
  float sa[MR], yp[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m)
    sa[m] = fmaf(S[m].w, a4.w, fmaf(S[m].z, a4.z, fmaf(S[m].y, a4.y, S[m].x * a4.x)));
#pragma unroll
  for (int m = 0; m < MR; ++m) sa[m] = row16_sum(sa[m]);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    S[m].x = fmaf(S[m].x, w4.x, fmaf(sa[m], b4.x, vm[m] * k4.x));
    S[m].y = fmaf(S[m].y, w4.y, fmaf(sa[m], b4.y, vm[m] * k4.y));
    S[m].z = fmaf(S[m].z, w4.z, fmaf(sa[m], b4.z, vm[m] * k4.z));
    S[m].w = fmaf(S[m].w, w4.w, fmaf(sa[m], b4.w, vm[m] * k4.w));
  }
#pragma unroll
  for (int m = 0; m < MR; ++m)
    yp[m] = fmaf(S[m].w, r4.w, fmaf(S[m].z, r4.z, fmaf(S[m].y, r4.y, S[m].x * r4.x)));
#pragma unroll
  for (int m = 0; m < MR; ++m) yp[m] = row16_sum(yp[m]);
  float yo = yp[0];
#pragma unroll
  for (int m = 1; m < MR; ++m) yo = (c == m) ? yp[m] : yo;
  return yo;
}

}  // namespace rwkv7
