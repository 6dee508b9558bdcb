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

}  // namespace rwkv7
