// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rwkv7 {

// One validated call. Input order in `in`: r, w, k, v, a, b.
struct WkvCall {
  const void* in[6];
  const void* s_in;  // may be null (zero state); element type given by sdtype
  float* y;
  void* s_out;  // may be null
  int64_t B, T, H;
  int dtype;   // RWKV7_DTYPE_*
  int sdtype;  // RWKV7_STATE_*: float32 unless a reduced-precision step
  hipStream_t stream;
};

// The prefill algorithm that RWKV7_ALGO_AUTO runs (an RWKV7_ALGO_* value):
//   float32 inputs                           sequential (their 1e-5 bar needs float32 operands)
//   bfloat16, T * H * 64 >= 2^31             sequential (the chunked kernels use 32-bit offsets
//                                            inside a sequence; the sequential one does not)
//   bfloat16, B * H >= CUs * (0.3 + 12.8 / chunks), chunks = ceil(T / 16)
//                                            the one-kernel chunked prefill (a workgroup per head
//                                            keeps enough compute units busy, and the sequence is
//                                            long enough to hide its pipeline's fill and drain)
//   bfloat16, otherwise                      the split chunked prefill (its prep kernel spreads
//                                            the chunks of few heads over the whole chip)
// The CU count comes from the current device (256 if it cannot be queried).
int auto_prefill_algo(int64_t B, int64_t T, int64_t H, int dtype);

// Token-by-token recurrence with the state resident in registers. Also the
// single-token step (T == 1), the only shape that takes a 16-bit stored state.
// Returns the launch status.
hipError_t launch_sequential(const WkvCall& c, bool decode_shape);

// Chunked (WY / UT) prefill with the intra-chunk products on MFMA, one
// workgroup per head: prep waves form the chunk records in an LDS ring that the
// head's scan waves consume (no workspace). hipErrorNotSupported outside its
// domain (bfloat16 inputs, T * H * 64 below 2^31).
hipError_t launch_chunked(const WkvCall& c);

// Chunked prefill split into a chunk-parallel prep kernel and a per-head scan
// kernel, with a record buffer cached per (device, stream).
hipError_t launch_chunked_split(const WkvCall& c);

// The split chunked prefill with its records in a static device array of
// kNoallocScratchBytes (one per device) instead of the per-stream workspace: it
// allocates nothing. hipErrorInvalidValue if one chunk of records for every head
// (plus the carried state when s_out is null) does not fit, before any launch.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t launch_chunked_split_noalloc(const WkvCall& c);
// Bytes of the static array a call with B * H == units needs at least (one chunk of
// records per head, plus the carried state when state_out is null).
size_t noalloc_scratch_need(int64_t units, bool state_out);

// The time-mix operator with its prologue (decay, normalised removal key, the
// a and b slots) and epilogue (ln_x GroupNorm) fused around the recurrence.
struct TmixParams {
  const void* r;
  const float* w_raw;
  const void* k;
  const void* v;
  const void* kk;
  const void* a_lr;
  const float* ln_w;  // may be null (weight 1)
  const float* ln_b;  // may be null (bias 0)
  const float* s_in;  // may be null (zero state)
  float* out;
  float* s_out;  // may be null
  int64_t T;
  int32_t H;
};
struct TmixCall {
  TmixParams p;
  int64_t B, H;
  int dtype;  // RWKV7_DTYPE_* of r, k, v, kk, a_lr
  hipStream_t stream;
  int algo = 0;  // RWKV7_ALGO_*: AUTO / SEQUENTIAL token by token; CHUNKED or CHUNKED_SPLIT (bfloat16, T > 1)
};
hipError_t launch_tmix(const TmixCall& c);
// The fused operator as a chunked prefill (bfloat16 inputs): the prep forms the
// decay, the unit key and the two slots, and the scan (one workgroup per head) applies
// ln_x to y as it writes out. Decays below 2^-15 are clamped, as in the chunked
// prefill of the recurrence.
hipError_t launch_tmix_chunked(const TmixCall& c);
// The same with the one-kernel chunked prefill (the prep's time-mix mode in the
// fused kernel), its scan waves applying ln_x before out is written.
hipError_t launch_tmix_fused(const TmixCall& c);

// Reverse-mode derivatives of the recurrence: a checkpointing forward pass and
// a reverse pass over the checkpoints, all gradients float32.
struct BwdCall {
  const void* in[6];     // r, w, k, v, a, b in dtype
  const float* s_in;     // may be null (zero state)
  const float* dy;
  const float* ds_out;   // may be null (zero)
  float* grad[6];        // dr, dw, dk, dv, da, db
  float* ds_in;          // may be null
  int64_t B, T, H;
  int dtype;
  hipStream_t stream;
};
hipError_t launch_backward(const BwdCall& c);
// The chunked backward on MFMA (bfloat16 inputs, T * H * 64 < 2^31; else
// hipErrorNotSupported before any launch): wkv7_bwd_chunk.hip.
hipError_t launch_backward_chunked(const BwdCall& c);

// L time-mix layers over a float32 residual stream x [B*T, H*64], in place, with
// the per-layer states [L, B, H, 64, 64] updated in place.
struct StackCall {
  const void* w_in;   // [L, D, 5D] in dtype
  const void* w_out;  // [L, D, D] in dtype
  const float* vecs;  // [L, 5, D]: w0, a0, k_k, ln_w, ln_b
  float* x;
  float* states;
  int64_t L, B, T, H;
  int dtype;
  hipStream_t stream;
};
hipError_t launch_stack(const StackCall& c);

// Device memory cached per (device, stream), shared by the launchers that need
// scratch: calls on one stream run in order, so they can share it. Grown on
// demand (at least doubling); a replaced buffer stays allocated until the process
// ends, since a HIP graph captured earlier may still use it. Growing while the
// stream is being captured returns hipErrorStreamCaptureUnsupported.
// Two independent buffers per (device, stream): the chunked kernels' records use
// their own, so a caller holding the general one (the layer stack) can run them.
constexpr int kWorkspaceGeneral = 0, kWorkspaceChunks = 1;
hipError_t device_workspace(hipStream_t stream, size_t bytes, void** out, int slot = kWorkspaceGeneral);

// state_out <- state_in (zeros when state_in is null) for B*H heads.
hipError_t launch_state_copy(const float* s_in, float* s_out, int64_t units, hipStream_t stream);

}  // namespace rwkv7
