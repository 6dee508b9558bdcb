/*
 * rwkv7_wkv.h -- C ABI of the MI355X (gfx950) RWKV-7 WKV time-mix library.
 *
 * The operation (per batch b and head h; the state S is N x N float32, row i =
 * value index, column j = key index):
 *
 *     S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T
 *     y_t = S_t r_t                      (read out after the update)
 *
 * Source: RWKV-7 G0 7.2B notes (lshu.cn/news/198401), section 7.1, "x070
 * architecture, the two core operators": the state is decayed by w, receives the
 * state*a*b transition term and the v k^T outer product, and is then read out
 * with r; an RWKV-7 layer passes a = -kk (the normalised removal key) and
 * b = kk * a_lr (kk scaled by the in-context learning rate). The library
 * computes the formula for any a and b. The head size is fixed at 64 (same page,
 * sections 3.2 and 3.4: the kernels are built for head size 64 only), and the
 * state is float32 because w can be very close to 1 (RWKV-LM README,
 * oa0.com/c/1004164, MiniPile-training section, note on keeping the state and w
 * in fp32).
 *
 * Layout (all row-major, contiguous, device memory):
 *   r, w, k, v, a, b : [B, T, H, N]   dtype given by `dtype` (all six alike)
 *   y                : [B, T, H, N]   float32
 *   state_in/out     : [B, H, N, N]   float32, element (i, j) = S_ij
 * w is the decay multiplier itself (typically exp(-exp(.)) in (0, 1]), not its log.
 *
 * Ownership: every pointer is caller-owned device memory (e.g. torch tensors).
 * The library never keeps, frees or reallocates them. Calls are asynchronous on
 * `stream` (a hipStream_t; NULL = the null stream): buffers must stay alive until
 * the caller synchronises that stream. Device faults surface at that sync.
 *
 * Nulls and aliasing:
 *   state_in  == NULL : start from a zero state (a fresh sequence; same page,
 *                        section 3.3: the per-layer state starts at zero).
 *   state_out == NULL : the final state is not written.
 *   state_out == state_in (exactly) is allowed: the state is updated in place,
 *   which is how a sequence is resumed (RWKV-LM README, "RWKV introduction":
 *   passing the returned state back continues the sequence).
 *   Any other overlap between y / state_out and any input, or between y and
 *   state_out, is RWKV7_ERR_ALIAS.
 *   A pointer to a zero-element tensor may be NULL (e.g. y when T == 0).
 * Alignment: every non-NULL pointer must be 16-byte aligned (RWKV7_ERR_ALIGN).
 * Empty work: B == 0 or H == 0 does nothing; T == 0 (prefill only) copies
 * state_in to state_out (zeros when state_in is NULL) and writes no y.
 *
 * Errors: every entry point returns RWKV7_OK or a negative code, never throws,
 * prints or aborts, and validates every argument before its first HIP call.
 * Entry points are thread-safe; concurrent calls on different streams are
 * independent.
 */
#ifndef RWKV7_WKV_H
#define RWKV7_WKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define RWKV7_OK 0
#define RWKV7_ERR_NULL (-1)      /* a required pointer is NULL */
#define RWKV7_ERR_SHAPE (-2)     /* B, T or H negative; step called with T != 1; sizes overflow */
#define RWKV7_ERR_HEAD_SIZE (-3) /* N != 64 */
#define RWKV7_ERR_DTYPE (-4)     /* dtype not one of RWKV7_DTYPE_*, or state dtype not one of RWKV7_STATE_* */
#define RWKV7_ERR_ALIGN (-5)     /* a pointer is not 16-byte aligned */
#define RWKV7_ERR_ALIAS (-6)     /* outputs overlap inputs or each other (other than state_out == state_in) */
#define RWKV7_ERR_ALGO (-7)      /* unknown algorithm, or one that does not support the arguments */
#define RWKV7_ERR_HIP (-8)       /* a HIP runtime call or kernel launch failed */
#define RWKV7_ERR_SCRATCH (-9)   /* rwkv7_wkv_prefill_noalloc: the call does not fit its static scratch array */

/* Input dtype of r, w, k, v, a, b. y is always float32; so is the state except in rwkv7_wkv_step_q. */
#define RWKV7_DTYPE_F32 0
#define RWKV7_DTYPE_BF16 1

/* Stored-state element format (rwkv7_wkv_step_q). The other entry points use float32. */
#define RWKV7_STATE_F32 0
#define RWKV7_STATE_BF16 1
#define RWKV7_STATE_F16 2

/* Prefill algorithm (rwkv7_wkv_prefill_ex). */
#define RWKV7_ALGO_AUTO 0       /* library's choice (what rwkv7_wkv_prefill does) */
#define RWKV7_ALGO_SEQUENTIAL 1 /* token-by-token recurrence, state resident in registers */
#define RWKV7_ALGO_CHUNKED 2    /* chunked (WY / UT) form, one workgroup per head doing every stage
                                   (chunk records pass from its prep waves to its scan waves in LDS) */
#define RWKV7_ALGO_CHUNKED_SPLIT 3 /* chunked form split into a chunk-parallel prep kernel and a
                                      per-head scan kernel (uses a cached device workspace) */

#define RWKV7_HEAD_SIZE 64

/*
 * Whole-sequence prefill ("GPT mode"; RWKV-7 G0 7.2B notes, section 3.2: one
 * parallel pass over the prompt, producing the same state as running the tokens
 * one by one). Runs T tokens for every (b, h) unit, writes y for every token and
 * the state after token T-1.
 *
 *   r, w, k, v, a, b  inputs [B,T,H,N], dtype `dtype`
 *   state_in          [B,H,N,N] float32 initial state, or NULL for zeros
 *   y                 [B,T,H,N] float32 output
 *   state_out         [B,H,N,N] float32 final state, or NULL; may equal state_in
 *   B, T, H           batch, tokens, heads (>= 0)
 *   N                 head size; must be 64
 *   dtype             RWKV7_DTYPE_F32 or RWKV7_DTYPE_BF16
 *   stream            hipStream_t to launch on (NULL = null stream)
 *
 * Algorithm (what RWKV7_ALGO_AUTO picks; rwkv7_wkv_prefill_algo reports it):
 *   float32 inputs                      RWKV7_ALGO_SEQUENTIAL (float32 throughout);
 *   bfloat16, T * H * 64 >= 2^31        RWKV7_ALGO_SEQUENTIAL (outside the chunked domain);
 *   bfloat16, B * H >= CUs * (0.3 + 12.8 / ceil(T / 16)), with CUs the current
 *     device's compute units            RWKV7_ALGO_CHUNKED (one workgroup per head;
 *                                       on 256 CUs: 96 heads from about 2,700 tokens,
 *                                       128 heads from 1,024, 256 heads from about 290);
 *   bfloat16, otherwise                 RWKV7_ALGO_CHUNKED_SPLIT (prep spread over the chip).
 * The chunked algorithms carry the state in float32 but round intra-chunk
 * operands, the state operand of a chunk's products included, to float16: the
 * domain described under rwkv7_wkv_prefill_ex applies (magnitudes below 2^15,
 * decays below 2^-15 treated as 2^-15), and results agree with the float32
 * recurrence to about 1e-3 relative. Callers outside that domain use
 * rwkv7_wkv_prefill_ex with RWKV7_ALGO_SEQUENTIAL.
 */
int rwkv7_wkv_prefill(const void *r, const void *w, const void *k, const void *v, const void *a,
                      const void *b, const float *state_in, float *y, float *state_out, int64_t B,
                      int64_t T, int64_t H, int64_t N, int dtype, void *stream);

/*
 * Batched single-token step ("RNN mode"; RWKV-7 G0 7.2B notes, sections 3.2
 * and 7.1: the single-step kernel applies the same formula to one token with the
 * state carried in and out). Same arguments and layouts as rwkv7_wkv_prefill
 * with T == 1 (else RWKV7_ERR_SHAPE). Typical use updates the state in place
 * (state_out == state_in). The result is bit-identical to the sequential
 * prefill run over the same tokens one call at a time.
 */
int rwkv7_wkv_step(const void *r, const void *w, const void *k, const void *v, const void *a,
                   const void *b, const float *state_in, float *y, float *state_out, int64_t B,
                   int64_t T, int64_t H, int64_t N, int dtype, void *stream);

/*
 * Single-token step with the state stored in a 16-bit format (reduced-precision
 * decode state). The RWKV-8 ROSA note (trdm.cn/news/547794, "why states are
 * worth quantising") writes the state size as a function of batch, heads, head
 * size, layers and Q, the bits per state element, and names lowering Q as the
 * direct way to raise the batch that fits; Q = 16 halves the state bytes that
 * this HBM-bound step reads and writes.
 *
 *   state_in   [B,H,N,N] in `state_dtype`, or NULL for zeros; widened exactly
 *   state_out  [B,H,N,N] in `state_dtype`, or NULL; may equal state_in
 *   state_dtype RWKV7_STATE_F32 (then identical to rwkv7_wkv_step),
 *              RWKV7_STATE_BF16 or RWKV7_STATE_F16
 *   all other arguments as for rwkv7_wkv_step (T == 1, inputs in `dtype`,
 *   y float32).
 *
 * The token is computed in float32 exactly as rwkv7_wkv_step does; y is read
 * from that float32 state, and the new state is rounded to nearest-even when
 * it is stored (float16: magnitudes must stay below 65504, and values below
 * 2^-14 keep fewer bits). The README's fp32 note (oa0.com/c/1004164: the state
 * update must be float32 because w can be very close to 1) is why float32
 * stays the default: with a 16-bit stored state, a decay that changes an
 * element by less than half a unit in its last place is lost at each store,
 * so the state drifts from the float32 trajectory over many steps. Callers
 * choose the trade-off.
 */
int rwkv7_wkv_step_q(const void *r, const void *w, const void *k, const void *v, const void *a,
                     const void *b, const void *state_in, float *y, void *state_out, int64_t B,
                     int64_t T, int64_t H, int64_t N, int dtype, int state_dtype, void *stream);

/*
 * Prefill with an explicit algorithm (RWKV7_ALGO_*), so a caller or a test can
 * force one kernel. Other arguments as for rwkv7_wkv_prefill.
 *
 * Domain of RWKV7_ALGO_CHUNKED and RWKV7_ALGO_CHUNKED_SPLIT (the sequential
 * algorithm has none beyond finite inputs):
 *   - bfloat16 inputs only (dtype RWKV7_DTYPE_BF16); float32 inputs return
 *     RWKV7_ERR_ALGO (their 1e-5 accuracy needs the sequential algorithm);
 *   - 0 <= w <= 1; any w below 2^-15 is treated as 2^-15, which changes a
 *     decayed term by at most 2^-15 of its size;
 *   - the decay-scaled inputs, the state and the intermediate chunk products
 *     are rounded to float16 as matrix-core operands, so their magnitudes must
 *     stay below 2^15 (RWKV-7 activations and states are far smaller);
 *   - T * H * 64 must be below 2^31 (32-bit in-sequence offsets);
 *     otherwise the call returns RWKV7_ERR_ALGO and launches nothing.
 * Results agree with the sequential algorithm to about 1e-3 relative (max-norm
 * over a tensor) rather than bit for bit.
 *
 * RWKV7_ALGO_CHUNKED uses no workspace: its chunk records stay in the
 * compute unit's LDS.
 *
 * Workspace of RWKV7_ALGO_CHUNKED_SPLIT (also the automatic choice for
 * bfloat16 inputs with few heads): the chunk records that pass from its first
 * kernel to its second live in a device buffer that the library allocates on
 * the first call that needs it and keeps for later calls, one buffer per
 * (device, stream), grown when a call needs more (at most about 256 MiB plus
 * one state copy: a longer sequence is processed in slabs of chunks that fit;
 * the environment variable RWKV7_SPLIT_SLAB_MB overrides the budget). A buffer
 * that growth replaces stays allocated until the process ends, because a HIP
 * graph captured earlier on that stream may still use it; growth at least
 * doubles the buffer, so that retired memory is bounded by the live buffer's
 * size. An allocation failure returns RWKV7_ERR_HIP before any launch, and so
 * does a call that would grow the buffer while its stream is being captured.
 */
int rwkv7_wkv_prefill_ex(const void *r, const void *w, const void *k, const void *v, const void *a,
                         const void *b, const float *state_in, float *y, float *state_out, int64_t B,
                         int64_t T, int64_t H, int64_t N, int dtype, int algo, void *stream);

/*
 * The time-mix operator with its prologue and epilogue fused around the
 * recurrence (RWKV-7 G0 7.2B notes, section 7.1, "x070 architecture, the two
 * core operators": the decay is exp(-exp(w)) of a soft-clamped w; the removal
 * key kk is L2-normalised per head with F.normalize; the kernel slots are
 * a = -kk and b = kk * a_lr, a_lr being the in-context learning rate; the
 * output goes through ln_x, a GroupNorm whose eps is 64e-5). Per (b, t, h):
 *
 *     w      = exp(-exp(w_raw))                    (float32)
 *     kk_hat = kk / max(|kk|_2, 1e-12)             (over the head's 64 channels)
 *     a      = -kk_hat,  b = kk_hat * a_lr
 *     S_t    = S_{t-1} (diag(w) + a b^T) + v k^T,  y = S_t r
 *     out    = (y - mean(y)) / sqrt(var(y) + 64e-5) * ln_w + ln_b
 *              (mean and population variance over the head's 64 channels;
 *               ln_w and ln_b are per channel, [H * 64])
 *
 * This saves the passes that would otherwise compute w, a and b into HBM
 * before the recurrence and normalise y after it.
 *
 *   r, k, v, kk, a_lr  [B,T,H,N] in `dtype` (RWKV7_DTYPE_F32 or _BF16)
 *   w_raw              [B,T,H,N] float32 (kept float32 for every dtype: decays
 *                      close to 1 need it, RWKV-LM README, fp32 note)
 *   ln_w, ln_b         [H*N] float32, or NULL for weight 1 / bias 0
 *   state_in           [B,H,N,N] float32, or NULL for zeros
 *   out                [B,T,H,N] float32, the normalised output
 *   state_out          [B,H,N,N] float32, or NULL; may equal state_in
 *   B, T, H, N         as for rwkv7_wkv_prefill (N must be 64)
 *
 * Layouts, ownership, alignment, aliasing and error codes are as for
 * rwkv7_wkv_prefill (every pointer 16-byte aligned; out and state_out may not
 * overlap any input; T == 0 copies the state). One workgroup per head runs the
 * token-by-token recurrence with float32 state; results match the float64
 * definition above to float32 rounding (bfloat16 inputs are widened exactly).
 */
int rwkv7_tmix_prefill(const void *r, const float *w_raw, const void *k, const void *v, const void *kk,
                       const void *a_lr, const float *ln_w, const float *ln_b, const float *state_in, float *out,
                       float *state_out, int64_t B, int64_t T, int64_t H, int64_t N, int dtype, void *stream);

/*
 * rwkv7_tmix_prefill with a choice of algorithm:
 *   RWKV7_ALGO_AUTO, RWKV7_ALGO_SEQUENTIAL  the token-by-token kernel (what
 *                      rwkv7_tmix_prefill runs; bit-identical to T single steps)
 *   RWKV7_ALGO_CHUNKED  bfloat16 inputs only: the one-kernel chunked prefill of
 *                      rwkv7_wkv_prefill_ex (one workgroup per head, no workspace),
 *                      with the decay exp(-exp(w_raw)), the unit key and the two
 *                      slots formed in its prep waves, and ln_x applied by its scan
 *                      waves before out is written (no second pass over out). Its
 *                      domain is that of the chunked prefill (T*H*64 < 2^31).
 *   RWKV7_ALGO_CHUNKED_SPLIT  bfloat16 inputs only: the same prologue in the split
 *                      prefill (prep and scan kernels, the cached device workspace;
 *                      one scan workgroup per head, so that ln_x is applied as out is
 *                      written).
 * Both chunked forms clamp decays below 2^-15 (as the chunked prefill does) and
 * match the definition to the chunked tolerance, not bit for bit with the steps.
 * Any other algo, a chunked algo with float32 inputs, or CHUNKED outside its
 * domain: RWKV7_ERR_ALGO.
 */
int rwkv7_tmix_prefill_ex(const void *r, const float *w_raw, const void *k, const void *v, const void *kk,
                          const void *a_lr, const float *ln_w, const float *ln_b, const float *state_in, float *out,
                          float *state_out, int64_t B, int64_t T, int64_t H, int64_t N, int dtype, int algo,
                          void *stream);

/*
 * Single-token step of the fused time-mix operator (RNN mode, G0 notes section
 * 3.2): rwkv7_tmix_prefill with T == 1 (else RWKV7_ERR_SHAPE). T consecutive
 * steps give the same bits as one rwkv7_tmix_prefill over the T tokens.
 */
int rwkv7_tmix_step(const void *r, const float *w_raw, const void *k, const void *v, const void *kk,
                    const void *a_lr, const float *ln_w, const float *ln_b, const float *state_in, float *out,
                    float *state_out, int64_t B, int64_t T, int64_t H, int64_t N, int dtype, void *stream);

/*
 * Gradients of the recurrence (training). The model is trained with the same
 * wkv7 operator (RWKV-7 G0 7.2B notes, section 7.2, the training scripts), which
 * needs its derivatives; the pages give only the forward formula (section 7.1),
 * so these are its reverse-mode derivatives. Given dy = dL/dy and
 * dstate_out = dL/dS_T, with G = dL/dS_t accumulated from the last token back:
 *
 *     G += dy_t r_t^T
 *     dr_t = S_t^T dy_t          dk_t = G^T v_t          dv_t = G k_t
 *     dw_t[j] = sum_i S_{t-1}[i,j] G[i,j]
 *     da_t = S_{t-1}^T (G b_t)   db_t = G^T (S_{t-1} a_t)
 *     G <- G diag(w_t) + (G b_t) a_t^T          and finally dstate_in = G.
 *
 *   r, w, k, v, a, b  [B,T,H,N] in `dtype` (the forward call's inputs)
 *   state_in          [B,H,N,N] float32, or NULL (zeros): the forward's S_0
 *   dy                [B,T,H,N] float32
 *   dstate_out        [B,H,N,N] float32, or NULL (zero: the final state unused)
 *   dr..db            [B,T,H,N] float32 outputs, all six required
 *   dstate_in         [B,H,N,N] float32 output, or NULL; may equal dstate_out
 *
 * Every pointer 16-byte aligned; outputs may not overlap any input or each
 * other (dstate_in == dstate_out exactly is allowed); T == 0 copies dstate_out
 * to dstate_in (zeros when NULL). The algorithm is RWKV7_ALGO_AUTO of
 * rwkv7_wkv_backward_ex below: the chunked backward for bfloat16 inputs (results
 * to the bfloat16 bar, in its decay domain), the token-by-token one otherwise.
 * The token-by-token backward recomputes the forward pass inside: a first kernel
 * stores the float32 state every 8 tokens, a second walks the sequence backwards,
 * rebuilding each 8-token stretch of states from its checkpoint; arithmetic is
 * float32 throughout (bfloat16 inputs widened exactly) and results match the
 * float64 derivatives to float32 rounding. Either algorithm keeps its stored
 * states in the per-(device, stream) workspace described for
 * rwkv7_wkv_prefill_ex, grown as needed (an allocation failure, or growth during
 * graph capture, returns RWKV7_ERR_HIP before any launch).
 */
int rwkv7_wkv_backward(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
                       const float *state_in, const float *dy, const float *dstate_out, float *dr, float *dw,
                       float *dk, float *dv, float *da, float *db, float *dstate_in, int64_t B, int64_t T,
                       int64_t H, int64_t N, int dtype, void *stream);

/*
 * rwkv7_wkv_backward with a choice of algorithm (rwkv7_wkv_backward runs
 * RWKV7_ALGO_AUTO):
 *   RWKV7_ALGO_SEQUENTIAL  the checkpointed token-by-token reverse pass above, float32
 *                      throughout, any dtype (AUTO for float32 inputs and for bfloat16
 *                      with T*H*64 >= 2^31).
 *   RWKV7_ALGO_CHUNKED  bfloat16 inputs with T*H*64 < 2^31 (else RWKV7_ERR_ALGO); AUTO for
 *                      them. The derivatives of the chunked prefill's chunk form, on
 *                      16x16 MFMA tiles: a checkpoint pass of the one-kernel chunked
 *                      prefill stores the float16 state at the start of every even
 *                      16-token chunk; a second kernel carries dL/dS back through the
 *                      chunks (one workgroup per head) and stores it, in float16, at the
 *                      end of every odd chunk and of the last one; a third forms each
 *                      chunk's input gradients (one wave per chunk and head, the two waves
 *                      of a chunk pair rebuilding the missing state and gradient for each
 *                      other). Both stored arrays (B*H*ceil(ceil(T/16)/2) * 8 KiB each)
 *                      live in the per-(device, stream) workspace of
 *                      rwkv7_wkv_prefill_ex. Intra-chunk
 *                      operands are float16 and the state gradient is carried in float32,
 *                      so results agree with the float64 derivatives to about 1e-3
 *                      relative (the bfloat16 bar). Domain: that of the chunked prefill
 *                      (decays below 2^-15 are clamped, and the gradient is that of the
 *                      clamped function) and, since the key-scaled inputs of a chunk enter
 *                      float16 products, every product of eight consecutive decays above
 *                      2^-15 (every decay above 0.28; the model's soft clamp keeps decays
 *                      above exp(-exp(-0.5)) = 0.545). Outside it, use RWKV7_ALGO_SEQUENTIAL.
 * Any other algo: RWKV7_ERR_ALGO.
 */
int rwkv7_wkv_backward_ex(const void *r, const void *w, const void *k, const void *v, const void *a,
                          const void *b, const float *state_in, const float *dy, const float *dstate_out, float *dr,
                          float *dw, float *dk, float *dv, float *da, float *db, float *dstate_in, int64_t B,
                          int64_t T, int64_t H, int64_t N, int dtype, int algo, void *stream);

/*
 * A stack of L time-mix layers over a residual stream: the hybrid ("fast")
 * inference mode of RWKV-7 G0 7.2B notes section 3.2, where a prompt goes
 * through every layer in one parallel call and generation then advances one
 * token at a time with a fixed-size state per layer (section 3.3). Call with the
 * prompt's T tokens, then with T == 1 per generated token; the per-layer states
 * carry everything between calls. With D = H * N and, per layer l (section 7.1
 * parameterisation: softplus soft clamp of the decay, sigmoid in-context
 * learning rate, per-channel scaled key that the operator L2-normalises, ln_x):
 *
 *     P     = x W_in[l]                          [B*T, 5D], blocks r | k | v | w | a
 *     w_raw = -softplus(-(w0 + P_w)) - 0.5       (float32)
 *     kk    = P_k * k_k,  a_lr = sigmoid(a0 + P_a)
 *     o     = rwkv7_tmix_prefill(r = P_r, w_raw, k = P_k, v = P_v, kk, a_lr,
 *                                ln_w, ln_b, states[l])   (state updated in place)
 *     x    += o W_out[l]
 *
 *   w_in    [L, D, 5D] in `dtype` (row-major: x[M, D] times w_in[l] gives [M, 5D])
 *   w_out   [L, D, D]  in `dtype`
 *   vecs    [L, 5, D]  float32: w0, a0, k_k, ln_w, ln_b of each layer
 *   x       [B, T, D]  float32, read and overwritten with the stack's output
 *   states  [L, B, H, N, N] float32, read and overwritten (zeros for a fresh sequence)
 *
 * With bfloat16 weights, x and o are rounded to bfloat16 for the projections and
 * r, k, v, kk, a_lr are bfloat16 operator inputs; projections accumulate in
 * float32. A bfloat16 call of T >= 32 tokens (a prompt) runs the operator as
 * rwkv7_tmix_prefill_ex with the chunked algorithm that RWKV7_ALGO_AUTO picks for
 * rwkv7_wkv_prefill_ex at the same B, T, H (the one-kernel or the split form;
 * sequential outside the chunked domain); other calls run it token by token. Token shift, the channel mix, the output gate and the low-rank
 * projections of the full model are not included. Every pointer is 16-byte
 * aligned; x and states may not overlap each other or the weights. B*T must be
 * below 2^31. L == 0 or an empty x does nothing. The projections run on rocBLAS
 * (one handle per device and stream); the intermediates (about 42 bytes per
 * element of x with bfloat16 weights, 56 with float32) live in the workspace
 * described for rwkv7_wkv_prefill_ex.
 *
 * HIP graphs: a call can be captured in a graph on a stream once one call of at
 * least the same size has run on that stream (it creates the workspace and the
 * rocBLAS handle, which capture cannot; a call that would have to grow the
 * workspace during capture fails with RWKV7_ERR_HIP); replays then launch the
 * same kernels on the same buffers, and remain valid after later, larger eager
 * calls have grown the workspace (the buffer a graph holds is never freed). The
 * same holds for every entry point of this header.
 */
int rwkv7_stack_forward(const void *w_in, const void *w_out, const float *vecs, float *x, float *states, int64_t L,
                        int64_t B, int64_t T, int64_t H, int64_t N, int dtype, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * rwkv7_wkv_prefill_ex with RWKV7_ALGO_CHUNKED_SPLIT, same arguments, layouts,
 * domain and results, except that the chunk records passing from the prep
 * kernel to the scan kernel live in a fixed device array of
 * RWKV7_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends. The call allocates nothing (no hipMalloc, no
 * library workspace). The array limits the size: one chunk of records
 * (9,472 bytes) for every (b, h) unit, plus B*H*16 KiB for the carried state
 * when state_out is NULL, must fit (B*H up to about 7,000 with state_out,
 * 2,500 without); a longer sequence runs in slabs of chunks that fit. A call
 * beyond that returns RWKV7_ERR_SCRATCH before any launch. bfloat16 inputs only
 * (RWKV7_ERR_ALGO otherwise, as for the split algorithm).
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (other streams, other host threads) race and give wrong
 * results; serialise them. No part of the array needs clearing between calls
 * (every record is written before it is read).
 */
#define RWKV7_NOALLOC_SCRATCH_BYTES (64LL << 20)
int rwkv7_wkv_prefill_noalloc(const void *r, const void *w, const void *k, const void *v, const void *a,
                              const void *b, const float *state_in, float *y, float *state_out, int64_t B,
                              int64_t T, int64_t H, int64_t N, int dtype, void *stream);

/*
 * The algorithm rwkv7_wkv_prefill would run for a bfloat16 or float32 prefill of
 * this shape on the current device (RWKV7_ALGO_SEQUENTIAL, RWKV7_ALGO_CHUNKED or
 * RWKV7_ALGO_CHUNKED_SPLIT; the rule is stated at rwkv7_wkv_prefill), or
 * RWKV7_ERR_DTYPE / RWKV7_ERR_SHAPE / RWKV7_ERR_HEAD_SIZE for arguments that
 * rwkv7_wkv_prefill would refuse. Launches nothing and allocates nothing; it may
 * query the current device's compute-unit count (256 is assumed if none can be
 * queried).
 */
int rwkv7_wkv_prefill_algo(int64_t B, int64_t T, int64_t H, int64_t N, int dtype);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *rwkv7_wkv_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* RWKV7_WKV_H */
