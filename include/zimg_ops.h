/*
 * zimg_ops.h -- lower-level entry points of the S3-DiT engine: single
 * blocks on a caller-supplied residual, the row layout of the sequence
 * buffer, the bf16 projection GEMM, and the sampler's Euler update.
 * Every pointer marked DEVICE is a HIP device pointer; every call is
 * asynchronous on ``stream`` (a hipStream_t, NULL = default stream) and
 * returns ZIMG_OK or a negative code (message: zimg_last_error()).
 */
#ifndef ZIMG_OPS_H
#define ZIMG_OPS_H

#include "zimg_dit.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Row layout of the single-stream sequence buffer the engine uses for B
 * samples with n_image_tokens each and the given caption lengths ("Z-Image"
 * (AI Toolkit docs), Architecture: text and image tokens share one
 * sequence).  Image rows of sample b start at img_off[b] = b * Npad, Npad =
 * n_image_tokens rounded up to 16; caption rows of sample b start at
 * cap_off[b], after all image rows, each caption padded to a multiple of 16
 * rows.  Padding rows belong to no sample.  S_total is the row count.
 * Output arrays are HOST [B]; any output pointer may be NULL.
 */
int zimg_row_layout(int32_t B, int32_t n_image_tokens, const int32_t* caption_lens,
                    int32_t* img_off, int32_t* cap_off, int32_t* S_total);

/* The same layout for samples with their own image token counts (HOST
 * n_image_tokens [B]): sample b's image rows start at img_off[b], the sum of
 * the earlier samples' counts each rounded up to 16 (the layout of
 * zimg_dit_forward_varsize). */
int zimg_row_layout_varsize(int32_t B, const int32_t* n_image_tokens, const int32_t* caption_lens,
                            int32_t* img_off, int32_t* cap_off, int32_t* S_total);

/*
 * Run blocks [first_block, first_block + n_blocks) of the model (execution
 * order: noise refiners, context refiners, joint blocks) in place on the
 * fp32 residual x_io (DEVICE [S_total, hidden], the row layout above), with
 * the modulation of model time t (HOST [B]).  Each block touches the rows of
 * its stage only: image rows (noise refiner), caption rows (context
 * refiner) or all rows (joint).  Same argument rules as zimg_dit_forward.
 */
int zimg_dit_run_blocks(zimg_dit* h, float* x_io, int32_t B, int32_t Hl, int32_t Wl,
                        const int32_t* caption_lens, const float* t, int32_t first_block,
                        int32_t n_blocks, void* stream);

/* Projection GEMM epilogues. */
#define ZIMG_EPI_BF16 0     /* C bf16 [M, N] = A W^T */
#define ZIMG_EPI_F32_BIAS 1 /* C fp32 [M, N] = A W^T + bias[N] (bias may be NULL) */
#define ZIMG_EPI_SWIGLU 2   /* W rows interleaved in groups of 32 (32 rows of w1, then the
                               same 32 rows of w3); C bf16 [M, N/2] = SiLU(h w1^T) * (h w3^T) */

/*
 * C = epilogue(A W^T): A DEVICE bf16 [M, K] (row stride lda), W DEVICE bf16
 * [N, K] (row stride ldw; a linear layer's weight), C DEVICE with row
 * stride ldc.  Constraints: K % 64 == 0, N % 64 == 0 (N % 256 for SwiGLU),
 * lda, ldw multiples of 8 and at most 4194304 (2^22); for bf16 outputs
 * (plain and SwiGLU) ldc a
 * multiple of 8 and C 16-byte aligned.  fp32 accumulation on bf16 MFMA; no
 * scratch.
 */
int zimg_gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc,
                   int32_t M, int32_t N, int32_t K, int32_t epilogue, const float* bias,
                   void* stream);

/*
 * Int8 projection GEMM: C = epilogue(dequant(A) dequant(W)^T) with the sums
 * taken exactly in int32: C[m][n] = (float(sum_k A[m][k] W[n][k]) * sa[m]) *
 * sw[n] (each product rounded to fp32), then the epilogue as for
 * zimg_gemm_bf16 (ZIMG_EPI_BF16, ZIMG_EPI_F32_BIAS, ZIMG_EPI_SWIGLU).  The
 * int8 block projections of "Z-Image-Turbo MNN (int8, fp16-safe)",
 * Conversion details (8-bit weights), with activations quantized too.
 * A DEVICE int8 [M, K] (row stride lda), W DEVICE int8 [N, K] (row stride
 * ldw), sa DEVICE fp32 [M], sw DEVICE fp32 [N], C as for zimg_gemm_bf16.
 * Constraints: K % 128 == 0, N % 256 == 0, lda, ldw multiples of 16, A and W
 * 16-byte aligned.  ZIMG_EINVAL otherwise.
 */
int zimg_gemm_i8(const void* A, int64_t lda, const float* sa, const void* W, int64_t ldw, const float* sw, void* C,
                 int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue, const float* bias, void* stream);

/*
 * Symmetric per-row int8 quantization (the rule the int8 projections apply
 * to weights and activations): for row r with amax = max_k |x[r][k]|,
 * scale[r] = amax / 127 and inv = 127 / amax (each a correctly rounded fp32
 * division), q[r][k] = rint(x[r][k] * inv) (fp32 product, ties to even)
 * clamped to [-127, 127]; a row of zeros gets scale 0 and codes 0, a row
 * holding NaN or an infinity a NaN scale.  rotate_block 128: every 128
 * consecutive values are first replaced by their unnormalised fast
 * Walsh-Hadamard transform in fp32 (butterflies (a, b) -> (a + b, a - b) of
 * stride 1, 2, ..., 64 in that order), the rotation the int8 projections
 * apply to w2's input and weight rows (after the ConvRot int8 model of
 * "Z-Image-Turbo, repackaged for H3ddle", What was changed: the activation
 * is rotated); 0: no rotation.
 * x DEVICE [rows, K] fp32 or bf16 (x_dtype; row stride ldx, 16-byte
 * aligned), q DEVICE int8 (row stride ldq, 8-byte aligned), scale DEVICE
 * fp32 [rows].  K % 8 == 0 (% 128 with rotation), K <= 16384, ldx and ldq
 * multiples of 8.
 */
int zimg_quantize_rows(const void* x, int32_t x_dtype, int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                       int32_t rows, int32_t K, int32_t rotate_block, void* stream);

/*
 * The FlowMatch Euler schedule of the sampler, on the host in float64
 * ("Z-Image-Turbo MNN (int8, fp16-safe)", Scheduler: sigmas evenly spaced
 * from 1 to 1/N, shifted by sigma' = s sigma / (1 + (s - 1) sigma), model
 * time t = (1000 - 1000 sigma')/1000; "Local component coverage and quality
 * handoff for the zimage FastVideo port", Pinned official pipeline context:
 * N + 1 points ending at sigma' = 0, where no model call is made).
 *   sigmas  HOST double [n_steps + 1]: sigma'_0 .. sigma'_{N-1}, then 0
 *   t       HOST double [n_steps]: the model time of each step (1 = clean)
 * Step k's Euler increment is sigmas[k + 1] - sigmas[k].  Each value is
 * computed with separately rounded operations in the order written above
 * (base sigma_i = i * ((1/N - 1)/(N - 1)) + 1, the last exactly 1/N), so the
 * results are reproducible bit for bit.  ZIMG_EINVAL for n_steps outside
 * 1..2^20, a shift that is not finite and positive, or NULL arrays.
 */
int zimg_flowmatch_schedule(int32_t n_steps, double shift, double* sigmas, double* t);

/*
 * Euler update of the FlowMatch sampler: x[i] += dt * (-model_out[i]) for
 * i < n ("Z-Image-Turbo MNN (int8, fp16-safe)", Scheduler: the model output
 * is negated before the Euler step; dt = sigma'_{k+1} - sigma'_k).
 * x, model_out DEVICE fp32.
 */
int zimg_euler_step(float* x, const float* model_out, float dt, int64_t n, void* stream);

/*
 * Guided Euler update with classifier-free guidance, one fused pass:
 * x[i] += dt * -(out_cond[i] + guidance * (out_cond[i] - out_uncond[i])).
 * ``guidance`` is the pipeline's scale, i.e. the user-facing scale minus
 * one ("Z-Image" (AI Toolkit docs), Specifics), so 0 is the unguided step;
 * the negated output and dt as for zimg_euler_step ("Local component
 * coverage and quality handoff for the zimage FastVideo port", Pinned
 * official pipeline context: negative prompt, guidance_scale).  x, out_cond,
 * out_uncond DEVICE fp32 [n]; x may not alias the outputs.  ZIMG_EINVAL for
 * NULL pointers (n > 0), n < 0, or a non-finite dt or guidance.
 */
int zimg_cfg_euler_step(float* x, const float* out_cond, const float* out_uncond, float guidance, float dt,
                        int64_t n, void* stream);

/*
 * Per-kernel timing of forwards on a handle, for measurement: while
 * enabled, every kernel (or small group of launches) of a forward is
 * bracketed by HIP events recorded on the forward's stream, and the elapsed
 * times are accumulated per class.  zimg_dit_profile(h, 1) creates the
 * event pool once and resets the totals; zimg_dit_profile(h, 0) stops
 * recording.  zimg_dit_profile_read() waits for recorded events and writes
 * up to max_stats entries (name, launches, total milliseconds); *n_stats
 * receives the number of classes.  Classes: gemm_qkv (with QK-RMSNorm,
 * RoPE and the V transpose in its epilogue), gemm_out,
 * gemm_w13_swiglu, gemm_w2, attention, pre_norm, post_norm,
 * embed (patchify + caption norm + both embed GEMMs), final_layer,
 * conditioning (timestep MLP + the adaLN projection), quant (int8
 * projections: the row quantization of the attention output and of the
 * SwiGLU product).
 */
typedef struct zimg_kernel_stat {
  const char* name; /* static string */
  int64_t launches;
  double total_ms;
} zimg_kernel_stat;

int zimg_dit_profile(zimg_dit* h, int32_t enable);
int zimg_dit_profile_read(zimg_dit* h, zimg_kernel_stat* stats, int32_t max_stats, int32_t* n_stats);

/*
 * The block's attention on caller buffers in the engine's layout: for each
 * sample b, the queries and keys are the rows of its two ranges of the
 * sequence buffer, o = softmax(q k^T / sqrt(128)) v per head, and no row
 * attends to another sample's rows ("Z-Image" (AI Toolkit docs),
 * Architecture: full bidirectional attention over one sample's shared
 * text + image sequence, heads of 128; "Local component coverage and quality
 * handoff for the zimage FastVideo port", Transformer: SDPA with a key mask
 * per sample).  bf16 operands, fp32 online softmax.
 *   qkv   DEVICE bf16 [rows, 3 H 128]: row r holds q (H x 128), k, then v
 *         (the v part is not read), q and k already QK-normalised and rotated;
 *         16-byte aligned
 *   vT    DEVICE bf16 [H 128][S_pad]: v transposed (element [h 128 + d][r]),
 *         16-byte aligned; S_pad a multiple of 8, 64..2^22
 *   out   DEVICE bf16 [rows, H 128], 8-byte aligned; only the rows of the
 *         segments are written
 *   seg   HOST int32 [B][4]: (start, rows) of the first range, (start, rows)
 *         of the second (rows may be 0); starts multiples of 8; each range,
 *         its length rounded up to 64, must lie inside [0, S_pad).  Keys
 *         past a range's end enter its last tile with weight 0: the vT
 *         columns from the end up to the next multiple of 8 must be finite
 *         (0 * v); further columns, and the k rows of those keys, may hold
 *         anything (another sample's rows: samples never interact)
 *   workspace  DEVICE, 256-byte aligned, ws_bytes long: the work list and
 *         the partial results of pairs split along keys (caller-owned; no
 *         state survives a call).  zimg_attention_workspace_size() gives
 *         the size that allows the plan the engine would use; a smaller
 *         workspace (at least the work list) runs with fewer or no splits.
 * B in 1..64, H in 1..256.  Asynchronous on ``stream``; ZIMG_EINVAL for bad
 * arguments (nothing is enqueued).
 */
int zimg_attention_workspace_size(int32_t H, int32_t B, const int32_t* seg, int64_t S_pad, size_t* bytes);
int zimg_attention(const void* qkv, const void* vT, int64_t S_pad, void* out, int32_t H, int32_t B,
                   const int32_t* seg, void* workspace, size_t ws_bytes, void* stream);

/*
 * zimg_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation and arguments without the workspace.  The work list
 * and split partials live in a static device array of
 * ZIMG_ATTENTION_SCRATCH_BYTES (40 MiB) per GPU, which the library holds
 * until the process ends; no call allocates or frees anything.  A problem
 * whose work list does not fit fails with ZIMG_EINVAL; when the partials of
 * the full split plan do not fit, fewer pairs are split.  Every call on a
 * GPU shares that GPU's array and nothing in it needs to start at zero (each
 * call writes its work list and partials before reading them), so calls
 * that overlap on one GPU (other streams, other host threads) race: they
 * must be ordered, e.g. on one stream.
 */
#define ZIMG_ATTENTION_SCRATCH_BYTES ((size_t)40 << 20)
int zimg_attention_noalloc(const void* qkv, const void* vT, int64_t S_pad, void* out, int32_t H, int32_t B,
                           const int32_t* seg, void* stream);

/*
 * Attention work decomposition chosen for one stage (0: noise refiner, the
 * image rows; 1: context refiner, the caption rows; 2: joint blocks, all
 * rows) at the geometry of the most recent forward or run_blocks call on the
 * handle.  Work is one 128-query tile of one head (a "pair"); when the last
 * round of resident workgroups would be at most half full, its pairs are
 * each split into chunks of their 64-key tiles, merged afterwards.  HOST
 * out[0] = pairs, out[1] = pairs computed whole, out[2] = chunks per other
 * pair (1: none).  ZIMG_ESTATE before any call has set a geometry; ZIMG_EINVAL
 * for a bad stage or NULL pointer.  For tests and measurement.
 */
int zimg_dit_attention_plan(zimg_dit* h, int32_t stage, int32_t out[3]);

#ifdef __cplusplus
}
#endif

#endif /* ZIMG_OPS_H */
