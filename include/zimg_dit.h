/*
 * zimg_dit.h -- C ABI of the Z-Image S3-DiT denoiser forward on gfx950.
 *
 * The operation: one forward of the single-stream diffusion transformer
 * (S3-DiT) of Z-Image: patch embed of a 16-channel latent, caption embed of
 * 2560-d text features, 2 noise-refiner blocks (image tokens), 2 unmodulated
 * context-refiner blocks (caption tokens), 30 joint blocks over the shared
 * [image; caption] sequence, then the final layer back to latent space.
 * Sources (page title, section):
 *   "Z-Image" (ostris AI Toolkit docs), Architecture: 30 single-stream
 *     blocks + 2 noise-refiner + 2 context-refiner, hidden 3840 (30 heads x
 *     128), SwiGLU FFN 10240, adaLN from a 256-d timestep embedding (context
 *     refiner unmodulated), RMSNorm, QK-RMSNorm, 3-axis RoPE [32, 48, 48]
 *     with theta 256, caption features of up to 512 tokens, padding dropped;
 *     Latent space: 16 channels, 2x2 patches; Specifics: model time
 *     t = (1000 - timestep)/1000 with 1 = clean, output negated by the sampler.
 *   "Z-Image-Turbo MNN (int8, fp16-safe)", Model files: unet takes
 *     sample (B,16,H/8,W/8), timestep, encoder_hidden_states (.., 2560) and
 *     returns out_sample of the sample's shape.
 *   "Local component coverage and quality handoff for the zimage FastVideo
 *     port", Component contracts (Transformer): strict loading accounts for
 *     every one of the 521 published keys.
 *
 * All functions return ZIMG_OK (0) or a negative error code; the message of
 * the most recent failure on the calling thread is returned by
 * zimg_last_error() (and, for a handle, by zimg_dit_last_error()).
 * Handles are not thread-safe: use one handle per host thread / stream.
 */
#ifndef ZIMG_DIT_H
#define ZIMG_DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ------------------------------------------------------ */
#define ZIMG_OK 0
#define ZIMG_EINVAL (-1)       /* bad argument: shape, range, null pointer, non-finite t */
#define ZIMG_EWEIGHT (-2)      /* missing, unknown, duplicate or mis-shaped weight tensor */
#define ZIMG_EUNSUPPORTED (-3) /* configuration the engine does not implement */
#define ZIMG_ENOMEM (-4)       /* device or host allocation failed */
#define ZIMG_EHIP (-5)         /* HIP runtime error (message carries hipGetErrorString) */
#define ZIMG_ESTATE (-6)       /* call out of order (e.g. forward before all weights set) */
#define ZIMG_ENONFINITE (-7)   /* check_finite: a NaN or infinity appeared (the message names
                                  the first stage: embeddings, block, or output) */

/* ---- element types ----------------------------------------------------- */
#define ZIMG_F32 0
#define ZIMG_BF16 1 /* bfloat16 bit patterns (uint16) */

/*
 * Model hyperparameters and workspace limits.  zimg_dit_default_config()
 * fills the full model of "Z-Image" (AI Toolkit docs), Architecture.
 * Readings the pages leave open (documented constants): t_mid 1024 (the
 * timestep MLP width that, with the rest, gives the published
 * 6,154,908,736 parameters), t_scale 1000, max_period 10000, norm_eps 1e-5,
 * final_eps 1e-6.
 */
typedef struct zimg_dit_config {
  int32_t hidden;            /* 3840; must equal n_heads * 128 */
  int32_t n_heads;           /* 30 */
  int32_t ffn;               /* 10240; multiple of 32 */
  int32_t n_layers;          /* 30 joint blocks */
  int32_t n_noise_refiner;   /* 2 (image tokens, modulated) */
  int32_t n_context_refiner; /* 2 (caption tokens, unmodulated) */
  int32_t in_channels;       /* 16 */
  int32_t patch;             /* 2 */
  int32_t cap_feat_dim;      /* 2560 */
  int32_t adaln_dim;         /* 256: sinusoid width and adaLN input width */
  int32_t t_mid;             /* 1024: timestep MLP hidden width */
  int32_t rope_axes[3];      /* {32, 48, 48}; sum 128, each even */
  float rope_theta;          /* 256 */
  float t_scale;             /* 1000: sinusoid argument is t_scale * t */
  float max_period;          /* 10000 */
  float norm_eps;            /* 1e-5: every RMSNorm */
  float final_eps;           /* 1e-6: final LayerNorm (no affine) */
  int32_t max_batch;         /* workspace sizing: samples per forward (1..64) */
  int32_t max_image_tokens;  /* per sample, (Hl/2)*(Wl/2) */
  int32_t max_caption_tokens;/* per sample, 1..512 */
  int32_t batch_invariant;   /* 0 (default): the last, partial round of GEMM tiles and
                                attention work is split along K / keys to fill the GPU,
                                which makes the fp32 summation order depend on the whole
                                batch; 1: no such splits, so each sample's result is
                                bitwise the same whatever else is in the batch (slower
                                when the last round is partial) */
  int32_t linear_int8;       /* 0 (default): bf16 block projections.  1: the seven
                                projections of every block (to_q, to_k, to_v, to_out, w1,
                                w2, w3) run on int8 codes with exact int32 sums: weights
                                quantized per output row at finalize (symmetric, scale =
                                max|w|/127), activations per token at run time (the same
                                rule; see zimg_quantize_rows); embedders, conditioning,
                                attention and the final layer stay as they are ("Z-Image-
                                Turbo MNN (int8, fp16-safe)", Conversion details: 8-bit
                                weights; "Z-Image" (AI Toolkit docs), Specifics: the
                                embedders and final layer are not quantized) */
  int32_t token_pad;         /* 0 (default): a sample's sequence holds exactly its image
                                and caption tokens ("Z-Image" (AI Toolkit docs),
                                Architecture: padding dropped).  32: each of the two runs
                                is padded to a multiple of 32 with the learned
                                x_pad_token / cap_pad_token, which take part in the
                                sample's attention like its other tokens; caption
                                positions continue through the pads, image positions
                                start after the padded caption, image pads sit at
                                position (0, 0, 0) ("Z-Image-Turbo, repackaged for
                                H3ddle", Measured performance: a 4,096 + 32 token
                                forward; "Local component coverage and quality handoff
                                for the zimage FastVideo port", Transformer: the padded
                                stream needs a key mask).  The row layout is then the
                                one of the padded counts (zimg_row_layout with each
                                count rounded up to 32). */
  int32_t check_finite;      /* 0 (default).  1 (a debug aid): after the embeddings,
                                after every block and on the outputs, the sequence rows
                                of every sample are scanned for NaN and infinity; the
                                forward then waits for its stream and returns
                                ZIMG_ENONFINITE naming the first stage whose values were
                                not finite.  Costs one read of the sequence per block
                                and makes the forward synchronous. */
} zimg_dit_config;

/* One named weight tensor handed to the engine.  ``data`` is a HOST
 * pointer to a dense row-major array of ``dtype`` (ZIMG_F32 or ZIMG_BF16).
 * The engine copies (and converts) it; the caller keeps ownership. */
typedef struct zimg_tensor {
  const char* name;
  const void* data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
} zimg_tensor;

typedef struct zimg_dit zimg_dit;

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* zimg_last_error(void);

/* Fill ``cfg`` with the full model and workspace limits for one 1024x1024
 * sample with a 512-token caption. */
void zimg_dit_default_config(zimg_dit_config* cfg);

/* Validate a configuration without touching the GPU.  ZIMG_EINVAL /
 * ZIMG_EUNSUPPORTED with a message when it is not usable. */
int zimg_dit_check_config(const zimg_dit_config* cfg);

/* The weight table the engine expects for ``cfg``: number of tensors, and
 * name / rank / shape of entry ``index`` (canonical order).  The name
 * pointer stays valid for the life of the process. */
int zimg_dit_manifest_size(const zimg_dit_config* cfg, int32_t* n_tensors);
int zimg_dit_manifest_entry(const zimg_dit_config* cfg, int32_t index,
                            const char** name, int32_t* ndim, int64_t shape[4]);

/*
 * Create an engine: allocate device weights (bf16 matrices, fp32 vectors)
 * and the whole forward workspace for the config's limits on the current
 * HIP device.  zimg_dit_create() takes every weight at once and fails with
 * ZIMG_EWEIGHT unless the set matches the manifest exactly (no missing,
 * unknown, duplicate or mis-shaped tensor).  The streaming variant
 * zimg_dit_alloc() + zimg_dit_set_weight() (one tensor at a time) +
 * zimg_dit_finalize() applies the same strict check at finalize.
 * ``stream`` (a hipStream_t, NULL = the default stream; owned by the caller,
 * who keeps it alive while the handle exists) carries the set-up work:
 * workspace clears, weight uploads and repacking.  Each call returns once
 * its work on that stream is done, so the caller may free its host weight
 * arrays as soon as the call returns.
 * On failure *out is NULL and everything allocated is released.
 */
int zimg_dit_create(const zimg_dit_config* cfg, const zimg_tensor* weights,
                    int32_t n_weights, void* stream, zimg_dit** out);
int zimg_dit_alloc(const zimg_dit_config* cfg, void* stream, zimg_dit** out);
int zimg_dit_set_weight(zimg_dit* h, const zimg_tensor* w);
int zimg_dit_finalize(zimg_dit* h);

/*
 * One forward, enqueued asynchronously on ``stream`` (a hipStream_t; NULL
 * is the default stream).  No allocation happens inside.
 *   latent         DEVICE fp32 [B, in_channels, Hl, Wl], row-major
 *   B              1..max_batch
 *   Hl, Wl         even (image side a multiple of 16 pixels);
 *                  (Hl/2)*(Wl/2) <= max_image_tokens
 *   caption_feats  DEVICE [sum_b L_b, cap_feat_dim], ZIMG_F32 or ZIMG_BF16
 *                  (cap_dtype), the B captions packed back to back with
 *                  their exact lengths (no padding)
 *   caption_lens   HOST int32 [B], each 1..max_caption_tokens
 *   t              HOST fp32 [B], model time in [0, 1], 1 = clean
 *                  (finite; t = (1000 - 1000 sigma')/1000 for shifted sigma')
 *   out            DEVICE fp32 [B, in_channels, Hl, Wl]: the raw model
 *                  output (the sampler negates it before its Euler step)
 * Samples never interact.  Returns ZIMG_EINVAL before enqueueing anything
 * when an argument is out of range; kernel faults surface as ZIMG_EHIP at a
 * later call or synchronisation.
 */
int zimg_dit_forward(zimg_dit* h, const float* latent, int32_t B, int32_t Hl, int32_t Wl,
                     const void* caption_feats, int32_t cap_dtype,
                     const int32_t* caption_lens, const float* t, float* out,
                     void* stream);

/*
 * One forward over a batch whose samples may differ in image size as well as
 * caption length ("Local component coverage and quality handoff for the
 * zimage FastVideo port", Transformer: parity on variable-length image/text
 * batches; the padded variable-length stream needs a key mask).  Each
 * sample's image and caption tokens form its own sequence; no token attends
 * across samples, so every sample's output equals that sample run alone.
 *   latents   HOST array [B] of DEVICE pointers, latent b fp32
 *             [in_channels, Hl[b], Wl[b]]
 *   Hl, Wl    HOST int32 [B], each even; (Hl[b]/2)*(Wl[b]/2) <= max_image_tokens
 *   outs      HOST array [B] of DEVICE pointers, output b fp32 of latent b's shape
 * Other arguments and errors as for zimg_dit_forward (which is this call for
 * B latents of one size stored back to back).
 */
int zimg_dit_forward_varsize(zimg_dit* h, const float* const* latents, int32_t B, const int32_t* Hl,
                             const int32_t* Wl, const void* caption_feats, int32_t cap_dtype,
                             const int32_t* caption_lens, const float* t, float* const* outs, void* stream);

/*
 * Weights from safetensors files ("Local component coverage and quality
 * handoff for the zimage FastVideo port", Component contracts: loading
 * accounts for every parameter and ignores nothing; "Z-Image" (AI Toolkit
 * docs), Specifics: one .safetensors file of the transformer).  ``paths``
 * (HOST, n_paths file names) together must hold exactly the tensors of the
 * config's weight table (zimg_dit_manifest_entry), each once, with the
 * table's shape, dtype F32 or BF16, and data_offsets inside the file and
 * matching the shape; "__metadata__" (string values only) is allowed.
 * Everything is validated before any tensor is uploaded: ZIMG_EWEIGHT for a
 * malformed file or a missing, unknown, duplicate or mis-shaped tensor,
 * ZIMG_EUNSUPPORTED for another dtype, ZIMG_EINVAL for a file that cannot
 * be opened.  The files are memory-mapped read-only and unmapped on return.
 *   zimg_safetensors_check: the validation alone (no GPU needed);
 *     *n_tensors (may be NULL) receives the tensor count.
 *   zimg_dit_load_safetensors: into a handle from zimg_dit_alloc (then
 *     zimg_dit_finalize); on failure the handle's weights are incomplete.
 *   zimg_dit_create_from_safetensors: alloc + load + finalize (on failure
 *     *out is NULL and nothing stays allocated).
 */
int zimg_safetensors_check(const zimg_dit_config* cfg, const char* const* paths, int32_t n_paths,
                           int32_t* n_tensors);
int zimg_dit_load_safetensors(zimg_dit* h, const char* const* paths, int32_t n_paths);
int zimg_dit_create_from_safetensors(const zimg_dit_config* cfg, const char* const* paths, int32_t n_paths,
                                     void* stream, zimg_dit** out);

/* SHA-256 of the config's weight names sorted bytewise, each followed by a
 * newline, as 64 lowercase hex digits and a NUL in ``hex`` (HOST, 65 bytes).
 * For the full model this is the sorted key digest the FastVideo handoff
 * ("Local component coverage and quality handoff for the zimage FastVideo
 * port", Component contracts, Transformer) states for the released
 * checkpoint's safetensors index. */
int zimg_dit_manifest_digest(const zimg_dit_config* cfg, char hex[65]);

/* Release all device and host memory of the handle (NULL is a no-op). */
void zimg_dit_destroy(zimg_dit* h);

/* Message of the last failure on this handle ("" if none). */
const char* zimg_dit_last_error(const zimg_dit* h);

/*
 * Test hook: after the next forwards, copy the fp32 residual stream into
 * ``dev_buf`` (DEVICE, ``bytes`` long) at these points, each as
 * [S_total, hidden] rows in the engine's row order (all image rows of the
 * batch, sample by sample, then all caption rows, sample by sample):
 *   slot 0: after the patch and caption embeds; slot 1 + i: after block i
 *   (noise refiners, context refiners, joint blocks, in execution order).
 * Requires bytes >= (n_blocks + 1) * S_total * hidden * 4 for the forward's
 * S_total, else that forward fails with ZIMG_EINVAL.  NULL disables.
 */
int zimg_dit_set_capture(zimg_dit* h, float* dev_buf, size_t bytes);

/* ---- host-side tables (no GPU needed) ---------------------------------- */

/* 3-axis integer positions of one sample: caption token k -> (k+1, 0, 0),
 * image token n = i*Wp + j -> (L+1, i, j).  cap_ids [L,3], img_ids [Hp*Wp,3]. */
int zimg_position_ids(int32_t L, int32_t Hp, int32_t Wp, int32_t* cap_ids, int32_t* img_ids);

/* RoPE tables for ``S`` rows of position ids [S,3]: cos and sin [S, 64]
 * fp32.  Pair p belongs to axis a (pairs 0..15 axis 0, 16..39 axis 1,
 * 40..63 axis 2 for axes {32,48,48}); with r its index inside the axis,
 * omega = theta^(-(2r)/d_a) and phi = pos_a * omega in double precision;
 * cos(phi), sin(phi) are taken in double and rounded to nearest float. */
int zimg_rope_tables(const zimg_dit_config* cfg, const int32_t* ids, int64_t S,
                     float* cos_out, float* sin_out);

#ifdef __cplusplus
}
#endif

#endif /* ZIMG_DIT_H */
