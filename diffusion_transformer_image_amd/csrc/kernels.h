// Launch interfaces of the gfx950 kernels (host side).  Every launcher
// enqueues on the given stream and returns the launch status; argument
// validation lives in the engine / C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace zimg {

// ---------------------------------------------------------------- GEMM
enum { EPI_BF16 = 0, EPI_F32_BIAS = 1, EPI_SWIGLU = 2, EPI_UNPATCH = 3, EPI_QKV_ROPE = 4 };
// which projection a launch is (selects the kernel symbol and tile shape)
enum { ROLE_ANY = 0, ROLE_QKV = 1, ROLE_OUT = 2, ROLE_W13 = 3, ROLE_W2 = 4, ROLE_EMBED = 5, ROLE_FINAL = 6 };

struct EpiArgs {
  void* C;            // output base
  int64_t ldc;        // row stride of C in elements (bf16 / f32 / swiglu)
  const float* bias;  // [N] for F32_BIAS and UNPATCH (may be null)
  // UNPATCH geometry: GEMM row = b*npad + n for token n = i*Wp + j of
  // sample b (rows with n >= ntok are alignment padding and are skipped),
  // GEMM column = (a*patch + b)*C_ch + ch; output [B, C_ch, Hp*patch, Wp*patch]
  int ntok, npad, Hp, Wp, C_ch, patch;
  // QKV_ROPE (C = the qkv buffer, width 3*D): q and k of every head are
  // RMS-normalised over 128 (weights wq, wk) and rotated by the row's table
  // (cos_t / sin_t [rows, 64], table row = trow0 + GEMM row) in place; v is
  // written transposed to vT[head*128 + d][trow0 + GEMM row] (row stride S_pad)
  const float* wq;
  const float* wk;
  const float* cos_t;
  const float* sin_t;
  bf16_t* vT;
  int trow0, S_pad, D;
  float eps;
  // int8 operands: the int32 sum of column n of row m is scaled as
  // (float(acc) * sa[m]) * sw[n] (row scales of A, of W's rows) before any
  // epilogue
  const float* sa;
  const float* sw;
};

// Split of the last, partial wave of tiles along K (see gemm.hip): null
// ``ws`` disables it.  ``ws`` holds the fp32 partial tiles (scratch; no
// state survives a launch).
struct GemmSplit {
  float* ws;
  size_t ws_bytes;
  int max_tiles;  // split tiles the workspace may hold
  int n_cu;       // compute units
};

// A and W are bf16, or (i8 = 1) int8 codes with the row scales in ep.sa /
// ep.sw; lda, ldw, K count elements.
struct GemmArgs {
  const void* A;
  int64_t lda;
  const void* W;
  int64_t ldw;
  int M, N, K;
  int i8;
  int epi;
  EpiArgs ep;
  int role;
  GemmSplit split;
};

const char* gemm_check(const GemmArgs& g);  // null if OK
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);

// ---------------------------------------------------------------- norms
// A per-sample fp32 vector v[sample * stride + d]: a norm weight with its
// modulation folded in (weight * (1 + scale), weight * tanh(gate), or the
// final layer's 1 + scale), written once per forward by fold_mod.
struct VecRef {
  const float* v;
  int64_t stride;
};

// h[r] = bf16( N(x[r]) * w[sample(r)] ) for rows r in [r0, r1), with N the
// unit RMSNorm (kind 0) or the LayerNorm without affine (kind 1).  With hq
// set, the row is written as int8 codes hq[r] and scale hs[r] instead.
struct PreNormArgs {
  const float* x;
  VecRef w;
  const int32_t* row_sample;
  bf16_t* h;
  int r0, r1, D;
  float eps;
  int kind;
  int8_t* hq;
  float* hs;
};
hipError_t launch_pre_norm(const PreNormArgs& a, hipStream_t s);

// For rows r in [r0, r1):  x[r] += RMSNorm_unit(y[r]) * wg[sample(r)]  (wg =
// post-norm weight * gate); then, for rows in [n0, n1),
// h[r] = bf16(N_next(x[r]) * wn[sample(r)]).
struct PostNormArgs {
  float* x;
  const bf16_t* y;
  VecRef wg;
  int r0, r1;
  int n0, n1;  // n0 >= n1: no next norm
  VecRef wn;
  int next_kind;  // 0 RMSNorm, 1 LayerNorm (no affine)
  float next_eps;
  const int32_t* row_sample;
  bf16_t* h;
  int D;
  float eps;
  int8_t* hq;  // as for PreNormArgs
  float* hs;
};
hipError_t launch_post_norm(const PostNormArgs& a, hipStream_t s);

// fold[b][slot][d] for slot = 4*block + chunk (chunks: attention pre-norm,
// attention post-norm, FFN pre-norm, FFN post-norm) and the final slot
// 4*n_blocks:  normw[slot][d] * (1 + s) for chunks 0 and 2, normw[slot][d] *
// tanh(g) for 1 and 3 (s, g = the block's adaLN output; unmodulated blocks,
// mod_idx < 0, take normw alone), and 1 + s_final for the final slot.
hipError_t launch_fold_mod(const float* mod, int64_t mod_stride, const float* normw, const int32_t* mod_idx,
                           int n_blocks, int n_mod, int D, int B, float* fold, hipStream_t s);

// Rows of width K (K % 8 == 0, K <= 16384) of bf16 or fp32 values, row
// stride ldx -> int8 codes (row stride ldq) and one scale per row, times
// post_scale (a power of two).  rotate: each 128 values of a row first go
// through the unnormalised fast Walsh-Hadamard transform (K % 128 == 0).
hipError_t launch_quant_rows(const void* x, int x_bf16, int64_t ldx, int8_t* q, int64_t ldq, float* scale, int rows,
                             int K, int rotate, float post_scale, hipStream_t s);

// Caption features (fp32 or bf16 rows of width Dc) -> bf16 RMSNorm(x; w).
hipError_t launch_rows_rmsnorm(const void* x, int x_bf16, const float* w, bf16_t* out,
                               int rows, int Dc, float eps, hipStream_t s);


// ---------------------------------------------------------------- attention
struct AttnSeg {
  int r0[2];
  int n[2];
};
struct AttnItem {
  int q0;
  int nq;
  int seg;
  int pad;
};
// Work units: the first n_full (item, head) pairs in logical order run whole;
// each remaining pair is split into ``split`` chunks of its key tiles, whose
// unnormalised outputs and (max, sum) go to ``part`` and are merged by a
// second kernel in chunk order (deterministic).
struct AttnArgs {
  const bf16_t* qkv;
  const bf16_t* vT;
  bf16_t* out;
  const AttnItem* items;
  const AttnSeg* segs;
  int n_items, H, S_pad;
  int rows;  // rows of qkv (key rows at or past it are never read)
  float scale_log2;
  int n_full;   // pairs computed whole (== n_items * H when nothing is split)
  int split;    // chunks per remaining pair (1: none)
  float* part;  // [units][128 q][128 d] fp32, then [units][128 q] (m, l)
};
// fp32 words of partial state one split unit needs
constexpr int ATTN_PART_FLOATS = 128 * 128 + 2 * 128;
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// Work list of the attention op on caller buffers, written on the device:
// segs[b] = seg[b], and sample b's q-tiles of 128 rows (its first range's,
// then its second's) at items[item_off[b] ...].  One workgroup per sample.
constexpr int ATTN_OP_MAX_B = 64;
struct AttnPlanArgs {
  int B;
  AttnSeg seg[ATTN_OP_MAX_B];
  int item_off[ATTN_OP_MAX_B + 1];
  AttnSeg* segs;
  AttnItem* items;
};
hipError_t launch_attention_plan(const AttnPlanArgs& p, hipStream_t s);

// The device scratch of the no-allocation attention entry point: a
// file-scope array of ATTN_SCRATCH_BYTES per GPU, its address looked up once
// per device (with that device current) and kept.  Returns null and sets
// *err on failure.
constexpr size_t ATTN_SCRATCH_BYTES = (size_t)40 << 20;
void* attention_scratch(int device, hipError_t* err);

// ---------------------------------------------------------------- small ops
// latent fp32 [B, C, Hp*p, Wp*p] -> tokens bf16, row b*npad + i*Wp + j, width p*p*C
hipError_t launch_patchify(const float* latent, bf16_t* out, int B, int C, int Hp, int Wp,
                           int patch, int npad, hipStream_t s);
// e[b] = [cos(t_scale t_b f_i), sin(t_scale t_b f_i)], f_i = max_period^(-i/half)
struct TimeArgs {
  float t[64];
};
hipError_t launch_timestep_embed(const TimeArgs& t, int B, int dim, float t_scale,
                                 float max_period, float* out, hipStream_t s);
// y[b][n] = W[n] . act(x[b]) + bias[n]; act 0 = identity, 1 = SiLU.  K % 256 == 0.
hipError_t launch_gemv(const bf16_t* W, const float* bias, const float* x, int64_t ldx,
                       float* y, int64_t ldy, int N, int K, int B, int act, hipStream_t s);
// x[i] += dt * (-o[i])
hipError_t launch_euler(float* x, const float* o, float dt, int64_t n, hipStream_t s);
// x += dt * -(oc + g (oc - ou)), n elements
hipError_t launch_cfg_euler(float* x, const float* oc, const float* ou, float g, float dt, int64_t n,
                            hipStream_t s);
// fill n floats with v
hipError_t launch_fill(float* p, float v, int64_t n, hipStream_t s);
// rows [r0, r0 + n) of x (row length and stride D) = v[0 .. D)
hipError_t launch_set_rows(float* x, int D, const float* v, int r0, int n, hipStream_t s);
// non-finite scan: *first_bad = min(*first_bad, tag) if x[0, n) holds a NaN or
// an infinity; set_int writes one int
hipError_t launch_scan_finite(const float* x, int64_t n, int tag, int* first_bad, hipStream_t s);
hipError_t launch_set_int(int* p, int v, hipStream_t s);

}  // namespace zimg
