// HBM-bound row kernels of the S3-DiT block: the adaLN-modulated pre-norm,
// the fused post-norm + tanh gate + residual (+ the next pre-norm), the
// caption RMSNorm, patchify.  (QK-RMSNorm + RoPE is fused into the QKV
// projection's epilogue.)
//
// Block structure ("Z-Image" (AI Toolkit docs), Architecture: RMSNorm,
// adaLN from the timestep embedding; "Z-Image-Turbo MNN (int8,
// fp16-safe)", Conversion details: the to_out and w2 outputs feed an
// RMSNorm).  Residual rows are fp32 and every reduction is fp32; activations
// handed to the GEMMs are bf16, or, for int8 projections, int8 codes with a
// per-row scale (also the row quantizer for bf16 activations and weights).
//
// One 64-lane wave owns one row of the residual: lane l holds float4 number
// l + 64 i of the row, so loads and stores are fully coalesced and the row
// statistics need only in-wave reductions.
#include "common.h"
#include "kernels.h"

namespace zimg {
namespace {

constexpr int MAXV = 16;  // float4 per lane: hidden size up to 4096

ZI_DEV float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

ZI_DEV void store_bf16x4(bf16_t* p, float a, float b, float c, float d) {
  u32x2 u = {pack2bf(a, b), pack2bf(c, d)};
  *reinterpret_cast<u32x2*>(p) = u;
}

// Row kernels are instantiated per NV, the float4 count per lane (hidden /
// 256): NV = 15 (hidden 3840) has compile-time trip counts, so its arrays hold
// exactly the row; NV = 0 is the generic instance (runtime count nv <= MAXV).
// Q8 selects int8 output (codes and a row scale) instead of bf16 at compile
// time, so the bf16 instance carries none of the int8 path's registers.
template <int NV>
ZI_DEV constexpr int row_cap() { return NV ? NV : MAXV; }

// normalise the row held in v[] (nv float4 per lane), scale by the folded
// vector w and write it: bf16 to h, or, with Q8, int8 codes to hq and the
// row's scale to *hs (per-row symmetric quantization of the fp32 values)
template <int NV, bool Q8>
ZI_DEV void norm_write(const float4* v, int nv, int lane, int D, int kind, float eps, const float* w, bf16_t* h,
                       int8_t* hq, float* hs) {
  constexpr int CAP = row_cap<NV>();
  float mean = 0.f;
  if (kind == 1) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < CAP; ++i)
      if (NV || i < nv) s += v[i].x + v[i].y + v[i].z + v[i].w;
    mean = wave_sum(s) / (float)D;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CAP; ++i)
    if (NV || i < nv) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      ss += a * a + b * b + c * c + d * d;
    }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)D + eps);
  if constexpr (Q8) {
    float4 o[CAP];
    float am = 0.f, nanck = 0.f;  // nanck: 0, or NaN if any value is NaN or infinite
#pragma unroll
    for (int i = 0; i < CAP; ++i)
      if (NV || i < nv) {
        const float4 ww = ld4(w + (lane + 64 * i) * 4);
        o[i] = make_float4((v[i].x - mean) * inv * ww.x, (v[i].y - mean) * inv * ww.y, (v[i].z - mean) * inv * ww.z,
                           (v[i].w - mean) * inv * ww.w);
        am = fmaxf(am, fmaxf(fmaxf(fabsf(o[i].x), fabsf(o[i].y)), fmaxf(fabsf(o[i].z), fabsf(o[i].w))));
        nanck += (o[i].x + o[i].y + o[i].z + o[i].w) * 0.f;
      }
    float sc, qi;
    quant_params(wave_max(am) + wave_sum(nanck), sc, qi);
#pragma unroll
    for (int i = 0; i < CAP; ++i)
      if (NV || i < nv) *reinterpret_cast<uint32_t*>(hq + (lane + 64 * i) * 4) = quant4(o[i].x, o[i].y, o[i].z, o[i].w, qi);
    if (lane == 0) *hs = sc;
  } else {
#pragma unroll
    for (int i = 0; i < CAP; ++i)
      if (NV || i < nv) {
        const int d = (lane + 64 * i) * 4;
        const float4 ww = ld4(w + d);
        store_bf16x4(h + d, (v[i].x - mean) * inv * ww.x, (v[i].y - mean) * inv * ww.y, (v[i].z - mean) * inv * ww.z,
                     (v[i].w - mean) * inv * ww.w);
      }
  }
}

template <bool Q8>
__global__ __launch_bounds__(256) void pre_norm_kernel(PreNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = a.r0 + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.r1) return;
  const int nv = a.D >> 8;
  const float* xr = a.x + (int64_t)r * a.D;
  float4 v[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i < nv) v[i] = ld4(xr + (lane + 64 * i) * 4);
  norm_write<0, Q8>(v, nv, lane, a.D, a.kind, a.eps, a.w.v + a.row_sample[r] * a.w.stride, a.h + (int64_t)r * a.D,
                    Q8 ? a.hq + (int64_t)r * a.D : nullptr, Q8 ? a.hs + r : nullptr);
}

// Both input rows (y bf16, x fp32) are requested before any arithmetic, so
// a wave has its whole row in flight at once.  With NV = 15 and bf16 output
// the kernel fits 128 VGPRs, four waves per SIMD (the generic instance with
// the int8 path needed 154, three waves per SIMD: 9 % slower per launch,
// 51.3 against 46.8 us at 4,608 rows).
template <int NV, bool Q8>
ZI_DEV void post_norm_row(const PostNormArgs& a) {
  constexpr int CAP = row_cap<NV>();
  const int lane = threadIdx.x & 63;
  const int r = a.r0 + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.r1) return;
  const int nv = NV ? NV : a.D >> 8;
  const int sample = a.row_sample[r];
  const bf16_t* yr = a.y + (int64_t)r * a.D;
  float* xr = a.x + (int64_t)r * a.D;
  u32x2 yu[CAP];
  float4 v[CAP];
#pragma unroll
  for (int i = 0; i < CAP; ++i)
    if (NV || i < nv) {
      yu[i] = *reinterpret_cast<const u32x2*>(yr + (lane + 64 * i) * 4);
      v[i] = ld4(xr + (lane + 64 * i) * 4);
    }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CAP; ++i)
    if (NV || i < nv) {
      const float p = __uint_as_float(yu[i].x << 16), q = __uint_as_float(yu[i].x & 0xffff0000u);
      const float s = __uint_as_float(yu[i].y << 16), t = __uint_as_float(yu[i].y & 0xffff0000u);
      ss += p * p + q * q + s * s + t * t;
    }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)a.D + a.eps);
  const float* wg = a.wg.v + sample * a.wg.stride;
#pragma unroll
  for (int i = 0; i < CAP; ++i)
    if (NV || i < nv) {
      const int d = (lane + 64 * i) * 4;
      const float4 g = ld4(wg + d);
      v[i].x += __uint_as_float(yu[i].x << 16) * inv * g.x;
      v[i].y += __uint_as_float(yu[i].x & 0xffff0000u) * inv * g.y;
      v[i].z += __uint_as_float(yu[i].y << 16) * inv * g.z;
      v[i].w += __uint_as_float(yu[i].y & 0xffff0000u) * inv * g.w;
      *reinterpret_cast<float4*>(xr + d) = v[i];
    }
  if (r >= a.n0 && r < a.n1)
    norm_write<NV, Q8>(v, nv, lane, a.D, a.next_kind, a.next_eps, a.wn.v + sample * a.wn.stride,
                       a.h + (int64_t)r * a.D, Q8 ? a.hq + (int64_t)r * a.D : nullptr, Q8 ? a.hs + r : nullptr);
}
template <int NV, bool Q8>
__global__ __launch_bounds__(256) void post_norm_kernel(PostNormArgs a) {
  post_norm_row<NV, Q8>(a);
}
// hidden 3840 with bf16 output in at most 128 VGPRs: four waves per SIMD
__global__ __launch_bounds__(256, 4) void post_norm_3840_kernel(PostNormArgs a) { post_norm_row<15, false>(a); }

__global__ void fold_mod_kernel(const float* __restrict__ mod, int64_t mod_stride, const float* __restrict__ normw,
                                const int32_t* __restrict__ mod_idx, int n_blocks, int n_mod, int D,
                                float* __restrict__ fold) {
  const int slots = 4 * n_blocks + 1;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)slots * D) return;
  const int b = blockIdx.y;
  const int slot = (int)(idx / D), d = (int)(idx - (int64_t)slot * D);
  const float* mb = mod + (int64_t)b * mod_stride;
  float v;
  if (slot < 4 * n_blocks) {
    const int bi = slot >> 2, ch = slot & 3, m = mod_idx[bi];
    const float w = normw[idx];
    if (m < 0) {
      v = w;
    } else {
      const float u = mb[(int64_t)(m * 4 + ch) * D + d];
      v = (ch & 1) ? w * tanhf(u) : w * (1.0f + u);
    }
  } else {
    v = 1.0f + mb[(int64_t)n_mod * 4 * D + d];
  }
  fold[(int64_t)b * slots * D + idx] = v;
}

// caption features: one wave per row, any width that is a multiple of 256
template <bool BF16_IN>
__global__ __launch_bounds__(256) void rows_rmsnorm_kernel(const void* x, const float* w, bf16_t* out,
                                                           int rows, int Dc, float eps) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int nv = Dc >> 8;  // float4 per lane (Dc <= 4096)
  float4 v[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i < nv) {
      const int d = (lane + 64 * i) * 4;
      if constexpr (BF16_IN) {
        const u32x2 u = *reinterpret_cast<const u32x2*>(reinterpret_cast<const bf16_t*>(x) + (int64_t)r * Dc + d);
        v[i] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
      } else {
        v[i] = ld4(reinterpret_cast<const float*>(x) + (int64_t)r * Dc + d);
      }
      ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)Dc + eps);
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i < nv) {
      const int d = (lane + 64 * i) * 4;
      const float4 ww = ld4(w + d);
      store_bf16x4(out + (int64_t)r * Dc + d, v[i].x * inv * ww.x, v[i].y * inv * ww.y,
                   v[i].z * inv * ww.z, v[i].w * inv * ww.w);
    }
}

// Per-row int8 quantization of bf16 or fp32 rows of width K (K % 8 == 0,
// K <= 8 * 256 * QMAXC): one workgroup per row holds the row in registers
// (16-byte chunks c = tid + 256 i), reduces max |v|, then writes 8 codes per
// chunk and the row's scale (times post_scale, a power of two).  Same
// arithmetic as the norm kernels' int8 output.  ROT: every 128 consecutive
// values first go through the unnormalised fast Walsh-Hadamard transform in
// fp32, butterflies (a, b) -> (a + b, a - b) of stride 1, 2, 4 (within a
// thread's 8 values) then 8, 16, 32, 64 (across the 16 lanes holding the
// block, lane stride 1, 2, 4, 8); K % 128 == 0.
constexpr int QMAXC = 8;

// one cross-lane butterfly stage (lane stride M) on all chunks a thread holds
// (slots i >= ni hold no chunk of any thread; ni is uniform)
// The lower lane of a pair keeps a + b, the upper a - b (a: the lower's
// value); both are the partner's value o plus this lane's value v times
// sg = +-1, one fma after the DPP move (v * sg is exact, so the fma rounds
// once, as o + v or o - v does).
template <int M>
ZI_DEV void rot_stage(float (&v)[QMAXC][8], int tid, int ni) {
  const float sg = (tid & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < QMAXC; ++i) {
    if (i >= ni) break;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[i][k] = fmaf(v[i][k], sg, lane_xor<M>(v[i][k]));
  }
}

template <bool BF16_IN, bool ROT>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ x, int64_t ldx,
                                                         int8_t* __restrict__ q, int64_t ldq, float* __restrict__ s,
                                                         int K, float post_scale) {
  __shared__ float red[8];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int nch = K >> 3;
  float v[QMAXC][8];
  float am = 0.f, nanck = 0.f;  // nanck: 0, or NaN if any value is NaN or infinite
#pragma unroll
  for (int i = 0; i < QMAXC; ++i) {
    const int c = tid + 256 * i;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[i][k] = 0.f;
    if (c < nch) {
      if constexpr (BF16_IN) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(x) + r * ldx + c * 8);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[i][2 * k] = __uint_as_float(u[k] << 16);
          v[i][2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
        }
      } else {
        const float* p = reinterpret_cast<const float*>(x) + r * ldx + c * 8;
        const float4 a = ld4(p), b = ld4(p + 4);
        v[i][0] = a.x, v[i][1] = a.y, v[i][2] = a.z, v[i][3] = a.w;
        v[i][4] = b.x, v[i][5] = b.y, v[i][6] = b.z, v[i][7] = b.w;
      }
    }
    if constexpr (ROT) {
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (!(k & h)) {
            const float a = v[i][k], b = v[i][k + h];
            v[i][k] = a + b;
            v[i][k + h] = a - b;
          }
    }
  }
  if constexpr (ROT) {
    // strides 8..64: the partner value sits in lane tid ^ 1, 2, 4, 8 of the
    // same 16-lane DPP row; every lane takes part (a 16-lane group is wholly
    // inside the row or wholly past it: nch is a multiple of 16)
    const int ni = (nch + 255) >> 8;
    rot_stage<1>(v, tid, ni);
    rot_stage<2>(v, tid, ni);
    rot_stage<4>(v, tid, ni);
    rot_stage<8>(v, tid, ni);
  }
#pragma unroll
  for (int i = 0; i < QMAXC; ++i) {
    const int c = tid + 256 * i;
    if (c < nch) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        am = fmaxf(am, fabsf(v[i][k]));
        nanck += v[i][k] * 0.f;
      }
    }
  }
  // fmaxf drops NaN operands, so the NaN check travels in a separate sum
  am = wave_max(am);
  nanck = wave_sum(nanck);
  if ((tid & 63) == 0) {
    red[tid >> 6] = am;
    red[4 + (tid >> 6)] = nanck;
  }
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) + (red[4] + red[5] + red[6] + red[7]);
  float sc, qi;
  quant_params(am, sc, qi);
#pragma unroll
  for (int i = 0; i < QMAXC; ++i) {
    const int c = tid + 256 * i;
    if (c < nch) {
      const u32x2 o = {quant4(v[i][0], v[i][1], v[i][2], v[i][3], qi), quant4(v[i][4], v[i][5], v[i][6], v[i][7], qi)};
      *reinterpret_cast<u32x2*>(q + r * ldq + c * 8) = o;
    }
  }
  if (tid == 0) s[r] = sc * post_scale;
}

__global__ void patchify_kernel(const float* lat, bf16_t* out, int B, int C, int Hp, int Wp, int p,
                                int npad) {
  const int64_t F = (int64_t)p * p * C;
  const int64_t total = (int64_t)B * Hp * Wp * F;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int f = (int)(idx % F);
  const int64_t tok = idx / F;
  const int ntok = Hp * Wp;
  const int b = (int)(tok / ntok), n = (int)(tok % ntok);
  const int i = n / Wp, j = n % Wp;
  const int ab = f / C, ch = f % C, pa = ab / p, pb = ab % p;
  const int Hl = Hp * p, Wl = Wp * p;
  out[((int64_t)b * npad + n) * F + f] = f2bf(lat[(((int64_t)b * C + ch) * Hl + i * p + pa) * Wl + j * p + pb]);
}

}  // namespace

hipError_t launch_pre_norm(const PreNormArgs& a, hipStream_t s) {
  const int rows = a.r1 - a.r0;
  if (rows <= 0) return hipSuccess;
  if (a.hq)
    hipLaunchKernelGGL(pre_norm_kernel<true>, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(pre_norm_kernel<false>, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

// the instance for the row length and output type (see row_cap)
hipError_t launch_post_norm(const PostNormArgs& a, hipStream_t s) {
  const int rows = a.r1 - a.r0;
  if (rows <= 0) return hipSuccess;
  const dim3 g((rows + 3) / 4), b(256);
  if (a.D == 15 * 256) {
    if (a.hq) hipLaunchKernelGGL((post_norm_kernel<15, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL(post_norm_3840_kernel, g, b, 0, s, a);
  } else {
    if (a.hq) hipLaunchKernelGGL((post_norm_kernel<0, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((post_norm_kernel<0, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, int x_bf16, int64_t ldx, int8_t* q, int64_t ldq, float* scale, int rows,
                             int K, int rotate, float post_scale, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
#define QR(B, R) hipLaunchKernelGGL((quant_rows_kernel<B, R>), dim3(rows), dim3(256), 0, s, x, ldx, q, ldq, scale, K, post_scale)
  if (x_bf16) {
    if (rotate) QR(true, true); else QR(true, false);
  } else {
    if (rotate) QR(false, true); else QR(false, false);
  }
#undef QR
  return hipGetLastError();
}

hipError_t launch_rows_rmsnorm(const void* x, int x_bf16, const float* w, bf16_t* out, int rows,
                               int Dc, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (x_bf16)
    hipLaunchKernelGGL(rows_rmsnorm_kernel<true>, dim3((rows + 3) / 4), dim3(256), 0, s, x, w, out, rows, Dc, eps);
  else
    hipLaunchKernelGGL(rows_rmsnorm_kernel<false>, dim3((rows + 3) / 4), dim3(256), 0, s, x, w, out, rows, Dc, eps);
  return hipGetLastError();
}

hipError_t launch_fold_mod(const float* mod, int64_t mod_stride, const float* normw, const int32_t* mod_idx,
                           int n_blocks, int n_mod, int D, int B, float* fold, hipStream_t s) {
  const int64_t n = (int64_t)(4 * n_blocks + 1) * D;
  hipLaunchKernelGGL(fold_mod_kernel, dim3((unsigned)((n + 255) / 256), B), dim3(256), 0, s, mod, mod_stride, normw,
                     mod_idx, n_blocks, n_mod, D, fold);
  return hipGetLastError();
}

hipError_t launch_patchify(const float* latent, bf16_t* out, int B, int C, int Hp, int Wp, int patch,
                           int npad, hipStream_t s) {
  const int64_t total = (int64_t)B * Hp * Wp * patch * patch * C;
  hipLaunchKernelGGL(patchify_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, latent, out, B, C,
                     Hp, Wp, patch, npad);
  return hipGetLastError();
}

}  // namespace zimg
