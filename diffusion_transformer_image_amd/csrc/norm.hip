// HBM-bound row kernels of the S3-DiT block: the adaLN-modulated pre-norm,
// the fused post-norm + tanh gate + residual (+ the next pre-norm), the
// caption RMSNorm, QK-RMSNorm + 3-axis RoPE with the V transpose, patchify.
//
// Block structure ("Z-Image" (AI Toolkit docs), Architecture: RMSNorm,
// QK RMSNorm, adaLN from the timestep embedding; "Z-Image-Turbo MNN (int8,
// fp16-safe)", Conversion details: the to_out and w2 outputs feed an
// RMSNorm).  Residual rows are fp32 and every reduction is fp32; activations
// handed to the GEMMs are bf16.
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

// modulation value for (sample, d): scale -> 1 + m, gate -> tanh(m)
ZI_DEV float4 mod_scale(const ModRef& m, int sample, int d) {
  if (!m.mod) return make_float4(1.f, 1.f, 1.f, 1.f);
  const float4 v = ld4(m.mod + (int64_t)sample * m.stride + m.off + d);
  return make_float4(1.f + v.x, 1.f + v.y, 1.f + v.z, 1.f + v.w);
}
ZI_DEV float4 mod_gate(const ModRef& m, int sample, int d) {
  if (!m.mod) return make_float4(1.f, 1.f, 1.f, 1.f);
  const float4 v = ld4(m.mod + (int64_t)sample * m.stride + m.off + d);
  return make_float4(tanhf(v.x), tanhf(v.y), tanhf(v.z), tanhf(v.w));
}

ZI_DEV void store_bf16x4(bf16_t* p, float a, float b, float c, float d) {
  u32x2 u = {pack2bf(a, b), pack2bf(c, d)};
  *reinterpret_cast<u32x2*>(p) = u;
}

// normalise the row held in v[] (nv float4 per lane) and write bf16
ZI_DEV void norm_write(const float4* v, int nv, int lane, int D, int kind, float eps,
                       const float* w, const ModRef& sc, int sample, bf16_t* h) {
  float mean = 0.f;
  if (kind == 1) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (i < nv) s += v[i].x + v[i].y + v[i].z + v[i].w;
    mean = wave_sum(s) / (float)D;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i < nv) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      ss += a * a + b * b + c * c + d * d;
    }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)D + eps);
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i < nv) {
      const int d = (lane + 64 * i) * 4;
      const float4 s = mod_scale(sc, sample, d);
      float4 ww = make_float4(1.f, 1.f, 1.f, 1.f);
      if (kind == 0) ww = ld4(w + d);
      store_bf16x4(h + d, (v[i].x - mean) * inv * ww.x * s.x, (v[i].y - mean) * inv * ww.y * s.y,
                   (v[i].z - mean) * inv * ww.z * s.z, (v[i].w - mean) * inv * ww.w * s.w);
    }
}

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
  norm_write(v, nv, lane, a.D, a.kind, a.eps, a.w, a.scale, a.row_sample[r], a.h + (int64_t)r * a.D);
}

__global__ __launch_bounds__(256) void post_norm_kernel(PostNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = a.r0 + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.r1) return;
  const int nv = a.D >> 8;
  const int sample = a.row_sample[r];
  const bf16_t* yr = a.y + (int64_t)r * a.D;
  float* xr = a.x + (int64_t)r * a.D;
  float4 y[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i < nv) {
      const u32x2 u = *reinterpret_cast<const u32x2*>(yr + (lane + 64 * i) * 4);
      y[i] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                         __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
      ss += y[i].x * y[i].x + y[i].y * y[i].y + y[i].z * y[i].z + y[i].w * y[i].w;
    }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)a.D + a.eps);
  float4 v[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i < nv) {
      const int d = (lane + 64 * i) * 4;
      const float4 g = mod_gate(a.gate, sample, d);
      const float4 w = ld4(a.w_post + d);
      float4 x = ld4(xr + d);
      x.x += g.x * (y[i].x * inv * w.x);
      x.y += g.y * (y[i].y * inv * w.y);
      x.z += g.z * (y[i].z * inv * w.z);
      x.w += g.w * (y[i].w * inv * w.w);
      *reinterpret_cast<float4*>(xr + d) = x;
      v[i] = x;
    }
  if (r >= a.n0 && r < a.n1)
    norm_write(v, nv, lane, a.D, a.next_kind, a.next_eps, a.w_next, a.scale_next, sample,
               a.h + (int64_t)r * a.D);
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

// QK-RMSNorm + RoPE for a tile of 64 rows of one head, plus the V transpose.
// Lane p of a wave owns channel pair (2p, 2p+1) of a 128-wide head, which is
// exactly RoPE pair p, so the rotation needs no data exchange.
constexpr int QK_ROWS = 64;
constexpr int VPAD = 136;  // LDS row stride (bf16) of the V staging tile

__global__ __launch_bounds__(256) void qknorm_rope_kernel(QKRopeArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t vs[QK_ROWS * VPAD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int rt0 = a.r0 + blockIdx.x * QK_ROWS;
  const int D = a.H * 128;
  const int64_t ld = 3 * (int64_t)D;
  const float wq0 = a.wq[2 * lane], wq1 = a.wq[2 * lane + 1];
  const float wk0 = a.wk[2 * lane], wk1 = a.wk[2 * lane + 1];

  for (int rr = wave; rr < QK_ROWS; rr += 4) {
    const int r = rt0 + rr;
    if (r >= a.r1) break;
    const float c = a.cos_t[(int64_t)r * 64 + lane], s = a.sin_t[(int64_t)r * 64 + lane];
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      uint32_t* p = reinterpret_cast<uint32_t*>(a.qkv + r * ld + part * D + h * 128) + lane;
      const uint32_t u = *p;
      const float x0 = __uint_as_float(u << 16), x1 = __uint_as_float(u & 0xffff0000u);
      const float inv = 1.0f / sqrtf(wave_sum(x0 * x0 + x1 * x1) * (1.0f / 128.0f) + a.eps);
      const float n0 = x0 * inv * (part ? wk0 : wq0);
      const float n1 = x1 * inv * (part ? wk1 : wq1);
      *p = pack2bf(n0 * c - n1 * s, n0 * s + n1 * c);
    }
  }

  // V tile -> LDS (rows past r1 are zero so the transposed copy stays finite)
  for (int i = 0; i < 4; ++i) {
    const int cidx = threadIdx.x + 256 * i, row = cidx >> 4, ch = cidx & 15;
    const int r = rt0 + row;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < a.r1) v = *reinterpret_cast<const u32x4*>(a.qkv + r * ld + 2 * D + h * 128 + ch * 8);
    *reinterpret_cast<u32x4*>(&vs[row * VPAD + ch * 8]) = v;
  }
  __syncthreads();
  // vT[h][d][rt0 + 8*rc .. +8]: 128 d-rows x 8 chunks of 8 rows
  for (int i = 0; i < 4; ++i) {
    const int cidx = threadIdx.x + 256 * i, d = cidx >> 3, rc = cidx & 7;
    if (rt0 + rc * 8 >= a.r1) continue;  // stage bounds are multiples of 8
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[u] = (uint32_t)vs[(rc * 8 + 2 * u) * VPAD + d] | ((uint32_t)vs[(rc * 8 + 2 * u + 1) * VPAD + d] << 16);
    u32x4 o = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(a.vT + ((int64_t)(h * 128 + d)) * a.S_pad + rt0 + rc * 8) = o;
  }
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
  hipLaunchKernelGGL(pre_norm_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_post_norm(const PostNormArgs& a, hipStream_t s) {
  const int rows = a.r1 - a.r0;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(post_norm_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, a);
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

hipError_t launch_qknorm_rope(const QKRopeArgs& a, hipStream_t s) {
  const int rows = a.r1 - a.r0;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(qknorm_rope_kernel, dim3((rows + QK_ROWS - 1) / QK_ROWS, a.H), dim3(256), 0, s, a);
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
