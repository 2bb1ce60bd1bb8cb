// Small kernels around the blocks: the timestep sinusoid, the bf16 GEMV used
// by the timestep MLP and by the one adaLN projection that produces every
// block's modulation at once, the Euler update of the sampler, and a fill.
//
// Timestep conditioning ("Z-Image" (AI Toolkit docs), Architecture: adaLN
// modulation from a 256-d timestep embedding; Specifics: model time
// t = (1000 - timestep)/1000).  Euler step ("Z-Image-Turbo MNN (int8,
// fp16-safe)", Scheduler: the model output is negated before the step).
#include "common.h"
#include "kernels.h"

namespace zimg {
namespace {

// e[b][i] = cos(t_scale * t_b * f_i) for i < half, sin(...) for the second
// half, f_i = exp(-ln(max_period) * i / half); evaluated in double.
__global__ void timestep_embed_kernel(TimeArgs ta, int B, int dim, float t_scale, float max_period,
                                      float* out) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * dim) return;
  const int b = idx / dim, i = idx % dim, half = dim / 2;
  const int fi = i < half ? i : i - half;
  const double f = exp(-log((double)max_period) * (double)fi / (double)half);
  const double arg = (double)t_scale * (double)ta.t[b] * f;
  out[idx] = (float)(i < half ? cos(arg) : sin(arg));
}

// y[b][n] = sum_k W[n][k] act(x[b][k]) + bias[n].  32 lanes per output row,
// 16-byte weight loads; up to 8 samples per launch share each weight read.
constexpr int GEMV_MAXB = 8;

__global__ __launch_bounds__(256) void gemv_kernel(const bf16_t* __restrict__ W, const float* __restrict__ bias,
                                                   const float* __restrict__ x, int64_t ldx, float* __restrict__ y,
                                                   int64_t ldy, int N, int K, int B, int act) {
  const int lane = threadIdx.x & 63;
  const int n = (blockIdx.x * 256 + threadIdx.x) >> 5;  // 8 rows per workgroup
  const int sub = lane & 31;
  float acc[GEMV_MAXB];
#pragma unroll
  for (int b = 0; b < GEMV_MAXB; ++b) acc[b] = 0.f;
  if (n < N) {
    const bf16_t* wr = W + (int64_t)n * K;
    for (int k = sub * 8; k < K; k += 256) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(wr + k);
      float w[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[2 * q] = __uint_as_float(u[q] << 16);
        w[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
      }
#pragma unroll
      for (int b = 0; b < GEMV_MAXB; ++b) {
        if (b >= B) break;
        const float* xb = x + b * ldx + k;
        const float4 x0 = *reinterpret_cast<const float4*>(xb);
        const float4 x1 = *reinterpret_cast<const float4*>(xb + 4);
        float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float v = act ? xv[q] / (1.0f + __expf(-xv[q])) : xv[q];
          s = fmaf(w[q], v, s);
        }
        acc[b] += s;
      }
    }
  }
#pragma unroll
  for (int b = 0; b < GEMV_MAXB; ++b) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) acc[b] += __shfl_xor(acc[b], o, 64);
  }
  if (n < N && sub == 0) {
    const float bv = bias ? bias[n] : 0.f;
    for (int b = 0; b < B; ++b) y[b * ldy + n] = acc[b] + bv;
  }
}

__global__ void euler_kernel(float* x, const float* o, float dt, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = fmaf(dt, -o[i], x[i]);
}

// Guided Euler update: the guided prediction c + g (c - u) and the step
// x += dt * (-prediction) in one pass (16 B of HBM traffic per element).
// Four elements per thread when every pointer is 16-byte aligned.
__global__ void cfg_euler4_kernel(float4* x, const float4* oc, const float4* ou, float g, float dt, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 c = oc[i], u = ou[i];
  float4 v = x[i];
  v.x = fmaf(dt, -fmaf(g, c.x - u.x, c.x), v.x);
  v.y = fmaf(dt, -fmaf(g, c.y - u.y, c.y), v.y);
  v.z = fmaf(dt, -fmaf(g, c.z - u.z, c.z), v.z);
  v.w = fmaf(dt, -fmaf(g, c.w - u.w, c.w), v.w);
  x[i] = v;
}
__global__ void cfg_euler_kernel(float* x, const float* oc, const float* ou, float g, float dt, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = fmaf(dt, -fmaf(g, oc[i] - ou[i], oc[i]), x[i]);
}

__global__ void fill_kernel(float* p, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_timestep_embed(const TimeArgs& t, int B, int dim, float t_scale, float max_period, float* out,
                                 hipStream_t s) {
  const int n = B * dim;
  hipLaunchKernelGGL(timestep_embed_kernel, dim3((n + 255) / 256), dim3(256), 0, s, t, B, dim, t_scale,
                     max_period, out);
  return hipGetLastError();
}

hipError_t launch_gemv(const bf16_t* W, const float* bias, const float* x, int64_t ldx, float* y, int64_t ldy,
                       int N, int K, int B, int act, hipStream_t s) {
  for (int b0 = 0; b0 < B; b0 += GEMV_MAXB) {
    const int nb = B - b0 < GEMV_MAXB ? B - b0 : GEMV_MAXB;
    hipLaunchKernelGGL(gemv_kernel, dim3((N + 7) / 8), dim3(256), 0, s, W, bias, x + b0 * ldx, ldx, y + b0 * ldy,
                       ldy, N, K, nb, act);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_euler(float* x, const float* o, float dt, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(euler_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, o, dt, n);
  return hipGetLastError();
}

hipError_t launch_cfg_euler(float* x, const float* oc, const float* ou, float g, float dt, int64_t n,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool vec = n % 4 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)oc & 15) == 0 && ((uintptr_t)ou & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(cfg_euler4_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, (float4*)x,
                       (const float4*)oc, (const float4*)ou, g, dt, n / 4);
  else
    hipLaunchKernelGGL(cfg_euler_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, oc, ou, g, dt, n);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, float v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace zimg
