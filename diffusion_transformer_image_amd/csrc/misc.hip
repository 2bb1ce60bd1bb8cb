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

#include <algorithm>

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

// y[b][n] = sum_k W[n][k] act(x[b][k]) + bias[n].  A group of 32 lanes owns
// GEMV_R consecutive output rows and reads them with one 16-byte weight load
// per lane and row, all in flight together; act(x) of a K-chunk is computed
// once for the group's rows.  NB samples (up to 8 per launch) share each
// weight read.
constexpr int GEMV_MAXB = 8;
constexpr int GEMV_R = 4;

template <int NB>
__global__ __launch_bounds__(256) void gemv_kernel(const bf16_t* __restrict__ W, const float* __restrict__ bias,
                                                   const float* __restrict__ x, int64_t ldx, float* __restrict__ y,
                                                   int64_t ldy, int N, int K, int act) {
  const int sub = threadIdx.x & 31;
  const int n0 = ((blockIdx.x * 256 + threadIdx.x) >> 5) * GEMV_R;
  float acc[GEMV_R][NB];
#pragma unroll
  for (int r = 0; r < GEMV_R; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
  for (int k = sub * 8; k < K; k += 256) {
    u32x4 u[GEMV_R];
#pragma unroll
    for (int r = 0; r < GEMV_R; ++r)
      u[r] = n0 + r < N ? *reinterpret_cast<const u32x4*>(W + (int64_t)(n0 + r) * K + k) : u32x4{0, 0, 0, 0};
    float xv[NB][8];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float4 x0 = *reinterpret_cast<const float4*>(x + b * ldx + k);
      const float4 x1 = *reinterpret_cast<const float4*>(x + b * ldx + k + 4);
      const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) xv[b][q] = act ? v[q] / (1.0f + __expf(-v[q])) : v[q];
    }
#pragma unroll
    for (int r = 0; r < GEMV_R; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s = fmaf(__uint_as_float(u[r][q] << 16), xv[b][2 * q], s);
          s = fmaf(__uint_as_float(u[r][q] & 0xffff0000u), xv[b][2 * q + 1], s);
        }
        acc[r][b] += s;
      }
  }
#pragma unroll
  for (int r = 0; r < GEMV_R; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) acc[r][b] += __shfl_xor(acc[r][b], o, 64);
  if (sub == 0) {
#pragma unroll
    for (int r = 0; r < GEMV_R; ++r)
      if (n0 + r < N) {
        const float bv = bias ? bias[n0 + r] : 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) y[b * ldy + n0 + r] = acc[r][b] + bv;
      }
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

// one workgroup per row: x[row][d] = v[d]
__global__ __launch_bounds__(256) void set_rows_kernel(float* x, int D, const float* __restrict__ v) {
  float* row = x + (int64_t)blockIdx.x * D;
  for (int d = threadIdx.x; d < D; d += 256) row[d] = v[d];
}

// *first_bad = min(*first_bad, tag) when x[0, n) holds a NaN or an infinity
__global__ __launch_bounds__(256) void scan_finite_kernel(const float* __restrict__ x, int64_t n, int tag,
                                                          int* first_bad) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    bad |= !__builtin_isfinite(x[i]);
  if (bad) atomicMin(first_bad, tag);
}

__global__ void set_int_kernel(int* p, int v) { *p = v; }

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
  const dim3 grid((unsigned)((N + 8 * GEMV_R - 1) / (8 * GEMV_R))), blk(256);
  for (int b0 = 0; b0 < B; b0 += GEMV_MAXB) {
    const int nb = B - b0 < GEMV_MAXB ? B - b0 : GEMV_MAXB;
    const float* xb = x + b0 * ldx;
    float* yb = y + b0 * ldy;
#define GV(NB_) hipLaunchKernelGGL(gemv_kernel<NB_>, grid, blk, 0, s, W, bias, xb, ldx, yb, ldy, N, K, act)
    switch (nb) {
      case 1: GV(1); break;
      case 2: GV(2); break;
      case 3: GV(3); break;
      case 4: GV(4); break;
      case 5: GV(5); break;
      case 6: GV(6); break;
      case 7: GV(7); break;
      default: GV(8); break;
    }
#undef GV
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

hipError_t launch_set_rows(float* x, int D, const float* v, int r0, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(set_rows_kernel, dim3(n), dim3(256), 0, s, x + (int64_t)r0 * D, D, v);
  return hipGetLastError();
}

hipError_t launch_scan_finite(const float* x, int64_t n, int tag, int* first_bad, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(scan_finite_kernel, dim3(grid), dim3(256), 0, s, x, n, tag, first_bad);
  return hipGetLastError();
}

hipError_t launch_set_int(int* p, int v, hipStream_t s) {
  hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(1), 0, s, p, v);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, float v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace zimg
