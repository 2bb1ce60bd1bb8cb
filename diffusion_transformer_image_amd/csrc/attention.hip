// Non-causal softmax attention over a segment of the single-stream sequence,
// head_dim 128, bf16 operands, fp32 online softmax ("Z-Image" (AI Toolkit
// docs), Architecture: full attention over the shared text+image sequence,
// 30 heads x 128; "Z-Image-Turbo MNN (int8, fp16-safe)", Performance:
// non-causal attention; scale 1/sqrt(128)).
//
// A segment is the union of up to two row ranges of the sequence buffer
// (one sample's image rows and its caption rows); queries of a segment see
// exactly the keys of that segment, so samples never interact.
//
// Workgroup = 4 waves = 128 queries of one head; each wave owns 32 queries.
// Keys stream through LDS in tiles of 64 (K as [key][128], V as the
// transposed [128][key] tile read from vT), double-buffered: the next tile's
// global loads are in flight while the current tile is computed.
//
// Orientation.  Scores are computed transposed, S^T = K Q^T, with the MFMA
// A operand = 32 keys and B operand = 32 queries, so every lane holds 16
// scores of a single query (its column): the row max and row sum of the
// online softmax are 32 in-lane operations plus one exchange with lane l^32.
// The output is also accumulated transposed, O^T = V^T P^T, so the per-query
// rescale factor is lane-uniform.  The score tile is consumed directly as the
// B operand of the PV product: K rows are placed in LDS so that accumulator
// element u of lane half h of key-step s is key 16 s + 8 h + u (LDS row r of
// a 32-key half holds key pi(r), pi = swap of bits 2 and 3), which makes the
// matching V^T operand one contiguous 16-byte LDS read.
#include "common.h"
#include "kernels.h"

namespace zimg {
namespace {

constexpr int HD = 128;  // head_dim
constexpr int KTILE = 64;

ZI_DEV int swap_bits23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KTILE * HD];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][HD * KTILE];

  const int total = a.n_items * a.H;
  const int lid = xcd_remap(blockIdx.x, total);
  const int h = lid / a.n_items;
  const AttnItem it = a.items[lid - h * a.n_items];
  const AttnSeg sg = a.segs[it.seg];
  const int D = a.H * HD;
  const int64_t ld = 3 * (int64_t)D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int swk = lrow & 15;         // K rows are 256 B: 16 rows per lane group on distinct banks
  const int swv = (lrow >> 1) & 7;   // V^T rows are 128 B: two rows per 256-byte bank line

  // this lane's query (B operand column): rows past the tile end are clamped
  const int qi = wave * 32 + lrow;
  const int qrow = it.q0 + min(qi, it.nq - 1);
  bf16x8 qf[8];
  {
    const bf16_t* qp = a.qkv + (int64_t)qrow * ld + h * HD + lhalf * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }

  const int nt0 = (sg.n[0] + KTILE - 1) / KTILE;
  const int nt1 = (sg.n[1] + KTILE - 1) / KTILE;
  const int ntiles = nt0 + nt1;

  u32x4 rk[4], rv[4];
  auto gload = [&](int t) {
    const bool first = t < nt0;
    const int off = (first ? t : t - nt0) * KTILE;
    const int kr0 = (first ? sg.r0[0] : sg.r0[1]) + off;
    const int nv = min(KTILE, (first ? sg.n[0] : sg.n[1]) - off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, key = c >> 4, hc = c & 15;
      rk[i] = *reinterpret_cast<const u32x4*>(a.qkv + (int64_t)(kr0 + min(key, nv - 1)) * ld + D + h * HD + hc * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, d = c >> 3, kc = c & 7;
      rv[i] = *reinterpret_cast<const u32x4*>(a.vT + (int64_t)(h * HD + d) * a.S_pad + kr0 + kc * 8);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, key = c >> 4, hc = c & 15;
      const int R = (key & 32) | swap_bits23(key & 31);
      *reinterpret_cast<u32x4*>(&Ks[buf][R * HD + ((hc ^ (R & 15)) << 3)]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, d = c >> 3, kc = c & 7;
      *reinterpret_cast<u32x4*>(&Vs[buf][d * KTILE + ((kc ^ ((d >> 1) & 7)) << 3)]) = rv[i];
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale_log2;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int nv = (t < nt0) ? min(KTILE, sg.n[0] - t * KTILE) : min(KTILE, sg.n[1] - (t - nt0) * KTILE);

    // S^T for 64 keys x 32 queries
    f32x16 st[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&Ks[buf][(tt * 32 + lrow) * HD + (((2 * ks + lhalf) ^ swk) << 3)]);
        st[tt] = mfma32(kf, qf[ks], st[tt]);
      }
    if (nv < KTILE) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = tt * 32 + 16 * (e >> 3) + lhalf * 8 + ((e >> 2) & 1) * 4 + (e & 3);
          if (key >= nv) st[tt][e] = -INFINITY;
        }
    }

    // online softmax in the log2 domain
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, st[tt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx * sl2);
    const float alpha = exp2f(m - mnew);
    float rs = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(fmaf(st[tt][e], sl2, -mnew));
        st[tt][e] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32, 64);
    l = fmaf(l, alpha, rs);
    m = mnew;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;

    // O^T += V^T P^T over 4 key-steps of 16
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 pf;
#pragma unroll
      for (int u = 0; u < 8; ++u) pf[u] = (__bf16)st[s >> 1][(s & 1) * 8 + u];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8*>(&Vs[buf][(dt * 32 + lrow) * KTILE + (((2 * s + lhalf) ^ swv) << 3)]);
        o[dt] = mfma32(vf, pf, o[dt]);
      }
    }
    if (t + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  if (qi < it.nq) {
    const float inv = 1.0f / l;
    bf16_t* op = a.out + (int64_t)(it.q0 + qi) * D + h * HD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = dt * 32 + i * 8 + lhalf * 4;
        u32x2 u = {pack2bf(o[dt][i * 4 + 0] * inv, o[dt][i * 4 + 1] * inv),
                   pack2bf(o[dt][i * 4 + 2] * inv, o[dt][i * 4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d0) = u;
      }
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  hipLaunchKernelGGL(attention_kernel, dim3(a.n_items * a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace zimg
