// MFMA GEMM for the S3-DiT projections: C = epilogue(A . W^T).
//
// A [M, K] row-major (activations), W [N, K] row-major (a linear layer's
// weight, out_features x in_features), both bf16 with fp32 accumulation on
// v_mfma_f32_32x32x16_bf16, or both int8 with exact int32 accumulation on
// v_mfma_i32_32x32x32_i8 (the int8 projections: per-row codes of A and W
// with fp32 row scales, applied to the sums before the epilogue).  Both
// operands are K-contiguous, which is what the MFMA operand layout wants, so
// no transposition happens anywhere.  A 16-byte chunk holds 8 bf16 or 16
// int8 values, and one MFMA consumes one chunk per lane of each operand in
// either case, so the data movement below is the same for both types: it
// counts K in bf16-sized units (an int8 row of K codes is K/2 units).
//
// Workgroup tile BM x BN, K-step 64, 512 threads = 8 waves (2 waves per
// SIMD, so one wave's MFMAs cover the other's memory waits).  Operands go
// global -> LDS directly (buffer_load_dwordx4 ... lds, no register staging),
// A into two stage buffers and W into three: early in each K-step the next
// stage of A and the stage after next of W are issued, and one barrier per
// K-step publishes a stage, waiting for all but the newest W loads.  LDS
// rows are
// 128 B (64 bf16); the 16-byte chunk c of row r
// is stored at position c ^ ((r >> 1) & 7): the LDS serves 16 lanes x 16 B
// per cycle, and with two rows per 256-byte bank line this makes the 16
// rows of each lane group land on 16 distinct bank groups.
//
// Epilogues (template): bf16 store; fp32 store with bias; SwiGLU, where W's
// rows are interleaved in groups of 32 (32 rows of w1, then the same 32 rows
// of w3) and the output is silu(a1) * a3 (the SwiGLU FFN of "Z-Image" (AI
// Toolkit docs), Architecture); and the final-layer scatter back to the
// [B, C, Hl, Wl] latent with bias (unpatchify of 2x2 patches, "Latent
// space"); and the QKV projection's QK-RMSNorm + 3-axis RoPE + V transpose
// ("Z-Image" (AI Toolkit docs), Architecture: QK RMSNorm and 3D RoPE).
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace zimg {
namespace {

constexpr int BK = 64;
constexpr int NT = 512;

// Tile order: groups of gm row-tiles, column-major inside a group, so the
// tiles that run together on one XCD share row and column panels in its L2.
// gm is chosen per projection (group_rows below).
ZI_DEV void grouped_tile(int lid, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
  const int per_group = gm * tiles_n;
  const int first_m = (lid / per_group) * gm;
  const int gsize = min(tiles_m - first_m, gm);
  tm = first_m + (lid % per_group) % gsize;
  tn = (lid % per_group) / gsize;
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// SiLU of an fp32 value for the SwiGLU epilogues: x / (1 + e^-x) with the
// hardware reciprocal (about 1 ulp; the result is rounded to bf16 next) in
// place of an IEEE division, which costs about ten instructions
ZI_DEV float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Epilogue: element e = ii*4 + jj of subtile (i, j) of a wave is row
// i*32 + ii*8 + lhalf*4 + jj, column j*32 + lrow of the wave tile.
template <bool I8>
struct AccOf {
  using T = f32x16;
};
template <>
struct AccOf<true> {
  using T = i32x16;
};

// int8 operands: accumulator element (i, j, e) of a wave is the exact sum of
// row rbase + i*32 + (e>>2)*8 + lhalf*4 + (e&3), column cbase + j*32 + lrow;
// scale it by the row's and the column's scale (rows or columns past the
// matrix read the last one; they are never stored).
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void scale_acc(const i32x16 (&acc)[BM / WM / 32][BN / WN / 32],
                                          f32x16 (&out)[BM / WM / 32][BN / WN / 32], int m0, int n0, int M, int N,
                                          const EpiArgs& ep) {
  constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int lrow = lane & 31, lhalf = lane >> 5;
  float cs[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) cs[j] = ep.sw[min(n0 + wn * WTN + j * 32 + lrow, N - 1)];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float rs = ep.sa[min(m0 + wm * WTM + i * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3), M - 1)];
#pragma unroll
      for (int j = 0; j < TN; ++j) out[i][j][e] = mul_rn(mul_rn((float)acc[i][j][e], rs), cs[j]);
    }
}

template <int BM, int BN, int WM, int WN, int EPI>
__device__ __forceinline__ void epilogue(f32x16 (&acc)[BM / WM / 32][BN / WN / 32], int m0, int n0, int M, int N,
                                         const EpiArgs& ep) {
  constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int rbase = m0 + wm * WTM;
  const int cbase = n0 + wn * WTN;
  if constexpr (EPI == EPI_SWIGLU) {
    bf16_t* C = reinterpret_cast<bf16_t*>(ep.C);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const int col = ((cbase + j * 32) >> 1) + lrow;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
          if (row < M) {
            const float a1 = acc[i][j][e], a3 = acc[i][j + 1][e];
            const float s = silu(a1);
            C[(int64_t)row * ep.ldc + col] = f2bf(s * a3);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = cbase + j * 32 + lrow;
        if (col >= N) continue;
        float bias = 0.f;
        if constexpr (EPI != EPI_BF16) bias = ep.bias ? ep.bias[col] : 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
          if (row >= M) continue;
          const float v = acc[i][j][e];
          if constexpr (EPI == EPI_BF16) {
            reinterpret_cast<bf16_t*>(ep.C)[(int64_t)row * ep.ldc + col] = f2bf(v);
          } else if constexpr (EPI == EPI_F32_BIAS) {
            reinterpret_cast<float*>(ep.C)[(int64_t)row * ep.ldc + col] = v + bias;
          } else {  // EPI_UNPATCH: row = token of the batch, col = (a*p + b)*C + ch
            const int b = row / ep.npad, n = row - b * ep.npad;
            if (n >= ep.ntok) continue;  // alignment padding row
            const int pi = n / ep.Wp, pj = n - pi * ep.Wp;
            const int ab = col / ep.C_ch, ch = col - ab * ep.C_ch;
            const int pa = ab / ep.patch, pb = ab - pa * ep.patch;
            const int Hl = ep.Hp * ep.patch, Wl = ep.Wp * ep.patch;
            reinterpret_cast<float*>(ep.C)[(((int64_t)b * ep.C_ch + ch) * Hl + pi * ep.patch + pa) * Wl +
                                           pj * ep.patch + pb] = v + bias;
          }
        }
      }
  }
}

// One 16-lane group's share of a (row, head) of q or k: lane k holds the
// head's values 8k .. 8k+7 (bf16 pairs in x), i.e. RoPE pairs 4k .. 4k+3.
// RMS over the group, weight, rotation by the row's table, 16-byte store
// (only if ``store``).  All 16 lanes of the group must be active.
ZI_DEV void qk_rope_unit(const u32x4& x, int k, const float (&wv)[8], float eps, const float* cos_row,
                         const float* sin_row, bf16_t* dst, bool store) {
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = __uint_as_float(x[q] << 16), b = __uint_as_float(x[q] & 0xffff0000u);
    ss = fmaf(a, a, ss);
    ss = fmaf(b, b, ss);
  }
  ss += lane_xor<1>(ss);  // sums over the 16 lanes, in registers (DPP)
  ss += lane_xor<2>(ss);
  ss += lane_xor<4>(ss);
  ss += lane_xor<8>(ss);
  const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / 128.0f) + eps);  // hardware 1/sqrt (about 1 ulp)
  const float4 cc = *reinterpret_cast<const float4*>(cos_row + k * 4);
  const float4 sc = *reinterpret_cast<const float4*>(sin_row + k * 4);
  const float cv[4] = {cc.x, cc.y, cc.z, cc.w}, sv[4] = {sc.x, sc.y, sc.z, sc.w};
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = __uint_as_float(x[q] << 16) * inv * wv[2 * q];
    const float b = __uint_as_float(x[q] & 0xffff0000u) * inv * wv[2 * q + 1];
    o[q] = pack2bf(a * cv[q] - b * sv[q], a * sv[q] + b * cv[q]);
  }
  if (store) *reinterpret_cast<u32x4*>(dst + k * 8) = o;
}

ZI_DEV void qk_weights(const EpiArgs& ep, int sec, int k, float (&wv)[8]) {
  const float* w = sec ? ep.wk : ep.wq;
  const float4 wa = *reinterpret_cast<const float4*>(w + k * 8);
  const float4 wb = *reinterpret_cast<const float4*>(w + k * 8 + 4);
  wv[0] = wa.x, wv[1] = wa.y, wv[2] = wa.z, wv[3] = wa.w, wv[4] = wb.x, wv[5] = wb.y, wv[6] = wb.z, wv[7] = wb.w;
}

// Fused epilogue of the QKV projection, 256 x 256 tiles of 8 waves (2 x 4).
// Hidden is a multiple of 256, so a tile lies inside one of the q, k, v
// column blocks and covers two heads.  The tile, rounded to bf16, is staged
// in LDS (the four 32 KB operand buffers, 64 rows or columns each), then:
//  - q, k: 16 lanes per (row, head) RMS-normalise the head's 128 values
//    (weight wq or wk), rotate pair (2p, 2p+1) by the row's table entry p,
//    and store the head back in place;
//  - v: 16-byte runs of 8 rows of one column are stored into the transposed
//    copy vT[head*128 + d][row].
// Staging layouts keep LDS accesses free of bank conflicts.  q/k rows of
// 512 B hold their 16-byte chunk c at position c ^ stage_swz(r); the
// accumulator-order writes go out as 4-byte pairs of adjacent columns (the
// two lanes of a column pair swap one of their two rows), and one such store
// covers rows r, r + 1, r + 4, r + 5, which qk_swz places in the four
// different 64-byte bank groups.  v columns of 512 B (256 rows) hold chunk k
// (rows 8k..8k+7) at position k ^ (col & 15).
ZI_DEV int stage_swz(int r) { return ((r & 1) << 2) | (((r >> 2) & 1) << 3); }
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void qkv_rope_epilogue(const f32x16 (&acc)[BM / WM / 32][BN / WN / 32], int m0, int n0,
                                                  int M, const EpiArgs& ep, bf16_t* s0, bf16_t* s1, bf16_t* s2,
                                                  bf16_t* s3) {
  static_assert(BM == 256 && BN == 256 && WM == 2 && WN == 4, "QKV epilogue tiling");
  constexpr int TM = 4, TN = 2;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int sec = n0 / ep.D;  // 0: q, 1: k, 2: v
  auto region = [&](int k) { return k == 0 ? s0 : k == 1 ? s1 : k == 2 ? s2 : s3; };
  __syncthreads();  // every wave has finished reading the operand buffers
  if (sec < 2) {
    // a lane holds rows r, r + 1 of its column; it stores row r + odd of the
    // column pair (col & ~1, col | 1), taking the other column from lane ^ 1
    const int odd = lrow & 1;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;  // [other.hi | own.hi] : [own.lo | other.lo]
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      bf16_t* rg = region(wm * 2 + (i >> 1));
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int cc = wn * 64 + j * 32 + (lrow & ~1);
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const uint32_t own = pack2bf(acc[i][j][e], acc[i][j][e + 1]);
          const uint32_t other = __float_as_uint(lane_xor<1>(__uint_as_float(own)));
          const int r = wm * 128 + i * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3) + odd;
          *reinterpret_cast<uint32_t*>(rg + (r & 63) * 256 + (((cc >> 3) ^ stage_swz(r)) << 3) + (cc & 7)) =
              __builtin_amdgcn_perm(other, own, sel);
        }
      }
    }
    __syncthreads();
    // 16 lanes per (row, head), so table reads and stores are 256-byte runs;
    // rows past M are computed from a clamped table row and not stored
    const int k = lane & 15;
    float wv[8];
    qk_weights(ep, sec, k, wv);
    bf16_t* C = reinterpret_cast<bf16_t*>(ep.C);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int u = p * 32 + wid * 4 + (lane >> 4);  // (row, head) unit
      const int r = u >> 1, hl = u & 1;               // r >> 6 == p >> 2
      const u32x4 x = *reinterpret_cast<const u32x4*>(region(p >> 2) + (r & 63) * 256 + (((hl * 16 + k) ^ stage_swz(r)) << 3));
      const int row = m0 + r;
      const int64_t trow = (int64_t)ep.trow0 + min(row, M - 1);
      qk_rope_unit(x, k, wv, ep.eps, ep.cos_t + trow * 64, ep.sin_t + trow * 64,
                   C + (int64_t)row * ep.ldc + n0 + hl * 128, row < M);
    }
  } else {
    bf16_t* rg = region(wn);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = j * 32 + lrow;  // within the wave's 64 columns = the region's
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int k = wm * 16 + i * 4 + g;  // 8-row chunk
          const u32x2 v = {pack2bf(acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1]),
                           pack2bf(acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3])};
          *reinterpret_cast<u32x2*>(rg + col * 256 + ((k ^ (col & 15)) << 3) + lhalf * 4) = v;
        }
      }
    __syncthreads();
    const int vcol0 = n0 - 2 * ep.D;  // head*128 + d of the tile's first column
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int unit = u * 512 + tid, k = unit & 31, c = unit >> 5;
      const int r = k * 8;
      if (m0 + r >= M) continue;  // stage row counts are multiples of 8
      const u32x4 v = *reinterpret_cast<const u32x4*>(region(u >> 2) + (c & 63) * 256 + ((k ^ (c & 15)) << 3));
      *reinterpret_cast<u32x4*>(ep.vT + (int64_t)(vcol0 + c) * ep.S_pad + ep.trow0 + m0 + r) = v;
    }
  }
}

// bf16 epilogues of full-width 256x256 tiles (plain, and SwiGLU with its
// 256x128 output) go through LDS so that global stores are 16-byte runs of
// whole rows instead of 2-byte stores from the accumulator layout.  The four
// 32 KB operand buffers hold the output tile, row r in buffer r / RPB; the
// 16-byte chunk k of a row is stored at position k ^ stage_swz(r), and the
// accumulator-order writes go out as 4-byte pairs of adjacent columns, as in
// the QKV epilogue, so neither they nor the row-order reads conflict.
template <int BM, int BN, int WM, int WN, int EPI>
__device__ __forceinline__ void staged_bf16_epilogue(const f32x16 (&acc)[BM / WM / 32][BN / WN / 32], int m0, int n0,
                                                     int M, const EpiArgs& ep, bf16_t* s0, bf16_t* s1, bf16_t* s2,
                                                     bf16_t* s3) {
  static_assert(BM == 256 && BN == 256 && WM == 2 && WN == 4, "staged epilogue tiling");
  static_assert(EPI == EPI_BF16 || EPI == EPI_SWIGLU, "bf16 outputs only");
  constexpr int TM = 4, TN = 2;
  constexpr int OW = EPI == EPI_SWIGLU ? BN / 2 : BN;  // output columns of the tile
  constexpr int CPR = OW / 8;                           // 16-byte chunks per output row
  constexpr int RPB = 16384 / OW;                       // rows per 32 KB buffer
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int lrow = lane & 31, lhalf = lane >> 5;
  auto region = [&](int k) { return k == 0 ? s0 : k == 1 ? s1 : k == 2 ? s2 : s3; };
  __syncthreads();  // every wave has finished reading the operand buffers
  const int odd = lrow & 1;
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;  // [other.hi | own.hi] : [own.lo | other.lo]
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int rb = wm * 128 + i * 32;  // 32 rows, all in one buffer
    bf16_t* rg = region(rb / RPB);
#pragma unroll
    for (int j = 0; j < TN; j += (EPI == EPI_SWIGLU ? 2 : 1)) {
      const int cc = (EPI == EPI_SWIGLU ? wn * 32 : wn * 64 + j * 32) + (lrow & ~1);
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float v0 = acc[i][j][e], v1 = acc[i][j][e + 1];
        if constexpr (EPI == EPI_SWIGLU) {
          v0 = silu(v0) * acc[i][j + 1][e];
          v1 = silu(v1) * acc[i][j + 1][e + 1];
        }
        const uint32_t own = pack2bf(v0, v1);
        const uint32_t other = __float_as_uint(lane_xor<1>(__uint_as_float(own)));
        const int r = rb + (e >> 2) * 8 + lhalf * 4 + (e & 3) + odd;
        *reinterpret_cast<uint32_t*>(rg + (r % RPB) * OW + (((cc >> 3) ^ stage_swz(r)) << 3) + (cc & 7)) =
            __builtin_amdgcn_perm(other, own, sel);
      }
    }
  }
  __syncthreads();
  bf16_t* C = reinterpret_cast<bf16_t*>(ep.C);
  const int c0 = EPI == EPI_SWIGLU ? n0 / 2 : n0;
#pragma unroll
  for (int it = 0; it < BM * CPR / 512; ++it) {
    const int q = it * 512 + tid, r = q / CPR, k = q % CPR;
    if (m0 + r >= M) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(region(r / RPB) + (r % RPB) * OW + ((k ^ stage_swz(r)) << 3));
    *reinterpret_cast<u32x4*>(C + (int64_t)(m0 + r) * ep.ldc + c0 + k * 8) = v;
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
__device__ __forceinline__ void run_epilogue(f32x16 (&acc)[BM / WM / 32][BN / WN / 32], int m0, int n0, int M, int N,
                                             const EpiArgs& ep, bf16_t* s0, bf16_t* s1, bf16_t* s2, bf16_t* s3) {
  if constexpr (EPI == EPI_QKV_ROPE)
    qkv_rope_epilogue<BM, BN, WM, WN>(acc, m0, n0, M, ep, s0, s1, s2, s3);
  else if constexpr ((EPI == EPI_BF16 || EPI == EPI_SWIGLU) && BM == 256 && BN == 256)
    staged_bf16_epilogue<BM, BN, WM, WN, EPI>(acc, m0, n0, M, ep, s0, s1, s2, s3);
  else
    epilogue<BM, BN, WM, WN, EPI>(acc, m0, n0, M, N, ep);
}

// ROLE only separates the symbols of the projections (qkv, out, w1|w3, w2,
// embeds, final) so that profiles attribute time per projection.  I8: int8
// operands (pointers, strides and K in bf16-sized units, see above).
template <int BM, int BN, int WM, int WN, int EPI, int ROLE, bool I8>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(const bf16_t* __restrict__ A, int64_t lda,
                                                     const bf16_t* __restrict__ W, int64_t ldw,
                                                     int M, int N, int K, EpiArgs ep, int tiles_m,
                                                     int tiles_n, int full_tiles, int nsplit, float* ws, int gm) {
  static_assert(WM * WN == NT / 64, "8 waves");
  constexpr int NW = NT / 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile at least 32x32");
  static_assert(EPI != EPI_SWIGLU || (TN % 2) == 0, "swiglu pairs 32-col subtiles");
  constexpr int NA = BM * 8 / 64 / NW;  // direct-to-LDS loads per wave per K-step (1 KB each)
  constexpr int NB = BN * 8 / 64 / NW;
  static_assert(NA >= 1 && NB >= 1, "tile too small for 8 waves");

  // A in two stage buffers (stage k in As<k % 2>), W in three (Bs<k % 3>),
  // separate arrays, so the compiler can see that loads into one buffer
  // never alias reads of another
  __shared__ __attribute__((aligned(16))) bf16_t As0[BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs0[BN * BK];
  __shared__ __attribute__((aligned(16))) bf16_t As1[BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs1[BN * BK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs2[BN * BK];

  // Work unit -> tile.  The first full_tiles units are whole tiles; each of
  // the remaining (total - full_tiles) tiles is split into nsplit K-ranges.
  const int total = tiles_m * tiles_n;
  // full tiles and split units are spread over the XCDs separately (the
  // full-tile count is a multiple of the CU count, hence of 8)
  const int units = full_tiles + (total - full_tiles) * nsplit;
  const int bid = blockIdx.x;
  const int uid = bid < full_tiles ? xcd_remap(bid, full_tiles)
                                   : full_tiles + xcd_remap(bid - full_tiles, units - full_tiles);
  const bool is_split = uid >= full_tiles;
  const int tail_idx = is_split ? (uid - full_tiles) / nsplit : 0;
  const int chunk = is_split ? (uid - full_tiles) - tail_idx * nsplit : 0;
  const int lid = is_split ? full_tiles + tail_idx : uid;  // tile id in grouped order
  int tm, tn;
  grouped_tile(lid, tiles_m, tiles_n, gm, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;

  // A wave's load i fills 1 KB of LDS = 64 chunks of 16 B, chunk p = (i*NW + wid)*64 + lane,
  // i.e. row p/8, stored position p%8; it fetches the logical chunk stored there
  // (rows past M or N are clamped: their results are never stored).
  // Sources are the tile's rows of A and W, read through buffer resources,
  // at a per-lane 32-bit byte offset that stays fixed for the whole K loop;
  // a K-step only changes the uniform (scalar) offset.
  const char* a_base = reinterpret_cast<const char*>(A + (int64_t)m0 * lda);
  const char* b_base = reinterpret_cast<const char*>(W + (int64_t)n0 * ldw);
  uint32_t a_off[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int p = (i * NW + wid) * 64 + lane, row = p >> 3, lc = (p & 7) ^ ((row >> 1) & 7);
    a_off[i] = (uint32_t)((min(m0 + row, M - 1) - m0) * lda * 2 + lc * 16);
  }
  uint32_t b_off[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int p = (i * NW + wid) * 64 + lane, row = p >> 3, lc = (p & 7) ^ ((row >> 1) & 7);
    b_off[i] = (uint32_t)((min(n0 + row, N - 1) - n0) * ldw * 2 + lc * 16);
  }
  // The loads read through buffer resources over the tile's rows of A and
  // W (their extent); a K-step's offset is the uniform scalar offset.
  const int a_ext = (int)(min(BM, M - m0) * lda * 2), b_ext = (int)(min(BN, N - n0) * ldw * 2);
  auto issue_a = [&](int kt, bf16_t* as) {
#pragma unroll
    for (int i = 0; i < NA; ++i) buffer_load_lds16(a_base, a_ext, as + (i * NW + wid) * 512, a_off[i], kt * (BK * 2));
  };
  auto issue_b = [&](int kt, bf16_t* bs) {
#pragma unroll
    for (int i = 0; i < NB; ++i) buffer_load_lds16(b_base, b_ext, bs + (i * NW + wid) * 512, b_off[i], kt * (BK * 2));
  };

  using AccT = typename AccOf<I8>::T;
  AccT acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = AccT{};

  const int lrow = lane & 31, lhalf = lane >> 5;
  const int sw = (lrow >> 1) & 7;  // subtile bases are multiples of 32 rows
  const int aoff = (wm * WTM + lrow) * BK, boff = (wn * WTN + lrow) * BK;
  bf16x8 af[2][TM], bfr[2][TN];
  auto frags = [&](const bf16_t* as, const bf16_t* bs, int kk, int set) {
    const int ch = ((kk * 2 + lhalf) ^ sw) << 3;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[set][i] = *reinterpret_cast<const bf16x8*>(as + aoff + i * 32 * BK + ch);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[set][j] = *reinterpret_cast<const bf16x8*>(bs + boff + j * 32 * BK + ch);
  };
  auto mfmas = [&](int set) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (I8)
          acc[i][j] = mfma32_i8(af[set][i], bfr[set][j], acc[i][j]);
        else
          acc[i][j] = mfma32(af[set][i], bfr[set][j], acc[i][j]);
      }
  };
  constexpr int PAIRS = (TM + TN) < (TM * TN) ? (TM + TN) : (TM * TN);
  auto pin_pairs = [&]() {  // MFMAs of one k16 step, one-for-one with the next step's operand reads
#pragma unroll
    for (int g = 0; g < PAIRS; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    if (TM + TN > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, TM + TN - PAIRS, 0);
    if (TM * TN > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - PAIRS, 0);
  };
  // One K-step, entered with the operands of its first k16 step in set 0:
  // the MFMAs of the previous K-step's last k16 step (held back, operands in
  // set 1; they cover the latency of the set-0 reads issued just before),
  // the loads of A one stage ahead and of W two stages ahead, then three
  // k16 steps whose MFMAs are interleaved one-for-one with the operand reads
  // of the step after (the scheduling barriers pin that order).  The fourth
  // k16 step's MFMAs are held back past the barrier that ends the K-step,
  // behind the next stage's first operand reads.
  auto step = [&](const bf16_t* as, const bf16_t* bs, bool prev_tail, bool do_issue, int kt_a, bf16_t* nas,
                  int kt_b, bf16_t* nbs) {
    if (prev_tail) mfmas(1);
    if (do_issue) {
      issue_a(kt_a, nas);
      issue_b(kt_b, nbs);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);  // DS reads of the first k16 step (before the call)
    if (prev_tail) __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);  // held-back MFMAs
    __builtin_amdgcn_sched_group_barrier(0x020, NA + NB, 0);  // VMEM (the loads above)
#pragma unroll
    for (int kk = 0; kk + 1 < BK / 16; ++kk) {
      frags(as, bs, kk + 1, (kk + 1) & 1);
      mfmas(kk & 1);
      pin_pairs();
    }
  };
  // The barrier that ends a K-step: all of this wave's loads but the newest
  // NB (W two stages ahead) have landed and its LDS reads are done, then all
  // waves meet.  Not __syncthreads(): its fence would also wait for the
  // newest loads.  The wait is the s_waitcnt builtin (vmcnt NB, lgkmcnt 0,
  // expcnt off), so the compiler knows which loads have landed; the empty
  // asm statements keep memory accesses from moving across the barrier.
  static_assert(NB <= 15, "vmcnt field");
  auto stage_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070 | NB);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int KTALL = K / BK;
  const int kt0 = is_split ? (int)((int64_t)chunk * KTALL / nsplit) : 0;
  const int KT = is_split ? (int)((int64_t)(chunk + 1) * KTALL / nsplit) : KTALL;
  const int n = KT - kt0;
  auto clamp_k = [&](int s) { return kt0 + min(s, n - 1); };
  auto abuf = [&](auto r) -> bf16_t* {
    if constexpr (decltype(r)::value % 2 == 0) return As0; else return As1;
  };
  auto bbuf = [&](auto r) -> bf16_t* {
    if constexpr (decltype(r)::value % 3 == 0) return Bs0;
    else if constexpr (decltype(r)::value % 3 == 1) return Bs1;
    else return Bs2;
  };
  // K-step s of the unit (stage kt0 + s) uses As<s % 2> and Bs<s % 3>; the
  // buffers are compile-time constants of s mod 6, so the steps run in
  // groups of six, then a tail of up to five.  Every step issues loads (of
  // the last stage again where none is left: into a free buffer, never read),
  // so the loop body has no branch that would keep them from interleaving
  // with the MFMAs; the loads are drained before the epilogue.
  auto kstep = [&](auto r, int s) {
    constexpr int R = decltype(r)::value;
    using C0 = std::integral_constant<int, R>;
    using C1 = std::integral_constant<int, R + 1>;
    using C2 = std::integral_constant<int, R + 2>;
    step(abuf(C0{}), bbuf(C0{}), true, true, clamp_k(s + 1), abuf(C1{}), clamp_k(s + 2), bbuf(C2{}));
    stage_barrier();
    frags(abuf(C1{}), bbuf(C1{}), 0, 0);
  };
  issue_a(kt0, As0);
  issue_b(kt0, Bs0);
  issue_b(clamp_k(1), Bs1);
  stage_barrier();  // A and W of stage kt0
  frags(As0, Bs0, 0, 0);
  // the first step has no held-back MFMAs before it
  step(As0, Bs0, false, true, clamp_k(1), As1, clamp_k(2), Bs2);
  stage_barrier();
  frags(As1, Bs1, 0, 0);
  int s = 1;
  for (; s + 6 <= n; s += 6) {
    kstep(std::integral_constant<int, 1>{}, s);
    kstep(std::integral_constant<int, 2>{}, s + 1);
    kstep(std::integral_constant<int, 3>{}, s + 2);
    kstep(std::integral_constant<int, 4>{}, s + 3);
    kstep(std::integral_constant<int, 5>{}, s + 4);
    kstep(std::integral_constant<int, 6>{}, s + 5);
  }
  if (s < n) kstep(std::integral_constant<int, 1>{}, s);
  if (s + 1 < n) kstep(std::integral_constant<int, 2>{}, s + 1);
  if (s + 2 < n) kstep(std::integral_constant<int, 3>{}, s + 2);
  if (s + 3 < n) kstep(std::integral_constant<int, 4>{}, s + 3);
  if (s + 4 < n) kstep(std::integral_constant<int, 5>{}, s + 4);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land in LDS the epilogue reuses
  mfmas(1);  // the last K-step's fourth k16 step

  if (is_split) {
    // A split unit stores its partial (accumulator order, lanes contiguous;
    // int8: the int32 sums, bit for bit) and stops; the reduce kernel sums
    // the partials of each split tile in chunk order and runs the epilogue.
    float* part = ws + ((int64_t)tail_idx * nsplit + chunk) * (BM * BN);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if constexpr (I8)
            part[((i * TN + j) * 16 + e) * NT + tid] = __int_as_float(acc[i][j][e]);
          else
            part[((i * TN + j) * 16 + e) * NT + tid] = acc[i][j][e];
        }
    return;
  }
  if constexpr (I8) {
    f32x16 accf[TM][TN];
    scale_acc<BM, BN, WM, WN>(acc, accf, m0, n0, M, N, ep);
    run_epilogue<BM, BN, WM, WN, EPI>(accf, m0, n0, M, N, ep, As0, Bs0, As1, Bs1);
  } else {
    run_epilogue<BM, BN, WM, WN, EPI>(acc, m0, n0, M, N, ep, As0, Bs0, As1, Bs1);
  }
}

// Sum of the nsplit partials of each split tile, in chunk order (so the
// result does not depend on which unit finished first), then the epilogue,
// element by element.  A partial holds the accumulators of the producing
// workgroup in order q = ((i*TN + j)*16 + e)*NT + tid; each thread of this
// kernel owns a few q and recovers (row, column) from them.  SwiGLU takes
// the w1/w3 pair (j, j+1) together.
constexpr int RED_PER_THREAD = 4;

template <int BM, int BN, int WM, int WN, int EPI, bool I8>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(int M, int N, EpiArgs ep, int tiles_m, int tiles_n,
                                                          int full_tiles, int nsplit, const float* __restrict__ ws,
                                                          int gm) {
  constexpr int WTM = BM / WM, WTN = BN / WN, TN = WTN / 32;
  constexpr int TILE_F = BM * BN;
  constexpr int SLOTS = (EPI == EPI_SWIGLU) ? TILE_F / 2 : TILE_F;  // outputs per tile
  constexpr int PER_WG = 256 * RED_PER_THREAD;
  constexpr int WG_PER_TILE = SLOTS / PER_WG;
  const int tail_idx = blockIdx.x / WG_PER_TILE;
  const int lid = full_tiles + tail_idx;
  int tm, tn;
  grouped_tile(lid, tiles_m, tiles_n, gm, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const float* part = ws + (int64_t)tail_idx * nsplit * TILE_F;
  int qs[RED_PER_THREAD];
#pragma unroll
  for (int r = 0; r < RED_PER_THREAD; ++r) {
    const int slot = (blockIdx.x % WG_PER_TILE) * PER_WG + r * 256 + threadIdx.x;
    // slot -> accumulator index q (SwiGLU: the w1 half, j even)
    qs[r] = slot;
    if constexpr (EPI == EPI_SWIGLU) {
      const int tid_ = slot % NT, rest = slot / NT;  // rest = (i*(TN/2) + jp)*16 + e
      const int e = rest % 16, ijp = rest / 16, jp = ijp % (TN / 2), i = ijp / (TN / 2);
      qs[r] = ((i * TN + 2 * jp) * 16 + e) * NT + tid_;
    }
  }
  // chunk-outer, so that all of a chunk's loads are in flight together
  // (int8: the partials are int32 sums, added exactly)
  float v[RED_PER_THREAD] = {}, v3[RED_PER_THREAD] = {};
  int vi[RED_PER_THREAD] = {}, v3i[RED_PER_THREAD] = {};
  for (int c = 0; c < nsplit; ++c, part += TILE_F)
#pragma unroll
    for (int r = 0; r < RED_PER_THREAD; ++r) {
      if constexpr (I8) {
        vi[r] += __float_as_int(part[qs[r]]);
        if constexpr (EPI == EPI_SWIGLU) v3i[r] += __float_as_int(part[qs[r] + 16 * NT]);
      } else {
        v[r] += part[qs[r]];
        if constexpr (EPI == EPI_SWIGLU) v3[r] += part[qs[r] + 16 * NT];
      }
    }
#pragma unroll
  for (int r = 0; r < RED_PER_THREAD; ++r) {
    const int q = qs[r];
    const int tid_ = q % NT, e = (q / NT) % 16, ij = q / NT / 16, j = ij % TN, i = ij / TN;
    const int wid = tid_ >> 6, lane = tid_ & 63, wm = wid / WN, wn = wid % WN;
    const int row = m0 + wm * WTM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
    const int col = n0 + wn * WTN + j * 32 + (lane & 31);
    if (row >= M || col >= N) continue;
    if constexpr (I8) {
      const float rs = ep.sa[row];
      v[r] = mul_rn(mul_rn((float)vi[r], rs), ep.sw[col]);
      if constexpr (EPI == EPI_SWIGLU) v3[r] = mul_rn(mul_rn((float)v3i[r], rs), ep.sw[col + 32]);
    }
    if constexpr (EPI == EPI_SWIGLU) {
      const float s = silu(v[r]);
      const int ocol = ((n0 + wn * WTN + j * 32) >> 1) + (lane & 31);
      reinterpret_cast<bf16_t*>(ep.C)[(int64_t)row * ep.ldc + ocol] = f2bf(s * v3[r]);
    } else if constexpr (EPI == EPI_BF16) {
      reinterpret_cast<bf16_t*>(ep.C)[(int64_t)row * ep.ldc + col] = f2bf(v[r]);
    } else if constexpr (EPI == EPI_F32_BIAS) {
      reinterpret_cast<float*>(ep.C)[(int64_t)row * ep.ldc + col] = v[r] + (ep.bias ? ep.bias[col] : 0.f);
    } else {
      const int b = row / ep.npad, n = row - b * ep.npad;
      if (n >= ep.ntok) continue;
      const int pi = n / ep.Wp, pj = n - pi * ep.Wp;
      const int ab = col / ep.C_ch, ch = col - ab * ep.C_ch;
      const int pa = ab / ep.patch, pb = ab - pa * ep.patch;
      const int Hl = ep.Hp * ep.patch, Wl = ep.Wp * ep.patch;
      reinterpret_cast<float*>(ep.C)[(((int64_t)b * ep.C_ch + ch) * Hl + pi * ep.patch + pa) * Wl + pj * ep.patch +
                                     pb] = v[r] + (ep.bias ? ep.bias[col] : 0.f);
    }
  }
}

// Split tiles of the QKV projection: a workgroup of 256 threads per 32-row
// slice of a split tile (slice = (wm, i) of the producing kernel's layout;
// thread (wn, lane) takes over that wave's accumulators of the slice) sums
// the partials in chunk order, then runs the epilogue on the slice: q / k
// rows staged in LDS (same swizzle as the tile epilogue) and handed to
// qk_rope_unit; v written transposed straight from the registers (lanes
// l and l + 32 hold 4 + 4 consecutive rows of one column).
template <int BM, int BN, int WM, int WN, bool I8>
__global__ __launch_bounds__(256) void gemm_qkv_reduce_kernel(int M, EpiArgs ep, int tiles_m, int tiles_n,
                                                              int full_tiles, int nsplit, const float* __restrict__ ws,
                                                              int gm) {
  static_assert(BM == 256 && BN == 256 && WM == 2 && WN == 4, "QKV epilogue tiling");
  constexpr int TN = 2, TILE_F = BM * BN;
  __shared__ __attribute__((aligned(16))) bf16_t st[32 * 256];
  const int tail_idx = blockIdx.x >> 3, slice = blockIdx.x & 7;
  const int wm = slice >> 2, i = slice & 3;  // rows wm*128 + i*32 .. +31 of the tile
  const int lid = full_tiles + tail_idx;
  int tm, tn;
  grouped_tile(lid, tiles_m, tiles_n, gm, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, wn = tid >> 6, lane = tid & 63, lrow = lane & 31, lhalf = lane >> 5;
  const int src_tid = (wm * WN + wn) * 64 + lane;
  const float* part = ws + (int64_t)tail_idx * nsplit * TILE_F + src_tid;
  f32x16 acc[TN];
  const int rs0 = wm * 128 + i * 32;  // slice's first row in the tile
  if constexpr (I8) {
    i32x16 ai[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) ai[j] = i32x16{};
    for (int c = 0; c < nsplit; ++c, part += TILE_F)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) ai[j][e] += __float_as_int(part[((i * TN + j) * 16 + e) * NT]);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float cs = ep.sw[n0 + wn * 64 + j * 32 + lrow];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float rsc = ep.sa[min(m0 + rs0 + (e >> 2) * 8 + lhalf * 4 + (e & 3), M - 1)];
        acc[j][e] = mul_rn(mul_rn((float)ai[j][e], rsc), cs);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[j] = f32x16{};
    for (int c = 0; c < nsplit; ++c, part += TILE_F)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] += part[((i * TN + j) * 16 + e) * NT];
  }
  const int sec = n0 / ep.D;
  if (sec < 2) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = wn * 64 + j * 32 + lrow;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = (e >> 2) * 8 + lhalf * 4 + (e & 3);
        st[r * 256 + (((col >> 3) ^ (r & 15)) << 3) + (col & 7)] = f2bf(acc[j][e]);
      }
    }
    __syncthreads();
    const int k = lane & 15;
    float wv[8];
    qk_weights(ep, sec, k, wv);
    bf16_t* C = reinterpret_cast<bf16_t*>(ep.C);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int u = p * 16 + (tid >> 4);  // (row, head) unit of the slice
      const int r = u >> 1, hl = u & 1;
      const u32x4 x = *reinterpret_cast<const u32x4*>(st + r * 256 + (((hl * 16 + k) ^ (r & 15)) << 3));
      const int row = m0 + rs0 + r;
      const int64_t trow = (int64_t)ep.trow0 + min(row, M - 1);
      qk_rope_unit(x, k, wv, ep.eps, ep.cos_t + trow * 64, ep.sin_t + trow * 64,
                   C + (int64_t)row * ep.ldc + n0 + hl * 128, row < M);
    }
  } else {
    const int vcol0 = n0 - 2 * ep.D;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = wn * 64 + j * 32 + lrow;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = m0 + rs0 + g * 8 + lhalf * 4;
        if (row >= M) continue;  // stage row counts are multiples of 8
        const u32x2 v = {pack2bf(acc[j][g * 4 + 0], acc[j][g * 4 + 1]), pack2bf(acc[j][g * 4 + 2], acc[j][g * 4 + 3])};
        *reinterpret_cast<u32x2*>(ep.vT + (int64_t)(vcol0 + col) * ep.S_pad + ep.trow0 + row) = v;
      }
    }
  }
}

// How to split the last wave: with P workgroups running at once, T tiles
// take T / P full waves plus a partial one of r = T % P tiles.  Splitting
// each of the r tiles into s K-ranges turns the partial wave into
// ceil(r s / P) waves of 1/s the length; pick the s (at least two K-steps per
// range, partial sums must fit the workspace) with the shortest time.
int choose_split(int T, int KT, int tile_bytes, const GemmSplit& sp) {
  if (!sp.ws || sp.n_cu <= 0) return 1;
  const int r = T % sp.n_cu;
  if (r == 0 || 2 * r > sp.n_cu) return 1;  // a more than half-full last wave is left alone
  int best = 1;
  double best_cost = 1.0;
  for (int s = 2; s <= 32 && KT / s >= 4; ++s) {  // at least 4 K-steps per range
    if (r > sp.max_tiles || (size_t)r * s * tile_bytes > sp.ws_bytes) break;
    // waves of the split part (in tile times) + the reduction's reads of s partials
    const double cost = (double)((r * s + sp.n_cu - 1) / sp.n_cu) / s + 0.01 * s;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

// Row-tiles per group of the tile order, per projection.  32 tiles run at
// once on each XCD (256 CUs, 8 XCDs, one workgroup per CU), so a group of gm
// rows spans about 32 / gm columns; which split shares its L2 best depends on
// the number of column tiles (80 for w1|w3, 45 for qkv, 15 for out and w2),
// and was chosen by measuring the forward with each value.
int group_rows(int role, int tiles_n) {
  switch (role) {
    case ROLE_QKV: return 4;
    case ROLE_W13: return 3;
    case ROLE_OUT:
    case ROLE_W2: return 8;
    default: return tiles_n >= 32 ? 3 : 6;
  }
}

template <int BM, int BN, int WM, int WN, int EPI, int ROLE, bool I8>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  static_assert((2 * BM + 3 * BN) * BK * 2 <= 160 * 1024, "LDS budget");
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int T = tiles_m * tiles_n;
  constexpr int LDS_BYTES = (2 * BM + 3 * BN) * BK * 2;
  constexpr int U = I8 ? 2 : 1;  // elements per bf16-sized unit
  const int K = g.K / U;
  // a tile's rows of A and W are read through 32-bit buffer extents
  if ((int64_t)BM * (g.lda / U) * 2 > INT32_MAX || (int64_t)BN * (g.ldw / U) * 2 > INT32_MAX) return hipErrorInvalidValue;
  GemmSplit sp = g.split;
  sp.n_cu *= (160 * 1024) / LDS_BYTES;  // workgroups resident at once
  const int gm = group_rows(ROLE, tiles_n);
  const int nsplit = choose_split(T, K / BK, BM * BN * 4, sp);
  const int full = nsplit > 1 ? T - T % sp.n_cu : T;
  const int units = full + (T - full) * nsplit;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI, ROLE, I8>), dim3(units), dim3(NT), 0, s,
                     (const bf16_t*)g.A, g.lda / U, (const bf16_t*)g.W, g.ldw / U, g.M, g.N, K, g.ep, tiles_m,
                     tiles_n, full, nsplit, g.split.ws, gm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  if constexpr (EPI == EPI_QKV_ROPE) {
    hipLaunchKernelGGL((gemm_qkv_reduce_kernel<BM, BN, WM, WN, I8>), dim3((T - full) * 8), dim3(256), 0, s, g.M,
                       g.ep, tiles_m, tiles_n, full, nsplit, g.split.ws, gm);
    return hipGetLastError();
  }
  constexpr int SLOTS = (EPI == EPI_SWIGLU) ? BM * BN / 2 : BM * BN;
  static_assert(SLOTS % (256 * RED_PER_THREAD) == 0, "reduce grid");
  hipLaunchKernelGGL((gemm_reduce_kernel<BM, BN, WM, WN, EPI, I8>),
                     dim3((T - full) * (SLOTS / (256 * RED_PER_THREAD))), dim3(256), 0, s, g.M, g.N, g.ep, tiles_m,
                     tiles_n, full, nsplit, g.split.ws, gm);
  return hipGetLastError();
}

template <int EPI, int ROLE, bool I8 = false>
hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  if (g.N % 256 == 0) return launch_cfg<256, 256, 2, 4, EPI, ROLE, I8>(g, s);
  if (g.N % 128 == 0) return launch_cfg<256, 128, 4, 2, EPI, ROLE, I8>(g, s);
  return launch_cfg<256, 64, 8, 1, EPI, ROLE, I8>(g, s);
}

}  // namespace

const char* gemm_check(const GemmArgs& g) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return "gemm: M, N, K must be positive";
  if (g.K % BK) return "gemm: K must be a multiple of 64";
  if (g.N % 64) return "gemm: N must be a multiple of 64";
  if (g.epi == EPI_SWIGLU && g.N % 256) return "gemm: SwiGLU needs N a multiple of 256";
  if (g.lda < g.K || g.ldw < g.K) return "gemm: leading dimension smaller than K";
  if ((g.lda % 8) || (g.ldw % 8)) return "gemm: lda and ldw must be multiples of 8";
  // a tile's 256 rows must span less than 2^32 bytes (32-bit load offsets)
  if (g.lda > (1 << 22) || g.ldw > (1 << 22)) return "gemm: lda and ldw must be at most 4194304";
  if ((g.epi == EPI_BF16 || g.epi == EPI_SWIGLU) && ((g.ep.ldc % 8) || ((uintptr_t)g.ep.C & 15)))
    return "gemm: bf16 output needs ldc a multiple of 8 and a 16-byte aligned C";
  if (!g.A || !g.W || !g.ep.C) return "gemm: null pointer";
  if (g.epi == EPI_UNPATCH && (g.ep.ntok <= 0 || g.ep.npad < g.ep.ntok || g.ep.Wp <= 0 || g.ep.C_ch <= 0 || g.ep.patch <= 0))
    return "gemm: bad unpatchify geometry";
  if (g.epi < 0 || g.epi > EPI_QKV_ROPE) return "gemm: unknown epilogue";
  if (g.epi == EPI_QKV_ROPE &&
      (g.N != 3 * g.ep.D || g.ep.D % 256 || g.M % 8 || !g.ep.wq || !g.ep.wk || !g.ep.cos_t || !g.ep.sin_t ||
       !g.ep.vT || g.ep.trow0 < 0 || g.ep.trow0 % 8 || g.ep.S_pad < g.ep.trow0 + g.M || g.ep.S_pad % 8))
    return "gemm: bad QKV epilogue arguments";
  if ((g.role == ROLE_QKV) != (g.epi == EPI_QKV_ROPE) || (g.role == ROLE_W13 && g.epi != EPI_SWIGLU) ||
      ((g.role == ROLE_OUT || g.role == ROLE_W2) && g.epi != EPI_BF16) ||
      (g.role == ROLE_EMBED && g.epi != EPI_F32_BIAS) || (g.role == ROLE_FINAL && g.epi != EPI_UNPATCH))
    return "gemm: role and epilogue disagree";
  if (g.i8) {
    if (g.K % 128) return "gemm: int8 operands need K a multiple of 128";
    if (g.N % 256) return "gemm: int8 operands need N a multiple of 256";
    if ((g.lda % 16) || (g.ldw % 16) || ((uintptr_t)g.A & 15) || ((uintptr_t)g.W & 15))
      return "gemm: int8 operands need lda, ldw multiples of 16 and 16-byte aligned A, W";
    if (!g.ep.sa || !g.ep.sw) return "gemm: int8 operands need row scales sa and sw";
    if (g.epi == EPI_UNPATCH || g.role == ROLE_EMBED || g.role == ROLE_FINAL)
      return "gemm: int8 operands serve the block projections only";
  }
  return nullptr;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.i8) {  // 256 x 256 tiles only (N % 256 == 0)
    switch (g.role) {
      case ROLE_QKV: return launch_cfg<256, 256, 2, 4, EPI_QKV_ROPE, ROLE_QKV, true>(g, s);
      case ROLE_OUT: return launch_cfg<256, 256, 2, 4, EPI_BF16, ROLE_OUT, true>(g, s);
      case ROLE_W13: return launch_cfg<256, 256, 2, 4, EPI_SWIGLU, ROLE_W13, true>(g, s);
      case ROLE_W2: return launch_cfg<256, 256, 2, 4, EPI_BF16, ROLE_W2, true>(g, s);
      default: break;
    }
    switch (g.epi) {
      case EPI_BF16: return launch_cfg<256, 256, 2, 4, EPI_BF16, ROLE_ANY, true>(g, s);
      case EPI_F32_BIAS: return launch_cfg<256, 256, 2, 4, EPI_F32_BIAS, ROLE_ANY, true>(g, s);
      default: return launch_cfg<256, 256, 2, 4, EPI_SWIGLU, ROLE_ANY, true>(g, s);
    }
  }
  switch (g.role) {
    case ROLE_QKV: return launch_cfg<256, 256, 2, 4, EPI_QKV_ROPE, ROLE_QKV, false>(g, s);
    case ROLE_OUT: return launch_epi<EPI_BF16, ROLE_OUT>(g, s);
    case ROLE_W13: return launch_cfg<256, 256, 2, 4, EPI_SWIGLU, ROLE_W13, false>(g, s);
    case ROLE_W2: return launch_epi<EPI_BF16, ROLE_W2>(g, s);
    case ROLE_EMBED: return launch_epi<EPI_F32_BIAS, ROLE_EMBED>(g, s);
    case ROLE_FINAL: return launch_epi<EPI_UNPATCH, ROLE_FINAL>(g, s);
    default: break;
  }
  switch (g.epi) {
    case EPI_BF16: return launch_epi<EPI_BF16, ROLE_ANY>(g, s);
    case EPI_F32_BIAS: return launch_epi<EPI_F32_BIAS, ROLE_ANY>(g, s);
    case EPI_SWIGLU: return launch_cfg<256, 256, 2, 4, EPI_SWIGLU, ROLE_ANY, false>(g, s);
    default: return launch_epi<EPI_UNPATCH, ROLE_ANY>(g, s);
  }
}

}  // namespace zimg
