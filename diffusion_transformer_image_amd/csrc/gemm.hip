// bf16 MFMA GEMM for the S3-DiT projections: C = epilogue(A . W^T).
//
// A [M, K] bf16 row-major (activations), W [N, K] bf16 row-major (a linear
// layer's weight, out_features x in_features), fp32 accumulation on
// v_mfma_f32_32x32x16_bf16.  Both operands are K-contiguous, which is what
// the MFMA operand layout wants, so no transposition happens anywhere.
//
// Workgroup tile BM x BN, K-step 64, 512 threads = 8 waves (2 waves per
// SIMD).  Each K-step is staged global -> registers -> LDS with a two-slot
// LDS ring: the next step's global loads are issued before the current
// step's MFMAs, and stored to the other slot after them, so one barrier per
// step suffices.  LDS rows are 128 B (64 bf16); the 16-byte chunk c of row r
// is stored at position c ^ (r & 7), so the 32 rows one MFMA operand read
// touches hit distinct bank groups.
//
// Epilogues (template): bf16 store; fp32 store with bias; SwiGLU, where W's
// rows are interleaved in groups of 32 (32 rows of w1, then the same 32 rows
// of w3) and the output is silu(a1) * a3 (the SwiGLU FFN of "Z-Image" (AI
// Toolkit docs), Architecture); and the final-layer scatter back to the
// [B, C, Hl, Wl] latent with bias (unpatchify of 2x2 patches, "Latent
// space").
#include "common.h"
#include "kernels.h"

namespace zimg {
namespace {

constexpr int BK = 64;
constexpr int NT = 512;
constexpr int GROUP_M = 8;

// ROLE only separates the symbols of the projections (qkv, out, w1|w3, w2,
// embeds, final) so that profiles attribute time per projection.
template <int BM, int BN, int WM, int WN, int EPI, int ROLE>
__global__ __launch_bounds__(NT) void gemm_kernel(const bf16_t* __restrict__ A, int64_t lda,
                                                  const bf16_t* __restrict__ W, int64_t ldw,
                                                  int M, int N, int K, EpiArgs ep, int tiles_m,
                                                  int tiles_n) {
  static_assert(WM * WN == NT / 64, "8 waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile at least 32x32");
  static_assert(EPI != EPI_SWIGLU || (TN % 2) == 0, "swiglu pairs 32-col subtiles");
  constexpr int A_CH = BM * 8 / NT;  // 16-byte chunks per thread per K-step
  constexpr int B_CH = BN * 8 / NT;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small for 512 threads");

  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * BK];

  // tile id: XCD-contiguous, then grouped along M
  const int total = tiles_m * tiles_n;
  const int lid = xcd_remap(blockIdx.x, total);
  const int per_group = GROUP_M * tiles_n;
  const int first_m = (lid / per_group) * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (lid % per_group) % gsize;
  const int tn = (lid % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;

  // global source pointers (rows clamped into range) and LDS destinations
  const bf16_t* a_src[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + NT * i, row = c >> 3, ch = c & 7;
    const int gr = min(m0 + row, M - 1);
    a_src[i] = A + (int64_t)gr * lda + ch * 8;
    a_dst[i] = row * BK + ((ch ^ (row & 7)) << 3);
  }
  const bf16_t* b_src[B_CH];
  int b_dst[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + NT * i, row = c >> 3, ch = c & 7;
    const int gr = min(n0 + row, N - 1);
    b_src[i] = W + (int64_t)gr * ldw + ch * 8;
    b_dst[i] = row * BK + ((ch ^ (row & 7)) << 3);
  }

  u32x4 ra[A_CH], rb[B_CH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + kt * BK);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) *reinterpret_cast<u32x4*>(&As[buf][a_dst[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) *reinterpret_cast<u32x4*>(&Bs[buf][b_dst[i]]) = rb[i];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // per-lane LDS read offsets for operand rows
  const int lrow = lane & 31, lhalf = lane >> 5;
  int a_off[TM], b_off[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_off[i] = (wm * WTM + i * 32 + lrow) * BK;
#pragma unroll
  for (int j = 0; j < TN; ++j) b_off[j] = (wn * WTN + j * 32 + lrow) * BK;
  const int sw = lrow & 7;  // (row & 7) is lrow & 7 because subtile bases are multiples of 32

  const int KT = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = ((kk * 2 + lhalf) ^ sw) << 3;
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][a_off[i] + ch]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][b_off[j] + ch]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: element e = ii*4 + jj of subtile (i, j) is row
  // i*32 + ii*8 + lhalf*4 + jj, column j*32 + lrow of the wave tile.
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
            const float s = a1 / (1.0f + __expf(-a1));
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

template <int BM, int BN, int WM, int WN, int EPI, int ROLE>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI, ROLE>), dim3(tiles_m * tiles_n), dim3(NT), 0, s,
                     g.A, g.lda, g.W, g.ldw, g.M, g.N, g.K, g.ep, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int EPI, int ROLE>
hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  if (g.N % 256 == 0) return launch_cfg<256, 256, 2, 4, EPI, ROLE>(g, s);
  if (g.N % 128 == 0) return launch_cfg<256, 128, 4, 2, EPI, ROLE>(g, s);
  return launch_cfg<256, 64, 8, 1, EPI, ROLE>(g, s);
}

}  // namespace

const char* gemm_check(const GemmArgs& g) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return "gemm: M, N, K must be positive";
  if (g.K % BK) return "gemm: K must be a multiple of 64";
  if (g.N % 64) return "gemm: N must be a multiple of 64";
  if (g.epi == EPI_SWIGLU && g.N % 256) return "gemm: SwiGLU needs N a multiple of 256";
  if (g.lda < g.K || g.ldw < g.K) return "gemm: leading dimension smaller than K";
  if ((g.lda % 8) || (g.ldw % 8)) return "gemm: lda and ldw must be multiples of 8";
  if (!g.A || !g.W || !g.ep.C) return "gemm: null pointer";
  if (g.epi == EPI_UNPATCH && (g.ep.ntok <= 0 || g.ep.npad < g.ep.ntok || g.ep.Wp <= 0 || g.ep.C_ch <= 0 || g.ep.patch <= 0))
    return "gemm: bad unpatchify geometry";
  if (g.epi < 0 || g.epi > EPI_UNPATCH) return "gemm: unknown epilogue";
  if ((g.role == ROLE_QKV && (g.epi != EPI_BF16 || g.N % 256)) || (g.role == ROLE_W13 && g.epi != EPI_SWIGLU) ||
      ((g.role == ROLE_OUT || g.role == ROLE_W2) && g.epi != EPI_BF16) ||
      (g.role == ROLE_EMBED && g.epi != EPI_F32_BIAS) || (g.role == ROLE_FINAL && g.epi != EPI_UNPATCH))
    return "gemm: role and epilogue disagree";
  return nullptr;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  switch (g.role) {
    case ROLE_QKV: return launch_cfg<256, 256, 2, 4, EPI_BF16, ROLE_QKV>(g, s);
    case ROLE_OUT: return launch_epi<EPI_BF16, ROLE_OUT>(g, s);
    case ROLE_W13: return launch_cfg<256, 256, 2, 4, EPI_SWIGLU, ROLE_W13>(g, s);
    case ROLE_W2: return launch_epi<EPI_BF16, ROLE_W2>(g, s);
    case ROLE_EMBED: return launch_epi<EPI_F32_BIAS, ROLE_EMBED>(g, s);
    case ROLE_FINAL: return launch_epi<EPI_UNPATCH, ROLE_FINAL>(g, s);
    default: break;
  }
  switch (g.epi) {
    case EPI_BF16: return launch_epi<EPI_BF16, ROLE_ANY>(g, s);
    case EPI_F32_BIAS: return launch_epi<EPI_F32_BIAS, ROLE_ANY>(g, s);
    case EPI_SWIGLU: return launch_cfg<256, 256, 2, 4, EPI_SWIGLU, ROLE_ANY>(g, s);
    default: return launch_epi<EPI_UNPATCH, ROLE_ANY>(g, s);
  }
}

}  // namespace zimg
