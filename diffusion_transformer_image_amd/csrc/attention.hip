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
// transposed [128][key] tile read from vT) by direct buffer->LDS loads, K
// into three buffers (loaded three tiles ahead) and V^T into two; scores of
// the next tile are computed while the current tile's softmax runs, so
// matrix-core and vector work overlap.
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

#include <mutex>

namespace zimg {
namespace {

constexpr int HD = 128;  // head_dim
constexpr int KTILE = 64;
constexpr float RESCALE_SLACK = 8.0f;  // log2 units: stale row max may lag by 2^8
constexpr int MAX_SPLIT = 16;          // key-tile chunks per split (item, head) pair
constexpr int AHEAD = 3;               // LDS operand reads issued ahead of their MFMA

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

ZI_DEV int swap_bits23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Lanes l and l ^ 32 hold the two key halves of one query.  v_permlane32_swap
// exchanges the 32-lane halves of two registers, so with both operands v the
// results hold v of lanes 0-31 and v of lanes 32-63 in every lane: the pair
// combines in registers, without an LDS round trip, and in the same order on
// both lanes.
ZI_DEV float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float lo = __uint_as_float(r[0]), hi = __uint_as_float(r[1]);
  return lo > hi ? lo : hi;
}
ZI_DEV float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs a) {
  // K tiles [64 keys][128], three (tile t in K<t % 3>), and V^T tiles
  // [128][64 keys], two (tile t in V<t % 2>): 80 KB, two workgroups per CU.
  // Separate arrays, so the compiler can see that a load into one buffer
  // never aliases reads of another (and waits only for the loads it must).
  __shared__ __attribute__((aligned(16))) bf16_t K0[KTILE * HD];
  __shared__ __attribute__((aligned(16))) bf16_t K1[KTILE * HD];
  __shared__ __attribute__((aligned(16))) bf16_t K2[KTILE * HD];
  __shared__ __attribute__((aligned(16))) bf16_t V0[HD * KTILE];
  __shared__ __attribute__((aligned(16))) bf16_t V1[HD * KTILE];

  // work unit -> (item, head) pair and key-tile chunk; split units are
  // numbered chunk-major so that neighbours share the same K/V range
  const int n_rest = a.n_items * a.H - a.n_full;
  int lid, chunk = 0, unit = -1;
  if ((int)blockIdx.x < a.n_full) {
    lid = xcd_remap(blockIdx.x, a.n_full);
  } else {
    unit = xcd_remap(blockIdx.x - a.n_full, n_rest * a.split);
    chunk = unit / n_rest;
    lid = a.n_full + (unit - chunk * n_rest);
  }
  const int h = lid / a.n_items;
  const AttnItem it = a.items[lid - h * a.n_items];
  const AttnSeg sg = a.segs[it.seg];
  const int D = a.H * HD;
  const int64_t ld = 3 * (int64_t)D;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int swk = lrow & 15;        // K rows are 256 B: 16 rows per lane group on distinct banks
  const int swv = (lrow >> 1) & 7;  // V^T rows are 128 B: two rows per 256-byte bank line

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
  const int T = nt0 + nt1;
  // this unit's key tiles [tb, tb + tn)
  int tb = 0, tn = T;
  if (unit >= 0) {
    tb = T * chunk / a.split;
    tn = T * (chunk + 1) / a.split - tb;
  }
  auto tile_start = [&](int t) { return t < nt0 ? sg.r0[0] + t * KTILE : sg.r0[1] + (t - nt0) * KTILE; };
  auto tile_valid = [&](int t) {
    return t < nt0 ? min(KTILE, sg.n[0] - t * KTILE) : min(KTILE, sg.n[1] - (t - nt0) * KTILE);
  };

  // Direct loads into LDS: a wave's load i fills 1 KB = 64 chunks of 16 B.
  // K: chunk p -> LDS row R = p/16 (holds key 32*(R/32) + swap_bits23(R%32)),
  //    stored position p%16 holds logical chunk (p%16) ^ (R & 15).
  // V^T: chunk p -> row d = p/8, stored position p%8 holds keys 8*((p%8) ^ ((d>>1)&7)).
  // With p = (4 i + wave) * 64 + lane these reduce to: K load i fetches key
  // 16 i + kk0 at chunk hc, V^T load i fetches row 32 i + dd0 at key chunk kc,
  // where kk0, hc, dd0, kc depend on the lane only -- so each lane keeps
  // fixed 32-bit offsets per operand and the per-tile address work is scalar.
  const int r0 = wave * 4 + (lane >> 4);
  const int kk0 = swap_bits23(r0), hc = (lane & 15) ^ r0;
  uint32_t koff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) koff[i] = (uint32_t)(((16 * i + kk0) * (int)ld + hc * 8) * 2);
  const int dd0 = wave * 8 + (lane >> 3);
  const uint32_t voff0 = (uint32_t)(dd0 * a.S_pad + (((lane & 7) ^ ((dd0 >> 1) & 7)) << 3));
  // K tiles are read through a buffer resource that spans this head's K
  // columns from the tile's first row to the last row of the buffer (at
  // most one tile): key rows past the end of qkv read as zero instead of
  // faulting, so every tile is loaded the same way, with no per-lane clamp
  // and no branch (keys past a range's end are masked before the softmax).
  const int64_t head_off = (int64_t)D + h * HD;
  auto dma_k = [&](int t, bf16_t* kb) {
    const int kr0 = tile_start(t);
    const int ext = min(a.rows - kr0, KTILE) * (int)ld * 2 - (int)head_off * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) buffer_load_lds16(a.qkv + (int64_t)kr0 * ld + head_off, ext, kb + (i * 4 + wave) * 512, koff[i], 0);
  };
  // V^T tiles through a buffer resource over this head's 128 rows of vT
  // (columns up to S_pad), with the tile's first column in the scalar offset
  const bf16_t* vbase = a.vT + (int64_t)(h * HD) * a.S_pad;
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (voff0 + (uint32_t)(i * 32 * a.S_pad)) * 2;
  // Keys past the end of a range get weight exactly 0, but 0 * v is NaN
  // where v is not finite, and a partial tile's last key columns hold the
  // rows after the range: another sample's tokens, or rows of no segment.
  // So in a partial tile the 8-key chunks that lie wholly past the range's
  // end are loaded from past the buffer extent, which fills them with zeros;
  // the keys after the end inside the last chunk are the range's own
  // alignment rows (ranges start at multiples of 8), which are kept finite.
  const int vkc = (lane & 7) ^ ((dd0 >> 1) & 7);  // the 8-key chunk this lane's V^T loads hold
  const int vext = HD * a.S_pad * 2;
  auto dma_v = [&](int t, bf16_t* vb) {
    const int c0 = tile_start(t) * 2, nv = tile_valid(t);
    if (nv == KTILE) {
#pragma unroll
      for (int i = 0; i < 4; ++i) buffer_load_lds16(vbase, vext, vb + (i * 4 + wave) * 512, voff[i], c0);
    } else {
      const bool past = vkc * 8 >= nv;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        buffer_load_lds16(vbase, vext, vb + (i * 4 + wave) * 512, past ? (uint32_t)vext : voff[i], c0);
    }
  };
  // S^T for 64 keys x this wave's 32 queries; with MASK, keys past nv -> -inf
  // Operand reads run AHEAD reads ahead of the MFMA that consumes them
  // (a small ring of fragments), so an MFMA never waits on the LDS read issued
  // just before it.
  // S^T score MFMAs [i0, i1) of a tile (16 in all) with their K fragment
  // reads AHEAD ahead, in a ring shared by the two calls that make one tile
  bf16x8 kf[AHEAD + 1];
  auto qk = [&](const bf16_t* kb, f32x16* st, int i0, int i1) {
    auto kread = [&](int i) {  // i = 2 ks + tt
      return *reinterpret_cast<const bf16x8*>(kb + ((i & 1) * 32 + lrow) * HD + (((2 * (i >> 1) + lhalf) ^ swk) << 3));
    };
    if (i0 == 0) {
      st[0] = f32x16{};
      st[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) kf[i] = kread(i);
    }
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      if (i + AHEAD < 16) kf[(i + AHEAD) % (AHEAD + 1)] = kread(i + AHEAD);
      st[i & 1] = mfma32(kf[i % (AHEAD + 1)], qf[i >> 1], st[i & 1]);
    }
  };
  auto mask = [&](f32x16* st, int nv) {
    // key of element e is c_e + 8*lhalf with c_e a compile-time constant;
    // comparing c_e against nv - 8*lhalf keeps the constants as immediates
    const int nvl = nv - lhalf * 8;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = tt * 32 + 16 * (e >> 3) + ((e >> 2) & 1) * 4 + (e & 3);
        st[tt][e] = c < nvl ? st[tt][e] : -INFINITY;
      }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m = -INFINITY, lp[2] = {0.f, 0.f};
  const float sl2 = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Online softmax in the log2 domain (raw v_exp_f32: weights below 2^-126
  // flush to zero).  The reference max m only moves when a lane's max exceeds
  // it by the slack, so p <= 2^slack; O and l are rescaled only when some lane
  // of the wave moved its m (a wave-uniform branch; after the first tile of a
  // row this is rare), since the rescale is as much vector work as the
  // exponentials themselves.  m is always an integer (the ceiling of the
  // max), so a weight 2^(s - m) rounds to bf16 the same way whatever m is:
  // a pair split into key chunks (each with its own m) weighs every key as
  // the whole pair would, and the merge scales chunks by exact powers of two.
  auto stats_max = [&](f32x16* st) {
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, st[tt][e]);
    mx = pair_max(mx) * sl2;
    return mx > m + RESCALE_SLACK ? ceilf(mx) : m;
  };
  auto stats_apply = [&](float mnew) {
    if (__any(mnew != m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
      for (int i = 0; i < 2; ++i) lp[i] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
      m = mnew;
    }
  };
  auto expsum = [&](f32x16* st) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) st[tt][e] = __builtin_amdgcn_exp2f(fmaf(st[tt][e], sl2, -m));
  };
  // O^T += V^T P^T over 4 key-steps of 16 (P converted to bf16 per step).
  // The row sum l adds up the same bf16 weights the product uses, two per
  // dot instruction, in two running parts (the parts and the lane pair are
  // summed once, at the end), so the normalised weights sum to one.
  auto pv = [&](const bf16_t* vb, const f32x16* st) {
    auto vread = [&](int i) {  // i = 4 s + dt
      return *reinterpret_cast<const bf16x8*>(vb + ((i & 3) * 32 + lrow) * KTILE + (((2 * (i >> 2) + lhalf) ^ swv) << 3));
    };
    bf16x8 vf[AHEAD + 1];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) vf[i] = vread(i);
    bf16x8 pf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + AHEAD < 16) vf[(i + AHEAD) % (AHEAD + 1)] = vread(i + AHEAD);
      if ((i & 3) == 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) pf[u] = (__bf16)st[i >> 3][((i >> 2) & 1) * 8 + u];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          lp[u & 1] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[2 * u], pf[2 * u + 1]}, ones, lp[u & 1], false);
      }
      o[i & 3] = mfma32(vf[i % (AHEAD + 1)], pf, o[i & 3]);
    }
  };
  // the issue order of the rest of a pipelined half: the remaining scores of
  // the next tile interleaved with the exponentials of the current one, then
  // the PV product
  // The first NPRE score MFMAs of the next tile are issued before the row
  // maxima of the current one, so that dependent chain (16 three-way maxima,
  // the lane-pair exchange, the ceiling) runs while they execute: -1.7 % per
  // launch against starting the scores after it with NPRE = 4, a further
  // 0.4-0.9 % with 8 (10 and 12 are slower).
  constexpr int NPRE = 8;
  constexpr int EXPV = (64 + (16 - NPRE) - 1) / (16 - NPRE);  // exponential-phase VALU per score MFMA
  auto pin_pre = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // first K operand reads
#pragma unroll
    for (int g = 0; g < NPRE; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read (K operand)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (scores)
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU (row-max chain)
    }
  };
  auto pin_order = [&]() {
#pragma unroll
    for (int g = NPRE; g < 16; ++g) {
      if (g + AHEAD < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read (K operand)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (scores)
      __builtin_amdgcn_sched_group_barrier(0x002, EXPV, 0);  // VALU (exponentials)
    }
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // first V operand reads
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      if (g + AHEAD < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read (V operand)
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU (conversion, row sums)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (PV)
    }
  };

  // Pipeline: in the half that handles tile t, the scores of tile t+1 are
  // computed while tile t is exponentiated and multiplied into O.  K(t+2) and
  // V(t+1) are loaded meanwhile into the buffers freed by the previous half.
  // Masking (partial tiles only) and the rescale are wave-uniform branches;
  // the first score MFMAs of tile t+1 are issued before the rescale's test.
  auto half = [&](const bf16_t* kn, const bf16_t* vc, f32x16* scur, f32x16* snext, int nv_cur) {
    if (nv_cur < KTILE) mask(scur, nv_cur);
    qk(kn, snext, 0, NPRE);
    const float mnew = stats_max(scur);
    pin_pre();
    stats_apply(mnew);
    qk(kn, snext, NPRE, 16);
    expsum(scur);
    pv(vc, scur);
    pin_order();
    // keeps the row-sum additions inside this half's interleave (otherwise
    // they are sunk past the next barrier, into the next half's serial part)
    asm volatile("" : "+v"(lp[0]), "+v"(lp[1]));
  };

  // The tile count is padded to an even number (>= 2) with an empty tile
  // whose scores are all masked (selected to -inf), so its weights are
  // exactly zero; the loop body is then the same for every pair of tiles,
  // with no tail.  Indexes j are relative to the unit's first tile tb; loads
  // of tiles past the range fetch the last real tile instead (into buffers
  // no one reads), so every half issues the same loads.
  //
  // Loads run ahead: the half that computes the scores of tile j+1 and the
  // PV product of tile j issues V(j+1) and then K(j+3).  Its closing barrier
  // waits for all but the last four loads of each wave (vmcnt(4): K(j+3) may
  // stay in flight), so a K tile has two halves to arrive and a V tile one.
  const int Tp = tn + (tn & 1);
  auto nvalid = [&](int j) { return j < tn ? tile_valid(tb + j) : 0; };
  auto clamp_t = [&](int j) { return tb + min(j, tn - 1); };
  // All but this wave's newest 4 loads have landed and its LDS reads are
  // done, then all waves meet.  Not __syncthreads(): its fence would also
  // wait for the newest loads (it covers every outstanding load into LDS).
  // The wait is the s_waitcnt builtin (vmcnt 4, lgkmcnt 0, expcnt off), so
  // the compiler knows which loads have landed; the empty asm statements
  // keep memory accesses from moving across the barrier.
  // a K or V^T tile is 16 KB: 4 loads of 1 KB per wave of the 4
  static_assert(KTILE * HD * 2 == 4 * 4 * 1024, "load_barrier's vmcnt(4) counts one tile's loads per wave");
  auto load_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0074);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // one pair of halves (tiles j, j+1): the K buffers of tiles j+1, j+2 and
  // the ones tiles j+3, j+4 are loaded into
  auto pair = [&](int j, bf16_t* kq1, bf16_t* kq2, bf16_t* kl3, bf16_t* kl4, f32x16* sa, f32x16* sb) {
    load_barrier();  // V(j), K(j+1) landed; everyone is done with K(j) and V(j-1)
    dma_v(clamp_t(j + 1), V1);
    dma_k(clamp_t(j + 3), kl3);
    half(kq1, V0, sa, sb, nvalid(j));
    load_barrier();  // V(j+1), K(j+2) landed; everyone is done with K(j+1) and V(j)
    dma_v(clamp_t(j + 2), V0);
    dma_k(clamp_t(j + 4), kl4);
    half(kq2, V1, sb, sa, nvalid(j + 1));  // j + 1 == tn: the padding tile, fully masked
  };
  dma_k(clamp_t(0), K0);
  dma_v(clamp_t(0), V0);
  dma_k(clamp_t(1), K1);
  dma_k(clamp_t(2), K2);
  load_barrier();  // K(0), V(0), K(1)
  f32x16 sc[2], sn[2];
  qk(K0, sc, 0, 16);
  // pairs cycle through the three K-buffer assignments (j = 0, 2, 4 mod 6)
  int j = 0;
  for (; j + 6 <= Tp; j += 6) {
    pair(j, K1, K2, K0, K1, sc, sn);
    pair(j + 2, K0, K1, K2, K0, sc, sn);
    pair(j + 4, K2, K0, K1, K2, sc, sn);
  }
  if (j < Tp) {
    pair(j, K1, K2, K0, K1, sc, sn);
    if (j + 2 < Tp) pair(j + 2, K0, K1, K2, K0, sc, sn);
  }
  // no load may still be writing this workgroup's LDS when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const float l = pair_sum(lp[0] + lp[1]);
  if (qi < it.nq && unit >= 0) {
    // partial state of this chunk: O unnormalised (relative to 2^m), m, l
    float* po = a.part + (int64_t)unit * (128 * HD) + qi * HD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = dt * 32 + i * 8 + lhalf * 4;
        *reinterpret_cast<f32x4*>(po + d0) = f32x4{o[dt][i * 4 + 0], o[dt][i * 4 + 1], o[dt][i * 4 + 2], o[dt][i * 4 + 3]};
      }
    if (lhalf == 0) {
      float* ml = a.part + (int64_t)n_rest * a.split * (128 * HD) + ((int64_t)unit * 128 + qi) * 2;
      *reinterpret_cast<float2*>(ml) = make_float2(m, l);
    }
  } else if (qi < it.nq) {
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

// Merge the chunks of one split (item, head) pair: with M the largest chunk
// reference max, weight w_c = 2^(m_c - M) (exact: the m_c are integers);
// O = sum_c w_c O_c / sum_c w_c l_c,
// summed in chunk order.  One workgroup per (pair, slice of CQ queries), so
// the merge spreads over many CUs; 16 lanes per query, 8 dims each, with all
// chunks' loads in flight together.
constexpr int CQ = 16;
__global__ __launch_bounds__(256) void attention_combine_kernel(AttnArgs a) {
  __shared__ float wt[MAX_SPLIT][CQ];
  const int n_rest = a.n_items * a.H - a.n_full;
  const int p = blockIdx.x;
  const int lid = a.n_full + p;
  const int h = lid / a.n_items;
  const AttnItem it = a.items[lid - h * a.n_items];
  const int qb = blockIdx.y * CQ;
  if (qb >= it.nq) return;  // the whole workgroup: a slice past the item's queries
  const float* ml = a.part + (int64_t)n_rest * a.split * (128 * HD);
  const int tid = threadIdx.x;
  if (tid < CQ && qb + tid < it.nq) {
    const int q = qb + tid;
    float M = -INFINITY;
    for (int c = 0; c < a.split; ++c) M = fmaxf(M, ml[((int64_t)(c * n_rest + p) * 128 + q) * 2]);
    float L = 0.f;
    for (int c = 0; c < a.split; ++c) {
      const float* v = ml + ((int64_t)(c * n_rest + p) * 128 + q) * 2;
      const float w = exp2f(v[0] - M);
      wt[c][tid] = w;
      L += w * v[1];
    }
    const float inv = 1.0f / L;
    for (int c = 0; c < a.split; ++c) wt[c][tid] *= inv;
  }
  __syncthreads();
  const int ql = tid >> 4, q = qb + ql, d = (tid & 15) * 8;
  if (q >= it.nq) return;
  const float* src = a.part + (int64_t)p * (128 * HD) + q * HD + d;
  const int64_t cstride = (int64_t)n_rest * (128 * HD);  // chunk c of pair p is unit c * n_rest + p
  f32x4 v0[MAX_SPLIT], v1[MAX_SPLIT];
#pragma unroll
  for (int c = 0; c < MAX_SPLIT; ++c)
    if (c < a.split) {
      v0[c] = *reinterpret_cast<const f32x4*>(src + c * cstride);
      v1[c] = *reinterpret_cast<const f32x4*>(src + c * cstride + 4);
    }
  f32x4 acc0 = {}, acc1 = {};
#pragma unroll
  for (int c = 0; c < MAX_SPLIT; ++c)
    if (c < a.split) {
      const float w = wt[c][ql];
      acc0 += w * v0[c];
      acc1 += w * v1[c];
    }
  const u32x4 u = {pack2bf(acc0[0], acc0[1]), pack2bf(acc0[2], acc0[3]), pack2bf(acc1[0], acc1[1]),
                   pack2bf(acc1[2], acc1[3])};
  *reinterpret_cast<u32x4*>(a.out + (int64_t)(it.q0 + q) * (a.H * HD) + h * HD + d) = u;
}

__global__ __launch_bounds__(256) void attention_plan_kernel(AttnPlanArgs p) {
  const int b = blockIdx.x;
  const AttnSeg sg = p.seg[b];
  if (threadIdx.x == 0) p.segs[b] = sg;
  const int t0 = (sg.n[0] + 127) / 128, t1 = (sg.n[1] + 127) / 128;
  for (int k = threadIdx.x; k < t0 + t1; k += blockDim.x) {
    const int r = k < t0 ? 0 : 1, q = k < t0 ? k : k - t0;
    p.items[p.item_off[b] + k] = AttnItem{sg.r0[r] + q * 128, min(128, sg.n[r] - q * 128), b, 0};
  }
}

// Scratch of the no-allocation entry point (see kernels.h): the work list
// and the split partials of zimg_attention_noalloc.  Host code never passes
// the array's name to a kernel (on the host it names a shadow, not the
// device memory); kernels get the address hipGetSymbolAddress returns.
__device__ __align__(256) unsigned char scratch[ATTN_SCRATCH_BYTES];

}  // namespace

void* attention_scratch(int device, hipError_t* err) {
  static std::mutex mu;
  static void* ptr[64] = {};
  *err = hipSuccess;
  if (device < 0 || device >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    ptr[device] = p;
  }
  return ptr[device];
}

hipError_t launch_attention_plan(const AttnPlanArgs& p, hipStream_t s) {
  if (p.B <= 0 || p.B > ATTN_OP_MAX_B) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attention_plan_kernel, dim3(p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int total = a.n_items * a.H;
  if (total <= 0) return hipSuccess;
  const int n_rest = total - a.n_full;
  if (a.n_full < 0 || n_rest < 0 || (n_rest > 0 && (a.split < 2 || a.split > MAX_SPLIT || !a.part)))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(attention_kernel, dim3(a.n_full + n_rest * (n_rest > 0 ? a.split : 0)), dim3(256), 0, s, a);
  if (n_rest > 0) hipLaunchKernelGGL(attention_combine_kernel, dim3(n_rest, 128 / CQ), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace zimg
