// Shared device-side definitions for the gfx950 kernels of the S3-DiT engine.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ZI_DEV __device__ __forceinline__

// bf16 <-> fp32.  The float -> bf16 cast rounds to nearest even (one
// v_cvt_pk_bf16_f32 per pair on gfx950).
ZI_DEV float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
ZI_DEV bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}
ZI_DEV uint32_t pack2bf(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// v_mfma_f32_32x32x16_bf16.  Lane l supplies A row (l % 32), k = (l/32)*8 + [0,8);
// B column (l % 32), same k; accumulator element i*4+j of lane l is
// C[i*8 + (l/32)*4 + j][l % 32].  (Layout checked on gfx950.)
ZI_DEV f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_i32_32x32x32_i8: each lane supplies 16 int8 of A (row l % 32) and
// 16 of B (column l % 32) in the same positions of K, so products pair A
// and B values of the same k whatever order the unit takes K in; the int32
// sums are exact.  Accumulator layout as for mfma32.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
ZI_DEV i32x16 mfma32_i8(const bf16x8& a, const bf16x8& b, const i32x16& c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// fp32 product rounded on its own: the optimizer cannot fuse it into a later
// add (HIP contracts a*b + c into one fma across statements by default).
ZI_DEV float mul_rn(float a, float b) {
  float r;
  asm("v_mul_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Symmetric per-row int8 quantization of the block projections' operands:
// for a row with amax = max |v|, scale = amax / 127 and inv = 127 / amax
// (each one correctly rounded fp32 division), code = rint(v * inv) clamped
// to [-127, 127] (rint: half to even); an all-zero row has scale 0, codes 0.
// Callers pass amax as NaN when the row holds a NaN or an infinity, which
// gives a NaN scale, so the fault stays visible downstream.
ZI_DEV void quant_params(float amax, float& scale, float& inv) {
  const bool z = amax == 0.f;
  scale = z ? 0.f : __fdiv_rn(amax, 127.0f);
  inv = z ? 0.f : __fdiv_rn(127.0f, amax);
}
ZI_DEV uint32_t quant_code(float v, float inv) {
  const float q = fminf(fmaxf(rintf(__fmul_rn(v, inv)), -127.f), 127.f);
  return (uint32_t)((int)q) & 0xffu;
}
ZI_DEV uint32_t quant4(float a, float b, float c, float d, float inv) {
  return quant_code(a, inv) | (quant_code(b, inv) << 8) | (quant_code(c, inv) << 16) | (quant_code(d, inv) << 24);
}

// Barrier that publishes direct loads into LDS: each wave first waits for
// its own outstanding loads (vmcnt), then all waves meet.  Written out
// explicitly because the compiler does not always place that wait before a
// loop-header barrier, and a wave's wait covers only its own loads.
ZI_DEV void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// One 16-byte-per-lane direct-to-LDS load through a raw buffer resource
// (base, extent in bytes; the per-lane offset in a register, a uniform offset
// in a scalar): lanes whose byte offset reaches past the extent read zeros.
// The buffer form is counted on the vector-memory counter only; the flat
// (global_load_lds) form is taken by the compiler as a possible LDS access
// of unknown order, after which it can only wait for all LDS reads at once.
// Lanes write LDS at lds + 16 * lane (the wave-uniform base goes to M0).
ZI_DEV void buffer_load_lds16(const void* base, int extent, void* lds, uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, extent,
                                                                     0x00020000);  // raw dword access
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// v from lane (lane ^ M) of the same 16-lane row, by DPP moves: quad
// permutations for 1 and 2 (and 3), a half-row mirror (lane ^ 7) after a
// quad xor 3 for 4, a row rotation by 8 for 8 (every source lane is inside
// the row, so bound_ctrl never applies)
template <int CTRL>
ZI_DEV float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int M>
ZI_DEV float lane_xor(float v) {
  if constexpr (M == 1) return dpp_mov<0xb1>(v);                 // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp_mov<0x4e>(v);            // quad_perm [2,3,0,1]
  else if constexpr (M == 4) return dpp_mov<0x141>(dpp_mov<0x1b>(v));  // quad [3,2,1,0], half-row mirror
  else return dpp_mov<0x128>(v);                                 // row_ror:8
}

ZI_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
ZI_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over a whole workgroup of NT threads (NT a multiple of 64); ``red`` is
// LDS scratch of NT/64 floats.  Every thread gets the total.
template <int NT>
ZI_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i % 8).  Renumber so that each XCD receives a contiguous range of
// logical ids, keeping tiles that share operands in one L2.
ZI_DEV int xcd_remap(int bid, int nblocks) {
  const int xcd = bid & 7;
  const int idx = bid >> 3;
  const int per = nblocks >> 3;
  const int rem = nblocks & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}
