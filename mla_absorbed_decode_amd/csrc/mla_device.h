// mla_device.h -- device-side building blocks for the gfx950 kernels of libmla:
// bf16 conversion, MFMA and LDS-transpose wrappers, the LDS tile swizzle and
// the explicit wait used with global->LDS loads. Host code never includes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define MLA_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- bf16
// f32 -> bf16, round to nearest even; NaN stays a quiet NaN of the same sign.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------- MFMA
// 16x16x32 bf16 -> f32. Lane l holds A[l%16][8*(l/16)+i], B[8*(l/16)+i][l%16]
// (i = 0..7) and receives D[4*(l/16)+j][l%16] (j = 0..3).
__device__ __forceinline__ f32x4_t mfma_16x16x32(i16x8_t a, i16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// 16x16x16 bf16 -> f32. Lane l holds A[l%16][4*(l/16)+i], B[4*(l/16)+i][l%16]
// (i = 0..3) and receives D[4*(l/16)+j][l%16].
__device__ __forceinline__ f32x4_t mfma_16x16x16(i16x4_t a, i16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// 16x16x4 f32 -> f32. Lane l holds A[l%16][l/16], B[l/16][l%16] and receives
// D[4*(l/16)+j][l%16].
__device__ __forceinline__ f32x4_t mfma_16x16x4f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------ LDS transpose read
// ds_read_b64_tr_b16: within each group of 16 lanes, local lane s supplies an
// 8-byte address (4 x 16-bit, S[s][0..3]); local lane i receives element j =
// S[4*j + i/4][i%4]. So if local lane s points at row (r0 + s/4), columns
// c0 + 4*(s%4) .. +3 of a row-major 16-bit matrix, lane i receives
// M[r0 + j][c0 + i] for j = 0..3: a 4x16 block read column-wise.
__device__ __forceinline__ i16x4_t lds_read_tr16(const MLA_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4_t*)p);
}

// ------------------------------------------------------------- LDS swizzle
// Latent rows are staged in LDS as rows of 16-byte chunks; chunk c of row r
// lives at chunk position c ^ swz(r). The permutation keeps both access
// patterns of the attention kernel free of bank conflicts: 16 rows read at one
// chunk (the K operand), and 4 rows x 2 adjacent chunks per 16 lanes (the
// transposed V operand), for 32 or 64 banks of 4 bytes.
__device__ __forceinline__ int lds_swz(int r) {
  const int lo = r & 3, hi = (r >> 2) & 1, top = (r >> 3) & 1;
  return ((((lo ^ hi) << 1) | hi) ^ top);
}

// --------------------------------------------------------------- waits
// Wait until at most N vector-memory operations of this wave are in flight
// (vmcnt <= N; expcnt and lgkmcnt are left unconstrained). Vector loads
// complete in issue order, so this retires every load issued before the last N.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Global -> LDS 16-byte load: each lane's 16 bytes land at lds_base + 16*lane.
__device__ __forceinline__ void load_lds_16(const void* gptr, MLA_LDS void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 16, 0, 0);
}

__device__ __forceinline__ float wave_max16(float v) {  // max over lanes l, l^16, l^32, l^48
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace mla
