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
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define MLA_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- bf16
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// f32 -> bf16 pairs with gfx950's v_cvt_pk_bf16_f32 (round to nearest even,
// NaN stays NaN); the compiler selects it for these conversions.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// ----------------------------------------------------------------- fp8
// OCP FP8 E4M3 ("e4m3fn": bias 7, subnormals m * 2^-9, S.1111.111 NaN, no
// infinities, largest magnitude 448), the format of gfx950's fp8 conversions.
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Eight e4m3 values (bytes 0..7 of v) as eight bf16 values: every e4m3 value
// is exact in bf16, so the widening is exact (NaN stays NaN).
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(u32x2_t v) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[0], false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[0], true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[1], false);
  const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[1], true);
  return u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]), pack_bf16x2(c[0], c[1]),
                 pack_bf16x2(d[0], d[1])};
}

// Four floats to e4m3 codes (byte i of the result from x[i]): nearest value,
// ties to the even mantissa (the hardware conversion), magnitudes above 448
// saturate (the conversion alone would give NaN), NaN gives S.1111.111 with
// the input's sign.
__device__ __forceinline__ uint32_t e4m3_pack4(float x0, float x1, float x2, float x3) {
  auto sat = [](float v) { return __builtin_isnan(v) ? 0.f : fminf(fmaxf(v, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(x0), sat(x1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(x2), sat(x3), w, true);
  uint32_t r = (uint32_t)w;
  const float xs[4] = {x0, x1, x2, x3};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (__builtin_isnan(xs[i])) {
      const uint32_t code = (__builtin_bit_cast(uint32_t, xs[i]) >> 31) ? 0xffu : 0x7fu;
      r = (r & ~(0xffu << (8 * i))) | (code << (8 * i));
    }
  return r;
}

// ---------------------------------------------------------------- MFMA
// 16x16x32 bf16 -> f32. Lane l holds A[l%16][8*(l/16)+i], B[8*(l/16)+i][l%16]
// (i = 0..7) and receives D[4*(l/16)+j][l%16] (j = 0..3).
__device__ __forceinline__ f32x4_t mfma_16x16x32(i16x8_t a, i16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// 32x32x16 bf16 -> f32. Lane l holds A[l%32][8*(l/32)+i], B[8*(l/32)+i][l%32]
// (i = 0..7) and receives D[8*(r/4) + 4*(l/32) + r%4][l%32] (r = 0..15).
__device__ __forceinline__ f32x16_t mfma_32x32x16(i16x8_t a, i16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
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
// lives at chunk position c ^ swz(r), swz(r) = r mod 8. Rows are 1152 B
// apart. The K operand reads 16 rows at one chunk per 16 lanes (four chunk
// groups per instruction) and the transposed V operand 4 consecutive rows x 2
// adjacent chunks per 16 lanes. Measured on MI355X with a probe that runs each
// lane-address pattern from 16 waves at once: with swz = r mod 8 the K
// pattern reads a 1 KB ds_read_b128 in 4.3 CU cycles, the same as 64 lanes
// reading one contiguous 1 KB; the transposed reads take 1.5 cycles with any
// of the permutations tried. A permutation chosen for a 32- or 64-bank model
// (rows 8-15 the rows 0-7 values xor 1) took 8.0 cycles.
__device__ __forceinline__ int lds_swz(int r) { return r & 7; }

// --------------------------------------------------------------- waits
// Wait until at most N vector-memory operations of this wave are in flight
// (vmcnt <= N; expcnt and lgkmcnt are left unconstrained). Vector loads
// complete in issue order, so this retires every load issued before the last N.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// vmcnt <= n * STEP for a wave-uniform n >= 0 (n above MAXN counts as MAXN).
template <int MAXN, int STEP>
__device__ __forceinline__ void wait_vmcnt_n(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      wait_vmcnt<MAXN * STEP>();
      return;
    }
    wait_vmcnt_n<MAXN - 1, STEP>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// Global -> LDS 16-byte load: each lane's 16 bytes land at lds_base + 16*lane
// (lds_base must be wave-uniform; it goes to M0). Issued as inline assembly so
// the compiler's wait insertion does not model it: callers wait for these
// loads themselves with wait_vmcnt<>. The compiler's own vector-memory waits
// stay correct because vector memory operations complete in issue order.
// STREAM sets the non-temporal cache policy, for data read exactly once (the
// latent rows): measured on MI355X, a grid streaming 1 GiB this way reaches
// 6.9 TB/s against 6.1 TB/s with the default policy.
template <bool STREAM = false>
__device__ __forceinline__ void load_lds_16(const void* gptr, MLA_LDS void* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  if (STREAM)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(gptr), "s"(m0v)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(m0v)
                 : "memory", "m0");
}

// The same load addressed as a wave-uniform 64-bit base (an SGPR pair, see
// uniform_ptr) plus a per-lane 32-bit byte offset: no per-lane 64-bit address
// arithmetic.
__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
  // readfirstlane returns a signed int: widen each half through uint32_t
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
template <bool STREAM = false>
__device__ __forceinline__ void load_lds_16_sbase(uint64_t sbase, uint32_t voff,
                                                  MLA_LDS void* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  if (STREAM)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
}

// 16-byte global load into registers, as an ordinary load: the compiler
// places the wait before the first use. Its wait does not see the LDS DMA
// reads above (they are inline assembly), so it may retire those too.
template <class T>
__device__ __forceinline__ void load_16(T& dst, const void* gptr) {
  static_assert(sizeof(T) == 16, "16-byte register");
  dst = *(const T*)gptr;
}

// Reductions over lanes {l, l^16, l^32, l^48} with gfx950's permlane swaps:
// v_permlane32_swap a, b exchanges a's upper 32 lanes with b's lower 32, so
// with a = b = v it leaves (v[l & ~32], v[l | 32]) in (a, b); v_permlane16_swap
// does the same for 16-lane halves. Both are plain VALU. They are issued as
// inline assembly with both registers as in/out operands (the compiler's
// builtin for them merged the two results into one), with the wait states
// the instruction needs around it.
__device__ __forceinline__ void lane_pairs(float v, int width, float& a, float& b) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  if (width == 32)
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  else
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float wave_max16(float v) {
  float a, b;
  lane_pairs(v, 32, a, b);
  v = fmaxf(a, b);
  lane_pairs(v, 16, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum16(float v) {
  float a, b;
  lane_pairs(v, 32, a, b);
  v = a + b;
  lane_pairs(v, 16, a, b);
  return a + b;
}

// Element e of a value row (bf16 bits or f32) as a double, and back (RNE).
template <bool F32>
__device__ __forceinline__ double load_value(const void* row, int64_t e) {
  if constexpr (F32) return (double)((const float*)row)[e];
  else return (double)bf16_to_f32(((const uint16_t*)row)[e]);
}
template <bool F32>
__device__ __forceinline__ void store_value(void* row, int64_t e, double v) {
  if constexpr (F32) ((float*)row)[e] = (float)v;
  else ((uint16_t*)row)[e] = f32_to_bf16((float)v);
}

// Interleaved rotary embedding of one pair (a, b) = (x[2i], x[2i+1]) of a
// d-wide vector at position pos (memra-engine 0.124.1 "tests/mla_gpu_forward.rs",
// gate 3): theta = pos * base^(-2i/d), (a, b) -> (a cos - b sin, a sin + b cos).
// The frequency, the angle and its reduction to [-pi, pi] are computed in
// double and the rotation too, so the single rounding to the output type is
// the only error that matters even for positions in the millions.
__device__ __forceinline__ void rope_angle(double& sn, double& cs, int pos, int i, int d,
                                           double log2_base) {
  const double freq = exp2(-(2.0 * i / d) * log2_base);
  const double theta = (double)pos * freq;
  constexpr double kTwoPi = 6.283185307179586476925;
  const double r = theta - kTwoPi * rint(theta * (1.0 / kTwoPi));
  sincos(r, &sn, &cs);
}
__device__ __forceinline__ void rope_rotate(double& a, double& b, int pos, int i, int d,
                                            double log2_base) {
  double sn, cs;
  rope_angle(sn, cs, pos, i, d, log2_base);
  const double x = a * cs - b * sn, y = a * sn + b * cs;
  a = x;
  b = y;
}

}  // namespace mla
