// value_round.h -- one correct rounding of a double to the storage types of
// the rotary-embedding paths: f32 round-to-nearest-even, and bf16
// round-to-nearest-even of the exact double, not of its float rounding. The
// bf16 case first rounds to float "to odd" (an inexact result takes whichever
// float neighbour has an odd significand), then to bf16 to nearest even;
// rounding to odd with at least two more significand bits than the final
// format makes the second rounding equal to one direct rounding (Boldo and
// Melquiond, "When double rounding is odd", 2005). A plain double -> float ->
// bf16 conversion can land on a bf16 midpoint and round it to even the wrong
// way. Device code only.
#pragma once

#include "mla_device.h"

namespace mla {

__device__ __forceinline__ float f64_to_f32_odd(double v) {
  float f = (float)v;  // round to nearest even
  if ((double)f != v && !__builtin_isnan(v)) {
    uint32_t bits = __builtin_bit_cast(uint32_t, f);
    if ((bits & 1u) == 0u) {  // even neighbour: take the other one, toward v
      bits += (double)__builtin_fabsf(f) < __builtin_fabs(v) ? 1u : 0xffffffffu;
      f = __builtin_bit_cast(float, bits);
    }
  }
  return f;
}

// Element e of a value row (bf16 bits or f32) set to v, rounded once.
template <bool F32>
__device__ __forceinline__ void store_rounded(void* row, int64_t e, double v) {
  if constexpr (F32) ((float*)row)[e] = (float)v;
  else ((uint16_t*)row)[e] = f32_to_bf16(f64_to_f32_odd(v));
}

}  // namespace mla
