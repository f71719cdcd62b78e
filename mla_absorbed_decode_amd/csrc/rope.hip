// rope.hip -- interleaved rotary position embedding, in place (memra-engine
// 0.124.1 "tests/mla_gpu_forward.rs", gate 3, gpu_mla_rope_interleaved_matches_cpu:
// vectors of d_rope 8 or 64 at positions 13 * p, base 8e6; d_rope 0 is a no-op).
//
// Pair (2i, 2i+1) of token t's vectors turns by positions[t] * base^(-2i/d).
// The angle's sine and cosine are computed once per (token, pair), in double,
// and applied to the pair in each of the token's V vectors (read, rotated in
// double, rounded once to the storage type). Rows with 16-byte aligned starts
// take 16-byte accesses (rope_kernel_vec); others one pair per access.
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "value_round.h"

namespace mla {
namespace {

template <bool F32, bool PAIR>
__global__ void __launch_bounds__(256) rope_kernel(RopeParams p) {
  const int64_t half = p.d / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.T * half) return;
  const int i = (int)(idx % half);
  const int64_t t = idx / half;
  double sn, cs;
  rope_angle(sn, cs, p.rope.pos[t], i, p.d, p.rope.log2_base);
  constexpr int ES = F32 ? 4 : 2;
  constexpr int U = 8;  // vectors whose pairs are read before any is written back
  for (int64_t v0 = 0; v0 < p.V; v0 += U) {
    double a[U], b[U];
    // pair type: both elements in one access when pairs are aligned
    typedef typename std::conditional<F32, uint64_t, uint32_t>::type PairBits;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (v0 + j < p.V) {
        const char* row = (const char*)p.x + (t * p.s0 + (v0 + j) * p.s1) * ES;
        if (PAIR) {
          const PairBits w = *(const PairBits*)(row + 2 * i * ES);
          a[j] = load_value<F32>(&w, 0);
          b[j] = load_value<F32>(&w, 1);
        } else {
          a[j] = load_value<F32>(row, 2 * i);
          b[j] = load_value<F32>(row, 2 * i + 1);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (v0 + j < p.V) {
        char* row = (char*)p.x + (t * p.s0 + (v0 + j) * p.s1) * ES;
        if (PAIR) {
          PairBits w;
          store_rounded<F32>(&w, 0, a[j] * cs - b[j] * sn);
          store_rounded<F32>(&w, 1, a[j] * sn + b[j] * cs);
          *(PairBits*)(row + 2 * i * ES) = w;
        } else {
          store_rounded<F32>(row, 2 * i, a[j] * cs - b[j] * sn);
          store_rounded<F32>(row, 2 * i + 1, a[j] * sn + b[j] * cs);
        }
      }
    }
  }
}

// 16-byte rows (aligned starts, d a multiple of one piece): one thread per
// (token, 16-byte piece of the rope vector), i.e. 4 bf16 or 2 f32 pairs. Their
// angles are computed once, in double, and applied to that piece of each of
// the token's V vectors with 16-byte reads and writes, 8 vectors read before
// any is written back. Same arithmetic per element as rope_kernel.
template <bool F32>
__global__ void __launch_bounds__(256) rope_kernel_vec(RopeParams p) {
  constexpr int ES = F32 ? 4 : 2;
  constexpr int PP = 16 / (2 * ES);  // pairs per 16-byte piece
  const int64_t pieces = p.d / (2 * PP);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.T * pieces) return;
  const int c = (int)(idx % pieces);
  const int64_t t = idx / pieces;
  double sn[PP], cs[PP];
#pragma unroll
  for (int k = 0; k < PP; ++k) rope_angle(sn[k], cs[k], p.rope.pos[t], PP * c + k, p.d, p.rope.log2_base);
  constexpr int U = 8;
  for (int64_t v0 = 0; v0 < p.V; v0 += U) {
    u32x4_t w[U];
#pragma unroll
    for (int j = 0; j < U; ++j)
      if (v0 + j < p.V)
        w[j] = *(const u32x4_t*)((const char*)p.x + (t * p.s0 + (v0 + j) * p.s1) * ES + 16 * c);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (v0 + j >= p.V) continue;
      u32x4_t o;
#pragma unroll
      for (int k = 0; k < PP; ++k) {
        const double a = load_value<F32>(&w[j], 2 * k), b = load_value<F32>(&w[j], 2 * k + 1);
        store_rounded<F32>(&o, 2 * k, a * cs[k] - b * sn[k]);
        store_rounded<F32>(&o, 2 * k + 1, a * sn[k] + b * cs[k]);
      }
      *(u32x4_t*)((char*)p.x + (t * p.s0 + (v0 + j) * p.s1) * ES + 16 * c) = o;
    }
  }
}

}  // namespace

hipError_t launch_rope(const RopeParams& p, hipStream_t s) {
  const int64_t pairs = p.T * (p.d / 2);
  if (pairs == 0 || p.V == 0) return hipSuccess;
  const int64_t es = p.is_f32 ? 4 : 2;
  const int64_t piece_elems = 16 / es;  // elements per 16-byte piece
  const bool vec16 = (uintptr_t)p.x % 16 == 0 && (p.s0 * es) % 16 == 0 && (p.s1 * es) % 16 == 0 &&
                     p.d % piece_elems == 0;
  if (vec16) {
    const int64_t blocks = (p.T * (p.d / piece_elems) + 255) / 256;
    if (p.is_f32) hipLaunchKernelGGL((rope_kernel_vec<true>), dim3(blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((rope_kernel_vec<false>), dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  const int64_t blocks = (pairs + 255) / 256;
  if (p.is_f32 && p.pair_aligned)
    hipLaunchKernelGGL((rope_kernel<true, true>), dim3(blocks), dim3(256), 0, s, p);
  else if (p.is_f32)
    hipLaunchKernelGGL((rope_kernel<true, false>), dim3(blocks), dim3(256), 0, s, p);
  else if (p.pair_aligned)
    hipLaunchKernelGGL((rope_kernel<false, true>), dim3(blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((rope_kernel<false, false>), dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
