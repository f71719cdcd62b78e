// cache_write.h -- the latent-cache write as device functions, shared by the
// cache-write kernel and the fold kernel that runs it in extra workgroups
// (one launch for a decode step's q fold and cache write).
//
// Token t's row [kv_c | k_pe] goes to slot_mapping[t] = block * page + offset
// of a paged, possibly block-major cache view (vLLM
// "test_mla_cross_layer_kernel_equivalence.py",
// test_concat_and_cache_mla_into_unified_slot_view; memra-engine 0.124.1
// "tests/mla_gpu_forward.rs", gate 2's latent append, checked bit for bit).
//
// A copy of bits: nothing is converted, so every value, NaN payload and
// signed zero arrives unchanged -- except, when positions are given, the rope
// part, which is written rotated by its token's position (interleaved rope,
// memra-engine 0.124.1 "tests/mla_gpu_forward.rs", gate 3). One item moves
// one 16-byte chunk (or one element when rows are not 16-byte aligned); a
// token whose slot is outside [0, num_blocks * page) is skipped, and nothing
// but the addressed rows is written, so neighbouring layers of a unified slot
// are never touched.
#pragma once

#include <type_traits>

#include "mla_device.h"
#include "value_round.h"
#include "mla_kernels.h"

namespace mla {


// Pair j of the rope part (token j / (R/2), pair j % (R/2)), rotated by the
// token's position (the angle once, in double) and written to its slot.
__device__ __forceinline__ void rope_pair(const CacheWriteParams& p, int64_t j) {
  const int64_t half = p.R / 2;
  if (j >= p.T * half) return;
  const int64_t t = j / half;
  const int i = (int)(j % half);
  const int64_t slot = p.slot_is_i64 ? ((const int64_t*)p.slots)[t] : (int64_t)((const int32_t*)p.slots)[t];
  if (slot < 0 || slot >= p.num_blocks * p.page) return;
  const char* row = (const char*)p.k_pe + t * p.k_pe_s0 * p.esize;
  const int64_t blk = slot / p.page, off = slot % p.page;
  char* dst = (char*)p.cache + (blk * p.cache_s0 + off * p.cache_s1 + p.L) * p.esize;
  if (p.esize == 4) {
    double a = load_value<true>(row, 2 * i), b = load_value<true>(row, 2 * i + 1);
    rope_rotate(a, b, p.rope.pos[t], i, (int)p.R, p.rope.log2_base);
    store_rounded<true>(dst, 2 * i, a);
    store_rounded<true>(dst, 2 * i + 1, b);
  } else {
    double a = load_value<false>(row, 2 * i), b = load_value<false>(row, 2 * i + 1);
    rope_rotate(a, b, p.rope.pos[t], i, (int)p.R, p.rope.log2_base);
    store_rounded<false>(dst, 2 * i, a);
    store_rounded<false>(dst, 2 * i + 1, b);
  }
}

// Work item idx of the write: a kv_c or k_pe chunk of VEC bytes (with
// rotation: a kv_c chunk, or past them one rope pair). Items past the end do
// nothing.
template <int VEC>  // bytes moved per item: 16, or the element size
__device__ __forceinline__ void cache_write_item(const CacheWriteParams& p, int64_t idx) {
  const int64_t es = p.esize;
  const int64_t cl = p.L * es / VEC, cr = p.R * es / VEC, cpr = cl + cr;
  if (p.rope.pos) {
    // kv_c chunks are copied as below; threads past them rotate one rope pair each
    if (idx >= p.T * cl) {
      rope_pair(p, idx - p.T * cl);
      return;
    }
  } else if (idx >= p.T * cpr) {
    return;
  }
  const int64_t t = p.rope.pos ? idx / cl : idx / cpr, c = p.rope.pos ? idx % cl : idx % cpr;
  // the row piece and the slot are independent loads: both go out before either is used
  const char* src = c < cl ? (const char*)p.kv_c + t * p.kv_c_s0 * es + c * VEC
                           : (const char*)p.k_pe + t * p.k_pe_s0 * es + (c - cl) * VEC;
  typedef typename std::conditional<VEC == 16, u32x4_t,
          typename std::conditional<VEC == 4, uint32_t, uint16_t>::type>::type V;
  const V v = *(const V*)src;
  const int64_t slot = p.slot_is_i64 ? ((const int64_t*)p.slots)[t] : (int64_t)((const int32_t*)p.slots)[t];
  if (slot < 0 || slot >= p.num_blocks * p.page) return;
  const int64_t blk = slot / p.page, off = slot % p.page;
  *(V*)((char*)p.cache + (blk * p.cache_s0 + off * p.cache_s1) * es + c * VEC) = v;
}


// Bytes per item of a write: 16 when every row start is 16-byte aligned,
// else one element.
__device__ __forceinline__ int cache_write_vec(const CacheWriteParams& p) {
  return p.vec16 ? 16 : p.esize;
}

// Items of a write (see cache_write_item).
__host__ __device__ inline int64_t cache_write_items(const CacheWriteParams& p) {
  const int64_t vec = p.vec16 ? 16 : p.esize;
  return p.rope.pos ? p.T * (p.L * p.esize / vec) + p.T * (p.R / 2)
                    : p.T * ((p.L + p.R) * p.esize / vec);
}

// Items first, first + stride, ... of a write.
__device__ __forceinline__ void cache_write_range(const CacheWriteParams& p, int64_t first,
                                                  int64_t stride) {
  const int64_t n = cache_write_items(p);
  const int vec = cache_write_vec(p);
  for (int64_t i = first; i < n; i += stride) {
    if (vec == 16) cache_write_item<16>(p, i);
    else if (vec == 4) cache_write_item<4>(p, i);
    else cache_write_item<2>(p, i);
  }
}

}  // namespace mla
