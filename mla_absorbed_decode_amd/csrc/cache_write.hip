// cache_write.hip -- the latent-cache write kernels: the copy of bits (one
// item per thread; the write itself is in cache_write.h) and the fp8 write
// (vLLM "test_mla_cross_layer_kernel_equivalence.py": concat_and_cache_mla's
// cache dtype and scale arguments; the dense fp8 decode tests read such a
// cache as torch.float8_e4m3fn).
#include "cache_write.h"

namespace mla {
namespace {

template <int VEC>
__global__ void __launch_bounds__(256) cache_write_kernel(CacheWriteParams p) {
  cache_write_item<VEC>(p, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// fp8 write: item idx stores G consecutive elements of one token's row (all in
// kv_c or all in k_pe, since L and R are multiples of G) as e4m3(x / scale),
// the quotient taken in float. G = 8 moves 16-byte (bf16) or two 16-byte
// (f32) reads and one 8-byte write; G = 1 serves unaligned rows.
template <int G, bool F32>
__global__ void __launch_bounds__(256) cache_write_fp8_kernel(CacheWriteParams p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gpr = (p.L + p.R) / G;
  if (idx >= p.T * gpr) return;
  const int64_t t = idx / gpr, c = (idx % gpr) * G;
  const char* src = c < p.L ? (const char*)p.kv_c + (t * p.kv_c_s0 + c) * (F32 ? 4 : 2)
                            : (const char*)p.k_pe + (t * p.k_pe_s0 + (c - p.L)) * (F32 ? 4 : 2);
  float x[8];
  if constexpr (G == 8) {
    if constexpr (F32) {
      const f32x4_t a = ((const f32x4_t*)src)[0], b = ((const f32x4_t*)src)[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
      }
    } else {
      const u32x4_t v = *(const u32x4_t*)src;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_to_f32((uint16_t)(v[i] & 0xffffu));
        x[2 * i + 1] = bf16_to_f32((uint16_t)(v[i] >> 16));
      }
    }
  } else {
    x[0] = F32 ? *(const float*)src : bf16_to_f32(*(const uint16_t*)src);
  }
  const int64_t slot = p.slot_is_i64 ? ((const int64_t*)p.slots)[t] : (int64_t)((const int32_t*)p.slots)[t];
  if (slot < 0 || slot >= p.num_blocks * p.page) return;
  const float sc = *p.fp8_scale;
  const int64_t blk = slot / p.page, off = slot % p.page;
  char* dst = (char*)p.cache + blk * p.cache_s0 + off * p.cache_s1 + c;
  if constexpr (G == 8) {
    *(u32x2_t*)dst = u32x2_t{e4m3_pack4(x[0] / sc, x[1] / sc, x[2] / sc, x[3] / sc),
                             e4m3_pack4(x[4] / sc, x[5] / sc, x[6] / sc, x[7] / sc)};
  } else {
    *(uint8_t*)dst = (uint8_t)(e4m3_pack4(x[0] / sc, 0.f, 0.f, 0.f) & 0xffu);
  }
}

template <int G>
hipError_t launch_fp8(const CacheWriteParams& p, hipStream_t s) {
  const int64_t blocks = (p.T * ((p.L + p.R) / G) + 255) / 256;
  if (p.esize == 4) hipLaunchKernelGGL((cache_write_fp8_kernel<G, true>), dim3(blocks), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((cache_write_fp8_kernel<G, false>), dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (p.fp8_scale) return p.vec16 ? launch_fp8<8>(p, s) : launch_fp8<1>(p, s);
  const int vec = p.vec16 ? 16 : p.esize;
  const int64_t blocks = (cache_write_items(p) + 255) / 256;
  if (vec == 16) hipLaunchKernelGGL(cache_write_kernel<16>, dim3(blocks), dim3(256), 0, s, p);
  else if (vec == 4) hipLaunchKernelGGL(cache_write_kernel<4>, dim3(blocks), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(cache_write_kernel<2>, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
