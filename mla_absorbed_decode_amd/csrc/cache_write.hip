// cache_write.hip -- the latent-cache write kernel (one item per thread; the
// write itself is in cache_write.h).
#include "cache_write.h"

namespace mla {
namespace {

template <int VEC>
__global__ void __launch_bounds__(256) cache_write_kernel(CacheWriteParams p) {
  cache_write_item<VEC>(p, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const int vec = p.vec16 ? 16 : p.esize;
  const int64_t blocks = (cache_write_items(p) + 255) / 256;
  if (vec == 16) hipLaunchKernelGGL(cache_write_kernel<16>, dim3(blocks), dim3(256), 0, s, p);
  else if (vec == 4) hipLaunchKernelGGL(cache_write_kernel<4>, dim3(blocks), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(cache_write_kernel<2>, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
