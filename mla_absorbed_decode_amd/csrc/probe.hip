// probe.hip -- the machine measurements the benchmark divides by: the bf16
// matrix-core rate and the HBM copy and read rates of the GPU it runs on. They are not
// part of the attention path; they give the measured peaks that the
// benchmark's roofline fractions are also quoted against, next to the
// published ones.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave: no dependent issue

// Every wave issues `iters` rounds of kChains independent MFMAs; one float per
// lane goes to `sink` so nothing is dead.
template <int SHAPE>
__global__ void mfma_peak_kernel(float* sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(63 - lane + i));
  }
  if constexpr (SHAPE == 0) {
    f32x4_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  } else {
    f32x16_t acc[kChains / 2];
#pragma unroll
    for (int c = 0; c < kChains / 2; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains / 2; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains / 2; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) s += acc[c][j];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  }
}

// Grid-stride copy of 16-byte words, four in flight per thread.
__global__ void __launch_bounds__(256) copy16_kernel(u32x4_t* __restrict__ dst,
                                                     const u32x4_t* __restrict__ src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4_t v0 = __builtin_nontemporal_load(src + i);
    const u32x4_t v1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4_t v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4_t v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + stride);
    __builtin_nontemporal_store(v2, dst + i + 2 * stride);
    __builtin_nontemporal_store(v3, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Grid-stride read of 16-byte words with non-temporal loads, UNROLL in flight
// per thread; one xor of everything read per thread goes to sink.
template <int UNROLL>
__global__ void __launch_bounds__(256) read16_kernel(uint32_t* __restrict__ sink,
                                                     const u32x4_t* __restrict__ src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
    u32x4_t v[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) acc ^= v[k];
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return n;
}

}  // namespace

extern "C" {

int mla_probe_mfma_bf16(float* sink, int shape, int iters, int waves_per_simd, int* workgroups,
                        double* flops, hipStream_t stream) {
  if (!sink || !workgroups || !flops) return -1;
  if ((shape != 0 && shape != 1) || iters <= 0 || waves_per_simd < 1 || waves_per_simd > 4)
    return -5;
  const int cus = cu_count();
  if (cus <= 0) return -7;
  *workgroups = cus;
  const int threads = 256 * waves_per_simd;  // 4 SIMDs per CU
  // flops of one wave-level instruction times instructions per wave
  const double per_inst = shape == 0 ? 2.0 * 16 * 16 * 32 : 2.0 * 32 * 32 * 16;
  const double insts = shape == 0 ? (double)kChains * iters : (double)(kChains / 2) * iters;
  *flops = per_inst * insts * (threads / 64) * (double)cus;
  if (shape == 0)
    hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(cus), dim3(threads), 0, stream, sink, iters);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(cus), dim3(threads), 0, stream, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int mla_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (!dst || !src) return -1;
  if (bytes % 16 || (uintptr_t)dst % 16 || (uintptr_t)src % 16) return -5;
  const int cus = cu_count();
  if (cus <= 0) return -7;
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return 0;
  int64_t grid = (int64_t)cus * 8;
  const int64_t need = (n + 255) / 256;
  if (grid > need) grid = need;
  hipLaunchKernelGGL(copy16_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (u32x4_t*)dst,
                     (const u32x4_t*)src, n);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int mla_probe_read(uint32_t* sink, const void* src, size_t bytes, int workgroups_per_cu,
                   hipStream_t stream) {
  if (!sink || !src) return -1;
  if (bytes % 16 || (uintptr_t)src % 16 || workgroups_per_cu < 1 || workgroups_per_cu > 32)
    return -5;
  const int cus = cu_count();
  if (cus <= 0) return -7;
  const int64_t n = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(read16_kernel<8>, dim3((unsigned)(cus * workgroups_per_cu)), dim3(256), 0,
                     stream, sink, (const u32x4_t*)src, n);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
