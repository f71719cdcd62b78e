// probe.hip -- the machine measurements the benchmark divides by: the bf16
// matrix-core rate and the HBM copy and read rates of the GPU it runs on. They are not
// part of the attention path; they give the measured peaks that the
// benchmark's roofline fractions are also quoted against, next to the
// published ones. A fourth probe streams tiles with the few-head decode's load
// schedule and no arithmetic: what reading the call's bytes alone costs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"
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

// The few-head decode's load schedule without its arithmetic: workgroup w
// reads tiles w * T .. w * T + T - 1 of kTileBytes each, tile t being half t % 2
// of page page_perm[t / 2] (2 * kTileBytes per page), global -> LDS with
// non-temporal 16-byte loads into a three-slot ring; four waves issue (nine
// 1 KB reads each per tile), two tiles in flight, one barrier per tile.
constexpr int kTileBytes = 32 * 1152;         // 32 latent rows of 576 bf16
constexpr int kTileReads = kTileBytes / 1024;  // 1 KB wave reads per tile
constexpr int kTileSlots = 3;

__global__ void __launch_bounds__(256) tile_stream_kernel(uint32_t* __restrict__ sink,
                                                          const char* __restrict__ base,
                                                          const int32_t* __restrict__ page_perm,
                                                          int tiles_per_workgroup) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  MLA_LDS char* ring = (MLA_LDS char*)smem;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int kPerWave = kTileReads / 4;
  static_assert(kPerWave * 4 == kTileReads, "tile reads split over four waves");
  const int T = tiles_per_workgroup;
  const int64_t t0 = (int64_t)blockIdx.x * T;
  auto issue = [&](int i) {
    const int64_t t = t0 + i;
    const char* a = base + (int64_t)page_perm[t >> 1] * (2 * kTileBytes) + (t & 1) * kTileBytes;
    MLA_LDS char* dst = ring + (i % kTileSlots) * kTileBytes;
#pragma unroll
    for (int n = 0; n < kPerWave; ++n) {
      const int piece = w + 4 * n;
      mla::load_lds_16<true>(a + piece * 1024 + lane * 16, dst + piece * 1024);
    }
  };
  for (int i = 0; i < kTileSlots - 1 && i < T; ++i) issue(i);
  for (int i = 0; i < T; ++i) {
    // tile i has landed; tile i + 1 may stay in flight
    mla::wait_vmcnt_n<kTileSlots - 2, kPerWave>(T - 1 - i);
    __syncthreads();  // every wave's part of tile i is in LDS; the slot of tile i - 1 is free
    if (i + kTileSlots - 1 < T) issue(i + kTileSlots - 1);
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = *(const MLA_LDS uint32_t*)ring;
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

int mla_probe_tile_stream(uint32_t* sink, const void* src, const int32_t* page_perm,
                          int tiles_per_workgroup, int workgroups, hipStream_t stream) {
  if (!sink || !src || !page_perm) return -1;
  if ((uintptr_t)src % 16 || tiles_per_workgroup < 1 || workgroups < 1 || workgroups > 65535)
    return -5;
  static bool attr = false;  // the attribute is per function, set once per process
  if (!attr) {
    if (hipFuncSetAttribute((const void*)tile_stream_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            kTileSlots * kTileBytes) != hipSuccess)
      return -7;
    attr = true;
  }
  hipLaunchKernelGGL(tile_stream_kernel, dim3((unsigned)workgroups), dim3(256),
                     kTileSlots * kTileBytes, stream, sink, (const char*)src, page_perm,
                     tiles_per_workgroup);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
