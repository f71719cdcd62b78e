/* mla_probe.h -- measurement probes of libmla_probe.so (not part of the MLA
 * attention interface in mla.h).
 *
 * The benchmark quotes each kernel against the published MI355X peaks and
 * also against the peaks these probes measure on the GPU it runs on: the
 * dense bf16 matrix-core rate and the HBM copy and read rates, and the cost of
 * the few-head decode's tile stream alone. Each enqueues one kernel
 * on `stream` and return at once; the caller times them (HIP events) and
 * owns every buffer. Return value: 0 on success, -1 for a NULL pointer, -5
 * for an argument outside the supported range, -7 for a HIP error.
 */
#ifndef MLA_PROBE_H
#define MLA_PROBE_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 MFMA throughput. One workgroup per compute unit, 4 *
 * waves_per_simd waves (1 <= waves_per_simd <= 4); every wave issues `iters`
 * (> 0) rounds of independent MFMAs with fp32 accumulation:
 * v_mfma_f32_16x16x32_bf16 (shape 0, eight chains) or
 * v_mfma_f32_32x32x16_bf16 (shape 1, four chains). sink: device buffer of at
 * least workgroups * 256 * waves_per_simd floats (written so that no work is
 * dead). On return *workgroups holds the grid size and *flops the flops the
 * launch performs (2 * M * N * K per instruction). */
int mla_probe_mfma_bf16(float* sink, int shape, int iters, int waves_per_simd, int* workgroups,
                        double* flops, hipStream_t stream);

/* Device copy of `bytes` (a multiple of 16; both pointers 16-byte aligned)
 * from src to dst with 16-byte non-temporal loads and stores, 8 workgroups
 * of 256 threads per compute unit. The HBM traffic is 2 * bytes. */
int mla_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

/* HBM read rate: a grid of workgroups_per_cu (1..32) workgroups of 256
 * threads per compute unit reads `bytes` (a multiple of 16; src 16-byte
 * aligned) with 16-byte non-temporal loads, eight in flight per thread, and
 * writes one word per thread to sink (at least cus * workgroups_per_cu * 256
 * words). The HBM traffic is `bytes`. */
int mla_probe_read(uint32_t* sink, const void* src, size_t bytes, int workgroups_per_cu,
                   hipStream_t stream);

/* The few-head decode's tile stream with no arithmetic: what reading the
 * attention call's latent rows in the partial kernel's partition costs.
 * `workgroups` (1..65535) workgroups of 256 threads; workgroup w reads tiles
 * w * T .. w * T + T - 1 (T = tiles_per_workgroup >= 1) of 36,864 bytes (32
 * rows of 576 bf16), tile t being half t % 2 of page page_perm[t / 2] of src,
 * whose pages are 73,728 bytes. The reads go global -> LDS with 16-byte
 * non-temporal loads into a three-slot ring, two tiles in flight, one
 * workgroup barrier per tile, as the partial kernel issues them. The caller
 * owns and sizes every buffer: page_perm (device) holds
 * ceil(workgroups * T / 2) page indices, each below the page count of src
 * (16-byte aligned); sink (device) takes one word per workgroup. The HBM
 * traffic is workgroups * T * 36,864 bytes. */
int mla_probe_tile_stream(uint32_t* sink, const void* src, const int32_t* page_perm,
                          int tiles_per_workgroup, int workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROBE_H */
