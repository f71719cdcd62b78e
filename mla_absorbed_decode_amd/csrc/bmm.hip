// bmm.hip -- the two absorption folds as strided batched matmuls on gfx950
// (vllm.cpp "tests/vt/test_ops_mla_absorb.cpp": the q-side W_UK fold and the
// W_UV un-projection, both batched over heads with transposed operand views;
// memra-engine 0.124.1 "tests/mla_gpu_forward.rs": mla_absorb_q and
// mla_decompress_v).
//
//   out[t, h, n] = sum_k a[t, h, k] * w[h, k, n]
// optionally followed (absorb_q) by the bit copy of the rope rows
//   out[t, h, N + r] = pe[t, h or 0, r].
//
// bf16: a 64 (tokens) x 64 (outputs) tile per workgroup of 4 waves, K in steps
// of 32. The weight tile is streamed global->LDS (two buffers); each wave
// reads its token rows of `a` straight from memory as the MFMA A operand and
// the weight tile with ds_read_b64_tr_b16, which turns the n-contiguous weight
// rows into the k-contiguous B operand of v_mfma_f32_16x16x32_bf16. fp32 uses
// v_mfma_f32_16x16x4_f32 on the same tiling (one element per lane, no
// transpose needed). Sizes the MFMA tiling does not cover (K not a multiple of
// 32, N not a multiple of 16) take a plain one-thread-per-output kernel.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kTM = 64, kTN = 64, kKB = 32;

__device__ __forceinline__ int wswz(int r) { return 2 * (r & 3); }  // bf16 weight-tile chunk swizzle

template <class T>
__device__ __forceinline__ void copy_rope(const BmmParams& p, int t0, int h) {
  // out[t, h, N + r] = pe[t, h', r] for the tile's tokens (bit copy)
  const int nt = (int)(p.T - t0 < kTM ? p.T - t0 : kTM);
  for (int e = threadIdx.x; e < nt * p.R; e += blockDim.x) {
    const int t = t0 + e / (int)p.R, r = e % (int)p.R;
    const T* src = (const T*)p.pe + (int64_t)t * p.pe_st + (int64_t)h * p.pe_sh + r;
    T* dst = (T*)p.out + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + p.N + r;
    *dst = *src;
  }
}

__global__ void __launch_bounds__(256) bmm_bf16_mfma(BmmParams p) {
  __shared__ __attribute__((aligned(16))) char wt[2][kKB * kTN * 2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
  const int n0 = blockIdx.x * kTN, t0 = blockIdx.y * kTM, h = blockIdx.z;
  const uint16_t* W = (const uint16_t*)p.w + (int64_t)h * p.w_sh;
  // this thread's 16-byte slot of the LDS weight tile: row wr, position wpos
  const int wr = threadIdx.x >> 3, wpos = threadIdx.x & 7;
  int wcol = n0 + 8 * (wpos ^ wswz(wr));
  if (wcol + 8 > p.N) wcol = (int)p.N - 8;  // columns past N are never stored
  const int t = t0 + 16 * w + li;
  const bool tvalid = t < p.T;
  const uint16_t* arow = (const uint16_t*)p.a + (int64_t)(tvalid ? t : 0) * p.a_st +
                         (int64_t)h * p.a_sh + 8 * g;
  const int nk = (int)(p.K / kKB);
  f32x4_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  i16x8_t av = tvalid ? *(const i16x8_t*)arow : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  load_lds_16(W + (int64_t)wr * p.w_sk + wcol, (MLA_LDS char*)&wt[0][w * 1024]);
  for (int kb = 0; kb < nk; ++kb) {
    wait_vmcnt<0>();
    __syncthreads();  // tile kb visible to every wave; all waves are done with kb-1
    const i16x8_t acur = av;
    if (kb + 1 < nk) {
      av = tvalid ? *(const i16x8_t*)(arow + (kb + 1) * kKB) : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      load_lds_16(W + (int64_t)((kb + 1) * kKB + wr) * p.w_sk + wcol,
                  (MLA_LDS char*)&wt[(kb + 1) & 1][w * 1024]);
    }
    const MLA_LDS char* tile = (const MLA_LDS char*)wt[kb & 1];
    const int rlo = 8 * g + (li >> 2), rhi = rlo + 4;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int c = 2 * nt + ((li & 3) >> 1);
      const i16x4_t b0 = lds_read_tr16(tile + rlo * 128 + ((c ^ wswz(rlo)) << 4) + (li & 1) * 8);
      const i16x4_t b1 = lds_read_tr16(tile + rhi * 128 + ((c ^ wswz(rhi)) << 4) + (li & 1) * 8);
      const i16x8_t bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      acc[nt] = mfma_16x16x32(acur, bv, acc[nt]);
    }
  }
  // lane holds out[t0 + 16w + 4g + j][n0 + 16nt + li]
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = n0 + 16 * nt + li;
    if (n >= p.N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + 16 * w + 4 * g + j;
      if (tt < p.T)
        ((uint16_t*)p.out)[(int64_t)tt * p.o_st + (int64_t)h * p.o_sh + n] = f32_to_bf16(acc[nt][j]);
    }
  }
  if (p.R > 0 && blockIdx.x == 0) copy_rope<uint16_t>(p, t0, h);
}

__global__ void __launch_bounds__(256) bmm_f32_mfma(BmmParams p) {
  __shared__ __attribute__((aligned(16))) float wt[2][kKB * kTN];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
  const int n0 = blockIdx.x * kTN, t0 = blockIdx.y * kTM, h = blockIdx.z;
  const float* W = (const float*)p.w + (int64_t)h * p.w_sh;
  const int t = t0 + 16 * w + li;
  const bool tvalid = t < p.T;
  const float* arow = (const float*)p.a + (int64_t)(tvalid ? t : 0) * p.a_st + (int64_t)h * p.a_sh + 4 * g;
  const int nk = (int)(p.K / kKB);
  f32x4_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the 32 x 64 float tile is 512 16-byte chunks: two per thread, slot = threadIdx.x + 256 * i
  auto issue = [&](int kb, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot = threadIdx.x + 256 * i;
      const int r = slot >> 4, c = slot & 15;
      int col = n0 + 4 * c;
      if (col + 4 > p.N) col = (int)p.N - 4;
      load_lds_16(W + (int64_t)(kb * kKB + r) * p.w_sk + col,
                  (MLA_LDS char*)&wt[buf][0] + (i * 256 + w * 64) * 16);
    }
  };
  f32x4_t a0 = tvalid ? *(const f32x4_t*)arow : f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t a1 = tvalid ? *(const f32x4_t*)(arow + 16) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  issue(0, 0);
  for (int kb = 0; kb < nk; ++kb) {
    wait_vmcnt<0>();
    __syncthreads();
    const f32x4_t c0 = a0, c1 = a1;
    if (kb + 1 < nk) {
      const float* an = arow + (kb + 1) * kKB;
      a0 = tvalid ? *(const f32x4_t*)an : f32x4_t{0.f, 0.f, 0.f, 0.f};
      a1 = tvalid ? *(const f32x4_t*)(an + 16) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      issue(kb + 1, (kb + 1) & 1);
    }
    const MLA_LDS float* tile = (const MLA_LDS float*)wt[kb & 1];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        // k = 4g + x (first half) and 16 + 4g + x (second half)
        acc[nt] = mfma_16x16x4f32(c0[x], tile[(4 * g + x) * kTN + 16 * nt + li], acc[nt]);
        acc[nt] = mfma_16x16x4f32(c1[x], tile[(16 + 4 * g + x) * kTN + 16 * nt + li], acc[nt]);
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = n0 + 16 * nt + li;
    if (n >= p.N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + 16 * w + 4 * g + j;
      if (tt < p.T) ((float*)p.out)[(int64_t)tt * p.o_st + (int64_t)h * p.o_sh + n] = acc[nt][j];
    }
  }
  if (p.R > 0 && blockIdx.x == 0) copy_rope<uint32_t>(p, t0, h);
}

// Any sizes: one thread per output element, fp32 accumulation in k order.
template <bool F32>
__global__ void __launch_bounds__(256) bmm_plain(BmmParams p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = p.T * p.H * p.N;
  if (idx < total) {
    const int64_t n = idx % p.N, th = idx / p.N, h = th % p.H, t = th / p.H;
    float acc = 0.f;
    for (int64_t k = 0; k < p.K; ++k) {
      float x, y;
      if constexpr (F32) {
        x = ((const float*)p.a)[t * p.a_st + h * p.a_sh + k];
        y = ((const float*)p.w)[h * p.w_sh + k * p.w_sk + n];
      } else {
        x = bf16_to_f32(((const uint16_t*)p.a)[t * p.a_st + h * p.a_sh + k]);
        y = bf16_to_f32(((const uint16_t*)p.w)[h * p.w_sh + k * p.w_sk + n]);
      }
      acc = fmaf(x, y, acc);
    }
    if constexpr (F32) ((float*)p.out)[t * p.o_st + h * p.o_sh + n] = acc;
    else ((uint16_t*)p.out)[t * p.o_st + h * p.o_sh + n] = f32_to_bf16(acc);
  }
  // rope rows: one thread per (t, h, r) element, in the blocks after the products
  const int64_t ridx = idx - ((total + 255) / 256) * 256;
  if (p.R > 0 && ridx >= 0 && ridx < p.T * p.H * p.R) {
    const int64_t r = ridx % p.R, th = ridx / p.R, h = th % p.H, t = th / p.H;
    if constexpr (F32)
      ((uint32_t*)p.out)[t * p.o_st + h * p.o_sh + p.N + r] =
          ((const uint32_t*)p.pe)[t * p.pe_st + h * p.pe_sh + r];
    else
      ((uint16_t*)p.out)[t * p.o_st + h * p.o_sh + p.N + r] =
          ((const uint16_t*)p.pe)[t * p.pe_st + h * p.pe_sh + r];
  }
}

}  // namespace

hipError_t launch_bmm(const BmmParams& p, hipStream_t s) {
  if (p.T == 0 || p.H == 0) return hipSuccess;
  const int64_t es = p.is_f32 ? 4 : 2;
  // the MFMA path reads 16-byte vectors from a and w rows
  const bool aligned =
      ((uintptr_t)p.a % 16 == 0) && ((uintptr_t)p.w % 16 == 0) && (p.a_st * es % 16 == 0) &&
      (p.a_sh * es % 16 == 0) && (p.w_sh * es % 16 == 0) && (p.w_sk * es % 16 == 0);
  const bool mfma_ok = aligned && p.K % kKB == 0 && p.N % 16 == 0 && p.N >= 16;
  if (mfma_ok) {
    dim3 grid((unsigned)((p.N + kTN - 1) / kTN), (unsigned)((p.T + kTM - 1) / kTM), (unsigned)p.H);
    if (p.is_f32) hipLaunchKernelGGL(bmm_f32_mfma, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(bmm_bf16_mfma, grid, dim3(256), 0, s, p);
  } else {
    const int64_t total = p.T * p.H * p.N;
    const int64_t blocks = (total + 255) / 256 + (p.T * p.H * p.R + 255) / 256;
    if (p.is_f32) hipLaunchKernelGGL(bmm_plain<true>, dim3((unsigned)blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(bmm_plain<false>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mla
