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
// bf16: a 64 (tokens) x TN (outputs) tile per workgroup of 4 waves. The
// workgroup's whole K x TN weight slab (up to 512 rows of K at a time) is
// staged global->LDS in one burst, and each wave holds its 16 token rows of
// `a` for all those k-steps in registers, so the tile costs one memory round
// trip rather than one per k-step. The slab is read with ds_read_b64_tr_b16,
// which turns the n-contiguous weight rows into the k-contiguous B operand of
// v_mfma_f32_16x16x32_bf16. TN is 64, or 16 when 64-wide tiles would leave
// the chip mostly idle (few heads x few outputs). fp32 uses
// v_mfma_f32_16x16x4_f32 on a 64 x 64 tiling (one element per lane, no
// transpose needed). Sizes the MFMA tiling does not cover (K not a multiple of
// 32, N not a multiple of 16) take a plain one-thread-per-output kernel.
#include "cache_write.h"
#include "gemm_tile.h"
#include "mla_device.h"
#include "mla_kernels.h"
#include "prefill_kernels.h"
#include "value_round.h"

namespace mla {
namespace {

constexpr int kTM = 64, kTN = 64, kKB = 32;

__device__ __forceinline__ int wswz(int r) { return 2 * (r & 3); }  // bf16 weight-tile chunk swizzle

// out[t, h, N + r] = pe[t, h', r] for the tile's tokens (a bit copy), shared by
// the workgroups of one (token tile, head): 16-byte pieces when the rows allow
// it, all of a thread's loads issued before its stores.
template <class T>
// (wx: this workgroup's column tile; the gridDim.x column tiles of a row tile
// share the copy)
__device__ __forceinline__ void copy_rope(const BmmParams& p, int t0, int h, int wx) {
  const int nt = (int)(p.T - t0 < kTM ? p.T - t0 : kTM);
  const int nwg = (int)gridDim.x, tid = (int)(wx * blockDim.x + threadIdx.x);
  const int stride = nwg * (int)blockDim.x;
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte piece
  if (p.rope.pos) {
    // rotated by the token's position: one pair per thread, the angle in double
    constexpr bool F32 = sizeof(T) == 4;
    const int half = (int)p.R / 2;
    for (int e = tid; e < nt * half; e += stride) {
      const int t = t0 + e / half, i = e % half;
      const T* src = (const T*)p.pe + (int64_t)t * p.pe_st + (int64_t)h * p.pe_sh;
      T* dst = (T*)p.out + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + p.N;
      double a = load_value<F32>(src, 2 * i), b = load_value<F32>(src, 2 * i + 1);
      rope_rotate(a, b, p.rope.pos[t], i, (int)p.R, p.rope.log2_base);
      store_rounded<F32>(dst, 2 * i, a);
      store_rounded<F32>(dst, 2 * i + 1, b);
    }
    return;
  }
  const bool vec = p.R % V == 0 && ((uintptr_t)p.pe % 16 == 0) && ((uintptr_t)p.out % 16 == 0) &&
                   (p.pe_st % V == 0) && (p.pe_sh % V == 0) && (p.o_st % V == 0) &&
                   (p.o_sh % V == 0) && ((p.N) % V == 0);
  if (vec) {
    const int per_row = (int)p.R / V, total = nt * per_row;
    constexpr int U = 4;
    for (int e0 = tid; e0 < total; e0 += U * stride) {
      u32x4_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * stride;
        if (e < total) {
          const int t = t0 + e / per_row, r = (e % per_row) * V;
          v[u] = *(const u32x4_t*)((const T*)p.pe + (int64_t)t * p.pe_st + (int64_t)h * p.pe_sh + r);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * stride;
        if (e < total) {
          const int t = t0 + e / per_row, r = (e % per_row) * V;
          *(u32x4_t*)((T*)p.out + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + p.N + r) = v[u];
        }
      }
    }
    return;
  }
  for (int e = tid; e < nt * p.R; e += stride) {
    const int t = t0 + e / (int)p.R, r = e % (int)p.R;
    const T* src = (const T*)p.pe + (int64_t)t * p.pe_st + (int64_t)h * p.pe_sh + r;
    T* dst = (T*)p.out + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + p.N + r;
    *dst = *src;
  }
}

constexpr int kSlabK = 512;  // weight rows staged per round trip

// LDS position of weight-slab row r and 16-byte chunk c (CW chunks per row).
// 128-byte rows: chunks are XOR-swizzled by 2*(r%4), so the four rows one
// transposed read touches fall in different banks. 32-byte rows: rows 8-11
// and 12-15 of every 16 trade places, so the four lane groups of a read
// (rows 8g..8g+3) alternate between the two halves of the banks.
template <int CW>
__device__ __forceinline__ int slab_off(int r, int c) {
  if constexpr (CW == 8) return r * 128 + ((c ^ wswz(r)) << 4);
  else return (r ^ (((r >> 3) & 1) << 2)) * (CW * 16) + (c << 4);
}

// With a fused cache write the grid has one more head slot: its workgroups
// perform the write (grid-stride over its items) and nothing else.
__device__ __forceinline__ bool cache_write_slot(const BmmParams& p) {
  if (!p.with_cw || (int64_t)blockIdx.z < p.H) return false;
  const int64_t per = (int64_t)gridDim.x * gridDim.y * blockDim.x;
  cache_write_range(p.cw, ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x,
                    per);
  return true;
}

template <int TN>
__global__ void __launch_bounds__(256) bmm_bf16_mfma(BmmParams p) {
  if (cache_write_slot(p)) return;
  extern __shared__ __attribute__((aligned(1024))) char slab_raw[];
  constexpr int CW = TN / 8;     // 16-byte chunks per weight row
  constexpr int NT = TN / 16;    // 16-column MFMA tiles
  constexpr int KS = kSlabK / kKB;
  MLA_LDS char* slab = (MLA_LDS char*)slab_raw;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(w);
  const int n0 = blockIdx.x * TN, t0 = blockIdx.y * kTM, h = blockIdx.z;
  const uint16_t* W = (const uint16_t*)p.w + (int64_t)h * p.w_sh;
  const int t = t0 + 16 * w + li;
  const bool tvalid = t < p.T;
  const uint16_t* arow = (const uint16_t*)p.a + (int64_t)(tvalid ? t : 0) * p.a_st +
                         (int64_t)h * p.a_sh + 8 * g;
  f32x4_t acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < p.K; k0 += kSlabK) {
    const int kc = p.K - k0 < kSlabK ? (int)(p.K - k0) : kSlabK;  // a multiple of 32
    if (k0 > 0) __syncthreads();  // every wave is done with the previous slab
    // stage rows k0 .. k0 + kc: LDS chunk q = inst * 64 + lane holds row q / CW at
    // chunk position q % CW; that position's source chunk is found by inverting slab_off
    const int ninst = kc * CW / 64;
    for (int inst = wave; inst < ninst; inst += 4) {
      const int q = inst * 64 + lane;
      const int rp = q / CW, cp = q % CW;
      int r, c;
      if constexpr (CW == 8) {
        r = rp;
        c = cp ^ wswz(rp);
      } else {
        r = rp ^ (((rp >> 3) & 1) << 2);
        c = cp;
      }
      int col = n0 + 8 * c;
      if (col + 8 > p.N) col = (int)p.N - 8;  // columns past N are never stored
      load_lds_16(W + (int64_t)(k0 + r) * p.w_sk + col, slab + inst * 1024);
    }
    i16x8_t av[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      if (ks * kKB < kc)
        av[ks] = tvalid ? *(const i16x8_t*)(arow + k0 + ks * kKB) : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks * kKB >= kc) break;
      const int rlo = ks * kKB + 8 * g + (li >> 2), rhi = rlo + 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int c = 2 * nt + ((li & 3) >> 1);
        const i16x4_t b0 = lds_read_tr16(slab + slab_off<CW>(rlo, c) + (li & 1) * 8);
        const i16x4_t b1 = lds_read_tr16(slab + slab_off<CW>(rhi, c) + (li & 1) * 8);
        const i16x8_t bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        acc[nt] = mfma_16x16x32(av[ks], bv, acc[nt]);
      }
    }
  }
  // lane holds out[t0 + 16w + 4g + j][n0 + 16nt + li]
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * nt + li;
    if (n >= p.N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + 16 * w + 4 * g + j;
      if (tt < p.T)
        ((uint16_t*)p.out)[(int64_t)tt * p.o_st + (int64_t)h * p.o_sh + n] = f32_to_bf16(acc[nt][j]);
    }
  }
  if (p.R > 0) copy_rope<uint16_t>(p, t0, h, (int)blockIdx.x);
}

// Prefill-sized token counts (bf16): 128 x 128 output tiles of the shared
// pipelined tile (gemm_tile.h); the rope rows are copied after the product,
// as in bmm_bf16_mfma.
__global__ void __launch_bounds__(256) bmm_bf16_big(BmmParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[kGLds];
  int nt, tt, h;
  gemm_tile_coords(nt, tt, h);
  GemmTileArgs g;
  g.a = (const uint16_t*)p.a + (int64_t)h * p.a_sh; g.a_st = p.a_st;
  g.w = (const uint16_t*)p.w + (int64_t)h * p.w_sh; g.w_s1 = p.w_sk;
  g.out = (uint16_t*)p.out + (int64_t)h * p.o_sh; g.o_st = p.o_st;
  g.T = (int)p.T; g.K = (int)p.K; g.N = (int)p.N;
  g.t0 = tt * kGT; g.n0 = nt * kGT;
  gemm_tile_128<false>(g, (MLA_LDS char*)lds_raw);
  if (p.R > 0) {
    copy_rope<uint16_t>(p, g.t0, h, nt);
    if (g.t0 + kTM < p.T) copy_rope<uint16_t>(p, g.t0 + kTM, h, nt);
  }
}

// NWV = 4: wave w computes rows 16w .. 16w + 15 of the 64 x 64 tile, all 64
// columns. NWV = 16 (grids too small to fill the chip): wave w computes the
// 16 x 16 block (rows 16 (w % 4), columns 16 (w / 4)) with four independent
// chains, a quarter of the MFMA chain per wave; the tiles are loaded the same way.
template <int NWV>
__global__ void __launch_bounds__(64 * NWV) bmm_f32_mfma(BmmParams p) {
  static_assert(NWV == 4 || NWV == 16, "four or sixteen waves");
  if (cache_write_slot(p)) return;
  // kDepth k-blocks of 32 rows in flight: block kb's weight tile and activation
  // tile are requested kDepth - 1 blocks before they are used, so a long
  // contraction (the un-projection, K = 512: 16 blocks) waits for about one round
  // trip rather than one per block. Both tiles travel global -> LDS, so every
  // wait below is explicit and counts exactly these loads.
  constexpr int kDepth = 4;
  // 16-byte loads per loading thread per tile: the 512 chunks of a tile over
  // 256 threads (two each) or over the first 512 of 1024 (one each)
  constexpr int NLD = NWV == 4 ? 2 : 1;
  constexpr int kOps = 2 * NLD;  // per block: W and A
  __shared__ __attribute__((aligned(16))) float wt[kDepth][kKB * kTN];  // [k][n]
  __shared__ __attribute__((aligned(16))) float at[kDepth][kTM * kKB];  // [t][k], swizzled
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
  const int n0 = blockIdx.x * kTN, t0 = blockIdx.y * kTM, h = blockIdx.z;
  const float* W = (const float*)p.w + (int64_t)h * p.w_sh;
  const int nk = (int)(p.K / kKB);
  const bool loads = threadIdx.x < 512;
  f32x4_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // A tile: row r (token t0 + r) holds 8 chunks of 4 floats; chunk c sits at
  // position c ^ ((r >> 1) & 7), so the 16 rows one read touches fall in distinct
  // banks. Thread slot q = threadIdx.x + 256 i loads position q % 8 of row q / 8.
  auto issue = [&](int kb, int buf) {
    if (!loads) return;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int slot = threadIdx.x + 256 * i;
      const int r = slot >> 4, c = slot & 15;
      int col = n0 + 4 * c;
      if (col + 4 > p.N) col = (int)p.N - 4;
      load_lds_16(W + (int64_t)(kb * kKB + r) * p.w_sk + col,
                  (MLA_LDS char*)&wt[buf][0] + (slot - lane) * 16);
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int slot = threadIdx.x + 256 * i;
      const int r = slot >> 3, pos = slot & 7, c = pos ^ ((r >> 1) & 7);
      int tr = t0 + r;
      if (tr >= p.T) tr = (int)p.T - 1;  // rows past T repeat the last one; never stored
      load_lds_16((const float*)p.a + (int64_t)tr * p.a_st + (int64_t)h * p.a_sh + kb * kKB + 4 * c,
                  (MLA_LDS char*)&at[buf][0] + (slot - lane) * 16);
    }
  };
  for (int kb = 0; kb < kDepth - 1 && kb < nk; ++kb) issue(kb, kb);
  // NWV = 4 and a tile of at most 16 tokens (the tail of a call): every wave
  // takes rows 0..15, each for one 16-column group, as NWV = 16 does.
  // Both conditions are uniform over the workgroup.
  const bool narrow = NWV == 16 || p.T - t0 <= 16;
  const int wr = NWV == 16 ? (w & 3) : (narrow ? 0 : w);  // 16-row group
  const int wq = NWV == 16 ? (w >> 2) : w;                // 16-column group when narrow
  const bool busy = t0 + 16 * wr < p.T;  // wave-uniform: its rows hold tokens
  const int r = 16 * wr + li;            // this lane's A row
  for (int kb = 0; kb < nk; ++kb) {
    // blocks kb + 1 .. min(kb + kDepth - 2, nk - 1) may stay in flight
    const int ahead = nk - 1 - kb < kDepth - 2 ? nk - 1 - kb : kDepth - 2;
    wait_vmcnt_n<kDepth - 2, kOps>(ahead);
    __syncthreads();  // block kb has landed for every wave; block kb - 1's buffers are free
    if (kb + kDepth - 1 < nk) issue(kb + kDepth - 1, (kb + kDepth - 1) % kDepth);
    if (!busy) continue;
    const int buf = kb % kDepth;
    const MLA_LDS float* tile = (const MLA_LDS float*)wt[buf];
    const MLA_LDS float* arow = (const MLA_LDS float*)at[buf] + r * kKB;
    // k = 4g + x (chunk g) and 16 + 4g + x (chunk 4 + g)
    const f32x4_t c0 = *(const MLA_LDS f32x4_t*)(arow + 4 * (g ^ ((r >> 1) & 7)));
    const f32x4_t c1 = *(const MLA_LDS f32x4_t*)(arow + 4 * ((4 + g) ^ ((r >> 1) & 7)));
    if (narrow) {
      // four independent chains (one per x), summed after the loop
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        acc[x] = mfma_16x16x4f32(c0[x], tile[(4 * g + x) * kTN + 16 * wq + li], acc[x]);
        acc[x] = mfma_16x16x4f32(c1[x], tile[(16 + 4 * g + x) * kTN + 16 * wq + li], acc[x]);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          acc[nt] = mfma_16x16x4f32(c0[x], tile[(4 * g + x) * kTN + 16 * nt + li], acc[nt]);
          acc[nt] = mfma_16x16x4f32(c1[x], tile[(16 + 4 * g + x) * kTN + 16 * nt + li], acc[nt]);
        }
      }
    }
  }
  if (narrow) {
    const int n = n0 + 16 * wq + li;
    if (busy && n < p.N) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tt = t0 + 16 * wr + 4 * g + j;
        if (tt < p.T)
          ((float*)p.out)[(int64_t)tt * p.o_st + (int64_t)h * p.o_sh + n] =
              (acc[0][j] + acc[1][j]) + (acc[2][j] + acc[3][j]);
      }
    }
    if (p.R > 0) copy_rope<uint32_t>(p, t0, h, (int)blockIdx.x);
    return;
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
  if (p.R > 0) copy_rope<uint32_t>(p, t0, h, (int)blockIdx.x);
}

// f32, a whole call of at most 16 tokens (a decode step): one workgroup per
// (16-column group, head), so the un-projection (N = 128) spreads over 8
// workgroups per head rather than 2. Wave w of the eight takes k-blocks w, w + 8,
// ... of 32 rows (two for K = 512, so all its loads are in flight together) with
// its operands loaded straight from global memory; the waves' partial tiles are
// summed through LDS in wave order.
constexpr int kNarrowWaves = 8;

__global__ void __launch_bounds__(64 * kNarrowWaves) bmm_f32_narrow(BmmParams p) {
  if (cache_write_slot(p)) return;
  __shared__ f32x4_t part[kNarrowWaves - 1][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
  const int n = blockIdx.x * 16 + li, h = blockIdx.z;  // N % 16 == 0 here, so n < N
  const int tr = li < p.T ? li : (int)p.T - 1;  // rows past T repeat the last one; never stored
  const float* arow = (const float*)p.a + (int64_t)tr * p.a_st + (int64_t)h * p.a_sh + 4 * g;
  const float* wcol = (const float*)p.w + (int64_t)h * p.w_sh + (int64_t)(4 * g) * p.w_sk + n;
  const int nk = (int)(p.K / kKB);
  f32x4_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int kb = w; kb < nk; kb += kNarrowWaves) {
    // this lane's A values at k = 4g + x and 16 + 4g + x of the block, and the
    // matching W rows of column n
    const f32x4_t c0 = *(const f32x4_t*)(arow + kb * kKB);
    const f32x4_t c1 = *(const f32x4_t*)(arow + kb * kKB + 16);
    const float* wk = wcol + (int64_t)kb * kKB * p.w_sk;
    float b0[4], b1[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      b0[x] = wk[x * p.w_sk];
      b1[x] = wk[(16 + x) * p.w_sk];
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      acc[x] = mfma_16x16x4f32(c0[x], b0[x], acc[x]);
      acc[x] = mfma_16x16x4f32(c1[x], b1[x], acc[x]);
    }
  }
  f32x4_t sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  if (w > 0) part[w - 1][lane] = sum;
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int i = 0; i < kNarrowWaves - 1; ++i) sum += part[i][lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = 4 * g + j;  // D row of this lane's j-th value
      if (tt < p.T) ((float*)p.out)[(int64_t)tt * p.o_st + (int64_t)h * p.o_sh + n] = sum[j];
    }
  }
  if (p.R > 0) copy_rope<uint32_t>(p, 0, h, (int)blockIdx.x);
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
  const unsigned hz = (unsigned)p.H + (p.with_cw ? 1u : 0u);  // head slots (+ the cache write)
  if (mfma_ok && p.is_f32 && p.T <= 16) {
    dim3 grid((unsigned)(p.N / 16), 1, hz);
    hipLaunchKernelGGL(bmm_f32_narrow, grid, dim3(64 * kNarrowWaves), 0, s, p);
  } else if (mfma_ok && p.is_f32) {
    dim3 grid((unsigned)((p.N + kTN - 1) / kTN), (unsigned)((p.T + kTM - 1) / kTM), hz);
    // a grid that leaves most of the chip idle takes sixteen waves per tile
    if ((int64_t)grid.x * grid.y * p.H < 256)
      hipLaunchKernelGGL(bmm_f32_mfma<16>, grid, dim3(1024), 0, s, p);
    else
      hipLaunchKernelGGL(bmm_f32_mfma<4>, grid, dim3(256), 0, s, p);
  } else if (mfma_ok && !p.with_cw && p.T >= kBigT && p.K <= INT32_MAX && p.T <= INT32_MAX &&
             (uintptr_t)p.out % 16 == 0 && p.o_st * es % 16 == 0 && p.o_sh * es % 16 == 0) {
    // (the 128 x 128 tile writes 16-byte pieces of out rows)
    dim3 grid((unsigned)((p.N + kGT - 1) / kGT), (unsigned)((p.T + kGT - 1) / kGT), (unsigned)p.H);
    hipLaunchKernelGGL(bmm_bf16_big, grid, dim3(256), 0, s, p);
  } else if (mfma_ok) {
    // 64-wide tiles when they give the chip at least 128 workgroups
    const int64_t tiles_t = (p.T + kTM - 1) / kTM;
    const bool wide = p.N % 64 == 0 && (p.N / 64) * tiles_t * p.H >= 128;
    const int tn = wide ? 64 : 16;
    const int64_t kc = p.K < kSlabK ? p.K : kSlabK;
    const size_t smem = (size_t)kc * tn * 2;
    dim3 grid((unsigned)((p.N + tn - 1) / tn), (unsigned)tiles_t, hz);
    if (wide) {
      static bool attr = false;
      if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void*)bmm_bf16_mfma<64>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           kSlabK * 64 * 2);
        if (e != hipSuccess) return e;
        attr = true;
      }
      hipLaunchKernelGGL(bmm_bf16_mfma<64>, grid, dim3(256), smem, s, p);
    } else {
      hipLaunchKernelGGL(bmm_bf16_mfma<16>, grid, dim3(256), smem, s, p);
    }
  } else {
    const int64_t total = p.T * p.H * p.N;
    const int64_t blocks = (total + 255) / 256 + (p.T * p.H * p.R + 255) / 256;
    if (p.is_f32) hipLaunchKernelGGL(bmm_plain<true>, dim3((unsigned)blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(bmm_plain<false>, dim3((unsigned)blocks), dim3(256), 0, s, p);
    if (p.with_cw) {  // the plain path has no head slots: the write is a launch of its own
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_cache_write(p.cw, s);
    }
  }
  return hipGetLastError();
}

}  // namespace mla
