// gemm_tile.h -- the 128 x 128 output tile of a bf16 batched product for
// token counts of a prefill (hundreds to thousands of rows per head), shared
// by the weight folds (bmm.hip) and the key decompression (prefill.hip).
//
//   out[t, h, n] = sum_k a[t, h, k] * B_h[k, n]
//   B_h[k, n] = w[h, k, n]  (NN: rows of w are k, n contiguous)
//            or w[h, n, k]  (NT: rows of w are n, k contiguous)
//
// Four waves, each owning 64 x 64 of the tile as 4 x 4 blocks of
// v_mfma_f32_16x16x32_bf16. Per 32-wide k step the workgroup reads a
// 128 x 32 slice of `a` and the matching 32 x 128 slice of B into registers
// (two 16-byte pieces per thread each), one step ahead of the arithmetic, and
// stores them to a two-slot LDS ring; one barrier per step. LDS rows are
// padded so the operand reads fall in distinct banks: the A (and NT B)
// operand reads 16 rows x 16 bytes per 16 lanes from 80-byte rows; the NN B
// operand is read transposed with ds_read_b64_tr_b16, 4 rows x 32 bytes per
// 16 lanes from 288-byte rows. Device code only.
#pragma once

#include "mla_device.h"

namespace mla {

constexpr int kGT = 128;       // tile rows (tokens) and columns (outputs)
constexpr int kGK = 32;        // k per step
constexpr int kGAP = 80;       // A / NT-B row pitch in LDS (64 bytes + 16)
constexpr int kGBP = 288;      // NN-B row pitch in LDS (256 bytes + 32)
constexpr int kGSlotA = kGT * kGAP;
constexpr int kGSlotB = kGT * kGAP > kGK * kGBP ? kGT * kGAP : kGK * kGBP;
constexpr int kGSlot = kGSlotA + kGSlotB;
constexpr int kGLds = 2 * kGSlot;
constexpr int kGOP = kGT * 2 + 16;  // output tile row pitch in LDS (bf16 row + 16 bytes)

struct GemmTileArgs {
  const uint16_t* a; int64_t a_st;  // row t of head h at a + t * a_st (head offset applied)
  const uint16_t* w; int64_t w_s1;  // head h's weight; NN: row k at w + k * w_s1; NT: row n
  uint16_t* out;     int64_t o_st;  // row t of head h at out + t * o_st (head offset applied)
  int T, K, N;                      // N >= 16, a multiple of 8; K a multiple of 32
  int t0, n0;                       // tile origin
};

// The (column tile, row tile, head) of this workgroup for a grid of
// (column tiles, row tiles, heads). Workgroup i runs on XCD i % 8; when the
// grid divides evenly, XCD x takes the x-th eighth of the tiles in
// column-fastest order, so the column tiles that share rows of `a`, and the
// tiles of one head's weight, run on one XCD and meet in its L2.
__device__ __forceinline__ void gemm_tile_coords(int& nt, int& tt, int& h) {
  const int gx = (int)gridDim.x, gy = (int)gridDim.y;
  const int total = gx * gy * (int)gridDim.z;
  int lin = (int)blockIdx.x + gx * ((int)blockIdx.y + gy * (int)blockIdx.z);
  if (total % 8 == 0) lin = (lin % 8) * (total / 8) + lin / 8;
  nt = lin % gx;
  tt = (lin / gx) % gy;
  h = lin / (gx * gy);
}

template <bool NT>
__device__ __forceinline__ void gemm_tile_128(const GemmTileArgs& g, MLA_LDS char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, li = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w >> 1, wc = w & 1;
  // this thread's two pieces of each slice: A (and NT B) rows r = idx / 4,
  // 16-byte piece c = idx % 4; NN B k-rows r = idx / 16, piece c = idx % 16
  const uint16_t* asrc[2];
  const uint16_t* bsrc[2];
  int aoff[2], boff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    const int r = idx >> 2, c = idx & 3;
    const int t = g.t0 + r < g.T ? g.t0 + r : g.T - 1;  // rows past T repeat the last one
    asrc[i] = g.a + (int64_t)t * g.a_st + 8 * c;
    aoff[i] = r * kGAP + 16 * c;
    if constexpr (NT) {
      const int n = g.n0 + r < g.N ? g.n0 + r : g.N - 1;
      bsrc[i] = g.w + (int64_t)n * g.w_s1 + 8 * c;
      boff[i] = r * kGAP + 16 * c;
    } else {
      const int rk = idx >> 4, ck = idx & 15;
      int col = g.n0 + 8 * ck;
      if (col + 8 > g.N) col = g.N - 8;  // columns past N are never stored
      bsrc[i] = g.w + (int64_t)rk * g.w_s1 + col;
      boff[i] = rk * kGBP + 16 * ck;
    }
  }
  const int64_t bstep = NT ? kGK : (int64_t)kGK * g.w_s1;
  u32x4_t ar[2], br[2];
  auto load = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ar[i] = *(const u32x4_t*)(asrc[i] + ks * kGK);
      br[i] = *(const u32x4_t*)(bsrc[i] + ks * bstep);
    }
  };
  auto store = [&](int slot) {
    MLA_LDS char* sa = lds + slot * kGSlot;
    MLA_LDS char* sb = sa + kGSlotA;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *(MLA_LDS u32x4_t*)(sa + aoff[i]) = ar[i];
      *(MLA_LDS u32x4_t*)(sb + boff[i]) = br[i];
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nsteps = g.K / kGK;
  load(0);
  store(0);
  __syncthreads();
  for (int ks = 0; ks < nsteps; ++ks) {
    const bool more = ks + 1 < nsteps;
    if (more) load(ks + 1);
    const MLA_LDS char* sa = lds + (ks & 1) * kGSlot;
    const MLA_LDS char* sb = sa + kGSlotA;
    i16x8_t av[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      av[i] = *(const MLA_LDS i16x8_t*)(sa + (64 * wr + 16 * i + li) * kGAP + 16 * gq);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (NT) {
        bv[j] = *(const MLA_LDS i16x8_t*)(sb + (64 * wc + 16 * j + li) * kGAP + 16 * gq);
      } else {
        // B[k = 8 gq + 0..7][n = 64 wc + 16 j + li] from two transposed reads
        const MLA_LDS char* p0 =
            sb + (8 * gq + (li >> 2)) * kGBP + 2 * (64 * wc + 16 * j + 4 * (li & 3));
        const i16x4_t b0 = lds_read_tr16(p0);
        const i16x4_t b1 = lds_read_tr16(p0 + 4 * kGBP);
        bv[j] = i16x8_t{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(av[i], bv[j], acc[i][j]);
    if (more) store((ks + 1) & 1);
    __syncthreads();
  }
  // The tile goes out through LDS (free after the last barrier): lane holds
  // out[64 wr + 16 i + 4 gq + jj][64 wc + 16 j + li] of the tile; it is
  // stored as bf16 rows of kGOP bytes, then every thread writes 16-byte pieces
  // of whole rows, so each row's 256 bytes leave in full lines (non-temporal:
  // the product is read by a later kernel, not by this one).
  static_assert(kGT * kGOP <= kGLds, "output tile fits the ring");
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *(MLA_LDS uint16_t*)(lds + (64 * wr + 16 * i + 4 * gq + jj) * kGOP +
                             2 * (64 * wc + 16 * j + li)) = f32_to_bf16(acc[i][j][jj]);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kGT * kGT / 8 / 256; ++i) {
    const int idx = tid + 256 * i;
    const int r = idx >> 4, c = idx & 15;  // row, 8-column piece
    const int t = g.t0 + r, n = g.n0 + 8 * c;
    if (t < g.T && n < g.N)  // N is a multiple of 8: a piece is all in or all out
      __builtin_nontemporal_store(*(const MLA_LDS u32x4_t*)(lds + r * kGOP + 16 * c),
                                  (u32x4_t*)(g.out + (int64_t)t * g.o_st + n));
  }
}

}  // namespace mla
