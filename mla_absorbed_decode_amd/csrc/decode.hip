// decode.hip -- split-KV absorbed MLA attention over a paged latent cache on
// gfx950 (MI355X), plus the log-sum-exp merge of the splits.
//
// What is computed (vLLM "test_mla_cross_layer_kernel_equivalence.py",
// test_flashmla_dense_decode_unified_slot_view and
// test_flashattn_mla_dense_decode_unified_slot_view; memra-engine 0.124.1
// "tests/mla_gpu_forward.rs", gates 1 and 2): for every (sequence b, query i,
// head h) row, score_j = scale * q[b,i,h,:] . key_j over the whole latent row
// [c_kv | k_pe] of every visible key j, softmax over j, and
// out = sum_j p_j * c_kv_j. One latent row per token serves all heads.
//
// Work decomposition
// ------------------
// Rows (query, head) of one sequence are cut into "units" of rows_per_unit
// rows that share every key. A unit's visible keys are cut into 64-token work
// blocks. With many units (prefill) each workgroup takes one unit. With few
// units (decode) the work blocks of all units are laid end to end and cut
// into `grid` equal chunks, one per workgroup; a unit that lands in more than
// one chunk is written as normalised fp32 partials plus a log2-domain lse per
// chunk and merged by decode_merge in chunk order (deterministic). The plan
// depends only on seqlens and sizes, never on strides or pointers.
//
// Inside a workgroup, keys are staged through LDS in tiles of TT tokens with
// direct global->LDS 16-byte loads, NSLOT tiles deep. Each wave holds the
// folded query of its 16*RT rows in registers and computes, per tile,
//   S^T[token, row]  = sum_e K[token, e] * Q[row, e]        (MFMA, bf16 -> f32)
//   online softmax per row (exp2 domain, lazy rescale when the max grows by
//   more than 2^8)
//   O^T[d, row]     += sum_token V[token, d] * P[row, token] (MFMA)
// where V is the first 512 columns of the staged K rows, read transposed with
// ds_read_b64_tr_b16. S^T's accumulator layout gives each lane one row and
// four tokens, which is exactly the B operand layout P^T needs, so P never
// leaves registers.
//
// Two wave layouts:
//   WR row-waves  x WT token-waves, with WR == 1 or WT == 1.
//   WT == 4 (few heads, the HBM-bound decode): 4 waves share one 16-row tile
//     and take alternate key tiles, each wave with its own LDS ring; the four
//     partial states are merged through LDS at the end.
//   WR == 4 (many heads or prefill rows): 4 waves take 4 row blocks of the
//     unit and share every key tile, loading a quarter each; one barrier per
//     tile.
#include <math.h>

#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

typedef __attribute__((address_space(4))) const int32_t cint32_t;  // scalar-loadable view

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kRescaleLog2 = 8.0f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int load_scalar_i32(const int32_t* p, int64_t idx) {
  return ((cint32_t*)(uintptr_t)p)[idx];
}

__device__ __forceinline__ int seq_len(const DecodeParams& p, int b) {
  int s = load_scalar_i32(p.seqlens, b);
  s = s < 0 ? 0 : s;
  return s > p.seq_cap ? p.seq_cap : s;
}

// Keys visible to query i of a sequence of length s (queries are the last Sq tokens).
__device__ __forceinline__ int row_limit(const DecodeParams& p, int s, int qi) {
  if (!p.causal) return s;
  int n = s - p.q_len + qi + 1;
  return n < 0 ? 0 : (n > s ? s : n);
}

// Keys a unit needs: the most any of its rows sees.
__device__ __forceinline__ int unit_kvlen(const DecodeParams& p, int u) {
  const int b = u / p.row_tiles, rt = u % p.row_tiles;
  const int s = seq_len(p, b);
  const int rows = p.q_len * p.n_heads;
  int r_last = (rt + 1) * p.rows_per_unit;
  r_last = (r_last > rows ? rows : r_last) - 1;
  return row_limit(p, s, r_last / p.n_heads);
}

// Inclusive prefix over units of their work-block counts, for up to 256 units
// (one per thread of a 256-thread block). Leaves the prefix in sh[0..255].
__device__ void unit_scan(const DecodeParams& p, int* sh) {
  const int t = threadIdx.x;
  int v = t < p.num_units ? ceil_div(unit_kvlen(p, t), kWorkBlock) : 0;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int x = t >= off ? sh[t - off] : 0;
    __syncthreads();
    sh[t] += x;
    __syncthreads();
  }
}

template <int R_, int WR_, int WT_, int RT_, int TT_, int NSLOT_, bool F32_>
struct Cfg {
  static constexpr int R = R_, WR = WR_, WT = WT_, RT = RT_, TT = TT_, NSLOT = NSLOT_;
  static constexpr bool F32 = F32_;
  static constexpr int ES = F32 ? 4 : 2;           // element bytes
  static constexpr int E = kKvRank + R;            // latent row width
  static constexpr int PITCH = E * ES;             // bytes per staged row
  static constexpr int CH = PITCH / 16;            // 16-byte chunks per row
  static constexpr int NW = WR * WT;
  static constexpr int NT = 64 * NW;
  static constexpr int ROWS_W = 16 * RT;
  static constexpr int RTILE = ROWS_W * WR;
  static constexpr int TILE_BYTES = TT * PITCH;
  static constexpr int LPT = TT * CH / 64;         // 16-byte loads per tile per 64 lanes
  static constexpr int LPW = LPT / WR;             // issued by each wave of a token group
  static constexpr int SUB = TT / 16;
  static constexpr int KSTEPS = F32 ? E / 16 : E / 32;
  static constexpr int RING_BYTES = WT * NSLOT * TILE_BYTES;
  static constexpr int DT = kKvRank / 16;          // 32 output column tiles
  static_assert(LPT * 64 == TT * CH, "tile chunk count");
  static_assert(LPW * WR == LPT, "tile loads split evenly over row waves");
  static_assert(WR == 1 || WT == 1, "rows or tokens are split over waves, not both");
  static_assert(NT == 256, "the split planner assumes 256-thread workgroups");
  static_assert(TT == 16 || TT == 32, "tile size");
  static_assert(!F32 || TT == 16, "f32 path uses 16-token tiles");
  static_assert(NSLOT >= 1 && NSLOT <= 4, "ring depth");
  // the token-split layout merges its waves' states through the same LDS
  static constexpr int MERGE_BYTES = WT > 1 ? WT * DT * 64 * 16 + 2 * WT * 16 * 4 : 0;
  static constexpr int SMEM_BYTES = RING_BYTES > MERGE_BYTES ? RING_BYTES : MERGE_BYTES;
  static_assert(SMEM_BYTES + 1024 <= 160 * 1024, "LDS budget");
};

// Everything a wave carries through one segment.
template <class C>
struct WaveState {
  f32x4_t o[C::RT][C::DT];
  float m[C::RT];
  float l[C::RT];
  int lim[C::RT];   // this lane's row: keys [.., lim) visible (already capped by the segment end)
};

// ---------------------------------------------------------------- one tile
template <class C, class QReg>
__device__ __forceinline__ void tile_compute(const MLA_LDS char* tile, int j0, const QReg& qreg,
                                             WaveState<C>& st, float scale_log2) {
  const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  f32x4_t s[C::SUB][C::RT];
#pragma unroll
  for (int a = 0; a < C::SUB; ++a)
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) s[a][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // ---- S^T = K . Q^T : lane (token li of sub-tile a, e-group g) x (row li, g)
  if constexpr (!C::F32) {
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
#pragma unroll
      for (int a = 0; a < C::SUB; ++a) {
        const int rr = 16 * a + li;
        const int c = (g + 4 * kk) ^ lds_swz(li);
        const i16x8_t k = *(const MLA_LDS i16x8_t*)(tile + rr * C::PITCH + c * 16);
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) s[a][rt] = mfma_16x16x32(k, qreg[rt][kk], s[a][rt]);
      }
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const int c = (g + 4 * kk) ^ lds_swz(li);
      const f32x4_t k = *(const MLA_LDS f32x4_t*)(tile + li * C::PITCH + c * 16);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
          s[0][rt] = mfma_16x16x4f32(k[x], qreg[rt][kk][x], s[0][rt]);
    }
  }

  // ---- online softmax (exp2 domain); lane holds row li, tokens 16a + 4g + j
  using PT = typename std::conditional<C::TT == 32, i16x8_t, i16x4_t>::type;
  PT pb[C::RT];
  float pf[C::RT][4];
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    float v[C::SUB][4];
    float mt = kNegInf;
#pragma unroll
    for (int a = 0; a < C::SUB; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = j0 + 16 * a + 4 * g + j;
        v[a][j] = tok < st.lim[rt] ? s[a][rt][j] * scale_log2 : kNegInf;
        mt = fmaxf(mt, v[a][j]);
      }
    mt = wave_max16(mt);
    const bool need = mt > st.m[rt] + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mn = fmaxf(st.m[rt], mt);
      const float alpha = mn == kNegInf ? 1.f : fast_exp2(st.m[rt] - mn);
#pragma unroll
      for (int d = 0; d < C::DT; ++d) st.o[rt][d] *= alpha;
      st.l[rt] *= alpha;
      st.m[rt] = mn;
    }
    const float ms = st.m[rt] == kNegInf ? 0.f : st.m[rt];
    float lsum = 0.f;
#pragma unroll
    for (int a = 0; a < C::SUB; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[a][j] = fast_exp2(v[a][j] - ms);
        lsum += v[a][j];
      }
    st.l[rt] += lsum;
    if constexpr (C::F32) {
#pragma unroll
      for (int j = 0; j < 4; ++j) pf[rt][j] = v[0][j];
    } else {
#pragma unroll
      for (int a = 0; a < C::SUB; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) pb[rt][4 * a + j] = (short)f32_to_bf16(v[a][j]);
    }
  }

  // ---- O^T += V^T . P^T : A = V^T (d = li, tokens by g), B = P^T (tokens by g, row li)
  if constexpr (!C::F32) {
    // local lane li points at token row (4g + li/4) [+16], columns 16*d + 4*(li%4)
    const int rr0 = 4 * g + (li >> 2);
    const int sw0 = lds_swz(rr0 & 15), sw1 = lds_swz((rr0 + 16) & 15);
    const int cx = (li & 3) >> 1, half8 = (li & 1) * 8;
#pragma unroll
    for (int d = 0; d < C::DT; ++d) {
      const int c = 2 * d + cx;
      const i16x4_t v0 = lds_read_tr16(tile + rr0 * C::PITCH + ((c ^ sw0) << 4) + half8);
      if constexpr (C::TT == 32) {
        const i16x4_t v1 =
            lds_read_tr16(tile + (rr0 + 16) * C::PITCH + ((c ^ sw1) << 4) + half8);
        const i16x8_t vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) st.o[rt][d] = mfma_16x16x32(vv, pb[rt], st.o[rt][d]);
      } else {
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) st.o[rt][d] = mfma_16x16x16(v0, pb[rt], st.o[rt][d]);
      }
    }
  } else {
#pragma unroll
    for (int d = 0; d < C::DT; ++d) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int rr = 4 * g + x;
        const int col = 16 * d + li;  // float index
        const float vv = *(const MLA_LDS float*)(tile + rr * C::PITCH +
                                                   (((col >> 2) ^ lds_swz(rr)) << 4) +
                                                   (col & 3) * 4);
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) st.o[rt][d] = mfma_16x16x4f32(vv, pf[rt][x], st.o[rt][d]);
      }
    }
  }
}

// ------------------------------------------------------ output of a segment
template <class C>
__device__ __forceinline__ void store_row(const DecodeParams& p, int b, int unit_row0,
                                          int local_row, int slot, const f32x4_t* o, float inv,
                                          float lse2) {
  // o[DT]: this lane's row, columns 16*d + 4*g + j
  const int lane = threadIdx.x & 63, g = lane >> 4;
  const int rows_seq = p.q_len * p.n_heads;
  const int r = unit_row0 + local_row;
  if (r >= rows_seq) return;
  if (slot >= 0) {
    float* dst = p.part_o + ((int64_t)slot * p.rows_per_unit + local_row) * kKvRank + 4 * g;
#pragma unroll
    for (int d = 0; d < C::DT; ++d) *(f32x4_t*)(dst + 16 * d) = o[d] * inv;
    if (g == 0) p.part_lse[(int64_t)slot * p.rows_per_unit + local_row] = lse2;
    return;
  }
  const int qi = r / p.n_heads, qh = r % p.n_heads;
  const int64_t ooff = (int64_t)b * p.o_s0 + (int64_t)qi * p.o_s1 + (int64_t)qh * p.o_s2 + 4 * g;
  if constexpr (C::F32) {
    float* dst = (float*)p.out + ooff;
#pragma unroll
    for (int d = 0; d < C::DT; ++d) *(f32x4_t*)(dst + 16 * d) = o[d] * inv;
  } else {
    uint16_t* dst = (uint16_t*)p.out + ooff;
#pragma unroll
    for (int d = 0; d < C::DT; ++d) {
      const f32x4_t x = o[d] * inv;
      *(u32x2_t*)(dst + 16 * d) = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    }
  }
  if (g == 0 && p.lse)
    p.lse[(int64_t)b * p.l_s0 + (int64_t)qi * p.l_s1 + (int64_t)qh * p.l_s2] =
        lse2 == kNegInf ? kNegInf : lse2 * kLn2;
}

// ------------------------------------------------------------- one segment
// Keys [tok_lo, tok_hi) of unit u; slot < 0 writes the final output.
template <class C>
__device__ void process_segment(const DecodeParams& p, int u, int tok_lo, int tok_hi, int slot,
                                MLA_LDS char* ring_all) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int wr = C::WT == 1 ? wave : 0;
  const int wt = C::WT == 1 ? 0 : wave;

  const int b = u / p.row_tiles, rtu = u % p.row_tiles;
  const int s = seq_len(p, b);
  const int kvlen = unit_kvlen(p, u);
  const int t_lo = tok_lo;
  const int t_hi = tok_hi < kvlen ? tok_hi : kvlen;
  const int ntiles = t_hi > t_lo ? ceil_div(t_hi - t_lo, C::TT) : 0;
  const int rows_seq = p.q_len * p.n_heads;
  const int unit_row0 = rtu * p.rows_per_unit;
  const int wrow0 = wr * C::ROWS_W;  // first local row of this wave

  // ---- folded query rows of this wave -> registers (B operand layout)
  using QV = typename std::conditional<C::F32, f32x4_t, i16x8_t>::type;
  QV qreg[C::RT][C::KSTEPS];
  WaveState<C> st;
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    const int r = unit_row0 + wrow0 + 16 * rt + li;
    const bool valid = r < rows_seq;
    const int qi = valid ? r / p.n_heads : 0, qh = valid ? r % p.n_heads : 0;
    const int64_t qoff = (int64_t)b * p.q_s0 + (int64_t)qi * p.q_s1 + (int64_t)qh * p.q_s2;
    if constexpr (C::F32) {
      const float* qp = (const float*)p.q + qoff + 4 * g;
#pragma unroll
      for (int kk = 0; kk < C::KSTEPS; ++kk)
        qreg[rt][kk] = valid ? *(const f32x4_t*)(qp + 16 * kk) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else {
      const uint16_t* qp = (const uint16_t*)p.q + qoff + 8 * g;
#pragma unroll
      for (int kk = 0; kk < C::KSTEPS; ++kk)
        qreg[rt][kk] = valid ? *(const i16x8_t*)(qp + 32 * kk) : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
    const int lim = valid ? row_limit(p, s, qi) : 0;
    st.lim[rt] = lim < t_hi ? lim : t_hi;
    st.m[rt] = kNegInf;
    st.l[rt] = 0.f;
#pragma unroll
    for (int d = 0; d < C::DT; ++d) st.o[rt][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  MLA_LDS char* ring = ring_all + wt * C::NSLOT * C::TILE_BYTES;
  const int nsteps = ntiles > wt ? ceil_div(ntiles - wt, C::WT) : 0;
  const char* kvbase = (const char*)p.kv;
  const int64_t pitch_g = p.kv_s1 * C::ES;

  auto issue = [&](int step) {
    const int j0 = t_lo + (wt + step * C::WT) * C::TT;
    const int nvalid = t_hi - j0 < C::TT ? t_hi - j0 : C::TT;
    MLA_LDS char* dst = ring + (step % C::NSLOT) * C::TILE_BYTES;
    // each 16-token half of the tile lies in one page (page is a multiple of 16)
    const int pg0 = j0 / p.page;
    int blk0 = load_scalar_i32(p.block_table, (int64_t)b * p.bt_s0 + pg0);
    blk0 = blk0 < 0 ? 0 : (blk0 >= p.num_blocks ? (int)p.num_blocks - 1 : blk0);
    const char* base0 = kvbase + (int64_t)blk0 * p.kv_s0 * C::ES + (int64_t)(j0 - pg0 * p.page) * pitch_g;
    const char* base1 = base0 + 16 * pitch_g;
    if constexpr (C::TT == 32) {
      const int j1 = j0 + 16;
      if (j1 < t_hi && (j1 / p.page) != pg0) {
        const int pg1 = j1 / p.page;
        int blk1 = load_scalar_i32(p.block_table, (int64_t)b * p.bt_s0 + pg1);
        blk1 = blk1 < 0 ? 0 : (blk1 >= p.num_blocks ? (int)p.num_blocks - 1 : blk1);
        base1 = kvbase + (int64_t)blk1 * p.kv_s0 * C::ES + (int64_t)(j1 - pg1 * p.page) * pitch_g;
      }
    }
#pragma unroll
    for (int n = 0; n < C::LPW; ++n) {
      // this lane's 16-byte slot of the tile: row r, stored chunk position cpos
      const int idx = (wr + n * C::WR) * 64 + lane;
      const int r = idx / C::CH, cpos = idx % C::CH;
      const int chunk = cpos ^ lds_swz(r & 15);
      const int rr = r < nvalid ? r : nvalid - 1;  // rows past the end repeat the last valid row
      const char* src = (C::TT == 32 && rr >= 16) ? base1 + (rr - 16) * pitch_g : base0 + rr * pitch_g;
      load_lds_16(src + chunk * 16, dst + (wr + n * C::WR) * 1024);
    }
  };

#pragma unroll
  for (int k = 0; k < C::NSLOT - 1; ++k)
    if (k < nsteps) issue(k);

  for (int k = 0; k < nsteps; ++k) {
    if constexpr (C::NSLOT == 1) {
      static_assert(C::WR == 1, "a one-slot ring is private to its wave");
      issue(k);  // the previous tile's reads are complete (compiler-inserted lgkmcnt wait)
      wait_vmcnt<0>();
    } else {
      // tiles k+1 .. k+NSLOT-2 may still be in flight; tile k must have landed
      int ahead = nsteps - 1 - k;
      ahead = ahead < C::NSLOT - 2 ? ahead : C::NSLOT - 2;
      if (ahead <= 0) wait_vmcnt<0>();
      else if (ahead == 1) wait_vmcnt<C::LPW>();
      else wait_vmcnt<(C::NSLOT >= 4 ? 2 * C::LPW : 0)>();
      // row-split: tile k is complete for every wave, and every wave is done
      // with tile k-1, whose slot the next issue overwrites
      if constexpr (C::WR > 1) __syncthreads();
      if (k + C::NSLOT - 1 < nsteps) issue(k + C::NSLOT - 1);
    }
    const int j0 = t_lo + (wt + k * C::WT) * C::TT;
    tile_compute<C>(ring + (k % C::NSLOT) * C::TILE_BYTES, j0, qreg, st, p.scale_log2);
  }

  // ---- finish
  if constexpr (C::WT == 1) {
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      const float lt = wave_sum16(st.l[rt]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse2 = lt > 0.f ? st.m[rt] + fast_log2(lt) : kNegInf;
      store_row<C>(p, b, unit_row0, wrow0 + 16 * rt + li, slot, st.o[rt], inv, lse2);
    }
    __syncthreads();  // the ring is reused by the next segment
  } else {
    // token-split: merge the WT waves' states for the shared 16 rows via LDS
    static_assert(C::RT == 1, "token-split layout holds one row tile");
    __syncthreads();  // every wave is done with its ring
    const float lt = wave_sum16(st.l[0]);
    MLA_LDS char* xo = ring_all;  // [WT][DT][64] f32x4
    MLA_LDS float* xs = (MLA_LDS float*)(ring_all + C::WT * C::DT * 64 * 16);  // m,l [WT][2][16]
#pragma unroll
    for (int d = 0; d < C::DT; ++d)
      *(MLA_LDS f32x4_t*)(xo + ((wt * C::DT + d) * 64 + lane) * 16) = st.o[0][d];
    if (g == 0) {
      xs[(wt * 2 + 0) * 16 + li] = st.m[0];
      xs[(wt * 2 + 1) * 16 + li] = lt;
    }
    __syncthreads();
    float mw[C::WT], aw[C::WT];
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < C::WT; ++w) {
      mw[w] = xs[(w * 2 + 0) * 16 + li];
      M = fmaxf(M, mw[w]);
    }
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < C::WT; ++w) {
      aw[w] = mw[w] == kNegInf ? 0.f : fast_exp2(mw[w] - M);
      Lt += aw[w] * xs[(w * 2 + 1) * 16 + li];
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    const float lse2 = Lt > 0.f ? M + fast_log2(Lt) : kNegInf;
    // wave wt finalises column tiles [wt*DT/WT, (wt+1)*DT/WT)
    constexpr int DPW = C::DT / C::WT;
    f32x4_t acc[DPW];
#pragma unroll
    for (int d = 0; d < DPW; ++d) acc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dd = 0; dd < DPW; ++dd) {
      const int d = wt * DPW + dd;
#pragma unroll
      for (int w = 0; w < C::WT; ++w)
        acc[dd] += aw[w] * *(const MLA_LDS f32x4_t*)(xo + ((w * C::DT + d) * 64 + lane) * 16);
    }
    // write this wave's quarter: reuse store_row on a shifted column window
    const int rows_seq2 = p.q_len * p.n_heads;
    const int r = unit_row0 + li;
    if (r < rows_seq2) {
      if (slot >= 0) {
        float* dst = p.part_o + ((int64_t)slot * p.rows_per_unit + li) * kKvRank + 4 * g;
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
          *(f32x4_t*)(dst + 16 * (wt * DPW + dd)) = acc[dd] * inv;
        if (g == 0 && wt == 0) p.part_lse[(int64_t)slot * p.rows_per_unit + li] = lse2;
      } else {
        const int qi = r / p.n_heads, qh = r % p.n_heads;
        const int64_t ooff =
            (int64_t)b * p.o_s0 + (int64_t)qi * p.o_s1 + (int64_t)qh * p.o_s2 + 4 * g;
        if constexpr (C::F32) {
          float* dst = (float*)p.out + ooff;
#pragma unroll
          for (int dd = 0; dd < DPW; ++dd) *(f32x4_t*)(dst + 16 * (wt * DPW + dd)) = acc[dd] * inv;
        } else {
          uint16_t* dst = (uint16_t*)p.out + ooff;
#pragma unroll
          for (int dd = 0; dd < DPW; ++dd) {
            const f32x4_t x = acc[dd] * inv;
            *(u32x2_t*)(dst + 16 * (wt * DPW + dd)) =
                u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
          }
        }
        if (g == 0 && wt == 0 && p.lse)
          p.lse[(int64_t)b * p.l_s0 + (int64_t)qi * p.l_s1 + (int64_t)qh * p.l_s2] =
              lse2 == kNegInf ? kNegInf : lse2 * kLn2;
      }
    }
    __syncthreads();
  }
}

template <class C>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
decode_partial(DecodeParams p) {
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  __shared__ int sh_scan[256];
  MLA_LDS char* ring = (MLA_LDS char*)smem_raw;
  if (!p.split) {
    const int u = p.num_units - 1 - (int)blockIdx.x;  // heaviest (latest) row tiles first
    process_segment<C>(p, u, 0, 0x7fffffff, -1, ring);
    return;
  }
  unit_scan(p, sh_scan);
  const int total = sh_scan[p.num_units - 1];
  const int chunk = total > 0 ? ceil_div(total, p.grid) : 1;
  const int w0 = (int)blockIdx.x * chunk;
  const int w1 = w0 + chunk < total ? w0 + chunk : total;
  if (w0 >= w1) return;
  // first unit whose work ends past w0
  int lo = 0, hi = p.num_units - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sh_scan[mid] > w0) hi = mid; else lo = mid + 1;
  }
  for (int u = lo; u < p.num_units; ++u) {
    const int end = sh_scan[u];
    const int start = u > 0 ? sh_scan[u - 1] : 0;
    if (start >= w1) break;
    if (end == start) continue;
    const int a = (w0 > start ? w0 : start) - start;
    const int e = (w1 < end ? w1 : end) - start;
    const bool split = (start / chunk) != ((end - 1) / chunk);
    process_segment<C>(p, u, a * kWorkBlock, e * kWorkBlock, split ? (int)blockIdx.x + u : -1, ring);
  }
}

// ------------------------------------------------------------------- merge
// One workgroup per (unit, 4 rows); 64 threads per row, 8 columns each.
template <bool F32>
__global__ void __launch_bounds__(256) decode_merge(DecodeParams p) {
  __shared__ int sh_scan[256];
  unit_scan(p, sh_scan);
  const int groups = (p.rows_per_unit + 3) / 4;
  const int u = blockIdx.x / groups;
  const int row = (blockIdx.x % groups) * 4 + (threadIdx.x >> 6);
  const int c0 = (threadIdx.x & 63) * 8;
  if (u >= p.num_units || row >= p.rows_per_unit) return;
  const int total = sh_scan[p.num_units - 1];
  const int chunk = total > 0 ? ceil_div(total, p.grid) : 1;
  const int end = sh_scan[u], start = u > 0 ? sh_scan[u - 1] : 0;
  const int b = u / p.row_tiles;
  const int r = (u % p.row_tiles) * p.rows_per_unit + row;
  if (r >= p.q_len * p.n_heads) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse2 = kNegInf;
  if (end > start) {
    const int first = start / chunk, last = (end - 1) / chunk;
    if (first == last) return;  // written directly by its only workgroup
    float M = kNegInf;
    for (int w = first; w <= last; ++w)
      M = fmaxf(M, p.part_lse[(int64_t)(w + u) * p.rows_per_unit + row]);
    float Lt = 0.f;
    for (int w = first; w <= last; ++w) {
      const float ls = p.part_lse[(int64_t)(w + u) * p.rows_per_unit + row];
      const float a = ls == kNegInf ? 0.f : fast_exp2(ls - M);
      Lt += a;
      const float* src = p.part_o + ((int64_t)(w + u) * p.rows_per_unit + row) * kKvRank + c0;
      const f32x4_t x0 = *(const f32x4_t*)src, x1 = *(const f32x4_t*)(src + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] += a * x0[j];
        acc[4 + j] += a * x1[j];
      }
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= inv;
    lse2 = Lt > 0.f ? M + fast_log2(Lt) : kNegInf;
  }
  const int qi = r / p.n_heads, qh = r % p.n_heads;
  const int64_t ooff = (int64_t)b * p.o_s0 + (int64_t)qi * p.o_s1 + (int64_t)qh * p.o_s2 + c0;
  if constexpr (F32) {
    float* dst = (float*)p.out + ooff;
    *(f32x4_t*)dst = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4_t*)(dst + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  } else {
    uint16_t* dst = (uint16_t*)p.out + ooff;
    *(u32x4_t*)dst = u32x4_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                             pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  }
  if (c0 == 0 && p.lse)
    p.lse[(int64_t)b * p.l_s0 + (int64_t)qi * p.l_s1 + (int64_t)qh * p.l_s2] =
        lse2 == kNegInf ? kNegInf : lse2 * kLn2;
}

// ------------------------------------------------------------- variants
// id: layout (token-split / row-split), rope width, dtype
using TokSplit64 = Cfg<64, 1, 4, 1, 16, 2, false>;
using TokSplit0 = Cfg<0, 1, 4, 1, 16, 2, false>;
using RowSplit64 = Cfg<64, 4, 1, 1, 32, 4, false>;
using RowSplit0 = Cfg<0, 4, 1, 1, 32, 4, false>;
using TokSplitF64 = Cfg<64, 1, 4, 1, 16, 1, true>;
using TokSplitF0 = Cfg<0, 1, 4, 1, 16, 1, true>;

enum Variant { kTok64 = 0, kTok0, kRow64, kRow0, kTokF64, kTokF0 };

template <class C>
hipError_t launch_variant(const DecodePlan& plan, const DecodeParams& p, hipStream_t s) {
  const size_t smem = C::SMEM_BYTES;
  static bool attr_set = false;  // the attribute is per function, set once per process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_partial<C>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipError_t e;
  hipLaunchKernelGGL(decode_partial<C>, dim3(plan.grid), dim3(C::NT), smem, s, p);
  e = hipGetLastError();
  if (e != hipSuccess || !plan.split) return e;
  const int groups = (plan.rows_per_unit + 3) / 4;
  hipLaunchKernelGGL(decode_merge<C::F32>, dim3(plan.num_units * groups), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int plan_decode(int64_t batch, int64_t q_len, int64_t n_heads, int64_t rope, int64_t max_seqlen,
                int is_f32, DecodePlan* plan) {
  const int64_t rows = q_len * n_heads;
  const bool row_split = !is_f32 && rows > 16;
  int variant;
  int rtile;
  if (is_f32) {
    variant = rope ? kTokF64 : kTokF0;
    rtile = 16;
  } else if (row_split) {
    variant = rope ? kRow64 : kRow0;
    rtile = RowSplit64::RTILE;
  } else {
    variant = rope ? kTok64 : kTok0;
    rtile = 16;
  }
  const int64_t row_tiles = (rows + rtile - 1) / rtile;
  const int64_t units = batch * row_tiles;
  if (units > (int64_t)1 << 30) return -1;
  plan->variant = variant;
  plan->rows_per_unit = rtile;
  plan->row_tiles = (int)row_tiles;
  plan->num_units = (int)units;
  const int64_t wb_bound = batch * row_tiles * ((max_seqlen + kWorkBlock - 1) / kWorkBlock);
  if (units < kSplitUnits && wb_bound > units) {
    plan->split = 1;
    int64_t g = 256;
    if (g > wb_bound) g = wb_bound;
    plan->grid = (int)g;
    const int64_t slots = g + units;
    plan->workspace_bytes = (size_t)(slots * rtile * (kKvRank + 1) * 4 + 256);
  } else {
    plan->split = 0;
    plan->grid = (int)units;
    plan->workspace_bytes = 0;
  }
  return 0;
}

hipError_t launch_decode(const DecodePlan& plan, DecodeParams p, int64_t rope, int is_f32,
                         hipStream_t s) {
  (void)rope;
  (void)is_f32;
  if (plan.grid <= 0) return hipSuccess;
  switch (plan.variant) {
    case kTok64: return launch_variant<TokSplit64>(plan, p, s);
    case kTok0: return launch_variant<TokSplit0>(plan, p, s);
    case kRow64: return launch_variant<RowSplit64>(plan, p, s);
    case kRow0: return launch_variant<RowSplit0>(plan, p, s);
    case kTokF64: return launch_variant<TokSplitF64>(plan, p, s);
    case kTokF0: return launch_variant<TokSplitF0>(plan, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mla
