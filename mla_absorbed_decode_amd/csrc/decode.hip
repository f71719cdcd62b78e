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
// rows that share every key. A unit's visible keys are cut into work blocks
// of one tile each. With many units (prefill) each workgroup takes one unit. With few
// units (decode) the work blocks of all units are laid end to end and cut
// into `grid` equal chunks, one per workgroup; a unit that lands in more than
// one chunk is written as normalised partial rows (bf16 for bf16 inputs, f32
// for f32) plus an f32 log2-domain lse per chunk and merged by decode_merge in
// chunk order (deterministic). The plan
// depends only on seqlens and sizes, never on strides or pointers.
//
// Inside a workgroup
// ------------------
// Keys are staged through LDS in tiles of TT tokens with direct global->LDS
// 16-byte loads, NSLOT tiles deep; four waves each load a quarter of every
// tile and one barrier per tile publishes it. The compute waves split the
// unit's rows (WR row tiles of 16) and the 512 output columns (WC groups):
// with few heads (the HBM-bound decode) four compute waves of 16 rows x 128
// columns fed by four dedicated loader waves; with 32 or 64 rows per unit
// eight waves (two per SIMD, so one wave's LDS waits hide behind the other's
// MFMAs) of 16 rows x 128 or 256 columns. The waves that share rows split the
// score contraction by k-step and add their partial scores through LDS, so
// nothing is recomputed. Per tile a wave computes
//   S^T[token, row]  = sum_e K[token, e] * Q[row, e]        (MFMA, bf16 -> f32)
//   online softmax per row (exp2 domain, lazy rescale when the max grows by
//   more than 2^8)
//   O^T[d, row]     += sum_token V[token, d] * P[row, token] (MFMA)
// where V is the first 512 columns of the staged K rows, read transposed with
// ds_read_b64_tr_b16. S^T's accumulator layout gives each lane one row and
// four tokens, which is exactly the B operand layout P^T needs, so P never
// leaves registers. Operand reads from LDS are software-pipelined in
// double-buffered batches so several are in flight behind each MFMA.
#include <math.h>

#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

typedef __attribute__((address_space(4))) const int32_t cint32_t;  // scalar-loadable view

constexpr float kLn2 = 0.693147180559945309f;
constexpr int kBlkCache = 1024;  // block-table entries a workgroup stages in LDS
constexpr float kRescaleLog2 = 8.0f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// n / d for n >= 0 with a FastDiv prepared on the host.
__device__ __forceinline__ int fdiv(int n, const FastDiv& d) {
  const uint32_t x = (uint32_t)n, t = __umulhi(x, d.mul);
  return (int)((t + ((x - t) >> d.sh1)) >> d.sh2);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Page of token j (a shift for power-of-two pages).
__device__ __forceinline__ int page_of(const DecodeParams& p, int j) {
  return p.page_shift >= 0 ? j >> p.page_shift : j / p.page;
}

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
// (the same for a sequence length s already read)
__device__ __forceinline__ int unit_kvlen_s(const DecodeParams& p, int u, int s) {
  const int b = fdiv(u, p.div_rt), rt = u - b * p.row_tiles;
  const int rows = p.q_len * p.n_heads;
  int r_last = (rt + 1) * p.rows_per_unit;
  r_last = (r_last > rows ? rows : r_last) - 1;
  return row_limit(p, s, p.q_len == 1 ? 0 : fdiv(r_last, p.div_nh));
}
__device__ __forceinline__ int unit_kvlen(const DecodeParams& p, int u) {
  return unit_kvlen_s(p, u, seq_len(p, fdiv(u, p.div_rt)));
}

// Split plan: unit u occupies plan positions [scan[u-1], scan[u]) where scan
// is the inclusive prefix of unit costs in work blocks of p.wb tokens. A unit
// with keys costs its work blocks plus p.alpha for entering it; the first
// alpha of its positions hold no keys, position scan[u-1] + alpha + i is work
// block i. A unit with no keys costs nothing. The positions are cut into
// chunks of ceil(total / grid), one per workgroup.
//
// The merge's copy of the plan: every unit's scan value, computed by wave 0
// with register shuffles (up to kSplitUnits units, kUPL per lane) and
// published in sh[0 .. kSplitUnits) with one barrier.
// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves (no
// LDS round trips): shifts by 1, 2, 4 and 8 within each row of 16 lanes, then
// lane 15 of rows 0 and 2 added to rows 1 and 3, then lane 31 to rows 2 and 3.
// Lanes without a source read 0.
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, true);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, true);  // row_bcast:31, rows 2 and 3
  return x;
}

// a wave-uniform value, held in a scalar register
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int lane_value(int x, int src) {
  return __builtin_amdgcn_readlane(x, src);
}

// Lane src's value of x for a wave-uniform src in [0, 64): v_readlane, a few
// cycles, where __shfl would be an LDS permute round trip per call. Indices
// past 63 wrap (their weights are never used).
__device__ __forceinline__ float lane_weight(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src & 63));
}

constexpr int kUPL = kSplitUnits / 64;  // units per lane of the planning wave

// A[k] for a wave-uniform k < N, as a chain of selects (no dynamic register indexing).
template <class T, int N>
__device__ __forceinline__ T pick(const T (&a)[N], int k) {
  T r = a[0];
#pragma unroll
  for (int j = 1; j < N; ++j)
    if (j == k) r = a[j];
  return r;
}

__device__ void plan_units(const DecodeParams& p, int* sh) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (p.num_units + 63) >> 6;  // units per lane, at most kUPL
    int v[kUPL], run = 0;
#pragma unroll
    for (int k = 0; k < kUPL; ++k) {
      if (k >= per) break;
      const int u = lane * per + k;
      const int n = u < p.num_units ? unit_kvlen(p, u) : 0;
      run += n > 0 ? ceil_div(n, p.wb) + p.alpha : 0;
      v[k] = run;
    }
    const int excl = wave_scan_incl(run) - run;
#pragma unroll
    for (int k = 0; k < kUPL; ++k) {
      if (k >= per) break;
      if (lane * per + k < kSplitUnits) sh[lane * per + k] = excl + v[k];
    }
  }
  __syncthreads();
}

// The part of the plan a workgroup walks.
struct SegHdr {
  int u0, u1;  // first and last unit with keys in the workgroup's positions (u0 > u1: none)
  int tlo0;    // first key of u0 (units after it start at key 0)
  int thi1;    // end key of u1 (units before it end at their last visible key)
  int nsteps;  // stream items: key tiles, plus a query tile per segment after the first (QT)
};
// The same in LDS, with per-unit tables indexed by u in split mode and by 0
// for the one unit of a workgroup without split: the unit's visible keys, its
// sequence's length and the staged block-table position of its first page,
// and bit masks of the units in range and of those whose keys reach other
// workgroups too (written as partials for the merge).
struct SegLds {
  int kv[kSplitUnits];
  int sl[kSplitUnits];
  int poff[kSplitUnits];
  uint64_t live[kUPL];
  uint64_t part[kUPL];
  SegHdr hdr;
  int ubase;    // the per-unit tables and masks hold units ubase, ubase + 1, ...
  int ncache;   // leading stream pages staged in sh_blk (the rest come from the block table)
  int nstaged;  // of those, the ones the segments use
  uint32_t xs_ctr;  // compute-wave rendezvous of the split score contraction (loader layouts)
  uint32_t xs_gaveup;  // set by a compute wave whose rendezvous wait gave up (follows xs_ctr)
};
// LDS besides the tile ring and score exchange: the workgroup's plan and the
// staged block table
constexpr int kStaticLds = (int)sizeof(SegLds) + kBlkCache * 4;
// the static LDS, rounded up to whole 4 KB for the budget check
constexpr int kStaticLdsAlloc = (kStaticLds + 4095) / 4096 * 4096;

// Block-table entries staged in LDS: entry e of the stage is read by lane
// e % 64 of wave 0, from block-table index idx[e / 64] (0, always a valid
// index, where e is past the segments' pages).
constexpr int kStagePer = kBlkCache / 64;
struct StageRefs {
  int64_t idx[kStagePer];
};
// Mark the stage entries [po, po + np) as pages pf, pf + 1, ... of sequence b.
__device__ __forceinline__ void stage_segment(const DecodeParams& p, StageRefs& st, int b, int pf,
                                              int po, int np) {
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)b * p.bt_s0 + pf - po;
#pragma unroll
  for (int k = 0; k < kStagePer; ++k) {
    const int e = 64 * k + lane;
    const bool in = (uint32_t)(e - po) < (uint32_t)np;  // po <= e < po + np
    st.idx[k] = in ? base + e : st.idx[k];
  }
}
// Read the first n stage entries (all in one round trip) into registers. n is
// wave-uniform; n > 0 implies a non-empty block table.
__device__ __forceinline__ void stage_fetch(const DecodeParams& p, const StageRefs& st, int n,
                                            int* v) {
#pragma unroll
  for (int k = 0; k < kStagePer; ++k)
    if (64 * k < n) v[k] = p.block_table[st.idx[k]];
}
// The fetched entries into sh_blk, clamped to [0, num_blocks) so every tile
// read stays inside the cache.
__device__ __forceinline__ void stage_store(const DecodeParams& p, int n, const int* v,
                                            int* sh_blk) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < kStagePer; ++k)
    if (64 * k < n)
      sh_blk[64 * k + lane] = v[k] < 0 ? 0 : (v[k] >= p.num_blocks ? (int)p.num_blocks - 1 : v[k]);
}
__device__ __forceinline__ void stage_read(const DecodeParams& p, const StageRefs& st, int n,
                                           int* sh_blk) {
  int v[kStagePer];
  stage_fetch(p, st, n, v);
  stage_store(p, n, v, sh_blk);
}

// Build the workgroup's SegLds and stage its block-table entries in one pass
// of wave 0, then one barrier. In split mode lane l holds units l, l + 64,
// l + 128, ... (kUPL of them), so that a ballot over the lanes is one 64-unit
// word of a mask; every unit's cost, plan positions, overlap with this workgroup's
// chunk, key range, tiles and pages are computed side by side rather than
// walked unit by unit. Without split the workgroup's one unit is the whole
// table. The stage holds the first kBlkCache pages of the segments in stream
// order; the loader reads any beyond that from global memory.
template <class C>
__device__ void plan_workgroup(const DecodeParams& p, SegLds* tab, int* sh_blk,
                               MLA_LDS int* scratch) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    StageRefs st;
#pragma unroll
    for (int k = 0; k < kStagePer; ++k) st.idx[k] = 0;
    if (!p.split) {
      const int u = p.num_units - 1 - (int)blockIdx.x;  // heaviest row tiles first
      const int b = fdiv(u, p.div_rt);
      // the first entries of the sequence's block-table row, read in the same
      // round trip as its length (the ones past its pages are not used)
      const int nb_max = p.max_blocks < kBlkCache ? p.max_blocks : kBlkCache;
      stage_segment(p, st, b, 0, 0, nb_max);
      int v[kStagePer];
      stage_fetch(p, st, nb_max, v);
      const int n = unit_kvlen(p, u);
      const int np = n > 0 ? page_of(p, n - 1) + 1 : 0;
      stage_store(p, np < kBlkCache ? np : kBlkCache, v, sh_blk);
      if (lane == 0) {
        tab->kv[0] = n;
        tab->sl[0] = seq_len(p, b);
        tab->poff[0] = 0;
        tab->live[0] = 1ull;  // the one unit, whole in this workgroup
        tab->part[0] = 0ull;
        tab->ubase = 0;
        tab->ncache = kBlkCache;
        tab->nstaged = np < kBlkCache ? np : kBlkCache;
        tab->hdr.u0 = tab->hdr.u1 = u;
        tab->hdr.tlo0 = 0;
        tab->hdr.thi1 = n;
        tab->hdr.nsteps = n > 0 ? ceil_div(n, C::TT) : 0;
      }
    } else {
      // Per-unit values go to LDS as they are computed -- tab's tables, and
      // scratch tables in the tile ring, which no tile has reached yet -- so
      // the pass keeps no register array per unit. Lane l handles units l,
      // l + 64, ...; each lane reads back only what it wrote itself, except
      // for the wave-uniform reads of the staging loop (one wave, so LDS
      // order is program order).
      MLA_LDS int* t_incl = scratch;
      MLA_LDS int* t_cost = scratch + kSplitUnits;
      MLA_LDS int* t_tlo = scratch + 2 * kSplitUnits;
      MLA_LDS int* t_thi = scratch + 3 * kSplitUnits;
      MLA_LDS int* t_pages = scratch + 4 * kSplitUnits;
      const int nk = (p.num_units + 63) >> 6;  // units per lane, at most kUPL
      int slv[kUPL];  // the lane's sequence lengths, all read in one round trip
#pragma unroll
      for (int k = 0; k < kUPL; ++k) {
        if (k >= nk) break;
        const int u = lane + 64 * k;
        slv[k] = u < p.num_units ? seq_len(p, fdiv(u, p.div_rt)) : 0;
      }
      int run = 0;
#pragma unroll
      for (int k = 0; k < kUPL; ++k) {
        if (k >= nk) break;
        const int u = lane + 64 * k;
        const int n = u < p.num_units ? unit_kvlen_s(p, u, slv[k]) : 0;
        const int cost = n > 0 ? ceil_div(n, C::TT) + p.alpha : 0;  // work blocks are tiles
        const int x = wave_scan_incl(cost);
        t_incl[u] = x + run;
        t_cost[u] = cost;
        tab->kv[u] = n;
        tab->sl[u] = slv[k];
        run += lane_value(x, 63);
      }
      const int total = run;
      const int chunk = total > 0 ? ceil_div(total, p.grid) : 1;
      const int w0 = (int)blockIdx.x * chunk;
      const int w1 = w0 + chunk < total ? w0 + chunk : total;
      int u0 = kSplitUnits, u1 = -1, steps = 0, prun = 0;
#pragma unroll
      for (int k = 0; k < kUPL; ++k) {
        if (k >= nk) break;
        const int u = lane + 64 * k;
        const int n = tab->kv[u], cost = t_cost[u], incl = t_incl[u];
        const int first = incl - cost + p.alpha, end = incl;
        const int lo = w0 > first ? w0 : first, hi = w1 < end ? w1 : end;
        const bool in = cost > 0 && lo < hi;
        const int tlo = (lo - first) * C::TT;
        const int thi = (hi - first) * C::TT < n ? (hi - first) * C::TT : n;
        const int pages = in ? page_of(p, thi - 1) - page_of(p, tlo) + 1 : 0;
        const uint64_t live = __ballot(in);
        // whole in this workgroup only if it starts and ends inside its chunk
        const uint64_t part = __ballot(in && !(first >= w0 && end <= w0 + chunk));
        if (live && u0 == kSplitUnits) u0 = 64 * k + __builtin_ctzll(live);
        if (live) u1 = 64 * k + 63 - __builtin_clzll(live);
        steps += (in ? ceil_div(thi - tlo, C::TT) : 0) + (C::QT && in && u != u0 ? 1 : 0);
        const int x = wave_scan_incl(pages);
        tab->poff[u] = x - pages + prun;
        prun += lane_value(x, 63);
        t_tlo[u] = tlo;
        t_thi[u] = thi;
        t_pages[u] = pages;
        if (lane == 0) {
          tab->live[k] = live;
          tab->part[k] = part;
        }
      }
      // key range ends of the first and last units
      const int a = u0 <= u1 ? t_tlo[u0] : 0, z = u0 <= u1 ? t_thi[u1] : 0;
      steps = lane_value(wave_scan_incl(steps), 63);
      // stage the pages of every unit in range, in unit order: one pass per segment
      for (int u = u0; u <= u1;) {
        stage_segment(p, st, fdiv(u, p.div_rt), page_of(p, uni(t_tlo[u])), uni(tab->poff[u]),
                      uni(t_pages[u]));
        // next unit in range
        int nu = kSplitUnits;
        for (int w = (u + 1) >> 6; w < nk; ++w) {
          const uint64_t lw = tab->live[w];
          const uint64_t m = w == ((u + 1) >> 6) ? lw & (~0ull << ((u + 1) & 63)) : lw;
          if (m) {
            nu = 64 * w + __builtin_ctzll(m);
            break;
          }
        }
        u = nu;
      }
      stage_read(p, st, prun < kBlkCache ? prun : kBlkCache, sh_blk);
      if (lane == 0) {
        tab->ubase = 0;
        tab->ncache = kBlkCache;
        tab->nstaged = prun < kBlkCache ? prun : kBlkCache;
        tab->hdr.u0 = u0;
        tab->hdr.u1 = u1;
        tab->hdr.tlo0 = a;
        tab->hdr.thi1 = z;
        tab->hdr.nsteps = steps;
      }
    }
  }
  __syncthreads();
}

// ------------------------------------------------ a plan shared by calls
// The call's sizes a plan is tied to: 16 header ints after the magic check.
__device__ __forceinline__ int plan_field(const DecodeParams& p, int i) {
  switch (i) {
    case 0: return kPlanMagic;
    case 1: return p.variant;
    case 2: return p.grid;
    case 3: return p.num_units;
    case 4: return p.batch;
    case 5: return p.q_len;
    case 6: return p.n_heads;
    case 7: return p.page;
    case 8: return p.wb;
    case 9: return p.alpha;
    case 10: return p.causal;
    case 11: return p.max_blocks;
    case 12: return (int)p.num_blocks;
    case 13: return p.seq_cap;
    case 14: return p.rows_per_unit;
    default: return p.row_tiles;
  }
}

// Read the merge's copy of the plan (the inclusive cost scan) into sh from
// p.plan; false (nothing read) when the plan's header is not this call's.
// Every thread of the workgroup takes part.
__device__ bool load_scan(const DecodeParams& p, int* sh) {
  __shared__ int ok;
  if (threadIdx.x == 0) ok = 1;
  __syncthreads();
  if (threadIdx.x < 16 && p.plan[threadIdx.x] != plan_field(p, threadIdx.x)) ok = 0;
  for (int u = threadIdx.x; u < p.num_units; u += blockDim.x) sh[u] = p.plan[kPlanHdrInts + u];
  __syncthreads();
  return ok != 0;
}

// This workgroup's part of a plan computed beforehand: the descriptor and the
// header in one round trip (through scratch LDS), then the per-unit tables,
// masks and staged block ids, as plan_workgroup leaves them (tables indexed
// from the first unit in range). False (nothing written) when the header is
// not this call's or the descriptor holds too many units.
template <class C>
__device__ bool load_plan(const DecodeParams& p, SegLds* tab, int* sh_blk, MLA_LDS int* scratch) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int* d = p.plan + kPlanHdrInts + kSplitUnits + (int64_t)blockIdx.x * kDescInts;
  for (int i = t; i < kDescInts / 4; i += C::NT) {
    const u32x4_t v = ((const u32x4_t*)d)[i];
    *(MLA_LDS u32x4_t*)(scratch + 4 * i) = v;
  }
  if (t < 16) scratch[kDescInts + t] = (int)(p.plan[t] != plan_field(p, t));
  __syncthreads();
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) bad |= scratch[kDescInts + i];
  const int n = scratch[5];
  const int npg = scratch[6] < 0 ? 0 : (scratch[6] < kDescPages ? scratch[6] : kDescPages);
  // the same values in every thread; the fallback plan overwrites scratch
  // only after every wave has read them
  if (bad || n < 0 || n > kDescUnits) {
    __syncthreads();
    return false;
  }
#pragma unroll
  for (int wd = wave; wd < kUPL; wd += C::NW + C::NP) {
    const int i = 64 * wd + lane;
    const int fl = i < n ? scratch[8 + 4 * i + 3] : 0;
    if (i < n) {
      tab->kv[i] = scratch[8 + 4 * i];
      tab->sl[i] = scratch[8 + 4 * i + 1];
      tab->poff[i] = scratch[8 + 4 * i + 2];
    }
    const uint64_t live = __ballot(fl & 1), part = __ballot(fl & 2);
    if (lane == 0) {
      tab->live[wd] = live;
      tab->part[wd] = part;
    }
  }
  for (int i = t; i < npg; i += C::NT) sh_blk[i] = scratch[kDescPageOff + i];
  if (t == 0) {
    tab->hdr.u0 = scratch[0];
    tab->hdr.u1 = scratch[1];
    tab->hdr.tlo0 = scratch[2];
    tab->hdr.thi1 = scratch[3];
    tab->hdr.nsteps = scratch[4];
    tab->ubase = scratch[0];
    tab->ncache = npg;
    tab->nstaged = npg;
  }
  __syncthreads();
  return true;
}

// R: rope width; WR x WC compute waves split the unit's rows and the 512
// output columns; RT row tiles of 16 per wave; TT-token tiles, NSLOT deep;
// F32 values; XS: the waves sharing rows split the score contraction; NP:
// dedicated loader waves (0: the compute waves load); KV8: an fp8 (e4m3) cache
// whose loader waves widen each row to bf16 on its way into LDS, so the LDS
// tile and the compute are the bf16 ones. KV8 reads every stream item (key
// tile or query tile) global->LDS into one of NS8 staging slots, NS8 items
// ahead; at its step each loader lane widens (or, for query rows,
// copies) the bytes it read itself into the NSLOT-deep bf16 ring.
template <int R_, int WR_, int WC_, int RT_, int TT_, int NSLOT_, bool F32_, bool XS_, int NP_,
          bool KV8_ = false>
struct Cfg {
  static constexpr int R = R_, WR = WR_, WC = WC_, RT = RT_, TT = TT_, NSLOT = NSLOT_;
  static constexpr bool F32 = F32_, XS = XS_ && WC_ > 1;
  static constexpr int NP = NP_;
  static constexpr bool KV8 = KV8_;
  static constexpr int ES = F32 ? 4 : 2;           // element bytes (queries, LDS tile)
  static constexpr int GES = KV8 ? 1 : ES;         // cache element bytes
  static constexpr int E = kKvRank + R;            // latent row width
  static constexpr int PITCH = E * ES;             // bytes per staged row
  static constexpr int CH = PITCH / 16;            // 16-byte chunks per row
  static constexpr int NW = WR * WC;               // compute waves
  // loader waves: the dedicated ones, else the first four compute waves
  static constexpr int LW = NP > 0 ? NP : (NW < 4 ? NW : 4);
  static constexpr int NT = 64 * (NW + NP);
  static constexpr int ROWS_W = 16 * RT;
  static constexpr int RTILE = ROWS_W * WR;        // rows per unit
  static constexpr int TILE_BYTES = TT * PITCH;
  static constexpr int LPT = TT * CH / 64;         // 16-byte loads per tile per 64 lanes
  static constexpr int LPW = LPT / LW;             // issued by each loader wave
  static constexpr int SUB = TT / 16;              // 16-token sub-tiles
  static constexpr int KSTEPS = F32 ? E / 16 : E / 32;  // 64-byte k-steps of a latent row
  static constexpr int DT = kKvRank / 16;          // 32 output column tiles
  static constexpr int DW = DT / WC;               // column tiles per wave
  // With XS the WC waves that share rows split the score contraction: wave
  // wc takes k-steps wc, wc + WC, wc + 2 WC, ... (at most KW of them) and the
  // partial scores are summed through LDS in wave order.
  static constexpr int KW = XS ? (KSTEPS + WC - 1) / WC : KSTEPS;
  // partial score blocks; the layouts without loader waves alternate between two
  // copies (their one barrier per tile sits at the exchange)
  static constexpr int XCHG_HALF = XS ? NW * SUB * RT * 64 : 0;  // f32x4 per copy
  static constexpr int XCHG_BYTES = XCHG_HALF * 16 * (NP == 0 ? 2 : 1);
  static constexpr int RING_BYTES = NSLOT * TILE_BYTES;
  // KV8 staging: a key tile as e4m3 bytes (TT rows of E) or a query tile as
  // bf16 (RTILE rows of 2E), P8 / QI 1 KB reads, L8 of them per loader wave
  static constexpr int P8 = KV8 ? TT * E / 1024 : 0;
  static constexpr int STAGE_SLOT = KV8 ? (TT * E > RTILE * E * 2 ? TT * E : RTILE * E * 2) : 0;
  // staging depth: items read ahead of the one being landed. Two: with more
  // bytes in flight per CU the stream gets slower on MI355X (the V2-Lite fp8
  // call measured 40.1 us with two, 40.7-40.8 with three, 41.0-41.4 with four)
  static constexpr int NS8 = KV8 ? 2 : 1;
  static constexpr int STAGE_BYTES = KV8 ? NS8 * STAGE_SLOT : 0;
  static constexpr int SMEM_BYTES = RING_BYTES + XCHG_BYTES + STAGE_BYTES;
  // With loader waves the query rows of every segment but the first travel
  // through the ring as a tile of their own ahead of its key tiles (QI 1 KB
  // reads); the first segment's are read straight into registers.
  static constexpr bool QT = NP > 0;
  static constexpr int QI = RTILE * CH / 64;
  static constexpr int L8 = KV8 ? ((P8 > QI ? P8 : QI) + NP - 1) / (NP > 0 ? NP : 1) : 0;
  // operand-read batches (rows not shared): K reads per batch kept at about 6
  static constexpr int KB = F32 ? (KSTEPS % 6 == 0 ? 6 : 4) : (SUB == 1 ? (KSTEPS % 6 == 0 ? 6 : 4)
                                                : (KSTEPS % 3 == 0 ? 3 : 4));
  static constexpr int PB = 4;
  // Latent rows stream with the non-temporal policy in the bf16 layouts of at
  // most 32 rows: on the 128-head decode's 32-row units (four units of a
  // sequence read the same keys) 28.1 us against 28.6 us with the default
  // policy. The 64-row layout keeps the default policy, which lets a
  // sequence's other units hit in the caches (non-temporal reads cost it 7 %).
  static constexpr bool STREAM = !F32 && RTILE <= 32;
  static_assert(NW == 4 || (NW == 8 && NP == 0), "four compute waves, or eight that load too");
  static_assert(NP == 0 || NP == 4, "no loader waves, or four");
  static_assert(!XS || NP == 0 || WR == 1, "with loader waves the exchange spans all compute waves");
  static_assert(!QT || (RTILE <= TT && QI * 64 == RTILE * CH && QI <= LPT), "query tile fits a slot");
  static_assert(!XS || WC % 2 == 0, "k-step parity is the wave's when WC is even");
  static_assert(LPT * 64 == TT * CH, "tile chunk count");
  static_assert(LPW * LW == LPT, "tile loads split evenly over the loader waves");
  static_assert(TT == 16 || TT == 32, "tile size");
  static_assert(!F32 || TT == 16, "the f32 path uses 16-token tiles");
  static_assert(NSLOT >= 2 && NSLOT <= 4, "ring depth");
  static_assert(KSTEPS % KB == 0 && DW % PB == 0, "batching");
  static_assert(SMEM_BYTES + kStaticLdsAlloc <= 160 * 1024, "LDS budget");
  static_assert(RING_BYTES >= 5 * kSplitUnits * 4, "the split plan's tables fit in the ring");
  static_assert(!KV8 || (!F32 && NP > 0 && TT * E % 1024 == 0 && L8 * NP >= P8 && L8 * NP >= QI &&
                         P8 <= 64 && QI <= 64),
                "fp8: bf16 compute, loader waves, whole 1 KB staging reads");
};

// Everything a wave carries through one segment.
template <class C>
struct WaveState {
  f32x4_t o[C::RT][C::DW];  // O^T: lane holds row li, columns 16*(dc0+d) + 4*g + j
  float m[C::RT];
  float l[C::RT];
  int lim[C::RT];   // this lane's row: keys [.., lim) visible (already capped by the segment end)
};

// ---------------------------------------------------------------- one tile
// hook(stage): the caller's work at three points of the tile (tile reads to
// issue); mid(): without loader waves, the workgroup barrier between storing
// the partial scores and reading them back.
template <class C, class QReg, class Hook, class Mid>
__device__ __forceinline__ void tile_compute(const MLA_LDS char* tile, MLA_LDS f32x4_t* xchg,
                                             int j0, const QReg& qreg, WaveState<C>& st,
                                             float scale_log2, int wr, int wc, int dc0,
                                             const Hook& hook, const Mid& mid,
                                             MLA_LDS uint32_t* xs_ctr,
                                             int& xs_seq, int& xs_bad, int rendezvous_polls) {
  const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  f32x4_t s[C::SUB][C::RT];

  if constexpr (C::XS) {
    // ---- partial S^T over this wave's k-steps kg = wc + WC*kk. Chunk 4kg + g
    // is stored at 8*(kg/2) + ((4*(kg%2) + g) ^ swz); kg%2 = wc%2 and
    // kg/2 = wc/2 + (WC/2)*kk, so one lane base and immediate offsets.
    using KV = typename std::conditional<C::F32, f32x4_t, i16x8_t>::type;
    const MLA_LDS char* kb = tile + li * C::PITCH + 128 * (wc >> 1) +
                             (((4 * (wc & 1) + g) ^ lds_swz(li)) << 4);
    const bool has_last = wc + C::WC * (C::KW - 1) < C::KSTEPS;
    KV kbuf[C::KW][C::SUB];
#pragma unroll
    for (int kk = 0; kk < C::KW; ++kk)
      if (kk < C::KW - 1 || has_last)
#pragma unroll
        for (int a = 0; a < C::SUB; ++a)
          kbuf[kk][a] = *(const MLA_LDS KV*)(kb + 16 * a * C::PITCH + 64 * C::WC * kk);
    hook(0);
    f32x4_t acc[2][C::SUB][C::RT];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int a = 0; a < C::SUB; ++a)
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) acc[e][a][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KW; ++kk)
      if (kk < C::KW - 1 || has_last)
#pragma unroll
        for (int a = 0; a < C::SUB; ++a)
#pragma unroll
          for (int rt = 0; rt < C::RT; ++rt) {
            if constexpr (C::F32) {
#pragma unroll
              for (int x = 0; x < 4; ++x)
                acc[kk & 1][a][rt] =
                    mfma_16x16x4f32(kbuf[kk][a][x], qreg[rt][kk][x], acc[kk & 1][a][rt]);
            } else {
              acc[kk & 1][a][rt] = mfma_16x16x32(kbuf[kk][a], qreg[rt][kk], acc[kk & 1][a][rt]);
            }
          }
    // ---- exchange: partials [wr][wc][a][rt][lane], summed in wave order so
    // every wave of the row group holds bit-identical scores
    MLA_LDS f32x4_t* mine = xchg + (wr * C::WC + wc) * (C::SUB * C::RT * 64) + lane;
#pragma unroll
    for (int a = 0; a < C::SUB; ++a)
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) mine[(a * C::RT + rt) * 64] = acc[0][a][rt] + acc[1][a][rt];
    if constexpr (C::NP > 0) {
      // The loader waves keep their own barrier schedule, so the compute waves
      // meet on a counter: each adds 1 once its partials are stored, then waits
      // until all NW have added for this tile. Every compute wave makes the same
      // sequence of tile_compute calls between the same workgroup barriers, so
      // the count is reached; the wait is bounded all the same (DecodeParams::rendezvous_polls,
      // 2^22 by default: seconds), and a wave that gives up marks its segments' outputs NaN
      // (xs_bad) rather than use partial scores that may not have landed.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0)
        __hip_atomic_fetch_add(xs_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const uint32_t target = (uint32_t)C::NW * (uint32_t)(xs_seq + 1);
      for (int it = 0; it < rendezvous_polls; ++it) {
        if (__hip_atomic_load(xs_ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target)
          break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (__hip_atomic_load(xs_ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        // tell the other compute waves: every wave that writes part of these
        // rows then marks them, so a row is NaN as a whole, lse included
        xs_bad = 1;
        __hip_atomic_store(xs_ctr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      ++xs_seq;
    } else {
      mid();
    }
    const MLA_LDS f32x4_t* grp = xchg + wr * C::WC * (C::SUB * C::RT * 64) + lane;
    f32x4_t part[C::WC][C::SUB][C::RT];
#pragma unroll
    for (int w = 0; w < C::WC; ++w)
#pragma unroll
      for (int a = 0; a < C::SUB; ++a)
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
          part[w][a][rt] = grp[(w * C::SUB * C::RT + a * C::RT + rt) * 64];
    hook(1);
#pragma unroll
    for (int a = 0; a < C::SUB; ++a)
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) {
        f32x4_t t = part[0][a][rt];
#pragma unroll
        for (int w = 1; w < C::WC; ++w) t += part[w][a][rt];
        s[a][rt] = t;
      }
  } else {
  // ---- S^T = K . Q^T : lane (token li of sub-tile a, e-group g) x (row li, g).
  // Chunk (g + 4kk) ^ swz(li) = 8*(kk/2) + ((g + 4*(kk%2)) ^ swz(li)): two lane
  // bases, the rest is an immediate offset. Two accumulators per block (even
  // and odd kk) halve the MFMA dependency chain.
  {
    const int sw = lds_swz(li);
    const MLA_LDS char* kb0 = tile + li * C::PITCH + ((g ^ sw) << 4);
    const MLA_LDS char* kb1 = tile + li * C::PITCH + (((g + 4) ^ sw) << 4);
    using KV = typename std::conditional<C::F32, f32x4_t, i16x8_t>::type;
    KV kbuf[2][C::KB][C::SUB];
    f32x4_t acc[2][C::SUB][C::RT];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int a = 0; a < C::SUB; ++a)
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) acc[e][a][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto load = [&](int bi, int buf) {
#pragma unroll
      for (int k = 0; k < C::KB; ++k) {
        const int kk = bi * C::KB + k;
        const MLA_LDS char* kb = (kk & 1) ? kb1 : kb0;
#pragma unroll
        for (int a = 0; a < C::SUB; ++a)
          kbuf[buf][k][a] = *(const MLA_LDS KV*)(kb + 16 * a * C::PITCH + 128 * (kk >> 1));
      }
    };
    constexpr int NB = C::KSTEPS / C::KB;
    load(0, 0);
    hook(0);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      if (bi + 1 < NB) load(bi + 1, (bi + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < C::KB; ++k) {
        const int kk = bi * C::KB + k;
#pragma unroll
        for (int a = 0; a < C::SUB; ++a)
#pragma unroll
          for (int rt = 0; rt < C::RT; ++rt) {
            if constexpr (C::F32) {
#pragma unroll
              for (int x = 0; x < 4; ++x)
                acc[kk & 1][a][rt] =
                    mfma_16x16x4f32(kbuf[bi & 1][k][a][x], qreg[rt][kk][x], acc[kk & 1][a][rt]);
            } else {
              acc[kk & 1][a][rt] = mfma_16x16x32(kbuf[bi & 1][k][a], qreg[rt][kk], acc[kk & 1][a][rt]);
            }
          }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int a = 0; a < C::SUB; ++a)
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) s[a][rt] = acc[0][a][rt] + acc[1][a][rt];
    hook(1);
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
      for (int d = 0; d < C::DW; ++d) st.o[rt][d] *= alpha;
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
        for (int j = 0; j < 4; j += 2) {
          const uint32_t w = pack_bf16x2(v[a][j], v[a][j + 1]);
          pb[rt][4 * a + j] = (short)(w & 0xffffu);
          pb[rt][4 * a + j + 1] = (short)(w >> 16);
        }
    }
  }

  // ---- O^T += V^T . P^T : A = V^T (d = li, tokens by g), B = P^T (tokens by g, row li)
  if constexpr (!C::F32) {
    // local lane li points at token row (4g + li/4) [+16], columns 16*d + 4*(li%4);
    // chunk (2d + cx) ^ swz = 8*(d/4) + ((2*(d%4) + cx) ^ swz): four lane bases
    // and immediate offsets (rows r and r + 16 share a swizzle)
    const int rr0 = 4 * g + (li >> 2);
    const int sw0 = lds_swz(rr0);
    const int cx = (li & 3) >> 1, half8 = (li & 1) * 8;
    const MLA_LDS char* vb[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
      vb[x] = tile + rr0 * C::PITCH + (((2 * x + cx) ^ sw0) << 4) + half8 + 32 * dc0;
    i16x4_t vbuf[2][C::PB][C::SUB];
    auto load = [&](int bj, int buf) {
#pragma unroll
      for (int x = 0; x < C::PB; ++x) {
        const int d = bj * C::PB + x;
        const MLA_LDS char* vp = vb[d & 3] + 128 * (d >> 2);
#pragma unroll
        for (int a = 0; a < C::SUB; ++a) vbuf[buf][x][a] = lds_read_tr16(vp + 16 * a * C::PITCH);
      }
    };
    constexpr int NB = C::DW / C::PB;
    load(0, 0);
    hook(2);
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
      if (bj + 1 < NB) load(bj + 1, (bj + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < C::PB; ++x) {
        const int d = bj * C::PB + x;
        if constexpr (C::TT == 32) {
          const i16x4_t v0 = vbuf[bj & 1][x][0], v1 = vbuf[bj & 1][x][1];
          const i16x8_t vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int rt = 0; rt < C::RT; ++rt) st.o[rt][d] = mfma_16x16x32(vv, pb[rt], st.o[rt][d]);
        } else {
#pragma unroll
          for (int rt = 0; rt < C::RT; ++rt)
            st.o[rt][d] = mfma_16x16x16(vbuf[bj & 1][x][0], pb[rt], st.o[rt][d]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // f32: A = V[token 4g + x][16d + li] (one element per lane), MFMA x per token
    float vbuf[2][C::PB][4];
    auto load = [&](int bj, int buf) {
#pragma unroll
      for (int y = 0; y < C::PB; ++y) {
        const int col = 16 * (dc0 + bj * C::PB + y) + li;  // float column
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int rr = 4 * g + x;
          vbuf[buf][y][x] = *(const MLA_LDS float*)(tile + rr * C::PITCH +
                                                      (((col >> 2) ^ lds_swz(rr)) << 4) + (col & 3) * 4);
        }
      }
    };
    constexpr int NB = C::DW / C::PB;
    load(0, 0);
    hook(2);
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
      if (bj + 1 < NB) load(bj + 1, (bj + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int y = 0; y < C::PB; ++y) {
        const int d = bj * C::PB + y;
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int rt = 0; rt < C::RT; ++rt)
            st.o[rt][d] = mfma_16x16x4f32(vbuf[bj & 1][y][x], pf[rt][x], st.o[rt][d]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ------------------------------------------------------ output of a segment
// This lane's row (local_row of the unit), columns 16*(dc0 + d) + 4*g + j.
template <class C>
__device__ __forceinline__ void store_row(const DecodeParams& p, int b, int unit_row0,
                                          int local_row, int slot, const f32x4_t* o, float inv,
                                          float lse2, int dc0, bool write_lse) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
  const int rows_seq = p.q_len * p.n_heads;
  const int r = unit_row0 + local_row;
  if (r >= rows_seq) return;
  const int c0 = 16 * dc0 + 4 * g;
  if (slot >= 0) {
    // split partials: f32 rows for f32 inputs, bf16 rows (the normalised
    // partial rounded once) for bf16 inputs, half the split traffic
    const int64_t off = ((int64_t)slot * p.rows_per_unit + local_row) * kKvRank + c0;
    if constexpr (C::F32) {
      float* dst = p.part_o + off;
#pragma unroll
      for (int d = 0; d < C::DW; ++d) *(f32x4_t*)(dst + 16 * d) = o[d] * inv;
    } else {
      uint16_t* dst = (uint16_t*)p.part_o + off;
#pragma unroll
      for (int d = 0; d < C::DW; ++d) {
        const f32x4_t v = o[d] * inv;
        const u32x2_t w = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        // the layouts without loader waves (32 and 64 rows: units that share keys)
        // and the fp8 layout write their partials with the non-temporal policy:
        // the 128-head decode measured 29.4 -> 28.1 us, the fp8 call 38.3 -> 37.6
        // us; the bf16 few-head layout measured slower with it (37.9 -> 41.0 us,
        // its merge then reading the partials from memory rather than the L2)
        if constexpr (C::NP == 0 || C::KV8) __builtin_nontemporal_store(w, (u32x2_t*)(dst + 16 * d));
        else *(u32x2_t*)(dst + 16 * d) = w;
      }
    }
    if (write_lse && g == 0) {
      float* lp = p.part_lse + (int64_t)slot * p.rows_per_unit + local_row;
      if constexpr (C::NP == 0 || C::KV8) __builtin_nontemporal_store(lse2, lp);
      else *lp = lse2;
    }
    return;
  }
  const int qi = fdiv(r, p.div_nh), qh = r - qi * p.n_heads;
  const int64_t ooff = (int64_t)b * p.o_s0 + (int64_t)qi * p.o_s1 + (int64_t)qh * p.o_s2 + c0;
  if constexpr (C::F32) {
    float* dst = (float*)p.out + ooff;
#pragma unroll
    for (int d = 0; d < C::DW; ++d) *(f32x4_t*)(dst + 16 * d) = o[d] * inv;
  } else {
    uint16_t* dst = (uint16_t*)p.out + ooff;
#pragma unroll
    for (int d = 0; d < C::DW; ++d) {
      const f32x4_t x = o[d] * inv;
      *(u32x2_t*)(dst + 16 * d) = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    }
  }
  if (write_lse && g == 0 && p.lse)
    p.lse[(int64_t)b * p.l_s0 + (int64_t)qi * p.l_s1 + (int64_t)qh * p.l_s2] =
        lse2 == kNegInf ? kNegInf : lse2 * kLn2;
}

// ------------------------------------------------------- a workgroup's keys
// One contiguous run of a unit's keys handled by this workgroup.
struct Seg {
  int u;       // unit
  int b;       // sequence
  int s;       // the sequence's length
  int t_lo;    // first key token
  int t_hi;    // one past the last key token (capped by the unit's visible keys)
  int ntiles;  // tiles of TT tokens
  int slot;    // partial slot, or -1 when this workgroup holds the whole unit
  int poff;    // staged block-table position of the segment's first page
};

__device__ __forceinline__ SegHdr read_hdr(const SegLds* tab) {
  SegHdr h;
  h.u0 = uni(tab->hdr.u0);
  h.u1 = uni(tab->hdr.u1);
  h.tlo0 = uni(tab->hdr.tlo0);
  h.thi1 = uni(tab->hdr.thi1);
  h.nsteps = uni(tab->hdr.nsteps);
  return h;
}

// Unit u's segment from the workgroup's plan (u past the last unit in range:
// an empty segment with u = num_units). The table reads go out together.
template <class C>
__device__ __forceinline__ Seg seg_of(const DecodeParams& p, const SegLds* tab, const SegHdr& h,
                                      int u) {
  const bool valid = u <= h.u1 && u < p.num_units;
  int i = p.split ? u - uni(tab->ubase) : 0;  // table index
  i = i < 0 ? 0 : (i < kSplitUnits ? i : kSplitUnits - 1);
  const int n = uni(tab->kv[i]), s = uni(tab->sl[i]), po = uni(tab->poff[i]);
  const int pw = uni((int)(tab->part[i >> 6] >> (i & 63)));
  Seg sg;
  sg.u = valid ? u : p.num_units;
  sg.b = valid ? fdiv(u, p.div_rt) : 0;
  sg.s = valid ? s : 0;
  sg.t_lo = valid && u == h.u0 ? h.tlo0 : 0;
  sg.t_hi = !valid ? 0 : (u == h.u1 ? h.thi1 : n);
  sg.slot = valid && (pw & 1) ? (int)blockIdx.x + u : -1;
  sg.ntiles = sg.t_hi > sg.t_lo ? ceil_div(sg.t_hi - sg.t_lo, C::TT) : 0;
  sg.poff = valid ? po : 0;
  return sg;
}

// Pages a segment touches (its block-table entries).
__device__ __forceinline__ int seg_pages(const DecodeParams& p, const Seg& sg) {
  return sg.ntiles > 0 ? page_of(p, sg.t_hi - 1) - page_of(p, sg.t_lo) + 1 : 0;
}

// The next unit in the workgroup's range after u, or num_units.
__device__ __forceinline__ int next_live(const DecodeParams& p, const SegLds* tab, int u) {
  if (!p.split) return p.num_units;
  const int base = uni(tab->ubase);
  const int iend = p.num_units - base < kSplitUnits ? p.num_units - base : kSplitUnits;
  for (int i = u + 1 - base; i < iend; i = (i | 63) + 1) {
    const uint64_t w = tab->live[i >> 6] >> (i & 63);
    const uint32_t lo = (uint32_t)uni((int)(uint32_t)w), hi = (uint32_t)uni((int)(uint32_t)(w >> 32));
    const uint64_t ws = ((uint64_t)hi << 32) | lo;
    if (ws) return base + i + __builtin_ctzll(ws);
  }
  return p.num_units;
}

// ------------------------------------------------------ the tile stream
// All tiles of the workgroup's segments form one stream staged through an LDS
// ring of NSLOT tiles, with one workgroup barrier per tile. With NP loader
// waves the barrier opens tile k: before it tile k has landed and every compute
// wave is done with tile k-1, whose slot the reads of tile k + NSLOT - 1 then
// refill, so reads run NSLOT - 1 tiles ahead and the compute waves never stall
// on a full memory queue. Without loader waves the barrier sits at tile k's
// score exchange: before it tile k + 1 has landed and every wave is done with
// tile k - 1, and the waves send the reads of tile k + NSLOT - 1 in three
// groups between their own phases. Either way the stream runs across segment
// boundaries; at a boundary the compute waves write the finished segment (final
// output, or a partial for the merge) and load the next segment's query rows.
template <class C>
__device__ __forceinline__ void process_range(const DecodeParams& p, const SegLds* tab, int* sh_blk,
                                              MLA_LDS char* ring, MLA_LDS f32x4_t* xchg) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const bool loader = C::NP == 0 ? wave < C::LW : wave >= C::NW;
  const bool compute = C::NP == 0 || wave < C::NW;
  const int lwave = C::NP == 0 ? wave : wave - C::NW;  // index among the loader waves
  const int g = lane >> 4, li = lane & 15;
  const int cw = compute ? wave : 0;
  const int wr = cw / C::WC, wc = cw % C::WC;
  const int dc0 = wc * C::DW;  // first output column tile of this wave
  const int wrow0 = wr * C::ROWS_W;
  const int rows_seq = p.q_len * p.n_heads;
  const char* kvbase = (const char*)p.kv;
  const int64_t pitch_g = p.kv_s1 * C::GES;

  const SegHdr h = read_hdr(tab);
  const int nsteps = h.nsteps;

  // ---- loader walker: this wave's share of each tile's reads. A full tile
  // inside one page is read as page base + per-lane offsets computed once
  // here; other tiles (a segment's last, or pages shorter than a tile) take
  // the general path.
  const bool fast_ok = p.page % C::TT == 0 && (int64_t)p.page * pitch_g < ((int64_t)1 << 31);
  uint32_t loff[C::LPW];  // full tile: row * pitch + chunk offset
  int lrow[C::LPW];       // the row; a partial tile clamps it to its last valid row
#pragma unroll
  for (int n = 0; n < C::LPW; ++n) {
    const int idx = (lwave + n * C::LW) * 64 + lane;
    const int r = idx / C::CH, cpos = idx % C::CH;
    lrow[n] = r;
    loff[n] = (uint32_t)(r * pitch_g) + (uint32_t)((cpos ^ lds_swz(r & 15)) << 4);
  }
  const Seg seg0 = seg_of<C>(p, tab, h, h.u0);
  Seg ls = seg0;
  int lk = 0;         // tile within ls
  bool lq = true;     // ls's query tile sent (the first segment has none)
  // cache block of page pg of segment ls (staged entry, or a global read past the stage)
  const int ncache = uni(tab->ncache);
  auto block_of = [&](int pg) -> int {
    const int ti = ls.poff + pg - page_of(p, ls.t_lo);
    int blk;
    if (ti < ncache) {
      blk = sh_blk[ti];
    } else {
      blk = load_scalar_i32(p.block_table, (int64_t)ls.b * p.bt_s0 + pg);
      blk = blk < 0 ? 0 : (blk >= p.num_blocks ? (int)p.num_blocks - 1 : blk);
    }
    return __builtin_amdgcn_readfirstlane(blk);
  };
  struct NextTile {
    const char* base0 = nullptr;
    const char* base1 = nullptr;
    int nvalid = 0;
    int slot = 0;
    bool fast = false;
    bool live = false;
    bool query = false;  // the query rows of a unit: sequence qb, first row qrow0
    int qb = 0;
    int qrow0 = 0;
  };
  auto prep_next = [&](int step) -> NextTile {
    // segments in split mode have tiles; an empty unit (no split) is never reached
    while (lk >= ls.ntiles && (lq || !C::QT) && ls.u < p.num_units) {
      ls = seg_of<C>(p, tab, h, next_live(p, tab, ls.u));
      lk = 0;
      lq = false;
    }
    NextTile t;
    t.live = true;
    t.slot = step % C::NSLOT;
    if (C::QT && !lq) {
      lq = true;
      t.query = true;
      t.qb = ls.b;
      t.qrow0 = (ls.u - ls.b * p.row_tiles) * p.rows_per_unit;
      return t;
    }
    const int j0 = ls.t_lo + lk * C::TT;
    t.nvalid = ls.t_hi - j0 < C::TT ? ls.t_hi - j0 : C::TT;
    ++lk;
    // each 16-token half of the tile lies in one page (page is a multiple of 16)
    const int pg0 = page_of(p, j0);
    const int blk0 = block_of(pg0);
    t.base0 = kvbase + (int64_t)blk0 * p.kv_s0 * C::GES + (int64_t)(j0 - pg0 * p.page) * pitch_g;
    t.fast = fast_ok;  // the whole tile lies in one page
    t.base1 = t.base0 + 16 * pitch_g;
    if constexpr (C::TT == 32) {
      const int j1 = j0 + 16;
      if (!t.fast && j1 < ls.t_hi && page_of(p, j1) != pg0) {
        const int pg1 = page_of(p, j1);
        const int blk1 = block_of(pg1);
        t.base1 = kvbase + (int64_t)blk1 * p.kv_s0 * C::GES + (int64_t)(j1 - pg1 * p.page) * pitch_g;
      }
    }
    return t;
  };
  // global->LDS reads n of this wave's share (n * 3 / LPW == stage) of tile t
  auto issue_part = [&](const NextTile& t, int stage) {
    if (!t.live || !loader) return;
    MLA_LDS char* dst = ring + t.slot * C::TILE_BYTES;
    if (t.query) {
      // query row i of the unit at row i of the slot, staged like a key row;
      // reads past QI repeat one (same bytes to the same place), so every
      // loader wave sends LPW reads for every tile
#pragma unroll
      for (int n = 0; n < C::LPW; ++n) {
        if (n * 3 / C::LPW != stage) continue;
        const int qinst = (lwave + n * C::LW) % C::QI;
        const int idx = qinst * 64 + lane;
        const int i = idx / C::CH, cpos = idx % C::CH;
        int r = t.qrow0 + i;
        r = r < rows_seq ? r : rows_seq - 1;  // rows past the end are zeroed by the compute waves
        const int qi = p.q_len == 1 ? 0 : fdiv(r, p.div_nh), qh = r - qi * p.n_heads;
        const char* src = (const char*)p.q +
                          ((int64_t)t.qb * p.q_s0 + (int64_t)qi * p.q_s1 + (int64_t)qh * p.q_s2) * C::ES +
                          ((cpos ^ lds_swz(i & 15)) << 4);
        load_lds_16(src, dst + qinst * 1024);
      }
    } else if (t.fast && t.nvalid == C::TT) {
      // a full tile inside one page: page base + per-lane offsets
      const uint64_t sb = uniform_ptr(t.base0);
#pragma unroll
      for (int n = 0; n < C::LPW; ++n) {
        if (n * 3 / C::LPW != stage) continue;
        load_lds_16_sbase<C::STREAM>(sb, loff[n], dst + (lwave + n * C::LW) * 1024);
      }
    } else if (t.fast) {
      // a partial tile inside one page: rows past its end repeat its last valid row
      const uint64_t sb = uniform_ptr(t.base0);
      const int last = t.nvalid - 1;
#pragma unroll
      for (int n = 0; n < C::LPW; ++n) {
        if (n * 3 / C::LPW != stage) continue;
        const int over = lrow[n] > last ? lrow[n] - last : 0;
        const uint32_t off = loff[n] - (uint32_t)(over * pitch_g);
        load_lds_16_sbase<C::STREAM>(sb, off, dst + (lwave + n * C::LW) * 1024);
      }
    } else {
#pragma unroll
      for (int n = 0; n < C::LPW; ++n) {
        if (n * 3 / C::LPW != stage) continue;
        // this lane's 16-byte slot of the tile: row r, stored chunk position cpos
        const int inst = lwave + n * C::LW;
        const int idx = inst * 64 + lane;
        const int r = idx / C::CH, cpos = idx % C::CH;
        const int chunk16 = cpos ^ lds_swz(r & 15);
        const int rr = r < t.nvalid ? r : t.nvalid - 1;  // rows past the end repeat the last valid row
        const char* src =
            (C::TT == 32 && rr >= 16) ? t.base1 + (rr - 16) * pitch_g : t.base0 + rr * pitch_g;
        load_lds_16<C::STREAM>(src + chunk16 * 16, dst + inst * 1024);
      }
    }
  };
  // ---- fp8 cache (KV8): stream item k is read into staging slot k % NS8 at
  // step k - NS8 and landed in ring slot k % NSLOT at step k, by the lanes that
  // read it (so each wave's own vmcnt wait covers the bytes it lands).
  MLA_LDS char* stage = ring + C::RING_BYTES + C::XCHG_BYTES;
  auto kv8_issue = [&](const NextTile& t, int k) {
    MLA_LDS char* stg = stage + (k % C::NS8) * C::STAGE_SLOT;
    if (t.query) {
      // query rows in the bf16 query-tile layout (as issue_part); reads past
      // QI repeat one, so every loader wave sends L8 reads per item
#pragma unroll
      for (int n = 0; n < C::L8; ++n) {
        const int qinst = (lwave + n * C::LW) % C::QI;
        const int idx = qinst * 64 + lane;
        const int i = idx / C::CH, cpos = idx % C::CH;
        int r = t.qrow0 + i;
        r = r < rows_seq ? r : rows_seq - 1;  // rows past the end are zeroed by the compute waves
        const int qi = p.q_len == 1 ? 0 : fdiv(r, p.div_nh), qh = r - qi * p.n_heads;
        const char* src = (const char*)p.q +
                          ((int64_t)t.qb * p.q_s0 + (int64_t)qi * p.q_s1 + (int64_t)qh * p.q_s2) * C::ES +
                          ((cpos ^ lds_swz(i & 15)) << 4);
        load_lds_16(src, stg + qinst * 1024);
      }
      return;
    }
    // key tile as e4m3 bytes: 16-byte piece c of tile row r at r * E + 16 c;
    // rows past the tile's end repeat its last valid row
    constexpr int PR = C::E / 16;
#pragma unroll
    for (int n = 0; n < C::L8; ++n) {
      const int d = (lwave + n * C::LW) % (C::P8 > 0 ? C::P8 : 1);
      const int idx = d * 64 + lane;
      const int r = idx / PR, c = idx % PR;
      const int rr = r < t.nvalid ? r : t.nvalid - 1;
      const char* src =
          (C::TT == 32 && rr >= 16) ? t.base1 + (rr - 16) * pitch_g : t.base0 + rr * pitch_g;
      load_lds_16<C::STREAM>(src + c * 16, stg + d * 1024);
    }
  };
  auto kv8_land = [&](int k, bool query) {
    const MLA_LDS char* stg = stage + (k % C::NS8) * C::STAGE_SLOT + lane * 16;
    MLA_LDS char* dst = ring + (k % C::NSLOT) * C::TILE_BYTES;
    if (query) {
#pragma unroll
      for (int n = 0; n < C::L8; ++n) {
        const int qinst = (lwave + n * C::LW) % C::QI;
        *(MLA_LDS u32x4_t*)(dst + qinst * 1024 + lane * 16) =
            *(const MLA_LDS u32x4_t*)(stg + qinst * 1024);
      }
      return;
    }
    // The staged bytes are the tile's e4m3 rows back to back. Each 1 KB read
    // (all 64 lanes of one instruction of this wave) lands as two halves:
    // lane j widens bytes 8j .. 8j + 7 of a half into one 16-byte bf16 chunk,
    // so the 64 lanes of a ring write cover consecutive chunks (no bank
    // conflicts). All of the lane's staged bytes are read before any ring write.
    constexpr int CR = C::E / 8;  // bf16 chunks of a row
    u32x2_t v8[C::L8 > 0 ? C::L8 : 1][2];
    const MLA_LDS char* stg0 = stage + (k % C::NS8) * C::STAGE_SLOT;
#pragma unroll
    for (int n = 0; n < C::L8; ++n) {
      const int d = (lwave + n * C::LW) % (C::P8 > 0 ? C::P8 : 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        v8[n][h] = *(const MLA_LDS u32x2_t*)(stg0 + d * 1024 + h * 512 + lane * 8);
    }
#pragma unroll
    for (int n = 0; n < C::L8; ++n) {
      const int d = (lwave + n * C::LW) % (C::P8 > 0 ? C::P8 : 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ci = d * 128 + h * 64 + lane;  // chunk of the tile
        const int r = ci / CR, c = ci % CR;
        *(MLA_LDS u32x4_t*)(dst + r * C::PITCH + ((c ^ lds_swz(r & 15)) << 4)) =
            fp8x8_to_bf16x8(v8[n][h]);
      }
    }
  };
  auto kv8_loader = [&]() {
    uint32_t qmask = 0;  // bit k % NS8: staging slot k % NS8 holds query rows
    auto issue = [&](int k) {
      const NextTile t = prep_next(k);
      kv8_issue(t, k);
      const uint32_t bit = 1u << (k % C::NS8);
      qmask = t.query ? (qmask | bit) : (qmask & ~bit);
    };
    for (int k = 0; k < C::NS8 && k < nsteps; ++k) issue(k);
    for (int k = 0; k < nsteps; ++k) {
      // item k's reads are older than those of the (at most NS8 - 1) items after it
      wait_vmcnt_n<C::NS8 - 1, C::L8>(nsteps - 1 - k);
      static_assert(C::NS8 * C::L8 < 64, "vmcnt range");
      kv8_land(k, (qmask >> (k % C::NS8)) & 1u);
      __syncthreads();
      if (k + C::NS8 < nsteps) issue(k + C::NS8);
    }
  };

  // wait until this loader wave's reads of tile k have landed
  auto wait_tile = [&](int k) { wait_vmcnt_n<C::NSLOT - 2, C::LPW>(nsteps - 1 - k); };

  // ---- compute walker state
  // fp8: the scores take q * descale_q and keys * descale_k, the values * descale_k
  float scale_log2 = p.scale_log2, vscale = 1.f;
  if constexpr (C::KV8) {
    scale_log2 = p.scale_log2 * (*p.descale_q * *p.descale_k);
    vscale = *p.descale_k;
  }
  int xs_bad = 0;  // set if a rendezvous wait gave up: the outputs written after it are NaN
  // the rendezvous counter; the word after it is the workgroup's give-up flag
  MLA_LDS uint32_t* xs_ctr = (MLA_LDS uint32_t*)const_cast<uint32_t*>(&tab->xs_ctr);
  using QV = typename std::conditional<C::F32, f32x4_t, i16x8_t>::type;
  // this wave's k-steps of the query rows: kg = wc + WC*kk (all of them when WC == 1)
  QV qreg[C::RT][C::KW];
  bool qvalid[C::RT];
  WaveState<C> st;
  Seg cs = seg0;
  int ck = 0;
  // state of a new segment: this lane's row limits, empty softmax state
  auto begin_state = [&]() {
    const int unit_row0 = (cs.u - cs.b * p.row_tiles) * p.rows_per_unit;
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      const int r = unit_row0 + wrow0 + 16 * rt + li;
      qvalid[rt] = r < rows_seq;
      const int lim = qvalid[rt] ? row_limit(p, cs.s, fdiv(r, p.div_nh)) : 0;
      st.lim[rt] = lim < cs.t_hi ? lim : cs.t_hi;
      st.m[rt] = kNegInf;
      st.l[rt] = 0.f;
#pragma unroll
      for (int d = 0; d < C::DW; ++d) st.o[rt][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  // folded query rows of the segment's unit -> registers (B operand layout),
  // loaded from global memory ahead of the tile reads (no query tiles); rows
  // past the end load row 0 and are zeroed by settle_q
  auto load_q = [&]() {
    const int unit_row0 = (cs.u - cs.b * p.row_tiles) * p.rows_per_unit;
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      const int r = unit_row0 + wrow0 + 16 * rt + li;
      const int qi = qvalid[rt] ? fdiv(r, p.div_nh) : 0, qh = qvalid[rt] ? r - qi * p.n_heads : 0;
      const int64_t qoff = (int64_t)cs.b * p.q_s0 + (int64_t)qi * p.q_s1 + (int64_t)qh * p.q_s2;
      const char* qp = (const char*)p.q + qoff * C::ES + 16 * g;
#pragma unroll
      for (int kk = 0; kk < C::KW; ++kk) {
        // with a split contraction a k-step past the row end (uneven split)
        // reloads the wave's first one, never used
        const int kg = !C::XS ? kk : (wc + C::WC * kk < C::KSTEPS ? wc + C::WC * kk : wc);
        load_16(qreg[rt][kk], qp + 64 * kg);
      }
    }
  };
  // the same from a query tile in the ring (staged like key rows)
  auto read_q_tile = [&](const MLA_LDS char* slot) {
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      const int row = wrow0 + 16 * rt + li;
      const MLA_LDS char* rb = slot + row * C::PITCH;
      const int sw = lds_swz(row & 15);
#pragma unroll
      for (int kk = 0; kk < C::KW; ++kk) {
        // with a split contraction the wave holds k-steps wc, wc + WC, ... (a
        // step past the row end, never used, rereads the first)
        const int kg = !C::XS ? kk : (wc + C::WC * kk < C::KSTEPS ? wc + C::WC * kk : wc);
        const int c = 4 * kg + g;  // 16-byte chunk of k-step kg
        const MLA_LDS QV* qp = (const MLA_LDS QV*)(rb + (((c & ~7) | ((c & 7) ^ sw)) << 4));
        qreg[rt][kk] = qvalid[rt] ? *qp : QV{};
      }
    }
  };
  auto settle_q = [&]() {
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
      for (int kk = 0; kk < C::KW; ++kk)
        if (!qvalid[rt]) qreg[rt][kk] = QV{};
  };
  auto end_seg = [&]() {
    const int unit_row0 = (cs.u - cs.b * p.row_tiles) * p.rows_per_unit;
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      const float lt = wave_sum16(st.l[rt]);
      if (C::XS && C::NP > 0 &&
          __hip_atomic_load(xs_ctr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))
        xs_bad = 1;
      const float nan = __builtin_nanf("");
      const float inv = xs_bad ? nan : (lt > 0.f ? vscale / lt : 0.f);
      const float lse2 = xs_bad ? nan : (lt > 0.f ? st.m[rt] + fast_log2(lt) : kNegInf);
      store_row<C>(p, cs.b, unit_row0, wrow0 + 16 * rt + li, cs.slot, st.o[rt], inv, lse2, dc0,
                   wc == 0);
    }
  };

  // The first segment's query rows. Where every wave computes and the unit's
  // rows fit in a tile (QD), the loader waves read them like a query tile into
  // ring slot NSLOT - 1, which the first tile reads leave free, so the wait
  // for them retires nothing younger; otherwise they are read into registers
  // ahead of the first tiles.
  constexpr bool QD = C::NP == 0 && C::RTILE <= C::TT && !C::KV8;
  if (compute) begin_state();
  if constexpr (QD) {
    NextTile qt;
    qt.live = true;
    qt.query = true;
    qt.slot = C::NSLOT - 1;
    qt.qb = cs.b;
    qt.qrow0 = (cs.u - cs.b * p.row_tiles) * p.rows_per_unit;
#pragma unroll
    for (int st3 = 0; st3 < 3; ++st3) issue_part(qt, st3);
  } else if (compute) {
    load_q();
  }
  // prologue: the first NSLOT - 1 tiles
  if (loader && !C::KV8) {
#pragma unroll
    for (int k = 0; k < C::NSLOT - 1; ++k)
      if (k < nsteps) {
        const NextTile t = prep_next(k);
#pragma unroll
        for (int st3 = 0; st3 < 3; ++st3) issue_part(t, st3);
      }
  }
  if constexpr (QD) {
    // the query reads are older than the prologue's tile reads
    const int pro = nsteps < C::NSLOT - 1 ? nsteps : C::NSLOT - 1;
    if (loader) wait_vmcnt_n<C::NSLOT - 1, C::LPW>(pro);
    __syncthreads();
    read_q_tile(ring + (C::NSLOT - 1) * C::TILE_BYTES);
  } else if (compute) {
    // the compiler's wait for the query loads also retires the tile reads
    wait_vmcnt<0>();
    settle_q();
  }
  int xs_seq = 0;  // tile_compute calls so far (the split-contraction rendezvous count)
  if constexpr (C::NP > 0) {
    // ---- separate roles: each runs its own loop (one barrier per stream item)
    if (loader && C::KV8) {
      kv8_loader();
    } else if (loader) {
      for (int k = 0; k < nsteps; ++k) {
        wait_tile(k);
        __syncthreads();
        if (k + C::NSLOT - 1 < nsteps) {
          const NextTile nt = prep_next(k + C::NSLOT - 1);
#pragma unroll
          for (int st3 = 0; st3 < 3; ++st3) issue_part(nt, st3);
        }
      }
    } else {
    bool q_tile = false;  // the next stream item is a segment's query tile
    for (int k = 0; k < nsteps; ++k) {
      __syncthreads();
      const MLA_LDS char* slot = ring + (k % C::NSLOT) * C::TILE_BYTES;
      if (q_tile) {
        read_q_tile(slot);
        q_tile = false;
        continue;
      }
      tile_compute<C>(slot, xchg, cs.t_lo + ck * C::TT, qreg, st, scale_log2, wr, wc, dc0,
                      [](int) {}, []() {}, xs_ctr, xs_seq, xs_bad, p.rendezvous_polls);
      if (++ck == cs.ntiles && k + 1 < nsteps) {
        end_seg();
        cs = seg_of<C>(p, tab, h, next_live(p, tab, cs.u));
        ck = 0;
        begin_state();
        q_tile = true;
      }
    }
    end_seg();
    }
  } else {
    // ---- every wave loads and computes. One workgroup barrier per tile, at the
    // score exchange of tile k: it publishes the partial scores (stored in the
    // copy k % 2 of the exchange), makes tile k + 1 visible (each loader wave
    // first waits for its reads of it, the only ones in flight) and frees the
    // slot of tile k - 1, into which tile k + NSLOT - 1 is then read. Tile 0 is
    // waited for before the loop.
    static_assert(C::XS, "the barrier sits at the score exchange");
    bool q_pending = false;
    if (nsteps > 0) {
      wait_tile(0);
      __syncthreads();
    }
    for (int k = 0; k < nsteps; ++k) {
      if (q_pending) {
        // a new segment's query rows: read and waited for here, on this path
        // only, so no other path has query loads in flight (the wait also
        // retires the tile reads)
        load_q();
        wait_vmcnt<0>();
        settle_q();
        q_pending = false;
      }
      const NextTile nt =
          loader && k + C::NSLOT - 1 < nsteps ? prep_next(k + C::NSLOT - 1) : NextTile{};
      tile_compute<C>(ring + (k % C::NSLOT) * C::TILE_BYTES, xchg + (k & 1) * C::XCHG_HALF,
                      cs.t_lo + ck * C::TT, qreg, st, scale_log2, wr, wc, dc0,
                      [&](int stage) {
                        if (stage > 0) issue_part(nt, stage);
                      },
                      [&]() {
                        wait_vmcnt<0>();
                        __syncthreads();
                        issue_part(nt, 0);
                      },
                      xs_ctr, xs_seq, xs_bad, p.rendezvous_polls);
      if (++ck == cs.ntiles && k + 1 < nsteps) {
        end_seg();
        cs = seg_of<C>(p, tab, h, next_live(p, tab, cs.u));
        ck = 0;
        begin_state();
        q_pending = true;
      }
    }
    end_seg();
  }
}

template <class C>
__global__ void __attribute__((amdgpu_flat_work_group_size(C::NT, C::NT),
                               amdgpu_waves_per_eu(C::NT / 256, C::NT / 256)))
decode_partial(DecodeParams p) {
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  __shared__ SegLds tab;
  __shared__ int sh_blk[kBlkCache];
  MLA_LDS char* ring = (MLA_LDS char*)smem_raw;
  MLA_LDS f32x4_t* xchg = (MLA_LDS f32x4_t*)(smem_raw + C::RING_BYTES);
  if (threadIdx.x == 0) {  // rendezvous counter and give-up flag; the plan's barrier publishes them
    tab.xs_ctr = 0u;
    tab.xs_gaveup = 0u;
  }
  if (!(p.plan && p.split && load_plan<C>(p, &tab, sh_blk, (MLA_LDS int*)ring)))
    plan_workgroup<C>(p, &tab, sh_blk, (MLA_LDS int*)ring);
  // a workgroup whose chunk holds no keys (split mode) has nothing to write;
  // without split an empty unit still writes its zero rows
  if (p.split && tab.hdr.u0 > tab.hdr.u1) return;
  process_range<C>(p, &tab, sh_blk, ring, xchg);
}

// The split plan of a call, computed once into p.plan for the calls that
// share its sequence lengths, block table and sizes (one layer's attention
// after another): one 64-thread workgroup per attention workgroup runs that
// workgroup's plan pass and writes its descriptor; workgroup 0 also writes the
// merge's cost scan and the header, last.
template <class C>
__global__ void __launch_bounds__(64) decode_plan(DecodeParams p) {
  __shared__ SegLds tab;
  __shared__ int sh_blk[kBlkCache];
  __shared__ int scratch[5 * kSplitUnits];
  plan_workgroup<C>(p, &tab, sh_blk, (MLA_LDS int*)scratch);
  const int lane = threadIdx.x;
  int* d = p.plan + kPlanHdrInts + kSplitUnits + (int64_t)blockIdx.x * kDescInts;
  const int u0 = tab.hdr.u0, u1 = tab.hdr.u1;
  const int n = u1 >= u0 ? u1 - u0 + 1 : 0;
  const int npg = tab.nstaged < kDescPages ? tab.nstaged : kDescPages;
  const bool fits = n <= kDescUnits;
  if (lane == 0) {
    d[0] = u0;
    d[1] = u1;
    d[2] = tab.hdr.tlo0;
    d[3] = tab.hdr.thi1;
    d[4] = tab.hdr.nsteps;
    d[5] = fits ? n : -1;
    d[6] = npg;
    d[7] = 0;
  }
  if (fits) {
    for (int i = lane; i < n; i += 64) {
      const int u = u0 + i;  // tables indexed by unit (ubase 0)
      d[8 + 4 * i] = tab.kv[u];
      d[8 + 4 * i + 1] = tab.sl[u];
      d[8 + 4 * i + 2] = tab.poff[u];
      d[8 + 4 * i + 3] = (int)((tab.live[u >> 6] >> (u & 63)) & 1u) |
                         ((int)((tab.part[u >> 6] >> (u & 63)) & 1u) << 1);
    }
  }
  for (int i = lane; i < npg; i += 64) d[kDescPageOff + i] = sh_blk[i];
  if (blockIdx.x == 0) {
    plan_units(p, scratch);
    for (int u = lane; u < p.num_units; u += 64) p.plan[kPlanHdrInts + u] = scratch[u];
    if (lane < 16) p.plan[lane] = plan_field(p, lane);
  }
}

// ------------------------------------------------------------------- merge
// Merge of the split partials. One workgroup per (unit, 4 rows), one wave
// per row, 8 columns per lane. A row's split lse values (one split per lane)
// and its first 8 partial rows are read together, so the merge costs one
// memory round trip after the plan; the weights reach every lane by shuffle.
// Splits are combined in split order (deterministic).
// One row of the merge: row `row` (0 .. rows_per_unit) of unit u, this lane's
// 8 columns c0 .. c0 + 7. Returns false when the unit was not split (its only
// workgroup wrote the row itself); else the merged row (acc0, acc1) and its
// log2-domain lse (-inf for a unit with no keys, whose row is zero).
// PART_F32: the split partials are f32 rows (f32 inputs), else bf16 rows.
// BATCH: partial rows read per round trip.
template <bool PART_F32, int BATCH = 8>
__device__ __forceinline__ bool merge_row(const DecodeParams& p, const int* sh_scan, int u, int row,
                                          f32x4_t& acc0, f32x4_t& acc1, float& lse2) {
  const int lane = threadIdx.x & 63, c0 = lane * 8;
  const int total = sh_scan[p.num_units - 1];
  const int chunk = total > 0 ? ceil_div(total, p.grid) : 1;
  const int end = sh_scan[u], start = u > 0 ? sh_scan[u - 1] : 0;
  acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
  acc1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
  lse2 = kNegInf;
  if (end > start) {
    const int first = (start + p.alpha) / chunk, last = (end - 1) / chunk;
    if (first == last) return false;  // written directly by its only workgroup
    const int n = last - first + 1;
    const int64_t srow = p.rows_per_unit;
    const float* lp = p.part_lse + (int64_t)(first + u) * srow + row;
    const int64_t obase = ((int64_t)(first + u) * srow + row) * kKvRank + c0;
    const int64_t ostride = srow * kKvRank;
    // split row k's columns c0 .. c0 + 7, as loaded: two f32x4 for f32
    // partials, one u32x4 of bf16 pairs otherwise (widened when summed)
    using Raw = std::conditional_t<PART_F32, f32x4_t[2], u32x4_t>;
    auto load_part = [&](int64_t k, Raw& x) {
      if constexpr (PART_F32) {
        const float* src = p.part_o + obase + k * ostride;
        x[0] = *(const f32x4_t*)src;
        x[1] = *(const f32x4_t*)(src + 4);
      } else {
        x = *(const u32x4_t*)((const uint16_t*)p.part_o + obase + k * ostride);
      }
    };
    auto add_part = [&](float wk, const Raw& x) {
      if constexpr (PART_F32) {
        acc0 += wk * x[0];
        acc1 += wk * x[1];
      } else {
        const f32x4_t lo{__builtin_bit_cast(float, x[0] << 16), __builtin_bit_cast(float, x[0] & 0xffff0000u),
                         __builtin_bit_cast(float, x[1] << 16), __builtin_bit_cast(float, x[1] & 0xffff0000u)};
        const f32x4_t hi{__builtin_bit_cast(float, x[2] << 16), __builtin_bit_cast(float, x[2] & 0xffff0000u),
                         __builtin_bit_cast(float, x[3] << 16), __builtin_bit_cast(float, x[3] & 0xffff0000u)};
        acc0 += wk * lo;
        acc1 += wk * hi;
      }
    };
    static_assert(BATCH == 8, "8 partial rows per round trip");
    float M = kNegInf, Lt = 0.f;
    for (int w0 = 0; w0 < n; w0 += 64) {
      // this lane's split lse, and the first BATCH partial rows, in one round trip
      const int cnt = n - w0 < 64 ? n - w0 : 64;
      const float ls = lane < cnt ? lp[(int64_t)(w0 + lane) * srow] : kNegInf;
      Raw x[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const bool in = k < cnt;
        load_part(w0 + (in ? k : 0), x[k]);
      }
      if (w0 == 0) {
        M = ls;
        for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        // splits past the first 64 cannot raise M above what the first pass saw
        // unless n > 64; then M is refined below before any weight is applied
        if (n > 64) {
          for (int w1 = 64; w1 < n; w1 += 64) {
            const float l2 = w1 + lane < n ? lp[(int64_t)(w1 + lane) * srow] : kNegInf;
            float m2 = l2;
            for (int off = 32; off >= 1; off >>= 1) m2 = fmaxf(m2, __shfl_xor(m2, off));
            M = fmaxf(M, m2);
          }
        }
      }
      const float a = ls == kNegInf ? 0.f : fast_exp2(ls - M);  // this lane's split weight
      float lsum = a;
      for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
      Lt += lsum;
      for (int k0 = 0; k0 < cnt; k0 += BATCH) {
        if (k0 > 0) {
#pragma unroll
          for (int k = 0; k < BATCH; ++k) {
            const bool in = k0 + k < cnt;
            load_part(w0 + (in ? k0 + k : 0), x[k]);
          }
        }
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const float wk = lane_weight(a, k0 + k);  // weight of split w0 + k0 + k
          if (k0 + k < cnt) add_part(wk, x[k]);
        }
      }
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    acc0 *= inv;
    acc1 *= inv;
    // no key: lse -inf; a NaN split (a wave that gave up) makes the row and its lse NaN
    lse2 = Lt > 0.f ? M + fast_log2(Lt) : (Lt == 0.f ? kNegInf : Lt);
  }
  return true;
}

// Merge of bf16 partials for plans that split units many ways (the 128-head
// decode of 4 sequences: 16 splits per unit). One wave per (unit, row, half of
// the 512 columns), 4 columns per lane, so the rows of a call spread over
// twice the waves of decode_merge; every split's lse and the first BATCH
// partial row pieces are requested in one round trip after the plan (BATCH
// near the split count: a batch past it re-reads the first split, which
// measured 1.6 us slower at 16 splits with 32). Splits are summed in split
// order with decode_merge's weights and reductions, so the result is the same
// bit for bit.
template <int kWideBatch>
__global__ void __launch_bounds__(256) decode_merge_wide(DecodeParams p) {
  __shared__ int sh_scan[kSplitUnits];
  if (!(p.plan && load_scan(p, sh_scan))) plan_units(p, sh_scan);
  const int lane = threadIdx.x & 63;
  const int item = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int half = item & 1, ur = item >> 1;
  const int u = ur / p.rows_per_unit, row = ur - u * p.rows_per_unit;
  if (u >= p.num_units) return;
  const int b = fdiv(u, p.div_rt);
  const int r = (u - b * p.row_tiles) * p.rows_per_unit + row;
  if (r >= p.q_len * p.n_heads) return;
  const int total = sh_scan[p.num_units - 1];
  const int chunk = total > 0 ? ceil_div(total, p.grid) : 1;
  const int end = sh_scan[u], start = u > 0 ? sh_scan[u - 1] : 0;
  const int qi = fdiv(r, p.div_nh), qh = r - qi * p.n_heads;
  const int c0 = half * (kKvRank / 2) + lane * 4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float lse2 = kNegInf;
  if (end > start) {
    const int first = (start + p.alpha) / chunk, last = (end - 1) / chunk;
    if (first == last) return;  // written directly by its only workgroup
    const int n = last - first + 1;
    const int64_t srow = p.rows_per_unit;
    const float* lp = p.part_lse + (int64_t)(first + u) * srow + row;
    const uint16_t* ob = (const uint16_t*)p.part_o + ((int64_t)(first + u) * srow + row) * kKvRank + c0;
    const int64_t ostride = srow * kKvRank;
    auto add_part = [&](float wk, u32x2_t x) {
      const f32x4_t v{__builtin_bit_cast(float, x[0] << 16), __builtin_bit_cast(float, x[0] & 0xffff0000u),
                      __builtin_bit_cast(float, x[1] << 16), __builtin_bit_cast(float, x[1] & 0xffff0000u)};
      acc += wk * v;
    };
    float M = kNegInf, Lt = 0.f;
    u32x2_t x[kWideBatch];
    for (int w0 = 0; w0 < n; w0 += 64) {
      const int cnt = n - w0 < 64 ? n - w0 : 64;
      // this lane's split lse and the first kWideBatch partial pieces, one round trip
      const float ls = lane < cnt ? lp[(int64_t)(w0 + lane) * srow] : kNegInf;
#pragma unroll
      for (int k = 0; k < kWideBatch; ++k)
        x[k] = *(const u32x2_t*)(ob + (int64_t)(w0 + (k < cnt ? k : 0)) * ostride);
      if (w0 == 0) {
        M = ls;
        for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        for (int w1 = 64; w1 < n; w1 += 64) {
          const float l2 = w1 + lane < n ? lp[(int64_t)(w1 + lane) * srow] : kNegInf;
          float m2 = l2;
          for (int off = 32; off >= 1; off >>= 1) m2 = fmaxf(m2, __shfl_xor(m2, off));
          M = fmaxf(M, m2);
        }
      }
      const float a = ls == kNegInf ? 0.f : fast_exp2(ls - M);  // this lane's split weight
      float lsum = a;
      for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
      Lt += lsum;
      for (int k0 = 0; k0 < cnt; k0 += kWideBatch) {
        if (k0 > 0) {
#pragma unroll
          for (int k = 0; k < kWideBatch; ++k)
            x[k] = *(const u32x2_t*)(ob + (int64_t)(w0 + (k0 + k < cnt ? k0 + k : 0)) * ostride);
        }
#pragma unroll
        for (int k = 0; k < kWideBatch; ++k) {
          const float wk = lane_weight(a, k0 + k);  // weight of split w0 + k0 + k
          if (k0 + k < cnt) add_part(wk, x[k]);
        }
      }
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    acc *= inv;
    // no key: lse -inf; a NaN split (a wave that gave up) makes the row and its lse NaN
    lse2 = Lt > 0.f ? M + fast_log2(Lt) : (Lt == 0.f ? kNegInf : Lt);
  }
  const int64_t ooff = (int64_t)b * p.o_s0 + (int64_t)qi * p.o_s1 + (int64_t)qh * p.o_s2 + c0;
  *(u32x2_t*)((uint16_t*)p.out + ooff) = u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  if (half == 0 && lane == 0 && p.lse)
    p.lse[(int64_t)b * p.l_s0 + (int64_t)qi * p.l_s1 + (int64_t)qh * p.l_s2] =
        lse2 == kNegInf ? kNegInf : lse2 * kLn2;
}

// Plans with few splits per unit (units split many ways take decode_merge_wide).
template <bool F32, int BATCH>
__global__ void __launch_bounds__(256) decode_merge(DecodeParams p) {
  __shared__ int sh_scan[kSplitUnits];
  if (!(p.plan && load_scan(p, sh_scan))) plan_units(p, sh_scan);
  const int groups = (p.rows_per_unit + 3) / 4;
  const int u = blockIdx.x / groups;
  const int lane = threadIdx.x & 63;
  const int row = (blockIdx.x % groups) * 4 + (threadIdx.x >> 6);
  const int c0 = lane * 8;
  if (u >= p.num_units || row >= p.rows_per_unit) return;
  const int b = fdiv(u, p.div_rt);
  const int r = (u - b * p.row_tiles) * p.rows_per_unit + row;
  if (r >= p.q_len * p.n_heads) return;
  f32x4_t acc0, acc1;
  float lse2;
  if (!merge_row<F32, BATCH>(p, sh_scan, u, row, acc0, acc1, lse2)) return;
  const int qi = fdiv(r, p.div_nh), qh = r - qi * p.n_heads;
  const int64_t ooff = (int64_t)b * p.o_s0 + (int64_t)qi * p.o_s1 + (int64_t)qh * p.o_s2 + c0;
  if constexpr (F32) {
    float* dst = (float*)p.out + ooff;
    *(f32x4_t*)dst = acc0;
    *(f32x4_t*)(dst + 4) = acc1;
  } else {
    uint16_t* dst = (uint16_t*)p.out + ooff;
    *(u32x4_t*)dst = u32x4_t{pack_bf16x2(acc0[0], acc0[1]), pack_bf16x2(acc0[2], acc0[3]),
                             pack_bf16x2(acc1[0], acc1[1]), pack_bf16x2(acc1[2], acc1[3])};
  }
  if (c0 == 0 && p.lse)
    p.lse[(int64_t)b * p.l_s0 + (int64_t)qi * p.l_s1 + (int64_t)qh * p.l_s2] =
        lse2 == kNegInf ? kNegInf : lse2 * kLn2;
}

// ------------------------------------------ merge + W_UV un-projection, fused
// For one head h, 16 query tokens and a group of 32 W_UV columns (the column
// groups of a head spread the call over 4x the workgroups; each group merges
// the same rows, the first writes o_lat and lse): merge each token's row of head h from
// its split partials (one wave per token; unsplit rows are read back from
// o_lat), keep the 16 merged rows in LDS as bf16 (the values written to
// o_lat), then out[token, h, :] = o_lat row . W_UV[h] with 16x16x32 MFMAs,
// W_UV[h] staged in LDS by one burst of global->LDS loads issued before the
// merge. The products run in the same k order as mla_v_up's kernel, so out
// is bit-identical to the two calls made one after the other.
constexpr int kVupTok = 16;                       // query tokens per workgroup
constexpr int kVupMaxV = 128;                     // W_UV columns one workgroup stages
constexpr int kVupAPitch = kKvRank * 2 + 32;      // bf16 o_lat row in LDS (padded: the 16
                                                  // rows of an A read fall in distinct banks)
// W_UV slab in LDS: 16-byte chunk c of row r at chunk position c ^ vswz(r), so
// the 16 rows one transposed B read touches (4 per lane group, 8 apart between
// groups) fall in distinct 32-byte bank segments.
__device__ __forceinline__ int vswz(int r) { return 2 * (((r >> 1) & 1) | (((r >> 3) & 3) << 1)); }

__global__ void __launch_bounds__(1024) decode_merge_vup(DecodeParams p, VupParams v) {
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  __shared__ int sh_scan[kSplitUnits];
  MLA_LDS char* wslab = (MLA_LDS char*)smem_raw;           // [kKvRank][V] bf16, dense
  MLA_LDS char* atile = wslab + kKvRank * (v.V / (int)gridDim.z) * 2;  // [16][kVupAPitch]
  // (token group, head, column group) of this workgroup. Workgroup i runs on
  // XCD i % 8: when the (head, column group) slabs divide evenly over the 8
  // XCDs, all token groups of one slab go to one XCD, so its W_UV columns are
  // read from HBM once and then found in that XCD's L2.
  const int ntg = (int)gridDim.x, nslab = (int)(gridDim.y * gridDim.z);
  int tg = (int)blockIdx.x, slab = (int)(blockIdx.y + gridDim.y * blockIdx.z);
  if (nslab % 8 == 0) {
    const int lin = (int)blockIdx.x + ntg * slab, k = lin / 8;
    slab = lin % 8 + 8 * (k / ntg);
    tg = k % ntg;
  }
  const int h = slab % (int)gridDim.y, cg = slab / (int)gridDim.y;
  const int tok0 = tg * kVupTok;
  // columns [col0, col0 + VW) of W_UV[h]: the workgroups of a (token group,
  // head) split the un-projection's columns and each merges the same rows
  const int VW = v.V / (int)gridDim.z, col0 = cg * VW;
  const bool first = cg == 0;  // writes o_lat and lse
  const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = p.batch * p.q_len;
  // W_UV[h][:, col0 : col0 + VW] -> LDS: chunk q (16 bytes) of the dense [L][VW] slab, 64 per load
  {
    const char* W = (const char*)v.w + (int64_t)h * v.w_sh * 2 + (int64_t)col0 * 2;
    const int cpr = VW / 8;  // 16-byte chunks per row
    const int ninst = kKvRank * cpr / 64;
    for (int inst = wave; inst < ninst; inst += 16) {
      const int q = inst * 64 + lane, r = q / cpr, cp = q % cpr;
      const int c = cp ^ (vswz(r) & (cpr - 1));  // the source chunk stored at position cp
      load_lds_16(W + (int64_t)r * v.w_sk * 2 + c * 16, wslab + inst * 1024);
    }
  }
  if (!(p.plan && load_scan(p, sh_scan))) plan_units(p, sh_scan);
  // merge: wave w takes token tok0 + w
  const int t = tok0 + wave;
  const int c0 = lane * 8;
  u32x4_t packed = {0u, 0u, 0u, 0u};
  if (t < T) {
    const int b = t / p.q_len, qi = t - b * p.q_len;
    const int r = qi * p.n_heads + h;
    const int rt = r / p.rows_per_unit, row = r - rt * p.rows_per_unit;
    const int u = b * p.row_tiles + rt;
    f32x4_t acc0, acc1;
    float lse2;
    const int64_t ooff = (int64_t)b * p.o_s0 + (int64_t)qi * p.o_s1 + (int64_t)h * p.o_s2 + c0;
    uint16_t* orow = (uint16_t*)p.out + ooff;
    if (merge_row<false>(p, sh_scan, u, row, acc0, acc1, lse2)) {
      packed = u32x4_t{pack_bf16x2(acc0[0], acc0[1]), pack_bf16x2(acc0[2], acc0[3]),
                       pack_bf16x2(acc1[0], acc1[1]), pack_bf16x2(acc1[2], acc1[3])};
      if (first) *(u32x4_t*)orow = packed;
      if (first && c0 == 0 && p.lse)
        p.lse[(int64_t)b * p.l_s0 + (int64_t)qi * p.l_s1 + (int64_t)h * p.l_s2] =
            lse2 == kNegInf ? kNegInf : lse2 * kLn2;
    } else {
      packed = *(const u32x4_t*)orow;  // the unit's only workgroup wrote it
    }
  }
  *(MLA_LDS u32x4_t*)(atile + wave * kVupAPitch + c0 * 2) = packed;
  wait_vmcnt<0>();  // this wave's part of the W_UV slab has landed
  __syncthreads();
  // out tile: waves 0 .. VW/16 - 1 take 16 columns each, all 16 tokens
  if (wave < VW / 16) {
    const int n0 = wave * 16;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int row_bytes = VW * 2, cmask = VW / 8 - 1;
#pragma unroll 4
    for (int ks = 0; ks < kKvRank / 32; ++ks) {
      const i16x8_t av = *(const MLA_LDS i16x8_t*)(atile + li * kVupAPitch + (ks * 32 + 8 * g) * 2);
      // rows k0 .. k0 + 3 and k0 + 4 .. k0 + 7, columns n0 + 4 (li % 4) .. + 3
      const int k0 = ks * 32 + 8 * g + (li >> 2), col = n0 + 4 * (li & 3);
      const int cw = col >> 3, within = (col & 7) * 2;
      const i16x4_t b0 =
          lds_read_tr16(wslab + k0 * row_bytes + ((cw ^ (vswz(k0) & cmask)) << 4) + within);
      const i16x4_t b1 = lds_read_tr16(wslab + (k0 + 4) * row_bytes +
                                       ((cw ^ (vswz(k0 + 4) & cmask)) << 4) + within);
      const i16x8_t bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      acc = mfma_16x16x32(av, bv, acc);
    }
    // lane holds out[token tok0 + 4g + j][column n0 + li]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = tok0 + 4 * g + j;
      if (tt < T) {
        const int b = tt / p.q_len, qi = tt - b * p.q_len;
        ((uint16_t*)v.out)[(int64_t)b * v.o_s0 + (int64_t)qi * v.o_s1 + (int64_t)h * v.o_s2 +
                           col0 + n0 + li] = f32_to_bf16(acc[j]);
      }
    }
  }
}

// ------------------------------------------------------------- variants
//                      R   WR WC RT TT NSLOT F32    XS     NP
// <= 16 rows: columns split over waves. Three ring slots (two tiles in flight
// per CU) stream faster than four here: the V2-Lite attention call measured
// 38.6 us against 39.5 us (and 44.9 us with two slots).
using Cols64  = Cfg<64, 1, 4, 1, 32, 3, false, true,  4>;
using Cols0   = Cfg<0,  1, 4, 1, 32, 3, false, true,  4>;
// 32 rows: eight waves, two 16-row tiles x four 128-column quarters
using Mixed64 = Cfg<64, 2, 4, 1, 32, 3, false, true,  0>;
using Mixed0  = Cfg<0,  2, 4, 1, 32, 3, false, true,  0>;
// 64 rows: eight waves, four 16-row tiles x two 256-column halves
using Rows64  = Cfg<64, 4, 2, 1, 32, 3, false, true,  0>;
using Rows0   = Cfg<0,  4, 2, 1, 32, 3, false, true,  0>;
using ColsF64 = Cfg<64, 1, 4, 1, 16, 3, true,  true,  0>;  // f32
using ColsF0  = Cfg<0,  1, 4, 1, 16, 3, true,  true,  0>;
using Cols64F8 = Cfg<64, 1, 4, 1, 32, 2, false, true,  4, true>;  // fp8 cache, any row count
using Cols0F8  = Cfg<0,  1, 4, 1, 32, 2, false, true,  4, true>;

constexpr int kColsEntryCost = 3;  // work blocks (measured: 3-4 best on V2-Lite)

enum Variant { kCols64 = 0, kCols0, kMixed64, kMixed0, kRows64, kRows0, kColsF64, kColsF0,
               kCols64F8, kCols0F8 };

template <class C>
hipError_t launch_partial(const DecodePlan& plan, const DecodeParams& p, hipStream_t s) {
  // the partial kernel plans in tiles; the merge reads the work block size
  if (plan.wb != C::TT || p.wb != C::TT) return hipErrorInvalidValue;
  const size_t smem = C::SMEM_BYTES;
  static bool attr_set = false;  // the attribute is per function, set once per process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_partial<C>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(decode_partial<C>, dim3(plan.grid), dim3(C::NT), smem, s, p);
  return hipGetLastError();
}

template <class C>
hipError_t launch_variant(const DecodePlan& plan, const DecodeParams& p, hipStream_t s) {
  hipError_t e = launch_partial<C>(plan, p, s);
  if (e != hipSuccess || !plan.split) return e;
  const int groups = (plan.rows_per_unit + 3) / 4;
  // units split about 8 ways or more on average: the 16-row batch
  if (!C::F32 && plan.grid >= 8 * plan.num_units) {
    // many splits per unit: two waves per row, every split in one round trip
    const int64_t waves = (int64_t)plan.num_units * plan.rows_per_unit * 2;
    const dim3 grid((unsigned)((waves + 3) / 4));
    // splits per unit: about grid / units (plus one where a chunk boundary falls inside)
    if (plan.grid <= 16 * plan.num_units)
      hipLaunchKernelGGL(decode_merge_wide<16>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(decode_merge_wide<32>, grid, dim3(256), 0, s, p);
  } else
    hipLaunchKernelGGL((decode_merge<C::F32, 8>), dim3(plan.num_units * groups), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool can_merge_vup(const DecodePlan& plan, int is_f32, const VupParams& v) {
  // V a power of two from 16 to 128: the slab swizzle stays inside a row
  return plan.split && !is_f32 && v.V >= 16 && v.V <= kVupMaxV && (v.V & (v.V - 1)) == 0 &&
         (uintptr_t)v.w % 16 == 0 && (v.w_sh * 2) % 16 == 0 && (v.w_sk * 2) % 16 == 0;
}

hipError_t launch_decode_vup(const DecodePlan& plan, DecodeParams p, const VupParams& v,
                             hipStream_t s) {
  if (!can_merge_vup(plan, 0, v)) return hipErrorInvalidValue;
  // the partial kernel exactly as launch_decode runs it, then the fused merge
  hipError_t e = hipSuccess;
  switch (plan.variant) {
    case kCols64: e = launch_partial<Cols64>(plan, p, s); break;
    case kCols0: e = launch_partial<Cols0>(plan, p, s); break;
    case kMixed64: e = launch_partial<Mixed64>(plan, p, s); break;
    case kMixed0: e = launch_partial<Mixed0>(plan, p, s); break;
    case kRows64: e = launch_partial<Rows64>(plan, p, s); break;
    case kRows0: e = launch_partial<Rows0>(plan, p, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  static bool attr_set = false;
  if (!attr_set) {
    e = hipFuncSetAttribute((const void*)decode_merge_vup,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)((size_t)kKvRank * kVupMaxV * 2 + (size_t)kVupTok * kVupAPitch));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t T = (int64_t)p.batch * p.q_len;
  // split W_UV's columns into groups of 32 (16 for V = 16) over workgroups
  const int csplit = v.V >= 32 ? v.V / 32 : 1;
  const size_t smem_w = (size_t)kKvRank * (v.V / csplit) * 2 + (size_t)kVupTok * kVupAPitch;
  dim3 grid((unsigned)((T + kVupTok - 1) / kVupTok), (unsigned)p.n_heads, (unsigned)csplit);
  hipLaunchKernelGGL(decode_merge_vup, grid, dim3(1024), smem_w, s, p, v);
  return hipGetLastError();
}

int plan_decode(int64_t batch, int64_t q_len, int64_t n_heads, int64_t rope, int64_t max_seqlen,
                int is_f32, DecodePlan* plan, int kv8) {
  const int64_t rows = q_len * n_heads;
  int variant, rtile;
  if (kv8) {
    if (is_f32) return -1;
    variant = rope ? kCols64F8 : kCols0F8;
    rtile = Cols64F8::RTILE;
  } else if (is_f32) {
    variant = rope ? kColsF64 : kColsF0;
    rtile = ColsF64::RTILE;
  } else if (rows <= 16) {
    variant = rope ? kCols64 : kCols0;
    rtile = Cols64::RTILE;
  } else if (rows <= 32 || batch * ((rows + Rows64::RTILE - 1) / Rows64::RTILE) < 64) {
    // 32-row units also where 64-row units would be too few to fill the GPU
    // without splitting each many ways (the 128-head decode of a few
    // sequences): their split partials are half as many bytes per key range
    variant = rope ? kMixed64 : kMixed0;
    rtile = Mixed64::RTILE;
  } else {
    variant = rope ? kRows64 : kRows0;
    rtile = Rows64::RTILE;
  }
  const int64_t row_tiles = (rows + rtile - 1) / rtile;
  const int64_t units = batch * row_tiles;
  if (units > (int64_t)1 << 30) return -1;
  plan->variant = variant;
  plan->rows_per_unit = rtile;
  plan->row_tiles = (int)row_tiles;
  plan->num_units = (int)units;
  // plan granularity: the variant's tile
  plan->wb = is_f32 ? ColsF64::TT : Cols64::TT;
  // entering a unit costs the few-head layout a query tile and a partial tile
  plan->alpha = (variant == kCols64 || variant == kCols0 || variant == kCols64F8 ||
                  variant == kCols0F8) ? kColsEntryCost : 0;
  const int64_t wb_bound = batch * row_tiles * ((max_seqlen + plan->wb - 1) / plan->wb);
  if (units < kSplitUnits && wb_bound > units) {
    plan->split = 1;
    int64_t g = 256;
    if (g > wb_bound) g = wb_bound;
    plan->grid = (int)g;
    const int64_t slots = g + units;
    // partials [slots][rtile][L] (f32 for f32 inputs, bf16 otherwise), then
    // lse [slots][rtile] f32
    plan->workspace_bytes = (size_t)(slots * rtile * ((int64_t)kKvRank * (is_f32 ? 4 : 2) + 4));
  } else {
    plan->split = 0;
    plan->grid = (int)units;
    plan->workspace_bytes = 0;
  }
  return 0;
}

hipError_t launch_decode_plan(const DecodePlan& plan, DecodeParams p, hipStream_t s) {
  if (!plan.split || !p.plan) return hipErrorInvalidValue;
  const dim3 grid((unsigned)plan.grid), block(64);
  switch (plan.variant) {
    case kCols64: hipLaunchKernelGGL(decode_plan<Cols64>, grid, block, 0, s, p); break;
    case kCols0: hipLaunchKernelGGL(decode_plan<Cols0>, grid, block, 0, s, p); break;
    case kMixed64: hipLaunchKernelGGL(decode_plan<Mixed64>, grid, block, 0, s, p); break;
    case kMixed0: hipLaunchKernelGGL(decode_plan<Mixed0>, grid, block, 0, s, p); break;
    case kRows64: hipLaunchKernelGGL(decode_plan<Rows64>, grid, block, 0, s, p); break;
    case kRows0: hipLaunchKernelGGL(decode_plan<Rows0>, grid, block, 0, s, p); break;
    case kColsF64: hipLaunchKernelGGL(decode_plan<ColsF64>, grid, block, 0, s, p); break;
    case kColsF0: hipLaunchKernelGGL(decode_plan<ColsF0>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;  // fp8 calls plan for themselves
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodePlan& plan, DecodeParams p, int64_t rope, int is_f32,
                         hipStream_t s) {
  (void)rope;
  (void)is_f32;
  if (plan.grid <= 0) return hipSuccess;
  switch (plan.variant) {
    case kCols64: return launch_variant<Cols64>(plan, p, s);
    case kCols0: return launch_variant<Cols0>(plan, p, s);
    case kMixed64: return launch_variant<Mixed64>(plan, p, s);
    case kMixed0: return launch_variant<Mixed0>(plan, p, s);
    case kRows64: return launch_variant<Rows64>(plan, p, s);
    case kRows0: return launch_variant<Rows0>(plan, p, s);
    case kColsF64: return launch_variant<ColsF64>(plan, p, s);
    case kColsF0: return launch_variant<ColsF0>(plan, p, s);
    case kCols64F8: return launch_variant<Cols64F8>(plan, p, s);
    case kCols0F8: return launch_variant<Cols0F8>(plan, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mla
