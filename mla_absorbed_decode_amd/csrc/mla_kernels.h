// mla_kernels.h -- internal interface between the C-ABI layer (mla_abi.cpp)
// and the kernel translation units. Plain structs of pointers and sizes; the
// launchers enqueue on the given stream and return the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kKvRank = 512;     // latent width L the attention kernels implement
constexpr int kSplitUnits = 1024; // fewer (sequence, row-tile) units than this => split KV

// ------------------------------------------------------------ rotary embedding
// Interleaved rotation of the rope part: pair (2i, 2i+1) of token t's vector
// turns by pos[t] * base^(-2i/d). pos == NULL: no rotation (a bit copy).
struct RopeSpec {
  const int32_t* pos;  // [T] positions, or NULL
  double log2_base;    // log2(base)
};

// In-place rotation of x [T, V, d] (strides s0, s1, 1).
struct RopeParams {
  void* x; int64_t s0, s1;
  int64_t T, V;
  int d;
  int is_f32;
  int pair_aligned;  // every pair starts on a 2-element boundary: one access per pair
  RopeSpec rope;
};
hipError_t launch_rope(const RopeParams& p, hipStream_t s);

// ------------------------------------------------------------ cache write
struct CacheWriteParams {
  const void* kv_c;  int64_t kv_c_s0;    // [T, L] row stride (elements)
  const void* k_pe;  int64_t k_pe_s0;    // [T, R] (NULL when R == 0)
  const void* slots; int slot_is_i64;    // [T]
  void* cache;       int64_t cache_s0, cache_s1;  // [NB, PG, L+R]
  int64_t num_blocks, page;
  int64_t T, L, R;
  int esize;         // 2 (bf16) or 4 (f32)
  int vec16;         // 1 when every row start is 16-byte aligned and L, R are multiples of 16/esize
  RopeSpec rope;     // rotate k_pe by its token's position before writing
  // fp8 cache (OCP e4m3fn bytes; strides in bytes): each element is stored as
  // e4m3(x / *fp8_scale); NULL for a bf16 / f32 cache. With it, vec16 means
  // 8-element items (16-byte aligned input rows, 8-byte aligned cache rows).
  const float* fp8_scale;
};
hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s);

// ------------------------------------------------------------- batched matmul
// out[t, h, n] = sum_k a[t, h, k] * w[h, k, n]  (+ optional copy of the rope
// rows into out[t, h, Nout : Nout + R], rotated when rope.pos is set).
struct BmmParams {
  const void* a; int64_t a_st, a_sh;        // a[t, h, k]: t stride, h stride (k stride 1)
  const void* w; int64_t w_sh, w_sk;        // w[h, k, n]: h stride, k stride (n stride 1)
  void* out;     int64_t o_st, o_sh;        // out[t, h, n]
  const void* pe; int64_t pe_st, pe_sh;     // rope rows [t, h or broadcast, R] (pe_sh 0 = broadcast)
  int64_t T, H, K, N, R;
  int is_f32;
  RopeSpec rope;  // rotate the rope rows by their token's position while copying
  int with_cw;    // also perform the cache write cw, in extra workgroups (head slot H)
  CacheWriteParams cw;
};
hipError_t launch_bmm(const BmmParams& p, hipStream_t s);

// ------------------------------------------------------------------ decode
// Division of 32-bit unsigned integers by a fixed d >= 1 as a multiply-high,
// an add and two shifts (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994, the round-up method): with
// l = ceil(log2 d) and mul = floor(2^32 (2^l - d) / d) + 1,
// n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0) where t = mulhi(n, mul),
// exact for every n < 2^32.
struct FastDiv {
  uint32_t mul, sh1, sh2;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && ((uint64_t)1 << l) < d) ++l;
  FastDiv f;
  f.mul = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
  f.sh1 = l < 1 ? l : 1;
  f.sh2 = l > 1 ? l - 1 : 0;
  return f;
}

struct DecodeParams {
  const void* q; int64_t q_s0, q_s1, q_s2;          // q [B, Sq, N, E]
  const void* kv; int64_t kv_s0, kv_s1;              // cache [NB, PG, E]
  int64_t num_blocks;
  int page;
  int page_shift;         // log2(page) when page is a power of two, else -1
  const int32_t* block_table; int64_t bt_s0; int max_blocks;
  const int32_t* seqlens;
  int batch, q_len, n_heads;
  int seq_cap;            // min(max_seqlen, max_blocks * page)
  float scale_log2;       // softmax_scale * log2(e)
  int causal;
  void* out; int64_t o_s0, o_s1, o_s2;              // out [B, Sq, N, L]
  float* lse; int64_t l_s0, l_s1, l_s2;             // lse [B, Sq, N] or NULL
  float* part_o;          // split partials [slots][rows_per_unit][L]: f32 rows for f32 inputs, else bf16
  float* part_lse;        // [slots][rows_per_unit] (log2 domain)
  int rows_per_unit;      // rows of (query, head) per unit
  int row_tiles;          // units per sequence
  FastDiv div_rt;         // divides by row_tiles
  FastDiv div_nh;         // divides by n_heads
  int num_units;
  int split;              // 1: split-KV over `grid` workgroups + merge
  int grid;
  int wb;                 // plan granularity: tokens per work block (the tile size)
  int alpha;              // plan cost of entering a unit, in work blocks
  // fp8 cache (OCP e4m3fn bytes, kv strides in bytes): the scores take
  // q * descale_q and keys * descale_k, the output values * descale_k. NULL
  // for a bf16 / f32 cache.
  const float* descale_q;
  const float* descale_k;
  // polls of the compute waves' LDS rendezvous before a wave gives up and
  // marks its outputs NaN (the few-head layouts)
  int rendezvous_polls;
  // a split plan computed once (decode_plan) for several calls: NULL = every
  // workgroup plans for itself. The plan kernel writes it; the attention and
  // merge kernels read it and plan for themselves when its header does not
  // match their call.
  int* plan;
  int variant;            // kernel variant of the call (checked against the plan)
};

// Plan buffer: kPlanHdrInts header ints, the merge's inclusive cost scan
// (kSplitUnits ints), then one descriptor of kDescInts ints per workgroup:
// [u0, u1, tlo0, thi1, nsteps, units stored (-1: too many, plan in the kernel),
// pages stored, 0], kDescUnits entries [visible keys, sequence length, first
// staged page, live | part << 1], then kDescPages staged block ids.
constexpr int kPlanMagic = 0x4d4c4150;
constexpr int kPlanHdrInts = 64;
constexpr int kDescInts = 1024;
constexpr int kDescUnits = 96;
constexpr int kDescPageOff = 8 + 4 * kDescUnits;
constexpr int kDescPages = 512;
static_assert(kDescPageOff + kDescPages <= kDescInts, "descriptor layout");
constexpr size_t plan_bytes_for(int grid) {
  return ((size_t)kPlanHdrInts + kSplitUnits + (size_t)grid * kDescInts) * 4;
}

// The W_UV un-projection fused into the split merge: out[b, i, h, 0:V] =
// o_lat[b, i, h, :] . W_UV[h] (o_lat is DecodeParams::out).
struct VupParams {
  const void* w; int64_t w_sh, w_sk;   // W_UV [N, L, V], V contiguous
  void* out; int64_t o_s0, o_s1, o_s2;  // out [B, Sq, N, V], V contiguous
  int V;
};

// Launch plan chosen on the host from sizes alone (never from seqlens).
struct DecodePlan {
  int variant;        // kernel variant id
  int rows_per_unit;
  int row_tiles;
  int num_units;
  int split;
  int grid;
  int wb;
  int alpha;
  size_t workspace_bytes;
};
// kv8: an fp8 cache (bf16 queries); its layout takes units of 16 rows.
int plan_decode(int64_t batch, int64_t q_len, int64_t n_heads, int64_t rope, int64_t max_seqlen,
                int is_f32, DecodePlan* plan, int kv8 = 0);
// Compute the split plan of a call into p.plan (a split plan only).
hipError_t launch_decode_plan(const DecodePlan& plan, DecodeParams p, hipStream_t s);
hipError_t launch_decode(const DecodePlan& plan, DecodeParams p, int64_t rope, int is_f32,
                         hipStream_t s);
// The same with the merge and the W_UV un-projection in one kernel; only for a
// split plan (see can_merge_vup). The caller launches the plain un-projection
// otherwise.
bool can_merge_vup(const DecodePlan& plan, int is_f32, const VupParams& v);
hipError_t launch_decode_vup(const DecodePlan& plan, DecodeParams p, const VupParams& v,
                             hipStream_t s);

}  // namespace mla
