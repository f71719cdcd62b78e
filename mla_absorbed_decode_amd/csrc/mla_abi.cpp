// mla_abi.cpp -- the extern "C" entry points of libmla (declared in
// include/mla.h). Each call validates every descriptor on the host, plans the
// launch from sizes alone and enqueues the kernels on the caller's stream.
// Validation failures return before anything is launched, so no output is
// touched ("reject malformed shapes and strides rather than mis-compute", as
// the batched-matmul tests of vllm.cpp "tests/vt/test_ops_mla_absorb.cpp"
// require of their op).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "mla.h"
#include "mla_kernels.h"
#include "prefill_kernels.h"

namespace {

int esize_of(int32_t dt) {
  switch (dt) {
    case MLA_BF16: return 2;
    case MLA_F32: return 4;
    case MLA_I32: return 4;
    case MLA_I64: return 8;
    case MLA_FP8_E4M3: return 1;
  }
  return 0;
}

bool is_value_dtype(int32_t dt) { return dt == MLA_BF16 || dt == MLA_F32; }

int64_t numel(const mla_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->rank; ++i) n *= t->shape[i];
  return n;
}

// rank, shape sign, inner stride 1, non-negative strides, data pointer present
int check_desc(const mla_tensor* t, int rank) {
  if (!t) return MLA_ERR_NULL;
  if (t->rank != rank || rank < 1 || rank > MLA_MAX_RANK) return MLA_ERR_SHAPE;
  for (int i = 0; i < rank; ++i) {
    if (t->shape[i] < 0) return MLA_ERR_SHAPE;
    if (t->stride[i] < 0) return MLA_ERR_STRIDE;
  }
  if (t->stride[rank - 1] != 1) return MLA_ERR_STRIDE;
  if (esize_of(t->dtype) == 0) return MLA_ERR_DTYPE;
  if (!t->data && numel(t) > 0) return MLA_ERR_NULL;
  return MLA_OK;
}

// every row start (all leading strides and the pointer) n-byte aligned
bool rows_aligned(const mla_tensor* t, int64_t n) {
  const int64_t es = esize_of(t->dtype);
  if ((uintptr_t)t->data % n) return false;
  for (int i = 0; i + 1 < t->rank; ++i)
    if ((t->stride[i] * es) % n) return false;
  return true;
}
bool rows_aligned16(const mla_tensor* t) { return rows_aligned(t, 16); }

// rotary positions [T] int32 contiguous, base finite and > 0
int check_rope(const mla_tensor* positions, int64_t T, double base, mla::RopeSpec* spec) {
  int rc;
  if ((rc = check_desc(positions, 1))) return rc;
  if (positions->dtype != MLA_I32) return MLA_ERR_DTYPE;
  if (positions->shape[0] != T) return MLA_ERR_SHAPE;
  if (!(base > 0.0) || !isfinite(base)) return MLA_ERR_UNSUPPORTED;
  spec->pos = (const int32_t*)positions->data;
  spec->log2_base = log2(base);
  return MLA_OK;
}

hipError_t g_last_hip = hipSuccess;

int launched(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip = e;
    return MLA_ERR_HIP;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_str(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer or descriptor is NULL";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: wrong or mismatched dtype";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: wrong rank or inconsistent sizes";
    case MLA_ERR_STRIDE: return "MLA_ERR_STRIDE: inner stride is not 1, or a stride is negative";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: sizes or alignment the kernels do not implement";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: the HIP runtime reported an error at launch";
  }
  return "unknown mla status";
}

// Validate a q fold and fill its launch parameters (nothing is launched).
static int build_absorb(const mla_tensor* q_nope, const mla_tensor* w_uk_t, const mla_tensor* q_pe,
                        const mla_tensor* positions, double base, const mla_tensor* q_out,
                        mla::BmmParams* out) {
  int rc;
  if ((rc = check_desc(q_nope, 3)) || (rc = check_desc(w_uk_t, 3)) || (rc = check_desc(q_out, 3)))
    return rc;
  if (q_pe && (rc = check_desc(q_pe, 3))) return rc;
  const int32_t dt = q_nope->dtype;
  if (!is_value_dtype(dt) || w_uk_t->dtype != dt || q_out->dtype != dt ||
      (q_pe && q_pe->dtype != dt))
    return MLA_ERR_DTYPE;
  const int64_t T = q_nope->shape[0], N = q_nope->shape[1], P = q_nope->shape[2];
  if (w_uk_t->shape[0] != N || w_uk_t->shape[1] != P) return MLA_ERR_SHAPE;
  const int64_t L = w_uk_t->shape[2];
  int64_t R = 0;
  if (q_pe) {
    if (q_pe->shape[0] != T || (q_pe->shape[1] != N && q_pe->shape[1] != 1)) return MLA_ERR_SHAPE;
    R = q_pe->shape[2];
  }
  if (q_out->shape[0] != T || q_out->shape[1] != N || q_out->shape[2] != L + R) return MLA_ERR_SHAPE;
  if (P == 0 || L == 0) return MLA_ERR_SHAPE;
  mla::RopeSpec rope;
  memset(&rope, 0, sizeof(rope));
  if (positions) {
    if (R % 2) return MLA_ERR_SHAPE;
    if ((rc = check_rope(positions, T, base, &rope))) return rc;
    if (R == 0) rope.pos = nullptr;  // no rope part: nothing to rotate
  }
  mla::BmmParams p;
  memset(&p, 0, sizeof(p));
  p.rope = rope;
  p.a = q_nope->data; p.a_st = q_nope->stride[0]; p.a_sh = q_nope->stride[1];
  p.w = w_uk_t->data; p.w_sh = w_uk_t->stride[0]; p.w_sk = w_uk_t->stride[1];
  p.out = q_out->data; p.o_st = q_out->stride[0]; p.o_sh = q_out->stride[1];
  if (q_pe) {
    p.pe = q_pe->data; p.pe_st = q_pe->stride[0]; p.pe_sh = q_pe->shape[1] == 1 ? 0 : q_pe->stride[1];
  }
  p.T = T; p.H = N; p.K = P; p.N = L; p.R = R;
  p.is_f32 = dt == MLA_F32;
  *out = p;
  return MLA_OK;
}

static int absorb_q(const mla_tensor* q_nope, const mla_tensor* w_uk_t, const mla_tensor* q_pe,
                    const mla_tensor* positions, double base, const mla_tensor* q_out,
                    mla_stream stream) {
  mla::BmmParams p;
  const int rc = build_absorb(q_nope, w_uk_t, q_pe, positions, base, q_out, &p);
  if (rc) return rc;
  return launched(mla::launch_bmm(p, (hipStream_t)stream));
}

int mla_absorb_q(const mla_tensor* q_nope, const mla_tensor* w_uk_t, const mla_tensor* q_pe,
                 const mla_tensor* q_out, mla_stream stream) {
  return absorb_q(q_nope, w_uk_t, q_pe, nullptr, 0.0, q_out, stream);
}

int mla_absorb_q_rope(const mla_tensor* q_nope, const mla_tensor* w_uk_t, const mla_tensor* q_pe,
                      const mla_tensor* positions, double base, const mla_tensor* q_out,
                      mla_stream stream) {
  if (!positions) return MLA_ERR_NULL;
  return absorb_q(q_nope, w_uk_t, q_pe, positions, base, q_out, stream);
}

int mla_v_up(const mla_tensor* o_lat, const mla_tensor* w_uv, const mla_tensor* out,
             mla_stream stream) {
  int rc;
  if ((rc = check_desc(o_lat, 3)) || (rc = check_desc(w_uv, 3)) || (rc = check_desc(out, 3)))
    return rc;
  const int32_t dt = o_lat->dtype;
  if (!is_value_dtype(dt) || w_uv->dtype != dt || out->dtype != dt) return MLA_ERR_DTYPE;
  const int64_t T = o_lat->shape[0], N = o_lat->shape[1], L = o_lat->shape[2];
  if (w_uv->shape[0] != N || w_uv->shape[1] != L) return MLA_ERR_SHAPE;
  const int64_t V = w_uv->shape[2];
  if (out->shape[0] != T || out->shape[1] != N || out->shape[2] != V) return MLA_ERR_SHAPE;
  if (L == 0 || V == 0) return MLA_ERR_SHAPE;
  mla::BmmParams p;
  memset(&p, 0, sizeof(p));
  p.a = o_lat->data; p.a_st = o_lat->stride[0]; p.a_sh = o_lat->stride[1];
  p.w = w_uv->data; p.w_sh = w_uv->stride[0]; p.w_sk = w_uv->stride[1];
  p.out = out->data; p.o_st = out->stride[0]; p.o_sh = out->stride[1];
  p.T = T; p.H = N; p.K = L; p.N = V; p.R = 0;
  p.is_f32 = dt == MLA_F32;
  return launched(mla::launch_bmm(p, (hipStream_t)stream));
}

// Validate a cache write and fill its launch parameters (nothing is launched).
static int build_cache(const mla_tensor* kv_c, const mla_tensor* k_pe,
                       const mla_tensor* slot_mapping, const mla_tensor* positions, double base,
                       const mla_tensor* kv_cache, mla::CacheWriteParams* out,
                       const float* fp8_scale = nullptr) {
  int rc;
  if ((rc = check_desc(kv_c, 2)) || (rc = check_desc(slot_mapping, 1)) ||
      (rc = check_desc(kv_cache, 3)))
    return rc;
  if (k_pe && (rc = check_desc(k_pe, 2))) return rc;
  const int32_t dt = kv_c->dtype;
  if (!is_value_dtype(dt) || kv_cache->dtype != (fp8_scale ? MLA_FP8_E4M3 : dt) ||
      (k_pe && k_pe->dtype != dt))
    return MLA_ERR_DTYPE;
  if (slot_mapping->dtype != MLA_I64 && slot_mapping->dtype != MLA_I32) return MLA_ERR_DTYPE;
  const int64_t T = kv_c->shape[0], L = kv_c->shape[1];
  const int64_t R = k_pe ? k_pe->shape[1] : 0;
  if (k_pe && k_pe->shape[0] != T) return MLA_ERR_SHAPE;
  if (slot_mapping->shape[0] != T) return MLA_ERR_SHAPE;
  if (kv_cache->shape[2] != L + R) return MLA_ERR_SHAPE;
  const int es = esize_of(dt);
  mla::CacheWriteParams p;
  memset(&p, 0, sizeof(p));
  if (positions) {
    if (R % 2) return MLA_ERR_SHAPE;
    if ((rc = check_rope(positions, T, base, &p.rope))) return rc;
    if (R == 0) p.rope.pos = nullptr;
  }
  p.kv_c = kv_c->data; p.kv_c_s0 = kv_c->stride[0];
  p.k_pe = k_pe ? k_pe->data : nullptr; p.k_pe_s0 = k_pe ? k_pe->stride[0] : 0;
  p.slots = slot_mapping->data; p.slot_is_i64 = slot_mapping->dtype == MLA_I64;
  p.cache = kv_cache->data; p.cache_s0 = kv_cache->stride[0]; p.cache_s1 = kv_cache->stride[1];
  p.num_blocks = kv_cache->shape[0]; p.page = kv_cache->shape[1];
  p.T = T; p.L = L; p.R = R; p.esize = es;
  p.vec16 = (L * es) % 16 == 0 && (R * es) % 16 == 0 && rows_aligned16(kv_c) &&
            (!k_pe || rows_aligned16(k_pe)) && rows_aligned16(kv_cache);
  if (fp8_scale) {
    // 8-element items: 16-byte aligned input rows, 8-byte aligned cache rows
    p.fp8_scale = fp8_scale;
    p.vec16 = L % 8 == 0 && R % 8 == 0 && rows_aligned16(kv_c) && (!k_pe || rows_aligned16(k_pe)) &&
              rows_aligned(kv_cache, 8);
  }
  *out = p;
  return MLA_OK;
}

static int concat_and_cache(const mla_tensor* kv_c, const mla_tensor* k_pe,
                            const mla_tensor* slot_mapping, const mla_tensor* positions,
                            double base, const mla_tensor* kv_cache, mla_stream stream) {
  mla::CacheWriteParams p;
  const int rc = build_cache(kv_c, k_pe, slot_mapping, positions, base, kv_cache, &p);
  if (rc) return rc;
  if (p.T == 0 || p.num_blocks == 0 || p.page == 0) return MLA_OK;
  return launched(mla::launch_cache_write(p, (hipStream_t)stream));
}

int mla_concat_and_cache(const mla_tensor* kv_c, const mla_tensor* k_pe,
                         const mla_tensor* slot_mapping, const mla_tensor* kv_cache,
                         mla_stream stream) {
  return concat_and_cache(kv_c, k_pe, slot_mapping, nullptr, 0.0, kv_cache, stream);
}

int mla_concat_and_cache_fp8(const mla_tensor* kv_c, const mla_tensor* k_pe,
                             const mla_tensor* slot_mapping, const mla_tensor* kv_cache,
                             const float* scale, mla_stream stream) {
  if (!scale) return MLA_ERR_NULL;
  mla::CacheWriteParams p;
  const int rc = build_cache(kv_c, k_pe, slot_mapping, nullptr, 0.0, kv_cache, &p, scale);
  if (rc) return rc;
  if (p.T == 0 || p.num_blocks == 0 || p.page == 0) return MLA_OK;
  return launched(mla::launch_cache_write(p, (hipStream_t)stream));
}

int mla_concat_and_cache_rope(const mla_tensor* kv_c, const mla_tensor* k_pe,
                              const mla_tensor* slot_mapping, const mla_tensor* positions,
                              double base, const mla_tensor* kv_cache, mla_stream stream) {
  if (!positions) return MLA_ERR_NULL;
  return concat_and_cache(kv_c, k_pe, slot_mapping, positions, base, kv_cache, stream);
}

int mla_absorb_q_and_cache(const mla_tensor* q_nope, const mla_tensor* w_uk_t,
                           const mla_tensor* q_pe, const mla_tensor* q_out,
                           const mla_tensor* kv_c, const mla_tensor* k_pe,
                           const mla_tensor* slot_mapping, const mla_tensor* kv_cache,
                           const mla_tensor* positions, double base, mla_stream stream) {
  mla::BmmParams p;
  mla::CacheWriteParams cw;
  int rc;
  if ((rc = build_absorb(q_nope, w_uk_t, q_pe, positions, base, q_out, &p))) return rc;
  if ((rc = build_cache(kv_c, k_pe, slot_mapping, positions, base, kv_cache, &cw))) return rc;
  if (cw.T != p.T) return MLA_ERR_SHAPE;  // one new latent row per query token
  if (p.T == 0) return MLA_OK;
  p.with_cw = cw.num_blocks > 0 && cw.page > 0;
  p.cw = cw;
  return launched(mla::launch_bmm(p, (hipStream_t)stream));
}

int mla_rope_interleaved(const mla_tensor* x, const mla_tensor* positions, double base,
                         mla_stream stream) {
  int rc;
  if ((rc = check_desc(x, 3))) return rc;
  if (!is_value_dtype(x->dtype)) return MLA_ERR_DTYPE;
  const int64_t T = x->shape[0], V = x->shape[1], d = x->shape[2];
  if (d % 2) return MLA_ERR_SHAPE;
  if (d > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  mla::RopeParams p;
  memset(&p, 0, sizeof(p));
  if (!positions) return MLA_ERR_NULL;
  if ((rc = check_rope(positions, T, base, &p.rope))) return rc;
  p.x = x->data; p.s0 = x->stride[0]; p.s1 = x->stride[1];
  p.T = T; p.V = V; p.d = (int)d;
  p.is_f32 = x->dtype == MLA_F32;
  p.pair_aligned = (uintptr_t)x->data % (2 * esize_of(x->dtype)) == 0 && p.s0 % 2 == 0 &&
                   p.s1 % 2 == 0;
  if (T == 0 || V == 0 || d == 0) return MLA_OK;  // nothing to rotate: nothing is launched
  return launched(mla::launch_rope(p, (hipStream_t)stream));
}

int mla_decode_workspace_size(int64_t batch, int64_t q_len, int64_t n_heads, int64_t kv_rank,
                              int64_t max_seqlen, int64_t page, int32_t dtype, size_t* bytes) {
  if (!bytes) return MLA_ERR_NULL;
  if (batch < 0 || q_len < 0 || n_heads < 0 || max_seqlen < 0 || page <= 0) return MLA_ERR_SHAPE;
  if (!is_value_dtype(dtype) && dtype != MLA_FP8_E4M3) return MLA_ERR_DTYPE;
  if (kv_rank != mla::kKvRank || page % 16) return MLA_ERR_UNSUPPORTED;
  *bytes = 0;
  if (batch == 0 || q_len == 0 || n_heads == 0) return MLA_OK;
  mla::DecodePlan plan;
  if (mla::plan_decode(batch, q_len, n_heads, 64, max_seqlen, dtype == MLA_F32, &plan,
                       dtype == MLA_FP8_E4M3))
    return MLA_ERR_UNSUPPORTED;
  *bytes = plan.workspace_bytes;
  return MLA_OK;
}

// Polls of the decode kernels' bounded LDS rendezvous before a wave gives up
// and writes NaN: 2^22 (seconds of waiting), or MLA_RENDEZVOUS_POLLS when it
// is set to a non-negative integer (tests force the give-up path with 0).
static int rendezvous_polls() {
  const char* e = getenv("MLA_RENDEZVOUS_POLLS");
  if (e && *e) {
    char* end = nullptr;
    const long v = strtol(e, &end, 10);
    if (end && *end == 0 && v >= 0 && v <= (1L << 30)) return (int)v;
  }
  return 1 << 22;
}

// Validate an attention call and fill its plan and launch parameters (nothing
// is launched). *empty is set when the call has nothing to do.
static int build_attend(const mla_tensor* q, const mla_tensor* kv_cache,
                        const mla_tensor* block_table, const mla_tensor* seqlens,
                        int64_t max_seqlen, float softmax_scale, int32_t causal,
                        const mla_tensor* out, const mla_tensor* lse, void* workspace,
                        size_t workspace_bytes, mla::DecodePlan* plan_out,
                        mla::DecodeParams* params_out, int* empty,
                        const float* descale_q = nullptr, const float* descale_k = nullptr,
                        const void* plan_buf = nullptr, size_t plan_bytes = 0,
                        bool plan_only = false) {
  int rc;
  *empty = 0;
  if ((rc = check_desc(q, 4)) || (rc = check_desc(kv_cache, 3)) ||
      (rc = check_desc(block_table, 2)) || (rc = check_desc(seqlens, 1)) ||
      (rc = check_desc(out, 4)))
    return rc;
  if (lse && (rc = check_desc(lse, 3))) return rc;
  const int32_t dt = q->dtype;
  const bool kv8 = descale_q != nullptr;  // fp8 cache, bf16 queries and output
  if (!is_value_dtype(dt) || out->dtype != dt) return MLA_ERR_DTYPE;
  if (kv8 ? (kv_cache->dtype != MLA_FP8_E4M3 || dt != MLA_BF16) : kv_cache->dtype != dt)
    return MLA_ERR_DTYPE;
  if (block_table->dtype != MLA_I32 || seqlens->dtype != MLA_I32) return MLA_ERR_DTYPE;
  if (lse && lse->dtype != MLA_F32) return MLA_ERR_DTYPE;
  const int64_t B = q->shape[0], Sq = q->shape[1], N = q->shape[2], E = q->shape[3];
  const int64_t L = out->shape[3];
  if (out->shape[0] != B || out->shape[1] != Sq || out->shape[2] != N) return MLA_ERR_SHAPE;
  if (kv_cache->shape[2] != E) return MLA_ERR_SHAPE;
  if (block_table->shape[0] != B || seqlens->shape[0] != B) return MLA_ERR_SHAPE;
  if (lse && (lse->shape[0] != B || lse->shape[1] != Sq || lse->shape[2] != N)) return MLA_ERR_SHAPE;
  if (max_seqlen < 0) return MLA_ERR_SHAPE;
  const int64_t R = E - L;
  const int64_t PG = kv_cache->shape[1], NB = kv_cache->shape[0], MB = block_table->shape[1];
  if (L != mla::kKvRank || (R != 0 && R != 64)) return MLA_ERR_UNSUPPORTED;
  if (PG <= 0 || PG % 16) return MLA_ERR_UNSUPPORTED;
  if (!rows_aligned16(q) || !rows_aligned(kv_cache, kv8 ? 8 : 16) || !rows_aligned16(out))
    return MLA_ERR_UNSUPPORTED;
  if (max_seqlen > INT32_MAX || B > INT32_MAX || Sq * N > INT32_MAX || PG > INT32_MAX ||
      MB > INT32_MAX)
    return MLA_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0 || N == 0) {
    *empty = 1;
    return MLA_OK;
  }
  mla::DecodePlan plan;
  if (mla::plan_decode(B, Sq, N, R, max_seqlen, dt == MLA_F32, &plan, kv8))
    return MLA_ERR_UNSUPPORTED;
  if (plan.workspace_bytes > 0 && !plan_only) {
    if (!workspace) return MLA_ERR_WORKSPACE;
    if (workspace_bytes < plan.workspace_bytes) return MLA_ERR_WORKSPACE;
    if ((uintptr_t)workspace % 16) return MLA_ERR_WORKSPACE;
  }
  // a plan buffer is used by split calls only (an unsplit call plans in one round trip)
  const bool use_plan = plan_buf != nullptr && plan.split;
  if (use_plan && (plan_bytes < mla::plan_bytes_for(plan.grid) || (uintptr_t)plan_buf % 16))
    return MLA_ERR_WORKSPACE;
  if (NB == 0) {
    // an empty pool can only serve empty sequences; the kernel never reads it
  }
  mla::DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.q = q->data; p.q_s0 = q->stride[0]; p.q_s1 = q->stride[1]; p.q_s2 = q->stride[2];
  p.kv = kv_cache->data; p.kv_s0 = kv_cache->stride[0]; p.kv_s1 = kv_cache->stride[1];
  p.num_blocks = NB > 0 ? NB : 1;
  p.page = (int)PG;
  p.block_table = (const int32_t*)block_table->data; p.bt_s0 = block_table->stride[0];
  p.max_blocks = (int)MB;
  p.seqlens = (const int32_t*)seqlens->data;
  p.batch = (int)B; p.q_len = (int)Sq; p.n_heads = (int)N;
  int64_t cap = MB * PG;
  if (NB == 0) cap = 0;
  p.seq_cap = (int)(max_seqlen < cap ? max_seqlen : cap);
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.causal = causal ? 1 : 0;
  p.out = out->data; p.o_s0 = out->stride[0]; p.o_s1 = out->stride[1]; p.o_s2 = out->stride[2];
  if (lse) {
    p.lse = (float*)lse->data; p.l_s0 = lse->stride[0]; p.l_s1 = lse->stride[1]; p.l_s2 = lse->stride[2];
  }
  if (plan.split) {
    const int64_t slots = (int64_t)plan.grid + plan.num_units;
    p.part_o = (float*)workspace;
    // partial rows are f32 for f32 inputs, bf16 otherwise
    const size_t pes = dt == MLA_F32 ? 4 : 2;
    p.part_lse = (float*)((char*)workspace + (size_t)slots * plan.rows_per_unit * mla::kKvRank * pes);
  }
  p.wb = plan.wb;
  p.alpha = plan.alpha;
  p.page_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if (((int64_t)1 << sh) == p.page) p.page_shift = sh;
  p.rows_per_unit = plan.rows_per_unit;
  p.row_tiles = plan.row_tiles;
  p.div_rt = mla::make_fastdiv((uint32_t)plan.row_tiles);
  p.div_nh = mla::make_fastdiv((uint32_t)N);
  p.num_units = plan.num_units;
  p.split = plan.split;
  p.grid = plan.grid;
  p.descale_q = descale_q;
  p.descale_k = descale_k;
  p.rendezvous_polls = rendezvous_polls();
  p.variant = plan.variant;
  p.plan = use_plan ? (int*)const_cast<void*>(plan_buf) : nullptr;
  *plan_out = plan;
  *params_out = p;
  return MLA_OK;
}

int mla_decode_attend(const mla_tensor* q, const mla_tensor* kv_cache,
                      const mla_tensor* block_table, const mla_tensor* seqlens,
                      int64_t max_seqlen, float softmax_scale, int32_t causal,
                      const mla_tensor* out, const mla_tensor* lse, void* workspace,
                      size_t workspace_bytes, mla_stream stream) {
  mla::DecodePlan plan;
  mla::DecodeParams p;
  int empty;
  const int rc = build_attend(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal,
                              out, lse, workspace, workspace_bytes, &plan, &p, &empty);
  if (rc || empty) return rc;
  const int64_t R = q->shape[3] - out->shape[3];
  return launched(mla::launch_decode(plan, p, R, q->dtype == MLA_F32, (hipStream_t)stream));
}

// ---------------------------------------------- one plan for several calls
int mla_decode_plan_size(int64_t batch, int64_t q_len, int64_t n_heads, int64_t kv_rank,
                         int64_t max_seqlen, int64_t page, int32_t dtype, size_t* bytes) {
  if (!bytes) return MLA_ERR_NULL;
  if (batch < 0 || q_len < 0 || n_heads < 0 || max_seqlen < 0 || page <= 0) return MLA_ERR_SHAPE;
  if (!is_value_dtype(dtype)) return MLA_ERR_DTYPE;
  if (kv_rank != mla::kKvRank || page % 16) return MLA_ERR_UNSUPPORTED;
  *bytes = 0;
  if (batch == 0 || q_len == 0 || n_heads == 0) return MLA_OK;
  mla::DecodePlan plan;
  if (mla::plan_decode(batch, q_len, n_heads, 64, max_seqlen, dtype == MLA_F32, &plan))
    return MLA_ERR_UNSUPPORTED;
  *bytes = plan.split ? mla::plan_bytes_for(plan.grid) : 0;
  return MLA_OK;
}

int mla_decode_plan(const mla_tensor* q, const mla_tensor* kv_cache, const mla_tensor* block_table,
                    const mla_tensor* seqlens, int64_t max_seqlen, int32_t causal, void* plan,
                    size_t plan_bytes, mla_stream stream) {
  int rc;
  if ((rc = check_desc(q, 4))) return rc;
  // the output's shape and layout as the attention call sees it: [B, Sq, N, L]
  // (only its sizes are used here)
  mla_tensor out = *q;
  out.shape[3] = mla::kKvRank;
  mla::DecodePlan pl;
  mla::DecodeParams p;
  int empty;
  if ((rc = build_attend(q, kv_cache, block_table, seqlens, max_seqlen, 1.f, causal, &out, nullptr,
                         nullptr, 0, &pl, &p, &empty, nullptr, nullptr, plan, plan_bytes, true)))
    return rc;
  if (empty || !pl.split) return MLA_OK;  // nothing to plan
  if (!plan) return MLA_ERR_WORKSPACE;
  return launched(mla::launch_decode_plan(pl, p, (hipStream_t)stream));
}

int mla_decode_attend_planned(const mla_tensor* q, const mla_tensor* kv_cache,
                              const mla_tensor* block_table, const mla_tensor* seqlens,
                              int64_t max_seqlen, float softmax_scale, int32_t causal,
                              const mla_tensor* out, const mla_tensor* lse, void* workspace,
                              size_t workspace_bytes, const void* plan, size_t plan_bytes,
                              mla_stream stream) {
  mla::DecodePlan pl;
  mla::DecodeParams p;
  int empty;
  const int rc = build_attend(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal,
                              out, lse, workspace, workspace_bytes, &pl, &p, &empty, nullptr,
                              nullptr, plan, plan_bytes);
  if (rc || empty) return rc;
  const int64_t R = q->shape[3] - out->shape[3];
  return launched(mla::launch_decode(pl, p, R, q->dtype == MLA_F32, (hipStream_t)stream));
}

// ---------------------------------------------- decode without allocation
// The scratch of mla_decode_attend_noalloc: a file-scope device array that
// each GPU holds from the library's load until the process ends. In host code
// the name `scratch` is only a host-side stand-in for the symbol; the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is passed to
// kernels.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // per device: the address of its copy of `scratch`

// The current device's scratch address (looked up on the first call on it).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MLA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}
}  // namespace

int mla_decode_attend_noalloc(const mla_tensor* q, const mla_tensor* kv_cache,
                              const mla_tensor* block_table, const mla_tensor* seqlens,
                              int64_t max_seqlen, float softmax_scale, int32_t causal,
                              const mla_tensor* out, const mla_tensor* lse, mla_stream stream) {
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc) return rc;
  // the same validation, plan and kernels as mla_decode_attend, with the
  // device's scratch as the workspace; a plan needing more than the scratch
  // is rejected (MLA_ERR_WORKSPACE) before anything is launched. The decode
  // workspace needs no initialisation, so nothing is cleared.
  return mla_decode_attend(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal,
                           out, lse, ws, (size_t)MLA_NOALLOC_SCRATCH_BYTES, stream);
}

int mla_decode_attend_fp8(const mla_tensor* q, const mla_tensor* kv_cache,
                          const mla_tensor* block_table, const mla_tensor* seqlens,
                          int64_t max_seqlen, float softmax_scale, int32_t causal,
                          const float* descale_q, const float* descale_k, const mla_tensor* out,
                          const mla_tensor* lse, void* workspace, size_t workspace_bytes,
                          mla_stream stream) {
  if (!descale_q || !descale_k) return MLA_ERR_NULL;
  mla::DecodePlan plan;
  mla::DecodeParams p;
  int empty;
  const int rc = build_attend(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal,
                              out, lse, workspace, workspace_bytes, &plan, &p, &empty, descale_q,
                              descale_k);
  if (rc || empty) return rc;
  const int64_t R = q->shape[3] - out->shape[3];
  return launched(mla::launch_decode(plan, p, R, 0, (hipStream_t)stream));
}

static int attend_v_up(const mla_tensor* q, const mla_tensor* kv_cache,
                       const mla_tensor* block_table, const mla_tensor* seqlens,
                       int64_t max_seqlen, float softmax_scale, int32_t causal,
                       const mla_tensor* w_uv, const mla_tensor* o_lat, const mla_tensor* out,
                       const mla_tensor* lse, void* workspace, size_t workspace_bytes,
                       const void* plan_buf, size_t plan_bytes, mla_stream stream) {
  mla::DecodePlan plan;
  mla::DecodeParams p;
  int empty, rc;
  if ((rc = build_attend(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal,
                         o_lat, lse, workspace, workspace_bytes, &plan, &p, &empty, nullptr,
                         nullptr, plan_buf, plan_bytes)))
    return rc;
  // the un-projection's arguments: o_lat [B, Sq, N, L] seen as [B*Sq, N, L] tokens
  if ((rc = check_desc(w_uv, 3)) || (rc = check_desc(out, 4))) return rc;
  const int32_t dt = q->dtype;
  if (w_uv->dtype != dt || out->dtype != dt) return MLA_ERR_DTYPE;
  const int64_t B = q->shape[0], Sq = q->shape[1], N = q->shape[2], L = o_lat->shape[3];
  if (w_uv->shape[0] != N || w_uv->shape[1] != L) return MLA_ERR_SHAPE;
  const int64_t V = w_uv->shape[2];
  if (out->shape[0] != B || out->shape[1] != Sq || out->shape[2] != N || out->shape[3] != V)
    return MLA_ERR_SHAPE;
  if (V == 0) return MLA_ERR_SHAPE;
  if (empty) return MLA_OK;
  const int64_t R = q->shape[3] - L;
  mla::VupParams v;
  memset(&v, 0, sizeof(v));
  v.w = w_uv->data; v.w_sh = w_uv->stride[0]; v.w_sk = w_uv->stride[1];
  v.out = out->data; v.o_s0 = out->stride[0]; v.o_s1 = out->stride[1]; v.o_s2 = out->stride[2];
  v.V = (int)V;
  if (mla::can_merge_vup(plan, dt == MLA_F32, v))
    return launched(mla::launch_decode_vup(plan, p, v, (hipStream_t)stream));
  // otherwise the attention call, then the un-projection over the B*Sq tokens,
  // which needs one token stride in o_lat and out
  if (Sq > 1 && (o_lat->stride[0] != Sq * o_lat->stride[1] || out->stride[0] != Sq * out->stride[1]))
    return MLA_ERR_UNSUPPORTED;
  rc = launched(mla::launch_decode(plan, p, R, dt == MLA_F32, (hipStream_t)stream));
  if (rc) return rc;
  mla::BmmParams b;
  memset(&b, 0, sizeof(b));
  b.a = o_lat->data; b.a_st = o_lat->stride[1]; b.a_sh = o_lat->stride[2];
  if (Sq == 1) b.a_st = o_lat->stride[0];
  b.w = w_uv->data; b.w_sh = w_uv->stride[0]; b.w_sk = w_uv->stride[1];
  b.out = out->data; b.o_st = Sq == 1 ? out->stride[0] : out->stride[1]; b.o_sh = out->stride[2];
  b.T = B * Sq; b.H = N; b.K = L; b.N = V; b.R = 0;
  b.is_f32 = dt == MLA_F32;
  return launched(mla::launch_bmm(b, (hipStream_t)stream));
}

int mla_decode_attend_v_up(const mla_tensor* q, const mla_tensor* kv_cache,
                           const mla_tensor* block_table, const mla_tensor* seqlens,
                           int64_t max_seqlen, float softmax_scale, int32_t causal,
                           const mla_tensor* w_uv, const mla_tensor* o_lat, const mla_tensor* out,
                           const mla_tensor* lse, void* workspace, size_t workspace_bytes,
                           mla_stream stream) {
  return attend_v_up(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal, w_uv,
                     o_lat, out, lse, workspace, workspace_bytes, nullptr, 0, stream);
}

int mla_decode_attend_v_up_planned(const mla_tensor* q, const mla_tensor* kv_cache,
                                   const mla_tensor* block_table, const mla_tensor* seqlens,
                                   int64_t max_seqlen, float softmax_scale, int32_t causal,
                                   const mla_tensor* w_uv, const mla_tensor* o_lat,
                                   const mla_tensor* out, const mla_tensor* lse, void* workspace,
                                   size_t workspace_bytes, const void* plan, size_t plan_bytes,
                                   mla_stream stream) {
  return attend_v_up(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal, w_uv,
                     o_lat, out, lse, workspace, workspace_bytes, plan, plan_bytes, stream);
}

int mla_decompress_kv(const mla_tensor* kv_c, const mla_tensor* k_pe, const mla_tensor* w_uk_t,
                      const mla_tensor* w_uv, const mla_tensor* k_out, const mla_tensor* v_out,
                      mla_stream stream) {
  int rc;
  if ((rc = check_desc(kv_c, 2)) || (rc = check_desc(w_uk_t, 3)) || (rc = check_desc(w_uv, 3)) ||
      (rc = check_desc(k_out, 3)) || (rc = check_desc(v_out, 3)))
    return rc;
  if (k_pe && (rc = check_desc(k_pe, 2))) return rc;
  const int32_t dt = kv_c->dtype;
  if (!is_value_dtype(dt) || w_uk_t->dtype != dt || w_uv->dtype != dt || k_out->dtype != dt ||
      v_out->dtype != dt || (k_pe && k_pe->dtype != dt))
    return MLA_ERR_DTYPE;
  const int64_t S = kv_c->shape[0], L = kv_c->shape[1];
  const int64_t N = w_uk_t->shape[0], P = w_uk_t->shape[1];
  if (w_uk_t->shape[2] != L || w_uv->shape[0] != N || w_uv->shape[1] != L) return MLA_ERR_SHAPE;
  const int64_t V = w_uv->shape[2];
  const int64_t R = k_pe ? k_pe->shape[1] : 0;
  if (k_pe && k_pe->shape[0] != S) return MLA_ERR_SHAPE;
  if (k_out->shape[0] != S || k_out->shape[1] != N || k_out->shape[2] != P + R) return MLA_ERR_SHAPE;
  if (v_out->shape[0] != S || v_out->shape[1] != N || v_out->shape[2] != V) return MLA_ERR_SHAPE;
  if (L == 0 || P == 0 || V == 0) return MLA_ERR_SHAPE;
  mla::BmmNtParams kp;
  memset(&kp, 0, sizeof(kp));
  kp.a = kv_c->data; kp.a_st = kv_c->stride[0]; kp.a_sh = 0;  // one latent row for every head
  kp.w = w_uk_t->data; kp.w_sh = w_uk_t->stride[0]; kp.w_sn = w_uk_t->stride[1];
  kp.out = k_out->data; kp.o_st = k_out->stride[0]; kp.o_sh = k_out->stride[1];
  if (k_pe) { kp.pe = k_pe->data; kp.pe_st = k_pe->stride[0]; }
  kp.T = S; kp.H = N; kp.K = L; kp.N = P; kp.R = R;
  kp.is_f32 = dt == MLA_F32;
  mla::BmmParams vp;
  memset(&vp, 0, sizeof(vp));
  vp.a = kv_c->data; vp.a_st = kv_c->stride[0]; vp.a_sh = 0;
  vp.w = w_uv->data; vp.w_sh = w_uv->stride[0]; vp.w_sk = w_uv->stride[1];
  vp.out = v_out->data; vp.o_st = v_out->stride[0]; vp.o_sh = v_out->stride[1];
  vp.T = S; vp.H = N; vp.K = L; vp.N = V; vp.R = 0;
  vp.is_f32 = dt == MLA_F32;
  if ((rc = launched(mla::launch_bmm_nt(kp, (hipStream_t)stream)))) return rc;
  return launched(mla::launch_bmm(vp, (hipStream_t)stream));
}

int mla_prefill_attend(const mla_tensor* q, const mla_tensor* k, const mla_tensor* v,
                       const mla_tensor* cu_seqlens_q, const mla_tensor* cu_seqlens_k,
                       int64_t max_seqlen_q, float softmax_scale, int32_t causal,
                       const mla_tensor* out, const mla_tensor* lse, mla_stream stream) {
  int rc;
  if ((rc = check_desc(q, 3)) || (rc = check_desc(k, 3)) || (rc = check_desc(v, 3)) ||
      (rc = check_desc(cu_seqlens_q, 1)) || (rc = check_desc(cu_seqlens_k, 1)) ||
      (rc = check_desc(out, 3)))
    return rc;
  if (lse && (rc = check_desc(lse, 2))) return rc;
  const int32_t dt = q->dtype;
  if (!is_value_dtype(dt) || k->dtype != dt || v->dtype != dt || out->dtype != dt)
    return MLA_ERR_DTYPE;
  if (cu_seqlens_q->dtype != MLA_I32 || cu_seqlens_k->dtype != MLA_I32) return MLA_ERR_DTYPE;
  if (lse && lse->dtype != MLA_F32) return MLA_ERR_DTYPE;
  const int64_t T = q->shape[0], N = q->shape[1], DK = q->shape[2];
  const int64_t S = k->shape[0], DV = v->shape[2];
  if (k->shape[1] != N || k->shape[2] != DK) return MLA_ERR_SHAPE;
  if (v->shape[0] != S || v->shape[1] != N) return MLA_ERR_SHAPE;
  if (out->shape[0] != T || out->shape[1] != N || out->shape[2] != DV) return MLA_ERR_SHAPE;
  if (lse && (lse->shape[0] != T || lse->shape[1] != N)) return MLA_ERR_SHAPE;
  const int64_t B = cu_seqlens_q->shape[0] - 1;
  if (B < 0 || cu_seqlens_k->shape[0] != B + 1) return MLA_ERR_SHAPE;
  if (max_seqlen_q < 0) return MLA_ERR_SHAPE;
  if (dt != MLA_BF16 || !mla::mha_supported((int)DK, (int)DV)) return MLA_ERR_UNSUPPORTED;
  if (!rows_aligned16(q) || !rows_aligned16(k) || !rows_aligned16(v) || !rows_aligned(out, 8))
    return MLA_ERR_UNSUPPORTED;
  if (T > INT32_MAX || S > INT32_MAX || max_seqlen_q > INT32_MAX || N > 65535 || B > 65535)
    return MLA_ERR_UNSUPPORTED;
  if (B == 0 || N == 0 || max_seqlen_q == 0 || T == 0) return MLA_OK;
  mla::MhaParams p;
  memset(&p, 0, sizeof(p));
  p.q = q->data; p.q_s0 = q->stride[0]; p.q_s1 = q->stride[1];
  p.k = k->data; p.k_s0 = k->stride[0]; p.k_s1 = k->stride[1];
  p.v = v->data; p.v_s0 = v->stride[0]; p.v_s1 = v->stride[1];
  p.out = out->data; p.o_s0 = out->stride[0]; p.o_s1 = out->stride[1];
  if (lse) { p.lse = (float*)lse->data; p.l_s0 = lse->stride[0]; p.l_s1 = lse->stride[1]; }
  p.cu_q = (const int32_t*)cu_seqlens_q->data;
  p.cu_k = (const int32_t*)cu_seqlens_k->data;
  p.T = T; p.S = S;
  p.n_heads = (int)N; p.batch = (int)B; p.max_q = (int)max_seqlen_q;
  p.dk = (int)DK; p.dv = (int)DV;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  return launched(mla::launch_mha(p, (hipStream_t)stream));
}

int mla_sparse_workspace_size(int64_t tokens, int64_t n_heads, int64_t topk, size_t* bytes) {
  if (!bytes) return MLA_ERR_NULL;
  if (tokens < 0 || n_heads < 0 || topk < 0) return MLA_ERR_SHAPE;
  if (topk > mla::kSparseMaxTopk) return MLA_ERR_UNSUPPORTED;
  int split_len, nsplit;
  *bytes = mla::plan_sparse(tokens, n_heads, topk, &split_len, &nsplit);
  return MLA_OK;
}

int mla_sparse_decode_fp8(const mla_tensor* q, const mla_tensor* kv_cache,
                          const mla_tensor* indices, float softmax_scale, const mla_tensor* out,
                          const mla_tensor* lse, void* workspace, size_t workspace_bytes,
                          mla_stream stream) {
  int rc;
  if ((rc = check_desc(q, 4)) || (rc = check_desc(kv_cache, 3)) || (rc = check_desc(indices, 3)) ||
      (rc = check_desc(out, 4)))
    return rc;
  if (lse && (rc = check_desc(lse, 3))) return rc;
  if (q->dtype != MLA_BF16 || out->dtype != MLA_BF16 || kv_cache->dtype != MLA_FP8_E4M3 ||
      indices->dtype != MLA_I32 || (lse && lse->dtype != MLA_F32))
    return MLA_ERR_DTYPE;
  const int64_t B = q->shape[0], Sq = q->shape[1], N = q->shape[2], E = q->shape[3];
  const int64_t NB = kv_cache->shape[0], PG = kv_cache->shape[1], K = indices->shape[2];
  if (out->shape[0] != B || out->shape[1] != Sq || out->shape[2] != N) return MLA_ERR_SHAPE;
  if (indices->shape[0] != B || indices->shape[1] != Sq) return MLA_ERR_SHAPE;
  if (lse && (lse->shape[0] != B || lse->shape[1] != Sq || lse->shape[2] != N)) return MLA_ERR_SHAPE;
  // the 656-byte entry of 512 e4m3 codes, 4 f32 scales and 64 bf16 rope values
  if (E != 576 || out->shape[3] != 512 || kv_cache->shape[2] != 656) return MLA_ERR_UNSUPPORTED;
  if (K > mla::kSparseMaxTopk || PG <= 0 || PG > INT32_MAX || B * Sq > INT32_MAX ||
      N > 65535 * 64)
    return MLA_ERR_UNSUPPORTED;
  if (!rows_aligned16(q) || !rows_aligned16(kv_cache) || !rows_aligned(out, 8))
    return MLA_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0 || N == 0) return MLA_OK;
  int split_len, nsplit;
  const size_t need = mla::plan_sparse(B * Sq, N, K, &split_len, &nsplit);
  if (need > 0 && (!workspace || workspace_bytes < need || (uintptr_t)workspace % 16))
    return MLA_ERR_WORKSPACE;
  mla::SparseParams p;
  memset(&p, 0, sizeof(p));
  p.q = q->data; p.q_s0 = q->stride[0]; p.q_s1 = q->stride[1]; p.q_s2 = q->stride[2];
  p.kv = (const uint8_t*)kv_cache->data; p.kv_s0 = kv_cache->stride[0]; p.kv_s1 = kv_cache->stride[1];
  p.num_slots = NB * PG; p.page = (int)PG;
  p.page_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if (((int64_t)1 << sh) == PG) p.page_shift = sh;
  p.idx = (const int32_t*)indices->data; p.i_s0 = indices->stride[0]; p.i_s1 = indices->stride[1];
  p.topk = (int)K;
  p.out = out->data; p.o_s0 = out->stride[0]; p.o_s1 = out->stride[1]; p.o_s2 = out->stride[2];
  if (lse) {
    p.lse = (float*)lse->data; p.l_s0 = lse->stride[0]; p.l_s1 = lse->stride[1]; p.l_s2 = lse->stride[2];
  }
  p.batch = (int)B; p.q_len = (int)Sq; p.n_heads = (int)N;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.split_len = split_len; p.nsplit = nsplit;
  if (nsplit > 1) {
    p.part_o = (float*)workspace;
    p.part_lse = (float*)((char*)workspace + (size_t)B * Sq * nsplit * N * 512 * sizeof(float));
  }
  return launched(mla::launch_sparse(p, (hipStream_t)stream));
}

}  // extern "C"
