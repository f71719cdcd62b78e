/*
 * mla.h -- C ABI of libmla: multi-head latent attention (MLA) in
 * weight-absorbed form, for decode and chunked prefill, on AMD Instinct
 * MI355X (gfx950).
 *
 * The compute calls follow the statement of the method on these pages:
 *   [P1] vllm.cpp "tests/vt/test_ops_mla_absorb.cpp" -- the batched matmul
 *        (q-side W_UK fold and W_UV un-projection) and the nope/rope concat;
 *   [P2] memra-engine 0.124.1 "tests/mla_gpu_forward.rs" -- absorb q,
 *        absorbed attention over the [c_kv | k_pe] latent cache, decompress v,
 *        latent append, gates 1 and 2;
 *   [P3] vLLM "tests/kernels/attention/test_mla_cross_layer_kernel_equivalence.py"
 *        -- concat_and_cache_mla into a paged, possibly block-major cache view,
 *        and paged dense decode returning (out, lse).
 *
 * Conventions shared by every call
 * --------------------------------
 * Tensors are passed as `mla_tensor` descriptors: a pointer to element
 * [0, 0, ...] (any storage offset already folded in), a dtype, a rank, and
 * per-dimension sizes and strides counted in ELEMENTS ([P1] keeps its tensor
 * descriptor the same way). The innermost stride must be 1; the others may be
 * anything non-negative, so transposed and block-major views are accepted as
 * they are.
 *
 * Memory: every data pointer is a DEVICE pointer on the current HIP device.
 * The caller owns every buffer, the workspace and the stream. The library
 * allocates no memory, keeps no pointer after a call returns and never
 * synchronises; all work is enqueued on `stream` (a hipStream_t, NULL = the
 * null stream), so results are ready when that stream reaches the call.
 *
 * Errors: each call returns MLA_OK (0) or a negative status. Arguments are
 * validated on the host before anything is launched; on any error nothing is
 * enqueued and no output is touched. MLA_ERR_HIP reports a failed launch.
 * mla_status_str() names a status.
 *
 * Data types: MLA_BF16 and MLA_F32 for values (all value tensors of one call
 * share one dtype); MLA_I32 / MLA_I64 for indices. bf16 arithmetic uses fp32
 * accumulation and rounds outputs to nearest-even; copies move bits.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum {
  MLA_BF16 = 1,
  MLA_F32 = 2,
  MLA_I32 = 3,
  MLA_I64 = 4,
  MLA_FP8_E4M3 = 5 /* OCP FP8 E4M3 ("e4m3fn") bytes: the fp8 latent cache */
};

/* status codes */
enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer or descriptor is NULL */
  MLA_ERR_DTYPE = -2,       /* wrong or mismatched dtype */
  MLA_ERR_SHAPE = -3,       /* wrong rank or inconsistent sizes */
  MLA_ERR_STRIDE = -4,      /* inner stride != 1, or a negative stride */
  MLA_ERR_UNSUPPORTED = -5, /* a size outside what the kernels implement */
  MLA_ERR_WORKSPACE = -6,   /* workspace missing or too small */
  MLA_ERR_HIP = -7          /* the HIP runtime reported an error at launch */
};

#define MLA_MAX_RANK 4

typedef struct mla_tensor {
  void* data;                     /* device address of element [0,...,0] */
  int32_t dtype;                  /* MLA_BF16 / MLA_F32 / MLA_I32 / MLA_I64 / MLA_FP8_E4M3 */
  int32_t rank;                   /* 1..MLA_MAX_RANK */
  int64_t shape[MLA_MAX_RANK];    /* sizes; entries >= rank are ignored */
  int64_t stride[MLA_MAX_RANK];   /* element strides; stride[rank-1] must be 1 */
} mla_tensor;

typedef void* mla_stream; /* a hipStream_t */

/*
 * mla_absorb_q -- fold the no-position part of the query through W_UK and
 * append the rotary part ([P1] the q-side W_UK fold as a strided batched
 * matmul whose transposed output feeds the nope/rope concat; [P2]
 * `mla_absorb_q`).
 *
 *   q_out[t, h, 0:L]   = sum_p q_nope[t, h, p] * w_uk_t[h, p, 0:L]
 *   q_out[t, h, L:L+R] = q_pe[t, h, :]      (bit copy; q_pe may be [T, 1, R],
 *                                            then its one row is broadcast)
 *
 *   q_nope  [T, N, P]     bf16 or f32, any strides (inner 1)
 *   w_uk_t  [N, P, L]     same dtype, any strides (inner 1)
 *   q_pe    [T, N, R] or [T, 1, R], same dtype; NULL when R == 0
 *   q_out   [T, N, L + R] same dtype, any strides (inner 1) -- e.g. a view
 *           into the attention query buffer
 * T may be 0 (nothing is launched). Sizes: N, P, L, R >= 1 except R == 0
 * with q_pe NULL. q_out must not overlap the inputs.
 */
int mla_absorb_q(const mla_tensor* q_nope, const mla_tensor* w_uk_t, const mla_tensor* q_pe,
                 const mla_tensor* q_out, mla_stream stream);

/*
 * mla_concat_and_cache -- write each token's latent row [kv_c | k_pe] into a
 * paged cache through a slot mapping ([P3] concat_and_cache_mla with
 * kv_cache_dtype "auto" and scale 1, written into the middle layer of a
 * block-major unified slot; [P2] `mla_append_latent`).
 *
 *   for t with 0 <= slot_mapping[t] < NB * PG:
 *     blk = slot / PG, off = slot % PG
 *     kv_cache[blk, off, 0:L]   = kv_c[t, :]
 *     kv_cache[blk, off, L:L+R] = k_pe[t, :]
 *
 *   kv_c          [T, L]      bf16 or f32, row stride any (inner 1)
 *   k_pe          [T, R]      same dtype; NULL when R == 0
 *   slot_mapping  [T]         MLA_I64 (or MLA_I32), contiguous
 *   kv_cache      [NB, PG, L + R] same dtype; stride[0] and stride[1] any
 *                 (a per-layer view of a block-major allocation has stride[0]
 *                 = n_layers * PG * (L + R) and a non-zero offset)
 * A copy of bits: every element is reproduced exactly. Tokens whose slot is
 * negative or >= NB * PG are skipped; nothing outside the written rows is
 * touched. Duplicate slots race: one of the writers' rows lands.
 */
int mla_concat_and_cache(const mla_tensor* kv_c, const mla_tensor* k_pe,
                         const mla_tensor* slot_mapping, const mla_tensor* kv_cache,
                         mla_stream stream);

/*
 * mla_concat_and_cache_fp8 -- the latent-cache write into an fp8 cache ([P3]
 * concat_and_cache_mla with its cache dtype and scale arguments; the dense
 * fp8 decode tests hold the cache as torch.float8_e4m3fn). As
 * mla_concat_and_cache, except that every element x of [kv_c | k_pe] is
 * stored as the OCP E4M3 code of x / *scale: the quotient in float, rounded
 * to the nearest e4m3 value with ties to the even mantissa; magnitudes above
 * 448 (infinities included) saturate to +-448, NaN becomes the NaN code with
 * x's sign, a zero result keeps its sign.
 *
 *   kv_c, k_pe     as mla_concat_and_cache (bf16 or f32)
 *   slot_mapping   as mla_concat_and_cache
 *   kv_cache       [NB, PG, L + R] MLA_FP8_E4M3, strides any (in bytes, since
 *                  an element is one byte)
 *   scale          device pointer to one float, read by the kernel when it
 *                  runs (so a captured graph follows later values); not NULL
 */
int mla_concat_and_cache_fp8(const mla_tensor* kv_c, const mla_tensor* k_pe,
                             const mla_tensor* slot_mapping, const mla_tensor* kv_cache,
                             const float* scale, mla_stream stream);

/*
 * Interleaved rotary position embedding (memra-engine 0.124.1
 * "tests/mla_gpu_forward.rs", gate 3, gpu_mla_rope_interleaved_matches_cpu:
 * d_rope 8 and 64, base 8e6, positions 13 * p; d_rope 0 is a no-op). With
 * d = the rope width, pair (2i, 2i+1) of token t's vector turns by
 * theta = positions[t] * base^(-2i/d):
 *   (x[2i], x[2i+1]) -> (x[2i] cos theta - x[2i+1] sin theta,
 *                        x[2i] sin theta + x[2i+1] cos theta)
 * The angle and the rotation are computed in double and rounded once to the
 * value dtype.
 *
 * mla_rope_interleaved -- rotate x in place.
 *   x          [T, V, d] bf16 or f32, any strides (inner 1); d even
 *   positions  [T] MLA_I32, contiguous (any values, negative included)
 *   base       > 0, finite
 * d == 0, T == 0 or V == 0: nothing is launched and x is untouched.
 */
int mla_rope_interleaved(const mla_tensor* x, const mla_tensor* positions, double base,
                         mla_stream stream);

/*
 * mla_absorb_q_rope -- mla_absorb_q with the rotary part rotated as it is
 * appended: q_out[t, h, L:L+R] = rope(q_pe[t, h, :], positions[t]) (the
 * rotation fused into the fold's epilogue). R must be even; positions and
 * base as for mla_rope_interleaved; positions may not be NULL.
 */
int mla_absorb_q_rope(const mla_tensor* q_nope, const mla_tensor* w_uk_t, const mla_tensor* q_pe,
                      const mla_tensor* positions, double base, const mla_tensor* q_out,
                      mla_stream stream);

/*
 * mla_concat_and_cache_rope -- mla_concat_and_cache with each token's k_pe
 * rotated by positions[t] as it is written: kv_cache[blk, off, L:L+R] =
 * rope(k_pe[t, :], positions[t]); the kv_c part stays a bit copy. R must be
 * even; positions [T] MLA_I32 contiguous, not NULL; base as above.
 */
int mla_concat_and_cache_rope(const mla_tensor* kv_c, const mla_tensor* k_pe,
                              const mla_tensor* slot_mapping, const mla_tensor* positions,
                              double base, const mla_tensor* kv_cache, mla_stream stream);

/*
 * mla_absorb_q_and_cache -- a decode step's two input calls in one launch:
 * mla_absorb_q (q_nope, w_uk_t, q_pe -> q_out) and mla_concat_and_cache
 * (kv_c, k_pe -> kv_cache at slot_mapping) for the same T new tokens, each
 * query token bringing its own latent row ([P2] gate 2: every decode step
 * appends the new token's [c_kv | k_pe] row and decodes its query). With
 * positions (not NULL) q_pe and k_pe are both rotated by their token's
 * position as in mla_absorb_q_rope and mla_concat_and_cache_rope; with NULL
 * both are copied. Every argument is validated as for those calls, and
 * kv_c must have T rows; on any error nothing is launched. The results equal
 * the two calls made one after the other, bit for bit.
 */
int mla_absorb_q_and_cache(const mla_tensor* q_nope, const mla_tensor* w_uk_t,
                           const mla_tensor* q_pe, const mla_tensor* q_out,
                           const mla_tensor* kv_c, const mla_tensor* k_pe,
                           const mla_tensor* slot_mapping, const mla_tensor* kv_cache,
                           const mla_tensor* positions, double base, mla_stream stream);

/*
 * mla_decode_workspace_size -- bytes of device workspace mla_decode_attend
 * needs for a call of these sizes (an upper bound that depends only on the
 * arguments, never on the device or on seqlens' contents).
 *
 *   batch B, q_len Sq (query tokens per sequence), n_heads N, kv_rank L,
 *   max_seqlen (>= every seqlens[b]), page PG, dtype of q -- or
 *   MLA_FP8_E4M3 for mla_decode_attend_fp8 (an fp8 cache plans differently).
 * Writes *bytes; returns MLA_OK or a validation error.
 */
int mla_decode_workspace_size(int64_t batch, int64_t q_len, int64_t n_heads, int64_t kv_rank,
                              int64_t max_seqlen, int64_t page, int32_t dtype, size_t* bytes);

/*
 * mla_decode_attend -- paged decode / chunked-prefill attention of N query
 * heads over the shared latent cache, in split-KV form with a log-sum-exp
 * merge ([P3] flash_mla_with_kvcache: q [B, Sq, N, 576], a paged cache with
 * block_table and cache_seqlens, head_dim_v 512, softmax scale 576^-0.5,
 * returning (out, lse); [P2] `mla_attn_absorbed`).
 *
 * For sequence b, query i sits at position pos = seqlens[b] - Sq + i (the
 * queries are the last Sq tokens of the sequence); with causal != 0 it sees
 * keys 0..pos, otherwise keys 0..seqlens[b]-1. Key j of sequence b is the
 * cache row kv_cache[block_table[b, j / PG], j % PG, :].
 *
 *   s_j      = softmax_scale * sum_e q[b, i, h, e] * key_j[e]   (e < L + R)
 *   out[...] = sum_j softmax(s)_j * key_j[0:L]    (the value is the c_kv part)
 *   lse[...] = ln sum_j exp(s_j)                  (-inf, and out = 0, when no
 *                                                  key is visible)
 *
 *   q            [B, Sq, N, L + R]  bf16 or f32, any strides (inner 1)
 *   kv_cache     [NB, PG, L + R]    same dtype; stride[0] any (block-major
 *                views allowed), stride[1] a multiple of 8 elements
 *   block_table  [B, MB]            MLA_I32, row stride any; only entries
 *                j < ceil(seqlens[b] / PG) are read. Entries must lie in
 *                [0, NB); one outside is clamped into that range, so every
 *                read stays inside the cache, but the rows of that sequence
 *                are then unspecified.
 *   seqlens      [B]                MLA_I32, contiguous, on the device; values
 *                are clamped to [0, min(max_seqlen, MB * PG)]
 *   max_seqlen   host upper bound of seqlens (sizes the launch; no D2H copy)
 *   out          [B, Sq, N, L]      same dtype as q, any strides (inner 1)
 *   lse          [B, Sq, N]         MLA_F32, any strides; or NULL
 *   workspace    device scratch of at least mla_decode_workspace_size()
 *                bytes (16-byte aligned); may be NULL when that size is 0.
 *                Its contents need no initialisation and carry nothing from
 *                one call to the next, so one buffer serves any sequence of
 *                calls on one stream; calls that run concurrently need
 *                separate workspaces.
 * Supported: L == 512; R == 0 or 64; PG a multiple of 16; L + R rows 16-byte
 * aligned (pointer and strides). The result depends only on the inputs'
 * values and sizes -- not on strides, pointers or the device -- so a
 * block-major view and a contiguous copy give bit-identical outputs, and so
 * do repeated calls.
 */
int mla_decode_attend(const mla_tensor* q, const mla_tensor* kv_cache,
                      const mla_tensor* block_table, const mla_tensor* seqlens,
                      int64_t max_seqlen, float softmax_scale, int32_t causal,
                      const mla_tensor* out, const mla_tensor* lse, void* workspace,
                      size_t workspace_bytes, mla_stream stream);

/*
 * mla_decode_attend_noalloc -- mla_decode_attend for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same validation, plan, kernels and results, bit for bit.
 * Instead of a caller's workspace the call uses a scratch array of
 * MLA_NOALLOC_SCRATCH_BYTES bytes held in device memory by the library on
 * every GPU it runs on, from its load until the process ends. The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * its first call on a device looks the array's address up once.
 * Errors: as mla_decode_attend; MLA_ERR_WORKSPACE when the call's plan needs
 * more than MLA_NOALLOC_SCRATCH_BYTES (mla_decode_workspace_size tells), before
 * anything is launched; MLA_ERR_HIP if the address lookup fails.
 * Every call on one GPU shares that GPU's array and leaves the last call's
 * contents in it: calls that overlap in time on one GPU (concurrent streams,
 * host threads) race and must not be issued; calls in order on one stream
 * are safe.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20)
int mla_decode_attend_noalloc(const mla_tensor* q, const mla_tensor* kv_cache,
                              const mla_tensor* block_table, const mla_tensor* seqlens,
                              int64_t max_seqlen, float softmax_scale, int32_t causal,
                              const mla_tensor* out, const mla_tensor* lse, mla_stream stream);

/*
 * mla_decode_attend_fp8 -- mla_decode_attend over an fp8 latent cache ([P3]
 * test_flashmla_dense_fp8_decode_unified_slot_view: flash_mla_with_kvcache_fp8
 * with a bf16 query, a float8_e4m3fn paged cache, descale_q and descale_k).
 * The query's values are q * descale_q and every cache value is its e4m3
 * value times descale_k (keys and values alike); then exactly the
 * mla_decode_attend definition:
 *   s_j      = softmax_scale * descale_q * descale_k * sum_e q[e] * k8_j[e]
 *   out[...] = descale_k * sum_j softmax(s)_j * k8_j[0:L]
 *   q          [B, Sq, N, L + R] MLA_BF16, as mla_decode_attend
 *   kv_cache   [NB, PG, L + R]  MLA_FP8_E4M3; stride[0] any (block-major views
 *              allowed); pointer and strides multiples of 8 bytes
 *   descale_q, descale_k   device pointers to one float each, read by the
 *              kernel when it runs; not NULL
 *   out        [B, Sq, N, L] MLA_BF16; lse, block_table, seqlens, workspace as
 *              mla_decode_attend, with the workspace sized by
 *              mla_decode_workspace_size(..., MLA_FP8_E4M3, ...)
 * Supported: L == 512, R == 0 or 64, PG a multiple of 16. Every e4m3 value is
 * exact in bf16: the widened rows enter the same bf16 MFMA arithmetic as a
 * bf16 cache, and the same determinism holds (bit-identical outputs for a
 * block-major view and a contiguous copy).
 */
int mla_decode_attend_fp8(const mla_tensor* q, const mla_tensor* kv_cache,
                          const mla_tensor* block_table, const mla_tensor* seqlens,
                          int64_t max_seqlen, float softmax_scale, int32_t causal,
                          const float* descale_q, const float* descale_k, const mla_tensor* out,
                          const mla_tensor* lse, void* workspace, size_t workspace_bytes,
                          mla_stream stream);

/*
 * mla_decode_attend_v_up -- mla_decode_attend followed by the W_UV
 * un-projection of its output, with the split merge and the un-projection in
 * one kernel where the plan splits ([P3] dense decode returning (out, lse);
 * [P2] gate 1, mla_attn_absorbed then mla_decompress_v). o_lat, lse and the
 * workspace are as for mla_decode_attend (o_lat is required: it receives the
 * latent output as usual); then
 *   out[b, i, h, 0:V] = sum_l o_lat[b, i, h, l] * w_uv[h, l, 0:V]
 *   w_uv  [N, L, V]    q's dtype, any strides (inner 1)
 *   out   [B, Sq, N, V] q's dtype, any strides (inner 1)
 * out equals mla_v_up on o_lat bit for bit. The fused kernel takes bf16, a
 * split plan, V = 16, 32, 64 or 128 and 16-byte aligned w_uv rows; other
 * calls run the two kernels one after the other (then, for Sq > 1, o_lat and
 * out must keep one token stride: stride[0] == Sq * stride[1], else
 * MLA_ERR_UNSUPPORTED before anything is launched).
 */
int mla_decode_attend_v_up(const mla_tensor* q, const mla_tensor* kv_cache,
                           const mla_tensor* block_table, const mla_tensor* seqlens,
                           int64_t max_seqlen, float softmax_scale, int32_t causal,
                           const mla_tensor* w_uv, const mla_tensor* o_lat, const mla_tensor* out,
                           const mla_tensor* lse, void* workspace, size_t workspace_bytes,
                           mla_stream stream);

/*
 * mla_decode_plan -- the split plan of a decode call, computed once for
 * several calls ([P3] dense decode tests: the tile-scheduler metadata and
 * split count are computed once from cache_seqlens and passed to every layer's
 * decode call). Without a plan every workgroup of an attention call plans its
 * own share (two dependent global round trips: sequence lengths, then block
 * table); with one it reads its share in one. The plan depends on q's sizes,
 * the cache's page size and page count, block_table, seqlens (their values),
 * max_seqlen and causal -- not on q's, the cache's or the output's values, so
 * one plan serves every layer of a decode step.
 *   q, kv_cache, block_table, seqlens, max_seqlen, causal: as the attention
 *     calls it serves (only sizes and the two int32 tables are read)
 *   plan, plan_bytes: device buffer of at least mla_decode_plan_size() bytes,
 *     16-byte aligned, caller-owned; written on `stream`
 * Nothing is launched when the call would not split (mla_decode_plan_size
 * gives 0; the planned calls then ignore the plan). Errors: as
 * mla_decode_attend; MLA_ERR_WORKSPACE for a missing or short plan buffer.
 *
 * mla_decode_attend_planned, mla_decode_attend_v_up_planned -- the calls
 * above reading a plan from mla_decode_plan instead of planning. Results are
 * bit-identical to the unplanned calls. The plan must come from mla_decode_plan
 * with the same sizes and with block_table and seqlens unchanged since; a plan
 * made for other sizes (its header says which) is ignored and the call plans
 * itself. A plan for other table contents gives unspecified rows (the plan's
 * indices stay within the sizes its header names). plan may be NULL (the
 * unplanned call). Only bf16 and f32 caches take a plan.
 */
int mla_decode_plan_size(int64_t batch, int64_t q_len, int64_t n_heads, int64_t kv_rank,
                         int64_t max_seqlen, int64_t page, int32_t dtype, size_t* bytes);
int mla_decode_plan(const mla_tensor* q, const mla_tensor* kv_cache, const mla_tensor* block_table,
                    const mla_tensor* seqlens, int64_t max_seqlen, int32_t causal, void* plan,
                    size_t plan_bytes, mla_stream stream);
int mla_decode_attend_planned(const mla_tensor* q, const mla_tensor* kv_cache,
                              const mla_tensor* block_table, const mla_tensor* seqlens,
                              int64_t max_seqlen, float softmax_scale, int32_t causal,
                              const mla_tensor* out, const mla_tensor* lse, void* workspace,
                              size_t workspace_bytes, const void* plan, size_t plan_bytes,
                              mla_stream stream);
int mla_decode_attend_v_up_planned(const mla_tensor* q, const mla_tensor* kv_cache,
                                   const mla_tensor* block_table, const mla_tensor* seqlens,
                                   int64_t max_seqlen, float softmax_scale, int32_t causal,
                                   const mla_tensor* w_uv, const mla_tensor* o_lat,
                                   const mla_tensor* out, const mla_tensor* lse, void* workspace,
                                   size_t workspace_bytes, const void* plan, size_t plan_bytes,
                                   mla_stream stream);

/*
 * mla_v_up -- un-project the latent attention output through W_UV ([P1] the
 * `_v_up_proj` bmm writing into a transposed [B, N, V] view; [P2]
 * `mla_decompress_v`).
 *
 *   out[t, h, :] = sum_l o_lat[t, h, l] * w_uv[h, l, :]
 *
 *   o_lat  [T, N, L]  bf16 or f32, any strides (inner 1)
 *   w_uv   [N, L, V]  same dtype, any strides (inner 1)
 *   out    [T, N, V]  same dtype, any strides (inner 1)
 * T may be 0.
 */
int mla_v_up(const mla_tensor* o_lat, const mla_tensor* w_uv, const mla_tensor* out,
             mla_stream stream);

/*
 * Naive (decompressed) prefill -- for long prompts, per-head keys and values
 * are rebuilt from the latent rows and attended with standard multi-head
 * attention, which costs 2 (d_nope + d_rope + d_v) flops per (query, key,
 * head) against 2 (2 kv_rank + d_rope) for the absorbed form.
 *
 * mla_decompress_kv -- the keys and values of every head (memra-engine 0.124.1
 * "tests/mla_gpu_forward.rs", the naive oracle mla_attend_naive, which
 * decompresses K and V per head; vllm.cpp "tests/vt/test_ops_mla_absorb.cpp",
 * "ConcatMlaNopeRope broadcasts the single k_pe head across every head": the
 * key of head h is [its k_nope | the token's one k_pe row]).
 *
 *   k_out[s, h, 0:P]   = sum_l kv_c[s, l] * w_uk_t[h, p, l]
 *   k_out[s, h, P:P+R] = k_pe[s, :]            (bit copy, the same for every head)
 *   v_out[s, h, :]     = sum_l kv_c[s, l] * w_uv[h, l, :]
 *
 *   kv_c   [S, L]       bf16 or f32, any strides (inner 1)
 *   k_pe   [S, R]       same dtype, or NULL (R = 0, NoPE)
 *   w_uk_t [N, P, L]    same dtype (the W_UK_T of mla_absorb_q)
 *   w_uv   [N, L, V]    same dtype (the W_UV of mla_v_up)
 *   k_out  [S, N, P+R]  same dtype, any strides (inner 1)
 *   v_out  [S, N, V]    same dtype, any strides (inner 1)
 * Products accumulate in f32 and round once (RNE) to the output dtype. S may
 * be 0. Two launches on `stream` (keys, then values); errors as everywhere:
 * nothing is launched when a check fails.
 */
int mla_decompress_kv(const mla_tensor* kv_c, const mla_tensor* k_pe, const mla_tensor* w_uk_t,
                      const mla_tensor* w_uv, const mla_tensor* k_out, const mla_tensor* v_out,
                      mla_stream stream);

/*
 * mla_prefill_attend -- causal (or full) multi-head attention of packed
 * sequences over their own per-head keys and values (memra-engine 0.124.1
 * gate 1, gpu_mla_prefill_parity_vs_cpu_oracle: the naive oracle's attention
 * after decompression; queries are the suffix of their sequence's keys, as in
 * the gate's chunked shape).
 *
 * Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and key
 * rows cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1. With lq queries and lk keys,
 * its query i sits at position lk - lq + i and, when causal, sees keys
 * 0 .. lk - lq + i; otherwise all lk keys.
 *   s_j          = softmax_scale * sum_e q[t, h, e] * k[j, h, e]
 *   out[t, h, :] = sum_j softmax(s)_j * v[j, h, :]
 *   lse[t, h]    = natural log of sum_j exp(s_j)
 * A query with no visible key gets out = 0 and lse = -inf.
 *
 *   q      [T, N, DK]  MLA_BF16, any strides (inner 1), rows 16-byte aligned
 *   k      [S, N, DK]  MLA_BF16, as q
 *   v      [S, N, DV]  MLA_BF16, as q
 *   cu_seqlens_q, cu_seqlens_k  [B + 1] MLA_I32 on the device, non-decreasing,
 *          within [0, T] and [0, S] (values outside are clamped to them)
 *   max_seqlen_q  host bound on every lq; query rows past it are not written
 *   out    [T, N, DV]  MLA_BF16, rows 8-byte aligned; rows no sequence owns
 *          are not written
 *   lse    [T, N]      MLA_F32, or NULL
 * Supported (DK, DV): (192, 128) (d_nope 128 + d_rope 64, V2-Lite/V3 heads),
 * (256, 256) (NoPE, d_nope 256), (128, 128), (64, 64); bf16 with f32
 * accumulation; otherwise MLA_ERR_UNSUPPORTED.
 */
int mla_prefill_attend(const mla_tensor* q, const mla_tensor* k, const mla_tensor* v,
                       const mla_tensor* cu_seqlens_q, const mla_tensor* cu_seqlens_k,
                       int64_t max_seqlen_q, float softmax_scale, int32_t causal,
                       const mla_tensor* out, const mla_tensor* lse, mla_stream stream);

/*
 * mla_sparse_decode_fp8 -- sparse absorbed decode over an fp8 cache of
 * 656-byte entries (vLLM "tests/kernels/attention/
 * test_mla_cross_layer_kernel_equivalence.py",
 * test_flashmla_fp8_sparse_decode_unified_slot_view: the DeepSeek V3.2 DSA
 * decode with per-token top-k slot indices padded with -1). An entry holds
 *   bytes   0..511  512 e4m3fn codes of c_kv,
 *   bytes 512..527  4 f32 scales, scale j for codes 128 j .. 128 j + 127,
 *   bytes 528..655  64 bf16 rope values;
 * latent value i is e4m3(code_i) * scale[i / 128]. Query token (b, i) attends
 * over the rows at the slots indices[b, i, :] (slot = block * PG + offset):
 *   s_j      = softmax_scale * sum_e q[b, i, h, e] * row_j[e]   (e < 576)
 *   out[...] = sum_j softmax(s)_j * row_j[0:512]
 *   lse      = natural log of sum_j exp(s_j)
 * Slots < 0 or >= NB * PG are no key; a slot listed twice is two keys; a
 * token with no key gets out = 0 and lse = -inf. No causal rule applies: the
 * list is the visibility.
 *
 *   q         [B, Sq, N, 576]  MLA_BF16, any strides (inner 1), rows 16-byte aligned
 *   kv_cache  [NB, PG, 656]    MLA_FP8_E4M3 (bytes; strides in bytes), entries
 *                              16-byte aligned; block-major views allowed
 *   indices   [B, Sq, topk]    MLA_I32, any strides (inner 1), topk <= 4096
 *   out       [B, Sq, N, 512]  MLA_BF16, rows 8-byte aligned
 *   lse       [B, Sq, N]       MLA_F32, or NULL
 *   workspace  device buffer of at least mla_sparse_workspace_size(B * Sq, N,
 *              topk) bytes (NULL allowed when that is 0), else MLA_ERR_WORKSPACE
 * Each dequantized value is rounded once to bf16 before the bf16 MFMA
 * products (f32 accumulation). Outputs for a block-major view equal those of a
 * contiguous copy bit for bit, and reruns are bit-identical (the split plan
 * depends only on the sizes; splits merge in order).
 */
int mla_sparse_decode_fp8(const mla_tensor* q, const mla_tensor* kv_cache,
                          const mla_tensor* indices, float softmax_scale, const mla_tensor* out,
                          const mla_tensor* lse, void* workspace, size_t workspace_bytes,
                          mla_stream stream);

/*
 * mla_sparse_workspace_size -- bytes of device workspace mla_sparse_decode_fp8
 * needs for `tokens` = B * Sq query tokens of n_heads heads and top-k lists
 * (0 when the call runs unsplit; then workspace may be NULL). When the tokens
 * and head groups alone would leave the chip idle, each slot list is split
 * over several workgroups, whose partial rows (normalised, rounded to bf16)
 * and f32 lse the workspace holds until the merge. Caller-owned, 16-byte aligned, needs no initialisation,
 * carries nothing between calls.
 */
int mla_sparse_workspace_size(int64_t tokens, int64_t n_heads, int64_t topk, size_t* bytes);

/* Human-readable name of a status code (static storage; never NULL). */
const char* mla_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
