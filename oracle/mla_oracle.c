/*
 * mla_oracle.c -- plain, slow CPU oracle for multi-head latent attention (MLA)
 * in weight-absorbed form, computed in double precision.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may load, call or link
 * this code: only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no code, header, table or helper with the HIP
 * library; the two meet only through seeded inputs generated elsewhere.
 *
 * Pages this oracle is written from (cited by title and section):
 *   [P1] vllm.cpp, "tests/vt/test_ops_mla_absorb.cpp": unit tests of the
 *        batched matmul and nope/rope concat primitives that weight absorption
 *        is built from (its double-precision bmm reference, the q concat tests).
 *   [P2] memra-engine 0.124.1, "tests/mla_gpu_forward.rs": GPU MLA core checked
 *        against CPU naive and absorbed oracles (gate 1 prefill parity, gate 2
 *        stepwise decode parity, the `Case` input bundle and its cache rows).
 *   [P3] vLLM, "tests/kernels/attention/test_mla_cross_layer_kernel_equivalence.py":
 *        latent-cache write (test_concat_and_cache_mla_into_unified_slot_view)
 *        and paged decode (test_flashmla_dense_decode_unified_slot_view,
 *        test_flashattn_mla_dense_decode_unified_slot_view).
 *
 * Notation (the pages' own): n_head heads, d_nope (P) and d_rope (R) query
 * widths, kv_rank (L) latent width, d_v (V) value width, entry = L + R.
 * A latent cache row is [c_kv (L) | k_pe (R)] ([P2] Case::cache_rows).
 * W_UK_T is [n_head, d_nope, kv_rank] and W_UV is [n_head, kv_rank, d_v] ([P1]
 * header comment on the V2-Lite shapes).
 *
 * Readings of points the pages leave open:
 *   - query i of t_q sits at absolute position t_kv - t_q + i (queries are a
 *     suffix of the cache, [P2] gate 1 "chunked" shape and gate 2); causal means
 *     it sees keys 0..pos, otherwise all t_kv keys.
 *   - a query with no visible key returns o = 0 and lse = -inf.
 *   - lse is the natural log of the sum of exp over the SCALED scores.
 *   - interleaved rope ([P2] gate 3) rotates the pairs (2i, 2i+1) of a vector
 *     by theta_i = position * base^(-2i/d), the standard rotary frequencies;
 *     the page names the rotation but does not print its body.
 *
 * All floating arrays are double, dense, row-major unless a stride is passed;
 * strides are in elements. Nothing here is blocked, fused or reordered beyond
 * the definitions; the only parallelism is an OpenMP loop over independent
 * output rows, which does not change any row's arithmetic.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int mla_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the following calls (the benchmark also times one thread). */
void mla_oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---------------------------------------------------------------------------
 * Batched matmul, straight from the definition of torch.bmm that [P1]'s
 * double-precision reference (RefBmm) checks against:
 *     out[g, m, n] = sum_k a[g, m, k] * b[g, k, n]
 * with every operand addressed through explicit strides, so transposed views
 * (the layouts both upstream call sites pass, [P1] "handles the TRANSPOSED
 * views") are evaluated in exactly the layout given. Sum runs k = 0..K-1.
 * ------------------------------------------------------------------------- */
void mla_oracle_bmm(int64_t G, int64_t M, int64_t K, int64_t N,
                    const double* a, int64_t as0, int64_t as1, int64_t as2,
                    const double* b, int64_t bs0, int64_t bs1, int64_t bs2,
                    double* out, int64_t os0, int64_t os1, int64_t os2) {
  int64_t gm;
#pragma omp parallel for schedule(static)
  for (gm = 0; gm < G * M; ++gm) {
    const int64_t g = gm / M, m = gm % M;
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += a[g * as0 + m * as1 + k * as2] * b[g * bs0 + k * bs1 + n * bs2];
      out[g * os0 + m * os1 + n * os2] = acc;
    }
  }
}

/* ---------------------------------------------------------------------------
 * One query row of absorbed attention against a contiguous run of latent rows.
 *   qrow  [entry]            folded query: q_lat (L) then q_pe (R)
 *   kv    [t_kv, entry]      latent rows [c_kv | k_pe]
 *   nvis                     keys 0..nvis-1 are visible
 * score_j = scale * sum_{e<entry} qrow[e] * kv[j][e]
 *   (the q_lat part meets c_kv, the q_pe part meets k_pe: [P3]
 *    test_flashattn_mla_dense_decode_unified_slot_view splits it exactly so)
 * p_j = exp(score_j - lse),  lse = log(sum_j exp(score_j))
 * o[0:L] = sum_j p_j * kv[j][0:L]   (the value of a key IS its c_kv: [P3]
 *   decode tests pass head_dim_v = kv_rank = 512 over the 576-wide cache)
 * `probs`, when given, receives p_j for j < nvis and 0 beyond.
 * ------------------------------------------------------------------------- */
static void attend_row(int64_t L, int64_t entry, int64_t t_kv, const double* qrow,
                       const double* kv, int64_t nvis, double scale, double* o,
                       double* lse_out, double* probs) {
  for (int64_t l = 0; l < L; ++l) o[l] = 0.0;
  if (probs)
    for (int64_t j = 0; j < t_kv; ++j) probs[j] = 0.0;
  if (nvis <= 0) {
    *lse_out = -INFINITY;
    return;
  }
  double* s = (double*)malloc((size_t)nvis * sizeof(double));
  double mx = -INFINITY;
  for (int64_t j = 0; j < nvis; ++j) {
    double acc = 0.0;
    for (int64_t e = 0; e < entry; ++e) acc += qrow[e] * kv[j * entry + e];
    s[j] = scale * acc;
    if (s[j] > mx) mx = s[j];
  }
  double sum = 0.0;
  for (int64_t j = 0; j < nvis; ++j) sum += exp(s[j] - mx);
  const double lse = mx + log(sum);
  for (int64_t j = 0; j < nvis; ++j) {
    const double p = exp(s[j] - lse);
    if (probs) probs[j] = p;
    for (int64_t l = 0; l < L; ++l) o[l] += p * kv[j * entry + l];
  }
  *lse_out = lse;
  free(s);
}

static int64_t visible_keys(int64_t pos, int64_t t_kv, int causal) {
  if (!causal) return t_kv;
  int64_t n = pos + 1;
  if (n < 0) n = 0;
  if (n > t_kv) n = t_kv;
  return n;
}

/* ---------------------------------------------------------------------------
 * Absorbed attention for nq query rows of one sequence ([P2] the absorbed
 * oracle `mla_attend_absorbed` and the kernel it gates, `mla_attn_absorbed`).
 *   q     [nq, n_head, entry]   entry = L + R
 *   pos   [nq]                  absolute position of each query row
 *   kv    [t_kv, entry]
 *   o_lat [nq, n_head, L]       lse [nq, n_head]   probs [nq, n_head, t_kv] or NULL
 * ------------------------------------------------------------------------- */
void mla_oracle_attend_seq(int64_t nq, int64_t n_head, int64_t L, int64_t R, int64_t t_kv,
                           const double* q, const int64_t* pos, const double* kv,
                           double scale, int causal, double* o_lat, double* lse,
                           double* probs) {
  const int64_t entry = L + R;
  int64_t r;
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < nq * n_head; ++r) {
    const int64_t i = r / n_head;
    attend_row(L, entry, t_kv, q + r * entry, kv, visible_keys(pos[i], t_kv, causal), scale,
               o_lat + r * L, lse + r, probs ? probs + r * t_kv : NULL);
  }
}

/* ---------------------------------------------------------------------------
 * Paged gather ([P3] paged decode: logical page i of sequence b lives in
 * physical block block_table[b][i]; a slot is block * page + offset).
 * Builds the contiguous latent rows 0..seqlen-1 of sequence b:
 *     rows[j] = pool[block_table[b][j / page]][j % page]
 *   pool        [num_blocks, page, entry]
 *   block_table [batch, max_blocks] (row b at block_table + b * max_blocks)
 * Returns 0, or -1 if a needed block id is outside [0, num_blocks) or the
 * sequence needs more than max_blocks pages.
 * ------------------------------------------------------------------------- */
int mla_oracle_gather_pages(int64_t entry, const double* pool, int64_t num_blocks,
                            int64_t page, const int32_t* block_table, int64_t max_blocks,
                            int64_t b, int64_t seqlen, double* rows) {
  for (int64_t j = 0; j < seqlen; ++j) {
    const int64_t i = j / page;
    if (i >= max_blocks) return -1;
    const int64_t blk = block_table[b * max_blocks + i];
    if (blk < 0 || blk >= num_blocks) return -1;
    memcpy(rows + j * entry, pool + (blk * page + j % page) * entry,
           (size_t)entry * sizeof(double));
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Batched paged decode/prefill attention in absorbed form ([P3]
 * test_flashmla_dense_decode_unified_slot_view: q [batch, t_q, n_head, 576],
 * a paged latent cache, block_table, cache_seqlens, head_dim_v = kv_rank,
 * returning (out, lse)). Sequence b's rows are gathered by the routine above,
 * then each query i sits at pos = seqlen_b - t_q + i.
 *   q     [batch, t_q, n_head, entry]     o_lat [batch, t_q, n_head, L]
 *   lse   [batch, t_q, n_head]
 * Returns 0, or -1 on a bad block id.
 * ------------------------------------------------------------------------- */
int mla_oracle_attend_paged(int64_t batch, int64_t t_q, int64_t n_head, int64_t L, int64_t R,
                            const double* q, const double* pool, int64_t num_blocks,
                            int64_t page, const int32_t* block_table, int64_t max_blocks,
                            const int32_t* seqlens, double scale, int causal, double* o_lat,
                            double* lse) {
  const int64_t entry = L + R;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t s = seqlens[b] > 0 ? seqlens[b] : 0;
    double* rows = (double*)malloc((size_t)(s > 0 ? s : 1) * entry * sizeof(double));
    if (mla_oracle_gather_pages(entry, pool, num_blocks, page, block_table, max_blocks, b, s,
                                rows) != 0) {
      free(rows);
      return -1;
    }
    int64_t* pos = (int64_t*)malloc((size_t)t_q * sizeof(int64_t));
    for (int64_t i = 0; i < t_q; ++i) pos[i] = s - t_q + i;
    mla_oracle_attend_seq(t_q, n_head, L, R, s, q + b * t_q * n_head * entry, pos, rows,
                          scale, causal, o_lat + b * t_q * n_head * L, lse + b * t_q * n_head,
                          NULL);
    free(pos);
    free(rows);
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Naive MLA ([P2] `mla_attend_naive`): decompress K and V per head from the
 * latent rows, then ordinary softmax attention per head.
 *   k_nope[j, h, p] = sum_l W_UK_T[h, p, l] * c_kv[j, l]
 *   v[j, h, d]      = sum_l W_UV[h, l, d]   * c_kv[j, l]
 *   score_j = scale * (sum_p q_nope[i,h,p] k_nope[j,h,p] + sum_r q_pe[i,h,r] k_pe[j,r])
 *   out[i, h, :] = sum_j softmax(score)_j * v[j, h, :]
 * k_pe is one row per token shared by every head ([P1] broadcast concat test).
 *   q_nope [nq, n_head, P]   q_pe [nq, n_head, R]   c_kv [t_kv, L]   k_pe [t_kv, R]
 *   w_uk_t [n_head, P, L]    w_uv [n_head, L, V]    out [nq, n_head, V]
 * ------------------------------------------------------------------------- */
void mla_oracle_naive(int64_t nq, int64_t n_head, int64_t P, int64_t R, int64_t V, int64_t L,
                      int64_t t_kv, const double* q_nope, const double* q_pe, const double* c_kv,
                      const double* k_pe, const double* w_uk_t, const double* w_uv,
                      const int64_t* pos, double scale, int causal, double* out) {
  /* decompressed keys and values, [t_kv, n_head, P] and [t_kv, n_head, V] */
  double* k_nope = (double*)malloc((size_t)(t_kv > 0 ? t_kv : 1) * n_head * P * sizeof(double));
  double* v = (double*)malloc((size_t)(t_kv > 0 ? t_kv : 1) * n_head * V * sizeof(double));
  int64_t jh;
#pragma omp parallel for schedule(static)
  for (jh = 0; jh < t_kv * n_head; ++jh) {
    const int64_t j = jh / n_head, h = jh % n_head;
    for (int64_t p = 0; p < P; ++p) {
      double acc = 0.0;
      for (int64_t l = 0; l < L; ++l) acc += w_uk_t[(h * P + p) * L + l] * c_kv[j * L + l];
      k_nope[jh * P + p] = acc;
    }
    for (int64_t d = 0; d < V; ++d) {
      double acc = 0.0;
      for (int64_t l = 0; l < L; ++l) acc += w_uv[(h * L + l) * V + d] * c_kv[j * L + l];
      v[jh * V + d] = acc;
    }
  }
  int64_t r;
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < nq * n_head; ++r) {
    const int64_t i = r / n_head, h = r % n_head;
    const int64_t nvis = visible_keys(pos[i], t_kv, causal);
    double* o = out + r * V;
    for (int64_t d = 0; d < V; ++d) o[d] = 0.0;
    if (nvis <= 0) continue;
    double* s = (double*)malloc((size_t)nvis * sizeof(double));
    double mx = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j) {
      double acc = 0.0;
      for (int64_t p = 0; p < P; ++p) acc += q_nope[r * P + p] * k_nope[(j * n_head + h) * P + p];
      for (int64_t e = 0; e < R; ++e) acc += q_pe[r * R + e] * k_pe[j * R + e];
      s[j] = scale * acc;
      if (s[j] > mx) mx = s[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j < nvis; ++j) sum += exp(s[j] - mx);
    for (int64_t j = 0; j < nvis; ++j) {
      const double pj = exp(s[j] - mx) / sum;
      for (int64_t d = 0; d < V; ++d) o[d] += pj * v[(j * n_head + h) * V + d];
    }
    free(s);
  }
  free(k_nope);
  free(v);
}

/* ---------------------------------------------------------------------------
 * Absorbed MLA end to end ([P2] `mla_attend_absorbed`; the three kernels its
 * gates drive in order: absorb q, absorbed attention, decompress v; [P1]
 * header: the q-side W_UK fold and the W_UV un-projection as bmm calls).
 *   q_lat[i, h, :] = sum_p q_nope[i, h, p] * W_UK_T[h, p, :]         (bmm)
 *   q[i, h, :]     = [q_lat | q_pe]                                  (concat)
 *   o_lat          = absorbed attention over [c_kv | k_pe] rows      (above)
 *   out[i, h, :]   = sum_l o_lat[i, h, l] * W_UV[h, l, :]            (bmm)
 * Shapes as for mla_oracle_naive. q_lat_out / o_lat_out / lse_out may be NULL;
 * when given they receive the stage outputs [nq, n_head, L] / [nq, n_head].
 * ------------------------------------------------------------------------- */
void mla_oracle_absorbed(int64_t nq, int64_t n_head, int64_t P, int64_t R, int64_t V, int64_t L,
                         int64_t t_kv, const double* q_nope, const double* q_pe,
                         const double* c_kv, const double* k_pe, const double* w_uk_t,
                         const double* w_uv, const int64_t* pos, double scale, int causal,
                         double* out, double* q_lat_out, double* o_lat_out, double* lse_out) {
  const int64_t entry = L + R;
  const size_t rows = (size_t)(nq > 0 ? nq : 1) * (size_t)n_head;
  double* q_lat = (double*)malloc(rows * L * sizeof(double));
  /* fold: batch over heads, a[h, i, p] = q_nope[i, h, p] (a transposed view) */
  mla_oracle_bmm(n_head, nq, P, L, q_nope, P, n_head * P, 1, w_uk_t, P * L, L, 1, q_lat, L,
                 n_head * L, 1);
  double* q = (double*)malloc(rows * entry * sizeof(double));
  for (int64_t r = 0; r < nq * n_head; ++r) {
    for (int64_t l = 0; l < L; ++l) q[r * entry + l] = q_lat[r * L + l];
    for (int64_t e = 0; e < R; ++e) q[r * entry + L + e] = q_pe[r * R + e];
  }
  double* kv = (double*)malloc((size_t)(t_kv > 0 ? t_kv : 1) * entry * sizeof(double));
  for (int64_t j = 0; j < t_kv; ++j) {
    for (int64_t l = 0; l < L; ++l) kv[j * entry + l] = c_kv[j * L + l];
    for (int64_t e = 0; e < R; ++e) kv[j * entry + L + e] = k_pe[j * R + e];
  }
  double* o_lat = (double*)malloc(rows * L * sizeof(double));
  double* lse = (double*)malloc(rows * sizeof(double));
  mla_oracle_attend_seq(nq, n_head, L, R, t_kv, q, pos, kv, scale, causal, o_lat, lse, NULL);
  /* un-projection: a[h, i, l] = o_lat[i, h, l], out[i, h, d] written through a view */
  mla_oracle_bmm(n_head, nq, L, V, o_lat, L, n_head * L, 1, w_uv, L * V, V, 1, out, V,
                 n_head * V, 1);
  if (q_lat_out) memcpy(q_lat_out, q_lat, (size_t)nq * n_head * L * sizeof(double));
  if (o_lat_out) memcpy(o_lat_out, o_lat, (size_t)nq * n_head * L * sizeof(double));
  if (lse_out) memcpy(lse_out, lse, (size_t)nq * n_head * sizeof(double));
  free(q_lat);
  free(q);
  free(kv);
  free(o_lat);
  free(lse);
}

/* ---------------------------------------------------------------------------
 * Split-KV attention with a log-sum-exp merge, in double. [P3] decode returns
 * (out, lse) and is driven by a split plan (tile_scheduler_metadata,
 * num_splits); the merge itself is not printed on the pages, so this follows
 * the plain identity it rests on:
 *   for split s over keys [bounds[s], bounds[s+1]) intersected with the visible
 *   range: lse_s = log sum exp(score), o_s = sum p_j kv_j with p_j = exp(score_j - lse_s)
 *   lse = log sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) * o_s
 * Splits with no visible key have lse_s = -inf and contribute nothing.
 *   bounds [nsplit + 1], 0 = bounds[0] <= ... <= bounds[nsplit] = t_kv
 * Shapes as for mla_oracle_attend_seq.
 * ------------------------------------------------------------------------- */
void mla_oracle_attend_split(int64_t nq, int64_t n_head, int64_t L, int64_t R, int64_t t_kv,
                             const double* q, const int64_t* pos, const double* kv,
                             double scale, int causal, const int64_t* bounds, int64_t nsplit,
                             double* o_lat, double* lse) {
  const int64_t entry = L + R;
  int64_t r;
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < nq * n_head; ++r) {
    const int64_t i = r / n_head;
    const int64_t nvis = visible_keys(pos[i], t_kv, causal);
    double* part_o = (double*)malloc((size_t)nsplit * L * sizeof(double));
    double* part_lse = (double*)malloc((size_t)nsplit * sizeof(double));
    for (int64_t s = 0; s < nsplit; ++s) {
      int64_t lo = bounds[s], hi = bounds[s + 1];
      if (hi > nvis) hi = nvis;
      const int64_t n = hi > lo ? hi - lo : 0;
      attend_row(L, entry, n, q + r * entry, kv + lo * entry, n, scale, part_o + s * L,
                 part_lse + s, NULL);
    }
    double mx = -INFINITY;
    for (int64_t s = 0; s < nsplit; ++s)
      if (part_lse[s] > mx) mx = part_lse[s];
    double* o = o_lat + r * L;
    for (int64_t l = 0; l < L; ++l) o[l] = 0.0;
    if (mx == -INFINITY) {
      lse[r] = -INFINITY;
    } else {
      double sum = 0.0;
      for (int64_t s = 0; s < nsplit; ++s) sum += exp(part_lse[s] - mx);
      const double tot = mx + log(sum);
      for (int64_t s = 0; s < nsplit; ++s) {
        const double w = exp(part_lse[s] - tot);
        for (int64_t l = 0; l < L; ++l) o[l] += w * part_o[s * L + l];
      }
      lse[r] = tot;
    }
    free(part_o);
    free(part_lse);
  }
}

/* ---------------------------------------------------------------------------
 * Latent cache write ([P3] test_concat_and_cache_mla_into_unified_slot_view;
 * [P2] gate 2 append, whose rows are checked bit for bit). A pure copy, done
 * on raw element bytes so every bit (NaN payloads, -0.0) is carried over:
 * for each token t whose slot lies in [0, num_blocks * page):
 *     blk = slot / page, off = slot % page
 *     buf[offset + blk*s0 + off*s1 + d] = kv_c[t][d]      for d <  L
 *                                       = k_pe[t][d - L]  for L <= d < L + R
 * Tokens with a slot outside that range are skipped (reading: a negative slot
 * marks a padded token). Everything else in `buf` is left as it was, which is
 * what the zero-bleed check of [P3] asserts for the neighbouring layers.
 *   esize     bytes per element (2 for bf16, 4 for f32)
 *   kv_c      token t's row at kv_c + t * kv_c_stride elements
 *   k_pe      token t's row at k_pe + t * k_pe_stride elements (unused if R == 0)
 *   slots     [T] int64
 *   buf       the whole allocation the cache view lives in, buf_elems elements
 *   offset, s0, s1   the view's storage offset and block / row strides
 * Returns 0, or -1 if a written element would fall outside buf.
 * ------------------------------------------------------------------------- */
int mla_oracle_cache_write(int64_t T, int64_t L, int64_t R, int64_t esize, const uint8_t* kv_c,
                           int64_t kv_c_stride, const uint8_t* k_pe, int64_t k_pe_stride,
                           const int64_t* slots, uint8_t* buf, int64_t buf_elems,
                           int64_t offset, int64_t num_blocks, int64_t page, int64_t s0,
                           int64_t s1) {
  for (int64_t t = 0; t < T; ++t) {
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_blocks * page) continue;
    const int64_t blk = slot / page, off = slot % page;
    for (int64_t d = 0; d < L + R; ++d) {
      const int64_t dst = offset + blk * s0 + off * s1 + d;
      if (dst < 0 || dst >= buf_elems) return -1;
      const uint8_t* src = d < L ? kv_c + (t * kv_c_stride + d) * esize
                                 : k_pe + (t * k_pe_stride + (d - L)) * esize;
      memcpy(buf + dst * esize, src, (size_t)esize);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Interleaved rotary position embedding ([P2] "tests/mla_gpu_forward.rs",
 * gate 3, gpu_mla_rope_interleaved_matches_cpu: d_rope 8 and 64, base 8e6,
 * positions 13 * p, and d_rope == 0 is a no-op).
 *
 * Every vector x[t, v, 0:d] of token t is rotated in place, pair by pair: for
 * i < d / 2, with theta = positions[t] * base^(-2i / d),
 *   x[2i]   <- x[2i] cos(theta) - x[2i+1] sin(theta)
 *   x[2i+1] <- x[2i] sin(theta) + x[2i+1] cos(theta)
 *   x      [T, V, d] double, dense
 *   pos    [T] int32
 * ------------------------------------------------------------------------- */
void mla_oracle_rope_interleaved(int64_t T, int64_t V, int64_t d, double* x, const int32_t* pos,
                                 double base) {
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t v = 0; v < V; ++v) {
      double* row = x + (t * V + v) * d;
      for (int64_t i = 0; i < d / 2; ++i) {
        const double theta = (double)pos[t] * pow(base, -2.0 * (double)i / (double)d);
        const double c = cos(theta), s = sin(theta);
        const double a = row[2 * i], b = row[2 * i + 1];
        row[2 * i] = a * c - b * s;
        row[2 * i + 1] = a * s + b * c;
      }
    }
  }
}

/* ---------------------------------------------------------------------------
 * fp8 latent cache ([P3] test_flashmla_dense_fp8_decode_unified_slot_view and
 * test_flashinfer_mla_dense_fp8_decode_unified_slot_view: the cache holds
 * torch.float8_e4m3fn values; the dense fp8 decode takes descale_q and
 * descale_k; concat_and_cache_mla takes a cache dtype and a scale).
 *
 * The element format is OCP FP8 E4M3 ("fn": finite, no infinities): one sign
 * bit, four exponent bits with bias 7, three mantissa bits. Exponent field 0
 * holds the subnormals m * 2^-9; the all-ones pattern S.1111.111 is NaN; the
 * largest finite magnitude is 1.75 * 2^8 = 448.
 *
 * Readings of what the pages leave open:
 *   - the write stores e4m3(x / scale) for every element x of [kv_c | k_pe],
 *     the quotient taken in float (the precision the kernel decides the code
 *     in), rounded to the nearest e4m3 value with ties to the even mantissa;
 *     magnitudes above 448 (infinities included) saturate to +-448, NaN stays
 *     NaN, and the sign of a zero result is kept.
 *   - dense fp8 decode: the query's values are q * descale_q, the key and value
 *     rows e4m3 values times descale_k; everything else is the bf16 decode.
 * ------------------------------------------------------------------------- */
double mla_oracle_e4m3_decode(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double mag;
  if (e == 15 && m == 7) return sign ? -NAN : NAN;
  if (e == 0) mag = ldexp((double)m, -9);
  else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

void mla_oracle_e4m3_decode_array(int64_t n, const uint8_t* codes, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = mla_oracle_e4m3_decode(codes[i]);
}

/* Nearest e4m3 code to v by exhaustive search over the 127 non-negative finite
 * codes (ties: the even code, i.e. the even mantissa). */
uint8_t mla_oracle_e4m3_encode(float v) {
  if (isnan(v)) return signbit(v) ? 0xff : 0x7f;
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double best_err = a;
  for (int c = 1; c <= 0x7e; ++c) {
    const double err = fabs(mla_oracle_e4m3_decode((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

void mla_oracle_e4m3_encode_array(int64_t n, const float* v, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = mla_oracle_e4m3_encode(v[i]);
}

/* fp8 latent-cache write: token t's row [kv_c[t] | k_pe[t]] (float values, the
 * inputs' values converted exactly) goes to slot slots[t] of a byte cache view
 * (offset, block stride s0, row stride s1, in bytes), each element stored as
 * e4m3(x / scale). Slots outside [0, num_blocks * page) are skipped. Returns 0,
 * or -1 if a written byte would fall outside buf. */
int mla_oracle_cache_write_fp8(int64_t T, int64_t L, int64_t R, const float* kv_c,
                               const float* k_pe, const int64_t* slots, float scale, uint8_t* buf,
                               int64_t buf_bytes, int64_t offset, int64_t num_blocks, int64_t page,
                               int64_t s0, int64_t s1) {
  for (int64_t t = 0; t < T; ++t) {
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_blocks * page) continue;
    const int64_t blk = slot / page, off = slot % page;
    for (int64_t d = 0; d < L + R; ++d) {
      const int64_t dst = offset + blk * s0 + off * s1 + d;
      if (dst < 0 || dst >= buf_bytes) return -1;
      const float x = d < L ? kv_c[t * L + d] : k_pe[t * R + (d - L)];
      const float q = x / scale;
      buf[dst] = mla_oracle_e4m3_encode(q);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Naive (decompressed) prefill, first step: per-head keys and values rebuilt
 * from the latent rows ([P2] the naive oracle `mla_attend_naive`, which
 * decompresses K and V per head; [P1] ConcatMlaNopeRope, the broadcast case
 * "broadcasts the single k_pe head across every head": the key of head h is
 * [k_nope of head h | the token's one k_pe row]).
 *   k[j, h, 0:P]   = sum_l W_UK_T[h, p, l] * c_kv[j, l]
 *   k[j, h, P:P+R] = k_pe[j, 0:R]            (the same row for every head)
 *   v[j, h, :]     = sum_l c_kv[j, l] * W_UV[h, l, :]
 *   c_kv [t_kv, L]  k_pe [t_kv, R]  w_uk_t [n_head, P, L]  w_uv [n_head, L, V]
 *   k_out [t_kv, n_head, P + R]     v_out [t_kv, n_head, V]
 * ------------------------------------------------------------------------- */
void mla_oracle_decompress_kv(int64_t t_kv, int64_t n_head, int64_t P, int64_t R, int64_t V,
                              int64_t L, const double* c_kv, const double* k_pe,
                              const double* w_uk_t, const double* w_uv, double* k_out,
                              double* v_out) {
  const int64_t DK = P + R;
  int64_t jh;
#pragma omp parallel for schedule(static)
  for (jh = 0; jh < t_kv * n_head; ++jh) {
    const int64_t j = jh / n_head, h = jh % n_head;
    for (int64_t p = 0; p < P; ++p) {
      double acc = 0.0;
      for (int64_t l = 0; l < L; ++l) acc += w_uk_t[(h * P + p) * L + l] * c_kv[j * L + l];
      k_out[jh * DK + p] = acc;
    }
    for (int64_t e = 0; e < R; ++e) k_out[jh * DK + P + e] = k_pe[j * R + e];
    for (int64_t d = 0; d < V; ++d) {
      double acc = 0.0;
      for (int64_t l = 0; l < L; ++l) acc += c_kv[j * L + l] * w_uv[(h * L + l) * V + d];
      v_out[jh * V + d] = acc;
    }
  }
}

/* ---------------------------------------------------------------------------
 * Naive (decompressed) prefill, second step: standard multi-head softmax
 * attention of one sequence over its own per-head keys and values ([P2] the
 * naive oracle's attention after decompression; causal queries are a suffix
 * of the keys as in gate 1's chunked shape).
 *   s_j        = scale * sum_e q[i, h, e] * k[j, h, e]     over visible j
 *   out[i,h,:] = sum_j softmax(s)_j * v[j, h, :]
 *   lse[i,h]   = natural log of sum_j exp(s_j)  (-inf, and out = 0, with no key)
 *   q [nq, n_head, DK]   k [t_kv, n_head, DK]   v [t_kv, n_head, DV]
 *   pos [nq] absolute query positions   out [nq, n_head, DV]   lse [nq, n_head]
 * ------------------------------------------------------------------------- */
void mla_oracle_mha(int64_t nq, int64_t t_kv, int64_t n_head, int64_t DK, int64_t DV,
                    const double* q, const double* k, const double* v, const int64_t* pos,
                    double scale, int causal, double* out, double* lse) {
  int64_t r;
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < nq * n_head; ++r) {
    const int64_t i = r / n_head, h = r % n_head;
    const int64_t nvis = visible_keys(pos[i], t_kv, causal);
    double* o = out + r * DV;
    for (int64_t d = 0; d < DV; ++d) o[d] = 0.0;
    if (nvis <= 0) {
      lse[r] = -INFINITY;
      continue;
    }
    double* s = (double*)malloc((size_t)nvis * sizeof(double));
    double mx = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j) {
      double acc = 0.0;
      for (int64_t e = 0; e < DK; ++e) acc += q[r * DK + e] * k[(j * n_head + h) * DK + e];
      s[j] = scale * acc;
      if (s[j] > mx) mx = s[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j < nvis; ++j) sum += exp(s[j] - mx);
    const double l = mx + log(sum);
    for (int64_t j = 0; j < nvis; ++j) {
      const double pj = exp(s[j] - l);
      for (int64_t d = 0; d < DV; ++d) o[d] += pj * v[(j * n_head + h) * DV + d];
    }
    lse[r] = l;
    free(s);
  }
}

/* ---------------------------------------------------------------------------
 * Sparse fp8 decode entries ([P3] test_flashmla_fp8_sparse_decode_unified_slot_view,
 * the DeepSeek V3.2 DSA path): a latent row is stored as one 656-byte entry,
 *   bytes   0..511  512 e4m3fn codes of c_kv,
 *   bytes 512..527  4 f32 scales (little-endian), scale j for codes 128j..128j+127,
 *   bytes 528..655  64 bf16 values of k_pe (little-endian).
 * Reading (the page builds the payload but does not print the kernel): the
 * latent value of code i is e4m3(code_i) * scale[i / 128]; the rope part is
 * the bf16 values as stored. The row [c_kv (512) | k_pe (64)] then enters the
 * absorbed attention unchanged.
 *   entries [n, 656] bytes (row i at entries + i * stride)   rows [n, 576]
 * ------------------------------------------------------------------------- */
void mla_oracle_dsmla_rows(int64_t n, const uint8_t* entries, int64_t stride, double* rows) {
  for (int64_t i = 0; i < n; ++i) {
    const uint8_t* e = entries + i * stride;
    double* r = rows + i * 576;
    for (int j = 0; j < 4; ++j) {
      uint32_t bits = (uint32_t)e[512 + 4 * j] | ((uint32_t)e[513 + 4 * j] << 8) |
                      ((uint32_t)e[514 + 4 * j] << 16) | ((uint32_t)e[515 + 4 * j] << 24);
      float sc;
      memcpy(&sc, &bits, 4);
      for (int c = 0; c < 128; ++c) r[128 * j + c] = mla_oracle_e4m3_decode(e[128 * j + c]) * (double)sc;
    }
    for (int c = 0; c < 64; ++c) {
      const uint32_t bits = ((uint32_t)e[528 + 2 * c] | ((uint32_t)e[529 + 2 * c] << 8)) << 16;
      float v;
      memcpy(&v, &bits, 4);
      r[512 + c] = (double)v;
    }
  }
}
