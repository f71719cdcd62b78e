// prefill_kernels.h -- internal interface of the prefill-sized products, the
// naive (decompressed) prefill and the sparse fp8 decode, between the C-ABI
// layer (mla_abi.cpp) and their translation units; kept apart from
// mla_kernels.h so that the sources of the paged decode kernels stay
// unchanged when these kernels change.
#pragma once

#include "mla_kernels.h"

namespace mla {

// token counts from which the bf16 products use 128 x 128 pipelined tiles
constexpr int64_t kBigT = 256;

// ------------------------------------------------- naive (decompressed) prefill
// Key decompression, a batched product with both operands contiguous along k:
//   out[t, h, n]       = sum_k a[t, h, k] * w[h, n, k]
//   out[t, h, N + r]   = pe[t, r]   (one rope row per token, copied to every head)
struct BmmNtParams {
  const void* a;  int64_t a_st, a_sh;   // a[t, h, k] (h stride 0: one latent row per token)
  const void* w;  int64_t w_sh, w_sn;   // w[h, n, k]
  void* out;      int64_t o_st, o_sh;   // out[t, h, 0 : N + R]
  const void* pe; int64_t pe_st;        // pe[t, r] (NULL when R == 0)
  int64_t T, H, K, N, R;
  int is_f32;
};
hipError_t launch_bmm_nt(const BmmNtParams& p, hipStream_t s);

// Multi-head attention over per-head keys and values of packed sequences:
// sequence b owns query rows cu_q[b] .. cu_q[b+1] and key rows cu_k[b] ..
// cu_k[b+1]; its queries are the suffix of its keys (causal: query i of a
// sequence with lq queries and lk keys sees keys 0 .. lk - lq + i).
struct MhaParams {
  const void* q; int64_t q_s0, q_s1;    // [T, N, DK] bf16
  const void* k; int64_t k_s0, k_s1;    // [S, N, DK] bf16
  const void* v; int64_t v_s0, v_s1;    // [S, N, DV] bf16
  void* out;     int64_t o_s0, o_s1;    // [T, N, DV] bf16
  float* lse;    int64_t l_s0, l_s1;    // [T, N] natural log, or NULL
  const int32_t* cu_q; const int32_t* cu_k;  // [B + 1] each
  int64_t T, S;                         // rows of q and of k / v (bounds for cu_q, cu_k)
  int n_heads, batch, max_q;
  int dk, dv;
  int causal;
  float scale_log2;                     // softmax scale * log2(e)
  int pair_tiles;                       // set by launch_mha: a workgroup takes two query tiles
};
hipError_t launch_mha(const MhaParams& p, hipStream_t s);
bool mha_supported(int dk, int dv);

// ------------------------------------------------------ sparse fp8 decode
// Query token (b, i) attends over the latent rows at the slots idx[b, i, :]
// of a cache of 656-byte entries (512 e4m3 codes, 4 f32 scales, 64 bf16 rope
// values); slots < 0 or >= num_slots are no key.
constexpr int kSparseMaxTopk = 4096;  // slot list held in LDS
struct SparseParams {
  const void* q;     int64_t q_s0, q_s1, q_s2;   // [B, Sq, N, 576] bf16
  const uint8_t* kv; int64_t kv_s0, kv_s1;       // [NB, PG, 656] bytes (strides in bytes)
  int64_t num_slots; int page;                   // NB * PG, PG
  int page_shift;                                // log2(PG) when PG is a power of two, else -1
  const int32_t* idx; int64_t i_s0, i_s1;        // [B, Sq, topk]
  int topk;
  void* out;         int64_t o_s0, o_s1, o_s2;   // [B, Sq, N, 512] bf16
  float* lse;        int64_t l_s0, l_s1, l_s2;   // [B, Sq, N] or NULL
  int batch, q_len, n_heads;
  float scale_log2;                              // softmax scale * log2(e)
  // split of each slot list over nsplit workgroups of split_len entries (a
  // multiple of 32); with nsplit > 1 each writes its normalised partial
  // output, rounded to bf16, as rows of 512 in the first half of part_o
  // ([token][split][N] rows; the region is sized for f32) and part_lse
  // [token][split][N] (natural log), and a merge kernel combines them
  int split_len, nsplit;
  float* part_o;
  float* part_lse;
};
// split plan for a call; returns the workspace bytes it needs
size_t plan_sparse(int64_t tokens, int64_t n_heads, int64_t topk, int* split_len, int* nsplit);
hipError_t launch_sparse(const SparseParams& p, hipStream_t s);

}  // namespace mla
