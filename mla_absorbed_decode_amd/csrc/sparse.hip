// sparse.hip -- sparse absorbed decode over an fp8 latent cache of 656-byte
// entries, each query token attending over its own list of slots (vLLM
// "tests/kernels/attention/test_mla_cross_layer_kernel_equivalence.py",
// test_flashmla_fp8_sparse_decode_unified_slot_view: the DeepSeek V3.2 DSA
// decode reads 128 heads x 576 against top-k slot lists padded with -1).
//
// Entry layout (bytes): 0..511 e4m3fn codes of c_kv, 512..527 four f32
// scales (scale j for codes 128 j .. 128 j + 127), 528..655 64 bf16 rope
// values. Latent value i = e4m3(code_i) * scale[i / 128].
//
// One workgroup per (query token, 64 heads, part of the slot list): eight
// waves, each 16 heads x 256 of the 512 output columns (the two waves of a
// head block both form its score block). When tokens x head groups alone would leave the chip
// idle, each list is cut into splits of whole tiles; each split writes its
// normalised partial and lse, and sparse_merge combines them in split order.
// The workgroup's part of the slot list goes to LDS once (invalid slots as -1). Keys stream in
// tiles of 32 entries: each thread reads its 16-byte pieces two tiles ahead
// into one of two register sets while the current tile is in use; at the tile boundary the
// e4m3 pieces are widened, multiplied by their block's scale and rounded to
// bf16 (the rope pieces are copied), forming a [32, 576] bf16 tile in a
// two-slot LDS ring. The arithmetic is the prefill attention's: S^T = K Q^T
// with the heads' queries in registers, P^T straight from S^T's
// accumulators, O^T += V^T P^T with V^T (the first 512 columns of the same
// rows) read by ds_read_b64_tr_b16, online softmax in the exp2 domain.
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "prefill_kernels.h"

namespace mla {
namespace {

constexpr int kSE = 656;       // entry bytes
constexpr int kSKT = 32;       // entries per tile
constexpr int kSP = 1152 + 16; // LDS row pitch: 576 bf16 + 16 bytes of padding
constexpr int kSSlot = kSKT * kSP;
constexpr int kSPieces = 40;   // 16-byte pieces per entry read: 32 of codes, 8 of rope
constexpr int kSThreads = 512;  // 8 waves: 4 head blocks x 2 column halves
constexpr int kSTasks = (kSKT * kSPieces + kSThreads - 1) / kSThreads;  // per thread, per tile
static_assert(kSE == 512 + 16 + 128, "entry layout: codes, scales, rope");
constexpr float kSRescale = 8.f;

// 8 e4m3 codes times a scale, as 8 bf16 values (round to nearest even)
__device__ __forceinline__ u32x4_t fp8x8_scaled_bf16(uint32_t lo, uint32_t hi, float s) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  return u32x4_t{pack_bf16x2(a[0] * s, a[1] * s), pack_bf16x2(b[0] * s, b[1] * s),
                 pack_bf16x2(c[0] * s, c[1] * s), pack_bf16x2(d[0] * s, d[1] * s)};
}

__global__ void __launch_bounds__(kSThreads, 2) sparse_fp8_decode(SparseParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  MLA_LDS char* ring = (MLA_LDS char*)smem_raw;
  MLA_LDS int32_t* slots = (MLA_LDS int32_t*)(ring + 2 * kSSlot + kSThreads * 2 * 16);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hb = w >> 1, half = w & 1;  // head block of 16, output columns 256 half .. + 255
  const int bi = blockIdx.x;  // query token b * Sq + i
  const int b = bi / p.q_len, qi = bi - b * p.q_len;
  const int h = (int)blockIdx.y * 64 + 16 * hb + li;  // this lane's head
  const bool hok = h < p.n_heads;
  // a wave past the last head only helps load the tiles (wave-uniform)
  const bool wave_heads = (int)blockIdx.y * 64 + 16 * hb < p.n_heads;

  // this workgroup's part of the slot list, invalid entries as -1
  const int split = (int)blockIdx.z;
  const int jbeg = split * p.split_len;
  const int jend = p.topk - jbeg < p.split_len ? p.topk : jbeg + p.split_len;
  const int nkeys = jend > jbeg ? jend - jbeg : 0;
  const int32_t* idx = p.idx + (int64_t)b * p.i_s0 + (int64_t)qi * p.i_s1 + jbeg;
  for (int j = tid; j < nkeys; j += kSThreads) {
    const int32_t s = idx[j];
    slots[j] = (s >= 0 && (int64_t)s < p.num_slots) ? s : -1;
  }

  // the two waves of a head block split the score contraction: wave half
  // takes k-steps KH half .. KH half + KH - 1. The head's query row as the B
  // operand: lane holds q[h][32 (KH half + kk) + 8 g .. + 7]
  constexpr int KH = 576 / 32 / 2;
  i16x8_t qreg[KH];
  {
    const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)b * p.q_s0 + (int64_t)qi * p.q_s1 +
                           (int64_t)(hok ? h : 0) * p.q_s2 + 32 * KH * half + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KH; ++kk)
      qreg[kk] = hok ? *(const i16x8_t*)(qrow + 32 * kk) : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }
  // partial scores of every wave, [wave][lane][kh] as f32x4
  MLA_LDS f32x4_t* xs = (MLA_LDS f32x4_t*)(ring + 2 * kSSlot);
  __syncthreads();  // the slot list is in LDS

  const int ntiles = (nkeys + kSKT - 1) / kSKT;
  // task n of this thread: piece c of entry r of the tile
  // two register sets: tile t + 2 is read from memory while tile t is in use
  // and tile t + 1 waits in the other set for its slot of the LDS ring
  u32x4_t raw2[2][kSTasks];
  float rsc2[2][kSTasks];
  uint32_t nokey2[2] = {0u, 0u};  // bit n: task n belongs to an entry that is no key
  auto load_tile = [&](int t, u32x4_t (&raw)[kSTasks], float (&rsc)[kSTasks], uint32_t& nokey) {
    nokey = 0;
#pragma unroll
    for (int n = 0; n < kSTasks; ++n) {
      const int id = tid + kSThreads * n;
      if (id >= kSKT * kSPieces) break;
      const int r = id / kSPieces, c = id - r * kSPieces;
      const int j = t * kSKT + r;
      int s = j < nkeys ? slots[j] : -1;
      if (s < 0) {  // no key: read a valid entry, store zeros in its place
        s = 0;
        nokey |= 1u << n;
      }
      const int blk = p.page_shift >= 0 ? s >> p.page_shift : s / p.page;
      const int off = s - blk * p.page;
      const uint8_t* e = p.kv + (int64_t)blk * p.kv_s0 + (int64_t)off * p.kv_s1;
      raw[n] = *(const u32x4_t*)(e + (c < 32 ? 16 * c : 528 + 16 * (c - 32)));
      rsc[n] = c < 32 ? *(const float*)(e + 512 + 4 * (c >> 3)) : 1.f;
    }
  };
  auto store_tile = [&](int slot, const u32x4_t (&raw)[kSTasks], const float (&rsc)[kSTasks],
                        uint32_t nokey) {
    MLA_LDS char* kb = ring + slot * kSSlot;
#pragma unroll
    for (int n = 0; n < kSTasks; ++n) {
      const int id = tid + kSThreads * n;
      if (id >= kSKT * kSPieces) break;
      const int r = id / kSPieces, c = id - r * kSPieces;
      MLA_LDS char* row = kb + r * kSP;
      if (nokey & (1u << n)) {  // zeros, so that no bits of an unused entry reach P V
        const u32x4_t z = {0u, 0u, 0u, 0u};
        if (c < 32) {
          *(MLA_LDS u32x4_t*)(row + 32 * c) = z;
          *(MLA_LDS u32x4_t*)(row + 32 * c + 16) = z;
        } else {
          *(MLA_LDS u32x4_t*)(row + 1024 + 16 * (c - 32)) = z;
        }
      } else if (c < 32) {
        *(MLA_LDS u32x4_t*)(row + 32 * c) = fp8x8_scaled_bf16(raw[n][0], raw[n][1], rsc[n]);
        *(MLA_LDS u32x4_t*)(row + 32 * c + 16) = fp8x8_scaled_bf16(raw[n][2], raw[n][3], rsc[n]);
      } else {
        *(MLA_LDS u32x4_t*)(row + 1024 + 16 * (c - 32)) = raw[n];
      }
    }
  };

  constexpr int DB = 256 / 16;  // this wave's 16 output column blocks
  f32x4_t o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;

  if (ntiles > 0) {
    load_tile(0, raw2[0], rsc2[0], nokey2[0]);
    store_tile(0, raw2[0], rsc2[0], nokey2[0]);
  }
  if (ntiles > 1) load_tile(1, raw2[1], rsc2[1], nokey2[1]);
  __syncthreads();
  // one tile of the loop; SET is t % 2 (a constant, so the register sets stay registers)
  auto tile_step = [&](int t, auto set_c) {
    constexpr int SET = decltype(set_c)::value;
    if (t + 2 < ntiles) load_tile(t + 2, raw2[SET], rsc2[SET], nokey2[SET]);
    const MLA_LDS char* kb = ring + SET * kSSlot;
    const int j0 = t * kSKT;
    // S^T[key 16 kh + 4 g + jj][head li]: this wave's half of the k-steps,
    // then the other wave's half through LDS (both waves add the same two
    // partials, so they hold the same scores)
    f32x4_t s[2];
    if (wave_heads) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        s[kh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const MLA_LDS char* krow = kb + (16 * kh + li) * kSP + 64 * KH * half + 16 * g;
#pragma unroll
        for (int kk = 0; kk < KH; ++kk)
          s[kh] = mfma_16x16x32(*(const MLA_LDS i16x8_t*)(krow + 64 * kk), qreg[kk], s[kh]);
        xs[(w * 64 + lane) * 2 + kh] = s[kh];
      }
    }
    __syncthreads();
    if (wave_heads) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) s[kh] += xs[((w ^ 1) * 64 + lane) * 2 + kh];
    float x[2][4];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = j0 + 16 * kh + 4 * g + jj;
        const bool ok = j < nkeys && slots[j < nkeys ? j : 0] >= 0;
        x[kh][jj] = ok ? s[kh][jj] * p.scale_log2 : -__builtin_inff();
        tmax = fmaxf(tmax, x[kh][jj]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // the reference maximum moves only when a tile exceeds it by more than 2^8
    const bool move = tmax > m + kSRescale;
    const float mnew = move ? tmax : m;
    const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
    const float alpha = move ? __builtin_amdgcn_exp2f(m - muse) : 1.f;
    m = mnew;
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      // the hardware exp2: arguments stay below 8 (the lazy maximum), -inf gives 0
      const float p0 = __builtin_amdgcn_exp2f(x[kh][0] - muse), p1 = __builtin_amdgcn_exp2f(x[kh][1] - muse);
      const float p2 = __builtin_amdgcn_exp2f(x[kh][2] - muse), p3 = __builtin_amdgcn_exp2f(x[kh][3] - muse);
      psum += (p0 + p1) + (p2 + p3);
      pk[2 * kh] = pack_bf16x2(p0, p1);
      pk[2 * kh + 1] = pack_bf16x2(p2, p3);
    }
    l = l * alpha + psum;
    if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    // P^T slots 8 g + i: keys 4 g + i (i < 4) and 16 + 4 g + (i - 4)
    const i16x8_t pb = __builtin_bit_cast(i16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
    const MLA_LDS char* vrow0 = kb + (4 * g + (li >> 2)) * kSP + 512 * half + 8 * (li & 3);
    const MLA_LDS char* vrow1 = vrow0 + 16 * kSP;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4_t a0 = lds_read_tr16(vrow0 + 32 * db);
      const i16x4_t a1 = lds_read_tr16(vrow1 + 32 * db);
      const i16x8_t av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      o[db] = mfma_16x16x32(av, pb, o[db]);
    }
    }
    if (t + 1 < ntiles) store_tile(SET ^ 1, raw2[SET ^ 1], rsc2[SET ^ 1], nokey2[SET ^ 1]);
    __syncthreads();
  };
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    tile_step(t, std::integral_constant<int, 0>{});
    tile_step(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < ntiles) tile_step(t, std::integral_constant<int, 0>{});

  // a head's four lanes hold partial sums over their keys
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!hok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (p.nsplit > 1) {  // normalised partial (rounded to bf16) and its lse, merged by sparse_merge
    const int64_t r = ((int64_t)bi * p.nsplit + split) * p.n_heads + h;
    uint16_t* po = (uint16_t*)p.part_o + r * 512 + 256 * half + 4 * g;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *(u32x2_t*)(po + 16 * db) = u32x2_t{pack_bf16x2(o[db][0] * inv, o[db][1] * inv),
                                          pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
    if (g == 0 && half == 0)
      p.part_lse[r] = l > 0.f ? (m + __log2f(l)) * 0.69314718055994530942f : -__builtin_inff();
    return;
  }
  uint16_t* orow = (uint16_t*)p.out + (int64_t)b * p.o_s0 + (int64_t)qi * p.o_s1 +
                   (int64_t)h * p.o_s2 + 256 * half + 4 * g;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const u32x2_t v = {pack_bf16x2(o[db][0] * inv, o[db][1] * inv),
                       pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
    *(u32x2_t*)(orow + 16 * db) = v;
  }
  if (p.lse && g == 0 && half == 0)
    p.lse[(int64_t)b * p.l_s0 + (int64_t)qi * p.l_s1 + (int64_t)h * p.l_s2] =
        l > 0.f ? (m + __log2f(l)) * 0.69314718055994530942f : -__builtin_inff();
}

// One wave per (token, head): lane l merges columns 8 l .. 8 l + 7 over the
// splits in split order, out = sum_s exp(lse_s - lse) o_s with
// lse = ln sum_s exp(lse_s); no key in any split gives 0 and -inf.
__global__ void __launch_bounds__(256) sparse_merge(SparseParams p) {
  const int lane = threadIdx.x & 63;
  const int bi = blockIdx.x, h = (int)blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= p.n_heads) return;
  const int b = bi / p.q_len, qi = bi - b * p.q_len;
  const int64_t r0 = (int64_t)bi * p.nsplit * p.n_heads + h;
  // four splits' lse values and bf16 rows per round trip, combined in split
  // order with a running maximum (the sum rescaled when it rises)
  float mx = -__builtin_inff(), sum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.nsplit; s0 += 4) {
    float ls[4];
    u32x4_t x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t r = r0 + (int64_t)(s0 + k < p.nsplit ? s0 + k : s0) * p.n_heads;
      ls[k] = s0 + k < p.nsplit ? p.part_lse[r] : -__builtin_inff();
      x[k] = *(const u32x4_t*)((const uint16_t*)p.part_o + r * 512 + 8 * lane);
    }
    const float gm = fmaxf(fmaxf(ls[0], ls[1]), fmaxf(ls[2], ls[3]));
    if (gm > mx) {
      const float c = mx == -__builtin_inff() ? 0.f : __expf(mx - gm);
      sum *= c;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= c;
      mx = gm;
    }
    if (mx == -__builtin_inff()) continue;  // no split so far holds a key
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (ls[k] == -__builtin_inff()) continue;  // past the splits, or a split with no key
      const float wgt = __expf(ls[k] - mx);
      sum += wgt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wgt * __builtin_bit_cast(float, x[k][i] << 16);
        acc[2 * i + 1] += wgt * __builtin_bit_cast(float, x[k][i] & 0xffff0000u);
      }
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  uint16_t* orow = (uint16_t*)p.out + (int64_t)b * p.o_s0 + (int64_t)qi * p.o_s1 +
                   (int64_t)h * p.o_s2 + 8 * lane;
  const u32x4_t v = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                     pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  *(u32x2_t*)orow = u32x2_t{v[0], v[1]};
  *(u32x2_t*)(orow + 4) = u32x2_t{v[2], v[3]};
  if (p.lse && lane == 0)
    p.lse[(int64_t)b * p.l_s0 + (int64_t)qi * p.l_s1 + (int64_t)h * p.l_s2] =
        sum > 0.f ? mx + __logf(sum) : -__builtin_inff();
}

}  // namespace

size_t plan_sparse(int64_t tokens, int64_t n_heads, int64_t topk, int* split_len, int* nsplit) {
  // aim for at least 256 workgroups, one per CU (a workgroup's 8 waves need over
  // 128 registers each, so one fills a CU), splits of whole 32-entry tiles
  const int64_t tiles = (topk + kSKT - 1) / kSKT;
  const int64_t base = tokens * ((n_heads + 63) / 64);
  int64_t want = base > 0 ? (256 + base - 1) / base : 1;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t per = (tiles + want - 1) / want;  // tiles per split
  *split_len = (int)(per * kSKT > 0 ? per * kSKT : kSKT);
  *nsplit = (int)(tiles > 0 ? (tiles + per - 1) / per : 1);
  if (*nsplit <= 1) return 0;
  return (size_t)tokens * *nsplit * n_heads * (512 + 1) * sizeof(float);
}

// two ring slots, the partial-score exchange, the slot list
constexpr int kSXs = kSThreads * 2 * 16;
size_t sparse_lds_bytes(int topk) {
  return 2 * (size_t)kSSlot + kSXs + 4 * (size_t)(topk > 0 ? topk : 1);
}

hipError_t launch_sparse(const SparseParams& p, hipStream_t s) {
  if (p.batch == 0 || p.q_len == 0 || p.n_heads == 0) return hipSuccess;
  const size_t lds = sparse_lds_bytes(p.split_len < p.topk ? p.split_len : p.topk);
  static size_t attr = 0;
  if (lds > attr) {
    const hipError_t e = hipFuncSetAttribute((const void*)sparse_fp8_decode,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)(2 * kSSlot + kSXs + 4 * kSparseMaxTopk));
    if (e != hipSuccess) return e;
    attr = 2 * kSSlot + kSXs + 4 * kSparseMaxTopk;
  }
  dim3 grid((unsigned)((int64_t)p.batch * p.q_len), (unsigned)((p.n_heads + 63) / 64),
            (unsigned)p.nsplit);
  hipLaunchKernelGGL(sparse_fp8_decode, grid, dim3(kSThreads), lds, s, p);
  if (p.nsplit > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 mg((unsigned)((int64_t)p.batch * p.q_len), (unsigned)((p.n_heads + 3) / 4));
    hipLaunchKernelGGL(sparse_merge, mg, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mla
