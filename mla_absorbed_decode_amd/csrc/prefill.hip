// prefill.hip -- the naive (decompressed) prefill route on gfx950: per-head
// keys and values rebuilt from the latent rows, then standard multi-head
// attention over them (memra-engine 0.124.1 "tests/mla_gpu_forward.rs": the
// naive oracle `mla_attend_naive`, which decompresses K and V per head;
// vllm.cpp "tests/vt/test_ops_mla_absorb.cpp": ConcatMlaNopeRope, the case
// that broadcasts the single k_pe head across every head). For long prompts
// this costs 2 (d_nope + d_rope + d_v) flops per (query, key, head) against
// 2 (2 kv_rank + d_rope) for the absorbed form.
//
// Key decompression (bmm_nt_bf16): out[t, h, n] = sum_k a[t, h, k] w[h, n, k]
// with the token's rope row copied behind every head's n columns. Both
// operands are contiguous along k, which is exactly the per-lane layout of
// v_mfma_f32_16x16x32_bf16's A and B operands (8 consecutive k per lane), so
// each lane loads its 16-byte pieces straight from global memory. A 64 x 64
// output tile per workgroup; each wave owns 32 x 32 of it (2 x 2 MFMA tiles,
// two A and two B loads per four MFMAs).
//
// Attention (mha_fwd<DK, DV>): one workgroup per (128 query rows, head,
// sequence): four waves of two 16-row query blocks (eight waves of one for
// the widest heads). 32-key tiles of K and V are loaded into
// registers one tile ahead and stored to a two-slot LDS ring (one barrier per
// tile). Scores are computed transposed, S^T = K Q^T, with the wave's query
// rows held in registers as the B operand: S^T's accumulator layout (lane l:
// keys 4(l/16) + j and 16 + 4(l/16) + j of query l % 16) is then the B-operand
// layout of P^T in O^T += V^T P^T, so P never leaves registers, and V^T comes
// from LDS through ds_read_b64_tr_b16. Online softmax in the exp2 domain; the
// running max is shared by a query's four lanes (two cross-lane exchanges per
// tile), each lane keeps its own partial sum until the end.
//
// mha_fwd32<DK, DV> does the same with 32-row query blocks and the
// 32x32x16 MFMA (half the LDS operand reads per flop), four waves per
// workgroup and two workgroups per CU. It serves every head width but the
// widest: at 256/256 its 32 x 256 accumulators and 32-row queries need more
// than the 256 registers two waves per SIMD allow, and with one wave per SIMD
// it measured 476 us against mha_fwd's 360 us on the NoPE prefill (64 heads,
// 2048 causal). Measured at 2048 causal tokens: 192/128 with 16 heads 124 ->
// 97 us, with 128 heads 464 -> 382 us; 128/128 (4096 tokens) 201 -> 192 us.
#include <type_traits>

#include "gemm_tile.h"
#include "mla_device.h"
#include "mla_kernels.h"
#include "prefill_kernels.h"

namespace mla {
namespace {

// ------------------------------------------------------------ key decompression
constexpr int kNtM = 64, kNtN = 64, kNtK = 32;

// out[t, h, N + r] = pe[t, r] for the tile's tokens, in the workgroups of the
// first column tile.
template <class T>
__device__ __forceinline__ void copy_rope_broadcast(const BmmNtParams& p, int t0, int h,
                                                    int rows = kNtM, int wx = -1) {
  if (p.R == 0 || (wx < 0 ? (int)blockIdx.x : wx) != 0) return;
  const int nt = (int)(p.T - t0 < rows ? p.T - t0 : rows);
  const int R = (int)p.R;
  for (int e = threadIdx.x; e < nt * R; e += blockDim.x) {
    const int t = t0 + e / R, r = e % R;
    ((T*)p.out)[(int64_t)t * p.o_st + (int64_t)h * p.o_sh + p.N + r] =
        ((const T*)p.pe)[(int64_t)t * p.pe_st + r];
  }
}

__global__ void __launch_bounds__(256) bmm_nt_bf16(BmmNtParams p) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
  const int wr = w >> 1, wc = w & 1;
  const int n0 = blockIdx.x * kNtN, t0 = blockIdx.y * kNtM, h = blockIdx.z;
  const uint16_t* arow[2];
  const uint16_t* brow[2];
  bool aok[2], bok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 32 * wr + 16 * i + li;
    aok[i] = t < p.T;
    arow[i] = (const uint16_t*)p.a + (int64_t)(aok[i] ? t : 0) * p.a_st + (int64_t)h * p.a_sh + 8 * g;
    const int n = n0 + 32 * wc + 16 * i + li;
    bok[i] = n < p.N;
    brow[i] = (const uint16_t*)p.w + (int64_t)h * p.w_sh + (int64_t)(bok[i] ? n : 0) * p.w_sn + 8 * g;
  }
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const i16x8_t zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 4
  for (int k0 = 0; k0 < p.K; k0 += kNtK) {
    i16x8_t av[2], bv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      av[i] = aok[i] ? *(const i16x8_t*)(arow[i] + k0) : zero;
      bv[i] = bok[i] ? *(const i16x8_t*)(brow[i] + k0) : zero;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma_16x16x32(av[i], bv[j], acc[i][j]);
  }
  // lane holds out[t0 + 32 wr + 16 i + 4 g + jj][n0 + 32 wc + 16 j + li]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 32 * wc + 16 * j + li;
      if (n >= p.N) continue;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int t = t0 + 32 * wr + 16 * i + 4 * g + jj;
        if (t < p.T)
          ((uint16_t*)p.out)[(int64_t)t * p.o_st + (int64_t)h * p.o_sh + n] = f32_to_bf16(acc[i][j][jj]);
      }
    }
  copy_rope_broadcast<uint16_t>(p, t0, h);
}

// Prefill-sized token counts: 128 x 128 output tiles of the shared pipelined
// tile (gemm_tile.h), then the rope rows of the tile's 128 tokens.
__global__ void __launch_bounds__(256) bmm_nt_big(BmmNtParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[kGLds];
  int nt, tt, h;
  gemm_tile_coords(nt, tt, h);
  GemmTileArgs g;
  g.a = (const uint16_t*)p.a + (int64_t)h * p.a_sh; g.a_st = p.a_st;
  g.w = (const uint16_t*)p.w + (int64_t)h * p.w_sh; g.w_s1 = p.w_sn;
  g.out = (uint16_t*)p.out + (int64_t)h * p.o_sh; g.o_st = p.o_st;
  g.T = (int)p.T; g.K = (int)p.K; g.N = (int)p.N;
  g.t0 = tt * kGT; g.n0 = nt * kGT;
  gemm_tile_128<true>(g, (MLA_LDS char*)lds_raw);
  copy_rope_broadcast<uint16_t>(p, g.t0, h, kGT, nt);
}

// f32 operands (16-byte aligned rows, K a multiple of 16): v_mfma_f32_16x16x4f32
// with both operands read along k straight from global memory. Each wave owns a
// 32 x 32 output tile (two row tiles x two column tiles). For a 16-wide k block
// lane (li, g) loads a[t][k0 + 4g .. + 3] and w[n][k0 + 4g .. + 3] as float4;
// MFMA c (c = 0..3) takes component c of both, i.e. k = k0 + 4g + c over the
// four lane groups, so the four MFMAs cover the block. The next block's
// operands are loaded while the current one is multiplied.
__global__ void __launch_bounds__(256) bmm_nt_f32(BmmNtParams p) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
  const int64_t t0 = (int64_t)blockIdx.y * kNtM + (w >> 1) * 32;
  const int64_t n0 = (int64_t)blockIdx.x * kNtN + (w & 1) * 32;
  const int h = blockIdx.z;
  const float* A = (const float*)p.a + (int64_t)h * p.a_sh;
  const float* W = (const float*)p.w + (int64_t)h * p.w_sh;
  // rows past T or N read row 0 (valid memory); their outputs are not stored
  const float* ap[2];
  const float* wp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t t = t0 + 16 * i + li, n = n0 + 16 * i + li;
    ap[i] = A + (t < p.T ? t : 0) * p.a_st + 4 * g;
    wp[i] = W + (n < p.N ? n : 0) * p.w_sn + 4 * g;
  }
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t ab[2][2], wb[2][2];
  auto load = [&](int64_t k0, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ab[buf][i] = *(const f32x4_t*)(ap[i] + k0);
      wb[buf][i] = *(const f32x4_t*)(wp[i] + k0);
    }
  };
  load(0, 0);
  const int64_t nk = p.K / 16;
  for (int64_t kb = 0; kb < nk; ++kb) {
    const int cur = (int)(kb & 1);
    if (kb + 1 < nk) load((kb + 1) * 16, cur ^ 1);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mfma_16x16x4f32(ab[cur][i][c], wb[cur][j][c], acc[i][j]);
  }
  // lane holds out[t0 + 16 i + 4 g + r][n0 + 16 j + li], r = 0..3
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + 16 * j + li;
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 16 * i + 4 * g + r;
        if (t < p.T) ((float*)p.out)[t * p.o_st + (int64_t)h * p.o_sh + n] = acc[i][j][r];
      }
    }
  if (blockIdx.x == 0 && (w & 1) == 0 && p.R > 0) {
    // the rope rows of this wave's 32 tokens, copied bit for bit behind every head's N columns
    for (int e = lane; e < 32 * (int)p.R; e += 64) {
      const int64_t t = t0 + e / p.R, r = e % p.R;
      if (t < p.T)
        ((uint32_t*)p.out)[t * p.o_st + (int64_t)h * p.o_sh + p.N + r] =
            ((const uint32_t*)p.pe)[t * p.pe_st + r];
    }
  }
}

// Any size or alignment, bf16 or f32: one thread per output element, f32
// accumulation in k order.
template <bool F32>
__global__ void __launch_bounds__(256) bmm_nt_plain(BmmNtParams p) {
  const int64_t W = p.N + p.R;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.T * p.H * W) return;
  const int64_t t = idx / (p.H * W), rem = idx % (p.H * W), h = rem / W, n = rem % W;
  float v;
  if (n < p.N) {
    float acc = 0.f;
    for (int64_t k = 0; k < p.K; ++k) {
      const int64_t ai = t * p.a_st + h * p.a_sh + k, wi = h * p.w_sh + n * p.w_sn + k;
      const float a = F32 ? ((const float*)p.a)[ai] : bf16_to_f32(((const uint16_t*)p.a)[ai]);
      const float b = F32 ? ((const float*)p.w)[wi] : bf16_to_f32(((const uint16_t*)p.w)[wi]);
      acc = __builtin_fmaf(a, b, acc);
    }
    v = acc;
    const int64_t oi = t * p.o_st + h * p.o_sh + n;
    if (F32) ((float*)p.out)[oi] = v;
    else ((uint16_t*)p.out)[oi] = f32_to_bf16(v);
  } else {  // the rope row, copied bit for bit
    const int64_t oi = t * p.o_st + h * p.o_sh + n, pi = t * p.pe_st + (n - p.N);
    if (F32) ((uint32_t*)p.out)[oi] = ((const uint32_t*)p.pe)[pi];
    else ((uint16_t*)p.out)[oi] = ((const uint16_t*)p.pe)[pi];
  }
}

// -------------------------------------------------------------------- attention
constexpr int kKT = 32;  // keys per tile

// Launch shape per head width: NW waves of QB 16-row query blocks each. A
// wave's query blocks share every K and V^T operand it reads from LDS, which
// is what bounds this kernel: two blocks halve the LDS bytes per flop. The
// widest heads keep one block per wave (two would not fit the registers).
template <int DK, int DV>
struct MhaShape {
  // Two blocks per wave (4 waves) passed the parity tests but ran slower than
  // one block per wave (8 waves) at 192/128 and 128/128 on MI355X: the kernel
  // waits on its tile loads more than on LDS.
  static constexpr int QB = 1;                             // query blocks per wave
  static constexpr int NW = QB == 2 ? 4 : 8;               // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int QT = 16 * QB * NW;                  // query rows per workgroup
  // LDS rows are padded so that the K-operand reads (16 consecutive rows, one
  // 16-byte piece each per 16 lanes) and the transposed V reads (4
  // consecutive rows x 32 bytes per 16 lanes) fall in distinct banks.
  static constexpr int KP = DK * 2 + 16;  // K row pitch, bytes
  static constexpr int VP = DV * 2 + 32;  // V row pitch, bytes
  static constexpr int KBYTES = kKT * KP, VBYTES = kKT * VP;
  static constexpr int SLOT = KBYTES + VBYTES;
  static constexpr int LDS = 2 * SLOT;
  static constexpr int KCH = DK / 8, VCH = DV / 8;  // 16-byte pieces per row
  static constexpr int KPC = kKT * KCH, VPC = kKT * VCH;  // pieces per tile
  static constexpr int NKL = (KPC + THREADS - 1) / THREADS;  // pieces per thread (at most)
  static constexpr int NVL = (VPC + THREADS - 1) / THREADS;
  static_assert(DK % 32 == 0 && DV % 16 == 0, "MFMA tiling");
};

// Rescale threshold of the online softmax (log2 domain): the running maximum
// a row's probabilities are taken against moves only when a score exceeds it
// by more than 2^8, so most tiles skip rescaling the output; probabilities
// stay below 2^8, well inside bf16 and f32 range.
constexpr float kRescale = 8.f;

// 2^x in the attention softmax (arguments below 8, the lazy maximum; -inf
// gives 0). The hardware instruction alone leaves the narrower instances
// (192/128: 154 -> 125 registers, a fourth wave per SIMD) 11-28 % faster;
// the 256-wide one measured 10 % slower with it and keeps exp2f.
template <int DK>
__device__ __forceinline__ float softmax_exp2(float x) {
  if constexpr (DK >= 256) return exp2f(x);
  else return __builtin_amdgcn_exp2f(x);
}

template <int DK, int DV>
__global__ void __launch_bounds__((MhaShape<DK, DV>::THREADS), 2) mha_fwd(MhaParams p) {
  using Sh = MhaShape<DK, DV>;
  constexpr int QB = Sh::QB, THREADS = Sh::THREADS, QT = Sh::QT;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.z;
  // (query tile x, head), longest causal tiles first; with p.pair_tiles the
  // workgroup takes query tiles ntq - 1 - x and x, so that under a causal mask
  // every workgroup streams about the same number of key tiles. Consecutive
  // workgroups go to the 8 XCDs in turn, each with its own L2: with a head
  // count divisible by 8, XCD x runs only heads x, x + 8, ..., so a head's
  // keys and values are read from one L2.
  const int nx = (int)gridDim.x;
  const int ntq = (p.max_q + QT - 1) / QT;
  int h, x;
  if (p.n_heads % 8 == 0) {
    const int i = (int)blockIdx.x + nx * (int)blockIdx.y, j = i >> 3;
    h = (j / nx) * 8 + (i & 7);
    x = nx - 1 - j % nx;
  } else {
    h = (int)blockIdx.y;
    x = nx - 1 - (int)blockIdx.x;
  }
  // the sequence's rows, clamped to the buffers
  int q0 = p.cu_q[b], q1 = p.cu_q[b + 1], k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
  q1 = q1 < 0 ? 0 : (q1 > p.T ? (int)p.T : q1);
  q0 = q0 < 0 ? 0 : (q0 > q1 ? q1 : q0);
  k1 = k1 < 0 ? 0 : (k1 > p.S ? (int)p.S : k1);
  k0 = k0 < 0 ? 0 : (k0 > k1 ? k1 : k0);
  const int lq = q1 - q0, lk = k1 - k0;
  for (int pass = 0; pass < 2; ++pass) {
    const int qt = p.pair_tiles && pass == 0 ? ntq - 1 - x : x;
    if (pass == 1) {
      // no pair, or an odd tile count: the middle tile has no partner
      if (!p.pair_tiles || qt == ntq - 1 - x) break;
      __syncthreads();  // every wave is done with the ring before it is refilled
    }
    const int qbase = qt * QT;
    if (qbase >= lq) continue;
    // keys this workgroup needs: up to the last visible key of its last row
    int kend = lk;
    if (p.causal) {
      const int last = (qbase + QT < lq ? qbase + QT : lq) - 1;
      kend = lk - lq + last + 1;
      kend = kend < 0 ? 0 : (kend > lk ? lk : kend);
    }
    const int ntiles = (kend + kKT - 1) / kKT;

    // this lane's query row in block qb: wrow + 16 qb + li (index in the sequence)
    const int wrow = qbase + 16 * QB * w;
    int vis_end[QB];
    bool qok[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = wrow + 16 * qb + li;
      qok[qb] = qi < lq;
      const int pos = lk - lq + qi;
      vis_end[qb] = p.causal ? (pos + 1 < lk ? pos + 1 : lk) : lk;  // keys [0, vis_end) visible
    }
    // keys past the wave's last visible key need no arithmetic (wave-uniform)
    int wave_end = 0;
    if (wrow < lq) {
      const int wlast = wrow + 16 * QB - 1 < lq ? wrow + 16 * QB - 1 : lq - 1;
      wave_end = p.causal ? lk - lq + wlast + 1 : lk;
      wave_end = wave_end < 0 ? 0 : (wave_end > lk ? lk : wave_end);
    }

    // the wave's query rows as the B operand: lane holds q[row][32 kk + 8 g .. + 7]
    constexpr int KK = DK / 32;
    i16x8_t qreg[QB][KK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = wrow + 16 * qb + li;
      const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)(q0 + (qok[qb] ? qi : 0)) * p.q_s0 +
                             (int64_t)h * p.q_s1 + 8 * g;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qreg[qb][kk] = qok[qb] ? *(const i16x8_t*)(qrow + 32 * kk) : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }

    const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)k0 * p.k_s0 + (int64_t)h * p.k_s1;
    const uint16_t* vbase = (const uint16_t*)p.v + (int64_t)k0 * p.v_s0 + (int64_t)h * p.v_s1;
    // two register sets: tile t + 2 is read from memory while tile t is in use
    // and tile t + 1 waits in the other set for its slot of the LDS ring
    u32x4_t kr2[2][Sh::NKL], vr2[2][Sh::NVL];
    // global -> registers: piece i of the tile starting at key j0 (rows past the
    // sequence repeat its last key; their scores are masked)
    auto load_tile = [&](int j0, u32x4_t (&kr)[Sh::NKL], u32x4_t (&vr)[Sh::NVL]) {
#pragma unroll
      for (int i = 0; i < Sh::NKL; ++i) {
        const int idx = tid + THREADS * i, r = idx / Sh::KCH, c = idx % Sh::KCH;
        const int j = j0 + r < lk ? j0 + r : lk - 1;
        if (idx < Sh::KPC) kr[i] = *(const u32x4_t*)(kbase + (int64_t)j * p.k_s0 + 8 * c);
      }
#pragma unroll
      for (int i = 0; i < Sh::NVL; ++i) {
        const int idx = tid + THREADS * i, r = idx / Sh::VCH, c = idx % Sh::VCH;
        const int j = j0 + r < lk ? j0 + r : lk - 1;
        if (idx < Sh::VPC) vr[i] = *(const u32x4_t*)(vbase + (int64_t)j * p.v_s0 + 8 * c);
      }
    };
    auto store_tile = [&](int slot, const u32x4_t (&kr)[Sh::NKL], const u32x4_t (&vr)[Sh::NVL]) {
      MLA_LDS char* kb = smem + slot * Sh::SLOT;
      MLA_LDS char* vb = kb + Sh::KBYTES;
#pragma unroll
      for (int i = 0; i < Sh::NKL; ++i) {
        const int idx = tid + THREADS * i, r = idx / Sh::KCH, c = idx % Sh::KCH;
        if (idx < Sh::KPC) *(MLA_LDS u32x4_t*)(kb + r * Sh::KP + 16 * c) = kr[i];
      }
#pragma unroll
      for (int i = 0; i < Sh::NVL; ++i) {
        const int idx = tid + THREADS * i, r = idx / Sh::VCH, c = idx % Sh::VCH;
        if (idx < Sh::VPC) *(MLA_LDS u32x4_t*)(vb + r * Sh::VP + 16 * c) = vr[i];
      }
    };

    constexpr int DB = DV / 16;
    f32x4_t o[QB][DB];
    float m[QB], l[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int d = 0; d < DB; ++d) o[qb][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m[qb] = -__builtin_inff();
      l[qb] = 0.f;
    }

    if (ntiles > 0) {
      load_tile(0, kr2[0], vr2[0]);
      store_tile(0, kr2[0], vr2[0]);
    }
    if (ntiles > 1) load_tile(kKT, kr2[1], vr2[1]);
    __syncthreads();
    // one tile of the loop; SET is t % 2 (a constant, so the register sets stay registers)
    auto tile_step = [&](int t, auto set_c) {
      constexpr int SET = decltype(set_c)::value;
      if (t + 2 < ntiles) load_tile((t + 2) * kKT, kr2[SET], vr2[SET]);
      const MLA_LDS char* kb = smem + SET * Sh::SLOT;
      const MLA_LDS char* vb = kb + Sh::KBYTES;
      const int j0 = t * kKT;
      if (j0 < wave_end) {
        // S^T[key 16 kh + 4 g + jj][query li] of each query block, one K read for all
        f32x4_t s[QB][2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          const MLA_LDS char* krow = kb + (16 * kh + li) * Sh::KP + 16 * g;
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const i16x8_t ka = *(const MLA_LDS i16x8_t*)(krow + 64 * kk);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][kh] = mfma_16x16x32(ka, qreg[qb][kk], s[qb][kh]);
          }
        }
        i16x8_t pb[QB];
        float alpha[QB];
        bool rescale = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float x[2][4];
          float tmax = -__builtin_inff();
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int key = j0 + 16 * kh + 4 * g + jj;
              x[kh][jj] = key < vis_end[qb] ? s[qb][kh][jj] * p.scale_log2 : -__builtin_inff();
              tmax = fmaxf(tmax, x[kh][jj]);
            }
          tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
          tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
          // move the reference maximum only when this tile exceeds it by more than 2^8
          const bool move = tmax > m[qb] + kRescale;
          const float mnew = move ? tmax : m[qb];
          const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
          alpha[qb] = move ? softmax_exp2<DK>(m[qb] - muse) : 1.f;
          rescale |= move;
          m[qb] = mnew;
          float psum = 0.f;
          uint32_t pk[4];
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const float p0 = softmax_exp2<DK>(x[kh][0] - muse);
            const float p1 = softmax_exp2<DK>(x[kh][1] - muse);
            const float p2 = softmax_exp2<DK>(x[kh][2] - muse);
            const float p3 = softmax_exp2<DK>(x[kh][3] - muse);
            psum += (p0 + p1) + (p2 + p3);
            pk[2 * kh] = pack_bf16x2(p0, p1);
            pk[2 * kh + 1] = pack_bf16x2(p2, p3);
          }
          l[qb] = l[qb] * alpha[qb] + psum;
          // P^T slots 8 g + i: keys 4 g + i (i < 4) and 16 + 4 g + (i - 4)
          pb[qb] = __builtin_bit_cast(i16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
        }
        if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < DB; ++db) o[qb][db] *= alpha[qb];
        }
        // V^T rows d = 16 db + li from two transposed reads (keys 4 g .. 4 g + 3,
        // then 16 + 4 g ..), shared by the query blocks
        const int vr0 = 4 * g + (li >> 2);
        const MLA_LDS char* vrow0 = vb + vr0 * Sh::VP + 8 * (li & 3);
        const MLA_LDS char* vrow1 = vrow0 + 16 * Sh::VP;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4_t a0 = lds_read_tr16(vrow0 + 32 * db);
          const i16x4_t a1 = lds_read_tr16(vrow1 + 32 * db);
          const i16x8_t av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma_16x16x32(av, pb[qb], o[qb][db]);
        }
      }
      if (t + 1 < ntiles) store_tile(SET ^ 1, kr2[SET ^ 1], vr2[SET ^ 1]);
      __syncthreads();
    };
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      tile_step(t, std::integral_constant<int, 0>{});
      tile_step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < ntiles) tile_step(t, std::integral_constant<int, 0>{});

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // a query's four lanes hold partial sums over their keys
      float lt = l[qb];
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
      if (!qok[qb]) continue;
      const int qi = wrow + 16 * qb + li;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* orow = (uint16_t*)p.out + (int64_t)(q0 + qi) * p.o_s0 + (int64_t)h * p.o_s1 + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2_t v = {pack_bf16x2(o[qb][db][0] * inv, o[qb][db][1] * inv),
                           pack_bf16x2(o[qb][db][2] * inv, o[qb][db][3] * inv)};
        *(u32x2_t*)(orow + 16 * db) = v;
      }
      if (p.lse && g == 0)
        p.lse[(int64_t)(q0 + qi) * p.l_s0 + (int64_t)h * p.l_s1] =
            lt > 0.f ? (m[qb] + __log2f(lt)) * 0.69314718055994530942f : -__builtin_inff();
    }
  }
}

// Attention with 32-row query blocks (mha_fwd32<DK, DV>): the same stream
// and softmax as mha_fwd, with v_mfma_f32_32x32x16_bf16. A wave owns 32 query
// rows, so each K operand and each V^T operand it reads from LDS feeds 32 rows
// instead of 16: four waves (128 rows) read half the LDS bytes per tile that
// eight waves of 16-row blocks do, for the same MFMA work.
//   S^T = K Q^T: A = K (lane: key l%32, dims 16 kk + 8 (l/32) .. + 7, a 16-byte
//   piece of the key's row), B = Q^T (lane: query l%32, the same dims).
//   S^T's lane l then holds query l%32 and keys 8 b + 4 h + j (h = l/32,
//   b, j = 0..3), so a query's 32 scores sit in lanes l and l ^ 32.
//   O^T += V^T P^T per 16-key step ks: B = P^T is the lane's own scores
//   8 ks .. 8 ks + 7 (keys 16 ks + 4 h + j, then 16 ks + 8 + 4 h + j), and
//   A = V^T holds dims l%32 of the same keys in the same order, read by two
//   ds_read_b64_tr_b16 (four consecutive keys each).
template <int DK, int DV>
struct Mha32Shape {
  static constexpr int NW = 4;                  // waves, one 32-row query block each
  static constexpr int THREADS = 64 * NW;
  static constexpr int QT = 32 * NW;            // query rows per workgroup
  static constexpr int KP = DK * 2 + 16;        // K row pitch, bytes (K reads: 32 rows, 2 pieces)
  static constexpr int VP = DV * 2 + 32;        // V row pitch, bytes (V^T reads: 4 rows x 32 B)
  static constexpr int KBYTES = kKT * KP, VBYTES = kKT * VP;
  static constexpr int SLOT = KBYTES + VBYTES;
  static constexpr int LDS = 2 * SLOT;
  static constexpr int KCH = DK / 8, VCH = DV / 8;
  static constexpr int KPC = kKT * KCH, VPC = kKT * VCH;
  static constexpr int NKL = (KPC + THREADS - 1) / THREADS;
  static constexpr int NVL = (VPC + THREADS - 1) / THREADS;
  static_assert(DK % 16 == 0 && DV % 32 == 0, "MFMA tiling");
};

template <int DK, int DV>
__global__ void __launch_bounds__((Mha32Shape<DK, DV>::THREADS), 2) mha_fwd32(MhaParams p) {
  using Sh = Mha32Shape<DK, DV>;
  constexpr int THREADS = Sh::THREADS, QT = Sh::QT;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  MLA_LDS char* smem = (MLA_LDS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.z;
  // (query tile x, head), longest causal tiles first; with p.pair_tiles the
  // workgroup takes query tiles ntq - 1 - x and x, so that under a causal mask
  // every workgroup streams about the same number of key tiles. Consecutive
  // workgroups go to the 8 XCDs in turn, each with its own L2: with a head
  // count divisible by 8, XCD x runs only heads x, x + 8, ..., so a head's
  // keys and values are read from one L2.
  const int nx = (int)gridDim.x;
  const int ntq = (p.max_q + QT - 1) / QT;
  int h, x;
  if (p.n_heads % 8 == 0) {
    const int i = (int)blockIdx.x + nx * (int)blockIdx.y, j = i >> 3;
    h = (j / nx) * 8 + (i & 7);
    x = nx - 1 - j % nx;
  } else {
    h = (int)blockIdx.y;
    x = nx - 1 - (int)blockIdx.x;
  }
  int q0 = p.cu_q[b], q1 = p.cu_q[b + 1], k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
  q1 = q1 < 0 ? 0 : (q1 > p.T ? (int)p.T : q1);
  q0 = q0 < 0 ? 0 : (q0 > q1 ? q1 : q0);
  k1 = k1 < 0 ? 0 : (k1 > p.S ? (int)p.S : k1);
  k0 = k0 < 0 ? 0 : (k0 > k1 ? k1 : k0);
  const int lq = q1 - q0, lk = k1 - k0;
  for (int pass = 0; pass < 2; ++pass) {
    const int qt = p.pair_tiles && pass == 0 ? ntq - 1 - x : x;
    if (pass == 1) {
      // no pair, or an odd tile count: the middle tile has no partner
      if (!p.pair_tiles || qt == ntq - 1 - x) break;
      __syncthreads();  // every wave is done with the ring before it is refilled
    }
    const int qbase = qt * QT;
    if (qbase >= lq) continue;
    int kend = lk;
    if (p.causal) {
      const int last = (qbase + QT < lq ? qbase + QT : lq) - 1;
      kend = lk - lq + last + 1;
      kend = kend < 0 ? 0 : (kend > lk ? lk : kend);
    }
    const int ntiles = (kend + kKT - 1) / kKT;

    // this lane's query row: wrow + lr
    const int wrow = qbase + 32 * w;
    const int qi = wrow + lr;
    const bool qok = qi < lq;
    const int pos = lk - lq + qi;
    const int vis_end = p.causal ? (pos + 1 < lk ? pos + 1 : lk) : lk;  // keys [0, vis_end)
    int wave_end = 0;
    if (wrow < lq) {
      const int wlast = wrow + 31 < lq ? wrow + 31 : lq - 1;
      wave_end = p.causal ? lk - lq + wlast + 1 : lk;
      wave_end = wave_end < 0 ? 0 : (wave_end > lk ? lk : wave_end);
    }

    // Q^T as the B operand: lane holds q[row][16 kk + 8 hh .. + 7]
    constexpr int KK = DK / 16;
    i16x8_t qreg[KK];
    {
      const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)(q0 + (qok ? qi : 0)) * p.q_s0 +
                             (int64_t)h * p.q_s1 + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qreg[kk] = qok ? *(const i16x8_t*)(qrow + 16 * kk) : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }

    const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)k0 * p.k_s0 + (int64_t)h * p.k_s1;
    const uint16_t* vbase = (const uint16_t*)p.v + (int64_t)k0 * p.v_s0 + (int64_t)h * p.v_s1;
    u32x4_t kr2[2][Sh::NKL], vr2[2][Sh::NVL];
    auto load_tile = [&](int j0, u32x4_t (&kr)[Sh::NKL], u32x4_t (&vr)[Sh::NVL]) {
#pragma unroll
      for (int i = 0; i < Sh::NKL; ++i) {
        const int idx = tid + THREADS * i, r = idx / Sh::KCH, c = idx % Sh::KCH;
        const int j = j0 + r < lk ? j0 + r : lk - 1;
        if (idx < Sh::KPC) kr[i] = *(const u32x4_t*)(kbase + (int64_t)j * p.k_s0 + 8 * c);
      }
#pragma unroll
      for (int i = 0; i < Sh::NVL; ++i) {
        const int idx = tid + THREADS * i, r = idx / Sh::VCH, c = idx % Sh::VCH;
        const int j = j0 + r < lk ? j0 + r : lk - 1;
        if (idx < Sh::VPC) vr[i] = *(const u32x4_t*)(vbase + (int64_t)j * p.v_s0 + 8 * c);
      }
    };
    auto store_tile = [&](int slot, const u32x4_t (&kr)[Sh::NKL], const u32x4_t (&vr)[Sh::NVL]) {
      MLA_LDS char* kb = smem + slot * Sh::SLOT;
      MLA_LDS char* vb = kb + Sh::KBYTES;
#pragma unroll
      for (int i = 0; i < Sh::NKL; ++i) {
        const int idx = tid + THREADS * i, r = idx / Sh::KCH, c = idx % Sh::KCH;
        if (idx < Sh::KPC) *(MLA_LDS u32x4_t*)(kb + r * Sh::KP + 16 * c) = kr[i];
      }
#pragma unroll
      for (int i = 0; i < Sh::NVL; ++i) {
        const int idx = tid + THREADS * i, r = idx / Sh::VCH, c = idx % Sh::VCH;
        if (idx < Sh::VPC) *(MLA_LDS u32x4_t*)(vb + r * Sh::VP + 16 * c) = vr[i];
      }
    };

    constexpr int DT = DV / 32;
    f32x16_t o[DT];
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    float m = -__builtin_inff(), l = 0.f;

    if (ntiles > 0) {
      load_tile(0, kr2[0], vr2[0]);
      store_tile(0, kr2[0], vr2[0]);
    }
    if (ntiles > 1) load_tile(kKT, kr2[1], vr2[1]);
    __syncthreads();
    // transposed V reads: local lane s of 16-lane group G points at key row
    // 4 hh + (s / 4) (+ 8 per read) and dims 16 (G % 2) + 4 (s % 4) .. + 3
    const int G = lane >> 4, sl = lane & 15;
    const int vrow = 4 * hh + (sl >> 2);
    const int vcol = 16 * (G & 1) + 4 * (sl & 3);
    auto tile_step = [&](int t, auto set_c) {
      constexpr int SET = decltype(set_c)::value;
      if (t + 2 < ntiles) load_tile((t + 2) * kKT, kr2[SET], vr2[SET]);
      const MLA_LDS char* kb = smem + SET * Sh::SLOT;
      const MLA_LDS char* vb = kb + Sh::KBYTES;
      const int j0 = t * kKT;
      if (j0 < wave_end) {
        // S^T over the wave's 32 rows: two accumulators (even and odd k-steps)
        f32x16_t sa = {}, sb = {};
        const MLA_LDS char* krow = kb + lr * Sh::KP + 16 * hh;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const i16x8_t ka = *(const MLA_LDS i16x8_t*)(krow + 32 * kk);
          if (kk & 1) sb = mfma_32x32x16(ka, qreg[kk], sb);
          else sa = mfma_32x32x16(ka, qreg[kk], sa);
        }
        float x[16];
        float tmax = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          x[r] = key < vis_end ? (sa[r] + sb[r]) * p.scale_log2 : -__builtin_inff();
          tmax = fmaxf(tmax, x[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool move = tmax > m + kRescale;
        const float mnew = move ? tmax : m;
        const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
        const float alpha = move ? softmax_exp2<DK>(m - muse) : 1.f;
        m = mnew;
        float psum = 0.f;
        uint32_t pk[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = softmax_exp2<DK>(x[r] - muse);
          const float p1 = softmax_exp2<DK>(x[r + 1] - muse);
          psum += p0 + p1;
          pk[r >> 1] = pack_bf16x2(p0, p1);
        }
        l = l * alpha + psum;
        if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
          for (int d = 0; d < DT; ++d) o[d] *= alpha;
        }
        // P^T for key steps 0 and 1: the lane's scores 0..7 and 8..15
        const i16x8_t pb0 = __builtin_bit_cast(i16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
        const i16x8_t pb1 = __builtin_bit_cast(i16x8_t, u32x4_t{pk[4], pk[5], pk[6], pk[7]});
        const MLA_LDS char* vr0 = vb + vrow * Sh::VP + 2 * vcol;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const i16x4_t a0 = lds_read_tr16(vr0 + (16 * ks) * Sh::VP + 64 * d);
            const i16x4_t a1 = lds_read_tr16(vr0 + (16 * ks + 8) * Sh::VP + 64 * d);
            const i16x8_t av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            o[d] = mfma_32x32x16(av, ks ? pb1 : pb0, o[d]);
          }
        }
      }
      if (t + 1 < ntiles) store_tile(SET ^ 1, kr2[SET ^ 1], vr2[SET ^ 1]);
      __syncthreads();
    };
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      tile_step(t, std::integral_constant<int, 0>{});
      tile_step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < ntiles) tile_step(t, std::integral_constant<int, 0>{});

    // a query's two lanes hold partial sums over their keys
    float lt = l + __shfl_xor(l, 32);
    if (qok) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* orow = (uint16_t*)p.out + (int64_t)(q0 + qi) * p.o_s0 + (int64_t)h * p.o_s1 + 4 * hh;
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const u32x2_t v = {pack_bf16x2(o[d][4 * bb] * inv, o[d][4 * bb + 1] * inv),
                             pack_bf16x2(o[d][4 * bb + 2] * inv, o[d][4 * bb + 3] * inv)};
          *(u32x2_t*)(orow + 32 * d + 8 * bb) = v;
        }
      if (p.lse && hh == 0)
        p.lse[(int64_t)(q0 + qi) * p.l_s0 + (int64_t)h * p.l_s1] =
            lt > 0.f ? (m + __log2f(lt)) * 0.69314718055994530942f : -__builtin_inff();
    }
  }
}

// Pair the query tiles of a causal call (the longest with the shortest) when
// the paired grid still has a workgroup for every CU: 16 causal query tiles
// of 64 heads (256/256, 2048 tokens) measured 350 -> 290 us paired, 16 tiles
// of 16 heads (192/128) 97 us unpaired against 103 us paired.
bool pair_query_tiles(const MhaParams& p, int ntq) {
  return p.causal && ntq > 1 && (int64_t)((ntq + 1) / 2) * p.n_heads * p.batch >= 256;
}

template <int DK, int DV>
hipError_t launch_mha_t(const MhaParams& p, hipStream_t s) {
  using Sh = MhaShape<DK, DV>;
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute((const void*)mha_fwd<DK, DV>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  MhaParams q = p;
  const int ntq = (int)((p.max_q + Sh::QT - 1) / Sh::QT);
  q.pair_tiles = pair_query_tiles(p, ntq);
  dim3 grid((unsigned)(q.pair_tiles ? (ntq + 1) / 2 : ntq), (unsigned)p.n_heads, (unsigned)p.batch);
  hipLaunchKernelGGL((mha_fwd<DK, DV>), grid, dim3(Sh::THREADS), Sh::LDS, s, q);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_mha32_t(const MhaParams& p, hipStream_t s) {
  using Sh = Mha32Shape<DK, DV>;
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute((const void*)mha_fwd32<DK, DV>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  MhaParams q = p;
  const int ntq = (int)((p.max_q + Sh::QT - 1) / Sh::QT);
  q.pair_tiles = pair_query_tiles(p, ntq);
  dim3 grid((unsigned)(q.pair_tiles ? (ntq + 1) / 2 : ntq), (unsigned)p.n_heads, (unsigned)p.batch);
  hipLaunchKernelGGL((mha_fwd32<DK, DV>), grid, dim3(Sh::THREADS), Sh::LDS, s, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bmm_nt(const BmmNtParams& p, hipStream_t s) {
  if (p.T == 0 || p.H == 0) return hipSuccess;
  const int64_t es = p.is_f32 ? 4 : 2;
  const bool aligned = ((uintptr_t)p.a % 16 == 0) && ((uintptr_t)p.w % 16 == 0) &&
                       (p.a_st * es % 16 == 0) && (p.a_sh * es % 16 == 0) &&
                       (p.w_sh * es % 16 == 0) && (p.w_sn * es % 16 == 0);
  // the 128 x 128 tile also writes 16-byte pieces of out rows
  const bool out_aligned = ((uintptr_t)p.out % 16 == 0) && (p.o_st * es % 16 == 0) &&
                           (p.o_sh * es % 16 == 0) && p.N % 8 == 0;
  if (!p.is_f32 && aligned && out_aligned && p.K % kNtK == 0 && p.K > 0 && p.N > 0 &&
      p.T >= kBigT && p.T <= INT32_MAX && p.K <= INT32_MAX) {
    dim3 grid((unsigned)((p.N + kGT - 1) / kGT), (unsigned)((p.T + kGT - 1) / kGT), (unsigned)p.H);
    hipLaunchKernelGGL(bmm_nt_big, grid, dim3(256), 0, s, p);
  } else if (!p.is_f32 && aligned && p.K % kNtK == 0 && p.K > 0 && p.N > 0) {
    dim3 grid((unsigned)((p.N + kNtN - 1) / kNtN), (unsigned)((p.T + kNtM - 1) / kNtM), (unsigned)p.H);
    hipLaunchKernelGGL(bmm_nt_bf16, grid, dim3(256), 0, s, p);
  } else if (p.is_f32 && aligned && p.K % 16 == 0 && p.K > 0 && p.N > 0 && p.T <= INT32_MAX) {
    dim3 grid((unsigned)((p.N + kNtN - 1) / kNtN), (unsigned)((p.T + kNtM - 1) / kNtM), (unsigned)p.H);
    hipLaunchKernelGGL(bmm_nt_f32, grid, dim3(256), 0, s, p);
  } else {
    const int64_t total = p.T * p.H * (p.N + p.R);
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (p.is_f32) hipLaunchKernelGGL(bmm_nt_plain<true>, dim3(blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(bmm_nt_plain<false>, dim3(blocks), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

bool mha_supported(int dk, int dv) {
  return (dk == 192 && dv == 128) || (dk == 256 && dv == 256) || (dk == 128 && dv == 128) ||
         (dk == 64 && dv == 64);
}

hipError_t launch_mha(const MhaParams& p, hipStream_t s) {
  if (p.batch == 0 || p.max_q == 0 || p.n_heads == 0) return hipSuccess;
  if (p.dk == 192 && p.dv == 128) return launch_mha32_t<192, 128>(p, s);
  if (p.dk == 256 && p.dv == 256) return launch_mha_t<256, 256>(p, s);
  if (p.dk == 128 && p.dv == 128) return launch_mha32_t<128, 128>(p, s);
  if (p.dk == 64 && p.dv == 64) return launch_mha32_t<64, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
