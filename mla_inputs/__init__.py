"""Seeded synthetic inputs for the MLA absorbed-decode workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the CPU oracle's tests and the HIP path's tests and
benchmark take their inputs from here, so the two sides see identical values.

Every tensor is drawn from numpy's PCG64 (``default_rng``) on its own stream
``seed * 1000 + k`` (k is a fixed per-tensor index), in float32, then rounded
to the device dtype (round-to-nearest-even through torch). Arrays are returned
as float32 numpy arrays that hold exactly the device values, so
``torch.from_numpy(x).to(dtype)`` is lossless and the oracle can widen the same
array to float64.

Workload recipes (shapes and distributions of the pages' tests; no public
dataset is involved, the pages use synthetic data throughout):

* tiny fp32 prefill+decode: 16 heads, d_nope 128, d_rope 64, d_v 128,
  kv_rank 512, t_q = t_kv = 64, batch 1; activations U[-1,1], weights
  U[-1/sqrt(512), 1/sqrt(512)] (memra-engine "tests/mla_gpu_forward.rs",
  `Case::new` scales), one contiguous 64-token page.
* latent cache write: 200 bf16 tokens of c_kv[512] + k_pe[64] ~ N(0,1),
  slots = the first 200 of a random permutation of 32 x 64 slots, written
  into the middle layer of a 3-layer block-major slot (vLLM
  "test_mla_cross_layer_kernel_equivalence.py",
  test_concat_and_cache_mla_into_unified_slot_view).
* V2-Lite decode bf16: 16 heads, W_UK_T [16,128,512], W_UV [16,512,128],
  batch 64, seqlens uniform on [512, 4096], 64-token pages, a random
  permutation block table, values N(0, 0.1^2).
* V3 decode bf16: 128 heads, entry 576 / v 512, batch 4, seqlen 4096 each,
  64-token pages, middle-layer view of a 3-layer block-major cache, q and KV
  N(0, 0.1^2) (test_flashmla_dense_decode_unified_slot_view geometry).
* NoPE absorbed prefill: 64 heads, d_nope 256, d_rope 0, d_v 256, kv_rank 512,
  t_q = t_kv = 2048 causal, batch 1, weights U[+-1/sqrt(512)], activations
  U[-1,1].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BF16 = "bf16"
F32 = "f32"
TORCH_DTYPE = {BF16: torch.bfloat16, F32: torch.float32}
# fp8 latent cache: OCP e4m3fn codes held as uint8 (the pages' torch.float8_e4m3fn)
FP8 = "fp8"
FP8_NAN = 0x7F


def fp8_codes(x) -> np.ndarray:
    """float32 values -> e4m3fn codes through torch's float8_e4m3fn conversion
    (how the pages build their fp8 caches)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def stream(seed: int, k: int) -> np.random.Generator:
    """The per-tensor random stream ``seed * 1000 + k``."""
    return np.random.default_rng(seed * 1000 + k)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the device dtype (RNE), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


def uniform(seed, k, shape, lo, hi, dtype) -> np.ndarray:
    return round_to(stream(seed, k).uniform(lo, hi, size=shape).astype(np.float32), dtype)


def normal(seed, k, shape, std, dtype) -> np.ndarray:
    return round_to((stream(seed, k).standard_normal(size=shape) * std).astype(np.float32), dtype)


@dataclass
class Dims:
    """MLA geometry in the pages' names (memra `MlaDims`)."""

    n_head: int
    d_nope: int
    d_rope: int
    d_v: int
    kv_rank: int

    @property
    def entry(self) -> int:
        return self.kv_rank + self.d_rope


V2_LITE = Dims(n_head=16, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
V3 = Dims(n_head=128, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
NOPE64 = Dims(n_head=64, d_nope=256, d_rope=0, d_v=256, kv_rank=512)


@dataclass
class DecodeCase:
    """Inputs of one paged absorbed-attention call (and optionally the folds).

    pool holds the physical pages [num_blocks, page, entry]; when ``n_layers``
    > 1 the pages are the middle layer of a block-major unified allocation
    ``unified`` [num_blocks, n_layers, page, entry] (the others hold
    ``neighbour_fill``)."""

    dims: Dims
    dtype: str
    batch: int
    q_len: int
    page: int
    seqlens: np.ndarray  # [B] int32
    block_table: np.ndarray  # [B, max_blocks] int32, -1 where unused
    pool: np.ndarray  # [num_blocks, page, entry] float32 (device values)
    q: np.ndarray  # [B, q_len, n_head, entry] folded query (q_lat | q_pe)
    scale: float
    causal: bool
    n_layers: int = 1
    layer: int = 0
    neighbour_fill: float = float("nan")
    extras: dict = field(default_factory=dict)
    kv_dtype: str = ""  # FP8: pool holds e4m3fn codes (uint8); else the value dtype
    descale_q: float = 1.0
    descale_k: float = 1.0

    @property
    def num_blocks(self) -> int:
        return self.pool.shape[0]

    @property
    def max_seqlen(self) -> int:
        return int(self.seqlens.max()) if self.seqlens.size else 0

    def unified(self) -> np.ndarray:
        """The block-major allocation [NB, n_layers, page, entry] with the
        pool in layer ``layer``."""
        NB, PG, E = self.pool.shape
        if self.kv_dtype == FP8:
            u = np.full((NB, self.n_layers, PG, E), FP8_NAN, dtype=np.uint8)
            u[:, self.layer] = self.pool
            return u
        u = np.full((NB, self.n_layers, PG, E), self.neighbour_fill, dtype=np.float32)
        u[:, self.layer] = self.pool
        return u


def paged_layout(seed, k, seqlens, page, num_blocks, max_blocks=None, permute=True):
    """Random block table: every sequence gets distinct physical blocks drawn
    from a permutation of the pool; entries past its last page are -1."""
    seqlens = np.asarray(seqlens, dtype=np.int64)
    need = [int(math.ceil(s / page)) for s in seqlens]
    if max_blocks is None:
        max_blocks = max([1] + need)
    if sum(need) > num_blocks:
        raise ValueError("pool too small for the sequences")
    order = stream(seed, k).permutation(num_blocks) if permute else np.arange(num_blocks)
    bt = np.full((len(seqlens), max_blocks), -1, dtype=np.int32)
    used = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[used: used + n]
        used += n
    return bt


def fill_pool(seed, k, num_blocks, page, entry, std, dtype, seqlens, block_table,
              tail_fill=float("nan"), dist="normal"):
    """Physical pages with valid rows drawn from the chosen distribution and
    every row that no sequence uses set to ``tail_fill`` (NaN by default, so a
    kernel that reads a stale row fails loudly)."""
    shape = (num_blocks, page, entry)
    if dist == "normal":
        pool = normal(seed, k, shape, std, dtype)
    else:
        pool = uniform(seed, k, shape, -std, std, dtype)
    valid = np.zeros((num_blocks, page), dtype=bool)
    for b, s in enumerate(np.asarray(seqlens)):
        for j in range(int(s)):
            valid[block_table[b, j // page], j % page] = True
    pool[~valid] = tail_fill
    return pool


def decode_case(seed, dims: Dims, dtype, seqlens, q_len=1, page=64, num_blocks=None,
                std=0.1, scale=None, causal=True, n_layers=1, layer=0,
                neighbour_fill=float("nan"), permute=True, tail_fill=float("nan"),
                max_blocks=None, dist="normal", kv_dtype="", descale_q=1.0,
                descale_k=1.0) -> DecodeCase:
    """A generic paged decode / chunked-prefill case. With kv_dtype FP8 the
    pool holds e4m3fn codes of the drawn values (rows no sequence uses hold
    the NaN code) and the case carries the decode's two descales."""
    seqlens = np.asarray(seqlens, dtype=np.int32)
    need = sum(int(math.ceil(int(s) / page)) for s in seqlens)
    if num_blocks is None:
        num_blocks = max(need, 1)
    bt = paged_layout(seed, 1, seqlens, page, num_blocks, max_blocks=max_blocks, permute=permute)
    if kv_dtype == FP8:
        vals = fill_pool(seed, 2, num_blocks, page, dims.entry, std, F32, seqlens, bt,
                         tail_fill=float("nan"), dist=dist)
        pool = fp8_codes(vals)
        pool[np.isnan(vals)] = FP8_NAN
    else:
        pool = fill_pool(seed, 2, num_blocks, page, dims.entry, std, dtype, seqlens, bt,
                         tail_fill=tail_fill, dist=dist)
    qshape = (len(seqlens), q_len, dims.n_head, dims.entry)
    q = normal(seed, 3, qshape, std, dtype) if dist == "normal" else uniform(
        seed, 3, qshape, -std, std, dtype)
    if scale is None:
        scale = dims.entry ** -0.5
    return DecodeCase(dims=dims, dtype=dtype, batch=len(seqlens), q_len=q_len, page=page,
                      seqlens=seqlens, block_table=bt, pool=pool, q=q, scale=float(scale),
                      causal=causal, n_layers=n_layers, layer=layer,
                      neighbour_fill=neighbour_fill, kv_dtype=kv_dtype,
                      descale_q=float(descale_q), descale_k=float(descale_k))


def mla_weights(seed, dims: Dims, dtype, dist="uniform", std=None):
    """W_UK_T [N, d_nope, kv_rank] and W_UV [N, kv_rank, d_v]. ``uniform``
    draws U[-1/sqrt(kv_rank), 1/sqrt(kv_rank)]; ``normal`` draws N(0, std^2)."""
    N, P, L, V = dims.n_head, dims.d_nope, dims.kv_rank, dims.d_v
    if dist == "uniform":
        ws = 1.0 / math.sqrt(L)
        w_uk_t = uniform(seed, 10, (N, P, L), -ws, ws, dtype)
        w_uv = uniform(seed, 11, (N, L, V), -ws, ws, dtype)
    else:
        w_uk_t = normal(seed, 10, (N, P, L), std, dtype)
        w_uv = normal(seed, 11, (N, L, V), std, dtype)
    return w_uk_t, w_uv


def mla_activations(seed, dims: Dims, t_q, t_kv, dtype, dist="uniform", std=1.0):
    """q_nope [t_q,N,P], q_pe [t_q,N,R], c_kv [t_kv,L], k_pe [t_kv,R]."""
    N, P, R, L = dims.n_head, dims.d_nope, dims.d_rope, dims.kv_rank
    draw = (lambda k, s: uniform(seed, k, s, -std, std, dtype)) if dist == "uniform" else (
        lambda k, s: normal(seed, k, s, std, dtype))
    return (draw(20, (t_q, N, P)), draw(21, (t_q, N, R)), draw(22, (t_kv, L)),
            draw(23, (t_kv, R)))


# --------------------------------------------------------------------------
# The named workloads.


def tiny_prefill_decode(seed=0):
    """Tiny fp32 absorbed MLA prefill + decode, one contiguous page."""
    d = V2_LITE
    T = 64
    q_nope, q_pe, c_kv, k_pe = mla_activations(seed, d, T, T, F32)
    w_uk_t, w_uv = mla_weights(seed, d, F32)
    return dict(dims=d, dtype=F32, t=T, q_nope=q_nope, q_pe=q_pe, c_kv=c_kv, k_pe=k_pe,
                w_uk_t=w_uk_t, w_uv=w_uv, scale=(d.d_nope + d.d_rope) ** -0.5, page=64)


def cache_write_case(seed=0, ntok=200, num_blocks=32, page=64, kv_rank=512, pe=64,
                     n_layers=3, layer=1, dtype=BF16):
    """Latent cache write into the middle layer of a block-major slot."""
    kv_c = normal(seed, 30, (ntok, kv_rank), 1.0, dtype)
    k_pe = normal(seed, 31, (ntok, pe), 1.0, dtype) if pe else np.zeros((ntok, 0), np.float32)
    slots = stream(seed, 32).permutation(num_blocks * page)[:ntok].astype(np.int64)
    entry = kv_rank + pe
    layer_elems = page * entry
    return dict(kv_c=kv_c, k_pe=k_pe, slots=slots, num_blocks=num_blocks, page=page,
                entry=entry, n_layers=n_layers, layer=layer, dtype=dtype,
                s0=n_layers * layer_elems, s1=entry, offset=layer * layer_elems,
                buf_shape=(num_blocks, n_layers * layer_elems))


def v2lite_decode(seed=0, batch=64, lo=512, hi=4096):
    """V2-Lite decode bf16 workload (paged, random table, NaN tails)."""
    seqlens = stream(seed, 40).integers(lo, hi, size=batch, endpoint=True).astype(np.int32)
    page = 64
    max_blocks = int(math.ceil(hi / page))
    c = decode_case(seed, V2_LITE, BF16, seqlens, q_len=1, page=page,
                    num_blocks=batch * max_blocks, std=0.1, causal=True, max_blocks=max_blocks)
    return c


def v3_decode(seed=0, batch=4, seqlen=4096, permute=False, neighbour_fill=float("nan")):
    """V3 decode bf16 workload: middle layer of a 3-layer block-major cache."""
    page = 64
    seqlens = np.full(batch, seqlen, dtype=np.int32)
    nb = batch * int(math.ceil(seqlen / page))
    return decode_case(seed, V3, BF16, seqlens, q_len=1, page=page, num_blocks=nb, std=0.1,
                       causal=True, n_layers=3, layer=1, neighbour_fill=neighbour_fill,
                       permute=permute)


def nope_prefill(seed=0, dtype=BF16, t=2048):
    """NoPE absorbed prefill: 64 heads x 256, rank 512, causal, one sequence."""
    d = NOPE64
    q_nope, _, c_kv, _ = mla_activations(seed, d, t, t, dtype)
    w_uk_t, w_uv = mla_weights(seed, d, dtype)
    return dict(dims=d, dtype=dtype, t=t, q_nope=q_nope, c_kv=c_kv, w_uk_t=w_uk_t, w_uv=w_uv,
                scale=(d.d_nope + d.d_rope) ** -0.5, page=64)


ROPE_BASE = 8_000_000.0  # the rotary base of the interleaved-rope gate


def rope_case(seed=0, n_pos=7, n_vec=5, d_rope=64, dtype=F32, pos_step=13, pos_offset=0):
    """Interleaved-rope inputs: x [n_pos, n_vec, d_rope] uniform in [-1, 1) and
    positions pos_offset + pos_step * p (the gate's shape: 7 positions 13 apart,
    5 vectors each)."""
    x = uniform(seed, 60, (n_pos, n_vec, d_rope), -1.0, 1.0, dtype)
    positions = (pos_offset + pos_step * np.arange(n_pos)).astype(np.int32)
    return x, positions


# --------------------------------------------------------------------------
# Sparse fp8 decode (656-byte entries: 512 e4m3 codes, 4 f32 scales, 64 bf16
# rope values), built the way the sparse-decode page builds its payload.
DSMLA_ENTRY = 656


def dsmla_payload(seed, num_blocks, page, std=0.1, scales="ones"):
    """[num_blocks, page, 656] uint8 entries: e4m3 codes of N(0, std^2) latent
    values, scales (all 1, or U[0.5, 2] per 128-code block), bf16 rope values
    N(0, std^2)."""
    nope = fp8_codes(stream(seed, 60).standard_normal((num_blocks, page, 512)) * std)
    if scales == "ones":
        sc = np.ones((num_blocks, page, 4), dtype=np.float32)
    else:
        sc = stream(seed, 61).uniform(0.5, 2.0, (num_blocks, page, 4)).astype(np.float32)
    rope = round_to((stream(seed, 62).standard_normal((num_blocks, page, 64)) * std)
                    .astype(np.float32), BF16)
    rope_bits = torch.from_numpy(rope).to(torch.bfloat16).view(torch.int16).numpy()
    payload = np.concatenate([nope.view(np.uint8), sc.view(np.uint8),
                              rope_bits.view(np.uint8)], axis=-1)
    assert payload.shape[-1] == DSMLA_ENTRY
    return np.ascontiguousarray(payload)


def dsmla_indices(seed, batch, q_len, topk, num_blocks, page, mode="disjoint", fill=0.75):
    """[batch, q_len, topk] int32 slot lists. ``disjoint``: sequence b takes the
    first topk slots of its own run of blocks, in order (the page's layout),
    padded with -1. ``random``: a random subset of ``fill * topk`` distinct slots
    in random order, the rest -1 at random positions."""
    idx = np.full((batch, q_len, topk), -1, dtype=np.int32)
    if mode == "disjoint":
        per = num_blocks // batch
        for b in range(batch):
            slots = np.arange(b * per * page, (b + 1) * per * page, dtype=np.int32)[:topk]
            idx[b, :, :slots.size] = slots
        return idx
    g = stream(seed, 63)
    n = int(fill * topk)
    for b in range(batch):
        for i in range(q_len):
            slots = g.permutation(num_blocks * page)[:n].astype(np.int32)
            pos = g.permutation(topk)[:n]
            idx[b, i, pos] = slots
    return idx
