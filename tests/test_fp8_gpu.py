"""GPU parity of the fp8 latent cache against the double-precision oracle.

vLLM "test_mla_cross_layer_kernel_equivalence.py" holds the dense decode
cache as torch.float8_e4m3fn and passes descale_q / descale_k
(test_flashmla_dense_fp8_decode_unified_slot_view: 128 heads x 576 / v 512,
page 64, bs 4, a unified-slot block-major view read bit-identically to a
contiguous cache); concat_and_cache_mla takes the cache dtype and a scale.
The write must equal the oracle's codes bit for bit; the decode meets the
bf16 bar (every e4m3 value is exact in bf16, so the device arithmetic is the
bf16 decode's). Unused cache rows hold the e4m3 NaN code, so any read of a
row outside a sequence fails.
"""
import numpy as np
import pytest
import torch

import mla_absorbed_decode_amd as mla
import mla_inputs as mi
import oracle
from helpers import assert_close, assert_lse_close, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

V2 = mi.V2_LITE
V3 = mi.V3


def fp8_dev(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(dev()).view(
        torch.float8_e4m3fn)


def scalar(x: float) -> torch.Tensor:
    return torch.tensor([x], dtype=torch.float32, device=dev())


# ----------------------------------------------------------------- write


def special_rows(T, E, scale, rng):
    """Rows whose quotients x / scale hit e4m3 ties, subnormals, the largest
    code, saturation, infinities, NaN and signed zeros, mixed with N(0, 1)."""
    pos = oracle.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    specials = np.concatenate([mids, -mids, pos, -pos, [448.0, 449.0, 1e6, -1e6, np.inf, -np.inf,
                                                        np.nan, 0.0, -0.0, 1e-12, -1e-12]])
    x = rng.standard_normal((T, E)).astype(np.float32) * 3
    flat = x.reshape(-1)
    idx = rng.choice(flat.size, size=specials.size, replace=False)
    flat[idx] = (specials * scale).astype(np.float32)
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fp8_cache_write_bit_exact(dtype):
    rng = np.random.default_rng(40)
    T, L, R, NB, PG, layers, layer = 300, 512, 64, 16, 64, 3, 1
    E = L + R
    scale = np.float32(0.37)
    rows = mi.round_to(special_rows(T, E, scale, rng), dtype)
    slots = rng.permutation(NB * PG)[:T].astype(np.int64)
    slots[5] = -1
    slots[9] = NB * PG + 3
    say(f"[fp8] cache write {dtype}: T={T} view of a {layers}-layer allocation")
    alloc = rng.integers(0, 256, size=(NB, layers, PG, E)).astype(np.uint8)
    cache = fp8_dev(alloc)
    view = cache[:, layer]
    kv_c = to_dev(rows[:, :L], dtype)
    k_pe = to_dev(rows[:, L:], dtype)
    mla.mla_concat_and_cache_fp8(kv_c, k_pe, torch.from_numpy(slots).to(dev()), view,
                                 scalar(float(scale)))
    torch.cuda.synchronize()
    got = cache.view(torch.uint8).cpu().numpy()
    want = oracle.cache_write_fp8(alloc, np.asarray(rows[:, :L]), np.asarray(rows[:, L:]), slots,
                                  scale, layer * PG * E, NB, PG, layers * PG * E, E)
    assert np.array_equal(got, want)


def test_fp8_cache_write_unaligned_rows_and_int32_slots():
    # kv_c rows at an odd element offset: the one-element path
    rng = np.random.default_rng(41)
    T, L, R, NB, PG = 40, 512, 64, 4, 16
    E = L + R
    scale = np.float32(2.5)
    rows = mi.round_to(special_rows(T, E, scale, rng), "bf16")
    slots = rng.permutation(NB * PG)[:T].astype(np.int32)
    say(f"[fp8] cache write unaligned rows T={T}")
    big = to_dev(np.pad(rows[:, :L], ((0, 0), (1, 0))), "bf16")
    kv_c = big[:, 1:]
    k_pe = to_dev(rows[:, L:], "bf16")
    alloc = np.full((NB, PG, E), 0x55, dtype=np.uint8)
    cache = fp8_dev(alloc)
    mla.mla_concat_and_cache_fp8(kv_c, k_pe, torch.from_numpy(slots).to(dev()), cache,
                                 scalar(float(scale)))
    torch.cuda.synchronize()
    want = oracle.cache_write_fp8(alloc, rows[:, :L], rows[:, L:], slots.astype(np.int64), scale,
                                  0, NB, PG, PG * E, E)
    assert np.array_equal(cache.view(torch.uint8).cpu().numpy(), want)


# ---------------------------------------------------------------- decode


def run_fp8(case, block_major=False, workspace=None):
    c = case
    q = to_dev(c.q, "bf16")
    if block_major and c.n_layers > 1:
        alloc = fp8_dev(c.unified())
        view = alloc[:, c.layer]
        assert not view.is_contiguous()
    else:
        view = fp8_dev(c.pool)
    bt = torch.from_numpy(c.block_table).to(dev())
    sl = torch.from_numpy(c.seqlens).to(dev())
    out = torch.full((c.batch, c.q_len, c.dims.n_head, c.dims.kv_rank), float("nan"),
                     dtype=torch.bfloat16, device=dev())
    lse = torch.full((c.batch, c.q_len, c.dims.n_head), float("nan"), dtype=torch.float32,
                     device=dev())
    mla.mla_decode_attend_fp8(q, view, bt, sl, c.max_seqlen, c.scale, c.causal,
                              scalar(c.descale_q), scalar(c.descale_k), out, lse,
                              workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def check(case, what, block_major=False):
    say(f"[fp8] {what}: B={case.batch} Sq={case.q_len} N={case.dims.n_head} E={case.dims.entry} "
        f"page={case.page} descales=({case.descale_q}, {case.descale_k}) "
        f"seqlens={case.seqlens.tolist()[:8]}")
    out, lse = run_fp8(case, block_major)
    want_o, want_l = oracle.attend_paged_fp8(case.q, case.pool, case.block_table, case.seqlens,
                                             case.scale, case.causal, case.dims.kv_rank,
                                             case.descale_q, case.descale_k)
    got_o, got_l = to_np(out), to_np(lse)
    dead = np.isneginf(want_l)
    if dead.any():
        assert np.all(got_o[dead] == 0.0), f"{what}: rows with no visible key are not zero"
    if (~dead).any():
        assert_close(got_o[~dead], want_o[~dead], "bf16", what)
    assert_lse_close(got_l, want_l, what)
    return out, lse


@pytest.mark.parametrize("rope", [64, 0])
def test_fp8_few_heads_ragged(rope):
    d = mi.Dims(n_head=16, d_nope=128, d_rope=rope, d_v=128, kv_rank=512)
    c = mi.decode_case(50, d, "bf16", [1, 77, 300, 64, 1000, 0], kv_dtype=mi.FP8)
    check(c, f"16 heads ragged rope={rope}")


def test_fp8_descales_and_wide_values():
    # values over most of the e4m3 range (subnormals to hundreds), scaled back
    # by the descales
    c = mi.decode_case(51, V2, "bf16", [33, 500, 1200], kv_dtype=mi.FP8, std=40.0,
                       descale_q=0.02, descale_k=0.01)
    check(c, "descales 0.02 / 0.01, cache std 40")


def test_fp8_many_heads_and_two_queries():
    d = mi.Dims(n_head=128, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    c = mi.decode_case(52, d, "bf16", [50, 700, 1], kv_dtype=mi.FP8, q_len=2)
    check(c, "128 heads x 2 queries")


def test_fp8_page16_and_long_sequence_past_the_stage():
    rng = mi.stream(53, 0)
    seqlens = rng.integers(1, 41, size=256).astype(np.int32)
    seqlens[77] = 20_000
    c = mi.decode_case(53, V2, "bf16", seqlens, page=16, kv_dtype=mi.FP8)
    check(c, "256 sequences, one of 1250 pages of 16")


def test_fp8_v3_full_config_block_major_bit_identical():
    # the page's dense fp8 case: 128 heads, bs 4 x 1024 tokens, 3-layer unified slot
    c = mi.decode_case(54, V3, "bf16", [1024, 1024, 1024, 1024], kv_dtype=mi.FP8, n_layers=3,
                       layer=1)
    out_v, lse_v = check(c, "V3 128 heads, block-major view", block_major=True)
    out_c, lse_c = run_fp8(c, block_major=False)
    assert torch.equal(out_c.view(torch.int16), out_v.view(torch.int16))
    assert torch.equal(lse_c, lse_v)


def test_fp8_v2lite_full_config_and_reruns():
    rng = mi.stream(55, 0)
    seqlens = rng.integers(512, 4097, size=64).astype(np.int32)
    c = mi.decode_case(55, V2, "bf16", seqlens, kv_dtype=mi.FP8)
    out, lse = check(c, "V2-Lite decode B=64 fp8")
    for _ in range(2):
        o2, l2 = run_fp8(c)
        assert torch.equal(out.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(lse, l2)


def test_fp8_write_then_decode_matches_oracle_end_to_end():
    # rows written by mla_concat_and_cache_fp8, then decoded: against the
    # oracle's write followed by its fp8 decode
    rng = np.random.default_rng(56)
    d = mi.Dims(n_head=16, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    B, PG, NB = 3, 64, 32
    seqlens = np.array([100, 513, 900], dtype=np.int32)
    bt = mi.paged_layout(56, 1, seqlens, PG, NB)
    slots = np.concatenate([bt[b, np.arange(s) // PG].astype(np.int64) * PG + np.arange(s) % PG
                            for b, s in enumerate(seqlens)])
    rows = mi.normal(56, 2, (slots.size, d.entry), 0.5, "bf16")
    scale = np.float32(0.05)
    say(f"[fp8] write then decode: {slots.size} rows")
    alloc = np.full((NB, PG, d.entry), mi.FP8_NAN, dtype=np.uint8)
    cache = fp8_dev(alloc)
    mla.mla_concat_and_cache_fp8(to_dev(rows[:, :512], "bf16"), to_dev(rows[:, 512:], "bf16"),
                                 torch.from_numpy(slots).to(dev()), cache, scalar(float(scale)))
    codes = oracle.cache_write_fp8(alloc, rows[:, :512], rows[:, 512:], slots, scale, 0, NB, PG,
                                   PG * d.entry, d.entry)
    torch.cuda.synchronize()
    assert np.array_equal(cache.view(torch.uint8).cpu().numpy(), codes)
    q = mi.normal(56, 3, (B, 1, d.n_head, d.entry), 0.1, "bf16")
    case = mi.DecodeCase(dims=d, dtype="bf16", batch=B, q_len=1, page=PG, seqlens=seqlens,
                         block_table=bt, pool=codes, q=q, scale=d.entry ** -0.5, causal=True,
                         kv_dtype=mi.FP8, descale_q=1.0, descale_k=float(scale))
    check(case, "decode of the written cache, descale_k = write scale")
