"""GPU parity of mla_decode_attend against the double-precision oracle.

Cases follow vLLM "test_mla_cross_layer_kernel_equivalence.py" (paged dense
decode over a block-major cache view: 128 heads x 576 / v 512, 16-head FA3
geometry, page 64, scale 576^-0.5, causal) and memra-engine 0.124.1
"tests/mla_gpu_forward.rs" (queries as a causal suffix of the cache), at sizes
the oracle finishes in seconds and at the full benchmark shapes. Page tails
and unused pages are NaN, so any read of a row outside a sequence fails.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from helpers import assert_close, assert_lse_close, run_decode, say, to_np

pytestmark = pytest.mark.gpu

V2 = mi.V2_LITE
V3 = mi.V3
NOPE = mi.Dims(n_head=64, d_nope=256, d_rope=0, d_v=256, kv_rank=512)


def oracle_of(case):
    return oracle.attend_paged(case.q, case.pool, case.block_table, case.seqlens, case.scale,
                               case.causal, case.dims.kv_rank)


def check(case, what, block_major=False):
    say(f"[decode] {what}: B={case.batch} Sq={case.q_len} N={case.dims.n_head} "
        f"E={case.dims.entry} page={case.page} dtype={case.dtype} seqlens={case.seqlens.tolist()[:8]}")
    out, lse = run_decode(case, block_major=block_major)
    want_o, want_lse = oracle_of(case)
    got_o = to_np(out)
    got_l = to_np(lse)
    # rows with no visible key must be exactly zero with lse -inf
    dead = np.isneginf(want_lse)
    if dead.any():
        assert np.all(got_o[dead] == 0.0), f"{what}: rows with no visible key are not zero"
    if (~dead).any():
        assert_close(got_o[~dead], want_o[~dead], case.dtype, what)
    assert_lse_close(got_l, want_lse, what)
    return out, lse


# --------------------------------------------------------------- few heads


@pytest.mark.parametrize("rope", [64, 0])
def test_few_heads_ragged(rope):
    d = mi.Dims(n_head=16, d_nope=128, d_rope=rope, d_v=128, kv_rank=512)
    c = mi.decode_case(1, d, "bf16", [1, 77, 300, 64, 1000])
    check(c, f"16 heads ragged rope={rope}")


def test_few_heads_single_long_sequence():
    c = mi.decode_case(2, V2, "bf16", [4096])
    check(c, "16 heads one 4096-token sequence")


def test_few_heads_empty_and_tiny_sequences():
    c = mi.decode_case(3, V2, "bf16", [0, 1, 2, 15, 16, 17, 0])
    out, lse = check(c, "16 heads with empty sequences")
    o = to_np(out)
    assert np.all(o[0] == 0) and np.all(o[6] == 0)
    assert np.all(np.isneginf(to_np(lse)[0]))


def test_fewer_heads_than_a_tile():
    d = mi.Dims(n_head=4, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    c = mi.decode_case(4, d, "bf16", [33, 500], q_len=2)
    check(c, "4 heads x 2 queries")


# ------------------------------------------------- 17 to 32 rows per unit


@pytest.mark.parametrize("rope", [64, 0])
def test_32_rows_ragged(rope):
    # 32 heads x 1 query: units of 32 rows, whose two waves per row group split
    # the score contraction and add the partial scores through LDS
    d = mi.Dims(n_head=32, d_nope=128, d_rope=rope, d_v=128, kv_rank=512)
    c = mi.decode_case(16, d, "bf16", [5, 333, 1200, 64, 2])
    check(c, f"32 heads ragged rope={rope}")


def test_32_rows_from_two_queries():
    # 16 heads x 2 queries: 32 rows per unit spanning two causal query positions
    d = mi.Dims(n_head=16, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    c = mi.decode_case(17, d, "bf16", [1, 2, 3, 700, 1500], q_len=2)
    check(c, "16 heads x 2 queries")


def test_24_rows_partial_unit():
    # 24 heads: the unit's last 8 rows are padding
    d = mi.Dims(n_head=24, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    c = mi.decode_case(18, d, "bf16", [100, 2000, 31])
    check(c, "24 heads")


# --------------------------------------------------------------- many heads


@pytest.mark.parametrize("rope", [64, 0])
def test_many_heads_ragged(rope):
    d = mi.Dims(n_head=128, d_nope=128, d_rope=rope, d_v=128, kv_rank=512)
    c = mi.decode_case(5, d, "bf16", [50, 700, 1])
    check(c, f"128 heads ragged rope={rope}")


@pytest.mark.parametrize("nseq", [24, 48])
def test_many_heads_many_tiny_sequences(nseq):
    # 128 heads over many sequences of 1 to 100 keys: the split plan gives most
    # workgroups several units, so their tile loops cross segment boundaries
    # (a new unit's query rows read between two tiles). 24 sequences take
    # 32-row units, 48 take 64-row units.
    d = mi.Dims(n_head=128, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    lens = [[1, 2, 3, 31, 32, 33, 64, 65, 100][i % 9] for i in range(nseq)]
    c = mi.decode_case(40 + nseq, d, "bf16", lens)
    check(c, f"128 heads x {nseq} tiny sequences")


def test_many_heads_page16_tiles_span_pages():
    c = mi.decode_case(6, V3, "bf16", [300, 129], page=16)
    check(c, "128 heads page 16")


def test_chunked_prefill_causal_suffix():
    d = mi.Dims(n_head=64, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    c = mi.decode_case(7, d, "bf16", [40, 100, 257], q_len=40)
    check(c, "64 heads x 40 queries causal suffix")


def test_more_queries_than_keys():
    d = mi.Dims(n_head=16, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    c = mi.decode_case(8, d, "bf16", [2, 10], q_len=4)
    out, lse = check(c, "queries before the first key")
    assert np.all(to_np(out)[0, :2] == 0)


def test_non_causal_multi_query():
    d = mi.Dims(n_head=32, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    c = mi.decode_case(9, d, "bf16", [90, 333], q_len=3, causal=False)
    check(c, "non-causal 3 queries")


def test_prefill_many_units_split():
    # 300 queries x 64 heads = 300 units of 64 rows, split over 256 workgroups
    c = mi.decode_case(10, NOPE, "bf16", [300], q_len=300, dist="uniform", std=1.0,
                       scale=1.0 / 16)
    check(c, "NoPE prefill 300 x 64 heads")


def test_prefill_many_units_no_split():
    # 1100 queries x 64 heads = 1100 units of 64 rows, past the 1024 units a
    # split plan holds: one workgroup per unit
    c = mi.decode_case(10, NOPE, "bf16", [1100], q_len=1100, dist="uniform", std=1.0,
                       scale=1.0 / 16)
    check(c, "NoPE prefill 1100 x 64 heads")


def test_long_sequence_past_the_staged_block_table():
    # 1100 sequences (one unit each, no split): the long one has 1250 pages of
    # 16 tokens, more than the 1024 block-table entries a workgroup stages, so
    # its last pages come through the loader's direct block-table reads
    rng = mi.stream(19, 0)
    seqlens = rng.integers(1, 41, size=1100).astype(np.int32)
    seqlens[777] = 20_000
    c = mi.decode_case(19, V2, "bf16", seqlens, page=16)
    check(c, "1100 sequences, one of 1250 pages")


def test_split_300_sequences_one_long():
    # 300 units (more than the 256 workgroups of a split grid): short
    # sequences and one of 8000 tokens, whose keys spread over many workgroups
    rng = mi.stream(23, 0)
    seqlens = rng.integers(0, 200, size=300).astype(np.int32)
    seqlens[123] = 8000
    c = mi.decode_case(23, V2, "bf16", seqlens)
    check(c, "300 sequences, one of 8000 tokens")


def test_split_1023_units_page16():
    # the largest split plan (16 units per planning lane, every bit of the
    # live/partial masks in use), empty sequences among them, pages of 16
    rng = mi.stream(24, 0)
    seqlens = rng.integers(0, 60, size=1023).astype(np.int32)
    seqlens[::97] = 0
    seqlens[1000] = 3000
    seqlens[5] = 2000
    c = mi.decode_case(24, V2, "bf16", seqlens, page=16)
    check(c, "1023 sequences, pages of 16")


def test_split_many_heads_two_units_per_sequence():
    # 128 heads over 64-row units: 2 units per sequence, 800 units in a split plan
    rng = mi.stream(25, 0)
    seqlens = rng.integers(1, 120, size=400).astype(np.int32)
    seqlens[0] = 3000
    c = mi.decode_case(25, V3, "bf16", seqlens)
    check(c, "400 sequences x 128 heads")


# -------------------------------------------------------------------- fp32


@pytest.mark.parametrize("rope", [64, 0])
def test_fp32(rope):
    d = mi.Dims(n_head=16, d_nope=128, d_rope=rope, d_v=128, kv_rank=512)
    c = mi.decode_case(11, d, "f32", [1, 64, 200], q_len=1, dist="uniform", std=1.0,
                       scale=192 ** -0.5)
    check(c, f"fp32 rope={rope}")


def test_fp32_prefill_tiny_config():
    # tiny fp32 prefill: 16 heads, t_q = t_kv = 64, one contiguous page
    c = mi.decode_case(12, V2, "f32", [64], q_len=64, dist="uniform", std=1.0,
                       scale=192 ** -0.5, permute=False)
    check(c, "fp32 prefill 64x64")


# --------------------------------------------------- layout and determinism


def test_block_major_view_bit_identical_to_contiguous():
    c = mi.decode_case(13, V3, "bf16", [1024, 1024, 1024, 1024], n_layers=3, layer=1)
    out_c, lse_c = run_decode(c, block_major=False)
    out_v, lse_v = run_decode(c, block_major=True)
    assert torch.equal(out_c.view(torch.int16), out_v.view(torch.int16))
    assert torch.equal(lse_c, lse_v)
    assert torch.isfinite(out_c.float()).all() and out_c.float().abs().max() > 0


def test_reruns_bit_identical():
    c = mi.decode_case(14, V2, "bf16", [700, 1500, 64])
    a, la = run_decode(c)
    for _ in range(3):
        b, lb = run_decode(c)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(la, lb)


def test_output_views_and_no_lse():
    # out written through a transposed view; lse omitted
    import mla_absorbed_decode_amd as mla
    from helpers import DeviceCache, dev, to_dev

    c = mi.decode_case(15, V2, "bf16", [100, 260])
    q = to_dev(c.q, "bf16")
    cache = DeviceCache(c, False)
    bt = torch.from_numpy(c.block_table).to(dev())
    sl = torch.from_numpy(c.seqlens).to(dev())
    store = torch.full((c.dims.n_head, c.batch, 1, 512), float("nan"), dtype=torch.bfloat16,
                       device=dev())
    out = store.permute(1, 2, 0, 3)  # [B, 1, N, L] view, not contiguous
    mla.mla_decode_attend(q, cache.view, bt, sl, c.max_seqlen, c.scale, True, out, None)
    torch.cuda.synchronize()
    want, _ = oracle_of(c)
    assert_close(to_np(out), want, "bf16", "transposed out view")


# ---------------------------------------------------------------- full size


def test_v2lite_full_config():
    c = mi.v2lite_decode(seed=0)
    check(c, "V2-Lite decode B=64 full")


def test_v3_full_config_block_major():
    c = mi.v3_decode(seed=0)
    out_v, lse_v = check(c, "V3 decode B=4 x 4096 block-major view", block_major=True)
    out_c, lse_c = run_decode(c, block_major=False)
    assert torch.equal(out_c.view(torch.int16), out_v.view(torch.int16))


def test_v3_full_config_permuted_block_table():
    # the same geometry with the pages in random pool order (a permuted block
    # table), element by element against the oracle, and bit-identical between
    # the block-major view and a contiguous copy
    c = mi.v3_decode(seed=1, permute=True)
    assert not np.array_equal(np.sort(c.block_table.ravel()), c.block_table.ravel())
    out_v, _ = check(c, "V3 decode B=4 x 4096 permuted pages, block-major view", block_major=True)
    out_c, _ = run_decode(c, block_major=False)
    assert torch.equal(out_c.view(torch.int16), out_v.view(torch.int16))


@pytest.mark.parametrize("seqlens", [[4096, 3000], [5000]])
def test_many_splits_per_unit(seqlens):
    # 128 heads over one or two sequences: 4 or 8 units of 32 rows split 64 or
    # 32 ways over the grid, past the 16 splits the merge reads in one batch
    c = mi.decode_case(26, V3, "bf16", seqlens)
    check(c, f"128 heads, {len(seqlens)} sequences, many splits per unit")


def test_workspace_reused_across_calls():
    # one uninitialised workspace serves a sequence of calls of different plans
    import mla_absorbed_decode_amd as mla
    from helpers import DeviceCache, dev, to_dev

    cases = [mi.decode_case(s, V2, "bf16", sl, max_blocks=40)
             for s, sl in ((21, [2500, 90, 700, 1300]), (22, [64, 2000, 2048, 5]),
                           (21, [2500, 90, 700, 1300]))]
    nbytes = mla.mla_decode_workspace_size(4, 1, 16, 512, 2560, 64, torch.bfloat16)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=dev())
    outs = []
    for i, c in enumerate(cases):
        say(f"[decode] workspace reuse call {i}")
        out = torch.empty(4, 1, 16, 512, dtype=torch.bfloat16, device=dev())
        mla.mla_decode_attend(to_dev(c.q, "bf16"), DeviceCache(c, False).view,
                              torch.from_numpy(c.block_table).to(dev()),
                              torch.from_numpy(c.seqlens).to(dev()), 2560, c.scale, True, out,
                              None, workspace=ws)
        torch.cuda.synchronize()
        want, _ = oracle_of(c)
        assert_close(to_np(out), want, "bf16", f"workspace reuse call {i}")
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))


def test_rendezvous_give_up_marks_rows_nan(monkeypatch):
    # The few-head layout's compute waves meet on a bounded LDS counter wait.
    # With the bound forced to zero polls a wave that arrives before the others
    # gives up at once: every output row must then be either the right value or
    # NaN (with a NaN lse), never a silently wrong value.
    monkeypatch.setenv("MLA_RENDEZVOUS_POLLS", "0")
    c = mi.decode_case(30, V2, "bf16", [700, 1500, 64, 300, 2222])
    say("[decode] rendezvous forced to give up (0 polls)")
    out, lse = run_decode(c)
    want_o, want_l = oracle_of(c)
    o, l = to_np(out), to_np(lse)
    bad = np.isnan(o).any(axis=-1)
    assert np.array_equal(bad, np.isnan(o).all(axis=-1)), "partly NaN rows"
    assert np.array_equal(bad, np.isnan(l)), "NaN rows and NaN lse differ"
    if (~bad).any():
        assert_close(o[~bad], want_o[~bad], "bf16", "rows that completed")
        assert_lse_close(l[~bad], want_l[~bad], "rows that completed")
    monkeypatch.delenv("MLA_RENDEZVOUS_POLLS")
    out2, _ = run_decode(c)  # the default bound again: a normal, finite result
    assert_close(to_np(out2), want_o, "bf16", "after the forced give-up")
