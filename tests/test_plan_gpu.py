"""GPU tests of the shared split plan: mla_decode_plan once, then planned
attention calls, one per layer.

[P3] "dense decode" tests compute the tile-scheduler metadata and split count
once from the cache sequence lengths and hand them to every layer's decode
call. Here the plan kernel writes each attention workgroup's share once; the
planned calls must give results bit-identical to the unplanned calls (which
the decode tests hold against the oracle element by element), and one case
is checked against the oracle directly. Calls whose sizes differ from the
plan's header, and workgroup shares too large for a descriptor, plan in the
kernel as before.
"""
import numpy as np
import pytest
import torch

import mla_absorbed_decode_amd as mla
import mla_inputs as mi
import oracle
from helpers import DeviceCache, assert_close, assert_lse_close, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

V2 = mi.V2_LITE
V3 = mi.V3
NOPE = mi.Dims(n_head=64, d_nope=256, d_rope=0, d_v=256, kv_rank=512)


def _inputs(c, block_major=False):
    cache = DeviceCache(c, block_major)
    return (to_dev(c.q, c.dtype), cache, torch.from_numpy(c.block_table).to(dev()),
            torch.from_numpy(c.seqlens).to(dev()))


def _outputs(c):
    td = mi.TORCH_DTYPE[c.dtype]
    out = torch.full((c.batch, c.q_len, c.dims.n_head, c.dims.kv_rank), float("nan"), dtype=td,
                     device=dev())
    lse = torch.full((c.batch, c.q_len, c.dims.n_head), float("nan"), dtype=torch.float32,
                     device=dev())
    return out, lse


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(a, b, what):
    assert torch.equal(_bits(a), _bits(b)), f"{what}: planned and unplanned results differ"


def _unplanned(c, q, cache_view, bt, sl, causal=None, max_seqlen=None):
    out, lse = _outputs(c)
    mla.mla_decode_attend(q, cache_view, bt, sl, c.max_seqlen if max_seqlen is None else max_seqlen,
                          c.scale, c.causal if causal is None else causal, out, lse)
    return out, lse


def _planned(c, q, cache_view, bt, sl, plan, causal=None, max_seqlen=None):
    out, lse = _outputs(c)
    mla.mla_decode_attend_planned(q, cache_view, bt, sl,
                                  c.max_seqlen if max_seqlen is None else max_seqlen, c.scale,
                                  c.causal if causal is None else causal, out, plan, lse)
    return out, lse


def _cases():
    rng = mi.stream(23, 0)
    s300 = rng.integers(0, 200, size=300).astype(np.int32)
    s300[123] = 8000
    rng = mi.stream(24, 0)
    s1023 = rng.integers(0, 60, size=1023).astype(np.int32)
    s1023[::97] = 0
    s1023[1000] = 3000
    s1023[5] = 2000
    rng = mi.stream(25, 0)
    s400 = rng.integers(1, 120, size=400).astype(np.int32)
    s400[0] = 3000
    few0 = mi.Dims(n_head=16, d_nope=128, d_rope=0, d_v=128, kv_rank=512)
    h32 = mi.Dims(n_head=32, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    h128_0 = mi.Dims(n_head=128, d_nope=128, d_rope=0, d_v=128, kv_rank=512)
    f32 = mi.Dims(n_head=16, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    return {
        "V2-Lite B=64": lambda: mi.v2lite_decode(seed=0),
        "V3 B=4 x 4096": lambda: mi.v3_decode(seed=0),
        "300 sequences one of 8000": lambda: mi.decode_case(23, V2, "bf16", s300),
        "1023 sequences page 16": lambda: mi.decode_case(24, V2, "bf16", s1023, page=16),
        "400 sequences x 128 heads": lambda: mi.decode_case(25, V3, "bf16", s400),
        "16 heads rope 0": lambda: mi.decode_case(1, few0, "bf16", [1, 77, 300, 64, 1000]),
        "32 heads": lambda: mi.decode_case(16, h32, "bf16", [5, 333, 1200, 64, 2]),
        "128 heads rope 0": lambda: mi.decode_case(5, h128_0, "bf16", [50, 700, 1]),
        "16 heads x 2 queries": lambda: mi.decode_case(17, f32, "bf16", [1, 2, 3, 700, 1500],
                                                       q_len=2),
        "fp32": lambda: mi.decode_case(11, f32, "f32", [1, 64, 200], dist="uniform", std=1.0,
                                       scale=192 ** -0.5),
        "NoPE prefill 300 x 64 heads": lambda: mi.decode_case(10, NOPE, "bf16", [300], q_len=300,
                                                              dist="uniform", std=1.0,
                                                              scale=1.0 / 16),
    }


CASES = _cases()


@pytest.mark.parametrize("name", list(CASES))
def test_planned_bit_identical_to_unplanned(name):
    c = CASES[name]()
    say(f"[plan] {name}: B={c.batch} Sq={c.q_len} N={c.dims.n_head} E={c.dims.entry} "
        f"page={c.page} dtype={c.dtype}")
    q, cache, bt, sl = _inputs(c)
    want_o, want_l = _unplanned(c, q, cache.view, bt, sl)
    plan = mla.mla_decode_plan(q, cache.view, bt, sl, c.max_seqlen, c.causal)
    assert plan is not None, "a split call has a plan"
    got_o, got_l = _planned(c, q, cache.view, bt, sl, plan)
    again_o, again_l = _planned(c, q, cache.view, bt, sl, plan)  # the plan is read, not used up
    torch.cuda.synchronize()
    _same(got_o, want_o, name)
    _same(got_l, want_l, name + " lse")
    _same(again_o, want_o, name + " (second planned call)")


def test_planned_against_oracle():
    c = CASES["300 sequences one of 8000"]()
    say("[plan] 300 sequences against the oracle")
    q, cache, bt, sl = _inputs(c)
    plan = mla.mla_decode_plan(q, cache.view, bt, sl, c.max_seqlen, c.causal)
    out, lse = _planned(c, q, cache.view, bt, sl, plan)
    torch.cuda.synchronize()
    want_o, want_l = oracle.attend_paged(c.q, c.pool, c.block_table, c.seqlens, c.scale, c.causal,
                                         c.dims.kv_rank)
    dead = np.isneginf(want_l)
    got_o = to_np(out)
    assert np.all(got_o[dead] == 0.0)
    assert_close(got_o[~dead], want_o[~dead], c.dtype, "planned 300 sequences")
    assert_lse_close(to_np(lse), want_l, "planned 300 sequences")


def test_one_plan_serves_every_layer():
    # the middle of three layers of a block-major cache is the usual view; here
    # each layer is attended with the one plan made from the shared tables
    c = mi.v3_decode(seed=2, permute=True)
    say("[plan] one plan for three layers, V3 B=4 x 4096 block-major")
    q, cache, bt, sl = _inputs(c, block_major=True)
    # the other layers' rows: values of their own (the case fills them with NaN)
    cache.alloc[:, 0] = -cache.alloc[:, 1]
    cache.alloc[:, 2] = cache.alloc[:, 1].roll(1, dims=-1)
    plan = mla.mla_decode_plan(q, cache.view, bt, sl, c.max_seqlen, c.causal)
    outs = []
    for layer in range(c.n_layers):
        view = cache.alloc[:, layer]
        want_o, want_l = _unplanned(c, q, view, bt, sl)
        got_o, got_l = _planned(c, q, view, bt, sl, plan)
        torch.cuda.synchronize()
        _same(got_o, want_o, f"layer {layer}")
        _same(got_l, want_l, f"layer {layer} lse")
        assert torch.isfinite(got_o.float()).all()
        outs.append(got_o)
    assert not torch.equal(outs[0], outs[2])


def test_plan_for_other_sizes_is_ignored():
    # a plan's header names the sizes it was made for: a call with other sizes
    # (here the causal flag, which moves the first query's keys) plans for itself
    d = mi.Dims(n_head=16, d_nope=128, d_rope=64, d_v=128, kv_rank=512)
    c = mi.decode_case(31, d, "bf16", [5, 700, 1500, 90], q_len=2)
    say("[plan] header mismatch: causal plan, non-causal call")
    q, cache, bt, sl = _inputs(c)
    cap = c.max_seqlen + 32  # a later call's larger max_seqlen (a larger grid here)
    assert cap <= c.block_table.shape[1] * c.page
    nbytes = max(mla.mla_decode_plan_size(c.batch, 2, 16, 512, m, c.page, torch.bfloat16)
                 for m in (c.max_seqlen, cap))
    plan = torch.empty(nbytes, dtype=torch.uint8, device=dev())
    mla.mla_decode_plan(q, cache.view, bt, sl, c.max_seqlen, True, plan)
    want_nc, want_nc_l = _unplanned(c, q, cache.view, bt, sl, causal=False)
    got_nc, got_nc_l = _planned(c, q, cache.view, bt, sl, plan, causal=False)
    want_c, _ = _unplanned(c, q, cache.view, bt, sl, causal=True)
    got_c, _ = _planned(c, q, cache.view, bt, sl, plan, causal=True)
    torch.cuda.synchronize()
    _same(got_nc, want_nc, "non-causal call with a causal plan")
    _same(got_nc_l, want_nc_l, "non-causal call with a causal plan, lse")
    _same(got_c, want_c, "causal call with its plan")
    assert not torch.equal(_bits(want_c), _bits(want_nc))  # the two calls do differ
    # a plan for another max_seqlen (another key cap) is ignored the same way
    want_m, _ = _unplanned(c, q, cache.view, bt, sl, max_seqlen=cap)
    got_m, _ = _planned(c, q, cache.view, bt, sl, plan, max_seqlen=cap)
    torch.cuda.synchronize()
    _same(got_m, want_m, "max_seqlen differs from the plan's")


def test_no_plan_and_no_split():
    # NULL plan: the unplanned call. A call that does not split has no plan
    # (size 0) and ignores a plan buffer it is given.
    c = mi.decode_case(14, V2, "bf16", [700, 1500, 64])
    q, cache, bt, sl = _inputs(c)
    say("[plan] NULL plan")
    want_o, _ = _unplanned(c, q, cache.view, bt, sl)
    got_o, _ = _planned(c, q, cache.view, bt, sl, None)
    torch.cuda.synchronize()
    _same(got_o, want_o, "NULL plan")
    n = mi.decode_case(10, NOPE, "bf16", [1100], q_len=1100, dist="uniform", std=1.0,
                       scale=1.0 / 16)
    assert mla.mla_decode_plan_size(1, 1100, 64, 512, n.max_seqlen, 64, torch.bfloat16) == 0
    q, cache, bt, sl = _inputs(n)
    say("[plan] 1100 units, no split")
    assert mla.mla_decode_plan(q, cache.view, bt, sl, n.max_seqlen, n.causal) is None
    junk = torch.full((1 << 20,), 0x5A, dtype=torch.uint8, device=dev())
    want_o, _ = _unplanned(n, q, cache.view, bt, sl)
    got_o, _ = _planned(n, q, cache.view, bt, sl, junk)
    torch.cuda.synchronize()
    _same(got_o, want_o, "unsplit call given a plan buffer")


def test_shares_past_the_descriptor():
    # 1000 sequences, one of 4M tokens (pages of 16, a table whose rows all
    # name the same pages of a 4096-page pool): the workgroups among the short
    # sequences hold more units than a descriptor stores (they plan in the
    # kernel), those on the long one more pages than it stages (the rest come
    # from the block table)
    B, page, pool_pages, long_len = 1000, 16, 4096, 4_000_000
    seqlens = mi.stream(32, 0).integers(1, 21, size=B).astype(np.int32)
    seqlens[500] = long_len
    mb = long_len // page
    pool = mi.normal(32, 1, (pool_pages, page, V2.entry), 0.1, "bf16")
    q_np = mi.normal(32, 2, (B, 1, V2.n_head, V2.entry), 0.1, "bf16")
    q = to_dev(q_np, "bf16")
    cache = to_dev(pool, "bf16")
    row = torch.arange(mb, dtype=torch.int32, device=dev()) % pool_pages
    bt = row.unsqueeze(0).expand(B, mb)  # row stride 0: every sequence names the same pages
    sl = torch.from_numpy(seqlens).to(dev())
    scale = V2.entry ** -0.5
    say(f"[plan] 1000 sequences, one of {long_len} tokens, page 16")
    outs = []
    plan = mla.mla_decode_plan(q, cache, bt, sl, long_len, True)
    for planned in (False, True):
        out = torch.full((B, 1, V2.n_head, 512), float("nan"), dtype=torch.bfloat16, device=dev())
        lse = torch.full((B, 1, V2.n_head), float("nan"), dtype=torch.float32, device=dev())
        if planned:
            mla.mla_decode_attend_planned(q, cache, bt, sl, long_len, scale, True, out, plan, lse)
        else:
            mla.mla_decode_attend(q, cache, bt, sl, long_len, scale, True, out, lse)
        torch.cuda.synchronize()
        outs.append((out, lse))
    _same(outs[1][0], outs[0][0], "shares past the descriptor")
    _same(outs[1][1], outs[0][1], "shares past the descriptor, lse")
    # the short sequences against the oracle (their pages are the table's first two)
    idx = [0, 1, 2, 3, 499, 501, 998, 999]
    sub_bt = np.tile((np.arange(2) % pool_pages).astype(np.int32), (len(idx), 1))
    want_o, want_l = oracle.attend_paged(q_np[idx], pool, sub_bt, seqlens[idx], scale, True, 512)
    assert_close(to_np(outs[1][0])[idx], want_o, "bf16", "short sequences, planned")
    assert_lse_close(to_np(outs[1][1])[idx], want_l, "short sequences, planned")


def _v_up_case(c, w_seed):
    _, w_uv_np = mi.mla_weights(w_seed, c.dims, c.dtype)
    return w_uv_np


@pytest.mark.parametrize("name", ["V2-Lite B=64", "V3 B=4 x 4096", "300 sequences one of 8000",
                                  "fp32", "16 heads x 2 queries"])
def test_planned_v_up_bit_identical(name):
    # the fused merge + un-projection where it applies; f32 and two-query calls take the
    # attention call and then the separate un-projection
    c = CASES[name]()
    say(f"[plan] attend + v_up planned: {name}")
    q, cache, bt, sl = _inputs(c)
    w_uv = to_dev(_v_up_case(c, 40), c.dtype)
    td = mi.TORCH_DTYPE[c.dtype]
    res = []
    plan = mla.mla_decode_plan(q, cache.view, bt, sl, c.max_seqlen, c.causal)
    for planned in (False, True):
        o_lat, lse = _outputs(c)
        out = torch.full((c.batch, c.q_len, c.dims.n_head, c.dims.d_v), float("nan"), dtype=td,
                         device=dev())
        if planned:
            mla.mla_decode_attend_v_up_planned(q, cache.view, bt, sl, c.max_seqlen, c.scale,
                                               c.causal, w_uv, o_lat, out, plan, lse)
        else:
            mla.mla_decode_attend_v_up(q, cache.view, bt, sl, c.max_seqlen, c.scale, c.causal,
                                       w_uv, o_lat, out, lse)
        torch.cuda.synchronize()
        res.append((o_lat, lse, out))
    _same(res[1][0], res[0][0], name + " o_lat")
    _same(res[1][1], res[0][1], name + " lse")
    _same(res[1][2], res[0][2], name + " out")
    assert torch.isfinite(res[1][2].float()).all()
