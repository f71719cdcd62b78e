"""GPU check of mla_decode_attend_noalloc, the decode entry point that
allocates nothing (its workspace is the library's device scratch): two calls
in a row, the second smaller, each against mla_decode_attend with a caller
workspace (bit for bit) and against the double-precision oracle (the bf16
bars), plus the rejection of a plan larger than the scratch."""
import numpy as np
import pytest
import torch

import mla_absorbed_decode_amd as mla
import mla_inputs as mi
import oracle
from helpers import DeviceCache, assert_close, assert_lse_close, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _both(case):
    q = to_dev(case.q, "bf16")
    cache = DeviceCache(case, block_major=True)
    bt = torch.from_numpy(case.block_table).to(dev())
    sl = torch.from_numpy(case.seqlens).to(dev())
    shape = (case.batch, case.q_len, case.dims.n_head, case.dims.kv_rank)
    o_ws = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev())
    o_na = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev())
    l_ws = torch.full(shape[:3], float("nan"), dtype=torch.float32, device=dev())
    l_na = torch.full(shape[:3], float("nan"), dtype=torch.float32, device=dev())
    mla.mla_decode_attend(q, cache.view, bt, sl, case.max_seqlen, case.scale, case.causal, o_ws,
                          l_ws)
    mla.mla_decode_attend_noalloc(q, cache.view, bt, sl, case.max_seqlen, case.scale, case.causal,
                                  o_na, l_na)
    torch.cuda.synchronize()
    return o_ws, l_ws, o_na, l_na


def test_noalloc_two_calls_match_workspace_call_and_oracle():
    cases = [
        ("128 heads, 3 sequences", mi.decode_case(41, mi.V3, "bf16", [1024, 2048, 777],
                                                  n_layers=3, layer=1)),
        ("16 heads, 2 sequences (smaller)", mi.decode_case(42, mi.V2_LITE, "bf16", [300, 17],
                                                           n_layers=3, layer=1)),
    ]
    for what, c in cases:
        say(f"[noalloc] {what}: B={c.batch} N={c.dims.n_head} seqlens={c.seqlens.tolist()}")
        o_ws, l_ws, o_na, l_na = _both(c)
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), what
        assert torch.equal(l_ws, l_na), what
        want_o, want_l = oracle.attend_paged(c.q, c.pool, c.block_table, c.seqlens, c.scale,
                                             c.causal, c.dims.kv_rank)
        assert_close(to_np(o_na), want_o, "bf16", what)
        assert_lse_close(to_np(l_na), want_l, what)


def test_noalloc_rejects_a_plan_larger_than_its_scratch():
    # 85 sequences x 192 heads: 255 split units of 64 rows, 511 partial slots of
    # 64 rows x 1028 bytes = 33.6 MB > 32 MiB; refused before any launch
    B, N = 85, 192
    say(f"[noalloc] oversized plan B={B} N={N}")
    q = torch.zeros(B, 1, N, 576, dtype=torch.bfloat16, device=dev())
    cache = torch.zeros(4, 64, 576, dtype=torch.bfloat16, device=dev())
    bt = torch.zeros(B, 4, dtype=torch.int32, device=dev())
    sl = torch.full((B,), 256, dtype=torch.int32, device=dev())
    out = torch.zeros(B, 1, N, 512, dtype=torch.bfloat16, device=dev())
    need = mla.mla_decode_workspace_size(B, 1, N, 512, 256, 64, torch.bfloat16)
    assert need > (32 << 20)
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_attend_noalloc(q, cache, bt, sl, 256, 0.04, True, out, None)
    assert e.value.status == -6  # MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert out.abs().max().item() == 0  # nothing was written
