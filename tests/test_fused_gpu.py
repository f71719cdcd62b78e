"""GPU checks of mla_absorb_q_and_cache: the decode step's q fold and latent
write in one launch equal the two calls made one after the other, bit for bit
(memra-engine 0.124.1 "tests/mla_gpu_forward.rs", gate 2: each decode step
appends the new token's latent row and decodes its query; vLLM
"test_mla_cross_layer_kernel_equivalence.py": the write into a block-major
unified slot leaves the neighbouring layers untouched)."""
import numpy as np
import pytest
import torch

import mla_absorbed_decode_amd as mla
import mla_inputs as mi
from helpers import dev, say

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("T", [9, 64, 200])
def test_fused_equals_two_calls(dtype, rope, T):
    d = mi.V2_LITE
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(td).to(dev())
    q_nope = t(mi.uniform(31, 1, (T, d.n_head, d.d_nope), -1, 1, dtype))
    q_pe = t(mi.uniform(31, 2, (T, d.n_head, d.d_rope), -1, 1, dtype))
    w_uk = t(mi.uniform(31, 3, (d.n_head, d.d_nope, d.kv_rank), -0.1, 0.1, dtype))
    c = mi.cache_write_case(seed=31, ntok=T, dtype=dtype)
    kv_c, k_pe = t(c["kv_c"]), t(c["k_pe"])
    slots = c["slots"].copy()
    slots[::17] = -1  # some tokens write nothing
    slots = torch.from_numpy(slots).to(dev())
    pos = torch.from_numpy((3000 + 7 * np.arange(T)).astype(np.int32)).to(dev()) if rope else None

    def views():
        big = torch.full(c["buf_shape"], float("nan"), dtype=td, device=dev())
        view = torch.as_strided(big.view(-1), (c["num_blocks"], c["page"], c["entry"]),
                                (c["s0"], c["s1"], 1), c["offset"])
        q = torch.full((T, d.n_head, d.entry), float("nan"), dtype=td, device=dev())
        return big, view, q

    say(f"[fused] T={T} {dtype} rope={rope}")
    big_a, view_a, q_a = views()
    if rope:
        mla.mla_absorb_q_rope(q_nope, w_uk, q_pe, pos, mi.ROPE_BASE, q_a)
        mla.mla_concat_and_cache_rope(kv_c, k_pe, slots, pos, mi.ROPE_BASE, view_a)
    else:
        mla.mla_absorb_q(q_nope, w_uk, q_pe, q_a)
        mla.mla_concat_and_cache(kv_c, k_pe, slots, view_a)
    big_b, view_b, q_b = views()
    mla.mla_absorb_q_and_cache(q_nope, w_uk, q_pe, q_b, kv_c, k_pe, slots, view_b, pos,
                               mi.ROPE_BASE if rope else 0.0)
    torch.cuda.synchronize()
    assert torch.equal(bits(q_a), bits(q_b))
    assert torch.equal(bits(big_a), bits(big_b))
    assert not torch.isnan(q_b.float()).any()


def test_fused_with_an_empty_pool_only_folds():
    d = mi.V2_LITE
    q_nope = torch.randn(4, d.n_head, d.d_nope, device=dev()).to(torch.bfloat16)
    q_pe = torch.randn(4, d.n_head, d.d_rope, device=dev()).to(torch.bfloat16)
    w = torch.randn(d.n_head, d.d_nope, d.kv_rank, device=dev()).to(torch.bfloat16)
    kv = torch.randn(4, d.kv_rank, device=dev()).to(torch.bfloat16)
    kpe = torch.randn(4, d.d_rope, device=dev()).to(torch.bfloat16)
    slots = torch.zeros(4, dtype=torch.int64, device=dev())
    cache = torch.empty(0, 64, d.entry, dtype=torch.bfloat16, device=dev())
    q_a = torch.empty(4, d.n_head, d.entry, dtype=torch.bfloat16, device=dev())
    q_b = torch.empty_like(q_a)
    mla.mla_absorb_q(q_nope, w, q_pe, q_a)
    mla.mla_absorb_q_and_cache(q_nope, w, q_pe, q_b, kv, kpe, slots, cache)
    torch.cuda.synchronize()
    assert torch.equal(bits(q_a), bits(q_b))


# ------------------------------------------- attention + W_UV un-projection


def run_attend_v_up(c, w_uv_np, fused):
    from helpers import DeviceCache, to_dev
    d = c.dims
    td = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    q = to_dev(c.q, c.dtype)
    cache = DeviceCache(c, False)
    bt = torch.from_numpy(c.block_table).to(dev())
    sl = torch.from_numpy(c.seqlens).to(dev())
    w_uv = to_dev(w_uv_np, c.dtype)
    o_lat = torch.full((c.batch, c.q_len, d.n_head, d.kv_rank), float("nan"), dtype=td, device=dev())
    lse = torch.full((c.batch, c.q_len, d.n_head), float("nan"), dtype=torch.float32, device=dev())
    V = w_uv_np.shape[2]
    out = torch.full((c.batch, c.q_len, d.n_head, V), float("nan"), dtype=td, device=dev())
    if fused:
        mla.mla_decode_attend_v_up(q, cache.view, bt, sl, c.max_seqlen, c.scale, c.causal, w_uv,
                                   o_lat, out, lse)
    else:
        mla.mla_decode_attend(q, cache.view, bt, sl, c.max_seqlen, c.scale, c.causal, o_lat, lse)
        mla.mla_v_up(o_lat.view(c.batch * c.q_len, d.n_head, d.kv_rank), w_uv,
                     out.view(c.batch * c.q_len, d.n_head, V))
    torch.cuda.synchronize()
    return o_lat, lse, out


CASES = [
    ("V2-Lite full batch", lambda: mi.v2lite_decode(seed=0), 128),
    ("16 heads ragged with empty sequences",
     lambda: mi.decode_case(41, mi.V2_LITE, "bf16", [0, 1, 77, 300, 2000, 0, 64]), 128),
    ("16 heads x 2 queries", lambda: mi.decode_case(42, mi.V2_LITE, "bf16", [3, 700, 1500], q_len=2), 128),
    ("128 heads (two units per sequence)", lambda: mi.decode_case(43, mi.V3, "bf16", [1024, 4096, 1]), 128),
    ("V = 64", lambda: mi.decode_case(44, mi.V2_LITE, "bf16", [500, 900]), 64),
    ("V = 16", lambda: mi.decode_case(49, mi.V2_LITE, "bf16", [33, 1300]), 16),
    ("V = 48 (two kernels)", lambda: mi.decode_case(50, mi.V2_LITE, "bf16", [33, 1300]), 48),
    ("V = 256 (two kernels)", lambda: mi.decode_case(45, mi.V2_LITE, "bf16", [500, 900]), 256),
    ("no split: 256 sequences", lambda: mi.decode_case(46, mi.V2_LITE, "bf16",
                                                       list(range(1, 257))), 128),
    ("fp32 (two kernels)", lambda: mi.decode_case(47, mi.V2_LITE, "f32", [200, 64, 5], q_len=1,
                                                  dist="uniform", std=1.0), 128),
]


@pytest.mark.parametrize("what,make,V", CASES, ids=[c[0] for c in CASES])
def test_attend_v_up_equals_two_calls(what, make, V):
    c = make()
    w_uv = mi.uniform(48, 5, (c.dims.n_head, c.dims.kv_rank, V), -0.05, 0.05, c.dtype)
    say(f"[fused] attend + v_up: {what}")
    o_a, l_a, out_a = run_attend_v_up(c, w_uv, fused=False)
    o_b, l_b, out_b = run_attend_v_up(c, w_uv, fused=True)
    assert torch.equal(bits(o_a), bits(o_b))
    assert torch.equal(l_a.view(torch.int32), l_b.view(torch.int32))
    assert torch.equal(bits(out_a), bits(out_b))
    assert not torch.isnan(out_b.float()).any()
