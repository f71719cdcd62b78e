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
@pytest.mark.parametrize("T", [64, 200])
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
