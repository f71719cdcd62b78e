"""GPU checks of mla_concat_and_cache: bit-exact against the oracle's image,
zero bleed into neighbouring layers, view == contiguous (vLLM
"test_mla_cross_layer_kernel_equivalence.py",
test_concat_and_cache_mla_into_unified_slot_view; memra-engine 0.124.1
"tests/mla_gpu_forward.rs", gate 2's bit-exact append)."""
import numpy as np
import pytest
import torch

import mla_absorbed_decode_amd as mla
import mla_inputs as mi
import oracle
from helpers import dev, say

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def run_case(c, fill, slot_dtype=torch.int64):
    td = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    kv_c = torch.from_numpy(c["kv_c"]).to(td).to(dev())
    k_pe = torch.from_numpy(c["k_pe"]).to(td).to(dev()) if c["k_pe"].shape[1] else None
    slots = torch.from_numpy(c["slots"]).to(slot_dtype).to(dev())
    big = torch.full(c["buf_shape"], fill, dtype=td, device=dev())
    view = torch.as_strided(big.view(-1), (c["num_blocks"], c["page"], c["entry"]),
                            (c["s0"], c["s1"], 1), c["offset"])
    assert not view.is_contiguous() or c["n_layers"] == 1
    say(f"[cache] T={kv_c.shape[0]} entry={c['entry']} layers={c['n_layers']} fill={fill} "
        f"dtype={c['dtype']} slots={slot_dtype}")
    mla.mla_concat_and_cache(kv_c, k_pe, slots, view)
    torch.cuda.synchronize()
    buf0 = torch.full(c["buf_shape"], fill, dtype=td)
    want = oracle.cache_write(bits(buf0), bits(kv_c), bits(k_pe) if k_pe is not None else None,
                              c["slots"], c["offset"], c["num_blocks"], c["page"], c["s0"], c["s1"])
    got = bits(big)
    return got, want


@pytest.mark.parametrize("fill", [0.0, float("nan")])
@pytest.mark.parametrize("slot_dtype", [torch.int64, torch.int32])
def test_unified_slot_middle_layer(fill, slot_dtype):
    c = mi.cache_write_case(seed=0)
    got, want = run_case(c, fill, slot_dtype)
    assert np.array_equal(got, want)
    # zero bleed: layers 0 and 2 of every block keep their fill bits
    le = c["page"] * c["entry"]
    g3 = got.reshape(c["num_blocks"], c["n_layers"], le)
    fill_bits = bits(torch.full((1,), fill, dtype=torch.bfloat16))[0]
    assert np.all(g3[:, 0] == fill_bits) and np.all(g3[:, 2] == fill_bits)


def test_contiguous_equals_view():
    c = mi.cache_write_case(seed=1)
    got_v, _ = run_case(c, 0.0)
    c1 = mi.cache_write_case(seed=1, n_layers=1, layer=0)
    got_c, _ = run_case(c1, 0.0)
    le = c["page"] * c["entry"]
    view_rows = got_v.reshape(c["num_blocks"], c["n_layers"], le)[:, 1]
    assert np.array_equal(view_rows, got_c.reshape(c["num_blocks"], le))


def test_invalid_slots_skipped_and_nan_bits_preserved():
    c = mi.cache_write_case(seed=2, ntok=40)
    c["slots"][3] = -1
    c["slots"][7] = c["num_blocks"] * c["page"]  # one past the end
    c["kv_c"][5, 9] = np.nan
    c["kv_c"][6, 0] = -0.0
    got, want = run_case(c, 0.0)
    assert np.array_equal(got, want)


def test_fp32_no_rope_and_unaligned_rows():
    c = mi.cache_write_case(seed=3, ntok=50, pe=0, dtype="f32", num_blocks=4)
    got, want = run_case(c, 0.0)
    assert np.array_equal(got, want)
    # rows that are not 16-byte aligned take the element-wise path
    wide = torch.randn(30, 520, device=dev()).to(torch.bfloat16)
    kv_c = wide[:, 1:513]                 # pointer off by 2 bytes
    k_pe = torch.randn(30, 64, device=dev()).to(torch.bfloat16)
    slots = torch.randperm(128, device=dev())[:30]
    cache = torch.zeros(2, 64, 576, dtype=torch.bfloat16, device=dev())
    mla.mla_concat_and_cache(kv_c, k_pe, slots, cache)
    torch.cuda.synchronize()
    want = oracle.cache_write(bits(torch.zeros(2, 64, 576, dtype=torch.bfloat16)), bits(kv_c.contiguous()),
                              bits(k_pe), slots.cpu().numpy(), 0, 2, 64, 64 * 576, 576)
    assert np.array_equal(bits(cache), want)


def test_append_rows_then_read_back():
    # memra gate 2: prefill rows appended at slot 0.., then one row per step
    c = mi.cache_write_case(seed=4, ntok=9, num_blocks=1, n_layers=1, layer=0)
    td = torch.bfloat16
    kv_c = torch.from_numpy(c["kv_c"]).to(td).to(dev())
    k_pe = torch.from_numpy(c["k_pe"]).to(td).to(dev())
    cache = torch.zeros(1, 64, 576, dtype=td, device=dev())
    mla.mla_concat_and_cache(kv_c[:5], k_pe[:5], torch.arange(5, device=dev()), cache)
    for pos in range(5, 9):
        mla.mla_concat_and_cache(kv_c[pos:pos + 1], k_pe[pos:pos + 1],
                                 torch.tensor([pos], device=dev()), cache)
    torch.cuda.synchronize()
    rows = torch.cat([kv_c, k_pe], dim=1)
    assert torch.equal(cache[0, :9].view(torch.int16), rows.view(torch.int16))
    assert not cache[0, 9:].float().abs().max().item()
