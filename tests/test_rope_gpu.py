"""GPU parity of the interleaved rotary embedding against the double-precision
oracle (memra-engine 0.124.1 "tests/mla_gpu_forward.rs", gate 3,
gpu_mla_rope_interleaved_matches_cpu: d_rope 8 and 64, base 8e6, 7 positions
13 apart, 5 vectors each, bound 1e-4 * max(1, max|want|); d_rope 0 is a no-op),
alone and fused into the query fold and the latent-cache write.

The kernels compute the angle and the rotation in double and round once, so
beyond the page's bound each element is held to one unit in the last place of
its storage type, plus the double arithmetic's own error: the angle
position * base^(-2i/d) carries a relative error of a few 2^-53 on either
side (the oracle's pow and the kernel's exp2 differ in the last place), so
1e-15 * max|x| * max(1, max|position|).
"""
import numpy as np
import pytest
import torch

import mla_absorbed_decode_amd as mla
import mla_inputs as mi
import oracle
from helpers import assert_close, dev, say, to_np

pytestmark = pytest.mark.gpu

ULP = {"f32": 2.0 ** -23, "bf16": 2.0 ** -7}  # relative spacing bound of each type


def t_dev(x, dtype):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(td).to(dev())


def assert_ulp(got, want, dtype, scale, what, max_pos=1):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    bound = ULP[dtype] * np.abs(want) + 1e-15 * max(scale, 1e-30) * max(1, abs(max_pos))
    bad = np.abs(got - want) > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond one ulp, worst "
                           f"{np.max(np.abs(got - want) - bound):.3e}")


@pytest.mark.parametrize("d_rope", [8, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_shape(d_rope, dtype):
    x, pos = mi.rope_case(0, d_rope=d_rope, dtype=dtype)
    say(f"[rope] gate shape d_rope={d_rope} {dtype}")
    xd = t_dev(x, dtype)
    mla.mla_rope_interleaved(xd, torch.from_numpy(pos).to(dev()), mi.ROPE_BASE)
    torch.cuda.synchronize()
    want = oracle.rope_interleaved(x, pos, mi.ROPE_BASE)
    got = to_np(xd)
    if dtype == "f32":  # the page's bound, stated for f32 data
        assert np.abs(got - want).max() <= 1e-4 * max(np.abs(want).max(), 1.0)
    assert_ulp(got, want, dtype, np.abs(x).max(), f"d_rope {d_rope} {dtype}", pos.max())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_long_context_and_negative_positions(dtype):
    # positions up to about 1.3 million and below zero; another base
    x, pos = mi.rope_case(1, n_pos=40, n_vec=3, d_rope=64, dtype=dtype, pos_step=33_331,
                          pos_offset=-20)
    say(f"[rope] long context {dtype}")
    xd = t_dev(x, dtype)
    mla.mla_rope_interleaved(xd, torch.from_numpy(pos).to(dev()), 10_000.0)
    torch.cuda.synchronize()
    want = oracle.rope_interleaved(x, pos, 10_000.0)
    assert_ulp(to_np(xd), want, dtype, np.abs(x).max(), f"long context {dtype}",
               np.abs(pos).max())


def test_strided_view_only_touches_the_view():
    # x is [T, V, d] inside a padded allocation: the padding keeps its bits
    x, pos = mi.rope_case(2, n_pos=9, n_vec=4, d_rope=64)
    big = torch.full((9, 6, 80), float("nan"), dtype=torch.float32, device=dev())
    view = big[:, 1:5, 8:72]
    view.copy_(torch.from_numpy(x).to(dev()))
    say("[rope] strided view")
    mla.mla_rope_interleaved(view, torch.from_numpy(pos).to(dev()), mi.ROPE_BASE)
    torch.cuda.synchronize()
    want = oracle.rope_interleaved(x, pos, mi.ROPE_BASE)
    assert_ulp(to_np(view), want, "f32", 1.0, "strided view", pos.max())
    b = big.cpu()
    mask = torch.ones_like(b, dtype=torch.bool)
    mask[:, 1:5, 8:72] = False
    assert torch.isnan(b[mask]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("width,start", [(129, 1), (66, 2)])
def test_unaligned_rows(dtype, width, start):
    # rows `width` elements apart, starting at element `start`: 129/1 leaves pairs
    # unaligned (element path), 66/2 leaves rows off 16 bytes but pairs aligned
    x, pos = mi.rope_case(3, n_pos=6, n_vec=4, d_rope=64, dtype=dtype)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    big = torch.full((6, 4, width), float("nan"), dtype=td, device=dev())
    view = big[:, :, start:start + 64]
    view.copy_(t_dev(x, dtype))
    say(f"[rope] rows {width} apart from {start}, {dtype}")
    mla.mla_rope_interleaved(view, torch.from_numpy(pos).to(dev()), mi.ROPE_BASE)
    torch.cuda.synchronize()
    want = oracle.rope_interleaved(x, pos, mi.ROPE_BASE)
    assert_ulp(to_np(view), want, dtype, 1.0, f"rows {width}/{start} {dtype}", pos.max())
    b = big.float().cpu()
    assert torch.isnan(b[:, :, :start]).all() and torch.isnan(b[:, :, start + 64:]).all()


def test_width_zero_is_a_no_op():
    # NoPE contract: d_rope 0 launches nothing and changes nothing
    host = torch.tensor([1.0, -2.0, 3.0], device=dev())
    mla.mla_rope_interleaved(host.view(1, 1, 3)[:, :, :0],
                             torch.zeros(1, dtype=torch.int32, device=dev()), mi.ROPE_BASE)
    torch.cuda.synchronize()
    assert host.cpu().tolist() == [1.0, -2.0, 3.0]


@pytest.mark.parametrize("broadcast", [False, True])
def test_fused_into_the_query_fold(broadcast):
    d = mi.V2_LITE
    T = 64
    q_nope = mi.uniform(3, 1, (T, d.n_head, d.d_nope), -1, 1, "bf16")
    q_pe = mi.uniform(3, 2, (T, 1 if broadcast else d.n_head, d.d_rope), -1, 1, "bf16")
    w_uk = mi.uniform(3, 3, (d.n_head, d.d_nope, d.kv_rank), -0.1, 0.1, "bf16")
    pos = (4000 + np.arange(T)).astype(np.int32)
    say(f"[rope] fused q fold, broadcast={broadcast}")
    qn, pe, w = t_dev(q_nope, "bf16"), t_dev(q_pe, "bf16"), t_dev(w_uk, "bf16")
    out = torch.full((T, d.n_head, d.entry), float("nan"), dtype=torch.bfloat16, device=dev())
    plain = torch.full_like(out, float("nan"))
    mla.mla_absorb_q_rope(qn, w, pe, torch.from_numpy(pos).to(dev()), mi.ROPE_BASE, out)
    mla.mla_absorb_q(qn, w, pe, plain)
    torch.cuda.synchronize()
    L = d.kv_rank
    # the fold is the plain fold, bit for bit
    assert torch.equal(out[..., :L].view(torch.int16), plain[..., :L].view(torch.int16))
    want = oracle.rope_interleaved(np.broadcast_to(q_pe, (T, d.n_head, d.d_rope)), pos,
                                   mi.ROPE_BASE)
    assert_ulp(to_np(out[..., L:]), want, "bf16", 1.0, "fused q rope", pos.max())


def test_fused_into_the_cache_write():
    c = mi.cache_write_case(seed=4)
    T = c["kv_c"].shape[0]
    pos = mi.stream(4, 61).integers(0, 200_000, size=T).astype(np.int32)
    td = torch.bfloat16
    kv_c, k_pe = torch.from_numpy(c["kv_c"]).to(td).to(dev()), torch.from_numpy(c["k_pe"]).to(td).to(dev())
    slots = torch.from_numpy(c["slots"]).to(dev())
    big = torch.full(c["buf_shape"], float("nan"), dtype=td, device=dev())
    view = torch.as_strided(big.view(-1), (c["num_blocks"], c["page"], c["entry"]),
                            (c["s0"], c["s1"], 1), c["offset"])
    say(f"[rope] fused cache write T={T}")
    mla.mla_concat_and_cache_rope(kv_c, k_pe, slots, torch.from_numpy(pos).to(dev()),
                                  mi.ROPE_BASE, view)
    torch.cuda.synchronize()
    # the image a plain write of the oracle-rotated k_pe would leave, rounded to bf16
    k_rot = oracle.rope_interleaved(c["k_pe"], pos, mi.ROPE_BASE)
    k_rot_bits = torch.from_numpy(k_rot.astype(np.float32)).to(td).view(torch.int16).numpy()
    buf0 = torch.full(c["buf_shape"], float("nan"), dtype=td).view(torch.int16).numpy()
    want_bits = oracle.cache_write(buf0, kv_c.cpu().view(torch.int16).numpy(), k_rot_bits,
                                   c["slots"], c["offset"], c["num_blocks"], c["page"], c["s0"],
                                   c["s1"])
    got = big.cpu()
    got_bits = got.view(torch.int16).numpy()
    L = c["entry"] - c["k_pe"].shape[1]
    # every element but the rotated part is the oracle's image bit for bit
    slots_ok = (c["slots"] >= 0) & (c["slots"] < c["num_blocks"] * c["page"])
    rot = np.zeros(got_bits.size, dtype=bool)
    for t in np.nonzero(slots_ok)[0]:
        blk, off = divmod(int(c["slots"][t]), c["page"])
        base = c["offset"] + blk * c["s0"] + off * c["s1"]
        rot[base + L: base + c["entry"]] = True
    g = got_bits.reshape(-1)
    w = want_bits.reshape(-1)
    assert np.array_equal(g[~rot], w[~rot])
    # the rotated part within one bf16 ulp of the exact rotation
    gv = got.float().numpy().reshape(-1)[rot]
    exact = np.zeros(got_bits.size)
    for t in np.nonzero(slots_ok)[0]:
        blk, off = divmod(int(c["slots"][t]), c["page"])
        base = c["offset"] + blk * c["s0"] + off * c["s1"]
        exact[base + L: base + c["entry"]] = k_rot[t]
    assert_ulp(gv, exact[rot], "bf16", 4.0, "fused cache rope", pos.max())


def test_decode_with_rope_against_the_naive_oracle():
    # positions rotate q_pe and k_pe; the attention of the rotated rows is the
    # naive (decompressed) MLA of the rotated inputs
    d = mi.V2_LITE
    t_kv, B = 300, 1
    q_nope, q_pe, c_kv, k_pe = mi.mla_activations(7, d, 1, t_kv, "bf16", std=0.5)
    w_uk, w_uv = mi.mla_weights(7, d, "bf16")
    scale = (d.d_nope + d.d_rope) ** -0.5
    pos_k = np.arange(t_kv, dtype=np.int32) + 5000
    pos_q = pos_k[-1:]
    say("[rope] decode step with rotated q_pe and k_pe, 300 keys")
    page = 64
    nb = (t_kv + page - 1) // page
    cache = torch.full((nb, page, d.entry), float("nan"), dtype=torch.bfloat16, device=dev())
    mla.mla_concat_and_cache_rope(t_dev(c_kv, "bf16"), t_dev(k_pe, "bf16"),
                                  torch.arange(t_kv, dtype=torch.int64, device=dev()),
                                  torch.from_numpy(pos_k).to(dev()), mi.ROPE_BASE, cache)
    q = torch.empty(B, 1, d.n_head, d.entry, dtype=torch.bfloat16, device=dev())
    mla.mla_absorb_q_rope(t_dev(q_nope, "bf16"), t_dev(w_uk, "bf16"), t_dev(q_pe, "bf16"),
                          torch.from_numpy(pos_q).to(dev()), mi.ROPE_BASE, q[:, 0])
    o_lat = torch.empty(B, 1, d.n_head, d.kv_rank, dtype=torch.bfloat16, device=dev())
    bt = torch.arange(nb, dtype=torch.int32, device=dev()).view(1, nb)
    mla.mla_decode_attend(q, cache, bt, torch.tensor([t_kv], dtype=torch.int32, device=dev()),
                          t_kv, scale, True, o_lat, None)
    out = torch.empty(1, d.n_head, d.d_v, dtype=torch.bfloat16, device=dev())
    mla.mla_v_up(o_lat[:, 0], t_dev(w_uv, "bf16"), out)
    torch.cuda.synchronize()
    q_pe_r = oracle.rope_interleaved(q_pe, pos_q, mi.ROPE_BASE)
    k_pe_r = oracle.rope_interleaved(k_pe, pos_k, mi.ROPE_BASE)
    want = oracle.naive(q_nope, q_pe_r, c_kv, k_pe_r, w_uk, w_uv, np.array([t_kv - 1]), scale,
                        True)
    assert_close(to_np(out), want, "bf16", "decode with rope")


def test_fused_cache_write_fp32_unaligned_rows():
    # rows that are not 16-byte multiples take the one-element-per-thread path
    c = mi.cache_write_case(seed=5, ntok=50, num_blocks=4, page=32, kv_rank=510, pe=6,
                            n_layers=1, layer=0, dtype="f32")
    T = c["kv_c"].shape[0]
    pos = (np.arange(T) * 977 - 100).astype(np.int32)
    kv_c, k_pe = t_dev(c["kv_c"], "f32"), t_dev(c["k_pe"], "f32")
    cache = torch.full((c["num_blocks"], c["page"], c["entry"]), float("nan"), device=dev())
    say("[rope] fused cache write, fp32 unaligned rows")
    mla.mla_concat_and_cache_rope(kv_c, k_pe, torch.from_numpy(c["slots"]).to(dev()),
                                  torch.from_numpy(pos).to(dev()), 10_000.0, cache)
    torch.cuda.synchronize()
    got = cache.cpu().numpy().reshape(-1, c["entry"])
    k_rot = oracle.rope_interleaved(c["k_pe"], pos, 10_000.0)
    written = np.zeros(got.shape[0], dtype=bool)
    for t, s in enumerate(c["slots"]):
        assert np.array_equal(got[s, :510].view(np.int32), c["kv_c"][t].view(np.int32))
        assert_ulp(got[s, 510:], k_rot[t], "f32", 1.0, f"token {t}", np.abs(pos).max())
        written[s] = True
    assert np.isnan(got[~written]).all()


def _round_bf16(v):
    """Round-to-nearest-even bf16 bits of float64 values, rounded once: to
    float "to odd" first, then to bf16 to nearest even (the two-step form of
    one correct rounding)."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    bits = f.view(np.uint32).copy()
    inexact = f.astype(np.float64) != v
    fix = inexact & ((bits & 1) == 0)
    up = np.abs(f.astype(np.float64)) < np.abs(v)
    bits[fix & up] += 1
    bits[fix & ~up] -= 1
    rounded = (bits.astype(np.uint64) + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def test_bf16_rounds_once_on_every_path():
    """A rotated value can sit within a float rounding of a bf16 midpoint
    (token 86 of this input: 1.6e-8 from one); converting double -> float ->
    bf16 would land on the midpoint and round it to even the wrong way. The
    16-byte path (aligned rows) and the pair path (rows 4-byte aligned only)
    give the same bits, and every element equals the correctly rounded bf16 of
    the oracle's double result (elements within 1e-12 of a midpoint, where the
    two doubles may legitimately differ, excepted)."""
    T, H, D = 333, 2, 64
    g = torch.Generator().manual_seed(0)
    x = (torch.rand((T, H, D), generator=g) * 2 - 1).to(torch.bfloat16)
    pos = np.arange(T, dtype=np.int32) * 13
    say("[rope] single rounding, aligned and unaligned rows")
    pd = torch.from_numpy(pos).to(dev())
    a = x.to(dev()).clone()
    mla.mla_rope_interleaved(a, pd, mi.ROPE_BASE)
    buf = torch.zeros(T * H * D + 2, dtype=torch.bfloat16, device=dev())
    b = buf[2:].view(T, H, D)
    b.copy_(x.to(dev()))
    mla.mla_rope_interleaved(b, pd, mi.ROPE_BASE)
    torch.cuda.synchronize()
    ab = a.view(torch.int16).cpu().numpy().view(np.uint16)
    bb = b.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(ab, bb)
    want = oracle.rope_interleaved(x.float().numpy(), pos, mi.ROPE_BASE)
    ref = _round_bf16(want)
    # distance of each double to the nearest bf16 midpoint, relative
    lo = (ref.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    step = np.abs(lo) * 2.0 ** -8
    near = np.minimum(np.abs(np.abs(want) - (np.abs(lo) - step / 2)),
                      np.abs(np.abs(want) - (np.abs(lo) + step / 2))) < 1e-12 * np.maximum(np.abs(want), 1e-30)
    assert np.array_equal(ab[~near], ref[~near])
    assert ab[86, 1, 52] == ref[86, 1, 52]
