"""Pins of the CPU oracle to things other than itself.

Each oracle function is checked against at least one of: a hand-derived
fixture under tests/golden/, a library routine computing the same definition
by another route (torch float64 bmm / scaled_dot_product_attention, numpy
indexing), a closed form, or an invariant of the method (naive = absorbed,
decode at step t = full recompute at t, split-and-merge = single pass, paged =
contiguous, softmax rows sum to one). The cases are chosen so a dropped term,
a wrong sign or index, or a transposed operand fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import mla_inputs as mi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa_mqa(q, kv, pos, scale, causal, L):
    """Absorbed attention as one-KV-head attention (K = [c_kv | k_pe],
    V = c_kv) through torch's float64 scaled_dot_product_attention."""
    q = torch.from_numpy(np.asarray(q, dtype=np.float64))  # [nq, N, E]
    kv = torch.from_numpy(np.asarray(kv, dtype=np.float64))  # [T, E]
    nq, N, E = q.shape
    T = kv.shape[0]
    qh = q.permute(1, 0, 2).contiguous()  # [N, nq, E]
    k = kv.unsqueeze(0).expand(N, T, E).contiguous()
    v = kv[:, :L].unsqueeze(0).expand(N, T, L).contiguous()
    j = torch.arange(T).unsqueeze(0)
    p = torch.as_tensor(np.asarray(pos)).unsqueeze(1)
    mask = (j <= p) if causal else torch.ones(nq, T, dtype=torch.bool)
    out = torch.nn.functional.scaled_dot_product_attention(qh, k, v, attn_mask=mask, scale=scale)
    return out.permute(1, 0, 2).numpy()


# --------------------------------------------------------------------- bmm


def test_bmm_golden():
    g = _golden("bmm.json")
    out = oracle.bmm(np.array(g["a"]), np.array(g["b"]))
    np.testing.assert_array_equal(out, np.array(g["out"]))


def test_bmm_golden_transposed_view():
    # a stored as [M, G, K]; the oracle reads it through strides as [G, M, K]
    g = _golden("bmm.json")
    a = np.array(g["a"])  # [G, M, K]
    store = np.ascontiguousarray(a.transpose(1, 0, 2))  # [M, G, K]
    G, M, K = a.shape
    b = np.array(g["b"])
    N = b.shape[2]
    out = oracle.bmm_strided(store, (0, K, G * K, 1), b, (0, K * N, N, 1), (G, M, K, N))
    np.testing.assert_array_equal(out, np.array(g["out"]))


@pytest.mark.parametrize("G,M,K,N", [(16, 7, 128, 512), (5, 6, 9, 4), (3, 1, 512, 128)])
def test_bmm_vs_torch_float64(G, M, K, N):
    rng = np.random.default_rng(G * 100 + M)
    a = rng.uniform(-1, 1, (G, M, K))
    b = rng.uniform(-1, 1, (G, K, N))
    want = torch.bmm(torch.from_numpy(a), torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(oracle.bmm(a, b), want, rtol=1e-12, atol=1e-12)


def test_fold_and_vup_vs_einsum_on_transposed_layouts():
    # the q-side fold reads q_nope [T,N,P] as the [N,T,P] view the upstream
    # call passes; the un-projection writes [T,N,V] (vllm.cpp transposed-view test)
    rng = np.random.default_rng(5)
    T, N, P, L, V = 6, 5, 9, 12, 4
    q_nope = rng.uniform(-1, 1, (T, N, P))
    w_uk_t = rng.uniform(-1, 1, (N, P, L))
    o_lat = rng.uniform(-1, 1, (T, N, L))
    w_uv = rng.uniform(-1, 1, (N, L, V))
    np.testing.assert_allclose(oracle.fold_q(q_nope, w_uk_t),
                               np.einsum("thp,hpl->thl", q_nope, w_uk_t), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.v_up(o_lat, w_uv),
                               np.einsum("thl,hlv->thv", o_lat, w_uv), rtol=1e-12, atol=1e-13)


def test_bmm_identity_and_zero_weights():
    rng = np.random.default_rng(9)
    a = rng.uniform(-1, 1, (3, 4, 5))
    eye = np.broadcast_to(np.eye(5), (3, 5, 5)).copy()
    np.testing.assert_array_equal(oracle.bmm(a, eye), a)
    np.testing.assert_array_equal(oracle.bmm(a, np.zeros((3, 5, 2))), np.zeros((3, 4, 2)))


# ------------------------------------------------------------ attention


@pytest.mark.parametrize("name", ["attend_basic.json", "attend_rope.json", "attend_causal.json"])
def test_attend_golden(name):
    g = _golden(name)
    o, lse, probs = oracle.attend_seq(np.array(g["q"]), np.array(g["kv"]), g["pos"], g["scale"],
                                      g["causal"], g["L"], want_probs=True)
    np.testing.assert_allclose(o, np.array(g["o_lat"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(g["lse"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(probs.sum(-1), 1.0, rtol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,N,L,R,T", [(1, 16, 512, 64, 300), (5, 3, 64, 8, 11), (7, 4, 32, 0, 7)])
def test_attend_vs_sdpa_float64(nq, N, L, R, T, causal):
    rng = np.random.default_rng(nq * 7 + T)
    q = rng.normal(0, 0.3, (nq, N, L + R))
    kv = rng.normal(0, 1.0, (T, L + R))
    pos = np.arange(T - nq, T)
    scale = (L + R) ** -0.5
    o, lse, _ = oracle.attend_seq(q, kv, pos, scale, causal, L)
    np.testing.assert_allclose(o, _sdpa_mqa(q, kv, pos, scale, causal, L), rtol=1e-11, atol=1e-12)
    # lse against scipy-free log-sum-exp of numpy scores
    s = np.einsum("ihe,je->ihj", q, kv) * scale
    if causal:
        s = np.where(np.arange(T)[None, None, :] <= pos[:, None, None], s, -np.inf)
    m = s.max(-1, keepdims=True)
    want_lse = (m + np.log(np.exp(s - m).sum(-1, keepdims=True)))[..., 0]
    np.testing.assert_allclose(lse, want_lse, rtol=1e-12, atol=1e-12)


def test_attend_closed_forms():
    rng = np.random.default_rng(11)
    L, R, T, N = 16, 4, 9, 3
    kv = rng.normal(0, 1, (T, L + R))
    # one visible key: output is that key's c_kv exactly, lse its score
    q = rng.normal(0, 1, (1, N, L + R))
    o, lse, _ = oracle.attend_seq(q, kv, [0], 0.7, True, L)
    np.testing.assert_allclose(o[0], np.broadcast_to(kv[0, :L], (N, L)), rtol=1e-15, atol=0)
    np.testing.assert_allclose(lse[0], 0.7 * q[0] @ kv[0], rtol=1e-14)
    # zero query: mean of visible rows, lse = ln(count)
    z = np.zeros((2, N, L + R))
    o, lse, _ = oracle.attend_seq(z, kv, [3, T - 1], 1.0, True, L)
    np.testing.assert_allclose(o[0], np.broadcast_to(kv[:4, :L].mean(0), (N, L)), rtol=1e-13)
    np.testing.assert_allclose(o[1], np.broadcast_to(kv[:, :L].mean(0), (N, L)), rtol=1e-13)
    np.testing.assert_allclose(lse[0], math.log(4.0), rtol=1e-15)
    np.testing.assert_allclose(lse[1], math.log(T), rtol=1e-15)
    # all keys identical: output is that row whatever q is
    same = np.broadcast_to(kv[2], (T, L + R)).copy()
    o, _, _ = oracle.attend_seq(q, same, [T - 1], 0.3, False, L)
    np.testing.assert_allclose(o[0], np.broadcast_to(kv[2, :L], (N, L)), rtol=1e-13)


def test_attend_no_visible_key_and_empty_sequence():
    q = np.ones((2, 2, 5))
    kv = np.ones((3, 5))
    o, lse, _ = oracle.attend_seq(q, kv, [-1, 0], 1.0, True, 4)  # query 0 sees nothing
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))
    o, lse, _ = oracle.attend_seq(q, np.zeros((0, 5)), [0, 0], 1.0, False, 4)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_attend_softmax_rows_sum_to_one_and_key_permutation():
    rng = np.random.default_rng(3)
    q = rng.normal(0, 1, (3, 4, 40))
    kv = rng.normal(0, 1, (25, 40))
    o, lse, p = oracle.attend_seq(q, kv, [24, 24, 24], 0.4, False, 32, want_probs=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)
    assert np.all(p >= 0)
    perm = rng.permutation(25)
    o2, lse2, _ = oracle.attend_seq(q, kv[perm], [24, 24, 24], 0.4, False, 32)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)


def test_causal_rows_ignore_future_keys():
    # changing keys beyond a query's position must not change its output
    rng = np.random.default_rng(4)
    q = rng.normal(0, 1, (1, 2, 12))
    kv = rng.normal(0, 1, (10, 12))
    o, _, _ = oracle.attend_seq(q, kv, [5], 0.5, True, 8)
    kv2 = kv.copy()
    kv2[6:] = 1e3
    o2, _, _ = oracle.attend_seq(q, kv2, [5], 0.5, True, 8)
    np.testing.assert_array_equal(o, o2)


# ------------------------------------------------------- naive vs absorbed

SHRUNK = [
    mi.Dims(n_head=4, d_nope=24, d_rope=8, d_v=32, kv_rank=64),
    mi.Dims(n_head=3, d_nope=12, d_rope=4, d_v=20, kv_rank=48),
    mi.Dims(n_head=4, d_nope=32, d_rope=0, d_v=32, kv_rank=64),
]


def test_naive_golden():
    g = _golden("naive.json")
    out = oracle.naive(np.array(g["q_nope"]), None, np.array(g["c_kv"]), None,
                       np.array(g["w_uk_t"]), np.array(g["w_uv"]), g["pos"], g["scale"], g["causal"])
    np.testing.assert_allclose(out, np.array(g["out"]), rtol=1e-14)
    out2, *_ = oracle.absorbed(np.array(g["q_nope"]), None, np.array(g["c_kv"]), None,
                               np.array(g["w_uk_t"]), np.array(g["w_uv"]), g["pos"], g["scale"],
                               g["causal"])
    np.testing.assert_allclose(out2, np.array(g["out"]), rtol=1e-14)


@pytest.mark.parametrize("d", SHRUNK + [mi.V2_LITE, mi.NOPE64], ids=lambda d: f"N{d.n_head}P{d.d_nope}R{d.d_rope}")
@pytest.mark.parametrize("t_q,t_kv", [(6, 6), (3, 11)])
def test_naive_equals_absorbed(d, t_q, t_kv):
    seed = d.n_head * 31 + t_kv
    q_nope, q_pe, c_kv, k_pe = mi.mla_activations(seed, d, t_q, t_kv, mi.F32)
    w_uk_t, w_uv = mi.mla_weights(seed, d, mi.F32)
    pos = np.arange(t_kv - t_q, t_kv)
    scale = (d.d_nope + d.d_rope) ** -0.5
    naive = oracle.naive(q_nope, q_pe if d.d_rope else None, c_kv, k_pe if d.d_rope else None,
                         w_uk_t, w_uv, pos, scale, True)
    absorbed, q_lat, o_lat, lse = oracle.absorbed(q_nope, q_pe if d.d_rope else None, c_kv,
                                                  k_pe if d.d_rope else None, w_uk_t, w_uv,
                                                  pos, scale, True)
    mx = max(np.abs(naive).max(), 1e-30)
    assert np.abs(naive - absorbed).max() <= 1e-12 * max(1.0, mx)
    assert np.abs(naive).max() > 1e-6
    # stage outputs agree with the stand-alone stages
    np.testing.assert_allclose(q_lat, oracle.fold_q(q_nope, w_uk_t), rtol=1e-13, atol=1e-14)
    kv = np.concatenate([c_kv, k_pe], axis=1) if d.d_rope else c_kv
    q = np.concatenate([q_lat, q_pe], axis=2) if d.d_rope else q_lat
    o2, lse2, _ = oracle.attend_seq(q, kv, pos, scale, True, d.kv_rank)
    np.testing.assert_allclose(o_lat, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13)


def test_naive_vs_sdpa_on_decompressed_heads():
    d = SHRUNK[0]
    q_nope, q_pe, c_kv, k_pe = mi.mla_activations(77, d, 5, 9, mi.F32)
    w_uk_t, w_uv = mi.mla_weights(77, d, mi.F32)
    pos = np.arange(4, 9)
    scale = 0.25
    out = oracle.naive(q_nope, q_pe, c_kv, k_pe, w_uk_t, w_uv, pos, scale, True)
    k_nope = np.einsum("hpl,jl->hjp", w_uk_t.astype(np.float64), c_kv.astype(np.float64))
    v = np.einsum("hld,jl->hjd", w_uv.astype(np.float64), c_kv.astype(np.float64))
    k = np.concatenate([k_nope, np.broadcast_to(k_pe, (d.n_head,) + k_pe.shape)], axis=2)
    q = np.concatenate([q_nope, q_pe], axis=2).transpose(1, 0, 2).astype(np.float64)
    mask = torch.from_numpy(np.arange(9)[None, :] <= pos[:, None])
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(q)), torch.from_numpy(np.ascontiguousarray(k)),
        torch.from_numpy(np.ascontiguousarray(v)), attn_mask=mask, scale=scale).numpy()
    np.testing.assert_allclose(out, want.transpose(1, 0, 2), rtol=1e-11, atol=1e-13)


def test_decode_step_equals_full_recompute():
    # memra gate 2: each decode step (one query at pos against rows 0..pos)
    # equals the full-sequence causal prefill's row at pos.
    d = SHRUNK[0]
    total = 9
    q_nope, q_pe, c_kv, k_pe = mi.mla_activations(0x57E9, d, total, total, mi.F32)
    w_uk_t, w_uv = mi.mla_weights(0x57E9, d, mi.F32)
    scale = (d.d_nope + d.d_rope) ** -0.5
    full, *_ = oracle.absorbed(q_nope, q_pe, c_kv, k_pe, w_uk_t, w_uv, np.arange(total), scale, True)
    for pos in range(5, total):
        step, *_ = oracle.absorbed(q_nope[pos:pos + 1], q_pe[pos:pos + 1], c_kv[:pos + 1],
                                   k_pe[:pos + 1], w_uk_t, w_uv, [pos], scale, True)
        assert np.abs(step[0] - full[pos]).max() <= 1e-13 * max(1.0, np.abs(full[pos]).max())


# ----------------------------------------------------- paging and splits


def test_gather_pages_vs_numpy_indexing():
    rng = np.random.default_rng(21)
    NB, PG, E = 10, 4, 6
    pool = rng.normal(0, 1, (NB, PG, E))
    bt = np.array([[7, 2, 9, -1], [0, 5, -1, -1]], dtype=np.int32)
    for b, s in [(0, 11), (1, 8), (1, 0)]:
        rows = oracle.gather_pages(pool, bt, b, s)
        j = np.arange(s)
        np.testing.assert_array_equal(rows, pool[bt[b, j // PG], j % PG])
    with pytest.raises(ValueError):
        oracle.gather_pages(pool, bt, 0, 13)  # needs page 3 = -1


def test_paged_equals_contiguous():
    d = mi.Dims(n_head=5, d_nope=8, d_rope=8, d_v=8, kv_rank=32)
    c = mi.decode_case(3, d, mi.F32, [1, 17, 64, 65, 130], q_len=3, page=16, num_blocks=40,
                       std=0.5)
    o, lse = oracle.attend_paged(c.q, c.pool, c.block_table, c.seqlens, c.scale, True, d.kv_rank)
    for b, s in enumerate(c.seqlens):
        j = np.arange(s)
        rows = c.pool[c.block_table[b, j // c.page], j % c.page].astype(np.float64)
        o2, lse2, _ = oracle.attend_seq(c.q[b], rows, np.arange(s - 3, s), c.scale, True, d.kv_rank)
        np.testing.assert_array_equal(o[b], o2)
        np.testing.assert_array_equal(lse[b], lse2)
    assert np.all(np.isfinite(o))  # NaN page tails never reached


def test_split_merge_golden():
    g = _golden("merge.json")
    o, lse = oracle.attend_split(np.array(g["q"]), np.array(g["kv"]), g["pos"], g["scale"],
                                 g["causal"], g["L"], g["bounds"])
    np.testing.assert_allclose(o, np.array(g["o_lat"]), rtol=1e-14)
    np.testing.assert_allclose(lse, np.array(g["lse"]), rtol=1e-14)


@pytest.mark.parametrize("bounds", [[0, 40], [0, 1, 40], [0, 13, 13, 27, 40], [0, 5, 10, 20, 30, 40]])
@pytest.mark.parametrize("causal", [False, True])
def test_split_merge_equals_single_pass(bounds, causal):
    rng = np.random.default_rng(len(bounds))
    q = rng.normal(0, 1, (4, 3, 24))
    kv = rng.normal(0, 1, (40, 24))
    pos = np.array([2, 15, 28, 39])
    o1, lse1, _ = oracle.attend_seq(q, kv, pos, 0.3, causal, 16)
    o2, lse2 = oracle.attend_split(q, kv, pos, 0.3, causal, 16, bounds)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse1, rtol=1e-13)


# -------------------------------------------------------------- cache write


def test_cache_write_golden():
    g = _golden("cache_write.json")
    buf = np.zeros(g["buf_elems"], dtype=np.float32)
    out = oracle.cache_write(buf, np.array(g["kv_c"], np.float32), np.array(g["k_pe"], np.float32),
                             g["slots"], g["offset"], g["num_blocks"], g["page"], g["s0"], g["s1"])
    np.testing.assert_array_equal(out, np.array(g["buf"], np.float32))


@pytest.mark.parametrize("pe", [64, 0])
def test_cache_write_vs_numpy_view_and_zero_bleed(pe):
    c = mi.cache_write_case(seed=0, pe=pe)
    bits = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy()
    kv_c, k_pe = bits(c["kv_c"]), bits(c["k_pe"])
    buf = np.zeros(c["buf_shape"], dtype=np.int16)
    out = oracle.cache_write(buf, kv_c, k_pe if pe else None, c["slots"], c["offset"],
                             c["num_blocks"], c["page"], c["s0"], c["s1"])
    # route 2: numpy strided view + fancy-index assignment
    want = np.zeros(c["buf_shape"], dtype=np.int16)
    flat = want.reshape(-1)
    view = np.lib.stride_tricks.as_strided(
        flat[c["offset"]:], shape=(c["num_blocks"], c["page"], c["entry"]),
        strides=(c["s0"] * 2, c["s1"] * 2, 2))
    blk, off = c["slots"] // c["page"], c["slots"] % c["page"]
    view[blk, off] = np.concatenate([kv_c, k_pe], axis=1) if pe else kv_c
    np.testing.assert_array_equal(out, want)
    # zero bleed: the neighbour layers stay zero
    le = c["page"] * c["entry"]
    o3 = out.reshape(c["num_blocks"], c["n_layers"], le)
    assert not o3[:, 0].any() and not o3[:, 2].any()
    # read-back: every token's row is found at its slot
    np.testing.assert_array_equal(o3[:, 1].reshape(-1, c["entry"])[c["slots"]][:, :512], kv_c)


def test_cache_write_skips_bad_slots_and_copies_bits():
    kv_c = np.array([[np.nan, -0.0], [1.0, 2.0], [3.0, 4.0]], dtype=np.float32)
    kv_c_bits = kv_c.view(np.int32).copy()
    kv_c_bits[0, 0] = 0x7FC01234  # a NaN with a payload
    k_pe = np.array([[5.0], [6.0], [7.0]], dtype=np.float32).view(np.int32)
    buf = np.full(2 * 2 * 3, 99, dtype=np.int32)
    out = oracle.cache_write(buf, kv_c_bits, k_pe, [0, -5, 4], 0, 2, 2, 6, 3)
    assert out[0] == 0x7FC01234 and out[1] == np.float32(-0.0).view(np.int32)
    assert out[2] == k_pe[0, 0]
    assert np.all(out[3:] == 99)  # slot -5 and slot 4 (= NB*page) are skipped


# ------------------------------------------------------------ interleaved rope


def _rope_complex(x, positions, base):
    """The rotation as complex multiplication (numpy complex exp): pair
    (2i, 2i+1) is the number x[2i] + j x[2i+1], turned by exp(j theta_i)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    freq = np.power(float(base), -np.arange(0, d, 2, dtype=np.float64) / d)
    angle = np.asarray(positions, dtype=np.float64).reshape(-1, *([1] * (x.ndim - 1))) * freq
    z = z * np.exp(1j * angle)
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


@pytest.mark.parametrize("d_rope", [2, 8, 64])
def test_rope_matches_complex_rotation(d_rope):
    x, pos = mi.rope_case(1, d_rope=d_rope)
    got = oracle.rope_interleaved(x, pos, mi.ROPE_BASE)
    want = _rope_complex(x, pos, mi.ROPE_BASE)
    assert np.max(np.abs(got - want)) < 1e-12
    # large positions (long contexts) and another base
    x, pos = mi.rope_case(2, d_rope=d_rope, pos_step=9973, pos_offset=100_000)
    got = oracle.rope_interleaved(x, pos, 10_000.0)
    assert np.max(np.abs(got - _rope_complex(x, pos, 10_000.0))) < 1e-9


def test_rope_first_pair_turns_by_the_position():
    # i = 0 has frequency base^0 = 1: (1, 0) goes to (cos p, sin p), counter-clockwise
    pos = np.array([0, 1, 13, 78], dtype=np.int32)
    x = np.zeros((4, 1, 8))
    x[:, 0, 0] = 1.0
    got = oracle.rope_interleaved(x, pos, mi.ROPE_BASE)
    for t, p in enumerate(pos):
        assert got[t, 0, 0] == pytest.approx(math.cos(p), abs=1e-15)
        assert got[t, 0, 1] == pytest.approx(math.sin(p), abs=1e-15)
        assert np.all(got[t, 0, 2:] == 0.0)
    # the last pair of d = 8 turns by p * base^(-6/8)
    x = np.zeros((1, 1, 8))
    x[0, 0, 6] = 1.0
    got = oracle.rope_interleaved(x, np.array([78], np.int32), mi.ROPE_BASE)
    th = 78 * mi.ROPE_BASE ** (-0.75)
    assert got[0, 0, 6] == pytest.approx(math.cos(th), abs=1e-15)
    assert got[0, 0, 7] == pytest.approx(math.sin(th), abs=1e-15)


def test_rope_invariants():
    x, pos = mi.rope_case(3, d_rope=64)
    x = x.astype(np.float64)
    y = oracle.rope_interleaved(x, pos, mi.ROPE_BASE)
    # position 0 is the identity, exactly
    assert np.array_equal(oracle.rope_interleaved(x, np.zeros_like(pos), mi.ROPE_BASE), x)
    # each pair keeps its length
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(n0 - n1)) < 1e-13
    # turning back by -p recovers x
    back = oracle.rope_interleaved(y, -pos, mi.ROPE_BASE)
    assert np.max(np.abs(back - x)) < 1e-13
    # [T, d] is the V = 1 case
    assert np.array_equal(oracle.rope_interleaved(x[:, 0, :], pos, mi.ROPE_BASE), y[:, 0, :])


def test_rope_width_zero_is_a_no_op():
    x = np.zeros((2, 3, 0))
    got = oracle.rope_interleaved(x, np.array([0, 5], np.int32), mi.ROPE_BASE)
    assert got.shape == x.shape


# ------------------------------------------------------------------ fp8 e4m3
# [P3] dense fp8 decode tests keep the cache as torch.float8_e4m3fn: torch's
# own conversion of that dtype is the library route the oracle's format code
# is pinned to, plus closed forms of the OCP E4M3 encoding.


def _torch_e4m3_values(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.double().numpy()


def _torch_e4m3_codes(values):
    return torch.from_numpy(np.asarray(values, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256)
    got = oracle.e4m3_decode(codes)
    want = _torch_e4m3_values(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.isnan(got).sum() == 2  # S.1111.111 only


def test_e4m3_decode_closed_forms():
    d = lambda c: float(oracle.e4m3_decode([c])[0])  # noqa: E731
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9  # subnormals m * 2^-9
    assert d(0x08) == 2.0 ** -6  # smallest normal: exponent 1 - 7
    assert d(0x38) == 1.0 and d(0x3C) == 1.5 and d(0xB8) == -1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    vals = oracle.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)  # codes order like their values


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    pos = oracle.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2  # exact ties between neighbours
    parts = [
        rng.standard_normal(20000) * 0.1,
        rng.standard_normal(20000) * 60.0,
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000),  # subnormal range
        mids, -mids,
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        np.nextafter(mids.astype(np.float32), np.float32(-np.inf)),
        pos, -pos,
    ]
    v = np.concatenate([np.asarray(x, dtype=np.float32) for x in parts])
    v = v[np.abs(v) <= 448.0]
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3_codes(v))


def test_e4m3_encode_ties_saturation_nan_and_sign():
    e = lambda x: int(oracle.e4m3_encode([x])[0])  # noqa: E731
    assert e(2.0 ** -10) == 0x00  # halfway between 0 and 2^-9: the even code 0
    assert e(3 * 2.0 ** -10) == 0x02  # halfway between codes 1 and 2: code 2
    assert e(1.0625) == 0x38  # halfway between 1 and 1.125: mantissa 0
    assert e(1.1875) == 0x3A  # halfway between 1.125 and 1.25: mantissa 2
    assert e(449.0) == 0x7E and e(1e9) == 0x7E and e(float("inf")) == 0x7E
    assert e(-1e9) == 0xFE and e(float("-inf")) == 0xFE
    assert e(float("nan")) in (0x7F, 0xFF)
    assert e(-0.0) == 0x80 and e(-1e-12) == 0x80 and e(1e-12) == 0x00
    fin = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(fin)), fin)


def test_fp8_cache_write_places_quantised_rows():
    # a layer view of a block-major byte allocation, skipped slots, and codes
    # that must equal torch's e4m3 conversion of x / scale taken in float32
    rng = np.random.default_rng(6)
    T, L, R, NB, PG, layers, layer = 40, 16, 8, 6, 8, 3, 1
    E = L + R
    kv_c = (rng.standard_normal((T, L)) * 3).astype(np.float32)
    k_pe = (rng.standard_normal((T, R)) * 3).astype(np.float32)
    slots = rng.permutation(NB * PG)[:T].astype(np.int64)
    slots[3] = -1
    slots[7] = NB * PG
    scale = np.float32(0.37)
    buf = rng.integers(0, 256, size=(NB, layers, PG, E)).astype(np.uint8)
    got = oracle.cache_write_fp8(buf, kv_c, k_pe, slots, scale, layer * PG * E, NB, PG,
                                 layers * PG * E, E)
    want = buf.copy()
    rows = np.concatenate([kv_c, k_pe], axis=1)
    codes = _torch_e4m3_codes(rows / scale)  # float32 division, as in the oracle
    for t in range(T):
        if 0 <= slots[t] < NB * PG:
            want[slots[t] // PG, layer, slots[t] % PG] = codes[t]
    assert np.array_equal(got, want)


def test_fp8_attend_reduces_to_the_bf16_decode():
    # descales 1: attention over the decoded cache (torch's decode); descales
    # a, b: scores see q * a and keys * b, values scale by b, which equals
    # b * attention with query q * a * b over the unscaled keys
    rng = np.random.default_rng(7)
    B, Sq, N, L, R, NB, PG = 2, 2, 4, 16, 8, 8, 16
    E = L + R
    q = rng.standard_normal((B, Sq, N, E))
    codes = _torch_e4m3_codes(rng.standard_normal((NB, PG, E)) * 0.5)
    bt = np.stack([rng.permutation(NB)[:4] for _ in range(B)]).astype(np.int32)
    sl = np.array([37, 50], dtype=np.int32)
    vals = _torch_e4m3_values(codes)
    o1, l1 = oracle.attend_paged_fp8(q, codes, bt, sl, 0.3, True, L, 1.0, 1.0)
    o0, l0 = oracle.attend_paged(q, vals, bt, sl, 0.3, True, L)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)
    a, b = 0.75, 2.5
    o2, l2 = oracle.attend_paged_fp8(q, codes, bt, sl, 0.3, True, L, a, b)
    o3, l3 = oracle.attend_paged(q * a * b, vals, bt, sl, 0.3, True, L)
    np.testing.assert_allclose(o2, b * o3, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l3, rtol=1e-12, atol=1e-12)


# ------------------------------------------------- naive (decompressed) prefill
def _rand(rng, *shape):
    return rng.uniform(-1.0, 1.0, size=shape)


def test_decompress_kv_against_einsum_and_broadcast_rope():
    """k = [c_kv . W_UK_T[h]^T | k_pe], v = c_kv . W_UV[h], by numpy einsum in
    float64; every head carries the token's one k_pe row ([P1] broadcast
    concat case)."""
    rng = np.random.default_rng(11)
    T, N, P, R, V, L = 7, 3, 5, 4, 6, 9
    c_kv, k_pe = _rand(rng, T, L), _rand(rng, T, R)
    w_uk_t, w_uv = _rand(rng, N, P, L), _rand(rng, N, L, V)
    k, v = oracle.decompress_kv(c_kv, k_pe, w_uk_t, w_uv)
    np.testing.assert_allclose(k[:, :, :P], np.einsum("tl,hpl->thp", c_kv, w_uk_t), rtol=1e-13,
                               atol=1e-14)
    np.testing.assert_allclose(v, np.einsum("tl,hlv->thv", c_kv, w_uv), rtol=1e-13, atol=1e-14)
    for h in range(N):
        assert np.array_equal(k[:, h, P:], k_pe)


def test_decompress_kv_selection_weights_closed_form():
    """W_UK_T[h, p, l] = [l == p + h] picks latent column p + h; W_UV[h, l, d]
    = [l == 2d + h] picks column 2d + h. A transposed weight or a swapped
    head index picks other columns."""
    rng = np.random.default_rng(12)
    T, N, P, V, L = 5, 3, 4, 3, 8
    c_kv = _rand(rng, T, L)
    w_uk_t = np.zeros((N, P, L))
    w_uv = np.zeros((N, L, V))
    for h in range(N):
        for p in range(P):
            w_uk_t[h, p, p + h] = 1.0
        for d in range(V):
            w_uv[h, 2 * d + h, d] = 1.0
    k, v = oracle.decompress_kv(c_kv, None, w_uk_t, w_uv)
    assert k.shape == (T, N, P)
    for h in range(N):
        assert np.array_equal(k[:, h, :], c_kv[:, h:h + P])
        assert np.array_equal(v[:, h, :], c_kv[:, h:h + 2 * V:2])


def _sdpa_heads(q, k, v, pos, scale, causal):
    """Per-head attention through torch's float64 scaled_dot_product_attention
    with an explicit suffix-aligned causal mask."""
    qt = torch.from_numpy(q).permute(1, 0, 2).contiguous()
    kt = torch.from_numpy(k).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).contiguous()
    j = torch.arange(k.shape[0]).unsqueeze(0)
    mask = (j <= torch.as_tensor(pos).unsqueeze(1)) if causal else torch.ones(len(pos), k.shape[0],
                                                                              dtype=torch.bool)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return out.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("nq,T,N,DK,DV,causal", [
    (6, 6, 3, 12, 5, True), (3, 11, 2, 8, 7, True), (4, 9, 4, 16, 16, False), (1, 13, 2, 6, 3, True),
])
def test_mha_vs_sdpa_float64(nq, T, N, DK, DV, causal):
    rng = np.random.default_rng(nq * 100 + T)
    q, k, v = _rand(rng, nq, N, DK), _rand(rng, T, N, DK), _rand(rng, T, N, DV)
    pos = np.arange(nq) + T - nq
    out, lse = oracle.mha(q, k, v, pos, 0.37, causal)
    np.testing.assert_allclose(out, _sdpa_heads(q, k, v, pos, 0.37, causal), rtol=1e-11, atol=1e-12)
    # lse against its definition, row by row with a visible-key count
    i, h = nq - 1, N - 1
    nvis = pos[i] + 1 if causal else T
    s = 0.37 * (k[:nvis, h, :] @ q[i, h, :])
    assert math.isclose(lse[i, h], math.log(np.exp(s).sum()), rel_tol=1e-12)


def test_mha_closed_forms():
    rng = np.random.default_rng(13)
    N, DK, DV, T = 2, 8, 4, 6
    q, k, v = _rand(rng, T, N, DK), _rand(rng, T, N, DK), _rand(rng, T, N, DV)
    pos = np.arange(T)
    # query 0 sees only key 0: out = v[0], lse = its scaled score
    out, lse = oracle.mha(q, k, v, pos, 0.5, True)
    np.testing.assert_allclose(out[0], v[0], rtol=1e-14)
    np.testing.assert_allclose(lse[0], 0.5 * np.einsum("hd,hd->h", q[0], k[0]), rtol=1e-13)
    # values all one: softmax rows sum to one
    out1, _ = oracle.mha(q, k, np.ones_like(v), pos, 0.5, True)
    np.testing.assert_allclose(out1, 1.0, rtol=1e-13)
    # q = 0: uniform weights, out = mean of the visible values, lse = ln n
    out0, lse0 = oracle.mha(np.zeros_like(q), k, v, pos, 0.5, True)
    for i in range(T):
        np.testing.assert_allclose(out0[i], v[:i + 1].mean(axis=0), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse0[i], math.log(i + 1), rtol=1e-13, atol=1e-15)
    # a query with no visible key (more queries than keys): 0 and -inf
    outn, lsen = oracle.mha(q[:3], k[:1], v[:1], np.array([-2, -1, 0]), 0.5, True)
    assert np.all(outn[:2] == 0.0) and np.all(np.isneginf(lsen[:2]))
    np.testing.assert_allclose(outn[2], v[0], rtol=1e-14)


@pytest.mark.parametrize("N,P,R,V,L,nq,T,causal", [
    (4, 24, 8, 32, 64, 6, 6, True), (3, 12, 4, 20, 48, 3, 11, True), (4, 32, 0, 32, 64, 5, 9, True),
    (2, 16, 8, 16, 32, 4, 7, False),
])
def test_decompressed_prefill_equals_absorbed(N, P, R, V, L, nq, T, causal):
    """The naive route (decompress, then multi-head attention) and the absorbed
    route (fold q, attend over latent rows, un-project) compute one result
    ([P2] gate 1 checks the kernels against both oracle forms); the absorbed
    route never forms per-head keys or values."""
    rng = np.random.default_rng(N * 1000 + T)
    q_nope, c_kv = _rand(rng, nq, N, P), _rand(rng, T, L)
    q_pe, k_pe = (_rand(rng, nq, N, R), _rand(rng, T, R)) if R else (None, None)
    w_uk_t, w_uv = _rand(rng, N, P, L) / math.sqrt(L), _rand(rng, N, L, V) / math.sqrt(L)
    pos = np.arange(nq) + T - nq
    scale = 1.0 / math.sqrt(P + R)
    k, v = oracle.decompress_kv(c_kv, k_pe, w_uk_t, w_uv)
    q = np.concatenate([q_nope, q_pe], axis=2) if R else q_nope
    out, lse = oracle.mha(q, k, v, pos, scale, causal)
    want, _, _, want_lse = oracle.absorbed(q_nope, q_pe, c_kv, k_pe, w_uk_t, w_uv, pos, scale,
                                           causal)
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, want_lse, rtol=1e-12, atol=1e-13)


def test_mha_varlen_equals_per_sequence_calls():
    rng = np.random.default_rng(14)
    N, DK, DV = 2, 8, 4
    lens_q, lens_k = [3, 0, 5, 2], [7, 4, 5, 1]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lens_q)]), np.concatenate([[0], np.cumsum(lens_k)])
    q, k, v = _rand(rng, cu_q[-1], N, DK), _rand(rng, cu_k[-1], N, DK), _rand(rng, cu_k[-1], N, DV)
    out, lse = oracle.mha_varlen(q, k, v, cu_q, cu_k, 0.3, True)
    for b in range(4):
        if lens_q[b] == 0:
            continue
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        pos = np.arange(lens_q[b]) + lens_k[b] - lens_q[b]
        np.testing.assert_allclose(out[qs], _sdpa_heads(q[qs], k[ks], v[ks], pos, 0.3, True)
                                   if min(pos) >= 0 else oracle.mha(q[qs], k[ks], v[ks], pos, 0.3,
                                                                    True)[0], rtol=1e-11, atol=1e-12)
    # sequence 3 has 2 queries on 1 key: its first query sees nothing
    assert np.all(out[cu_q[3]] == 0.0) and np.isneginf(lse[cu_q[3]]).all()


# ------------------------------------------------------- sparse fp8 decode
def test_dsmla_rows_against_torch_views():
    """Entry decode against torch's own float8_e4m3fn and bfloat16 views of the
    bytes and numpy's float32 view of the scales."""
    e = mi.dsmla_payload(3, 2, 16, scales="random").reshape(-1, oracle.DSMLA_ENTRY)
    rows = oracle.dsmla_rows(e)
    codes = torch.from_numpy(e[:, :512].copy()).view(torch.float8_e4m3fn).double().numpy()
    sc = np.frombuffer(e[:, 512:528].tobytes(), dtype=np.float32).reshape(-1, 4).astype(np.float64)
    rope = torch.from_numpy(e[:, 528:].copy()).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(rows[:, :512], codes * np.repeat(sc, 128, axis=1))
    np.testing.assert_array_equal(rows[:, 512:], rope)
    # scale j governs codes 128j .. 128j + 127 only
    e2 = e.copy()
    e2[:, 516:520] = np.frombuffer(np.float32(3.0).tobytes(), np.uint8)
    r2 = oracle.dsmla_rows(e2)
    np.testing.assert_array_equal(r2[:, 128:256], codes[:, 128:256] * 3.0)
    np.testing.assert_array_equal(r2[:, :128], rows[:, :128])


def test_sparse_decode_with_every_slot_equals_dense_decode():
    """Indices listing a sequence's slots in order give the dense paged decode
    over the same decoded rows (the page's sparse call reads the cache the
    dense call reads, through an index list instead of a block table)."""
    B, N, NB, PG = 2, 4, 8, 16
    pool = mi.dsmla_payload(4, NB, PG, scales="random")
    q = mi.normal(4, 64, (B, 1, N, 576), 0.1, mi.BF16)
    lens = [37, 64]
    bt = np.array([[0, 1, 2, 3], [4, 5, 6, 7]], dtype=np.int32)
    idx = np.full((B, 1, 80), -1, dtype=np.int32)
    for b in range(B):
        slots = (bt[b, np.arange(lens[b]) // PG] * PG + np.arange(lens[b]) % PG)
        idx[b, 0, :lens[b]] = slots
    o, lse = oracle.sparse_decode(q, pool, idx, 576 ** -0.5)
    od, lsed = oracle.attend_paged(q, oracle.dsmla_rows(pool), bt, lens, 576 ** -0.5, True, 512)
    np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, lsed, rtol=1e-13)


def test_sparse_decode_index_list_invariants():
    B, Sq, N, NB, PG, K = 2, 2, 3, 4, 16, 24
    pool = mi.dsmla_payload(5, NB, PG)
    q = mi.normal(5, 64, (B, Sq, N, 576), 0.1, mi.BF16)
    idx = mi.dsmla_indices(5, B, Sq, K, NB, PG, mode="random")
    o, lse = oracle.sparse_decode(q, pool, idx, 0.05)
    # order of the list does not matter; -1 and out-of-pool entries are no key
    perm = np.concatenate([idx[:, :, ::-1], np.full((B, Sq, 1), NB * PG + 5, np.int32)], 2)
    o2, lse2 = oracle.sparse_decode(q, pool, perm, 0.05)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)
    # every slot twice: the same output, lse grows by ln 2
    o3, lse3 = oracle.sparse_decode(q, pool, np.concatenate([idx, idx], 2), 0.05)
    np.testing.assert_allclose(o3, o, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse3, lse + math.log(2.0), rtol=1e-12)
    # no key at all: 0 and -inf
    o4, lse4 = oracle.sparse_decode(q, pool, np.full((B, Sq, 4), -1, np.int32), 0.05)
    assert np.all(o4 == 0.0) and np.all(np.isneginf(lse4))
    # one key: that key's latent row exactly
    one = np.full((B, Sq, 3), -1, np.int32)
    one[:, :, 1] = 7
    o5, _ = oracle.sparse_decode(q, pool, one, 0.05)
    np.testing.assert_array_equal(o5[0, 0, 0], oracle.dsmla_rows(pool)[0, 7, :512])
