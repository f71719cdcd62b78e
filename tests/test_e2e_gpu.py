"""End-to-end GPU parity: the four calls chained as a model layer uses them.

- Tiny fp32 prefill, then 32 decode steps that each append one latent row and
  decode one query (memra-engine 0.124.1 "tests/mla_gpu_forward.rs", gate 1
  prefill parity and gate 2 stepwise decode vs a full recompute).
- The NoPE absorbed prefill at full size (64 heads x 256, rank 512, 2048
  causal queries), checked stage by stage on sampled rows the oracle computes
  one by one.
- A bf16 decode step at V2-Lite geometry against the naive (decompressed)
  MLA oracle.
- HIP-graph capture of a step: every replay equals the eager result.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from helpers import assert_close, dev, say, to_np

pytestmark = pytest.mark.gpu


def t_dev(x, dtype):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(td).to(dev())


def test_tiny_fp32_prefill_then_stepwise_decode():
    import mla_absorbed_decode_amd as mla

    c = mi.tiny_prefill_decode(0)
    d, T, scale = c["dims"], c["t"], c["scale"]
    N, L, E = d.n_head, d.kv_rank, d.entry
    f32 = torch.float32
    w_uk, w_uv = t_dev(c["w_uk_t"], "f32"), t_dev(c["w_uv"], "f32")
    q_nope, q_pe = t_dev(c["q_nope"], "f32"), t_dev(c["q_pe"], "f32")
    c_kv, k_pe = t_dev(c["c_kv"], "f32"), t_dev(c["k_pe"], "f32")
    want = oracle.naive(c["q_nope"], c["q_pe"], c["c_kv"], c["k_pe"], c["w_uk_t"], c["w_uv"],
                        np.arange(T), scale, True)
    bt = torch.zeros(1, 1, dtype=torch.int32, device=dev())

    # prefill: all T rows written, T causal queries
    say("[e2e] tiny fp32 prefill 64 x 64")
    cache = torch.full((1, T, E), float("nan"), dtype=f32, device=dev())
    mla.mla_concat_and_cache(c_kv, k_pe, torch.arange(T, dtype=torch.int64, device=dev()), cache)
    q = torch.empty(1, T, N, E, dtype=f32, device=dev())
    mla.mla_absorb_q(q_nope, w_uk, q_pe, q[0])
    o_lat = torch.empty(1, T, N, L, dtype=f32, device=dev())
    mla.mla_decode_attend(q, cache, bt, torch.tensor([T], dtype=torch.int32, device=dev()), T,
                          scale, True, o_lat, None)
    out = torch.empty(T, N, d.d_v, dtype=f32, device=dev())
    mla.mla_v_up(o_lat[0], w_uv, out)
    torch.cuda.synchronize()
    assert_close(to_np(out), want, "f32", "tiny fp32 prefill")

    # decode: rows 0..31 resident, then each step appends row t and decodes query t
    say("[e2e] tiny fp32 stepwise decode, steps 32..63")
    cache.fill_(float("nan"))
    half = T // 2
    mla.mla_concat_and_cache(c_kv[:half], k_pe[:half],
                             torch.arange(half, dtype=torch.int64, device=dev()), cache)
    qs = torch.empty(1, 1, N, E, dtype=f32, device=dev())
    o1 = torch.empty(1, 1, N, L, dtype=f32, device=dev())
    o2 = torch.empty(1, N, d.d_v, dtype=f32, device=dev())
    for t in range(half, T):
        mla.mla_concat_and_cache(c_kv[t:t + 1], k_pe[t:t + 1],
                                 torch.tensor([t], dtype=torch.int64, device=dev()), cache)
        mla.mla_absorb_q(q_nope[t:t + 1], w_uk, q_pe[t:t + 1], qs[:, 0])
        mla.mla_decode_attend(qs, cache, bt, torch.tensor([t + 1], dtype=torch.int32, device=dev()),
                              t + 1, scale, True, o1, None)
        mla.mla_v_up(o1[:, 0], w_uv, o2)
        torch.cuda.synchronize()
        assert_close(to_np(o2)[0], want[t], "f32", f"decode step {t}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nope_prefill_full_size_sampled(dtype):
    import mla_absorbed_decode_amd as mla

    c = mi.nope_prefill(0, dtype=dtype)
    d, T, scale = c["dims"], c["t"], c["scale"]
    N, P, L, V = d.n_head, d.d_nope, d.kv_rank, d.d_v
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"[e2e] NoPE prefill {dtype}: {N} heads x {P}, {T} causal queries")
    q_nope = t_dev(c["q_nope"], dtype)
    w_uk, w_uv = t_dev(c["w_uk_t"], dtype), t_dev(c["w_uv"], dtype)
    c_kv = t_dev(c["c_kv"], dtype)
    page = 64
    nb = T // page
    cache = torch.full((nb, page, L), float("nan"), dtype=td, device=dev())
    mla.mla_concat_and_cache(c_kv, None, torch.arange(T, dtype=torch.int64, device=dev()), cache)
    q = torch.empty(1, T, N, L, dtype=td, device=dev())
    mla.mla_absorb_q(q_nope, w_uk, None, q[0])
    o_lat = torch.empty(1, T, N, L, dtype=td, device=dev())
    lse = torch.empty(1, T, N, dtype=torch.float32, device=dev())
    bt = torch.arange(nb, dtype=torch.int32, device=dev()).view(1, nb)
    mla.mla_decode_attend(q, cache, bt, torch.tensor([T], dtype=torch.int32, device=dev()), T,
                          scale, True, o_lat, lse)
    out = torch.empty(T, N, V, dtype=td, device=dev())
    mla.mla_v_up(o_lat[0], w_uv, out)
    torch.cuda.synchronize()

    # sampled queries, every head of each: the first two, the last, every 16th
    # from 5 (every tile of 32 queries and every 128-row block is hit) and a
    # seeded spread
    rng = np.random.default_rng(5)
    qs = np.unique(np.concatenate([[0, 1, T - 1], np.arange(5, T, 16), rng.integers(0, T, 9)]))
    q_dev = to_np(q[0])[qs]          # [nq, N, L] as the device stored it
    o_dev = to_np(o_lat[0])[qs]
    # stage 1: the fold of the sampled rows
    want_q = oracle.fold_q(c["q_nope"][qs], c["w_uk_t"])
    assert_close(q_dev, want_q, dtype, "NoPE fold (sampled rows)")
    # stage 2: attention of the device's q rows against the cache rows
    kv = c["c_kv"]
    want_o, want_lse, _ = oracle.attend_seq(q_dev, kv, qs, scale, True, L)
    assert_close(o_dev, want_o, dtype, "NoPE attention (sampled rows)")
    np.testing.assert_allclose(to_np(lse[0])[qs], want_lse, rtol=1e-4, atol=1e-4)
    # stage 3: the un-projection of the device's o_lat rows
    want_out = oracle.v_up(o_dev, c["w_uv"])
    assert_close(to_np(out)[qs], want_out, dtype, "NoPE v up (sampled rows)")
    # nothing left unwritten anywhere
    assert torch.isfinite(out.float()).all()


def test_bf16_step_at_v2lite_geometry_matches_naive():
    import mla_absorbed_decode_amd as mla

    d = mi.V2_LITE
    seqlens = np.array([700, 65, 1500, 2, 333], dtype=np.int32)
    B, page = len(seqlens), 64
    q_nope, q_pe, c_kv, k_pe = mi.mla_activations(3, d, B, int(seqlens.sum()), "bf16",
                                                  dist="normal", std=0.1)
    w_uk_t, w_uv = mi.mla_weights(3, d, "bf16", dist="normal", std=0.1)
    case = mi.decode_case(3, d, "bf16", seqlens, page=page)
    bt = case.block_table
    offs = np.concatenate([[0], np.cumsum(seqlens)[:-1]])
    rows = np.concatenate([c_kv, k_pe], axis=1)
    pool = np.full((case.num_blocks, page, d.entry), np.nan, dtype=np.float32)
    slots = []
    for b, s in enumerate(seqlens):
        for j in range(s - 1):
            pool[bt[b, j // page], j % page] = rows[offs[b] + j]
        j = s - 1
        slots.append(int(bt[b, j // page]) * page + j % page)
    last = offs + seqlens - 1
    say(f"[e2e] bf16 step, 16 heads, seqlens {seqlens.tolist()}")
    cache = t_dev(pool, "bf16")
    q = torch.empty(B, 1, d.n_head, d.entry, dtype=torch.bfloat16, device=dev())
    mla.mla_absorb_q(t_dev(q_nope, "bf16"), t_dev(w_uk_t, "bf16"), t_dev(q_pe, "bf16"), q[:, 0])
    mla.mla_concat_and_cache(t_dev(c_kv[last], "bf16"), t_dev(k_pe[last], "bf16"),
                             torch.tensor(slots, dtype=torch.int64, device=dev()), cache)
    o_lat = torch.empty(B, 1, d.n_head, d.kv_rank, dtype=torch.bfloat16, device=dev())
    mla.mla_decode_attend(q, cache, torch.from_numpy(bt).to(dev()),
                          torch.from_numpy(seqlens).to(dev()), int(seqlens.max()), d.entry ** -0.5,
                          True, o_lat, None)
    out = torch.empty(B, d.n_head, d.d_v, dtype=torch.bfloat16, device=dev())
    mla.mla_v_up(o_lat[:, 0], t_dev(w_uv, "bf16"), out)
    torch.cuda.synchronize()
    for b, s in enumerate(seqlens):
        sl = slice(offs[b], offs[b] + s)
        want = oracle.naive(q_nope[b:b + 1], q_pe[b:b + 1], c_kv[sl], k_pe[sl], w_uk_t, w_uv,
                            [s - 1], d.entry ** -0.5, True)
        assert_close(to_np(out[b:b + 1]), want, "bf16", f"sequence {b} (length {s})")


def test_graph_replays_equal_eager():
    """Each replay of a captured step, with other device work and host
    synchronisation between replays, reproduces the eager outputs bit for bit."""
    import mla_absorbed_decode_amd as mla

    d = mi.V2_LITE
    c = mi.decode_case(9, d, "bf16", [900, 64, 2100, 17], max_blocks=40)
    B = c.batch
    q_nope, q_pe, _, _ = mi.mla_activations(9, d, B, 1, "bf16", dist="normal", std=0.1)
    w_uk_t, w_uv = mi.mla_weights(9, d, "bf16", dist="normal", std=0.1)
    qn, qp = t_dev(q_nope, "bf16"), t_dev(q_pe, "bf16")
    wk, wv = t_dev(w_uk_t, "bf16"), t_dev(w_uv, "bf16")
    cache = t_dev(c.pool, "bf16")
    bt = torch.from_numpy(c.block_table).to(dev())
    sl = torch.from_numpy(c.seqlens).to(dev())
    q = torch.empty(B, 1, d.n_head, d.entry, dtype=torch.bfloat16, device=dev())
    o_lat = torch.empty(B, 1, d.n_head, d.kv_rank, dtype=torch.bfloat16, device=dev())
    lse = torch.empty(B, 1, d.n_head, dtype=torch.float32, device=dev())
    out = torch.empty(B, d.n_head, d.d_v, dtype=torch.bfloat16, device=dev())
    nbytes = mla.mla_decode_workspace_size(B, 1, d.n_head, d.kv_rank, c.max_seqlen, c.page,
                                           torch.bfloat16)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev())

    def step():
        mla.mla_absorb_q(qn, wk, qp, q[:, 0])
        mla.mla_decode_attend(q, cache, bt, sl, c.max_seqlen, c.scale, True, o_lat, lse,
                              workspace=ws)
        mla.mla_v_up(o_lat[:, 0], wv, out)

    say("[e2e] eager step")
    step()
    torch.cuda.synchronize()
    ref = (q.clone(), o_lat.clone(), lse.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device=dev())
    for i in range(4):
        for x in (q, o_lat, lse, out):
            x.fill_(float("nan"))
        scratch.add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        say(f"[e2e] graph replay {i}")
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((q, o_lat, lse, out), ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {i}"


def test_prefill_and_sparse_graph_replays_equal_eager():
    """The naive prefill (decompress, then attend; 300 tokens, so the pipelined
    product tiles run) and a split sparse decode, captured in one graph: every
    replay, with eager work and synchronisation between replays, reproduces
    the eager outputs bit for bit."""
    import mla_absorbed_decode_amd as mla

    d = mi.V2_LITE
    T = 300
    q_nope, q_pe, c_kv, k_pe = mi.mla_activations(10, d, T, T, "bf16")
    w_uk_t, w_uv = mi.mla_weights(10, d, "bf16")
    qd = t_dev(np.concatenate([q_nope, q_pe], 2), "bf16")
    ckv, kpe = t_dev(c_kv, "bf16"), t_dev(k_pe, "bf16")
    wk, wv = t_dev(w_uk_t, "bf16"), t_dev(w_uv, "bf16")
    k = torch.empty(T, d.n_head, d.d_nope + d.d_rope, dtype=torch.bfloat16, device=dev())
    v = torch.empty(T, d.n_head, d.d_v, dtype=torch.bfloat16, device=dev())
    out = torch.empty(T, d.n_head, d.d_v, dtype=torch.bfloat16, device=dev())
    plse = torch.empty(T, d.n_head, dtype=torch.float32, device=dev())
    cu = torch.tensor([0, 100, T], dtype=torch.int32, device=dev())
    # sparse: 2 tokens x 128 heads, top-256 random lists (split over workgroups)
    pool = torch.from_numpy(mi.dsmla_payload(10, 16, 64, scales="random")).to(dev())
    sq = t_dev(mi.normal(10, 64, (2, 1, 128, 576), 0.1, "bf16"), "bf16")
    idx = torch.from_numpy(mi.dsmla_indices(10, 2, 1, 256, 16, 64, mode="random")).to(dev())
    sout = torch.empty(2, 1, 128, 512, dtype=torch.bfloat16, device=dev())
    slse = torch.empty(2, 1, 128, dtype=torch.float32, device=dev())
    need = mla.mla_sparse_workspace_size(2, 128, 256)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())

    def step():
        mla.mla_decompress_kv(ckv, kpe, wk, wv, k, v)
        mla.mla_prefill_attend(qd, k, v, cu, cu, 200, (d.d_nope + d.d_rope) ** -0.5, True, out,
                               plse)
        mla.mla_sparse_decode_fp8(sq, pool, idx, 576 ** -0.5, sout, slse, workspace=ws)

    say("[e2e] eager prefill + sparse step")
    step()
    torch.cuda.synchronize()
    outs = (k, v, out, plse, sout, slse)
    ref = tuple(x.clone() for x in outs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device=dev())
    for i in range(4):
        for x in outs:
            x.fill_(float("nan"))
        scratch.add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        say(f"[e2e] prefill + sparse graph replay {i}")
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {i}"
