"""GPU parity of the naive (decompressed) prefill route.

- mla_decompress_kv: per-head keys [c_kv . W_UK_T[h]^T | k_pe] and values
  c_kv . W_UV[h] against the oracle (memra-engine 0.124.1
  "tests/mla_gpu_forward.rs", the naive oracle; vllm.cpp
  "tests/vt/test_ops_mla_absorb.cpp", the broadcast ConcatMlaNopeRope case:
  the rope part must be the token's k_pe row, bit for bit, in every head).
- mla_prefill_attend: packed causal / full multi-head attention against the
  oracle's per-sequence attention, at every supported head width, with ragged
  tails, empty sequences and queries that see no key.
- The two calls chained (gate 1 of the memra page: the naive route must meet
  both oracle forms), including the full-size NoPE prefill (64 heads x 256,
  rank 512, 2048 causal queries) on sampled rows.
"""
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from helpers import assert_close, assert_lse_close, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


def _mla():
    import mla_absorbed_decode_amd as mla
    return mla


def _poisoned(shape, dtype=torch.bfloat16):
    t = torch.empty(shape, dtype=dtype, device=dev())
    t.fill_(float("nan"))
    return t


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


# ------------------------------------------------------------ decompression
@pytest.mark.parametrize("S,N,P,R,V", [(200, 16, 128, 64, 128), (77, 8, 256, 0, 256),
                                       (33, 3, 32, 16, 48), (600, 4, 32, 16, 48),
                                       (300, 2, 256, 0, 256)])
def test_decompress_kv_matches_oracle(S, N, P, R, V):
    mla = _mla()
    L = 512
    say(f"decompress_kv bf16 S={S} N={N} P={P} R={R} V={V}")
    dims = mi.Dims(n_head=N, d_nope=P, d_rope=R, d_v=V, kv_rank=L)
    _, _, c_kv, k_pe = mi.mla_activations(1, dims, 1, S, mi.BF16)
    w_uk_t, w_uv = mi.mla_weights(1, dims, mi.BF16)
    kw, vw = oracle.decompress_kv(c_kv, k_pe if R else None, w_uk_t, w_uv)
    k_out, v_out = _poisoned((S, N, P + R)), _poisoned((S, N, V))
    mla.mla_decompress_kv(to_dev(c_kv, "bf16"), to_dev(k_pe, "bf16") if R else None,
                          to_dev(w_uk_t, "bf16"), to_dev(w_uv, "bf16"), k_out, v_out)
    torch.cuda.synchronize()
    assert_close(to_np(k_out[:, :, :P]), kw[:, :, :P], "bf16", "k_nope")
    assert_close(to_np(v_out), vw, "bf16", "v")
    if R:
        want = _bits(to_dev(k_pe, "bf16"))
        got = _bits(k_out[:, :, P:])
        for h in range(N):
            assert np.array_equal(got[:, h], want), f"rope row of head {h} is not k_pe"


def test_decompress_kv_strided_views_and_f32():
    """Outputs written through non-contiguous views (a head-major buffer and a
    padded one) leave the padding untouched; f32 takes the f32 MFMA kernel, and
    a latent view that is not 16-byte aligned the plain one."""
    mla = _mla()
    S, N, P, R, V, L = 70, 4, 64, 64, 64, 512
    dims = mi.Dims(n_head=N, d_nope=P, d_rope=R, d_v=V, kv_rank=L)
    for dt in ("bf16", "f32"):
        say(f"decompress_kv strided views {dt}")
        _, _, c_kv, k_pe = mi.mla_activations(2, dims, 1, S, dt)
        w_uk_t, w_uv = mi.mla_weights(2, dims, dt)
        kw, vw = oracle.decompress_kv(c_kv, k_pe, w_uk_t, w_uv)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        kbuf = _poisoned((N, S, P + R + 8), tdt)      # head-major, padded rows
        vbuf = _poisoned((S, N, V + 16), tdt)
        k_out = kbuf[:, :, :P + R].transpose(0, 1)
        v_out = vbuf[:, :, :V]
        c_dev = to_dev(np.concatenate([c_kv, np.zeros((S, 8), np.float32)], 1), dt)[:, :L]
        mla.mla_decompress_kv(c_dev, to_dev(k_pe, dt), to_dev(w_uk_t, dt), to_dev(w_uv, dt), k_out,
                              v_out)
        torch.cuda.synchronize()
        assert_close(to_np(k_out[:, :, :P]), kw[:, :, :P], dt, "k_nope")
        assert_close(to_np(v_out), vw, dt, "v")
        assert np.array_equal(to_np(k_out[:, :, P:]), np.broadcast_to(k_pe[:, None, :], (S, N, R)))
        assert torch.isnan(kbuf[:, :, P + R:]).all() and torch.isnan(vbuf[:, :, V:]).all()
        # the latent rows one element into a padded buffer: 4-byte alignment only
        c_odd = to_dev(np.concatenate([np.zeros((S, 1), np.float32), c_kv,
                                       np.zeros((S, 7), np.float32)], 1), dt)[:, 1:L + 1]
        k2 = _poisoned((S, N, P + R), tdt)
        v2 = _poisoned((S, N, V), tdt)
        mla.mla_decompress_kv(c_odd, to_dev(k_pe, dt), to_dev(w_uk_t, dt), to_dev(w_uv, dt), k2, v2)
        torch.cuda.synchronize()
        assert_close(to_np(k2[:, :, :P]), kw[:, :, :P], dt, "k_nope, unaligned latent rows")
        assert_close(to_np(v2), vw, dt, "v, unaligned latent rows")


# ---------------------------------------------------------------- attention
def _mha_inputs(seed, N, DK, DV, lens_q, lens_k):
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    q = mi.uniform(seed, 50, (int(cu_q[-1]), N, DK), -1, 1, mi.BF16)
    k = mi.uniform(seed, 51, (int(cu_k[-1]), N, DK), -1, 1, mi.BF16)
    v = mi.uniform(seed, 52, (int(cu_k[-1]), N, DV), -1, 1, mi.BF16)
    return q, k, v, cu_q, cu_k


def _run_mha(q, k, v, cu_q, cu_k, scale, causal, max_q=None):
    mla = _mla()
    T, N = q.shape[:2]
    out = _poisoned((T, N, v.shape[2]))
    lse = torch.full((T, N), float("nan"), dtype=torch.float32, device=dev())
    cq = torch.from_numpy(cu_q).to(dev())
    ck = torch.from_numpy(cu_k).to(dev())
    mq = int(np.diff(cu_q).max()) if max_q is None else max_q
    mla.mla_prefill_attend(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), cq, ck, mq,
                           scale, causal, out, lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("DK,DV,N", [(192, 128, 4), (256, 256, 3), (128, 128, 2), (64, 64, 2),
                                      (192, 128, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_attend_varlen_matches_oracle(DK, DV, N, causal):
    # ragged sequences: one row, a partial tile, exactly one tile, several tiles
    # with a ragged tail on a longer cache (chunked prefill), an empty one
    lens_q, lens_k = [1, 37, 64, 130, 0, 5], [1, 40, 64, 200, 3, 5]
    say(f"prefill_attend DK={DK} DV={DV} N={N} causal={causal} lens_q={lens_q} lens_k={lens_k}")
    q, k, v, cu_q, cu_k = _mha_inputs(3, N, DK, DV, lens_q, lens_k)
    scale = DK ** -0.5
    want, want_lse = oracle.mha_varlen(q, k, v, cu_q, cu_k, scale, causal)
    out, lse = _run_mha(q, k, v, cu_q, cu_k, scale, causal)
    assert_close(to_np(out), want, "bf16", "out")
    assert_lse_close(to_np(lse), want_lse, "lse")


@pytest.mark.parametrize("DK,DV", [(192, 128), (256, 256)])
def test_prefill_attend_paired_query_tiles(DK, DV):
    # enough heads x sequences that a causal call pairs its query tiles (the
    # longest with the shortest, one workgroup for both): three 128-row tiles
    # (an odd count: the middle one alone), sequences of other lengths, a
    # chunked-prefill suffix and a sequence of one query
    lens_q, lens_k = [300, 129, 1, 257], [300, 200, 5, 300]
    N = 32
    say(f"prefill_attend paired tiles DK={DK} DV={DV} N={N} lens_q={lens_q} lens_k={lens_k}")
    q, k, v, cu_q, cu_k = _mha_inputs(7, N, DK, DV, lens_q, lens_k)
    scale = DK ** -0.5
    want, want_lse = oracle.mha_varlen(q, k, v, cu_q, cu_k, scale, True)
    out, lse = _run_mha(q, k, v, cu_q, cu_k, scale, True)
    assert_close(to_np(out), want, "bf16", "out")
    assert_lse_close(to_np(lse), want_lse, "lse")


def test_prefill_attend_queries_without_keys():
    """More queries than keys: the first queries of the suffix see nothing
    (out 0, lse -inf); a sequence with no keys at all likewise."""
    lens_q, lens_k = [70, 4], [20, 0]
    say(f"prefill_attend no visible key lens_q={lens_q} lens_k={lens_k}")
    q, k, v, cu_q, cu_k = _mha_inputs(4, 2, 192, 128, lens_q, lens_k)
    want, want_lse = oracle.mha_varlen(q, k, v, cu_q, cu_k, 0.1, True)
    out, lse = _run_mha(q, k, v, cu_q, cu_k, 0.1, True)
    got = to_np(out)
    assert np.all(got[:50] == 0.0) and np.all(got[70:] == 0.0)
    assert np.all(np.isneginf(to_np(lse)[:50])) and np.all(np.isneginf(to_np(lse)[70:]))
    assert_close(got[50:70], want[50:70], "bf16", "visible rows")
    assert_lse_close(to_np(lse), want_lse, "lse")


def test_prefill_attend_reruns_bit_identical_and_strided_views():
    """Reruns give the same bits; q, k, v and out read and written through
    views with padded rows and a head-major layout give the same bits too."""
    mla = _mla()
    lens_q, lens_k = [100, 33], [150, 33]
    say("prefill_attend reruns and views")
    q, k, v, cu_q, cu_k = _mha_inputs(5, 4, 192, 128, lens_q, lens_k)
    a, la = _run_mha(q, k, v, cu_q, cu_k, 0.07, True)
    b, lb = _run_mha(q, k, v, cu_q, cu_k, 0.07, True)
    assert np.array_equal(_bits(a), _bits(b)) and torch.equal(la, lb)
    T, S, N = q.shape[0], k.shape[0], 4
    qv = to_dev(np.concatenate([q, np.zeros((T, N, 8), np.float32)], 2), "bf16")[:, :, :192]
    kh = to_dev(np.ascontiguousarray(k.transpose(1, 0, 2)), "bf16").transpose(0, 1)
    vv = to_dev(np.concatenate([v, np.zeros((S, N, 24), np.float32)], 2), "bf16")[:, :, :128]
    obuf = _poisoned((N, T, 128))
    out = obuf.transpose(0, 1)
    mla.mla_prefill_attend(qv, kh, vv, torch.from_numpy(cu_q).to(dev()),
                           torch.from_numpy(cu_k).to(dev()), 100, 0.07, True, out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out.contiguous()), _bits(a))


# ---------------------------------------------------- naive route end to end
@pytest.mark.parametrize("t_q,t_kv", [(300, 300), (100, 300)])
def test_naive_prefill_meets_both_oracles(t_q, t_kv):
    """V2-Lite heads: decompress, then attend; compared with the naive and the
    absorbed oracle (the two forms of gate 1), chunked shape included."""
    mla = _mla()
    d = mi.V2_LITE
    N, P, R, V, L = d.n_head, d.d_nope, d.d_rope, d.d_v, d.kv_rank
    say(f"naive prefill V2-Lite heads t_q={t_q} t_kv={t_kv}")
    q_nope, q_pe, c_kv, k_pe = mi.mla_activations(6, d, t_q, t_kv, mi.BF16)
    w_uk_t, w_uv = mi.mla_weights(6, d, mi.BF16)
    scale = (P + R) ** -0.5
    pos = np.arange(t_q) + t_kv - t_q
    want_naive = oracle.naive(q_nope, q_pe, c_kv, k_pe, w_uk_t, w_uv, pos, scale, True)
    want_abs = oracle.absorbed(q_nope, q_pe, c_kv, k_pe, w_uk_t, w_uv, pos, scale, True)[0]
    k_out = _poisoned((t_kv, N, P + R))
    v_out = _poisoned((t_kv, N, V))
    mla.mla_decompress_kv(to_dev(c_kv, "bf16"), to_dev(k_pe, "bf16"), to_dev(w_uk_t, "bf16"),
                          to_dev(w_uv, "bf16"), k_out, v_out)
    q = to_dev(np.concatenate([q_nope, q_pe], 2), "bf16")
    out = _poisoned((t_q, N, V))
    cu_q = torch.tensor([0, t_q], dtype=torch.int32, device=dev())
    cu_k = torch.tensor([0, t_kv], dtype=torch.int32, device=dev())
    mla.mla_prefill_attend(q, k_out, v_out, cu_q, cu_k, t_q, scale, True, out)
    torch.cuda.synchronize()
    assert_close(to_np(out), want_naive, "bf16", "vs naive")
    assert_close(to_np(out), want_abs, "bf16", "vs absorbed")


def test_naive_prefill_nope_full_size_sampled():
    """The NoPE prefill workload (64 heads x 256, rank 512, t = 2048 causal,
    U[-1,1] activations, U[+-1/sqrt(512)] weights) through the naive route at
    full size; sampled query rows of four heads against the oracle, and
    sampled decompressed rows."""
    mla = _mla()
    c = mi.nope_prefill(0, mi.BF16)
    d, t, scale = c["dims"], c["t"], c["scale"]
    N, P, V, L = d.n_head, d.d_nope, d.d_v, d.kv_rank
    say(f"naive prefill NoPE full size t={t} N={N}")
    c_kv = to_dev(c["c_kv"], "bf16")
    k_out, v_out = _poisoned((t, N, P)), _poisoned((t, N, V))
    mla.mla_decompress_kv(c_kv, None, to_dev(c["w_uk_t"], "bf16"), to_dev(c["w_uv"], "bf16"),
                          k_out, v_out)
    out = _poisoned((t, N, V))
    lse = torch.empty((t, N), dtype=torch.float32, device=dev())
    cu = torch.tensor([0, t], dtype=torch.int32, device=dev())
    mla.mla_prefill_attend(to_dev(c["q_nope"], "bf16"), k_out, v_out, cu, cu, t, scale, True, out,
                           lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and not torch.isnan(k_out).any()
    heads = [0, 17, 40, N - 1]
    # tile edges, the last row, and every 64th row from 3 (every 128-row block)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 700, 1500, t - 1], np.arange(3, t, 64)]))
    kw, vw = oracle.decompress_kv(c["c_kv"][rows], None, c["w_uk_t"][heads], c["w_uv"][heads])
    assert_close(to_np(k_out[rows][:, heads]), kw, "bf16", "k rows")
    assert_close(to_np(v_out[rows][:, heads]), vw, "bf16", "v rows")
    want = oracle.naive(c["q_nope"][rows][:, heads], None, c["c_kv"], None, c["w_uk_t"][heads],
                        c["w_uv"][heads], rows, scale, True)
    assert_close(to_np(out[rows][:, heads]), want, "bf16", "out rows")
    # softmax normalisation holds at every row: lse is finite everywhere
    assert torch.isfinite(lse).all()
