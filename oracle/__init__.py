"""Double-precision CPU oracle for weight-absorbed MLA (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library and its Python binding
never do, and this package imports nothing from them.

Every function takes numpy arrays holding the exact values the device sees
(already rounded to the device dtype), widens them to float64 and calls the
plain C loops in ``mla_oracle.c``. The C file documents, per function, the
passage of the pages it follows:

  [P1] vllm.cpp "tests/vt/test_ops_mla_absorb.cpp"
  [P2] memra-engine 0.124.1 "tests/mla_gpu_forward.rs"
  [P3] vLLM "tests/kernels/attention/test_mla_cross_layer_kernel_equivalence.py"

Every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` against something other than itself (a library
routine, a closed form, an invariant, or a hand-derived fixture under
``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over output rows)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, dp, ip32, ip64, dbl, c_int = (
            ctypes.c_int64,
            ctypes.POINTER(ctypes.c_double),
            ctypes.POINTER(ctypes.c_int32),
            ctypes.POINTER(ctypes.c_int64),
            ctypes.c_double,
            ctypes.c_int,
        )
        u8p = ctypes.POINTER(ctypes.c_uint8)
        lib.mla_oracle_num_threads.restype = c_int
        lib.mla_oracle_set_num_threads.argtypes = [c_int]
        lib.mla_oracle_set_num_threads.restype = None
        lib.mla_oracle_bmm.argtypes = [i64] * 4 + [dp, i64, i64, i64] * 3
        lib.mla_oracle_bmm.restype = None
        lib.mla_oracle_attend_seq.argtypes = [i64] * 5 + [dp, ip64, dp, dbl, c_int, dp, dp, dp]
        lib.mla_oracle_attend_seq.restype = None
        lib.mla_oracle_gather_pages.argtypes = [i64, dp, i64, i64, ip32, i64, i64, i64, dp]
        lib.mla_oracle_gather_pages.restype = c_int
        lib.mla_oracle_attend_paged.argtypes = (
            [i64] * 5 + [dp, dp, i64, i64, ip32, i64, ip32, dbl, c_int, dp, dp]
        )
        lib.mla_oracle_attend_paged.restype = c_int
        lib.mla_oracle_naive.argtypes = [i64] * 7 + [dp] * 6 + [ip64, dbl, c_int, dp]
        lib.mla_oracle_naive.restype = None
        lib.mla_oracle_absorbed.argtypes = [i64] * 7 + [dp] * 6 + [ip64, dbl, c_int] + [dp] * 4
        lib.mla_oracle_absorbed.restype = None
        lib.mla_oracle_attend_split.argtypes = (
            [i64] * 5 + [dp, ip64, dp, dbl, c_int, ip64, i64, dp, dp]
        )
        lib.mla_oracle_attend_split.restype = None
        lib.mla_oracle_cache_write.argtypes = [i64] * 4 + [u8p, i64, u8p, i64, ip64, u8p] + [i64] * 6
        lib.mla_oracle_cache_write.restype = c_int
        lib.mla_oracle_rope_interleaved.argtypes = [i64, i64, i64, dp, ip32, dbl]
        lib.mla_oracle_rope_interleaved.restype = None
        fp = ctypes.POINTER(ctypes.c_float)
        lib.mla_oracle_e4m3_decode_array.argtypes = [i64, u8p, dp]
        lib.mla_oracle_e4m3_decode_array.restype = None
        lib.mla_oracle_e4m3_encode_array.argtypes = [i64, fp, u8p]
        lib.mla_oracle_e4m3_encode_array.restype = None
        lib.mla_oracle_cache_write_fp8.argtypes = (
            [i64] * 3 + [fp, fp, ip64, ctypes.c_float, u8p] + [i64] * 6
        )
        lib.mla_oracle_cache_write_fp8.restype = c_int
        lib.mla_oracle_decompress_kv.argtypes = [i64] * 6 + [dp] * 6
        lib.mla_oracle_decompress_kv.restype = None
        lib.mla_oracle_mha.argtypes = [i64] * 5 + [dp] * 3 + [ip64, dbl, c_int, dp, dp]
        lib.mla_oracle_mha.restype = None
        lib.mla_oracle_dsmla_rows.argtypes = [i64, u8p, i64, dp]
        lib.mla_oracle_dsmla_rows.restype = None
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def num_threads() -> int:
    """OpenMP threads the oracle runs on (honours OMP_NUM_THREADS)."""
    return int(_load().mla_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the following oracle calls."""
    _load().mla_oracle_set_num_threads(int(n))


def bmm_strided(a_buf, a_view, b_buf, b_view, shape):
    """out[g,m,n] = sum_k a[g,m,k] b[g,k,n] with operands given as (flat buffer,
    (offset, s0, s1, s2)) element views. Returns a dense [G,M,N] float64 array.
    ``shape`` is (G, M, K, N)."""
    G, M, K, N = shape
    a = _f64(a_buf).ravel()
    b = _f64(b_buf).ravel()
    ao, a0, a1, a2 = a_view
    bo, b0, b1, b2 = b_view
    out = np.zeros((G, M, N), dtype=np.float64)
    ap = ctypes.cast(a.ctypes.data + 8 * ao, ctypes.POINTER(ctypes.c_double))
    bp = ctypes.cast(b.ctypes.data + 8 * bo, ctypes.POINTER(ctypes.c_double))
    _load().mla_oracle_bmm(G, M, K, N, ap, a0, a1, a2, bp, b0, b1, b2, _dp(out), M * N, N, 1)
    return out


def bmm(a, b):
    """Dense out[g] = a[g] @ b[g]; a [G,M,K], b [G,K,N]."""
    a = _f64(a)
    b = _f64(b)
    G, M, K = a.shape
    N = b.shape[2]
    return bmm_strided(a, (0, M * K, K, 1), b, (0, K * N, N, 1), (G, M, K, N))


def fold_q(q_nope, w_uk_t):
    """q_lat[t,h,:] = q_nope[t,h,:] @ W_UK_T[h] (the q-side absorption fold).
    q_nope [T,N,P], w_uk_t [N,P,L] -> [T,N,L]."""
    q_nope = _f64(q_nope)
    T, N, P = q_nope.shape
    L = w_uk_t.shape[2]
    out = bmm_strided(q_nope, (0, P, N * P, 1), w_uk_t, (0, P * L, L, 1), (N, T, P, L))
    return np.ascontiguousarray(out.transpose(1, 0, 2))


def v_up(o_lat, w_uv):
    """out[t,h,:] = o_lat[t,h,:] @ W_UV[h] (the W_UV un-projection).
    o_lat [T,N,L], w_uv [N,L,V] -> [T,N,V]."""
    o_lat = _f64(o_lat)
    T, N, L = o_lat.shape
    V = w_uv.shape[2]
    out = bmm_strided(o_lat, (0, L, N * L, 1), w_uv, (0, L * V, V, 1), (N, T, L, V))
    return np.ascontiguousarray(out.transpose(1, 0, 2))


def attend_seq(q, kv, pos, scale, causal, L, want_probs=False):
    """Absorbed attention of q [nq,N,E] against contiguous rows kv [T,E].
    pos [nq] absolute query positions. Returns (o_lat [nq,N,L], lse [nq,N]
    natural log, probs [nq,N,T] or None)."""
    q = _f64(q)
    nq, N, E = q.shape
    kv = _f64(kv).reshape(-1, E)
    T = kv.shape[0]
    R = E - L
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    o = np.zeros((nq, N, L))
    lse = np.zeros((nq, N))
    probs = np.zeros((nq, N, max(T, 1))) if want_probs else None
    kvp = kv if T else np.zeros((1, E))
    _load().mla_oracle_attend_seq(
        nq, N, L, R, T, _dp(q), _i64p(pos), _dp(kvp), float(scale), int(bool(causal)), _dp(o),
        _dp(lse), _dp(probs) if want_probs else None,
    )
    if want_probs:
        probs = probs[:, :, :T]
    return o, lse, probs


def gather_pages(pool, block_table, b, seqlen):
    """Contiguous latent rows of sequence b from a paged pool [NB,PG,E]."""
    pool = _f64(pool)
    NB, PG, E = pool.shape
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    rows = np.zeros((max(seqlen, 1), E))
    rc = _load().mla_oracle_gather_pages(E, _dp(pool), NB, PG, _i32p(bt), bt.shape[1], b, seqlen,
                                         _dp(rows))
    if rc != 0:
        raise ValueError("block table refers to a block outside the pool")
    return rows[:seqlen]


def attend_paged(q, pool, block_table, seqlens, scale, causal, L):
    """Batched paged absorbed attention. q [B,Sq,N,E], pool [NB,PG,E],
    block_table [B,MB] int32, seqlens [B]. Returns (o_lat [B,Sq,N,L], lse [B,Sq,N])."""
    q = _f64(q)
    pool = _f64(pool)
    B, Sq, N, E = q.shape
    NB, PG, _ = pool.shape
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    o = np.zeros((B, Sq, N, L))
    lse = np.zeros((B, Sq, N))
    rc = _load().mla_oracle_attend_paged(
        B, Sq, N, L, E - L, _dp(q), _dp(pool), NB, PG, _i32p(bt), bt.shape[1], _i32p(sl),
        float(scale), int(bool(causal)), _dp(o), _dp(lse),
    )
    if rc != 0:
        raise ValueError("block table refers to a block outside the pool")
    return o, lse


def naive(q_nope, q_pe, c_kv, k_pe, w_uk_t, w_uv, pos, scale, causal):
    """Naive MLA: decompress K and V per head, then softmax attention.
    Returns out [nq,N,V]."""
    q_nope, c_kv, w_uk_t, w_uv = map(_f64, (q_nope, c_kv, w_uk_t, w_uv))
    nq, N, P = q_nope.shape
    T, L = c_kv.shape
    V = w_uv.shape[2]
    R = 0 if q_pe is None else np.asarray(q_pe).shape[2]
    q_pe = _f64(q_pe) if R else np.zeros((1,))
    k_pe = _f64(k_pe) if R else np.zeros((1,))
    cp = c_kv if T else np.zeros((1, L))
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    out = np.zeros((nq, N, V))
    _load().mla_oracle_naive(
        nq, N, P, R, V, L, T, _dp(q_nope), _dp(q_pe), _dp(cp), _dp(k_pe), _dp(w_uk_t), _dp(w_uv),
        _i64p(pos), float(scale), int(bool(causal)), _dp(out),
    )
    return out


def absorbed(q_nope, q_pe, c_kv, k_pe, w_uk_t, w_uv, pos, scale, causal):
    """Absorbed MLA end to end. Returns (out [nq,N,V], q_lat [nq,N,L],
    o_lat [nq,N,L], lse [nq,N])."""
    q_nope, c_kv, w_uk_t, w_uv = map(_f64, (q_nope, c_kv, w_uk_t, w_uv))
    nq, N, P = q_nope.shape
    T, L = c_kv.shape
    V = w_uv.shape[2]
    R = 0 if q_pe is None else np.asarray(q_pe).shape[2]
    q_pe = _f64(q_pe) if R else np.zeros((1,))
    k_pe = _f64(k_pe) if R else np.zeros((1,))
    cp = c_kv if T else np.zeros((1, L))
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    out = np.zeros((nq, N, V))
    q_lat = np.zeros((nq, N, L))
    o_lat = np.zeros((nq, N, L))
    lse = np.zeros((nq, N))
    _load().mla_oracle_absorbed(
        nq, N, P, R, V, L, T, _dp(q_nope), _dp(q_pe), _dp(cp), _dp(k_pe), _dp(w_uk_t), _dp(w_uv),
        _i64p(pos), float(scale), int(bool(causal)), _dp(out), _dp(q_lat), _dp(o_lat), _dp(lse),
    )
    return out, q_lat, o_lat, lse


def attend_split(q, kv, pos, scale, causal, L, bounds):
    """Split-KV attention merged by log-sum-exp; bounds [S+1] key boundaries.
    Returns (o_lat [nq,N,L], lse [nq,N])."""
    q = _f64(q)
    kv = _f64(kv)
    nq, N, E = q.shape
    T = kv.shape[0]
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    bnd = np.ascontiguousarray(np.asarray(bounds, dtype=np.int64))
    o = np.zeros((nq, N, L))
    lse = np.zeros((nq, N))
    _load().mla_oracle_attend_split(
        nq, N, L, E - L, T, _dp(q), _i64p(pos), _dp(kv if T else np.zeros((1, E))), float(scale),
        int(bool(causal)), _i64p(bnd), len(bnd) - 1, _dp(o), _dp(lse),
    )
    return o, lse


def cache_write(buf, kv_c, k_pe, slots, offset, num_blocks, page, s0, s1):
    """Expected image of a latent-cache write. ``buf`` is the whole allocation
    (any numpy dtype of 2 or 4 bytes; copied, not modified), kv_c [T,L] and
    k_pe [T,R] (same dtype, or k_pe None when R == 0), slots [T] int64.
    Returns the new buffer (same dtype and shape as ``buf``)."""
    out = np.array(buf, copy=True)
    flat = out.reshape(-1)
    kv_c = np.ascontiguousarray(kv_c)
    T, L = kv_c.shape
    esize = kv_c.dtype.itemsize
    if flat.dtype.itemsize != esize:
        raise ValueError("cache and rows must share an element size")
    if k_pe is None or np.asarray(k_pe).size == 0:
        R = 0
        k_pe = np.zeros((1,), dtype=kv_c.dtype)
        kps = 0
    else:
        k_pe = np.ascontiguousarray(k_pe)
        R = k_pe.shape[1]
        kps = R
    sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int64))
    u8 = ctypes.POINTER(ctypes.c_uint8)
    rc = _load().mla_oracle_cache_write(
        T, L, R, esize, kv_c.ctypes.data_as(u8), L, k_pe.ctypes.data_as(u8), kps, _i64p(sl),
        flat.ctypes.data_as(u8), flat.size, offset, num_blocks, page, s0, s1,
    )
    if rc != 0:
        raise ValueError("cache write would fall outside the buffer")
    return out


def rope_interleaved(x, positions, base):
    """Interleaved rotary embedding ([P2] gate 3): x [T, V, d] (or [T, d]) rotated
    pair by pair, (2i, 2i+1) by positions[t] * base^(-2i/d). Returns a new
    float64 array of x's shape; d == 0 returns x unchanged."""
    x = _f64(x)
    shape = x.shape
    T = shape[0]
    d = shape[-1]
    if d % 2:
        raise ValueError("rope width must be even")
    y = np.array(x.reshape(T, -1, d) if d else x, dtype=np.float64, copy=True, order="C")
    if d == 0 or T == 0:
        return y.reshape(shape)
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    if pos.shape != (T,):
        raise ValueError("one position per token")
    _load().mla_oracle_rope_interleaved(T, y.shape[1], d, _dp(y), _i32p(pos), float(base))
    return y.reshape(shape)


# ------------------------------------------------------------------ fp8 cache
# [P3] dense fp8 decode tests: a float8_e4m3fn latent cache, descale_q and
# descale_k; concat_and_cache_mla with a cache dtype and a scale. The format,
# and the readings of what the pages leave open, are stated in mla_oracle.c.


def _u8p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _fp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def e4m3_decode(codes):
    """Values (float64) of OCP e4m3fn codes (any integer array of bytes)."""
    c = np.ascontiguousarray(np.asarray(codes).astype(np.uint8))
    out = np.zeros(c.shape, dtype=np.float64)
    _load().mla_oracle_e4m3_decode_array(c.size, _u8p(c), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def e4m3_encode(values):
    """Nearest e4m3fn codes (uint8) of float32 values: ties to the even
    mantissa, magnitudes past 448 saturate, NaN stays NaN."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    out = np.zeros(v.shape, dtype=np.uint8)
    _load().mla_oracle_e4m3_encode_array(v.size, _fp(v), _u8p(out))
    return out


def cache_write_fp8(buf, kv_c, k_pe, slots, scale, offset, num_blocks, page, s0, s1):
    """Expected image of an fp8 latent-cache write: ``buf`` is the whole byte
    allocation (uint8, copied, not modified); kv_c [T,L] and k_pe [T,R] (or None)
    as float32 values; the row of token t lands at slot slots[t] of the view
    (offset, s0, s1 in bytes) as e4m3(x / scale) per element."""
    out = np.array(buf, dtype=np.uint8, copy=True)
    flat = out.reshape(-1)
    kv = np.ascontiguousarray(np.asarray(kv_c, dtype=np.float32))
    T, L = kv.shape
    if k_pe is None or np.asarray(k_pe).size == 0:
        R = 0
        kp = np.zeros((1,), dtype=np.float32)
    else:
        kp = np.ascontiguousarray(np.asarray(k_pe, dtype=np.float32))
        R = kp.shape[1]
    sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int64))
    rc = _load().mla_oracle_cache_write_fp8(
        T, L, R, _fp(kv if T else np.zeros((1,), np.float32)), _fp(kp), _i64p(sl), float(scale),
        _u8p(flat), flat.size, offset, num_blocks, page, s0, s1,
    )
    if rc != 0:
        raise ValueError("cache write would fall outside the buffer")
    return out


def attend_paged_fp8(q, pool_codes, block_table, seqlens, scale, causal, L, descale_q, descale_k):
    """Dense decode over an fp8 cache: the query is q * descale_q and the cache
    rows are e4m3 values times descale_k; then attend_paged."""
    q = _f64(q) * float(descale_q)
    pool = e4m3_decode(pool_codes) * float(descale_k)
    return attend_paged(q, pool, block_table, seqlens, scale, causal, L)


# ------------------------------------------------------- naive prefill
# [P2] naive oracle (K and V decompressed per head, then plain attention);
# [P1] ConcatMlaNopeRope broadcast case (one k_pe row shared by every head).


def decompress_kv(c_kv, k_pe, w_uk_t, w_uv):
    """Per-head keys [T,N,P+R] = [c_kv . W_UK_T[h]^T | k_pe] and values
    [T,N,V] = c_kv . W_UV[h]. k_pe [T,R] or None (R = 0)."""
    c_kv, w_uk_t, w_uv = map(_f64, (c_kv, w_uk_t, w_uv))
    T, L = c_kv.shape
    N, P, _ = w_uk_t.shape
    V = w_uv.shape[2]
    R = 0 if k_pe is None else np.asarray(k_pe).shape[1]
    kp = _f64(k_pe) if R and T else np.zeros((1,))
    cp = c_kv if T else np.zeros((1, L))
    k = np.zeros((max(T, 1), N, P + R))
    v = np.zeros((max(T, 1), N, V))
    _load().mla_oracle_decompress_kv(T, N, P, R, V, L, _dp(cp), _dp(kp), _dp(w_uk_t), _dp(w_uv),
                                     _dp(k), _dp(v))
    return k[:T], v[:T]


def mha(q, k, v, pos, scale, causal):
    """Multi-head softmax attention of one sequence: q [nq,N,DK], k [T,N,DK],
    v [T,N,DV], pos [nq] absolute query positions. Returns (out [nq,N,DV],
    lse [nq,N] natural log)."""
    q, k, v = map(_f64, (q, k, v))
    nq, N, DK = q.shape
    T = k.shape[0]
    DV = v.shape[2]
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    kp = k if T else np.zeros((1, N, DK))
    vp = v if T else np.zeros((1, N, DV))
    out = np.zeros((nq, N, DV))
    lse = np.zeros((nq, N))
    _load().mla_oracle_mha(nq, T, N, DK, DV, _dp(q), _dp(kp), _dp(vp), _i64p(pos), float(scale),
                           int(bool(causal)), _dp(out), _dp(lse))
    return out, lse


def mha_varlen(q, k, v, cu_q, cu_k, scale, causal):
    """mha over packed sequences: sequence b owns query rows cu_q[b]:cu_q[b+1]
    and key rows cu_k[b]:cu_k[b+1]; its queries are the suffix of its keys."""
    q, k, v = map(_f64, (q, k, v))
    out = np.zeros(q.shape[:2] + (v.shape[2],))
    lse = np.zeros(q.shape[:2])
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        pos = np.arange(q1 - q0) + (k1 - k0) - (q1 - q0)
        out[q0:q1], lse[q0:q1] = mha(q[q0:q1], k[k0:k1], v[k0:k1], pos, scale, causal)
    return out, lse


# ------------------------------------------------------ sparse fp8 decode
# [P3] test_flashmla_fp8_sparse_decode_unified_slot_view: 656-byte entries
# (512 e4m3 codes, 4 f32 scales, 64 bf16 rope values) reached through per-token
# lists of top-k slot indices, -1 for none. Format and reading in mla_oracle.c.
DSMLA_ENTRY = 656


def dsmla_rows(entries):
    """[..., 656] uint8 entries -> [..., 576] float64 latent rows [c_kv | k_pe]."""
    e = np.ascontiguousarray(np.asarray(entries, dtype=np.uint8))
    lead = e.shape[:-1]
    flat = e.reshape(-1, DSMLA_ENTRY)
    rows = np.zeros((max(flat.shape[0], 1), 576))
    _load().mla_oracle_dsmla_rows(flat.shape[0], _u8p(flat if flat.size else np.zeros(
        (1, DSMLA_ENTRY), np.uint8)), DSMLA_ENTRY, _dp(rows))
    return rows[:flat.shape[0]].reshape(lead + (576,))


def sparse_decode(q, pool_entries, indices, scale, L=512):
    """Sparse absorbed decode: query token (b, i) of q [B,Sq,N,576] attends over
    the latent rows at the slots indices[b,i,:] (slot = block * page + offset
    into pool_entries [NB,PG,656]); slots < 0 or past the pool are no key; a
    slot listed twice is two keys. Returns (o_lat [B,Sq,N,L], lse [B,Sq,N])."""
    q = _f64(q)
    B, Sq, N, E = q.shape
    pool = dsmla_rows(pool_entries)
    NB, PG = pool.shape[:2]
    flat = pool.reshape(NB * PG, E)
    idx = np.asarray(indices, dtype=np.int64)
    o = np.zeros((B, Sq, N, L))
    lse = np.full((B, Sq, N), -np.inf)
    for b in range(B):
        for i in range(Sq):
            sl = idx[b, i]
            sl = sl[(sl >= 0) & (sl < NB * PG)]
            if sl.size == 0:
                continue
            o[b, i], lse[b, i], _ = attend_seq(q[b, i][None], flat[sl], [0], scale, False, L)
    return o, lse
