"""C-ABI boundary checks that need no GPU.

The library must load, export every entry point include/mla.h declares, and
reject malformed arguments with the documented status before it touches any
memory or launches anything (vllm.cpp "tests/vt/test_ops_mla_absorb.cpp":
the batched matmul rejects inner-dim, batch and inner-stride mismatches). The
descriptors below carry fake device addresses: on the error paths nothing may
dereference them.
"""
import ctypes

import pytest
import torch

import mla_absorbed_decode_amd as mla
from mla_absorbed_decode_amd import MlaTensor

OK, NULL, DTYPE, SHAPE, STRIDE, UNSUP, WS = 0, -1, -2, -3, -4, -5, -6
BF16, F32, I32, I64, FP8 = 1, 2, 3, 4, 5
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced on error paths


def T(shape, dtype=BF16, strides=None, data=FAKE):
    d = MlaTensor()
    d.data = data
    d.dtype = dtype
    d.rank = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        d.shape[i] = s
        d.stride[i] = st
    return d


def R(d):
    return ctypes.byref(d) if d is not None else None


@pytest.fixture(scope="module")
def lib():
    return mla.load()


def test_library_exports_every_declared_symbol(lib):
    names = mla.header_symbols()
    assert set(names) == {"mla_absorb_q", "mla_concat_and_cache", "mla_decode_workspace_size",
                          "mla_decode_attend", "mla_v_up", "mla_status_str",
                          "mla_rope_interleaved", "mla_absorb_q_rope", "mla_concat_and_cache_rope",
                          "mla_absorb_q_and_cache", "mla_decode_attend_v_up",
                          "mla_concat_and_cache_fp8", "mla_decode_attend_fp8",
                          "mla_decompress_kv", "mla_prefill_attend", "mla_sparse_decode_fp8",
                          "mla_sparse_workspace_size", "mla_decode_attend_noalloc",
                          "mla_decode_plan_size", "mla_decode_plan", "mla_decode_attend_planned",
                          "mla_decode_attend_v_up_planned"}
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_every_declared_symbol():
    # libmla_probe.so (the benchmark's measured peaks) against include/mla_probe.h
    import os
    import re

    from mla_absorbed_decode_amd import probe

    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "include", "mla_probe.h")
    names = re.findall(r"^int\s+(mla_probe_\w+)\s*\(", open(hdr).read(), flags=re.M)
    assert set(names) == {"mla_probe_mfma_bf16", "mla_probe_copy", "mla_probe_read",
                          "mla_probe_tile_stream"}
    plib = probe.load()
    for n in names:
        assert hasattr(plib, n), n
    # argument checks run before any HIP call
    assert plib.mla_probe_tile_stream(None, None, None, 17, 256, None) == -1
    assert plib.mla_probe_tile_stream(FAKE, FAKE, FAKE, 0, 256, None) == -5
    assert plib.mla_probe_tile_stream(FAKE, FAKE + 8, FAKE, 17, 256, None) == -5
    assert plib.mla_probe_tile_stream(FAKE, FAKE, FAKE, 17, 0, None) == -5


def test_status_strings(lib):
    for code, name in mla.STATUS.items():
        assert mla.mla_status_str(code).startswith(name)
    assert "unknown" in mla.mla_status_str(12345)


# ---------------------------------------------------------------- absorb_q


def absorb(lib, q_nope, w, q_pe, out):
    return lib.mla_absorb_q(R(q_nope), R(w), R(q_pe), R(out), None)


def test_absorb_q_validation(lib):
    good = dict(q_nope=T([4, 16, 128]), w=T([16, 128, 512]), q_pe=T([4, 16, 64]),
                out=T([4, 16, 576]))
    assert absorb(lib, None, good["w"], good["q_pe"], good["out"]) == NULL
    assert absorb(lib, T([4, 16, 128], data=0), good["w"], good["q_pe"], good["out"]) == NULL
    # inner-dim mismatch and head (batch) mismatch
    assert absorb(lib, good["q_nope"], T([16, 100, 512]), good["q_pe"], good["out"]) == SHAPE
    assert absorb(lib, good["q_nope"], T([8, 128, 512]), good["q_pe"], good["out"]) == SHAPE
    # output width must be L + R; q_pe heads must be N or 1
    assert absorb(lib, good["q_nope"], good["w"], good["q_pe"], T([4, 16, 512])) == SHAPE
    assert absorb(lib, good["q_nope"], good["w"], T([4, 3, 64]), good["out"]) == SHAPE
    # rank
    assert absorb(lib, T([4, 16, 128, 1]), good["w"], good["q_pe"], good["out"]) == SHAPE
    # innermost stride must be 1; strides must be non-negative
    assert absorb(lib, T([4, 16, 128], strides=[4096, 256, 2]), good["w"], good["q_pe"],
                  good["out"]) == STRIDE
    assert absorb(lib, T([4, 16, 128], strides=[-2048, 128, 1]), good["w"], good["q_pe"],
                  good["out"]) == STRIDE
    # dtypes
    assert absorb(lib, T([4, 16, 128], F32), good["w"], good["q_pe"], good["out"]) == DTYPE
    assert absorb(lib, T([4, 16, 128], I32), T([16, 128, 512], I32), None,
                  T([4, 16, 512], I32)) == DTYPE


def test_absorb_q_empty_batch_is_a_no_op(lib):
    # T == 0 launches nothing, so it is safe without a device
    assert absorb(lib, T([0, 16, 128]), T([16, 128, 512]), T([0, 16, 64]),
                  T([0, 16, 576])) == OK


def test_v_up_validation(lib):
    f = lambda o, w, out: lib.mla_v_up(R(o), R(w), R(out), None)
    assert f(T([4, 16, 512]), T([16, 512, 128]), T([4, 16, 64])) == SHAPE
    assert f(T([4, 16, 512]), T([16, 256, 128]), T([4, 16, 128])) == SHAPE
    assert f(T([4, 16, 512]), T([16, 512, 128], F32), T([4, 16, 128])) == DTYPE
    assert f(T([4, 16, 512], strides=[8192, 512, 3]), T([16, 512, 128]), T([4, 16, 128])) == STRIDE
    assert f(T([0, 16, 512]), T([16, 512, 128]), T([0, 16, 128])) == OK


# ------------------------------------------------------------ cache write


def test_concat_and_cache_validation(lib):
    f = lambda kv, pe, sl, c: lib.mla_concat_and_cache(R(kv), R(pe), R(sl), R(c), None)
    kv, pe, sl, cache = T([200, 512]), T([200, 64]), T([200], I64), T([32, 64, 576])
    assert f(kv, pe, sl, T([32, 64, 512])) == SHAPE   # entry must be L + R
    assert f(kv, pe, T([199], I64), cache) == SHAPE
    assert f(kv, T([100, 64]), sl, cache) == SHAPE
    assert f(kv, pe, T([200], F32), cache) == DTYPE   # slot mapping must be integer
    assert f(kv, pe, sl, T([32, 64, 576], F32)) == DTYPE
    assert f(None, pe, sl, cache) == NULL
    assert f(kv, pe, sl, T([32, 64, 576], strides=[110592, 576, 2])) == STRIDE
    assert f(T([0, 512]), T([0, 64]), T([0], I64), cache) == OK


# ------------------------------------------------------------- rotary embedding


def test_rope_validation(lib):
    f = lambda x, pos, base: lib.mla_rope_interleaved(R(x), R(pos), ctypes.c_double(base), None)
    x, pos = T([7, 5, 64], F32), T([7], I32)
    assert f(x, pos, 0.0) == UNSUP                     # base must be > 0 and finite
    assert f(x, pos, float("inf")) == UNSUP
    assert f(x, pos, float("nan")) == UNSUP
    assert f(T([7, 5, 63], F32), pos, 8e6) == SHAPE    # odd width
    assert f(x, T([6], I32), 8e6) == SHAPE             # one position per token
    assert f(x, T([7], I64), 8e6) == DTYPE             # positions are int32
    assert f(T([7, 5, 64], I32), pos, 8e6) == DTYPE
    assert f(x, None, 8e6) == NULL
    assert f(T([7, 64], F32), pos, 8e6) == SHAPE       # rank 3
    assert f(T([7, 5, 64], F32, strides=[640, 128, 2]), pos, 8e6) == STRIDE
    # width 0 (NoPE), no tokens or no vectors: nothing is launched
    assert f(T([7, 5, 0], F32), pos, 8e6) == OK
    assert f(T([0, 5, 64], F32), T([0], I32), 8e6) == OK
    assert f(T([7, 0, 64], F32), pos, 8e6) == OK


def test_fused_rope_validation(lib):
    dbl = ctypes.c_double
    q = lambda qn, w, pe, pos, out, base=8e6: lib.mla_absorb_q_rope(R(qn), R(w), R(pe), R(pos),
                                                                     dbl(base), R(out), None)
    qn, w, pe, out = T([4, 16, 128]), T([16, 128, 512]), T([4, 16, 64]), T([4, 16, 576])
    assert q(qn, w, pe, None, out) == NULL
    assert q(qn, w, pe, T([5], I32), out) == SHAPE
    assert q(qn, w, pe, T([4], I64), out) == DTYPE
    assert q(qn, w, pe, T([4], I32), out, base=-1.0) == UNSUP
    assert q(qn, w, T([4, 16, 63]), T([4], I32), T([4, 16, 575])) == SHAPE  # odd rope width
    assert q(T([0, 16, 128]), w, T([0, 16, 64]), T([0], I32), T([0, 16, 576])) == OK
    c = lambda kv, pe, sl, pos, cache, base=8e6: lib.mla_concat_and_cache_rope(
        R(kv), R(pe), R(sl), R(pos), dbl(base), R(cache), None)
    kv, pe, sl, cache = T([200, 512]), T([200, 64]), T([200], I64), T([32, 64, 576])
    assert c(kv, pe, sl, None, cache) == NULL
    assert c(kv, pe, sl, T([199], I32), cache) == SHAPE
    assert c(kv, pe, sl, T([200], I64), cache) == DTYPE
    assert c(kv, pe, sl, T([200], I32), cache, base=float("inf")) == UNSUP
    assert c(T([0, 512]), T([0, 64]), T([0], I64), T([0], I32), cache) == OK


def test_fused_fold_and_cache_validation(lib):
    dbl = ctypes.c_double
    f = lambda qn, w, pe, out, kv, kpe, sl, cache, pos=None, base=0.0: lib.mla_absorb_q_and_cache(
        R(qn), R(w), R(pe), R(out), R(kv), R(kpe), R(sl), R(cache), R(pos), dbl(base), None)
    qn, w, pe, out = T([64, 16, 128]), T([16, 128, 512]), T([64, 16, 64]), T([64, 16, 576])
    kv, kpe, sl, cache = T([64, 512]), T([64, 64]), T([64], I64), T([32, 64, 576])
    assert f(qn, w, pe, out, T([63, 512]), T([63, 64]), T([63], I64), cache) == SHAPE  # one row per token
    assert f(qn, w, pe, out, kv, kpe, sl, T([32, 64, 512])) == SHAPE   # fold ok, cache entry wrong
    assert f(qn, T([16, 100, 512]), pe, out, kv, kpe, sl, cache) == SHAPE
    assert f(qn, w, pe, out, kv, kpe, T([64], F32), cache) == DTYPE
    assert f(qn, w, pe, out, kv, kpe, sl, cache, T([64], I32), -1.0) == UNSUP
    assert f(qn, w, pe, out, None, kpe, sl, cache) == NULL
    assert f(T([0, 16, 128]), w, T([0, 16, 64]), T([0, 16, 576]), T([0, 512]), T([0, 64]),
             T([0], I64), cache) == OK


# ------------------------------------------------------------------ decode


def ws_size(lib, B, Sq, N, L, S, PG, dt=BF16):
    n = ctypes.c_size_t(0)
    rc = lib.mla_decode_workspace_size(B, Sq, N, L, S, PG, dt, ctypes.byref(n))
    return rc, n.value


def test_workspace_size(lib):
    rc, n = ws_size(lib, 64, 1, 16, 512, 4096, 64)
    assert rc == OK and n > 0          # few units: split KV, partials needed
    rc, n2 = ws_size(lib, 64, 1, 16, 512, 4096, 64)
    assert n2 == n                     # depends on the arguments only
    rc, n = ws_size(lib, 1, 2048, 64, 512, 2048, 64)
    assert rc == OK and n == 0         # many prefill units: one workgroup each, no partials
    assert ws_size(lib, 4, 1, 128, 256, 4096, 64)[0] == UNSUP
    assert ws_size(lib, 4, 1, 128, 512, 4096, 8)[0] == UNSUP
    assert ws_size(lib, 4, 1, 128, 512, 4096, 64, I32)[0] == DTYPE
    assert lib.mla_decode_workspace_size(4, 1, 128, 512, 4096, 64, BF16, None) == NULL
    assert ws_size(lib, 0, 1, 16, 512, 4096, 64) == (OK, 0)


def decode(lib, q, kv, bt, sl, out, lse=None, max_seqlen=128, ws=None, ws_bytes=0, causal=1):
    return lib.mla_decode_attend(R(q), R(kv), R(bt), R(sl), max_seqlen, ctypes.c_float(0.04),
                                 causal, R(out), R(lse), ws, ws_bytes, None)


def test_decode_validation(lib):
    B, N = 2, 16
    q, kv, bt, sl = T([B, 1, N, 576]), T([8, 64, 576]), T([B, 4], I32), T([B], I32)
    out, lse = T([B, 1, N, 512]), T([B, 1, N], F32)
    rc, need = ws_size(lib, B, 1, N, 512, 128, 64)
    assert rc == OK and need > 0
    # missing or short workspace
    assert decode(lib, q, kv, bt, sl, out, lse) == WS
    assert decode(lib, q, kv, bt, sl, out, lse, ws=FAKE, ws_bytes=need - 1) == WS
    assert decode(lib, q, kv, bt, sl, out, lse, ws=FAKE + 4, ws_bytes=need) == WS
    # unsupported geometry
    assert decode(lib, T([B, 1, N, 288]), T([8, 64, 288]), bt, sl, T([B, 1, N, 256])) == UNSUP
    assert decode(lib, T([B, 1, N, 544]), T([8, 64, 544]), bt, sl, out) == UNSUP   # rope 32
    assert decode(lib, q, T([8, 8, 576]), bt, sl, out) == UNSUP                    # page 8
    assert decode(lib, T([B, 1, N, 576], data=FAKE + 2), kv, bt, sl, out) == UNSUP  # misaligned
    assert decode(lib, q, T([8, 64, 576], strides=[36868, 576, 1]), bt, sl, out) == UNSUP
    # shapes and dtypes
    assert decode(lib, q, T([8, 64, 512]), bt, sl, out) == SHAPE
    assert decode(lib, q, kv, T([3, 4], I32), sl, out) == SHAPE
    assert decode(lib, q, kv, bt, T([3], I32), out) == SHAPE
    assert decode(lib, q, kv, bt, sl, out, T([B, 1, 8], F32)) == SHAPE
    assert decode(lib, q, kv, T([B, 4], I64), sl, out) == DTYPE
    assert decode(lib, q, kv, bt, sl, out, T([B, 1, N], BF16)) == DTYPE
    assert decode(lib, q, T([8, 64, 576], F32), bt, sl, out) == DTYPE
    assert decode(lib, q, kv, bt, sl, out, max_seqlen=-1) == SHAPE
    assert decode(lib, None, kv, bt, sl, out) == NULL
    # empty batch: nothing to do
    assert decode(lib, T([0, 1, N, 576]), kv, T([0, 4], I32), T([0], I32), T([0, 1, N, 512])) == OK


def test_decode_v_up_validation(lib):
    B, N = 2, 16
    q, kv, bt, sl = T([B, 1, N, 576]), T([8, 64, 576]), T([B, 4], I32), T([B], I32)
    o_lat, lse, w, out = T([B, 1, N, 512]), T([B, 1, N], F32), T([N, 512, 128]), T([B, 1, N, 128])
    rc, need = ws_size(lib, B, 1, N, 512, 128, 64)
    f = lambda w_, o_, out_, ws=FAKE, ws_bytes=need, q_=q: lib.mla_decode_attend_v_up(
        R(q_), R(kv), R(bt), R(sl), 128, ctypes.c_float(0.04), 1, R(w_), R(o_), R(out_), R(lse),
        ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)
    assert f(w, o_lat, out, ws=0) == WS                       # the attention's own checks first
    assert f(T([N, 256, 128]), o_lat, out) == SHAPE           # w_uv rows must be L
    assert f(T([8, 512, 128]), o_lat, out) == SHAPE           # one w_uv per head
    assert f(w, o_lat, T([B, 1, N, 64])) == SHAPE             # out width is V
    assert f(T([N, 512, 128], F32), o_lat, out) == DTYPE
    assert f(w, o_lat, None) == NULL
    assert f(w, None, out) == NULL                            # o_lat is required
    # two queries per sequence, o_lat without one token stride, fused kernel not
    # available (f32): refused before launching
    q2, o2 = T([B, 2, N, 576], F32), T([B, 2, N, 512], F32, strides=[4 * N * 512, N * 512, 512, 1])
    assert lib.mla_decode_attend_v_up(R(q2), R(T([8, 64, 576], F32)), R(bt), R(sl), 128,
                                      ctypes.c_float(0.04), 1, R(T([N, 512, 128], F32)), R(o2),
                                      R(T([B, 2, N, 128], F32)), None, ctypes.c_void_p(FAKE),
                                      ctypes.c_size_t(1 << 30), None) == UNSUP


def test_decode_plan_validation(lib):
    B, N = 2, 16
    q, kv, bt, sl = T([B, 1, N, 576]), T([8, 64, 576]), T([B, 4], I32), T([B], I32)
    out, lse = T([B, 1, N, 512]), T([B, 1, N], F32)
    n = ctypes.c_size_t(0)
    assert lib.mla_decode_plan_size(B, 1, N, 512, 128, 64, BF16, ctypes.byref(n)) == OK
    need = n.value
    assert need > 0                                            # few units: a split plan
    assert lib.mla_decode_plan_size(1, 2048, 64, 512, 2048, 64, BF16, ctypes.byref(n)) == OK
    assert n.value == 0                                        # no split, nothing to plan
    assert lib.mla_decode_plan_size(B, 1, N, 256, 128, 64, BF16, ctypes.byref(n)) == UNSUP
    assert lib.mla_decode_plan_size(B, 1, N, 512, 128, 64, I32, ctypes.byref(n)) == DTYPE
    assert lib.mla_decode_plan_size(B, 1, N, 512, 128, 64, BF16, None) == NULL
    plan = lambda q_=q, p=FAKE, nb=need: lib.mla_decode_plan(
        R(q_), R(kv), R(bt), R(sl), 128, 1, ctypes.c_void_p(p), ctypes.c_size_t(nb), None)
    assert plan(p=0) == WS                                     # a split call needs the buffer
    assert plan(nb=need - 1) == WS
    assert plan(p=FAKE + 4) == WS
    assert plan(q_=T([B, 1, N, 544])) == SHAPE                 # q and cache widths differ
    assert plan(q_=None) == NULL
    # an fp8 cache plans in its own call (mla_decode_attend_fp8 takes no plan)
    assert lib.mla_decode_plan(R(q), R(T([8, 64, 576], FP8)), R(bt), R(sl), 128, 1,
                               ctypes.c_void_p(FAKE), ctypes.c_size_t(need), None) == DTYPE
    rc, wneed = ws_size(lib, B, 1, N, 512, 128, 64)
    att = lambda p, nb: lib.mla_decode_attend_planned(
        R(q), R(kv), R(bt), R(sl), 128, ctypes.c_float(0.04), 1, R(out), R(lse),
        ctypes.c_void_p(FAKE), ctypes.c_size_t(wneed), ctypes.c_void_p(p), ctypes.c_size_t(nb),
        None)
    assert att(FAKE, need - 1) == WS                           # short plan
    assert att(FAKE + 8, need) == WS                           # misaligned plan
    assert lib.mla_decode_attend_planned(R(q), R(kv), R(bt), R(sl), 128, ctypes.c_float(0.04), 1,
                                         R(out), R(lse), None, 0, ctypes.c_void_p(FAKE),
                                         ctypes.c_size_t(need), None) == WS   # workspace still due
    w, o_lat, out2 = T([N, 512, 128]), T([B, 1, N, 512]), T([B, 1, N, 128])
    assert lib.mla_decode_attend_v_up_planned(
        R(q), R(kv), R(bt), R(sl), 128, ctypes.c_float(0.04), 1, R(w), R(o_lat), R(out2), R(lse),
        ctypes.c_void_p(FAKE), ctypes.c_size_t(wneed), ctypes.c_void_p(FAKE),
        ctypes.c_size_t(need - 1), None) == WS


# ------------------------------------------------------------------- fp8


def test_fp8_cache_write_validation(lib):
    T_, L, R_ = 5, 512, 64
    kv, kpe, sl = T([T_, L]), T([T_, R_]), T([T_], I64)
    cache = T([8, 64, L + R_], FP8)
    f = lambda kv_=kv, kpe_=kpe, c=cache, scale=FAKE: lib.mla_concat_and_cache_fp8(
        R(kv_), R(kpe_), R(sl), R(c), ctypes.c_void_p(scale), None)
    assert f(scale=0) == NULL                      # the scale pointer is required
    assert f(c=T([8, 64, L + R_])) == DTYPE        # the cache must be fp8
    assert f(kv_=T([T_, L], FP8)) == DTYPE         # the rows are bf16 or f32
    assert f(kpe_=T([T_, R_], F32)) == DTYPE       # one dtype for both row parts
    assert f(c=T([8, 64, 512], FP8)) == SHAPE      # entry = L + R
    # the copy-of-bits write takes no fp8 cache
    assert lib.mla_concat_and_cache(R(kv), R(kpe), R(sl), R(cache), None) == DTYPE
    # nothing to write: no launch
    assert lib.mla_concat_and_cache_fp8(R(T([0, L])), R(T([0, R_])), R(T([0], I64)), R(cache),
                                        ctypes.c_void_p(FAKE), None) == OK


def test_fp8_decode_validation(lib):
    B, N = 2, 16
    q, kv, bt, sl = T([B, 1, N, 576]), T([8, 64, 576], FP8), T([B, 4], I32), T([B], I32)
    out, lse = T([B, 1, N, 512]), T([B, 1, N], F32)
    rc, need = ws_size(lib, B, 1, N, 512, 128, 64)
    assert rc == OK
    need8 = ctypes.c_size_t(0)
    assert lib.mla_decode_workspace_size(B, 1, N, 512, 128, 64, FP8, ctypes.byref(need8)) == OK
    f = lambda q_=q, kv_=kv, out_=out, dq=FAKE, dk=FAKE, ws=FAKE: lib.mla_decode_attend_fp8(
        R(q_), R(kv_), R(bt), R(sl), 128, ctypes.c_float(0.04), 1, ctypes.c_void_p(dq),
        ctypes.c_void_p(dk), R(out_), R(lse), ctypes.c_void_p(ws), ctypes.c_size_t(need8.value),
        None)
    assert f(dq=0) == NULL and f(dk=0) == NULL
    assert f(kv_=T([8, 64, 576])) == DTYPE                      # the cache must be fp8
    assert f(q_=T([B, 1, N, 576], F32), out_=T([B, 1, N, 512], F32)) == DTYPE  # bf16 queries
    assert f(kv_=T([8, 64, 576], FP8, strides=[64 * 580, 580, 1])) == UNSUP  # 8-byte rows
    assert f(kv_=T([8, 64, 512], FP8)) == SHAPE
    assert f(ws=0) == WS
    # the bf16 entry point takes no fp8 cache
    assert decode(lib, q, kv, bt, sl, out) == DTYPE
    assert f(kv_=T([8, 64, 584], FP8), q_=T([B, 1, N, 584])) == UNSUP  # R = 72: not 0 or 64


# ----------------------------------------------------------- python layer


def test_binding_refuses_host_tensors():
    a = torch.zeros(4, 16, 128, dtype=torch.bfloat16)
    w = torch.zeros(16, 128, 512, dtype=torch.bfloat16)
    out = torch.zeros(4, 16, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mla.mla_absorb_q(a, w, None, out)


def test_binding_descriptor_matches_view():
    big = torch.zeros(32, 3 * 64 * 576, dtype=torch.bfloat16)
    view = torch.as_strided(big, (32, 64, 576), (3 * 64 * 576, 576, 1), 64 * 576)
    d = mla.desc(view)
    assert d.rank == 3 and list(d.shape[:3]) == [32, 64, 576]
    assert list(d.stride[:3]) == [110592, 576, 1]
    assert d.data == big.data_ptr() + 64 * 576 * 2  # storage offset folded into the pointer


# ------------------------------------------------------------ naive prefill


def test_decompress_kv_validation(lib):
    f = lambda c, pe, wk, wv, k, v: lib.mla_decompress_kv(R(c), R(pe), R(wk), R(wv), R(k), R(v),
                                                          None)
    S, N, P, Rr, V, L = 8, 16, 128, 64, 128, 512
    c, pe = T([S, L]), T([S, Rr])
    wk, wv = T([N, P, L]), T([N, L, V])
    k, v = T([S, N, P + Rr]), T([S, N, V])
    assert f(c, pe, wk, wv, T([S, N, P]), v) == SHAPE            # no room for the rope row
    assert f(T([0, L]), None, wk, wv, T([0, N, P]), T([0, N, V])) == OK  # NoPE, no rows
    assert f(c, pe, T([N, P, 256]), wv, k, v) == SHAPE           # latent width mismatch
    assert f(c, pe, wk, T([N, L, 64]), k, v) == SHAPE            # v width mismatch
    assert f(c, T([S + 1, Rr]), wk, wv, k, v) == SHAPE
    assert f(c, pe, wk, T([N, L, V], F32), k, v) == DTYPE
    assert f(c, pe, wk, wv, k, T([S, N, V], strides=[N * V * 2, V * 2, 2])) == STRIDE
    assert f(None, pe, wk, wv, k, v) == NULL
    assert f(T([0, L]), T([0, Rr]), wk, wv, T([0, N, P + Rr]), T([0, N, V])) == OK


def test_prefill_attend_validation(lib):
    def f(q, k, v, cq, ck, out, lse=None, max_q=64, scale=0.1, causal=1):
        return lib.mla_prefill_attend(R(q), R(k), R(v), R(cq), R(ck), max_q, scale, causal, R(out),
                                      R(lse), None)
    Tq, S, N = 64, 96, 16
    q, k, v = T([Tq, N, 192]), T([S, N, 192]), T([S, N, 128])
    cq, ck = T([3], I32), T([3], I32)
    out, lse = T([Tq, N, 128]), T([Tq, N], F32)
    assert f(q, k, v, cq, T([4], I32), out, lse) == SHAPE        # batch mismatch
    assert f(q, T([S, N, 128]), v, cq, ck, out) == SHAPE          # key width != query width
    assert f(q, k, T([S + 1, N, 128]), cq, ck, out) == SHAPE
    assert f(q, k, v, cq, ck, T([Tq, N, 64])) == SHAPE
    assert f(q, k, v, cq, ck, out, T([Tq, 8], F32)) == SHAPE
    assert f(q, k, v, cq, ck, out, max_q=-1) == SHAPE
    assert f(q, k, v, T([3], I64), ck, out) == DTYPE
    assert f(q, k, v, cq, ck, out, T([Tq, N], BF16)) == DTYPE
    assert f(q, k, T([S, N, 128], F32), cq, ck, out) == DTYPE
    # f32 and unsupported widths are refused, as are misaligned rows
    assert f(T([Tq, N, 192], F32), T([S, N, 192], F32), T([S, N, 128], F32), cq, ck,
             T([Tq, N, 128], F32)) == UNSUP
    assert f(T([Tq, N, 96]), T([S, N, 96]), v, cq, ck, out) == UNSUP
    assert f(T([Tq, N, 192], data=FAKE + 2), k, v, cq, ck, out) == UNSUP
    assert f(q, k, v, cq, ck, T([Tq, N, 128], data=FAKE + 4)) == UNSUP
    assert f(None, k, v, cq, ck, out) == NULL
    # nothing to do
    assert f(q, k, v, T([1], I32), T([1], I32), out) == OK        # no sequence
    assert f(q, k, v, cq, ck, out, max_q=0) == OK


# ------------------------------------------------------------ sparse fp8 decode


def test_sparse_decode_validation(lib):
    def f(q, kv, idx, out, lse=None, ws=FAKE, ws_bytes=1 << 40):
        return lib.mla_sparse_decode_fp8(R(q), R(kv), R(idx), 0.04, R(out), R(lse), ws, ws_bytes,
                                         None)
    B, Sq, N = 2, 1, 128
    q, kv, idx = T([B, Sq, N, 576]), T([32, 64, 656], FP8), T([B, Sq, 128], I32)
    out, lse = T([B, Sq, N, 512]), T([B, Sq, N], F32)
    assert f(q, kv, idx, out, T([B, Sq, 64], F32)) == SHAPE
    assert f(q, kv, T([B, 2, 128], I32), out) == SHAPE
    assert f(q, kv, idx, T([B, Sq, N - 1, 512])) == SHAPE
    assert f(q, T([32, 64, 656], BF16), idx, out) == DTYPE
    assert f(q, kv, T([B, Sq, 128], I64), out) == DTYPE
    assert f(T([B, Sq, N, 576], F32), kv, idx, T([B, Sq, N, 512], F32)) == DTYPE
    assert f(q, T([32, 64, 576], FP8), idx, out) == UNSUP               # not a 656-byte entry
    assert f(T([B, Sq, N, 512]), kv, idx, out) == UNSUP                  # no rope part
    assert f(q, kv, T([B, Sq, 8192], I32), out) == UNSUP                 # top-k past the LDS list
    assert f(q, T([32, 64, 656], FP8, strides=[64 * 656 + 8, 656, 1]), idx, out) == UNSUP
    assert f(None, kv, idx, out) == NULL
    assert f(T([0, Sq, N, 576]), kv, T([0, Sq, 128], I32), T([0, Sq, N, 512])) == OK
    # a split call needs its workspace; a call small enough to run unsplit does not
    need = ctypes.c_size_t(0)
    assert lib.mla_sparse_workspace_size(B * Sq, N, 2048, ctypes.byref(need)) == OK
    assert need.value > 0
    big = T([B, Sq, 2048], I32)
    assert f(q, kv, big, out, ws=None, ws_bytes=0) == WS
    assert f(q, kv, big, out, ws=FAKE, ws_bytes=need.value - 1) == WS
    assert f(q, kv, big, out, ws=FAKE + 4, ws_bytes=need.value) == WS
    assert lib.mla_sparse_workspace_size(1, 128, 32, ctypes.byref(need)) == OK and need.value == 0
    assert lib.mla_sparse_workspace_size(1, 128, 8192, ctypes.byref(need)) == UNSUP
    assert lib.mla_sparse_workspace_size(-1, 128, 32, ctypes.byref(need)) == SHAPE
