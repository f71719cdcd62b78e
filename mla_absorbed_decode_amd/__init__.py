"""Python binding of libmla: MLA in weight-absorbed form on MI355X (gfx950).

Argument marshalling only. Each function turns torch tensors into the C ABI's
``mla_tensor`` descriptors (data pointer, dtype, sizes and element strides),
passes the current HIP stream, and raises ``MlaError`` on a non-zero status.
Every step of the computation runs in the HIP kernels of ``libmla.so``; there
is no fallback of any kind, so a missing or unbuilt library raises at the first
call.

The compute calls mirror include/mla.h:

* ``mla_absorb_q(q_nope, w_uk_t, q_pe, q_out)``
* ``mla_concat_and_cache(kv_c, k_pe, slot_mapping, kv_cache)``
* ``mla_decode_attend(q, kv_cache, block_table, seqlens, max_seqlen,
  softmax_scale, causal, out, lse=None, workspace=None)``
* ``mla_v_up(o_lat, w_uv, out)``

and the interleaved rotary embedding, alone or fused into the fold and the
cache write:

* ``mla_rope_interleaved(x, positions, base)``
* ``mla_absorb_q_rope(q_nope, w_uk_t, q_pe, positions, base, q_out)``
* ``mla_concat_and_cache_rope(kv_c, k_pe, slot_mapping, positions, base, kv_cache)``

and the decode step's fold and cache write as one launch:

* ``mla_absorb_q_and_cache(q_nope, w_uk_t, q_pe, q_out, kv_c, k_pe, slot_mapping,
  kv_cache, positions=None, base=0.0)``
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "MlaError",
    "mla_absorb_q",
    "mla_concat_and_cache",
    "mla_decode_workspace_size",
    "mla_decode_attend",
    "mla_v_up",
    "mla_rope_interleaved",
    "mla_absorb_q_rope",
    "mla_concat_and_cache_rope",
    "mla_absorb_q_and_cache",
    "mla_decode_attend_v_up",
    "mla_decode_attend_noalloc",
    "mla_decode_plan_size",
    "mla_decode_plan",
    "mla_decode_attend_planned",
    "mla_decode_attend_v_up_planned",
    "mla_status_str",
    "lib_path",
    "load",
    "STATUS",
]

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")
_HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                       "mla.h")

MLA_BF16, MLA_F32, MLA_I32, MLA_I64, MLA_FP8_E4M3 = 1, 2, 3, 4, 5
# an fp8 cache is torch.float8_e4m3fn (as the pages hold it) or its uint8 bytes
_DTYPES = {torch.bfloat16: MLA_BF16, torch.float32: MLA_F32, torch.int32: MLA_I32,
           torch.int64: MLA_I64, torch.float8_e4m3fn: MLA_FP8_E4M3, torch.uint8: MLA_FP8_E4M3}
STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_DTYPE", -3: "MLA_ERR_SHAPE",
          -4: "MLA_ERR_STRIDE", -5: "MLA_ERR_UNSUPPORTED", -6: "MLA_ERR_WORKSPACE",
          -7: "MLA_ERR_HIP"}


class MlaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {mla_status_str(status)} ({status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmla.so (built in-tree by mla_absorbed_decode_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(
                f"{lib_path} is not built; run `python -m mla_absorbed_decode_amd.build` "
                "(hipcc, gfx950) first")
        lib = ctypes.CDLL(lib_path)
        P = ctypes.POINTER(MlaTensor)
        vp, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                 ctypes.c_size_t)
        lib.mla_absorb_q.argtypes = [P, P, P, P, vp]
        lib.mla_concat_and_cache.argtypes = [P, P, P, P, vp]
        lib.mla_decode_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i32,
                                                  ctypes.POINTER(sz)]
        lib.mla_decode_attend.argtypes = [P, P, P, P, i64, f32, i32, P, P, vp, sz, vp]
        lib.mla_v_up.argtypes = [P, P, P, vp]
        dbl = ctypes.c_double
        lib.mla_rope_interleaved.argtypes = [P, P, dbl, vp]
        lib.mla_absorb_q_rope.argtypes = [P, P, P, P, dbl, P, vp]
        lib.mla_concat_and_cache_rope.argtypes = [P, P, P, P, dbl, P, vp]
        lib.mla_absorb_q_and_cache.argtypes = [P, P, P, P, P, P, P, P, P, dbl, vp]
        lib.mla_decode_attend_v_up.argtypes = [P, P, P, P, i64, f32, i32, P, P, P, P, vp, sz, vp]
        lib.mla_decode_attend_noalloc.argtypes = [P, P, P, P, i64, f32, i32, P, P, vp]
        lib.mla_decode_plan_size.argtypes = [i64, i64, i64, i64, i64, i64, i32,
                                             ctypes.POINTER(sz)]
        lib.mla_decode_plan.argtypes = [P, P, P, P, i64, i32, vp, sz, vp]
        lib.mla_decode_attend_planned.argtypes = [P, P, P, P, i64, f32, i32, P, P, vp, sz, vp, sz,
                                                  vp]
        lib.mla_decode_attend_v_up_planned.argtypes = [P, P, P, P, i64, f32, i32, P, P, P, P, vp,
                                                       sz, vp, sz, vp]
        lib.mla_concat_and_cache_fp8.argtypes = [P, P, P, P, vp, vp]
        lib.mla_decode_attend_fp8.argtypes = [P, P, P, P, i64, f32, i32, vp, vp, P, P, vp, sz, vp]
        lib.mla_decompress_kv.argtypes = [P, P, P, P, P, P, vp]
        lib.mla_prefill_attend.argtypes = [P, P, P, P, P, i64, f32, i32, P, P, vp]
        lib.mla_sparse_decode_fp8.argtypes = [P, P, P, f32, P, P, vp, sz, vp]
        lib.mla_sparse_workspace_size.argtypes = [i64, i64, i64, ctypes.POINTER(sz)]
        for fn in ("mla_concat_and_cache_fp8", "mla_decode_attend_fp8", "mla_absorb_q",
                   "mla_concat_and_cache", "mla_decode_workspace_size",
                   "mla_decode_attend", "mla_v_up", "mla_rope_interleaved", "mla_absorb_q_rope",
                   "mla_concat_and_cache_rope", "mla_absorb_q_and_cache",
                   "mla_decode_attend_v_up", "mla_decompress_kv", "mla_prefill_attend",
                   "mla_decode_attend_noalloc", "mla_decode_plan_size", "mla_decode_plan",
                   "mla_decode_attend_planned", "mla_decode_attend_v_up_planned",
                   "mla_sparse_decode_fp8", "mla_sparse_workspace_size"):
            getattr(lib, fn).restype = ctypes.c_int
        lib.mla_status_str.argtypes = [ctypes.c_int]
        lib.mla_status_str.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def header_symbols() -> list[str]:
    """Names of the functions include/mla.h declares."""
    with open(_HEADER) as f:
        text = f.read()
    return re.findall(r"^(?:int|const char\*)\s+(mla_\w+)\s*\(", text, flags=re.M)


def mla_status_str(status: int) -> str:
    return load().mla_status_str(int(status)).decode()


def desc(t: torch.Tensor | None):
    """mla_tensor descriptor of a tensor (None -> NULL)."""
    if t is None:
        return None
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() < 1 or t.dim() > 4:
        raise ValueError("rank must be 1..4")
    d = MlaTensor()
    d.data = t.data_ptr() if t.numel() else 0
    d.dtype = _DTYPES[t.dtype]
    d.rank = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _device_check(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libmla operates on device tensors; got a CPU tensor")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(rc: int, what: str):
    if rc != 0:
        raise MlaError(rc, what)


def mla_absorb_q(q_nope, w_uk_t, q_pe, q_out):
    """q_out[t,h,:L] = q_nope[t,h,:] @ w_uk_t[h]; q_out[t,h,L:] = q_pe[t,h|0,:]."""
    _device_check(q_nope, w_uk_t, q_pe, q_out)
    lib = load()
    _check(lib.mla_absorb_q(_ref(desc(q_nope)), _ref(desc(w_uk_t)), _ref(desc(q_pe)),
                            _ref(desc(q_out)), _stream(q_out)), "mla_absorb_q")
    return q_out


def mla_concat_and_cache(kv_c, k_pe, slot_mapping, kv_cache):
    """kv_cache[slot // PG, slot % PG, :] = [kv_c[t] | k_pe[t]] for valid slots."""
    _device_check(kv_c, k_pe, slot_mapping, kv_cache)
    lib = load()
    _check(lib.mla_concat_and_cache(_ref(desc(kv_c)), _ref(desc(k_pe)), _ref(desc(slot_mapping)),
                                    _ref(desc(kv_cache)), _stream(kv_cache)),
           "mla_concat_and_cache")
    return kv_cache


def mla_rope_interleaved(x, positions, base):
    """Rotate x [T, V, d] in place: pair (2i, 2i+1) of token t by positions[t] * base^(-2i/d)."""
    _device_check(x, positions)
    lib = load()
    _check(lib.mla_rope_interleaved(_ref(desc(x)), _ref(desc(positions)), float(base),
                                    _stream(x)), "mla_rope_interleaved")
    return x


def mla_absorb_q_rope(q_nope, w_uk_t, q_pe, positions, base, q_out):
    """mla_absorb_q with q_out[t,h,L:] = q_pe[t,h|0,:] rotated by positions[t]."""
    _device_check(q_nope, w_uk_t, q_pe, positions, q_out)
    lib = load()
    _check(lib.mla_absorb_q_rope(_ref(desc(q_nope)), _ref(desc(w_uk_t)), _ref(desc(q_pe)),
                                 _ref(desc(positions)), float(base), _ref(desc(q_out)),
                                 _stream(q_out)), "mla_absorb_q_rope")
    return q_out


def mla_concat_and_cache_rope(kv_c, k_pe, slot_mapping, positions, base, kv_cache):
    """mla_concat_and_cache with k_pe[t] rotated by positions[t] as it is written."""
    _device_check(kv_c, k_pe, slot_mapping, positions, kv_cache)
    lib = load()
    _check(lib.mla_concat_and_cache_rope(_ref(desc(kv_c)), _ref(desc(k_pe)),
                                         _ref(desc(slot_mapping)), _ref(desc(positions)),
                                         float(base), _ref(desc(kv_cache)), _stream(kv_cache)),
           "mla_concat_and_cache_rope")
    return kv_cache


def mla_absorb_q_and_cache(q_nope, w_uk_t, q_pe, q_out, kv_c, k_pe, slot_mapping, kv_cache,
                           positions=None, base=0.0):
    """mla_absorb_q and mla_concat_and_cache for the same tokens in one launch
    (with positions: both rope parts rotated)."""
    _device_check(q_nope, w_uk_t, q_pe, q_out, kv_c, k_pe, slot_mapping, kv_cache, positions)
    lib = load()
    _check(lib.mla_absorb_q_and_cache(_ref(desc(q_nope)), _ref(desc(w_uk_t)), _ref(desc(q_pe)),
                                      _ref(desc(q_out)), _ref(desc(kv_c)), _ref(desc(k_pe)),
                                      _ref(desc(slot_mapping)), _ref(desc(kv_cache)),
                                      _ref(desc(positions)), float(base), _stream(q_out)),
           "mla_absorb_q_and_cache")
    return q_out


def mla_concat_and_cache_fp8(kv_c, k_pe, slot_mapping, kv_cache, scale):
    """kv_cache[slot // PG, slot % PG, :] = e4m3([kv_c[t] | k_pe[t]] / scale) for valid
    slots; kv_cache is float8_e4m3fn (or uint8), scale a one-element float32 device
    tensor read when the kernel runs."""
    _device_check(kv_c, k_pe, slot_mapping, kv_cache, scale)
    _scalar_check(scale, "scale")
    lib = load()
    _check(lib.mla_concat_and_cache_fp8(_ref(desc(kv_c)), _ref(desc(k_pe)),
                                        _ref(desc(slot_mapping)), _ref(desc(kv_cache)),
                                        scale.data_ptr(), _stream(kv_cache)),
           "mla_concat_and_cache_fp8")
    return kv_cache


def _scalar_check(t, what):
    if t is None or t.dtype != torch.float32 or t.numel() < 1:
        raise ValueError(f"{what} must be a float32 device tensor holding one value")


def mla_decode_workspace_size(batch, q_len, n_heads, kv_rank, max_seqlen, page, dtype) -> int:
    out = ctypes.c_size_t(0)
    _check(load().mla_decode_workspace_size(int(batch), int(q_len), int(n_heads), int(kv_rank),
                                            int(max_seqlen), int(page), _DTYPES[dtype],
                                            ctypes.byref(out)), "mla_decode_workspace_size")
    return int(out.value)


def mla_decode_attend(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal, out,
                      lse=None, workspace=None):
    """Paged absorbed attention; writes out [B,Sq,N,L] and (optionally) lse [B,Sq,N].
    ``workspace`` (uint8 device tensor of at least mla_decode_workspace_size()
    bytes, reusable across calls) is allocated here when not given."""
    _device_check(q, kv_cache, block_table, seqlens, out, lse, workspace)
    lib = load()
    if workspace is None:
        nbytes = mla_decode_workspace_size(q.shape[0], q.shape[1], q.shape[2], out.shape[3],
                                           max_seqlen, kv_cache.shape[1], q.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.mla_decode_attend(_ref(desc(q)), _ref(desc(kv_cache)), _ref(desc(block_table)),
                                 _ref(desc(seqlens)), int(max_seqlen), float(softmax_scale),
                                 int(bool(causal)), _ref(desc(out)), _ref(desc(lse)),
                                 workspace.data_ptr(), workspace.numel(), _stream(out)),
           "mla_decode_attend")
    return out


def mla_decode_attend_noalloc(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale,
                              causal, out, lse=None):
    """mla_decode_attend without a workspace: the library's own device scratch
    serves as one, and nothing is allocated (for callers that cannot allocate).
    Calls that overlap in time on one GPU must not be issued (they share it)."""
    _device_check(q, kv_cache, block_table, seqlens, out, lse)
    lib = load()
    _check(lib.mla_decode_attend_noalloc(_ref(desc(q)), _ref(desc(kv_cache)),
                                         _ref(desc(block_table)), _ref(desc(seqlens)),
                                         int(max_seqlen), float(softmax_scale), int(bool(causal)),
                                         _ref(desc(out)), _ref(desc(lse)), _stream(out)),
           "mla_decode_attend_noalloc")
    return out


def mla_decode_attend_fp8(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal,
                          descale_q, descale_k, out, lse=None, workspace=None):
    """mla_decode_attend over an fp8 (float8_e4m3fn / uint8) cache: the scores take
    q * descale_q and keys * descale_k, the output values * descale_k (descales: one-
    element float32 device tensors read when the kernel runs)."""
    _device_check(q, kv_cache, block_table, seqlens, descale_q, descale_k, out, lse, workspace)
    _scalar_check(descale_q, "descale_q")
    _scalar_check(descale_k, "descale_k")
    lib = load()
    if workspace is None:
        nbytes = mla_decode_workspace_size(q.shape[0], q.shape[1], q.shape[2], out.shape[3],
                                           max_seqlen, kv_cache.shape[1], torch.float8_e4m3fn)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.mla_decode_attend_fp8(_ref(desc(q)), _ref(desc(kv_cache)), _ref(desc(block_table)),
                                     _ref(desc(seqlens)), int(max_seqlen), float(softmax_scale),
                                     int(bool(causal)), descale_q.data_ptr(), descale_k.data_ptr(),
                                     _ref(desc(out)), _ref(desc(lse)), workspace.data_ptr(),
                                     workspace.numel(), _stream(out)),
           "mla_decode_attend_fp8")
    return out


def mla_decode_attend_v_up(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal,
                           w_uv, o_lat, out, lse=None, workspace=None):
    """mla_decode_attend into o_lat (and lse), then out[b,i,h,:] = o_lat[b,i,h,:] @ w_uv[h];
    the split merge and the un-projection run as one kernel where they can."""
    _device_check(q, kv_cache, block_table, seqlens, w_uv, o_lat, out, lse, workspace)
    lib = load()
    if workspace is None:
        nbytes = mla_decode_workspace_size(q.shape[0], q.shape[1], q.shape[2], o_lat.shape[3],
                                           max_seqlen, kv_cache.shape[1], q.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.mla_decode_attend_v_up(_ref(desc(q)), _ref(desc(kv_cache)),
                                      _ref(desc(block_table)), _ref(desc(seqlens)), int(max_seqlen),
                                      float(softmax_scale), int(bool(causal)), _ref(desc(w_uv)),
                                      _ref(desc(o_lat)), _ref(desc(out)), _ref(desc(lse)),
                                      workspace.data_ptr(), workspace.numel(), _stream(out)),
           "mla_decode_attend_v_up")
    return out


def mla_decode_plan_size(batch, q_len, n_heads, kv_rank, max_seqlen, page, dtype) -> int:
    """Bytes of the split plan mla_decode_plan writes (0: such calls do not split)."""
    out = ctypes.c_size_t(0)
    _check(load().mla_decode_plan_size(int(batch), int(q_len), int(n_heads), int(kv_rank),
                                       int(max_seqlen), int(page), _DTYPES[dtype],
                                       ctypes.byref(out)), "mla_decode_plan_size")
    return int(out.value)


def mla_decode_plan(q, kv_cache, block_table, seqlens, max_seqlen, causal, plan=None):
    """The split plan of attention calls with q's sizes over this block_table and
    seqlens, written once for several calls (one per layer). ``plan`` (uint8 device
    tensor of at least mla_decode_plan_size() bytes) is allocated here when not given;
    returns it, or None when such calls do not split."""
    _device_check(q, kv_cache, block_table, seqlens, plan)
    lib = load()
    if plan is None:
        nbytes = mla_decode_plan_size(q.shape[0], q.shape[1], q.shape[2], 512, max_seqlen,
                                      kv_cache.shape[1], q.dtype)
        if nbytes == 0:
            return None
        plan = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check(lib.mla_decode_plan(_ref(desc(q)), _ref(desc(kv_cache)), _ref(desc(block_table)),
                               _ref(desc(seqlens)), int(max_seqlen), int(bool(causal)),
                               plan.data_ptr(), plan.numel(), _stream(q)), "mla_decode_plan")
    return plan


def _plan_args(plan):
    return (0, 0) if plan is None else (plan.data_ptr(), plan.numel())


def mla_decode_attend_planned(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale, causal,
                              out, plan, lse=None, workspace=None):
    """mla_decode_attend reading the split plan from mla_decode_plan (None: plan here)."""
    _device_check(q, kv_cache, block_table, seqlens, out, lse, workspace, plan)
    lib = load()
    if workspace is None:
        nbytes = mla_decode_workspace_size(q.shape[0], q.shape[1], q.shape[2], out.shape[3],
                                           max_seqlen, kv_cache.shape[1], q.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.mla_decode_attend_planned(_ref(desc(q)), _ref(desc(kv_cache)),
                                         _ref(desc(block_table)), _ref(desc(seqlens)),
                                         int(max_seqlen), float(softmax_scale), int(bool(causal)),
                                         _ref(desc(out)), _ref(desc(lse)), workspace.data_ptr(),
                                         workspace.numel(), *_plan_args(plan), _stream(out)),
           "mla_decode_attend_planned")
    return out


def mla_decode_attend_v_up_planned(q, kv_cache, block_table, seqlens, max_seqlen, softmax_scale,
                                   causal, w_uv, o_lat, out, plan, lse=None, workspace=None):
    """mla_decode_attend_v_up reading the split plan from mla_decode_plan."""
    _device_check(q, kv_cache, block_table, seqlens, w_uv, o_lat, out, lse, workspace, plan)
    lib = load()
    if workspace is None:
        nbytes = mla_decode_workspace_size(q.shape[0], q.shape[1], q.shape[2], o_lat.shape[3],
                                           max_seqlen, kv_cache.shape[1], q.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.mla_decode_attend_v_up_planned(_ref(desc(q)), _ref(desc(kv_cache)),
                                              _ref(desc(block_table)), _ref(desc(seqlens)),
                                              int(max_seqlen), float(softmax_scale),
                                              int(bool(causal)), _ref(desc(w_uv)),
                                              _ref(desc(o_lat)), _ref(desc(out)), _ref(desc(lse)),
                                              workspace.data_ptr(), workspace.numel(),
                                              *_plan_args(plan), _stream(out)),
           "mla_decode_attend_v_up_planned")
    return out


def mla_v_up(o_lat, w_uv, out):
    """out[t,h,:] = o_lat[t,h,:] @ w_uv[h]."""
    _device_check(o_lat, w_uv, out)
    lib = load()
    _check(lib.mla_v_up(_ref(desc(o_lat)), _ref(desc(w_uv)), _ref(desc(out)), _stream(out)),
           "mla_v_up")
    return out


def mla_decompress_kv(kv_c, k_pe, w_uk_t, w_uv, k_out, v_out):
    """k_out[s,h,:P] = kv_c[s] @ w_uk_t[h]^T, k_out[s,h,P:] = k_pe[s] (every head),
    v_out[s,h,:] = kv_c[s] @ w_uv[h]."""
    _device_check(kv_c, k_pe, w_uk_t, w_uv, k_out, v_out)
    lib = load()
    _check(lib.mla_decompress_kv(_ref(desc(kv_c)), _ref(desc(k_pe)), _ref(desc(w_uk_t)),
                                 _ref(desc(w_uv)), _ref(desc(k_out)), _ref(desc(v_out)),
                                 _stream(k_out)), "mla_decompress_kv")
    return k_out, v_out


def mla_prefill_attend(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, softmax_scale, causal,
                       out, lse=None):
    """Multi-head attention of packed sequences over per-head k [S,N,DK], v [S,N,DV];
    queries of sequence b are the suffix of its keys. Writes out [T,N,DV] and lse [T,N]."""
    _device_check(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse)
    lib = load()
    _check(lib.mla_prefill_attend(_ref(desc(q)), _ref(desc(k)), _ref(desc(v)),
                                  _ref(desc(cu_seqlens_q)), _ref(desc(cu_seqlens_k)),
                                  int(max_seqlen_q), float(softmax_scale), int(bool(causal)),
                                  _ref(desc(out)), _ref(desc(lse)), _stream(out)),
           "mla_prefill_attend")
    return out


def mla_sparse_workspace_size(tokens, n_heads, topk) -> int:
    out = ctypes.c_size_t(0)
    _check(load().mla_sparse_workspace_size(int(tokens), int(n_heads), int(topk),
                                            ctypes.byref(out)), "mla_sparse_workspace_size")
    return int(out.value)


def mla_sparse_decode_fp8(q, kv_cache, indices, softmax_scale, out, lse=None, workspace=None):
    """Sparse decode: token (b, i) of q [B,Sq,N,576] attends over the 656-byte
    entries of kv_cache [NB,PG,656] (uint8) at the slots indices[b,i,:] (-1: none).
    Writes out [B,Sq,N,512] and lse [B,Sq,N]. ``workspace`` (uint8 device tensor
    of at least mla_sparse_workspace_size() bytes) is allocated here when not given."""
    _device_check(q, kv_cache, indices, out, lse, workspace)
    lib = load()
    if workspace is None:
        nbytes = mla_sparse_workspace_size(q.shape[0] * q.shape[1], q.shape[2], indices.shape[2])
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.mla_sparse_decode_fp8(_ref(desc(q)), _ref(desc(kv_cache)), _ref(desc(indices)),
                                     float(softmax_scale), _ref(desc(out)), _ref(desc(lse)),
                                     workspace.data_ptr(), workspace.numel(), _stream(out)),
           "mla_sparse_decode_fp8")
    return out
