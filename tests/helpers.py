"""Shared pieces of the GPU parity tests: device placement of the seeded
inputs, the paged-cache layouts, and the comparison bars.

Bars (floating point): max|got - want| <= tol * max(1, max|want|) with
tol = 1e-2 for bf16 inputs with fp32 accumulation and 1e-4 for fp32 inputs,
the form memra-engine's gpu_core_parity uses; because decode outputs here are
~1e-3..1e-2, a relative bar is added: max|got - want| <= rel * max|want| with
rel = 2e-2 (about five bf16 ulps) for bf16 and 1e-3 for fp32. Outputs must be
finite and not degenerate (max|got| > 1e-6).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {"bf16": 1e-2, "f32": 1e-4}
REL = {"bf16": 2e-2, "f32": 1e-3}


def say(*args):
    """Name the case on stdout (flushed) before a GPU step runs."""
    print(*args, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(td).to(dev())


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, want, dtype: str, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx = np.abs(want).max() if want.size else 0.0
    md = np.abs(got - want).max() if want.size else 0.0
    assert md <= TOL[dtype] * max(1.0, mx), f"{what}: maxdiff {md:.3e} vs scale {mx:.3e}"
    assert md <= REL[dtype] * mx + 1e-30, f"{what}: maxdiff {md:.3e} > {REL[dtype]} * {mx:.3e}"
    assert np.abs(got).max() > 1e-6, f"{what}: degenerate output"


def assert_lse_close(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    inf = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), inf), f"{what}: -inf pattern differs"
    if (~inf).any():
        d = np.abs(got[~inf] - want[~inf]) / np.maximum(1.0, np.abs(want[~inf]))
        assert d.max() <= 1e-3, f"{what}: lse rel diff {d.max():.3e}"


class DeviceCache:
    """A DecodeCase's pool on the device, either contiguous [NB, PG, E] or as
    the middle layer of a block-major allocation [NB, n_layers, PG, E]."""

    def __init__(self, case, block_major: bool):
        self.case = case
        dt = case.dtype
        if block_major and case.n_layers > 1:
            self.alloc = to_dev(case.unified(), dt)
            self.view = self.alloc[:, case.layer]
            assert not self.view.is_contiguous()
        else:
            self.alloc = to_dev(case.pool, dt)
            self.view = self.alloc


def run_decode(case, block_major=False, lse=True, workspace=None):
    """Run mla_decode_attend on a DecodeCase; returns (out, lse) device tensors."""
    import mla_absorbed_decode_amd as mla

    c = case
    q = to_dev(c.q, c.dtype)
    cache = DeviceCache(c, block_major)
    bt = torch.from_numpy(c.block_table).to(dev())
    sl = torch.from_numpy(c.seqlens).to(dev())
    td = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    out = torch.full((c.batch, c.q_len, c.dims.n_head, c.dims.kv_rank), float("nan"), dtype=td,
                     device=dev())
    lse_t = torch.full((c.batch, c.q_len, c.dims.n_head), float("nan"), dtype=torch.float32,
                       device=dev()) if lse else None
    mla.mla_decode_attend(q, cache.view, bt, sl, c.max_seqlen, c.scale, c.causal, out, lse_t,
                          workspace=workspace)
    torch.cuda.synchronize()
    return out, lse_t
