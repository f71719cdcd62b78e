"""Measured peaks of the GPU the benchmark runs on (libmla_probe.so, see
include/mla_probe.h): the dense bf16 MFMA rate and the HBM copy and read rates,
and the time of the few-head decode's tile stream with no arithmetic.

These are measurement tools for the benchmark, not part of the attention
path. Each function enqueues its probe kernel on the current stream, times it
with HIP events on that stream, and returns the rate.
"""
from __future__ import annotations

import ctypes
import os

import torch

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_probe.so")
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} is not built; run `python -m mla_absorbed_decode_amd.build`")
        lib = ctypes.CDLL(lib_path)
        lib.mla_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_int),
                                            ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
        lib.mla_probe_mfma_bf16.restype = ctypes.c_int
        lib.mla_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
        lib.mla_probe_copy.restype = ctypes.c_int
        lib.mla_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_int, ctypes.c_void_p]
        lib.mla_probe_read.restype = ctypes.c_int
        lib.mla_probe_tile_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.mla_probe_tile_stream.restype = ctypes.c_int
        _lib = lib
    return _lib


def _timed(fn, reps: int) -> float:
    """Median ms of `reps` launches of fn() on the current stream."""
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        fn()
        t1.record(stream)
        t1.synchronize()
        times.append(t0.elapsed_time(t1))
    times.sort()
    return times[len(times) // 2]


def mfma_bf16_tflops(shape: int = 0, waves_per_simd: int = 1, iters: int = 20000,
                     reps: int = 5) -> float:
    """Dense bf16 MFMA TFLOP/s over the whole GPU (shape 0: 16x16x32, 1: 32x32x16)."""
    lib = load()
    dev = torch.device("cuda:0")
    sink = torch.empty(1024 * 256 * waves_per_simd, dtype=torch.float32, device=dev)
    wgs, flops = ctypes.c_int(0), ctypes.c_double(0.0)
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        rc = lib.mla_probe_mfma_bf16(sink.data_ptr(), shape, iters, waves_per_simd,
                                     ctypes.byref(wgs), ctypes.byref(flops), stream)
        if rc:
            raise RuntimeError(f"mla_probe_mfma_bf16 failed ({rc})")

    run()
    ms = _timed(run, reps)
    return flops.value / (ms * 1e-3) / 1e12


def copy_gbs(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """HBM GB/s of a device copy of nbytes (read + write counted)."""
    lib = load()
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        rc = lib.mla_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream)
        if rc:
            raise RuntimeError(f"mla_probe_copy failed ({rc})")

    run()
    ms = _timed(run, reps)
    return 2 * nbytes / (ms * 1e-3) / 1e9


def read_gbs(nbytes: int = 1 << 30, workgroups_per_cu: int = 8, reps: int = 5) -> float:
    """HBM GB/s of a read-only stream over nbytes."""
    lib = load()
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(1024 * 256 * workgroups_per_cu, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        rc = lib.mla_probe_read(sink.data_ptr(), src.data_ptr(), nbytes, workgroups_per_cu, stream)
        if rc:
            raise RuntimeError(f"mla_probe_read failed ({rc})")

    run()
    ms = _timed(run, reps)
    return nbytes / (ms * 1e-3) / 1e9


TILE_BYTES = 32 * 1152   # a 32-row tile of 576 bf16 latent rows
PAGE_BYTES = 2 * TILE_BYTES


def tile_stream_us(workgroups: int = 256, tiles_per_workgroup: int = 17, copies: int = 4,
                   reps: int = 12, seed: int = 0) -> tuple[float, float]:
    """Median µs (and GB/s) of reading workgroups * tiles_per_workgroup 36 KB
    tiles in the few-head decode's partition and load schedule, with no
    arithmetic: the pages (two tiles each) in a seeded random order, as a
    shuffled block table gives them. Launches rotate over `copies` buffers so
    that the reads come from HBM."""
    import numpy as np

    lib = load()
    dev = torch.device("cuda:0")
    tiles = workgroups * tiles_per_workgroup
    pages = (tiles + 1) // 2
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(pages).astype(np.int32)).to(dev)
    bufs = [torch.ones(pages * PAGE_BYTES, dtype=torch.uint8, device=dev) for _ in range(copies)]
    sink = torch.empty(workgroups, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    turn = [0]

    def run():
        buf = bufs[turn[0] % copies]
        turn[0] += 1
        rc = lib.mla_probe_tile_stream(sink.data_ptr(), buf.data_ptr(), perm.data_ptr(),
                                       tiles_per_workgroup, workgroups, stream)
        if rc:
            raise RuntimeError(f"mla_probe_tile_stream failed ({rc})")

    for _ in range(copies):
        run()
    ms = _timed(run, reps)
    return ms * 1e3, tiles * TILE_BYTES / (ms * 1e-3) / 1e9
