"""Benchmark of one absorbed-MLA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-v3] [--no-fp8]

A step is one pass of the whole hot path over one batch of the V2-Lite decode
workload (16 heads, kv_rank 512 + rope 64, batch 64, seqlens uniform on
[512, 4096], 64-token pages, random block table, bf16, values N(0, 0.1^2)):

  1+2. mla_absorb_q_and_cache, one launch:
       q fold   q_nope [64,16,128] x W_UK_T [16,128,512] -> q[..., :512], q_pe -> q[..., 512:]
       cache    each sequence's newest [c_kv | k_pe] row into its page
  3+4. mla_decode_attend_v_up_planned: split-KV attention over the paged latent cache,
       then the log-sum-exp merge and o_lat [64,16,512] x W_UV [16,512,128] in one kernel

The split plan (each attention workgroup's share of the keys) depends only on
the block table, seqlens and sizes, which every layer of a token step shares:
one mla_decode_plan launch heads each graph of layer calls and its time is
counted (--no-plan: every call plans for itself, as mla_decode_attend does).

Inputs are resident in HBM before timing. The latent cache is held in enough
copies (rotated per step) that the step's working set exceeds twice the
256 MB last-level cache, so the cache read is an HBM read. A token step's
layer calls (27, DeepSeek-V2-Lite's depth; call k reads copy k mod copies)
are captured in one HIP graph, the way a serving decode loop captures a
token's step in one graph; a second graph holds the calls a count leaves
over. W warm-up steps, then exactly K timed steps between device
synchronisations; one JSON line is printed.

value = latent-KV bytes the step must read (sum of seqlens x 576 x 2 B) per
second of step time. The roofline object covers the attention call (its
partial and merge kernels, and its share of the step's plan): graphs of that
call alone, laid out as the steps', are replayed for K calls right after the
steps and timed with HIP events on the stream they run on; its fractions are of the published HBM peak and of
the read rate measured on this GPU (measured_peaks, libmla_probe.so).

The other objects of the line: v2lite_warm (the attention call over one
cache copy, labelled warm), v3_decode (128 heads, cold over enough copies of
the rows each call reads; warm and permuted-table runs beside it), fp8_cache,
rope, sparse_fp8, nope_prefill (bf16 and fp32), cache_write (200 rows into a
3-layer unified slot), tiny_fp32 (the 64-token fp32 prefill and 32 decode
steps) and cpu_baseline (the fp64 oracle on the host: the V2-Lite step, and
the V3 and NoPE attention calls).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mla_absorbed_decode_amd as mla  # noqa: E402
import mla_inputs as mi  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_MATRIX_PEAK_TFLOPS = 157.3
LLC_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
# the sources the attention kernels are compiled from
DECODE_SRC = [os.path.join(ROOT, "mla_absorbed_decode_amd", "csrc", f)
              for f in ("decode.hip", "mla_device.h", "mla_kernels.h")]


def src_sha(paths) -> str:
    """sha256 prefix of the concatenated source files."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# One split plan per token step (mla_decode_plan), read by every layer's
# attention call; --no-plan makes every call plan for itself.
USE_PLAN = True


class Plan:
    """The split plan of attention calls over one block table and seqlens: one
    mla_decode_plan launch serves every layer's call of a token step."""

    def __init__(self, q, cache, bt, sl, max_seqlen):
        self.args = (q, cache, bt, sl, max_seqlen)
        n = mla.mla_decode_plan_size(q.shape[0], q.shape[1], q.shape[2], 512, max_seqlen,
                                     cache.shape[1], q.dtype) if USE_PLAN else 0
        self.buf = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None

    def launch(self):
        if self.buf is not None:
            q, cache, bt, sl, max_seqlen = self.args
            mla.mla_decode_plan(q, cache, bt, sl, max_seqlen, True, self.buf)


def plan_label(layers: int) -> str:
    if not USE_PLAN:
        return "none: every call plans its split in its own kernels"
    return (f"one mla_decode_plan launch per token step of {layers} layer calls, its time "
            "included (a timed count's last part step reuses the plan made before it)")


class Step:
    """Device-resident inputs of one decode step and the four calls."""

    def __init__(self, case: mi.DecodeCase, seed: int, copies: int, dev):
        d = case.dims
        self.case = case
        B, N = case.batch, d.n_head
        bf = torch.bfloat16
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(bf).to(dev)
        # query-side activations, new latent rows, weights: N(0, 0.1^2)
        self.q_nope = t(mi.normal(seed, 50, (B, N, d.d_nope), 0.1, "bf16"))
        self.q_pe = t(mi.normal(seed, 51, (B, N, d.d_rope), 0.1, "bf16"))
        self.kv_new = t(mi.normal(seed, 52, (B, d.kv_rank), 0.1, "bf16"))
        self.pe_new = t(mi.normal(seed, 53, (B, d.d_rope), 0.1, "bf16"))
        self.w_uk_t = t(mi.normal(seed, 54, (N, d.d_nope, d.kv_rank), 0.1, "bf16"))
        self.w_uv = t(mi.normal(seed, 55, (N, d.kv_rank, d.d_v), 0.1, "bf16"))
        # the newest token of sequence b sits at position seqlen_b - 1
        s = case.seqlens.astype(np.int64)
        bt = case.block_table
        slots = np.array([bt[b, (s[b] - 1) // case.page] * case.page + (s[b] - 1) % case.page
                          for b in range(B)], dtype=np.int64)
        self.slots = torch.from_numpy(slots).to(dev)
        base = t(case.pool)
        self.caches = [base] + [base.clone() for _ in range(copies - 1)]
        self.bt = torch.from_numpy(bt).to(dev)
        self.seqlens = torch.from_numpy(case.seqlens).to(dev)
        self.q = torch.empty(B, 1, N, d.entry, dtype=bf, device=dev)
        self.o_lat = torch.empty(B, 1, N, d.kv_rank, dtype=bf, device=dev)
        self.lse = torch.empty(B, 1, N, dtype=torch.float32, device=dev)
        self.out = torch.empty(B, N, d.d_v, dtype=bf, device=dev)
        nbytes = mla.mla_decode_workspace_size(B, 1, N, d.kv_rank, case.max_seqlen, case.page, bf)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        self.max_seqlen = case.max_seqlen
        self.plan = Plan(self.q, self.caches[0], self.bt, self.seqlens, self.max_seqlen)

    def attend(self, i: int):
        c = self.caches[i % len(self.caches)]
        mla.mla_decode_attend_planned(self.q, c, self.bt, self.seqlens, self.max_seqlen,
                                      self.case.scale, True, self.o_lat, self.plan.buf, self.lse,
                                      workspace=self.ws)

    def run(self, i: int):
        c = self.caches[i % len(self.caches)]
        # q fold and latent write of the new tokens in one launch
        mla.mla_absorb_q_and_cache(self.q_nope, self.w_uk_t, self.q_pe, self.q[:, 0],
                                   self.kv_new, self.pe_new, self.slots, c)
        # attention, then the split merge fused with the W_UV un-projection
        mla.mla_decode_attend_v_up_planned(
            self.q, c, self.bt, self.seqlens, self.max_seqlen, self.case.scale, True, self.w_uv,
            self.o_lat, self.out.view(self.case.batch, 1, self.case.dims.n_head, -1),
            self.plan.buf, self.lse, workspace=self.ws)


def capture(fn, n: int):
    """One HIP graph per cache copy, each holding fn(i)."""
    graphs = []
    for i in range(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(i)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def replay(graphs, first: int, count: int):
    """Replay `count` graphs round-robin between two events; returns elapsed ms."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(first, first + count):
        graphs[i % len(graphs)].replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


# Attention calls per token step: the decoder layers of DeepSeek-V2-Lite (27)
# and DeepSeek-V3 (61), from the models' published configurations. A token
# step computes its split plan once and every layer's call reads it.
V2_LITE_LAYERS = 27
V3_LAYERS = 61


class Rotation:
    """Graphs of calls fn(0), fn(1), ..., call k reading cache copy k % n: one
    graph of `per` calls (the smallest multiple of n that is at least `layers`:
    one token step's attention calls) led by head() (the step's one split plan),
    and, captured before any timing, a graph of the calls a count leaves over
    (they read the plan already made: the same step's tables)."""

    def __init__(self, fn, n: int, layers: int, head=None):
        self.fn, self.head = fn, head
        self.per = n * math.ceil(max(layers, 1) / n)

        def every(_):
            if head:
                head()
            for k in range(self.per):
                fn(k)

        self.whole = capture(every, 1)[0]
        self.tails = {}

    def prepare(self, count: int):
        r = count % self.per
        if r and r not in self.tails:
            self.tails[r] = capture(lambda _: [self.fn(k) for k in range(r)], 1)[0]

    def replay(self, count: int) -> float:
        """Replay exactly `count` calls between two events; returns ms."""
        self.prepare(count)
        tail = self.tails.get(count % self.per)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(count // self.per):
            self.whole.replay()
        if tail is not None:
            tail.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    def whole_calls(self, count: int) -> int:
        """count rounded up to whole token steps."""
        return self.per * max(1, math.ceil(count / self.per))


def time_calls(fn, n: int, layers: int, steps: int, warmup: int, head=None) -> float:
    """ms per call of fn over n rotated cache copies, timed over whole token
    steps of graphs (at least `steps` calls)."""
    rot = Rotation(fn, n, layers, head)
    if warmup:
        rot.replay(rot.whole_calls(warmup))
    count = rot.whole_calls(steps)
    return rot.replay(count) / count


def time_steps_eager(step: Step, steps: int, warmup: int):
    """As time_steps, every call launched from the host (a plan per step)."""
    for i in range(warmup):
        step.plan.launch()
        step.run(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(warmup, warmup + steps):
        step.plan.launch()
        step.run(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    t0.record()
    for i in range(warmup, warmup + steps):
        step.plan.launch()
        step.attend(i)
    t1.record()
    torch.cuda.synchronize()
    return total_ms, wall, t0.elapsed_time(t1) / steps


def copy_calibration(dev):
    """A plain device copy of a known 256 MiB (three times)."""
    src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def time_steps(step: Step, steps: int, warmup: int):
    """(ms for exactly `steps` steps, host seconds for them, ms per attention call)."""
    n = len(step.caches)
    step.plan.launch()
    for i in range(n):  # eager pass: one-time kernel attributes are set outside capture
        step.run(i)
        step.attend(i)
    torch.cuda.synchronize()
    rot = Rotation(step.run, n, V2_LITE_LAYERS, step.plan.launch)
    if warmup:
        rot.replay(warmup)
    rot.prepare(steps)
    wall0 = time.perf_counter()
    total_ms = rot.replay(steps)
    wall = time.perf_counter() - wall0
    attn = Rotation(step.attend, n, V2_LITE_LAYERS, step.plan.launch)
    if warmup:
        attn.replay(warmup)
    attn_ms = attn.replay(steps) / steps
    return total_ms, wall, attn_ms


def measured_peaks() -> dict:
    """The GPU's own peaks, measured by the probes of libmla_probe.so: dense
    bf16 MFMA (v_mfma_f32_16x16x32_bf16, eight independent chains per wave),
    an HBM read stream and an HBM copy (1 GiB each, non-temporal 16-byte
    accesses). The best of a few launch shapes is kept."""
    from mla_absorbed_decode_amd import probe

    mfma = max(probe.mfma_bf16_tflops(0, w) for w in (2, 4))
    read = max(probe.read_gbs(1 << 30, w) for w in (1, 2, 4))
    copy = probe.copy_gbs(1 << 30)
    # the V2-Lite call's bytes read alone: 256 workgroups x 17 tiles of 36 KB
    tile_us, tile_gbs = probe.tile_stream_us(256, 17)
    return {"mfma_bf16_tflops": round(mfma, 1), "hbm_read_gbs": round(read, 1),
            "hbm_copy_gbs": round(copy, 1),
            "tile_stream_us": round(tile_us, 2), "tile_stream_gbs": round(tile_gbs, 1),
            "how": "libmla_probe.so: bf16 16x16x32 MFMA chains (2 or 4 waves/SIMD), "
                   "1 GiB non-temporal read stream (1, 2 or 4 workgroups/CU) and copy; best kept; "
                   "tile_stream: 256 workgroups x 17 tiles of 36 KB from random 72 KB pages "
                   "through a three-slot LDS ring, the few-head decode's load schedule with "
                   "no arithmetic"}


def attention_warm_ms(step: Step, steps: int, warmup: int) -> float:
    """ms per attention call over ONE cache copy, replayed back to back: its
    163 MB of latent rows are partly resident in the 256 MB last-level cache
    (a warm figure, reported apart from the cold headline)."""
    return time_calls(lambda i: step.attend(0), 1, V2_LITE_LAYERS, steps, warmup,
                      step.plan.launch)


def attention_bytes(case: mi.DecodeCase) -> int:
    """Algorithmic bytes of one attention call: every visible latent row once,
    plus q, out and lse."""
    d = case.dims
    kv = int(case.seqlens.astype(np.int64).sum()) * d.entry * 2
    rows = case.batch * case.q_len * d.n_head
    return kv + rows * (d.entry * 2 + d.kv_rank * 2 + 4)


def attention_flops(case: mi.DecodeCase) -> int:
    d = case.dims
    pairs = int(case.seqlens.astype(np.int64).sum()) * d.n_head * case.q_len
    return pairs * 2 * (d.entry + d.kv_rank)


def pmc_traffic(kernel_key: str, launches_per_call: int = 1):
    """HBM bytes per attention call from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel_key}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("decode_src_sha") != src_sha(DECODE_SRC):
        return None
    return rec.get("hbm_bytes_per_call")


def cpu_baseline(case: mi.DecodeCase, step: Step, budget_s: float = 10.0):
    """The double-precision oracle on the host: fold, paged attention and
    un-projection of the full batch, repeated until ~budget_s of CPU work."""
    import oracle

    f64 = lambda x: np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    q_nope = f64(step.q_nope.float().cpu().numpy())
    w_uk_t = f64(step.w_uk_t.float().cpu().numpy())
    w_uv = f64(step.w_uv.float().cpu().numpy())
    q_pe = f64(step.q_pe.float().cpu().numpy())
    pool = f64(case.pool)
    bt, sl = case.block_table, case.seqlens

    def run(budget, max_reps):
        reps, t_used = 0, 0.0
        while t_used < budget and reps < max_reps:
            t0 = time.perf_counter()
            q_lat = oracle.fold_q(q_nope, w_uk_t)
            q = np.concatenate([q_lat, q_pe], axis=2)[:, None]
            o_lat, _ = oracle.attend_paged(q, pool, bt, sl, case.scale, True, case.dims.kv_rank)
            oracle.v_up(o_lat[:, 0], w_uv)
            t_used += time.perf_counter() - t0
            reps += 1
        return reps, t_used

    cores = oracle.num_threads()
    reps, t_used = run(budget_s, 100)
    kv_bytes = int(sl.astype(np.int64).sum()) * case.dims.entry * 2
    # the same work on one thread (one repetition, or more within a few seconds)
    oracle.set_num_threads(1)
    reps1, t1 = run(3.0, 10)
    oracle.set_num_threads(cores)
    return {
        "value": round(reps * kv_bytes / t_used / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "value_1_thread": round(reps1 * kv_bytes / t1 / 1e9, 4),
        "kind": "oracle",
        "sample": f"full V2-Lite batch (64 sequences, {int(sl.sum())} latent rows) x {reps} "
                  f"repetitions in {t_used:.1f} s on {cores} threads, x {reps1} in {t1:.1f} s on "
                  "one: fold, paged attention, un-projection in fp64 (the 64-row cache write is "
                  "omitted)",
        "cpu": cpu_model(),
    }


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _oracle_timed(fn, budget_s: float):
    """Best of up to 3 runs of fn within budget_s, or one run if it takes longer
    than 30 s. Returns (seconds, runs)."""
    best, runs, used = float("inf"), 0, 0.0
    while runs < 3:
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        best, runs, used = min(best, dt), runs + 1, used + dt
        if dt > 30.0 or used > budget_s:
            break
    return best, runs


def cpu_baseline_more(budget_s: float = 20.0) -> dict:
    """The oracle's absorbed attention alone on the V3 decode batch and on the
    NoPE prefill (the call timed, its inputs prepared beforehand)."""
    import oracle

    cores = oracle.num_threads()
    res = {}
    c = mi.v3_decode(seed=0, neighbour_fill=0.0)
    f64 = lambda x: np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    q, pool = f64(c.q), f64(c.pool)
    sec, runs = _oracle_timed(lambda: oracle.attend_paged(q, pool, c.block_table, c.seqlens,
                                                          c.scale, True, c.dims.kv_rank), budget_s)
    kv = int(c.seqlens.astype(np.int64).sum()) * c.dims.entry * 2
    res["v3_decode"] = {"value": round(kv / sec / 1e9, 4), "unit": "GB/s", "cores": cores,
                        "gflops": round(attention_flops(c) / sec / 1e9, 2),
                        "seconds": round(sec, 3), "runs": runs,
                        "sample": "the whole V3 batch (4 x 4096 keys, 128 heads): paged "
                                  "absorbed attention in fp64"}
    n = mi.nope_prefill(0, mi.BF16)
    d, t = n["dims"], n["t"]
    q_lat = oracle.fold_q(f64(n["q_nope"]), f64(n["w_uk_t"]))[None]
    kvp = f64(n["c_kv"]).reshape(t // n["page"], n["page"], d.kv_rank)
    bt = np.arange(t // n["page"], dtype=np.int32)[None]
    sl = np.array([t], dtype=np.int32)
    sec, runs = _oracle_timed(lambda: oracle.attend_paged(q_lat, kvp, bt, sl, n["scale"], True,
                                                          d.kv_rank), budget_s)
    pairs = d.n_head * t * (t + 1) // 2
    res["nope_prefill"] = {"value": round(pairs * 2 * (2 * d.kv_rank) / sec / 1e9, 2),
                           "unit": "GFLOP/s", "cores": cores, "seconds": round(sec, 3),
                           "runs": runs,
                           "sample": "absorbed attention of the NoPE prefill (64 heads, 2048 "
                                     "causal queries over 2048 latent rows) in fp64"}
    return res


def v3_secondary(dev, steps: int, warmup: int, eager: bool = False):
    """128-head V3 decode (B=4 x 4096, block-major view): attention call only.
    Cold: the calls rotate over enough copies of the 3-layer allocation that
    the latent rows they read (sum(seqlens) x 1152 B per call) exceed twice
    the last-level cache; also with a permuted block table (cold), and warm
    (one copy, its rows LLC-resident). eager: every call launched from the
    host, for counter collection."""
    c = mi.v3_decode(seed=0, neighbour_fill=0.0)
    d = c.dims
    bf = torch.bfloat16
    q = torch.from_numpy(c.q).to(bf).to(dev)
    kv_read = int(c.seqlens.astype(np.int64).sum()) * d.entry * 2
    copies = math.ceil(2 * LLC_BYTES / kv_read) + 1
    unis = [torch.from_numpy(c.unified()).to(bf).to(dev)]
    unis += [unis[0].clone() for _ in range(copies - 1)]
    views = [u[:, 1] for u in unis]
    bt = torch.from_numpy(c.block_table).to(dev)
    # the same pool read through a permuted block table (pages in random order)
    perm = mi.stream(0, 77).permutation(c.num_blocks)
    bt_perm = torch.from_numpy(perm[c.block_table].astype(np.int32)).to(dev)
    sl = torch.from_numpy(c.seqlens).to(dev)
    out = torch.empty(c.batch, 1, d.n_head, d.kv_rank, dtype=bf, device=dev)
    lse = torch.empty(c.batch, 1, d.n_head, dtype=torch.float32, device=dev)
    nbytes = mla.mla_decode_workspace_size(c.batch, 1, d.n_head, d.kv_rank, c.max_seqlen,
                                           c.page, bf)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    plan = Plan(q, views[0], bt, sl, c.max_seqlen)
    run = lambda i: mla.mla_decode_attend_planned(q, views[i % len(views)], bt, sl, c.max_seqlen,
                                                  c.scale, True, out, plan.buf, lse, workspace=ws)
    plan.launch()
    for i in range(len(views)):
        run(i)
    torch.cuda.synchronize()
    if eager:
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        for i in range(warmup):
            plan.launch()
            run(i)
        t0.record()
        for i in range(steps):
            plan.launch()
            run(i)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        return _v3_line(c, ms)

    ms = time_calls(run, len(views), V3_LAYERS, steps, warmup, plan.launch)
    line = _v3_line(c, ms)
    line["cache_copies"] = copies
    line["kv_bytes_rotated"] = copies * kv_read
    line["split_plan"] = plan_label(V3_LAYERS)
    warm_ms = time_calls(lambda i: run(0), 1, V3_LAYERS, steps, warmup, plan.launch)
    line["warm_attention_us"] = round(warm_ms * 1e3, 2)
    line["warm_label"] = "one cache copy reused: its 18.9 MB of latent rows stay in the LLC"
    plan_p = Plan(q, views[0], bt_perm, sl, c.max_seqlen)
    runp = lambda i: mla.mla_decode_attend_planned(q, views[i % len(views)], bt_perm, sl,
                                                   c.max_seqlen, c.scale, True, out, plan_p.buf,
                                                   lse, workspace=ws)
    plan_p.launch()
    runp(0)
    torch.cuda.synchronize()
    line["permuted_table_attention_us"] = round(
        time_calls(runp, len(views), V3_LAYERS, steps, warmup, plan_p.launch) * 1e3, 2)
    return line


def _v3_line(c, ms):
    byts, flops = attention_bytes(c), attention_flops(c)
    return {
        "workload": "V3 decode bf16: 128 heads, entry 576 / v 512, batch 4 x 4096, 64-token "
                    "pages, middle layer of a 3-layer block-major cache",
        "attention_us": round(ms * 1e3, 2),
        "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "gbs": round(byts / (ms * 1e-3) / 1e9, 1),
    }


def fp8_secondary(step: Step, dev, steps: int, warmup: int, eager: bool = False):
    """The V2-Lite decode over an fp8 (e4m3) latent cache: the same sequences,
    pages and block table, the cache values converted to e4m3, descales 1.
    Times the attention call (mla_decode_attend_fp8) and a whole fp8 step: q
    fold, fp8 write of the new rows (mla_concat_and_cache_fp8), attention,
    W_UV un-projection. Cache copies as for the bf16 step."""
    c = step.case
    d = c.dims
    codes = torch.from_numpy(mi.fp8_codes(c.pool)).to(dev).view(torch.float8_e4m3fn)
    touched = int(c.seqlens.astype(np.int64).sum()) * d.entry
    copies = max(2, math.ceil(2 * LLC_BYTES / touched) + 1)
    caches = [codes] + [codes.clone() for _ in range(copies - 1)]
    one = torch.ones(1, dtype=torch.float32, device=dev)
    B, N = c.batch, d.n_head
    q = torch.from_numpy(np.ascontiguousarray(c.q)).to(torch.bfloat16).to(dev)
    o_lat = torch.empty(B, 1, N, d.kv_rank, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, 1, N, dtype=torch.float32, device=dev)
    nbytes = mla.mla_decode_workspace_size(B, 1, N, d.kv_rank, c.max_seqlen, c.page,
                                           torch.float8_e4m3fn)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

    def attend(i):
        mla.mla_decode_attend_fp8(q, caches[i % copies], step.bt, step.seqlens, c.max_seqlen,
                                  c.scale, True, one, one, o_lat, lse, workspace=ws)

    def run(i):
        cache = caches[i % copies]
        mla.mla_absorb_q(step.q_nope, step.w_uk_t, step.q_pe, step.q[:, 0])
        mla.mla_concat_and_cache_fp8(step.kv_new, step.pe_new, step.slots, cache, one)
        mla.mla_decode_attend_fp8(step.q, cache, step.bt, step.seqlens, c.max_seqlen, c.scale,
                                  True, one, one, step.o_lat, step.lse, workspace=ws)
        mla.mla_v_up(step.o_lat[:, 0], step.w_uv, step.out)

    for i in range(copies):
        run(i)
        attend(i)
    torch.cuda.synchronize()
    if eager:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        res_ms = []
        for fn in (attend, run):
            for i in range(warmup):
                fn(i)
            t0.record()
            for i in range(steps):
                fn(i)
            t1.record()
            torch.cuda.synchronize()
            res_ms.append(t0.elapsed_time(t1) / steps)
        attn_ms, step_ms = res_ms
    else:
        attn_ms = time_calls(attend, copies, V2_LITE_LAYERS, steps, warmup)
        step_ms = time_calls(run, copies, V2_LITE_LAYERS, steps, warmup)
    rows = B * N
    a_bytes = touched + rows * (d.entry * 2 + d.kv_rank * 2 + 4)
    gbs = a_bytes / (attn_ms * 1e-3) / 1e9
    return {
        "workload": "V2-Lite decode with an fp8 e4m3 latent cache (576 B rows): batch 64, "
                    "seqlens U[512,4096], 64-token pages, descales 1",
        "attention_us": round(attn_ms * 1e3, 2),
        "attention_gbs": round(gbs, 1),
        "attention_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "attention_algorithmic_bytes": a_bytes,
        "step_us": round(step_ms * 1e3, 2),
        "step_kv_gbs": round(touched / (step_ms * 1e-3) / 1e9, 1),
        "kv_bytes": touched,
        "cache_copies": copies,
    }


def prefill_secondary(dev, steps: int, warmup: int):
    """The NoPE prefill workload (64 heads x d_nope 256, rank 512, v 256, one
    causal sequence of 2048 tokens, bf16) by both routes: absorbed (fold q
    through W_UK_T, attend over the latent rows, un-project through W_UV) and
    naive (decompress per-head K and V, multi-head attention). Each call is
    timed on its own (events around `steps` eager launches: the calls run for
    tens to hundreds of microseconds, so launch gaps do not matter)."""
    c = mi.nope_prefill(0, mi.BF16)
    d, t, scale = c["dims"], c["t"], c["scale"]
    N, P, V, L = d.n_head, d.d_nope, d.d_v, d.kv_rank
    bf = torch.bfloat16
    to = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(bf).to(dev)
    q_nope, c_kv, w_uk_t, w_uv = to(c["q_nope"]), to(c["c_kv"]), to(c["w_uk_t"]), to(c["w_uv"])
    page = c["page"]
    nb = t // page
    cache = c_kv.view(nb, page, L)
    bt = torch.arange(nb, dtype=torch.int32, device=dev).view(1, nb)
    sl = torch.tensor([t], dtype=torch.int32, device=dev)
    q = torch.empty(1, t, N, L, dtype=bf, device=dev)
    o_lat = torch.empty(1, t, N, L, dtype=bf, device=dev)
    out = torch.empty(t, N, V, dtype=bf, device=dev)
    ws = torch.empty(max(1, mla.mla_decode_workspace_size(1, t, N, L, t, page, bf)),
                     dtype=torch.uint8, device=dev)
    k_out = torch.empty(t, N, P, dtype=bf, device=dev)
    v_out = torch.empty(t, N, V, dtype=bf, device=dev)
    out2 = torch.empty(t, N, V, dtype=bf, device=dev)
    cu = torch.tensor([0, t], dtype=torch.int32, device=dev)
    calls = {
        "fold_us": lambda: mla.mla_absorb_q(q_nope, w_uk_t, None, q[0]),
        "absorbed_attend_us": lambda: mla.mla_decode_attend(q, cache, bt, sl, t, scale, True,
                                                            o_lat, None, workspace=ws),
        "v_up_us": lambda: mla.mla_v_up(o_lat[0], w_uv, out),
        "decompress_kv_us": lambda: mla.mla_decompress_kv(c_kv, None, w_uk_t, w_uv, k_out, v_out),
        "naive_attend_us": lambda: mla.mla_prefill_attend(q_nope, k_out, v_out, cu, cu, t, scale,
                                                          True, out2),
    }
    res = {"workload": "NoPE prefill bf16: 64 heads, d_nope 256, d_rope 0, d_v 256, kv_rank 512, "
                       "one causal sequence of 2048 tokens, U[-1,1] activations, "
                       "U[+-1/sqrt(512)] weights"}
    for name, fn in calls.items():
        for _ in range(max(1, warmup)):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        res[name] = round(t0.elapsed_time(t1) / steps * 1e3, 2)
    pairs = N * t * (t + 1) // 2
    fold = 2 * t * N * P * L
    tf = lambda flop, us: flop / (us * 1e-6) / 1e12
    abs_att, nai_att = pairs * 2 * (L + L), pairs * 2 * (P + V)
    res["absorbed_attend_tflops"] = round(tf(abs_att, res["absorbed_attend_us"]), 1)
    res["absorbed_attend_mfma_frac"] = round(res["absorbed_attend_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4)
    res["naive_attend_tflops"] = round(tf(nai_att, res["naive_attend_us"]), 1)
    res["naive_attend_mfma_frac"] = round(res["naive_attend_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4)
    res["decompress_kv_tflops"] = round(tf(2 * fold, res["decompress_kv_us"]), 1)
    res["absorbed_route_us"] = round(res["fold_us"] + res["absorbed_attend_us"] + res["v_up_us"], 2)
    res["naive_route_us"] = round(res["decompress_kv_us"] + res["naive_attend_us"], 2)
    # the same absorbed route in fp32 (fp32 inputs, fp32 MFMA; the naive
    # attention kernel takes bf16 only)
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    c32 = mi.nope_prefill(0, mi.F32)
    qn32, ckv32, wk32, wv32 = f32(c32["q_nope"]), f32(c32["c_kv"]), f32(c32["w_uk_t"]), f32(c32["w_uv"])
    cache32 = ckv32.view(nb, page, L)
    q32 = torch.empty(1, t, N, L, dtype=torch.float32, device=dev)
    o32 = torch.empty(1, t, N, L, dtype=torch.float32, device=dev)
    out32 = torch.empty(t, N, V, dtype=torch.float32, device=dev)
    ws32 = torch.empty(max(1, mla.mla_decode_workspace_size(1, t, N, L, t, page, torch.float32)),
                       dtype=torch.uint8, device=dev)
    k32 = torch.empty(t, N, P, dtype=torch.float32, device=dev)
    v32 = torch.empty(t, N, V, dtype=torch.float32, device=dev)
    calls32 = {
        "fold_us": lambda: mla.mla_absorb_q(qn32, wk32, None, q32[0]),
        "absorbed_attend_us": lambda: mla.mla_decode_attend(q32, cache32, bt, sl, t, scale, True,
                                                            o32, None, workspace=ws32),
        "v_up_us": lambda: mla.mla_v_up(o32[0], wv32, out32),
        "decompress_kv_us": lambda: mla.mla_decompress_kv(ckv32, None, wk32, wv32, k32, v32),
    }
    r32 = {}
    for name, fn in calls32.items():
        fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        reps = 3
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        r32[name] = round(t0.elapsed_time(t1) / reps * 1e3, 2)
    r32["absorbed_attend_tflops"] = round(tf(abs_att, r32["absorbed_attend_us"]), 1)
    r32["absorbed_attend_frac_of_fp32_matrix_peak"] = round(
        r32["absorbed_attend_tflops"] / FP32_MATRIX_PEAK_TFLOPS, 4)
    r32["absorbed_route_us"] = round(r32["fold_us"] + r32["absorbed_attend_us"] + r32["v_up_us"], 2)
    res["fp32"] = r32
    res["algorithmic_gflop"] = {"absorbed_attend": round(abs_att / 1e9, 1),
                                "naive_attend": round(nai_att / 1e9, 1),
                                "fold": round(fold / 1e9, 1), "v_up": round(fold / 1e9, 1),
                                "decompress_kv": round(2 * fold / 1e9, 1)}
    return res


def skewed_secondary(dev, steps: int, warmup: int):
    """A ragged V2-Lite decode batch with more units than workgroups: 300
    sequences of 16 heads, 299 of U[128, 1024] tokens and one of 32768, 64-token
    pages. The split-KV plan spreads the long sequence's keys over the grid
    like everyone else's. Cold: the calls rotate over enough copies of the
    pool that the rows they read exceed twice the last-level cache."""
    rng = mi.stream(0, 90)
    seqlens = rng.integers(128, 1025, size=300).astype(np.int32)
    seqlens[150] = 32768
    c = mi.decode_case(0, mi.V2_LITE, mi.BF16, seqlens, tail_fill=0.0)
    d = c.dims
    bf = torch.bfloat16
    q = torch.from_numpy(c.q).to(bf).to(dev)
    kv_read = int(c.seqlens.astype(np.int64).sum()) * d.entry * 2
    copies = math.ceil(2 * LLC_BYTES / kv_read) + 1
    pools = [torch.from_numpy(c.pool).to(bf).to(dev)]
    pools += [pools[0].clone() for _ in range(copies - 1)]
    bt = torch.from_numpy(c.block_table).to(dev)
    sl = torch.from_numpy(c.seqlens).to(dev)
    out = torch.empty(c.batch, 1, d.n_head, d.kv_rank, dtype=bf, device=dev)
    lse = torch.empty(c.batch, 1, d.n_head, dtype=torch.float32, device=dev)
    nbytes = mla.mla_decode_workspace_size(c.batch, 1, d.n_head, d.kv_rank, c.max_seqlen,
                                           c.page, bf)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    plan = Plan(q, pools[0], bt, sl, c.max_seqlen)
    run = lambda i: mla.mla_decode_attend_planned(q, pools[i % copies], bt, sl, c.max_seqlen,
                                                  c.scale, True, out, plan.buf, lse, workspace=ws)
    plan.launch()
    for i in range(copies):
        run(i)
    torch.cuda.synchronize()
    ms = time_calls(run, copies, V2_LITE_LAYERS, steps, warmup, plan.launch)
    byts = attention_bytes(c)
    return {
        "workload": "V2-Lite decode bf16, 300 sequences: 299 of U[128,1024] tokens and one of "
                    "32768, 64-token pages, N(0,0.1^2); split-KV over 256 workgroups",
        "sum_seqlens": int(c.seqlens.sum()),
        "units": c.batch,
        "workspace_bytes": nbytes,
        "cache_copies": copies,
        "split_plan": plan_label(V2_LITE_LAYERS),
        "attention_us": round(ms * 1e3, 2),
        "gbs": round(byts / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }


def _attend_graph_us(c: mi.DecodeCase, dev, steps: int, warmup: int, layers: int) -> float:
    """Attention call time (us) of case c over rotated cache copies (cold)."""
    d = c.dims
    bf = torch.bfloat16
    q = torch.from_numpy(np.ascontiguousarray(c.q)).to(bf).to(dev)
    kv_read = int(c.seqlens.astype(np.int64).sum()) * d.entry * 2
    copies = max(2, math.ceil(2 * LLC_BYTES / kv_read) + 1)
    pools = [torch.from_numpy(c.pool).to(bf).to(dev)]
    pools += [pools[0].clone() for _ in range(copies - 1)]
    bt = torch.from_numpy(c.block_table).to(dev)
    sl = torch.from_numpy(c.seqlens).to(dev)
    out = torch.empty(c.batch, 1, d.n_head, d.kv_rank, dtype=bf, device=dev)
    lse = torch.empty(c.batch, 1, d.n_head, dtype=torch.float32, device=dev)
    nbytes = mla.mla_decode_workspace_size(c.batch, 1, d.n_head, d.kv_rank, c.max_seqlen,
                                           c.page, bf)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    plan = Plan(q, pools[0], bt, sl, c.max_seqlen)
    run = lambda i: mla.mla_decode_attend_planned(q, pools[i % copies], bt, sl, c.max_seqlen,
                                                  c.scale, True, out, plan.buf, lse, workspace=ws)
    plan.launch()
    for i in range(copies):
        run(i)
    torch.cuda.synchronize()
    return time_calls(run, copies, layers, steps, warmup, plan.launch) * 1e3


def _fit(xs, ys):
    """Least-squares line y = a + b x: (a, b)."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    return my - b * mx, b


def sweep_secondary(dev, steps: int, warmup: int):
    """Attention time against the work of a call, for the fixed cost (the
    intercept of a straight-line fit) and the streaming rate (its slope):
    V2-Lite sequences (16 heads, seqlens U[512,4096]) at batch 16..128, and
    the 128-head geometry (batch 4) at seqlen 1024..8192."""
    res = {"v2lite_batch": [], "v3_seqlen": []}
    for B in (16, 32, 64, 128):
        seqlens = mi.stream(0, 5).integers(512, 4097, size=B).astype(np.int32)
        c = mi.decode_case(0, mi.V2_LITE, mi.BF16, seqlens, tail_fill=0.0)
        us = _attend_graph_us(c, dev, steps, warmup, V2_LITE_LAYERS)
        res["v2lite_batch"].append({"batch": B, "kv_mb": round(attention_bytes(c) / 1e6, 2),
                                    "attention_us": round(us, 2)})
    for S in (1024, 2048, 4096, 8192):
        c = mi.decode_case(0, mi.V3, mi.BF16, [S] * 4, tail_fill=0.0)
        us = _attend_graph_us(c, dev, steps, warmup, V3_LAYERS)
        res["v3_seqlen"].append({"seqlen": S, "kv_mb": round(attention_bytes(c) / 1e6, 2),
                                 "attention_us": round(us, 2)})
    for key in ("v2lite_batch", "v3_seqlen"):
        a, b = _fit([r["kv_mb"] for r in res[key]], [r["attention_us"] for r in res[key]])
        res[key + "_fit"] = {"intercept_us": round(a, 2), "us_per_mb": round(b, 4),
                             "slope_gbs": round(1e3 / b, 1) if b > 0 else None}
    res["workload"] = ("attention calls (bf16, 64-token pages, rotated cache copies): V2-Lite "
                       "geometry over batch, 128-head geometry over seqlen")
    return res


def sparse_secondary(dev, steps: int, warmup: int):
    """Sparse fp8 decode over 656-byte entries: the sparse-decode page's shape
    (batch 2 x 128 heads, top-128 over 32 blocks of 64 entries) and a longer
    DSA-sized list (64 tokens x 128 heads, top-2048 random slots out of 2048
    blocks of 64). Bytes count every listed entry once per token plus q and out;
    flops are 2 (576 + 512) per (token, head, listed key)."""
    res = {}
    for name, (B, N, K, NB, mode) in {"page_case": (2, 128, 128, 32, "disjoint"),
                                      "dsa_2048": (64, 128, 2048, 2048, "random")}.items():
        PG = 64
        cache = torch.from_numpy(mi.dsmla_payload(0, NB, PG)).to(dev)
        q = torch.from_numpy(mi.normal(0, 64, (B, 1, N, 576), 0.1, mi.BF16)).to(torch.bfloat16).to(dev)
        idx = torch.from_numpy(mi.dsmla_indices(0, B, 1, K, NB, PG, mode=mode, fill=1.0)).to(dev)
        out = torch.empty(B, 1, N, 512, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(B, 1, N, dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, mla.mla_sparse_workspace_size(B, N, K)), dtype=torch.uint8,
                         device=dev)
        run = lambda i: mla.mla_sparse_decode_fp8(q, cache, idx, 576 ** -0.5, out, lse,
                                                  workspace=ws)
        run(0)  # eager first: one-time kernel attributes are set outside capture
        torch.cuda.synchronize()
        whole = capture(lambda _: [run(k) for k in range(4)], 1)[0]
        for _ in range(max(1, warmup)):
            whole.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            whole.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / (4 * steps) * 1e3
        byts = B * K * 656 + B * N * (576 + 512) * 2 + B * N * 4
        flops = B * N * K * 2 * (576 + 512)
        res[name] = {"batch": B, "heads": N, "topk": K, "us": round(us, 2),
                     "gbs": round(byts / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "tflops": round(flops / (us * 1e-6) / 1e12, 1),
                     "mfma_frac": round(flops / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
    res["workload"] = ("sparse fp8 decode, 656-byte entries (512 e4m3 + 4 f32 scales + 64 bf16 "
                       "rope), 64-entry pages, N(0,0.1^2) values, scales 1; graphs of 4 calls "
                       "on one pool (warm: the pools fit the last-level cache)")
    return res


def cache_write_secondary(dev, steps: int, warmup: int):
    """The latent cache write config: 200 bf16 [c_kv | k_pe] rows (N(0,1))
    through a random-permutation slot map into the middle layer of a 3-layer
    block-major unified slot [32, 3 x 64 x 576]. Graphs of 20 calls."""
    c = mi.cache_write_case(0)
    bf = torch.bfloat16
    kv_c = torch.from_numpy(c["kv_c"]).to(bf).to(dev)
    k_pe = torch.from_numpy(c["k_pe"]).to(bf).to(dev)
    slots = torch.from_numpy(c["slots"]).to(dev)
    buf = torch.zeros(c["buf_shape"], dtype=bf, device=dev)
    view = buf.view(c["num_blocks"], c["n_layers"], c["page"], c["entry"])[:, c["layer"]]
    reps = 20
    fn = lambda i: [mla.mla_concat_and_cache(kv_c, k_pe, slots, view) for _ in range(reps)]
    fn(0)
    graphs = capture(fn, 1)
    if warmup:
        replay(graphs, 0, warmup)
    us = replay(graphs, 0, steps) / (steps * reps) * 1e3
    nbytes = 2 * len(c["slots"]) * c["entry"] * 2  # each row read once and written once
    return {"workload": "cache write: 200 tokens x (512 + 64) bf16 into the middle layer of a "
                        "3-layer block-major unified slot [32, 3 x 64 x 576], random slots",
            "us": round(us, 2), "bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "bound": "latency (230 KB read + 230 KB written per call)"}


def tiny_fp32_secondary(dev, steps: int, warmup: int):
    """The tiny fp32 config (16 heads, d_nope 128, rope 64, v 128, rank 512,
    one 64-token page): the causal prefill of 64 tokens (fold, cache write,
    attention, un-projection), and the 32 decode steps of the stepwise gate
    (each writes row t, folds token t, attends over t + 1 keys and
    un-projects) as one graph."""
    c = mi.tiny_prefill_decode(0)
    d, T = c["dims"], c["t"]
    f = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    q_nope, q_pe, c_kv, k_pe = f(c["q_nope"]), f(c["q_pe"]), f(c["c_kv"]), f(c["k_pe"])
    w_uk_t, w_uv = f(c["w_uk_t"]), f(c["w_uv"])
    cache = torch.zeros(1, T, d.entry, dtype=torch.float32, device=dev)
    bt = torch.zeros(1, 1, dtype=torch.int32, device=dev)
    slots = torch.arange(T, dtype=torch.int64, device=dev)
    q = torch.empty(1, T, d.n_head, d.entry, dtype=torch.float32, device=dev)
    o_lat = torch.empty(1, T, d.n_head, d.kv_rank, dtype=torch.float32, device=dev)
    out = torch.empty(T, d.n_head, d.d_v, dtype=torch.float32, device=dev)
    sl_full = torch.tensor([T], dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, mla.mla_decode_workspace_size(1, T, d.n_head, d.kv_rank, T, T,
                                                          torch.float32)),
                     dtype=torch.uint8, device=dev)
    ws1 = torch.empty(max(1, mla.mla_decode_workspace_size(1, 1, d.n_head, d.kv_rank, T, T,
                                                           torch.float32)),
                      dtype=torch.uint8, device=dev)

    def prefill(_):
        mla.mla_absorb_q(q_nope, w_uk_t, q_pe, q[0])
        mla.mla_concat_and_cache(c_kv, k_pe, slots, cache)
        mla.mla_decode_attend(q, cache, bt, sl_full, T, c["scale"], True, o_lat, None,
                              workspace=ws)
        mla.mla_v_up(o_lat[0], w_uv, out)

    first = T // 2
    sls = [torch.tensor([t + 1], dtype=torch.int32, device=dev) for t in range(first, T)]
    q1 = torch.empty(1, 1, d.n_head, d.entry, dtype=torch.float32, device=dev)
    o1 = torch.empty(1, 1, d.n_head, d.kv_rank, dtype=torch.float32, device=dev)
    out1 = torch.empty(1, d.n_head, d.d_v, dtype=torch.float32, device=dev)

    def decode(_):
        for k, t in enumerate(range(first, T)):
            mla.mla_concat_and_cache(c_kv[t:t + 1], k_pe[t:t + 1], slots[t:t + 1], cache)
            mla.mla_absorb_q(q_nope[t:t + 1], w_uk_t, q_pe[t:t + 1], q1[:, 0])
            mla.mla_decode_attend(q1, cache, bt, sls[k], T, c["scale"], True, o1, None,
                                  workspace=ws1)
            mla.mla_v_up(o1[:, 0], w_uv, out1)

    res = {"workload": "tiny fp32: 16 heads, d_nope 128, d_rope 64, d_v 128, rank 512, "
                       "t_q = t_kv = 64 causal, one page; then 32 decode steps"}
    for name, fn in (("prefill_us", prefill), ("decode_32_steps_us", decode)):
        fn(0)
        graphs = capture(fn, 1)
        if warmup:
            replay(graphs, 0, warmup)
        res[name] = round(replay(graphs, 0, steps) / steps * 1e3, 2)
    pairs = d.n_head * T * (T + 1) // 2
    res["prefill_attention_pairs"] = pairs
    res["decode_step_us"] = round(res["decode_32_steps_us"] / (T - first), 2)
    return res


def rope_secondary(step: Step, dev, steps: int, warmup: int):
    """Interleaved rope at the V2-Lite decode step's shapes: the q fold and the
    cache write with and without the fused rotation (positions seqlen_b - 1),
    and the in-place rotation of a prefill-sized q_pe [32768, 16, 64] bf16
    (five copies, 335 MB, so the stream is not cache-resident)."""
    pos = (step.seqlens - 1).to(torch.int32)
    c0 = step.caches[0]
    calls = {
        "fold_us": lambda i: mla.mla_absorb_q(step.q_nope, step.w_uk_t, step.q_pe, step.q[:, 0]),
        "fold_rope_us": lambda i: mla.mla_absorb_q_rope(step.q_nope, step.w_uk_t, step.q_pe, pos,
                                                        mi.ROPE_BASE, step.q[:, 0]),
        "cache_write_us": lambda i: mla.mla_concat_and_cache(step.kv_new, step.pe_new, step.slots,
                                                             c0),
        "cache_write_rope_us": lambda i: mla.mla_concat_and_cache_rope(
            step.kv_new, step.pe_new, step.slots, pos, mi.ROPE_BASE, c0),
        "fold_and_cache_us": lambda i: mla.mla_absorb_q_and_cache(
            step.q_nope, step.w_uk_t, step.q_pe, step.q[:, 0], step.kv_new, step.pe_new,
            step.slots, c0),
        "fold_and_cache_rope_us": lambda i: mla.mla_absorb_q_and_cache(
            step.q_nope, step.w_uk_t, step.q_pe, step.q[:, 0], step.kv_new, step.pe_new,
            step.slots, c0, pos, mi.ROPE_BASE),
    }
    res = {"workload": "V2-Lite decode step shapes (64 tokens x 16 heads, d_rope 64, base 8e6); "
                       "in-place rope of [32768, 16, 64] bf16"}
    reps = 20  # calls per graph, so one replay's launch cost is spread over them

    def repeated(fn):
        def run(i):
            for _ in range(reps):
                fn(i)
        return run

    for name, fn in calls.items():
        for i in range(2):
            fn(i)
        graphs = capture(repeated(fn), 1)
        if warmup:
            replay(graphs, 0, warmup)
        res[name] = round(replay(graphs, 0, steps) / (steps * reps) * 1e3, 2)
    T, V, D = 32768, 16, 64
    xs = [torch.randn(T, V, D, device=dev).to(torch.bfloat16) for _ in range(5)]
    pos_l = torch.arange(T, dtype=torch.int32, device=dev)
    fn = lambda i: mla.mla_rope_interleaved(xs[i % len(xs)], pos_l, mi.ROPE_BASE)
    for i in range(len(xs)):
        fn(i)
    graphs = capture(fn, len(xs))
    if warmup:
        replay(graphs, 0, warmup)
    ms = replay(graphs, 0, steps) / steps
    nbytes = 2 * T * V * D * 2  # read and write each element once
    gbs = nbytes / (ms * 1e-3) / 1e9
    res["inplace_us"] = round(ms * 1e3, 2)
    res["inplace_gbs"] = round(gbs, 1)
    res["inplace_hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-v3", action="store_true", help="skip the 128-head secondary line")
    ap.add_argument("--no-rope", action="store_true", help="skip the rotary-embedding line")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-cache line")
    ap.add_argument("--no-skewed", action="store_true",
                    help="skip the 300-sequence ragged decode line")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the attention call over batch (V2-Lite) and seqlen "
                         "(128 heads): fixed cost and streaming rate")
    ap.add_argument("--no-sparse", action="store_true", help="skip the sparse fp8 decode line")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the NoPE prefill line (absorbed and naive routes)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call from the host instead of replaying graphs "
                         "(for counter collection)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA / HBM peaks (libmla_probe.so)")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the cache-write and tiny fp32 lines")
    ap.add_argument("--no-plan", action="store_true",
                    help="no shared split plan: every attention call plans for itself")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy three times (reference for "
                         "scaling HBM byte counters)")
    args = ap.parse_args()
    global USE_PLAN
    USE_PLAN = not args.no_plan
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this implementation runs on a single MI355X and has "
              "no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    mla.load()

    case = mi.v2lite_decode(seed=0)
    touched = int(case.seqlens.astype(np.int64).sum()) * case.dims.entry * 2
    copies = max(2, math.ceil(2 * LLC_BYTES / touched) + 1)
    step = Step(case, seed=0, copies=copies, dev=dev)
    print(f"# V2-Lite decode: B={case.batch} sum(seqlens)={int(case.seqlens.sum())} "
          f"KV {touched / 1e6:.1f} MB, {copies} cache copies", file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    timer = time_steps_eager if args.eager else time_steps
    total_ms, wall, attn_avg_ms = timer(step, args.steps, args.warmup)
    if args.copy_calibration:
        copy_calibration(dev)
    ms_per_step = total_ms / args.steps
    kv_gbs = touched / (ms_per_step * 1e-3) / 1e9
    pairs = int(case.seqlens.astype(np.int64).sum()) * case.dims.n_head
    a_bytes = attention_bytes(case)
    achieved = a_bytes / (attn_avg_ms * 1e-3) / 1e9
    roof = {
        "bound": "hbm",
        "kernel": "mla_decode_attend_planned (decode_partial + decode_merge; one decode_plan "
                  "per graph of calls)",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": pmc_traffic("decode_v2lite"),
        "algorithmic_bytes": a_bytes,
        "avg_us": round(attn_avg_ms * 1e3, 2),
    }
    line = {
        "metric": "MLA decode: latent-KV GB/s + query-heads·tokens/s; % HBM/MFMA roofline",
        "value": round(kv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "V2-Lite decode bf16: 16 heads, kv_rank 512 + rope 64, W_UK_T [16,128,512], "
                        "W_UV [16,512,128], batch 64, seqlens U[512,4096], 64-token pages, random "
                        "block table, N(0,0.1^2)",
            "global_batch": case.batch,
            "seq_len": int(case.max_seqlen),
            "sum_seqlens": int(case.seqlens.sum()),
            "parallelism": "single GPU",
        },
        "query_heads_tokens_per_s": round(pairs / (ms_per_step * 1e-3), 1),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "split_plan": plan_label(V2_LITE_LAYERS),
        "roofline": roof,
    }
    if not args.eager:
        warm_ms = attention_warm_ms(step, max(10, args.steps // 2), args.warmup)
        line["v2lite_warm"] = {
            "attention_us": round(warm_ms * 1e3, 2),
            "gbs": round(a_bytes / (warm_ms * 1e-3) / 1e9, 1),
            "label": "warm: one cache copy replayed back to back (its latent rows partly "
                     "LLC-resident); the headline and roofline are cold"}
    peaks = None
    if not args.no_peaks:
        peaks = measured_peaks()
        line["measured_peaks"] = peaks
        roof["peak_measured"] = peaks["hbm_read_gbs"]
        roof["frac_measured"] = round(achieved / peaks["hbm_read_gbs"], 4)
    if not args.no_v3:
        line["v3_decode"] = v3_secondary(dev, max(10, args.steps // 2), args.warmup,
                                         eager=args.eager)
        if peaks:
            line["v3_decode"]["mfma_frac_measured"] = round(
                line["v3_decode"]["tflops"] / peaks["mfma_bf16_tflops"], 4)
    if not args.no_skewed:
        line["skewed_300"] = skewed_secondary(dev, max(10, args.steps // 2), args.warmup)
    if args.sweep:
        line["sweep"] = sweep_secondary(dev, max(10, args.steps // 2), args.warmup)
    if not args.no_fp8:
        line["fp8_cache"] = fp8_secondary(step, dev, max(10, args.steps // 2), args.warmup,
                                          eager=args.eager)
    if not args.no_rope:
        line["rope"] = rope_secondary(step, dev, max(10, args.steps // 2), args.warmup)
    if not args.no_sparse:
        line["sparse_fp8"] = sparse_secondary(dev, max(5, args.steps // 5), min(args.warmup, 3))
    if not args.no_prefill:
        line["nope_prefill"] = prefill_secondary(dev, max(5, args.steps // 10), min(args.warmup, 3))
    if not args.no_small:
        line["cache_write"] = cache_write_secondary(dev, max(10, args.steps // 2), args.warmup)
        line["tiny_fp32"] = tiny_fp32_secondary(dev, max(10, args.steps // 2), args.warmup)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(case, step)
        line["cpu_baseline"].update(cpu_baseline_more())
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
