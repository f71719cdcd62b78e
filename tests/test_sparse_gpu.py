"""GPU parity of the sparse fp8 decode (vLLM
"tests/kernels/attention/test_mla_cross_layer_kernel_equivalence.py",
test_flashmla_fp8_sparse_decode_unified_slot_view): 656-byte entries of 512
e4m3 codes, 4 f32 scales and 64 bf16 rope values, reached through per-token
top-k slot lists padded with -1.

- The page's case: 128 heads x 576, batch 2, top-128 over 32 blocks of 64
  entries, each sequence on its own blocks, scales 1; the middle layer of a
  3-layer unified slot (neighbours random bytes) gives the same bits as a
  contiguous copy, finite and non-zero, and meets the oracle.
- Random slot lists with -1 at random places, random scales, a ragged last
  tile, two query tokens; slots past the pool; empty lists; unused entries
  holding NaN bytes (never read into the result); reruns bit-identical.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from helpers import assert_close, assert_lse_close, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

SCALE = 576 ** -0.5


def _mla():
    import mla_absorbed_decode_amd as mla
    return mla


def _run(q, cache, idx, lse=True):
    mla = _mla()
    B, Sq, N, _ = q.shape
    out = torch.full((B, Sq, N, 512), float("nan"), dtype=torch.bfloat16, device=dev())
    ls = torch.full((B, Sq, N), float("nan"), dtype=torch.float32, device=dev()) if lse else None
    if not isinstance(idx, torch.Tensor):
        idx = torch.from_numpy(np.ascontiguousarray(idx)).to(dev())
    mla.mla_sparse_decode_fp8(q, cache, idx, SCALE, out, ls)
    torch.cuda.synchronize()
    return out, ls


def test_page_case_unified_slot_view_bit_identical():
    B, Sq, N, NB, PG, K, layers, layer = 2, 1, 128, 32, 64, 128, 3, 1
    say(f"sparse fp8 decode: page case B={B} N={N} topk={K} block-major view")
    payload = mi.dsmla_payload(0, NB, PG)
    q_np = mi.normal(0, 64, (B, Sq, N, 576), 0.1, mi.BF16)
    idx = mi.dsmla_indices(0, B, Sq, K, NB, PG, mode="disjoint")
    q = to_dev(q_np, "bf16")
    contiguous = torch.from_numpy(payload).to(dev())
    noise = mi.stream(0, 65).integers(0, 256, size=(NB, layers, PG, 656), dtype=np.uint8)
    unified = torch.from_numpy(noise).to(dev())
    unified[:, layer].copy_(contiguous)
    view = unified[:, layer]
    assert not view.is_contiguous() and view.stride(0) == layers * PG * 656
    a, la = _run(q, contiguous, idx)
    b, lb = _run(q, view, idx)
    assert torch.isfinite(a).all() and a.abs().max().item() > 0
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
    want, want_lse = oracle.sparse_decode(q_np, payload, idx, SCALE)
    assert_close(to_np(a), want, "bf16", "out")
    assert_lse_close(to_np(la), want_lse, "lse")


@pytest.mark.parametrize("N,Sq,K,scales", [(16, 2, 100, "random"), (128, 1, 256, "random"),
                                           (20, 3, 37, "ones")])
def test_random_lists_match_oracle(N, Sq, K, scales):
    B, NB, PG = 3, 24, 64
    say(f"sparse fp8 decode: random lists B={B} Sq={Sq} N={N} topk={K} scales={scales}")
    payload = mi.dsmla_payload(1, NB, PG, scales=scales)
    q_np = mi.normal(1, 64, (B, Sq, N, 576), 0.1, mi.BF16)
    idx = mi.dsmla_indices(1, B, Sq, K, NB, PG, mode="random", fill=0.8)
    out, lse = _run(to_dev(q_np, "bf16"), torch.from_numpy(payload).to(dev()), idx)
    want, want_lse = oracle.sparse_decode(q_np, payload, idx, SCALE)
    assert_close(to_np(out), want, "bf16", "out")
    assert_lse_close(to_np(lse), want_lse, "lse")
    again, lse2 = _run(to_dev(q_np, "bf16"), torch.from_numpy(payload).to(dev()), idx)
    assert torch.equal(again.view(torch.int16), out.view(torch.int16)) and torch.equal(lse2, lse)


def test_out_of_pool_slots_empty_lists_and_nan_entries():
    """Slots past the pool and -1 are no key; a token whose list has no key
    gets 0 and -inf; entries no list names hold NaN codes and NaN scales
    (slot 0 included, the entry that no-key places read) and leave the
    result finite."""
    B, Sq, N, NB, PG, K = 2, 2, 32, 8, 64, 48
    say("sparse fp8 decode: out-of-pool slots, empty lists, NaN entries")
    payload = mi.dsmla_payload(2, NB, PG, scales="random")
    idx = mi.dsmla_indices(2, B, Sq, K, NB, PG, mode="random", fill=0.5)
    idx[idx == 0] = 1                                   # slot 0 is never a key
    idx[0, 1, :] = -1                                   # an empty list
    idx[1, 0, 3] = NB * PG                              # past the pool
    idx[1, 0, 5] = NB * PG + 1000
    used = np.zeros(NB * PG, dtype=bool)
    used[idx[(idx >= 0) & (idx < NB * PG)]] = True
    flat = payload.reshape(NB * PG, 656)
    flat[~used, :512] = mi.FP8_NAN
    flat[~used, 512:528] = np.frombuffer(np.float32(np.nan).tobytes() * 4, np.uint8)
    q_np = mi.normal(2, 64, (B, Sq, N, 576), 0.1, mi.BF16)
    out, lse = _run(to_dev(q_np, "bf16"), torch.from_numpy(payload).to(dev()), idx)
    want, want_lse = oracle.sparse_decode(q_np, payload, idx, SCALE)
    got = to_np(out)
    assert np.all(got[0, 1] == 0.0) and np.all(np.isneginf(to_np(lse)[0, 1]))
    assert_close(got, want, "bf16", "out")
    assert_lse_close(to_np(lse), want_lse, "lse")


def test_zero_topk_gives_zero_and_minus_inf():
    B, Sq, N = 2, 1, 16
    say("sparse fp8 decode: top-k 0")
    payload = mi.dsmla_payload(3, 4, 64)
    q = to_dev(mi.normal(3, 64, (B, Sq, N, 576), 0.1, mi.BF16), "bf16")
    empty = torch.empty((B, Sq, 0), dtype=torch.int32, device=dev())  # inner stride 1
    out, lse = _run(q, torch.from_numpy(payload).to(dev()), empty)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_unsplit_many_tokens_and_workspace_reuse():
    """Enough tokens to fill the chip unsplit (no workspace); then a split call
    reusing one workspace twice gives the same bits."""
    mla = _mla()
    B, Sq, N, NB, PG, K = 256, 2, 128, 16, 64, 64
    say(f"sparse fp8 decode: unsplit B={B} Sq={Sq} N={N} topk={K}")
    assert mla.mla_sparse_workspace_size(B * Sq, N, K) == 0
    payload = mi.dsmla_payload(4, NB, PG, scales="random")
    q_np = mi.normal(4, 64, (B, Sq, N, 576), 0.1, mi.BF16)
    idx = mi.dsmla_indices(4, B, Sq, K, NB, PG, mode="random", fill=0.9)
    out, lse = _run(to_dev(q_np, "bf16"), torch.from_numpy(payload).to(dev()), idx)
    want, want_lse = oracle.sparse_decode(q_np, payload, idx, SCALE)
    assert_close(to_np(out), want, "bf16", "out")
    assert_lse_close(to_np(lse), want_lse, "lse")
    # a split call (few tokens, long lists) on a reused workspace
    B2, K2 = 2, 1024
    q2 = to_dev(mi.normal(5, 64, (B2, 1, N, 576), 0.1, mi.BF16), "bf16")
    idx2 = torch.from_numpy(mi.dsmla_indices(5, B2, 1, K2, NB, PG, mode="random", fill=0.95)).to(dev())
    need = mla.mla_sparse_workspace_size(B2, N, K2)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev())
    cache = torch.from_numpy(payload).to(dev())
    runs = []
    for _ in range(2):
        o = torch.full((B2, 1, N, 512), float("nan"), dtype=torch.bfloat16, device=dev())
        mla.mla_sparse_decode_fp8(q2, cache, idx2, SCALE, o, None, workspace=ws)
        runs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(runs[0].view(torch.int16), runs[1].view(torch.int16))
    w2, _ = oracle.sparse_decode(to_np(q2), payload, idx2.cpu().numpy(), SCALE)
    assert_close(to_np(runs[0]), w2, "bf16", "split out")
