"""GPU parity of the absorption folds (mla_absorb_q, mla_v_up) against the
double-precision bmm oracle, at the shapes and views of vllm.cpp
"tests/vt/test_ops_mla_absorb.cpp": the V2-Lite W_UK fold and W_UV
un-projection, the V3 128-head fold, the single-token decode un-projection,
the transposed operand and output views, and the exact nope/rope concat."""
import numpy as np
import pytest
import torch

import mla_absorbed_decode_amd as mla
import oracle
from helpers import dev, say

pytestmark = pytest.mark.gpu


def rand(shape, seed, dtype=torch.bfloat16, scale=1.0):
    g = np.random.default_rng(seed)
    x = torch.from_numpy((g.uniform(-1, 1, shape) * scale).astype(np.float32)).to(dtype)
    return x


def worst_rel(got, want, floor):
    return float((np.abs(got - want) / np.maximum(floor, np.abs(want))).max())


# vllm.cpp GPU cases: (heads, batch, k, n) with a [heads, batch, k] operand
P1_CASES = [
    (16, 8, 128, 512, "V2-Lite W_UK fold"),
    (16, 8, 512, 128, "V2-Lite W_UV un-projection"),
    (128, 3, 128, 512, "V3 W_UK fold"),
    (16, 1, 512, 128, "single-token decode v-up"),
]


@pytest.mark.parametrize("H,Bt,K,N,what", P1_CASES)
def test_fold_matches_oracle_and_is_deterministic(H, Bt, K, N, what):
    say(f"[bmm] {what}")
    a_store = rand((H, Bt, K), 1234)            # [heads, batch, k] storage
    w = rand((H, K, N), 4321)
    a = a_store.to(dev()).permute(1, 0, 2)      # [batch, heads, k] view for the ABI
    wd = w.to(dev())
    out = torch.full((Bt, H, N), float("nan"), dtype=torch.bfloat16, device=dev())
    if N == 512:
        mla.mla_absorb_q(a, wd, None, out)
    else:
        mla.mla_v_up(a, wd, out)
    torch.cuda.synchronize()
    ref = oracle.bmm(a_store.float().numpy(), w.float().numpy())  # [H, Bt, N]
    got = out.permute(1, 0, 2).float().cpu().numpy()
    assert not np.isnan(got).any()
    assert worst_rel(got, ref, 1e-2) < 1e-2
    for _ in range(3):
        again = torch.full_like(out, float("nan"))
        if N == 512:
            mla.mla_absorb_q(a, wd, None, again)
        else:
            mla.mla_v_up(a, wd, again)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), out.view(torch.int16))


def test_transposed_input_and_output_views():
    # o_lat stored [B, N, L]; out written into a [N, B, V] buffer through its [B, N, V] view
    H, Bt, K, N = 16, 5, 512, 128
    raw = rand((Bt, H, K), 2468)
    w = rand((H, K, N), 8642)
    store = torch.full((H, Bt, N), float("nan"), dtype=torch.bfloat16, device=dev())
    out = store.permute(1, 0, 2)
    mla.mla_v_up(raw.to(dev()), w.to(dev()), out)
    torch.cuda.synchronize()
    ref = oracle.v_up(raw.float().numpy(), w.float().numpy())
    got = out.float().cpu().numpy()
    assert not np.isnan(got).any()
    assert worst_rel(got, ref, 1e-2) < 2e-2


@pytest.mark.parametrize("T,H", [(16, 128), (9, 16), (64, 16), (1, 16)])
def test_absorb_q_rope_concat_is_exact(T, H):
    say(f"[bmm] absorb_q + rope concat T={T} H={H}")
    qn_store = rand((H, T, 128), 55)
    q_nope = qn_store.to(dev()).permute(1, 0, 2)   # the transposed nope operand
    w = rand((H, 128, 512), 66, scale=512 ** -0.5).to(dev())
    q_pe = rand((T, H, 64), 77).to(dev())
    q_out = torch.full((T, H, 576), float("nan"), dtype=torch.bfloat16, device=dev())
    mla.mla_absorb_q(q_nope, w, q_pe, q_out)
    torch.cuda.synchronize()
    assert torch.equal(q_out[..., 512:].view(torch.int16), q_pe.view(torch.int16))
    ref = oracle.fold_q(q_nope.float().cpu().numpy(), w.float().cpu().numpy())
    got = q_out[..., :512].float().cpu().numpy()
    assert worst_rel(got, ref, 1e-2) < 1e-2


def test_absorb_q_broadcast_rope_row():
    T, H = 13, 16
    q_nope = rand((T, H, 128), 3690).to(dev())
    w = rand((H, 128, 512), 963, scale=512 ** -0.5).to(dev())
    q_pe = rand((T, 1, 64), 11).to(dev())
    q_out = torch.full((T, H, 576), float("nan"), dtype=torch.bfloat16, device=dev())
    mla.mla_absorb_q(q_nope, w, q_pe, q_out)
    torch.cuda.synchronize()
    assert torch.equal(q_out[..., 512:].view(torch.int16),
                       q_pe.expand(T, H, 64).contiguous().view(torch.int16))


@pytest.mark.parametrize("shape", [(6, 5, 9, 4), (11, 4, 24, 64), (6, 3, 12, 48), (7, 16, 512, 100)])
def test_odd_sizes(shape):
    T, H, K, N = shape
    say(f"[bmm] odd sizes {shape}")
    a = rand((T, H, K), 33).to(dev())
    w = rand((H, K, N), 44).to(dev())
    out = torch.full((T, H, N), float("nan"), dtype=torch.bfloat16, device=dev())
    mla.mla_v_up(a, w, out)
    torch.cuda.synchronize()
    ref = oracle.v_up(a.float().cpu().numpy(), w.float().cpu().numpy())
    got = out.float().cpu().numpy()
    assert np.all(np.abs(got - ref) <= 5e-3 * np.maximum(1.0, np.abs(ref)))


# 16 heads: calls of at most 16 tokens take the split-K kernel; the others take
# 64 x 64 tiles, whose tiles of at most 16 tokens (the 6-token tail of T = 70,
# the 16-token one of T = 272) use the narrow layout (each wave one 16-column group)
@pytest.mark.parametrize("T,K,N", [(64, 128, 512), (64, 512, 128), (3, 256, 512), (70, 512, 256),
                                   (1, 512, 128), (16, 128, 512), (70, 512, 80), (17, 256, 96),
                                   (300, 256, 512), (272, 128, 256)])
def test_fp32_folds(T, K, N):
    H = 16
    a = rand((T, H, K), 5, torch.float32).to(dev())
    w = rand((H, K, N), 6, torch.float32, scale=512 ** -0.5).to(dev())
    out = torch.full((T, H, N), float("nan"), dtype=torch.float32, device=dev())
    mla.mla_v_up(a, w, out)
    torch.cuda.synchronize()
    ref = oracle.v_up(a.cpu().numpy(), w.cpu().numpy())
    got = out.cpu().numpy()
    assert np.abs(got - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


# prefill-sized token counts take the 128 x 128 pipelined tiles
@pytest.mark.parametrize("T,H,N", [(256, 4, 512), (300, 3, 512), (700, 2, 512)])
def test_large_fold_with_rope_concat(T, H, N):
    say(f"[bmm] large absorb_q T={T} H={H} N={N}")
    qn_store = rand((H, T, 128), 56)
    q_nope = qn_store.to(dev()).permute(1, 0, 2)   # the transposed nope operand
    w = rand((H, 128, N), 67, scale=512 ** -0.5).to(dev())
    q_pe = rand((T, H, 64), 78).to(dev())
    q_out = torch.full((T, H, N + 64), float("nan"), dtype=torch.bfloat16, device=dev())
    mla.mla_absorb_q(q_nope, w, q_pe, q_out)
    torch.cuda.synchronize()
    assert torch.equal(q_out[..., N:].view(torch.int16), q_pe.view(torch.int16))
    ref = oracle.fold_q(q_nope.float().cpu().numpy(), w.float().cpu().numpy())
    got = q_out[..., :N].float().cpu().numpy()
    assert worst_rel(got, ref, 1e-2) < 1e-2
    for _ in range(2):
        again = torch.full_like(q_out, float("nan"))
        mla.mla_absorb_q(q_nope, w, q_pe, again)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), q_out.view(torch.int16))


def test_large_fold_with_rotated_rope():
    T, H = 333, 2
    say(f"[bmm] large absorb_q_rope T={T}")
    q_nope = rand((T, H, 128), 57).to(dev())
    w = rand((H, 128, 512), 68, scale=512 ** -0.5).to(dev())
    q_pe = rand((T, H, 64), 79).to(dev())
    pos = torch.arange(T, dtype=torch.int32, device=dev()) * 13
    a = torch.full((T, H, 576), float("nan"), dtype=torch.bfloat16, device=dev())
    mla.mla_absorb_q_rope(q_nope, w, q_pe, pos, 8e6, a)
    # the same rotation applied in place, then a plain concat
    q_rot = q_pe.clone()
    mla.mla_rope_interleaved(q_rot, pos, 8e6)
    b = torch.full_like(a, float("nan"))
    mla.mla_absorb_q(q_nope, w, q_rot, b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("T,H,K,N", [(333, 16, 512, 128), (260, 3, 512, 48), (512, 2, 256, 256)])
def test_large_v_up_transposed_output(T, H, K, N):
    say(f"[bmm] large v_up T={T} H={H} K={K} N={N}")
    o_lat = rand((T, H, K), 91).to(dev())
    w = rand((H, K, N), 92, scale=K ** -0.5).to(dev())
    store = torch.full((H, T, N + 8), float("nan"), dtype=torch.bfloat16, device=dev())
    out = store[:, :, :N].transpose(0, 1)           # [T, H, N] view of head-major rows
    mla.mla_v_up(o_lat, w, out)
    torch.cuda.synchronize()
    ref = oracle.v_up(o_lat.float().cpu().numpy(), w.float().cpu().numpy())
    got = out.float().cpu().numpy()
    assert not np.isnan(got).any()
    assert worst_rel(got, ref, 1e-2) < 1e-2
    assert torch.isnan(store[:, :, N:]).all()
