"""GPU checks of the measurement probes in libmla_probe.so (the benchmark's
measured peaks): each runs through its C entry point, and the rates it gives
are positive and below the published peaks of the GPU (HBM 8 TB/s, dense
bf16 MFMA 2.5 PFLOP/s), with a margin for timer resolution."""
import pytest
import torch

from helpers import say

pytestmark = pytest.mark.gpu


def test_probes_run_and_stay_below_published_peaks():
    from mla_absorbed_decode_amd import probe

    say("[probe] mfma, read, copy, tile stream")
    tf = probe.mfma_bf16_tflops(0, 2, iters=2000, reps=3)
    assert 100.0 < tf < 2500.0 * 1.05, tf
    rd = probe.read_gbs(1 << 28, 2, reps=3)
    assert 500.0 < rd < 8000.0 * 1.05, rd
    cp = probe.copy_gbs(1 << 28, reps=3)
    assert 500.0 < cp < 8000.0 * 1.05, cp
    # a small grid of the tile stream: 64 workgroups x 5 tiles (odd tile count:
    # the last page is read in its first half only)
    us, gbs = probe.tile_stream_us(64, 5, copies=2, reps=3)
    assert us > 0.0 and 0.0 < gbs < 8000.0 * 1.05, (us, gbs)
    torch.cuda.synchronize()
