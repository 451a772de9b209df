"""The vector-unit issue probe (a measurement aid beside the full-grid search's roofline): every
form runs, every chain's sum is the closed form of its fma recurrence evaluated in binary32 on the
host, and the clocks it reports are positive.  Through the C ABI (libcq.so)."""
import numpy as np
import pytest
import torch

import post_weight_quantization_group_amd as cq

pytestmark = pytest.mark.gpu


def _chains(mode, iters):
    """The eight chains of each of the 256 threads after `iters` steps, in binary32 with one
    rounding per fma (numpy float64 products of binary32 values are exact, then one rounding)."""
    a, b = np.float32(1.0 - 2.0 ** -20), np.float32(2.0 ** -20)
    tid = np.arange(256)
    x = np.stack([((tid + k).astype(np.float32) * np.float32(2.0 ** -10)) for k in range(8)]).astype(np.float32)
    y = np.stack([np.full(256, np.float32(k + 1) * b, np.float32) for k in range(8)])
    for _ in range(iters):
        if mode == 0:
            x = (x.astype(np.float64) * np.float64(a) + y.astype(np.float64)).astype(np.float32)
        elif mode == 1:
            x = (y.astype(np.float64) * np.float64(a) + x.astype(np.float64)).astype(np.float32)
        else:
            x = (x.astype(np.float64) * np.float64(a) + np.float64(b)).astype(np.float32)
    s = np.zeros(256, np.float32)
    for k in range(8):
        s = (s + x[k]).astype(np.float32)
    return s


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_probe_sums_and_clocks(mode):
    iters, blocks = 37, 3
    r = cq.probe_valu_fma(iters, blocks, mode)
    torch.cuda.synchronize()
    out = r["out"].cpu().numpy().reshape(blocks, 256)
    want = _chains(mode, iters)
    for blk in range(blocks):
        assert np.array_equal(out[blk], want), f"mode {mode}, workgroup {blk}"
    clk = r["clocks"].cpu().numpy()
    assert np.all(clk > 0) and r["wall_clock_hz"] > 0
