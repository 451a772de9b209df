"""GPU parity: environment diagonals from bf16 activations (cq_environment_diagonals) against the
oracle.  Both sides sum in binary64 (in different orders) and round once to binary32, so every
value must lie within one binary32 spacing of the oracle's; NaN exactly where the oracle has it."""
import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_group_amd as cq
import workloads as W
from parity import dev, say

pytestmark = pytest.mark.gpu


def _check(x_bits):
    E, T, n = x_bits.shape
    say(f"diagonals: E={E}, T={T}, in={n}")
    d = cq.environment_diagonals(dev(x_bits.view(np.int16)))
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    want = oracle.environment_diagonals(x_bits)
    assert got.shape == want.shape == (n // 128, E, 128)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    diff = np.abs(got[~nan].astype(np.float64) - want[~nan].astype(np.float64))
    assert np.all(diff <= np.spacing(np.abs(want[~nan])).astype(np.float64)), diff.max()
    return got


@pytest.mark.parametrize("E,T,n", [(3, 5, 128), (1, 1, 128), (4, 37, 384), (32, 19, 256), (2, 1001, 1536)])
def test_small_and_ragged_shapes(E, T, n):
    rng = np.random.default_rng(E * 1000 + T)
    x = (rng.standard_normal((E, T, n)) * rng.lognormal(0, 1, n)).astype(np.float32)
    _check(W.f32_to_bf16_bits(x))


def test_silent_environment_is_nan():
    x = np.random.default_rng(2).standard_normal((3, 40, 256)).astype(np.float32)
    x[1] = 0.0
    got = _check(W.f32_to_bf16_bits(x))
    assert np.all(np.isnan(got[:, 1])) and not np.any(np.isnan(got[:, 0]))


@pytest.mark.parametrize("m", [0, 2])
def test_config1_full_size(m):
    """The bench's shapes: config 1's gate/up (in = 1024) and down (in = 3584) inputs, E = 4,
    8,192 tokens per environment (32 windows of 256 tokens)."""
    _check(W.calibration_activations(1, m, 8192))
