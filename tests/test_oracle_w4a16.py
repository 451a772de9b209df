"""Pins of the oracle's W4A16 consumer check (oracle.w4a16_matmul): the dequantization it applies
to the packed tensors is fixed by the GPTQ-v1 layout, so products with one-hot activations read
single weights back, and a hand example fixes the scale per (group, output) and the zero point 8."""
import numpy as np

import oracle
import workloads as W


def _pack(codes, sbits):
    out, inp = codes.shape
    return oracle.pack_gptq_v1(codes, sbits, out, inp)


def test_one_hot_activations_read_back_each_weight():
    rng = np.random.default_rng(1)
    out, inp = 24, 256
    codes = rng.integers(-8, 8, (out, inp)).astype(np.int8)
    sv = rng.uniform(0.001, 0.1, (out, inp // 128)).astype(np.float16)
    qw, sc = _pack(codes, sv.view(np.uint16))
    ks = [0, 1, 127, 128, 200, 255]
    x = np.zeros((len(ks), inp), np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y, _ = oracle.w4a16_matmul(W.f32_to_bf16_bits(x), qw, sc)
    for r, k in enumerate(ks):
        want = codes[:, k].astype(np.float64) * sv[:, k // 128].astype(np.float64)
        assert np.array_equal(y[r], want)


def test_hand_example():
    """One output row, two groups: codes -8 and 7 at channel 0 and 128, scales 0.5 and 2."""
    codes = np.zeros((1, 256), np.int8)
    codes[0, 0], codes[0, 128], codes[0, 129] = -8, 7, 1
    sv = np.array([[0.5, 2.0]], np.float16)
    qw, sc = _pack(codes, sv.view(np.uint16))
    assert qw[0, 0] == 0x88888880 - (1 << 32)      # nibble 0 = -8 + 8 = 0, the rest 8 (zero)
    x = np.zeros((1, 256), np.float32)
    x[0, 0], x[0, 128], x[0, 129] = 3.0, -1.0, 0.25
    y, bound = oracle.w4a16_matmul(W.f32_to_bf16_bits(x), qw, sc)
    assert y[0, 0] == 3.0 * (-8 * 0.5) + (-1.0) * (7 * 2.0) + 0.25 * (1 * 2.0)   # -12 - 14 + 0.5
    assert bound[0, 0] == 12.0 + 14.0 + 0.5


def test_linearity_in_x():
    rng = np.random.default_rng(2)
    codes = rng.integers(-8, 8, (16, 128)).astype(np.int8)
    sv = np.full((16, 1), 0.25, np.float16)
    qw, sc = _pack(codes, sv.view(np.uint16))
    x1 = rng.integers(-4, 5, (3, 128)).astype(np.float32)
    x2 = rng.integers(-4, 5, (3, 128)).astype(np.float32)
    y1, _ = oracle.w4a16_matmul(W.f32_to_bf16_bits(x1), qw, sc)
    y2, _ = oracle.w4a16_matmul(W.f32_to_bf16_bits(x2), qw, sc)
    y12, _ = oracle.w4a16_matmul(W.f32_to_bf16_bits(x1 + x2), qw, sc)
    assert np.array_equal(y1 + y2, y12)             # small integers times 0.25: every sum exact
    assert np.array_equal(y1, (x1.astype(np.float64) @ (codes.astype(np.float64) * 0.25).T))
