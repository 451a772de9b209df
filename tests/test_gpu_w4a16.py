"""GPU parity: the W4A16 matmul over the GPTQ-v1 tensors (cq_w4a16_matmul) against the oracle.

Every product of a bf16 activation and a code is exact in fp32; a group's 128 products are summed
in fp32 on the matrix cores (at most 128 roundings), scaled once, and the groups added in fp32 (one
rounding each).  So |y - y_exact| <= (130 + G) 2^-24 sum_k |x_k| |W_ok|, G = in/128: the bound the
tests apply, with the oracle's exact product (binary64) and its bound sum."""
import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_group_amd as cq
import workloads as W
from parity import dev, say

pytestmark = pytest.mark.gpu


def _case(M, out, inp, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(-8, 8, (out, inp)).astype(np.int8)
    sv = rng.uniform(1e-3, 5e-2, (out, inp // 128)).astype(np.float16)
    qw, sc = oracle.pack_gptq_v1(codes, sv.view(np.uint16), out, inp)
    x = W.f32_to_bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    return x, qw, sc


def _check(x, qw, sc):
    M, inp = x.shape
    out = qw.shape[1]
    y = cq.w4a16_matmul(dev(x.view(np.int16)), dev(qw), dev(sc.view(np.int16)))
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    want, bound = oracle.w4a16_matmul(x, qw, sc)
    tol = (130 + inp // 128) * 2.0 ** -24 * bound
    err = np.abs(got - want)
    assert np.all(err <= tol), (err.max(), (err / np.maximum(tol, 1e-300)).max())
    return got


@pytest.mark.parametrize("M,out,inp", [(1, 64, 128), (17, 96, 384), (64, 64, 256), (100, 200, 1024),
                                       (130, 3584, 128)])
def test_shapes_against_oracle(M, out, inp):
    say(f"w4a16: M={M}, out={out}, in={inp}")
    _check(*_case(M, out, inp, M + out + inp))


def test_one_hot_rows_read_back_the_dequantized_weights():
    """x = rows of the identity: y row k is column k of W = s (u - 8), exactly."""
    x0, qw, sc = _case(1, 128, 256, 5)
    x = W.f32_to_bf16_bits(np.eye(256, dtype=np.float32)[:70])
    got = _check(x, qw, sc)
    codes, sbits = oracle.unpack_gptq_v1(qw, sc)
    Wd = codes.astype(np.float64) * np.repeat(sbits.view(np.float16).astype(np.float64), 128, axis=1)
    assert np.array_equal(got, Wd[:, :70].T)


def test_quantized_config1_matrix_end_to_end():
    """A config-1 matrix (gate, 3584 x 1024) quantized by the exhaustive solver and packed on the
    GPU, multiplied by 64 bf16 activation rows: against the oracle's product of the same packed
    tensors (the GPU's pack is pinned to the oracle's bit for bit elsewhere), and close to the
    unquantized product."""
    A, dmat = W.make_matrix(1, 0)
    w, d, p = W.matrix_groups(A, dmat)
    out, inp = A.shape
    r = cq.quantize_groups(dev(w), dev(d), p)
    qw, sc = cq.pack_gptq_v1(r["codes"].reshape(out, inp), r["scales"].reshape(out, inp // 128), out, inp)
    torch.cuda.synchronize()
    x = W.calibration_activations(1, 0, 16)[0]            # 16 tokens of environment 0
    got = _check(x, qw.cpu().numpy(), sc.cpu().numpy().view(np.uint16))
    ref = oracle.bf16_to_f64(x) @ A.astype(np.float64).T
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    say(f"  relative error against the unquantized product: {rel:.3f}")
    # 4-bit codes on weights with 1% eight-fold outliers: about 0.21 measured; a layout or
    # nibble-order mistake gives errors near 1 or above
    assert rel < 0.35
