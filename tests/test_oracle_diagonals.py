"""Pins of the oracle's environment diagonals (oracle.environment_diagonals) against closed forms
and invariants the definition fixes: a dropped square, a wrong axis of the mean, a missing
normalization or a transposed layout fails one of them."""
import numpy as np

import oracle
import workloads as W


def _bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_bf16_rounding_and_decoding():
    vals = np.array([1.0, -2.5, 3.140625, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9], np.float32)
    b = _bits(vals)
    assert list(b[:3]) == [0x3F80, 0xC020, 0x4049]
    assert b[3] == 0x3F80                       # a tie rounds to the even pattern
    assert b[4] == 0x3F81                       # 0.75 of a spacing above 1 rounds up
    assert list(oracle.bf16_to_f64(b[:3])) == [1.0, -2.5, 3.140625]


def test_constant_activations_give_ones():
    x = _bits(np.full((3, 5, 256), 0.75, np.float32))
    d = oracle.environment_diagonals(x)
    assert d.shape == (2, 3, 128) and np.all(d == 1.0)


def test_one_louder_channel_closed_form():
    """Channel 200 at twice the amplitude of the others: its mean square is 4 times theirs, so
    with n channels the normalized values are 4n/(n+3) and n/(n+3)."""
    n = 256
    x = np.ones((2, 4, n), np.float32)
    x[:, :, 200] = 2.0
    d = oracle.environment_diagonals(_bits(x))
    assert d[1, 0, 72] == np.float32(4 * n / (n + 3)) and d[1, 1, 72] == np.float32(4 * n / (n + 3))
    assert d[0, 0, 5] == np.float32(n / (n + 3))


def test_mean_of_squares_not_square_of_mean_and_per_environment():
    """Environment 0 alternates +1/-1 (mean 0, mean square 1) on channel 0 and is 1 elsewhere;
    environment 1 is scaled by 10 throughout: each environment is normalized on its own, so the
    two give the same diagonals."""
    x = np.ones((2, 4, 128), np.float32)
    x[0, ::2, 0] = -1.0
    x[1] *= 10.0
    d = oracle.environment_diagonals(_bits(x))
    assert np.all(d[0, 0] == 1.0) and np.all(d[0, 1] == 1.0)


def test_layout_is_group_major():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 7, 384)).astype(np.float32)
    d = oracle.environment_diagonals(_bits(x))
    xv = oracle.bf16_to_f64(_bits(x))
    m = (xv ** 2).mean(axis=1)
    ref = (m / m.mean(axis=1, keepdims=True)).astype(np.float32)
    for g in range(3):
        for e in range(3):
            assert np.array_equal(d[g, e], ref[e, 128 * g:128 * (g + 1)])
    assert abs(float(d.astype(np.float64).mean()) - 1.0) < 1e-6


def test_silent_environment_is_nan():
    x = np.ones((2, 3, 128), np.float32)
    x[1] = 0.0
    d = oracle.environment_diagonals(_bits(x))
    assert np.all(d[0, 0] == 1.0) and np.all(np.isnan(d[0, 1]))


def test_synthetic_activations_follow_the_diagonal_structure():
    x = W.calibration_activations(0, 0, 2048)
    d = oracle.environment_diagonals(x)
    E = x.shape[0]
    A, dmat = W.make_matrix(0, 0)
    _, dref, _ = W.matrix_groups(A, dmat)
    # the estimate tracks the structure it was drawn from (sampling noise ~ sqrt(2/T))
    r = d.astype(np.float64) / dref.astype(np.float64)
    assert d.shape == dref.shape and abs(np.median(r) - 1.0) < 0.05 and np.percentile(np.abs(r - 1), 90) < 0.1
