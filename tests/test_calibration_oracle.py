"""Pins of the calibration statistics (CPU): the per-column absolute maximum
by brute force on a small case, the running maximum over batches equals the
maximum over their concatenation, and lambda from the maxima equals the
one-shot calibration."""
import numpy as np

import oracle as O


def _bits(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_column_absmax_brute_force():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((7, 5)) * 3).astype(np.float32)
    x[:, 2] = 0.0
    x[3, 4] = -1e30
    xb = _bits(x)
    got = O.column_absmax(xb)
    xf = O.bf16_to_f32(xb)
    for j in range(5):
        m = 0.0
        for i in range(7):
            m = max(m, abs(float(xf[i, j])))
        assert got[j] == np.float32(m)
    assert got[2] == 0.0


def test_running_max_over_batches():
    rng = np.random.default_rng(1)
    batches = [_bits(rng.standard_normal((n, 64)) * np.exp(rng.uniform(-4, 4, 64))) for n in (5, 1, 12)]
    run = None
    for b in batches:
        run = O.column_absmax(b, run)
    assert np.array_equal(run, O.column_absmax(np.concatenate(batches)))


def test_lambda_from_absmax_is_the_calibration():
    rng = np.random.default_rng(2)
    X = _bits(rng.standard_normal((9, 128)) * np.exp(rng.uniform(-5, 5, 128)))
    W = _bits(rng.standard_normal((11, 128)) * 0.02)
    X[:, 3] = 0
    lam = O.lambda_from_absmax(O.column_absmax(X[:4], O.column_absmax(X[4:])), O.column_absmax(W))
    assert np.array_equal(lam.view(np.uint32), O.calibrate_lambda(X, W).view(np.uint32))
    assert lam[3] == 1.0
