"""The pooled-row tolerance of the GPU parity tests (helpers.pool_error_bound) against an
emulation of float32 pooling on the CPU: tokens summed one by one in float32 (rotated first
by float32 cos/sin of their chunk position), the sum rotated by its chunk-start angle and
divided once.  On adversarial chunks (large cancelling terms, a large offset, tiny means)
the emulated error must stay within the bound, which is what lets the GPU tests use it."""
import numpy as np
import pytest

from oracle import msa_oracle as O
from tests.helpers import pool_error_bound


def _emulate(X, off, chunk, rotated, base=1e6):
    f = np.float32
    X = np.asarray(X, dtype=np.float64)
    T, H, D = X.shape
    h = D // 2
    th = np.power(float(base), -2.0 * np.arange(h) / D)
    rows = []
    for d in range(len(off) - 1):
        for t0 in range(int(off[d]), int(off[d + 1]), chunk):
            t1 = min(t0 + chunk, int(off[d + 1]))
            acc = np.zeros((H, D), dtype=f)
            for t in range(t0, t1):
                x = X[t].astype(f)
                if rotated:
                    c = np.cos((t - t0) * th).astype(f)
                    s = np.sin((t - t0) * th).astype(f)
                    lo, hi = x[:, :h], x[:, h:]
                    x = np.concatenate([(lo * c) - (hi * s), (hi * c) + (lo * s)], axis=1).astype(f)
                acc = (acc + x).astype(f)
            if rotated:
                c = np.cos((t0 - int(off[d])) * th).astype(f)
                s = np.sin((t0 - int(off[d])) * th).astype(f)
                lo, hi = acc[:, :h], acc[:, h:]
                acc = np.concatenate([(lo * c) - (hi * s), (hi * c) + (lo * s)], axis=1).astype(f)
            rows.append((acc / f(t1 - t0)).astype(f))
    return np.stack(rows).astype(np.float64)


@pytest.mark.parametrize("rotated", [False, True])
@pytest.mark.parametrize("chunk", [64, 128])
def test_bound_covers_float32_pooling(rotated, chunk):
    rng = np.random.default_rng(5 + chunk + rotated)
    lens = np.array([1, chunk - 1, chunk, 3 * chunk + 7, 2 * chunk])
    off = np.concatenate([[0], np.cumsum(lens)])
    T, H, D = int(off[-1]), 2, 32
    X = rng.standard_normal((T, H, D))
    X[:chunk] *= 1e3                                  # large terms
    X[chunk:2 * chunk] += 50.0                        # a large common offset
    big = rng.choice([-1.0, 1.0], size=(T, H, D)) * 2.0 ** rng.integers(0, 20, size=(T, H, D))
    X[2 * chunk:3 * chunk] = big[2 * chunk:3 * chunk]  # wildly mixed magnitudes
    # pairs that cancel exactly in exact arithmetic: the mean is tiny, float32 sums are not
    X[3 * chunk:3 * chunk + chunk // 2] = X[3 * chunk + chunk // 2:4 * chunk] * -1.0 + 1e-7
    X = X.astype(np.float32).astype(np.float64)      # inputs are float32 values
    mask = O.ROPE_K if rotated else 0
    exact = O.pool(X, X, X, off, chunk, 1e6, mask)[0]
    emu = _emulate(X, off, chunk, rotated)
    B = pool_error_bound(X, off, chunk, rotated)
    err = np.abs(emu - exact)
    assert np.all(err <= B), f"max err/bound {np.max(err / B):.3g}"
    # the bound is not vacuous: it is within a factor of 2^12 of the largest error seen
    assert np.max(err / B) > 2.0 ** -12
