"""Pins for the oracle's Gaussian basis (CPU only).

The refreshed Gaussian projection is the variant the LoGRA paper compares
with the Rademacher one (section 3.4.1, Figure 5c).  What ties the oracle's
generator to something other than itself:
  * its bits come from numpy's independent Philox4x64-10 for counter
    (j // 8, i, 1, 0): inverting each Box-Muller pair with hypot and atan2
    recovers -2 ln u1 and 2 pi u2 computed from numpy's raw words;
  * the values are N(0, 1) (Kolmogorov-Smirnov against scipy's normal CDF,
    moments), pairs uncorrelated, and independent of the sign stream;
  * E[A^T A] = I, the exact error rate E||S A - G||^2 = ((k + 1) / r) ||G||^2
    of a Gaussian basis, and the closed-form reconstruction cosine
    sqrt(r / (r + k + 1)) for isotropic gradients, slightly below the
    Rademacher value sqrt(r / (r + k - 1)) as the paper's Figure 5c finds.
"""

import math

import numpy as np
import pytest
from scipy import stats

from oracle import (
    MASK64,
    gaussian_normals,
    gaussian_projection,
    rademacher_projection,
    reconstruction_cosine,
    sign_matrix,
)


def _numpy_block(ctr, key):
    # numpy's generator advances its counter before producing a block.
    c = sum(int(w) << (64 * i) for i, w in enumerate(ctr))
    c = (c - 1) % (1 << 256)
    start = [(c >> (64 * i)) & MASK64 for i in range(4)]
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(start, dtype=np.uint64))
    return [int(v) for v in g.random_raw(4)]


@pytest.mark.parametrize("seed,i,b", [(0, 0, 0), (7, 3, 5), (2**63 + 1, 255, 1000), (123456789, 511, 2175)])
def test_box_muller_pairs_invert_to_numpy_bits(seed, i, b):
    z = gaussian_normals(seed, i + 1, 8 * (b + 1))[i, 8 * b: 8 * b + 8]
    words = _numpy_block((b, i, 1, 0), (seed & MASK64, 0))
    halves = []
    for w in words:
        halves += [w & 0xFFFFFFFF, w >> 32]
    for p in range(4):
        u1 = ((halves[2 * p] >> 8) + 1) / 2.0**24
        u2 = (halves[2 * p + 1] >> 8) / 2.0**24
        zc, zs = z[2 * p], z[2 * p + 1]
        assert zc * zc + zs * zs == pytest.approx(-2.0 * math.log(u1), rel=1e-12, abs=1e-15)
        if zc * zc + zs * zs > 1e-20:
            gap = abs(math.atan2(zs, zc) % (2.0 * math.pi) - 2.0 * math.pi * u2)
            assert min(gap, 2.0 * math.pi - gap) < 1e-9


def test_values_are_standard_normal():
    z = gaussian_normals(11, 64, 8192).ravel()
    n = z.size
    assert abs(z.mean()) < 5.0 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5.0 * math.sqrt(2.0 / n)
    assert abs((z**4).mean() - 3.0) < 5.0 * math.sqrt(96.0 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # the two members of a pair are uncorrelated; neighbours across pairs too
    zz = gaussian_normals(12, 32, 4096)
    for a, b in ((0, 1), (1, 2), (0, 7)):
        c = np.corrcoef(zz[:, a::8].ravel(), zz[:, b::8].ravel())[0, 1]
        assert abs(c) < 5.0 / math.sqrt(zz[:, a::8].size)


def test_independent_of_sign_stream_and_prefix_stable():
    z = gaussian_normals(5, 16, 4096)
    s = sign_matrix(5, 16, 4096).astype(np.float64)
    c = np.corrcoef(z.ravel(), s.ravel())[0, 1]
    assert abs(c) < 5.0 / math.sqrt(z.size)
    # entry (i, j) does not depend on r or k
    np.testing.assert_array_equal(gaussian_normals(5, 7, 1000), z[:7, :1000])


def test_expected_gram_is_identity():
    r, k, N = 16, 24, 4000
    M = np.zeros((k, k))
    for n in range(N):
        A = gaussian_projection(1000 + n, r, k)
        M += A.T @ A
    M /= N
    # diag: mean 1, variance 2/r per draw; off-diagonal: mean 0, variance 1/r
    assert np.abs(np.diag(M) - 1.0).max() < 6.0 * math.sqrt(2.0 / r / N)
    off = M[~np.eye(k, dtype=bool)]
    assert np.abs(off).max() < 6.0 * math.sqrt(1.0 / r / N)


def test_exact_error_rate_and_cosine():
    # For a fixed G: E||S A - G||^2 = ((k + 1) / r) ||G||^2 with S = G A^T
    # (Gaussian A); the Rademacher rate is (k - 1) / r.
    rng = np.random.default_rng(4)
    d, k, r, N = 6, 40, 8, 3000
    G = rng.standard_normal((d, k))
    g2 = float((G * G).sum())
    err = 0.0
    for n in range(N):
        A = gaussian_projection(7000 + n, r, k)
        D = (G @ A.T) @ A - G
        err += float((D * D).sum())
    rate = err / N / g2
    assert rate == pytest.approx((k + 1) / r, rel=0.08)
    assert abs(rate - (k - 1) / r) > abs(rate - (k + 1) / r)
    # Reconstruction cosine for isotropic gradients (G = dY^T X, iid data).
    T, d, k, r = 4096, 64, 1024, 64
    X = rng.standard_normal((T, k))
    dY = rng.standard_normal((T, d))
    G = dY.T @ X
    cg = np.mean([reconstruction_cosine(G, gaussian_projection(50 + n, r, k)) for n in range(4)])
    cr = np.mean([reconstruction_cosine(G, rademacher_projection(50 + n, r, k)) for n in range(4)])
    assert cg == pytest.approx(math.sqrt(r / (r + k + 1)), rel=0.05)
    assert cr == pytest.approx(math.sqrt(r / (r + k - 1)), rel=0.05)
