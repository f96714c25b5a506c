"""Pins for the oracle's sign generator (CPU only).

The oracle's Philox4x64-10 is written from the published definition
(Salmon et al., SC'11).  numpy ships an independent implementation of the same
generator (numpy.random.Philox), so the oracle is checked bit for bit against
it.  numpy's bit generator advances its 256-bit counter before producing a
block, so the block for counter c comes from numpy started at c - 1.
"""

import math

import numpy as np
import pytest

from oracle import MASK64, philox4x64_10, rademacher_projection, sign_bits, sign_matrix


def _numpy_block(ctr, key):
    c = sum(int(w) << (64 * i) for i, w in enumerate(ctr))
    c = (c - 1) % (1 << 256)
    start = [(c >> (64 * i)) & MASK64 for i in range(4)]
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(start, dtype=np.uint64))
    return [int(v) for v in g.random_raw(4)]


@pytest.mark.parametrize(
    "ctr,key",
    [
        ((0, 0, 0, 0), (0, 0)),
        ((1, 0, 0, 0), (0, 0)),
        ((0, 1, 0, 0), (7, 0)),
        ((MASK64, MASK64, MASK64, MASK64), (MASK64, MASK64)),
        ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
         (0x452821E638D01377, 0xBE5466CF34E90C6C)),
        ((12345, 678, 9, 10), (0xDEADBEEFCAFEF00D, 42)),
    ],
)
def test_philox_matches_numpy(ctr, key):
    assert list(philox4x64_10(ctr, key)) == _numpy_block(ctr, key)


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(0)
    vals = [[int(x) for x in rng.integers(0, 2**63, size=6, dtype=np.int64)] for _ in range(4)]
    arrs = []
    for w in range(4):
        a = np.empty(6, dtype=object)
        a[:] = vals[w]
        arrs.append(a)
    out = philox4x64_10(tuple(arrs), (99, 3))
    for j in range(6):
        ref = philox4x64_10(tuple(vals[w][j] for w in range(4)), (99, 3))
        assert [int(out[w][j]) for w in range(4)] == list(ref)


@pytest.mark.parametrize("seed,r,k", [(0, 16, 512), (1, 3, 700), (2**63 + 5, 5, 257), (42, 64, 1536)])
def test_sign_bits_block_layout_vs_numpy(seed, r, k):
    """Every 256-column block of every sign row equals numpy's Philox block for
    counter (c, i, 0, 0) and key (seed, 0), unpacked LSB first from word 0."""
    b = sign_bits(seed, r, k)
    assert b.shape == (r, k) and b.dtype == np.uint8
    for i in range(r):
        for c in range((k + 255) // 256):
            words = _numpy_block((c, i, 0, 0), (seed & MASK64, 0))
            raw = np.array(words, dtype="<u8").view(np.uint8)
            ref = np.unpackbits(raw, bitorder="little")
            lo, hi = 256 * c, min(k, 256 * (c + 1))
            np.testing.assert_array_equal(b[i, lo:hi], ref[: hi - lo])


def test_sign_prefix_properties():
    """Signs of row i, column j do not depend on r or k (a caller may slice)."""
    big = sign_bits(11, 9, 1000)
    np.testing.assert_array_equal(sign_bits(11, 4, 300), big[:4, :300])
    np.testing.assert_array_equal(sign_bits(11, 9, 1), big[:, :1])


def test_rademacher_scale_and_diag():
    """Entries are +-1/sqrt(r); diag(A^T A) = 1 exactly (LoGRA section 2.1)."""
    r, k = 16, 2048
    A = rademacher_projection(3, r, k)
    assert np.all(np.abs(np.abs(A) - 1 / math.sqrt(r)) < 1e-15)
    np.testing.assert_allclose(np.diag(A.T @ A), 1.0, rtol=0, atol=1e-12)


def test_sign_balance_and_seed_independence():
    r, k = 64, 4096
    s0 = sign_matrix(0, r, k).astype(np.int64)
    n = r * k
    assert abs(int(s0.sum())) <= 4 * math.sqrt(n)  # +-1 balanced
    s1 = sign_matrix(1, r, k).astype(np.int64)
    agree = int((s0 == s1).sum())
    assert abs(agree - n / 2) <= 4 * math.sqrt(n) / 2  # seeds independent
    # off-diagonal entries of A^T A have mean 0 and variance 1/r (iid signs)
    A = s0[:, :512].astype(np.float64) / math.sqrt(r)
    M = A.T @ A
    off = M[~np.eye(512, dtype=bool)]
    assert abs(off.mean()) < 5 * math.sqrt(1 / r) / math.sqrt(off.size / 2)
    assert abs(off.var() * r - 1.0) < 0.05


def test_sign_edge_shapes():
    assert sign_bits(5, 0, 10).shape == (0, 10)
    assert sign_bits(5, 3, 0).shape == (3, 0)
    with pytest.raises(ValueError):
        sign_bits(5, -1, 3)
