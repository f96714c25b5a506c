"""Pins for the oracle's merge and RowAdam (CPU only).

Merge (LoGRA section 2.1, equations 3-4): special cases with known results,
hand-worked examples, rank and linearity.  RowAdam (appendix B, equation 15):
hand-worked values, the bias-correction invariant, norm preservation, the
zero-sketch rule and scale homogeneity.
"""

import math

import numpy as np
import pytest

from oracle import (
    low_rank_expand,
    merge_update,
    rademacher_projection,
    round_to_bf16,
    rowadam_scale,
)


def _bf16_matrix(rng, shape, std):
    return round_to_bf16(rng.standard_normal(shape) * std)


def test_merge_zero_scale_or_zero_sketch_is_identity():
    rng = np.random.default_rng(0)
    W = _bf16_matrix(rng, (8, 300), 0.02)
    U = rng.standard_normal((8, 16))
    A = rademacher_projection(0, 16, 300)
    np.testing.assert_array_equal(merge_update(W, U, A, 0.0), W)
    np.testing.assert_array_equal(merge_update(W, np.zeros_like(U), A, 1e-3), W)


def test_merge_zero_weight_isolates_update():
    rng = np.random.default_rng(1)
    U = rng.standard_normal((5, 4))
    A = rademacher_projection(1, 4, 33)
    out = merge_update(np.zeros((5, 33)), U, A, 0.5)
    np.testing.assert_array_equal(out, round_to_bf16(-0.5 * (U @ A)))


def test_merge_hand_worked():
    # r = k = d = 1: A = [[+-1]]; W' = RNE(W - c*U*A)
    A = rademacher_projection(0, 1, 1)
    a = A[0, 0]
    assert abs(a) == 1.0
    out = merge_update(np.array([[1.0]]), np.array([[2.0]]), A, 0.25)
    assert out[0, 0] == 1.0 - 0.5 * a
    # a tie: 1 + 2**-8 lies halfway between bf16 neighbours 1 and 1 + 2**-7
    out = merge_update(np.array([[1.0]]), np.array([[-(2.0**-8) * a]]), A, 1.0)
    assert out[0, 0] == 1.0
    out = merge_update(np.array([[1.0]]), np.array([[-(3 * 2.0**-8) * a]]), A, 1.0)
    assert out[0, 0] == 1.0 + 2.0**-6  # 1 + 3*2^-8 = tie between 1+2^-7 and 1+2^-6 -> even


def test_merge_loops_and_rank():
    rng = np.random.default_rng(2)
    d, k, r = 4, 9, 3
    W = _bf16_matrix(rng, (d, k), 1.0)
    U = rng.standard_normal((d, r))
    A = rademacher_projection(5, r, k)
    c = 0.125
    ref = np.empty((d, k))
    for i in range(d):
        for j in range(k):
            ref[i, j] = W[i, j] - c * sum(U[i, l] * A[l, j] for l in range(r))
    np.testing.assert_array_equal(merge_update(W, U, A, c), round_to_bf16(ref))
    dW = low_rank_expand(U, A)
    assert np.linalg.matrix_rank(dW) <= r
    np.testing.assert_allclose(low_rank_expand(2.5 * U, A), 2.5 * dW, rtol=1e-13, atol=1e-15)


def test_rowadam_hand_worked_first_step():
    """t = 1: vhat = mean-square of each row; each row is divided by its RMS
    (plus a 1e-8-relative epsilon), then the whole matrix is rescaled to the
    sketch's Frobenius norm."""
    S = np.array([[3.0, 4.0], [0.6, 0.8]])
    U, v = rowadam_scale(S, np.zeros(2), step=1, beta2=0.95)
    np.testing.assert_allclose(v, 0.05 * np.array([12.5, 0.5]), rtol=1e-15)
    rms = np.array([math.sqrt(12.5), math.sqrt(0.5)])
    eps = 1e-8 * rms.mean()
    Ut = S / (rms + eps)[:, None]
    expect = Ut * (math.sqrt(26.0) / math.sqrt(float((Ut**2).sum())))
    np.testing.assert_allclose(U, expect, rtol=1e-14)
    # both rows end with the same RMS: sqrt(26 / 4) up to the epsilon
    np.testing.assert_allclose(np.sqrt((U**2).mean(axis=1)), math.sqrt(26 / 4), rtol=1e-7)


def test_rowadam_hand_worked_second_step():
    beta2 = 0.95
    S1 = np.array([[2.0, 0.0]])  # ms = 2
    S2 = np.array([[0.0, 4.0]])  # ms = 8
    _, v1 = rowadam_scale(S1, np.zeros(1), 1, beta2)
    U2, v2 = rowadam_scale(S2, v1, 2, beta2)
    v_expect = beta2 * (1 - beta2) * 2 + (1 - beta2) * 8
    assert math.isclose(float(v2[0]), v_expect, rel_tol=1e-14)
    # one row: the rescale restores ||S2|| regardless of vhat
    np.testing.assert_allclose(U2, S2, rtol=1e-14)
    S3 = np.array([[0.0, 4.0], [1.0, 1.0]])
    U3, _ = rowadam_scale(S3, np.array([v2[0], 0.0]), 2, beta2)
    vhat = np.array([(beta2 * v2[0] + (1 - beta2) * 8) / (1 - beta2**2), (1 - beta2) * 1.0 / (1 - beta2**2)])
    root = np.sqrt(vhat)
    Ut = S3 / (root + 1e-8 * root.mean())[:, None]
    np.testing.assert_allclose(U3, Ut * math.sqrt(18.0) / np.linalg.norm(Ut), rtol=1e-13)


def test_rowadam_bias_correction_invariant():
    """Feeding the same sketch every step gives vhat_t = mean-square exactly,
    for every t, because v_t = (1 - beta2^t) ms (the correction undoes the
    zero initialisation)."""
    rng = np.random.default_rng(3)
    S = rng.standard_normal((7, 16))
    ms = (S**2).mean(axis=1)
    v = np.zeros(7)
    U1 = None
    for t in range(1, 6):
        U, v = rowadam_scale(S, v, t, 0.999)
        np.testing.assert_allclose(v / (1 - 0.999**t), ms, rtol=1e-10)
        if U1 is None:
            U1 = U
        np.testing.assert_allclose(U, U1, rtol=1e-9)


@pytest.mark.parametrize("beta2", [0.95, 0.999])
def test_rowadam_norm_preserved_and_zero(beta2):
    rng = np.random.default_rng(4)
    S = rng.standard_normal((50, 32)) * rng.uniform(0.01, 100, size=(50, 1))
    U, _ = rowadam_scale(S, np.zeros(50), 1, beta2)
    assert math.isclose(np.linalg.norm(U), np.linalg.norm(S), rel_tol=1e-12)
    Z, vz = rowadam_scale(np.zeros((50, 32)), np.zeros(50), 1, beta2)
    assert not Z.any() and not vz.any()


def test_rowadam_equal_rows_is_identity_and_homogeneous():
    rng = np.random.default_rng(5)
    base = rng.standard_normal((1, 8))
    signs = np.array([[1.0], [-1.0], [1.0]])
    S = signs * base  # all rows have the same mean-square
    U, _ = rowadam_scale(S, np.zeros(3), 1, 0.95)
    np.testing.assert_allclose(U, S, rtol=1e-12)
    S = rng.standard_normal((6, 8))
    v = rng.uniform(0.1, 2.0, size=6)
    lam = 37.0
    U1, v1 = rowadam_scale(S, v, 3, 0.95)
    U2, v2 = rowadam_scale(lam * S, lam**2 * v, 3, 0.95)
    np.testing.assert_allclose(U2, lam * U1, rtol=1e-12)
    np.testing.assert_allclose(v2, lam**2 * v1, rtol=1e-12)


def test_rowadam_rejects_step_zero():
    with pytest.raises(ValueError):
        rowadam_scale(np.ones((2, 2)), np.zeros(2), 0, 0.95)
