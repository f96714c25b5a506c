"""Pins for the oracle's sketch (CPU only).

What ties the oracle to the pages and to mathematics rather than to itself:
  * equation 2 evaluated with explicit loops on tiny inputs;
  * additivity over microbatches (Algorithm 1 sums microbatch contributions);
  * <G, S A> = ||S||_F^2 for every realisation of A;
  * unbiasedness E_A[S A] = G with the exact error rate ((k-1)/r) ||G||^2;
  * rank(S A) <= r (section 2.1);
  * the reconstruction cosine for isotropic gradients, which reproduces the
    values the paper prints for the 1.5B model (section 3.4.1);
  * the accumulator-size arithmetic the paper prints (section 2.2);
  * the projection-first path dY^T (X A^T) (section 2.1, after equation 2)
    equals the dense-gradient path, and projecting a unit row returns the
    matching column of A;
  * the variant with P rounded once to bf16 equals the exact sketch when P is
    exact in bf16, follows explicit loops over a pinned rounding, and drops
    exactly the part of P below half a bf16 spacing.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import (
    dense_gradient,
    low_rank_expand,
    project_inputs,
    rademacher_projection,
    reconstruction_cosine,
    round_to_bf16,
    sign_matrix,
    sketch_accumulate,
    sketch_accumulate_rounded_projection,
    sketch_from_gradient,
    sketch_projected_first,
)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def _tiny(seed, M, T, d, k):
    rng = np.random.default_rng(seed)
    Xs = [rng.standard_normal((T, k)) for _ in range(M)]
    dYs = [rng.standard_normal((T, d)) for _ in range(M)]
    return Xs, dYs


def test_equation2_brute_force_loops():
    M, T, d, k, r = 2, 5, 3, 7, 4
    Xs, dYs = _tiny(0, M, T, d, k)
    A = rademacher_projection(9, r, k)
    S0 = np.random.default_rng(1).standard_normal((d, r))
    S = sketch_accumulate(S0, Xs, dYs, A)
    ref = np.array(S0, copy=True)
    for i in range(d):
        for l in range(r):
            acc = 0.0
            for j in range(k):
                g = 0.0
                for m in range(M):
                    for t in range(T):
                        g += dYs[m][t, i] * Xs[m][t, j]
                acc += g * A[l, j]
            ref[i, l] += acc
    np.testing.assert_allclose(S, ref, rtol=1e-12, atol=1e-12)
    assert S.shape == (d, r)


def test_additivity_over_microbatches():
    Xs, dYs = _tiny(2, 4, 16, 6, 40)
    A = rademacher_projection(4, 8, 40)
    S0 = np.zeros((6, 8))
    split = sketch_accumulate(S0, Xs, dYs, A)
    whole = sketch_accumulate(S0, [np.concatenate(Xs)], [np.concatenate(dYs)], A)
    np.testing.assert_allclose(split, whole, rtol=1e-12, atol=1e-12)
    # one call per microbatch, each starting from the previous S, is the same
    S = S0
    for X, dY in zip(Xs, dYs):
        S = sketch_accumulate(S, [X], [dY], A)
    np.testing.assert_allclose(S, whole, rtol=1e-12, atol=1e-12)


def test_row_subset_matches_full():
    Xs, dYs = _tiny(3, 2, 10, 9, 30)
    A = rademacher_projection(1, 4, 30)
    S0 = np.random.default_rng(0).standard_normal((9, 4))
    full = sketch_accumulate(S0, Xs, dYs, A)
    rows = [0, 4, 8]
    np.testing.assert_allclose(sketch_accumulate(S0, Xs, dYs, A, rows=rows), full[rows], rtol=1e-13)


def test_inner_product_identity():
    """<G, S A> = tr(G A^T A G^T) = ||G A^T||^2 = ||S||^2 for every A."""
    rng = np.random.default_rng(5)
    G = rng.standard_normal((20, 300))
    for seed in range(3):
        A = rademacher_projection(seed, 12, 300)
        S = sketch_from_gradient(G, A)
        lhs = float((G * low_rank_expand(S, A)).sum())
        assert math.isclose(lhs, float((S * S).sum()), rel_tol=1e-12)


def test_unbiased_with_exact_rate():
    """E_A[S A] = G and E||S A - G||^2 = ((k-1)/r) ||G||^2 for iid +-1/sqrt(r)
    entries (E[A^T A] = I and E[(A^T A)^2] = (1 + (k-1)/r) I)."""
    rng = np.random.default_rng(6)
    d, k, r = 4, 64, 8
    G = rng.standard_normal((d, k))
    g2 = float((G * G).sum())
    N = 3000
    mean = np.zeros_like(G)
    sq_err = 0.0
    for seed in range(N):
        A = rademacher_projection(1000 + seed, r, k)
        Gh = low_rank_expand(sketch_from_gradient(G, A), A)
        mean += Gh
        sq_err += float(((Gh - G) ** 2).sum())
    mean /= N
    rate = (k - 1) / r
    assert abs(sq_err / N / g2 - rate) < 0.08 * rate
    rel = math.sqrt(float(((mean - G) ** 2).sum()) / g2)
    expect = math.sqrt(rate / N)
    assert 0.8 * expect < rel < 1.2 * expect


def test_rank_at_most_r():
    rng = np.random.default_rng(7)
    G = rng.standard_normal((40, 90))
    r = 6
    A = rademacher_projection(2, r, 90)
    sv = np.linalg.svd(low_rank_expand(sketch_from_gradient(G, A), A), compute_uv=False)
    assert sv[r] / sv[0] < 1e-12
    assert sv[r - 1] / sv[0] > 1e-6


def test_reconstruction_cosine_matches_printed_values():
    """For a gradient isotropic in its input dimension the reconstruction
    cosine is sqrt(r / (r + k - 1)).  Averaged over the seven matrices of a
    1.5B-class layer this reproduces the printed 0.046 (r=4) and 0.348
    (r=256).  The oracle's own measured cosine must agree with both."""
    g = GOLDEN["reconstruction_cosine"]
    widths = list(g["layer_input_widths"].values())
    for r, printed in ((4, g["r4"]), (256, g["r256"])):
        closed = float(np.mean([math.sqrt(r / (r + k - 1)) for k in widths]))
        assert abs(closed - printed) < 0.002, (r, closed, printed)
        rng = np.random.default_rng(r)
        measured = []
        for k in sorted(set(widths)):
            vals = []
            for seed in range(3):
                T = 512
                G = dense_gradient([rng.standard_normal((T, k))], [rng.standard_normal((T, 96))])
                vals.append(reconstruction_cosine(G, rademacher_projection(seed, r, k)))
            measured.append((k, float(np.mean(vals))))
        per_k = dict(measured)
        avg = float(np.mean([per_k[k] for k in widths]))
        assert abs(avg - printed) < 0.06 * printed, (r, avg, printed)


def test_accumulator_size_printed():
    """d = k = 4096, r = 64: a dense fp32 accumulator is 64 MiB, the sketch
    1 MiB (section 2.2)."""
    g = GOLDEN["accumulator_size"]
    d, k, r = g["d"], g["k"], g["r"]
    G = np.zeros((d, 8))  # only the shapes matter; keep memory small
    S = sketch_from_gradient(G, np.zeros((r, 8)))
    assert S.shape == (d, r)
    assert d * k * 4 == g["dense_fp32_MiB"] * 2**20
    assert S.astype(np.float32).nbytes == g["sketch_fp32_MiB"] * 2**20


@pytest.mark.parametrize("shape", [(0, 5, 7), (3, 0, 7), (3, 5, 0)])
def test_empty_inputs(shape):
    T, d, k = shape
    A = rademacher_projection(0, 4, k)
    S0 = np.ones((d, 4))
    S = sketch_accumulate(S0, [np.zeros((T, k))], [np.zeros((T, d))], A)
    np.testing.assert_array_equal(S, S0)


def test_projection_first_equals_gradient_path():
    # Projecting the inputs first and contracting with dY gives exactly the
    # sketch of the dense gradient (associativity), microbatch by microbatch.
    M, T, d, k, r = 3, 37, 11, 70, 16
    Xs, dYs = _tiny(5, M, T, d, k)
    A = rademacher_projection(3, r, k)
    S = sum(dY.T @ project_inputs(X, A) for X, dY in zip(Xs, dYs))
    ref = sketch_accumulate(np.zeros((d, r)), Xs, dYs, A)
    np.testing.assert_allclose(S, ref, rtol=1e-12, atol=1e-10)


def test_projection_of_unit_rows_is_columns_of_A():
    # Row t of X equal to the unit vector e_j projects to column j of A; a
    # zero row projects to zero; the projection is linear in X.
    k, r = 300, 8
    A = rademacher_projection(11, r, k)
    cols = [0, 1, 255, 256, 299]
    X = np.zeros((len(cols) + 1, k))
    for t, j in enumerate(cols):
        X[t, j] = 1.0
    P = project_inputs(X, A)
    for t, j in enumerate(cols):
        np.testing.assert_array_equal(P[t], A[:, j])
    np.testing.assert_array_equal(P[-1], np.zeros(r))
    Y = np.random.default_rng(0).standard_normal((4, k))
    np.testing.assert_allclose(project_inputs(2.0 * Y - X[:4], A), 2.0 * project_inputs(Y, A) - P[:4], atol=1e-12)
    # every entry of A has magnitude 1/sqrt(r), so |P[t, c]| <= sum_j |X[t, j]| / sqrt(r)
    assert np.all(np.abs(project_inputs(Y, A)) <= np.abs(Y).sum(axis=1, keepdims=True) / math.sqrt(r) + 1e-12)


def test_projected_first_oracle_matches_definition():
    # sketch_projected_first (never forms G) against the dense-gradient
    # definition, with an incoming S0 and a row subset, and against explicit
    # loops of equation 2 on a tiny case.
    M, T, d, k, r = 3, 41, 13, 300, 24
    Xs, dYs = _tiny(17, M, T, d, k)
    A = rademacher_projection(9, r, k)
    S0 = np.random.default_rng(3).standard_normal((d, r))
    np.testing.assert_allclose(sketch_projected_first(S0, Xs, dYs, A), sketch_accumulate(S0, Xs, dYs, A),
                               rtol=1e-12, atol=1e-10)
    rows = np.array([0, 5, 12])
    np.testing.assert_allclose(sketch_projected_first(S0, Xs, dYs, A, rows=rows),
                               sketch_accumulate(S0, Xs, dYs, A)[rows], rtol=1e-12, atol=1e-10)
    Xs, dYs = _tiny(4, 2, 5, 3, 7)
    A = rademacher_projection(2, 4, 7)
    want = np.zeros((3, 4))
    for X, dY in zip(Xs, dYs):
        for i in range(3):
            for c in range(4):
                want[i, c] += sum(dY[t, i] * X[t, j] * A[c, j] for t in range(5) for j in range(7))
    np.testing.assert_allclose(sketch_projected_first(np.zeros((3, 4)), Xs, dYs, A), want, rtol=1e-12, atol=1e-12)


def test_rounded_projection_exact_when_p_is_bf16():
    # X in {-1, 0, 1} and k <= 256: every entry of X s^T is an integer of
    # magnitude <= 256, exact in bf16, so rounding changes nothing.
    rng = np.random.default_rng(8)
    T, d, k, r, seed = 33, 9, 200, 16, 5
    Xs = [rng.integers(-1, 2, size=(T, k)).astype(np.float64) for _ in range(2)]
    dYs = [rng.standard_normal((T, d)) for _ in range(2)]
    S0 = rng.standard_normal((d, r))
    np.testing.assert_allclose(sketch_accumulate_rounded_projection(S0, Xs, dYs, seed, r),
                               sketch_accumulate(S0, Xs, dYs, rademacher_projection(seed, r, k)),
                               rtol=1e-12, atol=1e-12)


def test_rounded_projection_follows_loops_over_pinned_rounding():
    # Explicit loops: P[t, c] = sum_j X[t, j] s[c, j], rounded element by
    # element with round_to_bf16 (itself pinned against torch), then
    # S[i, c] = S0[i, c] + sum_t dY[t, i] P[t, c] / sqrt(r).
    rng = np.random.default_rng(12)
    T, d, k, r, seed = 6, 4, 9, 5, 77
    X = rng.standard_normal((T, k))
    dY = rng.standard_normal((T, d))
    S0 = rng.standard_normal((d, r))
    s = sign_matrix(seed, r, k).astype(np.float64)
    P = np.zeros((T, r))
    for t in range(T):
        for c in range(r):
            P[t, c] = float(round_to_bf16(np.array([sum(X[t, j] * s[c, j] for j in range(k))]))[0])
    want = S0.copy()
    for i in range(d):
        for c in range(r):
            want[i, c] += sum(dY[t, i] * P[t, c] for t in range(T)) / math.sqrt(r)
    got = sketch_accumulate_rounded_projection(S0, [X], [dY], seed, r)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
    # Row subset.
    np.testing.assert_allclose(sketch_accumulate_rounded_projection(S0, [X], [dY], seed, r, rows=np.array([1, 3])),
                               want[[1, 3]], rtol=1e-13, atol=1e-13)


def test_rounded_projection_drops_below_half_spacing():
    # X = [1, 2^-9]: P[c] = s[c,0] + s[c,1] 2^-9 is within half a bf16 spacing
    # of s[c,0] (above 1 the spacing is 2^-7; below 1 it is 2^-8 and
    # 1 - 2^-9 is a tie that goes to the even neighbour, 1), so the rounded
    # P is exactly s[:, 0] and S = s[:, 0] / sqrt(r) for dY = 1.
    r, seed = 16, 3
    X = np.array([[1.0, 2.0**-9]])
    dY = np.array([[1.0]])
    s = sign_matrix(seed, r, 2).astype(np.float64)
    got = sketch_accumulate_rounded_projection(np.zeros((1, r)), [X], [dY], seed, r)
    np.testing.assert_array_equal(got[0], s[:, 0] / math.sqrt(r))
    exact = sketch_accumulate(np.zeros((1, r)), [X], [dY], rademacher_projection(seed, r, 2))
    assert np.abs(exact[0] - got[0]).max() == pytest.approx(2.0**-9 / math.sqrt(r))
