"""Pins for the oracle's predicted-KL step size (CPU only).

What ties oracle/predicted_kl.py to the pages and to mathematics:
  * equation 7's printed examples (q = 4 delta halves the update; q = delta/4
    doubles it under a large enough cap) and the cap itself;
  * two tokens: Var = p1 p2 (zdot1 - zdot2)^2 in closed form;
  * equal logits: p is uniform and Var is numpy's plain population variance;
  * the appendix's invariances: a common shift of all score rates, or of all
    logits, changes nothing; identical rates give zero (appendix A.1);
  * temperature: scaling z and T together by c divides q by c^2;
  * the exact KL of a small step along D equals alpha^2 q + O(alpha^3)
    (equations 5, 11 and 12), computed from log-softmax without the variance;
  * the budget schedule's endpoints and midpoint (equation 16) and the
    mismatch floor (equation 17), with the pages' settings.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import (
    effective_budget,
    kl_budget,
    kl_step_scale,
    policy_kl_along,
    predicted_kl,
    score_rate_variance,
    token_probabilities,
)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def _logits(seed, n, V, zs=3.0, ds=1.0):
    rng = np.random.default_rng(seed)
    return zs * rng.standard_normal((n, V)), ds * rng.standard_normal((n, V))


def test_step_scale_printed_examples():
    ex = GOLDEN["kl_step_scale_examples"]
    delta = 2e-4
    for case in ex["cases"]:
        q = case["q_over_delta"] * delta
        assert kl_step_scale(q, delta, alpha_max=10.0) == pytest.approx(case["alpha"], rel=1e-15)
    # the cap: a quarter of the budget would double the update, a cap of 1.5 stops it
    assert kl_step_scale(0.25 * delta, delta, alpha_max=1.5) == 1.5
    # no predicted change: the cap applies; an infinite prediction stops the update
    assert kl_step_scale(0.0, delta, alpha_max=3.0) == 3.0
    assert kl_step_scale(math.inf, delta, alpha_max=3.0) == 0.0
    # alpha^2 q meets the budget exactly whenever the cap does not bind
    for q in (1e-6, 3e-4, 0.7):
        a = kl_step_scale(q, delta, alpha_max=1e9)
        assert a * a * q == pytest.approx(delta, rel=1e-14)
    with pytest.raises(ValueError):
        kl_step_scale(-1.0, delta, 1.0)
    with pytest.raises(ValueError):
        kl_step_scale(float("nan"), delta, 1.0)


def test_two_token_closed_form():
    rng = np.random.default_rng(1)
    for _ in range(20):
        z = rng.standard_normal(2) * 4
        zd = rng.standard_normal(2)
        T = float(rng.uniform(0.3, 2.0))
        p1 = 1.0 / (1.0 + math.exp(-(z[0] - z[1]) / T))
        p2 = 1.0 / (1.0 + math.exp((z[0] - z[1]) / T))
        ref = p1 * p2 * (zd[0] - zd[1]) ** 2
        assert score_rate_variance(z[None], zd[None], T)[0] == pytest.approx(ref, rel=1e-12, abs=1e-300)


def test_uniform_logits_give_plain_variance():
    _, zd = _logits(2, 5, 777)
    z = np.full_like(zd, 1.25)
    np.testing.assert_allclose(score_rate_variance(z, zd, 0.8), zd.var(axis=1), rtol=1e-12)
    np.testing.assert_allclose(token_probabilities(z, 0.8), np.full_like(z, 1.0 / 777), rtol=1e-14)


def test_invariances():
    z, zd = _logits(3, 7, 1000)
    T = 0.9
    q = predicted_kl(z, zd, T)
    shift = np.random.default_rng(4).standard_normal((7, 1)) * 50
    # a common shift of every score rate in a context changes no probability
    assert predicted_kl(z, zd + shift, T) == pytest.approx(q, rel=1e-9)
    # a common shift of the logits leaves p, hence q, unchanged
    assert predicted_kl(z + shift, zd, T) == pytest.approx(q, rel=1e-12)
    # identical rates: zero curvature
    assert predicted_kl(z, np.broadcast_to(shift, z.shape), T) <= 1e-25 * float((shift**2).max())
    # temperature: (c z, c T) gives the same p, and q picks up 1/c^2
    c = 2.5
    assert predicted_kl(c * z, zd, c * T) == pytest.approx(q / c**2, rel=1e-12)
    # q is quadratic in the proposal: zdot -> lambda zdot scales q by lambda^2
    assert predicted_kl(z, 3.0 * zd, T) == pytest.approx(9.0 * q, rel=1e-12)
    # and an average over contexts
    halves = [predicted_kl(z[:3], zd[:3], T), predicted_kl(z[3:], zd[3:], T)]
    assert (3 * halves[0] + 4 * halves[1]) / 7 == pytest.approx(q, rel=1e-12)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_exact_kl_of_small_step(T):
    """Equation 5: the average KL between the current policy and the policy
    after a step alpha D is alpha^2 q(D) + O(alpha^3) (appendix A.1).  The
    remainder must shrink like alpha^3: halving alpha divides it by ~8."""
    z, zd = _logits(5, 6, 500)
    q = predicted_kl(z, zd, T)
    rem = []
    for a in (2e-3, 1e-3, 5e-4):
        kl = policy_kl_along(z, zd, T, a)
        assert kl / (a * a) == pytest.approx(q, rel=5e-2)
        rem.append(abs(kl - a * a * q))
    assert 6.0 < rem[0] / rem[1] < 10.0
    assert 6.0 < rem[1] / rem[2] < 10.0


def test_budget_schedule():
    b = GOLDEN["kl_budget_schedule"]
    H, dmax, dmin = b["H"], b["delta_max"], b["delta_min"]
    assert kl_budget(1, H, dmax, dmin) == pytest.approx(dmax, rel=1e-15)
    assert kl_budget(H, H, dmax, dmin) == pytest.approx(dmin, rel=1e-12)
    # cos(pi/2) = 0 at the midpoint of an odd-length schedule
    assert kl_budget(151, 301, dmax, dmin) == pytest.approx(0.5 * (dmax + dmin), rel=1e-12)
    vals = [kl_budget(u, H, dmax, dmin) for u in range(1, H + 1)]
    assert all(x > y for x, y in zip(vals, vals[1:]))
    # held at the floor after the schedule
    assert kl_budget(H + 50, H, dmax, dmin) == pytest.approx(dmin, rel=1e-12)
    # equation 17: subtract the mismatch, never below half the budget
    f = b["budget_floor_fraction"]
    assert effective_budget(1e-4, 3e-5) == pytest.approx(7e-5, rel=1e-14)
    assert effective_budget(1e-4, 9e-5) == pytest.approx(f * 1e-4, rel=1e-14)
    assert effective_budget(1e-4, -1.0) == 1e-4  # a negative estimate is clamped to zero
    assert effective_budget(1e-4, None) == 1e-4
    assert effective_budget(1e-4, float("nan")) == 1e-4


def test_empty_and_degenerate():
    assert predicted_kl(np.zeros((0, 5)), np.zeros((0, 5)), 1.0) == 0.0
    # one token per context: probability 1, no variance
    assert predicted_kl(np.ones((4, 1)), np.arange(4.0)[:, None], 1.0) == 0.0
    # a dominant token: with p = (1 - 2e, e, e), e ~ exp(-50), the variance is
    # e ((zd2 - zd1)^2 + (zd3 - zd1)^2) to first order in e
    z = np.array([[50.0, 0.0, 0.0]])
    zd = np.array([[1.0, 2.0, -3.0]])
    e = math.exp(-50.0)
    assert predicted_kl(z, zd, 1.0) == pytest.approx(e * (1.0 + 16.0) / 2.0, rel=1e-15)
