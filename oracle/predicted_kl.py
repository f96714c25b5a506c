"""Plain float64 CPU oracle of the predicted-KL step size.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product package.  It shares no
code with the HIP library.

Source: "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
Sketches", section 2.3 (equations 5-7), appendix A.1 (equations 10-13),
appendix A.2 (equation 14) and appendix D.1 (equations 16-17).

Notation.  For each examined context s (a row), z(s) holds the logits over the
vocabulary and zdot(s) their rates of change along the proposed update D;
p(s) = softmax(z(s) / T) at sampling temperature T.  The predicted KL of the
unscaled proposal is

    q(D) = 1 / (2 |P| T^2) * sum_s Var_{v ~ p(s)} [ zdot_v(s) ]      (eq. 6)

and the update multiplier is alpha = min(alpha_max, sqrt(delta / q)) (eq. 7).

Pins live in tests/test_oracle_predicted_kl.py: the printed worked examples of
equation 7, the closed form for two tokens, uniform logits reducing to the
plain variance, the invariances the appendix states (a common shift of the
score rates changes nothing; constant rates give zero), and the exact KL of a
small step along D against alpha^2 q (equations 5, 11 and 12).
"""

from __future__ import annotations

import math

import numpy as np


def token_probabilities(z, temperature: float) -> np.ndarray:
    """p(s) = softmax(z(s) / T) per row, float64 (section 2.3, the
    definition before equation 6).  The row maximum is subtracted first; it
    cancels in the ratio."""
    z = np.asarray(z, dtype=np.float64) / float(temperature)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def score_rate_variance(z, zdot, temperature: float) -> np.ndarray:
    """Var_{v ~ p(s)}[zdot_v(s)] for every row s (equation 6; appendix A.1,
    the line after equation 13): the probability-weighted mean of the rates,
    then the probability-weighted mean squared deviation from it."""
    p = token_probabilities(z, temperature)
    zd = np.asarray(zdot, dtype=np.float64)
    mean = (p * zd).sum(axis=-1, keepdims=True)
    return (p * (zd - mean) ** 2).sum(axis=-1)


def predicted_kl(z, zdot, temperature: float) -> float:
    """q(D) of equation 6: half the average over the examined contexts of
    Var / T^2 (appendix A.1, equation 12 with K''(0) = Var / T^2)."""
    var = score_rate_variance(z, zdot, temperature)
    if var.size == 0:
        return 0.0
    return float(var.mean() / (2.0 * float(temperature) ** 2))


def policy_kl_along(z, zdot, temperature: float, alpha: float) -> float:
    """Average over rows of KL(p(z) || p(z + alpha zdot)) at temperature T:
    the left side of equation 5 when the logits move linearly along D
    (z(a) = z + a zdot).  Used only as a pin: for small alpha it equals
    alpha^2 q(D) + O(alpha^3) (appendix A.1, equations 11-12)."""
    z = np.asarray(z, dtype=np.float64)
    zd = np.asarray(zdot, dtype=np.float64)
    t = float(temperature)

    def log_softmax(x):
        x = x / t
        m = x.max(axis=-1, keepdims=True)
        return x - m - np.log(np.exp(x - m).sum(axis=-1, keepdims=True))

    lp = log_softmax(z)
    lq = log_softmax(z + alpha * zd)
    return float((np.exp(lp) * (lp - lq)).sum(axis=-1).mean())


def kl_step_scale(q: float, delta: float, alpha_max: float) -> float:
    """alpha = min(alpha_max, sqrt(delta / q)) (equation 7; appendix A.2,
    equation 14).  The pages state it for finite positive q; q = 0 reads as
    "no predicted change", where the cap applies, and q = +inf gives 0."""
    if not (delta > 0.0 and alpha_max > 0.0) or math.isnan(q) or q < 0.0:
        raise ValueError("need delta > 0, alpha_max > 0 and q >= 0")
    if q == 0.0:
        return float(alpha_max)
    return float(min(alpha_max, math.sqrt(delta / q)))


def kl_budget(u: int, H: int, delta_max: float, delta_min: float) -> float:
    """Cosine-annealed budget of update u = 1..H (appendix D.1, equation 16):
    delta_min + (delta_max - delta_min)/2 * (1 + cos(pi (u - 1)/(H - 1))).
    Past H the budget stays at delta_min (the 27B runs stop early and the
    Reasoning-Gym run holds it constant after the schedule, appendix D.2)."""
    if H < 2:
        return float(delta_min)
    uu = min(max(int(u), 1), int(H))
    return float(delta_min + 0.5 * (delta_max - delta_min) * (1.0 + math.cos(math.pi * (uu - 1) / (H - 1))))


def effective_budget(delta: float, kappa: float | None) -> float:
    """delta_eff = max(delta - kappa, delta / 2) (appendix D.1, equation 17),
    kappa the smoothed rollout-minus-trainer mismatch, clamped below at zero;
    without a valid measurement (None or NaN) no subtraction is applied."""
    if kappa is None or math.isnan(kappa):
        return float(delta)
    return float(max(delta - max(kappa, 0.0), 0.5 * delta))
