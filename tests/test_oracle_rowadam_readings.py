"""How far the alternative readings of RowAdam's lost words move U (CPU,
float64).

Appendix B of the LoGRA paper lost three words in the extracted text: what
the "normalized" sketch fed to the second-moment update is, which statistic
of sqrt(vhat) the stabiliser scales, and which norm of the original sketch
the scaled factor is matched to.  The oracle reads them as: the sketch as
passed, the mean, and the Frobenius norm.  This module re-runs RowAdam with
each alternative on 7B-class layer shapes over steps t = 1, 2, 3 and reports
||U_alt - U_oracle||_F / ||U_oracle||_F:

  * normalized: S / ||S||_F enters the v update (U is still matched to
    ||S||_F);
  * median: eps = 1e-8 * median_i sqrt(vhat_i);
  * row norms: each row of the scaled factor matched to that row of S.

Sketches: S_t from 1024 synthetic tokens of the layer shape with sign seeds
l, l + 100, l + 200 (S via the projected-first oracle).  The output
gradients carry a log-normal scale per output feature (sigma 1, fixed across
steps) so that rows of S differ in norm, and a per-step factor (1, 3, 0.5)
so that successive sketches differ in overall norm, the two conditions under
which the readings can differ at all.  Run with -s to see the table.
"""

import numpy as np
import pytest

import oracle

BETA2, EPS_REL = 0.999, 1e-8
LAYERS = [("q", 3584, 3584), ("up", 18944, 3584), ("down", 3584, 18944)]
STEP_SCALE = (1.0, 3.0, 0.5)


def rowadam_variant(S, v, t, normalized=False, stat="mean", match="frobenius"):
    S = np.asarray(S, dtype=np.float64)
    r = S.shape[1]
    ns = float(np.sqrt((S * S).sum()))
    Sin = S / ns if normalized and ns > 0 else S
    v_new = BETA2 * v + (1.0 - BETA2) * (Sin * Sin).sum(axis=1) / r
    root = np.sqrt(v_new / (1.0 - BETA2**t))
    eps = max(EPS_REL * float(np.mean(root) if stat == "mean" else np.median(root)), 1e-30)
    Ut = S / (root + eps)[:, None]
    if match == "frobenius":
        nt = float(np.sqrt((Ut * Ut).sum()))
        U = Ut * (ns / nt) if nt > 0 else np.zeros_like(S)
    else:
        rs = np.sqrt((S * S).sum(axis=1))
        rt = np.sqrt((Ut * Ut).sum(axis=1))
        U = Ut * np.where(rt > 0, rs / np.where(rt > 0, rt, 1.0), 0.0)[:, None]
    return U, v_new


def _sketches(li, d, k, r, T=1024):
    rng = np.random.default_rng(100 + li)
    feat = np.exp(rng.standard_normal(d))  # per output feature, fixed across steps
    out = []
    for t in (1, 2, 3):
        X = rng.standard_normal((T, k))
        dY = rng.standard_normal((T, d)) * feat[None, :] * (1e-3 * STEP_SCALE[t - 1])
        A = oracle.rademacher_projection(li + 100 * (t - 1), r, k)
        out.append(oracle.sketch_projected_first(np.zeros((d, r)), [X], [dY], A))
    return out


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("li", range(len(LAYERS)))
@pytest.mark.parametrize("r", [64, 256])
def test_readings_sensitivity(li, r):
    name, d, k = LAYERS[li]
    Ss = _sketches(li, d, k, r)
    v = {key: np.zeros(d) for key in ("oracle", "harness", "normalized", "median", "rows")}
    rows = []
    for t, S in zip((1, 2, 3), Ss):
        U_o, v["oracle"] = oracle.rowadam_scale(S, v["oracle"], t, BETA2, EPS_REL)
        U_h, v["harness"] = rowadam_variant(S, v["harness"], t)
        # the harness with the oracle's readings is the oracle
        assert _rel(U_h, U_o) < 1e-13
        U_n, v["normalized"] = rowadam_variant(S, v["normalized"], t, normalized=True)
        U_m, v["median"] = rowadam_variant(S, v["median"], t, stat="median")
        U_r, v["rows"] = rowadam_variant(S, v["rows"], t, match="rows")
        rows.append((t, _rel(U_n, U_o), _rel(U_m, U_o), _rel(U_r, U_o)))
    print(f"\n{name} {d}x{k} r={r}: t, normalized, median, row-norms")
    for t, a, b, c in rows:
        print(f"  t={t}: {a:.3e} {b:.3e} {c:.3e}")
    # t = 1: vhat is the first mean square exactly, so normalising S first
    # only rescales root and eps together: the same U.
    assert rows[0][1] < 1e-12
    # The stabiliser is 1e-8 of a typical root: mean or median hardly matter.
    assert all(b < 1e-6 for _, _, b, _ in rows)
    # Later steps: the readings that change the update measurably.
    assert rows[1][1] > 1e-4 and rows[2][1] > 1e-4
    assert all(c > 1e-2 for _, _, _, c in rows)
