"""Non-finite inputs propagate and nothing traps (include/logra.h: "NaN and
Inf in the inputs propagate to the outputs").

The float64 oracle gives the reference pattern: an entry of S or W is
non-finite exactly where the oracle's is; the finite entries still match it.
Where an Inf meets an exact zero the HIP path may give NaN where the oracle
gives Inf (P and U travel as a bf16 high/low pair, and Inf times a zero low
half is NaN), so the check is on finiteness, not on which non-finite value.
"""

import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import assert_sketch_close, f64, padded_ld

torch = pytest.importorskip("torch")
lg = pytest.importorskip("rank_gradient_sketching_accumulate_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lg.load_library()
    yield
    torch.cuda.synchronize()


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("T,k,d,r", [(700, 1300, 300, 64), (500, 2056, 260, 256), (300, 700, 90, 300)])
def test_sketch_nonfinite_inputs(T, k, d, r):
    _say("nonfinite sketch", T, k, d, r)
    seed = 4000 + r
    X = wl.gaussian_bf16((T, k), 1.0, seed, device=DEV, ld=padded_ld(k))
    dY = wl.gaussian_bf16((T, d), 1e-2, seed + 1, device=DEV, ld=padded_ld(d))
    # an Inf in one gradient entry: row i0 of S turns non-finite, the rest not
    i0, t0 = d // 3, T // 2
    dY[t0, i0] = math.inf
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    lg.sketch_accumulate(X, dY, seed, r, S)
    torch.cuda.synchronize()
    A = oracle.rademacher_projection(seed, r, k)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.sketch_projected_first(np.zeros((d, r)), [f64(X)], [f64(dY)], A)
    got = f64(S)
    assert np.array_equal(np.isfinite(got), np.isfinite(ref))
    assert not np.isfinite(got[i0]).any()
    keep = np.isfinite(ref).all(axis=1)
    assert_sketch_close(got[keep], ref[keep])
    # a NaN in one input entry reaches every entry of S (every sign multiplies it)
    X[T - 1, k - 1] = math.nan
    S.zero_()
    lg.sketch_accumulate(X, dY, seed, r, S)
    torch.cuda.synchronize()
    assert bool(torch.isnan(S).all())


@pytest.mark.parametrize("d,k,r", [(300, 1030, 64), (130, 2052, 256)])
def test_merge_nonfinite_inputs(d, k, r):
    _say("nonfinite merge", d, k, r)
    seed = 4100 + r
    U = wl.random_tensor((d, r), seed, device=DEV)
    W = wl.gaussian_bf16((d, k), 0.02, seed + 1, device=DEV, ld=padded_ld(k, 4))
    # a NaN weight stays NaN; an Inf in U's row i1 makes that row non-finite
    W[5, 7] = math.nan
    i1 = d - 2
    U[i1, r // 2] = math.inf
    W0 = f64(W)
    lg.merge_update(W, U, seed, r, 1e-3)
    torch.cuda.synchronize()
    got = f64(W)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.merge_update(W0, f64(U), oracle.rademacher_projection(seed, r, k), 1e-3)
    assert math.isnan(got[5, 7])
    assert not np.isfinite(got[i1]).any()
    assert np.array_equal(np.isfinite(got), np.isfinite(ref))
    keep = np.isfinite(ref).all(axis=1)
    err = np.abs(got[keep] - ref[keep])
    assert float(err.max()) <= 1e-2 * float(np.abs(ref[keep]).max())
