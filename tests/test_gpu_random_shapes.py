"""Seeded random shapes through the default plans, against the float64 oracle.

Every other parity test picks its shapes by hand; these draw T, k, d and r
(and, for the merge, d, k and r) at random from wide ranges, with ragged
leading dimensions, so that the planner's choices between tilings, splits and
kernels meet shapes nobody picked.  Sizes are capped so that the oracle
(projection first for the sketch, a float64 product for the merge) stays
quick; each case prints its shape first.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import assert_sketch_close, assert_weight_close, f64, padded_ld, update_error_bound

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


def _sketch_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.integers(1, 2600))
        k = int(rng.integers(1, 6000))
        d = int(rng.integers(1, 700))
        r = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 257)), int(rng.integers(257, 513))]))
        if T * k * r <= 3e8 and T * d * r <= 3e8:
            out.append((T, k, d, r))
    return out


def _merge_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.integers(1, 2000))
        k = int(rng.integers(1, 6000))
        r = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 257)), int(rng.integers(257, 513))]))
        if d * k * r <= 3e8:
            out.append((d, k, r))
    return out


@pytest.mark.parametrize("T,k,d,r", _sketch_shapes(40, 2026))
def test_sketch_random_shape(T, k, d, r):
    _say("random sketch", T, k, d, r)
    seed = T * 7 + k * 3 + d + r
    X = wl.gaussian_bf16((T, k), 1.0, seed, device=DEV, ld=padded_ld(k))
    dY = wl.gaussian_bf16((T, d), 1e-2, seed + 1, device=DEV, ld=padded_ld(d))
    S0 = wl.random_tensor((d, r), seed + 2, device=DEV)
    S = S0.clone()
    lg.sketch_accumulate(X, dY, seed, r, S)
    ref = oracle.sketch_projected_first(f64(S0), [f64(X)], [f64(dY)], oracle.rademacher_projection(seed, r, k))
    assert_sketch_close(f64(S), ref)


@pytest.mark.parametrize("d,k,r", _merge_shapes(30, 2027))
def test_merge_random_shape(d, k, r):
    _say("random merge", d, k, r)
    seed = d * 5 + k + r
    U = wl.random_tensor((d, r), seed, device=DEV, std=3.0)
    W = wl.gaussian_bf16((d, k), 0.02, seed + 1, device=DEV, ld=padded_ld(k, 4))
    W0 = W.clone()
    scale = 1e-3
    lg.merge_update(W, U, seed, r, scale)
    ref = oracle.merge_update(f64(W0), f64(U), oracle.rademacher_projection(seed, r, k), scale)
    assert_weight_close(f64(W), ref, bound=update_error_bound(f64(U), r, scale))
