"""GPU parity at every layer and rank of the five workloads, in the launch
configuration a plain call picks (no plan overrides), against the float64
oracle.

  * sketches of every (workload, layer, rank), plain and, for the 27B-class
    layers, with heavy-tailed activation rows: the oracle recomputes a
    seeded sample of rows of S from the dense gradient (rows of S are
    independent of each other);
  * two layers accumulated over all of their M microbatches, every row of S
    compared (the oracle projects the inputs first, which never forms the
    d x k gradient);
  * merges at every (workload, layer, rank) on sampled rows of W;
  * the 7B-class layers' RowAdam-then-merge over steps t = 1, 2, 3 with
    sign seeds l, l + 100, l + 200 (one fresh microbatch per step, the
    RowAdam state v carried across steps; each step's U is merged into a
    fresh copy of the layer's weight, so a one-ulp difference at one step
    does not carry into the next comparison).
"""

import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import assert_sketch_close, assert_weight_close, f64, rel_frob, update_error_bound

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


def _rows(d, n, seed):
    return np.sort(np.random.default_rng(seed).choice(d, size=min(n, d), replace=False))


def _pairs(keys):
    out = []
    for key in keys:
        w = wl.WORKLOADS[key]
        for li in range(len(w.layers)):
            for r in w.ranks:
                out.append((key, li, r))
    return out


SKETCH_CASES = [(k, li, r, False) for k, li, r in _pairs(("mlp1536", "set7b", "layer27b"))] + [
    ("layer27b", li, 256, True) for li in range(3)
]


def _case_id(c):
    key, li, r, heavy = c
    return f"{key}-{wl.WORKLOADS[key].layers[li].name}-r{r}" + ("-heavy" if heavy else "")


@pytest.mark.parametrize("case", SKETCH_CASES, ids=_case_id)
def test_sketch_every_layer_and_rank(case):
    key, li, r, heavy = case
    w = wl.WORKLOADS[key]
    L = w.layers[li]
    M = 1 if w.T >= 16384 else 2
    seed = wl.sign_seed(li)
    _say("config sketch", key, L, "r", r, "M", M, "heavy" if heavy else "")
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    rows = _rows(L.d, 128, 31 + li + r)
    rows_t = torch.as_tensor(rows, device=DEV)
    A = oracle.rademacher_projection(seed, r, L.k)
    G = np.zeros((len(rows), L.k))
    for m in range(M):
        X, dY = wl.layer_inputs(w, li, m, device=DEV, heavy=heavy)
        lg.sketch_accumulate(X, dY, seed, r, S)
        G += f64(dY[:, rows_t]).T @ f64(X)
        del X, dY
    ref = oracle.sketch_from_gradient(G, A)
    e = assert_sketch_close(f64(S[rows_t]), ref)
    _say("S rel err", e)


@pytest.mark.parametrize("key,li,r", [("mlp1536", 0, 128), ("set7b", 0, 128)])
def test_sketch_all_microbatches_every_row(key, li, r):
    w = wl.WORKLOADS[key]
    L = w.layers[li]
    seed = wl.sign_seed(li)
    _say("all microbatches", key, L, "r", r, "M", w.M)
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    A = oracle.rademacher_projection(seed, r, L.k)
    ref = np.zeros((L.d, r))
    for m in range(w.M):
        X, dY = wl.layer_inputs(w, li, m, device=DEV)
        lg.sketch_accumulate(X, dY, seed, r, S)
        ref = oracle.sketch_projected_first(ref, [f64(X)], [f64(dY)], A)
        del X, dY
    e = assert_sketch_close(f64(S), ref)
    _say("S rel err", e)


MERGE_CASES = _pairs(("mlp1536", "set7b", "layer27b"))


@pytest.mark.parametrize("key,li,r", MERGE_CASES, ids=[f"{k}-{wl.WORKLOADS[k].layers[l].name}-r{r}"
                                                      for k, l, r in MERGE_CASES])
def test_merge_every_layer_and_rank(key, li, r):
    w = wl.WORKLOADS[key]
    L = w.layers[li]
    seed = wl.sign_seed(li)
    _say("config merge", key, L, "r", r)
    # U of the size RowAdam leaves (rows of unit-ish RMS times a spread).
    U = wl.random_tensor((L.d, r), 700 + 10 * li + r, device=DEV, std=50.0)
    rows = _rows(L.d, 64, 3 + li + r)
    rows_t = torch.as_tensor(rows, device=DEV)
    A = oracle.rademacher_projection(seed, r, L.k)
    Ur = f64(U[rows_t])
    for scale in w.scales:
        W = wl.layer_weight(w, li, device=DEV)
        Wr = f64(W[rows_t])
        lg.merge_update(W, U, seed, r, scale)
        assert_weight_close(f64(W[rows_t]), oracle.merge_update(Wr, Ur, A, scale),
                            bound=update_error_bound(Ur, r, scale))
        del W


ROWADAM_CASES = [("set7b", li, 256) for li in range(4)] + [("set7b", 0, 64), ("set7b", 3, 128)]


@pytest.mark.parametrize("key,li,r", ROWADAM_CASES,
                         ids=[f"{wl.WORKLOADS[k].layers[l].name}-r{r}" for k, l, r in ROWADAM_CASES])
def test_rowadam_then_merge_three_steps(key, li, r):
    w = wl.WORKLOADS[key]
    L = w.layers[li]
    beta2, eps = w.beta2, w.eps_rel
    scale = w.scales[0]
    _say("rowadam+merge", key, L, "r", r)
    v = torch.zeros(L.d, dtype=torch.float32, device=DEV)
    v_ref = np.zeros(L.d)
    W0 = wl.layer_weight(w, li, device=DEV)
    rows = _rows(L.d, 64, 40 + li)
    rows_t = torch.as_tensor(rows, device=DEV)
    W0r = f64(W0[rows_t])
    for t in (1, 2, 3):
        seed = wl.sign_seed(li, refresh=t - 1)  # l, l + 100, l + 200
        X, dY = wl.layer_inputs(w, li, t - 1, device=DEV)
        S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
        lg.sketch_accumulate(X, dY, seed, r, S)
        A = oracle.rademacher_projection(seed, r, L.k)
        S_ref = oracle.sketch_projected_first(np.zeros((L.d, r)), [f64(X)], [f64(dY)], A)
        del X, dY
        assert_sketch_close(f64(S), S_ref, what=f"S at t={t}")
        lg.rowadam_scale(S, v, t, beta2, eps)
        # The library takes beta2 and eps_rel as fp32.
        U_ref, v_ref = oracle.rowadam_scale(S_ref, v_ref, t, float(np.float32(beta2)), float(np.float32(eps)))
        assert_sketch_close(f64(S), U_ref, what=f"U at t={t}")
        assert rel_frob(f64(v), v_ref) <= 1e-4, f"v at t={t}"
        W = W0.clone()
        lg.merge_update(W, S, seed, r, scale)
        Ur = U_ref[rows]
        assert_weight_close(f64(W[rows_t]), oracle.merge_update(W0r, Ur, A, scale),
                            bound=update_error_bound(Ur, r, scale), what=f"W at t={t}")
        del W, S
    assert math.isfinite(float(v.sum()))


@pytest.mark.parametrize("d,k,r,basis", [(300, 1032, 64, 0), (3584, 3584, 256, 0), (1000, 2048, 512, 0),
                                         (7, 520, 256, 0), (4000, 1024, 128, 1)])
def test_rowadam_folded_into_merge_is_bitwise_the_two_calls(d, k, r, basis):
    """logra_rowadam_merge over steps t = 1, 2, 3: W and v bitwise equal to
    RowAdam on a copy of S followed by the merge, S untouched."""
    _say("rowadam fold", d, k, r, basis)
    prev = lg.set_basis(basis)
    try:
        W1 = wl.gaussian_bf16((d, k), 0.02, 11, device=DEV)
        W2 = W1.clone()
        v1 = torch.zeros(d, dtype=torch.float32, device=DEV)
        v2 = torch.zeros_like(v1)
        for t in (1, 2, 3):
            S = wl.random_tensor((d, r), 20 + t, device=DEV, std=0.5 * t)
            S_keep = S.clone()
            U = S.clone()
            lg.rowadam_scale(U, v1, t, 0.999, 1e-8)
            lg.merge_update(W1, U, 5 + t, r, 1e-4)
            lg.rowadam_merge(W2, S, v2, 5 + t, r, t, 0.999, 1e-8, 1e-4)
            torch.cuda.synchronize()
            assert torch.equal(v1, v2), f"v at t={t}"
            assert torch.equal(W1, W2), f"W at t={t}"
            assert torch.equal(S, S_keep), "S was written"
    finally:
        lg.set_basis(prev)
