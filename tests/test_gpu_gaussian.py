"""GPU parity of the refreshed Gaussian basis (LoGRA section 3.4.1, Figure
5c) against the float64 oracle, through the C ABI: the generated normals,
the sketch (fused and split calls), the merge, the grouped merge and the
sync payload, at ranks up to 512.
"""

import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import S_TIGHT, W_MAX, assert_sketch_close, bf16_ulp, f64, padded_ld, rel_frob

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


@pytest.fixture
def gaussian():
    prev = lg.set_basis(lg.BASIS_GAUSSIAN)
    yield
    lg.set_basis(prev)


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(T, k, d, seed):
    X = wl.gaussian_bf16((T, k), 1.0, seed, device=DEV, ld=padded_ld(k))
    dY = wl.gaussian_bf16((T, d), 1e-2, seed + 1, device=DEV, ld=padded_ld(d))
    return X, dY


@pytest.mark.parametrize("seed,r,k", [(3, 16, 512), (2**63 + 1, 300, 1000), (7, 512, 37), (0, 1, 9)])
def test_normals_match_oracle(seed, r, k):
    _say("normals", seed, r, k)
    got = f64(lg.basis_normals(seed, r, k))
    ref = oracle.gaussian_normals(seed, r, k)
    # fp32 log, sqrt and sincospi against float64: a few fp32 ulps
    assert np.all(np.abs(got - ref) <= 2e-6 * (1.0 + np.abs(ref)))


@pytest.mark.parametrize("T,k,d,r", [(700, 1300, 300, 16), (700, 1300, 300, 64), (1000, 700, 900, 128),
                                     (700, 1300, 300, 256), (600, 900, 250, 300), (33, 264, 17, 5),
                                     (1500, 2056, 400, 512)])
def test_sketch_gaussian(T, k, d, r, gaussian):
    _say("gaussian sketch", T, k, d, r)
    seed = 70 + r
    X, dY = _inputs(T, k, d, 5 + r)
    X2, dY2 = _inputs(T, k, d, 9 + r)
    S0 = wl.random_tensor((d, r), 3, device=DEV)
    S = S0.clone()
    lg.sketch_accumulate(X, dY, seed, r, S)
    lg.sketch_accumulate(X2, dY2, seed, r, S)
    A = oracle.gaussian_projection(seed, r, k)
    ref = oracle.sketch_accumulate(f64(S0), [f64(X), f64(X2)], [f64(dY), f64(dY2)], A)
    e = assert_sketch_close(f64(S), ref)
    _say("S rel err", e)


def test_gaussian_differs_from_signs_and_noalloc_refuses(gaussian):
    T, k, d, r = 300, 512, 100, 32
    X, dY = _inputs(T, k, d, 1)
    Sg = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    lg.sketch_accumulate(X, dY, 4, r, Sg)
    lg.set_basis(lg.BASIS_RADEMACHER)
    Ss = torch.zeros_like(Sg)
    lg.sketch_accumulate(X, dY, 4, r, Ss)
    lg.set_basis(lg.BASIS_GAUSSIAN)
    torch.cuda.synchronize()
    assert rel_frob(f64(Sg), f64(Ss)) > 0.5
    with pytest.raises(lg.LograError) as ei:
        lg.sketch_accumulate(X, dY, 4, r, Sg, noalloc=True)
    assert ei.value.status == lg.LOGRA_ERR_RANGE


@pytest.mark.parametrize("T,k,d,r", [(700, 1300, 300, 64), (1000, 700, 900, 256), (600, 900, 250, 400)])
def test_split_gaussian(T, k, d, r, gaussian):
    _say("gaussian split", T, k, d, r)
    X, dY = _inputs(T, k, d, 40 + r)
    P = lg.project(X, 15, r)
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    lg.contract(dY, P, r, S)
    A = oracle.gaussian_projection(15, r, k)
    assert_sketch_close(f64(S), oracle.sketch_accumulate(np.zeros((d, r)), [f64(X)], [f64(dY)], A))
    S2 = torch.zeros_like(S)
    lg.sketch_accumulate(X, dY, 15, r, S2)
    torch.cuda.synchronize()
    assert rel_frob(f64(S2), f64(S)) <= S_TIGHT


def _assert_gauss_weight_close(got, ref, U, Z, r, scale):
    """Elementwise: within one bf16 ulp of the oracle, plus the error the
    update itself may carry (U and Z as bf16 hi/lo pairs: 2^-16 relative each,
    fp32 sums over r), doubled for margin."""
    err = np.abs(got - ref)
    mx = float(np.max(np.abs(ref)))
    assert float(err.max(initial=0.0)) <= W_MAX * mx
    bound = 2.0 * (2.0**-15 + r * 2.0**-24) * abs(scale) / math.sqrt(r) * (np.abs(U) @ np.abs(Z))
    ulp = bf16_ulp(np.maximum(np.abs(got), np.abs(ref)))
    bad = err > ulp * 1.0000001 + bound
    assert not bad.any(), f"{int(bad.sum())} elements beyond one ulp + bound"


@pytest.mark.parametrize("d,k,r", [(300, 1032, 16), (129, 2000, 64), (300, 1032, 128), (200, 520, 256),
                                   (70, 520, 512), (1000, 5120, 256)])
def test_merge_gaussian(d, k, r, gaussian):
    _say("gaussian merge", d, k, r)
    seed = 90 + r
    Z = oracle.gaussian_normals(seed, r, k)
    A = Z / math.sqrt(r)
    for scale in (1e-3, -2e-2):
        W = wl.gaussian_bf16((d, k), 0.02, 5 + d, device=DEV, ld=padded_ld(k, 4))
        U = wl.random_tensor((d, r), 6 + r, device=DEV)
        W0 = f64(W)
        lg.merge_update(W, U, seed, r, scale)
        _assert_gauss_weight_close(f64(W), oracle.merge_update(W0, f64(U), A, scale), f64(U), Z, r, scale)
    W = torch.zeros((d, padded_ld(k, 4)), dtype=torch.bfloat16, device=DEV)[:, :k]
    lg.merge_update(W, U, seed, r, 1e-2)
    _assert_gauss_weight_close(f64(W), oracle.merge_update(np.zeros((d, k)), f64(U), A, 1e-2), f64(U), Z, r, 1e-2)


def test_grouped_and_payload_gaussian(gaussian):
    """Grouped Gaussian merges equal separate ones bit for bit; a payload
    packed under the Gaussian basis records it, and a receiver whose own
    setting is Rademacher still applies it in the Gaussian basis and ends
    bitwise equal to the trainer."""
    r = 128
    shapes = [(300, 1032, 1e-3), (64, 520, 2e-3), (500, 2048, -1e-3)]
    items = []
    for j, (d, k, scale) in enumerate(shapes):
        W = wl.gaussian_bf16((d, k), 0.02, 600 + j, device=DEV)
        U = wl.random_tensor((d, r), 610 + j, device=DEV)
        items.append((W, U, 700 + j, scale))
    alone = [W.clone() for W, _, _, _ in items]
    recv = [W.clone() for W, _, _, _ in items]
    for (W, U, seed, scale), Wa in zip(items, alone):
        lg.merge_update(Wa, U, seed, r, scale)
    lg.merge_update_grouped(items, r)
    payload = lg.payload_pack([(U, seed, scale, W.shape[1]) for W, U, seed, scale in items], r)
    torch.cuda.synchronize()
    for (W, _, _, _), Wa in zip(items, alone):
        assert torch.equal(W, Wa)
    header, entries = lg.payload_parse(payload.cpu().numpy().tobytes())
    assert all(entries[j].basis == lg.BASIS_GAUSSIAN for j in range(len(items)))
    lg.set_basis(lg.BASIS_RADEMACHER)
    lg.payload_apply(payload.clone(), header, entries, recv)
    torch.cuda.synchronize()
    for (W, _, _, _), Wr in zip(items, recv):
        assert torch.equal(W, Wr)


def test_full_size_gaussian_sampled_rows(gaussian):
    """The 27B-class attention layer (16384 tokens, 5120 x 5120) at r = 256
    with the Gaussian basis, on sampled rows of S."""
    w = wl.WORKLOADS["layer27b"]
    L = w.layers[0]
    r, seed = 256, 0
    X, dY = wl.layer_inputs(w, 0, 0, device=DEV)
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    lg.sketch_accumulate(X, dY, seed, r, S)
    rows = np.sort(np.random.default_rng(6).choice(L.d, size=96, replace=False))
    rows_t = torch.as_tensor(rows, device=DEV)
    A = oracle.gaussian_projection(seed, r, L.k)
    ref = oracle.sketch_from_gradient(f64(dY[:, rows_t]).T @ f64(X), A)
    assert_sketch_close(f64(S[rows_t]), ref)
