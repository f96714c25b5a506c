"""GPU parity of the single-bf16 contraction (logra_set_precision).

With LOGRA_PRECISION_BF16 the fused sketch rounds the projected inputs P
once to bf16 (round to nearest even) before the backward multiply.  It is
compared (a) with the float64 oracle of the method, against the stated
bar of 2e-3 relative Frobenius error, and (b) with the oracle that rounds P
the same way (sketch_accumulate_rounded_projection), where the only
remaining differences are fp32 accumulation and the rare P entry whose fp32
sum rounds to a neighbouring bf16 value: 1e-4.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import S_TOL, f64, padded_ld, rel_frob

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
def bf16_mode():
    prev = lg.set_precision(lg.PRECISION_BF16)
    try:
        yield
    finally:
        lg.set_precision(prev)


def _inputs(T, k, d, seed, heavy=False):
    X = wl.gaussian_bf16((T, k), 1.0, seed, device=DEV, ld=padded_ld(k))
    if heavy:
        X[: max(1, T // 100)] *= 50
    dY = wl.gaussian_bf16((T, d), 1e-3, seed + 1, device=DEV, ld=padded_ld(d))
    return X, dY


@pytest.mark.parametrize(
    "T,k,d,r,env",
    [
        (700, 1300, 300, 64, {}),
        (700, 1300, 300, 256, {}),
        (1000, 700, 900, 128, {}),
        (700, 1300, 300, 256, {"LOGRA_CON_WIDE": 1}),
        (1500, 1536, 700, 256, {"LOGRA_CON_WIDE": 1}),
        (4096, 1024, 9216, 256, {}),
    ],
    ids=lambda v: str(v).replace(" ", ""),
)
def test_single_bf16_sketch(T, k, d, r, env, bf16_mode, monkeypatch):
    for k_, v_ in env.items():
        monkeypatch.setenv(k_, str(v_))
    print("[case] bf16", T, k, d, r, env, flush=True)
    seed = 70 + r
    X, dY = _inputs(T, k, d, seed)
    X2, dY2 = _inputs(T, k, d, seed + 10, heavy=True)
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    lg.sketch_accumulate(X, dY, seed, r, S)
    lg.sketch_accumulate(X2, dY2, seed, r, S)
    rows = None if d <= 1000 else np.arange(0, d, 23)
    got = f64(S) if rows is None else f64(S)[rows]
    A = oracle.rademacher_projection(seed, r, k)
    ref = oracle.sketch_accumulate(np.zeros((d, r)), [f64(X), f64(X2)], [f64(dY), f64(dY2)], A, rows=rows)
    ref_b = oracle.sketch_accumulate_rounded_projection(np.zeros((d, r)), [f64(X), f64(X2)], [f64(dY), f64(dY2)],
                                                        seed, r, rows=rows)
    e = rel_frob(got, ref)
    eb = rel_frob(got, ref_b)
    print(f"[case] bf16 error vs method {e:.3e}, vs rounded-projection oracle {eb:.3e}", flush=True)
    assert e <= S_TOL
    assert eb <= 1e-4
    # it really is the single-rounding mode (a hi/lo pair would be ~1e-5)
    assert e > 3e-4


def test_split_contract_keeps_both_planes(bf16_mode):
    """logra_contract reads both planes of a projection cache in either mode."""
    T, k, d, r = 700, 1300, 300, 256
    X, dY = _inputs(T, k, d, 5)
    P = lg.project(X, 5, r)
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    lg.contract(dY, P, r, S)
    ref = oracle.sketch_accumulate(np.zeros((d, r)), [f64(X)], [f64(dY)], oracle.rademacher_projection(5, r, k))
    assert rel_frob(f64(S), ref) <= 1e-4


def _layer_cases():
    out = []
    for key in ("mlp1536", "set7b", "layer27b"):
        w = wl.WORKLOADS[key]
        for li in range(len(w.layers)):
            for r in w.ranks:
                out.append((key, li, r))
    return out


@pytest.mark.parametrize("key,li,r", _layer_cases(),
                         ids=[f"{k}-{wl.WORKLOADS[k].layers[l].name}-r{r}" for k, l, r in _layer_cases()])
def test_bf16_mode_every_layer(key, li, r, bf16_mode):
    """The single-bf16 mode at every 1.5B/7B/27B-class layer and rank (one
    microbatch, sampled rows of S): within the 2e-3 bar of the method, and
    within 1e-4 of the oracle that rounds P the same way."""
    w = wl.WORKLOADS[key]
    L = w.layers[li]
    seed = wl.sign_seed(li)
    X, dY = wl.layer_inputs(w, li, 0, device=DEV)
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    lg.sketch_accumulate(X, dY, seed, r, S)
    rows = np.sort(np.random.default_rng(li + r).choice(L.d, size=min(96, L.d), replace=False))
    rows_t = torch.as_tensor(rows, device=DEV)
    got = f64(S[rows_t])
    Xh, dYr = f64(X), f64(dY[:, rows_t])
    exact = oracle.sketch_from_gradient(dYr.T @ Xh, oracle.rademacher_projection(seed, r, L.k))
    rounded = oracle.sketch_accumulate_rounded_projection(np.zeros((len(rows), r)), [Xh], [dYr], seed, r)
    e_m, e_r = rel_frob(got, exact), rel_frob(got, rounded)
    print(f"[case] bf16 mode {key} {L.name} r={r}: vs method {e_m:.3e}, vs rounded-P oracle {e_r:.3e}", flush=True)
    assert e_m <= S_TOL
    assert e_r <= 1e-4
