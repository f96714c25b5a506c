"""GPU parity of the predicted-KL reduction (equation 6) against the float64
oracle, through the C ABI.

Tolerance (derived in the design notes): the kernel forms each weight
2^(z log2(e)/T - m) in fp32 from z log2(e)/T rounded to fp32, so a weight
carries a relative error of about |z/T| 2^-24 plus one ulp of the exp2; the
moments accumulate in fp32 with pairwise (Chan) merges and float64 across
threads.  For logits up to |z/T| ~ 60 that is ~1e-5 relative on every
weight, hence on Var; Var per row and q are held to 1e-4 relative.
"""

import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import f64

torch = pytest.importorskip("torch")
lg = pytest.importorskip("rank_gradient_sketching_accumulate_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda"
RTOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lg.load_library()
    yield
    torch.cuda.synchronize()


def _say(*a):
    print("[case]", *a, flush=True)


def _run(z, zd, T):
    n = z.shape[0]
    rv = torch.full((n,), -1.0, dtype=torch.float32, device=DEV)
    q = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    lg.predicted_kl(z, zd, T, row_var=rv, q=q)
    return f64(rv), float(q.item())


def _ld(V, dtype):
    mult = 8 if dtype == torch.bfloat16 else 4
    return (V + mult - 1) // mult * mult


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize(
    "n,V,T",
    [(1, 1, 1.0), (3, 17, 1.0), (7, 1000, 0.7), (64, 4099, 1.0), (5, 4096 * 3 + 1, 1.3),
     (300, 32000, 1.0), (33, 151936, 1.0), (2, 151936, 0.6)],
)
def test_predicted_kl_matches_oracle(n, V, T, dtype):
    _say("predicted kl", n, V, T, dtype)
    z, zd = wl.kl_inputs(n, V, 1000 + n + V, device=DEV, dtype=dtype, ld=_ld(V, dtype) + 8)
    rv, q = _run(z, zd, T)
    zh, zdh = f64(z), f64(zd)
    ref_rv = oracle.score_rate_variance(zh, zdh, T)
    ref_q = oracle.predicted_kl(zh, zdh, T)
    np.testing.assert_allclose(rv, ref_rv, rtol=RTOL, atol=1e-30)
    assert q == pytest.approx(ref_q, rel=RTOL, abs=1e-30)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_predicted_kl_full_size_sampled_rows(dtype):
    """The probe at its benchmark size (2048 contexts x 151,936 tokens): a
    seeded sample of rows against the oracle, and q against the mean of the
    kernel's own per-row variances (a property that holds at any size)."""
    n, V, T = wl.KL_CONTEXTS, wl.KL_VOCAB, 1.0
    _say("predicted kl full size", n, V, dtype)
    z, zd = wl.kl_inputs(n, V, 77, device=DEV, dtype=dtype)
    rv, q = _run(z, zd, T)
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(3).choice(n, 48, replace=False)]))
    idx = torch.as_tensor(rows, device=DEV)
    ref = oracle.score_rate_variance(f64(z[idx]), f64(zd[idx]), T)
    np.testing.assert_allclose(rv[rows], ref, rtol=RTOL)
    assert q == pytest.approx(rv.mean() / (2 * T * T), rel=1e-6)


def test_predicted_kl_peaked_and_shifted_rows():
    """Nearly one-hot rows (the variance comes from tokens of probability
    ~e^-40) and score rates with a large common offset: both are where a
    sum-of-squares formula would lose every digit."""
    n, V, T = 16, 50000, 1.0
    z, zd = wl.kl_inputs(n, V, 5, device=DEV, peak=40.0, zdot_std=1.0)
    zd += 1000.0
    rv, q = _run(z, zd, T)
    ref = oracle.score_rate_variance(f64(z), f64(zd), T)
    np.testing.assert_allclose(rv, ref, rtol=RTOL)
    assert q == pytest.approx(oracle.predicted_kl(f64(z), f64(zd), T), rel=RTOL)


def test_predicted_kl_edge_cases():
    _say("predicted kl edge cases")
    # no rows: q = 0
    q = torch.full((1,), 7.0, dtype=torch.float32, device=DEV)
    e = torch.empty((0, 100), dtype=torch.float32, device=DEV)
    lg.predicted_kl(e, e, 1.0, q=q)
    assert float(q.item()) == 0.0
    # one token: probability one, zero variance
    z = torch.randn((4, 4), device=DEV)[:, :1]
    rv, qv = _run(z, torch.randn((4, 4), device=DEV)[:, :1], 1.0)
    assert np.all(rv == 0.0) and qv == 0.0
    # a single row may have any stride
    z, zd = wl.kl_inputs(1, 37, 13, device=DEV)
    rv, qv = _run(z, zd, 1.0)
    assert rv[0] == pytest.approx(oracle.score_rate_variance(f64(z), f64(zd), 1.0)[0], rel=RTOL)
    # constant rates give zero; equal logits give the plain variance
    V = 3000
    z = torch.full((2, V), 0.5, device=DEV)
    zd = torch.randn((2, V), device=DEV)
    zd[1] = 3.25
    rv, _ = _run(z, zd, 1.0)
    assert rv[0] == pytest.approx(float(f64(zd[0]).var()), rel=RTOL)
    assert abs(rv[1]) <= 1e-10
    # -inf logits carry no probability; an all -inf row has no distribution
    z, zd = wl.kl_inputs(3, 5000, 9, device=DEV)
    z[0, ::3] = -math.inf
    z[2, :] = -math.inf
    rv, qv = _run(z, zd, 1.0)
    ref0 = oracle.score_rate_variance(f64(z[0:1]), f64(zd[0:1]), 1.0)[0]
    assert rv[0] == pytest.approx(ref0, rel=RTOL)
    assert math.isnan(rv[2]) and math.isnan(qv)
    # NaN propagates
    z, zd = wl.kl_inputs(2, 5000, 10, device=DEV)
    zd[1, 1234] = math.nan
    rv, qv = _run(z, zd, 1.0)
    assert not math.isnan(rv[0]) and math.isnan(rv[1]) and math.isnan(qv)
    # deterministic: the same call twice gives the same bits
    z, zd = wl.kl_inputs(50, 20000, 11, device=DEV)
    a, qa = _run(z, zd, 0.9)
    b, qb = _run(z, zd, 0.9)
    assert np.array_equal(a, b) and qa == qb


def test_step_scale_from_device_q():
    """alpha from the device's q meets the budget: alpha^2 q = delta."""
    z, zd = wl.kl_inputs(64, 8192, 12, device=DEV, zdot_std=0.3)
    _, q = _run(z, zd, 1.0)
    delta = q / 4.0
    a = lg.kl_step_scale(q, delta, 10.0)
    assert a == pytest.approx(0.5, rel=1e-12)
    assert lg.kl_step_scale(q, 100.0 * q, 3.0) == 3.0
