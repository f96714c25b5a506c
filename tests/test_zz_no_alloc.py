"""GPU: logra_sketch_accumulate_noalloc (scratch in the library's static
device array) against logra_sketch_accumulate on the same inputs.

Two calls in a row, the second on a smaller input, so the second runs over
whatever the first left in the shared array; each result is compared with
the allocating entry point's and, on sampled rows, with the float64 oracle.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import S_TIGHT, assert_sketch_close, f64, padded_ld, rel_frob

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


def _inputs(T, k, d, r, seed):
    X = wl.gaussian_bf16((T, k), 1.0, seed, device=DEV, ld=padded_ld(k))
    dY = wl.gaussian_bf16((T, d), 1e-2, seed + 1, device=DEV, ld=padded_ld(d))
    S0 = wl.random_tensor((d, r), seed + 2, device=DEV)
    return X, dY, S0


def _check_pair(T, k, d, r, seed, n_rows=48):
    X, dY, S0 = _inputs(T, k, d, r, seed)
    S_ref = S0.clone()
    S_na = S0.clone()
    lg.sketch_accumulate(X, dY, seed, r, S_ref)
    lg.sketch_accumulate(X, dY, seed, r, S_na, noalloc=True)
    torch.cuda.synchronize()
    got, ref = f64(S_na), f64(S_ref)
    # Same sums in another order (atomic adds instead of partial tiles):
    # the two agree far inside the oracle tolerance.
    e = rel_frob(got - f64(S0), ref - f64(S0))
    assert e <= S_TIGHT, f"noalloc vs allocating entry: relative error of the increment {e:.3e}"
    rows = np.sort(np.random.default_rng(seed).choice(d, size=min(n_rows, d), replace=False))
    A = oracle.rademacher_projection(seed, r, k)
    want = oracle.sketch_accumulate(f64(S0), [f64(X)], [f64(dY)], A, rows=rows)
    assert_sketch_close(got[rows] - f64(S0)[rows], want - f64(S0)[rows], what="S increment (sampled rows)")
    return e


@pytest.mark.parametrize(
    "first,second",
    [
        # 18944-row layer at r = 256 (the allocating call parks three token
        # splits' partial tiles; this one adds them atomically), then a small
        # ragged call whose projection splits its columns (split counters).
        ((8192, 3584, 18944, 256), (700, 1300, 300, 64)),
        # Rank 200 (padded to 256) then rank 3; 32-token ragged tails.
        ((4096, 5120, 5120, 200), (1000, 700, 900, 3)),
    ],
)
def test_noalloc_matches_allocating_entry_twice(first, second):
    for i, (T, k, d, r) in enumerate((first, second)):
        _say("noalloc", i, "T k d r =", T, k, d, r)
        _check_pair(T, k, d, r, 1000 + 17 * i + r)


def test_noalloc_single_bf16_mode():
    prev = lg.set_precision(lg.PRECISION_BF16)
    try:
        for T, k, d, r in ((4096, 1024, 9216, 256), (700, 1300, 300, 256)):
            _say("noalloc bf16 mode", T, k, d, r)
            X, dY, S0 = _inputs(T, k, d, r, 77)
            S_ref, S_na = S0.clone(), S0.clone()
            lg.sketch_accumulate(X, dY, 77, r, S_ref)
            lg.sketch_accumulate(X, dY, 77, r, S_na, noalloc=True)
            torch.cuda.synchronize()
            e = rel_frob(f64(S_na) - f64(S0), f64(S_ref) - f64(S0))
            assert e <= S_TIGHT, f"bf16 mode: noalloc vs allocating {e:.3e}"
    finally:
        lg.set_precision(prev)


def test_noalloc_rejects_oversized_call_and_writes_nothing():
    # P alone would take 70144 x 256 x 4 bytes, above 64 MiB.
    T, k, d, r = 70000, 64, 64, 256
    _say("noalloc oversize", T, k, d, r)
    X = torch.zeros((T, k), dtype=torch.bfloat16, device=DEV)
    dY = torch.zeros((T, d), dtype=torch.bfloat16, device=DEV)
    S = torch.full((d, r), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(lg.LograError) as ei:
        lg.sketch_accumulate(X, dY, 1, r, S, noalloc=True)
    assert ei.value.status == lg.LOGRA_ERR_NOMEM
    assert "static" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((S == 3.0).all())


def test_noalloc_empty_and_invalid_arguments():
    X = torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV)
    dY = torch.zeros((0, 8), dtype=torch.bfloat16, device=DEV)
    S = torch.full((8, 4), 2.0, dtype=torch.float32, device=DEV)
    lg.sketch_accumulate(X, dY, 1, 4, S, noalloc=True)
    torch.cuda.synchronize()
    assert bool((S == 2.0).all())
    X = torch.zeros((32, 16), dtype=torch.bfloat16, device=DEV)
    dY = torch.zeros((32, 8), dtype=torch.bfloat16, device=DEV)
    lib = lg.load_library()
    # lds < r, then r above the maximum: rejected before anything is enqueued.
    st = lib.logra_sketch_accumulate_noalloc(X.data_ptr(), 16, dY.data_ptr(), 8, 32, 16, 8, 1, 4, S.data_ptr(), 3, None)
    assert st == lg.LOGRA_ERR_SHAPE
    st = lib.logra_sketch_accumulate_noalloc(X.data_ptr(), 16, dY.data_ptr(), 8, 32, 16, 8, 1, lg.MAX_RANK + 1,
                                             S.data_ptr(), 1024, None)
    assert st == lg.LOGRA_ERR_RANGE
    torch.cuda.synchronize()
    assert bool((S == 2.0).all())
