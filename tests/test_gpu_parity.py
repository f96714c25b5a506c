"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Every input is drawn once on the device by the seeded generators of
``workloads`` and copied to the host for the oracle, so both sides consume
identical bf16 values.  Sizes run from single elements through several
tiles with ragged tails to the full workloads; at the largest sizes the
oracle recomputes a seeded sample of rows of S (rows of S and of a plain
merge are independent of each other).
"""

import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import (
    assert_sketch_close,
    assert_weight_close,
    f64,
    padded_ld,
    rel_frob,
    update_error_bound,
)

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


def _ragged_inputs(T, k, d, seed, sx=1.0, sdy=1e-2):
    X = wl.gaussian_bf16((T, k), sx, seed, device=DEV, ld=padded_ld(k))
    dY = wl.gaussian_bf16((T, d), sdy, seed + 1, device=DEV, ld=padded_ld(d))
    return X, dY


# ---------------------------------------------------------------------------
# Signs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize(
    "seed,r,k",
    [(0, 16, 512), (1, 3, 700), (2**63 + 5, 5, 257), (42, 256, 1536), (7, 64, 33), (123, 1, 1), (9, 200, 5120),
     (5, 512, 700), (6, 300, 1300)],
)
def test_signs_bit_exact(seed, r, k):
    _say("signs", seed, r, k)
    got = lg.signs(seed, r, k).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.sign_matrix(seed, r, k))


# ---------------------------------------------------------------------------
# Sketch accumulation
# ---------------------------------------------------------------------------
def _oracle_sketch(S0, Xs, dYs, seed, r, k, rows=None):
    A = oracle.rademacher_projection(seed, r, k)
    return oracle.sketch_accumulate(f64(S0), [f64(x) for x in Xs], [f64(y) for y in dYs], A, rows=rows)


def test_sketch_tiny_workload():
    w = wl.WORKLOADS["tiny"]
    L = w.layers[0]
    r = w.ranks[0]
    seed = wl.sign_seed(0)
    _say("tiny workload", L, r)
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    Xs, dYs = [], []
    for m in range(w.M):
        X, dY = wl.layer_inputs(w, 0, m, device=DEV)
        Xs.append(X)
        dYs.append(dY)
        lg.sketch_accumulate(X, dY, seed, r, S)
    ref = _oracle_sketch(torch.zeros_like(S), Xs, dYs, seed, r, L.k)
    e = assert_sketch_close(f64(S), ref)
    _say("tiny S rel err", e)


@pytest.mark.parametrize(
    "T,k,d,r",
    [
        (1, 8, 1, 1),
        (33, 264, 17, 5),
        (100, 700, 77, 40),
        (257, 1000, 130, 16),
        (500, 520, 300, 100),
        (64, 256, 64, 256),
        (2000, 300, 50, 128),
        (96, 2056, 1100, 64),
        (1500, 1536, 700, 256),
    ],
)
def test_sketch_ragged(T, k, d, r):
    _say("sketch ragged", T, k, d, r)
    seed = 1000 + T + k
    S = wl.random_tensor((d, r), seed + 7, device=DEV)
    S0 = S.clone()
    Xs, dYs = [], []
    for m in range(2):
        X, dY = _ragged_inputs(T, k, d, seed + 10 * m)
        Xs.append(X)
        dYs.append(dY)
        lg.sketch_accumulate(X, dY, seed, r, S)
    ref = _oracle_sketch(S0, Xs, dYs, seed, r, k)
    # compare the accumulated increment, so the error is not diluted by S0
    assert_sketch_close(f64(S) - f64(S0), ref - f64(S0))


def test_sketch_attn1536_full():
    """The 1.5B-class attention workload in full: 8 microbatches of 4096 tokens."""
    w = wl.WORKLOADS["attn1536"]
    L = w.layers[0]
    r = w.ranks[0]
    _say("attn1536 full", L, r)
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    G = np.zeros((L.d, L.k))
    for m in range(w.M):
        X, dY = wl.layer_inputs(w, 0, m, device=DEV)
        lg.sketch_accumulate(X, dY, wl.sign_seed(0), r, S)
        G += f64(dY).T @ f64(X)
    ref = oracle.sketch_from_gradient(G, oracle.rademacher_projection(wl.sign_seed(0), r, L.k))
    e = assert_sketch_close(f64(S), ref)
    _say("attn1536 S rel err", e)


def _sampled_rows(d, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(d, size=min(d, n), replace=False).tolist())
    rows.update({0, d - 1})
    return np.array(sorted(rows))


@pytest.mark.parametrize(
    "key,layer,r,M,heavy",
    [
        ("mlp1536", 0, 128, 2, False),
        ("mlp1536", 1, 128, 1, False),
        ("set7b", 2, 256, 1, False),
        ("set7b", 3, 64, 1, False),
        ("layer27b", 1, 256, 1, False),
        ("layer27b", 0, 256, 1, True),
    ],
)
def test_sketch_full_size_sampled_rows(key, layer, r, M, heavy):
    """Full-size layers in the launch configuration the benchmark uses; the
    oracle recomputes a seeded sample of rows of S."""
    w = wl.WORKLOADS[key]
    L = w.layers[layer]
    seed = wl.sign_seed(layer)
    _say("full size", key, L, r, M, "heavy" if heavy else "")
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    rows = _sampled_rows(L.d, 256, 17 + layer)
    A = oracle.rademacher_projection(seed, r, L.k)
    ref = np.zeros((len(rows), r))
    for m in range(M):
        X, dY = wl.layer_inputs(w, layer, m, device=DEV, heavy=heavy)
        lg.sketch_accumulate(X, dY, seed, r, S)
        dYr = dY[:, torch.as_tensor(rows, device=DEV)]
        ref += oracle.sketch_from_gradient(f64(dYr).T @ f64(X), A)
        del X, dY, dYr
    got = f64(S)[rows]
    e = assert_sketch_close(got, ref)
    _say("full size S rel err", e)


PLAN_OVERRIDES = [
    {},
    {"LOGRA_PROJ_MB": 2},
    {"LOGRA_PROJ_SMALL": 0},
    {"LOGRA_PROJ_SMALL": 0, "LOGRA_PROJ_NK": 1},
    {"LOGRA_PROJ_SMALL": 0, "LOGRA_PROJ_NK": 3},
    {"LOGRA_PROJ_SMALL": 0, "LOGRA_PROJ_WK": 1, "LOGRA_PROJ_MB": 2},
    {"LOGRA_PROJ_SMALL": 0, "LOGRA_PROJ_WK": 2, "LOGRA_PROJ_MB": 1, "LOGRA_PROJ_NK": 2},
    {"LOGRA_CON_TS": 1},
    {"LOGRA_CON_TS": 7},
    {"LOGRA_CON_TS": 3, "LOGRA_PROJ_SMALL": 0, "LOGRA_PROJ_NK": 2},
    {"LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1},
    {"LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1, "LOGRA_CON_TS": 5},
    {"LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 0},
    {"LOGRA_CON_WM": 2},
    {"LOGRA_CON_WM": 4, "LOGRA_CON_TS": 2},
    {"LOGRA_PROJ_SMALL": 0, "LOGRA_PROJ_WK": 4, "LOGRA_PROJ_MB": 2},
    {"LOGRA_PROJ_SMALL": 0, "LOGRA_PROJ_WK": 4, "LOGRA_PROJ_MB": 1, "LOGRA_PROJ_NK": 2},
    {"LOGRA_CON_PART": 1, "LOGRA_CON_TS": 6},
    {"LOGRA_CON_PART": 1, "LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1, "LOGRA_CON_TS": 4},
    {"LOGRA_CON_PART": 1, "LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 0, "LOGRA_CON_TS": 3},
    {"LOGRA_CON_PART": 0, "LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1, "LOGRA_CON_TS": 5},
    {"LOGRA_PROJ_SMALL": 0, "LOGRA_PROJ_NW": 8, "LOGRA_PROJ_MB": 2, "LOGRA_PROJ_WK": 4},
    {"LOGRA_PROJ_SMALL": 0, "LOGRA_PROJ_NW": 8, "LOGRA_PROJ_MB": 2, "LOGRA_PROJ_WK": 2, "LOGRA_PROJ_NK": 3},
    {"LOGRA_CON_GRID": 7},
    {"LOGRA_CON_GRID": 3},
    {"LOGRA_CON_BANDS": 8, "LOGRA_CON_GRID": 16},
    {"LOGRA_CON_BANDS": 1, "LOGRA_CON_GRID": 5},
    {"LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1, "LOGRA_CON_BIGDP": 1, "LOGRA_CON_TS": 3},
    {"LOGRA_CON_TILE": 1, "LOGRA_CON_WM": 1},
    {"LOGRA_CON_TILE": 1, "LOGRA_CON_WM": 2},
    {"LOGRA_CON_TILE": 1, "LOGRA_CON_WM": 4},
    {"LOGRA_CON_TILE": 1, "LOGRA_CON_WM": 2, "LOGRA_CON_BANDS": 1, "LOGRA_CON_GRID": 37},
    {"LOGRA_CON_BANDS": 4},
    {"LOGRA_CON_BANDS": 8, "LOGRA_CON_GRID": 24},
    {"LOGRA_CON_BANDS": 4, "LOGRA_CON_GRID": 12},
    {"LOGRA_PROJ_NK": 2},
    {"LOGRA_PROJ_NK": 4, "LOGRA_CON_TS": 3},
]


def _plan_id(e):
    return ",".join(f"{k[6:]}={v}" for k, v in e.items()) or "default"


# Knobs of proj_kernel's tiling (waves along k, token blocks per wave, waves
# per workgroup); the LDS-staged projection has a fixed tiling.
PROJ_KERNEL_KNOBS = ("LOGRA_PROJ_MB", "LOGRA_PROJ_WK", "LOGRA_PROJ_NW")

# Tilings reachable at ranks 129-256 (NB = 16): the eight-wave projection
# (column splits NK), the four- and eight-wave proj_kernel
# (the latter with two token rows per workgroup), and the contraction's
# 256 x 256 tiles (one or two steps of prefetch), the one-wave-per-SIMD and
# shared-operand kernels, and the token-lane tiles.
R256_PLANS = [
    {},
    {"LOGRA_PROJ_NK": 1},
    {"LOGRA_PROJ_NK": 2},
    {"LOGRA_PROJ_NK": 4},
    {"LOGRA_PROJ_NK": 3},
    {"LOGRA_PROJ_NK": 8},
    {"LOGRA_PROJ_WIDE": 0},
    {"LOGRA_PROJ_WIDE": 0, "LOGRA_PROJ_NW": 8, "LOGRA_PROJ_MB": 2, "LOGRA_PROJ_WK": 4},
    {"LOGRA_PROJ_WIDE": 0, "LOGRA_PROJ_NW": 8, "LOGRA_PROJ_MB": 2, "LOGRA_PROJ_WK": 2, "LOGRA_PROJ_NK": 2},
    {"LOGRA_PROJ_WIDE": 0, "LOGRA_PROJ_WK": 1, "LOGRA_PROJ_MB": 1},
    {"LOGRA_CON_WIDE": 1},
    {"LOGRA_CON_WIDE": 2},
    {"LOGRA_CON_WIDE": 1, "LOGRA_CON_TS": 1},
    {"LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1, "LOGRA_CON_BIGDP": 1},
    {"LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1, "LOGRA_CON_HALF": 0},
    {"LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1, "LOGRA_CON_HALF": 1, "LOGRA_CON_TS": 5},
    {"LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1, "LOGRA_CON_HALF": 1, "LOGRA_CON_PART": 0, "LOGRA_CON_TS": 3},
    {"LOGRA_CON_TILE": 0, "LOGRA_CON_BIG": 1, "LOGRA_CON_TS": 2, "LOGRA_CON_PART": 0},
    {"LOGRA_CON_TILE": 1},
    {"LOGRA_CON_TILE": 1, "LOGRA_CON_WM": 2},
]


def test_sketch_consecutive_calls_changing_shapes():
    """Consecutive calls on one stream with changing shapes and inputs (so
    changing plans, tile counts and scratch layouts, including the column
    splits whose last-arriving workgroup sums the partials) each give the
    oracle's sketch: nothing one call leaves in the scratch leaks into the
    next."""
    cases = [(4096, 1536, 1536, 64), (700, 1300, 300, 64), (33, 264, 17, 5), (4096, 1536, 1536, 64),
             (9000, 520, 130, 16), (1, 8, 1, 1), (2500, 700, 77, 40), (700, 1300, 300, 64),
             (300, 5120, 96, 256), (1000, 2056, 200, 128), (300, 5120, 96, 256)]
    for j, (T, k, d, r) in enumerate(cases):
        _say("handoff", j, T, k, d, r)
        seed = 5000 + j
        X, dY = _ragged_inputs(T, k, d, seed)
        X2, dY2 = _ragged_inputs(T, k, d, seed + 50)
        S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
        lg.sketch_accumulate(X, dY, seed, r, S)
        lg.sketch_accumulate(X2, dY2, seed, r, S)  # same plan, new inputs
        rows = None if d <= 300 else np.arange(0, d, 37)
        ref = _oracle_sketch(torch.zeros_like(S), [X, X2], [dY, dY2], seed, r, k, rows=rows)
        got = f64(S) if rows is None else f64(S)[rows]
        assert_sketch_close(got, ref)


@pytest.mark.parametrize("r", [64, 128, 256])
@pytest.mark.parametrize("env", PLAN_OVERRIDES, ids=_plan_id)
def test_sketch_launch_plans(r, env, monkeypatch):
    """Every tiling the planner can pick (the all-signs-in-LDS projection, the
    round-based projection with column splits across workgroups and the
    last-arriver reduction, waves along k or tokens, token splits of the
    contraction) gives the oracle's sketch."""
    if r == 256 and env.get("LOGRA_PROJ_SMALL", 1):
        env = dict(env, LOGRA_PROJ_SMALL=0)  # rank 256 always takes the round-based projection
    if r >= 128 and any(k_ in env for k_ in PROJ_KERNEL_KNOBS):
        # ranks above 64 with two or more 256-column blocks take the
        # LDS-staged projection, whose tiling these knobs do not set: run
        # them on proj_kernel
        env = dict(env, LOGRA_PROJ_WIDE=0)
    for k_, v_ in env.items():
        monkeypatch.setenv(k_, str(v_))
    T, k, d = 700, 1300, 300
    _say("plans", r, env)
    X, dY = _ragged_inputs(T, k, d, 4242)
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    lg.sketch_accumulate(X, dY, 11, r, S)
    ref = _oracle_sketch(torch.zeros((d, r)), [X], [dY], 11, r, k)
    assert_sketch_close(f64(S), ref)


@pytest.mark.parametrize("T,k,d,r", [(700, 1300, 300, 256), (1500, 700, 900, 200), (4096, 5120, 600, 256)])
@pytest.mark.parametrize("env", R256_PLANS, ids=_plan_id)
def test_sketch_rank256_plans(T, k, d, r, env, monkeypatch):
    """Every rank-256 tiling, including k = 700 (three 256-column blocks: two
    waves along k in proj_kernel) and rank 200 (padded to 256 columns), gives
    the oracle's sketch over two microbatches."""
    for k_, v_ in env.items():
        monkeypatch.setenv(k_, str(v_))
    _say("r256 plans", T, k, d, r, env)
    seed = 60 + r
    X, dY = _ragged_inputs(T, k, d, 4545)
    X2, dY2 = _ragged_inputs(T, k, d, 4547)
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    lg.sketch_accumulate(X, dY, seed, r, S)
    lg.sketch_accumulate(X2, dY2, seed, r, S)
    rows = None if d <= 300 else np.arange(0, d, 7)
    ref = _oracle_sketch(torch.zeros((d, r)), [X, X2], [dY, dY2], seed, r, k, rows=rows)
    got = f64(S) if rows is None else f64(S)[rows]
    assert_sketch_close(got, ref)


@pytest.mark.parametrize("T,k,d,r", [(8192, 520, 2125, 256), (8192 - 37, 264, 2125, 200), (8192, 264, 3100, 128)])
def test_sketch_half_tiles_on_shorter_s(T, k, d, r):
    """The default plan at these sizes contracts with the half tiles (two
    256 x 128 workgroups per CU) on S of a few thousand rows: eight token
    splits of at least 32 steps above rank 128, sixteen at rank 128, partial
    tiles summed by the reduction kernel, a ragged last row tile, and a
    ragged last token step in the second case."""
    _say("half tiles", T, k, d, r)
    X, dY = _ragged_inputs(T, k, d, 9090 + r)
    S0 = wl.random_tensor((d, r), 9191, device=DEV)
    S = S0.clone()
    lg.sketch_accumulate(X, dY, 77, r, S)
    rows = np.arange(0, d, 11)
    ref = _oracle_sketch(S0, [X], [dY], 77, r, k, rows=rows)
    assert_sketch_close(f64(S)[rows], ref)


LDS_PROJ_EDGES = [(1, 264, 8, 128), (17, 520, 33, 65), (63, 1029, 40, 256), (65, 777, 20, 200),
                  (130, 264, 7, 256), (300, 2056, 50, 96), (64, 1031, 9, 129),
                  # ranks 33-64 take it from 14 sign blocks of k on
                  (63, 3600, 40, 64), (130, 4100, 33, 50), (300, 5000, 20, 33)]


@pytest.mark.parametrize("T,k,d,r", LDS_PROJ_EDGES)
@pytest.mark.parametrize("env", [{}, {"LOGRA_PROJ_NK": 2}, {"LOGRA_PROJ_NK": 8}], ids=_plan_id)
def test_sketch_lds_projection_edges(T, k, d, r, env, monkeypatch):
    """The LDS-staged projection (ranks above 64 with k > 256; ranks 33-64
    with k > 3328) at its edges: token tiles of 1 to 130 tokens (rows past T
    staged as zero), k with a ragged last 256-column block and k % 8 != 0
    (the slab's boundary chunk masked element by element), r = 129 padded to
    256 columns, r = 33 padded to 64, and column splits (with NK = 8 on small
    k most splits hold no block at all)."""
    for k_, v_ in env.items():
        monkeypatch.setenv(k_, str(v_))
    _say("lds projection edges", T, k, d, r, env)
    seed = 900 + T + r
    X, dY = _ragged_inputs(T, k, d, 300 + T)
    S0 = wl.random_tensor((d, r), 7 + T, device=DEV)
    S = S0.clone()
    lg.sketch_accumulate(X, dY, seed, r, S)
    assert_sketch_close(f64(S), _oracle_sketch(S0, [X], [dY], seed, r, k))


@pytest.mark.parametrize("T,k,d,r", [(700, 1300, 300, 16), (4096, 1536, 1536, 64), (1000, 700, 900, 128),
                                     (2048, 3584, 3584, 256), (33, 264, 17, 5)])
def test_sketch_deterministic_mode(T, k, d, r):
    """With the deterministic setting, two accumulations of the same inputs
    give the same bits, through the fused and the split calls alike, and
    match the oracle."""
    _say("deterministic", T, k, d, r)
    X, dY = _ragged_inputs(T, k, d, 777 + r)
    prev = lg.set_deterministic(True)
    try:
        S1 = torch.zeros((d, r), dtype=torch.float32, device=DEV)
        S2 = torch.zeros_like(S1)
        lg.sketch_accumulate(X, dY, 3, r, S1)
        lg.sketch_accumulate(X, dY, 3, r, S1)
        lg.sketch_accumulate(X, dY, 3, r, S2)
        lg.sketch_accumulate(X, dY, 3, r, S2)
        P = lg.project(X, 3, r)
        S3 = torch.zeros_like(S1)
        lg.contract(dY, P, r, S3)
        lg.contract(dY, P, r, S3)
        torch.cuda.synchronize()
    finally:
        lg.set_deterministic(prev)
    assert torch.equal(S1, S2)
    assert torch.equal(S1, S3)
    rows = None if d <= 1000 else np.arange(0, d, 29)
    ref = _oracle_sketch(torch.zeros((d, r)), [X, X], [dY, dY], 3, r, k, rows=rows)
    assert_sketch_close(f64(S1) if rows is None else f64(S1)[rows], ref)


def test_sketch_additivity_and_empty():
    """M calls equal one call on the concatenated tokens (Algorithm 1 sums
    microbatch contributions); empty calls leave S bitwise unchanged."""
    T, k, d, r = 384, 768, 200, 64
    seed = 5
    parts = [_ragged_inputs(T, k, d, 300 + m) for m in range(3)]
    S1 = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    for X, dY in parts:
        lg.sketch_accumulate(X, dY, seed, r, S1)
    Xc = torch.cat([p[0] for p in parts]).contiguous()
    dYc = torch.cat([p[1] for p in parts]).contiguous()
    S2 = torch.zeros_like(S1)
    lg.sketch_accumulate(Xc, dYc, seed, r, S2)
    assert rel_frob(f64(S1), f64(S2)) < 1e-5
    before = S2.clone()
    lg.sketch_accumulate(Xc[:0], dYc[:0], seed, r, S2)
    lg.sketch_accumulate(Xc[:, :0], dYc, seed, r, S2)
    torch.cuda.synchronize()
    assert torch.equal(before, S2)


def test_sketch_seed_changes_result():
    T, k, d, r = 256, 512, 128, 16
    X, dY = _ragged_inputs(T, k, d, 77)
    S1 = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    S2 = torch.zeros_like(S1)
    lg.sketch_accumulate(X, dY, 0, r, S1)
    lg.sketch_accumulate(X, dY, 1, r, S2)
    # same dense gradient, different projections: <G, S A> = ||S||^2 for both
    G = f64(dY).T @ f64(X)
    for seed, S in ((0, S1), (1, S2)):
        A = oracle.rademacher_projection(seed, r, k)
        Sg = f64(S)
        assert math.isclose(float((G * (Sg @ A)).sum()), float((Sg * Sg).sum()), rel_tol=2e-4)
    assert rel_frob(f64(S1), f64(S2)) > 0.5


# ---------------------------------------------------------------------------
# Merge
# ---------------------------------------------------------------------------
def _oracle_merge(W, U, seed, r, k, scale):
    return oracle.merge_update(f64(W), f64(U), oracle.rademacher_projection(seed, r, k), scale)


def test_merge_tiny_workload():
    w = wl.WORKLOADS["tiny"]
    L = w.layers[0]
    r = w.ranks[0]
    seed = wl.sign_seed(0)
    _say("merge tiny")
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    for m in range(w.M):
        X, dY = wl.layer_inputs(w, 0, m, device=DEV)
        lg.sketch_accumulate(X, dY, seed, r, S)
    W = wl.layer_weight(w, 0, device=DEV)
    W0 = W.clone()
    lg.merge_update(W, S, seed, r, w.scales[0])
    ref = _oracle_merge(W0, S, seed, r, L.k, w.scales[0])
    e, frac = assert_weight_close(f64(W), ref, bound=update_error_bound(f64(S), r, w.scales[0]))
    _say("merge tiny rel err", e, "differing fraction", frac)
    assert frac < 0.01
    # the update is visible: W moved
    assert not torch.equal(W, W0)


@pytest.mark.parametrize(
    "d,k,r",
    [(1, 4, 1), (17, 260, 5), (130, 1000, 40), (64, 256, 256), (300, 516, 100), (1536, 1536, 64), (65, 2052, 128)],
)
def test_merge_ragged_and_zero_weight(d, k, r):
    _say("merge", d, k, r)
    seed = 31 + d + k
    U = wl.random_tensor((d, r), seed, device=DEV, std=3.0)
    scale = 1e-2
    # W = 0 isolates the low-rank update: W' = -RNE(c U A)
    W = torch.zeros((d, padded_ld(k, 4)), dtype=torch.bfloat16, device=DEV)[:, :k]
    lg.merge_update(W, U, seed, r, scale)
    ref = _oracle_merge(torch.zeros((d, k)), U, seed, r, k, scale)
    assert_weight_close(f64(W), ref, what="dW", bound=update_error_bound(f64(U), r, scale))
    # and on a real weight
    W = wl.gaussian_bf16((d, k), 0.02, seed + 1, device=DEV, ld=padded_ld(k, 4))
    W0 = W.clone()
    lg.merge_update(W, U, seed, r, 1e-4)
    assert_weight_close(f64(W), _oracle_merge(W0, U, seed, r, k, 1e-4), bound=update_error_bound(f64(U), r, 1e-4))


@pytest.mark.parametrize("d,k,r", [(70, 520, 37), (300, 1030, 64)])
def test_merge_unaligned_u_rows(d, k, r):
    """U as a strided view (row stride r + 3, base offset by one float): the
    kernel reads it element by element."""
    seed = 7 + d
    big = wl.random_tensor((d, r + 3), seed, device=DEV, std=2.0)
    U = big[:, 1 : r + 1]
    W = wl.gaussian_bf16((d, k), 0.02, seed + 1, device=DEV, ld=padded_ld(k, 4))
    W0 = W.clone()
    lg.merge_update(W, U, seed, r, 3e-3)
    assert_weight_close(f64(W), _oracle_merge(W0, U, seed, r, k, 3e-3), bound=update_error_bound(f64(U), r, 3e-3))


MERGE_PLANS = [
    {},
    {"LOGRA_MERGE_WGS": 1},
    {"LOGRA_MERGE_WGS": 100000},
    {"LOGRA_MERGE_NBW": 1, "LOGRA_MERGE_CB": 8, "LOGRA_MERGE_WGS": 7},
    {"LOGRA_MERGE_NBW": 2, "LOGRA_MERGE_CB": 4, "LOGRA_MERGE_WGS": 30},
    {"LOGRA_MERGE_NBW": 2, "LOGRA_MERGE_CB": 8},
    {"LOGRA_MERGE_NBW": 1, "LOGRA_MERGE_CB": 4},
]


@pytest.mark.parametrize("r", [16, 64, 100, 256])
@pytest.mark.parametrize("env", MERGE_PLANS, ids=_plan_id)
def test_merge_launch_plans(r, env, monkeypatch):
    """Every tiling of the merge (rows per wave, chunk width, column ranges that
    start inside a sign block or span several blocks) gives the oracle's W."""
    for k_, v_ in env.items():
        monkeypatch.setenv(k_, str(v_))
    d, k = 150, 1100
    seed = 77 + r
    _say("merge plans", r, env)
    U = wl.random_tensor((d, r), seed, device=DEV, std=2.0)
    W = wl.gaussian_bf16((d, k), 0.02, seed + 1, device=DEV, ld=padded_ld(k, 4))
    W0 = W.clone()
    lg.merge_update(W, U, seed, r, 1e-2)
    assert_weight_close(f64(W), _oracle_merge(W0, U, seed, r, k, 1e-2), bound=update_error_bound(f64(U), r, 1e-2))


def test_merge_scale_zero_and_zero_sketch_identity():
    d, k, r = 200, 700, 32
    W = wl.gaussian_bf16((d, k), 0.02, 3, device=DEV, ld=704)
    W0 = W.clone()
    U = wl.random_tensor((d, r), 4, device=DEV)
    lg.merge_update(W, U, 9, r, 0.0)
    lg.merge_update(W, torch.zeros_like(U), 9, r, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(W, W0)


def test_merge_linearity():
    d, k, r = 256, 1024, 64
    U = wl.random_tensor((d, r), 12, device=DEV)
    W1 = torch.zeros((d, k), dtype=torch.bfloat16, device=DEV)
    W2 = torch.zeros_like(W1)
    lg.merge_update(W1, U, 3, r, 2.0**-6)
    lg.merge_update(W2, U, 3, r, 2.0**-5)
    # a power-of-two scale only moves the exponent: exactly twice, bit for bit
    torch.cuda.synchronize()
    assert torch.equal(W2.float(), 2 * W1.float())


@pytest.mark.parametrize("key,layer", [("layer27b", 0), ("set7b", 2)])
def test_merge_full_size_sampled_rows(key, layer):
    w = wl.WORKLOADS[key]
    L = w.layers[layer]
    r = 256
    seed = wl.sign_seed(layer)
    _say("merge full size", key, L)
    U = wl.random_tensor((L.d, r), 99 + layer, device=DEV, std=50.0)
    rows = _sampled_rows(L.d, 64, 5 + layer)
    A = oracle.rademacher_projection(seed, r, L.k)
    Ur = f64(U)[rows]
    for scale in w.scales:
        W = wl.layer_weight(w, layer, device=DEV)
        Wr = f64(W)[rows]
        lg.merge_update(W, U, seed, r, scale)
        assert_weight_close(f64(W)[rows], oracle.merge_update(Wr, Ur, A, scale),
                            bound=update_error_bound(Ur, r, scale))
        del W


# ---------------------------------------------------------------------------
# RowAdam
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("beta2", [0.95, 0.999])
@pytest.mark.parametrize("d,r", [(256, 16), (3584, 64), (1000, 100), (7, 256), (18944, 256), (500, 30), (65, 1),
                                 (2048, 64), (2049, 48)])
def test_rowadam_three_steps(beta2, d, r):
    _say("rowadam", d, r, beta2)
    v = torch.zeros(d, dtype=torch.float32, device=DEV)
    v_ref = np.zeros(d)
    for t in range(1, 4):
        S = wl.random_tensor((d, r), 500 + t + d, device=DEV) * torch.logspace(
            -2, 2, d, device=DEV
        ).unsqueeze(1)
        S_in = f64(S)
        lg.rowadam_scale(S, v, t, beta2, 1e-8)
        # the library takes beta2 and eps_rel as float32: give the oracle the same values
        U_ref, v_ref = oracle.rowadam_scale(S_in, v_ref, t, float(np.float32(beta2)), float(np.float32(1e-8)))
        assert_sketch_close(f64(S), U_ref, what=f"U step {t}")
        assert rel_frob(f64(v), v_ref) < 1e-5
        # Frobenius norm of the sketch is preserved
        assert math.isclose(float(np.linalg.norm(f64(S))), float(np.linalg.norm(S_in)), rel_tol=1e-5)


@pytest.mark.parametrize("d,r,ld", [(700, 64, 67), (300, 128, 132), (41, 256, 260)])
def test_rowadam_strided_rows(d, r, ld):
    """Rows with a padded stride (the scalar path when a row is not 16-byte
    aligned, the float4 path when it is); the padding is left untouched."""
    _say("rowadam strided", d, r, ld)
    base = wl.random_tensor((d, ld), 900 + d, device=DEV)
    S = base[:, :r]
    pad = base[:, r:].clone()
    S_in = f64(S)
    v = torch.zeros(d, dtype=torch.float32, device=DEV)
    lg.rowadam_scale(S, v, 1, 0.95, 1e-8)
    U_ref, v_ref = oracle.rowadam_scale(S_in, np.zeros(d), 1, float(np.float32(0.95)), float(np.float32(1e-8)))
    assert_sketch_close(f64(S), U_ref, what="U")
    assert rel_frob(f64(v), v_ref) < 1e-5
    assert torch.equal(base[:, r:], pad)


def test_rowadam_zero_sketch_gives_zero_update():
    d, r = 300, 32
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    v = torch.rand(d, device=DEV)
    lg.rowadam_scale(S, v, 2, 0.95, 1e-8)
    torch.cuda.synchronize()
    assert not S.any()


# ---------------------------------------------------------------------------
# Whole step on the small workload: sketch, RowAdam, merge.
# ---------------------------------------------------------------------------
def test_full_step_tiny_with_rowadam():
    w = wl.WORKLOADS["tiny"]
    L = w.layers[0]
    r = w.ranks[0]
    seed = wl.sign_seed(0)
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    Xs, dYs = [], []
    for m in range(w.M):
        X, dY = wl.layer_inputs(w, 0, m, device=DEV)
        Xs.append(X)
        dYs.append(dY)
        lg.sketch_accumulate(X, dY, seed, r, S)
    v = torch.zeros(L.d, dtype=torch.float32, device=DEV)
    lg.rowadam_scale(S, v, 1, 0.999, 1e-8)
    W = wl.layer_weight(w, 0, device=DEV)
    W0 = W.clone()
    lg.merge_update(W, S, seed, r, w.scales[0])
    S_ref = _oracle_sketch(torch.zeros((L.d, r)), Xs, dYs, seed, r, L.k)
    U_ref, _ = oracle.rowadam_scale(S_ref, np.zeros(L.d), 1, float(np.float32(0.999)), float(np.float32(1e-8)))
    assert_sketch_close(f64(S), U_ref, what="U")
    W_ref = oracle.merge_update(f64(W0), U_ref, oracle.rademacher_projection(seed, r, L.k), w.scales[0])
    assert_weight_close(f64(W), W_ref, bound=update_error_bound(U_ref, r, w.scales[0]))


# ---------------------------------------------------------------------------
# Error paths with real device buffers
# ---------------------------------------------------------------------------
def test_stream_read_leaves_buffers_alone():
    """The streaming-read measurement aid reads and discards: neither the
    buffer nor (except for one xor value in 2^32) the sink changes."""
    t = wl.random_tensor((3, 1000), 5, device=DEV)  # 12000 bytes, a ragged last thread block
    t0 = t.clone()
    sink = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    lg.stream_read(t, sink)
    torch.cuda.synchronize()
    assert torch.equal(t, t0) and int(sink.item()) == -7


def test_errors_on_device_buffers():
    X, dY = _ragged_inputs(64, 256, 64, 1)
    S = torch.zeros((64, 16), dtype=torch.float32, device=DEV)
    with pytest.raises(lg.LograError) as ei:
        lg.sketch_accumulate(X[:, 1:], dY, 0, 16, S)  # misaligned base
    assert ei.value.status == 3
    buf = torch.zeros(64 * 256, dtype=torch.bfloat16, device=DEV)
    Xa = buf.view(64, 256)
    Sa = buf[: 2 * 64 * 16].view(torch.float32).view(64, 16)  # S overlapping X
    with pytest.raises(lg.LograError) as ei:
        lg.sketch_accumulate(Xa, dY, 0, 16, Sa)
    assert ei.value.status == 5
    with pytest.raises(lg.LograError):
        lg.sketch_accumulate(X, dY, 0, 513, torch.zeros((64, 513), device=DEV))
