"""GPU parity at ranks 257-512, through the C ABI.

Above rank 256 the library runs the sketch as two column halves (sign rows
0..255 and 256..r-1) and the merge with a 16-step loop over r.  Every call is
compared with the float64 oracle, which knows nothing of halves: the sketch,
the split calls (the cache is decoded half by half per the documented
layout), the merge and grouped merge, RowAdam, the deterministic mode and the
no-allocation entry point.
"""

import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import (
    S_TIGHT,
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


def _inputs(T, k, d, seed):
    X = wl.gaussian_bf16((T, k), 1.0, seed, device=DEV, ld=padded_ld(k))
    dY = wl.gaussian_bf16((T, d), 1e-2, seed + 1, device=DEV, ld=padded_ld(d))
    return X, dY


SHAPES = [(700, 1300, 300, 300), (1500, 700, 900, 512), (4096, 5120, 600, 512), (33, 264, 17, 257),
          (1000, 2056, 200, 400)]


@pytest.mark.parametrize("T,k,d,r", SHAPES)
def test_sketch_above_256(T, k, d, r):
    _say("sketch r>256", T, k, d, r)
    seed = 900 + r
    X, dY = _inputs(T, k, d, 10 + r)
    X2, dY2 = _inputs(T, k, d, 20 + r)
    S0 = wl.random_tensor((d, r), 30 + r, device=DEV)
    S = S0.clone()
    lg.sketch_accumulate(X, dY, seed, r, S)
    lg.sketch_accumulate(X2, dY2, seed, r, S)
    A = oracle.rademacher_projection(seed, r, k)
    ref = oracle.sketch_accumulate(f64(S0), [f64(X), f64(X2)], [f64(dY), f64(dY2)], A)
    e = assert_sketch_close(f64(S), ref)
    _say("S rel err", e)


def test_sketch_above_256_strided_s():
    # S as the left columns of a wider buffer (lds > r): the upper half
    # starts 256 columns in.
    T, k, d, r = 600, 900, 250, 320
    X, dY = _inputs(T, k, d, 3)
    buf = torch.full((d, 400), 7.0, dtype=torch.float32, device=DEV)
    S = buf[:, :r]
    S.zero_()
    lg.sketch_accumulate(X, dY, 5, r, S)
    torch.cuda.synchronize()
    ref = oracle.sketch_accumulate(np.zeros((d, r)), [f64(X)], [f64(dY)], oracle.rademacher_projection(5, r, k))
    assert_sketch_close(f64(S), ref)
    assert bool((buf[:, r:] == 7.0).all()), "columns past r were written"


def test_sketch_above_256_deterministic_and_noalloc():
    T, k, d, r = 1500, 1300, 700, 512
    X, dY = _inputs(T, k, d, 44)
    prev = lg.set_deterministic(True)
    try:
        S1 = torch.zeros((d, r), dtype=torch.float32, device=DEV)
        S2 = torch.zeros_like(S1)
        lg.sketch_accumulate(X, dY, 8, r, S1)
        lg.sketch_accumulate(X, dY, 8, r, S2)
        torch.cuda.synchronize()
        assert torch.equal(S1, S2)
    finally:
        lg.set_deterministic(prev)
    ref = oracle.sketch_accumulate(np.zeros((d, r)), [f64(X)], [f64(dY)], oracle.rademacher_projection(8, r, k))
    assert_sketch_close(f64(S1), ref)
    S3 = torch.zeros_like(S1)
    lg.sketch_accumulate(X, dY, 8, r, S3, noalloc=True)
    torch.cuda.synchronize()
    assert rel_frob(f64(S3), f64(S1)) <= S_TIGHT


def _cache_cols(r):
    nb = (r + 15) // 16
    q = 1
    while q < nb:
        q *= 2
    return 16 * q


def _decode_half(raw, T, r):
    R = _cache_cols(r)
    Tc = (T + 255) // 256 * 256
    T32 = (T + 31) // 32 * 32
    t = np.arange(T32)[:, None]
    c = np.arange(r)[None, :]
    idx = ((((t // 32) * (R // 16) + c // 16) * 64 + ((t % 32) // 8) * 16 + c % 16) * 8 + t % 8)
    vals = oracle.bf16_bits_to_f64(raw[idx]) + oracle.bf16_bits_to_f64(raw[Tc * R + idx])
    return vals[:T], vals[T:], 2 * Tc * R  # values, padding tokens, uint16 entries used


def decode_cache(P, T, r):
    """(T, r) values of a projection cache of rank up to 512: the cache of
    columns 0..255, then a cache of rank r - 256, per the documented layout."""
    raw = P.cpu().numpy().view(np.uint16)
    if r <= 256:
        v, pad, _ = _decode_half(raw, T, r)
        return v, pad
    v0, p0, n0 = _decode_half(raw, T, 256)
    v1, p1, _ = _decode_half(raw[n0:], T, r - 256)
    return np.concatenate([v0, v1], axis=1), np.concatenate([p0, p1], axis=1)


@pytest.mark.parametrize("T,k,d,r", [(700, 1300, 300, 300), (1000, 700, 900, 512), (33, 264, 17, 257)])
def test_split_above_256(T, k, d, r):
    _say("split r>256", T, k, d, r)
    X, dY = _inputs(T, k, d, 60 + r)
    P = lg.project(X, 14, r)
    assert P.numel() == lg.projection_bytes(T, r)
    got, pad = decode_cache(P, T, r)
    A = oracle.rademacher_projection(14, r, k)
    assert rel_frob(got, oracle.project_inputs(f64(X), A) * math.sqrt(r)) <= 2e-5
    np.testing.assert_array_equal(pad, np.zeros_like(pad))
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    lg.contract(dY, P, r, S)
    ref = oracle.sketch_accumulate(np.zeros((d, r)), [f64(X)], [f64(dY)], A)
    assert_sketch_close(f64(S), ref)
    # the fused call adds the same
    S2 = torch.zeros_like(S)
    lg.sketch_accumulate(X, dY, 14, r, S2)
    torch.cuda.synchronize()
    assert rel_frob(f64(S2), f64(S)) <= S_TIGHT


@pytest.mark.parametrize("d,k,r", [(300, 1030, 300), (70, 520, 512), (1000, 5120, 512), (129, 2000, 257)])
def test_merge_above_256(d, k, r):
    _say("merge r>256", d, k, r)
    for scale in (1e-3, -2e-2):
        W = wl.gaussian_bf16((d, k), 0.02, 5 + d, device=DEV, ld=padded_ld(k, 4))
        U = wl.random_tensor((d, r), 6 + r, device=DEV)
        W0 = f64(W)
        lg.merge_update(W, U, 70 + r, r, scale)
        A = oracle.rademacher_projection(70 + r, r, k)
        assert_weight_close(f64(W), oracle.merge_update(W0, f64(U), A, scale),
                            bound=update_error_bound(f64(U), r, scale))
    # W = 0 isolates the update: RNE(-scale U A / sqrt r) element by element
    W = torch.zeros((d, padded_ld(k, 4)), dtype=torch.bfloat16, device=DEV)[:, :k]
    lg.merge_update(W, U, 70 + r, r, 1e-2)
    assert_weight_close(f64(W), oracle.merge_update(np.zeros((d, k)), f64(U), A, 1e-2),
                        bound=update_error_bound(f64(U), r, 1e-2))


def test_grouped_merge_above_256_equals_separate():
    r = 512
    shapes = [(300, 1032, 1e-3), (64, 520, 2e-3), (1000, 2048, -1e-3)]
    items = []
    for j, (d, k, scale) in enumerate(shapes):
        W = wl.gaussian_bf16((d, k), 0.02, 300 + j, device=DEV)
        U = wl.random_tensor((d, r), 310 + j, device=DEV)
        items.append((W, U, 400 + j, scale))
    alone = [W.clone() for W, _, _, _ in items]
    for (W, U, seed, scale), Wa in zip(items, alone):
        lg.merge_update(Wa, U, seed, r, scale)
    lg.merge_update_grouped(items, r)
    torch.cuda.synchronize()
    for (W, _, _, _), Wa in zip(items, alone):
        assert torch.equal(W, Wa)


def test_rowadam_rank_512():
    d, r = 1000, 512
    S = wl.random_tensor((d, r), 91, device=DEV)
    v = torch.zeros(d, dtype=torch.float32, device=DEV)
    v_ref = np.zeros(d)
    for t in (1, 2, 3):
        S_t = S * (1.0 + 0.5 * t)
        S_ref = f64(S_t)
        lg.rowadam_scale(S_t, v, t, 0.95, 1e-8)
        U_ref, v_ref = oracle.rowadam_scale(S_ref, v_ref, t, float(np.float32(0.95)), float(np.float32(1e-8)))
        assert_sketch_close(f64(S_t), U_ref, what=f"U t={t}")


def test_full_size_rank_512_sampled_rows():
    """The 27B-class attention layer (5120 x 5120, 16384 tokens) at r = 512:
    sketch on sampled rows of S, then a merge (random U of the size RowAdam
    leaves) on sampled rows of W."""
    w = wl.WORKLOADS["layer27b"]
    L = w.layers[0]
    r, seed = 512, 0
    X, dY = wl.layer_inputs(w, 0, 0, device=DEV)
    S = torch.zeros((L.d, r), dtype=torch.float32, device=DEV)
    lg.sketch_accumulate(X, dY, seed, r, S)
    rows = np.sort(np.random.default_rng(5).choice(L.d, size=96, replace=False))
    rows_t = torch.as_tensor(rows, device=DEV)
    A = oracle.rademacher_projection(seed, r, L.k)
    ref = oracle.sketch_from_gradient(f64(dY[:, rows_t]).T @ f64(X), A)
    assert_sketch_close(f64(S[rows_t]), ref)
    del X, dY
    W = wl.layer_weight(w, 0, device=DEV)
    Wr = f64(W[rows_t])
    U = wl.random_tensor((L.d, r), 77, device=DEV, std=50.0)
    lg.merge_update(W, U, seed, r, 1e-5)
    Ur = f64(U[rows_t])
    assert_weight_close(f64(W[rows_t]), oracle.merge_update(Wr, Ur, A, 1e-5), bound=update_error_bound(Ur, r, 1e-5))
