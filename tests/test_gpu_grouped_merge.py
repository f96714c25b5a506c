"""GPU tests of the grouped merge (several matrices of one rank in one
launch), through the C ABI.

The trainer merges a layer's matrices and the rollout side applies the same
received factors to its own copy of the weights (Algorithm 1; section 2.2):
both must end bitwise identical.  Here every W merged in a group must equal,
bit for bit, the same W merged alone by logra_merge_update, and one group is
also checked against the float64 oracle.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from tests._util import assert_weight_close, f64, update_error_bound

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


def _pad(n, m=8):
    return (n + m - 1) // m * m


def _items(shapes, r, seed0):
    items = []
    for j, (d, k, scale) in enumerate(shapes):
        W = wl.gaussian_bf16((d, k), 0.02, seed0 + 10 * j, device=DEV, ld=_pad(k))
        U = wl.random_tensor((d, r), seed0 + 10 * j + 1, device=DEV)
        items.append((W, U, 1000 + j, scale))
    return items


LAYER_1P5B = [(1536, 1536, 1e-3), (256, 1536, 2e-3), (256, 1536, 5e-4), (1536, 1536, 1e-3),
              (8960, 1536, 1e-3), (8960, 1536, 1e-3), (1536, 8960, 1e-3)]


@pytest.mark.parametrize("r", [16, 64, 128, 256])
def test_grouped_equals_separate_bitwise(r):
    """A 1.5B-class layer's seven matrices (q, k, v, o, gate, up, down shapes)."""
    _say("grouped vs separate", r)
    items = _items(LAYER_1P5B, r, 40 + r)
    alone = [W.clone() for W, _, _, _ in items]
    for (W, U, seed, scale), Wa in zip(items, alone):
        lg.merge_update(Wa, U, seed, r, scale)
    lg.merge_update_grouped(items, r)
    torch.cuda.synchronize()
    for j, ((W, _, _, _), Wa) in enumerate(zip(items, alone)):
        assert torch.equal(W, Wa), f"item {j} differs from its separate merge"
        assert not torch.equal(W, wl.gaussian_bf16(tuple(W.shape), 0.02, 40 + r + 10 * j, device=DEV)), "W unchanged"


def test_grouped_ragged_skips_and_many_launches():
    """Ragged shapes, skipped items (scale 0, empty), and more than sixteen
    matrices (several launches)."""
    r = 40
    shapes = [(1 + 37 * j, 8 + 120 * (j % 5), 1e-2 * (1 + j % 3)) for j in range(19)]
    shapes[3] = (200, 300, 0.0)
    items = _items(shapes, r, 7)
    ref = [W.clone() for W, _, _, _ in items]
    for (W, U, seed, scale), Wa in zip(items, ref):
        lg.merge_update(Wa, U, seed, r, scale)
    empty = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    lg.merge_update_grouped(items[:10] + [(empty, torch.empty((0, r), device=DEV), 5, 1.0)] + items[10:], r)
    torch.cuda.synchronize()
    for j, ((W, _, _, _), Wa) in enumerate(zip(items, ref)):
        assert torch.equal(W, Wa), f"item {j}"


def test_grouped_matches_oracle():
    r = 64
    shapes = [(300, 520, 1e-2), (129, 264, -3e-3), (64, 1000, 5e-3)]
    items = _items(shapes, r, 99)
    W0 = [f64(W) for W, _, _, _ in items]
    lg.merge_update_grouped(items, r)
    torch.cuda.synchronize()
    for (W, U, seed, scale), w0 in zip(items, W0):
        A = oracle.rademacher_projection(seed, r, W.shape[1])
        ref = oracle.merge_update(w0, f64(U), A, scale)
        assert_weight_close(f64(W), ref, bound=update_error_bound(f64(U), r, scale))


def test_sync_apply_trainer_and_receiver_agree():
    """Trainer and rollout copies of a layer, merged from the same factors
    and seeds (one grouped call each), stay bitwise identical."""
    r = 128
    items = _items(LAYER_1P5B, r, 5)
    recv = [(W.clone(), U.clone(), seed, scale) for W, U, seed, scale in items]
    lg.merge_update_grouped(items, r)
    lg.merge_update_grouped(recv, r)
    torch.cuda.synchronize()
    for (W, _, _, _), (Wr, _, _, _) in zip(items, recv):
        assert torch.equal(W, Wr)
    np.testing.assert_array_equal(f64(items[0][1]), f64(recv[0][1]))
