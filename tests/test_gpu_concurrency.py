"""Concurrent use of the library on one GPU, against the float64 oracle.

The library keeps its scratch per (device, stream) and its settings
(precision, determinism, basis) per host thread.  These tests run sketches
of different shapes on two streams at once, and from two host threads with
their own streams and settings (the ctypes calls release the GIL, so the
host side overlaps too), and check every result against the oracle.
"""

import threading

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


def _inputs(T, k, d, seed, n):
    Xs = [wl.gaussian_bf16((T, k), 1.0, seed + 2 * m, device=DEV, ld=padded_ld(k)) for m in range(n)]
    dYs = [wl.gaussian_bf16((T, d), 1e-2, seed + 2 * m + 1, device=DEV, ld=padded_ld(d)) for m in range(n)]
    return Xs, dYs


def _ref(Xs, dYs, seed, r, k):
    A = oracle.rademacher_projection(seed, r, k)
    d = dYs[0].shape[1]
    return oracle.sketch_accumulate(np.zeros((d, r)), [f64(x) for x in Xs], [f64(y) for y in dYs], A)


# (T, k, d, r, seed): a column-split projection with the last-arriver sum
# (64), the LDS-staged projection (128) and a rank above 256 (two halves).
CASES = [(700, 1300, 300, 64, 11), (1000, 2056, 200, 128, 12), (300, 700, 90, 300, 13)]


def test_two_streams_interleaved():
    """Three microbatches of each shape, issued alternately on two streams
    that run concurrently; each stream's scratch serves only its own calls."""
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    jobs = []
    for j, (T, k, d, r, seed) in enumerate(CASES[:2]):
        Xs, dYs = _inputs(T, k, d, 100 * seed, 3)
        S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
        jobs.append((Xs, dYs, S, seed, r, k))
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for m in range(3):
        for s, (Xs, dYs, S, seed, r, k) in zip(streams, jobs):
            _say("streams", m, r)
            with torch.cuda.stream(s):
                lg.sketch_accumulate(Xs[m], dYs[m], seed, r, S)
    torch.cuda.synchronize()
    for Xs, dYs, S, seed, r, k in jobs:
        assert_sketch_close(f64(S), _ref(Xs, dYs, seed, r, k))


def test_host_threads_with_own_streams_and_settings():
    """Three host threads, each on its own stream and with its own settings
    (one deterministic, one contracting with the high bf16 half of P only,
    one with the defaults), run their sketches at the same time; each result
    matches the oracle within its mode's bound, and the deterministic one is
    bitwise equal to a second deterministic run."""
    torch.cuda.synchronize()
    data = []
    for T, k, d, r, seed in CASES:
        Xs, dYs = _inputs(T, k, d, 100 * seed + 7, 3)
        data.append((Xs, dYs, seed, r, k, d))
    torch.cuda.synchronize()
    out = [None] * len(data)
    errors = []
    modes = ["det", "hi_only", "default"]

    def work(idx):
        try:
            Xs, dYs, seed, r, k, d = data[idx]
            mode = modes[idx]
            prev_det = lg.set_deterministic(mode == "det")
            prev_prec = lg.set_precision(lg.PRECISION_BF16 if mode == "hi_only" else lg.PRECISION_BF16X2)
            try:
                s = torch.cuda.Stream()
                with torch.cuda.stream(s):
                    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
                    for m in range(3):
                        lg.sketch_accumulate(Xs[m], dYs[m], seed, r, S)
                s.synchronize()
                out[idx] = S
            finally:
                lg.set_deterministic(prev_det)
                lg.set_precision(prev_prec)
        except Exception as e:  # reported on the main thread
            errors.append((idx, e))

    threads = [threading.Thread(target=work, args=(idx,)) for idx in range(len(data))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for idx, (Xs, dYs, seed, r, k, d) in enumerate(data):
        _say("thread", modes[idx], r)
        ref = _ref(Xs, dYs, seed, r, k)
        # single-bf16 P carries about 1.7e-3 relative error (within the 2e-3
        # bound); the other modes keep the hi/lo pair's tight bound
        assert_sketch_close(f64(out[idx]), ref, tight=modes[idx] != "hi_only")
    # the deterministic thread's sketch again, on this thread: bitwise equal
    Xs, dYs, seed, r, k, d = data[0]
    prev = lg.set_deterministic(True)
    try:
        S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
        for m in range(3):
            lg.sketch_accumulate(Xs[m], dYs[m], seed, r, S)
        torch.cuda.synchronize()
    finally:
        lg.set_deterministic(prev)
    assert torch.equal(S, out[0])
