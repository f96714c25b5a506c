"""Benchmark of the LoGRA per-layer hot path on one MI355X.

One step = one training step of one layer as Algorithm 1 of the LoGRA paper
runs it on the trainer: S <- 0, M sketch-accumulate calls (one per
microbatch), the fused expand-and-merge of W.  Inputs for every microbatch
are already resident in HBM; several distinct input sets rotate so that the
working set exceeds the 256 MB last-level (MALL) cache and each step streams
its inputs from HBM.

Prints ONE JSON line (rank 0): whole-step tokens/s of the layer, plus
  roofline     the sketch-accumulate call (projection + contraction kernels)
               against MI355X's 8 TB/s HBM peak: HIP events on the kernels'
               stream around M*K back-to-back calls over the rotating inputs,
               queued behind a sleep kernel so that they measure GPU time;
  merge        the fused merge against the same peak;
  rowadam      the optional RowAdam scaling of S (three small kernels);
  split        the forward/backward halves of a sketch call (project, contract);
  grouped_merge a 1.5B-class layer's seven merges in one launch vs seven;
  predicted_kl the predicted-KL reduction over a 2048 x 151,936 probe;
  cpu_baseline the float64 CPU oracle timed on this host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload layer27b --layer 1]
       python bench.py --sweep    (per-layer table, one JSON line per layer and rank)
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
CSRC = os.path.join(ROOT, "rank_gradient_sketching_accumulate_amd", "csrc")
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
MALL_BYTES = 256 * 2**20


def kernel_source_sha() -> str:
    """Hash of the library's sources with comments and trailing blanks
    stripped: a profile taken under the same code keeps matching after an
    edit of comments only."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(text.encode())
    return h.hexdigest()[:16]


def padded_rank(r):
    """Columns of P the kernels compute: 16-column blocks rounded up to a power
    of two, ranks above 256 as a 256-column half plus the rest."""
    def pow2_cols(n):
        b = 1
        while 16 * b < n:
            b *= 2
        return 16 * b
    return pow2_cols(r) if r <= 256 else 256 + pow2_cols(r - 256)


def sketch_bytes(T, k, d, r):
    """Algorithmic HBM bytes of one sketch call: X and dY read once (bf16),
    S read and written once (fp32)."""
    return 2 * T * (k + d) + 8 * d * r


def merge_bytes(d, k, r):
    """W read and written once (bf16), U read once (fp32)."""
    return 4 * d * k + 4 * d * r


def load_traffic(workload: str, layer: str, r: int, precision: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary:
    (bytes per sketch call, bytes per merge or None).  Both are None unless
    the summary was taken on the current kernel sources for this layer, rank
    and precision mode."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        t = json.load(f)
    if (t.get("kernel_source_sha") != kernel_source_sha() or t.get("layer") != layer or t.get("r") != r
            or t.get("precision") != precision):
        return None, None
    merge = [v for k, v in t.get("kernels", {}).items() if k.startswith("logra::merge_kernel")]
    return t.get("sketch_call_bytes"), (merge[0] if len(merge) == 1 else None)


def gpu_time_per_call(torch, stream, fn, n):
    """(GPU seconds, host seconds) per call of fn(i), i < n, issued back to
    back.  The loop runs once untimed (which also measures how fast the host
    issues it), then again behind a sleep kernel long enough for the host to
    queue every call before the first timed launch, so the HIP events on
    `stream` see GPU time only."""
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(n):
        fn(i)
    host = time.perf_counter() - h0
    torch.cuda.synchronize()
    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is not None:
        sleep(int(min(2.4e9, max(2.4e6, 3.0 * host * 2.4e9))))  # cycles at about 2.4 GHz
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    h0 = time.perf_counter()
    for i in range(n):
        fn(i)
    host = time.perf_counter() - h0
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n * 1e-3, host / n


def proj_cols(r):
    """Columns of the projection cache: 16 times the next power of two of ceil(r / 16)."""
    nb, q = (r + 15) // 16, 1
    while q < nb:
        q *= 2
    return 16 * q


def rowadam_bytes(d, r):
    """Algorithmic HBM bytes of RowAdam: S read twice and written once (fp32),
    v read and written once."""
    return 12 * d * r + 8 * d


def rowadam_time(torch, lg, stream, S, calls: int):
    """GPU time per RowAdam call over copies of S (each call rescales its copy
    in place; the values stay finite because the rescale keeps the norm)."""
    d, r = S.shape
    n = max(2, math.ceil(2.5 * MALL_BYTES / (4 * d * r)))
    Us = [S.clone() for _ in range(n)]
    vs = [torch.zeros(d, dtype=torch.float32, device=S.device) for _ in range(n)]
    t, h = gpu_time_per_call(torch, stream, lambda i: lg.rowadam_scale(Us[i % n], vs[i % n], 1 + i // n, 0.999, 1e-8),
                             max(calls, 2 * n))
    del Us, vs
    return t, h


def split_bytes(T, k, d, r):
    """Algorithmic HBM bytes of the split calls: the projection reads X and
    writes the cache (a bf16 hi/lo pair per entry); the contraction reads dY
    and the cache and reads and writes S."""
    R = proj_cols(r)
    return 2 * T * k + 4 * T * R, 2 * T * d + 4 * T * R + 8 * d * r


def kl_bytes(n, V, esz):
    """Algorithmic HBM bytes of one predicted-KL call: z and zdot read once,
    one float per row and q written."""
    return 2 * n * V * esz + 4 * n + 4


def predicted_kl_timing(torch, lg, wl, stream, dev, calls: int):
    """Predicted KL over the probe workload (2048 contexts x 151,936 tokens),
    fp32 and bf16, timed like the sketch calls."""
    out = {}
    n, V = wl.KL_CONTEXTS, wl.KL_VOCAB
    for name, dt, esz in (("fp32", torch.float32, 4), ("bf16", torch.bfloat16, 2)):
        per = 2 * n * V * esz
        ncopy = max(1, math.ceil(2.5 * MALL_BYTES / per))
        ins = [wl.kl_inputs(n, V, 500 + c, device=dev, dtype=dt) for c in range(ncopy)]
        rv = torch.empty(n, dtype=torch.float32, device=dev)
        q = torch.empty(1, dtype=torch.float32, device=dev)
        t, h = gpu_time_per_call(torch, stream, lambda i: lg.predicted_kl(ins[i % ncopy][0], ins[i % ncopy][1], 1.0,
                                                                          row_var=rv, q=q), calls)
        # the GPU's streaming-read time for the same two arrays (two launches)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        t_rd, _ = gpu_time_per_call(torch, stream, lambda i: (lg.stream_read(ins[i % ncopy][0], sink),
                                                              lg.stream_read(ins[i % ncopy][1], sink)), calls)
        b = kl_bytes(n, V, esz)
        out[name] = {"avg_us": t * 1e6, "achieved": b / t / 1e9, "frac": b / t / 1e9 / HBM_PEAK_GBS,
                     "algorithmic_bytes": b, "host_us_per_call": h * 1e6,
                     "read_ceiling_us": t_rd * 1e6, "frac_of_read_ceiling": t_rd / t}
        del ins
        torch.cuda.empty_cache()
    return {
        "kernel": "kl_rows_kernel + kl_finalize_kernel",
        "workload": f"predicted-KL probe: {n} contexts x {V}-token vocabulary, logits and score rates",
        "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s", **out,
    }


def grouped_merge_timing(torch, lg, wl, stream, dev, calls: int, r: int = 128, scale: float = 1e-5):
    """A 1.5B-class layer's seven sketched matrices (q, k, v, o: 1536 x 1536
    and 256 x 1536; gate, up: 8960 x 1536; down: 1536 x 8960) merged by one
    grouped launch and by seven separate merges, over enough copies of the
    layer's weights to exceed the MALL."""
    shapes = [(1536, 1536), (256, 1536), (256, 1536), (1536, 1536), (8960, 1536), (8960, 1536), (1536, 8960)]
    per = sum(2 * d * k for d, k in shapes)
    ncopy = max(2, math.ceil(2.5 * MALL_BYTES / per))
    Us = [wl.random_tensor((d, r), 900 + j, device=dev) for j, (d, k) in enumerate(shapes)]
    Ws = [[wl.gaussian_bf16((d, k), 0.02, 800 + j, device=dev) for j, (d, k) in enumerate(shapes)]]
    for _ in range(ncopy - 1):
        Ws.append([W.clone() for W in Ws[0]])
    items = [[(Ws[c][j], Us[j], 100 + j, scale) for j in range(len(shapes))] for c in range(ncopy)]
    t_g, _ = gpu_time_per_call(torch, stream, lambda i: lg.merge_update_grouped(items[i % ncopy], r), calls)

    def separate(i):
        for W, U, seed, sc in items[i % ncopy]:
            lg.merge_update(W, U, seed, r, sc)

    t_s, _ = gpu_time_per_call(torch, stream, separate, calls)
    b = sum(merge_bytes(d, k, r) for d, k in shapes)
    del Ws, items
    torch.cuda.empty_cache()
    return {
        "kernel": "merge_group_kernel",
        "workload": f"1.5B-class layer, 7 matrices, r={r}",
        "grouped_us": t_g * 1e6, "separate_us": t_s * 1e6,
        "achieved": b / t_g / 1e9, "frac": b / t_g / 1e9 / HBM_PEAK_GBS,
        "separate_frac": b / t_s / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": b,
        "unit": "GB/s", "peak": HBM_PEAK_GBS, "weight_copies_rotated": ncopy,
    }


def gpu_time_reps(torch, stream, fn, n, reps):
    """Per-call GPU seconds of `reps` separate repetitions of n back-to-back
    calls fn(i) (each repetition queued behind its own sleep kernel, timed
    with HIP events on `stream`): returns the sorted list."""
    out = []
    for rep in range(reps):
        t, _ = gpu_time_per_call(torch, stream, lambda i: fn(rep * n + i), n)
        out.append(t)
    return sorted(out)


def quantiles_us(ts):
    """p10, median and p90 of a sorted list of seconds, in microseconds."""
    def q(f):
        x = f * (len(ts) - 1)
        lo = int(math.floor(x))
        hi = min(lo + 1, len(ts) - 1)
        return (ts[lo] + (ts[hi] - ts[lo]) * (x - lo)) * 1e6
    return {"p10_us": q(0.1), "median_us": q(0.5), "p90_us": q(0.9), "repetitions": len(ts)}


def cpu_baseline(w, layer, r, seed, budget_s: float):
    """Time the float64 oracle (as it stands) on host copies of the
    workload's microbatches: the dense gradient G = dY^T X, then the
    projection.  On a large layer the oracle forms a seeded subset of the rows
    of G (rows of S are independent), and the rate is scaled to the whole
    layer: tokens/s = T * rows / (d * seconds)."""
    import numpy as np
    import torch

    import oracle
    import workloads as wl

    blas, threads = "unknown", os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info

        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            threads = max(p.get("num_threads", 1) for p in info)
            blas = ",".join(sorted({str(p.get("internal_api")) for p in info}))
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    L = w.layers[layer]
    A = oracle.rademacher_projection(seed, r, L.k)
    rows_n = min(L.d, 256)
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(L.d, size=rows_n, replace=False)) if rows_n < L.d else None
    host = []
    for m in range(min(w.M, 2)):
        X, dY = wl.layer_inputs(w, layer, m, device="cpu")
        host.append((X.float().numpy().astype(np.float64), dY.float().numpy().astype(np.float64)))
    S = np.zeros((L.d, r))
    tokens = 0
    t0 = time.perf_counter()
    n = 0
    while True:
        Xh, dYh = host[n % len(host)]
        oracle.sketch_accumulate(S, [Xh], [dYh], A, rows=rows)
        tokens += Xh.shape[0]
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    frac = (rows_n / L.d) if rows is not None else 1.0
    return {
        "value": tokens * frac / dt,
        "unit": "tokens/s/layer",
        "cores": int(threads),
        "affinity_cores": int(affinity),
        "blas": blas,
        "kind": "oracle",
        "sample": f"{n} microbatch sketch(es) of {w.T} tokens of the {L.name} {L.d}x{L.k} layer, r={r}, "
                  f"{'all' if rows is None else rows_n} of {L.d} rows of S: dense fp64 G rows = dY^T X, then G A^T; "
                  f"{dt:.1f} s of host time, rate scaled to all {L.d} rows",
    }


def sweep(steps: int):
    """Per-layer table: every layer and rank of every workload, one JSON line
    each.  Sketch calls are timed back to back over enough distinct seeded
    inputs to exceed the MALL; merges over enough copies of W."""
    import torch

    import rank_gradient_sketching_accumulate_amd as lg
    import workloads as wl

    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    seen = set()
    for name, w in wl.WORKLOADS.items():
        for li, L in enumerate(w.layers):
            for r in w.ranks:
                key = (w.T, L.d, L.k, r)
                if key in seen:
                    continue
                seen.add(key)
                T, d, k = w.T, L.d, L.k
                per = 2 * T * (k + d)
                ns = max(1, math.ceil(2.5 * MALL_BYTES / per))
                ins = [wl.layer_inputs(w, li, m, device=dev) for m in range(ns)]
                S = torch.zeros((d, r), dtype=torch.float32, device=dev)
                seed = wl.sign_seed(li)
                n = max(steps, 2 * ns)
                t_call, _ = gpu_time_per_call(
                    torch, stream, lambda j: lg.sketch_accumulate(ins[j % ns][0], ins[j % ns][1], seed, r, S), n)
                del ins
                torch.cuda.empty_cache()
                n_w = max(2, math.ceil(2.5 * MALL_BYTES / (2 * d * k)))
                Ws = [wl.layer_weight(w, li, device=dev) for _ in range(min(n_w, 4))]
                while len(Ws) < n_w:
                    Ws.append(Ws[len(Ws) % 4].clone())
                nm = max(steps, 2 * n_w)
                t_merge, _ = gpu_time_per_call(
                    torch, stream, lambda j: lg.merge_update(Ws[j % n_w], S, seed, r, w.scales[-1]), nm)
                prev = lg.set_precision(PRECISIONS["bf16"])
                try:
                    t_merge1, _ = gpu_time_per_call(
                        torch, stream, lambda j: lg.merge_update(Ws[j % n_w], S, seed, r, w.scales[-1]), nm)
                finally:
                    lg.set_precision(prev)
                t_ra, _ = rowadam_time(torch, lg, stream, S, steps)
                del Ws, S
                torch.cuda.empty_cache()
                sb, mb = sketch_bytes(T, k, d, r), merge_bytes(d, k, r)
                print(json.dumps({
                    "workload": name, "layer": L.name, "T": T, "d": d, "k": k, "r": r,
                    "sketch_call_us": t_call * 1e6, "sketch_tokens_per_s": T / t_call,
                    "sketch_GBps": sb / t_call / 1e9, "sketch_frac": sb / t_call / 1e9 / HBM_PEAK_GBS,
                    "merge_us": t_merge * 1e6, "merge_GBps": mb / t_merge / 1e9,
                    "merge_frac": mb / t_merge / 1e9 / HBM_PEAK_GBS,
                    "merge_bf16_us": t_merge1 * 1e6, "merge_bf16_frac": mb / t_merge1 / 1e9 / HBM_PEAK_GBS,
                    "rowadam_us": t_ra * 1e6, "rowadam_GBps": rowadam_bytes(d, r) / t_ra / 1e9,
                    "kernel_source_sha": kernel_source_sha(),
                }), flush=True)


def layer_rates(torch, lg, wl, stream, dev, w, li, r, calls, precisions=("bf16x2", "bf16")):
    """Sketch-call and merge timing of one layer (HBM-resident inputs, enough
    distinct microbatches to exceed the MALL), per precision mode."""
    L = w.layers[li]
    T, d, k = w.T, L.d, L.k
    ns = max(2, math.ceil(2.5 * MALL_BYTES / (2 * T * (k + d))))
    ins = [wl.layer_inputs(w, li, m, device=dev) for m in range(ns)]
    S = torch.zeros((d, r), dtype=torch.float32, device=dev)
    seed = wl.sign_seed(li)
    out = {"layer": f"{L.name} d={d} k={k}", "T": T, "r": r}
    sb = sketch_bytes(T, k, d, r)
    for prec in precisions:
        prev = lg.set_precision(PRECISIONS[prec])
        try:
            t, _ = gpu_time_per_call(torch, stream, lambda j: lg.sketch_accumulate(ins[j % ns][0], ins[j % ns][1],
                                                                                     seed, r, S), max(calls, 2 * ns))
        finally:
            lg.set_precision(prev)
        out[f"sketch_{prec}"] = {"us": t * 1e6, "GBps": sb / t / 1e9, "frac": sb / t / 1e9 / HBM_PEAK_GBS,
                                 "tokens_per_s": T / t}
    del ins
    torch.cuda.empty_cache()
    n_w = max(2, math.ceil(2.5 * MALL_BYTES / (2 * d * k)))
    Ws = [wl.layer_weight(w, li, device=dev) for _ in range(n_w)]
    mb = merge_bytes(d, k, r)
    for prec in precisions:
        prev = lg.set_precision(PRECISIONS[prec])
        try:
            t, _ = gpu_time_per_call(torch, stream, lambda j: lg.merge_update(Ws[j % n_w], S, seed, r, w.scales[-1]),
                                     max(calls, 2 * n_w))
        finally:
            lg.set_precision(prev)
        key = "merge" if prec == "bf16x2" else f"merge_{prec}"
        out[key] = {"us": t * 1e6, "GBps": mb / t / 1e9, "frac": mb / t / 1e9 / HBM_PEAK_GBS}
    del Ws, S
    torch.cuda.empty_cache()
    return out


PRECISIONS = {"bf16x2": 0, "bf16": 1}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="layer27b")
    ap.add_argument("--layer", type=int, default=1)
    ap.add_argument("--rank", type=int, default=0, help="rank r (default: the workload's first)")
    ap.add_argument("--precision", default="bf16x2", choices=sorted(PRECISIONS),
                    help="contraction precision of the timed step (bf16x2: P as a bf16 high/low pair)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kl", action="store_true", help="skip the predicted-KL probe timing")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline step, sketch call and merge (for profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a 1 GiB device copy (for counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="per-layer table over every workload, layer and rank (one JSON line each)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(
            "bench.py measures one GPU: the library has no multi-GPU path "
            "(the sketch is additive over tokens; sharding is described in the design notes).",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    import rank_gradient_sketching_accumulate_amd as lg
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    lg.load_library()

    if args.sweep:
        sweep(args.steps)
        return

    if args.calibrate_copy:
        n = 2**29  # 1 GiB of int16
        a = torch.ones(n, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 2 * n, "copies": 3}))
        return

    w = wl.WORKLOADS[args.workload]
    L = w.layers[args.layer]
    r = args.rank or w.ranks[0]
    T, M, d, k = w.T, w.M, L.d, L.k
    seed = wl.sign_seed(args.layer)
    scale = w.scales[-1]
    lg.set_precision(PRECISIONS[args.precision])

    set_bytes = M * 2 * T * (k + d)
    nsets = max(1, math.ceil(2.5 * MALL_BYTES / set_bytes)) if set_bytes < 2.5 * MALL_BYTES else 1
    sets = []
    for s_ in range(nsets):
        mbs = []
        for m in range(M):
            X, dY = wl.layer_inputs(w, args.layer, m + M * s_, device=dev)
            mbs.append((X, dY))
        sets.append(mbs)
    S = torch.zeros((d, r), dtype=torch.float32, device=dev)
    W = wl.layer_weight(w, args.layer, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        S.zero_()
        for X, dY in sets[i % nsets]:
            lg.sketch_accumulate(X, dY, seed, r, S)
        lg.merge_update(W, S, seed, r, scale)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Whole-step throughput: K steps between two synchronisations.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = e0.elapsed_time(e1) / args.steps

    # Per-launch durations, live, with events on the kernels' stream.  Each
    # loop is issued twice: once untimed (which also measures how fast the
    # host issues the calls), then behind a sleep kernel long enough for the
    # host to queue the whole loop before the first timed launch, so the
    # events see GPU time only.
    def gpu_time(fn, n):
        return gpu_time_per_call(torch, stream, fn, n)

    n_calls = args.steps * M

    def sketch_call(i):
        X, dY = sets[(i // M) % nsets][i % M]
        lg.sketch_accumulate(X, dY, seed, r, S)

    t_call, h_call = gpu_time(sketch_call, n_calls)
    sk_reps = quantiles_us(gpu_time_reps(torch, stream, sketch_call, M, 10))
    n_w = max(2, math.ceil(2.5 * MALL_BYTES / (2 * d * k)))
    Ws = [W.clone() for _ in range(n_w)]
    n_merges = max(args.steps, 2 * n_w)
    t_merge, h_merge = gpu_time(lambda i: lg.merge_update(Ws[i % n_w], S, seed, r, scale), n_merges)
    mg_reps = quantiles_us(gpu_time_reps(torch, stream, lambda i: lg.merge_update(Ws[i % n_w], S, seed, r, scale),
                                         4, 10))
    sb = sketch_bytes(T, k, d, r)
    mb = merge_bytes(d, k, r)
    sk_gbs = sb / t_call / 1e9
    mg_gbs = mb / t_merge / 1e9

    extras = {}
    if not args.no_extras:
        # Streaming ceilings measured on this GPU for the same bytes, timed
        # the same way: the sketch call's two input streams read as two
        # launches, one window of the same size read in a single launch, and
        # the merge's W as an in-place read-modify-write over the copies.
        sink = torch.zeros(1, dtype=torch.int32, device=dev)

        def read_two(i):
            X, dY = sets[(i // M) % nsets][i % M]
            lg.stream_read(X, sink)
            lg.stream_read(dY, sink)

        t_read2, _ = gpu_time(read_two, n_calls)
        t_rmw, _ = gpu_time(lambda i: Ws[i % n_w].mul_(1.0), n_merges)
        extras["ceiling"] = {
            "what": "streaming reads/writes of the same bytes on this GPU (logra_stream_read; torch in-place mul for W)",
            "sketch_bytes_two_reads_us": t_read2 * 1e6,
            "sketch_frac_of_two_reads": t_read2 / t_call,
            "merge_w_rmw_us": t_rmw * 1e6,
            "merge_frac_of_rmw": t_rmw / t_merge,
        }
        # The other precision mode on the same inputs (sketch call, merge and
        # the step they make up).
        other = "bf16" if args.precision == "bf16x2" else "bf16x2"
        prev = lg.set_precision(PRECISIONS[other])
        try:
            t_other, _ = gpu_time(sketch_call, n_calls)
            t_mother, _ = gpu_time(lambda i: lg.merge_update(Ws[i % n_w], S, seed, r, scale), n_merges)
        finally:
            lg.set_precision(prev)
        extras["sketch_" + other] = {"avg_call_us": t_other * 1e6, "achieved": sb / t_other / 1e9,
                                     "frac": sb / t_other / 1e9 / HBM_PEAK_GBS, "tokens_per_s": T / t_other,
                                     "merge_us": t_mother * 1e6, "merge_frac": mb / t_mother / 1e9 / HBM_PEAK_GBS,
                                     "step_tokens_per_s_from_kernel_times": M * T / (M * t_other + t_mother)}
        # The Gaussian basis on the same inputs (sketch call, and the merge
        # including its basis generation).
        prev = lg.set_basis(lg.BASIS_GAUSSIAN)
        try:
            t_gs, _ = gpu_time(sketch_call, n_calls)
            t_gm, _ = gpu_time(lambda i: lg.merge_update(Ws[i % n_w], S, seed, r, scale), n_merges)
        finally:
            lg.set_basis(prev)
        extras["basis_gaussian"] = {
            "what": "refreshed Gaussian basis (Box-Muller normals, bf16 hi/lo planes generated per call)",
            "sketch_call_us": t_gs * 1e6, "sketch_frac": sb / t_gs / 1e9 / HBM_PEAK_GBS,
            "merge_us": t_gm * 1e6, "merge_frac": mb / t_gm / 1e9 / HBM_PEAK_GBS,
            "rademacher_sketch_call_us": t_call * 1e6, "rademacher_merge_us": t_merge * 1e6,
        }
        # Split calls: the projection of every microbatch into its own cache
        # (forward time), then the contractions from the caches (backward).
        caches = [[lg.project(X, seed, r) for X, _ in mbs] for mbs in sets]
        t_proj, _ = gpu_time(lambda i: lg.project(sets[(i // M) % nsets][i % M][0], seed, r,
                                                  caches[(i // M) % nsets][i % M]), n_calls)
        t_con, _ = gpu_time(lambda i: lg.contract(sets[(i // M) % nsets][i % M][1], caches[(i // M) % nsets][i % M],
                                                  r, S), n_calls)
        del caches
        pb, cb = split_bytes(T, k, d, r)
        rpad = padded_rank(r)
        nplanes = 2 if args.precision == "bf16x2" else 1
        extras["split"] = {
            "what": "logra_project (forward, X -> cache: the projection kernel) and logra_contract (backward, dY "
                    "and cache -> S: the contraction kernels), per call",
            "project_us": t_proj * 1e6, "project_GBps": pb / t_proj / 1e9, "project_frac": pb / t_proj / 1e9 / HBM_PEAK_GBS,
            "contract_us": t_con * 1e6, "contract_GBps": cb / t_con / 1e9,
            "contract_frac": cb / t_con / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": [pb, cb],
            # The contraction's MFMA rate: 2 T d R flops per plane of P (R the
            # padded rank), two planes in the hi/lo mode, against the dense
            # bf16 peak.
            "contract_mfma": {
                "flops": 2 * T * d * rpad * nplanes, "planes": nplanes,
                "achieved_tflops": 2 * T * d * rpad * nplanes / t_con / 1e12,
                "peak_tflops": BF16_PEAK_TFLOPS,
                "frac": 2 * T * d * rpad * nplanes / t_con / 1e12 / BF16_PEAK_TFLOPS,
            },
        }
        t_ra, h_ra = rowadam_time(torch, lg, stream, S, args.steps)
        extras["rowadam"] = {
            "kernel": "rowadam_rows_kernel + rowadam_norm_kernel + rowadam_apply_kernel",
            "avg_us": t_ra * 1e6, "achieved": rowadam_bytes(d, r) / t_ra / 1e9,
            "frac": rowadam_bytes(d, r) / t_ra / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": rowadam_bytes(d, r),
            "host_us_per_call": h_ra * 1e6,
        }
    del Ws
    torch.cuda.empty_cache()
    if not args.no_extras:
        del sets
        torch.cuda.empty_cache()
        # The workload's other layers, both precision modes.
        others = {}
        for li, Lo in enumerate(w.layers):
            if li != args.layer:
                others[Lo.name] = layer_rates(torch, lg, wl, stream, dev, w, li, r, 2 * args.steps)
        extras["other_layers"] = others
        extras["grouped_merge"] = grouped_merge_timing(torch, lg, wl, stream, dev, max(10, args.steps))
        if not args.no_kl:
            extras["predicted_kl"] = predicted_kl_timing(torch, lg, wl, stream, dev, max(10, args.steps))

    traffic, merge_traffic = load_traffic(args.workload, f"{L.name} d={d} k={k}", r, args.precision)
    out = {
        "metric": "sketch-accumulate tokens/s/layer + merge GB/s, % of MI355X HBM roofline",
        "value": M * T / (step_ms * 1e-3),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "wall_s": wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs, fp32 accumulation",
        "data": "synthetic (seeded iid Gaussian activations and gradients, random-init bf16 weight)",
        "config": {
            "workload": w.title,
            "layer": f"{L.name} d={d} k={k}",
            "r": r,
            "microbatches": M,
            "tokens_per_microbatch": T,
            "merge_scale": scale,
            "precision": args.precision,
            "input_sets_rotated": nsets,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "sketch_accumulate call: the projection kernel (signs drawn in LDS), the contraction kernel, "
                      "and (above three token splits) the sum of the contraction's partial tiles (kernel names per "
                      "layer in the committed trace summary)",
            "bound": "hbm",
            "achieved": sk_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": sk_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_call": sb,
            "avg_call_us": t_call * 1e6,
            "calls_timed": n_calls,
            "host_us_per_call": h_call * 1e6,
            "per_call_over_repetitions": {"what": f"{M} calls (one step's microbatches) per repetition", **sk_reps},
        },
        "merge": {
            "kernel": "merge_kernel",
            "bound": "hbm",
            "achieved": mg_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": mg_gbs / HBM_PEAK_GBS,
            "traffic": merge_traffic,
            "algorithmic_bytes": mb,
            "avg_us": t_merge * 1e6,
            "merges_timed": n_merges,
            "host_us_per_call": h_merge * 1e6,
            "weight_copies_rotated": n_w,
            "per_call_over_repetitions": {"what": "4 merges per repetition", **mg_reps},
        },
        **extras,
        "kernel_source_sha": kernel_source_sha(),
    }
    if not args.no_cpu_baseline:
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(w, args.layer, r, seed, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
