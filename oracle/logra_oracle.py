"""Plain float64 CPU oracle of the LoGRA per-layer hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product package.  It is slow on
purpose: it forms the dense gradient G explicitly and then projects it, which
is the definition the method approximates without ever building G.

Notation (LoGRA paper, section 2.1): a linear layer Y = X W^T with
W in R^{d x k}; X (T x k) holds the layer inputs of one microbatch and dY
(T x d) the output gradients, so the weight gradient is G = dY^T X (d x k).
A in R^{r x k} is the random projection, S = G A^T (d x r) the sketch.

Every function below cites the passage it follows.  Where the pages leave a
step open, the reading taken here is stated in the docstring.

Pins (tests that tie this file to something other than itself) live in
tests/test_oracle_*.py.  Parity-unpinned parts: the RowAdam stabiliser
statistic (the word naming it is missing from the appendix text; this oracle
takes the mean) and the word "normalized" describing the sketch RowAdam
consumes (taken as: the sketch as passed in).
"""

from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1

# Philox4x64 constants, from the published definition [Philox, SC'11]:
# two round multipliers and the two Weyl-sequence key increments
# (golden ratio and sqrt(3)-1 in 0.64 fixed point).
_PHILOX_M0 = 0xD2E7470EE14C6C93
_PHILOX_M1 = 0xCA5A826395121157
_PHILOX_W0 = 0x9E3779B97F4A7C15
_PHILOX_W1 = 0xBB67AE8584CAA73B

PHILOX_BLOCK_BITS = 256  # one Philox4x64 call yields four 64-bit words


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds [Philox, SC'11, section 5].

    ``ctr`` is four 64-bit words (x0, x1, x2, x3) and ``key`` two words
    (k0, k1).  Each word may be a Python int or a numpy object array of
    Python ints (all of one shape), so the same arithmetic serves one block or
    many.  One round multiplies x0 and x2 by the two round constants into
    128-bit products, then
        x0' = hi(M1*x2) ^ x1 ^ k0,   x1' = lo(M1*x2),
        x2' = hi(M0*x0) ^ x3 ^ k1,   x3' = lo(M0*x0);
    the key advances by the Weyl constants between rounds.
    Returns the four output words.
    """
    x0, x1, x2, x3 = ctr
    k0, k1 = key
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _PHILOX_W0) & MASK64
            k1 = (k1 + _PHILOX_W1) & MASK64
        p0 = _PHILOX_M0 * x0
        p1 = _PHILOX_M1 * x2
        x0, x1, x2, x3 = (
            ((p1 >> 64) ^ x1 ^ k0) & MASK64,
            p1 & MASK64,
            ((p0 >> 64) ^ x3 ^ k1) & MASK64,
            p0 & MASK64,
        )
    return x0, x1, x2, x3


def sign_bits(seed: int, r: int, k: int) -> np.ndarray:
    """Raw sign bits b[i, j] in {0, 1} for i < r, j < k (uint8, r x k).

    The pages fix only that A's entries are independent random signs, drawn
    from a seed that the rollout side can use to regenerate A (LoGRA, section
    2.1 "A compact representation"; section 2.2 "Memory and
    synchronization"; Algorithm 1, "sample A from a fresh seed").  The
    generator is this library's own choice, fixed here:

      key      = (seed, 0)
      block    = Philox4x64-10(counter = (c, i, 0, 0), key) for sign row i and
                 column block c = j // 256
      bit      = bit (q % 64) of output word q // 64, q = j % 256 (LSB first)
      sign     = +1 for bit 0, -1 for bit 1.
    """
    if r < 0 or k < 0:
        raise ValueError("r and k must be non-negative")
    nblk = (k + PHILOX_BLOCK_BITS - 1) // PHILOX_BLOCK_BITS
    if r == 0 or k == 0:
        return np.zeros((r, k), dtype=np.uint8)
    rows = np.empty((r, nblk), dtype=object)
    cols = np.empty((r, nblk), dtype=object)
    zero = np.empty((r, nblk), dtype=object)
    for i in range(r):
        for c in range(nblk):
            rows[i, c] = i
            cols[i, c] = c
            zero[i, c] = 0
    seed &= MASK64
    words = philox4x64_10((cols, rows, zero, zero), (seed, 0))
    w = np.stack([np.asarray(wd, dtype=np.uint64) for wd in words], axis=-1)
    # (r, nblk, 4) uint64 -> bytes in little-endian word order -> bits LSB first
    raw = w.astype("<u8").view(np.uint8).reshape(r, nblk * 32)
    bits = np.unpackbits(raw, axis=1, bitorder="little")
    return np.ascontiguousarray(bits[:, :k])


def sign_matrix(seed: int, r: int, k: int) -> np.ndarray:
    """Signs s in {+1, -1}^{r x k} as int8 (see ``sign_bits``)."""
    return (1 - 2 * sign_bits(seed, r, k).astype(np.int8)).astype(np.int8)


def rademacher_projection(seed: int, r: int, k: int) -> np.ndarray:
    """A = s / sqrt(r) in float64 (LoGRA section 2.1: independent random signs
    scaled by 1/sqrt(r); Table 4 "Rank 256, Rademacher")."""
    return sign_matrix(seed, r, k).astype(np.float64) / math.sqrt(r)


GAUSS_PER_BLOCK = 8  # normals per Philox4x64 block: four Box-Muller pairs


def gaussian_normals(seed: int, r: int, k: int) -> np.ndarray:
    """Z[i, j] ~ N(0, 1) for i < r, j < k (float64): the entries of the
    refreshed Gaussian basis that the LoGRA paper compares with the
    Rademacher one (section 3.4.1, Figure 5c: "refreshed Rademacher and
    Gaussian projections resample at every update").  The pages name no
    generator; this library's choice, drawn from the same Philox stream as the
    signs but a separate counter range (counter word 2 = 1):

      block    = Philox4x64-10(counter = (j // 8, i, 1, 0), key = (seed, 0))
      halves   h[2m] = low 32 bits of output word m, h[2m+1] = high 32 bits
      pair     p = (j % 8) // 2 uses h[2p] and h[2p+1]
      uniforms u1 = ((h[2p] >> 8) + 1) / 2^24 in (0, 1],
               u2 = (h[2p+1] >> 8) / 2^24 in [0, 1)   (24-bit, exact in fp32)
      Box-Muller (Box and Muller, 1958): R = sqrt(-2 ln u1), theta = 2 pi u2,
               Z = R cos(theta) for even j % 8, R sin(theta) for odd.
    """
    if r < 0 or k < 0:
        raise ValueError("r and k must be non-negative")
    if r == 0 or k == 0:
        return np.zeros((r, k))
    nblk = (k + GAUSS_PER_BLOCK - 1) // GAUSS_PER_BLOCK
    rows = np.empty((r, nblk), dtype=object)
    cols = np.empty((r, nblk), dtype=object)
    one = np.empty((r, nblk), dtype=object)
    zero = np.empty((r, nblk), dtype=object)
    for i in range(r):
        for c in range(nblk):
            rows[i, c] = i
            cols[i, c] = c
            one[i, c] = 1
            zero[i, c] = 0
    words = philox4x64_10((cols, rows, one, zero), (seed & MASK64, 0))
    w = np.stack([np.asarray(wd, dtype=np.uint64) for wd in words], axis=-1)  # (r, nblk, 4)
    halves = w.astype("<u8").view("<u4").reshape(r, nblk, 8).astype(np.int64)  # h[2m] = low half of word m
    u1 = ((halves[:, :, 0::2] >> 8) + 1).astype(np.float64) / 2.0**24
    u2 = (halves[:, :, 1::2] >> 8).astype(np.float64) / 2.0**24
    R = np.sqrt(-2.0 * np.log(u1))
    theta = 2.0 * math.pi * u2
    z = np.empty((r, nblk, 8))
    z[:, :, 0::2] = R * np.cos(theta)
    z[:, :, 1::2] = R * np.sin(theta)
    return np.ascontiguousarray(z.reshape(r, nblk * 8)[:, :k])


def gaussian_projection(seed: int, r: int, k: int) -> np.ndarray:
    """A = Z / sqrt(r) (entries N(0, 1/r), so E[A^T A] = I as for the
    Rademacher basis); see ``gaussian_normals``."""
    return gaussian_normals(seed, r, k) / math.sqrt(r)


# ---------------------------------------------------------------------------
# bfloat16 helpers (the layer tensors are bf16, as in the pages' BF16 runs,
# LoGRA appendix D.1).
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, in one
    step (no intermediate float32).  bf16 keeps 8 significant bits: a value
    x = m * 2**e with 0.5 <= |m| < 1 is quantised to multiples of 2**(e-8);
    below the smallest normal (2**-126) the quantum stays 2**-133.  Results
    whose magnitude reaches 2**128 become infinities; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(x)
        e = np.maximum(e, -125)
        q = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
        q = np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, x), q)
    return np.where(np.isnan(x), x, q)


def f64_to_bf16_bits(x) -> np.ndarray:
    """RNE-round float64 to bf16 and return the uint16 bit patterns."""
    q = round_to_bf16(x).astype(np.float32)  # exact: q is a bf16 value
    return (q.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# The hot path, written as its plain definition.
# ---------------------------------------------------------------------------

def dense_gradient(X_list, dY_list, rows=None) -> np.ndarray:
    """G = sum over microbatches of dY_m^T X_m (float64, d x k, or only the
    rows listed in ``rows``).

    LoGRA section 2.1, equation 1 (G is the gradient of the loss w.r.t. W)
    and Algorithm 1: the batch is split into microbatches and each adds its
    own contribution; for a linear layer that contribution is dY_m^T X_m.
    The sum is a plain sum: any loss normalisation is already inside dY.
    """
    G = None
    for X, dY in zip(X_list, dY_list):
        X = np.asarray(X, dtype=np.float64)
        dY = np.asarray(dY, dtype=np.float64)
        if rows is not None:
            dY = dY[:, rows]
        part = dY.T @ X
        G = part if G is None else G + part
    return G


def sketch_from_gradient(G, A) -> np.ndarray:
    """S = G A^T (LoGRA section 2.1, equation 2)."""
    return np.asarray(G, dtype=np.float64) @ np.asarray(A, dtype=np.float64).T


def project_inputs(X, A) -> np.ndarray:
    """P = X A^T (T x r, float64): the layer inputs projected before the
    backward derivatives multiply them (LoGRA section 2.1, the paragraph after
    equation 2), the quantity kept as "cached projections" (section 2.2,
    "Memory and synchronization").  dY^T P is then this microbatch's G A^T."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(A, dtype=np.float64).T


def sketch_accumulate(S0, X_list, dY_list, A, rows=None) -> np.ndarray:
    """S = S0 + (sum_m dY_m^T X_m) A^T.

    Algorithm 1 of the LoGRA paper zeroes S once per step and adds each
    microbatch's projected gradient (nabla_W L_m) A^T to it; S0 is the value S
    holds when the call starts.  Computed the slow way: the dense gradient
    first, then the projection (equation 2).  ``rows`` restricts the result
    to a subset of the d rows (rows of S are independent of each other).
    """
    G = dense_gradient(X_list, dY_list, rows=rows)
    S0 = np.asarray(S0, dtype=np.float64)
    if rows is not None:
        S0 = S0[rows]
    return S0 + sketch_from_gradient(G, A)


def low_rank_expand(U, A) -> np.ndarray:
    """G_hat = U A, the d x k low-rank expansion (LoGRA section 2.1,
    equation 3; rank at most r)."""
    return np.asarray(U, dtype=np.float64) @ np.asarray(A, dtype=np.float64)


def merge_update(W, U, A, scale: float) -> np.ndarray:
    """W' = RNE_bf16(W - scale * U A), with scale = alpha * eta.

    LoGRA section 2.1, equation 4 (W <- W - alpha eta U A) and Algorithm 1's
    trainer update; the merged weight stays a full-size bf16 matrix
    (appendix D.1: BF16 computation).  W holds bf16 values widened to
    float64; the product and the difference are exact-ish float64 and the
    result is rounded to bf16 once.  Returns float64 bf16 values.
    """
    W = np.asarray(W, dtype=np.float64)
    return round_to_bf16(W - float(scale) * low_rank_expand(U, A))


def rowadam_scale(S, v, step: int, beta2: float, eps_rel: float = 1e-8,
                  eps_floor: float = 1e-30):
    """RowAdam row scaling of a sketch (LoGRA appendix B, equation 15).

    For row i of S (d x r):
        v_i    <- beta2 v_i + (1 - beta2) (1/r) sum_j S_ij^2
        vhat_i  = v_i / (1 - beta2^t)                 (t = step >= 1, v_0 = 0)
        eps     = max(eps_rel * mean_i sqrt(vhat_i), eps_floor)
        Utilde_i = S_i / (sqrt(vhat_i) + eps)
        U       = Utilde * ||S||_F / ||Utilde||_F     (U = 0 if Utilde = 0)

    Readings of words lost from the appendix text: the stabiliser is
    eps_rel times the MEAN over rows of sqrt(vhat) (a "relative" epsilon,
    Table 4) with a positive floor; the rescale matches the FROBENIUS norm of
    the incoming sketch ("preserving the sketch's overall magnitude"); the
    "normalized" sketch is the sketch as passed in.  Zero sketches give zero
    updates, as the appendix states.
    Returns (U, v_new) in float64.
    """
    if step < 1:
        raise ValueError("step counts RowAdam updates and starts at 1")
    S = np.asarray(S, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    r = S.shape[1]
    ms = (S * S).sum(axis=1) / r
    v_new = beta2 * v + (1.0 - beta2) * ms
    vhat = v_new / (1.0 - beta2 ** step)
    root = np.sqrt(vhat)
    eps = max(eps_rel * float(root.mean()) if root.size else 0.0, eps_floor)
    Ut = S / (root + eps)[:, None]
    nt = float(np.sqrt((Ut * Ut).sum()))
    ns = float(np.sqrt((S * S).sum()))
    if nt == 0.0:
        return np.zeros_like(S), v_new
    return Ut * (ns / nt), v_new


def reconstruction_cosine(G, A) -> float:
    """cos(G, (G A^T) A): the Frobenius cosine between the dense gradient
    and its reconstruction from the sketch (LoGRA section 3.4.1 and
    appendix D.3)."""
    G = np.asarray(G, dtype=np.float64)
    Gh = low_rank_expand(sketch_from_gradient(G, A), A)
    return float((G * Gh).sum() / (np.linalg.norm(G) * np.linalg.norm(Gh)))


def sketch_projected_first(S0, X_list, dY_list, A, rows=None) -> np.ndarray:
    """S = S0 + sum_m dY_m^T (X_m A^T): equation 2 with the layer inputs
    projected before the backward derivatives multiply them (LoGRA section
    2.1, the paragraph after equation 2), in float64.  The same quantity as
    ``sketch_accumulate`` with the products associated the other way; it
    never forms the d x k gradient, so whole large layers stay cheap.
    ``rows`` restricts the result to a subset of the d rows."""
    A = np.asarray(A, dtype=np.float64)
    S0 = np.asarray(S0, dtype=np.float64)
    S = (S0[rows] if rows is not None else S0).copy()
    for X, dY in zip(X_list, dY_list):
        P = project_inputs(X, A)
        dY = np.asarray(dY, dtype=np.float64)
        if rows is not None:
            dY = dY[:, rows]
        S += dY.T @ P
    return S


def sketch_accumulate_rounded_projection(S0, X_list, dY_list, seed: int, r: int, rows=None) -> np.ndarray:
    """S = S0 + (1/sqrt(r)) sum_m dY_m^T RNE_bf16(X_m s^T): the sketch with the
    projected inputs rounded once to bf16 before the backward multiply.

    This is the plain definition of a lower-precision way to evaluate
    equation 2 of LoGRA section 2.1 (inputs projected first, the paragraph
    after equation 2): P_m = X_m s^T (s the signs of ``sign_matrix``) is
    formed in float64, rounded to the nearest bf16 value (ties to even), and
    then multiplied by the backward derivatives.  With exact bf16 P it equals
    ``sketch_accumulate``.
    """
    s = sign_matrix(seed, r, np.asarray(X_list[0]).shape[1]).astype(np.float64)
    S0 = np.asarray(S0, dtype=np.float64)
    S = (S0[rows] if rows is not None else S0).copy()
    for X, dY in zip(X_list, dY_list):
        P = round_to_bf16(np.asarray(X, dtype=np.float64) @ s.T)
        dY = np.asarray(dY, dtype=np.float64)
        if rows is not None:
            dY = dY[:, rows]
        S += (dY.T @ P) / math.sqrt(r)
    return S
