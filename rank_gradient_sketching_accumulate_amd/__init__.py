"""LoGRA per-layer sketch-accumulate / RowAdam / merge on MI355X.

Thin ctypes binding over the C ABI of ``liblogra.so`` (declared in
``include/logra.h``).  This module only marshals arguments: every step of the
path runs in the library's HIP kernels.  torch is used for device memory and
for the current HIP stream; it is never used to compute.

Method: "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
Sketches" (arXiv 2610.06647v2), section 2.1 (equations 2-4), Algorithm 1 and
appendix B (RowAdam).

If the library has not been built, importing still works but every call
raises ``LograError``: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "LograError",
    "LIB_PATH",
    "MAX_RANK",
    "load_library",
    "library_loaded",
    "sketch_accumulate",
    "set_deterministic",
    "set_precision",
    "PRECISION_BF16X2",
    "PRECISION_BF16",
    "projection_bytes",
    "project",
    "contract",
    "merge_update",
    "merge_update_grouped",
    "payload_bytes",
    "set_basis",
    "basis_normals",
    "BASIS_RADEMACHER",
    "BASIS_GAUSSIAN",
    "payload_header_bytes",
    "payload_pack",
    "payload_parse",
    "payload_apply",
    "rowadam_scale",
    "rowadam_merge",
    "predicted_kl",
    "kl_step_scale",
    "kl_budget",
    "kl_effective_budget",
    "signs",
    "workspace_bytes",
    "workspace_reserve",
    "workspace_release",
    "stream_read",
    "abi_version",
    "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblogra.so")
MAX_RANK = 512
ABI_VERSION = 2  # LOGRA_ABI_VERSION this binding is written for
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # LOGRA_NOALLOC_SCRATCH_BYTES

# Every symbol include/logra.h declares.
EXPORTED_SYMBOLS = (
    "logra_sketch_accumulate",
    "logra_sketch_accumulate_noalloc",
    "logra_set_deterministic",
    "logra_set_precision",
    "logra_set_basis",
    "logra_basis_normals",
    "logra_projection_bytes",
    "logra_project",
    "logra_contract",
    "logra_merge_update",
    "logra_merge_update_grouped",
    "logra_payload_header_bytes",
    "logra_payload_bytes",
    "logra_payload_pack",
    "logra_payload_parse",
    "logra_payload_apply",
    "logra_rowadam_scale",
    "logra_rowadam_merge",
    "logra_predicted_kl",
    "logra_kl_step_scale",
    "logra_kl_budget",
    "logra_kl_effective_budget",
    "logra_signs",
    "logra_stream_read",
    "logra_workspace_bytes",
    "logra_workspace_reserve",
    "logra_workspace_release",
    "logra_status_string",
    "logra_last_error",
    "logra_abi_version",
)


# Status codes of include/logra.h.
LOGRA_OK = 0
LOGRA_ERR_NULL = 1
LOGRA_ERR_SHAPE = 2
LOGRA_ERR_ALIGN = 3
LOGRA_ERR_RANGE = 4
LOGRA_ERR_ALIAS = 5
LOGRA_ERR_HIP = 6
LOGRA_ERR_NOMEM = 7


class LograError(RuntimeError):
    """A nonzero status from the library, or the library is missing."""

    def __init__(self, msg: str, status: int | None = None):
        super().__init__(msg)
        self.status = status


_lib = None


class MergeItem(ctypes.Structure):
    """One matrix of a grouped merge (the C struct logra_merge_item)."""

    _fields_ = [
        ("W", ctypes.c_void_p), ("ldw", ctypes.c_int64),
        ("U", ctypes.c_void_p), ("ldu", ctypes.c_int64),
        ("d", ctypes.c_int64), ("k", ctypes.c_int64),
        ("seed", ctypes.c_uint64), ("scale", ctypes.c_float),
    ]


class PayloadHeader(ctypes.Structure):
    """The C struct logra_payload_header (32 bytes)."""

    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
        ("count", ctypes.c_int32), ("r", ctypes.c_int32),
        ("total_bytes", ctypes.c_uint64), ("reserved", ctypes.c_uint64),
    ]


class PayloadEntry(ctypes.Structure):
    """The C struct logra_payload_entry (48 bytes)."""

    _fields_ = [
        ("seed", ctypes.c_uint64), ("d", ctypes.c_int64), ("k", ctypes.c_int64),
        ("scale", ctypes.c_float), ("basis", ctypes.c_uint32),
        ("u_offset", ctypes.c_uint64), ("reserved1", ctypes.c_uint64),
    ]


PAYLOAD_MAX_ITEMS = 32


def _declare(lib):
    c_i64, c_u64, c_i32, c_vp, c_f = ctypes.c_int64, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
    lib.logra_sketch_accumulate.argtypes = [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_u64, c_i32, c_vp, c_i64, c_vp]
    lib.logra_sketch_accumulate.restype = ctypes.c_int
    lib.logra_sketch_accumulate_noalloc.argtypes = lib.logra_sketch_accumulate.argtypes
    lib.logra_sketch_accumulate_noalloc.restype = ctypes.c_int
    lib.logra_set_deterministic.argtypes = [ctypes.c_int]
    lib.logra_set_deterministic.restype = ctypes.c_int
    lib.logra_set_precision.argtypes = [ctypes.c_int]
    lib.logra_set_precision.restype = ctypes.c_int
    lib.logra_projection_bytes.argtypes = [c_i64, c_i32]
    lib.logra_projection_bytes.restype = ctypes.c_size_t
    lib.logra_project.argtypes = [c_vp, c_i64, c_i64, c_i64, c_u64, c_i32, c_vp, ctypes.c_size_t, c_vp]
    lib.logra_project.restype = ctypes.c_int
    lib.logra_contract.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, ctypes.c_size_t, c_i32, c_vp, c_i64, c_vp]
    lib.logra_contract.restype = ctypes.c_int
    lib.logra_merge_update.argtypes = [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_u64, c_i32, c_f, c_vp]
    lib.logra_merge_update.restype = ctypes.c_int
    lib.logra_merge_update_grouped.argtypes = [ctypes.POINTER(MergeItem), c_i32, c_i32, c_vp]
    lib.logra_merge_update_grouped.restype = ctypes.c_int
    lib.logra_set_basis.argtypes = [ctypes.c_int]
    lib.logra_set_basis.restype = ctypes.c_int
    lib.logra_basis_normals.argtypes = [c_u64, c_i32, c_i64, c_vp, c_vp]
    lib.logra_basis_normals.restype = ctypes.c_int
    lib.logra_payload_header_bytes.argtypes = [c_i32]
    lib.logra_payload_header_bytes.restype = ctypes.c_size_t
    lib.logra_payload_bytes.argtypes = [ctypes.POINTER(MergeItem), c_i32, c_i32]
    lib.logra_payload_bytes.restype = ctypes.c_size_t
    lib.logra_payload_pack.argtypes = [ctypes.POINTER(MergeItem), c_i32, c_i32, c_vp, ctypes.c_size_t, c_vp]
    lib.logra_payload_pack.restype = ctypes.c_int
    lib.logra_payload_parse.argtypes = [c_vp, ctypes.c_size_t, ctypes.POINTER(PayloadHeader),
                                        ctypes.POINTER(PayloadEntry), c_i32]
    lib.logra_payload_parse.restype = ctypes.c_int
    lib.logra_payload_apply.argtypes = [c_vp, ctypes.c_size_t, ctypes.POINTER(PayloadHeader),
                                        ctypes.POINTER(PayloadEntry), ctypes.POINTER(c_vp),
                                        ctypes.POINTER(c_i64), c_vp]
    lib.logra_payload_apply.restype = ctypes.c_int
    lib.logra_rowadam_merge.argtypes = [c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_i64, c_u64, c_i32, c_i64, c_f, c_f,
                                        c_f, c_vp]
    lib.logra_rowadam_merge.restype = ctypes.c_int
    lib.logra_rowadam_scale.argtypes = [c_vp, c_i64, c_vp, c_i64, c_i32, c_i64, c_f, c_f, c_vp]
    lib.logra_rowadam_scale.restype = ctypes.c_int
    lib.logra_predicted_kl.argtypes = [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i32, c_f, c_vp, c_vp, c_vp]
    lib.logra_predicted_kl.restype = ctypes.c_int
    c_d = ctypes.c_double
    lib.logra_kl_step_scale.argtypes = [c_d, c_d, c_d]
    lib.logra_kl_step_scale.restype = c_d
    lib.logra_kl_budget.argtypes = [c_i64, c_i64, c_d, c_d]
    lib.logra_kl_budget.restype = c_d
    lib.logra_kl_effective_budget.argtypes = [c_d, c_d]
    lib.logra_kl_effective_budget.restype = c_d
    lib.logra_signs.argtypes = [c_u64, c_i32, c_i64, c_vp, c_vp]
    lib.logra_signs.restype = ctypes.c_int
    lib.logra_stream_read.argtypes = [c_vp, ctypes.c_size_t, c_vp, c_vp]
    lib.logra_stream_read.restype = ctypes.c_int
    lib.logra_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i32]
    lib.logra_workspace_bytes.restype = ctypes.c_size_t
    lib.logra_workspace_reserve.argtypes = [c_i64, c_i64, c_i64, c_i32, c_vp]
    lib.logra_workspace_reserve.restype = ctypes.c_int
    lib.logra_workspace_release.argtypes = [c_vp]
    lib.logra_workspace_release.restype = ctypes.c_int
    lib.logra_status_string.argtypes = [ctypes.c_int]
    lib.logra_status_string.restype = ctypes.c_char_p
    lib.logra_last_error.argtypes = []
    lib.logra_last_error.restype = ctypes.c_char_p
    lib.logra_abi_version.argtypes = []
    lib.logra_abi_version.restype = ctypes.c_int


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle of liblogra.so."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise LograError(
            f"{p} is missing: build it with `python -m rank_gradient_sketching_accumulate_amd.build` "
            "(there is no fallback implementation)"
        )
    lib = ctypes.CDLL(p)
    _declare(lib)
    got = lib.logra_abi_version()
    if got != ABI_VERSION:
        raise LograError(f"{p} has ABI version {got}, this binding needs {ABI_VERSION}: rebuild the library")
    _lib = lib
    return lib


def library_loaded() -> bool:
    return _lib is not None


def _check(status: int):
    if status != 0:
        lib = load_library()
        name = lib.logra_status_string(status).decode()
        detail = lib.logra_last_error().decode()
        raise LograError(f"logra status {status} ({name}): {detail}", status)


_raw_stream = None


def _stream_or_current(stream) -> int:
    """Raw handle of a torch stream (or an int handle), or of torch's current
    stream on the current device when None."""
    import torch

    if stream is None:
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _stream_handle(tensor) -> int:
    """The raw handle of torch's current HIP stream on the tensor's device."""
    global _raw_stream
    if _raw_stream is None:
        import torch

        # torch's own raw accessor avoids building a Stream object per call.
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream = raw if raw is not None else (
            lambda dev: int(torch.cuda.current_stream(dev).cuda_stream))
    return int(_raw_stream(tensor.get_device()))


def _need(t, dtype, name, ndim=2):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    if ndim == 2:
        if t.size(1) > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must have unit column stride")
    elif t.dim() == 1 and t.numel() > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be contiguous")


class _OnDevice:
    """Makes the device of the call's device tensors current while the C ABI
    runs (it takes pointers on the current device and allocates its scratch
    there) and refuses device tensors on different devices.  Host tensors and
    None are ignored."""

    __slots__ = ("dev", "prev")
    _single = None  # True once the process is known to see one device

    def __init__(self, *tensors):
        self.prev = None
        if _OnDevice._single is None:
            import torch

            _OnDevice._single = torch.cuda.device_count() == 1
        if _OnDevice._single:
            self.dev = None  # one device: it is the current one
            return
        dev = None
        for t in tensors:
            if t is None or not t.is_cuda:
                continue
            di = t.get_device()
            if dev is None:
                dev = di
            elif di != dev:
                raise ValueError("the device tensors of one call must be on the same device")
        self.dev = dev

    def __enter__(self):
        if self.dev is not None:
            import torch

            cur = torch._C._cuda_getDevice()
            if cur != self.dev:
                self.prev = cur
                torch._C._cuda_setDevice(self.dev)
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            import torch

            torch._C._cuda_setDevice(self.prev)
        return False


def _ld(t) -> int:
    return int(t.stride(0)) if t.size(0) > 1 else max(int(t.stride(0)), int(t.size(1)))


def sketch_accumulate(X, dY, seed: int, r: int, S, noalloc: bool = False):
    """S += (1/sqrt(r)) dY^T (X s^T) on the current stream; returns S.

    X: (T, k) bf16, dY: (T, d) bf16, S: (d, r) float32 (updated in place).
    noalloc: call logra_sketch_accumulate_noalloc (scratch in the library's
    static device array; calls that overlap on one GPU race).
    """
    import torch

    lib = load_library()
    fn = lib.logra_sketch_accumulate_noalloc if noalloc else lib.logra_sketch_accumulate
    _need(X, torch.bfloat16, "X")
    _need(dY, torch.bfloat16, "dY")
    _need(S, torch.float32, "S")
    T, k = X.shape
    if dY.size(0) != T:
        raise ValueError("X and dY must have the same number of rows (tokens)")
    d = dY.size(1)
    if tuple(S.shape) != (d, r):
        raise ValueError(f"S must be ({d}, {r}), got {tuple(S.shape)}")
    with _OnDevice(X, dY, S):
        _check(
            fn(
                X.data_ptr(), _ld(X), dY.data_ptr(), _ld(dY), T, k, d,
                ctypes.c_uint64(seed & (2**64 - 1)), r, S.data_ptr(), _ld(S), _stream_handle(S),
            )
        )
    return S


def set_deterministic(enable: bool) -> bool:
    """Bitwise-reproducible sketches on the calling thread (one workgroup per
    row tile of S, no atomic adds; slower).  Returns the previous setting."""
    return bool(load_library().logra_set_deterministic(1 if enable else 0))


BASIS_RADEMACHER = 0
BASIS_GAUSSIAN = 1


def set_basis(basis: int) -> int:
    """Projection basis of the calling thread (BASIS_RADEMACHER or
    BASIS_GAUSSIAN); returns the previous one."""
    return int(load_library().logra_set_basis(int(basis)))


def basis_normals(seed: int, r: int, k: int, device="cuda"):
    """Z (r, k) float32 of the Gaussian basis for `seed` (unscaled)."""
    import torch

    out = torch.empty((r, k), dtype=torch.float32, device=device)
    with _OnDevice(out):
        _check(load_library().logra_basis_normals(ctypes.c_uint64(seed & (2**64 - 1)), r, k,
                                                  out.data_ptr() if out.numel() else None, _stream_handle(out)))
    return out


PRECISION_BF16X2 = 0
PRECISION_BF16 = 1


def set_precision(mode: int) -> int:
    """Precision on the calling thread: PRECISION_BF16X2 (P in the fused
    sketch, and U in the merges with the sign basis, as a bf16 high/low
    pair; the default) or PRECISION_BF16 (each rounded once to bf16).
    Returns the previous mode."""
    return int(load_library().logra_set_precision(int(mode)))


def projection_bytes(T: int, r: int) -> int:
    """Bytes of the projection cache for T tokens at rank r (0 if T <= 0)."""
    return int(load_library().logra_projection_bytes(T, r))


def project(X, seed: int, r: int, P=None):
    """Forward half of the split sketch: P = X s^T into a projection cache.

    X: (T, k) bf16.  P: a uint8 device tensor of at least projection_bytes(T, r)
    bytes (allocated when None); its layout is the one include/logra.h states.
    Returns P.
    """
    import torch

    lib = load_library()
    _need(X, torch.bfloat16, "X")
    T, k = X.shape
    nbytes = projection_bytes(T, r)
    if P is None:
        P = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=X.device)
    _need(P, torch.uint8, "P", ndim=1)
    with _OnDevice(X, P):
        _check(
            lib.logra_project(
                X.data_ptr() if X.numel() else None, _ld(X) if k else 0, T, k,
                ctypes.c_uint64(seed & (2**64 - 1)), r, P.data_ptr(), P.numel(), _stream_handle(P),
            )
        )
    return P


def contract(dY, P, r: int, S):
    """Backward half of the split sketch: S += (1/sqrt(r)) dY^T P; returns S.

    dY: (T, d) bf16, P: the cache logra_project filled for the same T and r,
    S: (d, r) float32 (updated in place).
    """
    import torch

    lib = load_library()
    _need(dY, torch.bfloat16, "dY")
    _need(P, torch.uint8, "P", ndim=1)
    _need(S, torch.float32, "S")
    T, d = dY.shape
    if tuple(S.shape) != (d, r):
        raise ValueError(f"S must be ({d}, {r}), got {tuple(S.shape)}")
    with _OnDevice(dY, P, S):
        _check(
            lib.logra_contract(
                dY.data_ptr(), _ld(dY), T, d, P.data_ptr(), P.numel(), r, S.data_ptr(), _ld(S),
                _stream_handle(S),
            )
        )
    return S


def merge_update(W, U, seed: int, r: int, scale: float):
    """W <- RNE_bf16(W - scale (1/sqrt(r)) U s) in place; returns W.

    W: (d, k) bf16, U: (d, r) float32, scale = alpha * eta.
    """
    import torch

    lib = load_library()
    _need(W, torch.bfloat16, "W")
    _need(U, torch.float32, "U")
    d, k = W.shape
    if tuple(U.shape) != (d, r):
        raise ValueError(f"U must be ({d}, {r}), got {tuple(U.shape)}")
    with _OnDevice(W, U):
        _check(
            lib.logra_merge_update(
                W.data_ptr(), _ld(W), U.data_ptr(), _ld(U), d, k,
                ctypes.c_uint64(seed & (2**64 - 1)), r, float(scale), _stream_handle(W),
            )
        )
    return W


def merge_update_grouped(items, r: int):
    """Grouped merge: items is a sequence of (W, U, seed, scale) with W (d, k)
    bf16 and U (d, r) float32; every W is updated in place as
    merge_update(W, U, seed, r, scale) would, in one launch.  Returns None."""
    import torch

    lib = load_library()
    arr = (MergeItem * max(1, len(items)))()
    stream = None
    for j, (W, U, seed, scale) in enumerate(items):
        _need(W, torch.bfloat16, "W")
        _need(U, torch.float32, "U")
        d, k = W.shape
        if tuple(U.shape) != (d, r):
            raise ValueError(f"item {j}: U must be ({d}, {r}), got {tuple(U.shape)}")
        arr[j] = MergeItem(W.data_ptr(), _ld(W), U.data_ptr(), _ld(U), d, k, seed & (2**64 - 1), float(scale))
        if stream is None:
            stream = _stream_handle(W)
    with _OnDevice(*[t for it in items for t in it[:2]]):
        _check(lib.logra_merge_update_grouped(arr, len(items), r, stream))


def _factor_items(factors, r: int):
    """ctypes items for a payload: factors is a sequence of (U, seed, scale,
    k) with U (d, r) float32 on the GPU."""
    import torch

    arr = (MergeItem * max(1, len(factors)))()
    for j, (U, seed, scale, k) in enumerate(factors):
        _need(U, torch.float32, "U")
        if U.dim() != 2 or U.size(1) != r:
            raise ValueError(f"factor {j}: U must be (d, {r}), got {tuple(U.shape)}")
        arr[j] = MergeItem(None, 0, U.data_ptr() if U.numel() else None, _ld(U), U.size(0), int(k),
                           seed & (2**64 - 1), float(scale))
    return arr


def payload_bytes(factors, r: int) -> int:
    """Size of the sync payload of factors [(U, seed, scale, k), ...]."""
    return int(load_library().logra_payload_bytes(_factor_items(factors, r), len(factors), r))


def payload_pack(factors, r: int, out=None):
    """Pack factors [(U, seed, scale, k), ...] (U: (d, r) float32 on the GPU,
    the matrix's alpha*eta `scale`, its column count k) into a uint8 device
    tensor (allocated when `out` is None); returns it."""
    import torch

    lib = load_library()
    arr = _factor_items(factors, r)
    n = int(lib.logra_payload_bytes(arr, len(factors), r))
    if n == 0:
        raise LograError("invalid payload items", LOGRA_ERR_RANGE)
    dev = factors[0][0].device
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=dev)
    with _OnDevice(out):
        _check(lib.logra_payload_pack(arr, len(factors), r, out.data_ptr(), out.numel(), _stream_handle(out)))
    return out


def payload_parse(header_bytes: bytes):
    """Parse and check the host copy of a payload's first bytes (at least
    payload_header_bytes(count)); returns (header, entries) as ctypes
    structures."""
    lib = load_library()
    h = PayloadHeader()
    es = (PayloadEntry * PAYLOAD_MAX_ITEMS)()
    buf = ctypes.create_string_buffer(bytes(header_bytes), len(header_bytes))
    _check(lib.logra_payload_parse(buf, len(header_bytes), ctypes.byref(h), es, PAYLOAD_MAX_ITEMS))
    return h, es


def payload_header_bytes(count: int) -> int:
    return int(load_library().logra_payload_header_bytes(count))


def payload_apply(payload, header, entries, Ws):
    """Receiver side: W_j <- merge of entry j for every entry of a parsed
    payload (payload: the uint8 device tensor); Ws: the receiver's (d_j, k_j)
    bf16 weights, in entry order."""
    import torch

    lib = load_library()
    n = header.count
    if len(Ws) != n:
        raise ValueError(f"{n} weights needed, got {len(Ws)}")
    ptrs = (ctypes.c_void_p * n)()
    lds = (ctypes.c_int64 * n)()
    for j, W in enumerate(Ws):
        _need(W, torch.bfloat16, "W")
        ptrs[j] = W.data_ptr() if W.numel() else None
        lds[j] = _ld(W)
    with _OnDevice(payload, *Ws):
        _check(lib.logra_payload_apply(payload.data_ptr(), payload.numel(), ctypes.byref(header), entries, ptrs, lds,
                                       _stream_handle(payload)))


def rowadam_merge(W, S, v, seed: int, r: int, step: int, beta2: float, eps_rel: float, scale: float):
    """W <- merge of RowAdam(S) without writing U (S unchanged, v updated);
    W: (d, k) bf16, S: (d, r) float32, v: (d,) float32.  Returns W."""
    import torch

    lib = load_library()
    _need(W, torch.bfloat16, "W")
    _need(S, torch.float32, "S")
    _need(v, torch.float32, "v", ndim=1)
    d, k = W.shape
    if tuple(S.shape) != (d, r) or v.numel() != d:
        raise ValueError(f"S must be ({d}, {r}) and v ({d},)")
    with _OnDevice(W, S, v):
        _check(lib.logra_rowadam_merge(W.data_ptr() if W.numel() else None, _ld(W), S.data_ptr(), _ld(S), v.data_ptr(),
                                       d, k, ctypes.c_uint64(seed & (2**64 - 1)), r, step, beta2, eps_rel, scale,
                                       _stream_handle(S)))
    return W


def rowadam_scale(S, v, step: int, beta2: float, eps_rel: float = 1e-8):
    """RowAdam: S -> U in place, v (d,) float32 updated in place; returns S."""
    import torch

    lib = load_library()
    _need(S, torch.float32, "S")
    _need(v, torch.float32, "v", ndim=1)
    d, r = S.shape
    if v.numel() != d:
        raise ValueError("v must have one value per row of S")
    with _OnDevice(S, v):
        _check(lib.logra_rowadam_scale(S.data_ptr(), _ld(S), v.data_ptr(), d, r, int(step),
                                       float(beta2), float(eps_rel), _stream_handle(S)))
    return S


DTYPE_F32 = 0
DTYPE_BF16 = 1


def predicted_kl(z, zdot, temperature: float, row_var=None, q=None):
    """q = 1/(2 n T^2) sum_s Var_{v ~ softmax(z_s/T)}[zdot_s,v] on the device.

    z, zdot: (n, V) float32 or bfloat16 (the same dtype), unit column stride.
    row_var: optional (n,) float32 output of the per-row variances.
    q: optional (1,) float32 output; allocated when None.  Returns q.
    """
    import torch

    lib = load_library()
    if z.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("z must be float32 or bfloat16")
    _need(z, z.dtype, "z")
    _need(zdot, z.dtype, "zdot")
    if zdot.shape != z.shape:
        raise ValueError("z and zdot must have the same shape")
    n, V = z.shape
    if q is None:
        q = torch.empty(1, dtype=torch.float32, device=z.device)
    _need(q, torch.float32, "q", ndim=1)
    if row_var is not None:
        _need(row_var, torch.float32, "row_var", ndim=1)
        if row_var.numel() != n:
            raise ValueError("row_var must have one entry per row")
    dt = DTYPE_BF16 if z.dtype == torch.bfloat16 else DTYPE_F32
    with _OnDevice(z, zdot, row_var, q):
        _check(
            lib.logra_predicted_kl(
                z.data_ptr() if n else None, _ld(z) if n else 0, zdot.data_ptr() if n else None,
                _ld(zdot) if n else 0, n, V, dt, float(temperature),
                row_var.data_ptr() if row_var is not None and n else None, q.data_ptr(), _stream_handle(q),
            )
        )
    return q


def kl_step_scale(q: float, delta: float, alpha_max: float) -> float:
    """alpha = min(alpha_max, sqrt(delta / q)) (host; NaN for invalid input)."""
    return float(load_library().logra_kl_step_scale(float(q), float(delta), float(alpha_max)))


def kl_budget(u: int, H: int, delta_max: float, delta_min: float) -> float:
    """Cosine-annealed KL budget of update u (host)."""
    return float(load_library().logra_kl_budget(int(u), int(H), float(delta_max), float(delta_min)))


def kl_effective_budget(delta: float, kappa: float) -> float:
    """max(delta - kappa, delta / 2); NaN kappa leaves delta unchanged (host)."""
    return float(load_library().logra_kl_effective_budget(float(delta), float(kappa)))


def signs(seed: int, r: int, k: int, device="cuda"):
    """The sign matrix s (r x k) as int8 +-1 (test and debugging aid)."""
    import torch

    lib = load_library()
    out = torch.empty((r, k), dtype=torch.int8, device=device)
    with _OnDevice(out):
        _check(lib.logra_signs(ctypes.c_uint64(seed & (2**64 - 1)), r, k, out.data_ptr() if k else None,
                               _stream_handle(out)))
    return out


def stream_read(t, sink):
    """Stream the bytes of the contiguous device tensor t (a measurement aid:
    the read ceiling for those bytes); sink is a one-element int32 device
    tensor that receives nothing in practice."""
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError("t must be a contiguous device tensor")
    if not isinstance(sink, torch.Tensor) or sink.dtype != torch.int32 or not sink.is_cuda:
        raise TypeError("sink must be an int32 device tensor")
    nbytes = t.numel() * t.element_size()
    with _OnDevice(t, sink):
        _check(load_library().logra_stream_read(t.data_ptr() if nbytes else None, nbytes, sink.data_ptr(),
                                                _stream_handle(t)))


def workspace_bytes(T: int, d: int, k: int, r: int) -> int:
    """Scratch bytes the sketch calls and RowAdam need for this shape (the
    calling thread's precision and determinism settings)."""
    return int(load_library().logra_workspace_bytes(T, d, k, r))


def workspace_reserve(T: int, d: int, k: int, r: int, stream=None) -> None:
    """Grow the library's scratch for `stream` (default: the current torch
    stream) to fit this shape, so later calls allocate nothing (for example
    under graph capture)."""
    _check(load_library().logra_workspace_reserve(T, d, k, r, _stream_or_current(stream)))


def workspace_release(stream=None) -> None:
    """Wait for `stream` and free every scratch buffer the library holds for
    it (graphs captured before must not be replayed afterwards)."""
    _check(load_library().logra_workspace_release(_stream_or_current(stream)))


def abi_version() -> int:
    return int(load_library().logra_abi_version())
