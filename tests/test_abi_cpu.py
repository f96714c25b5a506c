"""C-ABI checks that need no GPU.

* liblogra.so loads and exports every function include/logra.h declares;
* host-only entry points answer (version, status strings, workspace size);
* argument validation rejects bad calls with the documented status before any
  device work is enqueued (these calls return before touching HIP).
"""

import ctypes
import os
import re

import pytest

import rank_gradient_sketching_accumulate_amd as lg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "logra.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_RANGE, ERR_ALIAS, ERR_HIP, ERR_NOMEM = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lg.LIB_PATH):
        from rank_gradient_sketching_accumulate_amd.build import build_library

        build_library()
    return lg.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(logra_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(lg.EXPORTED_SYMBOLS) == _declared_functions()


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert lib.logra_abi_version() == 2
    for s in range(8):
        assert lib.logra_status_string(s)
    assert lib.logra_status_string(0) == b"ok"
    assert lib.logra_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    assert lib.logra_workspace_bytes(0, 64, 64, 64) == 0
    assert lib.logra_workspace_bytes(4096, 1536, 1536, 0) == 0
    assert lib.logra_workspace_bytes(4096, 1536, 1536, 513) == 0
    assert lib.logra_workspace_bytes(4096, 0, 1536, 64) == 0
    # P as a bf16 hi/lo pair: 4 bytes per (token, padded rank column) at
    # least, plus RowAdam's two floats per row; a rank above 256 reuses the
    # scratch of its two halves, so it needs no more than the larger half
    # plus what the row statistics add.
    for T in (512, 4096, 8192, 16384):
        for r in (16, 64, 128, 256, 300, 512):
            R = min(r, 256)
            assert lib.logra_workspace_bytes(T, 5120, 17408, r) >= T * R * 4 + 8 * 5120
    assert lib.logra_workspace_bytes(16384, 17408, 5120, 512) == lib.logra_workspace_bytes(16384, 17408, 5120, 256)


def test_workspace_reserve_validation(lib):
    assert lib.logra_workspace_reserve(-1, 4, 4, 4, None) == ERR_SHAPE
    assert lib.logra_workspace_reserve(16, 4, 4, 0, None) == ERR_RANGE
    assert lib.logra_workspace_reserve(16, 4, 4, 513, None) == ERR_RANGE
    # empty shapes need nothing (no device call)
    assert lib.logra_workspace_reserve(0, 4, 4, 4, None) == OK
    assert lib.logra_workspace_reserve(16, 0, 4, 4, None) == OK


FAKE = 0x10000  # a well-aligned non-null address; never dereferenced on these paths


def _sketch(lib, X=FAKE, ldx=512, dY=FAKE * 64, lddy=256, T=16, k=512, d=256, r=16, S=FAKE * 4096, lds=16):
    return lib.logra_sketch_accumulate(X, ldx, dY, lddy, T, k, d, 0, r, S, lds, None)


def test_sketch_validation(lib):
    assert _sketch(lib, r=0) == ERR_RANGE
    assert _sketch(lib, r=513) == ERR_RANGE
    assert _sketch(lib, T=-1) == ERR_SHAPE
    assert _sketch(lib, lds=8) == ERR_SHAPE
    assert _sketch(lib, X=None) == ERR_NULL
    assert b"non-null" in lib.logra_last_error()
    assert _sketch(lib, ldx=500) == ERR_SHAPE
    assert _sketch(lib, X=FAKE + 2) == ERR_ALIGN
    assert _sketch(lib, ldx=516) == ERR_ALIGN
    assert _sketch(lib, lddy=260) == ERR_ALIGN
    assert _sketch(lib, S=FAKE + 2) == ERR_ALIGN
    # S inside X's span
    assert _sketch(lib, S=FAKE + 1024) == ERR_ALIAS
    # empty problems are no-ops, even with null pointers
    assert _sketch(lib, T=0, X=None, dY=None, S=None) == OK
    assert _sketch(lib, k=0) == OK
    assert _sketch(lib, d=0) == OK


def test_set_deterministic_is_per_call_setting(lib):
    assert lib.logra_set_deterministic(1) == 0
    assert lib.logra_set_deterministic(7) == 1
    assert lib.logra_set_deterministic(0) == 1
    assert lib.logra_set_deterministic(0) == 0


def test_projection_bytes(lib):
    assert lib.logra_projection_bytes(0, 16) == 0
    assert lib.logra_projection_bytes(16, 0) == 0
    assert lib.logra_projection_bytes(16, 513) == 0
    # two bf16 planes of roundup(T, 256) tokens x (16 * next power of two of ceil(r / 16)) columns
    assert lib.logra_projection_bytes(1, 1) == 4 * 256 * 16
    assert lib.logra_projection_bytes(4096, 64) == 4 * 4096 * 64
    assert lib.logra_projection_bytes(4097, 48) == 4 * 4352 * 64
    assert lib.logra_projection_bytes(16384, 256) == 4 * 16384 * 256
    # above 256: the cache of columns 0..255, then one of rank r - 256
    assert lib.logra_projection_bytes(16384, 300) == 4 * 16384 * 256 + 4 * 16384 * 64
    assert lib.logra_projection_bytes(1000, 512) == 2 * 4 * 1024 * 256


PB = 4 * 256 * 16  # logra_projection_bytes(16, 16)


def _project(lib, X=FAKE, ldx=512, T=16, k=512, r=16, P=FAKE * 64, nbytes=PB):
    return lib.logra_project(X, ldx, T, k, 0, r, P, nbytes, None)


def _contract(lib, dY=FAKE, lddy=256, T=16, d=256, P=FAKE * 64, nbytes=PB, r=16, S=FAKE * 4096, lds=16):
    return lib.logra_contract(dY, lddy, T, d, P, nbytes, r, S, lds, None)


def test_split_validation(lib):
    assert _project(lib, r=0) == ERR_RANGE
    assert _project(lib, T=-1) == ERR_SHAPE
    assert _project(lib, T=0, X=None, P=None) == OK
    assert _project(lib, P=None) == ERR_NULL
    assert _project(lib, X=None) == ERR_NULL
    assert _project(lib, nbytes=PB - 1) == ERR_SHAPE
    assert b"logra_projection_bytes" in lib.logra_last_error()
    assert _project(lib, P=FAKE * 64 + 8) == ERR_ALIGN
    assert _project(lib, X=FAKE + 2) == ERR_ALIGN
    assert _project(lib, ldx=500) == ERR_SHAPE
    assert _project(lib, P=FAKE + 4096) == ERR_ALIAS  # inside X's 16 KiB span
    assert _contract(lib, r=513) == ERR_RANGE
    assert _contract(lib, lds=8) == ERR_SHAPE
    assert _contract(lib, T=0, dY=None, P=None, S=None) == OK
    assert _contract(lib, d=0) == OK
    assert _contract(lib, P=None) == ERR_NULL
    assert _contract(lib, nbytes=100) == ERR_SHAPE
    assert _contract(lib, P=FAKE * 64 + 4) == ERR_ALIGN
    assert _contract(lib, lddy=250) == ERR_SHAPE
    assert _contract(lib, S=FAKE + 2048) == ERR_ALIAS  # S inside dY's span
    assert _contract(lib, S=FAKE * 64 + 64) == ERR_ALIAS  # S inside P
    # a cache made for more tokens or a larger rank is large enough
    assert lib.logra_projection_bytes(16, 16) <= lib.logra_projection_bytes(300, 16)


def _kl(lib, z=FAKE, ldz=1024, zd=FAKE * 64, ldzd=1024, n=16, V=1000, dtype=0, T=1.0, rv=FAKE * 4096, q=FAKE * 8192):
    return lib.logra_predicted_kl(z, ldz, zd, ldzd, n, V, dtype, ctypes.c_float(T), rv, q, None)


def test_predicted_kl_validation(lib):
    assert _kl(lib, dtype=2) == ERR_RANGE
    assert _kl(lib, T=0.0) == ERR_RANGE
    assert _kl(lib, T=float("inf")) == ERR_RANGE
    assert _kl(lib, T=float("nan")) == ERR_RANGE
    assert _kl(lib, n=-1) == ERR_SHAPE
    assert _kl(lib, q=None) == ERR_NULL
    assert _kl(lib, z=None) == ERR_NULL
    assert _kl(lib, V=0) == ERR_SHAPE
    assert _kl(lib, ldz=999) == ERR_SHAPE
    assert _kl(lib, ldz=1002) == ERR_ALIGN  # fp32 rows must start on 16-byte boundaries
    assert _kl(lib, dtype=1, ldz=1004, ldzd=1008) == ERR_ALIGN  # bf16: multiples of 8 elements
    assert _kl(lib, z=FAKE + 4) == ERR_ALIGN
    assert _kl(lib, n=1, ldz=1001, ldzd=1003, q=None) == ERR_NULL  # one row: any stride passes the checks
    assert _kl(lib, q=FAKE * 8192 + 2) == ERR_ALIGN
    assert _kl(lib, rv=FAKE * 4096 + 1) == ERR_ALIGN
    assert _kl(lib, q=FAKE + 64) == ERR_ALIAS  # q inside z
    assert _kl(lib, rv=FAKE * 64 + 64) == ERR_ALIAS  # row_var inside zdot
    assert _kl(lib, rv=FAKE * 8192 - 8) == ERR_ALIAS  # row_var runs into q


def test_kl_host_helpers_match_oracle(lib):
    import math

    import oracle

    for q, delta, amax in [(8e-4, 2e-4, 10.0), (5e-5, 2e-4, 10.0), (5e-5, 2e-4, 1.5), (0.0, 1e-4, 3.0),
                           (math.inf, 1e-4, 3.0), (1.234e-7, 3e-5, 100.0)]:
        assert lib.logra_kl_step_scale(q, delta, amax) == oracle.kl_step_scale(q, delta, amax)
    for bad in [(-1.0, 1e-4, 1.0), (math.nan, 1e-4, 1.0), (1e-4, 0.0, 1.0), (1e-4, 1e-4, 0.0)]:
        assert math.isnan(lib.logra_kl_step_scale(*bad))
    for u in (-3, 0, 1, 2, 150, 299, 300, 301, 1000):
        for H in (1, 2, 300, 1000):
            got = lib.logra_kl_budget(u, H, 2e-4, 2e-5)
            assert got == pytest.approx(oracle.kl_budget(u, H, 2e-4, 2e-5), rel=1e-14, abs=1e-20)
    for delta, kappa in [(1e-4, 3e-5), (1e-4, 9e-5), (1e-4, -2e-5), (1e-4, 0.0), (2e-5, 1.0)]:
        assert lib.logra_kl_effective_budget(delta, kappa) == pytest.approx(oracle.effective_budget(delta, kappa),
                                                                             rel=1e-15)
    assert lib.logra_kl_effective_budget(1e-4, math.nan) == 1e-4


def _merge(lib, W=FAKE, ldw=512, U=FAKE * 64, ldu=16, d=256, k=512, r=16, scale=1e-3):
    return lib.logra_merge_update(W, ldw, U, ldu, d, k, 0, r, ctypes.c_float(scale), None)


def test_merge_validation(lib):
    assert _merge(lib, r=0) == ERR_RANGE
    assert _merge(lib, ldu=8) == ERR_SHAPE
    assert _merge(lib, W=None) == ERR_NULL
    assert _merge(lib, ldw=500) == ERR_SHAPE
    assert _merge(lib, W=FAKE + 4) == ERR_ALIGN
    assert _merge(lib, ldw=514) == ERR_ALIGN
    assert _merge(lib, U=FAKE * 64 + 2) == ERR_ALIGN
    assert _merge(lib, scale=float("inf")) == ERR_RANGE
    assert _merge(lib, U=FAKE + 256) == ERR_ALIAS
    assert _merge(lib, d=0) == OK
    # scale 0 leaves W unchanged without any device work
    assert _merge(lib, scale=0.0) == OK


def _items(*specs):
    arr = (lg.MergeItem * max(1, len(specs)))()
    for j, sp in enumerate(specs):
        base = dict(W=FAKE * (1 + 64 * j), ldw=512, U=FAKE * (2048 + 64 * j), ldu=16, d=256, k=512, seed=j, scale=1e-3)
        base.update(sp)
        arr[j] = lg.MergeItem(base["W"], base["ldw"], base["U"], base["ldu"], base["d"], base["k"], base["seed"],
                              base["scale"])
    return arr


def test_grouped_merge_validation(lib):
    assert lib.logra_merge_update_grouped(None, 0, 16, None) == OK
    assert lib.logra_merge_update_grouped(None, 2, 16, None) == ERR_NULL
    assert lib.logra_merge_update_grouped(_items({}), -1, 16, None) == ERR_SHAPE
    assert lib.logra_merge_update_grouped(_items({}), 1, 0, None) == ERR_RANGE
    # an invalid item names itself; nothing is enqueued
    assert lib.logra_merge_update_grouped(_items({}, {"W": None}), 2, 16, None) == ERR_NULL
    assert b"item 1" in lib.logra_last_error()
    assert lib.logra_merge_update_grouped(_items({}, {}, {"ldu": 8}), 3, 16, None) == ERR_SHAPE
    assert lib.logra_merge_update_grouped(_items({"scale": float("nan")}), 1, 16, None) == ERR_RANGE
    assert lib.logra_merge_update_grouped(_items({"W": FAKE + 4}), 1, 16, None) == ERR_ALIGN
    # item 1 writes a W that item 0 also writes, or reads as its U
    assert lib.logra_merge_update_grouped(_items({}, {"W": FAKE + 4096}), 2, 16, None) == ERR_ALIAS
    assert b"item 0" in lib.logra_last_error()
    assert lib.logra_merge_update_grouped(_items({}, {"W": FAKE * 2048}), 2, 16, None) == ERR_ALIAS
    # all items empty or with scale 0: nothing to do, no device work
    assert lib.logra_merge_update_grouped(_items({"d": 0}, {"scale": 0.0}, {"k": 0}), 3, 16, None) == OK


def _rowadam(lib, S=FAKE, lds=16, v=FAKE * 64, d=256, r=16, step=1, beta2=0.95, eps=1e-8):
    return lib.logra_rowadam_scale(S, lds, v, d, r, step, ctypes.c_float(beta2), ctypes.c_float(eps), None)


def test_rowadam_validation(lib):
    assert _rowadam(lib, step=0) == ERR_RANGE
    assert _rowadam(lib, beta2=1.0) == ERR_RANGE
    assert _rowadam(lib, beta2=-0.1) == ERR_RANGE
    assert _rowadam(lib, eps=-1.0) == ERR_RANGE
    assert _rowadam(lib, S=None) == ERR_NULL
    assert _rowadam(lib, lds=4) == ERR_SHAPE
    assert _rowadam(lib, v=FAKE + 64) == ERR_ALIAS
    assert _rowadam(lib, d=0) == OK


def test_signs_validation(lib):
    assert lib.logra_signs(0, 0, 10, FAKE, None) == ERR_RANGE
    assert lib.logra_signs(0, 4, -1, FAKE, None) == ERR_SHAPE
    assert lib.logra_signs(0, 4, 10, None, None) == ERR_NULL
    assert lib.logra_signs(0, 4, 0, None, None) == OK


def test_stream_read_validation(lib):
    assert lib.logra_stream_read(None, 0, None, None) == 0  # empty: no-op
    assert lib.logra_stream_read(None, 16, FAKE, None) == 1
    assert lib.logra_stream_read(FAKE, 16, None, None) == 1
    assert lib.logra_stream_read(FAKE + 8, 16, FAKE, None) == 3  # misaligned base
    assert lib.logra_stream_read(FAKE, 24, FAKE, None) == 3  # not a multiple of 16 bytes
    assert lib.logra_stream_read(FAKE, 16, FAKE + 2, None) == 3  # misaligned sink


def test_python_wrapper_type_checks(lib):
    import torch

    X = torch.zeros((4, 8), dtype=torch.bfloat16)
    S = torch.zeros((4, 4), dtype=torch.float32)
    with pytest.raises(ValueError):
        lg.sketch_accumulate(X, X, 0, 4, S)  # host tensors are refused
    with pytest.raises(TypeError):
        lg.sketch_accumulate(X.float(), X, 0, 4, S)


# ---------------------------------------------------------------------------
# Sync payload: host-side layout and checks (no device work).
# ---------------------------------------------------------------------------
import struct  # noqa: E402


def _payload_header(count=2, r=64, entries=None, magic=0x5052474C, version=1, total=None, reserved=0):
    """The documented layout written out with struct: header, then entries."""
    hb = (32 + 48 * count + 255) // 256 * 256
    if entries is None:
        entries = []
        off = hb
        for j in range(count):
            d, k = 100 + j, 300 + j
            entries.append((1000 + j, d, k, 1e-3 * (j + 1), 0, off, 0))
            off += (d * r * 4 + 255) // 256 * 256
        total = off if total is None else total
    b = struct.pack("<IIiiQQ", magic, version, count, r, total, reserved)
    for e in entries:
        b += struct.pack("<qqqfIQQ", *e)
    return b + bytes(hb - len(b)), entries, total


def _parse(lib, b, max_entries=32):
    from rank_gradient_sketching_accumulate_amd import PayloadEntry, PayloadHeader

    h = PayloadHeader()
    es = (PayloadEntry * 32)()
    st = lib.logra_payload_parse(b, len(b), ctypes.byref(h), es, max_entries)
    return st, h, es


def test_payload_layout_sizes(lib):
    from rank_gradient_sketching_accumulate_amd import MergeItem

    assert lib.logra_payload_header_bytes(0) == 0
    assert lib.logra_payload_header_bytes(1) == 256
    assert lib.logra_payload_header_bytes(4) == 256  # 32 + 192 bytes
    assert lib.logra_payload_header_bytes(5) == 512  # 32 + 240 bytes
    assert lib.logra_payload_header_bytes(33) == 0
    items = (MergeItem * 2)()
    items[0].d, items[0].k, items[1].d, items[1].k = 100, 300, 7, 5
    assert lib.logra_payload_bytes(items, 2, 64) == 256 + 25600 + 1792
    assert lib.logra_payload_bytes(items, 2, 0) == 0
    assert lib.logra_payload_bytes(items, 0, 64) == 0
    items[1].d = -1
    assert lib.logra_payload_bytes(items, 2, 64) == 0


def test_payload_parse_reads_documented_layout(lib):
    b, entries, total = _payload_header()
    st, h, es = _parse(lib, b)
    assert st == OK, lib.logra_last_error()
    assert (h.magic, h.version, h.count, h.r, h.total_bytes) == (0x5052474C, 1, 2, 64, total)
    for j, e in enumerate(entries):
        assert (es[j].seed, es[j].d, es[j].k, es[j].u_offset) == (e[0], e[1], e[2], e[5])
        assert es[j].scale == pytest.approx(e[3], rel=1e-7)


def test_payload_parse_rejects_malformed(lib):
    good, entries, total = _payload_header()
    assert _parse(lib, good[:31])[0] == ERR_SHAPE  # shorter than a header
    assert _parse(lib, good[:32 + 48])[0] == ERR_SHAPE  # second entry cut off
    assert _parse(lib, _payload_header(magic=0x12345678)[0])[0] == ERR_SHAPE
    assert _parse(lib, _payload_header(version=2)[0])[0] == ERR_SHAPE
    assert _parse(lib, _payload_header(reserved=1)[0])[0] == ERR_SHAPE
    assert _parse(lib, _payload_header(r=513)[0])[0] == ERR_SHAPE
    assert _parse(lib, good, max_entries=1)[0] == ERR_RANGE
    bad = list(entries)
    bad[1] = bad[1][:5] + (bad[1][5] + 8,) + bad[1][6:]  # misaligned factor
    assert _parse(lib, _payload_header(entries=bad, total=total)[0])[0] == ERR_SHAPE
    bad = list(entries)
    bad[1] = bad[1][:5] + (entries[0][5],) + bad[1][6:]  # overlaps entry 0's factor
    assert _parse(lib, _payload_header(entries=bad, total=total)[0])[0] == ERR_SHAPE
    assert _parse(lib, _payload_header(entries=entries, total=total - 256)[0])[0] == ERR_SHAPE  # past the end
    bad = list(entries)
    bad[0] = (bad[0][0], -1) + bad[0][2:]
    assert _parse(lib, _payload_header(entries=bad, total=total)[0])[0] == ERR_SHAPE
    bad = list(entries)
    bad[0] = bad[0][:3] + (float("inf"),) + bad[0][4:]
    assert _parse(lib, _payload_header(entries=bad, total=total)[0])[0] == ERR_SHAPE


def test_payload_pack_and_apply_validation(lib):
    from rank_gradient_sketching_accumulate_amd import MergeItem, PayloadEntry, PayloadHeader

    items = (MergeItem * 2)()
    for j in range(2):
        items[j].U, items[j].ldu, items[j].d, items[j].k, items[j].scale = FAKE * (1 + j), 64, 10, 20, 1e-3
    assert lib.logra_payload_pack(items, 0, 64, FAKE * 64, 1 << 20, None) == ERR_RANGE
    assert lib.logra_payload_pack(items, 2, 513, FAKE * 64, 1 << 20, None) == ERR_RANGE
    assert lib.logra_payload_pack(None, 2, 64, FAKE * 64, 1 << 20, None) == ERR_NULL
    assert lib.logra_payload_pack(items, 2, 64, FAKE * 64 + 16, 1 << 20, None) == ERR_ALIGN
    assert lib.logra_payload_pack(items, 2, 64, FAKE * 64, 100, None) == ERR_SHAPE
    items[1].ldu = 32
    assert lib.logra_payload_pack(items, 2, 64, FAKE * 64, 1 << 20, None) == ERR_SHAPE
    items[1].ldu = 64
    items[1].U = FAKE * 64 + 256  # inside the payload
    assert lib.logra_payload_pack(items, 2, 64, FAKE * 64, 1 << 20, None) == ERR_ALIAS
    h = PayloadHeader()
    es = (PayloadEntry * 2)()
    W = (ctypes.c_void_p * 2)(FAKE, FAKE * 2)
    ld = (ctypes.c_int64 * 2)(20, 20)
    assert lib.logra_payload_apply(FAKE * 64, 1 << 20, ctypes.byref(h), es, W, ld, None) == ERR_SHAPE  # unparsed
    assert lib.logra_payload_apply(None, 1 << 20, ctypes.byref(h), es, W, ld, None) == ERR_NULL


def test_basis_setting_and_validation(lib):
    assert lib.logra_set_basis(1) == 0
    assert lib.logra_set_basis(0) == 1
    assert lib.logra_set_basis(0) == 0
    assert lib.logra_basis_normals(1, 0, 16, FAKE, None) == ERR_RANGE
    assert lib.logra_basis_normals(1, 513, 16, FAKE, None) == ERR_RANGE
    assert lib.logra_basis_normals(1, 4, -1, FAKE, None) == ERR_SHAPE
    assert lib.logra_basis_normals(1, 4, 16, None, None) == ERR_NULL
    assert lib.logra_basis_normals(1, 4, 16, FAKE + 2, None) == ERR_ALIGN
    assert lib.logra_basis_normals(1, 4, 0, None, None) == OK
    # the no-allocation sketch refuses the Gaussian basis before any device work
    lib.logra_set_basis(1)
    try:
        st = lib.logra_sketch_accumulate_noalloc(FAKE, 512, FAKE * 64, 256, 16, 512, 256, 0, 16, FAKE * 4096, 16, None)
        assert st == ERR_RANGE and b"Gaussian" in lib.logra_last_error()
    finally:
        lib.logra_set_basis(0)


def test_rowadam_merge_validation(lib):
    args = dict(W=FAKE, ldw=512, S=FAKE * 64, lds=16, v=FAKE * 128, d=256, k=512, seed=0, r=16, step=1,
                beta2=0.95, eps=1e-8, scale=1e-3)

    def call(**kw):
        a = dict(args, **kw)
        return lib.logra_rowadam_merge(a["W"], a["ldw"], a["S"], a["lds"], a["v"], a["d"], a["k"], a["seed"], a["r"],
                                       a["step"], a["beta2"], a["eps"], a["scale"], None)

    assert call(r=0) == ERR_RANGE
    assert call(step=0) == ERR_RANGE
    assert call(beta2=1.0) == ERR_RANGE
    assert call(lds=8) == ERR_SHAPE
    assert call(v=None) == ERR_NULL
    assert call(ldw=500) == ERR_SHAPE
    assert call(W=FAKE * 64 + 64) == ERR_ALIAS  # W over S
    assert call(d=0) == OK


def test_workspace_holds_no_signs(lib):
    # The Rademacher signs are regenerated from the seed inside the kernels
    # and never kept in device memory [LoGRA §2.2, "Memory and
    # synchronization"], so no part of the scratch grows with the signs' r x k
    # bits.  Once k is long enough that the projection's column splits no
    # longer change (at 16384 tokens there are none), the scratch is the same
    # for every k; a sign table would add r * k / 8 bytes (2 MiB at r = 256,
    # k = 65536).
    for T, d in ((16384, 17408), (16384, 5120), (8192, 3584), (4096, 1536)):
        for r in (64, 128, 200, 256, 512):
            sizes = {lib.logra_workspace_bytes(T, d, k, r) for k in (17408, 32768, 65536)}
            assert len(sizes) == 1, (T, d, r, sizes)
    for r in (64, 128, 256):
        sizes = {lib.logra_workspace_bytes(16384, 17408, k, r) for k in (1024, 5120, 17408, 65536)}
        assert len(sizes) == 1, (r, sizes)


def test_bench_traffic_matches_only_its_own_configuration():
    """The committed counter summary fills `traffic` only for the layer, rank
    and precision mode it was taken on (and only on the current sources)."""
    import json
    import os

    import bench

    path = os.path.join(bench.ROOT, "profiles", "traffic_layer27b.json")
    with open(path) as f:
        t = json.load(f)
    layer, r, prec = t["layer"], t["r"], t["precision"]
    current = t["kernel_source_sha"] == bench.kernel_source_sha()
    sk, mg = bench.load_traffic("layer27b", layer, r, prec)
    if current:
        assert sk == t["sketch_call_bytes"] and mg is not None and mg > 0
    else:
        assert sk is None and mg is None
    assert bench.load_traffic("layer27b", layer, r + 1, prec) == (None, None)
    assert bench.load_traffic("layer27b", "other d=1 k=1", r, prec) == (None, None)
    other = "bf16" if prec == "bf16x2" else "bf16x2"
    assert bench.load_traffic("layer27b", layer, r, other) == (None, None)
    assert bench.load_traffic("no_such_workload", layer, r, prec) == (None, None)
