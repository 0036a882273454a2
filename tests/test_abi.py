"""The C-ABI library loads, exports every symbol include/ah.h and
include/ah_instrument.h declare, and
rejects bad arguments on the host before enqueueing anything (no GPU needed:
these calls return before any HIP API is touched)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ah.h")
INSTRUMENT_HEADER = os.path.join(ROOT, "include", "ah_instrument.h")
LIB = os.path.join(ROOT, "mips_ah_partition_amd", "libah.so")


def _declared(header=HEADER):
    txt = open(header).read()
    return sorted(set(re.findall(r"^(?:const char\*|int|size_t)\s+(ah_\w+)\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from mips_ah_partition_amd import build
        build.build()
    return C.CDLL(LIB)


def test_header_declares_the_four_path_calls():
    names = _declared()
    for n in ("ah_partition_score", "ah_build_lut", "ah_scan_topk", "ah_reorder_exact"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from mips_ah_partition_amd import ahlib
    names = _declared()
    assert sorted(ahlib.EXPORTS) == names
    inst = _declared(INSTRUMENT_HEADER)
    assert sorted(ahlib.INSTRUMENT_EXPORTS) == inst and not set(inst) & set(names)
    for n in names + inst:
        assert hasattr(lib, n), n


def test_instrument_hooks_validate_on_the_host(lib):
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.ah_hbm_read_probe.argtypes = [vp, sz, i32, vp, vp]
    lib.ah_scan_workspace_counters.argtypes = [i64, i32, i64, i32, i32, i32, C.POINTER(sz), C.POINTER(sz)]
    fake, odd = vp(4096), vp(4097)  # never dereferenced: every case below fails validation first
    assert lib.ah_hbm_read_probe(fake, 100, 8, fake, None) == -2      # not a multiple of 16
    assert lib.ah_hbm_read_probe(fake, 1024, 0, fake, None) == -2     # blocks per CU out of range
    assert lib.ah_hbm_read_probe(fake, 1024, 65, fake, None) == -2
    assert lib.ah_hbm_read_probe(None, 1024, 8, fake, None) == -1
    assert lib.ah_hbm_read_probe(odd, 1024, 8, fake, None) == -3
    assert lib.ah_hbm_read_probe(None, 0, 8, None, None) == 0         # nothing to read
    a, c = sz(), sz()
    assert lib.ah_scan_workspace_counters(10, 64, 1000, 0, 0, 50, C.byref(a), C.byref(c)) == 0
    lib.ah_scan_workspace_bytes.restype = sz
    lib.ah_scan_workspace_bytes.argtypes = [i64, i32, i64, i32, i32, i32]
    total = lib.ah_scan_workspace_bytes(10, 64, 1000, 0, 0, 50)
    assert a.value + 40 <= total and c.value + 64 <= total and a.value != c.value
    assert lib.ah_scan_workspace_counters(10, 64, 1000, 0, 0, 0, C.byref(a), C.byref(c)) == -2
    assert lib.ah_scan_workspace_counters(10, 64, 1000, 0, 0, 50, None, C.byref(c)) == -1


def test_status_strings(lib):
    lib.ah_status_string.restype = C.c_char_p
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.ah_status_string(s)
    assert lib.ah_version() >= 1


def test_host_side_validation(lib):
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.ah_scan_topk.argtypes = [vp, i64, i32, vp, i32, i64, vp, vp, i32, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.ah_build_lut.argtypes = [vp, i64, i32, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.ah_reorder_exact.argtypes = [vp, i64, i32, vp, i32, i64, vp, i32, i32, vp, vp, vp]
    lib.ah_partition_score.argtypes = [vp, i64, i32, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.ah_scan_workspace_bytes.restype = sz
    lib.ah_scan_workspace_bytes.argtypes = [i64, i32, i64, i32, i32, i32]
    fake = vp(4096)  # never dereferenced: every case below fails validation first
    # scan: stride too small, R < 1, nl > L, missing pointers, R too large, no workspace
    assert lib.ah_scan_topk(fake, 2, 8, fake, 3, 10, None, None, 0, None, 0, 5, fake, fake, fake, 1 << 30, None) == -2
    assert lib.ah_scan_topk(fake, 2, 8, fake, 4, 10, None, None, 0, None, 0, 0, fake, fake, fake, 1 << 30, None) == -2
    assert lib.ah_scan_topk(fake, 2, 8, fake, 4, 10, None, fake, 3, fake, 4, 5, fake, fake, fake, 1 << 30, None) == -2
    assert lib.ah_scan_topk(None, 2, 8, fake, 4, 10, None, None, 0, None, 0, 5, fake, fake, fake, 1 << 30, None) == -1
    assert lib.ah_scan_topk(fake, 2, 8, fake, 4, 10, None, None, 0, None, 0, 5000, fake, fake, fake, 1 << 30, None) == -3
    assert lib.ah_scan_topk(fake, 2, 8, fake, 4, 10, None, None, 0, None, 0, 5, fake, fake, None, 0, None) == -4
    need = lib.ah_scan_workspace_bytes(2, 8, 10, 0, 0, 5)
    assert need > 0
    assert lib.ah_scan_topk(fake, 2, 8, fake, 4, 10, None, None, 0, None, 0, 5, fake, fake, fake, need - 1, None) == -4
    # nq == 0 is a no-op even with NULL pointers
    assert lib.ah_scan_topk(None, 0, 8, None, 4, 10, None, None, 0, None, 0, 5, None, None, None, 0, None) == 0
    # LUT: d != B*dpb, dpb too large, NULL output
    assert lib.ah_build_lut(fake, 3, 10, fake, 4, 2, None, fake, fake, fake, None) == -2
    assert lib.ah_build_lut(fake, 3, 64, fake, 2, 32, None, fake, fake, fake, None) == -3
    assert lib.ah_build_lut(fake, 3, 8, fake, 4, 2, None, None, fake, fake, None) == -1
    # reorder: k > R (the page's "reorder not above k" failure mode), bad dtype
    assert lib.ah_reorder_exact(fake, 3, 8, fake, 0, 10, fake, 5, 6, fake, fake, None) == -2
    assert lib.ah_reorder_exact(fake, 3, 8, fake, 7, 10, fake, 5, 5, fake, fake, None) == -3
    # partition: nl > L, workspace too small
    assert lib.ah_partition_score(fake, 3, 8, fake, 4, 5, fake, None, fake, 1 << 30, None) == -2
    assert lib.ah_partition_score(fake, 3, 8, fake, 4, 2, fake, None, fake, 8, None) == -4


def test_tiled_layout_validation(lib):
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.ah_tiled_codes_bytes.restype = sz
    lib.ah_tiled_codes_bytes.argtypes = [i64, i32]
    lib.ah_tile_codes.argtypes = [vp, i32, i64, i32, vp, sz, vp]
    lib.ah_scan_topk.argtypes = [vp, i64, i32, vp, i32, i64, vp, vp, i32, vp, i32, i32, vp, vp, vp, sz, vp]
    # ceil(n / 64) tiles of 64 rows x ceil(ceil(B/2) / 16) segments of 16 bytes
    assert lib.ah_tiled_codes_bytes(1, 1) == 1024
    assert lib.ah_tiled_codes_bytes(64, 64) == 2048
    assert lib.ah_tiled_codes_bytes(65, 192) == 2 * 64 * 6 * 16
    assert lib.ah_tiled_codes_bytes(0, 8) == 0
    assert lib.ah_tiled_codes_bytes(-1, 8) == 0 and lib.ah_tiled_codes_bytes(5, 0) == 0
    fake, odd = vp(4096), vp(4097)  # never dereferenced: every case below fails validation first
    need = lib.ah_tiled_codes_bytes(100, 64)
    assert lib.ah_tile_codes(fake, 31, 100, 64, fake, need, None) == -2      # stride below ceil(B/2)
    assert lib.ah_tile_codes(fake, 32, 100, 64, fake, need - 1, None) == -2  # output too small
    assert lib.ah_tile_codes(fake, 4096, 100, 8192, fake, 1 << 40, None) == -3  # B above the limit
    assert lib.ah_tile_codes(None, 32, 100, 64, fake, need, None) == -1
    assert lib.ah_tile_codes(fake, 32, 100, 64, odd, need, None) == -3       # output not 16-byte aligned
    assert lib.ah_tile_codes(None, 32, 0, 64, None, 0, None) == 0            # n == 0: no-op
    # scan on tiled codes (code_stride AH_CODES_TILED) needs 16-byte aligned codes
    assert lib.ah_scan_topk(fake, 2, 8, odd, -1, 10, None, None, 0, None, 0, 5, fake, fake, fake, 1 << 30, None) == -3
    # a zero (or any other negative) stride is a caller error, not the tiled layout
    assert lib.ah_scan_topk(fake, 2, 8, fake, 0, 10, None, None, 0, None, 0, 5, fake, fake, fake, 1 << 30, None) == -2
    assert lib.ah_scan_topk(fake, 2, 8, fake, -2, 10, None, None, 0, None, 0, 5, fake, fake, fake, 1 << 30, None) == -2


def test_encode_validation(lib):
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    lib.ah_encode.argtypes = [vp, i32, i64, i32, vp, i32, i32, C.c_double, i32, vp, i32, vp]
    fake = vp(4096)  # never dereferenced: every case below fails validation first
    assert lib.ah_encode(fake, 0, 10, 9, fake, 4, 2, 4.0, 2, fake, 2, None) == -2   # d != B * dpb
    assert lib.ah_encode(fake, 0, 10, 8, fake, 4, 2, 4.0, 2, fake, 1, None) == -2   # stride below ceil(B/2)
    assert lib.ah_encode(fake, 0, 10, 8, fake, 4, 2, 4.0, 65, fake, 2, None) == -2  # too many sweeps
    assert lib.ah_encode(fake, 0, 10, 8, fake, 4, 2, -1.0, 2, fake, 2, None) == -2  # eta < 0
    assert lib.ah_encode(fake, 0, 10, 8, fake, 4, 2, float("nan"), 2, fake, 2, None) == -2
    assert lib.ah_encode(fake, 5, 10, 8, fake, 4, 2, 4.0, 2, fake, 2, None) == -3   # dtype
    assert lib.ah_encode(fake, 0, 10, 68, fake, 2, 34, 4.0, 2, fake, 1, None) == -3  # dpb above the limit
    assert lib.ah_encode(None, 0, 10, 8, fake, 4, 2, 4.0, 2, fake, 2, None) == -1
    assert lib.ah_encode(None, 0, 0, 8, None, 4, 2, 4.0, 2, None, 2, None) == 0     # n == 0: no-op


def test_assign_validation(lib):
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.ah_assign_workspace_bytes.restype = sz
    lib.ah_assign_workspace_bytes.argtypes = [i64, i32]
    lib.ah_assign_leaves.argtypes = [vp, i64, i32, vp, i32, vp, vp, vp, sz, vp]
    fake = vp(4096)  # never dereferenced: every case below fails validation first
    need = lib.ah_assign_workspace_bytes(1000, 64)
    assert need > 1000 * 64 * 4 and lib.ah_assign_workspace_bytes(5, 0) == 0
    assert lib.ah_assign_leaves(fake, 1000, 0, fake, 64, fake, None, fake, need, None) == -2
    assert lib.ah_assign_leaves(fake, 1000, 8, fake, 5000, fake, None, fake, 1 << 40, None) == -3
    assert lib.ah_assign_leaves(None, 1000, 8, fake, 64, fake, None, fake, need, None) == -1
    assert lib.ah_assign_leaves(fake, 1000, 8, fake, 64, fake, None, fake, need - 1, None) == -4
    assert lib.ah_assign_leaves(None, 0, 8, None, 64, None, None, None, 0, None) == 0


def test_sq8_validation(lib):
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.ah_sq8_quantize.argtypes = [vp, i64, i32, C.c_double, vp, vp, vp]
    lib.ah_sq8_workspace_bytes.restype = sz
    lib.ah_sq8_workspace_bytes.argtypes = [i64, i64, i32, i32]
    lib.ah_sq8_scan_topk.argtypes = [vp, vp, i64, vp, vp, i64, i32, i32, vp, vp, vp, sz, vp]
    fake, odd = vp(4096), vp(4097)  # never dereferenced: every case below fails validation first
    assert lib.ah_sq8_quantize(fake, 10, 0, 99.9, fake, fake, None) == -2
    assert lib.ah_sq8_quantize(fake, 10, 8, 100.5, fake, fake, None) == -2
    assert lib.ah_sq8_quantize(fake, 10, 20000, 99.9, fake, fake, None) == -3
    assert lib.ah_sq8_quantize(None, 10, 8, 99.9, fake, fake, None) == -1
    assert lib.ah_sq8_quantize(None, 0, 8, 99.9, None, None, None) == 0
    need = lib.ah_sq8_workspace_bytes(100, 1000, 64, 10)
    assert need >= 100 * 1000 * 4  # small n: the score block of all queries
    assert lib.ah_sq8_workspace_bytes(100, 1000, 64, 0) == 0
    assert lib.ah_sq8_scan_topk(fake, fake, 100, fake, fake, 1000, 64, 1001, fake, None, fake, need, None) == -2  # R > n
    assert lib.ah_sq8_scan_topk(fake, fake, 100, fake, fake, 1000, 40, 10, fake, None, fake, need, None) == -3   # d % 16
    assert lib.ah_sq8_scan_topk(odd, fake, 100, fake, fake, 1000, 64, 10, fake, None, fake, need, None) == -3    # alignment
    assert lib.ah_sq8_scan_topk(fake, fake, 100, fake, fake, 1000, 64, 10, fake, None, fake, need - 1, None) == -4
    assert lib.ah_sq8_scan_topk(fake, None, 100, fake, fake, 1000, 64, 10, fake, None, fake, need, None) == -1


def test_residual_validation(lib):
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.ah_scan_topk_residual.argtypes = [vp, i64, i32, vp, i32, i64, vp, vp, i32, vp, i32, vp, i32, i32, vp, vp, vp,
                                          sz, vp]
    lib.ah_residual_leaf_bias.argtypes = [vp, vp, i64, i32, i32, vp, vp]
    fake, odd = vp(4096), vp(4097)  # never dereferenced: every case below fails validation first
    big = 1 << 40
    # leaf terms: nl < 1, negative or too large bound, missing pointers, empty batch
    assert lib.ah_residual_leaf_bias(fake, fake, 4, 0, 10, fake, None) == -2
    assert lib.ah_residual_leaf_bias(fake, fake, 4, 3, -1, fake, None) == -2
    assert lib.ah_residual_leaf_bias(fake, fake, 4, 3, (1 << 24) + 1, fake, None) == -3
    assert lib.ah_residual_leaf_bias(None, fake, 4, 3, 10, fake, None) == -1
    assert lib.ah_residual_leaf_bias(None, None, 0, 3, 10, None, None) == 0
    # biased scan: no leaves, no bias, negative or too large bound, unaligned table, small workspace
    assert lib.ah_scan_topk_residual(fake, 2, 8, fake, 4, 100, None, None, 0, None, 0, fake, 10, 5, fake, fake, fake,
                                     big, None) == -2
    assert lib.ah_scan_topk_residual(fake, 2, 8, fake, 4, 100, None, fake, 4, fake, 2, None, 10, 5, fake, fake, fake,
                                     big, None) == -1
    assert lib.ah_scan_topk_residual(fake, 2, 8, fake, 4, 100, None, fake, 4, fake, 2, fake, -1, 5, fake, fake, fake,
                                     big, None) == -2
    assert lib.ah_scan_topk_residual(fake, 2, 8, fake, 4, 100, None, fake, 4, fake, 2, fake, (1 << 24) + 1, 5, fake,
                                     fake, fake, big, None) == -3
    assert lib.ah_scan_topk_residual(odd, 2, 8, fake, 4, 100, None, fake, 4, fake, 2, fake, 10, 5, fake, fake, fake,
                                     big, None) == -3
    assert lib.ah_scan_topk_residual(fake, 2, 8, fake, 4, 100, None, fake, 4, fake, 2, fake, 10, 5, fake, fake, fake,
                                     16, None) == -4
    assert lib.ah_scan_topk_residual(None, 0, 8, None, 4, 100, None, None, 4, None, 2, None, 10, 5, None, None, None,
                                     0, None) == 0


def test_rslm_validation(lib):
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.ah_rslm_rotate.argtypes = [vp, i64, i32, vp, vp, vp, vp]
    lib.ah_rslm_encode.argtypes = [vp, i64, i32, vp, vp, vp, vp]
    lib.ah_rslm_scan_topk.argtypes = [vp, vp, i64, vp, vp, i64, i32, vp, i32, vp, vp, vp, sz, vp]
    fake = vp(4096)  # device pointers are never dereferenced: every case fails validation first
    assert lib.ah_rslm_rotate(fake, 10, 0, fake, fake, fake, None) == -2
    assert lib.ah_rslm_rotate(fake, 10, 20000, fake, fake, fake, None) == -3
    assert lib.ah_rslm_rotate(None, 10, 8, fake, fake, fake, None) == -1
    assert lib.ah_rslm_rotate(None, 0, 8, None, None, None, None) == 0
    good = (C.c_float * 16)(*[float(c) - 7.5 for c in range(16)])
    flat = (C.c_float * 16)(*([0.0] * 16))
    assert lib.ah_rslm_encode(fake, 10, 8, C.cast(flat, vp), fake, fake, None) == -2  # not increasing
    assert lib.ah_rslm_encode(fake, 10, 8, None, fake, fake, None) == -1
    assert lib.ah_rslm_encode(None, 10, 8, C.cast(good, vp), fake, fake, None) == -1
    assert lib.ah_rslm_encode(None, 0, 8, C.cast(good, vp), None, None, None) == 0
    lv = (C.c_int8 * 16)(*range(-8, 8))
    big = 1 << 40
    assert lib.ah_rslm_scan_topk(fake, fake, 4, fake, fake, 100, 40, C.cast(lv, vp), 10, fake, None, fake, big,
                                 None) == -3  # d % 16
    assert lib.ah_rslm_scan_topk(fake, fake, 4, vp(4100), fake, 100, 64, C.cast(lv, vp), 10, fake, None, fake, big,
                                 None) == -3  # codes not 8-byte aligned
    assert lib.ah_rslm_scan_topk(fake, fake, 4, fake, fake, 100, 64, None, 10, fake, None, fake, big, None) == -1
    assert lib.ah_rslm_scan_topk(fake, fake, 4, fake, fake, 100, 64, C.cast(lv, vp), 101, fake, None, fake, big,
                                 None) == -2
    assert lib.ah_rslm_scan_topk(fake, fake, 4, fake, fake, 100, 64, C.cast(lv, vp), 10, fake, None, fake, 16,
                                 None) == -4


def test_workspace_sizes_zero_shapes(lib):
    """Every size query is host arithmetic and accepts empty shapes (no queries,
    no rows, no leaves) without faulting."""
    i32, i64 = C.c_int32, C.c_int64
    sig = {"ah_partition_workspace_bytes": [i64, i32], "ah_scan_workspace_bytes": [i64, i32, i64, i32, i32, i32],
           "ah_sq8_workspace_bytes": [i64, i64, i32, i32], "ah_kmeans_workspace_bytes": [i32, i32],
           "ah_pq_update_workspace_bytes": [i64, i32, i32], "ah_assign_workspace_bytes": [i64, i32],
           "ah_tiled_codes_bytes": [i64, i32]}
    for fn, args in (("ah_partition_workspace_bytes", (0, 5)), ("ah_partition_workspace_bytes", (3, 0)),
                     ("ah_partition_workspace_bytes", (0, 0)), ("ah_scan_workspace_bytes", (0, 8, 10, 0, 0, 5)),
                     ("ah_scan_workspace_bytes", (3, 8, 0, 0, 0, 5)), ("ah_scan_workspace_bytes", (0, 8, 10, 4, 2, 5)),
                     ("ah_sq8_workspace_bytes", (0, 10, 16, 5)), ("ah_sq8_workspace_bytes", (3, 0, 16, 5)),
                     ("ah_kmeans_workspace_bytes", (0, 16)), ("ah_pq_update_workspace_bytes", (0, 8, 2)),
                     ("ah_assign_workspace_bytes", (0, 5)), ("ah_assign_workspace_bytes", (5, 0)),
                     ("ah_tiled_codes_bytes", (0, 8))):
        f = getattr(lib, fn)
        f.argtypes, f.restype = sig[fn], C.c_size_t
        assert f(*args) < (1 << 40), (fn, args)


def test_noalloc_scan_rejects_on_the_host(lib):
    """ah_scan_topk_noalloc validates like ah_scan_topk and rejects a batch whose
    scratch exceeds AH_SCAN_SCRATCH_BYTES before touching the GPU."""
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    lib.ah_scan_topk_noalloc.argtypes = [vp, i64, i32, vp, i32, i64, vp, vp, i32, vp, i32, i32, vp, vp, vp]
    fake = vp(4096)  # never dereferenced: every case below fails validation first
    assert lib.ah_scan_topk_noalloc(fake, 16, 64, fake, 32, 20_000_000, None, None, 0, None, 0, 100,
                                    fake, fake, None) == -3           # 640 MB of fallback slots alone
    assert lib.ah_scan_topk_noalloc(fake, 2, 8, fake, 3, 10, None, None, 0, None, 0, 5, fake, fake, None) == -2
    assert lib.ah_scan_topk_noalloc(fake, 2, 8, fake, 4, 10, None, None, 0, None, 0, 0, fake, fake, None) == -2
    assert lib.ah_scan_topk_noalloc(None, 2, 8, fake, 4, 10, None, None, 0, None, 0, 5, fake, fake, None) == -1
    assert lib.ah_scan_topk_noalloc(None, 0, 8, None, 4, 10, None, None, 0, None, 0, 5, None, None, None) == 0

