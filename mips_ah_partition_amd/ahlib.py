"""Thin Python binding of the C ABI in include/ah.h (libah.so, built in-tree).

Argument marshalling only: every function takes torch CUDA (ROCm) tensors,
checks dtype/shape/contiguity, passes raw device pointers and the current
stream to the library and raises ``AHError`` on a non-zero status.  All work
runs in the library's HIP kernels; there is no fallback path: if libah.so is
missing or cannot be loaded, the import of this module's functions fails
loudly.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libah.so")

AH_OK, AH_ERR_NULL, AH_ERR_SHAPE, AH_ERR_UNSUPPORTED, AH_ERR_WORKSPACE, AH_ERR_HIP = 0, -1, -2, -3, -4, -5
AH_F32, AH_BF16 = 0, 1
AH_CODES_TILED = -1

# every symbol include/ah.h declares
EXPORTS = (
    "ah_status_string", "ah_version",
    "ah_partition_workspace_bytes", "ah_partition_score",
    "ah_build_lut",
    "ah_scan_workspace_bytes", "ah_scan_topk", "ah_scan_topk_noalloc",
    "ah_residual_leaf_bias", "ah_scan_topk_residual",
    "ah_sq8_quantize", "ah_sq8_workspace_bytes", "ah_sq8_scan_topk",
    "ah_rslm_rotate", "ah_rslm_encode", "ah_rslm_scan_topk",
    "ah_assign_workspace_bytes", "ah_assign_leaves",
    "ah_kmeans_workspace_bytes", "ah_kmeans_update",
    "ah_encode", "ah_encode_sweep", "ah_pq_update_workspace_bytes", "ah_pq_update",
    "ah_tiled_codes_bytes", "ah_tile_codes",
    "ah_reorder_exact",
)
# every symbol include/ah_instrument.h declares (measurement hooks)
INSTRUMENT_EXPORTS = ("ah_scan_topk_timed", "ah_scan_workspace_counters", "ah_hbm_read_probe")

_lib = None


class AHError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.ah_status_string.restype = C.c_char_p
        L.ah_status_string.argtypes = [C.c_int]
        L.ah_version.restype = C.c_int
        L.ah_partition_workspace_bytes.restype = sz
        L.ah_partition_workspace_bytes.argtypes = [i64, i32]
        L.ah_partition_score.restype = C.c_int
        L.ah_partition_score.argtypes = [vp, i64, i32, vp, i32, i32, vp, vp, vp, sz, vp]
        L.ah_build_lut.restype = C.c_int
        L.ah_build_lut.argtypes = [vp, i64, i32, vp, i32, i32, vp, vp, vp, vp, vp]
        L.ah_scan_workspace_bytes.restype = sz
        L.ah_scan_workspace_bytes.argtypes = [i64, i32, i64, i32, i32, i32]
        L.ah_scan_topk.restype = C.c_int
        L.ah_scan_topk.argtypes = [vp, i64, i32, vp, i32, i64, vp, vp, i32, vp, i32, i32, vp, vp, vp, sz, vp]
        L.ah_scan_topk_timed.restype = C.c_int
        L.ah_scan_topk_timed.argtypes = [vp, i64, i32, vp, i32, i64, vp, vp, i32, vp, i32, i32, vp, vp, vp, sz, vp,
                                         vp, vp]
        L.ah_scan_topk_residual.restype = C.c_int
        L.ah_scan_topk_residual.argtypes = [vp, i64, i32, vp, i32, i64, vp, vp, i32, vp, i32, vp, i32, i32, vp, vp,
                                            vp, sz, vp]
        L.ah_residual_leaf_bias.restype = C.c_int
        L.ah_residual_leaf_bias.argtypes = [vp, vp, i64, i32, i32, vp, vp]
        L.ah_rslm_rotate.restype = C.c_int
        L.ah_rslm_rotate.argtypes = [vp, i64, i32, vp, vp, vp, vp]
        L.ah_rslm_encode.restype = C.c_int
        L.ah_rslm_encode.argtypes = [vp, i64, i32, vp, vp, vp, vp]
        L.ah_rslm_scan_topk.restype = C.c_int
        L.ah_rslm_scan_topk.argtypes = [vp, vp, i64, vp, vp, i64, i32, vp, i32, vp, vp, vp, sz, vp]
        L.ah_kmeans_workspace_bytes.restype = sz
        L.ah_kmeans_workspace_bytes.argtypes = [i32, i32]
        L.ah_kmeans_update.restype = C.c_int
        L.ah_kmeans_update.argtypes = [vp, i64, i32, vp, i32, vp, vp, vp, sz, vp]
        L.ah_encode_sweep.restype = C.c_int
        L.ah_encode_sweep.argtypes = [vp, i32, i64, i32, vp, i32, i32, C.c_double, i32, vp, i32, vp]
        L.ah_pq_update_workspace_bytes.restype = sz
        L.ah_pq_update_workspace_bytes.argtypes = [i64, i32, i32]
        L.ah_pq_update.restype = C.c_int
        L.ah_pq_update.argtypes = [vp, i64, i32, vp, i32, i32, i32, C.c_double, vp, vp, sz, vp]
        L.ah_sq8_quantize.restype = C.c_int
        L.ah_sq8_quantize.argtypes = [vp, i64, i32, C.c_double, vp, vp, vp]
        L.ah_sq8_workspace_bytes.restype = sz
        L.ah_sq8_workspace_bytes.argtypes = [i64, i64, i32, i32]
        L.ah_sq8_scan_topk.restype = C.c_int
        L.ah_sq8_scan_topk.argtypes = [vp, vp, i64, vp, vp, i64, i32, i32, vp, vp, vp, sz, vp]
        L.ah_assign_workspace_bytes.restype = sz
        L.ah_assign_workspace_bytes.argtypes = [i64, i32]
        L.ah_assign_leaves.restype = C.c_int
        L.ah_assign_leaves.argtypes = [vp, i64, i32, vp, i32, vp, vp, vp, sz, vp]
        L.ah_encode.restype = C.c_int
        L.ah_encode.argtypes = [vp, i32, i64, i32, vp, i32, i32, C.c_double, i32, vp, i32, vp]
        L.ah_tiled_codes_bytes.restype = sz
        L.ah_tiled_codes_bytes.argtypes = [i64, i32]
        L.ah_tile_codes.restype = C.c_int
        L.ah_tile_codes.argtypes = [vp, i32, i64, i32, vp, sz, vp]
        L.ah_reorder_exact.restype = C.c_int
        L.ah_reorder_exact.argtypes = [vp, i64, i32, vp, i32, i64, vp, i32, i32, vp, vp, vp]
        L.ah_scan_topk_noalloc.restype = C.c_int
        L.ah_scan_topk_noalloc.argtypes = [vp, i64, i32, vp, i32, i64, vp, vp, i32, vp, i32, i32, vp, vp, vp]
        L.ah_scan_workspace_counters.restype = C.c_int
        L.ah_scan_workspace_counters.argtypes = [i64, i32, i64, i32, i32, i32, C.POINTER(sz), C.POINTER(sz)]
        L.ah_hbm_read_probe.restype = C.c_int
        L.ah_hbm_read_probe.argtypes = [vp, sz, i32, vp, vp]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ah_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != AH_OK:
        raise AHError(status, where)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name, ndim=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return t


# ----------------------------------------------------------------------------- step 1
def ah_partition_workspace_bytes(nq: int, L: int) -> int:
    return int(lib().ah_partition_workspace_bytes(nq, L))


def ah_partition_score(q, centroids, nl, leaves_out=None, leaf_scores_out=None, workspace=None, stream=None):
    """Best nl leaves per query (and their fp32 scores)."""
    q = _dev(q, torch.float32, "q", 2)
    centroids = _dev(centroids, torch.float32, "centroids", 2)
    nq, d = q.shape
    L = centroids.shape[0]
    if centroids.shape[1] != d:
        raise ValueError("centroids dimension differs from queries")
    if leaves_out is None:
        leaves_out = torch.empty((nq, nl), dtype=torch.int32, device=q.device)
    if leaf_scores_out is None:
        leaf_scores_out = torch.empty((nq, nl), dtype=torch.float32, device=q.device)
    _dev(leaves_out, torch.int32, "leaves_out")
    _dev(leaf_scores_out, torch.float32, "leaf_scores_out")
    need = ah_partition_workspace_bytes(nq, L)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().ah_partition_score(_ptr(q), nq, d, _ptr(centroids), L, nl, _ptr(leaves_out),
                                    _ptr(leaf_scores_out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "ah_partition_score")
    return leaves_out, leaf_scores_out


# ----------------------------------------------------------------------------- step 2
def ah_build_lut(q, codebooks, lut_i8_out=None, scale_out=None, bias_out=None, lut_f32_out=None,
                 want_f32=False, stream=None):
    """int8 tables (and optionally the fp32 ones) for a query batch.
    codebooks: float32 [B, 16, dpb]."""
    q = _dev(q, torch.float32, "q", 2)
    codebooks = _dev(codebooks, torch.float32, "codebooks", 3)
    nq, d = q.shape
    B, _, dpb = codebooks.shape
    dev = q.device
    if lut_i8_out is None:
        lut_i8_out = torch.empty((nq, B, 16), dtype=torch.int8, device=dev)
    if scale_out is None:
        scale_out = torch.empty(nq, dtype=torch.float32, device=dev)
    if bias_out is None:
        bias_out = torch.empty(nq, dtype=torch.float32, device=dev)
    if lut_f32_out is None and want_f32:
        lut_f32_out = torch.empty((nq, B, 16), dtype=torch.float32, device=dev)
    _dev(lut_i8_out, torch.int8, "lut_i8_out")
    _dev(scale_out, torch.float32, "scale_out")
    _dev(bias_out, torch.float32, "bias_out")
    _dev(lut_f32_out, torch.float32, "lut_f32_out")
    _check(lib().ah_build_lut(_ptr(q), nq, d, _ptr(codebooks), B, dpb, _ptr(lut_f32_out), _ptr(lut_i8_out),
                              _ptr(scale_out), _ptr(bias_out), _stream(stream)), "ah_build_lut")
    return lut_i8_out, scale_out, bias_out, lut_f32_out


# ----------------------------------------------------------------------------- steps 3+4
def ah_scan_workspace_bytes(nq: int, B: int, n: int, L: int, nl: int, R: int) -> int:
    return int(lib().ah_scan_workspace_bytes(nq, B, n, L, nl, R))


def ah_sq8_quantize(x, pct=99.9, codes_out=None, scale_out=None, stream=None):
    """Per-row int8 codes and float32 steps (robust percentile scale)."""
    x = _dev(x, torch.float32, "x", 2)
    n, d = x.shape
    if codes_out is None:
        codes_out = torch.empty((n, d), dtype=torch.int8, device=x.device)
    if scale_out is None:
        scale_out = torch.empty(n, dtype=torch.float32, device=x.device)
    _dev(codes_out, torch.int8, "codes_out", 2)
    _dev(scale_out, torch.float32, "scale_out", 1)
    _check(lib().ah_sq8_quantize(_ptr(x), n, d, float(pct), _ptr(codes_out), _ptr(scale_out), _stream(stream)),
           "ah_sq8_quantize")
    return codes_out, scale_out


def ah_sq8_workspace_bytes(nq: int, n: int, d: int, R: int) -> int:
    return int(lib().ah_sq8_workspace_bytes(nq, n, int(d), int(R)))


def ah_sq8_scan_topk(q8, q_scale, d8, d_scale, R, ids_out=None, scores_out=None, workspace=None, stream=None):
    """Top-R documents per query by ((float)(q8 . d8) * q_scale) * d_scale, ties to the lower id."""
    q8 = _dev(q8, torch.int8, "q8", 2)
    d8 = _dev(d8, torch.int8, "d8", 2)
    q_scale = _dev(q_scale, torch.float32, "q_scale", 1)
    d_scale = _dev(d_scale, torch.float32, "d_scale", 1)
    nq, d = q8.shape
    n = d8.shape[0]
    if ids_out is None:
        ids_out = torch.empty((nq, R), dtype=torch.int32, device=q8.device)
    if scores_out is None:
        scores_out = torch.empty((nq, R), dtype=torch.float32, device=q8.device)
    need = ah_sq8_workspace_bytes(nq, n, d, R)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q8.device)
    _check(lib().ah_sq8_scan_topk(_ptr(q8), _ptr(q_scale), nq, _ptr(d8), _ptr(d_scale), n, d, int(R), _ptr(ids_out),
                                  _ptr(scores_out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "ah_sq8_scan_topk")
    return ids_out, scores_out


def ah_rslm_rotate(x, signs, perm, y_out=None, stream=None):
    """Block Hadamard rotation of rows (sign flips, permutation, blocks of up to 128)."""
    x = _dev(x, torch.float32, "x", 2)
    n, d = x.shape
    signs = _dev(signs, torch.float32, "signs", 1)
    perm = _dev(perm, torch.int32, "perm", 1)
    if signs.numel() != d or perm.numel() != d:
        raise ValueError("signs and perm need d entries")
    if y_out is None:
        y_out = torch.empty_like(x)
    _dev(y_out, torch.float32, "y_out", 2)
    _check(lib().ah_rslm_rotate(_ptr(x), n, d, _ptr(signs), _ptr(perm), _ptr(y_out), _stream(stream)),
           "ah_rslm_rotate")
    return y_out


def ah_rslm_encode(y, levels, codes_out=None, step_out=None, stream=None):
    """4-bit nearest-level codes of rotated rows and the norm-restoring row steps;
    levels: 16 ascending floats (host)."""
    y = _dev(y, torch.float32, "y", 2)
    n, d = y.shape
    lv = np.ascontiguousarray(levels, dtype=np.float32)
    if lv.shape != (16,):
        raise ValueError("16 levels")
    if codes_out is None:
        codes_out = torch.empty((n, (d + 1) // 2), dtype=torch.uint8, device=y.device)
    if step_out is None:
        step_out = torch.empty(n, dtype=torch.float32, device=y.device)
    _dev(codes_out, torch.uint8, "codes_out", 2)
    _dev(step_out, torch.float32, "step_out", 1)
    _check(lib().ah_rslm_encode(_ptr(y), n, d, lv.ctypes.data_as(C.c_void_p), _ptr(codes_out), _ptr(step_out),
                                _stream(stream)), "ah_rslm_encode")
    return codes_out, step_out


def ah_rslm_scan_topk(q8, q_scale, codes, step, d, levels_i8, R, ids_out=None, scores_out=None, workspace=None,
                      stream=None):
    """Top-R documents per query over 4-bit codes standing for the int8 values levels_i8 (16, host)."""
    q8 = _dev(q8, torch.int8, "q8", 2)
    q_scale = _dev(q_scale, torch.float32, "q_scale", 1)
    codes = _dev(codes, torch.uint8, "codes", 2)
    step = _dev(step, torch.float32, "step", 1)
    nq = q8.shape[0]
    n = codes.shape[0]
    lv = np.ascontiguousarray(levels_i8, dtype=np.int8)
    if lv.shape != (16,) or q8.shape[1] != d or codes.shape[1] != (d + 1) // 2:
        raise ValueError("shapes")
    if ids_out is None:
        ids_out = torch.empty((nq, R), dtype=torch.int32, device=q8.device)
    if scores_out is None:
        scores_out = torch.empty((nq, R), dtype=torch.float32, device=q8.device)
    need = ah_sq8_workspace_bytes(nq, n, d, R)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q8.device)
    _check(lib().ah_rslm_scan_topk(_ptr(q8), _ptr(q_scale), nq, _ptr(codes), _ptr(step), n, d,
                                   lv.ctypes.data_as(C.c_void_p), int(R), _ptr(ids_out), _ptr(scores_out),
                                   _ptr(workspace), workspace.numel(), _stream(stream)), "ah_rslm_scan_topk")
    return ids_out, scores_out


def ah_kmeans_update(x, leaf_of_row, centroids, counts_out=None, workspace=None, stream=None):
    """In place: each leaf's centroid becomes the mean of its rows (empty leaves keep theirs).
    Returns (centroids, counts int32 [L])."""
    x = _dev(x, torch.float32, "x", 2)
    leaf_of_row = _dev(leaf_of_row, torch.int32, "leaf_of_row", 1)
    centroids = _dev(centroids, torch.float32, "centroids", 2)
    n, d = x.shape
    L = centroids.shape[0]
    if centroids.shape[1] != d or leaf_of_row.numel() != n:
        raise ValueError("shapes")
    if counts_out is None:
        counts_out = torch.empty(L, dtype=torch.int32, device=x.device)
    need = int(lib().ah_kmeans_workspace_bytes(L, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().ah_kmeans_update(_ptr(x), n, d, _ptr(leaf_of_row), L, _ptr(centroids), _ptr(counts_out),
                                  _ptr(workspace), workspace.numel(), _stream(stream)), "ah_kmeans_update")
    return centroids, counts_out


def ah_kmeans_workspace_bytes(L: int, d: int) -> int:
    return int(lib().ah_kmeans_workspace_bytes(L, d))


def ah_encode_sweep(rows, codebooks, eta, codes_inout, sweeps=1, stream=None):
    """Coupled-encoding sweeps started from the codes in codes_inout (updated in place)."""
    codebooks = _dev(codebooks, torch.float32, "codebooks", 3)
    B, _, dpb = codebooks.shape
    if rows.dtype == torch.bfloat16:
        dt = AH_BF16
    else:
        rows = _dev(rows, torch.float32, "rows", 2)
        dt = AH_F32
    n, d = rows.shape
    _dev(codes_inout, torch.uint8, "codes_inout", 2)
    _check(lib().ah_encode_sweep(_ptr(rows), dt, n, d, _ptr(codebooks), B, dpb, float(eta), int(sweeps),
                                 _ptr(codes_inout), codes_inout.shape[1], _stream(stream)), "ah_encode_sweep")
    return codes_inout


def ah_pq_update(x, codes, codebooks, eta, workspace=None, stream=None):
    """Block-by-block closed-form center update at fixed codes (codebooks updated in place)."""
    x = _dev(x, torch.float32, "x", 2)
    codes = _dev(codes, torch.uint8, "codes", 2)
    codebooks = _dev(codebooks, torch.float32, "codebooks", 3)
    n, d = x.shape
    B, _, dpb = codebooks.shape
    need = int(lib().ah_pq_update_workspace_bytes(n, B, dpb))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().ah_pq_update(_ptr(x), n, d, _ptr(codes), codes.shape[1], B, dpb, float(eta), _ptr(codebooks),
                              _ptr(workspace), workspace.numel(), _stream(stream)), "ah_pq_update")
    return codebooks


def ah_pq_update_workspace_bytes(n: int, B: int, dpb: int) -> int:
    return int(lib().ah_pq_update_workspace_bytes(n, B, dpb))


def ah_assign_workspace_bytes(n: int, L: int) -> int:
    return int(lib().ah_assign_workspace_bytes(n, L))


def ah_assign_leaves(x, centroids, leaf_out=None, score_out=None, workspace=None, want_scores=False, stream=None):
    """Nearest centroid of every row (lowest id on ties); returns (leaves int32 [n], scores or None)."""
    x = _dev(x, torch.float32, "x", 2)
    centroids = _dev(centroids, torch.float32, "centroids", 2)
    n, d = x.shape
    L = centroids.shape[0]
    if centroids.shape[1] != d:
        raise ValueError("centroids dimension differs from rows")
    if leaf_out is None:
        leaf_out = torch.empty(n, dtype=torch.int32, device=x.device)
    if score_out is None and want_scores:
        score_out = torch.empty(n, dtype=torch.float32, device=x.device)
    _dev(leaf_out, torch.int32, "leaf_out")
    _dev(score_out, torch.float32, "score_out")
    need = ah_assign_workspace_bytes(n, L)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().ah_assign_leaves(_ptr(x), n, d, _ptr(centroids), L, _ptr(leaf_out), _ptr(score_out), _ptr(workspace),
                                  workspace.numel(), _stream(stream)), "ah_assign_leaves")
    return leaf_out, score_out


def ah_encode(rows, codebooks, eta, sweeps=2, codes_out=None, stride=None, stream=None):
    """Anisotropic coupled codes of rows (float32 or bfloat16 [n, d]) for
    codebooks float32 [B, 16, dpb]; returns uint8 [n, stride]."""
    if rows.dtype == torch.float32:
        dt = AH_F32
    elif rows.dtype == torch.bfloat16:
        dt = AH_BF16
    else:
        raise TypeError("rows must be float32 or bfloat16")
    _dev(rows, rows.dtype, "rows", 2)
    codebooks = _dev(codebooks, torch.float32, "codebooks", 3)
    n, d = rows.shape
    B, _, dpb = codebooks.shape
    stride = (B + 1) // 2 if stride is None else int(stride)
    if codes_out is None:
        codes_out = torch.empty((n, stride), dtype=torch.uint8, device=rows.device)
    _dev(codes_out, torch.uint8, "codes_out", 2)
    _check(lib().ah_encode(_ptr(rows), dt, n, d, _ptr(codebooks), B, dpb, float(eta), int(sweeps), _ptr(codes_out),
                           codes_out.shape[1], _stream(stream)), "ah_encode")
    return codes_out


class TiledCodes:
    """Codes in the tiled layout of ah_tile_codes: ``data`` (uint8, device) holds
    ceil(n / 64) tiles; ``n`` rows of ``blocks`` 4-bit codes."""

    def __init__(self, data, n, blocks):
        self.data, self.n, self.blocks = data, int(n), int(blocks)


def ah_tiled_codes_bytes(n: int, B: int) -> int:
    return int(lib().ah_tiled_codes_bytes(n, B))


def ah_tile_codes(codes, B=None, stream=None) -> TiledCodes:
    """Row-major codes uint8 [n, stride] -> TiledCodes (B defaults to 2 * stride)."""
    codes = _dev(codes, torch.uint8, "codes", 2)
    n, stride = codes.shape
    B = 2 * stride if B is None else int(B)
    need = ah_tiled_codes_bytes(n, B)
    out = torch.empty(max(need, 16), dtype=torch.uint8, device=codes.device)
    _check(lib().ah_tile_codes(_ptr(codes), stride, n, B, _ptr(out), out.numel(), _stream(stream)), "ah_tile_codes")
    return TiledCodes(out, n, B)


def ah_scan_topk(lut_i8, codes, R, ids=None, leaf_offsets=None, leaves=None, cand_ids_out=None,
                 cand_scores_out=None, workspace=None, stream=None, main_events=None, leaf_bias=None,
                 bias_bound=0):
    """Top-R rows per query by exact int32 sum of table entries.
    codes: uint8 [n, stride] row-major, or TiledCodes; leaves: int32 [nq, nl] or
    None (scan all rows).  With leaf_bias (int32 [nq, nl], residual variant) the
    call is ah_scan_topk_residual: the j-th leaf's rows add its clipped bias."""
    lut_i8 = _dev(lut_i8, torch.int8, "lut_i8", 3)
    _dev(ids, torch.int32, "ids")
    _dev(leaf_offsets, torch.int64, "leaf_offsets")
    _dev(leaves, torch.int32, "leaves")
    nq, B, _ = lut_i8.shape
    if isinstance(codes, TiledCodes):
        if codes.blocks != B:
            raise ValueError("tiled codes were made for another number of blocks")
        n, stride = codes.n, AH_CODES_TILED
        codes = _dev(codes.data, torch.uint8, "codes", 1)
    else:
        codes = _dev(codes, torch.uint8, "codes", 2)
        n, stride = codes.shape
    L = 0 if leaf_offsets is None else leaf_offsets.numel() - 1
    nl = 0 if leaves is None else leaves.shape[1]
    dev = lut_i8.device
    if cand_ids_out is None:
        cand_ids_out = torch.empty((nq, R), dtype=torch.int32, device=dev)
    if cand_scores_out is None:
        cand_scores_out = torch.empty((nq, R), dtype=torch.int32, device=dev)
    _dev(cand_ids_out, torch.int32, "cand_ids_out")
    _dev(cand_scores_out, torch.int32, "cand_scores_out")
    Lw, nlw = (L, nl) if leaves is not None else (0, 0)
    need = ah_scan_workspace_bytes(nq, B, n, Lw, nlw, R)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if leaf_bias is not None:
        _dev(leaf_bias, torch.int32, "leaf_bias", 2)
        if main_events is not None:
            raise ValueError("main_events are not supported with leaf_bias")
        _check(lib().ah_scan_topk_residual(_ptr(lut_i8), nq, B, _ptr(codes), stride, n, _ptr(ids), _ptr(leaf_offsets),
                                           L, _ptr(leaves), nl, _ptr(leaf_bias), int(bias_bound), R,
                                           _ptr(cand_ids_out), _ptr(cand_scores_out), _ptr(workspace),
                                           workspace.numel(), _stream(stream)), "ah_scan_topk_residual")
        return cand_ids_out, cand_scores_out
    args = (_ptr(lut_i8), nq, B, _ptr(codes), stride, n, _ptr(ids), _ptr(leaf_offsets), L, _ptr(leaves), nl, R,
            _ptr(cand_ids_out), _ptr(cand_scores_out), _ptr(workspace), workspace.numel(), _stream(stream))
    if main_events is None:
        _check(lib().ah_scan_topk(*args), "ah_scan_topk")
    else:  # (start, stop) raw hipEvent_t handles bracketing the main scan kernel
        _check(lib().ah_scan_topk_timed(*args, C.c_void_p(main_events[0]), C.c_void_p(main_events[1])),
               "ah_scan_topk_timed")
    return cand_ids_out, cand_scores_out


AH_SCAN_SCRATCH_BYTES = 128 << 20


def ah_scan_topk_noalloc(lut_i8, codes, R, ids=None, leaf_offsets=None, leaves=None, cand_ids_out=None,
                         cand_scores_out=None, stream=None):
    """ah_scan_topk on the library's static per-GPU scratch (no workspace);
    the outputs are allocated here only when not given."""
    lut_i8 = _dev(lut_i8, torch.int8, "lut_i8", 3)
    _dev(ids, torch.int32, "ids")
    _dev(leaf_offsets, torch.int64, "leaf_offsets")
    _dev(leaves, torch.int32, "leaves")
    nq, B, _ = lut_i8.shape
    if isinstance(codes, TiledCodes):
        if codes.blocks != B:
            raise ValueError("tiled codes were made for another number of blocks")
        n, stride = codes.n, AH_CODES_TILED
        codes = _dev(codes.data, torch.uint8, "codes", 1)
    else:
        codes = _dev(codes, torch.uint8, "codes", 2)
        n, stride = codes.shape
    L = 0 if leaf_offsets is None else leaf_offsets.numel() - 1
    nl = 0 if leaves is None else leaves.shape[1]
    if cand_ids_out is None:
        cand_ids_out = torch.empty((nq, R), dtype=torch.int32, device=lut_i8.device)
    if cand_scores_out is None:
        cand_scores_out = torch.empty((nq, R), dtype=torch.int32, device=lut_i8.device)
    _dev(cand_ids_out, torch.int32, "cand_ids_out")
    _dev(cand_scores_out, torch.int32, "cand_scores_out")
    _check(lib().ah_scan_topk_noalloc(_ptr(lut_i8), nq, B, _ptr(codes), stride, n, _ptr(ids), _ptr(leaf_offsets), L,
                                      _ptr(leaves), nl, int(R), _ptr(cand_ids_out), _ptr(cand_scores_out),
                                      _stream(stream)), "ah_scan_topk_noalloc")
    return cand_ids_out, cand_scores_out


def ah_residual_leaf_bias(leaf_scores, step, bias_bound, bias_out=None, stream=None):
    """Residual variant's leaf term in table units: int32 [nq, nl] =
    clip(rint((s[q, j] - s[q, 0]) / step[q]), -bias_bound, bias_bound), 0 when step is 0."""
    leaf_scores = _dev(leaf_scores, torch.float32, "leaf_scores", 2)
    step = _dev(step, torch.float32, "step", 1)
    nq, nl = leaf_scores.shape
    if bias_out is None:
        bias_out = torch.empty((nq, nl), dtype=torch.int32, device=leaf_scores.device)
    _dev(bias_out, torch.int32, "bias_out", 2)
    _check(lib().ah_residual_leaf_bias(_ptr(leaf_scores), _ptr(step), nq, nl, int(bias_bound), _ptr(bias_out),
                                       _stream(stream)), "ah_residual_leaf_bias")
    return bias_out


# ----------------------------------------------------------------------------- step 5
def ah_reorder_exact(q, base, cand_ids, k, ids_out=None, scores_out=None, stream=None):
    """Exact rescoring of candidates; base is float32 [n, d] or bfloat16 [n, d]."""
    q = _dev(q, torch.float32, "q", 2)
    cand_ids = _dev(cand_ids, torch.int32, "cand_ids", 2)
    if base.dtype == torch.float32:
        dt = AH_F32
    elif base.dtype == torch.bfloat16:
        dt = AH_BF16
    else:
        raise TypeError("base must be float32 or bfloat16")
    _dev(base, base.dtype, "base", 2)
    nq, d = q.shape
    n = base.shape[0]
    R = cand_ids.shape[1]
    dev = q.device
    if ids_out is None:
        ids_out = torch.empty((nq, k), dtype=torch.int32, device=dev)
    if scores_out is None:
        scores_out = torch.empty((nq, k), dtype=torch.float32, device=dev)
    _dev(ids_out, torch.int32, "ids_out")
    _dev(scores_out, torch.float32, "scores_out")
    _check(lib().ah_reorder_exact(_ptr(q), nq, d, _ptr(base), dt, n, _ptr(cand_ids), R, k, _ptr(ids_out),
                                  _ptr(scores_out), _stream(stream)), "ah_reorder_exact")
    return ids_out, scores_out


# ----------------------------------------------------------------------------- measurement hooks
def ah_scan_workspace_counters(nq: int, B: int, n: int, L: int, nl: int, R: int):
    """(appended_offset, control_offset): byte offsets of the scan's counters in its workspace."""
    a, c = C.c_size_t(), C.c_size_t()
    _check(lib().ah_scan_workspace_counters(nq, B, n, L, nl, R, C.byref(a), C.byref(c)), "ah_scan_workspace_counters")
    return a.value, c.value


def scan_counters(workspace, nq: int, B: int, n: int, L: int, nl: int, R: int):
    """(appended rows per query int64 [nq], overflowed queries) as the last scan
    call on `workspace` left them (synchronises the device)."""
    a, c = ah_scan_workspace_counters(nq, B, n, L, nl, R)
    torch.cuda.synchronize()
    appended = workspace[a:a + 4 * nq].view(torch.int32).cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    ctrl = workspace[c:c + 64].view(torch.int32).cpu().numpy()
    return appended, int(ctrl[1])


def ah_hbm_read_probe(data, blocks_per_cu=8, sink=None, stream=None):
    """Plain-stream read of every byte of the device tensor `data` (16-byte loads)."""
    if not data.is_cuda or not data.is_contiguous():
        raise ValueError("data must be a contiguous device tensor")
    nbytes = data.numel() * data.element_size()
    if sink is None:
        sink = torch.zeros(4, dtype=torch.int32, device=data.device)
    _check(lib().ah_hbm_read_probe(_ptr(data), nbytes, int(blocks_per_cu), _ptr(sink), _stream(stream)),
           "ah_hbm_read_probe")
    return sink

