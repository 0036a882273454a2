"""CPU oracle for the asymmetric-hashing search path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``mips_ah_partition_amd``) and never imports it; both sides take their inputs
from ``synth``.

The arithmetic lives in ``oracle.c`` (plain scalar C, float64 for floating
point except the int8 table quantisation, which is defined in float32); this
module wraps it with ctypes and adds the recall measure.  Each function names
the passage it follows:

* page "ScaNN: Anisotropic Vector Quantization for Maximum Inner Product
  Search", section "Three stages of a search": partition scoring
  (``partition``), per-block table of q.center (``lut_f64``), approximate score
  = sum of the row's table entries (``scan_sums``/``scan_topk``), exact reorder
  of the best candidates (``reorder``);
* same page, section "Measuring recall honestly", and the compression lesson's
  "Measuring what compression costs: recall@k": ``recall_at_k`` and the exact
  ground truth ``brute_force``.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, brute force on tiny inputs, the pages' worked examples
(``tests/golden/``) and special cases.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")


def lib() -> C.CDLL:
    global _LIB
    if _LIB is None:
        from . import build as _build
        path = _build.build(force=False)
        L = C.CDLL(path)
        L.oracle_num_threads.restype = C.c_int
        L.oracle_set_threads.argtypes = [C.c_int]
        L.oracle_scan_sums.argtypes = [_i8p, C.c_int64, C.c_int32, _u8p, C.c_int64, C.c_int32, _i32p]
        L.oracle_scan_topk.argtypes = [_i8p, C.c_int64, C.c_int32, _u8p, C.c_int64, C.c_int32,
                                       C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32,
                                       C.c_int32, _i32p, _i32p]
        L.oracle_lut_f64.argtypes = [_f32p, C.c_int64, C.c_int32, _f32p, C.c_int32, C.c_int32, _f64p]
        L.oracle_quantize_lut.argtypes = [_f32p, C.c_int64, C.c_int32, _i8p, _f32p, _f32p]
        L.oracle_reorder.argtypes = [_f32p, C.c_int64, C.c_int32, C.c_void_p, C.c_int32, C.c_int64,
                                     _i32p, C.c_int32, C.c_int32, _i32p, _f64p]
        L.oracle_partition.argtypes = [_f32p, C.c_int64, C.c_int32, _f32p, C.c_int32, C.c_int32,
                                       _i32p, _f64p]
        L.oracle_brute_force.argtypes = [_f32p, C.c_int64, C.c_int32, C.c_void_p, C.c_int32,
                                         C.c_int64, C.c_int32, _i32p, _f64p]
        L.oracle_sq8_quantize.argtypes = [_f32p, C.c_int64, C.c_int32, C.c_double, _i8p, _f32p]
        L.oracle_sq8_topk.argtypes = [_i8p, _f32p, C.c_int64, _i8p, _f32p, C.c_int64, C.c_int32, C.c_int32,
                                      _i32p, _f32p]
        L.oracle_nearest.argtypes = [_f32p, C.c_int64, C.c_int32, _f32p, C.c_int32, _i32p, _f64p]
        L.oracle_encode.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int32, _f32p, C.c_int32, C.c_int32,
                                    C.c_double, C.c_int32, _u8p, C.c_int32]
        _LIB = L
    return _LIB


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(t: int) -> None:
    lib().oracle_set_threads(int(t))


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def scan_sums(lut_i8: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """int32 [nq, n]: sum over blocks of lut_i8[q, b, code(i, b)]."""
    lut_i8 = _c(lut_i8, np.int8)
    codes = _c(codes, np.uint8)
    nq, B, _ = lut_i8.shape
    n = codes.shape[0]
    out = np.empty((nq, n), dtype=np.int32)
    lib().oracle_scan_sums(lut_i8, nq, B, codes, n, codes.shape[1] if n else (B + 1) // 2, out)
    return out


def scan_topk(lut_i8, codes, R, ids=None, leaf_offsets=None, leaves=None):
    """Top-R (sum desc, id asc) per query over all rows, or over the rows of the
    leaves listed in ``leaves`` [nq, nl] (row ranges from ``leaf_offsets``).
    Returns (ids int32 [nq, R], sums int32 [nq, R]); empty slots (-1, INT32_MIN)."""
    lut_i8 = _c(lut_i8, np.int8)
    codes = _c(codes, np.uint8)
    nq, B, _ = lut_i8.shape
    n = codes.shape[0]
    stride = codes.shape[1] if codes.ndim == 2 and n else (B + 1) // 2
    ids = None if ids is None else _c(ids, np.int32)
    lo = None if leaf_offsets is None else _c(leaf_offsets, np.int64)
    lv = None if leaves is None else _c(leaves, np.int32)
    nl = 0 if lv is None else lv.shape[1]
    L = 0 if lo is None else lo.shape[0] - 1
    oi = np.empty((nq, R), dtype=np.int32)
    os_ = np.empty((nq, R), dtype=np.int32)
    lib().oracle_scan_topk(lut_i8, nq, B, codes, n, stride, _ptr(ids), _ptr(lo), L, _ptr(lv), nl,
                           R, oi, os_)
    return oi, os_


def lut_f64(Q: np.ndarray, codebooks: np.ndarray) -> np.ndarray:
    """float64 [nq, B, 16]: q . center for every block and center;
    codebooks is float32 [B, 16, dpb]."""
    Q = _c(Q, np.float32)
    cb = _c(codebooks, np.float32)
    B, _, dpb = cb.shape
    out = np.empty((Q.shape[0], B, 16), dtype=np.float64)
    lib().oracle_lut_f64(Q, Q.shape[0], Q.shape[1], cb, B, dpb, out)
    return out


def quantize_lut(lut_f32: np.ndarray):
    """int8 table, per-query step s and bias beta from a float32 table [nq, B, 16]."""
    t = _c(lut_f32, np.float32)
    nq, B, _ = t.shape
    out = np.empty((nq, B, 16), dtype=np.int8)
    s = np.empty(nq, dtype=np.float32)
    beta = np.empty(nq, dtype=np.float32)
    lib().oracle_quantize_lut(t, nq, B, out, s, beta)
    return out, s, beta


def _base_args(base: np.ndarray):
    if base.dtype == np.float32:
        return _c(base, np.float32), 0
    if base.dtype == np.uint16:  # raw bf16 bits
        return _c(base, np.uint16), 1
    raise TypeError("rows must be float32 or bf16 bits (uint16)")


def reorder(Q, base, cand_ids, k):
    """Exact float64 rescoring of each query's candidates (-1 = empty);
    best k by (score desc, id asc). Returns (ids int32, scores float64)."""
    Q = _c(Q, np.float32)
    b, dt = _base_args(base)
    cand = _c(cand_ids, np.int32)
    nq, R = cand.shape
    oi = np.empty((nq, k), dtype=np.int32)
    osc = np.empty((nq, k), dtype=np.float64)
    lib().oracle_reorder(Q, nq, Q.shape[1], _ptr(b), dt, b.shape[0], cand, R, k, oi, osc)
    return oi, osc


def partition(Q, centroids, nl):
    """float64 centroid scores; best nl leaves by (score desc, leaf asc)."""
    Q = _c(Q, np.float32)
    Cn = _c(centroids, np.float32)
    nq = Q.shape[0]
    ol = np.empty((nq, nl), dtype=np.int32)
    osc = np.empty((nq, nl), dtype=np.float64)
    lib().oracle_partition(Q, nq, Q.shape[1], Cn, Cn.shape[0], nl, ol, osc)
    return ol, osc


def brute_force(Q, base, k):
    """Exact top-k by float64 dot product over every stored row."""
    Q = _c(Q, np.float32)
    b, dt = _base_args(base)
    nq = Q.shape[0]
    oi = np.empty((nq, k), dtype=np.int32)
    osc = np.empty((nq, k), dtype=np.float64)
    lib().oracle_brute_force(Q, nq, Q.shape[1], _ptr(b), dt, b.shape[0], k, oi, osc)
    return oi, osc


def sq8_quantize(X, pct=99.9):
    """Per-vector int8 codes and float32 steps (robust percentile scale)."""
    X = _c(X, np.float32)
    n, d = X.shape
    codes = np.empty((n, d), dtype=np.int8)
    scale = np.empty(n, dtype=np.float32)
    lib().oracle_sq8_quantize(X, n, d, float(pct), codes, scale)
    return codes, scale


def sq8_topk(q8, qs, d8, ds, R):
    """Top-R documents per query by (float)(q8 . d8) * s_q * s_d, ties to the lower id."""
    q8, d8 = _c(q8, np.int8), _c(d8, np.int8)
    qs, ds = _c(qs, np.float32), _c(ds, np.float32)
    nq, d = q8.shape
    n = d8.shape[0]
    ids = np.empty((nq, R), dtype=np.int32)
    sc = np.empty((nq, R), dtype=np.float32)
    lib().oracle_sq8_topk(q8, qs, nq, d8, ds, n, d, int(R), ids, sc)
    return ids, sc


def nearest(X, centroids):
    """Nearest centroid per row (float64 squared distance, lowest id on ties):
    (ids int32 [n], squared distances float64 [n])."""
    X = _c(X, np.float32)
    Cn = _c(centroids, np.float32)
    n, d = X.shape
    ids = np.empty(n, dtype=np.int32)
    dist = np.empty(n, dtype=np.float64)
    lib().oracle_nearest(X, n, d, Cn, Cn.shape[0], ids, dist)
    return ids, dist


def encode(rows, codebooks, eta, sweeps=2, stride=None):
    """Anisotropic coupled encoding (block-coordinate descent from the per-block
    nearest centers).  rows: float32 [n, d] or bfloat16 bits as uint16 [n, d];
    codebooks float32 [B, 16, dpb].  Returns uint8 [n, stride] nibble codes."""
    b, dt = _base_args(rows)
    cb = _c(codebooks, np.float32)
    B, _, dpb = cb.shape
    n, d = b.shape
    if d != B * dpb:
        raise ValueError("rows do not have B * dpb columns")
    stride = (B + 1) // 2 if stride is None else int(stride)
    out = np.zeros((n, stride), dtype=np.uint8)
    lib().oracle_encode(_ptr(b), dt, n, d, cb, B, dpb, float(eta), int(sweeps), out, stride)
    return out


def recall_at_k(found: np.ndarray, truth: np.ndarray) -> float:
    """Mean over queries of |found_k intersect true_k| / k (intersection recall of
    the ScaNN page's "Measuring recall honestly" and the compression lesson's
    recall@k); entries < 0 in ``found`` are empty slots."""
    total = 0
    for f, t in zip(np.asarray(found), np.asarray(truth)):
        total += len(set(int(x) for x in f if x >= 0) & set(int(x) for x in t))
    return total / float(np.asarray(truth).size) if np.asarray(truth).size else 1.0


def search(Q, codebooks, codes, base, R, k, centroids=None, leaf_offsets=None, ids=None, nl=0):
    """The whole path on the CPU, each step fed the previous step's output:
    leaves (if partitioned) -> float64 table rounded to float32 -> int8 table ->
    top-R by integer sum -> exact reorder to the best k.
    Returns dict with every intermediate."""
    out = {}
    leaves = None
    if centroids is not None and nl > 0:
        leaves, lsc = partition(Q, centroids, nl)
        out["leaves"], out["leaf_scores"] = leaves, lsc
    lf = lut_f64(Q, codebooks)
    l32 = lf.astype(np.float32)
    t8, s, beta = quantize_lut(l32)
    out.update(lut_f64=lf, lut_f32=l32, lut_i8=t8, scale=s, bias=beta)
    ci, cs = scan_topk(t8, codes, R, ids=ids, leaf_offsets=leaf_offsets, leaves=leaves)
    out["cand_ids"], out["cand_sums"] = ci, cs
    fi, fs = reorder(Q, base, ci, k)
    out["ids"], out["scores"] = fi, fs
    return out
