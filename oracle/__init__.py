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
* page "RSLM: Training-Free Vector Quantization for Approximate Nearest
  Neighbor Search", relative mode (a row coded as its residual from a coarse
  approximation, here its leaf centroid): the biased ``scan_topk`` and
  ``residual_leaf_bias``; the same page's training-free rotation quantiser
  (block Hadamard rotation, Lloyd-Max levels, norm-restoring scale) in
  ``oracle.rslm``, whose scores are those of ``sq8_topk`` on the expanded levels;
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
                                       C.c_int32, _i32p, _i32p, C.c_void_p, C.c_int32]
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
        L.oracle_kmeans_update.argtypes = [_f32p, C.c_int64, C.c_int32, _i32p, C.c_int32, _f32p, _i32p]
        L.oracle_encode.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int32, _f32p, C.c_int32, C.c_int32,
                                    C.c_double, C.c_int32, _u8p, C.c_int32, C.c_void_p]
        L.oracle_pq_update.argtypes = [_f32p, C.c_int64, C.c_int32, _u8p, C.c_int32, C.c_int32, C.c_int32,
                                       C.c_double, _f32p]
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


def scan_topk(lut_i8, codes, R, ids=None, leaf_offsets=None, leaves=None, leaf_bias=None, bias_bound=0):
    """Top-R (sum desc, id asc) per query over all rows, or over the rows of the
    leaves listed in ``leaves`` [nq, nl] (row ranges from ``leaf_offsets``).
    Residual variant: with ``leaf_bias`` int32 [nq, nl], a row of the query's
    j-th leaf scores sum + clip(leaf_bias[q, j], -bias_bound, bias_bound).
    Returns (ids int32 [nq, R], scores int32 [nq, R]); empty slots (-1, INT32_MIN)."""
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
    lb = None if leaf_bias is None else _c(leaf_bias, np.int32)
    oi = np.empty((nq, R), dtype=np.int32)
    os_ = np.empty((nq, R), dtype=np.int32)
    lib().oracle_scan_topk(lut_i8, nq, B, codes, n, stride, _ptr(ids), _ptr(lo), L, _ptr(lv), nl,
                           R, oi, os_, _ptr(lb), int(bias_bound))
    return oi, os_


def residual_leaf_bias(part_scores, step, bound):
    """Residual variant's per-leaf term in table units (the RSLM summary page's
    relative mode: score = q.c_leaf + q.residual; the table approximates
    q.residual as bias + step * sum, so q.c_leaf enters as q.c_leaf / step):
    int32 [nq, nl] = clip(rint((s[q, j] - s[q, 0]) / step[q]), -bound, bound)
    from the query's leaf scores ``part_scores`` float32 [nq, nl] (first = the
    leaf everything is measured from), all in float32, rint half to even;
    a query with step 0 gets 0 everywhere."""
    s = _c(part_scores, np.float32)
    st = _c(step, np.float32)
    diff = s - s[:, :1]
    out = np.zeros(s.shape, dtype=np.int32)
    pos = st > 0
    v = np.rint(diff[pos] / st[pos][:, None])
    out[pos] = np.clip(v, -bound, bound).astype(np.int32)
    return out


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


def kmeans_update(X, leaf, centroids):
    """The k-means update: each leaf's centroid becomes the float64 mean of its
    rows (in row order), rounded to float32; empty leaves keep theirs.
    Returns (centroids float32 [L, d], counts int32 [L])."""
    X = _c(X, np.float32)
    lf = _c(leaf, np.int32)
    Cn = np.array(centroids, dtype=np.float32, copy=True, order="C")
    cnt = np.empty(Cn.shape[0], dtype=np.int32)
    lib().oracle_kmeans_update(X, X.shape[0], X.shape[1], lf, Cn.shape[0], Cn, cnt)
    return Cn, cnt


def pq_update(X, codes, codebooks, eta):
    """One block-by-block closed-form center update of anisotropic codebook
    training at fixed codes; returns the new codebooks float32 [B, 16, dpb]."""
    X = _c(X, np.float32)
    cd = _c(codes, np.uint8)
    cb = np.array(codebooks, dtype=np.float32, copy=True, order="C")
    B, _, dpb = cb.shape
    lib().oracle_pq_update(X, X.shape[0], X.shape[1], cd, cd.shape[1], B, dpb, float(eta), cb)
    return cb


def encode(rows, codebooks, eta, sweeps=2, stride=None, init_codes=None):
    """Anisotropic coupled encoding (block-coordinate descent from the per-block
    nearest centers, or from init_codes).  rows: float32 [n, d] or bfloat16 bits
    as uint16 [n, d]; codebooks float32 [B, 16, dpb].  Returns uint8 [n, stride]
    nibble codes."""
    b, dt = _base_args(rows)
    cb = _c(codebooks, np.float32)
    B, _, dpb = cb.shape
    n, d = b.shape
    if d != B * dpb:
        raise ValueError("rows do not have B * dpb columns")
    stride = (B + 1) // 2 if stride is None else int(stride)
    out = np.zeros((n, stride), dtype=np.uint8)
    ic = None if init_codes is None else _c(init_codes, np.uint8)
    if ic is not None and ic.shape != (n, stride):
        raise ValueError("init_codes must be [n, stride]")
    lib().oracle_encode(_ptr(b), dt, n, d, cb, B, dpb, float(eta), int(sweeps), out, stride, _ptr(ic))
    return out


def recall_at_k(found: np.ndarray, truth: np.ndarray) -> float:
    """Mean over queries of |found_k intersect true_k| / k (intersection recall of
    the ScaNN page's "Measuring recall honestly" and the compression lesson's
    recall@k); entries < 0 in ``found`` are empty slots."""
    total = 0
    for f, t in zip(np.asarray(found), np.asarray(truth)):
        total += len(set(int(x) for x in f if x >= 0) & set(int(x) for x in t))
    return total / float(np.asarray(truth).size) if np.asarray(truth).size else 1.0


def search(Q, codebooks, codes, base, R, k, centroids=None, leaf_offsets=None, ids=None, nl=0,
           residual_bound=None):
    """The whole path on the CPU, each step fed the previous step's output:
    leaves (if partitioned) -> float64 table rounded to float32 -> int8 table ->
    top-R by integer sum -> exact reorder to the best k.  With
    ``residual_bound`` (partitioned, codes of residuals from the leaf
    centroids), the leaf scores rounded to float32 become per-leaf terms in
    table units (``residual_leaf_bias``) added to the sums.
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
    lb = None
    if residual_bound is not None and leaves is not None:
        lb = residual_leaf_bias(out["leaf_scores"].astype(np.float32), s, residual_bound)
        out["leaf_bias"] = lb
    ci, cs = scan_topk(t8, codes, R, ids=ids, leaf_offsets=leaf_offsets, leaves=leaves, leaf_bias=lb,
                       bias_bound=0 if lb is None else residual_bound)
    out["cand_ids"], out["cand_sums"] = ci, cs
    fi, fs = reorder(Q, base, ci, k)
    out["ids"], out["scores"] = fi, fs
    return out
