"""Host-side index build: partition k-means, anisotropic PQ codebooks, coupled
encoding, leaf sort.

Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
Product Search": "The loss in one paragraph" (eta and its large-d limit),
"Training an anisotropic codebook yourself" (the trainer), "Three stages of a
search" (partition into leaves; blocks of dimensions_per_block dims, 16 centers
each) and "Using the library" (training on a sample of up to 250,000 rows).

Two builders of the same index:
- build(): on the host -- codebook training and encoding in the C++ host
  library (include/ah_index.h, libah_index.so), the partition k-means with
  numpy BLAS;
- build_gpu(): every step on the GPU through include/ah.h (ah_assign_leaves +
  ah_kmeans_update for the partition, ah_encode / ah_encode_sweep +
  ah_pq_update for the codebooks, ah_assign_leaves + ah_encode over all rows),
  for databases whose host build would take minutes (20M x 384).
Either way the index arrays are then passed to the search calls of
include/ah.h.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libah_index.so")
_hl = None

SAMPLE_ROWS = 250_000
ITERS = 10


def _host():
    global _hl
    if _hl is None:
        if not os.path.exists(HOST_LIB):
            from . import build
            build.build_host()
        L = C.CDLL(HOST_LIB)
        f32 = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        i64 = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        u8 = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
        L.ahx_train_pq.restype = C.c_int
        L.ahx_train_pq.argtypes = [f32, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_double, C.c_int32,
                                   i64, f32, C.c_void_p]
        L.ahx_encode.restype = C.c_int
        L.ahx_encode.argtypes = [f32, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_double, f32, C.c_int32,
                                 u8, C.c_int32]
        L.ahx_train_pq_dir.restype = C.c_int
        L.ahx_train_pq_dir.argtypes = [f32, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_double,
                                       C.c_int32, i64, f32, C.c_void_p]
        L.ahx_encode_dir.restype = C.c_int
        L.ahx_encode_dir.argtypes = [f32, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_double, f32,
                                     C.c_int32, u8, C.c_int32]
        L.ahx_loss.restype = C.c_double
        L.ahx_loss.argtypes = [f32, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_double, f32, u8, C.c_int32]
        _hl = L
    return _hl


# ------------------------------------------------------------------------- eta
def eta_for(d: int, T: float, norms) -> np.ndarray:
    """Large-dimension limit of h_par/h_perp for the threshold weight (ScaNN page,
    "The loss in one paragraph"): (d-1) r / (1-r), r = (T/|x|)^2."""
    r = (T / np.asarray(norms, dtype=np.float64)) ** 2
    if np.any(r >= 1):
        raise ValueError("T must be below every row norm")
    return (d - 1) * r / (1 - r)


def relative_threshold_for_eta(d: int, eta: float) -> float:
    """T/|x| that gives weight ratio eta in dimension d (inverse of eta_for)."""
    return float(np.sqrt(eta / (d - 1 + eta)))


# ------------------------------------------------------------------------- PQ
def _dirs(dirs, X):
    if dirs is None:
        return None, None
    V = np.ascontiguousarray(dirs, dtype=np.float32)
    if V.shape != X.shape:
        raise ValueError("direction rows must match the rows")
    return V, V.ctypes.data_as(C.c_void_p)


def train_codebooks(X: np.ndarray, dpb: int, eta: float, iters: int = ITERS, seed=0, init_rows=None,
                    return_loss: bool = False, dirs: np.ndarray | None = None):
    """Anisotropic PQ codebooks float32 [B, 16, dpb] trained on rows X (dirs:
    rows whose directions weight the loss instead of X's own, e.g. the original
    rows when X holds residuals)."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    V, vp = _dirs(dirs, X)
    m, d = X.shape
    B = d // dpb
    if init_rows is None:
        init_rows = np.random.default_rng(seed).choice(m, 16, replace=False)
    init_rows = np.ascontiguousarray(init_rows, dtype=np.int64)
    cb = np.empty((B, 16, dpb), dtype=np.float32)
    loss = np.empty(iters + 1, dtype=np.float64)
    rc = _host().ahx_train_pq_dir(X, vp, m, d, B, dpb, float(eta), iters, init_rows, cb,
                                  loss.ctypes.data_as(C.c_void_p))
    if rc != 0:
        raise ValueError("ahx_train_pq: bad arguments")
    return (cb, loss) if return_loss else cb


def encode(X: np.ndarray, codebooks: np.ndarray, eta: float, sweeps: int = 2, stride: int | None = None,
           dirs: np.ndarray | None = None) -> np.ndarray:
    """Row-major nibble codes uint8 [n, stride] (low nibble = even block); dirs
    as in train_codebooks."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    V, vp = _dirs(dirs, X)
    cb = np.ascontiguousarray(codebooks, dtype=np.float32)
    B, _, dpb = cb.shape
    stride = (B + 1) // 2 if stride is None else stride
    out = np.empty((X.shape[0], stride), dtype=np.uint8)
    rc = _host().ahx_encode_dir(X, vp, X.shape[0], X.shape[1], B, dpb, float(eta), cb, sweeps, out, stride)
    if rc != 0:
        raise ValueError("ahx_encode: bad arguments")
    return out


def pq_loss(X, codebooks, codes, eta) -> float:
    X = np.ascontiguousarray(X, dtype=np.float32)
    cb = np.ascontiguousarray(codebooks, dtype=np.float32)
    B, _, dpb = cb.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    return float(_host().ahx_loss(X, X.shape[0], X.shape[1], B, dpb, float(eta), cb, codes, codes.shape[1]))


# ------------------------------------------------------------------------- partition
def nearest_centroid(X: np.ndarray, Cn: np.ndarray, chunk: int = 32768) -> np.ndarray:
    """Index of the L2-nearest centroid of every row (lowest index on ties)."""
    Cd = Cn.astype(np.float64)
    cn2 = np.einsum("ij,ij->i", Cd, Cd)
    out = np.empty(X.shape[0], dtype=np.int32)
    for a in range(0, X.shape[0], chunk):
        xb = X[a:a + chunk].astype(np.float64)
        dist = cn2[None, :] - 2.0 * (xb @ Cd.T)
        out[a:a + chunk] = np.argmin(dist, axis=1)
    return out


def kmeans(X: np.ndarray, k: int, iters: int = ITERS, seed=0, init_rows=None):
    """Lloyd k-means (squared L2), init = k distinct rows, empty clusters keep
    their center.  Returns (centroids float32 [k, d], assignment)."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    if init_rows is None:
        init_rows = np.random.default_rng(seed).choice(X.shape[0], k, replace=False)
    Cn = X[np.asarray(init_rows)].astype(np.float32).copy()
    assign = nearest_centroid(X, Cn)
    for _ in range(iters):
        sums = np.zeros((k, X.shape[1]), dtype=np.float64)
        np.add.at(sums, assign, X.astype(np.float64))
        cnt = np.bincount(assign, minlength=k)
        nz = cnt > 0
        Cn[nz] = (sums[nz] / cnt[nz, None]).astype(np.float32)
        assign = nearest_centroid(X, Cn)
    return Cn, assign


def train_codebooks_gpu(X, dpb: int, eta: float, iters: int = ITERS, seed=0, init_rows=None):
    """The same training iterations as train_codebooks on the GPU: codebooks
    seeded from 16 rows, then per iteration one coupled-encoding sweep (from
    the per-block nearest centers the first time, else from the current codes)
    and the block-by-block center update.  X: float32 device tensor [m, d].
    Returns (codebooks float32 device tensor [B, 16, dpb], codes uint8 [m, ceil(B/2)])."""
    from . import ahlib
    import torch
    m, d = X.shape
    B = d // dpb
    if init_rows is None:
        init_rows = np.random.default_rng(seed).choice(m, 16, replace=False)
    rows = X[torch.as_tensor(np.asarray(init_rows), device=X.device, dtype=torch.long)]  # [16, d]
    cb = rows.view(16, B, dpb).permute(1, 0, 2).contiguous()
    ws = torch.empty(max(ahlib.ah_pq_update_workspace_bytes(m, B, dpb), 1), dtype=torch.uint8, device=X.device)
    codes = None
    for it in range(iters):
        if codes is None:
            codes = ahlib.ah_encode(X, cb, eta, sweeps=1)
        else:
            ahlib.ah_encode_sweep(X, cb, eta, codes, sweeps=1)
        ahlib.ah_pq_update(X, codes, cb, eta, workspace=ws)
    if codes is None:
        codes = ahlib.ah_encode(X, cb, eta, sweeps=0)
    return cb, codes


def kmeans_gpu(X, k: int, iters: int = ITERS, seed=0, init_rows=None):
    """The same Lloyd iterations as kmeans() on the GPU (ah_assign_leaves, then
    ah_kmeans_update).  X: float32 device tensor [n, d].  Returns (centroids
    float32 device tensor [k, d], assignment int32 device tensor [n])."""
    from . import ahlib
    n = X.shape[0]
    if init_rows is None:
        init_rows = np.random.default_rng(seed).choice(n, k, replace=False)
    import torch
    C = X[torch.as_tensor(np.asarray(init_rows), device=X.device, dtype=torch.long)].clone()
    ws_a = ws_k = None
    leaf = None
    for _ in range(iters):
        if ws_a is None:
            ws_a = torch.empty(ahlib.ah_assign_workspace_bytes(n, k), dtype=torch.uint8, device=X.device)
            ws_k = torch.empty(ahlib.ah_kmeans_workspace_bytes(k, X.shape[1]), dtype=torch.uint8, device=X.device)
        leaf, _ = ahlib.ah_assign_leaves(X, C, workspace=ws_a)
        ahlib.ah_kmeans_update(X, leaf, C, workspace=ws_k)
    leaf, _ = ahlib.ah_assign_leaves(X, C, workspace=ws_a) if iters else ahlib.ah_assign_leaves(X, C)
    return C, leaf


def leaf_sort(assign: np.ndarray, num_leaves: int):
    """Rows grouped by leaf, ascending id inside each leaf.
    Returns (ids int32 [n] original row of each position, leaf_offsets int64 [L+1])."""
    ids = np.argsort(assign, kind="stable").astype(np.int32)
    cnt = np.bincount(assign, minlength=num_leaves)
    offs = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int64)
    return ids, offs


# ------------------------------------------------------------------------- whole index
@dataclasses.dataclass
class HostIndex:
    codebooks: np.ndarray            # float32 [B, 16, dpb]
    codes: np.ndarray                # uint8 [n, stride], leaf-sorted when partitioned
    ids: np.ndarray | None           # int32 [n] original row of each code row (None = identity)
    centroids: np.ndarray | None     # float32 [L, d]
    leaf_offsets: np.ndarray | None  # int64 [L+1]
    eta: float
    residual: bool = False           # codes hold x - centroid(leaf) (the RSLM summary page's relative mode)


def build(X: np.ndarray, dpb: int, eta: float, num_leaves: int = 0, seed: int = 0, sample_rows: int = SAMPLE_ROWS,
          iters: int = ITERS, sweeps: int = 2, residual: bool = False) -> HostIndex:
    """Train and encode an index over rows X (float32 [n, d]).  residual (with
    num_leaves > 0): the codebooks are trained on, and the codes encode, each
    row's residual from its leaf centroid, x - c_leaf (float32), with the
    anisotropic weight along the original row x (the score error q.(r - r~)
    has its parallel part along x)."""
    n = X.shape[0]
    rng = np.random.default_rng(seed)
    sample = np.sort(rng.choice(n, min(n, sample_rows), replace=False)) if n > sample_rows else np.arange(n)
    Xs = X[sample]
    centroids = leaf_offsets = ids = assign = None
    if num_leaves > 0:
        centroids, _ = kmeans(Xs, num_leaves, iters, seed=rng)
        assign = nearest_centroid(X, centroids)
        ids, leaf_offsets = leaf_sort(assign, num_leaves)
    residual = residual and centroids is not None
    if residual:
        cb = train_codebooks(Xs - centroids[assign[sample]], dpb, eta, iters, seed=rng, dirs=Xs)
        codes = np.empty((n, (cb.shape[0] + 1) // 2), dtype=np.uint8)
        for a in range(0, n, 1 << 18):  # residual rows a chunk at a time
            b = min(n, a + (1 << 18))
            codes[a:b] = encode(X[a:b] - centroids[assign[a:b]], cb, eta, sweeps, dirs=X[a:b])
    else:
        cb = train_codebooks(Xs, dpb, eta, iters, seed=rng)
        codes = encode(X, cb, eta, sweeps)
    if ids is not None:
        codes = np.ascontiguousarray(codes[ids])
    return HostIndex(cb, codes, ids, centroids, leaf_offsets, eta, residual)


@dataclasses.dataclass
class DeviceIndex:
    """The index arrays as torch device tensors (same layout as HostIndex)."""
    codebooks: object                # float32 [B, 16, dpb]
    codes: object                    # uint8 [n, stride], leaf-sorted when partitioned
    ids: object | None               # int32 [n]
    centroids: object | None         # float32 [L, d]
    leaf_offsets: object | None      # int64 [L+1]
    eta: float
    residual: bool = False

    def to_host(self) -> HostIndex:
        g = lambda t: None if t is None else t.cpu().numpy()  # noqa: E731
        return HostIndex(g(self.codebooks), g(self.codes), g(self.ids), g(self.centroids), g(self.leaf_offsets),
                         self.eta, self.residual)


def build_gpu(X, dpb: int, eta: float, num_leaves: int = 0, seed=0, sample_rows: int = SAMPLE_ROWS,
              iters: int = ITERS, sweeps: int = 2, chunk_rows: int = 1 << 21, timings: dict | None = None):
    """The steps of build() on the GPU.  X: device tensor [n, d], float32 or
    bfloat16 (the stored rows; training sees them widened exactly to float32).
    Partition: Lloyd k-means on a sample of up to sample_rows rows (init = L
    distinct sample rows), then every row's nearest centroid; codebooks:
    anisotropic training on the same sample (train_codebooks_gpu); codes: the
    coupled encoding of every row; leaf sort: rows grouped by leaf, ascending
    row id inside a leaf.  The random draws (sample, initial rows) come from
    numpy's default_rng(seed) in the same order as build().  timings, if given,
    receives each step's wall time in seconds (device-synchronised).
    Returns a DeviceIndex."""
    import time
    import torch
    from . import ahlib
    n, d = X.shape
    dev = X.device
    rng = np.random.default_rng(seed)
    t = {} if timings is None else timings

    def mark(name, t0):
        torch.cuda.synchronize()
        t[name] = time.perf_counter() - t0
        return time.perf_counter()

    t0 = time.perf_counter()
    sample = np.sort(rng.choice(n, min(n, sample_rows), replace=False)) if n > sample_rows else np.arange(n)
    Xs = X[torch.as_tensor(sample, device=dev, dtype=torch.long)].to(torch.float32).contiguous()
    m = Xs.shape[0]
    centroids = ids = offsets = None
    if num_leaves > 0:
        centroids, _ = kmeans_gpu(Xs, num_leaves, iters, init_rows=rng.choice(m, num_leaves, replace=False))
        t0 = mark("partition_kmeans", t0)
        leaf = torch.empty(n, dtype=torch.int32, device=dev)
        ws = torch.empty(ahlib.ah_assign_workspace_bytes(min(n, chunk_rows), num_leaves), dtype=torch.uint8,
                         device=dev)
        for a in range(0, n, chunk_rows):
            b = min(n, a + chunk_rows)
            ahlib.ah_assign_leaves(X[a:b].to(torch.float32).contiguous(), centroids, leaf_out=leaf[a:b],
                                   workspace=ws)
        del ws
        t0 = mark("partition_assign", t0)
    cb, _ = train_codebooks_gpu(Xs, dpb, eta, iters, init_rows=rng.choice(m, 16, replace=False))
    del Xs
    t0 = mark("codebook_training", t0)
    # rows padded with zero bytes to a multiple of 16 (the scan's aligned,
    # one-load-per-segment code paths need it; 25-byte rows otherwise take
    # byte-wise loads everywhere)
    B = cb.shape[0]
    stride = ((B + 1) // 2 + 15) // 16 * 16
    codes = torch.zeros((n, stride), dtype=torch.uint8, device=dev)
    ahlib.ah_encode(X if X.dtype in (torch.float32, torch.bfloat16) else X.to(torch.float32), cb, eta,
                    sweeps=sweeps, codes_out=codes)
    t0 = mark("encode", t0)
    if num_leaves > 0:
        order = torch.sort(leaf, stable=True).indices
        ids = order.to(torch.int32)
        counts = torch.bincount(leaf, minlength=num_leaves)
        offsets = torch.zeros(num_leaves + 1, dtype=torch.int64, device=dev)
        offsets[1:] = torch.cumsum(counts, 0)
        codes = codes[order].contiguous()
        del order, leaf
        t0 = mark("leaf_sort", t0)
    return DeviceIndex(cb, codes, ids, centroids, offsets, float(eta))


def save(path: str, ix: HostIndex) -> None:
    arrs = {"codebooks": ix.codebooks, "codes": ix.codes, "eta": np.array(ix.eta), "residual": np.array(ix.residual)}
    for k in ("ids", "centroids", "leaf_offsets"):
        v = getattr(ix, k)
        if v is not None:
            arrs[k] = v
    tmp = path + ".tmp.npz"
    np.savez(tmp, **arrs)
    os.replace(tmp, path)


def load(path: str) -> HostIndex:
    z = np.load(path, allow_pickle=False)
    g = lambda k: z[k] if k in z.files else None  # noqa: E731
    res = bool(z["residual"]) if "residual" in z.files else False
    return HostIndex(z["codebooks"], z["codes"], g("ids"), g("centroids"), g("leaf_offsets"), float(z["eta"]), res)
