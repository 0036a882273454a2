"""Training-free rotation quantiser (RSLM) -- TEST INFRASTRUCTURE, part of the oracle.

Follows the page "RSLM: Training-Free Vector Quantization for Approximate
Nearest Neighbor Search", method points: a block-wise cascaded fast
Walsh-Hadamard rotation with block size 128, sign flips and a permutation to
even out the coordinates (tail dimensions handled by an overlapping block); a
fixed Lloyd-Max codebook of at most 16 centroids for the rotated, near-Gaussian
coordinates; and a global scale that restores the L2 norm of the final
reconstruction (important for inner-product ranking).

Plain float64 numpy; nothing here is shared with the GPU library.  Readings
where the page is silent:
  * block size b = min(128, largest power of two <= d); blocks [k b, (k+1) b)
    for k < d // b, then, when b does not divide d, the tail block [d-b, d);
    each block gets the orthonormal Sylvester Hadamard matrix H_b / sqrt(b),
    the blocks applied in that order (the tail overlaps and comes last);
  * before the blocks: y = x * signs, then y'[j] = y[perm[j]];
  * the 16 levels are the Lloyd-Max quantiser of N(0, 1) (the rotated
    coordinates of a vector scaled to norm sqrt(d) are near N(0, 1));
  * encoding in float32 decisions: ss = sum y_j^2 (float64), f =
    float32(sqrt(d) / sqrt(ss)) (0 when ss = 0), u_j = float32(y_j * f),
    code_j = number of midpoints m_c = float32((L_c + L_{c+1}) / 2) below u_j
    (strictly), i.e. the nearest level with ties to the lower one;
  * global scale gamma = sqrt(ss) / sqrt(sum_j L[code_j]^2) (float64, L as
    float32), so the reconstruction gamma * L[code] has the row's norm;
  * scoring on the int8 matrix cores: the levels as int8 lv_c = rint(L_c * Lam),
    Lam = 127 / L_15, the row's step float32(gamma / Lam), the query's int8
    codes and step from the int8 flat-search quantiser; the score is that of
    the int8 flat search, ((float)dot * s_q) * s_d, with dot the exact
    integer q8 . lv[code].
"""
from __future__ import annotations

import math

import numpy as np
from scipy.linalg import hadamard
from scipy.special import erf


def block_size(d: int) -> int:
    b = 1
    while b * 2 <= min(d, 128):
        b *= 2
    return b


def blocks(d: int):
    b = block_size(d)
    out = [(k * b, (k + 1) * b) for k in range(d // b)]
    if d % b:
        out.append((d - b, d))
    return out


def rotate(X, signs, perm):
    """float64 [n, d]: the sign flip, the permutation, then the cascaded
    orthonormal Hadamard blocks."""
    X = np.asarray(X, dtype=np.float64)
    n, d = X.shape
    Y = (X * np.asarray(signs, dtype=np.float64)[None, :])[:, np.asarray(perm)]
    b = block_size(d)
    H = hadamard(b).astype(np.float64) / math.sqrt(b)
    for a, z in blocks(d):
        Y[:, a:z] = Y[:, a:z] @ H.T
    return Y


def _phi(x):
    return np.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def _Phi(x):
    return 0.5 * (1.0 + erf(x / math.sqrt(2.0)))


def lloyd_max_gaussian(k: int = 16, iters: int = 100000, tol: float = 1e-15):
    """Levels (ascending, float64) of the k-level Lloyd-Max quantiser of N(0, 1):
    alternate boundaries = midpoints of neighbouring levels and levels =
    conditional means E[Z | cell] = (phi(a) - phi(b)) / (Phi(b) - Phi(a))."""
    L = np.linspace(-2.0, 2.0, k)
    for _ in range(iters):
        m = 0.5 * (L[:-1] + L[1:])
        a = np.concatenate([[-np.inf], m])
        b = np.concatenate([m, [np.inf]])
        pa = np.where(np.isinf(a), 0.0, _phi(np.where(np.isinf(a), 0.0, a)))
        pb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
        Lnew = (pa - pb) / (_Phi(b) - _Phi(a))
        if np.max(np.abs(Lnew - L)) < tol:
            L = Lnew
            break
        L = Lnew
    return L


def int8_levels(levels_f32):
    """(int8 levels rint(L * Lam), Lam = 127 / L[-1]) for float32 levels."""
    L = np.asarray(levels_f32, dtype=np.float32).astype(np.float64)
    lam = 127.0 / L[-1]
    return np.rint(L * lam).astype(np.int8), lam


def encode(Y, levels_f32):
    """Codes uint8 [n, ceil(d/2)] (low nibble = even dimension) and the rows'
    float32 steps gamma / Lam, from rotated rows Y (float32 [n, d])."""
    Y = np.asarray(Y, dtype=np.float32)
    n, d = Y.shape
    L = np.asarray(levels_f32, dtype=np.float32)
    mids = ((L[:-1].astype(np.float64) + L[1:].astype(np.float64)) / 2.0).astype(np.float32)
    _, lam = int8_levels(L)
    codes = np.zeros((n, (d + 1) // 2), dtype=np.uint8)
    step = np.zeros(n, dtype=np.float32)
    for i in range(n):
        y = Y[i]
        ss = float(np.sum(y.astype(np.float64) ** 2))
        f = np.float32(math.sqrt(d) / math.sqrt(ss)) if ss > 0 else np.float32(0.0)
        u = (y * f).astype(np.float32)
        c = np.array([int(np.sum(uj > mids)) for uj in u], dtype=np.uint8)
        lv = L[c].astype(np.float64)
        gamma = math.sqrt(ss) / math.sqrt(float(np.sum(lv * lv)))
        step[i] = np.float32(gamma / lam)
        for j in range(d):
            codes[i, j >> 1] |= np.uint8(c[j] << (4 * (j & 1)))
    return codes, step


def expand(codes, d, levels_i8):
    """int8 [n, d]: the int8 level of every dimension's code."""
    codes = np.asarray(codes, dtype=np.uint8)
    nib = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    return np.asarray(levels_i8, dtype=np.int8)[nib[:, :d]]
