"""Training-free rotation quantiser on the GPU: the levels table and the search.

Page "RSLM: Training-Free Vector Quantization for Approximate Nearest Neighbor
Search", method points: block Hadamard rotation (block 128, sign flips and a
permutation), a fixed 16-level Lloyd-Max codebook for the rotated coordinates,
and a per-row scale restoring the reconstruction's norm.  The rotation,
encoding and scan are the C-ABI calls ah_rslm_rotate / ah_rslm_encode /
ah_rslm_scan_topk; this module computes the fixed levels once on the host and
strings the calls together.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import ahlib


def _gauss_cell_mean(a: float, b: float) -> float:
    """E[Z | a < Z < b] for Z ~ N(0, 1)."""
    pdf = lambda z: 0.0 if math.isinf(z) else math.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)  # noqa: E731
    cdf = lambda z: 0.5 * (1.0 + math.erf(z / math.sqrt(2.0))) if not math.isinf(z) else (1.0 if z > 0 else 0.0)  # noqa: E731
    return (pdf(a) - pdf(b)) / (cdf(b) - cdf(a))


def gaussian_levels(k: int = 16, tol: float = 1e-14) -> np.ndarray:
    """The k-level Lloyd-Max quantiser of N(0, 1) (ascending), by Lloyd's
    alternation of cell means and midpoints, as float32."""
    lv = [-2.0 + 4.0 * i / (k - 1) for i in range(k)]
    for _ in range(200000):
        mids = [(lv[i] + lv[i + 1]) / 2.0 for i in range(k - 1)]
        edges = [-math.inf] + mids + [math.inf]
        new = [_gauss_cell_mean(edges[i], edges[i + 1]) for i in range(k)]
        done = max(abs(x - y) for x, y in zip(new, lv)) < tol
        lv = new
        if done:
            break
    return np.array(lv, dtype=np.float32)


def int8_levels(levels: np.ndarray) -> np.ndarray:
    """rint(L * 127 / L[15]) as int8: the levels the int8 matrix-core scan reads."""
    L = np.asarray(levels, dtype=np.float32).astype(np.float64)
    return np.rint(L * (127.0 / L[-1])).astype(np.int8)


class RSLMIndex:
    """4-bit codes of rotated rows on the GPU, searched by the int8 flat scan."""

    def __init__(self, X: torch.Tensor, signs: np.ndarray, perm: np.ndarray, levels: np.ndarray | None = None,
                 pct: float = 99.9):
        dev = X.device
        self.d = X.shape[1]
        self.signs = torch.from_numpy(np.ascontiguousarray(signs, dtype=np.float32)).to(dev)
        self.perm = torch.from_numpy(np.ascontiguousarray(perm, dtype=np.int32)).to(dev)
        self.levels = gaussian_levels() if levels is None else np.asarray(levels, dtype=np.float32)
        self.levels_i8 = int8_levels(self.levels)
        self.pct = pct
        Y = ahlib.ah_rslm_rotate(X, self.signs, self.perm)
        self.codes, self.step = ahlib.ah_rslm_encode(Y, self.levels)
        del Y
        self._ws = None

    def search(self, Q: torch.Tensor, R: int, base: torch.Tensor | None = None, k: int = 10):
        """Top-R candidates by the 4-bit approximate score; with base (the
        original rows), their exact rescore to the best k."""
        Qr = ahlib.ah_rslm_rotate(Q, self.signs, self.perm)
        q8, qs = ahlib.ah_sq8_quantize(Qr, self.pct)
        need = ahlib.ah_sq8_workspace_bytes(Q.shape[0], self.codes.shape[0], self.d, R)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
        cand, sc = ahlib.ah_rslm_scan_topk(q8, qs, self.codes, self.step, self.d, self.levels_i8, R,
                                           workspace=self._ws)
        if base is None:
            return cand, sc
        return ahlib.ah_reorder_exact(Q, base, cand, k)
