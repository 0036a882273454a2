"""AHIndex: a device-resident index and the batched search over the C ABI.

Mirrors the search interface of the page "ScaNN: Anisotropic Vector
Quantization for Maximum Inner Product Search", section "Using the library":
search_batched(Q, leaves_to_search=..., pre_reorder_num_neighbors=...,
final_num_neighbors=...) returning (neighbors, scores).  Each call runs the
path's four steps through include/ah.h; this class only owns device memory
(torch tensors) and the workspaces, reused across calls of the same shape.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ahlib
from .index import HostIndex


class AHIndex:
    def __init__(self, host: HostIndex, base: np.ndarray, num_leaves_to_search: int = 0, reorder: int = 100,
                 final_num_neighbors: int = 10, device: str = "cuda", base_is_bf16_bits: bool = False):
        dev = torch.device(device)
        self.device = dev
        self.codebooks = torch.from_numpy(np.ascontiguousarray(host.codebooks)).to(dev)
        self.codes = torch.from_numpy(np.ascontiguousarray(host.codes)).to(dev)
        self.ids = None if host.ids is None else torch.from_numpy(np.ascontiguousarray(host.ids)).to(dev)
        self.centroids = None if host.centroids is None else torch.from_numpy(
            np.ascontiguousarray(host.centroids)).to(dev)
        self.leaf_offsets = None if host.leaf_offsets is None else torch.from_numpy(
            np.ascontiguousarray(host.leaf_offsets)).to(dev)
        if base_is_bf16_bits:
            self.base = torch.from_numpy(np.ascontiguousarray(base).view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            self.base = torch.from_numpy(np.ascontiguousarray(base, dtype=np.float32)).to(dev)
        # residual (leaf-relative) codes: the leaves' scores enter the scan as
        # per-leaf terms in table units (ah_residual_leaf_bias), clipped to
        # +-2 * 255 * B (rows whose leaf lies further below the best one cannot
        # outrank any row of the best leaf)
        self.residual = bool(getattr(host, "residual", False)) and self.centroids is not None
        self.bias_bound = min(2 * 255 * int(host.codebooks.shape[0]), 1 << 24)
        self.num_leaves_to_search = num_leaves_to_search
        self.reorder = reorder
        self.final_num_neighbors = final_num_neighbors
        self._ws = {}

    @classmethod
    def from_device(cls, dix, base, num_leaves_to_search: int = 0, reorder: int = 100,
                    final_num_neighbors: int = 10):
        """An index whose arrays are already on the GPU (index.DeviceIndex) and
        base rows as a float32 or bfloat16 device tensor [n, d]."""
        self = cls.__new__(cls)
        self.device = base.device
        self.codebooks, self.codes, self.ids = dix.codebooks, dix.codes, dix.ids
        self.centroids, self.leaf_offsets = dix.centroids, dix.leaf_offsets
        self.base = base
        self.residual = bool(dix.residual) and self.centroids is not None
        self.bias_bound = min(2 * 255 * int(dix.codebooks.shape[0]), 1 << 24)
        self.num_leaves_to_search = num_leaves_to_search
        self.reorder = reorder
        self.final_num_neighbors = final_num_neighbors
        self._ws = {}
        return self

    @property
    def partitioned(self) -> bool:
        return self.centroids is not None and self.num_leaves_to_search > 0

    def _workspace(self, key, nbytes):
        t = self._ws.get(key)
        if t is None or t.numel() < nbytes:
            t = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
            self._ws[key] = t
        return t

    def search_batched(self, Q, leaves_to_search=None, pre_reorder_num_neighbors=None, final_num_neighbors=None,
                       stream=None, timers=None):
        """Q: float32 device tensor [nq, d].  Returns (ids int32 [nq, k], scores float32 [nq, k]).
        timers: optional dict stage -> (start, stop) callables recording events."""
        nl = self.num_leaves_to_search if leaves_to_search is None else leaves_to_search
        R = self.reorder if pre_reorder_num_neighbors is None else pre_reorder_num_neighbors
        k = self.final_num_neighbors if final_num_neighbors is None else final_num_neighbors
        nq = Q.shape[0]
        B = self.codebooks.shape[0]
        t = timers or {}
        leaves = None
        if self.centroids is not None and nl > 0:
            L = self.centroids.shape[0]
            ws = self._workspace("part", ahlib.ah_partition_workspace_bytes(nq, L))
            if "partition" in t:
                t["partition"][0]()
            leaves, leaf_scores = ahlib.ah_partition_score(Q, self.centroids, nl, workspace=ws, stream=stream)
            if "partition" in t:
                t["partition"][1]()
        if "lut" in t:
            t["lut"][0]()
        lut, scale, bias, _ = ahlib.ah_build_lut(Q, self.codebooks, stream=stream)
        if "lut" in t:
            t["lut"][1]()
        Lw = 0 if leaves is None else self.centroids.shape[0]
        nlw = 0 if leaves is None else nl
        ws = self._workspace("scan", ahlib.ah_scan_workspace_bytes(nq, B, self.codes.shape[0], Lw, nlw, R))
        if "scan" in t:
            t["scan"][0]()
        if self.residual and leaves is not None:
            lb = ahlib.ah_residual_leaf_bias(leaf_scores, scale, self.bias_bound, stream=stream)
            cand, _ = ahlib.ah_scan_topk(lut, self.codes, R, ids=self.ids, leaf_offsets=self.leaf_offsets,
                                         leaves=leaves, workspace=ws, stream=stream, leaf_bias=lb,
                                         bias_bound=self.bias_bound)
        else:
            cand, _ = ahlib.ah_scan_topk(lut, self.codes, R, ids=self.ids,
                                         leaf_offsets=self.leaf_offsets if leaves is not None else None,
                                         leaves=leaves, workspace=ws, stream=stream,
                                         main_events=t.get("scan_main"))
        if "scan" in t:
            t["scan"][1]()
        if "reorder" in t:
            t["reorder"][0]()
        out = ahlib.ah_reorder_exact(Q, self.base, cand, k, stream=stream)
        if "reorder" in t:
            t["reorder"][1]()
        return out
