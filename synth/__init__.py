"""Seeded synthetic inputs for the asymmetric-hashing search path.

This module holds only random-number generation and storage-format conversion:
no scoring, quantization, selection or training arithmetic of the method lives
here.  Both the CPU oracle and the GPU path draw their inputs from these
functions, so that each sees exactly the same bytes.

Workloads (database shapes follow the datasets named on the RSLM summary page,
"Key experiments": bigann 128d, glove 100d 1M, openai 1536d 2M, wiki_pca 384d;
none of those datasets is used, the generators below stand in for them):

  tiny   n=10,000   d=128  N(0,1) rows, L2-normalised; no partition; 32 blocks x 4 dims
  sift1m n=1,000,000 d=128 integers uniform in [0,255] stored as fp32 (unnormalised
         MIPS); no partition; 64 blocks x 2 dims
  glove1m n=1,000,000 d=100 1,000-component Gaussian mixture, L2-normalised;
         1,000 leaves, 50 searched; 50 blocks x 2 dims
  openai2m n=2,000,000 d=1536 4,096-component mixture, unit norm, bf16 originals;
         2,000 leaves, 100 searched; 768 blocks x 2 dims
  wiki20m n=20,000,000 d=384 16,384-component mixture, unit norm, bf16 originals;
         4,000 leaves, 200 searched; 192 blocks x 2 dims

Seeds: numpy ``default_rng([1000*cfg_index + role, chunk])`` with role 0 = data,
1 = queries, 2 = partition sample/init, 3 = codebook init, 4 = mixture means.
Rows are generated in chunks of ``CHUNK`` so that any row range can be rebuilt
on its own (used for sampled checks at full size).
"""
from __future__ import annotations

import dataclasses
import numpy as np

CHUNK = 1 << 20  # rows per independently seeded chunk

ROLE_DATA, ROLE_QUERY, ROLE_PARTITION, ROLE_CODEBOOK, ROLE_MEANS = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1-based position in the workload list (seed base)
    n: int              # database rows
    d: int              # dimension
    nq: int             # queries per batch
    dpb: int            # dimensions per AH block
    num_leaves: int     # 0 = no partitioning (scan every row)
    leaves_to_search: int
    reorder: int        # R: candidates kept before exact reorder
    k: int              # final neighbours
    kind: str           # 'gauss_unit' | 'uint8_grid' | 'mixture_unit'
    components: int = 0
    sigma: float = 0.0
    originals: str = "f32"   # 'f32' or 'bf16'
    eta: float = 1.0         # anisotropic weight ratio used to train the codebooks

    @property
    def blocks(self) -> int:
        return self.d // self.dpb

    @property
    def code_bytes(self) -> int:
        return (self.blocks + 1) // 2


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, 10_000, 128, 100, 4, 0, 0, 100, 10, "gauss_unit", eta=1.0),
        Workload("sift1m", 2, 1_000_000, 128, 10_000, 2, 0, 0, 200, 10, "uint8_grid", eta=4.0),
        Workload("glove1m", 3, 1_000_000, 100, 10_000, 2, 1000, 50, 200, 10, "mixture_unit",
                 components=1000, sigma=0.3, eta=4.0),
        Workload("openai2m", 4, 2_000_000, 1536, 1_000, 2, 2000, 100, 400, 10, "mixture_unit",
                 components=4096, sigma=0.3, originals="bf16", eta=4.0),
        Workload("wiki20m", 5, 20_000_000, 384, 10_000, 2, 4000, 200, 300, 10, "mixture_unit",
                 components=16384, sigma=0.3, originals="bf16", eta=4.0),
    ]
}


def rng_for(w: Workload, role: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng([1000 * w.index + role, chunk])


def _unit_rows(x: np.ndarray) -> np.ndarray:
    nrm = np.sqrt(np.einsum("ij,ij->i", x, x, dtype=np.float64))
    nrm[nrm == 0] = 1.0
    return (x / nrm[:, None]).astype(np.float32)


def mixture_means(w: Workload) -> np.ndarray:
    return rng_for(w, ROLE_MEANS).standard_normal((w.components, w.d), dtype=np.float32)


def _rows(w: Workload, role: int, chunk: int, count: int, means) -> np.ndarray:
    rng = rng_for(w, role, chunk)
    if w.kind == "gauss_unit":
        return _unit_rows(rng.standard_normal((count, w.d), dtype=np.float32))
    if w.kind == "uint8_grid":
        return rng.integers(0, 256, size=(count, w.d)).astype(np.float32)
    if w.kind == "mixture_unit":
        comp = rng.integers(0, w.components, size=count)
        x = means[comp] + np.float32(w.sigma) * rng.standard_normal((count, w.d), dtype=np.float32)
        return _unit_rows(x)
    raise ValueError(w.kind)


def rows(w: Workload, start: int, stop: int, role: int = ROLE_DATA) -> np.ndarray:
    """fp32 rows [start, stop) of the database (role 0) or query set (role 1)."""
    total = w.n if role == ROLE_DATA else w.nq
    stop = min(stop, total)
    means = mixture_means(w) if w.kind == "mixture_unit" else None
    out = np.empty((max(stop - start, 0), w.d), dtype=np.float32)
    c0, c1 = start // CHUNK, (stop - 1) // CHUNK if stop > start else start // CHUNK - 1
    for c in range(c0, c1 + 1):
        lo, hi = c * CHUNK, min((c + 1) * CHUNK, total)
        blk = _rows(w, role, c, hi - lo, means)
        a, b = max(lo, start), min(hi, stop)
        out[a - start:b - start] = blk[a - lo:b - lo]
    return out


def database(w: Workload, n: int | None = None) -> np.ndarray:
    return rows(w, 0, w.n if n is None else n, ROLE_DATA)


def queries(w: Workload, nq: int | None = None) -> np.ndarray:
    return rows(w, 0, w.nq if nq is None else nq, ROLE_QUERY)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even) and return the raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# --- generic random inputs for stage tests (no method arithmetic) ------------------

def random_codes(rng: np.random.Generator, n: int, blocks: int) -> np.ndarray:
    """Row-major nibble-packed codes, uint8 [n][ceil(blocks/2)]; an odd final
    block leaves the high nibble of the last byte at zero."""
    nib = rng.integers(0, 16, size=(n, blocks + (blocks & 1)), dtype=np.uint8)
    if blocks & 1:
        nib[:, -1] = 0
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def random_lut_i8(rng: np.random.Generator, nq: int, blocks: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=(nq, blocks, 16)).astype(np.int8)


def random_leaf_sizes(rng: np.random.Generator, n: int, num_leaves: int, skew: float = 1.0) -> np.ndarray:
    """Leaf sizes summing to n with a lognormal spread (skew=0: equal sizes)."""
    if num_leaves <= 0:
        return np.zeros(0, dtype=np.int64)
    wts = rng.lognormal(0.0, skew, size=num_leaves) if skew > 0 else np.ones(num_leaves)
    sizes = np.floor(wts / wts.sum() * n).astype(np.int64)
    sizes[: n - sizes.sum()] += 1
    return sizes


def random_probe_lists(rng: np.random.Generator, nq: int, num_leaves: int, nl: int) -> np.ndarray:
    """Distinct leaf ids per query, int32 [nq][nl]."""
    out = np.empty((nq, nl), dtype=np.int32)
    for i in range(nq):
        out[i] = rng.choice(num_leaves, size=nl, replace=False)
    return out


def gpu_normal_rows(torch, n: int, d: int, seed: int, dtype, chunk_rows: int = 1 << 20):
    """n x d standard-normal rows generated on the GPU (seeded, in chunks of
    chunk_rows), stored as dtype."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = torch.empty((n, d), dtype=dtype, device="cuda")
    for a in range(0, n, chunk_rows):
        b = min(n, a + chunk_rows)
        out[a:b] = torch.randn((b - a, d), generator=g, device="cuda").to(dtype)
    return out


def gpu_database(torch, w: Workload, n: int | None = None, chunk_rows: int = CHUNK):
    """The workload's database rows generated on the GPU, stored as the
    workload's originals dtype (float32, or bfloat16 rounded to nearest even).
    Same laws as ``rows`` (mixture: component uniform, mean + sigma N(0, I),
    L2-normalised; gauss_unit: N(0, I) normalised; uint8_grid: integers in
    [0, 255]); the mixture means are the host ones (``mixture_means``), the
    per-row draws come from torch's GPU generator seeded per chunk with
    1000*index + role and the chunk number, so any chunk can be rebuilt alone."""
    n = w.n if n is None else n
    dt = torch.bfloat16 if w.originals == "bf16" else torch.float32
    out = torch.empty((n, w.d), dtype=dt, device="cuda")
    means = torch.from_numpy(mixture_means(w)).cuda() if w.kind == "mixture_unit" else None
    for c, a in enumerate(range(0, n, chunk_rows)):
        b = min(n, a + chunk_rows)
        g = torch.Generator(device="cuda")
        g.manual_seed((1000 * w.index + ROLE_DATA) * 1_000_003 + c)
        if w.kind == "uint8_grid":
            x = torch.randint(0, 256, (b - a, w.d), generator=g, device="cuda").to(torch.float32)
        else:
            x = torch.randn((b - a, w.d), generator=g, device="cuda", dtype=torch.float32)
            if w.kind == "mixture_unit":
                comp = torch.randint(0, w.components, (b - a,), generator=g, device="cuda")
                x = means[comp] + np.float32(w.sigma) * x
            nrm = torch.linalg.vector_norm(x.double(), dim=1, keepdim=True)
            nrm[nrm == 0] = 1.0
            x = (x.double() / nrm).to(torch.float32)
        out[a:b] = x.to(dt)
    return out


def rotation_draws(d: int, seed: int):
    """The random draws of the training-free rotation: signs float32 [d] (+-1)
    and a permutation int32 [d]."""
    rng = np.random.default_rng([7000, seed])
    signs = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=d)
    perm = rng.permutation(d).astype(np.int32)
    return signs, perm
