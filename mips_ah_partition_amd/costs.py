"""Operation and byte counts of the search path, per query and per batch.

Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
Product Search", section "Worked example: cost of one query": raw bytes
n*d*4, blocks d/dpb of 4 bits each, partition L*d multiply-adds, table
B*16*dpb multiply-adds, scan (scanned rows)*B lookups, reorder R*d
multiply-adds.  The same counts give the algorithmic work the benchmark divides
by measured kernel times.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class QueryCost:
    raw_bytes: int
    blocks: int
    code_bytes_per_point: int
    code_bytes_total: int
    partition_macs: int
    lut_macs: int
    scanned_rows: float
    scan_lookups: float
    reorder_macs: int


def per_query(n: int, d: int, dpb: int, num_leaves: int = 0, leaves_to_search: int = 0,
              reorder: int = 100, elem_bytes: int = 4) -> QueryCost:
    B = d // dpb
    cbp = (B + 1) // 2
    scanned = n * leaves_to_search / num_leaves if num_leaves > 0 else float(n)
    return QueryCost(
        raw_bytes=n * d * elem_bytes,
        blocks=B,
        code_bytes_per_point=cbp,
        code_bytes_total=n * cbp,
        partition_macs=num_leaves * d if num_leaves > 0 else 0,
        lut_macs=B * 16 * dpb,
        scanned_rows=scanned,
        scan_lookups=scanned * B,
        reorder_macs=reorder * d,
    )


def scan_bytes(nq: int, B: int, scanned_rows_total: float, unique_rows: int) -> dict:
    """Algorithmic bytes of one scan launch: every code byte of the rows the
    batch touches read once, every query's int8 table read once, candidates
    (8 B) written by the final select counted separately."""
    cbp = (B + 1) // 2
    return {"codes": unique_rows * cbp, "tables": nq * B * 16, "lookups": scanned_rows_total * B}


def reorder_bytes(nq: int, R: int, d: int, elem_bytes: int) -> int:
    """Rows gathered by the exact reorder: R rows of d elements per query."""
    return nq * R * d * elem_bytes


def encode_flops_per_row(d: int, dpb: int, sweeps: int) -> int:
    """Float64 operations the coupled encoding needs per row: the squared norm
    (2 d); the nearest-center start (16 candidates x dpb x (subtract, square,
    add) per block); and per sweep and block the running parallel sum and the
    current center's term (each dpb x 6: r, (x * 1/|x|) r, r r and two adds)
    plus 16 candidates x (6 dpb + 4: par, ((eta - 1) par) par, + |r|^2)."""
    B = d // dpb
    init = B * 16 * 3 * dpb
    sweep = B * (6 * dpb + 6 * dpb + 16 * (6 * dpb + 4))
    return 2 * d + init + sweeps * sweep
