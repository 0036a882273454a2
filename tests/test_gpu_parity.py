"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Stage-chained: every GPU stage is compared with the oracle run on the same
inputs that stage received.  Integer results (int8 tables, scan sums, top-R id
sets) must match bit for bit; floating-point results (fp32 tables, centroid
scores, reorder scores) within 1e-4 relative, relative to
max(|ref|, sum_j |a_j b_j|) with the float64 oracle as reference.  Where two
items' float64 scores lie within that tolerance, either order is accepted.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mips_ah_partition_amd import ahlib
    ahlib.lib()
    return torch, ahlib


def _t(torch, a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def _np(t):
    return t.cpu().numpy()


# ----------------------------------------------------------------------------- LUT
@pytest.mark.parametrize("dpb,B,nq", [(1, 5, 3), (2, 64, 37), (4, 32, 100), (2, 200, 17), (2, 768, 5), (3, 7, 66),
                                      (1, 1, 2), (16, 300, 4), (2, 513, 9), (2, 4096, 3)])
def test_build_lut_parity(gpu, dpb, B, nq):
    torch, ah = gpu
    rng = np.random.default_rng(1000 + B * 10 + dpb)
    Q = rng.standard_normal((nq, B * dpb)).astype(np.float32)
    cb = rng.standard_normal((B, 16, dpb)).astype(np.float32)
    t8, s, beta, l32 = ah.ah_build_lut(_t(torch, Q), _t(torch, cb), want_f32=True)
    torch.cuda.synchronize()
    l32 = _np(l32)
    ref = oracle.lut_f64(Q, cb)
    denom = np.maximum(np.abs(ref), np.einsum("qbt,bct->qbc", np.abs(Q.reshape(nq, B, dpb)).astype(np.float64),
                                               np.abs(cb).astype(np.float64)))
    assert (np.abs(l32 - ref) <= TOL * denom + 1e-30).all()
    # the table is the float32 rounding of the float64 sum (include/ah.h), so it
    # equals the oracle's table rounded to float32 bit for bit, and the int8 table
    # follows from the oracle's own float32 table without chaining
    assert np.array_equal(l32, ref.astype(np.float32))
    o8, os_, ob = oracle.quantize_lut(ref.astype(np.float32))
    assert np.array_equal(_np(t8), o8)
    assert np.array_equal(_np(s), os_)
    assert np.array_equal(_np(beta), ob)


def test_build_lut_unaligned_outputs(gpu):
    """Output tables and inputs at odd offsets (element-wise stores and loads) equal the aligned results."""
    torch, ah = gpu
    rng = np.random.default_rng(33)
    nq, B, dpb = 6, 70, 2
    Q = _t(torch, rng.standard_normal((nq, B * dpb)).astype(np.float32))
    cb = _t(torch, rng.standard_normal((B, 16, dpb)).astype(np.float32))
    t8, s, beta, l32 = ah.ah_build_lut(Q, cb, want_f32=True)
    raw8 = torch.zeros(nq * B * 16 + 1, dtype=torch.int8, device=Q.device)
    raw32 = torch.zeros(nq * B * 16 + 1, dtype=torch.float32, device=Q.device)
    u8 = raw8[1:].view(nq, B, 16)
    u32 = raw32[1:].view(nq, B, 16)
    ah.ah_build_lut(Q, cb, lut_i8_out=u8, lut_f32_out=u32, want_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(u8, t8) and torch.equal(u32, l32)
    # inputs at odd offsets too (element-wise loads)
    rawq = torch.zeros(Q.numel() + 1, dtype=torch.float32, device=Q.device)
    rawc = torch.zeros(cb.numel() + 1, dtype=torch.float32, device=Q.device)
    uq = rawq[1:].view(Q.shape)
    uc = rawc[1:].view(cb.shape)
    uq.copy_(Q)
    uc.copy_(cb)
    v8, vs, vb, v32 = ah.ah_build_lut(uq, uc, want_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(v8, t8) and torch.equal(v32, l32) and torch.equal(vs, s) and torch.equal(vb, beta)


def test_build_lut_constant_table(gpu):
    torch, ah = gpu
    Q = np.zeros((4, 8), dtype=np.float32)
    cb = np.random.default_rng(2).standard_normal((4, 16, 2)).astype(np.float32)
    t8, s, beta, _ = ah.ah_build_lut(_t(torch, Q), _t(torch, cb))
    torch.cuda.synchronize()
    assert (_np(t8) == 0).all() and (_np(s) == 0).all() and (_np(beta) == 0).all()


# ----------------------------------------------------------------------------- scan
def _scan_check(torch, ah, lut, codes, R, ids=None, offs=None, leaves=None):
    g_ids, g_sc = ah.ah_scan_topk(_t(torch, lut), _t(torch, codes), R,
                                  ids=None if ids is None else _t(torch, ids),
                                  leaf_offsets=None if offs is None else _t(torch, offs),
                                  leaves=None if leaves is None else _t(torch, leaves))
    torch.cuda.synchronize()
    o_ids, o_sc = oracle.scan_topk(lut, codes, R, ids=ids, leaf_offsets=offs, leaves=leaves)
    g_ids, g_sc = _np(g_ids), _np(g_sc)
    bad = np.nonzero((g_ids != o_ids).any(axis=1) | (g_sc != o_sc).any(axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} queries differ, first {bad[:5]}: gpu {g_ids[bad[0], :8]} {g_sc[bad[0], :8]} oracle {o_ids[bad[0], :8]} {o_sc[bad[0], :8]}"
    return g_ids, g_sc


@pytest.mark.parametrize("B,n,nq,R,stride_pad", [
    (32, 10000, 100, 100, 0),   # tiny workload shape: 32 blocks, 16 B rows
    (64, 5000, 70, 200, 0),     # 64 blocks, ragged query group
    (50, 3001, 65, 37, 0),      # 25 B rows (unaligned path), ragged rows
    (8, 700, 9, 1000, 0),       # R > n: pads
    (200, 2000, 20, 300, 0),    # several 64-block chunks
    (768, 1500, 8, 400, 0),     # 768 blocks
    (33, 1234, 5, 10, 7),       # odd B, padded rows
    (16, 20000, 10, 1500, 0),   # R > 1024: the workgroup final selection
    (300, 3000, 6, 40, 0),      # 300 blocks: the workgroup warm-up
    (64, 12000, 70, 4096, 0),   # R at its maximum (AH_MAX_R)
])
def test_scan_full_parity(gpu, B, n, nq, R, stride_pad):
    torch, ah = gpu
    rng = np.random.default_rng(B * 7 + n)
    lut = synth.random_lut_i8(rng, nq, B)
    codes = synth.random_codes(rng, n, B)
    if stride_pad:
        codes = np.concatenate([codes, rng.integers(0, 256, size=(n, stride_pad), dtype=np.uint8)], axis=1)
    _scan_check(torch, ah, lut, codes, R)



def test_zero_rows_every_row_entry(gpu):
    """An empty set of rows is valid at every row-side call: assignment, the
    k-means update (counts 0, centroids kept, as for empty leaves), coupled
    encoding and sweeps, the codebook update (codebooks kept), the rotation
    quantiser, tiling and int8 quantisation."""
    torch, ah = gpu
    rng = np.random.default_rng(10)
    d, B, dpb, L = 16, 8, 2, 5
    X0 = torch.empty((0, d), dtype=torch.float32, device="cuda")
    C = rng.standard_normal((L, d)).astype(np.float32)
    cb = rng.standard_normal((B, 16, dpb)).astype(np.float32)
    leaf, _ = ah.ah_assign_leaves(X0, _t(torch, C))
    cent, counts = ah.ah_kmeans_update(X0, torch.empty(0, dtype=torch.int32, device="cuda"), _t(torch, C))
    codes = ah.ah_encode(X0, _t(torch, cb), 4.0)
    ah.ah_encode_sweep(X0, _t(torch, cb), 4.0, codes)
    cbt = _t(torch, cb)
    ah.ah_pq_update(X0, codes, cbt, 4.0)
    signs, perm = synth.rotation_draws(d, 2)
    y = ah.ah_rslm_rotate(X0, _t(torch, signs), _t(torch, perm))
    from mips_ah_partition_amd import rslm
    rc, rs = ah.ah_rslm_encode(y, rslm.gaussian_levels())
    tc = ah.ah_tile_codes(codes, B)
    c8, s8 = ah.ah_sq8_quantize(X0)
    torch.cuda.synchronize()
    assert tuple(leaf.shape) == (0,) and tuple(codes.shape) == (0, B // 2) and tuple(rc.shape) == (0, d // 2)
    assert tuple(rs.shape) == (0,) and tc.n == 0 and tuple(c8.shape) == (0, d) and tuple(s8.shape) == (0,)
    assert (_np(counts) == 0).all() and np.array_equal(_np(cent), C)
    assert np.array_equal(_np(cbt), cb)

@pytest.mark.parametrize("seed", range(3))
def test_scan_heavy_ties(gpu, seed):
    torch, ah = gpu
    rng = np.random.default_rng(50 + seed)
    B, n, nq, R = 16, 6000, 40, 150
    lut = rng.choice(np.array([-1, 1], dtype=np.int8), size=(nq, B, 16))
    codes = synth.random_codes(rng, n, B)
    _scan_check(torch, ah, lut, codes, R)


def test_scan_empty_database(gpu):
    torch, ah = gpu
    lut = np.ones((3, 4, 16), dtype=np.int8)
    codes = np.zeros((0, 2), dtype=np.uint8)
    ids, sc = ah.ah_scan_topk(_t(torch, lut), _t(torch, codes), 5)
    torch.cuda.synchronize()
    assert (_np(ids) == -1).all() and (_np(sc) == np.iinfo(np.int32).min).all()


def test_zero_queries_every_query_entry(gpu):
    """An empty query batch is valid at every query-side call (partition, tables,
    plain and partitioned and residual scans, reorder, int8 flat search, rotation
    quantiser): each returns empty outputs without an error."""
    torch, ah = gpu
    rng = np.random.default_rng(9)
    d, B, dpb, L, nl, n, R, k = 16, 8, 2, 6, 3, 60, 10, 4
    Q0 = torch.empty((0, d), dtype=torch.float32, device="cuda")
    X = rng.standard_normal((n, d)).astype(np.float32)
    leaves, lsc = ah.ah_partition_score(Q0, _t(torch, rng.standard_normal((L, d)).astype(np.float32)), nl)
    t8, step, _, _ = ah.ah_build_lut(Q0, _t(torch, rng.standard_normal((B, 16, dpb)).astype(np.float32)))
    codes = _t(torch, synth.random_codes(rng, n, B))
    offs = _t(torch, np.array([0, 10, 10, 25, 40, 55, 60], dtype=np.int64))
    ids, sc = ah.ah_scan_topk(t8, codes, R)
    pids, psc = ah.ah_scan_topk(t8, codes, R, leaf_offsets=offs, leaves=leaves)
    bias = ah.ah_residual_leaf_bias(lsc, step, 1000)
    rids, rsc = ah.ah_scan_topk(t8, codes, R, leaf_offsets=offs, leaves=leaves, leaf_bias=bias, bias_bound=1000)
    fid, fsc = ah.ah_reorder_exact(Q0, _t(torch, X), ids, k)
    q8, qs = ah.ah_sq8_quantize(Q0)
    d8, dsc = ah.ah_sq8_quantize(_t(torch, X))
    sid, ssc = ah.ah_sq8_scan_topk(q8, qs, d8, dsc, R)
    signs, perm = synth.rotation_draws(d, 1)
    y0 = ah.ah_rslm_rotate(Q0, _t(torch, signs), _t(torch, perm))
    torch.cuda.synchronize()
    for t, shape in ((leaves, (0, nl)), (lsc, (0, nl)), (t8, (0, B, 16)), (step, (0,)), (ids, (0, R)), (sc, (0, R)),
                     (pids, (0, R)), (bias, (0, nl)), (rids, (0, R)), (rsc, (0, R)), (fid, (0, k)), (fsc, (0, k)),
                     (q8, (0, d)), (sid, (0, R)), (ssc, (0, R)), (y0, (0, d))):
        assert tuple(t.shape) == shape


def test_scan_partitioned_parity(gpu):
    torch, ah = gpu
    rng = np.random.default_rng(77)
    B, n, nq, L, nl, R = 64, 30000, 150, 40, 6, 120
    sizes = np.concatenate([[20000], synth.random_leaf_sizes(rng, n - 20000, L - 1, skew=1.0)])
    sizes[6] += sizes[5]
    sizes[5] = 0  # an empty leaf; leaf 0 spans several 8192-row items
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    lut = synth.random_lut_i8(rng, nq, B)
    codes = synth.random_codes(rng, n, B)
    perm = rng.permutation(n).astype(np.int32)
    leaves = synth.random_probe_lists(rng, nq, L, nl)
    leaves[:, 0] = 0
    leaves[1, 1] = 5
    _scan_check(torch, ah, lut, codes, R, ids=perm, offs=offs, leaves=leaves)


@pytest.mark.parametrize("B,nq,stride_pad", [(768, 20, 0), (300, 9, 0), (200, 7, 12), (1001, 6, 11)])
def test_scan_partitioned_large_tables(gpu, B, nq, stride_pad):
    """Partitioned batches with tables past the one-wave warm-up's size: the
    workgroup warm-up sums rows of whole 16-byte segments a batch of segments at
    a time (384 B rows; 112 B rows whose 12 padding bytes hold random nibbles
    that must add nothing) or word by word (150 B and 512 B rows, unaligned)."""
    torch, ah = gpu
    rng = np.random.default_rng(500 + B + nq)
    n, L, nl, R = 6000, 12, 4, 100
    sizes = synth.random_leaf_sizes(rng, n, L, skew=1.0)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    lut = synth.random_lut_i8(rng, nq, B)
    codes = synth.random_codes(rng, n, B)
    if stride_pad:
        codes = np.concatenate([codes, rng.integers(0, 256, size=(n, stride_pad), dtype=np.uint8)], axis=1)
    leaves = synth.random_probe_lists(rng, nq, L, nl)
    _scan_check(torch, ah, lut, codes, R, offs=offs, leaves=leaves)


# Small batches (at most four queries) on rows aligned to 16 bytes take the
# streaming kernel: byte-pair tables for one or two queries per item, nibble
# tables (one query, or four packed) when pair tables would not fit.  Cases
# cover segment folds past 256 blocks, partial last segments, R > n, a 64 KB
# table and every row-length class (2, 6, 8 segments, longer).
@pytest.mark.parametrize("B,n,nq,R,stride_pad", [
    (32, 10000, 1, 100, 0),
    (64, 50000, 4, 200, 0),
    (50, 3001, 2, 37, 7),       # 25 code bytes in 32 B rows
    (50, 3001, 2, 37, 0),       # 25 B rows: unaligned, so the MFMA kernel
    (8, 700, 3, 1000, 0),       # R > n
    (200, 20000, 1, 300, 0),    # 100 B rows: partial last segment
    (300, 4000, 4, 50, 0),      # 300 blocks: packed fields folded mid-row
    (768, 5000, 4, 400, 0),     # 48 KB packed table
    (33, 1234, 1, 10, 15),      # odd B, 32 B stride
    (1, 999, 4, 5, 0),          # one block
    (4096, 600, 1, 20, 0),      # 64 KB single-query table
    (192, 20000, 1, 300, 0),    # 96 B rows: coalesced tiles of 32 rows in 3 load rounds
    (192, 20001, 4, 300, 0),    # the same, two query pairs
    (768, 6000, 1, 400, 0),     # 384 B rows: tiles of 8 rows, nibble table
    (768, 6000, 3, 400, 0),     # the same, packed nibble table
    (96, 7000, 2, 64, 0),       # 48 B rows: tiles of 64 rows in 3 rounds
    (192, 3001, 3, 37, 32),     # 96 B of codes in 128 B rows: whole-row registers
    (500, 4000, 1, 100, 6),     # one query, nibble table, partial last segment
    (1001, 3000, 1, 64, 11),    # odd B in 512 B rows
    (1536, 2000, 1, 50, 0),     # 768 B rows
    (64, 9000, 3, 4096, 0),     # R at its maximum (AH_MAX_R)
    (192, 300000, 1, 300, 0),   # warm-up sample spread over a longer array (every 2nd or 3rd row)
    (768, 140000, 2, 400, 0),   # the same, packed pair table
])
def test_scan_stream_parity(gpu, B, n, nq, R, stride_pad):
    torch, ah = gpu
    rng = np.random.default_rng(B * 13 + n + nq)
    lut = synth.random_lut_i8(rng, nq, B)
    codes = synth.random_codes(rng, n, B)
    if stride_pad:
        codes = np.concatenate([codes, rng.integers(0, 256, size=(n, stride_pad), dtype=np.uint8)], axis=1)
    _scan_check(torch, ah, lut, codes, R)


@pytest.mark.parametrize("nq,B", [(1, 96), (2, 128), (4, 256), (70, 256), (1, 768)])
def test_scan_extreme_tables(gpu, nq, B):
    """Entries of -128 and 127 only (streaming: packed fields at both ends of
    their range; one query: byte-pair table, two: packed pair table, four:
    packed nibble table, 70: MFMA); where present, one query all 127 and one
    all -128 (every sum -128 B, the lowest possible: a threshold must never be
    raised past it)."""
    torch, ah = gpu
    rng = np.random.default_rng(91 + nq)
    n, R = 3000, 64
    lut = rng.choice(np.array([-128, 127], dtype=np.int8), size=(nq, B, 16))
    if nq > 1:
        lut[-1] = -128
    if nq > 2:
        lut[1] = 127
    codes = synth.random_codes(rng, n, B)
    _scan_check(torch, ah, lut, codes, R)


@pytest.mark.parametrize("nq,B,L,nl", [(1, 48, 25, 5), (3, 48, 25, 5), (4, 48, 3, 2), (3, 400, 4, 3),
                                       (1, 192, 25, 5), (2, 192, 7, 3), (4, 64, 3, 2), (3, 768, 5, 2)])
def test_scan_stream_partitioned(gpu, nq, B, L, nl):
    """Few queries over leaves; with few leaves several queries share one, so a
    leaf has more than one query group (two per item with pair tables).  Rows of
    24 and 200 code bytes are not 16-byte multiples (MFMA kernel); 32, 96 and
    384 take the streaming kernel's coalesced tiles, starting at any row."""
    torch, ah = gpu
    rng = np.random.default_rng(300 + nq + B + L)
    n, R = 40000, 90
    sizes = synth.random_leaf_sizes(rng, n, L, skew=1.0)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    lut = synth.random_lut_i8(rng, nq, B)
    codes = synth.random_codes(rng, n, B)
    perm = rng.permutation(n).astype(np.int32)
    leaves = synth.random_probe_lists(rng, nq, L, nl)
    _scan_check(torch, ah, lut, codes, R, ids=perm, offs=offs, leaves=leaves)


def _tiled_reference(codes, B):
    """The tiled layout written out from its definition in ah.h (byte k of row r
    at (r // 64) * 64 * S * 16 + (k // 16) * 1024 + (r % 64) * 16 + k % 16)."""
    n = codes.shape[0]
    cb = (B + 1) // 2
    S = (cb + 15) // 16
    out = np.zeros(((n + 63) // 64) * 64 * S * 16, dtype=np.uint8)
    for r in range(n):
        for k in range(cb):
            out[(r // 64) * 64 * S * 16 + (k // 16) * 1024 + (r % 64) * 16 + k % 16] = codes[r, k]
    return out


@pytest.mark.parametrize("B,n,pad", [(64, 130, 0), (192, 64, 0), (50, 200, 7), (1, 5, 0), (600, 70, 3)])
def test_tile_codes_layout(gpu, B, n, pad):
    torch, ah = gpu
    rng = np.random.default_rng(B + n)
    codes = synth.random_codes(rng, n, B)
    if pad:
        codes = np.concatenate([codes, rng.integers(0, 256, size=(n, pad), dtype=np.uint8)], axis=1)
    tc = ah.ah_tile_codes(_t(torch, codes), B)
    torch.cuda.synchronize()
    assert tc.data.numel() == ah.ah_tiled_codes_bytes(n, B)
    assert np.array_equal(_np(tc.data), _tiled_reference(codes, B))


# The tiled layout through every kernel that reads codes: streaming (1-4
# queries), MFMA (more), warm-up (wave and workgroup), final selection and the
# exact fallback, full and partitioned scans (leaves start at any row, so a
# wave's rows may span two tiles).
@pytest.mark.parametrize("nq,B,n,R,parts", [
    (1, 192, 20000, 300, 0), (4, 192, 9000, 100, 0), (2, 64, 5001, 64, 0), (3, 768, 3000, 200, 0),
    (70, 64, 5000, 200, 0), (20, 200, 2000, 300, 0), (9, 300, 3000, 40, 0),
    (1, 192, 40000, 90, 25), (4, 64, 40000, 90, 3), (65, 96, 40000, 90, 30),
    (1, 768, 20000, 200, 0), (1, 768, 30000, 90, 12),  # one query with a nibble table, full and partitioned
])
def test_scan_tiled_parity(gpu, nq, B, n, R, parts):
    torch, ah = gpu
    rng = np.random.default_rng(7 * nq + B + n + parts)
    lut = synth.random_lut_i8(rng, nq, B)
    codes = synth.random_codes(rng, n, B)
    tc = ah.ah_tile_codes(_t(torch, codes), B)
    ids = offs = leaves = None
    kw = {}
    if parts:
        sizes = synth.random_leaf_sizes(rng, n, parts, skew=1.0)
        offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
        ids = rng.permutation(n).astype(np.int32)
        leaves = synth.random_probe_lists(rng, nq, parts, max(1, parts // 5))
        kw = dict(ids=_t(torch, ids), leaf_offsets=_t(torch, offs), leaves=_t(torch, leaves))
    g_ids, g_sc = ah.ah_scan_topk(_t(torch, lut), tc, R, **kw)
    torch.cuda.synchronize()
    o_ids, o_sc = oracle.scan_topk(lut, codes, R, ids=ids, leaf_offsets=offs, leaves=leaves)
    assert np.array_equal(_np(g_ids), o_ids) and np.array_equal(_np(g_sc), o_sc)


def test_scan_tiled_overflow_fallback(gpu):
    """Equal sums on tiled codes: lists overflow, the exact fallback reads the tiles."""
    torch, ah = gpu
    B, n, nq, R = 64, 40000, 6, 50
    lut = np.zeros((nq, B, 16), dtype=np.int8)
    codes = synth.random_codes(np.random.default_rng(3), n, B)
    tc = ah.ah_tile_codes(_t(torch, codes), B)
    g_ids, g_sc = ah.ah_scan_topk(_t(torch, lut), tc, R)
    torch.cuda.synchronize()
    o_ids, o_sc = oracle.scan_topk(lut, codes, R)
    assert np.array_equal(_np(g_ids), o_ids) and np.array_equal(_np(g_sc), o_sc)


def test_scan_overflow_fallback(gpu):
    """All sums equal: the threshold cannot rise, candidate lists overflow and the
    exact fallback must return the R lowest ids."""
    torch, ah = gpu
    B, n, nq, R = 4, 40000, 3, 50
    lut = np.zeros((nq, B, 16), dtype=np.int8)
    codes = synth.random_codes(np.random.default_rng(1), n, B)
    ids, sc = _scan_check(torch, ah, lut, codes, R)
    assert (ids == np.arange(R)).all() and (sc == 0).all()


def test_scan_deterministic(gpu):
    torch, ah = gpu
    rng = np.random.default_rng(5)
    lut = synth.random_lut_i8(rng, 64, 32, -3, 3)
    codes = synth.random_codes(rng, 20000, 32)
    a = [_np(x) for x in ah.ah_scan_topk(_t(torch, lut), _t(torch, codes), 64)]
    b = [_np(x) for x in ah.ah_scan_topk(_t(torch, lut), _t(torch, codes), 64)]
    torch.cuda.synchronize()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------------------- reorder
def _check_ranked(g_ids, g_sc, o_ids, o_sc, ref_fn, denom_fn):
    """GPU picks a valid best-k up to near-ties: its float64 scores match the
    oracle's ranked scores within tolerance, and its own scores are accurate."""
    for q in range(g_ids.shape[0]):
        valid = o_ids[q] >= 0
        assert ((g_ids[q] >= 0) == valid).all()
        gi = g_ids[q][valid]
        ref = ref_fn(q, gi)
        den = np.maximum(np.abs(ref), denom_fn(q, gi))
        assert (np.abs(g_sc[q][valid] - ref) <= TOL * den).all(), q
        assert (np.abs(ref - o_sc[q][valid]) <= 2 * TOL * den).all(), q
        assert len(set(gi.tolist())) == len(gi)


# Row lengths cover one, two and four 16-byte chunks per lane (two on a 32-lane
# group for bf16 rows of 33-63 chunks: 264, 384 and 504 dims), rows longer than
# 4 x 64 chunks (several passes; 12,288 dims: a dozen), and rows not in whole
# chunks (element path).
@pytest.mark.parametrize("dtype,d,R,k", [("f32", 128, 200, 10), ("f32", 100, 37, 37), ("bf16", 384, 300, 10),
                                         ("bf16", 1536, 64, 10), ("f32", 7, 10, 3), ("f32", 512, 50, 5),
                                         ("bf16", 4096, 40, 8), ("f32", 2048, 30, 30), ("f32", 32, 4096, 4096),
                                         ("f32", 12288, 64, 10), ("bf16", 12288, 32, 8), ("f32", 12289, 16, 4),
                                         ("f32", 64, 512, 64), ("f32", 64, 513, 64), ("bf16", 64, 512, 65),
                                         ("bf16", 264, 100, 10), ("bf16", 504, 70, 7)])
def test_reorder_parity(gpu, dtype, d, R, k):
    torch, ah = gpu
    rng = np.random.default_rng(d + R)
    n, nq = max(3000, R + 500), 45
    X = rng.standard_normal((n, d)).astype(np.float32)
    Q = rng.standard_normal((nq, d)).astype(np.float32)
    cand = np.stack([rng.permutation(n)[:R] for _ in range(nq)]).astype(np.int32)
    cand[3, R // 2:] = -1
    cand[4, :] = -1
    if dtype == "f32":
        base_np, base_t, Xr = X, _t(torch, X), X.astype(np.float64)
    else:
        bits = synth.to_bf16_bits(X)
        base_np = bits
        base_t = _t(torch, bits.view(np.int16)).view(torch.bfloat16)
        Xr = synth.bf16_bits_to_f32(bits).astype(np.float64)
    g_ids, g_sc = ah.ah_reorder_exact(_t(torch, Q), base_t, _t(torch, cand), k)
    torch.cuda.synchronize()
    o_ids, o_sc = oracle.reorder(Q, base_np, cand, k)
    Qd = Q.astype(np.float64)
    _check_ranked(_np(g_ids), _np(g_sc), o_ids, o_sc,
                  lambda q, ids: Xr[ids] @ Qd[q], lambda q, ids: np.abs(Xr[ids]) @ np.abs(Qd[q]))
    assert (_np(g_ids)[4] == -1).all() and np.isneginf(_np(g_sc)[4]).all()


# Scores that are small exact integers tie often: the best k, ties broken by
# the lower id, is then unique and the ids must match the oracle exactly.  The
# sizes straddle the one-wave selection (R <= 512, k <= 64) and the workgroup one.
@pytest.mark.parametrize("R,k", [(512, 64), (513, 64), (512, 65), (64, 64), (300, 1)])
def test_reorder_ties(gpu, R, k):
    torch, ah = gpu
    rng = np.random.default_rng(R * 100 + k)
    n, nq, d = 4000, 33, 8
    X = rng.integers(-1, 2, size=(n, d)).astype(np.float32)
    Q = rng.integers(-1, 2, size=(nq, d)).astype(np.float32)
    cand = np.stack([rng.permutation(n)[:R] for _ in range(nq)]).astype(np.int32)
    cand[5, ::3] = -1
    g_ids, g_sc = ah.ah_reorder_exact(_t(torch, Q), _t(torch, X), _t(torch, cand), k)
    torch.cuda.synchronize()
    o_ids, o_sc = oracle.reorder(Q, X, cand, k)
    assert np.array_equal(_np(g_ids), o_ids)
    assert np.array_equal(_np(g_sc), o_sc)


# ----------------------------------------------------------------------------- partition
# One wave per query selects the leaves up to 4096 leaves and 512 searched; the
# workgroup selection beyond (5000 leaves; 600 searched).  d = 9 and 130 leaves
# exercise the unaligned and ragged contraction tiles.
@pytest.mark.parametrize("nq,d,L,nl", [(100, 100, 1000, 50), (67, 128, 300, 7), (5, 1536, 130, 100), (3, 9, 5, 5),
                                       (20, 64, 5000, 30), (10, 32, 700, 600), (300, 384, 4000, 200)])
def test_partition_parity(gpu, nq, d, L, nl):
    torch, ah = gpu
    rng = np.random.default_rng(nq + L)
    Q = rng.standard_normal((nq, d)).astype(np.float32)
    Cn = rng.standard_normal((L, d)).astype(np.float32)
    lv, sc = ah.ah_partition_score(_t(torch, Q), _t(torch, Cn), nl)
    torch.cuda.synchronize()
    o_lv, o_sc = oracle.partition(Q, Cn, nl)
    Qd, Cd = Q.astype(np.float64), Cn.astype(np.float64)
    _check_ranked(_np(lv), _np(sc), o_lv, o_sc,
                  lambda q, ids: Cd[ids] @ Qd[q], lambda q, ids: np.abs(Cd[ids]) @ np.abs(Qd[q]))
    agree = (_np(lv) == o_lv).mean()
    assert agree > 0.99


def test_partition_tied_centroids(gpu):
    """Every centroid repeated four times: equal scores, ties go to the lower leaf id."""
    torch, ah = gpu
    rng = np.random.default_rng(17)
    Q = rng.integers(-3, 4, size=(40, 16)).astype(np.float32)
    Cn = np.repeat(rng.integers(-3, 4, size=(250, 16)).astype(np.float32), 4, axis=0)
    lv, sc = ah.ah_partition_score(_t(torch, Q), _t(torch, Cn), 37)
    torch.cuda.synchronize()
    o_lv, o_sc = oracle.partition(Q, Cn, 37)
    assert np.array_equal(_np(lv), o_lv)  # small integers: exact scores, unique order
    assert np.array_equal(_np(sc), o_sc.astype(np.float32))


@pytest.mark.parametrize("L,nl,kinds", [(3000, 300, 1), (1000, 50, 2), (4000, 200, 3), (200, 64, 1)])
def test_partition_few_score_values(gpu, L, nl, kinds):
    """All leaves share one to three distinct scores: the selection is decided by leaf id alone."""
    torch, ah = gpu
    rng = np.random.default_rng(L + kinds)
    Q = rng.integers(-3, 4, size=(9, 16)).astype(np.float32)
    rows = rng.integers(-3, 4, size=(kinds, 16)).astype(np.float32)
    Cn = rows[rng.integers(0, kinds, size=L)]
    lv, sc = ah.ah_partition_score(_t(torch, Q), _t(torch, Cn), nl)
    torch.cuda.synchronize()
    o_lv, o_sc = oracle.partition(Q, Cn, nl)
    assert np.array_equal(_np(lv), o_lv)
    assert np.array_equal(_np(sc), o_sc.astype(np.float32))


# ----------------------------------------------------------------------------- encoding (codes for the scan)
# Bit-exact against the oracle: both take the argmins in float64 in the same
# order.  dpb 1, 2 and 4 have their own kernels, 3 and 16 the generic one;
# small-integer rows make exact ties (lowest center wins) frequent, and a few
# rows are all zero (u = 0: the loss is |r|^2).
@pytest.mark.parametrize("dtype,n,B,dpb,eta,sweeps,pad", [
    ("f32", 3001, 64, 2, 4.0, 2, 0),
    ("bf16", 2000, 192, 2, 4.0, 2, 0),
    ("f32", 500, 7, 3, 6.0, 3, 5),
    ("f32", 1000, 32, 4, 1.0, 1, 0),
    ("bf16", 777, 50, 1, 4.0, 0, 0),
    ("f32", 300, 5, 16, 9.0, 4, 0),
    ("int", 1000, 16, 2, 4.0, 2, 3),
])
def test_encode_parity(gpu, dtype, n, B, dpb, eta, sweeps, pad):
    torch, ah = gpu
    rng = np.random.default_rng(n + B + dpb)
    d = B * dpb
    if dtype == "int":
        X = rng.integers(-2, 3, size=(n, d)).astype(np.float32)
        cb = rng.integers(-2, 3, size=(B, 16, dpb)).astype(np.float32)
    else:
        X = rng.standard_normal((n, d)).astype(np.float32)
        cb = (0.5 * rng.standard_normal((B, 16, dpb))).astype(np.float32)
    X[::97] = 0.0
    stride = (B + 1) // 2 + pad
    if dtype == "bf16":
        bits = synth.to_bf16_bits(X)
        rows_np, rows_t = bits, _t(torch, bits.view(np.int16)).view(torch.bfloat16)
    else:
        rows_np, rows_t = X, _t(torch, X)
    got = ah.ah_encode(rows_t, _t(torch, cb), eta, sweeps=sweeps, stride=stride)
    torch.cuda.synchronize()
    want = oracle.encode(rows_np, cb, eta, sweeps=sweeps, stride=stride)
    assert np.array_equal(_np(got), want)


# ----------------------------------------------------------------------------- partition assignment
# fp32 contraction against the float64 oracle: a GPU choice is accepted when its
# float64 distance is within the tolerance of the oracle's minimum (R10's rule);
# on small integers everything is exact and the ids must be equal.
@pytest.mark.parametrize("n,d,L,kind", [(5000, 100, 1000, "f"), (3000, 384, 4000, "f"), (70001, 16, 300, "f"),
                                       (2000, 12, 40, "int"), (100, 1536, 2000, "f"), (10, 3, 5, "f")])
def test_assign_leaves_parity(gpu, n, d, L, kind):
    torch, ah = gpu
    rng = np.random.default_rng(n + d + L)
    if kind == "int":
        X = rng.integers(-3, 4, size=(n, d)).astype(np.float32)
        Cn = rng.integers(-3, 4, size=(L, d)).astype(np.float32)
        Cn[L // 2] = Cn[1]
    else:
        X = rng.standard_normal((n, d)).astype(np.float32)
        Cn = rng.standard_normal((L, d)).astype(np.float32)
    X[::997] = 0.0
    ids, sc = ah.ah_assign_leaves(_t(torch, X), _t(torch, Cn), want_scores=True)
    torch.cuda.synchronize()
    ids, sc = _np(ids), _np(sc)
    o_ids, o_dist = oracle.nearest(X, Cn)
    if kind == "int":
        assert np.array_equal(ids, o_ids)
        return
    Xd, Cd = X.astype(np.float64), Cn.astype(np.float64)
    g_dist = ((Xd - Cd[ids]) ** 2).sum(1)
    scale = (Xd * Xd).sum(1) + (Cd[ids] * Cd[ids]).sum(1) + 2 * np.abs(Xd * Cd[ids]).sum(1)
    assert (g_dist <= o_dist + TOL * scale).all()
    assert (ids == o_ids).mean() > 0.99
    # the reported score is x.c - |c|^2/2 of the chosen leaf
    ref = (Xd * Cd[ids]).sum(1) - 0.5 * (Cd[ids] * Cd[ids]).sum(1)
    assert (np.abs(sc - ref) <= TOL * (np.abs(Xd * Cd[ids]).sum(1) + 0.5 * (Cd[ids] * Cd[ids]).sum(1))).all()


# ----------------------------------------------------------------------------- int8 flat search (next row 3)
@pytest.mark.parametrize("n,d,pct,kind", [(300, 512, 99.9, "f"), (200, 7, 99.9, "f"), (100, 1, 99.9, "f"),
                                          (257, 100, 50.0, "f"), (64, 4096, 100.0, "f"), (90, 33, 0.0, "f"),
                                          (500, 64, 99.9, "int")])
def test_sq8_quantize_parity(gpu, n, d, pct, kind):
    torch, ah = gpu
    rng = np.random.default_rng(n + d)
    X = (rng.integers(-4, 5, size=(n, d)) if kind == "int" else rng.standard_normal((n, d))).astype(np.float32)
    X[::37] = 0.0
    codes, scale = ah.ah_sq8_quantize(_t(torch, X), pct)
    torch.cuda.synchronize()
    o_codes, o_scale = oracle.sq8_quantize(X, pct)
    assert np.array_equal(_np(scale), o_scale)
    assert np.array_equal(_np(codes), o_codes)


# Stage-chained: the oracle ranks the GPU's own codes and steps.  The page's
# notebook shape (20,000 x 512, 200 queries, 20-center mixture), ragged tiles,
# R = n, R above the one-wave selection's limit, and both ways to the top R:
# the direct score block (n <= 4096, R > 512) and the candidate path (a bound
# from sampled 64-row group maxima, every gstep-th group when the sample is a
# fraction, then the candidate lists).  `dup` copies of one document at random
# positions make ties at the top (3,000 copies: a long tied run inside the
# lists; every document equal: the lists overflow and the exact redo answers).
@pytest.mark.parametrize("nq,n,d,R,dup", [(200, 20000, 512, 10, 2), (70, 3001, 64, 100, 2), (5, 500, 16, 500, 2),
                                          (130, 10000, 128, 600, 2), (1, 4097, 32, 64, 2),
                                          (300, 50000, 256, 512, 2), (100, 100000, 128, 100, 2),
                                          (150, 40000, 128, 100, 3000), (20, 30000, 64, 50, 30000)])
def test_sq8_topk_parity(gpu, nq, n, d, R, dup):
    torch, ah = gpu
    rng = np.random.default_rng(nq + n + d)
    centers = rng.standard_normal((20, d)).astype(np.float32)
    D = centers[rng.integers(0, 20, n)] + 0.5 * rng.standard_normal((n, d)).astype(np.float32)
    D /= np.linalg.norm(D, axis=1, keepdims=True)
    D[rng.choice(n, size=min(dup, n), replace=False)] = D[3]
    Q = centers[rng.integers(0, 20, nq)] + 0.5 * rng.standard_normal((nq, d)).astype(np.float32)
    if dup >= 3000:
        Q[::2] = D[3]  # half the queries score the copies highest
    d8, ds = ah.ah_sq8_quantize(_t(torch, D.astype(np.float32)))
    q8, qs = ah.ah_sq8_quantize(_t(torch, Q.astype(np.float32)))
    ids, sc = ah.ah_sq8_scan_topk(q8, qs, d8, ds, R)
    torch.cuda.synchronize()
    o_ids, o_sc = oracle.sq8_topk(_np(q8), _np(qs), _np(d8), _np(ds), R)
    assert np.array_equal(_np(ids), o_ids)
    assert np.array_equal(_np(sc), o_sc)


# ----------------------------------------------------------------------------- k-means update
@pytest.mark.parametrize("n,d,L", [(20000, 100, 300), (5000, 384, 4000), (1, 3, 2), (0, 8, 5)])
def test_kmeans_update_parity(gpu, n, d, L):
    """Stage-chained: the GPU's assignment of the rows to the centroids, then the
    update on both sides; float64 sums in another order, so one float32 unit."""
    torch, ah = gpu
    rng = np.random.default_rng(n + d + L)
    X = (rng.standard_normal((n, d)) * 4).astype(np.float32)
    C0 = rng.standard_normal((L, d)).astype(np.float32)
    if n:
        leaf, _ = ah.ah_assign_leaves(_t(torch, X), _t(torch, C0))
        lf = leaf.clone()
        lf[:: 97] = -1  # rows outside every leaf are left out
        lf_np = _np(lf)
    else:
        lf = torch.zeros(0, dtype=torch.int32, device="cuda")
        lf_np = np.zeros(0, np.int32)
    Cg, cnt = ah.ah_kmeans_update(_t(torch, X), lf, _t(torch, C0))
    torch.cuda.synchronize()
    keep = lf_np >= 0
    Co, cnto = oracle.kmeans_update(X[keep], lf_np[keep], C0)
    assert np.array_equal(_np(cnt), cnto)
    g = _np(Cg).astype(np.float64)
    o = Co.astype(np.float64)
    scale = np.abs(X).max() if n else 1.0
    ulp = np.spacing(np.abs(Co)).astype(np.float64)
    assert (np.abs(g - o) <= np.maximum(ulp, 1e-12 * scale)).all()


def test_kmeans_gpu_lloyd_objective_never_rises(gpu):
    """Lloyd iterations on the GPU (assignment, then update) never raise the
    within-leaf squared distance (float64, measured on the host)."""
    torch, ah = gpu
    from mips_ah_partition_amd import index as hix
    rng = np.random.default_rng(5)
    X = (rng.standard_normal((30000, 32)) + rng.integers(0, 5, (30000, 1))).astype(np.float32)
    Xd = _t(torch, X)
    init = rng.choice(30000, 100, replace=False)
    prev = np.inf
    for it in (1, 2, 4, 8):
        C, leaf = hix.kmeans_gpu(Xd, 100, iters=it, init_rows=init)
        torch.cuda.synchronize()
        obj = ((X.astype(np.float64) - _np(C).astype(np.float64)[_np(leaf)]) ** 2).sum()
        assert obj <= prev * (1 + 1e-6)
        prev = obj


# ----------------------------------------------------------------------------- codebook training
@pytest.mark.parametrize("n,B,dpb,eta,few", [(5000, 8, 2, 4.0, False), (3000, 3, 4, 2.5, False),
                                              (4000, 16, 1, 1.0, False), (2000, 6, 2, 4.0, True), (1, 2, 2, 4.0, False)])
def test_pq_update_parity(gpu, n, B, dpb, eta, few):
    """Stage-chained: the same codes and codebooks on both sides; float64 sums
    in another order, so the new centers agree to float32 rounding."""
    torch, ah = gpu
    rng = np.random.default_rng(n + B + dpb)
    X = (rng.standard_normal((n, B * dpb)) + 0.5).astype(np.float32)
    cb = rng.standard_normal((B, 16, dpb)).astype(np.float32)
    codes = synth.random_codes(rng, n, B)
    if few:  # most centers get no rows and keep their values
        codes &= np.uint8(0x11)
    got = ah.ah_pq_update(_t(torch, X), _t(torch, codes), _t(torch, cb), eta)
    torch.cuda.synchronize()
    want = oracle.pq_update(X, codes, cb, eta)
    assert np.allclose(_np(got), want, rtol=1e-5, atol=1e-6 * max(1.0, np.abs(want).max()))


@pytest.mark.parametrize("dpb,B,dtype", [(2, 24, "f32"), (4, 5, "f32"), (2, 48, "bf16"), (3, 7, "f32")])
def test_encode_sweep_from_codes_parity(gpu, dpb, B, dtype):
    torch, ah = gpu
    rng = np.random.default_rng(dpb * 100 + B)
    n = 1500
    X = rng.standard_normal((n, B * dpb)).astype(np.float32)
    cb = (0.7 * rng.standard_normal((B, 16, dpb))).astype(np.float32)
    init = synth.random_codes(rng, n, B)
    if dtype == "bf16":
        bits = synth.to_bf16_bits(X)
        rows = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        ref_rows = bits
    else:
        rows = _t(torch, X)
        ref_rows = X
    codes = _t(torch, init.copy())
    ah.ah_encode_sweep(rows, _t(torch, cb), 4.0, codes, sweeps=2)
    torch.cuda.synchronize()
    assert np.array_equal(_np(codes), oracle.encode(ref_rows, cb, 4.0, sweeps=2, init_codes=init))


def test_train_codebooks_gpu_loss_never_rises(gpu):
    torch, ah = gpu
    from mips_ah_partition_amd import index as hix
    rng = np.random.default_rng(8)
    X = rng.integers(0, 256, size=(20000, 16)).astype(np.float32)
    init = rng.choice(20000, 16, replace=False)
    prev = np.inf
    for it in (1, 2, 4, 6):
        cb, codes = hix.train_codebooks_gpu(_t(torch, X), 2, 4.0, iters=it, init_rows=init)
        torch.cuda.synchronize()
        loss = hix.pq_loss(X, _np(cb), _np(codes), 4.0)
        assert loss <= prev * (1 + 1e-6)
        prev = loss
    host_cb, host_loss = hix.train_codebooks(X, 2, 4.0, iters=6, init_rows=init, return_loss=True)
    assert prev <= host_loss[-1] * 1.01  # the same iterations as the host trainer, to float rounding
