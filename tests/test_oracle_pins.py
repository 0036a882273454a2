"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a golden
example printed on the pages, a closed form, an independent formulation
(one-hot matrix product, numpy lexsort), brute force on tiny inputs, or a
special case that reduces to the textbook exact search.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def _decode_nibbles(codes, B):
    lo = codes & 15
    hi = codes >> 4
    nib = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.int64)
    nib[:, 0::2] = lo
    nib[:, 1::2] = hi
    return nib[:, :B]


def _onehot_sums(lut_i8, codes, B):
    """Independent formulation: sums = onehot(codes) @ table^T in int64."""
    nib = _decode_nibbles(codes, B)
    n = codes.shape[0]
    oh = np.zeros((n, B * 16), dtype=np.int64)
    rows = np.repeat(np.arange(n), B)
    cols = (np.tile(np.arange(B), n) * 16 + nib.reshape(-1))
    oh[rows, cols] = 1
    return (oh @ lut_i8.reshape(lut_i8.shape[0], -1).astype(np.int64).T).T


# ---------------------------------------------------------------- code layout

def test_nibble_layout_golden():
    g = _golden("nibble_layout.txt")
    row = np.array([[int(h, 16) for h in g["bytes"]]], dtype=np.uint8)
    want = [int(c) for c in g["codes"]]
    B = len(want)
    # a table whose entry at (b, c) is 16*b + c reveals the code read for block b
    lut = np.zeros((1, B, 16), dtype=np.int8)
    for b in range(B):
        lut[0, b, :] = 0
    for b in range(B):
        single = np.zeros((1, B, 16), dtype=np.int8)
        single[0, b, :] = np.arange(16)
        s = oracle.scan_sums(single, row)
        assert int(s[0, 0]) == want[b], (b, int(s[0, 0]), want[b])


# ---------------------------------------------------------------- table (ADC identity)

@pytest.mark.parametrize("dpb,B", [(1, 5), (2, 8), (4, 6), (3, 3)])
def test_adc_identity_float64(dpb, B):
    """Sum of a row's table entries equals q . decode(codes) (ScaNN page,
    "Three stages of a search": the approximate score is the sum of the
    row's table entries, each table entry being q . center)."""
    rng = np.random.default_rng(11 + dpb)
    d = B * dpb
    Q = rng.standard_normal((7, d)).astype(np.float32)
    cb = rng.standard_normal((B, 16, dpb)).astype(np.float32)
    codes = synth.random_codes(rng, 50, B)
    lut = oracle.lut_f64(Q, cb)
    nib = _decode_nibbles(codes, B)
    decoded = np.concatenate([cb[b][nib[:, b]] for b in range(B)], axis=1).astype(np.float64)
    direct = Q.astype(np.float64) @ decoded.T
    via_table = np.zeros_like(direct)
    for b in range(B):
        via_table += lut[:, b, :][:, nib[:, b]]
    assert np.allclose(via_table, direct, rtol=1e-12, atol=1e-12)


def test_lut_transpose_would_fail():
    """A transposed codebook (center/dim swapped) must not satisfy the identity."""
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((2, 4)).astype(np.float32)
    cb = rng.standard_normal((2, 16, 2)).astype(np.float32)
    lut = oracle.lut_f64(Q, cb)
    want = np.einsum("qbt,bct->qbc", Q.reshape(2, 2, 2).astype(np.float64), cb.astype(np.float64))
    assert np.allclose(lut, want, rtol=1e-14)
    wrong = np.einsum("qbt,bct->qbc", Q.reshape(2, 2, 2)[:, ::-1].astype(np.float64), cb.astype(np.float64))
    assert not np.allclose(lut, wrong)


# ---------------------------------------------------------------- int8 quantisation

def test_round_half_even_golden():
    """The int8 lesson's example: 127.5 marks rounds to 128 (ties to even)."""
    g = _golden("int8_rounding_example.txt")
    x, lo, hi, lev = (float(g[k][0]) for k in ("x", "lo", "hi", "levels"))
    scaled = (x - lo) / (hi - lo) * lev
    assert scaled == float(g["scaled"][0])
    assert int(np.rint(scaled)) == int(g["code"][0])
    dec = lo + int(g["code"][0]) / lev * (hi - lo)
    assert round(dec, 5) == float(g["decoded"][0])


def test_quantizer_ties_go_to_even():
    """Build a table whose step makes (v - m_b) * 254/Rng land exactly on k + 0.5:
    Rng = 254/128 gives an exact multiplier of 128, so diffs of (k+0.5)/128 are ties."""
    rng_w = np.float32(254.0 / 128.0)
    half = np.float32(rng_w / 2)
    ks = np.array([0, 1, 2, 3, 10, 11, 62, 125, 126], dtype=np.float64)
    lut = np.zeros((1, 2, 16), dtype=np.float32)
    # block 0 spans [-half, +half] so m_0 = 0 and Rng = rng_w
    lut[0, 0, 0] = -half
    lut[0, 0, 1] = half
    lut[0, 0, 2:2 + len(ks)] = ((ks + 0.5) / 128.0).astype(np.float32)
    lut[0, 0, 2 + len(ks):] = 0
    lut[0, 1, :] = 0.0
    t8, s, beta = oracle.quantize_lut(lut)
    assert s[0] == np.float32(rng_w / np.float32(254.0))
    got = t8[0, 0, 2:2 + len(ks)].astype(int)
    want = [int(k) if int(k) % 2 == 0 else int(k) + 1 for k in ks]
    assert list(got) == want
    assert t8[0, 0, 0] == -127 and t8[0, 0, 1] == 127


def test_quantizer_error_bound_and_range():
    """|beta + s * sum T8 - sum of float table entries| <= B*s/2 (+ float slack)."""
    rng = np.random.default_rng(5)
    nq, B = 6, 40
    lut = (rng.standard_normal((nq, B, 16)) * rng.uniform(0.1, 3.0, size=(1, B, 1))).astype(np.float32)
    t8, s, beta = oracle.quantize_lut(lut)
    assert t8.min() >= -127 and t8.max() <= 127
    assert (np.abs(t8).reshape(nq, -1).max(axis=1) == 127).all()
    codes = synth.random_codes(rng, 300, B)
    nib = _decode_nibbles(codes, B)
    exact = np.zeros((nq, 300))
    for b in range(B):
        exact += lut[:, b, :].astype(np.float64)[:, nib[:, b]]
    isums = _onehot_sums(t8, codes, B)
    approx = beta[:, None].astype(np.float64) + s[:, None].astype(np.float64) * isums
    bound = B * s[:, None] / 2 * (1 + 1e-4) + 1e-4 * np.abs(exact).max()
    assert (np.abs(approx - exact) <= bound).all()
    # a sign flip of the entries breaks the bound
    flipped = beta[:, None] - s[:, None].astype(np.float64) * isums
    assert (np.abs(flipped - exact) > bound).any()


def test_quantizer_constant_table():
    lut = np.full((2, 3, 16), 1.25, dtype=np.float32)
    lut[1] = -0.5
    t8, s, beta = oracle.quantize_lut(lut)
    assert (t8 == 0).all() and (s == 0).all()
    assert beta[0] == np.float32(3.75) and beta[1] == np.float32(-1.5)


# ---------------------------------------------------------------- scan sums and top-R

def test_scan_sums_match_onehot_product():
    rng = np.random.default_rng(7)
    for B in (1, 2, 5, 32, 33):
        lut = synth.random_lut_i8(rng, 4, B)
        codes = synth.random_codes(rng, 257, B)
        got = oracle.scan_sums(lut, codes)
        assert np.array_equal(got.astype(np.int64), _onehot_sums(lut, codes, B))


def _lexsort_topr(sums_row, ids_row, R):
    order = np.lexsort((ids_row, -sums_row.astype(np.int64)))
    keep = order[:R]
    ids = np.full(R, -1, dtype=np.int32)
    sc = np.full(R, np.iinfo(np.int32).min, dtype=np.int32)
    ids[: len(keep)] = ids_row[keep]
    sc[: len(keep)] = sums_row[keep]
    return ids, sc


@pytest.mark.parametrize("seed", range(6))
def test_scan_topk_brute_force_heavy_ties(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 20))
    n = int(rng.integers(1, 900))
    nq = 5
    if seed % 2:
        lut = rng.choice(np.array([-3, 4], dtype=np.int8), size=(nq, B, 16))
    else:
        lut = synth.random_lut_i8(rng, nq, B)
    codes = synth.random_codes(rng, n, B)
    R = int(rng.integers(1, n + 6))
    ids, sc = oracle.scan_topk(lut, codes, R)
    sums = _onehot_sums(lut, codes, B)
    for q in range(nq):
        wi, ws = _lexsort_topr(sums[q].astype(np.int32), np.arange(n, dtype=np.int32), R)
        assert np.array_equal(ids[q], wi) and np.array_equal(sc[q], ws)


def test_scan_topk_partitioned_with_ids_and_empty_leaves():
    rng = np.random.default_rng(9)
    B, n, nq, L, nl, R = 6, 700, 8, 20, 7, 40
    lut = synth.random_lut_i8(rng, nq, B, -5, 5)
    codes = synth.random_codes(rng, n, B)
    sizes = synth.random_leaf_sizes(rng, n, L, skew=1.5)
    sizes[3] = 0
    sizes[4] += 0
    sizes[-1] += n - sizes.sum()
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    perm = rng.permutation(n).astype(np.int32)
    leaves = synth.random_probe_lists(rng, nq, L, nl)
    leaves[0, 0] = 3  # an empty leaf is searched
    ids, sc = oracle.scan_topk(lut, codes, R, ids=perm, leaf_offsets=offs, leaves=leaves)
    sums = _onehot_sums(lut, codes, B)
    for q in range(nq):
        rows = np.concatenate([np.arange(offs[l], offs[l + 1]) for l in leaves[q]]).astype(np.int64)
        wi, ws = _lexsort_topr(sums[q, rows].astype(np.int32), perm[rows], R)
        assert np.array_equal(ids[q], wi) and np.array_equal(sc[q], ws)


def test_scan_topk_empty_database():
    lut = np.zeros((2, 3, 16), dtype=np.int8)
    codes = np.zeros((0, 2), dtype=np.uint8)
    ids, sc = oracle.scan_topk(lut, codes, 4)
    assert (ids == -1).all() and (sc == np.iinfo(np.int32).min).all()


# ---------------------------------------------------------------- reorder, partition, ground truth

def test_reorder_exact_integer_rows_and_ties():
    rng = np.random.default_rng(12)
    X = rng.integers(-3, 4, size=(60, 9)).astype(np.float32)
    X[17] = X[5]  # duplicate row: equal score, lower id must win
    Q = rng.integers(-2, 3, size=(4, 9)).astype(np.float32)
    cand = np.stack([rng.permutation(60)[:30] for _ in range(4)]).astype(np.int32)
    cand[:, 0], cand[:, 1] = 17, 5
    cand[2, 5:9] = -1
    ids, sc = oracle.reorder(Q, X, cand, 8)
    exact = Q.astype(np.int64) @ X.astype(np.int64).T
    for q in range(4):
        c = cand[q][cand[q] >= 0]
        order = np.lexsort((c, -exact[q, c]))[:8]
        assert np.array_equal(ids[q], c[order])
        assert np.array_equal(sc[q], exact[q, c[order]].astype(np.float64))


def test_reorder_bf16_rows_upcast_exactly():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((40, 16)).astype(np.float32)
    bits = synth.to_bf16_bits(X)
    Xb = synth.bf16_bits_to_f32(bits).astype(np.float64)
    Q = rng.standard_normal((3, 16)).astype(np.float32)
    cand = np.tile(np.arange(40, dtype=np.int32), (3, 1))
    ids, sc = oracle.reorder(Q, bits, cand, 5)
    ref = Q.astype(np.float64) @ Xb.T
    for q in range(3):
        order = np.lexsort((np.arange(40), -ref[q]))[:5]
        assert np.array_equal(ids[q], order)
        assert np.allclose(sc[q], ref[q, order], rtol=1e-14, atol=1e-14)


def test_reorder_pads_when_few_candidates():
    X = np.eye(4, dtype=np.float32)
    Q = np.ones((1, 4), dtype=np.float32)
    ids, sc = oracle.reorder(Q, X, np.array([[2, -1, -1]], dtype=np.int32), 3)
    assert list(ids[0]) == [2, -1, -1]
    assert sc[0, 0] == 1.0 and np.isneginf(sc[0, 1:]).all()


def test_partition_hand_case_with_tie():
    Q = np.array([[1.0, 0.0]], dtype=np.float32)
    Cn = np.array([[1, 0], [0, 1], [1, 0], [2, 0]], dtype=np.float32)
    lv, sc = oracle.partition(Q, Cn, 3)
    assert list(lv[0]) == [3, 0, 2]
    assert list(sc[0]) == [2.0, 1.0, 1.0]


def test_brute_force_against_full_sort():
    rng = np.random.default_rng(14)
    X = rng.standard_normal((300, 12)).astype(np.float32)
    X /= np.linalg.norm(X, axis=1, keepdims=True)
    X[200] = X[100]
    Q = rng.standard_normal((6, 12)).astype(np.float32)
    Q[0] = X[100]
    ids, sc = oracle.brute_force(Q, X, 10)
    S = Q.astype(np.float64) @ X.astype(np.float64).T
    for q in range(6):
        order = np.lexsort((np.arange(300), -S[q]))[:10]
        assert np.array_equal(ids[q], order)
    assert ids[0, 0] == 100 and ids[0, 1] == 200


def test_full_reorder_reduces_to_exact_search():
    """With R >= n every row reaches the exact reorder, so the result is the
    textbook exact top-k (recall 1)."""
    rng = np.random.default_rng(15)
    w = synth.WORKLOADS["tiny"]
    X = synth.rows(w, 0, 400)
    Q = synth.rows(w, 0, 5, role=synth.ROLE_QUERY)
    B = w.d // w.dpb
    cb = rng.standard_normal((B, 16, w.dpb)).astype(np.float32)
    codes = synth.random_codes(rng, 400, B)
    res = oracle.search(Q, cb, codes, X, R=400, k=10)
    gt, _ = oracle.brute_force(Q, X, 10)
    assert np.array_equal(res["ids"], gt)
    assert oracle.recall_at_k(res["ids"], gt) == 1.0


# ---------------------------------------------------------------- recall

def test_recall_golden_example():
    g = _golden("recall_example.txt")
    t = np.array([[int(x) for x in g["true"]]])
    f = np.array([[int(x) for x in g["found"]]])
    assert round(oracle.recall_at_k(f, t), 2) == float(g["recall"][0])


def test_recall_ignores_empty_slots_and_averages():
    t = np.array([[1, 2], [3, 4]])
    f = np.array([[2, -1], [4, 3]])
    assert oracle.recall_at_k(f, t) == pytest.approx(0.75)


# ----------------------------------------------------------------------------- anisotropic encoding
def _decode(codes, cb):
    B, _, dpb = cb.shape
    n = codes.shape[0]
    out = np.zeros((n, B * dpb))
    for b in range(B):
        c = (codes[:, b >> 1] >> (4 * (b & 1))) & 15
        out[:, b * dpb:(b + 1) * dpb] = cb[b, c].astype(np.float64)
    return out


def _aniso_loss(X, codes, cb, eta):
    """(eta - 1)(u.r)^2 + |r|^2 per row, written from the definition in float64."""
    Xd = X.astype(np.float64)
    r = Xd - _decode(codes, cb)
    nrm = np.linalg.norm(Xd, axis=1, keepdims=True)
    u = np.divide(Xd, nrm, out=np.zeros_like(Xd), where=nrm > 0)
    return (eta - 1.0) * np.sum(u * r, axis=1) ** 2 + np.sum(r * r, axis=1)


@pytest.mark.parametrize("dpb,B", [(1, 5), (2, 7), (4, 3)])
def test_encode_eta_one_is_per_block_nearest(dpb, B):
    """eta = 1 drops the parallel term: each block takes its nearest center
    (lowest index on ties; small integers make ties frequent)."""
    rng = np.random.default_rng(dpb * 10 + B)
    X = rng.integers(-2, 3, size=(300, B * dpb)).astype(np.float32)
    cb = rng.integers(-2, 3, size=(B, 16, dpb)).astype(np.float32)
    got = oracle.encode(X, cb, 1.0, sweeps=3)
    for b in range(B):
        dist = ((X[:, None, b * dpb:(b + 1) * dpb].astype(np.float64) - cb[b][None].astype(np.float64)) ** 2).sum(-1)
        want = np.argmin(dist, axis=1)  # first minimum: the lowest index
        assert np.array_equal((got[:, b >> 1] >> (4 * (b & 1))) & 15, want)


def test_encode_zero_row_takes_nearest_centers():
    rng = np.random.default_rng(3)
    cb = rng.standard_normal((6, 16, 2)).astype(np.float32)
    X = np.zeros((2, 12), dtype=np.float32)
    got = oracle.encode(X, cb, 9.0, sweeps=2)
    want = np.argmin((cb.astype(np.float64) ** 2).sum(-1), axis=1)
    for b in range(6):
        assert ((got[:, b >> 1] >> (4 * (b & 1))) & 15 == want[b]).all()


def test_encode_sweeps_never_raise_the_loss():
    """Each coordinate step takes the minimiser with the other blocks fixed, so
    the row loss cannot rise from one sweep to the next."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((400, 24)).astype(np.float32)
    cb = rng.standard_normal((12, 16, 2)).astype(np.float32)
    prev = None
    for sw in range(5):
        loss = _aniso_loss(X, oracle.encode(X, cb, 4.0, sweeps=sw), cb, 4.0)
        if prev is not None:
            assert (loss <= prev * (1 + 1e-12) + 1e-12).all()
        prev = loss
    assert (prev < _aniso_loss(X, oracle.encode(X, cb, 4.0, sweeps=0), cb, 4.0) - 1e-9).any()


def test_encode_converged_blocks_are_coordinate_optima():
    """After many sweeps no single block can lower its row's loss (brute force
    over the 16 centers of every block)."""
    rng = np.random.default_rng(12)
    n, B, dpb, eta = 60, 4, 2, 6.0
    X = rng.standard_normal((n, B * dpb)).astype(np.float32)
    cb = rng.standard_normal((B, 16, dpb)).astype(np.float32)
    codes = oracle.encode(X, cb, eta, sweeps=40)
    base = _aniso_loss(X, codes, cb, eta)
    for b in range(B):
        for c in range(16):
            alt = codes.copy()
            alt[:, b >> 1] = (alt[:, b >> 1] & (0xF0 if b % 2 == 0 else 0x0F)) | (c << (4 * (b & 1)))
            assert (_aniso_loss(X, alt, cb, eta) >= base * (1 - 1e-12) - 1e-12).all()


def test_encode_bf16_rows_widen_exactly():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((100, 16)).astype(np.float32)
    bits = synth.to_bf16_bits(X)
    cb = rng.standard_normal((8, 16, 2)).astype(np.float32)
    assert np.array_equal(oracle.encode(bits, cb, 4.0), oracle.encode(synth.bf16_bits_to_f32(bits), cb, 4.0))


# ----------------------------------------------------------------------------- nearest centroid
def test_nearest_matches_exact_integer_argmax_form():
    """On small integers every quantity is exact: argmin |x - c|^2 equals the
    first argmax of x.c - |c|^2/2 computed in int64 (2 x.c - |c|^2)."""
    rng = np.random.default_rng(21)
    X = rng.integers(-3, 4, size=(500, 12)).astype(np.float32)
    Cn = rng.integers(-3, 4, size=(40, 12)).astype(np.float32)
    Cn[7] = Cn[3]  # a duplicate: the lower id must win
    ids, dist = oracle.nearest(X, Cn)
    Xi, Ci = X.astype(np.int64), Cn.astype(np.int64)
    score = 2 * Xi @ Ci.T - (Ci * Ci).sum(1)[None, :]
    assert np.array_equal(ids, np.argmax(score, axis=1))
    assert np.array_equal(dist, ((Xi[:, None, :] - Ci[None]) ** 2).sum(-1).min(1).astype(np.float64))
    assert not (ids == 7).any()


def test_nearest_zero_row_takes_smallest_norm():
    rng = np.random.default_rng(22)
    Cn = rng.standard_normal((30, 8)).astype(np.float32)
    ids, _ = oracle.nearest(np.zeros((3, 8), dtype=np.float32), Cn)
    assert (ids == np.argmin((Cn.astype(np.float64) ** 2).sum(1))).all()


# ----------------------------------------------------------------------------- int8 flat search (next row 3)
@pytest.mark.parametrize("d,pct", [(512, 99.9), (7, 99.9), (1, 99.9), (100, 50.0), (64, 100.0), (33, 0.0)])
def test_sq8_scale_is_numpy_linear_percentile(d, pct):
    rng = np.random.default_rng(d)
    X = rng.standard_normal((50, d)).astype(np.float32)
    X[3] = 0.0  # all zero: the 1e-8 floor
    _, s = oracle.sq8_quantize(X, pct)
    P = np.percentile(np.abs(X), pct, axis=1)
    want = np.maximum(P.astype(np.float32), np.float32(1e-8)) / np.float32(127.0)
    assert np.array_equal(s, want.astype(np.float32))


def test_sq8_codes_round_half_even_and_clip():
    """A row whose 99.9th percentile of |x| is exactly 127 has step 1: codes are
    x rounded half to even and clipped (127.5 -> 128 -> 127, 2.5 -> 2, 3.5 -> 4)."""
    d = 5001  # position 4995: the five largest values sit above the percentile
    x = np.full(d, 127.0, dtype=np.float32)
    x[:4] = [2.5, 3.5, -2.5, -0.5]
    x[-5:] = [127.5, -300.0, 200.0, -150.0, 128.0]
    codes, s = oracle.sq8_quantize(x[None], 99.9)
    assert s[0] == np.float32(1.0)
    assert list(codes[0, :4]) == [2, 4, -2, 0]
    assert list(codes[0, -5:]) == [127, -127, 127, -127, 127]


def test_sq8_topk_is_brute_force_over_exact_dots():
    rng = np.random.default_rng(5)
    D = rng.standard_normal((300, 40)).astype(np.float32)
    D[17] = D[5]  # a duplicate document: equal scores, the lower id first
    Q = rng.standard_normal((9, 40)).astype(np.float32)
    d8, ds = oracle.sq8_quantize(D)
    q8, qs = oracle.sq8_quantize(Q)
    ids, sc = oracle.sq8_topk(q8, qs, d8, ds, 25)
    dots = q8.astype(np.int64) @ d8.astype(np.int64).T  # exact
    full = (dots.astype(np.float32) * qs[:, None]).astype(np.float32) * ds[None, :]
    for q in range(9):
        order = np.lexsort((np.arange(300), -full[q]))[:25]
        assert np.array_equal(ids[q], order)
        assert np.array_equal(sc[q], full[q][order])
    assert all(list(ids[q]).index(5) < list(ids[q]).index(17) for q in range(9) if 5 in ids[q] and 17 in ids[q])


# ---------------------------------------------------------------- residual (leaf-relative) variant

def test_residual_leaf_bias_hand_cases():
    # step 0.25: differences 0, -0.5, -2, -0.125 leaf scores -> 0, -2, -8, -0.5 steps;
    # rint takes -0.5 to 0 and -1.5 to -2 (half to even); the bound clips
    s = np.array([[3.0, 2.5, 1.0, 2.875], [1.0, 0.625, 1.5, 1.0]], dtype=np.float32)
    step = np.array([0.25, 0.25], dtype=np.float32)
    assert oracle.residual_leaf_bias(s, step, 100).tolist() == [[0, -2, -8, 0], [0, -2, 2, 0]]
    assert oracle.residual_leaf_bias(s, step, 5).tolist() == [[0, -2, -5, 0], [0, -2, 2, 0]]
    # a constant table (step 0) carries no leaf term
    assert (oracle.residual_leaf_bias(s, np.zeros(2, np.float32), 100) == 0).all()


def test_residual_scores_decompose_exactly():
    # The variant's premise: with rows x = c_leaf + decode(codes), q.x equals the
    # leaf's centroid score plus the sum of the float64 table at the codes.
    rng = np.random.default_rng(31)
    B, dpb, L, n, nq = 6, 2, 5, 60, 3
    d = B * dpb
    cb = rng.standard_normal((B, 16, dpb)).astype(np.float32)
    cent = rng.standard_normal((L, d)).astype(np.float32)
    leaf = rng.integers(0, L, n)
    codes = synth.random_codes(rng, n, B)
    nib = _decode_nibbles(codes, B)
    dec = np.stack([cb[b, nib[:, b]] for b in range(B)], axis=1).reshape(n, d).astype(np.float64)
    X = cent[leaf].astype(np.float64) + dec
    Q = rng.standard_normal((nq, d)).astype(np.float32)
    lut = oracle.lut_f64(Q, cb)
    adc = np.stack([lut[q][np.arange(B)[None, :], nib].sum(1) for q in range(nq)])
    cs = Q.astype(np.float64) @ cent.astype(np.float64).T
    want = Q.astype(np.float64) @ X.T
    assert np.allclose(cs[:, leaf] + adc, want, rtol=0, atol=1e-9)


def test_scan_topk_zero_bias_is_the_plain_scan():
    rng = np.random.default_rng(32)
    B, n, nq, L, nl, R = 7, 500, 6, 12, 5, 30
    lut = synth.random_lut_i8(rng, nq, B)
    codes = synth.random_codes(rng, n, B)
    offs = np.concatenate([[0], np.cumsum(synth.random_leaf_sizes(rng, n, L))]).astype(np.int64)
    leaves = synth.random_probe_lists(rng, nq, L, nl)
    a = oracle.scan_topk(lut, codes, R, leaf_offsets=offs, leaves=leaves)
    b = oracle.scan_topk(lut, codes, R, leaf_offsets=offs, leaves=leaves,
                         leaf_bias=np.zeros((nq, nl), np.int32), bias_bound=50)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("seed,bound", [(0, 1000), (1, 7), (2, 0), (3, 40)])
def test_scan_topk_biased_brute_force(seed, bound):
    # independent formulation: one-hot sums plus each searched leaf's clipped
    # bias, ranked by numpy lexsort over (score desc, id asc)
    rng = np.random.default_rng(200 + seed)
    B, n, nq, L, nl = int(rng.integers(1, 12)), int(rng.integers(50, 600)), 4, 9, 4
    lut = synth.random_lut_i8(rng, nq, B, -6, 6)
    codes = synth.random_codes(rng, n, B)
    offs = np.concatenate([[0], np.cumsum(synth.random_leaf_sizes(rng, n, L, skew=1.0))]).astype(np.int64)
    leaves = synth.random_probe_lists(rng, nq, L, nl)
    bias = rng.integers(-60, 61, size=(nq, nl)).astype(np.int32)
    perm = rng.permutation(n).astype(np.int32)
    R = int(rng.integers(1, n))
    ids, sc = oracle.scan_topk(lut, codes, R, ids=perm, leaf_offsets=offs, leaves=leaves, leaf_bias=bias,
                               bias_bound=bound)
    sums = _onehot_sums(lut, codes, B)
    for q in range(nq):
        rows = [np.arange(offs[l], offs[l + 1]) for l in leaves[q]]
        tot = np.concatenate([sums[q, r] + int(np.clip(bias[q, j], -bound, bound)) for j, r in enumerate(rows)])
        allr = np.concatenate(rows).astype(np.int64)
        wi, ws = _lexsort_topr(tot.astype(np.int32), perm[allr], R)
        assert np.array_equal(ids[q], wi) and np.array_equal(sc[q], ws)


def test_scan_topk_bias_moves_a_row_across_leaves():
    # two one-row leaves, one block: sums 5 (leaf 0) and 3 (leaf 1); a +3 bias on
    # leaf 1 puts its row first, a +2 bias ties and the lower id wins
    lut = np.zeros((1, 1, 16), np.int8)
    lut[0, 0, 1], lut[0, 0, 2] = 5, 3
    codes = np.array([[1], [2]], np.uint8)
    offs = np.array([0, 1, 2], np.int64)
    leaves = np.array([[0, 1]], np.int32)
    ids, sc = oracle.scan_topk(lut, codes, 2, leaf_offsets=offs, leaves=leaves,
                               leaf_bias=np.array([[0, 3]], np.int32), bias_bound=10)
    assert ids.tolist() == [[1, 0]] and sc.tolist() == [[6, 5]]
    ids, sc = oracle.scan_topk(lut, codes, 2, leaf_offsets=offs, leaves=leaves,
                               leaf_bias=np.array([[0, 2]], np.int32), bias_bound=10)
    assert ids.tolist() == [[0, 1]] and sc.tolist() == [[5, 5]]


# ---------------------------------------------------------------- training-free rotation quantiser
from oracle import rslm  # noqa: E402


def test_rslm_block_layout():
    assert rslm.blocks(384) == [(0, 128), (128, 256), (256, 384)]
    assert rslm.blocks(100) == [(0, 64), (36, 100)]
    assert rslm.blocks(200) == [(0, 128), (72, 200)]
    assert rslm.blocks(5) == [(0, 4), (1, 5)]
    assert rslm.blocks(1) == [(0, 1)]


def test_rslm_rotate_hand_cases():
    s = 1 / np.sqrt(2)
    got = rslm.rotate(np.array([[1.0, 0.0]]), [1, 1], [0, 1])
    assert np.allclose(got, [[s, s]], atol=1e-15)
    # signs (1, -1), permutation (1, 0): (3, 4) -> (3, -4) -> (-4, 3) -> ((-4+3)/sqrt2, (-4-3)/sqrt2)
    got = rslm.rotate(np.array([[3.0, 4.0]]), [1, -1], [1, 0])
    assert np.allclose(got, [[-s, -7 * s]], atol=1e-14)


def _sylvester(b):
    H = np.array([[1.0]])
    while H.shape[0] < b:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("d", [4, 64, 128])
def test_rslm_single_block_is_sylvester_hadamard(d):
    got = rslm.rotate(np.eye(d), np.ones(d), np.arange(d))
    assert np.allclose(got, _sylvester(d) / np.sqrt(d), atol=1e-13)


@pytest.mark.parametrize("d", [5, 100, 200, 384])
def test_rslm_rotation_is_orthogonal(d):
    rng = np.random.default_rng(d)
    signs = rng.choice([-1.0, 1.0], d)
    perm = rng.permutation(d)
    R = rslm.rotate(np.eye(d), signs, perm)  # rows are the images of the unit vectors
    assert np.allclose(R @ R.T, np.eye(d), atol=1e-12)
    X = rng.standard_normal((20, d))
    assert np.allclose(np.linalg.norm(rslm.rotate(X, signs, perm), axis=1), np.linalg.norm(X, axis=1), rtol=1e-12)


def test_rslm_lloyd_max_levels():
    from scipy import integrate
    L = rslm.lloyd_max_gaussian(16)
    assert np.allclose(L, -L[::-1], atol=1e-12)
    # optimality: each level is the conditional mean of its cell (checked by quadrature)
    m = 0.5 * (L[:-1] + L[1:])
    edges = np.concatenate([[-np.inf], m, [np.inf]])
    pdf = lambda z: np.exp(-0.5 * z * z) / np.sqrt(2 * np.pi)  # noqa: E731
    for c in range(16):
        a, b = edges[c], edges[c + 1]
        num = integrate.quad(lambda z: z * pdf(z), a, b, epsabs=1e-13)[0]
        den = integrate.quad(pdf, a, b, epsabs=1e-13)[0]
        assert abs(num / den - L[c]) < 1e-8
    # Max's (1960) table for 16 levels
    want = [0.1284, 0.3881, 0.6568, 0.9424, 1.2562, 1.6180, 2.0690, 2.7326]
    assert np.allclose(L[8:], want, atol=5e-4)


def test_rslm_encode_hand_case():
    L = rslm.lloyd_max_gaussian(16).astype(np.float32)
    # y = (1, -1, 2, 0): |y|^2 = 6, u = y * 2/sqrt(6) = (0.816, -0.816, 1.633, 0): nearest
    # levels 0.9424 (index 11), -0.9424 (4), 1.6180 (13), and 0 lies on the midpoint of
    # +-0.1284, which goes to the lower level (7)
    codes, step = rslm.encode(np.array([[1.0, -1.0, 2.0, 0.0]], np.float32), L)
    assert codes.tolist() == [[11 | (4 << 4), 13 | (7 << 4)]]
    lv = L[[11, 4, 13, 7]].astype(np.float64)
    _, lam = rslm.int8_levels(L)
    assert step[0] == np.float32(np.sqrt(6.0) / np.sqrt((lv * lv).sum()) / lam)
    assert rslm.expand(codes, 4, rslm.int8_levels(L)[0]).tolist() == [
        [int(v) for v in np.rint(L[[11, 4, 13, 7]].astype(np.float64) * lam)]]


def test_rslm_reconstruction_keeps_the_norm():
    rng = np.random.default_rng(12)
    L = rslm.lloyd_max_gaussian(16).astype(np.float32)
    Y = rng.standard_normal((50, 96)).astype(np.float32) * rng.random((50, 1)).astype(np.float32) * 5
    codes, step = rslm.encode(Y, L)
    lv8, lam = rslm.int8_levels(L)
    nib = np.empty((50, 96), np.int64)
    nib[:, 0::2], nib[:, 1::2] = codes & 15, codes >> 4
    rec = (step.astype(np.float64) * lam)[:, None] * L[nib].astype(np.float64)
    assert np.allclose(np.linalg.norm(rec, axis=1), np.linalg.norm(Y.astype(np.float64), axis=1), rtol=1e-6)
    assert lv8[-1] == 127 and lv8[0] == -127 and (lv8 == -lv8[::-1]).all()


# ---------------------------------------------------------------- k-means update
def test_kmeans_update_hand_case_and_empty_leaf():
    X = np.array([[1, 2], [3, 4], [10, 10], [-1, 0]], np.float32)
    C0 = np.array([[0, 0], [5, 5], [7, 7]], np.float32)
    C, cnt = oracle.kmeans_update(X, np.array([0, 0, 1, 0]), C0)
    # leaf 0: mean of (1,2), (3,4), (-1,0) = (1, 2); leaf 1: (10, 10); leaf 2 empty: kept
    assert C.tolist() == [[1.0, 2.0], [10.0, 10.0], [7.0, 7.0]] and cnt.tolist() == [3, 1, 0]


def test_kmeans_update_minimises_the_within_leaf_squared_distance():
    rng = np.random.default_rng(21)
    X = rng.standard_normal((3000, 8)).astype(np.float32) * 3
    C0 = X[rng.choice(3000, 40, replace=False)]
    lf, _ = oracle.nearest(X, C0)
    C, cnt = oracle.kmeans_update(X, lf, C0)
    Xd = X.astype(np.float64)
    for l in range(40):
        m = lf == l
        if not m.any():
            continue
        # the gradient of sum |x - c|^2 vanishes (up to the float32 rounding of c)
        g = 2 * (C[l].astype(np.float64) * m.sum() - Xd[m].sum(0))
        assert np.abs(g).max() <= 1e-6 * m.sum() * (np.abs(Xd[m]).max() + 1)
    # a Lloyd step never raises the objective
    before = ((Xd - C0[lf]) ** 2).sum()
    after = ((Xd - C[lf].astype(np.float64)) ** 2).sum()
    assert after <= before


# ---------------------------------------------------------------- codebook training update
def test_pq_update_at_eta_one_is_the_per_block_mean():
    rng = np.random.default_rng(41)
    B, dpb, n = 5, 2, 800
    X = rng.standard_normal((n, B * dpb)).astype(np.float32)
    cb = rng.standard_normal((B, 16, dpb)).astype(np.float32)
    codes = synth.random_codes(rng, n, B)
    new = oracle.pq_update(X, codes, cb, 1.0)
    nib = _decode_nibbles(codes, B)
    for b in range(B):
        for c in range(16):
            m = nib[:, b] == c
            want = X[m, b * dpb:(b + 1) * dpb].astype(np.float64).mean(0) if m.any() else cb[b, c]
            assert np.allclose(new[b, c], want, rtol=1e-6, atol=1e-7)


def test_pq_update_one_block_is_the_stationary_vq_solution():
    # one block: s_i - p_ib = 0, so each center solves (sum (eta-1) u u^T + m I) c = sum eta... form
    rng = np.random.default_rng(42)
    d, eta, n = 4, 3.0, 600
    X = (rng.standard_normal((n, d)) + 1.5).astype(np.float32)
    cb = rng.standard_normal((1, 16, d)).astype(np.float32)
    codes = synth.random_codes(rng, n, 1)
    new = oracle.pq_update(X, codes, cb, eta)
    U = X / np.linalg.norm(X, axis=1, keepdims=True)
    for c in range(16):
        m = (codes[:, 0] & 15) == c
        if not m.any():
            assert np.array_equal(new[0, c], cb[0, c])
            continue
        Xm, Um = X[m].astype(np.float64), U[m].astype(np.float64)
        A = (eta - 1) * Um.T @ Um + m.sum() * np.eye(d)
        rhs = (Xm + (eta - 1) * (Um * Xm).sum(1, keepdims=True) * Um).sum(0)
        assert np.allclose(new[0, c], np.linalg.solve(A, rhs), rtol=1e-5, atol=1e-6)


def test_pq_training_step_never_raises_the_loss():
    rng = np.random.default_rng(43)
    B, dpb, n, eta = 6, 2, 1500, 4.0
    X = rng.standard_normal((n, B * dpb)).astype(np.float32)
    cb = X[rng.choice(n, 16, replace=False)].reshape(16, B, dpb).transpose(1, 0, 2).copy()
    def loss(codes, cbk):
        nib = _decode_nibbles(codes, B)
        rec = np.stack([cbk[b, nib[:, b]] for b in range(B)], 1).reshape(n, -1).astype(np.float64)
        R = X.astype(np.float64) - rec
        u = X.astype(np.float64) / np.linalg.norm(X.astype(np.float64), axis=1, keepdims=True)
        return ((eta - 1) * (R * u).sum(1) ** 2 + (R * R).sum(1)).sum()
    codes = oracle.encode(X, cb, eta, sweeps=1)
    prev = loss(codes, cb)
    for _ in range(3):
        cb = oracle.pq_update(X, codes, cb, eta)
        l1 = loss(codes, cb)
        codes = oracle.encode(X, cb, eta, sweeps=1, init_codes=codes)
        l2 = loss(codes, cb)
        assert l1 <= prev * (1 + 1e-9) and l2 <= l1 * (1 + 1e-9)
        prev = l2


def _pack_nibbles(nib):
    """uint8 [n, ceil(B/2)] from nibbles [n, B] (low nibble = even block)."""
    n, B = nib.shape
    full = np.zeros((n, B + (B & 1)), dtype=np.uint8)
    full[:, :B] = nib
    return (full[:, 0::2] | (full[:, 1::2] << 4)).astype(np.uint8)


def _aniso_grad_last_block(X, codes, cb, eta):
    """Gradient of sum_i (eta-1)(u_i.r_i)^2 + |r_i|^2 with respect to the last
    block's 16 centers, written from the loss's definition in float64 (r_i is the
    row minus its decoded codes, u_i the row's unit direction).  Also returns the
    scale of each center's gradient terms (sum of their magnitudes) and counts."""
    B, _, dpb = cb.shape
    Xd = X.astype(np.float64)
    r = Xd - _decode(codes, cb)
    u = Xd / np.linalg.norm(Xd, axis=1, keepdims=True)
    par = np.sum(u * r, axis=1, keepdims=True)
    sl = slice((B - 1) * dpb, B * dpb)
    term = -2.0 * ((eta - 1.0) * par * u[:, sl] + r[:, sl])
    nib = _decode_nibbles(codes, B)[:, B - 1]
    grad = np.zeros((16, dpb))
    scale = np.zeros(16)
    np.add.at(grad, nib, term)
    np.add.at(scale, nib, np.abs(term).sum(1))
    return grad, scale, np.bincount(nib, minlength=16)


def _rotate_blocks(X, nib, cb, j):
    """Move block j to the last position (blocks j+1.. move down by one)."""
    B, _, dpb = cb.shape
    order = [b for b in range(B) if b != j] + [j]
    cols = np.concatenate([np.arange(b * dpb, (b + 1) * dpb) for b in order])
    return np.ascontiguousarray(X[:, cols]), _pack_nibbles(nib[:, order]), np.ascontiguousarray(cb[order])


def _uncoupled_update(X, codes, cb, eta):
    """A plausible mistake, planted here on the CPU: each block's center solved
    as if the other blocks' parallel errors were zero (the coupling term dropped)."""
    B, _, dpb = cb.shape
    Xd = X.astype(np.float64)
    U = Xd / np.linalg.norm(Xd, axis=1, keepdims=True)
    nib = _decode_nibbles(codes, B)
    out = cb.astype(np.float64).copy()
    for b in range(B):
        sl = slice(b * dpb, (b + 1) * dpb)
        for c in range(16):
            m = nib[:, b] == c
            if not m.any():
                continue
            Ub, Xb = U[m, sl], Xd[m, sl]
            A = (eta - 1.0) * Ub.T @ Ub + m.sum() * np.eye(dpb)
            rhs = (Xb + (eta - 1.0) * np.sum(Ub * Xb, axis=1, keepdims=True) * Ub).sum(0)
            out[b, c] = np.linalg.solve(A, rhs)
    return out.astype(np.float32)


@pytest.mark.parametrize("B,dpb,eta", [(3, 2, 4.0), (4, 2, 0.5), (3, 3, 6.0), (2, 4, 2.5)])
def test_pq_update_last_block_is_stationary_with_coupling(B, dpb, eta):
    # ScaNN page, "Training an anisotropic codebook yourself": each center solves
    # the closed-form minimiser of the anisotropic loss, and with blocks the
    # parallel error couples them.  The update goes block by block (0 .. B-1), so
    # after it the last block's centers minimise the whole loss with every other
    # block at its new value: the gradient of the loss, written from its
    # definition, vanishes there.  Rotating the block order puts each block last.
    rng = np.random.default_rng(4500 + 10 * B + dpb)
    n = 1200
    X = (rng.standard_normal((n, B * dpb)) + 0.7).astype(np.float32)
    cb = rng.standard_normal((B, 16, dpb)).astype(np.float32)
    nib = _decode_nibbles(synth.random_codes(rng, n, B), B)
    nib[:5, :] = 3  # center 3 of every block has rows; some centers may be empty
    for j in range(B):
        Xr, cr, cbr = _rotate_blocks(X, nib, cb, j)
        new = oracle.pq_update(Xr, cr, cbr, eta)
        grad, scale, cnt = _aniso_grad_last_block(Xr, cr, new, eta)
        # the solve is float64; the stored center is float32, so the gradient is
        # the float32 rounding of each center times the loss's curvature
        tol = 2.0 * max(eta, 1.0) * cnt[:, None] * np.abs(new[-1]).max() * 2.0 ** -22 + 1e-9 * scale[:, None]
        assert (np.abs(grad) <= tol).all(), (j, np.abs(grad).max())
        assert np.array_equal(new[-1][cnt == 0], cbr[-1][cnt == 0])
        # the same check rejects an update that drops the coupling term
        bad = _uncoupled_update(Xr, cr, cbr, eta)
        gbad, _, _ = _aniso_grad_last_block(Xr, cr, bad, eta)
        assert (np.abs(gbad) > tol).any()


def test_encode_from_given_codes_with_zero_sweeps_returns_them():
    rng = np.random.default_rng(44)
    X = rng.standard_normal((50, 8)).astype(np.float32)
    cb = rng.standard_normal((4, 16, 2)).astype(np.float32)
    init = synth.random_codes(rng, 50, 4)
    assert np.array_equal(oracle.encode(X, cb, 4.0, sweeps=0, init_codes=init), init)
