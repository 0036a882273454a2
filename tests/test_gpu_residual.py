"""Parity of the residual (leaf-relative) variant on the GPU with the CPU oracle.

Stage-chained like tests/test_gpu_parity.py: the leaf-term kernel and the
biased scan receive the same inputs as the oracle's ``residual_leaf_bias`` and
biased ``scan_topk``; both are integer results and must match bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mips_ah_partition_amd import ahlib
    ahlib.lib()
    return torch, ahlib


def _t(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("nq,nl,bound", [(1, 1, 100), (37, 50, 1000), (300, 200, 64), (5, 7, 0)])
def test_residual_leaf_bias_parity(gpu, nq, nl, bound):
    torch, ah = gpu
    rng = np.random.default_rng(nq + nl)
    s = -np.sort(-rng.standard_normal((nq, nl)).astype(np.float32), axis=1)
    s[:, 1::3] = s[:, :-1:3][:, : s[:, 1::3].shape[1]]  # equal neighbours
    step = (rng.random(nq) * 0.05).astype(np.float32)
    step[::4] = 0.0       # constant tables
    step[1::7] = 1e-7     # tiny steps: the clip decides
    # exact half steps: differences that are odd multiples of step / 2
    if nl > 2:
        s[:, 2] = s[:, 0] - 2.5 * np.float32(0.25)
        step[2::5] = 0.25
    g = ah.ah_residual_leaf_bias(_t(torch, s), _t(torch, step), bound)
    torch.cuda.synchronize()
    assert np.array_equal(_np(g), oracle.residual_leaf_bias(s, step, bound))


def _case(rng, nq, B, n, L, nl, bias_lim, ties=False):
    lut = (rng.choice(np.array([-1, 1], np.int8), size=(nq, B, 16)) if ties
           else synth.random_lut_i8(rng, nq, B))
    codes = synth.random_codes(rng, n, B)
    sizes = synth.random_leaf_sizes(rng, n, L, skew=1.0)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    ids = rng.permutation(n).astype(np.int32)
    leaves = synth.random_probe_lists(rng, nq, L, nl)
    bias = rng.integers(-bias_lim, bias_lim + 1, size=(nq, nl)).astype(np.int32)
    return lut, codes, offs, ids, leaves, bias


# batches of 1-4 queries take the streaming kernel, larger ones the matrix-core
# kernel; unaligned rows (25 B), several 64-block chunks, a bias bound that clips,
# bound 0 (= the plain scan), heavy ties across leaves, R above the rows scanned
@pytest.mark.parametrize("nq,B,n,L,nl,R,bias_lim,bound,ties", [
    (70, 64, 20000, 100, 10, 200, 3000, 4000, False),
    (70, 64, 20000, 100, 10, 200, 3000, 500, False),
    (130, 32, 8000, 40, 8, 100, 50, 50, True),
    (65, 50, 6001, 30, 6, 37, 800, 1000, False),
    (20, 200, 4000, 16, 4, 300, 5000, 6000, False),
    (9, 16, 3000, 12, 5, 64, 200, 0, False),
    (1, 64, 30000, 50, 20, 100, 3000, 4000, False),
    (2, 64, 30000, 50, 20, 100, 3000, 4000, True),
    (4, 192, 8000, 20, 8, 300, 20000, 30000, False),
    (3, 16, 500, 40, 30, 1000, 100, 100, False),
])
def test_scan_residual_parity(gpu, nq, B, n, L, nl, R, bias_lim, bound, ties):
    torch, ah = gpu
    rng = np.random.default_rng(nq * 7 + B + n + bound)
    lut, codes, offs, ids, leaves, bias = _case(rng, nq, B, n, L, nl, bias_lim, ties)
    g_ids, g_sc = ah.ah_scan_topk(_t(torch, lut), _t(torch, codes), R, ids=_t(torch, ids),
                                  leaf_offsets=_t(torch, offs), leaves=_t(torch, leaves),
                                  leaf_bias=_t(torch, bias), bias_bound=bound)
    torch.cuda.synchronize()
    o_ids, o_sc = oracle.scan_topk(lut, codes, R, ids=ids, leaf_offsets=offs, leaves=leaves, leaf_bias=bias,
                                   bias_bound=bound)
    g_ids, g_sc = _np(g_ids), _np(g_sc)
    bad = np.nonzero((g_ids != o_ids).any(axis=1) | (g_sc != o_sc).any(axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} queries differ, first {bad[:5]}"


def test_scan_residual_tiled_layout(gpu):
    torch, ah = gpu
    rng = np.random.default_rng(41)
    nq, B, n, L, nl, R, bound = 66, 96, 12000, 60, 9, 150, 2000
    lut, codes, offs, ids, leaves, bias = _case(rng, nq, B, n, L, nl, 1500)
    tc = ah.ah_tile_codes(_t(torch, codes), B)
    g_ids, g_sc = ah.ah_scan_topk(_t(torch, lut), tc, R, ids=_t(torch, ids), leaf_offsets=_t(torch, offs),
                                  leaves=_t(torch, leaves), leaf_bias=_t(torch, bias), bias_bound=bound)
    torch.cuda.synchronize()
    o_ids, o_sc = oracle.scan_topk(lut, codes, R, ids=ids, leaf_offsets=offs, leaves=leaves, leaf_bias=bias,
                                   bias_bound=bound)
    assert np.array_equal(_np(g_ids), o_ids) and np.array_equal(_np(g_sc), o_sc)


def test_scan_residual_bias_from_leaf_scores(gpu):
    """The chain the residual search runs: leaf terms from the GPU's own leaf
    scores and steps, then the biased scan, each checked against the oracle
    on the inputs that stage received."""
    torch, ah = gpu
    rng = np.random.default_rng(43)
    nq, B, n, L, nl, R, bound = 100, 50, 40000, 200, 20, 200, 8 * 255 * 50
    X = rng.standard_normal((nq, B * 2)).astype(np.float32)
    C = rng.standard_normal((L, B * 2)).astype(np.float32)
    cb = (0.3 * rng.standard_normal((B, 16, 2))).astype(np.float32)
    leaves, lsc = ah.ah_partition_score(_t(torch, X), _t(torch, C), nl)
    t8, step, beta, _ = ah.ah_build_lut(_t(torch, X), _t(torch, cb))
    bias = ah.ah_residual_leaf_bias(lsc, step, bound)
    codes = synth.random_codes(rng, n, B)
    offs = np.concatenate([[0], np.cumsum(synth.random_leaf_sizes(rng, n, L))]).astype(np.int64)
    g_ids, g_sc = ah.ah_scan_topk(t8, _t(torch, codes), R, leaf_offsets=_t(torch, offs), leaves=leaves,
                                  leaf_bias=bias, bias_bound=bound)
    torch.cuda.synchronize()
    assert np.array_equal(_np(bias), oracle.residual_leaf_bias(_np(lsc), _np(step), bound))
    o_ids, o_sc = oracle.scan_topk(_np(t8), codes, R, leaf_offsets=offs, leaves=_np(leaves), leaf_bias=_np(bias),
                                   bias_bound=bound)
    assert np.array_equal(_np(g_ids), o_ids) and np.array_equal(_np(g_sc), o_sc)


def test_residual_search_end_to_end(gpu):
    """The whole residual search on trained indexes (60,000 rows of the 1M x 100
    mixture workload, 600 leaves, 30 searched, R = 50): the GPU's leaf terms and
    candidates equal the oracle's on the inputs those stages received, and the
    residual codes' final recall is at least the raw codes' at the same bytes
    (the RSLM page's reason for the relative mode)."""
    torch, ah = gpu
    from mips_ah_partition_amd import index as hix
    from mips_ah_partition_amd.search import AHIndex
    w = synth.WORKLOADS["glove1m"]
    X = synth.database(w, 60000)
    Q = synth.queries(w, 300)
    gt, _ = oracle.brute_force(Q, X, 10)
    Qd = _t(torch, Q)
    rec = {}
    for res in (False, True):
        host = hix.build(X, 2, 4.0, num_leaves=600, residual=res, iters=8)
        idx = AHIndex(host, X, num_leaves_to_search=30, reorder=50, final_num_neighbors=10)
        ids, _ = idx.search_batched(Qd)
        torch.cuda.synchronize()
        rec[res] = oracle.recall_at_k(_np(ids), gt)
        if res:
            leaves, lsc = ah.ah_partition_score(Qd, idx.centroids, 30)
            t8, step, _, _ = ah.ah_build_lut(Qd, idx.codebooks)
            lb = ah.ah_residual_leaf_bias(lsc, step, idx.bias_bound)
            cand, csc = ah.ah_scan_topk(t8, idx.codes, 50, ids=idx.ids, leaf_offsets=idx.leaf_offsets, leaves=leaves,
                                        leaf_bias=lb, bias_bound=idx.bias_bound)
            torch.cuda.synchronize()
            assert np.array_equal(_np(lb), oracle.residual_leaf_bias(_np(lsc), _np(step), idx.bias_bound))
            o_ids, o_sc = oracle.scan_topk(_np(t8), host.codes, 50, ids=host.ids, leaf_offsets=host.leaf_offsets,
                                           leaves=_np(leaves), leaf_bias=_np(lb), bias_bound=idx.bias_bound)
            assert np.array_equal(_np(cand), o_ids) and np.array_equal(_np(csc), o_sc)
    print(f"recall@10 raw {rec[False]:.4f} residual {rec[True]:.4f}")
    assert rec[True] >= rec[False] - 0.005
