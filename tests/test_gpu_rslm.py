"""Parity of the training-free rotation quantiser on the GPU with the oracle.

Stage-chained: the encoder receives the GPU's own rotated rows on both sides,
the scan the GPU's codes, steps and query codes.  Rotation: float32
butterflies against the float64 orthonormal matrix, every element within
1e-5 of the row's norm.  Codes, top-R ids and scores: bit for bit; row steps
within 1e-6 relative (float64 sums of squares in another order).
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import rslm as orslm

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


@pytest.mark.parametrize("n,d", [(300, 128), (257, 100), (64, 200), (40, 384), (17, 1536), (9, 5), (3, 1)])
def test_rslm_rotate_parity(gpu, n, d):
    torch, ah = gpu
    rng = np.random.default_rng(n + d)
    X = (rng.standard_normal((n, d)) * rng.random((n, 1)) * 3).astype(np.float32)
    X[0] = 0.0
    signs, perm = synth.rotation_draws(d, d)
    Y = ah.ah_rslm_rotate(_t(torch, X), _t(torch, signs), _t(torch, perm))
    torch.cuda.synchronize()
    ref = orslm.rotate(X, signs, perm)
    nrm = np.linalg.norm(X.astype(np.float64), axis=1, keepdims=True)
    assert (np.abs(_np(Y) - ref) <= 1e-5 * nrm + 1e-30).all()


@pytest.mark.parametrize("n,d", [(500, 128), (300, 100), (100, 384), (20, 1536), (5, 3)])
def test_rslm_encode_parity(gpu, n, d):
    torch, ah = gpu
    from mips_ah_partition_amd import rslm as prslm
    rng = np.random.default_rng(7 * n + d)
    X = (rng.standard_normal((n, d)) * rng.random((n, 1)) * 4).astype(np.float32)
    X[1] = 0.0
    signs, perm = synth.rotation_draws(d, 3)
    Y = ah.ah_rslm_rotate(_t(torch, X), _t(torch, signs), _t(torch, perm))
    L = prslm.gaussian_levels()
    codes, step = ah.ah_rslm_encode(Y, L)
    torch.cuda.synchronize()
    o_codes, o_step = orslm.encode(_np(Y), orslm.lloyd_max_gaussian(16).astype(np.float32))
    assert np.array_equal(_np(codes), o_codes)
    assert np.allclose(_np(step), o_step, rtol=1e-6, atol=0)


# the direct score block (n <= 4096, R > 512), the candidate path (sampled
# bound), d above 512 (the generic kernel), ties from duplicated documents
@pytest.mark.parametrize("nq,n,d,R,dup", [(200, 20000, 512, 10, 1), (70, 3001, 64, 100, 1), (5, 500, 16, 500, 1),
                                          (130, 10000, 128, 600, 1), (100, 60000, 128, 100, 2000),
                                          (3, 20000, 1536, 50, 1), (64, 9000, 384, 200, 1)])
def test_rslm_scan_parity(gpu, nq, n, d, R, dup):
    torch, ah = gpu
    from mips_ah_partition_amd import rslm as prslm
    rng = np.random.default_rng(nq + n + d)
    centers = rng.standard_normal((20, d)).astype(np.float32)
    X = centers[rng.integers(0, 20, n)] + 0.5 * rng.standard_normal((n, d)).astype(np.float32)
    X[rng.choice(n, size=dup, replace=False)] = X[3]
    Q = centers[rng.integers(0, 20, nq)] + 0.5 * rng.standard_normal((nq, d)).astype(np.float32)
    signs, perm = synth.rotation_draws(d, 5)
    sg, pm = _t(torch, signs), _t(torch, perm)
    L = prslm.gaussian_levels()
    lv8 = prslm.int8_levels(L)
    codes, step = ah.ah_rslm_encode(ah.ah_rslm_rotate(_t(torch, X), sg, pm), L)
    q8, qs = ah.ah_sq8_quantize(ah.ah_rslm_rotate(_t(torch, Q), sg, pm))
    ids, sc = ah.ah_rslm_scan_topk(q8, qs, codes, step, d, lv8, R)
    torch.cuda.synchronize()
    o_lv8, _ = orslm.int8_levels(orslm.lloyd_max_gaussian(16).astype(np.float32))
    d8 = orslm.expand(_np(codes), d, o_lv8)
    o_ids, o_sc = oracle.sq8_topk(_np(q8), _np(qs), d8, _np(step), R)
    assert np.array_equal(_np(ids), o_ids)
    assert np.array_equal(_np(sc), o_sc)
