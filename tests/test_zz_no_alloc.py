"""The allocation-free scan entry point (ah_scan_topk_noalloc, scratch in a
static per-GPU array) against ah_scan_topk with a caller workspace: identical
top-R ids and sums, bit for bit, on two calls in a row -- a partitioned batch
on 96-block tables (the staged matrix-core kernel), then a smaller full scan of
three queries (the streaming kernel), which must not see the first call's
leftovers -- and both against the oracle."""
import ctypes as C

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


def _case(rng, n, B, nq, L=0, nl=0):
    codes = synth.random_codes(rng, n, B)
    lut = synth.random_lut_i8(rng, nq, B)
    if L:
        sizes = synth.random_leaf_sizes(rng, n, L, skew=0.8)
        offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
        ids = rng.permutation(n).astype(np.int32)
        leaves = synth.random_probe_lists(rng, nq, L, nl)
        return lut, codes, ids, offs, leaves
    return lut, codes, None, None, None


def test_noalloc_scan_matches_workspace_scan_twice(gpu):
    torch, ah = gpu
    rng = np.random.default_rng(8080)
    T = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    cases = [(_case(rng, 200_000, 96, 48, L=100, nl=10), 100),   # larger: partitioned, staged tables
             (_case(rng, 30_000, 32, 3), 50)]                     # smaller: full scan, three queries
    for (lut, codes, ids, offs, leaves), R in cases:
        nq, B = lut.shape[0], lut.shape[1]
        L = 0 if offs is None else offs.size - 1
        nl = 0 if leaves is None else leaves.shape[1]
        assert ah.ah_scan_workspace_bytes(nq, B, codes.shape[0], L, nl, R) <= ah.AH_SCAN_SCRATCH_BYTES
        args = (T(lut), T(codes), R)
        kw = dict(ids=T(ids), leaf_offsets=T(offs), leaves=T(leaves))
        # the outputs start from a pattern, so stale or unwritten slots show
        out_i = torch.full((nq, R), 7, dtype=torch.int32, device="cuda")
        out_s = torch.full((nq, R), 7, dtype=torch.int32, device="cuda")
        ai, as_ = ah.ah_scan_topk_noalloc(*args, cand_ids_out=out_i, cand_scores_out=out_s, **kw)
        wi, ws_ = ah.ah_scan_topk(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(ai, wi) and torch.equal(as_, ws_)
        oi, os_ = oracle.scan_topk(lut, codes, R, ids=ids, leaf_offsets=offs, leaves=leaves)
        assert np.array_equal(ai.cpu().numpy(), oi) and np.array_equal(as_.cpu().numpy(), os_)


def test_noalloc_scan_rejects_a_batch_beyond_the_scratch(gpu):
    torch, ah = gpu
    lib = ah.lib()
    # 20M rows need 640 MB of fallback slots alone: rejected before anything is enqueued
    fake = C.c_void_p(4096)
    n = 20_000_000
    assert ah.ah_scan_workspace_bytes(16, 64, n, 0, 0, 100) > ah.AH_SCAN_SCRATCH_BYTES
    st = lib.ah_scan_topk_noalloc(fake, 16, 64, fake, 32, n, None, None, 0, None, 0, 100, fake, fake, None)
    assert st == ah.AH_ERR_UNSUPPORTED
