"""Parity at the workloads' full sizes, in the launch configuration the benchmark
uses, checked on sampled queries that the oracle computes one by one.

On trained (GPU-built) indexes the oracle computes each sampled query from its
own intermediates (tables, top-R), only the leaves being chained when two leaf
scores tie within the tolerance; on the random-structure shapes it receives the
GPU stage's inputs.  Integer results must match exactly; float scores within
1e-4 relative (float64 reference, denominator max(|ref|, sum |a_j b_j|)).
"""
import time

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


def _log(msg):
    print(f"[fullsize {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _sample(nq, k=6):
    return sorted(set([0, 1, nq // 3, nq // 2, nq - 2, nq - 1][:k]))


def _check_scan(lut_q, codes, R, gpu_ids, gpu_sc, ids=None, offs=None, leaves_q=None):
    o_ids, o_sc = oracle.scan_topk(lut_q, codes, R, ids=ids, leaf_offsets=offs, leaves=leaves_q)
    assert np.array_equal(gpu_ids, o_ids), "top-R ids differ"
    assert np.array_equal(gpu_sc, o_sc), "top-R sums differ"


def _check_reorder(Qs, rows_of, cand, k, g_ids, g_sc):
    """rows_of(ids) -> float64 rows; the oracle reorders the same candidates."""
    for i in range(Qs.shape[0]):
        c = cand[i][cand[i] >= 0]
        Xr = rows_of(c)
        ref = Xr @ Qs[i].astype(np.float64)
        den = np.abs(Xr) @ np.abs(Qs[i].astype(np.float64))
        order = np.lexsort((c, -ref))[:k]
        gi = g_ids[i][g_ids[i] >= 0]
        pos = {int(x): j for j, x in enumerate(c)}
        gref = np.array([ref[pos[int(x)]] for x in gi])
        gden = np.array([den[pos[int(x)]] for x in gi])
        assert len(gi) == len(order)
        assert (np.abs(g_sc[i][:len(gi)] - gref) <= TOL * np.maximum(np.abs(gref), gden)).all()
        assert (np.abs(gref - ref[order]) <= 2 * TOL * np.maximum(np.abs(gref), gden)).all()


def _trained(torch, w):
    """The benchmark's inputs and GPU-built index for workload w."""
    import bench
    from mips_ah_partition_amd import index as ixm
    from mips_ah_partition_amd.search import AHIndex
    base, X, Q = bench.make_inputs(w, torch)
    _log(f"{w.name}: rows ready; building the index on the GPU")
    dix = ixm.build_gpu(base, w.dpb, w.eta, num_leaves=w.num_leaves, seed=1000 * w.index + synth.ROLE_CODEBOOK)
    index = AHIndex.from_device(dix, base, num_leaves_to_search=w.leaves_to_search, reorder=w.reorder,
                                final_num_neighbors=w.k)
    torch.cuda.synchronize()
    _log(f"{w.name}: index ready")
    return base, X, Q, dix, index


def _trained_case(gpu, name):
    """Whole path at a workload's full size on its trained (GPU-built) index, in
    the launch configuration the benchmark times.  Sampled queries are checked
    stage by stage against the oracle on its own intermediates: leaves (near
    ties accepted, then the GPU's leaves are chained), the float32 and int8
    tables bit for bit, top-R ids and sums bit for bit, reorder within 1e-4.
    No query's candidate list may overflow (the exact fallback is not needed)."""
    torch, ah = gpu
    w = synth.WORKLOADS[name]
    base, X, Q, dix, index = _trained(torch, w)
    Qd = torch.from_numpy(Q).cuda()
    fid, fsc = index.search_batched(Qd)
    L = w.num_leaves if index.partitioned else 0
    nl = w.leaves_to_search if index.partitioned else 0
    appended, overflowed = ah.scan_counters(index._ws["scan"], w.nq, w.blocks, w.n, L, nl, w.reorder)
    _log(f"{name}: search done; {appended.mean():.0f} candidates appended per query, {overflowed} overflowed")
    assert overflowed == 0
    leaves = None
    if index.partitioned:
        leaves, lsc = ah.ah_partition_score(Qd, dix.centroids, nl)
    t8, s, beta, l32 = ah.ah_build_lut(Qd, dix.codebooks, want_f32=True)
    cand, csum = ah.ah_scan_topk(t8, dix.codes, w.reorder, ids=dix.ids,
                                 leaf_offsets=dix.leaf_offsets if leaves is not None else None, leaves=leaves)
    fid2, _ = ah.ah_reorder_exact(Qd, index.base, cand, w.k)
    torch.cuda.synchronize()
    assert torch.equal(fid, fid2), "search_batched differs from the same calls made one by one"
    S = _sample(w.nq)
    hix = dix.to_host()
    lv = None
    if leaves is not None:
        lv = leaves[S].cpu().numpy()
        o_lv, o_ls = oracle.partition(Q[S], hix.centroids, nl)
        Cd, Qs = hix.centroids.astype(np.float64), Q[S].astype(np.float64)
        for i in range(len(S)):
            ref = Cd[lv[i]] @ Qs[i]
            den = np.abs(Cd[lv[i]]) @ np.abs(Qs[i])
            assert (np.abs(ref - o_ls[i]) <= 2 * TOL * np.maximum(np.abs(ref), den)).all()
    l32o = oracle.lut_f64(Q[S], hix.codebooks).astype(np.float32)
    assert np.array_equal(l32[S].cpu().numpy(), l32o)
    o8, os_, ob = oracle.quantize_lut(l32o)
    assert np.array_equal(t8[S].cpu().numpy(), o8)
    assert np.array_equal(s[S].cpu().numpy(), os_) and np.array_equal(beta[S].cpu().numpy(), ob)
    _check_scan(o8, hix.codes, w.reorder, cand[S].cpu().numpy(), csum[S].cpu().numpy(), ids=hix.ids,
                offs=hix.leaf_offsets if lv is not None else None, leaves_q=lv)
    _log(f"{name}: sampled stage parity ok")
    cs = cand[S].cpu().numpy()
    rows = {}
    for i in range(len(S)):
        c = cs[i][cs[i] >= 0]
        r = index.base[torch.from_numpy(c.astype(np.int64)).cuda()].float().cpu().numpy().astype(np.float64)
        rows.update({int(x): r[j] for j, x in enumerate(c)})
    _check_reorder(Q[S], lambda c: np.stack([rows[int(x)] for x in c]), cs, w.k, fid[S].cpu().numpy(),
                   fsc[S].cpu().numpy())
    s_all = csum.cpu().numpy()
    assert (np.diff(s_all, axis=1) <= 0).all()
    del base, X, dix, index, cand, csum, fid, fid2
    torch.cuda.empty_cache()


def test_sift1m_trained_full_size(gpu):
    """1,000,000 x 128 integer rows, 64 blocks x 2 dims, eta = 4, 10,000 queries, R=200, k=10."""
    _trained_case(gpu, "sift1m")


def test_glove1m_trained_full_size(gpu):
    """1,000,000 x 100 mixture rows, 1,000 leaves / 50 searched, 50 blocks x 2 dims, R=200."""
    _trained_case(gpu, "glove1m")


def test_openai2m_trained_full_size(gpu):
    """2,000,000 x 1536 bf16 mixture rows, 2,000 leaves / 100 searched, 768 blocks, 1,000 queries, R=400."""
    _trained_case(gpu, "openai2m")


def test_wiki20m_trained_full_size(gpu):
    """20,000,000 x 384 bf16 mixture rows, 4,000 leaves / 200 searched, 192 blocks, 10,000 queries, R=300."""
    _trained_case(gpu, "wiki20m")


def test_tiny_whole_path_every_query(gpu):
    """10,000 x 128 unit rows, 32 blocks x 4 dims (eta = 1), 100 queries, R=100:
    every query through every stage, against the oracle on the GPU's inputs."""
    torch, ah = gpu
    from mips_ah_partition_amd import index as ixm
    w = synth.WORKLOADS["tiny"]
    X = synth.database(w)
    Q = synth.queries(w)
    ix = ixm.build(X, w.dpb, w.eta, seed=1000 * w.index + synth.ROLE_CODEBOOK)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    Qd = T(Q)
    t8, s, beta, l32 = ah.ah_build_lut(Qd, T(ix.codebooks), want_f32=True)
    cand, csum = ah.ah_scan_topk(t8, T(ix.codes), w.reorder)
    fid, fsc = ah.ah_reorder_exact(Qd, T(X), cand, w.k)
    torch.cuda.synchronize()
    l32, t8 = l32.cpu().numpy(), t8.cpu().numpy()
    assert np.array_equal(l32, oracle.lut_f64(Q, ix.codebooks).astype(np.float32))
    assert np.array_equal(t8, oracle.quantize_lut(l32)[0])
    _check_scan(t8, ix.codes, w.reorder, cand.cpu().numpy(), csum.cpu().numpy())
    _check_reorder(Q, lambda c: X[c].astype(np.float64), cand.cpu().numpy(), w.k, fid.cpu().numpy(),
                   fsc.cpu().numpy())
    gt, _ = oracle.brute_force(Q, X, w.k)
    res = oracle.search(Q, ix.codebooks, ix.codes, X, w.reorder, w.k)
    # the oracle's own whole path (its own tables, candidates and float64 reorder):
    # tables and candidates equal the GPU's bit for bit, and recall@10 is at least the oracle's
    assert np.array_equal(res["lut_i8"], t8) and np.array_equal(res["cand_ids"], cand.cpu().numpy())
    assert oracle.recall_at_k(fid.cpu().numpy(), gt) >= oracle.recall_at_k(res["ids"], gt)


def _partitioned_case(gpu, name, generate_originals_on_gpu):
    """Full-size partitioned shapes with synthetic structure: lognormal leaf sizes,
    random codes and id permutation, random centroids; real mixture queries."""
    torch, ah = gpu
    w = synth.WORKLOADS[name]
    rng = np.random.default_rng(7000 + w.index)
    B, n, L = w.blocks, w.n, w.num_leaves
    _log(f"{name}: generating {n} x {w.code_bytes} B codes")
    codes = np.empty((n, w.code_bytes), dtype=np.uint8)
    step = 1 << 21
    for a in range(0, n, step):
        codes[a:a + step] = rng.integers(0, 256, size=(min(step, n - a), w.code_bytes), dtype=np.uint8)
    sizes = synth.random_leaf_sizes(rng, n, L, skew=0.7)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    perm = rng.permutation(n).astype(np.int32)
    Q = synth.queries(w)
    cent = rng.standard_normal((L, w.d)).astype(np.float32)
    cb = (rng.standard_normal((B, 16, w.dpb)) * 0.1).astype(np.float32)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    Qd = T(Q)
    codes_d, offs_d, perm_d = T(codes), T(offs), T(perm)
    _log(f"{name}: running the path")
    leaves, lsc = ah.ah_partition_score(Qd, T(cent), w.leaves_to_search)
    t8, s, beta, l32 = ah.ah_build_lut(Qd, T(cb), want_f32=True)
    cand, csum = ah.ah_scan_topk(t8, codes_d, w.reorder, ids=perm_d, leaf_offsets=offs_d, leaves=leaves)
    g = torch.Generator(device="cuda")
    g.manual_seed(9000 + w.index)
    if generate_originals_on_gpu:
        base = torch.randn((n, w.d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    else:
        base = torch.randn((n, w.d), generator=g, device="cuda", dtype=torch.float32)
    fid, fsc = ah.ah_reorder_exact(Qd, base, cand, w.k)
    torch.cuda.synchronize()
    _log(f"{name}: gpu path done")
    S = _sample(w.nq, 4)
    lv = leaves[S].cpu().numpy()
    o_lv, o_ls = oracle.partition(Q[S], cent, w.leaves_to_search)
    gls = lsc[S].cpu().numpy()
    Cd, Qs = cent.astype(np.float64), Q[S].astype(np.float64)
    for i in range(len(S)):
        ref = Cd[lv[i]] @ Qs[i]
        den = np.abs(Cd[lv[i]]) @ np.abs(Qs[i])
        assert (np.abs(gls[i] - ref) <= TOL * np.maximum(np.abs(ref), den)).all()
        assert (np.abs(ref - o_ls[i]) <= 2 * TOL * np.maximum(np.abs(ref), den)).all()
    t8s = t8[S].cpu().numpy()
    assert np.array_equal(t8s, oracle.quantize_lut(l32[S].cpu().numpy())[0])
    _check_scan(t8s, codes, w.reorder, cand[S].cpu().numpy(), csum[S].cpu().numpy(), ids=perm, offs=offs,
                leaves_q=lv)
    _log(f"{name}: scan sampled parity ok")
    cs = cand[S].cpu().numpy()
    rows = {}
    for i in range(len(S)):
        c = cs[i][cs[i] >= 0]
        r = base[torch.from_numpy(c.astype(np.int64)).cuda()].float().cpu().numpy().astype(np.float64)
        rows.update({int(x): r[j] for j, x in enumerate(c)})
    _check_reorder(Q[S], lambda c: np.stack([rows[int(x)] for x in c]), cs, w.k, fid[S].cpu().numpy(),
                   fsc[S].cpu().numpy())
    s_all = csum.cpu().numpy()
    assert (np.diff(s_all, axis=1) <= 0).all()


def test_glove1m_partitioned_shape(gpu):
    _partitioned_case(gpu, "glove1m", False)


def test_openai2m_partitioned_shape(gpu):
    _partitioned_case(gpu, "openai2m", True)


def test_wiki20m_partitioned_shape(gpu):
    _partitioned_case(gpu, "wiki20m", True)


def test_encode_fullsize_sampled(gpu):
    """Coupled encoding of the 20M x 384 bf16 shape in one launch (as the
    benchmark times it); sampled rows re-encoded by the oracle must match bit
    for bit."""
    torch, ah = gpu
    w = synth.WORKLOADS["wiki20m"]
    _log("encode: generating 20M x 384 bf16 rows on the GPU")
    X = synth.gpu_normal_rows(torch, w.n, w.d, 6161, torch.bfloat16)
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    cb = 0.5 * torch.randn((w.blocks, 16, w.dpb), generator=g, device="cuda")
    codes = ah.ah_encode(X, cb, w.eta, sweeps=2)
    torch.cuda.synchronize()
    _log("encode: done; checking sampled rows")
    idx = torch.tensor(sorted(set([0, 1, 63, 64, w.n // 2, w.n - 2, w.n - 1] +
                                  list(range(1_000_003, w.n, 2_000_017)))), device="cuda")
    rows = X[idx].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.encode(rows, cb.cpu().numpy(), w.eta, sweeps=2)
    assert np.array_equal(codes[idx].cpu().numpy(), want)
    del X, codes
    torch.cuda.empty_cache()


def test_assign_fullsize_sampled(gpu):
    """Nearest of 4,000 centroids for all 20M x 384 rows in one call (row chunks
    inside); sampled rows checked against the float64 oracle with the fp32 rule."""
    torch, ah = gpu
    w = synth.WORKLOADS["wiki20m"]
    _log("assign: generating 20M x 384 fp32 rows on the GPU")
    X = synth.gpu_normal_rows(torch, w.n, w.d, 6363, torch.float32)
    g = torch.Generator(device="cuda")
    g.manual_seed(78)
    C = torch.randn((w.num_leaves, w.d), generator=g, device="cuda")
    ids, _ = ah.ah_assign_leaves(X, C)
    torch.cuda.synchronize()
    _log("assign: done; checking sampled rows")
    idx = torch.tensor(sorted(set([0, 1, 65535, 65536, w.n // 2, w.n - 1] +
                                  list(range(1_000_003, w.n, 1_000_033)))), device="cuda")
    Xs = X[idx].cpu().numpy()
    Cn = C.cpu().numpy()
    gi = ids[idx].cpu().numpy()
    o_ids, o_dist = oracle.nearest(Xs, Cn)
    Xd, Cd = Xs.astype(np.float64), Cn.astype(np.float64)
    g_dist = ((Xd - Cd[gi]) ** 2).sum(1)
    scale = (Xd * Xd).sum(1) + (Cd[gi] * Cd[gi]).sum(1) + 2 * np.abs(Xd * Cd[gi]).sum(1)
    assert (g_dist <= o_dist + TOL * scale).all()
    del X
    torch.cuda.empty_cache()


def test_sq8_flat_fullsize_sampled(gpu):
    """Int8 flat search at 1M x 512 with 10,000 queries and R = 100, in the
    launch configuration the benchmark times (one call, candidate path);
    sampled queries ranked by the oracle over the same codes and steps must
    match exactly."""
    torch, ah = gpu
    nd, dd, nqs, R = 1_000_000, 512, 10_000, 100
    _log("sq8: generating and quantising 1M x 512 documents, 10k queries")
    Dv = synth.gpu_normal_rows(torch, nd, dd, 6464, torch.float32)
    Qv = synth.gpu_normal_rows(torch, nqs, dd, 6465, torch.float32)
    d8, ds = ah.ah_sq8_quantize(Dv)
    q8, qs = ah.ah_sq8_quantize(Qv)
    del Dv, Qv
    ids, sc = ah.ah_sq8_scan_topk(q8, qs, d8, ds, R)
    torch.cuda.synchronize()
    _log("sq8: done; checking sampled queries")
    idx = _sample(nqs) + [4097, 7777]
    o_ids, o_sc = oracle.sq8_topk(q8[idx].cpu().numpy(), qs[idx].cpu().numpy(), d8.cpu().numpy(),
                                  ds.cpu().numpy(), R)
    assert np.array_equal(ids[idx].cpu().numpy(), o_ids)
    assert np.array_equal(sc[idx].cpu().numpy(), o_sc)
    del d8, q8
    torch.cuda.empty_cache()


def test_rslm_flat_fullsize_sampled(gpu):
    """The rotation quantiser at 1M x 512 with 10,000 queries and R = 100, in
    the configuration the benchmark times; sampled queries ranked by the
    oracle over the GPU's own codes, steps and query codes must match exactly."""
    torch, ah = gpu
    from mips_ah_partition_amd.rslm import RSLMIndex
    from oracle import rslm as orslm
    nd, dd, nqs, R = 1_000_000, 512, 10_000, 100
    _log("rslm: generating, rotating and encoding 1M x 512 documents")
    Dv = synth.gpu_normal_rows(torch, nd, dd, 6464, torch.float32)
    Qv = synth.gpu_normal_rows(torch, nqs, dd, 6465, torch.float32)
    signs, perm = synth.rotation_draws(dd, 1)
    rix = RSLMIndex(Dv, signs, perm)
    ids, sc = rix.search(Qv, R)
    Qr = ah.ah_rslm_rotate(Qv, rix.signs, rix.perm)
    q8, qs = ah.ah_sq8_quantize(Qr)
    torch.cuda.synchronize()
    _log("rslm: done; checking sampled queries")
    idx = _sample(nqs) + [4097]
    lv8, _ = orslm.int8_levels(orslm.lloyd_max_gaussian(16).astype(np.float32))
    d8 = orslm.expand(rix.codes.cpu().numpy(), dd, lv8)
    o_ids, o_sc = oracle.sq8_topk(q8[idx].cpu().numpy(), qs[idx].cpu().numpy(), d8, rix.step.cpu().numpy(), R)
    assert np.array_equal(ids[idx].cpu().numpy(), o_ids)
    assert np.array_equal(sc[idx].cpu().numpy(), o_sc)
    del Dv, rix
    torch.cuda.empty_cache()
