#!/usr/bin/env python3
"""Benchmark of the AH search path on one MI355X.

A step is one pass of the whole path over one query batch with every input
already resident in HBM: centroid scoring + leaf choice (partitioned workloads
only), per-query int8 tables, code scan + top-R, exact reorder to the final k.
Prints one JSON line: queries/s at the measured recall@10, the scan kernel's
roofline fraction (HIP events around the main scan kernel), and the CPU oracle
timed on a bounded sample of the same queries.

Usage: python bench.py [--steps K] [--warmup W] [--workload sift1m] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

CACHE = os.path.join(ROOT, "cache")
METRIC = "queries/sec at recall@10 (AH 4-bit scan + reorder); code-scan HBM GB/s"
INDEX_VERSION = 1

# MI355X published peaks
PEAK_HBM_GBPS = 8000.0
PEAK_INT8_TOPS = 5000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- HIP events
class HipEvents:
    def __init__(self):
        self.h = C.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.h.hipEventSynchronize.argtypes = [C.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.h.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        e = C.c_void_p()
        if self.h.hipEventCreate(C.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def record(self, e, stream):
        if self.h.hipEventRecord(C.c_void_p(e), C.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        self.h.hipEventSynchronize(C.c_void_p(b))
        ms = C.c_float()
        if self.h.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


# ----------------------------------------------------------------------------- inputs
def workload_arrays(w):
    X = synth.database(w)
    Q = synth.queries(w)
    return X, Q


def load_index(w, X):
    from mips_ah_partition_amd import index as ixm
    os.makedirs(CACHE, exist_ok=True)
    path = os.path.join(CACHE, f"{w.name}_index_v{INDEX_VERSION}.npz")
    if os.path.exists(path):
        return ixm.load(path)
    t0 = time.time()
    log(f"[bench] building index for {w.name} (n={w.n}, d={w.d}, {w.blocks} blocks, eta={w.eta}) ...")
    ix = ixm.build(X, w.dpb, w.eta, num_leaves=w.num_leaves, seed=1000 * w.index + synth.ROLE_CODEBOOK)
    ixm.save(path, ix)
    log(f"[bench] index built in {time.time() - t0:.1f}s")
    return ix


def ground_truth(w, X, Q, torch, k=10, shortlist=64):
    """Exact top-k by float64 score, (score desc, id asc), cached per workload."""
    path = os.path.join(CACHE, f"{w.name}_gt_v{INDEX_VERSION}.npy")
    if os.path.exists(path):
        return np.load(path)
    gt = exact_topk(X, Q, torch, k, shortlist)
    np.save(path, gt)
    return gt


def exact_topk(X, Q, torch, k=10, shortlist=64):
    """Exact top-k by float64 score, (score desc, id asc): an fp32 GPU shortlist
    of the best `shortlist` rows re-ranked in float64 on the host."""
    Xt = torch.from_numpy(X).cuda()
    gt = np.empty((Q.shape[0], k), dtype=np.int32)
    step = max(1, (1 << 31) // (4 * X.shape[0]))
    Xd = X.astype(np.float64)
    for a in range(0, Q.shape[0], step):
        qb = torch.from_numpy(Q[a:a + step]).cuda()
        cand = torch.topk(qb @ Xt.T, shortlist, dim=1).indices.cpu().numpy()
        for i in range(cand.shape[0]):
            c = cand[i]
            s = Xd[c] @ Q[a + i].astype(np.float64)
            gt[a + i] = c[np.lexsort((c, -s))[:k]]
    del Xt
    return gt


def profiled_traffic(workload):
    """HBM bytes per launch of the main scan kernel from the committed rocprofv3
    summary (profiles/scan_main_<workload>.txt), or None when the kernel source
    has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"scan_main_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = os.path.join(ROOT, "mips_ah_partition_amd", "csrc", "ah_scan.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel_source", "").split()[-1:] != [sha]:
        return None
    return float(fields["scan_main_traffic_bytes"])


def recall(found, truth):
    hit = 0
    for f, t in zip(found, truth):
        hit += len(set(f[f >= 0].tolist()) & set(t.tolist()))
    return hit / truth.size


# ----------------------------------------------------------------------------- CPU baseline
def cpu_baseline(w, ix, X, Q, gt, gpu_ids, budget_s=20.0):
    """The oracle as it stands, on the first queries of the batch (bounded sample)."""
    import oracle
    base = X if w.originals == "f32" else synth.to_bf16_bits(X)
    # calibrate on one query, then size the sample to the time budget
    t0 = time.perf_counter()
    oracle.search(Q[:1], ix.codebooks, ix.codes, base, w.reorder, w.k, centroids=ix.centroids,
                  leaf_offsets=ix.leaf_offsets, ids=ix.ids, nl=w.leaves_to_search)
    one = time.perf_counter() - t0
    threads = oracle.num_threads()
    ns = int(max(threads, min(Q.shape[0], budget_s / max(one, 1e-6) * threads * 0.8)))
    ns = min(ns, Q.shape[0])
    t0 = time.perf_counter()
    res = oracle.search(Q[:ns], ix.codebooks, ix.codes, base, w.reorder, w.k, centroids=ix.centroids,
                        leaf_offsets=ix.leaf_offsets, ids=ix.ids, nl=w.leaves_to_search)
    dt = time.perf_counter() - t0
    return {
        "value": ns / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
        "sample": f"first {ns} of {Q.shape[0]} queries, whole path (table, scan, top-{w.reorder}, reorder)",
        "seconds": dt,
        "recall_at_10": recall(res["ids"], gt[:ns]),
        "gpu_recall_at_10_same_sample": recall(gpu_ids[:ns], gt[:ns]),
        "final_ids_equal_fraction": float((res["ids"] == gpu_ids[:ns]).all(axis=1).mean()),
    }


# ----------------------------------------------------------------------------- code-scan HBM probe
# Single-pass streaming scans at low reuse: 1 and 4 queries over codes of the
# 20M x 384-dim (192 blocks, 96 B rows) and 2M x 1536-dim (768 blocks, 384 B
# rows) workloads' shapes, no partitioning.  Both code arrays exceed the 256 MB
# last-level cache, so every run reads them from HBM.  Codes are uniform random
# nibbles generated on the GPU (seeded); tables are uniform int8.
PROBE_SHAPES = (("wiki20m", 20_000_000, 192, 300), ("openai2m", 2_000_000, 768, 400))


def code_scan_probe(torch, ahlib, ev, runs=5):
    """Single-pass scans of 1 and 4 queries over all codes, in the tiled layout
    (ah_tile_codes; keys name_qN) and row-major (keys name_qN_rowmajor)."""
    out = {}
    for name, n, B, R in PROBE_SHAPES:
        g = torch.Generator(device="cuda")
        g.manual_seed(4242 + B)
        codes = torch.randint(0, 256, (n, (B + 1) // 2), generator=g, device="cuda", dtype=torch.uint8)
        tiled = ahlib.ah_tile_codes(codes, B)
        for nq in (1, 4):
            lut = torch.randint(-127, 128, (nq, B, 16), generator=g, device="cuda", dtype=torch.int8)
            ws = torch.empty(ahlib.ah_scan_workspace_bytes(nq, B, n, 0, 0, R), dtype=torch.uint8, device="cuda")
            e0, e1 = ev.create(), ev.create()
            for layout, src in (("", tiled), ("_rowmajor", codes)):
                ts = []
                for it in range(runs + 1):
                    ahlib.ah_scan_topk(lut, src, R, workspace=ws, main_events=(e0, e1))
                    torch.cuda.synchronize()
                    if it:
                        ts.append(ev.elapsed_ms(e0, e1))
                ms = float(np.median(ts))
                gbps = codes.numel() / (ms / 1e3) / 1e9
                o_cnt = (nq * 4 + 255) & ~255  # candidate counters follow the thresholds in the workspace
                appended = ws[o_cnt:o_cnt + nq * 4].view(torch.int32).cpu().numpy()
                out[f"{name}_q{nq}{layout}"] = {"code_bytes": int(codes.numel()), "blocks": B, "queries": nq,
                                                "layout": "tiled" if not layout else "row-major",
                                                "scan_ms": ms, "GBps": gbps, "frac_of_8TBps": gbps / PEAK_HBM_GBPS,
                                                "candidates_per_query": float(appended.mean())}
            del ws
        del codes, tiled
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- other rows at their shapes
# Centroid scoring (a1), table build (a2) and bf16 reorder (a5) at the shapes of
# the partitioned workloads, on seeded random inputs generated on the GPU, each
# against its roofline: a1 is a dense fp32 contraction (2 nq L d FLOP, MFMA fp32
# peak), a2 writes the int8 tables (nq B 16 bytes, HBM), a5 gathers the
# candidates' rows (nq R d 2 bytes for bf16, HBM).
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_FP64_TFLOPS = 78.6  # vector float64


def _time_ms(torch, fn, runs=5):
    ts = []
    for it in range(runs + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        if it:
            ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def stage_probes(torch, ahlib):
    from mips_ah_partition_amd import costs
    out = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(5151)
    for name in ("glove1m", "openai2m", "wiki20m"):
        w = synth.WORKLOADS[name]
        Q = torch.randn((w.nq, w.d), generator=g, device="cuda")
        C = torch.randn((w.num_leaves, w.d), generator=g, device="cuda")
        ms = _time_ms(torch, lambda: ahlib.ah_partition_score(Q, C, w.leaves_to_search))
        tf = 2.0 * w.nq * w.num_leaves * w.d / (ms / 1e3) / 1e12
        out[f"a1_partition_{name}"] = {"nq": w.nq, "leaves": w.num_leaves, "d": w.d, "searched": w.leaves_to_search,
                                       "ms": ms, "TFLOPs": tf, "frac_of_fp32_mfma": tf / PEAK_FP32_MFMA_TFLOPS}
        cb = torch.randn((w.blocks, 16, w.dpb), generator=g, device="cuda")
        ms = _time_ms(torch, lambda: ahlib.ah_build_lut(Q, cb))
        byt = w.nq * w.blocks * 16 + w.nq * w.d * 4
        out[f"a2_lut_{name}"] = {"nq": w.nq, "blocks": w.blocks, "ms": ms, "GBps": byt / (ms / 1e3) / 1e9,
                                 "frac_of_8TBps": byt / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS}
        del C
    # residual (leaf-relative) codes against raw codes at equal bytes: 100,000 rows of the
    # 1M x 100 mixture workload, 600 leaves (30 searched), 50 blocks x 2 dims, R = 50, k = 10,
    # 1,000 queries; indexes trained on the host, the search on the GPU
    from mips_ah_partition_amd import index as hix
    from mips_ah_partition_amd.search import AHIndex
    w = synth.WORKLOADS["glove1m"]
    Xr = synth.database(w, 100_000)
    Qr = synth.queries(w, 1000)
    gt_r = exact_topk(Xr, Qr, torch, 10)
    Qrd = torch.from_numpy(Qr).cuda()
    res = {"rows": Xr.shape[0], "d": w.d, "leaves": 600, "searched": 30, "R": 50, "k": 10, "queries": Qr.shape[0]}
    for tag, residual in (("raw", False), ("residual", True)):
        host = hix.build(Xr, w.dpb, w.eta, num_leaves=600, residual=residual, iters=8)
        ai = AHIndex(host, Xr, num_leaves_to_search=30, reorder=50, final_num_neighbors=10)
        ids_r, _ = ai.search_batched(Qrd)
        ms = _time_ms(torch, lambda: ai.search_batched(Qrd))
        res[f"{tag}_recall_at_10"] = recall(ids_r.cpu().numpy(), gt_r)
        res[f"{tag}_ms"] = ms
        res[f"{tag}_queries_per_s"] = Qr.shape[0] / (ms / 1e3)
    out["residual_vs_raw_glove_100k"] = res
    del Xr, Qrd
    # int8 flat search (second workload): 1M documents x 512 dims, 10,000 queries, R = 100,
    # then the exact fp32 rescore to k = 10; the contraction is int8 MFMA (2 nq n d ops)
    nd, dd, nqs, Rs = 1_000_000, 512, 10_000, 100
    Dv = synth.gpu_normal_rows(torch, nd, dd, 6464, torch.float32)
    Qv = synth.gpu_normal_rows(torch, nqs, dd, 6465, torch.float32)
    d8, dsc = ahlib.ah_sq8_quantize(Dv)
    q8, qsc = ahlib.ah_sq8_quantize(Qv)
    wss = torch.empty(ahlib.ah_sq8_workspace_bytes(nqs, nd, dd, Rs), dtype=torch.uint8, device="cuda")
    ids = torch.empty((nqs, Rs), dtype=torch.int32, device="cuda")
    scs = torch.empty((nqs, Rs), dtype=torch.float32, device="cuda")
    ms_q = _time_ms(torch, lambda: ahlib.ah_sq8_quantize(Qv, codes_out=q8, scale_out=qsc), runs=3)
    ms_s = _time_ms(torch, lambda: ahlib.ah_sq8_scan_topk(q8, qsc, d8, dsc, Rs, ids_out=ids, scores_out=scs,
                                                          workspace=wss), runs=3)
    ms_r = _time_ms(torch, lambda: ahlib.ah_reorder_exact(Qv, Dv, ids, 10), runs=3)
    gt_v = exact_topk(Dv.cpu().numpy(), Qv.cpu().numpy(), torch, 10)
    f_ids, _ = ahlib.ah_reorder_exact(Qv, Dv, ids, 10)
    sq8_recall = recall(f_ids.cpu().numpy(), gt_v)
    sq8_recall_cand = recall(ids[:, :10].cpu().numpy(), gt_v)
    # the training-free rotation quantiser on the same corpus: 4-bit codes (256 MB instead of
    # the int8 rows' 512 MB), the same int8 matrix-core scan reading them, the same rescore
    from mips_ah_partition_amd.rslm import RSLMIndex
    signs, perm = synth.rotation_draws(dd, 1)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    rix = RSLMIndex(Dv, signs, perm)
    t1.record()
    torch.cuda.synchronize()
    ms_build = t0.elapsed_time(t1)
    r_ids, _ = rix.search(Qv, Rs, base=Dv, k=10)
    r_cand, _ = rix.search(Qv, Rs)
    ms_rs = _time_ms(torch, lambda: rix.search(Qv, Rs, base=Dv, k=10), runs=3)
    out["rslm4_flat_1m_x_512"] = {"docs": nd, "d": dd, "queries": nqs, "R": Rs, "k": 10, "code_bytes_per_doc": dd // 2,
                                  "encode_ms": ms_build, "search_ms": ms_rs,
                                  "queries_per_s": nqs / (ms_rs / 1e3),
                                  "recall_at_10": recall(r_ids.cpu().numpy(), gt_v),
                                  "recall_at_10_before_rescore": recall(r_cand[:, :10].cpu().numpy(), gt_v),
                                  "int8_recall_at_10_same_corpus": sq8_recall,
                                  "int8_recall_at_10_before_rescore": sq8_recall_cand}
    del rix
    ops = 2.0 * nqs * nd * dd
    out["sq8_flat_1m_x_512"] = {"docs": nd, "d": dd, "queries": nqs, "R": Rs, "k": 10,
                                "quantize_queries_ms": ms_q, "scan_topk_ms": ms_s, "rescore_ms": ms_r,
                                "queries_per_s": nqs / ((ms_q + ms_s + ms_r) / 1e3),
                                "scan_int8_TOPs": ops / (ms_s / 1e3) / 1e12,
                                "scan_frac_of_int8_peak": ops / (ms_s / 1e3) / 1e12 / 5000.0}
    del Dv, Qv, d8, wss
    torch.cuda.empty_cache()
    # partition assignment (nearest of 4,000 centroids) for 4M rows of the 20M x 384 shape:
    # the fp32 MFMA contraction (2 n L d FLOP) plus the one-wave selection per row
    w = synth.WORKLOADS["wiki20m"]
    na = 4_000_000
    X = synth.gpu_normal_rows(torch, na, w.d, 6262, torch.float32)
    C = torch.randn((w.num_leaves, w.d), generator=g, device="cuda")
    lv = torch.empty(na, dtype=torch.int32, device="cuda")
    wsa = torch.empty(ahlib.ah_assign_workspace_bytes(na, w.num_leaves), dtype=torch.uint8, device="cuda")
    ms = _time_ms(torch, lambda: ahlib.ah_assign_leaves(X, C, leaf_out=lv, workspace=wsa), runs=3)
    tf = 2.0 * na * w.num_leaves * w.d / (ms / 1e3) / 1e12
    out["assign_wiki20m_4M_rows"] = {"rows": na, "leaves": w.num_leaves, "d": w.d, "ms": ms, "TFLOPs": tf,
                                     "frac_of_fp32_mfma": tf / PEAK_FP32_MFMA_TFLOPS}
    # the k-means update on the same rows and assignment (one Lloyd iteration = assignment + update):
    # reads the rows once (n d 4 bytes) plus n d float64 atomic adds into L d sums
    Cu = C.clone()
    wsk = torch.empty(ahlib.ah_kmeans_workspace_bytes(w.num_leaves, w.d), dtype=torch.uint8, device="cuda")
    ms_u = _time_ms(torch, lambda: ahlib.ah_kmeans_update(X, lv, Cu, workspace=wsk), runs=3)
    out["kmeans_update_wiki20m_4M_rows"] = {"rows": na, "leaves": w.num_leaves, "d": w.d, "ms": ms_u,
                                            "row_GBps": na * w.d * 4 / (ms_u / 1e3) / 1e9,
                                            "atomic_adds_per_s": na * w.d / (ms_u / 1e3)}
    del Cu, wsk
    del X, wsa, lv
    torch.cuda.empty_cache()
    # anisotropic codebook training on the GPU at the 20M x 384 shape's training sample:
    # 250,000 rows, 192 blocks x 2 dims, eta = 4, 10 iterations (sweep + block-by-block update)
    from mips_ah_partition_amd import index as hix
    Xt = synth.gpu_normal_rows(torch, 250_000, w.d, 6060, torch.float32)
    init = np.random.default_rng(60).choice(250_000, 16, replace=False)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    hix.train_codebooks_gpu(Xt, w.dpb, w.eta, iters=1, init_rows=init)
    t0.record()
    hix.train_codebooks_gpu(Xt, w.dpb, w.eta, iters=10, init_rows=init)
    t1.record()
    torch.cuda.synchronize()
    out["train_codebooks_wiki20m_sample"] = {"rows": 250_000, "d": w.d, "blocks": w.blocks, "iters": 10,
                                             "ms": t0.elapsed_time(t1)}
    del Xt
    # encoding (the codes the scan reads) at the 20M x 384 shape, bf16 rows, two sweeps:
    # a float64 vector-ALU kernel, counted by costs.encode_flops_per_row
    w = synth.WORKLOADS["wiki20m"]
    X = synth.gpu_normal_rows(torch, w.n, w.d, 6161, torch.bfloat16)
    cb = 0.5 * torch.randn((w.blocks, 16, w.dpb), generator=g, device="cuda")
    codes = torch.empty((w.n, (w.blocks + 1) // 2), dtype=torch.uint8, device="cuda")
    ms = _time_ms(torch, lambda: ahlib.ah_encode(X, cb, w.eta, sweeps=2, codes_out=codes), runs=3)
    fl = w.n * costs.encode_flops_per_row(w.d, w.dpb, 2)
    out["encode_wiki20m"] = {"rows": w.n, "d": w.d, "dtype": "bf16", "sweeps": 2, "ms": ms, "rows_per_s": w.n / (ms / 1e3),
                             "fp64_TFLOPs": fl / (ms / 1e3) / 1e12,
                             "frac_of_fp64_vector": fl / (ms / 1e3) / 1e12 / PEAK_FP64_TFLOPS}
    del X, codes
    torch.cuda.empty_cache()
    # bf16 reorder at the 2M x 1536 shape: 1,000 queries x 400 random candidates
    w = synth.WORKLOADS["openai2m"]
    base = torch.randn((w.n, w.d), generator=g, device="cuda").to(torch.bfloat16)
    Q = torch.randn((w.nq, w.d), generator=g, device="cuda")
    cand = torch.randint(0, w.n, (w.nq, w.reorder), generator=g, device="cuda", dtype=torch.int32)
    ms = _time_ms(torch, lambda: ahlib.ah_reorder_exact(Q, base, cand, w.k))
    byt = w.nq * w.reorder * w.d * 2
    out["a5_reorder_bf16_openai2m"] = {"nq": w.nq, "R": w.reorder, "d": w.d, "ms": ms,
                                       "GBps": byt / (ms / 1e3) / 1e9, "frac_of_8TBps": byt / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS}
    del base
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sift1m", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-probe", action="store_true", help="skip the code-scan HBM probe")
    ap.add_argument("--probe-only", action="store_true", help="only run the code-scan HBM probe")
    ap.add_argument("--stages-only", action="store_true", help="only run the other rows' probes (a1, a2, a5)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device 5 times (calibrates FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the search runs on one GPU only; --gpus must be 1 "
                                   "(sharding across GPUs is not implemented)"}))
        sys.exit(2)

    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": src.numel() * 4, "launches": 5}))
        return

    if args.stages_only:
        import torch
        from mips_ah_partition_amd import ahlib
        ahlib.lib()
        print(json.dumps({"stage_probes": stage_probes(torch, ahlib)}), flush=True)
        return
    if args.probe_only:
        import torch
        from mips_ah_partition_amd import ahlib
        ahlib.lib()
        print(json.dumps({"code_scan_hbm": code_scan_probe(torch, ahlib, HipEvents())}), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    t0 = time.time()
    X, Q = workload_arrays(w)
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
    ix = load_index(w, X)

    import torch
    from mips_ah_partition_amd import ahlib, costs
    from mips_ah_partition_amd.search import AHIndex
    ahlib.lib()
    gt = ground_truth(w, X, Q, torch, k=w.k)
    base = X if w.originals == "f32" else synth.to_bf16_bits(X)
    index = AHIndex(ix, base, num_leaves_to_search=w.leaves_to_search, reorder=w.reorder, final_num_neighbors=w.k,
                    base_is_bf16_bits=(w.originals == "bf16"))
    Qd = torch.from_numpy(Q).cuda()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    ev = HipEvents()
    stages = ["lut", "scan", "reorder"] + (["partition"] if index.partitioned else [])
    evs = {s: [(ev.create(), ev.create()) for _ in range(args.steps)] for s in stages + ["scan_main"]}

    def timers(i):
        t = {s: (lambda e=evs[s][i][0]: ev.record(e, sh), lambda e=evs[s][i][1]: ev.record(e, sh)) for s in stages}
        t["scan_main"] = evs["scan_main"][i]
        return t

    for _ in range(args.warmup):
        ids, scores = index.search_batched(Qd)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ids, scores = index.search_batched(Qd, timers=timers(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    qps = Q.shape[0] / (wall / args.steps)
    stage_ms = {s: float(np.mean([ev.elapsed_ms(*evs[s][i]) for i in range(args.steps)])) for s in evs}
    gpu_ids = ids.cpu().numpy()
    rec = recall(gpu_ids, gt)

    # roofline of the dominant kernel: the main code-scan kernel on the int8 matrix cores.
    qc = costs.per_query(w.n, w.d, w.dpb, w.num_leaves, w.leaves_to_search, w.reorder)
    if index.partitioned:
        L = ix.leaf_offsets
        sizes = np.diff(L)
        leaves, _ = ahlib.ah_partition_score(Qd, index.centroids, w.leaves_to_search)
        scanned_total = float(sizes[leaves.cpu().numpy()].sum())
    else:
        scanned_total = float(w.n) * Q.shape[0]
    lookups = scanned_total * w.blocks
    t_main = stage_ms["scan_main"] / 1e3
    ops = 32.0 * lookups  # 16 multiply-adds (one-hot over 16 centers) per table lookup
    achieved_tops = ops / t_main / 1e12
    elem = 4 if w.originals == "f32" else 2
    reorder_gbps = costs.reorder_bytes(Q.shape[0], w.reorder, w.d, elem) / (stage_ms["reorder"] / 1e3) / 1e9
    out = {
        "metric": METRIC,
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 scan (i32 accumulate), f32 table/reorder",
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "d": w.d, "nq": w.nq, "blocks": w.blocks,
                   "dims_per_block": w.dpb, "num_leaves": w.num_leaves, "leaves_to_search": w.leaves_to_search,
                   "reorder": w.reorder, "k": w.k, "originals": w.originals},
        "recall_at_10": rec,
        "stages_ms": stage_ms,
        "scan_lookups_per_s": lookups / t_main,
        "reorder_gather_GBps": reorder_gbps,
        "roofline": {"kernel": "scan_main_kernel", "bound": "mfma", "achieved": achieved_tops,
                     "peak": PEAK_INT8_TOPS, "unit": "TOP/s", "frac": achieved_tops / PEAK_INT8_TOPS,
                     "traffic": profiled_traffic(w.name)},
    }
    if not args.no_probe:
        out["code_scan_hbm"] = code_scan_probe(torch, ahlib, ev)
        out["stage_probes"] = stage_probes(torch, ahlib)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, ix, X, Q, gt, gpu_ids, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
