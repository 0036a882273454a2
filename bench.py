#!/usr/bin/env python3
"""Benchmark of the AH search path on one MI355X.

A step is one pass of the whole path over one query batch with every input
already resident in HBM: centroid scoring + leaf choice (partitioned workloads),
per-query int8 tables, code scan + top-R, exact reorder to the final k.

The headline (one JSON line) is the 20,000,000 x 384 workload (bf16 originals,
4,000 leaves with 200 searched, 192 blocks x 2 dims, eta = 4, 10,000 queries,
R = 300, k = 10): queries/s at the measured recall@10 over all queries, the main
scan kernel against its roofline (HIP events around that kernel), and the CPU
oracle timed on a bounded sample of the same queries on the same index.  The
index is built on the GPU at start-up (index.build_gpu), ground truth is exact
search over the stored rows (fp32 GPU shortlist re-ranked in float64).  The four
other workloads (tiny, sift1m, glove1m, openai2m) follow as extra keys with the
same measurements, then the code-scan HBM probe and the other rows' probes.

Usage: python bench.py [--steps K] [--warmup W] [--workload wiki20m] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "queries/sec at recall@10 (AH 4-bit scan + reorder); code-scan HBM GB/s"
HEADLINE = "wiki20m"
OTHERS = ("tiny", "sift1m", "glove1m", "openai2m")

# MI355X published peaks
PEAK_HBM_GBPS = 8000.0
PEAK_INT8_TOPS = 5000.0
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_FP64_TFLOPS = 78.6  # vector float64
# a table-gather scan's roof: one needed int8 entry per LDS byte returned,
# 256 CUs x 128 B/clock x 2.4 GHz
P_LDS_LOOKUPS = 256 * 128 * 2.4e9


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- HIP events
class HipEvents:
    """hipEvents recorded on an explicit stream (torch.cuda.Event only sees torch's current stream)."""

    def __init__(self):
        self.h = C.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.h.hipEventSynchronize.argtypes = [C.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]

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


def host_cpu():
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def recall(found, truth):
    hit = 0
    for f, t in zip(found, truth):
        hit += len(set(f[f >= 0].tolist()) & set(t.tolist()))
    return hit / truth.size


# ----------------------------------------------------------------------------- ground truth
def exact_topk_gpu(torch, base, Qd, k=10, shortlist=64, q_chunk=4096, r_chunk=1 << 20):
    """Exact top-k over the stored rows by float64 score, (score desc, id asc):
    a float32 shortlist of the best `shortlist` rows per query on the GPU, then
    the shortlist re-ranked in float64 (bf16 rows widen exactly)."""
    n = base.shape[0]
    out = []
    for qa in range(0, Qd.shape[0], q_chunk):
        Qc = Qd[qa:qa + q_chunk]
        best_s = best_i = None
        for ra in range(0, n, r_chunk):
            S = Qc @ base[ra:ra + r_chunk].to(torch.float32).T
            s, i = torch.topk(S, min(shortlist, S.shape[1]), dim=1)
            i = i + ra
            if best_s is not None:
                s, j = torch.topk(torch.cat([best_s, s], 1), min(shortlist, best_s.shape[1] + s.shape[1]), dim=1)
                i = torch.cat([best_i, i], 1).gather(1, j)
            best_s, best_i = s, i
            del S
        rows = base[best_i].to(torch.float64)
        ex = (rows * Qc.to(torch.float64)[:, None, :]).sum(-1)
        ids_sorted, perm = torch.sort(best_i, dim=1)
        _, p2 = torch.sort(-ex.gather(1, perm), dim=1, stable=True)
        out.append(ids_sorted.gather(1, p2)[:, :k].to(torch.int32).cpu())
        del rows, ex
    return torch.cat(out).numpy()


# ----------------------------------------------------------------------------- one workload
def make_inputs(w, torch):
    """(base rows on the GPU, the same rows on the host or None, queries on the host)."""
    Q = synth.queries(w)
    if w.n * w.d <= 200_000_000 and w.originals == "f32":
        X = synth.database(w)
        return torch.from_numpy(X).cuda(), X, Q
    return synth.gpu_database(torch, w), None, Q


def build_index(w, base, X, torch, timings):
    from mips_ah_partition_amd import index as ixm
    from mips_ah_partition_amd.search import AHIndex
    seed = 1000 * w.index + synth.ROLE_CODEBOOK
    if w.name == "tiny":
        # the tiny workload's codebooks come from k-means iterations on the host
        t0 = time.perf_counter()
        hix = ixm.build(X, w.dpb, w.eta, num_leaves=w.num_leaves, seed=seed)
        timings["host_build"] = time.perf_counter() - t0
        return AHIndex(hix, X, num_leaves_to_search=w.leaves_to_search, reorder=w.reorder,
                       final_num_neighbors=w.k), hix
    dix = ixm.build_gpu(base, w.dpb, w.eta, num_leaves=w.num_leaves, seed=seed, timings=timings)
    return AHIndex.from_device(dix, base, num_leaves_to_search=w.leaves_to_search, reorder=w.reorder,
                               final_num_neighbors=w.k), dix


def timed_steps(torch, index, Qd, steps, warmup, ev):
    """Wall time per step (inputs resident) and per-stage HIP-event means."""
    sh = torch.cuda.current_stream().cuda_stream
    stages = ["lut", "scan", "reorder"] + (["partition"] if index.partitioned else [])
    evs = {s: [(ev.create(), ev.create()) for _ in range(steps)] for s in stages + ["scan_main"]}

    def timers(i):
        t = {s: (lambda e=evs[s][i][0]: ev.record(e, sh), lambda e=evs[s][i][1]: ev.record(e, sh)) for s in stages}
        t["scan_main"] = evs["scan_main"][i]
        return t

    for _ in range(warmup):
        ids, scores = index.search_batched(Qd)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ids, scores = index.search_batched(Qd, timers=timers(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {s: float(np.mean([ev.elapsed_ms(*evs[s][i]) for i in range(steps)])) for s in evs}
    return wall / steps * 1e3, stage_ms, ids


def pcie_steps(torch, index, Q, k, steps):
    """Per-step time including the query upload from pinned host memory and the
    download of the results (ids and scores) to pinned host memory."""
    Qp = torch.from_numpy(Q).pin_memory()
    ids_h = torch.empty((Q.shape[0], k), dtype=torch.int32).pin_memory()
    sc_h = torch.empty((Q.shape[0], k), dtype=torch.float32).pin_memory()
    Qd = torch.empty(Q.shape, dtype=torch.float32, device="cuda")
    for _ in range(2):
        Qd.copy_(Qp, non_blocking=True)
        ids, sc = index.search_batched(Qd)
        ids_h.copy_(ids, non_blocking=True)
        sc_h.copy_(sc, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        Qd.copy_(Qp, non_blocking=True)
        ids, sc = index.search_batched(Qd)
        ids_h.copy_(ids, non_blocking=True)
        sc_h.copy_(sc, non_blocking=True)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def oracle_leg(w, hix, base_host, Q, gt, gpu_ids, budget_s, threads):
    """The oracle as it stands (whole path: leaves, table, scan, top-R, reorder),
    on the first queries of the batch, sized to about budget_s seconds with
    `threads` OpenMP threads."""
    import oracle
    oracle.set_threads(threads)
    kw = dict(centroids=hix.centroids, leaf_offsets=hix.leaf_offsets, ids=hix.ids, nl=w.leaves_to_search)
    cal = max(1, min(threads, Q.shape[0]))
    t0 = time.perf_counter()
    oracle.search(Q[:cal], hix.codebooks, hix.codes, base_host, w.reorder, w.k, **kw)
    per_q = (time.perf_counter() - t0) / cal * threads
    ns = int(min(Q.shape[0], max(cal, budget_s / max(per_q, 1e-9) * threads)))
    t0 = time.perf_counter()
    res = oracle.search(Q[:ns], hix.codebooks, hix.codes, base_host, w.reorder, w.k, **kw)
    dt = time.perf_counter() - t0
    return {
        "value": ns / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
        "sample": f"first {ns} of {Q.shape[0]} queries, whole path (leaves, table, scan, top-{w.reorder}, reorder)",
        "seconds": dt,
        "recall_at_10": recall(res["ids"], gt[:ns]),
        "gpu_recall_at_10_same_sample": recall(gpu_ids[:ns], gt[:ns]),
        "final_ids_equal_fraction": float((res["ids"] == gpu_ids[:ns]).all(axis=1).mean()),
    }


def profiled_traffic(workload):
    """HBM bytes per launch of the main scan kernel from the committed rocprofv3
    summary (profiles/scan_main_<workload>.txt), or None when the kernel source
    has changed since the counters were taken."""
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
    if fields.get("kernel_source", "").split()[-1:] != [sha] or "scan_main_traffic_bytes" not in fields:
        return None
    return float(fields["scan_main_traffic_bytes"])


def run_workload(w, torch, ev, steps, warmup, cpu_budget, one_core_budget, cores):
    from mips_ah_partition_amd import ahlib
    t_all = time.perf_counter()
    log(f"[bench] {w.name}: generating {w.n} x {w.d} rows ...")
    base, X, Q = make_inputs(w, torch)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_all
    build_t = {}
    log(f"[bench] {w.name}: building the index ...")
    index, ix = build_index(w, base, X, torch, build_t)
    torch.cuda.synchronize()
    Qd = torch.from_numpy(Q).cuda()
    log(f"[bench] {w.name}: exact ground truth ...")
    t0 = time.perf_counter()
    gt = exact_topk_gpu(torch, base, Qd, w.k)
    t_gt = time.perf_counter() - t0
    log(f"[bench] {w.name}: timed steps ...")
    ms_step, stage_ms, ids = timed_steps(torch, index, Qd, steps, warmup, ev)
    gpu_ids = ids.cpu().numpy()
    rec = recall(gpu_ids, gt)
    ms_pcie = pcie_steps(torch, index, Q, w.k, max(3, steps // 4))
    B = w.blocks
    n = w.n
    if index.partitioned:
        leaves, _ = ahlib.ah_partition_score(Qd, index.centroids, w.leaves_to_search)
        sizes = np.diff(index.leaf_offsets.cpu().numpy())
        scanned_total = float(sizes[leaves.cpu().numpy()].sum())
        L, nl = w.num_leaves, w.leaves_to_search
    else:
        scanned_total = float(n) * Q.shape[0]
        L = nl = 0
    index.search_batched(Qd)
    appended, overflowed = ahlib.scan_counters(index._ws["scan"], Q.shape[0], B, n, L, nl, w.reorder)
    lookups = scanned_total * B
    t_main = stage_ms["scan_main"] / 1e3
    elem = 4 if w.originals == "f32" else 2
    res = {
        "workload": w.name, "n": n, "d": w.d, "nq": Q.shape[0], "blocks": B, "dims_per_block": w.dpb,
        "num_leaves": w.num_leaves, "leaves_to_search": w.leaves_to_search, "reorder": w.reorder, "k": w.k,
        "originals": w.originals, "eta": w.eta,
        "queries_per_s": Q.shape[0] / (ms_step / 1e3), "ms_per_step": ms_step,
        "queries_per_s_with_pcie": Q.shape[0] / (ms_pcie / 1e3), "ms_per_step_with_pcie": ms_pcie,
        "recall_at_10": rec, "stages_ms": stage_ms,
        "scanned_rows_per_query": scanned_total / Q.shape[0],
        "scan_lookups_per_s": lookups / t_main,
        "candidates_appended_per_query": float(appended.mean()),
        "overflowed_queries": overflowed,
        "reorder_gather_GBps": Q.shape[0] * w.reorder * w.d * elem / (stage_ms["reorder"] / 1e3) / 1e9,
        "setup_s": {"generate": t_gen, "index": build_t, "ground_truth": t_gt},
    }
    if index.partitioned:
        res["partition_TFLOPs"] = 2.0 * Q.shape[0] * w.num_leaves * w.d / (stage_ms["partition"] / 1e3) / 1e12
    if "partition_assign" in build_t:
        res["index_rates"] = {
            "assign_TFLOPs": 2.0 * n * w.num_leaves * w.d / build_t["partition_assign"] / 1e12,
            "encode_rows_per_s": n / build_t["encode"],
        }
    # the oracle needs the index and the stored rows on the host
    res["_cpu"] = None
    hix = base_host = None
    if cpu_budget > 0:
        log(f"[bench] {w.name}: oracle sample ...")
        hix = ix if w.name == "tiny" else ix.to_host()
        if X is not None:
            base_host = X
        else:
            base_host = base.view(torch.int16).cpu().numpy().view(np.uint16)
        res["_cpu"] = oracle_leg(w, hix, base_host, Q, gt, gpu_ids, cpu_budget, cores)
        if one_core_budget > 0:
            one = oracle_leg(w, hix, base_host, Q, gt, gpu_ids, one_core_budget, 1)
            res["_cpu"]["one_core_queries_per_s"] = one["value"]
            res["_cpu"]["one_core_sample"] = one["sample"]
    res["_lookups"] = lookups
    res["_t_main"] = t_main
    res["_code_bytes"] = n * w.code_bytes
    res["wall_s"] = time.perf_counter() - t_all
    del index, ix, base, X, Qd, hix, base_host
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- code-scan HBM probe
# Single-pass streaming scans at low reuse: 1 and 4 queries over codes of the
# 20M x 384-dim (192 blocks, 96 B rows) and 2M x 1536-dim (768 blocks, 384 B
# rows) shapes, no partitioning.  Both code arrays exceed the 256 MB last-level
# cache, so every run reads them from HBM.  Codes are uniform random nibbles
# generated on the GPU (seeded); tables are uniform int8.  The plain-stream read
# of the same bytes (ah_hbm_read_probe) is the measured reference.
PROBE_SHAPES = (("wiki20m", 20_000_000, 192, 300), ("openai2m", 2_000_000, 768, 400))


def code_scan_probe(torch, ahlib, ev, runs=5):
    out = {}
    sh = torch.cuda.current_stream().cuda_stream
    for name, n, B, R in PROBE_SHAPES:
        g = torch.Generator(device="cuda")
        g.manual_seed(4242 + B)
        codes = torch.randint(0, 256, (n, (B + 1) // 2), generator=g, device="cuda", dtype=torch.uint8)
        tiled = ahlib.ah_tile_codes(codes, B)
        # plain-stream read of the same bytes, several launch widths; the best is the reference
        e0, e1 = ev.create(), ev.create()
        c0, c1 = ev.create(), ev.create()  # around the whole top-R call (warm-up, scan, selection)
        best = 0.0
        for bpc in (2, 4, 8, 16):
            ts = []
            for it in range(runs + 1):
                ev.record(e0, sh)
                ahlib.ah_hbm_read_probe(codes, blocks_per_cu=bpc)
                ev.record(e1, sh)
                if it:
                    ts.append(ev.elapsed_ms(e0, e1))
            best = max(best, codes.numel() / (float(np.median(ts)) / 1e3) / 1e9)
        out[f"{name}_plain_read"] = {"bytes": int(codes.numel()), "GBps": best, "frac_of_8TBps": best / PEAK_HBM_GBPS}
        for nq in (1, 4):
            lut = torch.randint(-127, 128, (nq, B, 16), generator=g, device="cuda", dtype=torch.int8)
            ws = torch.empty(ahlib.ah_scan_workspace_bytes(nq, B, n, 0, 0, R), dtype=torch.uint8, device="cuda")
            for layout, src in (("", tiled), ("_rowmajor", codes)):
                ts, tc = [], []
                for it in range(runs + 1):
                    ev.record(c0, sh)
                    ahlib.ah_scan_topk(lut, src, R, workspace=ws, main_events=(e0, e1))
                    ev.record(c1, sh)
                    torch.cuda.synchronize()
                    if it:
                        ts.append(ev.elapsed_ms(e0, e1))
                        tc.append(ev.elapsed_ms(c0, c1))
                ms = float(np.median(ts))
                gbps = codes.numel() / (ms / 1e3) / 1e9
                appended, _ = ahlib.scan_counters(ws, nq, B, n, 0, 0, R)
                out[f"{name}_q{nq}{layout}"] = {"code_bytes": int(codes.numel()), "blocks": B, "queries": nq,
                                                "layout": "tiled" if not layout else "row-major",
                                                "scan_ms": ms, "GBps": gbps, "frac_of_8TBps": gbps / PEAK_HBM_GBPS,
                                                "frac_of_plain_read": gbps / best,
                                                "candidates_per_query": float(appended.mean()),
                                                "call_ms": float(np.median(tc))}
            del ws
        del codes, tiled
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- other rows' probes
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
    """The residual variant against raw codes, the int8 flat search, the
    training-free rotation quantiser, and the bf16 reorder on random (uncached)
    candidates."""
    out = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(5151)
    # residual (leaf-relative) codes against raw codes at equal bytes: 100,000 rows of the
    # 1M x 100 mixture workload, 600 leaves (30 searched), 50 blocks x 2 dims, R = 50, k = 10,
    # 1,000 queries; indexes trained on the host, the search on the GPU
    from mips_ah_partition_amd import index as hix
    from mips_ah_partition_amd.search import AHIndex
    w = synth.WORKLOADS["glove1m"]
    Xr = synth.database(w, 100_000)
    Qr = synth.queries(w, 1000)
    Xrd = torch.from_numpy(Xr).cuda()
    Qrd = torch.from_numpy(Qr).cuda()
    gt_r = exact_topk_gpu(torch, Xrd, Qrd, 10)
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
    del Xrd, Qrd
    # int8 flat search: 1M documents x 512 dims, 10,000 queries, R = 100, then the exact
    # fp32 rescore to k = 10; the contraction is int8 MFMA (2 nq n d ops)
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
    gt_v = exact_topk_gpu(torch, Dv, Qv, 10)
    f_ids, _ = ahlib.ah_reorder_exact(Qv, Dv, ids, 10)
    sq8_recall = recall(f_ids.cpu().numpy(), gt_v)
    sq8_recall_cand = recall(ids[:, :10].cpu().numpy(), gt_v)
    # the training-free rotation quantiser on the same corpus: 4-bit codes, the same
    # int8 matrix-core scan reading them, the same rescore
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
                                "scan_frac_of_int8_peak": ops / (ms_s / 1e3) / 1e12 / PEAK_INT8_TOPS}
    del Dv, Qv, d8, wss
    torch.cuda.empty_cache()
    # bf16 reorder at the 2M x 1536 shape on random candidates (rows spread over 6 GB,
    # so the gather reads HBM): 1,000 queries x 400 candidates
    w = synth.WORKLOADS["openai2m"]
    base = torch.randn((w.n, w.d), generator=g, device="cuda").to(torch.bfloat16)
    Q = torch.randn((w.nq, w.d), generator=g, device="cuda")
    cand = torch.randint(0, w.n, (w.nq, w.reorder), generator=g, device="cuda", dtype=torch.int32)
    ms = _time_ms(torch, lambda: ahlib.ah_reorder_exact(Q, base, cand, w.k))
    byt = w.nq * w.reorder * w.d * 2
    out["a5_reorder_bf16_openai2m_random"] = {"nq": w.nq, "R": w.reorder, "d": w.d, "ms": ms,
                                              "GBps": byt / (ms / 1e3) / 1e9,
                                              "frac_of_8TBps": byt / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS}
    del base
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--others", default=",".join(OTHERS),
                    help="comma-separated workloads measured after the headline ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work on the headline")
    ap.add_argument("--other-cpu-budget", type=float, default=6.0, help="seconds of oracle work per other workload")
    ap.add_argument("--no-probe", action="store_true", help="skip the code-scan HBM probe and the other rows' probes")
    ap.add_argument("--probe-only", action="store_true", help="only run the code-scan HBM probe")
    ap.add_argument("--stages-only", action="store_true", help="only run the other rows' probes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device 5 times (calibrates FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the search runs on one GPU only; --gpus must be 1 "
                                   "(sharding across GPUs is not implemented)"}))
        sys.exit(2)

    import torch
    from mips_ah_partition_amd import ahlib
    ahlib.lib()
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": src.numel() * 4, "launches": 5}))
        return
    ev = HipEvents()
    if args.stages_only:
        print(json.dumps({"stage_probes": stage_probes(torch, ahlib)}), flush=True)
        return
    if args.probe_only:
        print(json.dumps({"code_scan_hbm": code_scan_probe(torch, ahlib, ev)}), flush=True)
        return

    cores, model = host_cpu()
    w = synth.WORKLOADS[args.workload]
    cpu_budget = 0.0 if args.no_cpu_baseline else args.cpu_budget
    # the code-scan probe first, on a fresh allocator (after the workloads'
    # tens of GB come and go its plain read and scans measured a few % lower)
    probe = None if args.no_probe else code_scan_probe(torch, ahlib, ev)
    torch.cuda.empty_cache()
    r = run_workload(w, torch, ev, args.steps, args.warmup, cpu_budget, 0.0, cores)
    lookups, t_main, code_bytes = r.pop("_lookups"), r.pop("_t_main"), r.pop("_code_bytes")
    cpu = r.pop("_cpu")
    achieved = 2.0 * lookups / t_main / 1e12
    out = {
        "metric": METRIC,
        "value": r["queries_per_s"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 scan (i32 accumulate), f32 table/partition/reorder",
        "data": "synthetic",
        "config": {k: r[k] for k in ("workload", "n", "d", "nq", "blocks", "dims_per_block", "num_leaves",
                                     "leaves_to_search", "reorder", "k", "originals", "eta")},
        "recall_at_10": r["recall_at_10"],
        "roofline": {
            "kernel": "scan_main_kernel", "bound": "mfma", "unit": "TOP/s",
            "achieved": achieved, "peak": PEAK_INT8_TOPS, "frac": achieved / PEAK_INT8_TOPS,
            "traffic": profiled_traffic(w.name),
            "work_per_unit": "2 int8 ops (one table lookup, one int32 add) per (query, scanned row, block)",
            "units_per_launch": lookups,
            "kernel_ms": t_main * 1e3,
            # the one-hot contraction on the 2:4 sparse int8 matrix instruction:
            # one instruction (16 rows x 16 queries x 8 blocks of 16 centers)
            # does 2048 lookups in the time of a dense 16x16x64 int8 product,
            # so at the dense peak rate of such instructions the method's ops
            # reach 2 x 2048 / (16 x 16 x 64 x 2) = 1/8 of the dense int8 peak
            "design_ceiling_frac": 1.0 / 8.0,
            "frac_of_design_ceiling": achieved / PEAK_INT8_TOPS * 8.0,
            "lookups_per_s": lookups / t_main,
            "lookups_frac_of_lds_gather_roof": lookups / t_main / P_LDS_LOOKUPS,
            "unique_code_bytes_GBps": code_bytes / t_main / 1e9,
        },
        "host_cpu": {"cores": cores, "model": model},
        "headline": r,
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps({"progress": "headline done", "value": out["value"], "recall_at_10": out["recall_at_10"]}),
          file=sys.stderr, flush=True)
    others = {}
    for name in [s for s in args.others.split(",") if s and s != w.name]:
        wo = synth.WORKLOADS[name]
        one = min(3.0, args.other_cpu_budget) if wo.n <= 1_000_000 and cpu_budget > 0 else 0.0
        ro = run_workload(wo, torch, ev, max(5, args.steps // 2), args.warmup,
                          args.other_cpu_budget if cpu_budget > 0 else 0.0, one, cores)
        ro.pop("_lookups"), ro.pop("_t_main"), ro.pop("_code_bytes")
        ro["oracle"] = ro.pop("_cpu")
        others[name] = ro
        orc = ro["oracle"]
        log(f"[bench] {name}: {ro['queries_per_s']:.0f} q/s, recall@10 {ro['recall_at_10']:.4f}"
            + (f" (oracle {orc['recall_at_10']:.4f} on {orc['sample']})" if orc else ""))
    if others:
        out["other_workloads"] = others
    if not args.no_probe:
        out["code_scan_hbm"] = probe
        out["stage_probes"] = stage_probes(torch, ahlib)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
