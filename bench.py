#!/usr/bin/env python3
"""Benchmark of the CSA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: CSA decode at 128K context, batch 32 (32768 compressed entries per
sequence, paged 64 per page under a random page table over 16384 pages;
FP8 index-K with Hadamard rotation, 64 indexer heads x 128; 64 attention
heads; top-512 plus a 128-token window). One step = the whole hot path for one
new token of every sequence: compress the block the token completes, append
the token to the raw window pool, prepare its index-K row, rotate + quantise
the indexer query, score every compressed entry, select the top 512 through
the page table, attend. Inputs are resident in HBM before timing; three
copies of the large pools rotate across steps so no step is served from the
last-level cache by its predecessor.

Prints one JSON line. `roofline` is for the dominant kernel (the indexer scan),
timed with HIP events on the launch stream; `cpu_baseline` is the plain CPU
oracle timed on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
# the scan kernel of the 128K decode step (FP8 index-K, 64-entry pages, the
# chunk top-512 selected on chip): the roofline kernel
DECODE_128K_SCAN = "indexer_mfma_kernel<false, true, true>"
SPIN_CYCLES = 2_000_000  # ~1 ms of GPU spin ahead of each eager timing step


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-queries", type=int, default=32)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the 1M decode, prefill and HCA workloads")
    ap.add_argument("--profile-only", choices=["decode_128k", "decode_1m", "spec_decode", "prefill", "hca_ragged", "copy"],
                    help="run only this workload's steps (eager, for a profiler) and print nothing else; "
                         "'copy' is a plain 1 GiB device copy that calibrates the HBM byte counters")
    ap.add_argument("--counters-from", metavar="DIR",
                    help="reduce rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv output of the decode_128k and "
                         "copy runs under DIR into profiles/counters.json, then exit (no GPU)")
    return ap.parse_args()


def kernel_source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "compressed_sparse_attention_c4_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, src_hash: str, launches_bytes_key="bytes_per_launch"):
    """HBM traffic per launch measured by rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy kernel), if taken on this exact kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(kernel)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get(launches_bytes_key)


COPY_BYTES = 4 << 28  # bytes read (and written) by one launch of the calibration copy


def _counter_means(csv_path, counter):
    """Mean value of `counter` per dispatch, by kernel name, from a rocprofv3
    counter_collection.csv."""
    import csv
    tot, cnt = {}, {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            k = r["Kernel_Name"]
            tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
            cnt[k] = cnt.get(k, 0) + 1
    return {k: (tot[k] / cnt[k], cnt[k]) for k in tot}


def _find_csv(d, stem):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", f"{stem}*counter_collection.csv"), recursive=True))
    if not hits:
        raise SystemExit(f"no {stem}*counter_collection.csv under {d}")
    return hits[-1]


def reduce_counters(d):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the decode indexer,
    scaled by what the same counters read for a copy of COPY_BYTES, written
    with the hash of the kernel source they were taken on."""
    out = {}
    cf = _counter_means(_find_csv(d, "copy_fetch"), "FETCH_SIZE")
    cw = _counter_means(_find_csv(d, "copy_write"), "WRITE_SIZE")
    copy_k = max(cf, key=lambda k: cf[k][0])  # the copy is the largest reader in its run
    f_scale = COPY_BYTES / (cf[copy_k][0] * 1024)
    w_scale = COPY_BYTES / (cw[copy_k][0] * 1024)
    kf = _counter_means(_find_csv(d, "decode128k_fetch"), "FETCH_SIZE")
    kw = _counter_means(_find_csv(d, "decode128k_write"), "WRITE_SIZE")
    name = DECODE_128K_SCAN
    hits = [k for k in kf if name in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one {name} in the fetch run, found {hits}")
    k = hits[0]
    fetch = kf[k][0] * 1024 * f_scale
    write = kw[k][0] * 1024 * w_scale
    out[name] = {"source_hash": kernel_source_hash("indexer.hip", "csa_device.hpp", "topk_select.hpp", "../build.py"),
                 "bytes_per_launch": round(fetch + write),
                 "fetch_bytes": round(fetch), "write_bytes": round(write),
                 "fetch_kib_raw": kf[k][0], "write_kib_raw": kw[k][0], "dispatches": kf[k][1],
                 "copy_kernel": copy_k, "copy_fetch_kib": cf[copy_k][0], "copy_write_kib": cw[copy_k][0],
                 "fetch_scale": f_scale, "write_scale": w_scale}
    path = os.path.join(ROOT, "profiles", "counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def capture_graphs(W, copies):
    """One HIP graph per pool copy, each holding a whole step (every launch of
    the library goes to the capturing stream; the step allocates nothing)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in range(copies):
            W.step(c)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for c in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            W.step(c)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_steps(W, steps, warmup, copies, graph=True):
    """(ms per step over the timed region, mean / median indexer kernel ms).
    The step time is taken over `steps` graph replays (or eager steps); the
    indexer kernel's duration from HIP events recorded around its launch on
    the launch stream during `steps` eager steps of the same work."""
    import torch
    for i in range(warmup):
        W.step(i % copies)
    torch.cuda.synchronize()
    graphs = capture_graphs(W, copies) if graph else None
    if graphs:
        for i in range(warmup):
            graphs[i % copies].replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        if graphs:
            graphs[i % copies].replay()
        else:
            W.step(i % copies)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    # the events' handles exist after a first record; made here, so that no
    # event is created on the stream in front of the kernel being timed
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(steps):
        # a spin ahead of the step keeps the GPU busy while the host queues the
        # step's launches, so the events bracket the kernel, not host gaps
        torch.cuda._sleep(SPIN_CYCLES)
        W.step(i % copies, evs[i])
    torch.cuda.synchronize()
    idx_ms = [a.elapsed_time(b) for a, b in evs]
    return ms, float(np.mean(idx_ms)), float(np.median(idx_ms))


def secondary(a):
    """The other workloads of the method, each timed the same way (graph
    replays for the step, HIP events around the indexer launch)."""
    import torch
    from workloads import specs
    from workloads.device import CsaDecode, CsaPrefill, CsaSpecDecode, HcaCsaRagged, hca_build_input
    import compressed_sparse_attention_c4_amd as csa
    out = {}
    steps = max(10, a.steps // 2)
    # decode at 1M context, batch 4, MXFP4 index-K, 128 heads
    wl = specs.DECODE_1M
    W = CsaDecode(wl, [wl.seq_len] * wl.batch, copies=a.copies, pool_pages=wl.pool_pages)
    ms, idx_ms, _ = time_steps(W, steps, a.warmup, a.copies, graph=not a.no_graph)
    gbs = W.indexer_bytes() / (idx_ms / 1e3) / 1e9
    out[wl.name] = {"queries_per_s": round(W.B / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
                    "indexer": {"kernel": W.indexer_kernel, "kernel_ms": round(idx_ms, 5),
                                "bytes_per_launch": W.indexer_bytes(), "achieved_GBs": round(gbs, 1),
                                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)},
                    "step_hbm_frac": round(W.step_bytes() / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    del W
    torch.cuda.empty_cache()
    # multi-token (speculative-verify) decode: 32 sequences x 4 query tokens at 128K
    wl = specs.SPEC_DECODE_128K
    W = CsaSpecDecode(wl, [wl.seq_len] * wl.batch, copies=a.copies, pool_pages=wl.pool_pages)
    ms, idx_ms, _ = time_steps(W, steps, a.warmup, a.copies, graph=not a.no_graph)
    gbs = W.indexer_bytes() / (idx_ms / 1e3) / 1e9
    out[wl.name] = {"queries_per_s": round(W.T / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
                    "indexer": {"kernel": W.indexer_kernel, "kernel_ms": round(idx_ms, 5),
                                "bytes_per_launch": W.indexer_bytes(), "achieved_GBs": round(gbs, 1),
                                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}}
    del W
    torch.cuda.empty_cache()
    # chunked prefill: 4096 new tokens on a 131072-token context
    wl = specs.PREFILL_4K
    W = CsaPrefill(wl)
    ms, idx_ms, _ = time_steps(W, max(5, steps // 4), 2, 1, graph=not a.no_graph)
    tf = W.indexer_flops() / (idx_ms / 1e3) / 1e12
    out[wl.name] = {"tokens_per_s": round(W.new / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
                    "indexer_gemm": {"kernel": "indexer_rows_kernel<false, 8>", "kernel_ms": round(idx_ms, 4),
                                     "flop_per_launch": W.indexer_flops(), "achieved_TFLOPs": round(tf, 1),
                                     "fp8_mfma_frac": round(tf / FP8_PEAK_TFLOPS, 4)}}
    del W
    torch.cuda.empty_cache()
    # HCA layer + CSA layer over 16 ragged sequences
    wl = specs.HCA_RAGGED
    W = HcaCsaRagged(wl, copies=a.copies)
    ms, idx_ms, _ = time_steps(W, steps, a.warmup, a.copies, graph=not a.no_graph)
    step_bytes = W.csa.step_bytes() + W.hca_bytes()
    out[wl.name] = {"queries_per_s": round(W.B / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
                    "raw_lengths": [int(x) for x in W.lens],
                    "step_hbm_frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    lens = W.lens
    del W
    torch.cuda.empty_cache()
    # HCA cache build (ratio 128 over every raw row)
    x, cu, st = hca_build_input(lens, wl.seed * 10 + 11)
    from workloads import gen
    gw, gb = gen.gate_params(gen.rng(wl.seed + 3), wl.hca_ratio)
    gw, gb = torch.from_numpy(gw).cuda(), torch.from_numpy(gb).cuda()
    hpages = [int(l) // wl.hca_ratio // 64 + 1 for l in lens]
    pool = csa.alloc_kv_pool(sum(hpages), 64, csa.CSA_FP8_E4M3)
    pt = np.zeros((len(lens), max(hpages)), np.int32)
    o = 0
    for b, k in enumerate(hpages):
        pt[b, :k] = np.arange(o, o + k)
        o += k
    ptd = torch.from_numpy(pt).cuda()
    args = (x, cu, st, int(max(lens)), wl.hca_ratio, gw, gb, ptd, pool)
    csa.c4_compress(*args)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        csa.c4_compress(*args)
    e1.record()
    torch.cuda.synchronize()
    bms = e0.elapsed_time(e1) / 3
    nbytes = x.numel() * 2 + int(np.sum(np.asarray(lens) // wl.hca_ratio)) * 644
    out["hca_cache_build_r128"] = {"raw_rows": int(np.sum(lens)), "ms": round(bms, 3),
                                   "GBs": round(nbytes / (bms / 1e3) / 1e9, 1),
                                   "hbm_frac": round(nbytes / (bms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    del x, pool
    torch.cuda.empty_cache()
    return out


def cpu_baseline(W, n_queries: int):
    """The oracle, as it stands, on n_queries of the same decode step: rotate +
    quantise the query, score all entries, top-512 through the page table,
    attend. The oracle's pools are quantised by the oracle from the same
    seeded raw draws (setup, not timed)."""
    import torch
    from oracle import csa_oracle as O
    from workloads import gen
    from workloads.device import _CHUNK
    from threadpoolctl import threadpool_info

    wl = W.wl
    seed = wl.seed * 10
    n_queries = min(n_queries, W.B)
    rows_needed = {}
    for b in range(n_queries):
        n = int(W.N[b])
        rows_needed[b] = O.page_slot(W.pt_host[b], np.arange(n), 64)
    all_rows = np.unique(np.concatenate(list(rows_needed.values())))

    def regen(rows, dim, seed_base):
        out = np.empty((len(rows), dim), np.float32)
        chunks = rows // _CHUNK
        for c in np.unique(chunks):
            sel = np.flatnonzero(chunks == c)
            n = min(_CHUNK, W.P * 64 - c * _CHUNK)
            v = gen.device_normal((n, dim), seed_base * 1000 + int(c))
            out[sel] = v[torch.as_tensor(rows[sel] - c * _CHUNK, device="cuda")].float().cpu().numpy()
        return out

    kraw = regen(all_rows, wl.index_dim, seed + 1)
    kvraw = regen(all_rows, 576, seed + 2)
    codes, sc = O.index_prep(kraw, wl.hadamard, wl.index_fmt)
    ipool_rows = {r: i for i, r in enumerate(all_rows)}
    lat, lsc, rope = O.quant_kv_entries(kvraw, "fp8")
    q_idx = W.q_idx[:n_queries].float().cpu().numpy()
    w_idx = W.w_idx[:n_queries].cpu().numpy()
    q_att = W.q_attn[:n_queries].float().cpu().numpy()
    # window rows: regenerate the raw tail draw
    tail = 2 * 256
    x = gen.device_normal((int(sum(np.minimum(W.lens, tail))), 576), seed + 3).float().cpu().numpy()
    raw_rows = O.quant_kv_entries(x, "fp8")
    cu = np.concatenate([[0], np.cumsum(np.minimum(W.lens, tail))])

    t0 = time.perf_counter()
    for b in range(n_queries):
        slots = rows_needed[b]
        loc = np.array([ipool_rows[s] for s in slots])
        n = len(slots)
        qc, qs = O.index_prep(q_idx[b], wl.hadamard, wl.index_fmt)
        qhat = O.index_dequant(qc, qs, wl.index_fmt)
        khat = O.index_dequant(codes[loc], sc[loc], wl.index_fmt)
        logits = O.indexer_logits(qhat, w_idx[b], khat)
        sel = O.topk_logical(logits, n)
        c4rows = O.dequant_kv_entries(lat[loc[sel]], lsc[loc[sel]], rope[loc[sel]], "fp8")
        p = int(W.lens[b]) - 1
        wpos = O.window_positions(p, wl.window) - (int(W.lens[b]) - min(int(W.lens[b]), tail))
        r0 = cu[b]
        rr = O.dequant_kv_entries(raw_rows[0][r0 + wpos], raw_rows[1][r0 + wpos], raw_rows[2][r0 + wpos], "fp8")
        O.csa_attention_query(q_att[b], c4rows, rr, wl.softmax_scale)
    dt = time.perf_counter() - t0
    threads = 1
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 1)))
    return {"value": n_queries / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_queries} of {W.B} decode queries at 128K (q prep, indexer over "
                      f"{int(W.N[0])} entries x 64 heads in float64, top-512, attention); "
                      f"{dt:.2f} s of CPU work"}


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if a.counters_from:
        reduce_counters(a.counters_from)
        return
    import torch
    from workloads import specs
    from workloads.device import CsaDecode

    torch.cuda.set_device(0)
    if a.profile_only:
        from workloads.device import CsaPrefill, HcaCsaRagged
        if a.profile_only == "decode_128k":
            wl = specs.DECODE_128K
            W = CsaDecode(wl, [wl.seq_len] * wl.batch, copies=a.copies, pool_pages=wl.pool_pages)
        elif a.profile_only == "decode_1m":
            wl = specs.DECODE_1M
            W = CsaDecode(wl, [wl.seq_len] * wl.batch, copies=a.copies, pool_pages=wl.pool_pages)
        elif a.profile_only == "spec_decode":
            from workloads.device import CsaSpecDecode
            wl = specs.SPEC_DECODE_128K
            W = CsaSpecDecode(wl, [wl.seq_len] * wl.batch, copies=a.copies, pool_pages=wl.pool_pages)
        elif a.profile_only == "copy":
            n = 1 << 28  # 1 GiB of float32 read and 1 GiB written per copy
            src = torch.ones(n, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(a.warmup + a.steps):
                dst.copy_(src)
            torch.cuda.synchronize()
            print(f"profiled copy: {a.warmup + a.steps} copies of {4 * n} B", flush=True)
            return
        elif a.profile_only == "prefill":
            W = CsaPrefill(specs.PREFILL_4K)
            a.copies = 1
        else:
            W = HcaCsaRagged(specs.HCA_RAGGED, copies=a.copies)
        for i in range(a.warmup + a.steps):
            W.step(i % a.copies)
        torch.cuda.synchronize()
        print(f"profiled {a.profile_only}: {a.warmup + a.steps} eager steps", flush=True)
        return
    wl = specs.DECODE_128K
    W = CsaDecode(wl, [wl.seq_len] * wl.batch, copies=a.copies, pool_pages=wl.pool_pages)
    ms, idx_ms, idx_med = time_steps(W, a.steps, a.warmup, a.copies, graph=not a.no_graph)
    qps = W.B / (ms / 1e3)
    ibytes = W.indexer_bytes()
    achieved = ibytes / (idx_ms / 1e3) / 1e9
    src_hash = kernel_source_hash("indexer.hip", "csa_device.hpp", "topk_select.hpp", "../build.py")
    assert W.indexer_kernel == DECODE_128K_SCAN, W.indexer_kernel
    traffic = stored_traffic(DECODE_128K_SCAN, src_hash)
    line = {
        "metric": "CSA decode queries/s @128K ctx",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": W.B, "seq_len": wl.seq_len,
                   "compressed_entries": int(W.N[0]), "index_format": "fp8_e4m3+hadamard",
                   "index_heads": wl.index_heads, "attn_heads": wl.heads, "topk": 512,
                   "window": wl.window, "pool_copies": a.copies, "hip_graph": not a.no_graph},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": DECODE_128K_SCAN,
                     "kernel_ms": round(idx_ms, 5), "bytes_per_launch": ibytes},
        "step_hbm_frac": round(W.step_bytes() / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W, a.cpu_queries)
        line["cpu_baseline"]["value"] = round(line["cpu_baseline"]["value"], 3)
    del W
    torch.cuda.empty_cache()
    if not a.no_secondary:
        line["secondary"] = secondary(a)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
