#!/usr/bin/env python3
"""Benchmark of the CSA / HCA step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: CSA decode at 128K context, batch 32 (32768 compressed
entries per sequence, paged 64 per page under a random page table over 16384
pages; FP8 index-K with Hadamard rotation, 64 indexer heads x 128; 64
attention heads; top-512 plus a 128-token window). One step = the whole hot
path for one new token of every sequence: compress the block the token
completes, append the token to the raw window pool, prepare its index-K row,
rotate + quantise the indexer query, score every compressed entry, select the
top 512 through the page table, attend.

Secondary lines (`secondary` in the same JSON line), each measured the same
way and each with its own roofline and CPU-oracle baseline: the tiny fp32
decode (latency), decode at 1M context (MXFP4 index-K), multi-token decode at
128K, chunked prefill of 4096 tokens on 128K, the ragged HCA + CSA step, and
the HCA cache build.

Inputs are resident in HBM before timing. Enough copies of the large pools
rotate across steps that a pool is re-read only after more than 1.5x the 256 MB
last-level cache has been streamed, so no step is served from the cache by an
earlier one. Steps are captured into HIP graphs and replayed.

Prints one JSON line. `roofline` is for the dominant kernel of the workload
(the indexer scan), its duration measured with HIP events on the launch stream;
`cpu_baseline` is the plain CPU oracle timed on a bounded sample of the same
step on this host.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0    # dense FP8 matrix peak
BF16_PEAK_TFLOPS = 2500.0   # dense BF16 matrix peak
LLC_BYTES = 256 << 20       # MI355X last-level (Infinity) cache
SPIN_CYCLES = 2_000_000     # ~1 ms of GPU spin ahead of each eager timing step
SIMD_COUNT = 256 * 4        # SIMDs on the chip (MFMA busy normalisation)
XCD_COUNT = 8               # GRBM_GUI_ACTIVE reads as the sum over the XCDs' clocks
COPY_BYTES = 4 << 28        # bytes read (and written) by one launch of the calibration copy
PROFILE_GAP_S = 1.0         # idle gap between setup and the profiled steps
KERNEL_SOURCES = ("indexer.hip", "csa_device.hpp", "topk_select.hpp", "wave_topk.hpp", "../build.py")

PROFILE_CHOICES = ["tiny", "decode_128k", "decode_1m", "spec_decode", "prefill", "hca_ragged", "copy"]


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=0,
                    help="pool copies rotated across steps (0: enough for a 1.5x LLC reuse distance)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="only the headline (128K decode) workload")
    ap.add_argument("--profile-only", choices=PROFILE_CHOICES,
                    help="run only this workload's steps (eager, for a profiler) and print nothing else; "
                         "'copy' is a plain 1 GiB device copy that calibrates the HBM byte counters")
    ap.add_argument("--counters-from", metavar="DIR",
                    help="reduce rocprofv3 --pmc csv output under DIR (FETCH_SIZE / WRITE_SIZE runs of "
                         "the copy and the decode workloads, MFMA counters of the prefill) into "
                         "profiles/counters.json, then exit (no GPU)")
    ap.add_argument("--trace-from", metavar="DIR",
                    help="reduce a rocprofv3 --kernel-trace csv under DIR into a per-step kernel table "
                         "(printed), then exit (no GPU)")
    ap.add_argument("--trace-steps", type=int, default=0, help="eager steps in the traced run")
    return ap.parse_args()


# ---------------------------------------------------------------- profiles


def kernel_source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "compressed_sparse_attention_c4_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_counters(kernel: str):
    """Counter figures of `kernel` from profiles/counters.json if they were
    taken on the current kernel source, else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash(*KERNEL_SOURCES):
        return None
    return e


def _counter_means(csv_path, counter):
    """Mean value of `counter` per dispatch, by kernel name, from a rocprofv3
    counter_collection.csv."""
    tot, cnt = {}, {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            k = r["Kernel_Name"]
            tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
            cnt[k] = cnt.get(k, 0) + 1
    return {k: (tot[k] / cnt[k], cnt[k]) for k in tot}


def _find_csv(d, stem, kind="counter_collection"):
    hits = sorted(glob.glob(os.path.join(d, "**", f"{stem}*{kind}.csv"), recursive=True))
    return hits[-1] if hits else None


def _one_kernel(means, name):
    hits = [k for k in means if name in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one {name} in the counter run, found {hits}")
    return means[hits[0]]


# kernels whose HBM bytes are taken from FETCH_SIZE / WRITE_SIZE runs: stem -> kernel
COUNTER_KERNELS = {
    "decode128k": "indexer_mfma_kernel<false, true, true>",
    "decode1m": "indexer_mfma_kernel<true, true, true>",
    "prefill": "indexer_rows_kernel<false, 8, true>",
    "spec": "indexer_rows_kernel<false, 4, false>",
    "ragged": "indexer_wide_kernel<false>",
}


def reduce_counters(d):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each roofline kernel,
    scaled by what the same counters read for a copy of COPY_BYTES, and the
    prefill indexer's MFMA counters, written with the hash of the kernel
    source they were taken on."""
    out = {}
    path = os.path.join(ROOT, "profiles", "counters.json")
    if os.path.exists(path):
        with open(path) as f:
            out = json.load(f)
    src = kernel_source_hash(*KERNEL_SOURCES)
    cf = _counter_means(_find_csv(d, "copy_fetch"), "FETCH_SIZE")
    cw = _counter_means(_find_csv(d, "copy_write"), "WRITE_SIZE")
    copy_k = max(cf, key=lambda k: cf[k][0])  # the copy is the largest reader in its run
    f_scale = COPY_BYTES / (cf[copy_k][0] * 1024)
    w_scale = COPY_BYTES / (cw[copy_k][0] * 1024)
    for stem, name in COUNTER_KERNELS.items():
        ff, fw = _find_csv(d, f"{stem}_fetch"), _find_csv(d, f"{stem}_write")
        if not ff or not fw:
            continue
        kf = _one_kernel(_counter_means(ff, "FETCH_SIZE"), name)
        kw = _one_kernel(_counter_means(fw, "WRITE_SIZE"), name)
        fetch, write = kf[0] * 1024 * f_scale, kw[0] * 1024 * w_scale
        e = out.get(name, {}) if out.get(name, {}).get("source_hash") == src else {}
        e.update({"source_hash": src, "bytes_per_launch": round(fetch + write),
                  "fetch_bytes": round(fetch), "write_bytes": round(write),
                  "fetch_kib_raw": kf[0], "write_kib_raw": kw[0], "dispatches": kf[1],
                  "copy_kernel": copy_k, "copy_fetch_kib": cf[copy_k][0],
                  "copy_write_kib": cw[copy_k][0], "fetch_scale": f_scale, "write_scale": w_scale})
        out[name] = e
    fm = _find_csv(d, "prefill_mfma")
    if fm:
        name = COUNTER_KERNELS["prefill"]
        mops = _one_kernel(_counter_means(fm, "SQ_INSTS_VALU_MFMA_MOPS_F8"), name)
        busy = _one_kernel(_counter_means(fm, "SQ_VALU_MFMA_BUSY_CYCLES"), name)
        gui = _one_kernel(_counter_means(fm, "GRBM_GUI_ACTIVE"), name)
        e = out.get(name, {}) if out.get(name, {}).get("source_hash") == src else {}
        e.update({"source_hash": src, "mfma_f8_flops": mops[0] * 512,
                  "mfma_busy_cycles": busy[0], "gui_active_cycles": gui[0],
                  # busy cycles summed over the SIMDs, against the kernel's
                  # active cycles on one XCD times the SIMD count
                  "mfma_busy_frac": busy[0] / (gui[0] / XCD_COUNT * SIMD_COUNT),
                  "mfma_dispatches": mops[1]})
        out[name] = e
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def reduce_trace(d, steps):
    """Per-step kernel table of a --profile-only run traced with
    rocprofv3 --kernel-trace: the dispatches after the run's idle gap between
    setup and the steps, grouped by kernel."""
    path = _find_csv(d, "", "kernel_trace")
    if not path:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    start = 0
    for i in range(1, len(rows)):
        if rows[i][0] - rows[i - 1][1] > PROFILE_GAP_S * 0.5e9:
            start = i
    rows = rows[start:]
    by = {}
    for s, e, k in rows:
        by.setdefault(k, []).append((e - s) / 1e3)
    print(f"# kernel                                                     per_step    avg_us    min_us    max_us   us/step")
    tot = 0.0
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        short = k.replace("(anonymous namespace)::", "").replace("csa::", "").replace("void ", "")
        short = short.split("(")[0]
        per = len(v) / steps if steps else float("nan")
        us = sum(v) / steps if steps else float("nan")
        tot += us
        print(f"  {short:<58s} {per:8.0f} {np.mean(v):9.2f} {np.min(v):9.2f} {np.max(v):9.2f} {us:9.2f}")
    wall = (rows[-1][1] - rows[0][0]) / 1e3 / steps if steps else float("nan")
    print(f"# kernel time per step {tot:.1f} us; eager wall time per step {wall:.1f} us "
          f"(the timed bench step replays a HIP graph of the same launches)")


# ---------------------------------------------------------------- timing


def auto_copies(bytes_per_copy: int, override: int) -> int:
    """Pool copies so that a copy is re-read only after 1.5x the LLC has been
    streamed from the others."""
    if override:
        return override
    return max(3, math.ceil(1.5 * LLC_BYTES / max(bytes_per_copy, 1)) + 1)


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
    """(ms per step over the timed region, mean / median roofline-kernel ms,
    per-step percentiles). The step time is taken over `steps` graph replays
    (or eager steps); the percentiles (p10 / p50 / p90, ms) over as many
    replays after it, each bracketed by its own events behind a GPU spin; the
    roofline kernel's duration from HIP events recorded around its launch on
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
    # per-step times: a spin ahead of each step lets the host queue it before
    # the GPU reaches its first event
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in sev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(steps):
        torch.cuda._sleep(SPIN_CYCLES)
        sev[i][0].record()
        if graphs:
            graphs[i % copies].replay()
        else:
            W.step(i % copies)
        sev[i][1].record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in sev])
    dist = {f"p{q}": round(float(np.percentile(per, q)), 5) for q in (10, 50, 90)}
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
    k_ms = [a.elapsed_time(b) for a, b in evs]
    del graphs
    return ms, float(np.mean(k_ms)), float(np.median(k_ms)), dist


def hbm_roofline(kernel, nbytes, k_ms):
    gbs = nbytes / (k_ms / 1e3) / 1e9
    c = stored_counters(kernel)
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": None if not c or "bytes_per_launch" not in c else c["bytes_per_launch"],
            "kernel": kernel, "kernel_ms": round(k_ms, 5), "bytes_per_launch": int(nbytes)}


# ---------------------------------------------------------------- CPU oracle baseline


def cpu_info():
    """Threads the oracle's numpy BLAS uses (capped by this process's CPU
    affinity), the affinity size and the CPU model."""
    from threadpoolctl import threadpool_info
    aff = len(os.sched_getaffinity(0))
    blas = 1
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            blas = max(blas, int(info.get("num_threads", 1)))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cores": min(blas, aff), "affinity_cpus": aff, "cpu_model": model}


def _cpu_line(n, dt, unit, sample):
    d = {"value": round(n / dt, 3), "unit": unit, "kind": "oracle", "sample": sample + f"; {dt:.2f} s of CPU work"}
    d.update(cpu_info())
    return d


def cpu_decode_rows(states, unit, what, min_s=0.0):
    """The oracle's whole step (query preparation, indexer over every visible
    entry in float64, top-512, attention) for each prepared row state, in
    whole passes over the states until at least `min_s` seconds have run; the
    states (the oracle's pools, rebuilt from the seeded draws) are untimed
    setup."""
    passes = 0
    t0 = time.perf_counter()
    while True:
        for st in states:
            st.oracle_query()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            break
    if passes > 1:
        what += f", {passes} passes"
    return _cpu_line(passes * len(states), dt, unit, what)


def cpu_baseline_decode(W, seqs, min_s=0.0):
    from tests import fullsize as F
    states = [F.decode_seq(W, b, bands=False) for b in seqs]
    n = int(W.N[seqs[0]])
    return cpu_decode_rows(states, "queries/s",
                           f"{len(seqs)} of {W.B} decode queries ({n} entries x {W.wl.index_heads} index heads "
                           f"in float64, top-512, attention over 512 + {W.wl.window} entries x {W.H} heads)",
                           min_s)


def cpu_baseline_spec(W, rows):
    from tests import fullsize as F
    states = [F.spec_decode_row(W, t, bands=False) for t in rows]
    return cpu_decode_rows(states, "queries/s",
                           f"{len(rows)} of {W.T} query rows of the multi-token decode (each row's indexer, "
                           f"top-512 and attention)")


def cpu_baseline_prefill(W, rows):
    from tests import fullsize as F
    states = [F.prefill_row(W, t, bands=False) for t in rows]
    return cpu_decode_rows(states, "tokens/s",
                           f"{len(rows)} of {W.new} query rows of the chunk, spread over it (causal "
                           f"indexer, top-512, attention per row; the chunk's compression not timed)")


def cpu_baseline_hca(Wh, seqs):
    from tests import fullsize as F
    hs = [F.hca_state(Wh, b) for b in seqs]
    cs = [F.decode_seq(Wh.csa, b, bands=False) for b in seqs]
    t0 = time.perf_counter()
    for h, st in zip(hs, cs):
        F.hca_query_of(*h)
        st.oracle_query()
    dt = time.perf_counter() - t0
    return _cpu_line(len(seqs), dt, "queries/s",
                     f"{len(seqs)} of {Wh.B} ragged sequences (HCA layer over every visible entry + "
                     f"window, CSA layer: indexer, top-512, attention)")


def cpu_baseline_tiny(W, reps):
    """The tiny fp32 decode step in the oracle: indexer, top-512, attention
    (the compressed pool is untimed setup)."""
    from oracle import csa_oracle as O
    from workloads import gen
    wl = W.wl
    g = gen.rng(wl.seed)
    L, N = W.L, W.N
    x = gen.normal(g, (L, 576))
    gw, gb = gen.gate_params(g, 4)
    kraw = gen.normal(g, (N, wl.index_dim))
    q_idx = gen.normal(g, (1, wl.index_heads, wl.index_dim))[0]
    w_idx = gen.uniform(g, (1, wl.index_heads))[0]
    q = gen.normal(g, (1, wl.heads, 576))[0]
    c4 = O.KVPool(*O.quant_kv_entries(O.compress_blocks(x, 0, 4, gw, gb), "f32"), "f32")
    raw = O.KVPool(*O.quant_kv_entries(x, "f32"), "f32")
    ip = O.IndexPool(kraw, None, "f32")
    ident = np.arange(L // 256)
    t0 = time.perf_counter()
    for _ in range(reps):
        O.csa_query(q_idx, w_idx, ip, c4, raw, ident, ident, N, L - 1, q, wl.window, wl.softmax_scale)
    dt = time.perf_counter() - t0
    return _cpu_line(reps, dt, "queries/s", f"the one decode query, {reps} times")


# ---------------------------------------------------------------- workloads


def line_decode(W, a, copies, roofline_kernel, cpu=None):
    ms, k_ms, _, dist = time_steps(W, a.steps, a.warmup, copies, graph=not a.no_graph)
    rows = getattr(W, "T", W.B)
    d = {"queries_per_s": round(rows / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
         "step_ms_percentiles": dist, "pool_copies": copies,
         "roofline": hbm_roofline(roofline_kernel, W.indexer_bytes(), k_ms),
         "step_bytes": int(W.step_bytes()),
         "step_hbm_frac": round(W.step_bytes() / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    if cpu is not None and not a.no_cpu_baseline:
        d["cpu_baseline"] = cpu(W)
    return d


def secondary(a):
    import torch
    from workloads import gen, specs
    from workloads.device import (CsaDecode, CsaPrefill, CsaSpecDecode, HcaCsaRagged, TinyDecode,
                                  hca_build_input)
    import compressed_sparse_attention_c4_amd as csa
    out = {}
    steps = max(10, a.steps // 2)
    sa = argparse.Namespace(**vars(a))
    sa.steps = steps

    # tiny all-fp32 decode: latency of one step
    W = TinyDecode(specs.TINY_FP32_DECODE)
    ms, k_ms, _, dist = time_steps(W, steps, a.warmup, 1, graph=not a.no_graph)
    out[specs.TINY_FP32_DECODE.name] = {
        "queries_per_s": round(1 / (ms / 1e3), 1), "latency_us": round(ms * 1e3, 2),
        "step_ms_percentiles": dist,
        "step_bytes": W.step_bytes(),
        "roofline": {"bound": "latency", "note": "1.8 MB per step is 0.2 us at 8 TB/s: launch and "
                     "latency bound; the step time is the figure", "frac": None},
        **({} if a.no_cpu_baseline else {"cpu_baseline": cpu_baseline_tiny(W, 400)})}
    del W

    # decode at 1M context, batch 4, MXFP4 index-K, 128 heads
    wl = specs.DECODE_1M
    probe = int(wl.batch * (wl.seq_len // 4) * (wl.index_dim // 2 + 4))
    copies = auto_copies(probe, a.copies)
    W = CsaDecode(wl, [wl.seq_len] * wl.batch, copies=copies, pool_pages=wl.pool_pages)
    out[wl.name] = line_decode(W, sa, copies, W.indexer_kernel,
                               lambda W: cpu_baseline_decode(W, list(range(W.B))))
    del W
    torch.cuda.empty_cache()

    # multi-token (speculative-verify) decode: 32 sequences x 4 query tokens at 128K
    wl = specs.SPEC_DECODE_128K
    probe = int(wl.batch * (wl.seq_len // 4) * (wl.index_dim + 4))
    copies = auto_copies(probe, a.copies)
    W = CsaSpecDecode(wl, [wl.seq_len] * wl.batch, copies=copies, pool_pages=wl.pool_pages)
    out[wl.name] = line_decode(W, sa, copies, W.indexer_kernel,
                               lambda W: cpu_baseline_spec(W, [0, 1, 2, 3, 40, 41, 42, 43, 124, 125, 126, 127]))
    del W
    torch.cuda.empty_cache()

    # chunked prefill: 4096 new tokens on a 131072-token context
    wl = specs.PREFILL_4K
    W = CsaPrefill(wl)
    ms, k_ms, _, dist = time_steps(W, max(5, steps // 4), 2, 1, graph=not a.no_graph)
    tf = W.indexer_flops() / (k_ms / 1e3) / 1e12
    kname = "indexer_rows_kernel<false, 8, true>"
    c = stored_counters(kname) or {}
    line = {"tokens_per_s": round(W.new / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
            "step_ms_percentiles": dist,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / FP8_PEAK_TFLOPS, 4),
                         "traffic": c.get("bytes_per_launch"), "kernel": kname,
                         "kernel_ms": round(k_ms, 4), "flop_per_launch": W.indexer_flops(),
                         "counter_mfma_f8_flops": c.get("mfma_f8_flops"),
                         "counter_mfma_busy_frac": (None if c.get("mfma_busy_frac") is None
                                                    else round(c["mfma_busy_frac"], 4))}}
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(W, [0, 511, 1024, 1709, 2048, 2600, 3001, 3500,
                                                        3800, 4000, 4094, 4095])
    out[wl.name] = line
    del W
    torch.cuda.empty_cache()

    # HCA layer + CSA layer over 16 ragged sequences
    wl = specs.HCA_RAGGED
    n, lo, hi = wl.ragged
    lens = gen.ragged_lengths(gen.rng(wl.seed), n, lo, hi)
    per_copy = int((lens // 4).sum()) * (wl.index_dim + 4) + int((lens // wl.hca_ratio).sum()) * 644
    copies = auto_copies(per_copy, a.copies)
    W = HcaCsaRagged(wl, copies=copies)
    ms, k_ms, _, dist = time_steps(W, steps, a.warmup, copies, graph=not a.no_graph)
    step_bytes = W.csa.step_bytes() + W.hca_bytes()
    line = {"queries_per_s": round(W.B / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
            "step_ms_percentiles": dist, "pool_copies": copies,
            "raw_lengths": [int(x) for x in W.lens],
            "roofline": hbm_roofline(W.csa.indexer_kernel, W.csa.indexer_bytes(), k_ms),
            "step_bytes": int(step_bytes),
            "step_hbm_frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    if not a.no_cpu_baseline:
        order = [int(b) for b in np.argsort(W.lens)]
        line["cpu_baseline"] = cpu_baseline_hca(W, order[::2])
    out[wl.name] = line
    del W
    torch.cuda.empty_cache()

    # HCA cache build (ratio 128 over every raw row)
    x, cu, st = hca_build_input(lens, wl.seed * 10 + 11)
    gw, gb = gen.gate_params(gen.rng(wl.seed + 3), wl.hca_ratio)
    gw, gb = torch.from_numpy(gw).cuda(), torch.from_numpy(gb).cuda()
    hpages = [int(n) // wl.hca_ratio // 64 + 1 for n in lens]
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
                                   "roofline": {"bound": "hbm", "achieved": round(nbytes / (bms / 1e3) / 1e9, 1),
                                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                "frac": round(nbytes / (bms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                                "traffic": None, "kernel": "compress_kernel",
                                                "bytes_per_launch": nbytes}}
    del x, pool
    torch.cuda.empty_cache()
    return out


def profile_only(a):
    import torch
    from workloads import specs
    from workloads import gen
    from workloads.device import CsaDecode, CsaPrefill, CsaSpecDecode, HcaCsaRagged, TinyDecode
    if a.profile_only == "copy":
        n = 1 << 28  # 1 GiB of float32 read and 1 GiB written per copy
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(a.warmup + a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profiled copy: {a.warmup + a.steps} copies of {4 * n} B", flush=True)
        return
    if a.profile_only == "tiny":
        W, copies = TinyDecode(specs.TINY_FP32_DECODE), 1
    elif a.profile_only in ("decode_128k", "decode_1m", "spec_decode"):
        # the pool copies of the timed bench run of the same workload
        wl = {"decode_128k": specs.DECODE_128K, "decode_1m": specs.DECODE_1M,
              "spec_decode": specs.SPEC_DECODE_128K}[a.profile_only]
        row = wl.index_dim // 2 + 4 if wl.index_fmt == "mxfp4" else wl.index_dim + 4
        copies = auto_copies(int(wl.batch * (wl.seq_len // 4) * row), a.copies)
        cls = CsaSpecDecode if a.profile_only == "spec_decode" else CsaDecode
        W = cls(wl, [wl.seq_len] * wl.batch, copies=copies, pool_pages=wl.pool_pages)
    elif a.profile_only == "prefill":
        W, copies = CsaPrefill(specs.PREFILL_4K), 1
    else:
        wl = specs.HCA_RAGGED
        n, lo, hi = wl.ragged
        lens = gen.ragged_lengths(gen.rng(wl.seed), n, lo, hi)
        per_copy = int((lens // 4).sum()) * (wl.index_dim + 4) + int((lens // wl.hca_ratio).sum()) * 644
        copies = auto_copies(per_copy, a.copies)
        W = HcaCsaRagged(wl, copies=copies)
    torch.cuda.synchronize()
    time.sleep(PROFILE_GAP_S)  # marks the start of the steps in a kernel trace
    for i in range(a.warmup + a.steps):
        W.step(i % copies)
    torch.cuda.synchronize()
    print(f"profiled {a.profile_only}: {a.warmup + a.steps} eager steps over {copies} pool copies",
          flush=True)


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if a.counters_from:
        reduce_counters(a.counters_from)
        return
    if a.trace_from:
        reduce_trace(a.trace_from, a.trace_steps)
        return
    import torch
    from workloads import specs
    from workloads.device import CsaDecode

    torch.cuda.set_device(0)
    if a.profile_only:
        profile_only(a)
        return
    wl = specs.DECODE_128K
    copies = auto_copies(int(wl.batch * (wl.seq_len // 4) * (wl.index_dim + 4)), a.copies)
    W = CsaDecode(wl, [wl.seq_len] * wl.batch, copies=copies, pool_pages=wl.pool_pages)
    kernel = W.indexer_kernel
    ms, k_ms, _, dist = time_steps(W, a.steps, a.warmup, copies, graph=not a.no_graph)
    qps = W.B / (ms / 1e3)
    line = {
        "metric": "CSA decode queries/s @128K ctx",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "step_ms_percentiles": dist,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": W.B, "seq_len": wl.seq_len,
                   "compressed_entries": int(W.N[0]), "index_format": "fp8_e4m3+hadamard",
                   "index_heads": wl.index_heads, "attn_heads": wl.heads, "topk": 512,
                   "window": wl.window, "pool_copies": copies, "hip_graph": not a.no_graph},
        "roofline": hbm_roofline(kernel, W.indexer_bytes(), k_ms),
        "step_bytes": int(W.step_bytes()),
        "step_hbm_frac": round(W.step_bytes() / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(W, list(range(W.B)), min_s=10.0)
    del W
    torch.cuda.empty_cache()
    if not a.no_secondary:
        line["secondary"] = secondary(a)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
