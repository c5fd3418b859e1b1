"""Decode-step benchmark: effective KV bandwidth of one zero-copy decode step.

Workload (default): eight Llama-3-70B-shaped layers (hidden 8192, 64 query /
8 KV heads, head_dim 128), batch 16, 131072 cached tokens per sequence, KV
100 % in host-pinned memory (8 GiB per layer, 64 GiB per step) read in place
over the host link; synthetic bf16 inputs from the seeded generator (W ~
N(0, 0.015^2), x and K/V ~ N(0, 1)). ``--workload`` selects any of the five
workloads (see synth/configs.py); for a multi-layer workload a step runs
every layer in order.

A step is one decode_step call per layer: QKV projection, attention over
every cached token plus the fresh one, fresh K/V write-back, split combine.
Inputs are resident (KV in its pool, x/W in HBM) before the timed region
starts.

Prints one JSON line: metric/value (effective KV GB/s = algorithmic KV bytes
per step / step time, steps enqueued eagerly), ms_per_step and
graph_ms_per_step (the same step replayed from one captured HIP graph),
roofline (dominant kernel = split attention, against the host link), the
measured host-link streaming-read ceiling, the same step with every page in
HBM (against 8 TB/s), the naive zero-copy, staging and host-CPU attention
comparators, and the fp64 oracle timed on the host cores on the same workload
(whole steps of a one-layer workload; one whole layer of a multi-layer one),
with the parity of the bench's own output against it.

``--sweep`` steps the host-resident share of the KV from 0 to 100 %;
``--sweep-ctx`` steps the context length (zero-copy, all-HBM, staging and
host-CPU attention at each length); ``--gemm S`` runs the host-operand GEMM
experiment.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PCIE_GEN5_X16_GBPS = 64.0     # published per-direction rate of the MI355X host interface
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
CHUNK = 8192                  # tokens per set-up append


def log(msg):
    print("[bench %s] %s" % (time.strftime("%H:%M:%S"), msg), file=sys.stderr, flush=True)


class Resident:
    """One workload's KV in its pools (placed by `tail`), plus x, W, ctx_lens
    in HBM, for every layer."""

    def __init__(self, dkv, wl, ctx, tail, kv_source, copy_from=None):
        """copy_from: a Resident of the same workload whose pool holds every
        page on the host; this one's (every page in HBM) is then filled by a
        copy-engine copy of that pool instead of drawing the KV again (pages
        are handed out in the same order, so every page keeps its offset)."""
        import torch
        self.dkv = dkv
        self.wl = wl
        self.n_layers = wl.n_layers
        self.shape = dkv.Shape.of(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                  wl.n_layers)
        cap = (ctx + 1).astype(np.int32)
        tail = np.asarray(tail, np.int32)
        n_host = n_hbm = 0
        for b in range(len(ctx)):
            n, first = dkv.kv_placement(int(cap[b]), int(tail[b]))
            n_host += first
            n_hbm += n - first
        n_host *= wl.n_layers
        n_hbm *= wl.n_layers
        self.host_pool = dkv.kv_alloc_host(self.shape, n_host) if n_host else None
        self.hbm_pool = dkv.kv_alloc_hbm(self.shape, n_hbm) if n_hbm else None
        self.page_bytes = dkv.kv_page_bytes(self.shape)
        self.n_host, self.n_hbm = n_host, n_hbm
        self.layout = dkv.kv_layout_create(self.shape, cap, tail, self.host_pool, self.hbm_pool)
        dev = torch.device("cuda", 0)
        self.x, self.W = [], []
        if copy_from is not None:
            src = copy_from.host_pool
            assert n_host == 0 and copy_from.hbm_pool is None and src.info()[1] == n_hbm * self.page_bytes
            dkv.kv_pool_copy(self.hbm_pool, src, src.info()[1])
            torch.cuda.synchronize()
        for layer in range(wl.n_layers):
            for b in range(len(ctx) if copy_from is None else 0):
                for t0 in range(0, int(ctx[b]), CHUNK):
                    t1 = min(int(ctx[b]), t0 + CHUNK)
                    k, v = kv_source(layer, b, t0, t1)
                    dkv.kv_append(self.layout, layer, b, t0, k, v)
            self.x.append(torch.from_numpy(wl.x(layer).view(np.int16)).to(dev).view(torch.bfloat16))
            self.W.append(torch.from_numpy(wl.W(layer).view(np.int16)).to(dev).view(torch.bfloat16))
            if wl.n_layers > 1 and copy_from is None:
                log("layer %d resident" % layer)
        self.ctx = torch.from_numpy(ctx.copy()).to(dev)
        self.out = [torch.empty((len(ctx), wl.n_q_heads * wl.head_dim), dtype=torch.bfloat16,
                                device=dev) for _ in range(wl.n_layers)]
        self.stream = torch.cuda.current_stream()

    def step(self, layers=None):
        for layer in (range(self.n_layers) if layers is None else layers):
            self.dkv.decode_step(self.layout, layer, self.x[layer], self.W[layer], self.ctx,
                                 self.out[layer], self.stream)

    def timed(self, steps, warmup, split_events=False):
        """Milliseconds per step over `steps` steps (HIP events on the step's
        stream around the whole run); per-step median / min / max from an
        event between consecutive steps are kept in self.step_stats. With
        split_events, the library also records two events around the split
        kernel of each of these same steps on their stream (only those two,
        so that short steps are barely disturbed), and self.kernel_ms["split"]
        gets its per-step milliseconds over the timed region."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        if split_events:
            self.layout.timing_enable(True, steps * self.n_layers, split_only=True)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(self.stream)
        for i in range(steps):
            self.step()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        if split_events:
            t = self.layout.timing_read()
            self.layout.timing_enable(False)
            self.kernel_ms = {"split": t["split"] / (max(1, t["steps"]) / self.n_layers)}
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        self.step_stats = {"median": round(float(np.median(per)), 4), "min": round(per[0], 4),
                           "max": round(per[-1], 4)}
        return ev[0].elapsed_time(ev[steps]) / steps

    def graph_timed(self, steps):
        """Milliseconds per step with one step (every layer) captured in a HIP
        graph and replayed `steps` times (events on the replaying stream)."""
        import torch
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for layer in range(self.n_layers):
                self.dkv.decode_step(self.layout, layer, self.x[layer], self.W[layer], self.ctx,
                                     self.out[layer])
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_time(e1) / steps

    def kernel_times(self, steps):
        """Per-step kernel milliseconds (summed over layers) from events the
        library records around each kernel on the step's stream."""
        import torch
        self.layout.timing_enable(True, steps * self.n_layers)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        t = self.layout.timing_read()
        self.layout.timing_enable(False)
        n = max(1, t["steps"]) / self.n_layers
        return {k: t[k] / n for k in ("projection", "fresh", "split", "combine")}

    def out_bits(self, layer=0):
        import torch
        return self.out[layer].view(torch.int16).cpu().numpy().view(np.uint16)

    def free(self):
        import torch
        torch.cuda.synchronize()
        self.layout.free()
        for p in (self.host_pool, self.hbm_pool):
            if p:
                p.free()


HOST_PROBE_BYTES = 4 << 30


def probe_ceiling(dkv, pool, configs_, max_bytes=HOST_PROBE_BYTES):
    base, nbytes, _ = pool.info()
    nbytes = min(nbytes, max_bytes)
    nbytes -= nbytes % (1 << 20)
    return probe_region(dkv, base, nbytes, configs_)


def probe_host_link(dkv, configs_, nbytes=HOST_PROBE_BYTES, flags=0):
    """The host-link streaming-read ceiling on a fresh pinned buffer of
    `nbytes` (4 GiB), allocated like a host pool (mapped, coherent)."""
    buf = dkv.HostBuffer(nbytes, flags)
    try:
        return probe_region(dkv, buf.device_ptr, nbytes, configs_)
    finally:
        buf.free()


def probe_region(dkv, base, nbytes, configs_):
    best = 0.0
    rows = []
    for grid, unroll in configs_:
        ms = dkv.probe_stream_read(base, nbytes, grid, unroll, reps=3)
        gbps = nbytes / ms / 1e6
        rows.append({"grid": grid, "in_flight": abs(unroll), "nontemporal": unroll < 0,
                     "GBps": round(gbps, 2)})
        best = max(best, gbps)
    return best, rows, nbytes


def probe_page_runs(dkv, pool, wl, max_bytes=8 << 30):
    """The HBM read ceiling in the split kernel's own access pattern, with no
    arithmetic: each wavefront streams one KV head's run (K then V rows) of
    every page of an item of consecutive pages, as the one-wavefront-per-item
    split kernel does; 2048 and 3072 wavefronts, items starting in step or
    staggered. Returns (best GB/s, rows)."""
    base, nbytes, _ = pool.info()
    shape = dkv.Shape.of(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, 1)
    page = dkv.kv_page_bytes(shape)
    runs = wl.n_kv_heads
    best, rows = 0.0, []
    for waves in PAGE_PROBE_WAVES:
        items = waves // runs
        pages = min(nbytes, max_bytes) // page
        pages -= pages % items
        if pages == 0:
            continue
        for skew in (False, True):
            ms = dkv.probe_page_read(base, pages * page, page, runs, waves, skew, reps=3)
            gbps = pages * page / ms / 1e6
            rows.append({"waves": waves, "pages_per_item": pages // items, "staggered": skew,
                         "bytes": pages * page, "GBps": round(gbps, 1)})
            best = max(best, gbps)
    return best, rows


PAGE_PROBE_WAVES = (2048, 3072)
HOST_PROBES = [(64, 1), (256, 1), (512, 1), (1024, 2), (256, -1), (1024, -2)]
SMALL_READ_BYTES = 64 << 20       # layers reading less than this over the link also get a same-size read
HBM_PROBES = [(1024, -2), (2048, -2), (4096, -4), (8192, -8), (2048, 4)]


SPLIT_KERNEL_SOURCES = ("attn_split.hip", "device_common.h")


def code_tokens(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed (the sources
    hashed here hold no string literal with a comment marker)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def split_kernel_sha256() -> str:
    """sha256 over the code the split-attention kernel is compiled from: its
    own source, the device helpers, and the StepArgs struct it reads, with
    comments and whitespace left out (so editing a comment keeps the counter
    records valid; any code change invalidates them)."""
    import hashlib
    csrc = os.path.join(ROOT, "decode_attention_zero_amd", "csrc")
    h = hashlib.sha256()
    for name in SPLIT_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(code_tokens(f.read()).encode())
    with open(os.path.join(csrc, "dkv_internal.h"), encoding="utf-8") as f:
        text = f.read()
    i = text.index("struct StepArgs {")
    h.update(code_tokens(text[i:text.index("};", i)]).encode())
    return h.hexdigest()


def traffic_record_path(workload: str, all_hbm: bool = False, kernel: str | None = None) -> str:
    return os.path.join(ROOT, "profiles", "attn_split_%s%s%s_traffic.json"
                        % (workload, "_allhbm" if all_hbm else "", "_" + kernel if kernel else ""))


def counter_traffic(workload: str, all_hbm: bool = False, kernel: str | None = None):
    """HBM + host-link bytes per split-kernel launch from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by a copy kernel of known
    size); None when the summary is missing or the kernel's sources have
    changed since the counters were taken. kernel: None for the layout's
    default split kernel, or a --split-kernel name (naive: the comparator)."""
    rec = counter_record(workload, all_hbm, kernel)
    return None if rec is None else int(rec["traffic_bytes_per_launch"])


def counter_record(workload: str, all_hbm: bool = False, kernel: str | None = None):
    """The committed counter record of a split kernel (see counter_traffic),
    or None when it is missing or stale."""
    path = traffic_record_path(workload, all_hbm, kernel)
    try:
        with open(path) as f:
            rec = json.load(f)
        sha = split_kernel_sha256()
    except OSError:
        return None
    return rec if rec.get("split_kernel_sources_sha256") == sha else None


def pmc_per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} from one rocprofv3
    `pmc_counter_collection.csv` (the counter's per-instance rows added up)."""
    import csv
    vals, names = {}, {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            i = int(row["Dispatch_Id"])
            vals[i] = vals.get(i, 0.0) + float(row["Counter_Value"])
            names[i] = row["Kernel_Name"]
    return {i: (names[i], vals[i]) for i in vals}


TCC_ROUTE_COUNTERS = ("TCC_EA0_RDREQ_IO_32B_sum", "TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_HIT_sum", "TCC_MISS_sum")


def write_traffic_record(wl, args) -> int:
    """Reduces the two counter runs of a workload (rocprofv3 --pmc FETCH_SIZE,
    then WRITE_SIZE, each over `bench.py --profile-run --calibrate` with the
    same --workload, --all-hbm, --steps and --warmup as this call; their -d
    directories are `<prefix>_FETCH_SIZE` and `<prefix>_WRITE_SIZE`) to the
    split kernel's traffic record under profiles/, which counter_traffic reads.
    FETCH_SIZE and WRITE_SIZE are scaled by what they read for the run's
    256 MiB HBM-to-HBM copy. Runs on the host alone; no GPU."""
    prefix = args.traffic_record
    fetch = pmc_per_dispatch(os.path.join(prefix + "_FETCH_SIZE", "pmc_counter_collection.csv"), "FETCH_SIZE")
    write = pmc_per_dispatch(os.path.join(prefix + "_WRITE_SIZE", "pmc_counter_collection.csv"), "WRITE_SIZE")

    def of(rows, key):
        return [v for name, v in rows.values() if key in name]

    split_f, split_w = of(fetch, "attn_split"), of(write, "attn_split")
    if not split_f or not split_w:
        print("no split-kernel dispatches under %s_{FETCH,WRITE}_SIZE" % prefix, file=sys.stderr)
        return 1
    kernel = [name for name, _ in fetch.values() if "attn_split" in name][0]
    kernel = kernel.replace("void dkv::(anonymous namespace)::", "").split("(dkv::StepArgs)")[0]
    copy_f, copy_w = max(of(fetch, "copyBuffer")), max(of(write, "copyBuffer"))
    fetch_scale, write_scale = 262144.0 / copy_f, 262144.0 / copy_w       # 256 MiB in KiB
    mf, mw = sum(split_f) / len(split_f), sum(split_w) / len(split_w)
    traffic = (mf * fetch_scale + mw * write_scale) * 1024
    alg = int(wl.ctx_lens().astype(np.int64).sum()) * wl.kv_bytes_per_token   # one layer = one launch
    sfx = ("_allhbm" if args.all_hbm else "") + ("_" + args.split_kernel if args.split_kernel else "")
    opts = (" --all-hbm" if args.all_hbm else "") + (" --split-kernel " + args.split_kernel if args.split_kernel else "")
    run = "python3 $REPO/bench.py --workload %s --profile-run%s --calibrate --steps %d --warmup %d" % (
        wl.name, opts, args.steps, args.warmup)
    rec = {"kernel": kernel,
           "workload": wl.name + (", every page in HBM" if args.all_hbm else "")
           + (", split kernel " + args.split_kernel if args.split_kernel else ""),
           "split_kernel_sources_sha256": split_kernel_sha256(),
           "fetch_size_kib_per_dispatch": round(mf, 3), "write_size_kib_per_dispatch": round(mw, 3),
           "dispatches": len(split_f),
           "calibration": {"copy_kernel": "__amd_rocclr_copyBuffer, 256 MiB HBM -> HBM",
                           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
                           "fetch_scale": fetch_scale, "write_scale": write_scale,
                           "stream_read_fetch_kib": sorted(of(fetch, "stream_read"))},
           "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": alg,
           "traffic_over_algorithmic": traffic / alg,
           "commands": ["cd /tmp && export TMPDIR=/tmp"] + [
               "rocprofv3 --pmc %s --output-format csv -d $REPO/gpurun_out/pmc_%s%s_%s -o pmc -- %s"
               % (c, wl.name, sfx, c, run) for c in ("FETCH_SIZE", "WRITE_SIZE")] + [
               "python3 $REPO/bench.py --workload %s%s --steps %d --warmup %d --traffic-record "
               "$REPO/gpurun_out/pmc_%s%s" % (wl.name, opts, args.steps, args.warmup, wl.name, sfx)],
           "hashed_sources": "attn_split.hip, device_common.h, struct StepArgs of dkv_internal.h; "
                             "comments and whitespace removed"}
    # Optional third pass: where the L2's read requests went (host link = IO,
    # HBM = DRAM, in 32-byte units) and its hit rate.
    tcc_dir = os.path.join(prefix + "_TCC", "pmc_counter_collection.csv")
    if os.path.exists(tcc_dir):
        cnt = {c: pmc_per_dispatch(tcc_dir, c) for c in TCC_ROUTE_COUNTERS}

        def mean_of(c, key="attn_split"):
            v = of(cnt[c], key)
            return sum(v) / len(v) if v else None

        io, dram = mean_of("TCC_EA0_RDREQ_IO_32B_sum"), mean_of("TCC_EA0_RDREQ_DRAM_32B_sum")
        hit, miss = mean_of("TCC_HIT_sum"), mean_of("TCC_MISS_sum")
        rec["l2_read_routes"] = {
            "host_link_read_bytes_per_dispatch": io * 32, "hbm_read_bytes_per_dispatch": dram * 32,
            "l2_hit_rate": hit / (hit + miss) if hit is not None and hit + miss > 0 else None,
            "host_link_reads_over_algorithmic": io * 32 / alg,
            "calibration_host_stream_read_bytes_per_dispatch": sorted(
                v * 32 for v in of(cnt["TCC_EA0_RDREQ_IO_32B_sum"], "stream_read")),
            "counters": list(TCC_ROUTE_COUNTERS)}
        rec["commands"].insert(3, "rocprofv3 --pmc %s --output-format csv -d $REPO/gpurun_out/pmc_%s%s_TCC -o pmc "
                                  "-- %s" % (" ".join(TCC_ROUTE_COUNTERS), wl.name, sfx, run))
    out = traffic_record_path(wl.name, args.all_hbm, args.split_kernel)
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"record": os.path.relpath(out, ROOT), "kernel": kernel, "dispatches": len(split_f),
                      "traffic_over_algorithmic": round(traffic / alg, 4),
                      "l2_read_routes": rec.get("l2_read_routes")}))
    return 0


def calibrate(dkv, r):
    """Kernels whose HBM / host traffic is known exactly, for counter scaling."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)                    # reads 256 MiB, writes 256 MiB of HBM
    torch.cuda.synchronize()
    if r.host_pool is not None:
        base, nbytes, _ = r.host_pool.info()
        dkv.probe_stream_read(base, min(1 << 30, nbytes - nbytes % (1 << 20)), 256, 1,
                              reps=1)                       # 2 x (up to) 1 GiB host reads
    dkv.probe_stream_read(dst.data_ptr(), n, 2048, 4, reps=1)   # 2 x 256 MiB HBM reads
    torch.cuda.synchronize()
    log("calibration kernels done")


def gemm_experiment(dkv, args):
    """C = A x B^T (S x S x S, bf16 in, fp32 out) with B in pinned host memory:
    swap (copy-engine copy of B into HBM, then the GEMM), naive zero-copy (the
    GEMM reading B in place in row-major tile order) and CPU-aware zero-copy
    (the tile order that fetches each B column block over the link once),
    next to the GEMM with B already in HBM. One JSON line."""
    import torch
    import synth
    S = args.gemm
    M = N = K = S
    dev = torch.device("cuda", 0)
    log("gemm %d^3: generating operands" % S)
    A = torch.from_numpy(synth.normal_bf16(7, 60, 0, M * K, 1.0).view(np.int16)).to(dev).view(torch.bfloat16)
    A = A.reshape(M, K)
    flags = dkv.HOST_NONCOHERENT if args.gemm_noncoherent else dkv.HOST_COHERENT
    hb = dkv.HostBuffer(N * K * 2, flags)
    Bh = hb.view(np.uint16, (N, K))
    synth.normal_bf16(7, 61, 0, N * K, 1.0, out=Bh.reshape(-1))
    B_hbm = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    flop = 2.0 * M * N * K
    b_bytes = N * K * 2

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def gemm(ptr, cpu_aware):
        return lambda: dkv.gemm_bf16_nt(A, ptr, C, M, N, K, cpu_aware, stream)

    ws = torch.empty(dkv.gemm_bstationary_workspace_bytes(M, N, K) // 4, dtype=torch.float32, device=dev)

    def bstationary(ptr):
        return lambda: dkv.gemm_bf16_nt_bstationary(A, ptr, C, M, N, K, ws, stream)

    def swap():
        dkv.copy(B_hbm.data_ptr(), hb.device_ptr, b_bytes, stream)
        dkv.gemm_bf16_nt(A, B_hbm.data_ptr(), C, M, N, K, False, stream)

    if args.gemm_profile:
        for cpu_aware in (True, False):
            gemm(hb.device_ptr, cpu_aware)()
        bstationary(hb.device_ptr)()
        dkv.copy(B_hbm.data_ptr(), hb.device_ptr, b_bytes, stream)
        gemm(B_hbm.data_ptr(), False)()
        torch.cuda.synchronize()
        hb.free()
        print(json.dumps({"gemm_profile_run": True, "S": S}), flush=True)
        return 0
    results, outs = {}, {}
    reps = max(1, min(args.steps, 10))
    variants = [("gemm_B_in_hbm", None, reps), ("swap", swap, reps),
                ("zero_copy_cpu_aware", gemm(hb.device_ptr, True), reps),
                ("zero_copy_b_stationary", bstationary(hb.device_ptr), reps),
                ("zero_copy_naive", gemm(hb.device_ptr, False), 1)]
    dkv.copy(B_hbm.data_ptr(), hb.device_ptr, b_bytes, stream)
    torch.cuda.synchronize()
    for name, fn, n in variants:
        fn = fn or gemm(B_hbm.data_ptr(), False)
        ms = timed(fn, n)
        results[name] = {"ms": round(ms, 3), "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 1)}
        outs[name] = C.view(torch.int32).cpu().numpy()
        log("gemm %s: %.3f ms" % (name, ms))
    ms_copy = timed(lambda: dkv.copy(B_hbm.data_ptr(), hb.device_ptr, b_bytes, stream), reps)
    results["swap"]["copy_ms"] = round(ms_copy, 3)
    results["swap"]["extra_hbm_bytes"] = b_bytes
    first = outs["gemm_B_in_hbm"]
    # One fp32 sum per entry in every variant but the B-stationary one, which
    # adds per-k-tile sums: identical bits among the first, the bound for both.
    identical = all(np.array_equal(v, first) for k, v in outs.items() if k != "zero_copy_b_stationary")
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
        rng = np.random.default_rng(5)
        rows, cols = rng.integers(0, M, 64), rng.integers(0, N, 64)
        Ah = A.view(torch.int16).cpu().numpy().view(np.uint16)
        ref = orc.gemm_nt_entries(Ah, Bh, rows, cols)
        got = first.view(np.float32)[rows, cols].astype(np.float64)
        a_abs = np.abs((Ah[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        b_abs = np.abs((Bh[cols].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        g = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
        bnd = g * np.einsum("ek,ek->e", a_abs, b_abs)
        got_bs = outs["zero_copy_b_stationary"].view(np.float32)[rows, cols].astype(np.float64)
        parity = {"sampled_entries": 64, "max_abs_err": float(np.abs(got - ref).max()),
                  "max_err_over_bound": float((np.abs(got - ref) / bnd).max()),
                  "within_fp32_summation_bound": bool(np.all(np.abs(got - ref) <= bnd)),
                  "b_stationary_max_err_over_bound": float((np.abs(got_bs - ref) / bnd).max()),
                  "b_stationary_within_bound": bool(np.all(np.abs(got_bs - ref) <= bnd))}
    hb.free()
    print(json.dumps({"experiment": "gemm_host_operand", "M": M, "N": N, "K": K,
                      "dtype": "bf16 in, fp32 accumulate and out",
                      "B_host_memory": "non-coherent" if args.gemm_noncoherent else "coherent",
                      "B_bytes": b_bytes, "results": results,
                      "bit_identical_one_sum_variants": identical,
                      "b_stationary_workspace_bytes": ws.numel() * 4,
                      "parity": parity}), flush=True)
    return 0


PROJ_SHAPES = (("llama3-8b", 4096, 32), ("llama3-70b", 8192, 64))
PROJ_BATCHES = (1, 2, 3, 4, 8, 16, 32, 64)
PROJ_COLD_BYTES = 640 << 20          # W copies cycled per step: past the 256 MiB last-level cache
PROJ_READ_PROBES = [(256, -2), (512, -2), (1024, -2), (1024, -4), (2048, -2), (2048, -4), (4096, -2)]


def projection_experiment(dkv, args):
    """The decode step's QKV projection on its own: for the Llama-3 8B and
    70B shapes (8 KV heads, head_dim 128) at batches 1-64, the projection
    kernel's and the fresh-token kernel's times from the layout's HIP events,
    with W cycled through enough copies that every step reads W from HBM;
    beside them, the best of several grid-stride streaming reads of the same
    W bytes, also cycled (the read a kernel of this size can reach, launch
    and ramp included). KV is 16 tokens per sequence, so the step's
    attention is negligible. One JSON line per (shape, batch)."""
    import torch
    dev = torch.device("cuda", 0)
    steps = max(args.steps, 8)
    batches = [int(v) for v in args.proj_batches.split(",")]
    shapes = args.proj_shapes.split(",")
    for name, hidden, Hq in PROJ_SHAPES:
        if name not in shapes:
            continue
        shape = dkv.Shape.of(hidden, Hq, 8, 128, 1)
        n_qkv = (Hq + 16) * 128
        w_elems = n_qkv * hidden
        w_bytes = w_elems * 2
        nW = max(4, -(-PROJ_COLD_BYTES // w_bytes))
        Wall = torch.empty(nW * w_elems, dtype=torch.bfloat16, device=dev)
        g = torch.Generator(device=dev).manual_seed(1)
        for i in range(nW):
            Wall[i * w_elems:(i + 1) * w_elems] = (torch.randn(w_elems, device=dev, generator=g) * 0.02).to(
                torch.bfloat16)
        Ws = [Wall[i * w_elems:(i + 1) * w_elems].view(n_qkv, hidden) for i in range(nW)]
        torch.cuda.synchronize()
        reads = {}
        for grid, unroll in PROJ_READ_PROBES:
            ms = dkv.probe_stream_read_cycled(Wall.data_ptr(), w_bytes, nW, grid, unroll, reps=2 * nW)
            reads["%dx%d%s" % (grid, abs(unroll), "nt" if unroll < 0 else "")] = round(ms * 1e3, 2)
        read_us = min(reads.values())
        log("projection %s: cold read of W (%d B) %.2f us" % (name, w_bytes, read_us))
        for B in batches:
            ctx = np.full(B, 16, np.int32)
            hbm = dkv.kv_alloc_hbm(shape, B * 2)
            layout = dkv.kv_layout_create(shape, ctx + 1, np.full(B, 1 << 30, np.int32), None, hbm)
            kernel = layout.projection_kernel
            x = (torch.randn(B, hidden, device=dev, generator=g)).to(torch.bfloat16)
            c = torch.from_numpy(ctx).to(dev)
            out = torch.empty(B, Hq * 128, dtype=torch.bfloat16, device=dev)
            for i in range(nW):
                dkv.decode_step(layout, 0, x, Ws[i], c, out)
            torch.cuda.synchronize()
            layout.timing_enable(True, steps)
            for i in range(steps):
                dkv.decode_step(layout, 0, x, Ws[i % nW], c, out)
            t = layout.timing_read()
            layout.timing_enable(False)
            layout.check_status()
            layout.free()
            hbm.free()
            n = t["steps"]
            proj_us, fresh_us = t["projection"] / n * 1e3, t["fresh"] / n * 1e3
            mfma = kernel != "qkv_proj_gemv_kernel"
            flop = 2.0 * B * hidden * n_qkv
            line = {"experiment": "qkv_projection", "shape": name, "hidden": hidden, "n_qkv": n_qkv,
                    "batch": B, "kernel": kernel,
                    "W_bytes": w_bytes, "W_copies_cycled": nW, "steps": n,
                    "projection_us": round(proj_us, 2), "fresh_token_us": round(fresh_us, 2),
                    "W_TBps": round(w_bytes / (proj_us * 1e-6) / 1e12, 3),
                    "W_frac_of_8TBps": round(w_bytes / (proj_us * 1e-6) / 8e12, 4),
                    "cold_read_us": read_us, "cold_read_TBps": round(w_bytes / (read_us * 1e-6) / 1e12, 3),
                    "projection_vs_cold_read": round(read_us / proj_us, 4),
                    "TFLOPs": round(flop / (proj_us * 1e-6) / 1e12, 2),
                    "mfma_utilisation": round(flop / (proj_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5)
                    if mfma else None,
                    "cold_read_probes_us": reads}
            print(json.dumps(line), flush=True)
        del Ws, Wall
        torch.cuda.empty_cache()
    return 0


SWEEP_HOST_FRACTIONS = (0.0, 0.01, 0.03, 0.1, 0.25, 0.5, 0.75, 1.0)
SWEEP_CTX_LENGTHS = [1024, 4096, 16384, 32768, 65536, 131072]


def host_facts() -> dict:
    """Host logistics of the run: CPU, memory, the GPU's NUMA node, IOMMU."""
    facts = {"cpu_model": cpu_model(), "nproc": os.cpu_count()}
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    facts["mem_total_GiB"] = round(int(line.split()[1]) / 2**20, 1)
    except OSError:
        pass
    try:
        import torch
        p = torch.cuda.get_device_properties(0)
        bus = "%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
        with open("/sys/bus/pci/devices/%s/numa_node" % bus) as f:
            facts["gpu_numa_node"] = int(f.read().strip())
    except Exception:          # not every container exposes sysfs
        facts["gpu_numa_node"] = None
    try:
        facts["iommu_groups"] = len(os.listdir("/sys/kernel/iommu_groups"))
    except OSError:
        facts["iommu_groups"] = None
    facts["host_page_bytes"] = os.sysconf("SC_PAGE_SIZE")
    try:
        with open("/sys/kernel/mm/transparent_hugepage/enabled") as f:
            facts["transparent_hugepages"] = f.read().strip()
    except OSError:
        facts["transparent_hugepages"] = None
    return facts


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16


def projection_facts(wl, ms, kernel):
    """The QKV projection of one step (summed over layers): which kernel (as
    the layout reports it), its W read rate and its matrix-core use against
    the dense bf16 peak."""
    B = wl.batch
    w_bytes = wl.n_qkv * wl.hidden * 2 * wl.n_layers
    flop = 2.0 * B * wl.hidden * wl.n_qkv * wl.n_layers
    return {"kernel": kernel, "ms": round(ms, 4), "W_bytes": w_bytes,
            "W_GBps": round(w_bytes / (ms * 1e-3) / 1e9, 1),
            "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2),
            "mfma_utilisation": (round(flop / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5)
                                 if kernel != "qkv_proj_gemv_kernel" else None)}


def window_only_leg(dkv, wl, ctx, tail, kv_source, args):
    """The HBM-resident window of a hybrid placement timed alone: a layout
    holding, for each sequence, as many cached tokens as its window has, every
    page in HBM, stepped like the workload. Returns the split kernel's time
    and rate on those bytes (a timing run: the tokens are the sequence's
    first ones, so the outputs are not the workload's)."""
    win = np.zeros(len(ctx), np.int32)
    for b in range(len(ctx)):
        n, first = dkv.kv_placement(int(ctx[b]) + 1, int(tail[b]))
        win[b] = int(ctx[b]) - min(int(ctx[b]), first * dkv.PAGE_TOKENS)
    if int(win.min()) <= 0:
        return None
    log("HBM window alone: %d-%d tokens per sequence" % (int(win.min()), int(win.max())))
    rw = Resident(dkv, wl, win, np.full(len(ctx), 1 << 30, np.int32), kv_source)
    steps = max(args.steps, 50) if wl.n_layers == 1 else args.steps
    ms_w = rw.timed(steps, args.warmup)
    kt_w = rw.kernel_times(steps)
    split_tokens = rw.layout.split_tokens
    rw.free()
    w_bytes = int(win.astype(np.int64).sum()) * wl.kv_bytes_per_token * wl.n_layers
    gbps = w_bytes / (kt_w["split"] * 1e-3) / 1e9
    return {"tokens_per_sequence": [int(win.min()), int(win.max())], "kv_bytes_per_step": w_bytes,
            "split_tokens": split_tokens, "ms_per_step": round(ms_w, 4),
            "split_kernel_ms": round(kt_w["split"], 4), "split_kernel_GBps": round(gbps, 1),
            "split_kernel_frac_of_8TBps": round(gbps / HBM_PEAK_GBPS, 4)}


def split_kernel_label(layout) -> str:
    """Name of the split-attention kernel a layout launches, and its wavefronts
    (the looping count applies to the register kernels only; the LDS-ring
    kernels and the naive comparator always run one workgroup per item)."""
    kind = layout.split_kernel
    if kind == "lds":
        return "attn_split_lds_kernel (one workgroup per item)"
    if kind == "ldsmfma":
        return "attn_split_lds_mfma_kernel (one workgroup per item)"
    if kind == "naive":
        return "per-query-head split kernel (one wavefront per query head and split)"
    mfma = kind == "mfma"
    if layout.split_waves > 0:
        return "%s (%d wavefronts)" % ("attn_split_mfma_persistent_kernel" if mfma
                                       else "attn_split_persistent_kernel", layout.split_waves)
    return "%s (one wavefront per item)" % ("attn_split_mfma_kernel" if mfma else "attn_split_kernel")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_step_inputs(wl, B):
    """Seeded queries (fp32) and fresh K/V (bf16) for the host-CPU attention comparator."""
    import synth
    d, Hq, Hkv = wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    q = np.stack([synth.normal_f64(wl.seed, 40, b, Hq * d) for b in range(B)]).astype(np.float32)
    kn = np.stack([synth.normal_bf16(wl.seed, 41, b, Hkv * d, 1.0) for b in range(B)])
    vn = np.stack([synth.normal_bf16(wl.seed, 42, b, Hkv * d, 1.0) for b in range(B)])
    return q.reshape(B, Hq, d), kn.reshape(B, Hkv, d), vn.reshape(B, Hkv, d)


def cpu_attention_timed(dkv, r, wl, ctx, threads, reps):
    """Seconds per step (every layer) of the host-CPU attention over r's host
    pages on `threads` threads: one warm-up layer, then the median of `reps`."""
    q, kn, vn = cpu_step_inputs(wl, len(ctx))
    dkv.cpu_attention(r.layout, 0, q, kn, vn, ctx, threads)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        for layer in range(wl.n_layers):
            _, used = dkv.cpu_attention(r.layout, layer, q, kn, vn, ctx, threads)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), used


def cpu_dram_read_GBps(dkv, threads, nbytes=1 << 30):
    """Host-DRAM streaming read by `threads` CPU threads over a fresh pinned buffer."""
    buf = dkv.HostBuffer(nbytes)
    try:
        buf.array[::4096] = 1        # touch every page
        dkv.cpu_stream_read(buf.host_ptr, nbytes, threads)
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            dkv.cpu_stream_read(buf.host_ptr, nbytes, threads)
            times.append(time.perf_counter() - t0)
        return nbytes / float(np.median(times)) / 1e9
    finally:
        buf.free()


def sweep_ctx(dkv, wl, args):
    """Step time against context length at the workload's batch: the method
    (every cached page on the host, read in place), the same KV all in HBM,
    staging (copy the host pool into HBM, then the HBM step) and attention on
    the host CPU next to DRAM. Prints one JSON line with a row per length."""
    import torch
    rows = []
    B = wl.batch
    stream = torch.cuda.current_stream()
    for L in SWEEP_CTX_LENGTHS:
        if L > args.sweep_ctx_max:
            break
        w = wl.replace(ctx=L, ctx_range=None, hbm_tail_tokens=0, hbm_fraction=None)
        ctx = w.ctx_lens()
        kv_bytes = int(ctx.astype(np.int64).sum()) * w.kv_bytes_per_token * w.n_layers

        def kv_source(layer, b, t0, t1):
            return w.kv("k", layer, b, t0, t1), w.kv("v", layer, b, t0, t1)

        steps = max(args.steps, 50) if L <= 8192 else args.steps
        r = Resident(dkv, w, ctx, np.zeros(B, np.int32), kv_source)
        ms_host = r.timed(steps, args.warmup)
        out_host = r.out_bits(0)
        cpu_s, used = cpu_attention_timed(dkv, r, w, ctx, args.cpu_threads, 3)
        rh = Resident(dkv, w, ctx, np.full(B, 1 << 30, np.int32), kv_source)
        ms_hbm = rh.timed(steps, args.warmup)
        same = bool(np.array_equal(out_host, rh.out_bits(0)))
        host_bytes = r.host_pool.info()[1]
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        copy_ms = step_ms = 0.0
        n_cmp = 3
        for i in range(n_cmp + 1):
            e0.record(stream)
            dkv.kv_pool_copy(rh.hbm_pool, r.host_pool, host_bytes, stream)
            e1.record(stream)
            rh.step()
            e2.record(stream)
            torch.cuda.synchronize()
            if i:
                copy_ms += e0.elapsed_time(e1) / n_cmp
                step_ms += e1.elapsed_time(e2) / n_cmp
        rh.free()
        r.free()
        row = {"ctx_tokens": L, "kv_bytes": kv_bytes,
               "zero_copy_ms": round(ms_host, 4), "all_hbm_ms": round(ms_hbm, 4),
               "staging_ms": round(copy_ms + step_ms, 4), "cpu_attention_ms": round(cpu_s * 1e3, 4),
               "zero_copy_GBps": round(kv_bytes / (ms_host * 1e-3) / 1e9, 2),
               "cpu_attention_GBps": round(kv_bytes / cpu_s / 1e9, 2),
               "placements_bit_identical": same}
        rows.append(row)
        log("sweep ctx %d: zero-copy %.3f ms, all-HBM %.3f ms, staging %.3f ms, CPU %.3f ms"
            % (L, ms_host, ms_hbm, copy_ms + step_ms, cpu_s * 1e3))
    print(json.dumps({"sweep": "context_length", "workload": wl.name, "batch": B,
                      "cpu_threads": args.cpu_threads, "cpu_model": cpu_model(), "rows": rows}), flush=True)
    return 0


def multistep(dkv, wl, kv_source, args):
    """Multi-step decode: one HIP graph holding decode_step (every layer) and
    kv_advance, replayed step after step while the contexts grow, on three
    layouts of the same KV: all host pages, a sliding HBM window of the most
    recent --window-tokens tokens per sequence over host pages (kv_advance
    demotes the window's oldest page every 16 tokens), and all HBM pages.
    Prints one JSON line with ms per step and effective KV GB/s of each, and
    whether the host and windowed layouts end with identical bits."""
    import torch
    ctx0 = wl.ctx_lens()
    B = len(ctx0)
    K, W = args.steps, args.warmup
    cap = (ctx0 + K + W + 2).astype(np.int32)
    shape = dkv.Shape.of(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_layers)
    dev = torch.device("cuda", 0)
    xs = [torch.from_numpy(wl.x(layer).view(np.int16)).to(dev).view(torch.bfloat16) for layer in range(wl.n_layers)]
    Ws = [torch.from_numpy(wl.W(layer).view(np.int16)).to(dev).view(torch.bfloat16) for layer in range(wl.n_layers)]
    pages = [int(dkv.kv_placement(int(c), 0)[0]) for c in cap]
    win_pages = -(-args.window_tokens // dkv.PAGE_TOKENS)
    rows, finals = [], {}
    for kind in ("host", "window", "hbm"):
        host = hbm = None
        if kind == "host":
            host = dkv.kv_alloc_host(shape, sum(pages) * wl.n_layers)
            layout = dkv.kv_layout_create(shape, cap, None, host, None)
        elif kind == "window":
            host = dkv.kv_alloc_host(shape, sum(pages) * wl.n_layers)
            hbm = dkv.kv_alloc_hbm(shape, sum(min(p, win_pages) for p in pages) * wl.n_layers)
            layout = dkv.kv_layout_create_windowed(shape, cap, args.window_tokens, ctx0, host, hbm)
        else:
            hbm = dkv.kv_alloc_hbm(shape, sum(pages) * wl.n_layers)
            layout = dkv.kv_layout_create(shape, cap, np.full(B, 1 << 30, np.int32), None, hbm)
        for layer in range(wl.n_layers):
            for b in range(B):
                for t0 in range(0, int(ctx0[b]), CHUNK):
                    t1 = min(int(ctx0[b]), t0 + CHUNK)
                    k, v = kv_source(layer, b, t0, t1)
                    dkv.kv_append(layout, layer, b, t0, k, v)
        ctx = torch.from_numpy(ctx0.copy()).to(dev)
        outs = [torch.empty((B, wl.n_q_heads * wl.head_dim), dtype=torch.bfloat16, device=dev)
                for _ in range(wl.n_layers)]
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for layer in range(wl.n_layers):
                dkv.decode_step(layout, layer, xs[layer], Ws[layer], ctx, outs[layer])
            dkv.kv_advance(layout, ctx)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        for _ in range(W):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        del graph
        layout.check_status()
        assert np.array_equal(ctx.cpu().numpy(), ctx0 + W + K)
        final = dkv.decode_step_f32(layout, 0, xs[0], Ws[0], ctx)
        finals[kind] = final.cpu().numpy().view(np.uint32)
        mean_ctx = ctx0.astype(np.float64) + W + (K - 1) / 2.0
        kv_bytes = float(mean_ctx.sum()) * wl.kv_bytes_per_token * wl.n_layers
        hbm_tokens = 0.0 if kind == "host" else (float(mean_ctx.sum()) if kind == "hbm" else
                                                  float(np.minimum(mean_ctx, args.window_tokens).sum()))
        rows.append({"layout": kind, "ms_per_step": round(ms, 4), "effective_kv_GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
                     "hbm_share_of_kv": round(hbm_tokens / float(mean_ctx.sum()), 4)})
        log("multistep %s: %.4f ms/step" % (kind, ms))
        torch.cuda.synchronize()
        layout.free()
        for p in (host, hbm):
            if p:
                p.free()
    print(json.dumps({"multistep": wl.name, "steps": K, "warmup": W, "window_tokens": args.window_tokens,
                      "graph": "decode_step per layer + kv_advance, replayed once per step", "rows": rows,
                      "window_and_host_bit_identical": bool(np.array_equal(finals["host"], finals["window"])),
                      "hbm_and_host_bit_identical": bool(np.array_equal(finals["host"], finals["hbm"]))}), flush=True)
    return 0


def sweep(dkv, wl, ctx, kv_source, kv_bytes, args):
    """Step time as the host-resident share of the same KV goes from 0 to 1:
    the first round(f * L_b) cached tokens of each sequence on the host, the
    rest (and the new slot) in HBM. Prints one JSON line with a row per share
    and the roofline model T* = max(host bytes / C_host, HBM bytes / 8 TB/s)."""
    B = len(ctx)
    rows = []
    ceiling = None
    for f in SWEEP_HOST_FRACTIONS:
        host_tokens = np.floor(ctx.astype(np.float64) * f).astype(np.int64)
        tail = (ctx.astype(np.int64) + 1 - host_tokens).astype(np.int32)
        r = Resident(dkv, wl, ctx, tail, kv_source)
        host_kv = 0
        for b in range(B):
            n, first = dkv.kv_placement(int(ctx[b]) + 1, int(tail[b]))
            host_kv += min(int(ctx[b]), first * dkv.PAGE_TOKENS) * wl.kv_bytes_per_token
        host_kv *= wl.n_layers
        steps = max(args.steps, 50) if f < 0.05 else args.steps
        ms = r.timed(steps, args.warmup)
        if r.host_pool is not None and r.host_pool.info()[1] >= (256 << 20):
            c, _, _ = probe_ceiling(dkv, r.host_pool, HOST_PROBES[:3])
            ceiling = max(ceiling or 0.0, c)
        r.free()
        rows.append({"host_fraction": f, "host_kv_bytes": host_kv, "ms_per_step": round(ms, 4),
                     "effective_kv_GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 2)})
        log("sweep f=%.2f: %.4f ms/step" % (f, ms))
    for row in rows:
        hb = row["host_kv_bytes"]
        t_star = max(hb / (ceiling * 1e9) if ceiling else 0.0, (kv_bytes - hb) / (HBM_PEAK_GBPS * 1e9))
        row["t_star_ms"] = round(t_star * 1e3, 4)
        row["frac_of_roofline"] = round(t_star * 1e3 / row["ms_per_step"], 4)
    print(json.dumps({"sweep": "host_fraction", "workload": wl.name, "kv_bytes_per_step": kv_bytes,
                      "host_link_ceiling_GBps": round(ceiling, 3) if ceiling else None,
                      "hbm_peak_GBps": HBM_PEAK_GBPS, "rows": rows}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3-70b-b16-ctx131072-8layers-host")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-leg", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="crossover sweep instead of the bench line: the workload's KV with the "
                         "host-resident share stepped from 0 to 100 %% (rest in HBM)")
    ap.add_argument("--multistep", action="store_true",
                    help="multi-step decode from one replayed HIP graph (decode_step + kv_advance) on "
                         "all-host, sliding-window and all-HBM layouts of the workload")
    ap.add_argument("--window-tokens", type=int, default=4096,
                    help="with --multistep: HBM window per sequence (tokens)")
    ap.add_argument("--sweep-ctx", action="store_true",
                    help="context-length sweep instead of the bench line: zero-copy, all-HBM, "
                         "staging and host-CPU attention at the workload's batch")
    ap.add_argument("--sweep-ctx-max", type=int, default=65536,
                    help="with --sweep-ctx: longest context swept (tokens per sequence)")
    ap.add_argument("--cpu-threads", type=int, default=16,
                    help="host threads of the CPU attention comparator and DRAM probe")
    ap.add_argument("--gemm", type=int, default=0, metavar="S",
                    help="host-operand GEMM experiment instead of the bench line: C = A x B^T, "
                         "S x S x S, B in pinned host memory (the pages use S = 10240)")
    ap.add_argument("--gemm-profile", action="store_true",
                    help="with --gemm: run each zero-copy order once and exit (for rocprofv3)")
    ap.add_argument("--gemm-noncoherent", action="store_true",
                    help="with --gemm: allocate B non-coherent (cacheable in the GPU's L2)")
    ap.add_argument("--projection", action="store_true",
                    help="QKV projection experiment instead of the bench line: the projection and "
                         "fresh-token kernels at batches 1-64 (8B and 70B shapes), W read cold, beside "
                         "a cold streaming read of the same bytes")
    ap.add_argument("--proj-batches", default=",".join(map(str, PROJ_BATCHES)),
                    help="with --projection: comma-separated batch sizes")
    ap.add_argument("--proj-shapes", default=",".join(n for n, _, _ in PROJ_SHAPES),
                    help="with --projection: comma-separated shapes (llama3-8b, llama3-70b)")
    ap.add_argument("--no-comparators", action="store_true",
                    help="skip the naive zero-copy and staging comparator legs")
    ap.add_argument("--profile-run", action="store_true",
                    help="only the timed leg in the workload's own placement (for rocprofv3)")
    ap.add_argument("--all-hbm", action="store_true",
                    help="with --profile-run: place every page in HBM instead of the "
                         "workload's own placement")
    ap.add_argument("--split-kernel", choices=("regs", "lds", "mfma", "ldsmfma", "naive"),
                    help="with --profile-run (and --traffic-record): the split kernel to run instead of "
                         "the layout's default (naive: the per-query-head comparator)")
    ap.add_argument("--calibrate", action="store_true",
                    help="with --profile-run: also run kernels of known traffic (a 256 MiB "
                         "HBM-to-HBM copy, 1 GiB streaming reads of the host pool and of HBM) "
                         "to scale counter readings")
    ap.add_argument("--traffic-record", metavar="PREFIX",
                    help="write the split kernel's traffic record under profiles/ from the "
                         "FETCH_SIZE and WRITE_SIZE counter runs in PREFIX_FETCH_SIZE/ and "
                         "PREFIX_WRITE_SIZE/ (host only, no GPU)")
    args = ap.parse_args(argv)
    if args.traffic_record:
        from synth import configs
        return write_traffic_record(configs.BY_NAME[args.workload], args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path runs on one MI355X and this build "
              "launches nothing on a second GPU (--gpus %d is not supported)." % args.gpus,
              file=sys.stderr)
        return 2

    import torch

    import decode_attention_zero_amd as dkv
    from synth import configs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.gemm:
        return gemm_experiment(dkv, args)
    if args.projection:
        return projection_experiment(dkv, args)
    wl = configs.BY_NAME[args.workload]
    if args.sweep_ctx:
        return sweep_ctx(dkv, wl, args)
    ctx = wl.ctx_lens()
    B, Hkv, d = wl.batch, wl.n_kv_heads, wl.head_dim
    tail = wl.hbm_tail(ctx)
    multi = wl.n_layers > 1
    # Layer 0's KV in logical order, for the oracle (the CPU baseline and the
    # parity of this run's own output): drawn once, and layer 0's pages are
    # appended from it; the other layers are drawn chunk by chunk.
    keep = not args.no_cpu_baseline and not args.profile_run and not args.sweep and not args.multistep
    K0 = V0 = None
    if keep:
        log("drawing layer 0's KV of %s" % wl.name)
        Lmax = int(ctx.max())
        K0 = np.zeros((B, Lmax, Hkv, d), np.uint16)
        V0 = np.zeros_like(K0)
        for b in range(B):
            wl.kv("k", 0, b, 0, int(ctx[b]), out=K0[b, :ctx[b]])
            wl.kv("v", 0, b, 0, int(ctx[b]), out=V0[b, :ctx[b]])

    def kv_source(layer, b, t0, t1):
        if layer == 0 and K0 is not None:
            return K0[b, t0:t1], V0[b, t0:t1]
        return wl.kv("k", layer, b, t0, t1), wl.kv("v", layer, b, t0, t1)

    kv_layer_bytes = int(ctx.astype(np.int64).sum()) * wl.kv_bytes_per_token
    kv_bytes = kv_layer_bytes * wl.n_layers
    w_bytes = wl.n_qkv * wl.hidden * 2
    step_bytes = wl.n_layers * (kv_layer_bytes + w_bytes + B * wl.hidden * 2 + B * Hkv * d * 4
                                + B * wl.n_q_heads * d * 2)

    if args.sweep:
        return sweep(dkv, wl, ctx, kv_source, kv_bytes, args)
    if args.multistep:
        return multistep(dkv, wl, kv_source, args)

    # ------------------------------------------------------------------ the workload's placement
    if args.profile_run and args.all_hbm:
        tail = np.full(B, 1 << 30, np.int32)
    log("%s: %s placement leg" % (wl.name, "all-HBM" if args.profile_run and args.all_hbm else "own"))
    r = Resident(dkv, wl, ctx, tail, kv_source)
    if args.split_kernel:
        r.layout.split_kernel = args.split_kernel
    proj_kernel = r.layout.projection_kernel
    host_kv_layer = 0
    for b in range(B):
        n, first = dkv.kv_placement(int(ctx[b]) + 1, int(tail[b]))
        host_tokens = min(int(ctx[b]), first * dkv.PAGE_TOKENS)
        host_kv_layer += host_tokens * wl.kv_bytes_per_token
    host_kv = host_kv_layer * wl.n_layers
    hbm_kv = kv_bytes - host_kv
    # The timed steps also carry the library's events around the split kernel
    # (on the step's stream): its duration behind `roofline.achieved` comes
    # from the timed region itself. The other kernels' times, reported for
    # information, come from a few more steps with events around every kernel.
    ms = r.timed(args.steps, args.warmup, split_events=True)
    step_stats = r.step_stats
    kt = dict(r.kernel_times(max(1, min(args.steps, 2 if multi else 5))), split=r.kernel_ms["split"])
    # The graph replay: every step of a one-layer workload again; a few steps
    # of a multi-layer one (each is 8 layers).
    n_aux = args.steps if not multi else max(1, min(args.steps, 3))
    if args.profile_run:
        if args.calibrate:
            calibrate(dkv, r)
        label = split_kernel_label(r.layout)
        r.free()
        print(json.dumps({"profile_run": True, "workload": wl.name, "all_hbm": bool(args.all_hbm),
                          "split_kernel": label, "ms_per_step": ms, "kernel_ms": kt}), flush=True)
        return 0
    ms_graph = r.graph_timed(n_aux)
    out_own = r.out_bits(0)
    split_kernel_name = split_kernel_label(r.layout)
    ceiling = ceiling_rows = probe_bytes = None
    if r.host_pool is not None:
        # On at least 4 GiB of pinned memory: the pool itself when it is that
        # large (a second pinned buffer beside a 64 GiB pool is refused on these
        # hosts), else a fresh 4 GiB buffer allocated like the pool.
        if r.host_pool.info()[1] >= HOST_PROBE_BYTES:
            ceiling, ceiling_rows, probe_bytes = probe_ceiling(dkv, r.host_pool, HOST_PROBES)
        else:
            ceiling, ceiling_rows, probe_bytes = probe_host_link(dkv, HOST_PROBES)
    log("own placement: %.3f ms/step, split kernel %.3f ms; host-link ceiling %.2f GB/s"
        % (ms, kt["split"], ceiling or 0.0))
    # A launch that reads only a few MiB over the link cannot reach the
    # ceiling of a long read (the link's latency and ramp weigh): for such
    # layers, also the best streaming read of the same number of bytes.
    small_ceiling = None
    if r.host_pool is not None and 0 < host_kv_layer < SMALL_READ_BYTES:
        nb = -(-host_kv_layer // (1 << 20)) * (1 << 20)
        buf = dkv.HostBuffer(nb)
        try:
            best = max(nb / dkv.probe_stream_read(buf.device_ptr, nb, grid, unroll, reps=21) / 1e6
                       for grid, unroll in HOST_PROBES)
        finally:
            buf.free()
        small_ceiling = {"bytes": nb, "GBps": round(best, 2),
                         "split_kernel_vs": round(host_kv_layer / (kt["split"] / wl.n_layers * 1e-3) / 1e9 / best, 4)}

    value = kv_bytes / (ms * 1e-3) / 1e9
    split_gbps = kv_bytes / (kt["split"] * 1e-3) / 1e9
    method_traffic = counter_traffic(wl.name)

    # ------------------------------------------------------------------ comparator: naive zero-copy
    comparators = {}
    if r.host_pool is not None and not args.no_comparators:
        default_kernel = r.layout.split_kernel
        r.layout.split_kernel = "naive"
        if multi:
            r.step(layers=[0])             # warm-up: one layer
            ms_n = r.timed(1, 0)
        else:
            ms_n = r.timed(max(1, min(args.steps, 5)), 1)
        out_naive = r.out_bits(0)
        r.layout.split_kernel = default_kernel
        naive_traffic = counter_traffic(wl.name, kernel="naive")
        per_step = lambda t: None if t is None else int(t * wl.n_layers)

        def link_reads(rec):
            routes = (rec or {}).get("l2_read_routes")
            return None if not routes else routes["host_link_read_bytes_per_dispatch"] * wl.n_layers

        naive_rec, method_rec = counter_record(wl.name, kernel="naive"), counter_record(wl.name)
        naive = {
            "what": "one work item per query head: each KV head's pages requested once per query "
                    "head of its group (%dx the bytes the grouped kernel requests)" % wl.group,
            "ms_per_step": round(ms_n, 4),
            "effective_kv_GBps": round(kv_bytes / (ms_n * 1e-3) / 1e9, 3),
            "requested_bytes_per_step": host_kv * wl.group + hbm_kv * wl.group,
            "link_bytes_bound_per_step": int(ceiling * 1e9 * ms_n * 1e-3) if ceiling else None,
            "counter_bytes_per_step": per_step(naive_traffic),
            "method_counter_bytes_per_step": per_step(method_traffic),
            "host_link_read_bytes_per_step": link_reads(naive_rec),
            "method_host_link_read_bytes_per_step": link_reads(method_rec),
            "l2_hit_rate": ((naive_rec or {}).get("l2_read_routes") or {}).get("l2_hit_rate"),
            "step_time_vs_method": round(ms_n / ms, 3),
            "bit_identical_to_method": bool(np.array_equal(out_own, out_naive)),
        }
        if naive_traffic and method_traffic:
            naive["method_transfer_vs_naive"] = round(method_traffic / naive_traffic, 4)
            naive["pages_claim"] = "up to 50% less CPU-GPU transfer than naive zero-copy (GH200)"
        if link_reads(naive_rec) and link_reads(method_rec):
            naive["method_host_link_reads_vs_naive"] = round(link_reads(method_rec) / link_reads(naive_rec), 4)
        comparators["naive_zero_copy"] = naive
        log("naive zero-copy: %.3f ms/step" % ms_n)

    # ------------------------------------------------------------------ comparator: attention on the CPU
    if r.host_pool is not None and r.hbm_pool is None and not args.no_comparators:
        cpu_s, used = cpu_attention_timed(dkv, r, wl, ctx, args.cpu_threads, 3 if not multi else 1)
        dram = cpu_dram_read_GBps(dkv, args.cpu_threads)
        comparators["cpu_attention"] = {
            "what": "attention computed by host threads reading the same host pages in place "
                    "(next to DRAM, no link transfer), fp32; projection and write-back not included",
            "threads": used,
            "cpu_model": cpu_model(),
            "ms_per_step": round(cpu_s * 1e3, 4),
            "effective_kv_GBps": round(kv_bytes / cpu_s / 1e9, 3),
            "host_dram_read_GBps": round(dram, 2),
            "step_time_vs_method": round(cpu_s * 1e3 / ms, 3),
        }
        log("CPU attention (%d threads): %.3f ms/step; host DRAM read %.1f GB/s" % (used, cpu_s * 1e3, dram))

    # ------------------------------------------------------------------ every page in HBM
    hbm = None
    if not args.no_hbm_leg:
        log("HBM-placement leg")
        all_host = r.hbm_pool is None
        rh = Resident(dkv, wl, ctx, np.full(B, 1 << 30, np.int32), kv_source, copy_from=r if all_host else None)
        n_hbm_steps = max(args.steps, 50) if not multi else args.steps
        ms_h = rh.timed(n_hbm_steps, args.warmup)
        kt_h = rh.kernel_times(n_hbm_steps)
        ms_h_graph = rh.graph_timed(n_hbm_steps)
        hbm_ceiling, hbm_rows, _ = probe_ceiling(dkv, rh.hbm_pool, HBM_PROBES)
        page_ceiling, page_rows = probe_page_runs(dkv, rh.hbm_pool, wl)
        out_hbm = rh.out_bits(0)
        hbm_split_gbps = kv_bytes / (kt_h["split"] * 1e-3) / 1e9
        hbm = {
            "roofline": {"bound": "hbm", "kernel": split_kernel_label(rh.layout),
                         "achieved": round(hbm_split_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(hbm_split_gbps / HBM_PEAK_GBPS, 4),
                         "traffic": counter_traffic(wl.name, all_hbm=True)},
            "kv_filled_by": "copy-engine copy of the host pool" if all_host else "the generator",
            "ms_per_step": round(ms_h, 4),
            "graph_ms_per_step": round(ms_h_graph, 4),
            "kv_GBps": round(kv_bytes / (ms_h * 1e-3) / 1e9, 1),
            "split_kernel_ms": round(kt_h["split"], 4),
            "split_kernel_GBps": round(kv_bytes / (kt_h["split"] * 1e-3) / 1e9, 1),
            "split_kernel_frac_of_8TBps": round(kv_bytes / (kt_h["split"] * 1e-3) / 1e9
                                                / HBM_PEAK_GBPS, 4),
            "kernel_ms": {k: round(v, 4) for k, v in kt_h.items()},
            "projection": projection_facts(wl, kt_h["projection"], proj_kernel),
            "measured_hbm_read_GBps": round(hbm_ceiling, 1),
            "hbm_probe": hbm_rows,
            "page_run_read_GBps": round(page_ceiling, 1) if page_rows else None,
            "split_kernel_vs_page_run_read": (round(hbm_split_gbps / page_ceiling, 4) if page_rows else None),
            "page_run_probe": page_rows,
            "bit_identical_to_own_placement": bool(np.array_equal(out_own, out_hbm)),
        }
        log("HBM leg: %.4f ms/step, split kernel %.1f GB/s" % (ms_h, hbm["split_kernel_GBps"]))

        # -------------------------------------------------------------- the HBM window alone
        if host_kv > 0 and hbm_kv > 0 and not args.no_comparators:
            hbm["window_only"] = window_only_leg(dkv, wl, ctx, tail, kv_source, args)

        # -------------------------------------------------------------- comparator: staging
        if r.hbm_pool is None and r.host_pool is not None and not args.no_comparators:
            stream = torch.cuda.current_stream()
            host_bytes = r.host_pool.info()[1]
            n_cmp = max(1, min(args.steps, 5)) if not multi else 1
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            copy_ms = step_ms = 0.0
            for i in range(n_cmp + 1):
                e0.record(stream)
                dkv.kv_pool_copy(rh.hbm_pool, r.host_pool, host_bytes, stream)
                e1.record(stream)
                rh.step()
                e2.record(stream)
                torch.cuda.synchronize()
                if i:      # the first round warms up
                    copy_ms += e0.elapsed_time(e1) / n_cmp
                    step_ms += e1.elapsed_time(e2) / n_cmp
            out_staged = rh.out_bits(0)
            comparators["staging"] = {
                "what": "copy-engine copy of the host pool into an HBM buffer of the same size "
                        "(hipMemcpyAsync), then the decode step on the HBM copy",
                "ms_per_step": round(copy_ms + step_ms, 4),
                "copy_ms": round(copy_ms, 4),
                "copy_GBps": round(host_bytes / (copy_ms * 1e-3) / 1e9, 2),
                "decode_ms": round(step_ms, 4),
                "effective_kv_GBps": round(kv_bytes / ((copy_ms + step_ms) * 1e-3) / 1e9, 3),
                "extra_hbm_bytes": host_bytes,
                "step_time_vs_method": round((copy_ms + step_ms) / ms, 3),
                "bit_identical_to_method": bool(np.array_equal(out_own, out_staged)),
            }
            log("staging: copy %.3f ms + step %.3f ms" % (copy_ms, step_ms))
        rh.free()
    r.free()

    # ------------------------------------------------------------------ CPU oracle
    cpu = None
    parity = None
    if K0 is not None:
        import oracle
        orc = oracle.default()
        threads = oracle.DEFAULT_THREADS
        x0, W0 = wl.x(0), wl.W(0)
        # A one-layer workload: whole steps, repeated until about 10 s (at
        # least one, at most 200). A multi-layer one: one whole layer (layer 0,
        # every sequence and query head), the same work as each other layer.
        reps, t_cpu, ref = 0, 0.0, None
        while reps == 0 or (not multi and t_cpu < 10.0 and reps < 200):
            t0 = time.perf_counter()
            out = orc.decode_step(x0, W0, ctx, K0, V0, wl.n_q_heads, Hkv, d, threads=threads)
            t_cpu += time.perf_counter() - t0
            ref = ref or out
            reps += 1
        log("oracle on %d threads: %d x layer 0 in %.2f s" % (threads, reps, t_cpu))
        layer_s = t_cpu / reps
        cpu = {"value": round(kv_layer_bytes * reps / t_cpu / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "seconds": round(t_cpu, 2),
               "ms_per_step": round(layer_s * wl.n_layers * 1e3, 2),
               "sample": ("%d full step(s) of the bench workload (all %d sequences x %d query heads, "
                          "%d KV bytes each), fp64, plain C + OpenMP" % (reps, B, wl.n_q_heads, kv_bytes))
               if not multi else
               ("layer 0 of the %d, whole (all %d sequences x %d query heads over %d KV bytes), fp64, plain "
                "C + OpenMP; every layer is the same work, so ms_per_step is %d x that layer"
                % (wl.n_layers, B, wl.n_q_heads, kv_layer_bytes, wl.n_layers))}
        got = (out_own.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        err = np.abs(got - ref["attn_out"])
        worst = np.unravel_index(int(np.argmax(err)), err.shape)
        parity = {"scope": ("whole attn_out" if not multi else
                            "whole attn_out of layer 0 (%d x %d)" % (B, wl.n_q_heads * d)),
                  "max_abs": float(err.max()),
                  "rel_l2": float(np.linalg.norm(got - ref["attn_out"]) / np.linalg.norm(ref["attn_out"])),
                  "worst": {"seq": int(worst[0]), "q_head": int(worst[1]) // d},
                  "gates": {"max_abs": 2e-2, "rel_l2": 5e-3}}
        parity["within_gates"] = parity["max_abs"] <= 2e-2 and parity["rel_l2"] <= 5e-3

    t_star = max(host_kv / (ceiling * 1e9) if ceiling else 0.0, hbm_kv / (HBM_PEAK_GBPS * 1e9))
    # The same two streams one after the other (the serial reading of the combined roofline).
    t_serial = (host_kv / (ceiling * 1e9) if ceiling else 0.0) + hbm_kv / (HBM_PEAK_GBPS * 1e9)
    placement = ("100% host-pinned, read in place" if hbm_kv == 0 else
                 "%.1f%% host-pinned (read in place) / %.1f%% HBM" %
                 (100.0 * host_kv / kv_bytes, 100.0 * hbm_kv / kv_bytes))
    result = {
        "metric": "effective KV GB/s per decode step (% of host-link+HBM roofline); step latency",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": step_stats,
        "graph_ms_per_step": round(ms_graph, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "layers": wl.n_layers,
                   "ctx_tokens": int(ctx[0]) if wl.ctx_range is None else list(wl.ctx_range),
                   "hidden": wl.hidden, "q_heads": wl.n_q_heads, "kv_heads": Hkv,
                   "head_dim": d, "kv_placement": placement,
                   "kv_bytes_per_step": kv_bytes, "host_kv_bytes_per_step": host_kv,
                   "algorithmic_bytes_per_step": step_bytes},
        "roofline": {"bound": "host_link", "kernel": split_kernel_name,
                     "achieved": round(split_gbps, 3), "peak": PCIE_GEN5_X16_GBPS,
                     "unit": "GB/s", "frac": round(split_gbps / PCIE_GEN5_X16_GBPS, 4),
                     "traffic": method_traffic,
                     "bytes_per_launch": kv_layer_bytes,
                     "measured_ceiling_GBps": round(ceiling, 3) if ceiling else None,
                     "ceiling_probe_bytes": probe_bytes,
                     "frac_of_measured_ceiling": round(split_gbps / ceiling, 4) if ceiling else None,
                     "same_size_read_ceiling": small_ceiling,
                     "host_GBps_vs_ceiling": round(host_kv / (kt["split"] * 1e-3) / 1e9 / ceiling, 4)
                     if ceiling else None,
                     "split_kernel_ms": round(kt["split"], 4)},
        "combined_roofline": {"t_star_ms": round(t_star * 1e3, 4),
                              "frac": round(t_star * 1e3 / ms, 4) if t_star else None,
                              "serial_ms": round(t_serial * 1e3, 4),
                              "frac_of_serial": round(t_serial * 1e3 / ms, 4) if t_serial else None},
        "kernel_ms": {k: round(v, 4) for k, v in kt.items()},
        "projection": projection_facts(wl, kt["projection"], proj_kernel),
        "host_link_probe": ceiling_rows,
        "hbm_placement": hbm,
        "comparators": comparators,
        "parity": parity,
        "cpu_baseline": cpu,
        "host": host_facts(),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
