#!/usr/bin/env python3
"""Paged <-> chunk KV gather/scatter throughput on one MI355X.

Default workload (the headline): Llama-3.1-8B KV shape (32 layers, 8 KV
heads, head_dim 128, bf16), 16-token pages in an 8192-page pool, 8 sequences
of 10000 tokens.  One step = one batched store (gather of all 8 x 40 chunks,
one launch) + one batched retrieve with the first 30 chunks of each sequence
hit (one launch).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  `value` = algorithmic bytes moved per step (every
payload byte read once and written once) / step time, in GB/s (1e9).
`roofline` is for the dominant kernel (the gather), timed with HIP events on
the stream it is launched on.  `cpu_baseline` times the CPU oracle on the
same workload's data on this host's cores.

Other workloads (`--workload layerwise-8b | layerwise-store-8b |
llama-70b-style | llama3.1-8b-tp8-share | fp8-8b | e5m2-8b | k16v8-8b |
cachegen-8b | offload-8b`) print their own JSON report line; they are not the
headline.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor peak
PCIE_PEAK_GBPS = 63.0           # PCIe 5.0 x16 host link, one direction, after 128b/130b coding
METRIC = "paged<->chunk KV gather/scatter GB/s and % of HBM peak (8B KV shape)"
# device sources of the gather kernel (kernel, launch shape, shared helpers)
KERNEL_SOURCES = ["paged_kv_movement_amd/csrc/kv_common.hpp", "paged_kv_movement_amd/csrc/kv_move_bf16.hpp"]
TRAFFIC_FILE = "profiles/hbm_traffic_gather_llama8b.txt"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per gather launch from the committed rocprofv3 counter
    summary, if it was taken on the kernel sources as they are now."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ setup

def chunk_plan(paged, seq, fmt):
    """Sizes of a sequence's chunks from the library (tokens per chunk: the
    last one holds the remainder)."""
    n = paged.num_chunks(seq.tok_start, seq.tok_end)
    toks = [min(paged.chunk_size, seq.tok_end - seq.tok_start - c * paged.chunk_size) for c in range(n)]
    return [paged.chunk_bytes(t, fmt) for t in toks]


def setup(w, fmt, where="device", pool=None):
    """Device pool (made here unless given), chunk buffers carved from one
    arena in device memory or, for where="host", in pinned host memory."""
    import numpy as np
    import torch
    import paged_kv_movement_amd as kvm
    from paged_kv_movement_amd import workloads as wl

    t = time.time()
    if pool is None:
        pool = wl.device_pool(w)
    paged = kvm.Paged.from_pool(pool, chunk_size=w.chunk_size)
    sizes = [chunk_plan(paged, sq, fmt) for sq in w.seqs]
    align = 256
    total = sum(-(-s // align) * align for ss in sizes for s in ss)
    if where == "host":
        arena = torch.empty(total, dtype=torch.uint8, pin_memory=True)
    else:
        arena = torch.empty(total, dtype=torch.uint8, device="cuda")
    base, at, seqs = arena.data_ptr(), 0, []
    for sq, ss in zip(w.seqs, sizes):
        addrs = []
        for s in ss:
            addrs.append(base + at)
            at += -(-s // align) * align
        bt = torch.from_numpy(np.ascontiguousarray(sq.block_table, np.int32)).cuda()
        seqs.append(kvm.Seq(bt, sq.tok_start, sq.tok_end,
                            torch.tensor(addrs, dtype=torch.int64).cuda()))
    batch = kvm.Batch(paged, seqs).set_masks([sq.hit_mask for sq in w.seqs])
    torch.cuda.synchronize()
    log(f"setup {w.name}: pool {pool.numel() * 2 / 1e9:.2f} GB, chunks {total / 1e9:.2f} GB in {where} "
        f"memory, {time.time() - t:.1f} s")
    return pool, paged, batch, arena


def kv_bytes_per_token(w):
    return w.num_layers * 2 * w.width * 2


def hit_tokens(w):
    out = []
    for sq in w.seqs:
        n_hit = 0
        while n_hit < len(sq.hit_mask) and sq.hit_mask[n_hit]:
            n_hit += 1
        out.append(min(sq.tok_end, sq.tok_start + n_hit * w.chunk_size) - sq.tok_start)
    return out


def timed(stream, fn, reps, warmup=3, stat="median"):
    """ms of fn() over reps (the median, or the mean with stat="mean"), HIP
    events on `stream`, after `warmup` untimed calls (short launches otherwise
    pay for the first calls' setup)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return median(ms) if stat == "median" else sum(ms) / reps


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


# ------------------------------------------------------------------ CPU baseline

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, pool, min_s=10.0, budget_s=20.0, max_threads=16, min_threaded_s=1.0):
    """The oracle, as it stands, on this host: store + retrieve of the
    workload's sequences one after another, cycling over them until at least
    min_s of CPU time (and stopping at budget_s), single-threaded; then the
    same calls for every sequence spread over threads, one (sequence, layer)
    pair per task (the oracle's one-layer form; ctypes lets the calls run
    concurrently, and the pairs touch disjoint bytes), repeated for at least
    min_threaded_s."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    t = time.time()
    arr = pool.view(__import__("torch").int16).cpu().numpy().view(np.uint16).reshape(
        w.num_layers, 2, w.num_pages, w.page_size, w.width)
    opool = oracle.Pool.from_array(arr, w.num_kv_heads, w.head_dim, w.chunk_size)
    log(f"cpu baseline: pool copied to host in {time.time() - t:.1f} s")
    n_seqs = len(w.seqs)
    moved, secs, runs = 0, 0.0, 0
    seq_bytes = {}
    while secs < min_s and secs < budget_s:
        i = runs % n_seqs
        sq = w.seqs[i]
        ch = oracle.alloc_chunks(opool, sq.tok_start, sq.tok_end, oracle.FMT_BF16)
        t0 = time.perf_counter()
        assert oracle.store(opool, sq.block_table, sq.tok_start, sq.tok_end, ch) == 0
        n = oracle.retrieve(opool, sq.block_table, sq.tok_start, sq.tok_end, sq.hit_mask, ch)
        secs += time.perf_counter() - t0
        seq_bytes[i] = 2 * ((sq.tok_end - sq.tok_start) + n) * kv_bytes_per_token(w)
        moved += seq_bytes[i]
        runs += 1
        del ch
    out = {"value": round(moved / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"store + retrieve (30-chunk hit mask) of the workload's sequences one at a time, "
                     f"{runs} sequence calls cycling over its {n_seqs} ({moved / 1e9:.2f} GB moved in "
                     f"{secs:.1f} s, single thread)",
           "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}

    threads = max(1, min(max_threads, os.cpu_count() or 1))
    done = min(runs, n_seqs)
    seqs = w.seqs[:done]
    chunks = [oracle.alloc_chunks(opool, sq.tok_start, sq.tok_end, oracle.FMT_BF16) for sq in seqs]

    def pair(job):
        i, l = job
        sq = seqs[i]
        assert oracle.store(opool, sq.block_table, sq.tok_start, sq.tok_end, chunks[i], oracle.FMT_BF16, l) == 0
        return oracle.retrieve(opool, sq.block_table, sq.tok_start, sq.tok_end, sq.hit_mask, chunks[i],
                               oracle.FMT_BF16, l)

    jobs = [(i, l) for i in range(len(seqs)) for l in range(w.num_layers)]
    per_layer = w.num_kv_heads * w.head_dim * 2 * 2
    secs_mt, moved_mt, passes = 0.0, 0, 0
    with ThreadPoolExecutor(threads) as ex:
        while secs_mt < min_threaded_s:
            t0 = time.perf_counter()
            hit = list(ex.map(pair, jobs))
            secs_mt += time.perf_counter() - t0
            one_pass = sum(2 * ((seqs[i].tok_end - seqs[i].tok_start) + n) * per_layer
                           for (i, _), n in zip(jobs, hit))
            assert one_pass == sum(seq_bytes[i] for i in range(done))
            moved_mt += one_pass
            passes += 1
    out["threaded"] = {"value": round(moved_mt / secs_mt / 1e9, 4), "unit": "GB/s", "cores": threads,
                       "kind": "oracle",
                       "sample": f"the first {done} sequences, {len(jobs)} (sequence, layer) tasks on {threads} "
                                 f"threads, {passes} passes ({moved_mt / 1e9:.2f} GB in {secs_mt:.2f} s)"}
    del chunks, arr, opool
    return out


def oracle_beside(w, pool, fmt, n_chunks=4, bins=None, layer=-1, budget_s=4.0):
    """The oracle timed beside a non-headline workload: store, then retrieve
    (all hit), of the first n_chunks chunks of the first sequence, repeated
    for about budget_s, single-threaded.  It runs on a host copy of only
    those chunks' pages, renumbered from 0 (what moves does not depend on
    page ids).  Bytes are counted as on the GPU side of the same workload."""
    import numpy as np
    import torch
    import oracle
    sq = w.seqs[0]
    s = sq.tok_start
    e = min(sq.tok_end, s + n_chunks * w.chunk_size)
    first = s // w.page_size
    pages = np.asarray(sq.block_table[first:(e + w.page_size - 1) // w.page_size], np.int64)
    full = pool.view(torch.int16).view(w.num_layers, 2, w.num_pages, w.page_size, w.width)
    part = full.index_select(2, torch.from_numpy(pages).to(pool.device)).cpu().numpy().view(np.uint16).copy()
    opool = oracle.Pool.from_array(part, w.num_kv_heads, w.head_dim, w.chunk_size)
    bt = np.concatenate([np.zeros(first, np.int32), np.arange(len(pages), dtype=np.int32)])
    ch = oracle.alloc_chunks(opool, s, e, fmt)
    mask = np.ones(len(ch), np.uint8)
    layers = 1 if layer >= 0 else w.num_layers
    elems = (e - s) * layers * w.width
    if fmt == oracle.FMT_CACHEGEN:
        nbytes = elems * 2 * 3 + (e - s) * layers * 2 * 4
    else:
        pb = PART_BYTES[fmt]
        nbytes = elems * sum(2 + b for b in pb) + 4 * sum(b == 1 for b in pb) * layers * len(ch)
    t_st = t_rt = 0.0
    reps = 0
    while reps == 0 or t_st + t_rt < budget_s:
        t0 = time.perf_counter()
        if fmt == oracle.FMT_CACHEGEN:
            assert oracle.store_cachegen(opool, bt, s, e, ch, bins[0], bins[1]) == 0
            t1 = time.perf_counter()
            assert oracle.retrieve_cachegen(opool, bt, s, e, mask, ch, bins[0], bins[1]) == e - s
        else:
            assert oracle.store(opool, bt, s, e, ch, fmt, layer) == 0
            t1 = time.perf_counter()
            assert oracle.retrieve(opool, bt, s, e, mask, ch, fmt, layer) == e - s
        t2 = time.perf_counter()
        t_st, t_rt, reps = t_st + t1 - t0, t_rt + t2 - t1, reps + 1
    return {"store_GBps": round(reps * nbytes / t_st / 1e9, 4), "retrieve_GBps": round(reps * nbytes / t_rt / 1e9, 4),
            "store_tokens_per_s": round(reps * (e - s) / t_st, 1),
            "retrieve_tokens_per_s": round(reps * (e - s) / t_rt, 1), "cores": 1, "kind": "oracle",
            "sample": f"{reps} x (store + retrieve) of {len(ch)} chunks, {e - s} tokens"
                      f"{', layer ' + str(layer) if layer >= 0 else ''}, of the same workload, single thread"}


# ------------------------------------------------------------------ workloads

def bench_llama8b(args):
    import torch
    import paged_kv_movement_amd as kvm
    from paged_kv_movement_amd import workloads as wl

    w = wl.llama8b()
    pool, paged, batch, arena = setup(w, kvm.FMT_BF16)
    stream = torch.cuda.Stream()
    bpt = kv_bytes_per_token(w)
    store_tokens = sum(sq.tok_end - sq.tok_start for sq in w.seqs)
    ret_tokens = sum(hit_tokens(w))
    store_bytes = 2 * store_tokens * bpt
    ret_bytes = 2 * ret_tokens * bpt

    # the retrieve visits its pages in pool-address order (kv_retrieve_chunks_ws)
    # unless --retrieve-order chunk asks for the chunk-major kv_retrieve_chunks;
    # the store gathers through its address plan (kv_store_chunks_ws) unless
    # --store-plan off asks for kv_store_chunks
    ws = paged.new_workspace() if args.retrieve_order == "address" else None
    sws = batch.new_store_workspace() if args.store_plan == "on" else None

    def store():
        kvm.store(paged, batch, stream=stream, workspace=sws)

    def retrieve():
        kvm.retrieve(paged, batch, stream=stream, workspace=ws)

    for _ in range(args.warmup):
        store()
        retrieve()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        store()
        ev[i][1].record(stream)
        ev[i][2].record(stream)
        retrieve()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert kvm.take_faults() == 0

    step_s = (t1 - t0) / K
    store_each = [e[0].elapsed_time(e[1]) for e in ev]
    ret_each = [e[2].elapsed_time(e[3]) for e in ev]
    store_ms = sum(store_each) / K
    ret_ms = sum(ret_each) / K
    value = (store_bytes + ret_bytes) / step_s / 1e9
    gather_gbps = store_bytes / (store_ms / 1e3) / 1e9
    scatter_gbps = ret_bytes / (ret_ms / 1e3) / 1e9

    # the other visiting order and the other store form, for context
    other_ms = timed(stream, lambda: kvm.retrieve(paged, batch, stream=stream,
                                                  workspace=None if ws is not None else paged.new_workspace()), 5)
    other_store_ms = timed(stream, lambda: kvm.store(paged, batch, stream=stream,
                                                     workspace=None if sws is not None else
                                                     batch.new_store_workspace()), 5)
    assert kvm.take_faults() == 0

    # same-run calibration: a plain contiguous copy of the gather's payload
    src = pool.view(-1).view(torch.uint8)
    n = (store_bytes // 2) // 16 * 16
    copy_ms = timed(stream, lambda: kvm.copy_bytes(arena, src, n, stream=stream), 5)
    copy_gbps = 2 * n / (copy_ms / 1e3) / 1e9
    # and the same copy with one side in page-sized blocks visited in a
    # scattered order: the access pattern of the gather (scattered reads) and
    # of the chunk-major scatter (scattered writes), with no block table
    page_bytes = w.page_size * w.width * 2
    nb = n // page_bytes * page_bytes
    scat = {}
    for name, side in (("reads", kvm.COPY_SCATTERED_READS), ("writes", kvm.COPY_SCATTERED_WRITES)):
        t = timed(stream, lambda: kvm.copy_blocks(arena, src, nb, page_bytes, side, stream=stream), 5)
        scat[name] = 2 * nb / (t / 1e3) / 1e9
    log(f"store {store_ms:.3f} ms ({gather_gbps:.0f} GB/s), retrieve {ret_ms:.3f} ms "
        f"({scatter_gbps:.0f} GB/s), step {step_s * 1e3:.3f} ms, copy ceiling {copy_gbps:.0f} GB/s "
        f"(scattered {page_bytes // 1024} KiB reads {scat['reads']:.0f}, writes {scat['writes']:.0f})")

    traffic = read_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3.1-8b KV shape: 8 seqs x 10000 tokens, batched store + retrieve "
                        "with 30 of 40 chunks hit",
            "layers": w.num_layers, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "page_tokens": w.page_size, "chunk_tokens": w.chunk_size, "pool_pages": w.num_pages,
            "seqs": len(w.seqs), "tokens_per_seq": 10000, "hit_chunks": 30,
            "bytes_per_step": store_bytes + ret_bytes,
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
            "tokens_per_s": round((store_tokens + ret_tokens) / step_s, 1),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("kvmove::gather_planned (gather; the store call, its plan kernel included)"
                       if sws is not None else "kvmove::move_bf16<true,...> (gather)"),
            "achieved": round(gather_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gather_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": store_bytes,
            "avg_launch_ms": round(store_ms, 4),
        },
        "detail": {
            "store_ms": round(store_ms, 4), "store_GBps": round(gather_gbps, 2),
            "retrieve_ms": round(ret_ms, 4), "retrieve_GBps": round(scatter_gbps, 2),
            # the median over the K timed steps (after the W warm-up steps)
            "store_ms_median": round(median(store_each), 4),
            "store_GBps_median": round(store_bytes / (median(store_each) / 1e3) / 1e9, 2),
            "retrieve_ms_median": round(median(ret_each), 4),
            "retrieve_GBps_median": round(ret_bytes / (median(ret_each) / 1e3) / 1e9, 2),
            "retrieve_order": "pool-address (kv_retrieve_chunks_ws)" if ws is not None
                              else "chunk-major (kv_retrieve_chunks)",
            "retrieve_other_order_ms": round(other_ms, 4),
            "retrieve_other_order_GBps": round(ret_bytes / (other_ms / 1e3) / 1e9, 2),
            "store_form": "address plan (kv_store_chunks_ws)" if sws is not None else "kv_store_chunks",
            "store_other_form_ms": round(other_store_ms, 4),
            "store_other_form_GBps": round(store_bytes / (other_store_ms / 1e3) / 1e9, 2),
            "copy_ceiling_GBps": round(copy_gbps, 2),
            "copy_scattered_reads_GBps": round(scat["reads"], 2),
            "copy_scattered_writes_GBps": round(scat["writes"], 2),
            "gather_frac_of_scattered_read_copy": round(gather_gbps / scat["reads"], 4),
            # HBM bytes the counters measured for one gather launch, over this run's launch time
            "gather_counter_GBps": (round(traffic / (store_ms / 1e3) / 1e9, 2) if traffic else None),
            "kernel_source_sha256_16": kernel_source_hash(),
        },
    }
    if not args.no_cpu_baseline:
        del arena
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(w, pool)
    return out


def bench_layers_only(args, store):
    """The 32 layer-by-layer scatters (store=False) or gathers (store=True) of
    the layerwise workload alone, no compute beside them: one call for all
    layers (kv_retrieve_layers / kv_store_layers) with every layer's grid
    capped at --layers-only workgroups (0: one per tile), repeated --steps
    times.  For kernel traces of one launch shape at a time."""
    import torch
    import paged_kv_movement_amd as kvm
    from paged_kv_movement_amd import workloads as wl

    w = wl.layerwise8b()
    pool, paged, batch, arena = setup(w, kvm.FMT_BF16)
    kvm.store(paged, batch)
    torch.cuda.synchronize()
    copy = torch.cuda.Stream()
    alt = torch.cuda.Stream() if args.alt_stream else None
    L, cap = w.num_layers, args.layers_only
    per_layer_bytes = 2 * 10240 * 2 * w.width * 2
    if store:
        def run():
            kvm.store_layers(paged, batch, 0, L, stream=copy, max_workgroups=[cap] * L, alt_stream=alt)
    else:
        def run():
            kvm.retrieve_layers(paged, batch, 0, L, stream=copy, max_workgroups=[cap] * L, alt_stream=alt)
    ms = timed(copy, run, max(3, args.steps), warmup=args.warmup, stat="median")
    assert kvm.take_faults() == 0
    return {"metric": f"layer {'gather' if store else 'scatter'} alone, 32 layers per call",
            "workload": "layerwise-8b: 1 seq x 10240 tokens, 32 layers", "max_workgroups": cap,
            "streams": 2 if alt is not None else 1,
            "calls": max(3, args.steps), "ms_per_32_layers_median": round(ms, 4),
            "layer_ms": round(ms / L, 4), "layer_GBps": round(per_layer_bytes / (ms / L / 1e3) / 1e9, 2)}


def bench_layerwise(args):
    """32 layer-by-layer scatters on a copy stream, each gating a bf16 GEMM
    (10240 x 4096 x 4096) on a compute stream.  Ways to enqueue the
    scatters: one call per layer (kv_retrieve_layer_ex, as an engine calling
    wait/load per layer does), either all at once or paced so that layer
    i+1's scatter starts with layer i's GEMM (the copy stream waits on an
    event the compute stream records before each GEMM); one call for all
    layers (kv_retrieve_layers, the start of the whole load at once), on one
    stream or two.  Each for several caps on the scatter's workgroups (0 =
    one per tile)."""
    import numpy as np
    import torch
    import paged_kv_movement_amd as kvm
    from paged_kv_movement_amd import workloads as wl

    w = wl.layerwise8b()
    pool, paged, batch, arena = setup(w, kvm.FMT_BF16)
    kvm.store(paged, batch)
    torch.cuda.synchronize()
    copy, compute = torch.cuda.Stream(), torch.cuda.Stream()
    x = torch.randn(10240, 4096, device="cuda", dtype=torch.bfloat16)
    wgt = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16) * 0.01
    L = w.num_layers
    events = [torch.cuda.Event() for _ in range(L)]
    per_layer_bytes = 2 * 10240 * 2 * w.width * 2

    def gemms():
        with torch.cuda.stream(compute):
            for _ in range(L):
                torch.mm(x, wgt)

    def wall(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps * 1e3

    def consume():
        for l in range(L):
            compute.wait_event(events[l])
            with torch.cuda.stream(compute):
                torch.mm(x, wgt)

    reps = max(3, args.steps)
    t_gemm = wall(gemms, reps)
    # the same pipelines with nothing hit: each layer's event is recorded and
    # nothing is launched, isolating the cost of the per-layer stream dependency
    empty = kvm.Batch(paged, batch.seqs).set_masks([np.zeros_like(sq.hit_mask) for sq in w.seqs])

    def deps_per_call():
        for l in range(L):
            kvm.retrieve_layer(paged, empty, l, stream=copy, event=events[l])
            compute.wait_event(events[l])
            with torch.cuda.stream(compute):
                torch.mm(x, wgt)

    # the pages' pipeline, layer l+1 loading while layer l computes: the copy
    # stream waits for the start of GEMM l-1 before layer l's scatter, so
    # each scatter runs beside one GEMM instead of all of them at once
    started = [torch.cuda.Event() for _ in range(L)]

    def paced(b, cap_of):
        def run():
            for l in range(L):
                if l > 0:
                    copy.wait_event(started[l - 1])
                kvm.retrieve_layer_ex(paged, b, l, stream=copy, event=events[l], max_workgroups=cap_of(l))
                compute.wait_event(events[l])
                started[l].record(compute)
                with torch.cuda.stream(compute):
                    torch.mm(x, wgt)
        return run

    def deps_one_call():
        kvm.retrieve_layers(paged, empty, 0, L, stream=copy, events=events)
        consume()

    alt = torch.cuda.Stream()

    def deps_two_streams():
        kvm.retrieve_layers(paged, empty, 0, L, stream=copy, events=events, alt_stream=alt)
        consume()

    t_deps = {"per-layer-calls": wall(deps_per_call, reps), "one-call": wall(deps_one_call, reps),
              "one-call-two-streams": wall(deps_two_streams, reps),
              "per-layer-calls-paced": wall(paced(empty, lambda l: 0), reps)}
    variants = []
    # (cap for layer 0, cap for layers 1..L-1): layer 0 has nothing to overlap
    # with, the others run beside the previous layer's GEMM
    for first_cap, cap in ((0, 0), (0, 32), (0, 48), (0, 64), (0, 96), (0, 128), (0, 256), (128, 128)):
        caps = [first_cap] + [cap] * (L - 1)

        def copies_per_call():
            for l in range(L):
                kvm.retrieve_layer_ex(paged, batch, l, stream=copy, event=events[l], max_workgroups=caps[l])

        def both_per_call():
            for l in range(L):
                kvm.retrieve_layer_ex(paged, batch, l, stream=copy, event=events[l], max_workgroups=caps[l])
                compute.wait_event(events[l])
                with torch.cuda.stream(compute):
                    torch.mm(x, wgt)

        def copies_one_call(a=None):
            kvm.retrieve_layers(paged, batch, 0, L, stream=copy, events=events, max_workgroups=caps, alt_stream=a)

        def both_one_call(a=None):
            kvm.retrieve_layers(paged, batch, 0, L, stream=copy, events=events, max_workgroups=caps, alt_stream=a)
            consume()

        for form, copies, both in (("per-layer-calls", copies_per_call, both_per_call),
                                   ("per-layer-calls-paced", copies_per_call, paced(batch, lambda l: caps[l])),
                                   ("one-call", copies_one_call, both_one_call),
                                   ("one-call-two-streams", lambda: copies_one_call(alt),
                                    lambda: both_one_call(alt))):
            t_copy, t_both = wall(copies, reps), wall(both, reps)
            v = {"form": form, "max_workgroups_layer0": first_cap, "max_workgroups": cap,
                 "t_copy_ms": round(t_copy, 3), "t_both_ms": round(t_both, 3),
                 "exposed_copy_ms": round(t_both - t_gemm, 3),
                 "exposed_vs_dependency_only_ms": round(t_both - t_deps[form], 3),
                 "overlap_efficiency": round((t_gemm + t_copy - t_both) / t_copy, 4)}
            if form.startswith("one-call"):
                # the 32 scatters back to back on the copy stream (every other
                # one on the second stream), HIP events around the one call
                # on the copy stream (the GPU, not the host, sets the pace):
                # median of 20 after 3 warm-ups, per layer
                a = alt if form.endswith("two-streams") else None
                lm = timed(copy, lambda: kvm.retrieve_layers(paged, batch, 0, L, stream=copy,
                                                             max_workgroups=[cap] * L, alt_stream=a),
                           20, stat="median") / L
                v["layer_scatter_ms"] = round(lm, 4)
                v["layer_scatter_GBps"] = round(per_layer_bytes / (lm / 1e3) / 1e9, 2)
            variants.append(v)
            log(f"layerwise caps {first_cap}/{cap} {form}: {v}")
    graph = layerwise_graph(paged, batch, empty, pool, copy, compute, x, wgt, events, started, wall, reps)
    assert kvm.take_faults() == 0
    best = min(variants, key=lambda v: v["t_both_ms"])
    return {
        "metric": "layerwise onload: copy time hidden behind per-layer GEMMs",
        "graph": graph,
        "workload": "layerwise-8b: 1 seq x 10240 tokens, 32 layers, GEMM 10240x4096x4096 bf16 per layer",
        "t_gemm_ms": round(t_gemm, 3),
        "t_dependency_only_ms": {k: round(v, 3) for k, v in t_deps.items()},
        "best": best, "variants": variants,
        "oracle_beside": oracle_beside(w, pool, kvm.FMT_BF16, n_chunks=40, layer=5),
    }


def layerwise_graph(paged, batch, empty, pool, copy, compute, x, wgt, events, started, wall, reps):
    """The paced pipeline (uncapped scatters) captured once into a HIP graph
    on the compute stream and replayed: the copy stream forks from the
    capture and joins it again through the layer events, so the 32
    scatters, the 32 GEMMs and their dependencies become graph nodes.  The
    same for the GEMMs alone and for the dependencies alone (nothing hit).
    Three replays write a sentinel-filled pool, each checked against the
    eager pipeline's pool."""
    import torch
    import paged_kv_movement_amd as kvm
    L = len(events)

    def body(b):
        copy.wait_stream(compute)
        for l in range(L):
            if l > 0:
                copy.wait_event(started[l - 1])
            kvm.retrieve_layer_ex(paged, b, l, stream=copy, event=events[l], max_workgroups=0)
            compute.wait_event(events[l])
            started[l].record(compute)
            with torch.cuda.stream(compute):
                torch.mm(x, wgt)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=compute):
            fn()
        torch.cuda.synchronize()
        return g

    def gemms_only():
        with torch.cuda.stream(compute):
            for _ in range(L):
                torch.mm(x, wgt)

    sentinel = 0x7E57
    pool.view(torch.int16).fill_(sentinel)
    torch.cuda.synchronize()
    body(batch)                                   # eager reference
    torch.cuda.synchronize()
    ref = pool.clone()
    g_both, g_deps, g_gemm = capture(lambda: body(batch)), capture(lambda: body(empty)), capture(gemms_only)
    for _ in range(3):
        pool.view(torch.int16).fill_(sentinel)
        torch.cuda.synchronize()
        g_both.replay()
        torch.cuda.synchronize()
        if not torch.equal(pool.view(torch.int16), ref.view(torch.int16)):
            raise RuntimeError("layerwise graph replay: pool differs from the eager pipeline's")
    del ref
    t_gemm, t_deps, t_both = wall(g_gemm.replay, reps), wall(g_deps.replay, reps), wall(g_both.replay, reps)
    return {"form": "per-layer-calls-paced, captured in one HIP graph", "max_workgroups": 0,
            "t_gemm_ms": round(t_gemm, 3), "t_dependency_only_ms": round(t_deps, 3), "t_both_ms": round(t_both, 3),
            "exposed_copy_ms": round(t_both - t_gemm, 3),
            "exposed_vs_dependency_only_ms": round(t_both - t_deps, 3), "replays_checked": 3}


def bench_layerwise_store(args):
    """Prefill-style layerwise store: layer l's KV is gathered on a copy stream
    once layer l's GEMM (10240 x 4096 x 4096 bf16, the producer) has finished,
    while layer l+1 computes.  Two ways to enqueue the stores: one call per
    layer after its GEMM (kv_store_layer), or one call for all layers after
    the GEMMs are enqueued, the library enqueueing each layer's wait on its
    GEMM's event (kv_store_layers).  Reports the exposed store time for
    several workgroup caps (layer 0 always at full width; the last layer's
    store has nothing left to hide behind)."""
    import torch
    import paged_kv_movement_amd as kvm
    from paged_kv_movement_amd import workloads as wl

    w = wl.layerwise8b()
    pool, paged, batch, arena = setup(w, kvm.FMT_BF16)
    copy, compute, alt = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    x = torch.randn(10240, 4096, device="cuda", dtype=torch.bfloat16)
    wgt = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16) * 0.01
    L = w.num_layers
    done = [torch.cuda.Event() for _ in range(L)]
    per_layer_bytes = 2 * 10240 * 2 * w.width * 2

    def wall(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps * 1e3

    def gemms():
        with torch.cuda.stream(compute):
            for _ in range(L):
                torch.mm(x, wgt)

    reps = max(3, args.steps)
    t_gemm = wall(gemms, reps)
    variants = []
    for cap in (0, 64, 128, 256):
        caps = [0] + [cap] * (L - 1)

        def stores_per_call():
            for l in range(L):
                kvm.store_layer(paged, batch, l, stream=copy, max_workgroups=caps[l])

        def both_per_call():
            for l in range(L):
                with torch.cuda.stream(compute):
                    torch.mm(x, wgt)
                    done[l].record(compute)
                copy.wait_event(done[l])
                kvm.store_layer(paged, batch, l, stream=copy, max_workgroups=caps[l])

        def stores_one_call(a=None):
            kvm.store_layers(paged, batch, 0, L, stream=copy, max_workgroups=caps, alt_stream=a)

        def both_one_call(a=None):
            for l in range(L):
                with torch.cuda.stream(compute):
                    torch.mm(x, wgt)
                    done[l].record(compute)
            kvm.store_layers(paged, batch, 0, L, stream=copy, wait_events=done, max_workgroups=caps, alt_stream=a)

        for form, stores, both in (("per-layer-calls", stores_per_call, both_per_call),
                                   ("one-call", stores_one_call, both_one_call),
                                   ("one-call-two-streams", lambda: stores_one_call(alt),
                                    lambda: both_one_call(alt))):
            t_store, t_both = wall(stores, reps), wall(both, reps)
            v = {"form": form, "max_workgroups": cap, "t_store_ms": round(t_store, 3), "t_both_ms": round(t_both, 3),
                 "exposed_store_ms": round(t_both - t_gemm, 3),
                 "overlap_efficiency": round((t_gemm + t_store - t_both) / t_store, 4)}
            if form.startswith("one-call"):
                a = alt if form.endswith("two-streams") else None
                lm = timed(copy, lambda: kvm.store_layers(paged, batch, 0, L, stream=copy, max_workgroups=[cap] * L,
                                                          alt_stream=a), 20, stat="median") / L
                v["layer_store_ms"] = round(lm, 4)
                v["layer_store_GBps"] = round(per_layer_bytes / (lm / 1e3) / 1e9, 2)
            variants.append(v)
            log(f"layerwise store cap {cap} {form}: {v}")
    assert kvm.take_faults() == 0
    return {"metric": "layerwise store: gather time hidden behind per-layer GEMMs",
            "workload": "layerwise-store-8b: 1 seq x 10240 tokens, 32 layers, GEMM 10240x4096x4096 bf16 per layer",
            "t_gemm_ms": round(t_gemm, 3), "best": min(variants, key=lambda v: v["t_both_ms"]),
            "variants": variants,
            "oracle_beside": oracle_beside(w, pool, kvm.FMT_BF16, n_chunks=40, layer=5)}


def bench_offload(args):
    """Offload to / onload from pinned host memory at the 8B shape.

    The chunk buffers live in pinned host memory and the same store / retrieve
    kernels write / read them over PCIe.  Reported next to it: the link's own
    ceiling (one 1 GiB hipMemcpy each way), the staged alternative (gather
    into device chunks, then copy each chunk; copy each chunk, then scatter),
    fp8 chunks (half the bytes on the link), a duplex run (offload of four
    sequences while the other four onload), and the layerwise onload from
    host behind the per-layer GEMMs."""
    import numpy as np
    import torch
    import paged_kv_movement_amd as kvm
    from paged_kv_movement_amd import workloads as wl

    w = wl.llama8b()
    reps = max(3, args.steps)
    stream = torch.cuda.Stream()
    pool, paged, hb, harena = setup(w, kvm.FMT_BF16, "host")
    _, _, db, darena = setup(w, kvm.FMT_BF16, "device", pool=pool)
    tokens = sum(sq.tok_end - sq.tok_start for sq in w.seqs)
    rtok = sum(hit_tokens(w))
    per_tok = kv_bytes_per_token(w)
    out = {"metric": "offload / onload GB/s over PCIe (chunks in pinned host memory)",
           "workload": "offload-8b: llama3.1-8b KV shape, 8 seqs x 10000 tokens, 30-chunk hit mask",
           "pcie_gen5_x16_GBps": PCIE_PEAK_GBPS}

    def gbps(nbytes, ms):
        return round(nbytes / (ms / 1e3) / 1e9, 2)

    # link ceiling: 1 GiB pinned <-> device copies
    big_d = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    big_h = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    with torch.cuda.stream(stream):
        big_d.copy_(big_h, non_blocking=True)
        big_h.copy_(big_d, non_blocking=True)
        h2d = timed(stream, lambda: big_d.copy_(big_h, non_blocking=True), reps)
        d2h = timed(stream, lambda: big_h.copy_(big_d, non_blocking=True), reps)
    out["link_ceiling"] = {"h2d_GBps": gbps(1 << 30, h2d), "d2h_GBps": gbps(1 << 30, d2h)}
    del big_d, big_h

    for _ in range(args.warmup):
        kvm.store(paged, hb, stream=stream)
        kvm.retrieve(paged, hb, stream=stream)
    st = timed(stream, lambda: kvm.store(paged, hb, stream=stream), reps)
    rt = timed(stream, lambda: kvm.retrieve(paged, hb, stream=stream), reps)
    out["offload"] = {"ms": round(st, 3), "GBps_link": gbps(tokens * per_tok, st),
                      "pct_of_link_ceiling": round(100 * tokens * per_tok / (st / 1e3) / 1e9
                                                   / out["link_ceiling"]["d2h_GBps"], 1),
                      "tokens_per_s": round(tokens / (st / 1e3), 1)}
    out["onload"] = {"ms": round(rt, 3), "GBps_link": gbps(rtok * per_tok, rt),
                     "pct_of_link_ceiling": round(100 * rtok * per_tok / (rt / 1e3) / 1e9
                                                  / out["link_ceiling"]["h2d_GBps"], 1),
                     "tokens_per_s": round(rtok / (rt / 1e3), 1)}
    log(f"offload {out['offload']}  onload {out['onload']}")

    # staged alternative: device chunks plus one copy per chunk
    nbytes = darena.numel()

    def staged_offload():
        kvm.store(paged, db, stream=stream)
        with torch.cuda.stream(stream):
            harena.copy_(darena, non_blocking=True)

    def staged_onload():
        with torch.cuda.stream(stream):
            darena.copy_(harena, non_blocking=True)
        kvm.retrieve(paged, db, stream=stream)

    so, sn = timed(stream, staged_offload, reps), timed(stream, staged_onload, reps)
    out["staged_offload"] = {"ms": round(so, 3), "GBps_link": gbps(tokens * per_tok, so),
                             "note": "gather into device chunks, then one device-to-host copy of all of them"}
    out["staged_onload"] = {"ms": round(sn, 3), "GBps_link": gbps(rtok * per_tok, sn),
                            "note": "one host-to-device copy of all chunks, then the scatter"}
    del darena, db
    torch.cuda.empty_cache()

    # duplex: sequences 0-3 offload while 4-7 onload
    a, b = kvm.Batch(paged, hb.seqs[:4]), kvm.Batch(paged, hb.seqs[4:])
    a.set_masks([sq.hit_mask for sq in w.seqs[:4]])
    b.set_masks([sq.hit_mask for sq in w.seqs[4:]])
    other = torch.cuda.Stream()

    def duplex():
        other.wait_stream(stream)
        kvm.store(paged, a, stream=stream)
        kvm.retrieve(paged, b, stream=other)
        stream.wait_stream(other)

    du = timed(stream, duplex, reps)
    du_bytes = (sum(sq.tok_end - sq.tok_start for sq in w.seqs[:4]) + sum(hit_tokens(w)[4:])) * per_tok
    out["duplex"] = {"ms": round(du, 3), "GBps_link_both_directions": gbps(du_bytes, du)}
    log(f"staged {out['staged_offload']} {out['staged_onload']} duplex {out['duplex']}")

    # fp8 chunks on the link
    del harena, hb
    _, _, fb, farena = setup(w, kvm.FMT_FP8, "host", pool=pool)
    for _ in range(args.warmup):
        kvm.store(paged, fb, kvm.FMT_FP8, stream=stream)
    fst = timed(stream, lambda: kvm.store(paged, fb, kvm.FMT_FP8, stream=stream), reps)
    frt = timed(stream, lambda: kvm.retrieve(paged, fb, fmt=kvm.FMT_FP8, stream=stream), reps)
    fb_st = sum(kvm_chunk_total(paged, sq, kvm.FMT_FP8, None) for sq in w.seqs)
    fb_rt = sum(kvm_chunk_total(paged, sq, kvm.FMT_FP8, sq.hit_mask) for sq in w.seqs)
    out["fp8_offload"] = {"ms": round(fst, 3), "GBps_link": gbps(fb_st, fst), "tokens_per_s": round(tokens / (fst / 1e3), 1)}
    out["fp8_onload"] = {"ms": round(frt, 3), "GBps_link": gbps(fb_rt, frt), "tokens_per_s": round(rtok / (frt / 1e3), 1)}
    log(f"fp8 {out['fp8_offload']} {out['fp8_onload']}")
    assert kvm.take_faults() == 0
    out["oracle_beside"] = oracle_beside(w, pool, kvm.FMT_BF16)
    del fb, farena, pool, paged
    torch.cuda.empty_cache()
    # the two streams already made: a third and fourth would share a
    # hardware queue with one of them and run in order with it
    out["layerwise_onload_from_host"] = layerwise_from_host(args, copy=stream, compute=other)
    return out


def kvm_chunk_total(paged, sq, fmt, mask):
    """Exact bytes of a sequence's chunks (only the leading hit ones if mask)."""
    n = -(-(sq.tok_end - sq.tok_start) // paged.chunk_size)
    if mask is not None:
        m = list(mask) + [0]
        n = m.index(0) if 0 in m[:n] else n
    return sum(paged.chunk_bytes(min(paged.chunk_size, sq.tok_end - sq.tok_start - c * paged.chunk_size), fmt)
               for c in range(n))


def layerwise_from_host(args, copy, compute):
    """Layer-by-layer onload of one 10240-token sequence whose chunks are in
    pinned host memory, each layer's event gating that layer's GEMM."""
    import torch
    import paged_kv_movement_amd as kvm
    from paged_kv_movement_amd import workloads as wl

    w = wl.layerwise8b()
    pool, paged, batch, arena = setup(w, kvm.FMT_BF16, "host")
    kvm.store(paged, batch)
    torch.cuda.synchronize()
    x = torch.randn(10240, 4096, device="cuda", dtype=torch.bfloat16)
    wgt = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16) * 0.01
    L = w.num_layers
    evs = [torch.cuda.Event() for _ in range(L)]
    layer_bytes = 10240 * 2 * w.width * 2
    reps = max(2, min(args.steps, 3))

    def wall(fn):
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps * 1e3

    def gemms():
        with torch.cuda.stream(compute):
            for _ in range(L):
                torch.mm(x, wgt)

    t_gemm = wall(gemms)
    variants = []
    for cap in (16, 32, 64, 0):
        def copies():
            for l in range(L):
                kvm.retrieve_layer_ex(paged, batch, l, stream=copy, max_workgroups=cap)

        def both():
            for l in range(L):
                kvm.retrieve_layer_ex(paged, batch, l, stream=copy, event=evs[l], max_workgroups=cap)
                compute.wait_event(evs[l])
                with torch.cuda.stream(compute):
                    torch.mm(x, wgt)

        t_copy, t_both = wall(copies), wall(both)
        variants.append({"max_workgroups": cap, "t_copy_ms": round(t_copy, 3), "t_both_ms": round(t_both, 3),
                         "layer_GBps_link": round(L * layer_bytes / (t_copy / 1e3) / 1e9, 2),
                         "exposed_ms": round(t_both - max(t_gemm, t_copy), 3),
                         "gemm_hidden_fraction": round((t_gemm + t_copy - t_both) / t_gemm, 4)})
        log(f"layerwise from host cap {cap}: {variants[-1]}")
    assert kvm.take_faults() == 0
    return {"workload": "1 seq x 10240 tokens, 32 layers, chunks in pinned host memory, "
                        "GEMM 10240x4096x4096 bf16 per layer",
            "t_gemm_ms": round(t_gemm, 3), "variants": variants}


FORMAT_NAMES = {0: "bf16", 1: "fp8-e4m3-scaled", 2: "fp8-e5m2-scaled", 3: "k16-v8"}
# chunk bytes per K element and per V element of each format
PART_BYTES = {0: (2, 2), 1: (1, 1), 2: (1, 1), 3: (2, 1)}


CACHEGEN_KEY_BINS, CACHEGEN_VALUE_BINS = 32, 16    # bins used for every layer by the benchmark


def bench_cachegen(args):
    """CacheGen quantiser at the 8B shape (the fp8 workload's inputs): store =
    gather + quantise, retrieve = dequantise + scatter of every chunk."""
    import torch
    import paged_kv_movement_amd as kvm
    from paged_kv_movement_amd import workloads as wl

    w = wl.fp8_8b()
    pool, paged, batch, arena = setup(w, kvm.FMT_CACHEGEN)
    stream = torch.cuda.Stream()
    kb, vb = [CACHEGEN_KEY_BINS] * w.num_layers, [CACHEGEN_VALUE_BINS] * w.num_layers
    tokens = sum(sq.tok_end - sq.tok_start for sq in w.seqs)
    rtok = sum(hit_tokens(w))
    # per element 2 bytes of bf16 and 1 symbol byte; per (layer, K/V, token) one float32 max1
    st_bytes = tokens * w.num_layers * 2 * (3 * w.width + 4)
    rt_bytes = rtok * w.num_layers * 2 * (3 * w.width + 4)
    for _ in range(args.warmup):
        kvm.store_cachegen(paged, batch, kb, vb, stream=stream)
        kvm.retrieve_cachegen(paged, batch, kb, vb, stream=stream)
    reps = max(3, args.steps)
    ws = paged.new_workspace()
    st_ms = timed(stream, lambda: kvm.store_cachegen(paged, batch, kb, vb, stream=stream), reps)
    rt_ms = timed(stream, lambda: kvm.retrieve_cachegen(paged, batch, kb, vb, stream=stream, workspace=ws), reps)
    cm_ms = timed(stream, lambda: kvm.retrieve_cachegen(paged, batch, kb, vb, stream=stream), reps)
    assert kvm.take_faults() == 0
    st, rt = st_bytes / (st_ms / 1e3) / 1e9, rt_bytes / (rt_ms / 1e3) / 1e9
    beside = oracle_beside(w, pool, kvm.FMT_CACHEGEN, 4, bins=(kb, vb))
    return {
        "metric": "store / retrieve algorithmic GB/s", "workload": "cachegen-8b",
        "oracle_beside": beside,
        "format": f"cachegen int8 symbols, key bins {CACHEGEN_KEY_BINS}, value bins {CACHEGEN_VALUE_BINS}",
        "store_ms": round(st_ms, 4), "store_GBps": round(st, 2), "store_pct_hbm_peak": round(100 * st / HBM_PEAK_GBPS, 2),
        "store_tokens_per_s": round(tokens / (st_ms / 1e3), 1),
        "retrieve_ms": round(rt_ms, 4), "retrieve_GBps": round(rt, 2),
        "retrieve_pct_hbm_peak": round(100 * rt / HBM_PEAK_GBPS, 2),
        "retrieve_tokens_per_s": round(rtok / (rt_ms / 1e3), 1),
        "retrieve_order": "pool-address (workspace)",
        "retrieve_chunk_major_ms": round(cm_ms, 4),
        "retrieve_chunk_major_GBps": round(rt_bytes / (cm_ms / 1e3) / 1e9, 2),
    }


def bench_simple(args, name, fmt):
    """Store + retrieve GB/s for the 70B-style workload and the quantised
    formats (the fp8 workload's inputs)."""
    import torch
    import paged_kv_movement_amd as kvm
    from paged_kv_movement_amd import workloads as wl

    w = wl.ALL[name]()
    pool, paged, batch, arena = setup(w, fmt)
    stream = torch.cuda.Stream()
    tokens = sum(sq.tok_end - sq.tok_start for sq in w.seqs)
    rtok = sum(hit_tokens(w))
    # per token and part: 2 bytes of bf16 on the pool side, the part's element
    # size on the chunk side; plus one float32 scale per quantised group
    part_elems_st = tokens * w.num_layers * w.width
    part_elems_rt = rtok * w.num_layers * w.width
    chunks_st = sum(-(-(sq.tok_end - sq.tok_start) // w.chunk_size) for sq in w.seqs)
    chunks_rt = sum(-(-t // w.chunk_size) for t in hit_tokens(w))
    n_q = sum(b == 1 for b in PART_BYTES[fmt])
    per_elem = sum(2 + b for b in PART_BYTES[fmt])
    st_bytes = per_elem * part_elems_st + 4 * n_q * w.num_layers * chunks_st
    rt_bytes = per_elem * part_elems_rt + 4 * n_q * w.num_layers * chunks_rt
    sws = batch.new_store_workspace(fmt)             # None for the fp8 formats (no bf16 part)
    for _ in range(args.warmup):
        kvm.store(paged, batch, fmt, stream=stream, workspace=sws)
        kvm.retrieve(paged, batch, fmt=fmt, stream=stream)
    reps = max(3, args.steps)
    ws = paged.new_workspace()
    st_ms = timed(stream, lambda: kvm.store(paged, batch, fmt, stream=stream, workspace=sws), reps)
    plain_ms = timed(stream, lambda: kvm.store(paged, batch, fmt, stream=stream), reps) if sws is not None else None
    rt_ms = timed(stream, lambda: kvm.retrieve(paged, batch, fmt=fmt, stream=stream, workspace=ws), reps)
    cm_ms = timed(stream, lambda: kvm.retrieve(paged, batch, fmt=fmt, stream=stream), reps)
    assert kvm.take_faults() == 0
    st, rt = st_bytes / (st_ms / 1e3) / 1e9, rt_bytes / (rt_ms / 1e3) / 1e9
    # bf16: the same-run copies of the gather's payload, contiguous and with
    # one side in page-sized blocks visited in a scattered order
    copies = {}
    page_bytes = w.page_size * w.width * 2
    if fmt == kvm.FMT_BF16 and page_bytes >= 4096 and page_bytes & (page_bytes - 1) == 0:
        src = pool.view(-1).view(torch.uint8)
        nb = (st_bytes // 2) // page_bytes * page_bytes
        t = timed(stream, lambda: kvm.copy_bytes(arena, src, nb, stream=stream), 5)
        copies["copy_ceiling_GBps"] = round(2 * nb / (t / 1e3) / 1e9, 2)
        for key, side in (("reads", kvm.COPY_SCATTERED_READS), ("writes", kvm.COPY_SCATTERED_WRITES)):
            t = timed(stream, lambda: kvm.copy_blocks(arena, src, nb, page_bytes, side, stream=stream), 5)
            copies[f"copy_scattered_{key}_GBps"] = round(2 * nb / (t / 1e3) / 1e9, 2)
        copies["gather_frac_of_scattered_read_copy"] = round(st / copies["copy_scattered_reads_GBps"], 4)
    beside = oracle_beside(w, pool, fmt, 4)
    return {
        "metric": "store / retrieve algorithmic GB/s", "workload": name,
        "format": FORMAT_NAMES[fmt],
        "oracle_beside": beside,
        "store_ms": round(st_ms, 4), "store_GBps": round(st, 2), "store_pct_hbm_peak": round(100 * st / HBM_PEAK_GBPS, 2),
        "store_tokens_per_s": round(tokens / (st_ms / 1e3), 1),
        "retrieve_ms": round(rt_ms, 4), "retrieve_GBps": round(rt, 2),
        "retrieve_pct_hbm_peak": round(100 * rt / HBM_PEAK_GBPS, 2),
        "retrieve_tokens_per_s": round(rtok / (rt_ms / 1e3), 1),
        "retrieve_order": "pool-address (workspace)",
        "retrieve_chunk_major_ms": round(cm_ms, 4),
        "retrieve_chunk_major_GBps": round(rt_bytes / (cm_ms / 1e3) / 1e9, 2),
        "store_form": "address plan (kv_store_chunks_ws)" if sws is not None else "kv_store_chunks (no bf16 part)",
        "store_plain_ms": round(plain_ms, 4) if plain_ms else None,
        "store_plain_GBps": round(st_bytes / (plain_ms / 1e3) / 1e9, 2) if plain_ms else None,
        **copies,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3.1-8b",
                    choices=["llama3.1-8b", "layerwise-8b", "layerwise-store-8b", "llama-70b-style",
                             "llama3.1-8b-tp8-share", "fp8-8b",
                             "e5m2-8b", "k16v8-8b", "cachegen-8b",
                             "offload-8b"])
    ap.add_argument("--retrieve-order", choices=["address", "chunk"], default="address",
                    help="headline retrieve: pool-address order with a workspace (default) or chunk-major")
    ap.add_argument("--store-plan", choices=["on", "off"], default="on",
                    help="headline store: through its address plan with a workspace (default) or kv_store_chunks")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (used for profiler runs)")
    ap.add_argument("--layers-only", type=int, default=None, metavar="CAP",
                    help="layerwise workloads: time only the 32 layer calls, one call for all layers, every "
                         "layer's grid capped at CAP workgroups (0: none); for kernel traces")
    ap.add_argument("--alt-stream", action="store_true",
                    help="with --layers-only: every other layer on a second stream (the calls' alt_stream)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the paged<->chunk movement runs on each GPU's own "
              "sequences with nothing exchanged, so there is no multi-GPU mode to time "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    import paged_kv_movement_amd as kvm
    kvm.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.workload == "llama3.1-8b":
        out = bench_llama8b(args)
    elif args.workload in ("layerwise-8b", "layerwise-store-8b") and args.layers_only is not None:
        out = bench_layers_only(args, store=args.workload == "layerwise-store-8b")
    elif args.workload == "layerwise-8b":
        out = bench_layerwise(args)
    elif args.workload == "layerwise-store-8b":
        out = bench_layerwise_store(args)
    elif args.workload == "offload-8b":
        out = bench_offload(args)
    elif args.workload == "llama-70b-style":
        out = bench_simple(args, "llama-70b-style", kvm.FMT_BF16)
    elif args.workload == "llama3.1-8b-tp8-share":
        out = bench_simple(args, "llama3.1-8b-tp8-share", kvm.FMT_BF16)
    elif args.workload == "e5m2-8b":
        out = bench_simple(args, "fp8-8b", kvm.FMT_FP8_E5M2)
    elif args.workload == "k16v8-8b":
        out = bench_simple(args, "fp8-8b", kvm.FMT_K16_V8)
    elif args.workload == "cachegen-8b":
        out = bench_cachegen(args)
    else:
        out = bench_simple(args, "fp8-8b", kvm.FMT_FP8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
