"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (one store call and one retrieve call over all sequences).

Every workload is compared in full against the oracle: every chunk's bytes
after the store, and the whole pool after the retrieve.  For the quantised
formats the oracle (one element at a time, slow) runs one task per
(sequence, chunk) on the host's threads; the round-trip error bound is then
checked over every element as well.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_movement_amd as kvm
from paged_kv_movement_amd import workloads as wl
from gpu_util import (say, host_from_dev_pool, oracle_pool, chunk_tokens, setup_device, host_chunks,
                      check_store, check_retrieve, equal_blocked, first_diff, sync, oracle_store_all,
                      oracle_retrieve_all)

pytestmark = pytest.mark.gpu

BF16, FP8, E5M2, K16V8 = kvm.FMT_BF16, kvm.FMT_FP8, kvm.FMT_FP8_E5M2, kvm.FMT_K16_V8
SENTINEL = 0x7E57


def _free():
    sync()
    torch.cuda.empty_cache()
    torch._C._host_emptyCache()     # give back pinned host blocks too


def _full_bf16(w, expect_tokens, where="device", workspaces=False):
    # workspaces: the store through its address plan and the retrieve in
    # pool-address order, as the benchmark runs them
    say("case", w.name, "pool GB", w.pool_nbytes() / 1e9, "chunks in", where, "workspaces", workspaces)
    pool = wl.device_pool(w)
    pool, paged, batch, chunk_sets = setup_device(w, pool=pool, fill=0xCD, where=where)
    kvm.store(paged, batch, workspace=batch.new_store_workspace() if workspaces else None)
    sync()
    assert kvm.take_faults() == 0
    arr = host_from_dev_pool(pool)
    say("  store done; checking against the oracle")
    check_store(w, arr, chunk_sets, BF16)
    del arr
    pool.view(torch.int16).fill_(SENTINEL)
    n = kvm.retrieve(paged, batch, workspace=paged.new_workspace() if workspaces else None)
    sync()
    assert kvm.take_faults() == 0
    assert n == expect_tokens
    say("  retrieve done; checking against the oracle")
    got = host_from_dev_pool(pool)
    before = np.full(got.shape, SENTINEL, np.uint16)
    counts = check_retrieve(w, before, got, chunk_sets, BF16, [s.hit_mask for s in w.seqs],
                            copy=False)
    assert counts == expect_tokens
    del got, before, pool, paged, batch, chunk_sets
    _free()


def test_full_llama8b_store_and_30_chunk_retrieve():
    # 8 sequences x 10000 tokens (39 full chunks + a 16-token tail), 8192-page
    # pool; retrieve with the first 30 chunks hit
    _full_bf16(wl.llama8b(), [30 * 256] * 8)


def test_full_llama8b_offload_to_host_and_onload():
    # the same workload with every chunk in pinned host memory: the store is
    # the offload over PCIe, the retrieve the onload
    _full_bf16(wl.llama8b(), [30 * 256] * 8, where="host")


@pytest.mark.parametrize("form", ["plain", "workspaces"])
def test_full_llama8b_tp8_share_store_and_30_chunk_retrieve(form):
    # one rank's share under 8-way tensor parallelism: one KV head, 4 KiB pages
    _full_bf16(wl.llama8b_tp8_share(), [30 * 256] * 8, workspaces=form == "workspaces")


@pytest.mark.parametrize("form", ["plain", "workspaces"])
def test_full_llama70b_store_and_retrieve(form):
    # 80 layers, one 32768-token sequence (128 chunks) on a 4096-page pool
    _full_bf16(wl.llama70b(), [32768], workspaces=form == "workspaces")


@pytest.mark.parametrize("form", ["per-layer-calls", "per-layer-calls-paced", "one-call", "one-call-two-streams"])
def test_full_layerwise_8b_with_compute_stream(form):
    # one 10240-token sequence retrieved layer by layer on a copy stream, each
    # layer's event gating a bf16 GEMM (tokens x 4096 x 4096) on the compute
    # stream; the layers enqueued one call each (paced: layer l's scatter
    # waits for the start of GEMM l-1), or all by one call (with every other
    # layer on a second stream)
    w = wl.layerwise8b()
    say("case", w.name, form)
    pool = wl.device_pool(w)
    pool, paged, batch, chunk_sets = setup_device(w, pool=pool, fill=0xCD)
    kvm.store(paged, batch)
    sync()
    pool.view(torch.int16).fill_(SENTINEL)
    sync()
    copy, compute = torch.cuda.Stream(), torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(w.num_layers)]
    x = torch.randn(10240, 4096, device="cuda", dtype=torch.bfloat16)
    wgt = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16) * 0.01
    outs = []
    # layer 0 at full width, the rest on a capped grid (as the benchmark's
    # overlap variants do)
    caps = [0] + [128] * (w.num_layers - 1)
    if form.startswith("one-call"):
        alt = torch.cuda.Stream() if form.endswith("two-streams") else None
        assert kvm.retrieve_layers(paged, batch, 0, w.num_layers, stream=copy, events=events,
                                   max_workgroups=caps, alt_stream=alt) == [10240]
    started = [torch.cuda.Event() for _ in range(w.num_layers)]
    for l in range(w.num_layers):
        if form == "per-layer-calls-paced" and l > 0:
            copy.wait_event(started[l - 1])
        if form.startswith("per-layer-calls"):
            assert kvm.retrieve_layer_ex(paged, batch, l, stream=copy, event=events[l],
                                         max_workgroups=caps[l]) == [10240]
        compute.wait_event(events[l])
        started[l].record(compute)
        with torch.cuda.stream(compute):
            outs.append(torch.mm(x, wgt))
    sync()
    assert kvm.take_faults() == 0
    assert all(torch.isfinite(o).all() for o in outs[:2])
    got = host_from_dev_pool(pool)
    before = np.full(got.shape, SENTINEL, np.uint16)
    check_retrieve(w, before, got, chunk_sets, BF16, [s.hit_mask for s in w.seqs], copy=False)
    del got, before, pool, paged, batch, chunk_sets, outs
    _free()


def _full_quantised(w, fmt, bins=None):
    """Store every chunk of the 8B-shape workload in a quantised format and
    compare every chunk's bytes (codes and scales, or symbols and max1) with
    the oracle's; retrieve every chunk into a zeroed pool and compare the
    whole pool with the oracle's retrieve; the same retrieve in pool-address
    order must give the same pool; a 30-chunk hit mask into a sentinel pool is
    compared with the oracle as a whole as well.  The oracle runs one task per
    (sequence, chunk) on the host's threads.  Returns the original and
    retrieved device pools, the chunk buffers and the oracle's chunks for
    the bound checks."""
    pool = wl.device_pool(w)
    pool, paged, batch, chunk_sets = setup_device(w, pool=pool, fmt=fmt, fill=0xCD)
    if fmt == kvm.FMT_CACHEGEN:
        kvm.store_cachegen(paged, batch, *bins)
    else:
        kvm.store(paged, batch, fmt)
    sync()
    assert kvm.take_faults() == 0
    arr = host_from_dev_pool(pool)
    exp = oracle_store_all(w, oracle_pool(w, arr), fmt, bins)
    del arr
    got = [host_chunks(cs) for cs in chunk_sets]
    n_chunks = 0
    for i, (g_seq, e_seq) in enumerate(zip(got, exp)):
        assert len(g_seq) == len(e_seq)
        for c, (g, e) in enumerate(zip(g_seq, e_seq)):
            assert g.size == e.size and np.array_equal(g, e), (w.name, fmt, "seq", i, "chunk", c, first_diff(g, e))
            n_chunks += 1
    say("  store: all", n_chunks, "chunks equal the oracle's, bit for bit")
    del exp

    def retrieve(masks=None, ws=None):
        if fmt == kvm.FMT_CACHEGEN:
            return kvm.retrieve_cachegen(paged, batch, *bins, masks=masks, workspace=ws)
        return kvm.retrieve(paged, batch, masks=masks, fmt=fmt, workspace=ws)

    orig = pool.clone()
    pool.zero_()
    all_hit = [np.ones(40, np.uint8)] * len(w.seqs)
    assert retrieve(all_hit) == [10000] * 8
    sync()
    assert kvm.take_faults() == 0
    got_pool = host_from_dev_pool(pool)
    exp_pool = np.zeros_like(got_pool)
    assert oracle_retrieve_all(w, oracle_pool(w, exp_pool), got, fmt, all_hit, bins) == [10000] * 8
    assert equal_blocked(got_pool, exp_pool), (w.name, fmt, first_diff(got_pool, exp_pool))
    say("  retrieve (all hit): the whole pool equals the oracle's")
    del got_pool
    # the retrieve in pool-address order gives the same pool, bit for bit
    retrieved = pool.clone()
    pool.zero_()
    assert retrieve(all_hit, paged.new_workspace()) == [10000] * 8
    sync()
    assert kvm.take_faults() == 0
    assert torch.equal(pool.view(torch.int16), retrieved.view(torch.int16))
    # 30-chunk hit mask into a sentinel pool: the whole pool vs the oracle's
    pool.view(torch.int16).fill_(SENTINEL)
    masks = [np.r_[np.ones(30, np.uint8), np.zeros(10, np.uint8)]] * 8
    assert retrieve(masks) == [7680] * 8
    sync()
    assert kvm.take_faults() == 0
    got_pool = host_from_dev_pool(pool)
    exp_pool[...] = SENTINEL
    assert oracle_retrieve_all(w, oracle_pool(w, exp_pool), got, fmt, masks, bins) == [7680] * 8
    assert equal_blocked(got_pool, exp_pool), (w.name, fmt, "mask", first_diff(got_pool, exp_pool))
    say("  retrieve (30 of 40 chunks): the whole pool equals the oracle's")
    del got_pool, exp_pool
    return pool, paged, batch, chunk_sets, orig, retrieved, got


@pytest.mark.parametrize("fmt", [FP8, E5M2, K16V8], ids=["fp8", "e5m2", "k16v8"])
def test_full_fp8_8b_every_chunk_and_whole_pool(fmt):
    w = wl.fp8_8b()
    say("case", w.name, fmt)
    pool, paged, batch, chunk_sets, orig, retrieved, ref = _full_quantised(w, fmt)
    # the round-trip error bound over every element, each group's floor
    # taken from the oracle's scale
    from test_gpu_parity import _assert_fp8_bound
    _assert_fp8_bound(w, orig, retrieved, chunk_sets, fmt, ref_chunks=ref)
    del pool, paged, batch, chunk_sets, orig, retrieved, ref
    _free()


@pytest.mark.parametrize("form", ["per-layer-calls", "one-call", "one-call-two-streams"])
def test_full_layerwise_store_8b_behind_compute(form):
    # prefill-style: layer l's KV is stored on a copy stream once layer l's
    # GEMM (the producer) is done, while layer l+1 computes; one store call
    # per layer, or one call for all layers after the GEMMs are enqueued
    w = wl.layerwise8b()
    say("case", w.name, "layerwise store", form)
    pool = wl.device_pool(w)
    pool, paged, batch, chunk_sets = setup_device(w, pool=pool, fill=0xCD)
    copy, compute = torch.cuda.Stream(), torch.cuda.Stream()
    done = [torch.cuda.Event() for _ in range(w.num_layers)]
    stored = [torch.cuda.Event() for _ in range(w.num_layers)]
    x = torch.randn(10240, 4096, device="cuda", dtype=torch.bfloat16)
    wgt = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16) * 0.01
    sync()
    caps = [0] + [128] * (w.num_layers - 1)
    for l in range(w.num_layers):
        with torch.cuda.stream(compute):
            torch.mm(x, wgt)
            done[l].record(compute)
        if form == "per-layer-calls":
            copy.wait_event(done[l])
            kvm.store_layer(paged, batch, l, stream=copy, event=stored[l], max_workgroups=caps[l])
    if form.startswith("one-call"):
        alt = torch.cuda.Stream() if form.endswith("two-streams") else None
        kvm.store_layers(paged, batch, 0, w.num_layers, stream=copy, wait_events=done, events=stored,
                         max_workgroups=caps, alt_stream=alt)
    sync()
    assert kvm.take_faults() == 0
    arr = host_from_dev_pool(pool)
    check_store(w, arr, chunk_sets, BF16)
    del arr, pool, paged, batch, chunk_sets
    _free()


def test_full_cachegen_8b_every_chunk_and_whole_pool():
    # the fp8 workload's inputs (N(0,1), 4 outlier channels x20) through the
    # CacheGen quantiser, seeded per-layer bins
    from gpu_util import cachegen_bins
    w = wl.fp8_8b()
    say("case", w.name, "cachegen")
    kb, vb = cachegen_bins(w.num_layers, 4)
    pool, paged, batch, chunk_sets, orig, retrieved, ref = _full_quantised(w, kvm.FMT_CACHEGEN, (kb, vb))
    # every element: |x' - x| <= max1 * (1/(2 MAX) + 2^-8 + 2^-20) (half a
    # quantisation step, the float32 steps, the bf16 rounding), max1 from the
    # oracle's chunks
    L, E, P, C = w.num_layers, w.width, w.page_size, w.chunk_size
    worst = 0.0
    for sq, ref_seq in zip(w.seqs, ref):
        bt = torch.from_numpy(sq.block_table.astype(np.int64)).cuda()
        for c, (b, n_c) in enumerate(zip(ref_seq, chunk_tokens(w, sq))):
            m1 = torch.from_numpy(b[L * 2 * n_c * E:].view(np.float32).reshape(L, 2, n_c).copy()).cuda()
            t = sq.tok_start + c * C + torch.arange(n_c, device="cuda")
            page, row = bt[t // P], t % P
            for l in range(L):
                for kv, bins in ((0, kb), (1, vb)):
                    MAX = float(bins[l] // 2 - 1)
                    x = orig[l, kv].view(-1, P, E)[page, row].double()
                    y = retrieved[l, kv].view(-1, P, E)[page, row].double()
                    lim = m1[l, kv].double()[:, None] * (0.5 / MAX + 2.0 ** -8 + 2.0 ** -20)
                    over = ((y - x).abs() - lim).max()
                    worst = max(worst, float(over))
    say("  worst excess over the bound", worst)
    assert worst <= 0.0
    del pool, paged, batch, chunk_sets, orig, retrieved, ref
    _free()


def test_full_llama8b_planned_store_and_ordered_retrieve():
    # the headline step as the benchmark runs it: the store through its
    # address plan, the retrieve (30 hit chunks of 8 x 10000 tokens) through
    # the ordered scatter; both compared in full
    _full_bf16(wl.llama8b(), [30 * 256] * 8, workspaces=True)
