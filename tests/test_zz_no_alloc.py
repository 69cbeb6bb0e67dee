"""The retrieve that allocates nothing (kv_retrieve_chunks_noalloc, the
ordered retrieve on the library's own scratch array) against the same
retrieve with a caller's workspace (kv_retrieve_chunks_ws), bit for bit, on
the same inputs.  The no-allocation calls run one after another, each on a
smaller input than the last, so every call finds the previous call's
leftovers in the shared scratch: a pool above 32768 pages (inverse map in the
scratch), then pools below it (inverse map in LDS), in every format."""
import numpy as np
import pytest
import torch

import paged_kv_movement_amd as kvm
from paged_kv_movement_amd import workloads as wl
from gpu_util import say, setup_device, host_from_dev_pool, sync

pytestmark = pytest.mark.gpu

SENTINEL = 0x7E57


def _case(w, fmt):
    """(pool, paged, batch, reference pool, reference token counts): the
    workload stored in fmt, then retrieved through kv_retrieve_chunks_ws into
    a sentinel pool; the pool is left at the sentinel again."""
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xCD)
    kvm.store(paged, batch, fmt)
    sync()
    pool.view(torch.int16).fill_(SENTINEL)
    ws = paged.new_workspace()
    ws.fill_(0x5C)
    n_ref = kvm.retrieve(paged, batch, fmt=fmt, workspace=ws)
    sync()
    ref = host_from_dev_pool(pool)
    pool.view(torch.int16).fill_(SENTINEL)
    sync()
    assert kvm.take_faults() == 0
    return pool, paged, batch, ref, n_ref, cs


def test_noalloc_retrieve_equals_workspace_retrieve_on_shrinking_inputs():
    big = wl.custom("noalloc-big", 601, 2, 1, 8, 40000, [(0, 30000), (256, 9000), (0, 20000)],
                    masks=[np.ones(118, np.uint8), np.r_[np.ones(20, np.uint8), np.zeros(15, np.uint8)],
                           np.r_[np.ones(50, np.uint8), [0, 1], np.ones(27, np.uint8)]])
    mid = wl.custom("noalloc-mid", 602, 3, 2, 32, 9000, [(0, 5000), (512, 3000)],
                    masks=[np.r_[np.ones(15, np.uint8), np.zeros(5, np.uint8)], np.ones(10, np.uint8)],
                    outliers=2)
    small = wl.custom("noalloc-small", 603, 2, 2, 64, 300, [(0, 700)], masks=[np.array([1, 1, 0], np.uint8)],
                      outliers=2)
    tiny = wl.custom("noalloc-tiny", 604, 1, 1, 8, 20, [(0, 17)], masks=[np.array([1], np.uint8)])
    calls = 0
    for fmt in (kvm.FMT_BF16, kvm.FMT_FP8, kvm.FMT_FP8_E5M2, kvm.FMT_K16_V8):
        cases = [(big, fmt), (mid, fmt), (small, fmt), (tiny, fmt)] if fmt == kvm.FMT_BF16 else \
            [(mid, fmt), (small, fmt), (tiny, fmt)]
        for w, f in cases:
            say("case noalloc", w.name, "fmt", f, "pool pages", w.num_pages)
            pool, paged, batch, ref, n_ref, cs = _case(w, f)
            n = kvm.retrieve_noalloc(paged, batch, fmt=f)
            sync()
            calls += 1
            assert kvm.take_faults() == 0
            assert n == n_ref
            got = host_from_dev_pool(pool)
            assert np.array_equal(got, ref), (w.name, f)
            # the same call again on the same inputs (the scratch now holds
            # this call's own list) gives the same pool
            pool.view(torch.int16).fill_(SENTINEL)
            assert kvm.retrieve_noalloc(paged, batch, fmt=f) == n_ref
            sync()
            assert np.array_equal(host_from_dev_pool(pool), ref), (w.name, f, "repeat")
            del pool, paged, batch, cs
    assert calls == 13
    torch.cuda.empty_cache()


def test_noalloc_retrieve_on_a_side_stream_and_zero_hits():
    w = wl.custom("noalloc-stream", 605, 2, 2, 32, 500, [(0, 1000), (256, 800)],
                  masks=[np.array([1, 0, 1, 1], np.uint8), np.array([0, 1, 1], np.uint8)])
    pool, paged, batch, ref, n_ref, cs = _case(w, kvm.FMT_BF16)
    assert n_ref == [256, 0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    assert kvm.retrieve_noalloc(paged, batch, stream=s) == [256, 0]
    s.synchronize()
    assert np.array_equal(host_from_dev_pool(pool), ref)
    none = kvm.Batch(paged, batch.seqs).set_masks([np.zeros(4, np.uint8), np.zeros(3, np.uint8)])
    assert kvm.retrieve_noalloc(paged, none, stream=s) == [0, 0]
    s.synchronize()
    assert np.array_equal(host_from_dev_pool(pool), ref)
    assert kvm.take_faults() == 0


def test_noalloc_retrieve_with_more_sequences_than_one_pass():
    # 150 sequences: the no-allocation retrieve takes them 64 at a time (its
    # token counts stay on the stack); the pool is that of one
    # kv_retrieve_chunks_ws call over all 150
    rng = np.random.default_rng(606)
    ranges, masks = [], []
    for i in range(150):
        start = 256 * int(rng.integers(0, 2))
        end = start + int(rng.integers(1, 600))
        n_chunks = -(-(end - start) // 256)
        m = np.ones(n_chunks, np.uint8)
        if i % 5 == 0:
            m[int(rng.integers(0, n_chunks))] = 0
        ranges.append((start, end))
        masks.append(m)
    w = wl.custom("noalloc-many", 606, 2, 1, 16, 8192, ranges, masks=masks)
    for fmt in (kvm.FMT_BF16, kvm.FMT_FP8):
        say("case noalloc many sequences fmt", fmt)
        pool, paged, batch, ref, n_ref, cs = _case(w, fmt)
        assert sum(1 for n in n_ref if n > 0) > 100 and any(n > 0 for n in n_ref[128:])
        assert kvm.retrieve_noalloc(paged, batch, fmt=fmt) == n_ref
        sync()
        assert kvm.take_faults() == 0
        assert np.array_equal(host_from_dev_pool(pool), ref), fmt
        del pool, paged, batch, cs
    torch.cuda.empty_cache()


def test_noalloc_retrieve_replays_from_a_graph():
    # Code under graph capture is one of the callers this entry point is for.
    # Captured once, the retrieve is replayed three times.  Before each replay
    # an eager call on another pool (above 32768 pages, so that its inverse
    # map goes through the scratch) leaves its own contents in the shared
    # scratch.  Every replay must still give the workspace retrieve's pool.
    w = wl.custom("noalloc-graph", 607, 2, 2, 32, 300, [(0, 700), (256, 1000)],
                  masks=[np.array([1, 1, 1], np.uint8), np.array([1, 0, 1], np.uint8)])
    other = wl.custom("noalloc-graph-other", 608, 1, 1, 8, 40000, [(0, 20000), (0, 9000)])
    say("case noalloc graph replay")
    pool, paged, batch, ref, n_ref, cs = _case(w, kvm.FMT_BF16)
    opool, opaged, obatch, oref, on_ref, ocs = _case(other, kvm.FMT_BF16)
    assert n_ref == [700, 256]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm-up outside capture
        kvm.retrieve_noalloc(paged, batch)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        n = kvm.retrieve_noalloc(paged, batch)
    assert n == n_ref
    for rep in range(3):
        say("replay", rep)
        opool.view(torch.int16).fill_(SENTINEL)
        assert kvm.retrieve_noalloc(opaged, obatch) == on_ref
        sync()
        assert np.array_equal(host_from_dev_pool(opool), oref)
        pool.view(torch.int16).fill_(SENTINEL)
        sync()
        g.replay()
        sync()
        assert kvm.take_faults() == 0
        assert np.array_equal(host_from_dev_pool(pool), ref), rep
    del g
    torch.cuda.empty_cache()
