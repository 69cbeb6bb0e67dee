"""Pools whose per-layer K and V slabs exceed 4 GiB: page offsets past 2^32
bytes, in every format and call form (store, planned store, one layer's
store; chunk-major, pool-address-ordered and no-allocation retrieves, one
layer's retrieve).

Two layers of 140000 pages of 16 tokens x 1024 elements (32 KiB pages): each
slab is 4.59 GB, and page ids from 131072 on start beyond 4 GiB into their
slab.  The touched pages (three sequences, most of them on such high pages)
are filled with seeded values; everything else holds a sentinel.  The oracle
runs on a compact host pool holding only the touched pages, with the block
tables renumbered to it: a store reads, and a retrieve writes, nothing but
the pages its block table names, so this is the same computation.  After
every retrieve the touched pages are compared with the oracle's, and every
other page of the 18.4 GB pool must still hold the sentinel.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_movement_amd as kvm
from paged_kv_movement_amd import workloads as wl
from gpu_util import say, sync, alloc_dev_chunks, host_chunks, first_diff, cachegen_bins

pytestmark = pytest.mark.gpu

L, H, D, P, C = 2, 8, 128, 16, 256
E = H * D
NUM_PAGES = 140_000
HIGH = (1 << 32) // (P * E * 2)          # 131072: the first page that starts beyond 4 GiB
SENTINEL = 0x7E57
FMTS = [kvm.FMT_BF16, kvm.FMT_FP8, kvm.FMT_FP8_E5M2, kvm.FMT_K16_V8, kvm.FMT_CACHEGEN]
RANGES = [(0, 2000), (256, 1500), (0, 777)]
MASKS = [np.ones(8, np.uint8), np.array([1, 1, 0, 1, 1], np.uint8), np.ones(4, np.uint8)]


def _workload():
    """Block tables: sequence 0 on high pages only, sequence 1 half high and
    half low (interleaved), sequence 2 high; no page is shared."""
    rng = np.random.default_rng(4242)
    n = [-(-e // P) for _, e in RANGES]
    n_high = n[0] + n[1] // 2 + n[2]
    high = rng.choice(np.arange(HIGH, NUM_PAGES), size=n_high, replace=False)
    low = rng.choice(HIGH, size=n[1] - n[1] // 2, replace=False)
    mixed = np.empty(n[1], np.int64)
    mixed[0::2], mixed[1::2] = high[n[0]:n[0] + (n[1] + 1) // 2], low[:n[1] // 2]
    if n[1] % 2:
        mixed[-1] = high[n[0] + n[1] // 2]
    bts = [high[:n[0]], mixed, high[n[0] + n[1] // 2:]]
    assert sum(b.size for b in bts) == len(np.unique(np.concatenate(bts)))
    w = wl.Workload("big-pool", 4242, L, H, D, P, C, NUM_PAGES)
    for (s, e), bt, m in zip(RANGES, bts, MASKS):
        w.seqs.append(wl.Sequence(np.ascontiguousarray(bt, np.int32), s, e, m))
    return w


@pytest.fixture(scope="module")
def big():
    w = _workload()
    used = np.unique(np.concatenate([sq.block_table for sq in w.seqs])).astype(np.int64)
    assert (used >= HIGH).sum() > 0.8 * used.size and used.max() < NUM_PAGES
    rng = np.random.default_rng(7)
    x = rng.standard_normal(size=(L, 2, used.size, P, E), dtype=np.float32)
    x[..., [5, 300, 301, 777]] *= np.float32(20.0)
    data = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    say("case big-pool: pool GB", L * 2 * NUM_PAGES * P * E * 2 / 1e9, "touched pages", used.size,
        "of them beyond 4 GiB", int((used >= HIGH).sum()))
    pool = torch.empty((L, 2, NUM_PAGES, P, H, D), dtype=torch.bfloat16, device="cuda")
    pool.view(torch.int16).fill_(SENTINEL)
    idx = torch.from_numpy(used).cuda()
    pool[:, :, idx] = torch.from_numpy(data.view(np.int16)).view(torch.bfloat16).reshape(
        L, 2, used.size, P, H, D).cuda()
    sync()
    yield w, pool, used, idx, data
    del pool
    sync()
    torch.cuda.empty_cache()


def _compact(w, used):
    """The block tables renumbered onto the compact pool's pages."""
    return [np.searchsorted(used, sq.block_table).astype(np.int32) for sq in w.seqs]


def _opool(arr):
    return oracle.Pool.from_array(arr, H, D, C)


def _device_pages(pool, idx):
    return pool[:, :, idx].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(L, 2, -1, P, E)


def _untouched_elsewhere(pool, used):
    """Every page outside `used` still holds the sentinel (checked slab by slab on the device)."""
    keep = torch.ones(NUM_PAGES, dtype=torch.bool, device="cuda")
    keep[torch.from_numpy(used).cuda()] = False
    for l in range(L):
        for kv in range(2):
            bad = pool[l, kv].view(torch.int16).reshape(NUM_PAGES, -1).ne(SENTINEL).any(dim=1) & keep
            assert not bool(bad.any()), ("page outside the block tables written", l, kv,
                                         int(torch.nonzero(bad)[0]))


def _setup(w, pool, fmt):
    paged = kvm.Paged.from_pool(pool, chunk_size=C)
    seqs, chunk_sets = [], []
    for sq in w.seqs:
        bufs, sizes = alloc_dev_chunks(paged, w, sq, fmt, fill=0xCD)
        bt = torch.from_numpy(sq.block_table).cuda()
        seqs.append(kvm.Seq(bt, sq.tok_start, sq.tok_end, bufs))
        chunk_sets.append((bufs, sizes))
    batch = kvm.Batch(paged, seqs).set_masks([sq.hit_mask for sq in w.seqs])
    sync()
    return paged, batch, chunk_sets


@pytest.mark.parametrize("fmt", FMTS, ids=["bf16", "fp8", "e5m2", "k16v8", "cachegen"])
def test_pool_slabs_beyond_4gib(big, fmt):
    w, pool, used, idx, data = big
    say("case big-pool fmt", fmt)
    bins = cachegen_bins(L, 99) if fmt == kvm.FMT_CACHEGEN else None
    bts = _compact(w, used)
    # store: every chunk of every sequence against the oracle's on the compact pool
    opool = _opool(data.copy())
    expected = []
    for sq, bt in zip(w.seqs, bts):
        exp = oracle.alloc_chunks(opool, sq.tok_start, sq.tok_end, fmt)
        if fmt == kvm.FMT_CACHEGEN:
            assert oracle.store_cachegen(opool, bt, sq.tok_start, sq.tok_end, exp, *bins) == 0
        else:
            assert oracle.store(opool, bt, sq.tok_start, sq.tok_end, exp, fmt) == 0
        expected.append(exp)
    paged, batch, chunk_sets = _setup(w, pool, fmt)
    forms = ["plain"] + (["planned"] if fmt in (kvm.FMT_BF16, kvm.FMT_K16_V8) else [])
    for form in forms:
        for bufs, sizes in chunk_sets:           # so that a store writing nothing would show
            for b, n in zip(bufs, sizes):
                b[:n].fill_(0xCD)
        if fmt == kvm.FMT_CACHEGEN:
            kvm.store_cachegen(paged, batch, *bins)
        else:
            kvm.store(paged, batch, fmt, workspace=batch.new_store_workspace(fmt) if form == "planned" else None)
        sync()
        assert kvm.take_faults() == 0
        for i, (cs, exp) in enumerate(zip(chunk_sets, expected)):
            got = host_chunks(cs)
            assert len(got) == len(exp)
            for c, (g, e) in enumerate(zip(got, exp)):
                assert g.size == e.size and np.array_equal(g, e), (fmt, form, "seq", i, "chunk", c, first_diff(g, e))
        say("  store", form, ": every chunk equals the oracle's")
    chunks = [host_chunks(cs) for cs in chunk_sets]

    # retrieve with the workload's hit masks into sentinel pages, chunk-major
    # and in pool-address order (the inverse map spans 140000 pages)
    exp_pages = np.full(data.shape, SENTINEL, np.uint16)
    opool = _opool(exp_pages)
    counts = []
    for sq, bt, ch in zip(w.seqs, bts, chunks):
        if fmt == kvm.FMT_CACHEGEN:
            counts.append(oracle.retrieve_cachegen(opool, bt, sq.tok_start, sq.tok_end, sq.hit_mask, ch, *bins))
        else:
            counts.append(oracle.retrieve(opool, bt, sq.tok_start, sq.tok_end, sq.hit_mask, ch, fmt))
    assert counts == [2000, 512, 777]
    calls = ["chunk-major", "ordered"] + (["no-alloc"] if fmt != kvm.FMT_CACHEGEN else [])
    for call in calls:
        pool.view(torch.int16)[:, :, idx] = SENTINEL
        sync()
        ws = paged.new_workspace() if call == "ordered" else None
        if fmt == kvm.FMT_CACHEGEN:
            n = kvm.retrieve_cachegen(paged, batch, *bins, workspace=ws)
        elif call == "no-alloc":
            n = kvm.retrieve_noalloc(paged, batch, fmt=fmt)
        else:
            n = kvm.retrieve(paged, batch, fmt=fmt, workspace=ws)
        sync()
        assert kvm.take_faults() == 0
        assert n == counts, (fmt, call)
        got = _device_pages(pool, idx)
        assert np.array_equal(got, exp_pages), (fmt, call, first_diff(got, exp_pages))
        _untouched_elsewhere(pool, used)
        say("  retrieve", call, ": the touched pages equal the oracle's; no other page written")

    # one layer (the second, whose slabs start 9.2 GB into the pool) on its own
    if fmt != kvm.FMT_CACHEGEN:
        exp_layer = np.full(data.shape, SENTINEL, np.uint16)
        opool = _opool(exp_layer)
        for sq, bt, ch in zip(w.seqs, bts, chunks):
            oracle.retrieve(opool, bt, sq.tok_start, sq.tok_end, sq.hit_mask, ch, fmt, 1)
        pool.view(torch.int16)[:, :, idx] = SENTINEL
        sync()
        assert kvm.retrieve_layer_ex(paged, batch, 1, fmt=fmt) == counts
        sync()
        assert kvm.take_faults() == 0
        got = _device_pages(pool, idx)
        assert np.array_equal(got, exp_layer), (fmt, "layer 1", first_diff(got, exp_layer))
        _untouched_elsewhere(pool, used)
        say("  retrieve_layer 1: the touched pages equal the oracle's")
    # leave the touched pages as they were for the next format
    pool[:, :, idx] = torch.from_numpy(data.view(np.int16)).view(torch.bfloat16).reshape(
        L, 2, used.size, P, H, D).cuda()
    sync()
    if fmt != kvm.FMT_CACHEGEN:
        # one layer's store (the second), from the restored pages, into chunks
        # holding a fill byte
        for bufs, sizes in chunk_sets:
            for b, n in zip(bufs, sizes):
                b[:n].fill_(0xCD)
        opool = _opool(data.copy())
        for i, (sq, bt, cs) in enumerate(zip(w.seqs, bts, chunk_sets)):
            exp = oracle.alloc_chunks(opool, sq.tok_start, sq.tok_end, fmt, fill=0xCD)
            assert oracle.store(opool, bt, sq.tok_start, sq.tok_end, exp, fmt, 1) == 0
            if i == 0:
                kvm.store_layer(paged, batch, 1, fmt)
                sync()
                assert kvm.take_faults() == 0
            for c, (g, e) in enumerate(zip(host_chunks(cs), exp)):
                assert np.array_equal(g, e), (fmt, "store_layer 1", "seq", i, "chunk", c, first_diff(g, e))
        say("  store_layer 1: every chunk equals the oracle's")
