"""Plumbing shared by the GPU parity tests: moving workloads between host
numpy arrays (what the oracle reads) and device tensors (what the HIP path
reads), and allocating guarded chunk buffers.  No movement arithmetic here
beyond sizes taken from the library and from the oracle."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import paged_kv_movement_amd as kvm

GUARD = 256          # bytes after each device chunk that must stay untouched
GUARD_FILL = 0x5A


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_pool_from_host(w, arr):
    L, _, n, P, E = arr.shape
    t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    return t.reshape(L, 2, n, P, w.num_kv_heads, w.head_dim).to("cuda")


def host_from_dev_pool(pool):
    L, two, n, P, H, D = pool.shape
    return pool.view(torch.int16).cpu().numpy().view(np.uint16).reshape(L, 2, n, P, H * D)


def oracle_pool(w, arr):
    return oracle.Pool.from_array(arr, w.num_kv_heads, w.head_dim, w.chunk_size)


def chunk_tokens(w, sq):
    """Token count of each chunk of a sequence, from the oracle."""
    n = oracle.num_chunks(sq.tok_start, sq.tok_end, w.chunk_size)
    return [oracle.chunk_tokens(sq.tok_start, sq.tok_end, w.chunk_size, c) for c in range(n)]


def alloc_dev_chunks(paged, w, sq, fmt, fill=0x00, where="device"):
    """One uint8 buffer per chunk: the library's exact size + a guard.  In
    device memory, or in pinned host memory when where == "host"."""
    bufs, sizes = [], []
    for n_c in chunk_tokens(w, sq):
        size = paged.chunk_bytes(n_c, fmt)
        if where == "host":
            b = torch.empty((size + GUARD,), dtype=torch.uint8, pin_memory=True)
            b.fill_(fill)
        else:
            b = torch.full((size + GUARD,), fill, dtype=torch.uint8, device="cuda")
        b[size:] = GUARD_FILL
        bufs.append(b)
        sizes.append(size)
    return bufs, sizes


def setup_device(w, arr=None, pool=None, fmt=kvm.FMT_BF16, fill=0x00, where="device"):
    """Device pool + Paged + per-sequence chunk buffers + a Batch.  Chunk
    buffers are in device memory, or pinned host memory for where="host"."""
    if pool is None:
        pool = dev_pool_from_host(w, arr)
    paged = kvm.Paged.from_pool(pool, chunk_size=w.chunk_size)
    seqs, chunk_sets = [], []
    for sq in w.seqs:
        bufs, sizes = alloc_dev_chunks(paged, w, sq, fmt, fill, where)
        bt = torch.from_numpy(np.ascontiguousarray(sq.block_table, np.int32)).to("cuda")
        seqs.append(kvm.Seq(bt, sq.tok_start, sq.tok_end, bufs))
        chunk_sets.append((bufs, sizes))
    batch = kvm.Batch(paged, seqs).set_masks([sq.hit_mask for sq in w.seqs])
    torch.cuda.synchronize()      # fills done before any side-stream call touches the buffers
    return pool, paged, batch, chunk_sets


def host_chunks(chunk_set):
    bufs, sizes = chunk_set
    out = []
    for b, s in zip(bufs, sizes):
        h = b.cpu().numpy()
        assert (h[s:] == GUARD_FILL).all(), "a kernel wrote past the end of a chunk buffer"
        out.append(np.ascontiguousarray(h[:s]))
    return out


def first_diff(a, b):
    d = np.nonzero(a.ravel() != b.ravel())[0]
    return None if d.size == 0 else (int(d[0]), int(a.ravel()[d[0]]), int(b.ravel()[d[0]]), int(d.size))


def equal_blocked(a, b):
    """np.array_equal without a full-size temporary (pools can be ~20 GB)."""
    if a.shape != b.shape:
        return False
    fa, fb = a.reshape(a.shape[0], -1), b.reshape(b.shape[0], -1)
    return all(np.array_equal(fa[i], fb[i]) for i in range(fa.shape[0]))


def sync():
    torch.cuda.synchronize()


def check_store(w, arr, chunk_sets, fmt):
    """Oracle store of every sequence vs the device chunks."""
    opool = oracle_pool(w, arr)
    for i, (sq, cs) in enumerate(zip(w.seqs, chunk_sets)):
        got = host_chunks(cs)
        exp = oracle.alloc_chunks(opool, sq.tok_start, sq.tok_end, fmt)
        assert oracle.store(opool, sq.block_table, sq.tok_start, sq.tok_end, exp, fmt) == 0
        assert len(got) == len(exp)
        for c, (g, e) in enumerate(zip(got, exp)):
            assert g.size == e.size, (i, c)
            assert np.array_equal(g, e), (w.name, "seq", i, "chunk", c, first_diff(g, e))


def check_retrieve(w, pool_before, got_pool, chunk_sets, fmt, masks, layer=-1, copy=True):
    """Oracle retrieve (from the device's chunks) into a copy of the pool as it
    was before the call (in place when copy=False), vs the device pool after
    it; returns the oracle's token counts."""
    exp = pool_before.copy() if copy else pool_before
    opool = oracle_pool(w, exp)
    counts = []
    for sq, cs, m in zip(w.seqs, chunk_sets, masks):
        ch = host_chunks(cs)
        counts.append(oracle.retrieve(opool, sq.block_table, sq.tok_start, sq.tok_end, m, ch, fmt,
                                      layer))
    assert equal_blocked(got_pool, exp), (w.name, first_diff(got_pool, exp))
    return counts


def cachegen_bins(L, seed):
    """Seeded per-layer bin counts for K and V in [4, 129], both ends included."""
    rng = np.random.default_rng(seed)
    kb = rng.integers(4, 130, size=L).astype(np.int32)
    vb = rng.integers(4, 130, size=L).astype(np.int32)
    kb[0], vb[-1] = 4, 129
    return kb, vb


def check_store_cachegen(w, arr, chunk_sets, kb, vb):
    """Oracle CacheGen store of every sequence vs the device chunks."""
    opool = oracle_pool(w, arr)
    for i, (sq, cs) in enumerate(zip(w.seqs, chunk_sets)):
        got = host_chunks(cs)
        exp = oracle.alloc_chunks(opool, sq.tok_start, sq.tok_end, oracle.FMT_CACHEGEN)
        assert oracle.store_cachegen(opool, sq.block_table, sq.tok_start, sq.tok_end, exp, kb, vb) == 0
        assert len(got) == len(exp)
        for c, (g, e) in enumerate(zip(got, exp)):
            assert g.size == e.size, (i, c)
            assert np.array_equal(g, e), (w.name, "seq", i, "chunk", c, first_diff(g, e))


def check_retrieve_cachegen(w, pool_before, got_pool, chunk_sets, masks, kb, vb):
    """Oracle CacheGen retrieve (from the device's chunks) into a copy of the
    pool as it was, vs the device pool; returns the oracle's token counts."""
    exp = pool_before.copy()
    opool = oracle_pool(w, exp)
    counts = [oracle.retrieve_cachegen(opool, sq.block_table, sq.tok_start, sq.tok_end, m, host_chunks(cs), kb, vb)
              for sq, cs, m in zip(w.seqs, chunk_sets, masks)]
    assert equal_blocked(got_pool, exp), (w.name, first_diff(got_pool, exp))
    return counts


ORACLE_THREADS = 16      # oracle worker threads (a 16-core share of the host)


def _oracle_pool_map(fn, tasks):
    """fn over tasks on up to ORACLE_THREADS threads (each oracle call goes
    through ctypes, which releases the interpreter lock)."""
    with ThreadPoolExecutor(max(1, min(ORACLE_THREADS, os.cpu_count() or 1))) as ex:
        return list(ex.map(fn, tasks))


def _chunk_range(w, sq, c):
    """Token range of chunk c of a sequence (its length from the oracle)."""
    s = sq.tok_start + c * w.chunk_size
    return s, s + oracle.chunk_tokens(sq.tok_start, sq.tok_end, w.chunk_size, c)


def oracle_store_all(w, opool, fmt, bins=None):
    """The oracle's store of every chunk of every sequence, one task per
    (sequence, chunk) over the thread pool; returns [sequence][chunk] arrays.
    bins = (key_bins, value_bins) for the CacheGen format."""
    tasks = [(i, c) for i, sq in enumerate(w.seqs)
             for c in range(oracle.num_chunks(sq.tok_start, sq.tok_end, w.chunk_size))]

    def one(task):
        i, c = task
        sq = w.seqs[i]
        s, e = _chunk_range(w, sq, c)
        exp = oracle.alloc_chunks(opool, s, e, fmt)
        if fmt == oracle.FMT_CACHEGEN:
            rc = oracle.store_cachegen(opool, sq.block_table, s, e, exp, bins[0], bins[1])
        else:
            rc = oracle.store(opool, sq.block_table, s, e, exp, fmt)
        assert rc == 0, task
        return exp[0]

    flat = _oracle_pool_map(one, tasks)
    out = [[] for _ in w.seqs]
    for (i, _), a in zip(tasks, flat):
        out[i].append(a)
    return out


def oracle_retrieve_all(w, opool, chunks, fmt, masks, bins=None):
    """The oracle's retrieve of each sequence's leading hit chunks into
    opool (in place), one task per (sequence, hit chunk) over the thread pool:
    hit chunks of one call write distinct pages, so the tasks touch disjoint
    rows.  chunks: [sequence][chunk] host arrays.  Returns the tokens made
    available per sequence."""
    tasks, counts = [], []
    for i, (sq, m) in enumerate(zip(w.seqs, masks)):
        n = oracle.num_chunks(sq.tok_start, sq.tok_end, w.chunk_size)
        n_hit = oracle.hit_chunks(np.asarray(m, np.uint8)[:n]) if n else 0
        tasks += [(i, c) for c in range(n_hit)]
        counts.append(sum(oracle.chunk_tokens(sq.tok_start, sq.tok_end, w.chunk_size, c) for c in range(n_hit)))

    def one(task):
        i, c = task
        sq = w.seqs[i]
        s, e = _chunk_range(w, sq, c)
        if fmt == oracle.FMT_CACHEGEN:
            got = oracle.retrieve_cachegen(opool, sq.block_table, s, e, [1], [chunks[i][c]], bins[0], bins[1])
        else:
            got = oracle.retrieve(opool, sq.block_table, s, e, [1], [chunks[i][c]], fmt)
        assert got == e - s, task

    _oracle_pool_map(one, tasks)
    return counts
