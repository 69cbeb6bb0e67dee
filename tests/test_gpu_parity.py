"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

bf16 movement must be bit-exact; fp8 bytes and scales bit-exact; the fp8
round trip within the closed-form bound.  Every input is seeded (see
paged_kv_movement_amd/workloads.py); every expected value comes from oracle/.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_movement_amd as kvm
from paged_kv_movement_amd import workloads as wl
from gpu_util import (say, dev_pool_from_host, host_from_dev_pool, oracle_pool, chunk_tokens,
                      setup_device, host_chunks, check_store, check_retrieve, first_diff, sync as _sync)

pytestmark = pytest.mark.gpu

BF16, FP8, E5M2, K16V8 = kvm.FMT_BF16, kvm.FMT_FP8, kvm.FMT_FP8_E5M2, kvm.FMT_K16_V8
SENTINEL = 0x7E57
ALL_FMTS = dict(argvalues=[BF16, FP8, E5M2, K16V8], ids=["bf16", "fp8", "e5m2", "k16v8"])
FP8_FMTS = dict(argvalues=[FP8, E5M2], ids=["fp8", "e5m2"])


def _outliers(fmt):
    return 0 if fmt == BF16 else 2


def _roundtrip(w, fmt=BF16, fill=0x0000, masks=None):
    say("case", w.name, "fmt", fmt, "fill", hex(fill))
    arr = wl.host_pool(w)
    pool, paged, batch, chunk_sets = setup_device(w, arr, fmt=fmt, fill=0xCD)
    kvm.store(paged, batch, fmt)
    _sync()
    assert kvm.take_faults() == 0
    assert np.array_equal(host_from_dev_pool(pool), arr), "store wrote the pool"
    check_store(w, arr, chunk_sets, fmt)
    masks = masks if masks is not None else [sq.hit_mask for sq in w.seqs]
    pool.view(torch.int16).fill_(int(np.uint16(fill).view(np.int16)))
    before = np.full_like(arr, fill)
    n = kvm.retrieve(paged, batch, masks=masks, fmt=fmt)
    _sync()
    assert kvm.take_faults() == 0
    counts = check_retrieve(w, before, host_from_dev_pool(pool), chunk_sets, fmt, masks)
    assert n == counts
    return n


# ------------------------------------------------------------------ small cases

def test_tiny_config():
    # L=2, 2 KV heads, head_dim 64, 64-page pool, one 256-token sequence on a
    # seeded permutation of pages: store, zero the pages, retrieve, compare
    n = _roundtrip(wl.tiny(), fill=0x0000)
    assert n == [256]
    assert _roundtrip(wl.tiny(), fill=0xA5A5) == [256]


SHAPES = [
    # name, seed, L, H, D, pages, ranges, extra kwargs
    ("tails", 101, 3, 2, 64, 400, [(0, 1), (0, 15), (0, 16), (0, 17), (0, 255), (0, 257), (0, 511)], {}),
    ("starts", 102, 2, 4, 32, 300, [(256, 700), (512, 513), (768, 1024), (0, 0), (512, 512)], {}),
    ("narrow", 103, 5, 1, 8, 200, [(0, 1000), (256, 600)], {}),
    ("wide", 104, 2, 32, 128, 96, [(0, 530), (0, 300)], {}),
    ("odd-width", 105, 3, 3, 24, 128, [(0, 777)], {}),
    ("page32", 106, 2, 2, 64, 200, [(0, 1000), (256, 301)], {"page_size": 32}),
    ("chunk128", 107, 4, 2, 16, 300, [(0, 1000), (128, 129)], {"chunk_size": 128}),
    ("page256", 108, 2, 2, 16, 40, [(0, 1000)], {"page_size": 256}),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("fmt", **ALL_FMTS)
def test_shapes_and_tails(shape, fmt):
    name, seed, L, H, D, pages, ranges, kw = shape
    w = wl.custom(name, seed, L, H, D, pages, ranges, outliers=_outliers(fmt), **kw)
    n = _roundtrip(w, fmt=fmt, fill=0x7E57)
    assert n == [e - s for (s, e) in ranges]


def test_many_sequences_span_several_launches():
    # 70 sequences: more than one launch's worth of sequence slots
    ranges = [(0, 1 + 37 * i) for i in range(70)]
    w = wl.custom("many", 111, 2, 2, 32, 6000, ranges)
    _roundtrip(w, fill=0x1234)
    for fmt in (FP8, E5M2, K16V8):
        w8 = wl.custom("many-q", 112, 2, 2, 32, 6000, ranges, outliers=2)
        _roundtrip(w8, fmt=fmt, fill=0x1234)


@pytest.mark.parametrize("fmt", **ALL_FMTS)
def test_hit_masks_holes_and_misses(fmt):
    ranges = [(0, 1000), (0, 1000), (256, 1000), (0, 1000), (0, 600)]
    masks = [np.array(m, np.uint8) for m in
             ([1, 1, 0, 1], [0, 1, 1, 1], [1, 0, 1], [1, 1, 1, 1], [1, 1, 1])]
    w = wl.custom("holes", 121, 3, 2, 32, 400, ranges, masks=masks, outliers=_outliers(fmt))
    n = _roundtrip(w, fmt=fmt, fill=0xA5A5)
    assert n == [512, 0, 256, 1000, 600]


def test_all_miss_leaves_pool_untouched():
    ranges = [(0, 700), (256, 900)]
    masks = [np.zeros(3, np.uint8), np.array([0, 1, 1], np.uint8)]
    w = wl.custom("miss", 131, 2, 2, 32, 200, ranges, masks=masks)
    assert _roundtrip(w, fill=0xBEEF) == [0, 0]


def test_byte_transparency_random_bits():
    w = wl.custom("bits", 141, 3, 2, 64, 300, [(0, 1000), (256, 777)], values="bits")
    _roundtrip(w, fill=0x0000)


def test_store_is_deterministic_and_leaves_pool():
    for fmt in (BF16, FP8, E5M2, K16V8):
        w = wl.custom("det", 151, 2, 2, 64, 200, [(0, 900)], outliers=4)
        arr = wl.host_pool(w)
        pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0x11)
        kvm.store(paged, batch, fmt)
        first = [b.clone() for b in cs[0][0]]
        for b in cs[0][0]:
            b[: b.numel() - 256].fill_(0x22)
        kvm.store(paged, batch, fmt)
        _sync()
        assert all(torch.equal(a, b) for a, b in zip(first, cs[0][0]))


# ------------------------------------------------------- store through an address plan

def _planned_store(w, fmt, ws=None):
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xCD)
    if ws is None:
        ws = batch.new_store_workspace(fmt)
    if fmt in (FP8, E5M2):
        assert ws is None                            # no bf16 part: nothing to plan
    kvm.store(paged, batch, fmt, workspace=ws)
    _sync()
    assert kvm.take_faults() == 0
    assert np.array_equal(host_from_dev_pool(pool), arr), "store wrote the pool"
    check_store(w, arr, cs, fmt)


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("fmt", **ALL_FMTS)
def test_planned_store_shapes_and_tails(shape, fmt):
    name, seed, L, H, D, pages, ranges, kw = shape
    say("case planned store", name, fmt)
    _planned_store(wl.custom(name, seed, L, H, D, pages, ranges, outliers=_outliers(fmt), **kw), fmt)


def test_planned_store_many_sequences_and_reused_workspace():
    # 70 sequences: several launches, each writing its plan over the last one's
    ranges = [(0, 1 + 37 * i) for i in range(70)]
    for fmt in (BF16, K16V8):
        _planned_store(wl.custom("plan-many", 113, 2, 2, 32, 6000, ranges, outliers=_outliers(fmt)), fmt)
    # one workspace, larger than needed, over two different calls
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    _planned_store(wl.custom("plan-reuse", 114, 3, 2, 64, 300, [(0, 1000), (256, 700)]), BF16, ws=ws)
    _planned_store(wl.custom("plan-reuse2", 115, 2, 4, 32, 200, [(0, 300)]), BF16, ws=ws)


def test_planned_store_bad_page_and_bad_chunk_are_skipped_and_reported():
    w = wl.custom("plan-bad", 202, 2, 2, 32, 64, [(0, 300)])
    arr = wl.host_pool(w)
    good_bt = w.seqs[0].block_table.copy()
    w.seqs[0].block_table = good_bt.copy()
    w.seqs[0].block_table[3] = 64                  # == num_pages: out of range
    pool, paged, batch, cs = setup_device(w, arr, fill=0xCD)
    assert kvm.take_faults() == 0
    kvm.store(paged, batch, workspace=batch.new_store_workspace())
    assert kvm.take_faults() == 1
    got = host_chunks(cs[0])
    exp = oracle.alloc_chunks(oracle_pool(w, arr), 0, 300, BF16)
    assert oracle.store(oracle_pool(w, arr), good_bt, 0, 300, exp) == 0
    E, L = w.width, w.num_layers
    g0 = got[0].view(np.uint16).reshape(L, 2, 256, E)
    e0 = exp[0].view(np.uint16).reshape(L, 2, 256, E)
    assert (g0[:, :, 48:64] == 0xCDCD).all()       # the bad page's rows untouched, every other row stored
    assert np.array_equal(np.delete(g0, range(48, 64), axis=2), np.delete(e0, range(48, 64), axis=2))
    assert np.array_equal(got[1], exp[1])
    # a misaligned chunk address: that chunk skipped, the other stored
    bufs = cs[0][0]
    bufs[0].fill_(0xCD)
    bufs[0][cs[0][1][0]:] = 0x5A
    addrs = torch.tensor([bufs[0].data_ptr() + 8, bufs[1].data_ptr()], dtype=torch.int64).cuda()
    seq = kvm.Seq(torch.from_numpy(good_bt).cuda(), 0, 300, addrs)
    b2 = kvm.Batch(paged, [seq])
    kvm.store(paged, b2, workspace=b2.new_store_workspace())
    assert kvm.take_faults() == 2
    assert (bufs[0].cpu().numpy()[: cs[0][1][0]] == 0xCD).all()
    assert np.array_equal(host_chunks(([bufs[1]], [cs[0][1][1]]))[0], exp[1])


# ------------------------------------------------------------------ layerwise

@pytest.mark.parametrize("fmt", **ALL_FMTS)
def test_layerwise_on_copy_stream_equals_full(fmt):
    w = wl.custom("layers", 161, 6, 2, 32, 300, [(0, 1000), (256, 530)],
                  masks=[np.array([1, 1, 0, 1], np.uint8), np.array([1, 1], np.uint8)],
                  outliers=_outliers(fmt))
    say("case layerwise fmt", fmt)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt)
    kvm.store(paged, batch, fmt)
    _sync()
    copy = torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(w.num_layers)]
    pool.view(torch.int16).fill_(0x0F0F)
    before = host_from_dev_pool(pool)
    _sync()
    prev = before
    for l in range(w.num_layers):
        # the boundary's own form (no cap, no token counts) ...
        assert kvm.retrieve_layer(paged, batch, l, fmt=fmt, stream=copy, event=events[l]) is None
        events[l].synchronize()
        now = host_from_dev_pool(pool)
        others = [x for x in range(w.num_layers) if x != l]
        assert np.array_equal(now[others], prev[others]), f"layer {l} call wrote another layer"
        prev = now
    masks = [sq.hit_mask for sq in w.seqs]
    assert check_retrieve(w, before, prev, cs, fmt, masks) == [512, 274]
    # ... and every layer in one call, each layer's event recorded after it:
    # a consumer stream that waits on event l copies layer l, which must
    # already hold its final bytes
    pool.view(torch.int16).fill_(0x0F0F)
    _sync()
    events = [torch.cuda.Event() for _ in range(w.num_layers)]
    consumer = torch.cuda.Stream()
    snaps = torch.empty_like(pool)
    assert kvm.retrieve_layers(paged, batch, 0, w.num_layers, fmt=fmt, stream=copy, events=events) == [512, 274]
    for l in range(w.num_layers):
        consumer.wait_event(events[l])
        with torch.cuda.stream(consumer):
            snaps[l].copy_(pool[l])
    _sync()
    assert np.array_equal(host_from_dev_pool(pool), prev)
    assert np.array_equal(host_from_dev_pool(snaps), prev)
    # ... and with a second stream taking every other layer: the sentinel
    # fill enqueued on the copy stream just before the call (behind a GEMM,
    # not waited for) must land before every layer, the per-layer snapshots
    # must see each layer final, and a copy enqueued on the copy stream after
    # the call must see every layer
    alt = torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(w.num_layers)]
    snaps.zero_()
    whole = torch.empty_like(pool)
    x = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    _sync()
    with torch.cuda.stream(copy):
        torch.mm(x, x)
        pool.view(torch.int16).fill_(0x0F0F)
    assert kvm.retrieve_layers(paged, batch, 0, w.num_layers, fmt=fmt, stream=copy, events=events,
                               alt_stream=alt) == [512, 274]
    with torch.cuda.stream(copy):
        whole.copy_(pool)
    for l in range(w.num_layers):
        consumer.wait_event(events[l])
        with torch.cuda.stream(consumer):
            snaps[l].copy_(pool[l])
    _sync()
    assert np.array_equal(host_from_dev_pool(pool), prev)
    assert np.array_equal(host_from_dev_pool(snaps), prev)
    assert np.array_equal(host_from_dev_pool(whole), prev)
    assert kvm.take_faults() == 0


def test_layer_event_recorded_without_hits():
    # the event must be recorded by the call even when nothing hits: record it
    # early, queue ~ms of work on the copy stream, then check the call moved it
    w = wl.custom("nohit", 171, 2, 1, 16, 64, [(0, 300)], masks=[np.array([0, 1], np.uint8)])
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr)
    s = torch.cuda.Stream()
    t0 = torch.cuda.Event(enable_timing=True)
    ev = torch.cuda.Event(enable_timing=True)
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.randn(4096, 4096, device="cuda")
    _sync()
    with torch.cuda.stream(s):
        t0.record(s)
        ev.record(s)
        for _ in range(8):
            c = torch.mm(a, b)
    assert kvm.retrieve_layer_ex(paged, batch, 1, stream=s, event=ev) == [0]
    ev.synchronize()
    assert t0.elapsed_time(ev) > 0.2, "the layer event was not re-recorded after the queued work"
    del c


# ------------------------------------------------------------------ fp8 specifics

@pytest.mark.parametrize("fmt", **FP8_FMTS)
def test_fp8_zero_nan_and_extreme_groups(fmt):
    w = wl.custom("fp8-special", 181, 2, 1, 16, 64, [(0, 40)], masks=[np.array([1], np.uint8)])
    arr = wl.host_pool(w)
    bt = w.seqs[0].block_table
    arr[0, 0, bt[:3]] = 0                       # layer 0 K: all zeros ...
    arr[0, 0, bt[0], 0, ::2] = 0x8000           # ... with some -0
    arr[0, 1, bt[1], 5, 3] = 0x7FC1             # layer 0 V: one NaN
    arr[1, 0, bt[2], 2, 7] = 0x7F80             # layer 1 K: +inf
    arr[1, 1, bt[:3]] = 0x0001                  # layer 1 V: smallest subnormal everywhere
    arr[1, 1, bt[0], 0, 0] = 0x8005
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xCD)
    kvm.store(paged, batch, fmt)
    _sync()
    got = host_chunks(cs[0])[0]
    exp = oracle.alloc_chunks(oracle_pool(w, arr), 0, 40, fmt)
    assert oracle.store(oracle_pool(w, arr), bt, 0, 40, exp, fmt) == 0
    exp = exp[0]
    n = 2 * 2 * 40 * w.width
    # NaN results (x / NaN, inf / inf) have fixed bits on both sides: codes
    # 0x7F | the element's sign, the scale 0x7FC00000
    assert np.array_equal(got, exp), first_diff(got, exp)
    se = exp[n:].view(np.float32)
    assert list(np.isnan(se)) == [False, True, False, False]
    assert se[0] == 1.0 and np.isinf(se[2]) and exp[n:].view(np.uint32)[1] == 0x7FC00000
    for ws in (None, paged.new_workspace()):          # both retrieve orders
        pool.view(torch.int16).fill_(0)
        kvm.retrieve(paged, batch, fmt=fmt, workspace=ws)
        _sync()
        got = host_from_dev_pool(pool)
        exp = np.zeros_like(arr)
        op = oracle_pool(w, exp)
        assert oracle.retrieve(op, bt, 0, 40, [1], host_chunks(cs[0]), fmt) == 40
        # NaN values are the bf16 quiet NaN with their code's sign, on both sides
        assert (((exp & 0x7F80) == 0x7F80) & ((exp & 0x7F) != 0)).any()
        assert np.array_equal(got, exp), first_diff(got, exp)


@pytest.mark.parametrize("fmt", **FP8_FMTS)
def test_fp8_retrieve_of_nan_and_infinite_codes_under_finite_scales(fmt):
    # chunk bytes the store never writes (NaN codes, and e5m2's infinity
    # codes, under a finite scale), as a chunk from elsewhere could hold them:
    # the retrieve gives the oracle's values bit for bit
    w = wl.custom("fp8-codes", 182, 2, 1, 16, 64, [(0, 40)], masks=[np.array([1], np.uint8)])
    arr = wl.host_pool(w)
    bt = w.seqs[0].block_table
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xCD)
    kvm.store(paged, batch, fmt)
    _sync()
    buf = cs[0][0][0]
    size = cs[0][1][0]
    host = buf[:size].cpu().numpy()
    kinds = [(0, 1)] if fmt == K16V8 else [(0, 0), (0, 1), (1, 0), (1, 1)]
    L, E = w.num_layers, w.width
    rng = np.random.default_rng(182)
    codes = [0x7F, 0xFF] + ([0x7C, 0xFC, 0x7D, 0xFE] if fmt == E5M2 else [])
    planted = 0
    for l, kv in kinds:
        # byte offset of (l, kv)'s section: every quantised part is 1 byte per
        # element here, except K16/V8's bf16 K sections before each V
        off = (l * 3 * 40 * E + 2 * 40 * E) if fmt == K16V8 else (l * 2 + kv) * 40 * E
        at = off + rng.choice(40 * E, size=12, replace=False)
        host[at] = rng.choice(codes, size=12)
        planted += 12
    buf[:size].copy_(torch.from_numpy(host))
    for ws in (None, paged.new_workspace()):
        pool.view(torch.int16).fill_(0)
        kvm.retrieve(paged, batch, fmt=fmt, workspace=ws)
        _sync()
        assert kvm.take_faults() == 0
        got = host_from_dev_pool(pool)
        exp = np.zeros_like(arr)
        assert oracle.retrieve(oracle_pool(w, exp), bt, 0, 40, [1], [host], fmt) == 40
        nan_e = ((exp & 0x7F80) == 0x7F80) & ((exp & 0x7F) != 0)
        assert nan_e.sum() >= planted // 3
        assert np.array_equal(got, exp), first_diff(got, exp)


@pytest.mark.parametrize("fmt", [FP8, E5M2, K16V8], ids=["fp8", "e5m2", "k16v8"])
def test_fp8_roundtrip_error_bound_small(fmt):
    w = wl.custom("fp8-err", 191, 4, 2, 64, 400, [(0, 1000), (0, 300)], outliers=4)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt)
    kvm.store(paged, batch, fmt)
    orig = pool.clone()
    pool.zero_()
    kvm.retrieve(paged, batch, fmt=fmt)
    _sync()
    _assert_fp8_bound(w, orig, pool, cs, fmt)


# How each format holds K and V: (element kind of K, of V).  Quantised parts
# carry a float32 scale each, after the payload, in (layer, K/V) order.
PARTS = {BF16: ("bf16", "bf16"), FP8: ("e4m3", "e4m3"), E5M2: ("e5m2", "e5m2"), K16V8: ("bf16", "e4m3")}
# closed-form round-trip bound of a quantised part, and its subnormal floor
# (smallest normal of the encoding, relative to the scale)
BOUND = {"e4m3": (1 + 2.0 ** -4) * (1 + 2.0 ** -24) * (1 + 2.0 ** -8) - 1,
         "e5m2": (1 + 2.0 ** -3) * (1 + 2.0 ** -24) * (1 + 2.0 ** -8) - 1}
FLOOR = {"e4m3": 2.0 ** -6, "e5m2": 2.0 ** -14}


def _assert_fp8_bound(w, orig, pool, chunk_sets, fmt=FP8, ref_chunks=None):
    """max |x' - x| / max(|x|, floor * scale) over every stored element of a
    quantised part <= the part's closed-form bound (e4m3: 0.0667, e5m2:
    0.1295); bf16 parts come back exactly.  The scales come from ref_chunks
    (the oracle's chunks, [sequence][chunk] host arrays) when given, else
    from the device chunks."""
    L, E, P, C = w.num_layers, w.width, w.page_size, w.chunk_size
    kinds = PARTS[fmt]
    n_q = sum(k != "bf16" for k in kinds)
    worst = {k: 0.0 for k in kinds}
    for i, (sq, (bufs, sizes)) in enumerate(zip(w.seqs, chunk_sets)):
        bt = torch.from_numpy(sq.block_table.astype(np.int64)).cuda()
        for c, (b, n_c) in enumerate(zip(bufs, chunk_tokens(w, sq))):
            payload = L * n_c * E * sum(2 if k == "bf16" else 1 for k in kinds)
            if ref_chunks is not None:
                b = torch.from_numpy(ref_chunks[i][c]).cuda()
            scales = b[payload: payload + L * n_q * 4].view(torch.float32).view(L, n_q)
            t = sq.tok_start + c * C + torch.arange(n_c, device="cuda")
            page, row = bt[t // P], t % P
            for l in range(L):
                for kv in range(2):
                    x = orig[l, kv].view(-1, P, E)[page, row]
                    y = pool[l, kv].view(-1, P, E)[page, row]
                    if kinds[kv] == "bf16":
                        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (l, kv)
                        continue
                    x, y = x.double(), y.double()
                    floor = FLOOR[kinds[kv]] * scales[l, kv if n_q == 2 else 0].double()
                    rel = ((y - x).abs() / torch.maximum(x.abs(), floor)).max()
                    worst[kinds[kv]] = max(worst[kinds[kv]], float(rel))
    say("fp8 worst relative error", worst)
    for k, v in worst.items():
        if k != "bf16":
            assert v <= BOUND[k], (k, v)
    assert BOUND["e4m3"] < 0.07


# ------------------------------------------------------------------ faults

def test_bad_page_id_is_skipped_and_reported():
    w = wl.custom("badpage", 201, 2, 2, 32, 64, [(0, 300)])
    arr = wl.host_pool(w)
    w.seqs[0].block_table = w.seqs[0].block_table.copy()
    good_bt = w.seqs[0].block_table.copy()
    w.seqs[0].block_table[3] = 64                  # == num_pages: out of range
    pool, paged, batch, cs = setup_device(w, arr, fill=0xCD)
    assert kvm.take_faults() == 0
    kvm.store(paged, batch)
    assert kvm.take_faults() == 1
    assert kvm.take_faults() == 0
    got = host_chunks(cs[0])
    # every row group except the bad page's is still correct; the bad one untouched
    w.seqs[0].block_table = good_bt
    exp = oracle.alloc_chunks(oracle_pool(w, arr), 0, 300, BF16)
    assert oracle.store(oracle_pool(w, arr), good_bt, 0, 300, exp) == 0
    E, L = w.width, w.num_layers
    g0 = got[0].view(np.uint16).reshape(L, 2, 256, E)
    e0 = exp[0].view(np.uint16).reshape(L, 2, 256, E)
    assert (g0[:, :, 48:64] == 0xCDCD).all()
    g0m, e0m = np.delete(g0, range(48, 64), axis=2), np.delete(e0, range(48, 64), axis=2)
    assert np.array_equal(g0m, e0m)
    assert np.array_equal(got[1], exp[1])


def test_misaligned_or_null_chunk_is_skipped_and_reported():
    w = wl.custom("badchunk", 211, 2, 2, 32, 64, [(0, 300)])
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fill=0xCD)
    bufs = cs[0][0]
    addrs = torch.tensor([bufs[0].data_ptr() + 8, bufs[1].data_ptr()], dtype=torch.int64).cuda()
    bt = torch.from_numpy(w.seqs[0].block_table).cuda()
    seq = kvm.Seq(bt, 0, 300, addrs)
    kvm.store(paged, [seq])
    assert kvm.take_faults() == 2
    assert (bufs[0].cpu().numpy()[: cs[0][1][0]] == 0xCD).all()
    exp = oracle.alloc_chunks(oracle_pool(w, arr), 0, 300, BF16)
    assert oracle.store(oracle_pool(w, arr), w.seqs[0].block_table, 0, 300, exp) == 0
    assert np.array_equal(host_chunks(([bufs[1]], [cs[0][1][1]]))[0], exp[1])
    addrs0 = torch.tensor([0, bufs[1].data_ptr()], dtype=torch.int64).cuda()
    kvm.store(paged, [kvm.Seq(bt, 0, 300, addrs0)])
    assert kvm.take_faults() == 2


def test_host_rejections_launch_nothing():
    w = wl.custom("rej", 221, 2, 2, 32, 64, [(0, 300)])
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fill=0xCD)
    bt = torch.from_numpy(w.seqs[0].block_table).cuda()
    with pytest.raises(kvm.KvError, match="multiple of chunk_size"):
        kvm.store(paged, [kvm.Seq(bt, 16, 300, cs[0][0])])
    with pytest.raises(kvm.KvError) as ei:
        kvm.store(paged, [kvm.Seq(bt[:2], 0, 300, cs[0][0])])
    assert ei.value.code == kvm.KV_ERANGE
    _sync()
    assert all((b.cpu().numpy() == 0xCD)[: b.numel() - 256].all() for b in cs[0][0])


@pytest.mark.parametrize("fmt", **FP8_FMTS)
def test_fp8_every_bf16_value_under_many_amax(fmt):
    # Each (chunk, K/V) group holds its amax followed by every bf16 value of
    # magnitude <= amax, both signs; the amax values span the whole bf16
    # range, on both sides of 2^-4 (where the kernel switches between its
    # quotient forms) and include subnormal, zero-only and largest-finite groups.
    rng = np.random.default_rng(17)
    amax = [0x3D80, 0x3D81, 0x3E00, 0x3F80, 0x3FC0, 0x4000, 0x40A0, 0x4120, 0x42A0, 0x4300, 0x4780,
            0x5000, 0x6000, 0x7000, 0x7F00, 0x7F7F, 0x3D7F, 0x3C00, 0x3000, 0x1000, 0x0080, 0x0001, 0x0000]
    amax += [int(x) for x in rng.integers(0x3D80, 0x7F7F, size=9)]
    n_groups = len(amax)                       # 32 groups = 16 chunks x (K, V), one layer
    n_chunks = n_groups // 2
    T = n_chunks * 256
    w = wl.custom("fp8-all-values", 231, 1, 8, 128, T // 16 + 8, [(0, T)])
    E = w.width
    logical = np.zeros((2, T, E), np.uint16)   # [kv, token, channel]
    for gi, a in enumerate(amax):
        c, kv = gi // 2, gi % 2
        vals = np.arange(0, a + 1, dtype=np.uint32)
        body = np.concatenate([[a], vals, vals | 0x8000]).astype(np.uint16)
        grp = np.zeros(256 * E, np.uint16)
        grp[:body.size] = body
        logical[kv, c * 256:(c + 1) * 256] = grp.reshape(256, E)
    arr = np.zeros(w.pool_shape(), np.uint16)
    bt = w.seqs[0].block_table
    t = np.arange(T)
    for kv in range(2):
        arr[0, kv][bt[t // 16], t % 16] = logical[kv]
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xCD)
    kvm.store(paged, batch, fmt)
    _sync()
    assert kvm.take_faults() == 0
    check_store(w, arr, cs, fmt)
    pool.view(torch.int16).fill_(0x7E57)
    assert kvm.retrieve(paged, batch, fmt=fmt) == [T]
    _sync()
    check_retrieve(w, np.full_like(arr, 0x7E57), host_from_dev_pool(pool), cs, fmt, [w.seqs[0].hit_mask])


@pytest.mark.parametrize("fmt", **ALL_FMTS)
@pytest.mark.parametrize("cap", [1, 7, 64])
def test_layerwise_with_capped_grid(fmt, cap):
    # a capped grid makes each workgroup walk a run of tiles; the result must
    # not depend on the cap
    w = wl.custom("capped", 241, 4, 2, 64, 300, [(0, 1000), (256, 531), (0, 17)],
                  masks=[np.array([1, 1, 0, 1], np.uint8), np.array([1, 1], np.uint8),
                         np.array([1], np.uint8)], outliers=_outliers(fmt))
    say("case capped layerwise", cap, fmt)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt)
    kvm.store(paged, batch, fmt)
    pool.view(torch.int16).fill_(0x2A2A)
    _sync()
    s = torch.cuda.Stream()
    for l in range(w.num_layers):
        assert kvm.retrieve_layer_ex(paged, batch, l, fmt=fmt, stream=s, max_workgroups=cap) == [512, 275, 17]
    torch.cuda.synchronize()
    assert kvm.take_faults() == 0
    before = np.full_like(arr, 0x2A2A)
    check_retrieve(w, before, host_from_dev_pool(pool), cs, fmt, [sq.hit_mask for sq in w.seqs])


def test_pool_from_per_layer_tensors():
    # an engine may keep one K and one V tensor per layer at unrelated addresses
    w = wl.custom("layers-separate", 251, 3, 2, 32, 80, [(0, 700), (256, 300)])
    arr = wl.host_pool(w)
    L, _, n, P, E = arr.shape
    k_layers, v_layers = [], []
    for l in range(L):
        pad = torch.empty(4096 * (l + 1), dtype=torch.uint8, device="cuda")   # unrelated allocations between layers
        k_layers.append(torch.from_numpy(arr[l, 0].view(np.int16)).view(torch.bfloat16)
                        .reshape(n, P, w.num_kv_heads, w.head_dim).cuda())
        v_layers.append(torch.from_numpy(arr[l, 1].view(np.int16)).view(torch.bfloat16)
                        .reshape(n, P, w.num_kv_heads, w.head_dim).cuda())
        del pad
    paged = kvm.Paged.from_layers(k_layers, v_layers, chunk_size=w.chunk_size)
    from gpu_util import alloc_dev_chunks
    seqs, sets = [], []
    for sq in w.seqs:
        bufs, sizes = alloc_dev_chunks(paged, w, sq, BF16, fill=0xCD)
        seqs.append(kvm.Seq(torch.from_numpy(sq.block_table).cuda(), sq.tok_start, sq.tok_end, bufs))
        sets.append((bufs, sizes))
    batch = kvm.Batch(paged, seqs).set_masks([sq.hit_mask for sq in w.seqs])
    kvm.store(paged, batch)
    _sync()
    check_store(w, arr, sets, BF16)
    for t in k_layers + v_layers:
        t.view(torch.int16).fill_(0x1111)
    assert kvm.retrieve(paged, batch) == [700, 44]
    _sync()
    got = np.stack([np.stack([k.view(torch.int16).cpu().numpy().view(np.uint16).reshape(n, P, E),
                              v.view(torch.int16).cpu().numpy().view(np.uint16).reshape(n, P, E)])
                    for k, v in zip(k_layers, v_layers)])
    check_retrieve(w, np.full_like(arr, 0x1111), got, sets, BF16, [sq.hit_mask for sq in w.seqs])


def test_copy_bytes_is_a_plain_copy():
    src = torch.randint(0, 256, (3 * 4096 * 1024 + 48,), dtype=torch.uint8, device="cuda")
    dst = torch.full_like(src, 7)
    n = src.numel() - 32
    kvm.copy_bytes(dst, src, n)
    _sync()
    assert torch.equal(dst[:n], src[:n])
    assert (dst[n:] == 7).all()


@pytest.mark.parametrize("n_blocks,block,mult", [(37, 8192, 7919), (7919, 4096, 7927), (64, 32768, 7919)])
@pytest.mark.parametrize("permute", [kvm.COPY_SCATTERED_READS, kvm.COPY_SCATTERED_WRITES], ids=["reads", "writes"])
def test_copy_blocks_is_a_block_permutation(n_blocks, block, mult, permute):
    # the measurement aid's order, as its header states it: block k of the
    # permuted side is block (k * m) mod n_blocks, m the first of 7919, 7927
    # that does not divide n_blocks; every destination byte written once
    print("case copy_blocks", n_blocks, block, permute, flush=True)
    n = n_blocks * block
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.full((n + 4096,), 7, dtype=torch.uint8, device="cuda")
    kvm.copy_blocks(dst, src, n, block, permute)
    _sync()
    perm = (np.arange(n_blocks, dtype=np.int64) * mult) % n_blocks
    assert np.array_equal(np.sort(perm), np.arange(n_blocks))
    s_blocks = src.cpu().numpy().reshape(n_blocks, block)
    want = np.empty_like(s_blocks)
    if permute == kvm.COPY_SCATTERED_READS:
        want[:] = s_blocks[perm]
    else:
        want[perm] = s_blocks
    got = dst.cpu().numpy()
    assert np.array_equal(got[:n].reshape(n_blocks, block), want)
    assert (got[n:] == 7).all()


@pytest.mark.parametrize("fmt", **ALL_FMTS)
@pytest.mark.parametrize("cap", [0, 5])
def test_layerwise_store_equals_full_store(fmt, cap):
    # storing layer by layer on a side stream (each call recording its event)
    # fills the chunks exactly as one full store; before its layer is stored,
    # a chunk section keeps what it held
    w = wl.custom("store-layers", 261, 5, 2, 32, 300, [(0, 1000), (256, 531), (0, 17)],
                  outliers=_outliers(fmt))
    say("case layerwise store", fmt, cap)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xC3)
    s = torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(w.num_layers)]
    for l in range(w.num_layers):
        kvm.store_layer(paged, batch, l, fmt=fmt, stream=s, event=events[l], max_workgroups=cap)
        events[l].synchronize()
        if l == 1:
            # layers >= 2 untouched so far: compare against an oracle store of
            # layers 0 and 1 into buffers of the same fill
            opool = oracle_pool(w, arr)
            for sq, chunk_set in zip(w.seqs, cs):
                exp = oracle.alloc_chunks(opool, sq.tok_start, sq.tok_end, fmt, fill=0xC3)
                for ll in (0, 1):
                    assert oracle.store(opool, sq.block_table, sq.tok_start, sq.tok_end, exp, fmt, ll) == 0
                got = host_chunks(chunk_set)
                assert all(np.array_equal(g, e) for g, e in zip(got, exp))
    torch.cuda.synchronize()
    assert kvm.take_faults() == 0
    check_store(w, arr, cs, fmt)


@pytest.mark.parametrize("fmt", [BF16, K16V8], ids=["bf16", "k16v8"])
def test_consumer_waiting_on_layer_event_sees_the_whole_layer(fmt):
    # the compute stream waits on layer l's event and then copies layer l of
    # the pool; the scatter runs on a one-workgroup grid (milliseconds per
    # layer), so an event recorded too early -- for k16v8, after the K launch
    # but before the V launch -- would let the copy see sentinels
    w = wl.custom("event-order", 271, 4, 8, 128, 1024, [(0, 4096), (0, 1000)], outliers=_outliers(fmt))
    say("case", w.name, fmt)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt)
    kvm.store(paged, batch, fmt)
    torch.cuda.synchronize()
    pool.view(torch.int16).fill_(SENTINEL)
    copy, compute = torch.cuda.Stream(), torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(w.num_layers)]
    torch.cuda.synchronize()
    snaps = []
    for l in range(w.num_layers):
        kvm.retrieve_layer_ex(paged, batch, l, fmt=fmt, stream=copy, event=events[l], max_workgroups=1)
        compute.wait_event(events[l])
        with torch.cuda.stream(compute):
            snaps.append(pool[l].clone())
    torch.cuda.synchronize()
    assert kvm.take_faults() == 0
    for l in range(w.num_layers):
        assert torch.equal(snaps[l].view(torch.int16), pool[l].view(torch.int16)), l
    got = host_from_dev_pool(pool)
    check_retrieve(w, np.full(got.shape, SENTINEL, np.uint16), got, cs, fmt,
                   [s.hit_mask for s in w.seqs], copy=False)


@pytest.mark.parametrize("form", ["per-layer-calls", "one-call", "one-call-two-streams"])
@pytest.mark.parametrize("fmt", [BF16, FP8, K16V8], ids=["bf16", "fp8", "k16v8"])
def test_store_waiting_on_producer_event_sees_the_layer(fmt, form):
    # the producer (compute stream) writes layer l of the pool after a GEMM and
    # records its event; the layer store on the copy stream waits on it, so the
    # chunks must hold the produced values, never the sentinel left before.
    # One store call per layer, or one call for every layer (kv_store_layers,
    # its waits on the producer's events enqueued by the library)
    w = wl.custom("producer-order", 272, 4, 8, 128, 1024, [(0, 4096), (256, 1300)],
                  outliers=_outliers(fmt))
    say("case", w.name, fmt, form)
    arr = wl.host_pool(w)
    src = dev_pool_from_host(w, arr)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xC3)
    pool.view(torch.int16).fill_(SENTINEL)
    x = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    copy, compute = torch.cuda.Stream(), torch.cuda.Stream()
    done = [torch.cuda.Event() for _ in range(w.num_layers)]
    torch.cuda.synchronize()
    for l in range(w.num_layers):
        with torch.cuda.stream(compute):
            torch.mm(x, x)
            pool[l].copy_(src[l])
            done[l].record(compute)
        if form == "per-layer-calls":
            copy.wait_event(done[l])
            kvm.store_layer(paged, batch, l, fmt=fmt, stream=copy)
    if form == "one-call":
        kvm.store_layers(paged, batch, 0, w.num_layers, fmt=fmt, stream=copy, wait_events=done)
    if form == "one-call-two-streams":
        kvm.store_layers(paged, batch, 0, w.num_layers, fmt=fmt, stream=copy, wait_events=done,
                         alt_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert kvm.take_faults() == 0
    check_store(w, arr, cs, fmt)


@pytest.mark.parametrize("fmt", **ALL_FMTS)
def test_host_chunks_offload_and_onload(fmt):
    # chunk buffers in pinned host memory: the store writes them over PCIe
    # (offload) and the retrieve reads them back (onload), bit for bit as
    # with device chunks; guards after each host buffer stay untouched
    w = wl.custom("host-chunks", 281, 3, 4, 64, 400, [(0, 1000), (256, 1555), (0, 17)],
                  masks=[[1, 1, 0, 1], [1, 1, 1, 1, 1, 1], [1]], outliers=_outliers(fmt))
    say("case", w.name, fmt)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xCD, where="host")
    assert all(b.is_pinned() for b in cs[0][0])
    kvm.store(paged, batch, fmt)
    _sync()
    assert kvm.take_faults() == 0
    check_store(w, arr, cs, fmt)
    # the offload through the address plan, over a refilled sentinel
    for bufs, sizes in cs:
        for b, n in zip(bufs, sizes):
            b[:n].fill_(0xCD)
    kvm.store(paged, batch, fmt, workspace=batch.new_store_workspace(fmt))
    _sync()
    assert kvm.take_faults() == 0
    check_store(w, arr, cs, fmt)
    masks = [s.hit_mask for s in w.seqs]
    pool.view(torch.int16).fill_(0x7E57)
    n = kvm.retrieve(paged, batch, fmt=fmt)
    _sync()
    assert kvm.take_faults() == 0
    got = host_from_dev_pool(pool)
    assert n == check_retrieve(w, np.full(got.shape, 0x7E57, np.uint16), got, cs, fmt, masks)
    # layer by layer from host chunks, on a side stream with a capped grid
    pool.view(torch.int16).fill_(0x7E57)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())       # the fill lands before the retrieve writes
    ev = torch.cuda.Event()
    for l in range(w.num_layers):
        kvm.retrieve_layer_ex(paged, batch, l, fmt=fmt, stream=s, event=ev, max_workgroups=3)
    ev.synchronize()
    assert kvm.take_faults() == 0
    assert np.array_equal(host_from_dev_pool(pool), got)


def test_host_and_device_chunks_in_one_call():
    # one batch whose sequences keep their chunks in different memories
    w = wl.custom("mixed-chunks", 282, 2, 2, 64, 200, [(0, 700), (0, 300)])
    arr = wl.host_pool(w)
    pool = dev_pool_from_host(w, arr)
    paged = kvm.Paged.from_pool(pool, chunk_size=w.chunk_size)
    from gpu_util import alloc_dev_chunks
    seqs, cs = [], []
    for sq, where in zip(w.seqs, ["host", "device"]):
        bufs, sizes = alloc_dev_chunks(paged, w, sq, BF16, 0, where)
        bt = torch.from_numpy(np.ascontiguousarray(sq.block_table, np.int32)).cuda()
        seqs.append(kvm.Seq(bt, sq.tok_start, sq.tok_end, bufs))
        cs.append((bufs, sizes))
    batch = kvm.Batch(paged, seqs).set_masks([s.hit_mask for s in w.seqs])
    kvm.store(paged, batch)
    _sync()
    check_store(w, arr, cs, BF16)
    pool.zero_()
    assert kvm.retrieve(paged, batch) == [700, 300]
    _sync()
    assert kvm.take_faults() == 0
    got = host_from_dev_pool(pool)
    check_retrieve(w, np.zeros(got.shape, np.uint16), got, cs, BF16, [s.hit_mask for s in w.seqs])


# ------------------------------------------------------------ CacheGen quantiser

from gpu_util import cachegen_bins, check_store_cachegen, check_retrieve_cachegen  # noqa: E402


def _cachegen_roundtrip(w, kb, vb, fill=0x7E57, where="device", arr=None):
    say("case cachegen", w.name, where)
    arr = wl.host_pool(w) if arr is None else arr
    pool, paged, batch, cs = setup_device(w, arr, fmt=kvm.FMT_CACHEGEN, fill=0xCD, where=where)
    kvm.store_cachegen(paged, batch, kb, vb)
    _sync()
    assert kvm.take_faults() == 0
    assert np.array_equal(host_from_dev_pool(pool), arr), "store wrote the pool"
    check_store_cachegen(w, arr, cs, kb, vb)
    masks = [sq.hit_mask for sq in w.seqs]
    pool.view(torch.int16).fill_(int(np.uint16(fill).view(np.int16)))
    n = kvm.retrieve_cachegen(paged, batch, kb, vb)
    _sync()
    assert kvm.take_faults() == 0
    counts = check_retrieve_cachegen(w, np.full_like(arr, fill), host_from_dev_pool(pool), cs, masks, kb, vb)
    assert n == counts
    return n


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_cachegen_shapes_and_tails(shape):
    name, seed, L, H, D, pages, ranges, kw = shape
    w = wl.custom(name, seed, L, H, D, pages, ranges, outliers=2, **kw)
    kb, vb = cachegen_bins(L, seed)
    assert _cachegen_roundtrip(w, kb, vb) == [e - s for (s, e) in ranges]


def test_cachegen_holes_and_host_chunks():
    ranges = [(0, 1000), (0, 1000), (256, 1000), (0, 600)]
    masks = [np.array(m, np.uint8) for m in ([1, 1, 0, 1], [0, 1, 1, 1], [1, 0, 1], [1, 1, 1])]
    w = wl.custom("cg-holes", 321, 3, 2, 32, 400, ranges, masks=masks, outliers=2)
    kb, vb = cachegen_bins(3, 321)
    assert _cachegen_roundtrip(w, kb, vb, fill=0xA5A5) == [512, 0, 256, 600]
    assert _cachegen_roundtrip(w, kb, vb, fill=0xA5A5, where="host") == [512, 0, 256, 600]


def test_cachegen_special_rows():
    # zero rows (with -0), a NaN, an infinity, rows of subnormals, rows whose
    # maximum is negative; bins at both ends of the range
    w = wl.custom("cg-special", 331, 2, 1, 64, 64, [(0, 40)], masks=[np.array([1], np.uint8)])
    arr = wl.host_pool(w)
    bt = w.seqs[0].block_table
    arr[0, 0, bt[0], 0] = 0                      # layer 0 K, token 0: zero row
    arr[0, 0, bt[0], 1, ::2] = 0x8000            # token 1: -0 in half the channels ...
    arr[0, 0, bt[0], 1, 1::2] = 0                # ... +0 in the rest
    arr[0, 1, bt[0], 2, 7] = 0x7FC1              # layer 0 V, token 2: one NaN
    arr[1, 0, bt[1], 3, 5] = 0x7F80              # layer 1 K, token 19: +inf
    arr[1, 1, bt[2], :, :] = 0x0003              # layer 1 V, tokens 32..39: subnormals
    arr[1, 1, bt[0], 4, 9] = 0xC2F0              # layer 1 V, token 4: the maximum is negative (-120)
    kb, vb = np.int32([4, 129]), np.int32([129, 4])
    pool, paged, batch, cs = setup_device(w, arr, fmt=kvm.FMT_CACHEGEN, fill=0xCD)
    kvm.store_cachegen(paged, batch, kb, vb)
    _sync()
    check_store_cachegen(w, arr, cs, kb, vb)
    pool.zero_()
    assert kvm.retrieve_cachegen(paged, batch, kb, vb) == [40]
    _sync()
    got = host_from_dev_pool(pool)
    exp = np.zeros_like(arr)
    op = oracle_pool(w, exp)
    assert oracle.retrieve_cachegen(op, bt, 0, 40, [1], host_chunks(cs[0]), kb, vb) == 40
    # NaN results (0 * inf, NaN * 0) are the bf16 quiet NaN 0x7FC0 on both sides
    assert (exp == 0x7FC0).any()
    assert np.array_equal(got, exp), first_diff(got, exp)
    # the same in pool-address order
    pool.zero_()
    assert kvm.retrieve_cachegen(paged, batch, kb, vb, workspace=paged.new_workspace()) == [40]
    _sync()
    assert np.array_equal(host_from_dev_pool(pool), exp)


# ------------------------------------------------- retrieve in pool-address order

def _ordered_roundtrip(w, fill=0x7E57, masks=None, ws=None, fmt=BF16):
    say("case ordered retrieve", w.name, fmt)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xCD)
    kvm.store(paged, batch, fmt)
    masks = masks if masks is not None else [sq.hit_mask for sq in w.seqs]
    ws = paged.new_workspace() if ws is None else ws
    ws.fill_(0x5C)                                   # contents on entry must not matter
    pool.view(torch.int16).fill_(int(np.uint16(fill).view(np.int16)))
    n = kvm.retrieve(paged, batch, masks=masks, fmt=fmt, workspace=ws)
    _sync()
    assert kvm.take_faults() == 0
    counts = check_retrieve(w, np.full_like(arr, fill), host_from_dev_pool(pool), cs, fmt, masks)
    assert n == counts
    return n


ORDERED_SHAPES = [s for s in SHAPES if s[0] in ("tails", "wide", "odd-width", "page32", "chunk128")]


@pytest.mark.parametrize("shape", ORDERED_SHAPES, ids=[s[0] for s in ORDERED_SHAPES])
@pytest.mark.parametrize("fmt", [FP8, E5M2, K16V8], ids=["fp8", "e5m2", "k16v8"])
def test_ordered_retrieve_quantised_formats(shape, fmt):
    name, seed, L, H, D, pages, ranges, kw = shape
    w = wl.custom(name, seed, L, H, D, pages, ranges, outliers=2, **kw)
    assert _ordered_roundtrip(w, fmt=fmt) == [e - s for (s, e) in ranges]


@pytest.mark.parametrize("shape", ORDERED_SHAPES, ids=[s[0] for s in ORDERED_SHAPES])
def test_ordered_retrieve_cachegen(shape):
    name, seed, L, H, D, pages, ranges, kw = shape
    w = wl.custom(name, seed, L, H, D, pages, ranges, outliers=2, **kw)
    kb, vb = cachegen_bins(L, seed + 7)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=kvm.FMT_CACHEGEN, fill=0xCD)
    kvm.store_cachegen(paged, batch, kb, vb)
    pool.view(torch.int16).fill_(0x7E57)
    ws = paged.new_workspace()
    ws.fill_(0xA3)
    n = kvm.retrieve_cachegen(paged, batch, kb, vb, workspace=ws)
    _sync()
    assert kvm.take_faults() == 0
    counts = check_retrieve_cachegen(w, np.full_like(arr, 0x7E57), host_from_dev_pool(pool), cs,
                                     [sq.hit_mask for sq in w.seqs], kb, vb)
    assert n == counts == [e - s for (s, e) in ranges]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_ordered_retrieve_shapes_and_tails(shape):
    name, seed, L, H, D, pages, ranges, kw = shape
    w = wl.custom(name, seed, L, H, D, pages, ranges, **kw)
    assert _ordered_roundtrip(w) == [e - s for (s, e) in ranges]


def test_ordered_retrieve_holes_many_sequences_and_reuse():
    ranges = [(0, 1000), (0, 1000), (256, 1000), (0, 1000), (0, 600)]
    masks = [np.array(m, np.uint8) for m in
             ([1, 1, 0, 1], [0, 1, 1, 1], [1, 0, 1], [1, 1, 1, 1], [1, 1, 1])]
    w = wl.custom("ord-holes", 351, 3, 2, 32, 400, ranges, masks=masks)
    assert _ordered_roundtrip(w, fill=0xA5A5) == [512, 0, 256, 1000, 600]
    # 70 sequences: several launches in one call, one workspace reused by each
    many = wl.custom("ord-many", 352, 2, 2, 32, 6000, [(0, 1 + 37 * i) for i in range(70)])
    _ordered_roundtrip(many, fill=0x1234)
    # one workspace across calls on different pools of the same page count
    w2 = wl.custom("ord-reuse", 353, 2, 2, 32, 400, [(0, 700), (256, 900)])
    ws = kvm.Paged.from_pool(dev_pool_from_host(w2, wl.host_pool(w2)), chunk_size=256).new_workspace()
    _ordered_roundtrip(w2, ws=ws)
    _ordered_roundtrip(wl.custom("ord-reuse2", 354, 2, 2, 32, 400, [(0, 300)]), ws=ws)


@pytest.mark.parametrize("fmt", [BF16, FP8], ids=["bf16", "fp8"])
def test_ordered_retrieve_writes_every_page_of_the_pool(fmt):
    # the call's pages are all 64 pages of the pool: the sorted list is as
    # long as the workspace allows, with no padding entry
    w = wl.custom("ord-fullpool", 357, 2, 2, 32, 64, [(0, 512), (0, 500)], outliers=2 if fmt == FP8 else 0)
    assert sum(len(sq.block_table) for sq in w.seqs) == 64
    assert _ordered_roundtrip(w, fmt=fmt) == [512, 500]


def test_ordered_retrieve_bad_page_is_skipped_and_reported():
    w = wl.custom("ord-badpage", 355, 2, 2, 32, 64, [(0, 300)])
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr)
    kvm.store(paged, batch)
    _sync()
    bt = w.seqs[0].block_table.copy()
    bt[3] = 64                                       # == num_pages: out of range
    bad = kvm.Batch(paged, [kvm.Seq(torch.from_numpy(bt.astype(np.int32)).cuda(), 0, 300, cs[0][0])])
    pool.view(torch.int16).fill_(0x7E57)
    kvm.retrieve(paged, bad, masks=[np.ones(2, np.uint8)], workspace=paged.new_workspace())
    _sync()
    assert kvm.take_faults() & 1
    # every other page was written as the oracle writes it; page 3 of the sequence was not
    got = host_from_dev_pool(pool)
    exp = np.full_like(arr, 0x7E57)
    good = w.seqs[0].block_table
    op = oracle_pool(w, exp)
    assert oracle.retrieve(op, good, 0, 300, [1, 1], host_chunks(cs[0]), BF16) == 300
    exp[:, :, good[3]] = 0x7E57                      # the skipped page keeps the sentinel
    assert np.array_equal(got, exp)


def test_ordered_retrieve_large_pool_spans_several_compaction_blocks():
    # the page-order compaction walks the inverse map 16384 pages at a time: a
    # 40000-page pool (tiny rows) takes three blocks, with hit pages in each
    w = wl.custom("ord-bigpool", 356, 2, 1, 8, 40000, [(0, 30000), (0, 20000), (256, 9000)],
                  masks=[np.ones(118, np.uint8), np.r_[np.ones(50, np.uint8), np.zeros(29, np.uint8)],
                         np.ones(35, np.uint8)])
    pages_used = np.concatenate([sq.block_table for sq in w.seqs])
    assert pages_used.max() > 32768 and pages_used.min() < 16384
    assert _ordered_roundtrip(w) == [30000, 50 * 256, 9000 - 256]


# ------------------------------------------------- page sizes that are not 16 or 32

ODD_PAGES = [(1, 128), (3, 48), (8, 64), (12, 96), (24, 48)]
ODD_FMTS = [BF16, FP8, E5M2, K16V8, kvm.FMT_CACHEGEN]


@pytest.mark.parametrize("fmt", ODD_FMTS, ids=["bf16", "fp8", "e5m2", "k16v8", "cachegen"])
@pytest.mark.parametrize("pc", ODD_PAGES, ids=[f"P{p}-C{c}" for p, c in ODD_PAGES])
def test_odd_page_sizes(pc, fmt):
    # one-row pages, page heights that are not a multiple of the four rows a
    # CacheGen retrieve tile holds, more than 64 pages per chunk (the fp8
    # store's two-pass path), tails, tok_start > 0, a one-token sequence and
    # a hole; every retrieve form against the oracle
    P, C = pc
    ranges = [(0, 3 * C + 5), (C, 2 * C + P + 1), (0, 1)]
    masks = [np.array([1, 1, 0, 1], np.uint8), np.array([1, 1], np.uint8), np.array([1], np.uint8)]
    pages = sum(-(-e // P) for (_, e) in ranges) + 7
    w = wl.custom(f"odd-P{P}", 400 + P, 2, 2, 24, pages, ranges, masks=masks, page_size=P, chunk_size=C,
                  outliers=0 if fmt == BF16 else 2)
    say("case odd page size", P, C, "fmt", fmt)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xCD)
    cg = fmt == kvm.FMT_CACHEGEN
    if cg:
        kb, vb = cachegen_bins(w.num_layers, 400 + P)
        kvm.store_cachegen(paged, batch, kb, vb)
    else:
        kvm.store(paged, batch, fmt)
    _sync()
    assert kvm.take_faults() == 0
    check_store_cachegen(w, arr, cs, kb, vb) if cg else check_store(w, arr, cs, fmt)
    if not cg:                                       # and through the address plan, over the sentinel
        for b in cs[0][0] + cs[1][0] + cs[2][0]:
            b[: b.numel() - 256].fill_(0xCD)
        kvm.store(paged, batch, fmt, workspace=batch.new_store_workspace(fmt))
        _sync()
        assert kvm.take_faults() == 0
        check_store(w, arr, cs, fmt)
    expect = [2 * C, 2 * C + P + 1 - C, 1]
    forms = ["chunk", "ordered"] if cg else ["chunk", "ordered", "layers"]
    for form in forms:
        pool.view(torch.int16).fill_(SENTINEL)
        ws = paged.new_workspace() if form == "ordered" else None
        if cg:
            n = kvm.retrieve_cachegen(paged, batch, kb, vb, workspace=ws)
        elif form == "layers":
            for l in range(w.num_layers):
                n = kvm.retrieve_layer_ex(paged, batch, l, fmt=fmt)
        else:
            n = kvm.retrieve(paged, batch, fmt=fmt, workspace=ws)
        _sync()
        assert kvm.take_faults() == 0
        before = np.full_like(arr, SENTINEL)
        got = host_from_dev_pool(pool)
        if cg:
            counts = check_retrieve_cachegen(w, before, got, cs, masks, kb, vb)
        else:
            counts = check_retrieve(w, before, got, cs, fmt, masks)
        assert n == counts == expect, (form, n, counts)


def test_cachegen_at_its_limits():
    # the largest layer count the CacheGen entry points take (128, bins per
    # layer all different) and the widest row (4096 elements), both orders
    w = wl.custom("cg-128-layers", 451, 128, 1, 8, 40, [(0, 300)], masks=[np.array([1, 1], np.uint8)],
                  page_size=16, chunk_size=256, outliers=1)
    kb = np.arange(128, dtype=np.int32) % 126 + 4
    vb = 129 - np.arange(128, dtype=np.int32) % 126
    assert _cachegen_roundtrip(w, kb, vb) == [300]
    w = wl.custom("cg-4096-wide", 452, 2, 32, 128, 40, [(0, 300)], masks=[np.array([1, 1], np.uint8)],
                  page_size=16, chunk_size=256, outliers=2)
    kb, vb = cachegen_bins(2, 452)
    assert _cachegen_roundtrip(w, kb, vb) == [300]
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=kvm.FMT_CACHEGEN, fill=0xCD)
    kvm.store_cachegen(paged, batch, kb, vb)
    pool.view(torch.int16).fill_(SENTINEL)
    assert kvm.retrieve_cachegen(paged, batch, kb, vb, workspace=paged.new_workspace()) == [300]
    _sync()
    assert kvm.take_faults() == 0
    check_retrieve_cachegen(w, np.full_like(arr, SENTINEL), host_from_dev_pool(pool), cs,
                            [sq.hit_mask for sq in w.seqs], kb, vb)


# ------------------------------------------------------------ HIP graph capture

@pytest.mark.parametrize("fmt", [BF16, FP8, kvm.FMT_CACHEGEN], ids=["bf16", "fp8", "cachegen"])
def test_store_and_ordered_retrieve_replay_from_a_graph(fmt):
    # The entry points enqueue kernels only (no allocation, no memset, no
    # host synchronisation), so a caller can capture them into a HIP graph.
    # One graph holds the store, another the ordered retrieve; each replay
    # runs on fresh pool contents written eagerly in between, and every
    # replay is checked against the oracle.
    ranges = [(0, 700), (256, 1000)]
    masks = [np.array([1, 1, 1], np.uint8), np.array([1, 0, 1], np.uint8)]
    w = wl.custom("graph", 461, 3, 2, 32, 200, ranges, masks=masks, outliers=0 if fmt == BF16 else 2)
    say("case graph replay", fmt)
    arr0 = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr0, fmt=fmt, fill=0xCD)
    cg = fmt == kvm.FMT_CACHEGEN
    kb, vb = cachegen_bins(w.num_layers, 461) if cg else (None, None)
    ws = paged.new_workspace()
    sws = None if cg else batch.new_store_workspace(fmt)    # the store's address plan (bf16 parts)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm-up outside capture
        if cg:
            kvm.store_cachegen(paged, batch, kb, vb)
            kvm.retrieve_cachegen(paged, batch, kb, vb, workspace=ws)
        else:
            kvm.store(paged, batch, fmt, workspace=sws)
            kvm.retrieve(paged, batch, fmt=fmt, workspace=ws)
    torch.cuda.synchronize()
    g_store, g_retrieve = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_store, stream=s):
        kvm.store_cachegen(paged, batch, kb, vb) if cg else kvm.store(paged, batch, fmt, workspace=sws)
    with torch.cuda.graph(g_retrieve, stream=s):
        if cg:
            n = kvm.retrieve_cachegen(paged, batch, kb, vb, workspace=ws)
        else:
            n = kvm.retrieve(paged, batch, fmt=fmt, workspace=ws)
    assert n == [700, 256]
    rng = np.random.default_rng(461)
    for rep in range(3):
        say("replay", rep)
        # new mantissa bits, same exponents: finite values stay finite
        arr = arr0 ^ rng.integers(0, 1 << 7, size=arr0.shape, dtype=np.uint16) if rep else arr0
        pool.copy_(dev_pool_from_host(w, arr))
        if sws is not None:
            sws.fill_(0x3A + rep)                        # the plan's contents on entry must not matter
        torch.cuda.synchronize()
        g_store.replay()
        torch.cuda.synchronize()
        assert kvm.take_faults() == 0
        check_store_cachegen(w, arr, cs, kb, vb) if cg else check_store(w, arr, cs, fmt)
        pool.view(torch.int16).fill_(SENTINEL + rep)
        ws.fill_(0x5C + rep)                             # workspace contents on entry must not matter
        torch.cuda.synchronize()
        g_retrieve.replay()
        torch.cuda.synchronize()
        assert kvm.take_faults() == 0
        before = np.full_like(arr, SENTINEL + rep)
        got = host_from_dev_pool(pool)
        if cg:
            counts = check_retrieve_cachegen(w, before, got, cs, masks, kb, vb)
        else:
            counts = check_retrieve(w, before, got, cs, fmt, masks)
        assert counts == [700, 256]


def test_layer_range_with_a_second_stream_replays_from_a_graph():
    # the fork onto the second stream and the join back are event record /
    # wait pairs, the form a stream capture turns into graph edges: one graph
    # holds the whole layer-range retrieve on two streams; each replay, after
    # an eager sentinel fill, must write every layer as the eager call does
    w = wl.custom("graph-2s", 462, 6, 2, 32, 300, [(0, 1000), (256, 900)],
                  masks=[np.array([1, 1, 0, 1], np.uint8), np.array([1, 1, 1], np.uint8)])
    say("case graph replay of a two-stream layer-range retrieve")
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr)
    kvm.store(paged, batch)
    s, alt = torch.cuda.Stream(), torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # eager, outside capture: the reference
        pool.view(torch.int16).fill_(SENTINEL)
        kvm.retrieve_layers(paged, batch, 0, w.num_layers, stream=s, alt_stream=alt)
    torch.cuda.synchronize()
    assert check_retrieve(w, np.full_like(arr, SENTINEL), host_from_dev_pool(pool), cs, BF16,
                          [sq.hit_mask for sq in w.seqs]) == [512, 644]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        kvm.retrieve_layers(paged, batch, 0, w.num_layers, stream=s, alt_stream=alt)
    for rep in range(3):
        pool.view(torch.int16).fill_(SENTINEL + 1 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert kvm.take_faults() == 0
        got = host_from_dev_pool(pool)
        assert check_retrieve(w, np.full_like(arr, SENTINEL + 1 + rep), got, cs, BF16,
                              [sq.hit_mask for sq in w.seqs]) == [512, 644], rep


def test_store_and_retrieve_on_two_streams_at_once():
    # an offload of two sequences on one stream while two others onload on a
    # second stream (disjoint pages, as the pool allocator guarantees): both
    # results match the oracle
    ranges = [(0, 900), (0, 650), (256, 1000), (0, 520)]
    masks = [np.ones(4, np.uint8), np.ones(3, np.uint8), np.array([1, 1, 0], np.uint8), np.ones(3, np.uint8)]
    w = wl.custom("two-streams", 471, 4, 2, 64, 300, ranges, masks=masks, outliers=2)
    say("case two streams")
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=FP8, fill=0xCD)
    a = kvm.Batch(paged, batch.seqs[:2]).set_masks(masks[:2])
    b = kvm.Batch(paged, batch.seqs[2:]).set_masks(masks[2:])
    kvm.store(paged, b, FP8)                          # b's chunks, to be onloaded
    _sync()
    # b's pages get a sentinel; a's pages keep their data for the store
    dev = host_from_dev_pool(pool)
    for sq in w.seqs[2:]:
        for p in sq.block_table:
            dev[:, :, p] = SENTINEL
    pool.copy_(dev_pool_from_host(w, dev))
    _sync()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    kvm.store(paged, a, FP8, stream=s1)
    n = kvm.retrieve(paged, b, fmt=FP8, stream=s2, workspace=paged.new_workspace())
    torch.cuda.synchronize()
    assert kvm.take_faults() == 0
    wa = wl.custom("two-streams", 471, 4, 2, 64, 300, ranges, masks=masks, outliers=2)
    wa.seqs = w.seqs[:2]
    check_store(wa, arr, cs[:2], FP8)
    wb = wl.custom("two-streams", 471, 4, 2, 64, 300, ranges, masks=masks, outliers=2)
    wb.seqs = w.seqs[2:]
    assert n == check_retrieve(wb, dev, host_from_dev_pool(pool), cs[2:], FP8, masks[2:]) == [512, 520]
