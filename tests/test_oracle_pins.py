"""Pins of the CPU oracle against things other than itself (no GPU needed).

* printed values of the pages / workload definitions (tests/golden),
* a numpy page-gather + reshape formulation of store (a different mechanism
  from the oracle's per-token slot loop),
* invariants: store-then-retrieve identity, untouched rows keep a sentinel,
  prefix-hit rule with holes, layer-by-layer equals all layers, byte
  transparency for arbitrary 16-bit patterns, store leaves the pool unchanged,
* library routines: torch float8_e4m3fn and bfloat16 casts (exhaustive over
  the meaningful fp32 range), numpy float32 division and products,
* the closed-form round-trip error bound of scaled e4m3.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_movement_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")


def _gold():
    with open(GOLDEN) as f:
        return json.load(f)


def _pool(w, arr=None):
    arr = wl.host_pool(w) if arr is None else arr
    return arr, oracle.Pool.from_array(arr, w.num_kv_heads, w.head_dim, w.chunk_size)


def _numpy_gather(arr, bt, s, e, C):
    """Independent formulation: take whole pages in block-table order, flatten
    them to a token-major row array, slice [s, e), cut every C rows."""
    L = arr.shape[0]
    pages = arr[:, :, np.asarray(bt, np.int64)]            # [L, 2, n_bt, P, E]
    rows = pages.reshape(L, 2, -1, arr.shape[-1])[:, :, s:e]  # [L, 2, e-s, E]
    out = []
    for c0 in range(0, e - s, C):
        out.append(np.ascontiguousarray(rows[:, :, c0:c0 + C]).view(np.uint8).ravel())
    return out


# ------------------------------------------------------------ printed values

def test_printed_chunk_plan_and_sizes():
    g = _gold()
    C = g["chunk_size_default"]["value"]
    seq = g["sequence_10000"]
    n = oracle.num_chunks(0, seq["tokens"], C)
    assert n == seq["full_chunks"] + 1
    sizes = [oracle.chunk_tokens(0, seq["tokens"], C, c) for c in range(n)]
    assert sizes[:-1] == [C] * seq["full_chunks"] and sizes[-1] == seq["tail_tokens"]
    assert oracle.num_chunks(0, 10240, C) == 40 and oracle.chunk_tokens(0, 10240, C, 39) == 256
    assert oracle.num_chunks(0, 0, C) == 0 and oracle.num_chunks(512, 512, C) == 0
    assert oracle.num_chunks(0, 1, C) == 1 and oracle.chunk_tokens(0, 1, C, 0) == 1

    s8 = g["llama8b_shape"]
    P = g["page_tokens"]["value"]
    arr = np.zeros((s8["layers"], 2, 1, P, s8["kv_heads"] * s8["head_dim"]), np.uint16)
    pool = oracle.Pool.from_array(arr, s8["kv_heads"], s8["head_dim"], C)
    lo, hi = g["page_bytes_range"]["value"]
    page_bytes = P * s8["kv_heads"] * s8["head_dim"] * 2
    assert lo <= page_bytes <= hi and page_bytes == 32 * 1024
    assert oracle.chunk_bytes(pool, C, oracle.FMT_BF16) == 32 * 1024 * 1024
    assert oracle.chunk_bytes(pool, seq["tail_tokens"], oracle.FMT_BF16) == 16 * 32 * 2 * 1024 * 2
    numel = s8["layers"] * 2 * C * s8["kv_heads"] * s8["head_dim"]
    bpe = g["fp8_bytes_per_element"]["value"]
    assert oracle.chunk_bytes(pool, C, oracle.FMT_FP8) == numel * bpe + s8["layers"] * 2 * 4

    s70 = g["llama70b_sequence"]
    arr70 = np.zeros((s70["layers"], 2, 1, P, s70["kv_heads"] * s70["head_dim"]), np.uint16)
    pool70 = oracle.Pool.from_array(arr70, s70["kv_heads"], s70["head_dim"], C)
    n70 = oracle.num_chunks(0, s70["tokens"], C)
    assert n70 == s70["chunks"]
    total = sum(oracle.chunk_bytes(pool70, oracle.chunk_tokens(0, s70["tokens"], C, c), oracle.FMT_BF16)
                for c in range(n70))
    assert total == s70["kv_bytes"]


def test_printed_hit_mask_with_hole():
    g = _gold()["hit_mask_with_hole"]
    assert oracle.hit_chunks(g["mask"]) * 256 == g["hit_tokens"]
    assert oracle.hit_chunks([0, 1, 1]) == 0
    assert oracle.hit_chunks([1, 1, 1]) == 3
    assert oracle.hit_chunks([]) == 0


def test_slot_formula_against_page_walk():
    # token t lives in row t % P of page bt[t // P]: walk the pages explicitly
    bt = np.array([7, 3, 11, 0], np.int32)
    expected = [p * 16 + r for p in bt for r in range(16)]
    assert [oracle.slot(bt, 16, t) for t in range(64)] == expected


# --------------------------------------------------------------- bf16 moves

@pytest.mark.parametrize("case", ["tiny", "ragged", "multi"])
def test_store_matches_numpy_page_gather(case):
    if case == "tiny":
        w = wl.tiny()
    elif case == "ragged":
        # 3 chunks, tail of 37 tokens: last page partly filled; odd head_dim
        w = wl.custom("ragged", 11, 3, 1, 24, 80, [(0, 549)])
    else:
        # several sequences, one starting at a chunk boundary past 0, one empty
        w = wl.custom("multi", 12, 2, 2, 16, 160, [(0, 300), (256, 700), (512, 512), (0, 17)])
    arr, pool = _pool(w)
    before = arr.copy()
    for sq in w.seqs:
        chunks = oracle.alloc_chunks(pool, sq.tok_start, sq.tok_end, oracle.FMT_BF16, fill=0xCD)
        assert oracle.store(pool, sq.block_table, sq.tok_start, sq.tok_end, chunks) == 0
        exp = _numpy_gather(arr, sq.block_table, sq.tok_start, sq.tok_end, w.chunk_size)
        assert len(chunks) == len(exp)
        for a, b in zip(chunks, exp):
            assert a.size == b.size and np.array_equal(a, b)
    assert np.array_equal(arr, before), "store must not write the pool"


def _slots_of(w, sq, n_tokens):
    return [oracle.slot(sq.block_table, w.page_size, sq.tok_start + j) for j in range(n_tokens)]


@pytest.mark.parametrize("sentinel", [0x0000, 0xA5A5])
def test_store_clear_retrieve_identity(sentinel):
    w = wl.custom("rt", 21, 3, 2, 32, 96, [(0, 600), (256, 300)])
    arr, pool = _pool(w)
    orig = arr.copy()
    stored = []
    for sq in w.seqs:
        ch = oracle.alloc_chunks(pool, sq.tok_start, sq.tok_end, oracle.FMT_BF16)
        assert oracle.store(pool, sq.block_table, sq.tok_start, sq.tok_end, ch) == 0
        stored.append(ch)
    arr[...] = sentinel
    touched = np.zeros(arr.shape[2] * arr.shape[3], bool)
    for sq, ch in zip(w.seqs, stored):
        n = oracle.retrieve(pool, sq.block_table, sq.tok_start, sq.tok_end, sq.hit_mask, ch)
        assert n == sq.tok_end - sq.tok_start
        touched[_slots_of(w, sq, n)] = True
    flat, oflat = arr.reshape(w.num_layers, 2, -1, w.width), orig.reshape(w.num_layers, 2, -1, w.width)
    assert np.array_equal(flat[:, :, touched], oflat[:, :, touched])
    assert (flat[:, :, ~touched] == sentinel).all()


def test_retrieve_prefix_hits_and_holes():
    w = wl.custom("holes", 31, 2, 1, 16, 64, [(0, 1000)])
    arr, pool = _pool(w)
    sq = w.seqs[0]
    ch = oracle.alloc_chunks(pool, 0, 1000, oracle.FMT_BF16)
    assert oracle.store(pool, sq.block_table, 0, 1000, ch) == 0
    orig = arr.copy()
    flat, oflat = arr.reshape(2, 2, -1, w.width), orig.reshape(2, 2, -1, w.width)
    for mask, n_tok in [([1, 1, 0, 1], 512), ([0, 1, 1, 1], 0), ([1, 0, 0, 0], 256),
                        ([1, 1, 1, 1], 1000), ([1, 1, 1, 0], 768)]:
        arr[...] = 0x7E57
        n = oracle.retrieve(pool, sq.block_table, 0, 1000, np.array(mask, np.uint8), ch)
        assert n == n_tok
        hit = _slots_of(w, sq, n_tok)
        miss = sorted(set(range(flat.shape[2])) - set(hit))
        assert np.array_equal(flat[:, :, hit], oflat[:, :, hit])
        assert (flat[:, :, miss] == 0x7E57).all()


def test_layer_by_layer_equals_all_layers():
    w = wl.custom("lw", 41, 4, 2, 16, 64, [(0, 530)])
    arr, pool = _pool(w)
    sq = w.seqs[0]
    ch = oracle.alloc_chunks(pool, 0, 530, oracle.FMT_BF16)
    assert oracle.store(pool, sq.block_table, 0, 530, ch) == 0
    arr[...] = 1
    assert oracle.retrieve(pool, sq.block_table, 0, 530, sq.hit_mask, ch) == 530
    full = arr.copy()
    arr[...] = 1
    for l in range(w.num_layers):
        before = arr.copy()
        assert oracle.retrieve(pool, sq.block_table, 0, 530, sq.hit_mask, ch, layer=l) == 530
        others = [x for x in range(w.num_layers) if x != l]
        assert np.array_equal(arr[others], before[others]), "a layerwise call wrote another layer"
    assert np.array_equal(arr, full)


def test_byte_transparency_random_bit_patterns():
    w = wl.custom("bits", 51, 2, 2, 32, 48, [(0, 513)], values="bits")
    arr, pool = _pool(w)
    assert (((arr & 0x7F80) == 0x7F80) & ((arr & 0x7F) != 0)).any()   # NaN codes are among them
    sq = w.seqs[0]
    orig = arr.copy()
    ch = oracle.alloc_chunks(pool, 0, 513, oracle.FMT_BF16)
    assert oracle.store(pool, sq.block_table, 0, 513, ch) == 0
    exp = _numpy_gather(orig, sq.block_table, 0, 513, 256)
    assert all(np.array_equal(a, b) for a, b in zip(ch, exp))
    arr[...] = 0
    assert oracle.retrieve(pool, sq.block_table, 0, 513, sq.hit_mask, ch) == 513
    s = _slots_of(w, sq, 513)
    assert np.array_equal(arr.reshape(2, 2, -1, w.width)[:, :, s], orig.reshape(2, 2, -1, w.width)[:, :, s])


def test_rejected_arguments():
    w = wl.custom("bad", 61, 2, 1, 16, 32, [(0, 300)])
    arr, pool = _pool(w)
    bt = w.seqs[0].block_table
    ch = oracle.alloc_chunks(pool, 0, 300, oracle.FMT_BF16)
    assert oracle.store(pool, bt, 16, 300, ch) == -1            # start not chunk-aligned
    assert oracle.store(pool, bt, 0, 16 * bt.size + 1, ch + ch) == -1   # beyond the block table
    assert oracle.store(pool, bt, 0, 300, ch, fmt=7) == -1
    assert oracle.store(pool, bt, 0, 300, ch, layer=2) == -1          # no layer 2
    bad = bt.copy()
    bad[3] = 32                                                  # page id out of range
    assert oracle.store(pool, bad, 0, 300, ch) == -1
    dup = bt.copy()
    dup[5] = dup[2]                                              # duplicate page on retrieve
    assert oracle.store(pool, dup, 0, 300, ch) == 0              # reading twice is fine
    assert oracle.retrieve(pool, dup, 0, 300, [1, 1], ch) == -1
    assert oracle.retrieve(pool, dup, 0, 300, [0, 1], ch) == 0   # nothing written, nothing races
    assert oracle.retrieve(pool, bt, 0, 300, [1, 1], ch, layer=2) == -1


# --------------------------------------------------------------- number formats

def _torch_e4m3(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _exhaustive(encode_range, torch_cast, lo, hi):
    """Every positive fp32 pattern in [lo, hi): oracle vs the torch cast, in
    blocks spread over threads (the oracle's ctypes calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    lo, hi = int(np.float32(lo).view(np.uint32)), int(np.float32(hi).view(np.uint32))
    step = 1 << 23

    def block(b0):
        n = min(step, hi - b0)
        got = encode_range(b0, n)
        y = np.arange(b0, b0 + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
        bad = np.nonzero(got != torch_cast(y))[0]
        return None if bad.size == 0 else (hex(b0 + int(bad[0])), int(got[bad[0]]))

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        fails = [r for r in ex.map(block, range(lo, hi, step)) if r is not None]
    assert not fails, fails[:3]


def test_e4m3_encode_exhaustive_meaningful_range():
    # every positive fp32 pattern from 2^-12 up to 2^10: covers all subnormal
    # and normal E4M3 rounding decisions, the ties, and saturation
    _exhaustive(oracle.e4m3_encode_bits_range, _torch_e4m3, 2.0 ** -12, 2.0 ** 10)


def test_e4m3_encode_sampled_everywhere_and_specials():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    got = oracle.e4m3_encode(y)
    fin = np.isfinite(y)
    assert np.array_equal(got[fin], _torch_e4m3(y[fin]))
    nan = np.isnan(y)
    assert np.array_equal(got[nan], np.where(np.signbit(y[nan]), 0xFF, 0x7F).astype(np.uint8))
    sp = np.array([np.inf, -np.inf, 0.0, -0.0, 448.0, 464.0, 464.0001, -480.0, 2.0 ** -10,
                   1.5 * 2.0 ** -10, 2.0 ** -9, 2.0 ** -6, 1e-30, -1e-45], np.float32)
    assert list(oracle.e4m3_encode(sp)) == [0x7E, 0xFE, 0x00, 0x80, 0x7E, 0x7E, 0x7E, 0xFE, 0x00,
                                            0x01, 0x01, 0x08, 0x00, 0x80]


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    exp = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(exp)) and np.isnan(got).sum() == 2
    ok = ~np.isnan(exp)
    assert np.array_equal(got[ok].view(np.uint32), exp[ok].view(np.uint32))  # incl. -0
    # decode then encode is the identity on every non-NaN code
    assert np.array_equal(oracle.e4m3_encode(got[ok]), codes[ok])


def _torch_e5m2(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, np.float32)).clamp(-57344.0, 57344.0)
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_encode_exhaustive_meaningful_range():
    # every positive fp32 pattern from 2^-18 up to 2^17: all subnormal (step
    # 2^-16) and normal E5M2 rounding decisions, the ties, and saturation
    # above 57344 (the cast is clamped first, torch's own cast overflows)
    _exhaustive(oracle.e5m2_encode_bits_range, _torch_e5m2, 2.0 ** -18, 2.0 ** 17)


def test_e5m2_encode_sampled_everywhere_and_specials():
    rng = np.random.default_rng(17)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    got = oracle.e5m2_encode(y)
    fin = np.isfinite(y)
    assert np.array_equal(got[fin], _torch_e5m2(y[fin]))
    nan = np.isnan(y)
    assert np.array_equal(got[nan], np.where(np.signbit(y[nan]), 0xFF, 0x7F).astype(np.uint8))
    sp = np.array([np.inf, -np.inf, 0.0, -0.0, 57344.0, 59391.0, 59392.0, -65536.0, 2.0 ** -17,
                   1.5 * 2.0 ** -16, 2.0 ** -16, 2.0 ** -14, 1.0, 1e-30], np.float32)
    assert list(oracle.e5m2_encode(sp)) == [0x7B, 0xFB, 0x00, 0x80, 0x7B, 0x7B, 0x7B, 0xFB, 0x00,
                                            0x02, 0x01, 0x04, 0x3C, 0x00]


def test_e5m2_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e5m2_decode(codes)
    exp = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float32).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(exp)) and np.isnan(got).sum() == 6
    ok = ~np.isnan(exp)
    assert np.array_equal(got[ok].view(np.uint32), exp[ok].view(np.uint32))  # incl. -0 and inf
    fin = ok & np.isfinite(exp)
    assert np.array_equal(oracle.e5m2_encode(got[fin]), codes[fin])


def _torch_bf16(y):
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_bf16_rne_against_torch():
    # exhaustive over chosen binades (subnormal, smallest normals, around 1,
    # largest normals incl. overflow to inf), sampled elsewhere
    for exp_field in [0, 1, 2, 126, 127, 128, 200, 253, 254]:
        b0 = exp_field << 23
        bits = np.arange(b0, b0 + (1 << 23), dtype=np.uint64).astype(np.uint32)
        for sign in (0, 0x80000000):
            y = (bits | np.uint32(sign)).view(np.float32)
            assert np.array_equal(oracle.bf16_from_float(y), _torch_bf16(y)), exp_field
    rng = np.random.default_rng(8)
    y = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    fin = ~np.isnan(y)
    assert np.array_equal(oracle.bf16_from_float(y[fin]), _torch_bf16(y[fin]))
    got_nan = oracle.bf16_from_float(y[~fin])
    assert ((got_nan & 0x7F80) == 0x7F80).all() and ((got_nan & 0x007F) != 0).all()


def test_fp8_scale_is_float32_division():
    rng = np.random.default_rng(9)
    a = np.abs(rng.standard_normal(20000).astype(np.float32)) * np.float32(30)
    a = np.concatenate([a, np.float32([1e-38, 3e38, 448.0, 1.0, 2.0 ** -133])])
    got = np.array([oracle.fp8_scale(float(x)) for x in a], np.float32)
    assert np.array_equal(got.view(np.uint32), (a / np.float32(448.0)).view(np.uint32))
    assert oracle.fp8_scale(0.0) == 1.0
    got5 = np.array([oracle.e5m2_scale(float(x)) for x in a], np.float32)
    assert np.array_equal(got5.view(np.uint32), (a / np.float32(57344.0)).view(np.uint32))
    assert oracle.e5m2_scale(0.0) == 1.0


# ------------------------------------------------------------------ fp8 serde

def _numpy_fp8_store(arr, bt, s, e, C):
    """Independent formulation of gather + quantise with numpy / torch ops."""
    L = arr.shape[0]
    out = []
    for c0 in range(0, e - s, C):
        n_c = min(C, e - s - c0)
        pages = arr[:, :, np.asarray(bt, np.int64)].reshape(L, 2, -1, arr.shape[-1])
        g = pages[:, :, s + c0:s + c0 + n_c]                       # [L, 2, n_c, E] bf16 bits
        x = (g.astype(np.uint32) << 16).view(np.float32)
        amax = np.abs(x).reshape(L, 2, -1).max(axis=2)
        scale = np.where(amax == 0, np.float32(1), amax / np.float32(448.0)).astype(np.float32)
        y = x / scale[:, :, None, None]
        q = _torch_e4m3(y.ravel()).reshape(y.shape)
        out.append((np.ascontiguousarray(q).ravel(), scale.astype(np.float32).ravel()))
    return out


def test_fp8_store_matches_numpy_formulation():
    w = wl.custom("fp8", 71, 3, 2, 32, 96, [(0, 600)], outliers=4)
    arr, pool = _pool(w)
    sq = w.seqs[0]
    ch = oracle.alloc_chunks(pool, 0, 600, oracle.FMT_FP8, fill=0xEE)
    assert oracle.store(pool, sq.block_table, 0, 600, ch, oracle.FMT_FP8) == 0
    exp = _numpy_fp8_store(arr, sq.block_table, 0, 600, 256)
    for buf, (q, sc) in zip(ch, exp):
        assert buf.size == q.size + sc.size * 4
        assert np.array_equal(buf[:q.size], q)
        assert np.array_equal(buf[q.size:].view(np.float32).view(np.uint32), sc.view(np.uint32))


def test_fp8_retrieve_matches_numpy_formulation_and_error_bound():
    w = wl.custom("fp8rt", 72, 2, 2, 64, 64, [(0, 520)], outliers=4)
    arr, pool = _pool(w)
    orig = arr.copy()
    sq = w.seqs[0]
    ch = oracle.alloc_chunks(pool, 0, 520, oracle.FMT_FP8)
    assert oracle.store(pool, sq.block_table, 0, 520, ch, oracle.FMT_FP8) == 0
    arr[...] = 0
    assert oracle.retrieve(pool, sq.block_table, 0, 520, sq.hit_mask, ch, oracle.FMT_FP8) == 520
    L, E = w.num_layers, w.width
    slots = _slots_of(w, sq, 520)
    got = arr.reshape(L, 2, -1, E)[:, :, slots]                       # [L, 2, 520, E]
    x = (orig.reshape(L, 2, -1, E)[:, :, slots].astype(np.uint32) << 16).view(np.float32)
    at = 0
    for c, buf in enumerate(ch):
        n_c = oracle.chunk_tokens(0, 520, 256, c)
        q = buf[:L * 2 * n_c * E].reshape(L, 2, n_c, E)
        sc = buf[L * 2 * n_c * E:].view(np.float32).reshape(L, 2)
        d = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
        prod = (d * sc[:, :, None, None]).astype(np.float32)
        exp = _torch_bf16(prod.ravel()).reshape(prod.shape)
        assert np.array_equal(got[:, :, at:at + n_c], exp)
        # round-trip error bound: |x' - x| <= 2^-4 relative (normal range of
        # e4m3) or 2^-10 * scale absolute (subnormal range), widened by one
        # fp32 and one bf16 rounding: (1 + 2^-4)(1 + 2^-24)(1 + 2^-8) - 1
        xr = (got[:, :, at:at + n_c].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        xo = x[:, :, at:at + n_c].astype(np.float64)
        floor = (2.0 ** -6) * sc[:, :, None, None].astype(np.float64)
        rel = np.abs(xr - xo) / np.maximum(np.abs(xo), floor)
        bound = (1 + 2.0 ** -4) * (1 + 2.0 ** -24) * (1 + 2.0 ** -8) - 1
        assert rel.max() <= bound <= 0.07
        at += n_c


def test_fp8_zero_group_and_signed_zero():
    w = wl.custom("zero", 81, 1, 1, 16, 16, [(0, 16)])
    arr = np.zeros(w.pool_shape(), np.uint16)
    arr[0, 0, :, :, ::2] = 0x8000                                       # -0 in every other lane
    _, pool = _pool(w, arr)
    sq = w.seqs[0]
    ch = oracle.alloc_chunks(pool, 0, 16, oracle.FMT_FP8)
    assert oracle.store(pool, sq.block_table, 0, 16, ch, oracle.FMT_FP8) == 0
    n = 2 * 16 * 16
    q, sc = ch[0][:n].reshape(2, 16, 16), ch[0][n:].view(np.float32)
    assert list(sc) == [1.0, 1.0]
    assert (q[0, :, ::2] == 0x80).all() and (q[0, :, 1::2] == 0).all() and (q[1] == 0).all()


def test_fp8_nan_group_follows_numpy_and_torch():
    # a NaN anywhere in a group: numpy's maximum propagates it, so the scale
    # and every quotient are NaN; the NaN reading fixes their bits (scale
    # 0x7FC00000, codes 0x7F | the element's sign); the other part of the
    # chunk is unaffected.  Retrieve: every value of the NaN part is the bf16
    # quiet NaN with its code's sign.
    w = wl.custom("nan", 82, 1, 1, 16, 16, [(0, 16)])
    rng = np.random.default_rng(82)
    x = rng.standard_normal(w.pool_shape()).astype(np.float32)
    arr = (x.view(np.uint32) >> 16).astype(np.uint16)
    arr[0, 0, 3, 5, 7] = 0xFFC1                                        # one negative NaN with a payload in K
    _, pool = _pool(w, arr)
    sq = w.seqs[0]
    k_bits = arr[0, 0, sq.block_table[0]].ravel()                     # K rows of the one page, token-major
    for fmt in (oracle.FMT_FP8, oracle.FMT_FP8_E5M2):
        ch = oracle.alloc_chunks(pool, 0, 16, fmt)
        assert oracle.store(pool, sq.block_table, 0, 16, ch, fmt) == 0
        exp = _numpy_store_any(arr, sq.block_table, 0, 16, 16, fmt)[0]
        assert np.array_equal(ch[0], exp)
        n = 16 * 16
        sign = ((k_bits >> 15) & 1).astype(np.uint8)
        assert np.array_equal(ch[0][:n], (sign << 7) | 0x7F)            # 0x7F | sign, element by element
        assert 0 < sign.sum() < n                                        # both signs occur
        sc = ch[0][2 * n:].view(np.uint32)
        assert sc[0] == 0x7FC00000 and np.isfinite(sc[1:].view(np.float32)).all()
        back = np.zeros_like(arr)
        bpool = oracle.Pool.from_array(back, w.num_kv_heads, w.head_dim, w.chunk_size)
        assert oracle.retrieve(bpool, sq.block_table, 0, 16, [1], ch, fmt) == 16
        k_back = back[0, 0, sq.block_table[0]].ravel()
        assert np.array_equal(k_back, (sign.astype(np.uint16) << 15) | 0x7FC0)


@pytest.mark.parametrize("fmt", [oracle.FMT_FP8, oracle.FMT_FP8_E5M2])
def test_fp8_infinite_group_follows_ieee(fmt):
    # a group whose maximum is infinite: scale = inf / fmax = inf; a finite
    # element's quotient is a signed zero, an infinite one's inf / inf is NaN
    # (0x7F | its sign).  Retrieve: +-0 * inf and NaN both give the bf16
    # quiet NaN with the code's sign.
    w = wl.custom("inf", 83, 1, 1, 16, 16, [(0, 16)])
    rng = np.random.default_rng(83)
    arr = (rng.standard_normal(w.pool_shape()).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    sq = w.seqs[0]
    page = sq.block_table[0]
    arr[0, 1, page, 2, 3] = 0xFF80                                     # -inf in V
    arr[0, 1, page, 9, 1] = 0x7F80                                     # +inf in V
    _, pool = _pool(w, arr)
    ch = oracle.alloc_chunks(pool, 0, 16, fmt)
    assert oracle.store(pool, sq.block_table, 0, 16, ch, fmt) == 0
    n = 16 * 16
    v_bits = arr[0, 1, page].ravel()
    sign = ((v_bits >> 15) & 1).astype(np.uint8)
    inf = (v_bits & 0x7FFF) == 0x7F80
    expect = np.where(inf, (sign << 7) | 0x7F, sign << 7).astype(np.uint8)
    assert np.array_equal(ch[0][n:2 * n], expect)
    assert ch[0][2 * n:].view(np.float32)[1] == np.inf
    back = np.zeros_like(arr)
    bpool = oracle.Pool.from_array(back, w.num_kv_heads, w.head_dim, w.chunk_size)
    assert oracle.retrieve(bpool, sq.block_table, 0, 16, [1], ch, fmt) == 16
    assert np.array_equal(back[0, 1, page].ravel(), (sign.astype(np.uint16) << 15) | 0x7FC0)


# ------------------------------------------- e5m2 and asymmetric K16/V8 formats

_PARTS = {oracle.FMT_BF16: ("bf16", "bf16"), oracle.FMT_FP8: ("e4m3", "e4m3"),
          oracle.FMT_FP8_E5M2: ("e5m2", "e5m2"), oracle.FMT_K16_V8: ("bf16", "e4m3")}
_FMAX = {"e4m3": np.float32(448.0), "e5m2": np.float32(57344.0)}
_CAST = {"e4m3": _torch_e4m3, "e5m2": _torch_e5m2}
_VIEW = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
# closed-form round-trip bound of a quantised part: half a unit in the last
# place of the fp8 significand (2^-4 for 3 mantissa bits, 2^-3 for 2),
# widened by the fp32 product and the bf16 rounding
_BOUND = {k: (1 + 2.0 ** -m) * (1 + 2.0 ** -24) * (1 + 2.0 ** -8) - 1 for k, m in (("e4m3", 4), ("e5m2", 3))}


def _numpy_store_any(arr, bt, s, e, C, fmt):
    """Independent formulation of a format's chunk bytes: whole pages gathered
    with numpy, each (layer, K/V) part appended in order -- raw bf16 bytes, or
    fp8 codes from numpy's amax, a float32 division and the torch cast --
    then the float32 scales of the quantised parts."""
    L, E = arr.shape[0], arr.shape[-1]
    rows = arr[:, :, np.asarray(bt, np.int64)].reshape(L, 2, -1, E)
    out = []
    for c0 in range(0, e - s, C):
        g = rows[:, :, s + c0:min(s + c0 + C, e)]
        parts, scales = [], []
        for l in range(L):
            for kv in range(2):
                kind = _PARTS[fmt][kv]
                if kind == "bf16":
                    parts.append(np.ascontiguousarray(g[l, kv]).view(np.uint8).ravel())
                    continue
                x = (g[l, kv].astype(np.uint32) << 16).view(np.float32)
                amax = np.abs(x).max()
                scale = np.float32(1.0) if amax == 0 else np.float32(amax / _FMAX[kind])
                if np.isnan(amax):               # the NaN reading: the default quiet NaN
                    scale = np.uint32(0x7FC00000).view(np.float32)
                y = (x / scale).ravel()
                # the NaN reading: a NaN quotient is 0x7F with the element's sign bit
                sign = (g[l, kv].ravel() >> 8).astype(np.uint8) & np.uint8(0x80)
                parts.append(np.where(np.isnan(y), sign | np.uint8(0x7F), _CAST[kind](y)).astype(np.uint8))
                scales.append(scale)
        out.append(np.concatenate(parts + [np.array(scales, np.float32).view(np.uint8)]))
    return out


@pytest.mark.parametrize("fmt", [oracle.FMT_BF16, oracle.FMT_FP8, oracle.FMT_FP8_E5M2, oracle.FMT_K16_V8])
def test_store_any_format_matches_numpy_formulation(fmt):
    w = wl.custom("anyfmt", 73, 3, 2, 32, 96, [(0, 600), (256, 531)], outliers=4)
    arr, pool = _pool(w)
    for sq in w.seqs:
        ch = oracle.alloc_chunks(pool, sq.tok_start, sq.tok_end, fmt, fill=0xEE)
        assert oracle.store(pool, sq.block_table, sq.tok_start, sq.tok_end, ch, fmt) == 0
        exp = _numpy_store_any(arr, sq.block_table, sq.tok_start, sq.tok_end, 256, fmt)
        assert len(ch) == len(exp)
        for got, e in zip(ch, exp):
            assert got.size == e.size and np.array_equal(got, e)


def test_chunk_bytes_of_every_format_from_the_layout():
    # L layers x (K + V) sections of n*E elements at each part's width, plus a
    # float32 scale per quantised part and layer
    pool = oracle.Pool(32, 8, 128, 16, 256, 1, [np.zeros(16 * 1024, np.uint16)] * 32,
                       [np.zeros(16 * 1024, np.uint16)] * 32)
    for n in (256, 16, 1):
        ne = n * 1024 * 32
        assert oracle.chunk_bytes(pool, n, oracle.FMT_BF16) == ne * 4
        assert oracle.chunk_bytes(pool, n, oracle.FMT_FP8) == ne * 2 + 32 * 2 * 4
        assert oracle.chunk_bytes(pool, n, oracle.FMT_FP8_E5M2) == ne * 2 + 32 * 2 * 4
        assert oracle.chunk_bytes(pool, n, oracle.FMT_K16_V8) == ne * 3 + 32 * 4
    assert oracle.chunk_bytes(pool, 256, 9) == -1


@pytest.mark.parametrize("fmt", [oracle.FMT_FP8, oracle.FMT_FP8_E5M2, oracle.FMT_K16_V8])
def test_retrieve_any_format_matches_numpy_formulation_and_bounds(fmt):
    w = wl.custom("anyrt", 75, 2, 2, 64, 64, [(0, 520)], outliers=4)
    arr, pool = _pool(w)
    orig = arr.copy()
    sq = w.seqs[0]
    ch = oracle.alloc_chunks(pool, 0, 520, fmt)
    assert oracle.store(pool, sq.block_table, 0, 520, ch, fmt) == 0
    arr[...] = 0
    assert oracle.retrieve(pool, sq.block_table, 0, 520, sq.hit_mask, ch, fmt) == 520
    L, E = w.num_layers, w.width
    slots = _slots_of(w, sq, 520)
    got = arr.reshape(L, 2, -1, E)[:, :, slots]
    x = (orig.reshape(L, 2, -1, E)[:, :, slots].astype(np.uint32) << 16).view(np.float32)
    at = 0
    for c, buf in enumerate(ch):
        n_c = oracle.chunk_tokens(0, 520, 256, c)
        kinds = _PARTS[fmt]
        widths = [2 if k == "bf16" else 1 for k in kinds]
        payload = L * n_c * E * sum(widths)
        scales = buf[payload:].view(np.float32)
        off, si = 0, 0
        for l in range(L):
            for kv in range(2):
                nb = n_c * E * widths[kv]
                sec = buf[off:off + nb]
                off += nb
                g = got[l, kv, at:at + n_c]
                xo = x[l, kv, at:at + n_c].astype(np.float64)
                if kinds[kv] == "bf16":
                    assert np.array_equal(g, sec.view(np.uint16).reshape(n_c, E))
                    assert np.array_equal(g, orig.reshape(L, 2, -1, E)[l, kv, slots[at:at + n_c]])
                    continue
                sc = scales[si]
                si += 1
                d = torch.from_numpy(sec.copy()).view(_VIEW[kinds[kv]]).to(torch.float32).numpy()
                exp = _torch_bf16((d * sc).astype(np.float32)).reshape(n_c, E)
                assert np.array_equal(g, exp)
                xr = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                floor = {"e4m3": 2.0 ** -6, "e5m2": 2.0 ** -14}[kinds[kv]] * float(sc)
                rel = np.abs(xr - xo) / np.maximum(np.abs(xo), floor)
                assert rel.max() <= _BOUND[kinds[kv]], (l, kv, rel.max())
        assert si == scales.size
        at += n_c
    assert _BOUND["e4m3"] <= 0.07 and _BOUND["e5m2"] <= 0.13


def test_store_is_deterministic():
    w = wl.custom("det", 91, 2, 2, 32, 64, [(0, 700)], outliers=4)
    arr, pool = _pool(w)
    sq = w.seqs[0]
    for fmt in (oracle.FMT_BF16, oracle.FMT_FP8):
        a = oracle.alloc_chunks(pool, 0, 700, fmt, fill=1)
        b = oracle.alloc_chunks(pool, 0, 700, fmt, fill=2)
        assert oracle.store(pool, sq.block_table, 0, 700, a, fmt) == 0
        assert oracle.store(pool, sq.block_table, 0, 700, b, fmt) == 0
        assert all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("fmt", [oracle.FMT_BF16, oracle.FMT_FP8, oracle.FMT_FP8_E5M2, oracle.FMT_K16_V8])
def test_layer_by_layer_store_equals_full_store(fmt):
    # storing layers 0..L-1 one call at a time fills the chunks exactly as one
    # full store does, and each call writes only its own layer's sections
    w = wl.custom("lws", 42, 4, 2, 16, 64, [(0, 530)], outliers=2)
    arr, pool = _pool(w)
    sq = w.seqs[0]
    full = oracle.alloc_chunks(pool, 0, 530, fmt, fill=0x5C)
    assert oracle.store(pool, sq.block_table, 0, 530, full, fmt) == 0
    part = oracle.alloc_chunks(pool, 0, 530, fmt, fill=0x5C)
    E = w.width
    for l in range(w.num_layers):
        before = [c.copy() for c in part]
        assert oracle.store(pool, sq.block_table, 0, 530, part, fmt, layer=l) == 0
        for c, (b, a) in enumerate(zip(before, part)):
            n_c = oracle.chunk_tokens(0, 530, 256, c)
            widths = [2 if k == "bf16" else 1 for k in _PARTS[fmt]]
            n_q = sum(k != "bf16" for k in _PARTS[fmt])     # scales per layer
            sec = n_c * E * sum(widths)                      # bytes of one layer's K and V sections
            changed = np.nonzero(b != a)[0]
            payload = w.num_layers * sec
            in_sections = (changed >= l * sec) & (changed < (l + 1) * sec)
            in_scales = (changed >= payload + 4 * n_q * l) & (changed < payload + 4 * n_q * (l + 1))
            assert (in_sections | in_scales).all(), "a layer call wrote outside its layer"
    assert all(np.array_equal(a, b) for a, b in zip(full, part))
    assert oracle.store(pool, sq.block_table, 0, 530, part, fmt, layer=4) == -1


# ------------------------------------------------------- CacheGen quantiser

def _torch_cachegen_store(arr, bt, s, e, C, key_bins, value_bins):
    """The quantiser as the CacheGen page writes it, in torch float32 ops:
    MAX = bins // 2 - 1 per layer; max1 = amax(|x|) over a token's channels;
    q = round(x * (MAX / max1) + MAX) (torch.round: half to even).  A zero
    row takes factor 0 (every symbol MAX)."""
    L, E = arr.shape[0], arr.shape[-1]
    rows = arr[:, :, np.asarray(bt, np.int64)].reshape(L, 2, -1, E)
    out = []
    for c0 in range(0, e - s, C):
        g = rows[:, :, s + c0:min(s + c0 + C, e)]
        syms, maxes = [], []
        for l in range(L):
            for kv in range(2):
                MAX = float((key_bins if kv == 0 else value_bins)[l] // 2 - 1)
                x = torch.from_numpy((g[l, kv].astype(np.uint32) << 16).view(np.float32).copy())
                max1 = torch.amax(torch.abs(x), dim=-1, keepdim=True)
                # MAX is a tensor on the page (indexed by layer), so this is a
                # tensor / tensor division; a Python float over a tensor would
                # go through torch's reciprocal-and-multiply instead
                factor = torch.where(max1 == 0, torch.zeros_like(max1), torch.full_like(max1, MAX) / max1)
                q = torch.round(x * factor + MAX).clamp(0, 2 * MAX).to(torch.uint8)
                syms.append(q.numpy().ravel())
                maxes.append(max1.numpy().ravel())
        out.append(np.concatenate(syms + [np.concatenate(maxes).astype(np.float32).view(np.uint8)]))
    return out


def _cg_bins(L, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(4, 130, size=L).astype(np.int32), rng.integers(4, 130, size=L).astype(np.int32)


def test_cachegen_store_matches_torch_formulation():
    w = wl.custom("cg", 301, 4, 2, 32, 96, [(0, 600), (256, 531)], outliers=4)
    arr, pool = _pool(w)
    kb, vb = _cg_bins(w.num_layers, 5)
    kb[0], vb[0] = 4, 129                                  # both ends of the bin range
    for sq in w.seqs:
        ch = oracle.alloc_chunks(pool, sq.tok_start, sq.tok_end, oracle.FMT_CACHEGEN, fill=0xEE)
        assert oracle.store_cachegen(pool, sq.block_table, sq.tok_start, sq.tok_end, ch, kb, vb) == 0
        exp = _torch_cachegen_store(arr, sq.block_table, sq.tok_start, sq.tok_end, 256, kb, vb)
        for got, e in zip(ch, exp):
            assert got.size == e.size and np.array_equal(got, e)


def test_cachegen_layout_symbols_and_extremes():
    # sizes from the layout; every symbol of layer l lies in [0, 2*MAX_l]; the
    # element that sets a row's max1 lands on 0 or 2*MAX; a zero row is all MAX
    w = wl.custom("cgx", 302, 3, 2, 32, 64, [(0, 300)])
    arr = wl.host_pool(w)
    bt = w.seqs[0].block_table
    arr[1, 0, bt[0], 3] = 0                                # layer 1 K, token 3: zero row
    arr[1, 0, bt[0], 4, ::3] = 0x8000                      # token 4: -0 mixed in
    _, pool = _pool(w, arr)
    kb, vb = np.int32([8, 32, 129]), np.int32([4, 16, 64])
    ch = oracle.alloc_chunks(pool, 0, 300, oracle.FMT_CACHEGEN)
    L, E = w.num_layers, w.width
    assert [c.size for c in ch] == [L * 2 * n * E + L * 2 * n * 4 for n in (256, 44)]
    assert oracle.store_cachegen(pool, bt, 0, 300, ch, kb, vb) == 0
    n = 256
    sym = ch[0][:L * 2 * n * E].reshape(L, 2, n, E)
    mx = ch[0][L * 2 * n * E:].view(np.float32).reshape(L, 2, n)
    x = (arr.reshape(L, 2, -1, E)[:, :, [oracle.slot(bt, 16, t) for t in range(n)]].astype(np.uint32) << 16).view(np.float32)
    for l in range(L):
        for kv, bins in ((0, kb), (1, vb)):
            MAX = bins[l] // 2 - 1
            assert sym[l, kv].max() <= 2 * MAX
            assert np.array_equal(mx[l, kv], np.abs(x[l, kv]).max(axis=1))
            for j in range(n):
                if mx[l, kv, j] == 0:
                    assert (sym[l, kv, j] == MAX).all()
                    continue
                i = int(np.argmax(np.abs(x[l, kv, j])))
                assert sym[l, kv, j, i] == (2 * MAX if x[l, kv, j, i] > 0 else 0)
    assert mx[1, 0, 3] == 0 and (sym[1, 0, 3] == kb[1] // 2 - 1).all()


def test_cachegen_retrieve_matches_torch_and_error_bound():
    w = wl.custom("cgr", 303, 3, 2, 64, 96, [(0, 700)], masks=[np.array([1, 1, 0], np.uint8)], outliers=4)
    arr, pool = _pool(w)
    orig = arr.copy()
    sq = w.seqs[0]
    kb, vb = _cg_bins(w.num_layers, 6)
    ch = oracle.alloc_chunks(pool, 0, 700, oracle.FMT_CACHEGEN)
    assert oracle.store_cachegen(pool, sq.block_table, 0, 700, ch, kb, vb) == 0
    arr[...] = 0xA5A5
    assert oracle.retrieve_cachegen(pool, sq.block_table, 0, 700, sq.hit_mask, ch, kb, vb) == 512
    L, E = w.num_layers, w.width
    slots = _slots_of(w, sq, 700)
    got = arr.reshape(L, 2, -1, E)
    for c in range(2):                                      # the two hit chunks
        n = 256
        sym = ch[c][:L * 2 * n * E].reshape(L, 2, n, E)
        mx = ch[c][L * 2 * n * E:].view(np.float32).reshape(L, 2, n)
        rows = slots[c * 256:(c + 1) * 256]
        for l in range(L):
            for kv, bins in ((0, kb), (1, vb)):
                MAX = float(bins[l] // 2 - 1)
                q = torch.from_numpy(sym[l, kv].astype(np.float32))
                m1 = torch.from_numpy(mx[l, kv].copy())[:, None]
                mt = torch.full_like(m1, MAX)               # a tensor, as on the page
                val = (q - mt) / mt * m1                     # the page's inverse, float32
                exp = val.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                g = got[l, kv, rows]
                assert np.array_equal(g, exp), (c, l, kv)
                # half a quantisation step, widened by the float32 steps and the bf16 rounding
                xo = (orig.reshape(L, 2, -1, E)[l, kv, rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                xr = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                bound = mx[l, kv].astype(np.float64)[:, None] * (0.5 / MAX + 2.0 ** -8 + 2.0 ** -20)
                assert (np.abs(xr - xo) <= bound).all(), (c, l, kv)
    # rows of the missed chunk keep the sentinel
    assert (got[:, :, slots[512:]] == 0xA5A5).all()


def test_cachegen_nan_and_infinite_rows():
    # the NaN reading: a row holding a NaN keeps max1 = 0x7FC00000 and every
    # symbol MAX; a row whose maximum is infinite has factor MAX / inf = 0, so
    # every symbol is MAX too (inf * 0 is NaN, which also gives MAX).  Back,
    # (MAX - MAX) / MAX * max1 is 0 * NaN or 0 * inf: NaN, written 0x7FC0.
    w = wl.custom("cgn", 305, 1, 1, 16, 32, [(0, 16)])
    arr = wl.host_pool(w)
    sq = w.seqs[0]
    page = sq.block_table[0]
    arr[0, 0, page, 2, 5] = 0xFFC1                         # K row 2: a negative NaN with a payload
    arr[0, 1, page, 7, 0] = 0xFF80                         # V row 7: -inf
    _, pool = _pool(w, arr)
    kb, vb = [32], [16]
    ch = oracle.alloc_chunks(pool, 0, 16, oracle.FMT_CACHEGEN)
    assert oracle.store_cachegen(pool, sq.block_table, 0, 16, ch, kb, vb) == 0
    E = w.width
    sym = ch[0][:2 * 16 * E].reshape(2, 16, E)
    mx = ch[0][2 * 16 * E:].view(np.uint32).reshape(2, 16)
    assert mx[0, 2] == 0x7FC00000 and (sym[0, 2] == 15).all()
    assert mx[1, 7] == np.float32(np.inf).view(np.uint32) and (sym[1, 7] == 7).all()
    back = np.zeros_like(arr)
    bpool = oracle.Pool.from_array(back, w.num_kv_heads, w.head_dim, w.chunk_size)
    assert oracle.retrieve_cachegen(bpool, sq.block_table, 0, 16, [1], ch, kb, vb) == 16
    assert (back[0, 0, page, 2] == 0x7FC0).all() and (back[0, 1, page, 7] == 0x7FC0).all()
    # the other rows are finite and follow the torch formulation
    exp = _torch_cachegen_store(arr, sq.block_table, 0, 16, 256, kb, vb)[0]
    keep = np.ones((2, 16), bool)
    keep[0, 2] = keep[1, 7] = False
    assert np.array_equal(sym[keep], exp[:2 * 16 * E].reshape(2, 16, E)[keep])
    assert np.isfinite((back[0][:, page][keep].astype(np.uint32) << 16).view(np.float32)).all()


def test_cachegen_rejects_bins_out_of_range():
    w = wl.custom("cgb", 304, 2, 1, 16, 32, [(0, 40)])
    _, pool = _pool(w)
    sq = w.seqs[0]
    ch = oracle.alloc_chunks(pool, 0, 40, oracle.FMT_CACHEGEN)
    for kb, vb in (([3, 8], [8, 8]), ([8, 130], [8, 8]), ([8, 8], [8, 2])):
        assert oracle.store_cachegen(pool, sq.block_table, 0, 40, ch, kb, vb) == -1
        assert oracle.retrieve_cachegen(pool, sq.block_table, 0, 40, [1], ch, kb, vb) == -1
    assert oracle.store_cachegen(pool, sq.block_table, 0, 40, ch, [4, 129], [129, 4]) == 0
