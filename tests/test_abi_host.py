"""The C ABI without a GPU: the library loads, exports every function that
include/kvmove.h declares, and its host-side checks reject malformed calls
before any HIP call (so these run on a machine with no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import paged_kv_movement_amd as kvm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvmove.h")


def _lib():
    if not os.path.exists(kvm.library_path()):
        from paged_kv_movement_amd import build
        build.build()
    return kvm.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ["kv_store_chunks", "kv_store_layer", "kv_store_layers", "kv_retrieve_chunks", "kv_retrieve_layer",
              "kv_retrieve_layer_ex", "kv_retrieve_layers", "kv_chunk_bytes", "kv_num_chunks", "kv_chunk_tokens",
              "kv_last_error", "kv_take_faults", "kv_copy_bytes", "kv_copy_blocks"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", kvm.library_path()], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (kv_[a-z_]+)$", out, flags=re.M))
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, missing
    L = _lib()
    for n in _declared_functions():
        assert hasattr(L, n)


def test_library_is_gfx950_code_object():
    _lib()
    out = subprocess.run(["/opt/rocm/llvm/bin/llvm-readelf", "-n", kvm.library_path()],
                         capture_output=True, text=True)
    blob = open(kvm.library_path(), "rb").read()
    assert b"gfx950" in blob


def _paged(L=32, H=8, D=128, P=16, C=256, n=8192, k=0x1000, v=0x2000):
    return kvm._KvPaged(L, H, D, P, C, n, k, v)


def test_chunk_bytes_and_num_chunks():
    L = _lib()
    p = _paged()
    assert L.kv_chunk_bytes(ctypes.byref(p), 256, kvm.FMT_BF16) == 32 * 1024 * 1024
    assert L.kv_chunk_bytes(ctypes.byref(p), 16, kvm.FMT_BF16) == 16 * 32 * 2 * 1024 * 2
    assert L.kv_chunk_bytes(ctypes.byref(p), 256, kvm.FMT_FP8) == 32 * 2 * 256 * 1024 + 32 * 2 * 4
    assert L.kv_chunk_bytes(ctypes.byref(p), 256, kvm.FMT_FP8_E5M2) == 32 * 2 * 256 * 1024 + 32 * 2 * 4
    assert L.kv_chunk_bytes(ctypes.byref(p), 256, kvm.FMT_K16_V8) == 32 * 3 * 256 * 1024 + 32 * 4
    assert L.kv_chunk_bytes(ctypes.byref(p), 16, kvm.FMT_K16_V8) == 32 * 3 * 16 * 1024 + 32 * 4
    assert L.kv_chunk_bytes(ctypes.byref(p), 0, kvm.FMT_BF16) == 0
    assert L.kv_chunk_bytes(ctypes.byref(p), 256, 9) == 0
    assert L.kv_chunk_bytes(ctypes.byref(p), 256, 5) == 0
    assert L.kv_num_chunks(ctypes.byref(p), 0, 10000) == 40
    assert L.kv_num_chunks(ctypes.byref(p), 0, 10240) == 40
    assert L.kv_num_chunks(ctypes.byref(p), 512, 513) == 1
    assert L.kv_num_chunks(ctypes.byref(p), 5, 3) == -1
    # one layer's K or V section of a chunk must fit 32-bit byte counts
    assert L.kv_chunk_bytes(ctypes.byref(_paged(C=1 << 20)), 256, kvm.FMT_BF16) == 256 * 32 * 2 * 1024 * 2
    assert L.kv_chunk_bytes(ctypes.byref(_paged(C=1 << 21)), 256, kvm.FMT_BF16) == 0
    assert "2^31" in L.kv_last_error().decode()


def _seq(s, e, n_bt, bt=0x3000, chunks=0x4000):
    return kvm._KvSeq(bt, n_bt, s, e, chunks)


def _store(p, seqs, fmt=kvm.FMT_BF16):
    L = _lib()
    arr = (kvm._KvSeq * max(1, len(seqs)))(*seqs)
    return L.kv_store_chunks(ctypes.byref(p) if p is not None else None, arr, len(seqs), fmt, None)


def test_store_rejections():
    L = _lib()
    p = _paged()
    assert _store(p, [_seq(16, 300, 40)]) == kvm.KV_EINVAL          # start not chunk-aligned
    assert "multiple of chunk_size" in L.kv_last_error().decode()
    assert _store(p, [_seq(0, 641, 40)]) == kvm.KV_ERANGE           # beyond 40 pages of 16
    assert _store(p, [_seq(0, 100, 40)], fmt=5) == kvm.KV_EINVAL
    assert _store(p, [_seq(0, 100, 40)], fmt=-1) == kvm.KV_EINVAL
    assert _store(p, [_seq(300, 200, 40)]) == kvm.KV_EINVAL
    assert _store(p, [_seq(0, 100, 40, bt=0)]) == kvm.KV_EINVAL
    assert _store(p, [_seq(0, 100, 40, chunks=0)]) == kvm.KV_EINVAL
    assert _store(None, [_seq(0, 100, 40)]) == kvm.KV_EINVAL
    assert _store(_paged(D=3, H=1), [_seq(0, 100, 40)]) == kvm.KV_EINVAL   # 6-byte rows
    assert _store(_paged(C=250), [_seq(0, 100, 40)]) == kvm.KV_EINVAL      # chunk % page
    assert _store(_paged(k=0), [_seq(0, 100, 40)]) == kvm.KV_EINVAL
    # a later bad sequence rejects the whole call before anything is launched
    assert _store(p, [_seq(0, 100, 40), _seq(0, 100, 2)]) == kvm.KV_ERANGE
    assert "seq 1" in L.kv_last_error().decode()


def test_store_layer_rejections_and_empty_work():
    L = _lib()
    p = _paged()
    ok = (kvm._KvSeq * 1)(_seq(0, 100, 40))
    for bad_layer in (-1, 32):
        assert L.kv_store_layer(ctypes.byref(p), ok, 1, 0, bad_layer, 0, None, None) == kvm.KV_EINVAL
    assert L.kv_store_layer(ctypes.byref(p), ok, 1, 0, 3, -1, None, None) == kvm.KV_EINVAL
    bad = (kvm._KvSeq * 1)(_seq(16, 100, 40))
    assert L.kv_store_layer(ctypes.byref(p), bad, 1, 0, 3, 0, None, None) == kvm.KV_EINVAL
    empty = (kvm._KvSeq * 1)(_seq(256, 256, 40))
    assert L.kv_store_layer(ctypes.byref(p), empty, 1, 1, 3, 0, None, None) == kvm.KV_OK


def test_empty_work_launches_nothing():
    # no sequences, or only empty ranges: KV_OK with no HIP call (no GPU here)
    p = _paged()
    assert _store(p, []) == kvm.KV_OK
    assert _store(p, [_seq(512, 512, 40), _seq(0, 0, 0, bt=0, chunks=0)]) == kvm.KV_OK


def test_retrieve_with_no_hits_launches_nothing():
    L = _lib()
    p = _paged()
    seqs = (kvm._KvSeq * 2)(_seq(0, 1000, 63), _seq(256, 700, 44))
    m0 = (ctypes.c_uint8 * 4)(0, 1, 1, 1)
    m1 = (ctypes.c_uint8 * 2)(0, 0)
    masks = (ctypes.c_void_p * 2)(ctypes.addressof(m0), ctypes.addressof(m1))
    out = (ctypes.c_int64 * 2)(-7, -7)
    assert L.kv_retrieve_chunks(ctypes.byref(p), seqs, masks, 2, kvm.FMT_BF16, out, None) == kvm.KV_OK
    assert list(out) == [0, 0]
    for layer in (0, 31):
        out[0] = out[1] = -7
        assert L.kv_retrieve_layer_ex(ctypes.byref(p), seqs, masks, 2, kvm.FMT_FP8, layer, out, 0, None,
                                      None) == kvm.KV_OK
        assert list(out) == [0, 0]
        assert L.kv_retrieve_layer(ctypes.byref(p), seqs, masks, 2, kvm.FMT_FP8, layer, None, None) == kvm.KV_OK
    # every layer in one call, no events: nothing is enqueued either
    out[0] = out[1] = -7
    assert L.kv_retrieve_layers(ctypes.byref(p), seqs, masks, 2, kvm.FMT_BF16, 0, 32, None, out, None, None,
                                None) == kvm.KV_OK
    assert list(out) == [0, 0]


def test_retrieve_rejections():
    L = _lib()
    p = _paged()
    seqs = (kvm._KvSeq * 1)(_seq(0, 1000, 63))
    m = (ctypes.c_uint8 * 4)(1, 1, 0, 1)
    masks = (ctypes.c_void_p * 1)(ctypes.addressof(m))
    out = (ctypes.c_int64 * 1)()
    assert L.kv_retrieve_chunks(ctypes.byref(p), seqs, None, 1, 0, out, None) == kvm.KV_EINVAL
    nullm = (ctypes.c_void_p * 1)(None)
    assert L.kv_retrieve_chunks(ctypes.byref(p), seqs, nullm, 1, 0, out, None) == kvm.KV_EINVAL
    for bad_layer in (-1, 32):
        assert L.kv_retrieve_layer(ctypes.byref(p), seqs, masks, 1, 0, bad_layer, None, None) == kvm.KV_EINVAL
        assert L.kv_retrieve_layer_ex(ctypes.byref(p), seqs, masks, 1, 0, bad_layer, out, 0, None,
                                      None) == kvm.KV_EINVAL
    assert L.kv_retrieve_layer_ex(ctypes.byref(p), seqs, masks, 1, 0, 0, out, -5, None,
                                  None) == kvm.KV_EINVAL
    assert L.kv_retrieve_layer(ctypes.byref(p), seqs, None, 1, 0, 0, None, None) == kvm.KV_EINVAL
    # layer ranges: empty, reversed or outside [0, L), and negative caps
    for lo, hi in ((3, 3), (5, 4), (-1, 2), (30, 33)):
        assert L.kv_retrieve_layers(ctypes.byref(p), seqs, masks, 1, 0, lo, hi, None, out, None, None,
                                    None) == kvm.KV_EINVAL
        assert L.kv_store_layers(ctypes.byref(p), seqs, 1, 0, lo, hi, None, None, None, None,
                                 None) == kvm.KV_EINVAL
    caps = (ctypes.c_int32 * 4)(0, 8, -1, 8)
    assert L.kv_retrieve_layers(ctypes.byref(p), seqs, masks, 1, 0, 4, 8, caps, out, None, None,
                                None) == kvm.KV_EINVAL
    assert "max_workgroups[2]" in L.kv_last_error().decode()
    assert L.kv_store_layers(ctypes.byref(p), seqs, 1, 0, 4, 8, caps, None, None, None, None) == kvm.KV_EINVAL
    # a second stream that is the first one is refused before any HIP call
    same = ctypes.c_void_p(0x1000)
    assert L.kv_retrieve_layers(ctypes.byref(p), seqs, masks, 1, 0, 0, 4, None, out, same, same,
                                None) == kvm.KV_EINVAL
    assert "alt_stream" in L.kv_last_error().decode()
    assert L.kv_store_layers(ctypes.byref(p), seqs, 1, 0, 0, 4, None, same, same, None, None) == kvm.KV_EINVAL
    assert "alt_stream" in L.kv_last_error().decode()
    bad = (kvm._KvSeq * 1)(_seq(100, 1000, 63))
    assert L.kv_retrieve_chunks(ctypes.byref(p), bad, masks, 1, 0, out, None) == kvm.KV_EINVAL


def test_copy_bytes_rejections():
    L = _lib()
    assert L.kv_copy_bytes(0x1000, 0x2000, 17, None) == kvm.KV_EINVAL
    assert L.kv_copy_bytes(0x1008, 0x2000, 32, None) == kvm.KV_EINVAL
    assert L.kv_copy_bytes(None, 0x2000, 32, None) == kvm.KV_EINVAL
    assert L.kv_copy_bytes(0x1000, 0x2000, 0, None) == kvm.KV_OK


def test_copy_blocks_rejections():
    # every case is refused (or is empty) on the host, before any HIP call
    L = _lib()
    assert L.kv_copy_blocks(0x1000, 0x2000, 1 << 20, 1000, 1, None) == kvm.KV_EINVAL       # not a power of two
    assert L.kv_copy_blocks(0x1000, 0x2000, 1 << 20, 2048, 1, None) == kvm.KV_EINVAL       # below the tile
    assert L.kv_copy_blocks(0x1000, 0x2000, 1 << 20, 1 << 31, 1, None) == kvm.KV_EINVAL    # above 2^30
    assert L.kv_copy_blocks(0x1000, 0x2000, 45056, 8192, 1, None) == kvm.KV_EINVAL        # not a multiple
    assert "multiple" in L.kv_last_error().decode()
    assert L.kv_copy_blocks(0x1000, 0x2000, 1 << 20, 32768, 0, None) == kvm.KV_EINVAL      # permute 0
    assert L.kv_copy_blocks(0x1000, 0x2000, 1 << 20, 32768, 3, None) == kvm.KV_EINVAL
    assert L.kv_copy_blocks(0x1008, 0x2000, 1 << 20, 32768, 1, None) == kvm.KV_EINVAL      # misaligned
    assert L.kv_copy_blocks(None, 0x2000, 1 << 20, 32768, 2, None) == kvm.KV_EINVAL
    assert L.kv_copy_blocks(0x1000, 0x2000, 0, 32768, 2, None) == kvm.KV_OK                # empty


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(kvm, "_LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(kvm, "_lib", None)
    with pytest.raises(kvm.KvError, match="no fallback"):
        kvm.load()


def test_binding_refuses_pageable_host_chunks():
    # the GPU cannot address pageable host memory: the binding refuses it
    # before any call (device and pinned host tensors are accepted)
    import torch
    bt = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(kvm.KvError, match="pageable"):
        kvm.Seq(bt, 0, 64, [torch.empty(1 << 16, dtype=torch.uint8)])
    with pytest.raises(kvm.KvError, match="contiguous"):
        t = torch.empty(1 << 16, dtype=torch.uint8, device="meta")
        kvm.Seq(bt, 0, 64, [t[::2]])


def test_binding_refuses_host_block_tables_and_pools():
    # the kernels read block tables, chunk-address arrays and pools from
    # device memory: host tensors are refused before any call
    import torch
    with pytest.raises(kvm.KvError, match="block_table"):
        kvm.Seq(torch.zeros(4, dtype=torch.int32), 0, 0, [])
    with pytest.raises(kvm.KvError, match="chunk addresses"):
        kvm.Seq(torch.zeros(4, dtype=torch.int32), 0, 64, torch.zeros(1, dtype=torch.int64))
    with pytest.raises(kvm.KvError, match="pool"):
        kvm.Paged.from_pool(torch.zeros(1, 2, 4, 16, 1, 8, dtype=torch.bfloat16))
    with pytest.raises(kvm.KvError, match="per-layer"):
        kvm.Paged.from_layers([torch.zeros(4, 16, 1, 8, dtype=torch.bfloat16)],
                              [torch.zeros(4, 16, 1, 8, dtype=torch.bfloat16)])


def _host_paged(L=2, H=2, D=64, P=16, C=256, n=64):
    """A Paged whose address arrays are host tensors: enough for the host-side
    checks (nothing here reaches a kernel)."""
    import torch
    z = torch.zeros(L, dtype=torch.int64)
    return kvm.Paged(z, z.clone(), L, H, D, P, C, n)


def _host_seq(s, e, chunks=None):
    """A Seq built past the device checks of its constructor (host tensors,
    for host-side checks only)."""
    import torch
    seq = kvm.Seq.__new__(kvm.Seq)
    seq.tok_start, seq.tok_end = s, e
    seq.block_table = torch.zeros(64, dtype=torch.int32)
    seq._chunks = chunks
    seq.chunk_addrs = torch.zeros(len(chunks) if chunks else 1, dtype=torch.int64)
    return seq


def test_binding_refuses_short_hit_masks():
    # one flag per chunk is read: a shorter mask would be read past its end;
    # the chunk count comes from the library (kv_num_chunks)
    _lib()
    b = kvm.Batch(_host_paged(), [_host_seq(256, 1000)])     # 3 chunks
    with pytest.raises(kvm.KvError, match="2 flags for 3 chunks"):
        b.set_masks([[1, 1]])
    assert b.set_masks([[1, 1, 0]]) is b
    with pytest.raises(kvm.KvError, match="hit masks"):
        b.set_masks([[1, 1, 0], [1]])


def test_binding_refuses_short_chunk_lists_and_small_chunks():
    # the kernels write each chunk buffer up to kv_chunk_bytes for its token
    # count and cannot see its end: too few chunk tensors, or one too small
    # for the format, is refused with KV_EINVAL before any library call that
    # would launch (here, with no GPU, a launch would fail with KV_EHIP)
    import torch
    _lib()
    paged = _host_paged()
    sizes = [paged.chunk_bytes(paged.chunk_tokens(0, 600, c), kvm.FMT_BF16) for c in range(3)]
    assert [paged.chunk_tokens(0, 600, c) for c in range(3)] == [256, 256, 88]
    ok = [torch.empty(n, dtype=torch.uint8) for n in sizes]
    short_list = kvm.Batch(paged, [_host_seq(0, 600, ok[:2])]).set_masks([[1, 1, 1]])
    with pytest.raises(kvm.KvError, match="2 chunk tensors for 3 chunks") as e:
        kvm.store(paged, short_list)
    assert e.value.code == kvm.KV_EINVAL
    with pytest.raises(kvm.KvError, match="2 chunk tensors for 3 chunks"):
        kvm.retrieve(paged, short_list)
    small = ok[:2] + [torch.empty(sizes[2] - 16, dtype=torch.uint8)]
    b = kvm.Batch(paged, [_host_seq(0, 600, small)]).set_masks([[1, 1, 1]])
    with pytest.raises(kvm.KvError, match="chunk 2") as e:
        kvm.retrieve_layer(paged, b, 0)
    assert e.value.code == kvm.KV_EINVAL
    # sized for fp8 (1 byte per element) but used as bf16 (2 bytes)
    fp8 = [torch.empty(paged.chunk_bytes(paged.chunk_tokens(0, 600, c), kvm.FMT_FP8), dtype=torch.uint8)
           for c in range(3)]
    b = kvm.Batch(paged, [_host_seq(0, 600, fp8)]).set_masks([[1, 1, 1]])
    b.check_chunks(kvm.FMT_FP8)
    with pytest.raises(kvm.KvError, match="format 0 needs"):
        kvm.store_layers(paged, b, 0, 2)
    # enough tensors of the right size pass the check (the call then goes on
    # to the library, which cannot launch without a GPU)
    good = kvm.Batch(paged, [_host_seq(0, 600, ok)]).set_masks([[1, 1, 1]])
    assert good.check_chunks(kvm.FMT_BF16) is good
    assert paged.chunk_tokens(0, 600, 2) == 88
    with pytest.raises(kvm.KvError, match="outside"):
        paged.chunk_tokens(0, 600, 3)


def test_boundary_signatures_match_the_contract():
    # the boundary's own calls keep their argument lists: pool, sequences,
    # (hit masks,) count, format, ..., stream, (event); the format typed
    # kv_fmt.  Parsed from include/kvmove.h.
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)

    def params(name):
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
        assert m, name
        return [re.sub(r"\s+", " ", a.strip()) for a in m.group(1).split(",")]

    assert params("kv_store_chunks") == ["const kv_paged* paged", "const kv_seq* seqs", "int n_seqs", "kv_fmt fmt",
                                         "hipStream_t stream"]
    assert params("kv_retrieve_chunks") == ["const kv_paged* paged", "const kv_seq* seqs",
                                            "const uint8_t* const* hit_mask", "int n_seqs", "kv_fmt fmt",
                                            "int64_t* out_tokens", "hipStream_t stream"]
    assert params("kv_retrieve_layer") == ["const kv_paged* paged", "const kv_seq* seqs",
                                           "const uint8_t* const* hit_mask", "int n_seqs", "kv_fmt fmt",
                                           "int32_t layer", "hipStream_t copy_stream", "hipEvent_t layer_done"]
    assert params("kv_chunk_bytes") == ["const kv_paged* paged", "int64_t n_tokens", "kv_fmt fmt"]
    assert params("kv_last_error") == ["void"]
    # every format argument of every entry point is a kv_fmt
    for m in re.finditer(r"\b(kv_[a-z_]+)\s*\(([^)]*)\)\s*;", text):
        for a in m.group(2).split(","):
            if re.search(r"\bfmt\b", a):
                assert a.split()[0] == "kv_fmt", (m.group(1), a)


def test_cachegen_entry_points_reject_bad_calls():
    L = _lib()
    p = _paged(L=4)
    ok = (kvm._KvSeq * 1)(_seq(0, 100, 40))
    good = (ctypes.c_int32 * 4)(4, 32, 64, 129)
    for bad_bins in ((3, 8, 8, 8), (8, 8, 8, 130), (0, 0, 0, 0)):
        b = (ctypes.c_int32 * 4)(*bad_bins)
        assert L.kv_store_chunks_cachegen(ctypes.byref(p), ok, 1, b, good, None) == kvm.KV_EINVAL
        assert "bin counts" in L.kv_last_error().decode()
        assert L.kv_store_chunks_cachegen(ctypes.byref(p), ok, 1, good, b, None) == kvm.KV_EINVAL
    assert L.kv_store_chunks_cachegen(ctypes.byref(p), ok, 1, None, good, None) == kvm.KV_EINVAL
    many = _paged(L=129)
    bins129 = (ctypes.c_int32 * 129)(*([16] * 129))
    assert L.kv_store_chunks_cachegen(ctypes.byref(many), ok, 1, bins129, bins129, None) == kvm.KV_EINVAL
    wide = _paged(L=4, H=40, D=128)                         # 5120-element rows
    assert L.kv_store_chunks_cachegen(ctypes.byref(wide), ok, 1, good, good, None) == kvm.KV_EINVAL
    bad_seq = (kvm._KvSeq * 1)(_seq(16, 100, 40))
    assert L.kv_store_chunks_cachegen(ctypes.byref(p), bad_seq, 1, good, good, None) == kvm.KV_EINVAL
    # the generic entry points refuse the format: its bins would be missing
    assert _store(p, [_seq(0, 100, 40)], fmt=kvm.FMT_CACHEGEN) == kvm.KV_EINVAL
    assert "cachegen" in L.kv_last_error().decode()
    # sizes: one byte per element, one float32 per (layer, K/V, token)
    assert L.kv_chunk_bytes(ctypes.byref(p), 256, kvm.FMT_CACHEGEN) == 4 * 2 * 256 * 1024 + 4 * 2 * 256 * 4
    # zero hits: nothing launched, out_tokens = 0 (no GPU here)
    seqs = (kvm._KvSeq * 1)(_seq(0, 1000, 63))
    m0 = (ctypes.c_uint8 * 4)(0, 1, 1, 1)
    masks = (ctypes.c_void_p * 1)(ctypes.addressof(m0))
    out = (ctypes.c_int64 * 1)(-7)
    assert L.kv_retrieve_chunks_cachegen(ctypes.byref(p), seqs, masks, 1, good, good, out, None, 0, None) == kvm.KV_OK
    assert out[0] == 0
    assert L.kv_retrieve_chunks_cachegen(ctypes.byref(p), seqs, None, 1, good, good, out, None, 0,
                                         None) == kvm.KV_EINVAL
    # a workspace that is too small or misaligned is refused
    m1 = (ctypes.c_uint8 * 4)(1, 1, 1, 1)
    masks1 = (ctypes.c_void_p * 1)(ctypes.addressof(m1))
    need = L.kv_retrieve_workspace_bytes(ctypes.byref(p))
    assert L.kv_retrieve_chunks_cachegen(ctypes.byref(p), seqs, masks1, 1, good, good, out, 0x10000, need - 1,
                                         None) == kvm.KV_EINVAL
    assert L.kv_retrieve_chunks_cachegen(ctypes.byref(p), seqs, masks1, 1, good, good, out, 0x10040, need,
                                         None) == kvm.KV_EINVAL


def test_ordered_retrieve_workspace_size_and_rejections():
    L = _lib()
    p = _paged(n=8192)
    assert L.kv_retrieve_workspace_bytes(ctypes.byref(p)) == 2 * 8192 * 4
    assert L.kv_retrieve_workspace_bytes(ctypes.byref(_paged(n=1000))) == 2 * 4096    # 4000 B rounded to 256
    assert L.kv_retrieve_workspace_bytes(None) == 0
    seqs = (kvm._KvSeq * 1)(_seq(0, 1000, 63))
    m = (ctypes.c_uint8 * 4)(1, 1, 1, 1)
    masks = (ctypes.c_void_p * 1)(ctypes.addressof(m))
    out = (ctypes.c_int64 * 1)()
    need = 2 * 8192 * 4
    args = (ctypes.byref(p), seqs, masks, 1, kvm.FMT_BF16, out)
    assert L.kv_retrieve_chunks_ws(*args, None, need, None) == kvm.KV_EINVAL
    assert L.kv_retrieve_chunks_ws(*args, 0x10000, need - 1, None) == kvm.KV_EINVAL
    assert "workspace" in L.kv_last_error().decode()
    assert L.kv_retrieve_chunks_ws(*args, 0x10080, need, None) == kvm.KV_EINVAL          # not 256-aligned
    # zero hits: KV_OK, nothing launched (no GPU here)
    m0 = (ctypes.c_uint8 * 4)(0, 1, 1, 1)
    masks0 = (ctypes.c_void_p * 1)(ctypes.addressof(m0))
    assert L.kv_retrieve_chunks_ws(ctypes.byref(p), seqs, masks0, 1, kvm.FMT_BF16, out, 0x10000, need,
                                   None) == kvm.KV_OK
    assert out[0] == 0


def test_store_workspace_size_and_rejections():
    # 32 bytes per page unit of the bf16 parts, rounded up to 256; refusals
    # before any HIP call
    L = _lib()
    p = _paged()
    seqs = (kvm._KvSeq * 2)(_seq(0, 1000, 63), _seq(256, 530, 34))
    units = (63 + 18) * 32 * 2                       # ceil(1000/16) + ceil(274/16) pages, 32 layers, K and V
    assert L.kv_store_workspace_bytes(ctypes.byref(p), seqs, 2, kvm.FMT_BF16) == units * 32
    assert L.kv_store_workspace_bytes(ctypes.byref(p), seqs, 2, kvm.FMT_K16_V8) == units * 16
    assert L.kv_store_workspace_bytes(ctypes.byref(p), seqs, 2, kvm.FMT_FP8) == 0
    assert L.kv_last_error().decode() == ""
    one = (kvm._KvSeq * 1)(_seq(0, 17, 2))
    assert L.kv_store_workspace_bytes(ctypes.byref(p), one, 1, kvm.FMT_BF16) == 2 * 64 * 32
    assert L.kv_store_workspace_bytes(ctypes.byref(_paged(L=1)), one, 1, kvm.FMT_BF16) == 256   # 128 B rounded up
    assert L.kv_store_workspace_bytes(ctypes.byref(p), seqs, 2, 9) == 0
    assert L.kv_last_error().decode() != ""
    assert L.kv_store_workspace_bytes(None, seqs, 2, kvm.FMT_BF16) == 0
    need = units * 32
    args = (ctypes.byref(p), seqs, 2, kvm.FMT_BF16)
    assert L.kv_store_chunks_ws(*args, None, need, None) == kvm.KV_EINVAL
    assert "workspace" in L.kv_last_error().decode()
    assert L.kv_store_chunks_ws(*args, 0x10000, need - 1, None) == kvm.KV_EINVAL
    assert L.kv_store_chunks_ws(*args, 0x10080, need, None) == kvm.KV_EINVAL          # not 256-aligned
    bad = (kvm._KvSeq * 1)(_seq(100, 1000, 63))
    assert L.kv_store_chunks_ws(ctypes.byref(p), bad, 1, kvm.FMT_BF16, 0x10000, need, None) == kvm.KV_EINVAL
    # nothing to move: no workspace needed, nothing launched (no GPU here)
    empty = (kvm._KvSeq * 1)(_seq(256, 256, 63))
    assert L.kv_store_workspace_bytes(ctypes.byref(p), empty, 1, kvm.FMT_BF16) == 0
    assert L.kv_store_chunks_ws(ctypes.byref(p), empty, 1, kvm.FMT_BF16, None, 0, None) == kvm.KV_OK


def test_ordered_retrieve_refuses_more_pages_than_the_pool():
    # 1100 tokens = 69 pages of 16 on a 64-page pool: the page ids cannot be
    # distinct and the sorted list would overrun the workspace, so the call
    # is refused before any launch (no GPU here)
    L = _lib()
    p = _paged(n=64)
    need = L.kv_retrieve_workspace_bytes(ctypes.byref(p))
    seqs = (kvm._KvSeq * 1)(_seq(0, 1100, 69))
    m = (ctypes.c_uint8 * 5)(1, 1, 1, 1, 1)
    masks = (ctypes.c_void_p * 1)(ctypes.addressof(m))
    out = (ctypes.c_int64 * 1)()
    assert L.kv_retrieve_chunks_ws(ctypes.byref(p), seqs, masks, 1, kvm.FMT_BF16, out, 0x10000, need,
                                   None) == kvm.KV_EINVAL
    assert "pages" in L.kv_last_error().decode() and "repeat" in L.kv_last_error().decode()
    kb = (ctypes.c_int32 * 32)(*([16] * 32))
    assert L.kv_retrieve_chunks_cachegen(ctypes.byref(p), seqs, masks, 1, kb, kb, out, 0x10000, need,
                                         None) == kvm.KV_EINVAL
    assert "repeat" in L.kv_last_error().decode()


def test_ordered_retrieve_refuses_a_sequence_too_large_for_one_launch():
    # a launch takes fewer than 2^32 threads, 2^26 - 1 one-wave workgroups:
    # a sequence of 2^25 pages (K and V: 2^26 units; here 256-byte pages, H=1,
    # D=8, on a pool of 2^27 pages) is refused on the host before any launch
    # (the addresses are fake; nothing may reach a device).  This also keeps
    # every page index within the 26 bits the sorted list packs it in.
    import numpy as np
    L = _lib()
    p = _paged(L=1, H=1, D=8, n=1 << 27)
    need = L.kv_retrieve_workspace_bytes(ctypes.byref(p))
    assert need == 2 * (1 << 27) * 4
    out = (ctypes.c_int64 * 1)()
    pages = 1 << 25
    tokens = pages * 16
    seqs = (kvm._KvSeq * 1)(_seq(0, tokens, pages))
    m = np.ones(-(-tokens // 256), np.uint8)
    masks = (ctypes.c_void_p * 1)(m.ctypes.data)
    for call in (lambda: L.kv_retrieve_chunks_ws(ctypes.byref(p), seqs, masks, 1, kvm.FMT_BF16, out, 0x10000, need,
                                                 None),
                 lambda: L.kv_retrieve_chunks(ctypes.byref(p), seqs, masks, 1, kvm.FMT_BF16, out, None),
                 lambda: L.kv_store_chunks(ctypes.byref(p), seqs, 1, kvm.FMT_BF16, None)):
        assert call() == kvm.KV_EINVAL
        assert "exceed one launch" in L.kv_last_error().decode()


def test_c_example_builds_against_the_header(tmp_path):
    # a plain C program (tests/abi_c_example.c) compiles against
    # include/kvmove.h and links libkvmove.so; a GPU test runs it
    _lib()
    from paged_kv_movement_amd import build
    out = build.build_c_example(str(tmp_path / "abi_c_example"))
    assert os.path.exists(out) and os.access(out, os.X_OK)


def test_noalloc_retrieve_refuses_pools_beyond_its_scratch():
    # the no-allocation retrieve keeps its page list in a fixed 8 MiB scratch
    # array per GPU: pools of more than 2^20 pages are refused before any HIP
    # call (no GPU here), and so are the usual malformed calls
    L = _lib()
    seqs = (kvm._KvSeq * 1)(_seq(0, 1000, 63))
    m = (ctypes.c_uint8 * 4)(1, 1, 1, 1)
    masks = (ctypes.c_void_p * 1)(ctypes.addressof(m))
    out = (ctypes.c_int64 * 1)()
    big = _paged(n=(1 << 20) + 1)
    assert L.kv_retrieve_chunks_noalloc(ctypes.byref(big), seqs, masks, 1, kvm.FMT_BF16, out, None) == kvm.KV_EINVAL
    assert "at most 1048576 pages" in L.kv_last_error().decode()
    p = _paged(n=8192)
    assert L.kv_retrieve_chunks_noalloc(ctypes.byref(p), seqs, masks, 1, kvm.FMT_CACHEGEN, out, None) == kvm.KV_EINVAL
    assert L.kv_retrieve_chunks_noalloc(ctypes.byref(p), seqs, None, 1, kvm.FMT_BF16, out, None) == kvm.KV_EINVAL
    bad = (kvm._KvSeq * 1)(_seq(100, 1000, 63))
    assert L.kv_retrieve_chunks_noalloc(ctypes.byref(p), bad, masks, 1, kvm.FMT_BF16, out, None) == kvm.KV_EINVAL


def test_noalloc_retrieve_checks_every_sequence_before_any_hip_call():
    # beyond 64 sequences too (the entry point takes them 64 at a time): a
    # NULL mask entry of sequence 80, or more pages moved in all than the pool
    # holds, is refused with KV_EINVAL, not the KV_EHIP a HIP call on this
    # GPU-less host would give
    L = _lib()
    n = 100
    seqs = (kvm._KvSeq * n)(*[_seq(0, 300, 19) for _ in range(n)])
    m = (ctypes.c_uint8 * 2)(1, 1)
    masks = (ctypes.c_void_p * n)(*([ctypes.addressof(m)] * n))
    out = (ctypes.c_int64 * n)()
    p = _paged(n=8192)
    masks[80] = None
    assert L.kv_retrieve_chunks_noalloc(ctypes.byref(p), seqs, masks, n, kvm.FMT_BF16, out, None) == kvm.KV_EINVAL
    assert "seq 80" in L.kv_last_error().decode()
    masks[80] = ctypes.addressof(m)
    small = _paged(n=100 * 19 - 1)          # 100 sequences x 19 pages moved
    assert L.kv_retrieve_chunks_noalloc(ctypes.byref(small), seqs, masks, n, kvm.FMT_BF16, out, None) == kvm.KV_EINVAL
    assert "page ids repeat" in L.kv_last_error().decode()
