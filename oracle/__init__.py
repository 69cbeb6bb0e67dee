"""CPU oracle for paged <-> chunk KV-cache movement (ctypes wrapper over kv_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product path never
does, and this package imports nothing from the product package.

The C side is plain nested loops over the byte layouts the method defines (see
kv_oracle.h for the cited passages).  This wrapper only marshals numpy arrays.

Pool arrays handed to the oracle are numpy ``uint16`` (raw bf16 bits) shaped
``[num_pages, page_size, num_kv_heads * head_dim]``, one per (layer, K/V).
Chunks are numpy ``uint8`` buffers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kv_oracle.c")
_LIB = os.path.join(_HERE, "libkvoracle.so")

FMT_BF16 = 0          # K and V bf16
FMT_FP8 = 1           # K and V e4m3, one float32 scale per (layer, K/V)
FMT_FP8_E5M2 = 2      # K and V e5m2, one float32 scale per (layer, K/V)
FMT_K16_V8 = 3        # K bf16, V e4m3, one float32 scale per layer
FMT_CACHEGEN = 4      # CacheGen symbols u8 [L][2][n][E], then float32 max1 [L][2][n]

_lib = None


def build() -> str:
    """Compile kv_oracle.c with gcc into oracle/libkvoracle.so (IEEE float, no fast-math)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    """Load the oracle library, building it first only if it is not there.
    KVO_ORACLE_LIB names another build of kv_oracle.c to load instead (the
    mutation tests point it at deliberately broken copies)."""
    global _lib
    if _lib is None:
        path = os.environ.get("KVO_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(path):
                build()
        _lib = _bind(ctypes.CDLL(path))
    return _lib


class _Pool(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("k", ctypes.POINTER(ctypes.c_void_p)),
        ("v", ctypes.POINTER(ctypes.c_void_p)),
    ]


def _bind(L):
    i32, i64, u8, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint8, ctypes.c_float, ctypes.c_void_p
    P = ctypes.POINTER(_Pool)
    sig = {
        "kvo_num_chunks": (i64, [i64, i64, i32]),
        "kvo_chunk_tokens": (i64, [i64, i64, i32, i64]),
        "kvo_chunk_bytes": (i64, [P, i64, ctypes.c_int]),
        "kvo_slot": (i64, [vp, i32, i64]),
        "kvo_hit_chunks": (i64, [vp, i64]),
        "kvo_store": (ctypes.c_int, [P, vp, i64, i64, i64, vp, ctypes.c_int, i32]),
        "kvo_retrieve": (i64, [P, vp, i64, i64, i64, vp, vp, ctypes.c_int, i32]),
        "kvo_store_cachegen": (ctypes.c_int, [P, vp, i64, i64, i64, vp, vp, vp]),
        "kvo_retrieve_cachegen": (i64, [P, vp, i64, i64, i64, vp, vp, vp, vp]),
        "kvo_e4m3_encode": (u8, [f32]),
        "kvo_e4m3_decode": (f32, [u8]),
        "kvo_bf16_from_float": (ctypes.c_uint16, [f32]),
        "kvo_float_from_bf16": (f32, [ctypes.c_uint16]),
        "kvo_fp8_scale": (f32, [f32]),
        "kvo_e5m2_scale": (f32, [f32]),
        "kvo_e5m2_encode": (u8, [f32]),
        "kvo_e5m2_decode": (f32, [u8]),
        "kvo_e5m2_encode_n": (None, [vp, vp, i64]),
        "kvo_e5m2_encode_bits_range": (None, [ctypes.c_uint64, i64, vp]),
        "kvo_e4m3_encode_n": (None, [vp, vp, i64]),
        "kvo_e4m3_encode_bits_range": (None, [ctypes.c_uint64, i64, vp]),
        "kvo_bf16_from_float_n": (None, [vp, vp, i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Pool:
    """The engine's paged KV pool as the oracle sees it (host memory).

    ``k[l]`` / ``v[l]``: C-contiguous uint16 arrays [num_pages, page_size, H*D].
    """

    def __init__(self, num_layers, num_kv_heads, head_dim, page_size, chunk_size,
                 num_pages, k, v):
        assert len(k) == num_layers and len(v) == num_layers
        width = num_kv_heads * head_dim
        for a in list(k) + list(v):
            assert a.dtype == np.uint16 and a.flags.c_contiguous
            assert a.size == num_pages * page_size * width
        self.k, self.v = list(k), list(v)
        self._kp = (ctypes.c_void_p * num_layers)(*[_ptr(a) for a in self.k])
        self._vp = (ctypes.c_void_p * num_layers)(*[_ptr(a) for a in self.v])
        self.c = _Pool(num_layers, num_kv_heads, head_dim, page_size, chunk_size, num_pages,
                       ctypes.cast(self._kp, ctypes.POINTER(ctypes.c_void_p)),
                       ctypes.cast(self._vp, ctypes.POINTER(ctypes.c_void_p)))
        self.num_layers, self.num_kv_heads, self.head_dim = num_layers, num_kv_heads, head_dim
        self.page_size, self.chunk_size, self.num_pages = page_size, chunk_size, num_pages

    @classmethod
    def from_array(cls, pool: np.ndarray, num_kv_heads, head_dim, chunk_size):
        """Wrap one array shaped [L, 2, num_pages, page_size, H*D] (views, no copy)."""
        L, two, num_pages, page_size, width = pool.shape
        assert two == 2 and width == num_kv_heads * head_dim
        return cls(L, num_kv_heads, head_dim, page_size, chunk_size, num_pages,
                   [pool[l, 0] for l in range(L)], [pool[l, 1] for l in range(L)])


def num_chunks(s: int, e: int, chunk_size: int) -> int:
    return int(lib().kvo_num_chunks(s, e, chunk_size))


def chunk_tokens(s: int, e: int, chunk_size: int, c: int) -> int:
    return int(lib().kvo_chunk_tokens(s, e, chunk_size, c))


def chunk_bytes(pool: Pool, n_tokens: int, fmt: int) -> int:
    return int(lib().kvo_chunk_bytes(ctypes.byref(pool.c), n_tokens, fmt))


def slot(block_table: np.ndarray, page_size: int, t: int) -> int:
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    return int(lib().kvo_slot(_ptr(bt), page_size, t))


def hit_chunks(mask) -> int:
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    return int(lib().kvo_hit_chunks(_ptr(m), m.size))


def alloc_chunks(pool: Pool, s: int, e: int, fmt: int, fill: int = 0):
    """Fresh chunk buffers for [s, e): one uint8 array per chunk, of exact size."""
    out = []
    for c in range(num_chunks(s, e, pool.chunk_size)):
        n_c = chunk_tokens(s, e, pool.chunk_size, c)
        out.append(np.full(chunk_bytes(pool, n_c, fmt), fill, dtype=np.uint8))
    return out


def _chunk_ptrs(chunks):
    for a in chunks:
        assert a.dtype == np.uint8 and a.flags.c_contiguous
    return (ctypes.c_void_p * max(1, len(chunks)))(*[_ptr(a) for a in chunks])


def store(pool: Pool, block_table, s: int, e: int, chunks, fmt: int = FMT_BF16,
          layer: int = -1) -> int:
    """Gather [s, e) into ``chunks`` (list from alloc_chunks); one layer only
    when layer >= 0.  Returns 0 or -1."""
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    ptrs = _chunk_ptrs(chunks)
    return int(lib().kvo_store(ctypes.byref(pool.c), _ptr(bt), bt.size, s, e, ptrs, fmt, layer))


def retrieve(pool: Pool, block_table, s: int, e: int, mask, chunks, fmt: int = FMT_BF16,
             layer: int = -1) -> int:
    """Scatter the leading hit chunks back into ``pool`` (in place).  Returns tokens or -1."""
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    m = np.ascontiguousarray(mask if mask is not None else [], dtype=np.uint8)
    ptrs = _chunk_ptrs(chunks)
    return int(lib().kvo_retrieve(ctypes.byref(pool.c), _ptr(bt), bt.size, s, e,
                                  _ptr(m) if m.size else None, ptrs, fmt, layer))


def _bins(b, n):
    a = np.ascontiguousarray(b, dtype=np.int32)
    assert a.size == n
    return a


def store_cachegen(pool: Pool, block_table, s: int, e: int, chunks, key_bins, value_bins) -> int:
    """CacheGen quantiser: gather + quantise [s, e) into ``chunks`` (from
    alloc_chunks(..., FMT_CACHEGEN)).  Returns 0 or -1."""
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    kb, vb = _bins(key_bins, pool.num_layers), _bins(value_bins, pool.num_layers)
    return int(lib().kvo_store_cachegen(ctypes.byref(pool.c), _ptr(bt), bt.size, s, e, _chunk_ptrs(chunks),
                                        _ptr(kb), _ptr(vb)))


def retrieve_cachegen(pool: Pool, block_table, s: int, e: int, mask, chunks, key_bins, value_bins) -> int:
    """Dequantise + scatter the leading hit chunks.  Returns tokens or -1."""
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    m = np.ascontiguousarray(mask if mask is not None else [], dtype=np.uint8)
    kb, vb = _bins(key_bins, pool.num_layers), _bins(value_bins, pool.num_layers)
    return int(lib().kvo_retrieve_cachegen(ctypes.byref(pool.c), _ptr(bt), bt.size, s, e,
                                           _ptr(m) if m.size else None, _chunk_ptrs(chunks), _ptr(kb), _ptr(vb)))


def e4m3_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().kvo_e4m3_encode_n(_ptr(y), _ptr(out), y.size)
    return out


def e4m3_encode_bits_range(first_bits: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    lib().kvo_e4m3_encode_bits_range(first_bits, n, _ptr(out))
    return out


def e4m3_decode(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    L = lib()
    return np.array([L.kvo_e4m3_decode(int(x)) for x in b.ravel()], dtype=np.float32).reshape(b.shape)


def e5m2_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().kvo_e5m2_encode_n(_ptr(y), _ptr(out), y.size)
    return out


def e5m2_encode_bits_range(first_bits: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    lib().kvo_e5m2_encode_bits_range(first_bits, n, _ptr(out))
    return out


def e5m2_decode(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    L = lib()
    return np.array([L.kvo_e5m2_decode(int(x)) for x in b.ravel()], dtype=np.float32).reshape(b.shape)


def e5m2_scale(amax: float) -> float:
    return float(lib().kvo_e5m2_scale(amax))


def bf16_from_float(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint16)
    lib().kvo_bf16_from_float_n(_ptr(y), _ptr(out), y.size)
    return out


def fp8_scale(amax: float) -> float:
    return float(lib().kvo_fp8_scale(amax))
