"""MI355X-native paged <-> chunk KV-cache movement: Python binding of libkvmove.so.

Argument marshalling only.  Every byte is moved by the HIP kernels behind the
C ABI in ``include/kvmove.h``; this module turns torch device tensors,
streams and events into the raw addresses and handles that ABI takes.  There
is no fallback: if ``libkvmove.so`` is missing the first call raises.

Typical use::

    import paged_kv_movement_amd as kvm
    pool = torch.empty(L, 2, num_pages, 16, H, D, dtype=torch.bfloat16, device="cuda")
    paged = kvm.Paged.from_pool(pool, chunk_size=256)
    chunks = [torch.empty(paged.chunk_bytes(n), dtype=torch.uint8, device="cuda") for n in ...]
    batch = kvm.Batch(paged, [kvm.Seq(block_table, 0, 10000, chunks)])
    kvm.store(paged, batch)                            # gather pages -> chunks
    n = kvm.retrieve(paged, batch, masks=[hit_mask])   # scatter hit chunks -> pages

Chunk tensors made with ``pin_memory=True`` instead of on the device turn the
same calls into the offload to host memory and the onload from it.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["FMT_BF16", "FMT_FP8", "FMT_FP8_E5M2", "FMT_K16_V8", "FMT_CACHEGEN", "KvError", "Paged", "Seq", "Batch",
           "store", "store_layer", "store_layers", "store_cachegen", "retrieve_cachegen",
           "retrieve", "retrieve_noalloc", "retrieve_layer", "retrieve_layer_ex", "retrieve_layers", "take_faults",
           "copy_bytes",
           "library_path", "load"]

FMT_BF16 = 0          # K and V bf16, copied bit for bit
FMT_FP8 = 1           # K and V e4m3 + one float32 scale per (layer, K/V)
FMT_FP8_E5M2 = 2      # K and V e5m2 + one float32 scale per (layer, K/V)
FMT_K16_V8 = 3        # K bf16, V e4m3 + one float32 scale per layer
FMT_CACHEGEN = 4      # CacheGen symbols + one float32 max1 per (layer, K/V, token); store_cachegen / retrieve_cachegen

KV_OK, KV_EINVAL, KV_ERANGE, KV_EHIP = 0, -1, -2, -3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvmove.so")
_lib = None


class KvError(RuntimeError):
    """A non-OK status from libkvmove (the message is kv_last_error())."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"kvmove error {code}: {msg}")
        self.code = code


class _KvPaged(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
    ]


class _KvSeq(ctypes.Structure):
    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("n_bt", ctypes.c_int64),
        ("tok_start", ctypes.c_int64),
        ("tok_end", ctypes.c_int64),
        ("chunks", ctypes.c_void_p),
    ]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libkvmove.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise KvError(KV_EHIP, f"{_LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_movement_amd.build` (there is no fallback)")
    L = ctypes.CDLL(_LIB_PATH)
    P, S = ctypes.POINTER(_KvPaged), ctypes.POINTER(_KvSeq)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "kv_chunk_bytes": (ctypes.c_size_t, [P, i64, ctypes.c_int]),
        "kv_num_chunks": (i64, [P, i64, i64]),
        "kv_chunk_tokens": (i64, [P, i64, i64, i64]),
        "kv_store_chunks": (ctypes.c_int, [P, S, ctypes.c_int, ctypes.c_int, vp]),
        "kv_store_layer": (ctypes.c_int, [P, S, ctypes.c_int, ctypes.c_int, i32, i32, vp, vp]),
        "kv_store_layers": (ctypes.c_int, [P, S, ctypes.c_int, ctypes.c_int, i32, i32, vp, vp, vp, vp, vp]),
        "kv_retrieve_chunks": (ctypes.c_int, [P, S, vp, ctypes.c_int, ctypes.c_int, vp, vp]),
        "kv_retrieve_layer": (ctypes.c_int, [P, S, vp, ctypes.c_int, ctypes.c_int, i32, vp, vp]),
        "kv_retrieve_layer_ex": (ctypes.c_int, [P, S, vp, ctypes.c_int, ctypes.c_int, i32, vp, i32, vp, vp]),
        "kv_retrieve_layers": (ctypes.c_int, [P, S, vp, ctypes.c_int, ctypes.c_int, i32, i32, vp, vp, vp, vp,
                                              vp]),
        "kv_store_chunks_cachegen": (ctypes.c_int, [P, S, ctypes.c_int, vp, vp, vp]),
        "kv_retrieve_workspace_bytes": (ctypes.c_size_t, [P]),
        "kv_store_workspace_bytes": (ctypes.c_size_t, [P, S, ctypes.c_int, ctypes.c_int]),
        "kv_store_chunks_ws": (ctypes.c_int, [P, S, ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t, vp]),
        "kv_retrieve_chunks_ws": (ctypes.c_int, [P, S, vp, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_size_t, vp]),
        "kv_retrieve_chunks_noalloc": (ctypes.c_int, [P, S, vp, ctypes.c_int, ctypes.c_int, vp, vp]),
        "kv_retrieve_chunks_cachegen": (ctypes.c_int, [P, S, vp, ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "kv_last_error": (ctypes.c_char_p, []),
        "kv_take_faults": (ctypes.c_int, []),
        "kv_copy_bytes": (ctypes.c_int, [vp, vp, ctypes.c_size_t, vp]),
        "kv_copy_blocks": (ctypes.c_int, [vp, vp, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(rc: int):
    if rc != KV_OK:
        raise KvError(rc, load().kv_last_error().decode())


def _need(cond, msg: str):
    """Argument check that stays on under ``python -O``."""
    if not cond:
        raise KvError(KV_EINVAL, msg)


def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    h = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return h or None


def _used_on(stream, tensors, seen=None) -> None:
    """Tell torch's caching allocator that kernels on ``stream`` read these
    tensors (``record_stream``): the binding makes some device tensors itself
    (address arrays) on the current stream, and a caller may pass a workspace
    made inline; without this, freeing them while the side stream still runs
    could hand their memory to new work too early.  With ``seen`` (a set kept
    by the owner of the tensors, which keeps them alive) each (tensor, stream)
    is recorded once.  Nothing is done for stream=None (the current stream)
    or a raw stream handle (the caller then keeps the tensors alive)."""
    if stream is None or not hasattr(stream, "cuda_stream"):
        return
    for t in tensors:
        if t is None or not getattr(t, "is_cuda", False):
            continue
        if seen is None:
            t.record_stream(stream)
            continue
        key = (id(t), stream.cuda_stream)
        if key not in seen:
            t.record_stream(stream)
            seen.add(key)


class Paged:
    """The engine's paged pool: per-layer K and V base addresses on the device.

    ``k_addrs`` / ``v_addrs`` are device int64 tensors [num_layers] holding the
    address of each layer's bf16 [num_pages][page_size][H][D] K / V pool.
    """

    def __init__(self, k_addrs, v_addrs, num_layers, num_kv_heads, head_dim, page_size,
                 chunk_size, num_pages, keepalive=()):
        self.k_addrs, self.v_addrs = k_addrs, v_addrs
        self._keep = tuple(keepalive)
        self.num_layers, self.num_kv_heads, self.head_dim = num_layers, num_kv_heads, head_dim
        self.page_size, self.chunk_size, self.num_pages = page_size, chunk_size, num_pages
        self.c = _KvPaged(num_layers, num_kv_heads, head_dim, page_size, chunk_size, num_pages,
                          k_addrs.data_ptr(), v_addrs.data_ptr())

    @classmethod
    def from_pool(cls, pool, chunk_size: int = 256) -> "Paged":
        """From one bf16 tensor [L, 2, num_pages, page_size, H, D] (K at [:, 0], V at [:, 1])."""
        import torch
        _need(pool.dtype == torch.bfloat16 and pool.is_contiguous() and pool.dim() == 6 and pool.is_cuda,
              "pool must be a contiguous bf16 device tensor [L, 2, num_pages, page_size, H, D]")
        L, two, n, P, H, D = pool.shape
        _need(two == 2, "pool's second dimension must be 2 (K, V)")
        slab = n * P * H * D * pool.element_size()
        base = pool.data_ptr()
        k = torch.tensor([base + (2 * l) * slab for l in range(L)], dtype=torch.int64)
        v = torch.tensor([base + (2 * l + 1) * slab for l in range(L)], dtype=torch.int64)
        return cls(k.to(pool.device), v.to(pool.device), L, H, D, P, chunk_size, n, keepalive=(pool,))

    @classmethod
    def from_layers(cls, k_layers, v_layers, chunk_size: int = 256) -> "Paged":
        """From per-layer bf16 tensors, each [num_pages, page_size, H, D]."""
        import torch
        n, P, H, D = k_layers[0].shape
        _need(len(k_layers) == len(v_layers) > 0, "need one K and one V tensor per layer")
        for t in list(k_layers) + list(v_layers):
            _need(t.dtype == torch.bfloat16 and t.is_contiguous() and t.is_cuda and tuple(t.shape) == (n, P, H, D),
                  "per-layer pools must be contiguous bf16 device tensors of one shape [num_pages, page_size, H, D]")
        dev = k_layers[0].device
        k = torch.tensor([t.data_ptr() for t in k_layers], dtype=torch.int64).to(dev)
        v = torch.tensor([t.data_ptr() for t in v_layers], dtype=torch.int64).to(dev)
        return cls(k, v, len(k_layers), H, D, P, chunk_size, n, keepalive=(*k_layers, *v_layers))

    def chunk_bytes(self, n_tokens: int, fmt: int = FMT_BF16) -> int:
        n = load().kv_chunk_bytes(ctypes.byref(self.c), n_tokens, fmt)
        if n == 0 and n_tokens > 0:
            _check(KV_EINVAL)
        return int(n)

    def retrieve_workspace_bytes(self) -> int:
        """Device bytes retrieve(..., workspace=...) needs for this pool."""
        n = load().kv_retrieve_workspace_bytes(ctypes.byref(self.c))
        if n == 0:
            _check(KV_EINVAL)
        return int(n)

    def new_workspace(self):
        """A device tensor of retrieve_workspace_bytes() bytes (torch aligns it to 256)."""
        import torch
        return torch.empty(self.retrieve_workspace_bytes(), dtype=torch.uint8, device="cuda")

    def num_chunks(self, tok_start: int, tok_end: int) -> int:
        n = load().kv_num_chunks(ctypes.byref(self.c), tok_start, tok_end)
        if n < 0:
            _check(KV_EINVAL)
        return int(n)

    def chunk_tokens(self, tok_start: int, tok_end: int, c: int) -> int:
        """Tokens of chunk c of [tok_start, tok_end) (kv_chunk_tokens)."""
        n = load().kv_chunk_tokens(ctypes.byref(self.c), tok_start, tok_end, c)
        if n < 0:
            _check(KV_EINVAL)
        return int(n)


class Seq:
    """One sequence's job: a device int32 block table, a token range and its
    chunk buffers (device int64 tensor of addresses, or uint8 tensors).

    A chunk tensor lives either in device memory or in pinned host memory
    (``pin_memory=True``): the kernels address pinned host memory directly,
    so a store into host chunks is the offload and a retrieve from them the
    onload, both over PCIe with no staging copy.  Pageable host tensors are
    refused, since the GPU cannot reach them."""

    def __init__(self, block_table, tok_start: int, tok_end: int, chunks):
        import torch
        self.block_table = block_table
        self.tok_start, self.tok_end = int(tok_start), int(tok_end)
        if isinstance(chunks, torch.Tensor) and chunks.dtype == torch.int64:
            _need(chunks.is_cuda and chunks.is_contiguous() and chunks.dim() == 1,
                  "chunk addresses must be a contiguous 1-D int64 device tensor")
            self.chunk_addrs, self._chunks = chunks, None
        else:
            self._chunks = list(chunks)
            for i, c in enumerate(self._chunks):
                if not c.is_contiguous():
                    raise KvError(KV_EINVAL, f"chunk {i} is not contiguous")
                if not (c.is_cuda or c.is_pinned()):
                    raise KvError(KV_EINVAL, f"chunk {i} is pageable host memory; "
                                             "use a device tensor or pin_memory=True")
            addrs = torch.tensor([c.data_ptr() for c in self._chunks], dtype=torch.int64)
            dev = block_table.device if isinstance(block_table, torch.Tensor) else "cuda"
            self.chunk_addrs = addrs.to(dev)
        # the kernels read the block table from device memory
        _need(isinstance(block_table, torch.Tensor) and block_table.dtype == torch.int32
              and block_table.is_contiguous() and block_table.is_cuda,
              "block_table must be a contiguous int32 device tensor")

    def c(self) -> _KvSeq:
        return _KvSeq(self.block_table.data_ptr(), self.block_table.numel(), self.tok_start,
                      self.tok_end, self.chunk_addrs.data_ptr() if self.chunk_addrs.numel() else 0)


class Batch:
    """Prebuilt C descriptors for a list of Seq (reusable across calls)."""

    def __init__(self, paged: Paged, seqs):
        self.seqs = list(seqs)
        self.paged = paged
        n = len(self.seqs)
        self.arr = (_KvSeq * max(1, n))(*[s.c() for s in self.seqs])
        self.n = n
        self._mask_bufs = None
        self._mask_ptrs = None
        self.out = (ctypes.c_int64 * max(1, n))()
        self._checked_fmts = set()      # formats whose chunk tensors were sized against the library
        self._on_streams = set()        # (tensor, stream) pairs already given to record_stream
        # device tensors the kernels read besides the caller's own
        self._dev_tensors = [paged.k_addrs, paged.v_addrs] + [s.chunk_addrs for s in self.seqs]

    def set_masks(self, masks):
        """Host hit masks, one uint8 flag per chunk per sequence."""
        _need(len(masks) == self.n, f"need {self.n} hit masks, got {len(masks)}")
        bufs = []
        for i, (sq, m) in enumerate(zip(self.seqs, masks)):
            b = bytes(int(x) & 0xFF for x in (m.tolist() if hasattr(m, "tolist") else m))
            # the library reads one flag for every chunk of the sequence
            n_chunks = self.paged.num_chunks(sq.tok_start, sq.tok_end)
            _need(len(b) >= n_chunks, f"sequence {i}: hit mask has {len(b)} flags for {n_chunks} chunks")
            bufs.append(ctypes.create_string_buffer(b, max(1, len(b))))
        self._mask_bufs = bufs
        self._mask_ptrs = (ctypes.c_void_p * max(1, self.n))(
            *[ctypes.cast(b, ctypes.c_void_p).value for b in bufs])
        return self

    def check_chunks(self, fmt: int) -> "Batch":
        """For sequences whose chunks were given as tensors: one tensor per
        chunk of the range, each at least kv_chunk_bytes(tokens of the chunk,
        fmt) bytes, sizes from the library (kv_num_chunks, kv_chunk_tokens,
        kv_chunk_bytes).  The kernels write every chunk buffer up to that size
        and cannot see a buffer's end, so a short list or a small tensor is
        refused here, before anything runs.  Chunks given as an address
        tensor cannot be checked.  Done once per format."""
        if fmt in self._checked_fmts:
            return self
        p = self.paged
        for i, sq in enumerate(self.seqs):
            if sq._chunks is None:
                continue
            n = p.num_chunks(sq.tok_start, sq.tok_end)
            _need(len(sq._chunks) >= n, f"sequence {i}: {len(sq._chunks)} chunk tensors for {n} chunks")
            for c in range(n):
                need = p.chunk_bytes(p.chunk_tokens(sq.tok_start, sq.tok_end, c), fmt)
                have = sq._chunks[c].numel() * sq._chunks[c].element_size()
                _need(have >= need, f"sequence {i}, chunk {c}: {have} bytes, format {fmt} needs {need}")
        self._checked_fmts.add(fmt)
        return self

    def store_workspace_bytes(self, fmt: int = FMT_BF16) -> int:
        """Device bytes store(..., workspace=...) needs for these sequences
        in this format (kv_store_workspace_bytes; 0 for the fp8 formats)."""
        n = load().kv_store_workspace_bytes(ctypes.byref(self.paged.c), self.arr, self.n, fmt)
        if n == 0:
            _check(KV_OK if load().kv_last_error() == b"" else KV_EINVAL)
        return int(n)

    def new_store_workspace(self, fmt: int = FMT_BF16):
        """A device tensor of store_workspace_bytes(fmt) bytes (torch aligns it
        to 256), or None when the format needs none."""
        import torch
        n = self.store_workspace_bytes(fmt)
        return torch.empty(n, dtype=torch.uint8, device="cuda") if n > 0 else None

    def used_on(self, stream, *extra) -> None:
        """record_stream for the Batch's own device tensors (once per stream)
        and for ``extra`` tensors of this call (every time)."""
        _used_on(stream, self._dev_tensors, self._on_streams)
        _used_on(stream, extra)


def _batch(paged, seqs, fmt, stream, *extra) -> Batch:
    """The Batch for a call: chunk tensors sized for fmt, and the device
    tensors the call reads marked as used on stream."""
    b = seqs if isinstance(seqs, Batch) else Batch(paged, seqs)
    b.check_chunks(fmt)
    b.used_on(stream, *extra)
    return b


def store(paged: Paged, seqs, fmt: int = FMT_BF16, stream=None, workspace=None) -> None:
    """Gather every chunk of every sequence (kv_store_chunks).  With
    ``workspace`` (a device uint8 tensor of at least
    batch.store_workspace_bytes(fmt)) the bf16 gather runs through an address
    plan (kv_store_chunks_ws)."""
    b = _batch(paged, seqs, fmt, stream, workspace)
    if workspace is None:
        _check(load().kv_store_chunks(ctypes.byref(paged.c), b.arr, b.n, fmt, _stream_handle(stream)))
    else:
        ws_ptr, ws_bytes = _workspace(workspace)
        _check(load().kv_store_chunks_ws(ctypes.byref(paged.c), b.arr, b.n, fmt, ws_ptr, ws_bytes,
                                         _stream_handle(stream)))


def _event_handle(event, stream):
    if event is None:
        return None
    if not event.cuda_event:        # torch creates the event lazily on first record
        import torch
        event.record(stream if stream is not None else torch.cuda.current_stream())
    return event.cuda_event


def store_layer(paged: Paged, seqs, layer: int, fmt: int = FMT_BF16, stream=None, event=None,
                max_workgroups: int = 0) -> None:
    """Gather one layer of every chunk on ``stream``, then record ``event``
    (a torch.cuda.Event) on it (kv_store_layer)."""
    b = _batch(paged, seqs, fmt, stream)
    _check(load().kv_store_layer(ctypes.byref(paged.c), b.arr, b.n, fmt, layer, max_workgroups,
                                 _stream_handle(stream), _event_handle(event, stream)))


def _alt_handle(alt_stream) -> int | None:
    """Handle of a layer-range call's second stream (None: none)."""
    if alt_stream is None:
        return None
    h = alt_stream.cuda_stream if hasattr(alt_stream, "cuda_stream") else int(alt_stream)
    _need(h != 0, "alt_stream must be a stream of its own, not the null stream")
    return h


def _layer_arrays(n, max_workgroups, events, stream):
    """Host arrays of a layer-range call: caps (or None) and event handles (or None)."""
    caps = None
    if max_workgroups is not None:
        caps = [int(m) for m in max_workgroups]
        _need(len(caps) == n, f"need {n} workgroup caps, got {len(caps)}")
        caps = (ctypes.c_int32 * n)(*caps)
    evs = None
    if events is not None:
        _need(len(events) == n, f"need {n} events, got {len(events)}")
        evs = (ctypes.c_void_p * n)(*[_event_handle(e, stream) for e in events])
    return caps, evs


def store_layers(paged: Paged, seqs, layer_begin: int, layer_end: int, fmt: int = FMT_BF16, stream=None,
                 wait_events=None, events=None, max_workgroups=None, alt_stream=None) -> None:
    """Gather layers [layer_begin, layer_end) on ``stream`` in one call
    (kv_store_layers): before layer l, wait for ``wait_events[l - layer_begin]``
    (torch.cuda.Event, already recorded by the producer); after it, record
    ``events[l - layer_begin]``.  ``max_workgroups``: one cap per layer.
    ``alt_stream``: a second torch stream that takes every other layer, so
    consecutive layers' kernels may overlap."""
    b = _batch(paged, seqs, fmt, stream)
    b.used_on(alt_stream)
    n = layer_end - layer_begin
    caps, evs = _layer_arrays(n, max_workgroups, events, stream)
    waits = None
    if wait_events is not None:
        _need(len(wait_events) == n, f"need {n} wait events, got {len(wait_events)}")
        _need(all(e.cuda_event for e in wait_events), "wait events must have been recorded")
        waits = (ctypes.c_void_p * n)(*[e.cuda_event for e in wait_events])
    _check(load().kv_store_layers(ctypes.byref(paged.c), b.arr, b.n, fmt, layer_begin, layer_end, caps,
                                  _stream_handle(stream), _alt_handle(alt_stream), waits, evs))


def _workspace(workspace):
    """(address, bytes) of a workspace tensor, or (None, 0)."""
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise KvError(KV_EINVAL, "workspace must be a contiguous device tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _bins(bins, n):
    """One bin count per layer as a host int32 array."""
    bins = [int(b) for b in bins]
    if len(bins) != n:
        raise KvError(KV_EINVAL, f"need {n} bin counts, got {len(bins)}")
    return (ctypes.c_int32 * max(1, n))(*bins)


def store_cachegen(paged: Paged, seqs, key_bins, value_bins, stream=None) -> None:
    """CacheGen quantiser: gather + quantise every chunk (kv_store_chunks_cachegen).
    key_bins / value_bins: one bin count per layer, each in [4, 129]."""
    b = _batch(paged, seqs, FMT_CACHEGEN, stream)
    L = paged.c.num_layers
    _check(load().kv_store_chunks_cachegen(ctypes.byref(paged.c), b.arr, b.n, _bins(key_bins, L),
                                           _bins(value_bins, L), _stream_handle(stream)))


def retrieve_cachegen(paged: Paged, seqs, key_bins, value_bins, masks=None, stream=None, workspace=None) -> list:
    """Dequantise + scatter the leading hit chunks (kv_retrieve_chunks_cachegen);
    in pool-address order when a ``workspace`` (as for retrieve) is given.
    Returns the tokens made available per sequence."""
    b = _batch(paged, seqs, FMT_CACHEGEN, stream, workspace)
    if masks is not None:
        b.set_masks(masks)
    _need(b._mask_ptrs is not None, "hit masks are required")
    L = paged.c.num_layers
    ws_ptr, ws_bytes = _workspace(workspace)
    _check(load().kv_retrieve_chunks_cachegen(ctypes.byref(paged.c), b.arr, b._mask_ptrs, b.n,
                                              _bins(key_bins, L), _bins(value_bins, L), b.out,
                                              ws_ptr, ws_bytes, _stream_handle(stream)))
    return [int(b.out[i]) for i in range(b.n)]


def retrieve(paged: Paged, seqs, masks=None, fmt: int = FMT_BF16, stream=None, workspace=None) -> list:
    """Scatter the leading hit chunks back into pages (kv_retrieve_chunks).
    With ``workspace`` (a device uint8 tensor of at least
    paged.retrieve_workspace_bytes()) the bf16 scatter runs in pool-address
    order (kv_retrieve_chunks_ws).  Returns the tokens made available per
    sequence."""
    b = _batch(paged, seqs, fmt, stream, workspace)
    if masks is not None:
        b.set_masks(masks)
    _need(b._mask_ptrs is not None, "hit masks are required")
    if workspace is None:
        _check(load().kv_retrieve_chunks(ctypes.byref(paged.c), b.arr, b._mask_ptrs, b.n, fmt, b.out,
                                         _stream_handle(stream)))
    else:
        ws_ptr, ws_bytes = _workspace(workspace)
        _check(load().kv_retrieve_chunks_ws(ctypes.byref(paged.c), b.arr, b._mask_ptrs, b.n, fmt, b.out,
                                            ws_ptr, ws_bytes, _stream_handle(stream)))
    return [int(b.out[i]) for i in range(b.n)]


def retrieve_noalloc(paged: Paged, seqs, masks=None, fmt: int = FMT_BF16, stream=None) -> list:
    """retrieve in pool-address order with the library's own scratch array
    instead of a caller's workspace (kv_retrieve_chunks_noalloc): no device
    allocation anywhere in the call.  Calls that overlap on one GPU race.
    Returns the tokens made available per sequence."""
    b = _masked(paged, seqs, masks, fmt, stream)
    _check(load().kv_retrieve_chunks_noalloc(ctypes.byref(paged.c), b.arr, b._mask_ptrs, b.n, fmt, b.out,
                                             _stream_handle(stream)))
    return [int(b.out[i]) for i in range(b.n)]


def _masked(paged, seqs, masks, fmt, stream) -> Batch:
    b = _batch(paged, seqs, fmt, stream)
    if masks is not None:
        b.set_masks(masks)
    _need(b._mask_ptrs is not None, "hit masks are required")
    return b


def retrieve_layer(paged: Paged, seqs, layer: int, masks=None, fmt: int = FMT_BF16, stream=None,
                   event=None) -> None:
    """Scatter one layer of the leading hit chunks on ``stream``, then record
    ``event`` (a torch.cuda.Event) on it (kv_retrieve_layer)."""
    b = _masked(paged, seqs, masks, fmt, stream)
    _check(load().kv_retrieve_layer(ctypes.byref(paged.c), b.arr, b._mask_ptrs, b.n, fmt, layer,
                                    _stream_handle(stream), _event_handle(event, stream)))


def retrieve_layer_ex(paged: Paged, seqs, layer: int, masks=None, fmt: int = FMT_BF16, stream=None,
                      event=None, max_workgroups: int = 0) -> list:
    """retrieve_layer with a workgroup cap (kv_retrieve_layer_ex): a positive
    ``max_workgroups`` caps the grid so compute on another stream keeps most
    of the GPU.  Returns the tokens made available per sequence."""
    b = _masked(paged, seqs, masks, fmt, stream)
    _check(load().kv_retrieve_layer_ex(ctypes.byref(paged.c), b.arr, b._mask_ptrs, b.n, fmt, layer,
                                       b.out, max_workgroups, _stream_handle(stream),
                                       _event_handle(event, stream)))
    return [int(b.out[i]) for i in range(b.n)]


def retrieve_layers(paged: Paged, seqs, layer_begin: int, layer_end: int, masks=None, fmt: int = FMT_BF16,
                    stream=None, events=None, max_workgroups=None, alt_stream=None) -> list:
    """Scatter layers [layer_begin, layer_end) of the leading hit chunks on
    ``stream`` in one call, recording ``events[l - layer_begin]`` after layer
    l (kv_retrieve_layers).  ``max_workgroups``: one cap per layer, or None.
    ``alt_stream``: a second torch stream that takes every other layer, so
    consecutive layers' kernels may overlap.  Returns the tokens made
    available per sequence."""
    b = _masked(paged, seqs, masks, fmt, stream)
    b.used_on(alt_stream)
    caps, evs = _layer_arrays(layer_end - layer_begin, max_workgroups, events, stream)
    _check(load().kv_retrieve_layers(ctypes.byref(paged.c), b.arr, b._mask_ptrs, b.n, fmt, layer_begin,
                                     layer_end, caps, b.out, _stream_handle(stream), _alt_handle(alt_stream), evs))
    return [int(b.out[i]) for i in range(b.n)]


def take_faults() -> int:
    """Synchronise the device; return and clear the kernels' fault bits."""
    rc = load().kv_take_faults()
    if rc < 0:
        _check(rc)
    return rc


def copy_bytes(dst, src, nbytes: int, stream=None) -> None:
    """Plain contiguous device copy (measurement aid)."""
    _check(load().kv_copy_bytes(dst.data_ptr(), src.data_ptr(), nbytes, _stream_handle(stream)))


COPY_SCATTERED_READS, COPY_SCATTERED_WRITES = 1, 2


def copy_blocks(dst, src, nbytes: int, block_bytes: int, permute: int, stream=None) -> None:
    """Device copy with one side visited in scattered blocks (measurement aid,
    kv_copy_blocks): permute = COPY_SCATTERED_READS or COPY_SCATTERED_WRITES."""
    _check(load().kv_copy_blocks(dst.data_ptr(), src.data_ptr(), nbytes, block_bytes, permute,
                                 _stream_handle(stream)))
