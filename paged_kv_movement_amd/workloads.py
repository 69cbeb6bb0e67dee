"""Seeded synthetic workloads for paged <-> chunk KV movement.

This module only draws inputs: pool contents, block tables, token ranges and
hit masks.  It holds none of the method's arithmetic (no slot, chunk or
quantisation computation), so both the GPU path and the CPU oracle can take
their inputs from it.

Recipe (every draw is seeded by the workload's seed):
  * block tables: ``numpy.random.default_rng(seed).permutation(num_pages)``,
    cut into disjoint consecutive slices, one per sequence;
  * outlier channels (fp8 workload): 4 distinct channel indices in [0, H*D)
    from the same generator, after the permutation;
  * pool values, host-sized workloads: ``default_rng(seed + 1000)``
    ``standard_normal(float32)``, outlier channels x20 in float32, then
    rounded to bfloat16 by torch (round-to-nearest-even);
  * pool values, HBM-sized workloads: ``torch.randn`` on the device with a
    ``torch.Generator`` seeded with the seed, one (layer, K/V) slab at a time,
    same outlier scaling and bfloat16 rounding;
  * ``bits`` variant: uniform 16-bit patterns (NaN payloads, infinities,
    subnormals, -0 included) to check byte transparency.

The shapes follow the KV caches of the models the pages evaluate (Llama-3.1-8B:
32 layers, 8 KV heads, head_dim 128; a 70B-style 80-layer shape) and the
pages' 10K-token multi-turn context, with 16-token pages and 256-token chunks.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Sequence:
    block_table: np.ndarray      # int32 page ids
    tok_start: int
    tok_end: int
    hit_mask: np.ndarray         # uint8, one flag per chunk (retrieve)


@dataclass
class Workload:
    name: str
    seed: int
    num_layers: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    chunk_size: int
    num_pages: int
    seqs: list = field(default_factory=list)
    outlier_channels: np.ndarray | None = None
    outlier_gain: float = 20.0
    values: str = "normal"       # "normal" | "bits"

    @property
    def width(self) -> int:
        return self.num_kv_heads * self.head_dim

    def pool_shape(self):
        return (self.num_layers, 2, self.num_pages, self.page_size, self.width)

    def pool_nbytes(self) -> int:
        return int(np.prod(self.pool_shape())) * 2


def _slices(perm: np.ndarray, pages_per_seq) -> list:
    out, at = [], 0
    for n in pages_per_seq:
        out.append(np.ascontiguousarray(perm[at:at + n], dtype=np.int32))
        at += n
    assert at <= perm.size
    return out


def tiny() -> Workload:
    """L=2, 2 KV heads, head_dim 64; pool of 64 pages; one 256-token sequence
    on 16 pages drawn as a permutation of the pool; mask [1]."""
    seed = 0
    rng = np.random.default_rng(seed)
    perm = rng.permutation(64)
    w = Workload("tiny", seed, 2, 2, 64, 16, 256, 64)
    w.seqs = [Sequence(_slices(perm, [16])[0], 0, 256, np.ones(1, np.uint8))]
    return w


def llama8b(n_hit: int = 30) -> Workload:
    """Llama-3.1-8B KV shape: L=32, 8 KV heads, head_dim 128; pool of 8192
    pages; 8 sequences of 10000 tokens (625 pages each, disjoint); retrieve
    mask = n_hit ones then zeros over the 40 chunks."""
    seed = 1
    rng = np.random.default_rng(seed)
    perm = rng.permutation(8192)
    w = Workload("llama3.1-8b", seed, 32, 8, 128, 16, 256, 8192)
    n_chunks = 40
    mask = np.zeros(n_chunks, np.uint8)
    mask[:n_hit] = 1
    w.seqs = [Sequence(bt, 0, 10000, mask.copy()) for bt in _slices(perm, [625] * 8)]
    return w


def llama8b_tp8_share(n_hit: int = 30) -> Workload:
    """One rank's share of the 8B workload under 8-way tensor parallelism:
    each rank caches its own KV head, so L=32, 1 KV head, head_dim 128
    (256-byte token rows, 4 KiB pages); the same 8 sequences of 10000 tokens
    on an 8192-page pool, retrieve mask n_hit ones then zeros."""
    seed = 5
    rng = np.random.default_rng(seed)
    perm = rng.permutation(8192)
    w = Workload("llama3.1-8b-tp8-share", seed, 32, 1, 128, 16, 256, 8192)
    mask = np.zeros(40, np.uint8)
    mask[:n_hit] = 1
    w.seqs = [Sequence(bt, 0, 10000, mask.copy()) for bt in _slices(perm, [625] * 8)]
    return w


def layerwise8b() -> Workload:
    """One 10240-token sequence (40 full chunks, 640 pages) at the 8B shape on
    an 8192-page pool; all chunks hit."""
    seed = 2
    rng = np.random.default_rng(seed)
    perm = rng.permutation(8192)
    w = Workload("layerwise-8b", seed, 32, 8, 128, 16, 256, 8192)
    w.seqs = [Sequence(_slices(perm, [640])[0], 0, 10240, np.ones(40, np.uint8))]
    return w


def llama70b() -> Workload:
    """70B-style KV shape: L=80, 8 KV heads, head_dim 128; one 32768-token
    sequence (128 chunks) on 2048 pages of a 4096-page pool; all chunks hit."""
    seed = 3
    rng = np.random.default_rng(seed)
    perm = rng.permutation(4096)
    w = Workload("llama-70b-style", seed, 80, 8, 128, 16, 256, 4096)
    w.seqs = [Sequence(_slices(perm, [2048])[0], 0, 32768, np.ones(128, np.uint8))]
    return w


def fp8_8b(n_hit: int = 40) -> Workload:
    """The 8B workload's sequences with N(0,1) values and 4 seeded outlier
    channels scaled by 20 (the same channels for K and V in every layer)."""
    seed = 4
    rng = np.random.default_rng(seed)
    perm = rng.permutation(8192)
    w = Workload("fp8-8b", seed, 32, 8, 128, 16, 256, 8192)
    mask = np.zeros(40, np.uint8)
    mask[:n_hit] = 1
    w.seqs = [Sequence(bt, 0, 10000, mask.copy()) for bt in _slices(perm, [625] * 8)]
    w.outlier_channels = np.sort(rng.choice(w.width, size=4, replace=False)).astype(np.int64)
    return w


def custom(name, seed, num_layers, num_kv_heads, head_dim, num_pages, seq_ranges,
           masks=None, page_size=16, chunk_size=256, pages_per_seq=None,
           outliers=0, values="normal") -> Workload:
    """A free-form workload for edge cases: ``seq_ranges`` is a list of
    (tok_start, tok_end); each sequence gets a disjoint slice of a seeded
    permutation of the pool, long enough to cover tok_end."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_pages)
    if pages_per_seq is None:
        pages_per_seq = [-(-e // page_size) for (_, e) in seq_ranges]
    w = Workload(name, seed, num_layers, num_kv_heads, head_dim, page_size, chunk_size, num_pages,
                 values=values)
    bts = _slices(perm, pages_per_seq)
    for i, ((s, e), bt) in enumerate(zip(seq_ranges, bts)):
        m = masks[i] if masks is not None else np.ones(max(0, -(-(e - s) // chunk_size)), np.uint8)
        w.seqs.append(Sequence(bt, s, e, np.asarray(m, np.uint8)))
    if outliers:
        w.outlier_channels = np.sort(rng.choice(w.width, size=outliers, replace=False)).astype(np.int64)
    return w


ALL = {"tiny": tiny, "llama3.1-8b": llama8b, "layerwise-8b": layerwise8b,
       "llama-70b-style": llama70b, "fp8-8b": fp8_8b, "llama3.1-8b-tp8-share": llama8b_tp8_share}


def host_pool(w: Workload) -> np.ndarray:
    """Pool contents in host memory, uint16 [L, 2, num_pages, P, H*D]."""
    import torch
    rng = np.random.default_rng(w.seed + 1000)
    shape = w.pool_shape()
    if w.values == "bits":
        return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if w.outlier_channels is not None:
        x[..., w.outlier_channels] *= np.float32(w.outlier_gain)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def device_pool(w: Workload, device="cuda"):
    """Pool contents generated on the device: torch bf16 [L, 2, num_pages, P, H, D]."""
    import torch
    L, two, n, P, E = w.pool_shape()
    pool = torch.empty((L, 2, n, P, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    if w.values == "bits":
        for l in range(L):
            for kv in range(2):
                r = torch.randint(-(1 << 15), 1 << 15, (n, P, E), generator=g, device=device,
                                  dtype=torch.int32)
                pool[l, kv].view(torch.int16).view(n, P, E).copy_(r.to(torch.int16))
        return pool
    for l in range(L):
        for kv in range(2):
            x = torch.randn((n, P, E), generator=g, device=device, dtype=torch.float32)
            if w.outlier_channels is not None:
                idx = torch.as_tensor(w.outlier_channels, device=device)
                x[..., idx] *= w.outlier_gain
            pool[l, kv].view(n, P, E).copy_(x.to(torch.bfloat16))
            del x
    return pool
