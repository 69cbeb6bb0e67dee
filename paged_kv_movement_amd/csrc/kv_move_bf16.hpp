// kv_move_bf16.hpp -- the bf16 movers (gather pages -> chunks, scatter
// chunks -> pages) and the plain copy used to calibrate measurements.
#pragma once

#include "kv_common.hpp"

namespace kvmove {

// Launch shapes, from sweeps on MI355X at the Llama-3.1-8B KV shape.  A full
// launch uses one-wave workgroups, each moving a 2 KiB tile (64 threads x 2
// vectors of 16 B; sixteen tiles per 32 KiB page): more, smaller workgroups
// kept HBM busier than 8 KiB tiles (gather +1 %, destination-ordered scatter
// +2 %).  A launch with a workgroup cap keeps 256-thread workgroups and 8 KiB
// tiles, so a cap means the same share of the GPU as before.  Streaming (nt)
// cache policy with sc1, loads and stores alike.
constexpr int kMoveBlock = 64;
constexpr int kMoveBlockCapped = 256;
constexpr int kMoveVpt = 2;
constexpr int kGatherAuxLoad = kCpolNt | kCpolSc1;
constexpr int kGatherAuxStore = kCpolNt | kCpolSc1;
constexpr int kScatterAuxLoad = kCpolNt | kCpolSc1;
constexpr int kScatterAuxStore = kCpolNt | kCpolSc1;
// The chunk-major scatter of a whole retrieve (every layer in one launch)
// writes gigabytes of pages in block-table order, that is at random places
// in the pool: there stores without the streaming hint (sc1 only) measured
// 0.6 % faster at the Llama-3.1-8B shape.  The ordered scatter, whose writes
// ascend, and the one-layer launches keep nt + sc1 (sc1 alone: -9 % and
// -2.5 %); the fp8 and CacheGen retrieves gained nothing from it.
constexpr int kScatterAuxStoreWhole = kCpolSc1;
// The plain copy (measurement aid): the fastest contiguous-copy shape of a
// sweep over tile size (1-16 KiB), workgroup size (64-1024 threads), vectors
// per lane (1-8), cache policy and workgroup order on the 8B workload's
// 10.49 GB: 256 threads x 1 vector, nt + sc1 both ways, XCD-contiguous
// order, 6.78 TB/s (512 x 1: 6.79; 64 x 1: 6.75; the movers' 64 x 2: 6.31).
constexpr int kCopyBlock = 256;
constexpr int kCopyVpt = 1;

// Gather (kToChunk) or scatter (!kToChunk) of tile `tile` of page unit u,
// bf16 copied bit for bit (the chunk part moved holds 2-byte elements).
template <bool kToChunk, int kBlock, int kVpt, int kAuxLoad, int kAuxStore>
__device__ __forceinline__ void move_unit_tile(const MoveArgs& a, const PageUnit& u, uint32_t tile)
{
    const uint32_t row_bytes = a.width * 2;
    const uint32_t nbytes = u.rows * row_bytes;
    const uint32_t lo = tile * (kBlock * kVpt * 16);
    if (lo >= nbytes) return;                         // tile past a short (tail) page
    if (u.page < 0 || u.page >= a.num_pages) { raise_fault(kFaultPage); return; }
    const uint64_t pool = wave_uniform(gptr<const gu64>(u.kv ? a.v_pages : a.k_pages)[u.l]);
    const uint64_t chunk = wave_uniform(gptr<const gu64>(a.seq[u.s].chunks)[u.c]);
    if (bad_addr(pool)) { raise_fault(kFaultPool); return; }
    if (bad_addr(chunk)) { raise_fault(kFaultChunk); return; }
    const uint32_t left = nbytes - lo;
    const uint32_t n = left < kBlock * kVpt * 16 ? left : kBlock * kVpt * 16;
    const uint64_t page_addr = pool + (uint64_t)u.page * a.page_size * row_bytes + lo;
    const uint64_t chunk_addr = chunk + section_offset(a, u.l, u.kv, u.n_c) + (uint64_t)u.j0 * row_bytes + lo;
    if (kToChunk) copy_tile<kBlock, kVpt, kAuxLoad, kAuxStore>(page_addr, chunk_addr, n);
    else copy_tile<kBlock, kVpt, kAuxLoad, kAuxStore>(chunk_addr, page_addr, n);
}

// Tile b of the launch: page units in chunk-major order, a.tiles tiles each.
template <bool kToChunk, int kBlock, int kVpt, int kAuxLoad, int kAuxStore>
__device__ __forceinline__ void move_tile(const MoveArgsLut& al, uint32_t b)
{
    const MoveArgs& a = al.m;
    const uint32_t unit = b / a.tiles;
    const uint32_t tile = b - unit * a.tiles;
    const uint32_t item = a.item_base + unit;
    move_unit_tile<kToChunk, kBlock, kVpt, kAuxLoad, kAuxStore>(a, locate_page_unit(a, item, find_seq_lut(al, item)),
                                                                 tile);
}

// Grid = one workgroup per tile (units * a.tiles), or fewer workgroups that
// each take a contiguous run of tiles.
template <bool kToChunk, int kBlock, int kVpt, int kAuxLoad, int kAuxStore>
__global__ __launch_bounds__(kBlock) void move_bf16(MoveArgsLut al)
{
    if (gridDim.x >= al.m.total_tiles) {      // one workgroup per tile: straight-line code
        move_tile<kToChunk, kBlock, kVpt, kAuxLoad, kAuxStore>(al, xcd_contiguous(blockIdx.x, gridDim.x));
        return;
    }
    const TileRange r = my_tiles(al.m.total_tiles);
    for (uint32_t b = r.first; b < r.last; ++b)
        move_tile<kToChunk, kBlock, kVpt, kAuxLoad, kAuxStore>(al, b);
}

// Address plan of a gather (kv_store_chunks_ws): one kPlanEntryBytes entry
// per page unit of a launch, in the launch's unit order -- the unit's
// page-side address, its chunk-side address and its byte count (0: the unit
// is skipped and its fault bit set) -- written by build_gather_plan, read by
// gather_planned.  With the addresses ready, a workgroup's first data load
// waits on one uniform load of its entry instead of the movers' chain of
// argument, block-table and address reads, and 4 KiB tiles of 256 threads
// (the fastest plain-copy shape) keep HBM busy: the 8B gather measured 2 %
// faster, plan included.
constexpr int kPlanEntryBytes = 32;
constexpr int kPlanBuildBlock = 256;
constexpr int kPlanBlock = 256;
constexpr int kPlanVpt = 1;

// One thread per page unit of the launch (units [0, n_units) from
// a.item_base): the unit's addresses, with the movers' checks.
__global__ __launch_bounds__(kPlanBuildBlock) void build_gather_plan(MoveArgsLut al, uint64_t plan, uint32_t n_units)
{
    const MoveArgs& a = al.m;
    const uint32_t i = blockIdx.x * kPlanBuildBlock + threadIdx.x;
    if (i >= n_units) return;
    const uint32_t item = a.item_base + i;
    uint32_t s = al.lut[item >> al.lut_shift];
    while (s + 1 < a.n_seqs && item >= a.seq[s + 1].item_begin) ++s;
    const PageUnit u = locate_page_unit(a, item, s);
    const uint64_t pool = gptr<const gu64>(u.kv ? a.v_pages : a.k_pages)[u.l];
    const uint64_t chunk = gptr<const gu64>(a.seq[u.s].chunks)[u.c];
    const uint32_t row_bytes = a.width * 2;
    uint64_t page_addr = 0, chunk_addr = 0;
    uint32_t bytes = 0;
    if (u.page < 0 || u.page >= a.num_pages) atomicOr(&g_kv_faults, kFaultPage);
    else if (bad_addr(pool)) atomicOr(&g_kv_faults, kFaultPool);
    else if (bad_addr(chunk)) atomicOr(&g_kv_faults, kFaultChunk);
    else {
        page_addr = pool + (uint64_t)u.page * a.page_size * row_bytes;
        chunk_addr = chunk + section_offset(a, u.l, u.kv, u.n_c) + (uint64_t)u.j0 * row_bytes;
        bytes = u.rows * row_bytes;
    }
    gu64* e = gptr<gu64>(plan + (uint64_t)i * kPlanEntryBytes);
    e[0] = page_addr;
    e[1] = chunk_addr;
    e[2] = bytes;
    e[3] = 0;
}

// The gather over a plan: tiles tiles of kBlock * kVpt vectors per unit, one
// workgroup per tile, XCD-contiguous.
template <int kBlock, int kVpt, int kAuxLoad, int kAuxStore>
__global__ __launch_bounds__(kBlock) void gather_planned(const uint64_t* __restrict__ plan, uint32_t tiles)
{
    const uint32_t b = xcd_contiguous(blockIdx.x, gridDim.x);
    const uint32_t unit = b / tiles, t = b - unit * tiles;
    const uint64_t* e = plan + (uint64_t)unit * (kPlanEntryBytes / 8);      // uniform: scalar loads
    const uint64_t page_addr = e[0], chunk_addr = e[1];
    const uint32_t bytes = (uint32_t)e[2];
    constexpr uint32_t tile = kBlock * kVpt * 16;
    const uint32_t lo = t * tile;
    if (lo >= bytes) return;                          // tile past a short page, or a skipped unit
    const uint32_t n = bytes - lo < tile ? bytes - lo : tile;
    copy_tile<kBlock, kVpt, kAuxLoad, kAuxStore>(page_addr + lo, chunk_addr + lo, n);
}

// Plain contiguous copy (measurement aid): one tile of kBlock*kVpt vectors
// per workgroup, the movers' instruction form (buffer loads and stores, nt +
// sc1, XCD-contiguous workgroup order) without their page lookups.
template <int kBlock, int kVpt>
__global__ __launch_bounds__(kBlock) void copy_contiguous(uint64_t src, uint64_t dst, int64_t nbytes)
{
    const int64_t tile = (int64_t)kBlock * kVpt * 16;
    const int64_t lo = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * tile;
    const int64_t left = nbytes - lo;
    copy_tile<kBlock, kVpt, kCpolNt | kCpolSc1, kCpolNt | kCpolSc1>(src + lo, dst + lo,
                                                                   (uint32_t)(left < tile ? left : tile));
}

}  // namespace kvmove
