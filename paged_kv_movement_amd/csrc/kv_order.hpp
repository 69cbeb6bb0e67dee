// kv_order.hpp -- the bf16 scatter in pool-address order.
//
// The chunk-major scatter writes each 32 KiB page at a random place in the
// pool (block tables are random), and DRAM takes random writes worse than
// random reads: write requests wait on DRAM credits about 1.6x as often as
// in the gather.  Visiting the same page units by destination address --
// layer, K/V, then page id -- was measured 6 % faster on the Llama-3.1-8B
// workload, with the reads from the chunks becoming the random side.
//
// The order needs the hit pages of a launch sorted by page id.  Page ids
// are distinct (a retrieve's precondition) and below num_pages, so the sort
// is an inverse map over the page ids followed by a compaction:
//   fill_u32       inv[0 .. num_pages) = kNoEntry
//   invert_pages   inv[page] = (sequence slot << 26) | page index in the sequence
//   compact_pages  list = the entries of inv in page order, padded with kNoEntry
//   (order_pages_small does all three in one workgroup, inv in LDS, for pools
//   of at most 32768 pages)
//   scatter_sorted one workgroup per tile of (layer, K/V, list entry); the
//                  fp8 and CacheGen retrieves have ordered variants too
//                  (retrieve_fp8_sorted, retrieve_cachegen_sorted)
// inv and list live in a workspace the caller provides (2 * num_pages words).
#pragma once

#include "kv_move_bf16.hpp"

namespace kvmove {

constexpr int kCompactBlock = 1024;
constexpr int kCompactPerThread = 16;

using gu32 = __attribute__((address_space(1))) uint32_t;

__global__ __launch_bounds__(256) void fill_u32(uint64_t dst, uint32_t n, uint32_t value)
{
    for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) gptr<gu32>(dst)[i] = value;
}

// Pages a sequence moves in this launch: its full chunks' pages, then the tail's.
__device__ __forceinline__ uint32_t seq_pages(const MoveArgs& a, const SeqArg& sq)
{
    return sq.n_full * a.pages_per_chunk + (sq.tail_tokens + a.page_size - 1) / a.page_size;
}

// One thread per page moved by the launch.  A page id out of range is left
// out of the map (its rows are not written) and reported as a fault.
__global__ __launch_bounds__(256) void invert_pages(MoveArgs a, uint64_t inv, uint32_t total_pages)
{
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i >= total_pages) return;
    uint32_t s = 0, first = 0;
    for (; s + 1 < a.n_seqs; ++s) {
        const uint32_t n = seq_pages(a, a.seq[s]);
        if (i < first + n) break;
        first += n;
    }
    const uint32_t q = i - first;
    const int64_t page = gptr<const gi32>(a.seq[s].bt)[a.seq[s].first_page + q];
    if (page < 0 || page >= a.num_pages) {
        atomicOr(&g_kv_faults, kFaultPage);
        return;
    }
    gptr<gu32>(inv)[page] = (s << kSeqShift) | q;
}

// The entries of src[0 .. num_pages) in page order, written to
// list[0 .. count), and kNoEntry in list[count .. list_len), by one
// workgroup of kCompactBlock threads (src: the inverse map, in global memory
// or LDS).
template <class Src>
__device__ __forceinline__ void compact_entries(Src src, uint32_t num_pages, uint64_t list, uint32_t list_len,
                                                uint32_t* wave_sum)
{
    const uint32_t t = threadIdx.x, lane = t % 64, wave = t / 64;
    uint32_t base = 0;
    for (uint32_t start = 0; start < num_pages; start += kCompactBlock * kCompactPerThread) {
        uint32_t v[kCompactPerThread];
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < kCompactPerThread; ++j) {
            const uint32_t idx = start + t * kCompactPerThread + j;
            v[j] = idx < num_pages ? src[idx] : kNoEntry;
            cnt += v[j] != kNoEntry;
        }
        // inclusive prefix of cnt over the wave, then over the waves
        uint32_t incl = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t o = __shfl_up(incl, off, 64);
            if (lane >= (uint32_t)off) incl += o;
        }
        if (lane == 63) wave_sum[wave] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
        for (int w = 0; w < kCompactBlock / 64; ++w) {
            before += (uint32_t)w < wave ? wave_sum[w] : 0u;
            total += wave_sum[w];
        }
        uint32_t at = base + before + incl - cnt;
#pragma unroll
        for (int j = 0; j < kCompactPerThread; ++j)
            if (v[j] != kNoEntry && at < list_len) gptr<gu32>(list)[at++] = v[j];
        base += total;
        __syncthreads();                              // wave_sum is reused
    }
    for (uint32_t k = base + t; k < list_len; k += kCompactBlock) gptr<gu32>(list)[k] = kNoEntry;
}

__global__ __launch_bounds__(kCompactBlock) void compact_pages(uint64_t inv, uint32_t num_pages, uint64_t list,
                                                               uint32_t list_len)
{
    __shared__ uint32_t wave_sum[kCompactBlock / 64];
    compact_entries(gptr<const gu32>(inv), num_pages, list, list_len, wave_sum);
}

// Pools of at most kSmallPoolPages pages: the inverse map lives in LDS, and
// one workgroup clears it, inverts the launch's pages and compacts them in
// one launch, with no round trip through global memory (the three kernels
// above take about 16 us plus two launch gaps at 8192 pages; this one
// replaces them for every pool up to 32768 pages).
constexpr uint32_t kSmallPoolPages = 32768;

__global__ __launch_bounds__(kCompactBlock) void order_pages_small(MoveArgs a, uint64_t list, uint32_t n_list,
                                                                   uint32_t num_pages)
{
    __shared__ uint32_t inv[kSmallPoolPages];
    __shared__ uint32_t wave_sum[kCompactBlock / 64];
    __shared__ uint32_t seq_end[kMaxSeqs];     // running page count after each sequence
    __shared__ uint64_t seq_bt[kMaxSeqs];      // block-table address of each sequence's first moved page
    const uint32_t t = threadIdx.x;
    if (num_pages > kSmallPoolPages) num_pages = kSmallPoolPages;   // the host launches it for such pools only
    if (t == 0) {
        uint32_t acc = 0;
        for (uint32_t s = 0; s < a.n_seqs; ++s) {
            acc += seq_pages(a, a.seq[s]);
            seq_end[s] = acc;
            seq_bt[s] = a.seq[s].bt + 4ull * a.seq[s].first_page;
        }
    }
    for (uint32_t i = t; i < num_pages; i += kCompactBlock) inv[i] = kNoEntry;
    __syncthreads();
    // invert: a thread's block-table loads are all issued before any is used,
    // so the phase costs one memory latency rather than one per entry
    constexpr int kBatch = 8;
    for (uint32_t i0 = 0; i0 < n_list; i0 += kBatch * kCompactBlock) {
        int32_t page[kBatch];
        uint32_t entry[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const uint32_t i = i0 + k * kCompactBlock + t;
            page[k] = -1;
            entry[k] = kNoEntry;
            if (i < n_list) {
                uint32_t s = 0;
                while (s + 1 < a.n_seqs && i >= seq_end[s]) ++s;
                const uint32_t q = i - (s > 0 ? seq_end[s - 1] : 0u);
                entry[k] = (s << kSeqShift) | q;
                page[k] = gptr<const gi32>(seq_bt[s])[q];
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (entry[k] == kNoEntry) continue;
            if (page[k] < 0 || page[k] >= a.num_pages || (uint32_t)page[k] >= num_pages) {
                atomicOr(&g_kv_faults, kFaultPage);
                continue;
            }
            inv[page[k]] = entry[k];
        }
    }
    __syncthreads();
    compact_entries(inv, num_pages, list, n_list, wave_sum);
}

// bf16 scatter in destination order: a.tiles tiles per sorted unit, one
// workgroup per tile.
template <int kBlock, int kVpt, int kAuxLoad, int kAuxStore>
__global__ __launch_bounds__(kBlock) void scatter_sorted(MoveArgs a, uint64_t list, uint32_t n_list)
{
    const uint32_t b = xcd_contiguous(blockIdx.x, gridDim.x);
    const uint32_t unit = b / a.tiles, tile = b - unit * a.tiles;
    PageUnit u;
    if (!sorted_unit<true>(a, list, n_list, unit, u)) return;
    move_unit_tile<false, kBlock, kVpt, kAuxLoad, kAuxStore>(a, u, tile);
}

}  // namespace kvmove
