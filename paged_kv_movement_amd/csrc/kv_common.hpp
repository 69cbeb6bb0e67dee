// kv_common.hpp -- shared device code of the paged <-> chunk KV movers
// (gfx950 / CDNA4): kernel arguments, work-unit decomposition, buffer
// descriptors, XCD-aware workgroup order, fault reporting.
//
// Pure data movement: no matrix cores.  Every kernel streams 16-byte vectors
// with coalesced accesses along a token row (H*D elements), one workgroup per
// unit (or tile of a unit) of work; the unit's page id and addresses are
// wave-uniform and computed in 32-bit scalar arithmetic from constants the
// host precomputes.
//
//   move_bf16<kToChunk>  work unit = (sequence, chunk, layer, K/V, page): a
//                        page's rows are contiguous in the pool and the same
//                        rows are contiguous in the chunk (each layer holds
//                        its K section, then its V section, of n rows), so a
//                        unit is one contiguous copy of rows*H*D*2 bytes
//                        (32 KiB for a full page at the Llama-3.1-8B shape).
//                        Each unit is cut into tiles of kBlock*kVpt 16-byte
//                        vectors, one workgroup per tile, and consecutive
//                        tiles are kept on one XCD.
//   store_fp8_onchip,    one workgroup per (sequence, chunk, layer, K/V)
//   store_fp8            group: the group's absolute maximum, then every
//                        element divided by the scale and encoded (e4m3 or
//                        e5m2).
//   retrieve_fp8         page units as move_bf16, decoding and scaling.
//
// A chunk format says, for K and for V, how many bytes an element takes (2:
// bf16 copied, 1: fp8) and how many float32 scales per layer follow the
// payload; a launch moves the K part, the V part or both, so a format that
// keeps K in bf16 and V in fp8 runs one kernel of each kind.
//
// The method these kernels implement is described on the LMCache paper-notes
// page ("LMCache: An Efficient KV Cache Layer for Enterprise-Scale LLM
// Inference", section "方法细节": configurable chunk size, layerwise
// pipeline) and on the serde framework page (section "7.1 fp8 量化").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvmove {

using u32x4 = __attribute__((ext_vector_type(4))) unsigned int;
using u32x2 = __attribute__((ext_vector_type(2))) unsigned int;

// Global-address-space views: loads and stores through these compile to
// global_* instructions (no flat aperture checks).
using gvec4 = __attribute__((address_space(1))) u32x4;
using gvec2 = __attribute__((address_space(1))) u32x2;
using gbyte = __attribute__((address_space(1))) uint8_t;
using gf32 = __attribute__((address_space(1))) float;
using gi32 = __attribute__((address_space(1))) int32_t;
using gu64 = __attribute__((address_space(1))) uint64_t;

constexpr int kMaxSeqs = 32;     // sequences per launch (kernel-argument budget)

enum : unsigned { kFaultPage = 1u, kFaultChunk = 2u, kFaultPool = 4u };

// Per-device fault word, set by kernels when a unit is skipped.
__device__ unsigned int g_kv_faults;

// Device addresses travel as integers (kernel arguments are built by host
// code) and become global-address-space pointers inside the kernels.
template <class T>
__device__ __forceinline__ T* gptr(uint64_t addr) { return reinterpret_cast<T*>(addr); }

struct SeqArg {
    uint64_t bt;              // block table: int32[]
    uint64_t chunks;          // chunk addresses: uint64[]
    uint32_t first_page;      // block-table index of the first token moved
    uint32_t n_full;          // full chunks moved
    uint32_t tail_tokens;     // tokens of a trailing partial chunk (0: none)
    uint32_t item_begin;      // first unit of this sequence in the launch
};

struct MoveArgs {
    uint64_t k_pages;         // uint64[L]: layer K pool addresses
    uint64_t v_pages;         // uint64[L]: layer V pool addresses
    int64_t num_pages;
    uint32_t item_base;       // unit index of blockIdx.x == 0
    uint32_t width;           // H*D elements per token row (multiple of 8)
    uint32_t page_size;       // P
    uint32_t chunk_size;      // C (multiple of P)
    uint32_t pages_per_chunk; // C / P
    uint32_t units_per_chunk; // units of one full chunk (depends on the kernel)
    uint32_t num_layers;      // L (chunk layout)
    uint32_t layer0;          // first layer moved
    uint32_t n_layers;        // layers moved
    uint32_t n_seqs;
    uint32_t tiles;           // tiles per page unit (tiled movers; 1 otherwise)
    uint32_t total_tiles;     // tiles in this launch; a workgroup may take several
    uint32_t kv0;             // first part moved: 0 = K, 1 = V
    uint32_t n_kv;            // parts moved (1 or 2)
    uint32_t elt_k;           // chunk bytes per K element (2: bf16, 1: fp8)
    uint32_t elt_v;           // chunk bytes per V element
    uint32_t n_scaled;        // float32 scales per layer after the payload (quantised parts)
    uint32_t pad_;
    SeqArg seq[kMaxSeqs];
};

// Byte offset, in a chunk of n_c tokens, of layer l's K (kv = 0) or V
// (kv = 1) section: layer by layer, K before V, n_c rows of the part's
// element size each.
__device__ __forceinline__ uint64_t section_offset(const MoveArgs& a, uint32_t l, uint32_t kv, uint32_t n_c)
{
    return ((uint64_t)l * (a.elt_k + a.elt_v) + kv * a.elt_k) * n_c * a.width;
}

// Byte offset of the float32 scale of quantised part (l, kv): the scales
// follow the payload in (layer, K/V) order, one per quantised part -- index
// 2l + kv when both parts are quantised, l when only V is.
__device__ __forceinline__ uint64_t scale_offset(const MoveArgs& a, uint32_t l, uint32_t kv, uint32_t n_c)
{
    return (uint64_t)a.num_layers * (a.elt_k + a.elt_v) * n_c * a.width +
           (l * a.n_scaled + kv + a.n_scaled - 2) * 4;
}

__device__ __forceinline__ void raise_fault(unsigned bit)
{
    if (threadIdx.x == 0) atomicOr(&g_kv_faults, bit);
}

__device__ __forceinline__ uint32_t find_seq(const MoveArgs& a, uint32_t item)
{
    uint32_t s = 0;
    while (s + 1 < a.n_seqs && item >= a.seq[s + 1].item_begin) ++s;
    return s;
}

// Arguments of the bf16 movers: the launch's arguments and a sequence lookup
// table, lut[k] = the sequence holding unit k << lut_shift (the host picks
// the shift so that 64 entries cover the launch).  A unit's sequence is then
// found from its table entry in a step or two instead of by a walk from the
// first sequence, one dependent argument load per step, ahead of every
// workgroup's first data load.
constexpr int kSeqLut = 64;
struct MoveArgsLut {
    MoveArgs m;
    uint32_t lut_shift;
    uint8_t lut[kSeqLut];
};

__device__ __forceinline__ uint32_t find_seq_lut(const MoveArgsLut& al, uint32_t item)
{
    uint32_t s = al.lut[item >> al.lut_shift];
    while (s + 1 < al.m.n_seqs && item >= al.m.seq[s + 1].item_begin) ++s;
    return s;
}

// Two float32 values -> two bf16 (round to nearest-even) packed in one word,
// a in bits [15:0] and b in [31:16]: one v_cvt_pk_bf16_f32 for the pair.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Running maximum of bf16 magnitude bits, two 16-bit lanes at once: m holds
// the maximum of the low halves in bits [15:0] and of the high halves in
// [31:16] (v_pk_max_u16, unsigned 16-bit lanes).  Integer order of the
// magnitude bits is magnitude order for non-NaN values; NaN codes sort above
// infinity.  pair_max folds the two halves at the end.
__device__ __forceinline__ uint32_t max_magnitude2(uint32_t m, const u32x4 x)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t mag = x[j] & 0x7FFF7FFFu;
        asm("v_pk_max_u16 %0, %1, %2" : "=v"(m) : "v"(m), "v"(mag));
    }
    return m;
}

__device__ __forceinline__ uint32_t pair_max(uint32_t m)
{
    const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    return lo > hi ? lo : hi;
}

__device__ __forceinline__ bool bad_addr(uint64_t p) { return p == 0 || (p & 15u) != 0; }

// A value every lane of the wave holds identically, moved into scalar
// registers (addresses read from device arrays arrive in vector registers;
// buffer descriptors built from them must be scalar).
__device__ __forceinline__ uint64_t wave_uniform(uint64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// A page unit: rows [j0, j0 + rows) of chunk c, layer l, K/V kv, held by
// pool page `page`.
struct PageUnit {
    int64_t page;
    uint32_t c;
    uint32_t n_c;    // tokens in chunk c
    uint32_t j0;     // first row inside the chunk
    uint32_t rows;
    uint32_t l;
    uint32_t kv;
    uint32_t s;      // sequence slot in the launch
};

// Units of a sequence run chunk-major: chunk, then layer, then K/V (the n_kv
// parts from kv0), then page, so consecutive workgroups fill consecutive
// bytes of a chunk.
__device__ __forceinline__ PageUnit locate_page_unit(const MoveArgs& a, uint32_t item, uint32_t seq)
{
    PageUnit u;
    u.s = seq;
    const SeqArg& sq = a.seq[u.s];
    uint32_t local = item - sq.item_begin;
    uint32_t pages_here;
    if (local < sq.n_full * a.units_per_chunk) {
        u.c = local / a.units_per_chunk;
        local -= u.c * a.units_per_chunk;
        u.n_c = a.chunk_size;
        pages_here = a.pages_per_chunk;
    } else {
        local -= sq.n_full * a.units_per_chunk;
        u.c = sq.n_full;
        u.n_c = sq.tail_tokens;
        pages_here = (sq.tail_tokens + a.page_size - 1) / a.page_size;
    }
    const uint32_t per_layer = a.n_kv * pages_here;
    u.l = a.layer0 + local / per_layer;
    const uint32_t r = local % per_layer;
    const uint32_t k = r >= pages_here ? 1u : 0u;     // second part (n_kv == 2 only)
    u.kv = a.kv0 + k;
    const uint32_t pi = r - k * pages_here;
    u.j0 = pi * a.page_size;
    const uint32_t left = u.n_c - u.j0;
    u.rows = left < a.page_size ? left : a.page_size;
    u.page = gptr<const gi32>(sq.bt)[sq.first_page + u.c * a.pages_per_chunk + pi];
    return u;
}

__device__ __forceinline__ PageUnit locate_page_unit(const MoveArgs& a, uint32_t item)
{
    return locate_page_unit(a, item, find_seq(a, item));
}

// Entries of a launch's page list sorted by page id (kv_order.hpp builds it):
// (sequence slot << 26) | page index in the sequence; kNoEntry pads it.
constexpr uint32_t kNoEntry = 0xFFFFFFFFu;
constexpr int kSeqShift = 26;
constexpr uint32_t kPageIndexMask = (1u << kSeqShift) - 1;

// The page unit of a pool-address-ordered launch: unit = slab * n_list + k,
// slab = the (layer, K/V) pair, k = the k-th smallest page id; false for a
// padding entry.  The list lives in caller memory (two calls racing on one
// workspace could leave a stray entry), so the sequence slot is masked into
// the launch's sequence array, and an entry naming no row its sequence moves
// gets page id -1 (its block-table read is redirected to its own list slot),
// which every tile function refuses with a fault bit before touching memory.
// Both checks are selects, not branches: a branch here held back the unit's
// remaining argument loads and cost the quantising ordered retrieves 8-14 %.
// kPinTail puts both candidates for n_c in registers before the select
// (otherwise the compiler loads from a selected address): measured 1 % faster
// for the bf16 scatter, but 6-10 % slower for the fp8 and CacheGen ones, so
// only the bf16 scatter sets it.
template <bool kPinTail = false>
__device__ __forceinline__ bool sorted_unit(const MoveArgs& a, uint64_t list, uint32_t n_list, uint32_t unit,
                                            PageUnit& u)
{
    static_assert((kMaxSeqs & (kMaxSeqs - 1)) == 0, "the sequence slot is masked");
    const uint32_t slab = unit / n_list, k = unit - slab * n_list;
    const uint32_t e = __builtin_amdgcn_readfirstlane(gptr<const gi32>(list)[k]);
    if (e == kNoEntry) return false;
    u.s = (e >> kSeqShift) & (kMaxSeqs - 1);
    const uint32_t q = e & kPageIndexMask;
    const SeqArg& sq = a.seq[u.s];
    uint32_t full = 0, tail = 0;
    if constexpr (kPinTail) {
        full = a.chunk_size;
        tail = sq.tail_tokens;
        asm volatile("" : "+s"(full), "+s"(tail));
    }
    u.c = q / a.pages_per_chunk;
    const uint32_t pi = q - u.c * a.pages_per_chunk;
    if constexpr (kPinTail)
        u.n_c = u.c < sq.n_full ? full : tail;
    else
        u.n_c = u.c < sq.n_full ? a.chunk_size : sq.tail_tokens;
    u.j0 = pi * a.page_size;
    const bool stray = u.c > sq.n_full || u.j0 >= u.n_c;
    const uint32_t left = u.n_c - u.j0;
    u.rows = stray || left > a.page_size ? a.page_size : left;
    u.l = a.layer0 + slab / a.n_kv;
    u.kv = a.kv0 + slab % a.n_kv;
    const uint64_t at = stray ? list + 4ull * k : sq.bt + 4ull * (sq.first_page + q);
    const int32_t page = *gptr<const gi32>(at);
    u.page = stray ? -1 : page;
    return true;
}

// Streams nvec 16-byte vectors src -> dst: kVpt loads in flight per thread
// before the matching stores; a strided remainder loop for partial pages.
template <int kBlock, int kVpt, bool kNtLoad, bool kNtStore>
__device__ __forceinline__ void copy_vectors(const gvec4* __restrict__ src, gvec4* __restrict__ dst,
                                             uint32_t nvec)
{
    const uint32_t t = threadIdx.x;
    uint32_t base = 0;
    for (; base + kBlock * kVpt <= nvec; base += kBlock * kVpt) {
        u32x4 v[kVpt];
#pragma unroll
        for (int k = 0; k < kVpt; ++k) {
            const gvec4* p = src + base + k * kBlock + t;
            v[k] = kNtLoad ? __builtin_nontemporal_load(p) : *p;
        }
#pragma unroll
        for (int k = 0; k < kVpt; ++k) {
            gvec4* p = dst + base + k * kBlock + t;
            if (kNtStore) __builtin_nontemporal_store(v[k], p); else *p = v[k];
        }
    }
    for (uint32_t i = base + t; i < nvec; i += kBlock) {
        const u32x4 v = kNtLoad ? __builtin_nontemporal_load(src + i) : src[i];
        if (kNtStore) __builtin_nontemporal_store(v, dst + i); else dst[i] = v;
    }
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  Renumber them so that each XCD walks one contiguous range of the
// grid: neighbouring tiles (the pieces of one page, the rows of one chunk)
// then run on the same XCD, one after the other.  A bijection on
// [0, 8 * (grid / 8)); the few workgroups past that keep their number.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t b, uint32_t grid)
{
    const uint32_t per = grid / 8;
    return b < per * 8 ? (b % 8) * per + b / 8 : b;
}

// Tiles [first, last) of this workgroup.  With one workgroup per tile (the
// default launch) that is a single tile; with a capped grid each workgroup
// walks a contiguous run of tiles, and the runs stay XCD-contiguous.
struct TileRange {
    uint32_t first, last;
};

__device__ __forceinline__ TileRange my_tiles(uint32_t total)
{
    const uint32_t w = xcd_contiguous(blockIdx.x, gridDim.x);
    const uint32_t per = (total + gridDim.x - 1) / gridDim.x;
    const uint32_t first = w * per;
    const uint32_t last = first + per < total ? first + per : total;
    return {first, last};
}

// Cache-policy bits of the buffer instructions (gfx94x/gfx950 encoding of
// the aux operand): 2 = nt (streaming, do not keep in cache), 16 = sc1.
enum : int { kCpolNt = 2, kCpolSc1 = 16 };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(uint64_t base, uint32_t nbytes)
{
    // raw buffer: stride 0, range-checked against nbytes (word 3 = gfx9 format)
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), (short)0, (int)nbytes,
                                             0x00020000);
}

// Copies nbytes (a multiple of 16, at most kBlock*kVpt*16) from src to dst:
// kVpt loads in flight per thread, then the stores.  Buffer accesses at or
// past nbytes are discarded by the hardware range check (loads return 0,
// stores are dropped), so a partial tile needs no per-vector guard.
template <int kBlock, int kVpt, int kAuxLoad, int kAuxStore>
__device__ __forceinline__ void copy_tile(uint64_t src, uint64_t dst, uint32_t nbytes)
{
    const __amdgpu_buffer_rsrc_t rs = byte_range(src, nbytes);
    const __amdgpu_buffer_rsrc_t rd = byte_range(dst, nbytes);
    u32x4 v[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k)
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (k * kBlock + threadIdx.x) * 16, 0, kAuxLoad);
#pragma unroll
    for (int k = 0; k < kVpt; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(v[k], rd, (k * kBlock + threadIdx.x) * 16, 0, kAuxStore);
}

}  // namespace kvmove
