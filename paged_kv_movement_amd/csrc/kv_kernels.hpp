// kv_kernels.hpp -- HIP kernels (gfx950 / CDNA4) for paged <-> chunk KV movement.
//
// Pure data movement: no matrix cores.  Every kernel streams 16-byte vectors
// (global_load/store_dwordx4) with coalesced accesses along a token row
// (H*D elements), one workgroup per unit of work; the unit's page id and
// addresses are wave-uniform and computed in 32-bit scalar arithmetic from
// constants the host precomputes.
//
//   move_bf16<kToChunk>  work unit = (sequence, chunk, layer, K/V, page): a
//                        page's rows are contiguous in the pool and the same
//                        rows are contiguous in the chunk ([L][2][n][H*D]
//                        layout), so a unit is one contiguous copy of
//                        rows*H*D*2 bytes (32 KiB for a full page at the
//                        Llama-3.1-8B shape).  Each unit is cut into tiles of
//                        kBlock*kVpt 16-byte vectors, one workgroup per tile,
//                        and consecutive tiles are kept on one XCD.
//   store_fp8            one workgroup per (sequence, chunk, layer, K/V)
//                        group: pass 1 takes the group's absolute maximum,
//                        pass 2 re-reads, divides by the scale, encodes e4m3.
//   retrieve_fp8         page units as move_bf16, decoding e4m3 and scaling.
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
    uint32_t tiles;           // workgroups per page unit (tiled movers; 1 otherwise)
    SeqArg seq[kMaxSeqs];
};

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

// Units of a sequence run chunk-major: chunk, then layer, then K/V, then page,
// so consecutive workgroups fill consecutive bytes of a chunk.
__device__ __forceinline__ PageUnit locate_page_unit(const MoveArgs& a, uint32_t item)
{
    PageUnit u;
    u.s = find_seq(a, item);
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
    const uint32_t per_layer = 2 * pages_here;
    u.l = a.layer0 + local / per_layer;
    const uint32_t r = local % per_layer;
    u.kv = r >= pages_here ? 1u : 0u;
    const uint32_t pi = r - u.kv * pages_here;
    u.j0 = pi * a.page_size;
    const uint32_t left = u.n_c - u.j0;
    u.rows = left < a.page_size ? left : a.page_size;
    u.page = gptr<const gi32>(sq.bt)[sq.first_page + u.c * a.pages_per_chunk + pi];
    return u;
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

// Gather (kToChunk) or scatter (!kToChunk) of one tile of one page unit,
// bf16 copied bit for bit.  Grid = units * a.tiles.
template <bool kToChunk, int kBlock, int kVpt, int kAuxLoad, int kAuxStore>
__global__ __launch_bounds__(kBlock) void move_bf16(MoveArgs a)
{
    const uint32_t b = xcd_contiguous(blockIdx.x, gridDim.x);
    const uint32_t unit = b / a.tiles;
    const uint32_t tile = b - unit * a.tiles;
    const PageUnit u = locate_page_unit(a, a.item_base + unit);
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
    const uint64_t chunk_addr =
        chunk + ((uint64_t)(u.l * 2 + u.kv) * u.n_c + u.j0) * row_bytes + lo;
    if (kToChunk) copy_tile<kBlock, kVpt, kAuxLoad, kAuxStore>(page_addr, chunk_addr, n);
    else copy_tile<kBlock, kVpt, kAuxLoad, kAuxStore>(chunk_addr, page_addr, n);
}

// ------------------------------------------------------------------ fp8 e4m3

// float -> OCP E4M3 ("fn") byte, round to nearest-even, saturating at 448.
// Integer form of the rounding: in the normal range the e4m3 code is bits
// [30:20] of the binary32 pattern re-biased (exponent bias 127 -> 7), rounded
// at bit 20; below 2^-6 the value is a multiple of 2^-9, rounded with
// v_rndne_f32 after an exact scaling by 512.
__device__ __forceinline__ uint32_t e4m3_from_float(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 0x7Fu;                      // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;                     // >= 448, inf: saturate
    if (a >= 0x3C800000u) {                                        // >= 2^-6: normal
        const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        return sign | ((r >> 20) - (120u << 3));
    }
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);  // 0 .. 8
    return sign | (uint32_t)m;
}

// OCP E4M3 byte -> float (exact).
__device__ __forceinline__ float float_from_e4m3(uint32_t b)
{
    const uint32_t sign = (b & 0x80u) << 24;
    const uint32_t em = b & 0x7Fu;
    if (em == 0x7Fu) return __uint_as_float(sign | 0x7FC00000u);   // NaN
    if (em < 8u) return __uint_as_float(sign | __float_as_uint((float)em * 0.001953125f));
    return __uint_as_float(sign | ((em + (120u << 3)) << 20));
}

// float -> bf16 bits, round to nearest-even; NaN kept quiet with its sign.
__device__ __forceinline__ uint32_t bf16_from_float(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// A group unit: chunk c, layer l, K/V kv of sequence s.
struct GroupUnit {
    uint32_t c;
    uint32_t n_c;
    uint32_t l;
    uint32_t kv;
    uint32_t s;
};

__device__ __forceinline__ GroupUnit locate_group_unit(const MoveArgs& a, uint32_t item)
{
    GroupUnit g;
    g.s = find_seq(a, item);
    const SeqArg& sq = a.seq[g.s];
    const uint32_t local = item - sq.item_begin;
    g.c = local / a.units_per_chunk;                 // units_per_chunk = 2 * n_layers
    const uint32_t r = local - g.c * a.units_per_chunk;
    g.l = a.layer0 + (r >> 1);
    g.kv = r & 1u;
    g.n_c = g.c < sq.n_full ? a.chunk_size : sq.tail_tokens;
    return g;
}

template <int kBlock>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* lds)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = __shfl_xor(v, off, 64);
        v = v > o ? v : o;
    }
    const int wave = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    uint32_t m = lds[0];
#pragma unroll
    for (int w = 1; w < kBlock / 64; ++w) m = m > lds[w] ? m : lds[w];
    return m;
}

// Gather + quantise one (chunk, layer, K/V) group into e4m3 bytes + scale.
template <int kBlock>
__global__ __launch_bounds__(kBlock) void store_fp8(MoveArgs a)
{
    __shared__ uint32_t red[kBlock / 64];
    const GroupUnit g = locate_group_unit(a, a.item_base + blockIdx.x);
    const SeqArg& sq = a.seq[g.s];
    const uint64_t pool = gptr<const gu64>(g.kv ? a.v_pages : a.k_pages)[g.l];
    const uint64_t chunk = gptr<const gu64>(sq.chunks)[g.c];
    if (bad_addr(pool)) { raise_fault(kFaultPool); return; }
    if (bad_addr(chunk)) { raise_fault(kFaultChunk); return; }
    const uint32_t first = sq.first_page + g.c * a.pages_per_chunk;
    const uint32_t n_pages = (g.n_c + a.page_size - 1) / a.page_size;
    for (uint32_t pi = 0; pi < n_pages; ++pi) {
        const int64_t page = gptr<const gi32>(sq.bt)[first + pi];
        if (page < 0 || page >= a.num_pages) { raise_fault(kFaultPage); return; }
    }
    const uint32_t vrow = a.width / 8;
    const int64_t page_vecs = (int64_t)a.page_size * vrow;
    const gvec4* pool_v = reinterpret_cast<const gvec4*>(pool);

    // pass 1: absolute maximum as bf16 magnitude bits (integer order equals
    // magnitude order for non-NaN; NaN codes sort above infinity).  Plain
    // 32-bit operations: a packed-u16 form (bit_cast of a vector element into
    // a u16x2 fed to __builtin_elementwise_max) was compiled by hipcc 7.2 into
    // a load of only the first dword of each 16-byte vector.
    uint32_t m1 = 0;
    for (uint32_t pi = 0; pi < n_pages; ++pi) {
        const int64_t page = gptr<const gi32>(sq.bt)[first + pi];
        const uint32_t left = g.n_c - pi * a.page_size;
        const uint32_t nvec = (left < a.page_size ? left : a.page_size) * vrow;
        const gvec4* src = pool_v + page * page_vecs;
        for (uint32_t i = threadIdx.x; i < nvec; i += kBlock) {
            const u32x4 v = src[i];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = v[k] & 0x7FFFu;
                const uint32_t hi = (v[k] >> 16) & 0x7FFFu;
                m1 = m1 > lo ? m1 : lo;
                m1 = m1 > hi ? m1 : hi;
            }
        }
    }
    const uint32_t amax_bits = block_max_u32<kBlock>(m1, red);
    const float amax = __uint_as_float(amax_bits << 16);
    const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;

    // pass 2: quantise
    gbyte* out = reinterpret_cast<gbyte*>(chunk) + (int64_t)(g.l * 2 + g.kv) * g.n_c * a.width;
    for (uint32_t pi = 0; pi < n_pages; ++pi) {
        const int64_t page = gptr<const gi32>(sq.bt)[first + pi];
        const uint32_t left = g.n_c - pi * a.page_size;
        const uint32_t nvec = (left < a.page_size ? left : a.page_size) * vrow;
        const gvec4* src = pool_v + page * page_vecs;
        gvec2* dst = reinterpret_cast<gvec2*>(out + (int64_t)pi * a.page_size * a.width);
        for (uint32_t i = threadIdx.x; i < nvec; i += kBlock) {
            const u32x4 v = src[i];
            u32x2 q;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t b0 = e4m3_from_float(lo_bf16(v[2 * k]) / scale);
                const uint32_t b1 = e4m3_from_float(hi_bf16(v[2 * k]) / scale);
                const uint32_t b2 = e4m3_from_float(lo_bf16(v[2 * k + 1]) / scale);
                const uint32_t b3 = e4m3_from_float(hi_bf16(v[2 * k + 1]) / scale);
                q[k] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
            }
            dst[i] = q;
        }
    }
    if (threadIdx.x == 0) {
        gf32* scales = reinterpret_cast<gf32*>(reinterpret_cast<gbyte*>(chunk) +
                                               (int64_t)a.num_layers * 2 * g.n_c * a.width);
        scales[g.l * 2 + g.kv] = scale;
    }
}

// Scatter + dequantise one page unit.
template <int kBlock>
__global__ __launch_bounds__(kBlock) void retrieve_fp8(MoveArgs a)
{
    const PageUnit u = locate_page_unit(a, a.item_base + blockIdx.x);
    if (u.page < 0 || u.page >= a.num_pages) { raise_fault(kFaultPage); return; }
    const uint64_t pool = gptr<const gu64>(u.kv ? a.v_pages : a.k_pages)[u.l];
    const uint64_t chunk = gptr<const gu64>(a.seq[u.s].chunks)[u.c];
    if (bad_addr(pool)) { raise_fault(kFaultPool); return; }
    if (bad_addr(chunk)) { raise_fault(kFaultChunk); return; }
    const gbyte* cbytes = reinterpret_cast<const gbyte*>(chunk);
    const float scale = *reinterpret_cast<const gf32*>(
        cbytes + (int64_t)a.num_layers * 2 * u.n_c * a.width + (u.l * 2 + u.kv) * 4);
    const gvec2* src = reinterpret_cast<const gvec2*>(
        cbytes + ((int64_t)(u.l * 2 + u.kv) * u.n_c + u.j0) * a.width);
    gvec4* dst = reinterpret_cast<gvec4*>(pool) + u.page * (int64_t)(a.page_size * (a.width / 8));
    const uint32_t nvec = u.rows * (a.width / 8);        // 8 elements each
    for (uint32_t i = threadIdx.x; i < nvec; i += kBlock) {
        const u32x2 q = src[i];
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint32_t w = q[k];
            const uint32_t h0 = bf16_from_float(float_from_e4m3(w & 0xFFu) * scale);
            const uint32_t h1 = bf16_from_float(float_from_e4m3((w >> 8) & 0xFFu) * scale);
            const uint32_t h2 = bf16_from_float(float_from_e4m3((w >> 16) & 0xFFu) * scale);
            const uint32_t h3 = bf16_from_float(float_from_e4m3(w >> 24) * scale);
            o[2 * k] = h0 | (h1 << 16);
            o[2 * k + 1] = h2 | (h3 << 16);
        }
        dst[i] = o;
    }
}

// Plain contiguous copy (measurement aid): one tile of kBlock*kVpt vectors
// per workgroup, the same instruction form as the movers.
template <int kBlock, int kVpt>
__global__ __launch_bounds__(kBlock) void copy_contiguous(uint64_t src, uint64_t dst, int64_t nbytes)
{
    const int64_t tile = (int64_t)kBlock * kVpt * 16;
    const int64_t lo = (int64_t)blockIdx.x * tile;
    const int64_t left = nbytes - lo;
    copy_tile<kBlock, kVpt, kCpolNt, kCpolNt>(src + lo, dst + lo, (uint32_t)(left < tile ? left : tile));
}

}  // namespace kvmove
