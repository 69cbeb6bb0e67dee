// kv_cachegen.hpp -- the CacheGen quantiser fused into the movers: gather +
// quantise pages into chunk symbols, and dequantise + scatter them back.
//
// The CacheGen page ("LMCache 中的 KV Cache 压缩：CacheGen 编解码原理...",
// section "2. 量化") quantises K and V layer by layer, each layer with its own
// bin count: MAX = bins / 2 - 1; for every token row, max1 = max |x| over its
// channels; the symbol is round(x * (MAX / max1) + MAX) and max1 is kept for
// the inverse (q - MAX) / MAX * max1.  Only the quantiser: the CDF and
// arithmetic coding that follow it on that page are not part of this path.
//
// Chunk of n tokens: symbols u8 [L][2][n][H*D] (the section layout of the
// 1-byte formats), then float32 max1 [L][2][n].
//
// Work unit = page unit as in the bf16 movers (sequence, chunk, layer, K/V,
// page), a whole token row per wave.  The store and the chunk-major retrieve
// take one 256-thread workgroup per unit, wave w handling rows w, w+4, ... of
// the page (a row's maximum is one wave reduction); the pool-address-ordered
// retrieve takes one workgroup per four rows of it, one row per wave.
#pragma once

#include "kv_common.hpp"

namespace kvmove {

// threads per workgroup of the store and the chunk-major retrieve (one
// page unit each): 8 waves measured 2 % faster than 4 for the store (1 and 2
// slower, 16 much slower) and the same for the retrieve
constexpr int kCgBlock = 512;
constexpr int kCgWaves = kCgBlock / 64;
// waves (one row each) per workgroup of the pool-address-ordered retrieve
constexpr int kCgSortedWaves = 1;
constexpr int kCgMaxLayers = 128;
constexpr int kCgMaxVpl = 8;            // 16-byte vectors per lane per row: rows up to 4096 elements

// Rows a wave loads before it converts the first: as many as keep the data
// within 8 vectors of 16 bytes per lane, at most 4 (rows past the unit's end
// are skipped, so a 16-row page gives each of 8 waves 2).
template <int kVpl>
constexpr int kCgRows = kVpl <= 2 ? 4 : 8 / kVpl;

struct CgArgs {
    MoveArgs m;
    uint8_t qmax[2][kCgMaxLayers];      // MAX = bins / 2 - 1 for K (0) and V (1) of each layer
};

// Maximum of v over the wave, returned in a scalar register.  DPP moves
// (no LDS round trip): within each 16-lane row, shifts right by 1, 2, 4 and 8
// leave the row's maximum in its lane 15 (lanes shifted in from outside the
// row read 0, the identity of an unsigned maximum); row_bcast:15 and
// row_bcast:31 then carry rows 0-1 into rows 1-3 and rows 0-1 into rows 2-3,
// so lane 63 holds the maximum of all 64 lanes.
__device__ __forceinline__ uint32_t umax_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = umax_u32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));   // row_shr:1
    v = umax_u32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));   // row_shr:2
    v = umax_u32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));   // row_shr:4
    v = umax_u32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));   // row_shr:8
    v = umax_u32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
    v = umax_u32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return __builtin_amdgcn_readlane(v, 63);
}

// One symbol: x * factor and + MAX as two float32 operations, rounded half to
// even, kept in [0, 2 * MAX]; a NaN gives MAX.  (The product and the sum must
// stay two roundings: no contraction into a fused multiply-add.)
__device__ __forceinline__ uint32_t cg_symbol(float x, float factor, float qmax)
{
#pragma clang fp contract(off)
    const float scaled = x * factor;
    const float y = scaled + qmax;
    if (y != y) return (uint32_t)qmax;
    float r = __builtin_rintf(y);
    r = r < 0.0f ? 0.0f : r;
    r = r > 2.0f * qmax ? 2.0f * qmax : r;
    return (uint32_t)r;
}

// Eight bf16 values (one 16-byte vector) -> eight symbol bytes.
__device__ __forceinline__ u32x2 cg_quantise8(const u32x4 x, float factor, float qmax)
{
    u32x2 q;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t w0 = x[2 * j], w1 = x[2 * j + 1];
        q[j] = cg_symbol(__uint_as_float(w0 << 16), factor, qmax) |
               (cg_symbol(__uint_as_float(w0 & 0xFFFF0000u), factor, qmax) << 8) |
               (cg_symbol(__uint_as_float(w1 << 16), factor, qmax) << 16) |
               (cg_symbol(__uint_as_float(w1 & 0xFFFF0000u), factor, qmax) << 24);
    }
    return q;
}

// The same symbol for a row whose max1 and factor are finite.  Then
// |x| <= max1 gives |x * factor| <= MAX (1 + 2^-22) even with a subnormal
// factor, so y = x * factor + MAX lies within 2^-17 of [0, 2 * MAX] and needs
// no clamp and no NaN test (a CPU test checks the extremes x = +-max1 for every
// MAX and every finite bf16 max1).  Adding 1.5 * 2^23 rounds y half to even
// to an integer -- the sum's unit in the last place is 1 -- and leaves that
// integer in the low bits of the sum; the symbol is its low byte.
__device__ __forceinline__ uint32_t cg_symbol_bits(float x, float factor, float qmax)
{
#pragma clang fp contract(off)
    const float scaled = x * factor;
    const float y = scaled + qmax;
    return __float_as_uint(y + 12582912.0f);
}

// Low bytes of a, b, c, d -> bytes 0, 1, 2, 3 of one word (v_perm_b32 picks
// bytes of its two sources; selector 0x0c gives a zero byte).
__device__ __forceinline__ uint32_t cg_pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return __builtin_amdgcn_perm(b, a, 0x0c0c0400u) | __builtin_amdgcn_perm(d, c, 0x04000c0cu);
}

// Eight bf16 values -> eight symbol bytes on the fast path (finite max1 and
// factor).
__device__ __forceinline__ u32x2 cg_quantise8_fast(const u32x4 x, float factor, float qmax)
{
    u32x2 q;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t w0 = x[2 * j], w1 = x[2 * j + 1];
        q[j] = cg_pack_low_bytes(cg_symbol_bits(__uint_as_float(w0 << 16), factor, qmax),
                                 cg_symbol_bits(__uint_as_float(w0 & 0xFFFF0000u), factor, qmax),
                                 cg_symbol_bits(__uint_as_float(w1 << 16), factor, qmax),
                                 cg_symbol_bits(__uint_as_float(w1 & 0xFFFF0000u), factor, qmax));
    }
    return q;
}

// (q - MAX) / MAX without a division: c = q - MAX is exact; c * r with
// r = 1/MAX plus one fused multiply-add for the residual and one to correct
// (Markstein).  An exhaustive check over every MAX in [1, 63] and every
// c in [-MAX, MAX] found the IEEE quotient in every case.
__device__ __forceinline__ float cg_unit(uint32_t q, float qmax, float r)
{
    const float c = (float)q - qmax;
    const float p = c * r;
    const float e = __builtin_fmaf(-p, qmax, c);
    return __builtin_fmaf(e, r, p);
}

// Two dequantised values -> two bf16 in one word.  In a row whose max1 is
// NaN or infinite (`special`, the same for the whole wave) a value can be NaN
// (NaN * x, 0 * inf); it is written as the quiet NaN 0x7FC0, whatever sign
// and payload the product had.  A finite max1 gives finite values only.
__device__ __forceinline__ uint32_t cg_pair(float a, float b, bool special)
{
    uint32_t o = bf16x2_rne(a, b);
    if (special) {
        if (a != a) o = (o & 0xFFFF0000u) | 0x7FC0u;
        if (b != b) o = (o & 0x0000FFFFu) | 0x7FC00000u;
    }
    return o;
}

__device__ __forceinline__ bool cg_special(float max1) { return !(__builtin_fabsf(max1) < __builtin_inff()); }

// Dequantise one row's kVpl vectors of 8 symbols and store them as bf16;
// kSpecial as cg_pair's `special`.
template <int kVpl, bool kSpecial>
__device__ __forceinline__ void cg_dequantise_row(const u32x2 (&q)[kVpl], float qmax, float rq, float max1,
                                                  __amdgpu_buffer_rsrc_t rd, uint32_t lane, int aux)
{
#pragma unroll
    for (int k = 0; k < kVpl; ++k) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t w = q[k][j];
            o[2 * j] = cg_pair(cg_unit(w & 0xFFu, qmax, rq) * max1, cg_unit((w >> 8) & 0xFFu, qmax, rq) * max1,
                               kSpecial);
            o[2 * j + 1] = cg_pair(cg_unit((w >> 16) & 0xFFu, qmax, rq) * max1, cg_unit(w >> 24, qmax, rq) * max1,
                                   kSpecial);
        }
        if (aux == (kCpolNt | kCpolSc1))
            __builtin_amdgcn_raw_buffer_store_b128(o, rd, (k * 64 + lane) * 16, 0, kCpolNt | kCpolSc1);
        else
            __builtin_amdgcn_raw_buffer_store_b128(o, rd, (k * 64 + lane) * 16, 0, kCpolNt);
    }
}

// Byte offset of the max1 of row j0 + row of (l, kv) in a chunk of n_c tokens.
__device__ __forceinline__ uint64_t cg_max_offset(const MoveArgs& a, uint32_t l, uint32_t kv, uint32_t n_c,
                                                  uint32_t row)
{
    return (uint64_t)a.num_layers * 2 * n_c * a.width + ((uint64_t)(l * 2 + kv) * n_c + row) * 4;
}

template <int kVpl>
__global__ __launch_bounds__(kCgBlock) void store_cachegen(CgArgs ca)
{
    const MoveArgs& a = ca.m;
    const PageUnit u = locate_page_unit(a, a.item_base + xcd_contiguous(blockIdx.x, gridDim.x));
    if (u.page < 0 || u.page >= a.num_pages) { raise_fault(kFaultPage); return; }
    const uint64_t pool = wave_uniform(gptr<const gu64>(u.kv ? a.v_pages : a.k_pages)[u.l]);
    const uint64_t chunk = wave_uniform(gptr<const gu64>(a.seq[u.s].chunks)[u.c]);
    if (bad_addr(pool)) { raise_fault(kFaultPool); return; }
    if (bad_addr(chunk)) { raise_fault(kFaultChunk); return; }
    const float qmax = (float)ca.qmax[u.kv][u.l];
    const uint32_t E = a.width, row_bytes = E * 2;
    // the wave index in a scalar register: row addresses, and the buffer
    // descriptors built from them, are then known to be wave-uniform
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
    const uint64_t page_rows = pool + (uint64_t)u.page * a.page_size * row_bytes;
    const uint64_t sym_rows = chunk + section_offset(a, u.l, u.kv, u.n_c) + (uint64_t)u.j0 * E;
    // kCgRows<kVpl> rows per wave in flight: every load of the batch is
    // issued before the first row is reduced.  A row past the unit's end
    // gets an empty range (loads return zero, nothing is touched).
    constexpr int kRows = kCgRows<kVpl>;
    // streaming policy with sc1 on the loads and the stores, as the movers
    // use (0.9 % faster than nt alone at the Llama-3.1-8B shape)
    constexpr int kAux = kCpolNt | kCpolSc1;
    for (uint32_t r0 = wave; r0 < u.rows; r0 += kCgWaves * kRows) {
        u32x4 v[kRows][kVpl];
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const uint32_t r = r0 + i * kCgWaves;
            // vectors past the row read as zero (range check), neutral for the maximum
            const __amdgpu_buffer_rsrc_t rs = byte_range(page_rows + (uint64_t)r * row_bytes, r < u.rows ? row_bytes : 0);
#pragma unroll
            for (int k = 0; k < kVpl; ++k)
                v[i][k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (k * 64 + lane) * 16, 0, kAux);
        }
        // the rows' maxima first, so that their cross-lane reductions overlap
        // (a row past the unit's end read zeros and is not used)
        uint32_t mrow[kRows];
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            uint32_t m2 = 0;
#pragma unroll
            for (int k = 0; k < kVpl; ++k) m2 = max_magnitude2(m2, v[i][k]);
            mrow[i] = wave_max_u32(pair_max(m2));
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const uint32_t r = r0 + i * kCgWaves;
            if (r >= u.rows) break;                       // the same for the whole wave
            const uint32_t m = mrow[i];
            // NaN magnitudes sort above infinity; any NaN makes max1 the quiet NaN
            const float max1 = m > 0x7F80u ? __uint_as_float(0x7FC00000u) : __uint_as_float(m << 16);
            const float factor = max1 == 0.0f ? 0.0f : qmax / max1;
            const bool fast = m < 0x7F80u && (__float_as_uint(factor) & 0x7F800000u) != 0x7F800000u;
            const __amdgpu_buffer_rsrc_t rd = byte_range(sym_rows + (uint64_t)r * E, E);
            if (fast) {                                   // the same for the whole wave
#pragma unroll
                for (int k = 0; k < kVpl; ++k)
                    __builtin_amdgcn_raw_buffer_store_b64(cg_quantise8_fast(v[i][k], factor, qmax), rd,
                                                          (k * 64 + lane) * 8, 0, kAux);
            } else {
#pragma unroll
                for (int k = 0; k < kVpl; ++k)
                    __builtin_amdgcn_raw_buffer_store_b64(cg_quantise8(v[i][k], factor, qmax), rd,
                                                          (k * 64 + lane) * 8, 0, kAux);
            }
            if (lane == 0) *gptr<gf32>(chunk + cg_max_offset(a, u.l, u.kv, u.n_c, u.j0 + r)) = max1;
        }
    }
}

// Dequantise + scatter a whole page unit with one workgroup, kCgRows<kVpl>
// rows per wave in flight (the chunk-major retrieve).
template <int kVpl>
__device__ __forceinline__ void retrieve_cachegen_unit(const CgArgs& ca, const PageUnit& u)
{
    const MoveArgs& a = ca.m;
    if (u.page < 0 || u.page >= a.num_pages) { raise_fault(kFaultPage); return; }
    const uint64_t pool = wave_uniform(gptr<const gu64>(u.kv ? a.v_pages : a.k_pages)[u.l]);
    const uint64_t chunk = wave_uniform(gptr<const gu64>(a.seq[u.s].chunks)[u.c]);
    if (bad_addr(pool)) { raise_fault(kFaultPool); return; }
    if (bad_addr(chunk)) { raise_fault(kFaultChunk); return; }
    const float qmax = (float)ca.qmax[u.kv][u.l];
    const float rq = 1.0f / qmax;
    const uint32_t E = a.width, row_bytes = E * 2;
    // the wave index in a scalar register: row addresses, and the buffer
    // descriptors built from them, are then known to be wave-uniform
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
    const uint64_t page_rows = pool + (uint64_t)u.page * a.page_size * row_bytes;
    const uint64_t sym_rows = chunk + section_offset(a, u.l, u.kv, u.n_c) + (uint64_t)u.j0 * E;
    // kCgRows<kVpl> rows per wave in flight, as in the store; a row past the
    // unit's end reads nothing (empty range, max1 not loaded).
    constexpr int kRows = kCgRows<kVpl>;
    for (uint32_t r0 = wave; r0 < u.rows; r0 += kCgWaves * kRows) {
        u32x2 q[kRows][kVpl];
        float max1[kRows];
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const uint32_t r = r0 + i * kCgWaves;
            max1[i] = r < u.rows ? *gptr<const gf32>(chunk + cg_max_offset(a, u.l, u.kv, u.n_c, u.j0 + r)) : 0.0f;
            const __amdgpu_buffer_rsrc_t rs = byte_range(sym_rows + (uint64_t)r * E, r < u.rows ? E : 0);
#pragma unroll
            for (int k = 0; k < kVpl; ++k)
                q[i][k] = __builtin_amdgcn_raw_buffer_load_b64(rs, (k * 64 + lane) * 8, 0, kCpolNt);
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const uint32_t r = r0 + i * kCgWaves;
            if (r >= u.rows) break;                       // the same for the whole wave
            const __amdgpu_buffer_rsrc_t rd = byte_range(page_rows + (uint64_t)r * row_bytes, row_bytes);
            if (cg_special(max1[i]))                      // the same for the whole wave
                cg_dequantise_row<kVpl, true>(q[i], qmax, rq, max1[i], rd, lane, kCpolNt);
            else
                cg_dequantise_row<kVpl, false>(q[i], qmax, rq, max1[i], rd, lane, kCpolNt);
        }
    }
}

// Dequantise + scatter tile `tile` of a page unit: kCgSortedWaves rows, one
// per wave (rows tile * kCgSortedWaves + wave); a.tiles = ceil(page rows /
// kCgSortedWaves) tiles per unit, one workgroup each (the pool-address-ordered
// retrieve).  In pool-address order these smaller workgroups measured 5.56
// TB/s (4 waves) against 5.39 for one workgroup per page at the Llama-3.1-8B
// shape, and one wave per workgroup 0.5 % faster again than 4 (2 and 8 were
// slower); in chunk-major order they measured slower (5.08 against 5.33), so
// that order keeps retrieve_cachegen_unit.  nt + sc1 on both sides (+0.8 %
// here; -0.4 % in the chunk-major kernel, which keeps nt).
template <int kVpl>
__device__ __forceinline__ void retrieve_cachegen_tile(const CgArgs& ca, const PageUnit& u, uint32_t tile)
{
    const MoveArgs& a = ca.m;
    // the wave index in a scalar register: row addresses, and the buffer
    // descriptors built from them, are then known to be wave-uniform
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
    const uint32_t r = tile * kCgSortedWaves + wave;
    if (tile * kCgSortedWaves >= u.rows) return;                // tile past a short (tail) page: whole workgroup
    if (u.page < 0 || u.page >= a.num_pages) { raise_fault(kFaultPage); return; }
    const uint64_t pool = wave_uniform(gptr<const gu64>(u.kv ? a.v_pages : a.k_pages)[u.l]);
    const uint64_t chunk = wave_uniform(gptr<const gu64>(a.seq[u.s].chunks)[u.c]);
    if (bad_addr(pool)) { raise_fault(kFaultPool); return; }
    if (bad_addr(chunk)) { raise_fault(kFaultChunk); return; }
    if (r >= u.rows) return;                              // this wave's row is past the unit's end
    const float qmax = (float)ca.qmax[u.kv][u.l];
    const float rq = 1.0f / qmax;
    const uint32_t E = a.width, row_bytes = E * 2;
    const float max1 = *gptr<const gf32>(chunk + cg_max_offset(a, u.l, u.kv, u.n_c, u.j0 + r));
    const __amdgpu_buffer_rsrc_t rs =
        byte_range(chunk + section_offset(a, u.l, u.kv, u.n_c) + (uint64_t)(u.j0 + r) * E, E);
    const __amdgpu_buffer_rsrc_t rd =
        byte_range(pool + ((uint64_t)u.page * a.page_size + r) * row_bytes, row_bytes);
    u32x2 q[kVpl];
#pragma unroll
    for (int k = 0; k < kVpl; ++k)
        q[k] = __builtin_amdgcn_raw_buffer_load_b64(rs, (k * 64 + lane) * 8, 0, kCpolNt | kCpolSc1);
    if (cg_special(max1))                                 // the same for the whole wave
        cg_dequantise_row<kVpl, true>(q, qmax, rq, max1, rd, lane, kCpolNt | kCpolSc1);
    else
        cg_dequantise_row<kVpl, false>(q, qmax, rq, max1, rd, lane, kCpolNt | kCpolSc1);
}

template <int kVpl>
__global__ __launch_bounds__(kCgBlock) void retrieve_cachegen(CgArgs ca)
{
    retrieve_cachegen_unit<kVpl>(ca, locate_page_unit(ca.m, ca.m.item_base + xcd_contiguous(blockIdx.x, gridDim.x)));
}

// The same in pool-address order (sorted page list, see sorted_unit).
template <int kVpl>
__global__ __launch_bounds__(kCgSortedWaves * 64) void retrieve_cachegen_sorted(CgArgs ca, uint64_t list, uint32_t n_list)
{
    const uint32_t b = xcd_contiguous(blockIdx.x, gridDim.x);
    const uint32_t unit = b / ca.m.tiles, tile = b - unit * ca.m.tiles;
    PageUnit u;
    if (!sorted_unit(ca.m, list, n_list, unit, u)) return;
    retrieve_cachegen_tile<kVpl>(ca, u, tile);
}

}  // namespace kvmove
