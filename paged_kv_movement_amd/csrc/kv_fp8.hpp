// kv_fp8.hpp -- fused fp8 serde movers: gather + quantise to OCP E4M3 with
// one float32 absmax scale per (chunk, layer, K/V) group, and scatter +
// dequantise.  The serde framework page ("LMCache 分布式 KV Cache 序列化框架
// Serde...", section "7.1 fp8 量化") casts every element to e4m3, one byte
// per element; the per-group scale is this library's addition.
#pragma once

#include "kv_common.hpp"

namespace kvmove {

constexpr int kFp8Block = 256;

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

}  // namespace kvmove
