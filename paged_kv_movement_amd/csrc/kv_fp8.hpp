// kv_fp8.hpp -- fused fp8 serde movers: gather + quantise to OCP E4M3 or
// E5M2 with one float32 absmax scale per (chunk, layer, K/V) group, and
// scatter + dequantise.  The serde framework page ("LMCache 分布式 KV Cache
// 序列化框架 Serde...", section "7.1 fp8 量化") casts every element to e4m3
// (default) or e5m2, one byte per element; the per-group scale is this
// library's addition.  kE5M2 selects the encoding throughout.
#pragma once

#include "kv_common.hpp"

namespace kvmove {

constexpr int kFp8StoreBlock = 512;     // two-pass store: threads per (chunk, layer, K/V) group
constexpr int kFp8StoreUnroll = 4;     // two-pass store: 16-byte loads in flight per thread
// single-pass store: the whole group on chip, 1024 threads x (26 vectors in
// VGPRs + 6 vectors in LDS) = 32768 16-byte vectors = 512 KiB, one
// (256-token chunk, layer, K/V) group at the Llama-3.1-8B shape.
constexpr int kOnchipBlock = 1024;
constexpr int kOnchipRegSlots = 26;
constexpr int kOnchipLdsSlots = 6;
constexpr int kOnchipMaxPages = 64;
constexpr uint32_t kOnchipMaxVectors = uint32_t(kOnchipBlock) * (kOnchipRegSlots + kOnchipLdsSlots);
// dequantising scatter: one-wave workgroups with 4 KiB tiles of bf16 output
// for a full chunk-major launch (about 1 % faster than 8 KiB tiles of 256
// threads); one-wave 2 KiB tiles for the pool-address-ordered launch (0.4-0.8 %
// faster than 256 x 8 KiB there, while 4 KiB one-wave tiles were 2 % slower);
// 256 threads x 8 KiB for a capped launch
constexpr int kFp8RetrieveBlock = 64;
constexpr int kFp8RetrieveVpt = 4;
constexpr int kFp8RetrieveBlockSorted = 64;
constexpr int kFp8RetrieveVptSorted = 2;
constexpr int kFp8RetrieveBlockCapped = 256;
constexpr int kFp8RetrieveVptCapped = 2;

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

// float -> OCP E5M2 byte, round to nearest-even, saturating at 57344 (also
// for infinity).  Normal range: bits [30:21] of the binary32 pattern
// re-biased (exponent bias 127 -> 15), rounded at bit 21; below 2^-14 the
// value is a multiple of 2^-16, rounded with v_rndne_f32 after an exact
// scaling by 65536.
__device__ __forceinline__ uint32_t e5m2_from_float(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 0x7Fu;                      // NaN
    if (a >= 0x47600000u) return sign | 0x7Bu;                     // >= 57344, inf: saturate
    if (a >= 0x38800000u) {                                        // >= 2^-14: normal
        const uint32_t r = a + 0xFFFFFu + ((a >> 21) & 1u);
        return sign | ((r >> 21) - (112u << 2));
    }
    const float m = __builtin_rintf(__uint_as_float(a) * 65536.0f);  // 0 .. 4
    return sign | (uint32_t)m;
}

// Largest finite value of the encoding: the group maximum maps onto it.
template <bool kE5M2>
__device__ __forceinline__ float fp8_max() { return kE5M2 ? 57344.0f : 448.0f; }

template <bool kE5M2>
__device__ __forceinline__ uint32_t fp8_from_float(float y) { return kE5M2 ? e5m2_from_float(y) : e4m3_from_float(y); }

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

// The order of a sequence's group units.  With K and V in one launch it is
// chunk-major, (chunk, layer, K/V): neighbouring workgroups then write
// neighbouring 256 KiB sections of one chunk (chunk-fastest measured 5 %
// slower).  A launch of one part (K16/V8's V) has no neighbouring sections
// to write -- its sections of one chunk lie a K section apart -- and takes
// the chunk fastest, (layer, chunk): 2 % faster for that launch.
__device__ __forceinline__ GroupUnit locate_group_unit(const MoveArgs& a, uint32_t item, uint32_t seq)
{
    GroupUnit g;
    g.s = seq;
    const SeqArg& sq = a.seq[g.s];
    const uint32_t local = item - sq.item_begin;
    uint32_t r;                                      // layer (and part) index in [0, units_per_chunk)
    if (a.n_kv == 2) {
        g.c = local / a.units_per_chunk;             // units_per_chunk = n_kv * n_layers
        r = local - g.c * a.units_per_chunk;
    } else {
        const uint32_t n_chunks = sq.n_full + (sq.tail_tokens > 0 ? 1u : 0u);
        r = local / n_chunks;
        g.c = local - r * n_chunks;
    }
    g.l = a.layer0 + (a.n_kv == 2 ? r >> 1 : r);
    g.kv = a.kv0 + (a.n_kv == 2 ? r & 1u : 0u);
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

// Quotient x / s for the fp8 encoder without a division: q0 = x * r with
// r = 1/s correctly rounded, one fused multiply-add for the exact residual
// (taken negated, q0*s - x), one to correct q0 (Markstein's correction).  The
// result is the correctly rounded quotient except for some |x| <= 2^-25; for
// groups whose amax is a finite bf16 value >= 2^-4 an exhaustive check over
// every (amax, x) bf16 pair showed the e4m3 code, and the e5m2 code, always
// equal those of the IEEE quotient, the sign of zero included (the negated
// residual makes a zero quotient keep the sign of x).
__device__ __forceinline__ float quotient_fast(float x, float s, float r)
{
    const float q0 = x * r;
    const float e = __builtin_fmaf(q0, s, -x);
    return __builtin_fmaf(-e, r, q0);
}

// Four floats -> four fp8 bytes (a, b, c, d from the low byte up) with the
// hardware converter, which rounds to nearest-even and matches the OCP
// encoding for |y| <= 464 (E4M3) and |y| < 59392 (E5M2; above, it overflows
// to infinity instead of saturating) -- checked against the CPU oracle on
// every float32 in those ranges.  The quotients fed to it stay within the
// scale's target maximum (448, 57344) plus a few units in the last place.
// The second conversion writes the upper half-word of the first's result;
// the pair was checked the same way, byte by byte, for both encodings.
template <bool kE5M2>
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d)
{
    if (kE5M2) {
        const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, d, lo, true);
    }
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// amax bits (bf16 magnitude) for which the fast quotient is exact in e4m3
__device__ __forceinline__ bool fast_quotient_ok(uint32_t amax_bits)
{
    return amax_bits >= 0x3D80u && amax_bits < 0x7F80u;     // [2^-4, largest finite]
}

// Code of one bf16 element (its 16 bits in h) on the slow path: IEEE
// division and the integer encoder.  A NaN quotient -- the group holds a NaN,
// or the element and the scale are both infinite -- encodes as 0x7F with the
// element's own sign bit (the sign a division gives a NaN is not fixed by
// IEEE 754; taking the element's makes the code deterministic).
template <bool kE5M2>
__device__ __forceinline__ uint32_t slow_code(uint32_t h, float scale)
{
    const float y = __uint_as_float(h << 16) / scale;
    return y != y ? (((h >> 8) & 0x80u) | 0x7Fu) : fp8_from_float<kE5M2>(y);
}

// Eight bf16 values (one 16-byte vector) -> eight fp8 bytes.  `fast`
// selects the division-free quotient (exact in both encodings for the
// group's amax, see quotient_fast); otherwise IEEE division and the integer
// encoder.
template <bool kE5M2>
__device__ __forceinline__ u32x2 quantize8(const u32x4 x, float scale, float r, bool fast)
{
    u32x2 q;
    if (fast) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t w0 = x[2 * j], w1 = x[2 * j + 1];
            q[j] = fp8x4<kE5M2>(quotient_fast(lo_bf16(w0), scale, r), quotient_fast(hi_bf16(w0), scale, r),
                                quotient_fast(lo_bf16(w1), scale, r), quotient_fast(hi_bf16(w1), scale, r));
        }
    } else {   // tiny, infinite or NaN amax
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t w0 = x[2 * j], w1 = x[2 * j + 1];
            q[j] = slow_code<kE5M2>(w0 & 0xFFFFu, scale) | (slow_code<kE5M2>(w0 >> 16, scale) << 8) |
                   (slow_code<kE5M2>(w1 & 0xFFFFu, scale) << 16) | (slow_code<kE5M2>(w1 >> 16, scale) << 24);
        }
    }
    return q;
}

// The scale of a group from its maximum (bf16 magnitude bits): amax / fmax,
// 1 for an all-zero group, and the default quiet NaN 0x7FC00000 when the
// group holds a NaN (NaN magnitudes sort above infinity).
template <bool kE5M2>
__device__ __forceinline__ float group_scale(uint32_t amax_bits)
{
    const float amax = __uint_as_float(amax_bits << 16);
    if (amax_bits > 0x7F80u) return __uint_as_float(0x7FC00000u);
    return amax == 0.0f ? 1.0f : amax / fp8_max<kE5M2>();
}

// Address of 16-byte vector v of a group (token-major) whose pool pages are
// listed in `pages`, page_vecs vectors per page.  (A plain function: a
// lambda returning this address-space-qualified pointer inside a template
// kernel made hipcc 7.2 drop the kernel's host-side launch stub.)
__device__ __forceinline__ const gvec4* group_vector(uint64_t pool, const int32_t* pages, uint32_t page_vecs,
                                                     uint64_t page_bytes, uint32_t v)
{
    const uint32_t pi = v / page_vecs;
    return reinterpret_cast<const gvec4*>(pool + (uint64_t)pages[pi] * page_bytes) + (v - pi * page_vecs);
}

// Single-pass gather + quantise of one (chunk, layer, K/V) group that fits
// on chip (at most kOnchipMaxVectors 16-byte vectors, kOnchipMaxPages
// pages): every vector is read from HBM once -- kOnchipRegSlots per thread
// into VGPRs, kOnchipLdsSlots per thread straight into LDS -- the group
// maximum is reduced, and the quantised bytes are written from the chip.
// One workgroup per group; vector v of the group (token-major, 8 elements)
// is held by thread v % 1024 in slot v / 1024.
template <bool kE5M2>
__global__ __launch_bounds__(kOnchipBlock) void store_fp8_onchip(MoveArgsLut al)
{
    const MoveArgs& a = al.m;
    constexpr int B = kOnchipBlock;
    __shared__ u32x4 lds[kOnchipLdsSlots * B];
    __shared__ uint32_t red[B / 64];
    __shared__ int32_t pages[kOnchipMaxPages];
    const uint32_t item = a.item_base + xcd_contiguous(blockIdx.x, gridDim.x);
    const GroupUnit g = locate_group_unit(a, item, find_seq_lut(al, item));
    const SeqArg& sq = a.seq[g.s];
    const uint64_t pool = wave_uniform(gptr<const gu64>(g.kv ? a.v_pages : a.k_pages)[g.l]);
    const uint64_t chunk = wave_uniform(gptr<const gu64>(sq.chunks)[g.c]);
    if (bad_addr(pool)) { raise_fault(kFaultPool); return; }
    if (bad_addr(chunk)) { raise_fault(kFaultChunk); return; }
    const uint32_t first = sq.first_page + g.c * a.pages_per_chunk;
    const uint32_t n_pages = (g.n_c + a.page_size - 1) / a.page_size;
    const uint32_t page_vecs = a.page_size * (a.width / 8);
    // The groups of one chunk's layers and parts, which run side by side,
    // read the same page ids in different layers' pools.  A full group whose
    // pages hold whole slots visits its pages rotated by spin = (2 l + kv)
    // mod n_pages, so that they start on different pages (0.2-0.8 % faster):
    // pages[] lists them rotated, and slot k's codes go to slot
    // (k + spin * slots per page) mod n_slots of the output.
    const uint32_t spin = (g.n_c == a.chunk_size && page_vecs % B == 0) ? (g.l * 2 + g.kv) % n_pages : 0u;
    if (threadIdx.x < n_pages) {
        uint32_t t = threadIdx.x + spin;
        if (t >= n_pages) t -= n_pages;
        pages[threadIdx.x] = gptr<const gi32>(sq.bt)[first + t];
    }
    __syncthreads();
    for (uint32_t pi = 0; pi < n_pages; ++pi) {       // same verdict in every thread
        if (pages[pi] < 0 || pages[pi] >= a.num_pages) { raise_fault(kFaultPage); return; }
    }
    const uint64_t page_bytes = (uint64_t)page_vecs * 16;
    const uint32_t total = g.n_c * (a.width / 8);
    const uint32_t n_slots = (total + B - 1) / B;
    const uint32_t slot_shift = spin * (page_vecs / B);   // 0 unless spun: then total = n_slots * B
    const uint32_t wave = threadIdx.x / 64;

    // LDS slots: direct-to-LDS loads (each lane's 16 bytes land at
    // base + lane * 16, base uniform per wave), streaming like the register
    // slots' loads (nt + sc1: 0.3-0.5 % faster than the default policy)
#pragma unroll
    for (int k = 0; k < kOnchipLdsSlots; ++k) {
        const uint32_t v = (kOnchipRegSlots + k) * B + threadIdx.x;
        if (v < total)
            __builtin_amdgcn_global_load_lds(group_vector(pool, pages, page_vecs, page_bytes, v),
                                             (__attribute__((address_space(3))) void*)&lds[k * B + wave * 64],
                                             16, 0, kCpolNt | kCpolSc1);
    }
    u32x4 reg[kOnchipRegSlots];
#pragma unroll
    for (int k = 0; k < kOnchipRegSlots; ++k) {
        const uint32_t v = k * B + threadIdx.x;
        reg[k] = u32x4{0u, 0u, 0u, 0u};                   // zero is neutral for the maximum
        if (v < total) reg[k] = __builtin_nontemporal_load(group_vector(pool, pages, page_vecs, page_bytes, v));
    }
    uint32_t m2 = 0;
#pragma unroll
    for (int k = 0; k < kOnchipRegSlots; ++k) m2 = max_magnitude2(m2, reg[k]);
    __builtin_amdgcn_s_waitcnt(0);                        // the LDS loads have landed
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kOnchipLdsSlots; ++k) {
        const uint32_t v = (kOnchipRegSlots + k) * B + threadIdx.x;
        if (v < total) m2 = max_magnitude2(m2, lds[k * B + threadIdx.x]);
    }
    const uint32_t amax_bits = block_max_u32<B>(pair_max(m2), red);
    const float scale = group_scale<kE5M2>(amax_bits);
    const bool fast = fast_quotient_ok(amax_bits);
    const float r = 1.0f / scale;

    gvec2* dst = reinterpret_cast<gvec2*>(chunk + section_offset(a, g.l, g.kv, g.n_c));
    // output slot of slot k (k < n_slots, as v < total below); k itself unless spun
    auto out_slot = [&](uint32_t k) {
        const uint32_t o = k + slot_shift;
        return o >= n_slots ? o - n_slots : o;
    };
#pragma unroll
    for (int k = 0; k < kOnchipRegSlots; ++k) {
        const uint32_t v = k * B + threadIdx.x;
        if (v < total)
            __builtin_nontemporal_store(quantize8<kE5M2>(reg[k], scale, r, fast), dst + out_slot(k) * B + threadIdx.x);
    }
#pragma unroll
    for (int k = 0; k < kOnchipLdsSlots; ++k) {
        const uint32_t v = (kOnchipRegSlots + k) * B + threadIdx.x;
        if (v < total)
            __builtin_nontemporal_store(quantize8<kE5M2>(lds[k * B + threadIdx.x], scale, r, fast),
                                        dst + out_slot(kOnchipRegSlots + k) * B + threadIdx.x);
    }
    if (threadIdx.x == 0) *gptr<gf32>(chunk + scale_offset(a, g.l, g.kv, g.n_c)) = scale;
}

// Gather + quantise one (chunk, layer, K/V) group of any size into fp8
// bytes + scale, in two passes: pass 1 reads the group's pages and takes
// max |x|; pass 2 re-reads them (streaming), quantises, and writes 8 bytes
// per 16-byte input vector.  Used for groups too large for store_fp8_onchip.
template <int kBlock, int kUnroll, bool kE5M2>
__global__ __launch_bounds__(kBlock) void store_fp8(MoveArgsLut al)
{
    const MoveArgs& a = al.m;
    __shared__ uint32_t red[kBlock / 64];
    const uint32_t item = a.item_base + xcd_contiguous(blockIdx.x, gridDim.x);
    const GroupUnit g = locate_group_unit(a, item, find_seq_lut(al, item));
    const SeqArg& sq = a.seq[g.s];
    const uint64_t pool = wave_uniform(gptr<const gu64>(g.kv ? a.v_pages : a.k_pages)[g.l]);
    const uint64_t chunk = wave_uniform(gptr<const gu64>(sq.chunks)[g.c]);
    if (bad_addr(pool)) { raise_fault(kFaultPool); return; }
    if (bad_addr(chunk)) { raise_fault(kFaultChunk); return; }
    const uint32_t first = sq.first_page + g.c * a.pages_per_chunk;
    const uint32_t n_pages = (g.n_c + a.page_size - 1) / a.page_size;
    for (uint32_t pi = 0; pi < n_pages; ++pi) {
        const int64_t page = gptr<const gi32>(sq.bt)[first + pi];
        if (page < 0 || page >= a.num_pages) { raise_fault(kFaultPage); return; }
    }
    const uint32_t page_bytes = a.page_size * a.width * 2;
    constexpr uint32_t kStep = kBlock * kUnroll * 16;

    // pass 1: absolute maximum as bf16 magnitude bits.  (A packed-u16 form
    // written with __builtin_elementwise_max on a bit_cast u16x2 was compiled
    // by hipcc 7.2 into a load of only the first dword of each 16-byte
    // vector; max_magnitude2 states the instruction directly.)
    uint32_t m2 = 0;
    for (uint32_t pi = 0; pi < n_pages; ++pi) {
        const int64_t page = gptr<const gi32>(sq.bt)[first + pi];
        const uint32_t left = g.n_c - pi * a.page_size;
        const uint32_t nb = (left < a.page_size ? left : a.page_size) * a.width * 2;
        const __amdgpu_buffer_rsrc_t rs = byte_range(pool + (uint64_t)page * page_bytes, nb);
        for (uint32_t base = 0; base < nb; base += kStep) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int k = 0; k < kUnroll; ++k)
                v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + (k * kBlock + threadIdx.x) * 16, 0, 0);
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) m2 = max_magnitude2(m2, v[k]);
        }
    }
    const uint32_t amax_bits = block_max_u32<kBlock>(pair_max(m2), red);
    const float scale = group_scale<kE5M2>(amax_bits);
    const bool fast = fast_quotient_ok(amax_bits);
    const float r = 1.0f / scale;

    // pass 2: quantise
    const uint64_t out = chunk + section_offset(a, g.l, g.kv, g.n_c);
    for (uint32_t pi = 0; pi < n_pages; ++pi) {
        const int64_t page = gptr<const gi32>(sq.bt)[first + pi];
        const uint32_t left = g.n_c - pi * a.page_size;
        const uint32_t nb = (left < a.page_size ? left : a.page_size) * a.width * 2;
        const __amdgpu_buffer_rsrc_t rs = byte_range(pool + (uint64_t)page * page_bytes, nb);
        const __amdgpu_buffer_rsrc_t rd = byte_range(out + (uint64_t)pi * a.page_size * a.width, nb / 2);
        for (uint32_t base = 0; base < nb; base += kStep) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int k = 0; k < kUnroll; ++k)
                v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + (k * kBlock + threadIdx.x) * 16, 0,
                                                            kCpolNt);
#pragma unroll
            for (int k = 0; k < kUnroll; ++k)
                __builtin_amdgcn_raw_buffer_store_b64(quantize8<kE5M2>(v[k], scale, r, fast), rd,
                                                      base / 2 + (k * kBlock + threadIdx.x) * 8, 0, kCpolNt);
        }
    }
    if (threadIdx.x == 0) *gptr<gf32>(chunk + scale_offset(a, g.l, g.kv, g.n_c)) = scale;
}

// Two bf16 results packed in o (from the products p0, p1 of the fp8 codes
// in bytes 0 and 1 of c): a NaN product becomes the quiet NaN 0x7FC0 with
// its code's sign.
__device__ __forceinline__ uint32_t nan_fix2(uint32_t o, float p0, float p1, uint32_t c)
{
    if (p0 != p0) o = (o & 0xFFFF0000u) | 0x7FC0u | ((c & 0x80u) << 8);
    if (p1 != p1) o = (o & 0x0000FFFFu) | 0x7FC00000u | ((c & 0x8000u) << 16);
    return o;
}

// Bit 7 of each byte of the result is set where that byte of w is an fp8
// NaN code: S.1111.111 (E4M3), S.11111.01 / .10 / .11 (E5M2) -- the low seven
// bits at or above 0x7F / 0x7D; adding 1 / 3 to them carries into bit 7
// there and nowhere else.
template <bool kE5M2>
__device__ __forceinline__ uint32_t nan_code_bits(uint32_t w)
{
    return ((w & 0x7F7F7F7Fu) + (kE5M2 ? 0x03030303u : 0x01010101u)) & 0x80808080u;
}

// The bf16 results of the four codes in c (bytes 0, 1 in lo; 2, 3 in hi) where
// a code is NaN: the quiet NaN 0x7FC0 with the code's sign.
template <bool kE5M2>
__device__ __forceinline__ void fix_nan_codes(uint32_t& lo, uint32_t& hi, uint32_t c)
{
    const uint32_t m = nan_code_bits<kE5M2>(c);
    if (m & 0x80u) lo = (lo & 0xFFFF0000u) | 0x7FC0u | ((c & 0x80u) << 8);
    if (m & 0x8000u) lo = (lo & 0x0000FFFFu) | 0x7FC00000u | ((c & 0x8000u) << 16);
    if (m & 0x800000u) hi = (hi & 0xFFFF0000u) | 0x7FC0u | ((c >> 8) & 0x8000u);
    if (m & 0x80000000u) hi = (hi & 0x0000FFFFu) | 0x7FC00000u | (c & 0x80000000u);
}

// How dequantise_store treats NaN results: kNanPlain leaves them to the
// hardware (for finite, nonzero scales and no NaN code, none arise);
// kNanByProduct writes every NaN product as the quiet NaN with its code's
// sign (any scale); kNanByCode does that for the NaN codes (finite, nonzero
// scales, where only a NaN code gives a NaN product).
enum NanMode { kNanPlain, kNanByProduct, kNanByCode };

// Decode kVpt x 8 fp8 codes, scale them, round to bf16 and store them
// (kBlock*kVpt 16-byte vectors per tile).
template <int kBlock, int kVpt, bool kE5M2, NanMode kNan>
__device__ __forceinline__ void dequantise_store(const u32x2 (&q)[kVpt], float scale, __amdgpu_buffer_rsrc_t rd)
{
#pragma unroll
    for (int k = 0; k < kVpt; ++k) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const auto d0 = kE5M2 ? __builtin_amdgcn_cvt_pk_f32_bf8(q[k][j], false)    // bytes 0, 1
                                  : __builtin_amdgcn_cvt_pk_f32_fp8(q[k][j], false);
            const auto d1 = kE5M2 ? __builtin_amdgcn_cvt_pk_f32_bf8(q[k][j], true)     // bytes 2, 3
                                  : __builtin_amdgcn_cvt_pk_f32_fp8(q[k][j], true);
            o[2 * j] = bf16x2_rne(d0[0] * scale, d0[1] * scale);
            o[2 * j + 1] = bf16x2_rne(d1[0] * scale, d1[1] * scale);
            if (kNan == kNanByProduct) {
                o[2 * j] = nan_fix2(o[2 * j], d0[0] * scale, d0[1] * scale, q[k][j]);
                o[2 * j + 1] = nan_fix2(o[2 * j + 1], d1[0] * scale, d1[1] * scale, q[k][j] >> 16);
            }
            if (kNan == kNanByCode) {
                uint32_t lo = o[2 * j], hi = o[2 * j + 1];
                fix_nan_codes<kE5M2>(lo, hi, q[k][j]);
                o[2 * j] = lo;
                o[2 * j + 1] = hi;
            }
        }
        __builtin_amdgcn_raw_buffer_store_b128(o, rd, (k * kBlock + threadIdx.x) * 16, 0, kCpolNt | kCpolSc1);
    }
}

// Scatter + dequantise one tile of one page unit: fp8 decoded by the
// hardware converter (exact; all 256 codes of both encodings checked against
// the CPU oracle), times the scale in float32, rounded to bf16 by the
// hardware converter (round to nearest-even; checked on every float32).
// Tiles are kBlock*kVpt*16 bytes of bf16 output; grid = units * a.tiles, or
// fewer workgroups each taking a contiguous run of tiles.
template <int kBlock, int kVpt, bool kE5M2>
__device__ __forceinline__ void retrieve_fp8_unit_tile(const MoveArgs& a, const PageUnit& u, uint32_t tile)
{
    const uint32_t out_bytes = u.rows * a.width * 2;
    const uint32_t lo = tile * (kBlock * kVpt * 16);
    if (lo >= out_bytes) return;
    if (u.page < 0 || u.page >= a.num_pages) { raise_fault(kFaultPage); return; }
    const uint64_t pool = wave_uniform(gptr<const gu64>(u.kv ? a.v_pages : a.k_pages)[u.l]);
    const uint64_t chunk = wave_uniform(gptr<const gu64>(a.seq[u.s].chunks)[u.c]);
    if (bad_addr(pool)) { raise_fault(kFaultPool); return; }
    if (bad_addr(chunk)) { raise_fault(kFaultChunk); return; }
    const float scale = *gptr<const gf32>(chunk + scale_offset(a, u.l, u.kv, u.n_c));
    const uint32_t left = out_bytes - lo;
    const uint32_t n = left < kBlock * kVpt * 16 ? left : kBlock * kVpt * 16;
    const __amdgpu_buffer_rsrc_t rs =
        byte_range(chunk + section_offset(a, u.l, u.kv, u.n_c) + (uint64_t)u.j0 * a.width + lo / 2, n / 2);
    const __amdgpu_buffer_rsrc_t rd =
        byte_range(pool + (uint64_t)u.page * a.page_size * a.width * 2 + lo, n);
    u32x2 q[kVpt];
#pragma unroll
    for (int k = 0; k < kVpt; ++k)
        q[k] = __builtin_amdgcn_raw_buffer_load_b64(rs, (k * kBlock + threadIdx.x) * 8, 0, kCpolNt | kCpolSc1);
    // Every NaN result is written as the quiet NaN 0x7FC0 with its code's
    // sign (the hardware's conversions do not keep that sign).  A scale that
    // is NaN, infinite or zero can turn any product into NaN (NaN * x,
    // +-0 * inf, inf * 0): such groups take the path that checks every
    // product.  Under any other scale only a NaN code gives a NaN, and the
    // store writes none there; a lane whose codes hold one (a chunk from
    // elsewhere) takes the path that checks the codes.
    if (!(__builtin_fabsf(scale) < __builtin_inff()) || scale == 0.0f) {   // the same for the whole wave
        dequantise_store<kBlock, kVpt, kE5M2, kNanByProduct>(q, scale, rd);
        return;
    }
    uint32_t nan_any = 0;
#pragma unroll
    for (int k = 0; k < kVpt; ++k) nan_any |= nan_code_bits<kE5M2>(q[k][0]) | nan_code_bits<kE5M2>(q[k][1]);
    if (nan_any != 0)
        dequantise_store<kBlock, kVpt, kE5M2, kNanByCode>(q, scale, rd);
    else
        dequantise_store<kBlock, kVpt, kE5M2, kNanPlain>(q, scale, rd);
}

template <int kBlock, int kVpt, bool kE5M2>
__device__ __forceinline__ void retrieve_fp8_tile(const MoveArgsLut& al, uint32_t b)
{
    const MoveArgs& a = al.m;
    const uint32_t unit = b / a.tiles;
    const uint32_t tile = b - unit * a.tiles;
    const uint32_t item = a.item_base + unit;
    retrieve_fp8_unit_tile<kBlock, kVpt, kE5M2>(a, locate_page_unit(a, item, find_seq_lut(al, item)), tile);
}

// The same in pool-address order (sorted page list, see sorted_unit).
template <int kBlock, int kVpt, bool kE5M2>
__global__ __launch_bounds__(kBlock) void retrieve_fp8_sorted(MoveArgs a, uint64_t list, uint32_t n_list)
{
    const uint32_t b = xcd_contiguous(blockIdx.x, gridDim.x);
    const uint32_t unit = b / a.tiles, tile = b - unit * a.tiles;
    PageUnit u;
    if (!sorted_unit(a, list, n_list, unit, u)) return;
    retrieve_fp8_unit_tile<kBlock, kVpt, kE5M2>(a, u, tile);
}

template <int kBlock, int kVpt, bool kE5M2>
__global__ __launch_bounds__(kBlock) void retrieve_fp8(MoveArgsLut al)
{
    if (gridDim.x >= al.m.total_tiles) {      // one workgroup per tile: straight-line code
        retrieve_fp8_tile<kBlock, kVpt, kE5M2>(al, xcd_contiguous(blockIdx.x, gridDim.x));
        return;
    }
    const TileRange r = my_tiles(al.m.total_tiles);
    for (uint32_t b = r.first; b < r.last; ++b) retrieve_fp8_tile<kBlock, kVpt, kE5M2>(al, b);
}

}  // namespace kvmove
