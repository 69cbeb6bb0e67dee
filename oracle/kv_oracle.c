/*
 * kv_oracle.c -- plain CPU oracle for paged <-> chunk KV-cache movement.
 *
 * TEST INFRASTRUCTURE ONLY (see kv_oracle.h): used by the tests, the smoke
 * check and the benchmark's CPU baseline leg, never by the product path.
 *
 * Written for a reader checking it against the pages by eye: one token at a
 * time, one element at a time, no blocking, fusion or reordering.  Floating
 * point conversions are done in double, where scaling by powers of two and
 * the rounding step are exact; the fp8 scale and the quotient x / scale are
 * IEEE single-precision operations, as the method fixes them (fp32 scale).
 * Build with plain -O2 (no -ffast-math): x86-64 float arithmetic is then
 * IEEE binary32 with round-to-nearest-even and no flush of subnormals.
 */
#include "kv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- chunking */

/* A C-token chunk is the unit of storage; the trailing chunk may hold fewer
 * tokens (LMCache source walkthrough, section "store()": chunk_size defaults
 * to 256, the tail is kept when partial chunks are saved). */
int64_t kvo_num_chunks(int64_t s, int64_t e, int32_t chunk_size)
{
    if (e <= s) return 0;
    return (e - s + chunk_size - 1) / chunk_size;
}

int64_t kvo_chunk_tokens(int64_t s, int64_t e, int32_t chunk_size, int64_t c)
{
    int64_t first = s + c * chunk_size;
    int64_t last = first + chunk_size;        /* one past the chunk */
    if (last > e) last = e;
    return last > first ? last - first : 0;
}

/* How a chunk of format fmt holds K (kv = 0) or V (kv = 1): copied bf16, or
 * quantised to one of the two fp8 encodings the serde page offers (section
 * "7.1 fp8 量化": e4m3fn by default, e5m2 on request); the asymmetric format
 * keeps K at 16 bits and V at 8 (section "7.3"). */
enum { PART_BF16, PART_E4M3, PART_E5M2 };

static int part_kind(int fmt, int kv)
{
    switch (fmt) {
    case KVO_FMT_BF16: return PART_BF16;
    case KVO_FMT_FP8: return PART_E4M3;
    case KVO_FMT_FP8_E5M2: return PART_E5M2;
    case KVO_FMT_K16_V8: return kv == 0 ? PART_BF16 : PART_E4M3;
    }
    return -1;
}

static int valid_fmt(int fmt)
{
    return fmt == KVO_FMT_BF16 || fmt == KVO_FMT_FP8 || fmt == KVO_FMT_FP8_E5M2 || fmt == KVO_FMT_K16_V8;
}

/* Bytes per element of a part: bf16 2; fp8 1 (serde page, section "7.1":
 * one byte per element). */
static int64_t part_bytes(int kind) { return kind == PART_BF16 ? 2 : 1; }

/* Byte offset of the (l, kv) section of a chunk of n_c tokens: the sections
 * run layer by layer, K before V, each n_c rows of the part's type. */
static int64_t section_offset(const kvo_pool* p, int fmt, int l, int kv, int64_t n_c)
{
    int64_t width = (int64_t)p->num_kv_heads * p->head_dim;
    int64_t off = 0;
    for (int ll = 0; ll < p->num_layers; ll++) {
        for (int k = 0; k < 2; k++) {
            if (ll == l && k == kv) return off;
            off += n_c * width * part_bytes(part_kind(fmt, k));
        }
    }
    return off;      /* (l, kv) = (num_layers, 0): the end of the payload */
}

/* Byte offset of the float32 scale of a quantised (l, kv) part: the scales
 * follow the payload, one per quantised part, in the sections' order. */
static int64_t scale_offset(const kvo_pool* p, int fmt, int l, int kv, int64_t n_c)
{
    int64_t off = section_offset(p, fmt, p->num_layers, 0, n_c);
    for (int ll = 0; ll < p->num_layers; ll++) {
        for (int k = 0; k < 2; k++) {
            if (ll == l && k == kv) return off;
            if (part_kind(fmt, k) != PART_BF16) off += 4;
        }
    }
    return off;
}

/* Exact serialized size (serde page, section "4.2": the estimate follows from
 * the layout alone, with no slack): the sections plus the scales. */
int64_t kvo_chunk_bytes(const kvo_pool* p, int64_t n_tokens, int fmt)
{
    if (fmt == KVO_FMT_CACHEGEN) {
        /* one byte per symbol, then one float32 max1 per (layer, K/V, token) */
        int64_t rows = (int64_t)p->num_layers * 2 * n_tokens;
        return rows * p->num_kv_heads * p->head_dim + rows * 4;
    }
    if (!valid_fmt(fmt)) return -1;
    return scale_offset(p, fmt, p->num_layers, 0, n_tokens);
}

/* The connector hands the mover the addresses of the pages that hold a
 * sequence (paper notes, section "端到端系统工作流" (end-to-end workflow):
 * "GPU memory addresses of the relevant pages"); token t lives in row t % P of
 * page block_table[t / P]. */
int64_t kvo_slot(const int32_t* block_table, int32_t page_size, int64_t t)
{
    return (int64_t)block_table[t / page_size] * page_size + t % page_size;
}

/* Prefix hits: count from chunk 0, stop at the first miss (LMCache source
 * walkthrough, section "retrieve()": lookup returns at the first unhit chunk,
 * and after a failed fetch every later hit flag is cleared). */
int64_t kvo_hit_chunks(const uint8_t* mask, int64_t n_chunks)
{
    int64_t c = 0;
    while (c < n_chunks && mask[c] != 0) c++;
    return c;
}

/* ------------------------------------------------------------ number formats */

/* bf16 bits -> float: the upper half of the binary32 pattern. */
float kvo_float_from_bf16(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* float -> bf16 by IEEE-754 round-to-nearest, ties-to-even.  bf16 has an
 * 8-bit significand and binary32's exponent range: in the binade [2^E, 2^E+1)
 * (E >= -126) representable values are spaced 2^(E-7); below 2^-126 the
 * subnormal spacing 2^-133 holds.  Overflow rounds to infinity.  NaN stays a
 * NaN: sign and upper payload kept, quiet bit set. */
uint16_t kvo_bf16_from_float(float y)
{
    uint32_t bits;
    memcpy(&bits, &y, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(y)) return (uint16_t)((bits >> 16) | 0x0040u);
    if (isinf(y)) return (uint16_t)(sign | 0x7F80u);
    double a = fabs((double)y);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    if (E < -126) E = -126;
    double q = ldexp(1.0, E - 7); /* spacing of bf16 values around a */
    double v = nearbyint(a / q) * q;   /* default rounding mode: ties to even */
    if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    if (v < ldexp(1.0, -126)) {
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -133)));
    }
    frexp(v, &e);
    E = e - 1;
    int mant = (int)((v / ldexp(1.0, E) - 1.0) * 128.0);
    return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)mant);
}

/* OCP 8-bit floating point, E4M3 ("fn": no infinities): exponent bias 7,
 * 3 mantissa bits, S.1111.111 is NaN, largest finite 448 = S.1111.110,
 * smallest normal 2^-6, subnormals m * 2^-9 for m = 1..7.  Closed-form decode. */
float kvo_e4m3_decode(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return s ? -NAN : NAN;
    if (e == 0) v = m * ldexp(1.0, -9);
    else v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return (float)(s ? -v : v);
}

/* float -> E4M3 with round-to-nearest-even over normals and subnormals, and
 * saturation: a magnitude that rounds above 448 (including infinity) becomes
 * 448.  +-0 keep their sign; NaN becomes S.1111.111. */
uint8_t kvo_e4m3_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return (uint8_t)(sign | 0x7F);
    if (isinf(y)) return (uint8_t)(sign | 0x7E);
    double a = fabs((double)y);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    if (E < -6) E = -6;           /* below 2^-6 the subnormal spacing 2^-9 holds */
    double q = ldexp(1.0, E - 3); /* spacing of E4M3 values around a */
    double v = nearbyint(a / q) * q;   /* ties to even */
    if (v > 448.0) return (uint8_t)(sign | 0x7E);
    if (v < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)(v / ldexp(1.0, -9)));
    frexp(v, &e);
    E = e - 1;
    int mant = (int)((v / ldexp(1.0, E) - 1.0) * 8.0);
    return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)mant);
}

/* OCP 8-bit floating point, E5M2: exponent bias 15, 2 mantissa bits,
 * S.11111.00 is infinity and S.11111.{01,10,11} NaN, largest finite
 * 57344 = S.11110.11, smallest normal 2^-14, subnormals m * 2^-16 for
 * m = 1..3.  Closed-form decode. */
float kvo_e5m2_decode(uint8_t b)
{
    int s = b >> 7, e = (b >> 2) & 31, m = b & 3;
    double v;
    if (e == 31) {
        if (m == 0) return s ? -INFINITY : INFINITY;
        return s ? -NAN : NAN;
    }
    if (e == 0) v = m * ldexp(1.0, -16);
    else v = (1.0 + m / 4.0) * ldexp(1.0, e - 15);
    return (float)(s ? -v : v);
}

/* float -> E5M2, round-to-nearest-even over normals and subnormals,
 * saturating: a magnitude that rounds above 57344, and infinity, become
 * 57344 (the saturating reading is the same as for E4M3).  +-0 keep their
 * sign; NaN becomes S.11111.11. */
uint8_t kvo_e5m2_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return (uint8_t)(sign | 0x7F);
    if (isinf(y)) return (uint8_t)(sign | 0x7B);
    double a = fabs((double)y);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    if (E < -14) E = -14;         /* below 2^-14 the subnormal spacing 2^-16 holds */
    double q = ldexp(1.0, E - 2); /* spacing of E5M2 values around a */
    double v = nearbyint(a / q) * q;   /* ties to even */
    if (v > 57344.0) return (uint8_t)(sign | 0x7B);
    if (v < ldexp(1.0, -14)) return (uint8_t)(sign | (uint8_t)(v / ldexp(1.0, -16)));
    frexp(v, &e);
    E = e - 1;
    int mant = (int)((v / ldexp(1.0, E) - 1.0) * 4.0);
    return (uint8_t)(sign | (uint8_t)((E + 15) << 2) | (uint8_t)mant);
}

/* The default quiet NaN of binary32 (sign 0, quiet bit, zero payload).  The
 * pages say nothing of NaN; the reading taken here gives every NaN the method
 * produces a fixed pattern, so that two implementations agree bit for bit:
 * the scale of a group holding a NaN, the max1 of a CacheGen row holding
 * one, and (as bf16 0x7FC0, with the sign noted where it is kept) a NaN
 * dequantised value. */
static float default_nan(void)
{
    const uint32_t bits = 0x7FC00000u;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* Code of an element whose quotient x / scale is NaN (the group holds a NaN,
 * or x and the scale are both infinite): the NaN code of the encoding with
 * the sign bit of the element itself, S.1111.111 (E4M3) or S.11111.11
 * (E5M2) -- both are 0x7F | sign. */
static uint8_t nan_code(uint16_t x_bits)
{
    return (uint8_t)(((x_bits >> 8) & 0x80u) | 0x7Fu);
}

/* bf16 result of a dequantised value that is NaN: the quiet NaN 0x7FC0, with
 * the sign of the fp8 code it came from (sign_bit 0 or 1). */
static uint16_t nan_bf16(int sign_bit)
{
    return (uint16_t)(0x7FC0u | (sign_bit ? 0x8000u : 0u));
}

/* One scale per (chunk, layer, K/V) group: the group's absolute maximum
 * mapped onto E4M3's largest finite value, so the group spans [-448, 448].
 * An all-zero group takes scale 1 (its elements encode as signed zeros). */
float kvo_fp8_scale(float amax)
{
    if (amax == 0.0f) return 1.0f;
    return amax / 448.0f;
}

/* As kvo_fp8_scale, for E5M2's largest finite value. */
float kvo_e5m2_scale(float amax)
{
    if (amax == 0.0f) return 1.0f;
    return amax / 57344.0f;
}

void kvo_e5m2_encode_n(const float* y, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = kvo_e5m2_encode(y[i]);
}

void kvo_e5m2_encode_bits_range(uint64_t first_bits, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; i++) {
        uint32_t bits = (uint32_t)(first_bits + (uint64_t)i);
        float y;
        memcpy(&y, &bits, 4);
        out[i] = kvo_e5m2_encode(y);
    }
}

void kvo_e4m3_encode_n(const float* y, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = kvo_e4m3_encode(y[i]);
}

/* Encode the n binary32 values whose bit patterns are first_bits,
 * first_bits + 1, ... (for exhaustive checks over all patterns). */
void kvo_e4m3_encode_bits_range(uint64_t first_bits, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; i++) {
        uint32_t bits = (uint32_t)(first_bits + (uint64_t)i);
        float y;
        memcpy(&y, &bits, 4);
        out[i] = kvo_e4m3_encode(y);
    }
}

void kvo_bf16_from_float_n(const float* y, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = kvo_bf16_from_float(y[i]);
}

/* ---------------------------------------------------------------- movement */

static int check_args(const kvo_pool* p, const int32_t* bt, int64_t n_bt,
                      int64_t s, int64_t e, int fmt)
{
    if (p == NULL || bt == NULL) return -1;
    if (p->num_layers <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0) return -1;
    if (p->page_size <= 0 || p->chunk_size <= 0 || p->num_pages <= 0) return -1;
    if (!valid_fmt(fmt)) return -1;
    /* the already-computed prefix must be a whole number of chunks (LMCache
     * source walkthrough, section "工程实践": the count of False mask entries
     * must be a multiple of chunk_size, else ValueError) */
    if (s < 0 || s > e || s % p->chunk_size != 0) return -1;
    if (e > n_bt * p->page_size) return -1;
    for (int64_t t = s; t < e; t++) {
        int32_t page = bt[t / p->page_size];
        if (page < 0 || page >= p->num_pages) return -1;
    }
    return 0;
}

/* Address of element (row, i) of layer l's K (kv = 0) or V (kv = 1) pool. */
static uint16_t* pool_elem(const kvo_pool* p, int l, int kv, int64_t row, int64_t i)
{
    int64_t width = (int64_t)p->num_kv_heads * p->head_dim;
    uint16_t* base = kv == 0 ? p->k[l] : p->v[l];
    return base + row * width + i;
}

/* Inside the (l, kv) section of a chunk, element (j, i) -- token j of the
 * chunk, element i of its row -- sits at byte (j * width + i) * element size.
 * For bf16 everywhere this is the blob [layers][K,V][tokens][heads *
 * head_size] of the CacheGen page, section "2. 量化". */

/* Store: the paper notes (section "可配置的块大小") describe a GPU kernel that
 * copies KV from scattered paged memory into a contiguous buffer, grouping
 * pages of all layers into 256-token chunks; the LMCache walkthrough's store()
 * gathers every chunk of the request in one batched call.  The layerwise
 * variant (paper notes, section "层级流水线" and Table 2's start_store_kv /
 * wait_store_kv(layer)) stores one layer per call. */
int kvo_store(const kvo_pool* p, const int32_t* bt, int64_t n_bt,
              int64_t s, int64_t e, uint8_t* const* chunks, int fmt, int32_t layer)
{
    if (check_args(p, bt, n_bt, s, e, fmt) != 0) return -1;
    if (layer >= p->num_layers) return -1;
    int64_t width = (int64_t)p->num_kv_heads * p->head_dim;
    int64_t n_chunks = kvo_num_chunks(s, e, p->chunk_size);
    for (int64_t c = 0; c < n_chunks; c++) {
        if (chunks[c] == NULL) return -1;
    }
    for (int64_t c = 0; c < n_chunks; c++) {
        int64_t n_c = kvo_chunk_tokens(s, e, p->chunk_size, c);
        int64_t t0 = s + c * p->chunk_size;
        uint8_t* buf = chunks[c];
        for (int l = 0; l < p->num_layers; l++) {
            if (layer >= 0 && l != layer) continue;
            for (int kv = 0; kv < 2; kv++) {
                int kind = part_kind(fmt, kv);
                uint8_t* sec = buf + section_offset(p, fmt, l, kv, n_c);
                int64_t eb = part_bytes(kind);
                if (kind == PART_BF16) {
                    for (int64_t j = 0; j < n_c; j++) {
                        int64_t row = kvo_slot(bt, p->page_size, t0 + j);
                        for (int64_t i = 0; i < width; i++) {
                            uint16_t x = *pool_elem(p, l, kv, row, i);
                            memcpy(sec + (j * width + i) * eb, &x, 2);
                        }
                    }
                } else {
                    /* group absolute maximum; any NaN makes it NaN */
                    float amax = 0.0f;
                    int saw_nan = 0;
                    for (int64_t j = 0; j < n_c; j++) {
                        int64_t row = kvo_slot(bt, p->page_size, t0 + j);
                        for (int64_t i = 0; i < width; i++) {
                            float x = kvo_float_from_bf16(*pool_elem(p, l, kv, row, i));
                            if (isnan(x)) saw_nan = 1;
                            else if (fabsf(x) > amax) amax = fabsf(x);
                        }
                    }
                    float scale;
                    if (saw_nan) scale = default_nan();
                    else scale = kind == PART_E4M3 ? kvo_fp8_scale(amax) : kvo_e5m2_scale(amax);
                    for (int64_t j = 0; j < n_c; j++) {
                        int64_t row = kvo_slot(bt, p->page_size, t0 + j);
                        for (int64_t i = 0; i < width; i++) {
                            uint16_t xb = *pool_elem(p, l, kv, row, i);
                            float x = kvo_float_from_bf16(xb);
                            float y = x / scale;          /* binary32 division */
                            uint8_t code;
                            if (isnan(y)) code = nan_code(xb);
                            else code = kind == PART_E4M3 ? kvo_e4m3_encode(y) : kvo_e5m2_encode(y);
                            sec[(j * width + i) * eb] = code;
                        }
                    }
                    memcpy(buf + scale_offset(p, fmt, l, kv, n_c), &scale, 4);
                }
            }
        }
    }
    return 0;
}

/* Retrieve: chunks go back into paged memory (paper notes, section
 * "可配置的块大小": on load the kernel splits the buffer into pages), only for
 * the leading hit chunks; the caller gets the token count counted from s,
 * which can exceed what it asked for because whole chunks come back (LMCache
 * walkthrough, section "retrieve()").  The layerwise variant moves a single
 * layer per call (paper notes, section "层级流水线"). */
int64_t kvo_retrieve(const kvo_pool* p, const int32_t* bt, int64_t n_bt,
                     int64_t s, int64_t e, const uint8_t* mask,
                     uint8_t* const* chunks, int fmt, int32_t layer)
{
    if (check_args(p, bt, n_bt, s, e, fmt) != 0) return -1;
    if (layer >= p->num_layers) return -1;
    int64_t width = (int64_t)p->num_kv_heads * p->head_dim;
    int64_t n_chunks = kvo_num_chunks(s, e, p->chunk_size);
    if (n_chunks > 0 && mask == NULL) return -1;
    int64_t n_hit = kvo_hit_chunks(mask, n_chunks);
    int64_t tokens = 0;
    for (int64_t c = 0; c < n_hit; c++) tokens += kvo_chunk_tokens(s, e, p->chunk_size, c);
    for (int64_t c = 0; c < n_hit; c++) {
        if (chunks[c] == NULL) return -1;
    }
    /* two writes into one page row would race on a parallel device: the page
     * ids written must be distinct */
    int64_t first_page = s / p->page_size;
    int64_t n_pages = (tokens + p->page_size - 1) / p->page_size;
    for (int64_t a = 0; a < n_pages; a++) {
        for (int64_t b = a + 1; b < n_pages; b++) {
            if (bt[first_page + a] == bt[first_page + b]) return -1;
        }
    }
    for (int64_t c = 0; c < n_hit; c++) {
        int64_t n_c = kvo_chunk_tokens(s, e, p->chunk_size, c);
        int64_t t0 = s + c * p->chunk_size;
        const uint8_t* buf = chunks[c];
        for (int l = 0; l < p->num_layers; l++) {
            if (layer >= 0 && l != layer) continue;
            for (int kv = 0; kv < 2; kv++) {
                int kind = part_kind(fmt, kv);
                const uint8_t* sec = buf + section_offset(p, fmt, l, kv, n_c);
                int64_t eb = part_bytes(kind);
                float scale = 1.0f;
                if (kind != PART_BF16) memcpy(&scale, buf + scale_offset(p, fmt, l, kv, n_c), 4);
                for (int64_t j = 0; j < n_c; j++) {
                    int64_t row = kvo_slot(bt, p->page_size, t0 + j);
                    for (int64_t i = 0; i < width; i++) {
                        const uint8_t* src = sec + (j * width + i) * eb;
                        uint16_t x;
                        if (kind == PART_BF16) {
                            memcpy(&x, src, 2);
                        } else {
                            float d = kind == PART_E4M3 ? kvo_e4m3_decode(*src) : kvo_e5m2_decode(*src);
                            float prod = d * scale;       /* binary32 product */
                            if (isnan(prod)) x = nan_bf16(*src >> 7);
                            else x = kvo_bf16_from_float(prod);
                        }
                        *pool_elem(p, l, kv, row, i) = x;
                    }
                }
            }
        }
    }
    return tokens;
}

/* ------------------------------------------------- CacheGen quantiser */

/* The CacheGen page (section "2. 量化") quantises K and V, each viewed as
 * [layers][tokens][channels], layer by layer with that layer's bin count:
 * MAX = bins / 2 - 1; max1 = max |x| over a token's channels; the symbol is
 * round(x * (MAX / max1) + MAX), rounded half to even as torch.round does,
 * and max1 is kept for the inverse (q - MAX) / MAX * max1.  All arithmetic
 * in float32, one rounding per operation.  Readings: an all-zero row
 * (max1 == 0) gives every element the symbol MAX (the division by zero has
 * no value there); a NaN from the arithmetic also gives MAX.  A row holding
 * a NaN keeps max1 = the default quiet NaN, and a dequantised value that is
 * NaN is written as the bf16 quiet NaN 0x7FC0. */
static int cachegen_max(const int32_t* bins, int l)
{
    return bins[l] / 2 - 1;
}

static int check_bins(const kvo_pool* p, const int32_t* key_bins, const int32_t* value_bins)
{
    if (key_bins == NULL || value_bins == NULL) return -1;
    for (int l = 0; l < p->num_layers; l++) {
        if (key_bins[l] < 4 || key_bins[l] > 129) return -1;
        if (value_bins[l] < 4 || value_bins[l] > 129) return -1;
    }
    return 0;
}

/* Chunk of n_c tokens: symbols u8 [L][2][n_c][width], then float32
 * max1 [L][2][n_c]. */
static int64_t cg_row(const kvo_pool* p, int l, int kv, int64_t n_c, int64_t j)
{
    return ((int64_t)l * 2 + kv) * n_c + j;
}

int kvo_store_cachegen(const kvo_pool* p, const int32_t* bt, int64_t n_bt,
                       int64_t s, int64_t e, uint8_t* const* chunks,
                       const int32_t* key_bins, const int32_t* value_bins)
{
    if (check_args(p, bt, n_bt, s, e, KVO_FMT_BF16) != 0) return -1;
    if (check_bins(p, key_bins, value_bins) != 0) return -1;
    int64_t width = (int64_t)p->num_kv_heads * p->head_dim;
    int64_t n_chunks = kvo_num_chunks(s, e, p->chunk_size);
    for (int64_t c = 0; c < n_chunks; c++) {
        if (chunks[c] == NULL) return -1;
    }
    for (int64_t c = 0; c < n_chunks; c++) {
        int64_t n_c = kvo_chunk_tokens(s, e, p->chunk_size, c);
        int64_t t0 = s + c * p->chunk_size;
        uint8_t* buf = chunks[c];
        uint8_t* max_area = buf + (int64_t)p->num_layers * 2 * n_c * width;
        for (int l = 0; l < p->num_layers; l++) {
            for (int kv = 0; kv < 2; kv++) {
                int MAX = cachegen_max(kv == 0 ? key_bins : value_bins, l);
                for (int64_t j = 0; j < n_c; j++) {
                    int64_t row = kvo_slot(bt, p->page_size, t0 + j);
                    float max1 = 0.0f;
                    int saw_nan = 0;
                    for (int64_t i = 0; i < width; i++) {
                        float x = kvo_float_from_bf16(*pool_elem(p, l, kv, row, i));
                        if (isnan(x)) saw_nan = 1;
                        else if (fabsf(x) > max1) max1 = fabsf(x);
                    }
                    if (saw_nan) max1 = default_nan();
                    float factor = max1 == 0.0f ? 0.0f : (float)MAX / max1;
                    uint8_t* out = buf + cg_row(p, l, kv, n_c, j) * width;
                    for (int64_t i = 0; i < width; i++) {
                        float x = kvo_float_from_bf16(*pool_elem(p, l, kv, row, i));
                        float scaled = x * factor;              /* binary32 product */
                        float y = scaled + (float)MAX;          /* binary32 sum */
                        int q;
                        if (isnan(y)) q = MAX;
                        else {
                            float r = nearbyintf(y);            /* ties to even */
                            q = r < 0.0f ? 0 : r > 2.0f * MAX ? 2 * MAX : (int)r;
                        }
                        out[i] = (uint8_t)q;
                    }
                    memcpy(max_area + 4 * cg_row(p, l, kv, n_c, j), &max1, 4);
                }
            }
        }
    }
    return 0;
}

int64_t kvo_retrieve_cachegen(const kvo_pool* p, const int32_t* bt, int64_t n_bt,
                              int64_t s, int64_t e, const uint8_t* mask, uint8_t* const* chunks,
                              const int32_t* key_bins, const int32_t* value_bins)
{
    if (check_args(p, bt, n_bt, s, e, KVO_FMT_BF16) != 0) return -1;
    if (check_bins(p, key_bins, value_bins) != 0) return -1;
    int64_t width = (int64_t)p->num_kv_heads * p->head_dim;
    int64_t n_chunks = kvo_num_chunks(s, e, p->chunk_size);
    if (n_chunks > 0 && mask == NULL) return -1;
    int64_t n_hit = kvo_hit_chunks(mask, n_chunks);
    int64_t tokens = 0;
    for (int64_t c = 0; c < n_hit; c++) tokens += kvo_chunk_tokens(s, e, p->chunk_size, c);
    for (int64_t c = 0; c < n_hit; c++) {
        if (chunks[c] == NULL) return -1;
    }
    int64_t first_page = s / p->page_size;
    int64_t n_pages = (tokens + p->page_size - 1) / p->page_size;
    for (int64_t a = 0; a < n_pages; a++) {
        for (int64_t b = a + 1; b < n_pages; b++) {
            if (bt[first_page + a] == bt[first_page + b]) return -1;
        }
    }
    for (int64_t c = 0; c < n_hit; c++) {
        int64_t n_c = kvo_chunk_tokens(s, e, p->chunk_size, c);
        int64_t t0 = s + c * p->chunk_size;
        const uint8_t* buf = chunks[c];
        const uint8_t* max_area = buf + (int64_t)p->num_layers * 2 * n_c * width;
        for (int l = 0; l < p->num_layers; l++) {
            for (int kv = 0; kv < 2; kv++) {
                int MAX = cachegen_max(kv == 0 ? key_bins : value_bins, l);
                for (int64_t j = 0; j < n_c; j++) {
                    int64_t row = kvo_slot(bt, p->page_size, t0 + j);
                    float max1;
                    memcpy(&max1, max_area + 4 * cg_row(p, l, kv, n_c, j), 4);
                    const uint8_t* in = buf + cg_row(p, l, kv, n_c, j) * width;
                    for (int64_t i = 0; i < width; i++) {
                        float centred = (float)in[i] - (float)MAX;   /* exact */
                        float unit = centred / (float)MAX;           /* binary32 quotient */
                        float x = unit * max1;                       /* binary32 product */
                        /* NaN (a NaN max1, or 0 times an infinite one): no sign to keep */
                        *pool_elem(p, l, kv, row, i) = isnan(x) ? nan_bf16(0) : kvo_bf16_from_float(x);
                    }
                }
            }
        }
    }
    return tokens;
}
