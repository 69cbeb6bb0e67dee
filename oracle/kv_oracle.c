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

/* Exact serialized size: 2 bytes per bf16 element, or, for fp8, 1 byte per
 * element (serde page, section "7.1 fp8 量化": the estimate is exactly the
 * element count) plus one fp32 scale per (layer, K/V). */
int64_t kvo_chunk_bytes(const kvo_pool* p, int64_t n_tokens, int fmt)
{
    int64_t elems = (int64_t)p->num_layers * 2 * n_tokens * p->num_kv_heads * p->head_dim;
    if (fmt == KVO_FMT_BF16) return elems * 2;
    if (fmt == KVO_FMT_FP8) return elems + (int64_t)p->num_layers * 2 * 4;
    return -1;
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

/* One scale per (chunk, layer, K/V) group: the group's absolute maximum
 * mapped onto E4M3's largest finite value, so the group spans [-448, 448].
 * An all-zero group takes scale 1 (its elements encode as signed zeros). */
float kvo_fp8_scale(float amax)
{
    if (amax == 0.0f) return 1.0f;
    return amax / 448.0f;
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
    if (fmt != KVO_FMT_BF16 && fmt != KVO_FMT_FP8) return -1;
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

/* Byte offset of element (l, kv, j, i) inside a chunk of n_c tokens laid out
 * [layers][K,V][tokens][heads * head_size], in units of elements. */
static int64_t chunk_index(const kvo_pool* p, int l, int kv, int64_t n_c, int64_t j, int64_t i)
{
    int64_t width = (int64_t)p->num_kv_heads * p->head_dim;
    return (((int64_t)l * 2 + kv) * n_c + j) * width + i;
}

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
                if (fmt == KVO_FMT_BF16) {
                    for (int64_t j = 0; j < n_c; j++) {
                        int64_t row = kvo_slot(bt, p->page_size, t0 + j);
                        for (int64_t i = 0; i < width; i++) {
                            uint16_t x = *pool_elem(p, l, kv, row, i);
                            memcpy(buf + 2 * chunk_index(p, l, kv, n_c, j, i), &x, 2);
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
                    if (saw_nan) amax = NAN;
                    float scale = kvo_fp8_scale(amax);
                    for (int64_t j = 0; j < n_c; j++) {
                        int64_t row = kvo_slot(bt, p->page_size, t0 + j);
                        for (int64_t i = 0; i < width; i++) {
                            float x = kvo_float_from_bf16(*pool_elem(p, l, kv, row, i));
                            float y = x / scale;          /* binary32 division */
                            buf[chunk_index(p, l, kv, n_c, j, i)] = kvo_e4m3_encode(y);
                        }
                    }
                    /* scales follow the payload as float32[layers][K,V] */
                    int64_t payload = (int64_t)p->num_layers * 2 * n_c * width;
                    memcpy(buf + payload + 4 * ((int64_t)l * 2 + kv), &scale, 4);
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
        int64_t payload = (int64_t)p->num_layers * 2 * n_c * width;
        for (int l = 0; l < p->num_layers; l++) {
            if (layer >= 0 && l != layer) continue;
            for (int kv = 0; kv < 2; kv++) {
                float scale = 1.0f;
                if (fmt == KVO_FMT_FP8) memcpy(&scale, buf + payload + 4 * ((int64_t)l * 2 + kv), 4);
                for (int64_t j = 0; j < n_c; j++) {
                    int64_t row = kvo_slot(bt, p->page_size, t0 + j);
                    for (int64_t i = 0; i < width; i++) {
                        uint16_t x;
                        if (fmt == KVO_FMT_BF16) {
                            memcpy(&x, buf + 2 * chunk_index(p, l, kv, n_c, j, i), 2);
                        } else {
                            float d = kvo_e4m3_decode(buf[chunk_index(p, l, kv, n_c, j, i)]);
                            float prod = d * scale;       /* binary32 product */
                            x = kvo_bf16_from_float(prod);
                        }
                        *pool_elem(p, l, kv, row, i) = x;
                    }
                }
            }
        }
    }
    return tokens;
}
