/*
 * kv_oracle.h -- plain CPU oracle for paged <-> chunk KV-cache movement.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no header, helper, table or
 * constant with the GPU library; the two meet only on the byte layouts that
 * the method defines, and on the seeded synthetic inputs.
 *
 * What it computes (sources are the web pages this project is built from,
 * cited by title and section):
 *
 *  - Chunking: a token range [s, e) is cut into C-token chunks (C = 256 by
 *    default), the last one partial.  "LMCache 源码解析：一个文件讲透KV缓存复用
 *    机制" (LMCache source walkthrough: cache_engine.py), section "store()：
 *    一条KV序列如何被分块、键控并批量写入" (how a KV sequence is chunked, keyed
 *    and written in batch); "LMCache: An Efficient KV Cache Layer for
 *    Enterprise-Scale LLM Inference" (paper notes), section "方法细节 /
 *    可配置的块大小" (configurable chunk size).
 *  - Store = gather: copy the KV of every token of a chunk, for every layer,
 *    K then V, out of the engine's scattered pages into one contiguous chunk
 *    buffer laid out [num_layers][2][n_c][num_heads][head_size] (the blob
 *    shape of "LMCache 中的 KV Cache 压缩：CacheGen 编解码原理..." (CacheGen
 *    page), section "2. 量化 (Quantization)").
 *  - Retrieve = scatter of the chunks back into pages, honouring the prefix
 *    hit rule: hits count from chunk 0 and stop at the first miss (LMCache
 *    source walkthrough, section "retrieve()：前缀匹配如何在首个未命中处停下").
 *  - The optional fp8 serde: every element cast to float8 e4m3fn (default)
 *    or e5m2, one byte per element ("LMCache 分布式 KV Cache 序列化框架 Serde
 *    双层接口设计与自定义扩展实战" (LMCache serde framework page), section
 *    "7.1 fp8 量化"), here with one fp32 absmax scale per (chunk, layer, K/V):
 *    scale = amax / fmax (448 for e4m3, 57344 for e5m2), q = fp8(x / scale)
 *    rounded to nearest-even and saturated.  NaN (the pages are silent):
 *    a group holding a NaN gets the default quiet NaN 0x7FC00000 as its
 *    scale; a NaN quotient encodes as 0x7F | the element's sign bit; a
 *    dequantised NaN is the bf16 quiet NaN 0x7FC0 with the code's sign.
 *  - The asymmetric K16/V8 serde named on the same page (section "7.3":
 *    K kept at 16 bits, V at 8): K copied as bf16, V quantised as scaled e4m3.
 *  - The CacheGen quantiser (CacheGen page, section "2. 量化"): per layer a
 *    bin count for K and one for V, MAX = bins / 2 - 1; per token row the
 *    absolute maximum max1 over its channels; symbol
 *    q = round(x * (MAX / max1) + MAX), kept with max1; dequantised as
 *    (q - MAX) / MAX * max1.  Only the quantiser, not the CDF and
 *    arithmetic coding that follow it on that page.  A row holding a NaN
 *    keeps max1 = 0x7FC00000; a dequantised NaN is written as 0x7FC0.
 *
 * Parity pins (tests marked "not gpu") tie each function to something other
 * than itself: numpy page-gather + reshape formulations, store-then-retrieve
 * identity, sentinel invariants, torch's float8_e4m3fn / bfloat16 casts over
 * exhaustive or large input sets, numpy float32 division and products, and a
 * closed-form round-trip error bound.
 */
#ifndef KV_ORACLE_H
#define KV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Chunk formats.  A chunk of n tokens holds, for each layer in order, its K
 * section then its V section, each n * H * D elements of the part's type
 * (bf16: 2 bytes, fp8: 1 byte), then one float32 scale for each quantised
 * (layer, K/V) part in the same order. */
enum {
    KVO_FMT_BF16 = 0,       /* K bf16, V bf16 */
    KVO_FMT_FP8 = 1,        /* K e4m3, V e4m3, scales [L][2] */
    KVO_FMT_FP8_E5M2 = 2,   /* K e5m2, V e5m2, scales [L][2] */
    KVO_FMT_K16_V8 = 3,     /* K bf16, V e4m3, scales [L] */
    KVO_FMT_CACHEGEN = 4    /* symbols u8 [L][2][n][H*D], then float32 max1 [L][2][n] */
};

/* The engine's paged pool, in host memory.  For layer l, k[l] and v[l] each
 * point at uint16 (raw bf16 bits) [num_pages][page_size][num_kv_heads*head_dim]. */
typedef struct {
    int32_t num_layers;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t chunk_size;
    int64_t num_pages;
    uint16_t* const* k;
    uint16_t* const* v;
} kvo_pool;

/* Chunk planning over [s, e): count, and tokens of chunk c. */
int64_t kvo_num_chunks(int64_t s, int64_t e, int32_t chunk_size);
int64_t kvo_chunk_tokens(int64_t s, int64_t e, int32_t chunk_size, int64_t c);
/* Exact size in bytes of one chunk holding n_tokens tokens. */
int64_t kvo_chunk_bytes(const kvo_pool* pool, int64_t n_tokens, int fmt);
/* Pool row holding token t: block_table[t / P] * P + t % P. */
int64_t kvo_slot(const int32_t* block_table, int32_t page_size, int64_t t);
/* Number of leading hit chunks: index of the first 0 in mask, else n_chunks. */
int64_t kvo_hit_chunks(const uint8_t* mask, int64_t n_chunks);

/* Store (gather) [s, e) into chunks[0 .. num_chunks).  layer < 0 stores every
 * layer, else only that layer's K and V sections of each chunk (the rest of
 * the chunk buffers is left as it was).  Returns 0, or -1 on a rejected
 * argument (s not chunk-aligned, e beyond the block table, a page id out of
 * range, bad format or layer). */
int kvo_store(const kvo_pool* pool, const int32_t* block_table, int64_t n_bt,
              int64_t s, int64_t e, uint8_t* const* chunks, int fmt, int32_t layer);

/* Retrieve (scatter) the leading hit chunks of [s, e) back into the pool.
 * layer < 0 moves every layer, else only that layer.  Returns the number of
 * tokens made available (counted from s), or -1 on a rejected argument
 * (as for store, plus duplicate page ids among the written pages). */
int64_t kvo_retrieve(const kvo_pool* pool, const int32_t* block_table, int64_t n_bt,
                     int64_t s, int64_t e, const uint8_t* mask,
                     uint8_t* const* chunks, int fmt, int32_t layer);

/* CacheGen quantiser: as kvo_store / kvo_retrieve in format KVO_FMT_CACHEGEN,
 * with per-layer bin counts key_bins[L] and value_bins[L], each in [4, 129]
 * (so every symbol 0 .. 2*MAX fits the page's int8).  Rejections as for
 * kvo_store / kvo_retrieve, plus a bin count out of range. */
int kvo_store_cachegen(const kvo_pool* pool, const int32_t* block_table, int64_t n_bt,
                       int64_t s, int64_t e, uint8_t* const* chunks,
                       const int32_t* key_bins, const int32_t* value_bins);
int64_t kvo_retrieve_cachegen(const kvo_pool* pool, const int32_t* block_table, int64_t n_bt,
                              int64_t s, int64_t e, const uint8_t* mask, uint8_t* const* chunks,
                              const int32_t* key_bins, const int32_t* value_bins);

/* Number formats. */
uint8_t  kvo_e4m3_encode(float y);       /* OCP E4M3 (fn), RNE, saturating */
float    kvo_e4m3_decode(uint8_t b);
uint8_t  kvo_e5m2_encode(float y);       /* OCP E5M2, RNE, saturating (infinity too) */
float    kvo_e5m2_decode(uint8_t b);
uint16_t kvo_bf16_from_float(float y);   /* IEEE-754 round-to-nearest-even */
float    kvo_float_from_bf16(uint16_t h);
float    kvo_fp8_scale(float amax);      /* amax == 0 ? 1 : amax / 448 */
float    kvo_e5m2_scale(float amax);     /* amax == 0 ? 1 : amax / 57344 */

/* Array forms of the conversions (for exhaustive checks). */
void kvo_e4m3_encode_n(const float* y, uint8_t* out, int64_t n);
void kvo_e4m3_encode_bits_range(uint64_t first_bits, int64_t n, uint8_t* out);
void kvo_e5m2_encode_n(const float* y, uint8_t* out, int64_t n);
void kvo_e5m2_encode_bits_range(uint64_t first_bits, int64_t n, uint8_t* out);
void kvo_bf16_from_float_n(const float* y, uint16_t* out, int64_t n);

#ifdef __cplusplus
}
#endif
#endif /* KV_ORACLE_H */
