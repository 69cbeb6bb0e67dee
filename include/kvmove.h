/*
 * kvmove.h -- C ABI of libkvmove.so: paged <-> chunk KV-cache movement on
 * AMD Instinct MI355X (gfx950).
 *
 * An inference engine keeps each layer's K and V cache in small fixed-size
 * pages (16 tokens here) scattered through a pool; a KV-cache layer moves it
 * in large contiguous chunks (256 tokens by default) instead.  This library
 * is the device-side mover between the two forms:
 *
 *   store    (gather)  pages -> chunk buffers, every layer, K then V;
 *   retrieve (scatter) chunk buffers -> pages, for the leading hit chunks;
 *   store / retrieve one layer, then record an event, so compute on another
 *            stream overlaps the movement of the neighbouring layer;
 *   optional fp8 serde: quantise to e4m3 on store, dequantise on retrieve.
 *
 * Sources (web pages, cited by title and section):
 *   [paper]  "LMCache: An Efficient KV Cache Layer for Enterprise-Scale LLM
 *            Inference" (paper notes): section "方法细节" (method details),
 *            paragraphs on configurable chunk size (a custom GPU kernel copies
 *            scattered pages into a contiguous streaming buffer as 256-token
 *            chunks, and splits loaded chunks back into pages) and on the
 *            layerwise pipeline (separate streams for compute and movement,
 *            layer i+1 loads while layer i computes); Table 2 (connector
 *            calls start_load_kv / wait_load_kv(layer)).
 *   [walk]   "LMCache 源码解析：一个文件讲透KV缓存复用机制" (cache_engine.py
 *            walkthrough): sections "store()" (chunking, batched gather of
 *            all chunks in one call), "retrieve()" (hits count from chunk 0
 *            and stop at the first miss; whole chunks may return more tokens
 *            than asked), "性能细节" (no transfer when nothing hits),
 *            "工程实践" (the computed prefix must be a whole number of chunks).
 *   [blob]   "LMCache 中的 KV Cache 压缩：CacheGen 编解码原理..." (CacheGen
 *            page), section "2. 量化": a chunk's KV blob is shaped
 *            [num_layers, 2, num_tokens, num_heads, head_size].
 *   [cachegen] the CacheGen page as [blob], section "2. 量化": per-layer bin
 *            counts, per-token absolute maximum, symbols round(x*MAX/max1+MAX).
 *   [serde]  "LMCache 分布式 KV Cache 序列化框架 Serde..." (serde framework
 *            page), sections "4.2" (exact, layout-only size estimate) and
 *            "7.1 fp8 量化" (fp8 e4m3 cast, one byte per element, lossy).
 *
 * Layouts (all little-endian):
 *   Pool   For layer l, k_pages[l] / v_pages[l] hold the device address of a
 *          bf16 array [num_pages][page_size][num_kv_heads][head_dim].  Token t
 *          of a sequence lives in row t % page_size of page
 *          block_table[t / page_size].
 *   Chunk  A chunk of n tokens (n <= chunk_size; only a sequence's last chunk
 *          is short) is one buffer holding, layer by layer, the layer's K
 *          section and then its V section, each n rows of H*D elements, then
 *          one float32 scale per quantised (layer, K/V) part in the same
 *          order.  Elements are 2 bytes (bf16, copied bit for bit) or 1 byte
 *          (fp8) according to the format:
 *            KV_FMT_BF16             K bf16, V bf16: exactly the blob
 *                                    [num_layers][2][n][H][D] of [blob];
 *            KV_FMT_FP8_E4M3_SCALED  K and V OCP E4M3 ("fn"), scales [L][2];
 *            KV_FMT_FP8_E5M2_SCALED  K and V OCP E5M2, scales [L][2];
 *            KV_FMT_K16_V8           K bf16, V E4M3, scales [L] ([serde]
 *                                    section "7.3" names this asymmetric
 *                                    K16/V8 serde).
 *          kv_chunk_bytes() gives the exact size.
 *
 * Where chunks live: a chunk buffer is either device memory or pinned host
 * memory that the device addresses directly (hipHostMalloc, or torch's
 * pin_memory=True).  With host buffers, store is the offload to CPU memory
 * and retrieve the onload from it: the kernels' own loads and stores cross
 * PCIe, with no staging buffer and no separate DMA step.  [paper] gathers
 * into a GPU streaming buffer and then copies that to CPU memory ("方法细节",
 * configurable-chunk-size paragraph); its section "实验结果", component-level
 * evaluation and Table 5, reports the load bandwidth from CPU memory that
 * this path is measured against.  Pageable host memory is not addressable
 * by the device and must not be passed.
 *
 * fp8 serde: per quantised (chunk, layer, K/V) group, amax = max |x| (a NaN
 * anywhere makes it NaN); scale = amax / fmax in float32 with fmax = 448
 * (E4M3) or 57344 (E5M2), and scale = 1 when amax == 0; q = fp8(x / scale)
 * with an IEEE float32 division, rounding to nearest-even and saturating at
 * +-fmax (infinity too).  Retrieve writes bf16(float(q) * scale), the product
 * in float32 and the bf16 rounding to nearest-even.  [serde] section "7.1"
 * casts to e4m3 (default) or e5m2 without a scale; the scale is this
 * library's addition.
 *
 * Ownership: every buffer is allocated and freed by the caller.  The library
 * allocates nothing and keeps no state between calls except, on each device,
 * a fault word (kv_take_faults) and the 8 MiB scratch array of
 * kv_retrieve_chunks_noalloc, both part of its code object.  Host arrays are
 * read only during the call.
 *
 * Ordering: every call enqueues work on the given HIP stream (0 = the null
 * stream) and returns without waiting for it.  Results computed from host
 * data (out_tokens) are final on return.
 *
 * Errors: every int-returning call returns KV_OK or a negative kv_status and
 * launches nothing on error; kv_last_error() then describes it (per thread).
 * Device-array contents (page ids, chunk addresses, their 16-byte
 * alignment) are checked inside the kernels: an offending row group is
 * skipped and a fault bit is set (kv_take_faults); the kernels never access
 * memory outside [page 0, page num_pages) of a layer's pool because of a bad
 * page id.  Chunk capacity cannot be checked: a chunk buffer must hold
 * kv_chunk_bytes() for its token count.
 */
#ifndef KVMOVE_H
#define KVMOVE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KV_OK = 0,
    KV_EINVAL = -1, /* malformed argument (null pointer, bad shape, misaligned start, bad format) */
    KV_ERANGE = -2, /* token range beyond the block table */
    KV_EHIP = -3    /* the HIP runtime refused a launch or an event record */
} kv_status;

typedef enum {
    KV_FMT_BF16 = 0,            /* bf16 copied bit for bit ("naive" serde) */
    KV_FMT_FP8_E4M3_SCALED = 1, /* e4m3 bytes + one float32 scale per (layer, K/V) */
    KV_FMT_FP8_E5M2_SCALED = 2, /* e5m2 bytes + one float32 scale per (layer, K/V) */
    KV_FMT_K16_V8 = 3,          /* K bf16, V e4m3 bytes + one float32 scale per layer */
    KV_FMT_CACHEGEN_INT8 = 4    /* CacheGen symbols + one float32 max1 per (layer, K/V, token);
                                   only through the *_cachegen entry points */
} kv_fmt;

/* The engine's paged pool.  All pointers are caller-owned. */
typedef struct {
    int32_t num_layers;     /* L  > 0 */
    int32_t num_kv_heads;   /* H  > 0 */
    int32_t head_dim;       /* D  > 0; H*D must be a multiple of 8 (16-byte rows) */
    int32_t page_size;      /* P  > 0 tokens per page (16 in vLLM-style engines) */
    int32_t chunk_size;     /* C  > 0 tokens per chunk, a multiple of P (256 by default);
                               C*H*D*2 <= 2^31 (one layer's K or V section of a chunk) */
    int64_t num_pages;      /* pages in each layer's K (and V) pool */
    const uint64_t* k_pages;/* DEVICE uint64[L]: address of layer l's K pool, 16-byte aligned */
    const uint64_t* v_pages;/* DEVICE uint64[L]: address of layer l's V pool, 16-byte aligned */
} kv_paged;

/* One sequence's job. */
typedef struct {
    const int32_t* block_table; /* DEVICE int32[n_bt]: page id of tokens [P*i, P*(i+1)) */
    int64_t n_bt;               /* entries in block_table */
    int64_t tok_start;          /* first token; a multiple of chunk_size ([walk] "工程实践") */
    int64_t tok_end;            /* one past the last token; tok_start <= tok_end <= P*n_bt */
    const uint64_t* chunks;     /* DEVICE uint64[n_chunks]: address of chunk c's buffer
                                   (device or pinned host memory), 16-byte aligned,
                                   >= kv_chunk_bytes(tokens of chunk c) */
} kv_seq;

/* Exact bytes of one chunk holding n_tokens tokens in format fmt ([serde]
 * "4.2": deterministic, from the layout alone); 0 on a malformed argument. */
size_t kv_chunk_bytes(const kv_paged* paged, int64_t n_tokens, kv_fmt fmt);

/* Chunks covering [tok_start, tok_end): ceil((tok_end - tok_start) / C); the
 * last one holds the remainder ([walk] "store()").  -1 on a malformed argument. */
int64_t kv_num_chunks(const kv_paged* paged, int64_t tok_start, int64_t tok_end);

/* Tokens of chunk c of [tok_start, tok_end): C, or the remainder for the
 * last chunk ([walk] "store()").  -1 on a malformed argument or a c outside
 * [0, kv_num_chunks).  With kv_chunk_bytes it sizes each chunk buffer. */
int64_t kv_chunk_tokens(const kv_paged* paged, int64_t tok_start, int64_t tok_end, int64_t c);

/* Store: gather every chunk of every sequence, all layers, K and V, into the
 * sequences' chunk buffers, in one batched launch ([paper] configurable chunk
 * size; [walk] "store()").  fmt KV_FMT_FP8_E4M3_SCALED quantises on the way
 * ([serde] "7.1").  The pool is only read.  Sequences with an empty range are
 * skipped.  To store a shorter prefix (e.g. after a failed allocation, [walk]
 * "store()"), pass a smaller tok_end. */
int kv_store_chunks(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt,
                    hipStream_t stream);

/* Store through an address plan: the same operation and result as
 * kv_store_chunks, with the bf16 parts' gather driven by a per-page-unit
 * address plan that a small kernel writes into `workspace` first (DEVICE
 * memory the caller owns, at least kv_store_workspace_bytes(paged, seqs,
 * n_seqs, fmt) bytes, 256-byte aligned; its contents on entry do not matter
 * and are overwritten).  Each workgroup then reads its addresses with one
 * load instead of the block-table and address chain, and the gather moves
 * 4 KiB tiles; it measured 2 % faster on the Llama-3.1-8B workload, the
 * plan's kernel included.  kv_store_workspace_bytes is 32 bytes per page
 * unit of the bf16 parts (every layer's K and V pages of every sequence; K
 * only for KV_FMT_K16_V8), rounded up to 256; 0 for the fp8 formats, whose
 * kernels need no plan (workspace may then be NULL), and on an invalid
 * call (kv_last_error says which).  Calls that share a workspace must be
 * ordered on one stream. */
size_t kv_store_workspace_bytes(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt);
int kv_store_chunks_ws(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Layerwise store ([paper] layerwise pipeline; Table 2 start_store_kv /
 * wait_store_kv(layer)): as kv_store_chunks but gathers layer `layer` only
 * (its K and V sections of every chunk; for fp8 also its two scales), on
 * stream, then records layer_done (if not NULL) on stream.  Calling it for
 * layers 0 .. L-1 fills the chunks as one kv_store_chunks call does.  Chunks
 * that are already stored are skipped by giving a later tok_start or an
 * earlier tok_end.  max_workgroups as for kv_retrieve_layer (bf16 only; the
 * fp8 store runs one workgroup per (chunk, K/V) group and ignores it). */
int kv_store_layer(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt, int32_t layer,
                   int32_t max_workgroups, hipStream_t stream, hipEvent_t layer_done);

/* Several layers of a store in one call: for k = 0 .. layer_end-layer_begin-1
 * and layer l = layer_begin + k, on stream: wait for wait_before[k] (if the
 * array and the entry are not NULL; an event the caller recorded after its
 * producer of layer l, e.g. that layer's compute), gather layer l as
 * kv_store_layer does with max_workgroups[k] (NULL: 0 for every layer), then
 * record layer_done[k] (if the array and the entry are not NULL).  The host
 * arguments are checked and the launch plan made once for all layers, so a
 * caller that has already enqueued its producers hands the whole pipeline
 * over in one call.  HOST arrays of layer_end - layer_begin entries; layers
 * [layer_begin, layer_end) must be a non-empty range inside [0, L).
 * alt_stream (NULL: none): a second stream of the caller's, on the current
 * device like stream; the odd k then run on it (wait, gather and record
 * alike).  It first waits for the work enqueued on stream before the call,
 * and stream ends waiting for its last layer, so work enqueued on stream
 * after the call still follows every layer; layer_done[k] then marks layer
 * l alone done.  Consecutive layers' kernels may then overlap, which hides
 * the start and the tail of each launch (32 layers of the Llama-3.1-8B
 * workload: 481 us against 561 us on one stream).  It helps only if the two
 * streams are on different hardware queues (GPU_MAX_HW_QUEUES); on one they
 * run in order, still correctly.  The fork and the join are event record /
 * wait pairs, so a capture of stream records the call as a graph with two
 * branches. */
int kv_store_layers(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt, int32_t layer_begin,
                    int32_t layer_end, const int32_t* max_workgroups, hipStream_t stream, hipStream_t alt_stream,
                    const hipEvent_t* wait_before, const hipEvent_t* layer_done);

/* Retrieve: for sequence i, n_hit = index of the first 0 in hit_mask[i][0 ..
 * n_chunks) (n_chunks if none); scatter chunks [0, n_hit) back into the
 * sequence's pages, all layers, K and V ([paper] configurable chunk size;
 * [walk] "retrieve()": a hole ends the hits even if later flags are set).
 * Page rows outside those chunks are not written.  out_tokens[i] (HOST,
 * may be NULL) = min(tok_end, tok_start + n_hit*C) - tok_start, which can
 * exceed what the engine lacked because whole chunks come back.  hit_mask is
 * a HOST array of n_seqs HOST pointers, entry i to at least
 * n_chunks = ceil((tok_end - tok_start) / C) flags, all of which may be read
 * (an entry may be NULL when the range is empty).  Nothing is launched when no chunk hits ([walk] "性能细节").
 * The page ids written by one call must be distinct. */
int kv_retrieve_chunks(const kv_paged* paged, const kv_seq* seqs,
                       const uint8_t* const* hit_mask, int n_seqs, kv_fmt fmt,
                       int64_t* out_tokens, hipStream_t stream);

/* Retrieve in pool-address order: the same operation and result as
 * kv_retrieve_chunks, with the scatter visiting its page units by
 * destination address (layer, K/V, page id) instead of chunk by chunk.
 * Random destination pages cost DRAM more on writes than on reads; this
 * order makes the writes near-sequential and measured about 6 % faster on
 * the Llama-3.1-8B workload.  It needs the hit pages sorted by page id,
 * which is done on the device in `workspace` (DEVICE memory the caller
 * owns, at least kv_retrieve_workspace_bytes(paged) bytes, 256-byte
 * aligned; its contents on entry do not matter and are overwritten).  Every
 * format has an ordered scatter (for KV_FMT_K16_V8 each of its two launches
 * builds the list).  A sequence moving 2^26 pages or more is rejected
 * (KV_EINVAL), and so, before anything is launched, is a call that moves
 * more pages than the pool holds (its page ids cannot all be distinct, and
 * its sorted list would not fit the workspace).  Calls that share a
 * workspace must be ordered on one stream. */
size_t kv_retrieve_workspace_bytes(const kv_paged* paged);   /* 0 on a malformed pool */
int kv_retrieve_chunks_ws(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs,
                          kv_fmt fmt, int64_t* out_tokens, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * kv_retrieve_chunks_ws with the workspace taken from a scratch array that
 * the library holds on each GPU (8 MiB, allocated when the library's code is
 * loaded onto the device and held until the process ends).  Same arguments,
 * result and errors as kv_retrieve_chunks, plus: a pool of more than 2^20
 * pages is refused (KV_EINVAL; use kv_retrieve_chunks_ws), and so is a
 * stream that belongs to another device than the current one.  It calls no
 * allocator, for device or host memory.  Every call on a GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (on streams not ordered with each other) race
 * and must not be made; calls ordered on one stream are safe. */
int kv_retrieve_chunks_noalloc(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask,
                               int n_seqs, kv_fmt fmt, int64_t* out_tokens, hipStream_t stream);

/* Layerwise retrieve ([paper] layerwise pipeline; Table 2 start_load_kv /
 * wait_load_kv(layer)): as kv_retrieve_chunks but writes layer `layer` only,
 * on copy_stream, then records layer_done (if not NULL) on copy_stream -- also
 * when nothing hits, so a stream or host waiting on it never hangs.  Calling
 * it for layers 0 .. L-1 leaves the pool as one kv_retrieve_chunks call does.
 * The scatter takes one workgroup per tile (one-wave workgroups: 2 KiB tiles
 * for bf16, 4 KiB of output for the fp8 retrieve).  Overlap needs copy_stream
 * and the compute stream on different hardware queues: HIP spreads a
 * process's streams over a few queues (GPU_MAX_HW_QUEUES, 4 by default), and
 * two streams that share a queue run in order. */
int kv_retrieve_layer(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs,
                      kv_fmt fmt, int32_t layer, hipStream_t copy_stream, hipEvent_t layer_done);

/* kv_retrieve_layer with two more arguments:
 *   out_tokens      HOST int64[n_seqs] or NULL: as for kv_retrieve_chunks;
 *   max_workgroups  0: one workgroup per tile (as kv_retrieve_layer, fastest
 *                   when the GPU is otherwise idle); > 0 caps the grid at that
 *                   many 256-thread workgroups, each moving a contiguous run of
 *                   8 KiB tiles, so the scatter occupies few wave slots while
 *                   compute on another stream runs beside it (page-unit
 *                   kernels: bf16 and the fp8 retrieve).  From host chunks
 *                   the scatter is bound by PCIe, and a cap of 32 workgroups
 *                   already moves at the link's rate. */
int kv_retrieve_layer_ex(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs,
                         kv_fmt fmt, int32_t layer, int64_t* out_tokens, int32_t max_workgroups,
                         hipStream_t copy_stream, hipEvent_t layer_done);

/* Several layers of a retrieve in one call ([paper] Table 2: start_load_kv
 * starts the load of every layer; wait_load_kv(layer) is the caller's wait on
 * layer_done[k]): for k = 0 .. layer_end-layer_begin-1, the scatter of layer
 * layer_begin + k as kv_retrieve_layer_ex does with max_workgroups[k] (HOST
 * array, NULL: 0 for every layer), then a record of layer_done[k] (HOST array
 * of events, NULL or NULL entries: none), all on copy_stream in layer order.
 * The hit mask is read and the plan made once; out_tokens as for
 * kv_retrieve_chunks.  Layers [layer_begin, layer_end) must be a non-empty
 * range inside [0, L).  A compute stream that waits on layer_done[k] before
 * layer k's work overlaps every later layer's load with that work.
 * alt_stream (NULL: none) as for kv_store_layers: the odd k's scatter and
 * record run on it, forked from and joined back into copy_stream, and
 * consecutive layers' kernels may overlap (32 layers of the Llama-3.1-8B
 * workload: 511 us against 582 us on one stream). */
int kv_retrieve_layers(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs,
                       kv_fmt fmt, int32_t layer_begin, int32_t layer_end, const int32_t* max_workgroups,
                       int64_t* out_tokens, hipStream_t copy_stream, hipStream_t alt_stream,
                       const hipEvent_t* layer_done);

/* CacheGen quantiser ([cachegen] section "2. 量化"): store gathers and
 * quantises every chunk, K and V of every layer, in format
 * KV_FMT_CACHEGEN_INT8; retrieve dequantises the leading hit chunks and
 * scatters them (hit rule, out_tokens and errors as kv_retrieve_chunks).
 * key_bins / value_bins: HOST int32[num_layers], the bin count of each
 * layer's K and V, each in [4, 129]; MAX = bins / 2 - 1.  For each token row
 * of H*D elements, max1 = max |x| (float32; a NaN in the row makes it NaN);
 * symbol q = round-half-even(x * (MAX / max1) + MAX) in float32, one rounding
 * per operation, kept in [0, 2*MAX] (fits the page's int8), MAX for a zero
 * row or a NaN; retrieve writes bf16((q - MAX) / MAX * max1).  Chunk of n
 * tokens: symbols u8 [L][2][n][H*D], then float32 max1 [L][2][n]
 * (kv_chunk_bytes with KV_FMT_CACHEGEN_INT8).  Limits: num_layers <= 128,
 * H*D <= 4096.  Only the quantiser: the CDF and arithmetic coding that
 * follow it on that page are not implemented.  workspace / workspace_bytes
 * as in kv_retrieve_chunks_ws: with one (DEVICE, caller-owned) the scatter
 * runs in pool-address order; NULL runs it chunk by chunk. */
int kv_store_chunks_cachegen(const kv_paged* paged, const kv_seq* seqs, int n_seqs, const int32_t* key_bins,
                             const int32_t* value_bins, hipStream_t stream);
int kv_retrieve_chunks_cachegen(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask,
                                int n_seqs, const int32_t* key_bins, const int32_t* value_bins,
                                int64_t* out_tokens, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Message for the last non-OK return on this thread ("" if none). */
const char* kv_last_error(void);

/* Waits for the current device, returns the fault bits the kernels set since
 * the last call on this device (1: page id out of range, 2: null or
 * misaligned chunk address, 4: null or misaligned pool address), and clears
 * them.  Returns -1 (KV_EHIP) if the device cannot be read. */
int kv_take_faults(void);

/* Measurement aid, not part of the movement path: a plain contiguous
 * device-to-device copy of `bytes` bytes (a multiple of 16; both addresses
 * 16-byte aligned) with the same vector width as the movers, used as the
 * achievable-copy ceiling and to calibrate HBM traffic counters. */
int kv_copy_bytes(void* dst, const void* src, size_t bytes, hipStream_t stream);

/* Measurement aid, not part of the movement path: kv_copy_bytes with one
 * side visited in blocks of block_bytes (a power of two from 4096 to 2^30;
 * bytes a multiple of it) in a fixed scattered order -- destination block
 * k <- source block (k * m) mod n_blocks for permute = 1 (scattered reads,
 * the gather's pattern when block_bytes is the page size), or destination
 * block (k * m) mod n_blocks <- source block k for permute = 2 (scattered
 * writes, the chunk-major scatter's), with m a prime the library picks coprime
 * with n_blocks (7919 unless it divides n_blocks).  Every destination byte is
 * written once.  The ceiling of each access pattern, with no block table.
 * Same alignment rules and errors as kv_copy_bytes, plus KV_EINVAL for a bad
 * block size or permute value. */
int kv_copy_blocks(void* dst, const void* src, size_t bytes, size_t block_bytes, int permute, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVMOVE_H */
