/*
 * abi_c_example.c -- the C ABI of libkvmove.so used from plain C (no Python):
 * a two-layer paged pool with a known pattern, one 300-token sequence
 * (a full 256-token chunk and a 44-token tail) on scattered pages, stored
 * into chunks (plainly and through the store's address plan), the pool
 * cleared, the chunks retrieved: in one call, layer by layer with one event
 * per layer, in pool-address order with a workspace and with the library's
 * scratch, and every layer in one call on two streams; last, every layer
 * stored in one call on two streams and retrieved.  Checks that every
 * row the sequence owns comes back bit for bit, that the other pages stay
 * clear, that the retrieve reports 300 tokens and that no fault bit is set.
 * Exit status 0 on success.  Built by the package's build step; run by a
 * GPU test.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvmove.h"

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

#define CHECK_KV(x)                                                                   \
    do {                                                                              \
        int r_ = (x);                                                                 \
        if (r_ != KV_OK) {                                                            \
            fprintf(stderr, "%s returned %d: %s\n", #x, r_, kv_last_error());         \
            return 3;                                                                 \
        }                                                                             \
    } while (0)

enum { L = 2, H = 2, D = 64, P = 16, C = 256, NUM_PAGES = 64, TOKENS = 300 };

/* Copies the device pool back and checks it: every row the sequence owns
 * holds the original pattern, every other row is still zero. */
static int check_pool(const uint16_t* pool, uint16_t* back, const uint16_t* host_pool, const int32_t* bt, int n_bt,
                      size_t pool_elems, size_t layer_elems, size_t row)
{
    CHECK_HIP(hipMemcpy(back, pool, pool_elems * 2, hipMemcpyDeviceToHost));
    size_t restored = 0;
    for (int l = 0; l < L; ++l) {
        for (int kv = 0; kv < 2; ++kv) {
            const size_t base = (size_t)(2 * l + kv) * layer_elems;
            for (int page = 0; page < NUM_PAGES; ++page) {
                for (int r = 0; r < P; ++r) {
                    /* token of this row, if the sequence owns it */
                    int token = -1;
                    for (int i = 0; i < n_bt; ++i)
                        if (bt[i] == page && i * P + r < TOKENS) token = i * P + r;
                    const size_t at = base + ((size_t)page * P + r) * row;
                    for (size_t e = 0; e < row; ++e) {
                        const uint16_t want = token >= 0 ? host_pool[at + e] : 0;
                        if (back[at + e] != want) {
                            fprintf(stderr, "layer %d kv %d page %d row %d elem %zu: %u, want %u\n", l, kv, page, r,
                                    e, back[at + e], want);
                            return 7;
                        }
                    }
                    restored += token >= 0;
                }
            }
        }
    }
    if (restored != (size_t)L * 2 * TOKENS) { fprintf(stderr, "%zu rows restored\n", restored); return 7; }
    return 0;
}

int main(void)
{
    const size_t row = (size_t)H * D;                       /* bf16 elements per token row */
    const size_t layer_elems = (size_t)NUM_PAGES * P * row; /* one layer's K (or V) pool */
    const int n_bt = (TOKENS + P - 1) / P;                  /* 19 pages */

    /* pool: [L][K, V][NUM_PAGES][P][H*D] bf16, every element a distinct pattern */
    const size_t pool_elems = (size_t)L * 2 * layer_elems;
    uint16_t* host_pool = (uint16_t*)malloc(pool_elems * 2);
    uint16_t* back = (uint16_t*)malloc(pool_elems * 2);
    if (!host_pool || !back) return 4;
    for (size_t i = 0; i < pool_elems; ++i) host_pool[i] = (uint16_t)(i * 2654435761u >> 7);

    /* block table: pages 3, 8, 13, ... (a stride coprime with the pool size keeps them distinct) */
    int32_t bt[32];
    for (int i = 0; i < n_bt; ++i) bt[i] = (3 + 5 * i) % NUM_PAGES;

    uint16_t* pool = NULL;
    int32_t* d_bt = NULL;
    CHECK_HIP(hipMalloc((void**)&pool, pool_elems * 2));
    CHECK_HIP(hipMalloc((void**)&d_bt, sizeof bt));
    CHECK_HIP(hipMemcpy(pool, host_pool, pool_elems * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_bt, bt, sizeof bt, hipMemcpyHostToDevice));

    uint64_t k_addr[L], v_addr[L];
    for (int l = 0; l < L; ++l) {
        k_addr[l] = (uint64_t)(uintptr_t)(pool + (size_t)(2 * l) * layer_elems);
        v_addr[l] = (uint64_t)(uintptr_t)(pool + (size_t)(2 * l + 1) * layer_elems);
    }
    uint64_t *d_k = NULL, *d_v = NULL;
    CHECK_HIP(hipMalloc((void**)&d_k, sizeof k_addr));
    CHECK_HIP(hipMalloc((void**)&d_v, sizeof v_addr));
    CHECK_HIP(hipMemcpy(d_k, k_addr, sizeof k_addr, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_v, v_addr, sizeof v_addr, hipMemcpyHostToDevice));

    kv_paged paged = {L, H, D, P, C, NUM_PAGES, d_k, d_v};

    /* chunk buffers, sized by the library */
    const int64_t n_chunks = kv_num_chunks(&paged, 0, TOKENS);
    if (n_chunks != 2) { fprintf(stderr, "expected 2 chunks, got %lld\n", (long long)n_chunks); return 5; }
    uint64_t chunk_addr[2];
    for (int c = 0; c < 2; ++c) {
        const int64_t n_c = c == 0 ? C : TOKENS - C;
        const size_t bytes = kv_chunk_bytes(&paged, n_c, KV_FMT_BF16);
        if (bytes != (size_t)L * 2 * n_c * row * 2) { fprintf(stderr, "chunk %d: %zu bytes\n", c, bytes); return 5; }
        void* p = NULL;
        CHECK_HIP(hipMalloc(&p, bytes));
        chunk_addr[c] = (uint64_t)(uintptr_t)p;
    }
    uint64_t* d_chunks = NULL;
    CHECK_HIP(hipMalloc((void**)&d_chunks, sizeof chunk_addr));
    CHECK_HIP(hipMemcpy(d_chunks, chunk_addr, sizeof chunk_addr, hipMemcpyHostToDevice));

    kv_seq seq = {d_bt, n_bt, 0, TOKENS, d_chunks};
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));

    CHECK_KV(kv_store_chunks(&paged, &seq, 1, KV_FMT_BF16, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    /* the same store through its address plan (kv_store_chunks_ws): the
     * chunks, cleared in between, must come out byte for byte the same */
    const size_t chunk_bytes[2] = {kv_chunk_bytes(&paged, C, KV_FMT_BF16), kv_chunk_bytes(&paged, TOKENS - C, KV_FMT_BF16)};
    uint8_t* saved[2];
    for (int c = 0; c < 2; ++c) {
        saved[c] = (uint8_t*)malloc(chunk_bytes[c]);
        if (!saved[c]) return 4;
        CHECK_HIP(hipMemcpy(saved[c], (void*)(uintptr_t)chunk_addr[c], chunk_bytes[c], hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemset((void*)(uintptr_t)chunk_addr[c], 0xEE, chunk_bytes[c]));
    }
    const size_t ws_bytes = kv_store_workspace_bytes(&paged, &seq, 1, KV_FMT_BF16);
    /* 32 bytes per page unit (every layer's K and V pages), rounded up to 256 */
    if (ws_bytes != ((size_t)n_bt * L * 2 * 32 + 255) / 256 * 256) { fprintf(stderr, "store workspace %zu bytes\n", ws_bytes); return 5; }
    void* ws = NULL;
    CHECK_HIP(hipMalloc(&ws, ws_bytes));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_KV(kv_store_chunks_ws(&paged, &seq, 1, KV_FMT_BF16, ws, ws_bytes, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    for (int c = 0; c < 2; ++c) {
        uint8_t* again = (uint8_t*)malloc(chunk_bytes[c]);
        if (!again) return 4;
        CHECK_HIP(hipMemcpy(again, (void*)(uintptr_t)chunk_addr[c], chunk_bytes[c], hipMemcpyDeviceToHost));
        if (memcmp(again, saved[c], chunk_bytes[c]) != 0) { fprintf(stderr, "chunk %d differs after the planned store\n", c); return 6; }
        free(again);
        free(saved[c]);
    }
    CHECK_HIP(hipFree(ws));
    CHECK_HIP(hipMemset(pool, 0, pool_elems * 2));
    CHECK_HIP(hipDeviceSynchronize());

    const uint8_t mask[2] = {1, 1};
    const uint8_t* masks[1] = {mask};
    int64_t out_tokens = -1;
    CHECK_KV(kv_retrieve_chunks(&paged, &seq, masks, 1, KV_FMT_BF16, &out_tokens, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    if (out_tokens != TOKENS) { fprintf(stderr, "out_tokens %lld\n", (long long)out_tokens); return 6; }
    const int faults = kv_take_faults();
    if (faults != 0) { fprintf(stderr, "fault bits %d\n", faults); return 6; }

    int rc = check_pool(pool, back, host_pool, bt, n_bt, pool_elems, layer_elems, row);
    if (rc != 0) return rc;

    /* the same retrieve layer by layer (the boundary's kv_retrieve_layer),
     * each layer's event recorded on the stream after its scatter; the host
     * waits on the last one */
    CHECK_HIP(hipMemset(pool, 0, pool_elems * 2));
    CHECK_HIP(hipDeviceSynchronize());
    hipEvent_t done[L];
    for (int l = 0; l < L; ++l) CHECK_HIP(hipEventCreateWithFlags(&done[l], hipEventDisableTiming));
    for (int l = 0; l < L; ++l) CHECK_KV(kv_retrieve_layer(&paged, &seq, masks, 1, KV_FMT_BF16, l, stream, done[l]));
    CHECK_HIP(hipEventSynchronize(done[L - 1]));
    rc = check_pool(pool, back, host_pool, bt, n_bt, pool_elems, layer_elems, row);
    if (rc != 0) return rc;
    if (kv_take_faults() != 0) { fprintf(stderr, "fault bits after the layer calls\n"); return 6; }

    /* in pool-address order with a workspace (kv_retrieve_chunks_ws), then
     * with the library's own scratch (kv_retrieve_chunks_noalloc) */
    const size_t rws_bytes = kv_retrieve_workspace_bytes(&paged);
    /* the inverse page map and the sorted list, one 32-bit word per pool page each, each rounded up to 256 */
    if (rws_bytes != 2 * (((size_t)NUM_PAGES * 4 + 255) / 256 * 256)) { fprintf(stderr, "retrieve workspace %zu bytes\n", rws_bytes); return 5; }
    void* rws = NULL;
    CHECK_HIP(hipMalloc(&rws, rws_bytes));
    for (int form = 0; form < 2; ++form) {
        CHECK_HIP(hipMemset(pool, 0, pool_elems * 2));
        CHECK_HIP(hipDeviceSynchronize());
        out_tokens = -1;
        if (form == 0)
            CHECK_KV(kv_retrieve_chunks_ws(&paged, &seq, masks, 1, KV_FMT_BF16, &out_tokens, rws, rws_bytes, stream));
        else
            CHECK_KV(kv_retrieve_chunks_noalloc(&paged, &seq, masks, 1, KV_FMT_BF16, &out_tokens, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        if (out_tokens != TOKENS) { fprintf(stderr, "ordered form %d: out_tokens %lld\n", form, (long long)out_tokens); return 6; }
        rc = check_pool(pool, back, host_pool, bt, n_bt, pool_elems, layer_elems, row);
        if (rc != 0) return rc;
    }
    CHECK_HIP(hipFree(rws));

    /* every layer in one call on two streams (kv_retrieve_layers with a
     * second stream: odd layers on it, joined back into the first); the
     * host waits on the stream, then checks each layer's event has fired */
    hipStream_t alt;
    CHECK_HIP(hipStreamCreate(&alt));
    CHECK_HIP(hipMemset(pool, 0, pool_elems * 2));
    CHECK_HIP(hipDeviceSynchronize());
    out_tokens = -1;
    CHECK_KV(kv_retrieve_layers(&paged, &seq, masks, 1, KV_FMT_BF16, 0, L, NULL, &out_tokens, stream, alt, done));
    CHECK_HIP(hipStreamSynchronize(stream));
    for (int l = 0; l < L; ++l)
        if (hipEventQuery(done[l]) != hipSuccess) { fprintf(stderr, "layer %d event not complete after the join\n", l); return 6; }
    if (out_tokens != TOKENS) { fprintf(stderr, "layer range: out_tokens %lld\n", (long long)out_tokens); return 6; }
    rc = check_pool(pool, back, host_pool, bt, n_bt, pool_elems, layer_elems, row);
    if (rc != 0) return rc;

    /* the store of every layer in one call on two streams (kv_store_layers)
     * into cleared chunks, then a retrieve from them */
    for (int c = 0; c < 2; ++c) CHECK_HIP(hipMemset((void*)(uintptr_t)chunk_addr[c], 0xEE, chunk_bytes[c]));
    CHECK_HIP(hipMemcpy(pool, host_pool, pool_elems * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_KV(kv_store_layers(&paged, &seq, 1, KV_FMT_BF16, 0, L, NULL, stream, alt, NULL, done));
    CHECK_HIP(hipMemsetAsync(pool, 0, pool_elems * 2, stream));
    out_tokens = -1;
    CHECK_KV(kv_retrieve_chunks(&paged, &seq, masks, 1, KV_FMT_BF16, &out_tokens, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    if (out_tokens != TOKENS) { fprintf(stderr, "after the layer-range store: out_tokens %lld\n", (long long)out_tokens); return 6; }
    rc = check_pool(pool, back, host_pool, bt, n_bt, pool_elems, layer_elems, row);
    if (rc != 0) return rc;
    if (kv_take_faults() != 0) { fprintf(stderr, "fault bits after the ordered and layer-range calls\n"); return 6; }
    CHECK_HIP(hipStreamDestroy(alt));
    for (int l = 0; l < L; ++l) CHECK_HIP(hipEventDestroy(done[l]));
    printf("C ABI round trip: %d tokens x %d layers x K,V stored alike with and without the address plan, "
           "restored bit for bit in one call and layer by layer; other rows untouched; the same in pool-address "
           "order (workspace, no-allocation), layer ranges on two streams both ways\n", TOKENS, L);
    return 0;
}
