// kvmove.hip -- host side of libkvmove.so: argument checks, unit planning and
// launches for the C ABI declared in include/kvmove.h.
//
// Every entry point validates everything it can see on the host first and
// returns an error without launching anything; the device-side contents
// (page ids, chunk addresses) are checked by the kernels themselves.
#include "kvmove.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kv_cachegen.hpp"
#include "kv_copy.hpp"
#include "kv_fp8.hpp"
#include "kv_move_bf16.hpp"
#include "kv_order.hpp"

namespace {

using namespace kvmove;

// Most workgroups of `block` threads one launch takes (gridDim.x * blockDim.x
// must stay below 2^32).
int64_t max_blocks(int block) { return ((int64_t(1) << 32) - 1) / block; }

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok()
{
    g_last_error.clear();
    return KV_OK;
}

int check_paged(const kv_paged* p)
{
    if (p == nullptr) return fail(KV_EINVAL, "paged is NULL");
    if (p->num_layers <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0)
        return fail(KV_EINVAL, "num_layers, num_kv_heads and head_dim must be > 0 (got %d, %d, %d)",
                    p->num_layers, p->num_kv_heads, p->head_dim);
    const int64_t width = int64_t(p->num_kv_heads) * p->head_dim;
    if (width % 8 != 0 || width > (int64_t(1) << 30))
        return fail(KV_EINVAL, "num_kv_heads*head_dim = %lld must be a multiple of 8 (16-byte rows)",
                    (long long)width);
    if (p->page_size <= 0 || p->chunk_size <= 0 || p->chunk_size % p->page_size != 0)
        return fail(KV_EINVAL, "page_size (%d) and chunk_size (%d) must be > 0, chunk a multiple of page",
                    p->page_size, p->chunk_size);
    // the kernels size a page, and a chunk's section of one layer's K or V,
    // in 32-bit byte counts
    if (int64_t(p->chunk_size) * width * 2 > (int64_t(1) << 31))
        return fail(KV_EINVAL, "chunk_size * num_kv_heads * head_dim * 2 = %lld bytes: one layer's K or V section "
                    "of a chunk must stay within 2^31 bytes", (long long)(int64_t(p->chunk_size) * width * 2));
    if (p->num_pages <= 0) return fail(KV_EINVAL, "num_pages must be > 0");
    if (p->k_pages == nullptr || p->v_pages == nullptr)
        return fail(KV_EINVAL, "k_pages / v_pages address arrays are NULL");
    return KV_OK;
}

int check_fmt(int fmt)
{
    if (fmt == KV_FMT_CACHEGEN_INT8)
        return fail(KV_EINVAL, "format %d needs bin counts: use the *_cachegen entry points", fmt);
    if (fmt != KV_FMT_BF16 && fmt != KV_FMT_FP8_E4M3_SCALED && fmt != KV_FMT_FP8_E5M2_SCALED &&
        fmt != KV_FMT_K16_V8)
        return fail(KV_EINVAL, "unknown format %d", fmt);
    return KV_OK;
}

// How a format holds K and V in a chunk: bytes per element of each part
// and float32 scales per layer (one per quantised part).
struct Layout {
    uint32_t elt_k, elt_v, n_scaled;
};

Layout layout_of(int fmt)
{
    switch (fmt) {
    case KV_FMT_BF16: return {2, 2, 0};
    case KV_FMT_FP8_E4M3_SCALED:
    case KV_FMT_FP8_E5M2_SCALED: return {1, 1, 2};
    default: return {2, 1, 1};        // KV_FMT_K16_V8
    }
}

int check_seq(const kv_paged* p, const kv_seq* s, int i)
{
    if (s->tok_start < 0 || s->tok_end < s->tok_start)
        return fail(KV_EINVAL, "seq %d: need 0 <= tok_start <= tok_end (got %lld, %lld)", i,
                    (long long)s->tok_start, (long long)s->tok_end);
    if (s->tok_start % p->chunk_size != 0)
        return fail(KV_EINVAL, "seq %d: tok_start %lld is not a multiple of chunk_size %d", i,
                    (long long)s->tok_start, p->chunk_size);
    if (s->n_bt < 0 || s->n_bt > INT32_MAX)
        return fail(KV_EINVAL, "seq %d: n_bt %lld outside [0, 2^31)", i, (long long)s->n_bt);
    if (s->tok_end > s->n_bt * p->page_size)
        return fail(KV_ERANGE, "seq %d: tok_end %lld beyond the block table (%lld pages of %d)", i,
                    (long long)s->tok_end, (long long)s->n_bt, p->page_size);
    if (s->tok_end > s->tok_start && (s->block_table == nullptr || s->chunks == nullptr))
        return fail(KV_EINVAL, "seq %d: block_table / chunks is NULL", i);
    return KV_OK;
}

int check_seqs(const kv_paged* p, const kv_seq* seqs, int n_seqs)
{
    if (n_seqs < 0) return fail(KV_EINVAL, "n_seqs < 0");
    if (n_seqs > 0 && seqs == nullptr) return fail(KV_EINVAL, "seqs is NULL");
    for (int i = 0; i < n_seqs; ++i) {
        int rc = check_seq(p, &seqs[i], i);
        if (rc != KV_OK) return rc;
    }
    return KV_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Leading hit chunks: first 0 in the mask ends the hits.
int64_t hit_chunks(const uint8_t* mask, int64_t n_chunks)
{
    int64_t c = 0;
    while (c < n_chunks && mask[c] != 0) ++c;
    return c;
}

enum class Unit { Page, Group };

using KernelFn = const void*;

// One kernel launch of an operation: the kernel, its shape, and the K/V
// parts of the chunk it moves.
struct Launch {
    KernelFn kernel;
    int block;        // threads per workgroup
    int tile_bytes;   // bytes of page-side data per workgroup (0: one workgroup per unit)
    Unit unit;
    uint32_t kv0, n_kv;
    KernelFn sorted;  // the scatter kernel in pool-address order (retrieves only; else nullptr)
    bool seq_lut;     // the kernel takes MoveArgsLut (the bf16 movers)
};

// The bf16 movers' arguments: a with its sequence lookup table over the
// launch's `total` units (lut[k] = the sequence holding unit k << lut_shift).
MoveArgsLut with_seq_lut(const MoveArgs& a, int64_t total)
{
    MoveArgsLut al{};
    al.m = a;
    uint32_t shift = 0;
    while ((uint64_t(total - 1) >> shift) >= uint64_t(kSeqLut)) ++shift;
    al.lut_shift = shift;
    uint32_t s = 0;
    for (int k = 0; k < kSeqLut; ++k) {
        const uint64_t item = uint64_t(k) << shift;
        while (s + 1 < a.n_seqs && item >= a.seq[s + 1].item_begin) ++s;
        al.lut[k] = uint8_t(s);
    }
    return al;
}

// The launches of one store or retrieve: one, or one per part when K and V
// are held differently.
struct Plan {
    Launch part[2];
    int n;
};

// Packs up to kMaxSeqs non-empty sequences per launch, keeping every launch
// within max_blocks workgroups (the kernels index units in 32 bits), and
// calls flush(args, units) for each launch.  n_tok[i] is the token count
// moved for sequence i (from its tok_start).
template <class Flush>
int pack_units(const Launch& L, const Layout& lay, const kv_paged* p, const kv_seq* seqs, const int64_t* n_tok,
               int n_seqs, int32_t layer0, int32_t n_layers, Flush&& flush)
{
    const int tile_bytes = L.tile_bytes;
    const Unit unit = L.unit;
    MoveArgs a{};
    a.kv0 = L.kv0;
    a.n_kv = L.n_kv;
    a.elt_k = lay.elt_k;
    a.elt_v = lay.elt_v;
    a.n_scaled = lay.n_scaled;
    a.k_pages = reinterpret_cast<uint64_t>(p->k_pages);
    a.v_pages = reinterpret_cast<uint64_t>(p->v_pages);
    a.num_pages = p->num_pages;
    a.width = uint32_t(p->num_kv_heads * p->head_dim);
    a.page_size = uint32_t(p->page_size);
    a.chunk_size = uint32_t(p->chunk_size);
    a.pages_per_chunk = uint32_t(p->chunk_size / p->page_size);
    a.units_per_chunk = unit == Unit::Page ? uint32_t(n_layers) * L.n_kv * a.pages_per_chunk
                                           : uint32_t(n_layers) * L.n_kv;
    a.num_layers = uint32_t(p->num_layers);
    a.layer0 = uint32_t(layer0);
    a.n_layers = uint32_t(n_layers);
    const int64_t page_bytes = int64_t(p->page_size) * a.width * 2;
    a.tiles = tile_bytes > 0 ? uint32_t(ceil_div(page_bytes, tile_bytes)) : 1u;
    const int64_t most = max_blocks(L.block);
    if (int64_t(a.tiles) > most) return fail(KV_EINVAL, "page too large for one launch");
    const int64_t max_units = most / a.tiles;

    int64_t total = 0;
    a.n_seqs = 0;
    for (int i = 0; i < n_seqs; ++i) {
        if (n_tok[i] <= 0) continue;
        const int64_t units = unit == Unit::Page
                                  ? ceil_div(n_tok[i], p->page_size) * n_layers * L.n_kv
                                  : ceil_div(n_tok[i], p->chunk_size) * n_layers * L.n_kv;
        if (units > max_units)
            return fail(KV_EINVAL, "seq %d: %lld work units exceed one launch", i, (long long)units);
        if (a.n_seqs == kMaxSeqs || total + units > max_units) {
            a.item_base = 0;
            a.total_tiles = uint32_t(total * a.tiles);
            int rc = flush(a, total);
            if (rc != KV_OK) return rc;
            a.n_seqs = 0;
            total = 0;
        }
        SeqArg& s = a.seq[a.n_seqs++];
        s.bt = reinterpret_cast<uint64_t>(seqs[i].block_table);
        s.chunks = reinterpret_cast<uint64_t>(seqs[i].chunks);
        s.first_page = uint32_t(seqs[i].tok_start / p->page_size);
        s.n_full = uint32_t(n_tok[i] / p->chunk_size);
        s.tail_tokens = uint32_t(n_tok[i] % p->chunk_size);
        s.item_begin = uint32_t(total);
        total += units;
    }
    if (a.n_seqs > 0) {
        a.item_base = 0;
        a.total_tiles = uint32_t(total * a.tiles);
        return flush(a, total);
    }
    return KV_OK;
}

int launch_units(const Launch& L, const Layout& lay, const kv_paged* p, const kv_seq* seqs,
                 const int64_t* n_tok, int n_seqs, int32_t layer0, int32_t n_layers, hipStream_t stream,
                 int32_t max_workgroups = 0, const uint8_t (*cg_qmax)[kCgMaxLayers] = nullptr)
{
    const KernelFn kernel = L.kernel;
    const int block = L.block;
    const Unit unit = L.unit;
    auto flush = [&](MoveArgs& a, int64_t total) -> int {
        int64_t grid = a.total_tiles;
        // only the tiled movers walk runs of tiles; group kernels need one
        // workgroup per group
        if (unit == Unit::Page && max_workgroups > 0 && grid > max_workgroups) grid = max_workgroups;
        hipError_t e;
        if (cg_qmax != nullptr) {            // CacheGen kernels take the bins beside the move arguments
            CgArgs ca{};
            ca.m = a;
            for (int kv = 0; kv < 2; ++kv)
                for (int l = 0; l < kCgMaxLayers; ++l) ca.qmax[kv][l] = cg_qmax[kv][l];
            void* args[] = {&ca};
            e = hipLaunchKernel(kernel, dim3(unsigned(grid)), dim3(block), args, 0, stream);
        } else if (L.seq_lut) {
            MoveArgsLut al = with_seq_lut(a, total);
            void* args[] = {&al};
            e = hipLaunchKernel(kernel, dim3(unsigned(grid)), dim3(block), args, 0, stream);
        } else {
            void* args[] = {&a};
            e = hipLaunchKernel(kernel, dim3(unsigned(grid)), dim3(block), args, 0, stream);
        }
        if (e != hipSuccess) return fail(KV_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
        return KV_OK;
    };
    return pack_units(L, lay, p, seqs, n_tok, n_seqs, layer0, n_layers, flush);
}

// bf16 mover launch; `capped` (a workgroup cap is given) selects the
// 256-thread shape, so a cap keeps its meaning in threads; `whole` (a
// scatter over every layer at once, uncapped) selects its store policy.
Launch bf16_launch(bool to_chunk, uint32_t kv0, uint32_t n_kv, bool capped, bool whole = false)
{
    if (capped) {
        constexpr int B = kMoveBlockCapped;
        const KernelFn k =
            to_chunk ? reinterpret_cast<KernelFn>(&move_bf16<true, B, kMoveVpt, kGatherAuxLoad, kGatherAuxStore>)
                     : reinterpret_cast<KernelFn>(&move_bf16<false, B, kMoveVpt, kScatterAuxLoad, kScatterAuxStore>);
        return {k, B, B * kMoveVpt * 16, Unit::Page, kv0, n_kv, nullptr, true};
    }
    constexpr int B = kMoveBlock;
    const KernelFn k =
        to_chunk ? reinterpret_cast<KernelFn>(&move_bf16<true, B, kMoveVpt, kGatherAuxLoad, kGatherAuxStore>)
        : whole  ? reinterpret_cast<KernelFn>(&move_bf16<false, B, kMoveVpt, kScatterAuxLoad, kScatterAuxStoreWhole>)
                 : reinterpret_cast<KernelFn>(&move_bf16<false, B, kMoveVpt, kScatterAuxLoad, kScatterAuxStore>);
    const KernelFn sorted =
        to_chunk ? nullptr
                 : reinterpret_cast<KernelFn>(&scatter_sorted<B, kMoveVpt, kScatterAuxLoad, kScatterAuxStore>);
    return {k, B, B * kMoveVpt * 16, Unit::Page, kv0, n_kv, sorted, true};
}

// Gather + quantise: a whole (chunk, layer, K/V) group on chip when it fits,
// else two passes.
Launch quantise_launch(const kv_paged* p, bool e5m2, uint32_t kv0, uint32_t n_kv)
{
    const int64_t group_vectors = int64_t(p->chunk_size) * p->num_kv_heads * p->head_dim / 8;
    if (group_vectors <= int64_t(kOnchipMaxVectors) && p->chunk_size / p->page_size <= kOnchipMaxPages) {
        const KernelFn k = e5m2 ? reinterpret_cast<KernelFn>(&store_fp8_onchip<true>)
                                : reinterpret_cast<KernelFn>(&store_fp8_onchip<false>);
        return {k, kOnchipBlock, 0, Unit::Group, kv0, n_kv, nullptr, true};
    }
    const KernelFn k = e5m2 ? reinterpret_cast<KernelFn>(&store_fp8<kFp8StoreBlock, kFp8StoreUnroll, true>)
                            : reinterpret_cast<KernelFn>(&store_fp8<kFp8StoreBlock, kFp8StoreUnroll, false>);
    return {k, kFp8StoreBlock, 0, Unit::Group, kv0, n_kv, nullptr, true};
}

template <int B, int V>
Launch dequantise_shape(bool e5m2, uint32_t kv0, uint32_t n_kv, bool sorted)
{
    const KernelFn k = e5m2 ? reinterpret_cast<KernelFn>(&retrieve_fp8<B, V, true>)
                            : reinterpret_cast<KernelFn>(&retrieve_fp8<B, V, false>);
    const KernelFn ks = !sorted ? nullptr
                        : e5m2  ? reinterpret_cast<KernelFn>(&retrieve_fp8_sorted<B, V, true>)
                                : reinterpret_cast<KernelFn>(&retrieve_fp8_sorted<B, V, false>);
    return {k, B, B * V * 16, Unit::Page, kv0, n_kv, ks, true};
}

// Scatter + dequantise.  The chunk-major and the pool-address-ordered
// launches take one-wave workgroups (4 KiB and 2 KiB tiles); a capped launch
// takes 256 threads x 8 KiB and is never ordered.
Launch dequantise_launch(bool e5m2, uint32_t kv0, uint32_t n_kv, bool capped, bool ordered)
{
    if (capped)
        return dequantise_shape<kFp8RetrieveBlockCapped, kFp8RetrieveVptCapped>(e5m2, kv0, n_kv, false);
    if (ordered)
        return dequantise_shape<kFp8RetrieveBlockSorted, kFp8RetrieveVptSorted>(e5m2, kv0, n_kv, true);
    return dequantise_shape<kFp8RetrieveBlock, kFp8RetrieveVpt>(e5m2, kv0, n_kv, false);
}

Plan gather_plan(const kv_paged* p, int fmt, bool capped)
{
    switch (fmt) {
    case KV_FMT_BF16: return {{bf16_launch(true, 0, 2, capped)}, 1};
    case KV_FMT_FP8_E4M3_SCALED: return {{quantise_launch(p, false, 0, 2)}, 1};
    case KV_FMT_FP8_E5M2_SCALED: return {{quantise_launch(p, true, 0, 2)}, 1};
    default: return {{bf16_launch(true, 0, 1, capped), quantise_launch(p, false, 1, 1)}, 2};   // K16_V8
    }
}

// The launches of a retrieve; `whole`: every layer in one uncapped launch
// (the chunk-major scatter's store policy, kScatterAuxStoreWhole).
Plan scatter_plan(int fmt, bool capped, bool ordered, bool whole = false)
{
    switch (fmt) {
    case KV_FMT_BF16: return {{bf16_launch(false, 0, 2, capped, whole)}, 1};
    case KV_FMT_FP8_E4M3_SCALED: return {{dequantise_launch(false, 0, 2, capped, ordered)}, 1};
    case KV_FMT_FP8_E5M2_SCALED: return {{dequantise_launch(true, 0, 2, capped, ordered)}, 1};
    default:                                                                                      // K16_V8
        return {{bf16_launch(false, 0, 1, capped, whole), dequantise_launch(false, 1, 1, capped, ordered)}, 2};
    }
}

// The bf16 gather (launch L of a store plan, uncapped) through an address
// plan in `plan` (device memory of at least kPlanEntryBytes per page unit of
// the largest packed launch): per launch, build_gather_plan writes the plan,
// then gather_planned moves 4 KiB tiles over it.
int gather_through_plan(const Launch& L, const Layout& lay, const kv_paged* p, const kv_seq* seqs,
                        const int64_t* n_tok, int n_seqs, uint64_t plan, hipStream_t stream)
{
    Launch P = L;
    P.block = kPlanBlock;
    P.tile_bytes = kPlanBlock * kPlanVpt * 16;
    auto flush = [&](MoveArgs& a, int64_t total) -> int {
        MoveArgsLut al = with_seq_lut(a, total);
        uint64_t plan_a = plan;
        uint32_t n = uint32_t(total);
        void* build_args[] = {&al, &plan_a, &n};
        hipError_t e = hipLaunchKernel(reinterpret_cast<KernelFn>(&build_gather_plan),
                                       dim3(unsigned(ceil_div(total, kPlanBuildBlock))), dim3(kPlanBuildBlock),
                                       build_args, 0, stream);
        if (e == hipSuccess) {
            const uint64_t* plan_p = reinterpret_cast<const uint64_t*>(plan);
            uint32_t tiles = a.tiles;
            void* move_args[] = {&plan_p, &tiles};
            e = hipLaunchKernel(
                reinterpret_cast<KernelFn>(&gather_planned<kPlanBlock, kPlanVpt, kGatherAuxLoad, kGatherAuxStore>),
                dim3(a.total_tiles), dim3(kPlanBlock), move_args, 0, stream);
        }
        if (e != hipSuccess) return fail(KV_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
        return KV_OK;
    };
    return pack_units(P, lay, p, seqs, n_tok, n_seqs, 0, p->num_layers, flush);
}

// The page units a store's bf16 parts move (the plan's entries): per
// sequence ceil(tokens / P) pages of each layer's K and V (K only for
// KV_FMT_K16_V8; none for the fp8 formats).
int64_t store_plan_units(const kv_paged* p, const int64_t* n_tok, int n_seqs, int fmt)
{
    const int64_t parts = fmt == KV_FMT_BF16 ? 2 : fmt == KV_FMT_K16_V8 ? 1 : 0;
    int64_t pages = 0;
    for (int i = 0; i < n_seqs; ++i) pages += ceil_div(n_tok[i], p->page_size);
    return pages * p->num_layers * parts;
}

int run_plan(const Plan& plan, int fmt, const kv_paged* p, const kv_seq* seqs, const int64_t* n_tok,
             int n_seqs, int32_t layer0, int32_t n_layers, hipStream_t stream, int32_t max_workgroups)
{
    const Layout lay = layout_of(fmt);
    for (int k = 0; k < plan.n; ++k) {
        const int rc = launch_units(plan.part[k], lay, p, seqs, n_tok, n_seqs, layer0, n_layers, stream,
                                    max_workgroups);
        if (rc != KV_OK) return rc;
    }
    return KV_OK;
}

// Workspace of the pool-address-ordered scatter: the inverse page map, then
// the sorted list, num_pages words each, 256-byte aligned.
int64_t ordered_half_bytes(int64_t num_pages) { return ceil_div(num_pages * 4, 256) * 256; }

// Scatter launch L (its `sorted` kernel) of the tokens n_tok[i] in
// pool-address order (kv_order.hpp): per packed launch, the page list is
// built in the workspace, then the ordered kernel runs over it.
int retrieve_ordered(const Launch& L, const Layout& lay, const kv_paged* p, const kv_seq* seqs,
                     const int64_t* n_tok, int n_seqs, int32_t layer0, int32_t n_layers, void* workspace,
                     hipStream_t stream, const uint8_t (*cg_qmax)[kCgMaxLayers] = nullptr)
{
    const uint64_t inv = reinterpret_cast<uint64_t>(workspace);
    const uint64_t list = inv + uint64_t(ordered_half_bytes(p->num_pages));
    const uint32_t num_pages = uint32_t(p->num_pages);
    auto flush = [&](MoveArgs& a, int64_t total) -> int {
        const int64_t n_list = total / (int64_t(n_layers) * a.n_kv);      // pages moved by this launch
        for (uint32_t s = 0; s < a.n_seqs; ++s)
            if (a.seq[s].n_full * a.pages_per_chunk + ceil_div(a.seq[s].tail_tokens, a.page_size) > kPageIndexMask)
                return fail(KV_EINVAL, "a sequence moves 2^26 pages or more: retrieve without a workspace");
        uint32_t none = kNoEntry, np = num_pages, nl = uint32_t(n_list);
        uint64_t inv_a = inv, list_a = list;
        hipError_t e = hipSuccess;
        if (num_pages <= kSmallPoolPages) {     // one launch, the inverse map in LDS
            void* args[] = {&a, &list_a, &nl, &np};
            e = hipLaunchKernel(reinterpret_cast<KernelFn>(&order_pages_small), dim3(1), dim3(kCompactBlock), args, 0,
                                stream);
        } else {
            const unsigned fill_grid = unsigned(std::min<int64_t>(ceil_div(num_pages, 256), 4096));
            void* fill_args[] = {&inv_a, &np, &none};
            e = hipLaunchKernel(reinterpret_cast<KernelFn>(&fill_u32), dim3(fill_grid), dim3(256), fill_args, 0, stream);
            if (e == hipSuccess) {
                void* inv_args[] = {&a, &inv_a, &nl};
                e = hipLaunchKernel(reinterpret_cast<KernelFn>(&invert_pages), dim3(unsigned(ceil_div(n_list, 256))),
                                    dim3(256), inv_args, 0, stream);
            }
            if (e == hipSuccess) {
                void* cmp_args[] = {&inv_a, &np, &list_a, &nl};
                e = hipLaunchKernel(reinterpret_cast<KernelFn>(&compact_pages), dim3(1), dim3(kCompactBlock), cmp_args,
                                    0, stream);
            }
        }
        if (e == hipSuccess) {
            if (cg_qmax != nullptr) {          // CacheGen kernels take the bins beside the move arguments
                CgArgs ca{};
                ca.m = a;
                for (int kv = 0; kv < 2; ++kv)
                    for (int l = 0; l < kCgMaxLayers; ++l) ca.qmax[kv][l] = cg_qmax[kv][l];
                void* sc_args[] = {&ca, &list_a, &nl};
                e = hipLaunchKernel(L.sorted, dim3(a.total_tiles), dim3(L.block), sc_args, 0, stream);
            } else {
                void* sc_args[] = {&a, &list_a, &nl};
                e = hipLaunchKernel(L.sorted, dim3(a.total_tiles), dim3(L.block), sc_args, 0, stream);
            }
        }
        if (e != hipSuccess) return fail(KV_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
        return KV_OK;
    };
    return pack_units(L, lay, p, seqs, n_tok, n_seqs, layer0, n_layers, flush);
}

// Tokens sequence i (s, with its hit mask) gets back: its leading hit
// chunks, from tok_start.
int seq_hit_tokens(const kv_paged* paged, const kv_seq& s, const uint8_t* mask, int i, int64_t* n_tok)
{
    const int64_t n_chunks = ceil_div(s.tok_end - s.tok_start, paged->chunk_size);
    if (n_chunks > 0 && mask == nullptr) return fail(KV_EINVAL, "seq %d: hit_mask entry is NULL", i);
    const int64_t n_hit = n_chunks > 0 ? hit_chunks(mask, n_chunks) : 0;
    const int64_t end = s.tok_start + n_hit * paged->chunk_size;
    *n_tok = (end < s.tok_end ? end : s.tok_end) - s.tok_start;
    return KV_OK;
}

int hit_tokens(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs,
               int64_t* n_tok)
{
    if (n_seqs > 0 && hit_mask == nullptr) return fail(KV_EINVAL, "hit_mask is NULL");
    for (int i = 0; i < n_seqs; ++i) {
        const int rc = seq_hit_tokens(paged, seqs[i], hit_mask[i], i, &n_tok[i]);
        if (rc != KV_OK) return rc;
    }
    return KV_OK;
}

// The ordered scatter's workspace holds one entry per pool page, and its
// sorted list one per page moved; page ids are distinct within a call, so a
// call that moves more pages than the pool holds breaks that rule and is
// refused before anything runs (its list would not fit).
int check_ordered_fits(const kv_paged* p, const int64_t* n_tok, int n_seqs)
{
    int64_t pages = 0;
    for (int i = 0; i < n_seqs; ++i) pages += ceil_div(n_tok[i], p->page_size);
    if (pages > p->num_pages)
        return fail(KV_EINVAL, "the call moves %lld pages but the pool holds %lld: page ids repeat",
                    (long long)pages, (long long)p->num_pages);
    return KV_OK;
}

// Shared body of the retrieve entry points; with a workspace the bf16
// scatter runs in pool-address order.
int retrieve(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs,
             int fmt, int32_t layer0, int32_t n_layers, int64_t* out_tokens, hipStream_t stream,
             int32_t max_workgroups = 0, void* workspace = nullptr)
{
    int64_t small[64];
    int64_t* n_tok = n_seqs <= 64 ? small : new int64_t[n_seqs];
    int rc = hit_tokens(paged, seqs, hit_mask, n_seqs, n_tok);
    if (rc != KV_OK) {
        if (n_tok != small) delete[] n_tok;
        return rc;
    }
    if (workspace != nullptr && max_workgroups == 0) {
        const Plan plan = scatter_plan(fmt, false, true);
        rc = check_ordered_fits(paged, n_tok, n_seqs);
        for (int k = 0; k < plan.n && rc == KV_OK; ++k)
            rc = retrieve_ordered(plan.part[k], layout_of(fmt), paged, seqs, n_tok, n_seqs, layer0, n_layers,
                                  workspace, stream);
    } else
        rc = run_plan(scatter_plan(fmt, max_workgroups > 0, false, max_workgroups == 0 && n_layers == paged->num_layers),
                      fmt, paged, seqs, n_tok, n_seqs, layer0, n_layers, stream, max_workgroups);
    if (rc == KV_OK && out_tokens != nullptr)
        for (int i = 0; i < n_seqs; ++i) out_tokens[i] = n_tok[i];
    if (n_tok != small) delete[] n_tok;
    return rc;
}

// CacheGen bins -> MAX table; rejects what the kernels cannot take.
int cachegen_setup(const kv_paged* p, const int32_t* key_bins, const int32_t* value_bins,
                   uint8_t (*qmax)[kCgMaxLayers], Launch* store, Launch* scatter, Launch* scatter_ordered)
{
    if (key_bins == nullptr || value_bins == nullptr) return fail(KV_EINVAL, "key_bins / value_bins is NULL");
    if (p->num_layers > kCgMaxLayers)
        return fail(KV_EINVAL, "the CacheGen format takes at most %d layers (got %d)", kCgMaxLayers, p->num_layers);
    const int64_t width = int64_t(p->num_kv_heads) * p->head_dim;
    if (width > int64_t(kCgMaxVpl) * 64 * 8)
        return fail(KV_EINVAL, "the CacheGen format takes rows of at most %d elements (got %lld)",
                    kCgMaxVpl * 64 * 8, (long long)width);
    for (int l = 0; l < kCgMaxLayers; ++l) qmax[0][l] = qmax[1][l] = 1;
    for (int l = 0; l < p->num_layers; ++l) {
        const int32_t kb = key_bins[l], vb = value_bins[l];
        if (kb < 4 || kb > 129 || vb < 4 || vb > 129)
            return fail(KV_EINVAL, "layer %d: bin counts must lie in [4, 129] (got %d, %d)", l, kb, vb);
        qmax[0][l] = uint8_t(kb / 2 - 1);
        qmax[1][l] = uint8_t(vb / 2 - 1);
    }
    // rows of the page unit, a whole row per wave: kVpl 16-byte vectors per lane
    const int64_t vpl = (width / 8 + 63) / 64;
    KernelFn ks, kr, ko;
    if (vpl <= 1) {
        ks = reinterpret_cast<KernelFn>(&store_cachegen<1>);
        kr = reinterpret_cast<KernelFn>(&retrieve_cachegen<1>);
        ko = reinterpret_cast<KernelFn>(&retrieve_cachegen_sorted<1>);
    } else if (vpl <= 2) {
        ks = reinterpret_cast<KernelFn>(&store_cachegen<2>);
        kr = reinterpret_cast<KernelFn>(&retrieve_cachegen<2>);
        ko = reinterpret_cast<KernelFn>(&retrieve_cachegen_sorted<2>);
    } else if (vpl <= 4) {
        ks = reinterpret_cast<KernelFn>(&store_cachegen<4>);
        kr = reinterpret_cast<KernelFn>(&retrieve_cachegen<4>);
        ko = reinterpret_cast<KernelFn>(&retrieve_cachegen_sorted<4>);
    } else {
        ks = reinterpret_cast<KernelFn>(&store_cachegen<8>);
        kr = reinterpret_cast<KernelFn>(&retrieve_cachegen<8>);
        ko = reinterpret_cast<KernelFn>(&retrieve_cachegen_sorted<8>);
    }
    // the store and the chunk-major retrieve take one workgroup per page
    // unit; the ordered retrieve one per kCgSortedWaves rows of it
    // (tile_bytes counts page-side bytes), through its sorted kernel only
    const int page_bytes = int(int64_t(p->page_size) * width * 2);
    *store = {ks, kCgBlock, page_bytes, Unit::Page, 0, 2, nullptr};
    *scatter = {kr, kCgBlock, page_bytes, Unit::Page, 0, 2, nullptr};
    *scatter_ordered = {nullptr, kCgSortedWaves * 64, int(kCgSortedWaves * width * 2), Unit::Page, 0, 2, ko};
    return KV_OK;
}

constexpr Layout kCgLayout = {1, 1, 0};     // symbol sections addressed as 1-byte parts

// Scratch of the ordered retrieve for callers that cannot allocate
// (kv_retrieve_chunks_noalloc): the workspace kv_retrieve_chunks_ws takes
// from its caller -- the inverse page map, then the sorted page list, one
// 32-bit word per pool page each -- as one device array per GPU, sized for
// pools of up to kScratchMaxPages pages (8 MiB).  Host code never names the
// array in a kernel argument or a copy: in host code `scratch` is a host-side
// stand-in, and the device address comes from hipGetSymbolAddress, once per
// device (scratch_address).  Every kernel that uses it rewrites what it
// reads (the inverse map is cleared by a kernel before it is filled; the
// list is written whole), so a call does not depend on what the last call
// left there.  Calls that use it concurrently on one GPU race.
constexpr int64_t kScratchMaxPages = int64_t(1) << 20;
__device__ __align__(256) uint32_t scratch[2 * kScratchMaxPages];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];     // device address of `scratch` on each device, once looked up

// Device address of `scratch` on the current device (looked up on the
// device's first call, with that device current).
int scratch_address(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KV_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KV_EINVAL, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(KV_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KV_OK;
}

int check_layers(const kv_paged* p, int32_t layer_begin, int32_t layer_end, const int32_t* max_workgroups)
{
    if (layer_begin < 0 || layer_end > p->num_layers || layer_begin >= layer_end)
        return fail(KV_EINVAL, "layers [%d, %d) not a non-empty range inside [0, %d)", layer_begin, layer_end,
                    p->num_layers);
    if (max_workgroups != nullptr)
        for (int32_t k = 0; k < layer_end - layer_begin; ++k)
            if (max_workgroups[k] < 0) return fail(KV_EINVAL, "max_workgroups[%d] < 0", k);
    return KV_OK;
}

int record(hipEvent_t ev, hipStream_t stream)
{
    if (ev == nullptr) return KV_OK;
    const hipError_t e = hipEventRecord(ev, stream);
    if (e != hipSuccess) return fail(KV_EHIP, "hipEventRecord failed: %s", hipGetErrorString(e));
    return KV_OK;
}

// The streams of a layer-range call: layer k of the range runs on
// lane[k % n].  With an alternate stream (n = 2) the alternate first waits
// for what the caller enqueued on the main stream before the call (fork),
// and the main stream ends waiting for the alternate's last layer (join), so
// work the caller enqueues on the main stream after the call still follows
// every layer, while consecutive layers' kernels, on two streams, may
// overlap: one layer's workgroups start while the last ones of the layer
// before are still finishing.  The fork and join events are the call's own.
struct LayerLanes {
    hipStream_t lane[2];
    int n;
    hipEvent_t join;
};

// Both streams must belong to the current device (the events are made there).
int open_lanes(LayerLanes& ll, hipStream_t main, hipStream_t alt)
{
    ll.lane[0] = ll.lane[1] = main;
    ll.n = 1;
    ll.join = nullptr;
    if (alt == nullptr) return KV_OK;
    if (alt == main) return fail(KV_EINVAL, "alt_stream is the main stream");
    int dev = -1, d_main = -1, d_alt = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipStreamGetDevice(alt, &d_alt);
    if (e == hipSuccess && main != nullptr) e = hipStreamGetDevice(main, &d_main);
    if (e != hipSuccess) return fail(KV_EHIP, "reading the device failed: %s", hipGetErrorString(e));
    if (d_alt != dev || (main != nullptr && d_main != dev))
        return fail(KV_EINVAL, "the streams belong to devices %d and %d, the current device is %d",
                    main != nullptr ? d_main : dev, d_alt, dev);
    hipEvent_t fork = nullptr;
    e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ll.join, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(fork, main);
    if (e == hipSuccess) e = hipStreamWaitEvent(alt, fork, 0);
    if (fork != nullptr) (void)hipEventDestroy(fork);       // released once its wait is done
    if (e != hipSuccess) {
        if (ll.join != nullptr) (void)hipEventDestroy(ll.join);
        ll.join = nullptr;
        return fail(KV_EHIP, "forking onto alt_stream failed: %s", hipGetErrorString(e));
    }
    ll.lane[1] = alt;
    ll.n = 2;
    return KV_OK;
}

// Joins the alternate stream back into the main one (also after a failed
// launch, so the main stream's order holds); returns rc, or the join's error.
int close_lanes(LayerLanes& ll, int rc)
{
    if (ll.n == 1) return rc;
    hipError_t e = hipEventRecord(ll.join, ll.lane[1]);
    if (e == hipSuccess) e = hipStreamWaitEvent(ll.lane[0], ll.join, 0);
    (void)hipEventDestroy(ll.join);
    ll.join = nullptr;
    if (e != hipSuccess && rc == KV_OK) return fail(KV_EHIP, "joining alt_stream failed: %s", hipGetErrorString(e));
    return rc;
}

// Layers [layer_begin, layer_end) of a retrieve, one scatter launch each
// (max_workgroups[k] caps layer_begin + k's grid; NULL: no cap), each
// followed by a record of layer_done[k] -- also when nothing hits -- on
// copy_stream, or alternately on copy_stream and alt_stream (LayerLanes).
// The hit plan is made once for all of them.  Host arguments are checked
// before anything is enqueued.
int retrieve_layers(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs, int fmt,
                    int32_t layer_begin, int32_t layer_end, const int32_t* max_workgroups, int64_t* out_tokens,
                    hipStream_t copy_stream, hipStream_t alt_stream, const hipEvent_t* layer_done)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_fmt(fmt);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc == KV_OK) rc = check_layers(paged, layer_begin, layer_end, max_workgroups);
    if (rc != KV_OK) return rc;
    int64_t small[64];
    int64_t* n_tok = n_seqs <= 64 ? small : new int64_t[n_seqs];
    rc = hit_tokens(paged, seqs, hit_mask, n_seqs, n_tok);
    LayerLanes ll;
    if (rc == KV_OK) rc = open_lanes(ll, copy_stream, alt_stream);
    if (rc == KV_OK) {
        const Plan full = scatter_plan(fmt, false, false), capped = scatter_plan(fmt, true, false);
        for (int32_t l = layer_begin; l < layer_end && rc == KV_OK; ++l) {
            const int32_t k = l - layer_begin, cap = max_workgroups != nullptr ? max_workgroups[k] : 0;
            hipStream_t st = ll.lane[k % ll.n];
            rc = run_plan(cap > 0 ? capped : full, fmt, paged, seqs, n_tok, n_seqs, l, 1, st, cap);
            if (rc == KV_OK && layer_done != nullptr) rc = record(layer_done[k], st);
        }
        rc = close_lanes(ll, rc);
    }
    if (rc == KV_OK && out_tokens != nullptr)
        for (int i = 0; i < n_seqs; ++i) out_tokens[i] = n_tok[i];
    if (n_tok != small) delete[] n_tok;
    return rc == KV_OK ? ok() : rc;
}

// Layers [layer_begin, layer_end) of a store, one gather launch each on
// stream, or alternately on stream and alt_stream (LayerLanes): first a wait
// on wait_before[k] (if given), then the launch, then a record of
// layer_done[k] (if given).
int store_layers(const kv_paged* paged, const kv_seq* seqs, int n_seqs, int fmt, int32_t layer_begin,
                 int32_t layer_end, const int32_t* max_workgroups, hipStream_t stream, hipStream_t alt_stream,
                 const hipEvent_t* wait_before, const hipEvent_t* layer_done)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_fmt(fmt);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc == KV_OK) rc = check_layers(paged, layer_begin, layer_end, max_workgroups);
    if (rc != KV_OK) return rc;
    int64_t small[64];
    int64_t* n_tok = n_seqs <= 64 ? small : new int64_t[n_seqs];
    for (int i = 0; i < n_seqs; ++i) n_tok[i] = seqs[i].tok_end - seqs[i].tok_start;
    LayerLanes ll;
    rc = open_lanes(ll, stream, alt_stream);
    if (rc == KV_OK) {
        const Plan full = gather_plan(paged, fmt, false), capped = gather_plan(paged, fmt, true);
        for (int32_t l = layer_begin; l < layer_end && rc == KV_OK; ++l) {
            const int32_t k = l - layer_begin, cap = max_workgroups != nullptr ? max_workgroups[k] : 0;
            hipStream_t st = ll.lane[k % ll.n];
            if (wait_before != nullptr && wait_before[k] != nullptr) {
                const hipError_t e = hipStreamWaitEvent(st, wait_before[k], 0);
                if (e != hipSuccess) rc = fail(KV_EHIP, "hipStreamWaitEvent failed: %s", hipGetErrorString(e));
            }
            if (rc == KV_OK) rc = run_plan(cap > 0 ? capped : full, fmt, paged, seqs, n_tok, n_seqs, l, 1, st, cap);
            if (rc == KV_OK && layer_done != nullptr) rc = record(layer_done[k], st);
        }
        rc = close_lanes(ll, rc);
    }
    if (n_tok != small) delete[] n_tok;
    return rc == KV_OK ? ok() : rc;
}


}  // namespace

extern "C" {

size_t kv_chunk_bytes(const kv_paged* paged, int64_t n_tokens, kv_fmt fmt)
{
    if (check_paged(paged) != KV_OK) return 0;
    if (n_tokens < 0) {
        fail(KV_EINVAL, "n_tokens < 0");
        return 0;
    }
    if (fmt == KV_FMT_CACHEGEN_INT8) {       // symbols, then one float32 max1 per (layer, K/V, token)
        const int64_t rows = int64_t(paged->num_layers) * 2 * n_tokens;
        return size_t(rows) * paged->num_kv_heads * paged->head_dim + size_t(rows) * sizeof(float);
    }
    if (check_fmt(fmt) != KV_OK) return 0;
    const Layout lay = layout_of(fmt);
    const int64_t part = int64_t(paged->num_layers) * n_tokens * paged->num_kv_heads * paged->head_dim;
    return size_t(part) * (lay.elt_k + lay.elt_v) + size_t(paged->num_layers) * lay.n_scaled * sizeof(float);
}

int64_t kv_num_chunks(const kv_paged* paged, int64_t tok_start, int64_t tok_end)
{
    if (check_paged(paged) != KV_OK) return -1;
    if (tok_start < 0 || tok_end < tok_start) {
        fail(KV_EINVAL, "need 0 <= tok_start <= tok_end");
        return -1;
    }
    return ceil_div(tok_end - tok_start, paged->chunk_size);
}

int kv_store_chunks(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt, hipStream_t stream)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_fmt(fmt);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc != KV_OK) return rc;
    int64_t small[64];
    int64_t* n_tok = n_seqs <= 64 ? small : new int64_t[n_seqs];
    for (int i = 0; i < n_seqs; ++i) n_tok[i] = seqs[i].tok_end - seqs[i].tok_start;
    rc = run_plan(gather_plan(paged, fmt, false), fmt, paged, seqs, n_tok, n_seqs, 0, paged->num_layers, stream, 0);
    if (n_tok != small) delete[] n_tok;
    return rc == KV_OK ? ok() : rc;
}

size_t kv_store_workspace_bytes(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_fmt(fmt);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc != KV_OK) return 0;
    int64_t units = 0;
    for (int i = 0; i < n_seqs; ++i) {
        const int64_t n = seqs[i].tok_end - seqs[i].tok_start;
        units += store_plan_units(paged, &n, 1, fmt);
    }
    ok();
    return size_t(ceil_div(units * kPlanEntryBytes, 256) * 256);
}

int kv_store_chunks_ws(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt, void* workspace,
                       size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_fmt(fmt);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc != KV_OK) return rc;
    int64_t small[64];
    int64_t* n_tok = n_seqs <= 64 ? small : new int64_t[n_seqs];
    for (int i = 0; i < n_seqs; ++i) n_tok[i] = seqs[i].tok_end - seqs[i].tok_start;
    const int64_t need = ceil_div(store_plan_units(paged, n_tok, n_seqs, fmt) * kPlanEntryBytes, 256) * 256;
    if (need > 0 && (workspace == nullptr || int64_t(workspace_bytes) < need ||
                     reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
        rc = fail(KV_EINVAL, "workspace of %lld bytes, 256-byte aligned, needed (got %zu at %p)", (long long)need,
                  workspace_bytes, workspace);
    const Plan plan = gather_plan(paged, fmt, false);
    const Layout lay = layout_of(fmt);
    for (int k = 0; k < plan.n && rc == KV_OK; ++k) {
        const bool bf16 = plan.part[k].kernel ==
                          reinterpret_cast<KernelFn>(&move_bf16<true, kMoveBlock, kMoveVpt, kGatherAuxLoad, kGatherAuxStore>);
        rc = bf16 ? gather_through_plan(plan.part[k], lay, paged, seqs, n_tok, n_seqs,
                                        reinterpret_cast<uint64_t>(workspace), stream)
                  : launch_units(plan.part[k], lay, paged, seqs, n_tok, n_seqs, 0, paged->num_layers, stream);
    }
    if (n_tok != small) delete[] n_tok;
    return rc == KV_OK ? ok() : rc;
}

int kv_store_layer(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt, int32_t layer,
                   int32_t max_workgroups, hipStream_t stream, hipEvent_t layer_done)
{
    return store_layers(paged, seqs, n_seqs, fmt, layer, layer + 1, &max_workgroups, stream, nullptr, nullptr,
                        &layer_done);
}

int kv_retrieve_chunks(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask,
                       int n_seqs, kv_fmt fmt, int64_t* out_tokens, hipStream_t stream)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_fmt(fmt);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc != KV_OK) return rc;
    rc = retrieve(paged, seqs, hit_mask, n_seqs, fmt, 0, paged->num_layers, out_tokens, stream);
    return rc == KV_OK ? ok() : rc;
}

size_t kv_retrieve_workspace_bytes(const kv_paged* paged)
{
    if (check_paged(paged) != KV_OK) return 0;
    if (paged->num_pages > INT32_MAX) {
        fail(KV_EINVAL, "num_pages above 2^31: the ordered scatter is not available");
        return 0;
    }
    return size_t(2 * ordered_half_bytes(paged->num_pages));
}

int kv_retrieve_chunks_ws(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs,
                          kv_fmt fmt, int64_t* out_tokens, void* workspace, size_t workspace_bytes,
                          hipStream_t stream)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_fmt(fmt);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc != KV_OK) return rc;
    const size_t need = kv_retrieve_workspace_bytes(paged);
    if (need == 0) return KV_EINVAL;
    if (workspace == nullptr || workspace_bytes < need)
        return fail(KV_EINVAL, "workspace of %zu bytes needed (got %zu at %p)", need, workspace_bytes, workspace);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(KV_EINVAL, "workspace must be 256-byte aligned");
    rc = retrieve(paged, seqs, hit_mask, n_seqs, fmt, 0, paged->num_layers, out_tokens, stream, 0, workspace);
    return rc == KV_OK ? ok() : rc;
}

int kv_retrieve_chunks_noalloc(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask,
                               int n_seqs, kv_fmt fmt, int64_t* out_tokens, hipStream_t stream)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_fmt(fmt);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc != KV_OK) return rc;
    if (paged->num_pages > kScratchMaxPages)
        return fail(KV_EINVAL, "pool of %lld pages: the no-allocation retrieve's scratch holds pools of at most "
                    "%lld pages (use kv_retrieve_chunks_ws with a workspace)", (long long)paged->num_pages,
                    (long long)kScratchMaxPages);
    // The host-side checks of the retrieve itself, before any HIP call, one
    // sequence at a time: this entry point allocates no host memory either.
    if (n_seqs > 0 && hit_mask == nullptr) return fail(KV_EINVAL, "hit_mask is NULL");
    int64_t pages = 0;
    for (int i = 0; i < n_seqs; ++i) {
        int64_t n = 0;
        rc = seq_hit_tokens(paged, seqs[i], hit_mask[i], i, &n);
        if (rc != KV_OK) return rc;
        pages += ceil_div(n, paged->page_size);
    }
    if (pages > paged->num_pages)
        return fail(KV_EINVAL, "the call moves %lld pages but the pool holds %lld: page ids repeat",
                    (long long)pages, (long long)paged->num_pages);
    int dev = -1, sdev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && stream != nullptr) e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(KV_EHIP, "reading the device failed: %s", hipGetErrorString(e));
    if (stream != nullptr && sdev != dev)
        return fail(KV_EINVAL, "the stream belongs to device %d, the current device is %d", sdev, dev);
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != KV_OK) return rc;
    // at most 64 sequences per pass, so that the retrieve keeps its token
    // counts on the stack (a launch packs at most kMaxSeqs of them anyway)
    static_assert(64 % kMaxSeqs == 0, "passes of 64 sequences pack as one pass would");
    for (int i0 = 0; i0 < n_seqs && rc == KV_OK; i0 += 64) {
        const int n = std::min(64, n_seqs - i0);
        rc = retrieve(paged, seqs + i0, hit_mask + i0, n, fmt, 0, paged->num_layers,
                      out_tokens != nullptr ? out_tokens + i0 : nullptr, stream, 0, ws);
    }
    return rc == KV_OK ? ok() : rc;
}

int kv_retrieve_layer_ex(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask,
                         int n_seqs, kv_fmt fmt, int32_t layer, int64_t* out_tokens, int32_t max_workgroups,
                         hipStream_t copy_stream, hipEvent_t layer_done)
{
    return retrieve_layers(paged, seqs, hit_mask, n_seqs, fmt, layer, layer + 1, &max_workgroups, out_tokens,
                           copy_stream, nullptr, &layer_done);
}

int kv_retrieve_layer(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs,
                      kv_fmt fmt, int32_t layer, hipStream_t copy_stream, hipEvent_t layer_done)
{
    return retrieve_layers(paged, seqs, hit_mask, n_seqs, fmt, layer, layer + 1, nullptr, nullptr, copy_stream,
                           nullptr, &layer_done);
}

int kv_retrieve_layers(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask, int n_seqs,
                       kv_fmt fmt, int32_t layer_begin, int32_t layer_end, const int32_t* max_workgroups,
                       int64_t* out_tokens, hipStream_t copy_stream, hipStream_t alt_stream,
                       const hipEvent_t* layer_done)
{
    return retrieve_layers(paged, seqs, hit_mask, n_seqs, fmt, layer_begin, layer_end, max_workgroups, out_tokens,
                           copy_stream, alt_stream, layer_done);
}

int kv_store_layers(const kv_paged* paged, const kv_seq* seqs, int n_seqs, kv_fmt fmt, int32_t layer_begin,
                    int32_t layer_end, const int32_t* max_workgroups, hipStream_t stream, hipStream_t alt_stream,
                    const hipEvent_t* wait_before, const hipEvent_t* layer_done)
{
    return store_layers(paged, seqs, n_seqs, fmt, layer_begin, layer_end, max_workgroups, stream, alt_stream,
                        wait_before, layer_done);
}

int64_t kv_chunk_tokens(const kv_paged* paged, int64_t tok_start, int64_t tok_end, int64_t c)
{
    const int64_t n = kv_num_chunks(paged, tok_start, tok_end);
    if (n < 0) return -1;
    if (c < 0 || c >= n) {
        fail(KV_EINVAL, "chunk %lld outside [0, %lld)", (long long)c, (long long)n);
        return -1;
    }
    const int64_t first = tok_start + c * paged->chunk_size;
    const int64_t last = first + paged->chunk_size < tok_end ? first + paged->chunk_size : tok_end;
    return last - first;
}

const char* kv_last_error(void) { return g_last_error.c_str(); }

int kv_take_faults(void)
{
    hipError_t e = hipDeviceSynchronize();
    unsigned int v = 0;
    const unsigned int zero = 0;
    if (e == hipSuccess) e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_kv_faults), sizeof v, 0, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_kv_faults), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(KV_EHIP, "reading the fault word failed: %s", hipGetErrorString(e));
    return int(v);
}

int kv_copy_bytes(void* dst, const void* src, size_t bytes, hipStream_t stream)
{
    if (dst == nullptr || src == nullptr) return fail(KV_EINVAL, "dst / src is NULL");
    if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
        return fail(KV_EINVAL, "kv_copy_bytes needs 16-byte aligned addresses and a multiple of 16 bytes");
    if (bytes == 0) return ok();
    const int64_t tile = int64_t(kCopyBlock) * kCopyVpt * 16;
    const int64_t grid = ceil_div(int64_t(bytes), tile);
    if (grid > max_blocks(kCopyBlock)) return fail(KV_EINVAL, "copy too large for one launch");
    uint64_t s = reinterpret_cast<uint64_t>(src);
    uint64_t d = reinterpret_cast<uint64_t>(dst);
    int64_t n = int64_t(bytes);
    void* args[] = {&s, &d, &n};
    hipError_t e = hipLaunchKernel(reinterpret_cast<KernelFn>(&copy_contiguous<kCopyBlock, kCopyVpt>),
                                   dim3((unsigned)grid), dim3(kCopyBlock), args, 0, stream);
    if (e != hipSuccess) return fail(KV_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int kv_copy_blocks(void* dst, const void* src, size_t bytes, size_t block_bytes, int permute, hipStream_t stream)
{
    if (dst == nullptr || src == nullptr) return fail(KV_EINVAL, "dst / src is NULL");
    if ((reinterpret_cast<uintptr_t>(dst) & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
        return fail(KV_EINVAL, "kv_copy_blocks needs 16-byte aligned addresses");
    const int64_t tile = int64_t(kCopyBlock) * kCopyVpt * 16;
    if (block_bytes < size_t(tile) || block_bytes > (size_t(1) << 30) || (block_bytes & (block_bytes - 1)) != 0)
        return fail(KV_EINVAL, "block_bytes must be a power of two from %lld to 2^30 (got %zu)", (long long)tile,
                    block_bytes);
    if (bytes % block_bytes != 0) return fail(KV_EINVAL, "bytes (%zu) must be a multiple of block_bytes", bytes);
    if (permute != 1 && permute != 2)
        return fail(KV_EINVAL, "permute must be 1 (source blocks) or 2 (destination blocks), got %d", permute);
    if (bytes == 0) return ok();
    const int64_t grid = int64_t(bytes) / tile;
    if (grid > max_blocks(kCopyBlock)) return fail(KV_EINVAL, "copy too large for one launch");
    // a prime multiplier that does not divide the block count is coprime with
    // it; at most 2^35 blocks, so at most two of these primes divide it
    const uint64_t n_blocks = bytes / block_bytes;
    uint64_t mult = 1;
    for (uint64_t p : {7919ull, 7927ull, 7933ull})
        if (n_blocks % p != 0) { mult = p; break; }
    uint32_t shift = 0;
    while ((size_t(1) << shift) < block_bytes) ++shift;
    uint64_t s = reinterpret_cast<uint64_t>(src);
    uint64_t d = reinterpret_cast<uint64_t>(dst);
    int64_t n = int64_t(bytes);
    void* args[] = {&s, &d, &n, &shift, &mult};
    const KernelFn k = permute == 1 ? reinterpret_cast<KernelFn>(&copy_permuted<kCopyBlock, kCopyVpt, true>)
                                    : reinterpret_cast<KernelFn>(&copy_permuted<kCopyBlock, kCopyVpt, false>);
    hipError_t e = hipLaunchKernel(k, dim3((unsigned)grid), dim3(kCopyBlock), args, 0, stream);
    if (e != hipSuccess) return fail(KV_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int kv_store_chunks_cachegen(const kv_paged* paged, const kv_seq* seqs, int n_seqs, const int32_t* key_bins,
                             const int32_t* value_bins, hipStream_t stream)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc != KV_OK) return rc;
    uint8_t qmax[2][kCgMaxLayers];
    Launch st, sc, so;
    rc = cachegen_setup(paged, key_bins, value_bins, qmax, &st, &sc, &so);
    if (rc != KV_OK) return rc;
    int64_t small[64];
    int64_t* n_tok = n_seqs <= 64 ? small : new int64_t[n_seqs];
    for (int i = 0; i < n_seqs; ++i) n_tok[i] = seqs[i].tok_end - seqs[i].tok_start;
    rc = launch_units(st, kCgLayout, paged, seqs, n_tok, n_seqs, 0, paged->num_layers, stream, 0, qmax);
    if (n_tok != small) delete[] n_tok;
    return rc == KV_OK ? ok() : rc;
}

int kv_retrieve_chunks_cachegen(const kv_paged* paged, const kv_seq* seqs, const uint8_t* const* hit_mask,
                                int n_seqs, const int32_t* key_bins, const int32_t* value_bins,
                                int64_t* out_tokens, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_paged(paged);
    if (rc == KV_OK) rc = check_seqs(paged, seqs, n_seqs);
    if (rc != KV_OK) return rc;
    uint8_t qmax[2][kCgMaxLayers];
    Launch st, sc, so;
    rc = cachegen_setup(paged, key_bins, value_bins, qmax, &st, &sc, &so);
    if (rc != KV_OK) return rc;
    int64_t small[64];
    int64_t* n_tok = n_seqs <= 64 ? small : new int64_t[n_seqs];
    rc = hit_tokens(paged, seqs, hit_mask, n_seqs, n_tok);
    if (rc == KV_OK && workspace != nullptr) {
        const size_t need = kv_retrieve_workspace_bytes(paged);
        if (need == 0 || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
            rc = fail(KV_EINVAL, "workspace of %zu bytes, 256-byte aligned, needed (got %zu at %p)", need,
                      workspace_bytes, workspace);
        if (rc == KV_OK) rc = check_ordered_fits(paged, n_tok, n_seqs);
        if (rc == KV_OK)
            rc = retrieve_ordered(so, kCgLayout, paged, seqs, n_tok, n_seqs, 0, paged->num_layers, workspace,
                                  stream, qmax);
    } else if (rc == KV_OK) {
        rc = launch_units(sc, kCgLayout, paged, seqs, n_tok, n_seqs, 0, paged->num_layers, stream, 0, qmax);
    }
    if (rc == KV_OK && out_tokens != nullptr)
        for (int i = 0; i < n_seqs; ++i) out_tokens[i] = n_tok[i];
    if (n_tok != small) delete[] n_tok;
    return rc == KV_OK ? ok() : rc;
}

}  // extern "C"
