// kvq_api.cpp -- host side of libkvq.so: validation, launch geometry and
// workspace sizing behind the C ABI of include/kvq.h.  Never allocates, frees
// or synchronizes device memory.
#include <algorithm>
#include <string.h>

#include "kvq.h"
#include "kvq_common.hpp"
#include "kvq_kernels.hpp"

namespace {

constexpr int32_t MAGIC = 0x4b565131;   // "KVQ1"

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int validate_layout(const kvq_layout_t *L) {
    if (L->head_dim != kvq::D) return KVQ_EINVAL;
    if (L->n_kv_heads < 1 || L->n_kv_heads > 65535) return KVQ_EINVAL;
    if (L->n_q_heads < L->n_kv_heads || L->n_q_heads % L->n_kv_heads != 0) return KVQ_EINVAL;
    const int qpk = L->n_q_heads / L->n_kv_heads;
    if (qpk > 8) return KVQ_EINVAL;
    if (L->batch < 1 || L->batch > 65535) return KVQ_EINVAL;
    if (L->max_pages < 1 || L->n_pages < 1) return KVQ_EINVAL;
    if (L->split_pages < 0 || L->split_pages > 64) return KVQ_EINVAL;
    if (L->flags & ~KVQ_FLAG_GENERIC_STAGE1) return KVQ_EINVAL;
    if (L->reserved != 0) return KVQ_EINVAL;
    // sink tokens: one stage-1 chunk of at most 64 fp16 tokens (KIVI2 / Kitty)
    if (L->sink < 0 || L->sink > kvq::PT) return KVQ_EINVAL;
    if (L->sink > 0 && (L->scheme == KVQ_SCHEME_WITCERT || L->scheme == KVQ_SCHEME_WITCERT_PAGED))
        return KVQ_EINVAL;
    switch (L->scheme) {
        case KVQ_SCHEME_KIVI2:
        case KVQ_SCHEME_KITTY:
        case KVQ_SCHEME_KITTY_DYN:
        case KVQ_SCHEME_KIVI4:
            if (L->group != 32 || L->value_group != 32) return KVQ_EINVAL;
            // the key residual is quantized in whole groups: R % G == 0, and
            // the flush writes whole 64-token pages
            if (L->residual % L->group != 0 || L->residual % kvq::PT != 0) return KVQ_EINVAL;
            if (L->residual < kvq::PT || L->residual > kvq::MAX_RESIDUAL) return KVQ_EINVAL;
            if (kvq::is_kitty(L->scheme) ? (L->n_boost != kvq::NB && L->n_boost != kvq::NB_MAX)
                                         : L->n_boost != 0)
                return KVQ_EINVAL;
            // the VALU stage 1 handles 16 boosted channels only
            if (L->n_boost > kvq::NB && (L->flags & KVQ_FLAG_GENERIC_STAGE1)) return KVQ_EINVAL;
            // nor 4-bit codes
            if (L->scheme == KVQ_SCHEME_KIVI4 && (L->flags & KVQ_FLAG_GENERIC_STAGE1)) return KVQ_EINVAL;
            // the VALU stage 1 reads the head's static boost table only
            if (L->scheme == KVQ_SCHEME_KITTY_DYN && (L->flags & KVQ_FLAG_GENERIC_STAGE1))
                return KVQ_EINVAL;
            break;
        case KVQ_SCHEME_WITCERT_PAGED:
            // scales per (token, 32-channel group); at most 4 bypassed pairs
            // (an 8-entry fp16 row per token)
            if (L->group != 32 || L->value_group != 32) return KVQ_EINVAL;
            if (L->n_boost < 0 || L->n_boost > 4) return KVQ_EINVAL;
            if (L->flags != 0) return KVQ_EINVAL;
            if (L->layer >= 65536u) return KVQ_EINVAL;
            if (qpk != 1 && qpk != 2 && qpk != 4 && qpk != 8) return KVQ_EINVAL;
            break;
        case KVQ_SCHEME_WITCERT:
            if (L->block != kvq::WPT) return KVQ_EINVAL;
            if (L->layer >= 65536u) return KVQ_EINVAL;
            if (qpk != 1 && qpk != 2 && qpk != 4 && qpk != 8) return KVQ_EINVAL;
            break;
        default:
            return KVQ_EINVAL;
    }
    return KVQ_OK;
}

kvq::KParams params(const kvq_cache_t *C) {
    kvq::KParams P;
    const kvq_layout_t &L = C->layout;
    P.pool = (uint8_t *)C->bufs.pool;
    P.table = C->bufs.page_table;
    P.state = C->bufs.state;
    P.res_k = C->bufs.res_k;
    P.res_v = C->bufs.res_v;
    P.boost_idx = C->bufs.boost_idx;
    P.status = C->bufs.status;
    P.sink_k = C->bufs.sink_k;
    P.sink_v = C->bufs.sink_v;
    P.sink = L.sink;
    P.nb = (kvq::is_kitty(L.scheme) || L.scheme == KVQ_SCHEME_WITCERT_PAGED) ? L.n_boost : 0;
    P.B = L.batch;
    P.Hq = L.n_q_heads;
    P.Hkv = L.n_kv_heads;
    P.R = L.scheme == KVQ_SCHEME_WITCERT ? kvq::WPT : L.residual;
    P.max_pages = L.max_pages;
    P.n_pages = L.n_pages;
    P.page_bytes = (int)C->page_bytes;
    P.scheme = L.scheme;
    P.qpk = L.n_q_heads / L.n_kv_heads;
    P.split_pages = C->split_pages;
    P.force_generic = (L.flags & KVQ_FLAG_GENERIC_STAGE1) ? 1 : 0;
    P.layer = L.layer;
    P.seed = L.seed;
    return P;
}

int check_cache(const kvq_cache_t *C) {
    if (!C) return KVQ_ENULL;
    if (C->magic != MAGIC) return KVQ_ENOLAYOUT;
    return KVQ_OK;
}

bool gqa4(const kvq_layout_t &L) {
    return kvq::gqa4_path(L.scheme, L.n_q_heads / L.n_kv_heads, (L.flags & KVQ_FLAG_GENERIC_STAGE1) != 0);
}

// partial rows per query head for the paged splits of a request of up to
// max_pages pages
int splits_for(const kvq_layout_t &L, int sp) {
    return gqa4(L) ? kvq::gqa_splits_bound(L.max_pages, sp) : (L.max_pages + sp - 1) / sp;
}

int max_splits(const kvq_cache_t *C) { return splits_for(C->layout, C->split_pages); }

// stage-1 work-list items the workspace holds: one per possible split of
// every (request, KV head) of the group kernel
size_t list_items(const kvq_cache_t *C) {
    const kvq_layout_t &L = C->layout;
    return (size_t)L.batch * L.n_kv_heads * max_splits(C);
}

// 64-token chunks of the fp16 window, each a stage-1 partial of its own
int n_win(const kvq_cache_t *C) {
    if (C->layout.scheme == KVQ_SCHEME_WITCERT_PAGED) return 0;   // no fp16 tail
    return C->layout.scheme == KVQ_SCHEME_WITCERT ? kvq::WPT / kvq::PT
                                                  : C->layout.residual / kvq::PT + (C->layout.sink > 0 ? 1 : 0);
}

}  // namespace

extern "C" {

int64_t kvq_page_bytes(const kvq_layout_t *L) {
    if (!L) return 0;
    if (L->scheme < KVQ_SCHEME_KIVI2 || L->scheme > KVQ_SCHEME_WITCERT_PAGED) return 0;
    return kvq::geom(L->scheme, L->n_boost).bytes;
}

int32_t kvq_page_tokens(const kvq_layout_t *L) {
    if (!L) return 0;
    if (L->scheme < KVQ_SCHEME_KIVI2 || L->scheme > KVQ_SCHEME_WITCERT_PAGED) return 0;
    return kvq::geom(L->scheme, L->n_boost).tokens;
}

double kvq_bytes_per_token(const kvq_layout_t *L) {
    const int32_t t = kvq_page_tokens(L);
    return t ? (double)kvq_page_bytes(L) / (double)t : 0.0;
}

int kvq_set_layout(kvq_cache_t *cache, const kvq_layout_t *layout, const kvq_buffers_t *bufs) {
    if (!cache || !layout || !bufs) return KVQ_ENULL;
    int rc = validate_layout(layout);
    if (rc != KVQ_OK) return rc;
    const bool wtok = layout->scheme == KVQ_SCHEME_WITCERT_PAGED;   // no residual buffers
    if (!bufs->pool || !bufs->page_table || !bufs->state || !bufs->status) return KVQ_ENULL;
    if (!wtok && (!bufs->res_k || !bufs->res_v)) return KVQ_ENULL;
    if (layout->scheme == KVQ_SCHEME_KITTY && !bufs->boost_idx) return KVQ_ENULL;
    if (wtok && layout->n_boost > 0 && !bufs->boost_idx) return KVQ_ENULL;
    if (layout->sink > 0 && (!bufs->sink_k || !bufs->sink_v)) return KVQ_ENULL;
    if ((bufs->sink_k && !aligned(bufs->sink_k, 16)) || (bufs->sink_v && !aligned(bufs->sink_v, 16)))
        return KVQ_EALIGN;
    if (!aligned(bufs->pool, 256) || !aligned(bufs->page_table, 16) || !aligned(bufs->state, 16) ||
        (bufs->res_k && !aligned(bufs->res_k, 16)) || (bufs->res_v && !aligned(bufs->res_v, 16)) ||
        !aligned(bufs->status, 4))
        return KVQ_EALIGN;
    memset(cache, 0, sizeof(*cache));
    cache->layout = *layout;
    cache->bufs = *bufs;
    const kvq::Geom G = kvq::geom(layout->scheme, layout->n_boost);
    cache->page_tokens = G.tokens;
    cache->page_bytes = G.bytes;
    int sp = layout->split_pages;
    if (sp == 0) {
        // default: one 256-token block per split for WITCERT; 4 pages for
        // the shortest caches (more splits to fill the chip), 8 up to 128
        // pages and 32 for longer ones (fewer splits to start and merge, the
        // window chunks filling the chip as the splits drain) -- 12 for
        // KIVI4, whose longer splits' binary32 sums lose accuracy against the
        // zero-point term at the 1e-5 bound; for the GQA kernel, whose splits
        // run from a work list with a tail of quarter-length splits, bodies
        // of 8 pages for short caches and 48 for longer ones; at least what
        // keeps <= 256 splits
        const bool g4 = gqa4(*layout);
        sp = layout->scheme == KVQ_SCHEME_WITCERT ? 1
             : wtok                                 ? 4      // 256 tokens, as one WITCERT block
             : g4                                   ? (layout->max_pages <= 128 ? 8 : 48)
             : layout->max_pages <= 32              ? 4
             : layout->max_pages <= 128             ? 8
             : layout->scheme == KVQ_SCHEME_KIVI4   ? 12
                                                    : 32;
        while (sp < 64 && splits_for(*layout, sp) > kvq::MAX_SPLITS) sp++;
    }
    // the merge takes at most MAX_SPLITS splits per query head
    if (sp > 64 || splits_for(*layout, sp) > kvq::MAX_SPLITS) return KVQ_EINVAL;
    cache->split_pages = sp;
    cache->magic = MAGIC;
    return KVQ_OK;
}

size_t kvq_workspace_bytes(const kvq_cache_t *cache) {
    if (check_cache(cache) != KVQ_OK) return 0;
    // one partial row per query head and split, and per 64-token chunk of the
    // fp16 window
    const size_t rows =
        (size_t)cache->layout.batch * cache->layout.n_q_heads * (max_splits(cache) + n_win(cache));
    // and the stage-1 work list: one item per (request, KV head, split), then
    // its length (in the last 256 bytes)
    const size_t items = list_items(cache);
    return rows * kvq::D * sizeof(float) + rows * sizeof(float2) + items * sizeof(uint4) + 256;
}

int kvq_append_token(const kvq_cache_t *cache, const uint16_t *k_new, const uint16_t *v_new,
                     hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != KVQ_OK) return rc;
    if (!k_new || !v_new) return KVQ_ENULL;
    if (!aligned(k_new, 16) || !aligned(v_new, 16)) return KVQ_EALIGN;
    return kvq::launch_append(params(cache), k_new, v_new, stream) == hipSuccess ? KVQ_OK
                                                                                 : KVQ_ELAUNCH;
}

int kvq_flush_key_group(const kvq_cache_t *cache, hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != KVQ_OK) return rc;
    return kvq::launch_flush(params(cache), stream) == hipSuccess ? KVQ_OK : KVQ_ELAUNCH;
}

namespace {
// the workspace's parts (kvq_workspace_bytes' order): partial rows, their
// log-sum-exps, the work list and its length
kvq::Workspace workspace_of(const kvq_cache_t *cache, void *workspace) {
    kvq::Workspace W;
    W.max_splits = max_splits(cache);
    W.n_win = n_win(cache);
    const size_t rows = (size_t)cache->layout.batch * cache->layout.n_q_heads * (W.max_splits + W.n_win);
    const size_t items = list_items(cache);
    W.o = (float *)workspace;
    W.ml = (float2 *)((char *)workspace + rows * kvq::D * sizeof(float));
    W.items = (uint4 *)((char *)W.ml + rows * sizeof(float2));
    W.n_items = (uint32_t *)(W.items + items);
    W.ev_begin = cache->ev_stage1_begin;
    W.ev_end = cache->ev_stage1_end;
    return W;
}

// kvq_decode_attention's launch once the workspace is known good
int decode_with(const kvq_cache_t *cache, const uint16_t *q, float *out, float *cert,
                float sm_scale, float kappa, void *workspace, hipStream_t stream) {
    const kvq::Workspace W = workspace_of(cache, workspace);
    return kvq::launch_decode(params(cache), q, out, cert, sm_scale, kappa, W, stream) == hipSuccess
               ? KVQ_OK
               : KVQ_ELAUNCH;
}

int check_decode_args(const uint16_t *q, const float *out, const float *cert) {
    if (!q || !out) return KVQ_ENULL;
    if (!aligned(q, 16) || !aligned(out, 16) || (cert && !aligned(cert, 4))) return KVQ_EALIGN;
    return KVQ_OK;
}
}  // namespace

int kvq_decode_attention(const kvq_cache_t *cache, const uint16_t *q, float *out, float *cert,
                         float sm_scale, float kappa, void *workspace, size_t ws_bytes,
                         hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != KVQ_OK) return rc;
    if ((rc = check_decode_args(q, out, cert)) != KVQ_OK) return rc;
    if (!workspace) return KVQ_ENULL;
    if (!aligned(workspace, 256)) return KVQ_EALIGN;
    if (ws_bytes < kvq_workspace_bytes(cache)) return KVQ_EWORKSPACE;
    return decode_with(cache, q, out, cert, sm_scale, kappa, workspace, stream);
}

int kvq_stage1_load_floor(const kvq_cache_t *cache, const uint16_t *q, float sm_scale,
                          void *workspace, size_t ws_bytes, hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != KVQ_OK) return rc;
    const kvq_layout_t &L = cache->layout;
    if (!kvq::gqa4_path(L.scheme, L.n_q_heads / L.n_kv_heads, (L.flags & KVQ_FLAG_GENERIC_STAGE1) != 0))
        return KVQ_EINVAL;
    if (!q || !workspace) return KVQ_ENULL;
    if (!aligned(q, 16) || !aligned(workspace, 256)) return KVQ_EALIGN;
    if (ws_bytes < kvq_workspace_bytes(cache)) return KVQ_EWORKSPACE;
    const kvq::Workspace W = workspace_of(cache, workspace);
    return kvq::launch_stage1_floor(params(cache), q, sm_scale, W, stream) == hipSuccess ? KVQ_OK
                                                                                         : KVQ_ELAUNCH;
}

int kvq_decode_attention_noalloc(const kvq_cache_t *cache, const uint16_t *q, float *out,
                                 float *cert, float sm_scale, float kappa, hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != KVQ_OK) return rc;
    if ((rc = check_decode_args(q, out, cert)) != KVQ_OK) return rc;
    // the size check comes before any device call
    if (kvq_workspace_bytes(cache) > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ENOSCRATCH;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (kvq::noalloc_scratch(&ws, &ws_bytes) != hipSuccess) return KVQ_ELAUNCH;
    if (ws_bytes < kvq_workspace_bytes(cache)) return KVQ_ENOSCRATCH;
    return decode_with(cache, q, out, cert, sm_scale, kappa, ws, stream);
}

int kvq_prefill(const kvq_cache_t *cache, int32_t req0, int32_t n_req, const uint16_t *K,
                const uint16_t *V, int64_t ld_tokens, const int32_t *lengths, hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != KVQ_OK) return rc;
    if (!K || !V || !lengths) return KVQ_ENULL;
    if (req0 < 0 || n_req < 1 || req0 + n_req > cache->layout.batch || ld_tokens < 1)
        return KVQ_EINVAL;
    if (!aligned(K, 16) || !aligned(V, 16) || !aligned(lengths, 4)) return KVQ_EALIGN;
    return kvq::launch_prefill(params(cache), req0, n_req, K, V, (long long)ld_tokens, lengths,
                               stream) == hipSuccess
               ? KVQ_OK
               : KVQ_ELAUNCH;
}

int kvq_kitty_calibrate(const kvq_cache_t *cache, const uint16_t *calib, int32_t n_tokens,
                        uint8_t *idx_out, hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != KVQ_OK) return rc;
    if (cache->layout.scheme != KVQ_SCHEME_KITTY) return KVQ_EINVAL;
    if (!calib || !idx_out) return KVQ_ENULL;
    if (n_tokens < 1) return KVQ_EINVAL;
    return kvq::launch_kitty_calibrate(params(cache), calib, n_tokens, idx_out, stream) == hipSuccess
               ? KVQ_OK
               : KVQ_ELAUNCH;
}

int kvq_witcert_calibrate(const kvq_cache_t *cache, const uint16_t *calib, int32_t n_tokens,
                          uint8_t *idx_out, hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != KVQ_OK) return rc;
    if (cache->layout.scheme != KVQ_SCHEME_WITCERT_PAGED || cache->layout.n_boost < 1)
        return KVQ_EINVAL;
    if (!calib || !idx_out) return KVQ_ENULL;
    if (n_tokens < 1) return KVQ_EINVAL;
    return kvq::launch_witcert_calibrate(params(cache), calib, n_tokens, idx_out, stream) ==
                   hipSuccess
               ? KVQ_OK
               : KVQ_ELAUNCH;
}

int kvq_set_stage1_events(kvq_cache_t *cache, hipEvent_t begin, hipEvent_t end) {
    int rc = check_cache(cache);
    if (rc != KVQ_OK) return rc;
    if ((begin == nullptr) != (end == nullptr)) return KVQ_ENULL;
    cache->ev_stage1_begin = begin;
    cache->ev_stage1_end = end;
    return KVQ_OK;
}

const char *kvq_strerror(int code) {
    if (code > 0) {                        // a device status word
        const unsigned known = KVQ_STATUS_RESIDUAL_FULL | KVQ_STATUS_CAPACITY |
                               KVQ_STATUS_UNMAPPED_PAGE | KVQ_STATUS_BAD_LENGTH | KVQ_STATUS_RANGE;
        const unsigned u = (unsigned)code;
        if (u & ~known) return "unknown";
        switch (u) {
            case KVQ_STATUS_RESIDUAL_FULL: return "append found the key residual or active block full (flush skipped)";
            case KVQ_STATUS_CAPACITY: return "append beyond the page table's capacity";
            case KVQ_STATUS_UNMAPPED_PAGE: return "page-table entry outside the pool";
            case KVQ_STATUS_BAD_LENGTH: return "prefill length outside [0, capacity]";
            case KVQ_STATUS_RANGE: return "outside the matrix-core stage 1's operand range (value scale above 255 or a non-finite split)";
            default: return "several device status bits";
        }
    }
    switch (code) {
        case KVQ_OK: return "ok";
        case KVQ_EINVAL: return "invalid layout or argument";
        case KVQ_ENULL: return "required pointer is NULL";
        case KVQ_EALIGN: return "device pointer misaligned";
        case KVQ_ENOLAYOUT: return "cache not initialised by kvq_set_layout";
        case KVQ_EWORKSPACE: return "workspace too small";
        case KVQ_ELAUNCH: return "kernel launch or HIP call failed";
        case KVQ_ENOSCRATCH: return "cache needs more workspace than the no-alloc scratch array holds";
        default: return "unknown";
    }
}

}  // extern "C"
