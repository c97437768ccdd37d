/*
 * kvq.h -- C ABI of libkvq.so: low-bit KV-cache quantization on write and
 * single-query decode attention with dequantization fused into the read, for
 * AMD Instinct MI355X (gfx950).
 *
 * Schemes
 *   KVQ_SCHEME_KIVI2   keys: 2-bit asymmetric, one group = one channel x G=32
 *                      consecutive tokens; values: 2-bit asymmetric, one group
 *                      = one token x 32 consecutive channels; fp16 scale and
 *                      zero point per group; the newest keys (1..R) and values
 *                      (R) stay fp16.  ("KIVI" explainer, sections 3.1-3.3
 *                      and section 4 steps 2-5.)
 *   KVQ_SCHEME_KITTY   KIVI2 with n_boost key channels per KV head stored at
 *                      4 bits, split into a dense low 2-bit plane (all
 *                      channels) and a structured high 2-bit plane (boosted
 *                      channels only); code = low | high << 2.  ("Kitty"
 *                      summary: Channel-Wise Precision Boost Mechanism;
 *                      Page-Centric Memory Layout and Dense-Sparse
 *                      Decomposition; Algorithm 1.)
 *   KVQ_SCHEME_KITTY_DYN
 *                      KITTY with the boosted set chosen per 64-token page:
 *                      the n_boost channels of largest mean |key| over the
 *                      page's tokens (ties to the lower channel), picked when
 *                      the page's keys are quantized; the page stores the
 *                      chosen channel ids in ascending order (16 bytes).
 *                      ("Kitty" summary: Channel-Wise Precision Boost
 *                      Mechanism, importance as the mean absolute value of a
 *                      group; a group here is one page.)  No calibration and
 *                      no boost_idx buffer.
 *   KVQ_SCHEME_KIVI4   KIVI2's groups, statistics and windows at 4 bits for
 *                      keys and values (16 levels per group; "KIVI"
 *                      explainer, its 2- and 4-bit variants): 160 B per
 *                      token and KV head.
 *   KVQ_SCHEME_WITCERT INT8 keys and values with subtractive dither:
 *                      x_hat = s (round(x/s + xi) - xi), s = amax/126.5 per
 *                      (256-token block, channel) stored fp16 and used for
 *                      quantization, xi from Philox4x32-10 keyed by (request,
 *                      layer, KV head, token, channel); the active block stays
 *                      fp16; a per-query certificate A = sum_t p_t exp(u_t) is
 *                      accumulated in the attention pass.  ("WitCert" page:
 *                      write-kernel paragraph, "Key structure", quantised-path
 *                      certificate paragraph.)
 *   KVQ_SCHEME_WITCERT_PAGED
 *                      WitCert's storage for token-granular paging: every
 *                      token quantized when written (no fp16 tail), INT8 with
 *                      subtractive dither and one fp16 scale s = amax/126.5
 *                      per (token, 32-channel group) on each side; the dither
 *                      keyed by (layer, KV head, slot, channel), slot =
 *                      page_id * 64 + position in the page, so it survives
 *                      paging and prefix sharing; n_boost = m fixed outlier
 *                      RoPE key pairs (channels i and i + 64) per KV head
 *                      stored fp16 and left out of their group's amax; the
 *                      certificate uses each token's group scales (a
 *                      bypassed channel adds no error).  136 B per token and
 *                      side + 16 B when m > 0.  ("WitCert" page, the
 *                      certified-deployment paragraphs.)
 *
 * Step order per decode step (all calls asynchronous on the caller's stream,
 * none synchronizes, allocates or frees, so a step can be captured in a HIP
 * graph):  kvq_flush_key_group -> kvq_append_token -> kvq_decode_attention.
 * The flush quantizes the key residual once it holds R tokens (the pipeline
 * order of the "Kitty" summary: attention runs on the fp16 group, the group is
 * quantized once it has gathered).
 *
 * Memory ownership: every device buffer is allocated and freed by the caller;
 * the library keeps only the pointers copied into kvq_cache_t.  Device
 * pointers must be 256-byte aligned (pool) or 16-byte aligned (all others).
 *
 * Errors: host-side checks return a negative KVQ_E* code and launch nothing.
 * Conditions only the device can see set sticky bits in the caller's status
 * word (KVQ_STATUS_*), read by the caller after its own synchronization; the
 * affected (request, KV head) is then left unmodified.
 *
 * fp16 values cross the ABI as uint16_t bit patterns.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KVQ_SCHEME_KIVI2 = 0,
    KVQ_SCHEME_KITTY = 1,
    KVQ_SCHEME_WITCERT = 2,
    KVQ_SCHEME_KITTY_DYN = 3,
    KVQ_SCHEME_KIVI4 = 4,
    KVQ_SCHEME_WITCERT_PAGED = 5
};

/* layout flags */
enum {
    KVQ_FLAG_GENERIC_STAGE1 = 1  /* KIVI2 / KITTY: run the per-query-head VALU
                                    stage 1 instead of the matrix-core one
                                    (a second implementation, for comparison);
                                    not available for KITTY_DYN */
};

/* host-side return codes */
enum {
    KVQ_OK = 0,
    KVQ_EINVAL = -1,      /* a layout field is out of range (see kvq_set_layout) */
    KVQ_ENULL = -2,       /* a required pointer is NULL */
    KVQ_EALIGN = -3,      /* a device pointer is misaligned */
    KVQ_ENOLAYOUT = -4,   /* cache was not filled by kvq_set_layout */
    KVQ_EWORKSPACE = -5,  /* workspace smaller than kvq_workspace_bytes() */
    KVQ_ELAUNCH = -6,     /* a kernel launch or HIP call failed (hipGetLastError) */
    KVQ_ENOSCRATCH = -7   /* kvq_decode_attention_noalloc: the cache needs more
                             than KVQ_NOALLOC_SCRATCH_BYTES of workspace */
};

/* Size of the device scratch array behind kvq_decode_attention_noalloc: one
 * array per GPU the library runs on, held until the process ends. */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* device status bits (sticky, OR-ed into *status) */
enum {
    KVQ_STATUS_RESIDUAL_FULL = 1u,  /* append found the key residual / active
                                       block full: flush was skipped */
    KVQ_STATUS_CAPACITY = 2u,       /* append beyond sink + max_pages * page_tokens */
    KVQ_STATUS_UNMAPPED_PAGE = 4u,  /* page-table entry outside [0, n_pages) */
    KVQ_STATUS_BAD_LENGTH = 8u,     /* prefill length outside [0, capacity]
                                       (capacity: sink + max_pages * page_tokens) */
    KVQ_STATUS_RANGE = 16u          /* outside the matrix-core stage 1's operand
                                       range (see kvq_decode_attention): append
                                       or prefill stored a value scale above
                                       255, or a stage-1 split's result was not
                                       finite (an f16 operand head |q_c s_c| or
                                       p_t s_t overflowed, or non-finite
                                       inputs); not set under
                                       KVQ_FLAG_GENERIC_STAGE1 or for WITCERT */
};

/* Layout.  Fields the caller fills before kvq_set_layout. */
typedef struct kvq_layout {
    int32_t scheme;          /* KVQ_SCHEME_* */
    int32_t head_dim;        /* D; must be 128 */
    int32_t n_q_heads;       /* Hq; multiple of n_kv_heads */
    int32_t n_kv_heads;      /* Hkv; 1 .. 65535 */
    int32_t batch;           /* B, requests; 1 .. 65535 */
    int32_t group;           /* G, key group tokens; must be 32 (KIVI2/KITTY) */
    int32_t value_group;     /* value group channels; must be 32 (KIVI2/KITTY) */
    int32_t residual;        /* R, key/value fp16 window; multiple of 64 (so of
                                G), 64 .. 256 (KIVI2/KITTY/KITTY_DYN) */
    int32_t block;           /* WitCert block tokens; must be 256 (WITCERT) */
    int32_t n_boost;         /* KITTY / KITTY_DYN boosted key channels: 16
                                or 32; WITCERT_PAGED: bypassed RoPE pairs
                                m, 0 .. 4; 0 for others */
    int32_t max_pages;       /* page-table row length per request */
    int32_t n_pages;         /* pages in the pool */
    int32_t split_pages;     /* stage-1 split size in pages; 0: the default.
                                KIVI2 with 2, 4 or 8 query heads per KV head
                                (the group kernel): body splits of 8 pages when
                                max_pages <= 128, else 48, each request's last
                                pages in tail splits of a quarter of that
                                (see kvq_decode_attention).  Others: 4 when
                                max_pages <= 32, 8 when max_pages <= 128, else
                                32 (12 for KIVI4; 1 for WITCERT, 4 for
                                WITCERT_PAGED).
                                Raised where a request of max_pages pages would
                                need more than 256 splits */
    int32_t flags;           /* KVQ_FLAG_* */
    uint32_t layer;          /* WITCERT(_PAGED) dither counter field; < 65536 */
    uint64_t seed;           /* WITCERT(_PAGED) dither key */
    int32_t sink;            /* KIVI2 / KITTY / KITTY_DYN: the first `sink`
                                tokens of every request stay fp16, keys and
                                values ("Kitty" summary, sink tokens); key
                                groups, pages and the value window count from
                                token `sink`; 0 .. 64, 0 for WITCERT and
                                WITCERT_PAGED */
    int32_t reserved;        /* must be 0 */
} kvq_layout_t;

/* Caller-owned device buffers. */
typedef struct kvq_buffers {
    void *pool;               /* n_pages * n_kv_heads * kvq_page_bytes() bytes */
    const int32_t *page_table;/* [batch][max_pages] physical page ids; a page
                                 holds page_tokens consecutive tokens */
    int32_t *state;           /* [batch][n_kv_heads][4]: {l, n_kq, 0, 0}:
                                 tokens appended, keys (WitCert: both sides)
                                 quantized */
    uint16_t *res_k;          /* [batch][n_kv_heads][W][D] fp16 key residual;
                                 W = residual (KIVI2/KITTY) or block (WITCERT) */
    uint16_t *res_v;          /* [batch][n_kv_heads][W][D] fp16 value window:
                                 ring by token index (KIVI2/KITTY) or active
                                 block (WITCERT); WITCERT_PAGED: unused, may
                                 be NULL (also res_k) */
    const uint8_t *boost_idx; /* KITTY: [n_kv_heads][D] offset of each channel
                                 in the high plane, or n_boost + 1;
                                 WITCERT_PAGED with n_boost > 0: offset of a
                                 bypassed key channel in its token's fp16
                                 bypass row (0 .. 2 n_boost - 1, both channels
                                 of each pair), or 2 n_boost + 1 */
    uint32_t *status;         /* one uint32 of sticky KVQ_STATUS_* bits */
    uint16_t *sink_k;         /* sink > 0: [batch][n_kv_heads][sink][D] fp16
                                 keys of the sink tokens; else may be NULL */
    uint16_t *sink_v;         /* sink > 0: the same for values */
} kvq_buffers_t;

/* Filled by kvq_set_layout; plain data, copyable. */
typedef struct kvq_cache {
    kvq_layout_t layout;
    kvq_buffers_t bufs;
    int32_t page_tokens;      /* 256 (WITCERT), else 64 */
    int32_t split_pages;      /* resolved stage-1 split, pages */
    int64_t page_bytes;       /* bytes of one (page, KV head) block */
    int32_t magic;            /* set by kvq_set_layout */
    int32_t reserved;
    hipEvent_t ev_stage1_begin; /* optional, see kvq_set_stage1_events */
    hipEvent_t ev_stage1_end;
} kvq_cache_t;

/* Validate `layout` and `bufs` and fill `cache`.  Host only, synchronous, no
 * device work.  Returns KVQ_OK, KVQ_ENULL (cache, layout, bufs or a required
 * buffer is NULL; boost_idx is required for KITTY only, sink_k and sink_v
 * when sink > 0), KVQ_EALIGN (pool not 256-byte aligned; page_table, state,
 * res_k, res_v, sink_k or sink_v not 16-byte aligned; status not 4-byte
 * aligned) or KVQ_EINVAL when a field is out of range:
 *   head_dim != 128; n_kv_heads outside [1, 65535]; n_q_heads not a multiple
 *   of n_kv_heads, or more than 8 query heads per KV head; batch outside
 *   [1, 65535]; max_pages or n_pages < 1; split_pages outside [0, 64] (0 picks
 *   a default), or max_pages needs more than 256 splits of the resolved size
 *   (at most 64 pages); flags other than KVQ_FLAG_*; unknown scheme;
 *   KIVI2 / KITTY / KITTY_DYN / KIVI4: group or value_group != 32; residual not a
 *   multiple of 64 or outside [64, 256] (the residual is quantized in whole
 *   key groups, so it must be divisible by the group, "KIVI" explainer 3.3,
 *   and the flush fills whole 64-token pages); n_boost other than 16 or 32
 *   for KITTY and KITTY_DYN, or != 0 for KIVI2 and KIVI4;
 *   KVQ_FLAG_GENERIC_STAGE1 with KITTY_DYN, KIVI4 or n_boost 32;
 *   sink outside [0, 64] or non-zero for WITCERT / WITCERT_PAGED; reserved
 *   != 0;
 *   WITCERT: block != 256; layer >= 65536; query heads per KV head not in
 *   {1, 2, 4, 8};
 *   WITCERT_PAGED: group or value_group != 32; n_boost outside [0, 4];
 *   layer >= 65536; query heads per KV head not in {1, 2, 4, 8}; any flag.
 * KVQ_ENULL also for a NULL boost_idx with KITTY, or with WITCERT_PAGED and
 * n_boost > 0. */
int kvq_set_layout(kvq_cache_t *cache, const kvq_layout_t *layout,
                   const kvq_buffers_t *bufs);

/* Append one token per (request, KV head).  k_new, v_new: device fp16
 * [batch][n_kv_heads][D].  KIVI2/KITTY: the key goes to residual slot
 * l - n_kq; the value goes to ring slot l mod R after the token leaving the
 * window (l - R, when l >= R) is quantized per token into the pages ("KIVI"
 * explainer 3.3 value FIFO).  WITCERT: key and value go to the active block.
 * WITCERT_PAGED: key and value are quantized into slot l mod 64 of page
 * page_table[b][l / 64] at once (n_kq = l + 1).
 * Then l += 1.  Device errors: RESIDUAL_FULL, CAPACITY, UNMAPPED_PAGE. */
int kvq_append_token(const kvq_cache_t *cache, const uint16_t *k_new,
                     const uint16_t *v_new, hipStream_t stream);

/* Quantize every (request, KV head) whose key residual holds R tokens
 * (KIVI2/KITTY: per channel, R/G groups of G tokens, written to the pages;
 * "KIVI" explainer 3.3) or whose active block holds 256 tokens (WITCERT:
 * keys and values, per channel).  A no-op elsewhere, so it may be called every
 * step (WITCERT_PAGED: always a no-op, nothing is launched). */
int kvq_flush_key_group(const kvq_cache_t *cache, hipStream_t stream);

/* Decode attention for one query token per request over the current state.
 * q: device fp16 [batch][n_q_heads][D]; out: device fp32 [batch][n_q_heads][D];
 * cert: device fp32 [batch][n_q_heads] (WITCERT certificate, may be NULL;
 * +inf is a valid value); sm_scale multiplies q.k; kappa multiplies the
 * certificate's per-block standard deviation.  Query head h reads KV head
 * h / (n_q_heads / n_kv_heads).  workspace: device, >= kvq_workspace_bytes().
 * Stage 1 covers the tokens whose key and value are both quantized in splits
 * of split_pages pages, and the fp16 window (and the sink tokens) in 64-token
 * chunks, each a partial of its own; stage 2 merges all partials with
 * log-sum-exp weights ("WitCert" Key structure).  KIVI2 with 2, 4 or 8 query
 * heads per KV head (no KVQ_FLAG_GENERIC_STAGE1) runs the group kernel, which
 * reads each page once for all the query heads of its KV head (one wave; up to
 * two sets of four query heads): a request of npg pages is cut
 * into splits of split_pages pages over all but its last min(npg / 8,
 * 2 split_pages) pages and splits of split_pages / 4 over the rest, run
 * longest first from a work list built on the device for each call.  A request with no token gets a zero
 * output row and a zero certificate.  Returns KVQ_EWORKSPACE if ws_bytes is
 * too small.
 * Range of the matrix-core stage 1 (KIVI2, KITTY, KITTY_DYN and KIVI4
 * without KVQ_FLAG_GENERIC_STAGE1): it feeds q_c s_c (key scales) and p_t s_t
 * (value scales, with softmax weights p_t <= 256 by the lazily moved
 * maximum) to f16 products as a head plus remainder pair, so the stated
 * accuracy needs |q_c s_c| < 65504 and every value scale s_t <= 255 (a
 * value group spanning at most 765 for 2-bit codes, 3825 for 4-bit);
 * beyond that the output is unspecified and may be non-finite.  The fp16
 * window, the VALU stage 1 and the WITCERT schemes compute in binary32 and
 * have no such limit.  The matrix-core path reports leaving that range
 * with KVQ_STATUS_RANGE. */
int kvq_decode_attention(const kvq_cache_t *cache, const uint16_t *q, float *out,
                         float *cert, float sm_scale, float kappa,
                         void *workspace, size_t ws_bytes, hipStream_t stream);

/* kvq_decode_attention without a caller-supplied workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The stage-1 partials go to a
 * file-scope device array of KVQ_NOALLOC_SCRATCH_BYTES on the current device
 * (hipGetDevice); its address is resolved once per device, on the first call
 * made with that device current.  Same kernels and results as
 * kvq_decode_attention with a workspace.  Allocates and frees nothing.
 * Returns KVQ_ENOSCRATCH, before any device work, when kvq_workspace_bytes()
 * of the cache exceeds KVQ_NOALLOC_SCRATCH_BYTES (for the GQA workload of 64
 * requests x 32 query heads with 32K-token page tables, 29 MB are needed);
 * KVQ_ELAUNCH if the device or the array's address cannot be obtained.
 * Every call on one GPU shares that GPU's array: calls whose execution
 * overlaps on one GPU (other streams, other threads) race on it and must be
 * ordered by the caller.  Nothing in the array needs clearing between calls:
 * each call writes every partial it reads. */
int kvq_decode_attention_noalloc(const kvq_cache_t *cache, const uint16_t *q, float *out,
                                 float *cert, float sm_scale, float kappa,
                                 hipStream_t stream);

/* Measurement aid for the group kernel (KIVI2 with 2, 4 or 8 query heads per
 * KV head, without KVQ_FLAG_GENERIC_STAGE1): the part of kvq_decode_attention
 * before its merge -- the work-list plan, then stage 1 with the same grid,
 * work list, page loads (descriptors, extents, the two-page ring, the
 * non-temporal hint), register budget, window chunks and partial-row writes
 * -- except that each page's loaded words are folded into one register
 * instead of entering the attention arithmetic.  Its stage-1 time is the
 * floor of the group kernel's access pattern on the current state.  It
 * writes meaningless partials into the workspace and nothing else: no
 * output, no merge, the cache unchanged.  The events of
 * kvq_set_stage1_events bracket its stage 1 as they bracket the decode's.
 * Returns KVQ_EINVAL for a layout that does not run the group kernel,
 * KVQ_ENULL, KVQ_EALIGN (q 16-byte, workspace 256-byte aligned) and
 * KVQ_EWORKSPACE as kvq_decode_attention. */
int kvq_stage1_load_floor(const kvq_cache_t *cache, const uint16_t *q, float sm_scale,
                          void *workspace, size_t ws_bytes, hipStream_t stream);

/* ---- helpers ---------------------------------------------------------- */

/* Bytes of one (page, KV head) block for a layout (0 if invalid). */
int64_t kvq_page_bytes(const kvq_layout_t *layout);

/* Tokens per page for a layout (64 or 256; 0 if invalid). */
int32_t kvq_page_tokens(const kvq_layout_t *layout);

/* Quantized bytes per token per KV head, keys and values together, statistics
 * included (96 for KIVI2, 100 for KITTY with 16 boosted, 160 for KIVI4, 258
 * for WITCERT, 272 + (16 when n_boost > 0) for WITCERT_PAGED). */
double kvq_bytes_per_token(const kvq_layout_t *layout);

/* Workspace bytes kvq_decode_attention needs for this cache. */
size_t kvq_workspace_bytes(const kvq_cache_t *cache);

/* Bulk state for a context ("KIVI" explainer 3.3 prefill split): for requests
 * [req0, req0 + n_req), K, V: device fp16 [n_req][n_kv_heads][ld_tokens][D],
 * lengths: device int32 [n_req].  Leaves each (request, KV head) exactly as
 * streaming its tokens through flush/append would: r_k = ((l-1) mod R) + 1 keys
 * (WITCERT: ((l-1) mod 256) + 1 tokens) stay fp16, values keep the newest R;
 * WITCERT_PAGED: every token quantized. */
int kvq_prefill(const kvq_cache_t *cache, int32_t req0, int32_t n_req,
                const uint16_t *K, const uint16_t *V, int64_t ld_tokens,
                const int32_t *lengths, hipStream_t stream);

/* KITTY static boost set from a calibration slice: calib: device fp16
 * [n_kv_heads][n_tokens][D]; idx_out: device uint8 [n_kv_heads][D].  The
 * n_boost channels with the largest max|x| are boosted (ties to the lower
 * channel), offsets in ascending channel order, others n_boost + 1
 * ("Kitty" summary: Selecting the Top-K Channels; The Boost Index Tensor). */
int kvq_kitty_calibrate(const kvq_cache_t *cache, const uint16_t *calib,
                        int32_t n_tokens, uint8_t *idx_out, hipStream_t stream);

/* WITCERT_PAGED fixed bypass set from a calibration slice: calib: device
 * fp16 [n_kv_heads][n_tokens][D]; idx_out: device uint8 [n_kv_heads][D] in
 * boost_idx's format.  The n_boost RoPE pairs (i, i + 64) with the largest
 * max_t (x_i^2 + x_{i+64}^2) over the slice are bypassed (each square exact
 * in binary32 and the sum rounded once; ties to the lower pair), offsets in
 * ascending channel order ("WitCert" page, certified deployment: a fixed
 * per-(layer, KV head) pair set chosen from the start of a sequence).
 * KVQ_EINVAL for another scheme, n_boost = 0 or n_tokens < 1. */
int kvq_witcert_calibrate(const kvq_cache_t *cache, const uint16_t *calib,
                          int32_t n_tokens, uint8_t *idx_out, hipStream_t stream);

/* Optional timing hook: when both events are non-NULL, kvq_decode_attention
 * records `begin` on its stream right before the stage-1 kernel and `end`
 * right after it (caller-owned events; NULL, NULL turns the hook off). */
int kvq_set_stage1_events(kvq_cache_t *cache, hipEvent_t begin, hipEvent_t end);

/* Static description of a host return code (KVQ_OK, KVQ_E*: code <= 0) or
 * of a device status word (code > 0): one KVQ_STATUS_* bit gets its own
 * description, several bits "several device status bits", a word with an
 * undefined bit "unknown". */
const char *kvq_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
