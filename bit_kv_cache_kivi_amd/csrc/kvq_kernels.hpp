// kvq_kernels.hpp -- kernel parameter block and launch declarations shared by
// the host API (kvq_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct KParams {
    uint8_t *pool;
    const int32_t *table;
    int32_t *state;
    uint16_t *res_k;
    uint16_t *res_v;
    const uint8_t *boost_idx;
    uint32_t *status;
    uint16_t *sink_k;             // [B][Hkv][sink][D] fp16 (sink > 0)
    uint16_t *sink_v;
    int B, Hq, Hkv, R, max_pages, n_pages, page_bytes, scheme, qpk, split_pages;
    int sink;                     // leading fp16 tokens; quantized positions are t - sink
    int nb;                       // Kitty boosted channels (16 or 32); WITCERT_PAGED
                                  // bypassed RoPE pairs (0 .. 4); 0 for others
    int force_generic;            // 1: use the per-query-head VALU stage 1
    uint32_t layer;
    uint64_t seed;
};

// Stage-1 partial results: per (request, query head, split):
//   o[128] fp32 (acc / l_s), then {lse_s, A_s} fp32 pairs.
// Stage-1 partials: per query head, rows 0 .. max_splits-1 for the paged
// splits and rows max_splits .. max_splits+n_win-1 for the 64-token chunks
// of the fp16 window, the last of them the sink tokens when there are any.
struct Workspace {
    float *o;        // [B][Hq][max_splits + n_win][128]
    float2 *ml;      // [B][Hq][max_splits + n_win]  (lse in log2 units, A)
    uint4 *items;    // [B * Hkv * max_splits] stage-1 work list (GQA kernel):
                     // {b Hkv + h, partial row, first page, pages | valid
                     // tokens of the pair's last page << 8 (0: none here)}
    uint32_t *n_items;  // its length
    int max_splits;
    int n_win;       // window chunks: residual / 64 (KIVI2 / KITTY) + 1 with sink tokens,
                     // 4 (WITCERT), 0 (WITCERT_PAGED)
    hipEvent_t ev_begin, ev_end;   // optional stage-1 timing events
};

// Row of the partial of query head hq of request b, split s (s >= max_splits:
// window chunk s - max_splits).
__host__ __device__ inline size_t part_row(const Workspace &W, int Hq, int b, int hq, int s) {
    return ((size_t)b * Hq + hq) * (size_t)(W.max_splits + W.n_win) + s;
}

// write path (kvq_write.hip)
hipError_t launch_append(const KParams &P, const uint16_t *k, const uint16_t *v, hipStream_t s);
hipError_t launch_flush(const KParams &P, hipStream_t s);
hipError_t launch_prefill(const KParams &P, int req0, int n_req, const uint16_t *K,
                          const uint16_t *V, long long ld, const int32_t *lengths,
                          hipStream_t s);
hipError_t launch_kitty_calibrate(const KParams &P, const uint16_t *calib, int n_tokens,
                                  uint8_t *idx_out, hipStream_t s);
hipError_t launch_witcert_calibrate(const KParams &P, const uint16_t *calib, int n_tokens,
                                    uint8_t *idx_out, hipStream_t s);

// read path (kvq_decode.hip)
hipError_t launch_decode(const KParams &P, const uint16_t *q, float *out, float *cert,
                         float sm_scale, float kappa, const Workspace &W, hipStream_t s);

// The work-list plan and the group kernel's load-only stage 1
// (kvq_stage1_load_floor); hipErrorInvalidValue for layouts that do not run
// the group kernel.
hipError_t launch_stage1_floor(const KParams &P, const uint16_t *q, float sm_scale, const Workspace &W,
                               hipStream_t s);

// Device address of the fixed scratch array of the current device (resolved
// once per device with hipGetSymbolAddress); *bytes gets its size.
hipError_t noalloc_scratch(void **ptr, size_t *bytes);

}  // namespace kvq
