// kvq_decode.hip -- read path: split-KV stage 1 over the quantized prefix and
// the fp16 window, stage 2 (log-sum-exp merge).
//
// Attention for query head h of KV head g: z_t = sm_scale q.k~_t over every
// token, p = softmax(z), o = sum_t p_t v~_t, with k~, v~ the dequantized or
// fp16 tokens ("KIVI" explainer eq. 3).  Stage 1 takes the prefix [0, n_vq)
// whose keys and values are both quantized, split into runs of pages, and the
// fp16 window (keys of [n_vq, n_kq) still 2-bit) and sink tokens in 64-token
// chunks, and emits per split or chunk (acc / l_s, lse_s, A_s); stage 2
// merges every partial with log-sum-exp weights; the certificate A_s merges
// with the same weights ("WitCert" Key structure).  Scores are kept in log2
// units: z2 = z log2(e).
//
// Folding: for a key group, q.k~ = sum_c (q_c s_c) code_c + sum_c q_c z_c;
// for a value group, sum_t p_t v~_t = sum_t (p_t s_t) code_t + sum_t p_t z_t.
// Only small integer codes are touched per element.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "kvq.h"
#include "kvq_common.hpp"
#include "kvq_kernels.hpp"

// Stage-1 partials of kvq_decode_attention_noalloc: one array per device,
// kept for the life of the process.  Host code must use the address from
// hipGetSymbolAddress (per device), never this name.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace kvq {

typedef float float2v __attribute__((ext_vector_type(2)));

__device__ inline const uint8_t *cpage(const KParams &P, int pid, int h) {
    return P.pool + ((size_t)pid * P.Hkv + h) * (size_t)P.page_bytes;
}

// Two codes (nibbles 2*sel, 2*sel+1 of a masked dword) as exact floats: a
// 2-bit code c in the low bits of a nibble is the fp4 (e2m1) value c/2.
__device__ inline float2v cvt2(uint32_t x, int sel) {
    switch (sel) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 2.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 2.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 2.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 2.0f, 3);
    }
}
#define CVT2(x, sel) cvt2((x), (sel))

// ---------------------------------------------------------------------------
// Stage 1, KIVI2 / KITTY, one query head per wave (VALU).
// Lane L = 16 g + r.  Key side: the lane's dwords hold tokens 16n + r
// (n = 0..3) for its 32 channels 32kc + 8g + j; partial scores are summed
// over g.  Value side: channels 16d + r (d = 0..7) over tokens 32ks + 8g + j;
// partial outputs are summed over g at the end.
// ---------------------------------------------------------------------------
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// Keeps a binary32 value opaque to the optimizer, so every later use sees the
// same rounded number (no re-derivation of it from its operands).
__device__ inline float pin(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// f16 remainder pair of two binary32 values against their packed f16 heads h
// (one per half): each half is fl16(a - head), formed by the mixed-precision
// fused multiply-add in one rounding (a - head is exact in binary32).
__device__ inline uint32_t rem_pair(float a0, float a1, uint32_t h) {
    uint32_t lo;
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=&v"(lo) : "v"(h), "v"(a0));
    asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(lo) : "v"(h), "v"(a1));
    return lo;
}

// LDS ordering for a workgroup of one wave.  The lanes run in lockstep and
// the LDS serves one wave's accesses in issue order, so keeping the compiler
// from moving LDS accesses across this point is enough.  Unlike a workgroup
// barrier with a fence it waits for nothing: the page loads in flight are
// not waited for.
__device__ inline void lds_sync() {
    asm volatile("" ::: "memory");
}

// A matrix-core stage-1 split whose result is not finite: an f16 operand head
// (q_c s_c or p_t s_t) overflowed, or the inputs were not finite.  Reported
// in the status word; the partial is written as it came out.
__device__ inline void flag_range(const KParams &P, bool bad, int lane) {
    if (__any(bad) && lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_RANGE);
}

// Loads through a buffer descriptor of a page's own extent.  With valid false
// the extent is zero: the loads return zeros and touch no memory, so a loop
// can issue them unconditionally (the wait counts stay exact and the
// prefetched pages stay in flight).  Page loads carry the non-temporal hint:
// every page is read once per step, so the caches should not keep it.
constexpr int LOAD_NT = 2;          // cache-policy bit of a buffer load: nt
__device__ inline __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t *page, bool valid, const Geom &G) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)page, (short)0, valid ? G.bytes : 0, 0x00020000);
}
__device__ inline uint4 bload(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, LOAD_NT));
}
__device__ inline uint32_t bload1(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, LOAD_NT);
}

__device__ inline float half_lo(uint32_t v) { return h2f((uint16_t)(v & 0xffffu)); }
__device__ inline float half_hi(uint32_t v) { return h2f((uint16_t)(v >> 16)); }

// ---------------------------------------------------------------------------
// The fp16-value window of one (request, KV head), as one more stage-1
// partial (row max_splits of each query head).  The window holds the newest
// values that are not quantized yet: the last R tokens for KIVI2 / KITTY
// (values are quantized per token as they leave it, keys per group of G
// tokens when the residual fills; "KIVI" explainer 3.3), the active block for
// WITCERT.  Keys of window tokens below n_kq are already quantized and are
// dequantized here; the others come from the fp16 key residual.
// One wave serves NQ queries of the KV head: lane = token of a 64-token chunk
// for the scores and the online softmax, lane = channel pair for P.V.
// ---------------------------------------------------------------------------
struct WinSmem {
    uint32_t ks[2][256];        // key {s, z} of the (at most two) pages of the chunk's quantized keys
    uint8_t bidx[2][D];         // KITTY_DYN: those pages' boost offsets per channel
    f4v zsh[2][PT];             // scores of the chunk: token -> queries 0..3, 4..7
    float4 pT[PT][2];           // p of the chunk: token -> queries 0..3, 4..7
};

// Two binary32 values split into f16 hi + lo (hi cut toward zero, lo the
// rounded remainder): hi + lo carries each value to within ~2^-22 of it.
__device__ inline void split_hl(float x0, float x1, uint32_t &hi, uint32_t &lo) {
    const float a0 = pin(x0), a1 = pin(x1);
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a0, a1));
    lo = rem_pair(a0, a1, hi);
}

template <int NQ, int VPF, int SCHEME>
__device__ void window_partial(const KParams &P, const uint16_t *__restrict__ q, const Workspace &W,
                               float qscale, int b, int h, int hq0, int wc, int lane, WinSmem &ws) {
    const Geom G = geom(SCHEME, P.nb);
    constexpr bool wit = SCHEME == KVQ_SCHEME_WITCERT;
    constexpr bool kitty = is_kitty(SCHEME);
    constexpr bool dyn = SCHEME == KVQ_SCHEME_KITTY_DYN;
    constexpr bool four = SCHEME == KVQ_SCHEME_KIVI4;
    const int g = lane >> 4, r = lane & 15;
    const size_t bh = (size_t)b * P.Hkv + h;
    const int l = P.state[bh * 4], nkq = P.state[bh * 4 + 1];
    const int S = wit ? 0 : P.sink;
    // the last chunk item is the sink segment [0, min(l, S)) when there is one
    const bool sinkc = S > 0 && wc == W.n_win - 1;
    const int W0 = wit ? nkq : max(S, l - P.R);                // first fp16-value token after the sink
    const int win = wit ? WPT : P.R;
    const int t0 = sinkc ? 0 : W0 + PT * wc;                      // this chunk: [t0, t0 + n)
    const int n = sinkc ? min(l, S) : max(0, min(PT, l - t0));
    const int pA = (t0 - S) / PT;                                 // quantized positions count from S
    const bool anyq = !wit && !sinkc && n > 0 && t0 < nkq;        // uniform: a key of the chunk is quantized

    // every load the chunk needs is issued first: page ids, values (lane =
    // channels 2*lane, 2*lane+1; VPF tokens per round) and the query operand
    int pid_l = -1;
    if (anyq && lane < 2 && S + (pA + lane) * PT < min(t0 + n, nkq)) {
        pid_l = P.table[(size_t)b * P.max_pages + pA + lane];
        if (pid_l < 0 || pid_l >= P.n_pages) {
            atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
            pid_l = 0;                            // read page 0 instead; the result is flagged
        }
    }
    // values of tokens tt0 .. tt0 + VPF - 1; with 2 VPF = PT the chunk's
    // values come in two batches, the second loaded once the scores no longer
    // hold the keys' registers
    constexpr bool two = 2 * VPF == PT;
    uint32_t vv[VPF], vv2[two ? VPF : 1];
    auto load_v = [&](int tt0, uint32_t *v) {
        if (sinkc) {
#pragma unroll
            for (int u = 0; u < VPF; u++)
                v[u] = tt0 + u < n ? *(const uint32_t *)(P.sink_v + (bh * S + (size_t)(tt0 + u)) * D + 2 * lane) : 0u;
            return;
        }
        int slot = wit ? t0 + tt0 - nkq : (t0 + tt0) % P.R;
#pragma unroll
        for (int u = 0; u < VPF; u++) {
            v[u] = tt0 + u < n ? *(const uint32_t *)(P.res_v + (bh * win + (size_t)slot) * D + 2 * lane) : 0u;
            if (++slot == win) slot = 0;          // the value ring wraps (KIVI2 / KITTY)
        }
    };
    load_v(0, vv);
    // A operand of the score product: row = query (exact in f16), k = channel
    // 32 kc + 8 g + i; rows NQ..15 are zero
    h8v aq[4];
#pragma unroll
    for (int kc = 0; kc < 4; kc++) {
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (r < NQ) raw = *(const uint4 *)(q + ((size_t)b * P.Hq + hq0 + r) * D + 32 * kc + 8 * g);
        aq[kc] = __builtin_bit_cast(h8v, raw);
    }
    // the fp16 keys of tile nt (token t0 + 16 nt + r, channels 32 kc + 8 g
    // ..; zero where the token has none), all four tiles loaded before the
    // first product
    auto load_kf16 = [&](int nt, uint4 (&k)[4]) {
        const int tt = 16 * nt + r, t = t0 + tt;
#pragma unroll
        for (int kc = 0; kc < 4; kc++) k[kc] = make_uint4(0u, 0u, 0u, 0u);
        if (tt < n && (wit || sinkc || t >= nkq)) {
            const uint4 *kr = sinkc ? (const uint4 *)(P.sink_k + (bh * S + (size_t)t) * D)
                                    : (const uint4 *)(P.res_k + (bh * win + (size_t)(t - nkq)) * D);
#pragma unroll
            for (int kc = 0; kc < 4; kc++) k[kc] = kr[4 * kc + g];
        }
    };
    uint4 kf16[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; nt++) load_kf16(nt, kf16[nt]);
    int pids[2] = {-1, -1};
    if (anyq) {
        pids[0] = __builtin_amdgcn_readlane(pid_l, 0);
        pids[1] = __builtin_amdgcn_readlane(pid_l, 1);
#pragma unroll
        for (int pi = 0; pi < 2; pi++)
            if (pids[pi] >= 0) ((uint4 *)ws.ks[pi])[lane] = ((const uint4 *)(cpage(P, pids[pi], h) + G.ks))[lane];
        if (dyn) {                                // channel -> offset from the pages' channel ids
#pragma unroll
            for (int pi = 0; pi < 2; pi++) {
                ws.bidx[pi][2 * lane] = (uint8_t)(NB_MAX + 1);
                ws.bidx[pi][2 * lane + 1] = (uint8_t)(NB_MAX + 1);
            }
            lds_sync();
            if (lane < 2 * P.nb) {
                const int pi = lane / P.nb, o = lane % P.nb;
                if (pids[pi] >= 0) ws.bidx[pi][cpage(P, pids[pi], h)[G.ki + o] & (D - 1)] = (uint8_t)o;
            }
        }
    }
    lds_sync();

    // ---- scores on the matrix cores: tile nt = tokens t0 + 16 nt .. + 15;
    // B lane: token t0 + 16 nt + r, channels 32 kc + 8 g + i ----
#pragma unroll 1
    for (int nt = 0; nt < 4; nt++) {
        f4v sc = f4v{0.f, 0.f, 0.f, 0.f};
        const int tt = 16 * nt + r, t = t0 + tt;
        uint4 bh4[4], bl4[4];
#pragma unroll
        for (int kc = 0; kc < 4; kc++) {
            bh4[kc] = kf16[0][kc];                // fp16 key (zero where none): exact in the operand
            bl4[kc] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 3; u++)               // the next tiles move down
#pragma unroll
            for (int kc = 0; kc < 4; kc++) kf16[u][kc] = kf16[u + 1][kc];
        if (tt < n) {
            if (wit || sinkc || t >= nkq) {
            } else {                              // quantized key: fl32(code s + z), split hi + lo
                const int pi = (t - S) / PT - pA, tp = (t - S) % PT, gi = tp >> 5, n16 = tp >> 4;
                const uint8_t *pg = cpage(P, pi ? pids[1] : pids[0], h);
                const uint32_t *kcw = (const uint32_t *)(pg + G.kc);
                uint32_t xa[4];                   // KIVI2: xa[0..1]; KIVI4: one dword per kc
#pragma unroll
                for (int a = 0; a < 4; a++) {
                    if (four) {
                        xa[a] = kcw[256 * n16 + 4 * (16 * g + (tp & 15)) + a];
                    } else if (a < 2) {
                        const int d = 2 * n16 + a;
                        xa[a] = kcw[(d >> 2) * 256 + (16 * g + (tp & 15)) * 4 + (d & 3)];
                    }
                }
                uint32_t kh[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};   // offsets 4u .. 4u+3
                if (kitty) {
#pragma unroll
                    for (int u = 0; u < 8; u++)
                        if (4 * u < P.nb)
                            kh[u] = ((const uint32_t *)(pg + G.kh))[64 * (u >> 2) + 16 * (u & 3) + (tp & 15)];
                }
                const int hsh = 2 * (n16 >> 1) + 16 * (n16 & 1);
#pragma unroll
                for (int kc = 0; kc < 4; kc++) {
                    const uint4 s0 = *(const uint4 *)&ws.ks[pi][128 * gi + 32 * kc + 8 * g];
                    const uint4 s1 = *(const uint4 *)&ws.ks[pi][128 * gi + 32 * kc + 8 * g + 4];
                    const uint32_t sz[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                    float kf[8];
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const uint32_t code0 = four ? (xa[kc] >> (8 * (i & 3) + 4 * (i >> 2))) & 15u
                                                    : (xa[kc >> 1] >> (4 * i + 2 * (kc & 1))) & 3u;
                        uint32_t code = code0;
                        if (kitty) {
                            const int o = dyn ? ws.bidx[pi][32 * kc + 8 * g + i]
                                              : P.boost_idx[(size_t)h * D + 32 * kc + 8 * g + i];
                            if (o < P.nb) code |= ((kh[o >> 2] >> (hsh + 4 * (o & 3))) & 3u) << 2;
                        }
                        kf[i] = fmaf((float)code, half_lo(sz[i]), half_hi(sz[i]));   // code * s exact
                    }
                    uint32_t hv[4], lv[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) split_hl(kf[2 * e], kf[2 * e + 1], hv[e], lv[e]);
                    bh4[kc] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
                    bl4[kc] = make_uint4(lv[0], lv[1], lv[2], lv[3]);
                }
            }
        }
#pragma unroll
        for (int kc = 0; kc < 4; kc++) {
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[kc], __builtin_bit_cast(h8v, bh4[kc]), sc, 0, 0, 0);
            if (anyq)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[kc], __builtin_bit_cast(h8v, bl4[kc]), sc, 0, 0, 0);
        }
        // C rows 0..3 (queries 0..3) sit in lanes 0..15, rows 4..7 in lanes 16..31
        if (lane < 16 * ((NQ + 3) / 4)) ws.zsh[g][16 * nt + r] = sc;
    }
    lds_sync();

    if (two && n > VPF) load_v(VPF, vv2);      // uniform

    // ---- softmax over the chunk, lane = token (log2 units) ----
    float zq[8];
    {
        const f4v z0 = ws.zsh[0][lane];
        zq[0] = z0[0]; zq[1] = z0[1]; zq[2] = z0[2]; zq[3] = z0[3];
        if (NQ > 4) {
            const f4v z1 = ws.zsh[1][lane];
            zq[4] = z1[0]; zq[5] = z1[1]; zq[6] = z1[2]; zq[7] = z1[3];
        }
    }
    float m[NQ], lsum[NQ], pv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NQ; j++) {
        const float zz = lane < n ? zq[j] * qscale : -INFINITY;
        float mx = zz;
#pragma unroll
        for (int msk = 1; msk < 64; msk <<= 1) mx = fmaxf(mx, shfl_xor(mx, msk));
        const float p = n > 0 ? __builtin_amdgcn_exp2f(zz - mx) : 0.f;
        float sum = p;
#pragma unroll
        for (int msk = 1; msk < 64; msk <<= 1) sum += shfl_xor(sum, msk);
        m[j] = mx;
        lsum[j] = sum;
        pv[j] = p;
    }
    ws.pT[lane][0] = make_float4(pv[0], pv[1], pv[2], pv[3]);
    if (NQ > 4) ws.pT[lane][1] = make_float4(pv[4], pv[5], pv[6], pv[7]);
    lds_sync();

    // ---- P.V, lane = channels 2*lane, 2*lane+1 ----
    float acc[NQ][2];
#pragma unroll
    for (int j = 0; j < NQ; j++) acc[j][0] = acc[j][1] = 0.f;
    auto pv_batch = [&](const uint32_t *v, int tt0) {
#pragma unroll
        for (int u = 0; u < VPF; u++) {
            const int tt = tt0 + u;
            if (tt < n) {
                const float v0 = half_lo(v[u]), v1 = half_hi(v[u]);
                const float4 pa = ws.pT[tt][0];
                float pq[8] = {pa.x, pa.y, pa.z, pa.w, 0.f, 0.f, 0.f, 0.f};
                if (NQ > 4) {
                    const float4 pb = ws.pT[tt][1];
                    pq[4] = pb.x; pq[5] = pb.y; pq[6] = pb.z; pq[7] = pb.w;
                }
#pragma unroll
                for (int j = 0; j < NQ; j++) {
                    acc[j][0] = fmaf(pq[j], v0, acc[j][0]);
                    acc[j][1] = fmaf(pq[j], v1, acc[j][1]);
                }
            }
        }
    };
    if (two) {
        pv_batch(vv, 0);
        if (n > VPF) pv_batch(vv2, VPF);
    } else {
#pragma unroll 1
        for (int tt0 = 0; tt0 < n; tt0 += VPF) {
            if (tt0 > 0) load_v(tt0, vv);
            pv_batch(vv, tt0);
        }
    }

    // ---- the chunk's partial (an empty chunk gets lse = -inf) ----
#pragma unroll
    for (int j = 0; j < NQ; j++) {
        const size_t row = part_row(W, P.Hq, b, hq0 + j, W.max_splits + wc);
        const float il = lsum[j] > 0.f ? 1.0f / lsum[j] : 0.f;
        *(float2 *)(W.o + row * D + 2 * lane) = make_float2(acc[j][0] * il, acc[j][1] * il);
        if (lane == 0) W.ml[row] = make_float2(n > 0 ? m[j] + log2f(lsum[j]) : -INFINITY, 1.0f);
    }
}

// Work item of a stage-1 workgroup.  The grid has max_splits + n_win items
// per (head, request): the paged splits of every (head, request) first in the
// dispatch order, then the window chunks, which are shorter and fill the
// compute units as the splits drain.
struct S1Item {
    bool window;
    int s, hd, b;        // s: paged split, or window chunk for a window item
};

__device__ inline S1Item s1_item(int max_splits, int n_win) {
    const int nh = gridDim.y, nb = gridDim.z;
    const int L = blockIdx.x + gridDim.x * (blockIdx.y + nh * blockIdx.z);
    const int npg = nh * nb * max_splits;
    S1Item it;
    if (L >= npg) {
        const int L2 = L - npg;
        it.window = true;
        it.s = L2 % n_win;
        const int rest = L2 / n_win;
        it.hd = rest % nh;
        it.b = rest / nh;
    } else {
        it.window = false;
        it.s = L % max_splits;
        const int rest = L / max_splits;
        it.hd = rest % nh;
        it.b = rest / nh;
    }
    return it;
}

template <bool KITTY>
__global__ __launch_bounds__(64) void stage1_valu_kernel(KParams P, const uint16_t *__restrict__ q,
                                                         Workspace W, float qscale) {
    const S1Item it = s1_item(W.max_splits, W.n_win);
    const int s = it.s, hq = it.hd, b = it.b;
    const int lane = threadIdx.x, g = lane >> 4, r = lane & 15;
    const int h = hq / P.qpk;
    const Geom G = geom(P.scheme, P.nb);
    __shared__ union {
        struct {
            uint32_t kss[256];
            float4 wsh[PT];
            int inv[NB];
        } pg;
        WinSmem win;
    } U;
    if (it.window) {                             // this query head's fp16 window
        window_partial<1, 16, KITTY ? KVQ_SCHEME_KITTY : KVQ_SCHEME_KIVI2>(P, q, W, qscale, b, h, hq, s, lane, U.win);
        return;
    }
    const size_t bh = (size_t)b * P.Hkv + h;
    const int l = P.state[bh * 4];
    const int nvq = max(0, l - P.sink - P.R);          // quantized values, counted from the sink
    const int npages = (nvq + PT - 1) / PT;
    const int p0 = s * P.split_pages;
    const int p1 = min(p0 + P.split_pages, npages);
    if (p0 >= p1) return;

    uint32_t *kss = U.pg.kss;
    float4 *wsh = U.pg.wsh;
    int *inv = U.pg.inv;

    const uint16_t *qh = q + ((size_t)b * P.Hq + hq) * D;
    float qv[32];
#pragma unroll
    for (int kc = 0; kc < 4; kc++) {
        const uint4 raw = *(const uint4 *)(qh + 32 * kc + 8 * g);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            qv[8 * kc + 2 * i] = h2f((uint16_t)(w4[i] & 0xffff));
            qv[8 * kc + 2 * i + 1] = h2f((uint16_t)(w4[i] >> 16));
        }
    }
    float qb[4] = {0.f, 0.f, 0.f, 0.f};
    int slotb[4] = {0, 0, 0, 0};
    if (KITTY) {
        if (lane < NB) inv[lane] = 0;
        lds_sync();
        for (int c = lane; c < D; c += 64) {
            const int o = P.boost_idx[(size_t)h * D + c];
            if (o < NB) inv[o] = c;
        }
        lds_sync();
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = inv[4 * g + i];
            qb[i] = h2f(qh[c]);
            slotb[i] = key_stat_slot(c);
        }
    }

    float m = -INFINITY;           // running max (log2 units)
    float lpart = 0.f;             // this lane's share of sum p (token = lane)
    float o[8];                    // channels 16d + r, tokens of lane group g
    float zacc[4] = {0.f, 0.f, 0.f, 0.f};   // sum_t p_t z_{t,jv}, token = lane
#pragma unroll
    for (int d = 0; d < 8; d++) o[d] = 0.f;

    // the split's page ids, one per lane (an id outside the pool is flagged
    // and page 0 read instead)
    const int np = p1 - p0;                      // <= split_pages <= 64
    int pid_l = (lane < np && p0 + lane < P.max_pages) ? P.table[(size_t)b * P.max_pages + p0 + lane] : 0;
    const bool bad = lane < np && (pid_l < 0 || pid_l >= P.n_pages);
    if (__any(bad)) {
        if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
        pid_l = bad ? 0 : pid_l;
    }
    const uint8_t *base = P.pool + (size_t)h * P.page_bytes;
    const size_t pstride = (size_t)P.Hkv * P.page_bytes;
    struct VPage {
        uint4 ksz, vsz, ka, kb, va, vb;
        uint32_t khw;
    };
    // two register sets used in turn: the next page loads while this one is
    // processed (unconditional loads, empty extent past the split's end)
    auto ldp = [&](int i) {
        const uint8_t *pg = base + (size_t)__builtin_amdgcn_readlane(pid_l, min(i, np - 1)) * pstride;
        const __amdgpu_buffer_rsrc_t rs = page_rsrc(pg, i < np, G);
        const int o = 16 * lane;
        VPage R;
        R.ksz = bload(rs, G.ks + o);
        R.vsz = bload(rs, G.vs + o);
        R.ka = bload(rs, G.kc + o);
        R.kb = bload(rs, G.kc + 1024 + o);
        R.va = bload(rs, G.vc + o);
        R.vb = bload(rs, G.vc + 1024 + o);
        R.khw = KITTY ? bload1(rs, G.kh + 4 * lane) : 0u;
        __builtin_amdgcn_sched_barrier(0);
        return R;
    };
    auto run_page = [&](const VPage &R, int p) {
        const uint4 ka = R.ka, kb = R.kb, va = R.va, vb = R.vb, vsz = R.vsz, ksz = R.ksz;
        const uint32_t khw = R.khw;
        lds_sync();                                 // previous page's LDS reads done
        ((uint4 *)kss)[lane] = ksz;
        lds_sync();

        // ---- scores --------------------------------------------------------
        const uint32_t kd[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
        float part[4];
#pragma unroll
        for (int gi = 0; gi < 2; gi++) {
            float a[32];
            float bias = 0.f;
#pragma unroll
            for (int i = 0; i < 32; i++) {
                const uint32_t sz = kss[128 * gi + 32 * (i >> 3) + 8 * g + (i & 7)];
                const float sc = h2f((uint16_t)(sz & 0xffff));
                const float ze = h2f((uint16_t)(sz >> 16));
                a[i] = qv[i] * sc;
                bias = fmaf(qv[i], ze, bias);
            }
            float ab[4] = {0.f, 0.f, 0.f, 0.f};
            if (KITTY) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint32_t sz = kss[128 * gi + slotb[i]];
                    ab[i] = 4.0f * qb[i] * h2f((uint16_t)(sz & 0xffff));
                }
            }
#pragma unroll
            for (int nn = 0; nn < 2; nn++) {
                const int n = 2 * gi + nn;
                float acc = bias;
#pragma unroll
                for (int dd = 0; dd < 2; dd++) {             // d = 2n + dd: kc = 2dd + h
                    const uint32_t x = kd[2 * n + dd];
                    const uint32_t x0 = x & 0x33333333u, x1 = (x >> 2) & 0x33333333u;
#pragma unroll
                    for (int sel = 0; sel < 4; sel++) {
                        const float2v c0 = CVT2(x0, sel), c1 = CVT2(x1, sel);
                        const int kcl = 2 * dd, kch = 2 * dd + 1;
                        acc = fmaf(a[8 * kcl + 2 * sel], c0.x, acc);
                        acc = fmaf(a[8 * kcl + 2 * sel + 1], c0.y, acc);
                        acc = fmaf(a[8 * kch + 2 * sel], c1.x, acc);
                        acc = fmaf(a[8 * kch + 2 * sel + 1], c1.y, acc);
                    }
                }
                if (KITTY) {
                    // high plane: n&1 selects nibble block, n>>1 the 2-bit half
                    const uint32_t hx = ((n >> 1) ? (khw >> 2) : khw) & 0x33333333u;
                    const int sb = 2 * (n & 1);
                    const float2v h0 = CVT2(hx, sb), h1 = CVT2(hx, sb + 1);
                    acc = fmaf(ab[0], h0.x, acc);
                    acc = fmaf(ab[1], h0.y, acc);
                    acc = fmaf(ab[2], h1.x, acc);
                    acc = fmaf(ab[3], h1.y, acc);
                }
                part[n] = acc;
            }
        }
#pragma unroll
        for (int n = 0; n < 4; n++) {
            part[n] += shfl_xor(part[n], 16);
            part[n] += shfl_xor(part[n], 32);
        }
        // ---- online softmax --------------------------------------------------
        const int tbase = p * PT;
        float z2[4];
        float mloc = -INFINITY;
#pragma unroll
        for (int n = 0; n < 4; n++) {
            const bool valid = tbase + 16 * n + r < nvq;
            z2[n] = valid ? part[n] * qscale : -INFINITY;
            mloc = fmaxf(mloc, z2[n]);
        }
#pragma unroll
        for (int msk = 1; msk < 16; msk <<= 1) mloc = fmaxf(mloc, shfl_xor(mloc, msk));
        const float mnew = fmaxf(m, mloc);
        const float alpha = exp2f(m - mnew);
        m = mnew;
        float pn[4];
#pragma unroll
        for (int n = 0; n < 4; n++) pn[n] = exp2f(z2[n] - mnew);     // -inf -> 0
        const float pt = g == 0 ? pn[0] : g == 1 ? pn[1] : g == 2 ? pn[2] : pn[3];
        const bool tvalid = tbase + lane < nvq;                    // token = lane
        lpart = lpart * alpha + pt;
        const uint32_t vw[4] = {vsz.x, vsz.y, vsz.z, vsz.w};
        float4 wv;
        float wtmp[4];
#pragma unroll
        for (int jv = 0; jv < 4; jv++) {
            const float sv = h2f((uint16_t)(vw[jv] & 0xffff));
            const float zv = h2f((uint16_t)(vw[jv] >> 16));
            wtmp[jv] = tvalid ? pt * sv : 0.f;
            zacc[jv] = zacc[jv] * alpha + (tvalid ? pt * zv : 0.f);
        }
        wv.x = wtmp[0]; wv.y = wtmp[1]; wv.z = wtmp[2]; wv.w = wtmp[3];
        wsh[lane] = wv;
#pragma unroll
        for (int d = 0; d < 8; d++) o[d] *= alpha;
        lds_sync();

        // ---- P.V -------------------------------------------------------------
        float4 wt[16];
#pragma unroll
        for (int ks = 0; ks < 2; ks++)
#pragma unroll
            for (int j = 0; j < 8; j++) wt[8 * ks + j] = wsh[32 * ks + 8 * g + j];
        const uint32_t vd[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int d = 0; d < 8; d++) {
            const int jv = d >> 1;
            const uint32_t x = vd[d];
            const uint32_t x0 = x & 0x33333333u, x1 = (x >> 2) & 0x33333333u;
            float acc = o[d];
#pragma unroll
            for (int sel = 0; sel < 4; sel++) {
                const float2v c0 = CVT2(x0, sel), c1 = CVT2(x1, sel);
                const float4 w0 = wt[2 * sel], w1 = wt[2 * sel + 1];
                const float4 w2 = wt[8 + 2 * sel], w3 = wt[8 + 2 * sel + 1];
                const float f0 = jv == 0 ? w0.x : jv == 1 ? w0.y : jv == 2 ? w0.z : w0.w;
                const float f1 = jv == 0 ? w1.x : jv == 1 ? w1.y : jv == 2 ? w1.z : w1.w;
                const float f2 = jv == 0 ? w2.x : jv == 1 ? w2.y : jv == 2 ? w2.z : w2.w;
                const float f3 = jv == 0 ? w3.x : jv == 1 ? w3.y : jv == 2 ? w3.z : w3.w;
                acc = fmaf(f0, c0.x, acc);
                acc = fmaf(f1, c0.y, acc);
                acc = fmaf(f2, c1.x, acc);
                acc = fmaf(f3, c1.y, acc);
            }
            o[d] = acc;
        }
    };
    VPage ra = ldp(0);
    for (int i = 0; i < np; i += 2) {
        VPage rb = ldp(i + 1);
        run_page(ra, p0 + i);
        ra = ldp(i + 2);
        if (i + 1 < np) run_page(rb, p0 + i + 1);
    }

    // ---- reduce and write the split's partial ----------------------------------
#pragma unroll
    for (int d = 0; d < 8; d++) {
        o[d] += shfl_xor(o[d], 16);
        o[d] += shfl_xor(o[d], 32);
    }
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) {
        lpart += shfl_xor(lpart, msk);
#pragma unroll
        for (int jv = 0; jv < 4; jv++) zacc[jv] += shfl_xor(zacc[jv], msk);
    }
    const float inv_l = 1.0f / lpart;
    const size_t row = part_row(W, P.Hq, b, hq, s);
    if (g == 0) {
#pragma unroll
        for (int d = 0; d < 8; d++) W.o[row * D + 16 * d + r] = (o[d] + zacc[d >> 1]) * inv_l;
    }
    if (lane == 0) W.ml[row] = make_float2(m + log2f(lpart), 1.0f);
}

// ---------------------------------------------------------------------------
// Stage 1, KIVI2, GQA group of 4 query heads per KV head, on the matrix cores.
// One wave per (split, KV head, request) streams each page once for all four
// query heads.
//
// Scores, C[m][t] = sum_c A[m][c] code_{t,c} with 16x16x32 f16 products:
//   rows m = 0..3 hold hi(q_h s_c), rows 4..7 lo(q_h s_c) = f16 remainder
//   (hi + lo carries the binary32 product to within 2^-22), rows 8..15 zero;
//   B is the page's key codes, exact in f16 (2-bit code c in a nibble is the
//   fp4 value c/2, scaled by 2 on conversion).  The accumulator starts at
//   sum_c q_h z_c; rows h and h+4 are added afterwards.
// P.V, transposed: O^T[c][col] = sum_t code_{t,c} B[t][col], A = value codes
//   (channel rows, token columns).  Channel tile nt (16 channels) lies in
//   value group j = nt / 2; B column (query h, part, js) holds the hi (part
//   0) or lo (part 1) half of p_{h,t} s_{t,j} with j = js for tiles 0..3 and
//   j = 2 + js for tiles 4..7, so one product per tile and 32-token step
//   carries both halves of all four queries; columns (h, 0, js) and
//   (h, 1, js) are added at the end.  sum_t p_{h,t} z_{t,j} is accumulated
//   on the side.
// Online softmax with lazy rescaling: the running maximum m moves only when a
// score exceeds m + 8 (log2 units), so p <= 256 and the rescale is rare; the
// split's lse = m + log2(l) stays exact.
// ---------------------------------------------------------------------------

__device__ inline h2v cvth(uint32_t x, int sel) {
    switch (sel) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 3);
    }
}


// eight codes held in the nibbles of a masked dword -> f16 fragment (k = nibble)
__device__ inline h8v frag8(uint32_t m) {
    const u4v v = {__builtin_bit_cast(uint32_t, cvth(m, 0)), __builtin_bit_cast(uint32_t, cvth(m, 1)),
                   __builtin_bit_cast(uint32_t, cvth(m, 2)), __builtin_bit_cast(uint32_t, cvth(m, 3))};
    return __builtin_bit_cast(h8v, v);
}


constexpr float LAZY_TAU = 8.0f;

// a = fl32(x * y) for two pairs, split into f16 hi + lo with hi + lo = a to
// within half an ulp of lo: hi is cut by round-toward-zero in one packed
// conversion and lo is the remainder.  a is pinned, so hi and lo come from the
// same rounded product.
__device__ inline void mul_split2(float x0, _Float16 y0, float x1, _Float16 y1, uint32_t &hi, uint32_t &lo) {
    const float a0 = pin(__builtin_fmaf(x0, (float)y0, 0.0f));     // the rounded product
    const float a1 = pin(__builtin_fmaf(x1, (float)y1, 0.0f));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a0, a1));
    lo = rem_pair(a0, a1, hi);
}

// hi + lo of the two products q0 s0 and q1 s1, q = (q0, q1) and s2 = (s0, s1)
// packed f16 pairs: hi = fl16(q s) by one packed f16 multiply and lo =
// fl16(q s - hi) by one packed fused multiply-add.  An f16 x f16 product is
// exact before its single rounding, so hi + lo is q s to within half an ulp
// of lo.
__device__ inline void split_qs_pk(uint32_t q, uint32_t s2, uint32_t &hi, uint32_t &lo) {
    const h2v qv = __builtin_bit_cast(h2v, q), sv = __builtin_bit_cast(h2v, s2);
    const h2v h = qv * sv;
    const h2v l = __builtin_elementwise_fma(qv, sv, -h);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

// hi + lo of p s0 and p s1 with p binary32 and s0, s1 the f16 in the low
// halves of their registers: hi = fl16(p s), lo = fl16(p s - hi) from the
// fused products, so hi + lo is p s to within ~2^-22 of it.
__device__ inline void split_ps(float p, uint32_t s0, uint32_t s1, uint32_t &hi, uint32_t &lo) {
    uint32_t h, l;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=&v"(h) : "v"(p), "v"(s0));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(h) : "v"(p), "v"(s1));
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,1,1]" : "=&v"(l) : "v"(p), "v"(s0), "v"(h));
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "+v"(l) : "v"(p), "v"(s1), "v"(h));
    hi = h;
    lo = l;
}

// x >> 2 for both dwords of a register pair by one 64-bit shift; the two bits
// the high dword moves into the low one land in its top nibble's upper half,
// which the code mask clears
__device__ inline void shr2_pairs(const uint32_t (&x)[8], uint32_t (&y)[8]) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        uint64_t v;
        asm("v_lshrrev_b64 %0, 2, %1" : "=v"(v) : "v"((((uint64_t)x[i + 1] << 32) | x[i])));
        y[i] = (uint32_t)v;
        y[i + 1] = (uint32_t)(v >> 32);
    }
}

// LDS read with a 4 x 4 transpose per group of four lanes (gfx950): within
// each 16-lane group, element e of lane j is element j & 3 of the 8 bytes
// that lane 4 e + (j >> 2) addresses
__device__ inline h4v lds_tr16(const uint32_t *p) {
    typedef short s4v __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(h4v, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4v *)(__attribute__((address_space(3))) void *)p));
}

template <int CTRL>
__device__ inline float dppf(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, x), CTRL, 0xf, 0xf, true));
}

__device__ inline _Float16 lo16h(uint32_t v) { return __builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu)); }
__device__ inline _Float16 hi16h(uint32_t v) { return __builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

struct PageRegs {
    uint4 ka, kb, va, vb, ks, vs;
};

__device__ inline PageRegs load_page_masked(const uint8_t *page, bool valid, const Geom &G, int lane) {
    const __amdgpu_buffer_rsrc_t rs = page_rsrc(page, valid, G);
    const int o = 16 * lane;
    PageRegs R;                                 // issued in the order of use
    R.ks = bload(rs, G.ks + o);
    R.vs = bload(rs, G.vs + o);
    R.ka = bload(rs, G.kc + o);
    R.kb = bload(rs, G.kc + 1024 + o);
    R.va = bload(rs, G.vc + o);
    R.vb = bload(rs, G.vc + 1024 + o);
    return R;
}

// sum over the 16 lanes of a row; the total lands in the row's lane 15
__device__ inline float row_sum16(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), 0x111, 0xf, 0xf, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), 0x112, 0xf, 0xf, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), 0x114, 0xf, 0xf, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), 0x118, 0xf, 0xf, true));
    return v;
}

struct Gqa4State {
    float m[4];                     // running maximum per query (log2 units), the same in every lane
    float ma, mb;                   // m of this lane's two queries a = 2 (lane >> 4 & 1), a + 1
    float la, lb;                   // this lane's share of l for queries a and a + 1
    float za[4], zb[4];             // sum_t p_t z_{t,j} over this lane's tokens [group j]
    f4v acc[8];
};

// A page's registers: key statistics and codes, the value statistics of the
// lane's two softmax tokens, and the value codes.
struct Gqa4Page {
    uint4 ks, vs0, vs1, ka, kb, va, vb;
};

constexpr int AS_STRIDE = 20;       // octets per score-operand row (16 + bank padding)

// The P.V operand token-major: a token's 16 f16 columns in one row of
// BT_DW dwords, so that a lane stores its token's eight columns of an operand
// with one 16-byte write; the operand fragments are read back column-major by
// transposing LDS reads.  12-dword rows (8 + 4 of padding): the 16-byte
// writes of 16 lanes (16 consecutive tokens) start on 16 distinct 4-bank
// groups of the 64 banks.
constexpr int BT_DW = 12;

// NQW query quads served by one wave (two for a group of 8): each quad its
// own score operand and P.V operand; the zero row is shared.
template <int NQW>
struct Gqa4Smem {
    static constexpr int BTW = BT_DW;   // dwords of a P.V operand row
    h8v As[NQW][2][8][AS_STRIDE];   // score A: [quad][key group][row 2h = hi(q_h s), 2h + 1 = lo][channel octet]
    h8v Az[AS_STRIDE];              // a zero row (the other key group's operand rows)
    uint32_t Bt[NQW][2][PT][BTW];   // P.V B: [quad][operand][token][column pair (h, part, js)]
};

// Token of this lane's first softmax score (the second is 16 later): lane
// 16 G + r holds tokens 32 (G >> 1) + r, + 16, both in key group G >> 1.
__device__ inline int gqa4_token(int lane) { return 32 * (lane >> 5) + (lane & 15); }

__device__ inline Gqa4Page load_gqa4_page(const uint8_t *page, int extent, const Geom &G, int lane) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)page, (short)0, extent, 0x00020000);
    const int o = 16 * lane, t0 = gqa4_token(lane);
    Gqa4Page R;                                 // issued in the order of use
    R.ks = bload(rs, G.ks + o);
    R.ka = bload(rs, G.kc + o);
    R.kb = bload(rs, G.kc + 1024 + o);
    R.vs0 = bload(rs, G.vs + 16 * t0);
    R.vs1 = bload(rs, G.vs + 16 * (t0 + 16));
    R.va = bload(rs, G.vc + o);
    R.vb = bload(rs, G.vc + 1024 + o);
    return R;
}

// One 64-token page.  nvalid < 64 only on the last page of the prefix.
//
// Scores: operand A1 carries key group 0's hi/lo rows in rows 0..7 and zeros
// in rows 8..15, A2 the zeros in rows 0..7 and group 1's rows in rows 8..15;
// accumulator s[n2] takes A1 x tile n2 and A2 x tile n2 + 2.  Lane 16 G + r
// then holds, for queries a = 2 (G & 1) and a + 1, the hi and lo sums of
// token 32 (G >> 1) + r in s[0] and of the token 16 later in s[1]: the
// softmax runs in the products' own layout, two tokens by two queries a
// lane, and every token of a lane is in key group G >> 1.
//
// With NQW = 2 quads a wave (a group of 8), every code fragment is converted
// once and enters the products of both quads; the rest of the step is each
// quad's own.
template <int NQW>
__device__ inline void gqa4_page(const Gqa4Page &R, Gqa4State (&S)[NQW], Gqa4Smem<NQW> &sm,
                                 const uint2 (&qw)[NQW][4], const h8v *const (&a1)[NQW],
                                 const h8v *const (&a2)[NQW], int lane, int nvalid, float qscale) {
    const int g = lane >> 4, r = lane & 15;
    const int hp = r >> 2;
    const uint32_t MSK = 0x33333333u;

    lds_sync();                            // previous page done with the LDS

    // ---- score operand from the lane's own key statistics (key group
    // lane >> 5, channels 4 (lane & 31) .. +3): hi/lo of q_h s_c for the four
    // queries of each quad, and the zero-point sums, added over the group's
    // 32 lanes ----
    const int gi_p = lane >> 5;
    const uint32_t sz[4] = {R.ks.x, R.ks.y, R.ks.z, R.ks.w};
    // the channel pairs' scales and zero points, packed (one permute each,
    // shared by the queries)
    const uint32_t s01 = __builtin_amdgcn_perm(sz[1], sz[0], 0x05040100u);
    const uint32_t s23 = __builtin_amdgcn_perm(sz[3], sz[2], 0x05040100u);
    const uint32_t z01 = __builtin_amdgcn_perm(sz[1], sz[0], 0x07060302u);
    const uint32_t z23 = __builtin_amdgcn_perm(sz[3], sz[2], 0x07060302u);
    // Sum the shares over the 32 lanes of the key group, reduce-scatter
    // style.  With f = (L & 1) ^ (L >> 4 & 1), the first quad exchange keeps
    // queries (0, 1) where f = 0 and (2, 3) where f = 1, the second keeps the
    // first of the pair where L & 2 = 0: quad position p holds query
    // 2 (p & 1 ^ L >> 4 & 1) + (p >> 1), so positions 0 and 2 hold the two
    // queries a, a + 1 of the lane's score layout.  Rotations within the row
    // add the row's quads; the two rows of the group hold a query at quad
    // positions differing in bit 0, hence the exchange with lane ^ 17.
    const bool f = ((lane ^ (lane >> 4)) & 1) != 0, b1 = (lane & 2) != 0;
    float bias_a[NQW], bias_b[NQW];
#pragma unroll
    for (int qd = 0; qd < NQW; qd++) {
        // bzp: this lane's share of sum_c q_h z_c per query, by two f16 dot
        // products into a binary32 sum (each f16 x f16 product exact)
        float bzp[4];
#pragma unroll
        for (int h = 0; h < 4; h++) {
            uint32_t hv0, lv0, hv1, lv1;
            split_qs_pk(qw[qd][h].x, s01, hv0, lv0);
            split_qs_pk(qw[qd][h].y, s23, hv1, lv1);
            ((uint2 *)&sm.As[qd][gi_p][2 * h][0])[lane & 31] = make_uint2(hv0, hv1);
            ((uint2 *)&sm.As[qd][gi_p][2 * h + 1][0])[lane & 31] = make_uint2(lv0, lv1);
            bzp[h] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qw[qd][h].y), __builtin_bit_cast(h2v, z23),
                                            __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qw[qd][h].x),
                                                                   __builtin_bit_cast(h2v, z01), 0.0f, false),
                                            false);
        }
        float k0 = f ? bzp[2] : bzp[0], k1 = f ? bzp[3] : bzp[1];
        k0 += dppf<0xB1>(f ? bzp[0] : bzp[2]);             // quad_perm [1,0,3,2]
        k1 += dppf<0xB1>(f ? bzp[1] : bzp[3]);
        float kq = b1 ? k1 : k0;
        kq += dppf<0x4E>(b1 ? k0 : k1);                    // quad_perm [2,3,0,1]
        kq += dppf<0x124>(kq);                             // row_ror:4
        kq += dppf<0x128>(kq);                             // row_ror:8
        kq += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, kq), 0x441F));  // lane ^ 17
        kq *= qscale;
        bias_a[qd] = dppf<0x00>(kq);
        bias_b[qd] = dppf<0xAA>(kq);
    }
    lds_sync();

    // ---- scores on the matrix cores ----
    const uint32_t kd[8] = {R.ka.x, R.ka.y, R.ka.z, R.ka.w, R.kb.x, R.kb.y, R.kb.z, R.kb.w};
    uint32_t kd2[8];                            // the same >> 2
    shr2_pairs(kd, kd2);
    f4v sc[NQW][2];
#pragma unroll
    for (int qd = 0; qd < NQW; qd++) sc[qd][0] = sc[qd][1] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; kc++) {
        h8v af1[NQW], af2[NQW];
#pragma unroll
        for (int qd = 0; qd < NQW; qd++) {
            af1[qd] = a1[qd][4 * kc + g];
            af2[qd] = a2[qd][4 * kc + g];
        }
        const uint32_t *kx = (kc & 1) ? kd2 : kd;
#pragma unroll
        for (int n2 = 0; n2 < 2; n2++) {
            const h8v bf = frag8(kx[2 * n2 + (kc >> 1)] & MSK);
#pragma unroll
            for (int qd = 0; qd < NQW; qd++)
                sc[qd][n2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af1[qd], bf, sc[qd][n2], 0, 0, 0);
        }
#pragma unroll
        for (int n2 = 0; n2 < 2; n2++) {
            const h8v bf = frag8(kx[2 * (n2 + 2) + (kc >> 1)] & MSK);
#pragma unroll
            for (int qd = 0; qd < NQW; qd++)
                sc[qd][n2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af2[qd], bf, sc[qd][n2], 0, 0, 0);
        }
    }

    const int t0 = gqa4_token(lane);
    // ---- online softmax: tokens t0 and t0 + 16, queries a and a + 1 of
    // each quad; one rescale test for all quads (a quad rescaled without
    // need only moves its maxima up to its scores, which stays exact) ----
    float z[NQW][2][2];                         // [quad][token][query a, a + 1], log2 units
    float d[NQW][2][2];
    float dmax = -INFINITY;
#pragma unroll
    for (int qd = 0; qd < NQW; qd++) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            z[qd][j][0] = fmaf(sc[qd][j][0] + sc[qd][j][1], qscale, bias_a[qd]);
            z[qd][j][1] = fmaf(sc[qd][j][2] + sc[qd][j][3], qscale, bias_b[qd]);
        }
        if (nvalid < PT) {                      // uniform: only the prefix's last page
#pragma unroll
            for (int j = 0; j < 2; j++)
                if (t0 + 16 * j >= nvalid) z[qd][j][0] = z[qd][j][1] = -INFINITY;
        }
        // the exponents against the running maxima; a rescale only when one
        // of them passes LAZY_TAU (-inf - -inf = NaN, where a first page's
        // masked token meets a maximum not yet set, is passed over by fmaxf:
        // the page's valid tokens give +inf)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            d[qd][j][0] = z[qd][j][0] - S[qd].ma;
            d[qd][j][1] = z[qd][j][1] - S[qd].mb;
        }
        dmax = fmaxf(dmax, fmaxf(fmaxf(d[qd][0][0], d[qd][1][0]), fmaxf(d[qd][0][1], d[qd][1][1])));
    }
    if (__any(dmax > LAZY_TAU)) {
#pragma unroll
        for (int qd = 0; qd < NQW; qd++) {
            Gqa4State &Sq = S[qd];
            // the new maxima: over the 32 lanes holding each query (lane bits
            // 0..3 and 5), then moved in every lane
            float mt[2] = {fmaxf(z[qd][0][0], z[qd][1][0]), fmaxf(z[qd][0][1], z[qd][1][1])};
#pragma unroll
            for (int k = 0; k < 2; k++) {
#pragma unroll
                for (int msk = 1; msk < 16; msk <<= 1) mt[k] = fmaxf(mt[k], shfl_xor(mt[k], msk));
                mt[k] = fmaxf(mt[k], shfl_xor(mt[k], 32));
            }
            float alpha[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                // query i lives in lanes 16 (i >> 1) + ..: slot i & 1 of lane 16 (i >> 1)
                const float mi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                     __builtin_bit_cast(int, mt[i & 1]), 16 * (i >> 1)));
                const float mn = fmaxf(Sq.m[i], mi);
                alpha[i] = __builtin_amdgcn_exp2f(Sq.m[i] - mn);
                Sq.m[i] = mn;
            }
            const bool hi2 = (g & 1) != 0;
            Sq.ma = hi2 ? Sq.m[2] : Sq.m[0];
            Sq.mb = hi2 ? Sq.m[3] : Sq.m[1];
            const float aa = hi2 ? alpha[2] : alpha[0], ab = hi2 ? alpha[3] : alpha[1];
            Sq.la *= aa;
            Sq.lb *= ab;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                Sq.za[j] *= aa;
                Sq.zb[j] *= ab;
            }
            const float ap = hp == 0 ? alpha[0] : hp == 1 ? alpha[1] : hp == 2 ? alpha[2] : alpha[3];
#pragma unroll
            for (int nt = 0; nt < 8; nt++) Sq.acc[nt] *= ap;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                d[qd][j][0] = z[qd][j][0] - Sq.ma;
                d[qd][j][1] = z[qd][j][1] - Sq.mb;
            }
        }
    }
#pragma unroll
    for (int qd = 0; qd < NQW; qd++) {
        Gqa4State &Sq = S[qd];
        float p[2][2];                          // [token][query a, a + 1]
#pragma unroll
        for (int j = 0; j < 2; j++) {
            p[j][0] = __builtin_amdgcn_exp2f(d[qd][j][0]);
            p[j][1] = __builtin_amdgcn_exp2f(d[qd][j][1]);
        }
        Sq.la += p[0][0] + p[1][0];
        Sq.lb += p[0][1] + p[1][1];

        // ---- P.V operand: p_{h,t} s_{t,j} split into f16 hi and lo, stored
        // as the B columns (h, part, js) of operand j >> 1 (js = j & 1) at
        // token t; sum_t p_{h,t} z_{t,j} on the side.  (Statistics of tokens
        // past nvalid read as zeros: the page's extent.) ----
        const int ha = 2 * (g & 1);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const uint4 v4 = j ? R.vs1 : R.vs0;
            const uint32_t vw[4] = {v4.x, v4.y, v4.z, v4.w};
            const int t = t0 + 16 * j;
            uint32_t h01[2], l01[2], h23[2], l23[2];
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const float pk = p[j][k];
                float *zk = k ? Sq.zb : Sq.za;
#pragma unroll
                for (int jv = 0; jv < 4; jv++) zk[jv] = fmaf(pk, (float)hi16h(vw[jv]), zk[jv]);
                split_ps(pk, vw[0], vw[1], h01[k], l01[k]);
                split_ps(pk, vw[2], vw[3], h23[k], l23[k]);
            }
            // columns 4 (ha + k) .. + 3 = (hi of groups 2o, 2o + 1, lo of
            // the same) for queries ha + k, k = 0, 1: dwords 2 ha .. + 3
            *(uint4 *)&sm.Bt[qd][0][t][2 * ha] = make_uint4(h01[0], l01[0], h01[1], l01[1]);
            *(uint4 *)&sm.Bt[qd][1][t][2 * ha] = make_uint4(h23[0], l23[0], h23[1], l23[1]);
        }
    }
    lds_sync();

    // ---- P.V on the matrix cores: channel tiles 0..3 (value groups 0, 1)
    // take operand 0, tiles 4..7 (groups 2, 3) operand 1; one product per tile,
    // quad and 32-token step carries both halves of the quad's four queries ----
    const uint32_t vd[8] = {R.va.x, R.va.y, R.va.z, R.va.w, R.vb.x, R.vb.y, R.vb.z, R.vb.w};
    uint32_t vd2[8];                            // the same >> 2
    shr2_pairs(vd, vd2);
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
        const uint32_t *vx = ks ? vd2 : vd;
#pragma unroll
        for (int o = 0; o < 2; o++) {
            // column r, tokens 32 ks + 8 g .. + 7: lane r of the 16-lane
            // group addresses token row 32 ks + 8 g + (r >> 2) (+ 4), columns
            // 4 (r & 3) .. + 3; the transposing read hands lane r column r
            h8v bv[NQW];
#pragma unroll
            for (int qd = 0; qd < NQW; qd++) {
                const uint32_t *rp = &sm.Bt[qd][o][32 * ks + 8 * g + (r >> 2)][2 * (r & 3)];
                const h4v b0 = lds_tr16(rp), b1 = lds_tr16(rp + 4 * Gqa4Smem<NQW>::BTW);
                bv[qd] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int nt = 4 * o + u;
                const h8v af = frag8(vx[nt] & MSK);
#pragma unroll
                for (int qd = 0; qd < NQW; qd++)
                    S[qd].acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bv[qd], S[qd].acc[nt], 0, 0, 0);
            }
        }
    }
}

// Stage-1 work list of the GQA kernel: every split of every (request, KV
// head) pair (gqa_splits), longest first -- the body splits of split_pages
// pages and then the full tail splits, each in (request, KV head, split)
// order, then the short last tail splits by length, longest first, each
// length in pair order.  (With two query quads per KV head, an item's
// wave serves both.)  Workgroups are dispatched in list order
// and round robin over the XCDs, so similar items sit side by side and the
// shortest run last.  PLAN_G workgroups each compute every pair's place (one pass per
// PLAN_T pairs: wave-level prefix sums of the counts and of the short splits
// per length, two barriers) and write the items of their own share of the
// pairs: a pair's items are scattered 16-byte stores, which one compute unit
// issues a lane at a time.
constexpr int PLAN_T = 1024;
constexpr int PLAN_W = PLAN_T / 64;
constexpr int PLAN_G = 8;
constexpr int PLAN_L = 16;                 // short split lengths: below the tail length (<= 16)

// inclusive prefix sums over the wave's lanes of three counters
__device__ inline void wave_scan3(int (&v)[3], int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
        for (int i = 0; i < 3; i++) {
            const int t = __shfl_up(v[i], off, 64);
            if (lane >= off) v[i] += t;
        }
    }
}

__global__ __launch_bounds__(PLAN_T) void plan_kernel(KParams P, Workspace W) {
    // pairs (request, KV head), pair index b Hkv + h
    const int npair = P.B * P.Hkv, sp = P.split_pages, tp = gqa_tail_pages(sp);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int per = (npair + (int)gridDim.x - 1) / (int)gridDim.x;   // this workgroup's pairs
    const int pr0 = (int)blockIdx.x * per, pr1 = min(npair, pr0 + per);
    __shared__ int wtot[3][PLAN_W];        // per-wave totals, then their exclusive prefixes
    __shared__ int wlen[PLAN_L][PLAN_W];   // per-wave short splits of each length, then prefixes
    __shared__ int ctot[3], tlen[PLAN_L];  // the pass's totals
    __shared__ int carry[3], clen[PLAN_L]; // placed by earlier passes
    __shared__ int base[2], blen[PLAN_L];  // region starts: body, full tail; short, by length
    // quantized values of a unit's pair, and its pages (capped by its
    // page-table row)
    auto nvq_of = [&](int pr) { return max(0, P.state[(size_t)pr * 4] - P.sink - P.R); };
    auto pages_of = [&](int nvq) { return min((nvq + PT - 1) / PT, P.max_pages); };
    // a pass: the counts {body, full tail, short} of a pair of npg pages,
    // their exclusive prefix over the pairs so far in v, the rank of its
    // short split among the pairs so far with one of the same length in
    // srank; the pass's totals in ctot and tlen
    auto pass = [&](int npg, int (&cnt)[3], int (&v)[3], int &rem, int &srank) {
        const int nb = gqa_body_splits(npg, sp), rest = npg - nb * sp;
        cnt[0] = nb;
        cnt[1] = rest / tp;
        rem = rest % tp;
        cnt[2] = rem ? 1 : 0;
#pragma unroll
        for (int i = 0; i < 3; i++) v[i] = cnt[i];
        wave_scan3(v, lane);
        if (lane == 63)
#pragma unroll
            for (int i = 0; i < 3; i++) wtot[i][wv] = v[i];
        int rk = 0;
        for (int len = 1; len < tp; len++) {
            const uint64_t m = __ballot(rem == len);
            if (lane == 0) wlen[len][wv] = __builtin_popcountll(m);
            if (rem == len) rk = __builtin_popcountll(m & ((1ull << lane) - 1));
        }
        __syncthreads();
        if (wv == 0) {
            int t[3];
#pragma unroll
            for (int i = 0; i < 3; i++) t[i] = lane < PLAN_W ? wtot[i][lane] : 0;
            int u[3] = {t[0], t[1], t[2]};
            wave_scan3(u, lane);
            if (lane < PLAN_W)
#pragma unroll
                for (int i = 0; i < 3; i++) wtot[i][lane] = u[i] - t[i];
            if (lane == PLAN_W - 1)
#pragma unroll
                for (int i = 0; i < 3; i++) ctot[i] = u[i];
        } else if (wv == 1 && lane < PLAN_L) {  // lane = length
            int acc = 0;
            for (int w = 0; w < PLAN_W; w++) {
                const int c = lane >= 1 && lane < tp ? wlen[lane][w] : 0;
                wlen[lane][w] = acc;
                acc += c;
            }
            tlen[lane] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 3; i++) v[i] += wtot[i][wv] - cnt[i] + carry[i];
        srank = rem ? clen[rem] + wlen[rem][wv] + rk : 0;
    };
    // after a pass: what it placed joins the carries
    auto advance = [&]() {
        __syncthreads();                   // every thread has read the carries
        if (tid < 3) carry[tid] += ctot[tid];
        if (tid < PLAN_L) clen[tid] += tlen[tid];
        __syncthreads();
    };
    // region starts from the totals (in ctot and tlen)
    auto set_bases = [&]() {
        base[0] = 0;
        base[1] = ctot[0];
        int o = ctot[0] + ctot[1];
        for (int len = tp - 1; len >= 1; len--) {
            blen[len] = o;
            o += tlen[len];
        }
        if (blockIdx.x == 0) *W.n_items = (uint32_t)o;
    };
    if (tid < 3) carry[tid] = 0;
    if (tid < PLAN_L) clen[tid] = 0;
    __syncthreads();
    const bool one_pass = npair <= PLAN_T;
    if (!one_pass) {                       // the region starts need every pair's counts first
        for (int c0 = 0; c0 < npair; c0 += PLAN_T) {
            int cnt[3], v[3], rem, srank;
            pass(c0 + tid < npair ? pages_of(nvq_of(c0 + tid)) : 0, cnt, v, rem, srank);
            advance();
        }
        if (tid < 3) ctot[tid] = carry[tid];
        if (tid < PLAN_L) tlen[tid] = clen[tid];
        __syncthreads();
        if (tid == 0) set_bases();
        if (tid < 3) carry[tid] = 0;
        if (tid < PLAN_L) clen[tid] = 0;
        __syncthreads();
    }
    for (int c0 = 0; c0 < npair; c0 += PLAN_T) {
        const int pr = c0 + tid;
        const int nvq = pr < npair ? nvq_of(pr) : 0;
        const int npg = pages_of(nvq);
        int cnt[3], v[3], rem, srank;
        pass(npg, cnt, v, rem, srank);
        if (one_pass && tid == 0) set_bases();  // one pass: its totals are the list's
        __syncthreads();
        if (pr >= pr0 && pr < pr1) {
            const uint32_t nv_last = npg ? (uint32_t)min(PT, nvq - (npg - 1) * PT) : 0u;
            // item of split r: pages [p0, p0 + n); the pair's last page
            // carries its valid-token count
            auto put = [&](int slot, int r, int p0, int n) {
                const uint32_t last = p0 + n == npg ? nv_last : 0u;
                W.items[slot] = make_uint4((uint32_t)pr, (uint32_t)r, (uint32_t)p0, (uint32_t)n | last << 8);
            };
            const int nb = cnt[0], nt = cnt[1];
            for (int k = 0; k < nb; k++) put(base[0] + v[0] + k, k, k * sp, sp);
            for (int k = 0; k < nt; k++) put(base[1] + v[1] + k, nb + k, nb * sp + k * tp, tp);
            if (rem) put(blen[rem] + srank, nb + nt, nb * sp + nt * tp, rem);
        }
        if (c0 + PLAN_T < npair) advance();   // only a later pass reads the carries
    }
}

// A workgroup is one wave serving every query quad of the KV head: with two
// quads (group of 8) each page is loaded and its codes converted once for
// both, at two waves per SIMD (about 250 VGPRs) instead of three.  FLOOR: the
// load-only copy behind
// kvq_stage1_load_floor -- the same work list, page loads, window chunks and
// partial writes, with each page's words folded into one register instead of
// gqa4_page, at the same register budget (so the same waves per SIMD).
template <int QPK, bool FLOOR>
__device__ __forceinline__ void gqa4_stage1(KParams P, const uint16_t *__restrict__ q,
                                            Workspace W, float qscale) {
    constexpr int NQW = QPK >= 4 ? QPK / 4 : 1;        // query quads of the KV head, all in this wave
    constexpr int NQV = QPK >= 4 ? 4 : QPK;            // queries of a quad that exist
    const int lane = threadIdx.x, g = lane >> 4, r = lane & 15;
    const Geom G = geom(P.scheme, P.nb);
    __shared__ union {
        Gqa4Smem<NQW> pg;
        WinSmem win;
    } U;
    // the paged splits first, in the order of the work list (longest first;
    // workgroups past its end exit), then the window chunks: shorter than the
    // body and tail splits, they fill the compute units as the list drains
    const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int nw = gridDim.y * gridDim.z * W.n_win;
    const int Lw = L - (int)(gridDim.x * gridDim.y * gridDim.z) + nw;
    if (Lw >= 0) {                               // the KV head's fp16 window
        const int wc = Lw % W.n_win, rest = Lw / W.n_win;
        const int hd = rest % (int)gridDim.y, bb = rest / (int)gridDim.y;
        window_partial<QPK, PT / 2, KVQ_SCHEME_KIVI2>(P, q, W, qscale, bb, hd, QPK * hd, wc, lane, U.win);
        return;
    }
    // the item is read together with the list length (the grid's paged part
    // is the list's capacity, so the read is in bounds either way)
    const uint4 item = W.items[L];
    const int n_items = (int)*W.n_items;
    asm volatile("" ::"s"(item.x), "s"(n_items));
    if (L >= n_items) return;
    const int b = (int)item.x / P.Hkv, h = (int)item.x % P.Hkv;
    const int hq0 = h * QPK;                          // the KV head's first query head
    const int s = (int)item.y, p0 = (int)item.z;           // partial row, first page
    const int np = item.w & 255, nv_last = (item.w >> 8) ? (int)(item.w >> 8) : PT;
    Gqa4Smem<NQW> &sm = U.pg;
    // valid tokens of the split's page i (only the prefix's last page is short)
    auto nvalid = [&](int i) { return i == np - 1 ? nv_last : PT; };

    // the split's page ids (one per lane) and the four queries at this lane's
    // score-operand channels 4 (lane & 31) .. +3 (unscaled: keeps q s in the
    // range where the f16 remainder is a normal number)
    int pid_l = (lane < np && p0 + lane < P.max_pages) ? P.table[(size_t)b * P.max_pages + p0 + lane] : 0;
    uint2 qw[NQW][4];                            // queries past the group's end: zero
#pragma unroll
    for (int qd = 0; qd < NQW; qd++)
#pragma unroll
        for (int hq = 0; hq < 4; hq++)
            qw[qd][hq] = hq < NQV ? *(const uint2 *)(q + ((size_t)b * P.Hq + (size_t)hq0 + 4 * qd + hq) * D +
                                                     4 * (lane & 31))
                                  : make_uint2(0u, 0u);

    const bool bad = lane < np && (pid_l < 0 || pid_l >= P.n_pages);
    if (__any(bad)) {
        if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
        pid_l = bad ? 0 : pid_l;                 // read page 0 instead; the result is flagged
    }

    if (lane < 16) sm.Az[lane] = h8v{0, 0, 0, 0, 0, 0, 0, 0};
    // this lane's score-operand rows: row r & 7 of key group 0 (A1) or 1 (A2)
    // where its row r belongs to that group's half, else the zero row
    const h8v *a1[NQW], *a2[NQW];
#pragma unroll
    for (int qd = 0; qd < NQW; qd++) {
        a1[qd] = r < 8 ? &sm.As[qd][0][r][0] : &sm.Az[0];
        a2[qd] = r < 8 ? &sm.Az[0] : &sm.As[qd][1][r - 8][0];
    }

    Gqa4State S[NQW];
#pragma unroll
    for (int qd = 0; qd < NQW; qd++) {
#pragma unroll
        for (int i = 0; i < 4; i++) S[qd].m[i] = -INFINITY;
        S[qd].ma = S[qd].mb = -INFINITY;
        S[qd].la = S[qd].lb = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j++) S[qd].za[j] = S[qd].zb[j] = 0.f;
#pragma unroll
        for (int nt = 0; nt < 8; nt++) S[qd].acc[nt] = f4v{0.f, 0.f, 0.f, 0.f};
    }

    const uint8_t *base = P.pool + (size_t)h * P.page_bytes;
    const size_t pstride = (size_t)P.Hkv * P.page_bytes;
    // two register sets used in turn: the page after the one being processed
    // is in flight.  (A deeper ring costs the registers of a third wave per
    // SIMD, which hides more latency than a second page in flight.)  Loads
    // past the split's end are issued too, with an empty extent.
    uint32_t fold = 0;                           // FLOOR: every loaded word, folded
    auto run_page = [&](const Gqa4Page &R, int i) {
        if constexpr (FLOOR) {
            const uint4 w[6] = {R.ka, R.kb, R.va, R.vb, R.ks, R.vs0};
            const uint4 w2 = R.vs1;
#pragma unroll
            for (int k = 0; k < 6; k++) fold ^= w[k].x ^ w[k].y ^ w[k].z ^ w[k].w;
            fold ^= w2.x ^ w2.y ^ w2.z ^ w2.w;
            (void)i;
        } else {
            gqa4_page(R, S, sm, qw, a1, a2, lane, nvalid(i), qscale);
        }
    };
    auto page_ld = [&](int i) {
        const uint8_t *pg = base + (size_t)__builtin_amdgcn_readlane(pid_l, min(i, np - 1)) * pstride;
        // extent: the whole page, up to the value statistics of its last
        // valid token on the prefix's last page, nothing past the split
        const int ext = i < np ? G.vs + 16 * nvalid(i) : 0;
        return load_gqa4_page(pg, ext, G, lane);
    };
    // (scheduling barriers keep each page's loads together and in order, so
    // the wait before a page counts only the loads of the pages after it)
    Gqa4Page ra = page_ld(0);
    __builtin_amdgcn_sched_barrier(0);
    for (int i = 0; i < np; i += 2) {
        Gqa4Page rb = page_ld(i + 1);
        __builtin_amdgcn_sched_barrier(0);
        run_page(ra, i);
        ra = page_ld(i + 2);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < np) run_page(rb, i + 1);
    }

    if constexpr (FLOOR) {
        // the partial rows' bytes: four output rows and log-sum-exps a split
        if constexpr (NQW == 2)                  // the group kernel's register budget
            asm volatile("" ::: "v255");
        else
            asm volatile("" ::: "v165");
        const float v = __builtin_bit_cast(float, fold & 0x007fffffu);   // finite
#pragma unroll
        for (int qd = 0; qd < NQW; qd++) {
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int e = lane + 64 * k, hp = e >> 5, c4 = e & 31;
                if (hp < NQV)
                    *(float4 *)(W.o + part_row(W, P.Hq, b, hq0 + 4 * qd + hp, s) * D + 4 * c4) =
                        make_float4(v, v, v, v);
            }
            if (lane < NQV) W.ml[part_row(W, P.Hq, b, hq0 + 4 * qd + lane, s)] = make_float2(v, 1.0f);
        }
        return;
    }
    // ---- reduce and write the split's partial ----
    // l and the zero-point sums of query a, a + 1: over the 32 lanes holding
    // them (lane bits 0..3 by DPP within the row, bit 5 by a permute), which
    // then all hold the sums; query i sits in the rows of parity i >> 1, slot
    // i & 1
    const int x32 = (lane ^ 32) << 2;
    auto red = [&](float v) {
        v += dppf<0xB1>(v);                          // quad_perm [1,0,3,2]
        v += dppf<0x4E>(v);                          // quad_perm [2,3,0,1]
        v += dppf<0x124>(v);                         // row_ror:4
        v += dppf<0x128>(v);                         // row_ror:8
        return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x32, __builtin_bit_cast(int, v)));
    };
#pragma unroll
    for (int qd = 0; qd < NQW; qd++) {
        Gqa4State &Sq = S[qd];
        const int hq1 = hq0 + 4 * qd;                // the quad's first query head
        Sq.la = red(Sq.la);
        Sq.lb = red(Sq.lb);
    #pragma unroll
        for (int j = 0; j < 4; j++) {
            Sq.za[j] = red(Sq.za[j]);
            Sq.zb[j] = red(Sq.zb[j]);
        }
        const int hp = r >> 2, part = (r >> 1) & 1, js = r & 1;
        // this lane's query hp: slot hp & 1 of its own row where the row's
        // parity is hp >> 1, else of lane ^ 16 (the same r, the other parity)
        const bool own = (g & 1) == (hp >> 1);
        auto of_hp = [&](float va, float vb) {
            const float t = (hp & 1) ? vb : va;
            const float u = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, t), 0x401F));  // lane ^ 16
            return own ? t : u;
        };
        const float lh = of_hp(Sq.la, Sq.lb);
        const float il = 1.0f / lh;
        const size_t row = part_row(W, P.Hq, b, hq1 + hp, s);
        bool nonfinite = !__builtin_isfinite(lh);
    #pragma unroll
        for (int nt = 0; nt < 8; nt++) {
            f4v lo;                                   // the lo column, two lanes up (lane ^ 2)
    #pragma unroll
            for (int i = 0; i < 4; i++) lo[i] = dppf<0x4E>(Sq.acc[nt][i]);
            const int j = nt >> 1;
            const float zj = of_hp(Sq.za[j], Sq.zb[j]);  // z sum of value group j, query hp
            if (part == 0 && js == (j & 1) && hp < NQV) {
                const f4v o = (Sq.acc[nt] + lo + zj) * il;
    #pragma unroll
                for (int i = 0; i < 4; i++) nonfinite |= !__builtin_isfinite(o[i]);
                *(float4 *)(W.o + row * D + 16 * nt + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
            }
        }
        flag_range(P, nonfinite && hp < NQV, lane);
        // lane i < NQV writes query i's log-sum-exp: its l and m sit in the rows
        // of parity i >> 1, slot i & 1 (as the maxima ma, mb)
        const float lt = (lane & 1) ? Sq.lb : Sq.la, mt = (lane & 1) ? Sq.mb : Sq.ma;
        const float lu = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, lt), 0x401F));
        const float mu = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, mt), 0x401F));
        if (lane < NQV) {
            const float li = (lane & 2) ? lu : lt;
            const float mi = (lane & 2) ? mu : mt;
            const size_t row_i = part_row(W, P.Hq, b, hq1 + lane, s);
            W.ml[row_i] = make_float2(mi + log2f(li), 1.0f);
        }
    }
}

template <int QPK>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(QPK == 8 ? 2 : 3, 8))) void stage1_gqa4_mfma_kernel(KParams P, const uint16_t *__restrict__ q,
                                                              Workspace W, float qscale) {
    gqa4_stage1<QPK, false>(P, q, W, qscale);
}

template <int QPK>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(QPK == 8 ? 2 : 3, 8))) void stage1_gqa4_floor_kernel(KParams P, const uint16_t *__restrict__ q,
                                                               Workspace W, float qscale) {
    gqa4_stage1<QPK, true>(P, q, W, qscale);
}

// ---------------------------------------------------------------------------
// Stage 1, KIVI2 / KITTY / KIVI4, one query head per wave on the matrix cores (any
// group size, MHA included).  The same 16x16x32 f16 products as the group
// kernel, with the one query spread over operand rows and columns instead of
// four queries:
//   scores: A row 0 = hi(q s_c), row 1 = lo(q s_c), rows 2..15 zero; lane
//     (group gi = L >> 5, channels 4 (L & 31) .. +3) forms the four products
//     of its own key statistics, so the operand costs four products a lane.
//   Kitty high plane: the 16 boosted channels' hi/lo operands (gathered from
//     the row-0/1 operand) against the plane's codes, converted with scale 8
//     so that each f16 is 4 * high; one product per 16-token tile, the A
//     fragment keeping the nibble half of that tile and zeroing the other.
//   P.V, transposed: A = value codes (channel rows, token k), B column
//     (part, j) = hi (part 0) or lo (part 1) of p_t s_{t,j}, columns 8..15
//     zero; lane = token forms its four products and stores them token-major
//     in LDS, one 16-byte write a page; the fragments are read back
//     column-major by transposing reads.  Channel tile nt keeps column nt/2
//     (hi) and 4 + nt/2 (lo).
// ---------------------------------------------------------------------------
struct HeadSmem {
    h8v As[2][3][AS_STRIDE];        // score A: [key group][row 0 hi, 1 lo, 2 zero][channel octet]
    uint32_t Bt[PT][BT_DW];         // P.V B: [token][column pair]: dwords 0..3 the hi and lo
                                    // halves of the four groups, 4..7 zero (columns 8..15)
    float zsh[PT];                  // scores, hi + lo rows [token]
    int inv[NB_MAX];                // Kitty: boosted offset -> channel
};

__device__ inline h8v frag8_x4(uint32_t m) {     // codes times 4
    const u4v v = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 8.0f, 0)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 8.0f, 1)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 8.0f, 2)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 8.0f, 3))};
    return __builtin_bit_cast(h8v, v);
}

// eight 4-bit codes of a dword (code k in byte k & 3, nibble k >> 2) -> f16
// fragment in k order: a byte b < 16 is the e4m3 number b / 512
__device__ inline h8v frag8_b4(uint32_t x) {
    const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
    const u4v v = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true))};
    return __builtin_bit_cast(h8v, v);
}

struct HeadPage {
    PageRegs R;
    uint4 k2, k3, v2, v3;           // KIVI4: the second halves of the key and value codes
    uint32_t khw[2];                // Kitty high planes (offsets 0..15, 16..31), dword = lane
    uint32_t kiw[2];                // KITTY_DYN: channel ids of offsets 16q + 4g .. +3
};

template <bool KITTY, bool DYN, bool FOUR>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(FOUR ? 2 : 3, 8)))
void stage1_head_mfma_kernel(KParams P, const uint16_t *__restrict__ q, Workspace W, float qscale) {
    constexpr int SCHEME = FOUR ? KVQ_SCHEME_KIVI4
                                : DYN ? KVQ_SCHEME_KITTY_DYN : KITTY ? KVQ_SCHEME_KITTY : KVQ_SCHEME_KIVI2;
    const S1Item it = s1_item(W.max_splits, W.n_win);
    const int s = it.s, hq = it.hd, b = it.b;
    const int lane = threadIdx.x, g = lane >> 4, r = lane & 15;
    const int h = hq / P.qpk;
    const Geom G = geom(P.scheme, P.nb);
    __shared__ union {
        HeadSmem pg;
        WinSmem win;
    } U;
    if (it.window) {                             // this query head's fp16 window
        window_partial<1, PT / 2, SCHEME>(P, q, W, qscale, b, h, hq, s, lane, U.win);
        return;
    }
    HeadSmem &sm = U.pg;
    const size_t bh = (size_t)b * P.Hkv + h;
    const int p0 = s * P.split_pages;
    const int l = P.state[bh * 4];
    int pid_l = (lane < P.split_pages && p0 + lane < P.max_pages) ? P.table[(size_t)b * P.max_pages + p0 + lane] : 0;
    // this lane's four channels of the score operand: 4 (lane & 31) .. +3
    const uint16_t *qh = q + ((size_t)b * P.Hq + hq) * D;
    const uint2 qraw = *(const uint2 *)(qh + 4 * (lane & 31));

    const int nvq = max(0, l - P.sink - P.R);          // quantized values, counted from the sink
    const int npages = (nvq + PT - 1) / PT;
    const int p1 = min(p0 + P.split_pages, npages);
    if (p0 >= p1) return;
    const int np = p1 - p0;                      // <= split_pages <= 64

    const bool bad = lane < np && (pid_l < 0 || pid_l >= P.n_pages);
    if (__any(bad)) {
        if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
        pid_l = bad ? 0 : pid_l;                 // read page 0 instead; the result is flagged
    }

    if (lane < 16) {
        sm.As[0][2][lane] = h8v{0, 0, 0, 0, 0, 0, 0, 0};
        sm.As[1][2][lane] = h8v{0, 0, 0, 0, 0, 0, 0, 0};
    }
    *(uint4 *)&sm.Bt[lane][4] = make_uint4(0u, 0u, 0u, 0u);     // columns 8..15 stay zero
    int kc_off[8] = {0, 0, 0, 0, 0, 0, 0, 0};    // Kitty: channels of offsets 16q + 4g + i
    const int planes = P.nb >> 4;                // Kitty high planes: 1 (16 boosted) or 2 (32)
    if (KITTY && !DYN) {
        if (lane < NB_MAX) sm.inv[lane] = 0;
        lds_sync();
        for (int c = lane; c < D; c += 64) {
            const int o = P.boost_idx[(size_t)h * D + c];
            if (o < P.nb) sm.inv[o] = c;
        }
        lds_sync();
#pragma unroll
        for (int i = 0; i < 8; i++) kc_off[i] = sm.inv[16 * (i >> 2) + 4 * g + (i & 3)];
    }

    // operand roles
    const int gi_p = lane >> 5;                  // key group of this lane's products
    const int arow = r < 2 ? r : 2;              // score A row read by this lane
    // P.V B fragment of this lane (column r, tokens 32 ks + 8 g .. + 7): lane
    // r of its 16-lane group addresses token row 32 ks + 8 g + (r >> 2) (+ 4),
    // columns 4 (r & 3) .. + 3, and the transposing read hands it column r
    const uint32_t *bsrc = &sm.Bt[8 * g + (r >> 2)][2 * (r & 3)];

    float m = -INFINITY, lsum = 0.f;             // lsum: this lane's tokens
    float zacc[4] = {0.f, 0.f, 0.f, 0.f};        // sum_t p_t z_{t,j}, this lane's tokens
    f4v acc[8];
#pragma unroll
    for (int nt = 0; nt < 8; nt++) acc[nt] = f4v{0.f, 0.f, 0.f, 0.f};
    const uint32_t MSK = 0x33333333u;

    auto run_page = [&](const HeadPage &HP, int nvalid) {
        const PageRegs &R = HP.R;
        lds_sync();                              // previous page done with the LDS
        // ---- score operand: four products of this lane, hi and lo ----
        float bias;
        {
            // the channel pairs' scales and zero points, packed
            const uint32_t s01 = __builtin_amdgcn_perm(R.ks.y, R.ks.x, 0x05040100u);
            const uint32_t s23 = __builtin_amdgcn_perm(R.ks.w, R.ks.z, 0x05040100u);
            const uint32_t z01 = __builtin_amdgcn_perm(R.ks.y, R.ks.x, 0x07060302u);
            const uint32_t z23 = __builtin_amdgcn_perm(R.ks.w, R.ks.z, 0x07060302u);
            uint32_t hv[2], lv[2];
            split_qs_pk(qraw.x, s01, hv[0], lv[0]);
            split_qs_pk(qraw.y, s23, hv[1], lv[1]);
            bias = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qraw.y), __builtin_bit_cast(h2v, z23),
                                          __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qraw.x),
                                                                 __builtin_bit_cast(h2v, z01), 0.0f, false),
                                          false);
            ((uint2 *)&sm.As[gi_p][0][0])[lane & 31] = make_uint2(hv[0], hv[1]);
            ((uint2 *)&sm.As[gi_p][1][0])[lane & 31] = make_uint2(lv[0], lv[1]);
        }
        bias = row_sum16(bias);                  // lanes 15, 31, 47, 63
        const float bias0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bias), 15)) +
                            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bias), 31));
        const float bias1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bias), 47)) +
                            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bias), 63));
        lds_sync();

        // ---- scores on the matrix cores ----
        // KIVI2: dword 2n + (kc >> 1) of token tile n holds kc's codes at
        // bit pair kc & 1 of each nibble; KIVI4: dword 4n + kc
        const uint32_t kd[16] = {R.ka.x, R.ka.y, R.ka.z, R.ka.w, R.kb.x, R.kb.y, R.kb.z, R.kb.w,
                                 HP.k2.x, HP.k2.y, HP.k2.z, HP.k2.w, HP.k3.x, HP.k3.y, HP.k3.z, HP.k3.w};
        f4v sc[4];
#pragma unroll
        for (int n = 0; n < 4; n++) sc[n] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; kc++) {
            h8v af[2], bf[4];
#pragma unroll
            for (int gi = 0; gi < 2; gi++) af[gi] = sm.As[gi][arow][4 * kc + g];
#pragma unroll
            for (int n = 0; n < 4; n++) {
                if (FOUR) {
                    bf[n] = frag8_b4(kd[4 * n + kc]);
                } else {
                    const uint32_t x = kd[2 * n + (kc >> 1)];
                    bf[n] = frag8((kc & 1) ? ((x >> 2) & MSK) : (x & MSK));
                }
            }
#pragma unroll
            for (int n = 0; n < 4; n++)
                sc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[n >> 1], bf[n], sc[n], 0, 0, 0);
        }
        if (KITTY) {
#pragma unroll
            for (int qp = 0; qp < 2; qp++) {
                if (qp < planes) {               // uniform
                    int co[4];                   // channels of offsets 16 qp + 4g + i
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        co[i] = DYN ? (HP.kiw[qp] >> (8 * i)) & (D - 1) : kc_off[4 * qp + i];
                    // tile n: key group n >> 1, plane half n >> 1 (bit 2), nibble half n & 1
                    const h8v bk0 = frag8_x4(HP.khw[qp] & MSK), bk1 = frag8_x4((HP.khw[qp] >> 2) & MSK);
#pragma unroll
                    for (int gi = 0; gi < 2; gi++) {
                        const _Float16 *row = (const _Float16 *)&sm.As[gi][arow][0];
                        const _Float16 a0 = row[co[0]], a1 = row[co[1]], a2 = row[co[2]], a3 = row[co[3]];
                        const _Float16 z = 0;
                        const h8v alo = h8v{a0, a1, a2, a3, z, z, z, z};
                        const h8v ahi = h8v{z, z, z, z, a0, a1, a2, a3};
                        const h8v bk = gi ? bk1 : bk0;
                        sc[2 * gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bk, sc[2 * gi], 0, 0, 0);
                        sc[2 * gi + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bk, sc[2 * gi + 1], 0, 0, 0);
                    }
                }
            }
        }
        if (lane < 16) {                         // rows 0 (hi) and 1 (lo) of each token tile
#pragma unroll
            for (int n = 0; n < 4; n++) sm.zsh[16 * n + r] = sc[n][0] + sc[n][1];
        }
        lds_sync();

        // ---- online softmax, lane = token ----
        float zt = sm.zsh[lane] * qscale + (lane < 32 ? bias0 : bias1) * qscale;     // log2 units
        if (lane >= nvalid) zt = -INFINITY;
        if (__any(zt > m + LAZY_TAU)) {
            float mt = zt;
#pragma unroll
            for (int msk = 1; msk < 64; msk <<= 1) mt = fmaxf(mt, shfl_xor(mt, msk));
            const float mn = fmaxf(m, mt);
            const float alpha = __builtin_amdgcn_exp2f(m - mn);
            m = mn;
            lsum *= alpha;
#pragma unroll
            for (int j = 0; j < 4; j++) zacc[j] *= alpha;
#pragma unroll
            for (int nt = 0; nt < 8; nt++) acc[nt] *= alpha;
        }
        const float pt = __builtin_amdgcn_exp2f(zt - m);                 // 0 past nvalid
        lsum += pt;

        // ---- P.V operand: p_t s_{t,j}, hi and lo, lane = token ----
        {
            // statistics past nvalid are not written yet: use zero
            const uint32_t keep = lane < nvalid ? 0xffffffffu : 0u;
            const uint32_t vw[4] = {R.vs.x & keep, R.vs.y & keep, R.vs.z & keep, R.vs.w & keep};
#pragma unroll
            for (int j = 0; j < 4; j++) zacc[j] = fmaf(pt, (float)hi16h(vw[j]), zacc[j]);
            uint32_t hv[2], lv[2];
            mul_split2(pt, lo16h(vw[0]), pt, lo16h(vw[1]), hv[0], lv[0]);
            mul_split2(pt, lo16h(vw[2]), pt, lo16h(vw[3]), hv[1], lv[1]);
            // columns 0..3: hi of groups 0..3, 4..7: lo
            *(uint4 *)&sm.Bt[lane][0] = make_uint4(hv[0], hv[1], lv[0], lv[1]);
        }
        lds_sync();

        // ---- P.V on the matrix cores ----
        // KIVI2: dword nt holds both 32-token steps (bit pair ks of each
        // nibble); KIVI4: dword 8 ks + nt
        const uint32_t vd[16] = {R.va.x, R.va.y, R.va.z, R.va.w, R.vb.x, R.vb.y, R.vb.z, R.vb.w,
                                 HP.v2.x, HP.v2.y, HP.v2.z, HP.v2.w, HP.v3.x, HP.v3.y, HP.v3.z, HP.v3.w};
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            const uint32_t *rp = bsrc + 32 * ks * BT_DW;
            const h4v b0 = lds_tr16(rp), b1 = lds_tr16(rp + 4 * BT_DW);
            const h8v bfr = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int nt = 0; nt < 8; nt++) {
                const uint32_t x = vd[nt];
                const h8v afr = FOUR ? frag8_b4(vd[8 * ks + nt]) : frag8(ks ? ((x >> 2) & MSK) : (x & MSK));
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, acc[nt], 0, 0, 0);
            }
        }
    };

    const uint8_t *base = P.pool + (size_t)h * P.page_bytes;
    const size_t pstride = (size_t)P.Hkv * P.page_bytes;
    auto page_ld = [&](int i) {
        const uint8_t *pg = base + (size_t)__builtin_amdgcn_readlane(pid_l, min(i, np - 1)) * pstride;
        HeadPage HP;
        HP.R = load_page_masked(pg, i < np, G, lane);
        if (FOUR) {
            const __amdgpu_buffer_rsrc_t rs = page_rsrc(pg, i < np, G);
            HP.k2 = bload(rs, G.kc + 2048 + 16 * lane);
            HP.k3 = bload(rs, G.kc + 3072 + 16 * lane);
            HP.v2 = bload(rs, G.vc + 2048 + 16 * lane);
            HP.v3 = bload(rs, G.vc + 3072 + 16 * lane);
        } else {
            HP.k2 = HP.k3 = HP.v2 = HP.v3 = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int qp = 0; qp < 2; qp++) {
            const bool on = qp < planes;
            HP.khw[qp] = KITTY && on ? bload1(page_rsrc(pg, i < np, G), G.kh + 256 * qp + 4 * lane) : 0u;
            HP.kiw[qp] = DYN && on ? bload1(page_rsrc(pg, i < np, G), G.ki + 16 * qp + 4 * g) : 0u;
        }
        return HP;
    };
    // two register sets used in turn (the page after the one being processed
    // is in flight); loads past the split's end are issued with an empty extent
    HeadPage ra = page_ld(0);
    __builtin_amdgcn_sched_barrier(0);
    for (int i = 0; i < np; i += 2) {
        HeadPage rb = page_ld(i + 1);
        __builtin_amdgcn_sched_barrier(0);
        run_page(ra, min(PT, nvq - (p0 + i) * PT));
        ra = page_ld(i + 2);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < np) run_page(rb, min(PT, nvq - (p0 + i + 1) * PT));
    }

    // ---- reduce and write the split's partial ----
    // sums over the wave: DPP within each row, then lane ^ 16 (swizzle) and
    // lane ^ 32 (permute)
    const int x32 = (lane ^ 32) << 2;
    auto wave_sum = [&](float v) {
        v += dppf<0xB1>(v);                          // quad_perm [1,0,3,2]
        v += dppf<0x4E>(v);                          // quad_perm [2,3,0,1]
        v += dppf<0x124>(v);                         // row_ror:4
        v += dppf<0x128>(v);                         // row_ror:8
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
        return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x32, __builtin_bit_cast(int, v)));
    };
    lsum = wave_sum(lsum);
#pragma unroll
    for (int j = 0; j < 4; j++) zacc[j] = wave_sum(zacc[j]);
    const float il = 1.0f / lsum;
    const size_t row = part_row(W, P.Hq, b, hq, s);
    bool nonfinite = !__builtin_isfinite(lsum);
#pragma unroll
    for (int nt = 0; nt < 8; nt++) {
        f4v lo;                                   // column 4 + j, four lanes up (row_shl:4)
#pragma unroll
        for (int i = 0; i < 4; i++) lo[i] = dppf<0x104>(acc[nt][i]);
        const int jv = nt >> 1;
        if (r == jv) {
            const float zj = jv == 0 ? zacc[0] : jv == 1 ? zacc[1] : jv == 2 ? zacc[2] : zacc[3];
            const f4v o = (acc[nt] + lo + zj) * il;
#pragma unroll
            for (int i = 0; i < 4; i++) nonfinite |= !__builtin_isfinite(o[i]);
            *(float4 *)(W.o + row * D + 16 * nt + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
        }
    }
    flag_range(P, nonfinite, lane);
    if (lane == 0) W.ml[row] = make_float2(m + log2f(lsum), 1.0f);
}

// ---------------------------------------------------------------------------
// Stage 1, WITCERT: INT8 codes with the Philox dither regenerated in the
// kernel, and the certificate accumulated next to the output.  One wave per
// (split, KV head, request) serves all QPK query heads of the KV head, so each
// dither draw is shared by the group.  Lane L: channel quad cq = L & 31 (one
// Philox4x32-10 block gives the four dither words of channels 4cq..4cq+3)
// and token phase tp = L >> 5.
// ---------------------------------------------------------------------------
// Sum over the 32 lanes of each half-wave, in every lane: a DPP butterfly
// within each 16-lane row (pair swaps, quad swaps, half-row and row mirrors)
// and one swizzle that swaps the two rows of a half.
template <int CTRL>
__device__ inline float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, x), CTRL, 0xf, 0xf, false));
}
__device__ inline float half_sum32(float v) {
    v += dpp_f<0xB1>(v);                // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);                // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x141>(v);               // row_half_mirror
    v += dpp_f<0x140>(v);               // row_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));  // lane ^ 16
    return v;
}

template <int QPK>
__global__ __launch_bounds__(64) void stage1_witcert_kernel(KParams P, const uint16_t *__restrict__ q,
                                                            Workspace W, float qscale, float sm_scale,
                                                            float kappa) {
    const S1Item it = s1_item(W.max_splits, W.n_win);
    const int s = it.s, h = it.hd, b = it.b;
    const int lane = threadIdx.x, cq = lane & 31, tp = lane >> 5;
    const Geom G = geom(P.scheme, P.nb);
    if (it.window) {                             // the KV head's active block (fp16 tail)
        __shared__ WinSmem win;
        window_partial<QPK, 16, KVQ_SCHEME_WITCERT>(P, q, W, qscale, b, h, QPK * h, s, lane, win);
        return;
    }
    const size_t bh = (size_t)b * P.Hkv + h;
    const int nq = P.state[bh * 4 + 1];
    const int npages = nq / WPT;
    const int p0 = s * P.split_pages;
    const int p1 = min(p0 + P.split_pages, npages);
    if (p0 >= p1) return;

    float qv[QPK][4];
#pragma unroll
    for (int hh = 0; hh < QPK; hh++) {
        const uint2 raw = *(const uint2 *)(q + ((size_t)b * P.Hq + h * QPK + hh) * D + 4 * cq);
        qv[hh][0] = h2f((uint16_t)(raw.x & 0xffff));
        qv[hh][1] = h2f((uint16_t)(raw.x >> 16));
        qv[hh][2] = h2f((uint16_t)(raw.y & 0xffff));
        qv[hh][3] = h2f((uint16_t)(raw.y >> 16));
    }
    float m[QPK], lp[QPK], ap[QPK], o[QPK][4];
#pragma unroll
    for (int hh = 0; hh < QPK; hh++) {
        m[hh] = -INFINITY; lp[hh] = 0.f; ap[hh] = 0.f;
        o[hh][0] = o[hh][1] = o[hh][2] = o[hh][3] = 0.f;
    }
    const uint32_t k0 = (uint32_t)P.seed;
    const uint32_t k1 = (uint32_t)(P.seed >> 32);
    const uint32_t c2 = (P.layer << 16) | (uint32_t)h;
    const float LOG2E = 1.4426950408889634f;

    for (int p = p0; p < p1; p++) {
        const int pid = P.table[(size_t)b * P.max_pages + p];
        if (pid < 0 || pid >= P.n_pages) {
            if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
            continue;
        }
        const uint8_t *page = cpage(P, pid, h);
        const int8_t *kcod = (const int8_t *)(page + G.kc);
        const int8_t *vcod = (const int8_t *)(page + G.vc);
        const uint2 ksr = *(const uint2 *)(page + G.ks + 8 * cq);
        const uint2 vsr = *(const uint2 *)(page + G.vs + 8 * cq);
        const float ks[4] = {h2f((uint16_t)(ksr.x & 0xffff)), h2f((uint16_t)(ksr.x >> 16)),
                             h2f((uint16_t)(ksr.y & 0xffff)), h2f((uint16_t)(ksr.y >> 16))};
        const float vs[4] = {h2f((uint16_t)(vsr.x & 0xffff)), h2f((uint16_t)(vsr.x >> 16)),
                             h2f((uint16_t)(vsr.y & 0xffff)), h2f((uint16_t)(vsr.y >> 16))};
        // certificate: varsigma^2 = (sm^2/12) sum_c q_c^2 s_c^2 for this block,
        // u = kappa sqrt(varsigma^2); e^u folded into the A accumulator
        float eu[QPK];
#pragma unroll
        for (int hh = 0; hh < QPK; hh++) {
            float v2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; e++) v2 = fmaf(qv[hh][e] * qv[hh][e], ks[e] * ks[e], v2);
#pragma unroll
            for (int msk = 1; msk < 32; msk <<= 1) v2 += shfl_xor(v2, msk);
            v2 *= sm_scale * sm_scale * (1.0f / 12.0f);
            eu[hh] = exp2f(kappa * sqrtf(v2) * LOG2E);
        }
        for (int i = 0; i < WPT / 2; i++) {
            const int t = 2 * i + tp;
            const uint32_t tok = (uint32_t)(p * WPT + t);
            const U4 uk = philox4x32_10(U4{tok, (uint32_t)cq, c2, (uint32_t)b}, k0, k1);
            const U4 uv = philox4x32_10(U4{tok, (uint32_t)cq, c2, (uint32_t)b}, k0, k1 ^ 1u);
            const uint32_t kw = *(const uint32_t *)(kcod + (size_t)t * D + 4 * cq);
            const uint32_t vw = *(const uint32_t *)(vcod + (size_t)t * D + 4 * cq);
            const uint32_t ukw[4] = {uk.x, uk.y, uk.z, uk.w};
            const uint32_t uvw[4] = {uv.x, uv.y, uv.z, uv.w};
            // x = s (code - xi), with code - xi = (code + 1/2) - (u >> 8) 2^-24
            // rounded once, as a subtraction of xi would round it
            float kx[4], vx[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float kcode = (float)(int8_t)((kw >> (8 * e)) & 0xff);
                const float vcode = (float)(int8_t)((vw >> (8 * e)) & 0xff);
                kx[e] = ks[e] * __builtin_fmaf((float)(ukw[e] >> 8), -0x1p-24f, kcode + 0.5f);
                vx[e] = vs[e] * __builtin_fmaf((float)(uvw[e] >> 8), -0x1p-24f, vcode + 0.5f);
            }
#pragma unroll
            for (int hh = 0; hh < QPK; hh++) {
                float part = 0.f;
#pragma unroll
                for (int e = 0; e < 4; e++) part = fmaf(qv[hh][e], kx[e], part);
                const float z2 = half_sum32(part) * qscale;
                // per token phase: each half-wave sees its own token stream.
                // Lazy rescaling: the running maximum moves only when a score
                // exceeds it by 8 (log2 units), so p <= 256 and the rescale is rare
                if (__any(z2 > m[hh] + LAZY_TAU)) {
                    const float mnew = fmaxf(m[hh], z2);
                    const float alpha = __builtin_amdgcn_exp2f(m[hh] - mnew);
                    m[hh] = mnew;
                    lp[hh] *= alpha;
                    ap[hh] *= alpha;
#pragma unroll
                    for (int e = 0; e < 4; e++) o[hh][e] *= alpha;
                }
                const float pr = __builtin_amdgcn_exp2f(z2 - m[hh]);
                lp[hh] += pr;
                ap[hh] = fmaf(pr, eu[hh], ap[hh]);
#pragma unroll
                for (int e = 0; e < 4; e++) o[hh][e] = fmaf(pr, vx[e], o[hh][e]);
            }
        }
    }
    // combine the two token phases (lanes L and L ^ 32)
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
    (void)zero4;
#pragma unroll
    for (int hh = 0; hh < QPK; hh++) {
        const float mo = shfl_xor(m[hh], 32);
        const float mt = fmaxf(m[hh], mo);
        const float sa = exp2f(m[hh] - mt);
        const float lo = shfl_xor(lp[hh] * sa, 32);
        const float ao = shfl_xor(ap[hh] * sa, 32);
        const float lt = lp[hh] * sa + lo;
        const float at = ap[hh] * sa + ao;
        float oo[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float mine = o[hh][e] * sa;
            oo[e] = mine + shfl_xor(mine, 32);
        }
        const size_t row = part_row(W, P.Hq, b, h * QPK + hh, s);
        if (tp == 0) {
            const float il = 1.0f / lt;
            *(float4 *)(W.o + row * D + 4 * cq) = make_float4(oo[0] * il, oo[1] * il, oo[2] * il, oo[3] * il);
        }
        if (lane == 0) W.ml[row] = make_float2(mt + log2f(lt), at / lt);
    }
}

// ---------------------------------------------------------------------------
// Stage 1, WITCERT_PAGED: every token of the split is quantized (no fp16
// tail); one wave per (split, KV head, request) serves the QPK query heads,
// lane = (channel quad cq, token phase tp) as in the block kernel, with the
// dither counter keyed by the token's slot (page_id * 64 + position) and one
// scale per (token, 32-channel group).  Per page, lane t first stages token
// t's key and value scales in LDS and computes e^{u_t} for the QPK queries:
// u_t = kappa sqrt((sm^2/12) sum_g s_{t,g}^2 Q_g) with Q_g the query's sum of
// q_c^2 over the group's quantized channels (a bypassed channel carries no
// error).  Bypassed key channels: their q is zeroed in the lane's operand and
// lane cq < 2 nb adds q_c x_c for the bypass row's entry cq instead.
// ---------------------------------------------------------------------------
struct WtokSmem {
    float ks[4][PT], vs[4][PT];
    float eu[PT][8];                // e^{u_t} per token and query head
    float kb[8][PT];                // bypass row entries [entry][token]
    int inv[8];                     // bypass row entry -> channel
};

template <int QPK>
__global__ __launch_bounds__(64) void stage1_witcert_paged_kernel(KParams P, const uint16_t *__restrict__ q,
                                                                  Workspace W, float qscale, float sm_scale,
                                                                  float kappa) {
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, cq = lane & 31, tp = lane >> 5;
    const Geom G = geom(P.scheme, P.nb);
    const size_t bh = (size_t)b * P.Hkv + h;
    const int l = P.state[bh * 4];
    const int npages = (l + PT - 1) / PT;
    const int p0 = s * P.split_pages;
    const int p1 = min(p0 + P.split_pages, npages);
    if (p0 >= p1) return;
    __shared__ WtokSmem sm;
    const int nbyp = 2 * P.nb;                   // bypassed key channels

    // bypass flags of this lane's channels and the channel of row entry cq
    bool byp[4] = {false, false, false, false};
    if (nbyp > 0) {
        const uint32_t ow = *(const uint32_t *)(P.boost_idx + (size_t)h * D + 4 * cq);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int o = (int)((ow >> (8 * e)) & 0xffu);
            byp[e] = o < nbyp;
            if (byp[e] && tp == 0) sm.inv[o] = 4 * cq + e;
        }
    }
    lds_sync();
    const bool bslot = cq < nbyp;                // this lane adds bypass entry cq
    const int bch = bslot ? sm.inv[cq] : 0;

    float qv[QPK][4], qb[QPK], Qg[QPK][4];
#pragma unroll
    for (int hh = 0; hh < QPK; hh++) {
        const uint16_t *qh = q + ((size_t)b * P.Hq + h * QPK + hh) * D;
        const uint2 raw = *(const uint2 *)(qh + 4 * cq);
        const float qq[4] = {h2f((uint16_t)(raw.x & 0xffff)), h2f((uint16_t)(raw.x >> 16)),
                             h2f((uint16_t)(raw.y & 0xffff)), h2f((uint16_t)(raw.y >> 16))};
        float q2 = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            qv[hh][e] = byp[e] ? 0.f : qq[e];
            q2 = fmaf(qv[hh][e], qv[hh][e], q2);
        }
        qb[hh] = bslot ? h2f(qh[bch]) : 0.f;
        // Q_g: the 8 lanes of group g = cq >> 3 hold its channels
#pragma unroll
        for (int msk = 1; msk < 8; msk <<= 1) q2 += shfl_xor(q2, msk);
#pragma unroll
        for (int g = 0; g < 4; g++)
            Qg[hh][g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q2), 8 * g));
    }
    float m[QPK], lp[QPK], ap[QPK], o[QPK][4];
#pragma unroll
    for (int hh = 0; hh < QPK; hh++) {
        m[hh] = -INFINITY; lp[hh] = 0.f; ap[hh] = 0.f;
        o[hh][0] = o[hh][1] = o[hh][2] = o[hh][3] = 0.f;
    }
    const uint32_t k0 = (uint32_t)P.seed;
    const uint32_t k1 = (uint32_t)(P.seed >> 32);
    const uint32_t c2 = (P.layer << 16) | (uint32_t)h;
    const float LOG2E = 1.4426950408889634f;
    const float cc = sm_scale * sm_scale * (1.0f / 12.0f);
    const int gq = cq >> 3;                      // this lane's scale group

    // the split's page ids, one per lane (at most 64 pages)
    const int np = p1 - p0;
    int pid_l = (lane < np && p0 + lane < P.max_pages) ? P.table[(size_t)b * P.max_pages + p0 + lane] : 0;
    {
        const bool bad = lane < np && (pid_l < 0 || pid_l >= P.n_pages);
        if (__any(bad)) {
            if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
            pid_l = bad ? 0 : pid_l;              // read page 0 instead; the result is flagged
        }
    }
    // per-page rows of lane = token: key scales, value scales, bypass row;
    // the next page's rows are loaded while the current page is processed
    struct Rows { uint2 ks, vs; uint4 br; };
    auto rows = [&](int i) {
        Rows r;
        const uint8_t *pg = cpage(P, __builtin_amdgcn_readlane(pid_l, i), h);
        const bool ok = lane < min(PT, l - (p0 + i) * PT);
        r.ks = ok ? *(const uint2 *)(pg + G.ks + 8 * lane) : make_uint2(0u, 0u);
        r.vs = ok ? *(const uint2 *)(pg + G.vs + 8 * lane) : make_uint2(0u, 0u);
        r.br = (ok && nbyp > 0) ? *(const uint4 *)(pg + G.kh + 16 * lane) : make_uint4(0u, 0u, 0u, 0u);
        return r;
    };
    Rows cur = rows(0);
    for (int pi = 0; pi < np; pi++) {
        const int p = p0 + pi;
        const int pid = __builtin_amdgcn_readlane(pid_l, pi);
        const uint8_t *page = cpage(P, pid, h);
        const int nvalid = min(PT, l - p * PT);
        lds_sync();                               // the previous page's LDS reads are done
        {
            // lane = token: scales and e^{u_t}
            const uint2 ksr = cur.ks, vsr = cur.vs;
            const float sg[4] = {h2f((uint16_t)(ksr.x & 0xffff)), h2f((uint16_t)(ksr.x >> 16)),
                                 h2f((uint16_t)(ksr.y & 0xffff)), h2f((uint16_t)(ksr.y >> 16))};
            const float sv[4] = {h2f((uint16_t)(vsr.x & 0xffff)), h2f((uint16_t)(vsr.x >> 16)),
                                 h2f((uint16_t)(vsr.y & 0xffff)), h2f((uint16_t)(vsr.y >> 16))};
#pragma unroll
            for (int g = 0; g < 4; g++) { sm.ks[g][lane] = sg[g]; sm.vs[g][lane] = sv[g]; }
            if (nbyp > 0) {
                const uint32_t bw[4] = {cur.br.x, cur.br.y, cur.br.z, cur.br.w};
#pragma unroll
                for (int e = 0; e < 8; e++)
                    sm.kb[e][lane] = e < nbyp ? h2f((uint16_t)((bw[e >> 1] >> (16 * (e & 1))) & 0xffffu)) : 0.f;
            }
#pragma unroll
            for (int hh = 0; hh < QPK; hh++) {
                float v2 = 0.f;
#pragma unroll
                for (int g = 0; g < 4; g++) v2 = fmaf(sg[g] * sg[g], Qg[hh][g], v2);
                sm.eu[lane][hh] = exp2f(kappa * sqrtf(v2 * cc) * LOG2E);
            }
        }
        if (pi + 1 < np) cur = rows(pi + 1);
        lds_sync();
        const int8_t *kcod = (const int8_t *)(page + G.kc);
        const int8_t *vcod = (const int8_t *)(page + G.vc);
        const uint32_t slot_lo0 = (uint32_t)pid * (uint32_t)PT;
        const uint32_t slot_hi = (uint32_t)((uint64_t)pid * PT >> 32);
        auto token = [&](auto chk, int t, uint32_t kw, uint32_t vw) {
            constexpr bool CHK = decltype(chk)::value;
            const bool valid = !CHK || t < nvalid;
            const uint32_t slot = slot_lo0 + (uint32_t)t;
            const U4 uk = philox4x32_10(U4{slot, (uint32_t)cq, c2, slot_hi}, k0, k1);
            const U4 uv = philox4x32_10(U4{slot, (uint32_t)cq, c2, slot_hi}, k0, k1 ^ 1u);
            const float kbv = nbyp > 0 ? sm.kb[cq & 7][t] : 0.f;     // 0 past the page's tokens
            const float ks = sm.ks[gq][t], vs = sm.vs[gq][t];
            const uint32_t ukw[4] = {uk.x, uk.y, uk.z, uk.w};
            const uint32_t uvw[4] = {uv.x, uv.y, uv.z, uv.w};
            float kx[4], vx[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float kcode = (float)(int8_t)((kw >> (8 * e)) & 0xff);
                const float vcode = (float)(int8_t)((vw >> (8 * e)) & 0xff);
                kx[e] = ks * __builtin_fmaf((float)(ukw[e] >> 8), -0x1p-24f, kcode + 0.5f);
                vx[e] = vs * __builtin_fmaf((float)(uvw[e] >> 8), -0x1p-24f, vcode + 0.5f);
            }
            float eut[QPK];
#pragma unroll
            for (int hh = 0; hh < QPK; hh++) eut[hh] = sm.eu[t][hh];
#pragma unroll
            for (int hh = 0; hh < QPK; hh++) {
                float part = qb[hh] * kbv;
#pragma unroll
                for (int e = 0; e < 4; e++) part = fmaf(qv[hh][e], kx[e], part);
                float z2 = half_sum32(part) * qscale;
                if (CHK && !valid) z2 = -INFINITY;
                if (__any(z2 > m[hh] + LAZY_TAU)) {
                    const float mnew = fmaxf(m[hh], z2);
                    // a half-wave with no valid token yet keeps m = -inf
                    const float alpha = mnew == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m[hh] - mnew);
                    m[hh] = mnew;
                    lp[hh] *= alpha;
                    ap[hh] *= alpha;
#pragma unroll
                    for (int e = 0; e < 4; e++) o[hh][e] *= alpha;
                }
                const float pr = valid ? __builtin_amdgcn_exp2f(z2 - m[hh]) : 0.f;
                lp[hh] += pr;
                ap[hh] = fmaf(pr, eut[hh], ap[hh]);
#pragma unroll
                for (int e = 0; e < 4; e++) o[hh][e] = fmaf(pr, vx[e], o[hh][e]);
            }
        };
        // every pair of tokens is whole except, for an odd count, the last
        // codes of the next token in flight while one is processed; a token
        // past the page's count has zero scales, so its codes read as 0
        const uint32_t *kq = (const uint32_t *)(kcod + 4 * cq), *vq = (const uint32_t *)(vcod + 4 * cq);
        uint32_t kwn = kq[tp * (D / 4)], vwn = vq[tp * (D / 4)];
#pragma unroll 1
        for (int i = 0; i < (nvalid >> 1); i++) {
            const uint32_t kw = kwn, vw = vwn;
            const int tn = min(2 * i + 2 + tp, PT - 1);
            kwn = kq[tn * (D / 4)];
            vwn = vq[tn * (D / 4)];
            token(std::false_type{}, 2 * i + tp, kw, vw);
        }
        if (nvalid & 1) token(std::true_type{}, (nvalid & ~1) + tp, kwn, vwn);
    }
    // combine the two token phases (lanes L and L ^ 32); the phase-0 half
    // always holds the split's first token
#pragma unroll
    for (int hh = 0; hh < QPK; hh++) {
        const float mo = shfl_xor(m[hh], 32);
        const float mt = fmaxf(m[hh], mo);
        const float sa = m[hh] == -INFINITY ? 0.f : exp2f(m[hh] - mt);
        const float lo = shfl_xor(lp[hh] * sa, 32);
        const float ao = shfl_xor(ap[hh] * sa, 32);
        const float lt = lp[hh] * sa + lo;
        const float at = ap[hh] * sa + ao;
        float oo[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float mine = o[hh][e] * sa;
            oo[e] = mine + shfl_xor(mine, 32);
        }
        const size_t row = part_row(W, P.Hq, b, h * QPK + hh, s);
        if (tp == 0) {
            const float il = 1.0f / lt;
            *(float4 *)(W.o + row * D + 4 * cq) = make_float4(oo[0] * il, oo[1] * il, oo[2] * il, oo[3] * il);
        }
        if (lane == 0) W.ml[row] = make_float2(mt + log2f(lt), at / lt);
    }
}



// ---------------------------------------------------------------------------
// Stage 2: log-sum-exp merge of one query head's partials (the paged splits
// and the fp16 window): weights w_s = 2^(lse_s - max), o = sum w_s o_s /
// sum w_s, and for WITCERT the certificate A = sum w_s A_s / sum w_s (the
// per-split form of A is exact under this merge; "WitCert" Key structure).
// One wave per (query head, request).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void merge_kernel(KParams P, float *__restrict__ out,
                                                   float *__restrict__ cert, Workspace W) {
    const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const bool wit = P.scheme == KVQ_SCHEME_WITCERT;
    const int h = hq / P.qpk;
    const size_t bh = (size_t)b * P.Hkv + h;
    const int l = P.state[bh * 4], nkq = P.state[bh * 4 + 1];
    const int npages = wit ? nkq / WPT
                       : P.scheme == KVQ_SCHEME_WITCERT_PAGED ? (l + PT - 1) / PT
                                                             : (max(0, l - P.sink - P.R) + PT - 1) / PT;
    const int nsplit = min(gqa4_path(P.scheme, P.qpk, P.force_generic)
                               ? gqa_splits(npages, P.split_pages)
                               : (npages + P.split_pages - 1) / P.split_pages,
                           W.max_splits);
    const int ne = nsplit + W.n_win;              // entries nsplit.. are the window chunks
    const size_t row0 = part_row(W, P.Hq, b, hq, 0);
    auto row_of = [&](int e) { return row0 + (size_t)(e < nsplit ? e : W.max_splits + e - nsplit); };

    // output rows: lane = (entry parity ph, channel quad c4); the first 32
    // entries' loads go out with the log-sum-exp reads
    constexpr int BATCH = 24;                // 48 entries per batch: one for caches up to ~540 pages
    const int ph = lane >> 5, c4 = lane & 31;
    float4 ov[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; k++) {
        const int e = ph + 2 * k;
        ov[k] = e < ne ? *(const float4 *)(W.o + row_of(e) * D + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // a weight per entry: at most MAX_SPLITS paged splits plus MAX_WIN window
    // chunks (kvq_set_layout keeps both bounds)
    __shared__ float wsh[MAX_SPLITS + MAX_WIN];
    float M = -INFINITY;
    for (int e = lane; e < ne; e += 64) M = fmaxf(M, W.ml[row_of(e)].x);
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) M = fmaxf(M, shfl_xor(M, msk));
    float ws = 0.f, an = 0.f;
    for (int e = lane; e < ne; e += 64) {
        const float2 ml = W.ml[row_of(e)];
        const float w = M == -INFINITY ? 0.f : exp2f(ml.x - M);
        wsh[e] = w;
        ws += w;
        an = fmaf(w, ml.y, an);
    }
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) {
        ws += shfl_xor(ws, msk);
        an += shfl_xor(an, msk);
    }
    lds_sync();
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int e0 = 0; e0 < ne; e0 += 2 * BATCH) {
        if (e0 > 0) {
#pragma unroll
            for (int k = 0; k < BATCH; k++) {
                const int e = e0 + ph + 2 * k;
                ov[k] = e < ne ? *(const float4 *)(W.o + row_of(e) * D + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int k = 0; k < BATCH; k++) {
            const int e = e0 + ph + 2 * k;
            const float w = e < ne ? wsh[e] : 0.f;
            acc.x = fmaf(w, ov[k].x, acc.x);
            acc.y = fmaf(w, ov[k].y, acc.y);
            acc.z = fmaf(w, ov[k].z, acc.z);
            acc.w = fmaf(w, ov[k].w, acc.w);
        }
    }
    acc.x += shfl_xor(acc.x, 32);
    acc.y += shfl_xor(acc.y, 32);
    acc.z += shfl_xor(acc.z, 32);
    acc.w += shfl_xor(acc.w, 32);
    const float inv = ws > 0.f ? 1.0f / ws : 0.f;
    if (ph == 0)
        *(float4 *)(out + ((size_t)b * P.Hq + hq) * D + 4 * c4) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (cert && lane == 0) cert[(size_t)b * P.Hq + hq] = ws > 0.f ? an / ws : 0.f;
}

// ---------------------------------------------------------------------------
namespace {
constexpr int MAX_DEVICES = 64;
std::atomic<void *> scratch_ptr[MAX_DEVICES];
std::mutex scratch_mu;
}  // namespace

hipError_t noalloc_scratch(void **ptr, size_t *bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));     // device `dev` is current
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    *bytes = sizeof(scratch);
    return hipSuccess;
}

hipError_t launch_stage1_floor(const KParams &P, const uint16_t *q, float sm_scale, const Workspace &W,
                              hipStream_t s) {
    if (!gqa4_path(P.scheme, P.qpk, P.force_generic)) return hipErrorInvalidValue;
    const float qscale = sm_scale * 1.4426950408889634f;
    plan_kernel<<<PLAN_G, PLAN_T, 0, s>>>(P, W);
    if (W.ev_begin) {
        hipError_t e = hipEventRecord(W.ev_begin, s);
        if (e != hipSuccess) return e;
    }
    dim3 g1(W.max_splits + W.n_win, P.Hkv, P.B);   // the group kernel's grid
    switch (P.qpk) {
        case 2: stage1_gqa4_floor_kernel<2><<<g1, 64, 0, s>>>(P, q, W, qscale); break;
        case 4: stage1_gqa4_floor_kernel<4><<<g1, 64, 0, s>>>(P, q, W, qscale); break;
        case 8: stage1_gqa4_floor_kernel<8><<<g1, 64, 0, s>>>(P, q, W, qscale); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (W.ev_end) e = hipEventRecord(W.ev_end, s);
    return e;
}

hipError_t launch_decode(const KParams &P, const uint16_t *q, float *out, float *cert,
                         float sm_scale, float kappa, const Workspace &W, hipStream_t s) {
    const float qscale = sm_scale * 1.4426950408889634f;
    const bool gqa4 = gqa4_path(P.scheme, P.qpk, P.force_generic);
    if (gqa4) plan_kernel<<<PLAN_G, PLAN_T, 0, s>>>(P, W);
    if (W.ev_begin) {
        hipError_t e = hipEventRecord(W.ev_begin, s);
        if (e != hipSuccess) return e;
    }
    if (P.scheme == KVQ_SCHEME_WITCERT_PAGED) {
        dim3 g1(W.max_splits, P.Hkv, P.B);            // no fp16 tail, no window chunks
        switch (P.qpk) {
            case 1: stage1_witcert_paged_kernel<1><<<g1, 64, 0, s>>>(P, q, W, qscale, sm_scale, kappa); break;
            case 2: stage1_witcert_paged_kernel<2><<<g1, 64, 0, s>>>(P, q, W, qscale, sm_scale, kappa); break;
            case 4: stage1_witcert_paged_kernel<4><<<g1, 64, 0, s>>>(P, q, W, qscale, sm_scale, kappa); break;
            case 8: stage1_witcert_paged_kernel<8><<<g1, 64, 0, s>>>(P, q, W, qscale, sm_scale, kappa); break;
            default: return hipErrorInvalidValue;
        }
    } else if (P.scheme == KVQ_SCHEME_WITCERT) {
        dim3 g1(W.max_splits + W.n_win, P.Hkv, P.B);  // + the window chunks of each KV head
        switch (P.qpk) {
            case 1: stage1_witcert_kernel<1><<<g1, 64, 0, s>>>(P, q, W, qscale, sm_scale, kappa); break;
            case 2: stage1_witcert_kernel<2><<<g1, 64, 0, s>>>(P, q, W, qscale, sm_scale, kappa); break;
            case 4: stage1_witcert_kernel<4><<<g1, 64, 0, s>>>(P, q, W, qscale, sm_scale, kappa); break;
            case 8: stage1_witcert_kernel<8><<<g1, 64, 0, s>>>(P, q, W, qscale, sm_scale, kappa); break;
            default: return hipErrorInvalidValue;
        }
    } else if (gqa4) {
        // room for every split of every KV head, then the window chunks; a
        // wave per query quad
        dim3 g1(W.max_splits + W.n_win, P.Hkv, P.B);
        switch (P.qpk) {
            case 2: stage1_gqa4_mfma_kernel<2><<<g1, 64, 0, s>>>(P, q, W, qscale); break;
            case 4: stage1_gqa4_mfma_kernel<4><<<g1, 64, 0, s>>>(P, q, W, qscale); break;
            case 8: stage1_gqa4_mfma_kernel<8><<<g1, 64, 0, s>>>(P, q, W, qscale); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        dim3 g1(W.max_splits + W.n_win, P.Hq, P.B);   // + the window chunks of each query head
        const bool kitty = P.scheme == KVQ_SCHEME_KITTY;
        if (P.force_generic) {
            if (kitty)
                stage1_valu_kernel<true><<<g1, 64, 0, s>>>(P, q, W, qscale);
            else
                stage1_valu_kernel<false><<<g1, 64, 0, s>>>(P, q, W, qscale);
        } else {
            if (P.scheme == KVQ_SCHEME_KITTY_DYN)
                stage1_head_mfma_kernel<true, true, false><<<g1, 64, 0, s>>>(P, q, W, qscale);
            else if (kitty)
                stage1_head_mfma_kernel<true, false, false><<<g1, 64, 0, s>>>(P, q, W, qscale);
            else if (P.scheme == KVQ_SCHEME_KIVI4)
                stage1_head_mfma_kernel<false, false, true><<<g1, 64, 0, s>>>(P, q, W, qscale);
            else
                stage1_head_mfma_kernel<false, false, false><<<g1, 64, 0, s>>>(P, q, W, qscale);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (W.ev_end) {
        e = hipEventRecord(W.ev_end, s);
        if (e != hipSuccess) return e;
    }
    merge_kernel<<<dim3(P.Hq, P.B), 64, 0, s>>>(P, out, cert, W);
    return hipGetLastError();
}

}  // namespace kvq
