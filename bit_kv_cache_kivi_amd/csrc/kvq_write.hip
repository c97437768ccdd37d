// kvq_write.hip -- write path: token append (value FIFO pack), key group
// flush, bulk prefill and Kitty calibration for KIVI2 / KITTY; active-block
// append, block flush and prefill for WITCERT.
//
// KIVI2: keys gather in an fp16 residual and are quantized per channel in
// groups of 32 tokens once R have gathered; values leave an R-token fp16 FIFO
// one at a time and are quantized per token in groups of 32 channels ("KIVI"
// explainer 3.3).  KITTY boosts 16 key channels to 4 bits and stores their
// high 2 bits in a separate plane ("Kitty" summary, Dense-Sparse
// Decomposition).  WITCERT quantizes whole 256-token blocks per channel with
// Philox dither ("WitCert" write-kernel paragraph).
#include "kvq_common.hpp"
#include "kvq_kernels.hpp"

namespace kvq {

__device__ inline uint8_t *page_ptr(const KParams &P, int pid, int h) {
    return P.pool + ((size_t)pid * P.Hkv + h) * (size_t)P.page_bytes;
}

// A stored value scale the matrix-core stage 1 cannot carry (above
// VALUE_SCALE_MAX): reported when the layout decodes on the matrix cores.
__device__ inline void flag_value_scale(const KParams &P, float s) {
    if (!P.force_generic && s > VALUE_SCALE_MAX) atomicOr(P.status, (uint32_t)KVQ_STATUS_RANGE);
}

__device__ inline bool page_ok(const KParams &P, int pid) {
    return pid >= 0 && pid < P.n_pages;
}

// ---------------------------------------------------------------------------
// KIVI2 / KITTY: quantize the keys of one 64-token page from fp16 rows
// src[t * D + c] (t in [0, 64)).  256 threads: thread (c = tid & 127,
// half = tid >> 7) takes the two 32-token groups half, half + 2 ... of its
// channel.  codes: LDS scratch [64][128].
// ---------------------------------------------------------------------------
// |x| * 2^24 of a binary16 value as an exact integer (finite values: at most
// 2^40, so 64 of them add exactly in 64 bits)
__device__ inline uint64_t mag24(uint16_t h) {
    const uint32_t e = (h >> 10) & 31u, m = h & 0x3ffu;
    return e == 0 ? (uint64_t)m : (uint64_t)(0x400u | m) << (e - 1);
}

// KITTY_DYN: the page's boosted channels, the NB largest sum_t |x_{t,c}| over
// its 64 tokens (the mean up to the fixed count; ties to the lower channel),
// into bits4 / inv and the page's KI bytes (channel ids, ascending)
__device__ void select_page_boost(const Geom &G, const uint16_t *src, uint8_t *page, int *inv,
                                  uint8_t *bits4, int nb, uint64_t *imp, int tid) {
    if (tid < D) {
        uint64_t sum = 0;
        for (int t = 0; t < PT; t++) sum += mag24(src[(size_t)t * D + tid]);
        imp[tid] = sum;
    }
    __syncthreads();
    if (tid < D) {
        const uint64_t mine = imp[tid];
        int rank = 0;
        for (int c2 = 0; c2 < D; c2++) {
            const uint64_t o = imp[c2];
            rank += (o > mine || (o == mine && c2 < tid)) ? 1 : 0;
        }
        bits4[tid] = rank < nb ? 1 : 0;
    }
    __syncthreads();
    if (tid < D && bits4[tid]) {
        int off = 0;
        for (int c2 = 0; c2 < tid; c2++) off += bits4[c2];
        inv[off] = tid;
        page[G.ki + off] = (uint8_t)tid;
    }
    __syncthreads();
}

// tid: the thread's index among the page's 256 (a block may quantize several
// pages side by side, each with its own LDS arrays; every thread of the block
// calls this once, so the barriers match).
__device__ void quant_key_page(const KParams &P, const Geom &G, const uint16_t *src,
                               uint8_t *page, int *inv, uint8_t *bits4,
                               uint8_t (*codes)[D], uint64_t *imp, int tid) {
    if (P.scheme == KVQ_SCHEME_KITTY_DYN) select_page_boost(G, src, page, inv, bits4, P.nb, imp, tid);
    const int c = tid & 127;
    const int gi = tid >> 7;                         // group 0 or 1 of the page
    const bool four = P.scheme == KVQ_SCHEME_KIVI4;
    const float lmax = (four || bits4[c]) ? 15.0f : 3.0f;
    float xs[32];
    float mn = 0.f, mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i++) {
        xs[i] = h2f(src[(size_t)(32 * gi + i) * D + c]);
        if (i == 0) { mn = xs[0]; mx = xs[0]; }
        else { mn = fminf(mn, xs[i]); mx = fmaxf(mx, xs[i]); }
    }
    AsymParams ap = asym_params(mn, mx, lmax);
#pragma unroll
    for (int i = 0; i < 32; i++) codes[32 * gi + i][c] = (uint8_t)asym_code(xs[i], ap, lmax);
    uint32_t *ks = (uint32_t *)(page + G.ks);
    ks[128 * gi + key_stat_slot(c)] = (uint32_t)ap.s16 | ((uint32_t)ap.z16 << 16);
    __syncthreads();
    uint32_t *kc = (uint32_t *)(page + G.kc);
    if (four) {                                      // 1024 dwords (see key_code_pos4)
        for (int w = tid; w < 1024; w += 256) {
            const int n = w >> 8, L = (w >> 2) & 63, kq = w & 3;
            const int t = 16 * n + (L & 15), c0 = 32 * kq + 8 * (L >> 4);
            uint32_t val = 0;
#pragma unroll
            for (int k = 0; k < 8; k++) val |= (uint32_t)codes[t][c0 + k] << (8 * (k & 3) + 4 * (k >> 2));
            kc[w] = val;
        }
    } else {
        for (int w = tid; w < 512; w += 256) {
            int d = 4 * (w >> 8) + (w & 3);
            int L = (w >> 2) & 63;
            int g = L >> 4, r = L & 15;
            int t = 16 * (d >> 1) + r;
            int kcb = 2 * (d & 1);
            uint32_t val = 0;
#pragma unroll
            for (int hh = 0; hh < 2; hh++)
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    int cc = 32 * (kcb + hh) + 8 * g + j;
                    val |= (uint32_t)(codes[t][cc] & 3) << (4 * j + 2 * hh);
                }
            kc[w] = val;
        }
    }
    if (is_kitty(P.scheme) && tid < 4 * P.nb) {
        // high plane q = tid >> 6 (offsets 16q ..): dword tid (see high_code_pos)
        uint32_t *kh = (uint32_t *)(page + G.kh);
        int q = tid >> 6, g = (tid >> 4) & 3, r = tid & 15;
        uint32_t val = 0;
        for (int n = 0; n < 4; n++)
            for (int i = 0; i < 4; i++) {
                int o = 16 * q + 4 * g + i;
                int cc = inv[o];
                uint32_t hi = (uint32_t)(codes[16 * n + r][cc] >> 2);
                val |= hi << (4 * (4 * (n & 1) + i) + 2 * (n >> 1));
            }
        kh[tid] = val;
    }
    __syncthreads();
}

// Kitty boost tables of KV head h in LDS: bits4[c] (channel takes 16 levels)
// and inv[o] (channel of high-plane offset o); tid as in quant_key_page.
__device__ void load_boost(const KParams &P, int h, int *inv, uint8_t *bits4, int tid) {
    if (tid < NB_MAX) inv[tid] = 0;
    __syncthreads();
    if (tid < D) {
        bits4[tid] = 0;
        if (P.scheme == KVQ_SCHEME_KITTY) {
            int o = P.boost_idx[(size_t)h * D + tid];
            if (o < P.nb) {
                bits4[tid] = 1;
                inv[o] = tid;
            }
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// append (KIVI2 / KITTY / KIVI4): one wave per (KV head, request)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void append_kivi_kernel(KParams P, const uint16_t *__restrict__ kn,
                                                         const uint16_t *__restrict__ vn) {
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const Geom G = geom(P.scheme, P.nb);
    const size_t bh = (size_t)b * P.Hkv + h;
    int32_t *st = P.state + bh * 4;
    // the new key and value and the state are loaded before anything waits
    // for them: {l, n_kq} as one pair
    const uint32_t knew = ((const uint32_t *)(kn + bh * D))[lane];
    const uint32_t vnew = ((const uint32_t *)(vn + bh * D))[lane];
    const int2 lk = *(const int2 *)st;
    const int l = lk.x, nkq = lk.y;
    asm volatile("" ::"s"(l), "s"(nkq));           // both halves before the branches below
    const int R = P.R, S = P.sink;
    if (l < S) {                                     // a sink token: kept fp16, outside the windows
        ((uint32_t *)P.sink_k)[(bh * S + (size_t)l) * (D / 2) + lane] = knew;
        ((uint32_t *)P.sink_v)[(bh * S + (size_t)l) * (D / 2) + lane] = vnew;
        if (lane == 0) {
            st[0] = l + 1;
            st[1] = l + 1;
        }
        return;
    }
    if (l - nkq >= R) {
        if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_RESIDUAL_FULL);
        return;
    }
    if (l >= S + P.max_pages * PT) {
        if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_CAPACITY);
        return;
    }
    uint32_t *rk = (uint32_t *)(P.res_k + (bh * R + (size_t)(l - nkq)) * D);
    uint32_t *rv = (uint32_t *)(P.res_v + (bh * R + (size_t)(l % R)) * D);
    if (l - S >= R) {
        // the token leaving the fp16 value window is quantized per token, at
        // quantized position t - S
        const int t = l - R - S;
        const int pid = P.table[(size_t)b * P.max_pages + t / PT];
        const uint32_t old = rv[lane];               // channels 2*lane, 2*lane+1 (issued with the id)
        asm volatile("" ::"v"(old));                  // loaded together with the id, not after its check
        if (!page_ok(P, pid)) {
            if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
            return;
        }
        uint8_t *page = page_ptr(P, pid, h);
        const float x0 = h2f((uint16_t)(old & 0xffffu)), x1 = h2f((uint16_t)(old >> 16));
        float mn = fminf(x0, x1), mx = fmaxf(x0, x1);
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) {           // 16 lanes = one 32-channel group
            mn = fminf(mn, shfl_xor(mn, m));
            mx = fmaxf(mx, shfl_xor(mx, m));
        }
        const bool four = P.scheme == KVQ_SCHEME_KIVI4;
        const float lmax = four ? 15.0f : 3.0f;
        const AsymParams ap = asym_params(mn, mx, lmax);
        const uint32_t code[2] = {asym_code(x0, ap, lmax), asym_code(x1, ap, lmax)};
        const int tp = t % PT;
        uint32_t *vc = (uint32_t *)(page + G.vc);
        const uint32_t cm = four ? 15u : 3u;
#pragma unroll
        for (int e = 0; e < 2; e++) {
            int dw, sh;
            if (four) value_code_pos4(tp, 2 * lane + e, dw, sh);
            else value_code_pos(tp, 2 * lane + e, dw, sh);
            uint32_t w = vc[dw];
            w = (w & ~(cm << sh)) | (code[e] << sh);
            vc[dw] = w;
        }
        if ((lane & 15) == 0) {
            uint32_t *vs = (uint32_t *)(page + G.vs);
            vs[tp * 4 + (lane >> 4)] = (uint32_t)ap.s16 | ((uint32_t)ap.z16 << 16);
            flag_value_scale(P, ap.s);
        }
    }
    rk[lane] = knew;
    rv[lane] = vnew;
    if (lane == 0) st[0] = l + 1;
}

// ---------------------------------------------------------------------------
// flush (KIVI2 / KITTY / KIVI4): 256 threads per page of the residual (R / 64
// pages, quantized side by side) per (KV head, request)
// ---------------------------------------------------------------------------
constexpr int FLUSH_MAX_PAGES = 4;                   // R <= 256
__global__ __launch_bounds__(256 * FLUSH_MAX_PAGES) void flush_kivi_kernel(KParams P) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int pi = threadIdx.x >> 8, tid = threadIdx.x & 255;   // page of the residual, thread in it
    const Geom G = geom(P.scheme, P.nb);
    const size_t bh = (size_t)b * P.Hkv + h;
    int32_t *st = P.state + bh * 4;
    const int l = st[0], nkq = st[1];
    if (l - nkq != P.R) return;
    __shared__ uint8_t codes[FLUSH_MAX_PAGES][PT][D];
    __shared__ int inv[FLUSH_MAX_PAGES][NB_MAX];
    __shared__ uint8_t bits4[FLUSH_MAX_PAGES][D];
    __shared__ uint64_t imp[FLUSH_MAX_PAGES][D];
    __shared__ int bad;
    const int np = P.R / PT;                         // = blockDim.x / 256
    const int p0 = (nkq - P.sink) / PT;              // quantized positions count from the sink
    if (threadIdx.x == 0) {
        bad = 0;
        for (int p = 0; p < np; p++)
            if (!page_ok(P, P.table[(size_t)b * P.max_pages + p0 + p])) bad = 1;
    }
    load_boost(P, h, inv[pi], bits4[pi], tid);       // contains __syncthreads
    if (bad) {
        if (threadIdx.x == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
        return;
    }
    const int pid = P.table[(size_t)b * P.max_pages + p0 + pi];
    quant_key_page(P, G, P.res_k + (bh * P.R + (size_t)pi * PT) * D, page_ptr(P, pid, h),
                   inv[pi], bits4[pi], codes[pi], imp[pi], tid);
    if (threadIdx.x == 0) st[1] = nkq + P.R;         // after the block's last barrier: all read nkq
}

// ---------------------------------------------------------------------------
// prefill (KIVI2 / KITTY / KIVI4): one 256-thread block per (page, KV head, request)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_kivi_kernel(KParams P, int req0,
                                                          const uint16_t *__restrict__ K,
                                                          const uint16_t *__restrict__ V,
                                                          long long ld,
                                                          const int32_t *__restrict__ lengths) {
    const int p = blockIdx.x, h = blockIdx.y, rr = blockIdx.z, b = req0 + rr;
    const int tid = threadIdx.x;
    const Geom G = geom(P.scheme, P.nb);
    const int R = P.R, S = P.sink;
    const int len = lengths[rr];
    if (len < 0 || len > S + P.max_pages * PT || (long long)len > ld) {
        if (p == 0 && tid == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_BAD_LENGTH);
        return;
    }
    // tokens past the sink: the key residual keeps ((lq - 1) mod R) + 1 of
    // them, the value window the newest min(lq, R)
    const int lq = max(0, len - S);
    const int rk = lq ? ((lq - 1) % R) + 1 : 0;
    const int nkq = len - rk;
    const int nvq = S + (lq > R ? lq - R : 0);
    const size_t bh = (size_t)b * P.Hkv + h;
    if (p == 0 && tid == 0) {
        P.state[bh * 4 + 0] = len;
        P.state[bh * 4 + 1] = nkq;
        P.state[bh * 4 + 2] = 0;
        P.state[bh * 4 + 3] = 0;
    }
    const uint16_t *Ks = K + ((size_t)rr * P.Hkv + h) * (size_t)ld * D;
    const uint16_t *Vs = V + ((size_t)rr * P.Hkv + h) * (size_t)ld * D;
    if (p == 0) {                                    // the sink tokens, fp16
        const int ns = min(len, S);
        for (int i = tid; i < ns * (D / 2); i += 256) {
            const int t = i / (D / 2), w = i % (D / 2);
            ((uint32_t *)P.sink_k)[(bh * S + (size_t)t) * (D / 2) + w] = ((const uint32_t *)Ks)[(size_t)t * (D / 2) + w];
            ((uint32_t *)P.sink_v)[(bh * S + (size_t)t) * (D / 2) + w] = ((const uint32_t *)Vs)[(size_t)t * (D / 2) + w];
        }
    }
    const int t0 = S + p * PT;                       // page p holds quantized positions p*64 ..
    if (t0 >= len) return;
    // fp16 windows: keys [nkq, len) and values [nvq, len) of this page
    for (int i = tid; i < PT * (D / 2); i += 256) {
        const int t = t0 + i / (D / 2), w = i % (D / 2);
        if (t >= len) break;
        if (t >= nkq)
            ((uint32_t *)P.res_k)[(bh * R + (size_t)(t - nkq)) * (D / 2) + w] =
                ((const uint32_t *)Ks)[(size_t)t * (D / 2) + w];
        if (t >= nvq)
            ((uint32_t *)P.res_v)[(bh * R + (size_t)(t % R)) * (D / 2) + w] =
                ((const uint32_t *)Vs)[(size_t)t * (D / 2) + w];
    }
    if (t0 >= nkq && t0 >= nvq) return;
    const int pid = P.table[(size_t)b * P.max_pages + p];
    if (!page_ok(P, pid)) {
        if (tid == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
        return;
    }
    uint8_t *page = page_ptr(P, pid, h);
    __shared__ uint8_t codes[PT][D];
    __shared__ int inv[NB_MAX];
    __shared__ uint8_t bits4[D];
    __shared__ uint64_t imp[D];
    load_boost(P, h, inv, bits4, tid);
    if (t0 < nkq)                                    // nkq - S is a multiple of 128: whole page
        quant_key_page(P, G, Ks + (size_t)t0 * D, page, inv, bits4, codes, imp, tid);
    if (t0 < nvq) {
        // values, per token, groups of 32 channels: thread (token tl, group jv)
        const int tl = tid >> 2, jv = tid & 3;
        const int t = t0 + tl;
        const bool four = P.scheme == KVQ_SCHEME_KIVI4;
        const float lmax = four ? 15.0f : 3.0f;
        if (t < nvq) {
            float xs[32];
            float mn = 0.f, mx = 0.f;
#pragma unroll
            for (int i = 0; i < 32; i++) {
                xs[i] = h2f(Vs[(size_t)t * D + 32 * jv + i]);
                if (i == 0) { mn = xs[0]; mx = xs[0]; }
                else { mn = fminf(mn, xs[i]); mx = fmaxf(mx, xs[i]); }
            }
            AsymParams ap = asym_params(mn, mx, lmax);
#pragma unroll
            for (int i = 0; i < 32; i++) codes[tl][32 * jv + i] = (uint8_t)asym_code(xs[i], ap, lmax);
            ((uint32_t *)(page + G.vs))[tl * 4 + jv] = (uint32_t)ap.s16 | ((uint32_t)ap.z16 << 16);
            flag_value_scale(P, ap.s);
        } else {
#pragma unroll
            for (int i = 0; i < 32; i++) codes[tl][32 * jv + i] = 0;
        }
        __syncthreads();
        uint32_t *vc = (uint32_t *)(page + G.vc);
        if (four) {                                  // 1024 dwords (see value_code_pos4)
            for (int w = tid; w < 1024; w += 256) {
                const int d = 4 * (w >> 8) + (w & 3), L = (w >> 2) & 63;
                const int c = 16 * (d & 7) + (L & 15), tb = 32 * (d >> 3) + 8 * (L >> 4);
                uint32_t val = 0;
#pragma unroll
                for (int k = 0; k < 8; k++) val |= (uint32_t)codes[tb + k][c] << (8 * (k & 3) + 4 * (k >> 2));
                vc[w] = val;
            }
        } else {
            for (int w = tid; w < 512; w += 256) {
                const int nt = 4 * (w >> 8) + (w & 3);
                const int L = (w >> 2) & 63;
                const int g = L >> 4, r = L & 15;
                const int c = 16 * nt + r;
                uint32_t val = 0;
#pragma unroll
                for (int ks = 0; ks < 2; ks++)
#pragma unroll
                    for (int j = 0; j < 8; j++)
                        val |= (uint32_t)codes[32 * ks + 8 * g + j][c] << (4 * j + 2 * ks);
                vc[w] = val;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Kitty calibration: static boost set per KV head from a calibration slice
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void kitty_calibrate_kernel(const uint16_t *__restrict__ calib,
                                                             int T, int nb, uint8_t *__restrict__ idx_out) {
    const int h = blockIdx.x, c = threadIdx.x;
    __shared__ float am[D];
    __shared__ uint8_t chosen[D];
    float a = 0.0f;
    for (int t = 0; t < T; t++) a = fmaxf(a, fabsf(h2f(calib[((size_t)h * T + t) * D + c])));
    am[c] = a;
    chosen[c] = 0;
    __syncthreads();
    if (c == 0) {
        for (int j = 0; j < nb; j++) {
            int best = -1;
            for (int cc = 0; cc < D; cc++)
                if (!chosen[cc] && (best < 0 || am[cc] > am[best])) best = cc;
            chosen[best] = 1;
        }
        int off = 0;
        for (int cc = 0; cc < D; cc++)
            idx_out[(size_t)h * D + cc] = chosen[cc] ? (uint8_t)(off++) : (uint8_t)(nb + 1);
    }
}

// ---------------------------------------------------------------------------
// WITCERT
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void append_witcert_kernel(KParams P, const uint16_t *__restrict__ kn,
                                                            const uint16_t *__restrict__ vn) {
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const size_t bh = (size_t)b * P.Hkv + h;
    int32_t *st = P.state + bh * 4;
    const int l = st[0], nq = st[1];
    if (l - nq >= WPT) {
        if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_RESIDUAL_FULL);
        return;
    }
    if (l >= P.max_pages * WPT) {
        if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_CAPACITY);
        return;
    }
    const size_t row = (bh * WPT + (size_t)(l - nq)) * (D / 2);
    ((uint32_t *)P.res_k)[row + lane] = ((const uint32_t *)kn)[bh * (D / 2) + lane];
    ((uint32_t *)P.res_v)[row + lane] = ((const uint32_t *)vn)[bh * (D / 2) + lane];
    if (lane == 0) st[0] = l + 1;
}

// Quantize one 256-token block (keys or values) of KV head h, request b from
// fp16 rows src[t * D + c].  256 threads.  Pass 1: amax per channel (thread
// (c, half) over 128 tokens, combined in LDS).  Pass 2: thread (channel quad
// cq = tid & 31, token phase tp = tid >> 5) draws one Philox4x32-10 block per
// token and uses all four words for channels 4cq .. 4cq+3.
__device__ void quant_witcert_block(const KParams &P, int b, int h, int blk, int side,
                                    const uint16_t *src, int8_t *codes, uint16_t *scales,
                                    float *amax_s) {
    const int tid = threadIdx.x;
    {
        const int c = tid & 127, half = tid >> 7;
        float a = 0.0f;
        for (int i = 0; i < 128; i++)
            a = fmaxf(a, fabsf(h2f(src[(size_t)(128 * half + i) * D + c])));
        amax_s[tid] = a;
    }
    __syncthreads();
    if (tid < D) {
#pragma clang fp contract(off)
        const float a = fmaxf(amax_s[tid], amax_s[tid + 128]);
        uint16_t s16 = 0;
        if (a > 0.0f) {
            s16 = f2h(a / 126.5f);
            if (127.0f * h2f(s16) <= a) s16 = (uint16_t)(s16 + 1);
        }
        scales[tid] = s16;
    }
    __syncthreads();
    const int cq = tid & 31, tp = tid >> 5;
    float s[4];
    bool nz[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const uint16_t s16 = scales[4 * cq + e];
        s[e] = h2f(s16);
        nz[e] = s16 != 0;
    }
    const uint32_t k0 = (uint32_t)P.seed;
    const uint32_t k1 = (uint32_t)(P.seed >> 32) ^ (uint32_t)side;
    for (int i = 0; i < WPT / 8; i++) {
        const int t = tp + 8 * i;
        const uint32_t tok = (uint32_t)(blk * WPT + t);
        U4 ctr{tok, (uint32_t)cq, (P.layer << 16) | (uint32_t)h, (uint32_t)b};
        U4 u = philox4x32_10(ctr, k0, k1);
        const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
        const uint2 xin = *(const uint2 *)(src + (size_t)t * D + 4 * cq);
        const uint16_t xb[4] = {(uint16_t)(xin.x & 0xffff), (uint16_t)(xin.x >> 16),
                                (uint16_t)(xin.y & 0xffff), (uint16_t)(xin.y >> 16)};
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
#pragma clang fp contract(off)
            float c = 0.0f;
            if (nz[e]) {
                const float xi = dither_from_word(wv[e]);
                const float q = h2f(xb[e]) / s[e];
                c = rintf(q + xi);
                c = fminf(fmaxf(c, -127.0f), 127.0f);
            }
            packed |= ((uint32_t)(uint8_t)(int8_t)(int)c) << (8 * e);
        }
        *(uint32_t *)(codes + (size_t)t * D + 4 * cq) = packed;
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void flush_witcert_kernel(KParams P) {
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const Geom G = geom(P.scheme, P.nb);
    const size_t bh = (size_t)b * P.Hkv + h;
    int32_t *st = P.state + bh * 4;
    const int l = st[0], nq = st[1];
    if (l - nq != WPT) return;
    const int blk = nq / WPT;
    const int pid = P.table[(size_t)b * P.max_pages + blk];
    if (!page_ok(P, pid)) {
        if (tid == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
        return;
    }
    __shared__ float amax_s[256];
    __shared__ uint16_t scales[D];
    uint8_t *page = page_ptr(P, pid, h);
    for (int side = 0; side < 2; side++) {
        const uint16_t *src = (side ? P.res_v : P.res_k) + bh * WPT * D;
        quant_witcert_block(P, b, h, blk, side, src, (int8_t *)(page + (side ? G.vc : G.kc)),
                            scales, amax_s);
        if (tid < D) ((uint16_t *)(page + (side ? G.vs : G.ks)))[tid] = scales[tid];
        __syncthreads();
    }
    if (tid == 0) st[1] = nq + WPT;
}

__global__ __launch_bounds__(256) void prefill_witcert_kernel(KParams P, int req0,
                                                             const uint16_t *__restrict__ K,
                                                             const uint16_t *__restrict__ V,
                                                             long long ld,
                                                             const int32_t *__restrict__ lengths) {
    const int p = blockIdx.x, h = blockIdx.y, rr = blockIdx.z, b = req0 + rr;
    const int tid = threadIdx.x;
    const Geom G = geom(P.scheme, P.nb);
    const int len = lengths[rr];
    if (len < 0 || len > P.max_pages * WPT || (long long)len > ld) {
        if (p == 0 && tid == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_BAD_LENGTH);
        return;
    }
    const int r = len ? ((len - 1) % WPT) + 1 : 0;
    const int nq = len - r;
    const size_t bh = (size_t)b * P.Hkv + h;
    if (p == 0 && tid == 0) {
        P.state[bh * 4 + 0] = len;
        P.state[bh * 4 + 1] = nq;
        P.state[bh * 4 + 2] = 0;
        P.state[bh * 4 + 3] = 0;
    }
    const int t0 = p * WPT;
    if (t0 >= len) return;
    const uint16_t *Ks = K + ((size_t)rr * P.Hkv + h) * (size_t)ld * D;
    const uint16_t *Vs = V + ((size_t)rr * P.Hkv + h) * (size_t)ld * D;
    if (t0 >= nq) {                                  // the active block: copy to fp16
        for (int i = tid; i < WPT * (D / 2); i += 256) {
            const int t = t0 + i / (D / 2), w = i % (D / 2);
            if (t >= len) break;
            const size_t dst = (bh * WPT + (size_t)(t - nq)) * (D / 2) + w;
            ((uint32_t *)P.res_k)[dst] = ((const uint32_t *)Ks)[(size_t)t * (D / 2) + w];
            ((uint32_t *)P.res_v)[dst] = ((const uint32_t *)Vs)[(size_t)t * (D / 2) + w];
        }
        return;
    }
    const int pid = P.table[(size_t)b * P.max_pages + p];
    if (!page_ok(P, pid)) {
        if (tid == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
        return;
    }
    __shared__ float amax_s[256];
    __shared__ uint16_t scales[D];
    uint8_t *page = page_ptr(P, pid, h);
    for (int side = 0; side < 2; side++) {
        const uint16_t *src = (side ? Vs : Ks) + (size_t)t0 * D;
        quant_witcert_block(P, b, h, p, side, src, (int8_t *)(page + (side ? G.vc : G.kc)),
                            scales, amax_s);
        if (tid < D) ((uint16_t *)(page + (side ? G.vs : G.ks)))[tid] = scales[tid];
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// WITCERT_PAGED: each token quantized as it is written ("WitCert" page,
// certified deployment): one fp16 scale s = amax/126.5 per (token, group of
// 32 channels) on each side, quantized with the stored scale; the dither of
// channel c from the Philox4x32-10 block with counter (slot_lo, c >> 2,
// (layer << 16) | KV head, slot_hi), word c & 3, slot = page_id * 64 +
// position in the page; bypassed key channels (the fixed outlier RoPE pairs)
// are left out of their group's amax, get code 0 and are kept fp16 in the
// token's bypass row.
// ---------------------------------------------------------------------------
__device__ inline uint16_t witcert_scale16(float a) {
#pragma clang fp contract(off)
    uint16_t s16 = 0;
    if (a > 0.0f) {
        s16 = f2h(a / 126.5f);
        if (127.0f * h2f(s16) <= a) s16 = (uint16_t)(s16 + 1);
    }
    return s16;
}

__device__ inline uint32_t witcert_code8(uint16_t xb, float s, bool nz, uint32_t word) {
#pragma clang fp contract(off)
    float c = 0.0f;
    if (nz) {
        const float xi = dither_from_word(word);
        const float q = h2f(xb) / s;
        c = rintf(q + xi);
        c = fminf(fmaxf(c, -127.0f), 127.0f);
    }
    return (uint32_t)(uint8_t)(int8_t)(int)c;
}

__device__ inline U4 slot_philox(const KParams &P, int h, uint64_t slot, uint32_t quad, int side) {
    return philox4x32_10(U4{(uint32_t)slot, quad, (P.layer << 16) | (uint32_t)h, (uint32_t)(slot >> 32)},
                         (uint32_t)P.seed, (uint32_t)(P.seed >> 32) ^ (uint32_t)side);
}

// Bypass offset of channel c of KV head h (2 nb + 1 when not bypassed).
__device__ inline int bypass_off(const KParams &P, int h, int c) {
    return P.nb > 0 ? (int)P.boost_idx[(size_t)h * D + c] : 1;
}

// One side of one token by one wave: lane = channels 2 lane, 2 lane + 1
// (quad lane >> 1, Philox words 2 (lane & 1) and 2 (lane & 1) + 1); the 16
// lanes of a group reduce its amax with shuffles.
__device__ inline void witcert_token_wave(const KParams &P, int h, uint64_t slot, int side,
                                          uint32_t xin, bool byp0, bool byp1,
                                          uint8_t *codes_row, uint16_t *scale_row) {
    const int lane = threadIdx.x;
    const uint16_t x0 = (uint16_t)(xin & 0xffffu), x1 = (uint16_t)(xin >> 16);
    float a = fmaxf(byp0 ? 0.0f : fabsf(h2f(x0)), byp1 ? 0.0f : fabsf(h2f(x1)));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) a = fmaxf(a, shfl_xor(a, m));
    const uint16_t s16 = witcert_scale16(a);
    const float s = h2f(s16);
    const U4 u = slot_philox(P, h, slot, (uint32_t)(lane >> 1), side);
    const uint32_t w0 = (lane & 1) ? u.z : u.x, w1 = (lane & 1) ? u.w : u.y;
    const uint32_t c0 = byp0 ? 0u : witcert_code8(x0, s, s16 != 0, w0);
    const uint32_t c1 = byp1 ? 0u : witcert_code8(x1, s, s16 != 0, w1);
    ((uint16_t *)codes_row)[lane] = (uint16_t)(c0 | (c1 << 8));
    if ((lane & 15) == 0) scale_row[lane >> 4] = s16;
}

__global__ __launch_bounds__(64) void append_witcert_paged_kernel(KParams P, const uint16_t *__restrict__ kn,
                                                                  const uint16_t *__restrict__ vn) {
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const Geom G = geom(P.scheme, P.nb);
    const size_t bh = (size_t)b * P.Hkv + h;
    int32_t *st = P.state + bh * 4;
    const int l = st[0];
    if (l >= P.max_pages * PT) {
        if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_CAPACITY);
        return;
    }
    const int pid = P.table[(size_t)b * P.max_pages + l / PT];
    if (!page_ok(P, pid)) {
        if (lane == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
        return;
    }
    uint8_t *page = page_ptr(P, pid, h);
    const int tp = l % PT;
    const uint64_t slot = (uint64_t)pid * PT + (uint64_t)tp;
    const uint32_t kin = ((const uint32_t *)kn)[bh * (D / 2) + lane];
    const uint32_t vin = ((const uint32_t *)vn)[bh * (D / 2) + lane];
    const int o0 = bypass_off(P, h, 2 * lane), o1 = bypass_off(P, h, 2 * lane + 1);
    const bool b0 = o0 < 2 * P.nb, b1 = o1 < 2 * P.nb;
    witcert_token_wave(P, h, slot, 0, kin, b0, b1, page + G.kc + (size_t)tp * D,
                       (uint16_t *)(page + G.ks) + 4 * tp);
    witcert_token_wave(P, h, slot, 1, vin, false, false, page + G.vc + (size_t)tp * D,
                       (uint16_t *)(page + G.vs) + 4 * tp);
    uint16_t *kb = (uint16_t *)(page + G.kh) + 8 * tp;
    if (b0) kb[o0] = (uint16_t)(kin & 0xffffu);
    if (b1) kb[o1] = (uint16_t)(kin >> 16);
    if (lane == 0) {
        st[0] = l + 1;
        st[1] = l + 1;
    }
}

// prefill: one 256-thread block per (page, KV head, request); thread (token
// tl = tid >> 2, group g = tid & 3) quantizes the group's 32 channels of one
// token on each side (eight Philox blocks per side).
__global__ __launch_bounds__(256) void prefill_witcert_paged_kernel(KParams P, int req0,
                                                                   const uint16_t *__restrict__ K,
                                                                   const uint16_t *__restrict__ V,
                                                                   long long ld,
                                                                   const int32_t *__restrict__ lengths) {
    const int p = blockIdx.x, h = blockIdx.y, rr = blockIdx.z, b = req0 + rr;
    const int tid = threadIdx.x;
    const Geom G = geom(P.scheme, P.nb);
    const int len = lengths[rr];
    if (len < 0 || len > P.max_pages * PT || (long long)len > ld) {
        if (p == 0 && tid == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_BAD_LENGTH);
        return;
    }
    const size_t bh = (size_t)b * P.Hkv + h;
    if (p == 0 && tid == 0) {
        P.state[bh * 4 + 0] = len;
        P.state[bh * 4 + 1] = len;
        P.state[bh * 4 + 2] = 0;
        P.state[bh * 4 + 3] = 0;
    }
    const int t0 = p * PT;
    if (t0 >= len) return;
    const int pid = P.table[(size_t)b * P.max_pages + p];
    if (!page_ok(P, pid)) {
        if (tid == 0) atomicOr(P.status, (uint32_t)KVQ_STATUS_UNMAPPED_PAGE);
        return;
    }
    uint8_t *page = page_ptr(P, pid, h);
    const int tl = tid >> 2, g = tid & 3;
    const int t = t0 + tl;
    if (t >= len) return;
    const uint64_t slot = (uint64_t)pid * PT + (uint64_t)tl;
    for (int side = 0; side < 2; side++) {
        const uint16_t *src = (side ? V : K) + (((size_t)rr * P.Hkv + h) * (size_t)ld + t) * D + 32 * g;
        uint16_t x[32];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint4 v4 = ((const uint4 *)src)[j];
            const uint32_t w[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                x[8 * j + 2 * e] = (uint16_t)(w[e] & 0xffffu);
                x[8 * j + 2 * e + 1] = (uint16_t)(w[e] >> 16);
            }
        }
        bool byp[32];
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; j++) {
            byp[j] = side == 0 && bypass_off(P, h, 32 * g + j) < 2 * P.nb;
            if (!byp[j]) a = fmaxf(a, fabsf(h2f(x[j])));
        }
        const uint16_t s16 = witcert_scale16(a);
        const float s = h2f(s16);
        uint32_t *crow = (uint32_t *)(page + (side ? G.vc : G.kc) + (size_t)tl * D + 32 * g);
#pragma unroll
        for (int qd = 0; qd < 8; qd++) {
            const U4 u = slot_philox(P, h, slot, (uint32_t)(8 * g + qd), side);
            const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int j = 4 * qd + e;
                const uint32_t c = byp[j] ? 0u : witcert_code8(x[j], s, s16 != 0, wv[e]);
                packed |= c << (8 * e);
            }
            crow[qd] = packed;
        }
        ((uint16_t *)(page + (side ? G.vs : G.ks)))[4 * tl + g] = s16;
        if (side == 0) {
            uint16_t *kb = (uint16_t *)(page + G.kh) + 8 * tl;
#pragma unroll
            for (int j = 0; j < 32; j++)
                if (byp[j]) kb[bypass_off(P, h, 32 * g + j)] = x[j];
        }
    }
}

// Fixed bypass set per KV head: pair i = channels (i, i + 64); importance
// max_t (x_i^2 + x_{i+64}^2) (squares exact in binary32, one rounding for
// the sum); the nb largest, ties to the lower pair; offsets in ascending
// channel order, others 2 nb + 1.  One wave per KV head, lane = pair.
__global__ __launch_bounds__(64) void witcert_calibrate_kernel(const uint16_t *__restrict__ calib, int T,
                                                               int nb, uint8_t *__restrict__ idx_out) {
    const int h = blockIdx.x, i = threadIdx.x;
    __shared__ float imp[D / 2];
    __shared__ uint8_t chosen[D];
    float e = 0.0f;
    for (int t = 0; t < T; t++) {
#pragma clang fp contract(off)
        const float a = h2f(calib[((size_t)h * T + t) * D + i]);
        const float c = h2f(calib[((size_t)h * T + t) * D + i + D / 2]);
        const float v = a * a + c * c;
        e = fmaxf(e, v);
    }
    imp[i] = e;
    chosen[i] = 0;
    chosen[i + D / 2] = 0;
    __syncthreads();
    if (i == 0) {
        for (int r = 0; r < nb; r++) {
            int best = -1;
            for (int j = 0; j < D / 2; j++)
                if (!chosen[j] && (best < 0 || imp[j] > imp[best])) best = j;
            chosen[best] = 1;
            chosen[best + D / 2] = 1;
        }
        int off = 0;
        for (int c = 0; c < D; c++)
            idx_out[(size_t)h * D + c] = chosen[c] ? (uint8_t)(off++) : (uint8_t)(2 * nb + 1);
    }
}

hipError_t launch_witcert_calibrate(const KParams &P, const uint16_t *calib, int n_tokens,
                                    uint8_t *idx_out, hipStream_t s) {
    witcert_calibrate_kernel<<<P.Hkv, 64, 0, s>>>(calib, n_tokens, P.nb, idx_out);
    return hipGetLastError();
}

hipError_t launch_append(const KParams &P, const uint16_t *k, const uint16_t *v, hipStream_t s) {
    dim3 grid(P.Hkv, P.B);
    if (P.scheme == KVQ_SCHEME_WITCERT)
        append_witcert_kernel<<<grid, 64, 0, s>>>(P, k, v);
    else if (P.scheme == KVQ_SCHEME_WITCERT_PAGED)
        append_witcert_paged_kernel<<<grid, 64, 0, s>>>(P, k, v);
    else
        append_kivi_kernel<<<grid, 64, 0, s>>>(P, k, v);
    return hipGetLastError();
}

hipError_t launch_flush(const KParams &P, hipStream_t s) {
    dim3 grid(P.Hkv, P.B);
    if (P.scheme == KVQ_SCHEME_WITCERT_PAGED) return hipSuccess;   // tokens are quantized on write
    if (P.scheme == KVQ_SCHEME_WITCERT)
        flush_witcert_kernel<<<grid, 256, 0, s>>>(P);
    else
        flush_kivi_kernel<<<grid, 256 * (P.R / PT), 0, s>>>(P);
    return hipGetLastError();
}

hipError_t launch_prefill(const KParams &P, int req0, int n_req, const uint16_t *K,
                          const uint16_t *V, long long ld, const int32_t *lengths,
                          hipStream_t s) {
    dim3 grid(P.max_pages, P.Hkv, n_req);
    if (P.scheme == KVQ_SCHEME_WITCERT)
        prefill_witcert_kernel<<<grid, 256, 0, s>>>(P, req0, K, V, ld, lengths);
    else if (P.scheme == KVQ_SCHEME_WITCERT_PAGED)
        prefill_witcert_paged_kernel<<<grid, 256, 0, s>>>(P, req0, K, V, ld, lengths);
    else
        prefill_kivi_kernel<<<grid, 256, 0, s>>>(P, req0, K, V, ld, lengths);
    return hipGetLastError();
}

hipError_t launch_kitty_calibrate(const KParams &P, const uint16_t *calib, int n_tokens,
                                  uint8_t *idx_out, hipStream_t s) {
    kitty_calibrate_kernel<<<P.Hkv, 128, 0, s>>>(calib, n_tokens, P.nb, idx_out);
    return hipGetLastError();
}

}  // namespace kvq
