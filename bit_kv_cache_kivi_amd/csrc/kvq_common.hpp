// kvq_common.hpp -- device-side layout and arithmetic shared by the kernels of
// libkvq.so (gfx950).  Host code includes it for the page geometry only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int D = 128;          // head dim
constexpr int PT = 64;          // tokens per KIVI2/KITTY page
constexpr int WPT = 256;        // tokens per WITCERT page (= one block)
constexpr int NB = 16;          // Kitty boosted channels per KV head (alpha = 1/8)
constexpr int NB_MAX = 32;      // Kitty-Pro: alpha = 1/4
// Largest value scale the matrix-core stage 1 carries: it forms p_t s_t with
// softmax weights p_t <= 256 as an f16 head, which must stay below 65504.
constexpr float VALUE_SCALE_MAX = 255.0f;
constexpr int MAX_RESIDUAL = 256;                  // largest fp16 window R (tokens)
constexpr int MAX_SPLITS = 256;                    // largest paged split count per query head
// window chunks per query head: R / 64 chunks plus one for the sink tokens
// (WITCERT: one 256-token block of four chunks)
constexpr int MAX_WIN = MAX_RESIDUAL / PT + 1;
static_assert(MAX_WIN >= WPT / PT, "window chunk bound");

// ---------------------------------------------------------------------------
// Page geometry.  One (page, KV head) block; the pool is
// [n_pages][n_kv_heads][page_bytes].
//
// KIVI2 / KITTY / KITTY_DYN, 64 tokens (nb boosted channels, 16 or 32):
//   KC  2048 B  low 2-bit key codes, token-major, arranged as the B operand of
//               a 16x16x32 f16 matrix-core product (see key_code_pos)
//   KH  16 nb B KITTY*: high 2-bit plane of the boosted channels, one 256-B
//               plane per 16 offsets (see high_code_pos)
//   KS  1024 B  key {scale, zero} fp16 pairs, [2 groups][128 channels]
//   VC  2048 B  value codes, channel-major (see value_code_pos)
//   VS  1024 B  value {scale, zero} fp16 pairs, [64 tokens][4 groups]
//   KI  max(16, nb) B  KITTY_DYN: the page's boosted channel ids, ascending
//               (the high-plane offset of KI[o] is o)
// KIVI4, 64 tokens:
//   KC 4096 B 4-bit key codes (see key_code_pos4), KS 1024 B as KIVI2,
//   VC 4096 B 4-bit value codes (see value_code_pos4), VS 1024 B as KIVI2
// WITCERT_PAGED, 64 tokens, every token quantized on write:
//   KC 8192 B int8 [64][128];  VC 8192 B int8 [64][128];
//   KS 512 B fp16 [64][4] key scales per (token, 32-channel group);
//   VS 512 B fp16 [64][4] value scales;
//   KH 1024 B fp16 [64][8] (nb > 0): the token's bypassed key channels, by
//   offset (ascending channel order), the rest of the row unused
// WITCERT, 256 tokens (one block):
//   KC 32768 B int8 [256][128];  KS 256 B fp16 [128];
//   VC 32768 B int8 [256][128];  VS 256 B fp16 [128]
// ---------------------------------------------------------------------------
struct Geom {
    int kc, kh, ks, vc, vs, ki, bytes, tokens;
};

__host__ __device__ constexpr bool is_kitty(int scheme) {
    return scheme == KVQ_SCHEME_KITTY || scheme == KVQ_SCHEME_KITTY_DYN;
}

// ---------------------------------------------------------------------------
// Splits of the group-of-4 stage 1 (KIVI2 with two, four or eight query heads
// per KV head, matrix-core kernel).  A (request, KV head) pair of npg pages is cut into
// body splits of sp pages over all but its last min(npg / 8, 2 sp) pages
// (and what rounding leaves), then tail splits of sp / 4 pages over the rest
// (the last one shorter): the work list runs the long body splits first and
// ends with small ones, which even out the workgroups' finishing times while
// most pages still go in long splits.  Split r of a pair writes partial row
// r.  Other stage-1 kernels cut every pair into splits of sp pages.
// ---------------------------------------------------------------------------
// The kernel serves query heads four at a time (a quad): a group of 8 is two
// quads per KV head, each page read once per quad; a group of 2 is one quad
// whose last two queries are zero and not written.
__host__ __device__ constexpr bool gqa4_path(int scheme, int qpk, bool generic) {
    return scheme == KVQ_SCHEME_KIVI2 && (qpk == 2 || qpk == 4 || qpk == 8) && !generic;
}
__host__ __device__ constexpr int gqa_quads(int qpk) { return qpk >= 4 ? qpk / 4 : 1; }
__host__ __device__ constexpr int gqa_tail_pages(int sp) { return sp >= 4 ? sp / 4 : 1; }
__host__ __device__ constexpr int gqa_tail_target(int npg, int sp) {
    return npg / 8 < 2 * sp ? npg / 8 : 2 * sp;
}
__host__ __device__ constexpr int gqa_body_splits(int npg, int sp) {
    return (npg - gqa_tail_target(npg, sp)) / sp;
}
// splits (partial rows) of a pair of npg pages
__host__ __device__ constexpr int gqa_splits(int npg, int sp) {
    return gqa_body_splits(npg, sp) +
           (npg - gqa_body_splits(npg, sp) * sp + gqa_tail_pages(sp) - 1) / gqa_tail_pages(sp);
}
// a bound on gqa_splits(npg, sp) over all npg <= m: the body count and the
// tail target are each non-decreasing in npg, and the tail holds at most the
// target plus sp - 1 pages
__host__ __device__ constexpr int gqa_splits_bound(int m, int sp) {
    return (m - gqa_tail_target(m, sp)) / sp +
           (gqa_tail_target(m, sp) + sp - 1 + gqa_tail_pages(sp) - 1) / gqa_tail_pages(sp);
}

__host__ __device__ inline Geom geom(int scheme, int nb = NB) {
    Geom g{};
    if (scheme == KVQ_SCHEME_WITCERT) {
        g.kc = 0; g.kh = 0; g.ks = 32768; g.vc = 33024; g.vs = 65792; g.bytes = 66048;
        g.tokens = WPT;
    } else if (is_kitty(scheme)) {
        g.kc = 0; g.kh = 2048; g.ks = 2048 + 16 * nb; g.vc = g.ks + 1024; g.vs = g.vc + 2048;
        g.bytes = g.vs + 1024;
        if (scheme == KVQ_SCHEME_KITTY_DYN) {
            g.ki = g.bytes;
            g.bytes += nb > 16 ? nb : 16;
        }
        g.tokens = PT;
    } else if (scheme == KVQ_SCHEME_WITCERT_PAGED) {
        // nb = bypassed RoPE pairs; KH holds the fp16 bypass row of each token
        g.kc = 0; g.vc = 8192; g.ks = 16384; g.vs = 16896; g.kh = 17408;
        g.bytes = 17408 + (nb > 0 ? 1024 : 0);
        g.tokens = PT;
    } else if (scheme == KVQ_SCHEME_KIVI4) {
        g.kc = 0; g.kh = 0; g.ks = 4096; g.vc = 5120; g.vs = 9216; g.bytes = 10240;
        g.tokens = PT;
    } else {
        g.kc = 0; g.kh = 0; g.ks = 2048; g.vc = 3072; g.vs = 5120; g.bytes = 6144;
        g.tokens = PT;
    }
    return g;
}

// Key code of (token t in page, channel c): dword index into KC and bit shift.
// Lane L = 16*((c>>3)&3) + (t&15) of a wave loads dwords {256*p + 4*L + i},
// i.e. 16 contiguous bytes per lane per 1 KB; dword d = 4p + i holds the 16
// codes of token 16*(d>>1) + (t&15), channels 32*kc + 8*((c>>3)&3) + j with
// kc = 2*(d&1) + h, at bit 4j + 2h.  Masking with 0x33333333 (h = 0) or
// (x >> 2) & 0x33333333 (h = 1) leaves eight codes in nibble j, ready for the
// packed fp4 -> f16 / f32 converters.
__host__ __device__ inline void key_code_pos(int t, int c, int &dword, int &shift) {
    int n = t >> 4, r = t & 15, kc = c >> 5, g = (c >> 3) & 3, j = c & 7;
    int lane = 16 * g + r;
    int d = 2 * n + (kc >> 1), h = kc & 1;
    dword = (d >> 2) * 256 + lane * 4 + (d & 3);
    shift = 4 * j + 2 * h;
}

// Value code of (token t in page, channel c).  Lane L = 16*((t>>3)&3) + (c&15)
// holds dword d = c >> 4 (channel 16d + (c&15)) with the 16 codes of tokens
// 32*ks + 8*((t>>3)&3) + j at bit 4j + 2ks.
__host__ __device__ inline void value_code_pos(int t, int c, int &dword, int &shift) {
    int nt = c >> 4, r = c & 15, ks = t >> 5, g = (t >> 3) & 3, j = t & 7;
    int lane = 16 * g + r;
    dword = (nt >> 2) * 256 + lane * 4 + (nt & 3);
    shift = 4 * j + 2 * ks;
}

// KIVI4 codes, eight to a dword: the dword's code k (k = 0..7) sits in byte
// k & 3 at nibble k >> 2, so the dword masked with 0x0F0F0F0F holds codes
// 0..3 one per byte and (x >> 4) & 0x0F0F0F0F codes 4..7.  A byte holding
// b < 16 reads as the e4m3 number b / 512 (subnormal for b < 8, exponent 1
// above), so the packed fp8 -> f16 converter with scale 512 yields the codes
// exactly, in k order.
// Keys: lane L = 16*((c>>3)&3) + (t&15) loads dwords {256*p + 4*L + i},
// p = t >> 4 (token tile), i = c >> 5; code k = c & 7.
__host__ __device__ inline void key_code_pos4(int t, int c, int &dword, int &shift) {
    int n = t >> 4, r = t & 15, kc = c >> 5, g = (c >> 3) & 3, k = c & 7;
    dword = 256 * n + 4 * (16 * g + r) + kc;
    shift = 8 * (k & 3) + 4 * (k >> 2);
}

// Values: lane L = 16*((t>>3)&3) + (c&15) holds dword d = 8*(t>>5) + (c>>4)
// at 256*(d>>2) + 4*L + (d&3); code k = t & 7.
__host__ __device__ inline void value_code_pos4(int t, int c, int &dword, int &shift) {
    int nt = c >> 4, r = c & 15, ks = t >> 5, g = (t >> 3) & 3, k = t & 7;
    int d = 8 * ks + nt;
    dword = 256 * (d >> 2) + 4 * (16 * g + r) + (d & 3);
    shift = 8 * (k & 3) + 4 * (k >> 2);
}

// Kitty high plane: (token t in page, boosted offset o in [0, nb)).  Plane
// q = o >> 4 holds offsets 16q .. 16q+15 in 64 dwords: dword
// 64q + 16*((o&15)>>2) + (t&15) (the lane whose KC data holds token t), bit
// 4*(4*(n&1) + (o&3)) + 2*(n>>1) with n = t >> 4.
__host__ __device__ inline void high_code_pos(int t, int o, int &dword, int &shift) {
    int n = t >> 4, r = t & 15, q = o >> 4, g = (o & 15) >> 2, i = o & 3;
    dword = 64 * q + 16 * g + r;
    shift = 4 * (4 * (n & 1) + i) + 2 * (n >> 1);
}

// Key statistic slot of channel c inside a group (channel order).
__host__ __device__ inline int key_stat_slot(int c) {
    return c;
}

// ---------------------------------------------------------------------------
// binary16 helpers (bit patterns in uint16_t)
// ---------------------------------------------------------------------------
__device__ inline float h2f(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ inline uint16_t f2h(float x) {          // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// ---------------------------------------------------------------------------
// Asymmetric RTN group quantizer ("Kitty" summary, Observation 1 and the
// quantization step: x_q = round((x - z)/s) clamped to [0, 2^b-1]):
//   z = min (canonical +0), s = fp16(fl32(fl32(max - min)/(2^b - 1))),
//   s raised one fp16 step when (2^b - 1/2) s < max - min (fp16-subnormal s
//   only), s = 0 for a constant group; code = clamp(rint(fl32(x - z)/s)).
// Every operation is a single IEEE binary32 operation (no contraction).
// ---------------------------------------------------------------------------
struct AsymParams {
    float s, z;
    uint16_t s16, z16;
};

__device__ inline AsymParams asym_params(float mn, float mx, float lmax) {
#pragma clang fp contract(off)
    AsymParams p;
    p.z = mn + 0.0f;
    float d = mx - mn;
    uint16_t s16 = 0;
    if (d > 0.0f) {
        s16 = f2h(d / lmax);
        if ((lmax + 0.5f) * h2f(s16) < d) s16 = (uint16_t)(s16 + 1);
    }
    p.s16 = s16;
    p.s = h2f(s16);
    p.z16 = f2h(p.z);
    return p;
}

__device__ inline uint32_t asym_code(float x, const AsymParams &p, float lmax) {
#pragma clang fp contract(off)
    if (p.s16 == 0) return 0u;
    float t = x - p.z;
    float c = rintf(t / p.s);
    c = fminf(fmaxf(c, 0.0f), lmax);
    return (uint32_t)c;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11) and the WitCert dither
// (counter = (token, channel>>2, layer<<16 | kv_head, request),
//  key = (seed_lo, seed_hi ^ side), word = channel & 3,
//  xi = fl32((u >> 8) * 2^-24) - 1/2).
// ---------------------------------------------------------------------------
struct U4 {
    uint32_t x, y, z, w;
};

// 32 x 32 -> 64-bit product in one multiply-add instruction (both halves at
// once: about a quarter faster per round than separate high and low
// multiplies, with identical results)
__device__ inline uint64_t mul_wide(uint32_t m, uint32_t x) {
    uint64_t r;
    asm("v_mad_u64_u32 %0, vcc, %1, %2, 0" : "=v"(r) : "v"(x), "s"(m) : "vcc");
    return r;
}

// a ^ b ^ k in one three-input bitwise instruction (truth table 0x96, the
// same for any order of the inputs); k is uniform across the wave
__device__ inline uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
    uint32_t d;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(d) : "v"(a), "v"(b), "s"(k));
    return d;
}

__device__ inline U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; r++) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = mul_wide(0xD2511F53u, c.x);
        const uint64_t p1 = mul_wide(0xCD9E8D57u, c.z);
        const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
        const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
        U4 n;
        n.x = xor3(hi1, c.y, k0);
        n.y = lo1;
        n.z = xor3(hi0, c.w, k1);
        n.w = lo0;
        c = n;
    }
    return c;
}

__device__ inline float dither_from_word(uint32_t u) {
#pragma clang fp contract(off)
    return (float)(u >> 8) * 0x1p-24f - 0.5f;
}

// ---------------------------------------------------------------------------
// wave64 cross-lane helpers
// ---------------------------------------------------------------------------
__device__ inline float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

}  // namespace kvq
