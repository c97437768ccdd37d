/*
 * kvq_oracle.c -- plain, slow CPU oracle for low-bit KV-cache quantization
 * and single-query decode attention over the dequantized cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and
 * the benchmark's cpu_baseline leg may load this file's library.  It shares
 * no code, header, table or helper with the HIP library and includes none of
 * its files; the two are compared, never combined.
 *
 * Build: gcc -std=c11 -O2 -fPIC -shared -ffp-contract=off -fno-fast-math
 * (x86-64 SSE float: every float operation below is one IEEE-754 binary32
 * operation rounded to nearest-even, no fused multiply-add, no flush-to-zero).
 *
 * Sources followed (page title; section):
 *   [KIVI]  "KIVI: key per-channel / value per-token tuning-free asymmetric
 *           2bit KV cache quantization" explainer; sections 3.1-3.3 (RTN
 *           quantizer, per-channel keys, per-token values, grouped cache plus
 *           full-precision residual, concatenated attention eq. 3) and
 *           section 4 (data path steps 2-5).
 *   [KITTY] "Kitty" summary; "Observation 1" (uniform affine quantizer and
 *           the [0,10] -> 10/3 step example), "The Channel-Wise Precision
 *           Boost Mechanism" (top-K selection, mixed INT4/INT2 quantization
 *           step), "Page-Centric Memory Layout and Dense-Sparse
 *           Decomposition" (low/high planes, boost index with sentinel),
 *           "GPU Dequantization Kernel (Algorithm 1)" (X = low | high << 2),
 *           "Lightweight Attention Execution Pipeline" (stage order).
 *   [WITCERT] "WitCert: Sound Runtime Risk Observability and Gating for
 *           KV-Cache Quantization"; write-kernel paragraph (subtractive
 *           dither, s = amax/126.5 stored fp16 and reused, Philox4x32-10
 *           five-tuple), "Key structure" paragraph (certificate A and the
 *           split LSE merge), the quantised-path certificate paragraph
 *           (varsigma^2 formula), and the certified-deployment paragraphs
 *           (per-token scales over groups of G_c channels, the slot-keyed
 *           Philox tuple, the fixed outlier RoPE-pair bypass left out of
 *           the group amax).
 *   Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
 *           as easy as 1, 2, 3" (SC'11), the reference WitCert cites for
 *           its dither generator.
 *
 * Where the pages are silent, the reading taken is stated at the function
 * that takes it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* binary16 <-> binary32, written from the IEEE-754 encoding definition.    */
/* ------------------------------------------------------------------------ */

float ko_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);              /* zero / subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(m | 0x400), e - 25); /* (1024 + m) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* Round-to-nearest-even conversion.  The value is handled in double, where a
 * binary32 input and every scaling by a power of two below are exact, and
 * rint() (default rounding mode) supplies the ties-to-even step. */
uint16_t ko_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    double v = fabs((double)f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7e00u);
    if (v < ldexp(1.0, -14)) {                   /* subnormal range */
        double m = rint(v * ldexp(1.0, 24));     /* units of 2^-24 */
        return (uint16_t)(sign | (uint16_t)m);   /* m == 1024 encodes 2^-14 */
    }
    int e2;
    (void)frexp(v, &e2);                         /* v = f * 2^e2, f in [0.5,1) */
    int e = e2 - 1;                              /* v in [2^e, 2^(e+1)) */
    double m = rint(v * ldexp(1.0, 10 - e));     /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e > 15)
        return (uint16_t)(sign | 0x7c00u);       /* overflow -> inf */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

/* ------------------------------------------------------------------------ */
/* Asymmetric uniform (round-to-nearest) group quantizer.                   */
/* [KITTY] Observation 1: x_q = round((x - z)/s); [KITTY] quantization step: */
/* clamp to [0, 2^b - 1]; Algorithm 1: x_hat = X * scale + zero_point.      */
/* [KIVI] 3.1: RTN with a per-group zero point and scale.                    */
/* Readings (pages silent or garbled):                                       */
/*   z = group minimum (canonical +0 for a zero minimum), stored fp16;       */
/*   s = fp16_rne( fl32( fl32(max - min) / (2^b - 1) ) ), the min-max range  */
/*       split into 2^b - 1 steps ([KITTY] [0,10] -> 10/3 example);          */
/*   guard: if (2^b - 1/2) * s < max - min, s is raised to the next fp16     */
/*       value (only reachable for fp16-subnormal s);                        */
/*   constant group: s = 0 and every code is 0;                              */
/*   code = clamp(rint(fl32(fl32(x - z) / s)), 0, 2^b - 1), rint = nearest   */
/*       with ties to even.                                                  */
/* ------------------------------------------------------------------------ */

void ko_quant_asym(const uint16_t *x, long n, long stride, int bits,
                   uint16_t *s_out, uint16_t *z_out,
                   uint8_t *codes, long code_stride)
{
    const float lmax = (float)((1 << bits) - 1);
    float mn = ko_f16_to_f32(x[0]);
    float mx = mn;
    for (long i = 1; i < n; i++) {
        float v = ko_f16_to_f32(x[i * stride]);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    float z = mn + 0.0f;                 /* -0 + 0 = +0 under round-to-nearest */
    float d = mx - mn;
    uint16_t s16 = 0;
    if (d > 0.0f) {
        s16 = ko_f32_to_f16(d / lmax);
        if ((lmax + 0.5f) * ko_f16_to_f32(s16) < d)
            s16 = (uint16_t)(s16 + 1);   /* next larger positive fp16 */
    }
    float s = ko_f16_to_f32(s16);
    for (long i = 0; i < n; i++) {
        float v = ko_f16_to_f32(x[i * stride]);
        float c = 0.0f;
        if (s16 != 0) {
            float t = v - z;
            c = rintf(t / s);
            if (c < 0.0f) c = 0.0f;
            if (c > lmax) c = lmax;
        }
        codes[i * code_stride] = (uint8_t)c;
    }
    *s_out = s16;
    *z_out = ko_f32_to_f16(z);
}

/* x_hat = code * s + z in binary32; code * s is exact (<= 4 + 11 bits). */
float ko_dequant_asym(int code, uint16_t s16, uint16_t z16)
{
    float cs = (float)code * ko_f16_to_f32(s16);
    return cs + ko_f16_to_f32(z16);
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11): ten rounds of the 4x32 S-box with   */
/* multipliers 0xD2511F53, 0xCD9E8D57 and Weyl key increments 0x9E3779B9,    */
/* 0xBB67AE85; round r uses key + r * increment.                            */
/* ------------------------------------------------------------------------ */

void ko_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; r++) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* WitCert dither for one element.  [WITCERT] write kernel: xi from
 * Philox4x32-10 keyed by the five-tuple (request, layer, KV head, token,
 * channel), reconstructed exactly at read.  Readings:
 *   counter = (token, channel >> 2, (layer << 16) | kv_head, request),
 *   key     = (seed_lo, seed_hi ^ side), side 0 = keys, 1 = values,
 *   word    = channel & 3 (all four outputs of one call are used),
 *   xi      = fl32((u >> 8) * 2^-24) - 0.5, uniform on [-1/2, 1/2). */
float ko_dither(uint64_t seed, int side, uint32_t req, uint32_t layer,
                uint32_t kvh, uint32_t token, uint32_t ch)
{
    uint32_t ctr[4] = { token, ch >> 2, (layer << 16) | kvh, req };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) ^ (uint32_t)side };
    uint32_t out[4];
    ko_philox4x32_10(ctr, key, out);
    uint32_t u = out[ch & 3];
    return (float)(u >> 8) * 0x1p-24f - 0.5f;
}

/* Paging-safe WitCert dither ([WITCERT] certified deployment: the counter
 * is keyed by the cache slot, which paging, prefix sharing and retraction
 * never change, instead of the sequence position).  Reading: the tuple
 * (layer, KV head, slot, channel) fills the same counter words, the slot's
 * low and high halves taking the places of token and request:
 *   counter = (slot_lo, channel >> 2, (layer << 16) | kv_head, slot_hi),
 * key, output word and xi as in ko_dither. */
float ko_dither_slot(uint64_t seed, int side, uint32_t layer, uint32_t kvh,
                     uint64_t slot, uint32_t ch)
{
    uint32_t ctr[4] = { (uint32_t)slot, ch >> 2, (layer << 16) | kvh, (uint32_t)(slot >> 32) };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) ^ (uint32_t)side };
    uint32_t out[4];
    ko_philox4x32_10(ctr, key, out);
    uint32_t u = out[ch & 3];
    return (float)(u >> 8) * 0x1p-24f - 0.5f;
}

/* ------------------------------------------------------------------------ */
/* WitCert INT8 subtractive-dither block quantizer for one channel of one   */
/* block of n tokens.  [WITCERT] write kernel: x_hat = s (round(x/s + xi)  */
/* - xi), s = amax_blk / 126.5 stored fp16 and used for quantization.       */
/* Readings: guard raises s to the next fp16 if 127 s <= amax (only for     */
/* coarse fp16-subnormal s); amax = 0 gives s = 0 and codes 0;              */
/* code = clamp(rint(fl32(fl32(x / s) + xi)), -127, 127).                   */
/* ------------------------------------------------------------------------ */

void ko_witcert_quant(const uint16_t *x, long n, long stride, const float *xi,
                      uint16_t *s_out, int8_t *codes, long code_stride)
{
    float amax = 0.0f;
    for (long i = 0; i < n; i++) {
        float a = fabsf(ko_f16_to_f32(x[i * stride]));
        if (a > amax) amax = a;
    }
    uint16_t s16 = 0;
    if (amax > 0.0f) {
        s16 = ko_f32_to_f16(amax / 126.5f);
        if (127.0f * ko_f16_to_f32(s16) <= amax)
            s16 = (uint16_t)(s16 + 1);
    }
    float s = ko_f16_to_f32(s16);
    for (long i = 0; i < n; i++) {
        float c = 0.0f;
        if (s16 != 0) {
            float v = ko_f16_to_f32(x[i * stride]);
            float t = v / s;
            c = rintf(t + xi[i]);
            if (c < -127.0f) c = -127.0f;
            if (c > 127.0f) c = 127.0f;
        }
        codes[i * code_stride] = (int8_t)c;
    }
    *s_out = s16;
}

/* x_hat = s * (code - xi), both operations binary32 (reading: this order). */
float ko_witcert_dequant(int code, uint16_t s16, float xi)
{
    float t = (float)code - xi;
    return ko_f16_to_f32(s16) * t;
}

/* ------------------------------------------------------------------------ */
/* Outlier RoPE-pair selection for the paging-safe WitCert storage.         */
/* [WITCERT] certified deployment: a fixed set of m RoPE pairs per (layer,  */
/* KV head), chosen from the leading part of a sequence, is stored fp16.    */
/* Readings: pair i is channels (i, i + D/2) (the rotate-half RoPE layout); */
/* its importance is max over the calibration tokens of x_i^2 + x_{i+D/2}^2 */
/* (the pair's squared norm, which the rotation keeps), each square exact   */
/* in binary32 and the sum rounded once; the m largest are taken, ties to   */
/* the lower pair.  mask[c] = 1 for both channels of a chosen pair.         */
/* ------------------------------------------------------------------------ */

void ko_witcert_select_pairs(const uint16_t *k, long T, int D, int m, uint8_t *mask)
{
    int H = D / 2;
    float imp[128];
    for (int i = 0; i < H; i++) {
        imp[i] = 0.0f;
        for (long t = 0; t < T; t++) {
            float a = ko_f16_to_f32(k[t * D + i]);
            float b = ko_f16_to_f32(k[t * D + i + H]);
            float e = a * a + b * b;
            if (e > imp[i]) imp[i] = e;
        }
    }
    for (int c = 0; c < D; c++) mask[c] = 0;
    for (int r = 0; r < m && r < H; r++) {
        int best = -1;
        for (int i = 0; i < H; i++) {
            if (mask[i]) continue;
            if (best < 0 || imp[i] > imp[best]) best = i;
        }
        mask[best] = 1;
        mask[best + H] = 1;
    }
}

/* ------------------------------------------------------------------------ */
/* Kitty static boost selection.  [KITTY] "Selecting the Top-K Channels":    */
/* the K = alpha * D channels with the highest importance are boosted;       */
/* "The Boost Index Tensor": boosted channel -> offset into the high plane, */
/* others -> sentinel D_boosted + 1.  Readings: importance = max |x| over a */
/* calibration slice (static per head); ties go to the lower channel index; */
/* offsets follow ascending channel order.                                  */
/* ------------------------------------------------------------------------ */

void ko_kitty_select(const uint16_t *k, long T, int D, int nb, uint8_t *idx)
{
    float *amax = (float *)calloc((size_t)D, sizeof(float));
    char *chosen = (char *)calloc((size_t)D, 1);
    for (long t = 0; t < T; t++)
        for (int c = 0; c < D; c++) {
            float a = fabsf(ko_f16_to_f32(k[t * D + c]));
            if (a > amax[c]) amax[c] = a;
        }
    for (int j = 0; j < nb; j++) {
        int best = -1;
        for (int c = 0; c < D; c++)
            if (!chosen[c] && (best < 0 || amax[c] > amax[best]))
                best = c;
        chosen[best] = 1;
    }
    int off = 0;
    for (int c = 0; c < D; c++)
        idx[c] = chosen[c] ? (uint8_t)(off++) : (uint8_t)(nb + 1);
    free(amax);
    free(chosen);
}

/* ------------------------------------------------------------------------ */
/* Kitty dynamic boost selection for one selection unit of T tokens.        */
/* [KITTY] "Channel-Wise Precision Boost Mechanism": the importance of a    */
/* channel within a group is its mean absolute value, and the top K of the  */
/* group are boosted.  Readings: the unit is one 64-token page of the cache */
/* (the pages' groups are their own pages); the mean is compared through    */
/* the exact sum sum_t |x_{t,c}| (T is fixed, and binary16 values add       */
/* exactly in binary64 at these sizes); ties go to the lower channel;       */
/* offsets follow ascending channel order, others get the sentinel nb + 1. */
/* ------------------------------------------------------------------------ */

void ko_kitty_select_dyn(const uint16_t *k, long T, long ld, int D, int nb, uint8_t *idx)
{
    double *imp = (double *)calloc((size_t)D, sizeof(double));
    char *chosen = (char *)calloc((size_t)D, 1);
    for (long t = 0; t < T; t++)
        for (int c = 0; c < D; c++)
            imp[c] += fabs((double)ko_f16_to_f32(k[t * ld + c]));
    for (int j = 0; j < nb; j++) {
        int best = -1;
        for (int c = 0; c < D; c++)
            if (!chosen[c] && (best < 0 || imp[c] > imp[best]))
                best = c;
        chosen[best] = 1;
    }
    int off = 0;
    for (int c = 0; c < D; c++)
        idx[c] = chosen[c] ? (uint8_t)(off++) : (uint8_t)(nb + 1);
    free(imp);
    free(chosen);
}

/* ------------------------------------------------------------------------ */
/* One (request, KV head) stream: the raw fp16 history plus the quantized   */
/* record, advanced by the same three calls as the library:                 */
/*   flush  -> append -> decode   (the Kitty pipeline order: attention runs  */
/*   on the fp16 group, quantization happens once G tokens have gathered;   */
/*   here expressed as "flush at the start of the next step").              */
/* Keeping the raw history is equivalent to keeping the residual buffers:   */
/* a token's fp16 value is read only while it is inside a residual window. */
/* ------------------------------------------------------------------------ */

/* KO_KIVI4: the KIVI scheme at 4 bits for keys and values ([KIVI] reports
 * its quantizer at 2 and 4 bits; the same groups, statistics and windows). */
/* KO_WITCERT_TOK: the paging-safe WitCert storage ([WITCERT] certified
 * deployment): every token is quantized when it is written, keys and values
 * alike, with one scale per (token, group of VG channels), the dither keyed
 * by the token's cache slot, and a fixed set of key channels (outlier RoPE
 * pairs) kept fp16 and left out of their group's amax. */
enum { KO_KIVI = 0, KO_KITTY = 1, KO_WITCERT = 2, KO_KITTY_DYN = 3, KO_KIVI4 = 4,
       KO_WITCERT_TOK = 5 };

typedef struct ko_stream {
    int scheme, D, G, R, VG, BLK, nb, bits_v;
    long cap;
    long l;       /* tokens appended */
    long n_kq;    /* keys [0, n_kq) quantized (KIVI/Kitty); blocks for WitCert */
    long n_vq;    /* values [0, n_vq) quantized */
    uint16_t *Kraw, *Vraw;   /* [cap][D] */
    uint8_t *Kc;             /* [cap][D] key codes (WitCert: int8 bit pattern) */
    uint8_t *Vc;             /* [cap][D] */
    uint16_t *Ks, *Kz;       /* KIVI/Kitty: [cap/G][D];  WitCert Ks: [cap/BLK][D] */
    uint16_t *Vs, *Vz;       /* KIVI/Kitty: [cap][D/VG]; WitCert Vs: [cap/BLK][D] */
    uint8_t idx[256];        /* Kitty boost index per channel (static) */
    long sel;                /* Kitty dynamic: tokens per selection unit */
    long sink;               /* leading tokens kept fp16 for keys and values */
    uint8_t *uidx;           /* Kitty dynamic: [cap/sel + 1][D] boost index per unit */
    uint64_t *slot;          /* KO_WITCERT_TOK: cache slot of each token [cap] */
    uint8_t byp[256];        /* KO_WITCERT_TOK: 1 = key channel stored fp16 */
    uint64_t seed;
    uint32_t req, layer, kvh;
} ko_stream;

/* sel: tokens per selection unit for KO_KITTY_DYN (a multiple of G that
 * divides R, so a flush always quantizes whole units); ignored otherwise.
 * KO_WITCERT_TOK: idx[c] != 0 marks a bypassed key channel (NULL: none);
 * VG is the scale group; token t sits in slot t until ko_stream_set_slots.
 * sink: the first `sink` tokens of the stream stay fp16, keys and values
 * ([KITTY] sink tokens; KIVI2 / Kitty only); groups, selection units and the
 * value FIFO then start at token `sink`. */
ko_stream *ko_stream_new(int scheme, int D, int G, int R, int VG, int BLK,
                         int nb, const uint8_t *idx, long cap,
                         uint64_t seed, uint32_t req, uint32_t layer, uint32_t kvh, long sel,
                         long sink)
{
    if (sink < 0 || (sink > 0 && (scheme == KO_WITCERT || scheme == KO_WITCERT_TOK))) return NULL;
    if (D <= 0 || D > 256 || cap <= 0) return NULL;
    if (scheme < KO_KIVI || scheme > KO_WITCERT_TOK) return NULL;
    if (scheme == KO_WITCERT_TOK) {
        if (VG <= 0 || D % VG != 0) return NULL;
    } else if (scheme != KO_WITCERT) {
        if (G <= 0 || R <= 0 || R % G != 0 || VG <= 0 || D % VG != 0) return NULL;
        if (nb < 0 || nb > D) return NULL;
    } else if (BLK <= 0) {
        return NULL;
    }
    if (scheme == KO_KITTY_DYN && (sel <= 0 || sel % G != 0 || R % sel != 0)) return NULL;
    ko_stream *s = (ko_stream *)calloc(1, sizeof(ko_stream));
    s->scheme = scheme; s->D = D; s->G = G; s->R = R; s->VG = VG; s->BLK = BLK;
    s->nb = (scheme == KO_KITTY || scheme == KO_KITTY_DYN) ? nb : 0;
    s->bits_v = (scheme == KO_KIVI4) ? 4 : 2;
    if (scheme == KO_KITTY_DYN) {
        s->sel = sel;
        s->uidx = (uint8_t *)calloc((size_t)((cap / sel + 1) * D), 1);
    }
    s->cap = cap;
    s->sink = sink;
    s->seed = seed; s->req = req; s->layer = layer; s->kvh = kvh;
    s->Kraw = (uint16_t *)calloc((size_t)(cap * D), 2);
    s->Vraw = (uint16_t *)calloc((size_t)(cap * D), 2);
    s->Kc = (uint8_t *)calloc((size_t)(cap * D), 1);
    s->Vc = (uint8_t *)calloc((size_t)(cap * D), 1);
    long ngk = (scheme == KO_WITCERT) ? cap / BLK + 1 : cap / G + 1;
    if (scheme == KO_WITCERT_TOK) ngk = cap * (D / VG) / D + 1;
    s->Ks = (uint16_t *)calloc((size_t)(ngk * D), 2);
    s->Kz = (uint16_t *)calloc((size_t)(ngk * D), 2);
    long nvs = (scheme == KO_WITCERT) ? (cap / BLK + 1) * D : cap * (D / VG);
    if (scheme == KO_WITCERT_TOK) {
        s->slot = (uint64_t *)calloc((size_t)cap, sizeof(uint64_t));
        for (long t = 0; t < cap; t++) s->slot[t] = (uint64_t)t;
        for (int c = 0; c < D; c++) s->byp[c] = (idx && idx[c]) ? 1 : 0;
    }
    s->Vs = (uint16_t *)calloc((size_t)nvs, 2);
    s->Vz = (uint16_t *)calloc((size_t)nvs, 2);
    for (int c = 0; c < D; c++)
        s->idx[c] = (s->nb > 0 && idx) ? idx[c] : (uint8_t)(s->nb + 1);
    return s;
}

/* KO_WITCERT_TOK: cache slot of every token (cap values), before any token
 * is written.  Returns 0, or -1 for another scheme or a stream in use. */
int ko_stream_set_slots(ko_stream *s, const uint64_t *slots)
{
    if (s->scheme != KO_WITCERT_TOK || s->l != 0) return -1;
    memcpy(s->slot, slots, sizeof(uint64_t) * (size_t)s->cap);
    return 0;
}

void ko_stream_free(ko_stream *s)
{
    if (!s) return;
    free(s->Kraw); free(s->Vraw); free(s->Kc); free(s->Vc);
    free(s->Ks); free(s->Kz); free(s->Vs); free(s->Vz);
    free(s->uidx); free(s->slot);
    free(s);
}

/* Key groups and selection units count from token `sink`: group g holds
 * tokens [sink + gG, sink + (g+1)G). */

/* Boost index of key group g, channel c: the head's static index, or the
 * index of the selection unit holding the group. */
static int boost_off(const ko_stream *s, long g, int c)
{
    if (s->scheme == KO_KITTY) return s->idx[c];
    if (s->scheme == KO_KITTY_DYN) return s->uidx[(g * s->G / s->sel) * s->D + c];
    return s->nb + 1;
}

static int key_bits(const ko_stream *s, long g, int c)
{
    if (s->scheme == KO_KIVI4) return 4;
    return boost_off(s, g, c) < s->nb ? 4 : 2;
}

/* [KIVI] 3.3: keys gather in the residual; once R have gathered they are
 * quantized per channel in R/G groups of G tokens and the residual clears.
 * Kitty dynamic: the first group of a selection unit selects the unit's
 * boosted channels from the unit's raw keys (all present: units divide R). */
static void quant_key_group(ko_stream *s, long g)
{
    long t0 = s->sink + g * s->G;
    if (s->scheme == KO_KITTY_DYN && (g * s->G) % s->sel == 0) {
        long u = g * s->G / s->sel;
        ko_kitty_select_dyn(&s->Kraw[(s->sink + u * s->sel) * s->D], s->sel, s->D, s->D, s->nb,
                            &s->uidx[u * s->D]);
    }
    for (int c = 0; c < s->D; c++)
        ko_quant_asym(&s->Kraw[t0 * s->D + c], s->G, s->D, key_bits(s, g, c),
                      &s->Ks[g * s->D + c], &s->Kz[g * s->D + c],
                      &s->Kc[t0 * s->D + c], s->D);
}

/* [KIVI] 3.3: values leave the R-token FIFO one at a time, each quantized per
 * token in groups of VG consecutive channels. */
static void quant_value_token(ko_stream *s, long t)
{
    int ng = s->D / s->VG;
    for (int j = 0; j < ng; j++)
        ko_quant_asym(&s->Vraw[t * s->D + j * s->VG], s->VG, 1, s->bits_v,
                      &s->Vs[t * ng + j], &s->Vz[t * ng + j],
                      &s->Vc[t * s->D + j * s->VG], 1);
}

/* [WITCERT]: a completed block of BLK tokens is quantized channel by channel
 * (one scale per 256-token block and channel), keys and values alike. */
static void quant_witcert_block(ko_stream *s, long b)
{
    float *xi = (float *)malloc(sizeof(float) * (size_t)s->BLK);
    for (int side = 0; side < 2; side++) {
        uint16_t *raw = side ? s->Vraw : s->Kraw;
        uint8_t *codes = side ? s->Vc : s->Kc;
        uint16_t *sc = side ? s->Vs : s->Ks;
        for (int c = 0; c < s->D; c++) {
            for (int i = 0; i < s->BLK; i++)
                xi[i] = ko_dither(s->seed, side, s->req, s->layer, s->kvh,
                                  (uint32_t)(b * s->BLK + i), (uint32_t)c);
            ko_witcert_quant(&raw[b * s->BLK * s->D + c], s->BLK, s->D, xi,
                             &sc[b * s->D + c],
                             (int8_t *)&codes[b * s->BLK * s->D + c], s->D);
        }
    }
    free(xi);
}

/* KO_WITCERT_TOK: token t is quantized as it is written, per group of VG
 * channels on each side ([WITCERT] certified deployment: the scale depends
 * on the current token only).  Each group is the block quantizer above over
 * its non-bypassed channels (bypassed key channels are left out of the amax
 * and get code 0; they are read back fp16), with the dither of the token's
 * slot. */
static void quant_witcert_token(ko_stream *s, long t)
{
    int ng = s->D / s->VG;
    uint16_t x[256];
    float xi[256];
    int8_t cd[256];
    int ch[256];
    for (int side = 0; side < 2; side++) {
        const uint16_t *raw = (side ? s->Vraw : s->Kraw) + t * s->D;
        uint8_t *codes = (side ? s->Vc : s->Kc) + t * s->D;
        uint16_t *sc = (side ? s->Vs : s->Ks) + t * ng;
        for (int g = 0; g < ng; g++) {
            int n = 0;
            for (int c = g * s->VG; c < (g + 1) * s->VG; c++) {
                codes[c] = 0;
                if (side == 0 && s->byp[c]) continue;
                ch[n] = c;
                x[n] = raw[c];
                xi[n] = ko_dither_slot(s->seed, side, s->layer, s->kvh, s->slot[t], (uint32_t)c);
                n++;
            }
            uint16_t s16 = 0;
            if (n > 0) ko_witcert_quant(x, n, 1, xi, &s16, cd, 1);
            for (int i = 0; i < n; i++) codes[ch[i]] = (uint8_t)cd[i];
            sc[g] = s16;
        }
    }
}

/* Flush: KIVI/Kitty quantize the key residual when it holds R tokens;
 * WitCert quantizes the active block when it holds BLK tokens.
 * Returns 1 when something was quantized, 0 otherwise. */
int ko_stream_flush(ko_stream *s)
{
    if (s->scheme == KO_WITCERT_TOK) return 0;      /* nothing waits: tokens are quantized on write */
    if (s->scheme == KO_WITCERT) {
        if (s->l - s->n_kq != s->BLK) return 0;
        quant_witcert_block(s, s->n_kq / s->BLK);
        s->n_kq += s->BLK;
        s->n_vq = s->n_kq;
        return 1;
    }
    if (s->l - s->n_kq != s->R) return 0;
    for (long g = (s->n_kq - s->sink) / s->G; g < (s->n_kq - s->sink + s->R) / s->G; g++)
        quant_key_group(s, g);
    s->n_kq += s->R;
    return 1;
}

/* Append one token.  Returns 0, or -1 when the key residual / active block is
 * already full (the caller skipped the flush) or the capacity is exhausted;
 * the stream is then left unchanged. */
int ko_stream_append(ko_stream *s, const uint16_t *k, const uint16_t *v)
{
    long lim = (s->scheme == KO_WITCERT) ? s->BLK : s->R;
    if (s->scheme != KO_WITCERT_TOK && s->l - s->n_kq >= lim) return -1;
    if (s->l >= s->cap) return -1;
    memcpy(&s->Kraw[s->l * s->D], k, 2 * (size_t)s->D);
    memcpy(&s->Vraw[s->l * s->D], v, 2 * (size_t)s->D);
    if (s->scheme == KO_WITCERT_TOK) {
        quant_witcert_token(s, s->l);
        s->l += 1;
        s->n_kq = s->n_vq = s->l;
        return 0;
    }
    if (s->l < s->sink) {
        /* a sink token: kept fp16, never in the residual or the FIFO */
        s->l += 1;
        s->n_kq = s->n_vq = s->l;
        return 0;
    }
    if (s->scheme != KO_WITCERT && s->l - s->sink >= s->R) {
        /* the FIFO overflows: the oldest value, token l - R, is quantized */
        quant_value_token(s, s->l - s->R);
        s->n_vq = s->l - s->R + 1;
    }
    s->l += 1;
    return 0;
}

/* Bulk state for a context of l0 tokens, equal token for token to streaming
 * the same tokens through flush/append: the key residual holds
 * r_k = ((l0 - 1) mod R) + 1 tokens, values keep the newest min(l0, R).
 * WitCert keeps ((l0 - 1) mod BLK) + 1 tokens in the active block. */
int ko_stream_prefill(ko_stream *s, const uint16_t *K, const uint16_t *V, long l0)
{
    if (l0 < 0 || l0 > s->cap || s->l != 0) return -1;
    memcpy(s->Kraw, K, 2 * (size_t)(l0 * s->D));
    memcpy(s->Vraw, V, 2 * (size_t)(l0 * s->D));
    s->l = l0;
    if (l0 == 0) return 0;
    if (s->scheme == KO_WITCERT_TOK) {
        for (long t = 0; t < l0; t++) quant_witcert_token(s, t);
        s->n_kq = s->n_vq = l0;
        return 0;
    }
    if (s->scheme == KO_WITCERT) {
        long r = ((l0 - 1) % s->BLK) + 1;
        s->n_kq = l0 - r;
        for (long b = 0; b < s->n_kq / s->BLK; b++)
            quant_witcert_block(s, b);
        s->n_vq = s->n_kq;
        return 0;
    }
    if (l0 <= s->sink) {                 /* all sink tokens */
        s->n_kq = s->n_vq = l0;
        return 0;
    }
    long lq = l0 - s->sink;              /* tokens after the sink */
    long rk = ((lq - 1) % s->R) + 1;
    s->n_kq = l0 - rk;
    for (long g = 0; g < (s->n_kq - s->sink) / s->G; g++)
        quant_key_group(s, g);
    s->n_vq = s->sink + (lq > s->R ? lq - s->R : 0);
    for (long t = s->sink; t < s->n_vq; t++)
        quant_value_token(s, t);
    return 0;
}

void ko_stream_state(const ko_stream *s, long *out3)
{
    out3[0] = s->l; out3[1] = s->n_kq; out3[2] = s->n_vq;
}

/* Read-back of the quantized record for parity checks. */
const uint8_t *ko_stream_kcodes(const ko_stream *s) { return s->Kc; }
const uint8_t *ko_stream_vcodes(const ko_stream *s) { return s->Vc; }
const uint16_t *ko_stream_kscale(const ko_stream *s) { return s->Ks; }
const uint16_t *ko_stream_kzero(const ko_stream *s) { return s->Kz; }
const uint16_t *ko_stream_vscale(const ko_stream *s) { return s->Vs; }
const uint16_t *ko_stream_vzero(const ko_stream *s) { return s->Vz; }
const uint8_t *ko_stream_uidx(const ko_stream *s) { return s->uidx; }

/* Dequantized (or raw fp16) key / value of token t, channel c, as binary32.
 * [KIVI] eq. 3: the key is the quantized group for t < n_kq and the fp16
 * residual after; the value is quantized for t < n_vq and fp16 after. */
static float key_tilde(const ko_stream *s, long t, int c)
{
    if (t < s->sink || t >= s->n_kq)
        return ko_f16_to_f32(s->Kraw[t * s->D + c]);
    if (s->scheme == KO_WITCERT_TOK) {
        if (s->byp[c]) return ko_f16_to_f32(s->Kraw[t * s->D + c]);
        float xi = ko_dither_slot(s->seed, 0, s->layer, s->kvh, s->slot[t], (uint32_t)c);
        return ko_witcert_dequant((int8_t)s->Kc[t * s->D + c], s->Ks[t * (s->D / s->VG) + c / s->VG], xi);
    }
    if (s->scheme == KO_WITCERT) {
        long b = t / s->BLK;
        float xi = ko_dither(s->seed, 0, s->req, s->layer, s->kvh, (uint32_t)t, (uint32_t)c);
        return ko_witcert_dequant((int8_t)s->Kc[t * s->D + c], s->Ks[b * s->D + c], xi);
    }
    long g = (t - s->sink) / s->G;
    return ko_dequant_asym(s->Kc[t * s->D + c], s->Ks[g * s->D + c], s->Kz[g * s->D + c]);
}

static float value_tilde(const ko_stream *s, long t, int c)
{
    if (t < s->sink || t >= s->n_vq)
        return ko_f16_to_f32(s->Vraw[t * s->D + c]);
    if (s->scheme == KO_WITCERT_TOK) {
        float xi = ko_dither_slot(s->seed, 1, s->layer, s->kvh, s->slot[t], (uint32_t)c);
        return ko_witcert_dequant((int8_t)s->Vc[t * s->D + c], s->Vs[t * (s->D / s->VG) + c / s->VG], xi);
    }
    if (s->scheme == KO_WITCERT) {
        long b = t / s->BLK;
        float xi = ko_dither(s->seed, 1, s->req, s->layer, s->kvh, (uint32_t)t, (uint32_t)c);
        return ko_witcert_dequant((int8_t)s->Vc[t * s->D + c], s->Vs[b * s->D + c], xi);
    }
    int ng = s->D / s->VG;
    int j = c / s->VG;
    return ko_dequant_asym(s->Vc[t * s->D + c], s->Vs[t * ng + j], s->Vz[t * ng + j]);
}

void ko_stream_dequant(const ko_stream *s, long t0, long t1, float *Kt, float *Vt)
{
    for (long t = t0; t < t1; t++)
        for (int c = 0; c < s->D; c++) {
            if (Kt) Kt[(t - t0) * s->D + c] = key_tilde(s, t, c);
            if (Vt) Vt[(t - t0) * s->D + c] = value_tilde(s, t, c);
        }
}

/* ------------------------------------------------------------------------ */
/* Attention.  [KIVI] eq. 3 / [KITTY] stage 2: scores sm_scale * q . K~_t    */
/* over every token, softmax, output sum_t p_t V~_t.  Everything in binary64 */
/* over the binary32 dequantized operands.                                  */
/* [WITCERT] certificate, computed from its definition:                     */
/*   varsigma^2_{h,b} = (sm_scale^2 / 12) sum_c q_{h,c}^2 s_{c,b}^2 (key     */
/*   scales of block b), u_t = kappa * sqrt(varsigma^2) for quantized keys,  */
/*   u_t = 0 for fp16 keys, A_h = sum_t p_t exp(u_t).                        */
/* KO_WITCERT_TOK: s_{c,t} is the scale of channel c's group at token t, and */
/* 0 for a bypassed (fp16) key channel, which carries no quantization error. */
/* Reading: kappa is a caller-supplied multiplier of the standard deviation. */
/* ------------------------------------------------------------------------ */

/* Partial over tokens [t0, t1): o_part = sum p' V / sum p', lse = m + log
 * sum exp(z - m), a_part = sum p' e^u / sum p' with p' = exp(z - m).
 * (The split form of [WITCERT] "Key structure"; empty range -> lse = -inf.) */
void ko_stream_attend_range(const ko_stream *s, const uint16_t *q, int nq,
                            float sm_scale, float kappa, long t0, long t1,
                            double *o_part, double *lse, double *a_part)
{
    int D = s->D;
    long n = t1 - t0;
    double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *u = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    float *Kt = (float *)malloc(sizeof(float) * (size_t)(D * (n > 0 ? n : 1)));
    float *Vt = (float *)malloc(sizeof(float) * (size_t)(D * (n > 0 ? n : 1)));
    if (n > 0) ko_stream_dequant(s, t0, t1, Kt, Vt);
    for (int h = 0; h < nq; h++) {
        const uint16_t *qh = q + (size_t)h * D;
        double m = -INFINITY;
        for (long i = 0; i < n; i++) {
            double acc = 0.0;
            for (int c = 0; c < D; c++)
                acc += (double)ko_f16_to_f32(qh[c]) * (double)Kt[i * D + c];
            z[i] = (double)sm_scale * acc;
            if (z[i] > m) m = z[i];
            u[i] = 0.0;
            long t = t0 + i;
            if ((s->scheme == KO_WITCERT || s->scheme == KO_WITCERT_TOK) && t < s->n_kq) {
                long b = t / s->BLK;
                double v2 = 0.0;
                for (int c = 0; c < D; c++) {
                    double qc = ko_f16_to_f32(qh[c]);
                    double sc;
                    if (s->scheme == KO_WITCERT)
                        sc = ko_f16_to_f32(s->Ks[b * D + c]);
                    else
                        sc = s->byp[c] ? 0.0 : ko_f16_to_f32(s->Ks[t * (D / s->VG) + c / s->VG]);
                    v2 += qc * qc * sc * sc;
                }
                v2 *= (double)sm_scale * (double)sm_scale / 12.0;
                u[i] = (double)kappa * sqrt(v2);
            }
        }
        double l = 0.0, a = 0.0;
        for (int c = 0; c < D; c++) o_part[(size_t)h * D + c] = 0.0;
        for (long i = 0; i < n; i++) {
            double p = exp(z[i] - m);
            l += p;
            a += p * exp(u[i]);
            for (int c = 0; c < D; c++)
                o_part[(size_t)h * D + c] += p * (double)Vt[i * D + c];
        }
        if (n > 0) {
            for (int c = 0; c < D; c++) o_part[(size_t)h * D + c] /= l;
            lse[h] = m + log(l);
            a_part[h] = a / l;
        } else {
            lse[h] = -INFINITY;
            a_part[h] = 0.0;
        }
    }
    free(z); free(u); free(Kt); free(Vt);
}

/* LSE merge of split partials ([WITCERT] "Key structure"):
 * lse = log sum_s e^{lse_s}; o = sum_s e^{lse_s - lse} o_s; same for A. */
void ko_merge(int nsplit, int nq, int D, const double *o_parts,
              const double *lses, const double *a_parts,
              double *o, double *a)
{
    for (int h = 0; h < nq; h++) {
        double m = -INFINITY;
        for (int sp = 0; sp < nsplit; sp++)
            if (lses[sp * nq + h] > m) m = lses[sp * nq + h];
        double tot = 0.0;
        for (int sp = 0; sp < nsplit; sp++)
            if (lses[sp * nq + h] > -INFINITY) tot += exp(lses[sp * nq + h] - m);
        for (int c = 0; c < D; c++) o[(size_t)h * D + c] = 0.0;
        a[h] = 0.0;
        for (int sp = 0; sp < nsplit; sp++) {
            if (!(lses[sp * nq + h] > -INFINITY)) continue;
            double w = exp(lses[sp * nq + h] - m) / tot;
            for (int c = 0; c < D; c++)
                o[(size_t)h * D + c] += w * o_parts[((size_t)sp * nq + h) * D + c];
            a[h] += w * a_parts[sp * nq + h];
        }
    }
}

/* Whole attention for the current state: one range over [0, l). */
void ko_stream_decode(const ko_stream *s, const uint16_t *q, int nq,
                      float sm_scale, float kappa, double *out, double *cert)
{
    double *lse = (double *)malloc(sizeof(double) * (size_t)nq);
    double *a = (double *)malloc(sizeof(double) * (size_t)nq);
    ko_stream_attend_range(s, q, nq, sm_scale, kappa, 0, s->l, out, lse, a);
    if (cert)
        for (int h = 0; h < nq; h++) cert[h] = a[h];
    free(lse); free(a);
}
