/*
 * oracle.c -- plain, slow CPU oracle for the NVFP4 MoE expert path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library; the HIP path never does.
 * It shares no code, header, table or constant generator with the HIP path.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off (no fast-math): every float
 * operation below is one IEEE fp32 or fp64 operation rounded to nearest even,
 * in the order written.
 *
 * Precision rule. Where a floating-point value decides an integer (a code, a
 * scale byte) the oracle computes it in fp32 with the same operation sequence
 * the method defines, so the decision is taken in the kernel's precision. All
 * other results (GEMMs, SwiGLU, the combine) are computed exactly in int64 or
 * in fp64.
 *
 * Citations name the page by its title and the section the fact comes from:
 *   [AIC] page "Thinking Machines Details End-to-End 4-Bit Training for
 *         Inkling 2 Small" (aicoder.com), sections "Key Takeaways",
 *         "Background", "Architecture highlights".
 *   [T01] page "Thinking Machines 详解 Inkling 2 Small 原生 4-bit 前向训练完整流程"
 *         (news.t0001.com), list "训练数值格式分工清单".
 *   [GDC] page "goldendata.cloud daily brief 2026-11-14", "Signal 02".
 *   [T10] page "AI模型库 · 今日一模 Inkling 2 Small" (10100.com), "01 PART".
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* bf16                                                                      */
/* ------------------------------------------------------------------------- */

float o_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* Nearest bf16 to v (ties to even): bf16 keeps 8 significant bits and fp32's
 * exponent range; below 2^-126 its spacing is 2^-133. */
uint16_t o_f64_to_bf16_rne(double v) {
    double a = fabs(v);
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (a == 0.0) return sign;
    if (isnan(v)) return 0x7FC0u;
    int ex;
    frexp(a, &ex);                               /* a = m * 2^ex, m in [0.5,1) */
    double q = (ex - 1 < -126) ? ldexp(1.0, -133) : ldexp(1.0, ex - 1 - 7);
    double r = nearbyint(a / q) * q;             /* a/q is exact */
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80u;
    float rf = (float)r;                         /* exact: r is a bf16 value */
    return sign | (uint16_t)(f32_bits(rf) >> 16);
}

/* ------------------------------------------------------------------------- */
/* FP4 E2M1, FP8 E4M3, E8M0                                                  */
/* ------------------------------------------------------------------------- */

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is
 * subnormal (m * 0.5). */
float o_e2m1_decode(uint8_t code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? m * 0.5 : ldexp(1.0 + m * 0.5, e - 1);
    return (float)(s ? -mag : mag);
}

/* E4M3 (the "FN" variant): bias 7, no infinities, 0x7F/0xFF are NaN, max 448. */
float o_e4m3_decode(uint8_t b) {
    int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    if ((b & 0x7F) == 0x7F) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -mag : mag);
}

/* E8M0: a bare biased exponent, 2^(b-127); 0xFF is NaN. */
float o_e8m0_decode(uint8_t b) {
    if (b == 0xFF) return NAN;
    return (float)ldexp(1.0, (int)b - 127);
}

/* Round to the E2M1 grid {0,0.5,1,1.5,2,3,4,6}: nearest value, ties to the even
 * code (mantissa bit 0), values past 6 saturate to 6, the sign bit is copied
 * (a negative value that rounds to zero keeps code 0x8). Reading: the pages
 * name no rounding rule for the forward pass; nearest-even is the plain one. */
uint8_t o_e2m1_rne(float y) {
    double a = fabs((double)y);
    if (a >= 6.0) return (uint8_t)(7 | (signbit(y) ? 8 : 0));
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(a - (double)o_e2m1_decode((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(best | (signbit(y) ? 8 : 0));
}

/* Stochastic rounding between the two neighbouring grid values lo <= |y| < hi:
 * round up iff u < f * 2^16 with f = (|y| - lo) / (hi - lo), u a 16-bit draw,
 * so P(up) = ceil(f * 2^16) / 2^16 (unbiased to 2^-16 of a step). Magnitudes at
 * or above the top of the grid saturate without a draw. The pages ask for
 * stochastic rounding to keep gradient bias down [AIC "Key Takeaways"]; the
 * 16-bit comparison rule is a reading. */
uint8_t o_e2m1_sr(float y, uint32_t u16) {
    double a = fabs((double)y);
    uint8_t sign = signbit(y) ? 8 : 0;
    if (a >= 6.0) return sign | 7;
    int lo = 0;
    for (int c = 0; c < 8; ++c)
        if ((double)o_e2m1_decode((uint8_t)c) <= a) lo = c;
    double glo = o_e2m1_decode((uint8_t)lo), ghi = o_e2m1_decode((uint8_t)(lo + 1));
    double f = (a - glo) / (ghi - glo);
    int up = (double)(u16 & 0xFFFFu) < f * 65536.0;
    return (uint8_t)(sign | (lo + up));
}

/* Spacing of the E4M3 grid at magnitude a < 448: 2^(e-3) in binade [2^e,2^e+1)
 * for e >= -6, and 2^-9 among the subnormals below 2^-6. */
static double e4m3_quantum(double a) {
    if (a < 0x1p-6) return 0x1p-9;
    int ex;
    frexp(a, &ex);
    return ldexp(1.0, ex - 1 - 3);
}

/* Byte for an exactly representable non-negative E4M3 magnitude r <= 448:
 * subnormal r = m * 2^-9 gives byte m; normal r = (1 + m/8) * 2^e gives
 * ((e + 7) << 3) | m. */
static uint8_t e4m3_encode_exact(double r) {
    if (r < 0x1p-6) return (uint8_t)(r / 0x1p-9);
    int ex;
    frexp(r, &ex);
    int e = ex - 1;
    int m = (int)((ldexp(r, -e) - 1.0) * 8.0);
    return (uint8_t)(((e + 7) << 3) | m);
}

/* Nearest E4M3 value, ties to even mantissa, finite values past 448 saturate
 * to 448 (reading: saturation, as for the E2M1 codes), sign copied. */
uint8_t o_e4m3_rne_sat(float v) {
    double a = fabs((double)v);
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (a >= 448.0) return sign | 0x7E;
    double q = e4m3_quantum(a);
    double r = nearbyint(a / q) * q; /* even multiple of q <=> even mantissa */
    return sign | e4m3_encode_exact(r);
}

uint8_t o_e4m3_sr(float v, uint32_t u16) {
    double a = fabs((double)v);
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (a >= 448.0) return sign | 0x7E;
    double q = e4m3_quantum(a);
    double lo = floor(a / q) * q;
    double f = (a - lo) / q;
    int up = (double)(u16 & 0xFFFFu) < f * 65536.0;
    return sign | e4m3_encode_exact(lo + (up ? q : 0.0));
}

/* ------------------------------------------------------------------------- */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as    */
/* easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies with the  */
/* paper's multipliers and Weyl key increments.                              */
/* ------------------------------------------------------------------------- */

void o_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Reading: the 16-bit draw for logical element index i of the tensor being
 * rounded comes from counter (lo32(i>>3), hi32(i>>3), stream, 0) under key
 * (lo32(seed), hi32(seed)); word (i>>1)&3, half i&1. Eight draws per call, and
 * a draw depends only on (seed, stream, i), never on layout or launch shape. */
uint32_t o_draw_u16(uint64_t seed, uint32_t stream, uint64_t idx) {
    uint64_t c = idx >> 3;
    uint32_t ctr[4] = {(uint32_t)c, (uint32_t)(c >> 32), stream, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    o_philox4x32_10(ctr, key, out);
    return (out[(idx >> 1) & 3] >> (16 * (idx & 1))) & 0xFFFFu;
}

/* ------------------------------------------------------------------------- */
/* NVFP4 (4.5 bits/value [AIC "Background"]: a 4-bit E2M1 code per value plus  */
/* one E4M3 byte per 16 values, and one FP32 scale per tensor).              */
/* ------------------------------------------------------------------------- */

/* Readings:
 *  - one tensor scale over the whole call; S = 2688/amax encodes (2688 = 6 *
 *    448, the product of the two grids' maxima) and D = amax/2688 is stored as
 *    the decode multiplier, two independent fp32 divisions; S and the per-block
 *    multiplier r are clamped to FLT_MAX;
 *  - block scale byte = nearest-even E4M3 of (amax_block / 6) * S, saturating;
 *  - elements y = x * r with r = S / e4m3(byte) (r = 0 when the byte is 0), then
 *    E2M1 nearest-even or stochastic; an all-zero tensor gets S = D = 1 and all
 *    bytes 0;
 *  - codes are packed two per byte, even element in the low nibble; scales are
 *    row-major, one per 16 consecutive values. */
static float amax_f32(const float* x, int64_t n) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    return amax;
}

/* idx0: element index of x[0] within its tensor (for the stochastic draws). */
static int nvfp4_quantize_given_amax(const float* x, int64_t n, float amax, int64_t idx0, int mode,
                                     uint64_t seed, uint32_t stream, uint8_t* codes, uint8_t* scales,
                                     float* D) {
    if (n < 0 || (n % 16) != 0) return -2;
    if (amax == 0.0f) {
        memset(codes, 0, (size_t)(n / 2));
        memset(scales, 0, (size_t)(n / 16));
        *D = 1.0f;
        return 0;
    }
    float S = 2688.0f / amax;
    if (S > FLT_MAX) S = FLT_MAX;
    *D = amax / 2688.0f;
    for (int64_t b = 0; b < n / 16; ++b) {
        const float* xb = x + 16 * b;
        float amax_b = 0.0f;
        for (int j = 0; j < 16; ++j) {
            float a = fabsf(xb[j]);
            if (a > amax_b) amax_b = a;
        }
        float v = (amax_b / 6.0f) * S;
        uint8_t sc = o_e4m3_rne_sat(v);
        float r = 0.0f;
        if (sc != 0) {
            r = S / o_e4m3_decode(sc);
            if (r > FLT_MAX) r = FLT_MAX;
        }
        scales[b] = sc;
        uint8_t q[16];
        for (int j = 0; j < 16; ++j) {
            float y = xb[j] * r;
            q[j] = (mode == 0) ? o_e2m1_rne(y)
                               : o_e2m1_sr(y, o_draw_u16(seed, stream, (uint64_t)(idx0 + 16 * b + j)));
        }
        for (int j = 0; j < 8; ++j) codes[8 * b + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
    }
    return 0;
}

static int nvfp4_quantize_core(const float* x, int64_t n, int mode, uint64_t seed,
                               uint32_t stream, uint8_t* codes, uint8_t* scales, float* D) {
    if (n < 0 || (n % 16) != 0) return -2;
    return nvfp4_quantize_given_amax(x, n, amax_f32(x, n), 0, mode, seed, stream, codes, scales, D);
}

int oracle_nvfp4_quantize_f32(const float* x, int64_t n, int mode, uint64_t seed,
                              uint32_t stream, uint8_t* codes, uint8_t* scales, float* D) {
    if (!x || !codes || !scales || !D) return -1;
    return nvfp4_quantize_core(x, n, mode, seed, stream, codes, scales, D);
}

/* The same encoding for a slice x[0..n) of a larger tensor whose maximum |x|
 * is amax and whose element index of x[0] is idx0 (rows sampled from a tensor
 * too large to encode whole). */
int oracle_nvfp4_quantize_f32_slice(const float* x, int64_t n, float amax, int64_t idx0, int mode,
                                    uint64_t seed, uint32_t stream, uint8_t* codes, uint8_t* scales,
                                    float* D) {
    if (!x || !codes || !scales || !D) return -1;
    if (idx0 < 0 || (idx0 % 16) != 0) return -2;
    return nvfp4_quantize_given_amax(x, n, amax, idx0, mode, seed, stream, codes, scales, D);
}

float oracle_amax_f32(const float* x, int64_t n) { return x ? amax_f32(x, n) : 0.0f; }

int oracle_nvfp4_quantize_bf16(const uint16_t* x, int64_t n, int mode, uint64_t seed,
                               uint32_t stream, uint8_t* codes, uint8_t* scales, float* D) {
    if (!x || !codes || !scales || !D) return -1;
    if (n < 0 || (n % 16) != 0) return -2;
    float* xf = (float*)malloc(sizeof(float) * (size_t)(n ? n : 1));
    if (!xf) return -3;
    for (int64_t i = 0; i < n; ++i) xf[i] = o_bf16_to_f32(x[i]);
    int rc = nvfp4_quantize_core(xf, n, mode, seed, stream, codes, scales, D);
    free(xf);
    return rc;
}

/* x' = (e2m1(q) * e4m3(sc)) * D: the first product is exact, the second is one
 * fp32 rounding. */
int oracle_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, float D, int64_t n,
                            float* out) {
    if (!codes || !scales || !out) return -1;
    if (n < 0 || (n % 16) != 0) return -2;
    for (int64_t i = 0; i < n; ++i) {
        uint8_t q = (uint8_t)((codes[i / 2] >> (4 * (i & 1))) & 0xF);
        float qs = o_e2m1_decode(q) * o_e4m3_decode(scales[i / 16]);
        out[i] = qs * D;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* MXFP8: E4M3 elements with an E8M0 scale per 32 (the backward format [AIC  */
/* "Key Takeaways"], [T01]).                                                 */
/* ------------------------------------------------------------------------- */

/* Reading (OCP MX rule, rule 0): shared exponent = floor(log2 amax) - 8 (8 =
 * exponent of E4M3's largest power of two), clamped to [-127,127]; element =
 * E4M3(x * 2^-se) with saturation; amax 0 gives scale byte 0 and zero codes.
 * x * 2^-se is one correctly rounded fp32 product. Rule 1 (the alternative
 * reading): se = ceil(log2(amax / 448)), the smallest exponent at which no
 * element exceeds E4M3's largest value, then the same element rule. */
static int mx_shared_exp(float amax, int rule) {
    int ex;
    frexpf(amax, &ex);          /* amax = m * 2^ex, m in [0.5,1) */
    int se = (ex - 1) - 8;
    if (rule == 1) {
        /* the alternative reading: the smallest se with amax <= 448 * 2^se
         * (ceil(log2(amax / 448))), so no element saturates; exact in double */
        se = (ex - 1) - 10;
        while ((double)amax > ldexp(448.0, se)) ++se;
    }
    if (se < -127) se = -127;
    if (se > 127) se = 127;
    return se;
}

static void mx_block(const float* xv, const int64_t* idx, int n, int mode, int rule, uint64_t seed,
                     uint32_t stream, uint8_t* out_e, uint8_t* out_s) {
    float amax = 0.0f;
    for (int j = 0; j < n; ++j) {
        float a = fabsf(xv[j]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *out_s = 0;
        for (int j = 0; j < n; ++j) out_e[j] = 0;
        return;
    }
    int se = mx_shared_exp(amax, rule);
    *out_s = (uint8_t)(se + 127);
    for (int j = 0; j < n; ++j) {
        float y = (float)ldexp((double)xv[j], -se); /* exact product, one rounding */
        out_e[j] = (mode == 0) ? o_e4m3_rne_sat(y)
                               : o_e4m3_sr(y, o_draw_u16(seed, stream, (uint64_t)idx[j]));
    }
}

int oracle_mxfp8_quantize(const uint16_t* x, int64_t R, int64_t C, int axis,
                          const int32_t* row_gather, int32_t gather_div,
                          const int32_t* seg_offsets, int64_t nseg, int mode,
                          uint64_t seed, uint32_t stream, int64_t ld,
                          uint8_t* elems, uint8_t* scales, int64_t row0, int rule) {
    if (!x || !elems || !scales) return -1;
    if (R < 0 || C <= 0 || gather_div <= 0 || row0 < 0) return -2;
    if (rule != 0 && rule != 1) return -5;
    if (axis == 0 && (C % 32) != 0) return -2;
    float xv[32];
    int64_t idx[32];
    uint8_t qe[32];
#define SRC_ROW(r) (row_gather ? (int64_t)(row_gather[(r)] / gather_div) : (int64_t)(r))
    if (axis == 0) {
        for (int64_t r = 0; r < R; ++r) {
            const uint16_t* xr = x + SRC_ROW(r) * C;
            for (int64_t b = 0; b < C / 32; ++b) {
                for (int j = 0; j < 32; ++j) {
                    xv[j] = o_bf16_to_f32(xr[32 * b + j]);
                    idx[j] = (row0 + r) * C + 32 * b + j;
                }
                mx_block(xv, idx, 32, mode, rule, seed, stream, elems + r * C + 32 * b,
                         scales + r * (C / 32) + b);
            }
        }
        return 0;
    }
    if (axis != 1) return -5;
    if ((ld % 32) != 0) return -2;
    int32_t one_seg[2] = {0, (int32_t)R};
    if (!seg_offsets) { seg_offsets = one_seg; nseg = 1; }
    int64_t pad = 0;
    for (int64_t s = 0; s < nseg; ++s) {
        int64_t r0 = seg_offsets[s], r1 = seg_offsets[s + 1];
        int64_t n = r1 - r0, nb = (n + 31) / 32;
        if (pad + 32 * nb > ld) return -3;
        for (int64_t c = 0; c < C; ++c) {
            for (int64_t b = 0; b < nb; ++b) {
                int64_t rs = r0 + 32 * b;
                int cnt = (int)((r1 - rs) < 32 ? (r1 - rs) : 32);
                for (int j = 0; j < cnt; ++j) {
                    xv[j] = o_bf16_to_f32(x[SRC_ROW(rs + j) * C + c]);
                    idx[j] = (row0 + rs + j) * C + c;
                }
                uint8_t* dst = elems + c * ld + pad + 32 * b;
                mx_block(xv, idx, cnt, mode, rule, seed, stream, qe, scales + c * (ld / 32) + pad / 32 + b);
                for (int j = 0; j < 32; ++j) dst[j] = (j < cnt) ? qe[j] : 0;
            }
        }
        pad += 32 * nb;
    }
    for (int64_t c = 0; c < C; ++c) {
        for (int64_t p = pad; p < ld; ++p) elems[c * ld + p] = 0;
        for (int64_t p = pad / 32; p < ld / 32; ++p) scales[c * (ld / 32) + p] = 0;
    }
#undef SRC_ROW
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Routing metadata: expert segments in a stable order (top-8 of 384 per      */
/* token [T10]). Reading: rows of an expert are kept in assignment order.    */
/* ------------------------------------------------------------------------- */

int oracle_route(const int32_t* topk_ids, int64_t A, int64_t E, int32_t* offsets,
                 int32_t* sorted2assign) {
    if (!topk_ids || !offsets || !sorted2assign) return -1;
    if (A < 0 || E <= 0) return -2;
    int64_t pos = 0;
    for (int64_t e = 0; e < E; ++e) {
        offsets[e] = (int32_t)pos;
        for (int64_t a = 0; a < A; ++a)
            if (topk_ids[a] == e) sorted2assign[pos++] = (int32_t)a;
    }
    offsets[E] = (int32_t)pos;
    return 0;
}

/* Router of the expert layer (page "Thinking Machines首發大模型：9750億參數，
 * 完整開放權重", section "架構", on the lab's earlier Inkling model; the Inkling 2
 * Small pages give only 8 of 384 experts per token, and this reading takes the
 * same design: it follows DeepSeek-V3, scores are sigmoids, a load-balancing
 * bias without an auxiliary loss steers the choice, and the chosen scores are
 * normalized into the combine weights). Per token t:
 * s_e = 1 / (1 + exp(-logit[t][e])) and key_e = s_e + bias[e], both in fp64;
 * k times, the expert with the largest key among those not yet chosen (the
 * lower index on a tie) is appended to ids[t]; w[t][j] = s_{ids[t][j]} divided
 * by the sum of the chosen s, summed in choice order. The bias only steers the
 * choice; the weights use the plain scores. Shared experts, whose scores the
 * page folds into the same normalization, are not part of the routed path. */
int oracle_router_sigmoid_topk(const float* logits, const float* bias, int64_t T, int64_t E, int k,
                               int32_t* ids, double* w) {
    if (!logits || !bias || !ids || !w) return -1;
    if (T < 0 || E <= 0 || k < 1 || k > E) return -2;
    double* s = (double*)malloc(sizeof(double) * (size_t)E);
    double* key = (double*)malloc(sizeof(double) * (size_t)E);
    if (!s || !key) { free(s); free(key); return -3; }
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            s[e] = 1.0 / (1.0 + exp(-(double)logits[t * E + e]));
            key[e] = s[e] + (double)bias[e];
        }
        double sum = 0.0;
        for (int j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int i = 0; i < j; ++i) taken |= ids[t * k + i] == e;
                if (!taken && (best < 0 || key[e] > key[best])) best = e;
            }
            ids[t * k + j] = (int32_t)best;
            sum += s[best];
        }
        for (int j = 0; j < k; ++j) w[t * k + j] = s[ids[t * k + j]] / sum;
    }
    free(s);
    free(key);
    return 0;
}

/* Router of the expert layer, softmax reading: 8 of 384 experts per token
 * (page "AI模型库 · 今日一模 Inkling 2 Small", section "01 PART"); the pages give
 * no routing formula, so this takes the plain top-k softmax router with a
 * selection-only load-balancing bias (the design the page "Thinking Machines
 * 首發大模型：9750億參數，完整開放權重", section "架構", reports for the lab's
 * earlier model, there with sigmoid scores). Per token t:
 *   key_e = (double)logit[t][e] + (double)bias[e]   (bias NULL: 0);
 *   k times, the expert with the largest key among those not yet chosen (the
 *   lower index on a tie) is appended to ids[t];
 *   with m the largest chosen raw logit and p_j = exp(logit_j - m) in fp64,
 *   w[t][j] = p_j / (p_0 + ... + p_{k-1}) (summed in choice order).
 * The bias only steers the choice; the weights are the softmax of the chosen
 * raw logits. The caller rounds w to fp32. */
int oracle_router_softmax_topk(const float* logits, const float* bias, int64_t T, int64_t E, int k,
                               int32_t* ids, double* w) {
    if (!logits || !ids || !w) return -1;
    if (T < 0 || E <= 0 || k < 1 || k > E) return -2;
    double* key = (double*)malloc(sizeof(double) * (size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)k);
    if (!key || !p) { free(key); free(p); return -3; }
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        for (int64_t e = 0; e < E; ++e) key[e] = (double)l[e] + (bias ? (double)bias[e] : 0.0);
        for (int j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int i = 0; i < j; ++i) taken |= ids[t * k + i] == e;
                if (!taken && (best < 0 || key[e] > key[best])) best = e;
            }
            ids[t * k + j] = (int32_t)best;
        }
        double m = (double)l[ids[t * k]];
        for (int j = 1; j < k; ++j)
            if ((double)l[ids[t * k + j]] > m) m = (double)l[ids[t * k + j]];
        double sum = 0.0;
        for (int j = 0; j < k; ++j) {
            p[j] = exp((double)l[ids[t * k + j]] - m);
            sum += p[j];
        }
        for (int j = 0; j < k; ++j) w[t * k + j] = p[j] / sum;
    }
    free(key);
    free(p);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Exact NVFP4 GEMMs. A dequantized operand before its tensor scale is        */
/* e2m1 * e4m3 = I * 2^-10 with I an integer, |I| <= 12 * 229376 < 2^22, so a  */
/* dot product over K <= 2^12 terms is exact in int64 and the only rounding is */
/* the final fp64 scaling.                                                   */
/* ------------------------------------------------------------------------- */

/* Decoded values cached as integers: 2*e2m1 for the 16 codes and 512*e4m3 for
 * the 256 bytes (NaN bytes map to 0; they are never produced). */
static int32_t g_e2m1x2[16], g_e4m3x512[256];
static int g_luts_ready = 0;

static void init_luts(void) {
    if (g_luts_ready) return;
    for (int c = 0; c < 16; ++c) g_e2m1x2[c] = (int32_t)((double)o_e2m1_decode((uint8_t)c) * 2.0);
    for (int b = 0; b < 256; ++b) {
        float v = o_e4m3_decode((uint8_t)b);
        g_e4m3x512[b] = isnan(v) ? 0 : (int32_t)((double)v * 512.0);
    }
    g_luts_ready = 1;
}

static int32_t nvfp4_int(const uint8_t* codes, const uint8_t* scales, int64_t i) {
    uint8_t q = (uint8_t)((codes[i / 2] >> (4 * (i & 1))) & 0xF);
    return g_e2m1x2[q] * g_e4m3x512[scales[i / 16]]; /* exact integer */
}

/* Decode one row of an NVFP4 matrix to integers I with value = I * 2^-10. */
static void nvfp4_row_int(const uint8_t* codes, const uint8_t* scales, int64_t K, int32_t* dst) {
    for (int64_t k = 0; k < K; ++k) dst[k] = nvfp4_int(codes, scales, k);
}

static int find_expert(const int32_t* offsets, int64_t E, int64_t r) {
    for (int64_t e = 0; e < E; ++e)
        if (r >= offsets[e] && r < offsets[e + 1]) return (int)e;
    return -1;
}

/* fc1 of the expert FFN [AIC "Key Takeaways": NVFP4 in the expert-layer
 * forward]. Reading: W1_e rows [0,d_ff) are the gate projection and rows
 * [d_ff,2 d_ff) the up projection; no biases. */
int oracle_moe_fc1(const uint8_t* xc, const uint8_t* xs, float Dx, int64_t d,
                   const int32_t* offsets, const int32_t* sorted2assign, int32_t topk,
                   int64_t E, int64_t d_ff, const uint8_t* w1c, const uint8_t* w1s,
                   const float* Dw1, const int32_t* rows, int64_t nrows, double* G) {
    if (!xc || !xs || !offsets || !sorted2assign || !w1c || !w1s || !Dw1 || !G) return -1;
    if (d <= 0 || (d % 16) != 0 || topk <= 0 || E <= 0 || d_ff <= 0) return -2;
    init_luts();
    if (!rows) nrows = offsets[E];
    int32_t* xi = (int32_t*)malloc(sizeof(int32_t) * (size_t)d);
    int32_t* wi = (int32_t*)malloc(sizeof(int32_t) * (size_t)(2 * d_ff * d));
    if (!xi || !wi) { free(xi); free(wi); return -3; }
    int cached = -1;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        int e = find_expert(offsets, E, r);
        if (e < 0) { free(xi); free(wi); return -2; }
        if (e != cached) {
            for (int64_t nn = 0; nn < 2 * d_ff; ++nn)
                nvfp4_row_int(w1c + ((int64_t)e * 2 * d_ff + nn) * (d / 2),
                              w1s + ((int64_t)e * 2 * d_ff + nn) * (d / 16), d, wi + nn * d);
            cached = e;
        }
        int64_t t = sorted2assign[r] / topk;
        nvfp4_row_int(xc + t * (d / 2), xs + t * (d / 16), d, xi);
        double scale = ldexp((double)Dx * (double)Dw1[e], -20);
        for (int64_t nn = 0; nn < 2 * d_ff; ++nn) {
            int64_t acc = 0;
            for (int64_t kk = 0; kk < d; ++kk) acc += (int64_t)xi[kk] * wi[nn * d + kk];
            G[i * 2 * d_ff + nn] = (double)acc * scale;
        }
    }
    free(xi);
    free(wi);
    return 0;
}

/* SwiGLU: h = silu(g) * u = g * u / (1 + exp(-g)) in fp64. */
int oracle_swiglu(const double* G, int64_t nrows, int64_t d_ff, double* H) {
    if (!G || !H) return -1;
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t j = 0; j < d_ff; ++j) {
            double g = G[i * 2 * d_ff + j], u = G[i * 2 * d_ff + d_ff + j];
            H[i * d_ff + j] = g * u / (1.0 + exp(-g));
        }
    return 0;
}

int oracle_moe_fc2(const uint8_t* hc, const uint8_t* hs, float DH, int64_t d_ff,
                   const int32_t* offsets, int64_t E, int64_t d, const uint8_t* w2c,
                   const uint8_t* w2s, const float* Dw2, const int32_t* rows, int64_t nrows,
                   double* Y) {
    if (!hc || !hs || !offsets || !w2c || !w2s || !Dw2 || !Y) return -1;
    if (d_ff <= 0 || (d_ff % 16) != 0 || E <= 0 || d <= 0) return -2;
    init_luts();
    if (!rows) nrows = offsets[E];
    int32_t* hi = (int32_t*)malloc(sizeof(int32_t) * (size_t)d_ff);
    int32_t* wi = (int32_t*)malloc(sizeof(int32_t) * (size_t)(d * d_ff));
    if (!hi || !wi) { free(hi); free(wi); return -3; }
    int cached = -1;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        int e = find_expert(offsets, E, r);
        if (e < 0) { free(hi); free(wi); return -2; }
        if (e != cached) {
            for (int64_t nn = 0; nn < d; ++nn)
                nvfp4_row_int(w2c + ((int64_t)e * d + nn) * (d_ff / 2),
                              w2s + ((int64_t)e * d + nn) * (d_ff / 16), d_ff, wi + nn * d_ff);
            cached = e;
        }
        nvfp4_row_int(hc + r * (d_ff / 2), hs + r * (d_ff / 16), d_ff, hi);
        double scale = ldexp((double)DH * (double)Dw2[e], -20);
        for (int64_t nn = 0; nn < d; ++nn) {
            int64_t acc = 0;
            for (int64_t j = 0; j < d_ff; ++j) acc += (int64_t)hi[j] * wi[nn * d_ff + j];
            Y[i * d + nn] = (double)acc * scale;
        }
    }
    free(hi);
    free(wi);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* NVFP4 backward GEMMs: the backward in the forward's 4-bit format, which   */
/* the pages name as their next step (page "Thinking Machines Details End-to- */
/* End 4-Bit Training for Inkling 2 Small", section "Developer quick start":  */
/* exploring FP4 backward passes). Same exact arithmetic as the forward:      */
/* every dequantized operand value before its tensor scale is I * 2^-10, the  */
/* dot products are int64 sums, and the scales apply once in fp64.           */
/* ------------------------------------------------------------------------- */

/* dgrad: for listed sorted rows r of expert e (rows == NULL: all offsets[E]),
 * out[i][n] = Da * Db[e] * sum_k deq(A[arow])[k] * deq(B[e][n])[k], with
 * arow = a_gather ? a_gather[r] : r. A codes [*, K/2], scales [*, K/16];
 * B codes [E, N, K/2], scales [E, N, K/16]. */
int oracle_nvfp4_gemm_dgrad(const uint8_t* ac, const uint8_t* as, float Da, const int32_t* a_gather,
                            const int32_t* offsets, int64_t E, int64_t N, int64_t K, const uint8_t* bc,
                            const uint8_t* bs, const float* Db, const int32_t* rows, int64_t nrows,
                            double* out) {
    if (!ac || !as || !offsets || !bc || !bs || !Db || !out) return -1;
    if (E <= 0 || N <= 0 || K <= 0 || (K % 16) != 0) return -2;
    init_luts();
    if (!rows) nrows = offsets[E];
    int32_t* ai = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    int32_t* bi = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N * K));
    if (!ai || !bi) { free(ai); free(bi); return -3; }
    int cached = -1;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        int e = find_expert(offsets, E, r);
        if (e < 0) { free(ai); free(bi); return -2; }
        if (e != cached) {
            for (int64_t n = 0; n < N; ++n)
                nvfp4_row_int(bc + ((int64_t)e * N + n) * (K / 2), bs + ((int64_t)e * N + n) * (K / 16), K,
                              bi + n * K);
            cached = e;
        }
        int64_t arow = a_gather ? a_gather[r] : r;
        nvfp4_row_int(ac + arow * (K / 2), as + arow * (K / 16), K, ai);
        double scale = ldexp((double)Da * (double)Db[e], -20);
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += (int64_t)ai[k] * bi[n * K + k];
            out[i * N + n] = (double)acc * scale;
        }
    }
    free(ai);
    free(bi);
    return 0;
}

/* wgrad: for listed experts e (experts == NULL: all E),
 * out[i][m][n] = Da * Db * sum over k in [pad_offsets[e], pad_offsets[e+1]) of
 * deq(A[m])[k] * deq(B[n])[k]; A codes [M, ld/2], scales [M, ld/16]; B codes
 * [N, ld/2], scales [N, ld/16] (the transposed, segment-padded layout). */
int oracle_nvfp4_gemm_wgrad(const uint8_t* ac, const uint8_t* as, float Da, const uint8_t* bc,
                            const uint8_t* bs, float Db, const int32_t* pad_offsets, int64_t E, int64_t M,
                            int64_t N, int64_t ld, const int32_t* experts, int64_t nexp, double* out) {
    if (!ac || !as || !bc || !bs || !pad_offsets || !out) return -1;
    if (E <= 0 || M <= 0 || N <= 0 || ld <= 0 || (ld % 16) != 0) return -2;
    init_luts();
    if (!experts) nexp = E;
    double scale = ldexp((double)Da * (double)Db, -20);
    for (int64_t i = 0; i < nexp; ++i) {
        int64_t e = experts ? experts[i] : i;
        int64_t k0 = pad_offsets[e], k1 = pad_offsets[e + 1];
        if (k0 < 0 || k1 > ld || k1 < k0) return -2;
        int64_t w = k1 - k0;
        int32_t* ai = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * (w > 0 ? w : 1)));
        int32_t* bi = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N * (w > 0 ? w : 1)));
        if (!ai || !bi) { free(ai); free(bi); return -3; }
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < w; ++k) ai[m * w + k] = nvfp4_int(ac + m * (ld / 2), as + m * (ld / 16), k0 + k);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t k = 0; k < w; ++k) bi[n * w + k] = nvfp4_int(bc + n * (ld / 2), bs + n * (ld / 16), k0 + k);
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n) {
                int64_t acc = 0;
                for (int64_t k = 0; k < w; ++k) acc += (int64_t)ai[m * w + k] * bi[n * w + k];
                out[(i * M + m) * N + n] = (double)acc * scale;
            }
        free(ai);
        free(bi);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Exact MXFP8 GEMMs: e4m3 * 2^9 is an integer (< 2^18), a 32-term block      */
/* product sum is exact in int64 (< 2^41) and is scaled exactly by            */
/* 2^(sa + sb - 18); blocks are summed in fp64.                               */
/* ------------------------------------------------------------------------- */

static int32_t e4m3_int(uint8_t b) { return g_e4m3x512[b]; }

static double mx_dot(const uint8_t* ae, const uint8_t* as, const uint8_t* be, const uint8_t* bs,
                     int64_t k0, int64_t k1) {
    double sum = 0.0;
    for (int64_t b = k0 / 32; b < k1 / 32; ++b) {
        int64_t acc = 0;
        for (int j = 0; j < 32; ++j) acc += (int64_t)e4m3_int(ae[32 * b + j]) * e4m3_int(be[32 * b + j]);
        sum += ldexp((double)acc, ((int)as[b] - 127) + ((int)bs[b] - 127) - 18);
    }
    return sum;
}

int oracle_mxfp8_gemm_dgrad(const uint8_t* ae, const uint8_t* as, const uint8_t* be,
                            const uint8_t* bs, const int32_t* offsets, int64_t E, int64_t N,
                            int64_t K, const int32_t* rows, int64_t nrows, double* out) {
    if (!ae || !as || !be || !bs || !offsets || !out) return -1;
    if (E <= 0 || N <= 0 || K <= 0 || (K % 32) != 0) return -2;
    init_luts();
    if (!rows) nrows = offsets[E];
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        int e = find_expert(offsets, E, r);
        if (e < 0) return -2;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* brow = be + ((int64_t)e * N + n) * K;
            const uint8_t* bsrow = bs + ((int64_t)e * N + n) * (K / 32);
            out[i * N + n] = mx_dot(ae + r * K, as + r * (K / 32), brow, bsrow, 0, K);
        }
    }
    return 0;
}

int oracle_mxfp8_gemm_wgrad(const uint8_t* ae, const uint8_t* as, const uint8_t* be,
                            const uint8_t* bs, const int32_t* pad_offsets, int64_t E,
                            int64_t M, int64_t N, int64_t ld, const int32_t* experts,
                            int64_t nexp, double* out) {
    if (!ae || !as || !be || !bs || !pad_offsets || !out) return -1;
    if (E <= 0 || M <= 0 || N <= 0 || (ld % 32) != 0) return -2;
    init_luts();
    if (!experts) nexp = E;
    for (int64_t i = 0; i < nexp; ++i) {
        int64_t e = experts ? experts[i] : i;
        int64_t k0 = pad_offsets[e], k1 = pad_offsets[e + 1];
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n)
                out[(i * M + m) * N + n] =
                    mx_dot(ae + m * ld, as + m * (ld / 32), be + n * ld, bs + n * (ld / 32), k0, k1);
    }
    return 0;
}

/* SwiGLU backward, h = g * sigma(g) * u:
 *   dg = dh * u * sigma(g) * (1 + g * (1 - sigma(g))),  du = dh * g * sigma(g). */
int oracle_swiglu_bwd(const float* dH, const uint16_t* gu, int64_t n, int64_t d_ff,
                      double* dA) {
    if (!dH || !gu || !dA) return -1;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < d_ff; ++j) {
            double g = o_bf16_to_f32(gu[i * 2 * d_ff + j]);
            double u = o_bf16_to_f32(gu[i * 2 * d_ff + d_ff + j]);
            double dh = dH[i * d_ff + j];
            double sg = 1.0 / (1.0 + exp(-g));
            dA[i * 2 * d_ff + j] = dh * u * sg * (1.0 + g * (1.0 - sg));
            dA[i * 2 * d_ff + d_ff + j] = dh * g * sg;
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* 32-point random Hadamard transform before the expert-parallel combine is    */
/* quantized [AIC "Key Takeaways", "Architecture highlights"].               */
/* Readings: one 32-sign vector for the whole tensor, bit j of Philox word 0  */
/* at counter (0,0,4,0) under key = sign seed, set bit = -1; z = (1/sqrt 32)  */
/* H32 (s .* x) with H32 in Sylvester (natural) order, computed as the radix-2 */
/* butterfly with strides 1,2,4,8,16 in fp32, then one multiply by the fp32    */
/* constant (float)(1/sqrt(32)).                                               */
/* ------------------------------------------------------------------------- */

uint32_t o_rht32_signs(uint64_t sign_seed) {
    uint32_t ctr[4] = {0u, 0u, 4u, 0u};
    uint32_t key[2] = {(uint32_t)sign_seed, (uint32_t)(sign_seed >> 32)};
    uint32_t out[4];
    o_philox4x32_10(ctr, key, out);
    return out[0];
}

static void fwht32_f32(float* v) {
    for (int h = 1; h < 32; h <<= 1)
        for (int i = 0; i < 32; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

int oracle_rht32_forward(const uint16_t* x, int64_t n, uint64_t sign_seed, float* z) {
    if (!x || !z) return -1;
    if (n < 0 || (n % 32) != 0) return -2;
    uint32_t sw = o_rht32_signs(sign_seed);
    const float c32 = (float)(1.0 / sqrt(32.0));
    float v[32];
    for (int64_t base = 0; base < n; base += 32) {
        for (int j = 0; j < 32; ++j) {
            float xj = o_bf16_to_f32(x[base + j]);
            v[j] = ((sw >> j) & 1u) ? -xj : xj;
        }
        fwht32_f32(v);
        for (int j = 0; j < 32; ++j) z[base + j] = v[j] * c32;
    }
    return 0;
}

/* Combine: each output row t is the weighted sum over its k slots of the
 * inverse transform of the dequantized rows t*k+s; the inverse of the
 * orthonormal H32 * diag(s) is diag(s) * H32 / sqrt(32). Computed in fp64 as a
 * plain matrix product with H[i][j] = (-1)^popcount(i & j). */
int oracle_rht32_combine(const uint8_t* codes, const uint8_t* scales, float D, int64_t T,
                         int32_t topk, int64_t C, uint64_t sign_seed, const float* w,
                         double* out) {
    if (!codes || !scales || !w || !out) return -1;
    if (T < 0 || topk <= 0 || C <= 0 || (C % 32) != 0) return -2;
    uint32_t sw = o_rht32_signs(sign_seed);
    double inv = 1.0 / sqrt(32.0);
    double zc[32];
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < C; ++j) out[t * C + j] = 0.0;
        for (int s = 0; s < topk; ++s) {
            int64_t row = t * topk + s;
            double ws = w[t * topk + s];
            for (int64_t base = 0; base < C; base += 32) {
                for (int j = 0; j < 32; ++j) {
                    int64_t i = row * C + base + j;
                    uint8_t q = (uint8_t)((codes[i / 2] >> (4 * (i & 1))) & 0xF);
                    zc[j] = (double)o_e2m1_decode(q) * (double)o_e4m3_decode(scales[i / 16]) * (double)D;
                }
                for (int i = 0; i < 32; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < 32; ++j)
                        acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -zc[j] : zc[j];
                    double yi = ((sw >> i) & 1u) ? -acc * inv : acc * inv;
                    out[t * C + base + i] += ws * yi;
                }
            }
        }
    }
    return 0;
}
