/*
 * oracle.h -- plain, slow CPU oracle for the NVFP4 MoE expert path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The HIP library and its
 * Python binding never include, link or call it, and it shares no code with
 * them.
 *
 * Sources. The pages describe the recipe, not its formulas:
 *   - page "Thinking Machines Details End-to-End 4-Bit Training for Inkling 2
 *     Small" (aicoder.com), sections "Key Takeaways", "Background" and
 *     "Architecture highlights": NVFP4 for the MoE expert-layer forward only,
 *     about 4.5 bits per value; MXFP8 backward with re-quantization and
 *     stochastic rounding; a 32-dimensional random Hadamard transform before
 *     the expert-parallel combine is quantized to a block-scaled format.
 *   - page "Thinking Machines 详解 Inkling 2 Small 原生 4-bit 前向训练完整流程"
 *     (news.t0001.com), list "训练数值格式分工清单": the same split of formats.
 *   - page "AI模型库 · 今日一模 Inkling 2 Small" (10100.com), "01 PART":
 *     top-8 of 384 experts per token.
 * The element formats (E2M1 values, E4M3 scale per 16, FP32 tensor scale;
 * E4M3 elements with an E8M0 scale per 32) are the standard NVFP4 and OCP MX
 * layouts; every step the pages leave open is a stated reading, listed at the
 * function that takes it.
 *
 * Conventions: all pointers are host pointers; arrays are row-major and
 * contiguous; bf16 values travel as uint16_t bit patterns. Functions return
 * 0 on success and a negative value on a bad argument.
 */
#ifndef NVQ_ORACLE_H
#define NVQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar codecs ---- */
float    o_bf16_to_f32(uint16_t b);
uint16_t o_f64_to_bf16_rne(double v);
float    o_e2m1_decode(uint8_t code);            /* low 4 bits used */
float    o_e4m3_decode(uint8_t byte);            /* NaN for 0x7F / 0xFF */
float    o_e8m0_decode(uint8_t byte);            /* NaN for 0xFF */
uint8_t  o_e2m1_rne(float y);                    /* nearest, ties to even, saturate at 6 */
uint8_t  o_e2m1_sr(float y, uint32_t u16);       /* stochastic, 16-bit draw */
uint8_t  o_e4m3_rne_sat(float v);                /* nearest, ties to even, saturate at 448 */
uint8_t  o_e4m3_sr(float v, uint32_t u16);

/* ---- counter-based generator ---- */
void     o_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t o_draw_u16(uint64_t seed, uint32_t stream, uint64_t idx);

/* ---- NVFP4 ---- */
/* x: [n] values (bf16 bits or fp32), n % 16 == 0; one tensor scale over all n.
 * codes [n/2], scales [n/16] (E4M3 bytes), *D = decode tensor scale.
 * mode 0 = round to nearest even, 1 = stochastic (Philox index = element index). */
int oracle_nvfp4_quantize_bf16(const uint16_t* x, int64_t n, int mode, uint64_t seed,
                               uint32_t stream, uint8_t* codes, uint8_t* scales, float* D);
int oracle_nvfp4_quantize_f32(const float* x, int64_t n, int mode, uint64_t seed,
                              uint32_t stream, uint8_t* codes, uint8_t* scales, float* D);
/* The encoding of a slice x[0..n) of a larger tensor with maximum |x| = amax,
 * x[0] being element idx0 (idx0 % 16 == 0) of that tensor. */
int oracle_nvfp4_quantize_f32_slice(const float* x, int64_t n, float amax, int64_t idx0, int mode,
                                    uint64_t seed, uint32_t stream, uint8_t* codes, uint8_t* scales,
                                    float* D);
float oracle_amax_f32(const float* x, int64_t n);
/* out[i] = (e2m1(q_i) * e4m3(sc)) * D in fp32. */
int oracle_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, float D, int64_t n,
                            float* out);

/* ---- MXFP8 ---- */
/* axis 0: x [R,C] (optionally gathered: row r reads source row row_gather[r]/gather_div),
 *         elems [R,C], scales [R,C/32].
 * axis 1: per segment [seg_offsets[s], seg_offsets[s+1]) of rows, 32-row blocks
 *         restart at each segment; output transposed: elems [C,ld], scales [C,ld/32],
 *         zero padding after each segment's last row and after the last segment.
 *         seg_offsets == NULL means one segment [0,R).
 * mode 0 = RNE, 1 = stochastic; Philox index of element (r,c) = (row0 + r)*C + c, so
 * rows [row0, row0 + R) of a larger tensor (and segments of it) can be encoded alone.
 * rule 0: shared exponent floor(log2 amax) - 8, elements saturate; rule 1:
 * ceil(log2(amax / 448)), no element saturates (-5 for another rule). */
int oracle_mxfp8_quantize(const uint16_t* x, int64_t R, int64_t C, int axis,
                          const int32_t* row_gather, int32_t gather_div,
                          const int32_t* seg_offsets, int64_t nseg, int mode,
                          uint64_t seed, uint32_t stream, int64_t ld,
                          uint8_t* elems, uint8_t* scales, int64_t row0, int rule);

/* ---- routing ---- */
/* topk_ids [A] (A = T*k, assignment a = t*k + s). counts [E], offsets [E+1],
 * sorted2assign [A]: assignments grouped by expert, ascending a inside each group.
 * Ids outside [0,E) are dropped (they appear in no group). */
/* Sigmoid router with a selection-only bias: top-k ids [T,k] and normalized weights [T,k]. */
int oracle_router_sigmoid_topk(const float* logits, const float* bias, int64_t T, int64_t E, int k,
                               int32_t* ids, double* w);
/* Softmax router with a selection-only bias (bias may be NULL): top-k of logit + bias
 * in fp64, ties to the lower id; weights = softmax over the k chosen raw logits (fp64). */
int oracle_router_softmax_topk(const float* logits, const float* bias, int64_t T, int64_t E, int k,
                               int32_t* ids, double* w);
int oracle_route(const int32_t* topk_ids, int64_t A, int64_t E, int32_t* offsets,
                 int32_t* sorted2assign);

/* ---- NVFP4 expert GEMMs (exact) ---- */
/* fc1: for each listed sorted row r (rows==NULL: all offsets[E] rows) of expert e,
 * G[r][n] = sum_k deq(Xq[sorted2assign[r]/k])[k] * deq(W1q_e)[n][k] * Dx * Dw1[e],
 * n in [0, 2*d_ff): gate half then up half. Output row i of G is listed row i. */
int oracle_moe_fc1(const uint8_t* xc, const uint8_t* xs, float Dx, int64_t d,
                   const int32_t* offsets, const int32_t* sorted2assign, int32_t topk,
                   int64_t E, int64_t d_ff, const uint8_t* w1c, const uint8_t* w1s,
                   const float* Dw1, const int32_t* rows, int64_t nrows, double* G);
/* H = silu(g) * u in fp64 from G [nrows, 2*d_ff]. */
int oracle_swiglu(const double* G, int64_t nrows, int64_t d_ff, double* H);
/* fc2: Y[r][n] = sum_j deq(Hq[r])[j] * deq(W2q_e)[n][j] * DH * Dw2[e] for listed
 * sorted rows r of expert e; Hq rows are indexed by sorted row. */
int oracle_moe_fc2(const uint8_t* hc, const uint8_t* hs, float DH, int64_t d_ff,
                   const int32_t* offsets, int64_t E, int64_t d, const uint8_t* w2c,
                   const uint8_t* w2s, const float* Dw2, const int32_t* rows, int64_t nrows,
                   double* Y);

/* ---- NVFP4 backward GEMMs (exact) ---- */
/* dgrad: out[i][n] = Da*Db[e] * sum_k deq(A[arow])[k]*deq(B[e][n])[k] for listed sorted rows r
 *   of expert e, arow = a_gather ? a_gather[r] : r. B codes [E, N, K/2].
 * wgrad: out[i][m][n] = Da*Db * sum over k in [pad_offsets[e], pad_offsets[e+1]) of
 *   deq(A[m])[k]*deq(B[n])[k]; A codes [M, ld/2], B codes [N, ld/2]. */
int oracle_nvfp4_gemm_dgrad(const uint8_t* ac, const uint8_t* as, float Da, const int32_t* a_gather,
                            const int32_t* offsets, int64_t E, int64_t N, int64_t K, const uint8_t* bc,
                            const uint8_t* bs, const float* Db, const int32_t* rows, int64_t nrows,
                            double* out);
int oracle_nvfp4_gemm_wgrad(const uint8_t* ac, const uint8_t* as, float Da, const uint8_t* bc,
                            const uint8_t* bs, float Db, const int32_t* pad_offsets, int64_t E, int64_t M,
                            int64_t N, int64_t ld, const int32_t* experts, int64_t nexp, double* out);

/* ---- MXFP8 backward GEMMs (exact blocks, fp64 sum) ---- */
/* DGRAD (mode 0): out[r][n] = sum_k A[r][k] * B_e[n][k] for rows r of expert e.
 *   A: elems [Rrows, K] + scales [Rrows, K/32]; B: elems [E, N, K] + scales [E, N, K/32].
 * WGRAD (mode 1): out[e][m][n] = sum over the padded K range of expert e of
 *   A[m][k] * B[n][k]; A: elems [M, ld] + scales [M, ld/32]; B: elems [N, ld] + scales.
 *   pad_offsets [E+1] are the 32-aligned segment starts in the padded K space. */
int oracle_mxfp8_gemm_dgrad(const uint8_t* ae, const uint8_t* as, const uint8_t* be,
                            const uint8_t* bs, const int32_t* offsets, int64_t E, int64_t N,
                            int64_t K, const int32_t* rows, int64_t nrows, double* out);
int oracle_mxfp8_gemm_wgrad(const uint8_t* ae, const uint8_t* as, const uint8_t* be,
                            const uint8_t* bs, const int32_t* pad_offsets, int64_t E,
                            int64_t M, int64_t N, int64_t ld, const int32_t* experts,
                            int64_t nexp, double* out);
/* SwiGLU backward in fp64: dA [n, 2*d_ff] from dH [n, d_ff] (fp32) and saved g,u
 * [n, 2*d_ff] (bf16 bits, gate half then up half). */
int oracle_swiglu_bwd(const float* dH, const uint16_t* gu, int64_t n, int64_t d_ff,
                      double* dA);

/* ---- 32-point random Hadamard transform ---- */
uint32_t o_rht32_signs(uint64_t sign_seed);
/* z = (1/sqrt 32) * H32 * (s .* x) per 32-chunk, fp32 butterfly (the precision the
 * quantizer decides in). x [n] bf16, n % 32 == 0. */
int oracle_rht32_forward(const uint16_t* x, int64_t n, uint64_t sign_seed, float* z);
/* out[t][j] = sum_s w[t][s] * s_j * ((1/sqrt 32) H32 zdeq[t*k+s])_j in fp64,
 * zdeq = (e2m1*e4m3)*D. codes [T*k*C/2], scales [T*k*C/16]. out [T, C]. */
int oracle_rht32_combine(const uint8_t* codes, const uint8_t* scales, float D, int64_t T,
                         int32_t topk, int64_t C, uint64_t sign_seed, const float* w,
                         double* out);

#ifdef __cplusplus
}
#endif
#endif
