/*
 * nvq.h -- C ABI of libnvq.so, the MI355X (gfx950) library for the NVFP4
 * forward pass through MoE expert layers and its two companions (MXFP8
 * backward requantization with stochastic rounding; the 32-point random
 * Hadamard transform plus block quantization of the expert-combine tensor).
 *
 * Source pages (cited by title and section):
 *   [AIC] "Thinking Machines Details End-to-End 4-Bit Training for Inkling 2
 *         Small" (aicoder.com): "Key Takeaways" (NVFP4 only in the MoE expert
 *         forward; MXFP8 backward with re-quantization and stochastic
 *         rounding; RHT32 before quantizing the combine), "Background" (about
 *         4.5 bits per value), "Architecture highlights" (a dedicated kernel;
 *         a fully deterministic MoE kernel stack).
 *   [T01] "Thinking Machines 详解 Inkling 2 Small 原生 4-bit 前向训练完整流程"
 *         (news.t0001.com), "训练数值格式分工清单": the same split of formats.
 *   [T10] "AI模型库 · 今日一模 Inkling 2 Small" (10100.com), "01 PART":
 *         8 of 384 experts per token.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated; bf16 travels as uint16_t
 *     bit patterns; arrays are row-major and densely packed; data pointers
 *     must be 16-byte aligned.
 *   - Ownership: the caller allocates every input, output and workspace
 *     buffer. The library never allocates or frees memory, keeps no
 *     pointer after a call returns and holds no mutable setting (the one
 *     exception: nvfp4_quantize_noalloc's per-device address of its own
 *     static buffer); every call is safe to make from several host threads.
 *   - Asynchrony: all work is enqueued on `stream` (a hipStream_t; NULL is the
 *     default stream). No call synchronizes with the host.
 *   - Determinism: identical inputs give identical output bytes (no atomics;
 *     maxima are folded from partial maxima written with plain stores).
 *   - Errors: every call returns an NVQ_* status. Argument errors are
 *     detected on the host before anything is launched. Preconditions that
 *     would need a device read (finite inputs, 0 <= topk_ids < E) are not
 *     checked; out-of-range expert ids are dropped by the routing step.
 *   - Workspace: calls that need one take (ws, ws_bytes) and have a
 *     *_workspace_size() query; ws must be 256-byte aligned.
 */
#ifndef NVQ_H
#define NVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* nvq_stream_t; /* hipStream_t */

enum {
    NVQ_OK = 0,
    NVQ_ERR_NULL = -1,        /* a required pointer is NULL */
    NVQ_ERR_DIM = -2,         /* a size is out of range or not a multiple the call needs */
    NVQ_ERR_WORKSPACE = -3,   /* ws_bytes below the *_workspace_size() query */
    NVQ_ERR_LAUNCH = -4,      /* the HIP runtime rejected a launch */
    NVQ_ERR_UNSUPPORTED = -5, /* an option value the library does not implement */
    NVQ_ERR_ALIGN = -6        /* a pointer is not 16-byte (ws: 256-byte) aligned */
};

enum { NVQ_RTN = 0, NVQ_SR = 1 };             /* nearest-even / stochastic rounding */
enum { NVQ_OUT_BF16 = 0, NVQ_OUT_F32 = 1 };   /* dequantize output type */
enum { NVQ_DGRAD = 0, NVQ_WGRAD = 1, NVQ_FWD = 2 };  /* MXFP8 grouped GEMM modes */

const char* nvq_status_string(int status);
int nvq_abi_version(void);

/* ------------------------------------------------------------------------ */
/* NVFP4 block quantization ([AIC] "Background": about 4.5 bits per value).  */
/* Layout: E2M1 codes two per byte, even element in the low nibble; one E4M3 */
/* scale byte per 16 consecutive values; one FP32 decode scale D per tensor. */
/* Numerics: S = 2688/amax, D = amax/2688 (fp32 divisions); block byte =      */
/* nearest-even E4M3 of (amax_block/6)*S, saturating at 448; element code =  */
/* E2M1 of x*(S/e4m3(byte)), nearest-even (saturating at 6, sign kept) or    */
/* stochastic with a Philox4x32-10 16-bit draw per element, keyed by (seed,  */
/* stream_id, element index within its tensor). An all-zero tensor gives     */
/* D = 1 and all-zero bytes.                                                 */
/* ------------------------------------------------------------------------ */

/* Quantize B independent tensors x [B, R, C] (bf16), C % 16 == 0,
 * 1 <= B <= 65535, one tensor scale per batch entry. Outputs: codes
 * [B, R, C/2], scales [B, R, C/16], tscale [B] (fp32 D). Two passes: partial
 * maxima of each tensor (into ws), then encode. */
size_t nvfp4_quantize_workspace_size(int64_t B, int64_t R, int64_t C);
int nvfp4_quantize(const uint16_t* x, int64_t B, int64_t R, int64_t C,
                   uint8_t* codes, uint8_t* scales, float* tscale,
                   int round_mode, uint64_t seed, uint32_t stream_id,
                   void* ws, size_t ws_bytes, nvq_stream_t stream);

/* nvfp4_quantize without workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, checks, results and status codes as
 * nvfp4_quantize, with the partial maxima kept in a fixed 256 KiB array of the
 * library on each device (65536 words, enough for every B <= 65535; a size
 * beyond it would return NVQ_ERR_WORKSPACE). The array of the device current
 * at the call is used, so `stream` must belong to that device. Calls that
 * overlap on one device (two streams, or two host threads) share that array
 * and race; calls on one stream are ordered. Allocates nothing. */
int nvfp4_quantize_noalloc(const uint16_t* x, int64_t B, int64_t R, int64_t C,
                           uint8_t* codes, uint8_t* scales, float* tscale,
                           int round_mode, uint64_t seed, uint32_t stream_id,
                           nvq_stream_t stream);

/* out[b][r][c] = (e2m1(code) * e4m3(scale)) * tscale[b], one fp32 rounding;
 * NVQ_OUT_BF16 rounds that fp32 value to bf16 (nearest even).
 * 1 <= B <= 65535, C % 16 == 0. */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tscale,
                     int64_t B, int64_t R, int64_t C, void* out, int out_dtype,
                     nvq_stream_t stream);

/* ------------------------------------------------------------------------ */
/* MoE expert forward in NVFP4 ([AIC] "Key Takeaways": NVFP4 only in the     */
/* forward of the expert layers; "Architecture highlights": re-quantization; */
/* [T10] "01 PART": top-8 of 384).                                          */
/* For every assignment a = t*k + s (token t, slot s) with e = topk_ids[a]:  */
/*   g,u = deq(Xq[t]) . deq(W1q_e)^T  (W1_e rows [0,d_ff) gate, [d_ff,2d_ff) */
/*         up; the fp32 accumulator times Dx*Dw1[e])                         */
/*   h   = silu(g) * u, rounded to bf16; one NVFP4 tensor scale over all of H */
/*   y[t][s] = deq(Hq[a]) . deq(W2q_e)^T (times DH*Dw2[e]) rounded to bf16    */
/* Expert rows are processed in a stable expert-sorted order.                */
/* Weights: w1 codes [E, 2*d_ff, d/2], scales [E, 2*d_ff, d/16], tscale [E];  */
/*          w2 codes [E, d, d_ff/2],   scales [E, d, d_ff/16],   tscale [E]  */
/*          (one NVFP4 tensor per expert matrix, as nvfp4_quantize with B=E). */
/* Limits: d % 128 == 0, d_ff % 128 == 0, 1 <= k <= E <= 4096, T*k < 2^31, */
/*   T*d/2, T*k*d_ff/2 and d*d_ff below 2^32 (code offsets are 32-bit), and  */
/*   the output tiles of each GEMM ((T*k/256 + E + 1) * max(d_ff/64, d/128)) */
/*   below 2^31; else NVQ_ERR_DIM.                                           */
/* ------------------------------------------------------------------------ */

/* Optional caller-owned intermediates. Any field may be NULL; a NULL field is
 * carved from the workspace instead. A = T*k rows in expert-sorted order.  */
typedef struct {
    uint8_t* xq_codes;      /* [T, d/2]      quantized input               */
    uint8_t* xq_scales;     /* [T, d/16]                                    */
    float* xq_tscale;       /* [1]                                          */
    int32_t* offsets;       /* [E+1]         expert segment starts          */
    int32_t* sorted2assign; /* [A]           sorted row -> assignment index */
    uint16_t* h;            /* [A, d_ff]     bf16 SwiGLU output (sorted)    */
    uint8_t* hq_codes;      /* [A, d_ff/2]   re-quantized H                 */
    uint8_t* hq_scales;     /* [A, d_ff/16]                                 */
    float* hq_tscale;       /* [1]                                          */
    uint16_t* gu;           /* [A, 2*d_ff]   bf16 g,u saved for backward;   */
                            /*               NULL = not saved               */
    int gemm_workgroups;    /* persistent grid cap of fc1 and fc2 (see the */
                            /* stage calls below); 0 = default              */
} nvq_moe_buffers;

size_t moe_expert_fwd_nvfp4_workspace_size(int64_t T, int64_t d, int k, int64_t E,
                                           int64_t d_ff);
int moe_expert_fwd_nvfp4(const uint16_t* x, int64_t T, int64_t d,
                         const int32_t* topk_ids, int k, int64_t E, int64_t d_ff,
                         const uint8_t* w1_codes, const uint8_t* w1_scales, const float* w1_tscale,
                         const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_tscale,
                         uint16_t* y, const nvq_moe_buffers* bufs,
                         void* ws, size_t ws_bytes, nvq_stream_t stream);

/* Stages of moe_expert_fwd_nvfp4, exported for staged checks and timing.   */

/* Router of the configs ([T10] "01 PART": 8 of 384 experts per token; the   */
/* pages give no routing formula, so this takes the plain top-k softmax      */
/* router with a selection-only load-balancing bias). Per token t:           */
/*   key_e = (double)logits[t][e] + (double)bias[e]   (bias NULL: 0);        */
/*   topk_ids[t] = the k experts of largest key, in descending key order     */
/*   (equal keys: the lower index first);                                    */
/*   weights[t][j] = p_j / (p_0 + ... + p_{k-1}) (sum in choice order),       */
/*   p_j = exp(logit_j - m) in fp64, m the largest chosen raw logit, rounded */
/*   to fp32: the softmax of the chosen raw logits (the bias only steers).   */
/* When offsets is not NULL the same call also routes the chosen ids (as     */
/* moe_route with A = T*k): offsets [E+1], sorted2assign [T*k] and, if not   */
/* NULL, tile_offsets [E+1]; then ws (256-byte aligned, at least             */
/* moe_router_softmax_topk_workspace_size) is required. logits [T, E] fp32,  */
/* bias [E] fp32, topk_ids [T, k] int32, weights [T, k] fp32. Limits:        */
/* 1 <= k <= min(E, 64), E <= 1024, T*E < 2^31 (else NVQ_ERR_DIM).           */
/* Non-finite logits are undefined behaviour.                                */
size_t moe_router_softmax_topk_workspace_size(int64_t T, int64_t E, int k);
int moe_router_softmax_topk(const float* logits, int64_t T, int64_t E, const float* bias, int k,
                            int32_t* topk_ids, float* weights,
                            int32_t* offsets, int32_t* sorted2assign, int32_t* tile_offsets,
                            void* ws, size_t ws_bytes, nvq_stream_t stream);

/* Sigmoid router: the reading from the lab's EARLIER model (page "Thinking */
/* Machines首發大模型：9750億參數，完整開放權重", section "架構"), kept beside the */
/* softmax router above: DeepSeek-V3 style, sigmoid scores, an auxiliary-    */
/* loss-free load-balancing bias, the chosen scores normalized).             */
/* Per token t: s_e = 1/(1 + exp(-logits[t][e])), key_e = s_e + bias[e], both */
/* in fp64; topk_ids[t] = the k experts of largest key in descending order   */
/* (equal keys: the lower index first); weights[t][j] = s of the j-th expert  */
/* over the sum of the k chosen s (summed in that order), rounded to fp32.    */
/* logits [T, E] fp32, bias [E] fp32 -> topk_ids [T, k] int32, weights [T, k] */
/* fp32. Limits: 1 <= k <= min(E, 64), E <= 1024, T*E < 2^31 (else           */
/* NVQ_ERR_DIM). Non-finite logits are undefined behaviour.                  */
int moe_router_sigmoid_topk(const float* logits, int64_t T, int64_t E, const float* bias, int k,
                            int32_t* topk_ids, float* weights, nvq_stream_t stream);

/* Routing: topk_ids [A] -> offsets [E+1], sorted2assign [A] (rows of each
 * expert in ascending assignment order; entries past offsets[E] are unused).
 * tile_offsets (nullable) [E+1]: prefix sums of ceil(n_e / 256) (the grouped GEMMs' row tiles). */
size_t moe_route_workspace_size(int64_t A, int64_t E);
int moe_route(const int32_t* topk_ids, int64_t A, int64_t E, int32_t* offsets,
              int32_t* sorted2assign, int32_t* tile_offsets,
              void* ws, size_t ws_bytes, nvq_stream_t stream);

/* fc1 + SwiGLU: h [A, d_ff] bf16 in sorted order; gu (nullable) saves g,u;
 * h_amax (nullable, device fp32 [1]) receives max|h|. */
size_t moe_fc1_workspace_size(int64_t A, int64_t E);
int moe_fc1_swiglu_nvfp4(const uint8_t* xq_codes, const uint8_t* xq_scales, const float* xq_tscale,
                         int64_t T, int64_t d, const int32_t* offsets, const int32_t* sorted2assign,
                         int k, int64_t E, int64_t d_ff,
                         const uint8_t* w1_codes, const uint8_t* w1_scales, const float* w1_tscale,
                         uint16_t* h, uint16_t* gu, float* h_amax, int workgroups,
                         void* ws, size_t ws_bytes, nvq_stream_t stream);

/* fc2: y[sorted2assign[r]] = deq(Hq[r]) . deq(W2q_e)^T * DH * Dw2[e] (bf16);
 * A = number of rows of Hq and of y. */
size_t moe_fc2_workspace_size(int64_t A, int64_t E);
int moe_fc2_nvfp4(const uint8_t* hq_codes, const uint8_t* hq_scales, const float* hq_tscale,
                  int64_t A, int64_t d_ff, const int32_t* offsets, const int32_t* sorted2assign,
                  int64_t E, int64_t d,
                  const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_tscale,
                  uint16_t* y, int workgroups, void* ws, size_t ws_bytes, nvq_stream_t stream);

/* workgroups (fc1, fc2, and nvq_moe_buffers.gemm_workgroups of the fused
 * call): the persistent grid of the grouped GEMM. At most `workgroups`
 * 256-thread workgroups walk the output tiles, each taking every G-th tile
 * and carrying its operand prefetch from one tile into the next; 0 = as
 * many as the compute units hold at once (one per CU for 256-column tiles,
 * two for 128-column tiles). For leaving compute units to concurrent work,
 * or for making each workgroup walk many tiles. The output bytes do not
 * depend on it. NVQ_ERR_DIM below 0 or above 1024. */

/* ------------------------------------------------------------------------ */
/* MXFP8 requantization for the backward ([AIC] "Key Takeaways": MXFP8       */
/* backward with re-quantization and stochastic rounding). E4M3 elements,    */
/* one E8M0 scale per 32; shared exponent floor(log2 amax) - 8 (clamped to   */
/* [-127,127]); elements saturate at 448; an all-zero block is all zeros.    */
/* axis 0: blocks along each row; elems [R, C], scales [R, C/32], C % 32 == 0.*/
/* axis 1: blocks along the rows of each segment [seg_offsets[s],            */
/*   seg_offsets[s+1]) (nseg segments; NULL = one segment [0,R)), restarting */
/*   at each segment; output transposed: elems [C, ld], scales [C, ld/32],   */
/*   segment s occupying columns [pad_s, pad_s + 32*ceil(n_s/32)) with zero  */
/*   padding, zeros after the last segment; ld % 32 == 0 and                 */
/*   ld >= mxfp8_axis1_ld(R, nseg) = 128*ceil((R + 31*nseg)/128) (a multiple */
/*   of 128 keeps every row of scales a whole number of 32-bit words).       */
/* Row r of the logical tensor reads source row row_gather[r] / gather_div   */
/* when row_gather is not NULL. The SR draw of element (r, c) is keyed by    */
/* (seed, stream_id, r*C + c). scale_rule 0: the shared exponent above;     */
/* scale_rule 1: ceil(log2(amax / 448)) (clamped likewise), so no element    */
/* saturates; any other value NVQ_ERR_UNSUPPORTED.                           */
/* ------------------------------------------------------------------------ */
int64_t mxfp8_axis1_ld(int64_t R, int64_t nseg);
size_t mxfp8_requant_workspace_size(int64_t R, int64_t nseg);
int mxfp8_requant_sr(const uint16_t* x, int64_t R, int64_t C, int axis,
                     const int32_t* row_gather, int32_t gather_div,
                     const int32_t* seg_offsets, int64_t nseg, int64_t ld,
                     int round_mode, int scale_rule, uint64_t seed, uint32_t stream_id,
                     uint8_t* elems, uint8_t* scales,
                     void* ws, size_t ws_bytes, nvq_stream_t stream);

/* E8M0-scaled FP8 grouped GEMMs of the expert backward, fp32 accumulate and
 * fp32 output (gfx950 block-scaled MFMA; the E8M0 bytes go to the hardware).
 * Operands are MXFP8 as produced by mxfp8_requant_sr: elems [rows, lde] and
 * scales [rows, lde / 32] (lde = the row stride), K contiguous.
 *  NVQ_DGRAD: for each expert e and row r in [seg[e], seg[e+1]):
 *             out[r][n] = sum_{k<K} A[r][k] * B[n][e*K + k],  out [R, N]
 *             (A: axis-0 quantized rows, lda >= K; B: an axis-1 quantized
 *             stack of E weight matrices with no padding, ldb >= E*K).
 *  NVQ_FWD:   as NVQ_DGRAD with B expert-major, the layout in which the
 *             weights are stored: out[r][n] = sum_{k<K} A[r][k] * B[e*N + n][k]
 *             (B: axis-0 quantized rows of the stacked [E*N, K] weights,
 *             ldb >= K): the forward GEMMs on the FP8 matrix pipe, whose
 *             in-block alignment can exceed the fp32-output tolerance on
 *             heavy-tailed operands; moe_expert_fwd_mxfp8 below uses exact
 *             bf16 dequantization instead.
 *  NVQ_WGRAD: for each expert e: out[e][m][n] = sum over the padded K range of
 *             segment e (32*ceil((seg[e+1]-seg[e])/32) columns starting at
 *             the sum of the earlier segments' padded lengths) of A[m][k]*B[n][k],
 *             out [E, M, N] (A, B: axis-1 quantized with the same segments).
 * seg_offsets [E+1] are the token-row segment offsets (moe_route's offsets).
 * Limits: N % 128 == 0; WGRAD M % 128 == 0; DGRAD K % 32 == 0; E <= 4096;
 * element and output pointers 16-byte aligned (else NVQ_ERR_ALIGN).
 * Fast path: lda % 128 == 0, ldb % 128 == 0 (mxfp8_axis1_ld gives that),
 * 4-byte aligned scale pointers and, for DGRAD and FWD, K % 128 == 0; other
 * shapes take a masked path with the same results. */
size_t moe_grouped_gemm_mxfp8_workspace_size(int mode, int64_t E, int64_t R);
int moe_grouped_gemm_mxfp8(int mode, const uint8_t* a_elems, const uint8_t* a_scales,
                           const uint8_t* b_elems, const uint8_t* b_scales,
                           const int32_t* seg_offsets, int64_t lda, int64_t ldb, int64_t E,
                           int64_t M, int64_t N, int64_t K, float* out,
                           void* ws, size_t ws_bytes, nvq_stream_t stream);

/* SwiGLU backward for h = silu(g) * u from the bf16 g,u saved by the forward
 * (gu [n, 2*d_ff], gate half first): dA [n, 2*d_ff] bf16 with
 *   dA[:, j] = dh * u * s * (1 + g * (1 - s)),  dA[:, d_ff + j] = dh * g * s,
 *   s = 1 / (1 + exp(-g)), computed in fp32; dH [n, d_ff] fp32. */
int swiglu_bwd(const float* dH, const uint16_t* gu, int64_t n, int64_t d_ff, uint16_t* dA,
               nvq_stream_t stream);

/* ------------------------------------------------------------------------ */
/* MXFP8 forward through the expert layers: the same chain as                */
/* moe_expert_fwd_nvfp4 with MXFP8 operands, the precision the NVFP4 forward */
/* is compared against ([AIC] "Key Takeaways": versus full MXFP8 training)   */
/* and that the last layers keep ([AIC] "Architecture highlights").          */
/*   Xq = MXFP8 (nearest even, blocks along d) of X [T, d] (per-row blocks:  */
/*        the bytes of the expert-sorted row r are those of token            */
/*        sorted2assign[r] / k)                                              */
/*   G  = Xq . W1_e^T per expert, rows [0,d_ff) gate, [d_ff,2d_ff) up        */
/*   H  = bf16(g * u * sigmoid(g)) in fp32 (the fc1 epilogue)                */
/*   Hq = MXFP8 (nearest even, blocks along d_ff) of H                       */
/*   y[sorted2assign[r]] = bf16(Hq . W2_e^T)                                  */
/* Both GEMMs form every operand value e4m3 * 2^(e8m0 - 127) exactly in      */
/* bf16 and accumulate bf16 MFMA products in fp32 (exact for every block     */
/* whose largest magnitude is at least 2^-116; smaller blocks round to bf16  */
/* subnormals). Weights: w1 elems [E*2*d_ff, d], scales [E*2*d_ff, d/32];    */
/* w2 elems [E*d, d_ff], scales [E*d, d_ff/32] (mxfp8_requant_sr, axis 0, of */
/* the stacked weights). Rows of y whose expert id is out of range are left  */
/* untouched. Limits: d % 128 == 0, d_ff % 128 == 0, 1 <= k <= E <= 4096,    */
/* T*k < 2^31, T*d, T*k*d_ff and 2*d*d_ff below 2^32 (else NVQ_ERR_DIM); x, */
/* y and the element arrays 16-byte aligned, ws 256-byte aligned (else       */
/* NVQ_ERR_ALIGN).                                                           */
/* ------------------------------------------------------------------------ */
size_t moe_expert_fwd_mxfp8_workspace_size(int64_t T, int64_t d, int k, int64_t E, int64_t d_ff);
int moe_expert_fwd_mxfp8(const uint16_t* x, int64_t T, int64_t d, const int32_t* topk_ids, int k, int64_t E,
                         int64_t d_ff, const uint8_t* w1_elems, const uint8_t* w1_scales,
                         const uint8_t* w2_elems, const uint8_t* w2_scales, uint16_t* y,
                         void* ws, size_t ws_bytes, nvq_stream_t stream);

/* Stages of moe_expert_fwd_mxfp8 (workspace: moe_fc1_workspace_size(T*k, E),
 * moe_fc2_workspace_size(A, E); workgroups as for the NVFP4 stages).
 * fc1 + SwiGLU: h[r] = bf16(swiglu(deq(Xq[sorted2assign[r] / k]) . deq(W1q_e)^T))
 * for the rows r < offsets[E] (x elems [T, d], scales [T, d/32]); gu
 * (nullable) receives bf16 g and u [A, 2*d_ff]. */
int moe_fc1_swiglu_mxfp8(const uint8_t* x_elems, const uint8_t* x_scales, int64_t T, int64_t d,
                         const int32_t* offsets, const int32_t* sorted2assign, int k, int64_t E, int64_t d_ff,
                         const uint8_t* w1_elems, const uint8_t* w1_scales, uint16_t* h, uint16_t* gu,
                         int workgroups, void* ws, size_t ws_bytes, nvq_stream_t stream);
/* fc2: y[sorted2assign[r]] = bf16(deq(Hq[r]) . deq(W2q_e)^T) for r < offsets[E]
 * (h elems [A, d_ff], scales [A, d_ff/32]). */
int moe_fc2_mxfp8(const uint8_t* h_elems, const uint8_t* h_scales, int64_t A, int64_t d_ff,
                  const int32_t* offsets, const int32_t* sorted2assign, int64_t E, int64_t d,
                  const uint8_t* w2_elems, const uint8_t* w2_scales, uint16_t* y, int workgroups,
                  void* ws, size_t ws_bytes, nvq_stream_t stream);

/* SwiGLU forward on an fp32 G [n, 2*d_ff] (gate half first, e.g. the output
 * of moe_grouped_gemm_mxfp8 in NVQ_FWD mode) -> H [n, d_ff] bf16, h = g * u / (1 + exp(-g)) in fp32 with
 * the hardware reciprocal and exponential, nearest-even to bf16.
 * Limits: d_ff % 8 == 0, n*d_ff/8 < 2^31; G, H 16-byte aligned. */
int swiglu_fwd(const float* G, int64_t n, int64_t d_ff, uint16_t* H, nvq_stream_t stream);

/* ------------------------------------------------------------------------ */
/* 32-point random Hadamard transform + NVFP4 of the combine tensor ([AIC]   */
/* "Key Takeaways", "Architecture highlights"). z = (1/sqrt 32) H32 (s .* x) */
/* per contiguous 32-element chunk, one sign vector s (bit j of Philox word 0*/
/* at counter (0,0,4,0), key sign_seed; set bit = -1), fp32 butterfly with  */
/* strides 1,2,4,8,16, then the NVFP4 rule above with one scale over all z.  */
/* y [R, C], C % 32 == 0 -> codes [R, C/2], scales [R, C/16], tscale [1].    */
/* ------------------------------------------------------------------------ */
size_t rht32_blockquant_workspace_size(int64_t R, int64_t C);
int rht32_blockquant(const uint16_t* y, int64_t R, int64_t C, uint64_t sign_seed,
                     uint8_t* codes, uint8_t* scales, float* tscale,
                     void* ws, size_t ws_bytes, nvq_stream_t stream);

/* Dequantize rows t*k+s of the RHT-quantized tensor, invert the transform
 * (H32/sqrt(32) then the signs) and combine: out[t] = sum_s w[t][s] * y'_s,
 * rounded to bf16. The inverse transform is linear, so it is applied once to
 * the fp32 weighted sum of the dequantized slots (accumulated in slot order
 * with fused multiply-adds) rather than to every slot.
 * codes [T*k, C/2], scales [T*k, C/16], tscale [1], w [T, k] fp32, out [T, C].
 * Limits: C % 32 == 0, k >= 1, T*k*C/8 < 2^31 (else NVQ_ERR_DIM); codes and
 * out 16-byte aligned, scales 2-byte aligned (else NVQ_ERR_ALIGN).          */
int rht32_dequant_combine(const uint8_t* codes, const uint8_t* scales, const float* tscale,
                          int64_t T, int k, int64_t C, uint64_t sign_seed, const float* w,
                          uint16_t* out, nvq_stream_t stream);

/* ------------------------------------------------------------------------ */
/* NVFP4 backward of the expert layers: the backward in the forward's 4-bit  */
/* format, which the pages name as their next step ([AIC] "Developer quick  */
/* start": exploring FP4 backward passes), with the recipe's companions:     */
/* stochastic rounding for the gradients ([AIC] "Key Takeaways") and the     */
/* 32-point random Hadamard transform ([AIC] "Architecture highlights") on   */
/* both operands of each weight gradient, along the token axis, where the    */
/* orthogonal transform cancels in the product.                              */
/* ------------------------------------------------------------------------ */

/* Transposed, segment-padded NVFP4 layout: row c of the [C, ld] output holds
 * column c of the input; segment s (logical rows [seg[s], seg[s+1])) occupies
 * columns [pad_s, pad_s + 32*ceil(n_s/32)), pad_0 = 0, zero rows padding each
 * segment to a multiple of 32; columns past the last segment are zero.
 * nvfp4_axis1_ld(R, nseg) = 128*ceil((R + 31*nseg)/128) + 128 is a row length
 * with room for every segmentation of R rows plus the 128 columns of slack the
 * grouped GEMM's K steps read past a segment's end. */
int64_t nvfp4_axis1_ld(int64_t R, int64_t nseg);

/* Quantize bf16 x along its rows into that layout: codes [C, ld/2] (element j
 * of row c in nibble j%2 of byte j/2), scales [C, ld/16] (E4M3 per 16 along the
 * row), tscale. Logical row r reads row row_gather[r] / gather_div of x
 * (row_gather NULL: row r), x [*, C]. seg_offsets [nseg+1] (NULL: one segment
 * [0, R), nseg must be 1). rht != 0: every 32-value chunk of the segments goes
 * through z = (1/sqrt 32) H32 (s .* x) (as rht32_blockquant: the sign word of
 * sign_seed, fp32 butterfly with strides 1..16) before the NVFP4 rule, with one
 * tensor scale over all of z. round_mode NVQ_SR: the draw of output element
 * (c, j) is keyed by (seed, stream_id, c*ld + j). scale_per_segment != 0 (the
 * transposed weights of the dgrad GEMMs): nseg equal contiguous segments of
 * R/nseg rows each (a multiple of 32), one tensor scale per segment into
 * tscale[nseg]; requires seg_offsets and row_gather NULL, rht 0, NVQ_RTN and
 * ld == R (else NVQ_ERR_UNSUPPORTED / NVQ_ERR_DIM). Otherwise tscale[1] and
 * ld >= nvfp4_axis1_ld(R, nseg) - 128, ld % 32 == 0. nseg <= 4096.
 * codes 16-byte aligned, scales 2-byte aligned, ws 256-byte aligned. */
size_t nvfp4_quantize_axis1_workspace_size(int64_t R, int64_t C, int64_t nseg);
int nvfp4_quantize_axis1(const uint16_t* x, int64_t R, int64_t C, const int32_t* row_gather,
                         int32_t gather_div, const int32_t* seg_offsets, int64_t nseg, int64_t ld,
                         int rht, uint64_t sign_seed, int scale_per_segment, int round_mode,
                         uint64_t seed, uint32_t stream_id, uint8_t* codes, uint8_t* scales,
                         float* tscale, void* ws, size_t ws_bytes, nvq_stream_t stream);

/* Grouped NVFP4 GEMMs of the backward, fp32 accumulate and output. Operand
 * values are dequantized exactly (e2m1 * e4m3 is an fp16 value) and contracted
 * with fp16 MFMA; the tensor scales apply once to each output.
 *  NVQ_DGRAD: for each expert e and sorted row r in [seg[e], seg[e+1]):
 *    out[r][n] = Da * Db[e] * sum_{k<K} A[arow][k] * B[n][e*K + k],
 *    arow = a_gather ? a_gather[r] : r. A codes [*, lda/2] (nvfp4_quantize of
 *    the gradient rows), B the transposed weights [N, ldb >= E*K] with one
 *    scale per expert (b_tscale [E]); M = the number of output rows
 *    (>= seg[E]); out [M, N]. K % 128 == 0, lda >= K; M * lda/2 and
 *    N * ldb/2 below 2^32, and with a_gather every arow * lda/2 below 2^32
 *    (32-bit operand offsets; the last is a precondition). Runs on the
 *    forward's grouped GEMM (256-row m-tiles of each expert's rows).
 *  NVQ_WGRAD: out[e][m][n] = Da * Db * sum over expert e's padded columns of
 *    A[m][k] * B[n][k]; A [M, lda], B [N, ldb] in the segment-padded layout
 *    above (the same seg_offsets), one scale each; K = the rows the segments
 *    cover (seg[E]); lda, ldb >= nvfp4_axis1_ld(K, E); M % 128 == 0;
 *    out [E, M, N] (an empty segment gives zeros).
 * N % 128 == 0, E <= 4096, lda and ldb multiples of 32; codes and out 16-byte
 * aligned, scales 2-byte aligned, ws 256-byte aligned. */
size_t moe_grouped_gemm_nvfp4_bwd_workspace_size(int mode, int64_t E, int64_t M);
int moe_grouped_gemm_nvfp4_bwd(int mode, const uint8_t* a_codes, const uint8_t* a_scales,
                               const float* a_tscale, const int32_t* a_gather,
                               const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tscale,
                               const int32_t* seg_offsets, int64_t lda, int64_t ldb, int64_t E,
                               int64_t M, int64_t N, int64_t K, float* out,
                               void* ws, size_t ws_bytes, nvq_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Converter checks. Every code, scale byte and bf16 output above comes from */
/* a handful of gfx950 conversion instructions (and two software encoders);  */
/* their exactness against the format rules (NVFP4 about 4.5 bits per value */
/* with E2M1 codes and E4M3 block scales, [AIC] "Background"; MXFP8 E4M3     */
/* elements, [AIC] "Key Takeaways"; nearest-even bf16) is what makes the     */
/* library's results bit-exact. This call runs those steps exactly as the    */
/* kernels do, so a test can compare them with the rules.                    */
/*  NVQ_CVT_DQ_F16:  in uint32 [n][2] = (8 E2M1 codes, element 0 in the low  */
/*    nibble; 4 E4M3 scale bytes); out uint16 [n][40] fp16 bits: the 4 scale */
/*    bytes as fp16, 4 zeros, then the 8 codes times scale j at 8 + 8j + q    */
/*    for j = 0..3 (the NVFP4 GEMMs' operand dequantization). 0 <= n <= 2^24; */
/*    out 16-byte aligned (else NVQ_ERR_ALIGN).                              */
/*  NVQ_CVT_FP4_F32: in uint32 [n] (8 codes) -> out float [n][8].            */
/*  NVQ_CVT_SR: in uint32 [n][2] = (fp32 bits of y, 16-bit draw u) -> out    */
/*    uint32 [n]: the stochastic E2M1 code of y (bits 0-3) and the           */
/*    stochastic E4M3 byte of y (bits 8-15), as the SR encoders decide them  */
/*    (both by the gfx950 stochastic converters; the E2M1 code with y in     */
/*    all eight positions of one call, bit 31 set if those disagree), and    */
/*    the E2M1 code (bits 16-19) and E4M3 byte (bits 20-27) of the software  */
/*    form of the same rule.                                                 */
/*  NVQ_CVT_SR_E2M1_SWEEP / NVQ_CVT_SR_E4M3_SWEEP: in unused; n must be 4;   */
/*    out uint64 [4]: the converter and software forms above compared on the */
/*    device for every fp32 y with |y| <= 8 (E2M1) or <= 512 (E4M3), both    */
/*    signs: [0] values whose codes at draws 0 and 65535 or whose first      */
/*    changing draw differ, [1] values whose code depends on the draw, [2]   */
/*    differing (value, draw) pairs over all 65536 draws of every 65521st    */
/*    value, [3] such values. A second or two each.                          */
/*  NVQ_CVT_SCAN_*: in unused; n must be 65536; out uint32 [65536][18]. Row  */
/*    t covers the fp32 bit patterns [t*2^16, (t+1)*2^16) of one encoder:    */
/*    word 0 = output at the first pattern, word 1 = number of output        */
/*    changes in the range (bit 31 set when above 8, or when the two values  */
/*    of one converter call disagreed), words 2..9 the first 8 patterns      */
/*    where the output changes, words 10..17 the new outputs. Rows of the    */
/*    infinity/NaN patterns hold zeros. Encoders: E2M1 code (with sign bit)  */
/*    by the fp32 -> fp4 converter; E4M3 byte by the +-448 clamp and the     */
/*    fp32 -> fp8 converter (MXFP8 nearest-even elements), and by the        */
/*    software encoder of block scales; bf16 bits by the pair converter and  */
/*    by the software rounding.                                              */
/*  NVQ_CVT_DQ_MX_BF16: in unused; n must be 256; out uint16 [256][256]: row */
/*    e, column c = bf16 bits of E4M3 byte c times 2^(e - 127) as the MXFP8   */
/*    GEMMs of moe_expert_fwd_mxfp8 form their operands.                     */
/*  NVQ_CVT_E4M3_PAIR_F32: in unused; n must be 65536; out float [65536][2]: */
/*    pair i (byte 0 = i & 0xFF, byte 1 = i >> 8) as fp32, decoded as        */
/*    rht32_dequant_combine decodes its two block scales per 32 values.      */
/* Returns NVQ_ERR_UNSUPPORTED for an unknown `which`.                       */
/* ------------------------------------------------------------------------ */
enum {
    NVQ_CVT_DQ_F16 = 0,
    NVQ_CVT_FP4_F32 = 1,
    NVQ_CVT_SCAN_E2M1 = 2,
    NVQ_CVT_SCAN_E4M3_HW = 3,
    NVQ_CVT_SCAN_E4M3_SW = 4,
    NVQ_CVT_SCAN_BF16_HW = 5,
    NVQ_CVT_SCAN_BF16_SW = 6,
    NVQ_CVT_SR = 7,
    NVQ_CVT_DQ_MX_BF16 = 8,
    NVQ_CVT_SR_E2M1_SWEEP = 9,
    NVQ_CVT_SR_E4M3_SWEEP = 10,
    NVQ_CVT_E4M3_PAIR_F32 = 11
};
int nvq_convert_probe(int which, const void* in, int64_t n, void* out, nvq_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif
