// nvq_bwd4.hip -- the expert-layer backward in NVFP4 on gfx950: the
// transposed, segment-padded NVFP4 quantizer (with the 32-point random
// Hadamard transform along the token axis for the weight-gradient operands)
// and the grouped dgrad / wgrad GEMMs on exactly dequantized operands.
//
// The pages run only the forward in NVFP4 and name FP4 backward passes as the
// next step (page "Thinking Machines Details End-to-End 4-Bit Training for
// Inkling 2 Small", section "Developer quick start"). This is that backward in
// the forward's format, with the recipe's companions: stochastic rounding for
// the gradients (section "Key Takeaways") and the combine's 32-point RHT
// ("Architecture highlights") on both operands of each weight gradient,
// along the token axis, where it cancels in the product.
//
// Layouts. dgrad operands are NVFP4 along the contraction axis: the gradient
// rows as nvfp4_quantize writes them, the weights transposed (expert e's
// K x N matrix at columns [e K, (e+1) K) of an [N, >= E K] tensor, one tensor
// scale per expert). wgrad operands are [C, ld]: column block s holds segment
// s's rows, padded with zero rows to a multiple of 32, one tensor scale over
// the whole tensor.
#include <algorithm>

#include "nvq_device.hpp"
#include "nvq_host.hpp"

namespace nvq {

// ------------------------------------------------------------------ axis-1 quantizer
// A 256-thread workgroup takes a tile of 256 padded rows (eight 32-row
// chunks, padded output columns [256 g, 256 g + 256)) x 64 input columns:
//  - load: every thread issues eight 16-byte row loads (thread t: tile row
//    32 k + t / 8, columns 8 (t % 8) .. + 7), 32 KiB in flight per workgroup,
//    gathered or padding rows resolved per chunk, into a row-major LDS tile;
//  - encode: thread (column pair p = t % 32, chunk b = t / 32) reads its two
//    columns' 32 values with 32-bit LDS reads, applies the RHT, encodes;
//  - store: the codes go back through LDS so that every 16-byte store
//    instruction covers eight whole 128-byte output lines (a column's eight
//    chunks are one line), and a column's 16 scale bytes leave together.
// Tiles are remapped so that each XCD walks contiguous row groups.
constexpr int kA1MaxBlocks = 2048;            // persistent grid of the maximum pass
constexpr int kA1TileRows = 256, kA1TileCols = 64;
constexpr int kA1CodeStride = 144;            // bytes per column in the code exchange (128 + 16: spreads banks)

struct A1Args {
    const uint16_t* x;
    int R, C;
    const int32_t* gather;  // nullable: logical row r reads row gather[r] / gdiv
    int gdiv;
    const int32_t* seg;     // nullable: then nseg equal segments of seg_rows rows, seg_pad columns each
    const int32_t* pad;     // [nseg + 1] padded segment starts (with seg)
    const int2* chunks;     // with seg: rows [x, y) of padded chunk c (x == y: past the last segment)
    int nchunks;            // entries of chunks
    int nseg;
    int seg_rows, seg_pad;
    int ld;
    int groups;             // ceil(ld / 256)
    int tiles;              // groups * ctiles
    int ctiles;             // ceil(C / 64)
    uint64_t sign_seed;
    bool wide_scales;       // a column's 16 scale bytes may go out as two 8-byte stores
};

// Rows [*r0, *r1) of the chunk at padded column col and its segment, or
// false for a column past the last segment. With several segments starting
// at col (empty ones before a non-empty one) the last is the one holding rows.
__device__ __forceinline__ bool a1_chunk_rows(const A1Args& p, int col, int* s_out, int* r0, int* r1) {
    if (!p.seg) {
        const int s = col / p.seg_pad;
        if (s >= p.nseg) return false;
        *s_out = s;
        *r0 = s * p.seg_rows + (col - s * p.seg_pad);
        *r1 = (s + 1) * p.seg_rows;
        return true;
    }
    // one load from the chunk table (launch_chunk_rows) rather than a binary
    // search of dependent loads over the padded starts; the segment index is
    // not needed with explicit segments (one tensor scale)
    if ((col >> 5) >= p.nchunks) return false;
    const int2 e = p.chunks[col >> 5];
    *s_out = 0;
    *r0 = e.x;
    *r1 = e.y;
    return e.x < e.y;
}


__device__ __forceinline__ int a1_tile_of(const A1Args& p, int id, int G) {
    // consecutive tiles on one XCD (workgroups are dealt to the 8 XCDs round robin)
    const int G8 = G / 8 * 8;
    return id < G8 ? (id % 8) * (G8 / 8) + id / 8 : id;
}

// Load tile (g, ct) into the row-major bf16 LDS tile [256][64]. NT: whole
// 16-byte pieces with the non-temporal hint where the encode pass reads each
// source byte once (not with a gather divisor above 1, whose source rows are
// read by several rows and should stay cached).
template <bool NT = false>
__device__ __forceinline__ void a1_load_tile(const A1Args& p, int g, int c0, uint16_t* tile) {
    const int t = threadIdx.x;
    const int cc = c0 + 8 * (t & 7);
    const bool full = cc + 8 <= p.C && (p.C & 7) == 0;
    const bool nt = NT && p.gdiv == 1;
    uint4 w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        // tile rows 32 k .. 32 k + 31 are chunk k (uniform)
        int s, r0, r1;
        const bool used = a1_chunk_rows(p, 256 * g + 32 * k, &s, &r0, &r1);
        const int r = r0 + (t >> 3);
        w[k] = make_uint4(0u, 0u, 0u, 0u);
        if (used && r < r1 && cc < p.C) {
            const int64_t src = p.gather ? (int64_t)(p.gather[r] / p.gdiv) : (int64_t)r;
            const uint16_t* rp = p.x + src * p.C + cc;
            if (full) {
                w[k] = nt ? load_stream(reinterpret_cast<const uint4*>(rp)) : *reinterpret_cast<const uint4*>(rp);
            } else {
                uint16_t e[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = cc + i < p.C ? rp[i] : (uint16_t)0;
                w[k] = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                                  e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
        *reinterpret_cast<uint4*>(tile + (32 * k + (t >> 3)) * kA1TileCols + 8 * (t & 7)) = w[k];
}

// The 32 values of columns 2 cp and 2 cp + 1 of chunk b from the LDS tile;
// with RHT, signs, butterfly and 1/sqrt 32 follow.
template <bool RHT>
__device__ __forceinline__ void a1_columns(const uint16_t* tile, int cp, int b, uint32_t signs, float (&v0)[32],
                                           float (&v1)[32]) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const uint32_t pr = *reinterpret_cast<const uint32_t*>(tile + (32 * b + j) * kA1TileCols + 2 * cp);
        float x0 = bf16_to_f32(pr & 0xFFFFu), x1 = bf16_to_f32(pr >> 16);
        if (RHT && ((signs >> j) & 1u)) {
            x0 = -x0;
            x1 = -x1;
        }
        v0[j] = x0;
        v1[j] = x1;
    }
    if (RHT) {
        butterfly32(v0);
        butterfly32(v1);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            v0[j] *= kInvSqrt32;
            v1[j] *= kInvSqrt32;
        }
    }
}

// Pass 1 (one tensor scale): max |value| over every tile, one partial
// maximum per workgroup of a persistent grid (plain store).
template <bool RHT>
__global__ __launch_bounds__(256) void k_a1_amax(A1Args p, uint32_t* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[kA1TileRows * kA1TileCols];
    const int t = threadIdx.x, cp = t & 31, b = t >> 5;
    const uint32_t signs = RHT ? rht_sign_word(p.sign_seed) : 0u;
    float m = 0.0f;
    for (int id = blockIdx.x; id < p.tiles; id += gridDim.x) {
        const int v = id;  // order does not matter for a maximum
        const int g = v / p.ctiles, c0 = (v - g * p.ctiles) * kA1TileCols;
        __syncthreads();  // the previous tile is consumed
        a1_load_tile(p, g, c0, tile);
        __syncthreads();
        float v0[32], v1[32];
        a1_columns<RHT>(tile, cp, b, signs, v0, v1);
#pragma unroll
        for (int j = 0; j < 32; ++j) m = fmaxf(m, fmaxf(fabsf(v0[j]), fabsf(v1[j])));
    }
    const uint32_t mb = block_max_u32(__float_as_uint(m));
    if (threadIdx.x == 0) part[blockIdx.x] = mb;
}

// The multiplier of each block is nvfp4_scale_mult(byte, S), divided per
// block: a thread encodes four blocks per tile, as many divisions as a
// 128-entry table per chunk would cost it, and without the table the
// workgroup's LDS is the 32 KiB tile alone (five workgroups per CU).
// FAST: the scale byte's quotient by div6_fma.
template <int MODE, bool FAST>
__device__ __forceinline__ void a1_encode_col(const float (&v)[32], float S, uint64_t unit0,
                                              uint32_t stream_id, uint64_t seed, uint4* code, uint32_t* scale) {
    uint32_t word[4], sc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const float* z = v + 16 * blk;
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(z[i]));
        sc[blk] = nvfp4_scale_byte_hw<FAST>(am, S);
        const float r = nvfp4_scale_mult(sc[blk] & 0x7Fu, S);  // byte <= 0x7E for finite inputs
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
            const float* zz = z + 8 * hw;
            uint32_t wd = 0;
            if (MODE == NVQ_RTN) {
                wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, zz[0] * r, zz[1] * r, 1.0f, 0);
                wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, zz[2] * r, zz[3] * r, 1.0f, 1);
                wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, zz[4] * r, zz[5] * r, 1.0f, 2);
                wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, zz[6] * r, zz[7] * r, 1.0f, 3);
            } else {
                const float y[8] = {zz[0] * r, zz[1] * r, zz[2] * r, zz[3] * r,
                                    zz[4] * r, zz[5] * r, zz[6] * r, zz[7] * r};
                wd = e2m1_sr8_hw(y, draws8(unit0 + 2 * blk + hw, stream_id, seed));
            }
            word[2 * blk + hw] = wd;
        }
    }
    *code = make_uint4(word[0], word[1], word[2], word[3]);
    *scale = sc[0] | (sc[1] << 8);
}

// The thread's two columns of chunk b, one after the other (registers for
// one column at a time), encoded into code[h] / sc[h] for column 2 cp + h.
template <bool RHT, int MODE, bool FAST>
__device__ __forceinline__ void a1_encode_cols(const A1Args& p, const uint16_t* tile, int cp,
                                               int b, int c0, int col, bool live, float S, uint32_t signs,
                                               uint32_t stream_id, uint64_t seed, uint4 (&code)[2],
                                               uint32_t (&sc)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        code[h] = make_uint4(0u, 0u, 0u, 0u);
        sc[h] = 0u;
    }
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
        const int cl = 2 * cp + h;
        if (live) {
            float vv[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                float x = bf16_to_f32(tile[(32 * b + j) * kA1TileCols + cl]);
                if (RHT && ((signs >> j) & 1u)) x = -x;
                vv[j] = x;
            }
            if (RHT) {
                butterfly32(vv);
#pragma unroll
                for (int j = 0; j < 32; ++j) vv[j] *= kInvSqrt32;
            }
            // element (c, j) draws with index c * ld + j
            uint4 cd;
            uint32_t sw;
            a1_encode_col<MODE, FAST>(vv, S, (uint64_t)(((int64_t)(c0 + cl) * p.ld + col) / 8), stream_id,
                                      seed, &cd, &sw);
            // register arrays indexed by the loop counter stay in registers
            // only with constant indices
            if (h == 0) { code[0] = cd; sc[0] = sw; } else { code[1] = cd; sc[1] = sw; }
        }
    }
}

// Between the passes: workgroup s folds the partial maxima of segment s
// (part[s * n_part, + n_part); one segment without per-segment scales) into
// fold[s] and writes its tensor scale, so that every encode workgroup reads
// one word instead of folding all partials itself before its tile load.
__global__ __launch_bounds__(256) void k_a1_fold(const uint32_t* __restrict__ part, int n_part,
                                                 uint32_t* __restrict__ fold, float* __restrict__ tscale) {
    const int s = blockIdx.x;
    const float amax = block_max_partials(part + (int64_t)s * n_part, n_part);
    if (threadIdx.x == 0) {
        fold[s] = __float_as_uint(amax);
        tscale[s] = nvfp4_decode_scale(amax);
    }
}

// Pass 2: encode, one tile per workgroup, with the maximum of its chunk's
// segment (per_seg) or of the whole tensor from fold.
template <bool RHT, int MODE>
__global__ __launch_bounds__(256) void k_a1_encode(A1Args p, const uint32_t* __restrict__ fold, bool per_seg,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                   uint64_t seed, uint32_t stream_id) {
    // the code exchange reuses the tile's memory once every value is read
    // (32 KiB of LDS in all: five workgroups per CU)
    __shared__ __attribute__((aligned(16))) uint16_t tile[kA1TileRows * kA1TileCols];
    static_assert(kA1TileCols * kA1CodeStride + kA1TileCols * 16 <= (int)sizeof(tile), "exchange fits the tile");
    uint8_t* ex = reinterpret_cast<uint8_t*>(tile);
    const int t = threadIdx.x, cp = t & 31, b = t >> 5;
    const uint32_t signs = RHT ? rht_sign_word(p.sign_seed) : 0u;
    // the one-scale maximum goes out with the tile's loads (its latency
    // overlaps theirs)
    float amax = per_seg ? 0.0f : __uint_as_float(fold[0]);
    const int v = a1_tile_of(p, blockIdx.x, gridDim.x);
    const int g = v / p.ctiles, c0 = (v - g * p.ctiles) * kA1TileCols;
    a1_load_tile<true>(p, g, c0, tile);
    const int col = 256 * g + 32 * b;  // this thread's chunk
    int s = 0, r0, r1;
    const bool used = col < p.ld && a1_chunk_rows(p, col, &s, &r0, &r1);
    if (per_seg && used) amax = __uint_as_float(fold[s]);
    const float S = nvfp4_encode_scale(amax);
    __syncthreads();  // the tile is in LDS
    // the FMA quotient where the chunk's S allows it (uniform over a wave in
    // practice: its two chunks share a tensor scale unless they lie in two
    // segments; a wave with both kinds takes both paths, each exact)
    uint4 code[2];
    uint32_t sc[2];
    if (S <= kFastDiv6MaxS)
        a1_encode_cols<RHT, MODE, true>(p, tile, cp, b, c0, col, used && amax > 0.0f, S, signs,
                                        stream_id, seed, code, sc);
    else
        a1_encode_cols<RHT, MODE, false>(p, tile, cp, b, c0, col, used && amax > 0.0f, S, signs,
                                         stream_id, seed, code, sc);
    __syncthreads();  // every tile value has been read
    uint8_t* exs = ex + kA1TileCols * kA1CodeStride;  // [64 columns][16 scale bytes]
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int cl = 2 * cp + h;
        *reinterpret_cast<uint4*>(ex + cl * kA1CodeStride + 16 * b) = code[h];
        *reinterpret_cast<uint16_t*>(exs + cl * 16 + 2 * b) = (uint16_t)sc[h];
    }
    __syncthreads();
    const int nb = min(8, (p.ld - 256 * g) / 32);  // chunks of this group inside the row
    const int64_t ldb = p.ld / 2, lds_ = p.ld / 16;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        // 16-byte piece q of the 64 columns x 8 pieces: column q / 8, piece q % 8
        const int q = 256 * k + t, c = q >> 3, pc = q & 7;
        if (c0 + c < p.C && pc < nb)
            *reinterpret_cast<uint4*>(codes + (int64_t)(c0 + c) * ldb + 128 * (int64_t)g + 16 * pc) =
                *reinterpret_cast<const uint4*>(ex + c * kA1CodeStride + 16 * pc);
    }
    if (t < kA1TileCols && c0 + t < p.C) {
        uint8_t* sp = scales + (int64_t)(c0 + t) * lds_ + 16 * (int64_t)g;
        const uint16_t* sv = reinterpret_cast<const uint16_t*>(exs + t * 16);
        if (nb == 8 && p.wide_scales) {
            reinterpret_cast<uint2*>(sp)[0] = *reinterpret_cast<const uint2*>(sv);
            reinterpret_cast<uint2*>(sp)[1] = *reinterpret_cast<const uint2*>(sv + 4);
        } else {
#pragma unroll
            for (int ch = 0; ch < 8; ++ch)
                if (ch < nb) reinterpret_cast<uint16_t*>(sp)[ch] = sv[ch];
        }
    }
}

// ------------------------------------------------------------------ grouped GEMM
// C = deq(A) deq(B)^T per expert with fp32 accumulation, for the two weight-
// and data-gradient shapes:
//   DGRAD: out[r][n] = sum_k A[arow(r)][k] B[n][e K + k] for the sorted rows r
//          of expert e (arow = gather[r] or r), times Da * Db[e];
//   WGRAD: out[e][m][n] = sum over expert e's padded token range of A[m][k]
//          B[n][k], times Da * Db.
// Every operand value e2m1 * e4m3 is an exact fp16 (at most 6 significant
// bits in [2^-10, 2688]): codes and scale bytes go through the gfx950
// converters and one packed fp16 multiply (the forward's dequantization),
// land in LDS as fp16, and feed v_mfma_f32_32x32x16_f16.
//
// Tile 128 x 128 per 256-thread workgroup (four waves of 64 x 64, 2 x 2 MFMA
// blocks each), K steps of 128. Thread t stages half a row (64 values: 32
// code bytes and 4 scale bytes) of each operand per step; the next step's
// codes are loaded into registers before the current step's MFMAs, so the
// global loads are in flight while the matrix cores run. LDS rows are 256
// bytes; 16-byte chunk c of row r sits at chunk c ^ (r & 15), so both the
// staging writes (8 rows x 2 halves per 16 lanes) and the operand reads (16
// rows per 16 lanes) fall on distinct banks.
constexpr int kBT = 128;
constexpr int kBK = 128;
constexpr int kBRowB = kBK * 2;        // fp16 bytes of one staged row
constexpr int kBOpB = kBT * kBRowB;    // 32 KiB per operand

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct BwArgs {
    const uint8_t* ac;
    const uint8_t* as;
    int64_t lda;            // values per A row
    const uint8_t* bc;
    const uint8_t* bs;
    int64_t ldb;
    const float* ats;       // [1]
    const float* bts;       // [1]
    const int32_t* seg;     // [E + 1] token-row segments
    const int32_t* tiles;   // padded K offsets [E + 1]
    float* out;
    int E, M, N, K;
    int n_tiles, m_tiles;
};

__device__ __forceinline__ uint32_t bw_lds_off(int row, int chunk) {
    return (uint32_t)(row * kBRowB + ((chunk ^ (row & 15)) << 4));
}

struct BwStage {
    uint4 c0, c1;
    uint32_t sw;
    uint32_t keep;  // the scale bytes of blocks inside the K range
};

// Half a row of one step: codes of values [k, k + 64) relative to the row's
// K base, and their 4 scale bytes; blocks at or past k_end get scale 0 (so
// their values are exact zeros whatever the codes), a row outside the
// operand reads nothing. The range mask is applied when the stage is
// written to LDS, not here: a use of the loaded word right after its load
// would make the wave wait for it before the step's MFMAs.
__device__ __forceinline__ void bw_load(BwStage& st, const uint8_t* rc, const uint8_t* rs, int k, int k_end,
                                        bool row_ok) {
    st.c0 = make_uint4(0u, 0u, 0u, 0u);
    st.c1 = st.c0;
    st.sw = 0u;
    st.keep = 0u;
    if (!row_ok || k >= k_end) return;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (k + 16 * j < k_end) st.keep |= 0xFFu << (8 * j);
    const uint4* cp = reinterpret_cast<const uint4*>(rc + k / 2);
    st.c0 = cp[0];
    st.c1 = cp[1];
    const uint16_t* sp = reinterpret_cast<const uint16_t*>(rs + k / 16);  // 2-byte aligned (k % 32 == 0)
    st.sw = (uint32_t)sp[0] | ((uint32_t)sp[1] << 16);
}

__device__ __forceinline__ void bw_stage(uint8_t* lds, int row, int half, const BwStage& st) {
    const Scales s = word_scales(st.sw & st.keep, 0xFFFFFFFFu);
    const uint32_t w[8] = {st.c0.x, st.c0.y, st.c0.z, st.c0.w, st.c1.x, st.c1.y, st.c1.z, st.c1.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const _Float16 sc = q < 2 ? s.lo[0] : q < 4 ? s.lo[1] : q < 6 ? s.hi[0] : s.hi[1];
        *reinterpret_cast<uint4*>(lds + bw_lds_off(row, 8 * half + q)) = __builtin_bit_cast(uint4, dq8(w[q], sc));
    }
}

// wgrad: out[e] = deq(A)[:, seg e] . deq(B)[:, seg e]^T over expert e's
// padded token columns, tiles (expert, m-tile, n-tile).
struct BwTile {
    int e, nt, row0, row_end, k_len;
    int64_t a_off_c, a_off_s, b_off_c, b_off_s;
};

__device__ __forceinline__ BwTile bw_tile(const BwArgs& p, int tile, int srow) {
    BwTile T;
    const int per_e = p.m_tiles * p.n_tiles;
    T.e = tile / per_e;
    const int rem = tile - T.e * per_e;
    const int mt = rem / p.n_tiles;
    T.nt = rem - mt * p.n_tiles;
    T.row0 = mt * kBT;
    T.row_end = T.row0 + kBT;
    const int kb = p.tiles[T.e];
    T.k_len = p.tiles[T.e + 1] - kb;
    const int64_t m = T.row0 + srow, n = (int64_t)T.nt * kBT + srow;
    T.a_off_c = m * (p.lda / 2) + kb / 2;
    T.a_off_s = m * (p.lda / 16) + kb / 16;
    T.b_off_c = n * (p.ldb / 2) + kb / 2;
    T.b_off_s = n * (p.ldb / 16) + kb / 16;
    return T;
}

// Epilogue rows per pass and their LDS row stride (floats): a wave's 32 x 64
// block of one pass, padded so the two lane halves (4 rows apart) fall on
// different banks.
constexpr int kBEStride = 68;

__global__ __launch_bounds__(256, 2) void k_nvfp4_wgrad(BwArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBOpB];
    uint8_t* la = lds;
    uint8_t* lb = lds + kBOpB;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int srow = t >> 1, shalf = t & 1;
    const int l32 = lane & 31, lh = lane >> 5;
    const int total = p.E * p.m_tiles * p.n_tiles;
    const int G = gridDim.x;
    const int v = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    if (v >= total) return;
    const float scale = p.ats[0] * p.bts[0];
    // the first step's operands of a tile go out before the previous tile's
    // output stores: gfx9 counts loads and stores in one in-order counter, so
    // the wait for these loads then skips those stores
    BwTile T = bw_tile(p, v, srow);
    BwStage sa, sb;
    bw_load(sa, p.ac + T.a_off_c, p.as + T.a_off_s, 64 * shalf, T.k_len, T.row0 + srow < T.row_end);
    bw_load(sb, p.bc + T.b_off_c, p.bs + T.b_off_s, 64 * shalf, T.k_len, true);
    for (int tile = v; tile < total; tile += G) {
        const bool a_ok = T.row0 + srow < T.row_end;
        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        for (int k0 = 0; k0 < T.k_len; k0 += kBK) {
            __syncthreads();  // the previous step's operand reads (or the epilogue's) are done
            bw_stage(la, srow, shalf, sa);
            bw_stage(lb, srow, shalf, sb);
            __syncthreads();
            if (k0 + kBK < T.k_len) {
                bw_load(sa, p.ac + T.a_off_c, p.as + T.a_off_s, k0 + kBK + 64 * shalf, T.k_len, a_ok);
                bw_load(sb, p.bc + T.b_off_c, p.bs + T.b_off_s, k0 + kBK + 64 * shalf, T.k_len, true);
            }
#pragma unroll
            for (int q = 0; q < kBK / 16; ++q) {
                half8 av[2], bv[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    av[i] = *reinterpret_cast<const half8*>(la + bw_lds_off(wm * 64 + i * 32 + l32, 2 * q + lh));
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bv[j] = *reinterpret_cast<const half8*>(lb + bw_lds_off(wn * 64 + j * 32 + l32, 2 * q + lh));
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
            }
        }
        // the next tile (past the last one: this tile again, loads never used)
        // and its first loads
        const int e = T.e, nt = T.nt, row0 = T.row0, row_end = T.row_end;
        const int tn = tile + G < total ? tile + G : tile;
        T = bw_tile(p, tn, srow);
        bw_load(sa, p.ac + T.a_off_c, p.as + T.a_off_s, 64 * shalf, T.k_len, T.row0 + srow < T.row_end);
        bw_load(sb, p.bc + T.b_off_c, p.bs + T.b_off_s, 64 * shalf, T.k_len, true);
        // epilogue through LDS, one 32-row block of the wave at a time: lane l,
        // register r of a 32 x 32 block holds column l % 32, row 8 (r / 4) +
        // 4 (l / 32) + r % 4; each row's 64 columns of the wave (256 bytes)
        // then leave as 16 lanes' 16-byte non-temporal stores
        float* eb = reinterpret_cast<float*>(lds) + wave * 32 * kBEStride;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            __syncthreads();  // operand reads (i == 0) or the previous pass's reads are done
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 8 * (r >> 2) + (r & 3) + 4 * lh;
#pragma unroll
                for (int j = 0; j < 2; ++j) eb[lr * kBEStride + 32 * j + l32] = acc[i][j][r] * scale;
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int lr = 4 * k + (lane >> 4), c4 = lane & 15;  // row, 16-byte piece
                const int row = row0 + wm * 64 + i * 32 + lr;
                typedef float f32x4v __attribute__((ext_vector_type(4)));
                const f32x4v val = *reinterpret_cast<const f32x4v*>(eb + lr * kBEStride + 4 * c4);
                // every row is inside the tile (M is a multiple of the tile
                // height): stores without a branch, so the wait for the next
                // tile's first loads (issued before them) skips them
                __builtin_nontemporal_store(val, reinterpret_cast<f32x4v*>(p.out + ((int64_t)e * p.M + row) * p.N +
                                                                           (int64_t)nt * kBT + wn * 64 + 4 * c4));
            }
        }
    }
}

static int bwd_blocks(int64_t tiles) {
    int64_t g = tiles < 1 ? 1 : tiles;
    if (g > 1024) g = 1024;  // two per CU, walking the tiles
    return (int)g;
}

}  // namespace nvq

using namespace nvq;

extern "C" {

int64_t nvfp4_axis1_ld(int64_t R, int64_t nseg) {
    if (R < 0 || nseg < 1) return -1;
    return 128 * ((R + 31 * nseg + 127) / 128) + 128;
}

size_t nvfp4_quantize_axis1_workspace_size(int64_t R, int64_t C, int64_t nseg) {
    Carver c(nullptr);
    c.take<int32_t>((size_t)(nseg > 0 ? nseg : 1) + 1);
    c.take<uint32_t>((size_t)kA1MaxBlocks + 2048);
    c.take<uint32_t>((size_t)(nseg > 0 ? nseg : 1));  // folded maxima
    c.take<int2>((size_t)chunk_table_len(R, nseg));    // chunk rows
    return c.need;
}

int nvfp4_quantize_axis1(const uint16_t* x, int64_t R, int64_t C, const int32_t* row_gather, int32_t gather_div,
                         const int32_t* seg_offsets, int64_t nseg, int64_t ld, int rht, uint64_t sign_seed,
                         int scale_per_segment, int round_mode, uint64_t seed, uint32_t stream_id, uint8_t* codes,
                         uint8_t* scales, float* tscale, void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!x || !codes || !scales || !tscale || !ws) return NVQ_ERR_NULL;
    if (R < 0 || C <= 0 || nseg < 1 || nseg > 4096 || gather_div < 1 || ld <= 0 || (ld % 32) != 0) return NVQ_ERR_DIM;
    if (round_mode != NVQ_RTN && round_mode != NVQ_SR) return NVQ_ERR_UNSUPPORTED;
    if (scale_per_segment && (rht || row_gather || seg_offsets || round_mode != NVQ_RTN)) return NVQ_ERR_UNSUPPORTED;
    if (scale_per_segment && ((R % nseg) != 0 || ((R / nseg) % 32) != 0 || ld != R)) return NVQ_ERR_DIM;
    if (!scale_per_segment && ld < nvfp4_axis1_ld(R, nseg) - 128) return NVQ_ERR_DIM;
    if (R >= ((int64_t)1 << 31) || C >= ((int64_t)1 << 31) || ld >= ((int64_t)1 << 31) ||
        ((ld + 255) / 256) * ((C + 63) / 64) >= ((int64_t)1 << 31))
        return NVQ_ERR_DIM;
    if (!aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 1u) || !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < nvfp4_quantize_axis1_workspace_size(R, C, nseg)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    int32_t* pad = cv.take<int32_t>((size_t)nseg + 1);
    uint32_t* part = cv.take<uint32_t>((size_t)kA1MaxBlocks + 2048);
    uint32_t* fold = cv.take<uint32_t>((size_t)nseg);
    int2* chunks = cv.take<int2>((size_t)chunk_table_len(R, nseg));
    A1Args a{};
    a.x = x;
    a.R = (int)R;
    a.C = (int)C;
    a.gather = row_gather;
    a.gdiv = gather_div;
    a.pad = pad;
    a.ld = (int)ld;
    a.ctiles = (int)((C + 63) / 64);
    a.groups = (int)((ld + 255) / 256);
    a.tiles = a.groups * a.ctiles;
    a.wide_scales = (ld % 128) == 0 && (reinterpret_cast<uintptr_t>(scales) & 7u) == 0;
    a.sign_seed = sign_seed;
    if (seg_offsets) {
        a.seg = seg_offsets;
        a.nseg = (int)nseg;
        a.seg_rows = a.seg_pad = 1;
        launch_pad_offsets(seg_offsets, nseg, R, pad, s);
        a.chunks = chunks;
        a.nchunks = (int)chunk_table_len(R, nseg);
        launch_chunk_rows(seg_offsets, pad, nseg, a.nchunks, chunks, s);
    } else if (scale_per_segment) {
        // nseg equal contiguous segments whose rows fill whole 32-row chunks
        a.seg = nullptr;
        a.nseg = (int)nseg;
        a.seg_rows = a.seg_pad = (int)(R / nseg);
    } else {
        // one segment [0, R) padded to 32 rows
        if (nseg != 1) return NVQ_ERR_DIM;
        a.seg = nullptr;
        a.nseg = 1;
        a.seg_rows = (int)R;
        a.seg_pad = (int)std::max<int64_t>(32, 32 * ((R + 31) / 32));
    }
    const int G = (int)std::min<int64_t>(kA1MaxBlocks, std::max<int64_t>(1, a.tiles));
    int n_part;
    if (scale_per_segment) {
        n_part = stream_blocks(R / nseg * C / 8, nseg);
        if (nseg * (int64_t)n_part > (int64_t)kA1MaxBlocks + 2048) return NVQ_ERR_DIM;
        launch_amax_bf16(x, nseg, R / nseg * C, part, n_part, s);
    } else {
        n_part = G;
        if (rht) hipLaunchKernelGGL(k_a1_amax<true>, dim3(G), dim3(256), 0, s, a, part);
        else hipLaunchKernelGGL(k_a1_amax<false>, dim3(G), dim3(256), 0, s, a, part);
    }
    NVQ_CHECK_LAUNCH();
    const bool ps = scale_per_segment != 0;
    hipLaunchKernelGGL(k_a1_fold, dim3(ps ? (unsigned)nseg : 1u), dim3(256), 0, s, part, n_part, fold, tscale);
#define NVQ_A1ENC(RHT_, MODE_)                                                                                  \
    hipLaunchKernelGGL((k_a1_encode<RHT_, MODE_>), dim3((unsigned)a.tiles), dim3(256), 0, s, a, fold, ps, codes, \
                       scales, seed, stream_id)
    if (rht && round_mode == NVQ_SR) NVQ_A1ENC(true, NVQ_SR);
    else if (rht) NVQ_A1ENC(true, NVQ_RTN);
    else if (round_mode == NVQ_SR) NVQ_A1ENC(false, NVQ_SR);
    else NVQ_A1ENC(false, NVQ_RTN);
#undef NVQ_A1ENC
    return launch_status();
}

size_t moe_grouped_gemm_nvfp4_bwd_workspace_size(int mode, int64_t E, int64_t R) {
    Carver c(nullptr);
    const int64_t e = E > 0 ? E : 1;
    c.take<int32_t>((size_t)e + 1);
    if (mode == NVQ_DGRAD) {
        c.take<int32_t>((size_t)((R > 0 ? R : 0) + kBT - 1) / kBT + (size_t)e);  // m-tile map (tiles >= kBT rows)
        c.take<uint8_t>(gemm_dummy_bytes());
    }
    return c.need;
}

int moe_grouped_gemm_nvfp4_bwd(int mode, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tscale,
                               const int32_t* a_gather, const uint8_t* b_codes, const uint8_t* b_scales,
                               const float* b_tscale, const int32_t* seg_offsets, int64_t lda, int64_t ldb,
                               int64_t E, int64_t M, int64_t N, int64_t K, float* out, void* ws, size_t ws_bytes,
                               nvq_stream_t stream) {
    if (!a_codes || !a_scales || !a_tscale || !b_codes || !b_scales || !b_tscale || !seg_offsets || !out || !ws)
        return NVQ_ERR_NULL;
    if (mode != NVQ_DGRAD && mode != NVQ_WGRAD) return NVQ_ERR_UNSUPPORTED;
    if (E < 1 || E > 4096 || M < 0 || N <= 0 || (N % kBT) != 0 || K < 0) return NVQ_ERR_DIM;
    if (mode == NVQ_DGRAD) {
        // M = rows of A in sorted order (the output rows), K = the contraction length
        if (K == 0 || (K % kBK) != 0 || lda < K || (lda % 32) != 0 || ldb < E * K || (ldb % 32) != 0) return NVQ_ERR_DIM;
        if (M >= ((int64_t)1 << 31) || M * N >= ((int64_t)1 << 40)) return NVQ_ERR_DIM;
        if (M * (lda / 2) >= ((int64_t)1 << 32) || N * (ldb / 2) >= ((int64_t)1 << 32)) return NVQ_ERR_DIM;
    } else {
        // M, N = the output's sizes; K = the token rows the segments cover
        if ((M % kBT) != 0 || M == 0) return NVQ_ERR_DIM;
        if (lda < nvfp4_axis1_ld(K, E) || ldb < nvfp4_axis1_ld(K, E) || (lda % 32) != 0 || (ldb % 32) != 0)
            return NVQ_ERR_DIM;
        if (E * (M / kBT) * (N / kBT) >= ((int64_t)1 << 31)) return NVQ_ERR_DIM;
    }
    if (!aligned16(a_codes) || !aligned16(b_codes) || (reinterpret_cast<uintptr_t>(a_scales) & 1u) ||
        (reinterpret_cast<uintptr_t>(b_scales) & 1u) || !aligned16(out) || !aligned256(ws))
        return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_grouped_gemm_nvfp4_bwd_workspace_size(mode, E, M)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    int32_t* tiles = cv.take<int32_t>((size_t)E + 1);
    BwArgs p;
    p.ac = a_codes;
    p.as = a_scales;
    p.lda = lda;
    p.bc = b_codes;
    p.bs = b_scales;
    p.ldb = ldb;
    p.ats = a_tscale;
    p.bts = b_tscale;
    p.seg = seg_offsets;
    p.tiles = tiles;
    p.out = out;
    p.E = (int)E;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.n_tiles = (int)(N / kBT);
    int64_t bound;
    if (mode == NVQ_DGRAD) {
        // the forward's grouped GEMM with an fp32 epilogue
        int32_t* tmap = cv.take<int32_t>((size_t)(M + kBT - 1) / kBT + (size_t)E);
        uint16_t* dummy = cv.take<uint16_t>(gemm_dummy_bytes() / 2);
        launch_tile_offsets(seg_offsets, E, gemm_tile_m(), tiles, tmap, s);
        launch_dgrad_nvfp4(a_codes, a_scales, a_tscale, a_gather, b_codes, b_scales, b_tscale, seg_offsets, tiles,
                           tmap, lda, ldb, E, N, K, out, dummy, s);
    } else {
        p.m_tiles = (int)(M / kBT);
        launch_pad_offsets(seg_offsets, E, 0, tiles, s);
        bound = E * p.m_tiles * p.n_tiles;
        NVQ_CHECK_LAUNCH();
        hipLaunchKernelGGL(k_nvfp4_wgrad, dim3(bwd_blocks(bound)), dim3(256), 0, s, p);
    }
    return launch_status();
}

}  // extern "C"
