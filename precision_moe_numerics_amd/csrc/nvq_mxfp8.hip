// nvq_mxfp8.hip -- the MXFP8 backward of the expert layers on gfx950:
// requantization (nearest-even or Philox stochastic rounding) along either
// axis, the E8M0-scaled FP8 grouped GEMMs (dgrad and wgrad) and the SwiGLU
// backward.
//
// The recipe keeps the backward in MXFP8 with re-quantization and stochastic
// rounding to limit gradient bias (page "Thinking Machines Details End-to-End
// 4-Bit Training for Inkling 2 Small", sections "Key Takeaways" and
// "Architecture highlights"; page "Thinking Machines 详解 Inkling 2 Small 原生
// 4-bit 前向训练完整流程", list "训练数值格式分工清单").
//
// MXFP8 = E4M3 elements with one E8M0 scale per 32. Shared exponent
// floor(log2 amax) - 8 (or, with scale rule 1, ceil(log2(amax / 448)); clamped
// to [-127, 127]); elements E4M3(x * 2^-se),
// saturating at 448; an all-zero block has scale byte 0 and zero elements.
// Unlike NVFP4, this is exactly the operand format of gfx950's block-scaled
// MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), so the GEMMs hand the E8M0 bytes
// to the hardware and contract at the FP8 rate.
#include <algorithm>

#include "nvq_device.hpp"
#include "nvq_host.hpp"

namespace nvq {


// ------------------------------------------------------------------ scale rule
// Rule 0 (OCP): floor(log2 amax) - 8, elements saturate at 448. Rule 1:
// ceil(log2(amax / 448)), so no element saturates: since 448 = 1.75 * 2^8,
// that is one more than rule 0 exactly when amax's significand exceeds 1.75
// (its fraction field above 0x600000).
__device__ __forceinline__ int mx_shared_exp(float amax, int rule) {  // amax > 0
    const uint32_t b = __float_as_uint(amax);
    int e;
    uint32_t frac;
    if (b >= 0x800000u) {
        e = (int)(b >> 23) - 127;
        frac = b & 0x7FFFFFu;
    } else {  // subnormal: normalize the significand
        const int top = 31 - __clz((int)b);
        e = top - 149;
        frac = (b << (23 - top)) & 0x7FFFFFu;
    }
    const int se = e - 8 + ((rule == 1 && frac > 0x600000u) ? 1 : 0);
    return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// 2^-se as an exact fp32 value (se in [-127, 127]; 2^-127 is subnormal).
__device__ __forceinline__ float mx_pow2_neg(int se) {
    const int ex = 127 - se;
    return ex >= 1 ? __uint_as_float((uint32_t)ex << 23) : __uint_as_float(0x400000u);
}

template <int MODE>
__device__ __forceinline__ uint32_t mx_elem(float x, float p2, uint32_t u16) {
    const float y = x * p2;  // one correctly rounded product
    if (MODE != NVQ_RTN) return e4m3_sr_hw(y, u16);
    return e4m3_rne_mag(fabsf(y)) | ((__float_as_uint(y) >> 24) & 0x80u);
}

// ------------------------------------------------------------------ axis 0
// One lane = 8 consecutive values of a row; a 32-value block = 4 lanes.
// IDX: uint32_t index math when the tensor has fewer than 2^31 units (the
// row of a unit is then a 32-bit division), int64_t otherwise. NT: loads with
// the non-temporal hint (a large tensor read once).
template <int MODE, typename IDX, bool NT>
__global__ __launch_bounds__(256) void k_mxfp8_rows(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                    const int32_t* __restrict__ gather, int gdiv,
                                                    uint2* __restrict__ elems, uint8_t* __restrict__ scales,
                                                    uint64_t seed, uint32_t stream_id, int rule) {
    const IDX upr = (IDX)(C / 8), n8 = (IDX)(R * (C / 8));
    const int lane = threadIdx.x & 63;
    const IDX stride = (IDX)gridDim.x * 256u;
    // a group's four scale bytes go out as one 32-bit store where aligned
    const bool scales_al = (reinterpret_cast<uintptr_t>(scales) & 3u) == 0;
    for (IDX wbase = (IDX)blockIdx.x * 256u + (IDX)(threadIdx.x & ~63); wbase < n8; wbase += stride) {
        const IDX u = wbase + (IDX)lane;
        const bool valid = u < n8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (valid) {
            const IDX r = u / upr, cu = u - r * upr;
            const int64_t src = gather ? (int64_t)(gather[r] / gdiv) : (int64_t)r;
            const uint4* q = reinterpret_cast<const uint4*>(x + src * C + (int64_t)cu * 8);
            v = NT ? load_stream(q) : *q;
        }
        float f[8];
        f[0] = bf16_to_f32(v.x & 0xFFFFu); f[1] = bf16_to_f32(v.x >> 16);
        f[2] = bf16_to_f32(v.y & 0xFFFFu); f[3] = bf16_to_f32(v.y >> 16);
        f[4] = bf16_to_f32(v.z & 0xFFFFu); f[5] = bf16_to_f32(v.z >> 16);
        f[6] = bf16_to_f32(v.w & 0xFFFFu); f[7] = bf16_to_f32(v.w >> 16);
        float am = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(f[j]));
        am = fmaxf(am, dpp_swap1(am));
        am = fmaxf(am, dpp_swap2(am));
        uint32_t sbyte = 0, lo = 0, hi = 0;
        if (am > 0.0f) {
            const int se = mx_shared_exp(am, rule);
            const float p2 = mx_pow2_neg(se);
            sbyte = (uint32_t)(se + 127);
            if (MODE == NVQ_SR) {
                const uint4 dr = draws8((uint64_t)u, stream_id, seed);
#pragma unroll
                for (int j = 0; j < 4; ++j) lo |= mx_elem<MODE>(f[j], p2, draw_of(dr, j)) << (8 * j);
#pragma unroll
                for (int j = 0; j < 4; ++j) hi |= mx_elem<MODE>(f[4 + j], p2, draw_of(dr, 4 + j)) << (8 * j);
            } else {
                lo = mx_rne_pair(f[0], f[1], p2) | (mx_rne_pair(f[2], f[3], p2) << 16);
                hi = mx_rne_pair(f[4], f[5], p2) | (mx_rne_pair(f[6], f[7], p2) << 16);
            }
        }
        if (valid) elems[u] = make_uint2(lo, hi);
        // lanes 16g..16g+15 hold blocks 4g..4g+3 (lane 16g + 4j owns block
        // 4g + j): lane 16g gathers the other three bytes by DPP row shifts
        const uint32_t s4 = dpp_row_shl<4>(sbyte), s8 = dpp_row_shl<8>(sbyte), s12 = dpp_row_shl<12>(sbyte);
        if (scales_al && (u | 15u) < n8) {
            if ((lane & 15) == 0)
                *reinterpret_cast<uint32_t*>(scales + u / 4) = sbyte | (s4 << 8) | (s8 << 16) | (s12 << 24);
        } else if (valid && (lane & 3) == 0) {
            scales[u / 4] = (uint8_t)sbyte;
        }
    }
}

// ------------------------------------------------------------------ axis 1
// Padded 32-aligned segment starts: pad[s] = sum_{s'<s} 32 * ceil(n_s' / 32).
__device__ __forceinline__ int64_t seg_at(const int32_t* seg, int s, int64_t R) {
    return seg ? (int64_t)seg[s] : (s == 0 ? 0 : R);
}

// seg == nullptr means one segment [0, R).
__global__ __launch_bounds__(1024) void k_pad_offsets(const int32_t* __restrict__ seg, int nseg, int64_t R,
                                                      int32_t* __restrict__ pad) {
    __shared__ int buf[1024];
    const int t = threadIdx.x;
    int local = 0;
    for (int j = 0; j < 4; ++j) {
        const int s = 4 * t + j;
        if (s < nseg) local += (int)((seg_at(seg, s + 1, R) - seg_at(seg, s, R) + 31) / 32 * 32);
    }
    int total;
    int base = block_exclusive_scan(local, buf, &total);
    for (int j = 0; j < 4; ++j) {
        const int s = 4 * t + j;
        if (s < nseg) {
            pad[s] = base;
            base += (int)((seg_at(seg, s + 1, R) - seg_at(seg, s, R) + 31) / 32 * 32);
        }
    }
    if (t == 0) pad[nseg] = total;
}

void launch_pad_offsets(const int32_t* seg, int64_t nseg, int64_t R, int32_t* pad, hipStream_t s) {
    hipLaunchKernelGGL(k_pad_offsets, dim3(1), dim3(1024), 0, s, seg, (int)nseg, R, pad);
}

// Rows of every padded 32-row block c of explicit segments: [seg[s] + 32c -
// pad[s], seg[s+1]) for the last segment s with pad[s] <= 32c (empty
// segments before a non-empty one start at the same block), or {0, 0} past
// pad[nseg]. A kernel then reads one entry per block instead of searching
// the padded starts with a chain of dependent loads.
__global__ __launch_bounds__(256) void k_chunk_rows(const int32_t* __restrict__ seg, const int32_t* __restrict__ pad,
                                                    int nseg, int nchunks, int2* __restrict__ chunks) {
    for (int c = blockIdx.x * 256 + threadIdx.x; c < nchunks; c += gridDim.x * 256) {
        const int col = 32 * c;
        int2 e = make_int2(0, 0);
        if (col < pad[nseg]) {
            int lo = 0, hi = nseg - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pad[mid] <= col) lo = mid;
                else hi = mid - 1;
            }
            e = make_int2(seg[lo] + (col - pad[lo]), seg[lo + 1]);
        }
        chunks[c] = e;
    }
}

int64_t chunk_table_len(int64_t R, int64_t nseg) {
    return (std::max<int64_t>(R, 0) + 31 * std::max<int64_t>(nseg, 1) + 31) / 32;
}

void launch_chunk_rows(const int32_t* seg, const int32_t* pad, int64_t nseg, int64_t nchunks, int2* chunks,
                       hipStream_t s) {
    hipLaunchKernelGGL(k_chunk_rows, dim3((unsigned)std::min<int64_t>(1024, (nchunks + 255) / 256)), dim3(256), 0, s,
                       seg, pad, (int)nseg, (int)nchunks, chunks);
}

// One thread = two adjacent columns x four 32-row padded blocks (128 output
// bytes per column). It reads the column pair row by row (32-bit loads; a
// wave covers 256 contiguous bytes of each row). Whole blocks of contiguous
// rows advance one row pointer with no per-row checks; gathered or partial
// blocks fetch the source rows once per lane (lane j holds row j) and
// broadcast them, so the row loads do not wait on scalar loads one by one.
// Nearest-even encoding uses the hardware fp32 -> E4M3 converter; it then
// keeps the four blocks' codes in registers and writes each column's 128
// bytes as one burst of 16-byte stores, so L2 receives whole lines (stored
// block by block, a workgroup's partial lines outgrow L2 and reach HBM in
// pieces: 1.8x slower). Stochastic rounding is bound by the Philox rounds
// and stores block by block, which keeps fewer registers live.
// Stochastic rounding: when C % 8 == 0 the eight draws of one Philox call are
// the 8 columns of one row held by a lane quad, so each lane computes the
// call for one of four rows and the quad trades words through LDS (every
// draw is used once); otherwise every lane computes its own calls.
// The 32 codes and the scale byte of padded block pb of columns c0 and c0 + 1.
__device__ __forceinline__ void mx_store_block(uint8_t* __restrict__ elems, uint8_t* __restrict__ scales, int64_t C,
                                               int64_t ld, int64_t nblk, int64_t c0, int64_t pb, const uint32_t (&w0)[8],
                                               const uint32_t (&w1)[8], uint32_t s0, uint32_t s1) {
    uint4* d0 = reinterpret_cast<uint4*>(elems + c0 * ld + pb * 32);
    d0[0] = make_uint4(w0[0], w0[1], w0[2], w0[3]);
    d0[1] = make_uint4(w0[4], w0[5], w0[6], w0[7]);
    scales[c0 * nblk + pb] = (uint8_t)s0;
    if (c0 + 1 < C) {
        uint4* d1 = reinterpret_cast<uint4*>(elems + (c0 + 1) * ld + pb * 32);
        d1[0] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        d1[1] = make_uint4(w1[4], w1[5], w1[6], w1[7]);
        scales[(c0 + 1) * nblk + pb] = (uint8_t)s1;
    }
}

template <int MODE, bool OCT>
__global__ __launch_bounds__(256) void k_mxfp8_cols(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                    const int32_t* __restrict__ gather, int gdiv,
                                                    const int32_t* __restrict__ seg, const int32_t* __restrict__ pad,
                                                    int nseg, const int2* __restrict__ chunks, int nchunks, int64_t ld,
                                                    uint8_t* __restrict__ elems,
                                                    uint8_t* __restrict__ scales, uint64_t seed, uint32_t stream_id,
                                                    int rule) {
    __shared__ uint4 xch[4][64];  // per-wave Philox words, SR with OCT only
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
    const bool col_ok = c0 < C;  // no early exit: a quad may trade draws
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, quad = lane & 3;
    const int64_t nblk = ld / 32;
    const int32_t pad_end = pad[nseg];
    constexpr int kSlots = (MODE == NVQ_RTN) ? 4 : 1;  // blocks whose codes are held before storing
    uint32_t wa0[kSlots][8], wa1[kSlots][8];              // codes of columns c0 and c0 + 1
    uint32_t sa0[kSlots], sa1[kSlots];                     // their scale bytes
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
        const int64_t pb = (int64_t)blockIdx.y * 4 + bb;
        const int64_t p = pb * 32;
        if (pb >= nblk) break;
        const int slot = (MODE == NVQ_RTN) ? bb : 0;
        uint32_t(&w0)[8] = wa0[slot];
        uint32_t(&w1)[8] = wa1[slot];
        uint32_t& s0 = sa0[slot];
        uint32_t& s1 = sa1[slot];
        s0 = 0; s1 = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) { w0[q] = 0; w1[q] = 0; }
        if (p < pad_end) {
            int64_t rs, re;
            if (chunks) {  // explicit segments: the block's rows from the table
                const int2 e = chunks[pb];
                rs = e.x; re = e.y;
            } else {       // one segment [0, R)
                rs = p; re = R;
            }
            const int nvalid = (int)min((int64_t)32, re - rs);  // rows of this block inside the segment
            uint32_t v[32];
            if (!gather && nvalid == 32) {
                // whole block, rows contiguous: one row pointer advanced by C
                const uint16_t* rp = x + rs * C + (col_ok ? c0 : 0);
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    v[j] = col_ok ? *reinterpret_cast<const uint32_t*>(rp) : 0u;
                    rp += C;
                }
            } else {
                // gathered or partial block: source row of block row (lane & 31)
                // fetched once per lane and broadcast; rows past the segment read 0
                int32_t src_l = 0;
                {
                    const int64_t r = rs + (lane & 31);
                    if (r < re) src_l = gather ? gather[r] / gdiv : (int32_t)r;
                }
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    const int64_t src = (int64_t)__shfl(src_l, j, 64);
                    v[j] = (col_ok && j < nvalid) ? *reinterpret_cast<const uint32_t*>(x + src * C + c0) : 0u;
                }
            }
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                a0 = fmaxf(a0, fabsf(bf16_to_f32(v[j] & 0xFFFFu)));
                a1 = fmaxf(a1, fabsf(bf16_to_f32(v[j] >> 16)));
            }
            // padding rows hold zeros, which encode to zero bytes in both modes
            const int se0 = a0 > 0.0f ? mx_shared_exp(a0, rule) : 0, se1 = a1 > 0.0f ? mx_shared_exp(a1, rule) : 0;
            const float p0 = a0 > 0.0f ? mx_pow2_neg(se0) : 0.0f, p1 = a1 > 0.0f ? mx_pow2_neg(se1) : 0.0f;
            s0 = a0 > 0.0f ? (uint32_t)(se0 + 127) : 0u;
            s1 = a1 > 0.0f ? (uint32_t)(se1 + 127) : 0u;
            if (MODE == NVQ_RTN) {
#pragma unroll
                for (int j = 0; j < 32; j += 2) {
                    // pairs (column c0, rows j, j+1) and (column c0+1, rows j, j+1)
                    const uint32_t q0 = mx_rne_pair(bf16_to_f32(v[j] & 0xFFFFu), bf16_to_f32(v[j + 1] & 0xFFFFu), p0);
                    const uint32_t q1 = mx_rne_pair(bf16_to_f32(v[j] >> 16), bf16_to_f32(v[j + 1] >> 16), p1);
                    w0[j / 4] |= q0 << (8 * (j & 3));
                    w1[j / 4] |= q1 << (8 * (j & 3));
                }
            } else {
#pragma unroll
                for (int j0 = 0; j0 < 32; j0 += 4) {
                    uint32_t dw[4];  // draw word (columns c0, c0+1) of rows j0..j0+3
                    if (OCT) {
                        // lane `quad` draws for row rs + j0 + quad: counter (r*C + c0) / 8
                        const uint64_t g = (uint64_t)(rs + j0 + quad) * (uint64_t)(C / 8) + (uint64_t)(c0 >> 3);
                        xch[wave][lane] = draws8(g, stream_id, seed);
                        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            dw[t] = reinterpret_cast<const uint32_t*>(&xch[wave][(lane & ~3) + t])[quad];
                        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const uint64_t i = (uint64_t)((rs + j0 + t) * C + c0);  // even: i, i+1 share a word
                            const uint4 dr = draws8(i >> 3, stream_id, seed);
                            dw[t] = draw_of(dr, (int)(i & 7)) | (draw_of(dr, (int)(i & 7) + 1) << 16);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int j = j0 + t;
                        const uint32_t e0 = mx_elem<MODE>(bf16_to_f32(v[j] & 0xFFFFu), p0, dw[t] & 0xFFFFu);
                        const uint32_t e1 = mx_elem<MODE>(bf16_to_f32(v[j] >> 16), p1, dw[t] >> 16);
                        w0[j / 4] |= e0 << (8 * (j & 3));
                        w1[j / 4] |= e1 << (8 * (j & 3));
                    }
                }
            }
            // an all-zero column block has scale byte 0 and zero bytes (also for -0 inputs)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (!(a0 > 0.0f)) w0[q] = 0u;
                if (!(a1 > 0.0f)) w1[q] = 0u;
            }
        }
        if (MODE != NVQ_RTN && col_ok) mx_store_block(elems, scales, C, ld, nblk, c0, pb, w0, w1, s0, s1);
    }
    if (MODE == NVQ_RTN && col_ok) {
        // column by column: the 8 stores of one column's 128 bytes back to back
        const int64_t pb0 = (int64_t)blockIdx.y * 4;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t c = c0 + half;
            if (c >= C) break;
            uint4* d = reinterpret_cast<uint4*>(elems + c * ld + pb0 * 32);
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                if (pb0 + bb < nblk) {
                    const uint32_t(&w)[8] = half ? wa1[bb] : wa0[bb];
                    d[2 * bb] = make_uint4(w[0], w[1], w[2], w[3]);
                    d[2 * bb + 1] = make_uint4(w[4], w[5], w[6], w[7]);
                    scales[c * nblk + pb0 + bb] = (uint8_t)(half ? sa1[bb] : sa0[bb]);
                }
            }
        }
    }
}

// Axis-1 requantization, tiled (C % 8 == 0): a 256-thread workgroup takes
// 128 padded rows (four 32-row blocks) x 128 columns. The rows come in with coalesced 16-byte loads
// (16 lanes per 256-byte row piece, gathered or padding rows resolved per
// row) into a row-major LDS tile; thread (cp, b) then encodes block b of
// columns 2cp and 2cp+1 exactly as the per-column kernel does; the codes go
// back through LDS so that every 16-byte store covers whole 128-byte output
// lines (8 columns x 128 bytes per store instruction), and each column's four
// scale bytes leave as one 32-bit store. Workgroups are dealt to the 8 XCDs
// round robin; tile ids are remapped so that each XCD walks a contiguous range
// of row groups (all column tiles of one group, then the next): the pieces of
// one output row then meet in one L2 and reach HBM as longer runs. A column's
// four scale bytes are one 32-bit store where that is aligned (ld % 128 ==
// 0 and aligned scales), else four byte stores. Stochastic rounding: a wave
// is one block and 64 column pairs; the eight draws of one Philox call are
// the 8 columns of one row held by a lane quad, so each lane computes the
// call for one of four rows and the quad trades words through LDS (as in
// k_mxfp8_cols).
constexpr int kCTPlane = 4096 + 64;  // bytes per block plane of the code exchange (padded: planes on other banks)

template <int MODE>
__global__ __launch_bounds__(256) void k_mxfp8_cols_tile(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                         const int32_t* __restrict__ gather, int gdiv,
                                                         const int32_t* __restrict__ seg,
                                                         const int32_t* __restrict__ pad, int nseg,
                                                         const int2* __restrict__ chunks, int nchunks, int64_t ld,
                                                         uint8_t* __restrict__ elems, uint8_t* __restrict__ scales,
                                                         uint64_t seed, uint32_t stream_id, int rule, bool nt) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[128 * 256];  // bf16 [128 rows][128 cols]; then codes
    __shared__ uint4 xch[4][64];                                       // per-wave Philox words (SR)
    const int t = threadIdx.x;
    const int64_t ntc = (C + 127) / 128, N = (int64_t)gridDim.x, N8 = N / 8 * 8, id = blockIdx.x;
    const int64_t v = id < N8 ? (id % 8) * (N8 / 8) + id / 8 : id;
    const int64_t cb = (v % ntc) * 128;  // first column
    const int64_t nblk = ld / 32, pb0 = (v / ntc) * 4;
    const int32_t pad_end = pad[nseg];
    // per block (uniform): first source row and end of its segment
    int64_t rs[4], re[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int64_t p = (pb0 + b) * 32;
        rs[b] = 0; re[b] = 0;  // padding block: no valid rows
        if (pb0 + b < nblk && p < pad_end) {
            if (chunks) {  // explicit segments: the block's rows from the table
                const int2 e = chunks[pb0 + b];
                rs[b] = e.x; re[b] = e.y;
            } else {       // one segment [0, R)
                rs[b] = p; re[b] = R;
            }
        }
    }
    // load: instruction k covers tile rows 16k .. 16k+15, lane group t / 16 one row, t % 16 its 16-byte chunk
    {
        const int ch = t & 15;
        const int64_t col = cb + 8 * ch;
        const bool col_ok = col < C;  // C % 8 == 0: a chunk is wholly inside or outside
        uint4 w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = 16 * k + (t >> 4), b = i >> 5, jj = i & 31;
            const int64_t r = rs[b] + jj;
            const bool ok = col_ok && r < re[b];
            int64_t src = r;
            if (gather && ok) src = gather[r] / gdiv;
            const uint4* q = reinterpret_cast<const uint4*>(x + src * C + col);
            w[k] = ok ? (nt ? load_stream(q) : *q) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = 16 * k + (t >> 4);
            *reinterpret_cast<uint4*>(tile + i * 256 + ch * 16) = w[k];
        }
    }
    __syncthreads();
    // encode: thread (cp, b) = columns 2cp, 2cp+1 of block b
    const int cp = t & 63, b = t >> 6;
    uint32_t w0[8], w1[8], s0 = 0, s1 = 0;
    {
        uint32_t v[32];
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) v[jj] = *reinterpret_cast<const uint32_t*>(tile + (32 * b + jj) * 256 + 4 * cp);
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) {
            a0 = fmaxf(a0, fabsf(bf16_to_f32(v[jj] & 0xFFFFu)));
            a1 = fmaxf(a1, fabsf(bf16_to_f32(v[jj] >> 16)));
        }
        // padding rows hold zeros, which encode to zero bytes
        const int se0 = a0 > 0.0f ? mx_shared_exp(a0, rule) : 0, se1 = a1 > 0.0f ? mx_shared_exp(a1, rule) : 0;
        const float p0 = a0 > 0.0f ? mx_pow2_neg(se0) : 0.0f, p1 = a1 > 0.0f ? mx_pow2_neg(se1) : 0.0f;
        s0 = a0 > 0.0f ? (uint32_t)(se0 + 127) : 0u;
        s1 = a1 > 0.0f ? (uint32_t)(se1 + 127) : 0u;
#pragma unroll
        for (int q = 0; q < 8; ++q) { w0[q] = 0u; w1[q] = 0u; }
        if (MODE == NVQ_RTN) {
#pragma unroll
            for (int jj = 0; jj < 32; jj += 2) {
                const uint32_t q0 = mx_rne_pair(bf16_to_f32(v[jj] & 0xFFFFu), bf16_to_f32(v[jj + 1] & 0xFFFFu), p0);
                const uint32_t q1 = mx_rne_pair(bf16_to_f32(v[jj] >> 16), bf16_to_f32(v[jj + 1] >> 16), p1);
                w0[jj / 4] |= q0 << (8 * (jj & 3));
                w1[jj / 4] |= q1 << (8 * (jj & 3));
            }
        } else {
            const int lane = t & 63, quad = lane & 3;
            // element (r, c) draws from the call at counter (r * C + c) / 8 of
            // its logical row r (padding rows draw but hold zeros)
            const uint64_t gcol = (uint64_t)((cb + 2 * cp) >> 3);
#pragma unroll
            for (int j0 = 0; j0 < 32; j0 += 4) {
                const uint64_t g = (uint64_t)(rs[b] + j0 + quad) * (uint64_t)(C / 8) + gcol;
                xch[b][lane] = draws8(g, stream_id, seed);
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
                uint32_t dw[4];  // draw word (columns 2cp, 2cp + 1) of rows j0 .. j0 + 3
#pragma unroll
                for (int u = 0; u < 4; ++u) dw[u] = reinterpret_cast<const uint32_t*>(&xch[b][(lane & ~3) + u])[quad];
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int jj = j0 + u;
                    const uint32_t e0 = mx_elem<MODE>(bf16_to_f32(v[jj] & 0xFFFFu), p0, dw[u] & 0xFFFFu);
                    const uint32_t e1 = mx_elem<MODE>(bf16_to_f32(v[jj] >> 16), p1, dw[u] >> 16);
                    w0[jj / 4] |= e0 << (8 * (jj & 3));
                    w1[jj / 4] |= e1 << (8 * (jj & 3));
                }
            }
        }
        // an all-zero column block has scale byte 0 and zero bytes (also for -0 inputs)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (!(a0 > 0.0f)) w0[q] = 0u;
            if (!(a1 > 0.0f)) w1[q] = 0u;
        }
    }
    __syncthreads();  // the bf16 tile is consumed: the same LDS takes the codes
    // codes: plane b, column c at b * kCTPlane + 32 c (a wave writes 4 KiB contiguous)
    {
        uint4* d = reinterpret_cast<uint4*>(tile + b * kCTPlane + 64 * cp);
        d[0] = make_uint4(w0[0], w0[1], w0[2], w0[3]);
        d[1] = make_uint4(w0[4], w0[5], w0[6], w0[7]);
        d[2] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        d[3] = make_uint4(w1[4], w1[5], w1[6], w1[7]);
        uint8_t* sc = tile + 4 * kCTPlane;  // [128 columns][4 blocks]
        sc[(2 * cp) * 4 + b] = (uint8_t)s0;
        sc[(2 * cp + 1) * 4 + b] = (uint8_t)s1;
    }
    __syncthreads();
    // stores: 16-byte piece q = 256 k + t of the 128 columns x 128 bytes, column q / 8, piece q % 8
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int q = 256 * k + t, c = q >> 3, pc = q & 7, bb = pc >> 1;
        const uint4 val = *reinterpret_cast<const uint4*>(tile + bb * kCTPlane + 32 * c + 16 * (pc & 1));
        if (cb + c < C && pb0 + bb < nblk)
            *reinterpret_cast<uint4*>(elems + (cb + c) * ld + pb0 * 32 + 16 * pc) = val;
    }
    if (t < 128 && cb + t < C) {
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(tile + 4 * kCTPlane + 4 * t);
        uint8_t* sp = scales + (cb + t) * nblk + pb0;
        if (pb0 + 4 <= nblk && (reinterpret_cast<uintptr_t>(sp) & 3u) == 0) {
            *reinterpret_cast<uint32_t*>(sp) = sw;
        } else {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
                if (pb0 + bb < nblk) sp[bb] = (uint8_t)(sw >> (8 * bb));
        }
    }
}

// ------------------------------------------------------------------ grouped GEMM
// v_mfma_scale_f32_32x32x64_f8f6f4 contracts 64 E4M3 values per lane pair with
// one E8M0 scale per 32 per row, exactly the MXFP8 operand format, so codes
// and scale bytes go to the hardware untouched (no decode).
//
// Tiling (mirrors the NVFP4 kernel): a 256-thread workgroup owns a 256 x 128
// output tile; wave w owns rows [64w, 64w+64) x all 128 columns (2 x 4 MFMA
// 32x32 blocks, 128 fp32 accumulators); K advances 128 values (bytes) per
// step, two MFMA K substeps of 64.
//
// Both operands reach the MFMAs through LDS. Loading straight into the MFMA
// register layout (one row per lane) would touch 32 cache lines with every
// load instruction; a staging load instead gives lane t chunk t % 8 of row
// t / 8 of an 8-row group, so each 16-byte load instruction covers 8 whole
// 128-byte rows. The B tile (128 rows shared by the four waves) lives in a
// two-stage ring (16 KiB + 512 scale bytes per stage), written between the
// MFMAs of the previous step and ordered by the per-step barrier. Each wave's
// 64 A rows go through a private 8 KiB buffer: the step's operands are read
// out and the next step's rows written in their place (the LDS operations of
// one wave complete in issue order, so this needs no barrier). Global loads
// run two steps ahead in registers, the A scale words one step ahead.
//
// Operand layout: lane l holds row l % 32; for K substep kk its bytes 0-15
// are values 16h..16h+15 (h = l / 32) of 32-block 2kk and bytes 16-31 the same
// of block 2kk+1, i.e. 16-byte chunks 4kk+h and 4kk+2+h of the row's 128-byte
// step; the scale lane l supplies is that of block 2kk+h, selected as byte 2kk
// of the step's scale word shifted right by 8h.
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kXTM = 256, kXTN = 128, kXTK = 128;  // tile rows, columns; K bytes per step
constexpr int kXMB = 2, kXNB = 4;                  // 32-row / 32-column MFMA blocks per wave
constexpr int kXStage = kXTN * kXTK;               // 16 KiB of B codes per stage
constexpr int kXAWave = 64 * kXTK;                 // 8 KiB of A codes per wave

struct MxArgs {
    const uint8_t* a; const uint8_t* as; int64_t lda;   // A elems [*, lda], scales [*, lda/32]
    const uint8_t* b; const uint8_t* bs; int64_t ldb;
    const int32_t* seg;      // [E+1]
    const int32_t* tiles;    // DGRAD: m-tile offsets [E+1] (kXTM rows)
    const int32_t* kpad;     // WGRAD: padded K offsets [E+1]
    float* out;
    float* dummy;            // 64 x 16-byte slots for the stores of rows past the end
    int E, M, N, K;
    int n_tiles, m_tiles;    // N / kXTN; WGRAD: ceil(M / kXTM)
    int b_em;                // DGRAD kernel: B expert-major [E*N, ldb] (the forward) rather than [N, ldb >= E*K]
    uint16_t* out_bf16;      // BF16OUT kernels: bf16 output rows out_bf16[row_map[r]] (the forward's fc2)
    const int32_t* row_map;  // [rows]: destination row of each expert-sorted row
};

// Global operands are read with buffer loads: a workgroup-uniform resource
// (base pointer in scalar registers) plus a 32-bit per-lane byte offset, which
// keeps 64-bit address arithmetic out of the vector registers.
typedef int mx_v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ uint4 mx_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const mx_v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// The 4 scale bytes of a row's K step at byte offset off of the scale
// buffer; nvalid (>= 1) blocks are inside the K range, the others read as 0
// and only ever meet zeroed elements. ALIGNED (128-multiple rows and steps):
// one 32-bit load; otherwise byte loads that stay inside the range.
template <bool ALIGNED>
__device__ __forceinline__ uint32_t mx_scale_word(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t nvalid) {
    if (ALIGNED) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    uint32_t w = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
    if (nvalid > 1) w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off + 1, 0, 0) << 8;
    if (nvalid > 2) w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off + 2, 0, 0) << 16;
    if (nvalid > 3) w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off + 3, 0, 0) << 24;
    return w;
}

// Staging fragments: B, chunk t % 8 of tile rows t / 8 + 32q (q = 0..3) and,
// for threads t < 128, the scale word of row t; A, chunk l % 8 of the wave's
// rows l / 8 + 8q (q = 0..7).
struct XB {
    uint4 c[4];
    uint32_t s;
};
struct XG {
    uint4 c[8];
};

// Addressing of one wave for one tile: buffer resources based at the tile's
// first A row and first B row, 32-bit row offsets, and K positions as byte
// offsets inside a row (A positions; B's are offset by b_k0 - a_k0).
// The per-lane offsets are rederived from the thread index (mx_lanes) where
// they are used, so only the workgroup-uniform fields live across loops.
struct XOps {
    __amdgpu_buffer_rsrc_t a, as, b, bs;
    // per lane
    uint32_t a_off[kXMB];        // operand rows 32i + l32 of the wave (elems), for their scale words
    uint32_t g_off;              // staging row l / 8 of the wave (tile-relative), as an offset (elems)
    uint32_t b_off;              // staging row t / 8 (elems); row t / 8 + 32q is b_off + q * b_ld32
    uint32_t bs_off;             // scale row t (threads t < 128)
    uint32_t ga_soff;            // grouped: scale row of the wave's row l (clamped like the staging rows)
    // uniform
    uint32_t lda, ldb;           // row strides (elems)
    int32_t a_rows;              // valid rows from the wave's first (rows past them read the tile's first)
    int32_t tile_rows;           // valid rows of the tile (at most 256)
    uint32_t g_step;             // 8 rows (elems)
    uint32_t g_max;              // offset of the tile's last valid row: staging rows past it read it
    uint32_t b_ld32;
    uint32_t a_k0, a_kend;       // first step position; end of A's valid K range
    uint32_t a_lo;               // start of A's valid K range (<= a_k0 + 127)
    uint32_t b_k0, b_kend;       // B's K range (same length)
};

__device__ __forceinline__ void mx_lanes(XOps& o, int t, int wave) {
    const int lane = t & 63, l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < kXMB; ++i) {
        const int r = i * 32 + l32;
        o.a_off[i] = r < o.a_rows ? (uint32_t)(wave * 64 + r) * o.lda : 0u;
    }
    o.g_off = (uint32_t)(wave * 64 + (lane >> 3)) * o.lda;
    o.b_off = (uint32_t)(t >> 3) * o.ldb;
    o.bs_off = (uint32_t)t * (o.ldb >> 5);
    o.ga_soff = (uint32_t)min(wave * 64 + lane, o.tile_rows - 1) * (o.lda >> 5);
}

// Loads of K positions at or past the range end (32-multiple strides only)
// read the row's last valid chunk, which stays in bounds; A chunks outside the
// valid range are zeroed in registers before use, so whatever B holds there
// contributes nothing. With 128-multiple strides every 128-byte step lies
// inside its row, so no clamping is needed.

// LDS swizzle of 128-byte rows of 8 chunks: chunk c of row n lives at
// c ^ ((n >> 1) & 7), so 16 consecutive rows reading one chunk position, and
// 8-lane groups writing whole rows, hit distinct bank groups.
__device__ __forceinline__ int mx_sw(int n) { return (n >> 1) & 7; }

// (wave < 2 selects the threads t < 128 that carry B scale words; wave is a
// scalar, so this is a scalar branch.)
template <bool ALIGNED, bool WORD>
__device__ __forceinline__ void mx_load_b_half(XB& f, const XOps& o, uint32_t k0, int c, int wave, int half) {
    const uint32_t k = k0 + 16u * c;
    const uint32_t kc = ALIGNED ? k : min(k, o.b_kend - 16u);
#pragma unroll
    for (int q = 2 * half; q < 2 * half + 2; ++q) f.c[q] = mx_ld16(o.b, o.b_off + (uint32_t)q * o.b_ld32 + kc);
    if (WORD && half == 0)
        f.s = wave < 2 ? mx_scale_word<ALIGNED>(o.bs, o.bs_off + (k0 >> 5), (o.b_kend - k0) >> 5) : 0u;
}

// Scale words four K steps at a time (one 16-byte load at a 4-byte aligned
// offset; K a multiple of 512 steps so tiles hold whole groups): a row's scale
// line is then requested once per four steps instead of every step.
__device__ __forceinline__ uint4 mx_scale_group(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return mx_ld16(r, off);
}

// Scale state of one thread: per-step A words (w); with grouped loads the
// group in flight to the LDS tables: A words of the wave's row l (ra), B
// words of tile row t (rb, threads t < 128).
struct XS {
    uint32_t w[kXMB];
    uint4 ra, rb;
};

// Grouped scale tables in LDS, word of step phase ph (0..3) of a row at
// [ph][row]: per wave for its 64 A rows (rewritten in place at the group's
// last step, after that step's reads), and for the 128 B rows in two
// buffers by group parity (written one step before the group starts).
struct XScaleLds {
    uint32_t a[4][4][64];
    uint32_t b[2][4][kXTN];
};
__device__ __forceinline__ void mx_put_group(uint32_t* tbl, int stride, int row, uint4 g) {
    tbl[row] = g.x;
    tbl[stride + row] = g.y;
    tbl[2 * stride + row] = g.z;
    tbl[3 * stride + row] = g.w;
}

// The row offsets are recomputed from one opaque base per call (an add and a
// min each) instead of living in 8 registers for the whole K loop.
template <bool ALIGNED>
__device__ __forceinline__ void mx_load_g(XG& g, const XOps& o, uint32_t k0, int c) {
    const uint32_t k = k0 + 16u * c;
    const uint32_t kc = ALIGNED ? k : min(k, o.a_kend - 16u);
    uint32_t go = o.g_off;
    asm volatile("" : "+v"(go));
#pragma unroll
    for (int q = 0; q < 8; ++q) g.c[q] = mx_ld16(o.a, min(go + (uint32_t)q * o.g_step, o.g_max) + kc);
}

template <bool ALIGNED>
__device__ __forceinline__ uint32_t mx_load_a_scale(const XOps& o, int i, uint32_t k0) {
    return mx_scale_word<ALIGNED>(o.as, (o.a_off[i] >> 5) + (k0 >> 5), (o.a_kend - k0) >> 5);
}

// LDS addresses are derived from one per-lane base each (chunk 0 swizzled):
// the swizzled chunk index is an XOR of the row's swizzle with the chunk
// number. Bases are passed through an opaque move once per step so the
// derived addresses are recomputed (one XOR) rather than hoisted into
// registers for the whole K loop.
//   B staging thread t:  (t/8) * 128 + ((c ^ sw(t/8)) << 4), rows + 32q at + 4096 q
//   A staging lane l:    (l/8) * 128 + ((c ^ sw(l/8)) << 4), rows + 8q at
//                        + 1024 q, XOR 64 for odd q (sw(8q + r) = sw(r) ^ 4 (q & 1))
//   operand lane (l32, h): l32 * 128 + ((h ^ sw(l32)) << 4), rows + 32j at + 4096 j
__device__ __forceinline__ uint32_t mx_stage_base(int n, int c) {
    return (uint32_t)(n * kXTK + ((c ^ mx_sw(n)) << 4));
}
__device__ __forceinline__ uint32_t mx_read_base(int l32, int h) {
    return (uint32_t)(l32 * kXTK + ((h ^ mx_sw(l32)) << 4));
}

// Chunks 2half, 2half+1 of the B staging fragment into the LDS stage; the
// scale word (threads t < 128) with half 0.
template <bool WORD>
__device__ __forceinline__ void mx_store_b_half(uint8_t* stage, uint32_t* sstage, uint32_t sbase, int t,
                                                int wave, const XB& f, int half) {
#pragma unroll
    for (int q = 2 * half; q < 2 * half + 2; ++q)
        *reinterpret_cast<uint4*>(stage + q * 32 * kXTK + sbase) = f.c[q];
    if (WORD && half == 0 && wave < 2) sstage[t] = f.s;
}

__device__ __forceinline__ void mx_store_g(uint8_t* abuf, uint32_t gbase, const XG& g) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
        *reinterpret_cast<uint4*>(abuf + q * 8 * kXTK + (gbase ^ ((uint32_t)(q & 1) << 6))) = g.c[q];
}

// Operand of 32-row block j, K substep kk: chunks 4kk + h and 4kk + 2 + h of
// row j * 32 + l32 (B stage or a wave's A buffer).
__device__ __forceinline__ v8i mx_read_op(const uint8_t* buf, uint32_t rbase, int j, int kk) {
    const uint8_t* rp = buf + j * 32 * kXTK;
    const uint4 lo = *reinterpret_cast<const uint4*>(rp + (rbase ^ ((uint32_t)(4 * kk) << 4)));
    const uint4 hi = *reinterpret_cast<const uint4*>(rp + (rbase ^ ((uint32_t)(4 * kk + 2) << 4)));
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// Zero the A values outside the valid K range [k_lo, k_end) of a partial
// first or last step: the operand's chunks sit at k0 + 16 (4kk + h) and 32
// bytes further.
__device__ __forceinline__ v8i mx_mask_op(v8i v, uint32_t k0, uint32_t k_lo, uint32_t k_end, int h, int kk) {
    const uint32_t klo = k0 + 16u * (4 * kk + h), khi = klo + 32u;
    const bool zlo = klo < k_lo || klo >= k_end, zhi = khi < k_lo || khi >= k_end;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        v[r] = zlo ? 0 : v[r];
        v[r + 4] = zhi ? 0 : v[r + 4];
    }
    return v;
}

__device__ __forceinline__ void mx_lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One K step of one wave (ACTIVE: with MFMAs; otherwise it only stages the
// next B tile). abuf holds this step's A rows, ga the next step's A rows, fb
// the next step's B fragment (stored into `nxt`). As registers die they are
// reloaded: A and B rows for two steps ahead (kb), the A scale words for the
// next step (at ks). GROUP: scale words in groups of four steps through the
// LDS tables, ph (a scalar) the step's place in its group, gp the group's
// parity; the next group's A words (ks) load at phase 1 and B words (kg) at
// phase 2, each under a scalar branch, and both go to LDS at phase 3.
template <bool ACTIVE, bool ALIGNED, bool MAYMASK, bool GROUP>
__device__ __forceinline__ void mx_step(f32x16 (&acc)[kXMB][kXNB], XG& ga, XS& sc, XB& fb, uint8_t* abuf,
                                        const uint8_t* cur, const uint32_t* scur, uint8_t* nxt, uint32_t* snxt,
                                        XScaleLds& st, int t0, int wave, const XOps& og, uint32_t k0, uint32_t ks,
                                        uint32_t kb, uint32_t kg, bool mask, int ph, int gp) {
    // every lane quantity of the step comes from an opaque copy of the
    // thread index: recomputed per step, none of it lives across the loop
    int t = t0;
    asm volatile("" : "+v"(t));
    const int lane = t & 63, l32 = lane & 31, h = lane >> 5;
    uint32_t sbase = mx_stage_base(t >> 3, t & 7), rbase = mx_read_base(l32, h),
             gbase = mx_stage_base(lane >> 3, lane & 7);
    asm volatile("" : "+v"(sbase), "+v"(rbase), "+v"(gbase));
    XOps o = og;
    mx_lanes(o, t, wave);
    // the lane's scale operands: substep kk takes byte 2kk of sa / sb
    constexpr bool kGroup = GROUP;
    uint32_t sa[kXMB];
    if (ACTIVE) {
#pragma unroll
        for (int i = 0; i < kXMB; ++i) sa[i] = (kGroup ? st.a[wave][ph][32 * i + l32] : sc.w[i]) >> (8 * h);
    }
    if (kGroup && ph == 3 && wave < 2) mx_put_group(&st.b[gp ^ 1][0][0], kXTN, t, sc.rb);
    const uint32_t dbk = o.b_k0 - o.a_k0;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        // the B scale word staged with the next step: word (PH + 1) % 4 of the group
        if (kGroup) mx_store_b_half<false>(nxt, snxt, sbase, t, wave, fb, kk);
        else mx_store_b_half<true>(nxt, snxt, sbase, t, wave, fb, kk);
        if (ACTIVE) {
            v8i av[kXMB];
#pragma unroll
            for (int i = 0; i < kXMB; ++i) {
                av[i] = mx_read_op(abuf, rbase, i, kk);
                if (MAYMASK && mask) av[i] = mx_mask_op(av[i], k0, o.a_lo, o.a_kend, h, kk);
            }
            if (kk == 1) {
                // every A value of this step has been read: the next step's
                // rows take their place, and the registers fetch the step after
                if (!kGroup) {
#pragma unroll
                    for (int i = 0; i < kXMB; ++i) sc.w[i] = mx_load_a_scale<ALIGNED>(o, i, ks);
                }
                mx_store_g(abuf, gbase, ga);
                // the next group's A words replace this group's (read at the
                // step start); placed after the wait for ga, which covers them
                if (kGroup && ph == 3) mx_put_group(&st.a[wave][0][0], 64, lane, sc.ra);
                mx_load_g<ALIGNED>(ga, o, kb, lane & 7);
                // after the row loads, so waits on older loads never wait on these
                if (kGroup && ph == 1) sc.ra = mx_scale_group(o.as, o.ga_soff + (ks >> 5));
            }
            // B operands two blocks ahead of their MFMAs (16 registers, not 32)
            v8i bq[2];
            uint32_t sq[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bq[j] = mx_read_op(cur, rbase, j, kk);
                sq[j] = kGroup ? st.b[gp][ph][j * 32 + l32] : scur[j * 32 + l32];
            }
#pragma unroll
            for (int j = 0; j < kXNB; ++j) {
                const v8i bv = bq[j & 1];
                const uint32_t sb = sq[j & 1] >> (8 * h);
#pragma unroll
                for (int i = 0; i < kXMB; ++i) {
                    if (kk == 0)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[i], bv, acc[i][j], 0, 0, 0,
                                                                                      (int)sa[i], 0, (int)sb);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[i], bv, acc[i][j], 0, 0, 2,
                                                                                      (int)sa[i], 2, (int)sb);
                    // pin the MFMA here: otherwise it can sink past the scalar
                    // branches below, keeping every operand read live until then
                    if (kGroup) asm volatile("" : "+v"(acc[i][j]));
                }
                if (j + 2 < kXNB) {
                    bq[j & 1] = mx_read_op(cur, rbase, j + 2, kk);
                    sq[j & 1] = kGroup ? st.b[gp][ph][(j + 2) * 32 + l32] : scur[(j + 2) * 32 + l32];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the B chunks just staged are dead: fetch those of two steps ahead
        mx_load_b_half<ALIGNED, !kGroup>(fb, o, kb + dbk, t & 7, wave, kk);
        if (kGroup && kk == 0 && ph == 2 && wave < 2) sc.rb = mx_scale_group(o.bs, o.bs_off + ((kg + dbk) >> 5));
        // keep each substep's stores and loads in place: hoisting the second
        // half's B store would wait on loads issued just before the barrier
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Position of one tile: expert, column tile, row range, K steps. Rows past
// row_end are never stored; a wave wholly past it only stages B.
struct XTile {
    int e, nt, nk;
    int64_t row0, row_end, wrow0;
    bool active;
};

// Tile tables are read through constant-address-space pointers: they do not
// change during the kernel, and at the workgroup-uniform indices used here
// that makes them scalar loads, which the vector-memory counter (and so the
// output stores in flight) does not hold up. Read after a fence, a plain
// load would be a vector load.
__device__ __forceinline__ int32_t mx_tload(const int32_t* tbl, int64_t i) {
    typedef const __attribute__((address_space(4))) int32_t cint32;
    return ((cint32*)tbl)[i];
}

template <int MODE, bool ALIGNED>
__device__ __forceinline__ void mx_setup(const MxArgs& p, int64_t t, int wave, int tid, XTile& T, XOps& o) {
    int64_t a_k0, a_kend, b_k0;
    if (MODE == NVQ_DGRAD) {
        const int mg = (int)(t / p.n_tiles);
        T.nt = (int)(t % p.n_tiles);
        int lo = 0, hi = p.E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (mx_tload(p.tiles, mid) <= mg) lo = mid; else hi = mid;
        }
        T.e = lo;
        T.row0 = mx_tload(p.seg, T.e) + (int64_t)(mg - mx_tload(p.tiles, T.e)) * kXTM;
        T.row_end = mx_tload(p.seg, T.e + 1);
        a_k0 = 0; a_kend = p.K;
        b_k0 = p.b_em ? 0 : (int64_t)T.e * p.K;
    } else {
        T.e = (int)(t / ((int64_t)p.m_tiles * p.n_tiles));
        const int rem = (int)(t % ((int64_t)p.m_tiles * p.n_tiles));
        T.nt = rem % p.n_tiles;
        T.row0 = (int64_t)(rem / p.n_tiles) * kXTM;
        T.row_end = p.M;
        a_k0 = mx_tload(p.kpad, T.e); a_kend = mx_tload(p.kpad, T.e + 1);
        b_k0 = a_k0;
    }
    const int64_t klen = a_kend - a_k0;
    // ALIGNED: steps start on a 128-byte boundary (whole cache lines);
    // positions before a_k0 are masked like those past a_kend
    const int64_t ks = ALIGNED && klen > 0 ? (a_k0 & ~(int64_t)(kXTK - 1)) : a_k0;
    T.nk = (int)((a_kend - ks + kXTK - 1) / kXTK);
    T.wrow0 = T.row0 + wave * 64;
    T.active = T.wrow0 < T.row_end;  // wave-uniform
    const int64_t row0 = T.row0, row_end = T.row_end;
    o.a = mx_rsrc(p.a + row0 * p.lda);
    o.as = mx_rsrc(p.as + row0 * (p.lda / 32));
    o.lda = (uint32_t)p.lda;
    o.ldb = (uint32_t)p.ldb;
    // rows past the end read the tile's first row (results for them are never stored)
    o.a_rows = (int32_t)max(min(row_end - T.wrow0, (int64_t)64), (int64_t)0);
    o.tile_rows = (int32_t)min(row_end - row0, (int64_t)kXTM);
    o.g_step = 8u * o.lda;
    o.g_max = (uint32_t)(o.tile_rows - 1) * o.lda;
    o.a_k0 = (uint32_t)ks; o.a_kend = (uint32_t)a_kend; o.a_lo = (uint32_t)a_k0;
    // first B row of the tile: expert-major B (the forward) starts expert e at row e*N
    const int64_t b_row0 = (MODE == NVQ_DGRAD && p.b_em ? (int64_t)T.e * p.N : 0) + (int64_t)T.nt * kXTN;
    o.b = mx_rsrc(p.b + b_row0 * p.ldb);
    o.bs = mx_rsrc(p.bs + b_row0 * (p.ldb / 32));
    o.b_ld32 = 32u * o.ldb;
    o.b_k0 = (uint32_t)(b_k0 - (a_k0 - ks)); o.b_kend = (uint32_t)(b_k0 + klen);
    mx_lanes(o, tid, wave);
}

// SG4: scale words in groups of four steps (DGRAD on the aligned path with K
// a multiple of 512, so every tile has whole groups).
//
// Tiles are processed back to back and overlapped at the seams: after a
// tile's last step the next tile's first loads (A and B of step 0, the first
// scale groups) are issued, then the finished tile's output is stored, and
// only then does the wave wait for those loads. gfx9 counts stores and loads
// in one in-order counter, so loads issued after the stores would wait for
// all of them; issued before, their wait skips the stores. That needs a
// fixed number of stores with no branch in between (a branch makes the
// compiler assume the path with fewer stores): every lane of every wave
// issues all of its stores, those of rows past the end going to a dummy
// workspace slot, and the loads for the next tile are unconditional (past
// the last tile they re-read the current tile; an empty K range reads its
// rows' first step).
template <int MODE, bool ALIGNED, bool SG4, bool BF16OUT = false>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm_mxfp8(MxArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][kXStage];
    __shared__ __attribute__((aligned(16))) uint8_t alds[4][kXAWave];
    __shared__ uint32_t slds[2][kXTN];
    __shared__ XScaleLds sclds;
    // wave index as a scalar, so the active test below is a scalar branch
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    int64_t total;
    if (MODE == NVQ_DGRAD) total = (int64_t)mx_tload(p.tiles, p.E) * p.n_tiles;
    else total = (int64_t)p.E * p.m_tiles * p.n_tiles;
    const int G = gridDim.x;
    const int v = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
    if (v >= total) return;

    // lane math is rederived from an opaque thread index where it is used
    // (tile setup, steps, epilogue) rather than kept live across the loops
#define NVQ_MX_LANES                                                                                           \
    int tid = (int)threadIdx.x;                                                                                \
    asm volatile("" : "+v"(tid));                                                                              \
    const int lane = tid & 63, l32 = lane & 31, h = lane >> 5, c = tid & 7;                                   \
    (void)l32; (void)h; (void)c;
    uint8_t* abuf = alds[wave];
    // partial steps zero A outside the K range (never with DGRAD on
    // 128-multiples, where K is a whole number of steps)
    constexpr bool kMayMask = !(MODE == NVQ_DGRAD && ALIGNED);

    XG ga;
    XB fb;
    XS sc;
#pragma unroll
    for (int i = 0; i < kXMB; ++i) sc.w[i] = 0u;
    sc.ra = sc.rb = make_uint4(0u, 0u, 0u, 0u);

    // first loads of a tile: A and B of its first step (position 0 of the
    // rows for an empty K range) and the first scale groups
#define NVQ_MX_FIRST_LOADS(T, O)                                                                               \
    {                                                                                                          \
        const uint32_t ka = (T).nk > 0 ? (O).a_k0 : 0u, kbb = (T).nk > 0 ? (O).b_k0 : 0u;                     \
        if ((T).active) mx_load_g<ALIGNED>(ga, (O), ka, lane & 7);                                              \
        mx_load_b_half<ALIGNED, !SG4>(fb, (O), kbb, c, wave, 0);                                               \
        mx_load_b_half<ALIGNED, !SG4>(fb, (O), kbb, c, wave, 1);                                               \
        if (SG4) {                                                                                             \
            if (wave < 2) sc.rb = mx_scale_group((O).bs, (O).bs_off + (kbb >> 5));                             \
            if ((T).active) sc.ra = mx_scale_group((O).as, (O).ga_soff + (ka >> 5));                           \
        }                                                                                                      \
    }
    // rest of a tile's prologue (nk > 0): step 0 into LDS; then, in the order
    // the steps issue them, B of step 1, the A scale words of step 0 and A of
    // step 1 in flight
#define NVQ_MX_STAGE_FIRST(T, O)                                                                               \
    {                                                                                                          \
        const uint32_t ka0 = (O).a_k0, dbk = (O).b_k0 - (O).a_k0;                                             \
        const uint32_t k1 = ka0 + ((T).nk > 1 ? kXTK : 0);                                                    \
        mx_store_b_half<!SG4>(lds[0], slds[0], mx_stage_base(tid >> 3, c), tid, wave, fb, 0);                  \
        mx_store_b_half<!SG4>(lds[0], slds[0], mx_stage_base(tid >> 3, c), tid, wave, fb, 1);                  \
        if (SG4) {                                                                                             \
            if (wave < 2) mx_put_group(&sclds.b[0][0][0], kXTN, tid, sc.rb);                                   \
            if ((T).active) mx_put_group(&sclds.a[wave][0][0], 64, lane, sc.ra);                               \
        }                                                                                                      \
        if ((T).active) mx_store_g(abuf, mx_stage_base(lane >> 3, lane & 7), ga);                              \
        mx_load_b_half<ALIGNED, !SG4>(fb, (O), k1 + dbk, c, wave, 0);                                          \
        if ((T).active) {                                                                                      \
            _Pragma("unroll") for (int i = 0; i < kXMB; ++i) if (!SG4) sc.w[i] =                               \
                mx_load_a_scale<ALIGNED>((O), i, ka0);                                                         \
            mx_load_g<ALIGNED>(ga, (O), k1, lane & 7);                                                         \
        }                                                                                                      \
        mx_load_b_half<ALIGNED, !SG4>(fb, (O), k1 + dbk, c, wave, 1);                                          \
        mx_lds_barrier();                                                                                      \
    }

    XTile T;
    XOps o;
    {
        NVQ_MX_LANES
        mx_setup<MODE, ALIGNED>(p, v, wave, tid, T, o);
        NVQ_MX_FIRST_LOADS(T, o)
        if (T.nk > 0) NVQ_MX_STAGE_FIRST(T, o)
    }

    for (int64_t t = v;;) {
        f32x16 acc[kXMB][kXNB];
#pragma unroll
        for (int i = 0; i < kXMB; ++i)
#pragma unroll
            for (int j = 0; j < kXNB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        if (T.nk > 0) {
            NVQ_MX_LANES
            const int nk = T.nk;
            const uint32_t ka0 = o.a_k0;
            // one step at position st: kb two steps ahead (clamped), the A
            // scale words of the next step or (grouped) next group, the B
            // scale group starting two steps ahead
#define NVQ_MX_STEP(ACT, ST)                                                                                   \
    {                                                                                                          \
        const int st = (ST);                                                                                   \
        const uint32_t k0 = ka0 + (uint32_t)st * kXTK;                                                         \
        const uint32_t kb = ka0 + (uint32_t)min(st + 2, nk - 1) * kXTK;                                        \
        const uint32_t ks = ka0 + (uint32_t)(!SG4 ? min(st + 1, nk - 1) : min(st + 3, nk - 4)) * kXTK;       \
        const uint32_t kg = ka0 + (uint32_t)min(st + 2, nk - 4) * kXTK;                                        \
        const bool mask = ACT && kMayMask && (k0 < o.a_lo || k0 + kXTK > o.a_kend);                           \
        mx_step<ACT, ALIGNED, ACT && kMayMask, SG4>(acc, ga, sc, fb, abuf, lds[st & 1], slds[st & 1],         \
                                                    lds[(st + 1) & 1], slds[(st + 1) & 1], sclds, tid, wave, o, \
                                                    k0, ks, kb, kg, mask, st & 3, (st >> 2) & 1);               \
        mx_lds_barrier();                                                                                      \
    }
            // separate loops for active and staging-only waves (a branch inside
            // one loop lets the compiler merge the two paths' code)
            // (SG4: nk % 4 == 0, whole groups)
            if (T.active) {
                for (int step = 0; step < nk; ++step) NVQ_MX_STEP(true, step)
            } else {
                for (int step = 0; step < nk; ++step) NVQ_MX_STEP(false, step)
            }
#undef NVQ_MX_STEP
        }

        NVQ_MX_LANES
        // epilogue through the wave's A buffer (free after the last step's
        // barrier), 8 rows at a time. Lane l, register r of a 32x32 block
        // holds column l % 32, row 8 (r / 4) + 4 (l / 32) + r % 4; a round
        // takes the registers with one r / 4 of one row block, writes them to
        // LDS rows of 136 floats (the two lane halves land 32 banks apart)
        // and reads back 16-byte row pieces, so each global store covers two
        // rows x 512 contiguous bytes: whole cache lines, a quarter of the
        // store instructions of per-register stores. The fp32 output is
        // written once and never read here: non-temporal stores keep it from
        // evicting the operand lines the neighbouring tiles re-read from L2.
        // The next tile's first loads go out after the first row block,
        // once its 64 accumulators are free.
        constexpr int kERow = 136;
        float* ebuf = reinterpret_cast<float*>(abuf);
        float* obase = (MODE == NVQ_DGRAD) ? p.out : p.out + (int64_t)T.e * p.M * p.N;
        const int64_t tn = t + G;
        const bool more = tn < total;
        XTile Tn;
        XOps on;
        // BF16OUT: destination rows of the wave's 64 rows, one per lane, loaded
        // before any store (a load issued after the stores would wait for them);
        // each row's lanes fetch it from the lane that holds it
        int32_t rmap = 0;
        if constexpr (BF16OUT) {
            const int64_t rr = T.wrow0 + lane;
            rmap = p.row_map[rr < T.row_end ? rr : 0];
        }
#pragma unroll
        for (int i = 0; i < kXMB; ++i) {
            if (i == 1) {
                // the next tile (past the last one: this tile again, for
                // loads that are never used) and its first loads
                mx_setup<MODE, ALIGNED>(p, more ? tn : t, wave, tid, Tn, on);
                NVQ_MX_FIRST_LOADS(Tn, on)
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                    for (int j = 0; j < kXNB; ++j) ebuf[(4 * h + rr) * kERow + j * 32 + l32] = acc[i][j][4 * q + rr];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int lr = 2 * k + h;  // local row; lane l32 holds its 16-byte piece l32
                    const f32x4 val = *reinterpret_cast<const f32x4*>(ebuf + lr * kERow + 4 * l32);
                    const int64_t row = T.wrow0 + i * 32 + q * 8 + lr;
                    if constexpr (BF16OUT) {
                        // four values as two nearest-even bf16 pairs: 256 contiguous bytes per row
                        const int64_t drow = __builtin_amdgcn_ds_bpermute((i * 32 + q * 8 + lr) << 2, rmap);
                        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                        u32x2* dst = row < T.row_end
                                         ? reinterpret_cast<u32x2*>(p.out_bf16 + drow * p.N + T.nt * kXTN + 4 * l32)
                                         : reinterpret_cast<u32x2*>(p.dummy + 4 * lane);
                        const u32x2 pk = {bf16x2_rne(val[0], val[1]), bf16x2_rne(val[2], val[3])};
                        __builtin_nontemporal_store(pk, dst);
                    } else {
                        float* dst =
                            row < T.row_end ? obase + row * p.N + T.nt * kXTN + 4 * l32 : p.dummy + 4 * lane;
                        __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(dst));
                    }
                }
            }
        }
        if (!more) break;
        t = tn;
        T = Tn;
        o = on;
        if (T.nk > 0) NVQ_MX_STAGE_FIRST(T, o)
    }
#undef NVQ_MX_FIRST_LOADS
#undef NVQ_MX_STAGE_FIRST
#undef NVQ_MX_LANES
}

// two 4-wave workgroups per CU
static int mx_gemm_grid() { return device_cus() * 2; }

// ------------------------------------------------------------------ SwiGLU backward
// dA[:, j] = dh * u * sg * (1 + g * (1 - sg)),  dA[:, d_ff + j] = dh * g * sg,
// sg = 1 / (1 + exp(-g)), in fp32 from the saved bf16 g, u; bf16 out.
__global__ __launch_bounds__(256) void k_swiglu_bwd(const float* __restrict__ dH, const uint16_t* __restrict__ gu,
                                                    int64_t n, int64_t d_ff, uint16_t* __restrict__ dA) {
    const int64_t total = n * d_ff;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / d_ff, j = i - r * d_ff;
        const float g = bf16_to_f32(gu[r * 2 * d_ff + j]);
        const float u = bf16_to_f32(gu[r * 2 * d_ff + d_ff + j]);
        const float dh = dH[i];
        const float sg = 1.0f / (1.0f + expf(-g));
        const float dg = dh * u * sg * (1.0f + g * (1.0f - sg));
        const float du = dh * g * sg;
        dA[r * 2 * d_ff + j] = (uint16_t)f32_to_bf16(dg);
        dA[r * 2 * d_ff + d_ff + j] = (uint16_t)f32_to_bf16(du);
    }
}


// The same per element, eight consecutive columns per lane (d_ff % 8 == 0,
// 16-byte aligned arrays, fewer than 2^31 units of 8): 16-byte loads of g,
// u and dH, 16-byte stores of both dA halves, one index division per 8.
__global__ __launch_bounds__(256) void k_swiglu_bwd8(const float4* __restrict__ dH, const uint4* __restrict__ gu,
                                                     int units, int d8, uint4* __restrict__ dA) {
    const int stride = gridDim.x * 256;
    for (int q = blockIdx.x * 256 + threadIdx.x; q < units; q += stride) {
        const int r = q / d8, j8 = q - r * d8;
        const uint4 gw = gu[(int64_t)r * 2 * d8 + j8];
        const uint4 uw = gu[(int64_t)r * 2 * d8 + d8 + j8];
        const float4 h0 = dH[2 * (int64_t)q], h1 = dH[2 * (int64_t)q + 1];
        const uint32_t gs[4] = {gw.x, gw.y, gw.z, gw.w}, us[4] = {uw.x, uw.y, uw.z, uw.w};
        const float dh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        uint32_t og[4], ou[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float dg[2], du[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float g = bf16_to_f32(t ? gs[k] >> 16 : gs[k] & 0xFFFFu);
                const float u = bf16_to_f32(t ? us[k] >> 16 : us[k] & 0xFFFFu);
                const float sg = 1.0f / (1.0f + expf(-g));
                dg[t] = dh[2 * k + t] * u * sg * (1.0f + g * (1.0f - sg));
                du[t] = dh[2 * k + t] * g * sg;
            }
            og[k] = bf16x2_rne(dg[0], dg[1]);
            ou[k] = bf16x2_rne(du[0], du[1]);
        }
        dA[(int64_t)r * 2 * d8 + j8] = make_uint4(og[0], og[1], og[2], og[3]);
        dA[(int64_t)r * 2 * d8 + d8 + j8] = make_uint4(ou[0], ou[1], ou[2], ou[3]);
    }
}

// ---------------------------------------------------------------- MXFP8 forward
// SwiGLU from fp32 g,u (G [n, 2 d_ff], gate half first) to bf16 H [n, d_ff]:
// h = g * u * sigmoid(g), the same formula and instructions as the NVFP4 fc1
// epilogue; eight columns per lane (d_ff % 8 == 0, fewer than 2^31 units).
__global__ __launch_bounds__(256) void k_swiglu_fwd8(const float4* __restrict__ G, int units, int d8,
                                                     uint4* __restrict__ H) {
    const int stride = gridDim.x * 256;
    for (int q = blockIdx.x * 256 + threadIdx.x; q < units; q += stride) {
        const int r = q / d8, j8 = q - r * d8;
        const float4* gr = G + (int64_t)r * 4 * d8;  // a row of G: 2 d_ff floats = 4 d8 float4
        const float4 g0 = gr[2 * j8], g1 = gr[2 * j8 + 1];
        const float4 u0 = gr[2 * d8 + 2 * j8], u1 = gr[2 * d8 + 2 * j8 + 1];
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        float h[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) h[t] = g[t] * u[t] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[t]));
        H[(int64_t)r * d8 + j8] = make_uint4(bf16x2_rne(h[0], h[1]), bf16x2_rne(h[2], h[3]),
                                             bf16x2_rne(h[4], h[5]), bf16x2_rne(h[6], h[7]));
    }
}

static unsigned elementwise_grid(int64_t units) {
    int64_t g = (units + 255) / 256;
    if (g > 8192) g = 8192;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace nvq

using namespace nvq;

extern "C" {

int64_t mxfp8_axis1_ld(int64_t R, int64_t nseg) {
    if (nseg < 1) nseg = 1;
    return (R + 31 * nseg + 127) / 128 * 128;  // 128-aligned rows: whole 4-byte scale words
}

size_t mxfp8_requant_workspace_size(int64_t R, int64_t nseg) {
    Carver c(nullptr);
    c.take<int32_t>((size_t)(nseg > 0 ? nseg : 1) + 1);  // padded offsets
    c.take<int2>((size_t)chunk_table_len(R, nseg));      // rows of each padded block
    return c.need;
}

int mxfp8_requant_sr(const uint16_t* x, int64_t R, int64_t C, int axis, const int32_t* row_gather,
                     int32_t gather_div, const int32_t* seg_offsets, int64_t nseg, int64_t ld, int round_mode,
                     int scale_rule, uint64_t seed, uint32_t stream_id, uint8_t* elems, uint8_t* scales, void* ws,
                     size_t ws_bytes, nvq_stream_t stream) {
    if (!x || !elems || !scales) return NVQ_ERR_NULL;
    if (round_mode != NVQ_RTN && round_mode != NVQ_SR) return NVQ_ERR_UNSUPPORTED;
    if (scale_rule != 0 && scale_rule != 1) return NVQ_ERR_UNSUPPORTED;
    if (R < 0 || C <= 0 || gather_div <= 0 || R >= ((int64_t)1 << 31)) return NVQ_ERR_DIM;
    if (!aligned16(x) || !aligned16(elems)) return NVQ_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    if (axis == 0) {
        if (C % 32 != 0) return NVQ_ERR_DIM;
        const int64_t n8 = R * C / 8;
        if (n8 == 0) return NVQ_OK;
        int64_t g = (n8 + 255) / 256;
        if (g > 8192) g = 8192;
        auto ek = reinterpret_cast<uint2*>(elems);
        const bool small = n8 < ((int64_t)1 << 31);
        // the hint only where each source row is read once and the tensor outgrows the Infinity Cache
        const bool nt = gather_div == 1 && R * C * 2 >= kStreamHintBytes;
#define NVQ_ROWS(MODE_, IDX_, NT_)                                                                                \
    hipLaunchKernelGGL((k_mxfp8_rows<MODE_, IDX_, NT_>), dim3((unsigned)g), dim3(256), 0, s, x, R, C, row_gather,  \
                       gather_div, ek, scales, seed, stream_id, scale_rule)
        if (round_mode == NVQ_SR) {
            if (small) { if (nt) NVQ_ROWS(NVQ_SR, uint32_t, true); else NVQ_ROWS(NVQ_SR, uint32_t, false); }
            else { if (nt) NVQ_ROWS(NVQ_SR, int64_t, true); else NVQ_ROWS(NVQ_SR, int64_t, false); }
        } else {
            if (small) { if (nt) NVQ_ROWS(NVQ_RTN, uint32_t, true); else NVQ_ROWS(NVQ_RTN, uint32_t, false); }
            else { if (nt) NVQ_ROWS(NVQ_RTN, int64_t, true); else NVQ_ROWS(NVQ_RTN, int64_t, false); }
        }
#undef NVQ_ROWS
        return launch_status();
    }
    if (axis != 1) return NVQ_ERR_UNSUPPORTED;
    if (!ws) return NVQ_ERR_NULL;
    if (!seg_offsets) nseg = 1;
    if (nseg < 1 || nseg > 4096 || C % 2 != 0) return NVQ_ERR_DIM;
    if (ld % 32 != 0 || ld < mxfp8_axis1_ld(R, nseg)) return NVQ_ERR_DIM;
    if (!aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < mxfp8_requant_workspace_size(R, nseg)) return NVQ_ERR_WORKSPACE;
    Carver cv(ws);
    int32_t* pad = cv.take<int32_t>((size_t)nseg + 1);
    int2* chunks = cv.take<int2>((size_t)chunk_table_len(R, nseg));
    const int32_t* seg = seg_offsets;  // nullptr: one segment [0, R)
    hipLaunchKernelGGL(k_pad_offsets, dim3(1), dim3(1024), 0, s, seg, (int)nseg, R, pad);
    // explicit segments: rows of each padded block in a table (offsets are
    // int32, so R < 2^31 there); one segment needs no search
    const int nchunks = seg ? (int)chunk_table_len(R, nseg) : 0;
    if (seg) launch_chunk_rows(seg, pad, nseg, nchunks, chunks, s);
    const int2* ctab = seg ? chunks : nullptr;
    const dim3 tgrid((unsigned)(((C + 127) / 128) * ((ld / 32 + 3) / 4)));
    // non-temporal loads where each source row is read once and the tensor outgrows the Infinity Cache
    const bool nt = gather_div == 1 && R * C * 2 >= kStreamHintBytes;
    if (round_mode == NVQ_RTN && !row_gather && C % 8 == 0 && ld % 128 == 0 &&
        (reinterpret_cast<uintptr_t>(scales) & 3u) == 0) {
        hipLaunchKernelGGL(k_mxfp8_cols_tile<NVQ_RTN>, tgrid, dim3(256), 0, s, x, R, C, row_gather, gather_div, seg,
                           pad, (int)nseg, ctab, nchunks, ld, elems, scales, seed, stream_id, scale_rule, nt);
        return launch_status();
    }
    if (round_mode == NVQ_SR && C % 8 == 0) {
        hipLaunchKernelGGL(k_mxfp8_cols_tile<NVQ_SR>, tgrid, dim3(256), 0, s, x, R, C, row_gather, gather_div, seg,
                           pad, (int)nseg, ctab, nchunks, ld, elems, scales, seed, stream_id, scale_rule, nt);
        return launch_status();
    }
    dim3 grid((unsigned)((C / 2 + 255) / 256), (unsigned)((ld / 32 + 3) / 4));
    if (round_mode == NVQ_SR && C % 8 == 0)
        hipLaunchKernelGGL((k_mxfp8_cols<NVQ_SR, true>), grid, dim3(256), 0, s, x, R, C, row_gather, gather_div, seg,
                           pad, (int)nseg, ctab, nchunks, ld, elems, scales, seed, stream_id, scale_rule);
    else if (round_mode == NVQ_SR)
        hipLaunchKernelGGL((k_mxfp8_cols<NVQ_SR, false>), grid, dim3(256), 0, s, x, R, C, row_gather, gather_div, seg,
                           pad, (int)nseg, ctab, nchunks, ld, elems, scales, seed, stream_id, scale_rule);
    else
        hipLaunchKernelGGL((k_mxfp8_cols<NVQ_RTN, false>), grid, dim3(256), 0, s, x, R, C, row_gather, gather_div,
                           seg, pad, (int)nseg, ctab, nchunks, ld, elems, scales, seed, stream_id, scale_rule);
    return launch_status();
}

size_t moe_grouped_gemm_mxfp8_workspace_size(int mode, int64_t E, int64_t R) {
    (void)mode; (void)R;
    Carver c(nullptr);
    c.take<int32_t>((size_t)(E > 0 ? E : 1) + 1);
    c.take<float>(256);
    return c.need;
}

}  // extern "C"

// The grouped GEMM behind moe_grouped_gemm_mxfp8. With out_bf16 (NVQ_FWD
// only) the rows are written as bf16 to out_bf16[row_map[r]] instead of fp32
// to out[r] (the MXFP8 forward's fc2, scattered in its epilogue).
static int mx_grouped_gemm(int mode, const uint8_t* a_elems, const uint8_t* a_scales, const uint8_t* b_elems,
                           const uint8_t* b_scales, const int32_t* seg_offsets, int64_t lda, int64_t ldb, int64_t E,
                           int64_t M, int64_t N, int64_t K, float* out, uint16_t* out_bf16,
                           const int32_t* row_map, void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!a_elems || !a_scales || !b_elems || !b_scales || !seg_offsets || !ws) return NVQ_ERR_NULL;
    if (out_bf16 ? (!row_map || mode != NVQ_FWD) : !out) return NVQ_ERR_NULL;
    if (out_bf16 && (reinterpret_cast<uintptr_t>(out_bf16) & 7u)) return NVQ_ERR_ALIGN;
    if (mode != NVQ_DGRAD && mode != NVQ_WGRAD && mode != NVQ_FWD) return NVQ_ERR_UNSUPPORTED;
    if (E < 1 || E > 4096 || N <= 0 || N % kXTN != 0 || lda % 32 != 0 || ldb % 32 != 0) return NVQ_ERR_DIM;
    if (mode == NVQ_DGRAD && (K <= 0 || K % 32 != 0 || lda < K || ldb < E * K)) return NVQ_ERR_DIM;
    if (mode == NVQ_FWD && (K <= 0 || K % 32 != 0 || lda < K || ldb < K)) return NVQ_ERR_DIM;
    if (mode == NVQ_WGRAD && (M <= 0 || M % 128 != 0)) return NVQ_ERR_DIM;
    if (!aligned16(a_elems) || !aligned16(b_elems) || (out && !aligned16(out)) || !aligned256(ws))
        return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_grouped_gemm_mxfp8_workspace_size(mode, E, M)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    int32_t* aux = cv.take<int32_t>((size_t)E + 1);
    float* dummy = cv.take<float>(256);
    MxArgs p{};
    p.a = a_elems; p.as = a_scales; p.lda = lda;
    p.b = b_elems; p.bs = b_scales; p.ldb = ldb;
    p.seg = seg_offsets; p.out = out; p.dummy = dummy;
    p.out_bf16 = out_bf16; p.row_map = row_map;
    p.E = (int)E; p.M = (int)M; p.N = (int)N; p.K = (int)K;
    p.n_tiles = (int)(N / kXTN);
    p.b_em = mode == NVQ_FWD ? 1 : 0;
    if (mode == NVQ_FWD) mode = NVQ_DGRAD;  // the same kernel, B addressed expert-major
    // 128-multiple rows: K steps on whole cache lines and 4-byte scale words
    // (DGRAD: also K % 128, as B's experts start at multiples of K)
    const bool aligned = lda % 128 == 0 && ldb % 128 == 0 && (mode == NVQ_WGRAD || K % 128 == 0) &&
                         (reinterpret_cast<uintptr_t>(a_scales) & 3u) == 0 &&
                         (reinterpret_cast<uintptr_t>(b_scales) & 3u) == 0;
    // scale words four steps at a time: whole groups of steps (the 16-byte
    // group loads need only the 4-byte alignment of the aligned path)
    const bool grouped = aligned && K % 512 == 0;
    const dim3 grid(mx_gemm_grid());
    if (mode == NVQ_DGRAD) {
        launch_tile_offsets(seg_offsets, E, kXTM, aux, nullptr, s);
        p.tiles = aux;
        if (out_bf16) {
            if (grouped)
                hipLaunchKernelGGL((k_grouped_gemm_mxfp8<NVQ_DGRAD, true, true, true>), grid, dim3(256), 0, s, p);
            else if (aligned)
                hipLaunchKernelGGL((k_grouped_gemm_mxfp8<NVQ_DGRAD, true, false, true>), grid, dim3(256), 0, s, p);
            else
                hipLaunchKernelGGL((k_grouped_gemm_mxfp8<NVQ_DGRAD, false, false, true>), grid, dim3(256), 0, s, p);
        } else if (grouped)
            hipLaunchKernelGGL((k_grouped_gemm_mxfp8<NVQ_DGRAD, true, true>), grid, dim3(256), 0, s, p);
        else if (aligned)
            hipLaunchKernelGGL((k_grouped_gemm_mxfp8<NVQ_DGRAD, true, false>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((k_grouped_gemm_mxfp8<NVQ_DGRAD, false, false>), grid, dim3(256), 0, s, p);
    } else {
        hipLaunchKernelGGL(k_pad_offsets, dim3(1), dim3(1024), 0, s, seg_offsets, (int)E, (int64_t)0, aux);
        p.kpad = aux;
        p.m_tiles = (int)((M + kXTM - 1) / kXTM);
        if (aligned)
            hipLaunchKernelGGL((k_grouped_gemm_mxfp8<NVQ_WGRAD, true, false>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((k_grouped_gemm_mxfp8<NVQ_WGRAD, false, false>), grid, dim3(256), 0, s, p);
    }
    return launch_status();
}

extern "C" {

int moe_grouped_gemm_mxfp8(int mode, const uint8_t* a_elems, const uint8_t* a_scales, const uint8_t* b_elems,
                           const uint8_t* b_scales, const int32_t* seg_offsets, int64_t lda, int64_t ldb, int64_t E,
                           int64_t M, int64_t N, int64_t K, float* out, void* ws, size_t ws_bytes,
                           nvq_stream_t stream) {
    if (!out) return NVQ_ERR_NULL;
    return mx_grouped_gemm(mode, a_elems, a_scales, b_elems, b_scales, seg_offsets, lda, ldb, E, M, N, K, out,
                           nullptr, nullptr, ws, ws_bytes, stream);
}

int swiglu_bwd(const float* dH, const uint16_t* gu, int64_t n, int64_t d_ff, uint16_t* dA, nvq_stream_t stream) {
    if (!dH || !gu || !dA) return NVQ_ERR_NULL;
    if (n < 0 || d_ff <= 0) return NVQ_ERR_DIM;
    const int64_t total = n * d_ff;
    if (total == 0) return NVQ_OK;
    if (d_ff % 8 == 0 && aligned16(dH) && aligned16(gu) && aligned16(dA) && total / 8 < ((int64_t)1 << 31)) {
        const int64_t units = total / 8;
        int64_t g = (units + 255) / 256;
        if (g > 8192) g = 8192;
        hipLaunchKernelGGL(k_swiglu_bwd8, dim3((unsigned)g), dim3(256), 0, as_stream(stream),
                           reinterpret_cast<const float4*>(dH), reinterpret_cast<const uint4*>(gu), (int)units,
                           (int)(d_ff / 8), reinterpret_cast<uint4*>(dA));
        return launch_status();
    }
    int64_t g = (total + 255) / 256;
    if (g > 16384) g = 16384;
    hipLaunchKernelGGL(k_swiglu_bwd, dim3((unsigned)g), dim3(256), 0, as_stream(stream), dH, gu, n, d_ff, dA);
    return launch_status();
}


int swiglu_fwd(const float* G, int64_t n, int64_t d_ff, uint16_t* H, nvq_stream_t stream) {
    if (!G || !H) return NVQ_ERR_NULL;
    if (n < 0 || d_ff <= 0 || d_ff % 8 != 0 || n * d_ff / 8 >= ((int64_t)1 << 31)) return NVQ_ERR_DIM;
    if (!aligned16(G) || !aligned16(H)) return NVQ_ERR_ALIGN;
    const int64_t units = n * d_ff / 8;
    if (units == 0) return NVQ_OK;
    hipLaunchKernelGGL(k_swiglu_fwd8, dim3(elementwise_grid(units)), dim3(256), 0, as_stream(stream),
                       reinterpret_cast<const float4*>(G), (int)units, (int)(d_ff / 8), reinterpret_cast<uint4*>(H));
    return launch_status();
}

}  // extern "C"
