// nvq_rht.hip -- 32-point random Hadamard transform + NVFP4 of the expert-
// combine tensor, and the receiving side (dequantize, inverse transform,
// weighted top-k combine).
//
// Once the NVFP4 forward got faster, expert-parallel communication became the
// bottleneck, so the combine traffic is quantized to a block-scaled format
// after a 32-dimensional random Hadamard transform (page "Thinking Machines
// Details End-to-End 4-Bit Training for Inkling 2 Small", sections "Key
// Takeaways" and "Architecture highlights"). The block-scaled format here is
// NVFP4, the forward format of the same recipe.
//
// Transform: z = (1/sqrt 32) H32 (s .* x) for every contiguous 32-value chunk
// of a row, H32 in natural (Sylvester) order, one 32-sign vector s for the
// tensor (bit j of the first Philox4x32-10 word at counter (0,0,4,0) under
// the sign seed; a set bit negates). The butterfly runs in fp32 with strides
// 1, 2, 4, 8, 16 in that order, each stage (a, b) -> (a + b, a - b); the
// quantizer decides on these fp32 values, so the order is part of the
// definition.
//
// Layout on the wave: one lane owns a whole 32-value chunk, so the butterfly
// runs in its registers with no cross-lane step and a 16-value NVFP4 block is
// half a lane. Loads stay coalesced: each wave reads 64 consecutive chunks
// with 16-byte loads and redistributes them through LDS.
#include <algorithm>

#include "nvq_device.hpp"
#include "nvq_host.hpp"

namespace nvq {

// One wave stages 64 chunks (4 KiB of bf16) per trip: lane l loads units
// 64q + l (q = 0..3; coalesced 16-byte loads, indices clamped to the
// workgroup's last unit), writes them to its wave's LDS strip, and reads
// back the four units of chunk l. Unit q of chunk c sits in slot (q + c / 4) % 4
// of the chunk's 64 bytes, which keeps both the writes (16 lanes = 4 whole
// chunks) and the reads (16 lanes = 16 chunks at a 64-byte stride) on 16
// distinct bank groups. The wave's LDS operations complete in issue order,
// so the strip needs no barrier.
__device__ __forceinline__ uint32_t rht_slot(uint32_t c, uint32_t q) { return c * 64u + (((q + (c >> 2)) & 3u) << 4); }

// NT: loads with the non-temporal hint (the pass reads every byte once and,
// for the maximum pass, the tensor is larger than the Infinity Cache).
template <bool NT>
__device__ __forceinline__ void rht_load_strip(const uint4* __restrict__ y, int64_t c0, int64_t c_end, int lane,
                                               uint4 (&w)[4]) {
    const int64_t u_last = 4 * c_end - 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4* p = y + min(4 * c0 + 64 * q + lane, u_last);
        w[q] = NT ? load_stream(p) : *p;
    }
}

__device__ __forceinline__ void rht_stage_chunk(const uint4 (&w)[4], int lane, uint4* strip, float (&v)[32],
                                                const uint32_t (&smask)[16]) {
    uint8_t* sb = reinterpret_cast<uint8_t*>(strip);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t u = 64u * q + (uint32_t)lane;
        *reinterpret_cast<uint4*>(sb + rht_slot(u >> 2, u & 3u)) = w[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 x = *reinterpret_cast<const uint4*>(sb + rht_slot((uint32_t)lane, (uint32_t)q));
        const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // sign flips on the packed pair, then bf16 -> fp32 (exact)
            const uint32_t p = xw[i] ^ smask[4 * q + i];
            v[8 * q + 2 * i] = __uint_as_float(p << 16);
            v[8 * q + 2 * i + 1] = __uint_as_float(p & 0xFFFF0000u);
        }
    }
}

// Sign masks of the 16 packed bf16 pairs of a chunk: bit 15 negates the low
// value (position 2i), bit 31 the high one (2i + 1).
__device__ __forceinline__ void rht_sign_masks(uint32_t signs, uint32_t (&smask)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        smask[i] = (((signs >> (2 * i)) & 1u) << 15) | (((signs >> (2 * i + 1)) & 1u) << 31);
}

// Pass 1: max |z| over each workgroup's contiguous share of chunks (z is not
// stored), stored as that workgroup's partial maximum. fl(|v| / sqrt 32) is
// monotone in |v|, so the maximum of the scaled values is the scaled maximum
// of the butterfly outputs: one multiply per lane instead of one per value.
// The last stage's outputs only enter through their magnitudes, and of
// fl(a + b) and fl(a - b) the larger magnitude is exactly fl(|a| + |b|)
// (one of the two has magnitude |a| + |b|, the other at most that, and
// rounding is sign-symmetric and monotone): one add per pair.
template <bool NT>
__global__ __launch_bounds__(256) void k_rht32_amax(const uint4* __restrict__ y, int64_t n_chunks,
                                                    uint64_t sign_seed, uint32_t* __restrict__ part) {
    __shared__ uint4 strips[4][256];
    uint32_t smask[16];
    rht_sign_masks(rht_sign_word(sign_seed), smask);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t beg, end;
    block_chunk(n_chunks, blockIdx.x, gridDim.x, &beg, &end);
    float m = 0.0f;
    for (int64_t c0 = beg + 64 * wave; c0 < end; c0 += 256) {
        uint4 w[4];
        float v[32];
        rht_load_strip<NT>(y, c0, end, lane, w);
        rht_stage_chunk(w, lane, strips[wave], v, smask);
        butterfly32<16>(v);
        float mc = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) mc = fmaxf(mc, fabsf(v[i]) + fabsf(v[i + 16]));
        // a lane past the share's last chunk staged copies of the last unit
        // (clamped loads), which is no chunk of the tensor: left out
        m = (c0 + lane < end) ? fmaxf(m, mc) : m;
    }
    m *= kInvSqrt32;
    const uint32_t mb = block_max_u32(__float_as_uint(m));
    if (threadIdx.x == 0) part[blockIdx.x] = mb;
}

// The encode loop of k_rht32_quant; FAST: the block-scale quotient by
// div6_fma (S <= kFastDiv6MaxS, uniform over the tensor).
template <bool FAST>
__device__ __forceinline__ void rht_quant_loop(const uint4* __restrict__ y, int64_t beg, int64_t end, int lane,
                                               int wave, uint4* strip, const uint32_t (&smask)[16], float S,
                                               bool zero, const float* rtab, uint4* __restrict__ codes,
                                               uint16_t* __restrict__ scales) {
    for (int64_t c0 = beg + 64 * wave; c0 < end; c0 += 256) {
        uint4 w[4];
        float v[32];
        rht_load_strip<true>(y, c0, end, lane, w);
        rht_stage_chunk(w, lane, strip, v, smask);
        butterfly32(v);
        uint32_t word[4], sc[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            float z[16];
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                z[i] = v[16 * blk + i] * kInvSqrt32;
                am = fmaxf(am, fabsf(z[i]));
            }
            sc[blk] = nvfp4_scale_byte_hw<FAST>(am, S);
            const float r = rtab[sc[blk] & 0x7Fu];  // byte <= 0x7E for finite inputs
#pragma unroll
            for (int hw = 0; hw < 2; ++hw) {
                // gfx950 converter at scale 1.0: nearest even, saturating at 6
                uint32_t wd = 0;
                const float* zz = z + 8 * hw;
                wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, zz[0] * r, zz[1] * r, 1.0f, 0);
                wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, zz[2] * r, zz[3] * r, 1.0f, 1);
                wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, zz[4] * r, zz[5] * r, 1.0f, 2);
                wd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wd, zz[6] * r, zz[7] * r, 1.0f, 3);
                word[2 * blk + hw] = wd;
            }
        }
        const int64_t c = c0 + lane;
        if (c < end) {
            codes[c] = zero ? make_uint4(0u, 0u, 0u, 0u) : make_uint4(word[0], word[1], word[2], word[3]);
            scales[c] = zero ? (uint16_t)0 : (uint16_t)(sc[0] | (sc[1] << 8));
        }
    }
}

// Pass 2: recompute z and encode it to NVFP4 (nearest even); the tensor
// maximum is folded from the n_part partial maxima of pass 1. A lane owns
// one chunk = two 16-value blocks: its 16 code bytes go out as one 16-byte
// store and its two scale bytes as one 2-byte store (consecutive across the
// wave). A block's multiplier min(S / e4m3(b), FLT_MAX) depends only on its
// scale byte b, so the workgroup divides once per byte value into an LDS
// table instead of twice per block (same quotients, bit for bit).
__global__ __launch_bounds__(256) void k_rht32_quant(const uint4* __restrict__ y, int64_t n_chunks,
                                                     uint64_t sign_seed, const uint32_t* __restrict__ part,
                                                     int n_part, uint4* __restrict__ codes,
                                                     uint16_t* __restrict__ scales, float* __restrict__ tscale) {
    __shared__ uint4 strips[4][256];
    __shared__ float rtab[128];
    uint32_t smask[16];
    rht_sign_masks(rht_sign_word(sign_seed), smask);
    const float amax = block_max_partials(part, n_part);
    const bool zero = !(amax > 0.0f);
    const float S = nvfp4_encode_scale(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) tscale[0] = nvfp4_decode_scale(amax);
    if (threadIdx.x < 128) {
        const uint32_t b = threadIdx.x;
        rtab[b] = nvfp4_scale_mult(b, S);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t beg, end;
    block_chunk(n_chunks, blockIdx.x, gridDim.x, &beg, &end);
    if (S <= kFastDiv6MaxS)
        rht_quant_loop<true>(y, beg, end, lane, wave, strips[wave], smask, S, zero, rtab, codes, scales);
    else
        rht_quant_loop<false>(y, beg, end, lane, wave, strips[wave], smask, S, zero, rtab, codes, scales);
}

// Receiving side: out[t][p] = sum_s w[t][s] * y'[t*k+s][p], y' = s .* (H32
// z' / sqrt 32), z' = (e2m1 * e4m3) * D, rounded to bf16. The inverse
// transform and the sign flips are linear, so they are applied once to the
// weighted sum of the dequantized slots instead of once per slot:
//   acc = sum_s (w[t][s] * D * e4m3_s) * e2m1_s   (fp32, fma per value)
//   out = bf16(s .* (H32 acc) / sqrt 32)
// (k times fewer butterflies; the fp32 rounding differs from the per-slot
// order by a few fp32 ulps, far inside the bf16 result). E2M1 codes are
// decoded by the gfx950 fp4 -> fp32 converter (exact). One lane produces one
// whole 32-value chunk of an output row: per slot it loads the chunk's 16
// code bytes and its two scale bytes (16- and 2-byte loads, consecutive
// across the lanes of a row), and the whole butterfly runs in its registers.
typedef float f32x2v __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void k_rht32_combine(const uint4* __restrict__ codes,
                                                       const uint16_t* __restrict__ scales,
                                                       const float* __restrict__ tscale, int64_t T, int k,
                                                       int64_t chunks_per_row, uint64_t sign_seed,
                                                       const float* __restrict__ w, uint4* __restrict__ out) {
    const uint32_t signs = rht_sign_word(sign_seed);
    const float D = tscale[0];
    // 32-bit index math: the host guarantees T * k * chunks_per_row < 2^31
    const uint32_t nc = (uint32_t)(T * chunks_per_row), cpr = (uint32_t)chunks_per_row;
    constexpr int kS = 8;  // slots whose loads are in flight together
    // output staging: a lane's 64 bytes go through its wave's 4 KiB strip so
    // that each 16-byte store instruction covers 1 KiB of consecutive output
    __shared__ uint4 xs[4][256];
    const uint32_t lane = threadIdx.x & 63u;
    uint4* xw = xs[threadIdx.x >> 6];
    // wave-uniform trip count (the strip exchange needs every lane); a lane
    // past the last chunk recomputes the last one and stores nothing
    for (uint32_t ub = blockIdx.x * 256u + (threadIdx.x & ~63u); ub < nc; ub += gridDim.x * 256u) {
        const uint32_t u = min(ub + lane, nc - 1u);
        const uint32_t t = u / cpr, cb = u - t * cpr;
        float acc[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] = 0.0f;
        for (int s0 = 0; s0 < k; s0 += kS) {
            uint4 cw[kS];
            uint32_t sc[kS];
            float ws[kS];
#pragma unroll
            for (int j = 0; j < kS; ++j) {
                const int sl = s0 + j;
                const bool ok = sl < k;
                const uint32_t src = (t * (uint32_t)k + (uint32_t)sl) * cpr + cb;
                cw[j] = ok ? load_stream(codes + src) : make_uint4(0u, 0u, 0u, 0u);
                sc[j] = ok ? scales[src] : 0u;
                ws[j] = ok ? w[t * (uint32_t)k + (uint32_t)sl] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < kS; ++j) {
                // both E4M3 scale bytes by the hardware converter
                const nvq_f32x2 sv = e4m3_pair_to_f32(sc[j]);
                const float f0 = (ws[j] * D) * sv.x;  // values 0-15
                const float f1 = (ws[j] * D) * sv.y;  // values 16-31
                const uint32_t word[4] = {cw[j].x, cw[j].y, cw[j].z, cw[j].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float f = q < 2 ? f0 : f1;
                    f32x2v v[4];
                    v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word[q], 1.0f, 0);
                    v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word[q], 1.0f, 1);
                    v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word[q], 1.0f, 2);
                    v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word[q], 1.0f, 3);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[8 * q + 2 * i] = __builtin_fmaf(f, v[i].x, acc[8 * q + 2 * i]);
                        acc[8 * q + 2 * i + 1] = __builtin_fmaf(f, v[i].y, acc[8 * q + 2 * i + 1]);
                    }
                }
            }
        }
        butterfly32(acc);
        uint4 r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                y[i] = acc[8 * q + i] * kInvSqrt32;
                if ((signs >> (8 * q + i)) & 1u) y[i] = -y[i];
            }
            r[q] = make_uint4(bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3]), bf16x2_rne(y[4], y[5]),
                              bf16x2_rne(y[6], y[7]));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) xw[4 * lane + q] = r[q];
        // in-order LDS within the wave: the reads below see these writes
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t unit = 64u * q + lane;  // 16-byte unit of the wave's 64 chunks
            if (ub + unit / 4u < nc) out[4 * (size_t)ub + unit] = xw[unit];
        }
    }
}

static unsigned stream_grid(int64_t n8) {
    int64_t g = (n8 + 255) / 256;
    if (g > 8192) g = 8192;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace nvq

using namespace nvq;

extern "C" {

// partial maxima: at most one per workgroup of a resident grid (8 per CU at
// most for these kernels' LDS use), over-allocated for 2048 CUs' worth
size_t rht32_blockquant_workspace_size(int64_t R, int64_t C) {
    Carver c(nullptr);
    const int64_t g = std::max<int64_t>(1, std::min<int64_t>((R * C / 32 + 255) / 256, 16384));
    c.take<uint32_t>((size_t)g);
    return c.need;
}

int rht32_blockquant(const uint16_t* y, int64_t R, int64_t C, uint64_t sign_seed, uint8_t* codes, uint8_t* scales,
                     float* tscale, void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!y || !codes || !scales || !tscale || !ws) return NVQ_ERR_NULL;
    if (R < 0 || C <= 0 || (C % 32) != 0) return NVQ_ERR_DIM;
    if (!aligned16(y) || !aligned16(codes) || !aligned16(scales) || !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < rht32_blockquant_workspace_size(R, C)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    uint32_t* part = static_cast<uint32_t*>(ws);
    const int64_t n_chunks = R * C / 32;
    const bool nt = R * C * 2 >= kStreamHintBytes;
    // grids of the two passes: as many workgroups as stay resident together
    // (one round, no second partial round), each at least one trip of 256
    // chunks; the maximum pass's two variants use the same registers
    static const int res_amax = resident_blocks((const void*)k_rht32_amax<true>);
    static const int res_quant = resident_blocks((const void*)k_rht32_quant);
    const int64_t trips = (n_chunks + 255) / 256;
    const int G = (int)std::max<int64_t>(1, std::min<int64_t>(trips, (int64_t)device_cus() * res_amax));
    const int Gq = (int)std::max<int64_t>(1, std::min<int64_t>(trips, (int64_t)device_cus() * res_quant));
    const auto yk = reinterpret_cast<const uint4*>(y);
    if (nt)
        hipLaunchKernelGGL(k_rht32_amax<true>, dim3((unsigned)G), dim3(256), 0, s, yk, n_chunks, sign_seed, part);
    else
        hipLaunchKernelGGL(k_rht32_amax<false>, dim3((unsigned)G), dim3(256), 0, s, yk, n_chunks, sign_seed, part);
    hipLaunchKernelGGL(k_rht32_quant, dim3((unsigned)Gq), dim3(256), 0, s, yk, n_chunks, sign_seed, part, G,
                       reinterpret_cast<uint4*>(codes), reinterpret_cast<uint16_t*>(scales), tscale);
    return launch_status();
}

int rht32_dequant_combine(const uint8_t* codes, const uint8_t* scales, const float* tscale, int64_t T, int k,
                          int64_t C, uint64_t sign_seed, const float* w, uint16_t* out, nvq_stream_t stream) {
    if (!codes || !scales || !tscale || !w || !out) return NVQ_ERR_NULL;
    if (T < 0 || k < 1 || C <= 0 || (C % 32) != 0) return NVQ_ERR_DIM;
    if (T * (int64_t)k * (C / 8) >= ((int64_t)1 << 31)) return NVQ_ERR_DIM;
    if (!aligned16(codes) || !aligned16(out) || (reinterpret_cast<uintptr_t>(scales) & 1u)) return NVQ_ERR_ALIGN;
    const int64_t cpr = C / 32;  // 32-value chunks per row
    const int64_t nc = T * cpr;
    if (nc == 0) return NVQ_OK;
    hipLaunchKernelGGL(k_rht32_combine, dim3(stream_grid(nc)), dim3(256), 0, as_stream(stream),
                       reinterpret_cast<const uint4*>(codes), reinterpret_cast<const uint16_t*>(scales), tscale, T,
                       k, cpr, sign_seed, w, reinterpret_cast<uint4*>(out));
    return launch_status();
}

}  // extern "C"
