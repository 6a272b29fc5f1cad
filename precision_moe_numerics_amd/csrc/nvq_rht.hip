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
// Layout on the wave: a chunk is 4 lanes x 8 values (16-byte loads). Strides
// 1, 2, 4 stay inside a lane; strides 8 and 16 pair lanes 1 and 2 apart and
// use DPP quad permutations. A 16-value NVFP4 block is a lane pair, as in
// the plain quantizer, so the encode step is shared with it.
#include "nvq_device.hpp"
#include "nvq_host.hpp"

namespace nvq {

constexpr float kInvSqrt32 = 0x1.6a09e6p-3f;  // fp32 nearest to 1/sqrt(32)

__device__ __forceinline__ uint32_t rht_sign_word(uint64_t sign_seed) {
    return philox10(make_uint4(0u, 0u, 4u, 0u), (uint32_t)sign_seed, (uint32_t)(sign_seed >> 32)).x;
}

// In-lane stages (strides 1, 2, 4) of the butterfly on 8 values.
__device__ __forceinline__ void butterfly8(float (&v)[8]) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
}

// Cross-lane stage with partner lane ^ (h/8): the lane holding the lower
// index keeps a + b, the other keeps a - b (a = lower value, b = upper). Both
// are one addition o + t of the partner's value o and this lane's own value
// t = v (lower lane) or t = -v (upper lane, a sign flip, exact), so a stage is
// a sign XOR plus one DPP-fed add per value.
template <int H>
__device__ __forceinline__ void butterfly_cross(float (&v)[8], int lane) {
    const uint32_t flip = (lane & (H / 8)) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float o = (H == 8) ? dpp_swap1(v[i]) : dpp_swap2(v[i]);
        v[i] = o + __uint_as_float(__float_as_uint(v[i]) ^ flip);
    }
}

// Full forward transform of one lane's 8 values (lane holds chunk positions
// 8*(lane&3) .. +7); sign bits applied first, the 1/sqrt(32) factor last.
__device__ __forceinline__ void rht32_lane(float (&v)[8], uint32_t signs, int lane) {
    const int p0 = (lane & 3) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if ((signs >> (p0 + i)) & 1u) v[i] = -v[i];
    butterfly8(v);
    butterfly_cross<8>(v, lane);
    butterfly_cross<16>(v, lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= kInvSqrt32;
}

__device__ __forceinline__ void load8_bf16(const uint4& w, float (&f)[8]) {
    f[0] = bf16_to_f32(w.x & 0xFFFFu); f[1] = bf16_to_f32(w.x >> 16);
    f[2] = bf16_to_f32(w.y & 0xFFFFu); f[3] = bf16_to_f32(w.y >> 16);
    f[4] = bf16_to_f32(w.z & 0xFFFFu); f[5] = bf16_to_f32(w.z >> 16);
    f[6] = bf16_to_f32(w.w & 0xFFFFu); f[7] = bf16_to_f32(w.w >> 16);
}

// Pass 1: max |z| over each workgroup's contiguous chunk (z is not stored),
// stored as that workgroup's partial maximum. n8 = units of 8 values. As in
// the plain quantizer, a lane issues kStreamP loads (units 256 apart,
// indices clamped into the chunk; a re-read unit leaves the max unchanged)
// before transforming them; trip counts are wave-uniform for the DPP stages.
__global__ __launch_bounds__(256) void k_rht32_amax(const uint4* __restrict__ y, int64_t n8, uint64_t sign_seed,
                                                    uint32_t* __restrict__ part) {
    const uint32_t signs = rht_sign_word(sign_seed);
    const int lane = threadIdx.x & 63;
    int64_t beg, end;
    block_chunk(n8, blockIdx.x, gridDim.x, &beg, &end);
    float m = 0.0f;
    for (int64_t wb = beg + (threadIdx.x & ~63); wb < end; wb += 256 * kStreamP) {
        uint4 w[kStreamP];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) w[p] = y[min(wb + lane + 256 * p, end - 1)];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) {
            float v[8];
            load8_bf16(w[p], v);
            rht32_lane(v, signs, lane);
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
        }
    }
    const uint32_t mb = block_max_u32(__float_as_uint(m));
    if (threadIdx.x == 0) part[blockIdx.x] = mb;
}

// Pass 2: recompute z and encode it to NVFP4 (nearest even); the tensor
// maximum is folded from the n_part partial maxima of pass 1.
__global__ __launch_bounds__(256) void k_rht32_quant(const uint4* __restrict__ y, int64_t n8, uint64_t sign_seed,
                                                     const uint32_t* __restrict__ part, int n_part,
                                                     uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                     float* __restrict__ tscale) {
    const uint32_t signs = rht_sign_word(sign_seed);
    const float amax = block_max_partials(part, n_part);
    const bool zero = !(amax > 0.0f);
    const float S = nvfp4_encode_scale(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) tscale[0] = nvfp4_decode_scale(amax);
    const int lane = threadIdx.x & 63;
    int64_t beg, end;
    block_chunk(n8, blockIdx.x, gridDim.x, &beg, &end);
    for (int64_t wb = beg + (threadIdx.x & ~63); wb < end; wb += 256 * kStreamP) {
        uint4 w[kStreamP];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) w[p] = y[min(wb + lane + 256 * p, end - 1)];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) {
            const int64_t u = wb + lane + 256 * p;
            float v[8];
            load8_bf16(w[p], v);
            rht32_lane(v, signs, lane);
            uint32_t sc;
            uint32_t word = nvfp4_encode8<0>(v, S, &sc, (uint64_t)u, 0u, 0ull);
            if (zero) { word = 0; sc = 0; }
            if (u < end) codes[u] = word;
            store_block_scales(scales, u, end, sc);
        }
    }
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

// Butterfly with strides 1, 2, 4, 8, 16 on one lane's 32 values.
__device__ __forceinline__ void butterfly32(float (&v)[32]) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_rht32_combine(const uint4* __restrict__ codes,
                                                       const uint16_t* __restrict__ scales,
                                                       const float* __restrict__ tscale, int64_t T, int k,
                                                       int64_t chunks_per_row, uint64_t sign_seed,
                                                       const float* __restrict__ w, uint4* __restrict__ out) {
    const uint32_t signs = rht_sign_word(sign_seed);
    const float D = tscale[0];
    // 32-bit index math: the host guarantees T * k * chunks_per_row < 2^31
    const uint32_t nc = (uint32_t)(T * chunks_per_row), cpr = (uint32_t)chunks_per_row;
    constexpr int kS = 4;  // slots whose loads are in flight together
    for (uint32_t u = blockIdx.x * 256u + threadIdx.x; u < nc; u += gridDim.x * 256u) {
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
                cw[j] = ok ? codes[src] : make_uint4(0u, 0u, 0u, 0u);
                sc[j] = ok ? scales[src] : 0u;
                ws[j] = ok ? w[t * (uint32_t)k + (uint32_t)sl] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < kS; ++j) {
                const float f0 = (ws[j] * D) * e4m3_mag_to_f32(sc[j] & 0x7Fu);         // values 0-15
                const float f1 = (ws[j] * D) * e4m3_mag_to_f32((sc[j] >> 8) & 0x7Fu);  // values 16-31
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
            uint32_t b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float y = acc[8 * q + i] * kInvSqrt32;
                if ((signs >> (8 * q + i)) & 1u) y = -y;
                b[i] = f32_to_bf16(y);
            }
            r[q] = make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) out[4 * (size_t)u + q] = r[q];
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

size_t rht32_blockquant_workspace_size(int64_t R, int64_t C) {
    Carver c(nullptr);
    c.take<uint32_t>((size_t)stream_blocks(R * C / 8, 1));
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
    const int64_t n8 = R * C / 8;
    const int G = stream_blocks(n8, 1);
    const auto yk = reinterpret_cast<const uint4*>(y);
    hipLaunchKernelGGL(k_rht32_amax, dim3((unsigned)G), dim3(256), 0, s, yk, n8, sign_seed, part);
    hipLaunchKernelGGL(k_rht32_quant, dim3((unsigned)G), dim3(256), 0, s, yk, n8, sign_seed, part, G,
                       reinterpret_cast<uint32_t*>(codes), scales, tscale);
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
