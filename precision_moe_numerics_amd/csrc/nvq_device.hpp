// nvq_device.hpp -- device-side numerics shared by the gfx950 kernels of
// libnvq.so: bf16, E2M1, E4M3 and E8M0 codecs, Philox4x32-10, and wave64
// reductions. Everything here is exact integer or single-rounding fp32 work,
// so the same inputs give the same bits on every launch shape.
//
// Formats: NVFP4 (E2M1 codes, E4M3 scale per 16, fp32 tensor scale; the
// ~4.5 bits/value of page "Thinking Machines Details End-to-End 4-Bit
// Training for Inkling 2 Small", section "Background") and MXFP8 (E4M3
// elements, E8M0 scale per 32; the backward format of the same page,
// section "Key Takeaways").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvq {

constexpr float kFltMax = 3.40282346638528859812e+38f;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, nearest even (finite inputs; infinities pass through).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 values -> their bf16 pair (a in the low half), nearest-even, by
// the gfx950 pair converter (v_cvt_pk_bf16_f32): for finite values the same
// bits as f32_to_bf16, in one instruction.
typedef __bf16 nvq_bf16x2 __attribute__((ext_vector_type(2)));
typedef float nvq_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((nvq_f32x2){a, b}, nvq_bf16x2));
}

// ---------------------------------------------------------------- E4M3 (FN)
// Magnitude byte (0..0x7E) of the nearest E4M3 value to a >= 0, ties to even
// mantissa, saturating at 448. Subnormals (below 2^-6) have spacing 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne_mag(float a) {
    a = fminf(a, 448.0f);
    if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8, exact scaling
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);  // keep 3 mantissa bits, carry into exponent
    return (u >> 20) - (120u << 3);    // rebias 127 -> 7
}

// Value of an E4M3 magnitude byte (0..0x7E).
__device__ __forceinline__ float e4m3_mag_to_f32(uint32_t b) {
    uint32_t e = b >> 3, m = b & 7u;
    if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Stochastic E4M3 rounding of a >= 0 with a 16-bit draw u: the two
// neighbours lo <= a < hi are a's value truncated to 3 mantissa bits and the
// next grid value; round up iff u < frac * 2^16, where frac is the truncated
// remainder over the spacing (an exact integer comparison).
__device__ __forceinline__ uint32_t e4m3_sr_mag(float a, uint32_t u16) {
    if (a >= 448.0f) return 0x7Eu;
    if (a < 0.015625f) {
        float n = a * 512.0f;              // exact
        float lo = __builtin_floorf(n);
        float f = n - lo;                  // exact
        uint32_t up = (float)u16 < f * 65536.0f ? 1u : 0u;
        return (uint32_t)lo + up;          // 8 == 2^-6, the first normal
    }
    uint32_t u = __float_as_uint(a);
    uint32_t rem = u & 0xFFFFFu;           // 20 dropped mantissa bits
    uint32_t up = (u16 << 4) < rem ? 1u : 0u;
    return ((u >> 20) - (120u << 3)) + up; // carry into the exponent is exact
}

// ---------------------------------------------------------------- E2M1
// Code (with sign bit 3) of the nearest E2M1 value to y, ties to the even code,
// saturating at 6; the sign of y is kept even when the magnitude rounds to 0.
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
    float a = fabsf(y);
    uint32_t s = (__float_as_uint(y) >> 28) & 8u;
    uint32_t c;
    if (a < 1.0f) {
        c = (uint32_t)__builtin_rintf(a * 2.0f);          // 0, 0.5, 1.0 -> codes 0..2
    } else {
        uint32_t u = __float_as_uint(a);
        u += 0x1FFFFFu + ((u >> 22) & 1u);                 // keep 1 mantissa bit
        c = min((u >> 22) - 252u, 7u);                      // exponent 127 -> code 2
    }
    return c | s;
}

// Stochastic E2M1 rounding: lo = largest grid value <= |y|, round up iff
// u < (|y| - lo) / step * 2^16 (all steps exact); |y| >= 6 saturates.
// Branch-free: the binade [0,2), [2,4) or [4,6) picks the step (0.5, 1, 2)
// by selects, lo = floor(a / step) * step, code = lo / step + (0, 2, 4).
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u16) {
    const float a = fabsf(y);
    const uint32_t s = (__float_as_uint(y) >> 28) & 8u;
    const bool b2 = a < 2.0f, b4 = a < 4.0f;
    const float inv_step = b2 ? 2.0f : b4 ? 1.0f : 0.5f;
    const float step = b2 ? 0.5f : b4 ? 1.0f : 2.0f;
    const float lo = __builtin_floorf(fminf(a, 5.0f) * inv_step) * step;  // exact
    const uint32_t c = (uint32_t)(lo * inv_step) + (b2 ? 0u : b4 ? 2u : 4u);
    const float f = (a - lo) * inv_step;  // exact (Sterbenz, power-of-two step)
    const uint32_t up = (float)u16 < f * 65536.0f ? 1u : 0u;
    return (a >= 6.0f ? 7u : c + up) | s;
}

// ---------------------------------------------------------------- Philox4x32-10
// Counter-based generator of Salmon et al. (SC'11): ten rounds, each two
// 32x32->64 multiplies, key bumped by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        // one 32x32->64 product each (a single v_mad_u64_u32 rather than
        // separate low and high multiplies)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
        c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// The eight 16-bit draws of elements 8*g .. 8*g+7 of a tensor: element
// 8*g + j takes half (j & 1) of word (j >> 1) of counter (lo(g), hi(g),
// stream, 0) under key (lo(seed), hi(seed)).
__device__ __forceinline__ uint4 draws8(uint64_t g, uint32_t stream, uint64_t seed) {
    return philox10(make_uint4((uint32_t)g, (uint32_t)(g >> 32), stream, 0u), (uint32_t)seed,
                    (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t draw_of(const uint4& w, int j) {
    uint32_t word = (j >> 1) == 0 ? w.x : (j >> 1) == 1 ? w.y : (j >> 1) == 2 ? w.z : w.w;
    return (word >> (16 * (j & 1))) & 0xFFFFu;
}

// ---------------------------------------------------------------- wave64 helpers
// Swap with the neighbouring lane (lane ^ 1) through a DPP quad permutation.
__device__ __forceinline__ float dpp_swap1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
// Swap with lane ^ 2 (quad_perm 2,3,0,1).
__device__ __forceinline__ float dpp_swap2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}


// E4M3 scale byte of a 16-value block with max |x| amb under the tensor's
// encode scale S, and the multiplier that takes a block with scale byte b to
// the E2M1 grid (0 for an all-zero block).
__device__ __forceinline__ uint32_t nvfp4_scale_byte(float amb, float S) { return e4m3_rne_mag((amb / 6.0f) * S); }
__device__ __forceinline__ float nvfp4_scale_mult(uint32_t b, float S) {
    return b ? fminf(S / e4m3_mag_to_f32(b), kFltMax) : 0.0f;
}

// ---------------------------------------------------------------- NVFP4 encode of one lane
// One lane holds 8 consecutive values of a 16-value block whose other half
// sits in lane ^ 1. Given the tensor's encode scale S: block byte = nearest-
// even E4M3 of (amax_block / 6) * S (saturating), r = S / e4m3(byte) (0 for
// byte 0, clamped to FLT_MAX), codes = E2M1 of x * r, nearest-even or
// stochastic with the eight Philox draws of unit `unit` (elements 8*unit..).
// Returns the packed code word (element 0 in the low nibble); *sc gets the byte.
template <int MODE>
__device__ __forceinline__ uint32_t nvfp4_encode8(const float (&f)[8], float S, uint32_t* sc,
                                                  uint64_t unit, uint32_t stream_id, uint64_t seed) {
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(f[j]));
    const float amb = fmaxf(am, dpp_swap1(am));
    const uint32_t b = nvfp4_scale_byte(amb, S);
    const float r = nvfp4_scale_mult(b, S);
    uint32_t word = 0;
    if (MODE == 0) {
        // gfx950 converter, scale 1.0: nearest-even, saturating at 6, sign of
        // zero kept (checked against e2m1_rne on every fp32 input); src0 goes
        // to the low nibble of the selected byte.
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, f[0] * r, f[1] * r, 1.0f, 0);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, f[2] * r, f[3] * r, 1.0f, 1);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, f[4] * r, f[5] * r, 1.0f, 2);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, f[6] * r, f[7] * r, 1.0f, 3);
    } else {
        const uint4 dr = draws8(unit, stream_id, seed);
#pragma unroll
        for (int j = 0; j < 8; ++j) word |= e2m1_sr(f[j] * r, draw_of(dr, j)) << (4 * j);
    }
    *sc = b;
    return word;
}

// Encode scale S and stored decode scale D of a tensor with maximum |x| amax.
__device__ __forceinline__ float nvfp4_encode_scale(float amax) {
    return amax > 0.0f ? fminf(2688.0f / amax, kFltMax) : 1.0f;
}
__device__ __forceinline__ float nvfp4_decode_scale(float amax) {
    return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

// Stores the scale bytes of a wave's 32 blocks: lanes 8g..8g+7 hold units
// 8g..8g+7 = blocks 4g..4g+3 (each byte owned by the even lane). Whole 32-bit
// words where the group is complete and aligned, single bytes otherwise.
// Must be called by all 64 lanes.
__device__ __forceinline__ void store_block_scales(uint8_t* sb, int64_t u, int64_t n_units, uint32_t sc) {
    const int lane = threadIdx.x & 63;
    const uint32_t s2 = __shfl_down(sc, 2, 64), s4 = __shfl_down(sc, 4, 64), s6 = __shfl_down(sc, 6, 64);
    const bool whole = ((u | 7) < n_units) && (((reinterpret_cast<uintptr_t>(sb) + (uintptr_t)(u / 2)) & 3u) == 0);
    const bool whole_group = __shfl((int)whole, lane & ~7, 64) != 0;
    if (whole_group) {
        if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(sb + u / 2) = sc | (s2 << 8) | (s4 << 16) | (s6 << 24);
    } else if (u < n_units && (lane & 1) == 0) {
        sb[u / 2] = (uint8_t)sc;
    }
}

// ---------------------------------------------------------------- tensor maxima
// A tensor's max |x| is kept as G partial maxima (fp32 bits of non-negative
// values, so unsigned order is float order), each written by one workgroup
// or wave with a plain store; the consumer folds them. This avoids G
// same-address atomics, which the memory system serializes.

// Max over a 256-thread block of a per-thread value; the result is returned
// to every thread. Must be reached by all threads of the block.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t m) {
    __shared__ uint32_t red[4];
    m = wave_max_u32(m);
    __syncthreads();  // red may still be read by an earlier call
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    return max(max(red[0], red[1]), max(red[2], red[3]));
}

// Max of partial maxima part[0..G) as a float, in every thread of a
// 256-thread block.
__device__ __forceinline__ float block_max_partials(const uint32_t* __restrict__ part, int G) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < G; i += 256) m = max(m, part[i]);
    return __uint_as_float(block_max_u32(m));
}

// Units (16-byte loads) a lane of the streaming kernels keeps in flight.
constexpr int kStreamP = 4;

// Contiguous share of workgroup g out of G over n units: a multiple of 64
// units (one unit per lane), so every wave starts on a 64-unit boundary.
__device__ __forceinline__ void block_chunk(int64_t n, int64_t g, int64_t G, int64_t* beg, int64_t* end) {
    const int64_t c = ((n + G - 1) / G + 63) & ~(int64_t)63;
    *beg = min(n, g * c);
    *end = min(n, *beg + c);
}

// Exclusive prefix sum over a 1024-thread block (Hillis-Steele in LDS);
// *total receives the sum over the block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* buf, int* total) {
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int add = t >= off ? buf[t - off] : 0;
        __syncthreads();
        buf[t] += add;
        __syncthreads();
    }
    const int incl = buf[t];
    *total = buf[1023];
    __syncthreads();
    return incl - v;
}

}  // namespace nvq
