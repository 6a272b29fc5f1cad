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

// The two E4M3 bytes of the low half of w as fp32 (byte 0 in x), by the
// gfx950 converter at scale 1: exact, OCP E4M3 with the sign bit honoured and
// 0x7F / 0xFF as NaN (checked on all 65536 pairs through nvq_convert_probe).
typedef float nvq_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ nvq_f32x2 e4m3_pair_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
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

// The same decision, with the sign of a attached, by the gfx950 stochastic
// converter (v_cvt_scalef32_sr_fp8_f32) with random operand ~(u << 16) | 0xFFFF:
// it adds the operand's top bits to the value's fraction of its grid step,
// which equals the rule for a fraction of at most 20 bits, as every normal
// E4M3 range gives but the subnormal steps of 2^-9 below 2^-6 do not. Every
// |y| is first rounded up to a multiple of 2^-25, the finest decision
// resolution (2^-16 of the smallest step 2^-9): that keeps every decision
// (integer u and c: u + c < (|y| - lo) * 2^25 iff u + c < ceil(|y| * 2^25) -
// lo * 2^25) and leaves at most 16 fraction bits below 2^-6; from |y| = 2^-2
// on it changes nothing. |y| above 448 is clamped (both saturate). Only byte 0
// of the builtin's result is defined. Equal to e4m3_sr_mag with the sign of y
// on every finite |y| <= 512 with every draw (the device sweep of
// nvq_convert_probe).
__device__ __forceinline__ float e4m3_sr_input(float y) {
    const float up = __builtin_copysignf(__builtin_ceilf(fabsf(y) * 0x1p25f) * 0x1p-25f, y);
    return __builtin_amdgcn_fmed3f(up, -448.0f, 448.0f);
}
__device__ __forceinline__ uint32_t e4m3_sr_hw(float y, uint32_t u16) {
    return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0, e4m3_sr_input(y), ~(u16 << 16) | 0xFFFFu, 1.0f, 0) &
           0xFFu;
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
// u < (|y| - lo) / step * 2^16; |y| >= 6 saturates without a draw. The
// dropped fraction is read from the fp32 bits, so the decision is an integer
// compare (as e4m3_sr_mag does):
//   [1, 6):   one mantissa bit kept (steps 0.5, 1, 2), frac = low 22 bits / 2^22,
//             up iff 64 u < low 22 bits;
//   [0.5, 1): no mantissa bit kept (step 0.5), up iff 128 u < low 23 bits;
//   [0, 0.5): frac = |y| / 0.5, up iff u < |y| * 2^17 (an exact product).
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u16) {
    const uint32_t b = __float_as_uint(y);
    const uint32_t s = (b >> 28) & 8u;
    const uint32_t m = b & 0x7FFFFFFFu;
    const uint32_t c_hi = (m >> 22) - 252u + ((u16 << 6) < (m & 0x3FFFFFu) ? 1u : 0u);
    const uint32_t c_mid = 1u + ((u16 << 7) < (m & 0x7FFFFFu) ? 1u : 0u);
    const uint32_t c_lo = (float)u16 < __uint_as_float(m) * 131072.0f ? 1u : 0u;
    uint32_t c = m >= 0x3F800000u ? c_hi : (m >= 0x3F000000u ? c_mid : c_lo);
    c = m >= 0x40C00000u ? 7u : c;
    return c | s;
}

// The same decisions by the gfx950 stochastic converter
// (v_cvt_scalef32_sr_pk_fp4_f32), eight values with the draws of draws8 (value
// j takes draw_of(dr, j)). One value per converter call, so that each value
// gets its own draw (the second value of a call sees the random operand
// shifted left by one). With the operand ~(u << 16) the converter rounds up
// exactly when u < frac * 2^16 provided the value's fraction of its grid step
// has at most 22 bits, which holds for every |y| >= 1 (steps 0.5, 1, 2) but
// not below. Every |y| is therefore first rounded up to a multiple of 2^-17:
// the decision compares u with frac * 2^16 = (|y| - lo) * 2^16 / step, whose
// resolution 2^-16 * step is 2^-17 or coarser for every step, so for integers
// u and c, u + c < (|y| - lo) * 2^17 iff u + c < ceil(|y| * 2^17) - lo * 2^17
// and no decision changes; the fraction is left with at most 17 bits. (From
// |y| = 64 on the fp32 spacing is already 2^-17 or coarser and the rounding
// is exact.) |y| > 6 saturates to 6 in the converter as in the rule. Equal to
// e2m1_sr on every finite |y| <= 8 with every draw (the exhaustive device
// sweep of nvq_convert_probe).
__device__ __forceinline__ float e2m1_sr_input(float y) {
    return __builtin_copysignf(__builtin_ceilf(fabsf(y) * 131072.0f) * 0x1p-17f, y);
}

typedef float nvq_sr_f32x2 __attribute__((ext_vector_type(2)));
// values 2Q (draw in the low half of nw = ~draw word Q) and 2Q + 1 (high
// half) into byte Q of word. The stochastic converter builtin does not carry
// its `old` operand into the destination (unlike the nearest-even one): only
// the selected byte 0 of its result is defined, whose high nibble encodes the
// second source 0.0 as code 0.
template <int Q>
__device__ __forceinline__ uint32_t e2m1_sr_pair_hw(uint32_t word, float y0, float y1, uint32_t nw) {
    const nvq_sr_f32x2 a = {e2m1_sr_input(y0), 0.0f};
    const nvq_sr_f32x2 b = {e2m1_sr_input(y1), 0.0f};
    const uint32_t c0 = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, a, (nw << 16) | 0xFFFFu, 1.0f, 0) & 0xFu;
    const uint32_t c1 = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, b, nw | 0xFFFFu, 1.0f, 0) & 0xFu;
    return word | (c0 << (8 * Q)) | (c1 << (8 * Q + 4));
}

__device__ __forceinline__ uint32_t e2m1_sr8_hw(const float (&y)[8], const uint4& dr) {
    uint32_t word = 0;
    word = e2m1_sr_pair_hw<0>(word, y[0], y[1], ~dr.x);
    word = e2m1_sr_pair_hw<1>(word, y[2], y[3], ~dr.y);
    word = e2m1_sr_pair_hw<2>(word, y[4], y[5], ~dr.z);
    word = e2m1_sr_pair_hw<3>(word, y[6], y[7], ~dr.w);
    return word;
}

// ---------------------------------------------------------------- gfx950 converters
// The conversion instructions the kernels rely on, in the exact form they use
// them (the converter-sweep entry point runs these same helpers).
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Eight codes (element 0 in the low nibble) times an fp16 scale -> 8 exact fp16.
__device__ __forceinline__ half8 dq8(uint32_t w, _Float16 sc) {
    const half2v s2 = {sc, sc};
    const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    return half8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// MXFP8 exact dequantization to bf16: an E8M0 byte e as the fp32 scale
// 2^(e - 127) of the gfx950 scaled converters (they read only its exponent
// field, so e = 0 gives 2^-127 although the float itself is zero), and four
// E4M3 bytes of w times that scale as two bf16 pairs (low pair first). The
// products are exact while they lie in bf16's range.
__device__ __forceinline__ float mx_scale_f32(uint32_t e8m0) { return __uint_as_float((e8m0 & 0xFFu) << 23); }
__device__ __forceinline__ uint2 dq4_mx(uint32_t w, float s) {
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, true)));
}

// fp16 scale pairs of a fragment: blocks (0,1) and (2,3). smask is all ones,
// or 0 for a lane outside the operand: its values all become exact zeros.
// (Masking here rather than at the load keeps the load's latency hidden.)
struct Scales {
    half2v lo, hi;
};
__device__ __forceinline__ Scales word_scales(uint32_t word, uint32_t smask) {
    Scales s;
    s.lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word & smask, 1.0f, false);
    s.hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word & smask, 1.0f, true);
    return s;
}

typedef short mx_short2 __attribute__((ext_vector_type(2)));

// Nearest-even E4M3 bytes of x0 * p2 and x1 * p2 (low byte first): the
// gfx950 fp32 -> fp8 converter at scale 1.0 rounds to nearest even but turns
// magnitudes above 464 into NaN, so the product is first clamped to +-448
// (the saturation of the format here). Checked equal to the software encoder
// on every finite fp32 input.
__device__ __forceinline__ uint32_t mx_rne_pair(float x0, float x1, float p2) {
    const float y0 = __builtin_amdgcn_fmed3f(x0 * p2, -448.0f, 448.0f);
    const float y1 = __builtin_amdgcn_fmed3f(x1 * p2, -448.0f, 448.0f);
    const mx_short2 z = {0, 0};
    const mx_short2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, y0, y1, 1.0f, false);
    return (uint32_t)(uint16_t)w[0];
}

// ---------------------------------------------------------------- Philox4x32-10
// Counter-based generator of Salmon et al. (SC'11): ten rounds, each two
// 32x32->64 multiplies, key bumped by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        // one 32x32->64 product each (a single v_mad_u64_u32 rather than
        // separate low and high multiplies); each three-way XOR is one
        // v_bitop3_b32 (truth table 0x96), which the compiler does not form
        // from two XORs by itself
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
        c = make_uint4(__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96), (uint32_t)p1,
                       __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96), (uint32_t)p0);
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

// ---------------------------------------------------------------- 32-point RHT
// z = (1/sqrt 32) H32 (s .* x) per 32-value chunk: one sign vector (bit j of
// the first Philox4x32-10 word at counter (0,0,4,0) under the sign seed; a set
// bit negates), Sylvester H32, fp32 butterfly with strides 1, 2, 4, 8, 16.
constexpr float kInvSqrt32 = 0x1.6a09e6p-3f;  // fp32 nearest to 1/sqrt(32)

__device__ __forceinline__ uint32_t rht_sign_word(uint64_t sign_seed) {
    return philox10(make_uint4(0u, 0u, 4u, 0u), (uint32_t)sign_seed, (uint32_t)(sign_seed >> 32)).x;
}

// Butterfly with strides 1, 2, 4, 8, 16 on one lane's 32 values (stages
// with stride below HEND only).
template <int HEND = 32>
__device__ __forceinline__ void butterfly32(float (&v)[32]) {
#pragma unroll
    for (int h = 1; h < HEND; h <<= 1) {
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

// ---------------------------------------------------------------- wave64 helpers
// Swap with the neighbouring lane (lane ^ 1) through a DPP quad permutation.
__device__ __forceinline__ float dpp_swap1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
// Swap with lane ^ 2 (quad_perm 2,3,0,1).
__device__ __forceinline__ float dpp_swap2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}

// Value of lane + N within the lane's row of 16 (DPP row_shl:N; lanes whose
// source falls outside the row read 0).
template <int N>
__device__ __forceinline__ uint32_t dpp_row_shl(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x100 + N, 0xF, 0xF, true);
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

// amb / 6 as one multiply and one FMA correction (Markstein's scheme with
// the fp32 nearest to 1/6): the IEEE quotient for every finite amb >= 2^-125
// (checked on every such input). Below 2^-125 its last bit may differ, which
// cannot change a block's scale byte while the tensor's encode scale S is at
// most 2^100: (amb / 6) * S < 2^-27 then, far below half the smallest E4M3
// step (2^-10), so both quotients give byte 0.
constexpr float kFastDiv6MaxS = 0x1p100f;
__device__ __forceinline__ float div6_fma(float a) {
    const float y = 0x1.555556p-3f;
    const float q0 = a * y;
    const float r = __builtin_fmaf(-q0, 6.0f, a);
    return __builtin_fmaf(r, y, q0);
}

// Scale byte of a block (as nvfp4_scale_byte) by the MXFP8 elements'
// converter path: clamp to 448, gfx950 fp32 -> fp8 at scale 1.0, which equals
// e4m3_rne_mag on every finite input >= 0 (the converter sweep runs
// mx_rne_pair itself). FAST: the quotient by div6_fma (S <= kFastDiv6MaxS).
template <bool FAST>
__device__ __forceinline__ uint32_t nvfp4_scale_byte_hw(float amb, float S) {
    const float q = FAST ? div6_fma(amb) : amb / 6.0f;
    return mx_rne_pair(q * S, 0.0f, 1.0f) & 0xFFu;
}

// ---------------------------------------------------------------- NVFP4 encode of one lane
// One lane holds 8 consecutive values of a 16-value block whose other half
// sits in lane ^ 1. Given the tensor's encode scale S: block byte = nearest-
// even E4M3 of (amax_block / 6) * S (saturating), r = S / e4m3(byte) (0 for
// byte 0, clamped to FLT_MAX) read from rtab[byte] (a per-workgroup table of
// nvfp4_scale_mult, one division per byte value instead of one per block),
// codes = E2M1 of x * r, nearest-even or stochastic with the eight Philox
// draws of unit `unit` (elements 8*unit..). Returns the packed code word
// (element 0 in the low nibble); *sc gets the byte.
template <int MODE, bool FAST>
__device__ __forceinline__ uint32_t nvfp4_encode8(const float (&f)[8], float S, const float* rtab, uint32_t* sc,
                                                  uint64_t unit, uint32_t stream_id, uint64_t seed) {
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(f[j]));
    const float amb = fmaxf(am, dpp_swap1(am));
    const uint32_t b = nvfp4_scale_byte_hw<FAST>(amb, S);
    const float r = rtab[b & 0x7Fu];  // b <= 0x7E for finite inputs
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
        const float y[8] = {f[0] * r, f[1] * r, f[2] * r, f[3] * r, f[4] * r, f[5] * r, f[6] * r, f[7] * r};
        word = e2m1_sr8_hw(y, draws8(unit, stream_id, seed));
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

// A 16-byte load with the non-temporal hint, for data a pass reads once and
// does not return to. On gfx950 a read-only pass over 1-6 GB runs at
// 6.8-7.0 TB/s with the hint against 6.0-6.2 TB/s without it (measured).
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Tensors at least this large are read with the non-temporal hint by a
// first pass. Smaller ones are left to the 256 MB Infinity Cache, from which
// the second pass then reads part of them.
constexpr int64_t kStreamHintBytes = 192ll << 20;

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
