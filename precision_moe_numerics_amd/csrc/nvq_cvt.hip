// nvq_cvt.hip -- runs the gfx950 conversion steps the kernels rely on, in the
// form the kernels use them, so their exactness can be checked against the
// format rules: NVFP4's E2M1 codes with E4M3 block scales (about 4.5 bits per
// value, page "Thinking Machines Details End-to-End 4-Bit Training for Inkling
// 2 Small", section "Background") and MXFP8's E4M3 elements (section "Key
// Takeaways" of the same page), and the bf16 rounding of every bf16 output.
//
// Two kinds of calls:
//  - decode tables: the exact-dequantization chain of the NVFP4 GEMMs (E4M3
//    scale byte -> fp16, 8 E2M1 codes -> fp16, packed fp16 multiply), the
//    E2M1 -> fp32 decode of the dequantizer and the combine, on given words,
//    and the MXFP8 GEMMs' E4M3 x 2^(E8M0 - 127) -> bf16 for every byte pair;
//  - sweeps over all 2^32 fp32 bit patterns of an encoder: every output is a
//    monotone step function of the input within one sign, so a sweep reports,
//    per range of 2^16 consecutive patterns, the first output and the
//    patterns where the output changes. A checker that evaluates the rule at
//    both ends of every run of equal outputs has then covered every input.
#include "nvq_device.hpp"
#include "nvq_host.hpp"

namespace nvq {

constexpr int kScanCap = 8;                 // changes recorded per range
constexpr int kScanWords = 2 + 2 * kScanCap;  // first, count, positions, values

template <int WHICH>
__device__ __forceinline__ uint32_t scan_out(float x, bool* pair_ok) {
    if (WHICH == NVQ_CVT_SCAN_E2M1) {
        // nvfp4_encode8 / the RHT encoder: two values per converter call
        const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x, x, 1.0f, 0);
        *pair_ok = (w & 0xFu) == ((w >> 4) & 0xFu) && (w >> 8) == 0u;
        return w & 0xFu;
    } else if (WHICH == NVQ_CVT_SCAN_E4M3_HW) {
        // the MXFP8 nearest-even elements: clamp to +-448, then the converter
        const uint32_t w = mx_rne_pair(x, x, 1.0f);
        *pair_ok = (w & 0xFFu) == (w >> 8);
        return w & 0xFFu;
    } else if (WHICH == NVQ_CVT_SCAN_E4M3_SW) {
        // the software encoder of block scales and SR neighbours, sign attached
        *pair_ok = true;
        return e4m3_rne_mag(fabsf(x)) | ((__float_as_uint(x) >> 24) & 0x80u);
    } else if (WHICH == NVQ_CVT_SCAN_BF16_HW) {
        const uint32_t w = bf16x2_rne(x, x);
        *pair_ok = (w & 0xFFFFu) == (w >> 16);
        return w & 0xFFFFu;
    } else {  // NVQ_CVT_SCAN_BF16_SW
        *pair_ok = true;
        return f32_to_bf16(x);
    }
}

// Thread t sweeps patterns [t * 2^16, (t + 1) * 2^16); ranges whose patterns
// are infinities or NaNs (exponent field all ones) are skipped. out[t] holds
// the first output, the number of changes (bit 31: more than kScanCap, or
// the two values of a converter call disagreed), then up to kScanCap
// (pattern, new output) pairs.
template <int WHICH>
__global__ __launch_bounds__(256) void k_cvt_scan(uint32_t* __restrict__ out) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;  // 0 .. 65535
    uint32_t* o = out + (size_t)t * kScanWords;
    if ((t & 0x7FFFu) >= 0x7F80u) {
        o[0] = 0u;
        o[1] = 0u;
        return;
    }
    bool ok = true, pk;
    const uint32_t base = t << 16;
    uint32_t prev = scan_out<WHICH>(__uint_as_float(base), &pk);
    ok &= pk;
    o[0] = prev;
    uint32_t n = 0;
    for (uint32_t i = 1; i < 65536u; ++i) {
        const uint32_t p = base + i;
        const uint32_t v = scan_out<WHICH>(__uint_as_float(p), &pk);
        ok &= pk;
        if (v != prev) {
            if (n < (uint32_t)kScanCap) {
                o[2 + n] = p;
                o[2 + kScanCap + n] = v;
            }
            ++n;
            prev = v;
        }
    }
    o[1] = (n > (uint32_t)kScanCap || !ok) ? (n | 0x80000000u) : n;
}

// Decode tables. in[i] = (code word, scale word) -> out fp16 [i][40]: the
// four scale bytes as fp16 (word_scales) and four zero halves, then dq8 of
// the code word with each of the four scales (the NVFP4 GEMMs' operand
// dequantization). Every result is stored as the whole vector the GEMM
// feeds to its MFMAs (element-wise extraction from these converter results
// is not what the kernels do, and the compiler mishandles it).
__global__ __launch_bounds__(256) void k_cvt_dq_f16(const uint2* __restrict__ in, int64_t n,
                                                     uint4* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const uint2 cw = in[i];
    const Scales s = word_scales(cw.y, 0xFFFFFFFFu);
    uint4* o = out + i * 5;
    o[0] = make_uint4(__builtin_bit_cast(uint32_t, s.lo), __builtin_bit_cast(uint32_t, s.hi), 0u, 0u);
    o[1] = __builtin_bit_cast(uint4, dq8(cw.x, s.lo[0]));
    o[2] = __builtin_bit_cast(uint4, dq8(cw.x, s.lo[1]));
    o[3] = __builtin_bit_cast(uint4, dq8(cw.x, s.hi[0]));
    o[4] = __builtin_bit_cast(uint4, dq8(cw.x, s.hi[1]));
}

// Stochastic-rounding decisions: in[i] = (fp32 bits of y, 16-bit draw u) ->
// out[i] = the E2M1 code (with sign) the SR encoders produce (e2m1_sr8_hw,
// y in all eight positions, every draw u; bit 31 set if the eight disagree),
// the E4M3 byte they produce (e4m3_sr_hw, bits 8-15), the software rules'
// E2M1 code e2m1_sr (bits 16-19) and E4M3 byte e4m3_sr_mag(|y|) with the
// sign of y (bits 20-27).
__device__ __forceinline__ uint32_t e4m3_sr_sw(float y, uint32_t u) {
    return e4m3_sr_mag(fabsf(y), u) | ((__float_as_uint(y) >> 24) & 0x80u);
}

__device__ __forceinline__ uint32_t sr_hw_code(float y, uint32_t u, bool* same) {
    const float y8[8] = {y, y, y, y, y, y, y, y};
    const uint32_t d = u | (u << 16);
    const uint32_t w = e2m1_sr8_hw(y8, make_uint4(d, d, d, d));
    *same = w == (w & 0xFu) * 0x11111111u;
    return w & 0xFu;
}

__global__ __launch_bounds__(256) void k_cvt_sr(const uint2* __restrict__ in, int64_t n, uint32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const uint2 v = in[i];
    const float y = __uint_as_float(v.x);
    const uint32_t u = v.y & 0xFFFFu;
    bool same;
    const uint32_t hw = sr_hw_code(y, u, &same);
    out[i] = hw | (e4m3_sr_hw(y, u) << 8) | (e2m1_sr(y, u) << 16) | (e4m3_sr_sw(y, u) << 20) |
             (same ? 0u : 0x80000000u);
}

// Exhaustive check of the converter paths against the software rules: E2M1
// (e2m1_sr8_hw against e2m1_sr, every fp32 y with |y| <= 8) and E4M3
// (e4m3_sr_hw against e4m3_sr_mag with the sign, |y| <= 512). Both sides
// decide "round up iff u < threshold(y)", a step function of the draw u, so
// per value it suffices to compare the codes at u = 0 and u = 65535 and the
// first draw at which the code changes (a binary search on each side).
// k_cvt_sr_sweep does that for every such y of both signs, and k_cvt_sr_all
// compares every one of the 65536 draws for every 65521st of those values.
// cnt: [0] values whose codes or threshold differ, [1] values with a decision
// (the code depends on the draw), [2] (value, draw) pairs that differ in the
// full comparison, [3] values fully compared.
template <int FMT>
struct SrSweep {
    static constexpr uint64_t half = FMT == 0 ? 0x41000001ull : 0x44000001ull;  // patterns 0 .. bits(8 or 512)
    __device__ static uint32_t pattern(uint64_t i) {
        return i < half ? (uint32_t)i : ((uint32_t)(i - half) | 0x80000000u);
    }
    __device__ static uint32_t sw(float y, uint32_t u) { return FMT == 0 ? e2m1_sr(y, u) : e4m3_sr_sw(y, u); }
    __device__ static uint32_t hw(float y, uint32_t u, bool* same) {
        if (FMT == 0) return sr_hw_code(y, u, same);
        *same = true;
        return e4m3_sr_hw(y, u);
    }
};

template <int FMT>
__global__ __launch_bounds__(256) void k_cvt_sr_sweep(unsigned long long* __restrict__ cnt) {
    using W = SrSweep<FMT>;
    unsigned long long bad = 0, decided = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < 2 * W::half; i += (uint64_t)gridDim.x * 256) {
        const float y = __uint_as_float(W::pattern(i));
        bool s0, s1;
        const uint32_t w0 = W::sw(y, 0u), w1 = W::sw(y, 65535u);
        const uint32_t h0 = W::hw(y, 0u, &s0), h1 = W::hw(y, 65535u, &s1);
        if (w0 != h0 || w1 != h1 || !s0 || !s1) { ++bad; continue; }
        if (w0 == w1) continue;
        ++decided;
        uint32_t lo = 0, hi = 65535, lo2 = 0, hi2 = 65535;
        bool ok = true;
        while (lo < hi) {
            const uint32_t m = (lo + hi) >> 1;
            if (W::sw(y, m) == w1) hi = m; else lo = m + 1;
        }
        while (lo2 < hi2) {
            const uint32_t m = (lo2 + hi2) >> 1;
            bool sm;
            if (W::hw(y, m, &sm) == h1) hi2 = m; else lo2 = m + 1;
            ok &= sm;
        }
        if (lo != lo2 || !ok) ++bad;
    }
    atomicAdd(cnt + 0, bad);
    atomicAdd(cnt + 1, decided);
}

constexpr uint32_t kSrAllStride = 65521u;

template <int FMT>
__global__ __launch_bounds__(256) void k_cvt_sr_all(unsigned long long* __restrict__ cnt) {
    using W = SrSweep<FMT>;
    // thread t: value (t >> 8) * stride, draws (t & 255) * 256 .. + 255
    const uint64_t ny = (2 * W::half + kSrAllStride - 1) / kSrAllStride;
    unsigned long long bad = 0, done = 0;
    for (uint64_t t = (uint64_t)blockIdx.x * 256 + threadIdx.x; t < ny * 256; t += (uint64_t)gridDim.x * 256) {
        const float y = __uint_as_float(W::pattern((t >> 8) * kSrAllStride));
        const uint32_t u0 = (uint32_t)(t & 255) * 256u;
        for (uint32_t u = u0; u < u0 + 256u; ++u) {
            bool sm;
            if (W::hw(y, u, &sm) != W::sw(y, u) || !sm) ++bad;
        }
        if ((t & 255) == 0) ++done;
    }
    atomicAdd(cnt + 2, bad);
    atomicAdd(cnt + 3, done);
}

__global__ void k_cvt_zero_u64(unsigned long long* __restrict__ p, int n) {
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

// in[i] = 8 E2M1 codes -> out fp32 [i][8] by the E2M1 -> fp32 converter.
__global__ __launch_bounds__(256) void k_cvt_fp4_f32(const uint32_t* __restrict__ in, int64_t n,
                                                      float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const uint32_t w = in[i];
    f32x2 q[4];
    q[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    q[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    q[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    q[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out[i * 8 + 2 * j] = q[j].x;
        out[i * 8 + 2 * j + 1] = q[j].y;
    }
}

}  // namespace nvq

using namespace nvq;

extern "C" {

// Row e (the E8M0 scale byte) of the MXFP8 operand table: thread t decodes
// E4M3 bytes 4t .. 4t + 3 as the MXFP8 GEMMs do.
__global__ __launch_bounds__(64) void k_cvt_dq_mx(uint2* __restrict__ out) {
    const uint32_t e = blockIdx.x, t = threadIdx.x, c = 4u * t;
    const uint32_t w = c | ((c + 1u) << 8) | ((c + 2u) << 16) | ((c + 3u) << 24);
    out[e * 64u + t] = dq4_mx(w, mx_scale_f32(e));
}

// Pair i of all 65536 (byte 0 = i & 0xFF, byte 1 = i >> 8) decoded as the
// combine decodes its block scales.
__global__ __launch_bounds__(256) void k_cvt_e4m3_pairs(float2* __restrict__ out) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    const nvq_f32x2 v = e4m3_pair_to_f32(i);
    out[i] = make_float2(v.x, v.y);
}

int nvq_convert_probe(int which, const void* in, int64_t n, void* out, nvq_stream_t stream) {
    if (!out) return NVQ_ERR_NULL;
    if (!aligned16(out)) return NVQ_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    switch (which) {
        case NVQ_CVT_DQ_F16:
        case NVQ_CVT_FP4_F32:
        case NVQ_CVT_SR: {
            if (!in) return NVQ_ERR_NULL;
            if (n < 0 || n > ((int64_t)1 << 24)) return NVQ_ERR_DIM;
            if (n == 0) return NVQ_OK;
            const unsigned g = (unsigned)((n + 255) / 256);
            if (which == NVQ_CVT_DQ_F16)
                hipLaunchKernelGGL(k_cvt_dq_f16, dim3(g), dim3(256), 0, s, static_cast<const uint2*>(in), n,
                                   static_cast<uint4*>(out));
            else if (which == NVQ_CVT_SR)
                hipLaunchKernelGGL(k_cvt_sr, dim3(g), dim3(256), 0, s, static_cast<const uint2*>(in), n,
                                   static_cast<uint32_t*>(out));
            else
                hipLaunchKernelGGL(k_cvt_fp4_f32, dim3(g), dim3(256), 0, s, static_cast<const uint32_t*>(in), n,
                                   static_cast<float*>(out));
            return launch_status();
        }
        case NVQ_CVT_SCAN_E2M1:
        case NVQ_CVT_SCAN_E4M3_HW:
        case NVQ_CVT_SCAN_E4M3_SW:
        case NVQ_CVT_SCAN_BF16_HW:
        case NVQ_CVT_SCAN_BF16_SW: {
            if (n != 65536) return NVQ_ERR_DIM;
            uint32_t* o = static_cast<uint32_t*>(out);
            const dim3 g(256), b(256);
            switch (which) {
                case NVQ_CVT_SCAN_E2M1: hipLaunchKernelGGL(k_cvt_scan<NVQ_CVT_SCAN_E2M1>, g, b, 0, s, o); break;
                case NVQ_CVT_SCAN_E4M3_HW: hipLaunchKernelGGL(k_cvt_scan<NVQ_CVT_SCAN_E4M3_HW>, g, b, 0, s, o); break;
                case NVQ_CVT_SCAN_E4M3_SW: hipLaunchKernelGGL(k_cvt_scan<NVQ_CVT_SCAN_E4M3_SW>, g, b, 0, s, o); break;
                case NVQ_CVT_SCAN_BF16_HW: hipLaunchKernelGGL(k_cvt_scan<NVQ_CVT_SCAN_BF16_HW>, g, b, 0, s, o); break;
                default: hipLaunchKernelGGL(k_cvt_scan<NVQ_CVT_SCAN_BF16_SW>, g, b, 0, s, o); break;
            }
            return launch_status();
        }
        case NVQ_CVT_E4M3_PAIR_F32: {
            if (n != 65536) return NVQ_ERR_DIM;
            hipLaunchKernelGGL(k_cvt_e4m3_pairs, dim3(256), dim3(256), 0, s, static_cast<float2*>(out));
            return launch_status();
        }
        case NVQ_CVT_DQ_MX_BF16: {
            if (n != 256) return NVQ_ERR_DIM;
            hipLaunchKernelGGL(k_cvt_dq_mx, dim3(256), dim3(64), 0, s, static_cast<uint2*>(out));
            return launch_status();
        }
        case NVQ_CVT_SR_E2M1_SWEEP:
        case NVQ_CVT_SR_E4M3_SWEEP: {
            if (n != 4) return NVQ_ERR_DIM;
            auto* c = static_cast<unsigned long long*>(out);
            hipLaunchKernelGGL(k_cvt_zero_u64, dim3(1), dim3(64), 0, s, c, 4);
            if (which == NVQ_CVT_SR_E2M1_SWEEP) {
                hipLaunchKernelGGL(k_cvt_sr_sweep<0>, dim3(8192), dim3(256), 0, s, c);
                hipLaunchKernelGGL(k_cvt_sr_all<0>, dim3(8192), dim3(256), 0, s, c);
            } else {
                hipLaunchKernelGGL(k_cvt_sr_sweep<1>, dim3(8192), dim3(256), 0, s, c);
                hipLaunchKernelGGL(k_cvt_sr_all<1>, dim3(8192), dim3(256), 0, s, c);
            }
            return launch_status();
        }
        default:
            return NVQ_ERR_UNSUPPORTED;
    }
}

}  // extern "C"
