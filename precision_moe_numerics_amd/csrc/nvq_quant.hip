// nvq_quant.hip -- NVFP4 block quantization on gfx950: tensor amax, encode
// (nearest-even or Philox stochastic rounding) and decode.
//
// NVFP4 carries about 4.5 bits per value (page "Thinking Machines Details
// End-to-End 4-Bit Training for Inkling 2 Small", section "Background"): a
// 4-bit E2M1 code per value, one E4M3 byte per 16 values and one fp32 scale
// per tensor. Encoding is two passes by construction (the tensor scale
// depends on the whole tensor): an amax pass, then an encode pass.
//
// Memory plan (HBM-bound): each lane moves 16 bytes (8 bf16) per load; a
// 16-value block spans a lane pair whose block maximum is one DPP swap; a
// lane writes its 8 codes as one 32-bit word, and lanes 0,8,16,.. of a wave
// pack four block scales into one 32-bit store.
#include "nvq_device.hpp"
#include "nvq_host.hpp"

namespace nvq {

__global__ void k_zero_u32(uint32_t* __restrict__ p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

void launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s) {
    if (n <= 0) return;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
}

// ------------------------------------------------------------------ amax
__device__ __forceinline__ uint32_t max_abs_bf16x2(uint32_t m, uint32_t w) {
    return max(m, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
}

// Block-wide max of a per-thread value (blockDim.x == 256), then one atomic.
__device__ __forceinline__ void block_max_atomic(uint32_t m, uint32_t* dst) {
    __shared__ uint32_t part[4];
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = max(max(part[0], part[1]), max(part[2], part[3]));
        if (r) atomicMax(dst, r);
    }
}

// x: B tensors of n16 uint4 (8 bf16 each). amax_bits[b] gets max|x| as fp32 bits.
__global__ __launch_bounds__(256) void k_amax_bf16(const uint4* __restrict__ x, int64_t n16,
                                                   uint32_t* __restrict__ amax_bits) {
    const uint4* xb = x + (int64_t)blockIdx.y * n16;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t m = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        uint4 v0 = xb[i];
        uint4 v1 = xb[i + stride];
        uint4 v2 = xb[i + 2 * stride];
        uint4 v3 = xb[i + 3 * stride];
        m = max_abs_bf16x2(m, v0.x); m = max_abs_bf16x2(m, v0.y);
        m = max_abs_bf16x2(m, v0.z); m = max_abs_bf16x2(m, v0.w);
        m = max_abs_bf16x2(m, v1.x); m = max_abs_bf16x2(m, v1.y);
        m = max_abs_bf16x2(m, v1.z); m = max_abs_bf16x2(m, v1.w);
        m = max_abs_bf16x2(m, v2.x); m = max_abs_bf16x2(m, v2.y);
        m = max_abs_bf16x2(m, v2.z); m = max_abs_bf16x2(m, v2.w);
        m = max_abs_bf16x2(m, v3.x); m = max_abs_bf16x2(m, v3.y);
        m = max_abs_bf16x2(m, v3.z); m = max_abs_bf16x2(m, v3.w);
    }
    for (; i < n16; i += stride) {
        uint4 v = xb[i];
        m = max_abs_bf16x2(m, v.x); m = max_abs_bf16x2(m, v.y);
        m = max_abs_bf16x2(m, v.z); m = max_abs_bf16x2(m, v.w);
    }
    block_max_atomic(m << 16, amax_bits + blockIdx.y);
}

static unsigned grid_x_for(int64_t work_per_batch, int64_t per_block, int64_t B, int64_t target) {
    int64_t want = (work_per_batch + per_block - 1) / per_block;
    int64_t cap = target / (B > 0 ? B : 1);
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    return (unsigned)want;
}

void launch_amax_bf16(const uint16_t* x, int64_t B, int64_t n, uint32_t* amax_bits, hipStream_t s) {
    int64_t n16 = n / 8;
    if (B <= 0) return;
    dim3 grid(grid_x_for(n16, 256 * 4, B, 4096), (unsigned)B);
    hipLaunchKernelGGL(k_amax_bf16, grid, dim3(256), 0, s, reinterpret_cast<const uint4*>(x), n16,
                       amax_bits);
}

// ------------------------------------------------------------------ encode
// One lane encodes 8 consecutive values (a unit); units 2j and 2j+1 form
// block j and sit in neighbouring lanes. Trip counts are uniform per wave so
// the cross-lane exchanges always see all 64 lanes.
template <int MODE>
__global__ __launch_bounds__(256) void k_nvfp4_encode_bf16(
    const uint4* __restrict__ x, int64_t n8, const uint32_t* __restrict__ amax_bits,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ tscale,
    uint64_t seed, uint32_t stream_id) {
    const int64_t b = blockIdx.y;
    const float amax = __uint_as_float(amax_bits[b]);
    const bool zero = !(amax > 0.0f);
    const float S = nvfp4_encode_scale(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) tscale[b] = nvfp4_decode_scale(amax);

    const uint4* xb = x + b * n8;
    uint32_t* cb = codes + b * n8;
    uint8_t* sb = scales + b * (n8 / 2);
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t wbase = (int64_t)blockIdx.x * 256 + (threadIdx.x & ~63); wbase < n8; wbase += stride) {
        const int64_t u = wbase + lane;
        const bool valid = u < n8;
        const uint4 v = valid ? xb[u] : make_uint4(0, 0, 0, 0);
        float f[8];
        f[0] = bf16_to_f32(v.x & 0xFFFFu); f[1] = bf16_to_f32(v.x >> 16);
        f[2] = bf16_to_f32(v.y & 0xFFFFu); f[3] = bf16_to_f32(v.y >> 16);
        f[4] = bf16_to_f32(v.z & 0xFFFFu); f[5] = bf16_to_f32(v.z >> 16);
        f[6] = bf16_to_f32(v.w & 0xFFFFu); f[7] = bf16_to_f32(v.w >> 16);
        uint32_t sc;
        uint32_t word = nvfp4_encode8<MODE>(f, S, &sc, (uint64_t)u, stream_id, seed);
        if (zero) { word = 0; sc = 0; }
        if (valid) cb[u] = word;
        store_block_scales(sb, u, n8, sc);
    }
}

void launch_nvfp4_encode_bf16(const uint16_t* x, int64_t B, int64_t n, const uint32_t* amax_bits,
                              uint8_t* codes, uint8_t* scales, float* tscale, int mode,
                              uint64_t seed, uint32_t stream_id, hipStream_t s) {
    if (B <= 0) return;
    int64_t n8 = n / 8;
    dim3 grid(grid_x_for(n8, 256, B, 8192), (unsigned)B);
    auto xk = reinterpret_cast<const uint4*>(x);
    auto ck = reinterpret_cast<uint32_t*>(codes);
    if (mode == NVQ_SR)
        hipLaunchKernelGGL(k_nvfp4_encode_bf16<NVQ_SR>, grid, dim3(256), 0, s, xk, n8, amax_bits, ck,
                           scales, tscale, seed, stream_id);
    else
        hipLaunchKernelGGL(k_nvfp4_encode_bf16<NVQ_RTN>, grid, dim3(256), 0, s, xk, n8, amax_bits, ck,
                           scales, tscale, seed, stream_id);
}

// ------------------------------------------------------------------ decode
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    uint32_t m = c & 7u;
    float mag = m < 2u ? (float)m * 0.5f : __uint_as_float((((m >> 1) + 126u) << 23) | ((m & 1u) << 22));
    return __uint_as_float(__float_as_uint(mag) | ((c & 8u) << 28));
}

template <int OUT>
__global__ __launch_bounds__(256) void k_nvfp4_decode(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ tscale, int64_t n8,
                                                      void* __restrict__ out) {
    const int64_t b = blockIdx.y;
    const float D = tscale[b];
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < n8; u += stride) {
        const uint32_t w = codes[b * n8 + u];
        const float sc = e4m3_mag_to_f32(scales[b * (n8 / 2) + u / 2] & 0x7Fu);
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (e2m1_to_f32((w >> (4 * j)) & 0xFu) * sc) * D;
        if (OUT == NVQ_OUT_BF16) {
            uint4 r;
            r.x = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
            r.y = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
            r.z = f32_to_bf16(o[4]) | (f32_to_bf16(o[5]) << 16);
            r.w = f32_to_bf16(o[6]) | (f32_to_bf16(o[7]) << 16);
            reinterpret_cast<uint4*>(out)[b * n8 + u] = r;
        } else {
            float4* op = reinterpret_cast<float4*>(out) + 2 * (b * n8 + u);
            op[0] = make_float4(o[0], o[1], o[2], o[3]);
            op[1] = make_float4(o[4], o[5], o[6], o[7]);
        }
    }
}

}  // namespace nvq

using namespace nvq;

extern "C" {

const char* nvq_status_string(int status) {
    switch (status) {
        case NVQ_OK: return "ok";
        case NVQ_ERR_NULL: return "a required pointer is NULL";
        case NVQ_ERR_DIM: return "a size is out of range or not a required multiple";
        case NVQ_ERR_WORKSPACE: return "workspace smaller than the size query";
        case NVQ_ERR_LAUNCH: return "HIP kernel launch failed";
        case NVQ_ERR_UNSUPPORTED: return "unsupported option value";
        case NVQ_ERR_ALIGN: return "pointer not 16-byte aligned (workspace: 256-byte)";
        default: return "unknown status";
    }
}

int nvq_abi_version(void) { return 1; }

size_t nvfp4_quantize_workspace_size(int64_t B, int64_t R, int64_t C) {
    (void)R; (void)C;
    Carver c(nullptr);
    c.take<uint32_t>((size_t)(B > 0 ? B : 1));
    return c.need;
}

int nvfp4_quantize(const uint16_t* x, int64_t B, int64_t R, int64_t C, uint8_t* codes, uint8_t* scales,
                   float* tscale, int round_mode, uint64_t seed, uint32_t stream_id, void* ws,
                   size_t ws_bytes, nvq_stream_t stream) {
    if (!x || !codes || !scales || !tscale || !ws) return NVQ_ERR_NULL;
    if (B <= 0 || R < 0 || C <= 0 || (C % 16) != 0) return NVQ_ERR_DIM;
    if (round_mode != NVQ_RTN && round_mode != NVQ_SR) return NVQ_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < nvfp4_quantize_workspace_size(B, R, C)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    uint32_t* amax = cv.take<uint32_t>((size_t)B);
    const int64_t n = R * C;
    launch_zero_u32(amax, B, s);
    launch_amax_bf16(x, B, n, amax, s);
    launch_nvfp4_encode_bf16(x, B, n, amax, codes, scales, tscale, round_mode, seed, stream_id, s);
    return launch_status();
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tscale, int64_t B, int64_t R,
                     int64_t C, void* out, int out_dtype, nvq_stream_t stream) {
    if (!codes || !scales || !tscale || !out) return NVQ_ERR_NULL;
    if (B <= 0 || R < 0 || C <= 0 || (C % 16) != 0) return NVQ_ERR_DIM;
    if (out_dtype != NVQ_OUT_BF16 && out_dtype != NVQ_OUT_F32) return NVQ_ERR_UNSUPPORTED;
    if (!aligned16(codes) || !aligned16(out)) return NVQ_ERR_ALIGN;
    const int64_t n8 = R * C / 8;
    if (n8 == 0) return NVQ_OK;
    dim3 grid(grid_x_for(n8, 256, B, 8192), (unsigned)B);
    hipStream_t s = as_stream(stream);
    auto ck = reinterpret_cast<const uint32_t*>(codes);
    if (out_dtype == NVQ_OUT_BF16)
        hipLaunchKernelGGL(k_nvfp4_decode<NVQ_OUT_BF16>, grid, dim3(256), 0, s, ck, scales, tscale, n8, out);
    else
        hipLaunchKernelGGL(k_nvfp4_decode<NVQ_OUT_F32>, grid, dim3(256), 0, s, ck, scales, tscale, n8, out);
    return launch_status();
}

}  // extern "C"
