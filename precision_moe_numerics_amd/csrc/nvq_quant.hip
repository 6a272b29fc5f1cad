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
__device__ __forceinline__ uint32_t max_abs_bf16x8(uint32_t m, const uint4& v) {
    const uint32_t a = max_abs_bf16x2(max_abs_bf16x2(m, v.x), v.y);
    const uint32_t b = max_abs_bf16x2(max_abs_bf16x2(0u, v.z), v.w);
    return max(a, b);
}

// x: B tensors of n8 uint4 (8 bf16 each). Workgroup g of tensor b reads its
// contiguous chunk with kStreamP 4 KiB strips in flight and stores the
// chunk's max|x| (fp32 bits) into part[b * gridDim.x + g]. Load indices are
// clamped to the chunk's last unit (re-reading a unit leaves the max
// unchanged), so every load is an unconditional global load.
__global__ __launch_bounds__(256) void k_amax_bf16(const uint4* __restrict__ x, int64_t n8,
                                                   uint32_t* __restrict__ part) {
    const uint4* xb = x + (int64_t)blockIdx.y * n8;
    int64_t beg, end;
    block_chunk(n8, blockIdx.x, gridDim.x, &beg, &end);
    uint32_t m = 0;
    for (int64_t i = beg + threadIdx.x; i < end; i += 256 * kStreamP) {
        uint4 v[kStreamP];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) v[p] = xb[min(i + 256 * p, end - 1)];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) m = max_abs_bf16x8(m, v[p]);
    }
    m = block_max_u32(m);
    if (threadIdx.x == 0) part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m << 16;
}

// Workgroups per tensor for the streaming kernels: about 2048 in flight over
// all B tensors (eight 4-wave workgroups per CU), each at least 2048 units.
int stream_blocks(int64_t n8, int64_t B) {
    int64_t cap = 2048 / (B > 0 ? B : 1);
    int64_t want = (n8 + 2047) / 2048;
    if (want > cap) want = cap;
    return (int)(want < 1 ? 1 : want);
}

void launch_amax_bf16(const uint16_t* x, int64_t B, int64_t n, uint32_t* part, int G, hipStream_t s) {
    if (B <= 0) return;
    hipLaunchKernelGGL(k_amax_bf16, dim3((unsigned)G, (unsigned)B), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(x), n / 8, part);
}

__global__ void k_fold_partials(const uint32_t* __restrict__ part, int n_part, uint32_t* __restrict__ out) {
    const uint32_t m = __float_as_uint(block_max_partials(part, n_part));
    if (threadIdx.x == 0) out[0] = m;
}

void launch_fold_partials(const uint32_t* part, int n_part, uint32_t* out, hipStream_t s) {
    hipLaunchKernelGGL(k_fold_partials, dim3(1), dim3(256), 0, s, part, n_part, out);
}

// ------------------------------------------------------------------ encode
// One lane encodes 8 consecutive values (a unit); units 2j and 2j+1 form
// block j and sit in neighbouring lanes. Each workgroup walks its contiguous
// chunk 256 * kStreamP units at a time: a lane first issues its kStreamP
// loads (units 256 apart, indices clamped into the chunk), then encodes
// them. Trip counts are uniform per wave so the cross-lane exchanges always
// see all 64 lanes. The tensor maximum is folded from n_part partial maxima
// at part + b * part_stride.
template <int MODE>
__global__ __launch_bounds__(256) void k_nvfp4_encode_bf16(
    const uint4* __restrict__ x, int64_t n8, const uint32_t* __restrict__ part, int n_part,
    int64_t part_stride, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tscale, uint64_t seed, uint32_t stream_id) {
    const int64_t b = blockIdx.y;
    const float amax = block_max_partials(part + b * part_stride, n_part);
    const bool zero = !(amax > 0.0f);
    const float S = nvfp4_encode_scale(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) tscale[b] = nvfp4_decode_scale(amax);

    const uint4* xb = x + b * n8;
    uint32_t* cb = codes + b * n8;
    uint8_t* sb = scales + b * (n8 / 2);
    const int lane = threadIdx.x & 63;
    int64_t beg, end;
    block_chunk(n8, blockIdx.x, gridDim.x, &beg, &end);
    for (int64_t wb = beg + (threadIdx.x & ~63); wb < end; wb += 256 * kStreamP) {
        uint4 v[kStreamP];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) v[p] = xb[min(wb + lane + 256 * p, end - 1)];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) {
            const int64_t u = wb + lane + 256 * p;
            float f[8];
            f[0] = bf16_to_f32(v[p].x & 0xFFFFu); f[1] = bf16_to_f32(v[p].x >> 16);
            f[2] = bf16_to_f32(v[p].y & 0xFFFFu); f[3] = bf16_to_f32(v[p].y >> 16);
            f[4] = bf16_to_f32(v[p].z & 0xFFFFu); f[5] = bf16_to_f32(v[p].z >> 16);
            f[6] = bf16_to_f32(v[p].w & 0xFFFFu); f[7] = bf16_to_f32(v[p].w >> 16);
            uint32_t sc;
            uint32_t word = nvfp4_encode8<MODE>(f, S, &sc, (uint64_t)u, stream_id, seed);
            if (zero) { word = 0; sc = 0; }
            if (u < end) cb[u] = word;
            store_block_scales(sb, u, end, sc);
        }
    }
}

void launch_nvfp4_encode_bf16(const uint16_t* x, int64_t B, int64_t n, const uint32_t* part, int n_part,
                              int64_t part_stride, uint8_t* codes, uint8_t* scales, float* tscale, int mode,
                              uint64_t seed, uint32_t stream_id, hipStream_t s) {
    if (B <= 0) return;
    int64_t n8 = n / 8;
    dim3 grid((unsigned)stream_blocks(n8, B), (unsigned)B);
    auto xk = reinterpret_cast<const uint4*>(x);
    auto ck = reinterpret_cast<uint32_t*>(codes);
    if (mode == NVQ_SR)
        hipLaunchKernelGGL(k_nvfp4_encode_bf16<NVQ_SR>, grid, dim3(256), 0, s, xk, n8, part, n_part, part_stride,
                           ck, scales, tscale, seed, stream_id);
    else
        hipLaunchKernelGGL(k_nvfp4_encode_bf16<NVQ_RTN>, grid, dim3(256), 0, s, xk, n8, part, n_part, part_stride,
                           ck, scales, tscale, seed, stream_id);
}

// ------------------------------------------------------------------ decode
// value = (e2m1 * e4m3) * D in fp32: the first product is exact, so one
// rounding. The E2M1 -> fp32 step is the gfx950 converter at scale 1.0
// (exact: every E2M1 value is an fp32).
template <int OUT>
__global__ __launch_bounds__(256) void k_nvfp4_decode(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ tscale, int64_t n8,
                                                      void* __restrict__ out) {
    const int64_t b = blockIdx.y;
    const float D = tscale[b];
    const uint32_t* cb = codes + b * n8;
    const uint8_t* sb = scales + b * (n8 / 2);
    int64_t beg, end;
    block_chunk(n8, blockIdx.x, gridDim.x, &beg, &end);
    for (int64_t i = beg + threadIdx.x; i < end; i += 256 * kStreamP) {
        uint32_t w[kStreamP], sc[kStreamP];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) {
            const int64_t u = min(i + 256 * p, end - 1);
            w[p] = cb[u];
            sc[p] = sb[u / 2];
        }
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) {
            const int64_t u = i + 256 * p;
            if (u >= end) continue;
            const float s = e4m3_mag_to_f32(sc[p] & 0x7Fu);
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            f32x2 q[4];
            q[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], 1.0f, 0);
            q[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], 1.0f, 1);
            q[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], 1.0f, 2);
            q[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[p], 1.0f, 3);
            float o[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                o[2 * j] = (q[j].x * s) * D;
                o[2 * j + 1] = (q[j].y * s) * D;
            }
            if (OUT == NVQ_OUT_BF16) {
                uint4 r;
                // software rounding: measured faster here than the pair converter
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
    const int64_t b = B > 0 ? B : 1;
    Carver c(nullptr);
    c.take<uint32_t>((size_t)(b * stream_blocks(R * C / 8, b)));
    return c.need;
}

int nvfp4_quantize(const uint16_t* x, int64_t B, int64_t R, int64_t C, uint8_t* codes, uint8_t* scales,
                   float* tscale, int round_mode, uint64_t seed, uint32_t stream_id, void* ws,
                   size_t ws_bytes, nvq_stream_t stream) {
    if (!x || !codes || !scales || !tscale || !ws) return NVQ_ERR_NULL;
    if (B <= 0 || B > 65535 || R < 0 || C <= 0 || (C % 16) != 0) return NVQ_ERR_DIM;
    if (round_mode != NVQ_RTN && round_mode != NVQ_SR) return NVQ_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < nvfp4_quantize_workspace_size(B, R, C)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    const int64_t n = R * C;
    const int G = stream_blocks(n / 8, B);
    Carver cv(ws);
    uint32_t* part = cv.take<uint32_t>((size_t)(B * G));
    launch_amax_bf16(x, B, n, part, G, s);
    launch_nvfp4_encode_bf16(x, B, n, part, G, G, codes, scales, tscale, round_mode, seed, stream_id, s);
    return launch_status();
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tscale, int64_t B, int64_t R,
                     int64_t C, void* out, int out_dtype, nvq_stream_t stream) {
    if (!codes || !scales || !tscale || !out) return NVQ_ERR_NULL;
    if (B <= 0 || B > 65535 || R < 0 || C <= 0 || (C % 16) != 0) return NVQ_ERR_DIM;
    if (out_dtype != NVQ_OUT_BF16 && out_dtype != NVQ_OUT_F32) return NVQ_ERR_UNSUPPORTED;
    if (!aligned16(codes) || !aligned16(out)) return NVQ_ERR_ALIGN;
    const int64_t n8 = R * C / 8;
    if (n8 == 0) return NVQ_OK;
    dim3 grid((unsigned)stream_blocks(n8, B), (unsigned)B);
    hipStream_t s = as_stream(stream);
    auto ck = reinterpret_cast<const uint32_t*>(codes);
    if (out_dtype == NVQ_OUT_BF16)
        hipLaunchKernelGGL(k_nvfp4_decode<NVQ_OUT_BF16>, grid, dim3(256), 0, s, ck, scales, tscale, n8, out);
    else
        hipLaunchKernelGGL(k_nvfp4_decode<NVQ_OUT_F32>, grid, dim3(256), 0, s, ck, scales, tscale, n8, out);
    return launch_status();
}

}  // extern "C"
