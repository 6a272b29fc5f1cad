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
#include <algorithm>
#include <mutex>

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

// x: B tensors of n8 uint4 (8 bf16 each). The G workgroups of tensor b
// walk it in grid-stride order, kStreamP 4 KiB strips per workgroup and
// step, and workgroup g stores its max|x| (fp32 bits) into
// part[b * G + g]. Load indices are clamped to the last unit (re-reading a
// unit leaves the max unchanged), so every load is an unconditional global
// load. NT: loads with the non-temporal hint (tensors larger than the
// Infinity Cache; a smaller one is left there for the encode pass).
template <bool NT>
__global__ __launch_bounds__(256) void k_amax_bf16(const uint4* __restrict__ x, int64_t n8,
                                                   uint32_t* __restrict__ part) {
    const uint4* xb = x + (int64_t)blockIdx.y * n8;
    const int64_t step = (int64_t)gridDim.x * (256 * kStreamP);
    uint32_t m = 0;
    for (int64_t i = (int64_t)blockIdx.x * (256 * kStreamP) + threadIdx.x; i < n8; i += step) {
        uint4 v[kStreamP];
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) {
            const uint4* q = xb + min(i + 256 * p, n8 - 1);
            v[p] = NT ? load_stream(q) : *q;
        }
#pragma unroll
        for (int p = 0; p < kStreamP; ++p) m = max_abs_bf16x8(m, v[p]);
    }
    m = block_max_u32(m);
    if (threadIdx.x == 0) part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m << 16;
}

// Workgroups per tensor of the maximum pass (and so partial maxima per
// tensor): about 1024 for one tensor (enough to stream it at the copy rate,
// half the partials the encode pass folds of 2048), about 2048 over all B
// tensors of a batch, each at least 2048 units.
int stream_blocks(int64_t n8, int64_t B) {
    int64_t cap = (B > 1 ? 2048 : 1024) / (B > 0 ? B : 1);
    int64_t want = (n8 + 2047) / 2048;
    if (want > cap) want = cap;
    return (int)(want < 1 ? 1 : want);
}

void launch_amax_bf16(const uint16_t* x, int64_t B, int64_t n, uint32_t* part, int G, hipStream_t s) {
    if (B <= 0) return;
    if (B * n * 2 >= kStreamHintBytes)
        hipLaunchKernelGGL(k_amax_bf16<true>, dim3((unsigned)G, (unsigned)B), dim3(256), 0, s,
                           reinterpret_cast<const uint4*>(x), n / 8, part);
    else
        hipLaunchKernelGGL(k_amax_bf16<false>, dim3((unsigned)G, (unsigned)B), dim3(256), 0, s,
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
// block j and sit in neighbouring lanes. The workgroups of tensor b walk it
// in grid-stride order, 256 * kStreamP units per workgroup and step (wave w
// takes the four 64-unit slices at 64 w + 256 p), so at any moment the whole
// grid reads and writes one contiguous window of the tensor. Each step's
// loads (non-temporal: the pass reads every byte once) are issued one step
// ahead into the other of two register buffers, and the first ones before
// the tensor maximum is folded from the n_part partial maxima at
// part + b * part_stride, which hides the fold. Trip counts are uniform per
// wave so the cross-lane exchanges always see all 64 lanes; load indices
// are clamped to the last unit. IDX: uint32_t for tensors under 4 GiB (unit
// byte offsets fit 32 bits, so addresses are a scalar base plus a 32-bit
// lane offset), int64_t otherwise.
template <typename IDX>
__device__ __forceinline__ const uint4* unit_at(const uint4* base, IDX u) {
    if constexpr (sizeof(IDX) == 4)
        return reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + (uint32_t)(u << 4));
    else
        return base + u;
}

template <typename IDX>
__device__ __forceinline__ uint32_t* word_at(uint32_t* base, IDX u) {
    if constexpr (sizeof(IDX) == 4)
        return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(base) + (uint32_t)(u << 2));
    else
        return base + u;
}

template <typename IDX>
__device__ __forceinline__ void load_units(uint4 (&v)[kStreamP], const uint4* xb, IDX first, IDX n8) {
#pragma unroll
    for (int p = 0; p < kStreamP; ++p) v[p] = load_stream(unit_at(xb, min(first + (IDX)(256 * p), n8 - 1)));
}

struct EncodeOut {
    uint32_t* codes;    // the tensor's code words
    uint8_t* scales;    // its scale bytes
    bool scales_al;     // scales 4-byte aligned: whole groups of four bytes are 32-bit stores
};

// Encodes the kStreamP units of one step and stores codes and scale bytes.
// Lanes 8g..8g+7 hold units u..u+7 = blocks u/2..u/2+3; their bytes go out as
// one 32-bit store by lane 8g (bytes of lanes 8g+2, +4, +6 by DPP row
// shifts) where the group is complete and the bytes aligned, else as single
// bytes from the even lanes.
template <int MODE, bool FAST, typename IDX>
__device__ __forceinline__ void encode_step(const uint4 (&v)[kStreamP], IDX wb, IDX n8, int lane, float S,
                                            bool zero, const float* rtab, const EncodeOut& o, uint32_t stream_id,
                                            uint64_t seed) {
#pragma unroll
    for (int p = 0; p < kStreamP; ++p) {
        const IDX u = wb + (IDX)(lane + 256 * p);
        float f[8];
        f[0] = bf16_to_f32(v[p].x & 0xFFFFu); f[1] = bf16_to_f32(v[p].x >> 16);
        f[2] = bf16_to_f32(v[p].y & 0xFFFFu); f[3] = bf16_to_f32(v[p].y >> 16);
        f[4] = bf16_to_f32(v[p].z & 0xFFFFu); f[5] = bf16_to_f32(v[p].z >> 16);
        f[6] = bf16_to_f32(v[p].w & 0xFFFFu); f[7] = bf16_to_f32(v[p].w >> 16);
        uint32_t sc;
        uint32_t word = nvfp4_encode8<MODE, FAST>(f, S, rtab, &sc, (uint64_t)u, stream_id, seed);
        if (zero) { word = 0; sc = 0; }
        const uint32_t s2 = dpp_row_shl<2>(sc), s4 = dpp_row_shl<4>(sc), s6 = dpp_row_shl<6>(sc);
        if (u < n8) *word_at(o.codes, u) = word;
        if (o.scales_al && (u | 7) < n8) {
            if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(o.scales + u / 2) = sc | (s2 << 8) | (s4 << 16) | (s6 << 24);
        } else if (u < n8 && (lane & 1) == 0) {
            o.scales[u / 2] = (uint8_t)sc;
        }
    }
}

template <int MODE, bool FAST, typename IDX>
__device__ __forceinline__ void encode_loop(uint4 (&va)[kStreamP], IDX wb, IDX step, IDX n8, int lane,
                                            const uint4* xb, float S, bool zero, const float* rtab,
                                            const EncodeOut& o, uint32_t stream_id, uint64_t seed) {
    uint4 vb[kStreamP];
    while (wb < n8) {
        if (wb + step < n8) load_units(vb, xb, wb + step + (IDX)lane, n8);
        encode_step<MODE, FAST>(va, wb, n8, lane, S, zero, rtab, o, stream_id, seed);
        wb += step;
        if (wb >= n8) break;
        if (wb + step < n8) load_units(va, xb, wb + step + (IDX)lane, n8);
        encode_step<MODE, FAST>(vb, wb, n8, lane, S, zero, rtab, o, stream_id, seed);
        wb += step;
    }
}

template <int MODE, typename IDX>
__global__ __launch_bounds__(256) void k_nvfp4_encode_bf16(
    const uint4* __restrict__ x, int64_t n8_, const uint32_t* __restrict__ part, int n_part,
    int64_t part_stride, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tscale, uint64_t seed, uint32_t stream_id) {
    __shared__ float rtab[128];
    const int64_t b = blockIdx.y;
    const IDX n8 = (IDX)n8_;
    const uint4* xb = x + b * n8_;
    EncodeOut o{codes + b * n8_, scales + b * (n8_ / 2), false};
    o.scales_al = (reinterpret_cast<uintptr_t>(o.scales) & 3u) == 0;
    const int lane = threadIdx.x & 63;
    const IDX step = (IDX)gridDim.x * (IDX)(256 * kStreamP);
    const IDX wb = (IDX)blockIdx.x * (IDX)(256 * kStreamP) + (IDX)(threadIdx.x & ~63);
    uint4 va[kStreamP];
    if (wb < n8) load_units(va, xb, wb + (IDX)lane, n8);
    const float amax = block_max_partials(part + b * part_stride, n_part);
    const bool zero = !(amax > 0.0f);
    const float S = nvfp4_encode_scale(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) tscale[b] = nvfp4_decode_scale(amax);
    if (threadIdx.x < 128) rtab[threadIdx.x] = nvfp4_scale_mult(threadIdx.x, S);
    __syncthreads();
    // S is uniform over the tensor, so is the choice of quotient
    if (S <= kFastDiv6MaxS)
        encode_loop<MODE, true>(va, wb, step, n8, lane, xb, S, zero, rtab, o, stream_id, seed);
    else
        encode_loop<MODE, false>(va, wb, step, n8, lane, xb, S, zero, rtab, o, stream_id, seed);
}

void launch_nvfp4_encode_bf16(const uint16_t* x, int64_t B, int64_t n, const uint32_t* part, int n_part,
                              int64_t part_stride, uint8_t* codes, uint8_t* scales, float* tscale, int mode,
                              uint64_t seed, uint32_t stream_id, hipStream_t s) {
    if (B <= 0) return;
    int64_t n8 = n / 8;
    auto xk = reinterpret_cast<const uint4*>(x);
    auto ck = reinterpret_cast<uint32_t*>(codes);
    const bool small = n8 < ((int64_t)1 << 28);  // unit byte offsets fit 32 bits
    // grid-stride: as many workgroups as stay resident together (one round),
    // split over the B tensors, at most stream_blocks per tensor
#define NVQ_ENC(MODE_, IDX_)                                                                                        \
    do {                                                                                                            \
        static const int per_cu = resident_blocks((const void*)k_nvfp4_encode_bf16<MODE_, IDX_>);                 \
        const int64_t gx = std::max<int64_t>(1, std::min<int64_t>(stream_blocks(n8, B),                             \
                                                                     (int64_t)device_cus() * per_cu / B));          \
        hipLaunchKernelGGL((k_nvfp4_encode_bf16<MODE_, IDX_>), dim3((unsigned)gx, (unsigned)B), dim3(256), 0, s, xk, \
                           n8, part, n_part, part_stride, ck, scales, tscale, seed, stream_id);                      \
    } while (0)
    if (mode == NVQ_SR) {
        if (small) NVQ_ENC(NVQ_SR, uint32_t); else NVQ_ENC(NVQ_SR, int64_t);
    } else {
        if (small) NVQ_ENC(NVQ_RTN, uint32_t); else NVQ_ENC(NVQ_RTN, int64_t);
    }
#undef NVQ_ENC
}

// ------------------------------------------------------------------ decode
// value = (e2m1 * e4m3) * D in fp32: the first product is exact, so one
// rounding. The E2M1 -> fp32 step is the gfx950 converter at scale 1.0
// (exact: every E2M1 value is an fp32).
constexpr int kDecodeP = 2;  // units a lane of the decoder has in flight

template <int OUT>
__global__ __launch_bounds__(256) void k_nvfp4_decode(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ tscale, int64_t n8,
                                                      void* __restrict__ out) {
    const int64_t b = blockIdx.y;
    const float D = tscale[b];
    const uint32_t* cb = codes + b * n8;
    const uint8_t* sb = scales + b * (n8 / 2);
    // grid-stride order (the whole grid writes one contiguous window at a time)
    const int64_t step = (int64_t)gridDim.x * (256 * kDecodeP);
    for (int64_t i = (int64_t)blockIdx.x * (256 * kDecodeP) + threadIdx.x; i < n8; i += step) {
        uint32_t w[kDecodeP], sc[kDecodeP];
#pragma unroll
        for (int p = 0; p < kDecodeP; ++p) {
            const int64_t u = min(i + 256 * p, n8 - 1);
            w[p] = __builtin_nontemporal_load(cb + u);
            sc[p] = sb[u / 2];
        }
#pragma unroll
        for (int p = 0; p < kDecodeP; ++p) {
            const int64_t u = i + 256 * p;
            if (u >= n8) continue;
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

// ------------------------------------------------------------------ no-allocation variant
// Partial maxima of nvfp4_quantize_noalloc: a file-scope device array. Its
// host-side name is only a stand-in, so host code uses the device address
// hipGetSymbolAddress gives for the current device (each device holds its own
// copy), looked up once per device and kept.
constexpr int64_t kNoAllocWords = 65536;  // >= B * stream_blocks(n8, B) for every B <= 65535
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint32_t scratch[kNoAllocWords];
static std::mutex g_scratch_mu;
static uint32_t* g_scratch[kMaxDevices] = {};

static int scratch_for_current_device(uint32_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return NVQ_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return NVQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NVQ_ERR_LAUNCH;
        g_scratch[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch[dev];
    return NVQ_OK;
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

int nvfp4_quantize_noalloc(const uint16_t* x, int64_t B, int64_t R, int64_t C, uint8_t* codes, uint8_t* scales,
                           float* tscale, int round_mode, uint64_t seed, uint32_t stream_id, nvq_stream_t stream) {
    if (!x || !codes || !scales || !tscale) return NVQ_ERR_NULL;
    if (B <= 0 || B > 65535 || R < 0 || C <= 0 || (C % 16) != 0) return NVQ_ERR_DIM;
    if (round_mode != NVQ_RTN && round_mode != NVQ_SR) return NVQ_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return NVQ_ERR_ALIGN;
    const int64_t n = R * C;
    const int G = stream_blocks(n / 8, B);
    if (B * (int64_t)G > kNoAllocWords) return NVQ_ERR_WORKSPACE;
    uint32_t* part = nullptr;
    const int st = scratch_for_current_device(&part);
    if (st != NVQ_OK) return st;
    hipStream_t s = as_stream(stream);
    // every partial maximum is written by the amax pass before the encode
    // pass reads it (stream order), so nothing is cleared
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
    // two steps of 256 * kDecodeP units per workgroup: on gfx950 a short
    // pass finishes sooner with the hardware spreading many small workgroups
    // than with a resident grid looping (29.4 against 31.9 us at 8192 x 8192)
    const int64_t per_tensor = (n8 + 512 * kDecodeP - 1) / (512 * kDecodeP);
    if (per_tensor > 0x7FFFFFFF) return NVQ_ERR_DIM;
    dim3 grid((unsigned)per_tensor, (unsigned)B);
    hipStream_t s = as_stream(stream);
    auto ck = reinterpret_cast<const uint32_t*>(codes);
    if (out_dtype == NVQ_OUT_BF16)
        hipLaunchKernelGGL(k_nvfp4_decode<NVQ_OUT_BF16>, grid, dim3(256), 0, s, ck, scales, tscale, n8, out);
    else
        hipLaunchKernelGGL(k_nvfp4_decode<NVQ_OUT_F32>, grid, dim3(256), 0, s, ck, scales, tscale, n8, out);
    return launch_status();
}

}  // extern "C"
