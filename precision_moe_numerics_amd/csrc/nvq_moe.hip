// nvq_moe.hip -- NVFP4 forward through the MoE expert layers on gfx950:
// grouped GEMM fc1 -> SwiGLU -> NVFP4 re-quantization -> fc2.
//
// The recipe runs only the expert-layer forward in NVFP4 and re-quantizes
// between the two GEMMs (page "Thinking Machines Details End-to-End 4-Bit
// Training for Inkling 2 Small", sections "Key Takeaways" and "Architecture
// highlights"); 8 of 384 experts per token (page "AI模型库 · 今日一模 Inkling 2
// Small", "01 PART").
//
// Contraction design for CDNA4. NVFP4 scales are E4M3 per 16 elements, while
// the block-scaled MFMA of gfx950 takes E8M0 per 32, so the scales cannot be
// handed to the hardware. Instead every operand value e2m1 * e4m3 (at most 6
// significant bits, magnitude in [2^-10, 2688]) is formed EXACTLY in fp16 on
// the way from HBM into LDS and fed to fp16 MFMA (v_mfma_f32_32x32x16_f16)
// with fp32 accumulation; the two per-tensor fp32 scales are applied once in
// the epilogue. The contraction therefore runs at the 16-bit MFMA rate and
// reads 4.5 bits per operand value from HBM.
//
// Tiling: a 256-thread workgroup computes a 128x128 output tile as 2x2 waves
// of 64x64 (2x2 MFMA blocks each), K in steps of 64 with LDS double
// buffering (2 x 32 KiB) and register prefetch of the next step's codes.
// LDS rows are 128 bytes; 16-byte chunks are XOR-swizzled by row so the
// MFMA operand reads (ds_read_b128) are bank-conflict free. A persistent grid
// walks (expert, m-tile, n-tile) tiles from device-side tile offsets, so no
// host sync is needed for the ragged expert segments; consecutive tiles go
// to workgroups on the same XCD so their shared rows stay in one L2.
#include "nvq_device.hpp"
#include "nvq_host.hpp"

namespace nvq {

void launch_tile_offsets(const int32_t* offsets, int64_t E, int tile_m, int32_t* tile_offsets, hipStream_t s);

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kRowBytes = kBK * 2;                 // fp16 row of a K step
constexpr int kTileBytes = kBM * kRowBytes;        // 16 KiB per operand per stage
constexpr int kGemmThreads = 256;

enum { kFC1 = 0, kFC2 = 1 };

struct GemmArgs {
    const uint8_t* a_codes;      // FC1: Xq [T, K/2]; FC2: Hq [A, K/2]
    const uint8_t* a_scales;
    const float* a_tscale;
    const int32_t* offsets;      // [E+1]
    const int32_t* sorted2assign;
    const int32_t* tile_offsets; // [E+1], m-tiles of kBM rows
    const uint8_t* b_codes;      // [E, b_rows, K/2]
    const uint8_t* b_scales;
    const float* b_tscale;       // [E]
    uint16_t* out;               // FC1: H [A, n_half]; FC2: y [A, N]
    uint16_t* gu;                // FC1 only, nullable: [A, 2*n_half]
    uint32_t* amax;              // FC1 only, nullable: max |h| as fp32 bits
    int E, K, b_rows, topk;
    int n_out;                   // FC1: d_ff; FC2: d
    int n_tiles;                 // output tiles along N
};

// fp16 bits of an E4M3 magnitude byte, duplicated into both halves.
__device__ __forceinline__ uint32_t e4m3_to_f16x2(uint32_t b) {
    _Float16 h = (_Float16)e4m3_mag_to_f32(b & 0x7Fu);  // exact: E4M3 values are fp16 normals
    uint32_t u = (uint32_t)__builtin_bit_cast(uint16_t, h);
    return u | (u << 16);
}

// Eight E2M1 codes (one 32-bit word, element 0 in the low nibble) times one
// fp16 scale -> eight exact fp16 values. The code magnitudes {0,.5,1,1.5,2,3,
// 4,6} have fp16 patterns 0xHH00, so one byte permute looks up four high
// bytes at once; the sign bit of each code lands on bit 15.
__device__ __forceinline__ uint4 dequant8_f16(uint32_t w, uint32_t s2) {
    const uint32_t lut_lo = 0x3E3C3800u;   // 0, 0.5, 1, 1.5
    const uint32_t lut_hi = 0x46444240u;   // 2, 3, 4, 6
    const uint32_t mag = w & 0x77777777u;
    const uint32_t ev = mag & 0x0F0F0F0Fu;           // codes 0,2,4,6 in bytes 0..3
    const uint32_t od = (mag >> 4) & 0x0F0F0F0Fu;    // codes 1,3,5,7
    const uint32_t he = __builtin_amdgcn_perm(lut_hi, lut_lo, ev) | ((w << 4) & 0x80808080u);
    const uint32_t ho = __builtin_amdgcn_perm(lut_hi, lut_lo, od) | (w & 0x80808080u);
    const half2v sc = __builtin_bit_cast(half2v, s2);
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(ho, he, 0x040C000Cu)) * sc);
    r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(ho, he, 0x050C010Cu)) * sc);
    r.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(ho, he, 0x060C020Cu)) * sc);
    r.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(ho, he, 0x070C030Cu)) * sc);
    return r;
}

// One thread's share of a K step: 32 codes (16 bytes) of one tile row and
// the two scale bytes of their 16-element blocks.
struct Frag {
    uint4 c;
    uint32_t s;
};

__device__ __forceinline__ Frag load_frag(const uint8_t* codes, const uint8_t* scales, bool valid) {
    Frag f;
    if (valid) {
        f.c = *reinterpret_cast<const uint4*>(codes);
        f.s = *reinterpret_cast<const uint16_t*>(scales);
    } else {
        f.c = make_uint4(0, 0, 0, 0);
        f.s = 0;
    }
    return f;
}

// Writes the 32 dequantized fp16 values as four 16-byte chunks of tile row
// `row`, logical chunks 4*half .. 4*half+3, swizzled by (row & 7).
__device__ __forceinline__ void store_frag(uint8_t* tile, int row, int half, const Frag& f) {
    const uint32_t s0 = e4m3_to_f16x2(f.s & 0xFFu), s1 = e4m3_to_f16x2(f.s >> 8);
    uint8_t* rp = tile + row * kRowBytes;
    const int sw = row & 7;
    *reinterpret_cast<uint4*>(rp + (((4 * half + 0) ^ sw) << 4)) = dequant8_f16(f.c.x, s0);
    *reinterpret_cast<uint4*>(rp + (((4 * half + 1) ^ sw) << 4)) = dequant8_f16(f.c.y, s0);
    *reinterpret_cast<uint4*>(rp + (((4 * half + 2) ^ sw) << 4)) = dequant8_f16(f.c.z, s1);
    *reinterpret_cast<uint4*>(rp + (((4 * half + 3) ^ sw) << 4)) = dequant8_f16(f.c.w, s1);
}

// MFMA operand: 8 consecutive K values (logical chunk `chunk`) of tile row `row`.
__device__ __forceinline__ half8 load_operand(const uint8_t* tile, int row, int chunk) {
    return *reinterpret_cast<const half8*>(tile + row * kRowBytes + ((chunk ^ (row & 7)) << 4));
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 2) void k_grouped_gemm_nvfp4(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];  // [stage][A|B]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = tid >> 1, lhalf = tid & 1;  // loader role: tile row, K half
    const int64_t total = (int64_t)p.tile_offsets[p.E] * p.n_tiles;
    const int G = gridDim.x;
    // consecutive virtual ids on one XCD (workgroups are dealt to the 8 XCDs round robin)
    const int v = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
    const int nk = p.K / kBK;
    const int64_t a_row_codes = p.K / 2, a_row_scales = p.K / 16;

    for (int64_t t = v; t < total; t += G) {
        const int mt = (int)(t / p.n_tiles), nt = (int)(t % p.n_tiles);
        int lo = 0, hi = p.E;  // tile_offsets[lo] <= mt < tile_offsets[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.tile_offsets[mid] <= mt) lo = mid; else hi = mid;
        }
        const int e = lo;
        const int row0 = p.offsets[e] + (mt - p.tile_offsets[e]) * kBM;
        const int row_end = p.offsets[e + 1];

        // loader sources for this tile
        const int ar = row0 + lrow;
        const bool a_valid = ar < row_end;
        int64_t a_src = 0;
        if (a_valid) a_src = (MODE == kFC1) ? (int64_t)(p.sorted2assign[ar] / p.topk) : (int64_t)ar;
        const uint8_t* a_c = p.a_codes + a_src * a_row_codes + lhalf * 16;
        const uint8_t* a_s = p.a_scales + a_src * a_row_scales + lhalf * 2;
        int brow;
        if (MODE == kFC1) {
            // tile columns: [gate j0..+31 | up j0..+31 | gate j0+32..+63 | up j0+32..+63]
            const int blk = lrow >> 5;
            const int j = nt * (kBN / 2) + (blk >> 1) * 32 + (lrow & 31);
            brow = (blk & 1) ? p.n_out + j : j;
        } else {
            brow = nt * kBN + lrow;
        }
        const uint8_t* b_c = p.b_codes + ((int64_t)e * p.b_rows + brow) * a_row_codes + lhalf * 16;
        const uint8_t* b_s = p.b_scales + ((int64_t)e * p.b_rows + brow) * a_row_scales + lhalf * 2;

        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        Frag fa = load_frag(a_c, a_s, a_valid);
        Frag fb = load_frag(b_c, b_s, true);
        store_frag(lds[0][0], lrow, lhalf, fa);
        store_frag(lds[0][1], lrow, lhalf, fb);
        __syncthreads();

        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) {
                fa = load_frag(a_c + (kt + 1) * 32, a_s + (kt + 1) * 4, a_valid);
                fb = load_frag(b_c + (kt + 1) * 32, b_s + (kt + 1) * 4, true);
            }
            const uint8_t* ta = lds[cur][0];
            const uint8_t* tb = lds[cur][1];
#pragma unroll
            for (int kk = 0; kk < kBK / 16; ++kk) {
                const int chunk = kk * 2 + (lane >> 5);
                half8 av[2], bv[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) av[i] = load_operand(ta, wm * 64 + i * 32 + (lane & 31), chunk);
#pragma unroll
                for (int j = 0; j < 2; ++j) bv[j] = load_operand(tb, wn * 64 + j * 32 + (lane & 31), chunk);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
            }
            if (more) {
                store_frag(lds[cur ^ 1][0], lrow, lhalf, fa);
                store_frag(lds[cur ^ 1][1], lrow, lhalf, fb);
            }
            __syncthreads();
        }

        // ---------------- epilogue
        const float scale = p.a_tscale[0] * p.b_tscale[e];
        const int col = lane & 31;
        if (MODE == kFC1) {
            const int j = nt * (kBN / 2) + wn * 32 + col;   // column of H (and of the gate)
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    if (row < row_end) {
                        const float g = acc[i][0][r] * scale;
                        const float u = acc[i][1][r] * scale;
                        const float h = (g / (1.0f + expf(-g))) * u;
                        const uint32_t hb = f32_to_bf16(h);
                        p.out[(int64_t)row * p.n_out + j] = (uint16_t)hb;
                        m = max(m, hb & 0x7FFFu);
                        if (p.gu) {
                            p.gu[(int64_t)row * 2 * p.n_out + j] = (uint16_t)f32_to_bf16(g);
                            p.gu[(int64_t)row * 2 * p.n_out + p.n_out + j] = (uint16_t)f32_to_bf16(u);
                        }
                    }
                }
            }
            if (p.amax) {
                m = wave_max_u32(m);
                if (lane == 0 && m) atomicMax(p.amax, m << 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    if (row < row_end) {
                        uint16_t* yrow = p.out + (int64_t)p.sorted2assign[row] * p.n_out;
#pragma unroll
                        for (int jb = 0; jb < 2; ++jb) {
                            const int n = nt * kBN + wn * 64 + jb * 32 + col;
                            yrow[n] = (uint16_t)f32_to_bf16(acc[i][jb][r] * scale);
                        }
                    }
                }
            }
        }
    }
}

static int gemm_grid() {
    static int g = 0;
    if (g == 0) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
                cus = prop.multiProcessorCount;
        }
        g = cus * 2;  // two 64 KiB-LDS workgroups per CU
    }
    return g;
}

void launch_fc1(const uint8_t* xc, const uint8_t* xs, const float* xt, const int32_t* offsets,
                const int32_t* s2a, const int32_t* tiles, int topk, int64_t E, int64_t d, int64_t d_ff,
                const uint8_t* wc, const uint8_t* wsc, const float* wt, uint16_t* h, uint16_t* gu,
                uint32_t* amax, hipStream_t s) {
    GemmArgs p{};
    p.a_codes = xc; p.a_scales = xs; p.a_tscale = xt;
    p.offsets = offsets; p.sorted2assign = s2a; p.tile_offsets = tiles;
    p.b_codes = wc; p.b_scales = wsc; p.b_tscale = wt;
    p.out = h; p.gu = gu; p.amax = amax;
    p.E = (int)E; p.K = (int)d; p.b_rows = (int)(2 * d_ff); p.topk = topk;
    p.n_out = (int)d_ff; p.n_tiles = (int)(d_ff / (kBN / 2));
    hipLaunchKernelGGL(k_grouped_gemm_nvfp4<kFC1>, dim3(gemm_grid()), dim3(kGemmThreads), 0, s, p);
}

void launch_fc2(const uint8_t* hc, const uint8_t* hs, const float* ht, const int32_t* offsets,
                const int32_t* s2a, const int32_t* tiles, int64_t E, int64_t d_ff, int64_t d,
                const uint8_t* wc, const uint8_t* wsc, const float* wt, uint16_t* y, hipStream_t s) {
    GemmArgs p{};
    p.a_codes = hc; p.a_scales = hs; p.a_tscale = ht;
    p.offsets = offsets; p.sorted2assign = s2a; p.tile_offsets = tiles;
    p.b_codes = wc; p.b_scales = wsc; p.b_tscale = wt;
    p.out = y;
    p.E = (int)E; p.K = (int)d_ff; p.b_rows = (int)d; p.topk = 1;
    p.n_out = (int)d; p.n_tiles = (int)(d / kBN);
    hipLaunchKernelGGL(k_grouped_gemm_nvfp4<kFC2>, dim3(gemm_grid()), dim3(kGemmThreads), 0, s, p);
}

static bool moe_dims_ok(int64_t T, int64_t d, int k, int64_t E, int64_t d_ff) {
    return T >= 0 && d > 0 && d % kBN == 0 && d_ff > 0 && d_ff % (kBN / 2) == 0 && k >= 1 && E >= 1 &&
           k <= E && E <= 4096 && T * k < ((int64_t)1 << 31) && d_ff % kBK == 0 && d % kBK == 0;
}

}  // namespace nvq

using namespace nvq;

extern "C" {

size_t moe_fc1_workspace_size(int64_t A, int64_t E) {
    (void)A;
    Carver c(nullptr);
    c.take<int32_t>((size_t)(E > 0 ? E : 1) + 1);
    return c.need;
}

int moe_fc1_swiglu_nvfp4(const uint8_t* xq_codes, const uint8_t* xq_scales, const float* xq_tscale, int64_t T,
                         int64_t d, const int32_t* offsets, const int32_t* sorted2assign, int k, int64_t E,
                         int64_t d_ff, const uint8_t* w1_codes, const uint8_t* w1_scales,
                         const float* w1_tscale, uint16_t* h, uint16_t* gu, float* h_amax, void* ws,
                         size_t ws_bytes, nvq_stream_t stream) {
    if (!xq_codes || !xq_scales || !xq_tscale || !offsets || !sorted2assign || !w1_codes || !w1_scales ||
        !w1_tscale || !h || !ws)
        return NVQ_ERR_NULL;
    if (!moe_dims_ok(T, d, k, E, d_ff)) return NVQ_ERR_DIM;
    if (!aligned16(xq_codes) || !aligned16(w1_codes) || !aligned16(h) || !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_fc1_workspace_size(T * k, E)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    int32_t* tiles = cv.take<int32_t>((size_t)E + 1);
    launch_tile_offsets(offsets, E, kBM, tiles, s);
    uint32_t* amax = reinterpret_cast<uint32_t*>(h_amax);
    if (amax) launch_zero_u32(amax, 1, s);
    launch_fc1(xq_codes, xq_scales, xq_tscale, offsets, sorted2assign, tiles, k, E, d, d_ff, w1_codes,
               w1_scales, w1_tscale, h, gu, amax, s);
    return launch_status();
}

size_t moe_fc2_workspace_size(int64_t A, int64_t E) { return moe_fc1_workspace_size(A, E); }

int moe_fc2_nvfp4(const uint8_t* hq_codes, const uint8_t* hq_scales, const float* hq_tscale, int64_t A,
                  int64_t d_ff, const int32_t* offsets, const int32_t* sorted2assign, int64_t E, int64_t d,
                  const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_tscale, uint16_t* y,
                  void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!hq_codes || !hq_scales || !hq_tscale || !offsets || !sorted2assign || !w2_codes || !w2_scales ||
        !w2_tscale || !y || !ws)
        return NVQ_ERR_NULL;
    if (!moe_dims_ok(A, d, 1, E > 0 ? E : 1, d_ff)) return NVQ_ERR_DIM;
    if (!aligned16(hq_codes) || !aligned16(w2_codes) || !aligned16(y) || !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_fc2_workspace_size(A, E)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    int32_t* tiles = cv.take<int32_t>((size_t)E + 1);
    launch_tile_offsets(offsets, E, kBM, tiles, s);
    launch_fc2(hq_codes, hq_scales, hq_tscale, offsets, sorted2assign, tiles, E, d_ff, d, w2_codes, w2_scales,
               w2_tscale, y, s);
    return launch_status();
}

// Workspace plan of the fused forward (every carve 256-byte aligned):
//   amax words [2] | route scratch | tile offsets [E+1] | then any
//   intermediate the caller did not supply: Xq, offsets, sorted2assign, H, Hq.
static size_t moe_fwd_carve(Carver& c, int64_t T, int64_t d, int k, int64_t E, int64_t d_ff,
                            const nvq_moe_buffers* b, uint32_t** amax, uint32_t** rws, int32_t** tiles,
                            nvq_moe_buffers* out) {
    const int64_t A = T * k;
    *amax = c.take<uint32_t>(2);
    *rws = c.take<uint32_t>(route_ws_words(A, E));
    *tiles = c.take<int32_t>((size_t)E + 1);
    nvq_moe_buffers z{};
    const nvq_moe_buffers& in = b ? *b : z;
    out->xq_codes = in.xq_codes ? in.xq_codes : c.take<uint8_t>((size_t)(T * d / 2));
    out->xq_scales = in.xq_scales ? in.xq_scales : c.take<uint8_t>((size_t)(T * d / 16));
    out->xq_tscale = in.xq_tscale ? in.xq_tscale : c.take<float>(1);
    out->offsets = in.offsets ? in.offsets : c.take<int32_t>((size_t)E + 1);
    out->sorted2assign = in.sorted2assign ? in.sorted2assign : c.take<int32_t>((size_t)(A > 0 ? A : 1));
    out->h = in.h ? in.h : c.take<uint16_t>((size_t)(A * d_ff > 0 ? A * d_ff : 1));
    out->hq_codes = in.hq_codes ? in.hq_codes : c.take<uint8_t>((size_t)(A * d_ff / 2 > 0 ? A * d_ff / 2 : 16));
    out->hq_scales = in.hq_scales ? in.hq_scales : c.take<uint8_t>((size_t)(A * d_ff / 16 > 0 ? A * d_ff / 16 : 16));
    out->hq_tscale = in.hq_tscale ? in.hq_tscale : c.take<float>(1);
    out->gu = in.gu;
    return c.need;
}

size_t moe_expert_fwd_nvfp4_workspace_size(int64_t T, int64_t d, int k, int64_t E, int64_t d_ff) {
    Carver c(nullptr);
    uint32_t *a, *r;
    int32_t* t;
    nvq_moe_buffers o{};
    return moe_fwd_carve(c, T, d, k, E, d_ff, nullptr, &a, &r, &t, &o);
}

int moe_expert_fwd_nvfp4(const uint16_t* x, int64_t T, int64_t d, const int32_t* topk_ids, int k, int64_t E,
                         int64_t d_ff, const uint8_t* w1_codes, const uint8_t* w1_scales, const float* w1_tscale,
                         const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_tscale, uint16_t* y,
                         const nvq_moe_buffers* bufs, void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!x || !topk_ids || !w1_codes || !w1_scales || !w1_tscale || !w2_codes || !w2_scales || !w2_tscale || !y ||
        !ws)
        return NVQ_ERR_NULL;
    if (!moe_dims_ok(T, d, k, E, d_ff)) return NVQ_ERR_DIM;
    if (!aligned16(x) || !aligned16(w1_codes) || !aligned16(w2_codes) || !aligned16(y) || !aligned256(ws))
        return NVQ_ERR_ALIGN;
    Carver need(nullptr);
    {
        uint32_t *a, *r;
        int32_t* t;
        nvq_moe_buffers o{};
        if (ws_bytes < moe_fwd_carve(need, T, d, k, E, d_ff, bufs, &a, &r, &t, &o)) return NVQ_ERR_WORKSPACE;
    }
    if (bufs) {
        const nvq_moe_buffers& b = *bufs;
        const void* ptrs[] = {b.xq_codes, b.xq_scales, b.h, b.hq_codes, b.hq_scales, b.gu};
        for (const void* q : ptrs)
            if (q && !aligned16(q)) return NVQ_ERR_ALIGN;
    }
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    uint32_t *amax, *rws;
    int32_t* tiles;
    nvq_moe_buffers m{};
    moe_fwd_carve(cv, T, d, k, E, d_ff, bufs, &amax, &rws, &tiles, &m);
    const int64_t A = T * k;

    launch_zero_u32(amax, 2, s);
    // 1. NVFP4 of X (one tensor scale over X; rows are gathered later)
    launch_amax_bf16(x, 1, T * d, amax, s);
    launch_nvfp4_encode_bf16(x, 1, T * d, amax, m.xq_codes, m.xq_scales, m.xq_tscale, NVQ_RTN, 0, 1, s);
    // 2. expert segments
    launch_route(topk_ids, A, E, m.offsets, m.sorted2assign, tiles, kBM, rws, s);
    // 3. fc1 + SwiGLU, max |H| into amax[1]
    launch_fc1(m.xq_codes, m.xq_scales, m.xq_tscale, m.offsets, m.sorted2assign, tiles, k, E, d, d_ff, w1_codes,
               w1_scales, w1_tscale, m.h, m.gu, amax + 1, s);
    // 4. NVFP4 of H with one tensor scale over all of H
    launch_nvfp4_encode_bf16(m.h, 1, A * d_ff, amax + 1, m.hq_codes, m.hq_scales, m.hq_tscale, NVQ_RTN, 0, 1, s);
    // 5. fc2, scattered back to (token, slot) order
    launch_fc2(m.hq_codes, m.hq_scales, m.hq_tscale, m.offsets, m.sorted2assign, tiles, E, d_ff, d, w2_codes,
               w2_scales, w2_tscale, y, s);
    return launch_status();
}

}  // extern "C"
