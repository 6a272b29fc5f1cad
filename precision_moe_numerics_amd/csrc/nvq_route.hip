// nvq_route.hip -- expert segments for the grouped GEMMs: a stable sort of
// the T*k (token, slot) assignments by expert id (8 of 384 experts per token
// on page "AI模型库 · 今日一模 Inkling 2 Small", "01 PART").
//
// Determinism without ordered atomics: assignments are cut into chunks of
// 1024; each chunk sorts the keys (expert << 10 | position) in LDS with a
// bitonic network (keys are unique, so the order is the stable one), and
// records per-expert run starts and lengths. One block turns the per-chunk
// counts into global bases (a prefix over chunks, then over experts); a
// scatter pass writes each assignment to base + rank-within-run.
#include "nvq_device.hpp"
#include "nvq_host.hpp"

namespace nvq {

constexpr int kChunk = 1024;
constexpr int kMaxExperts = 4096;
constexpr uint32_t kNoKey = 0xFFFFFFFFu;

static int64_t route_chunks(int64_t A) { return A > 0 ? (A + kChunk - 1) / kChunk : 1; }

// ws words: keys [nch*1024] | base [nch*E] | start [nch*E]
size_t route_ws_words(int64_t A, int64_t E) {
    int64_t nch = route_chunks(A);
    return (size_t)(nch * kChunk + 2 * nch * E);
}

__global__ __launch_bounds__(1024) void k_route_sort(const int32_t* __restrict__ ids, int64_t A, int E,
                                                     uint32_t* __restrict__ keys, int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ start) {
    __shared__ uint32_t sk[kChunk];
    __shared__ int32_t s_first[kMaxExperts];
    __shared__ int32_t s_end[kMaxExperts];
    const int t = threadIdx.x;
    const int64_t a = (int64_t)blockIdx.x * kChunk + t;
    uint32_t key = kNoKey;
    if (a < A) {
        int id = ids[a];
        if (id >= 0 && id < E) key = ((uint32_t)id << 10) | (uint32_t)t;
    }
    sk[t] = key;
    for (int e = t; e < E; e += kChunk) { s_first[e] = 0; s_end[e] = 0; }
    __syncthreads();
    for (int size = 2; size <= kChunk; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const int partner = t ^ stride;
            if (partner > t) {
                const uint32_t x = sk[t], y = sk[partner];
                const bool ascending = (t & size) == 0;
                if ((x > y) == ascending) { sk[t] = y; sk[partner] = x; }
            }
            __syncthreads();
        }
    }
    const uint32_t k = sk[t];
    keys[(int64_t)blockIdx.x * kChunk + t] = k;
    if (k != kNoKey) {
        const uint32_t e = k >> 10;
        if (t == 0 || (sk[t - 1] >> 10) != e) s_first[e] = t;
        if (t == kChunk - 1 || (sk[t + 1] >> 10) != e) s_end[e] = t + 1;
    }
    __syncthreads();
    int32_t* crow = cnt + (int64_t)blockIdx.x * E;
    int32_t* srow = start + (int64_t)blockIdx.x * E;
    for (int e = t; e < E; e += kChunk) {
        crow[e] = s_end[e] - s_first[e];
        srow[e] = s_first[e];
    }
}

// Per-expert totals -> offsets [E+1], optional tile offsets [E+1] (prefix
// sums of ceil(n_e / tile_m)) and optional tile map (the expert of every
// m-tile); converts cnt [nch][E] into absolute per-chunk bases. Each thread
// owns experts [4t, 4t+4).
__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ cnt, int nch, int E,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ tile_offsets,
                                                     int32_t* __restrict__ tile_map, int tile_m) {
    __shared__ int32_t tot[kMaxExperts];
    __shared__ int buf[1024];
    const int t = threadIdx.x;
    // Column walks over the chunks, 16 loads in flight at a time (a walk
    // with one dependent load per chunk pays the memory latency nch times).
    constexpr int kB = 16;
    for (int e = t; e < E; e += 1024) {
        int run = 0;
        for (int c0 = 0; c0 < nch; c0 += kB) {
            int v[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) v[u] = c0 + u < nch ? cnt[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                if (c0 + u < nch) cnt[(int64_t)(c0 + u) * E + e] = run;
                run += v[u];
            }
        }
        tot[e] = run;
    }
    __syncthreads();
    int local = 0, local_tiles = 0;
    for (int j = 0; j < 4; ++j) {
        int e = 4 * t + j;
        if (e < E) { local += tot[e]; local_tiles += (tot[e] + tile_m - 1) / tile_m; }
    }
    int total, total_tiles;
    int base = block_exclusive_scan(local, buf, &total);
    int tbase = block_exclusive_scan(local_tiles, buf, &total_tiles);
    int32_t mine[4];
    for (int j = 0; j < 4; ++j) {
        int e = 4 * t + j;
        mine[j] = base;
        if (e < E) {
            offsets[e] = base;
            const int nt = (tot[e] + tile_m - 1) / tile_m;
            if (tile_offsets) tile_offsets[e] = tbase;
            if (tile_map)
                for (int m = 0; m < nt; ++m) tile_map[tbase + m] = e;
            base += tot[e];
            tbase += nt;
        }
    }
    if (t == 0) {
        offsets[E] = total;
        if (tile_offsets) tile_offsets[E] = total_tiles;
    }
    __syncthreads();  // every thread has read tot[] for its own experts
    for (int j = 0; j < 4; ++j) {
        int e = 4 * t + j;
        if (e < E) tot[e] = mine[j];  // exclusive offset of expert e, kept in LDS
    }
    __syncthreads();
    for (int e = t; e < E; e += 1024) {
        const int off = tot[e];
        for (int c0 = 0; c0 < nch; c0 += kB) {
            int v[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) v[u] = c0 + u < nch ? cnt[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < kB; ++u)
                if (c0 + u < nch) cnt[(int64_t)(c0 + u) * E + e] = v[u] + off;
        }
    }
}

__global__ __launch_bounds__(1024) void k_route_scatter(const uint32_t* __restrict__ keys,
                                                        const int32_t* __restrict__ base,
                                                        const int32_t* __restrict__ start, int E,
                                                        int32_t* __restrict__ sorted2assign) {
    const int t = threadIdx.x;
    const uint32_t k = keys[(int64_t)blockIdx.x * kChunk + t];
    if (k == kNoKey) return;
    const int e = (int)(k >> 10);
    const int64_t row = (int64_t)blockIdx.x * E + e;
    sorted2assign[base[row] + (t - start[row])] = (int32_t)((int64_t)blockIdx.x * kChunk + (k & 1023u));
}

// tile_offsets [E+1] from offsets [E+1] (prefix sums of ceil(n_e / tile_m))
// and, if tile_map is not null, the expert of every m-tile.
__global__ __launch_bounds__(1024) void k_tile_offsets(const int32_t* __restrict__ offsets, int E, int tile_m,
                                                       int32_t* __restrict__ tile_offsets,
                                                       int32_t* __restrict__ tile_map) {
    __shared__ int buf[1024];
    const int t = threadIdx.x;
    int local = 0;
    for (int j = 0; j < 4; ++j) {
        int e = 4 * t + j;
        if (e < E) local += (offsets[e + 1] - offsets[e] + tile_m - 1) / tile_m;
    }
    int total;
    int tb = block_exclusive_scan(local, buf, &total);
    for (int j = 0; j < 4; ++j) {
        int e = 4 * t + j;
        if (e < E) {
            const int nt = (offsets[e + 1] - offsets[e] + tile_m - 1) / tile_m;
            tile_offsets[e] = tb;
            if (tile_map)
                for (int m = 0; m < nt; ++m) tile_map[tb + m] = e;
            tb += nt;
        }
    }
    if (t == 0) tile_offsets[E] = total;
}

void launch_route(const int32_t* topk_ids, int64_t A, int64_t E, int32_t* offsets, int32_t* sorted2assign,
                  int32_t* tile_offsets, int32_t* tile_map, int tile_m, uint32_t* ws, hipStream_t s) {
    const int64_t nch = route_chunks(A);
    uint32_t* keys = ws;
    int32_t* cnt = reinterpret_cast<int32_t*>(ws + nch * kChunk);
    int32_t* start = cnt + nch * E;
    hipLaunchKernelGGL(k_route_sort, dim3((unsigned)nch), dim3(kChunk), 0, s, topk_ids, A, (int)E, keys, cnt,
                       start);
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, s, cnt, (int)nch, (int)E, offsets, tile_offsets,
                       tile_map, tile_m);
    hipLaunchKernelGGL(k_route_scatter, dim3((unsigned)nch), dim3(kChunk), 0, s, keys, cnt, start, (int)E,
                       sorted2assign);
}

void launch_tile_offsets(const int32_t* offsets, int64_t E, int tile_m, int32_t* tile_offsets, int32_t* tile_map,
                         hipStream_t s) {
    hipLaunchKernelGGL(k_tile_offsets, dim3(1), dim3(1024), 0, s, offsets, (int)E, tile_m, tile_offsets, tile_map);
}

// ------------------------------------------------------------------ router
// Sigmoid router with a selection-only load-balancing bias (page "Thinking
// Machines首發大模型：9750億參數，完整開放權重", section "架構", on the lab's
// earlier Inkling model, whose design this reading takes for Inkling 2 Small:
// DeepSeek-V3 style, sigmoid scores, a bias without an auxiliary loss for
// balance, the chosen scores normalized).
// One wave per token; lane l holds experts l + 64 j. Scores and keys are fp64
// (s = 1 / (1 + exp(-logit)), key = s + bias), so that the choice does not
// hinge on how a single-precision exponential rounds. k rounds of a wave-wide
// argmax (largest key, then the lower expert index) pick the experts in order;
// lane j < k writes the j-th id and its weight s / (sum of the chosen s, in
// choice order).
constexpr int kRouterPerLane = 16;  // experts per lane at most: E <= 1024

// P: expert slots per lane (a power of two with 64 P >= E), so that the
// rounds scan only the slots the expert count needs.
template <int P>
__global__ __launch_bounds__(256) void k_router_sigmoid_topk(const float* __restrict__ logits,
                                                             const float* __restrict__ bias, int T, int E, int k,
                                                             int32_t* __restrict__ ids, float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (t >= T) return;  // whole waves
    double s[P], key[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        const int e = lane + 64 * j;
        s[j] = 0.0;
        key[j] = -__builtin_inf();
        if (e < E) {
            s[j] = 1.0 / (1.0 + exp(-(double)logits[(int64_t)t * E + e]));
            key[j] = s[j] + (double)bias[e];
        }
    }
    double sum = 0.0, my_s = 0.0;
    int my_id = 0;
    for (int r = 0; r < k; ++r) {
        double bk = -__builtin_inf();
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < P; ++j)
            if (key[j] > bk) { bk = key[j]; be = lane + 64 * j; }  // ascending j: the first of equal keys stays
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const double ok = __shfl_xor(bk, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (ok > bk || (ok == bk && oe < be)) { bk = ok; be = oe; }
        }
        // every lane now holds the winner; its owner supplies the score and drops it
        double sw = 0.0;
#pragma unroll
        for (int j = 0; j < P; ++j)
            if (lane + 64 * j == be) { sw = s[j]; key[j] = -__builtin_inf(); }
        sw = __shfl(sw, be & 63, 64);
        sum += sw;
        if (lane == r) { my_id = be; my_s = sw; }
    }
    if (lane < k) {
        ids[(int64_t)t * k + lane] = my_id;
        w[(int64_t)t * k + lane] = (float)(my_s / sum);
    }
}

}  // namespace nvq

using namespace nvq;

extern "C" {

int moe_router_sigmoid_topk(const float* logits, int64_t T, int64_t E, const float* bias, int k, int32_t* topk_ids,
                            float* weights, nvq_stream_t stream) {
    if (!logits || !bias || !topk_ids || !weights) return NVQ_ERR_NULL;
    if (T < 0 || E < 1 || E > 64 * kRouterPerLane || k < 1 || k > E || k > 64 || T * E >= ((int64_t)1 << 31))
        return NVQ_ERR_DIM;
    if (T == 0) return NVQ_OK;
    const dim3 grid((unsigned)((T + 3) / 4));
    hipStream_t s = as_stream(stream);
#define NVQ_ROUTER(P_) \
    hipLaunchKernelGGL(k_router_sigmoid_topk<P_>, grid, dim3(256), 0, s, logits, bias, (int)T, (int)E, k, topk_ids, weights)
    if (E <= 64) NVQ_ROUTER(1);
    else if (E <= 128) NVQ_ROUTER(2);
    else if (E <= 256) NVQ_ROUTER(4);
    else if (E <= 512) NVQ_ROUTER(8);
    else NVQ_ROUTER(16);
#undef NVQ_ROUTER
    return launch_status();
}


size_t moe_route_workspace_size(int64_t A, int64_t E) {
    Carver c(nullptr);
    c.take<uint32_t>(route_ws_words(A, E > 0 ? E : 1));
    c.take<int32_t>((size_t)(E > 0 ? E : 1) + 1);
    return c.need;
}

int moe_route(const int32_t* topk_ids, int64_t A, int64_t E, int32_t* offsets, int32_t* sorted2assign,
              int32_t* tile_offsets, void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!topk_ids || !offsets || !sorted2assign || !ws) return NVQ_ERR_NULL;
    if (A < 0 || A >= (int64_t)1 << 31 || E <= 0 || E > kMaxExperts) return NVQ_ERR_DIM;
    if (!aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_route_workspace_size(A, E)) return NVQ_ERR_WORKSPACE;
    Carver cv(ws);
    uint32_t* rw = cv.take<uint32_t>(route_ws_words(A, E));
    int32_t* tiles = tile_offsets ? tile_offsets : cv.take<int32_t>((size_t)E + 1);
    launch_route(topk_ids, A, E, offsets, sorted2assign, tiles, nullptr, 256, rw, as_stream(stream));
    return launch_status();
}

}  // extern "C"
