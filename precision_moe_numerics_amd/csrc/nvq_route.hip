// nvq_route.hip -- expert segments for the grouped GEMMs: a stable sort of
// the T*k (token, slot) assignments by expert id (8 of 384 experts per token
// on page "AI模型库 · 今日一模 Inkling 2 Small", "01 PART").
//
// Determinism without ordered atomics: assignments are cut into chunks of
// 1024; each chunk sorts the keys (expert << 10 | position) with a bitonic
// network (keys are unique, so the order is the stable one), and records
// per-expert run starts and lengths. One block turns the per-chunk counts
// into global bases (a prefix over chunks, then over experts); a scatter
// pass writes each assignment to base + rank-within-run. When every
// assignment fits one chunk, one workgroup does all of it in one launch.
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

// The bitonic network over a chunk's 1024 keys, one key per thread, in
// place of v. Of its 55 compare-exchange stages, the 45 with partners less
// than 64 apart stay inside a wave and exchange through lane shuffles; the
// other 10 go through LDS, alternating between the two halves of sk so that
// each needs one barrier. Ends with the sorted keys in sk[0] (visible to the
// whole workgroup).
__device__ __forceinline__ uint32_t chunk_bitonic_sort(uint32_t v, uint32_t (*sk)[kChunk]) {
    const int t = threadIdx.x;
    int buf = 0;
    for (int size = 2; size <= kChunk; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            uint32_t y;
            if (stride >= 64) {
                sk[buf][t] = v;
                __syncthreads();
                y = sk[buf][t ^ stride];
                buf ^= 1;
            } else {
                y = (uint32_t)__shfl_xor((int)v, stride, 64);
            }
            // the lower index of a pair keeps the smaller key in an ascending
            // run of the network, the larger one in a descending run
            const bool keep_min = ((t & size) == 0) == ((t & stride) == 0);
            v = keep_min ? min(v, y) : max(v, y);
        }
    }
    __syncthreads();  // every read of the last LDS stage is done
    sk[0][t] = v;
    __syncthreads();
    return v;
}

// The key of assignment a of a chunk (thread t): expert << 10 | t, or kNoKey
// for positions past the end and ids outside [0, E).
__device__ __forceinline__ uint32_t route_key(const int32_t* ids, int64_t a, int64_t A, int E, int t) {
    if (a >= A) return kNoKey;
    const int id = ids[a];
    return id >= 0 && id < E ? ((uint32_t)id << 10) | (uint32_t)t : kNoKey;
}

// First position and end of each expert's run in the sorted chunk sk (the
// entries of experts without keys stay as initialised).
__device__ __forceinline__ void chunk_runs(const uint32_t* sk, uint32_t k, int32_t* s_first, int32_t* s_end) {
    const int t = threadIdx.x;
    if (k != kNoKey) {
        const uint32_t e = k >> 10;
        if (t == 0 || (sk[t - 1] >> 10) != e) s_first[e] = t;
        if (t == kChunk - 1 || (sk[t + 1] >> 10) != e) s_end[e] = t + 1;
    }
}

__global__ __launch_bounds__(1024) void k_route_sort(const int32_t* __restrict__ ids, int64_t A, int E,
                                                     uint32_t* __restrict__ keys, int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ start) {
    __shared__ uint32_t sk[2][kChunk];
    __shared__ int32_t s_first[kMaxExperts];
    __shared__ int32_t s_end[kMaxExperts];
    const int t = threadIdx.x;
    const uint32_t key = route_key(ids, (int64_t)blockIdx.x * kChunk + t, A, E, t);
    for (int e = t; e < E; e += kChunk) { s_first[e] = 0; s_end[e] = 0; }
    const uint32_t k = chunk_bitonic_sort(key, sk);
    keys[(int64_t)blockIdx.x * kChunk + t] = k;
    chunk_runs(sk[0], k, s_first, s_end);
    __syncthreads();
    int32_t* crow = cnt + (int64_t)blockIdx.x * E;
    int32_t* srow = start + (int64_t)blockIdx.x * E;
    for (int e = t; e < E; e += kChunk) {
        crow[e] = s_end[e] - s_first[e];
        srow[e] = s_first[e];
    }
}

// All assignments in one chunk (A <= 1024): the sort, the offsets, tile
// offsets and tile map (as k_route_scan computes them) and the scatter in one
// workgroup, with the same results as the three-pass path.
__global__ __launch_bounds__(1024) void k_route_one(const int32_t* __restrict__ ids, int64_t A, int E,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ sorted2assign,
                                                    int32_t* __restrict__ tile_offsets,
                                                    int32_t* __restrict__ tile_map, int tile_m) {
    __shared__ uint32_t sk[2][kChunk];
    __shared__ int32_t s_first[kMaxExperts];
    __shared__ int32_t s_end[kMaxExperts];
    __shared__ int buf[1024];
    const int t = threadIdx.x;
    const uint32_t key = route_key(ids, t, A, E, t);
    for (int e = t; e < E; e += kChunk) { s_first[e] = 0; s_end[e] = 0; }
    const uint32_t k = chunk_bitonic_sort(key, sk);
    chunk_runs(sk[0], k, s_first, s_end);
    __syncthreads();
    // thread t owns experts [4t, 4t + 4)
    int n[4], local = 0, local_tiles = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * t + j;
        n[j] = e < E ? s_end[e] - s_first[e] : 0;
        local += n[j];
        local_tiles += (n[j] + tile_m - 1) / tile_m;
    }
    int total, total_tiles;
    int base = block_exclusive_scan(local, buf, &total);
    int tbase = block_exclusive_scan(local_tiles, buf, &total_tiles);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * t + j;
        if (e < E) {
            offsets[e] = base;
            const int nt = (n[j] + tile_m - 1) / tile_m;
            if (tile_offsets) tile_offsets[e] = tbase;
            if (tile_map)
                for (int m = 0; m < nt; ++m) tile_map[tbase + m] = e;
            // the run's destination base replaces its end (only this thread
            // reads the experts it owns)
            s_end[e] = base - s_first[e];
            base += n[j];
            tbase += nt;
        }
    }
    if (t == 0) {
        offsets[E] = total;
        if (tile_offsets) tile_offsets[E] = total_tiles;
    }
    __syncthreads();
    if (k != kNoKey) sorted2assign[s_end[k >> 10] + t] = (int32_t)(k & 1023u);
}

// Per-expert totals -> offsets [E+1], optional tile offsets [E+1] (prefix
// sums of ceil(n_e / tile_m)) and optional tile map (the expert of every
// m-tile); converts cnt [nch][E] into absolute per-chunk bases. Each thread
// owns experts [4t, 4t+4).
// Given every expert's count in tot[] (a 1024-thread block, E <= 4096):
// segment offsets, tile offsets and the tile map; tot[e] then holds expert
// e's exclusive offset.
__device__ __forceinline__ void scan_expert_totals(int32_t* tot, int E, int tile_m, int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ tile_offsets,
                                                   int32_t* __restrict__ tile_map, int* buf) {
    const int t = threadIdx.x;
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
}

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
    scan_expert_totals(tot, E, tile_m, offsets, tile_offsets, tile_map, buf);
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

// The same scan with each expert's column of chunk counts split over P
// threads (t = h * E + e, P * E <= 1024) that hold their at most kR counts in
// registers: every count is loaded once, all loads are in flight together,
// and the results are stored once. (The loop above loads each column twice,
// in dependent batches behind its own stores.)
template <int kR>
__global__ __launch_bounds__(1024) void k_route_scan_reg(int32_t* __restrict__ cnt, int nch, int E, int P,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ tile_offsets,
                                                         int32_t* __restrict__ tile_map, int tile_m) {
    __shared__ int32_t tot[kMaxExperts];
    __shared__ int32_t part[1024];
    __shared__ int buf[1024];
    const int t = threadIdx.x;
    const bool act = t < P * E;
    const int e = act ? t % E : 0, h = act ? t / E : 0;
    const int len = (nch + P - 1) / P;
    const int c0 = h * len, c1 = min(nch, c0 + len);
    int v[kR];
    int sum = 0;
    if (act && c0 < c1) {
#pragma unroll
        for (int u = 0; u < kR; ++u) {
            const int c = min(c0 + u, c1 - 1);
            v[u] = cnt[(uint32_t)(c * E + e)];  // < 2^16 entries here: 32-bit offsets
        }
#pragma unroll
        for (int u = 0; u < kR; ++u) {
            v[u] = c0 + u < c1 ? v[u] : 0;
            sum += v[u];
        }
    }
    part[t] = act ? sum : 0;
    __syncthreads();
    int pre = 0;
    if (act)
        for (int g = 0; g < h; ++g) pre += part[g * E + e];
    for (int x = t; x < E; x += 1024) {
        int s = 0;
        for (int g = 0; g < P; ++g) s += part[g * E + x];
        tot[x] = s;
    }
    __syncthreads();
    scan_expert_totals(tot, E, tile_m, offsets, tile_offsets, tile_map, buf);
    if (act && c0 < c1) {
        int run = tot[e] + pre;
#pragma unroll
        for (int u = 0; u < kR; ++u) {
            if (c0 + u < c1) cnt[(uint32_t)((c0 + u) * E + e)] = run;
            run += v[u];
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
    if (nch == 1) {
        hipLaunchKernelGGL(k_route_one, dim3(1), dim3(kChunk), 0, s, topk_ids, A, (int)E, offsets, sorted2assign,
                           tile_offsets, tile_map, tile_m);
        return;
    }
    uint32_t* keys = ws;
    int32_t* cnt = reinterpret_cast<int32_t*>(ws + nch * kChunk);
    int32_t* start = cnt + nch * E;
    hipLaunchKernelGGL(k_route_sort, dim3((unsigned)nch), dim3(kChunk), 0, s, topk_ids, A, (int)E, keys, cnt,
                       start);
    // columns of at most kScanR counts per thread when P * E threads cover them
    constexpr int kScanR = 64;
    const int64_t P = (nch + kScanR - 1) / kScanR;
    if (P * E <= 1024)
        hipLaunchKernelGGL(k_route_scan_reg<kScanR>, dim3(1), dim3(1024), 0, s, cnt, (int)nch, (int)E, (int)P, offsets,
                           tile_offsets, tile_map, tile_m);
    else
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

// ------------------------------------------------------------------ softmax router
// Router of the configs: top-k of logit + bias, softmax over the k chosen raw
// logits (8 of 384 experts per token: page "AI模型库 · 今日一模 Inkling 2 Small",
// section "01 PART"; the bias only steers the choice, the design the page
// "Thinking Machines首發大模型：9750億參數，完整開放權重", section "架構",
// reports for the lab's earlier model).
//
// A group of G lanes (16 or 64) owns one token; lane g holds experts g + G j.
// Keys are fp64 (logit + bias of two fp32 values), mapped to unsigned
// integers with the same order (-0 first turned into +0, so equal keys stay
// equal). Each of the k rounds takes the lane's best slot (the lowest slot
// among equal keys, i.e. the lowest expert of that lane) and an all-reduce over
// the group's lanes by DPP (largest key, then the lower expert id); the owner
// drops the winner. The chosen raw logits then give the weights: p_j =
// exp(l_j - m) in fp64 with m the largest chosen logit, divided by the sum of
// the p_j taken in choice order, rounded to fp32.
__device__ __forceinline__ uint64_t order_key(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v + 0.0);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ void argmax_take(uint64_t& k, int& e, uint64_t ok, int oe) {
    const bool take = ok > k || (ok == k && oe < e);
    k = take ? ok : k;
    e = take ? oe : e;
}

template <int CTRL>
__device__ __forceinline__ void argmax_dpp(uint64_t& k, int& e) {
    const uint64_t ok = ((uint64_t)dpp_u32<CTRL>((uint32_t)(k >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)k);
    argmax_take(k, e, ok, (int)dpp_u32<CTRL>((uint32_t)e));
}

__device__ __forceinline__ void argmax_xor(uint64_t& k, int& e, int off) {
    const uint64_t ok = ((uint64_t)(uint32_t)__shfl_xor((int)(k >> 32), off, 64) << 32) |
                        (uint32_t)__shfl_xor((int)(uint32_t)k, off, 64);
    argmax_take(k, e, ok, __shfl_xor(e, off, 64));
}

// All-reduce over aligned groups of G lanes: every lane ends with the
// group's (largest key, lowest expert among those).
template <int G>
__device__ __forceinline__ void group_argmax(uint64_t& k, int& e) {
    argmax_dpp<0xB1>(k, e);   // lane ^ 1
    argmax_dpp<0x4E>(k, e);   // lane ^ 2
    argmax_dpp<0x141>(k, e);  // mirror within 8 lanes
    argmax_dpp<0x140>(k, e);  // mirror within 16 lanes
    if (G == 64) {
        argmax_xor(k, e, 16);
        argmax_xor(k, e, 32);
    }
}

template <int G, int P>
__global__ __launch_bounds__(256) void k_router_softmax_topk(const float* __restrict__ logits,
                                                             const float* __restrict__ bias, int T, int E, int k,
                                                             int32_t* __restrict__ ids, float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int g = lane & (G - 1);
    const int t = (int)((blockIdx.x * 256u + threadIdx.x) / G);
    const bool live = t < T;  // whole groups; every lane still joins the cross-lane steps
    const float* lt = logits + (int64_t)(live ? t : 0) * E;
    uint64_t key[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        const int e = g + G * j;
        key[j] = 0;  // below every finite key
        if (live && e < E) key[j] = order_key((double)lt[e] + (bias ? (double)bias[e] : 0.0));
    }
    int my_id = 0;
    for (int r = 0; r < k; ++r) {
        uint64_t bk = 0;
        int bj = 0;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const bool gt = key[j] > bk;  // strict: the lowest slot among equal keys stays
            bk = gt ? key[j] : bk;
            bj = gt ? j : bj;
        }
        int be = bk ? g + G * bj : 0x7FFFFFFF;
        group_argmax<G>(bk, be);
        if ((be & (G - 1)) == g) {
            const int wj = be / G;
#pragma unroll
            for (int j = 0; j < P; ++j) key[j] = (j == wj) ? 0 : key[j];
        }
        my_id = (g == r) ? be : my_id;
    }
    // weights over the chosen raw logits, summed in choice order
    const bool chosen = g < k;
    const double l = (live && chosen) ? (double)lt[my_id] : -__builtin_inf();
    double m = l;
#pragma unroll
    for (int off = 1; off < G; off <<= 1) m = fmax(m, __shfl_xor(m, off, 64));
    const double pj = chosen ? exp(l - m) : 0.0;
    const int base = lane & ~(G - 1);
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += __shfl(pj, base + j, 64);
    if (live && chosen) {
        ids[(int64_t)t * k + g] = my_id;
        w[(int64_t)t * k + g] = (float)(pj / sum);
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


size_t moe_router_softmax_topk_workspace_size(int64_t T, int64_t E, int k) {
    Carver c(nullptr);
    const int64_t A = T * (k > 0 ? k : 1);
    c.take<uint32_t>(route_ws_words(A > 0 ? A : 1, E > 0 ? E : 1));
    c.take<int32_t>((size_t)(E > 0 ? E : 1) + 1);
    return c.need;
}

int moe_router_softmax_topk(const float* logits, int64_t T, int64_t E, const float* bias, int k, int32_t* topk_ids,
                            float* weights, int32_t* offsets, int32_t* sorted2assign, int32_t* tile_offsets,
                            void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!logits || !topk_ids || !weights) return NVQ_ERR_NULL;
    const bool route = offsets != nullptr;
    if (route && (!sorted2assign || !ws)) return NVQ_ERR_NULL;
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 64 || T * E >= ((int64_t)1 << 31)) return NVQ_ERR_DIM;
    if (route && E > kMaxExperts) return NVQ_ERR_DIM;
    if (route && !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (route && ws_bytes < moe_router_softmax_topk_workspace_size(T, E, k)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    if (T > 0) {
#define NVQ_SROUTER(G_, P_)                                                                                    \
    hipLaunchKernelGGL((k_router_softmax_topk<G_, P_>), dim3((unsigned)((T + 256 / G_ - 1) / (256 / G_))), \
                       dim3(256), 0, s, logits, bias, (int)T, (int)E, k, topk_ids, weights)
        if (k <= 16 && E <= 512) {
            if (E <= 64) NVQ_SROUTER(16, 4);
            else if (E <= 128) NVQ_SROUTER(16, 8);
            else if (E <= 256) NVQ_SROUTER(16, 16);
            else if (E <= 384) NVQ_SROUTER(16, 24);
            else NVQ_SROUTER(16, 32);
        } else if (E <= 512) {
            NVQ_SROUTER(64, 8);
        } else {
            NVQ_SROUTER(64, 16);
        }
#undef NVQ_SROUTER
        NVQ_CHECK_LAUNCH();
    }
    if (route) {
        const int64_t A = T * k;
        Carver cv(ws);
        uint32_t* rw = cv.take<uint32_t>(route_ws_words(A > 0 ? A : 1, E));
        int32_t* tiles = tile_offsets ? tile_offsets : cv.take<int32_t>((size_t)E + 1);
        launch_route(topk_ids, A, E, offsets, sorted2assign, tiles, nullptr, 256, rw, s);
    }
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
