// nvq_host.hpp -- host-side helpers shared by the libnvq.so entry points:
// argument checks, workspace carving and launch-status mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nvq.h"

namespace nvq {

inline hipStream_t as_stream(nvq_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Compute units of the current device (256 if the query fails).
inline int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

// Workgroups of 256 threads of `kernel` that one CU holds at once (from its
// register and LDS use), at least 1.
inline int resident_blocks(const void* kernel) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess || n < 1) n = 1;
    return n;
}

// Bump allocator over a caller-provided workspace; every carve is 256-byte
// aligned. `need` accumulates the size so the same code answers the
// *_workspace_size() queries (with base == nullptr).
struct Carver {
    char* base;
    size_t need = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <class T>
    T* take(size_t count) {
        size_t off = need;
        need = round_up(need + count * sizeof(T), 256);
        return base ? reinterpret_cast<T*>(base + off) : nullptr;
    }
};

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? NVQ_OK : NVQ_ERR_LAUNCH;
}

#define NVQ_CHECK_LAUNCH()                       \
    do {                                         \
        int _st = ::nvq::launch_status();        \
        if (_st != NVQ_OK) return _st;           \
    } while (0)

// ---- internal launchers shared between translation units (all enqueue on
// `s`, no checks beyond what the kernels need) ----

// Zero n 32-bit words (a fill kernel rather than a memset node, so the call
// sequence stays safe to capture in a graph).
void launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);

// Workgroups per tensor of the streaming quantizer kernels (amax, encode)
// over B tensors of n8 8-value units each.
int stream_blocks(int64_t n8, int64_t B);

// Partial maxima of B tensors of n bf16 values: part[b * G + g] = max|x| over
// chunk g of tensor b (fp32 bits), G = stream_blocks(n / 8, B).
void launch_amax_bf16(const uint16_t* x, int64_t B, int64_t n, uint32_t* part, int G, hipStream_t s);

// out[0] = max of n_part partial maxima (fp32 bits).
void launch_fold_partials(const uint32_t* part, int n_part, uint32_t* out, hipStream_t s);

// NVFP4 encode of B tensors of n values each; the maximum of tensor b is
// folded from part[b * part_stride .. + n_part).
void launch_nvfp4_encode_bf16(const uint16_t* x, int64_t B, int64_t n, const uint32_t* part, int n_part,
                              int64_t part_stride, uint8_t* codes, uint8_t* scales, float* tscale, int mode,
                              uint64_t seed, uint32_t stream_id, hipStream_t s);

// Routing (stable expert sort). ws_words must hold route_ws_words(A, E) u32.
// tile_offsets [E+1] and tile_map (the expert of each of the at most
// ceil(A / tile_m) + E m-tiles) are optional.
size_t route_ws_words(int64_t A, int64_t E);
// tile_offsets [E+1] (and, if not null, the tile map) from segment offsets.
void launch_tile_offsets(const int32_t* offsets, int64_t E, int tile_m, int32_t* tile_offsets, int32_t* tile_map,
                         hipStream_t s);
void launch_route(const int32_t* topk_ids, int64_t A, int64_t E, int32_t* offsets,
                  int32_t* sorted2assign, int32_t* tile_offsets, int32_t* tile_map, int tile_m, uint32_t* ws,
                  hipStream_t s);

// 32-aligned segment starts pad[0..nseg] of the transposed, segment-padded
// layouts (pad[s+1] = pad[s] + 32 ceil(n_s / 32)); seg NULL means one
// segment [0, R). At most 4096 segments.
void launch_pad_offsets(const int32_t* seg, int64_t nseg, int64_t R, int32_t* pad, hipStream_t s);

// Rows [x, y) of every padded 32-row block of explicit segments ({0, 0} past
// the last), from pad (launch_pad_offsets): chunk_table_len(R, nseg) entries.
int64_t chunk_table_len(int64_t R, int64_t nseg);
void launch_chunk_rows(const int32_t* seg, const int32_t* pad, int64_t nseg, int64_t nchunks, int2* chunks,
                       hipStream_t s);

// NVFP4 backward dgrad on the forward's grouped GEMM (nvq_moe.hip); its m-tile
// height and the bytes of its dummy store slots.
void launch_dgrad_nvfp4(const uint8_t* ac, const uint8_t* as, const float* at, const int32_t* gather,
                        const uint8_t* bc, const uint8_t* bs, const float* bt, const int32_t* offsets,
                        const int32_t* tiles, const int32_t* tile_map, int64_t lda, int64_t ldb, int64_t E, int64_t N,
                        int64_t K, float* out, uint16_t* dummy, hipStream_t s);
int gemm_tile_m();
size_t gemm_dummy_bytes();

}  // namespace nvq
