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
// significant bits, magnitude in [2^-10, 2688]) is formed EXACTLY in fp16 in
// registers and fed to fp16 MFMA (v_mfma_f32_32x32x16_f16) with fp32
// accumulation; the two per-tensor fp32 scales are applied once in the
// epilogue. The contraction runs at the 16-bit MFMA rate and reads 4.5 bits
// per operand value.
//
// Dequantization uses gfx950's converters, both checked exhaustively on the
// device to be exact here: v_cvt_scalef32_pk_f16_fp4 with scale 1.0 turns two
// E2M1 codes into two fp16 values (it only applies the scale's exponent, so
// the E4M3 block scale cannot ride on it), and v_cvt_scalef32_pk_f16_fp8 with
// scale 1.0 turns the two E4M3 block-scale bytes of a fragment into an fp16
// pair; one packed fp16 multiply per two values applies the scale (exact).
//
// Tiling: a 256-thread workgroup owns a 256 x 128 output tile; wave w owns
// rows [64w, 64w+64) x all 128 columns (2 x 4 MFMA 32x32 blocks, 128 fp32
// accumulators); K advances 128 values per step. The two operands take
// different routes:
//  - the weight tile (128 rows, shared by all four waves) is loaded once per
//    workgroup per step (32 bytes of codes per thread; scale words four steps
//    at a time), dequantized once and stored to LDS as fp16 (32 KiB per stage,
//    two stages, 16-byte chunks placed so that both the operand reads and the
//    dequant writes are free of bank conflicts);
//  - the activation rows (distinct for every wave) go straight from L2/L1
//    into registers and are dequantized right before their MFMAs, never
//    touching LDS.
// Inside a step, lanes 0-31 cover K values [0,64) and lanes 32-63 cover
// [64,128) of it (the same permutation of K for both operands, so the sum is
// unchanged). The next step's weight stage is written one chunk per substep
// between the MFMAs, operand fragments are reloaded for later steps as soon
// as their halves die, and the per-step barrier orders LDS only, so global
// prefetch stays in flight across it. Two workgroups share a CU, so the
// waves of one cover the other's barrier and load latency, and a wave whose
// 64 rows lie past the end of its expert segment skips its MFMAs (ragged
// last tiles cost roughly in proportion to their rows). A persistent grid
// walks (expert m-tile, n-tile) tiles from device-side tile offsets (no host
// sync for the ragged segments); consecutive tiles go to workgroups on the
// same XCD so shared operand rows stay in one L2.
#include "nvq_device.hpp"
#include "nvq_host.hpp"

namespace nvq {


typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTM = 256;          // rows per tile (4 waves x 64)
constexpr int kTK = 128;          // K values per NVFP4 step (the host's divisibility unit)
constexpr int kMB = 2;            // 32-row blocks per wave
constexpr int kGemmThreads = 256;
constexpr int kMaxGemmBlocks = 1024;  // persistent grid cap; FC1 leaves 4 partial maxima per workgroup
constexpr int kDummySlots = 256;      // one 512-byte slot per wave (modulo), spread over many cache lines
constexpr int kDummySlotB = 512;
// Output columns per tile: NB 32-column blocks per wave, every wave of the
// workgroup covering all of them (NB = 8: 256 columns, one workgroup per CU;
// NB = 4: 128 columns, two per CU).
template <int NB>
constexpr int tile_n() { return NB * 32; }

// FC1: gathered A rows, SwiGLU epilogue (bf16 H); FC2: bf16 rows scattered
// to (token, slot); DG: gathered (or direct) A rows, fp32 rows in sorted
// order (the backward's dgrad).
enum { kFC1 = 0, kFC2 = 1, kDG = 2 };

// Operand formats. Both are dequantized exactly into 16-bit MFMA operands
// and both read 64 code bytes per row per K step:
//  - NVFP4: e2m1 * e4m3 (one scale per 16 values) in fp16, 128 values per
//    step in 8 substeps of 16 (v_mfma_f32_32x32x16_f16); the two tensor
//    scales are applied in the epilogue;
//  - MXFP8: e4m3 * 2^(e8m0 - 127) (one scale per 32 values) in bf16, 64
//    values per step in 4 substeps (v_mfma_f32_32x32x16_bf16); no tensor
//    scale. The scale is a power of two, so the converter applies it exactly
//    whenever the product lies in bf16's range (every block whose largest
//    magnitude is at least 2^-116: the scale exponent is then >= -124).
enum { kFmtNV = 0, kFmtMX = 1 };
template <int FMT>
constexpr int step_k() { return FMT == kFmtNV ? 128 : 64; }
template <int FMT>
constexpr int substeps() { return step_k<FMT>() / 16; }
// LDS bytes of one dequantized weight row per K step (256 or 128)
template <int FMT>
constexpr int row_bytes() { return step_k<FMT>() * 2; }

struct GemmArgs {
    const uint8_t* a_codes;      // FC1: Xq [T, K/2]; FC2: Hq [A, K/2] (MXFP8: K bytes per row)
    const uint8_t* a_scales;
    const float* a_tscale;       // NVFP4 only
    const int32_t* offsets;      // [E+1]
    const int32_t* sorted2assign;
    const int32_t* tile_offsets; // [E+1], m-tiles of kTM rows
    const int32_t* tile_map;     // expert of each m-tile
    const uint8_t* b_codes;      // [E, b_rows, K/2] (MXFP8: K bytes per row)
    const uint8_t* b_scales;
    const float* b_tscale;       // [E], NVFP4 only
    uint16_t* out;               // FC1: H [A, n_out]; FC2: y [A, n_out]
    float* out32;                // DG: [rows, n_out] fp32
    uint16_t* gu;                // FC1 only, nullable: [A, 2*n_out]
    uint32_t* amax_part;         // FC1 only, nullable: per-wave max |h| (fp32 bits), 4 per workgroup
    uint16_t* dummy;             // kDummySlots slots of kDummySlotB bytes: stores of rows past the end
    int E, K, b_rows, topk;
    uint32_t a_ld;               // code bytes per A row
    uint32_t b_ld;               // code bytes per B row
    int64_t b_estride;           // code bytes from one expert's B rows to the next's
    int n_out;                   // FC1: d_ff; FC2: d
    int n_tiles;                 // output tiles along N
};

// One lane's share of a 32-row block for one K step: 32 code bytes (64
// NVFP4 or 32 MXFP8 values).
struct Frag {
    uint4 c0, c1;
};

// Scale words of a fragment for SG consecutive K steps: word p holds the
// lane's scales of step p of the group (NVFP4: four E4M3 bytes; MXFP8: one
// E8M0 byte in the low bits).
template <int SG>
struct SWords {
    uint32_t w[SG];
};

// fp16 operand of K substep q (0..7) of a fragment: code word q, scale q / 2.
__device__ __forceinline__ half8 operand(const Frag& f, const Scales& sc, int q) {
    const uint4& c = q < 4 ? f.c0 : f.c1;
    const int w = q & 3;
    const uint32_t word = w == 0 ? c.x : w == 1 ? c.y : w == 2 ? c.z : c.w;
    const _Float16 s = q < 2 ? sc.lo[0] : q < 4 ? sc.lo[1] : q < 6 ? sc.hi[0] : sc.hi[1];
    return dq8(word, s);
}

// MXFP8 decode state of a fragment for one step: the scale 2^(e - 127) in
// the converters' form (mx_scale_f32) and the code mask (0 for a lane
// outside the operand: code 0 is +0).
struct MxScale {
    float s;
    uint32_t m;
};
__device__ __forceinline__ MxScale mx_scale(uint32_t e8m0, uint32_t msk) { return MxScale{mx_scale_f32(e8m0), msk}; }
// bf16 operand (as 16 raw bytes) of K substep q (0..3): code words 2(q & 1)
// and 2(q & 1) + 1 of half q / 2, eight E4M3 values scaled by 2^(e - 127).
__device__ __forceinline__ half8 operand_mx(const Frag& f, const MxScale& sc, int q) {
    const uint4& c = q < 2 ? f.c0 : f.c1;
    const uint2 lo = dq4_mx(((q & 1) ? c.z : c.x) & sc.m, sc.s), hi = dq4_mx(((q & 1) ? c.w : c.y) & sc.m, sc.s);
    return __builtin_bit_cast(half8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Decode state and operand of either format.
template <int FMT>
using DScale = typename std::conditional<FMT == kFmtNV, Scales, MxScale>::type;
template <int FMT>
__device__ __forceinline__ DScale<FMT> dscale(uint32_t word, uint32_t msk) {
    if constexpr (FMT == kFmtNV) return word_scales(word, msk);
    else return mx_scale(word, msk);
}
template <int FMT>
__device__ __forceinline__ half8 decode(const Frag& f, const DScale<FMT>& sc, int q) {
    if constexpr (FMT == kFmtNV) return operand(f, sc, q);
    else return operand_mx(f, sc, q);
}
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
template <int FMT>
__device__ __forceinline__ f32x16 mfma16(const half8& a, const half8& b, const f32x16& c) {
    if constexpr (FMT == kFmtNV) return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                        c, 0, 0, 0);
}

// LDS bytes of one weight stage: 32 KiB (NVFP4) or 16 KiB (MXFP8) for NB = 4
template <int FMT, int NB>
constexpr int stage_bytes() { return tile_n<NB>() * row_bytes<FMT>(); }

// Placement of the 16-byte chunks of a 256-byte LDS weight row (64 banks).
// Logical chunk 8*half + q (K values of substep q for lane half `half`) sits
// at physical chunk (2q + half) ^ key(row), key a bijection of row & 15:
//  - operand reads: 16 lanes per cycle read one logical chunk of 16
//    consecutive rows, which key spreads over all 16 chunk positions;
//  - dequant writes: 8 consecutive lanes write both halves of 4 rows, which
//    land in one 128-byte half of the banks, the next 8 lanes in the other
//    half. The write path serves that at its full rate (13 cycles per KiB on
//    gfx950, against 16 for a plain XOR with row & 15).
__device__ __forceinline__ int lds_row_key(int row) {
    return ((row & 3) << 1) | (((row >> 2) & 1) << 3) | ((row >> 3) & 1);
}
// MXFP8 rows are 128 bytes (8 chunks, two rows per bank line): key is a
// bijection of bits 1-3 of the row, which spreads both the 16-row operand
// reads and the 8-row dequant writes over all 16 chunk positions of a line.
__device__ __forceinline__ int lds_row_key_mx(int row) {
    return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}
template <int FMT>
__device__ __forceinline__ int row_key(int row) {
    return FMT == kFmtNV ? lds_row_key(row) : lds_row_key_mx(row);
}
__device__ __forceinline__ int lds_chunk(int half, int q, int key) { return (2 * q + half) ^ key; }

// Dequantize this thread's weight values of one step (64 NVFP4 or 32 MXFP8)
// into LDS row `row`, logical 16-byte chunks of half `half` (swizzled).
template <int FMT>
__device__ __forceinline__ void store_b(uint8_t* stage, int row, int half, const Frag& f, uint32_t sword,
                                        uint32_t smask) {
    const DScale<FMT> sc = dscale<FMT>(sword, smask);
    uint8_t* rp = stage + row * row_bytes<FMT>();
    const int key = row_key<FMT>(row);
#pragma unroll
    for (int q = 0; q < substeps<FMT>(); ++q)
        *reinterpret_cast<half8*>(rp + (lds_chunk(half, q, key) << 4)) = decode<FMT>(f, sc, q);
}

// Physical chunk (2q + half) ^ key = (half ^ key) ^ 2q, and the row offset
// has no bits in common with the chunk field, so every LDS address of a
// step is one per-lane base XOR (q << 5): the read base of lane (l32, h)
// serves rows j * 32 + l32 (same key; their offset j * 8192 is an
// immediate), the store base serves staging thread (br, hb). Bases pass
// through an opaque move once per step so the 16 derived offsets are
// recomputed (one XOR each) rather than held in registers across the loop.
template <int FMT>
__device__ __forceinline__ uint32_t lds_base(int row, int half) {
    return (uint32_t)(row * row_bytes<FMT>() + ((half ^ row_key<FMT>(row)) << 4));
}
// 16-bit operand of K substep q for weight row j * 32 + l32.
template <int FMT>
__device__ __forceinline__ half8 read_b_at(const uint8_t* stage, uint32_t rbase, int j, int q) {
    return *reinterpret_cast<const half8*>(stage + j * 32 * row_bytes<FMT>() + (rbase ^ ((uint32_t)q << 5)));
}

// Workgroup barrier that orders LDS accesses only: global loads still in
// flight (operand prefetch for later K steps) are not waited for, unlike
// __syncthreads(), whose fence covers global memory too.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One lane's share of a 32-row block for one K step lives at codes cbase +
// off (32 bytes) and scales sbase + off / 8 (NVFP4: a row of K/2 code bytes
// has K/16 scale bytes) or sbase + off / 32 (MXFP8: K code bytes, K/32
// scale bytes); lane offsets are multiples of 32 bytes. Loads never branch:
// a lane outside the operand reads a valid row and its values are masked to
// zero when they are decoded.
// Fragment halves: codes c0 feed the first half of the substeps, c1 the
// second. Each half is reloaded for a later K step as soon as it is dead, so
// one register set per operand serves as its own prefetch buffer.
__device__ __forceinline__ void load_lo(Frag& f, const uint8_t* cbase, uint32_t off) {
    f.c0 = *reinterpret_cast<const uint4*>(cbase + off);
}
__device__ __forceinline__ void load_hi(Frag& f, const uint8_t* cbase, uint32_t off) {
    f.c1 = *(reinterpret_cast<const uint4*>(cbase + off) + 1);
}
// Scale word of one K step (NVFP4: 4 bytes per lane and step; MXFP8: 1).
template <int FMT>
__device__ __forceinline__ void load_word(uint32_t& w, const uint8_t* sbase, uint32_t off) {
    if constexpr (FMT == kFmtNV) w = *reinterpret_cast<const uint32_t*>(sbase + (off >> 3));
    else w = sbase[off >> 5];
}
// Scale words of four K steps with one 16-byte load per lane. A 4-byte word
// per lane and step would touch one cache line per row for 4 bytes, every
// step, and the L1 does not keep those lines from one step to the next. The
// 32 bytes of a row's group (steps g..g+3, both K halves) are split between
// the two lanes that share the row: the half-0 lane loads steps g and g+1,
// the half-1 lane steps g+2 and g+3; the exchange below hands each lane its
// own half of every step. MXFP8: a row's group is 8 bytes (step g + p,
// half h at byte 2p + h), which both lanes of the row load whole.
// off: code offset of the lane's fragment in the group's first step.
template <int FMT>
__device__ __forceinline__ void load_group(SWords<4>& s, const uint8_t* sbase, uint32_t off, int h) {
    if constexpr (FMT == kFmtNV) {
        const uint4 v = *reinterpret_cast<const uint4*>(sbase + ((off >> 3) + 12u * (uint32_t)h));
        s.w[0] = v.x; s.w[1] = v.y; s.w[2] = v.z; s.w[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(sbase + ((off >> 5) & ~7u));
        s.w[0] = v.x; s.w[1] = v.y;
    }
}
// MXFP8: word p becomes this lane's scale byte of step g + p (low bits).
__device__ __forceinline__ void group_to_steps_mx(SWords<4>& s, int h) {
    const uint32_t sh = 8u * (uint32_t)h, x = s.w[0], y = s.w[1];
    s.w[0] = x >> sh;
    s.w[1] = x >> (16u + sh);
    s.w[2] = y >> sh;
    s.w[3] = y >> (16u + sh);
}
// Activation fragments: the two lanes of a row are l and l + 32. After the
// exchange word p is this lane's half of step g + p.
__device__ __forceinline__ void group_to_steps_a(SWords<4>& s) {
    const auto r01 = __builtin_amdgcn_permlane32_swap(s.w[0], s.w[1], false, false);  // steps g, g+2
    const auto r23 = __builtin_amdgcn_permlane32_swap(s.w[2], s.w[3], false, false);  // steps g+1, g+3
    s.w[0] = r01[0]; s.w[1] = r23[0]; s.w[2] = r01[1]; s.w[3] = r23[1];
}
// Weight fragments: the two lanes of a row are adjacent (half = lane & 1).
__device__ __forceinline__ uint32_t pair_swap(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ void group_to_steps_b(SWords<4>& s, bool half1) {
    const uint32_t w0 = s.w[0], w1 = s.w[1], w2 = s.w[2], w3 = s.w[3];
    const uint32_t r0 = pair_swap(half1 ? w0 : w1);  // half 0 receives step g+2, half 1 step g
    const uint32_t r1 = pair_swap(half1 ? w2 : w3);  // half 0 receives step g+3, half 1 step g+1
    s.w[0] = half1 ? r0 : w0;
    s.w[1] = half1 ? r1 : w2;
    s.w[2] = half1 ? w1 : r0;
    s.w[3] = half1 ? w3 : r1;
}

// Operand addressing of one wave for one tile. Element pointers are wave-
// uniform (the expert's weight matrix, the activation tensor); the lane
// offsets stay below 2^32 (host-checked), so loads take a scalar base and a
// 32-bit vector offset.
// A thread stages NF = NB / 4 weight half-rows per K step: tile rows
// br + 128 f (f < NF), K half hb.
template <int NB>
struct WaveOps {
    static constexpr int NF = NB / 4;
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    uint32_t a_off[kMB];
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    uint32_t b_off[NF];
};

// One K step of one wave. A wave with NA active 32-row blocks (0-2) runs 8
// substeps x (NA x NB) MFMAs on the current LDS stage, loading and decoding
// only those blocks' activations; every wave also dequantizes its weight
// fragments of the next step into the other stage (one 16-byte chunk per
// fragment and substep) and issues the global loads of later steps as fragment halves
// die: activations of step +1 (NL blocks at oa + ka), weights of step +2
// (at ob + kb). oa and ob are the current tile's addressing except in the
// last steps of a tile, where the look-ahead continues into the next tile
// (NL is then all blocks, whatever NA is); a_msk always belongs to the
// current tile. The weight reads and activation decode of substep q+1 are
// issued during substep q, and the schedule groups put VALU, LDS and memory
// instructions between the MFMAs so one wave keeps the matrix pipe fed while
// its own non-matrix work proceeds.
// Scale words: SG = 1 loads each step's word with the step's codes. SG = 4
// keeps a group of four steps per fragment; PA is this step's position in
// the activation group and PB the position of the staged weight step in the
// weight group (the weights run one step ahead). The next group is loaded
// when the last word of the current one has been used (code offsets ga, gb
// of its first step) and reordered when its first step begins.
template <int FMT, int NB, int NA, int NL, int SG, int PA, int PB>
__device__ __forceinline__ void k_step(f32x16 (&acc)[kMB][NB], Frag (&fa)[kMB], SWords<SG> (&swa)[kMB],
                                       Frag (&fb)[NB / 4], SWords<SG> (&swb)[NB / 4], const uint8_t* cur,
                                       uint8_t* nxt, int l32, int h, int br, int hb, const uint32_t (&a_msk)[kMB],
                                       const WaveOps<NB>& oa, const WaveOps<NB>& ob, uint32_t ka, uint32_t kb,
                                       uint32_t ga, uint32_t gb) {
    constexpr int NF = NB / 4;
    constexpr int QS = substeps<FMT>();
    uint32_t rbase = lds_base<FMT>(l32, h), sbase = lds_base<FMT>(br, hb);
    asm volatile("" : "+v"(rbase), "+v"(sbase));
    DScale<FMT> sa[kMB];
    half8 bcur[NB], av[kMB];
    if (NA > 0) {
        if constexpr (SG > 1 && PA == 0) {
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                if constexpr (FMT == kFmtNV) group_to_steps_a(swa[i]);
                else group_to_steps_mx(swa[i], h);
            }
        }
#pragma unroll
        for (int i = 0; i < NA; ++i) sa[i] = dscale<FMT>(swa[i].w[PA], a_msk[i]);
#pragma unroll
        for (int j = 0; j < NB; ++j) bcur[j] = read_b_at<FMT>(cur, rbase, j, 0);
#pragma unroll
        for (int i = 0; i < NA; ++i) av[i] = decode<FMT>(fa[i], sa[i], 0);
    }
    DScale<FMT> sb[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        if constexpr (SG > 1 && PB == 0) {
            if constexpr (FMT == kFmtNV) group_to_steps_b(swb[f], hb != 0);
            else group_to_steps_mx(swb[f], hb);
        }
        sb[f] = dscale<FMT>(swb[f].w[PB], 0xFFFFFFFFu);
    }
#pragma unroll
    for (int q = 0; q < QS; ++q) {
        half8 bnxt[NB], avn[kMB];
        if (NA > 0 && q < QS - 1) {
            // The weight reads of substep q+1 go out before any MFMA of q and
            // nothing may be scheduled across them: left to itself, the
            // scheduler sinks each read next to its MFMA to save registers,
            // and the LDS latency then stalls the wave on every MFMA pair.
#pragma unroll
            for (int j = 0; j < NB; ++j) bnxt[j] = read_b_at<FMT>(cur, rbase, j, q + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NA; ++i) avn[i] = decode<FMT>(fa[i], sa[i], q + 1);
        }
        // staged rows br + 128 f: the same swizzle key, 128 rows further on
#pragma unroll
        for (int f = 0; f < NF; ++f)
            *reinterpret_cast<half8*>(nxt + f * 128 * row_bytes<FMT>() + (sbase ^ ((uint32_t)q << 5))) =
                decode<FMT>(fb[f], sb[f], q);
        if (q == QS / 2 - 1) {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                load_lo(fa[i], oa.a_codes, oa.a_off[i] + ka);
                if constexpr (SG == 1) load_word<FMT>(swa[i].w[0], oa.a_scales, oa.a_off[i] + ka);
                if constexpr (SG > 1 && PA == SG - 1) load_group<FMT>(swa[i], oa.a_scales, oa.a_off[i] + ga, h);
            }
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                load_lo(fb[f], ob.b_codes, ob.b_off[f] + kb);
                if constexpr (SG == 1) load_word<FMT>(swb[f].w[0], ob.b_scales, ob.b_off[f] + kb);
                if constexpr (SG > 1 && PB == SG - 1) load_group<FMT>(swb[f], ob.b_scales, ob.b_off[f] + gb, hb);
            }
        }
        if (q == QS - 1) {
#pragma unroll
            for (int i = 0; i < NL; ++i) load_hi(fa[i], oa.a_codes, oa.a_off[i] + ka);
#pragma unroll
            for (int f = 0; f < NF; ++f) load_hi(fb[f], ob.b_codes, ob.b_off[f] + kb);
        }
        if (NA > 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < NA; ++i)
                    acc[i][j] = mfma16<FMT>(av[i], bcur[j], acc[i][j]);
            // MFMA, up to 6 VALU, then the LDS write(s) or the memory loads. A
            // substep has about 30 VALU instructions, so this front-loads the
            // decode of the next substep into the first MFMA slots (measured:
            // 6 beats 3, 4, 5, 8 and 12 by 2-4 %).
#pragma unroll
            for (int t = 0; t < 2 * NB; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                if (t == 4 || t == 8) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                if (t == 5) __builtin_amdgcn_sched_group_barrier(0x020, NB == 4 ? 6 : 8, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (q < QS - 1) {
#pragma unroll
                for (int j = 0; j < NB; ++j) bcur[j] = bnxt[j];
#pragma unroll
                for (int i = 0; i < NA; ++i) av[i] = avn[i];
            }
        }
    }
}

// a, b: fp32 values of rows r and r + 1 in this lane's column. Returns the
// word this lane stores: the even lane's row r (its column, then the odd
// neighbour's), the odd lane's row r + 1 (the even neighbour's column, then
// its own), low half first. Rounding to bf16 is nearest-even by the gfx950
// pair converter (v_cvt_pk_bf16_f32; for finite values the same bits as
// f32_to_bf16). sel is pair_sel(odd). Must be called by all lanes of the wave.
__device__ __forceinline__ uint32_t pair_sel(bool odd) { return odd ? 0x03020706u : 0x05040100u; }
__device__ __forceinline__ uint32_t pair_rows_bf16(float a, float b, uint32_t sel) {
    const uint32_t own = bf16x2_rne(a, b);
    const uint32_t nbr = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, true);
    // bytes 0-3 select from own, 4-7 from nbr: even [own.lo | nbr.lo], odd [nbr.hi | own.hi]
    return __builtin_amdgcn_perm(nbr, own, sel);
}

// Tile tables and tensor scales are read through constant-address-space
// pointers: nothing in the kernel writes them, and at wave-uniform indices
// that makes them scalar loads. Read after a barrier, a plain load would be a
// vector load, and a vector load waits for every vector memory operation
// issued before it (the operand look-ahead and the output stores).
template <typename T>
__device__ __forceinline__ T cload(const T* base, int64_t i) {
    typedef const __attribute__((address_space(4))) T ct;
    return ((ct*)base)[i];
}

// One wave's view of an output tile (all wave-uniform).
struct NTile {
    int e, nt, row0, row_end;  // expert, n-tile, first row of the wave, end of the expert's rows
};

// Divisors pass through an opaque move: the reciprocal behind a division is
// then formed per tile instead of being hoisted out of the tile loop, where it
// would hold a vector register for the whole kernel.
__device__ __forceinline__ NTile tile_at(const GemmArgs& p, int t, int wave) {
    NTile T;
    int n_tiles = p.n_tiles;
    asm volatile("" : "+s"(n_tiles));
    const int mt = t / n_tiles;
    T.nt = t % n_tiles;
    T.e = cload(p.tile_map, mt);  // one scalar load rather than a search over tile_offsets
    T.row0 = cload(p.offsets, T.e) + (mt - cload(p.tile_offsets, T.e)) * kTM + wave * 64;
    T.row_end = cload(p.offsets, T.e + 1);
    return T;
}

// Source rows of this lane in the wave's two 32-row blocks: FC1 reads the
// token of each expert-sorted row (unconditionally, at row 0 past the end, so
// no branch separates the load from its use), FC2 uses the row itself.
template <int MODE>
__device__ __forceinline__ void row_src(const GemmArgs& p, const NTile& T, int l32, int32_t (&src)[kMB]) {
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        const int r = T.row0 + i * 32 + l32;
        if (MODE == kFC1) src[i] = p.sorted2assign[r < T.row_end ? r : 0];
        else if (MODE == kDG) src[i] = p.sorted2assign ? p.sorted2assign[r < T.row_end ? r : 0] : r;
        else src[i] = r;
    }
}

// Operand addressing and decode masks of tile T for lane tid (inactive lanes
// read row 0, their scales masked to zero at decode). Every column block of
// every tile exists: n_out is a multiple of the tile's columns (FC1: of half
// of them; host-checked).
template <int FMT, int MODE, int NB>
__device__ __forceinline__ void tile_ops(const GemmArgs& p, const NTile& T, const int32_t (&src)[kMB], int tid,
                                         WaveOps<NB>& o, uint32_t (&a_msk)[kMB]) {
    constexpr int TN = tile_n<NB>();
    const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const uint32_t a_ld = p.a_ld;
    int topk = p.topk;  // opaque, as in tile_at
    asm volatile("" : "+s"(topk));
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        const bool ok = T.row0 + i * 32 + l32 < T.row_end;
        const uint32_t s = MODE == kFC1 ? (uint32_t)src[i] / (uint32_t)topk : (uint32_t)src[i];
        o.a_off[i] = (ok ? s : 0u) * a_ld + (uint32_t)h * 32;
        a_msk[i] = ok ? 0xFFFFFFFFu : 0u;
    }
    // weight rows loaded by this thread: tile rows br + 128 f, K half hb
    const int hb = tid & 1;
    const int64_t e_off = (int64_t)T.e * p.b_estride;
    o.a_codes = p.a_codes;
    o.a_scales = p.a_scales;
    o.b_codes = p.b_codes + e_off;
    o.b_scales = p.b_scales + e_off / (FMT == kFmtNV ? 8 : 32);
#pragma unroll
    for (int f = 0; f < NB / 4; ++f) {
        const int br = (tid >> 1) + 128 * f;
        int wrow;
        if (MODE == kFC1) {
            // tile columns: [gate j0..+31 | up j0..+31 | gate j0+32.. | up ..], j0 = (TN / 2) nt
            const int blk = br >> 5;
            wrow = ((blk & 1) ? p.n_out : 0) + T.nt * (TN / 2) + (blk >> 1) * 32 + (br & 31);
        } else {
            wrow = T.nt * TN + br;
        }
        o.b_off[f] = (uint32_t)wrow * p.b_ld + (uint32_t)hb * 32;
    }
}

// First tile of a workgroup: step 0 of both operands, weights of step 0 into
// stage 0, weights of step k1 in flight. The loads that stay in flight into
// the loop are issued in the order the loop body issues them (low halves,
// then high halves last): the waits at the loop head are derived from both
// this order and the loop's own, and high halves issued early here would
// make every step wait for the high halves its previous step issued just
// before the barrier.
template <int FMT, int NB, int SG>
__device__ __forceinline__ void prologue(Frag (&fa)[kMB], SWords<SG> (&swa)[kMB], Frag (&fb)[NB / 4],
                                         SWords<SG> (&swb)[NB / 4], uint8_t* stage0, int br, int hb, int h,
                                         const WaveOps<NB>& o, uint32_t k1) {
    constexpr int NF = NB / 4;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        load_lo(fb[f], o.b_codes, o.b_off[f]);
        load_hi(fb[f], o.b_codes, o.b_off[f]);
        if constexpr (SG == 1) {
            load_word<FMT>(swb[f].w[0], o.b_scales, o.b_off[f]);
        } else {
            load_group<FMT>(swb[f], o.b_scales, o.b_off[f], hb);
            if constexpr (FMT == kFmtNV) group_to_steps_b(swb[f], hb != 0);
            else group_to_steps_mx(swb[f], hb);
        }
        store_b<FMT>(stage0, br + 128 * f, hb, fb[f], swb[f].w[0], 0xFFFFFFFFu);
    }
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        load_lo(fa[i], o.a_codes, o.a_off[i]);
        if constexpr (SG == 1) load_word<FMT>(swa[i].w[0], o.a_scales, o.a_off[i]);
        else load_group<FMT>(swa[i], o.a_scales, o.a_off[i], h);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        load_lo(fb[f], o.b_codes, o.b_off[f] + k1);
        if constexpr (SG == 1) load_word<FMT>(swb[f].w[0], o.b_scales, o.b_off[f] + k1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kMB; ++i) load_hi(fa[i], o.a_codes, o.a_off[i]);
#pragma unroll
    for (int f = 0; f < NF; ++f) load_hi(fb[f], o.b_codes, o.b_off[f] + k1);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
}

// a if ok else b, computed without a branch (left alone, the compiler guards
// the address arithmetic of a with the condition, a branch per row). The
// result is typed as a global pointer: through the opaque move the compiler
// would no longer know it, and stores through a generic pointer are flat
// stores, which also count against the LDS wait counter.
typedef __attribute__((address_space(1))) uint16_t g_u16;
typedef __attribute__((address_space(1))) uint32_t g_u32;
__device__ __forceinline__ g_u16* pick(bool ok, uint16_t* a, uint16_t* b) {
    asm volatile("" : "+v"(a));
    return ok ? (g_u16*)a : (g_u16*)b;
}
typedef __attribute__((address_space(1))) float g_f32;
__device__ __forceinline__ g_f32* pick_f32(bool ok, float* a, float* b) {
    asm volatile("" : "+v"(a));
    return ok ? (g_f32*)a : (g_f32*)b;
}

// Epilogue of tile T (lane l, register r of a 32x32 block: column l % 32,
// row 8 (r / 4) + 4 (l / 32) + r % 4). Lanes l and l ^ 1 hold adjacent
// columns: they exchange their bf16 pairs of rows r, r + 1 so the even lane
// writes row r and the odd lane row r + 1, two adjacent bf16 columns each,
// as one 32-bit store. Nothing here branches: a row past the end of the expert's
// rows is written to the wave's dummy slot instead, so the stores never sit
// between the operand look-ahead loads and their waits on one path only.
// FC2: rs is sorted2assign of row T.row0 + lane (any valid index past the
// end); each lane fetches the destinations of its rows from the lane that
// holds them.
template <int MODE, int NB, bool GU>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const f32x16 (&acc)[kMB][NB], const NTile& T,
                                         float scale, int32_t rs, uint16_t* dslot, int lane, uint32_t& h_max) {
    constexpr int TN = tile_n<NB>();
    const int l32 = lane & 31, h = lane >> 5;
    const bool odd = (lane & 1) != 0;
    const uint32_t sel = pair_sel(odd);
    const int rl = h * 4 + (odd ? 1 : 0);  // lane part of the row of register pair r
    const int cl = l32 & ~1;               // first of the two columns this lane writes
    if (MODE == kFC1) {
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int row = T.row0 + i * 32 + (r >> 2) * 8 + (r & 3) + rl;
                const bool ok = row < T.row_end;
                const int64_t col = (int64_t)T.nt * (TN / 2) + cl;
                g_u16* hp = pick(ok, p.out + (int64_t)row * p.n_out + col, dslot + cl);
                g_u16* gp = (g_u16*)(dslot + cl);
                g_u16* up = gp;
                if (GU) {
                    gp = pick(ok, p.gu + (int64_t)row * 2 * p.n_out + col, dslot + cl);
                    up = pick(ok, p.gu + (int64_t)row * 2 * p.n_out + p.n_out + col, dslot + cl);
                }
#pragma unroll
                for (int pj = 0; pj < NB / 2; ++pj) {
                    float hv[2], gv[2], uv[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        gv[t] = acc[i][2 * pj][r + t] * scale;
                        uv[t] = acc[i][2 * pj + 1][r + t] * scale;
                        hv[t] = gv[t] * uv[t] * __builtin_amdgcn_rcpf(1.0f + __expf(-gv[t]));
                    }
                    const uint32_t wh = pair_rows_bf16(hv[0], hv[1], sel);
                    *(g_u32*)(hp + pj * 32) = wh;
                    const uint32_t m = max(wh & 0x7FFFu, (wh >> 16) & 0x7FFFu);
                    h_max = max(h_max, ok ? m : 0u);
                    if (GU) {
                        *(g_u32*)(gp + pj * 32) = pair_rows_bf16(gv[0], gv[1], sel);
                        *(g_u32*)(up + pj * 32) = pair_rows_bf16(uv[0], uv[1], sel);
                    }
                }
            }
        }
    } else if (MODE == kDG) {
        // fp32 rows in sorted order: each lane stores its own column of rows
        // r and r + 1 (two 128-byte row pieces per store instruction)
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = T.row0 + i * 32 + (r >> 2) * 8 + (r & 3) + h * 4;
                const bool ok = row < T.row_end;
                g_f32* op = pick_f32(ok, p.out32 + (int64_t)row * p.n_out + (int64_t)T.nt * TN + l32,
                                     reinterpret_cast<float*>(dslot) + l32);
#pragma unroll
                for (int j = 0; j < NB; ++j) op[j * 32] = acc[i][j][r] * scale;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int ro = i * 32 + (r >> 2) * 8 + (r & 3) + rl;  // row within the wave's 64
                const int32_t dst = __builtin_amdgcn_ds_bpermute(ro << 2, rs);
                const bool ok = T.row0 + ro < T.row_end;
                g_u16* yp = pick(ok, p.out + (int64_t)dst * p.n_out + (int64_t)T.nt * TN + cl, dslot + cl);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    *(g_u32*)(yp + j * 32) = pair_rows_bf16(acc[i][j][r] * scale, acc[i][j][r + 1] * scale, sel);
            }
        }
    }
}

// FC2 epilogue through LDS (NVFP4, 128-column tiles, streamed K): each 32-row
// block of the wave's 64 rows is written as bf16 pairs (the pair exchange
// above) into the wave's 8 KiB of the weight stage the tile's last step read
// (free until the next tile's first step stages into it, after a barrier),
// then read back as 16-byte row pieces: each store instruction then covers
// four whole 256-byte row pieces, 16 store instructions per wave instead of
// 64 four-byte ones. 16-byte chunk c of row r sits at chunk c ^ 4 g(r),
// g(r) = (r & 1) | ((r >> 1) & 2): the four rows of one pair write (r, r + 1,
// r + 4, r + 5) land in four different 64-byte bank groups, and each eight-
// lane group of a read covers eight different chunks of one row.
template <int NB>
__device__ __forceinline__ void epilogue_fc2_lds(const GemmArgs& p, const f32x16 (&acc)[kMB][NB], const NTile& T,
                                                 float scale, int32_t rs, uint16_t* dslot, int lane,
                                                 uint8_t* ebuf) {
    static_assert(NB == 4, "one 32-row block of 128 bf16 columns per 8 KiB");
    constexpr int TN = tile_n<NB>();
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) u32x4 g_u4;
    const int l32 = lane & 31, h = lane >> 5;
    const bool odd = (lane & 1) != 0;
    const uint32_t sel = pair_sel(odd);
    const int rl = h * 4 + (odd ? 1 : 0);
    const int cl = l32 & ~1;
    const int cc = lane & 15;
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int row = (r >> 2) * 8 + (r & 3) + rl;
            const int g = (row & 1) | ((row >> 1) & 2);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const uint32_t v = pair_rows_bf16(acc[i][j][r] * scale, acc[i][j][r + 1] * scale, sel);
                const int off = row * 256 + (((4 * j + (cl >> 3)) ^ (4 * g)) << 4) + ((cl * 2) & 15);
                *reinterpret_cast<uint32_t*>(ebuf + off) = v;
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int row = 4 * k + (lane >> 4);
            const int g = (row & 1) | ((row >> 1) & 2);
            const u32x4 val = *reinterpret_cast<const u32x4*>(ebuf + row * 256 + ((cc ^ (4 * g)) << 4));
            const int ro = i * 32 + row;
            const int32_t dst = __builtin_amdgcn_ds_bpermute(ro << 2, rs);
            const bool ok = T.row0 + ro < T.row_end;
            g_u16* yp = pick(ok, p.out + (int64_t)dst * p.n_out + (int64_t)T.nt * TN + cc * 8, dslot + cc * 8);
            *(g_u4*)yp = val;
        }
    }
}

// Grouped NVFP4 GEMM over expert segments, persistent over (m-tile, n-tile)
// pairs. With SG = 4 (K a multiple of 512) the K steps of consecutive tiles
// of a workgroup form one stream: the look-ahead loads of a tile's last two
// steps fetch the next tile's first steps, and its last step stages the next
// tile's first weight stage, so a tile costs its epilogue and no prologue.
// With SG = 1 each tile has its own prologue.
template <int FMT, int MODE, int NB, int SG, bool GU>
__global__ __launch_bounds__(kGemmThreads, NB == 8 ? 1 : 2) void k_grouped_gemm_dq(GemmArgs p) {
    constexpr int NF = NB / 4;
    constexpr uint32_t kStepB = 64;  // code bytes per row per K step
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][stage_bytes<FMT, NB>()];
    // wave index as a scalar: everything derived from it (rows, the active
    // test) is then known to be wave-uniform and branches on it are scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int total = cload(p.tile_offsets, p.E) * p.n_tiles;  // < 2^31 (host-checked)
    const int G = gridDim.x;
    uint32_t h_max = 0;  // FC1: running max |h| (bf16 magnitude bits) of this lane
    // consecutive virtual ids on one XCD (workgroups are dealt to the 8 XCDs round robin)
    const int v = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
    const int nk = p.K / step_k<FMT>();
    const uint32_t k_last = (uint32_t)(nk - 1) * kStepB;
    uint16_t* dslot = p.dummy + (size_t)((blockIdx.x * 4 + wave) % kDummySlots) * (kDummySlotB / 2);
    // The lane index is re-derived per tile through an opaque move: lane-
    // dependent address math would otherwise be hoisted out of the tile loop
    // and pin registers for the whole kernel.
#define NVQ_TID(name)                      \
    int name = (int)threadIdx.x;           \
    asm volatile("" : "+v"(name));
    f32x16 acc[kMB][NB];
    Frag fb[NF], fa[kMB];
    SWords<SG> swb[NF], swa[kMB];
#define NVQ_ZERO_ACC                                      \
    _Pragma("unroll") for (int i = 0; i < kMB; ++i)       \
        _Pragma("unroll") for (int j = 0; j < NB; ++j)    \
            _Pragma("unroll") for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if constexpr (SG == 1) {
        for (int t = v; t < total; t += G) {
            NVQ_TID(tid)
            const int lane = tid & 63, l32 = lane & 31, h = lane >> 5, br = tid >> 1, hb = tid & 1;
            const NTile T = tile_at(p, t, wave);
            int32_t src[kMB];
            row_src<MODE>(p, T, l32, src);
            WaveOps<NB> o;
            uint32_t a_msk[kMB];
            tile_ops<FMT, MODE, NB>(p, T, src, tid, o, a_msk);
            // active 32-row blocks of this wave (wave-uniform): MFMAs, activation
            // loads and decodes of a block that lies wholly past the segment are
            // skipped, so ragged segments cost rows in 32-row rather than 64-row
            // granularity
            const int na = T.row0 >= T.row_end ? 0 : T.row0 + 32 >= T.row_end ? 1 : 2;
            NVQ_ZERO_ACC
            prologue<FMT, NB, SG>(fa, swa, fb, swb, lds[0], br, hb, h, o, min(kStepB, k_last));
            // Two separate loops rather than a branch inside one: with the
            // branch inside, the weight decode common to both paths is hoisted
            // above it and its 32 results stay live across the whole step,
            // which leaves no registers for reading the next substep's weights
            // ahead of use. Look-ahead offsets are clamped to the last step, so
            // loads never branch (a clamped reload is never used).
#define NVQ_LOOP1(NACT)                                                                                         \
    for (int step = 0; step < nk; ++step) {                                                                     \
        const uint32_t sa1 = (uint32_t)(step + 1) * kStepB, sb2 = (uint32_t)(step + 2) * kStepB;                 \
        k_step<FMT, NB, NACT, NACT, SG, 0, 0>(acc, fa, swa, fb, swb, lds[step & 1], lds[(step + 1) & 1], l32, h, br, hb,  \
                                     a_msk, o, o, NACT ? min(sa1, k_last) : 0u, min(sb2, k_last), 0u, 0u);      \
        lds_barrier();                                                                                          \
    }
            if (na == 0) {
                NVQ_LOOP1(0)
                continue;
            }
            if (na == 1) {
                NVQ_LOOP1(1)
            } else {
                NVQ_LOOP1(2)
            }
#undef NVQ_LOOP1
            const float scale = FMT == kFmtNV ? cload(p.a_tscale, 0) * cload(p.b_tscale, T.e) : 1.0f;
            int32_t rs = 0;
            if (MODE == kFC2) rs = p.sorted2assign[T.row0 + lane < T.row_end ? T.row0 + lane : 0];
            epilogue<MODE, NB, GU>(p, acc, T, scale, rs, dslot, lane, h_max);
        }
    } else if (v < total) {
        // K steps stream in groups of four, so a tile's last step reads stage
        // 1 and stages the next tile's first step into stage 0
        constexpr bool kLdsEpi = MODE == kFC2 && FMT == kFmtNV && NB == 4 && stage_bytes<FMT, NB>() == 4 * 8192;
        // the workgroup's first tile
        NTile T;
        WaveOps<NB> o;
        uint32_t a_msk[kMB];
        {
            NVQ_TID(tid)
            const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
            T = tile_at(p, v, wave);
            int32_t src[kMB];
            row_src<MODE>(p, T, l32, src);
            tile_ops<FMT, MODE, NB>(p, T, src, tid, o, a_msk);
            prologue<FMT, NB, SG>(fa, swa, fb, swb, lds[0], tid >> 1, tid & 1, h, o, kStepB);
        }
        for (int t = v;;) {
            const int tn = t + G;
            const bool more = tn < total;
            // the next tile (past the last one: this tile again, whose loads are
            // valid and never used); its scalars are waited for here, before
            // the K loop, where a pending scalar load would turn the loop's
            // LDS waits into full drains
            const NTile N = tile_at(p, more ? tn : t, wave);
            const float scale = FMT == kFmtNV ? cload(p.a_tscale, 0) * cload(p.b_tscale, T.e) : 1.0f;
            asm volatile("" ::"s"(N.e), "s"(N.row0), "s"(N.row_end), "s"(scale));
            const int na = T.row0 >= T.row_end ? 0 : T.row0 + 32 >= T.row_end ? 1 : 2;
            NVQ_ZERO_ACC
            WaveOps<NB> on;
            uint32_t n_msk[kMB];
            int32_t rs = 0;
            // Steps 0 .. nk-5 in groups of four; then the last group, whose
            // look-ahead crosses into tile N: the weights of steps nk and
            // nk+1 (N's steps 0 and 1, with N's first scale group) from the
            // step before last, N's activations of step 0 and scale group
            // from the last step, which also stages N's step 0 weights.
            // The epilogue follows in the same branch: at the join after the
            // three variants the compiler moves the look-ahead fragments
            // between registers, and each such copy waits for its load, so a
            // join before the epilogue would stall it on the loads it should
            // overlap. A wave with no rows has nothing to store.
#define NVQ_SSTEP(NACT, NLD, PH, OA, OB, KA, KB, G_A, G_B)                                                        \
    {                                                                                                           \
        k_step<FMT, NB, NACT, NLD, SG, (PH), ((PH) + 1) & (SG - 1)>(acc, fa, swa, fb, swb, lds[((PH) + step) & 1],        \
                                                         lds[((PH) + step + 1) & 1], l32, h, br, hb, a_msk, OA, \
                                                         OB, KA, KB, G_A, G_B);                                 \
        lds_barrier();                                                                                          \
    }
#define NVQ_STREAM(NACT)                                                                                        \
    {                                                                                                           \
        for (int step = 0; step < nk - 4; step += 4) {                                                          \
            NVQ_TID(tid)                                                                                        \
            const int l32 = tid & 31, h = (tid >> 5) & 1, br = tid >> 1, hb = tid & 1;                          \
            const uint32_t s1 = (uint32_t)(step + 1) * kStepB;                                                  \
            NVQ_SSTEP(NACT, NACT, 0, o, o, s1, s1 + 64u, 0u, 0u)                                                \
            NVQ_SSTEP(NACT, NACT, 1, o, o, s1 + 64u, s1 + 128u, 0u, 0u)                                         \
            NVQ_SSTEP(NACT, NACT, 2, o, o, s1 + 128u, s1 + 192u, 0u, s1 + 192u)                                 \
            NVQ_SSTEP(NACT, NACT, 3, o, o, s1 + 192u, s1 + 256u, s1 + 192u, 0u)                                 \
        }                                                                                                       \
        {                                                                                                       \
            const int step = nk - 4;                                                                            \
            NVQ_TID(tid)                                                                                        \
            const int lane = tid & 63, l32 = lane & 31, h = lane >> 5, br = tid >> 1, hb = tid & 1;             \
            int32_t nsrc[kMB];                                                                                  \
            row_src<MODE>(p, N, l32, nsrc);                                                                     \
            if (MODE == kFC2) rs = p.sorted2assign[T.row0 + lane < T.row_end ? T.row0 + lane : 0];              \
            const uint32_t s1 = (uint32_t)(step + 1) * kStepB;                                                  \
            NVQ_SSTEP(NACT, NACT, 0, o, o, s1, s1 + 64u, 0u, 0u)                                                \
            NVQ_SSTEP(NACT, NACT, 1, o, o, s1 + 64u, s1 + 128u, 0u, 0u)                                         \
            tile_ops<FMT, MODE, NB>(p, N, nsrc, tid, on, n_msk);                                                         \
            NVQ_SSTEP(NACT, NACT, 2, o, on, s1 + 128u, 0u, 0u, 0u)                                              \
            {                                                                                                   \
                /* N's activation offsets again, behind a fresh opaque lane index, so that   */               \
                /* they are formed here and not held (or spilled) across the step before      */               \
                NVQ_TID(tid3)                                                                                   \
                if (MODE == kFC2) row_src<MODE>(p, N, tid3 & 31, nsrc);                                         \
                tile_ops<FMT, MODE, NB>(p, N, nsrc, tid3, on, n_msk);                                                    \
            }                                                                                                   \
            NVQ_SSTEP(NACT, kMB, 3, on, on, 0u, 64u, 0u, 0u)                                                    \
            if (NACT > 0) {                                                                                     \
                if constexpr (kLdsEpi)                                                                          \
                    epilogue_fc2_lds<NB>(p, acc, T, scale, rs, dslot, lane, lds[1] + wave * 8192);              \
                else                                                                                            \
                    epilogue<MODE, NB, GU>(p, acc, T, scale, rs, dslot, lane, h_max);                           \
            }                                                                                                   \
        }                                                                                                       \
    }
            if (na == 0) {
                NVQ_STREAM(0)
            } else if (na == 1) {
                NVQ_STREAM(1)
            } else {
                NVQ_STREAM(2)
            }
#undef NVQ_STREAM
#undef NVQ_SSTEP
            // the next tile's first step stages weights into the LDS stage
            // the FC2 epilogue used
            if constexpr (kLdsEpi) lds_barrier();
            if (!more) break;
            T = N;
            o = on;
#pragma unroll
            for (int i = 0; i < kMB; ++i) a_msk[i] = n_msk[i];
            t = tn;
        }
    }
#undef NVQ_ZERO_ACC
#undef NVQ_TID
    if (MODE == kFC1 && p.amax_part) {
        h_max = wave_max_u32(h_max);
        if ((threadIdx.x & 63) == 0) p.amax_part[blockIdx.x * 4 + wave] = h_max << 16;
    }
}

// Column blocks per wave of both GEMMs. The kernel is written for NB = 4
// (128-column tiles, two workgroups per CU) and NB = 8 (256-column tiles,
// 256 accumulators in AGPRs, one workgroup per CU: a third less decode VALU
// per MFMA and half the activation re-reads); at the moe_layer shapes the
// two take the same time (NB = 8 runs at a higher clock with a less busy
// matrix pipe), so the two-workgroup form is the one launched.
constexpr int kGemmNB = 4;
static int gemm_nb(int, int64_t) { return kGemmNB; }

// Workgroups of a persistent grid: the caller's cap when it gives one
// (1 .. kMaxGemmBlocks), else as many as the CUs hold at once: two per CU
// for 128-column tiles, one for 256-column tiles (whose two 64 KiB weight
// stages take most of a CU's LDS).
static int gemm_grid(int cap, int nb) {
    if (cap > 0) return cap;
    return std::min(device_cus() * (nb == 8 ? 1 : 2), kMaxGemmBlocks);
}

// Scale words four K steps at a time when K allows it and both scale arrays
// are 16-byte aligned (row strides of K / 16 bytes are then multiples of 32).
// (Scale groups need whole 16-byte (NVFP4) or 8-byte (MXFP8) pieces at every
// scale row start and expert offset.)
template <int FMT, int MODE, int NB, bool GU>
static void launch_gemm(const GemmArgs& p, int G, hipStream_t s) {
    const uint32_t q = FMT == kFmtNV ? 8 : 32, w = FMT == kFmtNV ? 16 : 8;
    const bool sg4 = (p.K / step_k<FMT>()) % 4 == 0 && aligned16(p.a_scales) && aligned16(p.b_scales) &&
                     (p.a_ld / q) % w == 0 && (p.b_ld / q) % w == 0 && (p.b_estride / q) % w == 0;
    if (sg4)
        hipLaunchKernelGGL((k_grouped_gemm_dq<FMT, MODE, NB, 4, GU>), dim3(G), dim3(kGemmThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_grouped_gemm_dq<FMT, MODE, NB, 1, GU>), dim3(G), dim3(kGemmThreads), 0, s, p);
}

// Returns the workgroups launched (fc1 leaves four partial maxima per workgroup).
// xt, wt NULL: MXFP8 operands (K code bytes and K/32 E8M0 scales per row).
int launch_fc1(const uint8_t* xc, const uint8_t* xs, const float* xt, const int32_t* offsets,
               const int32_t* s2a, const int32_t* tiles, const int32_t* tile_map, int topk, int64_t E,
               int64_t d, int64_t d_ff,
               const uint8_t* wc, const uint8_t* wsc, const float* wt, uint16_t* h, uint16_t* gu,
               uint32_t* amax_part, uint16_t* dummy, int cap, hipStream_t s) {
    const bool mx = xt == nullptr;
    GemmArgs p{};
    p.a_codes = xc; p.a_scales = xs; p.a_tscale = xt;
    p.offsets = offsets; p.sorted2assign = s2a; p.tile_offsets = tiles; p.tile_map = tile_map;
    p.b_codes = wc; p.b_scales = wsc; p.b_tscale = wt;
    p.out = h; p.gu = gu; p.amax_part = amax_part; p.dummy = dummy;
    p.E = (int)E; p.K = (int)d; p.b_rows = (int)(2 * d_ff); p.topk = topk;
    p.a_ld = p.b_ld = (uint32_t)(mx ? d : d / 2);
    p.b_estride = (int64_t)p.b_rows * p.b_ld;
    const int nb = gemm_nb(kFC1, d_ff), G = gemm_grid(cap, nb);
    p.n_out = (int)d_ff; p.n_tiles = (int)(d_ff / (nb * 16));
    if (mx) {
        if (gu) launch_gemm<kFmtMX, kFC1, kGemmNB, true>(p, G, s);
        else launch_gemm<kFmtMX, kFC1, kGemmNB, false>(p, G, s);
    } else {
        if (gu) launch_gemm<kFmtNV, kFC1, kGemmNB, true>(p, G, s);
        else launch_gemm<kFmtNV, kFC1, kGemmNB, false>(p, G, s);
    }
    return G;
}

void launch_fc2(const uint8_t* hc, const uint8_t* hs, const float* ht, const int32_t* offsets,
                const int32_t* s2a, const int32_t* tiles, const int32_t* tile_map, int64_t E, int64_t d_ff,
                int64_t d,
                const uint8_t* wc, const uint8_t* wsc, const float* wt, uint16_t* y, uint16_t* dummy, int cap,
                hipStream_t s) {
    GemmArgs p{};
    p.a_codes = hc; p.a_scales = hs; p.a_tscale = ht;
    p.offsets = offsets; p.sorted2assign = s2a; p.tile_offsets = tiles; p.tile_map = tile_map;
    p.b_codes = wc; p.b_scales = wsc; p.b_tscale = wt;
    p.out = y; p.dummy = dummy;
    p.E = (int)E; p.K = (int)d_ff; p.b_rows = (int)d; p.topk = 1;
    p.a_ld = p.b_ld = (uint32_t)(ht == nullptr ? d_ff : d_ff / 2);
    p.b_estride = (int64_t)p.b_rows * p.b_ld;
    const int nb = gemm_nb(kFC2, d), G = gemm_grid(cap, nb);
    p.n_out = (int)d; p.n_tiles = (int)(d / (nb * 32));
    if (ht == nullptr) launch_gemm<kFmtMX, kFC2, kGemmNB, false>(p, G, s);
    else launch_gemm<kFmtNV, kFC2, kGemmNB, false>(p, G, s);
}

// The NVFP4 backward's dgrad on the same kernel: out[r] = deq(A[gather[r]]
// (or A[r])) . deq(B_e)^T * Da * Db[e] in fp32 for the rows r of expert e's
// segment, B_e = the K columns starting at e*K of B's N rows. A rows are lda/2
// and B rows ldb/2 code bytes apart (host-checked to keep lane offsets below
// 2^32). tiles / tile_map: m-tiles of kTM rows (launch_tile_offsets).
void launch_dgrad_nvfp4(const uint8_t* ac, const uint8_t* as, const float* at, const int32_t* gather,
                        const uint8_t* bc, const uint8_t* bs, const float* bt, const int32_t* offsets,
                        const int32_t* tiles, const int32_t* tile_map, int64_t lda, int64_t ldb, int64_t E, int64_t N,
                        int64_t K, float* out, uint16_t* dummy, hipStream_t s) {
    GemmArgs p{};
    p.a_codes = ac; p.a_scales = as; p.a_tscale = at;
    p.offsets = offsets; p.sorted2assign = gather; p.tile_offsets = tiles; p.tile_map = tile_map;
    p.b_codes = bc; p.b_scales = bs; p.b_tscale = bt;
    p.out32 = out; p.dummy = dummy;
    p.E = (int)E; p.K = (int)K; p.b_rows = (int)N; p.topk = 1;
    p.a_ld = (uint32_t)(lda / 2);
    p.b_ld = (uint32_t)(ldb / 2);
    p.b_estride = K / 2;
    p.n_out = (int)N; p.n_tiles = (int)(N / tile_n<kGemmNB>());
    launch_gemm<kFmtNV, kDG, kGemmNB, false>(p, gemm_grid(0, kGemmNB), s);
}

size_t gemm_dummy_bytes() { return (size_t)kDummySlots * kDummySlotB; }
int gemm_tile_m() { return kTM; }

// Tile index of A expert-sorted rows: tile offsets [E+1] followed by the
// expert of each m-tile (at most ceil(A / kTM) + E of them).
static size_t tile_words(int64_t A, int64_t E) {
    return (size_t)(E + 1) + (size_t)((A + kTM - 1) / kTM) + (size_t)E;
}

// K of both GEMMs must be a multiple of 128 (a whole number of K steps in
// either format), and so then is N (d for fc2, d_ff for fc1): every
// 128-column (fc1: 64 gate + 64 up) block of an output tile exists. Code
// offsets within X, H and one expert's weight matrix (half a byte per value
// in NVFP4, one in MXFP8) fit in 32 bits (the kernels address them as a
// scalar base plus a 32-bit lane offset), and so does the number of output
// tiles.
static bool moe_dims_ok(int64_t T, int64_t d, int k, int64_t E, int64_t d_ff, bool mx = false) {
    const int64_t lim = (int64_t)1 << (mx ? 31 : 32);  // code bytes x 2 below 2^32
    if (!(T >= 0 && d > 0 && d % kTK == 0 && d_ff > 0 && d_ff % kTK == 0 && k >= 1 && E >= 1 && k <= E &&
          E <= 4096 && T * k < ((int64_t)1 << 31) && T * d / 2 < lim && T * k * d_ff / 2 < lim && d * d_ff < lim))
        return false;
    // output tiles of either GEMM (m-tiles at most A / kTM + E) fit an int
    const int64_t n_tiles = std::max(d_ff / 64, d / 128);
    return (T * k / kTM + E + 1) * n_tiles < ((int64_t)1 << 31);
}

static size_t dummy_bytes() { return (size_t)kDummySlots * kDummySlotB; }

}  // namespace nvq

using namespace nvq;

extern "C" {

size_t moe_fc1_workspace_size(int64_t A, int64_t E) {
    Carver c(nullptr);
    c.take<int32_t>(tile_words(A > 0 ? A : 0, E > 0 ? E : 1));
    c.take<uint32_t>((size_t)kMaxGemmBlocks * 4);
    c.take<uint8_t>(dummy_bytes());
    return c.need;
}

int moe_fc1_swiglu_nvfp4(const uint8_t* xq_codes, const uint8_t* xq_scales, const float* xq_tscale, int64_t T,
                         int64_t d, const int32_t* offsets, const int32_t* sorted2assign, int k, int64_t E,
                         int64_t d_ff, const uint8_t* w1_codes, const uint8_t* w1_scales,
                         const float* w1_tscale, uint16_t* h, uint16_t* gu, float* h_amax, int workgroups,
                         void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!xq_codes || !xq_scales || !xq_tscale || !offsets || !sorted2assign || !w1_codes || !w1_scales ||
        !w1_tscale || !h || !ws)
        return NVQ_ERR_NULL;
    if (!moe_dims_ok(T, d, k, E, d_ff) || workgroups < 0 || workgroups > kMaxGemmBlocks) return NVQ_ERR_DIM;
    if (!aligned16(xq_codes) || !aligned16(w1_codes) || !aligned16(h) || !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_fc1_workspace_size(T * k, E)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    int32_t* tiles = cv.take<int32_t>(tile_words(T * k, E));
    uint32_t* part = cv.take<uint32_t>((size_t)kMaxGemmBlocks * 4);
    uint16_t* dummy = cv.take<uint16_t>(dummy_bytes() / 2);
    launch_tile_offsets(offsets, E, kTM, tiles, tiles + E + 1, s);
    const int G = launch_fc1(xq_codes, xq_scales, xq_tscale, offsets, sorted2assign, tiles, tiles + E + 1, k, E, d,
                             d_ff, w1_codes, w1_scales, w1_tscale, h, gu, h_amax ? part : nullptr, dummy, workgroups, s);
    if (h_amax) launch_fold_partials(part, G * 4, reinterpret_cast<uint32_t*>(h_amax), s);
    return launch_status();
}

size_t moe_fc2_workspace_size(int64_t A, int64_t E) { return moe_fc1_workspace_size(A, E); }

int moe_fc2_nvfp4(const uint8_t* hq_codes, const uint8_t* hq_scales, const float* hq_tscale, int64_t A,
                  int64_t d_ff, const int32_t* offsets, const int32_t* sorted2assign, int64_t E, int64_t d,
                  const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_tscale, uint16_t* y,
                  int workgroups, void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!hq_codes || !hq_scales || !hq_tscale || !offsets || !sorted2assign || !w2_codes || !w2_scales ||
        !w2_tscale || !y || !ws)
        return NVQ_ERR_NULL;
    if (!moe_dims_ok(A, d, 1, E > 0 ? E : 1, d_ff) || workgroups < 0 || workgroups > kMaxGemmBlocks)
        return NVQ_ERR_DIM;
    if (!aligned16(hq_codes) || !aligned16(w2_codes) || !aligned16(y) || !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_fc2_workspace_size(A, E)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    int32_t* tiles = cv.take<int32_t>(tile_words(A, E));
    cv.take<uint32_t>((size_t)kMaxGemmBlocks * 4);
    uint16_t* dummy = cv.take<uint16_t>(dummy_bytes() / 2);
    launch_tile_offsets(offsets, E, kTM, tiles, tiles + E + 1, s);
    launch_fc2(hq_codes, hq_scales, hq_tscale, offsets, sorted2assign, tiles, tiles + E + 1, E, d_ff, d, w2_codes,
               w2_scales, w2_tscale, y, dummy, workgroups, s);
    return launch_status();
}

// ------------------------------------------------------------------ MXFP8 forward
int moe_fc1_swiglu_mxfp8(const uint8_t* x_elems, const uint8_t* x_scales, int64_t T, int64_t d,
                         const int32_t* offsets, const int32_t* sorted2assign, int k, int64_t E, int64_t d_ff,
                         const uint8_t* w1_elems, const uint8_t* w1_scales, uint16_t* h, uint16_t* gu,
                         int workgroups, void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!x_elems || !x_scales || !offsets || !sorted2assign || !w1_elems || !w1_scales || !h || !ws)
        return NVQ_ERR_NULL;
    if (!moe_dims_ok(T, d, k, E, d_ff, true) || workgroups < 0 || workgroups > kMaxGemmBlocks) return NVQ_ERR_DIM;
    if (!aligned16(x_elems) || !aligned16(w1_elems) || !aligned16(h) || (gu && !aligned16(gu)) || !aligned256(ws))
        return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_fc1_workspace_size(T * k, E)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    int32_t* tiles = cv.take<int32_t>(tile_words(T * k, E));
    cv.take<uint32_t>((size_t)kMaxGemmBlocks * 4);
    uint16_t* dummy = cv.take<uint16_t>(dummy_bytes() / 2);
    launch_tile_offsets(offsets, E, kTM, tiles, tiles + E + 1, s);
    launch_fc1(x_elems, x_scales, nullptr, offsets, sorted2assign, tiles, tiles + E + 1, k, E, d, d_ff, w1_elems,
               w1_scales, nullptr, h, gu, nullptr, dummy, workgroups, s);
    return launch_status();
}

int moe_fc2_mxfp8(const uint8_t* h_elems, const uint8_t* h_scales, int64_t A, int64_t d_ff, const int32_t* offsets,
                  const int32_t* sorted2assign, int64_t E, int64_t d, const uint8_t* w2_elems,
                  const uint8_t* w2_scales, uint16_t* y, int workgroups, void* ws, size_t ws_bytes,
                  nvq_stream_t stream) {
    if (!h_elems || !h_scales || !offsets || !sorted2assign || !w2_elems || !w2_scales || !y || !ws)
        return NVQ_ERR_NULL;
    if (!moe_dims_ok(A, d, 1, E > 0 ? E : 1, d_ff, true) || workgroups < 0 || workgroups > kMaxGemmBlocks)
        return NVQ_ERR_DIM;
    if (!aligned16(h_elems) || !aligned16(w2_elems) || !aligned16(y) || !aligned256(ws)) return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_fc2_workspace_size(A, E)) return NVQ_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    int32_t* tiles = cv.take<int32_t>(tile_words(A, E));
    cv.take<uint32_t>((size_t)kMaxGemmBlocks * 4);
    uint16_t* dummy = cv.take<uint16_t>(dummy_bytes() / 2);
    launch_tile_offsets(offsets, E, kTM, tiles, tiles + E + 1, s);
    launch_fc2(h_elems, h_scales, nullptr, offsets, sorted2assign, tiles, tiles + E + 1, E, d_ff, d, w2_elems,
               w2_scales, nullptr, y, dummy, workgroups, s);
    return launch_status();
}

// Workspace plan of the MXFP8 forward (every carve 256-byte aligned):
//   GEMM dummy slots | route scratch | tile offsets | offsets | sorted2assign
//   | Xq elems, scales [T, d] | H [A, d_ff] | Hq elems, scales | quantizer scratch.
static size_t mx_fwd_carve(Carver& c, int64_t T, int64_t d, int k, int64_t E, int64_t d_ff, uint16_t** dummy,
                           uint32_t** rws, int32_t** tiles, int32_t** offsets, int32_t** s2a, uint8_t** xe,
                           uint8_t** xs, uint16_t** H, uint8_t** he, uint8_t** hs, void** qws, size_t* qws_bytes) {
    const int64_t A = T * k, A1 = A > 0 ? A : 1, T1 = T > 0 ? T : 1;
    *dummy = c.take<uint16_t>(dummy_bytes() / 2);
    *rws = c.take<uint32_t>(route_ws_words(A, E));
    *tiles = c.take<int32_t>(tile_words(A, E));
    *offsets = c.take<int32_t>((size_t)E + 1);
    *s2a = c.take<int32_t>((size_t)A1);
    *xe = c.take<uint8_t>((size_t)(T1 * d));
    *xs = c.take<uint8_t>((size_t)(T1 * d / 32));
    *H = c.take<uint16_t>((size_t)(A1 * d_ff));
    *he = c.take<uint8_t>((size_t)(A1 * d_ff));
    *hs = c.take<uint8_t>((size_t)(A1 * d_ff / 32));
    *qws_bytes = std::max(mxfp8_requant_workspace_size(T1, 1), mxfp8_requant_workspace_size(A1, 1));
    *qws = c.take<uint8_t>(*qws_bytes);
    return c.need;
}

size_t moe_expert_fwd_mxfp8_workspace_size(int64_t T, int64_t d, int k, int64_t E, int64_t d_ff) {
    Carver c(nullptr);
    uint16_t *dm, *H;
    uint32_t* r;
    int32_t *t, *o, *s2;
    uint8_t *xe, *xs, *he, *hs;
    void* q;
    size_t qb;
    return mx_fwd_carve(c, T, d, k, E > 0 ? E : 1, d_ff, &dm, &r, &t, &o, &s2, &xe, &xs, &H, &he, &hs, &q, &qb);
}

int moe_expert_fwd_mxfp8(const uint16_t* x, int64_t T, int64_t d, const int32_t* topk_ids, int k, int64_t E,
                         int64_t d_ff, const uint8_t* w1_elems, const uint8_t* w1_scales, const uint8_t* w2_elems,
                         const uint8_t* w2_scales, uint16_t* y, void* ws, size_t ws_bytes, nvq_stream_t stream) {
    if (!x || !topk_ids || !w1_elems || !w1_scales || !w2_elems || !w2_scales || !y || !ws) return NVQ_ERR_NULL;
    if (!moe_dims_ok(T, d, k, E, d_ff, true)) return NVQ_ERR_DIM;
    if (!aligned16(x) || !aligned16(w1_elems) || !aligned16(w2_elems) || !aligned16(y) || !aligned256(ws))
        return NVQ_ERR_ALIGN;
    if (ws_bytes < moe_expert_fwd_mxfp8_workspace_size(T, d, k, E, d_ff)) return NVQ_ERR_WORKSPACE;
    const int64_t A = T * k;
    if (A == 0) return NVQ_OK;
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    uint16_t *dummy, *H;
    uint32_t* rws;
    int32_t *tiles, *offsets, *s2a;
    uint8_t *xe, *xs, *he, *hs;
    void* qws;
    size_t qb;
    mx_fwd_carve(cv, T, d, k, E, d_ff, &dummy, &rws, &tiles, &offsets, &s2a, &xe, &xs, &H, &he, &hs, &qws, &qb);
    // 1. MXFP8 of X along d, nearest even (per-row blocks: the bytes of a
    //    gathered row equal those of the token's row, so X is quantized once)
    int rc = mxfp8_requant_sr(x, T, d, 0, nullptr, 1, nullptr, 1, 0, NVQ_RTN, 0, 0, 0, xe, xs, qws, qb, stream);
    if (rc != NVQ_OK) return rc;
    // 2. expert segments and their m-tiles
    launch_route(topk_ids, A, E, offsets, s2a, tiles, tiles + E + 1, kTM, rws, s);
    // 3. fc1 + SwiGLU: exact bf16 operands, bf16 MFMA, H in bf16
    launch_fc1(xe, xs, nullptr, offsets, s2a, tiles, tiles + E + 1, k, E, d, d_ff, w1_elems, w1_scales, nullptr, H,
               nullptr, nullptr, dummy, 0, s);
    // 4. MXFP8 of H along d_ff, nearest even (rows past the last segment are
    //    quantized too and never read)
    rc = mxfp8_requant_sr(H, A, d_ff, 0, nullptr, 1, nullptr, 1, 0, NVQ_RTN, 0, 0, 0, he, hs, qws, qb, stream);
    if (rc != NVQ_OK) return rc;
    // 5. fc2, rounded to bf16 and scattered to (token, slot) in the epilogue
    launch_fc2(he, hs, nullptr, offsets, s2a, tiles, tiles + E + 1, E, d_ff, d, w2_elems, w2_scales, nullptr, y,
               dummy, 0, s);
    return launch_status();
}

// Workspace plan of the fused forward (every carve 256-byte aligned):
//   partial maxima of X | of H | GEMM dummy slots | route scratch | tile offsets
//   [E+1] | then any intermediate the caller did not supply: Xq, offsets,
//   sorted2assign, H, Hq.
static size_t moe_fwd_carve(Carver& c, int64_t T, int64_t d, int k, int64_t E, int64_t d_ff,
                            const nvq_moe_buffers* b, uint32_t** xpart, uint32_t** hpart, uint16_t** dummy,
                            uint32_t** rws, int32_t** tiles, nvq_moe_buffers* out) {
    const int64_t A = T * k;
    *xpart = c.take<uint32_t>((size_t)stream_blocks(T * d / 8, 1));
    *hpart = c.take<uint32_t>((size_t)kMaxGemmBlocks * 4);
    *dummy = c.take<uint16_t>(dummy_bytes() / 2);
    *rws = c.take<uint32_t>(route_ws_words(A, E));
    *tiles = c.take<int32_t>(tile_words(A, E));
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
    out->gemm_workgroups = in.gemm_workgroups;
    return c.need;
}

size_t moe_expert_fwd_nvfp4_workspace_size(int64_t T, int64_t d, int k, int64_t E, int64_t d_ff) {
    Carver c(nullptr);
    uint32_t *a, *a2, *r;
    uint16_t* dm;
    int32_t* t;
    nvq_moe_buffers o{};
    return moe_fwd_carve(c, T, d, k, E, d_ff, nullptr, &a, &a2, &dm, &r, &t, &o);
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
        uint32_t *a, *a2, *r;
        uint16_t* dm;
        int32_t* t;
        nvq_moe_buffers o{};
        if (ws_bytes < moe_fwd_carve(need, T, d, k, E, d_ff, bufs, &a, &a2, &dm, &r, &t, &o))
            return NVQ_ERR_WORKSPACE;
    }
    if (bufs) {
        const nvq_moe_buffers& b = *bufs;
        if (b.gemm_workgroups < 0 || b.gemm_workgroups > kMaxGemmBlocks) return NVQ_ERR_DIM;
        const void* ptrs[] = {b.xq_codes, b.xq_scales, b.h, b.hq_codes, b.hq_scales, b.gu};
        for (const void* q : ptrs)
            if (q && !aligned16(q)) return NVQ_ERR_ALIGN;
    }
    hipStream_t s = as_stream(stream);
    Carver cv(ws);
    uint32_t *xpart, *hpart, *rws;
    uint16_t* dummy;
    int32_t* tiles;
    nvq_moe_buffers m{};
    moe_fwd_carve(cv, T, d, k, E, d_ff, bufs, &xpart, &hpart, &dummy, &rws, &tiles, &m);
    const int64_t A = T * k;

    // 1. NVFP4 of X (one tensor scale over X; rows are gathered later)
    const int gx = stream_blocks(T * d / 8, 1);
    launch_amax_bf16(x, 1, T * d, xpart, gx, s);
    launch_nvfp4_encode_bf16(x, 1, T * d, xpart, gx, gx, m.xq_codes, m.xq_scales, m.xq_tscale, NVQ_RTN, 0, 1, s);
    // 2. expert segments
    launch_route(topk_ids, A, E, m.offsets, m.sorted2assign, tiles, tiles + E + 1, kTM, rws, s);
    // 3. fc1 + SwiGLU, per-wave partial maxima of |H| (four per workgroup of its grid)
    const int G = launch_fc1(m.xq_codes, m.xq_scales, m.xq_tscale, m.offsets, m.sorted2assign, tiles, tiles + E + 1,
                             k, E, d, d_ff, w1_codes, w1_scales, w1_tscale, m.h, m.gu, hpart, dummy,
                             m.gemm_workgroups, s);
    // 4. NVFP4 of H with one tensor scale over all of H
    const int gh = G * 4;
    launch_nvfp4_encode_bf16(m.h, 1, A * d_ff, hpart, gh, gh, m.hq_codes, m.hq_scales, m.hq_tscale, NVQ_RTN, 0, 1,
                             s);
    // 5. fc2, scattered back to (token, slot) order
    launch_fc2(m.hq_codes, m.hq_scales, m.hq_tscale, m.offsets, m.sorted2assign, tiles, tiles + E + 1, E, d_ff, d,
               w2_codes, w2_scales, w2_tscale, y, dummy, m.gemm_workgroups, s);
    return launch_status();
}

}  // extern "C"
