// Routed-expert MoE decode layer for CDNA4 (gfx950), one persistent launch per call.
//
// The layer is the chain the Ling-3.0-flash decode pages describe ("Chasing the Batch-1
// Floor", section "PDL: stacking the latency floors of small kernels": router chain
// gate matvec -> top-k, MoE chain align -> up-GEMM -> activation -> down-GEMM -> combine), cut
// for a batch of at most 16 tokens on an MI355X.  One workgroup of 8 waves runs on every CU and
// all of them are resident at once; the page's launch-ordered chain becomes counters in memory,
// and, as with its "producer-independent loads before the wait", work that needs no routing
// result runs before the routing barrier:
//
//   A  stage the token rows in LDS and copy this workgroup's slice of the shared expert's down
//      rows into LDS; compute this workgroup's router rows (tagged fp32 logits); compute a share
//      of the shared expert's gate/up rows.
//   B  routing: below three tokens every workgroup redoes the per-token top-k from the tagged
//      logits; from three tokens on workgroup m selects token m's experts and publishes them as
//      tagged words that every workgroup reads.  Each workgroup builds the batch compaction
//      (distinct experts ascending, token bitmask and pair rows per unit) in its own LDS;
//      workgroup 0 writes the caller-visible outputs.
//   C  all routed units' gate/up rows: each weight row is read once and applied to every token of
//      its unit, silu(g) * v in fp32 (bf16 weights on the vector ALU, a static share and then
//      chunks from per-XCD pools; MXFP4 weights on the matrix cores).  Meanwhile as many of this
//      workgroup's down rows as fit stream into LDS.
//   D  slice mode (few pair rows, or MXFP4 rows that fit): every workgroup computes its own y
//      columns of every unit on the matrix cores from LDS; otherwise a cost-weighted share of
//      all units' down rows as one task list, fp32 partial outputs per pair row.
//   E  every workgroup owns a fixed slice of y's columns: it sums each token's partials in slot
//      order (slice mode: from LDS; otherwise once every workgroup's partials have landed),
//      adds the shared expert and casts once.
//
// The streaming loops never store to global memory: vector memory operations retire in order
// on gfx9, so a store in the loop would make the next wait for prefetched weights also wait
// for the store to be acknowledged.  Results are staged in LDS and written at the end of a
// phase.  Data that crosses workgroups goes through device-scope (sc1) stores and loads, and a
// counter is bumped only after the stores have completed; there are no cache-wide fences.
// Every wait is bounded: on a timeout the status word is flagged and the kernel still finishes.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

#define LDS __attribute__((address_space(3)))

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------------
// cross-lane reductions (wave64)
// ------------------------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_rows(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}

// every lane of each 16-lane row receives the row's sum
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    return v;
}
// DPP-only reductions (no LDS crossbar): the sum of each 32-lane half lands in its upper row
// (lanes 16..31 and 48..63); the sum of the whole wave lands in row 3 (lanes 48..63).
__device__ __forceinline__ float half_sum_hi(float v) {
    v = row16_sum(v);
    const int b = __builtin_bit_cast(int, v);
    return v + __builtin_bit_cast(float, dpp_rows<0x142, 0xA>(0, b));  // row_bcast:15 into rows 1, 3
}
__device__ __forceinline__ float wave_sum_hi(float v) {
    v = half_sum_hi(v);
    const int b = __builtin_bit_cast(int, v);
    return v + __builtin_bit_cast(float, dpp_rows<0x143, 0xC>(0, b));  // row_bcast:31 into rows 2, 3
}
// Sum over each group of LPR consecutive lanes; valid in the group's last lane.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPR == 64) {
        return wave_sum_hi(v);
    } else if constexpr (LPR == 32) {
        return half_sum_hi(v);
    } else if constexpr (LPR == 16) {
        return row16_sum(v);
    } else {
        static_assert(LPR == 8, "lane groups of 8, 16, 32 or 64");
        v += dpp<0xB1>(v);
        v += dpp<0x4E>(v);
        return v + dpp<0x141>(v);  // row_half_mirror pairs the two quads of each 8-lane half
    }
}
// The maximum over the wave, uniform in every lane (row max by DPP, then rows by broadcast).
__device__ __forceinline__ float wave_max_bcast(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    int b = __builtin_bit_cast(int, v);
    v = fmaxf(v, __builtin_bit_cast(float, dpp_rows<0x142, 0xA>(b, b)));  // row_bcast:15 into rows 1, 3
    b = __builtin_bit_cast(int, v);
    v = fmaxf(v, __builtin_bit_cast(float, dpp_rows<0x143, 0xC>(b, b)));  // row_bcast:31 into rows 2, 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Maximum of an unsigned value over the wave, in every lane (0 is the identity).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto step = [](uint32_t x, int y) { return max(x, (uint32_t)y); };
    int b = (int)v;
    v = step(v, __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
    b = (int)v;
    v = step(v, __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
    b = (int)v;
    v = step(v, __builtin_amdgcn_update_dpp(0, b, 0x141, 0xF, 0xF, true));  // row_half_mirror
    b = (int)v;
    v = step(v, __builtin_amdgcn_update_dpp(0, b, 0x140, 0xF, 0xF, true));  // row_mirror
    b = (int)v;
    v = step(v, __builtin_amdgcn_update_dpp(0, b, 0x142, 0xA, 0xF, false));  // row_bcast:15 into rows 1, 3
    b = (int)v;
    v = step(v, __builtin_amdgcn_update_dpp(0, b, 0x143, 0xC, 0xF, false));  // row_bcast:31 into rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// The wave's index in the workgroup, as a scalar the compiler knows to be wave-uniform.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
// Number of the tasks b, b + G, b + 2G, ... below T: tasks are dealt to the G workgroups round
// robin, so at any moment the whole grid streams one contiguous window of the weights (every HBM
// channel busy, every workgroup with the same bytes to move).
__device__ __forceinline__ int n_strided(int T, int b, int G) { return b < T ? (T - 1 - b) / G + 1 : 0; }


// ------------------------------------------------------------------------------------------
// number formats and weight geometry
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// E8M0 scale byte -> the fp32 value 2^(S-127) (S = 0 is the fp32 subnormal 2^-127, 255 is NaN)
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
    return __uint_as_float(s == 0 ? 0x00400000u : (s == 255 ? 0x7FC00000u : (s << 23)));
}

// Weights are streamed in 16-byte chunks: 4 binary32, 8 bfloat16, or 32 E2M1 codes (one MX
// block, whose E8M0 scale byte travels with it).  A matrix row is covered by LPR lanes, each
// taking chunks c = lane % LPR + LPR * j; a wave covers 64 / LPR rows at once and every lane
// holds RL rows, so one wave task is RT = RL * 64 / LPR rows.  _G: gate/up rows (K = hidden),
// _D: down rows (K = intermediate).
template <int WF>
struct Geo;
template <>
struct Geo<MOE_FMT_F32> {
    static constexpr int EPC = 4, LPR_G = 64, RL_G = 1, LPR_D = 64, RL_D = 1;
};
template <>
struct Geo<MOE_FMT_BF16> {
    static constexpr int EPC = 8, LPR_G = 64, RL_G = 1, LPR_D = 32, RL_D = 4;
};
template <>
struct Geo<MOE_FMT_MXFP4> {
    static constexpr int EPC = 32, LPR_G = 16, RL_G = 1, LPR_D = 8, RL_D = 1;
};
// FP8: 16 E4M3 codes per chunk, all in one 128-column scale block.  32 lanes per gate/up row (two
// rows of 2,560 codes per wave and 10 KB per task, the bytes of a bf16 task) and two rows per lane
// group of a down task (8 rows, 6 KB): a task's loads are what one wave keeps in flight, so tasks
// of half a bf16 task's bytes streamed at half its rate
template <>
struct Geo<MOE_FMT_FP8> {
    static constexpr int EPC = 16, LPR_G = 32, RL_G = 1, LPR_D = 16, RL_D = 2;
};
constexpr int kFp8Block = 128;  // FP8 weights: one binary32 scale per 128 x 128 block
template <int WF>
__host__ __device__ constexpr int rt_gate() { return Geo<WF>::RL_G * (64 / Geo<WF>::LPR_G); }
template <int WF>
__host__ __device__ constexpr int rt_down() { return Geo<WF>::RL_D * (64 / Geo<WF>::LPR_D); }

// bytes of one row of K elements (MXFP4: the codes; the scales are K / 32 bytes more)
template <int WF>
__host__ __device__ constexpr int64_t row_bytes(int64_t K) {
    return WF == MOE_FMT_F32 ? 4 * K : (WF == MOE_FMT_BF16 ? 2 * K : (WF == MOE_FMT_FP8 ? K : K / 2));
}

// Tasks per gate/up pool chunk (about 20 KB of weights: 10 KB went no faster and 40 KB was slower
// at six bf16 tokens).  The kernel claims chunks of this size and the host sizes each wave's
// staging room for two of them, so both must use this one definition.
template <int WF>
__host__ __device__ constexpr int gu_chunk_tasks(int H) {
    const int c = 20480 / (2 * rt_gate<WF>() * (int)row_bytes<WF>(H));  // 32-bit: on the path to gate/up
    return c > 1 ? c : 1;
}

// Block scales.  scale_mat: the scales of matrix e of a stack [E][rows][K]; scale_row: the scales
// that apply to absolute row r of one matrix (MXFP4: its K / 32 E8M0 bytes; FP8: the K / 128
// binary32 scales of its 128-row block).  Other formats have none.
template <int WF>
__device__ __forceinline__ const uint8_t* scale_mat(const uint8_t* s, int64_t e, int64_t rows, int64_t K) {
    if constexpr (WF == MOE_FMT_MXFP4) return s + e * rows * (K / 32);
    if constexpr (WF == MOE_FMT_FP8) return s + 4 * e * (rows / kFp8Block) * (K / kFp8Block);
    return nullptr;
}
template <int WF>
__device__ __forceinline__ const uint8_t* scale_row(const uint8_t* m, int64_t r, int64_t K) {
    if constexpr (WF == MOE_FMT_MXFP4) return m + r * (K / 32);
    if constexpr (WF == MOE_FMT_FP8) return m + 4 * (r / kFp8Block) * (K / kFp8Block);
    return nullptr;
}

struct Chunk {
    u32x4 q;
    uint32_t s;  // MXFP4: the block's E8M0 byte; FP8: the block's binary32 scale bits
};

// Makes the compiler wait for a chunk's load here, in straight-line code, and treat the value as
// an ordinary register afterwards, so the waits inside the compute loops never drain the next
// task's prefetch.
template <int WF>
__device__ __forceinline__ void settle(Chunk& r) {
    if constexpr (WF == MOE_FMT_MXFP4 || WF == MOE_FMT_FP8)
        asm volatile("" : "+v"(r.q), "+v"(r.s));
    else
        asm volatile("" : "+v"(r.q));
}

// Chunks past the end of a row are loaded from the row's last chunk (so every load is in bounds
// and the number of loads in flight is static) and zeroed here, once the load has landed, so the
// compute loops need no per-chunk branch.
template <int WF>
__device__ __forceinline__ void settle_mask(Chunk& r, bool valid) {
    settle<WF>(r);
    if (!valid) r.q = u32x4{0u, 0u, 0u, 0u};
}

// chunk c of a weight row in global memory (streamed once: non-temporal)
template <int WF>
__device__ __forceinline__ void ld_chunk(Chunk& r, const uint8_t* row, const uint8_t* srow, int c) {
    r.q = __builtin_nontemporal_load((const u32x4*)(row + 16 * c));
    if constexpr (WF == MOE_FMT_MXFP4) r.s = __builtin_nontemporal_load(srow + c);
    if constexpr (WF == MOE_FMT_FP8) r.s = ((const uint32_t*)srow)[c / (kFp8Block / 16)];
}
// chunk c of a weight row held in LDS (the MXFP4 scales stay in global memory)
template <int WF>
__device__ __forceinline__ void ld_chunk_lds(Chunk& r, const LDS uint8_t* row, const uint8_t* srow, int c) {
    r.q = *(const LDS u32x4*)(row + 16 * c);
    if constexpr (WF == MOE_FMT_MXFP4) r.s = srow[c];
    if constexpr (WF == MOE_FMT_FP8) r.s = ((const uint32_t*)srow)[c / (kFp8Block / 16)];
}

// Reinterprets a dword as two bf16.  Takes the dword by value: bit-casting a vector component
// lvalue directly (v.y) makes clang read the vector's first element instead.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Independent partial sums of one dot product: a chain of dependent v_dot2 would run at the
// instruction's latency, four interleaved chains at its issue rate.  Summed in a fixed order.
constexpr int kAcc = 4;
__device__ __forceinline__ float acc_sum(const float (&a)[kAcc]) { return (a[0] + a[1]) + (a[2] + a[3]); }

// Dot of weight chunk c with the matching elements of a token row x (LDS; bf16, or binary32 for
// the binary32 layer), fp32 accumulation into the partial sums acc.
template <int AF, int WF>
__device__ __forceinline__ void dot_x(const Chunk& r, const LDS char* xrow, int c, float (&acc)[kAcc]) {
    if constexpr (WF == MOE_FMT_BF16) {
        const u32x4 x = *(const LDS u32x4*)(xrow + 16 * c);
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        const uint32_t x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
        acc[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(x0), acc[0], false);
        acc[1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(x1), acc[1], false);
        acc[2] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(x2), acc[2], false);
        acc[3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(x3), acc[3], false);
    } else if constexpr (WF == MOE_FMT_MXFP4) {
        // dword d of the codes holds elements 8d .. 8d+7; byte s of it elements 8d+2s (low
        // nibble) and 8d+2s+1, which is dword s of the d-th 16 bytes of x
        const LDS u32x4* xp = (const LDS u32x4*)(xrow + 64 * c);
        const float sc = e8m0_to_f32(r.s);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u32x4 x = xp[d];
            const uint32_t w = r.q[d];
            const uint32_t x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
            acc[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0), as_bf16x2(x0), acc[0], false);
            acc[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1), as_bf16x2(x1), acc[1], false);
            acc[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2), as_bf16x2(x2), acc[2], false);
            acc[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3), as_bf16x2(x3), acc[3], false);
        }
    } else if constexpr (WF == MOE_FMT_FP8) {
        // dword d of the codes holds elements 4d .. 4d+3 (byte b = element 4d+b), which are dwords
        // 2d and 2d+1 of the 32 bytes of x; each E4M3 pair becomes a bfloat16 pair exactly (scale 1),
        // and the chunk's partial sums take the block's scale once
        const LDS u32x4* xp = (const LDS u32x4*)(xrow + 32 * c);
        const u32x4 xa = xp[0], xb = xp[1];
        const uint32_t xd[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
        const float sc = __uint_as_float(r.s);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w = r.q[d];
            float t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false),
                                                      as_bf16x2(xd[2 * d]), 0.0f, false);
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true),
                                                as_bf16x2(xd[2 * d + 1]), t, false);
            acc[d] = fmaf(t, sc, acc[d]);
        }
    } else {
        const f32x4 x = *(const LDS f32x4*)(xrow + 16 * c);
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        acc[0] = fmaf(__uint_as_float(w0), x[0], acc[0]);
        acc[1] = fmaf(__uint_as_float(w1), x[1], acc[1]);
        acc[2] = fmaf(__uint_as_float(w2), x[2], acc[2]);
        acc[3] = fmaf(__uint_as_float(w3), x[3], acc[3]);
    }
}

// How the vector down path stages a SwiGLU output row in LDS (act_mode): 0 fp32 (binary32
// weights); 1 two bfloat16 planes (bf16 weights), hi = the fp32 value with its low 16 bits cleared
// and lo = the rest rounded to bfloat16 (at `lo_off` bytes from the row), so hi + lo carries ~16
// significant bits and every product pair is one v_dot2_f32_bf16; 2 one bfloat16 plane rounded to
// nearest even (MXFP4 and FP8 weights: the rounding the matrix cores apply; their rows decode to
// bfloat16 in the same instructions, and the second plane doubled the LDS reads and products of
// the phase: FP8 at 16 tokens 125.8 -> 122.1 us, at 6 tokens 62.9 -> 59.5 us, MXFP4 at 16 tokens
// 98.0 -> 93.1 us).
template <int WF>
__host__ __device__ constexpr int act_mode() {
    return WF == MOE_FMT_F32 ? 0 : (WF == MOE_FMT_BF16 ? 1 : 2);
}

// Dot of weight chunk c with the matching elements of a SwiGLU output row in LDS (staged as
// act_mode<WF>), fp32 accumulation.
template <int WF>
__device__ __forceinline__ void dot_a(const Chunk& r, const LDS char* arow, int lo_off, int c, float (&acc)[kAcc]) {
    if constexpr (WF == MOE_FMT_BF16) {
        const u32x4 hi = *(const LDS u32x4*)(arow + 16 * c);
        const u32x4 lo = *(const LDS u32x4*)(arow + lo_off + 16 * c);
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        const uint32_t h0 = hi[0], h1 = hi[1], h2 = hi[2], h3 = hi[3];
        const uint32_t l0 = lo[0], l1 = lo[1], l2 = lo[2], l3 = lo[3];
        acc[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(h0), acc[0], false);
        acc[1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(h1), acc[1], false);
        acc[2] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(h2), acc[2], false);
        acc[3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(h3), acc[3], false);
        acc[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(l0), acc[0], false);
        acc[1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(l1), acc[1], false);
        acc[2] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(l2), acc[2], false);
        acc[3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(l3), acc[3], false);
    } else if constexpr (WF == MOE_FMT_MXFP4) {
        const float sc = e8m0_to_f32(r.s);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u32x4 a = *(const LDS u32x4*)(arow + 64 * c + 16 * d);
            const uint32_t w = r.q[d];
            const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
            const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
            const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
            const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
            const uint32_t a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
            acc[0] = __builtin_amdgcn_fdot2_f32_bf16(p0, as_bf16x2(a0), acc[0], false);
            acc[1] = __builtin_amdgcn_fdot2_f32_bf16(p1, as_bf16x2(a1), acc[1], false);
            acc[2] = __builtin_amdgcn_fdot2_f32_bf16(p2, as_bf16x2(a2), acc[2], false);
            acc[3] = __builtin_amdgcn_fdot2_f32_bf16(p3, as_bf16x2(a3), acc[3], false);
        }
    } else if constexpr (WF == MOE_FMT_FP8) {
        // as dot_x: chunk c covers elements 16c .. 16c+15, 32 bytes of the bfloat16 row
        const LDS u32x4* ap = (const LDS u32x4*)(arow + 32 * c);
        const u32x4 aa = ap[0], ab = ap[1];
        const uint32_t ad[8] = {aa[0], aa[1], aa[2], aa[3], ab[0], ab[1], ab[2], ab[3]};
        const float sc = __uint_as_float(r.s);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w = r.q[d];
            const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
            const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
            float t = __builtin_amdgcn_fdot2_f32_bf16(p0, as_bf16x2(ad[2 * d]), 0.0f, false);
            t = __builtin_amdgcn_fdot2_f32_bf16(p1, as_bf16x2(ad[2 * d + 1]), t, false);
            acc[d] = fmaf(t, sc, acc[d]);
        }
    } else {
        const f32x4 a = *(const LDS f32x4*)(arow + 16 * c);
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        acc[0] = fmaf(__uint_as_float(w0), a[0], acc[0]);
        acc[1] = fmaf(__uint_as_float(w1), a[1], acc[1]);
        acc[2] = fmaf(__uint_as_float(w2), a[2], acc[2]);
        acc[3] = fmaf(__uint_as_float(w3), a[3], acc[3]);
    }
}

__device__ __forceinline__ float silu_mul(float g, float v) { return g / (1.0f + __expf(-g)) * v; }

// LDS tables of the batch dispatch, in words (at most kMaxUnits routed units plus the shared one)
constexpr int kMaxUnits = kMaxTokens * kMaxTopK;
constexpr int kTabMask = 0;                                  // [kMaxUnits + 1] token bitmask per unit
constexpr int kTabOff = kTabMask + kMaxUnits + 1;            // [kMaxUnits + 2] first pair row per unit
constexpr int kTabExp = kTabOff + kMaxUnits + 2;             // [kMaxUnits + 1] expert id per unit
constexpr int kTabPair = kTabExp + kMaxUnits + 1;            // [kMaxTokens * kMaxTopK] pair row of (m, j)
constexpr int kTabRowW = kTabPair + kMaxTokens * kMaxTopK;   // [kMaxTokens * (kMaxTopK + 1)] weight per row
constexpr int kTabMisc = kTabRowW + kMaxTokens * (kMaxTopK + 1);  // [8] U, flags
constexpr int kTabWords = (kTabMisc + 8 + 3) / 4 * 4;
// routing scratch (token masks, expert row offsets, per-token ids / weights / logits), in the
// staging area
constexpr int kSelBytes = (2 * kMaxExperts + 3 * kMaxTokens * kMaxTopK) * 4;
constexpr int kMaxSeg = 4;  // unit-major: segments (one per unit) of a workgroup's down rows in one flat task list

constexpr int kCostBase = 8;  // cost of one weight row's bytes in cost_split units
constexpr int kSpinLimit = 1 << 20;  // ~1 s of polling; normal waits are microseconds

// Phase timestamps for performance analysis, compiled out unless MOE_PHASE_TRACE is defined.
// Thread 0 keeps them in LDS and writes them out when the workgroup finishes, so recording a
// timestamp never waits on the vector-memory counter.
#ifdef MOE_PHASE_TRACE
__device__ uint64_t* g_moe_trace;
__shared__ uint64_t s_trace[32];
#define MOE_TRACE_INIT                                  \
    do {                                                \
        if (threadIdx.x < 32) s_trace[threadIdx.x] = 0; \
    } while (0)
#define MOE_TRACE(slot)                                                           \
    do {                                                                          \
        if (threadIdx.x == 0) s_trace[(slot)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#define MOE_TRACE_FLUSH                                                                \
    do {                                                                               \
        if (threadIdx.x == 0) {                                                        \
            s_trace[31] = __builtin_amdgcn_s_memrealtime();                            \
            uint64_t* t = g_moe_trace;                                                 \
            if (t)                                                                     \
                for (int i_ = 0; i_ < 32; ++i_) t[blockIdx.x * 32 + i_] = s_trace[i_]; \
        }                                                                              \
    } while (0)
#else
#define MOE_TRACE_INIT \
    do {               \
    } while (0)
#define MOE_TRACE(slot) \
    do {                \
    } while (0)
#define MOE_TRACE_FLUSH \
    do {                \
    } while (0)
#endif

// ---- device-scope memory operations (coherent across XCDs without cache maintenance) -------

__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte device-scope load (sc1) through a buffer resource covering `bytes` from `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 ld_dev16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */));
}
// All of this workgroup's device-scope stores have completed when it returns.
__device__ __forceinline__ void publish() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
}
// Where a wait that gives up reports it: the workspace status word (sticky until moe_read_status)
// and this call's fault line, which the workgroups read before they write y.  s_fault is the
// workgroup's own record.  A wait gives up only if the grid is not fully resident or a producer
// never arrives; its results are then invalid and y is written as NaN.
struct Fault {
    uint32_t* status;
    uint32_t* flag;
    int spin;  // polls before a wait gives up
};
__shared__ uint32_t s_fault;
// Called by one lane.  The flag has reached memory before this wave issues anything else, so a
// consumer that sees data this workgroup publishes later also sees the flag.
__device__ __forceinline__ void raise_timeout(const Fault& f) {
    __hip_atomic_fetch_or(f.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(f.flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_fault = 1u;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Thread 0 waits until *c >= target (bounded); the whole workgroup continues together.
__device__ __forceinline__ void wait_geq(const uint32_t* c, uint32_t target, const Fault& f) {
    if (threadIdx.x == 0) {
        int i = 0;
        while (ld_dev(c) < target && i < f.spin) {
            __builtin_amdgcn_s_sleep(1);
            ++i;
        }
        if (i >= f.spin) raise_timeout(f);
    }
    __syncthreads();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ uint32_t* line(uint32_t* set, int l) { return set + (int64_t)l * kLineWords; }

// Routed SwiGLU rows landed so far: the sum of the counter's stripes (each workgroup adds to
// stripe b mod kRoutedStripes, so 256 atomics do not queue on one address).  Uniform in the wave.
__device__ __forceinline__ uint32_t routed_rows(uint32_t* set) {
    const int lane = threadIdx.x & 63;
    const uint32_t v = lane < kRoutedStripes ? ld_dev(line(set, kLineRouted + lane)) : 0u;
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kRoutedStripes; ++i) sum += (uint32_t)__builtin_amdgcn_readlane((int)v, i);
    return sum;
}
// Every wave of the workgroup continues once the routed SwiGLU rows have reached `target` and the
// shared expert's counter `sh_target` (bounded).
__device__ __forceinline__ void wait_units(uint32_t* set, uint32_t target, uint32_t sh_target, const Fault& f) {
    if (wave_id() == 0) {
        const int lane = threadIdx.x & 63;
        for (int it = 0;; ++it) {
            const uint32_t rr = routed_rows(set);  // every lane takes part
            bool ok = rr >= target;
            if (lane == 0) ok = ok && ld_dev(line(set, kLineShared)) >= sh_target;
            if (__ballot(!ok) == 0ull) break;
            if (it >= f.spin) {
                if (lane == 0) raise_timeout(f);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Starts an asynchronous copy of n bytes (a multiple of 16) from global memory to LDS with every
// wave of the workgroup.  The data is usable after the issuing waves' next s_waitcnt vmcnt(0) and
// a workgroup barrier.  Instruction i (i KB in) is issued by wave (i + rot) mod 8: a caller that
// copies many small pieces passes the number of instructions issued so far, so the pieces do not
// all start on wave 0.
__device__ __forceinline__ int rot_wave(int rot) { return (wave_id() + kWaves - rot % kWaves) % kWaves; }
__device__ __forceinline__ void async_to_lds(char* lds, const uint8_t* src, int n, int rot = 0) {
    const int lane = threadIdx.x & 63, wave = rot_wave(rot);
    constexpr int chunk = 64 * 16;
    for (int base = wave * chunk; base < n; base += kWaves * chunk) {
        if (base + lane * 16 < n) {
            auto* dst = (LDS void*)(lds + base);
            __builtin_amdgcn_global_load_lds(src + base + lane * 16, dst, 16, 0, 0);
        }
    }
}

// The same with 4-byte pieces, for n bytes (a multiple of 4) from a 4-byte aligned source.
__device__ __forceinline__ void async_dwords_to_lds(char* lds, const uint8_t* src, int n, int rot = 0) {
    const int lane = threadIdx.x & 63, wave = rot_wave(rot);
    constexpr int chunk = 64 * 4;
    for (int base = wave * chunk; base < n; base += kWaves * chunk) {
        if (base + lane * 4 < n) {
            auto* dst = (LDS void*)(lds + base);
            __builtin_amdgcn_global_load_lds(src + base + lane * 4, dst, 4, 0, 0);
        }
    }
}

// The same for nrows rows of rb bytes (a multiple of 16) that land `pitch` bytes apart in LDS.
__device__ __forceinline__ void async_rows_pitch(char* lds, const uint8_t* src, int nrows, int rb, int pitch) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    constexpr int chunk = 64 * 16;
    const int cpr = (rb + chunk - 1) / chunk;  // instructions per row
    for (int c = wave; c < nrows * cpr; c += kWaves) {
        const int row = c / cpr, o = (c - row * cpr) * chunk;
        if (o + lane * 16 < rb) {
            auto* dst = (LDS void*)(lds + (int64_t)row * pitch + o);
            __builtin_amdgcn_global_load_lds(src + (int64_t)row * rb + o + lane * 16, dst, 16, 0, 0);
        }
    }
}

// The same for n bytes of whole rows of rb bytes, with the 16-byte chunks of each row permuted so
// that chunk c of row r lands in slot c ^ chunk_swz(r, rb): lanes that read one chunk position of
// 16 (rows of a multiple of 256 bytes) or 8 (of 128 bytes) consecutive rows then hit different
// bank groups.  Each lane fetches the global chunk that belongs in its slot, so the copy stays one
// 16-byte load per lane.
__host__ __device__ __forceinline__ int chunk_swz(int row, int64_t rb) {
    return (rb & 255) == 0 ? (row & 15) : ((rb & 127) == 0 ? (row & 7) : 0);
}
__device__ __forceinline__ void async_rows_to_lds(char* lds, const uint8_t* src, int n, int rb, int rot = 0) {
    const int lane = threadIdx.x & 63, wave = rot_wave(rot);
    constexpr int chunk = 64 * 16;
    for (int base = wave * chunk; base < n; base += kWaves * chunk) {
        const int o = base + lane * 16;
        if (o < n) {
            const int row = o / rb, c = (o - row * rb) >> 4;
            auto* dst = (LDS void*)(lds + base);
            __builtin_amdgcn_global_load_lds(src + (int64_t)row * rb + 16 * (c ^ chunk_swz(row, rb)), dst, 16, 0, 0);
        }
    }
}

// fp32 logits rows are padded to whole 16-byte chunks
__host__ __device__ __forceinline__ int logit_stride(int E) { return (E + 3) / 4 * 4; }

// Stages `tcount` fp32 SwiGLU rows of K elements (global rows of `stride` floats from `src`) into
// LDS rows of 4 * K bytes with 16-byte device-scope loads, as dot_a reads them (act_mode MODE):
// 0 the fp32 values; 1 the bfloat16 planes hi (K values) then lo (K values); 2 the K values
// rounded to bfloat16 (the rest of the row unused).
template <int MODE>
__device__ __forceinline__ void stage_rows(LDS float* dst, const float* src, int stride, int tcount, int K) {
    const __amdgpu_buffer_rsrc_t r = dev_rsrc(src, (uint32_t)(tcount * stride * 4));
    const int q4 = K / 4, n = tcount * q4;
    for (int i0 = threadIdx.x; i0 < n; i0 += 4 * kThreads) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n) {
                const int t = i / q4, c4 = i - t * q4;
                v[u] = ld_dev16(r, (uint32_t)((t * stride + 4 * c4) * 4));
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n) {
                if constexpr (MODE == 2) {
                    const int t = i / q4, c4 = i - t * q4;
                    LDS char* row = (LDS char*)dst + (int64_t)t * K * 4;
                    *(LDS u32x2*)(row + 8 * c4) =
                        u32x2{(uint32_t)f32_to_bf16_rne(v[u][0]) | ((uint32_t)f32_to_bf16_rne(v[u][1]) << 16),
                              (uint32_t)f32_to_bf16_rne(v[u][2]) | ((uint32_t)f32_to_bf16_rne(v[u][3]) << 16)};
                } else if constexpr (MODE == 1) {
                    const int t = i / q4, c4 = i - t * q4;
                    uint32_t h[4], l[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t bits = __float_as_uint(v[u][e]);
                        h[e] = bits >> 16;
                        l[e] = f32_to_bf16_rne(v[u][e] - __uint_as_float(bits & 0xFFFF0000u));
                    }
                    LDS char* row = (LDS char*)dst + (int64_t)t * K * 4;
                    *(LDS u32x2*)(row + 8 * c4) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                    *(LDS u32x2*)(row + 2 * K + 8 * c4) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
                } else {
                    ((LDS f32x4*)dst)[i] = v[u];
                }
            }
        }
    }
}

// Device-scope (sc1) store of v rounded to bfloat16 (nearest even) at byte byte_off of r.
__device__ __forceinline__ void st_dev_bf16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), r, (int)byte_off, 0, 16 /* sc1 */);
}

// Stages `tcount` bfloat16 SwiGLU rows of K elements (global rows of `stride` elements from `src`)
// into LDS rows of `pitch` bytes with 16-byte device-scope loads.
__device__ __forceinline__ void stage_rows_b16(LDS char* dst, const uint16_t* src, int stride, int tcount, int K,
                                               int pitch) {
    const __amdgpu_buffer_rsrc_t r = dev_rsrc(src, (uint32_t)(tcount * stride * 2));
    const int q8 = K / 8, n = tcount * q8;
    for (int i0 = threadIdx.x; i0 < n; i0 += 4 * kThreads) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n) {
                const int t = i / q8, c8 = i - t * q8;
                v[u] = ld_dev16(r, (uint32_t)((t * stride + 8 * c8) * 2));
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n) {
                const int t = i / q8, c8 = i - t * q8;
                *(LDS f32x4*)(dst + (int64_t)t * pitch + 16 * c8) = v[u];
            }
        }
    }
}

// Stages `tcount` fp32 SwiGLU rows of K elements (global rows of `stride` floats from `src`) into
// LDS as bfloat16 (round to nearest even), rows of `pitch` bytes, with 16-byte device-scope loads.
__device__ __forceinline__ void stage_rows_bf16(LDS char* dst, const float* src, int stride, int tcount, int K,
                                                int pitch) {
    const __amdgpu_buffer_rsrc_t r = dev_rsrc(src, (uint32_t)(tcount * stride * 4));
    const int q4 = K / 4, n = tcount * q4;
    for (int i0 = threadIdx.x; i0 < n; i0 += 4 * kThreads) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n) {
                const int t = i / q4, c4 = i - t * q4;
                v[u] = ld_dev16(r, (uint32_t)((t * stride + 4 * c4) * 4));
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n) {
                const int t = i / q4, c4 = i - t * q4;
                const uint32_t b0 = f32_to_bf16_rne(v[u][0]), b1 = f32_to_bf16_rne(v[u][1]);
                const uint32_t b2 = f32_to_bf16_rne(v[u][2]), b3 = f32_to_bf16_rne(v[u][3]);
                *(LDS u32x2*)(dst + (int64_t)t * pitch + 8 * c4) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// router prologue: RMSNorm of the token rows ("Chasing the Batch-1 Floor", section "PDL:
// stacking the latency floors of small kernels": the router chain norm -> gate matvec -> top-k)
// ------------------------------------------------------------------------------------------

// Token rows xn = bf16(g * (x * r)), r = 1 / sqrt(mean(x^2) + eps), written into the LDS token rows
// that the router and every expert read.  One wave per token: lane l holds the 16-byte chunks
// l + 64 j of the row and of the gain in registers; the sum of squares (each exact in fp32) runs
// in a fixed order per lane and a fixed DPP tree across lanes, so the result does not depend on
// timing.  bfloat16 activations only.
template <int NJ>
__device__ __forceinline__ void rms_norm_rows(const Params& p, LDS char* xs) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int H = p.H, nch = H / 8;
    if (wave >= p.M) return;
    u32x4 g[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) g[j] = *(const u32x4*)((const uint8_t*)p.norm_w + 16 * min(lane + 64 * j, nch - 1));
    for (int m = wave; m < p.M; m += kWaves) {
        const uint8_t* xrow = (const uint8_t*)p.x + (int64_t)m * H * 2;
        u32x4 xv[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) xv[j] = *(const u32x4*)(xrow + 16 * min(lane + 64 * j, nch - 1));
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (lane + 64 * j < nch) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w = xv[j][q];
                    const float a = __uint_as_float(w << 16), c = __uint_as_float(w & 0xFFFF0000u);
                    ss = fmaf(a, a, ss);
                    ss = fmaf(c, c, ss);
                }
            }
        }
        const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_sum_hi(ss)), 63));
        const float r = 1.0f / __builtin_sqrtf(tot / (float)H + p.norm_eps);
        LDS char* dst = xs + (int64_t)m * p.xpitch;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = lane + 64 * j;
            if (c < nch) {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w = xv[j][q], gw = g[j][q];
                    const float a = __uint_as_float(w << 16) * r, b2 = __uint_as_float(w & 0xFFFF0000u) * r;
                    const float ga = __uint_as_float(gw << 16), gb = __uint_as_float(gw & 0xFFFF0000u);
                    o[q] = (uint32_t)f32_to_bf16_rne(ga * a) | ((uint32_t)f32_to_bf16_rne(gb * b2) << 16);
                }
                *(LDS u32x4*)(dst + 16 * c) = o;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// routing: top-k of one token with one wave, batch compaction with one workgroup
// ------------------------------------------------------------------------------------------

// Top-k of one token's E logits with one wave, once every logit of this call has arrived (bounded
// polling on the tags: one read in flight, since M waves of every workgroup poll at once and the
// polls share the saturated memory path; on a timeout the status word is flagged and the selection
// proceeds).  Lane l
// owns experts 8l .. 8l+7, read with four 16-byte device-scope loads.  Order: larger logit first,
// equal logits -> lower expert id first.  Every round takes the wave-wide maximum of the lanes'
// current maxima; among equal maxima the lowest lane holds the lowest id, and inside a lane the
// lowest index is kept, so ties resolve to the lower id.  The winning lane drops that logit and
// recomputes its maximum.  Writes ids, logits and softmax-over-the-k weights in order.  Every id
// written is in [0, E).
// With `early` (one token, no bias): after round r, early[r] holds the r-th selected id and
// early[kMaxTopK] the number of rounds done, so other waves can start on an expert once it is known.
__device__ __forceinline__ void wave_topk(const uint64_t* lrow, int E, int k, uint32_t tag, const Fault& fault,
                                          const float* bias, LDS int* out_id, LDS float* out_w, LDS float* out_v,
                                          volatile LDS int* early = nullptr) {
    const int lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rs = dev_rsrc(lrow, (uint32_t)E * 8);  // loads past E return 0
    // selection bias of the lane's experts, loaded while the logits are polled (past E: 0)
    float bv[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (bias) {
        const __amdgpu_buffer_rsrc_t rb = dev_rsrc(bias, (uint32_t)E * 4);
        const f32x4 b0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (uint32_t)lane * 32, 0, 0));
        const f32x4 b1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (uint32_t)lane * 32 + 16, 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bv[i] = b0[i];
            bv[4 + i] = b1[i];
        }
    }
    float v[8];
    bool gave_up = false;
    for (int it = 0;; ++it) {
        bool ok = true;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const u32x4 q = __builtin_bit_cast(u32x4, ld_dev16(rs, (uint32_t)lane * 64 + 16 * h));
            v[2 * h] = __uint_as_float(q[0]);
            v[2 * h + 1] = __uint_as_float(q[2]);
            ok = ok && (8 * lane + 2 * h >= E || q[1] == tag) && (8 * lane + 2 * h + 1 >= E || q[3] == tag);
        }
        if (__ballot(!ok) == 0ull) break;
        if (it >= fault.spin) {
            if (lane == 0) raise_timeout(fault);
            gave_up = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        asm volatile("" ::: "memory");  // the next iteration reads memory again
    }
    MOE_TRACE(23);
    // Selection.  Each lane sorts its 8 entries once, descending, as 64-bit words (selection key as
    // an order-preserving integer << 32 | 7 - index: larger key first, then the lower index), so a
    // round is one wave maximum of the lanes' heads and a shift in the winning lane (recomputing the
    // winner's maximum instead was a chain of 21 dependent instructions per round).  Equal heads:
    // the lowest lane holds the lowest ids.  Past E: 0, below every real key.  With a bias the raw
    // logits travel with their keys (the weights use them).
    uint64_t c[8];
    float rv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t u = __float_as_uint(v[i] + bv[i]);
        const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        c[i] = 8 * lane + i >= E ? 0ull : ((uint64_t)key << 32) | (uint32_t)(7 - i);
        rv[i] = v[i];
    }
    auto sort8 = [&](auto with_raw) {
        auto ce = [&](int i, int j) {  // c[i] >= c[j] afterwards
            const uint64_t a = c[i], bb = c[j];
            const bool sw = bb > a;
            c[i] = sw ? bb : a;
            c[j] = sw ? a : bb;
            if constexpr (decltype(with_raw)::value) {
                const float ra = rv[i], rb = rv[j];
                rv[i] = sw ? rb : ra;
                rv[j] = sw ? ra : rb;
            }
        };
        ce(0, 2), ce(1, 3), ce(4, 6), ce(5, 7);
        ce(0, 4), ce(1, 5), ce(2, 6), ce(3, 7);
        ce(0, 1), ce(2, 3), ce(4, 5), ce(6, 7);
        ce(2, 4), ce(3, 5);
        ce(1, 4), ce(3, 6);
        ce(1, 2), ce(3, 4), ce(5, 6);
    };
    uint32_t my_key = 0u;  // lane r < k: the selection key of the r-th selected expert
    float my_raw = 0.0f;   // with a bias: its raw logit
    int my_id = 0;
    // The rounds keep each lane's sorted keys as 32-bit words and the entries' indices as nibbles of
    // one word (nibble j: the index of the j-th largest), and pop the winning lane without a branch:
    // every lane selects between its word and the next one, so a round is the wave maximum, two
    // lane reads and a few independent selects (with the 64-bit list shifted inside a branch on the
    // winning lane, a round was about 80 instructions and 4 branches).
    auto rounds = [&](auto with_raw) {
        constexpr bool RAW = decltype(with_raw)::value;
        sort8(with_raw);
        uint32_t key[8], ixw = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            key[i] = (uint32_t)(c[i] >> 32);
            ixw |= ((7u - (uint32_t)c[i]) & 7u) << (4 * i);
        }
        for (int r = 0; r < k; ++r) {
            const uint32_t K = wave_max_u32(key[0]);
            const uint64_t ball = __ballot(key[0] == K);  // never empty: K is one lane's head
            const int wl = __builtin_amdgcn_readfirstlane(ball ? __ffsll((unsigned long long)ball) - 1 : 0);
            const int wi = __builtin_amdgcn_readlane((int)ixw, wl) & 7;
            if (early != nullptr && lane == 0) {
                early[r] = min(8 * wl + wi, E - 1);
                early[kMaxTopK] = r + 1;  // after the id (volatile: in this order)
            }
            const bool mine = lane == r;
            my_key = mine ? K : my_key;
            my_id = mine ? min(8 * wl + wi, E - 1) : my_id;
            if constexpr (RAW)
                my_raw = mine ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rv[0]), wl))
                              : my_raw;
            const bool w = lane == wl;
#pragma unroll
            for (int i = 0; i < 7; ++i) key[i] = w ? key[i + 1] : key[i];
            key[7] = w ? 0u : key[7];
            ixw = w ? ixw >> 4 : ixw;
            if constexpr (RAW) {
#pragma unroll
                for (int i = 0; i < 7; ++i) rv[i] = w ? rv[i + 1] : rv[i];
            }
        }
    };
    if (bias)
        rounds(std::true_type{});
    else
        rounds(std::false_type{});
    float my_v;
    if (bias) {
        my_v = lane < k ? my_raw : -INFINITY;
    } else {  // the key is the logit itself
        const uint32_t u = (my_key & 0x80000000u) ? (my_key & 0x7FFFFFFFu) : ~my_key;
        my_v = lane < k ? __uint_as_float(u) : -INFINITY;
    }
    MOE_TRACE(24);
    // weights: softmax over the k selected logits (lanes 0..k-1 of row 0; k <= 16); without a bias
    // the first selected logit is the largest
    float top;
    if (bias) {
        float t = my_v;  // lanes >= k hold -inf
        t = fmaxf(t, dpp<0xB1>(t));
        t = fmaxf(t, dpp<0x4E>(t));
        t = fmaxf(t, dpp<0x141>(t));
        t = fmaxf(t, dpp<0x140>(t));
        top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), 0));
    } else {
        top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
    }
    const float ex = lane < k ? __expf(my_v - top) : 0.0f;
    const float z = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, row16_sum(ex)), 0));
    // output position: selection order, or with a bias the rank by (logit desc, id asc)
    int pos = lane;
    if (bias) {
        pos = 0;
        for (int j = 0; j < k; ++j) {
            const float vj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), j));
            const int ij = __builtin_amdgcn_readlane(my_id, j);
            pos += (vj > my_v || (vj == my_v && ij < my_id)) ? 1 : 0;
        }
    }
    if (lane < k) {
        out_id[pos] = my_id;
        out_v[pos] = my_v;
        out_w[pos] = gave_up ? __builtin_nanf("") : ex / z;  // NaN weights: every use of this token is invalid
    }
}

// Inclusive prefix sum over the 64 lanes (DPP: shifts inside each 16-lane row, then row
// broadcasts).
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += dpp_rows<0x142, 0xA>(0, v);                                 // row_bcast:15 into rows 1, 3
    v += dpp_rows<0x143, 0xC>(0, v);                                 // row_bcast:31 into rows 2, 3
    return v;
}

// Top-k of all M tokens (each top-k wave waits for its token's logits of this call, tagged `tag`)
// and the batch compaction into this workgroup's LDS tables.  Workgroup 0 (`publish_outputs`)
// also writes the caller-visible routing outputs.  Returns U.
// early, pre (one token without a bias): the selecting wave publishes each round's expert at early
// (see wave_topk) and the other waves run pre() while it selects.
template <typename Pre>
__device__ __forceinline__ int route_and_compact(const Params& p, LDS int* tab, LDS char* sel, bool publish_outputs,
                                                 uint32_t tag, int poll_wave, const Fault& fault,
                                                 volatile LDS int* early, Pre pre) {
    const int E = p.E, M = p.M, k = p.k, NP = M * k;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const bool has_sh = p.Is > 0;
    const float* rbias = (p.router_flags & MOE_ROUTER_BIAS) ? p.rbias : nullptr;
    LDS uint32_t* tokmask = (LDS uint32_t*)sel;              // [kMaxExperts]
    LDS int* offe = (LDS int*)(tokmask + kMaxExperts);       // [kMaxExperts] first pair row of an expert
    LDS int* sid = offe + kMaxExperts;                       // [kMaxTokens * kMaxTopK]
    LDS float* sw = (LDS float*)(sid + kMaxTokens * kMaxTopK);  // [kMaxTokens * kMaxTopK]
    LDS float* sv = sw + kMaxTokens * kMaxTopK;                 // [kMaxTokens * kMaxTopK]
    LDS uint32_t* s_mask = (LDS uint32_t*)tab + kTabMask;
    LDS int* s_off = tab + kTabOff;
    LDS int* s_exp = tab + kTabExp;
    LDS int* s_pair = tab + kTabPair;
    LDS float* s_roww = (LDS float*)(tab + kTabRowW);

    if (!p.route_delegate) {
        for (int m = wave; m < M; m += kWaves)
            wave_topk(p.ws.logits + (int64_t)m * logit_stride(E), E, k, tag, fault, rbias, sid + m * k,
                      sw + m * k, sv + m * k, M == 1 ? early : nullptr);
        if (M == 1 && wave != 0) pre();
    } else {
        // workgroup m < M selects token m's experts and publishes them as tagged words; every
        // workgroup then reads the M * k published (id, weight) pairs instead of M * E logits
        const int b = blockIdx.x;
        if (b < M && wave == 0) {
            wave_topk(p.ws.logits + (int64_t)b * logit_stride(E), E, k, tag, fault, rbias, sid + b * k,
                      sw + b * k, sv + b * k);
            if (lane < k) {
                uint64_t* dst = p.ws.route + 2 * (int64_t)(b * k + lane);
                const uint64_t hi = (uint64_t)tag << 32;
                __hip_atomic_store(dst, hi | (uint32_t)sid[b * k + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + 1, hi | __float_as_uint(sw[b * k + lane]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (wave == poll_wave) {  // pairs q = lane + 64 i, i < 4 (M * k <= 256), written once all are current
            const __amdgpu_buffer_rsrc_t rs = dev_rsrc(p.ws.route, (uint32_t)NP * 16);
            u32x4 v[kMaxTokens * kMaxTopK / 64];
            for (int it = 0;; ++it) {
                bool ok = true;
#pragma unroll
                for (int i = 0; i < kMaxTokens * kMaxTopK / 64; ++i) {
                    const int q = lane + 64 * i;
                    if (q < NP) {
                        v[i] = __builtin_bit_cast(u32x4, ld_dev16(rs, (uint32_t)q * 16));
                        ok = ok && v[i][1] == tag && v[i][3] == tag;
                    }
                }
                if (__ballot(!ok) == 0ull) {
#pragma unroll
                    for (int i = 0; i < kMaxTokens * kMaxTopK / 64; ++i) {
                        const int q = lane + 64 * i;
                        if (q < NP) {
                            sid[q] = min((int)v[i][0], E - 1);
                            sw[q] = __uint_as_float(v[i][2]);
                        }
                    }
                    break;
                }
                if (it >= fault.spin) {
                    if (lane == 0) raise_timeout(fault);
                    for (int q = lane; q < NP; q += 64) {  // the routing is invalid: NaN weights
                        sid[q] = 0;
                        sw[q] = __builtin_nanf("");
                    }
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                asm volatile("" ::: "memory");  // the next iteration reads memory again
            }
        }
    }
    if (M > 1) __syncthreads();  // one token: wave 0 selected it and builds the tables below
    MOE_TRACE(13);
    if (wave == 0 && M == 1) {
        // one token: unit j is the j-th selected expert and pair j its row.  Every workgroup takes
        // the same order and the combine sums by selection slot, so no ranking is needed here (the
        // ranks by id, once a barrier and a dependent loop on this path, are taken only where the
        // dispatch tables are written).  This wave wrote the selection; its LDS operations complete
        // in order.
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (lane < k) {
            s_mask[lane] = 1u;
            s_off[lane] = lane;
            s_exp[lane] = min(max(sid[lane], 0), E - 1);
            s_pair[lane] = lane;
            s_roww[lane] = sw[lane];
        }
        if (lane == 0) {
            s_mask[k] = has_sh ? 1u : 0u;
            s_off[k] = k;
            s_off[k + 1] = k + (has_sh ? 1 : 0);
            s_exp[k] = E;
            tab[kTabMisc] = k;
            s_roww[k] = 1.0f;
        }
    } else if (wave == 0) {
        // token bitmask of every expert (one wave: its LDS operations complete in order)
        for (int e = lane; e < kMaxExperts; e += 64) tokmask[e] = 0u;
        for (int q = lane; q < NP; q += 64) atomicOr((uint32_t*)&tokmask[sid[q]], 1u << (q / k));
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // lane l owns experts 8l .. 8l+7, so ascending ids are lane-major
        const u32x4 ta = ((const LDS u32x4*)tokmask)[2 * lane], tb = ((const LDS u32x4*)tokmask)[2 * lane + 1];
        const uint32_t tm[8] = {ta[0], ta[1], ta[2], ta[3], tb[0], tb[1], tb[2], tb[3]};
        int npres = 0, nrows = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            npres += tm[i] ? 1 : 0;
            nrows += __popc(tm[i]);
        }
        // one scan of (units << 16 | pair rows): both stay below 2^16
        const int packed = (npres << 16) | nrows;
        const int incl = wave_incl_scan(packed);
        const int excl = incl - packed;
        const int U = __builtin_amdgcn_readlane(incl, 63) >> 16;
        int u = excl >> 16;       // first unit index of this lane
        int off = excl & 0xFFFF;  // first pair row of this lane
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = 8 * lane + i;
            if (tm[i]) {
                s_mask[u] = tm[i];
                s_off[u] = off;
                s_exp[u] = e;
                offe[e] = off;
                ++u;
                off += __popc(tm[i]);
            }
        }
        if (lane == 0) {
            s_mask[U] = has_sh ? ((1u << M) - 1u) : 0u;
            s_off[U] = NP;
            s_off[U + 1] = NP + (has_sh ? M : 0);
            s_exp[U] = E;
            tab[kTabMisc] = U;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        for (int q = lane; q < NP; q += 64) {
            const int m = q / k, ex = sid[q];
            const int row = offe[ex] + __popc(tokmask[ex] & ((1u << m) - 1u));
            s_pair[q] = row;
            s_roww[row] = sw[q];
        }
        for (int m = lane; m < M; m += 64) s_roww[NP + m] = 1.0f;
    }
    __syncthreads();
    MOE_TRACE(14);
    const int U = tab[kTabMisc];

    if (publish_outputs) {
        // the caller's tables list the units by ascending expert id; one token keeps its units in
        // selection order internally, so unit (and row) u is written at its rank by id (ties: slot),
        // kept in the compaction's scratch (unused at one token)
        LDS int* rk = offe;
        if (M == 1) {
            const int u = threadIdx.x;
            if (u < k) {
                int rank = 0;
                for (int j = 0; j < k; ++j) rank += (s_exp[j] < s_exp[u] || (s_exp[j] == s_exp[u] && j < u)) ? 1 : 0;
                rk[u] = rank;
            }
            __syncthreads();
        }
        auto ro = [&](int u) { return M == 1 && u < k ? rk[u] : u; };
        for (int q = threadIdx.x; q < NP; q += kThreads) {
            const int row = ro(s_pair[q]);
            if (p.topk_ids) p.topk_ids[q] = sid[q];
            if (p.topk_w) p.topk_w[q] = sw[q];
            if (p.disp.row_token) p.disp.row_token[row] = q / k;
            if (p.disp.row_slot) p.disp.row_slot[row] = q % k;
            if (p.disp.row_weight) p.disp.row_weight[row] = sw[q];
        }
        for (int u = threadIdx.x; u < U + (has_sh ? 1 : 0); u += kThreads) {
            const int ru = ro(u);  // one token: the unit's first row is its own index, u
            if (p.disp.unit_expert) p.disp.unit_expert[ru] = s_exp[u];
            if (p.disp.unit_off) p.disp.unit_off[ru] = M == 1 ? ru : s_off[u];
        }
        if (threadIdx.x == 0) {
            if (p.disp.unit_count) *p.disp.unit_count = U;
            if (p.disp.unit_off) p.disp.unit_off[U + (has_sh ? 1 : 0)] = s_off[U + (has_sh ? 1 : 0)];
        }
        if (has_sh) {
            for (int m = threadIdx.x; m < M; m += kThreads) {
                if (p.disp.row_token) p.disp.row_token[NP + m] = m;
                if (p.disp.row_slot) p.disp.row_slot[NP + m] = k;
                if (p.disp.row_weight) p.disp.row_weight[NP + m] = 1.0f;
            }
        }
        // packed-request offsets: validate, and count distinct routed experts per request
        if (p.req_off) {
            __shared__ int s_bad;
            __shared__ int s_req_unique[kMaxTokens];
            if (threadIdx.x == 0) {
                int bad = (p.R < 1 || p.req_off[0] != 0 || p.req_off[p.R] != M) ? 1 : 0;
                for (int r = 0; r < p.R && !bad; ++r) bad = p.req_off[r + 1] < p.req_off[r];
                s_bad = bad;
                if (bad) atomicOr(p.ws.hdr + kHdrStatus, kStatusOffsets);
            }
            if (threadIdx.x < kMaxTokens) s_req_unique[threadIdx.x] = 0;
            __syncthreads();
            if (!s_bad && p.disp.req_unique) {
                for (int r = 0; r < p.R; ++r) {
                    const int a = p.req_off[r], b = p.req_off[r + 1];
                    if (M == 1) {  // no token bitmasks: the one token's U experts, in the request holding it
                        if (threadIdx.x == 0 && a == 0 && b >= 1) s_req_unique[r] = U;
                        continue;
                    }
                    const uint32_t rm = ((1u << b) - 1u) & ~((1u << a) - 1u);
                    for (int i = threadIdx.x; i < E; i += kThreads)
                        if (tokmask[i] & rm) atomicAdd(&s_req_unique[r], 1);
                }
                __syncthreads();
                for (int r = threadIdx.x; r < p.R; r += kThreads) p.disp.req_unique[r] = s_req_unique[r];
            }
        }
        __syncthreads();
    }
    return U;
}

// ------------------------------------------------------------------------------------------
// streaming GEMV pieces
// ------------------------------------------------------------------------------------------

// Router rows [e0, e1): one wave per row, every token.  Each logit goes out as one 64-bit
// device-scope store of its fp32 bits and `tag` (the call index + 1), so a reader that sees the tag
// sees the value: no acknowledgement wait and no separate arrival flag.  Each wave's first row was
// loaded before the token rows landed in LDS (`first`).  The weight is in
// the activation format, so its geometry is the gate/up geometry of that format.
template <int AF, int NJ>
__device__ __forceinline__ void router_rows(const Params& p, const LDS char* xs, int e0, int e1, const Chunk (&first)[NJ],
                                            uint32_t tag) {
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    const int H = p.H, E = p.E, M = p.M;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int nch = H / Geo<AF>::EPC;
    for (int e = e0 + wave; e < e1; e += kWaves) {
        Chunk r[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (e == e0 + wave)
                r[j] = first[j];
            else
                ld_chunk<AF>(r[j], (const uint8_t*)p.wr + (int64_t)e * H * XB, nullptr, min(lane + 64 * j, nch - 1));
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) settle_mask<AF>(r[j], lane + 64 * j < nch);
        for (int m = 0; m < M; ++m) {
            const LDS char* xrow = xs + (int64_t)m * p.xpitch;
            float acc[kAcc] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < NJ; ++j) dot_x<AF, AF>(r[j], xrow, min(lane + 64 * j, nch - 1), acc);
            const float s = wave_sum_hi(acc_sum(acc));
            if (lane == 63)
                __hip_atomic_store(p.ws.logits + (int64_t)m * logit_stride(E) + e,
                                   ((uint64_t)tag << 32) | __float_as_uint(s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// One gate/up task: RT consecutive rows of a unit's gate and up matrices, applied to the unit's
// tokens.  Pointers are at the task's first row.
struct GUTask {
    const uint8_t* g;
    const uint8_t* u;
    const uint8_t* gs;  // block scales of those rows (scale_row of the first row; the rows of an FP8
                        // task lie in one 128-row block and share it)
    const uint8_t* us;
    uint32_t mask;      // the unit's tokens
    int slot;           // staging row of the task's first row
    int dummy;          // 1: a stand-in for the prefetch after the last task (one chunk, every lane)
};

// This wave's gate/up tasks, in the order next(0), next(1), ... until next returns -1 (called once
// per position, in order, one position ahead of the compute).  info(q, s, task) describes task q
// at position s.  out(r, i, v) receives silu(g) * v of the task's row r - t.slot and the unit's
// i-th token (in the row's last lane).  Each wave keeps the next task's loads in flight while it
// computes the current one; the prefetch is unconditional (the last task re-reads itself) so the
// number of loads in flight is static and the compiler waits for exactly the task it needs.
// Returns the number of tasks computed.
// The loads of one gate/up task into this wave's chunk registers (a stand-in task: one chunk).
template <int WF, int NJ>
__device__ __forceinline__ void gateup_load(int H, Chunk (&g)[Geo<WF>::RL_G][NJ], Chunk (&u)[Geo<WF>::RL_G][NJ],
                                            const GUTask& t) {
    constexpr int LPR = Geo<WF>::LPR_G, RL = Geo<WF>::RL_G;
    const int lane = threadIdx.x & 63, gi = lane / LPR, sl = lane % LPR;
    const int nch = H / Geo<WF>::EPC;
    const int64_t rb = row_bytes<WF>(H), sb = H / 32;
#pragma unroll
    for (int rl = 0; rl < RL; ++rl) {
        const int64_t ro = t.dummy ? 0 : gi * RL + rl;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = t.dummy ? 0 : min(sl + LPR * j, nch - 1);
            ld_chunk<WF>(g[rl][j], t.g + ro * rb, WF == MOE_FMT_FP8 ? t.gs : t.gs + ro * sb, c);
            ld_chunk<WF>(u[rl][j], t.u + ro * rb, WF == MOE_FMT_FP8 ? t.us : t.us + ro * sb, c);
        }
    }
}

// (pre: the first task's loads were issued into ga / ua before the call, by gateup_load)
template <int AF, int WF, int NJ, typename Next, typename Info, typename Out>
__device__ __forceinline__ int gateup_seq(const Params& p, const LDS char* xs, Next next, Info info, Out out,
                                          Chunk (&ga)[Geo<WF>::RL_G][NJ], Chunk (&ua)[Geo<WF>::RL_G][NJ],
                                          bool pre = false) {
    constexpr int LPR = Geo<WF>::LPR_G, RL = Geo<WF>::RL_G;
    const int lane = threadIdx.x & 63, gi = lane / LPR, sl = lane % LPR;
    const int H = p.H;
    const int nch = H / Geo<WF>::EPC;
    static_assert(WF != MOE_FMT_FP8 || kFp8Block % rt_gate<WF>() == 0, "an FP8 gate/up task lies in one row block");
    int q = next(0);
    if (q < 0) return 0;
    Chunk gb[RL][NJ], ub[RL][NJ];
    GUTask ta, tb;
    auto load = [&](Chunk(&g)[RL][NJ], Chunk(&u)[RL][NJ], const GUTask& t) { gateup_load<WF, NJ>(H, g, u, t); };
    auto settle_all = [&](Chunk(&g)[RL][NJ], Chunk(&u)[RL][NJ]) {
#pragma unroll
        for (int rl = 0; rl < RL; ++rl)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                settle_mask<WF>(g[rl][j], sl + LPR * j < nch);
                settle_mask<WF>(u[rl][j], sl + LPR * j < nch);
            }
    };
    auto compute = [&](Chunk(&g)[RL][NJ], Chunk(&u)[RL][NJ], const GUTask& t) {
        int i = 0;
        for (uint32_t m = t.mask; m; m &= m - 1u, ++i) {
            const int tok = __builtin_ctz(m);
            if constexpr (WF == MOE_FMT_MXFP4) {
                // keep the E2M1 decode inside the token loop: hoisted, the decoded rows of a task
                // would need 160 registers
#pragma unroll
                for (int rl = 0; rl < RL; ++rl)
#pragma unroll
                    for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(g[rl][j].q), "+v"(u[rl][j].q));
            }
            const LDS char* xrow = xs + (int64_t)tok * p.xpitch;
            float ag[RL][kAcc], au[RL][kAcc];
#pragma unroll
            for (int rl = 0; rl < RL; ++rl)
#pragma unroll
                for (int q = 0; q < kAcc; ++q) ag[rl][q] = au[rl][q] = 0.0f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c = min(sl + LPR * j, nch - 1);
#pragma unroll
                for (int rl = 0; rl < RL; ++rl) {
                    dot_x<AF, WF>(g[rl][j], xrow, c, ag[rl]);
                    dot_x<AF, WF>(u[rl][j], xrow, c, au[rl]);
                }
                if constexpr (WF == MOE_FMT_MXFP4) __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int rl = 0; rl < RL; ++rl) {
                const float gs = group_sum<LPR>(acc_sum(ag[rl]));
                const float us = group_sum<LPR>(acc_sum(au[rl]));
                if (sl == LPR - 1) out(t.slot + gi * RL + rl, i, silu_mul(gs, us));
            }
        }
    };
    // the prefetch after the last task stays unconditional (a static number of loads in flight) but
    // reads one chunk of the current task's first row in every lane: one cache line, not a task
    int s = 0;
    info(q, 0, ta);
    ta.dummy = 0;
    if (!pre) load(ga, ua, ta);
    MOE_TRACE(16);
    while (true) {
        const int qb = next(s + 1);
        info(qb >= 0 ? qb : q, s + 1, tb);
        tb.dummy = qb < 0;
        load(gb, ub, tb);
        settle_all(ga, ua);
        if (s == 0) MOE_TRACE(17);
        compute(ga, ua, ta);
        ++s;
        if (qb < 0) break;
        const int qa = next(s + 1);
        info(qa >= 0 ? qa : qb, s + 1, ta);
        ta.dummy = qa < 0;
        load(ga, ua, ta);
        settle_all(gb, ub);
        if (s == 1) MOE_TRACE(18);
        compute(gb, ub, tb);
        ++s;
        if (qa < 0) break;
        q = qa;
    }
    MOE_TRACE(19);
    return s;
}

// The static form: local tasks i = wslot, wslot + kWaves, ... < n; info(i, task) describes task i.
template <int AF, int WF, int NJ, typename Info, typename Out>
__device__ __forceinline__ void gateup_run(const Params& p, const LDS char* xs, int n, int wslot, Info info, Out out) {
    Chunk g[Geo<WF>::RL_G][NJ], u[Geo<WF>::RL_G][NJ];
    gateup_seq<AF, WF, NJ>(
        p, xs, [&](int s) { return wslot + kWaves * s < n ? wslot + kWaves * s : -1; },
        [&](int i, int, GUTask& t) { info(i, t); }, out, g, u);
}

// Routed gate/up rows on the matrix cores, for MXFP4 weights in slice mode from three tokens on (a
// wave has a few (tile, stage) items, and whole 10 KB items issued at once beat the line-wise
// stages of gateup_mfma below there; at one token the line-wise form is faster).  The workgroup's tasks are nloc
// tiles of 8 consecutive rows of the flattened (unit, row) list (local tile i = rows 8 (b + i G) ..
// + 7), dealt to its waves round robin.  A tile is one 16-row A operand: the 8 gate rows (A rows
// 0..7) and the same 8 up rows (A rows 8..15).
// B holds the rows x of all M tokens (column n = token n, whichever unit the row belongs to), so a
// chain of v_mfma_f32_16x16x32_bf16 gives g and v of the 8 rows for every token and each E2M1 code
// is decoded once, not once per token.  Operand layout of the instruction: lane l holds A[l % 16][8
// (l / 16) + 0..7], B[8 (l / 16) + 0..7][l % 16] and D[4 (l / 16) + 0..3][l % 16].  Lane (r, kq) =
// (l % 16, l / 16) owns whole MX blocks 4q + kq of its row (16 bytes of codes and the block's scale
// byte) and feeds elements 8m .. 8m + 7 of the block to the m-th product of block group q; B lane
// (n, kq) holds the same elements of token n's row.  Stages of NQ block groups are double-buffered
// (the last one re-read, so the number of loads in flight is static).  Blocks past H are zeroed.
// silu(g) * v of row 8 (b + i G) + s of local tile i and the unit's n-th token goes to
// cst[(8 i + s) * M + n].
// With `part` (LDS, nloc * nstage * 16 * M floats) the work items are (tile, stage) pairs instead of
// tiles, dealt to the waves round robin: every wave carries about the same bytes even when a
// workgroup has few tiles (9 tiles of 2 stages on 8 waves: 3 stages at most per wave, not 4).  Each
// item's partial g and v go to `part`; after a barrier the stages of a tile are summed in stage
// order and silu(g) * v is staged as above.  Every wave of the workgroup must call this.
template <int NQ, bool WIDE>
__device__ __forceinline__ void gateup_mfma_mx(const Params& p, const LDS char* xs, int nloc,
                                               const LDS uint32_t* s_mask, const LDS int* s_exp, LDS float* cst,
                                               LDS float* part) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r = lane & 15, kq = lane >> 4;
    const int H = p.H, I = p.I, M = p.M, G = gridDim.x, b = blockIdx.x;
    const int nblk = H / 32, nquad = (nblk + 3) / 4, nstage = (nquad + NQ - 1) / NQ;
    const int64_t rb = H / 2, sb = H / 32;
    const bool ks = part != nullptr;
    // this wave's steps: items wave, wave + kWaves, ... (split), or all stages of tiles wave,
    // wave + kWaves, ...
    const int nsteps = ks ? n_strided(nloc * nstage, wave, kWaves) : n_strided(nloc, wave, kWaves) * nstage;
    const uint8_t* mat = r < 8 ? (const uint8_t*)p.w.gate : (const uint8_t*)p.w.up;
    const uint8_t* mats = r < 8 ? p.w.gate_s : p.w.up_s;
    auto row_mask = [&](int64_t f) -> uint32_t { return s_mask[(int)f / I]; };  // the unit's tokens
    const LDS char* xrow = xs + (int64_t)min(r, M - 1) * p.xpitch;  // columns past M are dropped
    // local tile and stage of this wave's step t; a local tile's first flat row and staging slot
    auto tile_of = [&](int t, int& i, int& sg) {
        if (ks) {
            const int k = wave + kWaves * t;
            i = k / nstage;
            sg = k - i * nstage;
        } else {
            i = wave + kWaves * (t / nstage);
            sg = t - (t / nstage) * nstage;
        }
    };
    auto tile_row = [&](int i) { return (int64_t)(b + i * G) * 8; };
    auto tile_slot = [&](int i) { return i * 8; };
    // A stage's scale bytes: blocks 4 NQ sg .. 4 NQ sg + 4 NQ - 1 of the row.  When the rows' scale
    // bytes are 16-byte aligned (H a multiple of 512) they come as NS 16-byte loads from the
    // aligned dword (NQ sg) & ~3 on, and block 4 (NQ sg + q) + kq is byte kq of dword
    // ((NQ sg) & 3) + q; otherwise one byte load per block.
    constexpr int NS = (NQ + 3 + 3) / 4;
    struct Stage {
        u32x4 c[NQ];
        uint32_t s[WIDE ? 4 * NS : NQ];
    };
    // t == nsteps: the stand-in prefetch after the last stage (static loads in flight): every lane
    // reads the first block of the last tile's first row, one cache line
    auto load = [&](Stage& st, int t) {
        const bool dummy = t >= nsteps;
        t = min(t, nsteps - 1);
        int j, sg;
        tile_of(t, j, sg);
        const int64_t f = tile_row(j) + (dummy ? 0 : (r & 7));
        const int u = (int)f / I;
        const int64_t row = (int64_t)s_exp[u] * I + (f - (int64_t)u * I);
        const uint8_t* w = (dummy ? (const uint8_t*)p.w.gate : mat) + row * rb;
        const uint8_t* sc = (dummy ? p.w.gate_s : mats) + row * sb;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int bc = dummy ? 0 : min(4 * (NQ * sg + q) + kq, nblk - 1);
            st.c[q] = __builtin_nontemporal_load((const u32x4*)(w + 16 * bc));
        }
        if constexpr (WIDE) {
            const int d0 = (NQ * sg) & ~3;  // first dword of the stage's scales, 16-byte aligned
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int o = dummy ? 0 : min(4 * d0 + 16 * i, (int)sb - 16);  // in the row (a clamped load is never used)
                const u32x4 v = __builtin_nontemporal_load((const u32x4*)(sc + o));
                st.s[4 * i] = v[0];
                st.s[4 * i + 1] = v[1];
                st.s[4 * i + 2] = v[2];
                st.s[4 * i + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int bc = min(4 * (NQ * sg + q) + kq, nblk - 1);
                st.s[q] = __builtin_nontemporal_load(sc + bc);
            }
        }
    };
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
    auto compute = [&](Stage& st, int t) {
        int j, sg;
        tile_of(t, j, sg);
#pragma unroll
        for (int q = 0; q < NQ; ++q) asm volatile("" : "+v"(st.c[q]));
        if (t == 0) MOE_TRACE(17);
        if (t == 1) MOE_TRACE(18);
#pragma unroll
        for (int i = 0; i < (WIDE ? 4 * NS : NQ); ++i) asm volatile("" : "+v"(st.s[i]));
        const int sh = (NQ * sg) & 3;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int blk = 4 * (NQ * sg + q) + kq;
            const bool valid = blk < nblk;
            uint32_t sbyte;
            if constexpr (WIDE) {
                const uint32_t dw = sh == 0 ? st.s[q] : (sh == 1 ? st.s[q + 1] : (sh == 2 ? st.s[q + 2] : st.s[q + 3]));
                sbyte = (dw >> (8 * kq)) & 0xFFu;
            } else {
                sbyte = st.s[q];
            }
            const float sc = e8m0_to_f32(valid ? sbyte : 127u);
            const u32x4 c = valid ? st.c[q] : u32x4{0u, 0u, 0u, 0u};
            const LDS char* xp = xrow + 64 * min(blk, nblk - 1);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const bf16x8 bop = *(const LDS bf16x8*)(xp + 16 * m);
                const uint32_t wd = c[m];
                const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 0);
                const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 1);
                const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 2);
                const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 3);
                const bf16x8 aop = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                if (m & 1)
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop, acc1, 0, 0, 0);
                else
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop, acc0, 0, 0, 0);
            }
        }
        if (ks) {  // item done: its partial g (rows 0..7) and v (rows 8..15) of the M tokens to part
            if (r < M) *(LDS f32x4*)(part + (((int64_t)(j * nstage + sg) * 4 + kq) * M + r) * 4) = acc0 + acc1;
            acc0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            acc1 = acc0;
        } else if (sg == nstage - 1) {  // tile j done: lanes kq < 2 hold g of rows 4 kq + i, lanes kq + 2 their v
            const f32x4 d = acc0 + acc1;
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __shfl_xor(d[i], 32);
            if (kq < 2 && r < M) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t mk = row_mask(tile_row(j) + 4 * kq + i);
                    if ((mk >> r) & 1u)
                        cst[(tile_slot(j) + 4 * kq + i) * M + __popc(mk & ((1u << r) - 1u))] = silu_mul(d[i], v[i]);
                }
            }
            acc0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            acc1 = acc0;
        }
    };
    if (nsteps > 0) {
        Stage sa, sb2;
        load(sa, 0);
        MOE_TRACE(16);
        int t = 0;
        while (true) {
            load(sb2, t + 1);
            compute(sa, t);
            if (++t >= nsteps) break;
            load(sa, t + 1);
            compute(sb2, t);
            if (++t >= nsteps) break;
        }
    }
    MOE_TRACE(19);
    if (ks) {  // sum each tile's stages in stage order, then silu(g) * v for the unit's tokens
        __syncthreads();
        for (int idx = threadIdx.x; idx < nloc * 8 * M; idx += kThreads) {
            const int i = idx / (8 * M), rem = idx - i * 8 * M;
            const int jr = rem / M, n = rem - jr * M;
            float g = 0.0f, v = 0.0f;
            for (int sg = 0; sg < nstage; ++sg) {
                const LDS float* pp = part + (int64_t)(i * nstage + sg) * 4 * M * 4;
                g += pp[((jr >> 2) * M + n) * 4 + (jr & 3)];
                v += pp[((2 + (jr >> 2)) * M + n) * 4 + (jr & 3)];
            }
            const uint32_t mk = row_mask(tile_row(i) + jr);
            if ((mk >> n) & 1u) cst[(tile_slot(i) + jr) * M + __popc(mk & ((1u << n) - 1u))] = silu_mul(g, v);
        }
    }
}

// Routed gate/up rows on the matrix cores, for MXFP4 and FP8 weights.  The
// workgroup's tasks are nloc tiles of 8 consecutive rows of the flattened (unit, row) list (local
// tile i = rows 8 (b + i G) .. + 7).  A tile is one 16-row A operand: the 8 gate rows (A rows 0..7)
// and the same 8 up rows (A rows 8..15).  B holds the rows x of all M tokens (column n = token n,
// whichever unit the row belongs to), so a chain of v_mfma_f32_16x16x32_bf16 gives g and v of the
// 8 rows for every token and each code is decoded once, not once per token.  Operand layout of
// the instruction: lane l holds A[l % 16][8 (l / 16) + 0..7], B[8 (l / 16) + 0..7][l % 16] and
// D[4 (l / 16) + 0..3][l % 16].
//
// A tile streams in stages of 256 bytes per row.  A stage is four loads, each lane 16 bytes, four A
// rows of 256 contiguous bytes per instruction (the operand layout itself, 16 rows of 64 bytes per
// instruction, streamed at 2.5-3.5 TB/s here).  It goes through a 4 KB LDS buffer of the wave's
// own: chunk c of A row a is stored at slot c ^ a, and lane (r, kq) reads chunks 4 j + kq (j =
// 0..3) of A row r (the 16 lanes of one chunk position hit 16 different bank groups).  R - 1 stages
// are in flight while one is computed.
//   MXFP4: a chunk is one MX block (32 codes) and its E8M0 scale byte, decoded with
// v_cvt_scalef32_pk_bf16_fp4; elements 8 m .. 8 m + 7 feed product m, and B lane (n, kq) holds the
// same elements of token n's row.
//   FP8: a chunk is 16 E4M3 codes, decoded exactly to bfloat16 (scale 1) and fed to two products
// (elements 8 h .. 8 h + 7).  Chunks j = 0, 1 and j = 2, 3 of a stage lie in its two 128-column
// blocks: each pair's products go to a fresh accumulator that joins the running sum times the
// block's scale for the lane's D rows (rows 0..7: the gate rows' 128-row block, 8..15: the up
// rows'; the 8 rows of a tile lie in one 128-row block).
// Chunks past the end of a row are loaded from the row's last chunk and zeroed.
//
// With `part` the workgroup's nloc * nstage (tile, stage) steps are split into 8 contiguous ranges,
// one per wave, so the waves carry the same bytes to within one stage.  A tile inside one wave's
// range is finished there; a tile cut by range boundaries leaves a partial sum per wave (at most the
// first and the last tile of a range: `part`, 2 * M * 64 bytes per wave), added in wave (= stage)
// order after a barrier.  Without it (no LDS to spare: many tokens and tiles) whole tiles go to the
// waves round robin.  silu(g) * v of row 8 (b + i G) + s of local tile i and the unit's n-th token
// goes to cst[(8 i + s) * M + n].  trb: kWaves LDS buffers of 4 KB.  Every wave of the workgroup
// must call this.
template <int WF>
__device__ __forceinline__ void gateup_mfma(const Params& p, const LDS char* xs, int nloc,
                                            const LDS uint32_t* s_mask, const LDS int* s_exp, LDS float* cst,
                                            LDS float* part, LDS char* trb) {
    static_assert(WF == MOE_FMT_MXFP4 || WF == MOE_FMT_FP8, "4- and 8-bit weights");
    constexpr bool MX = WF == MOE_FMT_MXFP4;
    constexpr int R = 4;  // stages in flight per wave (VGPR ring)
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r = lane & 15, kq = lane >> 4;
    const int H = p.H, I = p.I, M = p.M, G = gridDim.x, b = blockIdx.x;
    const int64_t rb = MX ? H / 2 : H;           // bytes of a row
    const int nch = (int)(rb / 16);              // 16-byte chunks of a row
    const int nstage = (nch + 15) / 16;          // stages of 16 chunks
    const int64_t sb = H / 32;                   // MXFP4: scale bytes of a row
    const bool WIDE = sb % 16 == 0;              // MXFP4: a stage's scale bytes are one aligned 16-byte load
    const int nsb = H / kFp8Block;               // FP8: column blocks of a row
    const bool split = part != nullptr;
    const int T = nloc * nstage;
    // this wave's steps: [a0, a0 + nsteps) of the workgroup's, or all stages of tiles wave, wave + 8, ...
    const int a0 = split ? T * wave / kWaves : 0;
    const int nsteps = split ? T * (wave + 1) / kWaves - a0 : n_strided(nloc, wave, kWaves) * nstage;
    auto step_of = [&](int t, int& i, int& sg) {
        if (split) {
            const int g = a0 + t;
            i = g / nstage;
            sg = g - i * nstage;
        } else {
            i = wave + kWaves * (t / nstage);
            sg = t - (t / nstage) * nstage;
        }
    };
    LDS char* tb = trb + wave * 4096;
    const uint8_t* gmat = (const uint8_t*)p.w.gate;
    const uint8_t* umat = (const uint8_t*)p.w.up;
    const uint8_t* gsc = p.w.gate_s;
    const uint8_t* usc = p.w.up_s;
    auto row_mask = [&](int64_t f) -> uint32_t { return s_mask[(int)f / I]; };  // the unit's tokens
    // expert and row within it of flat row f
    auto locate = [&](int64_t f, int64_t& e, int64_t& rl) {
        const int u = (int)f / I;
        e = s_exp[u];
        rl = f - (int64_t)u * I;
    };
    const LDS char* xrow = xs + (int64_t)min(r, M - 1) * p.xpitch;  // columns past M are dropped
    auto tile_row = [&](int i) { return (int64_t)(b + i * G) * 8; };
    auto tile_slot = [&](int i) { return i * 8; };
    struct Stage {
        u32x4 c[4];  // instruction i: A row 4 i + kq, chunk 16 sg + r
        u32x4 s;     // MXFP4: scale bytes of blocks 16 sg .. + 15 of A row r (WIDE; else the bytes of
                     // blocks 16 sg + 4 j + kq in s[j]); FP8: s[0], s[1] = the stage's two block
                     // scales for the lane's D rows
    };
    // t >= nsteps: the stand-in prefetch after the last step (a static number of loads in flight):
    // every lane reads the first chunk of the last step's first row, one cache line
    auto load = [&](Stage& st, int t) {
        const bool dummy = t >= nsteps;
        int i, sg;
        step_of(min(t, nsteps - 1), i, sg);
        const int64_t f0 = tile_row(i);
        const int ch = dummy ? 0 : min(16 * sg + r, nch - 1);
        int64_t e, rl;  // the tile's 8 rows lie in one unit: rows rl .. rl + 7 of expert e
        locate(f0, e, rl);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int a = dummy ? 0 : 4 * q + kq;
            st.c[q] = __builtin_nontemporal_load(
                (const u32x4*)((a < 8 ? gmat : umat) + (e * I + rl + (a & 7)) * rb + 16 * ch));
        }
        if constexpr (MX) {
            const uint8_t* sc = (r < 8 || dummy ? gsc : usc) + (e * I + rl + (dummy ? 0 : (r & 7))) * sb;
            if (WIDE) {
                st.s = __builtin_nontemporal_load((const u32x4*)(sc + (dummy ? 0 : 16 * sg)));
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) st.s[q] = sc[dummy ? 0 : min(16 * sg + 4 * q + kq, (int)sb - 1)];
            }
        } else {
            const float* srow = (const float*)scale_row<WF>(scale_mat<WF>(kq < 2 || dummy ? gsc : usc, e, I, H), rl, H);
            st.s[0] = __float_as_uint(srow[dummy ? 0 : min(2 * sg, nsb - 1)]);
            st.s[1] = __float_as_uint(srow[dummy ? 0 : min(2 * sg + 1, nsb - 1)]);
            st.s[2] = st.s[3] = 0u;
        }
    };
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
    const int i0 = a0 / nstage;  // the first tile of this wave's range
    auto compute = [&](Stage& st, int t) {
        int i, sg;
        step_of(t, i, sg);
#pragma unroll
        for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(st.c[q]));
        asm volatile("" : "+v"(st.s));
        if (t == 0) MOE_TRACE(17);
        if (t == 1) MOE_TRACE(18);
        // the stage into the operand layout, through this wave's LDS buffer
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int a = 4 * q + kq;
            *(LDS u32x4*)(tb + a * 256 + 16 * (r ^ a)) = st.c[q];
        }
        asm volatile("" ::: "memory");  // a wave's LDS operations complete in order
        u32x4 av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) av[q] = *(const LDS u32x4*)(tb + r * 256 + 16 * ((4 * q + kq) ^ r));
        asm volatile("" ::: "memory");
        if constexpr (MX) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int blk = 16 * sg + 4 * q + kq;  // MX block of the row
                const bool valid = blk < nch;
                const uint32_t sbyte = WIDE ? (st.s[q] >> (8 * kq)) & 0xFFu : st.s[q];
                const float sc = e8m0_to_f32(valid ? sbyte : 127u);
                const u32x4 c = valid ? av[q] : u32x4{0u, 0u, 0u, 0u};
                const LDS char* xp = xrow + 64 * min(blk, nch - 1);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bf16x8 bop = *(const LDS bf16x8*)(xp + 16 * m);
                    const uint32_t wd = c[m];
                    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 0);
                    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 1);
                    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 2);
                    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 3);
                    const bf16x8 aop = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                    if (m & 1)
                        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop, acc1, 0, 0, 0);
                    else
                        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop, acc0, 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {  // column block 2 sg + hb: chunks q = 2 hb, 2 hb + 1
                f32x4 tmp = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int qq = 0; qq < 2; ++qq) {
                    const int q = 2 * hb + qq;
                    const int ch = 16 * sg + 4 * q + kq;  // chunk of the row
                    const bool valid = ch < nch;
                    const u32x4 code = valid ? av[q] : u32x4{0u, 0u, 0u, 0u};
                    const LDS char* xp = xrow + 32 * min(ch, nch - 1);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const bf16x8 bop = *(const LDS bf16x8*)(xp + 16 * h);
                        const uint32_t d0 = code[2 * h], d1 = code[2 * h + 1];
                        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
                        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
                        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
                        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
                        const bf16x8 aop = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                        tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop, tmp, 0, 0, 0);
                    }
                }
                const float sc = 2 * sg + hb < nsb ? __uint_as_float(st.s[hb]) : 0.0f;
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) acc0[k2] = fmaf(tmp[k2], sc, acc0[k2]);
            }
        }
        if (sg == nstage - 1 || (split && t == nsteps - 1)) {  // the end of a tile, or of this wave's range
            const f32x4 d = acc0 + acc1;
            if (!split || (i * nstage >= a0 && sg == nstage - 1)) {
                // the whole tile in this range: lanes kq < 2 hold g of rows 4 kq + k2, lanes kq + 2 their v
                f32x4 v;
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) v[k2] = __shfl_xor(d[k2], 32);
                if (kq < 2 && r < M) {
#pragma unroll
                    for (int k2 = 0; k2 < 4; ++k2) {
                        const uint32_t mk = row_mask(tile_row(i) + 4 * kq + k2);
                        if ((mk >> r) & 1u)
                            cst[(tile_slot(i) + 4 * kq + k2) * M + __popc(mk & ((1u << r) - 1u))] = silu_mul(d[k2], v[k2]);
                    }
                }
            } else if (r < M) {  // a partial sum: slot 0 for the range's first tile, 1 for its last
                *(LDS f32x4*)(part + ((((wave * 2 + (i == i0 ? 0 : 1)) * M) + r) * 4 + kq) * 4) = d;
            }
            acc0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            acc1 = acc0;
        }
    };
    Stage st[R];
    if (nsteps <= R) {
        // a short range: every load at once, no stand-in loads (a load queued behind a saturated
        // memory path holds its wave at issue)
#pragma unroll
        for (int q = 0; q < R; ++q)
            if (q < nsteps) load(st[q], q);
        MOE_TRACE(16);
#pragma unroll
        for (int q = 0; q < R; ++q)
            if (q < nsteps) compute(st[q], q);
    } else {
        // R stages in flight; the loads are unconditional (past the end: stand-ins) so the number
        // in flight is static and each stage waits for its own loads only
#pragma unroll
        for (int q = 0; q < R; ++q) load(st[q], q);
        MOE_TRACE(16);
        for (int t0 = 0; t0 < nsteps; t0 += R) {
#pragma unroll
            for (int q = 0; q < R; ++q) {
                if (t0 + q < nsteps) compute(st[q], t0 + q);
                load(st[q], t0 + q + R);
            }
        }
    }
    MOE_TRACE(19);
    if (!split) return;
    __syncthreads();
    // tiles cut by range boundaries: the partial sums of the waves that share them, in wave order
    for (int idx = threadIdx.x; idx < nloc * 8 * M; idx += kThreads) {
        const int i = idx / (8 * M), rem = idx - i * 8 * M;
        const int jr = rem / M, n = rem - jr * M;
        int wf = 0, wl = 0;  // the waves whose ranges hold the tile's first and last step
        for (int w = 0; w < kWaves; ++w) {
            const int lo = T * w / kWaves, hi = T * (w + 1) / kWaves;
            if (lo <= i * nstage && i * nstage < hi) wf = w;
            if (lo <= (i + 1) * nstage - 1 && (i + 1) * nstage - 1 < hi) wl = w;
        }
        if (wf == wl) continue;  // finished inside one range
        float g = 0.0f, v = 0.0f;
        for (int w = wf; w <= wl; ++w) {
            const int lo = T * w / kWaves, hi = T * (w + 1) / kWaves;
            if (lo == hi) continue;  // an empty range
            const LDS float* pp = part + (int64_t)((w * 2 + (i == lo / nstage ? 0 : 1)) * M + n) * 16;
            g += pp[(jr >> 2) * 4 + (jr & 3)];
            v += pp[(2 + (jr >> 2)) * 4 + (jr & 3)];
        }
        const uint32_t mk = row_mask(tile_row(i) + jr);
        if ((mk >> n) & 1u) cst[(tile_slot(i) + jr) * M + __popc(mk & ((1u << n) - 1u))] = silu_mul(g, v);
    }
}

// Down rows [0, nrows) of one unit (row 0 at wbase, in LDS when FROM_LDS; its block scales are those of
// absolute row srow0 of the scale matrix smat) with K inputs,
// for the unit's t tokens whose fp32 activations are at acts ([t][K], LDS).  Tasks of RT rows go
// to the waves round robin (every `step`-th task from task `wslot` on; step 1: all of them).
// `ready()` is called by every wave after its first loads are issued and before any compute (it
// may contain workgroup barriers).  out(row, i, value) receives each result in the row's last lane.
template <int WF, int NJD, bool FROM_LDS, typename Ready, typename Out>
__device__ __forceinline__ void down_run(const uint8_t* wbase, const uint8_t* smat, int64_t srow0, int K, int nrows,
                                         const LDS float* acts, int t, int wslot, Ready ready, Out out,
                                         int step = kWaves) {
    constexpr int LPR = Geo<WF>::LPR_D, RL = Geo<WF>::RL_D, RT = rt_down<WF>();
    const int lane = threadIdx.x & 63, gi = lane / LPR, sl = lane % LPR;
    const int nch = K / Geo<WF>::EPC;
    const int64_t rb = row_bytes<WF>(K);
    const int ntask = (nrows + RT - 1) / RT;
    int n = wslot;
    Chunk wa[RL][NJD], wb[RL][NJD];
    // task >= ntask: the stand-in prefetch after the last task (a static number of loads in flight):
    // every lane reads the first chunk of row 0, one line, not a task (a re-read of the last task
    // was in flight when the phase's stores were waited for)
    auto load = [&](Chunk(&w)[RL][NJD], int task) {
        const bool dummy = task >= ntask;
#pragma unroll
        for (int rl = 0; rl < RL; ++rl) {
            const int64_t row = dummy ? 0 : min(task * RT + gi * RL + rl, nrows - 1);
            const uint8_t* srow = scale_row<WF>(smat, srow0 + row, K);
#pragma unroll
            for (int j = 0; j < NJD; ++j) {
                const int c = dummy ? 0 : min(sl + LPR * j, nch - 1);
                if constexpr (FROM_LDS)
                    ld_chunk_lds<WF>(w[rl][j], (const LDS uint8_t*)wbase + row * rb, srow, c);
                else
                    ld_chunk<WF>(w[rl][j], wbase + row * rb, srow, c);
            }
        }
    };
    auto settle_all = [&](Chunk(&w)[RL][NJD]) {
#pragma unroll
        for (int rl = 0; rl < RL; ++rl)
#pragma unroll
            for (int j = 0; j < NJD; ++j) settle_mask<WF>(w[rl][j], sl + LPR * j < nch);
    };
    auto compute = [&](const Chunk(&w)[RL][NJD], int task) {
        for (int i = 0; i < t; ++i) {
            const LDS char* arow = (const LDS char*)acts + (int64_t)i * K * 4;
            float acc[RL][kAcc];
#pragma unroll
            for (int rl = 0; rl < RL; ++rl)
#pragma unroll
                for (int q = 0; q < kAcc; ++q) acc[rl][q] = 0.0f;
#pragma unroll
            for (int j = 0; j < NJD; ++j) {
                const int c = min(sl + LPR * j, nch - 1);
#pragma unroll
                for (int rl = 0; rl < RL; ++rl) dot_a<WF>(w[rl][j], arow, 2 * K, c, acc[rl]);
                if constexpr (WF == MOE_FMT_MXFP4) __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int rl = 0; rl < RL; ++rl) {
                const float s = group_sum<LPR>(acc_sum(acc[rl]));
                const int row = task * RT + gi * RL + rl;
                if (sl == LPR - 1 && row < nrows) out(row, i, s);
            }
        }
    };
    if (n < ntask) load(wa, n);
    ready();
    if (n >= ntask) return;
    while (true) {
        load(wb, n + step);
        settle_all(wa);
        compute(wa, n);
        n += step;
        if (n >= ntask) break;
        load(wa, n + step);
        settle_all(wb);
        compute(wb, n);
        n += step;
        if (n >= ntask) break;
    }
}

// One task of a flattened list of down rows: up to RT rows of one unit.
struct DNTask {
    const uint8_t* w;       // the task's first weight row (an LDS address when lds)
    const uint8_t* s;       // the scale matrix of the task's rows (scale_mat; global memory)
    int srow;               // absolute row of the task's first row in that matrix
    const LDS float* acts;  // the unit's SwiGLU rows [t][astride] in LDS
    int lds;                // 1: the weights are in LDS
    int nrows;              // valid rows of the task
    int t;                  // tokens of the unit
    int K;                  // inputs per row
    int orow;               // index of the task's first row in the output slice
    int prow;               // first pair row of the unit
    int dummy;              // 1: the stand-in prefetch past the list (one line, every lane)
};

// This wave's tasks n = wslot, wslot + kWaves, ... < ntask of a flattened down-row list described by
// info(n, task); the source of each task (LDS or HBM) is its own.  The first task (PRE2: the first
// two) is loaded before ready(), and the next task's loads are in flight during the current task's
// compute.  out(task, row, i, v) receives row `row` of the task for token i.  A task's token rows
// are `pitch` bytes apart in LDS; the low plane of a bf16 hi/lo row starts 2 * astride bytes into
// it.  Two tasks ahead of the wait pay where the wait is long against the tasks (slice mode: FP8 at
// one token 27.2 against 28.5 us) and cost where the tasks are many (unit-major FP8: +0.4 us at six
// tokens, +1.4 at 16).
template <int WF, int NJD, bool PRE2, int RLX = 0, typename Info, typename Ready, typename Out>
__device__ __forceinline__ void down_flat(int ntask, int astride, int pitch, int wslot, Info info, Ready ready,
                                          Out out) {
    constexpr int LPR = Geo<WF>::LPR_D, RL = RLX > 0 ? RLX : Geo<WF>::RL_D;  // rows per lane group
    const int lane = threadIdx.x & 63, gi = lane / LPR, sl = lane % LPR;
    int n = wslot;
    Chunk wa[RL][NJD], wb[RL][NJD];
    DNTask ta, tb;
    // task i of the list; past its end the stand-in prefetch (the last task's description, one line
    // read by every lane) that keeps the number of loads in flight static
    auto task_of = [&](int i, DNTask& t) {
        info(min(i, ntask - 1), t);
        t.dummy = i >= ntask ? 1 : 0;
    };
    auto load = [&](Chunk(&w)[RL][NJD], const DNTask& t) {
        const int nch = t.K / Geo<WF>::EPC;
        const int64_t rb = row_bytes<WF>(t.K);
#pragma unroll
        for (int rl = 0; rl < RL; ++rl) {
            const int64_t row = t.dummy ? 0 : min(gi * RL + rl, t.nrows - 1);
            const uint8_t* srow = scale_row<WF>(t.s, t.srow + row, t.K);
#pragma unroll
            for (int j = 0; j < NJD; ++j) {
                const int c = t.dummy ? 0 : min(sl + LPR * j, nch - 1);
                if (t.lds)
                    ld_chunk_lds<WF>(w[rl][j], (const LDS uint8_t*)t.w + row * rb, srow, c);
                else
                    ld_chunk<WF>(w[rl][j], t.w + row * rb, srow, c);
            }
        }
    };
    auto settle_all = [&](Chunk(&w)[RL][NJD], const DNTask& t) {
        const int nch = t.K / Geo<WF>::EPC;
#pragma unroll
        for (int rl = 0; rl < RL; ++rl)
#pragma unroll
            for (int j = 0; j < NJD; ++j) settle_mask<WF>(w[rl][j], sl + LPR * j < nch);
    };
    auto compute = [&](const Chunk(&w)[RL][NJD], const DNTask& t) {
        const int nch = t.K / Geo<WF>::EPC;
        for (int i = 0; i < t.t; ++i) {
            const LDS char* arow = (const LDS char*)t.acts + i * pitch;
            float acc[RL][kAcc];
#pragma unroll
            for (int rl = 0; rl < RL; ++rl)
#pragma unroll
                for (int q = 0; q < kAcc; ++q) acc[rl][q] = 0.0f;
#pragma unroll
            for (int j = 0; j < NJD; ++j) {
                const int c = min(sl + LPR * j, nch - 1);
#pragma unroll
                for (int rl = 0; rl < RL; ++rl) dot_a<WF>(w[rl][j], arow, 2 * astride, c, acc[rl]);
                if constexpr (WF == MOE_FMT_MXFP4) __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int rl = 0; rl < RL; ++rl) {
                const float v = group_sum<LPR>(acc_sum(acc[rl]));
                const int row = gi * RL + rl;
                if (sl == LPR - 1 && row < t.nrows) out(t, row, i, v);
            }
        }
    };
    if constexpr (PRE2) {
        // the first two tasks load before ready() (past the list: the stand-in); then each task's
        // loads go out right after the compute of the task before the one in flight
        if (n < ntask) {
            task_of(n, ta);
            load(wa, ta);
            task_of(n + kWaves, tb);
            load(wb, tb);
        }
        ready();
        if (n >= ntask) return;
        while (true) {
            settle_all(wa, ta);
            compute(wa, ta);
            n += kWaves;
            if (n >= ntask) break;
            task_of(n + kWaves, ta);
            load(wa, ta);
            settle_all(wb, tb);
            compute(wb, tb);
            n += kWaves;
            if (n >= ntask) break;
            task_of(n + kWaves, tb);
            load(wb, tb);
        }
    } else {
        if (n < ntask) {
            task_of(n, ta);
            load(wa, ta);
        }
        ready();
        if (n >= ntask) return;
        while (true) {
            task_of(n + kWaves, tb);
            load(wb, tb);
            settle_all(wa, ta);
            compute(wa, ta);
            n += kWaves;
            if (n >= ntask) break;
            task_of(n + kWaves, ta);
            load(wa, ta);
            settle_all(wb, tb);
            compute(wb, tb);
            n += kWaves;
            if (n >= ntask) break;
        }
    }
}

// One unit of the slice-mode down projection: its weight rows [h0, h0 + nown) (row 0 at w, an LDS
// address when lds, stored by async_rows_to_lds), K inputs, t tokens whose bfloat16 SwiGLU rows
// start at acts (LDS rows of the caller's pitch), and the pair row of its first token.
struct SliceUnit {
    const uint8_t* w;
    const uint8_t* s;        // MXFP4 scales of row 0 (global memory)
    const LDS uint8_t* sl;   // the same scales copied into LDS, or null
    const LDS char* acts;
    int lds, K, t, prow;
};

// Slice-mode down rows on the matrix cores.  The workgroup computes y columns [h0, h0 + nown),
// nown <= 16, of all nun units; one wave takes a whole unit (units w + 1, w + 9, ... for wave w) as a
// chain of v_mfma_f32_16x16x32_bf16 products over the unit's 32-wide K blocks: A = its weight rows
// (MXFP4 codes dequantised to bfloat16 on the way), B = its tokens' bfloat16 SwiGLU rows, one
// column per token (t <= 16).  Results go to pst[(prow + token) * nown + row].  Units [0, npre) need
// no wait and are computed before ready(); units [npre, npre + ng) read their rows from global
// memory (a wave's first such unit is loaded before ready()), the rest from LDS.  Operand layout of the instruction (16x16x32, bf16): lane l holds A[l % 16][8 (l / 16) + 0..7],
// B[8 (l / 16) + 0..7][l % 16] and D[4 (l / 16) + 0..3][l % 16].
template <int WF, int KB, typename UnitOf, typename Ready>
__device__ __forceinline__ void down_slice_mfma(int nun, int npre, int ng, int nown, int apitch, UnitOf unit_of,
                                                Ready ready, LDS float* pst) {
    static_assert(WF == MOE_FMT_BF16 || WF == MOE_FMT_MXFP4, "bf16 or MXFP4 weights");
    static_assert(KB % 8 == 0, "K blocks in batches of 8");
    constexpr int BB = 8;  // B chunks per batch
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r = lane & 15, kq = lane >> 4;  // A row / token column; the lane's 8-wide K slice
    const int rr = min(r, nown - 1);          // rows past nown load row nown - 1 (results dropped)
    // A chunks: 8 bfloat16, or 8 E2M1 codes and their block's scale byte
    struct AOpB {
        u32x4 q;
    };
    struct AOpF {
        uint32_t c, s;
    };
    using AOp = std::conditional_t<WF == MOE_FMT_BF16, AOpB, AOpF>;
    AOp a[KB];
    // Only lanes of live rows read weights and only lanes of live tokens read SwiGLU rows (the LDS
    // port, not the matrix core, bounds this phase); other lanes keep stale operands, which reach
    // only the rows and columns of D that are dropped.
    auto load_a = [&](const SliceUnit& u, auto from_lds) {
        const int64_t rb = row_bytes<WF>(u.K);
        if (r >= nown) return;
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const int k0 = min(32 * i + 8 * kq, u.K - 8);  // in bounds; past K the B side is zero
            if constexpr (decltype(from_lds)::value) {
                const LDS uint8_t* row = (const LDS uint8_t*)u.w + rr * rb;
                const int sw = chunk_swz(rr, rb);
                if constexpr (WF == MOE_FMT_BF16)
                    a[i].q = *(const LDS u32x4*)(row + 16 * ((k0 >> 3) ^ sw));
                else
                    a[i].c = *(const LDS uint32_t*)(row + 16 * ((k0 >> 5) ^ sw) + 4 * ((k0 >> 3) & 3));
            } else {
                const uint8_t* row = u.w + rr * rb;
                if constexpr (WF == MOE_FMT_BF16)
                    a[i].q = __builtin_nontemporal_load((const u32x4*)(row + 2 * k0));
                else
                    a[i].c = __builtin_nontemporal_load((const uint32_t*)(row + k0 / 2));
            }
        }
        if constexpr (WF == MOE_FMT_MXFP4) {
            // scale bytes: from the LDS copy when there is one (no global round trip per unit)
            if (u.sl) {
#pragma unroll
                for (int i = 0; i < KB; ++i) a[i].s = u.sl[rr * (u.K / 32) + min(32 * i + 8 * kq, u.K - 8) / 32];
            } else {
#pragma unroll
                for (int i = 0; i < KB; ++i) a[i].s = u.s[rr * (u.K / 32) + min(32 * i + 8 * kq, u.K - 8) / 32];
            }
        }
    };
    auto a_operand = [&](int i) {
        if constexpr (WF == MOE_FMT_BF16) {
            asm volatile("" : "+v"(a[i].q));
            return __builtin_bit_cast(bf16x8, a[i].q);
        } else {
            asm volatile("" : "+v"(a[i].c), "+v"(a[i].s));
            const uint32_t c = a[i].c;
            const float sc = e8m0_to_f32(a[i].s);
            const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0);
            const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1);
            const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 2);
            const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 3);
            return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        }
    };
    // One column per token, one B read per K block.
    auto compute_many = [&](const SliceUnit& u) {
        const LDS char* brow = u.acts + (int64_t)min(r, u.t - 1) * apitch;
        auto load_b = [&](u32x4(&b)[BB], int i0) {
            if (r >= u.t) return;
#pragma unroll
            for (int j = 0; j < BB; ++j) b[j] = *(const LDS u32x4*)(brow + 2 * min(32 * (i0 + j) + 8 * kq, u.K - 8));
        };
        f32x4 acc[4] = {};
        u32x4 ba[BB] = {}, bb[BB] = {};
        auto batch = [&](u32x4(&b)[BB], int i0) {
#pragma unroll
            for (int j = 0; j < BB; ++j) asm volatile("" : "+v"(b[j]));
#pragma unroll
            for (int j = 0; j < BB; ++j) {
                const int i = i0 + j;
                const bool kv = 32 * i + 8 * kq < u.K;
                acc[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    a_operand(i), __builtin_bit_cast(bf16x8, kv ? b[j] : u32x4{0u, 0u, 0u, 0u}), acc[j & 3], 0, 0, 0);
            }
        };
        load_b(ba, 0);
#pragma unroll
        for (int i0 = 0; i0 < KB; i0 += 2 * BB) {
            if (i0 + BB < KB) load_b(bb, i0 + BB);
            batch(ba, i0);
            if (i0 + BB >= KB) break;
            if (i0 + 2 * BB < KB) load_b(ba, i0 + 2 * BB);
            batch(bb, i0 + BB);
        }
        const f32x4 d = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        if (r < u.t) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = 4 * kq + q;
                if (row < nown) pst[(u.prow + r) * nown + row] = d[q];
            }
        }
    };
    auto compute = [&](const SliceUnit& u) { compute_many(u); };
    SliceUnit u;
    int q = (wave + 1) % kWaves;  // unit 0 to the last wave: wave 0 also polls in ready()
    for (; q < npre; q += kWaves) {  // units that need no wait (rows in LDS, SwiGLU rows staged)
        unit_of(q, u);
        load_a(u, std::true_type{});
        compute(u);
    }
    const int q0 = q;
    const bool pre = q < npre + ng;
    if (pre) {  // a unit streamed from global memory: its loads overlap the wait
        unit_of(q, u);
        load_a(u, std::false_type{});
    }
    ready();
    MOE_TRACE(27);
    for (; q < nun; q += kWaves) {
        if (q != q0 || !pre) {
            unit_of(q, u);
            if (q < npre + ng)
                load_a(u, std::false_type{});
            else
                load_a(u, std::true_type{});
        }
        if (q == q0) MOE_TRACE(28);
        compute(u);
        if (q == q0) MOE_TRACE(29);
    }
}

// The MXFP4 form of down_slice_mfma (same units, order, waits and outputs).  K is permuted alike
// for A and B: lane (r, kq) owns whole MX blocks 4j + kq of its row (16 bytes of codes, one scale
// byte), and product 4j + m takes sub-chunk m of those blocks, so B lane (n, kq) of that product
// holds elements 32 (4j + kq) + 8m .. + 7 of token n's row.  A unit's A operand is then KB / 4
// 16-byte reads and KB / 4 scale bytes per lane instead of KB 4-byte reads and KB scale bytes:
// small enough for a wave to hold two units, so the next unit's reads are in flight while the
// current one is computed (units past the LDS window stream their rows from global memory, and a
// wait per unit would serialise their latencies).  Rows of the LDS window are in place before the
// call, so any unit's reads may start before ready().
template <int KB, typename UnitOf, typename Ready>
__device__ __forceinline__ void down_slice_mfma_mx(int nun, int npre, int nown, int apitch, UnitOf unit_of,
                                                   Ready ready, LDS float* pst) {
    static_assert(KB % 8 == 0, "K blocks in batches of 8");
    constexpr int NB = KB / 4;  // MX blocks per lane
    constexpr int BB = 8;       // B chunks per batch
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r = lane & 15, kq = lane >> 4;
    const int rr = min(r, nown - 1);
    struct AOp {
        u32x4 q[NB];
        uint32_t s[NB];
    };
    // lanes of rows past nown keep stale operands, which reach only dropped rows of D
    auto load_a = [&](AOp& a, const SliceUnit& u) {
        if (r >= nown) return;
        const int nblk = u.K / 32;
        const int64_t rb = u.K / 2;
        if (u.lds) {
            const LDS uint8_t* row = (const LDS uint8_t*)u.w + rr * rb;
            const int sw = chunk_swz(rr, rb);
#pragma unroll
            for (int j = 0; j < NB; ++j) a.q[j] = *(const LDS u32x4*)(row + 16 * (min(4 * j + kq, nblk - 1) ^ sw));
        } else {
            const uint8_t* row = u.w + rr * rb;
#pragma unroll
            for (int j = 0; j < NB; ++j)
                a.q[j] = __builtin_nontemporal_load((const u32x4*)(row + 16 * min(4 * j + kq, nblk - 1)));
        }
        if (u.sl) {
#pragma unroll
            for (int j = 0; j < NB; ++j) a.s[j] = u.sl[rr * nblk + min(4 * j + kq, nblk - 1)];
        } else {
#pragma unroll
            for (int j = 0; j < NB; ++j) a.s[j] = u.s[rr * nblk + min(4 * j + kq, nblk - 1)];
        }
    };
    auto compute = [&](AOp& a, const SliceUnit& u) {
        const int nblk = u.K / 32;
        const LDS char* brow = u.acts + (int64_t)min(r, u.t - 1) * apitch;
        auto boff = [&](int i) {  // byte offset of product i's 8 elements, 0 past K
            return 4 * (i >> 2) + kq < nblk ? 2 * (128 * (i >> 2) + 32 * kq + 8 * (i & 3)) : 0;
        };
        auto load_b = [&](u32x4(&b)[BB], int i0) {
            if (r >= u.t) return;
#pragma unroll
            for (int j = 0; j < BB; ++j) b[j] = *(const LDS u32x4*)(brow + boff(i0 + j));
        };
        f32x4 acc[4] = {};
        u32x4 ba[BB] = {}, bb[BB] = {};
        auto batch = [&](u32x4(&b)[BB], int i0) {
#pragma unroll
            for (int j = 0; j < BB; ++j) asm volatile("" : "+v"(b[j]));
#pragma unroll
            for (int j = 0; j < BB; ++j) {
                const int i = i0 + j, jb = i >> 2;
                const bool kv = 4 * jb + kq < nblk;
                asm volatile("" : "+v"(a.q[jb]), "+v"(a.s[jb]));
                const uint32_t c = a.q[jb][i & 3];
                const float sc = e8m0_to_f32(a.s[jb]);
                const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0);
                const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1);
                const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 2);
                const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 3);
                const bf16x8 av = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                acc[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    av, __builtin_bit_cast(bf16x8, kv ? b[j] : u32x4{0u, 0u, 0u, 0u}), acc[j & 3], 0, 0, 0);
            }
        };
        load_b(ba, 0);
#pragma unroll
        for (int i0 = 0; i0 < KB; i0 += 2 * BB) {
            if (i0 + BB < KB) load_b(bb, i0 + BB);
            batch(ba, i0);
            if (i0 + BB >= KB) break;
            if (i0 + 2 * BB < KB) load_b(ba, i0 + 2 * BB);
            batch(bb, i0 + BB);
        }
        const f32x4 d = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        if (r < u.t) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = 4 * kq + q;
                if (row < nown) pst[(u.prow + r) * nown + row] = d[q];
            }
        }
    };
    SliceUnit u0, u1;
    AOp a0, a1;
    int q = (wave + 1) % kWaves;  // unit 0 to the last wave: wave 0 also polls in ready()
    for (; q < npre; q += kWaves) {  // units that need no wait (rows in LDS, SwiGLU rows staged)
        unit_of(q, u0);
        load_a(a0, u0);
        compute(a0, u0);
    }
    // two units in flight from here on; both reads are issued before the wait
    if (q < nun) {
        unit_of(q, u0);
        load_a(a0, u0);
    }
    if (q + kWaves < nun) {
        unit_of(q + kWaves, u1);
        load_a(a1, u1);
    }
    ready();
    MOE_TRACE(27);
    while (q < nun) {
        if (q < kWaves) MOE_TRACE(28);
        compute(a0, u0);
        if (q < kWaves) MOE_TRACE(29);
        if (q + 2 * kWaves < nun) {
            unit_of(q + 2 * kWaves, u0);
            load_a(a0, u0);
        }
        q += kWaves;
        if (q >= nun) break;
        compute(a1, u1);
        if (q + 2 * kWaves < nun) {
            unit_of(q + 2 * kWaves, u1);
            load_a(a1, u1);
        }
        q += kWaves;
    }
    MOE_TRACE(30);
}

// Splits a list of U units of n items each (rows or tasks; item i of unit u has flat index
// u * n + i) over G workgroups by cost, an item of unit u costing c0 + c1 * t_u where t_u is the
// unit's token count: every workgroup gets an equal share of the total cost, so units that many
// tokens chose (more compute per weight byte) are spread over more workgroups.  Returns the flat
// range [lo, hi) of workgroup b; consecutive workgroups' ranges tile [0, U * n).  Every lane
// computes the same scalar result.
__device__ __forceinline__ void cost_split(const LDS uint32_t* s_mask, int U, int n, int c0, int c1, int G, int b,
                                           int64_t* lo, int64_t* hi) {
    // lane l holds units 4 l .. 4 l + 3 (U <= 256), so the unit costs come from LDS in one round
    // trip and their running sum is one wave scan (a loop over the units, one dependent LDS read
    // each, took 11 us at 77 units).  A unit's cost n * c is at most 2,560 * (8 + 6 * 16): the
    // total fits in 32 bits.
    const int lane = threadIdx.x & 63;
    int c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int u = 4 * lane + q;
        c[q] = u < U ? c0 + c1 * __popc(s_mask[u]) : 0;
        sum += n * c[q];
    }
    const int incl = wave_incl_scan(sum);
    const int64_t total = __builtin_amdgcn_readlane(incl, 63);
    const int first = incl - sum;  // the cost of units before 4 l
    // flat index of the first item whose cost interval ends after x (the unit holding x is unique)
    auto at = [&](int64_t x) -> int64_t {
        if (x >= total) return (int64_t)U * n;
        int64_t r = -1;
        int64_t acc = first;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t w = (int64_t)n * c[q];
            if (acc <= x && x < acc + w) r = (int64_t)(4 * lane + q) * n + (int)(x - acc + c[q] - 1) / c[q];
            acc += w;
        }
        const uint64_t ball = __ballot(r >= 0);
        const int src = __ffsll((unsigned long long)ball) - 1;
        const int rl = __builtin_amdgcn_readlane((int)(uint32_t)r, src), rh = __builtin_amdgcn_readlane((int)(r >> 32), src);
        return (int64_t)(((uint64_t)(uint32_t)rh << 32) | (uint32_t)rl);
    };
    // total * b / G without 64-bit division (total < 2^27)
    auto share = [&](int bb) { return (int64_t)((int)total / G) * bb + (int)((int)total % G) * bb / G; };
    *lo = at(share(b));
    *hi = at(share(b + 1));
}

// First row of workgroup o's slice of y's columns: [slice0(o), slice0(o + 1)).
__device__ __forceinline__ int slice0(int H, int G, int o) { return H * o / G; }  // H * G < 2^31

// ------------------------------------------------------------------------------------------
// the layer kernel
// ------------------------------------------------------------------------------------------

// SL: 1 for slice mode (the down rows of each workgroup's own y columns), 0 for unit-major down
// rows; one instance per mode keeps each kernel's code to the path it runs.
template <int AF, int WF, int NJ, int NJD, int SL>
__global__ __launch_bounds__(kThreads) void k_layer(Params p) {
    constexpr bool SLICE = SL != 0;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int G = gridDim.x, b = blockIdx.x;
    const int H = p.H, E = p.E, M = p.M, k = p.k, I = p.I, Is = p.Is;
    const int NP = M * k;
    const bool has_sh = Is > 0;
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    constexpr int RTG = rt_gate<WF>();
    constexpr int RTD = rt_down<WF>();
    // NJ is also the chunks per lane of a router row and of a token row (64 lanes a row)
    static_assert(Geo<AF>::EPC * Geo<AF>::LPR_G == Geo<WF>::EPC * Geo<WF>::LPR_G,
                  "router and gate/up rows cover the same elements per chunk column");
    LDS char* lds = (LDS char*)smem;
    LDS int* tab = (LDS int*)(lds + p.lds_tab);
    LDS char* xs = lds + p.lds_x;        // token rows; after phase C the staged SwiGLU rows
    LDS float* cst = (LDS float*)(lds + p.lds_cst);
    LDS char* shw = lds + p.lds_sh;
    LDS float* ysh = (LDS float*)(lds + p.lds_ysh);
    LDS char* dnw = lds + p.lds_dn;
    LDS char* trb = lds + p.lds_tr;     // the waves' transpose buffers of the matrix-core gate/up
    // MXFP4 scale bytes of the shared expert's slice rows in LDS, or null
    const LDS uint8_t* sclw_sh = WF == MOE_FMT_MXFP4 && p.scl_sh ? (const LDS uint8_t*)(lds + p.lds_scl) : nullptr;
    __shared__ uint32_t s_call, s_spin;
    MOE_TRACE_INIT;
    MOE_TRACE(0);

    // this workgroup's slice of y's columns (shared down rows, and the final combine)
    const int h0 = slice0(H, G, b), h1 = slice0(H, G, b + 1), nown = h1 - h0;
    const int64_t rbIs = row_bytes<WF>(Is);
    const int64_t rbI = row_bytes<WF>(I);

    // ---- A: call index, token rows, router rows, shared-expert down rows of the slice ----
    uint32_t* const call_ctr = p.ws.hdr + kHdrCall + kCallStride * b;  // this workgroup's own call counter
    if (threadIdx.x == 0) {
        s_call = ld_dev(call_ctr);
        s_spin = ld_dev(p.ws.hdr + kHdrSpin);
        s_fault = 0u;
    }
    const bool norm = AF == MOE_FMT_BF16 && (p.router_flags & MOE_ROUTER_NORM) != 0;
    if (!norm) async_rows_pitch((char*)xs, (const uint8_t*)p.x, M, H * XB, p.xpitch);
    const int e0 = E * b / G, e1 = E * (b + 1) / G;
    const int nrw = min(e1 - e0, kWaves);  // waves with router rows
    Chunk rfirst[NJ];
    {
        const int e = e0 + wave_id(), lane = threadIdx.x & 63, nch = H / Geo<AF>::EPC;
        if (e < e1) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                ld_chunk<AF>(rfirst[j], (const uint8_t*)p.wr + (int64_t)e * H * XB, nullptr, min(lane + 64 * j, nch - 1));
        }
    }
    // slice mode on the matrix cores reads the LDS windows row-interleaved: store them swizzled
    const bool mf_slice = p.slice_mfma != 0;
    const bool mf_sh = p.sh_mfma != 0;  // shared down rows on the matrix cores (window stored swizzled)
    // slice mode on the matrix cores rounds the SwiGLU rows to bfloat16 for its B operands: the
    // producers write them as bfloat16 (the same rounding, half the bytes every workgroup stages)
    // (and so do the producers for MXFP4 and FP8 weights everywhere: their vector down path takes
    // the rows as one bfloat16 plane)
    const bool bf_act = (SLICE && mf_slice) || act_mode<WF>() == 2;
    const uint16_t* act16 = (const uint16_t*)p.ws.act;
    const __amdgpu_buffer_rsrc_t act_rs =
        dev_rsrc(p.ws.act, (uint32_t)((int64_t)(NP + M) * p.act_stride * 4));
    if (has_sh && !p.route_only && nown > 0) {
        if (mf_sh)
            async_rows_to_lds((char*)shw, (const uint8_t*)p.w.sh_down + h0 * rbIs, (int)(nown * rbIs), (int)rbIs);
        else
            async_to_lds((char*)shw, (const uint8_t*)p.w.sh_down + h0 * rbIs, (int)(nown * rbIs));
        if (sclw_sh)
            async_dwords_to_lds((char*)sclw_sh, p.w.sh_down_s + (int64_t)h0 * (Is / 32), nown * (Is / 32));
    }
    if constexpr (AF == MOE_FMT_BF16)
        if (norm) rms_norm_rows<NJ>(p, xs);  // the normed token rows replace x everywhere
    // one bf16 token: the selection's round counter (see gu_first below) starts at zero
    if constexpr (SLICE && WF == MOE_FMT_BF16)
        if (M == 1 && threadIdx.x == 0) ((volatile LDS int*)(lds + p.lds_sel))[kMaxTopK] = 0;
    __builtin_amdgcn_s_waitcnt(0);  // token rows (and the slice's shared down rows) in LDS
    __syncthreads();
    MOE_TRACE(1);
    const uint32_t call = s_call;
    if (threadIdx.x == 0) __hip_atomic_store(call_ctr, call + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t* set = p.ws.ctr + (int64_t)(call & 1u) * kSetWords;
    const Fault fault{p.ws.hdr + kHdrStatus, line(set, kLineFault), s_spin ? (int)min(s_spin, (uint32_t)kSpinLimit) : kSpinLimit};
    // this call's fault line, read after the last wait for other workgroups' data (a producer
    // raises it before it publishes anything): nonzero -> y is written as NaN
    uint32_t call_fault = 0u;
    if (b == 0) {
        uint32_t* nxt = p.ws.ctr + (int64_t)((call + 1u) & 1u) * kSetWords;
        for (int l = threadIdx.x; l < kSetLines; l += kThreads) line(nxt, l)[0] = 0u;
    }
    // router rows (tagged logits: no arrival counter)
    if (wave_id() < nrw) router_rows<AF, NJ>(p, xs, e0, e1, rfirst, call + 1u);
    MOE_TRACE(2);
    if (p.route_only && b != 0) {
        MOE_TRACE_FLUSH;
        return;
    }

    // ---- A': shared expert gate/up (needs no routing), on the waves without router rows first;
    //      results go straight to the workspace and are counted after the routing barrier ----
    int sh_rows = 0;
    int sh_waves = 0;  // waves kWaves - sh_waves .. kWaves - 1 have shared gate/up tasks
    if (has_sh && !p.route_only) {
        const int T = Is / RTG;  // a contiguous range of tasks per workgroup
        const int qa = T * b / G, qb = T * (b + 1) / G;
        sh_rows = (qb - qa) * RTG;
        bool split = false;
        if constexpr (!SLICE && WF == MOE_FMT_MXFP4) {
            // Unit-major MXFP4 from 8 tokens on: a workgroup's one or two tasks would each decode
            // every code once per token on one wave (at 16 tokens the routing barrier waited 8 us
            // for them).  Their tokens are split over the waves without router rows instead (wave 0
            // also runs the top-k): wave slot w takes task w / parts for tokens [t0, t1) of part
            // w % parts (every part loads the task's rows; the copies after the first come from
            // cache).  At 16 tokens 102.8 -> 98.7 us; FP8 gained nothing and bf16 lost 0.9 us.
            const int nt = qb - qa, free_waves = kWaves - nrw;
            if (M >= 8 && nt > 0 && nt < free_waves) {
                split = true;
                const int parts = free_waves / nt, tw = (M + parts - 1) / parts;
                const int w = kWaves - 1 - wave_id(), task = w / parts;
                const int t0 = min(M, (w - task * parts) * tw), t1 = min(M, t0 + tw);
                sh_waves = min(nt * parts, kWaves);
                gateup_run<AF, WF, NJ>(
                    p, xs, task < nt && t1 > t0 ? 1 : 0, 0,
                    [&](int, GUTask& t) {
                        const int64_t r0 = (int64_t)(qa + task) * RTG;
                        t.g = (const uint8_t*)p.w.sh_gate + r0 * row_bytes<WF>(H);
                        t.u = (const uint8_t*)p.w.sh_up + r0 * row_bytes<WF>(H);
                        t.gs = scale_row<WF>(p.w.sh_gate_s, r0, H);
                        t.us = scale_row<WF>(p.w.sh_up_s, r0, H);
                        t.mask = ((1u << (t1 - t0)) - 1u) << t0;  // tokens t0 .. t1 - 1 (t1 - t0 <= 16)
                        t.slot = (int)r0;
                    },
                    [&](int r, int i, float v) {  // i: the i-th token of the mask, token t0 + i
                        st_dev_bf16(act_rs, (uint32_t)(((int64_t)(NP + t0 + i) * p.act_stride + r) * 2), v);
                    });
            }
        }
        if (!split) {
        sh_waves = min(qb - qa, kWaves);
        gateup_run<AF, WF, NJ>(
            p, xs, qb - qa, kWaves - 1 - wave_id(),
            [&](int i, GUTask& t) {
                const int64_t r0 = (int64_t)(qa + i) * RTG;
                t.g = (const uint8_t*)p.w.sh_gate + r0 * row_bytes<WF>(H);
                t.u = (const uint8_t*)p.w.sh_up + r0 * row_bytes<WF>(H);
                t.gs = scale_row<WF>(p.w.sh_gate_s, r0, H);
                t.us = scale_row<WF>(p.w.sh_up_s, r0, H);
                t.mask = (1u << M) - 1u;
                t.slot = (int)r0;
            },
            [&](int r, int i, float v) {
                if (bf_act)
                    st_dev_bf16(act_rs, (uint32_t)(((int64_t)(NP + i) * p.act_stride + r) * 2), v);
                else
                    st_dev(p.ws.act + (int64_t)(NP + i) * p.act_stride + r, v);
            });
        }
    }
    MOE_TRACE(3);

    // The vector gate/up's task split (phase C) for nu units: T tasks of RTG rows of the flattened
    // (unit, row) list.  Each wave first takes a static share (about 70% of the work); the rest is
    // handed out in chunks of ch tasks from npool pools of eight workgroups each.
    struct GUPlan {
        int T, P0, sa, ns, pool, pa, pb, ch, nch;
        bool dyn;
    };
    auto gu_plan = [&](int nu) {
        GUPlan g;
        g.T = nu * (I / RTG);
        // below six tasks per wave the chunks' granularity costs more than the balance gains
        g.dyn = g.T >= 6 * kWaves * G;
        const int Rs = g.dyn ? 7 * g.T / (80 * G) : (g.T + kWaves * G - 1) / (kWaves * G);  // 7 T < 2^31
        g.P0 = g.dyn ? kWaves * G * Rs : g.T;
        // this workgroup's static tasks: a contiguous range of the static part, dealt to its
        // waves round robin (consecutive rows: whole DRAM pages, contiguous write-out); one 32-bit
        // division per split
        const int sq = g.P0 / G, sr = g.P0 - sq * G;
        g.sa = b * sq + min(b, sr);
        const int sbnd = g.sa + sq + (b < sr ? 1 : 0);
        g.ns = n_strided(sbnd - g.sa, wave_id(), kWaves);  // static positions of this wave
        // consecutive workgroups sit on different XCDs (round robin), so pool b / 8 gathers one
        // workgroup of every XCD: whole XCDs stream at different rates (up to 15% apart at 16
        // bf16 tokens, depending on the box and the data), and a pool within one XCD could not
        // even that out (pools per XCD: the XCDs' gate/up ends 15 us apart at 16 bf16 tokens,
        // these: 4 us; bf16 16 tokens 181.6 -> 180.3 us, 6 tokens 75.4 -> 74.8 us)
        const int npool = max(1, G / 8);
        g.pool = (b / 8) % npool;
        const int pq = (g.T - g.P0) / npool, pr = (g.T - g.P0) - pq * npool;
        g.pa = g.P0 + g.pool * pq + min(g.pool, pr);
        g.pb = g.pa + pq + (g.pool < pr ? 1 : 0);
        g.ch = gu_chunk_tasks<WF>(H);
        g.nch = (g.pb - g.pa + g.ch - 1) / g.ch;
        return g;
    };
    // One token always has k units: with bf16 weights its split is worked out while the routing is
    // pending, not between the routing and the first gate/up load (bf16 one token 30.8 -> 30.1 us;
    // the second copy of the split's code cost the MXFP4 instance 1 us at six tokens)
    const bool gu_early = WF == MOE_FMT_BF16 && SLICE && M == 1 && !p.gu_mfma && !p.route_only;
    GUPlan gpe{};
    if constexpr (SLICE && WF == MOE_FMT_BF16)
        if (gu_early) gpe = gu_plan(k);
    // ... and the waves the selection leaves idle issue their first gate/up task as soon as its
    // expert has been selected (the selecting wave publishes each round's id in LDS; without a bias
    // the units are the experts in selection order), so those loads run during the selection
    Chunk gfirst_g[Geo<WF>::RL_G][NJ], gfirst_u[Geo<WF>::RL_G][NJ];
    bool gfirst = false;
    volatile LDS int* sel_early =
        gu_early && !(p.router_flags & MOE_ROUTER_BIAS) ? (volatile LDS int*)(lds + p.lds_sel) : nullptr;
    auto gu_first = [&]() {
        if constexpr (SLICE && WF == MOE_FMT_BF16) {
            if (sel_early != nullptr && gpe.ns > 0) {
                const int q0 = gpe.sa + wave_id();  // this wave's first static task
                const int u = q0 / (I / RTG);
                for (int it = 0; sel_early[kMaxTopK] <= u && it < kSpinLimit; ++it) __builtin_amdgcn_s_sleep(1);
                if (sel_early[kMaxTopK] > u) {
                    const int64_t e = uni(sel_early[u]);
                    const int64_t r0 = (int64_t)q0 * RTG - (int64_t)u * I;
                    const int64_t rb = row_bytes<WF>(H);
                    GUTask t;
                    t.g = (const uint8_t*)p.w.gate + (e * I + r0) * rb;
                    t.u = (const uint8_t*)p.w.up + (e * I + r0) * rb;
                    t.gs = t.us = nullptr;
                    t.mask = 1u;
                    t.slot = 0;
                    t.dummy = 0;
                    gateup_load<WF, NJ>(H, gfirst_g, gfirst_u, t);
                    gfirst = true;
                }
            }
        }
    };

    // ---- B: routing barrier, top-k and compaction in every workgroup ----
    // the published expert pairs are polled by the highest wave without shared gate/up tasks (those
    // run on the vector ALU and, at 16 tokens with E2M1 decode, would hold the poll back by µs)
    const int U = route_and_compact(p, tab, lds + p.lds_sel, b == 0, call + 1u,
                                    sh_waves >= kWaves ? kWaves - 1 : kWaves - 1 - sh_waves, fault, sel_early,
                                    gu_first);
    MOE_TRACE(5);
    if (p.route_only) {
        MOE_TRACE_FLUSH;
        return;
    }
    if (sh_rows > 0) {  // the shared rows' stores completed long ago; this wait is short
        publish();
        if (threadIdx.x == 0) add_dev(line(set, kLineShared), (uint32_t)sh_rows);
    }
    MOE_TRACE(20);
    const LDS uint32_t* s_mask = (const LDS uint32_t*)tab + kTabMask;
    const LDS int* s_off = tab + kTabOff;
    const LDS int* s_exp = tab + kTabExp;

    // ---- start streaming this workgroup's routed down rows into LDS (as far as the window goes):
    //      slice mode: rows [h0, h1) of every unit; otherwise an equal share of all units' rows ----
    int64_t d0 = 0, d1 = 0;  // unit-major: this workgroup's (unit, row) range, split by cost
    if constexpr (!SLICE) cost_split(s_mask, U, H, kCostBase, p.cost_dn, G, b, &d0, &d1);
    int nfit = 0;  // slice mode: units whose slice rows are in the window
    // Slice mode keeps an LDS window of down rows for bf16 (and f32) weights only.  With bf16 on
    // the matrix cores the window streams in after this workgroup's gate/up rows have been
    // published (during the wait for the other workgroups): issued before them, it would sit ahead
    // of the gate/up loads in every wave's in-order memory counter and delay the whole phase (0.8 us
    // at one token).  Unit-major down rows stream from global memory inside the down phase (an LDS
    // prefetch of them issued here cost ~1 us at six tokens).
    const bool late_window = WF == MOE_FMT_BF16 && mf_slice;
    auto slice_window = [&]() {
        if (nown > 0) {
            // a unit's slice is a few instructions: each unit starts on the wave after the last
            // one's, so every wave issues its share.  The units' expert ids are read into a register
            // first (lane u: unit u): an LDS read between two copies would wait for every earlier
            // copy into LDS, since the compiler cannot tell which bytes a copy writes (eight bf16
            // units took 2.7 us to issue one after the other)
            const int per = (int)((nown * rbI + 1023) / 1024);
            const int ex_l = s_exp[min((int)(threadIdx.x & 63), max(U - 1, 0))];
            for (int u = 0; u < nfit; ++u) {
                const int e = u < 64 ? __builtin_amdgcn_readlane(ex_l, u) : s_exp[u];
                const uint8_t* src = (const uint8_t*)p.w.down + ((int64_t)e * H + h0) * rbI;
                if (mf_slice)
                    async_rows_to_lds((char*)(dnw + (int64_t)u * nown * rbI), src, (int)(nown * rbI), (int)rbI, u * per);
                else
                    async_to_lds((char*)(dnw + (int64_t)u * nown * rbI), src, (int)(nown * rbI), u * per);
            }
        }
    };
    if constexpr (SLICE) {
        if (nown > 0) nfit = min(U, p.dn_bytes / (int)(nown * rbI));  // 32-bit: on the path to gate/up
        if (!late_window) slice_window();
    }
    MOE_TRACE(21);

    // ---- C: routed gate/up over the flattened (unit, row) list.  Results are staged in LDS,
    //      written at the end, and counted on one counter ----
    {
        const int64_t nrows = (int64_t)U * I;
        int my_rows = 0;
        if (p.gu_mfma) {
            // tiles of 8 rows dealt to the workgroups round robin
            const int nloc = n_strided((int)(nrows / 8), b, G);
            MOE_TRACE(22);
            if (WF == MOE_FMT_MXFP4 && SLICE && p.gu_items) {
                if (nloc > 0) {
                    LDS float* part = p.gu_ksplit ? cst + p.gu_part : nullptr;
                    if ((H / 32) % 16 == 0)
                        gateup_mfma_mx<10, true>(p, xs, nloc, s_mask, s_exp, cst, part);
                    else
                        gateup_mfma_mx<10, false>(p, xs, nloc, s_mask, s_exp, cst, part);
                }
            } else if constexpr (WF == MOE_FMT_MXFP4 || WF == MOE_FMT_FP8) {
                if (nloc > 0)
                    gateup_mfma<WF>(p, xs, nloc, s_mask, s_exp, cst, p.gu_part >= 0 ? cst + p.gu_part : nullptr, trb);
            }
            __syncthreads();
            MOE_TRACE(6);
            const int n = nloc * 8 * M;
            for (int i = threadIdx.x; i < n; i += kThreads) {
                const int sl = i / M, m = i - sl * M;
                const int64_t f = (int64_t)(b + (sl / 8) * G) * 8 + sl % 8;
                const int u = (int)f / I;
                if (m < __popc(s_mask[u]))
                {
                    const int64_t o = (int64_t)(s_off[u] + m) * p.act_stride + (f - (int64_t)u * I);
                    if (bf_act)
                        st_dev_bf16(act_rs, (uint32_t)(o * 2), cst[i]);
                    else
                        st_dev(p.ws.act + o, cst[i]);
                }
            }
            my_rows = nloc * 8;
        } else {
            // Tasks of RTG rows, split by gu_plan: some CUs stream persistently faster than others,
            // and the fast ones take more chunks.  A wave claims its next chunk one chunk ahead, so
            // the atomic's round trip overlaps the current chunk, and claims only what its staging
            // room holds (room for twice the average dynamic share, so the pools always drain).
            // Each wave logs the task at every position for the write-out.
            const int cap = p.gu_cap, lane = threadIdx.x & 63, w = wave_id();
            LDS int* qlog = (LDS int*)(cst + (int64_t)kWaves * cap * RTG * M);  // [kWaves][cap]
            LDS int* nwv = qlog + kWaves * cap;                                 // [kWaves]
            const GUPlan g = gu_early ? gpe : gu_plan(U);
            const int T = g.T, P0 = g.P0, sa = g.sa, ns = g.ns, pool = g.pool, pa = g.pa, pb = g.pb, ch = g.ch,
                      nch = g.nch;
            const bool dyn = g.dyn;
            const int rb = (int)row_bytes<WF>(H);
            uint32_t* pctr = line(set, kLinePoolC0 + pool);
            bool has_pend = dyn && ns + ch <= cap;
            uint32_t pend = 0;
            if (has_pend && lane == 0) pend = add_dev(pctr, 1u);
            int cstart = 0;
            MOE_TRACE(22);
            const int n = gateup_seq<AF, WF, NJ>(
                p, xs,
                [&](int s) -> int {
                    int q;
                    if (s < ns) {
                        q = sa + w + kWaves * s;
                    } else {
                        const int o = (s - ns) % ch;
                        if (o == 0) {
                            if (!has_pend) return -1;
                            const int c = __builtin_amdgcn_readlane((int)pend, 0);
                            has_pend = false;
                            if (c >= nch) return -1;
                            cstart = pa + c * ch;
                            if (s + 2 * ch <= cap) {
                                has_pend = true;
                                if (lane == 0) pend = add_dev(pctr, 1u);
                            }
                        }
                        q = cstart + o;
                        if (q >= pb) return -1;
                    }
                    if (lane == 0) qlog[w * cap + s] = q;
                    return q;
                },
                [&](int q, int s, GUTask& t) {
                    const int64_t f = (int64_t)q * RTG;  // the task's first flat row
                    const int u = uni((int)f / I);
                    const int64_t e = uni(s_exp[u]);
                    const int64_t r0 = f - (int64_t)u * I;
                    t.g = (const uint8_t*)p.w.gate + (e * I + r0) * rb;
                    t.u = (const uint8_t*)p.w.up + (e * I + r0) * rb;
                    t.gs = scale_row<WF>(scale_mat<WF>(p.w.gate_s, e, I, H), r0, H);
                    t.us = scale_row<WF>(scale_mat<WF>(p.w.up_s, e, I, H), r0, H);
                    t.mask = uni(s_mask[u]);
                    t.slot = (w * cap + s) * RTG;
                },
                [&](int r, int i, float v) { cst[r * M + i] = v; }, gfirst_g, gfirst_u, gfirst);
            if (lane == 0) nwv[w] = n;
            __syncthreads();
            MOE_TRACE(6);
            const int per = cap * RTG * M;  // staged values of one wave
            for (int i = threadIdx.x; i < kWaves * per; i += kThreads) {
                const int wv = i / per, rem = i - wv * per;
                const int sl = rem / M, m = rem - sl * M;
                const int sp = sl / RTG;
                if (sp < nwv[wv]) {
                    const int64_t f = (int64_t)qlog[wv * cap + sp] * RTG + sl % RTG;
                    const int u = (int)f / I;
                    if (m < __popc(s_mask[u]))
                    {
                    const int64_t o = (int64_t)(s_off[u] + m) * p.act_stride + (f - (int64_t)u * I);
                    if (bf_act)
                        st_dev_bf16(act_rs, (uint32_t)(o * 2), cst[i]);
                    else
                        st_dev(p.ws.act + o, cst[i]);
                }
                }
            }
            for (int wv = 0; wv < kWaves; ++wv) my_rows += nwv[wv] * RTG;
        }
        publish();
        MOE_TRACE(7);
        if (my_rows > 0 && threadIdx.x == 0) add_dev(line(set, kLineRouted + b % kRoutedStripes), (uint32_t)my_rows);
    }
    if constexpr (SLICE)
        if (late_window) slice_window();

    // ---- B': the shared expert's down rows of this slice (weights in LDS) -> ysh [M][nown], while
    //      the routed units' counters complete (measured: doing it after the down rows instead,
    //      on the workgroups that finish gate/up last, is slower) ----
    //      (slice mode: in its down phase, before the wait for the routed units) ----
    auto shared_down = [&]() {
        if constexpr ((WF == MOE_FMT_BF16 || WF == MOE_FMT_MXFP4) && NJD <= 3) {
            if (has_sh && nown > 0 && mf_sh && !SLICE) {
                wait_geq(line(set, kLineShared), (uint32_t)Is, fault);
                MOE_TRACE(25);
                const int apitch = 2 * p.act_stride + 16;  // rows 4 banks apart: no conflicts among the B columns
                if (bf_act)
                    stage_rows_b16((LDS char*)xs, act16 + (int64_t)NP * p.act_stride, p.act_stride, M, Is, apitch);
                else
                    stage_rows_bf16((LDS char*)xs, p.ws.act + (int64_t)NP * p.act_stride, p.act_stride, M, Is, apitch);
                __syncthreads();
                MOE_TRACE(26);
                auto unit_of = [&](int, SliceUnit& t) {
                    t.prow = 0;
                    t.t = M;
                    t.K = Is;
                    t.lds = 1;
                    t.w = (const uint8_t*)shw;
                    t.s = WF == MOE_FMT_MXFP4 ? p.w.sh_down_s + (int64_t)h0 * (Is / 32) : nullptr;
                    if constexpr (WF == MOE_FMT_MXFP4) t.sl = sclw_sh;
                    t.acts = (const LDS char*)xs;
                };
                down_slice_mfma<WF, 8 * NJD>(1, 1, 0, nown, apitch, unit_of, []() {}, ysh);
                __syncthreads();
            }
        }
        if (has_sh && nown > 0 && !SLICE && !mf_sh) {
            wait_geq(line(set, kLineShared), (uint32_t)Is, fault);
            MOE_TRACE(25);
            if constexpr (act_mode<WF>() == 2)
                stage_rows_b16((LDS char*)xs, act16 + (int64_t)NP * p.act_stride, p.act_stride, M, Is, 4 * Is);
            else
                stage_rows<act_mode<WF>()>((LDS float*)xs, p.ws.act + (int64_t)NP * p.act_stride, p.act_stride, M, Is);
            __syncthreads();
            MOE_TRACE(26);
            // the slice's rows make one or two tasks, so the tokens are split over the waves instead:
            // wave w takes every row for tokens [w tw, w tw + tw) (with the rows dealt to the waves,
            // two waves ran all 16 tokens and FP8 at 16 tokens spent 12.8 us here)
            const int tw = (M + kWaves - 1) / kWaves, t0 = min(M, wave_id() * tw), t1 = min(M, t0 + tw);
            if (t1 > t0)
                down_run<WF, NJD, true>((const uint8_t*)shw, p.w.sh_down_s, h0, Is, nown,
                                        (const LDS float*)xs + (int64_t)t0 * Is, t1 - t0, 0, []() {},
                                        [&](int row, int i, float v) { ysh[(t0 + i) * nown + row] = v; }, 1);
            __syncthreads();
        }
    };
    if constexpr (!SLICE)
        if (has_sh && nown > 0) shared_down();
    MOE_TRACE(8);

    if constexpr (SLICE) {
        // ---- D (slice mode): rows [h0, h1) of every routed unit and of the shared expert, as one
        //      flattened task list (units past the LDS window first, so their loads are in flight
        //      during the waits); every pair row's SwiGLU output is staged once; partial outputs
        //      stay in LDS: pst [NP + M][nown] ----
        if (nown > 0) {
            LDS float* pst = cst;
            const int astride = p.act_stride;
            // vector path: a token row takes 2 bytes per element as one bf16 plane, else 4
            const int spitch = (act_mode<WF>() == 2 ? 2 : 4) * astride;
            // FP8 tasks of 12 rows (three per lane group): one task covers a 10-row slice of a unit,
            // where 8-row tasks left every unit a 2-row task
            constexpr int RLS = WF == MOE_FMT_FP8 ? 3 : Geo<WF>::RL_D;
            constexpr int RTS = RLS * (64 / Geo<WF>::LPR_D);
            const int nblk = (nown + RTS - 1) / RTS;
            const int nun = U + (has_sh ? 1 : 0);
            const int ng = U - nfit;  // routed units read from HBM in this phase
            auto info = [&](int tt, DNTask& t) {
                const int pidx = tt / nblk, bk = tt - pidx * nblk;
                const int r0 = bk * RTS;
                t.nrows = min(RTS, nown - r0);
                t.orow = r0;
                if (pidx < U) {
                    const int u = pidx < ng ? nfit + pidx : pidx - ng;
                    const int64_t e = uni(s_exp[u]);
                    t.prow = uni(s_off[u]);
                    t.t = __popc(uni(s_mask[u]));
                    t.K = I;
                    t.lds = pidx >= ng ? 1 : 0;
                    t.w = t.lds ? (const uint8_t*)(dnw + ((int64_t)u * nown + r0) * rbI)
                                : (const uint8_t*)p.w.down + (e * H + h0 + r0) * rbI;
                    t.s = scale_mat<WF>(p.w.down_s, e, H, I);
                    t.srow = h0 + r0;
                } else {
                    t.prow = NP;
                    t.t = M;
                    t.K = Is;
                    t.lds = 1;
                    t.w = (const uint8_t*)(shw + (int64_t)r0 * rbIs);
                    t.s = p.w.sh_down_s;
                    t.srow = h0 + r0;
                }
                t.acts = (const LDS float*)((const LDS char*)xs + t.prow * spitch);
            };
            auto ready = [&]() {
                wait_units(set, (uint32_t)(U * I), has_sh ? (uint32_t)Is : 0u, fault);
                call_fault = ld_dev(fault.flag);  // used at the y write, long after it lands
                MOE_TRACE(9);
                if constexpr (act_mode<WF>() == 2)
                    stage_rows_b16((LDS char*)xs, act16, astride, NP + (has_sh ? M : 0), astride, spitch);
                else
                    stage_rows<act_mode<WF>()>((LDS float*)xs, p.ws.act, astride, NP + (has_sh ? M : 0), astride);
                __syncthreads();
                MOE_TRACE(10);
            };
            if constexpr ((WF == MOE_FMT_BF16 || WF == MOE_FMT_MXFP4) && NJD <= 3) {
                if (mf_slice) {
                    // matrix-core path: SwiGLU rows staged as bfloat16, one wave per unit
                    const int apitch = 2 * astride + 16;  // rows 4 banks apart: no conflicts among the B columns
                    const int nsh = has_sh ? 1 : 0;  // the shared unit first: it needs no wait
                    if (has_sh) {
                        wait_geq(line(set, kLineShared), (uint32_t)Is, fault);
                        stage_rows_b16((LDS char*)xs + (int64_t)NP * apitch, act16 + (int64_t)NP * astride, astride,
                                        M, Is, apitch);
                        __syncthreads();
                    }
                    auto unit_of = [&](int q0, SliceUnit& t) {
                        const int q = q0 - nsh;
                        if (q >= 0) {
                            const int u = q < ng ? nfit + q : q - ng;
                            const int64_t e = uni(s_exp[u]);
                            t.prow = uni(s_off[u]);
                            t.t = __popc(uni(s_mask[u]));
                            t.K = I;
                            t.lds = q >= ng ? 1 : 0;
                            t.w = t.lds ? (const uint8_t*)(dnw + (int64_t)u * nown * rbI)
                                        : (const uint8_t*)p.w.down + (e * H + h0) * rbI;
                            t.s = WF == MOE_FMT_MXFP4 ? p.w.down_s + (e * H + h0) * (I / 32) : nullptr;
                            if constexpr (WF == MOE_FMT_MXFP4) t.sl = nullptr;  // routed scale bytes from global memory
                        } else {
                            t.prow = NP;
                            t.t = M;
                            t.K = Is;
                            t.lds = 1;
                            t.w = (const uint8_t*)shw;
                            t.s = WF == MOE_FMT_MXFP4 ? p.w.sh_down_s + (int64_t)h0 * (Is / 32) : nullptr;
                            if constexpr (WF == MOE_FMT_MXFP4) t.sl = sclw_sh;
                        }
                        t.acts = (const LDS char*)xs + (int64_t)t.prow * apitch;
                    };
                    auto ready_bf16 = [&]() {  // the shared expert's rows were staged above
                        wait_units(set, (uint32_t)(U * I), 0u, fault);
                        call_fault = ld_dev(fault.flag);  // used at the y write, long after it lands
                        MOE_TRACE(9);
                        stage_rows_b16((LDS char*)xs, act16, astride, NP, astride, apitch);
                        if constexpr (WF == MOE_FMT_BF16)
                            __builtin_amdgcn_s_waitcnt(0);  // this wave's share of the late window has landed
                        __syncthreads();
                        MOE_TRACE(10);
                    };
                    if constexpr (WF == MOE_FMT_MXFP4)
                        down_slice_mfma_mx<8 * NJD>(U + nsh, nsh, nown, apitch, unit_of, ready_bf16, pst);
                    else
                        down_slice_mfma<WF, 8 * NJD>(U + nsh, nsh, ng, nown, apitch, unit_of, ready_bf16, pst);
                    __syncthreads();
                    MOE_TRACE(11);
                    const LDS int* s_pair = tab + kTabPair;
                    const LDS float* s_roww = (const LDS float*)(tab + kTabRowW);
                    const bool bad = (call_fault | s_fault) != 0u;
                    for (int i = threadIdx.x; i < M * nown; i += kThreads) {
                        const int m = i / nown, hh = i - m * nown, h = h0 + hh;
                        float acc = 0.0f;
                        for (int j = 0; j < k; ++j) {
                            const int row = s_pair[m * k + j];
                            acc = fmaf(s_roww[row], pst[row * nown + hh], acc);
                        }
                        if (has_sh) acc += pst[(NP + m) * nown + hh];
                        ((uint16_t*)p.y)[(int64_t)m * H + h] = f32_to_bf16_rne(bad ? __builtin_nanf("") : acc);
                    }
                    MOE_TRACE_FLUSH;
                    return;
                }
            }
            down_flat<WF, NJD, true, RLS>(nun * nblk, astride, spitch, wave_id(), info, ready,
                               [&](const DNTask& t, int row, int i, float v) { pst[(t.prow + i) * nown + t.orow + row] = v; });
            __syncthreads();
            MOE_TRACE(11);
            // ---- E (slice mode): combine from LDS ----
            const LDS int* s_pair = tab + kTabPair;
            const LDS float* s_roww = (const LDS float*)(tab + kTabRowW);
            const bool bad = (call_fault | s_fault) != 0u;
            for (int i = threadIdx.x; i < M * nown; i += kThreads) {
                const int m = i / nown, hh = i - m * nown, h = h0 + hh;
                float acc = 0.0f;
                for (int j = 0; j < k; ++j) {
                    const int row = s_pair[m * k + j];
                    acc = fmaf(s_roww[row], pst[row * nown + hh], acc);
                }
                if (has_sh) acc += pst[(NP + m) * nown + hh];
                if (bad) acc = __builtin_nanf("");
                if constexpr (AF == MOE_FMT_F32)
                    ((float*)p.y)[(int64_t)m * H + h] = acc;
                else
                    ((uint16_t*)p.y)[(int64_t)m * H + h] = f32_to_bf16_rne(acc);
            }
        }
        MOE_TRACE_FLUSH;
        return;
    }

    // ---- D: routed down rows, unit by unit.  Partial outputs are staged in LDS and written once at
    //      the end when the whole range fits the staging area (no store in flight while the next
    //      unit's weights stream), else per pass ----
    {
        LDS float* pst = cst;
        const int cap = p.cst_bytes / 4;
        int64_t need = 0;
        for (int64_t q = d0; q < d1;) {
            const int u = (int)q / H;
            const int ha = (int)(q - (int64_t)u * H);
            const int hb = (int)min<int64_t>(H, ha + (d1 - q));
            q += hb - ha;
            need += (int64_t)(hb - ha) * __popc(s_mask[u]);
        }
        const bool once = need <= cap;
        // The range's segments (one per unit).  When every segment's SwiGLU rows fit the staging
        // area together and the partials fit at once, the whole range is one task list: one wait,
        // one staging pass, and the next task's loads stay in flight across segment boundaries.
        int nseg = 0;
        int sg_u[kMaxSeg], sg_ha[kMaxSeg], sg_hb[kMaxSeg];
        bool flat = once;
        {
            int64_t abytes = 0;
            for (int64_t q = d0; q < d1;) {
                const int u = (int)q / H;
                const int ha = (int)(q - (int64_t)u * H);
                const int hb = (int)min<int64_t>(H, ha + (d1 - q));
                q += hb - ha;
                if (nseg == kMaxSeg) {
                    flat = false;
                    break;
                }
                sg_u[nseg] = u;
                sg_ha[nseg] = ha;
                sg_hb[nseg] = hb;
                ++nseg;
                abytes += (int64_t)__popc(s_mask[u]) * I * 4;
            }
            if (abytes > p.lds_cst - p.lds_x) flat = false;
        }
        if (flat && nseg > 0) {
            // tasks of 12 rows (FP8 121.4 -> 120.7, bf16 177.4 -> 176.7 us at sixteen tokens) and
            // 16 rows for MXFP4 (92.3 -> 89.1 us)
            constexpr int RLU = WF == MOE_FMT_FP8 ? 3 : (WF == MOE_FMT_BF16 ? 6 : (WF == MOE_FMT_MXFP4 ? 2 : Geo<WF>::RL_D));
            constexpr int RTU = RLU * (64 / Geo<WF>::LPR_D);
            int toff[kMaxSeg + 1], aoff[kMaxSeg], poff[kMaxSeg];
            toff[0] = 0;
            int ao = 0, po = 0;
            for (int sg = 0; sg < nseg; ++sg) {
                const int t = __popc(s_mask[sg_u[sg]]);
                toff[sg + 1] = toff[sg] + (sg_hb[sg] - sg_ha[sg] + RTU - 1) / RTU;
                aoff[sg] = ao;
                poff[sg] = po;
                ao += t * I;  // floats
                po += (sg_hb[sg] - sg_ha[sg]) * t;
            }
            auto info = [&](int n, DNTask& t) {
                int sg = 0;
                while (sg + 1 < nseg && n >= toff[sg + 1]) ++sg;
                const int u = sg_u[sg], ha = sg_ha[sg];
                const int r0 = ha + (n - toff[sg]) * RTU;
                const int64_t e = uni(s_exp[u]);
                t.nrows = min(RTU, sg_hb[sg] - r0);
                t.t = __popc(uni(s_mask[u]));
                t.K = I;
                t.orow = r0 - ha;
                t.prow = poff[sg];
                t.lds = 0;
                t.w = (const uint8_t*)p.w.down + (e * H + r0) * rbI;
                t.s = scale_mat<WF>(p.w.down_s, e, H, I);
                t.srow = r0;
                t.acts = (const LDS float*)xs + aoff[sg];
            };
            auto ready = [&]() {
                wait_units(set, (uint32_t)(U * I), 0u, fault);
                MOE_TRACE(9);
                for (int sg = 0; sg < nseg; ++sg) {
                    const int u = sg_u[sg];
                    if constexpr (act_mode<WF>() == 2)
                        stage_rows_b16((LDS char*)((LDS float*)xs + aoff[sg]), act16 + (int64_t)s_off[u] * p.act_stride,
                                       p.act_stride, __popc(s_mask[u]), I, 4 * I);
                    else
                        stage_rows<act_mode<WF>()>((LDS float*)xs + aoff[sg], p.ws.act + (int64_t)s_off[u] * p.act_stride,
                                                   p.act_stride, __popc(s_mask[u]), I);
                }
                __syncthreads();
                MOE_TRACE(10);
            };
            down_flat<WF, NJD, false, RLU>(toff[nseg], I, 4 * I, wave_id(), info, ready, [&](const DNTask& t, int row, int i, float v) {
                pst[t.prow + (t.orow + row) * t.t + i] = v;
            });
            __syncthreads();
        }
        int pbase = 0;
        bool first = true;
        for (int64_t q = flat ? d1 : d0; q < d1;) {
            const int u = (int)q / H;
            const int ha = (int)(q - (int64_t)u * H);
            const int hb = (int)min<int64_t>(H, ha + (d1 - q));
            q += hb - ha;
            const int t = __popc(s_mask[u]);
            const int row0 = s_off[u];
            const int64_t e = s_exp[u];
            const int rows_per_pass = once ? hb - ha : max(RTD, (cap / t) / RTD * RTD);
            bool staged = false;
            // rows [ha, hb) in passes that fit the partial staging area
            for (int pa = ha; pa < hb; pa += rows_per_pass) {
                const int pb = min(hb, pa + rows_per_pass);
                auto ready = [&]() {
                    if (!staged) {
                        wait_units(set, (uint32_t)(U * I), 0u, fault);
                        if (first) MOE_TRACE(9);
                        if constexpr (act_mode<WF>() == 2)
                            stage_rows_b16((LDS char*)xs, act16 + (int64_t)row0 * p.act_stride, p.act_stride, t, I, 4 * I);
                        else
                            stage_rows<act_mode<WF>()>((LDS float*)xs, p.ws.act + (int64_t)row0 * p.act_stride, p.act_stride, t,
                                                       I);
                        __syncthreads();
                        if (first) MOE_TRACE(10);
                        staged = true;
                        first = false;
                    }
                };
                LDS float* pout = pst + pbase;
                auto out = [&](int row, int i, float v) { pout[row * t + i] = v; };
                down_run<WF, NJD, false>((const uint8_t*)p.w.down + (e * H + pa) * rbI, scale_mat<WF>(p.w.down_s, e, H, I),
                                         pa, I, pb - pa, (const LDS float*)xs, t, wave_id(), ready,
                                         [&](int row, int i, float v) { out(row, i, v); });
                __syncthreads();
                if (once) {
                    pbase += (pb - pa) * t;
                } else {
                    const int nr = pb - pa, n = nr * t;
                    for (int i = threadIdx.x; i < n; i += kThreads) {
                        const int m = i / nr, rr = i - m * nr;
                        st_dev(p.ws.part + (int64_t)(row0 + m) * H + pa + rr, pst[rr * t + m]);
                    }
                    __syncthreads();
                }
            }
        }
        if (once) {  // every partial of the range, in the order it was staged
            int base = 0;
            for (int64_t q = d0; q < d1;) {
                const int u = (int)q / H;
                const int ha = (int)(q - (int64_t)u * H);
                const int hb = (int)min<int64_t>(H, ha + (d1 - q));
                q += hb - ha;
                const int t = __popc(s_mask[u]);
                const int row0 = s_off[u];
                const int nr = hb - ha, n = nr * t;
                for (int i = threadIdx.x; i < n; i += kThreads) {  // token-major: contiguous runs of y
                    const int m = i / nr, rr = i - m * nr;
                    st_dev(p.ws.part + (int64_t)(row0 + m) * H + ha + rr, pst[base + rr * t + m]);
                }
                base += n;
            }
        }
    }
    MOE_TRACE(15);
    publish();
    MOE_TRACE(11);
    // every slice of y takes partials from most workgroups: one counter of finished workgroups
    if (threadIdx.x == 0) add_dev(line(set, kLineDownDone), 1u);

    // ---- E: combine this workgroup's slice of y ----
    if (nown > 0) {
        wait_geq(line(set, kLineDownDone), (uint32_t)G, fault);
        MOE_TRACE(12);
        call_fault = ld_dev(fault.flag);  // in flight with the partials' loads
        const LDS int* s_pair = tab + kTabPair;
        const LDS float* s_roww = (const LDS float*)(tab + kTabRowW);
        for (int i = threadIdx.x; i < M * nown; i += kThreads) {
            const int m = i / nown, hh = i - m * nown, h = h0 + hh;
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int row = s_pair[m * k + j];
                acc = fmaf(s_roww[row], ld_dev(p.ws.part + (int64_t)row * H + h), acc);
            }
            if (has_sh) acc += ysh[m * nown + hh];
            if ((call_fault | s_fault) != 0u) acc = __builtin_nanf("");
            if constexpr (AF == MOE_FMT_F32)
                ((float*)p.y)[(int64_t)m * H + h] = acc;
            else
                ((uint16_t*)p.y)[(int64_t)m * H + h] = f32_to_bf16_rne(acc);
        }
    }
    MOE_TRACE_FLUSH;
}

// ------------------------------------------------------------------------------------------
// launch
// ------------------------------------------------------------------------------------------

int round16(int64_t v) { return (int)((v + 15) / 16 * 16); }

constexpr int kLdsBudget = kLdsBytes - 512;  // dynamic LDS; the rest holds the static LDS variables

// Chunks per lane: NJ for the router and gate/up rows (K = H), NJD for the down rows (K = I, Is).
// Two instances per format: the Ling shapes (H <= 2560, I, Is <= 768) and small layers
// (H <= 512, I, Is <= 256); the host rejects larger shapes.
template <int WF>
void chunks(const Params& p, int* nj, int* njd) {
    const int ka = std::max(p.I, p.Is);
    *nj = (p.H / Geo<WF>::EPC + Geo<WF>::LPR_G - 1) / Geo<WF>::LPR_G;
    *njd = (ka / Geo<WF>::EPC + Geo<WF>::LPR_D - 1) / Geo<WF>::LPR_D;
}

// The launch plan of one call: modes and the LDS layout, on the host.
template <int AF, int WF>
hipError_t plan_t(Params& p, int G) {
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    int nj, njd;
    chunks<WF>(p, &nj, &njd);
    const bool fits = (nj <= 1 && njd <= 1) || (WF != MOE_FMT_F32 && nj <= 5 && njd <= 3);
    if (!fits) return hipErrorInvalidValue;  // no kernel instance for this shape
    const int M = p.M, H = p.H;
    const int64_t NP = (int64_t)p.k * M;
    const int ka = std::max(p.I, p.Is);
    const int nown = (H + G - 1) / G;
    // slice mode (each workgroup finishes its own y columns of every unit) while M * k is small,
    // and while all pair rows' SwiGLU outputs fit in 96 KB of LDS as bfloat16 (bf16 and MXFP4 at a
    // padded pitch for the matrix cores, FP8 packed for the vector path): every workgroup stages
    // all pair rows' SwiGLU outputs, every workgroup has the same rows to do, and there is no
    // partial write-out and no hand-off before the combine (six tokens, unit-major against slice:
    // bf16 73.5 -> 67.9 us, FP8 59.9 -> 54.0 us); otherwise unit-major down rows
    const bool mf_fit = (WF == MOE_FMT_BF16 || WF == MOE_FMT_MXFP4) && njd <= 3 && nown <= 16 &&
                        (NP + M) * (ka * 2 + 16) <= 96 * 1024;
    const bool f8_fit = WF == MOE_FMT_FP8 && nown <= 16 && (NP + M) * ka * 2 <= 96 * 1024;
    p.slice_mode = (NP <= 16 || mf_fit || f8_fit) ? 1 : 0;
    // from three tokens on, the M * E logits that every workgroup would read are more polling traffic
    // than one extra hand-off costs: workgroup m selects token m's experts and publishes them
    p.route_delegate = (!p.route_only && M >= 3 && M <= G) ? 1 : 0;
    // slice mode on the matrix cores (bf16 and MXFP4 weights, up to 16 rows per workgroup, K <= 768):
    // bfloat16 SwiGLU rows, swizzled weight windows
    p.sh_mfma = ((WF == MOE_FMT_BF16 || WF == MOE_FMT_MXFP4) && njd <= 3 && nown <= 16) ? 1 : 0;
    p.slice_mfma = (p.slice_mode && p.sh_mfma) ? 1 : 0;
    // staging area: routing scratch; routed SwiGLU results of one workgroup's tasks; down partials
    // (slice mode: [NP][nown]; unit-major: any size, larger means fewer passes)
    // per-token cost of a gate/up task and of a down row relative to the weight bytes (kCostBase),
    // from phase traces: bf16 down rows of 5-token units ran ~1.8x longer than 1-token ones; the
    // decode of E2M1 codes makes MXFP4 rows four times denser in work
    // MXFP4 gate/up rows on the matrix cores from 2 tokens on: each code is decoded once for all
    // tokens, so the work per weight byte no longer grows with the unit's token count.  At one token
    // the vector path decodes each code once as well and reads whole rows (MXFP4 22.3 against
    // 22.6 us).  FP8 from 3 tokens on (15 of the 16 token columns of a product would be empty at
    // one token: 34.0 against 31.8 us at Ling width)
    p.gu_mfma = ((WF == MOE_FMT_MXFP4 && M >= 2) || (WF == MOE_FMT_FP8 && M >= 3)) ? 1 : 0;
    // The shared expert's gate/up stays on the vector path at every token count: its rows run while
    // the routing is still pending, and on the matrix cores at 16 tokens the layer took longer
    // (FP8 136.0 against 129.7 us, MXFP4 106.3 against 103.9 us)
    // per-token cost of a down row (a row's bytes cost kCostBase = 8), from sweeps of the
    // whole-layer time: bf16 over 0, 1, 2, 3, 4 and 6 at 6 and 16 tokens (3 is fastest at both);
    // MXFP4 and FP8 over 3, 4, 6 and 9 at 6 and 16 tokens, with their SwiGLU rows as one bf16 plane
    // (4 is fastest: the vector path decodes every code once per token)
    p.cost_dn = WF == MOE_FMT_MXFP4 ? 4 : (WF == MOE_FMT_BF16 ? 3 : (WF == MOE_FMT_FP8 ? 4 : 0));
    // gate/up staging: MXFP4 tiles of 8 rows dealt round robin (at most ceil(T / G) per workgroup);
    // otherwise per wave the static share plus up to twice the average dynamic share (the split
    // the kernel makes from the actual number of units, bounded here by its maximum)
    const int64_t units = std::min<int64_t>(NP, p.E);
    int64_t cst, cst_nopart = -1;
    p.gu_part = -1;
    // MXFP4 slice mode from three tokens on keeps its gate/up rows in whole-item form
    // (gateup_mfma_mx); the other matrix-core gate/up runs through the line-wise form with its
    // transpose buffers (MXFP4 at one token: 23.0 against 24.2 us; at six tokens the item form is
    // faster, 43.4 against 44.2 us)
    const bool mx_items = WF == MOE_FMT_MXFP4 && p.slice_mode && M >= 3;
    p.gu_items = mx_items ? 1 : 0;
    p.gu_ksplit = 0;
    if (p.gu_mfma && mx_items) {
        // tiles of 8 rows dealt round robin; (tile, stage) items with partials in LDS while they fit
        const int64_t tiles = (units * p.I / 8 + G - 1) / G;
        const int64_t nstage = ((H / 32 + 3) / 4 + 9) / 10;  // stages of 10 groups of 4 MX blocks
        const int64_t pbytes = tiles * nstage * 16 * M * 4;
        p.gu_ksplit = pbytes <= 16 * 1024 ? 1 : 0;
        p.gu_part = (int)(tiles * 8 * M);
        cst = tiles * 8 * M * 4 + (p.gu_ksplit ? pbytes : 0);
        p.gu_cap = 0;
    } else if (p.gu_mfma) {
        // tiles of 8 rows per workgroup; (tile, stage) steps split into contiguous ranges per wave
        const int64_t tiles = (units * p.I / 8 + G - 1) / G;
        // outputs [tiles * 8][M], then two partial tiles per wave [kWaves][2][M][16] (the shared
        // expert's gate/up, at most one tile per workgroup, uses the same areas); dropped below if
        // the LDS budget has no room for them
        p.gu_part = (int)(tiles * 8 * M);
        cst = tiles * 8 * M * 4 + (int64_t)kWaves * 2 * M * 64;
        cst_nopart = tiles * 8 * M * 4;
        p.gu_cap = 0;
    } else {
        const int64_t rtg = rt_gate<WF>();
        const int64_t T = units * p.I / rtg;
        const int64_t Rs = 7 * T / (80 * (int64_t)G), dyn = T - (int64_t)kWaves * G * Rs;
        const int64_t ch = gu_chunk_tasks<WF>(H);
        p.gu_cap = (int)(Rs + 2 * ((dyn + kWaves * G - 1) / (kWaves * G)) + 2 * ch + 5);
        cst = (int64_t)kWaves * p.gu_cap * (rtg * M * 4 + 4) + kWaves * 4;
    }
    const int64_t cst_min = p.slice_mode ? (NP + M) * nown * 4 : 16 * 1024;
    // token rows 16 bytes further apart than their size: the 16 token columns of a matrix-core B
    // operand then start in 16 different bank groups
    p.xpitch = H * XB + 16;
    int64_t xb = std::max<int64_t>((int64_t)M * p.xpitch, (int64_t)M * ka * 4);
    if (p.slice_mode)
        xb = std::max<int64_t>(xb, (NP + M) * (p.slice_mfma ? 2 * ka + 16 : (act_mode<WF>() == 2 ? 2 : 4) * ka));
    p.lds_tab = 0;
    p.lds_x = round16(kTabWords * 4);
    p.lds_cst = p.lds_x + round16(xb);
    const int budget = kLdsBudget;
    const int gu_part0 = p.gu_part;
    // The routing scratch sits at the head of the slice-mode down window, which stays empty until
    // the routing has finished (at one bf16 token the window then holds all eight units' slices,
    // not seven); without a window, or one too small for it, it is part of the staging area.
    // slice mode keeps an LDS window of routed down rows for bf16 and f32 weights; MXFP4 and FP8
    // slice rows are read from global memory in the down phase (their windows were copied one unit
    // at a time, each copy waiting for the last, and the MXFP4 gate/up waited for the whole window:
    // without them MXFP4 took 24.2 against 26.0 us at one token and 44.5 against 45.8 at six, FP8
    // 28.0 against 28.4 at one token)
    const bool win = p.slice_mode && !p.route_only && (WF == MOE_FMT_BF16 || WF == MOE_FMT_F32);
    for (int sel_win = win ? 1 : 0;; sel_win = 0) {
        const int64_t floor = std::max<int64_t>(cst_min, sel_win ? 0 : kSelBytes);
        p.gu_part = gu_part0;
        p.cst_bytes = round16(std::max<int64_t>(cst, floor));
        // the fixed regions; a second pass without the partial tiles if they do not fit
        for (int pass = 0;; ++pass) {
            p.lds_sh = p.lds_cst + p.cst_bytes;
            p.lds_ysh = p.lds_sh + round16(p.Is > 0 ? nown * row_bytes<WF>(p.Is) : 0);
            p.lds_scl = p.lds_ysh + round16((int64_t)M * nown * 4);
            // MXFP4 scale bytes of the shared expert's slice rows in LDS when its down rows run on
            // the matrix cores (copied in 4-byte pieces: whole dwords per row block)
            p.scl_sh = 0;
            if constexpr (WF == MOE_FMT_MXFP4)
                if (!p.route_only && p.sh_mfma && p.Is > 0 && (p.Is / 32) % 4 == 0)
                    p.scl_sh = (int)round16((int64_t)nown * (p.Is / 32));
            p.lds_tr = p.lds_scl + p.scl_sh;
            p.lds_dn = p.lds_tr + (p.gu_mfma && !mx_items && !p.route_only ? kWaves * 4096 : 0);
            if (pass == 0 && p.lds_dn > budget && cst_nopart >= 0) {  // no room for the partial tiles
                p.gu_part = -1;
                p.cst_bytes = round16(std::max<int64_t>(cst_nopart, floor));
                continue;
            }
            break;
        }
        // slice mode: the rest of LDS is the window its routed down rows stream into (unit-major
        // down rows stream from global memory)
        p.dn_bytes = win ? std::max(0, (budget - p.lds_dn) / 16 * 16) : 0;
        if (sel_win && p.dn_bytes < kSelBytes) continue;
        p.lds_sel = sel_win ? p.lds_dn : p.lds_cst;
        break;
    }
    p.lds_total = p.lds_dn + p.dn_bytes;
    if (p.lds_total > budget) return hipErrorInvalidValue;
    return hipSuccess;
}

constexpr int kMaxDevices = 64;

// Per device and kernel instance, once: allow the whole LDS budget and check that one workgroup
// fits a CU.  Idempotent, so concurrent first calls are harmless.
template <typename K>
hipError_t prepare(K kern, int dev) {
    static std::atomic<int> state[kMaxDevices];  // 0 unknown, 1 ready, 2 failed
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int st = state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        st = 2;
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) ==
            hipSuccess) {
            int occ = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)kern, kThreads, kLdsBudget) ==
                    hipSuccess &&
                occ >= 1)
                st = 1;
        }
        state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? hipSuccess : hipErrorInvalidConfiguration;
}

template <int AF, int WF, int NJ, int NJD>
hipError_t launch_t(const Params& p, int G, int dev, hipStream_t s) {
    auto go = [&](auto kern) -> hipError_t {
        const hipError_t e = prepare(kern, dev);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(G), dim3(kThreads), p.lds_total, s, p);
        return hipGetLastError();
    };
    return p.slice_mode ? go(k_layer<AF, WF, NJ, NJD, 1>) : go(k_layer<AF, WF, NJ, NJD, 0>);
}

template <int AF, int WF>
hipError_t launch_fmt(const Params& p, int G, int dev, hipStream_t s) {
    int nj, njd;
    chunks<WF>(p, &nj, &njd);
    if (nj <= 1 && njd <= 1) return launch_t<AF, WF, 1, 1>(p, G, dev, s);
    if constexpr (WF != MOE_FMT_F32)
        if (nj <= 5 && njd <= 3) return launch_t<AF, WF, 5, 3>(p, G, dev, s);
    return hipErrorInvalidValue;
}

}  // namespace

#ifdef MOE_PHASE_TRACE
extern "C" int moe_trace_set(void* buf) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_moe_trace), &buf, sizeof(buf)) == hipSuccess ? 0 : -1;
}
#endif

hipError_t plan_layer(Params& p, int G) {
    if (G < 1 || G > kMaxGrid) return hipErrorInvalidValue;
    if (p.act_fmt == MOE_FMT_F32) return plan_t<MOE_FMT_F32, MOE_FMT_F32>(p, G);
    if (p.w_fmt == MOE_FMT_BF16) return plan_t<MOE_FMT_BF16, MOE_FMT_BF16>(p, G);
    if (p.w_fmt == MOE_FMT_FP8) return plan_t<MOE_FMT_BF16, MOE_FMT_FP8>(p, G);
    return plan_t<MOE_FMT_BF16, MOE_FMT_MXFP4>(p, G);
}

hipError_t launch_layer(const Params& p, int G, hipStream_t s) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (p.act_fmt == MOE_FMT_F32) return launch_fmt<MOE_FMT_F32, MOE_FMT_F32>(p, G, dev, s);
    if (p.w_fmt == MOE_FMT_BF16) return launch_fmt<MOE_FMT_BF16, MOE_FMT_BF16>(p, G, dev, s);
    if (p.w_fmt == MOE_FMT_FP8) return launch_fmt<MOE_FMT_BF16, MOE_FMT_FP8>(p, G, dev, s);
    return launch_fmt<MOE_FMT_BF16, MOE_FMT_MXFP4>(p, G, dev, s);
}

}  // namespace moe
