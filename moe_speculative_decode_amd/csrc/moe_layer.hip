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
//      rows into LDS; compute this workgroup's router rows (fp32 logits) and arrive at the
//      routing barrier; compute a share of the shared expert's gate/up rows.
//   B  wait for the routing barrier; every workgroup redoes the per-token top-k and the batch
//      compaction (distinct experts ascending, token bitmask and pair rows per unit) in its own
//      LDS, so no second hand-off is needed; workgroup 0 writes the caller-visible outputs.
//      Then the shared expert's down rows of this workgroup's y slice, from LDS.
//   C  an equal share of all routed units' gate/up rows: each weight row is read once and
//      applied to every token of its unit, silu(g) * v in fp32.  Meanwhile as many of this
//      workgroup's routed down rows as fit stream into LDS.
//   D  an equal share of all routed units' down rows, writing fp32 partial outputs per pair row
//      once the unit's SwiGLU rows are complete.
//   E  every workgroup owns a fixed slice of y's columns: once all routed partials of the slice
//      have landed it sums each token's partials in slot order, adds the shared expert and
//      casts once.
//
// The streaming loops never store to global memory: vector memory operations retire in order
// on gfx9, so a store in the loop would make the next wait for prefetched weights also wait
// for the store to be acknowledged.  Results are staged in LDS and written at the end of a
// phase.  Data that crosses workgroups goes through device-scope (sc1) stores and loads, and a
// counter is bumped only after the stores have completed; there are no cache-wide fences.
// Every wait is bounded: on a timeout the status word is flagged and the kernel still finishes.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

#define LDS __attribute__((address_space(3)))

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
// The wave's index in the workgroup, as a scalar the compiler knows to be wave-uniform.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

__device__ __forceinline__ uint64_t lanes_below() {
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ------------------------------------------------------------------------------------------
// number formats and weight geometry
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

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
    static constexpr int EPC = 8, LPR_G = 64, RL_G = 2, LPR_D = 32, RL_D = 2;
};
template <>
struct Geo<MOE_FMT_MXFP4> {
    static constexpr int EPC = 32, LPR_G = 16, RL_G = 1, LPR_D = 8, RL_D = 1;
};
template <int WF>
__host__ __device__ constexpr int rt_gate() { return Geo<WF>::RL_G * (64 / Geo<WF>::LPR_G); }
template <int WF>
__host__ __device__ constexpr int rt_down() { return Geo<WF>::RL_D * (64 / Geo<WF>::LPR_D); }

// bytes of one row of K elements (MXFP4: the codes; the scales are K / 32 bytes more)
template <int WF>
__host__ __device__ constexpr int64_t row_bytes(int64_t K) {
    return WF == MOE_FMT_F32 ? 4 * K : (WF == MOE_FMT_BF16 ? 2 * K : K / 2);
}

struct Chunk {
    u32x4 q;
    uint32_t s;  // MXFP4 scale byte
};

// Makes the compiler wait for a chunk's load here, in straight-line code, and treat the value as
// an ordinary register afterwards, so the waits inside the compute loops never drain the next
// task's prefetch.
template <int WF>
__device__ __forceinline__ void settle(Chunk& r) {
    if constexpr (WF == MOE_FMT_MXFP4)
        asm volatile("" : "+v"(r.q), "+v"(r.s));
    else
        asm volatile("" : "+v"(r.q));
}

// chunk c of a weight row in global memory (streamed once: non-temporal)
template <int WF>
__device__ __forceinline__ void ld_chunk(Chunk& r, const uint8_t* row, const uint8_t* srow, int c) {
    r.q = __builtin_nontemporal_load((const u32x4*)(row + 16 * c));
    if constexpr (WF == MOE_FMT_MXFP4) r.s = __builtin_nontemporal_load(srow + c);
}
// chunk c of a weight row held in LDS (the MXFP4 scales stay in global memory)
template <int WF>
__device__ __forceinline__ void ld_chunk_lds(Chunk& r, const LDS uint8_t* row, const uint8_t* srow, int c) {
    r.q = *(const LDS u32x4*)(row + 16 * c);
    if constexpr (WF == MOE_FMT_MXFP4) r.s = srow[c];
}

// Reinterprets a dword as two bf16.  Takes the dword by value: bit-casting a vector component
// lvalue directly (v.y) makes clang read the vector's first element instead.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Dot of weight chunk c with the matching elements of a token row x (LDS; bf16, or binary32 for
// the binary32 layer), fp32 accumulation.
template <int AF, int WF>
__device__ __forceinline__ float dot_x(const Chunk& r, const LDS char* xrow, int c, float acc) {
    if constexpr (WF == MOE_FMT_BF16) {
        const u32x4 x = *(const LDS u32x4*)(xrow + 16 * c);
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        const uint32_t x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(x0), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(x1), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(x2), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(x3), acc, false);
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
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0), as_bf16x2(x0), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1), as_bf16x2(x1), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2), as_bf16x2(x2), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3), as_bf16x2(x3), acc, false);
        }
    } else {
        const f32x4 x = *(const LDS f32x4*)(xrow + 16 * c);
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        acc = fmaf(__uint_as_float(w0), x[0], acc);
        acc = fmaf(__uint_as_float(w1), x[1], acc);
        acc = fmaf(__uint_as_float(w2), x[2], acc);
        acc = fmaf(__uint_as_float(w3), x[3], acc);
    }
    return acc;
}

// Dot of weight chunk c with the matching elements of an fp32 row (LDS) -- the SwiGLU output
// consumed by the down projection.
template <int WF>
__device__ __forceinline__ float dot_a(const Chunk& r, const LDS float* arow, int c, float acc) {
    if constexpr (WF == MOE_FMT_BF16) {
        const LDS f32x4* ap = (const LDS f32x4*)(arow + 8 * c);
        const f32x4 a0 = ap[0], a1 = ap[1];
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        acc = fmaf(bf16lo(w0), a0[0], acc);
        acc = fmaf(bf16hi(w0), a0[1], acc);
        acc = fmaf(bf16lo(w1), a0[2], acc);
        acc = fmaf(bf16hi(w1), a0[3], acc);
        acc = fmaf(bf16lo(w2), a1[0], acc);
        acc = fmaf(bf16hi(w2), a1[1], acc);
        acc = fmaf(bf16lo(w3), a1[2], acc);
        acc = fmaf(bf16hi(w3), a1[3], acc);
    } else if constexpr (WF == MOE_FMT_MXFP4) {
        const LDS f32x4* ap = (const LDS f32x4*)(arow + 32 * c);
        const float sc = e8m0_to_f32(r.s);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w = r.q[d];
            const f32x4 a0 = ap[2 * d], a1 = ap[2 * d + 1];
            const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
            const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
            const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
            const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
            acc = fmaf(p0[0], a0[0], acc);
            acc = fmaf(p0[1], a0[1], acc);
            acc = fmaf(p1[0], a0[2], acc);
            acc = fmaf(p1[1], a0[3], acc);
            acc = fmaf(p2[0], a1[0], acc);
            acc = fmaf(p2[1], a1[1], acc);
            acc = fmaf(p3[0], a1[2], acc);
            acc = fmaf(p3[1], a1[3], acc);
        }
    } else {
        const f32x4 a = *(const LDS f32x4*)(arow + 4 * c);
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        acc = fmaf(__uint_as_float(w0), a[0], acc);
        acc = fmaf(__uint_as_float(w1), a[1], acc);
        acc = fmaf(__uint_as_float(w2), a[2], acc);
        acc = fmaf(__uint_as_float(w3), a[3], acc);
    }
    return acc;
}

__device__ __forceinline__ float silu_mul(float g, float v) { return g / (1.0f + __expf(-g)) * v; }

// LDS tables of the batch dispatch, in words
constexpr int kTabMask = 0;                                  // [kMaxExperts + 1] token bitmask per unit
constexpr int kTabOff = kTabMask + kMaxExperts + 1;          // [kMaxExperts + 2] first pair row per unit
constexpr int kTabExp = kTabOff + kMaxExperts + 2;           // [kMaxExperts + 1] expert id per unit
constexpr int kTabPair = kTabExp + kMaxExperts + 1;          // [kMaxTokens * kMaxTopK] pair row of (m, j)
constexpr int kTabRowW = kTabPair + kMaxTokens * kMaxTopK;   // [kMaxTokens * (kMaxTopK + 1)] weight per row
constexpr int kTabMisc = kTabRowW + kMaxTokens * (kMaxTopK + 1);  // [8] U, flags
constexpr int kTabWords = (kTabMisc + 8 + 3) / 4 * 4;
// routing scratch (token masks, expert row offsets, per-token ids / weights / logits), in the
// staging area
constexpr int kSelBytes = (2 * kMaxExperts + 3 * kMaxTokens * kMaxTopK) * 4;
constexpr int kMaxPre = 4;  // routed down-row segments prefetched into LDS per workgroup

constexpr int kSpinLimit = 1 << 20;  // ~1 s of polling; normal waits are microseconds

// Phase timestamps for performance analysis, compiled out unless MOE_PHASE_TRACE is defined.
#ifdef MOE_PHASE_TRACE
__device__ uint64_t* g_moe_trace;
#define MOE_TRACE(slot)                                                                             \
    do {                                                                                            \
        if (threadIdx.x == 0 && g_moe_trace) g_moe_trace[blockIdx.x * 32 + (slot)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define MOE_TRACE(slot) \
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
// Thread 0 waits until *c >= target (bounded); the whole workgroup continues together.
__device__ __forceinline__ void wait_geq(const uint32_t* c, uint32_t target, uint32_t* status) {
    if (threadIdx.x == 0) {
        int i = 0;
        while (ld_dev(c) < target && i < kSpinLimit) {
            __builtin_amdgcn_s_sleep(1);
            ++i;
        }
        if (i == kSpinLimit) atomicOr(status, kStatusTimeout);
    }
    __syncthreads();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ uint32_t* line(uint32_t* set, int l) { return set + (int64_t)l * kLineWords; }

// Starts an asynchronous copy of n bytes (a multiple of 16) from global memory to LDS with every
// wave of the workgroup.  The data is usable after the issuing waves' next s_waitcnt vmcnt(0) and
// a workgroup barrier.
__device__ __forceinline__ void async_to_lds(char* lds, const uint8_t* src, int n) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    constexpr int chunk = 64 * 16;
    for (int base = wave * chunk; base < n; base += kWaves * chunk) {
        if (base + lane * 16 < n) {
            auto* dst = (LDS void*)(lds + base);
            __builtin_amdgcn_global_load_lds(src + base + lane * 16, dst, 16, 0, 0);
        }
    }
}

// fp32 logits rows are padded to whole 16-byte chunks
__host__ __device__ __forceinline__ int logit_stride(int E) { return (E + 3) / 4 * 4; }

// Stages `tcount` fp32 rows of K elements (global rows of `stride` floats from `src`) into LDS
// [tcount][K] with 16-byte device-scope loads.
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
            if (i < n) ((LDS f32x4*)dst)[i] = v[u];
        }
    }
}

// ------------------------------------------------------------------------------------------
// routing: top-k of one token with one wave, batch compaction with one workgroup
// ------------------------------------------------------------------------------------------

// Top-k of one token's E logits with one wave.  Lane l owns experts 8l .. 8l+7, read with two
// 16-byte device-scope loads.  Order: larger logit first, equal logits -> lower expert id first.
// Every round takes the wave-wide maximum of the lanes' current maxima; among equal maxima the
// lowest lane holds the lowest id, and inside a lane the lowest index is kept, so ties resolve
// to the lower id.  The winning lane drops that logit and recomputes its maximum.  Writes ids,
// logits and softmax-over-the-k weights in order.  Every id written is in [0, E).
__device__ __forceinline__ void wave_topk(const float* lrow, int E, int k, LDS int* out_id, LDS float* out_w,
                                          LDS float* out_v) {
    const int lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rs = dev_rsrc(lrow, (uint32_t)E * 4);  // loads past E return 0
    const f32x4 a = ld_dev16(rs, (uint32_t)lane * 32), b = ld_dev16(rs, (uint32_t)lane * 32 + 16);
    float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (8 * lane + i >= E) v[i] = -INFINITY;
    auto local_max = [&](float& m, int& mi) {
        m = v[0];
        mi = 0;
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            const bool gt = v[i] > m;
            m = gt ? v[i] : m;
            mi = gt ? i : mi;
        }
    };
    float lm;
    int li;
    local_max(lm, li);
    float my_v = -INFINITY;
    int my_id = 0;
    for (int r = 0; r < k; ++r) {
        const float mx = wave_max_bcast(lm);
        const uint64_t ball = __ballot(lm == mx);
        const int wl = ball ? __ffsll((unsigned long long)ball) - 1 : 0;  // no match only for NaN inputs
        const int wi = __builtin_amdgcn_readlane(li, wl);
        if (lane == r) {
            my_v = mx;
            my_id = min(8 * wl + wi, E - 1);
        }
        if (lane == wl) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = i == wi ? -INFINITY : v[i];
            local_max(lm, li);
        }
    }
    // weights: softmax over the k selected logits (lanes 0..k-1 of row 0; k <= 16)
    const float top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
    const float ex = lane < k ? __expf(my_v - top) : 0.0f;
    const float z = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, row16_sum(ex)), 0));
    if (lane < k) {
        out_id[lane] = my_id;
        out_v[lane] = my_v;
        out_w[lane] = ex / z;
    }
}

// Exclusive prefix over the lanes of a non-negative count below 2^BITS, and the wave total.
template <int BITS>
__device__ __forceinline__ int wave_excl(int c, int* total) {
    int pre = 0, tot = 0;
    const uint64_t below = lanes_below();
#pragma unroll
    for (int bit = 0; bit < BITS; ++bit) {
        const uint64_t b = __ballot((c >> bit) & 1);
        pre += __popcll(b & below) << bit;
        tot += __popcll(b) << bit;
    }
    *total = tot;
    return pre;
}

// Top-k of all M tokens and the batch compaction into this workgroup's LDS tables.  Workgroup 0
// (`publish_outputs`) also writes the caller-visible routing outputs.  Returns U.
__device__ __forceinline__ int route_and_compact(const Params& p, LDS int* tab, LDS char* sel, bool publish_outputs) {
    const int E = p.E, M = p.M, k = p.k, NP = M * k;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const bool has_sh = p.Is > 0;
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

    for (int m = wave; m < M; m += kWaves)
        wave_topk(p.ws.logits + (int64_t)m * logit_stride(E), E, k, sid + m * k, sw + m * k, sv + m * k);
    __syncthreads();
    MOE_TRACE(13);
    if (wave == 0) {
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
        int U, tot_rows;
        int u = wave_excl<4>(npres, &U);            // first unit index of this lane
        int off = wave_excl<8>(nrows, &tot_rows);   // first pair row of this lane
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
        for (int q = threadIdx.x; q < NP; q += kThreads) {
            const int row = s_pair[q];
            if (p.topk_ids) p.topk_ids[q] = sid[q];
            if (p.topk_w) p.topk_w[q] = sw[q];
            if (p.disp.row_token) p.disp.row_token[row] = q / k;
            if (p.disp.row_slot) p.disp.row_slot[row] = q % k;
            if (p.disp.row_weight) p.disp.row_weight[row] = sw[q];
        }
        for (int u = threadIdx.x; u < U + (has_sh ? 1 : 0); u += kThreads) {
            if (p.disp.unit_expert) p.disp.unit_expert[u] = s_exp[u];
            if (p.disp.unit_off) p.disp.unit_off[u] = s_off[u];
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

// Router rows [e0, e1): one wave per row, every token; fp32 logits by device-scope stores.  Each
// wave's first row was loaded before the token rows landed in LDS (`first`).  The weight is in
// the activation format, so its geometry is the gate/up geometry of that format.
template <int AF, int NJ>
__device__ __forceinline__ void router_rows(const Params& p, const LDS char* xs, int e0, int e1, const Chunk (&first)[NJ]) {
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
        for (int j = 0; j < NJ; ++j) settle<AF>(r[j]);
        for (int m = 0; m < M; ++m) {
            const LDS char* xrow = xs + (int64_t)m * H * XB;
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c = lane + 64 * j;
                if (c < nch) acc = dot_x<AF, AF>(r[j], xrow, c, acc);
            }
            const float s = wave_sum_hi(acc);
            if (lane == 63) st_dev(p.ws.logits + (int64_t)m * logit_stride(E) + e, s);
        }
    }
}

// One gate/up task: RT consecutive rows of a unit's gate and up matrices, applied to the unit's
// tokens.  Pointers are at the task's first row.
struct GUTask {
    const uint8_t* g;
    const uint8_t* u;
    const uint8_t* gs;  // MXFP4 scales of those rows
    const uint8_t* us;
    uint32_t mask;      // the unit's tokens
    int slot;           // staging row of the task's first row
};

// This wave's gate/up tasks q = qa + wave, qa + wave + kWaves, ... < qb.  info(q, task) describes
// task q.  silu(g) * v of staged row s and the unit's i-th token goes to stage[s * M + i].  Each
// wave keeps the next task's loads in flight while it computes the current one; the prefetch is
// unconditional (the last task re-reads itself) so the number of loads in flight is static and
// the compiler waits for exactly the task it needs.
template <int AF, int WF, int NJ, typename Info>
__device__ __forceinline__ void gateup_run(const Params& p, const LDS char* xs, LDS float* stage, int qa, int qb,
                                           Info info) {
    constexpr int LPR = Geo<WF>::LPR_G, RL = Geo<WF>::RL_G;
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    const int lane = threadIdx.x & 63, gi = lane / LPR, sl = lane % LPR;
    const int H = p.H, M = p.M;
    const int nch = H / Geo<WF>::EPC;
    const int64_t rb = row_bytes<WF>(H), sb = H / 32;
    int q = qa + wave_id();
    if (q >= qb) return;
    Chunk ga[RL][NJ], ua[RL][NJ], gb[RL][NJ], ub[RL][NJ];
    GUTask ta, tb;
    auto load = [&](Chunk(&g)[RL][NJ], Chunk(&u)[RL][NJ], const GUTask& t) {
#pragma unroll
        for (int rl = 0; rl < RL; ++rl) {
            const int64_t ro = gi * RL + rl;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c = min(sl + LPR * j, nch - 1);
                ld_chunk<WF>(g[rl][j], t.g + ro * rb, t.gs + ro * sb, c);
                ld_chunk<WF>(u[rl][j], t.u + ro * rb, t.us + ro * sb, c);
            }
        }
    };
    auto settle_all = [](Chunk(&g)[RL][NJ], Chunk(&u)[RL][NJ]) {
#pragma unroll
        for (int rl = 0; rl < RL; ++rl)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                settle<WF>(g[rl][j]);
                settle<WF>(u[rl][j]);
            }
    };
    auto compute = [&](const Chunk(&g)[RL][NJ], const Chunk(&u)[RL][NJ], const GUTask& t) {
        int i = 0;
        for (uint32_t m = t.mask; m; m &= m - 1u, ++i) {
            const int tok = __builtin_ctz(m);
            const LDS char* xrow = xs + (int64_t)tok * H * XB;
            float ag[RL], au[RL];
#pragma unroll
            for (int rl = 0; rl < RL; ++rl) ag[rl] = au[rl] = 0.0f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c = sl + LPR * j;
                if (c < nch) {
#pragma unroll
                    for (int rl = 0; rl < RL; ++rl) {
                        ag[rl] = dot_x<AF, WF>(g[rl][j], xrow, c, ag[rl]);
                        au[rl] = dot_x<AF, WF>(u[rl][j], xrow, c, au[rl]);
                    }
                }
            }
#pragma unroll
            for (int rl = 0; rl < RL; ++rl) {
                const float gs = group_sum<LPR>(ag[rl]);
                const float us = group_sum<LPR>(au[rl]);
                if (sl == LPR - 1) stage[(t.slot + gi * RL + rl) * M + i] = silu_mul(gs, us);
            }
        }
    };
    info(q, ta);
    load(ga, ua, ta);
    while (true) {
        info(min(q + kWaves, qb - 1), tb);
        load(gb, ub, tb);
        settle_all(ga, ua);
        compute(ga, ua, ta);
        q += kWaves;
        if (q >= qb) break;
        info(min(q + kWaves, qb - 1), ta);
        load(ga, ua, ta);
        settle_all(gb, ub);
        compute(gb, ub, tb);
        q += kWaves;
        if (q >= qb) break;
    }
}

// Down rows [0, nrows) of one unit (row 0 at wbase / sbase, in LDS when FROM_LDS) with K inputs,
// for the unit's t tokens whose fp32 activations are at acts ([t][K], LDS).  Tasks of RT rows go
// to the waves round robin.  `ready()` is called by every wave after its first loads are issued
// and before any compute (it may contain workgroup barriers).  out(row, i, value) receives each
// result in the row's last lane.
template <int WF, int NJD, bool FROM_LDS, typename Ready, typename Out>
__device__ __forceinline__ void down_run(const uint8_t* wbase, const uint8_t* sbase, int K, int nrows,
                                         const LDS float* acts, int t, Ready ready, Out out) {
    constexpr int LPR = Geo<WF>::LPR_D, RL = Geo<WF>::RL_D, RT = rt_down<WF>();
    const int lane = threadIdx.x & 63, gi = lane / LPR, sl = lane % LPR;
    const int nch = K / Geo<WF>::EPC;
    const int64_t rb = row_bytes<WF>(K), sb = K / 32;
    const int ntask = (nrows + RT - 1) / RT;
    int n = wave_id();
    Chunk wa[RL][NJD], wb[RL][NJD];
    auto load = [&](Chunk(&w)[RL][NJD], int task) {
#pragma unroll
        for (int rl = 0; rl < RL; ++rl) {
            const int64_t row = min(task * RT + gi * RL + rl, nrows - 1);
#pragma unroll
            for (int j = 0; j < NJD; ++j) {
                const int c = min(sl + LPR * j, nch - 1);
                if constexpr (FROM_LDS)
                    ld_chunk_lds<WF>(w[rl][j], (const LDS uint8_t*)wbase + row * rb, sbase + row * sb, c);
                else
                    ld_chunk<WF>(w[rl][j], wbase + row * rb, sbase + row * sb, c);
            }
        }
    };
    auto settle_all = [](Chunk(&w)[RL][NJD]) {
#pragma unroll
        for (int rl = 0; rl < RL; ++rl)
#pragma unroll
            for (int j = 0; j < NJD; ++j) settle<WF>(w[rl][j]);
    };
    auto compute = [&](const Chunk(&w)[RL][NJD], int task) {
        for (int i = 0; i < t; ++i) {
            const LDS float* arow = acts + i * K;
            float acc[RL];
#pragma unroll
            for (int rl = 0; rl < RL; ++rl) acc[rl] = 0.0f;
#pragma unroll
            for (int j = 0; j < NJD; ++j) {
                const int c = sl + LPR * j;
                if (c < nch) {
#pragma unroll
                    for (int rl = 0; rl < RL; ++rl) acc[rl] = dot_a<WF>(w[rl][j], arow, c, acc[rl]);
                }
            }
#pragma unroll
            for (int rl = 0; rl < RL; ++rl) {
                const float s = group_sum<LPR>(acc[rl]);
                const int row = task * RT + gi * RL + rl;
                if (sl == LPR - 1 && row < nrows) out(row, i, s);
            }
        }
    };
    if (n < ntask) load(wa, n);
    ready();
    if (n >= ntask) return;
    while (true) {
        load(wb, min(n + kWaves, ntask - 1));
        settle_all(wa);
        compute(wa, n);
        n += kWaves;
        if (n >= ntask) break;
        load(wa, min(n + kWaves, ntask - 1));
        settle_all(wb);
        compute(wb, n);
        n += kWaves;
        if (n >= ntask) break;
    }
}

// First row of workgroup o's slice of y's columns: [slice0(o), slice0(o + 1)).
__device__ __forceinline__ int slice0(int H, int G, int o) { return (int)((int64_t)H * o / G); }
// The workgroup whose slice holds column h.
__device__ __forceinline__ int slice_of(int H, int G, int h) {
    int o = (int)(((int64_t)h * G) / H);
    while (o + 1 < G && slice0(H, G, o + 1) <= h) ++o;
    while (o > 0 && slice0(H, G, o) > h) --o;
    return o;
}

// ------------------------------------------------------------------------------------------
// the layer kernel
// ------------------------------------------------------------------------------------------

template <int AF, int WF, int NJ, int NJD>
__global__ __launch_bounds__(kThreads) void k_layer(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int G = gridDim.x, b = blockIdx.x;
    const int H = p.H, E = p.E, M = p.M, k = p.k, I = p.I, Is = p.Is;
    const int NP = M * k;
    const bool has_sh = Is > 0;
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    constexpr int RTG = rt_gate<WF>();
    constexpr int RTD = rt_down<WF>();
    LDS char* lds = (LDS char*)smem;
    LDS int* tab = (LDS int*)(lds + p.lds_tab);
    LDS char* xs = lds + p.lds_x;
    LDS float* cst = (LDS float*)(lds + p.lds_cst);
    LDS char* shw = lds + p.lds_sh;
    LDS float* ysh = (LDS float*)(lds + p.lds_ysh);
    LDS char* dnw = lds + p.lds_dn;
    __shared__ uint32_t s_call;
    __shared__ int s_arrive;
    MOE_TRACE(0);

    // this workgroup's slice of y's columns (shared down rows, and the final combine)
    const int h0 = slice0(H, G, b), h1 = slice0(H, G, b + 1), nown = h1 - h0;
    const int64_t rbIs = row_bytes<WF>(Is);

    // ---- A: call index, token rows, router rows, shared-expert down rows of the slice ----
    if (threadIdx.x == 0) {
        s_call = ld_dev(p.ws.hdr + kHdrCall);
        s_arrive = 0;
    }
    async_to_lds((char*)xs, (const uint8_t*)p.x, M * H * XB);
    const int e0 = (int)((int64_t)E * b / G), e1 = (int)((int64_t)E * (b + 1) / G);
    Chunk rfirst[NJ];
    {
        const int e = e0 + wave_id(), lane = threadIdx.x & 63, nch = H / Geo<AF>::EPC;
        if (e < e1) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                ld_chunk<AF>(rfirst[j], (const uint8_t*)p.wr + (int64_t)e * H * XB, nullptr, min(lane + 64 * j, nch - 1));
        }
    }
    if (has_sh && !p.route_only && nown > 0)
        async_to_lds((char*)shw, (const uint8_t*)p.w.sh_down + h0 * rbIs, (int)(nown * rbIs));
    __builtin_amdgcn_s_waitcnt(0);  // token rows (and the slice's shared down rows) in LDS
    __syncthreads();
    MOE_TRACE(1);
    const uint32_t call = s_call;
    uint32_t* set = p.ws.ctr + (int64_t)(call & 1u) * kSetWords;
    if (b == 0) {
        uint32_t* nxt = p.ws.ctr + (int64_t)((call + 1u) & 1u) * kSetWords;
        const int nl = kLineOwner0 + G;
        for (int l = threadIdx.x; l < nl; l += kThreads) line(nxt, l)[0] = 0u;
    }
    // router rows; the last router wave of the workgroup arrives for it once its stores landed
    {
        const int nrw = min(e1 - e0, kWaves);  // waves with router rows
        const int s = b % kRouteSubs;
        const uint32_t members = G / kRouteSubs + (s < G % kRouteSubs ? 1 : 0);
        if (wave_id() < nrw) {
            router_rows<AF, NJ>(p, xs, e0, e1, rfirst);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if ((threadIdx.x & 63) == 0 && atomicAdd(&s_arrive, 1) + 1 == nrw) {
                if (add_dev(line(set, s), 1u) + 1u == members) add_dev(line(set, kLineRouteTop), 1u);
            }
        } else if (nrw == 0 && threadIdx.x == 0) {
            if (add_dev(line(set, s), 1u) + 1u == members) add_dev(line(set, kLineRouteTop), 1u);
        }
    }
    MOE_TRACE(2);
    if (p.route_only && b != 0) return;

    // ---- A': shared expert gate/up (needs no routing) ----
    if (has_sh && !p.route_only) {
        const int T = Is / RTG;
        const int qa = (int)((int64_t)T * b / G), qb = (int)((int64_t)T * (b + 1) / G);
        if (qb > qa) {
            const uint32_t all = (1u << M) - 1u;
            gateup_run<AF, WF, NJ>(p, xs, cst, qa, qb, [&](int q, GUTask& t) {
                const int64_t r0 = (int64_t)q * RTG;
                t.g = (const uint8_t*)p.w.sh_gate + r0 * row_bytes<WF>(H);
                t.u = (const uint8_t*)p.w.sh_up + r0 * row_bytes<WF>(H);
                t.gs = WF == MOE_FMT_MXFP4 ? p.w.sh_gate_s + r0 * (H / 32) : nullptr;
                t.us = WF == MOE_FMT_MXFP4 ? p.w.sh_up_s + r0 * (H / 32) : nullptr;
                t.mask = all;
                t.slot = (q - qa) * RTG;
            });
            __syncthreads();
            const int n = (qb - qa) * RTG * M;
            for (int i = threadIdx.x; i < n; i += kThreads) {
                const int r = qa * RTG + i / M, m = i - (i / M) * M;
                st_dev(p.ws.act + (int64_t)(NP + m) * p.act_stride + r, cst[i]);
            }
            publish();
            if (threadIdx.x == 0) add_dev(line(set, kLineShared), (uint32_t)((qb - qa) * RTG));
        }
    }
    MOE_TRACE(3);

    // ---- B: routing barrier, top-k and compaction in every workgroup ----
    wait_geq(line(set, kLineRouteTop), (uint32_t)min(G, kRouteSubs), p.ws.hdr + kHdrStatus);
    MOE_TRACE(4);
    const int U = route_and_compact(p, tab, (LDS char*)cst, b == 0);
    MOE_TRACE(5);
    if (b == 0 && threadIdx.x == 0)
        __hip_atomic_store(p.ws.hdr + kHdrCall, call + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.route_only) return;
    const LDS uint32_t* s_mask = (const LDS uint32_t*)tab + kTabMask;
    const LDS int* s_off = tab + kTabOff;
    const LDS int* s_exp = tab + kTabExp;

    // ---- B': the shared expert's down rows of this slice (weights in LDS) -> ysh [M][nown] ----
    if (has_sh && nown > 0) {
        const int tb = min(M, p.dn_bytes / (Is * 4));  // tokens per pass through the staging area
        for (int m0 = 0; m0 < M; m0 += tb) {
            const int tc = min(tb, M - m0);
            const uint8_t* dsb = WF == MOE_FMT_MXFP4 ? p.w.sh_down_s + (int64_t)h0 * (Is / 32) : nullptr;
            down_run<WF, NJD, true>((const uint8_t*)shw, dsb, Is, nown, (const LDS float*)dnw, tc,
                                    [&]() {
                                        if (m0 == 0) wait_geq(line(set, kLineShared), (uint32_t)Is, p.ws.hdr + kHdrStatus);
                                        MOE_TRACE(6);
                                        stage_rows((LDS float*)dnw, p.ws.act + (int64_t)(NP + m0) * p.act_stride,
                                                   p.act_stride, tc, Is);
                                        __syncthreads();
                                    },
                                    [&](int row, int i, float v) { ysh[(m0 + i) * nown + row] = v; });
            __syncthreads();
        }
    }
    MOE_TRACE(7);

    // ---- start streaming this workgroup's routed down rows into LDS (as far as the window goes) ----
    const int64_t rbI = row_bytes<WF>(I);
    const int64_t dtotal = (int64_t)U * H;
    const int64_t d0 = dtotal * b / G, d1 = dtotal * (b + 1) / G;
    int pre_rows[kMaxPre];
    int pre_off[kMaxPre];
    {
        int64_t room = p.dn_bytes;
        int seg = 0;
        for (int64_t q = d0; q < d1 && seg < kMaxPre; ++seg) {
            const int u = (int)(q / H);
            const int ha = (int)(q - (int64_t)u * H);
            const int hb = (int)min<int64_t>(H, ha + (d1 - q));
            q += hb - ha;
            const int n = (int)min<int64_t>(hb - ha, room / rbI);
            pre_rows[seg] = n;
            pre_off[seg] = (int)(p.dn_bytes - room);
            if (n > 0)
                async_to_lds((char*)(dnw + pre_off[seg]), (const uint8_t*)p.w.down + ((int64_t)s_exp[u] * H + ha) * rbI,
                             (int)(n * rbI));
            room -= n * rbI;
        }
        for (; seg < kMaxPre; ++seg) pre_rows[seg] = pre_off[seg] = 0;
    }

    // ---- C: routed gate/up, an equal share of all routed tasks ----
    {
        const int TPU = I / RTG;
        const int T = U * TPU;
        const int qa = (int)((int64_t)T * b / G), qb = (int)((int64_t)T * (b + 1) / G);
        if (qb > qa) {
            const int64_t rb = row_bytes<WF>(H);
            gateup_run<AF, WF, NJ>(p, xs, cst, qa, qb, [&](int q, GUTask& t) {
                const int u = q / TPU;
                const int64_t e = uni(s_exp[u]);
                const int64_t r0 = (int64_t)(q - u * TPU) * RTG;
                t.g = (const uint8_t*)p.w.gate + (e * I + r0) * rb;
                t.u = (const uint8_t*)p.w.up + (e * I + r0) * rb;
                t.gs = WF == MOE_FMT_MXFP4 ? p.w.gate_s + (e * I + r0) * (H / 32) : nullptr;
                t.us = WF == MOE_FMT_MXFP4 ? p.w.up_s + (e * I + r0) * (H / 32) : nullptr;
                t.mask = uni(s_mask[u]);
                t.slot = (q - qa) * RTG;
            });
        }
        __syncthreads();
        MOE_TRACE(8);
        // write the staged SwiGLU rows; then count them per unit once they have landed
        if (qb > qa) {
            const int n = (qb - qa) * RTG * M;
            for (int i = threadIdx.x; i < n; i += kThreads) {
                const int s = i / M, m = i - s * M;
                const int q = qa + s / RTG;
                const int u = q / TPU;
                if (m < __popc(s_mask[u])) {
                    const int r = (q - u * TPU) * RTG + s % RTG;
                    st_dev(p.ws.act + (int64_t)(s_off[u] + m) * p.act_stride + r, cst[i]);
                }
            }
        }
        publish();
        MOE_TRACE(9);
        if (qb > qa && threadIdx.x == 0) {
            for (int u = qa / TPU; u <= (qb - 1) / TPU; ++u) {
                const int a = max(qa, u * TPU), c = min(qb, (u + 1) * TPU);
                add_dev(line(set, kLineUnit0 + u), (uint32_t)((c - a) * RTG));
            }
        }
    }

    // ---- D: routed down rows, unit by unit; partial outputs staged in LDS, written per pass ----
    MOE_TRACE(10);
    {
        LDS float* pst = cst;
        const int cap = p.cst_bytes / 4;
        int seg = 0;
        bool first = true;
        for (int64_t q = d0; q < d1; ++seg) {
            const int u = (int)(q / H);
            const int ha = (int)(q - (int64_t)u * H);
            const int hb = (int)min<int64_t>(H, ha + (d1 - q));
            q += hb - ha;
            const int t = __popc(s_mask[u]);
            const int row0 = s_off[u];
            const int64_t e = s_exp[u];
            const int npre = seg < kMaxPre ? pre_rows[seg] : 0;
            const int rows_per_pass = max(RTD, (cap / t) / RTD * RTD);
            bool staged = false;
            // rows [ha, hb) in passes that fit the partial staging area
            for (int pa = ha; pa < hb; pa += rows_per_pass) {
                const int pb = min(hb, pa + rows_per_pass);
                auto ready = [&]() {
                    if (!staged) {
                        wait_geq(line(set, kLineUnit0 + u), (uint32_t)I, p.ws.hdr + kHdrStatus);
                        if (first) MOE_TRACE(11);
                        stage_rows((LDS float*)xs, p.ws.act + (int64_t)row0 * p.act_stride, p.act_stride, t, I);
                        __syncthreads();
                        if (first) MOE_TRACE(12);
                        staged = true;
                        first = false;
                    }
                };
                auto out = [&](int row, int i, float v) { pst[(row + 0) * t + i] = v; };
                // part from the LDS window: rows [pa, min(pb, ha + npre))
                const int la = pa, lb = min(pb, ha + npre);
                if (lb > la) {
                    const uint8_t* dsb = WF == MOE_FMT_MXFP4 ? p.w.down_s + (e * H + la) * (I / 32) : nullptr;
                    down_run<WF, NJD, true>((const uint8_t*)(dnw + pre_off[seg] + (int64_t)(la - ha) * rbI), dsb, I,
                                            lb - la, (const LDS float*)xs, t, ready,
                                            [&](int row, int i, float v) { out(row + la - pa, i, v); });
                }
                const int ga = max(pa, ha + npre), gb = pb;
                if (gb > ga) {
                    const uint8_t* dsb = WF == MOE_FMT_MXFP4 ? p.w.down_s + (e * H + ga) * (I / 32) : nullptr;
                    down_run<WF, NJD, false>((const uint8_t*)p.w.down + (e * H + ga) * rbI, dsb, I, gb - ga,
                                             (const LDS float*)xs, t, ready,
                                             [&](int row, int i, float v) { out(row + ga - pa, i, v); });
                }
                __syncthreads();
                const int n = (pb - pa) * t;
                for (int i = threadIdx.x; i < n; i += kThreads) {
                    const int rr = i / t, m = i - rr * t;
                    st_dev(p.ws.part + (int64_t)(row0 + m) * H + pa + rr, pst[i]);
                }
                __syncthreads();
            }
        }
    }
    publish();
    MOE_TRACE(15);
    // count the landed partial rows for the slices they fall in
    if (threadIdx.x == 0) {
        for (int64_t q = d0; q < d1;) {
            const int u = (int)(q / H);
            const int ha = (int)(q - (int64_t)u * H);
            const int hb = (int)min<int64_t>(H, ha + (d1 - q));
            q += hb - ha;
            for (int o = slice_of(H, G, ha); o < G && slice0(H, G, o) < hb; ++o) {
                const int a = max(ha, slice0(H, G, o)), c = min(hb, slice0(H, G, o + 1));
                if (c > a) add_dev(line(set, kLineOwner0 + o), (uint32_t)(c - a));
            }
        }
    }

    // ---- E: combine this workgroup's slice of y ----
    if (nown > 0) {
        if (U > 0) wait_geq(line(set, kLineOwner0 + b), (uint32_t)(U * nown), p.ws.hdr + kHdrStatus);
        MOE_TRACE(16);
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
            if constexpr (AF == MOE_FMT_F32)
                ((float*)p.y)[(int64_t)m * H + h] = acc;
            else
                ((uint16_t*)p.y)[(int64_t)m * H + h] = f32_to_bf16_rne(acc);
        }
    }
    MOE_TRACE(17);
}

// ------------------------------------------------------------------------------------------
// launch
// ------------------------------------------------------------------------------------------

int round16(int64_t v) { return (int)((v + 15) / 16 * 16); }

template <int AF, int WF, int NJ, int NJD>
hipError_t launch_t(Params p, int num_cus, hipStream_t s) {
    auto kern = k_layer<AF, WF, NJ, NJD>;
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    const int G = std::min(num_cus, kMaxGrid);
    const int M = p.M, H = p.H;
    const int ka = std::max(p.I, p.Is);
    const int nown = (H + G - 1) / G;
    // staging area: routing scratch; shared / routed SwiGLU results of one workgroup's tasks;
    // down partials (any size works, larger means fewer passes)
    const int64_t tpu = p.I / rt_gate<WF>();
    const int64_t units = std::min<int64_t>((int64_t)p.k * M, p.E);
    const int64_t c_tasks = (units * tpu + G - 1) / G + 1;
    const int64_t s_tasks = p.Is > 0 ? (p.Is / rt_gate<WF>() + G - 1) / G + 1 : 0;
    int64_t cst = std::max<int64_t>(kSelBytes, std::max(c_tasks, s_tasks) * rt_gate<WF>() * M * 4);
    cst = std::max<int64_t>(cst, 16 * 1024);
    p.lds_tab = 0;
    p.lds_x = round16(kTabWords * 4);
    p.lds_cst = p.lds_x + round16(std::max<int64_t>((int64_t)M * H * XB, (int64_t)M * ka * 4));
    p.cst_bytes = round16(cst);
    p.lds_sh = p.lds_cst + p.cst_bytes;
    p.lds_ysh = p.lds_sh + round16(p.Is > 0 ? nown * row_bytes<WF>(p.Is) : 0);
    p.lds_dn = p.lds_ysh + round16((int64_t)M * nown * 4);
    const int budget = kLdsBytes - 1024;  // room for the static LDS variables
    if (p.route_only) {
        p.dn_bytes = 0;
    } else {
        p.dn_bytes = (budget - p.lds_dn) / 16 * 16;
        if (p.Is > 0 && p.dn_bytes < p.Is * 4) return hipErrorInvalidConfiguration;  // one shared activation row
        if (p.dn_bytes < 0) return hipErrorInvalidConfiguration;
    }
    p.lds_total = p.lds_dn + p.dn_bytes;
    if (p.lds_total > budget) return hipErrorInvalidConfiguration;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_total);
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)kern, kThreads, p.lds_total) != hipSuccess)
        return hipErrorInvalidValue;
    if (occ < 1) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3(G), dim3(kThreads), p.lds_total, s, p);
    return hipGetLastError();
}

// chunks per lane: NJ for the router and gate/up rows (K = H), NJD for the down rows (K = I, Is)
template <int AF, int WF>
hipError_t launch_shape(const Params& p, int num_cus, hipStream_t s) {
    const int nj = (p.H / Geo<WF>::EPC + Geo<WF>::LPR_G - 1) / Geo<WF>::LPR_G;
    const int ka = std::max(p.I, p.Is);
    const int njd = (ka / Geo<WF>::EPC + Geo<WF>::LPR_D - 1) / Geo<WF>::LPR_D;
    if (nj <= 1 && njd <= 1) return launch_t<AF, WF, 1, 1>(p, num_cus, s);
    if (nj <= 5 && njd <= 3) return launch_t<AF, WF, 5, 3>(p, num_cus, s);
    if (nj <= 8 && njd <= 8) return launch_t<AF, WF, 8, 8>(p, num_cus, s);
    return hipErrorInvalidConfiguration;
}

}  // namespace

#ifdef MOE_PHASE_TRACE
extern "C" int moe_trace_set(void* buf) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_moe_trace), &buf, sizeof(buf)) == hipSuccess ? 0 : -1;
}
#endif

hipError_t launch_layer(const Params& p, int num_cus, hipStream_t s) {
    if (p.act_fmt == MOE_FMT_F32) return launch_shape<MOE_FMT_F32, MOE_FMT_F32>(p, num_cus, s);
    if (p.w_fmt == MOE_FMT_BF16) return launch_shape<MOE_FMT_BF16, MOE_FMT_BF16>(p, num_cus, s);
    return launch_shape<MOE_FMT_BF16, MOE_FMT_MXFP4>(p, num_cus, s);
}

}  // namespace moe
