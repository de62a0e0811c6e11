// Routed-expert MoE decode layer for CDNA4 (gfx950), one persistent launch per call.
//
// The layer is the chain the Ling-3.0-flash decode pages describe ("Chasing the Batch-1
// Floor", section "PDL: stacking the latency floors of small kernels": router chain
// gate matvec -> top-k, MoE chain align -> up-GEMM -> activation -> down-GEMM -> combine), cut
// for a batch of at most 16 tokens on an MI355X.  Every workgroup of one grid (all resident at
// once) walks the same phases; the page's launch-ordered chain becomes counters in memory, and,
// as with its "producer-independent loads before the wait", work that needs no routing result
// runs before the routing barrier:
//
//   A  stage the token rows in LDS; start an async copy of this workgroup's share of the shared
//      expert's down rows into LDS; compute this workgroup's router rows (fp32 logits); arrive
//      at the routing barrier; compute this workgroup's share of the shared expert's gate/up
//      rows.
//   B  wait for the routing barrier; every workgroup redoes the per-token top-k and the batch
//      compaction (distinct experts ascending, token bitmask and pair rows per unit) in its own
//      LDS, so no second hand-off is needed; workgroup 0 writes the caller-visible outputs.
//   C  an equal share of all routed units' gate/up rows: each weight row is read once and
//      applied to every token of its unit, silu(g) * v in fp32; per-unit row counters.
//   D  an equal share of all units' down rows (shared expert first, from LDS), writing fp32
//      partial outputs per pair row once the unit's SwiGLU rows are complete.
//   E  per 64-row tile of y, the last workgroup to contribute sums each token's partials in slot
//      order, adds the shared expert and casts once.
//
// Data that crosses workgroups goes through device-scope (sc1) stores and loads, and a counter
// is bumped only after the stores have completed; there are no cache-wide fences.  Every wait
// is bounded: on a timeout the status word is flagged and the kernel still finishes.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

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
// every lane of each 32-lane half receives the half's sum
__device__ __forceinline__ float half_sum(float v) {
    v = row16_sum(v);
    return v + __shfl_xor(v, 16);
}
__device__ __forceinline__ float wave_sum(float v) {
    v = half_sum(v);
    return v + __shfl_xor(v, 32);
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
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    v = fmaxf(v, __shfl_xor(v, 16));
    return fmaxf(v, __shfl_xor(v, 32));
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
__device__ __forceinline__ int wave_min_bcast(int v) {
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, true));
    v = min(v, dpp_rows<0x142, 0xA>(v, v));
    v = min(v, dpp_rows<0x143, 0xC>(v, v));
    return __builtin_amdgcn_readlane(v, 63);
}
// The wave's index in the workgroup, as a scalar the compiler knows to be wave-uniform (loops on
// it stay scalar loops, which keeps the memory-wait analysis exact).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ uint64_t lanes_below() {
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ------------------------------------------------------------------------------------------
// number formats
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

// One lane's slice of a weight row: 8 consecutive K elements.
//   F32   : 32 bytes; BF16: 16 bytes; MXFP4: one dword of 8 E2M1 codes + the block's scale byte
template <int WF>
struct Raw;
template <>
struct Raw<MOE_FMT_F32> {
    f32x4 a, b;
};
template <>
struct Raw<MOE_FMT_BF16> {
    u32x4 q;
};
template <>
struct Raw<MOE_FMT_MXFP4> {
    uint32_t q;
    uint32_t s;
};

// Makes the compiler wait for a chunk's load here, in straight-line code, and treat the value as
// an ordinary register afterwards.  Without it the waits inside the branchy compute loops drain
// every outstanding load, including the next group's prefetch.
template <int WF>
__device__ __forceinline__ void settle(Raw<WF>& r) {
    if constexpr (WF == MOE_FMT_F32) {
        asm volatile("" : "+v"(r.a), "+v"(r.b));
    } else if constexpr (WF == MOE_FMT_BF16) {
        asm volatile("" : "+v"(r.q));
    } else {
        asm volatile("" : "+v"(r.q), "+v"(r.s));
    }
}

typedef __attribute__((address_space(3))) const uint8_t lds_u8;

// chunk c of a row held in LDS (weights prefetched there); the scales stay in global memory
template <int WF>
__device__ __forceinline__ void load_raw_lds(Raw<WF>& r, lds_u8* row, const uint8_t* srow, int c) {
    if constexpr (WF == MOE_FMT_F32) {
        r.a = *(__attribute__((address_space(3))) const f32x4*)(row + 32 * c);
        r.b = *(__attribute__((address_space(3))) const f32x4*)(row + 32 * c + 16);
    } else if constexpr (WF == MOE_FMT_BF16) {
        r.q = *(__attribute__((address_space(3))) const u32x4*)(row + 16 * c);
    } else {
        r.q = *(__attribute__((address_space(3))) const uint32_t*)(row + 4 * c);
        r.s = srow[c >> 2];
    }
}

// chunk c of a row (elements 8c .. 8c+7); `row` points at the row's first byte, `srow` at its scales
template <int WF>
__device__ __forceinline__ void load_raw(Raw<WF>& r, const uint8_t* row, const uint8_t* srow, int c) {
    if constexpr (WF == MOE_FMT_F32) {
        r.a = *(const f32x4*)(row + 32 * c);
        r.b = *(const f32x4*)(row + 32 * c + 16);
    } else if constexpr (WF == MOE_FMT_BF16) {
        r.q = *(const u32x4*)(row + 16 * c);
    } else {
        r.q = *(const uint32_t*)(row + 4 * c);
        r.s = srow[c >> 2];
    }
}

// Reinterprets a dword as two bf16.  Takes the dword by value: bit-casting a vector component
// lvalue directly (v.y) makes clang read the vector's first element instead.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Dot of a weight chunk with 8 bf16 activations (the row x of the gate/up GEMV), fp32 result.
template <int WF>
__device__ __forceinline__ float dot8_bf16x(const Raw<WF>& r, const u32x4& x, float acc) {
    const uint32_t x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
    if constexpr (WF == MOE_FMT_BF16) {
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(x0), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(x1), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(x2), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(x3), acc, false);
    } else if constexpr (WF == MOE_FMT_MXFP4) {
        const float sc = e8m0_to_f32(r.s);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.q, sc, 0), as_bf16x2(x0), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.q, sc, 1), as_bf16x2(x1), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.q, sc, 2), as_bf16x2(x2), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.q, sc, 3), as_bf16x2(x3), acc, false);
    }
    return acc;
}

// Dot of a weight chunk with 8 fp32 values (activations of the F32 layer, or the SwiGLU outputs
// consumed by the down GEMV).
template <int WF>
__device__ __forceinline__ float dot8_f32x(const Raw<WF>& r, const f32x4& x0, const f32x4& x1, float acc) {
    if constexpr (WF == MOE_FMT_F32) {
        acc = fmaf(r.a.x, x0.x, acc);
        acc = fmaf(r.a.y, x0.y, acc);
        acc = fmaf(r.a.z, x0.z, acc);
        acc = fmaf(r.a.w, x0.w, acc);
        acc = fmaf(r.b.x, x1.x, acc);
        acc = fmaf(r.b.y, x1.y, acc);
        acc = fmaf(r.b.z, x1.z, acc);
        acc = fmaf(r.b.w, x1.w, acc);
    } else if constexpr (WF == MOE_FMT_BF16) {
        const uint32_t w0 = r.q[0], w1 = r.q[1], w2 = r.q[2], w3 = r.q[3];
        acc = fmaf(bf16lo(w0), x0[0], acc);
        acc = fmaf(bf16hi(w0), x0[1], acc);
        acc = fmaf(bf16lo(w1), x0[2], acc);
        acc = fmaf(bf16hi(w1), x0[3], acc);
        acc = fmaf(bf16lo(w2), x1[0], acc);
        acc = fmaf(bf16hi(w2), x1[1], acc);
        acc = fmaf(bf16lo(w3), x1[2], acc);
        acc = fmaf(bf16hi(w3), x1[3], acc);
    } else {
        const float sc = e8m0_to_f32(r.s);
        const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q, sc, 0);
        const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q, sc, 1);
        const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q, sc, 2);
        const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q, sc, 3);
        acc = fmaf(p0[0], x0.x, acc);
        acc = fmaf(p0[1], x0.y, acc);
        acc = fmaf(p1[0], x0.z, acc);
        acc = fmaf(p1[1], x0.w, acc);
        acc = fmaf(p2[0], x1.x, acc);
        acc = fmaf(p2[1], x1.y, acc);
        acc = fmaf(p3[0], x1.z, acc);
        acc = fmaf(p3[1], x1.w, acc);
    }
    return acc;
}

// bytes of one row of K elements, and of its scale row
template <int WF>
__device__ __forceinline__ int64_t row_bytes(int K) {
    return WF == MOE_FMT_F32 ? 4 * (int64_t)K : (WF == MOE_FMT_BF16 ? 2 * (int64_t)K : (int64_t)K / 2);
}



// LDS tables of the batch dispatch, in words
constexpr int kTabMask = 0;                                  // [kMaxExperts + 1] token bitmask per unit
constexpr int kTabOff = kTabMask + kMaxExperts + 1;          // [kMaxExperts + 2] first pair row per unit
constexpr int kTabExp = kTabOff + kMaxExperts + 2;           // [kMaxExperts + 1] expert id per unit
constexpr int kTabPair = kTabExp + kMaxExperts + 1;          // [kMaxTokens * kMaxTopK] pair row of (m, j)
constexpr int kTabRowW = kTabPair + kMaxTokens * kMaxTopK;   // [kMaxTokens * (kMaxTopK + 1)] weight per row
constexpr int kTabMisc = kTabRowW + kMaxTokens * (kMaxTopK + 1);  // [8] U, flags
constexpr int kTabWords = (kTabMisc + 8 + 3) / 4 * 4;
// routing scratch (token masks, expert row offsets, per-token ids / weights / logits), aliased
// with the SwiGLU staging area
constexpr int kSelBytes = (2 * kMaxExperts + 3 * kMaxTokens * kMaxTopK) * 4;
constexpr int kMaxPre = 4;  // down-row segments prefetched into LDS per workgroup

constexpr int kSpinLimit = 1 << 20;

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
#endif  // ~1 s of polling; normal waits are microseconds

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

// ---- small helpers ---------------------------------------------------------------------------

// Copies n bytes (multiple of 16) from global to LDS with every thread of the workgroup.
__device__ __forceinline__ void stage16(void* dst, const void* src, int n) {
    for (int i = threadIdx.x; i < n / 16; i += kThreads) ((u32x4*)dst)[i] = ((const u32x4*)src)[i];
}

// Starts an asynchronous copy of n bytes (multiple of `unit`, 4 or 16) from global to LDS.  The
// data is usable after the issuing waves' next s_waitcnt vmcnt(0) and a workgroup barrier.
template <int UNIT>
__device__ __forceinline__ void async_to_lds(char* lds, const uint8_t* src, int n) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int chunk = 64 * UNIT;
    for (int base = wave * chunk; base < n; base += kWaves * chunk) {
        if (base + lane * UNIT < n) {
            auto* dst = (__attribute__((address_space(3))) void*)(lds + base);
            if constexpr (UNIT == 16)
                __builtin_amdgcn_global_load_lds(src + base + lane * UNIT, dst, 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds(src + base + lane * UNIT, dst, 4, 0, 0);
        }
    }
}

// fp32 logits rows are padded to whole 16-byte chunks
__host__ __device__ __forceinline__ int logit_stride(int E) { return (E + 3) / 4 * 4; }

__device__ __forceinline__ float silu_mul(float g, float v) { return g / (1.0f + __expf(-g)) * v; }

// ------------------------------------------------------------------------------------------
// routing: top-k of one token with one wave, batch compaction with one workgroup
// ------------------------------------------------------------------------------------------

// Top-k of one token's E logits with one wave.  Lane l owns experts 8l .. 8l+7, read with two
// 16-byte device-scope loads.  Order: larger logit first, equal logits -> lower expert id first.
// Every round takes the wave-wide maximum of the lanes' current maxima; among equal maxima the
// lowest lane holds the lowest id, and inside a lane the lowest index is kept, so ties resolve
// to the lower id.  The winning lane drops that logit and recomputes its maximum.  Writes ids,
// logits and softmax-over-the-k weights in order.  Every id written is in [0, E).
__device__ __forceinline__ void wave_topk(const float* lrow, int E, int k, int* out_id, float* out_w, float* out_v) {
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
__device__ __forceinline__ int route_and_compact(const Params& p, int* tab, char* sel, bool publish_outputs) {
    const int E = p.E, M = p.M, k = p.k, NP = M * k;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const bool has_sh = p.Is > 0;
    uint32_t* tokmask = (uint32_t*)sel;                 // [kMaxExperts]
    int* offe = (int*)(tokmask + kMaxExperts);          // [kMaxExperts] first pair row of an expert
    int* sid = offe + kMaxExperts;                      // [kMaxTokens * kMaxTopK]
    float* sw = (float*)(sid + kMaxTokens * kMaxTopK);  // [kMaxTokens * kMaxTopK]
    float* sv = sw + kMaxTokens * kMaxTopK;             // [kMaxTokens * kMaxTopK]
    uint32_t* s_mask = (uint32_t*)tab + kTabMask;
    int* s_off = tab + kTabOff;
    int* s_exp = tab + kTabExp;
    int* s_pair = tab + kTabPair;
    float* s_roww = (float*)(tab + kTabRowW);
    MOE_TRACE(15);

    for (int m = wave; m < M; m += kWaves)
        wave_topk(p.ws.logits + (int64_t)m * logit_stride(E), E, k, sid + m * k, sw + m * k, sv + m * k);
    __syncthreads();
    MOE_TRACE(13);
    if (wave == 0) {
        // token bitmask of every expert (one wave: its LDS operations complete in order)
        for (int e = lane; e < kMaxExperts; e += 64) tokmask[e] = 0u;
        for (int q = lane; q < NP; q += 64) atomicOr(&tokmask[sid[q]], 1u << (q / k));
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // lane l owns experts 8l .. 8l+7, so ascending ids are lane-major
        const u32x4 ta = ((const u32x4*)tokmask)[2 * lane], tb = ((const u32x4*)tokmask)[2 * lane + 1];
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

// Router rows [e0, e1): one wave per row, every token; fp32 logits by device-scope stores.
// The first row of each wave is loaded before the token rows have landed in LDS (`first` holds
// it); any further rows (grids smaller than E / 4) are loaded in the loop.
template <int AF, int NJ>
__device__ __forceinline__ void router_rows(const Params& p, const char* xs, int e0, int e1, const Raw<AF> (&first)[NJ]) {
    const int H = p.H, E = p.E, M = p.M;
    const int lane = threadIdx.x & 63, wave = wave_id();
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    const int nch = H / 8;
    for (int e = e0 + wave; e < e1; e += kWaves) {
        Raw<AF> r[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = lane + 64 * j;
            if (e == e0 + wave)
                r[j] = first[j];
            else if (c < nch)
                load_raw<AF>(r[j], (const uint8_t*)p.wr + (int64_t)e * H * XB, nullptr, c);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) settle<AF>(r[j]);
        float acc[kMaxTokens];
#pragma unroll
        for (int m = 0; m < kMaxTokens; ++m) acc[m] = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = lane + 64 * j;
            if (c < nch) {
#pragma unroll
                for (int m = 0; m < kMaxTokens; ++m) {
                    if (m < M) {
                        if constexpr (AF == MOE_FMT_F32) {
                            const f32x4* xr = (const f32x4*)(xs + (int64_t)m * H * 4) + 2 * c;
                            acc[m] = dot8_f32x<AF>(r[j], xr[0], xr[1], acc[m]);
                        } else {
                            const u32x4 xq = *((const u32x4*)(xs + (int64_t)m * H * 2) + c);
                            acc[m] = dot8_bf16x<AF>(r[j], xq, acc[m]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < kMaxTokens; ++m) {
            if (m < M) {
                const float s = wave_sum_hi(acc[m]);
                if (lane == 63) st_dev(p.ws.logits + (int64_t)m * logit_stride(E) + e, s);
            }
        }
    }
}

// Loads the R gate rows and R up rows of group g (row r0 = g * R) for this lane.  Every load is
// issued (chunks past the row end re-read its last chunk and are ignored by the compute), so the
// number of loads in flight is static and the compiler waits for exactly the group it needs.
template <int WF, int R, int NJ>
__device__ __forceinline__ void gateup_load(Raw<WF> (&wg)[R][NJ], Raw<WF> (&wu)[R][NJ], const uint8_t* gb,
                                            const uint8_t* ub, const uint8_t* gsb, const uint8_t* usb, int g,
                                            int nch, int64_t rb, int64_t sb) {
    const int lane = threadIdx.x & 63;
    const int r0 = g * R;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = min(lane + 64 * j, nch - 1);
            load_raw<WF>(wg[rr][j], gb + (int64_t)(r0 + rr) * rb, gsb + (int64_t)(r0 + rr) * sb, c);
            load_raw<WF>(wu[rr][j], ub + (int64_t)(r0 + rr) * rb, usb + (int64_t)(r0 + rr) * sb, c);
        }
    }
}

// silu(g) * v of group g for the unit's tokens, written to their pair rows.
template <int AF, int WF, int R, int NJ, int MT>
__device__ __forceinline__ void gateup_compute(const Params& p, const char* xs, const Raw<WF> (&wg)[R][NJ],
                                               const Raw<WF> (&wu)[R][NJ], int g, int nch, uint32_t mask,
                                               int row0) {
    const int H = p.H;
    const int lane = threadIdx.x & 63;
    const int r0 = g * R;
    float ag[R][MT], av[R][MT];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int t = 0; t < MT; ++t) ag[rr][t] = av[rr][t] = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int c = lane + 64 * j;
        if (c < nch) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if ((mask >> t) & 1u) {
                    if constexpr (AF == MOE_FMT_F32) {
                        const f32x4* xr = (const f32x4*)(xs + (int64_t)t * H * 4) + 2 * c;
                        const f32x4 x0 = xr[0], x1 = xr[1];
#pragma unroll
                        for (int rr = 0; rr < R; ++rr) {
                            ag[rr][t] = dot8_f32x<WF>(wg[rr][j], x0, x1, ag[rr][t]);
                            av[rr][t] = dot8_f32x<WF>(wu[rr][j], x0, x1, av[rr][t]);
                        }
                    } else {
                        const u32x4 xq = *((const u32x4*)(xs + (int64_t)t * H * 2) + c);
#pragma unroll
                        for (int rr = 0; rr < R; ++rr) {
                            ag[rr][t] = dot8_bf16x<WF>(wg[rr][j], xq, ag[rr][t]);
                            av[rr][t] = dot8_bf16x<WF>(wu[rr][j], xq, av[rr][t]);
                        }
                    }
                }
            }
        }
    }
    int i = 0;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if ((mask >> t) & 1u) {
            float* arow = p.ws.act + (int64_t)(row0 + i) * p.act_stride + r0;
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const float gs = wave_sum_hi(ag[rr][t]);
                const float vs = wave_sum_hi(av[rr][t]);
                if (lane == 48 + rr) st_dev(arow + rr, silu_mul(gs, vs));
            }
            ++i;
        }
    }
}

// Gate/up rows of one unit: groups [g0, g1) of R consecutive rows counted from row 0 of the
// weight matrices gb/ub (scales gsb/usb for MXFP4).  Tokens = set bits of `mask`; the i-th of
// them owns pair row row0 + i.  Each wave keeps the next group's loads in flight while it
// computes the current one.
template <int AF, int WF, int R, int NJ, int MT>
__device__ __forceinline__ void gateup_rows(const Params& p, const char* xs, const uint8_t* gb, const uint8_t* ub,
                            const uint8_t* gsb, const uint8_t* usb, int g0, int g1, uint32_t mask, int row0) {
    const int wave = wave_id();
    const int nch = p.H / 8;
    const int64_t rb = row_bytes<WF>(p.H);
    const int64_t sb = p.H / 32;
    Raw<WF> ga[R][NJ], ua[R][NJ], gb2[R][NJ], ub2[R][NJ];
    int g = g0 + wave;  // callers pass g1 > g0
    gateup_load<WF, R, NJ>(ga, ua, gb, ub, gsb, usb, min(g, g1 - 1), nch, rb, sb);
    auto settle_all = [](Raw<WF>(&a)[R][NJ], Raw<WF>(&b)[R][NJ]) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                settle<WF>(a[rr][j]);
                settle<WF>(b[rr][j]);
            }
    };
    // the prefetch is unconditional (the last group re-reads itself) so the waits stay exact
    while (g < g1) {
        gateup_load<WF, R, NJ>(gb2, ub2, gb, ub, gsb, usb, min(g + kWaves, g1 - 1), nch, rb, sb);
        settle_all(ga, ua);
        gateup_compute<AF, WF, R, NJ, MT>(p, xs, ga, ua, g, nch, mask, row0);
        g += kWaves;
        if (g >= g1) break;
        gateup_load<WF, R, NJ>(ga, ua, gb, ub, gsb, usb, min(g + kWaves, g1 - 1), nch, rb, sb);
        settle_all(gb2, ub2);
        gateup_compute<AF, WF, R, NJ, MT>(p, xs, gb2, ub2, g, nch, mask, row0);
        g += kWaves;
    }
}

// Loads the RD down rows starting at h (rows counted from h0 = row 0 of db/dsb); FROM_LDS: db is an
// LDS address.
template <int WF, int RD, int NJD, bool FROM_LDS>
__device__ __forceinline__ void down_load(Raw<WF> (&wd)[RD][NJD], const uint8_t* db, const uint8_t* dsb, int h,
                                          int h0, int h1, int nch, int64_t rb, int64_t sb) {
    const int hl = threadIdx.x & 31;
#pragma unroll
    for (int rr = 0; rr < RD; ++rr) {
#pragma unroll
        for (int j = 0; j < NJD; ++j) {
            const int c = hl + 32 * j;
            if constexpr (FROM_LDS) {
                if (c < nch && h + rr < h1)
                    load_raw_lds<WF>(wd[rr][j], (lds_u8*)db + (h - h0 + rr) * rb, dsb + (int64_t)(h - h0 + rr) * sb, c);
            } else {  // unconditional (clamped) so the number of loads in flight is static
                const int hr = min(h + rr, h1 - 1) - h0;
                load_raw<WF>(wd[rr][j], db + (int64_t)hr * rb, dsb + (int64_t)hr * sb, min(c, nch - 1));
            }
        }
    }
}

template <int WF, int RD, int NJD, int MT>
__device__ __forceinline__ void down_compute(const Params& p, const Raw<WF> (&wd)[RD][NJD], int h, int h1, int K,
                                             int nch, const float* acts, int tcount, int row0) {
    const int H = p.H;
    const int hl = threadIdx.x & 31;
    float acc[RD][MT];
#pragma unroll
    for (int rr = 0; rr < RD; ++rr)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[rr][t] = 0.0f;
#pragma unroll
    for (int j = 0; j < NJD; ++j) {
        const int c = hl + 32 * j;
        if (c < nch) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < tcount) {
                    const f32x4* ar = (const f32x4*)(acts + t * K) + 2 * c;
                    const f32x4 a0 = ar[0], a1 = ar[1];
#pragma unroll
                    for (int rr = 0; rr < RD; ++rr)
                        if (h + rr < h1) acc[rr][t] = dot8_f32x<WF>(wd[rr][j], a0, a1, acc[rr][t]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t < tcount) {
#pragma unroll
            for (int rr = 0; rr < RD; ++rr) {
                const float s = half_sum_hi(acc[rr][t]);
                if (hl == 16 + rr && h + rr < h1) st_dev(p.ws.part + (int64_t)(row0 + t) * H + h + rr, s);
            }
        }
    }
}

// Down rows [h0, h1) of one unit with K inputs: a half-wave owns RD rows at a time, lane l of
// the half covers elements 8c..8c+7 for c = l + 32 j.  `db`/`dsb` point at row h0 of the weights
// (global or LDS).  `ready()` is called by the whole workgroup after the first loads are issued
// and before any compute: it waits for the unit's SwiGLU rows and stages them at `acts`
// ([tcount][K] fp32 in LDS).  Partial outputs go to pair rows row0 + t.
template <int WF, int RD, int NJD, int MT, bool FROM_LDS, typename Ready>
__device__ __forceinline__ void down_rows(const Params& p, const uint8_t* db, const uint8_t* dsb, int K, int h0, int h1,
                                          const float* acts, int tcount, int row0, Ready ready) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int hsel = (lane >> 5) * RD;  // the upper half-wave takes the wave's second RD rows
    constexpr int WSTEP = kWaves * 2 * RD;
    const int nch = K / 8;
    const int64_t rb = row_bytes<WF>(K);
    const int64_t sb = K / 32;
    Raw<WF> wa[RD][NJD], wb[RD][NJD];
    int hw = h0 + wave * 2 * RD;  // wave-uniform; the loop is a scalar loop
    down_load<WF, RD, NJD, FROM_LDS>(wa, db, dsb, min(hw + hsel, h1 - 1), h0, h1, nch, rb, sb);
    ready();
    auto settle_all = [](Raw<WF>(&a)[RD][NJD]) {
#pragma unroll
        for (int rr = 0; rr < RD; ++rr)
#pragma unroll
            for (int j = 0; j < NJD; ++j) settle<WF>(a[rr][j]);
    };
    while (hw < h1) {
        down_load<WF, RD, NJD, FROM_LDS>(wb, db, dsb, min(hw + WSTEP + hsel, h1 - 1), h0, h1, nch, rb, sb);
        settle_all(wa);
        down_compute<WF, RD, NJD, MT>(p, wa, hw + hsel, h1, K, nch, acts, tcount, row0);
        hw += WSTEP;
        if (hw >= h1) break;
        down_load<WF, RD, NJD, FROM_LDS>(wa, db, dsb, min(hw + WSTEP + hsel, h1 - 1), h0, h1, nch, rb, sb);
        settle_all(wb);
        down_compute<WF, RD, NJD, MT>(p, wb, hw + hsel, h1, K, nch, acts, tcount, row0);
        hw += WSTEP;
    }
}

// Stages `tcount` SwiGLU rows (K floats each, starting at pair row row0) into LDS with batched
// 16-byte device-scope loads.
__device__ __forceinline__ void stage_acts(const Params& p, float* acts, int row0, int tcount, int K) {
    const float* base = p.ws.act + (int64_t)row0 * p.act_stride;
    const __amdgpu_buffer_rsrc_t r = dev_rsrc(base, (uint32_t)(tcount * p.act_stride * 4));
    const int q4 = K / 4, n = tcount * q4;
    for (int i0 = threadIdx.x; i0 < n; i0 += 8 * kThreads) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n) {
                const int t = i / q4, c4 = i - t * q4;
                v[u] = ld_dev16(r, (uint32_t)((t * p.act_stride + 4 * c4) * 4));
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n) ((f32x4*)acts)[i] = v[u];
        }
    }
}

// ------------------------------------------------------------------------------------------
// the layer kernel
// ------------------------------------------------------------------------------------------

template <int AF, int WF, int MT, int NJ, int NJD>
__global__ __launch_bounds__(kThreads) void k_layer(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int G = gridDim.x, b = blockIdx.x;
    const int H = p.H, E = p.E, M = p.M, k = p.k, I = p.I, Is = p.Is;
    const int NP = M * k;
    const bool has_sh = Is > 0;
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    constexpr int R = WF == MOE_FMT_MXFP4 ? 2 : 1;  // gate/up rows per wave task
    constexpr int RD = 2;                           // down rows per half-wave task
    int* tab = (int*)smem;
    char* xs = smem + p.lds_x;
    char* shw = smem + p.lds_sh;
    float* acts = (float*)(smem + p.lds_act);
    char* dnw = smem + p.lds_dn;
    __shared__ uint32_t s_call;
    MOE_TRACE(0);

    // ---- A: call index, token rows, router rows, shared-expert down prefetch ----
    if (threadIdx.x == 0) s_call = ld_dev(p.ws.hdr + kHdrCall);
    async_to_lds<16>(xs, (const uint8_t*)p.x, M * H * XB);
    const int e0 = (int)((int64_t)E * b / G), e1 = (int)((int64_t)E * (b + 1) / G);
    Raw<AF> rfirst[NJ];
    {
        const int e = e0 + wave_id(), lane = threadIdx.x & 63;
        if (e < e1) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                if (lane + 64 * j < H / 8) load_raw<AF>(rfirst[j], (const uint8_t*)p.wr + (int64_t)e * H * XB, nullptr, lane + 64 * j);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // token rows in LDS
    __syncthreads();
    MOE_TRACE(1);
    const uint32_t call = s_call;
    uint32_t* set = p.ws.ctr + (int64_t)(call & 1u) * kSetWords;
    if (b == 0) {
        uint32_t* nxt = p.ws.ctr + (int64_t)((call + 1u) & 1u) * kSetWords;
        for (int l = threadIdx.x; l < kSetLines; l += kThreads) line(nxt, l)[0] = 0u;
    }
    router_rows<AF, NJ>(p, xs, e0, e1, rfirst);
    publish();
    if (threadIdx.x == 0) {
        const int s = b % kRouteSubs;
        const uint32_t members = G / kRouteSubs + (s < G % kRouteSubs ? 1 : 0);
        if (add_dev(line(set, s), 1u) + 1u == members) add_dev(line(set, kLineRouteTop), 1u);
    }
    MOE_TRACE(2);
    if (p.route_only && b != 0) return;
    const int sh0 = (int)((int64_t)H * b / G), sh1 = (int)((int64_t)H * (b + 1) / G);
    const int64_t rb_sh = row_bytes<WF>(Is);
    if (has_sh && !p.route_only && sh1 > sh0)  // rows are 16-byte multiples in every format
        async_to_lds<16>(shw, (const uint8_t*)p.w.sh_down + sh0 * rb_sh, (int)((sh1 - sh0) * rb_sh));

    // ---- A': shared expert gate/up (needs no routing); published after routing ----
    int sh_rows_done = 0;
    if (has_sh && !p.route_only) {
        const int gS = Is / R;
        const int g0 = (int)((int64_t)gS * b / G), g1 = (int)((int64_t)gS * (b + 1) / G);
        if (g1 > g0) {
            const uint8_t* gsb = nullptr;
            const uint8_t* usb = nullptr;
            if constexpr (WF == MOE_FMT_MXFP4) {
                gsb = p.w.sh_gate_s;
                usb = p.w.sh_up_s;
            }
            gateup_rows<AF, WF, R, NJ, MT>(p, xs, (const uint8_t*)p.w.sh_gate, (const uint8_t*)p.w.sh_up, gsb, usb,
                                           g0, g1, (1u << M) - 1u, NP);
            sh_rows_done = (g1 - g0) * R;
        }
    }

    // ---- B: routing barrier, top-k and compaction in every workgroup ----
    MOE_TRACE(3);
    wait_geq(line(set, kLineRouteTop), (uint32_t)min(G, kRouteSubs), p.ws.hdr + kHdrStatus);
    MOE_TRACE(4);
    const int U = route_and_compact(p, tab, (char*)acts, b == 0);
    MOE_TRACE(5);
    if (b == 0 && threadIdx.x == 0)
        __hip_atomic_store(p.ws.hdr + kHdrCall, call + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.route_only) return;
    if (sh_rows_done) {  // the shared rows' stores completed long ago; this wait is short
        publish();
        if (threadIdx.x == 0) add_dev(line(set, kLineShared), (uint32_t)sh_rows_done);
    }
    const uint32_t* s_mask = (const uint32_t*)tab + kTabMask;
    const int* s_off = tab + kTabOff;
    const int* s_exp = tab + kTabExp;

    // ---- start streaming this workgroup's routed down rows into LDS (as far as the window goes) ----
    const int64_t rbI = row_bytes<WF>(I);
    const int64_t dtotal = (int64_t)U * H;
    const int64_t d0 = dtotal * b / G, d1 = dtotal * (b + 1) / G;
    int pre_rows[kMaxPre];
    int pre_off[kMaxPre];
    {
        int64_t room = p.lds_dn_bytes;
        int seg = 0;
        for (int64_t q = d0; q < d1; ++seg) {
            const int u = (int)(q / H);
            const int ha = (int)(q - (int64_t)u * H);
            const int hb = (int)min<int64_t>(H, ha + (d1 - q));
            q += hb - ha;
            if (seg >= kMaxPre) break;
            const int n = (int)min<int64_t>(hb - ha, room / rbI);
            pre_rows[seg] = n;
            pre_off[seg] = (int)(p.lds_dn_bytes - room);
            if (n > 0)
                async_to_lds<16>(dnw + pre_off[seg], (const uint8_t*)p.w.down + ((int64_t)s_exp[u] * H + ha) * rbI,
                                 (int)(n * rbI));
            room -= n * rbI;
        }
        for (; seg < kMaxPre; ++seg) pre_rows[seg] = pre_off[seg] = 0;
    }

    // ---- C: routed gate/up, an equal share of all routed rows ----
    {
        const int gI = I / R;
        const int64_t total = (int64_t)U * gI;
        const int64_t q0 = total * b / G, q1 = total * (b + 1) / G;
        const int64_t rb = row_bytes<WF>(H);
        for (int64_t q = q0; q < q1;) {
            const int u = (int)(q / gI);
            const int ga = (int)(q - (int64_t)u * gI);
            const int gb_ = (int)min<int64_t>(gI, ga + (q1 - q));
            q += gb_ - ga;
            const int64_t e = s_exp[u];
            const uint8_t* gsb = nullptr;
            const uint8_t* usb = nullptr;
            if constexpr (WF == MOE_FMT_MXFP4) {
                gsb = p.w.gate_s + e * I * (H / 32);
                usb = p.w.up_s + e * I * (H / 32);
            }
            gateup_rows<AF, WF, R, NJ, MT>(p, xs, (const uint8_t*)p.w.gate + e * I * rb,
                                           (const uint8_t*)p.w.up + e * I * rb, gsb, usb, ga, gb_, s_mask[u],
                                           s_off[u]);
            publish();
            if (threadIdx.x == 0) add_dev(line(set, kLineUnit0 + u), (uint32_t)(gb_ - ga) * R);
        }
    }

    // ---- D: down rows; the shared expert's share first (weights already in LDS) ----
    MOE_TRACE(6);
    __builtin_amdgcn_s_waitcnt(0);  // every async copy into LDS has landed
    __syncthreads();
    if (has_sh && sh1 > sh0) {
        const uint8_t* dsb = nullptr;  // MXFP4 scales are read from global memory
        if constexpr (WF == MOE_FMT_MXFP4) dsb = p.w.sh_down_s + (int64_t)sh0 * (Is / 32);
        down_rows<WF, RD, NJD, MT, true>(p, (const uint8_t*)shw, dsb, Is, sh0, sh1, acts, M, NP, [&]() {
            wait_geq(line(set, kLineShared), (uint32_t)Is, p.ws.hdr + kHdrStatus);
            MOE_TRACE(7);
            stage_acts(p, acts, NP, M, Is);
            __syncthreads();
            MOE_TRACE(16);
        });
        __syncthreads();
    }
    MOE_TRACE(8);
    bool first_wait = true;
    {
        int seg = 0;
        for (int64_t q = d0; q < d1; ++seg) {
            const int u = (int)(q / H);
            const int ha = (int)(q - (int64_t)u * H);
            const int hb = (int)min<int64_t>(H, ha + (d1 - q));
            q += hb - ha;
            const uint32_t mask = s_mask[u];
            const int tcount = __popc(mask);
            const int64_t e = s_exp[u];
            const int npre = seg < kMaxPre ? pre_rows[seg] : 0;
            auto ready = [&]() {
                wait_geq(line(set, kLineUnit0 + u), (uint32_t)I, p.ws.hdr + kHdrStatus);
                if (first_wait) MOE_TRACE(9);
                else MOE_TRACE(20);
                stage_acts(p, acts, s_off[u], tcount, I);
                __syncthreads();
                if (first_wait) MOE_TRACE(17);
                first_wait = false;
            };
            if (npre > 0) {  // rows [ha, ha + npre) from the LDS window
                const uint8_t* dsb = nullptr;
                if constexpr (WF == MOE_FMT_MXFP4) dsb = p.w.down_s + (e * H + ha) * (I / 32);
                down_rows<WF, RD, NJD, MT, true>(p, (const uint8_t*)(dnw + pre_off[seg]), dsb, I, ha, ha + npre, acts,
                                           tcount, s_off[u], ready);
                if (seg == 0) MOE_TRACE(18);
            }
            if (ha + npre < hb) {  // the rest straight from global memory
                const uint8_t* dsb = nullptr;
                if constexpr (WF == MOE_FMT_MXFP4) dsb = p.w.down_s + (e * H + ha + npre) * (I / 32);
                const uint8_t* db = (const uint8_t*)p.w.down + (e * H + ha + npre) * rbI;
                if (npre > 0)
                    down_rows<WF, RD, NJD, MT, false>(p, db, dsb, I, ha + npre, hb, acts, tcount, s_off[u], []() {});
                else
                    down_rows<WF, RD, NJD, MT, false>(p, db, dsb, I, ha + npre, hb, acts, tcount, s_off[u], ready);
                if (seg == 0) MOE_TRACE(19);
            }
            __syncthreads();
        }
    }
    MOE_TRACE(21);
    publish();
    MOE_TRACE(10);

    // ---- E: finished rows per y tile; the last contributor of a tile combines it ----
    __shared__ int s_done[kMaxTiles];
    __shared__ int s_ndone;
    if (threadIdx.x == 0) s_ndone = 0;
    __syncthreads();
    const int ntiles = (H + kCombineTile - 1) / kCombineTile;
    const int nunits = U + (has_sh ? 1 : 0);
    for (int tile = threadIdx.x; tile < ntiles; tile += kThreads) {
        const int ta = tile * kCombineTile, tb = min(H, ta + kCombineTile);
        int64_t mine = 0;
        if (has_sh) mine += max(0, min(sh1, tb) - max(sh0, ta));
        for (int64_t u = d0 / H; d1 > d0 && u <= (d1 - 1) / H; ++u) {
            const int64_t a = max(d0, u * H + ta), c = min(d1, u * H + tb);
            if (c > a) mine += c - a;
        }
        if (mine > 0) {
            const uint32_t need = (uint32_t)nunits * (uint32_t)(tb - ta);
            if (add_dev(line(set, kLineTile0 + tile), (uint32_t)mine) + (uint32_t)mine == need)
                s_done[atomicAdd(&s_ndone, 1)] = tile;
        }
    }
    __syncthreads();
    MOE_TRACE(11);
    const int nd = s_ndone;
    const int* s_pair = tab + kTabPair;
    const float* s_roww = (const float*)(tab + kTabRowW);
    const __amdgpu_buffer_rsrc_t prs = dev_rsrc(p.ws.part, (uint32_t)((NP + M) * H * 4));
    for (int d = 0; d < nd; ++d) {
        const int tile = s_done[d];
        const int ta = tile * kCombineTile, tb = min(H, ta + kCombineTile);
        const int nq = (tb - ta) / 4;  // H is a multiple of 8
        for (int i = threadIdx.x; i < M * nq; i += kThreads) {
            const int m = i / nq, h = ta + 4 * (i - m * nq);
            f32x4 v[kMaxTopK + 1];
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                if (j < k) v[j] = ld_dev16(prs, (uint32_t)(((int64_t)s_pair[m * k + j] * H + h) * 4));
            if (has_sh) v[kMaxTopK] = ld_dev16(prs, (uint32_t)(((int64_t)(NP + m) * H + h) * 4));
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                if (j < k) {
                    const float wj = s_roww[s_pair[m * k + j]];
                    acc[0] = fmaf(wj, v[j][0], acc[0]);
                    acc[1] = fmaf(wj, v[j][1], acc[1]);
                    acc[2] = fmaf(wj, v[j][2], acc[2]);
                    acc[3] = fmaf(wj, v[j][3], acc[3]);
                }
            }
            if (has_sh) {
                acc[0] += v[kMaxTopK][0];
                acc[1] += v[kMaxTopK][1];
                acc[2] += v[kMaxTopK][2];
                acc[3] += v[kMaxTopK][3];
            }
            if constexpr (AF == MOE_FMT_F32) {
                *(f32x4*)((float*)p.y + (int64_t)m * H + h) = acc;
            } else {
                const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
                *(uint2*)((uint16_t*)p.y + (int64_t)m * H + h) = make_uint2(lo, hi);
            }
        }
    }
    MOE_TRACE(12);
}

// ------------------------------------------------------------------------------------------
// launch
// ------------------------------------------------------------------------------------------

constexpr int kLdsPerCu = 160 * 1024;

int round16(int64_t v) { return (int)((v + 15) / 16 * 16); }

template <int AF, int WF, int MT, int NJ, int NJD>
hipError_t launch_t(Params p, int num_cus, hipStream_t s) {
    auto kern = k_layer<AF, WF, MT, NJ, NJD>;
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    const int ka = p.I > p.Is ? p.I : p.Is;
    // grid: up to two workgroups per CU, all resident (the phases wait on each other)
    int grid = 0;
    for (int per_cu = 2; per_cu >= 1 && grid == 0; --per_cu) {
        const int g = per_cu * num_cus;
        const int sh_rows = (p.H + g - 1) / g;
        int64_t shb = 0;
        if (p.Is > 0) {
            const int64_t rb = WF == MOE_FMT_F32 ? 4LL * p.Is : (WF == MOE_FMT_BF16 ? 2LL * p.Is : p.Is / 2);
            shb = sh_rows * rb;
        }
        p.lds_x = kTabWords * 4;
        p.lds_sh = p.lds_x + round16((int64_t)p.M * p.H * XB);
        p.lds_act = p.lds_sh + round16(shb);
        const int64_t act_bytes = (int64_t)(p.route_only ? 0 : MT * ka * 4);
        p.lds_dn = p.lds_act + round16(act_bytes > kSelBytes ? act_bytes : kSelBytes);
        p.sh_rows = sh_rows;
        const int budget = kLdsPerCu / per_cu - 2048;  // room for the static LDS variables
        if (p.lds_dn > budget) continue;
        // the routed down-row window takes what is left, up to this workgroup's share
        const int64_t rbI = WF == MOE_FMT_F32 ? 4LL * p.I : (WF == MOE_FMT_BF16 ? 2LL * p.I : p.I / 2);
        const int64_t share = ((int64_t)p.k * p.M < p.E ? (int64_t)p.k * p.M : p.E) * p.H / g + 2;
        int64_t dn = p.route_only ? 0 : std::min<int64_t>(budget - p.lds_dn, share * rbI);
        dn = dn / 16 * 16;
        p.lds_dn_bytes = (int)dn;
        p.lds_total = p.lds_dn + (int)dn;
        int occ = 0;
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_total);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)kern, kThreads, p.lds_total) != hipSuccess)
            return hipErrorInvalidValue;
        if (occ >= per_cu) grid = g;
    }
    if (grid == 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), p.lds_total, s, p);
    return hipGetLastError();
}

template <int AF, int WF, int MT>
hipError_t launch_shape(const Params& p, int num_cus, hipStream_t s) {
    const int nj = (p.H / 8 + 63) / 64;
    const int ka = p.I > p.Is ? p.I : p.Is;
    const int njd = (ka / 8 + 31) / 32;
    if (nj <= 1 && njd <= 1) return launch_t<AF, WF, MT, 1, 1>(p, num_cus, s);
    if (nj <= 5 && njd <= 3) return launch_t<AF, WF, MT, 5, 3>(p, num_cus, s);
    return launch_t<AF, WF, MT, 8, 8>(p, num_cus, s);
}

}  // namespace

#ifdef MOE_PHASE_TRACE
extern "C" int moe_trace_set(void* buf) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_moe_trace), &buf, sizeof(buf)) == hipSuccess ? 0 : -1;
}
#endif

hipError_t launch_layer(const Params& p, int num_cus, hipStream_t s) {
    if (p.act_fmt == MOE_FMT_F32) return launch_shape<MOE_FMT_F32, MOE_FMT_F32, kMaxTokens>(p, num_cus, s);
    if (p.w_fmt == MOE_FMT_BF16) {
        if (p.M == 1) return launch_shape<MOE_FMT_BF16, MOE_FMT_BF16, 1>(p, num_cus, s);
        return launch_shape<MOE_FMT_BF16, MOE_FMT_BF16, kMaxTokens>(p, num_cus, s);
    }
    if (p.M == 1) return launch_shape<MOE_FMT_BF16, MOE_FMT_MXFP4, 1>(p, num_cus, s);
    return launch_shape<MOE_FMT_BF16, MOE_FMT_MXFP4, kMaxTokens>(p, num_cus, s);
}

}  // namespace moe
