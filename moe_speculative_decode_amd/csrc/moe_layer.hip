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
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    v = fmaxf(v, __shfl_xor(v, 16));
    return fmaxf(v, __shfl_xor(v, 32));
}
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
// top-k / compaction scratch, aliased with the SwiGLU staging area
constexpr int kSelBytes = kWaves * kMaxExperts * 8 + 2 * kMaxExperts * 4 + kWaves * 4 +
                          3 * kMaxTokens * kMaxTopK * 4;

constexpr int kSpinLimit = 1 << 20;  // ~1 s of polling; normal waits are microseconds

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
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

__device__ __forceinline__ float silu_mul(float g, float v) { return g / (1.0f + __expf(-g)) * v; }

// ------------------------------------------------------------------------------------------
// routing: top-k of one token with one wave, batch compaction with one workgroup
// ------------------------------------------------------------------------------------------

// Top-k of one token's E logits (device-scope loads).  Ties go to the lower expert id.  Writes
// ids and weights (softmax over the k selected logits) in descending order.  `cv`/`ci` are
// per-wave LDS scratch of kMaxExperts entries.  Every id written is in [0, E).
__device__ void wave_topk(const float* lrow, int E, int k, float* cv, int* ci, int* out_id, float* out_w,
                          float* out_v) {
    const int lane = threadIdx.x & 63;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? ld_dev(lrow + e) : -INFINITY;
    }
    if (lane < k) {
        out_id[lane] = lane;  // placeholder ids (distinct, in range) for inputs with NaNs
        out_v[lane] = -INFINITY;
    }
    // tau = the k-th largest of the 64 lane maxima; at least k logits are >= tau
    float lm = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) lm = fmaxf(lm, v[i]);
    float cur = lm, tau = -INFINITY;
    for (int r = 0; r < k; ++r) {
        const float mx = wave_max(cur);
        const uint64_t b = __ballot(cur == mx);
        if (b && lane == __ffsll((unsigned long long)b) - 1) cur = -INFINITY;
        tau = mx;
    }
    // compact the candidates (logits >= tau) into LDS in lane order
    bool cand[8];
    int c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        cand[i] = v[i] >= tau && lane + 64 * i < E;
        c += cand[i] ? 1 : 0;
    }
    int pre = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 4; ++bit) {
        const uint64_t b = __ballot((c >> bit) & 1);
        pre += __popcll(b & lanes_below()) << bit;
        total += __popcll(b) << bit;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (cand[i]) {
            cv[pre] = v[i];
            ci[pre] = lane + 64 * i;
            ++pre;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // exact rank of each candidate: (value desc, id asc)
    for (int base = 0; base < total; base += 64) {
        const int i = base + lane;
        if (i < total) {
            const float vi = cv[i];
            const int ii = ci[i];
            int rank = 0;
            for (int j = 0; j < total; ++j) {
                const float vj = cv[j];
                const int ij = ci[j];
                rank += (vj > vi || (vj == vi && ij < ii)) ? 1 : 0;
            }
            if (rank < k) {
                out_v[rank] = vi;
                out_id[rank] = ii;
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const float vmax = out_v[0];
    const float ex = lane < k ? __expf(out_v[lane] - vmax) : 0.0f;
    const float z = wave_sum(ex);
    if (lane < k) out_w[lane] = ex / z;
}

// Exclusive scan over n <= 2 * kThreads uint32 values in LDS (in place); returns the total.
__device__ uint32_t block_exclusive_scan(uint32_t* a, int n, uint32_t* wave_tot) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint32_t v0 = 2 * t < n ? a[2 * t] : 0u;
    const uint32_t v1 = 2 * t + 1 < n ? a[2 * t + 1] : 0u;
    uint32_t s = v0 + v1, incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t base = 0, total = 0;
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) base += wave_tot[w];
        total += wave_tot[w];
    }
    const uint32_t ex = base + incl - s;
    __syncthreads();
    if (2 * t < n) a[2 * t] = ex;
    if (2 * t + 1 < n) a[2 * t + 1] = ex + v0;
    __syncthreads();
    return total;
}

// Top-k of all M tokens and the batch compaction into this workgroup's LDS tables.  Workgroup 0
// (`publish_outputs`) also writes the caller-visible routing outputs.  Returns U.
__device__ int route_and_compact(const Params& p, int* tab, char* sel, bool publish_outputs) {
    const int E = p.E, M = p.M, k = p.k, NP = M * k;
    const int wave = threadIdx.x >> 6;
    const bool has_sh = p.Is > 0;
    float* cand_v = (float*)sel;                                  // [kWaves][kMaxExperts]
    int* cand_i = (int*)(cand_v + kWaves * kMaxExperts);          // [kWaves][kMaxExperts]
    uint32_t* tokmask = (uint32_t*)(cand_i + kWaves * kMaxExperts);  // [kMaxExperts]
    uint32_t* scan = tokmask + kMaxExperts;                       // [kMaxExperts]
    uint32_t* wtot = scan + kMaxExperts;                          // [kWaves]
    int* sid = (int*)(wtot + kWaves);                             // [kMaxTokens * kMaxTopK]
    float* sw = (float*)(sid + kMaxTokens * kMaxTopK);
    float* sv = sw + kMaxTokens * kMaxTopK;
    uint32_t* s_mask = (uint32_t*)tab + kTabMask;
    int* s_off = tab + kTabOff;
    int* s_exp = tab + kTabExp;
    int* s_pair = tab + kTabPair;
    float* s_roww = (float*)(tab + kTabRowW);

    for (int m = wave; m < M; m += kWaves)
        wave_topk(p.ws.logits + (int64_t)m * E, E, k, cand_v + wave * kMaxExperts, cand_i + wave * kMaxExperts,
                  sid + m * k, sw + m * k, sv + m * k);
    for (int i = threadIdx.x; i < E; i += kThreads) tokmask[i] = 0u;
    __syncthreads();
    for (int q = threadIdx.x; q < NP; q += kThreads) {
        sid[q] = min(max(sid[q], 0), E - 1);  // ids are in range by construction; keep it provable
        atomicOr(&tokmask[sid[q]], 1u << (q / k));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += kThreads) {
        const uint32_t tm = tokmask[i];
        scan[i] = tm ? ((1u << 16) | (uint32_t)__popc(tm)) : 0u;
    }
    __syncthreads();
    const uint32_t tot = block_exclusive_scan(scan, E, wtot);
    const int U = (int)(tot >> 16);
    for (int i = threadIdx.x; i < E; i += kThreads) {
        const uint32_t tm = tokmask[i];
        if (tm) {
            const int u = (int)(scan[i] >> 16);
            s_mask[u] = tm;
            s_off[u] = (int)(scan[i] & 0xFFFFu);
            s_exp[u] = i;
        }
    }
    if (threadIdx.x == 0) {
        s_mask[U] = has_sh ? ((1u << M) - 1u) : 0u;
        s_off[U] = NP;
        s_off[U + 1] = NP + (has_sh ? M : 0);
        s_exp[U] = E;
        tab[kTabMisc] = U;
    }
    for (int q = threadIdx.x; q < NP; q += kThreads) {
        const int m = q / k, ex = sid[q];
        const int row = (int)(scan[ex] & 0xFFFFu) + __popc(tokmask[ex] & ((1u << m) - 1u));
        s_pair[q] = row;
        s_roww[row] = sw[q];
    }
    for (int m = threadIdx.x; m < M; m += kThreads) s_roww[NP + m] = 1.0f;
    __syncthreads();

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
template <int AF>
__device__ void router_rows(const Params& p, const char* xs, int e0, int e1) {
    const int H = p.H, E = p.E, M = p.M;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    const int nch = H / 8;
    for (int e = e0 + wave; e < e1; e += kWaves) {
        const uint8_t* row = (const uint8_t*)p.wr + (int64_t)e * H * XB;
        float acc[kMaxTokens];
#pragma unroll
        for (int m = 0; m < kMaxTokens; ++m) acc[m] = 0.0f;
        for (int c = lane; c < nch; c += 64) {
            Raw<AF> r;
            load_raw<AF>(r, row, nullptr, c);
#pragma unroll
            for (int m = 0; m < kMaxTokens; ++m) {
                if (m < M) {
                    if constexpr (AF == MOE_FMT_F32) {
                        const f32x4* xr = (const f32x4*)(xs + (int64_t)m * H * 4) + 2 * c;
                        acc[m] = dot8_f32x<AF>(r, xr[0], xr[1], acc[m]);
                    } else {
                        const u32x4 xq = *((const u32x4*)(xs + (int64_t)m * H * 2) + c);
                        acc[m] = dot8_bf16x<AF>(r, xq, acc[m]);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < kMaxTokens; ++m) {
            if (m < M) {
                const float s = wave_sum(acc[m]);
                if (lane == 0) st_dev(p.ws.logits + (int64_t)m * E + e, s);
            }
        }
    }
}

// Gate/up rows of one unit: groups [g0, g1) of R consecutive rows starting at row 0 of the
// weight matrices gb/ub (scales gsb/usb for MXFP4).  Tokens = set bits of `mask`; the i-th of
// them owns pair row row0 + i of the SwiGLU buffer.
template <int AF, int WF, int R, int NJ, int MT>
__device__ void gateup_rows(const Params& p, const char* xs, const uint8_t* gb, const uint8_t* ub,
                            const uint8_t* gsb, const uint8_t* usb, int g0, int g1, uint32_t mask, int row0) {
    const int H = p.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nch = H / 8;
    const int64_t rb = row_bytes<WF>(H);
    const int64_t sb = H / 32;
    for (int g = g0 + wave; g < g1; g += kWaves) {
        const int r0 = g * R;
        Raw<WF> wg[R][NJ], wu[R][NJ];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c = lane + 64 * j;
                if (c < nch) {
                    load_raw<WF>(wg[rr][j], gb + (int64_t)(r0 + rr) * rb, gsb + (int64_t)(r0 + rr) * sb, c);
                    load_raw<WF>(wu[rr][j], ub + (int64_t)(r0 + rr) * rb, usb + (int64_t)(r0 + rr) * sb, c);
                }
            }
        }
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
                    const float g = wave_sum(ag[rr][t]);
                    const float v = wave_sum(av[rr][t]);
                    if (lane == rr) st_dev(arow + rr, silu_mul(g, v));
                }
                ++i;
            }
        }
    }
}

// Down rows [h0, h1) of one unit with K inputs: a half-wave owns RD rows at a time, lane l of
// the half covers elements 8c..8c+7 for c = l + 32 j.  `db`/`dsb` point at row 0 of the weights
// (global or LDS).  The unit's `tcount` SwiGLU rows are in LDS at `acts` ([tcount][K] fp32).
// Partial outputs go to pair rows row0 + t of the partial buffer.
template <int WF, int RD, int NJD, int MT>
__device__ void down_rows(const Params& p, const uint8_t* db, const uint8_t* dsb, int K, int h0, int h1,
                          const float* acts, int tcount, int row0) {
    const int H = p.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hl = lane & 31, half = wave * 2 + (lane >> 5);
    constexpr int NH = kWaves * 2;
    const int nch = K / 8;
    const int64_t rb = row_bytes<WF>(K);
    const int64_t sb = K / 32;
    for (int h = h0 + half * RD; h < h1; h += NH * RD) {
        Raw<WF> wd[RD][NJD];
#pragma unroll
        for (int rr = 0; rr < RD; ++rr) {
#pragma unroll
            for (int j = 0; j < NJD; ++j) {
                const int c = hl + 32 * j;
                if (c < nch && h + rr < h1)
                    load_raw<WF>(wd[rr][j], db + (int64_t)(h - h0 + rr) * rb, dsb + (int64_t)(h - h0 + rr) * sb, c);
            }
        }
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
                    const float s = half_sum(acc[rr][t]);
                    if (hl == rr && h + rr < h1) st_dev(p.ws.part + (int64_t)(row0 + t) * H + h + rr, s);
                }
            }
        }
    }
}

// Stages `tcount` SwiGLU rows (K floats each, starting at pair row row0) into LDS.
__device__ __forceinline__ void stage_acts(const Params& p, float* acts, int row0, int tcount, int K) {
    for (int i = threadIdx.x; i < tcount * K; i += kThreads) {
        const int t = i / K, c = i - t * K;
        acts[i] = ld_dev(p.ws.act + (int64_t)(row0 + t) * p.act_stride + c);
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
    __shared__ uint32_t s_call;

    // ---- A: call index, token rows, shared-expert down prefetch, router rows ----
    if (threadIdx.x == 0) s_call = ld_dev(p.ws.hdr + kHdrCall);
    stage16(xs, p.x, M * H * XB);
    __syncthreads();
    const uint32_t call = s_call;
    uint32_t* set = p.ws.ctr + (int64_t)(call & 1u) * kSetWords;
    if (b == 0) {
        uint32_t* nxt = p.ws.ctr + (int64_t)((call + 1u) & 1u) * kSetWords;
        for (int l = threadIdx.x; l < kSetLines; l += kThreads) line(nxt, l)[0] = 0u;
    }
    const int sh0 = (int)((int64_t)H * b / G), sh1 = (int)((int64_t)H * (b + 1) / G);
    const int64_t rb_sh = row_bytes<WF>(Is);
    if (has_sh && !p.route_only && sh1 > sh0)  // rows are 16-byte multiples in every format
        async_to_lds<16>(shw, (const uint8_t*)p.w.sh_down + sh0 * rb_sh, (int)((sh1 - sh0) * rb_sh));
    router_rows<AF>(p, xs, (int)((int64_t)E * b / G), (int)((int64_t)E * (b + 1) / G));
    publish();
    if (threadIdx.x == 0) {
        const int s = b % kRouteSubs;
        const uint32_t members = G / kRouteSubs + (s < G % kRouteSubs ? 1 : 0);
        if (add_dev(line(set, s), 1u) + 1u == members) add_dev(line(set, kLineRouteTop), 1u);
    }
    if (p.route_only && b != 0) return;

    // ---- A': shared expert gate/up (needs no routing) ----
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
            const uint32_t all = (1u << M) - 1u;
            gateup_rows<AF, WF, R, NJ, MT>(p, xs, (const uint8_t*)p.w.sh_gate, (const uint8_t*)p.w.sh_up, gsb, usb,
                                           g0, g1, all, NP);
            publish();
            if (threadIdx.x == 0) add_dev(line(set, kLineShared), (uint32_t)(g1 - g0) * R);
        }
    }

    // ---- B: routing barrier, top-k and compaction in every workgroup ----
    wait_geq(line(set, kLineRouteTop), (uint32_t)min(G, kRouteSubs), p.ws.hdr + kHdrStatus);
    const int U = route_and_compact(p, tab, (char*)acts, b == 0);
    if (b == 0 && threadIdx.x == 0) __hip_atomic_store(p.ws.hdr + kHdrCall, call + 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
    if (p.route_only) return;
    const uint32_t* s_mask = (const uint32_t*)tab + kTabMask;
    const int* s_off = tab + kTabOff;
    const int* s_exp = tab + kTabExp;

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
    if (has_sh && sh1 > sh0) {
        wait_geq(line(set, kLineShared), (uint32_t)Is, p.ws.hdr + kHdrStatus);
        stage_acts(p, acts, NP, M, Is);
        __builtin_amdgcn_s_waitcnt(0);  // the async copy of the weights has landed
        __syncthreads();
        const uint8_t* dsb = nullptr;  // MXFP4 scales are read from global memory
        if constexpr (WF == MOE_FMT_MXFP4) dsb = p.w.sh_down_s + (int64_t)sh0 * (Is / 32);
        down_rows<WF, RD, NJD, MT>(p, (const uint8_t*)shw, dsb, Is, sh0, sh1, acts, M, NP);
        __syncthreads();
    }
    const int64_t dtotal = (int64_t)U * H;
    const int64_t d0 = dtotal * b / G, d1 = dtotal * (b + 1) / G;
    {
        const int64_t rbI = row_bytes<WF>(I);
        for (int64_t q = d0; q < d1;) {
            const int u = (int)(q / H);
            const int ha = (int)(q - (int64_t)u * H);
            const int hb = (int)min<int64_t>(H, ha + (d1 - q));
            q += hb - ha;
            const uint32_t mask = s_mask[u];
            const int tcount = __popc(mask);
            const int64_t e = s_exp[u];
            wait_geq(line(set, kLineUnit0 + u), (uint32_t)I, p.ws.hdr + kHdrStatus);
            stage_acts(p, acts, s_off[u], tcount, I);
            __syncthreads();
            const uint8_t* dsb = nullptr;
            if constexpr (WF == MOE_FMT_MXFP4) dsb = p.w.down_s + (e * H + ha) * (I / 32);
            down_rows<WF, RD, NJD, MT>(p, (const uint8_t*)p.w.down + (e * H + ha) * rbI, dsb, I, ha, hb, acts, tcount,
                                       s_off[u]);
            __syncthreads();
        }
    }
    publish();

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
    const int nd = s_ndone;
    const int* s_pair = tab + kTabPair;
    const float* s_roww = (const float*)(tab + kTabRowW);
    for (int d = 0; d < nd; ++d) {
        const int tile = s_done[d];
        const int ta = tile * kCombineTile, tb = min(H, ta + kCombineTile);
        for (int i = threadIdx.x; i < M * (tb - ta); i += kThreads) {
            const int m = i / (tb - ta), h = ta + i % (tb - ta);
            float s = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int row = s_pair[m * k + j];
                s = fmaf(s_roww[row], ld_dev(p.ws.part + (int64_t)row * H + h), s);
            }
            if (has_sh) s += ld_dev(p.ws.part + (int64_t)(NP + m) * H + h);
            if constexpr (AF == MOE_FMT_F32)
                ((float*)p.y)[(int64_t)m * H + h] = s;
            else
                ((uint16_t*)p.y)[(int64_t)m * H + h] = f32_to_bf16_rne(s);
        }
    }
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
        p.lds_total = p.lds_act + round16(act_bytes > kSelBytes ? act_bytes : kSelBytes);
        p.sh_rows = sh_rows;
        if ((int64_t)per_cu * (p.lds_total + 1024) > kLdsPerCu && per_cu > 1) continue;
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
