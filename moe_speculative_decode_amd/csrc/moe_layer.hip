// Routed-expert MoE decode layer for CDNA4 (gfx950): router GEMV + softmax top-k + dispatch
// compaction, fused gate/up SwiGLU GEMV, and down GEMV with a deterministic weighted combine.
//
// The layer follows the chain the Ling-3.0-flash decode pages describe ("Chasing the Batch-1
// Floor", section "PDL: stacking the latency floors of small kernels": router chain
// gate matvec -> top-k and MoE chain align -> up-GEMM -> activation -> down-GEMM -> combine),
// re-cut for a batch of at most 16 tokens on an MI355X:
//
//   k_route    one wave per router row; the last workgroup to finish (arrival counter) does
//              the per-token top-k on the fp32 logits and compacts the batch into units: the
//              distinct selected experts in ascending id order, each with a token bitmask and a
//              block of pair rows, plus the shared expert as the last unit.
//   k_gateup   every workgroup streams an equal share of all units' gate/up rows; each weight
//              row is loaded once and applied to every token of its unit (so a unique expert's
//              weights cross HBM once per call), silu(g) * v is formed in fp32.
//   k_down     every workgroup streams an equal share of all units' down rows and writes fp32
//              per-pair partial outputs; the last workgroup to finish a 64-row tile of y sums the
//              partials of each token in slot order, adds the shared expert and casts once.
//
// No workgroup ever waits for another, so a launch cannot hang: cross-workgroup hand-offs use
// "last arriver does the follow-up" counters, and every counter is reset by its last user.
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

// Copies n bytes (multiple of 16) from global to LDS with every thread of the workgroup.
__device__ __forceinline__ void stage16(void* dst, const void* src, int n) {
    for (int i = threadIdx.x; i < n / 16; i += kThreads) ((u32x4*)dst)[i] = ((const u32x4*)src)[i];
}

// LDS ints holding the unit tables (mask, first row, expert of up to kMaxExperts + 1 units)
constexpr int kTableInts = 1552;  // >= 3 * (kMaxExperts + 1), multiple of 4
constexpr int kTileSlots = 68;    // >= ceil(4096 / kCombineTile), multiple of 4

__device__ __forceinline__ float silu_mul(float g, float v) { return g / (1.0f + __expf(-g)) * v; }

// ------------------------------------------------------------------------------------------
// k_route: router GEMV (one wave per expert row), then top-k + compaction in the last workgroup
// ------------------------------------------------------------------------------------------

// Top-k of one token's E logits with one wave.  Ties go to the lower expert id.  Results in
// descending order: ids and softmax-over-the-k weights.  `cv`/`ci` are per-wave LDS scratch of
// kMaxExperts entries.  Every id written is in [0, E).
__device__ void wave_topk(const float* lrow, int E, int k, float* cv, int* ci, int* out_id, float* out_w,
                          float* out_v) {
    const int lane = threadIdx.x & 63;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? lrow[e] : -INFINITY;
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
        cand[i] = v[i] >= tau && lane + 64 * i < E;  // padding lanes never become candidates
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

template <int AF>
__global__ __launch_bounds__(kThreads) void k_route(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int H = p.H, E = p.E, M = p.M, k = p.k;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;  // bytes per activation

    stage16(smem, p.x, M * H * XB);
    __syncthreads();

    // ---- logits: row e = this wave's router row, all tokens ----
    const int e = blockIdx.x * kWaves + wave;
    if (e < E) {
        const uint8_t* row = (const uint8_t*)p.wr + (int64_t)e * H * XB;
        const int nch = H / 8;
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
                        const f32x4* xr = (const f32x4*)(smem + (int64_t)m * H * 4) + 2 * c;
                        acc[m] = dot8_f32x<AF>(r, xr[0], xr[1], acc[m]);
                    } else {
                        const u32x4 xq = *((const u32x4*)(smem + (int64_t)m * H * 2) + c);
                        acc[m] = dot8_bf16x<AF>(r, xq, acc[m]);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < kMaxTokens; ++m) {
            if (m < M) {
                const float s = wave_sum(acc[m]);
                if (lane == 0) p.ws.logits[(int64_t)m * E + e] = s;
            }
        }
    }

    // ---- last workgroup: top-k and compaction ----
    __shared__ int s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(p.ws.route_cnt, 1u) == gridDim.x - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (threadIdx.x == 0) *p.ws.route_cnt = 0u;

    // LDS layout for this phase (reuses the x area)
    float* cand_v = (float*)smem;                                 // [kWaves][kMaxExperts]
    int* cand_i = (int*)(cand_v + kWaves * kMaxExperts);          // [kWaves][kMaxExperts]
    int* sid = cand_i + kWaves * kMaxExperts;                     // [M*k]
    float* sw = (float*)(sid + kMaxTokens * kMaxTopK);            // [M*k]
    float* sv = sw + kMaxTokens * kMaxTopK;                       // [M*k] selected logits
    uint32_t* tokmask = (uint32_t*)(sv + kMaxTokens * kMaxTopK);  // [E]
    uint32_t* scan = tokmask + kMaxExperts;                       // [E]
    uint32_t* wtot = scan + kMaxExperts;                          // [kWaves]
    __shared__ int s_req_unique[kMaxTokens];

    for (int m = wave; m < M; m += kWaves)
        wave_topk(p.ws.logits + (int64_t)m * E, E, k, cand_v + wave * kMaxExperts, cand_i + wave * kMaxExperts,
                  sid + m * k, sw + m * k, sv + m * k);
    for (int i = threadIdx.x; i < E; i += kThreads) tokmask[i] = 0u;
    __syncthreads();
    const int NP = M * k;
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
    const bool has_sh = p.Is > 0;
    for (int i = threadIdx.x; i < E; i += kThreads) {
        const uint32_t tm = tokmask[i];
        if (tm) {
            const int u = (int)(scan[i] >> 16);
            const int off = (int)(scan[i] & 0xFFFFu);
            p.ws.unit_expert[u] = i;
            p.ws.unit_mask[u] = tm;
            p.ws.unit_off[u] = off;
            if (p.disp.unit_expert) p.disp.unit_expert[u] = i;
            if (p.disp.unit_off) p.disp.unit_off[u] = off;
        }
    }
    if (threadIdx.x == 0) {
        *p.ws.n_units = U;
        p.ws.unit_expert[U] = E;
        p.ws.unit_mask[U] = has_sh ? ((1u << M) - 1u) : 0u;
        p.ws.unit_off[U] = NP;
        p.ws.unit_off[U + 1] = NP + (has_sh ? M : 0);
        if (p.disp.unit_count) *p.disp.unit_count = U;
        if (p.disp.unit_off) p.disp.unit_off[U] = NP;
        if (has_sh) {
            if (p.disp.unit_expert) p.disp.unit_expert[U] = E;
            if (p.disp.unit_off) p.disp.unit_off[U + 1] = NP + M;
        }
    }
    for (int q = threadIdx.x; q < NP; q += kThreads) {
        const int m = q / k, j = q % k, ex = sid[q];
        const int row = (int)(scan[ex] & 0xFFFFu) + __popc(tokmask[ex] & ((1u << m) - 1u));
        p.ws.pair_row[q] = row;
        p.ws.row_w[row] = sw[q];
        if (p.topk_ids) p.topk_ids[q] = ex;
        if (p.topk_w) p.topk_w[q] = sw[q];
        if (p.disp.row_token) p.disp.row_token[row] = m;
        if (p.disp.row_slot) p.disp.row_slot[row] = j;
        if (p.disp.row_weight) p.disp.row_weight[row] = sw[q];
    }
    for (int m = threadIdx.x; m < (has_sh ? M : 0); m += kThreads) {
        p.ws.row_w[NP + m] = 1.0f;
        if (p.disp.row_token) p.disp.row_token[NP + m] = m;
        if (p.disp.row_slot) p.disp.row_slot[NP + m] = k;
        if (p.disp.row_weight) p.disp.row_weight[NP + m] = 1.0f;
    }
    // packed-request offsets: validate, and count distinct routed experts per request
    if (p.req_off) {
        __shared__ int s_bad;
        if (threadIdx.x == 0) {
            int bad = (p.R < 1 || p.req_off[0] != 0 || p.req_off[p.R] != M) ? 1 : 0;
            for (int r = 0; r < p.R && !bad; ++r) bad = p.req_off[r + 1] < p.req_off[r];
            s_bad = bad;
            if (bad) atomicOr(p.ws.status, kStatusOffsets);
        }
        if (threadIdx.x < kMaxTokens) s_req_unique[threadIdx.x] = 0;
        __syncthreads();
        if (!s_bad && p.disp.req_unique) {
            for (int r = 0; r < p.R; ++r) {
                const int a = p.req_off[r], b = p.req_off[r + 1];
                const uint32_t rm = (b >= 32 ? ~0u : ((1u << b) - 1u)) & ~((1u << a) - 1u);
                for (int i = threadIdx.x; i < E; i += kThreads)
                    if (tokmask[i] & rm) atomicAdd(&s_req_unique[r], 1);
            }
            __syncthreads();
            for (int r = threadIdx.x; r < p.R; r += kThreads) p.disp.req_unique[r] = s_req_unique[r];
        }
    }
}

// ------------------------------------------------------------------------------------------
// k_gateup: a[row, r] = silu(Wg[r,:] . x) * (Wu[r,:] . x) for every unit row r and pair row
// ------------------------------------------------------------------------------------------
// Work is split in groups of R consecutive intermediate rows of one unit; workgroup b takes the
// b-th equal share of all groups (routed units first, then the shared unit) and its waves take
// groups round-robin.  One lane covers elements 8c..8c+7 for c = lane + 64 j of each row, so a
// weight row is read as 64-lane-contiguous 16-byte (bf16) or 4-byte (MXFP4) pieces.
template <int AF, int WF, int R, int NJ, int MT>
__global__ __launch_bounds__(kThreads) void k_gateup(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int H = p.H, M = p.M;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;

    const int U = *p.ws.n_units;
    const bool has_sh = p.Is > 0;
    const int nun = U + (has_sh ? 1 : 0);
    uint32_t* s_mask = (uint32_t*)smem;           // [kMaxExperts + 1]
    int* s_off = (int*)(s_mask + kMaxExperts + 1);  // [kMaxExperts + 1]
    int* s_exp = s_off + kMaxExperts + 1;           // [kMaxExperts + 1]
    char* xs = smem + kTableInts * 4;               // x [M][H], 16-byte aligned
    for (int u = threadIdx.x; u < nun; u += kThreads) {
        s_mask[u] = p.ws.unit_mask[u];
        s_off[u] = p.ws.unit_off[u];
        s_exp[u] = p.ws.unit_expert[u];
    }
    stage16(xs, p.x, M * H * XB);
    __syncthreads();

    const int gI = p.I / R, gS = has_sh ? p.Is / R : 0;
    const int64_t total = (int64_t)U * gI + gS;
    const int64_t q0 = total * blockIdx.x / gridDim.x, q1 = total * (blockIdx.x + 1) / gridDim.x;
    const int nch = H / 8;
    const int64_t rb_bytes = row_bytes<WF>(H);
    const int64_t srow_bytes = H / 32;

    for (int64_t q = q0 + wave; q < q1; q += kWaves) {
        int u, r0;
        const uint8_t *gb, *ub, *gsb = nullptr, *usb = nullptr;
        if (q < (int64_t)U * gI) {
            u = (int)(q / gI);
            r0 = (int)(q % gI) * R;
            const int64_t e = s_exp[u];
            const int64_t row0 = e * p.I + r0;
            gb = (const uint8_t*)p.w.gate + row0 * rb_bytes;
            ub = (const uint8_t*)p.w.up + row0 * rb_bytes;
            if constexpr (WF == MOE_FMT_MXFP4) {
                gsb = p.w.gate_s + row0 * srow_bytes;
                usb = p.w.up_s + row0 * srow_bytes;
            }
        } else {
            u = U;
            r0 = (int)(q - (int64_t)U * gI) * R;
            gb = (const uint8_t*)p.w.sh_gate + (int64_t)r0 * rb_bytes;
            ub = (const uint8_t*)p.w.sh_up + (int64_t)r0 * rb_bytes;
            if constexpr (WF == MOE_FMT_MXFP4) {
                gsb = p.w.sh_gate_s + (int64_t)r0 * srow_bytes;
                usb = p.w.sh_up_s + (int64_t)r0 * srow_bytes;
            }
        }
        // issue every load of the group first
        Raw<WF> wg[R][NJ], wu[R][NJ];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c = lane + 64 * j;
                if (c < nch) {
                    load_raw<WF>(wg[rr][j], gb + rr * rb_bytes, gsb + rr * srow_bytes, c);
                    load_raw<WF>(wu[rr][j], ub + rr * rb_bytes, usb + rr * srow_bytes, c);
                }
            }
        }
        const uint32_t mask = s_mask[u];
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
        // reduce and write: the i-th token of the unit owns pair row s_off[u] + i
        int i = 0;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if ((mask >> t) & 1u) {
                float* arow = p.ws.act + (int64_t)(s_off[u] + i) * p.act_stride + r0;
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    const float g = wave_sum(ag[rr][t]);
                    const float v = wave_sum(av[rr][t]);
                    if (lane == rr) arow[rr] = silu_mul(g, v);
                }
                ++i;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// k_down: part[row, h] = Wd[h,:] . a[row,:] per unit, then the per-tile combine into y
// ------------------------------------------------------------------------------------------
// Rows h of all units form one flat range split in equal shares over workgroups.  A half-wave
// owns RD rows at a time; lane l of the half covers elements 8c..8c+7, c = l + 32 j, of each row.
// The unit's SwiGLU rows are staged in LDS once per workgroup segment.
template <int AF, int WF, int RD, int NJD, int MT>
__global__ __launch_bounds__(kThreads) void k_down(Params p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int H = p.H, M = p.M, k = p.k;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hl = lane & 31, half = wave * 2 + (lane >> 5);  // half-wave id in the workgroup
    constexpr int NH = kWaves * 2;

    const int U = *p.ws.n_units;
    const bool has_sh = p.Is > 0;
    const int nun = U + (has_sh ? 1 : 0);
    uint32_t* s_mask = (uint32_t*)smem;
    int* s_off = (int*)(s_mask + kMaxExperts + 1);
    int* s_exp = s_off + kMaxExperts + 1;
    int* s_tiles = (int*)smem + kTableInts;           // [ntiles] tiles this workgroup finishes
    float* s_act = (float*)(s_tiles + kTileSlots);    // [MT][max(I,Is)] (16-byte aligned)
    __shared__ int s_ntiles_done;
    for (int u = threadIdx.x; u < nun; u += kThreads) {
        s_mask[u] = p.ws.unit_mask[u];
        s_off[u] = p.ws.unit_off[u];
        s_exp[u] = p.ws.unit_expert[u];
    }
    if (threadIdx.x == 0) s_ntiles_done = 0;
    __syncthreads();

    const int64_t total = (int64_t)nun * H;
    const int64_t q0 = total * blockIdx.x / gridDim.x, q1 = total * (blockIdx.x + 1) / gridDim.x;

    for (int64_t seg = q0; seg < q1;) {
        const int u = (int)(seg / H);
        const int h0 = (int)(seg % H);
        const int h1 = (int)min<int64_t>((int64_t)H, h0 + (q1 - seg));
        seg += h1 - h0;
        const bool shared = u == U;
        const int K = shared ? p.Is : p.I;
        const uint32_t mask = s_mask[u];
        const int tcount = __popc(mask);
        const int base_row = s_off[u];
        // stage this unit's SwiGLU rows
        __syncthreads();
        for (int i = threadIdx.x; i < tcount * K / 4; i += kThreads) {
            const int t = i / (K / 4), c4 = i % (K / 4);
            ((f32x4*)s_act)[t * (K / 4) + c4] = ((const f32x4*)(p.ws.act + (int64_t)(base_row + t) * p.act_stride))[c4];
        }
        __syncthreads();
        const int64_t rb_bytes = row_bytes<WF>(K);
        const int64_t srow_bytes = K / 32;
        const uint8_t *db, *dsb = nullptr;
        if (shared) {
            db = (const uint8_t*)p.w.sh_down;
            if constexpr (WF == MOE_FMT_MXFP4) dsb = p.w.sh_down_s;
        } else {
            const int64_t e = s_exp[u];
            db = (const uint8_t*)p.w.down + e * H * rb_bytes;
            if constexpr (WF == MOE_FMT_MXFP4) dsb = p.w.down_s + e * H * srow_bytes;
        }
        const int nch = K / 8;
        for (int h = h0 + half * RD; h < h1; h += NH * RD) {
            Raw<WF> wd[RD][NJD];
#pragma unroll
            for (int rr = 0; rr < RD; ++rr) {
#pragma unroll
                for (int j = 0; j < NJD; ++j) {
                    const int c = hl + 32 * j;
                    if (c < nch && h + rr < h1)
                        load_raw<WF>(wd[rr][j], db + (int64_t)(h + rr) * rb_bytes, dsb + (int64_t)(h + rr) * srow_bytes, c);
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
                            const f32x4* ar = (const f32x4*)(s_act + t * K) + 2 * c;
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
                        if (hl == rr && h + rr < h1) p.ws.part[(int64_t)(base_row + t) * H + h + rr] = s;
                    }
                }
            }
        }
    }

    // ---- report finished rows per y tile; the last contributor of a tile combines it ----
    __threadfence();
    __syncthreads();
    const int ntiles = (H + kCombineTile - 1) / kCombineTile;
    for (int tile = threadIdx.x; tile < ntiles; tile += kThreads) {
        const int ta = tile * kCombineTile, tb = min(H, ta + kCombineTile);
        int64_t mine = 0;
        for (int64_t u = q0 / H; u <= (q1 - 1) / H && q1 > q0; ++u) {
            const int64_t a = max(q0, u * H + ta), b = min(q1, u * H + tb);
            if (b > a) mine += b - a;
        }
        if (mine > 0) {
            const uint32_t need = (uint32_t)nun * (uint32_t)(tb - ta);
            const uint32_t old = atomicAdd(&p.ws.tile_cnt[tile], (uint32_t)mine);
            if (old + (uint32_t)mine == need) s_tiles[atomicAdd(&s_ntiles_done, 1)] = tile;
        }
    }
    __syncthreads();
    const int nd = s_ntiles_done;
    if (nd == 0) return;
    __threadfence();
    const int NP = M * k;
    for (int d = 0; d < nd; ++d) {
        const int tile = s_tiles[d];
        const int ta = tile * kCombineTile, tb = min(H, ta + kCombineTile);
        for (int i = threadIdx.x; i < M * (tb - ta); i += kThreads) {
            const int m = i / (tb - ta), h = ta + i % (tb - ta);
            float s = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int row = p.ws.pair_row[m * k + j];
                s = fmaf(p.ws.row_w[row], p.ws.part[(int64_t)row * H + h], s);
            }
            if (has_sh) s += p.ws.part[(int64_t)(NP + m) * H + h];
            if constexpr (AF == MOE_FMT_F32)
                ((float*)p.y)[(int64_t)m * H + h] = s;
            else
                ((uint16_t*)p.y)[(int64_t)m * H + h] = f32_to_bf16_rne(s);
        }
        if (threadIdx.x == 0) p.ws.tile_cnt[tile] = 0u;
    }
}

// ------------------------------------------------------------------------------------------
// launch helpers
// ------------------------------------------------------------------------------------------

template <typename K>
hipError_t launch(K kernel, int grid, size_t lds, hipStream_t s, const Params& p) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

size_t table_lds() { return (size_t)kTableInts * sizeof(int); }
constexpr size_t kLdsPerCu = 160 * 1024;

template <int AF, int WF, int MT>
hipError_t launch_experts(const Params& p, int num_cus, hipStream_t s) {
    constexpr int XB = AF == MOE_FMT_F32 ? 4 : 2;
    const int nj = (p.H / 8 + 63) / 64;
    const int ka = p.Is > p.I ? p.Is : p.I;
    const int njd = (ka / 8 + 31) / 32;
    const size_t lds_g = table_lds() + (size_t)p.M * p.H * XB;
    const size_t lds_d = table_lds() + kTileSlots * sizeof(int) + (size_t)MT * ka * sizeof(float);
    // two workgroups per CU where their LDS fits
    const int grid_g = (2 * lds_g <= kLdsPerCu ? 2 : 1) * num_cus;
    const int grid_d = (2 * lds_d <= kLdsPerCu ? 2 : 1) * num_cus;
    hipError_t err = hipErrorInvalidValue;
    constexpr int R = WF == MOE_FMT_MXFP4 ? 2 : 1;
#define GATEUP(NJV)                                                                          \
    if (nj <= NJV) {                                                                         \
        auto kern = k_gateup<AF, WF, R, NJV, MT>;                                            \
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_g); \
        err = launch(kern, grid_g, lds_g, s, p);                                               \
    } else
    GATEUP(1) GATEUP(2) GATEUP(5) GATEUP(8) { return hipErrorInvalidValue; }
#undef GATEUP
    if (err != hipSuccess) return err;
#define DOWN(NJV)                                                                            \
    if (njd <= NJV) {                                                                        \
        auto kern = k_down<AF, WF, 2, NJV, MT>;                                              \
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_d); \
        err = launch(kern, grid_d, lds_d, s, p);                                               \
    } else
    DOWN(1) DOWN(2) DOWN(3) DOWN(4) DOWN(8) { return hipErrorInvalidValue; }
#undef DOWN
    return err;
}

}  // namespace

hipError_t launch_layer(const Params& p, bool route_only, int num_cus, hipStream_t s) {
    const int XB = p.act_fmt == MOE_FMT_F32 ? 4 : 2;
    const size_t lds_route_x = (size_t)p.M * p.H * XB;
    const size_t lds_route_sel = (size_t)kWaves * kMaxExperts * 8 + 3 * kMaxTokens * kMaxTopK * 4 +
                                 2 * kMaxExperts * 4 + kWaves * 4;
    const size_t lds_r = lds_route_x > lds_route_sel ? lds_route_x : lds_route_sel;
    const int grid_r = (p.E + kWaves - 1) / kWaves;
    hipError_t err;
    if (p.act_fmt == MOE_FMT_F32) {
        (void)hipFuncSetAttribute((const void*)k_route<MOE_FMT_F32>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_r);
        err = launch(k_route<MOE_FMT_F32>, grid_r, lds_r, s, p);
    } else {
        (void)hipFuncSetAttribute((const void*)k_route<MOE_FMT_BF16>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_r);
        err = launch(k_route<MOE_FMT_BF16>, grid_r, lds_r, s, p);
    }
    if (err != hipSuccess || route_only) return err;
    if (p.act_fmt == MOE_FMT_F32) return launch_experts<MOE_FMT_F32, MOE_FMT_F32, kMaxTokens>(p, num_cus, s);
    if (p.w_fmt == MOE_FMT_BF16) {
        if (p.M == 1) return launch_experts<MOE_FMT_BF16, MOE_FMT_BF16, 1>(p, num_cus, s);
        return launch_experts<MOE_FMT_BF16, MOE_FMT_BF16, kMaxTokens>(p, num_cus, s);
    }
    if (p.M == 1) return launch_experts<MOE_FMT_BF16, MOE_FMT_MXFP4, 1>(p, num_cus, s);
    return launch_experts<MOE_FMT_BF16, MOE_FMT_MXFP4, kMaxTokens>(p, num_cus, s);
}

}  // namespace moe
