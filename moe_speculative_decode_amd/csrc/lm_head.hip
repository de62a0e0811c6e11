// The LM head of the decode step: logits [M][V] = x [M][H] . W [V][H]^T with fp32 accumulation,
// for a batch-1 token or a small verify window.  At these M the projection is a bandwidth-bound
// GEMV over the whole weight ("Chasing the Batch-1 Floor", section "bf16 router gate and lm_head":
// every decode step cold-reads the vocabulary projection, with no arithmetic to hide the read;
// "3 ways to boost MoE inference on NVIDIA DGX Spark", "Optimization 2: Online FP8 LM head
// quantization": 157,184 x 2,560, and FP8 weights halve the read).
//
// One workgroup of 8 waves per compute unit; every wave streams a contiguous range of rows once
// with 16-byte non-temporal loads (bf16: one row of 64 lanes per step, 1 KB per load instruction;
// FP8: two rows of 32 lanes per step, 512 B per row and instruction), keeps the next step's loads
// in flight while it computes the current one, applies each row to all M token rows staged in LDS
// (a fixed lane split and DPP tree per row: results do not depend on timing), and stages its
// logits in LDS.  They are written out once, token-major and coalesced, after the stream: a store
// inside the loop would make every later wait for prefetched rows also wait for it (vector memory
// operations retire in order).  No workspace, no cross-workgroup waits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/moe_decode.h"

namespace {

#define LDS __attribute__((address_space(3)))

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsBytes = 160 * 1024 - 512;
constexpr int kMaxHidden = 2560;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_rows(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
// Sum over each group of LPR consecutive lanes (32 or 64), valid in the group's last lane.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror: every lane of a 16-lane row holds its row's sum
    v += __builtin_bit_cast(float, dpp_rows<0x142, 0xA>(0, __builtin_bit_cast(int, v)));  // rows 1, 3 += rows 0, 2
    if constexpr (LPR == 64)
        v += __builtin_bit_cast(float, dpp_rows<0x143, 0xC>(0, __builtin_bit_cast(int, v)));  // rows 2, 3 += row 1
    else
        static_assert(LPR == 32, "rows of 32 or 64 lanes");
    return v;
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

struct LMParams {
    int H, V, M;
    const void* x;
    const uint8_t* w;
    const float* scale;  // FP8: [V]
    float* logits;       // [M][V]
    int stage_rows;      // rows a wave stages (the largest row range of any wave)
    int lds_stage;       // byte offset of the logit staging area
    int xpitch;          // matrix-core form: bytes between token rows in LDS
    int lds_tr;          // matrix-core form: byte offset of the waves' transpose buffers
};

// WF: MOE_FMT_BF16 (8 elements a chunk, 64 lanes a row) or MOE_FMT_FP8 (16 E4M3 codes a chunk,
// 32 lanes a row).  NJ chunks per lane cover a row.
template <int WF, int NJ>
__global__ __launch_bounds__(kThreads) void k_lm_head(LMParams p) {
    constexpr bool F8 = WF == MOE_FMT_FP8;
    constexpr int EPC = F8 ? 16 : 8;
    constexpr int LPR = F8 ? 32 : 64;
    constexpr int RS = 64 / LPR;  // rows per wave step
    extern __shared__ __attribute__((aligned(16))) char smem[];
    LDS char* xs = (LDS char*)smem;                        // [M][H] bf16
    LDS float* stage = (LDS float*)(smem + p.lds_stage);   // [kWaves][stage_rows][M]
    const int lane = threadIdx.x & 63, wave = wave_id(), gi = lane / LPR, sl = lane % LPR;
    const int H = p.H, M = p.M, nch = H / EPC;
    const int64_t rb = F8 ? H : 2 * H;

    // token rows into LDS: each wave copies 1 KB lines; lane l's 16 bytes land at the line's LDS
    // base (wave-uniform) plus 16 l
    {
        const int n = M * H * 2;
        for (int base = wave * 1024; base < n; base += kWaves * 1024)
            if (base + lane * 16 < n)
                __builtin_amdgcn_global_load_lds((const uint8_t*)p.x + base + lane * 16, (LDS void*)(xs + base), 16, 0, 0);
    }

    // this wave's rows [r0, r1)
    const int64_t W = (int64_t)gridDim.x * kWaves, gw = (int64_t)blockIdx.x * kWaves + wave;
    const int r0 = (int)(p.V * gw / W), r1 = (int)(p.V * (gw + 1) / W);
    const int nsteps = (r1 - r0 + RS - 1) / RS;
    LDS float* my_stage = stage + (int64_t)wave * p.stage_rows * M;

    struct Buf {
        u32x4 q[NJ];
        float s;
    };
    // step t's rows; past the range (and for the stand-in prefetch after the last step) the last
    // row is re-read, so every load is in bounds and the number of loads in flight is static
    auto load = [&](Buf& b, int t) {
        const int row = min(r0 + t * RS + gi, r1 - 1);
        const uint8_t* wr = p.w + (int64_t)row * rb;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            b.q[j] = __builtin_nontemporal_load((const u32x4*)(wr + 16 * min(sl + LPR * j, nch - 1)));
        if constexpr (F8) b.s = p.scale[row];
    };
    auto compute = [&](Buf& b, int t) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(b.q[j]));
        if constexpr (F8) asm volatile("" : "+v"(b.s));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if (sl + LPR * j >= nch) b.q[j] = u32x4{0u, 0u, 0u, 0u};
        const int lr = t * RS + gi;  // row of the wave's range
        for (int m = 0; m < M; ++m) {
            const LDS char* xr = xs + (int64_t)m * H * 2;
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c = min(sl + LPR * j, nch - 1);
                if constexpr (F8) {
                    const LDS u32x4* xp = (const LDS u32x4*)(xr + 32 * c);
                    const u32x4 xa = xp[0], xb = xp[1];
                    const uint32_t xd[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t w = b.q[j][d];
                        acc[d] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false),
                                                                 as_bf16x2(xd[2 * d]), acc[d], false);
                        acc[d] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true),
                                                                 as_bf16x2(xd[2 * d + 1]), acc[d], false);
                    }
                } else {
                    const u32x4 xv = *(const LDS u32x4*)(xr + 16 * c);
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        acc[d] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(b.q[j][d]), as_bf16x2(xv[d]), acc[d], false);
                }
            }
            float s = group_sum<LPR>((acc[0] + acc[1]) + (acc[2] + acc[3]));
            if constexpr (F8) s *= b.s;
            if (sl == LPR - 1 && r0 + lr < r1) my_stage[lr * M + m] = s;
        }
    };
    Buf ba, bb;
    if (nsteps > 0) load(ba, 0);
    __builtin_amdgcn_s_waitcnt(0);  // the token rows have landed (and the first step's rows)
    __syncthreads();
    for (int t = 0; t < nsteps;) {
        load(bb, min(t + 1, nsteps - 1));
        compute(ba, t);
        if (++t >= nsteps) break;
        load(ba, min(t + 1, nsteps - 1));
        compute(bb, t);
        ++t;
    }
    // the wave's logits, token-major (contiguous runs of each token's row of logits)
    const int nr = r1 - r0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    for (int i = lane; i < nr * M; i += 64) {
        const int m = i / nr, r = i - m * nr;
        p.logits[(int64_t)m * p.V + r0 + r] = my_stage[r * M + m];
    }
}

// The matrix-core form, for verify windows (2 <= M <= 16 tokens).  On the vector ALU every weight
// element is applied once per token, and with the token rows in LDS each 16 bytes of weights cost
// M 16-byte LDS reads: at six tokens the bf16 projection ran at 5.2 TB/s and the FP8 one at 3.9.
// Here a chain of v_mfma_f32_16x16x32_bf16 applies a tile of 16 weight rows to all tokens at once
// (A = the tile, B = the token rows, column n = token n; columns past M repeat the last token and
// are dropped).  Each wave streams its rows as tiles of 16 rows in stages of 256 bytes per row:
// four loads per stage, each lane 16 bytes, four rows of 256 contiguous bytes per instruction
// (whole cache lines; the operand layout itself, 16 rows of 64 bytes per instruction, streams
// slower).  The stage goes through a 4 KB LDS buffer of the wave's own to reach the operand layout:
// chunk c of tile row r is stored at slot c ^ r, so the 16 lanes that read one chunk position of
// 16 rows hit 16 different bank groups.  The next R - 1 stages are in flight while one is
// computed.  bf16: a stage is 128 elements, 4 products; FP8: 256 codes, lane (r, kq) takes 16
// codes (two K-groups of 8) per read and decodes them exactly to bf16 (scale 1), 8 products; the
// row's scale multiplies its logit when the logits are written.  Results: one fixed MFMA chain per
// tile, independent of timing.
template <int WF, int R>
__global__ __launch_bounds__(kThreads) void k_lm_head_mfma(LMParams p) {
    constexpr bool F8 = WF == MOE_FMT_FP8;
    constexpr int SE = F8 ? 256 : 128;  // elements of a row per stage (256 bytes)
    constexpr int NP = F8 ? 8 : 4;      // products per stage
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r = lane & 15, kq = lane >> 4;
    const int H = p.H, M = p.M, xp = p.xpitch;
    LDS char* xs = (LDS char*)smem;                               // [M][xpitch] bf16
    LDS char* tb = (LDS char*)smem + p.lds_tr + wave * 4096;      // this wave's [16][256 B]
    LDS float* stage = (LDS float*)(smem + p.lds_stage);          // [kWaves][stage_rows][M]
    const int64_t rb = F8 ? H : 2 * H;

    // token rows into LDS at the padded pitch, 1 KB lines (the LDS base of a line is wave-uniform)
    {
        const int cpr = (2 * H + 1023) / 1024;
        for (int c = wave; c < M * cpr; c += kWaves) {
            const int row = c / cpr, o = (c - row * cpr) * 1024;
            if (o + lane * 16 < 2 * H)
                __builtin_amdgcn_global_load_lds((const uint8_t*)p.x + (int64_t)row * 2 * H + o + lane * 16,
                                                 (LDS void*)(xs + row * xp + o), 16, 0, 0);
        }
    }

    // this wave's rows [r0, r1): tiles of 16 rows (rows past r1 re-read row r1 - 1 and are dropped)
    const int64_t W = (int64_t)gridDim.x * kWaves, gw = (int64_t)blockIdx.x * kWaves + wave;
    const int r0 = (int)(p.V * gw / W), r1 = (int)(p.V * (gw + 1) / W);
    const int nst = H / SE, ntile = (r1 - r0 + 15) / 16, nsteps = ntile * nst;
    LDS float* my_stage = stage + (int64_t)wave * p.stage_rows * M;

    struct Buf {
        u32x4 q[4];
    };
    // step s = (tile s / nst, stage s % nst): instruction i, lane l -> tile row 4 i + l / 16, chunk l % 16
    auto load = [&](Buf& b, int s) {
        const int t = s / nst, g = s - t * nst;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = min(r0 + 16 * t + 4 * i + kq, r1 - 1);
            b.q[i] = __builtin_nontemporal_load((const u32x4*)(p.w + (int64_t)row * rb + 256 * g + 16 * r));
        }
    };
    const LDS char* xrow = xs + min(r, M - 1) * xp;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](Buf& b, int s) {
        const int t = s / nst, g = s - t * nst;
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(b.q[i]));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tr = 4 * i + kq;  // the tile row this lane loaded
            *(LDS u32x4*)(tb + tr * 256 + 16 * (r ^ tr)) = b.q[i];
        }
        asm volatile("" ::: "memory");  // a wave's LDS operations complete in order
        u32x4 a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = *(const LDS u32x4*)(tb + r * 256 + 16 * ((4 * j + kq) ^ r));
        asm volatile("" ::: "memory");
        const LDS char* xg = xrow + 2 * SE * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (F8) {
                const LDS u32x4* xq = (const LDS u32x4*)(xg + 2 * (64 * j + 16 * kq));
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t d0 = a[j][2 * h], d1 = a[j][2 * h + 1];
                    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
                    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
                    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
                    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
                    const bf16x8 av = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, xq[h]), acc, 0, 0, 0);
                }
            } else {
                const u32x4 bv = *(const LDS u32x4*)(xg + 2 * (32 * j + 8 * kq));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                               __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
            }
        }
        if (g == nst - 1) {  // tile done: lane (n, kq) holds rows 4 kq .. 4 kq + 3 of token n
            if (r < M) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = 16 * t + 4 * kq + i;
                    if (r0 + lr < r1) my_stage[lr * M + r] = acc[i];
                }
            }
            acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    static_assert(NP == 4 || NP == 8, "products per stage");
    Buf buf[R];
    if (nsteps > 0) {  // a wave without rows loads nothing
#pragma unroll
        for (int b = 0; b < R; ++b) load(buf[b], min(b, nsteps - 1));
    }
    __builtin_amdgcn_s_waitcnt(0);  // the token rows have landed (and the first stages)
    __syncthreads();
    for (int s = 0; s < nsteps; s += R) {
#pragma unroll
        for (int b = 0; b < R; ++b) {
            if (s + b < nsteps) compute(buf[b], s + b);
            load(buf[b], min(s + b + R, nsteps - 1));  // past the end: a stand-in re-read
        }
    }
    // the wave's logits, token-major; FP8 rows take their scale here
    const int nr = r1 - r0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    for (int i = lane; i < nr * M; i += 64) {
        const int m = i / nr, rr = i - m * nr;
        float v = my_stage[rr * M + m];
        if constexpr (F8) v *= p.scale[r0 + rr];
        p.logits[(int64_t)m * p.V + r0 + rr] = v;
    }
}

constexpr int kMaxDevices = 64;

int grid_size() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <typename K>
hipError_t prepare(K kern) {
    static std::atomic<int> state[kMaxDevices];  // 0 unknown, 1 ready, 2 failed
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int st = state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        st = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) ==
                     hipSuccess
                 ? 1
                 : 2;
        state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? hipSuccess : hipErrorInvalidConfiguration;
}

template <int WF, int NJ>
int launch(LMParams& p, int G, hipStream_t s) {
    auto kern = k_lm_head<WF, NJ>;
    if (prepare(kern) != hipSuccess) return MOE_ERR_HIP;
    const int64_t W = (int64_t)G * kWaves;
    p.stage_rows = (int)((p.V + W - 1) / W);
    p.lds_stage = (p.M * p.H * 2 + 15) / 16 * 16;
    const int lds = p.lds_stage + kWaves * p.stage_rows * p.M * 4;
    if (lds > kLdsBytes) return MOE_ERR_SHAPE;
    hipLaunchKernelGGL(kern, dim3(G), dim3(kThreads), lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int WF>
int launch_mfma(LMParams& p, int G, hipStream_t s) {
    auto kern = k_lm_head_mfma<WF, 4>;
    if (prepare(kern) != hipSuccess) return MOE_ERR_HIP;
    const int64_t W = (int64_t)G * kWaves;
    p.stage_rows = (int)((p.V + W - 1) / W);
    p.xpitch = 2 * p.H + 16;  // 16 token columns of an operand start in 16 bank groups
    p.lds_tr = (p.M * p.xpitch + 15) / 16 * 16;
    p.lds_stage = p.lds_tr + kWaves * 4096;
    const int lds = p.lds_stage + kWaves * p.stage_rows * p.M * 4;
    if (lds > kLdsBytes) return MOE_ERR_SHAPE;
    hipLaunchKernelGGL(kern, dim3(G), dim3(kThreads), lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

bool aligned16(const void* q) { return ((uintptr_t)q & 15u) == 0; }

}  // namespace

extern "C" int moe_lm_head(const moe_lm_head_desc_t* d, int32_t M, const void* x, const void* w, const float* w_scale,
                           float* logits, void* stream) {
    if (!d) return MOE_ERR_NULL;
    const bool f8 = d->weight_format == MOE_FMT_FP8;
    if (d->weight_format != MOE_FMT_BF16 && !f8) return MOE_ERR_FORMAT;
    const int H = d->hidden, V = d->vocab;
    if (H <= 0 || H > kMaxHidden || H % (f8 ? 16 : 8) || V <= 0 || M < 1 || M > MOE_MAX_TOKENS) return MOE_ERR_SHAPE;
    if (!x || !w || !logits || (f8 && !w_scale)) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(logits) || (f8 && ((uintptr_t)w_scale & 3u))) return MOE_ERR_ALIGN;
    const int G = grid_size();
    if (G <= 0) return MOE_ERR_HIP;
    LMParams p{};
    p.H = H;
    p.V = V;
    p.M = M;
    p.x = x;
    p.w = (const uint8_t*)w;
    p.scale = w_scale;
    p.logits = logits;
    hipStream_t s = (hipStream_t)stream;
    // verify windows on the matrix cores (rows in whole stages of 256 bytes)
    if (M >= 2 && H % (f8 ? 256 : 128) == 0)
        return f8 ? launch_mfma<MOE_FMT_FP8>(p, G, s) : launch_mfma<MOE_FMT_BF16>(p, G, s);
    // chunks per lane: bf16 rows of H / 8 chunks over 64 lanes, FP8 rows of H / 16 over 32 lanes
    const int nj = f8 ? (H / 16 + 31) / 32 : (H / 8 + 63) / 64;
    if (f8) return nj <= 1 ? launch<MOE_FMT_FP8, 1>(p, G, s) : launch<MOE_FMT_FP8, 5>(p, G, s);
    return nj <= 1 ? launch<MOE_FMT_BF16, 1>(p, G, s) : launch<MOE_FMT_BF16, 5>(p, G, s);
}
