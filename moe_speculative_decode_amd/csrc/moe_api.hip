// C ABI of the routed-expert MoE decode layer: argument validation, workspace layout and the
// launch sequence.  Everything here runs on the host and enqueues work only; nothing reads device
// memory or synchronises, except moe_read_status which says so in its name.
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace {

using moe::Params;
using moe::Workspace;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool is_aligned(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// byte offsets of the workspace regions for a description (validated by the caller)
struct Layout {
    size_t hdr, ctr, logits, route, act, part, total;
};

Layout layout(const moe_desc_t& d) {
    const size_t Mx = (size_t)d.max_tokens, E = (size_t)d.num_experts, k = (size_t)d.top_k, H = (size_t)d.hidden;
    const size_t ka = (size_t)(d.inter > d.shared_inter ? d.inter : d.shared_inter);
    const size_t rows = Mx * (k + 1);
    Layout L;
    size_t o = 0;
    L.hdr = o;
    o += moe::kHdrBytes;
    L.ctr = o;
    o = up(o + 2 * sizeof(uint32_t) * (size_t)moe::kSetWords);
    L.logits = o;
    o = up(o + 8 * Mx * ((E + 3) / 4 * 4));
    L.route = o;
    o = up(o + 16 * Mx * k);
    L.act = o;
    o = up(o + 4 * rows * ka);
    L.part = o;
    o = up(o + 4 * rows * H);
    L.total = o;
    return L;
}

int check_desc(const moe_desc_t* d) {
    if (!d) return MOE_ERR_NULL;
    const bool f32 = d->act_format == MOE_FMT_F32;
    if (d->act_format != MOE_FMT_F32 && d->act_format != MOE_FMT_BF16) return MOE_ERR_FORMAT;
    if (f32 && d->weight_format != MOE_FMT_F32) return MOE_ERR_FORMAT;
    if (!f32 && d->weight_format != MOE_FMT_BF16 && d->weight_format != MOE_FMT_MXFP4 &&
        d->weight_format != MOE_FMT_FP8)
        return MOE_ERR_FORMAT;
    const int mult = d->weight_format == MOE_FMT_MXFP4 ? 32 : (d->weight_format == MOE_FMT_FP8 ? 128 : 8);
    // the kernel instances cover H <= 2560 and I, Is <= 768 (bf16, MXFP4), and the small binary32
    // layer H, I, Is <= 256
    const int maxH = f32 ? MOE_MAX_HIDDEN_F32 : MOE_MAX_HIDDEN, maxI = f32 ? MOE_MAX_INTER_F32 : MOE_MAX_INTER;
    if (d->hidden <= 0 || d->hidden > maxH || d->hidden % mult) return MOE_ERR_SHAPE;
    if (d->num_experts <= 0 || d->num_experts > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
    if (d->top_k <= 0 || d->top_k > MOE_MAX_TOPK || d->top_k > d->num_experts) return MOE_ERR_SHAPE;
    if (d->inter <= 0 || d->inter > maxI || d->inter % mult) return MOE_ERR_SHAPE;
    if (d->shared_inter < 0 || d->shared_inter > maxI || d->shared_inter % mult) return MOE_ERR_SHAPE;
    if (d->max_tokens <= 0 || d->max_tokens > MOE_MAX_TOKENS) return MOE_ERR_SHAPE;
    if (d->router_flags & ~(MOE_ROUTER_NORM | MOE_ROUTER_BIAS)) return MOE_ERR_FORMAT;
    if ((d->router_flags & MOE_ROUTER_NORM) && f32) return MOE_ERR_FORMAT;  // bf16 activations only
    if ((d->router_flags & MOE_ROUTER_NORM) && !(d->norm_eps >= 0.0f)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// The router prologue tensors of a call (checked on the host).
int check_router(const moe_desc_t* d) {
    if (d->router_flags & MOE_ROUTER_NORM) {
        if (!d->norm_weight) return MOE_ERR_NULL;
        if (!is_aligned(d->norm_weight)) return MOE_ERR_ALIGN;
    }
    if (d->router_flags & MOE_ROUTER_BIAS) {
        if (!d->router_bias) return MOE_ERR_NULL;
        if (!is_aligned(d->router_bias)) return MOE_ERR_ALIGN;
    }
    return MOE_OK;
}

// Checks the description, M, x and the router, and fills the call's parameters with the workspace
// regions of layout L at base.
int fill_params(Params& p, const moe_desc_t* d, int32_t M, const void* x, const void* wr, char* base,
                const Layout& L) {
    if (M < 1 || M > d->max_tokens) return MOE_ERR_SHAPE;
    if (!x || !wr || !base) return MOE_ERR_NULL;
    if (!is_aligned(x) || !is_aligned(wr) || !is_aligned(base)) return MOE_ERR_ALIGN;
    int st = check_router(d);
    if (st) return st;
    memset(&p, 0, sizeof(p));
    p.router_flags = d->router_flags;
    p.norm_eps = d->norm_eps;
    p.norm_w = d->norm_weight;
    p.rbias = d->router_bias;
    p.H = d->hidden;
    p.E = d->num_experts;
    p.k = d->top_k;
    p.I = d->inter;
    p.Is = d->shared_inter;
    p.M = M;
    p.act_fmt = d->act_format;
    p.w_fmt = d->weight_format;
    p.act_stride = d->inter > d->shared_inter ? d->inter : d->shared_inter;
    p.x = x;
    p.wr = wr;
    Workspace& W = p.ws;
    W.hdr = (uint32_t*)(base + L.hdr);
    W.ctr = (uint32_t*)(base + L.ctr);
    W.logits = (uint64_t*)(base + L.logits);
    W.route = (uint64_t*)(base + L.route);
    W.act = (float*)(base + L.act);
    W.part = (float*)(base + L.part);
    return MOE_OK;
}

int fill_common(Params& p, const moe_desc_t* d, int32_t M, const void* x, const void* wr, void* ws, size_t ws_bytes) {
    int st = check_desc(d);
    if (st) return st;
    if (M < 1 || M > d->max_tokens) return MOE_ERR_SHAPE;
    if (!ws) return MOE_ERR_NULL;
    const Layout L = layout(*d);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    return fill_params(p, d, M, x, wr, (char*)ws, L);
}

int check_weights(const moe_desc_t* d, const moe_weights_t* w) {
    if (!w) return MOE_ERR_NULL;
    const bool mx = d->weight_format == MOE_FMT_MXFP4 || d->weight_format == MOE_FMT_FP8;  // block scales
    const void* need[] = {w->gate, w->up, w->down};
    for (const void* q : need) {
        if (!q) return MOE_ERR_NULL;
        if (!is_aligned(q)) return MOE_ERR_ALIGN;
    }
    if (mx) {
        const void* sc[] = {w->gate_s, w->up_s, w->down_s};
        for (const void* q : sc) {
            if (!q) return MOE_ERR_NULL;
            if (!is_aligned(q)) return MOE_ERR_ALIGN;
        }
    }
    if (d->shared_inter > 0) {
        const void* sh[] = {w->sh_gate, w->sh_up, w->sh_down};
        for (const void* q : sh) {
            if (!q) return MOE_ERR_NULL;
            if (!is_aligned(q)) return MOE_ERR_ALIGN;
        }
        if (mx) {
            const void* ss[] = {w->sh_gate_s, w->sh_up_s, w->sh_down_s};
            for (const void* q : ss) {
                if (!q) return MOE_ERR_NULL;
                if (!is_aligned(q)) return MOE_ERR_ALIGN;
            }
        }
    }
    return MOE_OK;
}

// Workgroups per call: one per compute unit of the current device (cached per device).
int grid_size(int* out) {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return MOE_ERR_HIP;
        n = std::min(n, moe::kMaxGrid);
        cache[dev].store(n, std::memory_order_relaxed);
    }
    *out = n;
    return MOE_OK;
}

// Plans the call for this device's grid (a shape whose LDS layout does not fit is rejected here,
// before anything is enqueued) and launches it.
int plan_and_launch(Params& p, hipStream_t stream) {
    int G = 0;
    int st = grid_size(&G);
    if (st) return st;
    if (moe::plan_layer(p, G) != hipSuccess) return MOE_ERR_SHAPE;
    return moe::launch_layer(p, G, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// The forward call's weights, outputs and request offsets (checked on the host).
int fill_forward(Params& p, const moe_desc_t* d, const moe_weights_t* w, const int32_t* req_offsets, int32_t R,
                 void* y, int32_t* topk_ids_out, float* topk_w_out, const moe_dispatch_t* disp) {
    int st = check_weights(d, w);
    if (st) return st;
    if (!y) return MOE_ERR_NULL;
    if (!is_aligned(y)) return MOE_ERR_ALIGN;
    if (req_offsets && (R < 1 || R > MOE_MAX_TOKENS)) return MOE_ERR_OFFSETS;
    p.w = *w;
    p.req_off = req_offsets;
    p.R = req_offsets ? R : 0;
    p.y = y;
    p.topk_ids = topk_ids_out;
    p.topk_w = topk_w_out;
    if (disp) p.disp = *disp;
    if (!req_offsets) p.disp.req_unique = nullptr;
    return MOE_OK;
}

// ---- the fixed scratch of moe_decode_forward_noalloc ---------------------------------------
// Its regions sit at fixed offsets sized for the largest description it serves (max_tokens * (k + 1)
// <= kScratchRows pair rows, E <= 512, H <= 2560, I, Is <= 768), so a region only ever holds its
// own kind of data whatever the description: the tagged logit and routing words never share bytes
// with SwiGLU rows or partial outputs of an earlier call.
constexpr int64_t kScratchRows = 144;  // 16 tokens x (8 routed + 1 shared)

constexpr Layout scratch_layout() {
    Layout L{};
    size_t o = 0;
    L.hdr = o;
    o += moe::kHdrBytes;
    L.ctr = o;
    o = (o + 2 * sizeof(uint32_t) * (size_t)moe::kSetWords + kAlign - 1) / kAlign * kAlign;
    L.logits = o;
    o = (o + 8 * (size_t)MOE_MAX_TOKENS * MOE_MAX_EXPERTS + kAlign - 1) / kAlign * kAlign;
    L.route = o;
    o = (o + 16 * (size_t)kScratchRows + kAlign - 1) / kAlign * kAlign;
    L.act = o;
    o = (o + 4 * (size_t)kScratchRows * MOE_MAX_INTER + kAlign - 1) / kAlign * kAlign;
    L.part = o;
    o = (o + 4 * (size_t)kScratchRows * MOE_MAX_HIDDEN + kAlign - 1) / kAlign * kAlign;
    L.total = o;
    return L;
}
constexpr size_t kScratchBytes = scratch_layout().total;  // 2,138,112 bytes
static_assert(kScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "header and layout disagree");

// One copy per GPU, held until the process ends.  In host code `scratch` names a host-side
// stand-in: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Zero-fill of n 16-byte words (plain vector stores).
__global__ void k_clear(u32x4_t* p, uint32_t n) {
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = u32x4_t{0, 0, 0, 0};
}

// This device's scratch address.  The first call on a device looks it up (with that device
// current) and enqueues, on the caller's stream, a clear of the header, the counter sets and the
// tagged logit and routing words: everything that must start at zero.  The SwiGLU rows and
// partial outputs need no clearing (counters gate every read of them).  Replaying the clear (if
// the first call was captured into a graph) only restores that initial state.
int scratch_on_device(hipStream_t stream, char** out) {
    static std::mutex mu;
    static std::atomic<char*> addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
    char* a = addr[dev].load(std::memory_order_acquire);
    if (!a) {
        std::lock_guard<std::mutex> g(mu);
        a = addr[dev].load(std::memory_order_acquire);
        if (!a) {
            void* ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
            constexpr Layout L = scratch_layout();
            const uint32_t n16 = (uint32_t)((L.act - L.hdr) / 16);
            hipLaunchKernelGGL(k_clear, dim3(64), dim3(256), 0, stream, (u32x4_t*)ptr, n16);
            if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
            a = (char*)ptr;
            addr[dev].store(a, std::memory_order_release);
        }
    }
    *out = a;
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_desc_t* d) {
    if (check_desc(d)) return 0;
    return layout(*d).total;
}

int moe_route(const moe_desc_t* d, int32_t M, const void* x, const void* w_router, int32_t* topk_ids, float* topk_w,
              const moe_dispatch_t* disp, void* ws, size_t ws_bytes, void* stream) {
    Params p;
    int st = fill_common(p, d, M, x, w_router, ws, ws_bytes);
    if (st) return st;
    if (!topk_ids || !topk_w) return MOE_ERR_NULL;
    p.topk_ids = topk_ids;
    p.topk_w = topk_w;
    if (disp) p.disp = *disp;
    p.disp.req_unique = nullptr;
    p.route_only = 1;
    return plan_and_launch(p, (hipStream_t)stream);
}

int moe_decode_forward(const moe_desc_t* d, int32_t M, const void* x, const void* w_router, const moe_weights_t* w,
                       const int32_t* req_offsets, int32_t R, void* y, int32_t* topk_ids_out, float* topk_w_out,
                       const moe_dispatch_t* disp, void* ws, size_t ws_bytes, void* stream) {
    Params p;
    int st = fill_common(p, d, M, x, w_router, ws, ws_bytes);
    if (st) return st;
    if ((st = fill_forward(p, d, w, req_offsets, R, y, topk_ids_out, topk_w_out, disp))) return st;
    return plan_and_launch(p, (hipStream_t)stream);
}

int moe_decode_forward_noalloc(const moe_desc_t* d, int32_t M, const void* x, const void* w_router,
                               const moe_weights_t* w, const int32_t* req_offsets, int32_t R, void* y,
                               int32_t* topk_ids_out, float* topk_w_out, const moe_dispatch_t* disp, void* stream) {
    int st = check_desc(d);
    if (st) return st;
    if ((int64_t)d->max_tokens * (d->top_k + 1) > kScratchRows) return MOE_ERR_SCRATCH;
    char* base = nullptr;
    if ((st = scratch_on_device((hipStream_t)stream, &base))) return st;
    Params p;
    if ((st = fill_params(p, d, M, x, w_router, base, scratch_layout()))) return st;
    if ((st = fill_forward(p, d, w, req_offsets, R, y, topk_ids_out, topk_w_out, disp))) return st;
    return plan_and_launch(p, (hipStream_t)stream);
}

int moe_read_status(void* ws, void* stream, int32_t* status) {
    if (!ws || !status) return MOE_ERR_NULL;
    uint32_t v = 0;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_ERR_HIP;
    if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
    const uint32_t zero = 0;
    if (hipMemcpy(ws, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return MOE_ERR_HIP;
    *status = (v & moe::kStatusTimeout) ? MOE_ERR_TIMEOUT : ((v & moe::kStatusOffsets) ? MOE_ERR_OFFSETS : MOE_OK);
    return MOE_OK;
}

const char* moe_status_string(int status) {
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or not a supported multiple";
    case MOE_ERR_FORMAT: return "unsupported format or format pair";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_OFFSETS: return "request offsets out of range or not monotone from 0 to M";
    case MOE_ERR_HIP: return "a HIP runtime call failed";
    case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOE_ERR_SCRATCH: return "the description needs more than the fixed scratch of moe_decode_forward_noalloc (max_tokens * (top_k + 1) > 144 pair rows); use moe_decode_forward with a workspace";
    case MOE_ERR_TIMEOUT: return "a cross-workgroup wait timed out; that call's y was written as NaN";
    default: return "unknown status";
    }
}

}  // extern "C"
