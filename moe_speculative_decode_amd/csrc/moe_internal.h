// Internal interface between the C ABI (moe_api.hip) and the kernels (moe_layer.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_decode.h"

namespace moe {

constexpr int kMaxTokens = MOE_MAX_TOKENS;
constexpr int kMaxExperts = MOE_MAX_EXPERTS;
constexpr int kMaxTopK = MOE_MAX_TOPK;
constexpr int kThreads = 256;       // threads per workgroup of every kernel (4 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kCombineTile = 64;    // rows of y finished together by the last contributing workgroup

// status bits OR-ed into the workspace status word by the kernels
constexpr uint32_t kStatusOffsets = 1u;

// Device-side views of the caller's workspace.  All counters are zero between calls.
struct Workspace {
    uint32_t* status;     // [1]
    uint32_t* route_cnt;  // [1]   router workgroups finished
    uint32_t* tile_cnt;   // [ceil(H / kCombineTile)] down-projection rows finished per y tile
    float* logits;        // [max_tokens][E]
    // dispatch tables (written by the router's last workgroup)
    int32_t* n_units;     // [1]   U (routed units; the shared unit, if any, follows them)
    int32_t* unit_expert; // [E + 1]
    uint32_t* unit_mask;  // [E + 1] token bitmask of the unit
    int32_t* unit_off;    // [E + 2] first pair row of the unit
    int32_t* pair_row;    // [max_tokens][k] pair row of (token, slot)
    float* row_w;         // [max_tokens * (k + 1)] routing weight of a pair row
    float* act;           // [max_tokens * (k + 1)][max(I, Is)] SwiGLU outputs per pair row (fp32)
    float* part;          // [max_tokens * (k + 1)][H] down-projection outputs per pair row (fp32)
};

struct Params {
    int H, E, k, I, Is, M;
    int act_fmt, w_fmt;
    int act_stride;       // row stride (elements) of Workspace::act
    const void* x;
    const void* wr;
    moe_weights_t w;
    const int32_t* req_off;
    int R;
    void* y;
    int32_t* topk_ids;
    float* topk_w;
    moe_dispatch_t disp;
    Workspace ws;
};

// Launch sequence (implemented in moe_layer.hip).  `route_only` stops after routing.
hipError_t launch_layer(const Params& p, bool route_only, int num_cus, hipStream_t stream);

}  // namespace moe
