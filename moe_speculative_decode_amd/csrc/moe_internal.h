// Internal interface between the C ABI (moe_api.hip) and the kernel (moe_layer.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_decode.h"

namespace moe {

constexpr int kMaxTokens = MOE_MAX_TOKENS;
constexpr int kMaxExperts = MOE_MAX_EXPERTS;
constexpr int kMaxTopK = MOE_MAX_TOPK;
constexpr int kWaves = 8;                 // waves per workgroup; one workgroup per CU
constexpr int kThreads = 64 * kWaves;     // 512
constexpr int kMaxGrid = 1024;            // workgroups (CUs) the counter sets are sized for
constexpr int kLdsBytes = 160 * 1024;     // LDS of one CU (gfx950)

// Cross-workgroup counters.  Each counter owns a 256-byte line (atomics on one line serialise).
// Two sets alternate between consecutive calls: call c counts in set c & 1 and clears set
// (c + 1) & 1, which the previous call used and the next call will use.
constexpr int kLineWords = 64;
constexpr int kLineShared = 0;                            // shared-expert SwiGLU rows finished
constexpr int kRoutedStripes = 8;                         // routed-row counter lines (atomics spread)
constexpr int kLineRouted = 1;                            // [kRoutedStripes] routed SwiGLU rows finished
constexpr int kMaxPools = kMaxGrid / 8;                   // work pools: one per 8 workgroups
constexpr int kLinePoolC0 = kLineRouted + kRoutedStripes; // [kMaxPools] gate/up chunks handed out
constexpr int kLinePoolD0 = kLinePoolC0 + kMaxPools;      // [kMaxPools] down chunks handed out
constexpr int kLineDownDone = kLinePoolD0 + kMaxPools;    // workgroups whose down partials have landed
constexpr int kLineFault = kLineDownDone + 1;             // nonzero: a wait of this call gave up
constexpr int kSetLines = kLineFault + 1;
constexpr int kSetWords = kSetLines * kLineWords;

// Workspace header.  Word 0 is the status word (OR of status bits, cleared by moe_read_status).
// The call index is counted per workgroup: workgroup b reads its own counter at word
// kHdrCall + kCallStride * b and stores it plus one.  No other workgroup touches that word and the
// next call reads it only after this kernel has ended, so every workgroup of a call takes the same
// index (each has been launched once per call) and no read can race an advance.
constexpr int kHdrStatus = 0;
constexpr int kHdrSpin = 1;  // test hook: nonzero = polls before a wait gives up (0: the default, ~1 s)
constexpr int kHdrCall = kLineWords;
constexpr int kCallStride = 4;  // words between two workgroups' counters
constexpr int kHdrBytes = 4 * (kHdrCall + kCallStride * kMaxGrid);

// status bits set by the kernel
constexpr uint32_t kStatusOffsets = 1u;
constexpr uint32_t kStatusTimeout = 2u;

struct Workspace {
    uint32_t* hdr;    // [kHdrBytes / 4]
    uint32_t* ctr;    // [2][kSetWords]
    uint64_t* logits; // [max_tokens][E] (rows padded to 4): fp32 logit bits | (call index + 1) << 32
    uint64_t* route;  // [max_tokens * k][2]: expert id, fp32 weight bits, each | (call index + 1) << 32
    float* act;       // [max_tokens * (k + 1)][act_stride]  SwiGLU output per pair row
    float* part;      // [max_tokens * (k + 1)][H]           down projection per pair row
};

struct Params {
    int H, E, k, I, Is, M;
    int act_fmt, w_fmt;
    int act_stride;   // row stride (elements) of Workspace::act = max(I, Is)
    int route_only;   // 1: routing outputs only (moe_route)
    int route_delegate;  // 1: workgroup m selects token m's experts and publishes them
    // LDS layout, byte offsets from the dynamic LDS base (filled by launch_layer)
    int lds_tab, lds_x, lds_cst, lds_sh, lds_ysh, lds_dn, lds_total;
    int lds_tr;       // matrix-core gate/up: kWaves transpose buffers of 4 KB
    int lds_sel;      // routing scratch (the head of the slice-mode down window while it is empty, else cst)
    int cst_bytes;    // staging area (SwiGLU results, down partials; the routing scratch unless lds_sel is elsewhere)
    int dn_bytes;     // slice mode: routed down-row window
    int slice_mode;   // 1: every workgroup computes its y slice of every routed unit (small M*k)
    int slice_mfma;   // 1: slice mode on the matrix cores (bfloat16 SwiGLU rows, swizzled windows)
    int sh_mfma;      // 1: the shared expert's down rows on the matrix cores (swizzled window)
    int gu_mfma;      // 1: routed gate/up rows on the matrix cores (MXFP4, FP8 from 3 tokens)
    int gu_cap;       // gate/up tasks one wave may stage (static share plus the chunks it takes)
    int xpitch;       // bytes between consecutive token rows staged in LDS (padded)
    int cost_dn;      // per-token cost of a down row relative to its weight bytes (8 units): work
                      // is split so that high-token units get more CUs
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
    int lds_scl;         // MXFP4: LDS scale window of the shared expert's slice rows at this offset,
    int scl_sh;          // of this size in bytes (0: none)
    int gu_ksplit;       // MXFP4 slice mode: (tile, stage) items with partials in the staging area
    int gu_items;        // MXFP4 slice mode: the whole-item matrix-core gate/up (else the line form)
    int gu_part;         // matrix-core gate/up: float offset of the partials in the staging area (-1: none)
    int router_flags;    // MOE_ROUTER_NORM | MOE_ROUTER_BIAS
    float norm_eps;
    const void* norm_w;  // [H] activation format
    const float* rbias;  // [E] binary32
};

// Fills the launch plan of p (modes, LDS layout) for a grid of G workgroups.  Returns
// hipErrorInvalidValue when the shape does not fit (LDS); nothing is launched then.
hipError_t plan_layer(Params& p, int G);

// Enqueues one call planned by plan_layer with the same G.
hipError_t launch_layer(const Params& p, int G, hipStream_t stream);

}  // namespace moe
