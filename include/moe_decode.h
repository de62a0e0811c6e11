/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) routed-expert MoE decode layer.
 *
 * The operation is one MoE layer of Ling-3.0-flash at decode: M tokens (1 for plain batch-1
 * decode, or a packed speculative-verify window of several tokens) go through a router gate,
 * softmax top-k routing with renormalised weights, SwiGLU routed experts and one shared expert,
 * and a weighted combine.
 *   - shapes: hidden 2,560, eight of 512 routed experts plus one shared expert per token
 *     ("3 ways to boost MoE inference on NVIDIA DGX Spark", section "Model and baseline
 *     configuration"); moe_intermediate_size 768 ("Chasing the Batch-1 Floor: Ling-3.0-flash
 *     Speculative Decode on Blackwell", section "Where the time goes now");
 *   - router chain norm -> gate matvec -> top-k, gate weight in bf16 with fp32 accumulation
 *     (same page, sections "PDL: stacking the latency floors of small kernels" and
 *     "bf16 router gate and lm_head");
 *   - silu(gate) * up computed in float and rounded once (same page, "Two fusions and a retune");
 *   - the combine is one fp32 sum of weight x expert output with a single final cast (same page,
 *     PDL section);
 *   - a packed ragged verify batch described by cu_seqlens-style offsets ("DSpark in SGLang",
 *     section "Ragged verify under full CUDA graphs");
 *   - MXFP4 expert weights ("3 ways to boost MoE inference on NVIDIA DGX Spark", "Optimization 1"),
 *     laid out per the OCP Microscaling v1.0 format: E2M1 codes, two per byte with element 2i in
 *     the low nibble, and one E8M0 scale byte per 32 consecutive elements along K.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller; pointers are borrowed only until
 *     the enqueued work finishes.  Struct arguments (moe_desc_t, moe_weights_t, moe_dispatch_t)
 *     are host memory, read during the call and not retained.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls only enqueue
 *     work on it: they never synchronise, never allocate, never read device memory on the host,
 *     and can be captured into a hipGraph.
 *   - Arguments are validated on the host before anything is enqueued; a call that returns a
 *     negative status has enqueued nothing.  MOE_ERR_HIP reports a failed launch.  Faults inside
 *     the kernels surface at the caller's next synchronisation, as for any HIP kernel.
 *   - The workspace `ws` (size from moe_workspace_bytes) must be zero-filled once before its first
 *     use and stays bound to one device; the calls keep its counters consistent from then on.
 *   - At most ONE moe_route / moe_decode_forward may be in flight per device at any time, whatever
 *     the workspaces: a call runs one workgroup on every compute unit and its workgroups wait on
 *     each other, so two calls running at once could each hold part of the GPU and wait on the
 *     other.  Order the calls (one stream, or events between streams).
 *   - A wait between workgroups that gives up (bounded at about a second; it happens only if the
 *     rule above is broken) never leaves output that looks valid: the call's y elements, and the
 *     routing weights of a token whose routing was cut short, are written as NaN, and the
 *     workspace status word records MOE_ERR_TIMEOUT (see moe_read_status).
 *   - The library's only host state is a per-device cache of device properties and kernel set-up,
 *     filled on first use; it is safe to call from several host threads.
 *   - Matrices are row-major [out][in] with the input dimension K contiguous (nn.Linear layout).
 *     Every pointer must be 16-byte aligned.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element storage formats. */
typedef enum {
    MOE_FMT_F32 = 0,   /* IEEE binary32 */
    MOE_FMT_BF16 = 1,  /* bfloat16 */
    MOE_FMT_MXFP4 = 2, /* OCP MX v1.0 FP4 (E2M1) codes + E8M0 scale per 32 elements of K */
    MOE_FMT_FP8 = 3    /* OCP FP8 E4M3 codes, one per byte, + one binary32 scale per block of
                          128 rows x 128 columns ("Chasing the Batch-1 Floor", section "Where the
                          time goes now": fp8 expert weights with block 128) */
} moe_format_t;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,      /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,     /* a size is out of range or not a supported multiple */
    MOE_ERR_FORMAT = -3,    /* unsupported format or format pair */
    MOE_ERR_WORKSPACE = -4, /* ws_bytes smaller than moe_workspace_bytes(desc) */
    MOE_ERR_OFFSETS = -5,   /* R out of range (host); or, in the device status word, offsets that
                               are not 0 = o[0] <= o[1] <= ... <= o[R] = M */
    MOE_ERR_HIP = -6,       /* a HIP runtime call failed */
    MOE_ERR_ALIGN = -7,     /* a pointer is not 16-byte aligned */
    MOE_ERR_TIMEOUT = -8,   /* device status only: a cross-workgroup wait gave up; that call's y
                               was written as NaN (happens only if calls overlap on one device) */
    MOE_ERR_SCRATCH = -9    /* moe_decode_forward_noalloc: the description needs more than its fixed
                               scratch (max_tokens * (top_k + 1) > 144 pair rows) */
} moe_status_t;

/* Largest supported values (checked on the host). */
#define MOE_MAX_TOKENS 16      /* tokens per call (M) */
#define MOE_MAX_EXPERTS 512    /* routed experts (E) */
#define MOE_MAX_TOPK 16        /* experts per token (k) */
#define MOE_MAX_HIDDEN 2560    /* H, bf16 and MXFP4 weights */
#define MOE_MAX_INTER 768      /* I and Is, bf16 and MXFP4 weights */
#define MOE_MAX_HIDDEN_F32 256 /* H, binary32 layer */
#define MOE_MAX_INTER_F32 256  /* I and Is, binary32 layer */

/* Layer description.  H, I, Is multiples of 8 (of 32 for MXFP4, of 128 for FP8), within the maxima
   above (FP8 and MXFP4 use the bf16 maxima);
   1 <= k <= min(E, 16); E <= 512; 1 <= max_tokens <= 16.  A call whose shape leaves no room for the
   kernel's on-chip (LDS) layout at the given M is rejected with MOE_ERR_SHAPE before anything is
   enqueued (for example k = 16 with 16 tokens of Ling width). */
typedef struct {
    int32_t hidden;        /* H */
    int32_t num_experts;   /* E */
    int32_t top_k;         /* k */
    int32_t inter;         /* I, routed expert intermediate size */
    int32_t shared_inter;  /* Is, shared expert intermediate size; 0 = no shared expert */
    int32_t max_tokens;    /* largest M the workspace is sized for */
    int32_t act_format;    /* x, router weight and y: MOE_FMT_BF16, or MOE_FMT_F32 with F32 weights */
    int32_t weight_format; /* routed and shared expert weights: F32 (with F32 act), BF16, MXFP4 or FP8 */
    /* The router chain's optional steps either side of the gate matvec ("Chasing the Batch-1
       Floor", section "PDL: stacking the latency floors of small kernels": norm -> gate matvec ->
       top-k, the top-k with a bias).  All zero (the default of a zero-filled struct): neither. */
    int32_t router_flags;  /* MOE_ROUTER_NORM | MOE_ROUTER_BIAS */
    float norm_eps;        /* MOE_ROUTER_NORM: the epsilon (> 0 recommended, e.g. 1e-6) */
    const void* norm_weight;  /* MOE_ROUTER_NORM: gain g [H], device memory, activation format */
    const float* router_bias; /* MOE_ROUTER_BIAS: selection bias b [E], device memory, binary32 */
} moe_desc_t;

/* router_flags.
   MOE_ROUTER_NORM: every token row is RMSNorm'd first, xn = bf16(g * (x / sqrt(mean(x^2) + eps)))
     (mean over the H elements, fp32 arithmetic, rounded once to bfloat16), and xn replaces x for
     the router and for every expert: y = MoE(RMSNorm(x)).  bfloat16 activations only
     (MOE_ERR_FORMAT otherwise).
   MOE_ROUTER_BIAS: the k experts kept per token are those with the largest l_e + b_e (ties: lower
     id); their weights are still the softmax of the logits l over the kept experts, and topk_ids /
     topk_w list them by descending weight (ties: lower id). */
#define MOE_ROUTER_NORM 1
#define MOE_ROUTER_BIAS 2

/* Expert weights.  Routed stacks are expert-major: gate, up [E][I][H]; down [E][H][I].
   Shared expert: sh_gate, sh_up [Is][H]; sh_down [H][Is].  For MXFP4 the data pointers hold the
   packed codes (K/2 bytes per row) and the *_s pointers the scales ([rows][K/32] bytes).  For FP8
   the data pointers hold one E4M3 code per element ([rows][K] bytes) and the *_s pointers binary32
   scales [rows/128][K/128] per matrix (expert-major like the codes): element (r, c) is
   E4M3(code) * scale[r/128][c/128].  The *_s pointers are ignored (may be NULL) for bf16 and f32. */
typedef struct {
    const void *gate, *up, *down;
    const uint8_t *gate_s, *up_s, *down_s;
    const void *sh_gate, *sh_up, *sh_down;
    const uint8_t *sh_gate_s, *sh_up_s, *sh_down_s;
} moe_weights_t;

/* Optional device outputs describing the dispatch of a call (each member nullable).
   Units are the distinct routed experts of the batch in ascending id order, then the shared
   expert (id reported as E).  Pair rows are the (token, slot) pairs grouped by unit, ascending
   token inside a unit; the shared unit's rows hold every token with slot k and weight 1.
   ("Chasing the Batch-1 Floor", "Two fusions and a retune": stable per-expert order, 512 routed
   + 1 shared dispatch axis.)  Sizes for U distinct experts: */
typedef struct {
    int32_t* unit_count;  /* [1]   U */
    int32_t* unit_expert; /* [U+1] (allocate min(M*k, E) + 1) */
    int32_t* unit_off;    /* [U+2] unit u owns rows [unit_off[u], unit_off[u+1]) (alloc min(M*k,E)+2) */
    int32_t* row_token;   /* [M*k+M] */
    int32_t* row_slot;    /* [M*k+M] */
    float* row_weight;    /* [M*k+M] routing weight of the row */
    int32_t* req_unique;  /* [R] distinct routed experts per request; needs req_offsets */
} moe_dispatch_t;

/* Workspace size in bytes for this description, or 0 when the description is invalid. */
size_t moe_workspace_bytes(const moe_desc_t* d);

/* Router only ("Chasing the Batch-1 Floor", section "PDL: stacking the latency floors of small
   kernels": the router chain gate matvec -> top-k; section "bf16 router gate and lm_head": bf16 gate
   weight, fp32 accumulation; "3 ways to boost MoE inference on NVIDIA DGX Spark", "Model and
   baseline configuration": eight of 512 routed experts per token).
   logits = x [M][H] . w_router [E][H]^T with fp32 accumulation, then per token the k
   largest logits (ties: lower expert id) and weights softmax-renormalised over those k.
   topk_ids [M][k] and topk_w [M][k] receive them in descending weight order.  `disp` (nullable)
   additionally receives the batch dispatch.  Same routing as inside moe_decode_forward. */
int moe_route(const moe_desc_t* d, int32_t M, const void* x, const void* w_router, int32_t* topk_ids,
              float* topk_w, const moe_dispatch_t* disp, void* ws, size_t ws_bytes, void* stream);

/* The whole layer ("Chasing the Batch-1 Floor", section "PDL: stacking the latency floors of small
   kernels": router chain, then align -> up-GEMM -> activation -> down-GEMM -> combine, the combine an
   fp32 sum of weight x expert output with one final cast; section "Two fusions and a retune":
   silu(gate) * up in float, 512 routed + 1 shared experts on the dispatch axis; "DSpark in SGLang",
   "Ragged verify under full CUDA graphs": a packed ragged verify batch with cu_seqlens offsets).
   y [M][H] = sum_j w[m,j] * expert_{id[m,j]}(x_m) + shared(x_m), where
   expert(x) = Wd (silu(Wg x) * (Wu x)).  Each distinct selected expert's weights are read from
   memory once per call, however many of the M tokens chose it.
   req_offsets: device int32 [R+1] packed-request offsets (0 = o[0] <= ... <= o[R] = M, requests may
   be empty, 1 <= R <= MOE_MAX_TOKENS) or NULL (then R is ignored).  They do not change y; they feed disp->req_unique and are checked on the
   device (a violation sets MOE_ERR_OFFSETS in the status word, see moe_read_status).
   topk_ids_out, topk_w_out, disp: nullable extra outputs as in moe_route. */
int moe_decode_forward(const moe_desc_t* d, int32_t M, const void* x, const void* w_router,
                       const moe_weights_t* w, const int32_t* req_offsets, int32_t R, void* y,
                       int32_t* topk_ids_out, float* topk_w_out, const moe_dispatch_t* disp, void* ws,
                       size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under hipGraph capture, tight serving loops,
   harnesses that forbid hipMalloc): moe_decode_forward without a workspace argument.  The library's
   own per-device scratch of MOE_NOALLOC_SCRATCH_BYTES (a static device array, held by every GPU the
   library runs on until the process ends) takes the workspace's place, so nothing is allocated by
   this call or by the library.  It serves descriptions with max_tokens * (top_k + 1) <= 144 pair
   rows (every Ling-shaped workload up to 16 tokens at top-8); larger ones return MOE_ERR_SCRATCH
   before anything is enqueued.  The first call on a device also enqueues, on `stream`, a clear of
   the scratch's counters.  All calls on one GPU share its scratch and its state carries over from
   call to call, so these calls must not overlap on one device (the same rule as for every call of
   this library); overlapping calls race.  Arguments, outputs and results are those of
   moe_decode_forward; the device status word of the scratch is not readable by the caller (a wait
   that gives up still writes y as NaN). */
#define MOE_NOALLOC_SCRATCH_BYTES 2138112
int moe_decode_forward_noalloc(const moe_desc_t* d, int32_t M, const void* x, const void* w_router,
                               const moe_weights_t* w, const int32_t* req_offsets, int32_t R, void* y,
                               int32_t* topk_ids_out, float* topk_w_out, const moe_dispatch_t* disp,
                               void* stream);

/* ---- The LM head --------------------------------------------------------------------------
   The vocabulary projection of the decode step ("3 ways to boost MoE inference on NVIDIA DGX
   Spark", "Model and baseline configuration": hidden 2,560 onto a vocabulary of 157,184;
   "Optimization 2: Online FP8 LM head quantization": FP8 weights halve the read of this GEMM;
   "Chasing the Batch-1 Floor", "bf16 router gate and lm_head": bf16 weights, fp32 accumulation,
   a pure bandwidth cost at batch 1). */
typedef struct {
    int32_t hidden;        /* H: multiple of 8 (bf16) or 16 (FP8), at most 2560 */
    int32_t vocab;         /* V: rows of the weight, >= 1 */
    int32_t weight_format; /* MOE_FMT_BF16, or MOE_FMT_FP8: E4M3 codes with one binary32 scale per row */
} moe_lm_head_desc_t;

/* logits [M][V] (binary32) = x [M][H] (bf16) . W [V][H]^T, fp32 accumulation; with FP8 weights row v
   is E4M3(code) * w_scale[v] (w_scale: device binary32 [V], NULL for bf16).  1 <= M <= 16.  Device
   pointers x, w, logits 16-byte aligned (w_scale 4-byte).  Asynchronous on `stream`, allocates
   nothing, uses no workspace and no cross-workgroup waits (so it may run beside other work);
   graph capturable.  Host-side validation as for the layer; a shape whose logit staging does not
   fit on chip (very large V) returns MOE_ERR_SHAPE. */
int moe_lm_head(const moe_lm_head_desc_t* d, int32_t M, const void* x, const void* w, const float* w_scale,
                float* logits, void* stream);

/* Debug helper, NOT for the hot path: synchronises `stream`, copies the workspace's device status
   word to *status (MOE_OK, MOE_ERR_OFFSETS or MOE_ERR_TIMEOUT, accumulated over the calls since the
   last read), then clears it. */
int moe_read_status(void* ws, void* stream, int32_t* status);

/* Static description of a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
