/*
 * moe_oracle.c -- plain, slow, fp64 CPU oracle of the routed-expert MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only the test suite,
 * the package's smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or constant with the HIP library, and includes nothing from it.
 *
 * What it computes, per token, in the order the definition states it (every input is first
 * widened exactly to double; no blocking, fusion or reordering beyond that):
 *   0. optional RMSNorm prologue (the first link of the router chain norm -> gate matvec -> top-k,
 *      "Chasing the Batch-1 Floor", section "PDL: stacking the latency floors of small kernels"):
 *      r = 1 / sqrt(mean_h x[h]^2 + eps), xn[h] = bf16(g[h] * (x[h] * r)), the normed activation
 *      rounded once to the activation format (bfloat16) as a norm kernel of a bf16 model writes it;
 *      xn then replaces x for the router and for every expert
 *   1. router logits  l_e = sum_h x[h] * Wr[e,h], summed in ascending h
 *      ("Chasing the Batch-1 Floor", sections "PDL: stacking the latency floors of small kernels"
 *       and "bf16 router gate and lm_head": router chain norm -> gate matvec -> top-k, bf16 gate)
 *   2. p = softmax(l) over all E experts, keep the k largest (ties: lower expert id first),
 *      renormalise the kept probabilities to sum to 1.  With the bias-corrected selection (the
 *      page's "the router top-k prefetches its bias"), the kept experts are instead the k largest
 *      keys l_e + b_e (ties: lower id), while their weights are still p renormalised over them;
 *      the kept experts are reported in descending weight order (ties: lower id)
 *      ("3 ways to boost MoE inference on NVIDIA DGX Spark", "Model and baseline configuration":
 *       each token goes to eight of 512 routed experts plus one shared expert)
 *   3. for each kept expert: g = Wg x, v = Wu x, a = silu(g) * v with silu(z) = z / (1 + exp(-z)),
 *      o = Wd a   ("Chasing the Batch-1 Floor", "Two fusions and a retune": silu(gate) * up,
 *      kept in float before the multiply)
 *   4. the shared expert the same way, unweighted
 *   5. y = sum_j w_j o_j + o_shared, one sum, no intermediate rounding
 *      ("Chasing the Batch-1 Floor", PDL section: fp32 sum x scale with a single final cast;
 *       here the whole sum is exact-as-fp64 and never rounded)
 *
 * Storage formats it decodes (each from its published definition, see the decode functions):
 *   fmt 0 = IEEE binary32, fmt 1 = bfloat16 (upper half of a binary32), fmt 2 = MXFP4
 *   (OCP Microscaling v1.0: E2M1 element codes, two per byte with element 2i in the low nibble,
 *   one E8M0 scale byte per 32 consecutive elements along the input dimension K), fmt 3 = FP8
 *   block-quantised weights (OCP 8-bit floating point E4M3 codes, one per byte, times one binary32
 *   scale per block of 128 rows x 128 columns: "Chasing the Batch-1 Floor", section "Where the
 *   time goes now": fp8 weights with block 128, which with moe_intermediate_size 768 rules out a
 *   four-way split of the intermediate dimension, so the blocks span 128 along both dimensions).
 *
 * Batch-level dispatch (oracle_compact): the unique selected experts across all M tokens in
 * ascending id order, each with its (token, slot, weight) list stable in pair index m*k+j, and
 * the shared expert appended as the last unit holding every token with weight 1.
 * ("Chasing the Batch-1 Floor", "Two fusions and a retune": the pair-axis alignment orders pairs
 *  stably inside each expert bucket; the dispatch axis is 512 routed + 1 shared.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OF_F32 = 0, OF_BF16 = 1, OF_MXFP4 = 2, OF_FP8 = 3 };
enum { FP8_BLOCK = 128 };

/* ---- element decoders ------------------------------------------------------------------ */

/* binary32 bits -> double (exact widening). */
static double dec_f32(uint32_t bits) {
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* bfloat16 = the high 16 bits of a binary32 with the low 16 bits zero. */
double oracle_bf16_to_f64(uint16_t b) { return dec_f32((uint32_t)b << 16); }

/* E2M1 (OCP MX v1.0): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
   exponent field 0 is subnormal: 0.m * 2^(1-1); otherwise 1.m * 2^(e-1). */
double oracle_e2m1_to_f64(uint8_t code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E8M0 (OCP MX v1.0): an unsigned biased exponent, value 2^(S-127); S = 255 is NaN. */
double oracle_e8m0_to_f64(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* E4M3 (OCP 8-bit floating point, E4M3): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
   no infinities; exponent and mantissa all ones is NaN.  Exponent field 0 is subnormal:
   0.m * 2^(1-7); otherwise 1.m * 2^(e-7).  The largest finite magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3_to_f64(uint8_t code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* The bfloat16 value nearest to v (ties: the even significand), as a double: bfloat16 keeps 8
   significant bits, its normal exponents run from -126 to 127 and below 2^-126 its spacing stays
   2^-133 (subnormals).  Values beyond the largest finite bfloat16 round to infinity. */
double oracle_round_bf16(double v) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    int e;
    frexp(fabs(v), &e); /* |v| = f * 2^e, f in [0.5, 1): the leading bit has weight 2^(e-1) */
    int lead = e - 1;
    if (lead < -126) lead = -126;
    const double ulp = ldexp(1.0, lead - 7);
    double q = v / ulp; /* exact: a power-of-two scale */
    double fl = floor(q), r = q - fl;
    double n = (r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0)) ? fl + 1.0 : fl;
    double out = n * ulp;
    if (fabs(out) >= ldexp(2.0 - ldexp(1.0, -8), 127)) return v > 0 ? INFINITY : -INFINITY;
    return out;
}

/* RMSNorm of one activation row: xn[h] = bf16(g[h] * (x[h] * r)), r = 1 / sqrt(mean(x^2) + eps),
   the mean summed in ascending h. */
static void rms_norm(const double* x, const double* g, int H, double eps, double* xn) {
    double ss = 0.0;
    for (int h = 0; h < H; ++h) ss += x[h] * x[h];
    const double r = 1.0 / sqrt(ss / H + eps);
    for (int h = 0; h < H; ++h) xn[h] = oracle_round_bf16(g[h] * (x[h] * r));
}

/* A row-major [rows][cols] matrix in one of the storage formats. */
typedef struct {
    int fmt;
    const void* data;      /* f32 / bf16 elements, MXFP4 packed codes [rows][cols/2], FP8 codes [rows][cols] */
    const uint8_t* scales; /* MXFP4: E8M0 bytes [rows][cols/32]; FP8: binary32 [rows/128][cols/128] */
    int64_t rows, cols;
} omat;

static double mat_at(const omat* A, int64_t r, int64_t c) {
    switch (A->fmt) {
    case OF_F32: return dec_f32(((const uint32_t*)A->data)[r * A->cols + c]);
    case OF_BF16: return oracle_bf16_to_f64(((const uint16_t*)A->data)[r * A->cols + c]);
    case OF_FP8: {
        const uint8_t code = ((const uint8_t*)A->data)[r * A->cols + c];
        uint32_t sbits;
        memcpy(&sbits, A->scales + 4 * ((r / FP8_BLOCK) * (A->cols / FP8_BLOCK) + c / FP8_BLOCK), 4);
        return oracle_e4m3_to_f64(code) * dec_f32(sbits);
    }
    default: {
        uint8_t byte = ((const uint8_t*)A->data)[r * (A->cols / 2) + c / 2];
        uint8_t code = (c & 1) ? (byte >> 4) : (byte & 15);
        return oracle_e2m1_to_f64(code) * oracle_e8m0_to_f64(A->scales[r * (A->cols / 32) + c / 32]);
    }
    }
}

/* y[r] = sum_c A[r,c] * v[c], c ascending. */
static void matvec(const omat* A, const double* v, double* y) {
    for (int64_t r = 0; r < A->rows; ++r) {
        double s = 0.0;
        for (int64_t c = 0; c < A->cols; ++c) s += mat_at(A, r, c) * v[c];
        y[r] = s;
    }
}

/* Matrix of expert e inside an expert-major stack [E][rows][cols]. */
static omat expert_mat(int fmt, const void* data, const uint8_t* scales, int64_t e, int64_t rows, int64_t cols) {
    omat A;
    A.fmt = fmt;
    A.rows = rows;
    A.cols = cols;
    if (fmt == OF_MXFP4) {
        A.data = (const uint8_t*)data + e * rows * (cols / 2);
        A.scales = scales + e * rows * (cols / 32);
    } else if (fmt == OF_FP8) {
        A.data = (const uint8_t*)data + e * rows * cols;
        A.scales = scales + 4 * e * (rows / FP8_BLOCK) * (cols / FP8_BLOCK);
    } else {
        A.data = (const uint8_t*)data + e * rows * cols * (fmt == OF_F32 ? 4 : 2);
        A.scales = NULL;
    }
    return A;
}

/* ---- layer description ------------------------------------------------------------------ */

typedef struct {
    int32_t hidden, num_experts, top_k, inter, shared_inter; /* H, E, k, I, Is (Is = 0: none) */
    int32_t act_fmt;    /* x and Wr: OF_F32 or OF_BF16 */
    int32_t weight_fmt; /* routed + shared expert weights: OF_F32, OF_BF16 or OF_MXFP4 */
    int32_t router_flags; /* ORACLE_NORM: RMSNorm prologue; ORACLE_BIAS: bias-corrected selection */
    double norm_eps;      /* the RMSNorm epsilon */
} oracle_desc;

enum { ORACLE_NORM = 1, ORACLE_BIAS = 2 };

/* The router's optional tensors (either may be NULL when its flag is off). */
typedef struct {
    const void* norm_w; /* [H] in the activation format: the RMSNorm gain g */
    const float* bias;  /* [E] binary32: the selection bias b */
} oracle_router_aux;

typedef struct {
    const void *gate, *up, *down;          /* [E][I][H], [E][I][H], [E][H][I] */
    const uint8_t *gate_s, *up_s, *down_s; /* MXFP4 scales, NULL otherwise */
    const void *sh_gate, *sh_up, *sh_down; /* [Is][H], [Is][H], [H][Is] */
    const uint8_t *sh_gate_s, *sh_up_s, *sh_down_s;
} oracle_weights;

/* ---- step 1 + 2: routing of one token --------------------------------------------------- */

typedef struct {
    double v;
    int32_t id;
} keyed;

/* sort order: larger value first, equal values -> lower id first */
static int cmp_desc(const void* a, const void* b) {
    const keyed* x = (const keyed*)a;
    const keyed* y = (const keyed*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

/* Routes one token.  logits[E] out (may be NULL); ids[k], w[k] out in descending-weight order
   (ties: lower id); *gap out = the k-th largest selection key minus the (k+1)-th (+inf when k == E).
   The selection key of expert e is l_e, or l_e + bias[e] with the bias-corrected selection. */
static void route_token(const oracle_desc* d, const double* x, const omat* Wr, const float* bias,
                        double* logits_out, int32_t* ids, double* w, double* gap) {
    const int E = d->num_experts, k = d->top_k;
    const int biased = (d->router_flags & ORACLE_BIAS) != 0;
    double* l = (double*)malloc(sizeof(double) * E);
    double* p = (double*)malloc(sizeof(double) * E);
    keyed* key = (keyed*)malloc(sizeof(keyed) * E);
    keyed* kept = (keyed*)malloc(sizeof(keyed) * k);
    matvec(Wr, x, l); /* step 1 */
    /* step 2: softmax over all E, stabilised by the max logit */
    double lmax = l[0];
    for (int e = 1; e < E; ++e) lmax = l[e] > lmax ? l[e] : lmax;
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += exp(l[e] - lmax);
    for (int e = 0; e < E; ++e) {
        p[e] = exp(l[e] - lmax) / z;
        key[e].v = biased ? l[e] + (double)bias[e] : l[e]; /* the selection key */
        key[e].id = e;
    }
    qsort(key, E, sizeof(keyed), cmp_desc); /* the k largest keys, ties: lower id */
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += p[key[j].id];
    for (int j = 0; j < k; ++j) {
        kept[j].id = key[j].id;
        kept[j].v = p[key[j].id] / sum; /* renormalise over the kept experts */
    }
    qsort(kept, k, sizeof(keyed), cmp_desc); /* reported by descending weight, ties: lower id */
    for (int j = 0; j < k; ++j) {
        ids[j] = kept[j].id;
        w[j] = kept[j].v;
    }
    *gap = (k < E) ? key[k - 1].v - key[k].v : INFINITY;
    if (logits_out) memcpy(logits_out, l, sizeof(double) * E);
    free(l);
    free(p);
    free(key);
    free(kept);
}

/* ---- step 3 + 4: one SwiGLU expert on one token ----------------------------------------- */

static void swiglu_expert(const omat* Wg, const omat* Wu, const omat* Wd, const double* x, double* o) {
    const int64_t I = Wg->rows;
    double* g = (double*)malloc(sizeof(double) * I);
    double* v = (double*)malloc(sizeof(double) * I);
    double* a = (double*)malloc(sizeof(double) * I);
    matvec(Wg, x, g);
    matvec(Wu, x, v);
    for (int64_t r = 0; r < I; ++r) a[r] = g[r] / (1.0 + exp(-g[r])) * v[r];
    matvec(Wd, a, o);
    free(g);
    free(v);
    free(a);
}

static void load_row(int fmt, const void* base, int64_t m, int64_t n, double* out) {
    omat X = {fmt, base, NULL, 0, n};
    X.rows = m + 1;
    for (int64_t c = 0; c < n; ++c) out[c] = mat_at(&X, m, c);
}

/* ---- public entry points ---------------------------------------------------------------- */

/* The routing input of token m: its activation row, RMSNorm'd when the prologue is on. */
static void token_input(const oracle_desc* d, const oracle_router_aux* aux, const void* x, int64_t m, double* out) {
    const int H = d->hidden;
    load_row(d->act_fmt, x, m, H, out);
    if (d->router_flags & ORACLE_NORM) {
        double* g = (double*)malloc(sizeof(double) * H);
        double* raw = (double*)malloc(sizeof(double) * H);
        load_row(d->act_fmt, aux->norm_w, 0, H, g);
        memcpy(raw, out, sizeof(double) * H);
        rms_norm(raw, g, H, d->norm_eps, out);
        free(g);
        free(raw);
    }
}

/* Routing only (steps 0-2) for M tokens.  x [M][H] and Wr [E][H] in d->act_fmt; aux nullable
   when no router flag is set.  logits [M][E] (nullable), ids [M][k], w [M][k], gap [M]. */
void oracle_route(const oracle_desc* d, int32_t M, const void* x, const void* wr, const oracle_router_aux* aux,
                  double* logits, int32_t* ids, double* w, double* gap) {
    const int H = d->hidden, E = d->num_experts, k = d->top_k;
    omat Wr = {d->act_fmt, wr, NULL, E, H};
    double* xm = (double*)malloc(sizeof(double) * H);
    for (int m = 0; m < M; ++m) {
        token_input(d, aux, x, m, xm);
        route_token(d, xm, &Wr, aux ? aux->bias : NULL, logits ? logits + (int64_t)m * E : NULL,
                    ids + (int64_t)m * k, w + (int64_t)m * k, gap + m);
    }
    free(xm);
}

/* The whole layer (steps 1-5) for M tokens; y [M][H] fp64.  ids/w/gap as in oracle_route
   (nullable).  Work is spread over threads (nthreads <= 0: the OpenMP default) without changing
   any result: the routing of every token first, then each (token, expert) output o_{m,j} on its
   own (j = k: the shared expert), then per token the same sum in the same order,
   y = ((w_0 o_0 + w_1 o_1) + ... + w_{k-1} o_{k-1}) + o_shared. */
void oracle_moe_forward(const oracle_desc* d, const oracle_weights* W, int32_t M, const void* x,
                        const void* wr, const oracle_router_aux* aux, double* y, int32_t* ids_out,
                        double* w_out, double* gap_out, int32_t nthreads) {
    const int H = d->hidden, E = d->num_experts, k = d->top_k, I = d->inter, Is = d->shared_inter;
    const int wf = d->weight_fmt;
    const int units = k + 1; /* per token: k routed experts and the shared one */
    omat Wr = {d->act_fmt, wr, NULL, E, H};
    double* xs = (double*)malloc(sizeof(double) * (size_t)M * H);
    double* ws = (double*)malloc(sizeof(double) * (size_t)M * k);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)M * k);
    double* gaps = (double*)malloc(sizeof(double) * (size_t)M);
    double* o = (double*)malloc(sizeof(double) * (size_t)M * units * H);
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#endif
    /* steps 0-2 per token */
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int m = 0; m < M; ++m) {
        token_input(d, aux, x, m, xs + (int64_t)m * H);
        route_token(d, xs + (int64_t)m * H, &Wr, aux ? aux->bias : NULL, NULL, ids + (int64_t)m * k,
                    ws + (int64_t)m * k, gaps + m);
    }
    /* steps 3-4: every expert output of every token */
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int q = 0; q < M * units; ++q) {
        const int m = q / units, j = q % units;
        const double* xm = xs + (int64_t)m * H;
        double* oq = o + (int64_t)q * H;
        if (j < k) {
            const int32_t e = ids[(int64_t)m * k + j];
            omat Wg = expert_mat(wf, W->gate, W->gate_s, e, I, H);
            omat Wu = expert_mat(wf, W->up, W->up_s, e, I, H);
            omat Wd = expert_mat(wf, W->down, W->down_s, e, H, I);
            swiglu_expert(&Wg, &Wu, &Wd, xm, oq);
        } else if (Is > 0) {
            omat Sg = expert_mat(wf, W->sh_gate, W->sh_gate_s, 0, Is, H);
            omat Su = expert_mat(wf, W->sh_up, W->sh_up_s, 0, Is, H);
            omat Sd = expert_mat(wf, W->sh_down, W->sh_down_s, 0, H, Is);
            swiglu_expert(&Sg, &Su, &Sd, xm, oq);
        }
    }
    /* step 5 per token */
    for (int m = 0; m < M; ++m) {
        double* ym = y + (int64_t)m * H;
        for (int h = 0; h < H; ++h) ym[h] = 0.0;
        for (int j = 0; j < k; ++j) {
            const double wj = ws[(int64_t)m * k + j];
            const double* oj = o + ((int64_t)m * units + j) * H;
            for (int h = 0; h < H; ++h) ym[h] += wj * oj[h];
        }
        if (Is > 0) {
            const double* osh = o + ((int64_t)m * units + k) * H;
            for (int h = 0; h < H; ++h) ym[h] += osh[h];
        }
        if (ids_out)
            for (int j = 0; j < k; ++j) ids_out[(int64_t)m * k + j] = ids[(int64_t)m * k + j];
        if (w_out)
            for (int j = 0; j < k; ++j) w_out[(int64_t)m * k + j] = ws[(int64_t)m * k + j];
        if (gap_out) gap_out[m] = gaps[m];
    }
    free(xs);
    free(ws);
    free(ids);
    free(gaps);
    free(o);
}

/* Dispatch compaction over the (token, slot) pairs of a batch.
   In:  ids [M][k], w [M][k] (w nullable: weights then reported as 0).
   Out: returns U, the number of distinct routed experts;
        unit_expert [U+1]: the distinct ids ascending, then E for the shared unit;
        unit_off [U+2]: unit u owns pair rows [unit_off[u], unit_off[u+1]);
        row_token, row_slot [M*k+M], row_w [M*k+M]: per pair row its token, slot and weight, rows
        of a unit in ascending pair index m*k+j; shared rows use slot k and weight 1.
   A plain counting pass: for every expert id in ascending order, scan all pairs in pair order. */
int32_t oracle_compact(int32_t M, int32_t k, int32_t E, const int32_t* ids, const double* w,
                       int32_t* unit_expert, int32_t* unit_off, int32_t* row_token, int32_t* row_slot,
                       double* row_w) {
    int32_t U = 0, row = 0;
    for (int32_t e = 0; e < E; ++e) {
        int32_t first = 1;
        for (int32_t p = 0; p < M * k; ++p) {
            if (ids[p] != e) continue;
            if (first) {
                unit_expert[U] = e;
                unit_off[U] = row;
                ++U;
                first = 0;
            }
            row_token[row] = p / k;
            row_slot[row] = p % k;
            row_w[row] = w ? w[p] : 0.0;
            ++row;
        }
    }
    unit_expert[U] = E;
    unit_off[U] = row;
    for (int32_t m = 0; m < M; ++m) {
        row_token[row] = m;
        row_slot[row] = k;
        row_w[row] = 1.0;
        ++row;
    }
    unit_off[U + 1] = row;
    return U;
}

/* Decodes a whole [rows][cols] matrix of format fmt into out (row-major fp64). */
void oracle_decode_matrix(int32_t fmt, const void* data, const uint8_t* scales, int64_t rows, int64_t cols,
                          double* out) {
    omat A = {fmt, data, scales, rows, cols};
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = mat_at(&A, r, c);
}

/* ---- the LM head (vocabulary projection) ------------------------------------------------ */

/* logits[m][v] = sum_h x[m][h] * W[v][h], summed in ascending h, for M bfloat16 token rows.
   ("3 ways to boost MoE inference on NVIDIA DGX Spark", "Model and baseline configuration": the LM
   head projects the hidden dimension 2,560 onto the vocabulary of 157,184; "Optimization 2: Online
   FP8 LM head quantization": the same GEMM with FP8 weights halves the read; "Chasing the Batch-1
   Floor", "bf16 router gate and lm_head": bf16 weights with fp32 accumulation.)
   fmt OF_BF16: W [V][H] bfloat16.  fmt OF_FP8: W [V][H] E4M3 codes times one binary32 scale per row
   (output channel), scales[v]; the reading of an online quantisation of a bf16 matrix. */
void oracle_lm_head(int32_t fmt, int32_t H, int32_t V, int32_t M, const void* x, const void* w, const float* scales,
                    double* logits, int32_t nthreads) {
    double* xs = (double*)malloc(sizeof(double) * (size_t)M * H);
    for (int m = 0; m < M; ++m) load_row(OF_BF16, x, m, H, xs + (int64_t)m * H);
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int v = 0; v < V; ++v) {
        double* wv = (double*)malloc(sizeof(double) * H);
        if (fmt == OF_FP8) {
            const uint8_t* codes = (const uint8_t*)w + (int64_t)v * H;
            const double sc = (double)scales[v];
            for (int h = 0; h < H; ++h) wv[h] = oracle_e4m3_to_f64(codes[h]) * sc;
        } else {
            load_row(OF_BF16, w, v, H, wv);
        }
        for (int m = 0; m < M; ++m) {
            const double* xrow = xs + (int64_t)m * H;
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += xrow[h] * wv[h];
            logits[(int64_t)m * V + v] = acc;
        }
        free(wv);
    }
    free(xs);
}

int32_t oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
