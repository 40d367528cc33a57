/*
 * oracle.c - CPU reference of the DeepSeek-style MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): plain C, no blocking or fusion beyond what
 * the definitions below state; OpenMP only distributes independent rows / pairs.
 * Build with -ffp-contract=off so that every fp32 operation is the one written here.
 *
 * Page references are by title, see oracle.h: [PR123] and [Epic56].
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------
 * scalar helpers
 * ------------------------------------------------------------------------------------ */
static inline float bf16f(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static inline float act_at(const void* p, int32_t dtype, int64_t i) {
    return dtype == 1 ? bf16f(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

/*
 * exp(x) in fp32 by Cody & Waite range reduction (W. J. Cody, W. Waite, "Software Manual
 * for the Elementary Functions", 1980):
 *   n = rint(x * log2(e))                       (round half to even)
 *   r = (x - n*LN2_HI) - n*LN2_LO               (two fused multiply-adds)
 *   p = 1 + r + r^2/2! + ... + r^7/7!           (Taylor series, Horner form, fused multiply-adds)
 *   exp(x) = p * 2^n                            (ldexpf: exact scaling)
 * LN2_HI holds the leading 16 bits of ln 2 and LN2_LO = ln 2 - LN2_HI rounded to fp32.
 * Inputs above ln(FLT_MAX) give +inf; inputs below ln(FLT_MIN) give 0 (results that would be
 * subnormal are flushed; 1 + such a value is 1 in fp32, so the sigmoid is unaffected); NaN
 * passes through.
 */
#define EXP_HI_CUT 0x1.62e430p+6f   /* 88.72283935546875 > ln(FLT_MAX): above it +inf */
#define EXP_LO_CUT (-0x1.5d589ep+6f) /* -87.33654022216797 >= ln(FLT_MIN): below it 0 */
#define LOG2E_F 0x1.715476p+0f      /* log2(e) rounded to fp32 */
#define LN2_HI 0x1.62e400p-1f       /* leading 16 bits of ln 2 */
#define LN2_LO 0x1.7f7d1cp-20f      /* ln 2 - LN2_HI rounded to fp32 */
/* Taylor coefficients 1/k! rounded to fp32 */
#define C7 0x1.a01a02p-13f
#define C6 0x1.6c16c2p-10f
#define C5 0x1.111112p-7f
#define C4 0x1.555556p-5f
#define C3 0x1.555556p-3f

float oracle_exp(float x) {
    if (x != x) return x;
    if (x > EXP_HI_CUT) return INFINITY;
    if (x < EXP_LO_CUT) return 0.0f;
    float n = rintf(x * LOG2E_F);
    float r = fmaf(-n, LN2_HI, x);
    r = fmaf(-n, LN2_LO, r);
    float p = C7;
    p = fmaf(p, r, C6);
    p = fmaf(p, r, C5);
    p = fmaf(p, r, C4);
    p = fmaf(p, r, C3);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

/* [PR123] "Algorithm": scores = sigmoid(f32(gates)) */
float oracle_sigmoid(float x) { return 1.0f / (1.0f + oracle_exp(-x)); }

/* ------------------------------------------------------------------------------------
 * router: the linear layer whose output the gate consumes ([PR123] merge recommendation:
 * callers compose fwd_linear(router) -> route).  Precision: fp32 logits.  Order: one
 * fused multiply-add per k, k ascending, starting from +0.0f; then the optional offset.
 * ------------------------------------------------------------------------------------ */
void oracle_router(const void* x, const void* w, int32_t dtype, int64_t T, int32_t H, int32_t E,
                   const float* offset, float* logits) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            float acc = 0.0f;
            for (int32_t k = 0; k < H; ++k)
                acc = fmaf(act_at(x, dtype, t * (int64_t)H + k), act_at(w, dtype, (int64_t)e * H + k), acc);
            if (offset) acc = acc + offset[e];
            logits[t * (int64_t)E + e] = acc;
        }
    }
}

/* ------------------------------------------------------------------------------------
 * gate
 * ------------------------------------------------------------------------------------ */
typedef struct {
    float v;
    int32_t i;
} vi_t;

#define MAX_TOPK_ORACLE 1024

/* Total order used for every selection: larger value first; equal values (so -0 == +0)
 * by smaller index; NaN after every number. */
static int vi_cmp(const void* pa, const void* pb) {
    const vi_t* a = (const vi_t*)pa;
    const vi_t* b = (const vi_t*)pb;
    int an = a->v != a->v, bn = b->v != b->v;
    if (an != bn) return an ? 1 : -1;
    if (!an) {
        if (a->v > b->v) return -1;
        if (a->v < b->v) return 1;
    }
    return (a->i > b->i) - (a->i < b->i);
}

/* [PR123] "API" and the prologue reject matrix of the reviews: null args, top_k == 0,
 * top_k > E, E % n_group != 0, topk_group outside [1, n_group], n_group > 1 with fewer
 * than 2 experts per group.  Negative row counts are also rejected. */
static int route_args_ok(const float* logits, int64_t T, int32_t E, const float* bias,
                         const oracle_route_params* p, const int32_t* inds, const float* scores) {
    if (!logits || !bias || !p || !inds || !scores) return 0;
    if (T < 0 || E < 1) return 0;
    if (p->top_k < 1 || p->top_k > E) return 0;
    if (p->n_group < 1 || E % p->n_group != 0) return 0;
    if (p->topk_group < 1 || p->topk_group > p->n_group) return 0;
    if (p->n_group > 1 && E / p->n_group < 2) return 0;
    return 1;
}

/* One row of the gate, in the order of [PR123] "Algorithm":
 *   1. orig = sigmoid(f32(logits))
 *   2. biased = orig + bias                         (selection only, S1)
 *   3. if n_group > 1 and some groups are dropped:   (k_drop == 0 skips it, D7)
 *        group score = sum of the two largest biased scores of the group (S5: top-2 sum),
 *        keep the topk_group best groups, set every expert of a dropped group to 0.0
 *   4. inds = top_k of biased (ties -> lower index; order: value desc, index asc)
 *   5. w = orig[inds]                                (pre-bias weights, S1)
 *   6. if top_k > 1 and norm_topk_prob: w /= sum(w)  (S2; no epsilon, no zero-sum guard)
 *   7. w *= routed_scaling_factor
 */
static void route_row(const float* lg, int32_t E, const float* bias, const oracle_route_params* p,
                      float* orig, vi_t* b, vi_t* grp, int32_t* inds, float* scores) {
    const int32_t G = p->n_group, TG = p->topk_group, K = p->top_k;
    for (int32_t e = 0; e < E; ++e) {
        orig[e] = oracle_sigmoid(lg[e]);
        b[e].v = orig[e] + bias[e];
        b[e].i = e;
    }
    if (G > 1 && TG < G) {
        const int32_t Eg = E / G;
        vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * (size_t)Eg);
        for (int32_t g = 0; g < G; ++g) {
            memcpy(tmp, b + (int64_t)g * Eg, sizeof(vi_t) * (size_t)Eg);
            qsort(tmp, (size_t)Eg, sizeof(vi_t), vi_cmp);
            grp[g].v = tmp[0].v + tmp[1].v;
            grp[g].i = g;
        }
        free(tmp);
        qsort(grp, (size_t)G, sizeof(vi_t), vi_cmp);
        for (int32_t r = TG; r < G; ++r) {
            int32_t g = grp[r].i;
            for (int32_t e = g * Eg; e < (g + 1) * Eg; ++e) b[e].v = 0.0f;
        }
    }
    qsort(b, (size_t)E, sizeof(vi_t), vi_cmp);
    for (int32_t j = 0; j < K; ++j) {
        inds[j] = b[j].i;
        scores[j] = orig[b[j].i];
    }
    if (K > 1 && p->norm_topk_prob) {
        float s = scores[0];
        for (int32_t j = 1; j < K; ++j) s = s + scores[j];
        for (int32_t j = 0; j < K; ++j) scores[j] = scores[j] / s;
    }
    for (int32_t j = 0; j < K; ++j) scores[j] = scores[j] * p->routed_scaling_factor;
}

int oracle_route(const float* logits, int64_t T, int32_t E, const float* bias, const oracle_route_params* p,
                 int32_t* inds, float* scores) {
    if (!route_args_ok(logits, T, E, bias, p, inds, scores)) return -1;
#pragma omp parallel
    {
        float* orig = (float*)malloc(sizeof(float) * (size_t)E);
        vi_t* b = (vi_t*)malloc(sizeof(vi_t) * (size_t)E);
        vi_t* grp = (vi_t*)malloc(sizeof(vi_t) * (size_t)p->n_group);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t)
            route_row(logits + t * E, E, bias, p, orig, b, grp, inds + t * p->top_k, scores + t * p->top_k);
        free(orig);
        free(b);
        free(grp);
    }
    return 0;
}

/* Softmax gate, the sibling route of [PR123] ("API": it shares the DeepSeek route's output
 * contract, inds and scores [.., K]; second review, S2: unlike the DeepSeek route's top_k > 1
 * guard, it normalises its weights in every case).  The pages print nothing more; the
 * reading taken, one row:
 *   m = max_e logit_e;  ex_e = oracle_exp(logit_e - m)  (fp32)
 *   S = ((ex_0 + ex_1) + ex_2) + ...                       (fp32, index order)
 *   inds = top_k of ex (ties -> lower index; order: ex desc, index asc)
 *   p_j = ex[inds_j] / S;  W = ((p_0 + p_1) + ...);  scores_j = p_j / W
 * No bias, no groups, no scaling factor.  Ranking by ex (rather than by ex / S) keeps the
 * selection independent of how S is summed. */
static void route_softmax_row(const float* lg, int32_t E, int32_t K, vi_t* b, int32_t* inds, float* scores) {
    float m = lg[0];
    for (int32_t e = 1; e < E; ++e) m = lg[e] > m ? lg[e] : m;
    float S = 0.0f;
    for (int32_t e = 0; e < E; ++e) {
        b[e].v = oracle_exp(lg[e] - m);
        b[e].i = e;
        S = e == 0 ? b[e].v : S + b[e].v;
    }
    float ex[MAX_TOPK_ORACLE];
    qsort(b, (size_t)E, sizeof(vi_t), vi_cmp);
    for (int32_t j = 0; j < K; ++j) {
        inds[j] = b[j].i;
        ex[j] = b[j].v / S;
    }
    float W = 0.0f;
    for (int32_t j = 0; j < K; ++j) W = j == 0 ? ex[0] : W + ex[j];
    for (int32_t j = 0; j < K; ++j) scores[j] = ex[j] / W;
}

int oracle_route_softmax(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t* inds, float* scores) {
    if (!logits || !inds || !scores || T < 0 || E < 1 || top_k < 1 || top_k > E || top_k > MAX_TOPK_ORACLE)
        return -1;
#pragma omp parallel
    {
        vi_t* b = (vi_t*)malloc(sizeof(vi_t) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) route_softmax_row(logits + t * E, E, top_k, b, inds + t * top_k, scores + t * top_k);
        free(b);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------
 * experts
 * ------------------------------------------------------------------------------------ */
/*
 * OCP 8-bit floating point, E4M3 ("FN" variant: no infinities): bit 7 sign, bits 6..3 exponent
 * with bias 7, bits 2..0 mantissa.  Exponent field 0 holds the subnormals m * 2^-9; S.1111.111
 * is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.  Written from that definition.
 */
double oracle_e4m3(uint8_t c) {
    const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* The 256 E4M3 values, each oracle_e4m3(c), filled once when the library loads, so that the
 * expert loops look a code up instead of decoding it at every use (same values). */
static double e4m3_value[256];
__attribute__((constructor)) static void fill_e4m3_values(void) {
    for (int c = 0; c < 256; ++c) e4m3_value[c] = oracle_e4m3((uint8_t)c);
}

/* element (o, i) of one expert matrix [out, in] in `dtype`:
 *   2 (q4): affine group-64 code, weight = s*q + b (s, b bf16 [out, in/64]);
 *   3 (fp8): E4M3 code times the fp32 scale of its 128 x 128 block (s fp32
 *            [ceil(out/128), ceil(in/128)]), the load-time dequantisation of an fp8 checkpoint
 *            ([Epic56] weight loading: fp8 dequantisation), exact in fp64. */
static inline double w_at(const void* w, int32_t dtype, const void* s, const void* b, int32_t in, int64_t o,
                          int64_t i) {
    if (dtype == 2) {
        uint32_t word = ((const uint32_t*)w)[o * (in / 8) + i / 8];
        int q = (int)((word >> (4 * (i % 8))) & 0xFu);
        int64_t g = o * (in / 64) + i / 64;
        return (double)bf16f(((const uint16_t*)s)[g]) * (double)q + (double)bf16f(((const uint16_t*)b)[g]);
    }
    if (dtype == 3) {
        const int64_t nib = ((int64_t)in + 127) / 128;
        const double sc = (double)((const float*)s)[(o / 128) * nib + i / 128];
        return e4m3_value[((const uint8_t*)w)[o * (int64_t)in + i]] * sc;
    }
    return (double)act_at(w, dtype, o * (int64_t)in + i);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU expert: h = silu(x W_gate^T) * (x W_up^T); out = h W_down^T (gate is the first
 * projection and goes through silu; up is linear). */
void oracle_swiglu(const double* x, int32_t H, int32_t I, int32_t dtype, const void* wg, const void* wu,
                   const void* wd, const void* sg, const void* bg, const void* su, const void* bu,
                   const void* sd, const void* bd, double* out) {
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    for (int32_t n = 0; n < I; ++n) {
        double g = 0.0, u = 0.0;
        for (int32_t k = 0; k < H; ++k) {
            g += x[k] * w_at(wg, dtype, sg, bg, H, n, k);
            u += x[k] * w_at(wu, dtype, su, bu, H, n, k);
        }
        h[n] = silu(g) * u;
    }
    for (int32_t m = 0; m < H; ++m) {
        double o = 0.0;
        for (int32_t n = 0; n < I; ++n) o += h[n] * w_at(wd, dtype, sd, bd, I, m, n);
        out[m] = o;
    }
    free(h);
}

static size_t expert_elem_bytes(int32_t dtype) { return dtype == 0 ? 4 : dtype == 3 ? 1 : 2; }

/* pointer to expert e's matrix [out,in] inside a stacked [E,out,in] tensor */
static const void* expert_mat(const void* base, int32_t dtype, int64_t e, int32_t out, int32_t in) {
    if (dtype == 2) return (const uint32_t*)base + e * (int64_t)out * (in / 8);
    return (const char*)base + e * (int64_t)out * in * expert_elem_bytes(dtype);
}

/* expert e's scales (or q4 offsets) inside their stacked tensor: q4 bf16 [E,out,in/64], fp8 fp32
 * [E,ceil(out/128),ceil(in/128)]; NULL stays NULL */
static const void* expert_sb(const void* base, int32_t dtype, int64_t e, int32_t out, int32_t in) {
    if (!base) return NULL;
    if (dtype == 3) return (const float*)base + e * (((int64_t)out + 127) / 128) * (((int64_t)in + 127) / 128);
    return (const uint16_t*)base + e * (int64_t)out * (in / 64);
}

/*
 * Layer forward ([Epic56] opening paragraph and "Decision 5" item 2; [PR123] merge
 * recommendation: router -> route -> switch_glu -> combine with an always-active shared
 * expert and no shared-expert gate):
 *   y[t] = shared(x[t]) + sum_j scores[t,j] * expert_{inds[t,j]}(x[t])
 */
int oracle_forward(const oracle_layer* L, const int64_t* rows, int64_t n_rows, double* y, int32_t* inds,
                   float* scores, float* logits) {
    if (!L || !y || !L->x || !L->router || !L->wg || !L->wu || !L->wd) return -1;
    if (L->route_kind != 0 && L->route_kind != 1) return -1;
    if (L->route_kind == 0 && !L->bias) return -1;
    const int32_t H = L->H, E = L->E, I = L->I, Is = L->Is, K = L->route.top_k;
    if (L->T < 0 || n_rows < 0 || H < 1 || I < 1 || Is < 0 || K < 1 || K > E) return -1;
    if (L->act != 0 && L->act != 1) return -1;
    if (L->expert < 0 || L->expert > 3) return -1;
    if (L->expert == 2 && (H % 64 || I % 64 || !L->sg || !L->bg || !L->su || !L->bu || !L->sd || !L->bd))
        return -1;
    if (L->expert == 3 && (!L->sg || !L->su || !L->sd)) return -1;
    if (Is > 0 && (!L->swg || !L->swu || !L->swd)) return -1;
    if (!rows) n_rows = L->T;

    /* gather the selected token rows of x */
    size_t xb = L->act == 1 ? 2 : 4;
    char* xs = (char*)malloc(xb * (size_t)n_rows * H + 1);
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t t = rows ? rows[r] : r;
        if (t < 0 || t >= L->T) {
            free(xs);
            return -1;
        }
        memcpy(xs + xb * (size_t)r * H, (const char*)L->x + xb * (size_t)t * H, xb * (size_t)H);
    }
    float* lg = (float*)malloc(sizeof(float) * (size_t)n_rows * E + 1);
    int32_t* id = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_rows * K + 1);
    float* sc = (float*)malloc(sizeof(float) * (size_t)n_rows * K + 1);
    oracle_router(xs, L->router, L->act, n_rows, H, E, L->offset, lg);
    const int rrc = L->route_kind == 0 ? oracle_route(lg, n_rows, E, L->bias, &L->route, id, sc)
                                       : oracle_route_softmax(lg, n_rows, E, K, id, sc);
    /* shared-expert gate: g = sigmoid(x . w_sgate), the dot product in the router's order */
    float* sgl = NULL;
    if (Is > 0 && L->sgate) {
        sgl = (float*)malloc(sizeof(float) * (size_t)n_rows + 1);
        oracle_router(xs, L->sgate, L->act, n_rows, H, 1, NULL, sgl);
    }
    if (rrc != 0) {
        free(sgl);
        free(xs);
        free(lg);
        free(id);
        free(sc);
        return -1;
    }

    /* expert outputs for every (row, j) pair; j == K is the shared expert */
    const int32_t KS = K + (Is > 0 ? 1 : 0);
    double* o = (double*)malloc(sizeof(double) * (size_t)n_rows * KS * H + 1);
#pragma omp parallel
    {
        double* xd = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t pr = 0; pr < n_rows * KS; ++pr) {
            int64_t r = pr / KS;
            int32_t j = (int32_t)(pr % KS);
            for (int32_t k = 0; k < H; ++k) xd[k] = (double)act_at(xs, L->act, r * (int64_t)H + k);
            double* out = o + (size_t)pr * H;
            if (j < K) {
                int64_t e = id[r * K + j];
                int32_t dt = L->expert;
                oracle_swiglu(xd, H, I, dt, expert_mat(L->wg, dt, e, I, H), expert_mat(L->wu, dt, e, I, H),
                              expert_mat(L->wd, dt, e, H, I), expert_sb(L->sg, dt, e, I, H),
                              expert_sb(L->bg, dt, e, I, H), expert_sb(L->su, dt, e, I, H),
                              expert_sb(L->bu, dt, e, I, H), expert_sb(L->sd, dt, e, H, I),
                              expert_sb(L->bd, dt, e, H, I), out);
            } else {
                oracle_swiglu(xd, H, Is, L->act, L->swg, L->swu, L->swd, NULL, NULL, NULL, NULL, NULL, NULL,
                              out);
            }
        }
        free(xd);
    }
    /* combine: shared output (weight 1, or its sigmoid gate) plus the weighted routed
     * outputs, j ascending */
    for (int64_t r = 0; r < n_rows; ++r) {
        const double gs = sgl ? (double)oracle_sigmoid(sgl[r]) : 1.0;
        for (int32_t m = 0; m < H; ++m) {
            double acc = Is > 0 ? gs * o[((size_t)r * KS + K) * H + m] : 0.0;
            for (int32_t j = 0; j < K; ++j) acc += (double)sc[r * K + j] * o[((size_t)r * KS + j) * H + m];
            y[r * (int64_t)H + m] = acc;
        }
    }
    if (inds) memcpy(inds, id, sizeof(int32_t) * (size_t)n_rows * K);
    if (scores) memcpy(scores, sc, sizeof(float) * (size_t)n_rows * K);
    if (logits) memcpy(logits, lg, sizeof(float) * (size_t)n_rows * E);
    free(xs);
    free(lg);
    free(id);
    free(sc);
    free(o);
    free(sgl);
    return 0;
}

/* ------------------------------------------------------------------------------------
 * dispatch
 * ------------------------------------------------------------------------------------ */
/*
 * Expert dispatch ([Epic56] opening paragraph: forwardMoeWith hands each expert its tokens through
 * gather_mm / gather_qmm).  The grouping written out as a counting sort, in three passes:
 *   1. histogram: counts[e] = #{ s : inds[s] == e } over the slots s = t*K + j;
 *   2. exclusive prefix sum: offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e];
 *   3. placement: walking the slots in ascending s, slot s goes to the next free row of its
 *      expert's segment, so slots keep ascending order inside each expert (a stable sort);
 *      slot_row records where each slot went.
 */
int oracle_dispatch(const int32_t* inds, int64_t T, int32_t K, int32_t E, int32_t* counts, int32_t* offsets,
                    int32_t* sorted_slot, int32_t* slot_row) {
    if (!counts || !offsets || T < 0 || K < 1 || E < 1) return -1;
    const int64_t n = T * (int64_t)K;
    if (n > 0 && (!inds || !sorted_slot || !slot_row)) return -1;
    if (n >= ((int64_t)1 << 31)) return -1;
    for (int64_t s = 0; s < n; ++s)
        if (inds[s] < 0 || inds[s] >= E) return -1;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t s = 0; s < n; ++s) counts[inds[s]] += 1;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    for (int32_t e = 0; e < E; ++e) next[e] = offsets[e];
    for (int64_t s = 0; s < n; ++s) {
        const int32_t r = next[inds[s]]++;
        sorted_slot[r] = (int32_t)s;
        slot_row[s] = r;
    }
    free(next);
    return 0;
}

/* Dense SwiGLU MLP layer ([Epic56] "Decision 5 superseded" item 2: DeepSeek mixes dense and MoE
 * layers): y[t] = W_down (silu(W_gate x_t) * (W_up x_t)) for every token, fp64 (oracle_swiglu
 * on each row).  Returns 0, or -1 on invalid arguments. */
int oracle_dense_mlp(const void* x, int32_t act, int64_t T, int32_t H, int32_t I, const void* wg, const void* wu,
                     const void* wd, double* y) {
    if (!x || !wg || !wu || !wd || !y || T < 0 || H < 1 || I < 1 || (act != 0 && act != 1)) return -1;
#pragma omp parallel
    {
        double* xd = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            for (int32_t k = 0; k < H; ++k) xd[k] = (double)act_at(x, act, t * (int64_t)H + k);
            oracle_swiglu(xd, H, I, act, wg, wu, wd, NULL, NULL, NULL, NULL, NULL, NULL, y + t * (int64_t)H);
        }
        free(xd);
    }
    return 0;
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* number of host threads the OpenMP loops above use */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
