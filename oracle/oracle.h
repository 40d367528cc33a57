/*
 * oracle.h - CPU reference ("oracle") of the DeepSeek-style MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously correct C.  Only the tests,
 * the package's smoke check and the benchmark's CPU-baseline leg may load it; the
 * GPU library never links or calls it, and the two share no code.  Inputs come
 * from the separate `synth` generator.
 *
 * Sources (pages given by title):
 *   [PR123]  "feat(engine): E1 DeepSeek-style MoE gate (sigmoid, group top-k, bias) (#108)"
 *            - sections "API", "Algorithm (mlx-lm group_expert_select)", "Scope decisions",
 *              and the two code reviews (validation matrix, S1/S2/S5, D7, zero-sum note,
 *              masked-to-zero non-issue).
 *   [Epic56] "Epic: Engine Inference Core Stage E - MoE + hybrid families"
 *            - opening paragraph (expert dispatch via gather_qmm / gather_mm) and
 *              "Decision 5 superseded" item 2 (sigmoid gating, group selection, shared
 *              experts always active).
 *
 * Precision: the gate is fp32 because [PR123] "Algorithm" casts the gate logits to f32
 * before the sigmoid.  The router dot product is fp32 with a fixed order (see
 * oracle_router).  The expert SwiGLU, shared expert and combine are computed in fp64
 * (at least the fp32 accumulation the layer requires).
 *
 * Dtype codes: 0 = fp32, 1 = bf16 (uint16 bit patterns), 2 = 4-bit affine, group 64,
 * 3 = fp8 E4M3 codes with fp32 scales per 128 x 128 block.
 */
#ifndef DSMOE_ORACLE_H
#define DSMOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oracle_route_params {
    int32_t top_k;
    int32_t n_group;
    int32_t topk_group;
    int32_t norm_topk_prob;
    float routed_scaling_factor;
} oracle_route_params;

typedef struct oracle_layer {
    int64_t T;
    int32_t H, E, I, Is; /* Is == 0: no shared expert */
    int32_t act;         /* 0 fp32, 1 bf16: x, router, shared weights */
    int32_t expert;      /* 0 fp32, 1 bf16, 2 q4g64, 3 fp8 block-scaled: routed expert weights */
    oracle_route_params route;
    const void* x;        /* [T,H] act */
    const void* router;   /* [E,H] act */
    const float* bias;    /* [E] e_score_correction_bias */
    const float* offset;  /* NULL or [E]: added to the router logits */
    const void* wg;       /* [E,I,H] (q4: uint32 [E,I,H/8]) */
    const void* wu;       /* [E,I,H] */
    const void* wd;       /* [E,H,I] (q4: uint32 [E,H,I/8]; fp8: uint8 [E,H,I]) */
    /* q4: bf16 scale s* / offset b* [E,out,in/64]; fp8: fp32 scales s* [E,ceil(out/128),ceil(in/128)],
     * b* unused */
    const void *sg, *bg, *su, *bu, *sd, *bd;
    const void* swg;      /* [Is,H] act */
    const void* swu;      /* [Is,H] act */
    const void* swd;      /* [H,Is] act */
    int32_t route_kind;   /* 0: DeepSeek sigmoid gate (oracle_route); 1: softmax gate (oracle_route_softmax) */
    const void* sgate;    /* NULL, or [H] act: the shared expert's output is scaled by sigmoid(x . sgate) */
} oracle_layer;

/* exp by Cody-Waite range reduction + degree-7 Taylor polynomial, fp32 (see oracle.c) */
float oracle_exp(float x);
/* 1 / (1 + oracle_exp(-x)), IEEE fp32 division */
float oracle_sigmoid(float x);

/* Router: logits[t,e] = sum_k x[t,k]*W[e,k] (fp32 fma, k ascending from 0) [+ offset[e]]. */
void oracle_router(const void* x, const void* w, int32_t dtype, int64_t T, int32_t H, int32_t E,
                   const float* offset, float* logits);

/* DeepSeek gate over T rows.  Returns 0, or -1 on invalid arguments (outputs untouched). */
int oracle_route(const float* logits, int64_t T, int32_t E, const float* bias, const oracle_route_params* p,
                 int32_t* inds, float* scores);

/* Softmax gate over T rows (see oracle.c for the reading taken).  Returns 0, or -1 on
 * invalid arguments (outputs untouched). */
int oracle_route_softmax(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t* inds, float* scores);
/* Value of one OCP E4M3 code (NaN for S.1111.111), exact. */
double oracle_e4m3(uint8_t c);
/* SwiGLU expert on one fp64 input row: out[H] = W_down (silu(W_gate x) * (W_up x)).
 * w* point at ONE expert's matrices in `dtype`; s*, b* are its q4 scale/offset or fp8 block
 * scales (or NULL). */
void oracle_swiglu(const double* x, int32_t H, int32_t I, int32_t dtype, const void* wg, const void* wu,
                   const void* wd, const void* sg, const void* bg, const void* su, const void* bu,
                   const void* sd, const void* bd, double* out);

/* Whole layer for the tokens rows[0..n_rows) (rows == NULL: all T tokens in order).
 * y: fp64 [n_rows,H]; inds/scores: [n_rows,K] (may be NULL); logits: [n_rows,E] (may be NULL).
 * Returns 0, or -1 on invalid arguments. */
int oracle_forward(const oracle_layer* L, const int64_t* rows, int64_t n_rows, double* y, int32_t* inds,
                   float* scores, float* logits);

/* Dispatch: the expert-major grouping of the T*K token slots (slot s = t*K + j) behind the
 * gather_mm / gather_qmm expert calls.  counts[e] = number of slots routed to e; offsets[e] =
 * counts[0] + ... + counts[e-1], offsets[E] = T*K; sorted_slot[offsets[e] .. offsets[e+1]) are
 * the slots routed to e in ascending order; slot_row[s] = the row r with sorted_slot[r] == s.
 * Returns 0, or -1 on invalid arguments or an index outside [0, E) (outputs untouched). */
int oracle_dispatch(const int32_t* inds, int64_t T, int32_t K, int32_t E, int32_t* counts, int32_t* offsets,
                    int32_t* sorted_slot, int32_t* slot_row);

/* Dense SwiGLU MLP over T rows of x ([T,H] act), weights [I,H], [I,H], [H,I] in act; y fp64 [T,H].
 * Returns 0, or -1 on invalid arguments. */
int oracle_dense_mlp(const void* x, int32_t act, int64_t T, int32_t H, int32_t I, const void* wg, const void* wu,
                     const void* wd, double* y);
/* host threads used by the OpenMP loops */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
