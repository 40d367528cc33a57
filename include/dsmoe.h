/*
 * dsmoe.h - C ABI of the MI355X (gfx950) DeepSeek-style mixture-of-experts layer forward.
 *
 * The library (libdsmoe.so) is hand-written HIP.  Every entry point takes plain pointers and
 * sizes; device pointers must be HIP device allocations (e.g. torch tensors on a ROCm device),
 * and `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *
 * Pages cited (by title):
 *   [PR123]  "feat(engine): E1 DeepSeek-style MoE gate (sigmoid, group top-k, bias) (#108)":
 *            sections "API", "Algorithm (mlx-lm group_expert_select)", "Scope decisions" and
 *            the two code reviews (validation matrix, ownership, merge recommendation).
 *   [Epic56] "Epic: Engine Inference Core Stage E - MoE + hybrid families": opening paragraph
 *            (forwardMoeWith: expert dispatch via gather_qmm / gather_mm) and "Decision 5
 *            superseded" item 2 (sigmoid gating with group selection, shared experts always
 *            active, fp8 / 4-bit checkpoints).
 *
 * Conventions shared by all entry points
 *   - Return codes: MOE_OK (0); MOE_ERR_INVALID (-1) invalid argument, the pages' convention;
 *     MOE_ERR_HIP (-2) a HIP launch/runtime error; MOE_ERR_WORKSPACE (-3) workspace too small;
 *     MOE_ERR_UNSUPPORTED (-4) valid but beyond this implementation's documented limits.
 *   - All scalar and pointer checks run on the host before any HIP call; on every error
 *     detected there (-1, -3, -4) no output buffer is written ([PR123] reviews: outputs are
 *     left unchanged on failure).  After a -2 the outputs are unspecified.
 *   - Calls are asynchronous on `stream`: results are valid once the stream has synchronised.
 *     Nothing here synchronises the host or reads device memory back.
 *   - The library never allocates device memory: scratch comes from the caller's workspace.
 *     Every entry point may be called from any host thread; calls that may run at the same time
 *     on the device need distinct workspaces and outputs.
 *   - Results are bitwise deterministic from run to run (no atomics on floating-point data).
 *   - Layouts are row-major.  Stacked expert weights are [E, out, in] with `in` contiguous
 *     ([Epic56] "expert stacking" at load time).  bf16 tensors hold raw bf16 bit patterns.
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef DSMOE_H
#define DSMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID (-1)
#define MOE_ERR_HIP (-2)
#define MOE_ERR_WORKSPACE (-3)
#define MOE_ERR_UNSUPPORTED (-4)

/* element types */
#define MOE_F32 0   /* IEEE binary32 */
#define MOE_BF16 1  /* bfloat16 (uint16 bit patterns) */
#define MOE_Q4G64 2 /* 4-bit affine, groups of 64 along the input axis (expert weights only) */
#define MOE_FP8 3   /* OCP E4M3 codes, one fp32 scale per 128 x 128 block (expert weights only) */

/* gate kinds (moe_layer_desc.route_kind) */
#define MOE_ROUTE_DEEPSEEK 0 /* sigmoid gate with correction bias and groups (moe_route_deepseek) */
#define MOE_ROUTE_SOFTMAX 1  /* softmax gate, always renormalised (moe_route_softmax) */

/* implementation limits (-4 beyond them) */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOP_K 64

/* Gate parameters ([PR123] "API": the DeepSeek route's own params struct). */
typedef struct moe_route_params {
    int32_t top_k;                 /* experts per token, 1 <= top_k <= E */
    int32_t n_group;               /* expert groups; E % n_group == 0 */
    int32_t topk_group;            /* groups kept per token, 1 <= topk_group <= n_group */
    int32_t norm_topk_prob;        /* nonzero: renormalise the weights when top_k > 1 */
    float routed_scaling_factor;   /* multiplies every returned weight, after the norm */
} moe_route_params;

/* Shapes and types of one MoE layer. */
typedef struct moe_layer_desc {
    int64_t T;           /* tokens (rows of x); 0 is a valid no-op */
    int32_t H;           /* hidden size */
    int32_t E;           /* routed experts */
    int32_t I;           /* routed expert intermediate size */
    int32_t I_shared;    /* shared expert intermediate size; 0 = no shared expert */
    int32_t act_dtype;   /* MOE_F32 or MOE_BF16: x, y, router weight and shared weights */
    int32_t expert_dtype;/* MOE_F32 (with act F32); MOE_BF16, MOE_Q4G64 or MOE_FP8 (with act BF16) */
    moe_route_params route; /* the softmax gate reads only route.top_k */
    int32_t route_kind;  /* MOE_ROUTE_DEEPSEEK or MOE_ROUTE_SOFTMAX */
} moe_layer_desc;

/* Routed expert weights, stacked along E.
 *   w_gate, w_up: [E, I, H]; w_down: [E, H, I] in expert_dtype.
 *   MOE_Q4G64: w_* are uint32 [E, out, in/8] holding eight 4-bit codes q (element i of a row at
 *   bits 4*(i%8) of word i/8); s_* and b_* are bf16 [E, out, in/64]; the weight is s*q + b.
 *   MOE_FP8: w_* are uint8 [E, out, in] OCP E4M3 codes (bias 7, no infinities; NaN codes are
 *   outside the contract); s_* are fp32 [E, ceil(out/128), ceil(in/128)], one scale per
 *   128 x 128 block; the weight is value(code) * scale -- the load-time dequantisation of fp8
 *   checkpoints ([Epic56] weight loading), done here in registers: the kernels multiply in fp32
 *   and round the product to bf16 (nearest even) before the bf16 matrix products.  b_* ignored.
 *   For the other dtypes s_* and b_* are ignored. */
typedef struct moe_expert_weights {
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    const void* s_gate;
    const void* b_gate;
    const void* s_up;
    const void* b_up;
    const void* s_down;
    const void* b_down;
} moe_expert_weights;

/* Shared expert ([Epic56] "Decision 5" item 2: always active, weight 1, no gate):
 * w_gate, w_up [I_shared, H]; w_down [H, I_shared]; act_dtype.
 * w_sgate: NULL (the DeepSeek body: weight 1), or [H] act_dtype: the shared expert's output of
 * token t is scaled by sigmoid(x[t] . w_sgate) -- the combine's shared-expert gate switch that
 * [PR123]'s reviews name (the dot product in moe_router_logits' order, the sigmoid as in the
 * gate). */
typedef struct moe_shared_weights {
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    const void* w_sgate;
} moe_shared_weights;

/*
 * Router logits: logits[t,e] = sum_k x[t,k] * W[e,k] (+ logit_offset[e]).
 * The linear layer in front of the gate ([PR123] merge recommendation: router linear, then
 * route); the gate consumes fp32 logits ([PR123] "Algorithm": sigmoid of f32 gates).
 * Arithmetic: fp32, one fused multiply-add per k in ascending k order starting from +0, then
 * one fp32 add of the offset.  This fixed order makes the logits, and hence the selection,
 * reproducible bit for bit by any implementation of the same order.
 *   x:        [T, H] act_dtype (device)      router_w: [E, H] act_dtype (device)
 *   logit_offset: NULL or fp32 [E] (device)  logits:   fp32 [T, E] (device, written)
 * Errors: -1 for NULL x/router_w/logits, T < 0, H < 1, E < 1, bad act_dtype, misalignment.
 */
int moe_router_logits(const void* x, const void* router_w, int32_t act_dtype, int64_t T, int32_t H, int32_t E,
                      const float* logit_offset, float* logits, void* stream);

/*
 * DeepSeek gate ([PR123] "API" and "Algorithm"), one row per token:
 *   s = sigmoid(logits) in fp32; b = s + bias (bias only selects, the weights use s);
 *   if n_group > 1 and topk_group < n_group: the score of a group is the sum of its two largest
 *   b; the topk_group best groups are kept (ties: lower group index) and every expert of the
 *   other groups gets b = 0.0;
 *   inds = the top_k experts by b, ordered by b descending then index ascending;
 *   scores = s[inds]; if top_k > 1 and norm_topk_prob: scores /= (left-to-right sum of scores);
 *   scores *= routed_scaling_factor.
 * The sigmoid uses exp by Cody-Waite reduction and a degree-7 Taylor polynomial with the exact
 * fp32 operation sequence documented in the route kernel, and IEEE division.
 *   logits: fp32 [T, E] (device; leading dims of a [..., E] tensor flatten to T rows)
 *   bias:   fp32 [bias_len] (device) -- e_score_correction_bias, required (zeros when the model
 *           has none); bias_len must equal E (rank-1 [E] per the reviews)
 *   inds:   int32 [T, top_k] (device, written)   scores: fp32 [T, top_k] (device, written)
 * Errors: -1 for NULL pointers, T < 0, top_k outside [1, E], n_group < 1, E % n_group != 0,
 * topk_group outside [1, n_group], n_group > 1 with E/n_group < 2, bias_len != E, misaligned
 * pointers; -4 for E > MOE_MAX_EXPERTS or top_k > MOE_MAX_TOP_K.
 */
int moe_route_deepseek(const float* logits, int64_t T, int32_t E, const float* bias, int64_t bias_len,
                       const moe_route_params* p, int32_t* inds, float* scores, void* stream);

/*
 * Softmax gate, the DeepSeek route's sibling ([PR123] "API": same output contract; second
 * review, S2: its weights are renormalised in every case, unlike the DeepSeek route's
 * top_k > 1 guard).  The pages define nothing further; this implementation, one row per token:
 *   ex_e = exp(logit_e - max_e logit_e) in fp32 (the gate's exp);
 *   inds = the top_k experts by ex, ordered by ex descending then index ascending;
 *   p_j = ex[inds_j] / sum_e ex_e;  scores_j = p_j / (left-to-right sum of the p_j).
 * No bias, groups or scaling factor.  The sum over all experts is formed in a fixed tree order
 * (it cancels in the renormalisation up to rounding).
 *   logits: fp32 [T, E] (device)   inds: int32 [T, top_k]   scores: fp32 [T, top_k] (written)
 * Errors: -1 for NULL pointers, T < 0, E < 1, top_k outside [1, E], misaligned pointers;
 * -4 for E > MOE_MAX_EXPERTS or top_k > MOE_MAX_TOP_K.
 */
int moe_route_softmax(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t* inds, float* scores,
                      void* stream);

/*
 * Dispatch (the grouping behind gather_mm / gather_qmm, [Epic56] opening paragraph): a stable
 * counting sort of the T*K token slots (slot s = t*K + j) by expert.
 *   counts[e]      = number of slots routed to e                          int32 [E]
 *   offsets[e]     = sum of counts[0..e); offsets[E] = T*K                int32 [E+1]
 *   sorted_slot[r] = the slot at expert-major row r; within an expert,
 *                    slots are in ascending order                         int32 [T*K]
 *   slot_row[s]    = r such that sorted_slot[r] == s                      int32 [T*K]
 * inds: int32 [T, K] (device), values must lie in [0, E); out-of-range values are clamped
 * into [0, E) on the device (never written out of bounds).
 * workspace: device scratch of at least moe_dispatch_workspace_size(T, K, E) bytes.
 * Errors: -1 for NULL pointers / T < 0 / K < 1 / E < 1; -3 for a small workspace;
 * -4 for E > MOE_MAX_EXPERTS or T*K >= 2^31.
 */
size_t moe_dispatch_workspace_size(int64_t T, int32_t K, int32_t E);
int moe_dispatch(const int32_t* inds, int64_t T, int32_t K, int32_t E, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_slot, int32_t* slot_row, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Whole layer ([Epic56] forwardMoeWith; [PR123] merge recommendation: router -> route ->
 * switch_glu -> combine, shared expert always active, no shared-expert gate):
 *   y[t] = g_t * shared(x[t]) + sum_{j<K} scores[t,j] * expert_{inds[t,j]}(x[t])
 *   (g_t = 1, or sigmoid(x[t] . w_sgate) when the shared weights carry a gate vector)
 *   expert(x) = W_down (silu(W_gate x) * (W_up x))   (SwiGLU; the gate projection is the one
 *                                                      that goes through silu)
 * Steps, all on `stream`: router logits (as moe_router_logits) -> gate (as moe_route_deepseek,
 * or moe_route_softmax when route_kind is MOE_ROUTE_SOFTMAX) -> dispatch (as moe_dispatch) ->
 * grouped gate/up GEMM with SwiGLU in the epilogue -> grouped down GEMM -> combine.  For bf16
 * layers with T > 64, each grouped GEMM is split by group size: weight streaming for the expert
 * groups of at most 64 rows, MFMA tiles (one launch) for the larger groups and the shared
 * expert.  For 4-bit and fp8 layers with T > 64, every quantised routed group is tiled, in a
 * launch of its own beside the bf16 shared expert's.  With T <= 64 every group is streamed.
 * The combine adds, per token and output element, the (gated) shared expert's output and then
 * the K weighted expert outputs in j order in fp32, with no atomics.
 * Precision: bf16 layers run bf16 MFMA with fp32 accumulation; the SwiGLU intermediate and the
 * per-expert outputs are rounded to bf16; y is rounded to act_dtype (nearest-even).  4-bit
 * weights are dequantised in registers (s*q + b, rounded to bf16) before the MFMA; fp8 weights
 * likewise (value * block scale in fp32, rounded to bf16).
 *   d:            shapes, dtypes and gate parameters (host)
 *   x:            [T, H] act_dtype (device)          router_w: [E, H] act_dtype (device)
 *   bias:         fp32 [E] (device; may be NULL with the softmax gate)
 *   logit_offset: NULL or fp32 [E] (device),
 *                 added to the router logits (a router bias; NULL for DeepSeek checkpoints)
 *   ew:           routed expert weights (host struct of device pointers)
 *   sw:           shared expert weights (host struct of device pointers); NULL iff I_shared == 0
 *   y:            [T, H] act_dtype (device, written)
 *   inds_out:     NULL or int32 [T, top_k] (device, written): the gate's selection
 *   scores_out:   NULL or fp32 [T, top_k] (device, written): the gate's weights
 *   workspace:    device scratch, at least moe_forward_workspace_size(d) bytes, 256-byte aligned
 * Errors: -1 for invalid shapes/params/pointers (as above, plus H, I < 1, I_shared < 0, a
 * dtype combination other than F32/F32, BF16/BF16, BF16/Q4G64, BF16/FP8, and for MOE_Q4G64
 * missing scales or offsets, for MOE_FP8 missing scales); -3 for a small workspace; -4 for
 * E > MOE_MAX_EXPERTS, top_k > MOE_MAX_TOP_K, T*top_k + T >= 2^31, or (bf16 / 4-bit / fp8
 * layers) H, I or I_shared not a multiple of 64.
 * moe_forward_workspace_size returns 0 for a descriptor that moe_forward would reject.
 */
size_t moe_forward_workspace_size(const moe_layer_desc* d);
int moe_forward(const moe_layer_desc* d, const void* x, const void* router_w, const float* bias,
                const float* logit_offset, const moe_expert_weights* ew, const moe_shared_weights* sw, void* y,
                int32_t* inds_out, float* scores_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_forward without a workspace argument, for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.  The
 * layer, its arguments (other than the workspace), its results and its errors are those of
 * moe_forward; the scratch is a fixed array of MOE_STATIC_SCRATCH_BYTES inside the library, one
 * per device, allocated when the library's code is loaded on that device and held until the
 * process ends.  The call allocates and frees nothing.  Layers whose
 * moe_forward_workspace_size exceeds MOE_STATIC_SCRATCH_BYTES (at DeepSeek-V3 shapes, batches
 * above 401 tokens) return MOE_ERR_WORKSPACE (-3) with no output written.
 * Every call on a device uses that device's one array: calls whose kernels may overlap on the
 * device (several streams, several threads) race on it and give undefined results; calls on one
 * stream are safe.  Nothing in the array needs to start at zero.
 */
#define MOE_STATIC_SCRATCH_BYTES (64 * 1024 * 1024)
int moe_forward_static(const moe_layer_desc* d, const void* x, const void* router_w, const float* bias,
                       const float* logit_offset, const moe_expert_weights* ew, const moe_shared_weights* sw, void* y,
                       int32_t* inds_out, float* scores_out, void* stream);

/*
 * Dense SwiGLU MLP layer: y = W_down (silu(W_gate x) * (W_up x)) per token -- the dense layers
 * that DeepSeek models interleave with MoE layers ([Epic56] "Decision 5 superseded" item 2:
 * dense/MoE layer mixing); the computation is the shared expert's path on its own, with the same
 * kernels (weight streaming for T <= 64, MFMA tiles above) and the same precision (bf16 MFMA with
 * fp32 accumulation, the SwiGLU intermediate rounded to bf16; fp32 layers in fp32).
 *   x:  [T, H] act_dtype (device)        y: [T, H] act_dtype (device, written)
 *   w_gate, w_up: [I, H]; w_down: [H, I]; act_dtype (device)
 *   workspace: device scratch, at least moe_dense_workspace_size(T, H, I, act_dtype) bytes,
 *              256-byte aligned
 * Errors: -1 for T < 0, H < 1, I < 1, act_dtype other than MOE_F32 / MOE_BF16, NULL or
 * misaligned pointers; -3 for a small workspace; -4 for bf16 with H or I not a multiple of 64,
 * or T >= 2^31.  moe_dense_workspace_size returns 0 for arguments moe_dense_mlp would reject.
 */
size_t moe_dense_workspace_size(int64_t T, int32_t H, int32_t I, int32_t act_dtype);
int moe_dense_mlp(int64_t T, int32_t H, int32_t I, int32_t act_dtype, const void* x, const void* w_gate,
                  const void* w_up, const void* w_down, void* y, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Measurement hook (not part of the computation).  Stages of moe_forward, in launch order:
 *   MOE_STAGE_ROUTER (router logits), MOE_STAGE_ROUTE (gate), MOE_STAGE_DISPATCH (count, scan,
 *   scatter), MOE_STAGE_GEMM1 (gate/up + SwiGLU), MOE_STAGE_GEMM2 (down), MOE_STAGE_COMBINE.
 * While a hook is set, every moe_forward call records events[2*i] on its stream right before
 * the first kernel of `stage` and events[2*i + 1] right after the stage's last kernel, with
 * i = (moe_forward calls since the hook was set) mod n_pairs.  When a grouped GEMM is split
 * into streaming and tiled kernels (see moe_forward), the GEMM1 and GEMM2 pairs bracket the
 * tiled launches only.  events are hipEvent_t handles
 * owned by the caller (created with timing enabled) and must outlive the hook.  stage = -1 (or
 * n_pairs = 0) clears the hook.  The hook is process-wide: setting it and moe_forward calls may
 * come from any thread (each call takes its event pair once, at entry, under a lock), but the
 * calls of all threads advance one counter, so per-call timings are meaningful only while one
 * thread drives moe_forward.  Errors: -1 for a stage out of range, n_pairs < 0, or NULL events
 * with n_pairs > 0 (the hook is then unchanged).
 */
#define MOE_STAGE_ROUTER 0
#define MOE_STAGE_ROUTE 1
#define MOE_STAGE_DISPATCH 2
#define MOE_STAGE_GEMM1 3
#define MOE_STAGE_GEMM2 4
#define MOE_STAGE_COMBINE 5
int moe_set_stage_events(int32_t stage, void* const* events, int32_t n_pairs);

/* Text for a return code (static storage). */
const char* moe_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* DSMOE_H */
