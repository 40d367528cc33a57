// combine.hip - deterministic weighted combine of the expert outputs.
//
// y[t] = g_t * shared(x[t]) + sum_j scores[t,j] * o[slot_row[t*K + j]]  (page "feat(engine): E1
// DeepSeek-style MoE gate ...", merge recommendation: combine with an always-active shared
// expert and no shared-expert gate, g_t = 1; the reviews also name the combine's shared-expert
// gate switch, read here as g_t = sigmoid(x[t] . w_sgate)).  Each output element is owned by one
// thread, which adds, in fp32, the (gated) shared expert's output first and then the K weighted
// expert outputs in j order;
// no atomics, so the result is the same bits on every run.  bf16 layers move 8 elements per
// thread with 16-byte loads; the result is rounded to the activation type (nearest even).  Every
// expert-output row is read exactly once here, so those loads carry the non-temporal hint (the
// DeepSeek-V3 prefill combine, T = 8192: 235 -> 200 us).
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

constexpr int CB = 256;  // threads per token block

__global__ __launch_bounds__(CB) void combine_bf16(const bf16_t* __restrict__ o, const float* __restrict__ scores,
                                                  const int32_t* __restrict__ slot_row, int32_t H, int32_t K,
                                                  int32_t TK, int32_t has_shared, const float* __restrict__ sgl,
                                                  bf16_t* __restrict__ y) {
    const int64_t t = blockIdx.x;
    const float gs = sgl ? sigmoid_cw(sgl[t]) : 1.0f;  // shared-expert gate
    __shared__ float w[MOE_MAX_TOP_K];
    __shared__ int32_t row[MOE_MAX_TOP_K];
    if (threadIdx.x < K) {
        w[threadIdx.x] = scores[t * K + threadIdx.x];
        row[threadIdx.x] = slot_row[t * K + threadIdx.x];
    }
    __syncthreads();
    for (int32_t c = (blockIdx.y * CB + threadIdx.x) * 8; c < H; c += gridDim.y * CB * 8) {
        float acc[8];
        if (has_shared) {
            const u32x4 v = __builtin_nontemporal_load((const u32x4*)(o + (TK + t) * H + c));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = gs * bf16_to_f32((bf16_t)(v[i] & 0xffffu));
                acc[2 * i + 1] = gs * bf16_to_f32((bf16_t)(v[i] >> 16));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        }
        // the K expert rows in batches of eight: a batch's loads are issued together, then added
        // in j order
        for (int32_t j0 = 0; j0 < K; j0 += 8) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = j0 + u < K ? __builtin_nontemporal_load((const u32x4*)(o + (int64_t)row[j0 + u] * H + c))
                                  : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u >= K) break;
                const float wj = w[j0 + u];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = __builtin_fmaf(wj, bf16_to_f32((bf16_t)(v[u][i] & 0xffffu)), acc[2 * i]);
                    acc[2 * i + 1] = __builtin_fmaf(wj, bf16_to_f32((bf16_t)(v[u][i] >> 16)), acc[2 * i + 1]);
                }
            }
        }
        u32x4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
        *(u32x4*)(y + t * H + c) = out;
    }
}

__global__ __launch_bounds__(CB) void combine_f32(const float* __restrict__ o, const float* __restrict__ scores,
                                                 const int32_t* __restrict__ slot_row, int32_t H, int32_t K,
                                                 int32_t TK, int32_t has_shared, const float* __restrict__ sgl,
                                                 float* __restrict__ y) {
    const int64_t t = blockIdx.x;
    const float gs = sgl ? sigmoid_cw(sgl[t]) : 1.0f;  // shared-expert gate
    for (int32_t c = blockIdx.y * CB + threadIdx.x; c < H; c += gridDim.y * CB) {
        float acc = has_shared ? gs * o[(TK + t) * H + c] : 0.0f;
        for (int32_t j = 0; j < K; ++j)
            acc = __builtin_fmaf(scores[t * K + j], o[(int64_t)slot_row[t * K + j] * H + c], acc);
        y[t * H + c] = acc;
    }
}

}  // namespace

hipError_t launch_combine(const GroupedArgs& a, int32_t act, const float* scores, const int32_t* slot_row,
                          const float* sgate_logits, void* y, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    const int has_shared = a.Is > 0 ? 1 : 0;
    if (act == MOE_BF16) {
        const int per_block = CB * 8;
        const unsigned cy = (unsigned)((a.H + per_block - 1) / per_block);
        hipLaunchKernelGGL(combine_bf16, dim3((unsigned)a.T, cy), dim3(CB), 0, s, (const bf16_t*)a.o, scores,
                           slot_row, a.H, a.K, a.TK, has_shared, sgate_logits, (bf16_t*)y);
    } else {
        const unsigned cy = (unsigned)((a.H + CB - 1) / CB);
        hipLaunchKernelGGL(combine_f32, dim3((unsigned)a.T, cy), dim3(CB), 0, s, (const float*)a.o, scores, slot_row,
                           a.H, a.K, a.TK, has_shared, sgate_logits, (float*)y);
    }
    return hipGetLastError();
}

}  // namespace dsmoe
