// router.hip - router logits in a fixed fp32 order.
//
// logits[t,e] = sum_k x[t,k] * W[e,k] (+ offset[e]): the linear layer in front of the gate
// (gate page "feat(engine): E1 DeepSeek-style MoE gate ...", merge recommendation: router
// linear, then route; "Algorithm": the gate takes fp32 logits).
//
// Every output element is accumulated by one fused multiply-add per k, k ascending, starting
// from +0.0f, then one fp32 add of the offset.  Because the order is fixed the logits are
// reproducible bit for bit, which keeps the expert selection stable.  That rules out MFMA
// (its internal summation order is not specified), so this is a VALU kernel: a workgroup
// stages a [BM tokens x 32] tile of x and a [BN experts x 32] tile of W in LDS as fp32
// (k-major, so a thread reads its MT tokens / NT experts at one k as one vector), and each
// thread keeps an MT x NT register tile of accumulators.  The k loop is never split across
// threads.  The zero tail of a partial k chunk is never fed to an FMA.
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

template <typename TA>
__device__ __forceinline__ float ld_act(const TA* p, int64_t i);
template <>
__device__ __forceinline__ float ld_act<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_act<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

constexpr int KC = 32;

template <typename TA, int MT, int NT>
__global__ __launch_bounds__(256) void router_kernel(const TA* __restrict__ x, const TA* __restrict__ w,
                                                     const float* __restrict__ off, float* __restrict__ logits,
                                                     int64_t T, int32_t H, int32_t E) {
    constexpr int BM = 16 * MT, BN = 16 * NT;
    __shared__ float xs[KC][BM + 4];
    __shared__ float ws[KC][BN + 4];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int32_t n0 = blockIdx.x * BN;

    float acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = 0.0f;

    for (int32_t k0 = 0; k0 < H; k0 += KC) {
        const int kc = min(KC, H - k0);
        for (int i = threadIdx.x; i < BM * KC; i += 256) {
            const int m = i / KC, k = i % KC;
            const int64_t t = m0 + m;
            xs[k][m] = (t < T && k < kc) ? ld_act(x, t * H + k0 + k) : 0.0f;
        }
        for (int i = threadIdx.x; i < BN * KC; i += 256) {
            const int n = i / KC, k = i % KC;
            const int32_t e = n0 + n;
            ws[k][n] = (e < E && k < kc) ? ld_act(w, (int64_t)e * H + k0 + k) : 0.0f;
        }
        __syncthreads();
        for (int k = 0; k < kc; ++k) {
            float a[MT], b[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i) a[i] = xs[k][ty * MT + i];
#pragma unroll
            for (int j = 0; j < NT; ++j) b[j] = ws[k][tx * NT + j];
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t t = m0 + ty * MT + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int32_t e = n0 + tx * NT + j;
            if (e >= E) continue;
            float v = acc[i][j];
            if (off) v = v + off[e];
            logits[t * E + e] = v;
        }
    }
}

template <typename TA, int MT, int NT>
hipError_t launch_t(const TA* x, const TA* w, int64_t T, int32_t H, int32_t E, const float* off, float* logits,
                    hipStream_t s) {
    const dim3 grid((E + 16 * NT - 1) / (16 * NT), (unsigned)((T + 16 * MT - 1) / (16 * MT)));
    hipLaunchKernelGGL((router_kernel<TA, MT, NT>), grid, dim3(256), 0, s, x, w, off, logits, T, H, E);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const void* x, const void* w, int32_t act, int64_t T, int32_t H, int32_t E,
                         const float* offset, float* logits, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const bool big = T * (int64_t)E >= (int64_t)1 << 19;  // enough outputs for 4x4 register tiles
    if (act == MOE_BF16) {
        const bf16_t* xb = (const bf16_t*)x;
        const bf16_t* wb = (const bf16_t*)w;
        return big ? launch_t<bf16_t, 4, 4>(xb, wb, T, H, E, offset, logits, s)
                   : launch_t<bf16_t, 1, 1>(xb, wb, T, H, E, offset, logits, s);
    }
    const float* xf = (const float*)x;
    const float* wf = (const float*)w;
    return big ? launch_t<float, 4, 4>(xf, wf, T, H, E, offset, logits, s)
               : launch_t<float, 1, 1>(xf, wf, T, H, E, offset, logits, s);
}

}  // namespace dsmoe
