// experts_f32.hip - grouped SwiGLU expert GEMMs for fp32 layers.
//
// Same computation as the bf16 path (gate/up projection with SwiGLU, then down projection;
// page "Epic: Engine Inference Core Stage E - MoE + hybrid families", opening paragraph), for
// layers whose activations and weights are fp32.  MFMA has no fp32 input path that pays at
// these sizes, so one thread computes one output element with fp32 fused multiply-adds.
// Rows are the dispatch's expert-major rows; rows TK + t belong to the shared expert.
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// grid: x = row blocks of 4, y = column blocks of 64
__global__ __launch_bounds__(256) void gemm1_f32(GroupedArgs a) {
    const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.y;
    const int32_t n = blockIdx.y * 64 + threadIdx.x;
    if (r >= a.TK + a.T) return;
    const bool shared = r >= a.TK;
    const int32_t N = shared ? a.Is : a.I;
    if (n >= N) return;
    const int32_t H = a.H;
    int64_t tok;
    const float *wg, *wu;
    if (shared) {
        tok = r - a.TK;
        wg = (const float*)a.swg + (int64_t)n * H;
        wu = (const float*)a.swu + (int64_t)n * H;
    } else {
        const int32_t slot = a.sorted_slot[r];
        const int64_t e = a.inds[slot];
        tok = slot / a.K;
        wg = (const float*)a.wg + (e * a.I + n) * H;
        wu = (const float*)a.wu + (e * a.I + n) * H;
    }
    const float* xr = (const float*)a.x + tok * H;
    float g = 0.0f, u = 0.0f;
    for (int32_t k = 0; k < H; ++k) {
        g = __builtin_fmaf(xr[k], wg[k], g);
        u = __builtin_fmaf(xr[k], wu[k], u);
    }
    ((float*)a.h)[r * a.ldh + n] = silu_f(g) * u;
}

__global__ __launch_bounds__(256) void gemm2_f32(GroupedArgs a) {
    const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.y;
    const int32_t n = blockIdx.y * 64 + threadIdx.x;
    if (r >= a.TK + a.T) return;
    const bool shared = r >= a.TK;
    if (shared && a.Is == 0) return;
    const int32_t H = a.H;
    if (n >= H) return;
    const int32_t KD = shared ? a.Is : a.I;
    const float* wd;
    if (shared) {
        wd = (const float*)a.swd + (int64_t)n * KD;
    } else {
        const int64_t e = a.inds[a.sorted_slot[r]];
        wd = (const float*)a.wd + (e * H + n) * KD;
    }
    const float* hr = (const float*)a.h + r * a.ldh;
    float acc = 0.0f;
    for (int32_t k = 0; k < KD; ++k) acc = __builtin_fmaf(hr[k], wd[k], acc);
    ((float*)a.o)[r * H + n] = acc;
}

}  // namespace

hipError_t launch_gemm1_f32(const GroupedArgs& a, hipStream_t s) {
    const int64_t rows = a.TK + (a.Is > 0 ? a.T : 0);
    if (rows == 0) return hipSuccess;
    const int32_t N = max(a.I, a.Is);
    hipLaunchKernelGGL(gemm1_f32, dim3((unsigned)((rows + 3) / 4), (N + 63) / 64), dim3(64, 4), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm2_f32(const GroupedArgs& a, hipStream_t s) {
    const int64_t rows = a.TK + (a.Is > 0 ? a.T : 0);
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm2_f32, dim3((unsigned)((rows + 3) / 4), (a.H + 63) / 64), dim3(64, 4), 0, s, a);
    return hipGetLastError();
}

}  // namespace dsmoe
