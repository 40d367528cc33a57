// experts.hip - grouped SwiGLU expert GEMMs on bf16 MFMA (bf16 or 4-bit weights).
//
// Role: the per-expert matmuls that gather_mm / gather_qmm perform in the reference design
// (page "Epic: Engine Inference Core Stage E - MoE + hybrid families", opening paragraph), with
// the SwiGLU of the expert MLP fused into the first GEMM's epilogue:
//   GEMM-1: h[r, n] = bf16( silu(x[tok(r)] . W_gate[g, n]) * (x[tok(r)] . W_up[g, n]) )
//   GEMM-2: o[r, n] = bf16( h[r] . W_down[g, n] )
// for every row r of group g (rows come from the dispatch; group E is the shared expert, whose
// rows TK + t are the tokens in order).
//
// This file holds the weight-streaming kernel ("stream"): one wavefront owns 16 output
// columns of one group and walks the whole reduction axis once per 64-row chunk of the
// group, so weights are read from HBM exactly once when a group has at most 64 rows -- the
// decode regime, where the layer is bound by HBM bandwidth.  Each lane loads 64 contiguous
// bytes of its weight row per 128-element step (16-byte loads) and the same k range of its
// activation row; the four 16-byte pieces feed four v_mfma_f32_16x16x32_bf16.  The k index
// inside a step is permuted identically for both operands, so the sum is unchanged.
// MFMA 16x16x32 bf16 operand layout: lane l supplies row/column (l % 16) and eight
// consecutive k values of block (l / 16); result element v of lane l is row 4*(l/16)+v,
// column l % 16.
//
// 4-bit weights (affine, groups of 64 along the input axis): each lane loads the 16 bytes of
// codes covering its 32 k values plus that group's bf16 scale and offset, and forms
// bf16(s*q + b) in registers before the MFMA.
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

enum { WF_BF16 = 0, WF_Q4 = 1 };

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s, float b) {
    uint4 r;
    uint32_t* rp = (uint32_t*)&r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = __builtin_fmaf(s, (float)((w >> (8 * j)) & 0xFu), b);
        const float hi = __builtin_fmaf(s, (float)((w >> (8 * j + 4)) & 0xFu), b);
        rp[j] = pack_bf16x2(lo, hi);
    }
    return as_bf16x8(r);
}

// Weight operand source for one output column (row of the weight matrix).
struct WRow {
    const bf16_t* w;   // bf16 row (WF_BF16)
    const uint32_t* q; // packed codes row (WF_Q4)
    const bf16_t* s;   // scale row (WF_Q4)
    const bf16_t* b;   // offset row (WF_Q4)
};

// NP pieces of 8 k values starting at k (8*NP contiguous elements of the row)
template <int WF, int NP>
__device__ __forceinline__ void load_w(const WRow& r, int k, bf16x8 (&out)[4]) {
    if constexpr (WF == WF_BF16) {
        const uint4* p = (const uint4*)(r.w + k);
#pragma unroll
        for (int i = 0; i < NP; ++i) out[i] = as_bf16x8(p[i]);
    } else {
        const float s = bf16_to_f32(r.s[k >> 6]);
        const float b = bf16_to_f32(r.b[k >> 6]);
        if constexpr (NP == 4) {
            const uint4 w = *(const uint4*)(r.q + (k >> 3));
            out[0] = dequant8(w.x, s, b);
            out[1] = dequant8(w.y, s, b);
            out[2] = dequant8(w.z, s, b);
            out[3] = dequant8(w.w, s, b);
        } else {
            const uint2 w = *(const uint2*)(r.q + (k >> 3));
            out[0] = dequant8(w.x, s, b);
            out[1] = dequant8(w.y, s, b);
        }
    }
}

template <int NP>
__device__ __forceinline__ void load_a(const bf16_t* row, int k, bf16x8 (&out)[4]) {
    if (row) {
        const uint4* p = (const uint4*)(row + k);
#pragma unroll
        for (int i = 0; i < NP; ++i) out[i] = as_bf16x8(p[i]);
    } else {
#pragma unroll
        for (int i = 0; i < NP; ++i) out[i] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
}

__device__ __forceinline__ void group_rows(const GroupedArgs& a, int32_t g, int32_t& r0, int32_t& cnt) {
    if (g < a.E) {
        r0 = a.offsets[g];
        cnt = a.offsets[g + 1] - r0;
    } else {
        r0 = a.TK;
        cnt = (int32_t)a.T;
    }
}

__device__ __forceinline__ int32_t row_token(const GroupedArgs& a, int32_t r) {
    return r < a.TK ? a.sorted_slot[r] / a.K : r - a.TK;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

template <int WF>
__device__ __forceinline__ WRow weight_row(const GroupedArgs& a, int sel, int32_t g, bool shared, int32_t n,
                                           int32_t out_dim, int32_t in_dim) {
    // sel: 0 gate, 1 up, 2 down
    WRow r = {nullptr, nullptr, nullptr, nullptr};
    if (shared) {
        const bf16_t* base = (const bf16_t*)(sel == 0 ? a.swg : sel == 1 ? a.swu : a.swd);
        r.w = base + (int64_t)n * in_dim;
        return r;
    }
    const int64_t row = (int64_t)g * out_dim + n;
    if constexpr (WF == WF_BF16) {
        const bf16_t* base = (const bf16_t*)(sel == 0 ? a.wg : sel == 1 ? a.wu : a.wd);
        r.w = base + row * in_dim;
    } else {
        const uint32_t* base = (const uint32_t*)(sel == 0 ? a.wg : sel == 1 ? a.wu : a.wd);
        r.q = base + row * (in_dim / 8);
        r.s = (sel == 0 ? a.sg : sel == 1 ? a.su : a.sd) + row * (in_dim / 64);
        r.b = (sel == 0 ? a.bg : sel == 1 ? a.bu : a.bd) + row * (in_dim / 64);
    }
    return r;
}

// One reduction step of NP*32 k values (NP = 4 -> 128, NP = 2 -> 64) for GEMM-1.
template <int WF, int NP>
__device__ __forceinline__ void step1(const WRow& rg, const WRow& ru, const bf16_t* const (&arow)[4], int nrb,
                                      int k, f32x4 (&ag)[4], f32x4 (&au)[4]) {
    bf16x8 bgv[4], buv[4];
    load_w<WF, NP>(rg, k, bgv);
    load_w<WF, NP>(ru, k, buv);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        if (rb >= nrb) break;
        bf16x8 av[4];
        load_a<NP>(arow[rb], k, av);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            ag[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bgv[i], ag[rb], 0, 0, 0);
            au[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], buv[i], au[rb], 0, 0, 0);
        }
    }
}

template <int WF, int NP>
__device__ __forceinline__ void step2(const WRow& rd, const bf16_t* const (&arow)[4], int nrb, int k,
                                      f32x4 (&ac)[4]) {
    bf16x8 bv[4];
    load_w<WF, NP>(rd, k, bv);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        if (rb >= nrb) break;
        bf16x8 av[4];
        load_a<NP>(arow[rb], k, av);
#pragma unroll
        for (int i = 0; i < NP; ++i) ac[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[i], ac[rb], 0, 0, 0);
    }
}

// grid: x = ceil(max(I, Is) / 64) column blocks, y = groups [g0, g0 + gridDim.y)
template <int WF>
__global__ __launch_bounds__(256) void gemm1_stream(GroupedArgs a, int32_t g0) {
    const int32_t g = g0 + blockIdx.y;
    int32_t r0, cnt;
    group_rows(a, g, r0, cnt);
    if (cnt <= 0 || cnt > a.stream_max_rows) return;
    const bool shared = g == a.E;
    const int32_t N = shared ? a.Is : a.I;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int32_t n0 = (blockIdx.x * 4 + wave) * 16;
    if (n0 >= N) return;  // wave-uniform
    const int32_t H = a.H;
    const int32_t col = n0 + (lane & 15);
    const WRow rg = weight_row<WF>(a, 0, g, shared, col, N, H);
    const WRow ru = weight_row<WF>(a, 1, g, shared, col, N, H);
    const bf16_t* x = (const bf16_t*)a.x;
    bf16_t* h = (bf16_t*)a.h;
    const int kq4 = (lane >> 4) * 32, kq2 = (lane >> 4) * 16;
    const int32_t Hmain = H & ~127;

    for (int32_t m0 = 0; m0 < cnt; m0 += 64) {
        const int nrb = min(4, (cnt - m0 + 15) >> 4);
        const bf16_t* arow[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int32_t rr = m0 + rb * 16 + (lane & 15);
            arow[rb] = (rb < nrb && rr < cnt) ? x + (int64_t)row_token(a, r0 + rr) * H : nullptr;
        }
        f32x4 ag[4], au[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) ag[rb] = au[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int32_t k = 0; k < Hmain; k += 128) step1<WF, 4>(rg, ru, arow, nrb, k + kq4, ag, au);
        if (Hmain < H) step1<WF, 2>(rg, ru, arow, nrb, Hmain + kq2, ag, au);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            if (rb >= nrb) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int32_t rr = m0 + rb * 16 + (lane >> 4) * 4 + v;
                if (rr < cnt) h[(int64_t)(r0 + rr) * a.ldh + col] = f32_to_bf16(silu_f(ag[rb][v]) * au[rb][v]);
            }
        }
    }
}

// grid: x = H / 64 column blocks, y = groups
template <int WF>
__global__ __launch_bounds__(256) void gemm2_stream(GroupedArgs a, int32_t g0) {
    const int32_t g = g0 + blockIdx.y;
    int32_t r0, cnt;
    group_rows(a, g, r0, cnt);
    if (cnt <= 0 || cnt > a.stream_max_rows) return;
    const bool shared = g == a.E;
    const int32_t KD = shared ? a.Is : a.I;  // reduction length
    const int32_t H = a.H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int32_t n0 = (blockIdx.x * 4 + wave) * 16;
    if (n0 >= H) return;
    const int32_t col = n0 + (lane & 15);
    const WRow rd = weight_row<WF>(a, 2, g, shared, col, H, KD);
    const bf16_t* h = (const bf16_t*)a.h;
    bf16_t* o = (bf16_t*)a.o;
    const int kq4 = (lane >> 4) * 32, kq2 = (lane >> 4) * 16;
    const int32_t Kmain = KD & ~127;

    for (int32_t m0 = 0; m0 < cnt; m0 += 64) {
        const int nrb = min(4, (cnt - m0 + 15) >> 4);
        const bf16_t* arow[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int32_t rr = m0 + rb * 16 + (lane & 15);
            arow[rb] = (rb < nrb && rr < cnt) ? h + (int64_t)(r0 + rr) * a.ldh : nullptr;
        }
        f32x4 ac[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) ac[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int32_t k = 0; k < Kmain; k += 128) step2<WF, 4>(rd, arow, nrb, k + kq4, ac);
        if (Kmain < KD) step2<WF, 2>(rd, arow, nrb, Kmain + kq2, ac);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            if (rb >= nrb) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int32_t rr = m0 + rb * 16 + (lane >> 4) * 4 + v;
                if (rr < cnt) o[(int64_t)(r0 + rr) * H + col] = f32_to_bf16(ac[rb][v]);
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm1_bf16(const GroupedArgs& a, int32_t g0, int32_t g1, int32_t wdt, hipStream_t s) {
    if (g1 <= g0) return hipSuccess;
    const int32_t N = max(a.I, a.Is);
    const dim3 grid((N + 63) / 64, g1 - g0);
    if (wdt == MOE_Q4G64)
        hipLaunchKernelGGL(gemm1_stream<WF_Q4>, grid, dim3(256), 0, s, a, g0);
    else
        hipLaunchKernelGGL(gemm1_stream<WF_BF16>, grid, dim3(256), 0, s, a, g0);
    return hipGetLastError();
}

hipError_t launch_gemm2_bf16(const GroupedArgs& a, int32_t g0, int32_t g1, int32_t wdt, hipStream_t s) {
    if (g1 <= g0) return hipSuccess;
    const dim3 grid((a.H + 63) / 64, g1 - g0);
    if (wdt == MOE_Q4G64)
        hipLaunchKernelGGL(gemm2_stream<WF_Q4>, grid, dim3(256), 0, s, a, g0);
    else
        hipLaunchKernelGGL(gemm2_stream<WF_BF16>, grid, dim3(256), 0, s, a, g0);
    return hipGetLastError();
}

}  // namespace dsmoe
