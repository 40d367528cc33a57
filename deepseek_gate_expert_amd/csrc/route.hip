// route.hip - the DeepSeek gate (and its softmax sibling), one wavefront (64 lanes) per token.
//
// Page: "feat(engine): E1 DeepSeek-style MoE gate (sigmoid, group top-k, bias) (#108)",
// sections "API" and "Algorithm" (S1 bias selects but does not weigh, S2 norm only for
// top_k > 1, S5 top-2 group sum, D7 no masking when no group is dropped), and the reviews
// (dropped groups are set to 0.0, not -inf).
//
// Lane l owns the P consecutive experts e = l*P + i (P = 1, 2, 4, 8 or 16, so E <= 64*P).
// Per token:
//   1. s = 1 / (1 + exp(-logit)) in fp32 (exp below), b = s + bias.
//   2. Groups (only when n_group > 1 and topk_group < n_group).  When a group is a
//      power-of-two run of L lanes (Eg = L*P), each lane folds its P values into a top-2 pair
//      and the pairs are merged by a butterfly over the L lanes with DPP (quad_perm,
//      row_half_mirror, row_mirror) and ds_swizzle; otherwise the group scores are formed
//      from an LDS copy of b.  Group score = top1 + top2 (duplicates count).  A group is
//      kept when fewer than topk_group groups beat it (higher score, or equal score and lower
//      index); experts of the other groups get b = 0.0.
//   3. Top-k: k rounds of a wave-wide maximum of 64-bit keys (value key << 32 | ~index), so
//      ties go to the lower index and the output is ordered by b descending, index ascending.
//      The value key maps fp32 to uint32 monotonically with -0 == +0 and NaN lowest.
//   4. w_j = s[inds_j]; if top_k > 1 and norm: S = ((w_0 + w_1) + w_2) + ..., w_j = w_j / S;
//      then w_j = w_j * routed_scaling_factor.  Lane j writes output j.
//
// Softmax gate (mode 3): ex = exp(logit - max over the row) ranks the experts (same 64-bit
// keys, so ties go to the lower index); w_j = ex[inds_j] / (sum of all ex), then
// w_j = w_j / (left-to-right sum of the w_j) always; no bias, groups or scale.
//
// exp: Cody & Waite range reduction with a degree-7 Taylor polynomial (W. J. Cody, W. Waite,
// "Software Manual for the Elementary Functions", 1980), evaluated with exactly these fp32
// operations, no contraction:
//   x > 0x1.62e430p+6 -> +inf;  x < -0x1.5d589ep+6 -> 0;  NaN -> NaN;
//   n = rint(x * 0x1.715476p+0);  r = fma(-n, 0x1.62e4p-1, x);  r = fma(-n, 0x1.7f7d1cp-20, r);
//   p = 0x1.a01a02p-13; p = fma(p,r,0x1.6c16c2p-10); p = fma(p,r,0x1.111112p-7);
//   p = fma(p,r,0x1.555556p-5); p = fma(p,r,0x1.555556p-3); p = fma(p,r,0.5);
//   p = fma(p,r,1); p = fma(p,r,1);  result = ldexp(p, n).
// The division 1/(1+e) is IEEE correctly rounded (HIP's default for fp32 division).
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

constexpr int WAVES = 4;  // tokens per 256-thread workgroup

// monotone fp32 -> uint32: larger value, larger key; -0 and +0 share a key; NaN is 0 (lowest)
__device__ __forceinline__ uint32_t vkey(float v) {
    if (v != v) return 0u;
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float vkey_inv(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within each 16 lanes
constexpr int SWZ_XOR16 = 0x401F;      // ds_swizzle bitmask mode: lane ^ 16 within 32

// Exchange with the butterfly partner of stage `st` (partners 1, 2, 4, 8, 16, 32 lanes away in
// the sense that after stages 0..st every lane holds the reduction over its 2^(st+1) lanes).
__device__ __forceinline__ uint32_t partner(uint32_t v, int st) {
    switch (st) {
        case 0: return dpp<DPP_XOR1>(v);
        case 1: return dpp<DPP_XOR2>(v);
        case 2: return dpp<DPP_HALF_MIRROR>(v);
        case 3: return dpp<DPP_MIRROR>(v);
        case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, SWZ_XOR16);
        default: return (uint32_t)__shfl_xor((int)v, 32);
    }
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int st = 0; st < 6; ++st) {
        const uint32_t hi = partner((uint32_t)(v >> 32), st);
        const uint32_t lo = partner((uint32_t)v, st);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ void top2_merge(uint32_t& m1, uint32_t& m2, uint32_t o1, uint32_t o2) {
    const uint32_t hi = m1 > o1 ? m1 : o1;
    const uint32_t lo = m1 > o1 ? o1 : m1;
    const uint32_t s2 = m2 > o2 ? m2 : o2;
    m1 = hi;
    m2 = lo > s2 ? lo : s2;
}

struct RouteArgs {
    const float* logits;
    const float* bias;
    int32_t* inds;
    float* scores;
    int64_t T;
    int32_t E, K, G, TG, norm;
    float rsf;
    int32_t mode;  // 0: no group masking, 1: lane-segment groups, 2: LDS groups, 3: softmax gate
    int32_t L;     // lanes per group in mode 1
};

template <int P>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    __shared__ float lds_b[WAVES][MOE_MAX_EXPERTS];
    __shared__ uint32_t lds_gk[WAVES][MOE_MAX_EXPERTS / 2];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * WAVES + wave;
    if (t >= a.T) return;  // wave-uniform; no workgroup barrier below
    const int32_t E = a.E;

    float sg[P];
    uint32_t bk[P];  // value keys of the biased scores (softmax: of the exponentials)
    float s_all = 0.0f;  // softmax: sum of the exponentials over all experts
    if (a.mode != 3) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int32_t e = lane * P + i;
            if (e < E) {
                sg[i] = sigmoid_cw(a.logits[t * E + e]);
                bk[i] = vkey(sg[i] + a.bias[e]);
            } else {
                sg[i] = 0.0f;
                bk[i] = 0u;
            }
        }
    } else {
        // softmax gate: ex = exp(logit - max) ranks the experts; the weights are ex / sum(ex),
        // renormalised over the selection below
        float lg[P];
        float m = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int32_t e = lane * P + i;
            lg[i] = e < E ? a.logits[t * E + e] : -__builtin_inff();
            m = lg[i] > m ? lg[i] : m;
        }
        for (int off = 32; off > 0; off >>= 1) {
            const float o = __shfl_xor(m, off);
            m = o > m ? o : m;
        }
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            if (lane * P + i < E) {
                sg[i] = exp_cw(lg[i] - m);
                bk[i] = vkey(sg[i]);
                part = part + sg[i];
            } else {
                sg[i] = 0.0f;
                bk[i] = 0u;
            }
        }
        for (int off = 32; off > 0; off >>= 1) part = part + __shfl_xor(part, off);
        s_all = part;
    }

    if (a.mode == 1) {
        // top-2 of my P values (all in one group), then a butterfly over the group's L lanes
        uint32_t m1 = 0u, m2 = 0u;
#pragma unroll
        for (int i = 0; i < P; ++i) top2_merge(m1, m2, bk[i], 0u);
        for (int st = 0; (1 << st) < a.L; ++st) {
            const uint32_t o1 = partner(m1, st);
            const uint32_t o2 = partner(m2, st);
            top2_merge(m1, m2, o1, o2);
        }
        const uint32_t gk = vkey(vkey_inv(m1) + vkey_inv(m2));
        const int32_t g = lane / a.L;
        int32_t rank = 0;
        for (int32_t q = 0; q < a.G; ++q) {
            const uint32_t ok = (uint32_t)__shfl((int)gk, q * a.L);
            rank += (ok > gk) || (ok == gk && q < g);
        }
        if (rank >= a.TG) {
#pragma unroll
            for (int i = 0; i < P; ++i) bk[i] = (lane * P + i < E) ? vkey(0.0f) : 0u;
        }
    } else if (a.mode == 2) {
        const int32_t Eg = E / a.G;
#pragma unroll
        for (int i = 0; i < P; ++i)
            if (lane * P + i < E) lds_b[wave][lane * P + i] = vkey_inv(bk[i]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int32_t g = lane; g < a.G; g += 64) {
            uint32_t m1 = 0u, m2 = 0u;
            for (int32_t e = g * Eg; e < (g + 1) * Eg; ++e) top2_merge(m1, m2, vkey(lds_b[wave][e]), 0u);
            lds_gk[wave][g] = vkey(vkey_inv(m1) + vkey_inv(m2));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int32_t e = lane * P + i;
            if (e >= E) continue;
            const int32_t g = e / Eg;
            const uint32_t gk = lds_gk[wave][g];
            int32_t rank = 0;
            for (int32_t q = 0; q < a.G; ++q) {
                const uint32_t ok = lds_gk[wave][q];
                rank += (ok > gk) || (ok == gk && q < g);
            }
            if (rank >= a.TG) bk[i] = vkey(0.0f);
        }
    }

    uint64_t key[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t e = (uint32_t)(lane * P + i);
        key[i] = ((int32_t)e < E) ? (((uint64_t)bk[i] << 32) | (uint32_t)~e) : 0ull;
    }
    float S = 0.0f, my_w = 0.0f;
    int32_t my_e = 0;
    for (int32_t j = 0; j < a.K; ++j) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < P; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int32_t esel = (int32_t)~(uint32_t)best;
        const int32_t owner = esel / P;
        float sv = 0.0f;
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < P; ++i)
                if (esel == lane * P + i) {
                    sv = sg[i];
                    key[i] = 0ull;
                }
        }
        const float wraw = __shfl(sv, owner);
        const float wj = a.mode == 3 ? wraw / s_all : wraw;
        S = (j == 0) ? wj : S + wj;
        if (lane == j) {
            my_e = esel;
            my_w = wj;
        }
    }
    if (a.mode == 3) {
        my_w = my_w / S;  // always renormalised, no scale
    } else {
        if (a.K > 1 && a.norm) my_w = my_w / S;
        my_w = my_w * a.rsf;
    }
    if (lane < a.K) {
        a.inds[t * a.K + lane] = my_e;
        a.scores[t * a.K + lane] = my_w;
    }
}

template <int P>
hipError_t launch_p(const RouteArgs& a, hipStream_t s) {
    const unsigned blocks = (unsigned)((a.T + WAVES - 1) / WAVES);
    hipLaunchKernelGGL(route_kernel<P>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, int64_t T, int32_t E, const float* bias, const moe_route_params& p,
                        int32_t* inds, float* scores, hipStream_t s) {
    if (T == 0) return hipSuccess;
    int P = 1;
    while (64 * P < E) P *= 2;
    RouteArgs a;
    a.logits = logits;
    a.bias = bias;
    a.inds = inds;
    a.scores = scores;
    a.T = T;
    a.E = E;
    a.K = p.top_k;
    a.G = p.n_group;
    a.TG = p.topk_group;
    a.norm = p.norm_topk_prob ? 1 : 0;
    a.rsf = p.routed_scaling_factor;
    a.mode = 0;
    a.L = 1;
    if (p.n_group > 1 && p.topk_group < p.n_group) {
        const int32_t Eg = E / p.n_group;
        const int32_t L = Eg / P;
        const bool pow2 = L >= 1 && (L & (L - 1)) == 0 && L <= 64;
        if (Eg % P == 0 && pow2 && E % P == 0) {
            a.mode = 1;
            a.L = L;
        } else {
            a.mode = 2;
        }
    }
    switch (P) {
        case 1: return launch_p<1>(a, s);
        case 2: return launch_p<2>(a, s);
        case 4: return launch_p<4>(a, s);
        case 8: return launch_p<8>(a, s);
        default: return launch_p<16>(a, s);
    }
}

hipError_t launch_route_softmax(const float* logits, int64_t T, int32_t E, int32_t K, int32_t* inds, float* scores,
                                hipStream_t s) {
    if (T == 0) return hipSuccess;
    int P = 1;
    while (64 * P < E) P *= 2;
    RouteArgs a;
    a.logits = logits;
    a.bias = nullptr;
    a.inds = inds;
    a.scores = scores;
    a.T = T;
    a.E = E;
    a.K = K;
    a.G = 1;
    a.TG = 1;
    a.norm = 1;
    a.rsf = 1.0f;
    a.mode = 3;
    a.L = 1;
    switch (P) {
        case 1: return launch_p<1>(a, s);
        case 2: return launch_p<2>(a, s);
        case 4: return launch_p<4>(a, s);
        case 8: return launch_p<8>(a, s);
        default: return launch_p<16>(a, s);
    }
}

}  // namespace dsmoe
