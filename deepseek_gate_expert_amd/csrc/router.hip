// router.hip - router logits in a fixed fp32 order.
//
// logits[t,e] = sum_k x[t,k] * W[e,k] (+ offset[e]): the linear layer in front of the gate
// (gate page "feat(engine): E1 DeepSeek-style MoE gate ...", merge recommendation: router
// linear, then route; "Algorithm": the gate takes fp32 logits).
//
// Every output element is accumulated by one fused multiply-add per k, k ascending, starting
// from +0.0f, then one fp32 add of the offset.  Because the order is fixed the logits are
// reproducible bit for bit, which keeps the expert selection stable.  That rules out MFMA
// (its internal summation order is not specified), so these are VALU kernels in which the k
// loop of an output is never split across threads and the zero tail of a partial k chunk is
// never fed to an FMA.
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

template <typename TA>
__device__ __forceinline__ float ld_act(const TA* p, int64_t i);
template <>
__device__ __forceinline__ float ld_act<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_act<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// 8 consecutive activations as loaded (16 or 32 bytes), widened to fp32 only when staged: a
// conversion right after the load would make the load's wait come first, and the staging
// loads would then no longer run ahead of the multiply.
template <typename TA>
struct Raw8 {
    u32x4 q[sizeof(TA) / 2];
};

// elements [i, i + 8) of row `row` (length H), zero past the end of the row
template <typename TA>
__device__ __forceinline__ void raw8_load(const TA* row, int32_t i, int32_t H, bool vec, Raw8<TA>& r) {
    if (vec && i + 8 <= H) {
#pragma unroll
        for (int v = 0; v < (int)sizeof(TA) / 2; ++v) r.q[v] = *(const u32x4*)(row + i + v * (16 / (int)sizeof(TA)));
        return;
    }
    if constexpr (sizeof(TA) == 2) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = i + 2 * m < H ? row[i + 2 * m] : 0u, hi = i + 2 * m + 1 < H ? row[i + 2 * m + 1] : 0u;
            r.q[0][m] = lo | (hi << 16);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) r.q[j >> 2][j & 3] = i + j < H ? __float_as_uint(row[i + j]) : 0u;
    }
}

// element j of a Raw8 as fp32 (exact)
template <typename TA>
__device__ __forceinline__ float raw8_at(const Raw8<TA>& r, int j) {
    if constexpr (sizeof(TA) == 2) return __uint_as_float((j & 1) ? (r.q[0][j >> 1] & 0xffff0000u) : (r.q[0][j >> 1] << 16));
    else return __uint_as_float(r.q[j >> 2][j & 3]);
}

// Many tokens: 256 threads, MT x NT register tile per thread (BM = 16 MT tokens x BN = 16 NT
// experts per workgroup), k chunks of KC staged in LDS as fp32 (k-major), double buffered.  The
// global loads run RD chunks ahead in a ring of raw registers, so with x coming from HBM (as in
// a layer) their latency stays hidden.  Full chunks run a fully unrolled k loop, so the LDS
// reads of later k steps issue ahead of the FMAs.
constexpr int RD = 3;

template <typename TA, int MT, int NT, int KC>
__global__ __launch_bounds__(256) void router_kernel(const TA* __restrict__ x, const TA* __restrict__ w,
                                                     const float* __restrict__ off, float* __restrict__ logits,
                                                     int64_t T, int32_t H, int32_t E) {
    constexpr int BM = 16 * MT, BN = 16 * NT;
    constexpr int LPR = KC / 8;                                     // 8-element loads per row
    constexpr int XL = BM * LPR / 256, WL = BN * LPR / 256;  // 8-element loads per thread
    static_assert(XL >= 1 && WL >= 1 && BM * LPR % 256 == 0 && BN * LPR % 256 == 0,
                  "tile does not fit the staging layout");
    __shared__ float xs[2][KC][BM + 4];
    __shared__ float ws[2][KC][BN + 4];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int32_t n0 = blockIdx.y * BN;
    const bool vec = (H % 8) == 0;

    // staging assignment: load i of this thread covers row (tid + 256 i) / LPR, k (tid % LPR) * 8
    const TA* xrow[XL];
    const TA* wrow[WL];
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        int64_t t = m0 + (tid + 256 * i) / LPR;
        xrow[i] = x + (t < T ? t : T - 1) * H;
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
        int32_t e = n0 + (tid + 256 * i) / LPR;
        wrow[i] = w + (int64_t)(e < E ? e : E - 1) * H;
    }
    const int kq = (tid % LPR) * 8;
    Raw8<TA> xq[RD][XL], wq[RD][WL];

    float acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = 0.0f;

    const int nch = (H + KC - 1) / KC;
    auto load = [&](int u, int c) {
#pragma unroll
        for (int i = 0; i < XL; ++i) raw8_load(xrow[i], c * KC + kq, H, vec, xq[u][i]);
#pragma unroll
        for (int i = 0; i < WL; ++i) raw8_load(wrow[i], c * KC + kq, H, vec, wq[u][i]);
    };
#pragma unroll
    for (int u = 0; u < RD; ++u)
        if (u < nch) load(u, u);
    for (int c0 = 0; c0 < nch; c0 += RD) {
#pragma unroll
        for (int u = 0; u < RD; ++u) {  // chunk c lives in ring slot c % RD
            const int c = c0 + u;
            if (c >= nch) break;
            const int b = c & 1;
#pragma unroll
            for (int i = 0; i < XL; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) xs[b][kq + j][(tid + 256 * i) / LPR] = raw8_at(xq[u][i], j);
#pragma unroll
            for (int i = 0; i < WL; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) ws[b][kq + j][(tid + 256 * i) / LPR] = raw8_at(wq[u][i], j);
            __syncthreads();
            if (c + RD < nch) load(u, c + RD);
            auto step = [&](int k) {
                float a[MT], bb[NT];
#pragma unroll
                for (int i = 0; i < MT; ++i) a[i] = xs[b][k][ty * MT + i];
#pragma unroll
                for (int j = 0; j < NT; ++j) bb[j] = ws[b][k][tx * NT + j];
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[i][j] = __builtin_fmaf(a[i], bb[j], acc[i][j]);
            };
            const int kc = min(KC, H - c * KC);  // the zero tail of the last chunk is never used
            if (kc == KC) {
#pragma unroll
                for (int k = 0; k < KC; ++k) step(k);
            } else {
                for (int k = 0; k < kc; ++k) step(k);
            }
            // buffer b is rewritten two chunks later, after the next chunk's barrier
        }
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

// Few tokens: a workgroup is ONE wave that computes one expert for 64 tokens (lane = token),
// so even a single 64-token batch spreads over E workgroups.  Each lane streams its own token's
// row of x and the (wave-uniform) expert row in chunks of 32 k, kept in a ring of four register
// buffers so that three chunks of loads are in flight while the current one is multiplied.
// One accumulator per lane, k ascending.  grid: x = E, y = ceil(T / 64).
//
// The ring looks only 1.5 cache lines ahead, too little to hide HBM latency when x and the
// expert row are not in cache (as in a layer, after the previous layer's weights have streamed
// through).  So each wave first touches, with loads spread over its lanes, its whole expert row
// (16 loads of 1 KB) and one slice of the 64 token rows: waves of one block that share an XCD
// (expert ids congruent mod 8, with E a multiple of 8) split those rows between them.  The
// values are discarded; the ring then hits in cache.  All twenty touching loads are issued
// before any is waited for (lanes past a row's end re-touch its last line), so they cost about
// one memory latency: loading them under per-lane conditions made the compiler wait for each in
// turn (67 against 61 us for the DeepSeek-V3 decode batch, T = 64).
constexpr int GV_CK = 32;

template <typename TA>
__device__ __forceinline__ uint32_t warm_rows(const TA* x, const TA* wr, int64_t T, int32_t H, int32_t E,
                                              int32_t e, int lane) {
    uint32_t sink = 0;
    if (H % 8 != 0 || E < 64 || (E & 7) != 0) return sink;  // 16-byte aligned rows; 8+ waves per XCD
    const int64_t wbytes = (int64_t)H * sizeof(TA);
    const char* wb = (const char*)wr;
    uint32_t got[20];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int64_t o = (int64_t)i * 1024 + lane * 16;
        o = o + 16 <= wbytes ? o : wbytes - 16;
        got[i] = *(const uint32_t*)(wb + o);  // one word per lane touches each 128-byte line
    }
    const int64_t t0 = (int64_t)blockIdx.y * 64;
    const int64_t rows = T - t0 < 64 ? T - t0 : 64;
    const int64_t xbytes = rows * H * (int64_t)sizeof(TA);  // the block's rows are contiguous
    const int64_t lines = (xbytes + 127) / 128;
    const int32_t q = E >> 3;                                // waves of this block on one XCD
    const int64_t per = (lines + q - 1) / q;
    const int64_t l0 = (int64_t)(e >> 3) * per;
    const char* xb = (const char*)(x + t0 * H);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t j = i * 64 + lane;
        int64_t l = l0 + (j < per ? j : per - 1);
        l = l < lines ? l : lines - 1;
        got[16 + i] = *(const uint32_t*)(xb + l * 128);
    }
#pragma unroll
    for (int i = 0; i < 20; ++i) sink ^= got[i];
    return sink;
}

template <typename TA>
__device__ __forceinline__ void fma_chunk(const u32x4 (&xq)[GV_CK * sizeof(TA) / 16],
                                          const u32x4 (&wq)[GV_CK * sizeof(TA) / 16], float& acc);
template <>
__device__ __forceinline__ void fma_chunk<bf16_t>(const u32x4 (&xq)[4], const u32x4 (&wq)[4], float& acc) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = __builtin_fmaf(__uint_as_float(xq[v][i] << 16), __uint_as_float(wq[v][i] << 16), acc);
            acc = __builtin_fmaf(__uint_as_float(xq[v][i] & 0xffff0000u), __uint_as_float(wq[v][i] & 0xffff0000u),
                                 acc);
        }
}
template <>
__device__ __forceinline__ void fma_chunk<float>(const u32x4 (&xq)[8], const u32x4 (&wq)[8], float& acc) {
#pragma unroll
    for (int v = 0; v < 8; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(__uint_as_float(xq[v][i]), __uint_as_float(wq[v][i]), acc);
}

template <typename TA>
__global__ __launch_bounds__(64) void router_gemv(const TA* __restrict__ x, const TA* __restrict__ w,
                                                  const float* __restrict__ off, float* __restrict__ logits,
                                                  int64_t T, int32_t H, int32_t E) {
    constexpr int NV = GV_CK * (int)sizeof(TA) / 16;  // 16-byte vectors per chunk
    const int lane = threadIdx.x;
    const int64_t t = (int64_t)blockIdx.y * 64 + lane;
    const int32_t e = blockIdx.x;
    const TA* xr = x + (t < T ? t : T - 1) * H;
    const TA* wr = w + (int64_t)e * H;
    const uint32_t sink = warm_rows<TA>(x, wr, T, H, E, e, lane);
    float acc = 0.0f;
    const int nch = H / GV_CK;
    if (H % GV_CK == 0) {
        u32x4 xb[4][NV], wb[4][NV];
#define DSMOE_GV_LOAD(SLOT, C)                                                       \
    do {                                                                             \
        _Pragma("unroll") for (int v_ = 0; v_ < NV; ++v_) {                          \
            xb[SLOT][v_] = *(const u32x4*)(xr + (C) * GV_CK + v_ * (16 / sizeof(TA))); \
            wb[SLOT][v_] = *(const u32x4*)(wr + (C) * GV_CK + v_ * (16 / sizeof(TA))); \
        }                                                                            \
    } while (0)
#pragma unroll
        for (int u = 0; u < 3; ++u)
            if (u < nch) DSMOE_GV_LOAD(u, u);
        for (int c = 0; c < nch; c += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (c + u + 3 < nch) DSMOE_GV_LOAD((u + 3) & 3, c + u + 3);
                if (c + u < nch) fma_chunk<TA>(xb[u], wb[u], acc);
            }
        }
#undef DSMOE_GV_LOAD
    } else {
        for (int32_t k = 0; k < H; ++k) acc = __builtin_fmaf(ld_act(xr, k), ld_act(wr, k), acc);
    }
    asm volatile("" ::"v"(sink));  // keeps the warming loads
    if (t < T) {
        float v = acc;
        if (off) v = v + off[e];
        logits[t * E + e] = v;
    }
}

template <typename TA>
hipError_t launch_gemv(const TA* x, const TA* w, int64_t T, int32_t H, int32_t E, const float* off, float* logits,
                       hipStream_t s) {
    const dim3 grid(E, (unsigned)((T + 63) / 64));
    hipLaunchKernelGGL(router_gemv<TA>, grid, dim3(64), 0, s, x, w, off, logits, T, H, E);
    return hipGetLastError();
}

template <typename TA, int MT, int NT, int KC>
hipError_t launch_t(const TA* x, const TA* w, int64_t T, int32_t H, int32_t E, const float* off, float* logits,
                    hipStream_t s) {
    const dim3 grid((unsigned)((T + 16 * MT - 1) / (16 * MT)), (E + 16 * NT - 1) / (16 * NT));
    hipLaunchKernelGGL((router_kernel<TA, MT, NT, KC>), grid, dim3(256), 0, s, x, w, off, logits, T, H, E);
    return hipGetLastError();
}

// Few tokens or few experts: one output per lane (GEMV shape).  Otherwise the largest register
// tile that still gives at least 256 workgroups (one per CU): 4 x 4 (64 x 64 logits per
// workgroup), then 2 x 4, then 2 x 2 with 64-k chunks.  The summation order is the same in all.
template <typename TA>
hipError_t route_shape(const TA* x, const TA* w, int64_t T, int32_t H, int32_t E, const float* off,
                       float* logits, hipStream_t s) {
    if (T <= 512 || E < 16) return launch_gemv<TA>(x, w, T, H, E, off, logits, s);
    const int64_t ecols = (E + 63) / 64;
    if (((T + 63) / 64) * ecols >= 256) return launch_t<TA, 4, 4, 32>(x, w, T, H, E, off, logits, s);
    if (((T + 31) / 32) * ecols >= 256) return launch_t<TA, 2, 4, 64>(x, w, T, H, E, off, logits, s);
    return launch_t<TA, 2, 2, 64>(x, w, T, H, E, off, logits, s);
}

}  // namespace

hipError_t launch_router(const void* x, const void* w, int32_t act, int64_t T, int32_t H, int32_t E,
                         const float* offset, float* logits, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (act == MOE_BF16) return route_shape<bf16_t>((const bf16_t*)x, (const bf16_t*)w, T, H, E, offset, logits, s);
    return route_shape<float>((const float*)x, (const float*)w, T, H, E, offset, logits, s);
}

}  // namespace dsmoe
