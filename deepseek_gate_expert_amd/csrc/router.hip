// router.hip - router logits in a fixed fp32 order.
//
// logits[t,e] = sum_k x[t,k] * W[e,k] (+ offset[e]): the linear layer in front of the gate
// (gate page "feat(engine): E1 DeepSeek-style MoE gate ...", merge recommendation: router
// linear, then route; "Algorithm": the gate takes fp32 logits).
//
// Every output element is accumulated by one fused multiply-add per k, k ascending, starting
// from +0.0f, then one fp32 add of the offset.  Because the order is fixed the logits are
// reproducible bit for bit, which keeps the expert selection stable.  That rules out the matrix
// instructions that sum several k inside (their internal order and rounding are not specified),
// but not the fp32 ones that take a single k (see router_mfma).  In every kernel the k loop of
// an output is never split across threads and the zero tail of a partial k chunk is never
// multiplied.
#include <type_traits>

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

// Many tokens, on the matrix cores.  v_mfma_f32_16x16x1_4b_f32 multiplies four independent
// 16 x 1 by 1 x 16 fp32 blocks and adds each product to its accumulator: one k per instruction,
// so every output receives exactly one multiply-add, C + a * b rounded once.  Checked on MI355X
// against fmaf for about 10^8 operand triples (bf16-valued and general fp32 operands, subnormal,
// infinite and NaN operands, signed zeros): the same bits in every case.  A chain of these
// instructions over k ascending, from +0.0f, is therefore the same fixed-order FMA chain as in
// the VALU kernel, at the matrix cores' fp32 rate (twice the non-packed vector rate).
//
// Workgroup: 64 tokens x 64 experts, four waves, wave w owning experts [16 w, 16 w + 16) of the
// tile for all 64 tokens: A operand lane l = token l (block l / 16 = tokens [16 b, 16 b + 16)),
// B operand lane l = expert 16 w + l % 16 (the same 16 experts in all four blocks).  Output
// register r of lane l: block r / 4, token 16 (r / 4) + 4 (l / 16) + r % 4, expert l % 16.
// Operands are staged as fp32 in LDS, [row][k] with rows padded by four floats so that the
// 16-byte reads of 16 consecutive rows fall in distinct banks; each 16-byte read supplies four
// consecutive k.  Three LDS buffers: while chunk c is multiplied, chunk c + 2 is widened into
// the buffer that chunk c - 1 used, and the first operands of chunk c + 1 (staged during chunk
// c - 1) are read before the end-of-chunk barrier, so that the barrier, the staging and the LDS
// latency stay off the matrix pipe's path as far as the schedule allows.  Global loads run
// RM_RD chunks ahead of the staging in raw registers.  Tiles are ordered so that the expert
// tiles of one token tile run on one XCD, where they share the token rows in L2.
constexpr int RM_KC = 32;          // k per staged chunk
constexpr int RM_LD = RM_KC + 4;   // LDS row stride in floats
constexpr int RM_NB = 3;           // LDS buffers
constexpr int RM_RD = 3;           // raw register ring (chunks)

template <typename TA, bool VEC>
__global__ __launch_bounds__(256) void router_mfma(const TA* __restrict__ x, const TA* __restrict__ w,
                                                   const float* __restrict__ off, float* __restrict__ logits,
                                                   int64_t T, int32_t H, int32_t E, int32_t ntt, int32_t nte) {
    __shared__ __attribute__((aligned(16))) float xs[RM_NB][64][RM_LD];
    __shared__ __attribute__((aligned(16))) float ws[RM_NB][64][RM_LD];
    // workgroup L runs on XCD L % 8; its position in that XCD's sequence picks the tile
    const int32_t L = blockIdx.x;
    const int32_t full = (ntt / 8) * 8 * nte;
    int32_t tt, te;
    if (L < full) {
        const int32_t q = L >> 3;
        tt = (q / nte) * 8 + (L & 7);
        te = q % nte;
    } else {
        const int32_t r = L - full;
        tt = (ntt / 8) * 8 + r / nte;
        te = r % nte;
    }
    const int64_t t0 = (int64_t)tt * 64;
    const int32_t e0 = te * 64;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

    // staging: thread tid loads 8 k of token row tid / 4 and of expert row tid / 4
    const int srow = tid >> 2, kq = (tid & 3) * 8;
    const int64_t st = t0 + srow;
    const int32_t se = e0 + srow;
    const TA* xrow = x + (st < T ? st : T - 1) * H;
    const TA* wrow = w + (int64_t)(se < E ? se : E - 1) * H;
    Raw8<TA> xq[RM_RD], wq[RM_RD];
    // With 8-aligned rows (VEC) every load is one unconditional 16-byte vector (two for fp32),
    // its start clamped to the row's last 8 elements; the k it then covers lie past the row's
    // end, where the staged values are never multiplied.  (Element loads under per-lane
    // conditions would make the compiler wait for every load in flight before each staging.)
    auto load = [&](int u, int c) {
        if constexpr (VEC) {
            const int32_t i = min(c * RM_KC + kq, H - 8);
#pragma unroll
            for (int v = 0; v < (int)sizeof(TA) / 2; ++v) {
                xq[u].q[v] = *(const u32x4*)(xrow + i + v * (16 / (int)sizeof(TA)));
                wq[u].q[v] = *(const u32x4*)(wrow + i + v * (16 / (int)sizeof(TA)));
            }
        } else {
            raw8_load(xrow, c * RM_KC + kq, H, false, xq[u]);
            raw8_load(wrow, c * RM_KC + kq, H, false, wq[u]);
        }
    };
    auto stage = [&](int u, int b) {
        f32x4 lo, hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo[j] = raw8_at(xq[u], j);
            hi[j] = raw8_at(xq[u], j + 4);
        }
        *(f32x4*)&xs[b][srow][kq] = lo;
        *(f32x4*)&xs[b][srow][kq + 4] = hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo[j] = raw8_at(wq[u], j);
            hi[j] = raw8_at(wq[u], j + 4);
        }
        *(f32x4*)&ws[b][srow][kq] = lo;
        *(f32x4*)&ws[b][srow][kq + 4] = hi;
    };

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    const int nch = (H + RM_KC - 1) / RM_KC, nfull = H / RM_KC;
    const int brow = 16 * wv + (lane & 15);
    // Chunk s is loaded into ring slot s % RM_RD and staged into buffer s % RM_NB.  Loads and
    // staging run unconditionally (a chunk index past the last one re-reads the last chunk, and
    // its staging fills a buffer that no later chunk reads), so the number of loads in flight is
    // the same on every path and the wait before a staging step can leave the later chunks'
    // loads in flight.
#pragma unroll
    for (int u = 0; u < RM_RD; ++u) load(u, min(u, nch - 1));
#pragma unroll
    for (int s0 = 0; s0 < 2; ++s0) {
        stage(s0, s0);
        load(s0, min(s0 + RM_RD, nch - 1));
    }
    __syncthreads();

    f32x4 av = *(const f32x4*)&xs[0][lane][0], bv = *(const f32x4*)&ws[0][brow][0];
    // chunk c (full) from buffer U = c % 3; staging of chunk c + 2 from slot (U + 2) % 3
    auto chunk = [&](auto U, int c) {
        constexpr int u = decltype(U)::value;
#pragma unroll
        for (int g = 0; g < RM_KC / 4; ++g) {
            f32x4 an, bn;
            if (g + 1 < RM_KC / 4) {
                an = *(const f32x4*)&xs[u][lane][4 * g + 4];
                bn = *(const f32x4*)&ws[u][brow][4 * g + 4];
            } else {  // chunk c + 1 was staged during chunk c - 1 (an unused read past the end is harmless)
                an = *(const f32x4*)&xs[(u + 1) % RM_NB][lane][0];
                bn = *(const f32x4*)&ws[(u + 1) % RM_NB][brow][0];
            }
            if (g == 2) {  // buffer (u + 2) % 3 last held chunk c - 1
                constexpr int su = (u + 2) % RM_RD;
                stage(su, (u + 2) % RM_NB);
                load(su, min(c + 2 + RM_RD, nch - 1));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x1f32(av[j], bv[j], acc, 0, 0, 0);
            av = an;
            bv = bn;
        }
        __syncthreads();  // buffer u is restaged during chunk c + 1; chunk c + 2 becomes visible
    };
    // whole triples in the loop (no exit inside an iteration, so every path into the loop has the
    // same loads in flight), then the remaining full chunks
    int c0 = 0;
    for (; c0 + RM_NB <= nfull; c0 += RM_NB) {
        chunk(std::integral_constant<int, 0>{}, c0);
        chunk(std::integral_constant<int, 1>{}, c0 + 1);
        chunk(std::integral_constant<int, 2>{}, c0 + 2);
    }
    if (c0 < nfull) chunk(std::integral_constant<int, 0>{}, c0);
    if (c0 + 1 < nfull) chunk(std::integral_constant<int, 1>{}, c0 + 1);
    if (nfull < nch) {  // partial last chunk: its zero tail is never used
        const int b = nfull % RM_NB, kc = H - nfull * RM_KC;
        for (int k = 0; k < kc; ++k)
            acc = __builtin_amdgcn_mfma_f32_16x16x1f32(xs[b][lane][k], ws[b][brow][k], acc, 0, 0, 0);
    }
    // the accumulators are read right after the last MFMA, possibly behind the tail branch:
    // issue the MFMA-to-VALU wait states explicitly before any of them is read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
    const int32_t e = e0 + 16 * wv + (lane & 15);
    if (e >= E) return;
    const float o = off ? off[e] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t t = t0 + 16 * (r >> 2) + 4 * (lane >> 4) + (r & 3);
        if (t >= T) continue;
        float v = acc[r];
        if (off) v = v + o;
        logits[t * E + e] = v;
    }
}

// Few tokens: a workgroup is ONE wave that computes one expert for 64 tokens (lane = token),
// so even a single 64-token batch spreads over E workgroups.  Each lane streams its own token's
// row of x and the (wave-uniform) expert row in chunks of 32 k, kept in a ring of four register
// buffers so that three chunks of loads are in flight while the current one is multiplied.
// One accumulator per lane, k ascending.  grid: x = E, y = ceil(T / 64).  (router_gemv_lds
// below serves the rows that fit in LDS; this kernel takes the others.)
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

// The same GEMV with the expert row widened once into LDS as fp32 (rows of up to 16384 k, k a
// multiple of 32).  In router_gemv the wave-uniform expert row goes through scalar loads, and
// scalar loads complete out of order: every use waits for all of them, including the chunks
// just prefetched, so the ring hides little.  Here each lane loads its share of the row once
// (all loads issued before any is waited for), widens it and writes it to LDS; the k loop reads
// it with broadcast 16-byte LDS reads one chunk ahead (two register sets in turn), and the
// token rows stream through a ring of four 32-k chunks whose loads are unconditional (a chunk
// past the last re-reads the last), so that the wait before a chunk counts only its own loads.
// Per k the loop issues two vector instructions (the widening of x and the FMA).  DeepSeek-V3
// decode batch (T = 64) in the layer: 61 us for router_gemv, 49.6 with the row in LDS, 44.5
// with its reads one chunk ahead; a ring of eight token-row chunks, or touching the token rows
// first as router_gemv does, was slower or no faster.
constexpr int GL_MAXH = 16384;

template <typename TA>
__global__ __launch_bounds__(64) void router_gemv_lds(const TA* __restrict__ x, const TA* __restrict__ w,
                                                      const float* __restrict__ off, float* __restrict__ logits,
                                                      int64_t T, int32_t H, int32_t E) {
    extern __shared__ __attribute__((aligned(16))) float wl[];  // the expert row, fp32
    constexpr int NV = GV_CK * (int)sizeof(TA) / 16;  // 16-byte vectors per chunk
    constexpr int PE = 16 / (int)sizeof(TA);          // elements per 16-byte piece
    const int lane = threadIdx.x;
    const int64_t t = (int64_t)blockIdx.y * 64 + lane;
    const int32_t e = blockIdx.x;
    const TA* xr = x + (t < T ? t : T - 1) * H;
    const TA* wr = w + (int64_t)e * H;
    const int nch = H / GV_CK;

    // the ring's first chunks, then the expert row in batches of 8 pieces per lane
    u32x4 xb[4][NV];
    auto ldx = [&](int slot, int c) {
        const int cc = min(c, nch - 1);
#pragma unroll
        for (int v = 0; v < NV; ++v) xb[slot][v] = *(const u32x4*)(xr + cc * GV_CK + v * PE);
    };
    ldx(0, 0);
    ldx(1, 1);
    ldx(2, 2);
    const int np = H / PE;  // pieces in the row
    for (int b0 = 0; b0 < np; b0 += 8 * 64) {
        u32x4 q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = *(const u32x4*)(wr + min(b0 + i * 64 + lane, np - 1) * PE);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int p = b0 + i * 64 + lane;
            if (p >= np) continue;
            if constexpr (sizeof(TA) == 2) {
                f32x4 lo, hi;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    lo[2 * j] = __uint_as_float(q[i][j] << 16);
                    lo[2 * j + 1] = __uint_as_float(q[i][j] & 0xffff0000u);
                    hi[2 * j] = __uint_as_float(q[i][j + 2] << 16);
                    hi[2 * j + 1] = __uint_as_float(q[i][j + 2] & 0xffff0000u);
                }
                *(f32x4*)&wl[p * 8] = lo;
                *(f32x4*)&wl[p * 8 + 4] = hi;
            } else {
                *(u32x4*)&wl[p * 4] = q[i];
            }
        }
    }
    __syncthreads();

    // the expert row's values of chunk c + 1 are read from LDS while chunk c is multiplied (two
    // register sets in turn)
    constexpr int WV = GV_CK / 4;  // 16-byte LDS reads per chunk
    f32x4 wA[WV], wB[WV];
    auto ldw = [&](f32x4 (&wr4)[WV], int c) {
        const float* wc = wl + min(c, nch - 1) * GV_CK;
#pragma unroll
        for (int j = 0; j < WV; ++j) wr4[j] = *(const f32x4*)(wc + 4 * j);
    };
    float acc = 0.0f;
    auto mul = [&](const u32x4 (&xq)[NV], const f32x4 (&wr4)[WV]) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if constexpr (sizeof(TA) == 2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float wa = wr4[2 * v + i / 2][2 * (i % 2)], wb = wr4[2 * v + i / 2][2 * (i % 2) + 1];
                    acc = __builtin_fmaf(__uint_as_float(xq[v][i] << 16), wa, acc);
                    acc = __builtin_fmaf(__uint_as_float(xq[v][i] & 0xffff0000u), wb, acc);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(__uint_as_float(xq[v][i]), wr4[v][i], acc);
            }
        }
    };
    ldw(wA, 0);
    for (int c = 0; c < nch; c += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            ldx((u + 3) & 3, c + u + 3);
            if (u & 1) ldw(wA, c + u + 1);
            else ldw(wB, c + u + 1);
            __builtin_amdgcn_sched_group_barrier(0x100, WV, 0);  // those LDS reads first
            if (c + u < nch) {
                if (u & 1) mul(xb[u], wB);
                else mul(xb[u], wA);
            }
        }
    }
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
    if (H % GV_CK == 0 && H <= GL_MAXH)
        hipLaunchKernelGGL(router_gemv_lds<TA>, grid, dim3(64), H * sizeof(float), s, x, w, off, logits, T, H, E);
    else
        hipLaunchKernelGGL(router_gemv<TA>, grid, dim3(64), 0, s, x, w, off, logits, T, H, E);
    return hipGetLastError();
}

template <typename TA>
hipError_t launch_mfma(const TA* x, const TA* w, int64_t T, int32_t H, int32_t E, const float* off, float* logits,
                       hipStream_t s) {
    const int32_t ntt = (int32_t)((T + 63) / 64), nte = (E + 63) / 64;
    if (H % 8 == 0)
        hipLaunchKernelGGL((router_mfma<TA, true>), dim3((unsigned)ntt * nte), dim3(256), 0, s, x, w, off, logits, T, H,
                           E, ntt, nte);
    else
        hipLaunchKernelGGL((router_mfma<TA, false>), dim3((unsigned)ntt * nte), dim3(256), 0, s, x, w, off, logits, T,
                           H, E, ntt, nte);
    return hipGetLastError();
}

// Few tokens or few experts: one output per lane (GEMV shape).  Otherwise the matrix-core
// kernel.  The summation order is the same in both.
template <typename TA>
hipError_t route_shape(const TA* x, const TA* w, int64_t T, int32_t H, int32_t E, const float* off,
                       float* logits, hipStream_t s) {
    if (T <= 512 || E < 16) return launch_gemv<TA>(x, w, T, H, E, off, logits, s);
    if (((T + 63) / 64) * ((E + 63) / 64) > (int64_t)INT32_MAX) return hipErrorInvalidValue;
    return launch_mfma<TA>(x, w, T, H, E, off, logits, s);
}

}  // namespace

hipError_t launch_router(const void* x, const void* w, int32_t act, int64_t T, int32_t H, int32_t E,
                         const float* offset, float* logits, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (act == MOE_BF16) return route_shape<bf16_t>((const bf16_t*)x, (const bf16_t*)w, T, H, E, offset, logits, s);
    return route_shape<float>((const float*)x, (const float*)w, T, H, E, offset, logits, s);
}

}  // namespace dsmoe
