// experts.hip - grouped SwiGLU expert GEMMs on bf16 MFMA (bf16, 4-bit or fp8 weights).
//
// Role: the per-expert matmuls that gather_mm / gather_qmm perform in the reference design
// (page "Epic: Engine Inference Core Stage E - MoE + hybrid families", opening paragraph), with
// the SwiGLU of the expert MLP fused into the first GEMM's epilogue:
//   GEMM-1: h[r, n] = bf16( silu(x[tok(r)] . W_gate[g, n]) * (x[tok(r)] . W_up[g, n]) )
//   GEMM-2: o[r, n] = bf16( h[r] . W_down[g, n] )
// for every row r of group g (rows come from the dispatch; group E is the shared expert, whose
// rows TK + t are the tokens in order).
//
// This file holds the weight-streaming kernels for groups of up to 64 rows -- the decode regime,
// where the layer is bound by HBM bandwidth: the register-streaming kernel ("stream") described
// here, and for fp8 layers a kernel that moves the codes of small groups through an LDS DMA ring
// (stream_f8, further down) and runs the register-streaming body for the rest.  A workgroup of four wavefronts
// owns 64 output columns of one group; each wavefront owns 16 of them and reads its weight
// rows from HBM exactly once per 64-row chunk of the group, straight into registers, two
// 128-element steps ahead of the MFMAs that consume them (three for fp8 and for the bf16 down
// projection).  The activation rows of the chunk (gathered x rows for GEMM-1, h rows for
// GEMM-2) are shared by the four wavefronts: they are copied by LDS DMA into a ring of three
// 16 KB LDS buffers, two steps ahead, so every activation byte leaves L2 once per workgroup and
// the loads of a step are waited for with a single count and barrier.  A step feeds four v_mfma_f32_16x16x32_bf16 per 16-row block (gate
// and up each for GEMM-1).  The k index inside a step is permuted identically for both
// operands (KLayout), so the sum is unchanged.
// MFMA 16x16x32 bf16 operand layout: lane l supplies row/column (l % 16) and eight
// consecutive k values of block (l / 16); result element v of lane l is row 4*(l/16)+v,
// column l % 16.
//
// 4-bit weights (affine, groups of 64 along the input axis): each lane loads the 16 bytes of
// codes covering its 32 k values plus that group's bf16 scale and offset, and forms
// bf16(s*q + b) in registers before the MFMA.  fp8 weights (OCP E4M3 codes, one fp32 scale per
// 128 x 128 block): each lane loads the 32 code bytes of its 32 k values plus the block's scale,
// and forms bf16(value * scale) in registers (hardware E4M3 -> fp32 conversion, fp32 multiply,
// round to nearest even).
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

enum { WF_BF16 = 0, WF_Q4 = 1, WF_F8 = 2 };

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight 4-bit codes (code i at bits 4i) -> bf16(s q + b), given s512 = 512 s.  A code q in the
// low nibble of a byte, read as an OCP E4M3 code, has the value q * 2^-9 (a subnormal for q < 8,
// exponent field 1 above), so one hardware E4M3 -> fp32 conversion turns two codes into exact
// floats; 512 s * (q * 2^-9) is exactly s q, so the fma rounds s q + b once, as fma(s, q, b) would.
// (512 s overflows only for |s| > 6.6e35.)
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s512, float b) {
    u32x4 r;
    const uint32_t lo4 = w & 0x0F0F0F0Fu, hi4 = (w >> 4) & 0x0F0F0F0Fu;  // codes 0,2,4,6 / 1,3,5,7
    const auto e02 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo4, false);  // codes 0, 2
    const auto e46 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo4, true);   // codes 4, 6
    const auto e13 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi4, false);  // codes 1, 3
    const auto e57 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi4, true);   // codes 5, 7
    r[0] = pack_bf16x2(__builtin_fmaf(s512, e02[0], b), __builtin_fmaf(s512, e13[0], b));
    r[1] = pack_bf16x2(__builtin_fmaf(s512, e02[1], b), __builtin_fmaf(s512, e13[1], b));
    r[2] = pack_bf16x2(__builtin_fmaf(s512, e46[0], b), __builtin_fmaf(s512, e57[0], b));
    r[3] = pack_bf16x2(__builtin_fmaf(s512, e46[1], b), __builtin_fmaf(s512, e57[1], b));
    return as_bf16x8(r);
}

// eight E4M3 codes (two words, code i at bits 8*(i%4) of word i/4) -> bf16(value * s)
__device__ __forceinline__ bf16x8 dequant_f8x8(uint32_t lo, uint32_t hi, float s) {
    u32x4 r;
    const auto v0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);  // codes 0, 1
    const auto v1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);   // codes 2, 3
    const auto v2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const auto v3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    r[0] = pack_bf16x2(v0[0] * s, v0[1] * s);
    r[1] = pack_bf16x2(v1[0] * s, v1[1] * s);
    r[2] = pack_bf16x2(v2[0] * s, v2[1] * s);
    r[3] = pack_bf16x2(v3[0] * s, v3[1] * s);
    return as_bf16x8(r);
}

// Weight operand source for one output column (row of the weight matrix).
struct WRow {
    const bf16_t* w;   // bf16 row (WF_BF16)
    const uint32_t* q; // packed codes row (WF_Q4)
    const bf16_t* s;   // scale row (WF_Q4)
    const bf16_t* b;   // offset row (WF_Q4)
    const uint8_t* c8; // E4M3 codes row (WF_F8)
    const float* fs;   // block scales of the row's 128-row block, one per 128 k (WF_F8)
};

// k layout of one reduction step inside a wave.  Lane l (group q = l / 16) supplies, for the
// step's i-th MFMA, the 8 k values starting at k0 + kq + i * PS.  bf16 rows: kq = 8 q, PS = 32,
// so the 4 lanes of a row read 64 contiguous bytes per load instruction; 4-bit rows: kq = 32 q,
// PS = 8, so a lane's codes for a step are one 16-byte word group.  A and B use the same layout.
template <int WF>
struct KLayout {  // 4-bit and fp8 rows share one layout
    static constexpr int PS = WF == WF_BF16 ? 32 : 8;
    static __device__ __forceinline__ int kq(int lane, int np) { return (lane >> 4) * (WF == WF_BF16 ? 8 : 8 * np); }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One weight row's operands for one step, as loaded: bf16 pieces, or 4-bit codes plus the
// row's scale and offset for the step's quantisation group (dequantised only when used, so the
// loads can run ahead of the MFMAs).
template <int WF>
struct WRegs;
template <>
struct WRegs<WF_BF16> {
    bf16x8 v[4];
    __device__ __forceinline__ bf16x8 frag(int i) const { return v[i]; }
};
template <>
struct WRegs<WF_Q4> {
    u32x4 q;
    bf16_t s, b;
    __device__ __forceinline__ bf16x8 frag(int i) const { return dequant8(q[i], 512.0f * bf16_to_f32(s), bf16_to_f32(b)); }
};
template <>
struct WRegs<WF_F8> {
    u32x4 q[2];  // 32 codes; piece i is words 2(i%2), 2(i%2)+1 of q[i/2]
    float s;
    __device__ __forceinline__ bf16x8 frag(int i) const {
        return dequant_f8x8(q[i >> 1][2 * (i & 1)], q[i >> 1][2 * (i & 1) + 1], s);
    }
};

// NP pieces of 8 k values (see KLayout) starting at k.  Vector-memory operations issued: NP
// 16-byte loads (bf16), codes + scale + offset = 3 (4-bit), or NP/2 16-byte code loads + scale
// (fp8: 3 for a full step).
template <int WF, int NP>
__device__ __forceinline__ void load_w(const WRow& r, int k, WRegs<WF>& out) {
    if constexpr (WF == WF_BF16) {
#pragma unroll
        for (int i = 0; i < NP; ++i) out.v[i] = as_bf16x8(*(const u32x4*)(r.w + k + i * KLayout<WF>::PS));
    } else if constexpr (WF == WF_F8) {
        out.s = r.fs[k >> 7];
#pragma unroll
        for (int i = 0; i < NP / 2; ++i) out.q[i] = *(const u32x4*)(r.c8 + k + 16 * i);
    } else {
        out.s = r.s[k >> 6];
        out.b = r.b[k >> 6];
        if constexpr (NP == 4) {
            out.q = *(const u32x4*)(r.q + (k >> 3));
        } else {
            const u32x2 w = *(const u32x2*)(r.q + (k >> 3));
            out.q[0] = w[0];
            out.q[1] = w[1];
        }
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
    WRow r = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    if (shared) {
        const bf16_t* base = (const bf16_t*)(sel == 0 ? a.swg : sel == 1 ? a.swu : a.swd);
        r.w = base + (int64_t)n * in_dim;
        return r;
    }
    const int64_t row = (int64_t)g * out_dim + n;
    if constexpr (WF == WF_BF16) {
        const bf16_t* base = (const bf16_t*)(sel == 0 ? a.wg : sel == 1 ? a.wu : a.wd);
        r.w = base + row * in_dim;
    } else if constexpr (WF == WF_F8) {
        r.c8 = (const uint8_t*)(sel == 0 ? a.wg : sel == 1 ? a.wu : a.wd) + row * in_dim;
        const int64_t nbo = (out_dim + 127) / 128, nbi = (in_dim + 127) / 128;
        r.fs = (sel == 0 ? a.fsg : sel == 1 ? a.fsu : a.fsd) + ((int64_t)g * nbo + n / 128) * nbi;
    } else {
        const uint32_t* base = (const uint32_t*)(sel == 0 ? a.wg : sel == 1 ? a.wu : a.wd);
        r.q = base + row * (in_dim / 8);
        r.s = (sel == 0 ? a.sg : sel == 1 ? a.su : a.sd) + row * (in_dim / 64);
        r.b = (sel == 0 ? a.bg : sel == 1 ? a.bu : a.bd) + row * (in_dim / 64);
    }
    return r;
}

// k layout as 16-byte chunk indices inside a step: lane l's i-th piece of an NP-piece step
template <int WF, int NP>
__device__ __forceinline__ int piece_chunk(int lane, int i) {
    return WF == WF_BF16 ? (lane >> 4) + 4 * i : NP * (lane >> 4) + i;
}

constexpr int S_ROWS = 64;               // rows per chunk of a group
constexpr int S_ROWB = 256;              // LDS bytes per activation row: one 128-element step
constexpr int S_TILE = S_ROWS * S_ROWB;  // one LDS buffer

// byte offset of 16-byte chunk c of row r in an activation buffer; the chunks of a row are
// permuted by r mod 16, so the 16 rows a fragment read touches hit 16 different bank groups
__device__ __forceinline__ uint32_t s_off(int r, int c) { return (uint32_t)(r * S_ROWB + ((c ^ (r & 15)) << 4)); }

#define DSMOE_S_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Wait until this wave's vector-memory operations (register loads and LDS DMA) are complete,
// then barrier: afterwards the step's activation buffer is filled for every wave.
__device__ __forceinline__ void s_wait_all_barrier() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// Same, but the newest N operations (the next step's weight loads) may stay in flight.
template <int N>
__device__ __forceinline__ void s_wait_barrier() { asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory"); }

// GEMM-1 (G1): h = SwiGLU of x rows against W_gate / W_up;  GEMM-2: o = h rows against W_down.
// One workgroup's share of group g: 64 output columns (column block cb), every row of the group.
// N is a multiple of 64 (bf16, 4-bit and fp8 layers), so every wave of a live workgroup has
// columns.  As: the activation ring (three buffers, two steps ahead).
template <int WF, bool G1>
__device__ __forceinline__ void stream_body(const GroupedArgs& a, int32_t g, int32_t cb, char* As) {
    int32_t r0, cnt;
    group_rows(a, g, r0, cnt);
    if (cnt <= 0 || cnt > a.stream_max_rows) return;
    const bool shared = g == a.E;
    const int32_t N = G1 ? (shared ? a.Is : a.I) : a.H;   // output columns
    const int32_t KD = G1 ? a.H : (shared ? a.Is : a.I);  // reduction length, a multiple of 64
    if (cb * 64 >= N) return;                             // workgroup-uniform
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int32_t col = cb * 64 + wave * 16 + (lane & 15);
    const WRow w0 = weight_row<WF>(a, G1 ? 0 : 2, g, shared, col, N, KD);
    const WRow w1 = G1 ? weight_row<WF>(a, 1, g, shared, col, N, KD) : w0;
    const bf16_t* abase = G1 ? (const bf16_t*)a.x : (const bf16_t*)a.h;
    const int64_t lda = G1 ? a.H : a.ldh;
    const int nfull = KD >> 7;       // 128-wide steps
    const bool tail = (KD & 64) != 0;  // plus one 64-wide step
    const int nsteps = nfull + (tail ? 1 : 0);  // >= 1
    constexpr int NW = G1 ? 2 : 1;   // weight matrices

    for (int32_t m0 = 0; m0 < cnt; m0 += S_ROWS) {
        const int nrb = min(4, (cnt - m0 + 15) >> 4);  // live 16-row blocks
        // LDS DMA sources: wave w fills rows [16 w, 16 w + 16) of the buffer (only for w < nrb),
        // instruction j rows 16 w + 4 j + lane / 16; lane i writes chunk slot i % 16 of its row,
        // which holds logical chunk (i % 16) ^ (row % 16)
        const bf16_t* arow[4];
        int cj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int32_t rr = m0 + wave * 16 + j * 4 + (lane >> 4);
            rr = rr < cnt ? rr : cnt - 1;  // rows past the group are computed, never stored
            const int64_t src = G1 ? (int64_t)row_token(a, r0 + rr) : (int64_t)(r0 + rr);
            arow[j] = abase + src * lda;
            cj[j] = (lane & 15) ^ (j * 4 + (lane >> 4));
        }
        auto issue_a = [&](int s, int buf) {
            if (wave >= nrb) return;  // wave-uniform
            const int32_t k = s << 7;
            // the 64-wide tail step has chunks 0..7 only: the lanes of slots holding chunks 8..15
            // fetch chunk c - 8 instead (in bounds, never read), so every lane of the DMA is active
            const int cm = s == nfull ? 7 : 15;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_amdgcn_global_load_lds((const void*)(arow[j] + k + (cj[j] & cm) * 8),
                                                 DSMOE_S_LDS(As + buf * S_TILE + (wave * 4 + j) * 1024), 16, 0, 0);
        };
        // weights of a full step (NP = 4) or of the tail step (NP = 2)
        using W = WRegs<WF>;
        auto load_full = [&](int s, W (&wv)[NW]) {
            const int32_t k = (s << 7) + KLayout<WF>::kq(lane, 4);
            load_w<WF, 4>(w0, k, wv[0]);
            if (G1) load_w<WF, 4>(w1, k, wv[NW - 1]);
        };
        auto load_tail = [&](W (&wv)[NW]) {
            const int32_t k = (nfull << 7) + KLayout<WF>::kq(lane, 2);
            load_w<WF, 2>(w0, k, wv[0]);
            if (G1) load_w<WF, 2>(w1, k, wv[NW - 1]);
        };
        f32x4 acc[NW][4];
#pragma unroll
        for (int m = 0; m < NW; ++m)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) acc[m][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](auto np_tag, int buf, const W (&wv)[NW]) {
            constexpr int NP = decltype(np_tag)::value;
            const char* st = As + buf * S_TILE;
            bf16x8 wf[NW][NP];
#pragma unroll
            for (int m = 0; m < NW; ++m)
#pragma unroll
                for (int i = 0; i < NP; ++i) wf[m][i] = wv[m].frag(i);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                if (rb >= nrb) break;
                bf16x8 av[NP];
#pragma unroll
                for (int i = 0; i < NP; ++i)
                    av[i] = __builtin_bit_cast(
                        bf16x8, *(const u32x4*)(st + s_off(rb * 16 + (lane & 15), piece_chunk<WF, NP>(lane, i))));
#pragma unroll
                for (int i = 0; i < NP; ++i)
#pragma unroll
                    for (int m = 0; m < NW; ++m)
                        acc[m][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], wf[m][i], acc[m][rb], 0, 0, 0);
            }
        };

        // One full step: publish its activations, start the loads of steps s+2 (activations) and
        // s+D (weights), run its MFMAs.  Activations run two steps ahead in three LDS buffers;
        // weights run D steps ahead in D+1 rotating register sets (D = 3 for fp8, whose steps
        // carry half the bytes of bf16 ones, so more of them must be in flight, and for the bf16
        // down projection, whose reduction of I is only a few steps long, so its pipeline fill
        // weighs more; else 2).  Per wave
        // the issue order is A(s+2), W(s+D) during step s.  At the top of step s, A(s) and W(s)
        // must have landed; what may stay in flight is everything issued after them -- for
        // D = 2: A(s+1), W(s+1); for D > 2 (W(s) is older than A(s)): W(s+D-2), A(s+1),
        // W(s+D-1) -- the DMA counted only for the waves that copy rows.  Past the end the loads
        // repeat the last step (L2 hits, never consumed) instead of being skipped: with the same
        // load sequence on every path the compiler's own waits for the weight registers stay
        // exact rather than falling back to waiting for everything.
        constexpr int WL = NW * (WF == WF_BF16 ? 4 : 3);  // vector-memory operations of one load_full
        constexpr int D = (WF == WF_F8 || (WF == WF_BF16 && !G1)) ? 3 : 2;
        constexpr int NWS = D + 1;
        constexpr int LATER_COPY = D == 2 ? 4 + WL : 4 + 2 * WL;  // waves that copy activation rows
        constexpr int LATER_NOCOPY = (D - 1) * WL;                // waves that do not
        auto step = [&](int s, const W (&cur)[NW], W (&nxt)[NW]) {
            if (wave < nrb) s_wait_barrier<LATER_COPY>();  // wave-uniform; both arms hold one barrier
            else s_wait_barrier<LATER_NOCOPY>();
            // the buffer written here was last read in step s-1; past the last step it is not
            // read again in this chunk
            issue_a(min(s + 2, nsteps - 1), (s + 2) % 3);
            load_full(min(s + D, nfull - 1), nxt);
            compute(std::integral_constant<int, 4>{}, s % 3, cur);
        };

        __syncthreads();  // the previous chunk's reads of every buffer are done
        W ws[NWS][NW];
        issue_a(0, 0);
        if (nfull > 0) {
            // the prologue loads are issued unconditionally (past the last full step they repeat
            // it and are never used), so the compiler's own wait before the loop's first MFMAs
            // sees the same load order on entry as around the loop and stays exact
            load_full(0, ws[0]);
            issue_a(min(1, nsteps - 1), 1);
#pragma unroll
            for (int j = 1; j < D; ++j) load_full(min(j, nfull - 1), ws[j]);
            for (int s = 0; s < nfull; s += NWS) {  // W(k) lives in set k % NWS
#pragma unroll
                for (int u = 0; u < NWS; ++u)
                    if (s + u < nfull) step(s + u, ws[u], ws[(u + D) % NWS]);
            }
        }
        if (tail) {  // a 64-wide last step (reduction lengths of 64 mod 128 only): weights unprefetched
            W wt[NW];
            load_tail(wt);
            s_wait_all_barrier();
            compute(std::integral_constant<int, 2>{}, nfull % 3, wt);
        }
        // The epilogue reads the accumulators right after the last MFMA, which may sit behind a
        // branch (the 16-row blocks past nrb are skipped).  This compiler's hazard recognizer
        // has been seen to read an accumulator at such a join without the MFMA-to-VALU wait
        // states, so they are issued explicitly: every accumulator passes through an empty asm
        // that follows the wait states in program order, so no read of it can come earlier.
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0][0]));
#pragma unroll
        for (int m = 0; m < NW; ++m)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                if (m | rb) asm volatile("" : "+a"(acc[m][rb]));

#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            if (rb >= nrb) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int32_t rr = m0 + rb * 16 + (lane >> 4) * 4 + v;
                if (rr >= cnt) continue;
                if (G1)
                    ((bf16_t*)a.h)[(int64_t)(r0 + rr) * a.ldh + col] =
                        f32_to_bf16(silu_f(acc[0][rb][v]) * acc[NW - 1][rb][v]);
                else
                    ((bf16_t*)a.o)[(int64_t)(r0 + rr) * a.H + col] = f32_to_bf16(acc[0][rb][v]);
            }
        }
    }
}

// grid: x = ceil(N / 64) column blocks (N = max(I, Is), resp. H), y = groups [g0, g0 + gridDim.y).
// The shared expert (group E) always has bf16 weights: in a launch over quantised routed groups
// it takes the bf16 body, so it streams beside the routed groups instead of in a launch of its
// own with only N / 64 workgroups.
template <int WF, bool G1>
__global__ __launch_bounds__(256) void stream_gemm(GroupedArgs a, int32_t g0) {
    __shared__ __attribute__((aligned(1024))) char As[3 * S_TILE];
    const int32_t g = g0 + blockIdx.y;
    if (WF != WF_BF16 && g == a.E)  // workgroup-uniform
        stream_body<WF_BF16, G1>(a, g, blockIdx.x, As);
    else
        stream_body<WF, G1>(a, g, blockIdx.x, As);
}

// ---- fp8 groups of at most 32 rows: codes through an LDS DMA ring ----
//
// Register loads in the MFMA operand layout cover half of a 128-byte line per weight row per
// instruction and top out near 6.1 TB/s.  LDS DMA instructions in which eight lanes fetch one
// whole line reach about 7.1 TB/s on the streaming pattern below (128 code rows per workgroup,
// one line of each per stage, two stages in flight, two workgroups per CU), and still about
// 6.9 TB/s with an fp8 stage's dequantisation and MFMAs between the waits; with one workgroup
// per CU the same work drops to about 5 TB/s (measured on MI355X).  So the codes of fp8 groups
// of up to 32 rows (the decode regime) stream this way.  Per 128-k stage a workgroup receives
// one line of each of its 128 code rows -- GEMM-1: the gate rows of its 64 output columns,
// then their up rows; GEMM-2: 128 output columns as two halves of 64 -- beside 256 bytes of
// each of the chunk's 32 activation rows, in a ring of three 24 KB stages (72 KB: two
// workgroups per CU).  The workgroup's output columns lie in one 128-row scale block, so each
// stage needs one fp32 block scale per weight matrix; the block-scale rows (at most 64 stages)
// are copied into LDS once by wave 0 before the first stage and read there by broadcast.
// Slots: code chunk c (16 codes) of slot row rho sits at chunk c ^ f8d_swz(rho) and activation
// chunk c (8 k) of row r at chunk c ^ (r mod 16), so the 8-byte code reads and 16-byte
// activation reads of a 16-row MFMA operand fall in distinct banks.
constexpr int F8D_NS = 3;                                   // ring depth
constexpr int F8D_WROWS = 128;                              // code rows per stage
constexpr int F8D_AROWS = 32;                               // activation rows (the largest group)
constexpr int F8D_A_BYTES = F8D_AROWS * 256;                // 128 k of bf16 per activation row
constexpr int F8D_STAGE = F8D_A_BYTES + F8D_WROWS * 128;    // 24 KB
constexpr int F8D_SCALES = 2 * 256;                         // 64 fp32 scales per weight matrix
constexpr int F8D_LDS = F8D_NS * F8D_STAGE + F8D_SCALES;
constexpr int F8D_MAX_STAGES = 64;

__device__ __forceinline__ int f8d_swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int N>
__device__ __forceinline__ void f8d_wait_barrier() { asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory"); }

// group g (rows [r0, r0 + cnt), 1 <= cnt <= 32, fp8 codes), the workgroup's nbw column blocks
// from nbw * blockIdx.x on: 64 output columns each for GEMM-1, 128 for GEMM-2.  The blocks'
// stages form one stream through the ring (the next block's first stages load under the last
// stages of the one before), so a short reduction does not refill the ring per block.  The
// reduction length is a multiple of 128, and nbw times its stages at most 64 (checked by the
// launcher).
template <bool G1>
__device__ __forceinline__ void stream_f8_dma_body(const GroupedArgs& a, int32_t g, int32_t r0, int32_t cnt,
                                                   int32_t nbw, char* smem) {
    const int32_t N = G1 ? a.I : a.H;
    const int32_t KD = G1 ? a.H : a.I;
    constexpr int CW = G1 ? 64 : 128;  // output columns per block
    const int32_t cb0 = (int32_t)blockIdx.x * nbw;
    const int32_t col0 = cb0 * CW;
    if (col0 >= N) return;  // workgroup-uniform
    const int nb = min(nbw, (N + CW - 1) / CW - cb0);  // live blocks
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int nst = KD >> 7;
    const int ntot = nb * nst;  // stages of all blocks, at most 64
    constexpr int WT = F8D_WROWS / 8 / 4;  // code DMA instructions per wave per stage
    constexpr int NW = 2;                  // weight row blocks: gate and up, or two halves of 64 columns

    // code rows: uniform expert bases plus per-lane 32-bit byte offsets (N * KD < 2^32)
    const int64_t ebase = (int64_t)g * N * KD;
    const char* wb0 = (const char*)(G1 ? a.wg : a.wd) + ebase;
    const char* wb1 = (const char*)(G1 ? a.wu : a.wd) + ebase;
    // byte offset of each DMA instruction's source in the first block's code rows; a later GEMM-2
    // block adds 128 rows, clamped to the last row (rows past N are never stored)
    int w_rho[WT];
    uint32_t w_c[WT], w_off[WT];
#pragma unroll
    for (int t = 0; t < WT; ++t) {
        w_rho[t] = (wave * WT + t) * 8 + (lane >> 3);  // slot row
        w_c[t] = (uint32_t)(((lane & 7) ^ f8d_swz(w_rho[t])) * 16);
        const int32_t n = G1 ? col0 + (w_rho[t] & 63) : min(col0 + w_rho[t], N - 1);
        w_off[t] = (uint32_t)n * (uint32_t)KD + w_c[t];
    }
    // block-scale rows of the workgroup's 128-row blocks: [E][ceil(N / 128)][nst] per matrix; the
    // rows of consecutive GEMM-2 blocks follow each other, so stage u of the stream has scale u
    const int64_t srow = ((int64_t)g * ((N + 127) >> 7) + (col0 >> 7)) * nst;
    const float* fs0 = (G1 ? a.fsg : a.fsd) + srow;
    const float* fs1 = (G1 ? a.fsu : a.fsd) + srow;
    char* scl = smem + F8D_NS * F8D_STAGE;

    // activation rows: wave w (w < nrb) copies rows [16 w, 16 w + 16), instruction j rows
    // 16 w + 4 j + lane / 16; lane i fills chunk slot i % 16 of its row
    const int nrb = (cnt + 15) >> 4;     // live 16-row blocks (1 or 2)
    const bool copier = wave < nrb;      // wave-uniform
    const char* abase = G1 ? (const char*)a.x : (const char*)a.h;
    const int64_t lda = G1 ? a.H : a.ldh;
    const char* arow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = wave * 16 + j * 4 + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        int32_t rr = r < cnt ? r : cnt - 1;  // rows past the group are computed, never stored
        const int64_t src = G1 ? (int64_t)row_token(a, r0 + rr) : (int64_t)(r0 + rr);
        arow[j] = abase + (src * lda + c * 8) * 2;
    }
    // stage u of the stream: block u / nst, reduction stage u % nst (GEMM-2 issues in order and
    // counts them in ib, iks; GEMM-1 has one block)
    int ib = 0, iks = 0;
    auto issue = [&](int u) {
        if constexpr (G1) iks = u;
        char* st = smem + (u % F8D_NS) * F8D_STAGE;
        if (copier) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_amdgcn_global_load_lds((const void*)(arow[j] + iks * 256),
                                                 DSMOE_S_LDS(st + (wave * 4 + j) * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < WT; ++t) {
            const int rho0 = (wave * WT + t) * 8;
            const char* wb = (G1 && rho0 >= 64) ? wb1 : wb0;
            uint32_t off = w_off[t];
            if constexpr (!G1) {
                if (ib > 0) off = (uint32_t)min(col0 + ib * CW + w_rho[t], N - 1) * (uint32_t)KD + w_c[t];
            }
            __builtin_amdgcn_global_load_lds((const void*)(wb + off + iks * 128),
                                             DSMOE_S_LDS(st + F8D_A_BYTES + rho0 * 128), 16, 0, 2 /* non-temporal */);
        }
        if constexpr (!G1) {
            if (++iks == nst) iks = 0, ++ib;
        }
    };

    f32x4 acc[NW][2];
#pragma unroll
    for (int m = 0; m < NW; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int q = lane >> 4, ln = lane & 15;
    auto compute = [&](int u) {
        const char* st = smem + (u % F8D_NS) * F8D_STAGE;
        const float sc0 = *(const float*)(scl + u * 4), sc1 = *(const float*)(scl + 256 + u * 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {  // four 32-k steps per stage
            const int p = t * 4 + q;   // the lane's 8-k piece of the stage
            bf16x8 wf[NW];
#pragma unroll
            for (int m = 0; m < NW; ++m) {
                const int rho = m * 64 + wave * 16 + ln;
                const u32x2 cw = *(const u32x2*)(st + F8D_A_BYTES + rho * 128 + (((p >> 1) ^ f8d_swz(rho)) << 4) + (p & 1) * 8);
                wf[m] = dequant_f8x8(cw[0], cw[1], (G1 && m) ? sc1 : sc0);
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                if (rb >= nrb) break;
                const bf16x8 af = as_bf16x8(*(const u32x4*)(st + (rb * 16 + ln) * 256 + ((p ^ ln) << 4)));
#pragma unroll
                for (int m = 0; m < NW; ++m)
                    acc[m][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf[m], acc[m][rb], 0, 0, 0);
            }
        }
    };

    // block b's results: GEMM-1 bf16(silu(gate) * up), GEMM-2 its two halves of 64 columns
    auto epilogue = [&](int b) {
        // the accumulators are read right after the last MFMAs, possibly behind the row-block
        // branch: issue the MFMA-to-VALU wait states explicitly before any of them is read
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0][0]));
#pragma unroll
        for (int m = 0; m < NW; ++m)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                if (m | rb) asm volatile("" : "+a"(acc[m][rb]));
        const int32_t col = col0 + b * CW + wave * 16 + ln;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            if (rb >= nrb) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int32_t rr = rb * 16 + q * 4 + v;
                if (rr >= cnt) continue;
                if (G1) {
                    ((bf16_t*)a.h)[(int64_t)(r0 + rr) * a.ldh + col] =
                        f32_to_bf16(silu_f(acc[0][rb][v]) * acc[1][rb][v]);
                } else {
                    bf16_t* orow = (bf16_t*)a.o + (int64_t)(r0 + rr) * a.H;
                    orow[col] = f32_to_bf16(acc[0][rb][v]);
                    if (col + 64 < N) orow[col + 64] = f32_to_bf16(acc[1][rb][v]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < NW; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // wave 0 (always a copier) copies the scale rows first; the first stage's wait covers them
    if (wave == 0) {
        const int i = min(lane, ntot - 1);
        __builtin_amdgcn_global_load_lds((const void*)(fs0 + i), DSMOE_S_LDS(scl), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(fs1 + i), DSMOE_S_LDS(scl + 256), 4, 0, 0);
    }
    issue(0);
    if (ntot > 1) issue(1);
    auto stage = [&](int u) {
        // stage u has landed for every wave; stage u+1 (if issued) may still be in flight
        if (u + 1 < ntot) {
            if (copier) f8d_wait_barrier<WT + 4>();  // wave-uniform; both arms hold one barrier
            else f8d_wait_barrier<WT>();
        } else {
            f8d_wait_barrier<0>();
        }
        // the slot of stage u+2 held stage u-1, which every wave finished before this barrier
        if (u + 2 < ntot) issue(u + 2);
        compute(u);
    };
    if constexpr (G1) {
        for (int u = 0; u < ntot; ++u) stage(u);
        epilogue(0);
    } else {
        int cks = 0, cbk = 0;  // block and reduction stage of the stage computed
        for (int u = 0; u < ntot; ++u) {
            stage(u);
            if (++cks == nst) {
                epilogue(cbk);
                cks = 0;
                ++cbk;
            }
        }
    }
}

// fp8 layers' weight streaming: routed groups of at most 32 rows through the DMA ring above; the
// shared expert (bf16) and fp8 groups of 33 or more rows by the register-streaming body, which
// owns 64 output columns per call (a GEMM-2 workgroup here owns 128: two calls).
// grid: x = ceil(N / 64) (GEMM-1, N = max(I, Is)) or ceil(H / 128) (GEMM-2) column blocks,
// y = groups [g0, g0 + gridDim.y), the last group first: workgroups are dispatched in grid
// order, and the last group -- the shared expert, whose workgroups move twice the bytes of a
// routed fp8 one, through registers -- would otherwise run alone at the end of the launch.
template <bool G1>
__global__ __launch_bounds__(256) void stream_f8(GroupedArgs a, int32_t g0, int32_t nbw) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int32_t g = g0 + (int32_t)((blockIdx.y + gridDim.y - 1) % gridDim.y);
    int32_t r0, cnt;
    group_rows(a, g, r0, cnt);
    if (cnt <= 0 || cnt > a.stream_max_rows) return;  // workgroup-uniform
    if (g < a.E && cnt <= F8D_AROWS) {
        stream_f8_dma_body<G1>(a, g, r0, cnt, G1 ? 1 : nbw, smem);
        return;
    }
    // the workgroup's columns in calls of 64: GEMM-1 workgroups own one block of 64 (nbw = 1),
    // GEMM-2 ones nbw blocks of 128
    const int32_t per = G1 ? 1 : 2 * nbw;
    const int32_t cb = (int32_t)blockIdx.x * per;
    for (int h = 0; h < per; ++h) {
        if (g == a.E) stream_body<WF_BF16, G1>(a, g, cb + h, smem);
        else stream_body<WF_F8, G1>(a, g, cb + h, smem);
    }
}

}  // namespace

hipError_t launch_gemm1_bf16(const GroupedArgs& a, int32_t g0, int32_t g1, int32_t wdt, hipStream_t s) {
    if (g1 <= g0) return hipSuccess;
    const int32_t N = max(a.I, a.Is);
    const dim3 grid((N + 63) / 64, g1 - g0);
    if (wdt == MOE_FP8)
        hipLaunchKernelGGL((stream_gemm<WF_F8, true>), grid, dim3(256), 0, s, a, g0);
    else if (wdt == MOE_Q4G64)
        hipLaunchKernelGGL((stream_gemm<WF_Q4, true>), grid, dim3(256), 0, s, a, g0);
    else
        hipLaunchKernelGGL((stream_gemm<WF_BF16, true>), grid, dim3(256), 0, s, a, g0);
    return hipGetLastError();
}

hipError_t launch_gemm2_bf16(const GroupedArgs& a, int32_t g0, int32_t g1, int32_t wdt, hipStream_t s) {
    if (g1 <= g0) return hipSuccess;
    const dim3 grid((a.H + 63) / 64, g1 - g0);
    if (wdt == MOE_FP8)
        hipLaunchKernelGGL((stream_gemm<WF_F8, false>), grid, dim3(256), 0, s, a, g0);
    else if (wdt == MOE_Q4G64)
        hipLaunchKernelGGL((stream_gemm<WF_Q4, false>), grid, dim3(256), 0, s, a, g0);
    else
        hipLaunchKernelGGL((stream_gemm<WF_BF16, false>), grid, dim3(256), 0, s, a, g0);
    return hipGetLastError();
}

hipError_t configure_stream_f8() {
    hipError_t e = hipFuncSetAttribute((const void*)stream_f8<true>, hipFuncAttributeMaxDynamicSharedMemorySize, F8D_LDS);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)stream_f8<false>, hipFuncAttributeMaxDynamicSharedMemorySize, F8D_LDS);
}

// the DMA ring takes reduction lengths that are multiples of 128 of at most 64 stages
bool stream_f8_fits(const GroupedArgs& a) {
    return a.H % 128 == 0 && a.I % 128 == 0 && a.H <= 128 * F8D_MAX_STAGES && a.I <= 128 * F8D_MAX_STAGES;
}

hipError_t launch_stream_f8(const GroupedArgs& a, bool gemm1, int32_t g0, int32_t g1, hipStream_t s) {
    if (g1 <= g0) return hipSuccess;
    if (gemm1) {
        const int32_t N = max(a.I, a.Is);
        hipLaunchKernelGGL((stream_f8<true>), dim3((N + 63) / 64, g1 - g0), dim3(256), F8D_LDS, s, a, g0, 1);
    } else {
        // GEMM-2 reductions are short (I / 128 stages): two column blocks per workgroup when
        // their stages fit the scale buffer
        const int32_t nbw = (a.I / 128) * 2 <= F8D_MAX_STAGES ? 2 : 1;
        const int32_t nblk = (a.H + 127) / 128;
        hipLaunchKernelGGL((stream_f8<false>), dim3((nblk + nbw - 1) / nbw, g1 - g0), dim3(256), F8D_LDS, s, a, g0,
                           nbw);
    }
    return hipGetLastError();
}

}  // namespace dsmoe
