// experts_tiled.hip - LDS-tiled grouped expert GEMMs for groups with many rows.
//
// Same computation as experts.hip (page "Epic: Engine Inference Core Stage E - MoE + hybrid
// families", opening paragraph: the per-expert matmuls of gather_mm / gather_qmm; SwiGLU fused
// into the gate/up GEMM's epilogue), organised for the prefill regime where a group holds
// hundreds or thousands of rows and the work is bound by MFMA throughput:
//
//   * a workgroup (4 waves) computes a BM x 256 tile: BM rows of one group against 256 rows of
//     weights -- for GEMM-1 the gate and up rows of the same 128 output columns, for GEMM-2 256
//     rows of W_down -- with v_mfma_f32_32x32x16_bf16 and fp32 accumulators;
//   * A (gathered activation rows, or the contiguous h rows) and B (weights) are staged through
//     LDS in k-steps of 64 with two buffers: the global loads of step s+1 are in flight while
//     step s runs on the matrix cores; one barrier per step;
//   * LDS rows are 128 bytes (64 bf16); the eight 16-byte chunks of a row are XOR-swizzled with
//     the row index so that both the staging writes and the MFMA operand reads are free of bank
//     conflicts;
//   * 4-bit weights are dequantised (bf16(s*q + b)) once per LDS tile while staging, so the cost
//     is amortised over the BM rows of the tile;
//   * the list of (group, first row) tiles is built on the device from the dispatch offsets, so
//     no count ever returns to the host; the grid is an upper bound and surplus workgroups exit;
//   * workgroup ids are remapped so that the workgroups an XCD receives (ids congruent mod 8)
//     form a contiguous run of tiles, keeping the A and B panels they share in that XCD's L2.
//
// MFMA 32x32x16 bf16 layout: lane l supplies row/column (l % 32) and the 8 k values of chunk
// (l / 32) of each 16-k step; result element v of lane l is row 8*(v/4) + 4*(l/32) + v%4,
// column l % 32.
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

enum { WF_BF16 = 0, WF_Q4 = 1 };

constexpr int BK = 64;        // k per LDS stage (one 4-bit scale group)
constexpr int NB = 256;       // weight rows per tile
constexpr int THREADS = 256;  // 4 waves, 2 x 2

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// byte offset of 16-byte chunk c of row r in a [rows][64] bf16 LDS tile
__device__ __forceinline__ uint32_t lds_off(int r, int c) { return (uint32_t)(r * 128 + ((c ^ (r & 7)) << 4)); }

__device__ __forceinline__ u32x4 dequant8(uint32_t w, float s, float b) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = __builtin_fmaf(s, (float)((w >> (8 * j)) & 0xFu), b);
        const float hi = __builtin_fmaf(s, (float)((w >> (8 * j + 4)) & 0xFu), b);
        r[j] = pack_bf16x2(lo, hi);
    }
    return r;
}

// silu with the hardware reciprocal (about 1 ulp; the product is rounded to bf16 anyway)
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

struct TileArgs {
    GroupedArgs a;
    const int32_t* tile_count;  // [1]
    const int32_t* tile_info;   // [max_tiles][2]: group, first row within the group
    int32_t g0, g1;             // groups handled by this launch
    int32_t col_tiles;          // output column tiles per row tile
    int32_t nwg;                // workgroups launched
};

// Workgroup -> (tile, column tile).  The logical space holds tile_count * col_tiles items in
// bands of 4 column tiles: items of one band walk the row tiles with the column fastest, so the
// workgroups running at once share both A panels (same rows) and B panels (same group and
// columns).  Workgroup ids congruent mod 8 land on the same XCD; each XCD takes one contiguous
// eighth of the logical space, sized by the tile count actually built (the grid is a bound).
__device__ __forceinline__ bool map_tile(const TileArgs& ta, int32_t& tile, int32_t& ct) {
    const int32_t ntiles = ta.tile_count[0];
    const int32_t total = ntiles * ta.col_tiles;
    const int32_t per_xcd = (total + 7) / 8;
    const int32_t bid = blockIdx.x;
    const int32_t pos = bid >> 3;
    if (pos >= per_xcd) return false;
    const int32_t l = (bid & 7) * per_xcd + pos;
    if (l >= total) return false;
    constexpr int32_t CB = 4;
    const int32_t band = l / (ntiles * CB);
    const int32_t bw = min(CB, ta.col_tiles - band * CB);
    const int32_t rem = l - band * ntiles * CB;
    tile = rem / bw;
    ct = band * CB + rem % bw;
    return true;
}

// SWIGLU = true: GEMM-1 (gate/up + SwiGLU -> h); false: GEMM-2 (down -> o)
template <int BM, bool SWIGLU, int WF>
__global__ __launch_bounds__(THREADS) void gemm_tiled(TileArgs ta) {
    constexpr int WM = BM / 2;          // rows per wave
    constexpr int MT = WM / 32;         // 32-row MFMA tiles per wave
    constexpr int A_LD = BM * 8 / THREADS;  // 16-byte A chunks staged per thread per step
    constexpr int B_LD = NB * 8 / THREADS;  // 16-byte B chunks per thread per step (bf16)
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // LDS: A buffers [2][BM][128 B], then B buffers [2][NB][128 B]
    auto As = [&](int buf) -> char* { return smem + buf * (BM * 128); };
    auto Bs = [&](int buf) -> char* { return smem + 2 * BM * 128 + buf * (NB * 128); };

    const GroupedArgs& a = ta.a;
    int32_t tile, ct;
    if (!map_tile(ta, tile, ct)) return;
    const int32_t g = ta.tile_info[2 * tile], m0 = ta.tile_info[2 * tile + 1];
    if (g < ta.g0 || g >= ta.g1) return;
    const bool shared = g == a.E;
    int32_t r0, cnt;
    if (!shared) {
        r0 = a.offsets[g];
        cnt = a.offsets[g + 1] - r0;
    } else {
        r0 = a.TK;
        cnt = (int32_t)a.T;
    }
    const int32_t N = SWIGLU ? (shared ? a.Is : a.I) : a.H;       // output columns of this group
    const int32_t KD = SWIGLU ? a.H : (shared ? a.Is : a.I);      // reduction length
    constexpr int OUT_COLS = SWIGLU ? NB / 2 : NB;
    const int32_t n0 = ct * OUT_COLS;
    if (n0 >= N) return;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- per-thread global sources: uniform 64-bit bases + 32-bit element offsets -----------
    const bf16_t* a_base = SWIGLU ? (const bf16_t*)a.x : (const bf16_t*)a.h;
    uint32_t a_off[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int id = tid + THREADS * i;
        int32_t rr = m0 + id / 8;
        rr = rr < cnt ? rr : cnt - 1;  // clamp: rows past the group are computed, never stored
        const int32_t row = r0 + rr;
        const int c = id % 8;
        if (SWIGLU) {
            const int32_t tok = row < a.TK ? a.sorted_slot[row] / a.K : row - a.TK;
            a_off[i] = (uint32_t)tok * (uint32_t)a.H + c * 8;
        } else {
            a_off[i] = (uint32_t)row * (uint32_t)a.ldh + c * 8;
        }
    }
    // weight matrices of this group (uniform); B-tile row br maps to output column w_row(br),
    // clamped to N - 1 past the last column (such columns are never stored)
    const bf16_t *wb0 = nullptr, *wb1 = nullptr;   // bf16: gate/up (GEMM-1) or down (both = down)
    const uint32_t *qb0 = nullptr, *qb1 = nullptr; // 4-bit codes
    const bf16_t *sb0 = nullptr, *sb1 = nullptr, *zb0 = nullptr, *zb1 = nullptr;
    {
        const int32_t out_dim = SWIGLU ? a.I : a.H;
        const int64_t eoff = (int64_t)g * out_dim;  // first row of this expert
        if (WF == WF_BF16) {
            if (SWIGLU) {
                wb0 = shared ? (const bf16_t*)a.swg : (const bf16_t*)a.wg + eoff * KD;
                wb1 = shared ? (const bf16_t*)a.swu : (const bf16_t*)a.wu + eoff * KD;
            } else {
                wb0 = wb1 = shared ? (const bf16_t*)a.swd : (const bf16_t*)a.wd + eoff * KD;
            }
        } else {
            if (SWIGLU) {
                qb0 = (const uint32_t*)a.wg + eoff * (KD / 8);
                qb1 = (const uint32_t*)a.wu + eoff * (KD / 8);
                sb0 = a.sg + eoff * (KD / 64);
                sb1 = a.su + eoff * (KD / 64);
                zb0 = a.bg + eoff * (KD / 64);
                zb1 = a.bu + eoff * (KD / 64);
            } else {
                qb0 = qb1 = (const uint32_t*)a.wd + eoff * (KD / 8);
                sb0 = sb1 = a.sd + eoff * (KD / 64);
                zb0 = zb1 = a.bd + eoff * (KD / 64);
            }
        }
    }
    constexpr int QL = B_LD / 4;  // 4-bit: 16-byte code loads per thread per step
    uint32_t b_off[WF == WF_BF16 ? B_LD : QL];
    bool b_hi[WF == WF_BF16 ? B_LD : QL];  // row belongs to the second matrix (up)
#pragma unroll
    for (int i = 0; i < (WF == WF_BF16 ? B_LD : QL); ++i) {
        const int id = tid + THREADS * i;
        const int br = WF == WF_BF16 ? id / 8 : id / 2;
        int32_t n = n0 + (SWIGLU ? br % (NB / 2) : br);
        n = n < N ? n : N - 1;
        b_hi[i] = SWIGLU && br >= NB / 2;
        if (WF == WF_BF16)
            b_off[i] = (uint32_t)n * (uint32_t)KD + (id % 8) * 8;
        else
            b_off[i] = (uint32_t)n * (uint32_t)(KD / 8) + (id % 2) * 4;  // word offset of the half row
    }

    // ---- staging registers --------------------------------------------------------------
    u32x4 ra[A_LD];
    u32x4 rb[WF == WF_BF16 ? B_LD : QL];
    float rs[QL], rz[QL];

    // ---- accumulators -------------------------------------------------------------------
    // wave tile: WM rows x 128 weight rows = MT x 4 MFMA tiles of 32 x 32
    f32x16 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // B-tile rows of this wave's 4 column tiles
    int brow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (SWIGLU)  // tiles 0,1: gate rows; 2,3: the matching up rows
            brow[j] = (j < 2 ? 0 : NB / 2) + wn * 64 + (j & 1) * 32;
        else
            brow[j] = wn * 128 + j * 32;
    }

    const int nk = KD / BK;
#define DSMOE_GLOAD(K0)                                                                       \
    do {                                                                                      \
        const int32_t k_ = (K0);                                                              \
        _Pragma("unroll") for (int i = 0; i < A_LD; ++i) ra[i] = *(const u32x4*)(a_base + a_off[i] + k_); \
        if constexpr (WF == WF_BF16) {                                                        \
            _Pragma("unroll") for (int i = 0; i < B_LD; ++i)                                  \
                rb[i] = *(const u32x4*)((b_hi[i] ? wb1 : wb0) + b_off[i] + k_);               \
        } else {                                                                              \
            _Pragma("unroll") for (int i = 0; i < QL; ++i) {                                  \
                const int br_ = (tid + THREADS * i) / 2;                                      \
                int32_t n_ = n0 + (SWIGLU ? br_ % (NB / 2) : br_);                            \
                n_ = n_ < N ? n_ : N - 1;                                                     \
                const uint32_t so_ = (uint32_t)n_ * (uint32_t)(KD / 64) + k_ / 64;            \
                rb[i] = *(const u32x4*)((b_hi[i] ? qb1 : qb0) + b_off[i] + k_ / 8);           \
                rs[i] = bf16_to_f32((b_hi[i] ? sb1 : sb0)[so_]);                              \
                rz[i] = bf16_to_f32((b_hi[i] ? zb1 : zb0)[so_]);                              \
            }                                                                                 \
        }                                                                                     \
    } while (0)
#define DSMOE_LSTORE(BUF)                                                                     \
    do {                                                                                      \
        char* as_ = As(BUF);                                                                  \
        char* bs_ = Bs(BUF);                                                                  \
        _Pragma("unroll") for (int i = 0; i < A_LD; ++i) {                                    \
            const int id = tid + THREADS * i;                                                 \
            *(u32x4*)(as_ + lds_off(id / 8, id % 8)) = ra[i];                                 \
        }                                                                                     \
        if constexpr (WF == WF_BF16) {                                                        \
            _Pragma("unroll") for (int i = 0; i < B_LD; ++i) {                                \
                const int id = tid + THREADS * i;                                             \
                *(u32x4*)(bs_ + lds_off(id / 8, id % 8)) = rb[i];                             \
            }                                                                                 \
        } else {                                                                              \
            _Pragma("unroll") for (int i = 0; i < QL; ++i) {                                  \
                const int id = tid + THREADS * i;                                             \
                const int br_ = id / 2, hf_ = id % 2;                                         \
                *(u32x4*)(bs_ + lds_off(br_, hf_ * 4 + 0)) = dequant8(rb[i][0], rs[i], rz[i]); \
                *(u32x4*)(bs_ + lds_off(br_, hf_ * 4 + 1)) = dequant8(rb[i][1], rs[i], rz[i]); \
                *(u32x4*)(bs_ + lds_off(br_, hf_ * 4 + 2)) = dequant8(rb[i][2], rs[i], rz[i]); \
                *(u32x4*)(bs_ + lds_off(br_, hf_ * 4 + 3)) = dequant8(rb[i][3], rs[i], rz[i]); \
            }                                                                                 \
        }                                                                                     \
    } while (0)
    DSMOE_GLOAD(0);
    DSMOE_LSTORE(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) DSMOE_GLOAD((kt + 1) * BK);
        const char* Ab = As(buf);
        const char* Bb = Bs(buf);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int c = 2 * s + (lane >> 5);
            bf16x8 af[MT], bfr[4];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int r = wm * WM + i * 32 + (lane & 31);
                af[i] = as_bf16x8(*(const u32x4*)(Ab + lds_off(r, c)));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = brow[j] + (lane & 31);
                bfr[j] = as_bf16x8(*(const u32x4*)(Bb + lds_off(r, c)));
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) DSMOE_LSTORE(buf ^ 1);
        __syncthreads();
    }
#undef DSMOE_GLOAD
#undef DSMOE_LSTORE

    // ---- epilogue -----------------------------------------------------------------------
    const int col_l = lane & 31, rgrp = (lane >> 5) * 4;
    if (SWIGLU) {
        bf16_t* h = (bf16_t*)a.h;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int32_t col = n0 + wn * 64 + j * 32 + col_l;
                if (col >= N) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int32_t rr = m0 + wm * WM + i * 32 + (v >> 2) * 8 + rgrp + (v & 3);
                    if (rr < cnt)
                        h[(int64_t)(r0 + rr) * a.ldh + col] = f32_to_bf16(silu_f(acc[i][j][v]) * acc[i][j + 2][v]);
                }
            }
    } else {
        bf16_t* o = (bf16_t*)a.o;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int32_t col = n0 + wn * 128 + j * 32 + col_l;
                if (col >= N) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int32_t rr = m0 + wm * WM + i * 32 + (v >> 2) * 8 + rgrp + (v & 3);
                    if (rr < cnt) o[(int64_t)(r0 + rr) * a.H + col] = f32_to_bf16(acc[i][j][v]);
                }
            }
    }
}


// ---------------------------------------------------------------------------------------------
// bf16 weights: direct-to-LDS loads into a 4-stage ring.
//
// global_load_lds_dwordx4 moves 16 bytes per lane straight into LDS (lane i of an instruction
// fills bytes [16 i, 16 i + 16) of a 1 KB block), so no staging registers are needed and three
// k-stages of 32 can be in flight while the matrix cores work on the fourth.  LDS rows are 64
// bytes (32 bf16); the four 16-byte chunks of row r sit at chunk c ^ (((r >> 1) ^ (r >> 2)) & 3),
// which makes the lanes of each ds_read_b128 phase (8 or 16 consecutive rows) hit distinct
// 16-byte bank groups.  A lane of a
// DMA instruction therefore fetches the logical chunk that its LDS slot holds.  The compiler
// does not track these LDS writes, so the waits are explicit: before stage s is read, each wave
// waits until at most the later stages' loads are outstanding (vmcnt) and then meets the others
// at a barrier; the slot refilled after that barrier is the one every wave finished reading in
// the previous iteration.
// ---------------------------------------------------------------------------------------------
namespace dma {
constexpr int BKD = 64;        // k per stage: a whole 128-byte line of every row
constexpr int ROWB = 128;      // bytes per LDS row
constexpr int NST = 2;         // ring depth
constexpr int LDS_MAX = 160 * 1024;
constexpr int ring_bytes(int bm) { return NST * (bm + 256) * ROWB; }
// chunk swizzle: the 8 chunks of row r are permuted by (r ^ r/8) mod 8, which keeps the MFMA
// operand reads free of bank conflicts whether a ds_read_b128 phase serves 8 lanes (rows r..r+7)
// or 16 lanes (rows r..r+15)
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ uint32_t off(int r, int c) { return (uint32_t)(r * ROWB + ((c ^ swz(r)) << 4)); }
}  // namespace dma

#define DSMOE_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Wait until at most N vector-memory operations of this wave are outstanding and its LDS reads
// have returned, then barrier.  The LDS DMA writes are invisible to the compiler's own wait
// insertion, hence the explicit counts.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// wait until at most `later` stages of D loads each are outstanding, then barrier
template <int D>
__device__ __forceinline__ void wait_stages(int later) {
    if (later <= 0) wait_vm_barrier<0>();
    else wait_vm_barrier<D>();
}

template <int BM, bool SWIGLU>
__global__ __launch_bounds__(THREADS) void gemm_dma(TileArgs ta) {
    using namespace dma;
    constexpr int WM = BM / 2;
    constexpr int MT = WM / 32;
    constexpr int A_BYTES = BM * ROWB, B_BYTES = NB * ROWB, ST_BYTES = A_BYTES + B_BYTES;
    constexpr int A_DMA = A_BYTES / 1024 / 4;  // DMA instructions per wave per stage
    constexpr int B_DMA = B_BYTES / 1024 / 4;
    constexpr int D = A_DMA + B_DMA;
    static_assert(ring_bytes(BM) <= LDS_MAX, "ring exceeds LDS");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const GroupedArgs& a = ta.a;
    int32_t tile, ct;
    if (!map_tile(ta, tile, ct)) return;
    const int32_t g = ta.tile_info[2 * tile], m0 = ta.tile_info[2 * tile + 1];
    if (g < ta.g0 || g >= ta.g1) return;
    const bool shared = g == a.E;
    int32_t r0, cnt;
    if (!shared) {
        r0 = a.offsets[g];
        cnt = a.offsets[g + 1] - r0;
    } else {
        r0 = a.TK;
        cnt = (int32_t)a.T;
    }
    const int32_t N = SWIGLU ? (shared ? a.Is : a.I) : a.H;
    const int32_t KD = SWIGLU ? a.H : (shared ? a.Is : a.I);
    constexpr int OUT_COLS = SWIGLU ? NB / 2 : NB;
    const int32_t n0 = ct * OUT_COLS;
    if (n0 >= N) return;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- DMA sources: instruction j of this wave fills LDS rows [8 (wave*X + j), +8); lane i
    // writes chunk i % 8 of row i / 8, so it fetches the logical chunk that the swizzle puts there
    const bf16_t* a_base = SWIGLU ? (const bf16_t*)a.x : (const bf16_t*)a.h;
    uint32_t a_off[A_DMA];
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
        const int r = (wave * A_DMA + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        int32_t rr = m0 + r;
        rr = rr < cnt ? rr : cnt - 1;  // rows past the group are computed, never stored
        const int32_t row = r0 + rr;
        if (SWIGLU) {
            const int32_t tok = row < a.TK ? a.sorted_slot[row] / a.K : row - a.TK;
            a_off[j] = (uint32_t)tok * (uint32_t)a.H + c * 8;
        } else {
            a_off[j] = (uint32_t)row * (uint32_t)a.ldh + c * 8;
        }
    }
    const bf16_t *wb0, *wb1;
    {
        const int64_t eoff = (int64_t)g * (SWIGLU ? a.I : a.H);
        if (SWIGLU) {
            wb0 = shared ? (const bf16_t*)a.swg : (const bf16_t*)a.wg + eoff * KD;
            wb1 = shared ? (const bf16_t*)a.swu : (const bf16_t*)a.wu + eoff * KD;
        } else {
            wb0 = wb1 = shared ? (const bf16_t*)a.swd : (const bf16_t*)a.wd + eoff * KD;
        }
    }
    uint32_t b_off[B_DMA];
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) {
        const int br = (wave * B_DMA + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(br);
        int32_t n = n0 + (SWIGLU ? br % (NB / 2) : br);
        n = n < N ? n : N - 1;  // columns past N are computed, never stored
        b_off[j] = (uint32_t)n * (uint32_t)KD + c * 8;
    }
    // a wave's B instruction j covers 8 rows, all gate or all up (NB/2 is a multiple of 8)
    auto issue = [&](int kt) {
        char* st = smem + (kt % NST) * ST_BYTES;
        const int32_t k0 = kt * BKD;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(a_base + a_off[j] + k0),
                                             DSMOE_LDS_PTR(st + (wave * A_DMA + j) * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j) {
            const int br0 = (wave * B_DMA + j) * 8;
            const bf16_t* wb = (SWIGLU && br0 >= NB / 2) ? wb1 : wb0;
            __builtin_amdgcn_global_load_lds((const void*)(wb + b_off[j] + k0),
                                             DSMOE_LDS_PTR(st + A_BYTES + (wave * B_DMA + j) * 1024), 16, 0, 0);
        }
    };

    f32x16 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    int brow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) brow[j] = SWIGLU ? (j < 2 ? 0 : NB / 2) + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32;

    // Software pipeline over k16 steps (four per stage): the fragments of the next step are read
    // from LDS while the current step's MFMAs run.  The wait + barrier that publishes stage kt+1
    // sits before the last step of stage kt; once every wave has passed it, the fragments of
    // stage kt are all in registers, so its slot is refilled with stage kt+NST right away and
    // those loads have the next four steps to land.
    const int nk = KD / BKD;  // >= 1
    bf16x8 fa[2][MT], fb[2][4];
    auto read_frags = [&](int kt, int s, int buf) {
        const char* st = smem + (kt % NST) * ST_BYTES;
        const int c = 2 * s + (lane >> 5);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fb[buf][j] = as_bf16x8(*(const u32x4*)(st + A_BYTES + off(brow[j] + (lane & 31), c)));
#pragma unroll
        for (int i = 0; i < MT; ++i) fa[buf][i] = as_bf16x8(*(const u32x4*)(st + off(wm * WM + i * 32 + (lane & 31), c)));
    };
    // one k16 step: its first MFMA, then (optionally) the next step's fragment reads, then the
    // remaining MFMAs -- pinned in that order so each LDS read issues under a running MFMA
    auto mfma_step = [&](int buf, bool then_read, int rkt, int rs, int rbuf) {
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][0], fb[buf][0], acc[0][0], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (then_read) {
            read_frags(rkt, rs, rbuf);
            __builtin_amdgcn_sched_group_barrier(0x100, MT + 4, 0);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (i | j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MT * 4 - 1, 0);
    };
    const int pro = min(nk, NST);  // stages issued up front
    for (int j = 0; j < pro; ++j) issue(j);
    wait_stages<D>(pro - 1);
    read_frags(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        mfma_step(0, true, kt, 1, 1);
        mfma_step(1, true, kt, 2, 0);
        mfma_step(0, true, kt, 3, 1);
        const bool next = kt + 1 < nk;
        if (next) {
            // issued so far: stages < min(nk, kt + NST); wait for kt+1, let the later ones fly
            wait_stages<D>(min(nk, kt + NST) - (kt + 2));
            if (kt + NST < nk) issue(kt + NST);
        }
        mfma_step(1, next, kt + 1, 0, 0);
    }

    const int col_l = lane & 31, rgrp = (lane >> 5) * 4;
    if (SWIGLU) {
        bf16_t* h = (bf16_t*)a.h;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int32_t col = n0 + wn * 64 + j * 32 + col_l;
                if (col >= N) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int32_t rr = m0 + wm * WM + i * 32 + (v >> 2) * 8 + rgrp + (v & 3);
                    if (rr < cnt)
                        h[(int64_t)(r0 + rr) * a.ldh + col] = f32_to_bf16(silu_f(acc[i][j][v]) * acc[i][j + 2][v]);
                }
            }
    } else {
        bf16_t* o = (bf16_t*)a.o;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int32_t col = n0 + wn * 128 + j * 32 + col_l;
                if (col >= N) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int32_t rr = m0 + wm * WM + i * 32 + (v >> 2) * 8 + rgrp + (v & 3);
                    if (rr < cnt) o[(int64_t)(r0 + rr) * a.H + col] = f32_to_bf16(acc[i][j][v]);
                }
            }
    }
}

// Tile list: every group in [0, E] (E = shared expert) with more than `min_rows` rows gets
// ceil(rows / BM) tiles, in group order.  One workgroup; group 1024 (only possible with
// E == 1024 plus a shared expert) is appended by thread 0.
__global__ __launch_bounds__(1024) void tiles_kernel(const int32_t* __restrict__ offsets, int32_t E, int64_t T,
                                                     int32_t has_shared, int32_t BM, int32_t min_rows,
                                                     int32_t* __restrict__ tile_count,
                                                     int32_t* __restrict__ tile_info) {
    __shared__ int32_t buf[1024];
    const int t = threadIdx.x;
    const int32_t ng = E + has_shared;
    auto ntiles = [&](int32_t g) -> int32_t {
        const int32_t cnt = g < E ? offsets[g + 1] - offsets[g] : (int32_t)T;
        return cnt > min_rows ? (cnt + BM - 1) / BM : 0;
    };
    const int32_t n = t < ng ? ntiles(t) : 0;
    buf[t] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = t >= off ? buf[t - off] : 0;
        __syncthreads();
        buf[t] += v;
        __syncthreads();
    }
    const int32_t start = buf[t] - n;
    for (int32_t m = 0; m < n; ++m) {
        tile_info[2 * (start + m)] = t;
        tile_info[2 * (start + m) + 1] = m * BM;
    }
    if (t == 0) {
        int32_t total = buf[1023];
        if (ng > 1024) {
            const int32_t nn = ntiles(1024);
            for (int32_t m = 0; m < nn; ++m) {
                tile_info[2 * (total + m)] = 1024;
                tile_info[2 * (total + m) + 1] = m * BM;
            }
            total += nn;
        }
        tile_count[0] = total;
    }
}

template <int BM, bool SW>
hipError_t launch_dma_t(const TileArgs& ta, hipStream_t s) {
    const size_t lds = (size_t)dma::ring_bytes(BM);
    const unsigned grid = (unsigned)(((ta.nwg + 7) / 8) * 8);
    hipLaunchKernelGGL((gemm_dma<BM, SW>), dim3(grid), dim3(THREADS), lds, s, ta);
    return hipGetLastError();
}

template <int BM, bool SW, int WF>
hipError_t launch_tiled_t(const TileArgs& ta, hipStream_t s) {
    const size_t lds = 2 * (size_t)(BM + NB) * 128;
    const unsigned grid = (unsigned)(((ta.nwg + 7) / 8) * 8);  // the XCD remap needs a multiple of 8
    hipLaunchKernelGGL((gemm_tiled<BM, SW, WF>), dim3(grid), dim3(THREADS), lds, s, ta);
    return hipGetLastError();
}

}  // namespace

int32_t tiled_max_tiles(int64_t T, int32_t K, int32_t E, int32_t BM) {
    const int64_t rows = T * K + T;
    return (int32_t)((rows + BM - 1) / BM + E + 1);
}

// largest dynamic LDS any tiled kernel of this tile height uses
int32_t tiled_lds_bytes(int32_t BM) {
    const int32_t reg_staged = 2 * (BM + NB) * 128, dma_ring = dma::ring_bytes(BM);
    return reg_staged > dma_ring ? reg_staged : dma_ring;
}

hipError_t configure_tiled_kernels() {
    // allow the large dynamic LDS allocations (up to 128 KB) of the tiled kernels
    const void* ks[] = {
        (const void*)gemm_dma<256, true>,          (const void*)gemm_dma<256, false>,
        (const void*)gemm_tiled<256, true, WF_Q4>, (const void*)gemm_tiled<256, false, WF_Q4>,
        (const void*)gemm_dma<128, true>,          (const void*)gemm_dma<128, false>,
        (const void*)gemm_tiled<128, true, WF_Q4>, (const void*)gemm_tiled<128, false, WF_Q4>,
    };
    const int bms[] = {256, 256, 256, 256, 128, 128, 128, 128};
    for (int i = 0; i < 8; ++i) {
        hipError_t e = hipFuncSetAttribute(ks[i], hipFuncAttributeMaxDynamicSharedMemorySize, tiled_lds_bytes(bms[i]));
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_tiles(const GroupedArgs& a, int32_t BM, int32_t min_rows, int32_t* tile_count, int32_t* tile_info,
                        hipStream_t s) {
    hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.E, a.T, a.Is > 0 ? 1 : 0, BM, min_rows,
                       tile_count, tile_info);
    return hipGetLastError();
}

hipError_t launch_gemm_tiled(const GroupedArgs& a, bool gemm1, int32_t BM, int32_t g0, int32_t g1, int32_t wdt,
                             const int32_t* tile_count, const int32_t* tile_info, int32_t max_tiles, hipStream_t s) {
    if (g1 <= g0 || max_tiles <= 0) return hipSuccess;
    TileArgs ta;
    ta.a = a;
    ta.tile_count = tile_count;
    ta.tile_info = tile_info;
    ta.g0 = g0;
    ta.g1 = g1;
    const int32_t N = gemm1 ? (a.I > a.Is ? a.I : a.Is) : a.H;
    const int32_t out_cols = gemm1 ? NB / 2 : NB;
    ta.col_tiles = (N + out_cols - 1) / out_cols;
    ta.nwg = max_tiles * ta.col_tiles;
    const bool q4 = wdt == MOE_Q4G64;
    if (!q4) {
        if (BM == 256) return gemm1 ? launch_dma_t<256, true>(ta, s) : launch_dma_t<256, false>(ta, s);
        return gemm1 ? launch_dma_t<128, true>(ta, s) : launch_dma_t<128, false>(ta, s);
    }
    if (BM == 256) return gemm1 ? launch_tiled_t<256, true, WF_Q4>(ta, s) : launch_tiled_t<256, false, WF_Q4>(ta, s);
    return gemm1 ? launch_tiled_t<128, true, WF_Q4>(ta, s) : launch_tiled_t<128, false, WF_Q4>(ta, s);
}

}  // namespace dsmoe
