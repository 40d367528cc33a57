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
//   * operands reach LDS by direct-to-LDS DMA in k-stages of 64 (one 128-byte line per row),
//     through a ring of stages, with one barrier per stage (gemm_dma); 4-bit weights skip LDS and
//     are dequantised in registers (gemm_dma_q4);
//   * the list of (group, first row) tiles is built on the device from the dispatch offsets, so
//     no count ever returns to the host; the grid is an upper bound and surplus workgroups exit;
//   * workgroup ids are remapped so that the workgroups an XCD receives (ids congruent mod 8)
//     form a contiguous run of tiles, keeping the A and B panels they share in that XCD's L2.
//
// MFMA 32x32x16 bf16 layout: lane l supplies row/column (l % 32) and the 8 k values of chunk
// (l / 32) of each 16-k step; result element v of lane l is row 8*(v/4) + 4*(l/32) + v%4,
// column l % 32.  Which 8 k values a chunk holds is free as long as both operands agree.
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

constexpr int NB = 256;       // weight rows per tile
constexpr int THREADS = 256;  // 4 waves

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }


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

// ---------------------------------------------------------------------------------------------
// bf16 weights: direct-to-LDS loads into a ring of 64-k stages.
//
// global_load_lds_dwordx4 moves 16 bytes per lane straight into LDS (lane i of an instruction
// fills bytes [16 i, 16 i + 16) of a 1 KB block), so no staging registers are needed.  A stage
// holds 64 k of every row -- one whole 128-byte line, so each DMA instruction fetches 8 full
// lines (fetching half lines per instruction measured about a third slower).  The eight 16-byte
// chunks of row r sit at chunk c ^ ((r ^ r/8) & 7), which makes the lanes of each ds_read_b128
// phase (8 or 16 consecutive rows) hit distinct 16-byte bank groups; a lane of a DMA instruction
// therefore fetches the logical chunk that its LDS slot holds.  The compiler does not track
// these LDS writes, so the waits are explicit: before stage s is read, each wave waits until at
// most the later stages' loads are outstanding (vmcnt) and then meets the others at a barrier;
// the slot refilled after that barrier is the one every wave finished reading.  The 2 x 2 waves
// each own a 128-row x 128-weight-row quarter of the tile.
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

// Epilogue of a 32x32-MFMA tile: rows [mrow, mrow + 32 MT) of the group, the wave's output
// columns.  GEMM-1 holds gate accumulators in j = 0, 1 and up in j = 2, 3 (64 output columns
// per wave) and writes bf16(silu(gate) * up) to h; GEMM-2 writes its 128 columns to o.
template <int MT, bool SWIGLU>
__device__ __forceinline__ void tile_epilogue(const GroupedArgs& a, const f32x16 (&acc)[MT][4], int32_t r0,
                                              int32_t cnt, int32_t mrow, int32_t n0, int32_t N, int wn, int lane) {
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
                    const int32_t rr = mrow + i * 32 + (v >> 2) * 8 + rgrp + (v & 3);
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
                    const int32_t rr = mrow + i * 32 + (v >> 2) * 8 + rgrp + (v & 3);
                    if (rr < cnt) o[(int64_t)(r0 + rr) * a.H + col] = f32_to_bf16(acc[i][j][v]);
                }
            }
    }
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

    // the wave index is uniform: keep it scalar so the DMA destinations (M0) are scalar too
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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
            a_off[j] = ((uint32_t)tok * (uint32_t)a.H + c * 8) * 2u;
        } else {
            a_off[j] = ((uint32_t)row * (uint32_t)a.ldh + c * 8) * 2u;
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
        b_off[j] = ((uint32_t)n * (uint32_t)KD + c * 8) * 2u;
    }
    // a wave's B instruction j covers 8 rows, all gate or all up (NB/2 is a multiple of 8)
    // DMA sources are a uniform base (advanced by the stage) plus a per-lane 32-bit byte offset,
    // so no per-lane 64-bit address arithmetic is issued per instruction
    auto issue = [&](int kt) {
        char* st = smem + (kt % NST) * ST_BYTES;
        const int32_t k0 = kt * BKD;
        const char* ab = (const char*)(a_base + k0);
#pragma unroll
        for (int j = 0; j < A_DMA; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(ab + a_off[j]),
                                             DSMOE_LDS_PTR(st + (wave * A_DMA + j) * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j) {
            const int br0 = (wave * B_DMA + j) * 8;
            const char* wb = (const char*)(((SWIGLU && br0 >= NB / 2) ? wb1 : wb0) + k0);
            __builtin_amdgcn_global_load_lds((const void*)(wb + b_off[j]),
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

    tile_epilogue<MT, SWIGLU>(a, acc, r0, cnt, m0 + wm * WM, n0, N, wn, lane);
}


// ---------------------------------------------------------------------------------------------
// 4-bit weights (affine, groups of 64 along the reduction axis), tiles of 128 rows.  Same tile
// shape, activation ring and tile list as gemm_dma; the packed codes are four times smaller than
// bf16 rows, so they skip LDS: each lane loads the codes it multiplies straight into registers,
// two stages ahead, with its row's scale and offset for the stage (one 64-k stage is one
// quantisation group), and forms bf16(s*q + b) one k16 step before the MFMAs that consume it.
// The dequantisation runs on the vector ALU beside the matrix cores; to keep it at one pass per
// weight the four waves split the tile by columns (1 x 4): wave w owns all 128 rows and, for
// GEMM-1, the gate and up rows of output columns [32 w, 32 w + 32), for GEMM-2 the 64 columns
// [64 w, 64 w + 64).  Within a stage the k chunks are taken in the order 4h + s (lane half h,
// step s) for both operands, so a lane's codes for the whole stage are one 16-byte load.
// Per wave and stage the vector-memory issue order is: codes/scales of stage kt+2, then the
// activation DMA of stage kt+NQ (A_DMA loads).  At the barrier before the last step of stage
// kt everything but the newest A_DMA operations must have landed: that covers the activations
// and the codes of stage kt+1.
// ---------------------------------------------------------------------------------------------
namespace q4t {
constexpr int BM = 128;
constexpr int NQ = 3;  // activation ring depth
constexpr int ring_bytes() { return NQ * BM * dma::ROWB; }
}  // namespace q4t

template <bool SWIGLU>
__global__ __launch_bounds__(THREADS) void gemm_dma_q4(TileArgs ta) {
    using namespace dma;
    using q4t::NQ;
    constexpr int BM = q4t::BM;
    constexpr int MT = BM / 32;                // 32-row blocks per wave (all rows of the tile)
    constexpr int A_BYTES = BM * ROWB;
    constexpr int A_DMA = A_BYTES / 1024 / 4;  // DMA instructions per wave per stage
    static_assert(q4t::ring_bytes() <= LDS_MAX, "ring exceeds LDS");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const GroupedArgs& a = ta.a;
    int32_t tile, ct;
    if (!map_tile(ta, tile, ct)) return;
    const int32_t g = ta.tile_info[2 * tile], m0 = ta.tile_info[2 * tile + 1];
    if (g < ta.g0 || g >= ta.g1 || g >= a.E) return;  // routed groups only (the shared expert is bf16)
    const int32_t r0 = a.offsets[g];
    const int32_t cnt = a.offsets[g + 1] - r0;
    const int32_t N = SWIGLU ? a.I : a.H;
    const int32_t KD = SWIGLU ? a.H : a.I;
    constexpr int OUT_COLS = SWIGLU ? NB / 2 : NB;
    const int32_t n0 = ct * OUT_COLS;
    if (n0 >= N) return;

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, half = lane >> 5;

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
            const int32_t tok = a.sorted_slot[row] / a.K;
            a_off[j] = ((uint32_t)tok * (uint32_t)a.H + c * 8) * 2u;
        } else {
            a_off[j] = ((uint32_t)row * (uint32_t)a.ldh + c * 8) * 2u;
        }
    }
    // output column of B block j for this lane: GEMM-1 gate (j = 0) and up (j = 1) rows of
    // column 32 w + lane % 32; GEMM-2 rows 64 w + 32 j + lane % 32.  The expert's matrices are
    // uniform bases; per lane only 32-bit offsets within them are kept.
    const int64_t eq = (int64_t)g * N * (KD / 8), es = (int64_t)g * N * (KD / 64);
    const uint32_t* qb0 = (const uint32_t*)(SWIGLU ? a.wg : a.wd) + eq;
    const uint32_t* qb1 = (const uint32_t*)(SWIGLU ? a.wu : a.wd) + eq;
    const bf16_t* sb0 = (SWIGLU ? a.sg : a.sd) + es;
    const bf16_t* sb1 = (SWIGLU ? a.su : a.sd) + es;
    const bf16_t* bb0 = (SWIGLU ? a.bg : a.bd) + es;
    const bf16_t* bb1 = (SWIGLU ? a.bu : a.bd) + es;
    int32_t ncol[2];
    uint32_t qoff[2], soff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        ncol[j] = n0 + (SWIGLU ? wave * 32 : wave * 64 + j * 32) + (lane & 31);
        const int32_t n = ncol[j] < N ? ncol[j] : N - 1;  // columns past N are computed, never stored
        qoff[j] = (uint32_t)n * (uint32_t)(KD / 8) + half * 4;
        soff[j] = (uint32_t)n * (uint32_t)(KD / 64);
    }
    struct BStage {
        u32x4 q[2];
        bf16_t s[2], b[2];
    };
    auto load_b = [&](int kt, BStage& st) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            st.q[j] = *(const u32x4*)((j ? qb1 : qb0) + qoff[j] + kt * 8);
            st.s[j] = (j ? sb1 : sb0)[soff[j] + kt];
            st.b[j] = (j ? bb1 : bb0)[soff[j] + kt];
        }
    };
    auto issue_a = [&](int kt) {
        char* st = smem + (kt % NQ) * A_BYTES;
        const char* ab = (const char*)(a_base + kt * BKD);
#pragma unroll
        for (int j = 0; j < A_DMA; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(ab + a_off[j]),
                                             DSMOE_LDS_PTR(st + (wave * A_DMA + j) * 1024), 16, 0, 0);
    };

    f32x16 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i][0] = acc[i][1] = f32x16{};

    const int nk = KD / BKD;  // >= 1
    bf16x8 fa[2][MT], fb[2][2];
    // operands of step s of stage kt: activations from LDS, weights dequantised from registers
    auto frags = [&](int kt, int s, int buf, const BStage& bs) {
        const char* st = smem + (kt % NQ) * A_BYTES;
        const int c = 4 * half + s;
#pragma unroll
        for (int i = 0; i < MT; ++i) fa[buf][i] = as_bf16x8(*(const u32x4*)(st + off(i * 32 + (lane & 31), c)));
#pragma unroll
        for (int j = 0; j < 2; ++j)
            fb[buf][j] = as_bf16x8(dequant8(bs.q[j][s], bf16_to_f32(bs.s[j]), bf16_to_f32(bs.b[j])));
    };
    auto mfma_step = [&](int buf) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
    };
    // one stage; `cur` holds its codes, `nxt` those of stage kt+1 (landed by the barrier)
    auto stage = [&](int kt, BStage& cur, const BStage& nxt) {
        frags(kt, 1, 1, cur);
        mfma_step(0);
        frags(kt, 2, 0, cur);
        mfma_step(1);
        frags(kt, 3, 1, cur);
        mfma_step(0);
        const bool next = kt + 1 < nk;
        if (next) {
            // A(kt+2) (issued last, during stage kt-1) may still fly; all older loads must land
            if (kt >= 1 && kt + 2 < nk) wait_vm_barrier<A_DMA>();
            else wait_vm_barrier<0>();
            if (kt + 2 < nk) load_b(kt + 2, cur);  // cur's codes are all dequantised
            if (kt + NQ < nk) issue_a(kt + NQ);    // the slot of stage kt is fully read
            frags(kt + 1, 0, 0, nxt);
        }
        mfma_step(1);
    };

    BStage b0, b1;
    const int pro = min(nk, NQ);
    for (int j = 0; j < pro; ++j) issue_a(j);
    load_b(0, b0);
    if (nk > 1) load_b(1, b1);
    wait_vm_barrier<0>();
    frags(0, 0, 0, b0);
    for (int kt = 0; kt < nk; kt += 2) {  // two code sets, alternating by stage parity
        stage(kt, b0, b1);
        if (kt + 1 < nk) stage(kt + 1, b1, b0);
    }

    // the accumulators of the last MFMAs are read right away: give the MFMA-to-VALU wait states
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0][0]));
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (i | j) asm volatile("" : "+a"(acc[i][j]));

    const int rgrp = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < (SWIGLU ? 1 : 2); ++j) {
            const int32_t col = ncol[j];
            if (col >= N) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int32_t rr = m0 + i * 32 + (v >> 2) * 8 + rgrp + (v & 3);
                if (rr >= cnt) continue;
                if (SWIGLU)
                    ((bf16_t*)a.h)[(int64_t)(r0 + rr) * a.ldh + col] =
                        f32_to_bf16(silu_f(acc[i][0][v]) * acc[i][1][v]);
                else
                    ((bf16_t*)a.o)[(int64_t)(r0 + rr) * a.H + col] = f32_to_bf16(acc[i][j][v]);
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

template <bool SW>
hipError_t launch_dma_q4_t(const TileArgs& ta, hipStream_t s) {
    const size_t lds = (size_t)q4t::ring_bytes();
    const unsigned grid = (unsigned)(((ta.nwg + 7) / 8) * 8);
    hipLaunchKernelGGL((gemm_dma_q4<SW>), dim3(grid), dim3(THREADS), lds, s, ta);
    return hipGetLastError();
}


}  // namespace

int32_t tiled_max_tiles(int64_t T, int32_t K, int32_t E, int32_t BM) {
    const int64_t rows = T * K + T;
    return (int32_t)((rows + BM - 1) / BM + E + 1);
}

// largest dynamic LDS any tiled kernel of this tile height uses
int32_t tiled_lds_bytes(int32_t BM) {
    const int32_t dma_ring = dma::ring_bytes(BM), q4_ring = q4t::ring_bytes();
    return BM == q4t::BM && q4_ring > dma_ring ? q4_ring : dma_ring;
}

hipError_t configure_tiled_kernels() {
    // allow the large dynamic LDS allocations (up to 128 KB) of the tiled kernels
    const void* ks[] = {
        (const void*)gemm_dma<256, true>, (const void*)gemm_dma<256, false>, (const void*)gemm_dma<128, true>,
        (const void*)gemm_dma<128, false>, (const void*)gemm_dma_q4<true>,   (const void*)gemm_dma_q4<false>,
    };
    const int bms[] = {256, 256, 128, 128, 128, 128};
    for (int i = 0; i < 6; ++i) {
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
    // 4-bit layers always use tiles of 128 rows (plan_tiles)
    if (BM != 128) return hipErrorInvalidValue;
    return gemm1 ? launch_dma_q4_t<true>(ta, s) : launch_dma_q4_t<false>(ta, s);
}

}  // namespace dsmoe
