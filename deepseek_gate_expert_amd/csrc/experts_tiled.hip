// experts_tiled.hip - LDS-tiled grouped expert GEMMs for groups with many rows.
//
// Same computation as experts.hip (page "Epic: Engine Inference Core Stage E - MoE + hybrid
// families", opening paragraph: the per-expert matmuls of gather_mm / gather_qmm; SwiGLU fused
// into the gate/up GEMM's epilogue), organised for the prefill regime where a group holds
// hundreds or thousands of rows and the work is bound by MFMA throughput:
//
//   * a workgroup computes a BM x 256 tile: BM rows of one group against 256 rows of weights --
//     for GEMM-1 the gate and up rows of the same 128 output columns, for GEMM-2 256 rows of
//     W_down -- with v_mfma_f32_32x32x16_bf16 and fp32 accumulators, multiplying only the
//     32-row blocks that hold rows of the group;
//   * operands reach LDS by direct-to-LDS DMA in k-stages of 64 (one 128-byte line per row),
//     through a ring of stages, with one barrier per stage: bf16 weights in 8-wave workgroups
//     (gemm_dma); 4-bit and fp8 codes and scales in 4-wave workgroups that dequantise them in
//     registers before the MFMA (gemm_dma_wq);
//   * the list of (group, first row) tiles is built on the device from the dispatch offsets, so
//     no count ever returns to the host; the grid is an upper bound and surplus workgroups exit;
//   * workgroup ids are remapped so that the workgroups an XCD receives (ids congruent mod 8)
//     form a contiguous run of tiles, keeping the A and B panels they share in that XCD's L2.
//
// MFMA 32x32x16 bf16 layout: lane l supplies row/column (l % 32) and the 8 k values of chunk
// (l / 32) of each 16-k step; result element v of lane l is row 8*(v/4) + 4*(l/32) + v%4,
// column l % 32.  Which 8 k values a chunk holds is free as long as both operands agree.
#include <type_traits>
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

constexpr int NB = 256;       // weight rows per tile
constexpr int THREADS = 256;  // 4 waves

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }


// Eight 4-bit codes (code i at bits 4i) -> bf16(s q + b), given s512 = 512 s.  A code q in the
// low nibble of a byte, read as an OCP E4M3 code, has the value q * 2^-9 (a subnormal for q < 8,
// exponent field 1 above), so one hardware E4M3 -> fp32 conversion turns two codes into exact
// floats; 512 s * (q * 2^-9) is exactly s q, so the fma rounds s q + b once, as fma(s, q, b) would.
// (512 s overflows only for |s| > 6.6e35.)
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float s512, float b) {
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
    return r;
}

// eight E4M3 codes (two words, code i at bits 8*(i%4) of word i/4) -> bf16(value * s): hardware
// E4M3 -> fp32 conversion, fp32 multiply, round to nearest even
__device__ __forceinline__ u32x4 dequant_f8x8(uint32_t lo, uint32_t hi, float s) {
    u32x4 r;
    const auto v0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);  // codes 0, 1
    const auto v1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);   // codes 2, 3
    const auto v2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const auto v3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    r[0] = pack_bf16x2(v0[0] * s, v0[1] * s);
    r[1] = pack_bf16x2(v1[0] * s, v1[1] * s);
    r[2] = pack_bf16x2(v2[0] * s, v2[1] * s);
    r[3] = pack_bf16x2(v3[0] * s, v3[1] * s);
    return r;
}

// silu with the hardware reciprocal (about 1 ulp; the product is rounded to bf16 anyway)
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

struct TileArgs {
    GroupedArgs a;
    const int32_t* tile_count;  // [2]: tiles in the list, tiles of the groups below E (the routed
                                //   ones; the shared expert's tiles follow them)
    const int32_t* tile_info;   // [max_tiles][4]: group, first row within the group, the group's
                                //   first row in the row space, its row count
    int32_t g0, g1;             // groups handled by this launch
    int32_t part;               // tiles it maps: 0 all, 1 those below E, 2 those from E on
    int32_t col_tiles;          // output column tiles per row tile
    int32_t nwg;                // workgroups launched
};

// Workgroup -> (tile, column tile).  The logical space holds the launch's tiles (all of the
// list, or only the routed or only the shared part of it, so that a launch over one part spreads
// that part over every XCD) times col_tiles items, in bands of CB column tiles (measured: 2 for
// the bf16 gate/up kernel and 8 for the bf16 down projection, whose 256 x 256 tiles hold 144 KB
// of LDS, one per CU; 16 for the 4-bit gate/up kernel, 32 for its down projection and 8 for the
// fp8 kernel, two per CU, whose small groups put few row tiles in a band): items of one
// band walk the row tiles with the column fastest, so the workgroups running at once share both A
// panels (same rows) and B panels (same group and columns).  Workgroup ids congruent mod 8 land
// on the same XCD; each XCD takes one contiguous eighth of the logical space, sized by the tile
// count actually built (the grid is a bound).
template <int32_t CB>
__device__ __forceinline__ bool map_tile(const TileArgs& ta, int32_t& tile, int32_t& ct) {
    const int32_t t0 = ta.part == 2 ? ta.tile_count[1] : 0;
    const int32_t ntiles = (ta.part == 1 ? ta.tile_count[1] : ta.tile_count[0]) - t0;
    const int32_t total = ntiles * ta.col_tiles;
    const int32_t per_xcd = (total + 7) / 8;
    const int32_t bid = blockIdx.x;
    const int32_t pos = bid >> 3;
    if (pos >= per_xcd) return false;
    const int32_t l = (bid & 7) * per_xcd + pos;
    if (l >= total) return false;
    const int32_t band = l / (ntiles * CB);
    const int32_t bw = min(CB, ta.col_tiles - band * CB);
    const int32_t rem = l - band * ntiles * CB;
    tile = t0 + rem / bw;
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
constexpr int THREADS = 512;   // 8 waves, two per SIMD
constexpr int PRODUCERS = 4;   // waves 0..3 issue the DMA, one per SIMD
constexpr int ring_bytes(int bm) { return NST * (bm + 256) * ROWB; }
// after the ring: each producer lane's DMA source offsets (A and B, up to 8 each), kept in LDS
// rather than in 16 registers (one ds_read_b128 per four offsets at each stage's issue; this
// lowers the kernel's register count by about 10 and measured no slower);
// [producer][A 0..3, A 4..7, B 0..3, B 4..7][lane] 16-byte groups
constexpr int OFFS_BYTES = 4 * 4 * 64 * 16;
constexpr int lds_bytes(int bm) { return ring_bytes(bm) + OFFS_BYTES; }
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

// Epilogue of a gemm_dma tile, staged through LDS (the stage ring is free once every wave has
// left the k loop): each wave writes its bf16 results -- GEMM-1: bf16(silu(gate) * up), gate
// accumulators in j = 0 and up in j = 1, 32 output columns per wave; GEMM-2: 64 columns -- into
// a row-major image of the output tile, then all threads copy it out in 16-byte row pieces.
// The k loop multiplies with the weights as the MFMA's first operand, so a lane's accumulator
// elements 4q .. 4q+3 are four consecutive output columns of one token row: each goes to the
// image as one 8-byte write (16 per lane for GEMM-2 where 2-byte writes took 128).  In the image
// the 16-byte chunk c of row r sits at chunk c ^ (r mod CPR), so the 32 rows of one write
// instruction spread over every bank.  Rows past the group and columns past N are not stored.
template <int BM, bool SWIGLU>
__device__ __forceinline__ void tile_epilogue(const GroupedArgs& a, const f32x16 (&acc)[BM / 64][2], char* smem,
                                              int32_t r0, int32_t cnt, int32_t m0, int32_t n0, int32_t N, int wm,
                                              int wn, int tid) {
    constexpr int MT = BM / 64;
    constexpr int WM = BM / 2;
    constexpr int OUT_COLS = SWIGLU ? NB / 2 : NB;
    constexpr int RB = OUT_COLS * 2;  // bytes per image row
    constexpr int CPR = OUT_COLS / 8;  // 16-byte chunks per row
    static_assert(BM * RB <= dma::ring_bytes(BM), "output image exceeds the ring");
    static_assert((CPR & (CPR - 1)) == 0, "chunks per row: a power of two");
    const int lane = tid & 63, trow = lane & 31, half = lane >> 5;
    auto chunk_at = [](int r, int c) { return r * RB + ((c ^ (r & (CPR - 1))) << 4); };
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every wave is done with the ring
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int row = wm * WM + i * 32 + trow;
#pragma unroll
        for (int j = 0; j < (SWIGLU ? 1 : 2); ++j) {
            const int c0 = SWIGLU ? wn * 4 : wn * 8 + j * 4;  // first 16-byte chunk of the 32 columns
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = SWIGLU ? silu_f(acc[i][0][4 * q + e]) * acc[i][1][4 * q + e] : acc[i][j][4 * q + e];
                *(u32x2*)(smem + chunk_at(row, c0 + q) + half * 8) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    bf16_t* dst = SWIGLU ? (bf16_t*)a.h : (bf16_t*)a.o;
    const int64_t ld = SWIGLU ? a.ldh : a.H;
#pragma unroll
    for (int k = 0; k < BM * CPR / dma::THREADS; ++k) {
        const int q = tid + k * dma::THREADS;
        const int row = q / CPR, c = q % CPR;
        const int32_t col = n0 + c * 8;
        if (m0 + row >= cnt || col >= N) continue;
        const u32x4 v = *(const u32x4*)(smem + chunk_at(row, c));
        *(u32x4*)(dst + (int64_t)(r0 + m0 + row) * ld + col) = v;
    }
}

template <int BM, bool SWIGLU>
__global__ __launch_bounds__(dma::THREADS) void gemm_dma(TileArgs ta) {
    using namespace dma;
    constexpr int WM = BM / 2;
    constexpr int MT = WM / 32;
    constexpr int A_BYTES = BM * ROWB, B_BYTES = NB * ROWB, ST_BYTES = A_BYTES + B_BYTES;
    constexpr int A_DMA = A_BYTES / 1024 / PRODUCERS;  // DMA instructions per producer wave per stage
    constexpr int B_DMA = B_BYTES / 1024 / PRODUCERS;
    constexpr int D = A_DMA + B_DMA;
    static_assert(lds_bytes(BM) <= LDS_MAX && A_DMA <= 8 && B_DMA <= 8, "ring exceeds LDS");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const GroupedArgs& a = ta.a;
    int32_t tile, ct;
    if (!map_tile<SWIGLU ? 2 : 8>(ta, tile, ct)) return;
    const i32x4 ti = *(const i32x4*)(ta.tile_info + 4 * tile);  // group, first row, group rows
    const int32_t g = ti[0], m0 = ti[1], r0 = ti[2], cnt = ti[3];
    if (g < ta.g0 || g >= ta.g1) return;
    const bool shared = g == a.E;
    const int32_t N = SWIGLU ? (shared ? a.Is : a.I) : a.H;
    const int32_t KD = SWIGLU ? a.H : (shared ? a.Is : a.I);
    constexpr int OUT_COLS = SWIGLU ? NB / 2 : NB;
    const int32_t n0 = ct * OUT_COLS;
    if (n0 >= N) return;

    // the wave index is uniform: keep it scalar so the DMA destinations (M0) are scalar too
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wm = wave >> 2, wn = wave & 3;
    const int pw = wave & (PRODUCERS - 1);  // producer index (waves >= PRODUCERS issue no DMA)

    // ---- DMA sources: instruction j of producer pw fills LDS rows [8 (pw*X + j), +8); lane i
    // writes chunk i % 8 of row i / 8, so it fetches the logical chunk that the swizzle puts there
    const bf16_t* a_base = SWIGLU ? (const bf16_t*)a.x : (const bf16_t*)a.h;
    uint32_t a_off[8], b_off[8];
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
        const int r = (pw * A_DMA + j) * 8 + (lane >> 3);
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
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) {
        const int br = (pw * B_DMA + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(br);
        int32_t n = n0 + (SWIGLU ? br % (NB / 2) : br);
        n = n < N ? n : N - 1;  // columns past N are computed, never stored
        b_off[j] = ((uint32_t)n * (uint32_t)KD + c * 8) * 2u;
    }
    // the offsets live in LDS between stages (each lane reads back only what it wrote)
    u32x4* offs = (u32x4*)(smem + ring_bytes(BM)) + pw * 4 * 64 + lane;
    if (wave < PRODUCERS) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            offs[q * 64] = u32x4{a_off[4 * q], a_off[4 * q + 1], a_off[4 * q + 2], a_off[4 * q + 3]};
            offs[(2 + q) * 64] = u32x4{b_off[4 * q], b_off[4 * q + 1], b_off[4 * q + 2], b_off[4 * q + 3]};
        }
    }
    // a wave's B instruction j covers 8 rows, all gate or all up (NB/2 is a multiple of 8)
    // DMA sources are a uniform base (advanced by the stage) plus a per-lane 32-bit byte offset,
    // so no per-lane 64-bit address arithmetic is issued per instruction
    auto issue = [&](int kt) {
        if (wave >= PRODUCERS) return;  // wave-uniform
        char* st = smem + (kt % NST) * ST_BYTES;
        const int32_t k0 = kt * BKD;
        const char* ab = (const char*)(a_base + k0);
        uint32_t a_off[8], b_off[8];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const u32x4 va = offs[q * 64], vb = offs[(2 + q) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a_off[4 * q + e] = va[e];
                b_off[4 * q + e] = vb[e];
            }
        }
#pragma unroll
        for (int j = 0; j < A_DMA; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(ab + a_off[j]),
                                             DSMOE_LDS_PTR(st + (pw * A_DMA + j) * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j) {
            const int br0 = (pw * B_DMA + j) * 8;
            const char* wb = (const char*)(((SWIGLU && br0 >= NB / 2) ? wb1 : wb0) + k0);
            __builtin_amdgcn_global_load_lds((const void*)(wb + b_off[j]),
                                             DSMOE_LDS_PTR(st + A_BYTES + (pw * B_DMA + j) * 1024), 16, 0, 0);
        }
    };

    f32x16 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i][0] = acc[i][1] = f32x16{};
    // B rows of the wave's two 32-row blocks: GEMM-1 gate rows (j = 0) and up rows (j = 1) of
    // output columns [32 wn, 32 wn + 32); GEMM-2 rows [64 wn, 64 wn + 64)
    int brow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) brow[j] = SWIGLU ? j * (NB / 2) + wn * 32 : wn * 64 + j * 32;

    // Software pipeline over k16 steps (four per stage): the fragments of the next step are read
    // from LDS while the current step's MFMAs run.  The wait + barrier that publishes stage kt+1
    // sits before the last step of stage kt; once every wave has passed it, the fragments of
    // stage kt are all in registers, so its slot is refilled with stage kt+NST right away and
    // those loads have the next four steps to land.
    // A wave multiplies only its NV row blocks of 32 that hold rows of the group (the last tile of
    // a group is ragged); NV = 0 leaves the wave to the barriers, so the other wave on its SIMD
    // has the matrix core to itself.  Every variant passes the same barriers.
    const int nk = KD / BKD;  // >= 1
    bf16x8 fa[2][MT], fb[2][2];
    auto kloop = [&](auto nv_c) {
        constexpr int NV = decltype(nv_c)::value;
        auto read_frags = [&](int kt, int s, int buf) {
            if constexpr (NV > 0) {
                const char* st = smem + (kt % NST) * ST_BYTES;
                const int c = 2 * s + (lane >> 5);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    fb[buf][j] = as_bf16x8(*(const u32x4*)(st + A_BYTES + off(brow[j] + (lane & 31), c)));
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    fa[buf][i] = as_bf16x8(*(const u32x4*)(st + off(wm * WM + i * 32 + (lane & 31), c)));
            }
        };
        // one k16 step: its MFMAs with (optionally) the next step's fragment reads pinned one after
        // each MFMA, so every LDS read issues under a running MFMA (measured about 1 % faster than
        // issuing all reads after the first MFMA)
        auto mfma_step = [&](int buf, bool then_read, int rkt, int rs, int rbuf) {
            if constexpr (NV > 0) {
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][0], fa[buf][0], acc[0][0], 0, 0, 0);
                if (then_read) read_frags(rkt, rs, rbuf);
#pragma unroll
                for (int i = 0; i < NV; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        if (i | j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
                // one MFMA, then one LDS read of the next step, alternating until the reads run out
#pragma unroll
                for (int q = 0; q < 2 * NV; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (then_read && q < NV + 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
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
    };
    {
        const int32_t rows = min(cnt - m0, (int32_t)BM) - wm * WM;  // rows of the group in this wave's half
        const int nv = rows <= 0 ? 0 : min((rows + 31) >> 5, MT);
        static_assert(MT == 2 || MT == 4, "row blocks per wave");
        if (nv >= MT) kloop(std::integral_constant<int, MT>{});
        else if (nv == 0) kloop(std::integral_constant<int, 0>{});
        else if (nv == 1) kloop(std::integral_constant<int, 1>{});
        else if constexpr (MT == 4) {
            if (nv == 2) kloop(std::integral_constant<int, 2>{});
            else kloop(std::integral_constant<int, 3>{});
        }
    }

    tile_epilogue<BM, SWIGLU>(a, acc, smem, r0, cnt, m0, n0, N, wm, wn, tid);
}


// ---------------------------------------------------------------------------------------------
// Quantised weights: 4-bit (affine, groups of 64 along the reduction axis) or fp8 (OCP E4M3
// codes, one fp32 scale per 128 x 128 block), tiles of 160 (4-bit) or 128 (fp8) rows x 256
// weight rows, same tile list as gemm_dma.  A tile computes only its real rows rounded up to
// 32 (a variant per height), while its weights are staged and dequantised once whatever its
// height.  Every operand of a 64-k stage -- the activation rows, the weight codes and the
// scales (and 4-bit offsets) -- enters LDS by DMA, in a ring of two stages (stage kt+1 in flight
// while kt is computed).  With no register loads in the loop the compiler inserts no waits of
// its own: the only waits are the explicit count + barrier per stage.  (Loading the
// codes into registers beside an LDS DMA ring made the compiler wait for every outstanding load
// before each use of them, which exposed the full memory latency once per stage.)
// The dequantisation -- bf16(s*q + b), resp. bf16(value * scale) -- runs on the vector ALU
// beside the matrix cores, one k16 step ahead of the MFMAs that consume it; to keep it at one
// pass per weight the four waves split the tile by columns (1 x 4): wave w owns all rows
// and, for GEMM-1, the gate and up rows of output columns [32 w, 32 w + 32), for GEMM-2 the 64
// columns [64 w, 64 w + 64).  Wave w also fetches those 64 weight rows' codes and scales.
// Within a stage the k chunks are taken in the order 4h + s (lane half h, step s) for both
// operands, so a lane's codes for the whole stage are one (4-bit) or two (fp8) 16-byte chunks.
//
// LDS layout of one stage slot:
//   activations  BM rows x 128 bytes, chunk swizzle dma::swz (as gemm_dma)
//   codes        256 weight rows x CB bytes (CB = 32 for 4-bit, 64 for fp8); weight row
//                rho = 64 w + 32 j + i is column i of wave w's block j; 16-byte chunk c of
//                row rho sits at chunk c ^ cswz(rho), which keeps each phase of the lanes' reads
//                (consecutive rows, one chunk each) spread over all banks
//   side data    fp8: one fp32 scale per weight row (4 * 256 bytes); 4-bit: the aligned 32-bit
//                word holding the row's bf16 scale for the stage, then the one holding its
//                offset (2 * 4 * 256 bytes); the bf16 half is picked by the element's parity
// ---------------------------------------------------------------------------------------------
enum { WQ_Q4 = 0, WQ_F8 = 1 };

namespace wq {
// rows of the tile list's tiles: 160 for 4-bit, 128 for fp8, so two workgroups (at most 80 KB of
// LDS and two waves per SIMD each) share a CU and one's dequantisation runs under the other's
// MFMAs.  A tile dequantises all of its 256 weight rows whatever its height, so the tallest tile
// whose accumulators still fit two waves per SIMD (160 rows: 160 of a wave's 256 registers)
// takes a group of 129..160 rows in one tile instead of two: 4.49 -> 4.39 ms on the DeepSeek-V3
// 4-bit prefill layer (T = 4096, groups of about 150 rows).  (256-row 4-bit tiles -- one
// workgroup per CU -- measured about 2 % slower than 128-row ones.)
constexpr int bm(int wqt) { return wqt == WQ_Q4 ? 160 : 128; }
template <int WQ>
struct Fmt {
    static constexpr int BM = bm(WQ);
    static constexpr int A_BYTES = BM * dma::ROWB;              // activation slot of one stage
    // ring depth: two stages (4-bit: 52 KB, or 48 KB plus 16 KB of chunked side data; fp8: 66 KB)
    static constexpr int NS = 2;
    static constexpr int CB = WQ == WQ_F8 ? 64 : 32;            // code bytes per weight row per stage
    static constexpr int ROWS_PER_DMA = 1024 / CB;              // weight rows per DMA instruction
    static constexpr int C_DMA = 64 / ROWS_PER_DMA;             // code DMAs per wave per stage
    static constexpr int S_DMA = WQ == WQ_F8 ? 1 : 2;           // side-data DMAs per wave per stage
    static constexpr int C_BYTES = 256 * CB;
    static constexpr int S_BYTES = 1024 * S_DMA;
    static constexpr int STAGE = A_BYTES + C_BYTES + S_BYTES;
};
constexpr int ring_bytes(int wqt) {
    return wqt == WQ_F8 ? Fmt<WQ_F8>::NS * Fmt<WQ_F8>::STAGE : Fmt<WQ_Q4>::NS * Fmt<WQ_Q4>::STAGE;
}
// 4-bit tiles with the scales and offsets in chunks of 8 stages: a ring without side data plus two
// chunk slots of [2 kinds][256 rows][16 bytes]
constexpr int SIDE8_BYTES = 2 * 2 * 256 * 16;
constexpr int ring_bytes_side8() {
    return Fmt<WQ_Q4>::NS * (Fmt<WQ_Q4>::A_BYTES + Fmt<WQ_Q4>::C_BYTES) + SIDE8_BYTES;
}
// dynamic LDS of a launch: the stage ring, or the epilogue's bf16 image of the output tile
// (bm x 128 for GEMM-1, bm x 256 for GEMM-2) when that is larger
constexpr int lds_bytes(int wqt, bool swiglu, bool side8 = false) {
    const int img = bm(wqt) * (swiglu ? 128 : 256) * 2;
    const int ring = side8 ? ring_bytes_side8() : ring_bytes(wqt);
    return ring > img ? ring : img;
}
template <int WQ>
__device__ __forceinline__ int cswz(int rho) { return WQ == WQ_F8 ? (rho >> 1) & 3 : (rho >> 2) & 1; }
}  // namespace wq

// one stage of one lane's codes for its two 32-column blocks, with their scales (and offsets)
template <int WQ>
struct BStage;
template <>
struct BStage<WQ_Q4> {
    u32x4 q[2];
    float s[2], b[2];  // s: 512 times the scale
    __device__ __forceinline__ u32x4 deq(int j, int st) const { return dequant8(q[j][st], s[j], b[j]); }
};
template <>
struct BStage<WQ_F8> {
    u32x4 q[2][2];  // block j: 32 codes; step st is words 2(st%2), 2(st%2)+1 of q[j][st/2]
    float s[2];
    __device__ __forceinline__ u32x4 deq(int j, int st) const {
        return dequant_f8x8(q[j][st >> 1][2 * (st & 1)], q[j][st >> 1][2 * (st & 1) + 1], s[j]);
    }
};

// The computed rows of one tile: MT blocks of 32 (the tile's rows rounded up to a multiple of 32).
// Only those rows are staged and multiplied; the weights' codes and scales are staged and
// dequantised once per tile whatever its height, so a group of up to 256 rows pays for its
// dequantisation once.
template <int WQ, bool SWIGLU, bool SIDE8, int MT>
__device__ __forceinline__ void wq_tile(const TileArgs& ta, char* smem, int32_t g, int32_t m0, int32_t r0,
                                        int32_t cnt, int32_t n0) {
    using namespace dma;
    using F = wq::Fmt<WQ>;
    static_assert(!SIDE8 || WQ == WQ_Q4, "chunked side data is a 4-bit layout");
    constexpr int NS = F::NS;
    constexpr int A_DMA = MT;                  // activation DMAs per wave per stage: 32 MT rows of 128 bytes
    // SIDE8: the scales and offsets arrive once per 8 stages (below), not with every stage
    constexpr int STAGE = SIDE8 ? F::A_BYTES + F::C_BYTES : F::STAGE;
    constexpr int D = A_DMA + F::C_DMA + (SIDE8 ? 0 : F::S_DMA);
    static_assert(NS >= 2 && NS * STAGE + (SIDE8 ? wq::SIDE8_BYTES : 0) <= LDS_MAX, "ring depth / size");
    static_assert(MT >= 1 && MT * 32 <= F::BM, "row blocks");
    constexpr int A_BYTES = F::A_BYTES;
    const GroupedArgs& a = ta.a;
    const int32_t N = SWIGLU ? a.I : a.H;
    const int32_t KD = SWIGLU ? a.H : a.I;

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, half = lane >> 5;

    // activation DMA sources, as gemm_dma
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

    // weight row (output column) of block j of this wave at in-block index i: GEMM-1 gate (j = 0)
    // and up (j = 1) rows of column 32 w + i; GEMM-2 rows 64 w + 32 j + i.  Columns past N are
    // computed from row N - 1 and never stored.
    auto wcol = [&](int j, int i) -> int32_t { return n0 + (SWIGLU ? wave * 32 : wave * 64 + j * 32) + i; };
    auto wrow = [&](int j, int i) -> int32_t { const int32_t n = wcol(j, i); return n < N ? n : N - 1; };
    const void* wb[2] = {SWIGLU ? a.wg : a.wd, SWIGLU ? a.wu : a.wd};
    // code DMA t of this wave: lane -> weight row rho = 64 w + t * ROWS_PER_DMA + lane / (CB/16),
    // LDS chunk p = lane % (CB/16), holding logical chunk p ^ cswz(rho); per lane a 32-bit byte
    // offset of (row, chunk) within the expert's code matrix
    constexpr int CPR = F::CB / 16;  // chunks per weight row per stage
    uint32_t c_off[F::C_DMA];
    const char* c_base[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) c_base[j] = (const char*)wb[j] + (int64_t)g * N * (WQ == WQ_F8 ? KD : KD / 2);
#pragma unroll
    for (int t = 0; t < F::C_DMA; ++t) {
        const int rho = wave * 64 + t * F::ROWS_PER_DMA + lane / CPR;
        const int jj = (rho >> 5) & 1, i = rho & 31;
        const int cl = (lane % CPR) ^ wq::cswz<WQ>(rho);
        const uint32_t row_bytes = WQ == WQ_F8 ? (uint32_t)KD : (uint32_t)KD / 2;
        c_off[t] = (uint32_t)wrow(jj, i) * row_bytes + cl * 16;
    }
    // side-data sources: lane -> weight row rho = 64 w + lane (block lane / 32, column lane % 32)
    const int sj = lane >> 5, si = lane & 31;
    const int32_t srow = wrow(sj, si);
    const float* fs_ptr = nullptr;          // fp8: scale of (srow's block row, stage's k block)
    const uint32_t* qs_ptr = nullptr;       // 4-bit: words holding the scale / offset
    const uint32_t* qb_ptr = nullptr;
    int32_t nq = 0;                         // 4-bit: element index of (srow, group 0)
    if constexpr (WQ == WQ_F8) {
        const int64_t nbo = (N + 127) / 128, nbi = (KD + 127) / 128;
        const float* base = (SWIGLU ? (sj ? a.fsu : a.fsg) : a.fsd) + (int64_t)g * nbo * nbi;
        fs_ptr = base + (int64_t)(srow / 128) * nbi;
    } else {
        // the element counts N * KD / 64 per expert are even (N is a multiple of 64), so the
        // aligned word holding any element lies inside the array
        const int64_t es = (int64_t)g * N * (KD / 64);
        qs_ptr = (const uint32_t*)((SWIGLU ? (sj ? a.su : a.sg) : a.sd) + es);
        qb_ptr = (const uint32_t*)((SWIGLU ? (sj ? a.bu : a.bg) : a.bd) + es);
        nq = srow * (KD / 64);
    }

    // Each DMA source is a uniform base (advanced by the stage) plus the lane's 32-bit offset.  The
    // offsets pass through an empty asm (which the compiler must assume changes them) first:
    // otherwise it hoists base + offset out of the loop as per-lane 64-bit pointers and adds the
    // stage's advance to each with a 64-bit vector add on every stage.
    auto issue = [&](int kt) {
        char* st = smem + (kt % NS) * STAGE;
        const char* ab = (const char*)(a_base + kt * BKD);
#pragma unroll
        for (int j = 0; j < A_DMA; ++j) {
            asm volatile("" : "+v"(a_off[j]));
            __builtin_amdgcn_global_load_lds((const void*)(ab + a_off[j]), DSMOE_LDS_PTR(st + (wave * A_DMA + j) * 1024),
                                             16, 0, 0);
        }
        char* cst = st + A_BYTES + wave * 64 * F::CB;
#pragma unroll
        for (int t = 0; t < F::C_DMA; ++t) {
            const int jj = ((t * F::ROWS_PER_DMA) >> 5) & 1;  // block of this instruction's rows
            asm volatile("" : "+v"(c_off[t]));
            __builtin_amdgcn_global_load_lds((const void*)(c_base[jj] + kt * F::CB + c_off[t]),
                                             DSMOE_LDS_PTR(cst + t * 1024), 16, 0, 0);
        }
        char* sst = st + A_BYTES + F::C_BYTES + wave * 256;
        if constexpr (WQ == WQ_F8) {
            __builtin_amdgcn_global_load_lds((const void*)(fs_ptr + (kt >> 1)), DSMOE_LDS_PTR(sst), 4, 0, 0);
        } else if constexpr (!SIDE8) {
            const int32_t e = (nq + kt) >> 1;
            __builtin_amdgcn_global_load_lds((const void*)(qs_ptr + e), DSMOE_LDS_PTR(sst), 4, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(qb_ptr + e), DSMOE_LDS_PTR(sst + 1024), 4, 0, 0);
        }
    };
    // SIDE8: chunk c holds, for every weight row of the tile, the bf16 scales and offsets of
    // groups [8c, 8c + 8) (stages 8c .. 8c + 7): 16 bytes per row and kind, so lane l of wave w
    // fetches the 16 bytes of row 64 w + l with one instruction per kind.  Two chunk slots follow
    // the stage ring: [slot][scale, offset][256 rows][8 groups].  (Needs KD / 64 to be a multiple
    // of 8, so the 16-byte pieces are aligned and no chunk runs past a row.)
    char* side8 = smem + NS * STAGE;
    auto issue_side = [&](int c) {
        if constexpr (SIDE8) {
            char* d = side8 + (c & 1) * (wq::SIDE8_BYTES / 2) + wave * 1024;
            const bf16_t* sb = (const bf16_t*)qs_ptr + nq + 8 * c;  // element (srow, group 8c)
            const bf16_t* bb = (const bf16_t*)qb_ptr + nq + 8 * c;
            __builtin_amdgcn_global_load_lds((const void*)sb, DSMOE_LDS_PTR(d), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)bb, DSMOE_LDS_PTR(d + wq::SIDE8_BYTES / 4), 16, 0, 0);
        }
    };

    // this lane's codes and scales of stage kt, from LDS
    using BS = BStage<WQ>;
    auto read_b = [&](int kt, BS& bs) {
        const char* st = smem + (kt % NS) * STAGE;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int rho = wave * 64 + j * 32 + (lane & 31);
            const char* row = st + A_BYTES + rho * F::CB;
            const int sw = wq::cswz<WQ>(rho);
            const char* side = st + A_BYTES + F::C_BYTES + rho * 4;
            if constexpr (WQ == WQ_F8) {
                bs.q[j][0] = *(const u32x4*)(row + (((2 * half) ^ sw) << 4));
                bs.q[j][1] = *(const u32x4*)(row + (((2 * half + 1) ^ sw) << 4));
                bs.s[j] = *(const float*)side;
            } else if constexpr (SIDE8) {
                bs.q[j] = *(const u32x4*)(row + ((half ^ sw) << 4));
                const char* sd = side8 + ((kt >> 3) & 1) * (wq::SIDE8_BYTES / 2) + rho * 16 + (kt & 7) * 2;
                bs.s[j] = 512.0f * bf16_to_f32(*(const bf16_t*)sd);  // dequant8 takes 512 s
                bs.b[j] = bf16_to_f32(*(const bf16_t*)(sd + wq::SIDE8_BYTES / 4));
            } else {
                bs.q[j] = *(const u32x4*)(row + ((half ^ sw) << 4));
                // the row's element for this stage is (its group index + kt); odd ones are the
                // word's upper half
                const int32_t nqj = wrow(j, lane & 31) * (KD / 64) + kt;
                const uint32_t sw32 = *(const uint32_t*)side, bw32 = *(const uint32_t*)(side + 1024);
                const int sh = (nqj & 1) * 16;
                bs.s[j] = 512.0f * bf16_to_f32((bf16_t)(sw32 >> sh));  // dequant8 takes 512 s
                bs.b[j] = bf16_to_f32((bf16_t)(bw32 >> sh));
            }
        }
    };

    f32x16 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i][0] = acc[i][1] = f32x16{};

    const int nk = KD / BKD;  // >= 1
    bf16x8 fa[2][MT], fb[2][2];
    // operands of step s of stage kt: activations from LDS, weights dequantised from registers
    auto frags = [&](int kt, int s, int buf, const BS& bs) {
        const char* st = smem + (kt % NS) * STAGE;
        const int c = 4 * half + s;
#pragma unroll
        for (int i = 0; i < MT; ++i) fa[buf][i] = as_bf16x8(*(const u32x4*)(st + off(i * 32 + (lane & 31), c)));
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[buf][j] = as_bf16x8(bs.deq(j, s));
    };
    // the MFMAs of step `buf`, with the next step's operand work (issued just before, in program
    // order) spread between them: after each MFMA one of its LDS reads (while they last) and a
    // few dequantisation instructions, so the LDS and the vector ALU run while the matrix core does
    // the next step's dequantisation (about 40 vector instructions for fp8, 48 for 4-bit) spread
    // evenly over this step's 2 MT MFMAs
    constexpr int VPM = ((WQ == WQ_F8 ? 40 : 48) + 2 * MT - 1) / (2 * MT);
    auto mfma_step = [&](int buf) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 2 * MT; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (q < MT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // an LDS read of the next step's A
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // then vector ALU work
        }
    };
    // One stage.  At the barrier everything but the newest (NS-2) D operations (stage kt+NS-1,
    // issued during stage kt-1) has landed: stage kt+1 is complete in LDS, and every wave is done
    // with stage kt's slot, which then receives stage kt+NS.  Past the last stage the DMA repeats
    // stage nk-1 into its own slot (the same bytes; never consumed), so every path issues the
    // same sequence and the counts stay exact.  (Reading the next stage's codes into a second
    // register set ahead of the barrier, from the wave's own DMAs, measured slower: the compiler
    // then waited on each of those reads in turn.)
    BS bs;
    auto stage = [&](int kt) {
        frags(kt, 1, 1, bs);
        mfma_step(0);
        frags(kt, 2, 0, bs);
        mfma_step(1);
        frags(kt, 3, 1, bs);
        mfma_step(0);
        wait_vm_barrier<(NS - 2) * D>();
        issue(kt + NS < nk ? kt + NS : nk - 1);
        // SIDE8: chunk c + 1 goes into the slot of chunk c - 1 (this wave read it last at stage
        // 8c - 2), 7 stages before it is read; issued after the stage's D operations, so the
        // waits above stay exact for the stages (they only wait a little earlier for two of them)
        if (SIDE8 && (kt & 7) == 0 && kt + 8 < nk) issue_side((kt >> 3) + 1);
        const int kn = kt + 1 < nk ? kt + 1 : nk - 1;
        read_b(kn, bs);
        frags(kn, 0, 0, bs);
        mfma_step(1);
    };

    issue_side(0);  // oldest of the prologue's operations, so the wait below covers it
#pragma unroll
    for (int j = 0; j < NS; ++j) issue(j < nk ? j : nk - 1);
    wait_vm_barrier<(NS - 1) * D>();
    read_b(0, bs);
    frags(0, 0, 0, bs);
    for (int kt = 0; kt < nk; ++kt) stage(kt);

    // the accumulators of the last MFMAs are read right away: give the MFMA-to-VALU wait states
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0][0]));
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (i | j) asm volatile("" : "+a"(acc[i][j]));

    // Epilogue through an LDS image of the output tile, as in gemm_dma: each lane writes its bf16
    // results -- GEMM-1: bf16(silu(gate) * up), 32 output columns per wave; GEMM-2: 64 -- into a
    // row-major image, four consecutive columns of one row per 8-byte write (the weights are the
    // MFMA's first operand), chunk c of row r at c ^ (r mod OCPR); then every thread copies
    // 16-byte row pieces out.  The ring is reused for the image once every wave's DMAs have
    // landed (the loop's tail repeats the last stage's DMA) and every wave is past its last LDS
    // read.
    constexpr int OUT_COLS = SWIGLU ? NB / 2 : NB;
    constexpr int RB = OUT_COLS * 2;   // bytes per image row
    constexpr int OCPR = OUT_COLS / 8;  // 16-byte chunks per image row
    constexpr int NT = 256;             // threads of the workgroup
    static_assert(MT * 32 * RB <= wq::lds_bytes(WQ, SWIGLU, SIDE8), "output image exceeds the LDS allocation");
    static_assert((OCPR & (OCPR - 1)) == 0, "chunks per row: a power of two");
    auto chunk_at = [](int r, int c) { return r * RB + ((c ^ (r & (OCPR - 1))) << 4); };
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int row = i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < (SWIGLU ? 1 : 2); ++j) {
            const int c0 = SWIGLU ? wave * 4 : wave * 8 + j * 4;  // first 16-byte chunk of the 32 columns
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = SWIGLU ? silu_f(acc[i][0][4 * q + e]) * acc[i][1][4 * q + e] : acc[i][j][4 * q + e];
                *(u32x2*)(smem + chunk_at(row, c0 + q) + half * 8) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    bf16_t* dst = SWIGLU ? (bf16_t*)a.h : (bf16_t*)a.o;
    const int64_t ld = SWIGLU ? a.ldh : a.H;
    const int32_t rows = min(cnt - m0, MT * 32);
#pragma unroll
    for (int k = 0; k < (MT * 32 * OCPR + NT - 1) / NT; ++k) {
        const int q = tid + k * NT;
        const int row = q / OCPR, c = q % OCPR;
        const int32_t col = n0 + c * 8;
        if (row >= rows || col >= N) continue;
        const u32x4 v = *(const u32x4*)(smem + chunk_at(row, c));
        *(u32x4*)(dst + (int64_t)(r0 + m0 + row) * ld + col) = v;
    }
}

template <int WQ, bool SWIGLU, bool SIDE8>
__global__ __launch_bounds__(THREADS) void gemm_dma_wq(TileArgs ta) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const GroupedArgs& a = ta.a;
    int32_t tile, ct;
    if (!map_tile<WQ == WQ_Q4 ? (SWIGLU ? 16 : 32) : 8>(ta, tile, ct)) return;
    const i32x4 ti = *(const i32x4*)(ta.tile_info + 4 * tile);  // group, first row, group rows
    const int32_t g = ti[0], m0 = ti[1], r0 = ti[2], cnt = ti[3];
    if (g < ta.g0 || g >= ta.g1 || g >= a.E) return;  // routed groups only (the shared expert is bf16)
    const int32_t N = SWIGLU ? a.I : a.H;
    constexpr int OUT_COLS = SWIGLU ? NB / 2 : NB;
    const int32_t n0 = ct * OUT_COLS;
    if (n0 >= N) return;
    // rows of this tile, rounded up to 32: selects the variant (uniform over the workgroup)
    constexpr int BM = wq::bm(WQ);
    const int32_t rows = min(cnt - m0, (int32_t)BM);
    const int32_t q32 = __builtin_amdgcn_readfirstlane((rows + 31) >> 5);
    static_assert(BM == 128 || BM == 160, "tile height");
    if constexpr (BM >= 160) {
        if (q32 >= 5) {
            wq_tile<WQ, SWIGLU, SIDE8, 5>(ta, smem, g, m0, r0, cnt, n0);
            return;
        }
    }
    if (q32 >= 4) wq_tile<WQ, SWIGLU, SIDE8, 4>(ta, smem, g, m0, r0, cnt, n0);
    else if (q32 == 3) wq_tile<WQ, SWIGLU, SIDE8, 3>(ta, smem, g, m0, r0, cnt, n0);
    else if (q32 == 2) wq_tile<WQ, SWIGLU, SIDE8, 2>(ta, smem, g, m0, r0, cnt, n0);
    else wq_tile<WQ, SWIGLU, SIDE8, 1>(ta, smem, g, m0, r0, cnt, n0);
}

// Tile list (offsets is read only for routed groups: it may be NULL when E == 0): every group in
// [0, E] (E = shared expert) with more than `min_rows` rows gets
// ceil(rows / BM) tiles (ceil(T / BMs) for the shared expert, whose tiles a launch of their own
// may compute with a different tile height), in group order; tile_count[0] is the number of
// tiles, tile_count[1] the number of routed ones (those before the shared expert's).  One
// workgroup; group 1024 (only possible with E == 1024 plus a shared expert) is appended by
// thread 0.
__global__ __launch_bounds__(1024) void tiles_kernel(const int32_t* __restrict__ offsets, int32_t E, int64_t T,
                                                     int32_t TK, int32_t has_shared, int32_t BM, int32_t BMs,
                                                     int32_t min_rows,
                                                     int32_t* __restrict__ tile_count,
                                                     int32_t* __restrict__ tile_info) {
    __shared__ int32_t buf[1024];
    const int t = threadIdx.x;
    const int32_t ng = E + has_shared;
    auto bm_of = [&](int32_t g) -> int32_t { return g < E ? BM : BMs; };
    auto ntiles = [&](int32_t g) -> int32_t {
        const int32_t cnt = g < E ? offsets[g + 1] - offsets[g] : (int32_t)T;
        return cnt > min_rows ? (cnt + bm_of(g) - 1) / bm_of(g) : 0;
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
    auto put = [&](int32_t i, int32_t g, int32_t m) {
        const int32_t r0 = g < E ? offsets[g] : TK;  // the shared rows follow the routed ones
        const int32_t cnt = g < E ? offsets[g + 1] - offsets[g] : (int32_t)T;
        *(i32x4*)(tile_info + 4 * i) = i32x4{g, m * bm_of(g), r0, cnt};
    };
    for (int32_t m = 0; m < n; ++m) put(start + m, t, m);
    if (t == E) tile_count[1] = start;  // the tiles of groups 0 .. E-1 come first
    if (t == 0) {
        int32_t total = buf[1023];
        if (E >= 1024) tile_count[1] = total;
        if (ng > 1024) {
            const int32_t nn = ntiles(1024);
            for (int32_t m = 0; m < nn; ++m) put(total + m, 1024, m);
            total += nn;
        }
        tile_count[0] = total;
    }
}

template <int BM, bool SW>
hipError_t launch_dma_t(const TileArgs& ta, hipStream_t s) {
    const size_t lds = (size_t)dma::lds_bytes(BM);
    const unsigned grid = (unsigned)(((ta.nwg + 7) / 8) * 8);
    hipLaunchKernelGGL((gemm_dma<BM, SW>), dim3(grid), dim3(dma::THREADS), lds, s, ta);
    return hipGetLastError();
}

template <int WQ, bool SW, bool SIDE8 = false>
hipError_t launch_dma_wq_t(const TileArgs& ta, hipStream_t s) {
    const size_t lds = (size_t)wq::lds_bytes(WQ, SW, SIDE8);
    const unsigned grid = (unsigned)(((ta.nwg + 7) / 8) * 8);
    hipLaunchKernelGGL((gemm_dma_wq<WQ, SW, SIDE8>), dim3(grid), dim3(THREADS), lds, s, ta);
    return hipGetLastError();
}


}  // namespace

int32_t tiled_max_tiles(int64_t T, int32_t K, int32_t E, int32_t BM) {
    const int64_t rows = T * K + T;
    return (int32_t)((rows + BM - 1) / BM + E + 1);
}

// largest dynamic LDS any tiled kernel of this tile height uses
int32_t tiled_lds_bytes(int32_t BM) {
    int32_t r = dma::lds_bytes(BM);
    if (BM == wq::bm(WQ_F8)) r = max(r, max(wq::lds_bytes(WQ_F8, true), wq::lds_bytes(WQ_F8, false)));
    if (BM == wq::bm(WQ_Q4))
        r = max(r, max(max(wq::lds_bytes(WQ_Q4, true), wq::lds_bytes(WQ_Q4, false)),
                       max(wq::lds_bytes(WQ_Q4, true, true), wq::lds_bytes(WQ_Q4, false, true))));
    return r;
}

int32_t tiled_quant_bm(int32_t wdt) { return wq::bm(wdt == MOE_FP8 ? WQ_F8 : WQ_Q4); }

hipError_t configure_tiled_kernels() {
    // allow the large dynamic LDS allocations (up to 128 KB) of the tiled kernels
    const void* ks[] = {
        (const void*)gemm_dma<256, true>,           (const void*)gemm_dma<256, false>,
        (const void*)gemm_dma<128, true>,           (const void*)gemm_dma<128, false>,
        (const void*)gemm_dma_wq<WQ_Q4, true, false>,  (const void*)gemm_dma_wq<WQ_Q4, false, false>,
        (const void*)gemm_dma_wq<WQ_Q4, true, true>,   (const void*)gemm_dma_wq<WQ_Q4, false, true>,
        (const void*)gemm_dma_wq<WQ_F8, true, false>,  (const void*)gemm_dma_wq<WQ_F8, false, false>,
    };
    const int bms[] = {256, 256, 128, 128, wq::bm(WQ_Q4), wq::bm(WQ_Q4), wq::bm(WQ_Q4), wq::bm(WQ_Q4),
                       wq::bm(WQ_F8), wq::bm(WQ_F8)};
    for (int i = 0; i < 10; ++i) {
        hipError_t e = hipFuncSetAttribute(ks[i], hipFuncAttributeMaxDynamicSharedMemorySize, tiled_lds_bytes(bms[i]));
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_tiles(const GroupedArgs& a, int32_t BM, int32_t BMs, int32_t min_rows, int32_t* tile_count,
                        int32_t* tile_info, hipStream_t s) {
    hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.E, a.T, a.TK, a.Is > 0 ? 1 : 0, BM,
                       BMs, min_rows, tile_count, tile_info);
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
    ta.part = g0 >= a.E ? 2 : g1 <= a.E ? 1 : 0;
    const int32_t N = gemm1 ? (a.I > a.Is ? a.I : a.Is) : a.H;
    const int32_t out_cols = gemm1 ? NB / 2 : NB;
    ta.col_tiles = (N + out_cols - 1) / out_cols;
    ta.nwg = max_tiles * ta.col_tiles;
    if (wdt == MOE_BF16) {
        if (BM == 256) return gemm1 ? launch_dma_t<256, true>(ta, s) : launch_dma_t<256, false>(ta, s);
        return gemm1 ? launch_dma_t<128, true>(ta, s) : launch_dma_t<128, false>(ta, s);
    }
    // quantised layers use the tile height of their format (plan_tiles)
    if (BM != tiled_quant_bm(wdt)) return hipErrorInvalidValue;
    if (wdt == MOE_FP8) return gemm1 ? launch_dma_wq_t<WQ_F8, true>(ta, s) : launch_dma_wq_t<WQ_F8, false>(ta, s);
    if (wdt == MOE_Q4G64) {
        // scales and offsets in chunks of 8 groups when the reduction length allows it
        const int32_t KD = gemm1 ? a.H : a.I;
        if (KD % 512 == 0)
            return gemm1 ? launch_dma_wq_t<WQ_Q4, true, true>(ta, s) : launch_dma_wq_t<WQ_Q4, false, true>(ta, s);
        return gemm1 ? launch_dma_wq_t<WQ_Q4, true>(ta, s) : launch_dma_wq_t<WQ_Q4, false>(ta, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dsmoe
