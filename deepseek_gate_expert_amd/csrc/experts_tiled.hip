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

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// byte offset of 16-byte chunk c of row r in a [rows][64] bf16 LDS tile
__device__ __forceinline__ uint32_t lds_off(int r, int c) { return (uint32_t)(r * 128 + ((c ^ (r & 7)) << 4)); }

__device__ __forceinline__ uint4 dequant8(uint32_t w, float s, float b) {
    uint4 r;
    uint32_t* rp = (uint32_t*)&r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = __builtin_fmaf(s, (float)((w >> (8 * j)) & 0xFu), b);
        const float hi = __builtin_fmaf(s, (float)((w >> (8 * j + 4)) & 0xFu), b);
        rp[j] = pack_bf16x2(lo, hi);
    }
    return r;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

struct TileArgs {
    GroupedArgs a;
    const int32_t* tile_count;  // [1]
    const int32_t* tile_info;   // [max_tiles][2]: group, first row within the group
    int32_t g0, g1;             // groups handled by this launch
    int32_t col_tiles;          // output column tiles per row tile
    int32_t nwg;                // workgroups launched
};

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
    // XCD-aware remap: ids i, i+8, i+16, ... run on one XCD; give them consecutive tiles.
    const int32_t nwg8 = gridDim.x / 8;
    const int32_t bid = blockIdx.x;
    const int32_t logical = (bid & 7) * nwg8 + (bid >> 3);
    if (logical >= ta.nwg) return;
    const int32_t tile = logical / ta.col_tiles, ct = logical % ta.col_tiles;
    if (tile >= ta.tile_count[0]) return;
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

    // ---- per-thread global sources ------------------------------------------------------
    const bf16_t* a_src[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int id = tid + THREADS * i;
        int32_t rr = m0 + id / 8;
        rr = rr < cnt ? rr : cnt - 1;  // clamp: rows past the group are computed, never stored
        const int32_t row = r0 + rr;
        const int c = id % 8;
        if (SWIGLU) {
            const int32_t tok = row < a.TK ? a.sorted_slot[row] / a.K : row - a.TK;
            a_src[i] = (const bf16_t*)a.x + (int64_t)tok * a.H + c * 8;
        } else {
            a_src[i] = (const bf16_t*)a.h + (int64_t)row * a.ldh + c * 8;
        }
    }
    // weight row (output column) of B-tile row `br`; columns past N are clamped (never stored)
    auto w_row = [&](int br) -> int64_t {
        const int32_t n = n0 + (SWIGLU ? br % (NB / 2) : br);
        return n < N ? n : N - 1;
    };
    const bf16_t* b_src[B_LD];
    const uint32_t* q_src[B_LD];
    const bf16_t* s_src[B_LD];
    const bf16_t* z_src[B_LD];
    if constexpr (WF == WF_BF16) {
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int id = tid + THREADS * i;
            const int br = id / 8, c = id % 8;
            const int64_t n = w_row(br);
            const bf16_t* base;
            if (SWIGLU) {
                const bool up = br >= NB / 2;
                base = shared ? (const bf16_t*)(up ? a.swu : a.swg)
                              : (const bf16_t*)(up ? a.wu : a.wg) + (int64_t)g * a.I * a.H;
            } else {
                base = shared ? (const bf16_t*)a.swd : (const bf16_t*)a.wd + (int64_t)g * a.H * a.I;
            }
            b_src[i] = base + n * KD + c * 8;
            q_src[i] = nullptr;
            s_src[i] = z_src[i] = nullptr;
        }
    } else {
        // 4-bit: one 16-byte load covers 32 k of one row; a row of a 64-k step is two loads
#pragma unroll
        for (int i = 0; i < B_LD / 4; ++i) {
            const int id = tid + THREADS * i;  // NB * 2 = 512 half-rows per step
            const int br = id / 2, hf = id % 2;
            const int64_t n = w_row(br);
            int32_t out_dim;
            const uint32_t* qb;
            const bf16_t *sb, *zb;
            if (SWIGLU) {
                const bool up = br >= NB / 2;
                out_dim = a.I;
                qb = (const uint32_t*)(up ? a.wu : a.wg);
                sb = up ? a.su : a.sg;
                zb = up ? a.bu : a.bg;
            } else {
                out_dim = a.H;
                qb = (const uint32_t*)a.wd;
                sb = a.sd;
                zb = a.bd;
            }
            const int64_t row = (int64_t)g * out_dim + n;
            q_src[i] = qb + row * (KD / 8) + hf * 4;
            s_src[i] = sb + row * (KD / 64);
            z_src[i] = zb + row * (KD / 64);
            b_src[i] = nullptr;
        }
    }

    // ---- staging registers ------------------------------------------------------------
    uint4 ra[A_LD];
    uint4 rb[WF == WF_BF16 ? B_LD : B_LD / 4];
    float rs[WF == WF_BF16 ? 1 : B_LD / 4], rz[WF == WF_BF16 ? 1 : B_LD / 4];

    auto gload = [&](int32_t k) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) ra[i] = *(const uint4*)(a_src[i] + k);
        if constexpr (WF == WF_BF16) {
#pragma unroll
            for (int i = 0; i < B_LD; ++i) rb[i] = *(const uint4*)(b_src[i] + k);
        } else {
#pragma unroll
            for (int i = 0; i < B_LD / 4; ++i) {
                rb[i] = *(const uint4*)(q_src[i] + k / 8);
                rs[i] = bf16_to_f32(s_src[i][k / 64]);
                rz[i] = bf16_to_f32(z_src[i][k / 64]);
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int id = tid + THREADS * i;
            *(uint4*)(As(buf) + lds_off(id / 8, id % 8)) = ra[i];
        }
        if constexpr (WF == WF_BF16) {
#pragma unroll
            for (int i = 0; i < B_LD; ++i) {
                const int id = tid + THREADS * i;
                *(uint4*)(Bs(buf) + lds_off(id / 8, id % 8)) = rb[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_LD / 4; ++i) {
                const int id = tid + THREADS * i;
                const int br = id / 2, hf = id % 2;
                const uint32_t* w = (const uint32_t*)&rb[i];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(uint4*)(Bs(buf) + lds_off(br, hf * 4 + j)) = dequant8(w[j], rs[i], rz[i]);
            }
        }
    };

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
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const char* Ab = As(buf);
        const char* Bb = Bs(buf);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int c = 2 * s + (lane >> 5);
            bf16x8 af[MT], bfr[4];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int r = wm * WM + i * 32 + (lane & 31);
                af[i] = as_bf16x8(*(const uint4*)(Ab + lds_off(r, c)));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = brow[j] + (lane & 31);
                bfr[j] = as_bf16x8(*(const uint4*)(Bb + lds_off(r, c)));
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

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

int32_t tiled_lds_bytes(int32_t BM) { return 2 * (BM + NB) * 128; }

hipError_t configure_tiled_kernels() {
    // allow the large dynamic LDS allocations (up to 128 KB) of the tiled kernels
    const void* ks[] = {
        (const void*)gemm_tiled<256, true, WF_BF16>, (const void*)gemm_tiled<256, false, WF_BF16>,
        (const void*)gemm_tiled<256, true, WF_Q4>,   (const void*)gemm_tiled<256, false, WF_Q4>,
        (const void*)gemm_tiled<128, true, WF_BF16>, (const void*)gemm_tiled<128, false, WF_BF16>,
        (const void*)gemm_tiled<128, true, WF_Q4>,   (const void*)gemm_tiled<128, false, WF_Q4>,
    };
    const int bms[] = {256, 256, 256, 256, 128, 128, 128, 128};
    for (int i = 0; i < 8; ++i) {
        const int lds = 2 * (bms[i] + NB) * 128;
        hipError_t e = hipFuncSetAttribute(ks[i], hipFuncAttributeMaxDynamicSharedMemorySize, lds);
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
    if (BM == 256) {
        if (gemm1) return q4 ? launch_tiled_t<256, true, WF_Q4>(ta, s) : launch_tiled_t<256, true, WF_BF16>(ta, s);
        return q4 ? launch_tiled_t<256, false, WF_Q4>(ta, s) : launch_tiled_t<256, false, WF_BF16>(ta, s);
    }
    if (gemm1) return q4 ? launch_tiled_t<128, true, WF_Q4>(ta, s) : launch_tiled_t<128, true, WF_BF16>(ta, s);
    return q4 ? launch_tiled_t<128, false, WF_Q4>(ta, s) : launch_tiled_t<128, false, WF_BF16>(ta, s);
}

}  // namespace dsmoe
