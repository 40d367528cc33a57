// experts_stream.hip - weight streaming through an LDS DMA ring, for bf16 expert groups of up to
// 64 rows (the decode regime, and the small groups of prefill batches).
//
// Same computation as the streaming kernel of experts.hip (page "Epic: Engine Inference Core
// Stage E - MoE + hybrid families", opening paragraph: the per-expert matmuls of gather_mm, SwiGLU
// fused into the first GEMM's epilogue):
//   GEMM-1: h[r, n] = bf16( silu(x[tok(r)] . W_gate[g, n]) * (x[tok(r)] . W_up[g, n]) )
//   GEMM-2: o[r, n] = bf16( h[r] . W_down[g, n] )
// These groups are bound by reading their weights from HBM once.  A load instruction in the MFMA
// operand layout covers half of a 128-byte line per weight row (four lanes of 16 bytes), and
// such loads reach about 6.1 TB/s whether or not they carry the non-temporal hint; LDS DMA
// instructions in which eight lanes fetch one whole line, with the hint, reach about 7.2 TB/s
// with 32 KB in flight per CU (measured on MI355X).  So here the weights enter LDS by DMA, one
// whole line per weight row per 64-k stage, through a ring of three stages (two in flight while
// one is multiplied), and the MFMA operands are read from LDS.
//
// Workgroup: four waves, every row of the group in chunks of 64, and 128 weight rows: for GEMM-1
// the gate rows of 64 output columns, then their up rows; for GEMM-2 128 output columns, as two
// halves of 64 (wave w: columns [16 w, 16 w + 16) of each; 128 rather than 64 columns per
// workgroup measured 607 -> 598 us for the DeepSeek-V3 decode batch).  Stage slot: the chunk's
// activation rows [64][128 B], then the weight rows [128][128 B].  Chunk c of row r sits at
// chunk c ^ swz(r) (the swizzle of the tiled kernels), so the
// 16 rows of an MFMA operand read fall in distinct banks.  Weight DMA: instruction t of wave w
// fetches rows [8 (w T + t), +8), lane i row + i / 8, the logical chunk its LDS slot holds.
// Activation DMA: as in experts.hip, wave w copies rows [16 w, 16 w + 16) when the chunk has a
// row there (the waits below count per wave).  MFMA 16x16x32 bf16: lane l supplies row/column
// (l % 16) and the 8 k values of chunk (l / 16) of a 32-k step.
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

constexpr int SD_THREADS = 256;
constexpr int SD_NS = 3;      // ring depth
constexpr int SD_ROWB = 128;  // bytes per row and stage: 64 k of bf16
constexpr int SD_AROWS = 64;  // activation rows per chunk
constexpr int SD_A_BYTES = SD_AROWS * SD_ROWB;
constexpr int sd_wrows(bool) { return 128; }
constexpr int sd_stage_bytes(bool g1) { return SD_A_BYTES + sd_wrows(g1) * SD_ROWB; }
constexpr int sd_lds_bytes(bool g1) { return SD_NS * sd_stage_bytes(g1); }

// cache-policy bits of a load: non-temporal (the weights are read once)
constexpr int SD_NT = 2;

#define DSMOE_SD_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ int sd_swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ uint32_t sd_off(int r, int c) { return (uint32_t)(r * SD_ROWB + ((c ^ sd_swz(r)) << 4)); }
__device__ __forceinline__ bf16x8 sd_frag(const char* p) { return __builtin_bit_cast(bf16x8, *(const u32x4*)p); }
__device__ __forceinline__ float sd_silu(float z) { return z / (1.0f + __expf(-z)); }

template <int N>
__device__ __forceinline__ void sd_wait_barrier() { asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory"); }

template <bool G1>
__global__ __launch_bounds__(SD_THREADS) void stream_dma(GroupedArgs a, int32_t g0) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    constexpr int WR = sd_wrows(G1);
    constexpr int ST = sd_stage_bytes(G1);
    constexpr int WT = WR / 8 / 4;  // weight DMA instructions per wave per stage
    constexpr int NW = 2;           // weight row blocks: gate and up (G1), or two 64-column halves
    // the last group of the launch first: workgroups are dispatched in grid order, and the last
    // group -- the shared expert, whose chunk holds every token -- would otherwise end the launch
    const int32_t g = g0 + (int32_t)((blockIdx.y + gridDim.y - 1) % gridDim.y);
    int32_t r0, cnt;
    if (g < a.E) {
        r0 = a.offsets[g];
        cnt = a.offsets[g + 1] - r0;
    } else {
        r0 = a.TK;
        cnt = (int32_t)a.T;
    }
    if (cnt <= 0 || cnt > a.stream_max_rows) return;  // workgroup-uniform
    const bool shared = g == a.E;
    const int32_t N = G1 ? (shared ? a.Is : a.I) : a.H;
    const int32_t KD = G1 ? a.H : (shared ? a.Is : a.I);  // a multiple of 64
    const int32_t col0 = blockIdx.x * (G1 ? 64 : 128);
    if (col0 >= N) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int nst = KD >> 6;
    // GEMM-2 weight rows are I * 2 bytes apart, a power of two for the usual I: when every
    // workgroup in flight fetches the same line offset of its rows, the loads crowd a few memory
    // channels.  Each GEMM-2 workgroup therefore starts its pass over k at its own stage and wraps.
    const int rot = G1 ? 0 : (int)((blockIdx.x * 7u) % (unsigned)nst);

    // weight rows: uniform bases (64-bit) plus per-lane 32-bit byte offsets
    const char* wbase[2];
    {
        const int64_t eo = (int64_t)g * N;  // first weight row of the expert
        if (G1) {
            wbase[0] = shared ? (const char*)a.swg : (const char*)((const bf16_t*)a.wg + eo * KD);
            wbase[1] = shared ? (const char*)a.swu : (const char*)((const bf16_t*)a.wu + eo * KD);
        } else {
            wbase[0] = wbase[1] = shared ? (const char*)a.swd : (const char*)((const bf16_t*)a.wd + eo * KD);
        }
    }
    uint32_t w_off[WT];
#pragma unroll
    for (int t = 0; t < WT; ++t) {
        const int rho = (wave * WT + t) * 8 + (lane >> 3);  // slot row
        const int c = (lane & 7) ^ sd_swz(rho);
        const int32_t n = G1 ? col0 + (rho & 63) : min(col0 + rho, N - 1);  // rows past N: never stored
        w_off[t] = ((uint32_t)n * (uint32_t)KD + c * 8) * 2u;
    }
    const char* abase = G1 ? (const char*)a.x : (const char*)a.h;
    const int64_t lda = G1 ? a.H : a.ldh;

    for (int32_t m0 = 0; m0 < cnt; m0 += SD_AROWS) {
        const int nrb = min(4, (cnt - m0 + 15) >> 4);  // live 16-row blocks
        // activation DMA sources of this wave (rows [16 w, 16 w + 16), when w < nrb)
        const char* arow[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = wave * 16 + j * 8 + (lane >> 3);
            const int c = (lane & 7) ^ sd_swz(r);
            int32_t rr = m0 + r;
            rr = rr < cnt ? rr : cnt - 1;  // rows past the group are computed, never stored
            const int64_t src = G1 ? (int64_t)(r0 + rr < a.TK ? a.sorted_slot[r0 + rr] / a.K : r0 + rr - a.TK)
                                   : (int64_t)(r0 + rr);
            arow[j] = abase + (src * lda + c * 8) * 2;
        }
        const bool copier = wave < nrb;  // wave-uniform
        auto issue = [&](int s) {
            char* st = smem + (s % SD_NS) * ST;
            int sr = s + rot;
            if (sr >= nst) sr -= nst;
            const int32_t kb = sr * 128;  // byte offset of the stage's 64 k
            if (copier) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    __builtin_amdgcn_global_load_lds((const void*)(arow[j] + kb),
                                                     DSMOE_SD_LDS(st + (wave * 2 + j) * 1024), 16, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < WT; ++t) {
                const int rho0 = (wave * WT + t) * 8;
                const char* wb = wbase[G1 && rho0 >= 64 ? 1 : 0];
                __builtin_amdgcn_global_load_lds((const void*)(wb + w_off[t] + kb),
                                                 DSMOE_SD_LDS(st + SD_A_BYTES + rho0 * SD_ROWB), 16, 0, SD_NT);
            }
        };
        f32x4 acc[NW][4];
#pragma unroll
        for (int m = 0; m < NW; ++m)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) acc[m][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int q = lane >> 4, ln = lane & 15;
        auto compute = [&](int s) {
            const char* st = smem + (s % SD_NS) * ST;
#pragma unroll
            for (int t = 0; t < 2; ++t) {  // two 32-k steps per stage
                const int c = t * 4 + q;
                bf16x8 wf[NW];
#pragma unroll
                for (int m = 0; m < NW; ++m) wf[m] = sd_frag(st + SD_A_BYTES + sd_off(m * 64 + wave * 16 + ln, c));
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    if (rb >= nrb) break;
                    const bf16x8 af = sd_frag(st + sd_off(rb * 16 + ln, c));
#pragma unroll
                    for (int m = 0; m < NW; ++m)
                        acc[m][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf[m], acc[m][rb], 0, 0, 0);
                }
            }
        };
        // per wave, the DMA operations of one stage
        constexpr int D_COPY = WT + 2, D_NOCOPY = WT;

        __syncthreads();  // the previous chunk's reads of every slot are done
        issue(0);
        if (nst > 1) issue(1);
        for (int s = 0; s < nst; ++s) {
            // stage s has landed for every wave; stage s+1 (if issued) may still be in flight
            if (s + 1 < nst) {
                if (copier) sd_wait_barrier<D_COPY>();  // wave-uniform; both arms hold one barrier
                else sd_wait_barrier<D_NOCOPY>();
            } else {
                sd_wait_barrier<0>();
            }
            // the slot of stage s+2 held stage s-1, which every wave finished before this barrier
            if (s + 2 < nst) issue(s + 2);
            compute(s);
        }
        // the accumulators are read right after the last MFMAs, possibly behind the row-block
        // branch: issue the MFMA-to-VALU wait states explicitly before any of them is read
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0][0]));
#pragma unroll
        for (int m = 0; m < NW; ++m)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                if (m | rb) asm volatile("" : "+a"(acc[m][rb]));
        const int32_t col = col0 + wave * 16 + ln;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            if (rb >= nrb) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int32_t rr = m0 + rb * 16 + q * 4 + v;
                if (rr >= cnt) continue;
                if (G1) {
                    ((bf16_t*)a.h)[(int64_t)(r0 + rr) * a.ldh + col] = f32_to_bf16(sd_silu(acc[0][rb][v]) * acc[1][rb][v]);
                } else {
                    bf16_t* orow = (bf16_t*)a.o + (int64_t)(r0 + rr) * a.H;
                    orow[col] = f32_to_bf16(acc[0][rb][v]);
                    if (col + 64 < N) orow[col + 64] = f32_to_bf16(acc[1][rb][v]);
                }
            }
        }
    }
}

}  // namespace

hipError_t configure_stream_dma() {
    hipError_t e = hipFuncSetAttribute((const void*)stream_dma<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       sd_lds_bytes(true));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)stream_dma<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               sd_lds_bytes(false));
}

// the weight rows are addressed with 32-bit byte offsets within an expert
bool stream_dma_fits(const GroupedArgs& a) {
    const int64_t n = a.I > a.Is ? a.I : a.Is;
    return n * a.H * 2 < ((int64_t)1 << 32);
}

hipError_t launch_stream_dma(const GroupedArgs& a, bool gemm1, int32_t g0, int32_t g1, hipStream_t s) {
    if (g1 <= g0) return hipSuccess;
    if (gemm1) {
        const int32_t N = max(a.I, a.Is);
        hipLaunchKernelGGL((stream_dma<true>), dim3((N + 63) / 64, g1 - g0), dim3(SD_THREADS), sd_lds_bytes(true), s, a,
                           g0);
    } else {
        hipLaunchKernelGGL((stream_dma<false>), dim3((a.H + 127) / 128, g1 - g0), dim3(SD_THREADS), sd_lds_bytes(false),
                           s, a, g0);
    }
    return hipGetLastError();
}

}  // namespace dsmoe
