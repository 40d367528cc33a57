// dispatch.hip - stable counting sort of token slots by expert.
//
// The grouping behind the gather_mm / gather_qmm expert calls (page "Epic: Engine Inference
// Core Stage E - MoE + hybrid families", opening paragraph): slot s = t*K + j goes to expert
// inds[s]; the expert-major row space lists every expert's slots contiguously, experts in
// ascending order and, inside an expert, slots in ascending order (a stable sort, so the
// layout is deterministic).
//
// Three launches, no atomics on global memory, no host round trip:
//   count   - each workgroup of DB slots builds an LDS histogram (LDS atomics only change
//             the order of increments, not the counts) and writes its row of blk[nblk][E];
//   scan    - one workgroup: column prefix over workgroups, expert totals, an exclusive scan
//             over experts (offsets), then blk[b][e] becomes the first output row of
//             workgroup b's slots of expert e;
//   scatter - each slot's row = blk[b][e] + (same-expert slots in earlier waves of its
//             workgroup) + (same-expert slots in earlier lanes of its wave).
#include "dsmoe_internal.hpp"

namespace dsmoe {
namespace {

constexpr int NW = 8;        // waves per dispatch workgroup
constexpr int DB = 64 * NW;  // slots per dispatch workgroup

__device__ __forceinline__ int32_t clamp_e(int32_t e, int32_t E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(DB) void count_kernel(const int32_t* __restrict__ inds, int32_t TK, int32_t E,
                                                   int32_t* __restrict__ blk) {
    __shared__ int32_t hist[MOE_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += DB) hist[e] = 0;
    __syncthreads();
    const int32_t s = blockIdx.x * DB + threadIdx.x;
    if (s < TK) atomicAdd(&hist[clamp_e(inds[s], E)], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += DB) blk[(int64_t)blockIdx.x * E + e] = hist[e];
}

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk, int32_t nblk, int32_t E, int32_t TK,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
    __shared__ int32_t buf[1024];
    const int e = threadIdx.x;  // E <= 1024
    constexpr int U = 16;       // column entries read before any is written back: the loads of a
                                // batch are in flight together instead of one after each store
    int32_t tot = 0;
    if (e < E) {
        for (int32_t b0 = 0; b0 < nblk; b0 += U) {
            int32_t c[U];
#pragma unroll
            for (int j = 0; j < U; ++j) c[j] = b0 + j < nblk ? blk[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < U; ++j) {
                if (b0 + j < nblk) blk[(int64_t)(b0 + j) * E + e] = tot;
                tot += c[j];
            }
        }
        counts[e] = tot;
    }
    buf[e] = tot;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v = e >= off ? buf[e - off] : 0;
        __syncthreads();
        buf[e] += v;
        __syncthreads();
    }
    const int32_t excl = buf[e] - tot;
    if (e < E) {
        offsets[e] = excl;
        for (int32_t b0 = 0; b0 < nblk; b0 += U) {
            int32_t c[U];
#pragma unroll
            for (int j = 0; j < U; ++j) c[j] = b0 + j < nblk ? blk[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < U; ++j)
                if (b0 + j < nblk) blk[(int64_t)(b0 + j) * E + e] = c[j] + excl;
        }
    }
    if (e == 0) offsets[E] = TK;
}

__global__ __launch_bounds__(DB) void scatter_kernel(const int32_t* __restrict__ inds, int32_t TK, int32_t E,
                                                     const int32_t* __restrict__ blk,
                                                     int32_t* __restrict__ sorted_slot,
                                                     int32_t* __restrict__ slot_row) {
    __shared__ int32_t wcnt[NW][MOE_MAX_EXPERTS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < NW * E; i += DB) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int32_t s = blockIdx.x * DB + threadIdx.x;
    const bool valid = s < TK;
    const int32_t e = valid ? clamp_e(inds[s], E) : -1;
    if (valid) atomicAdd(&wcnt[wave][e], 1);
    __syncthreads();
    // same-expert slots in earlier lanes of this wave
    int32_t rank = 0;
    for (int j = 0; j < 64; ++j) {
        const int32_t ej = __builtin_amdgcn_readlane(e, j);
        rank += (j < lane) && (ej == e);
    }
    if (valid) {
        for (int w = 0; w < wave; ++w) rank += wcnt[w][e];
        const int32_t row = blk[(int64_t)blockIdx.x * E + e] + rank;
        sorted_slot[row] = s;
        slot_row[s] = row;
    }
}

}  // namespace

int32_t dispatch_blocks(int64_t TK) { return (int32_t)((TK + DB - 1) / DB); }

hipError_t launch_dispatch(const int32_t* inds, int64_t T, int32_t K, int32_t E, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_slot, int32_t* slot_row, int32_t* blk, hipStream_t s) {
    const int32_t TK = (int32_t)(T * K);
    const int32_t nblk = dispatch_blocks(TK);
    if (nblk > 0) {
        hipLaunchKernelGGL(count_kernel, dim3(nblk), dim3(DB), 0, s, inds, TK, E, blk);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, blk, nblk, E, TK, counts, offsets);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || nblk == 0) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3(nblk), dim3(DB), 0, s, inds, TK, E, blk, sorted_slot, slot_row);
    return hipGetLastError();
}

}  // namespace dsmoe
