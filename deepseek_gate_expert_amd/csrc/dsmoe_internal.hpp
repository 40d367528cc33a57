// dsmoe_internal.hpp - device helpers and kernel launchers of libdsmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsmoe.h"  // include/ is on the include path

namespace dsmoe {

// exp by Cody & Waite range reduction with a degree-7 Taylor polynomial, evaluated with exactly
// the fp32 operations spelled out in route.hip's header (used by the gate and by the shared-
// expert gate in the combine, so both follow one definition)
__device__ __forceinline__ float exp_cw(float x) {
    if (x != x) return x;
    if (x > 0x1.62e430p+6f) return __builtin_inff();
    if (x < -0x1.5d589ep+6f) return 0.0f;
    const float n = __builtin_rintf(x * 0x1.715476p+0f);
    float r = __builtin_fmaf(-n, 0x1.62e400p-1f, x);
    r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
    float p = 0x1.a01a02p-13f;
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float sigmoid_cw(float x) { return 1.0f / (1.0f + exp_cw(-x)); }

typedef uint16_t bf16_t;  // raw bf16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native 16-byte vector (promotes to VGPRs)
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

static_assert(sizeof(bf16x8) == 16, "bf16x8 is 16 bytes");

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(bf16_t, b);
}

// two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// One launch of the grouped expert GEMMs.  Groups g in [0, E) are the routed experts with
// rows [offsets[g], offsets[g+1]) of the expert-major row space; group E is the shared expert
// with rows [TK, TK + T) (row TK + t is token t).
struct GroupedArgs {
    int64_t T;
    int32_t H, E, I, Is, K;      // K = top_k
    int32_t TK;                  // T * K
    int32_t ldh;                 // row stride of h (max(I, Is))
    const int32_t* offsets;      // [E + 1]
    const int32_t* sorted_slot;  // [TK]
    const int32_t* inds;         // [T, K]
    const void* x;               // [T, H] act
    void* h;                     // [TK + T, ldh] act (SwiGLU intermediate)
    void* o;                     // [TK + T, H] act (per-row expert output)
    const void* wg;              // routed [E, I, H] (q4: uint32 [E, I, H/8]; fp8: uint8 codes)
    const void* wu;
    const void* wd;              // routed [E, H, I]
    const bf16_t *sg, *bg, *su, *bu, *sd, *bd;  // q4 scale / offset [E, out, in/64]
    const float *fsg, *fsu, *fsd;  // fp8 block scales [E, ceil(out/128), ceil(in/128)]
    const void* swg;             // shared [Is, H] act
    const void* swu;
    const void* swd;             // shared [H, Is] act
    int32_t stream_max_rows;     // weight-streaming kernels skip groups with more rows than this
};

// launchers (return hipSuccess or the launch error)
hipError_t launch_router(const void* x, const void* w, int32_t act, int64_t T, int32_t H, int32_t E,
                         const float* offset, float* logits, hipStream_t s);
hipError_t launch_route(const float* logits, int64_t T, int32_t E, const float* bias, const moe_route_params& p,
                        int32_t* inds, float* scores, hipStream_t s);
int32_t dispatch_blocks(int64_t TK);
hipError_t launch_dispatch(const int32_t* inds, int64_t T, int32_t K, int32_t E, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_slot, int32_t* slot_row, int32_t* blk, hipStream_t s);
// bf16-activation expert GEMMs for groups [g0, g1); wdt = weight dtype of the routed groups
// (MOE_BF16, MOE_Q4G64 or MOE_FP8; the shared group E is always bf16 and may be in the range)
hipError_t launch_gemm1_bf16(const GroupedArgs& a, int32_t g0, int32_t g1, int32_t wdt, hipStream_t s);
hipError_t launch_gemm2_bf16(const GroupedArgs& a, int32_t g0, int32_t g1, int32_t wdt, hipStream_t s);
// bf16 weights of groups [g0, g1) streamed through an LDS DMA ring (groups of at most
// stream_max_rows rows); configure once per device before the first launch
hipError_t configure_stream_dma();
bool stream_dma_fits(const GroupedArgs& a);
hipError_t launch_stream_dma(const GroupedArgs& a, bool gemm1, int32_t g0, int32_t g1, hipStream_t s);
// fp8 layers: routed groups of at most 32 rows stream their codes through an LDS DMA ring, the
// rest as launch_gemm1_bf16 / launch_gemm2_bf16 would; configure once per device
hipError_t configure_stream_f8();
bool stream_f8_fits(const GroupedArgs& a);
hipError_t launch_stream_f8(const GroupedArgs& a, bool gemm1, int32_t g0, int32_t g1, hipStream_t s);
// fp32 layers: all routed rows and the shared rows in one launch each
hipError_t launch_gemm1_f32(const GroupedArgs& a, hipStream_t s);
hipError_t launch_gemm2_f32(const GroupedArgs& a, hipStream_t s);
// tiled grouped GEMMs (groups with more than min_rows rows; tile list built on the device)
int32_t tiled_max_tiles(int64_t T, int32_t K, int32_t E, int32_t BM);
int32_t tiled_lds_bytes(int32_t BM);
// tile height of the quantised tiled kernels for expert dtype wdt (MOE_Q4G64 or MOE_FP8)
int32_t tiled_quant_bm(int32_t wdt);
hipError_t configure_tiled_kernels();
// tile list: routed groups in tiles of BM rows, the shared expert (group E) in tiles of BMs rows
hipError_t launch_tiles(const GroupedArgs& a, int32_t BM, int32_t BMs, int32_t min_rows, int32_t* tile_count,
                        int32_t* tile_info, hipStream_t s);
hipError_t launch_gemm_tiled(const GroupedArgs& a, bool gemm1, int32_t BM, int32_t g0, int32_t g1, int32_t wdt,
                             const int32_t* tile_count, const int32_t* tile_info, int32_t max_tiles, hipStream_t s);
hipError_t launch_route_softmax(const float* logits, int64_t T, int32_t E, int32_t K, int32_t* inds, float* scores,
                                hipStream_t s);
// sgate_logits: NULL, or [T] fp32 logits of the shared-expert gate (the shared row is scaled by
// their sigmoid)
hipError_t launch_combine(const GroupedArgs& a, int32_t act, const float* scores, const int32_t* slot_row,
                          const float* sgate_logits, void* y, hipStream_t s);

}  // namespace dsmoe
