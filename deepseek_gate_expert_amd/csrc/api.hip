// api.hip - the C ABI of libdsmoe: host-side validation, workspace layout and the launch
// sequence of the MoE layer forward.  Contract and citations: include/dsmoe.h.
//
// Everything here is host code.  All argument checks run before the first HIP call, so a
// rejected call touches no device memory.  No call synchronises the stream or reads device
// memory back; expert counts stay on the device and the expert kernels read them there.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "dsmoe_internal.hpp"
#include "stage_hook.hpp"

using namespace dsmoe;

namespace {

constexpr size_t ALIGN = 256;

inline size_t up(size_t v) { return (v + ALIGN - 1) & ~(ALIGN - 1); }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// pointer may be NULL only when `may_be_null`
inline bool ptr_ok(const void* p, bool may_be_null) { return p ? aligned16(p) : may_be_null; }

int check_route_params(int32_t E, const moe_route_params* p) {
    if (!p) return MOE_ERR_INVALID;
    if (E < 1) return MOE_ERR_INVALID;
    if (p->top_k < 1 || p->top_k > E) return MOE_ERR_INVALID;
    if (p->n_group < 1 || E % p->n_group != 0) return MOE_ERR_INVALID;
    if (p->topk_group < 1 || p->topk_group > p->n_group) return MOE_ERR_INVALID;
    if (p->n_group > 1 && E / p->n_group < 2) return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || p->top_k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

size_t dispatch_ws_bytes(int64_t T, int32_t K, int32_t E) {
    return up((size_t)dispatch_blocks(T * K) * (size_t)E * sizeof(int32_t));
}

// Groups with more rows than this go to the LDS-tiled GEMMs (when T exceeds it); the rest are
// streamed (each weight read once per 64 rows).
constexpr int32_t STREAM_MAX_ROWS = 64;

struct TilePlan {
    bool on;
    int32_t BM;         // tile height of the routed groups
    int32_t BMs;        // tile height of the shared expert
    int32_t max_tiles;  // bound on the tile list (for the smaller of the two heights)
    int32_t min_rows;   // groups with more rows than this are tiled, the others streamed
};

// Shapes-only decision (no device reads).  bf16 weights: tiles of 256 rows when the average
// group is large, else 128.  4-bit and fp8 weights: the height of their kernel (160 and 128
// rows), each tile computed at its real height rounded up to 32 rows.
TilePlan plan_tiles(const moe_layer_desc* d, bool allow256) {
    TilePlan p{false, 128, 128, 0, STREAM_MAX_ROWS};
    if (d->act_dtype != MOE_BF16 || d->T <= STREAM_MAX_ROWS) return p;
    // the tiled kernels address activation and weight rows with 32-bit byte offsets
    const int64_t rows = d->T * d->route.top_k + d->T;
    const int64_t ldh = d->I > d->I_shared ? d->I : d->I_shared;
    const int64_t lim = (int64_t)1 << 31;  // elements of 2 bytes
    if (d->T * (int64_t)d->H >= lim || rows * ldh >= lim || (int64_t)d->I * d->H >= lim ||
        (int64_t)d->I_shared * d->H >= lim)
        return p;
    const bool quant = d->expert_dtype != MOE_BF16;
    if (quant && tiled_quant_bm(d->expert_dtype) > (allow256 ? 256 : 128)) return p;
    p.on = true;
    const int64_t avg = d->T * d->route.top_k / d->E;
    p.BM = quant ? tiled_quant_bm(d->expert_dtype) : (allow256 && avg >= 192) ? 256 : 128;
    // bf16 layers run the shared expert in the routed groups' launch; quantised layers give its
    // bf16 weights a launch of their own, with 256-row tiles once it has that many rows
    p.BMs = d->expert_dtype == MOE_BF16 ? p.BM : (allow256 && d->T >= 256 ? 256 : 128);
    p.max_tiles = tiled_max_tiles(d->T, d->route.top_k, d->E, p.BM < p.BMs ? p.BM : p.BMs);
    // Quantised routed groups of any size go to the tiled kernel, whose 64-row variant moves
    // the codes by DMA and dequantises each weight once: for small groups it outruns the
    // streaming kernel, whose 4-bit steps are a few short loads per lane and a barrier.
    if (quant) p.min_rows = 0;
    return p;
}

struct FwdLayout {
    size_t logits, sgl, inds, scores, blk, counts, offsets, sorted_slot, slot_row, tiles, h, o, total;
};

FwdLayout fwd_layout(const moe_layer_desc* d) {
    FwdLayout L;
    const size_t T = (size_t)d->T, K = (size_t)d->route.top_k, E = (size_t)d->E;
    const size_t TK = T * K;
    const size_t rows = TK + (d->I_shared > 0 ? T : 0);
    const size_t el = d->act_dtype == MOE_F32 ? 4 : 2;
    const size_t ldh = (size_t)(d->I > d->I_shared ? d->I : d->I_shared);
    size_t off = 0;
    L.logits = off;
    off += up(T * E * 4);
    L.sgl = off;  // shared-expert gate logits
    off += up(T * 4);
    L.inds = off;
    off += up(TK * 4);
    L.scores = off;
    off += up(TK * 4);
    L.blk = off;
    off += dispatch_ws_bytes(d->T, d->route.top_k, d->E);
    L.counts = off;
    off += up(E * 4);
    L.offsets = off;
    off += up((E + 1) * 4);
    L.sorted_slot = off;
    off += up(TK * 4);
    L.slot_row = off;
    off += up(TK * 4);
    L.tiles = off;  // tile count + 16-byte tile entries; sized for the smaller tile height
    off += up(256 + 16 * (size_t)tiled_max_tiles(d->T, d->route.top_k, d->E, 128));
    L.h = off;
    off += up(rows * ldh * el);
    L.o = off;
    off += up(rows * (size_t)d->H * el);
    L.total = off;
    return L;
}

int check_desc(const moe_layer_desc* d) {
    if (!d) return MOE_ERR_INVALID;
    if (d->T < 0 || d->H < 1 || d->E < 1 || d->I < 1 || d->I_shared < 0) return MOE_ERR_INVALID;
    const int32_t a = d->act_dtype, w = d->expert_dtype;
    const bool combo =
        (a == MOE_F32 && w == MOE_F32) || (a == MOE_BF16 && (w == MOE_BF16 || w == MOE_Q4G64 || w == MOE_FP8));
    if (!combo) return MOE_ERR_INVALID;
    if (d->route_kind != MOE_ROUTE_DEEPSEEK && d->route_kind != MOE_ROUTE_SOFTMAX) return MOE_ERR_INVALID;
    int rc = MOE_OK;
    if (d->route_kind == MOE_ROUTE_DEEPSEEK) {
        rc = check_route_params(d->E, &d->route);
    } else if (d->route.top_k < 1 || d->route.top_k > d->E) {
        rc = MOE_ERR_INVALID;
    } else if (d->E > MOE_MAX_EXPERTS || d->route.top_k > MOE_MAX_TOP_K) {
        rc = MOE_ERR_UNSUPPORTED;
    }
    if (rc != MOE_OK) return rc;
    if ((int64_t)d->T * (d->route.top_k + 1) >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (a == MOE_BF16 && (d->H % 64 || d->I % 64 || d->I_shared % 64)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

inline int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Per device: 1 tiles of 256 rows fit in LDS, 2 only 128, 3 tiled kernels unusable.  Found once
// per device (the first call on it configures the tiled kernels' LDS limits); std::call_once
// makes concurrent first calls safe.
constexpr int MAX_DEVICES = 64;
int g_tiled_state[MAX_DEVICES];
bool g_stream_dma_ok[MAX_DEVICES];  // the DMA weight-streaming kernels may take their LDS
bool g_stream_f8_ok[MAX_DEVICES];   // likewise the fp8 ones
std::once_flag g_tiled_once[MAX_DEVICES];

int tiled_state() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 3;
    std::call_once(g_tiled_once[dev], [dev] {
        int lds = 0;
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        int st = 3;
        if (configure_tiled_kernels() == hipSuccess) {
            if (lds >= tiled_lds_bytes(256)) st = 1;
            else if (lds >= tiled_lds_bytes(128)) st = 2;
        }
        g_stream_dma_ok[dev] = configure_stream_dma() == hipSuccess;
        g_stream_f8_ok[dev] = configure_stream_f8() == hipSuccess;
        (void)hipGetLastError();
        g_tiled_state[dev] = st;
    });
    return g_tiled_state[dev];
}

// bf16 weight streaming through the LDS DMA ring when the device allows its LDS and the weight
// offsets fit 32 bits; else the register-streaming kernel
bool use_stream_dma(const GroupedArgs& a) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return false;
    tiled_state();
    return g_stream_dma_ok[dev] && stream_dma_fits(a);
}

// fp8 codes of small groups through the LDS DMA ring when the device allows its LDS and the
// reduction lengths suit it; else the register-streaming kernel for every group
bool use_stream_f8(const GroupedArgs& a) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return false;
    tiled_state();
    return g_stream_f8_ok[dev] && stream_f8_fits(a);
}

// Dense SwiGLU MLP: the shared-expert path on its own (group E with E = 0 routed experts).
struct DenseLayout {
    size_t tiles, h, total;
};

int32_t dense_bm(int64_t T, bool allow256) { return (allow256 && T >= 192) ? 256 : 128; }

DenseLayout dense_layout(int64_t T, int32_t I, int32_t act) {
    DenseLayout L;
    const size_t el = act == MOE_F32 ? 4 : 2;
    size_t off = 0;
    L.tiles = off;
    off += up(256 + 16 * (size_t)tiled_max_tiles(T, 0, 0, 128));
    L.h = off;
    off += up((size_t)T * (size_t)I * el);
    L.total = off;
    return L;
}

int check_dense(int64_t T, int32_t H, int32_t I, int32_t act) {
    if (T < 0 || H < 1 || I < 1 || (act != MOE_F32 && act != MOE_BF16)) return MOE_ERR_INVALID;
    if (act == MOE_BF16 && (H % 64 || I % 64)) return MOE_ERR_UNSUPPORTED;
    if (T >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// measurement hook state (see moe_set_stage_events)
StageHookRegistry g_hook;

// the events one moe_forward call records (stage -1: none)
struct HookCall {
    HookPair p;
    // records the start (edge 0) or stop (edge 1) event of `st` for this call
    hipError_t mark(int32_t st, int edge, hipStream_t s) const {
        if (st != p.stage) return hipSuccess;
        return hipEventRecord((hipEvent_t)(edge ? p.stop : p.start), s);
    }
};

// Argument checks of moe_forward, all on the host, except those of the workspace.
int check_forward(const moe_layer_desc* d, const void* x, const void* router_w, const float* bias,
                  const float* logit_offset, const moe_expert_weights* ew, const moe_shared_weights* sw, const void* y,
                  const int32_t* inds_out, const float* scores_out) {
    int rc = check_desc(d);
    if (rc != MOE_OK) return rc;
    const bool empty = d->T == 0;
    const bool softmax = d->route_kind == MOE_ROUTE_SOFTMAX;
    if (!ptr_ok(x, empty) || !ptr_ok(router_w, false) || !ptr_ok(bias, softmax) || !ptr_ok(logit_offset, true) ||
        !ptr_ok(y, empty) || !ptr_ok(inds_out, true) || !ptr_ok(scores_out, true))
        return MOE_ERR_INVALID;
    if (!ew || !ptr_ok(ew->w_gate, false) || !ptr_ok(ew->w_up, false) || !ptr_ok(ew->w_down, false))
        return MOE_ERR_INVALID;
    if (d->expert_dtype == MOE_Q4G64 &&
        (!ptr_ok(ew->s_gate, false) || !ptr_ok(ew->b_gate, false) || !ptr_ok(ew->s_up, false) ||
         !ptr_ok(ew->b_up, false) || !ptr_ok(ew->s_down, false) || !ptr_ok(ew->b_down, false)))
        return MOE_ERR_INVALID;
    if (d->expert_dtype == MOE_FP8 &&
        (!ptr_ok(ew->s_gate, false) || !ptr_ok(ew->s_up, false) || !ptr_ok(ew->s_down, false)))
        return MOE_ERR_INVALID;
    if (d->I_shared > 0) {
        if (!sw || !ptr_ok(sw->w_gate, false) || !ptr_ok(sw->w_up, false) || !ptr_ok(sw->w_down, false) ||
            !ptr_ok(sw->w_sgate, true))
            return MOE_ERR_INVALID;
    } else if (sw) {
        return MOE_ERR_INVALID;
    }
    return MOE_OK;
}

// The launch sequence of the layer into a checked workspace `ws` laid out as L (T > 0).
int launch_forward(const moe_layer_desc* d, const void* x, const void* router_w, const float* bias,
                   const float* logit_offset, const moe_expert_weights* ew, const moe_shared_weights* sw, void* y,
                   int32_t* inds_out, float* scores_out, char* ws, const FwdLayout& L, void* stream) {
    int rc = MOE_OK;
    const bool softmax = d->route_kind == MOE_ROUTE_SOFTMAX;
    hipStream_t s = (hipStream_t)stream;
    const HookCall hook{g_hook.take()};
    auto mark = [&hook](int32_t st, int edge, hipStream_t q) { return hook.mark(st, edge, q); };
    float* logits = (float*)(ws + L.logits);
    float* sgl = (d->I_shared > 0 && sw->w_sgate) ? (float*)(ws + L.sgl) : nullptr;
    int32_t* inds = inds_out ? inds_out : (int32_t*)(ws + L.inds);
    float* scores = scores_out ? scores_out : (float*)(ws + L.scores);
    int32_t* blk = (int32_t*)(ws + L.blk);
    int32_t* counts = (int32_t*)(ws + L.counts);
    int32_t* offsets = (int32_t*)(ws + L.offsets);
    int32_t* sorted_slot = (int32_t*)(ws + L.sorted_slot);
    int32_t* slot_row = (int32_t*)(ws + L.slot_row);
    int32_t* tile_count = (int32_t*)(ws + L.tiles);
    int32_t* tile_info = tile_count + 64;  // keep the entries 256-byte aligned

    if ((rc = hip_rc(mark(MOE_STAGE_ROUTER, 0, s)))) return rc;
    if ((rc = hip_rc(launch_router(x, router_w, d->act_dtype, d->T, d->H, d->E, logit_offset, logits, s))))
        return rc;
    if ((rc = hip_rc(mark(MOE_STAGE_ROUTER, 1, s)))) return rc;
    if ((rc = hip_rc(mark(MOE_STAGE_ROUTE, 0, s)))) return rc;
    if ((rc = hip_rc(softmax ? launch_route_softmax(logits, d->T, d->E, d->route.top_k, inds, scores, s)
                             : launch_route(logits, d->T, d->E, bias, d->route, inds, scores, s))))
        return rc;
    if ((rc = hip_rc(mark(MOE_STAGE_ROUTE, 1, s)))) return rc;
    if ((rc = hip_rc(mark(MOE_STAGE_DISPATCH, 0, s)))) return rc;
    if ((rc = hip_rc(launch_dispatch(inds, d->T, d->route.top_k, d->E, counts, offsets, sorted_slot, slot_row, blk,
                                     s))))
        return rc;
    if ((rc = hip_rc(mark(MOE_STAGE_DISPATCH, 1, s)))) return rc;

    GroupedArgs a;
    memset(&a, 0, sizeof(a));
    a.T = d->T;
    a.H = d->H;
    a.E = d->E;
    a.I = d->I;
    a.Is = d->I_shared;
    a.K = d->route.top_k;
    a.TK = (int32_t)(d->T * d->route.top_k);
    a.ldh = d->I > d->I_shared ? d->I : d->I_shared;
    a.offsets = offsets;
    a.sorted_slot = sorted_slot;
    a.inds = inds;
    a.x = x;
    a.h = ws + L.h;
    a.o = ws + L.o;
    a.wg = ew->w_gate;
    a.wu = ew->w_up;
    a.wd = ew->w_down;
    if (d->expert_dtype == MOE_Q4G64) {
        a.sg = (const bf16_t*)ew->s_gate;
        a.bg = (const bf16_t*)ew->b_gate;
        a.su = (const bf16_t*)ew->s_up;
        a.bu = (const bf16_t*)ew->b_up;
        a.sd = (const bf16_t*)ew->s_down;
        a.bd = (const bf16_t*)ew->b_down;
    } else if (d->expert_dtype == MOE_FP8) {
        a.fsg = (const float*)ew->s_gate;
        a.fsu = (const float*)ew->s_up;
        a.fsd = (const float*)ew->s_down;
    }
    if (d->I_shared > 0) {
        a.swg = sw->w_gate;
        a.swu = sw->w_up;
        a.swd = sw->w_down;
    }

    const int32_t E = d->E;
    const int32_t gend = E + (d->I_shared > 0 ? 1 : 0);
    const bool f32 = d->act_dtype == MOE_F32;
    const bool quant = d->expert_dtype == MOE_Q4G64 || d->expert_dtype == MOE_FP8;
    TilePlan tp{false, 128, 128, 0, STREAM_MAX_ROWS};
    if (!f32) {
        const int ts = tiled_state();
        if (ts != 3) tp = plan_tiles(d, ts == 1);
    }
    a.stream_max_rows = tp.on ? tp.min_rows : 0x7fffffff;
    const int32_t rdt = quant ? d->expert_dtype : MOE_BF16;
    const int32_t split = quant ? E : gend;  // tiled: quantised routed groups vs the bf16 (shared) group
    // weight-streaming kernels of one expert-GEMM pass (groups of at most stream_max_rows rows);
    // one launch covers the routed groups and the shared expert, which streams its bf16 weights
    // also in quantised layers
    auto streamed = [&](bool first) -> int {
        if (f32) return hip_rc(first ? launch_gemm1_f32(a, s) : launch_gemm2_f32(a, s));
        if (tp.on && tp.min_rows == 0) return MOE_OK;  // every group is tiled
        if (!quant && use_stream_dma(a)) return hip_rc(launch_stream_dma(a, first, 0, gend, s));
        if (rdt == MOE_FP8 && use_stream_f8(a)) return hip_rc(launch_stream_f8(a, first, 0, gend, s));
        return hip_rc(first ? launch_gemm1_bf16(a, 0, gend, rdt, s) : launch_gemm2_bf16(a, 0, gend, rdt, s));
    };
    // tiled kernels of one pass (the other groups)
    auto tiled = [&](bool first) -> int {
        if (!tp.on) return MOE_OK;
        int r = hip_rc(launch_gemm_tiled(a, first, tp.BM, 0, split, rdt, tile_count, tile_info, tp.max_tiles, s));
        if (!r && split < gend)
            r = hip_rc(launch_gemm_tiled(a, first, tp.BMs, split, gend, MOE_BF16, tile_count, tile_info,
                                         tp.max_tiles, s));
        return r;
    };
    if (tp.on && (rc = hip_rc(launch_tiles(a, tp.BM, tp.BMs, tp.min_rows, tile_count, tile_info, s)))) return rc;
    // With tiles on, the GEMM1 / GEMM2 stage events bracket the tiled kernels only (the
    // dominant kernels of prefill layers); the streaming kernels run right before them.
    for (int pass = 0; pass < 2; ++pass) {
        const bool first = pass == 0;
        const int32_t stage = first ? MOE_STAGE_GEMM1 : MOE_STAGE_GEMM2;
        if (!tp.on && (rc = hip_rc(mark(stage, 0, s)))) return rc;
        if ((rc = streamed(first))) return rc;
        if (tp.on && (rc = hip_rc(mark(stage, 0, s)))) return rc;
        if ((rc = tiled(first))) return rc;
        if ((rc = hip_rc(mark(stage, 1, s)))) return rc;
    }
    if ((rc = hip_rc(mark(MOE_STAGE_COMBINE, 0, s)))) return rc;
    if (sgl && (rc = hip_rc(launch_router(x, sw->w_sgate, d->act_dtype, d->T, d->H, 1, nullptr, sgl, s))))
        return rc;
    if ((rc = hip_rc(launch_combine(a, d->act_dtype, scores, slot_row, sgl, y, s)))) return rc;
    if ((rc = hip_rc(mark(MOE_STAGE_COMBINE, 1, s)))) return rc;
    return MOE_OK;
}

// Scratch of moe_forward_static: one array per device, allocated by the runtime when the library's
// code object is loaded on that device and held until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device memory: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address
// is ever passed to kernels.
__device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

void* g_scratch_ptr[MAX_DEVICES];
hipError_t g_scratch_err[MAX_DEVICES];
std::once_flag g_scratch_once[MAX_DEVICES];

// device address of the current device's scratch array (MOE_ERR_HIP if it cannot be had)
int static_scratch(void** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MOE_ERR_HIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
        (void)hipGetLastError();
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return MOE_ERR_HIP;
    *ptr = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_dense_workspace_size(int64_t T, int32_t H, int32_t I, int32_t act_dtype) {
    if (check_dense(T, H, I, act_dtype) != MOE_OK) return 0;
    return dense_layout(T, I, act_dtype).total;
}

int moe_dense_mlp(int64_t T, int32_t H, int32_t I, int32_t act_dtype, const void* x, const void* w_gate,
                  const void* w_up, const void* w_down, void* y, void* workspace, size_t workspace_bytes,
                  void* stream) {
    int rc = check_dense(T, H, I, act_dtype);
    if (rc != MOE_OK) return rc;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr_ok(y, empty) || !ptr_ok(w_gate, false) || !ptr_ok(w_up, false) ||
        !ptr_ok(w_down, false))
        return MOE_ERR_INVALID;
    const DenseLayout L = dense_layout(T, I, act_dtype);
    if (!ptr_ok(workspace, false) || ((uintptr_t)workspace & (ALIGN - 1))) return MOE_ERR_INVALID;
    if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (empty) return MOE_OK;

    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    GroupedArgs a;
    memset(&a, 0, sizeof(a));
    a.T = T;
    a.H = H;
    a.E = 0;
    a.I = 0;
    a.Is = I;
    a.K = 0;
    a.TK = 0;
    a.ldh = I;
    a.x = x;
    a.h = ws + L.h;
    a.o = y;  // row TK + t of the expert-output space is token t: the down projection writes y
    a.swg = w_gate;
    a.swu = w_up;
    a.swd = w_down;
    if (act_dtype == MOE_F32) {
        if ((rc = hip_rc(launch_gemm1_f32(a, s)))) return rc;
        return hip_rc(launch_gemm2_f32(a, s));
    }
    const int ts = tiled_state();
    const int64_t lim = (int64_t)1 << 31;
    const bool tiled = ts != 3 && T > STREAM_MAX_ROWS && T * (int64_t)H < lim && T * (int64_t)I < lim &&
                       (int64_t)I * H < lim;
    a.stream_max_rows = tiled ? STREAM_MAX_ROWS : 0x7fffffff;
    if (!tiled) {
        if (use_stream_dma(a)) {
            if ((rc = hip_rc(launch_stream_dma(a, true, 0, 1, s)))) return rc;
            return hip_rc(launch_stream_dma(a, false, 0, 1, s));
        }
        if ((rc = hip_rc(launch_gemm1_bf16(a, 0, 1, MOE_BF16, s)))) return rc;
        return hip_rc(launch_gemm2_bf16(a, 0, 1, MOE_BF16, s));
    }
    const int32_t BM = dense_bm(T, ts == 1);
    const int32_t max_tiles = tiled_max_tiles(T, 0, 0, BM);
    int32_t* tile_count = (int32_t*)(ws + L.tiles);
    int32_t* tile_info = tile_count + 64;
    if ((rc = hip_rc(launch_tiles(a, BM, BM, STREAM_MAX_ROWS, tile_count, tile_info, s)))) return rc;
    if ((rc = hip_rc(launch_gemm_tiled(a, true, BM, 0, 1, MOE_BF16, tile_count, tile_info, max_tiles, s))))
        return rc;
    return hip_rc(launch_gemm_tiled(a, false, BM, 0, 1, MOE_BF16, tile_count, tile_info, max_tiles, s));
}

int moe_set_stage_events(int32_t stage, void* const* events, int32_t n_pairs) {
    return g_hook.set(stage, events, n_pairs, MOE_STAGE_COMBINE) ? MOE_OK : MOE_ERR_INVALID;
}

const char* moe_strerror(int code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID: return "invalid argument";
        case MOE_ERR_HIP: return "HIP launch or runtime error";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_UNSUPPORTED: return "valid but unsupported by this implementation";
        default: return "unknown error code";
    }
}

int moe_router_logits(const void* x, const void* router_w, int32_t act_dtype, int64_t T, int32_t H, int32_t E,
                      const float* logit_offset, float* logits, void* stream) {
    if (T < 0 || H < 1 || E < 1) return MOE_ERR_INVALID;
    if (act_dtype != MOE_F32 && act_dtype != MOE_BF16) return MOE_ERR_INVALID;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr_ok(router_w, false) || !ptr_ok(logits, empty) || !ptr_ok(logit_offset, true))
        return MOE_ERR_INVALID;
    if (empty) return MOE_OK;
    return hip_rc(launch_router(x, router_w, act_dtype, T, H, E, logit_offset, logits, (hipStream_t)stream));
}

int moe_route_softmax(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t* inds, float* scores,
                      void* stream) {
    if (T < 0 || E < 1 || top_k < 1 || top_k > E) return MOE_ERR_INVALID;
    const bool empty = T == 0;
    if (!ptr_ok(logits, empty) || !ptr_ok(inds, empty) || !ptr_ok(scores, empty)) return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
    if (empty) return MOE_OK;
    return hip_rc(launch_route_softmax(logits, T, E, top_k, inds, scores, (hipStream_t)stream));
}

int moe_route_deepseek(const float* logits, int64_t T, int32_t E, const float* bias, int64_t bias_len,
                       const moe_route_params* p, int32_t* inds, float* scores, void* stream) {
    if (T < 0) return MOE_ERR_INVALID;
    const bool empty = T == 0;
    if (!ptr_ok(logits, empty) || !ptr_ok(bias, false) || !ptr_ok(inds, empty) || !ptr_ok(scores, empty))
        return MOE_ERR_INVALID;
    if (bias_len != E) return MOE_ERR_INVALID;
    const int rc = check_route_params(E, p);
    if (rc != MOE_OK) return rc;
    if (empty) return MOE_OK;
    return hip_rc(launch_route(logits, T, E, bias, *p, inds, scores, (hipStream_t)stream));
}

size_t moe_dispatch_workspace_size(int64_t T, int32_t K, int32_t E) {
    if (T < 0 || K < 1 || E < 1 || E > MOE_MAX_EXPERTS || T * K >= ((int64_t)1 << 31)) return 0;
    return dispatch_ws_bytes(T, K, E);
}

int moe_dispatch(const int32_t* inds, int64_t T, int32_t K, int32_t E, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_slot, int32_t* slot_row, void* workspace, size_t workspace_bytes, void* stream) {
    if (T < 0 || K < 1 || E < 1) return MOE_ERR_INVALID;
    const bool empty = T == 0;
    if (!ptr_ok(inds, empty) || !ptr_ok(counts, false) || !ptr_ok(offsets, false) || !ptr_ok(sorted_slot, empty) ||
        !ptr_ok(slot_row, empty))
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || T * K >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    const size_t need = dispatch_ws_bytes(T, K, E);
    if (need > 0 && !ptr_ok(workspace, false)) return MOE_ERR_INVALID;
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
    return hip_rc(launch_dispatch(inds, T, K, E, counts, offsets, sorted_slot, slot_row, (int32_t*)workspace,
                                  (hipStream_t)stream));
}

int moe_forward_static(const moe_layer_desc* d, const void* x, const void* router_w, const float* bias,
                       const float* logit_offset, const moe_expert_weights* ew, const moe_shared_weights* sw, void* y,
                       int32_t* inds_out, float* scores_out, void* stream) {
    int rc = check_forward(d, x, router_w, bias, logit_offset, ew, sw, y, inds_out, scores_out);
    if (rc != MOE_OK) return rc;
    const FwdLayout L = fwd_layout(d);
    if (L.total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    if (d->T == 0) return MOE_OK;
    void* ws = nullptr;
    if ((rc = static_scratch(&ws)) != MOE_OK) return rc;
    return launch_forward(d, x, router_w, bias, logit_offset, ew, sw, y, inds_out, scores_out, (char*)ws, L, stream);
}

size_t moe_forward_workspace_size(const moe_layer_desc* d) {
    if (check_desc(d) != MOE_OK) return 0;
    return fwd_layout(d).total;
}

int moe_forward(const moe_layer_desc* d, const void* x, const void* router_w, const float* bias,
                const float* logit_offset, const moe_expert_weights* ew, const moe_shared_weights* sw, void* y,
                int32_t* inds_out, float* scores_out, void* workspace, size_t workspace_bytes, void* stream) {
    const int rc = check_forward(d, x, router_w, bias, logit_offset, ew, sw, y, inds_out, scores_out);
    if (rc != MOE_OK) return rc;
    const FwdLayout L = fwd_layout(d);
    if (!ptr_ok(workspace, false) || ((uintptr_t)workspace & (ALIGN - 1))) return MOE_ERR_INVALID;
    if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (d->T == 0) return MOE_OK;
    return launch_forward(d, x, router_w, bias, logit_offset, ew, sw, y, inds_out, scores_out, (char*)workspace, L,
                          stream);
}

}  // extern "C"
