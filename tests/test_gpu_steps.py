"""GPU parity of the router logits (bit-exact, fixed fp32 order) and the dispatch (bit-exact
stable counting sort) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import deepseek_gate_expert_amd as dg
from deepseek_gate_expert_amd.tensors import to_device
from _gpu import DEV, log

pytestmark = pytest.mark.gpu

ROUTER_SHAPES = [
    # T,    H,    E,   act
    (16, 64, 8, "f32"),
    (512, 1024, 64, "bf16"),
    (64, 7168, 256, "bf16"),
    (8192, 7168, 256, "bf16"),   # matrix-core kernel, DeepSeek-V3 prefill shape
    (37, 200, 96, "f32"),        # GEMV, rows not a multiple of 32 (the scalar-load kernel)
    (2049, 96, 1000, "bf16"),    # many experts, ragged token and expert tiles
    (1, 7168, 256, "bf16"),
    (2048, 7168, 256, "bf16"),
    (2500, 136, 256, "f32"),     # fp32 operands, partial last chunk
    (1000, 7168, 256, "bf16"),   # ragged tokens
    (700, 200, 96, "f32"),       # partial last chunk, ragged experts
    (777, 99, 64, "bf16"),       # rows not a multiple of 8: element loads, partial last chunk
    (600, 37, 20, "f32"),        # rows not a multiple of 8, one partial chunk, 20 of 64 experts
    (1030, 24, 48, "bf16"),      # rows shorter than one chunk (only the partial chunk)
    (3000, 7168, 1, "bf16"),     # one expert (the shared-expert gate): GEMV at many tokens
    (37, 7168, 256, "bf16"),     # GEMV, ragged token block: row touching clamped to the block's rows
    (300, 520, 64, "bf16"),      # GEMV, short rows: every touching lane past a row's end clamped
    (100, 16416, 32, "bf16"),    # GEMV with rows too long to stage in LDS (the scalar-load kernel)
]


@pytest.mark.parametrize("T,H,E,act", ROUTER_SHAPES, ids=[f"T{s[0]}H{s[1]}E{s[2]}{s[3]}" for s in ROUTER_SHAPES])
@pytest.mark.parametrize("with_offset", [False, True])
def test_router_logits_bit_exact(T, H, E, act, with_offset):
    log(f"[router] T={T} H={H} E={E} {act} offset={with_offset}")
    gen = synth.normal_f32 if act == "f32" else synth.normal_bf16
    x = gen(T + H, 1, T * H, 1.0).reshape(T, H)
    w = gen(T + H, 2, E * H, 1.0 / np.sqrt(H)).reshape(E, H)
    off = synth.normal_f32(T + H, 10, E, 2.0) if with_offset else None
    ref = oracle.router(x, w, act, off)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    rc = dg.moe_router_logits(to_device(x, DEV), to_device(w, DEV), lg, None if off is None else to_device(off, DEV))
    assert rc == 0
    torch.cuda.synchronize()
    got = lg.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
        f"{np.count_nonzero(got != ref)} logits differ, max abs {np.max(np.abs(got - ref))}"



@pytest.mark.parametrize("T,H,E,act", [(600, 64, 32, "f32"), (40, 64, 32, "f32"), (700, 72, 48, "bf16")])
def test_router_logits_bit_exact_subnormal(T, H, E, act):
    """Products and partial sums in the subnormal range, and exact zeros: the matrix-core router
    (T > 512) and the GEMV (T <= 512) keep the fused multiply-add chain bit for bit there too."""
    log(f"[router-subnormal] T={T} H={H} E={E} {act}")
    def gen(tid, n):
        if act == "f32":
            return synth.normal_f32(T + H + 7, tid, n, 1.0)
        return (synth.normal_bf16(T + H + 7, tid, n, 1.0).astype(np.uint32) << 16).view(np.float32)
    x = gen(1, T * H).reshape(T, H)
    w = gen(2, E * H).reshape(E, H)
    x *= np.float32(2.0 ** -70)   # products near 2^-140: below the normal range (2^-126)
    w *= np.float32(2.0 ** -70)
    x[:, ::5] = 0.0               # exact zeros, and rows of zeros
    w[::7, :] = 0.0
    if act == "bf16":             # scaled by powers of two, so still bf16 values
        x = x.view(np.uint32)
        w = w.view(np.uint32)
        assert not (x & 0xFFFF).any() and not (w & 0xFFFF).any()
        x = (x >> 16).astype(np.uint16)
        w = (w >> 16).astype(np.uint16)
    ref = oracle.router(x, w, act, None)
    assert np.any((ref != 0) & (np.abs(ref) < np.float32(2.0 ** -126))), "no subnormal logits in the case"
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    assert dg.moe_router_logits(to_device(x, DEV), to_device(w, DEV), lg, None) == 0
    torch.cuda.synchronize()
    got = lg.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{np.count_nonzero(got != ref)} logits differ"

DISPATCH = [
    # T,    K,  E,   distribution
    (1, 1, 8, "uniform"),
    (16, 2, 8, "uniform"),
    (64, 8, 256, "uniform"),
    (8192, 8, 256, "zipf"),
    (4096, 8, 256, "uniform"),
    (777, 6, 64, "zipf"),      # T*K not a multiple of the workgroup size
    (300, 3, 1024, "uniform"),
    (1000, 4, 5, "one-hot"),   # almost every slot to one expert
]


@pytest.mark.parametrize("T,K,E,dist", DISPATCH, ids=[f"T{d[0]}K{d[1]}E{d[2]}{d[3]}" for d in DISPATCH])
def test_dispatch_matches_stable_sort(T, K, E, dist):
    log(f"[dispatch] T={T} K={K} E={E} {dist}")
    u = synth.uniform(T * K + E, 12, T * K)
    if dist == "uniform":
        inds = (u * E).astype(np.int32)
    elif dist == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        cdf = np.cumsum(p) / p.sum()
        inds = np.searchsorted(cdf, u).astype(np.int32)
    else:
        inds = np.where(u < 0.97, 3, (u * E).astype(np.int32) % E).astype(np.int32)
    inds = np.minimum(inds, E - 1).reshape(T, K)
    want = oracle.dispatch(inds, E)
    ws = torch.empty(max(1, dg.moe_dispatch_workspace_size(T, K, E)), dtype=torch.uint8, device=DEV)
    outs = [torch.full((n,), -5, dtype=torch.int32, device=DEV) for n in (E, E + 1, T * K, T * K)]
    rc = dg.moe_dispatch(to_device(inds, DEV), E, *outs, ws)
    assert rc == 0
    torch.cuda.synchronize()
    for name, got, ref in zip(("counts", "offsets", "sorted_slot", "slot_row"), outs, want):
        assert np.array_equal(got.cpu().numpy(), ref), name
