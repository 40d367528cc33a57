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
    (8192, 7168, 256, "bf16"),   # 4x4 register tiles
    (37, 200, 96, "f32"),        # ragged everywhere, partial k chunk
    (2049, 96, 1000, "bf16"),    # many experts, ragged tiles
    (1, 7168, 256, "bf16"),
    (2048, 7168, 256, "bf16"),   # 2x4 register tiles, 64-k chunks
    (2500, 136, 256, "f32"),     # 2x4, partial last chunk
    (1000, 7168, 256, "bf16"),   # 2x2 register tiles, ragged tokens
    (700, 200, 96, "f32"),       # 2x2, partial last chunk, ragged experts
    (3000, 7168, 1, "bf16"),     # one expert (the shared-expert gate): GEMV at many tokens
    (37, 7168, 256, "bf16"),     # GEMV, ragged token block: row touching clamped to the block's rows
    (300, 520, 64, "bf16"),      # GEMV, short rows: every touching lane past a row's end clamped
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
