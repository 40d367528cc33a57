"""GPU parity of the dense SwiGLU MLP layer (moe_dense_mlp) against the oracle.

Page: "Epic: Engine Inference Core Stage E - MoE + hybrid families", "Decision 5 superseded"
item 2 (dense/MoE layer mixing).  Tolerances as for the MoE layer (relative L2 1e-5 fp32,
1e-2 bf16).  Shapes straddle the weight-streaming / tiled boundary (T = 64 / 65), both tile
heights, 64-wide tails of the reduction, and a DeepSeek-V3 dense layer (H 7168, I 18432) checked
on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import deepseek_gate_expert_amd as dg
from deepseek_gate_expert_amd.tensors import to_device
from _gpu import DEV, act_to_f64, log, rel_l2

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


def _case(T, H, I, act, seed=0):
    gen = synth.normal_bf16 if act == "bf16" else synth.normal_f32
    x = gen(seed + T + H, 1, T * H, 1.0).reshape(T, H)
    wg = gen(seed + I, 7, I * H, 1 / np.sqrt(H)).reshape(I, H)
    wu = gen(seed + I, 8, I * H, 1 / np.sqrt(H)).reshape(I, H)
    wd = gen(seed + I, 9, H * I, 1 / np.sqrt(I)).reshape(H, I)
    return x, wg, wu, wd


def _run(x, wg, wu, wd, act):
    """The workspace and y are filled with 0xFF bytes (NaN) first, so an unwritten row shows up."""
    dt = torch.bfloat16 if act == "bf16" else torch.float32
    xd, g, u, d = (to_device(a, DEV) for a in (x, wg, wu, wd))
    T, H = x.shape
    y = torch.empty((T, H), dtype=dt, device=DEV)
    y.view(torch.uint8).fill_(0xFF)
    ws = torch.full((max(1, dg.moe_dense_workspace_size(T, H, wg.shape[0], dg.act_code(dt))),), 0xFF,
                    dtype=torch.uint8, device=DEV)
    rc = dg.moe_dense_mlp(xd, g, u, d, y, ws)
    torch.cuda.synchronize()
    return rc, y


SHAPES = [
    # T,    H,    I,   act
    (1, 128, 64, "bf16"),
    (37, 192, 128, "bf16"),     # 64-wide reduction tail in the gate/up GEMM
    (64, 256, 192, "bf16"),     # last streamed size, tail in the down GEMM
    (65, 256, 192, "bf16"),     # first tiled size (128-row tiles)
    (300, 320, 256, "bf16"),    # ragged tiles and columns
    (2048, 256, 512, "bf16"),   # 256-row tiles
    (21, 40, 24, "f32"),
    (130, 64, 96, "f32"),
]


@pytest.mark.parametrize("T,H,I,act", SHAPES, ids=[f"T{s[0]}H{s[1]}I{s[2]}{s[3]}" for s in SHAPES])
def test_dense_matches_oracle(T, H, I, act):
    log(f"[dense] T={T} H={H} I={I} {act}")
    x, wg, wu, wd = _case(T, H, I, act)
    rc, y = _run(x, wg, wu, wd, act)
    assert rc == 0, dg.moe_strerror(rc)
    ref = oracle.dense_mlp(x, wg, wu, wd, act)
    err = rel_l2(act_to_f64(y), ref)
    log(f"[dense] rel L2 {err:.3e}")
    assert err <= TOL[act]


def test_dense_deepseek_v3_layer_sampled_rows():
    """DeepSeek-V3 dense layer shape (H 7168, I 18432), 512 tokens through 256-row tiles; the
    oracle checks 12 sampled rows."""
    T, H, I = 512, 7168, 18432
    log(f"[dense] DSV3 T={T} H={H} I={I}")
    x, wg, wu, wd = _case(T, H, I, "bf16", seed=11)
    rc, y = _run(x, wg, wu, wd, "bf16")
    assert rc == 0
    rows = np.array([0, 1, 63, 64, 127, 128, 200, 255, 256, 383, 500, 511])
    ref = oracle.dense_mlp(x[rows], wg, wu, wd, "bf16")
    err = rel_l2(act_to_f64(y)[rows], ref)
    log(f"[dense] DSV3 sampled rel L2 {err:.3e}")
    assert err <= TOL["bf16"]


def test_dense_zero_tokens_and_rejects():
    x, wg, wu, wd = _case(4, 128, 64, "bf16")
    g, u, d = (to_device(a, DEV) for a in (wg, wu, wd))
    empty = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    assert dg.moe_dense_mlp(empty, g, u, d, torch.empty_like(empty)) == dg.MOE_OK
    xd = to_device(x, DEV)
    y = torch.full((4, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    assert dg.moe_dense_mlp(xd, g, u, d.t(), y) == dg.MOE_ERR_INVALID        # wrong down shape
    assert dg.moe_dense_mlp(xd, g, u, d, y[:, :64]) == dg.MOE_ERR_INVALID    # wrong output shape
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
