"""Pins of the oracle's dense SwiGLU MLP layer (CPU only).

Page: "Epic: Engine Inference Core Stage E - MoE + hybrid families", "Decision 5 superseded"
item 2 (DeepSeek mixes dense and MoE layers).  A dense layer is the shared expert's SwiGLU on its
own.  Pins: torch fp64 matmuls (different code), zero input, and the MoE layer with every routed
down projection set to zero, whose output is then exactly its shared expert's.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle_layer import _f64


def _weights(seed, H, I, act):
    gen = synth.normal_bf16 if act == "bf16" else synth.normal_f32
    return (gen(seed, 7, I * H, 1 / np.sqrt(H)).reshape(I, H), gen(seed, 8, I * H, 1 / np.sqrt(H)).reshape(I, H),
            gen(seed, 9, H * I, 1 / np.sqrt(I)).reshape(H, I))


@pytest.mark.parametrize("T,H,I,act", [(5, 64, 32, "f32"), (9, 128, 192, "bf16"), (1, 40, 24, "f32")])
def test_dense_against_torch(T, H, I, act):
    gen = synth.normal_bf16 if act == "bf16" else synth.normal_f32
    x = gen(T + H, 1, T * H, 1.0).reshape(T, H)
    wg, wu, wd = _weights(T + I, H, I, act)
    y = oracle.dense_mlp(x, wg, wu, wd, act)
    X, G, U, D = (_f64(a, act) for a in (x, wg, wu, wd))
    ref = ((torch.nn.functional.silu(X @ G.T) * (X @ U.T)) @ D.T).numpy()
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_dense_zero_input():
    wg, wu, wd = _weights(1, 64, 32, "f32")
    y = oracle.dense_mlp(np.zeros((3, 64), np.float32), wg, wu, wd, "f32")
    assert np.all(y == 0.0)


def test_dense_equals_a_moe_layer_with_silent_routed_experts():
    w = synth.WORKLOADS["c1"].with_(T=10, H=128, I=64, Is=96, planted=0)
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    ex = synth.gen_expert_weights(w)
    ex["down"] = np.zeros_like(ex["down"])
    sh = synth.gen_shared(w)
    y, *_ = oracle.forward_workload(w, x, r, b, ex, sh)
    yd = oracle.dense_mlp(x, sh["gate"], sh["up"], sh["down"], w.act)
    assert np.array_equal(y, yd)
