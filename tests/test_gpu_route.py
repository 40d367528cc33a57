"""GPU parity of the route kernel (moe_route_deepseek) against the oracle.

Page: "feat(engine): E1 DeepSeek-style MoE gate (sigmoid, group top-k, bias) (#108)".
Indices must be bit-exact; weights within relative 1e-6 (the kernel reproduces the oracle's
fp32 operation sequence, so they are expected to be bit-identical too, which is checked
separately).  Shapes cover every lane layout of the kernel (P = 1..16 experts per lane), both
group paths (DPP lane segments and the LDS path), ragged token counts, ties, saturated
sigmoids, signed zeros, masked-zero selection, and the five workload shapes.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import deepseek_gate_expert_amd as dg
from _gpu import DEV, log

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def run_gpu(logits: np.ndarray, bias: np.ndarray, K, G, TG, norm, rsf):
    T = logits.shape[0]
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(DEV)
    b = torch.from_numpy(np.ascontiguousarray(bias, np.float32)).to(DEV)
    inds = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    scores = torch.full((T, K), -7.0, dtype=torch.float32, device=DEV)
    rc = dg.moe_route_deepseek(lg, b, inds, scores, K, G, TG, norm, rsf)
    torch.cuda.synchronize()
    return rc, inds.cpu().numpy(), scores.cpu().numpy()


def check(logits, bias, K, G, TG, norm=True, rsf=2.5, label=""):
    log(f"[route] {label} T={logits.shape[0]} E={logits.shape[1]} K={K} G={G} TG={TG}")
    rc, gi, gs = run_gpu(logits, bias, K, G, TG, norm, rsf)
    assert rc == 0, dg.moe_strerror(rc)
    orc, oi, os_ = oracle.route(logits, bias, oracle.params(K, G, TG, norm, rsf))
    assert orc == 0
    bad = np.nonzero(np.any(gi != oi, axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} rows differ, first {bad[:3]}: gpu {gi[bad[0]]} oracle {oi[bad[0]]}"
    den = np.maximum(np.abs(os_.astype(np.float64)), 1e-30)
    assert np.max(np.abs(gs.astype(np.float64) - os_) / den) <= 1e-6
    return gi, gs, oi, os_


SHAPES = [
    # T,    E,    K,  G,  TG, logit_std
    (16, 8, 2, 1, 1, 1.0),        # tiny fp32 layer's gate
    (512, 64, 6, 4, 2, 1.0),      # group-routing stress
    (64, 256, 8, 8, 4, 1.0),      # DeepSeek-V3 decode
    (8192, 256, 8, 8, 4, 1.0),    # DeepSeek-V3 prefill
    (37, 256, 8, 8, 4, 3.0),      # ragged token count, wide logits
    (5, 8, 3, 4, 2, 1.0),         # two experts per group
    (33, 96, 5, 4, 2, 1.0),       # groups of 24 experts: LDS group path
    (19, 1000, 7, 8, 3, 1.0),     # 125-expert groups, 16 experts per lane: LDS group path
    (11, 1024, 16, 8, 4, 1.0),    # 16 experts per lane, lane-segment groups
    (9, 128, 1, 4, 1, 1.0),       # top_k = 1
    (9, 48, 48, 1, 1, 1.0),       # top_k = E
    (13, 64, 40, 8, 2, 1.0),      # top_k above kept experts: masked zeros selected
    (21, 200, 6, 1, 1, 1.0),      # E not a multiple of 64, no groups
    (7, 64, 64, 2, 1, 1.0),       # top_k = 64 (limit)
]


@pytest.mark.parametrize("T,E,K,G,TG,std", SHAPES, ids=[f"T{s[0]}E{s[1]}K{s[2]}G{s[3]}TG{s[4]}" for s in SHAPES])
def test_route_matches_oracle(T, E, K, G, TG, std):
    seed = T * 7919 + E * 31 + K
    logits = synth.normal_f32(seed, 1, T * E, std).reshape(T, E)
    bias = synth.normal_f32(seed, 3, E, 0.3)
    check(logits, bias, K, G, TG, True, 2.5, "random")
    check(logits, bias, K, G, TG, False, 1.0, "random-nonorm")


def test_route_scores_bit_identical():
    logits = synth.normal_f32(5, 1, 8192 * 256, 1.0).reshape(8192, 256)
    bias = synth.normal_f32(5, 3, 256, 0.1)
    gi, gs, oi, os_ = check(logits, bias, 8, 8, 4, True, 2.5, "bitwise")
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32))


def test_route_D7_no_drop_equals_single_group():
    logits = synth.normal_f32(6, 1, 300 * 256, 1.0).reshape(300, 256)
    bias = synth.normal_f32(6, 3, 256, 0.2)
    _, a_s, _, _ = check(logits, bias, 8, 8, 8, True, 2.5, "TG=G")
    rc, bi, b_s = run_gpu(logits, bias, 8, 1, 1, True, 2.5)
    rc2, ai, _ = run_gpu(logits, bias, 8, 8, 8, True, 2.5)
    assert np.array_equal(ai, bi) and np.array_equal(a_s, b_s)


def test_route_ties_and_saturation():
    T, E = 64, 256
    rng = np.random.default_rng(0)
    base = rng.choice(np.array([0.0, -0.0, 100.0, -100.0, 30.0, -30.0, 1.5], np.float32), size=(T, E))
    check(base.astype(np.float32), np.zeros(E, np.float32), 8, 8, 4, True, 2.5, "ties")
    check(np.zeros((T, E), np.float32), np.zeros(E, np.float32), 8, 8, 4, True, 2.5, "all-equal")
    check(base.astype(np.float32), rng.choice(np.array([0, 0.5], np.float32), size=E), 8, 8, 4, True, 2.5, "ties+bias")


def test_route_planted_rows():
    w = synth.WORKLOADS["c1"]
    bias = synth.gen_bias(w)
    z = synth.planted_logits(w, bias, 256)
    gi, *_ = check(z, bias, w.K, w.G, w.TG, True, w.rsf, "planted")
    astar = int(np.argmax(bias))
    assert not np.any(gi == astar)


def test_route_golden_cases():
    cases = json.load(open(os.path.join(HERE, "golden", "gate_cases.json")))["cases"]
    for c in cases:
        rc, gi, gs = run_gpu(np.array([c["logits"]], np.float32), np.array(c["bias"], np.float32), c["top_k"],
                             c["n_group"], c["topk_group"], c["norm"], c["rsf"])
        assert rc == 0
        assert gi[0].tolist() == c["expect_inds"], c["name"]
        assert gs[0].tolist() == [float(np.float32(v)) for v in c["expect_scores"]], c["name"]


def test_route_deterministic():
    logits = synth.normal_f32(8, 1, 4096 * 256, 1.0).reshape(4096, 256)
    bias = synth.normal_f32(8, 3, 256, 0.1)
    a = run_gpu(logits, bias, 8, 8, 4, True, 2.5)
    b = run_gpu(logits, bias, 8, 8, 4, True, 2.5)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))


def test_route_leading_dims_flatten():
    lg3 = synth.normal_f32(9, 1, 2 * 5 * 64, 1.0).reshape(2, 5, 64)
    bias = synth.normal_f32(9, 3, 64, 0.3)
    lg = torch.from_numpy(lg3).to(DEV)
    b = torch.from_numpy(bias).to(DEV)
    inds = torch.empty((2, 5, 6), dtype=torch.int32, device=DEV)
    scores = torch.empty((2, 5, 6), dtype=torch.float32, device=DEV)
    assert dg.moe_route_deepseek(lg, b, inds, scores, 6, 4, 2, True, 2.5) == 0
    torch.cuda.synchronize()
    _, oi, os_ = oracle.route(lg3.reshape(10, 64), bias, oracle.params(6, 4, 2, True, 2.5))
    assert np.array_equal(inds.cpu().numpy().reshape(10, 6), oi)
    assert np.array_equal(scores.cpu().numpy().reshape(10, 6), os_)


def test_route_rejects_leave_outputs_untouched():
    lg = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
    inds = torch.full((4, 2), -7, dtype=torch.int32, device=DEV)
    scores = torch.full((4, 2), -7.0, dtype=torch.float32, device=DEV)
    bad_bias = [
        torch.zeros((1, 8), dtype=torch.float32, device=DEV),   # rank 2
        torch.zeros((7,), dtype=torch.float32, device=DEV),     # length != E
        torch.zeros((8,), dtype=torch.float64, device=DEV),     # dtype
        torch.zeros((8,), dtype=torch.float32),                 # host tensor
    ]
    for b in bad_bias:
        assert dg.moe_route_deepseek(lg, b, inds, scores, 2) == dg.MOE_ERR_INVALID
    good = torch.zeros((8,), dtype=torch.float32, device=DEV)
    assert dg.moe_route_deepseek(lg, good, inds, scores, 0) == dg.MOE_ERR_INVALID
    assert dg.moe_route_deepseek(lg, good, inds, scores, 2, 2, 3) == dg.MOE_ERR_INVALID
    torch.cuda.synchronize()
    assert bool((inds == -7).all()) and bool((scores == -7.0).all())


# ---- softmax gate (moe_route_softmax) --------------------------------------------------------

def run_gpu_softmax(logits: np.ndarray, K):
    T = logits.shape[0]
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(DEV)
    inds = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    scores = torch.full((T, K), -7.0, dtype=torch.float32, device=DEV)
    rc = dg.moe_route_softmax(lg, inds, scores, K)
    torch.cuda.synchronize()
    return rc, inds.cpu().numpy(), scores.cpu().numpy()


SOFTMAX_SHAPES = [
    # T,   E,    K,  logit_std
    (16, 8, 2, 1.0),
    (512, 64, 6, 1.0),
    (64, 256, 8, 1.0),
    (4096, 256, 8, 2.0),
    (37, 200, 5, 3.0),     # E not a multiple of 64
    (19, 1000, 7, 1.0),    # 16 experts per lane
    (9, 128, 1, 1.0),      # top_k = 1: weights exactly 1
    (9, 48, 48, 1.0),      # top_k = E
    (7, 64, 64, 0.5),      # top_k = 64 (limit)
    (3, 1, 1, 1.0),        # a single expert
]


@pytest.mark.parametrize("T,E,K,std", SOFTMAX_SHAPES, ids=[f"T{s[0]}E{s[1]}K{s[2]}" for s in SOFTMAX_SHAPES])
def test_route_softmax_matches_oracle(T, E, K, std):
    log(f"[route-softmax] T={T} E={E} K={K}")
    seed = T * 7919 + E * 31 + K + 17
    logits = synth.normal_f32(seed, 1, T * E, std).reshape(T, E)
    rc, gi, gs = run_gpu_softmax(logits, K)
    assert rc == 0, dg.moe_strerror(rc)
    orc, oi, os_ = oracle.route_softmax(logits, K)
    assert orc == 0
    assert np.array_equal(gi, oi)
    den = np.maximum(np.abs(os_.astype(np.float64)), 1e-30)
    assert np.max(np.abs(gs.astype(np.float64) - os_) / den) <= 1e-6
    if K == 1:
        assert np.all(gs == 1.0)


def test_route_softmax_ties_and_large_logits():
    # equal logits: the lowest indices win and the weights are exactly 1/K; a row shifted by 1000
    # (exp(l - max) never overflows) and a row with one dominant logit
    E, K = 64, 4
    lg = np.zeros((3, E), np.float32)
    lg[0, :] = 2.5
    lg[1, :] = 1000.0 + synth.normal_f32(3, 1, E, 1.0)
    lg[2, :] = -5.0
    lg[2, 17] = 80.0
    rc, gi, gs = run_gpu_softmax(lg, K)
    assert rc == 0
    orc, oi, os_ = oracle.route_softmax(lg, K)
    assert np.array_equal(gi, oi)
    assert list(gi[0]) == [0, 1, 2, 3] and np.all(gs[0] == 0.25)
    assert gi[2, 0] == 17 and np.all(np.isfinite(gs))
    np.testing.assert_allclose(gs, os_, rtol=1e-6, atol=0)


def test_route_softmax_rejects_leave_outputs_untouched():
    lg = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
    inds = torch.full((4, 2), -7, dtype=torch.int32, device=DEV)
    scores = torch.full((4, 2), -7.0, dtype=torch.float32, device=DEV)
    assert dg.moe_route_softmax(lg, inds, scores, 0) == dg.MOE_ERR_INVALID
    assert dg.moe_route_softmax(lg, inds, scores, 9) == dg.MOE_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.all(inds == -7) and torch.all(scores == -7.0)
