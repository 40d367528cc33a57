"""Pins of the oracle's fp8 expert weights (CPU only).

Page: "Epic: Engine Inference Core Stage E - MoE + hybrid families", weight loading (fp8
checkpoints are dequantised when loaded).  Reading taken where the page stops: codes are OCP
E4M3 ("FN": bias 7, no infinities, NaN at S.1111.111, largest finite 448) and every 128 x 128
block of an [out, in] matrix carries one fp32 scale; the weight is code value x block scale,
exact.

Pins: the decode of all 256 codes against PyTorch's float8_e4m3fn dtype (a library routine);
closed forms of the format's landmarks; the layer against a dense fp64 brute force whose
weights are decoded by PyTorch and scaled by blocks expanded with numpy (block grids that are
not square, so a transposed block index fails); the quantiser's round trip within half an
E4M3 step.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle_layer import _f64


def test_decode_matches_library_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(lib)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])
    # signed zero is kept
    assert math.copysign(1.0, mine[0x80]) == -1.0 and math.copysign(1.0, mine[0x00]) == 1.0


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x7E, 448.0), (0xFE, -448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x08, 2.0 ** -6), (0x40, 2.0), (0xC0, -2.0), (0x3C, 1.5), (0x77, 240.0), (0x30, 0.5),
])
def test_decode_landmarks(code, value):
    assert oracle.e4m3([code])[0] == value


def _blocks(s, rows, cols):
    """Expand [.., ceil(rows/128), ceil(cols/128)] block scales to [.., rows, cols]."""
    return np.repeat(np.repeat(s, 128, axis=-2), 128, axis=-1)[..., :rows, :cols].astype(np.float64)


def _dequant_torch(ex, nm, rows, cols):
    dec = torch.from_numpy(np.ascontiguousarray(ex[nm])).view(torch.float8_e4m3fn).double().numpy()
    return dec * _blocks(ex["s_" + nm], rows, cols)


def test_quantiser_round_trip_within_half_a_step():
    nmat, rows, cols, std = 2, 200, 320, 0.05
    q, s = synth.fp8_normal(7, 5, nmat, rows, cols, std)
    w = synth.normal_f32(7, 5, nmat * rows * cols, std).reshape(nmat, rows, cols).astype(np.float64)
    d = _dequant_torch({"w": q, "s_w": s}, "w", rows, cols)
    sc = _blocks(s, rows, cols)
    # E4M3 spacing at |v| in [2^E, 2^(E+1)) is 2^(E-3), subnormal spacing 2^-9; half of it is
    # the rounding bound, plus the fp32 rounding of w / scale
    v = np.abs(w) / sc
    E = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    half = 0.5 * 2.0 ** (E - 3) * sc
    assert np.all(np.abs(w - d) <= half * (1 + 1e-6) + 1e-30)
    # every block's largest magnitude maps to 448 (the scale is max |w| / 448)
    mag = q.astype(np.int32) & 0x7F
    for m in range(nmat):
        for r0 in range(0, rows, 128):
            for c0 in range(0, cols, 128):
                assert mag[m, r0:r0 + 128, c0:c0 + 128].max() == 0x7E


LAYERS = [
    synth.WORKLOADS["c4"].with_(name="fp8-tiny", expert="fp8", T=10, H=384, I=128, Is=64, E=16, G=4, TG=2, K=4),
    synth.WORKLOADS["c1"].with_(name="fp8-ragged", expert="fp8", T=12, H=192, I=320, Is=0, E=8, G=4, TG=2, K=3,
                                planted=0),
]


@pytest.mark.parametrize("w", LAYERS, ids=[w.name for w in LAYERS])
def test_layer_against_dense_brute_force(w):
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    ex, sh = synth.gen_expert_weights(w), synth.gen_shared(w)
    y, inds, scores, _ = oracle.forward_workload(w, x, r, b, ex, sh)
    X = _f64(x, w.act)
    Wg = torch.from_numpy(_dequant_torch(ex, "gate", w.I, w.H))
    Wu = torch.from_numpy(_dequant_torch(ex, "up", w.I, w.H))
    Wd = torch.from_numpy(_dequant_torch(ex, "down", w.H, w.I))
    h = torch.nn.functional.silu(torch.einsum("th,eih->eti", X, Wg)) * torch.einsum("th,eih->eti", X, Wu)
    o = torch.einsum("eti,ehi->eth", h, Wd)
    M = torch.zeros(w.T, w.E, dtype=torch.float64)
    for t in range(w.T):
        for j in range(w.K):
            M[t, int(inds[t, j])] += float(scores[t, j])
    ref = torch.einsum("te,eth->th", M, o)
    if sh is not None:
        Sg, Su, Sd = _f64(sh["gate"], w.act), _f64(sh["up"], w.act), _f64(sh["down"], w.act)
        ref = ref + (torch.nn.functional.silu(X @ Sg.T) * (X @ Su.T)) @ Sd.T
    ref = ref.numpy()
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    # routing does not depend on the expert dtype
    _, i2, s2, _ = oracle.forward_workload(w.with_(expert="bf16"), x, r, b, synth.gen_expert_weights(
        w.with_(expert="bf16")), sh)
    assert np.array_equal(inds, i2) and np.array_equal(scores, s2)


def test_a_wrong_block_index_would_be_seen():
    """Planted mistake on the CPU side only: transposing the block grid of the gate scales
    changes the layer output, so the brute-force pin above discriminates it."""
    w = LAYERS[0]
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    ex, sh = synth.gen_expert_weights(w), synth.gen_shared(w)
    y, *_ = oracle.forward_workload(w, x, r, b, ex, sh)
    bad = dict(ex)
    sgt = ex["s_gate"]  # [E, 1, 3]
    bad["s_gate"] = np.ascontiguousarray(np.roll(sgt, 1, axis=2))
    y2, *_ = oracle.forward_workload(w, x, r, b, bad, sh)
    assert np.max(np.abs(y - y2)) > 1e-3 * np.max(np.abs(y))


def test_rejects_missing_scales():
    w = LAYERS[0]
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    ex = dict(synth.gen_expert_weights(w))
    ex["s_up"] = None
    with pytest.raises(ValueError):
        oracle.forward_workload(w, x, r, b, ex, synth.gen_shared(w))
