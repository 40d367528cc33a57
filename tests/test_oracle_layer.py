"""Pins of the oracle's whole-layer forward (CPU only).

Pages: "Epic: Engine Inference Core Stage E - MoE + hybrid families" (expert dispatch
through gather_mm / gather_qmm; shared experts always active) and the gate page's merge
recommendation (router -> route -> switch_glu -> combine with an always-active shared
expert and no shared-expert gate).  Pins: a dense brute-force sum over ALL experts with
the routing mask, written with torch fp64 matmuls (a different computation from the
oracle's per-pair loop); closed forms (x = 0, zero down-projection, one expert, a scalar
SwiGLU); symmetries (token permutation, expert relabelling); the 4-bit format against the
same weights dequantised independently here.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _f64(a, dt):
    if dt == "bf16":
        return torch.from_numpy(synth.bf16_to_f32(a).reshape(a.shape).astype(np.float64))
    return torch.from_numpy(np.asarray(a, np.float64))


def dense_reference(w, x, router_w, bias, ex, sh, inds, scores):
    """y = shared(x) + sum over every expert e of mask[t,e] * weight[t,e] * SwiGLU_e(x)."""
    X = _f64(x, w.act)
    Wg, Wu, Wd = _f64(ex["gate"], w.expert), _f64(ex["up"], w.expert), _f64(ex["down"], w.expert)
    g = torch.einsum("th,eih->eti", X, Wg)
    u = torch.einsum("th,eih->eti", X, Wu)
    h = torch.nn.functional.silu(g) * u
    o = torch.einsum("eti,ehi->eth", h, Wd)  # [E, T, H] every expert on every token
    M = torch.zeros(w.T, w.E, dtype=torch.float64)
    for t in range(w.T):
        for j in range(w.K):
            M[t, int(inds[t, j])] += float(scores[t, j])
    y = torch.einsum("te,eth->th", M, o)
    if sh is not None:
        Sg, Su, Sd = _f64(sh["gate"], w.act), _f64(sh["up"], w.act), _f64(sh["down"], w.act)
        y = y + (torch.nn.functional.silu(X @ Sg.T) * (X @ Su.T)) @ Sd.T
    return y.numpy()


def _inputs(w):
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    return x, r, b, synth.gen_expert_weights(w), synth.gen_shared(w)


SMALL = [
    synth.WORKLOADS["c0"],
    synth.WORKLOADS["c1"].with_(name="c1-small", T=24, H=128, I=64, Is=64, planted=0),
    synth.WORKLOADS["c1"].with_(name="c1-small-f32", T=12, H=64, I=32, Is=48, act="f32", expert="f32", planted=0),
    synth.WORKLOADS["c2"].with_(name="dsv3-tiny", T=6, H=64, I=64, Is=64, E=32, G=8, TG=4, K=8),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_dense_brute_force(w):
    x, r, b, ex, sh = _inputs(w)
    y, inds, scores, _ = oracle.forward_workload(w, x, r, b, ex, sh)
    ref = dense_reference(w, x, r, b, ex, sh, inds, scores)
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_route_inside_forward_matches_route_on_router_logits():
    w = synth.WORKLOADS["c1"].with_(T=40, H=256, I=64, Is=64, planted=0)
    x, r, b, ex, sh = _inputs(w)
    _, inds, scores, logits = oracle.forward_workload(w, x, r, b, ex, sh)
    assert np.array_equal(logits, oracle.router(x, r, w.act))
    _, i2, s2 = oracle.route(logits, b, oracle.params(w.K, w.G, w.TG, w.norm, w.rsf))
    assert np.array_equal(inds, i2) and np.array_equal(scores, s2)


def test_zero_input_gives_zero_output():
    w = synth.WORKLOADS["c0"]
    x, r, b, ex, sh = _inputs(w)
    y, *_ = oracle.forward_workload(w, np.zeros_like(x), r, b, ex, sh)
    assert np.all(y == 0.0)


def test_zero_down_projection_leaves_shared_expert():
    w = synth.WORKLOADS["c0"]
    x, r, b, ex, sh = _inputs(w)
    ex = dict(ex, down=np.zeros_like(ex["down"]))
    y, *_ = oracle.forward_workload(w, x, r, b, ex, sh)
    X = torch.from_numpy(x.astype(np.float64))
    ys = (torch.nn.functional.silu(X @ torch.from_numpy(sh["gate"].astype(np.float64)).T)
          * (X @ torch.from_numpy(sh["up"].astype(np.float64)).T)) @ torch.from_numpy(sh["down"].astype(np.float64)).T
    assert np.max(np.abs(y - ys.numpy())) < 1e-12


def test_one_expert_closed_form():
    """E = K = 1, no shared expert: y = rsf * sigmoid(logit) * SwiGLU(x)."""
    w = synth.WORKLOADS["c0"].with_(E=1, K=1, Is=0, rsf=2.5)
    x, r, b, ex, _ = _inputs(w)
    y, inds, scores, logits = oracle.forward_workload(w, x, r, b, ex, None)
    assert np.all(inds == 0)
    assert np.array_equal(scores[:, 0], (oracle.sigmoid(logits[:, 0]) * np.float32(2.5)).astype(np.float32))
    X = torch.from_numpy(x.astype(np.float64))
    Wg, Wu, Wd = (torch.from_numpy(ex[k][0].astype(np.float64)) for k in ("gate", "up", "down"))
    f = (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
    ref = scores[:, :1].astype(np.float64) * f.numpy()
    assert np.max(np.abs(y - ref)) < 1e-12


def test_scalar_swiglu_closed_form():
    """H = I = 1: W_down * silu(W_gate x) * (W_up x); silu(z) = z / (1 + e^-z).  Swapping gate
    and up must change the result (the gate is the projection that goes through silu)."""
    silu = lambda z: z / (1.0 + math.exp(-z))
    one = np.ones(1, np.float64)
    a = oracle.swiglu(one, np.array([[1.0]], np.float32), np.array([[2.0]], np.float32),
                      np.array([[3.0]], np.float32), "f32")
    assert abs(a[0] - 3.0 * 2.0 * silu(1.0)) < 1e-15
    b = oracle.swiglu(one, np.array([[2.0]], np.float32), np.array([[1.0]], np.float32),
                      np.array([[3.0]], np.float32), "f32")
    assert abs(b[0] - 3.0 * 1.0 * silu(2.0)) < 1e-15
    assert abs(a[0] - b[0]) > 0.5


def test_token_permutation_permutes_output():
    w = synth.WORKLOADS["c1"].with_(T=20, H=128, I=64, Is=64, planted=0)
    x, r, b, ex, sh = _inputs(w)
    y, inds, scores, _ = oracle.forward_workload(w, x, r, b, ex, sh)
    perm = np.random.default_rng(0).permutation(w.T)
    y2, i2, s2, _ = oracle.forward_workload(w, np.ascontiguousarray(x[perm]), r, b, ex, sh)
    assert np.array_equal(y2, y[perm]) and np.array_equal(i2, inds[perm]) and np.array_equal(s2, scores[perm])


def test_expert_relabelling_inside_groups_is_invisible():
    """Permuting experts within each group (router rows, bias, weights alike) relabels the
    selection and leaves y bit-identical."""
    w = synth.WORKLOADS["c1"].with_(T=20, H=128, I=64, Is=64, planted=0)
    x, r, b, ex, sh = _inputs(w)
    y, inds, _, _ = oracle.forward_workload(w, x, r, b, ex, sh)
    Eg = w.E // w.G
    rng = np.random.default_rng(1)
    perm = np.concatenate([g * Eg + rng.permutation(Eg) for g in range(w.G)])  # new e' holds old perm[e']
    ex2 = {k: np.ascontiguousarray(v[perm]) for k, v in ex.items()}
    y2, i2, _, _ = oracle.forward_workload(w, x, np.ascontiguousarray(r[perm]), np.ascontiguousarray(b[perm]), ex2, sh)
    assert np.array_equal(perm[i2], inds)
    assert np.array_equal(y2, y)


def _dequant_numpy(q, s, b, cols):
    """Independent statement of the packed format: nibble i%8 of word i//8, value s*q + b."""
    rows = q.shape[0]
    shifts = (4 * np.arange(8, dtype=np.uint32))
    codes = ((q[:, :, None] >> shifts) & 0xF).reshape(rows, cols).astype(np.float64)
    sf = synth.bf16_to_f32(s).reshape(s.shape).astype(np.float64)
    bf = synth.bf16_to_f32(b).reshape(b.shape).astype(np.float64)
    return codes * np.repeat(sf, 64, axis=1) + np.repeat(bf, 64, axis=1)


def test_q4_roundtrip_bound():
    rows, cols, std = 64, 256, 1 / 16
    q, s, b = synth.q4_normal(9, 5, rows, cols, std)
    w = synth.normal_f32(9, 5, rows * cols, std).reshape(rows, cols).astype(np.float64)
    d = _dequant_numpy(q, s, b, cols)
    sf = np.repeat(synth.bf16_to_f32(s).reshape(s.shape).astype(np.float64), 64, axis=1)
    mn = np.repeat(w.reshape(rows, cols // 64, 64).min(axis=2), 64, axis=1)
    # half a step of rounding plus the bf16 rounding of the offset and the scale over 15 steps
    bound = sf / 2 + np.abs(mn) * 2.0 ** -8 + 15 * sf * 2.0 ** -8 + 1e-12
    assert np.all(np.abs(w - d) <= bound)


def test_q4_forward_equals_forward_on_dequantised_weights():
    w = synth.WORKLOADS["c4"].with_(T=10, H=128, I=64, Is=64, E=16, G=4, TG=2, K=4)
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    ex = synth.gen_expert_weights(w)
    sh = synth.gen_shared(w)
    y, inds, scores, _ = oracle.forward_workload(w, x, r, b, ex, sh)
    deq = {}
    for nm, (o, i) in (("gate", (w.I, w.H)), ("up", (w.I, w.H)), ("down", (w.H, w.I))):
        d = _dequant_numpy(ex[nm].reshape(w.E * o, i // 8), ex["s_" + nm].reshape(w.E * o, i // 64),
                           ex["b_" + nm].reshape(w.E * o, i // 64), i)
        d32 = d.astype(np.float32)
        assert np.array_equal(d32.astype(np.float64), d)  # the dequantised values are exact in fp32
        deq[nm] = d32.reshape(w.E, o, i)
    y2, i2, s2, _ = oracle.forward_workload(w.with_(expert="f32"), x, r, b, deq, sh)
    assert np.array_equal(inds, i2) and np.array_equal(scores, s2)
    assert np.max(np.abs(y - y2)) == 0.0


def test_offset_shifts_logits_only():
    w = synth.WORKLOADS["c3"].with_(T=16, H=128, I=32, Is=32, E=32, G=8, TG=4, K=8)
    x, r, b, ex, sh = _inputs(w)
    off = synth.gen_logit_offset(w)
    _, _, _, l0 = oracle.forward_workload(w, x, r, b, ex, sh)
    _, _, _, l1 = oracle.forward_workload(w, x, r, b, ex, sh, offset=off)
    assert np.array_equal(l1, (l0 + off).astype(np.float32))


def test_subset_rows_equal_full_rows():
    w = synth.WORKLOADS["c1"].with_(T=32, H=128, I=64, Is=64, planted=0)
    x, r, b, ex, sh = _inputs(w)
    y, inds, scores, _ = oracle.forward_workload(w, x, r, b, ex, sh)
    rows = [31, 0, 7, 7]
    y2, i2, s2, _ = oracle.forward_workload(w, x, r, b, ex, sh, rows=rows)
    assert np.array_equal(y2, y[rows]) and np.array_equal(i2, inds[rows]) and np.array_equal(s2, scores[rows])


def test_planted_rows_put_the_max_expert_in_a_losing_group():
    """c1's planted rows: on the oracle's own logits, the expert with the single largest
    biased score is NOT selected (its group loses on the top-2 sum)."""
    w = synth.WORKLOADS["c1"]
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    rows = synth.planted_rows(w)
    logits = oracle.router(np.ascontiguousarray(x[rows]), r, "bf16")
    _, inds, _ = oracle.route(logits, b, oracle.params(w.K, w.G, w.TG, w.norm, w.rsf))
    biased = oracle.sigmoid(logits) + b
    top = np.argmax(biased, axis=1)
    lost = [int(top[i]) not in set(inds[i].tolist()) for i in range(len(rows))]
    assert sum(lost) >= 32, sum(lost)


@pytest.mark.parametrize("a,b_", [(2.5, 1.0), (0.75, 3.0)])
def test_layer_scaling_linearity(a, b_):
    """The routed part of y scales linearly with routed_scaling_factor (the gate page, "Algorithm":
    the weights are multiplied by it after the norm): (y(a) - ys) = (a / b) (y(b) - ys), where ys
    is the shared expert's output alone (the dense MLP of the shared weights), and the selection
    does not depend on the factor.  Each weight is rounded once more in fp32 after the scaling, so
    the two sides agree to a few fp32 ulps of the weights."""
    w = synth.WORKLOADS["c1"].with_(T=24, H=128, I=64, Is=64, planted=0)
    x, r, b, ex, sh = _inputs(w)
    ya, ia, sa, _ = oracle.forward_workload(w.with_(rsf=a), x, r, b, ex, sh)
    yb, ib, sb, _ = oracle.forward_workload(w.with_(rsf=b_), x, r, b, ex, sh)
    assert np.array_equal(ia, ib)
    ys = oracle.dense_mlp(x, sh["gate"], sh["up"], sh["down"], w.act)
    ra, rb = ya - ys, (yb - ys) * (a / b_)
    assert np.linalg.norm(ra) > 0.1 * np.linalg.norm(ya)  # the routed part is not negligible
    assert np.linalg.norm(ra - rb) <= 4 * 2.0 ** -24 * np.linalg.norm(ra)
    # and a wrong factor is visible at this tolerance
    assert np.linalg.norm(ra - rb * 1.0001) > 4 * 2.0 ** -24 * np.linalg.norm(ra)
