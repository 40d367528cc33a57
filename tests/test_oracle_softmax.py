"""Pins of the oracle's softmax gate and of the shared-expert gate (CPU only).

Page: "feat(engine): E1 DeepSeek-style MoE gate (sigmoid, group top-k, bias) (#108)" -- the
softmax route is the DeepSeek route's sibling: same output contract ("API"), and it normalises
its weights in every case (second review, S2).  Reading taken where the pages stop: weights are
the softmax probabilities of the selected experts renormalised over the selection, experts ranked
by their unnormalised exponentials (ties to the lower index), no bias, groups or scale.  The
shared-expert gate (the combine's has_shared_expert_gate switch named in the reviews) is read as
sigmoid(x . w) scaling the shared expert's output.

Pins: the weights equal a softmax over just the selected logits computed in fp64 (a different
formula, equal in exact arithmetic); the selection equals a brute-force sort of the logits;
top_k = 1 gives exactly 1.0; all-equal logits give 1/K by index order; shift invariance; the
reject matrix; the layer against a dense fp64 brute force with those weights; the shared gate's
closed forms (w = 0 halves the shared output; in general y_gated = y_ungated - (1 - g) * shared).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle_layer import _f64


def _distinct_logits(rng, T, E, spread=4.0):
    """Rows of distinct logits at least 1e-3 apart, so their exponentials cannot tie."""
    base = np.arange(E, dtype=np.float64) * (spread / E)
    out = np.empty((T, E), np.float32)
    for t in range(T):
        out[t] = (rng.permutation(base) + rng.normal() * 0.5).astype(np.float32)
    return out


@pytest.mark.parametrize("E,K", [(8, 2), (64, 6), (256, 8), (160, 64), (1, 1)])
def test_selection_is_a_sort_and_weights_are_a_softmax_over_the_selection(E, K):
    rng = np.random.default_rng(E * 100 + K)
    lg = _distinct_logits(rng, 50, E)
    rc, inds, scores = oracle.route_softmax(lg, K)
    assert rc == 0
    for t in range(lg.shape[0]):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:K]
        assert list(inds[t]) == order
        sel = lg[t, order].astype(np.float64)
        ref = np.exp(sel - sel.max())
        ref /= ref.sum()
        np.testing.assert_allclose(scores[t], ref, rtol=2e-6, atol=0)


def test_top_k_one_gives_exactly_one():
    rng = np.random.default_rng(3)
    lg = rng.normal(size=(40, 32)).astype(np.float32)
    rc, inds, scores = oracle.route_softmax(lg, 1)
    assert rc == 0
    assert np.all(scores == 1.0)
    assert np.array_equal(inds[:, 0], np.argmax(lg, axis=1))  # argmax takes the first maximum


def test_equal_logits_split_evenly_by_index():
    lg = np.full((3, 16), 2.5, np.float32)
    rc, inds, scores = oracle.route_softmax(lg, 4)
    assert rc == 0
    assert np.array_equal(inds, np.tile(np.arange(4, dtype=np.int32), (3, 1)))
    assert np.all(scores == 0.25)


def test_shift_invariance_and_large_logits():
    rng = np.random.default_rng(5)
    lg = _distinct_logits(rng, 30, 48)
    _, i0, s0 = oracle.route_softmax(lg, 5)
    _, i1, s1 = oracle.route_softmax(lg + np.float32(1000.0), 5)  # no overflow: exp(l - max) <= 1
    assert np.array_equal(i0, i1)
    np.testing.assert_allclose(s1, s0, rtol=1e-3)  # the shift rounds the logits at 1000 + x
    assert np.all(np.isfinite(s1))
    np.testing.assert_allclose(s0.sum(axis=1), 1.0, rtol=4e-7)


@pytest.mark.parametrize("T,E,K", [(2, 8, 0), (2, 8, 9), (2, 0, 1), (-1, 8, 2)])
def test_rejects_leave_outputs_untouched(T, E, K):
    lg = np.zeros((max(T, 0), max(E, 1)), np.float32)
    inds = np.full((max(T, 1), max(K, 1)), -7, np.int32)
    scores = np.full((max(T, 1), max(K, 1)), -7.0, np.float32)
    p = oracle._p
    rc = oracle._L().oracle_route_softmax(p(lg), T, E, K, p(inds), p(scores))
    assert rc == -1
    assert np.all(inds == -7) and np.all(scores == -7.0)


def _softmax_dense_reference(w, x, ex, sh, logits, shared_gate=None):
    """Dense fp64 layer over ALL experts with the softmax weights computed here."""
    X = _f64(x, w.act)
    Wg, Wu, Wd = _f64(ex["gate"], w.expert), _f64(ex["up"], w.expert), _f64(ex["down"], w.expert)
    h = torch.nn.functional.silu(torch.einsum("th,eih->eti", X, Wg)) * torch.einsum("th,eih->eti", X, Wu)
    o = torch.einsum("eti,ehi->eth", h, Wd)
    M = torch.zeros(w.T, w.E, dtype=torch.float64)
    for t in range(w.T):
        order = sorted(range(w.E), key=lambda e: (-float(logits[t, e]), e))[: w.K]
        sel = logits[t, order].astype(np.float64)
        p = np.exp(sel - sel.max())
        p /= p.sum()
        for e, v in zip(order, p):
            M[t, e] = v
    y = torch.einsum("te,eth->th", M, o)
    if sh is not None:
        Sg, Su, Sd = _f64(sh["gate"], w.act), _f64(sh["up"], w.act), _f64(sh["down"], w.act)
        ys = (torch.nn.functional.silu(X @ Sg.T) * (X @ Su.T)) @ Sd.T
        if shared_gate is not None:
            g = torch.sigmoid(X @ _f64(shared_gate, w.act))
            ys = ys * g[:, None]
        y = y + ys
    return y.numpy()


LAYERS = [
    synth.WORKLOADS["c1"].with_(name="softmax-bf16", T=20, H=128, I=64, Is=64, planted=0, route="softmax"),
    synth.WORKLOADS["c0"].with_(name="softmax-f32", route="softmax"),
    synth.WORKLOADS["c1"].with_(name="softmax-gated-bf16", T=16, H=128, I=64, Is=96, planted=0, route="softmax",
                                shared_gate=True),
    synth.WORKLOADS["c0"].with_(name="deepseek-gated-f32", shared_gate=True),
]


@pytest.mark.parametrize("w", LAYERS, ids=[w.name for w in LAYERS])
def test_layer_against_dense_brute_force(w):
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    ex, sh, sg = synth.gen_expert_weights(w), synth.gen_shared(w), synth.gen_shared_gate(w)
    y, inds, scores, logits = oracle.forward_workload(w, x, r, b, ex, sh, shared_gate=sg)
    if w.route == "softmax":
        ref = _softmax_dense_reference(w, x, ex, sh, logits, sg)
        tol = 2e-6  # the weights are fp32 in the oracle, fp64 here
    else:
        from test_oracle_layer import dense_reference
        ref = dense_reference(w, x, r, b, ex, None, inds, scores)
        X = _f64(x, w.act)
        Sg, Su, Sd = _f64(sh["gate"], w.act), _f64(sh["up"], w.act), _f64(sh["down"], w.act)
        ys = ((torch.nn.functional.silu(X @ Sg.T) * (X @ Su.T)) @ Sd.T).numpy()
        g = torch.sigmoid(X @ _f64(sg, w.act)).numpy()
        ref = ref + g[:, None] * ys
        tol = 2e-6  # the gate is an fp32 sigmoid of an fp32 dot product in the oracle
    assert np.max(np.abs(y - ref)) <= tol * max(1.0, np.max(np.abs(ref)))


def test_zero_shared_gate_halves_the_shared_output():
    """sigmoid(0) = 1/2 exactly, so y(w_sgate = 0) = y(no gate) - shared / 2 up to fp64 rounding."""
    w = synth.WORKLOADS["c1"].with_(T=12, H=128, I=64, Is=64, planted=0)
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    ex, sh = synth.gen_expert_weights(w), synth.gen_shared(w)
    y0, *_ = oracle.forward_workload(w, x, r, b, ex, sh)
    zero = np.zeros(w.H, np.uint16)  # bf16 zeros
    yg, *_ = oracle.forward_workload(w, x, r, b, ex, sh, shared_gate=zero)
    ys = np.stack([oracle.swiglu(_f64(x, w.act)[t].numpy(), sh["gate"], sh["up"], sh["down"], w.act)
                   for t in range(w.T)])
    np.testing.assert_allclose(yg, y0 - 0.5 * ys, rtol=0, atol=1e-12 * np.max(np.abs(y0)))
