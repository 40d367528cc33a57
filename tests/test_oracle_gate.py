"""Pins of the oracle's DeepSeek gate (CPU only).

Page: "feat(engine): E1 DeepSeek-style MoE gate (sigmoid, group top-k, bias) (#108)",
sections "API", "Algorithm", "Tests" and the two code reviews.  Pins used here:
hand-derived golden cases (tests/golden/gate_cases.json), brute-force search on tiny
inputs (exhaustive pair / subset maximisation, a different algorithm from the oracle's
sorting), and the invariants the pages state (S1 bias selects but does not weigh, S2 norm
only for top_k > 1, scaling after norm, D7 k_drop == 0 equals no grouping, flattening of
leading dims, the prologue reject matrix with outputs left untouched).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "gate_cases.json")))["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_cases(case):
    p = oracle.params(case["top_k"], case["n_group"], case["topk_group"], case["norm"], case["rsf"])
    rc, inds, scores = oracle.route(np.array([case["logits"]], np.float32), np.array(case["bias"], np.float32), p)
    assert rc == 0
    assert inds[0].tolist() == case["expect_inds"]
    assert scores[0].tolist() == [float(np.float32(v)) for v in case["expect_scores"]]


# --------------------------------------------------------------------------------------------
# prologue reject matrix: -1 and outputs untouched
# --------------------------------------------------------------------------------------------
REJECTS = [
    ("top_k_zero", 8, dict(top_k=0, n_group=1, topk_group=1)),
    ("top_k_gt_E", 8, dict(top_k=9, n_group=1, topk_group=1)),
    ("E_not_divisible", 8, dict(top_k=2, n_group=3, topk_group=1)),
    ("topk_group_zero", 8, dict(top_k=2, n_group=2, topk_group=0)),
    ("topk_group_gt_n_group", 8, dict(top_k=2, n_group=2, topk_group=3)),
    ("topk_group_2_with_n_group_1", 8, dict(top_k=2, n_group=1, topk_group=2)),
    ("group_of_one_expert", 8, dict(top_k=2, n_group=8, topk_group=2)),
    ("n_group_zero", 8, dict(top_k=2, n_group=0, topk_group=1)),
]


@pytest.mark.parametrize("name,E,kw", REJECTS, ids=[r[0] for r in REJECTS])
def test_reject_matrix_leaves_outputs_untouched(name, E, kw):
    p = oracle.params(kw["top_k"], kw["n_group"], kw["topk_group"], True, 1.0)
    rc, inds, scores = oracle.route(np.zeros((3, E), np.float32), np.zeros(E, np.float32), p)
    assert rc == -1
    assert np.all(inds == -7) and np.all(scores == -7.0)


def test_reject_null_bias():
    lib = oracle._L()
    lg = np.zeros((2, 8), np.float32)
    inds = np.full((2, 2), -7, np.int32)
    sc = np.full((2, 2), -7.0, np.float32)
    p = oracle.params(2)
    import ctypes
    assert lib.oracle_route(lg.ctypes.data, 2, 8, None, ctypes.byref(p), inds.ctypes.data, sc.ctypes.data) == -1
    assert np.all(inds == -7) and np.all(sc == -7.0)


# --------------------------------------------------------------------------------------------
# G = 1: a full sort of sigmoid + bias (textbook sort as the independent statement)
# --------------------------------------------------------------------------------------------
def test_n_group_1_equals_full_sort():
    rng = np.random.default_rng(1)
    for trial in range(200):
        E = int(rng.integers(1, 40))
        K = int(rng.integers(1, E + 1))
        lg = rng.normal(0, 2, (1, E)).astype(np.float32)
        bias = rng.normal(0, 0.3, E).astype(np.float32)
        rc, inds, _ = oracle.route(lg, bias, oracle.params(K))
        assert rc == 0
        b = oracle.sigmoid(lg[0]) + bias  # fp32 add, same rounding as any IEEE add
        order = np.lexsort((np.arange(E), -b.astype(np.float64)))
        assert inds[0].tolist() == order[:K].tolist()


# --------------------------------------------------------------------------------------------
# brute force with groups: exhaustive maximisation instead of sorting
# --------------------------------------------------------------------------------------------
def brute_force_select(sig, bias, G, TG, K):
    """Selected expert set by exhaustive search.  Group score = max over expert pairs of the
    pair sum (== the top-2 sum); kept groups = the TG-subset of groups with the largest total
    score; selection = the K-subset of kept experts with the largest total biased score.
    Valid when all these maxima are unique and K <= TG*Eg with positive biased scores."""
    E = len(sig)
    Eg = E // G
    b = (sig + bias).astype(np.float32)
    if G > 1 and TG < G:
        gs = [max(float(np.float32(b[g * Eg + i] + b[g * Eg + j])) for i, j in itertools.combinations(range(Eg), 2))
              for g in range(G)]
        kept = max(itertools.combinations(range(G), TG), key=lambda S: sum(gs[g] for g in S))
        allowed = [e for g in kept for e in range(g * Eg, (g + 1) * Eg)]
    else:
        allowed = list(range(E))
    best = max(itertools.combinations(allowed, K), key=lambda S: sum(float(b[e]) for e in S))
    return set(best), b


def test_brute_force_group_selection():
    rng = np.random.default_rng(7)
    n = 0
    for trial in range(400):
        G = int(rng.choice([2, 3, 4]))
        Eg = int(rng.integers(2, 5))
        E = G * Eg
        TG = int(rng.integers(1, G + 1))
        K = int(rng.integers(1, min(TG * Eg, 5) + 1))
        lg = rng.normal(0, 1.5, (1, E)).astype(np.float32)
        bias = np.abs(rng.normal(0, 0.2, E)).astype(np.float32)  # positive: kept scores > 0.0
        sig = oracle.sigmoid(lg[0])
        want, b = brute_force_select(sig, bias, G, TG, K)
        rc, inds, scores = oracle.route(lg, bias, oracle.params(K, G, TG, True, 1.0))
        assert rc == 0
        assert set(inds[0].tolist()) == want, (trial, G, TG, K)
        # output order: biased score descending
        assert np.all(np.diff(b[inds[0]].astype(np.float64)) <= 0)
        n += 1
    assert n == 400


# --------------------------------------------------------------------------------------------
# stated invariants
# --------------------------------------------------------------------------------------------
def test_S1_bias_that_keeps_selection_keeps_scores_bitwise():
    """A bias that shifts every biased score by the same exact amount keeps the order, so the
    returned weights (pre-bias) must be bit-identical to the bias-free ones."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        E, K = 32, 6
        lg = rng.uniform(0.1, 2.0, (4, E)).astype(np.float32)  # sigmoid in [0.52, 0.88]
        p = oracle.params(K, 1, 1, True, 2.5)
        _, i0, s0 = oracle.route(lg, np.zeros(E, np.float32), p)
        _, i1, s1 = oracle.route(lg, np.full(E, 0.0625, np.float32), p)
        assert np.array_equal(i0, i1)
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))


def test_S1_bias_that_changes_selection_weighs_by_pre_bias_sigmoid():
    rng = np.random.default_rng(4)
    changed = 0
    for _ in range(100):
        E, K = 16, 4
        lg = rng.normal(0, 1, (1, E)).astype(np.float32)
        bias = rng.normal(0, 0.5, E).astype(np.float32)
        p = oracle.params(K, 1, 1, False, 1.0)  # no norm: weight j must be sigmoid(logit[inds[j]])
        _, i0, _ = oracle.route(lg, np.zeros(E, np.float32), p)
        _, i1, s1 = oracle.route(lg, bias, p)
        changed += set(i0[0]) != set(i1[0])
        assert np.array_equal(s1[0], oracle.sigmoid(lg[0][i1[0]]))
    assert changed > 20


def test_S2_top_k_1_no_norm_both_flags():
    rng = np.random.default_rng(5)
    lg = rng.normal(0, 1, (64, 12)).astype(np.float32)
    bias = rng.normal(0, 0.1, 12).astype(np.float32)
    for rsf in (1.0, 2.5, 0.3):
        _, ia, sa = oracle.route(lg, bias, oracle.params(1, 1, 1, True, rsf))
        _, ib, sb = oracle.route(lg, bias, oracle.params(1, 1, 1, False, rsf))
        assert np.array_equal(ia, ib) and np.array_equal(sa, sb)
        expect = (oracle.sigmoid(lg[np.arange(64), ia[:, 0]]) * np.float32(rsf)).astype(np.float32)
        assert np.array_equal(sa[:, 0], expect)


def test_S2_norm_sums_to_scaling_factor():
    rng = np.random.default_rng(6)
    lg = rng.normal(0, 1, (256, 64)).astype(np.float32)
    bias = rng.normal(0, 0.5, 64).astype(np.float32)
    for K in (2, 6, 8):
        _, _, s = oracle.route(lg, bias, oracle.params(K, 4, 2, True, 2.5))
        tot = s.astype(np.float64).sum(axis=1)
        assert np.max(np.abs(tot - 2.5)) < 2.5 * K * 2.0 ** -22


def test_scaling_is_one_rounding_after_norm():
    rng = np.random.default_rng(8)
    lg = rng.normal(0, 1, (128, 64)).astype(np.float32)
    bias = rng.normal(0, 0.5, 64).astype(np.float32)
    _, i1, s1 = oracle.route(lg, bias, oracle.params(6, 4, 2, True, 1.0))
    for rsf in (2.5, 0.1, 16.0):
        _, ir, sr = oracle.route(lg, bias, oracle.params(6, 4, 2, True, rsf))
        assert np.array_equal(i1, ir)
        assert np.array_equal(sr, (s1 * np.float32(rsf)).astype(np.float32))


def test_D7_no_dropped_group_equals_one_group():
    rng = np.random.default_rng(9)
    lg = rng.normal(0, 1, (64, 32)).astype(np.float32)
    bias = rng.normal(0, 0.5, 32).astype(np.float32)
    for G in (2, 4, 8, 16):
        a = oracle.route(lg, bias, oracle.params(5, G, G, True, 2.5))
        b = oracle.route(lg, bias, oracle.params(5, 1, 1, True, 2.5))
        assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def test_leading_dims_flatten_to_rows():
    rng = np.random.default_rng(10)
    lg = rng.normal(0, 1, (3, 5, 16)).astype(np.float32)
    bias = rng.normal(0, 0.2, 16).astype(np.float32)
    p = oracle.params(3, 4, 2, True, 2.5)
    _, ia, sa = oracle.route(lg, bias, p)
    for b in range(3):
        for s in range(5):
            _, ir, sr = oracle.route(lg[b, s][None], bias, p)
            assert np.array_equal(ia[b * 5 + s], ir[0]) and np.array_equal(sa[b * 5 + s], sr[0])


def test_K_larger_than_kept_experts_selects_masked_zeros_by_index():
    """top_k above topk_group*Eg: the remaining slots go to the masked zeros, lowest index first."""
    lg = np.zeros((1, 8), np.float32)
    bias = np.array([0.4, 0.3, 0.2, 0.1, 0.0, 0.0, 0.0, 0.0], np.float32)
    rc, inds, _ = oracle.route(lg, bias, oracle.params(4, 4, 1, True, 1.0))
    assert rc == 0 and inds[0].tolist() == [0, 1, 2, 3]  # kept group 0: [0.9, 0.8]; zeros 2, 3 by index


def test_zero_rows_is_a_noop():
    rc, inds, scores = oracle.route(np.zeros((0, 8), np.float32), np.zeros(8, np.float32), oracle.params(2))
    assert rc == 0 and inds.shape == (0, 2)


def test_case_b_recipe_runs():
    """Input recipe of the pages' second golden case (gates = RandomState(42).randn(16),
    bias = 0.5 * the next randn(16), 4 groups).  Its outputs are not printed on the pages
    and its top_k / topk_group / scaling are not stated, so only invariants are checked:
    parity with the pages' frozen vectors stays unpinned."""
    rs = np.random.RandomState(42)
    gates = rs.randn(16).astype(np.float32)
    bias = (0.5 * rs.randn(16)).astype(np.float32)
    rc, inds, scores = oracle.route(gates[None], bias, oracle.params(4, 4, 2, True, 1.0))
    assert rc == 0
    kept_groups = {int(i) // 4 for i in inds[0]}
    assert len(kept_groups) <= 2
    assert abs(float(scores.sum()) - 1.0) < 1e-6
