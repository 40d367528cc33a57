"""Pins of the oracle's dispatch (CPU only).

Page: "Epic: Engine Inference Core Stage E - MoE + hybrid families", opening paragraph: the
layer hands every expert its tokens through gather_mm / gather_qmm.  The grouping this implies
is defined by: counts[e] = number of slots s = t*K + j routed to e; offsets = exclusive prefix
sum of counts (offsets[E] = T*K); sorted_slot lists, expert after expert, the slots routed to
that expert in ascending order; slot_row is its inverse permutation.

Pins: hand-derived cases worked out from that definition (written below with their
derivation); a brute-force restatement that filters the slot list once per expert (a different
computation from the oracle's counting sort); the permutation properties; the reject path.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth


def test_hand_case_three_experts():
    # slots: s0=(t0,j0)->2, s1=(t0,j1)->0, s2=(t1,j0)->0, s3=(t1,j1)->2, s4=(t2,j0)->1, s5=(t2,j1)->0
    # expert 0 gets s1, s2, s5; expert 1 gets s4; expert 2 gets s0, s3
    counts, offsets, sorted_slot, slot_row = oracle.dispatch(np.array([[2, 0], [0, 2], [1, 0]], np.int32), 3)
    assert counts.tolist() == [3, 1, 2]
    assert offsets.tolist() == [0, 3, 4, 6]
    assert sorted_slot.tolist() == [1, 2, 5, 4, 0, 3]
    # s0 sits at row 4, s1 at 0, s2 at 1, s3 at 5, s4 at 3, s5 at 2
    assert slot_row.tolist() == [4, 0, 1, 5, 3, 2]


def test_hand_case_empty_experts_and_k1():
    # K = 1, E = 5: tokens pick 4, 1, 4, 4; experts 0, 2, 3 receive nothing
    counts, offsets, sorted_slot, slot_row = oracle.dispatch(np.array([[4], [1], [4], [4]], np.int32), 5)
    assert counts.tolist() == [0, 1, 0, 0, 3]
    assert offsets.tolist() == [0, 0, 1, 1, 1, 4]
    assert sorted_slot.tolist() == [1, 0, 2, 3]
    assert slot_row.tolist() == [1, 0, 2, 3]


def test_hand_case_one_expert_keeps_slot_order():
    # every slot to expert 1 of 2: the stable order is the slot order itself
    counts, offsets, sorted_slot, slot_row = oracle.dispatch(np.ones((3, 2), np.int32), 2)
    assert counts.tolist() == [0, 6]
    assert offsets.tolist() == [0, 0, 6]
    assert sorted_slot.tolist() == list(range(6))
    assert slot_row.tolist() == list(range(6))


def brute_force(inds, E):
    flat = [int(v) for v in np.asarray(inds).ravel()]
    segs = [[s for s in range(len(flat)) if flat[s] == e] for e in range(E)]
    counts = [len(g) for g in segs]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    sorted_slot = [s for g in segs for s in g]
    slot_row = [0] * len(flat)
    for r, s in enumerate(sorted_slot):
        slot_row[s] = r
    return counts, offsets, sorted_slot, slot_row


@pytest.mark.parametrize("T,K,E,seed", [(1, 1, 1, 0), (7, 3, 4, 1), (40, 6, 64, 2), (33, 8, 256, 3),
                                        (100, 2, 3, 4), (0, 4, 8, 5)])
def test_brute_force_small(T, K, E, seed):
    u = synth.uniform(seed, 12, max(T * K, 1))[: T * K]
    # a skewed draw so some experts are empty and some crowded
    inds = np.minimum((u ** 3 * E).astype(np.int32), E - 1).reshape(T, K)
    got = oracle.dispatch(inds, E)
    want = brute_force(inds, E)
    for g, w, name in zip(got, want, ("counts", "offsets", "sorted_slot", "slot_row")):
        assert g.tolist() == w, name


def test_permutation_properties_large():
    T, K, E = 8192, 8, 256
    u = synth.uniform(3, 12, T * K)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    inds = np.minimum(np.searchsorted(np.cumsum(p) / p.sum(), u), E - 1).astype(np.int32).reshape(T, K)
    counts, offsets, sorted_slot, slot_row = oracle.dispatch(inds, E)
    flat = inds.ravel()
    n = T * K
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == n and np.all(np.diff(offsets) == counts)
    assert np.array_equal(np.sort(sorted_slot), np.arange(n))            # a permutation
    assert np.array_equal(slot_row[sorted_slot], np.arange(n))            # slot_row is its inverse
    for e in range(E):
        seg = sorted_slot[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)                                     # the expert's own slots
        assert np.all(np.diff(seg) > 0)                                   # in ascending order


def test_rejects_leave_outputs_untouched():
    lib = oracle._L()
    inds = np.array([[0, 3]], np.int32)  # 3 is outside [0, E) for E = 3
    outs = [np.full(n, -7, np.int32) for n in (3, 4, 2, 2)]
    ptrs = [o.ctypes.data for o in outs]
    assert lib.oracle_dispatch(inds.ctypes.data, 1, 2, 3, *ptrs) == -1
    assert all(np.all(o == -7) for o in outs)
    neg = np.array([[-1, 0]], np.int32)
    assert lib.oracle_dispatch(neg.ctypes.data, 1, 2, 3, *ptrs) == -1
    assert lib.oracle_dispatch(inds.ctypes.data, -1, 2, 3, *ptrs) == -1
    assert lib.oracle_dispatch(inds.ctypes.data, 1, 0, 3, *ptrs) == -1
    assert lib.oracle_dispatch(inds.ctypes.data, 1, 2, 0, *ptrs) == -1
    assert lib.oracle_dispatch(None, 1, 2, 3, *ptrs) == -1
    assert all(np.all(o == -7) for o in outs)
    with pytest.raises(ValueError):
        oracle.dispatch(inds, 3)
