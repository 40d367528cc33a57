"""C-ABI checks that need no GPU: the library loads, exports every entry point that
include/dsmoe.h declares, and rejects invalid arguments before any HIP call (the gate page's
validation matrix, reviews L1/L2: null args, top_k == 0, top_k > E, E % n_group, topk_group
bounds, groups of one expert, bias rank / length), returning -1 and leaving outputs untouched.

Only rejected calls are made here: every check runs on the host before the first HIP call,
so the pointers below are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import deepseek_gate_expert_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "dsmoe.h")

# fake, 256-byte aligned, never dereferenced (host validation fails first)
P = 0x7f0000001000


@pytest.fixture(scope="module")
def lib():
    return dg.load_library()


def declared_functions():
    src = open(HDR).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", src, re.M)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(dg.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror(lib):
    assert dg.moe_strerror(0) == "ok"
    assert "invalid" in dg.moe_strerror(-1)
    assert "workspace" in dg.moe_strerror(-3)
    assert "unknown" in dg.moe_strerror(12345)


def route(lib, T=4, E=8, bias_len=None, params=(2, 1, 1, 1, 1.0), logits=P, bias=P, inds=P, scores=P):
    p = dg.RouteParams(*params)
    return lib.moe_route_deepseek(logits, T, E, bias, E if bias_len is None else bias_len, ctypes.byref(p), inds,
                                  scores, None)


ROUTE_REJECTS = {
    "top_k_zero": dict(params=(0, 1, 1, 1, 1.0)),
    "top_k_gt_E": dict(params=(9, 1, 1, 1, 1.0)),
    "E_not_divisible_by_n_group": dict(params=(2, 3, 1, 1, 1.0)),
    "n_group_zero": dict(params=(2, 0, 1, 1, 1.0)),
    "topk_group_zero": dict(params=(2, 2, 0, 1, 1.0)),
    "topk_group_gt_n_group": dict(params=(2, 2, 3, 1, 1.0)),
    "topk_group_2_n_group_1": dict(params=(2, 1, 2, 1, 1.0)),
    "one_expert_per_group": dict(params=(2, 8, 2, 1, 1.0)),
    "null_bias": dict(bias=None),
    "null_logits": dict(logits=None),
    "null_inds": dict(inds=None),
    "null_scores": dict(scores=None),
    "bias_len_ne_E": dict(bias_len=7),
    "negative_T": dict(T=-1),
    "misaligned_logits": dict(logits=P + 4),
}


@pytest.mark.parametrize("name", sorted(ROUTE_REJECTS))
def test_route_reject_matrix(lib, name):
    assert route(lib, **ROUTE_REJECTS[name]) == dg.MOE_ERR_INVALID


def test_route_null_params(lib):
    assert lib.moe_route_deepseek(P, 4, 8, P, 8, None, P, P, None) == dg.MOE_ERR_INVALID


def test_route_limits_are_unsupported_not_invalid(lib):
    assert route(lib, E=2048, params=(2, 1, 1, 1, 1.0)) == dg.MOE_ERR_UNSUPPORTED
    assert route(lib, E=256, params=(65, 1, 1, 1, 1.0)) == dg.MOE_ERR_UNSUPPORTED


def test_route_empty_rows_is_ok_without_touching_gpu(lib):
    assert route(lib, T=0, logits=None, inds=None, scores=None) == dg.MOE_OK


def test_router_logits_rejects(lib):
    f = lib.moe_router_logits
    assert f(None, P, 1, 4, 64, 8, None, P, None) == -1
    assert f(P, None, 1, 4, 64, 8, None, P, None) == -1
    assert f(P, P, 1, 4, 64, 8, None, None, None) == -1
    assert f(P, P, 7, 4, 64, 8, None, P, None) == -1
    assert f(P, P, 1, -1, 64, 8, None, P, None) == -1
    assert f(P, P, 1, 4, 0, 8, None, P, None) == -1
    assert f(P, P, 1, 4, 64, 0, None, P, None) == -1
    assert f(P, P, 1, 4, 64, 8, P + 2, P, None) == -1
    assert f(None, P, 1, 0, 64, 8, None, None, None) == 0


def test_dispatch_rejects(lib):
    f = lib.moe_dispatch
    need = lib.moe_dispatch_workspace_size(16, 2, 8)
    assert need > 0
    assert lib.moe_dispatch_workspace_size(-1, 2, 8) == 0
    assert f(None, 16, 2, 8, P, P, P, P, P, need, None) == -1
    assert f(P, 16, 0, 8, P, P, P, P, P, need, None) == -1
    assert f(P, 16, 2, 0, P, P, P, P, P, need, None) == -1
    assert f(P, 16, 2, 8, P, P, P, P, P, need - 1, None) == dg.MOE_ERR_WORKSPACE
    assert f(P, 16, 2, 2000, P, P, P, P, P, 1 << 30, None) == dg.MOE_ERR_UNSUPPORTED


def desc(**kw):
    base = dict(T=16, H=128, E=8, I=64, I_shared=64, act_dtype=1, expert_dtype=1, top_k=2, n_group=2, topk_group=1,
                norm_topk_prob=True, routed_scaling_factor=2.5)
    base.update(kw)
    return dg.layer_desc(**base)


def forward(lib, d, ws_bytes=None, shared=True, q4=False, x=P, y=P, ew_null=None, ws=P):
    ew = dg.ExpertWeights(*([P] * 9 if q4 else [P, P, P] + [None] * 6))
    if ew_null:
        setattr(ew, ew_null, None)
    sw = dg.SharedWeights(P, P, P) if shared else None
    need = lib.moe_forward_workspace_size(ctypes.byref(d))
    nbytes = need if ws_bytes is None else ws_bytes
    return lib.moe_forward(ctypes.byref(d), x, P, P, None, ctypes.byref(ew), None if sw is None else ctypes.byref(sw),
                           y, None, None, ws, nbytes, None)


FWD_REJECTS = {
    "negative_T": (dict(T=-1), {}),
    "zero_H": (dict(H=0), {}),
    "zero_I": (dict(I=0), {}),
    "negative_I_shared": (dict(I_shared=-1), {}),
    "bad_act_dtype": (dict(act_dtype=5), {}),
    "f32_act_with_bf16_experts": (dict(act_dtype=0, expert_dtype=1), {}),
    "bf16_act_with_f32_experts": (dict(act_dtype=1, expert_dtype=0), {}),
    "top_k_zero": (dict(top_k=0), {}),
    "top_k_gt_E": (dict(top_k=9), {}),
    "E_not_divisible": (dict(n_group=3), {}),
    "topk_group_gt_n_group": (dict(topk_group=3), {}),
    "one_expert_per_group": (dict(n_group=8, topk_group=2), {}),
    "null_x": (dict(), dict(x=None)),
    "null_y": (dict(), dict(y=None)),
    "null_w_gate": (dict(), dict(ew_null="w_gate")),
    "null_w_down": (dict(), dict(ew_null="w_down")),
    "q4_null_scale": (dict(expert_dtype=2), dict(q4=True, ew_null="s_up")),
    "fp8_null_scale": (dict(expert_dtype=3), dict(q4=True, ew_null="s_down")),
    "f32_act_with_fp8_experts": (dict(act_dtype=0, expert_dtype=3), {}),
    "unknown_expert_dtype": (dict(expert_dtype=4), {}),
    "shared_weights_missing": (dict(), dict(shared=False)),
    "shared_weights_without_shared_expert": (dict(I_shared=0), dict(shared=True)),
    "null_workspace": (dict(), dict(ws=None)),
    "misaligned_workspace": (dict(), dict(ws=P + 16)),
}


@pytest.mark.parametrize("name", sorted(FWD_REJECTS))
def test_forward_reject_matrix(lib, name):
    kw, fkw = FWD_REJECTS[name]
    d = desc(**kw)
    assert forward(lib, d, **fkw) == dg.MOE_ERR_INVALID


def test_forward_fp8_ignores_offsets(lib):
    """fp8 layers read only the block scales: NULL offsets pass the argument checks (the short
    workspace is then the first error, still found on the host)."""
    d = desc(expert_dtype=3)
    need = lib.moe_forward_workspace_size(ctypes.byref(d))
    assert need > 0
    ew = dg.ExpertWeights(P, P, P, P, None, P, None, P, None)
    sw = dg.SharedWeights(P, P, P)
    assert lib.moe_forward(ctypes.byref(d), P, P, P, None, ctypes.byref(ew), ctypes.byref(sw), P, None, None, P,
                           need - 1, None) == dg.MOE_ERR_WORKSPACE


def test_forward_workspace_too_small(lib):
    d = desc()
    need = lib.moe_forward_workspace_size(ctypes.byref(d))
    assert need > 0
    assert forward(lib, d, ws_bytes=need - 1) == dg.MOE_ERR_WORKSPACE


def test_forward_unsupported_shapes(lib):
    assert forward(lib, desc(H=96)) == dg.MOE_ERR_UNSUPPORTED     # bf16 needs multiples of 64
    assert forward(lib, desc(E=2048, n_group=1)) == dg.MOE_ERR_UNSUPPORTED
    assert forward(lib, desc(E=128, top_k=65, n_group=1)) == dg.MOE_ERR_UNSUPPORTED


def test_workspace_size_rejects_invalid(lib):
    assert lib.moe_forward_workspace_size(None) == 0
    d = desc(top_k=0)
    assert lib.moe_forward_workspace_size(ctypes.byref(d)) == 0


def test_forward_zero_tokens_is_a_noop(lib):
    assert forward(lib, desc(T=0), x=None, y=None) == dg.MOE_OK


def test_workspace_grows_with_tokens(lib):
    a = lib.moe_forward_workspace_size(ctypes.byref(desc(T=16)))
    b = lib.moe_forward_workspace_size(ctypes.byref(desc(T=1024)))
    assert b > a > 0


def route_softmax(lib, T=4, E=8, K=2, logits=P, inds=P, scores=P):
    return lib.moe_route_softmax(logits, T, E, K, inds, scores, None)


SOFTMAX_REJECTS = {
    "top_k_zero": dict(K=0),
    "top_k_gt_E": dict(K=9),
    "zero_E": dict(E=0, K=1),
    "negative_T": dict(T=-1),
    "null_logits": dict(logits=None),
    "null_inds": dict(inds=None),
    "null_scores": dict(scores=None),
    "misaligned_scores": dict(scores=P + 4),
}


@pytest.mark.parametrize("name", sorted(SOFTMAX_REJECTS))
def test_route_softmax_reject_matrix(lib, name):
    assert route_softmax(lib, **SOFTMAX_REJECTS[name]) == dg.MOE_ERR_INVALID


def test_route_softmax_limits_and_empty(lib):
    assert route_softmax(lib, E=2048, K=2) == dg.MOE_ERR_UNSUPPORTED
    assert route_softmax(lib, E=256, K=65) == dg.MOE_ERR_UNSUPPORTED
    assert route_softmax(lib, T=0, logits=None, inds=None, scores=None) == dg.MOE_OK


def _forward_raw(lib, d, bias=P, sgate=None, shared=True):
    ew = dg.ExpertWeights(P, P, P)
    sw = dg.SharedWeights(P, P, P, sgate) if shared else None
    need = lib.moe_forward_workspace_size(ctypes.byref(d))
    return lib.moe_forward(ctypes.byref(d), None, P, bias, None, ctypes.byref(ew),
                           None if sw is None else ctypes.byref(sw), None, None, None, P, need, None)


def test_forward_route_kind_validation(lib):
    # T = 0 passes validation without touching the GPU, so only the checks are exercised
    soft = dict(T=0, route_kind=dg.MOE_ROUTE_SOFTMAX)
    assert _forward_raw(lib, desc(**soft), bias=None) == dg.MOE_OK           # bias optional for softmax
    assert _forward_raw(lib, desc(T=0), bias=None) == dg.MOE_ERR_INVALID     # required for the DeepSeek gate
    assert _forward_raw(lib, desc(**soft, n_group=3), bias=None) == dg.MOE_OK  # group params ignored
    assert _forward_raw(lib, desc(**soft, top_k=9)) == dg.MOE_ERR_INVALID
    assert _forward_raw(lib, desc(**soft, top_k=65, E=128)) == dg.MOE_ERR_UNSUPPORTED
    assert _forward_raw(lib, desc(T=0, route_kind=2)) == dg.MOE_ERR_INVALID
    assert _forward_raw(lib, desc(T=0), sgate=P) == dg.MOE_OK
    assert _forward_raw(lib, desc(T=0), sgate=P + 2) == dg.MOE_ERR_INVALID  # misaligned gate vector


def test_dense_rejects(lib):
    f = lib.moe_dense_mlp
    need = lib.moe_dense_workspace_size(16, 128, 64, 1)
    assert need > 0
    assert lib.moe_dense_workspace_size(16, 96, 64, 1) == 0      # bf16 needs multiples of 64
    assert lib.moe_dense_workspace_size(-1, 128, 64, 1) == 0
    assert f(16, 128, 64, 1, None, P, P, P, P, P, need, None) == dg.MOE_ERR_INVALID
    assert f(16, 128, 64, 1, P, None, P, P, P, P, need, None) == dg.MOE_ERR_INVALID
    assert f(16, 128, 64, 1, P, P, P, P, None, P, need, None) == dg.MOE_ERR_INVALID
    assert f(16, 128, 64, 5, P, P, P, P, P, P, need, None) == dg.MOE_ERR_INVALID
    assert f(16, 0, 64, 1, P, P, P, P, P, P, need, None) == dg.MOE_ERR_INVALID
    assert f(16, 128, 64, 1, P, P, P, P, P, P + 16, need, None) == dg.MOE_ERR_INVALID  # misaligned workspace
    assert f(16, 128, 64, 1, P, P, P, P, P, P, need - 1, None) == dg.MOE_ERR_WORKSPACE
    assert f(16, 96, 64, 1, P, P, P, P, P, P, need, None) == dg.MOE_ERR_UNSUPPORTED
    assert f(0, 128, 64, 1, None, P, P, P, None, P, need, None) == dg.MOE_OK


def test_forward_static_host_checks(lib):
    """moe_forward_static checks its arguments like moe_forward, then the scratch limit, all before
    any HIP call: an invalid descriptor is -1, a layer needing more than the fixed scratch is -3,
    and zero tokens is a no-op."""
    def static(d, x=P, y=P, shared=True):
        ew = dg.ExpertWeights(P, P, P)
        sw = dg.SharedWeights(P, P, P) if shared else None
        return lib.moe_forward_static(ctypes.byref(d), x, P, P, None, ctypes.byref(ew),
                                      None if sw is None else ctypes.byref(sw), y, None, None, None)
    assert static(desc(top_k=0)) == dg.MOE_ERR_INVALID
    assert static(desc(), x=None) == dg.MOE_ERR_INVALID
    assert static(desc(), shared=False) == dg.MOE_ERR_INVALID
    big = dg.layer_desc(8192, 7168, 256, 2048, 2048, 1, 1, 8, 8, 4, True, 2.5)
    assert lib.moe_forward_workspace_size(ctypes.byref(big)) > dg.MOE_STATIC_SCRATCH_BYTES
    assert static(big) == dg.MOE_ERR_WORKSPACE
    assert static(desc(T=0), x=None, y=None) == dg.MOE_OK
