"""The moe_forward binding checks every tensor against the layer descriptor before any launch
(CPU only: the checks need no device).  The kernels index x, y, the router, the expert and
shared weights, the 4-bit / fp8 side arrays and the route outputs by the descriptor's sizes, so
a tensor that does not match would be read or written out of bounds on the device; the binding
refuses such a call with MOE_ERR_INVALID (-1), the gate page's reject convention."""
import pytest
import torch

import deepseek_gate_expert_amd as dg

T, H, E, I, IS, K = 8, 128, 4, 64, 64, 2


def desc(expert=dg.MOE_BF16, act=dg.MOE_BF16, Is=IS, kind=dg.MOE_ROUTE_DEEPSEEK):
    return dg.layer_desc(T, H, E, I, Is, act, expert, K, 2, 1, True, 2.5, kind)


def tensors(expert="bf16", act=torch.bfloat16, Is=IS):
    a = dict(x=torch.zeros(T, H, dtype=act), y=torch.zeros(T, H, dtype=act), router_w=torch.zeros(E, H, dtype=act),
             bias=torch.zeros(E), logit_offset=None, inds_out=torch.zeros(T, K, dtype=torch.int32),
             scores_out=torch.zeros(T, K))
    ex = {}
    for nm, o, i in (("gate", I, H), ("up", I, H), ("down", H, I)):
        if expert == "q4":
            ex[nm] = torch.zeros(E, o, i // 8, dtype=torch.int32)
            ex["s_" + nm] = torch.zeros(E, o, i // 64, dtype=torch.bfloat16)
            ex["b_" + nm] = torch.zeros(E, o, i // 64, dtype=torch.bfloat16)
        elif expert == "fp8":
            ex[nm] = torch.zeros(E, o, i, dtype=torch.uint8)
            ex["s_" + nm] = torch.zeros(E, (o + 127) // 128, (i + 127) // 128)
        else:
            ex[nm] = torch.zeros(E, o, i, dtype=act)
    sh = None if Is == 0 else {"gate": torch.zeros(Is, H, dtype=act), "up": torch.zeros(Is, H, dtype=act),
                               "down": torch.zeros(H, Is, dtype=act)}
    a["experts"], a["shared"] = ex, sh
    return a


def errors(d, a):
    return dg.forward_arg_errors(d, a["x"], a["router_w"], a["bias"], a["experts"], a["shared"], a["y"],
                                 a["logit_offset"], a["inds_out"], a["scores_out"])


@pytest.mark.parametrize("expert,code,act", [("bf16", dg.MOE_BF16, torch.bfloat16), ("q4", dg.MOE_Q4G64, torch.bfloat16),
                                             ("fp8", dg.MOE_FP8, torch.bfloat16), ("f32", dg.MOE_F32, torch.float32)])
def test_matching_tensors_pass(expert, code, act):
    d = desc(expert=code, act=dg.MOE_F32 if act == torch.float32 else dg.MOE_BF16)
    assert errors(d, tensors(expert, act)) == []


def _mut(a, path, value):
    if isinstance(path, tuple):
        a[path[0]] = dict(a[path[0]])
        a[path[0]][path[1]] = value
    else:
        a[path] = value
    return a


BAD = {
    "x_too_few_rows": ("bf16", "x", torch.zeros(T - 1, H, dtype=torch.bfloat16)),
    "x_wrong_dtype": ("bf16", "x", torch.zeros(T, H)),
    "y_too_narrow": ("bf16", "y", torch.zeros(T, H - 64, dtype=torch.bfloat16)),
    "y_fp32_with_bf16_desc": ("bf16", "y", torch.zeros(T, H)),
    "router_transposed": ("bf16", "router_w", torch.zeros(H, E, dtype=torch.bfloat16)),
    "bias_rank2": ("bf16", "bias", torch.zeros(1, E)),
    "bias_missing_deepseek": ("bf16", "bias", None),
    "bias_wrong_length": ("bf16", "bias", torch.zeros(E + 1)),
    "offset_bf16": ("bf16", "logit_offset", torch.zeros(E, dtype=torch.bfloat16)),
    "inds_int64": ("bf16", "inds_out", torch.zeros(T, K, dtype=torch.int64)),
    "scores_short": ("bf16", "scores_out", torch.zeros(T, K - 1)),
    "gate_fewer_experts": ("bf16", ("experts", "gate"), torch.zeros(E - 1, I, H, dtype=torch.bfloat16)),
    "down_transposed": ("bf16", ("experts", "down"), torch.zeros(E, I, H, dtype=torch.bfloat16)),
    "q4_codes_unpacked": ("q4", ("experts", "up"), torch.zeros(E, I, H, dtype=torch.int32)),
    "q4_scale_fp32": ("q4", ("experts", "s_down"), torch.zeros(E, H, I // 64)),
    "q4_offset_missing": ("q4", ("experts", "b_gate"), None),
    "fp8_codes_bf16": ("fp8", ("experts", "gate"), torch.zeros(E, I, H, dtype=torch.bfloat16)),
    "fp8_scale_per_row": ("fp8", ("experts", "s_up"), torch.zeros(E, I, (H + 127) // 128)),
    "shared_down_transposed": ("bf16", ("shared", "down"), torch.zeros(IS, H, dtype=torch.bfloat16)),
    "shared_gate_vector_long": ("bf16", ("shared", "sgate"), torch.zeros(H + 1, dtype=torch.bfloat16)),
    "shared_missing": ("bf16", "shared", None),
}


@pytest.mark.parametrize("name", sorted(BAD))
def test_mismatch_is_reported(name):
    expert, path, value = BAD[name]
    code = {"bf16": dg.MOE_BF16, "q4": dg.MOE_Q4G64, "fp8": dg.MOE_FP8}[expert]
    a = _mut(tensors(expert), path, value)
    errs = errors(desc(expert=code), a)
    assert len(errs) >= 1, name


def test_shared_weights_without_shared_expert():
    a = tensors()
    assert errors(desc(Is=0), a)  # desc says no shared expert but weights are given
    a["shared"] = None
    assert errors(desc(Is=0), a) == []


def test_softmax_gate_may_omit_bias():
    a = tensors()
    a["bias"] = None
    assert errors(desc(kind=dg.MOE_ROUTE_SOFTMAX), a) == []


def test_non_contiguous_rejected():
    a = tensors()
    a["x"] = torch.zeros(H, T, dtype=torch.bfloat16).t()
    assert any("contiguous" in e for e in errors(desc(), a))


def test_moe_forward_returns_invalid_before_any_call():
    """On CPU tensors the call is refused by the checks; the library is never entered."""
    a = tensors()
    a["y"] = torch.zeros(T + 1, H, dtype=torch.bfloat16)
    rc = dg.moe_forward(desc(), a["x"], a["router_w"], a["bias"], a["experts"], a["shared"], a["y"])
    assert rc == dg.MOE_ERR_INVALID
