"""MI355X (gfx950) DeepSeek-style mixture-of-experts layer forward.

Thin ctypes binding of ``libdsmoe.so`` (hand-written HIP, built by ``build.py``).  The names
and arguments mirror the C ABI in ``include/dsmoe.h``; this module only checks tensor
properties (device, dtype, shape, contiguity) and passes device pointers, sizes and the current
HIP stream.  Every step of the layer runs in the library's kernels; there is no fallback: if
the library is missing, importing the functions works but calling them raises.

Tensor conventions: torch tensors on a ROCm device; bf16 data as ``torch.bfloat16``; 4-bit
expert weights as ``torch.int32``/``torch.uint32`` words with bf16 scales and offsets.
Return values are the library's codes (``MOE_OK`` == 0), never exceptions, so the
validation matrix can be tested as the pages test it (rejects return -1 and leave the outputs
untouched).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_HIP, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_Q4G64, MOE_FP8 = 0, 1, 2, 3
MOE_MAX_EXPERTS, MOE_MAX_TOP_K = 1024, 64
MOE_ROUTE_DEEPSEEK, MOE_ROUTE_SOFTMAX = 0, 1
MOE_STAGE_ROUTER, MOE_STAGE_ROUTE, MOE_STAGE_DISPATCH, MOE_STAGE_GEMM1, MOE_STAGE_GEMM2, MOE_STAGE_COMBINE = range(6)
EXPORTS = ("moe_router_logits", "moe_route_deepseek", "moe_route_softmax", "moe_dispatch_workspace_size", "moe_dispatch",
           "moe_forward_workspace_size", "moe_forward", "moe_dense_workspace_size", "moe_dense_mlp",
           "moe_set_stage_events", "moe_strerror", "moe_forward_static")
MOE_STATIC_SCRATCH_BYTES = 64 * 1024 * 1024


class RouteParams(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32), ("I", ctypes.c_int32),
                ("I_shared", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
                ("route", RouteParams), ("route_kind", ctypes.c_int32)]


class ExpertWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_gate", "w_up", "w_down", "s_gate", "b_gate", "s_up", "b_up", "s_down", "b_down")]


class SharedWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gate", "w_up", "w_down", "w_sgate")]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m deepseek_gate_expert_amd.build`")
        # PyTorch ships its own HIP runtime with the same soname as the system one; loading torch
        # first makes the library bind to that runtime, so both share one device context.  (Loaded
        # the other way round, torch would pick up the system runtime and the library's launches
        # would not reach the device torch uses.)
        import torch  # noqa: F401
        lib = ctypes.CDLL(path)
        p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.moe_strerror.restype = ctypes.c_char_p
        lib.moe_strerror.argtypes = [ctypes.c_int]
        lib.moe_router_logits.restype = ctypes.c_int
        lib.moe_router_logits.argtypes = [p, p, i32, i64, i32, i32, p, p, p]
        lib.moe_route_deepseek.restype = ctypes.c_int
        lib.moe_route_deepseek.argtypes = [p, i64, i32, p, i64, ctypes.POINTER(RouteParams), p, p, p]
        lib.moe_dense_workspace_size.restype = sz
        lib.moe_dense_workspace_size.argtypes = [i64, i32, i32, i32]
        lib.moe_dense_mlp.restype = ctypes.c_int
        lib.moe_dense_mlp.argtypes = [i64, i32, i32, i32, p, p, p, p, p, p, sz, p]
        lib.moe_route_softmax.restype = ctypes.c_int
        lib.moe_route_softmax.argtypes = [p, i64, i32, i32, p, p, p]
        lib.moe_dispatch_workspace_size.restype = sz
        lib.moe_dispatch_workspace_size.argtypes = [i64, i32, i32]
        lib.moe_dispatch.restype = ctypes.c_int
        lib.moe_dispatch.argtypes = [p, i64, i32, i32, p, p, p, p, p, sz, p]
        lib.moe_forward_workspace_size.restype = sz
        lib.moe_forward_workspace_size.argtypes = [ctypes.POINTER(LayerDesc)]
        lib.moe_forward.restype = ctypes.c_int
        lib.moe_forward.argtypes = [ctypes.POINTER(LayerDesc), p, p, p, p, ctypes.POINTER(ExpertWeights),
                                    ctypes.POINTER(SharedWeights), p, p, p, p, sz, p]
        lib.moe_forward_static.restype = ctypes.c_int
        lib.moe_forward_static.argtypes = [ctypes.POINTER(LayerDesc), p, p, p, p, ctypes.POINTER(ExpertWeights),
                                           ctypes.POINTER(SharedWeights), p, p, p, p]
        lib.moe_set_stage_events.restype = ctypes.c_int
        lib.moe_set_stage_events.argtypes = [i32, p, i32]
        _lib = lib
    return _lib


def _ptr(t) -> Optional[int]:
    return None if t is None else (t.data_ptr() or None)


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream or None


def _is_dev(t) -> bool:
    return t is None or t.is_cuda


def _same_device(*ts) -> bool:
    devs = {t.device for t in ts if t is not None}
    return len(devs) <= 1 and all(_is_dev(t) for t in ts)


def _contig(*ts) -> bool:
    return all(t is None or t.is_contiguous() for t in ts)


def act_code(dtype) -> int:
    import torch
    if dtype == torch.float32:
        return MOE_F32
    if dtype == torch.bfloat16:
        return MOE_BF16
    raise ValueError(f"unsupported activation dtype {dtype}")


def route_params(top_k, n_group=1, topk_group=1, norm_topk_prob=True, routed_scaling_factor=1.0) -> RouteParams:
    return RouteParams(int(top_k), int(n_group), int(topk_group), int(bool(norm_topk_prob)),
                       float(routed_scaling_factor))


def moe_strerror(code: int) -> str:
    return load_library().moe_strerror(int(code)).decode()


def moe_router_logits(x, router_w, logits, logit_offset=None, stream=None) -> int:
    """logits[T, E] (fp32) = x[T, H] @ router_w[E, H]^T (+ logit_offset[E]), fixed fp32 order."""
    import torch
    if x.dim() != 2 or router_w.dim() != 2 or logits.dim() != 2 or logits.dtype != torch.float32:
        return MOE_ERR_INVALID
    if x.dtype != router_w.dtype or not _same_device(x, router_w, logits, logit_offset) or \
            not _contig(x, router_w, logits, logit_offset):
        return MOE_ERR_INVALID
    T, H = x.shape
    E = router_w.shape[0]
    if router_w.shape[1] != H or tuple(logits.shape) != (T, E):
        return MOE_ERR_INVALID
    if logit_offset is not None and (logit_offset.dtype != torch.float32 or tuple(logit_offset.shape) != (E,)):
        return MOE_ERR_INVALID
    return load_library().moe_router_logits(_ptr(x), _ptr(router_w), act_code(x.dtype), T, H, E,
                                            _ptr(logit_offset), _ptr(logits), _stream(stream))


def moe_route_deepseek(logits, bias, inds, scores, top_k, n_group=1, topk_group=1, norm_topk_prob=True,
                       routed_scaling_factor=1.0, stream=None) -> int:
    """DeepSeek gate on logits [..., E] (leading dims flatten to rows).  inds (int32) and
    scores (fp32) are [..., top_k] and are written only on success."""
    import torch
    if logits.dim() < 1 or logits.dtype != torch.float32:
        return MOE_ERR_INVALID
    # the reviewed contract: bias is rank-1 [E], fp32, on the logits' device
    if bias is None or bias.dim() != 1 or bias.dtype != torch.float32:
        return MOE_ERR_INVALID
    if inds.dtype != torch.int32 or scores.dtype != torch.float32:
        return MOE_ERR_INVALID
    if not _same_device(logits, bias, inds, scores) or not _contig(logits, bias, inds, scores):
        return MOE_ERR_INVALID
    E = logits.shape[-1]
    T = logits.numel() // E if E > 0 else 0
    if inds.numel() != T * max(int(top_k), 0) or scores.numel() != inds.numel():
        return MOE_ERR_INVALID
    p = route_params(top_k, n_group, topk_group, norm_topk_prob, routed_scaling_factor)
    return load_library().moe_route_deepseek(_ptr(logits), T, E, _ptr(bias), bias.shape[0], ctypes.byref(p),
                                             _ptr(inds), _ptr(scores), _stream(stream))


def moe_route_softmax(logits, inds, scores, top_k, stream=None) -> int:
    """Softmax gate on logits [..., E] (leading dims flatten to rows).  inds (int32) and scores
    (fp32) are [..., top_k] and are written only on success."""
    import torch
    if logits.dim() < 1 or logits.dtype != torch.float32:
        return MOE_ERR_INVALID
    if inds.dtype != torch.int32 or scores.dtype != torch.float32:
        return MOE_ERR_INVALID
    if not _same_device(logits, inds, scores) or not _contig(logits, inds, scores):
        return MOE_ERR_INVALID
    E = logits.shape[-1]
    T = logits.numel() // E if E > 0 else 0
    if inds.numel() != T * max(int(top_k), 0) or scores.numel() != inds.numel():
        return MOE_ERR_INVALID
    return load_library().moe_route_softmax(_ptr(logits), T, E, int(top_k), _ptr(inds), _ptr(scores),
                                            _stream(stream))


def moe_dispatch_workspace_size(T: int, K: int, E: int) -> int:
    return int(load_library().moe_dispatch_workspace_size(T, K, E))


def moe_dispatch(inds, E, counts, offsets, sorted_slot, slot_row, workspace, stream=None) -> int:
    """Stable counting sort of the T*K slots of inds [T, K] by expert (see dsmoe.h)."""
    import torch
    ts = (inds, counts, offsets, sorted_slot, slot_row)
    if any(t.dtype != torch.int32 for t in ts) or inds.dim() != 2:
        return MOE_ERR_INVALID
    if not _same_device(*ts, workspace) or not _contig(*ts):
        return MOE_ERR_INVALID
    T, K = inds.shape
    if counts.numel() != E or offsets.numel() != E + 1 or sorted_slot.numel() != T * K or slot_row.numel() != T * K:
        return MOE_ERR_INVALID
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return load_library().moe_dispatch(_ptr(inds), T, K, E, _ptr(counts), _ptr(offsets), _ptr(sorted_slot),
                                       _ptr(slot_row), _ptr(workspace), nbytes, _stream(stream))


def layer_desc(T, H, E, I, I_shared, act_dtype, expert_dtype, top_k, n_group=1, topk_group=1, norm_topk_prob=True,
               routed_scaling_factor=1.0, route_kind=MOE_ROUTE_DEEPSEEK) -> LayerDesc:
    return LayerDesc(int(T), int(H), int(E), int(I), int(I_shared), int(act_dtype), int(expert_dtype),
                     route_params(top_k, n_group, topk_group, norm_topk_prob, routed_scaling_factor),
                     int(route_kind))


def moe_forward_workspace_size(desc: LayerDesc) -> int:
    return int(load_library().moe_forward_workspace_size(ctypes.byref(desc)))


_ACT_TORCH = {MOE_F32: "float32", MOE_BF16: "bfloat16"}


def _shape_err(name, t, shape, dtypes) -> Optional[str]:
    if t is None:
        return f"{name} is missing"
    if tuple(t.shape) != tuple(shape):
        return f"{name} has shape {tuple(t.shape)}, the descriptor needs {tuple(shape)}"
    if str(t.dtype).replace("torch.", "") not in dtypes:
        return f"{name} has dtype {t.dtype}, the descriptor needs one of {dtypes}"
    return None


def forward_arg_errors(desc: LayerDesc, x, router_w, bias, experts: dict, shared: Optional[dict], y,
                       logit_offset=None, inds_out=None, scores_out=None) -> list:
    """Every mismatch between the tensors and the descriptor that moe_forward would hand to the
    kernels (shape, dtype, contiguity), as messages; empty when they agree.  The kernels index
    these buffers by the descriptor's sizes, so a mismatch here would read or write out of
    bounds on the device."""
    errs = []
    T, H, E, I, Is, K = int(desc.T), int(desc.H), int(desc.E), int(desc.I), int(desc.I_shared), int(desc.route.top_k)
    act = _ACT_TORCH.get(int(desc.act_dtype))
    if act is None:
        return [f"unsupported act_dtype {int(desc.act_dtype)}"]
    wdt = int(desc.expert_dtype)
    A = (act,)
    for name, t, shape, dts in (("x", x, (T, H), A), ("y", y, (T, H), A), ("router_w", router_w, (E, H), A)):
        errs.append(_shape_err(name, t, shape, dts))
    if bias is not None or int(desc.route_kind) == MOE_ROUTE_DEEPSEEK:
        errs.append(_shape_err("bias", bias, (E,), ("float32",)))
    if logit_offset is not None:
        errs.append(_shape_err("logit_offset", logit_offset, (E,), ("float32",)))
    if inds_out is not None:
        errs.append(_shape_err("inds_out", inds_out, (T, K), ("int32",)))
    if scores_out is not None:
        errs.append(_shape_err("scores_out", scores_out, (T, K), ("float32",)))
    mats = (("gate", I, H), ("up", I, H), ("down", H, I))
    for nm, o, i in mats:
        t = experts.get(nm)
        if wdt in (MOE_F32, MOE_BF16):
            errs.append(_shape_err(f"experts[{nm!r}]", t, (E, o, i), (_ACT_TORCH[wdt],)))
        elif wdt == MOE_Q4G64:
            errs.append(_shape_err(f"experts[{nm!r}]", t, (E, o, i // 8), ("int32", "uint32")))
            for side in ("s_", "b_"):
                errs.append(_shape_err(f"experts[{side + nm!r}]", experts.get(side + nm), (E, o, i // 64),
                                       ("bfloat16",)))
        elif wdt == MOE_FP8:
            errs.append(_shape_err(f"experts[{nm!r}]", t, (E, o, i), ("uint8",)))
            errs.append(_shape_err(f"experts['s_{nm}']", experts.get("s_" + nm), (E, (o + 127) // 128, (i + 127) // 128),
                                   ("float32",)))
        else:
            return [f"unsupported expert_dtype {wdt}"]
    if Is > 0:
        if shared is None:
            errs.append("shared weights are missing (I_shared > 0)")
        else:
            for nm, shape in (("gate", (Is, H)), ("up", (Is, H)), ("down", (H, Is))):
                errs.append(_shape_err(f"shared[{nm!r}]", shared.get(nm), shape, A))
            if shared.get("sgate") is not None:
                errs.append(_shape_err("shared['sgate']", shared.get("sgate"), (H,), A))
    elif shared is not None:
        errs.append("shared weights given but I_shared == 0")
    errs = [e for e in errs if e]
    tensors = [x, router_w, bias, y, logit_offset, inds_out, scores_out] + list(experts.values()) + \
        ([] if shared is None else list(shared.values()))
    if not _contig(*tensors):
        errs.append("every tensor must be contiguous")
    return errs


def moe_forward(desc: LayerDesc, x, router_w, bias, experts: dict, shared: Optional[dict], y, logit_offset=None,
                inds_out=None, scores_out=None, workspace=None, stream=None) -> int:
    """Whole MoE layer forward (see dsmoe.h).  experts: dict with 'gate', 'up', 'down' (and for
    4-bit weights 's_gate', 'b_gate', 's_up', 'b_up', 's_down', 'b_down'; for fp8 weights the
    fp32 block scales 's_gate', 's_up', 's_down'); shared: dict with
    'gate', 'up', 'down' (and optionally 'sgate', the [H] gate vector) or None.  bias may be
    None with the softmax gate.  Every tensor's shape and dtype is checked against the
    descriptor first (forward_arg_errors); a mismatch returns MOE_ERR_INVALID with no launch."""
    if forward_arg_errors(desc, x, router_w, bias, experts, shared, y, logit_offset, inds_out, scores_out):
        return MOE_ERR_INVALID
    if not _contig(workspace):
        return MOE_ERR_INVALID
    ew = ExpertWeights(*[_ptr(experts.get(k)) for k in
                         ("gate", "up", "down", "s_gate", "b_gate", "s_up", "b_up", "s_down", "b_down")])
    sw = None
    if shared is not None:
        sw = SharedWeights(_ptr(shared["gate"]), _ptr(shared["up"]), _ptr(shared["down"]), _ptr(shared.get("sgate")))
    tensors = [x, router_w, bias, y, logit_offset, inds_out, scores_out, workspace] + \
        [v for v in experts.values()] + ([] if shared is None else list(shared.values()))
    if not _same_device(*tensors):
        return MOE_ERR_INVALID
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return load_library().moe_forward(ctypes.byref(desc), _ptr(x), _ptr(router_w), _ptr(bias), _ptr(logit_offset),
                                      ctypes.byref(ew), None if sw is None else ctypes.byref(sw), _ptr(y),
                                      _ptr(inds_out), _ptr(scores_out), _ptr(workspace), nbytes, _stream(stream))


def moe_forward_static(desc: LayerDesc, x, router_w, bias, experts: dict, shared: Optional[dict], y,
                       logit_offset=None, inds_out=None, scores_out=None, stream=None) -> int:
    """moe_forward with the library's own fixed scratch instead of a workspace (see dsmoe.h):
    for callers that cannot allocate; MOE_ERR_WORKSPACE when the layer needs more scratch than
    MOE_STATIC_SCRATCH_BYTES.  Same argument checks as moe_forward."""
    if forward_arg_errors(desc, x, router_w, bias, experts, shared, y, logit_offset, inds_out, scores_out):
        return MOE_ERR_INVALID
    ew = ExpertWeights(*[_ptr(experts.get(k)) for k in
                         ("gate", "up", "down", "s_gate", "b_gate", "s_up", "b_up", "s_down", "b_down")])
    sw = None
    if shared is not None:
        sw = SharedWeights(_ptr(shared["gate"]), _ptr(shared["up"]), _ptr(shared["down"]), _ptr(shared.get("sgate")))
    tensors = [x, router_w, bias, y, logit_offset, inds_out, scores_out] + \
        [v for v in experts.values()] + ([] if shared is None else list(shared.values()))
    if not _same_device(*tensors):
        return MOE_ERR_INVALID
    return load_library().moe_forward_static(ctypes.byref(desc), _ptr(x), _ptr(router_w), _ptr(bias),
                                             _ptr(logit_offset), ctypes.byref(ew),
                                             None if sw is None else ctypes.byref(sw), _ptr(y), _ptr(inds_out),
                                             _ptr(scores_out), _stream(stream))


def moe_dense_workspace_size(T: int, H: int, I: int, act_dtype: int) -> int:
    return int(load_library().moe_dense_workspace_size(int(T), int(H), int(I), int(act_dtype)))


def moe_dense_mlp(x, w_gate, w_up, w_down, y, workspace=None, stream=None) -> int:
    """Dense SwiGLU MLP (see dsmoe.h): x, y [T, H]; w_gate, w_up [I, H]; w_down [H, I]; one
    activation dtype.  Allocates the workspace when none is given."""
    import torch
    if x.dim() != 2 or w_gate.dim() != 2 or w_up.shape != w_gate.shape or w_down.dim() != 2:
        return MOE_ERR_INVALID
    T, H = x.shape
    I = w_gate.shape[0]
    if w_gate.shape[1] != H or tuple(w_down.shape) != (H, I) or tuple(y.shape) != (T, H):
        return MOE_ERR_INVALID
    if len({t.dtype for t in (x, w_gate, w_up, w_down, y)}) != 1:
        return MOE_ERR_INVALID
    if not _contig(x, w_gate, w_up, w_down, y, workspace) or not _same_device(x, w_gate, w_up, w_down, y, workspace):
        return MOE_ERR_INVALID
    act = act_code(x.dtype)
    if workspace is None:
        need = moe_dense_workspace_size(T, H, I, act)
        if need == 0:
            return load_library().moe_dense_mlp(T, H, I, act, _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                                _ptr(y), None, 0, _stream(stream))
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    nbytes = workspace.numel() * workspace.element_size()
    return load_library().moe_dense_mlp(T, H, I, act, _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y),
                                        _ptr(workspace), nbytes, _stream(stream))


def moe_set_stage_events(stage: int, events, n_pairs: int) -> int:
    """Measurement hook (see dsmoe.h): `events` is a ctypes array of 2*n_pairs hipEvent_t
    handles; stage -1 clears."""
    return load_library().moe_set_stage_events(int(stage), events, int(n_pairs))
