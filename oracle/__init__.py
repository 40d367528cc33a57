"""CPU oracle of the DeepSeek-style MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The GPU library never links, loads or calls it, and the two
share no code: the oracle's arithmetic is in ``oracle.c`` (plain C, built with gcc,
``-ffp-contract=off``), this module only marshals numpy arrays into it.

Every function cites the passage it follows in ``oracle.c``; the page titles are:
  * "feat(engine): E1 DeepSeek-style MoE gate (sigmoid, group top-k, bias) (#108)"
    (gate API, algorithm, reviews);
  * "Epic: Engine Inference Core Stage E - MoE + hybrid families" (expert dispatch
    through gather_mm / gather_qmm, sigmoid gating with group selection, shared experts
    always active).

Parity pins: every function here is pinned by CPU tests in ``tests/test_oracle_*.py``
(closed forms, invariants the pages state, brute force on tiny inputs, an exhaustive
accuracy sweep of the fp32 exponential).  None is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

DT_F32, DT_BF16, DT_Q4, DT_FP8 = 0, 1, 2, 3
_DT = {"f32": DT_F32, "bf16": DT_BF16, "q4": DT_Q4, "fp8": DT_FP8}


def _digest(cmd) -> str:
    h = hashlib.sha256(" ".join(os.path.basename(c) for c in cmd).encode())
    for f in ['oracle.c', 'oracle.h']:
        with open(os.path.join(_HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def build(force: bool = False) -> str:
    """Compile liboracle.so (gcc, OpenMP, no fast-math, no fp contraction).
    Rebuilds when forced, when the library is missing, or when its sources or flags changed
    since it was built (sha256 stamp beside it)."""
    cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-mavx2", "-mfma", "-Wall", "-Wno-unknown-pragmas",
           os.path.join(_HERE, "oracle.c"), "-o", _SO + ".tmp", "-lm"]
    stamp = _SO + ".sha256"
    digest = _digest(cmd)
    try:
        with open(stamp) as fh:
            current = os.path.exists(_SO) and fh.read().strip() == digest
    except OSError:
        current = False
    if force or not current:
        subprocess.check_call(cmd)
        os.replace(_SO + ".tmp", _SO)
        with open(stamp, "w") as fh:
            fh.write(digest + "\n")
    return _SO


class RouteParams(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float)]


class Layer(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32), ("I", ctypes.c_int32),
                ("Is", ctypes.c_int32), ("act", ctypes.c_int32), ("expert", ctypes.c_int32),
                ("route", RouteParams)] + [(n, ctypes.c_void_p) for n in (
                    "x", "router", "bias", "offset", "wg", "wu", "wd", "sg", "bg", "su", "bu", "sd", "bd",
                    "swg", "swu", "swd")] + [("route_kind", ctypes.c_int32), ("sgate", ctypes.c_void_p)]


_lib = None


def _L():
    global _lib
    if _lib is None:
        # DSMOE_ORACLE_LIB: an alternative build of the same source (the sanitizer test builds one with
        # AddressSanitizer / UndefinedBehaviorSanitizer and runs the pins against it)
        path = os.environ.get("DSMOE_ORACLE_LIB")
        if not path:
            path = build()
        lib = ctypes.CDLL(path)
        p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.oracle_exp.restype = ctypes.c_float
        lib.oracle_exp.argtypes = [ctypes.c_float]
        lib.oracle_sigmoid.restype = ctypes.c_float
        lib.oracle_sigmoid.argtypes = [ctypes.c_float]
        lib.oracle_router.restype = None
        lib.oracle_router.argtypes = [p, p, i32, i64, i32, i32, p, p]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_route.argtypes = [p, i64, i32, p, ctypes.POINTER(RouteParams), p, p]
        lib.oracle_route_softmax.restype = ctypes.c_int
        lib.oracle_route_softmax.argtypes = [p, i64, i32, i32, p, p]
        lib.oracle_e4m3.restype = ctypes.c_double
        lib.oracle_e4m3.argtypes = [ctypes.c_uint8]
        lib.oracle_swiglu.restype = None
        lib.oracle_swiglu.argtypes = [p, i32, i32, i32] + [p] * 9 + [p]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [ctypes.POINTER(Layer), p, i64, p, p, p, p]
        lib.oracle_dense_mlp.restype = ctypes.c_int
        lib.oracle_dense_mlp.argtypes = [p, i32, i64, i32, i32, p, p, p, p]
        lib.oracle_dispatch.restype = ctypes.c_int
        lib.oracle_dispatch.argtypes = [p, i64, i32, i32, p, p, p, p]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_L().oracle_num_threads())


def lib_path() -> str:
    _L()
    return _SO


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def params(top_k, n_group=1, topk_group=1, norm=True, rsf=1.0) -> RouteParams:
    return RouteParams(int(top_k), int(n_group), int(topk_group), int(bool(norm)), float(rsf))


def exp(x: float) -> float:
    return float(_L().oracle_exp(float(x)))


def sigmoid(x) -> np.ndarray:
    x = np.asarray(x, np.float32)
    f = _L().oracle_sigmoid
    return np.array([f(float(v)) for v in x.ravel()], np.float32).reshape(x.shape)


def router(x: np.ndarray, w: np.ndarray, dtype: str, offset: Optional[np.ndarray] = None) -> np.ndarray:
    T, H = x.shape
    E = w.shape[0]
    out = np.empty((T, E), np.float32)
    off = None if offset is None else np.ascontiguousarray(offset, np.float32)
    _L().oracle_router(_p(x), _p(w), _DT[dtype], T, H, E, _p(off), _p(out))
    return out


def route(logits: np.ndarray, bias: np.ndarray, p: RouteParams):
    """Returns (rc, inds, scores); on rc != 0 the output arrays are the untouched sentinels."""
    logits = np.ascontiguousarray(logits, np.float32)
    E = logits.shape[-1]
    T = logits.size // E if E else 0
    bias = np.ascontiguousarray(bias, np.float32)
    K = max(int(p.top_k), 1)
    inds = np.full((T, K), -7, np.int32)
    scores = np.full((T, K), -7.0, np.float32)
    rc = _L().oracle_route(_p(logits), T, E, _p(bias), ctypes.byref(p), _p(inds), _p(scores))
    return rc, inds, scores


def route_softmax(logits: np.ndarray, top_k: int):
    """Softmax gate; returns (rc, inds, scores) like `route`."""
    logits = np.ascontiguousarray(logits, np.float32)
    E = logits.shape[-1]
    T = logits.size // E if E else 0
    K = max(int(top_k), 1)
    inds = np.full((T, K), -7, np.int32)
    scores = np.full((T, K), -7.0, np.float32)
    rc = _L().oracle_route_softmax(_p(logits), T, E, int(top_k), _p(inds), _p(scores))
    return rc, inds, scores


def e4m3(codes) -> np.ndarray:
    """Values (fp64) of OCP E4M3 codes (uint8), one oracle call per code."""
    c = np.asarray(codes, np.uint8).ravel()
    f = _L().oracle_e4m3
    return np.array([f(int(v)) for v in c], np.float64).reshape(np.shape(codes))


def swiglu(x: np.ndarray, wg, wu, wd, dtype: str, q4: Optional[dict] = None) -> np.ndarray:
    """One expert on one row: W_down(silu(W_gate x) * (W_up x)), fp64.  `q4` holds the
    quantisation side arrays: q4 scales/offsets ('s_*', 'b_*') or fp8 block scales ('s_*')."""
    x = np.ascontiguousarray(x, np.float64)
    H = x.shape[0]
    I = wg.shape[0]
    out = np.empty(H, np.float64)
    q4 = q4 or {}
    _L().oracle_swiglu(_p(x), H, I, _DT[dtype], _p(wg), _p(wu), _p(wd),
                       *[_p(q4.get(k)) for k in ("s_gate", "b_gate", "s_up", "b_up", "s_down", "b_down")],
                       _p(out))
    return out


def dense_mlp(x, wg, wu, wd, act: str) -> np.ndarray:
    """Dense SwiGLU MLP layer on every row of x; fp64 [T, H]."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    I = wg.shape[0]
    y = np.empty((T, H), np.float64)
    keep = [np.ascontiguousarray(a) for a in (wg, wu, wd)]
    rc = _L().oracle_dense_mlp(_p(x), _DT[act], T, H, I, *[_p(a) for a in keep], _p(y))
    if rc != 0:
        raise ValueError(f"oracle_dense_mlp rejected its arguments (rc={rc})")
    return y


def forward(x, router_w, bias, experts: dict, shared: Optional[dict], *, T, H, E, I, Is, K, G, TG, norm,
            rsf, act: str, expert: str, offset: Optional[np.ndarray] = None,
            rows: Optional[Sequence[int]] = None, route_kind: str = "deepseek",
            shared_gate: Optional[np.ndarray] = None):
    """Whole layer; returns (y fp64 [n,H], inds [n,K], scores [n,K], logits [n,E]) for the
    tokens `rows` (all tokens when None).  route_kind: "deepseek" (sigmoid gate with bias and
    groups) or "softmax"; shared_gate: optional [H] vector gating the shared expert."""
    keep = []

    def c(a, dt=None):
        if a is None:
            return None
        a = np.ascontiguousarray(a) if dt is None else np.ascontiguousarray(a, dt)
        keep.append(a)
        return a.ctypes.data

    L = Layer()
    L.T, L.H, L.E, L.I, L.Is = T, H, E, I, Is
    L.act, L.expert = _DT[act], _DT[expert]
    L.route = params(K, G, TG, norm, rsf)
    L.x, L.router, L.bias = c(x), c(router_w), c(bias, np.float32)
    L.offset = c(offset, np.float32)
    L.wg, L.wu, L.wd = c(experts["gate"]), c(experts["up"]), c(experts["down"])
    if expert == "q4":
        L.sg, L.bg = c(experts["s_gate"]), c(experts["b_gate"])
        L.su, L.bu = c(experts["s_up"]), c(experts["b_up"])
        L.sd, L.bd = c(experts["s_down"]), c(experts["b_down"])
    elif expert == "fp8":
        L.sg, L.su, L.sd = (c(experts[k], np.float32) for k in ("s_gate", "s_up", "s_down"))
    if shared is not None and Is > 0:
        L.swg, L.swu, L.swd = c(shared["gate"]), c(shared["up"]), c(shared["down"])
    L.route_kind = {"deepseek": 0, "softmax": 1}[route_kind]
    L.sgate = c(shared_gate)
    rr = None if rows is None else np.ascontiguousarray(np.asarray(rows, np.int64))
    n = T if rr is None else len(rr)
    y = np.empty((n, H), np.float64)
    inds = np.empty((n, K), np.int32)
    scores = np.empty((n, K), np.float32)
    logits = np.empty((n, E), np.float32)
    rc = _L().oracle_forward(ctypes.byref(L), _p(rr), n, _p(y), _p(inds), _p(scores), _p(logits))
    if rc != 0:
        raise ValueError(f"oracle_forward rejected its arguments (rc={rc})")
    return y, inds, scores, logits


def forward_workload(w, x, router_w, bias, experts, shared, offset=None, rows=None, shared_gate=None):
    """`forward` with the shape/route parameters taken from a synth.Workload."""
    return forward(x, router_w, bias, experts, shared, T=w.T, H=w.H, E=w.E, I=w.I, Is=w.Is, K=w.K, G=w.G,
                   TG=w.TG, norm=w.norm, rsf=w.rsf, act=w.act, expert=w.expert, offset=offset, rows=rows,
                   route_kind=getattr(w, "route", "deepseek"), shared_gate=shared_gate)


def dispatch(inds: np.ndarray, E: int):
    """Expert-major grouping of the T*K token slots (slot s = t*K + j), the grouping that the
    gather_mm / gather_qmm expert calls imply ("Epic: Engine Inference Core Stage E - MoE +
    hybrid families", opening paragraph): experts ascending, slots ascending inside an expert.
    Returns (counts [E], offsets [E+1], sorted_slot [T*K], slot_row [T*K]) from the counting
    sort ``oracle_dispatch`` in oracle.c; raises on an index outside [0, E)."""
    inds = np.ascontiguousarray(inds, np.int32)
    if inds.ndim != 2:
        raise ValueError("inds must be [T, K]")
    T, K = inds.shape
    n = T * K
    counts = np.full(E, -7, np.int32)
    offsets = np.full(E + 1, -7, np.int32)
    sorted_slot = np.full(n, -7, np.int32)
    slot_row = np.full(n, -7, np.int32)
    rc = _L().oracle_dispatch(_p(inds), T, max(K, 1), int(E), _p(counts), _p(offsets), _p(sorted_slot),
                              _p(slot_row))
    if rc != 0:
        raise ValueError(f"oracle_dispatch rejected its arguments (rc={rc})")
    return counts, offsets, sorted_slot, slot_row
