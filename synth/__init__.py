"""Seeded synthetic inputs for the DeepSeek-style MoE layer.

This package only generates inputs; it holds none of the layer's arithmetic.
Both the CPU oracle (``oracle/``) and the GPU path read what it produces, so
the two sides see bit-identical inputs.  The generator itself is in
``synth.c`` (counter-based SplitMix64 + Box-Muller, see its header); this
module wraps it and defines the workloads.

Storage conventions (numpy):
  * fp32 tensors are ``float32`` arrays;
  * bf16 tensors are ``uint16`` arrays holding the bf16 bit patterns;
  * 4-bit packed expert weights are ``uint32`` arrays ``[..., out, in/8]``
    (element i of a row at bits ``4*(i%8)`` of word ``i//8``) with bf16
    scale and offset arrays ``[..., out, in/64]``;
  * fp8 expert weights are ``uint8`` OCP E4M3 codes ``[..., out, in]`` with
    fp32 scales ``[..., ceil(out/128), ceil(in/128)]`` (one per 128 x 128 block).
Weight layout is "expert stacking": ``[E, out, in]`` with the input axis
contiguous; the router is ``[E, H]``; shared weights are ``[Is, H]``,
``[Is, H]``, ``[H, Is]``.
"""
from __future__ import annotations

import ctypes
import hashlib
import math
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")

# tensor ids of the counter-based generator
TID_X, TID_ROUTER, TID_BIAS, TID_WG, TID_WU, TID_WD = 1, 2, 3, 4, 5, 6
TID_SWG, TID_SWU, TID_SWD, TID_ZIPF, TID_PLANT, TID_SGATE = 7, 8, 9, 10, 11, 12


def _digest(cmd) -> str:
    h = hashlib.sha256(" ".join(os.path.basename(c) for c in cmd).encode())
    for f in ['synth.c']:
        with open(os.path.join(_HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (host code only).
    Rebuilds when forced, when the library is missing, or when its sources or flags changed
    since it was built (sha256 stamp beside it)."""
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
           os.path.join(_HERE, "synth.c"), "-o", _SO + ".tmp", "-lm"]
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


_lib = None


def _L():
    global _lib
    if _lib is None:
        # DSMOE_SYNTH_LIB: an alternative build of the same source (the sanitizer test builds one with
        # AddressSanitizer / UndefinedBehaviorSanitizer and runs the pins against it)
        path = os.environ.get("DSMOE_SYNTH_LIB")
        if not path:
            path = build()
        lib = ctypes.CDLL(path)
        u64, i64, d, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.synth_bits.restype = u64
        lib.synth_bits.argtypes = [u64, u64, u64]
        lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, d, d, p]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, d, d, p]
        lib.synth_f32_to_bf16.argtypes = [p, i64, p]
        lib.synth_q4_normal.argtypes = [u64, u64, u64, i64, i64, d, p, p, p]
        lib.synth_fp8_normal.argtypes = [u64, u64, u64, i64, i64, i64, d, p, p]
        lib.synth_uniform_f64.argtypes = [u64, u64, u64, i64, p]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def bits(seed: int, tid: int, c: int) -> int:
    return int(_L().synth_bits(seed, tid, c))


def normal_f32(seed, tid, n, std=1.0, mean=0.0, start=0, out=None) -> np.ndarray:
    out = np.empty(n, np.float32) if out is None else out
    _L().synth_normal_f32(seed, tid, start, n, mean, std, _ptr(out))
    return out


def normal_bf16(seed, tid, n, std=1.0, mean=0.0, start=0, out=None) -> np.ndarray:
    out = np.empty(n, np.uint16) if out is None else out
    _L().synth_normal_bf16(seed, tid, start, n, mean, std, _ptr(out))
    return out


def uniform(seed, tid, n, start=0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _L().synth_uniform_f64(seed, tid, start, n, _ptr(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    _L().synth_f32_to_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def q4_normal(seed, tid, rows, cols, std, start=0):
    """4-bit affine quantisation (group 64 along `cols`) of normal draws."""
    assert cols % 64 == 0
    q = np.empty((rows, cols // 8), np.uint32)
    s = np.empty((rows, cols // 64), np.uint16)
    b = np.empty((rows, cols // 64), np.uint16)
    _L().synth_q4_normal(seed, tid, start, rows, cols, std, _ptr(q), _ptr(s), _ptr(b))
    return q, s, b


def fp8_normal(seed, tid, nmat, rows, cols, std, start=0):
    """fp8 (OCP E4M3) quantisation of normal draws with one fp32 scale per 128 x 128 block of
    each of `nmat` stacked [rows, cols] matrices: (codes uint8 [nmat, rows, cols], scales fp32
    [nmat, ceil(rows/128), ceil(cols/128)])."""
    assert cols % 2 == 0 and start % 2 == 0
    q = np.empty((nmat, rows, cols), np.uint8)
    s = np.empty((nmat, (rows + 127) // 128, (cols + 127) // 128), np.float32)
    _L().synth_fp8_normal(seed, tid, start, nmat, rows, cols, std, _ptr(q), _ptr(s))
    return q, s


def permutation(seed: int, tid: int, n: int) -> np.ndarray:
    """Seeded Fisher-Yates permutation of 0..n-1 (uniform draws from the same generator)."""
    p = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = bits(seed, tid, i) % (i + 1)
        p[i], p[j] = p[j], p[i]
    return p


# --------------------------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    K: int
    G: int
    TG: int
    I: int
    Is: int
    act: str        # "f32" | "bf16"
    expert: str     # "f32" | "bf16" | "q4" | "fp8"
    bias_std: float
    norm: bool
    rsf: float
    seed: int       # seed of x, bias, offsets and planted rows
    wseed: int      # seed of router, expert and shared weights
    zipf_s: float = 0.0      # >0: per-expert logit offset -s*ln(1+perm(e))
    planted: int = 0         # rows realised so that the max expert's group loses on top-2 sum
    note: str = ""
    route: str = "deepseek"  # gate: "deepseek" (sigmoid, bias, groups) or "softmax"
    shared_gate: bool = False  # shared expert output scaled by sigmoid(x . w_sgate)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def desc(self) -> str:
        return (f"{self.name}: T={self.T} H={self.H} E={self.E} K={self.K} G={self.G} TG={self.TG} "
                f"I={self.I} Is={self.Is} {self.act}/{self.expert}")


WORKLOADS = {
    # tiny fp32 layer
    "c0": Workload("c0", T=16, H=64, E=8, K=2, G=1, TG=1, I=32, Is=32, act="f32", expert="f32",
                   bias_std=0.1, norm=True, rsf=1.0, seed=0, wseed=0),
    # group-routing stress
    "c1": Workload("c1", T=512, H=1024, E=64, K=6, G=4, TG=2, I=512, Is=512, act="bf16", expert="bf16",
                   bias_std=0.5, norm=True, rsf=2.5, seed=1, wseed=1, planted=64),
    # DeepSeek-V3-shaped decode batch
    "c2": Workload("c2", T=64, H=7168, E=256, K=8, G=8, TG=4, I=2048, Is=2048, act="bf16", expert="bf16",
                   bias_std=0.1, norm=True, rsf=2.5, seed=2, wseed=2),
    # DeepSeek-V3-shaped prefill with Zipf-skewed expert load
    "c3": Workload("c3", T=8192, H=7168, E=256, K=8, G=8, TG=4, I=2048, Is=2048, act="bf16", expert="bf16",
                   bias_std=0.1, norm=True, rsf=2.5, seed=3, wseed=2, zipf_s=1.1),
    # DeepSeek-V3 shapes with 4-bit routed experts
    "c4": Workload("c4", T=4096, H=7168, E=256, K=8, G=8, TG=4, I=2048, Is=2048, act="bf16", expert="q4",
                   bias_std=0.1, norm=True, rsf=2.5, seed=4, wseed=2),
    # DeepSeek-V3 shapes with fp8 (E4M3, 128 x 128 block scales) routed experts: prefill and decode
    "c5": Workload("c5", T=4096, H=7168, E=256, K=8, G=8, TG=4, I=2048, Is=2048, act="bf16", expert="fp8",
                   bias_std=0.1, norm=True, rsf=2.5, seed=5, wseed=2),
    "c6": Workload("c6", T=64, H=7168, E=256, K=8, G=8, TG=4, I=2048, Is=2048, act="bf16", expert="fp8",
                   bias_std=0.1, norm=True, rsf=2.5, seed=6, wseed=2),
}


def _act_normal(w: Workload, tid: int, n: int, std: float, seed: int, start: int = 0):
    if w.act == "f32":
        return normal_f32(seed, tid, n, std, start=start)
    return normal_bf16(seed, tid, n, std, start=start)


def gen_router(w: Workload) -> np.ndarray:
    return _act_normal(w, TID_ROUTER, w.E * w.H, 1.0 / math.sqrt(w.H), w.wseed).reshape(w.E, w.H)


def gen_bias(w: Workload) -> np.ndarray:
    return normal_f32(w.seed, TID_BIAS, w.E, w.bias_std)


def gen_logit_offset(w: Workload) -> Optional[np.ndarray]:
    """Zipf-skewed per-expert router-logit offset: -s * ln(rank), rank = 1 + perm(e)."""
    if w.zipf_s <= 0:
        return None
    p = permutation(w.seed, TID_ZIPF, w.E)
    return (-w.zipf_s * np.log1p(p.astype(np.float64))).astype(np.float32)


def planted_rows(w: Workload) -> np.ndarray:
    if w.planted <= 0:
        return np.zeros(0, np.int64)
    stride = max(1, w.T // w.planted)
    return (np.arange(w.planted, dtype=np.int64) * stride + stride // 2)[: w.planted]


def planted_logits(w: Workload, bias: np.ndarray, n: int, seed_offset: int = 0) -> np.ndarray:
    """Target router logits [n, E] for rows in which the group holding the single largest
    biased score loses on the top-2 group sum.

    Construction (input shaping only): group A is the group of the largest-bias expert a*;
    a* gets sigmoid ~0.97, the rest of A gets ~0.03; in every other group the two
    largest-bias experts get sigmoid 0.98 and the rest get small random values.  The
    property is re-checked on the oracle's own logits by the tests, never assumed."""
    E, G = w.E, w.G
    Eg = E // G
    astar = int(np.argmax(bias))
    A = astar // Eg
    uu = uniform(w.seed, TID_PLANT, n * E, start=seed_offset * n * E).reshape(n, E)
    sig = 0.01 + 0.2 * uu
    for g in range(G):
        idx = np.arange(g * Eg, (g + 1) * Eg)
        if g == A:
            sig[:, idx] = 0.01 + 0.04 * uu[:, idx]
            sig[:, astar] = 0.95 + 0.04 * uu[:, astar]
        else:
            top2 = idx[np.argsort(-bias[idx], kind="stable")[:2]]
            sig[:, top2] = 0.98
    return np.log(sig / (1.0 - sig)).astype(np.float32)


def gen_x(w: Workload, router: Optional[np.ndarray] = None, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Activations [T, H] ~ N(0,1); planted rows (if any) are set to the minimum-norm
    x with router(x) = planted target logits, solved in fp64 and rounded to the act dtype."""
    x = _act_normal(w, TID_X, w.T * w.H, 1.0, w.seed).reshape(w.T, w.H)
    rows = planted_rows(w)
    if len(rows):
        assert router is not None and bias is not None
        R = router.astype(np.float64) if w.act == "f32" else bf16_to_f32(router).astype(np.float64)
        z = planted_logits(w, bias, len(rows)).astype(np.float64)
        xs = R.T @ np.linalg.solve(R @ R.T, z.T)  # [H, n]
        xs = np.ascontiguousarray(xs.T.astype(np.float32))
        x[rows] = xs if w.act == "f32" else f32_to_bf16(xs)
    return x


def gen_expert_weights(w: Workload, e0: int = 0, e1: Optional[int] = None) -> dict:
    """Routed expert weights for experts [e0, e1): gate/up [n, I, H], down [n, H, I].
    For expert dtype q4 returns packed uint32 codes plus bf16 scale ('s_*') and offset ('b_*');
    for fp8, uint8 E4M3 codes plus fp32 scales per 128 x 128 block ('s_*')."""
    e1 = w.E if e1 is None else e1
    n = e1 - e0
    sg, sd = 1.0 / math.sqrt(w.H), 1.0 / math.sqrt(w.I)
    out = {}
    for nm, tid, o, i, std in (("gate", TID_WG, w.I, w.H, sg), ("up", TID_WU, w.I, w.H, sg),
                               ("down", TID_WD, w.H, w.I, sd)):
        start = e0 * o * i
        if w.expert == "fp8":
            out[nm], out["s_" + nm] = fp8_normal(w.wseed, tid, n, o, i, std, start=start)
        elif w.expert == "q4":
            q, s, b = q4_normal(w.wseed, tid, n * o, i, std, start=start)
            out[nm] = q.reshape(n, o, i // 8)
            out["s_" + nm] = s.reshape(n, o, i // 64)
            out["b_" + nm] = b.reshape(n, o, i // 64)
        elif w.expert == "bf16":
            out[nm] = normal_bf16(w.wseed, tid, n * o * i, std, start=start).reshape(n, o, i)
        else:
            out[nm] = normal_f32(w.wseed, tid, n * o * i, std, start=start).reshape(n, o, i)
    return out


def gen_shared_gate(w: Workload) -> Optional[np.ndarray]:
    """[H] gate vector of the shared expert, N(0, 1/sqrt(H)) in the activation dtype, or None."""
    if not w.shared_gate or w.Is <= 0:
        return None
    return _act_normal(w, TID_SGATE, w.H, 1.0 / math.sqrt(w.H), w.wseed)


def gen_shared(w: Workload) -> Optional[dict]:
    if w.Is <= 0:
        return None
    sg, sd = 1.0 / math.sqrt(w.H), 1.0 / math.sqrt(w.Is)
    return {
        "gate": _act_normal(w, TID_SWG, w.Is * w.H, sg, w.wseed).reshape(w.Is, w.H),
        "up": _act_normal(w, TID_SWU, w.Is * w.H, sg, w.wseed).reshape(w.Is, w.H),
        "down": _act_normal(w, TID_SWD, w.H * w.Is, sd, w.wseed).reshape(w.H, w.Is),
    }


def expert_bytes(w: Workload) -> int:
    """Bytes of one routed expert's weights (gate+up+down, including q4 scales/offsets)."""
    n = 3 * w.I * w.H
    if w.expert == "q4":
        return n // 2 + 2 * 2 * (n // 64)
    if w.expert == "fp8":
        nb = 2 * (-(-w.I // 128)) * (-(-w.H // 128)) + (-(-w.H // 128)) * (-(-w.I // 128))
        return n + 4 * nb
    return n * (4 if w.expert == "f32" else 2)


def act_bytes(w: Workload) -> int:
    return 4 if w.act == "f32" else 2
