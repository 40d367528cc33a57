"""Helpers shared by the GPU tests: device, seeded inputs per workload (cached so the
DeepSeek-V3-sized weights are generated and uploaded once per session), and metrics."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
from deepseek_gate_expert_amd.tensors import to_device, to_host, upload_layer

DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (n if n > 0 else 1.0))


def act_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


# fp8 layers keep the bf16 bar: the kernels round each dequantised weight to bf16 (relative
# error <= 2^-9, the oracle's weights are exact), which adds about 1e-3 to the relative L2 error
TOL = {"f32": 1e-5, "bf16": 1e-2, "q4": 2e-2, "fp8": 1e-2}


def tol_of(w) -> float:
    return TOL[w.expert] if w.expert in ("q4", "fp8") else TOL[w.act]


_HOST, _DEVW = {}, {}


def _wkey(w):
    return (w.H, w.E, w.I, w.Is, w.act, w.expert, w.wseed)


def host_weights(w):
    """(router, expert dict, shared dict) of a layer; cached per (shapes, dtypes, weight seed)
    so workloads with the same layer (c2 and c3) share one copy."""
    k = _wkey(w)
    if k not in _HOST:
        log(f"[gen] weights H={w.H} E={w.E} I={w.I} Is={w.Is} {w.act}/{w.expert} wseed={w.wseed}")
        _HOST[k] = (synth.gen_router(w), synth.gen_expert_weights(w), synth.gen_shared(w))
    return _HOST[k]


def device_weights(w):
    k = _wkey(w)
    if k not in _DEVW:
        r, ex, sh = host_weights(w)
        log(f"[upload] weights H={w.H} E={w.E} {w.expert}")
        _DEVW[k] = (to_device(r, DEV), {n: to_device(v, DEV) for n, v in ex.items()},
                    None if sh is None else {n: to_device(v, DEV) for n, v in sh.items()})
    return _DEVW[k]


class Case:
    """Inputs of one workload on host and device."""

    def __init__(self, w):
        self.w = w
        self.router, self.experts, self.shared = host_weights(w)
        self.bias = synth.gen_bias(w)
        self.x = synth.gen_x(w, self.router, self.bias)
        self.offset = synth.gen_logit_offset(w)
        r_d, ex_d, sh_d = device_weights(w)
        from deepseek_gate_expert_amd.tensors import DeviceLayer, make_desc
        self.layer = DeviceLayer(make_desc(w), r_d, to_device(np.ascontiguousarray(self.bias, np.float32), DEV), ex_d,
                                 sh_d, None if self.offset is None else to_device(self.offset, DEV), poison=True)
        self.x_d = to_device(self.x, DEV)

    def gpu(self):
        y, inds, scores = self.layer(self.x_d, want_route=True)
        torch.cuda.synchronize()
        return y, inds, scores

    def oracle_route_all(self):
        w = self.w
        logits = oracle.router(self.x, self.router, w.act, self.offset)
        rc, inds, scores = oracle.route(logits, self.bias, oracle.params(w.K, w.G, w.TG, w.norm, w.rsf))
        assert rc == 0
        return logits, inds, scores

    def oracle_rows(self, rows=None):
        return oracle.forward_workload(self.w, self.x, self.router, self.bias, self.experts, self.shared,
                                       offset=self.offset, rows=rows)
