"""Host -> device marshalling for the MoE layer binding.

Converts numpy arrays in the storage conventions of the input generator (fp32, bf16 bit
patterns as uint16, 4-bit codes as uint32, fp8 codes as uint8) into torch device tensors, and bundles the device
weights of one layer with its descriptor and workspace.  No arithmetic of the layer lives here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import (MOE_BF16, MOE_F32, MOE_FP8, MOE_OK, MOE_Q4G64, MOE_ROUTE_DEEPSEEK, MOE_ROUTE_SOFTMAX, LayerDesc, layer_desc,
               moe_forward, moe_forward_workspace_size, moe_strerror)

_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "q4": MOE_Q4G64, "fp8": MOE_FP8}


def to_device(a: np.ndarray, device, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """numpy -> device tensor: float32 -> float32, uint16 (bf16 bits) -> bfloat16,
    uint32 -> int32 (same bits), int32 -> int32, uint8 (fp8 codes) -> uint8."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        t = torch.from_numpy(a)
    elif a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif a.dtype in (np.uint32, np.int32):
        t = torch.from_numpy(a.view(np.int32))
    elif a.dtype == np.uint8:
        t = torch.from_numpy(a)
    else:
        raise TypeError(f"unsupported host dtype {a.dtype}")
    if out is not None:
        out.copy_(t, non_blocking=False)
        return out
    return t.to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """device -> numpy with the same conventions (bf16 -> uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def empty_like_host(shape, kind: str, device) -> torch.Tensor:
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "u32": torch.int32, "i32": torch.int32}[kind]
    return torch.empty(shape, dtype=dt, device=device)


@dataclass
class DeviceLayer:
    """Device-resident weights of one MoE layer plus its descriptor and workspace."""
    desc: LayerDesc
    router: torch.Tensor
    bias: torch.Tensor
    experts: dict
    shared: Optional[dict]
    offset: Optional[torch.Tensor] = None
    workspace: Optional[torch.Tensor] = None
    # test aid: before every call, fill the workspace and the fresh outputs with 0xFF bytes (NaN in
    # bf16 and fp32, -1 in int32), so anything the kernels read without having written shows up
    poison: bool = False

    def ensure_workspace(self):
        need = moe_forward_workspace_size(self.desc)
        if need == 0:
            raise ValueError("descriptor rejected by moe_forward_workspace_size")
        if self.workspace is None or self.workspace.numel() < need:
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.router.device)
        return self.workspace

    def forward(self, x: torch.Tensor, y: torch.Tensor, inds=None, scores=None, stream=None) -> int:
        self.ensure_workspace()
        if self.poison:
            self.workspace.fill_(0xFF)
        return moe_forward(self.desc, x, self.router, self.bias, self.experts, self.shared, y, self.offset, inds,
                           scores, self.workspace, stream)

    def __call__(self, x: torch.Tensor, want_route: bool = False):
        T = x.shape[0]
        y = torch.empty((T, self.desc.H), dtype=x.dtype, device=x.device)
        K = self.desc.route.top_k
        inds = torch.empty((T, K), dtype=torch.int32, device=x.device) if want_route else None
        scores = torch.empty((T, K), dtype=torch.float32, device=x.device) if want_route else None
        if self.poison:
            for t in (y, inds, scores):
                if t is not None:
                    t.view(torch.uint8).fill_(0xFF)
        rc = self.forward(x, y, inds, scores)
        if rc != MOE_OK:
            raise RuntimeError(f"moe_forward failed: {rc} ({moe_strerror(rc)})")
        return (y, inds, scores) if want_route else y


def make_desc(w, T: Optional[int] = None) -> LayerDesc:
    """Layer descriptor from a workload-like object (fields T,H,E,I,Is,K,G,TG,norm,rsf,act,expert)."""
    kind = MOE_ROUTE_SOFTMAX if getattr(w, "route", "deepseek") == "softmax" else MOE_ROUTE_DEEPSEEK
    return layer_desc(w.T if T is None else T, w.H, w.E, w.I, w.Is, _DT[w.act], _DT[w.expert], w.K, w.G, w.TG,
                      w.norm, w.rsf, kind)


def upload_layer(w, router: np.ndarray, bias: np.ndarray, experts: dict, shared: Optional[dict],
                 offset: Optional[np.ndarray], device, T: Optional[int] = None,
                 shared_gate: Optional[np.ndarray] = None, poison: bool = False) -> DeviceLayer:
    dev = torch.device(device)
    ex = {k: to_device(v, dev) for k, v in experts.items()}
    sh = None if shared is None else {k: to_device(v, dev) for k, v in shared.items()}
    if sh is not None and shared_gate is not None:
        sh["sgate"] = to_device(shared_gate, dev)
    off = None if offset is None else to_device(np.ascontiguousarray(offset, np.float32), dev)
    return DeviceLayer(make_desc(w, T), to_device(router, dev), to_device(np.ascontiguousarray(bias, np.float32), dev),
                       ex, sh, off, poison=poison)
