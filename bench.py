#!/usr/bin/env python3
"""Benchmark of the DeepSeek-V3-shaped MoE layer forward on one MI355X.

One "step" is one moe_forward call: router -> gate -> dispatch -> grouped gate/up GEMM with
SwiGLU -> grouped down GEMM -> combine, over one batch of seeded synthetic tokens with all
inputs already resident in HBM.  Headline workload: the DeepSeek-V3-shaped prefill batch
(T=8192, H=7168, 256 experts, top-8 of 8 groups keeping 4, expert and shared intermediate 2048,
bf16, Zipf-skewed expert load).  The decode batch (T=64, same layer) is reported beside it.

Prints ONE JSON line: throughput (tokens/s), the dominant kernel's roofline (measured with HIP
events around that kernel inside the timed steps), and the CPU oracle's throughput on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MoE-layer tokens/sec (DeepSeek-V3 shape, bf16) + % HBM/MFMA peak"

# Memory-side traffic of the dominant kernel, GB per launch, comes from a committed counter
# summary under profiles/ (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, over this script, each
# scaled by what the same counter reads for the plain 256 MiB device copy that main() runs
# first).  FETCH_SIZE counts the L2's reads from the memory side, so it includes reads that the
# memory-attached last-level cache serves.  The summary records a sha256 of the kernel's source
# file, taken over its code with comments removed and whitespace collapsed, when the counters were
# taken; if that code has changed since, the figure no longer describes the kernel and "traffic"
# is null (a change to comments alone keeps it).
TRAFFIC_PROFILES = {
    "c3": ("gemm_dma_gate_up_dsv3_prefill_T8192_hbm_traffic.md", "experts_tiled.hip"),
    "c2": ("stream_dma_gate_up_dsv3_decode_T64_hbm_traffic.md", "experts_stream.hip"),
    "c4": ("gemm_dma_wq_q4_dsv3_T4096_traffic.md", "experts_tiled.hip"),
}


def code_sha256(path: str) -> str:
    """sha256 of a C/HIP source's code: comments removed, whitespace runs collapsed to one space."""
    import hashlib
    src = open(path).read()
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return hashlib.sha256(" ".join("".join(out).split()).encode()).hexdigest()


def traffic_gb(workload: str):
    """(GB per launch, summary file) from the committed summary, or (None, reason)."""
    import re
    if workload not in TRAFFIC_PROFILES:
        return None, "no counter summary for this workload"
    prof, src = TRAFFIC_PROFILES[workload]
    path = os.path.join(ROOT, "profiles", prof)
    try:
        text = open(path).read()
    except OSError:
        return None, f"profiles/{prof} missing"
    m_gb = re.search(r"^traffic_gb_per_launch:\s*([0-9.]+)\s*$", text, re.M)
    m_sha = re.search(r"^code_sha256:\s*(\S+)\s+(\S+)\s*$", text, re.M)
    if not (m_gb and m_sha) or m_sha.group(1) != src:
        return None, f"profiles/{prof} has no machine-readable figure"
    if code_sha256(os.path.join(ROOT, "deepseek_gate_expert_amd", "csrc", src)) != m_sha.group(2):
        return None, f"{src} changed since the counters in profiles/{prof} were taken"
    return float(m_gb.group(1)), f"profiles/{prof}"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles created through the HIP runtime (timing enabled)."""

    def __init__(self, n: int):
        # the HIP runtime torch has loaded (torch ships its own copy): events must come from it
        mapped = [ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln]
        self.hip = ctypes.CDLL(mapped[0] if mapped else "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = ev
        self.n = n

    def elapsed_ms(self, i: int, j: int) -> float:
        self.hip.hipEventSynchronize(self.arr[j])
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.arr[i])


def layer_bytes(w, n_hit: int) -> float:
    """Algorithmic HBM bytes of one layer call: weights of the experts hit, shared expert,
    router, x and y."""
    import synth
    act = synth.act_bytes(w)
    return (n_hit * synth.expert_bytes(w) + 3 * w.Is * w.H * act + w.E * w.H * act + 2 * w.T * w.H * act)


def gemm1_bytes(w, n_hit: int) -> float:
    """Algorithmic bytes of the gate/up GEMM: gate+up weights of the experts hit and of the
    shared expert, plus x."""
    import synth
    act = synth.act_bytes(w)
    per_expert = synth.expert_bytes(w) * 2 / 3
    return n_hit * per_expert + 2 * w.Is * w.H * act + w.T * w.H * act


# when T exceeds it, the library computes bf16 expert groups of more than this many rows (and the
# shared expert, whose group holds all T rows) in the MFMA-tiled kernels and streams the smaller
# groups; 4-bit and fp8 routed groups of every size are tiled
STREAM_MAX_ROWS = 64


def tiled_gemm1_flops(w, counts) -> float:
    """Algorithmic flops of the tiled gate/up launches: 2 (gate, up) x 2 x H x I per row of every
    tiled group, plus the shared expert's T rows."""
    lim = 0 if w.expert in ("q4", "fp8") else STREAM_MAX_ROWS
    rows = int(counts[counts > lim].sum())
    return 4.0 * w.H * (w.I * rows + w.Is * w.T)


def layer_flops(w) -> float:
    return 2.0 * w.T * w.H * w.E + 6.0 * w.H * w.I * w.T * w.K + 6.0 * w.H * w.Is * w.T


def synth_T(name: str) -> int:
    import synth
    return synth.WORKLOADS[name].T


def run_workload(name: str, steps: int, warmup: int, cache: dict):
    import numpy as np
    import torch

    import synth
    import deepseek_gate_expert_amd as dg
    from deepseek_gate_expert_amd.tensors import DeviceLayer, make_desc, to_device

    w = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    wkey = (w.H, w.E, w.I, w.Is, w.act, w.expert, w.wseed)
    if wkey not in cache:
        t0 = time.time()
        router, experts, shared = synth.gen_router(w), synth.gen_expert_weights(w), synth.gen_shared(w)
        log(f"[bench] generated {w.expert} weights in {time.time() - t0:.1f}s")
        t0 = time.time()
        dev_w = (to_device(router, dev), {k: to_device(v, dev) for k, v in experts.items()},
                 {k: to_device(v, dev) for k, v in shared.items()})
        torch.cuda.synchronize()
        log(f"[bench] uploaded weights in {time.time() - t0:.1f}s")
        cache.clear()
        cache[wkey] = ((router, experts, shared), dev_w)
    (router, experts, shared), (r_d, ex_d, sh_d) = cache[wkey]
    bias = synth.gen_bias(w)
    x = synth.gen_x(w, router, bias)
    offset = synth.gen_logit_offset(w)
    layer = DeviceLayer(make_desc(w), r_d, to_device(np.ascontiguousarray(bias, np.float32), dev), ex_d, sh_d,
                        None if offset is None else to_device(offset, dev))
    layer.ensure_workspace()
    xd = to_device(x, dev)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    inds = torch.empty((w.T, w.K), dtype=torch.int32, device=dev)
    scores = torch.empty((w.T, w.K), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        rc = layer.forward(xd, y, inds, scores)
        if rc != 0:
            raise RuntimeError(f"moe_forward failed: {dg.moe_strerror(rc)}")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    counts = np.bincount(inds.cpu().numpy().ravel(), minlength=w.E)
    n_hit = int(np.count_nonzero(counts))

    # events: pairs (2 i, 2 i + 1) around the dominant kernel of step i (the library records them),
    # then steps + 1 step boundaries recorded here on the same stream
    ev = HipEvents(2 * steps + steps + 1)
    bnd = [2 * steps + i for i in range(steps + 1)]
    assert dg.moe_set_stage_events(dg.MOE_STAGE_GEMM1, ev.arr, steps) == 0
    try:
        torch.cuda.synchronize()
        hip = ev.hip
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        sp = ctypes.c_void_p(stream.cuda_stream)
        t0 = time.perf_counter()
        hip.hipEventRecord(ev.arr[bnd[0]], sp)
        for i in range(steps):
            step()
            hip.hipEventRecord(ev.arr[bnd[i + 1]], sp)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        per_step = [ev.elapsed_ms(bnd[i], bnd[i + 1]) for i in range(steps)]
        per_g1 = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)]
    finally:
        dg.moe_set_stage_events(-1, None, 0)
        ev.close()
    step_ms, g1_ms = statistics.median(per_step), statistics.median(per_g1)
    mean_ms = sum(per_step) / steps
    log(f"[bench] {name}: median {step_ms:.3f} ms/step (mean {mean_ms:.3f}, min {min(per_step):.3f}, "
        f"max {max(per_step):.3f}; wall {wall_ms:.3f}), gemm1 median {g1_ms:.3f} ms, experts hit {n_hit}, "
        f"max load {counts.max()}")
    return dict(w=w, step_ms=step_ms, mean_ms=mean_ms, wall_ms=wall_ms, gemm1_ms=g1_ms, n_hit=n_hit,
                max_load=int(counts.max()),
                counts=counts,
                x=x, bias=bias, offset=offset, router=router, experts=experts, shared=shared)


def run_dense(steps: int, warmup: int):
    """DeepSeek-V3 dense SwiGLU layer (H 7168, I 18432) on 8192 tokens, bf16."""
    import numpy as np
    import torch

    import synth
    import deepseek_gate_expert_amd as dg
    from deepseek_gate_expert_amd.tensors import to_device

    T, H, I = 8192, 7168, 18432
    dev = torch.device("cuda:0")
    t0 = time.time()
    x = synth.normal_bf16(5, synth.TID_X, T * H, 1.0).reshape(T, H)
    wg = synth.normal_bf16(2, 13, I * H, 1 / np.sqrt(H)).reshape(I, H)
    wu = synth.normal_bf16(2, 14, I * H, 1 / np.sqrt(H)).reshape(I, H)
    wd = synth.normal_bf16(2, 15, H * I, 1 / np.sqrt(I)).reshape(H, I)
    log(f"[bench] generated dense weights in {time.time() - t0:.1f}s")
    xd, g, u, d = (to_device(a, dev) for a in (x, wg, wu, wd))
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(dg.moe_dense_workspace_size(T, H, I, dg.MOE_BF16), dtype=torch.uint8, device=dev)

    def step():
        rc = dg.moe_dense_mlp(xd, g, u, d, y, ws)
        if rc != 0:
            raise RuntimeError(f"moe_dense_mlp failed: {dg.moe_strerror(rc)}")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents(steps + 1)
    stream = torch.cuda.current_stream()
    ev.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    sp = ctypes.c_void_p(stream.cuda_stream)
    ev.hip.hipEventRecord(ev.arr[0], sp)
    for i in range(steps):
        step()
        ev.hip.hipEventRecord(ev.arr[i + 1], sp)
    torch.cuda.synchronize()
    ms = statistics.median(ev.elapsed_ms(i, i + 1) for i in range(steps))
    ev.close()
    flops = 6.0 * T * H * I
    ach = flops / (ms / 1e3) / 1e12
    log(f"[bench] dense: {ms:.3f} ms/step, {ach:.0f} TFLOP/s")
    return {"metric": "dense SwiGLU MLP tokens/sec (DeepSeek-V3 dense layer shape, bf16) + % MFMA peak",
            "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"dense SwiGLU layer, T={T} H={H} I={I}, bf16", "global_batch": T,
                       "parallelism": "single GPU"},
            "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": ach / PEAK_BF16_TFLOPS, "traffic": None,
                         "kernel": "whole dense layer: gemm_dma<256, true> (gate/up + SwiGLU) and "
                                   "gemm_dma<256, false> (down)"}}


def cpu_baseline(res, budget_s: float):
    """The oracle as it stands on the host cores, on the first n tokens of the same workload:
    a few doubling runs find its rate, then one run of about `budget_s` seconds is timed."""
    import oracle
    w = res["w"]

    def run(n):
        t0 = time.perf_counter()
        oracle.forward_workload(w, res["x"], res["router"], res["bias"], res["experts"], res["shared"],
                                offset=res["offset"], rows=list(range(n)))
        return time.perf_counter() - t0

    n = 2
    dt = run(n)
    while dt < min(1.5, budget_s / 4) and n * 2 <= w.T:
        n *= 2
        dt = run(n)
    target = max(n, min(w.T, int(n * 0.8 * budget_s / max(dt, 1e-6))))
    if target > n:
        n = target
        dt = run(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {n} of {w.T} tokens of the {w.name} workload, full layer per token "
                      f"(router, gate, {w.K} routed + 1 shared SwiGLU expert, combine), fp64 expert math; "
                      f"{dt:.1f}s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3", choices=["c2", "c3", "c4", "c5", "c6", "dense"],
                    help="c3: DSV3 prefill (headline); c2: decode; c4: 4-bit experts; c5 / c6: fp8 experts, "
                         "prefill / decode; dense: DSV3 dense MLP layer")
    ap.add_argument("--no-secondary", action="store_true", help="skip the decode batch")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this layer forward runs on a single MI355X and has no multi-GPU path; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    from __graft_entry__ import _ensure_built
    _ensure_built()
    import torch
    torch.cuda.init()

    # plain device-to-device copy of a known size (256 MiB): the reference dispatch against which
    # HBM byte counters of the profiled kernels are calibrated; outside every timed region
    cal_src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    if args.workload == "dense":
        print(json.dumps(run_dense(args.steps, args.warmup)))
        return

    cache = {}
    main_res = run_workload(args.workload, args.steps, args.warmup, cache)
    w = main_res["w"]
    sec = None
    if not args.no_secondary:
        other = {"c2": "c3", "c5": "c6", "c6": "c5"}.get(args.workload, "c2")
        small = synth_T(other) <= 256
        sec = run_workload(other, max(args.steps, 20) if small else args.steps, args.warmup, cache)

    def summary(res):
        wl = res["w"]
        tps = wl.T / (res["step_ms"] / 1e3)
        decode = wl.T <= 256
        tr, tr_src = traffic_gb(wl.name)
        if decode:
            ach = gemm1_bytes(wl, res["n_hit"]) / (res["gemm1_ms"] / 1e3) / 1e9
            roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                    "traffic": tr, "traffic_unit": "GB per launch (memory-side reads + writes)",
                    "traffic_source": tr_src,
                    "kernel": ("stream_dma<gate/up> (bf16 weights streamed through an LDS DMA ring, gate/up + SwiGLU)"
                               if wl.expert == "bf16" else
                               "stream_f8<gate/up> (fp8 codes of groups of <= 32 rows streamed through an LDS DMA "
                               "ring, the bf16 shared expert through registers, gate/up + SwiGLU)"
                               if wl.expert == "fp8" else
                               f"stream_gemm<{wl.expert}, gate/up> (weight-streaming gate/up + SwiGLU)")}
            layer = layer_bytes(wl, res["n_hit"]) / (res["step_ms"] / 1e3) / 1e9
            roof["layer_achieved"] = layer
            roof["layer_frac"] = layer / PEAK_HBM_GBS
        else:
            ach = tiled_gemm1_flops(wl, res["counts"]) / (res["gemm1_ms"] / 1e3) / 1e12
            roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": ach / PEAK_BF16_TFLOPS, "traffic": tr,
                    "traffic_unit": "GB per launch (memory-side reads + writes)", "traffic_source": tr_src,
                    "kernel": ("gemm_dma<256, true> (tiled gate/up + SwiGLU: groups above 64 rows and the "
                               "shared expert)") if wl.expert == "bf16" else
                              (f"tiled gate/up + SwiGLU kernels: gemm_dma_wq<{wl.expert}, true> for the {wl.expert} "
                               "routed groups, gemm_dma<256, true> for the bf16 shared expert")}
            layer = layer_flops(wl) / (res["step_ms"] / 1e3) / 1e12
            roof["layer_achieved"] = layer
            roof["layer_frac"] = layer / PEAK_BF16_TFLOPS
        return tps, roof

    tps, roof = summary(main_res)
    cpu = cpu_baseline(main_res, args.cpu_budget)
    out = {
        "metric": METRIC, "value": tps, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_res["step_ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: DeepSeek-V3-shaped {'prefill' if w.T > 256 else 'decode'} batch, "
                               f"T={w.T} H={w.H} E={w.E} top_k={w.K} n_group={w.G} topk_group={w.TG} "
                               f"I={w.I} shared I={w.Is}, bf16 activations, {w.expert} routed experts"
                               + (f", Zipf s={w.zipf_s} expert load"
                                                                    if w.zipf_s else ""),
                   "global_batch": w.T, "experts_hit": main_res["n_hit"], "max_expert_load": main_res["max_load"],
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if sec is not None:
        stps, sroof = summary(sec)
        sw = sec["w"]
        out["secondary"] = {"workload": f"{sw.name}: T={sw.T} (same layer)", "value": stps, "unit": "tokens/s",
                            "ms_per_step": sec["step_ms"], "experts_hit": sec["n_hit"], "roofline": sroof}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
