"""GPU parity of the whole layer (moe_forward) against the oracle.

Pages: "Epic: Engine Inference Core Stage E - MoE + hybrid families" (gather_mm / gather_qmm
expert dispatch, shared experts always active) and the gate page's merge recommendation
(router -> route -> switch_glu -> combine).  Bar: routing indices bit-exact, gate weights
within relative 1e-6, y within relative L2 1e-5 (fp32 layers), 1e-2 (bf16, fp8) and 2e-2 (4-bit),
against the oracle's fp64 expert math.  The five workloads run at full size; for the two
largest the oracle computes y on a sample of tokens (its routing covers every token).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import deepseek_gate_expert_amd as dg
from deepseek_gate_expert_amd.tensors import to_device, upload_layer
from _gpu import DEV, Case, act_to_f64, log, rel_l2, tol_of

pytestmark = pytest.mark.gpu


def check_route(gi, gs, oi, os_):
    bad = np.nonzero(np.any(gi != oi, axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} token rows routed differently, first {bad[:4]}"
    den = np.maximum(np.abs(os_.astype(np.float64)), 1e-30)
    assert np.max(np.abs(gs.astype(np.float64) - os_) / den) <= 1e-6


@pytest.mark.parametrize("name", ["c0", "c1", "c2"])
def test_layer_full(name):
    w = synth.WORKLOADS[name]
    log(f"[layer] {w.desc}")
    c = Case(w)
    y, inds, scores = c.gpu()
    y_ref, oi, os_, _ = c.oracle_rows()
    check_route(inds.cpu().numpy(), scores.cpu().numpy(), oi, os_)
    err = rel_l2(act_to_f64(y), y_ref)
    log(f"[layer] {name} rel L2 {err:.3e}")
    assert err <= tol_of(w)


def tile_rows(oi, K, BM=128):
    """Tokens that put a row into every BM-row tile of every expert group, in the layout the
    dispatch gives a group (its slots in ascending order): the first row of each group and the
    last row of each of its tiles (so every ragged last tile too).  128-row tiles cover the
    256-row tiles of the bf16 kernel twice, the 4-bit kernel's 160-row tiles and the fp8 kernel's
    128-row tiles at least once (every span of 128 or more rows holds the end of a 128-row block);
    a group of at most 64 rows (streamed in bf16 layers) is one tile."""
    flat = oi.ravel()
    rows = set()
    for e in np.unique(flat):
        slots = np.nonzero(flat == e)[0]
        rows.add(int(slots[0] // K))
        for m0 in range(0, len(slots), BM):
            rows.add(int(slots[min(m0 + BM, len(slots)) - 1] // K))
    return sorted(rows)


def check_rows(name, w, y, rows, y_ref):
    got = act_to_f64(y)[rows]
    err = rel_l2(got, y_ref)
    per_row = np.linalg.norm(got - y_ref, axis=1) / np.maximum(np.linalg.norm(y_ref, axis=1), 1e-30)
    worst = int(np.argmax(per_row))
    log(f"[layer] {name}: {len(rows)} rows, rel L2 {err:.3e}, worst row {rows[worst]} {per_row[worst]:.3e}")
    assert np.all(np.isfinite(got)), "non-finite outputs (a row read unwritten workspace)"
    assert err <= tol_of(w)
    assert per_row[worst] <= 2 * tol_of(w), f"token {rows[worst]}: rel L2 {per_row[worst]:.3e}"


@pytest.mark.parametrize("name", ["c3", "c4", "c5", "c6"])
def test_layer_full_size_sampled(name):
    """Full-size workloads, workspace and outputs poisoned with NaN before the call: routing of
    every token against the oracle, y on tokens that cover every tile of every group (every row
    for the decode batch), with a per-token bound beside the aggregate."""
    w = synth.WORKLOADS[name]
    log(f"[layer] {w.desc} (sampled)")
    c = Case(w)
    y, inds, scores = c.gpu()
    _, oi, os_ = c.oracle_route_all()
    check_route(inds.cpu().numpy(), scores.cpu().numpy(), oi, os_)
    counts = np.bincount(oi.ravel(), minlength=w.E)
    rows = list(range(w.T)) if w.T <= 64 else tile_rows(oi, w.K)
    log(f"[layer] {name}: experts hit {int(np.count_nonzero(counts))}, max load {counts.max()}; "
        f"oracle on {len(rows)} tokens")
    y_ref, _, _, _ = c.oracle_rows(rows)
    check_rows(name, w, y, rows, y_ref)


def test_layer_prefill_bitwise_repeatable():
    """The DeepSeek-V3 prefill batch (8192 tokens, Zipf load) twice through the same layer, the
    workspace poisoned before each call: y, inds and scores are the same bits."""
    c = Case(synth.WORKLOADS["c3"])
    y1, i1, s1 = c.gpu()
    y2, i2, s2 = c.gpu()
    assert torch.equal(i1, i2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert bool(torch.isfinite(y1.float()).all())


def small_case(w, seed_shift=0):
    w = w.with_(seed=w.seed + seed_shift)
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    ex = synth.gen_expert_weights(w)
    sh = synth.gen_shared(w)
    off = synth.gen_logit_offset(w)
    return w, r, b, x, ex, sh, off


def run_small(w, r, b, x, ex, sh, off):
    layer = upload_layer(w, r, b, ex, sh if w.Is > 0 else None, off, DEV, shared_gate=synth.gen_shared_gate(w),
                         poison=True)
    y, inds, scores = layer(to_device(x, DEV), want_route=True)
    torch.cuda.synchronize()
    return y, inds.cpu().numpy(), scores.cpu().numpy()


C1 = synth.WORKLOADS["c1"]
EDGE = [
    ("T1", C1.with_(T=1, planted=0)),
    ("ragged_T", C1.with_(T=37, planted=0)),
    ("top_k_1", C1.with_(T=64, K=1, planted=0)),
    ("no_dropped_group", C1.with_(T=64, TG=4, planted=0)),
    ("K_above_kept", C1.with_(T=32, K=40, G=8, TG=2, planted=0)),
    ("top_k_max_streamed", C1.with_(T=24, K=64, G=2, TG=1, planted=0)),  # top_k at its limit (64)
    ("top_k_max_tiled", C1.with_(T=200, H=256, I=128, Is=128, K=64, G=2, TG=1, planted=0)),
    ("no_shared", C1.with_(T=48, Is=0, planted=0)),
    ("shared_narrower", C1.with_(T=48, I=256, Is=128, planted=0)),
    ("shared_wider", C1.with_(T=48, I=128, Is=320, planted=0)),
    ("H_tail_64", C1.with_(T=40, H=192, I=192, Is=64, planted=0)),
    ("q4_small", C1.with_(T=50, expert="q4", planted=0)),
    ("q4_tail", C1.with_(T=20, H=320, I=192, Is=192, expert="q4", planted=0)),
    ("f32_ragged", synth.WORKLOADS["c0"].with_(T=21, H=40, I=24, Is=12)),
    ("f32_groups", synth.WORKLOADS["c0"].with_(T=30, E=16, K=4, G=4, TG=2, H=72)),
    ("zipf_skew", C1.with_(T=400, zipf_s=3.0, planted=0)),
    ("dsv3_decode_small_batch", synth.WORKLOADS["c2"].with_(T=3, H=512, I=256, Is=256)),
    # T above the streaming limit: groups with more than 64 rows go to the LDS-tiled GEMMs
    ("tiled_ragged_cols", C1.with_(T=300, H=320, I=192, Is=320, planted=0)),
    ("tiled_q4", C1.with_(T=400, H=512, I=256, Is=192, expert="q4", planted=0)),
    ("tiled_rows256", C1.with_(T=2048, H=256, I=128, Is=128, planted=0)),
    ("tiled_rows256_q4", C1.with_(T=2048, H=256, I=128, Is=128, expert="q4", planted=0)),
    # reduction lengths that are multiples of 512: the 4-bit kernel takes the scales and offsets in
    # chunks of 8 groups (two chunks in gate/up, one in down)
    ("tiled_q4_side_chunks", C1.with_(T=600, H=1024, I=512, Is=256, expert="q4", planted=0)),
    ("tiled_1024_experts_shared", C1.with_(T=100, H=128, I=64, Is=64, E=1024, K=2, G=1, TG=1, planted=0)),
    ("tiled_skewed", C1.with_(T=1500, H=192, I=128, Is=64, zipf_s=2.0, planted=0)),
    # softmax gate and sigmoid-gated shared expert
    ("softmax_streamed", C1.with_(T=48, route="softmax", planted=0)),
    ("softmax_tiled", C1.with_(T=600, H=256, I=128, Is=128, route="softmax", planted=0)),
    ("shared_gate_streamed", C1.with_(T=40, shared_gate=True, planted=0)),
    ("shared_gate_tiled_router", C1.with_(T=700, H=256, I=128, Is=128, shared_gate=True, planted=0)),
    ("softmax_gated_q4", C1.with_(T=300, H=256, I=128, Is=128, expert="q4", route="softmax", shared_gate=True,
                                  planted=0)),
    ("softmax_gated_f32", synth.WORKLOADS["c0"].with_(route="softmax", shared_gate=True)),
    # fp8 experts: streamed, ragged blocks (H = 320: k blocks of 128, 128, 64 and a 64-wide tail
    # step; I = 192: output blocks of 128 and 64), tiled, tiled with long groups, softmax + gate
    ("fp8_small", C1.with_(T=50, expert="fp8", planted=0)),
    ("fp8_tail", C1.with_(T=20, H=320, I=192, Is=192, expert="fp8", planted=0)),
    # fp8 decode through the DMA ring with an odd number of 128-column down blocks (H = 384: the
    # last down workgroup owns one block) and two-stage reductions
    ("fp8_stream_odd_blocks", C1.with_(T=40, H=384, I=256, Is=128, expert="fp8", planted=0)),
    ("tiled_fp8", C1.with_(T=400, H=512, I=256, Is=192, expert="fp8", planted=0)),
    ("tiled_fp8_ragged_blocks", C1.with_(T=500, H=320, I=192, Is=128, expert="fp8", planted=0)),
    ("tiled_rows_fp8", C1.with_(T=2048, H=256, I=128, Is=128, expert="fp8", planted=0)),
    ("softmax_gated_fp8", C1.with_(T=300, H=256, I=128, Is=128, expert="fp8", route="softmax", shared_gate=True,
                                   planted=0)),
    # one 64-wide k stage in both GEMMs (H = I = Is = 64) with tiles on: every tiled kernel's
    # prologue and loop run a single stage
    ("tiled_one_stage_bf16", C1.with_(T=400, H=64, E=8, K=2, G=1, TG=1, I=64, Is=64, planted=0)),
    ("tiled_one_stage_q4", C1.with_(T=400, H=64, E=8, K=2, G=1, TG=1, I=64, Is=64, expert="q4", planted=0)),
    ("tiled_one_stage_fp8", C1.with_(T=400, H=64, E=8, K=2, G=1, TG=1, I=64, Is=64, expert="fp8", planted=0)),
]


@pytest.mark.parametrize("label,w", EDGE, ids=[e[0] for e in EDGE])
def test_layer_edge_cases(label, w):
    log(f"[edge] {label}: {w.desc}")
    args = small_case(w)
    y, gi, gs = run_small(*args)
    w_, r, b, x, ex, sh, off = args
    y_ref, oi, os_, _ = oracle.forward_workload(w_, x, r, b, ex, sh if w_.Is > 0 else None, offset=off,
                                                shared_gate=synth.gen_shared_gate(w_))
    check_route(gi, gs, oi, os_)
    err = rel_l2(act_to_f64(y), y_ref)
    log(f"[edge] {label} rel L2 {err:.3e}")
    assert err <= tol_of(args[0])


def test_layer_one_hot_expert_load():
    """Every token picks the same top expert (a large bias): that expert's group holds all T rows,
    which exercises the row-chunk loop of the expert kernels."""
    w = C1.with_(T=300, K=2, planted=0)
    w_, r, b, x, ex, sh, off = small_case(w)
    b = b.copy()
    b[5] = 50.0
    y, gi, gs = run_small(w_, r, b, x, ex, sh, off)
    assert np.all(gi[:, 0] == 5)
    y_ref, oi, os_, _ = oracle.forward_workload(w_, x, r, b, ex, sh)
    check_route(gi, gs, oi, os_)
    assert rel_l2(act_to_f64(y), y_ref) <= 1e-2


def test_layer_zero_tokens_and_deterministic():
    w = C1.with_(T=64, planted=0)
    w_, r, b, x, ex, sh, off = small_case(w)
    layer = upload_layer(w_, r, b, ex, sh, off, DEV, poison=True)
    xd = to_device(x, DEV)
    y1 = layer(xd)
    y2 = layer(xd)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # T = 0 is a no-op that returns OK
    desc0 = dg.layer_desc(0, w.H, w.E, w.I, w.Is, dg.MOE_BF16, dg.MOE_BF16, w.K, w.G, w.TG, w.norm, w.rsf)
    ws = layer.ensure_workspace()
    y0 = torch.empty((0, w.H), dtype=torch.bfloat16, device=DEV)
    assert dg.moe_forward(desc0, xd[:0], layer.router, layer.bias, layer.experts, layer.shared, y0, workspace=ws) == 0


def test_layer_rejects_leave_output_untouched():
    w = C1.with_(T=16, planted=0)
    w_, r, b, x, ex, sh, off = small_case(w)
    layer = upload_layer(w_, r, b, ex, sh, off, DEV)
    xd = to_device(x, DEV)
    y = torch.full((w.T, w.H), 7.0, dtype=torch.bfloat16, device=DEV)
    ws = layer.ensure_workspace()
    bad = dg.layer_desc(w.T, w.H, w.E, w.I, w.Is, dg.MOE_BF16, dg.MOE_BF16, w.K, 3, 1, True, 2.5)  # 64 % 3 != 0
    assert dg.moe_forward(bad, xd, layer.router, layer.bias, layer.experts, layer.shared, y, workspace=ws) == -1
    small = ws[: ws.numel() // 2]
    assert dg.moe_forward(layer.desc, xd, layer.router, layer.bias, layer.experts, layer.shared, y,
                          workspace=small) == dg.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())


def test_layer_bias_changes_selection_not_weights():
    """S1 at layer level: raising one expert's bias moves it into every token's selection; its
    weight is still its pre-bias sigmoid share."""
    w = C1.with_(T=32, G=1, TG=1, K=2, norm=False, rsf=1.0, planted=0)
    w_, r, b, x, ex, sh, off = small_case(w)
    b2 = b.copy()
    b2[9] = 10.0
    _, gi, gs = run_small(w_, r, b2, x, ex, sh, off)
    assert np.all(gi[:, 0] == 9)
    logits = oracle.router(x, r, "bf16")
    assert np.array_equal(gs[:, 0], oracle.sigmoid(logits[:, 9]))


@pytest.mark.parametrize("T", [40, 300], ids=["streamed", "tiled"])
def test_layer_fp8_every_code(T):
    """fp8 weights whose codes cycle through all 254 finite E4M3 codes (both signs, subnormals,
    the largest magnitude), so the in-register decode meets every code on both GEMM paths."""
    w = C1.with_(T=T, H=256, I=128, Is=64, expert="fp8", planted=0)
    w_, r, b, x, ex, sh, off = small_case(w)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    ex = dict(ex)
    for k, nm in enumerate(("gate", "up", "down")):
        n = ex[nm].size
        ex[nm] = finite[(np.arange(n) * 7 + 31 * k) % len(finite)].reshape(ex[nm].shape)
    log(f"[fp8 codes] T={T}")
    y, gi, gs = run_small(w_, r, b, x, ex, sh, off)
    y_ref, oi, os_, _ = oracle.forward_workload(w_, x, r, b, ex, sh, offset=off)
    check_route(gi, gs, oi, os_)
    err = rel_l2(act_to_f64(y), y_ref)
    log(f"[fp8 codes] T={T} rel L2 {err:.3e}")
    assert err <= tol_of(w_)


# Group sizes chosen to meet every tile-height variant: the last tile of a group holds 1..BM rows,
# which selects how many 32-row blocks each wave of the bf16 kernel multiplies (0..4 per half of a
# 256-row tile, 0..2 per half of a 128-row one) and which height variant of the quantised kernels
# runs (1..5 blocks of 32 rows of the 4-bit kernel's 160-row tiles, 1..4 of the fp8 kernel's
# 128-row ones); groups of at most 64 rows are streamed in
# bf16 layers and tiled in quantised ones; two experts receive no rows.  SIZES_256 has a mean
# group (over all 18 experts) of 192 rows, so bf16 layers use 256-row tiles; SIZES_128 a mean of
# 133 (128-row tiles).
SIZES_256 = [1, 33, 64, 65, 96, 0, 128, 129, 160, 161, 200, 0, 250, 256, 257, 300, 511, 849]
SIZES_128 = [1, 40, 64, 65, 80, 0, 96, 97, 127, 128, 129, 0, 150, 200, 255, 256, 300, 412]


# Streamed layers (T <= 64): groups of 1..64 rows.  fp8 groups of at most 32 rows stream their
# codes through the LDS DMA ring (one or two 16-row blocks), larger ones and the bf16 shared
# expert through registers, in the same launch; H = 256 / I = 128 give one- and two-stage
# reductions, H = 1024 / I = 512 several stages.
SIZES_STREAM = [1, 15, 16, 17, 31, 32, 33, 0, 47, 64]


def exact_group_case(sizes, K, expert, H=256, I=128):
    """A layer whose routing puts exactly sizes[e] rows in group e: the router is the identity on
    the first E input columns and token t carries 4.0 in the columns of its K experts (0 in the
    other routing columns, N(0,1) elsewhere), so its K largest logits are exactly those experts."""
    E = len(sizes)
    TK = sum(sizes)
    assert TK % K == 0
    T = TK // K
    assert max(sizes) <= T
    w = C1.with_(T=T, H=H, E=E, K=K, G=1, TG=1, I=I, Is=64, expert=expert, planted=0)
    slots = np.repeat(np.arange(E), sizes)          # expert of each slot, expert-major
    chosen = slots.reshape(K, T).T                    # token t: slots t, t + T, ..., distinct experts
    x = synth.normal_bf16(w.seed, 1, T * w.H).reshape(T, w.H)
    x[:, :E] = 0
    x[np.arange(T)[:, None], chosen] = synth.f32_to_bf16(np.array([4.0], np.float32))[0]
    r = np.zeros((E, w.H), np.uint16)
    r[np.arange(E), np.arange(E)] = synth.f32_to_bf16(np.array([1.0], np.float32))[0]
    b = np.zeros(E, np.float32)
    return w, r, b, x, synth.gen_expert_weights(w), synth.gen_shared(w), None


@pytest.mark.parametrize("sizes,expert,H,I", [(SIZES_256, "bf16", 256, 128), (SIZES_128, "bf16", 256, 128),
                                              (SIZES_256, "q4", 256, 128), (SIZES_256, "q4", 1024, 512),
                                              (SIZES_128, "fp8", 256, 128), (SIZES_256, "fp8", 256, 128),
                                              (SIZES_STREAM, "fp8", 256, 128), (SIZES_STREAM, "fp8", 1024, 512),
                                              (SIZES_STREAM, "bf16", 1024, 512)],
                         ids=["bf16_tiles256", "bf16_tiles128", "q4", "q4_side_chunks", "fp8", "fp8_tall_groups",
                              "fp8_streamed", "fp8_streamed_long", "bf16_streamed"])
def test_layer_exact_group_sizes(sizes, expert, H, I):
    w, r, b, x, ex, sh, off = exact_group_case(sizes, 4, expert, H, I)
    log(f"[groups] {expert}: T={w.T} sizes {sizes}")
    y, gi, gs = run_small(w, r, b, x, ex, sh, off)
    y_ref, oi, os_, _ = oracle.forward_workload(w, x, r, b, ex, sh, offset=off,
                                                shared_gate=synth.gen_shared_gate(w))
    assert np.array_equal(np.bincount(oi.ravel(), minlength=w.E), np.array(sizes))
    check_route(gi, gs, oi, os_)
    err = rel_l2(act_to_f64(y), y_ref)
    log(f"[groups] {expert} rel L2 {err:.3e}")
    assert err <= tol_of(w)
    # the tiled paths sum in a fixed order with no atomics: a second call gives the same bits
    y2, gi2, gs2 = run_small(w, r, b, x, ex, sh, off)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert np.array_equal(gi, gi2) and np.array_equal(gs.view(np.uint32), gs2.view(np.uint32))
