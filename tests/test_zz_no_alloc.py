"""GPU check of moe_forward_static, the entry point that allocates nothing (it uses the library's
fixed per-device scratch array instead of a workspace): through the C ABI, two calls in a row --
a batch whose large groups run on the MFMA-tiled kernels, then a smaller one that streams every
group -- each against moe_forward on the same inputs (routing bit-exact, y the same bits, since
both run the same kernels in the same order) and against the oracle (the layer tolerance).
The scratch keeps the previous call's contents, so the second call also shows that nothing in
it needs to start cleared."""
import numpy as np
import pytest
import torch

import oracle
import synth
import deepseek_gate_expert_amd as dg
from deepseek_gate_expert_amd.tensors import to_device, upload_layer
from _gpu import DEV, act_to_f64, log, rel_l2, tol_of

pytestmark = pytest.mark.gpu


def _inputs(w):
    r = synth.gen_router(w)
    b = synth.gen_bias(w)
    x = synth.gen_x(w, r, b)
    return r, b, x, synth.gen_expert_weights(w), synth.gen_shared(w)


def _outs(w):
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    y.view(torch.uint8).fill_(0xFF)
    inds = torch.full((w.T, w.K), -1, dtype=torch.int32, device=DEV)
    scores = torch.full((w.T, w.K), -1.0, dtype=torch.float32, device=DEV)
    return y, inds, scores


@pytest.mark.parametrize("expert", ["bf16", "q4"])
def test_static_matches_workspace_entry_two_calls(expert):
    base = synth.WORKLOADS["c1"].with_(H=256, I=128, Is=128, expert=expert, planted=0)
    for T in (300, 40):
        w = base.with_(T=T)
        log(f"[no-alloc] {expert} T={T}")
        r, b, x, ex, sh = _inputs(w)
        layer = upload_layer(w, r, b, ex, sh, None, DEV)
        xd = to_device(x, DEV)
        need = dg.moe_forward_workspace_size(layer.desc)
        assert 0 < need <= dg.MOE_STATIC_SCRATCH_BYTES
        y0, i0, s0 = _outs(w)
        assert layer.forward(xd, y0, i0, s0) == dg.MOE_OK
        y1, i1, s1 = _outs(w)
        rc = dg.moe_forward_static(layer.desc, xd, layer.router, layer.bias, layer.experts, layer.shared, y1,
                                   None, i1, s1)
        assert rc == dg.MOE_OK, dg.moe_strerror(rc)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(s0.view(torch.int32), s1.view(torch.int32))
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
        y_ref, oi, os_, _ = oracle.forward_workload(w, x, r, b, ex, sh)
        assert np.array_equal(i1.cpu().numpy(), oi)
        err = rel_l2(act_to_f64(y1), y_ref)
        log(f"[no-alloc] {expert} T={T} rel L2 {err:.3e}")
        assert err <= tol_of(w)


def test_static_rejects_layers_beyond_the_scratch():
    w = synth.WORKLOADS["c1"].with_(T=2048, H=1024, I=512, Is=512, planted=0)
    d = dg.layer_desc(20000, w.H, w.E, w.I, w.Is, dg.MOE_BF16, dg.MOE_BF16, w.K, w.G, w.TG, w.norm, w.rsf)
    assert dg.moe_forward_workspace_size(d) > dg.MOE_STATIC_SCRATCH_BYTES
    r, b, x, ex, sh = _inputs(w.with_(T=16))
    layer = upload_layer(w.with_(T=16), r, b, ex, sh, None, DEV)
    xs = torch.zeros((20000, w.H), dtype=torch.bfloat16, device=DEV)
    y = torch.full((20000, w.H), 7.0, dtype=torch.bfloat16, device=DEV)
    rc = dg.moe_forward_static(d, xs, layer.router, layer.bias, layer.experts, layer.shared, y)
    assert rc == dg.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
