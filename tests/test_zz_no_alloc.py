"""moe_layer_static -- the layer on the library's static per-device workspace,
for callers that cannot allocate -- against moe_layer with a caller
workspace: the same kernels, so the outputs must have the same bits.  Two
calls in a row on the shared array, the second with a smaller input (fewer
tokens), then a different element type; a problem whose workspace exceeds
the array is rejected with MOE_ERR_WORKSPACE and its output left untouched.
Calls go through the C ABI."""
import dataclasses

import numpy as np
import pytest

from moe_expert_layer_gate_amd import inputs as synth
from tests.gpu_util import say, small_cfg, torch_cuda

pytestmark = pytest.mark.gpu


def _mods():
    from moe_expert_layer_gate_amd import device as dv
    from moe_expert_layer_gate_amd import moelayer as ml
    return ml, dv


def _both(torch, p, dev, T=None):
    """(moe_layer_static output bits, moe_layer output bits) on the first T tokens."""
    ml, dv = _mods()
    T = p.T if T is None else T
    q = dataclasses.replace(p, T=T)
    lg, x = dev["logits"][:T].contiguous(), dev["x"][:T].contiguous()
    W = dv.weights_of(dev, p.quantized)
    y_s = torch.full((T, p.H), 3.0, dtype=torch.bfloat16, device="cuda")
    y_w = torch.full((T, p.H), 5.0, dtype=torch.bfloat16, device="cuda")
    ml.moe_layer_static(q, lg, x, W, y_s)
    ml.moe_layer(q, lg, x, W, y_w, dv.workspace(q))
    torch.cuda.synchronize()
    return dv.bits_from_bf16(y_s), dv.bits_from_bf16(y_w)


@pytest.mark.parametrize("name,T2", [
    ("dsv3_ep8_decode", 17),            # the one-launch decode FFN
    ("tiny", 100),                      # 128-row tiles
    ("dsv3_ep8_decode_fp8", 40),        # block-FP8 weights and activations
    ("dsv3_ep8_decode_mxfp4", 9)])      # MXFP4 weights
def test_static_workspace_matches_moe_layer(name, T2):
    torch = torch_cuda()
    ml, dv = _mods()
    cfg = synth.config(name)
    d = synth.make_inputs(cfg, 31)
    dev = dv.upload(d, cfg.fp8, mx=cfg.mx)
    p = ml.Problem.from_config(cfg)
    assert ml.workspace_bytes(p) - 256 <= ml.STATIC_SCRATCH_BYTES
    say("static workspace", name, p.T)
    a, b = _both(torch, p, dev)
    np.testing.assert_array_equal(a, b)
    assert np.any(a & 0x7FFF)
    # the second call reuses the array, with fewer tokens
    say("static workspace, smaller", name, T2)
    a2, b2 = _both(torch, p, dev, T2)
    np.testing.assert_array_equal(a2, b2)
    # a token's output depends on its own row only
    np.testing.assert_array_equal(a2, a[:T2])


def test_static_workspace_too_small_is_rejected():
    torch = torch_cuda()
    ml, dv = _mods()
    cfg = small_cfg(T=32768, H=1024, E=8, E_L=8, k=4, I=512)
    p = ml.Problem.from_config(cfg)
    assert ml.workspace_bytes(p) - 256 > ml.STATIC_SCRATCH_BYTES
    lg = torch.zeros((p.T, p.E), dtype=torch.float32, device="cuda")
    x = torch.zeros((p.T, p.H), dtype=torch.bfloat16, device="cuda")
    w13 = torch.zeros((p.E_L, 2 * p.I, p.H), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((p.E_L, p.H, p.I), dtype=torch.bfloat16, device="cuda")
    y = torch.full((p.T, p.H), 7.0, dtype=torch.bfloat16, device="cuda")
    say("static workspace, too large")
    with pytest.raises(ml.MoEError) as ei:
        ml.moe_layer_static(p, lg, x, ml.weights_struct(w13, w2), y)
    assert ei.value.status == ml.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
