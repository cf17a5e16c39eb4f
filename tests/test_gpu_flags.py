"""The FFN status flags (moe_workspace_flags) on the GPU.

The one-launch decode FFN bounds the wait of a down tile for the up tiles of
its rows; a wait that gives up sets MOE_FLAG_WAIT_TIMEOUT and skips the tile.
The library's own ordering makes every wait end, so the test forces the
timeout from the host: MOE_TEST_FUSED_WAIT_UNREACHABLE=1 makes every down
tile wait for one more up tile than exists, for a few polls, so every kernel
still ends.  Checked: the flag is clear after a normal call, set after the
forced one, and clear again (with the normal output bits) after the next
normal call; the large-tile path reports no flags.  Calls go through the C
ABI."""
import os

import numpy as np
import pytest

from moe_expert_layer_gate_amd import inputs as synth
from tests.gpu_util import say, small_cfg, torch_cuda

pytestmark = pytest.mark.gpu

ENV = "MOE_TEST_FUSED_WAIT_UNREACHABLE"


def _mods():
    from moe_expert_layer_gate_amd import device as dv
    from moe_expert_layer_gate_amd import moelayer as ml
    return ml, dv


def _layer_and_flags(torch, p, dev, ws):
    ml, dv = _mods()
    y = torch.full((p.T, p.H), 3.0, dtype=torch.bfloat16, device="cuda")
    flags = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    ml.moe_layer(p, dev["logits"], dev["x"], dv.weights_of(dev, p.quantized), y, ws)
    ml.moe_workspace_flags(p, ml.STAGE_LAYER, ws, flags)
    torch.cuda.synchronize()
    return dv.bits_from_bf16(y), int(flags[0].item())


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mx"])
def test_fused_decode_wait_timeout_is_reported(fmt):
    torch = torch_cuda()
    ml, dv = _mods()
    # 32 rows per local expert on average: the one-launch (skinny) FFN
    cfg = small_cfg(T=64, H=512, E=16, E_L=8, k=4, I=256, fp8=fmt == "fp8", mx=fmt == "mx")
    d = synth.make_inputs(cfg, 21, x_std=1.0, std=0.05)
    dev = dv.upload(d, cfg.fp8, mx=cfg.mx)
    p = ml.Problem.from_config(cfg)
    ws = dv.workspace(p)
    assert os.environ.get(ENV) is None
    say("flags: normal call", fmt)
    y0, f0 = _layer_and_flags(torch, p, dev, ws)
    assert f0 == 0
    # a zeroed workspace, so that the rows of skipped down tiles read 0
    ws1 = torch.zeros_like(ws)
    try:
        os.environ[ENV] = "1"
        say("flags: forced timeout", fmt)
        y1, f1 = _layer_and_flags(torch, p, dev, ws1)
    finally:
        del os.environ[ENV]
    assert f1 == ml.FLAG_WAIT_TIMEOUT
    # every down tile was skipped: y_perm kept its zeros, and so did y
    assert not np.any(y1 & 0x7FFF)
    say("flags: normal call again", fmt)
    y2, f2 = _layer_and_flags(torch, p, dev, ws1)
    assert f2 == 0
    np.testing.assert_array_equal(y2, y0)


def test_large_tile_path_has_no_flags():
    torch = torch_cuda()
    ml, dv = _mods()
    cfg = small_cfg(T=1024, H=256, E=8, E_L=8, k=4, I=256)   # 512 rows per expert
    d = synth.make_inputs(cfg, 22)
    dev = dv.upload(d, False)
    p = ml.Problem.from_config(cfg)
    ws = dv.workspace(p)
    ws.fill_(0xFF)       # whatever the workspace held, the FFN clears its flags
    say("flags: large tiles")
    _, f = _layer_and_flags(torch, p, dev, ws)
    assert f == 0
    ws_f = dv.workspace(p, ml.STAGE_FFN)
    flags = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    ws_f.fill_(0xFF)
    ml.moe_workspace_flags(p, ml.STAGE_FFN, ws_f, flags)
    torch.cuda.synchronize()
    assert int(flags[0].item()) == -1        # nothing ran on it yet: its bytes as left
