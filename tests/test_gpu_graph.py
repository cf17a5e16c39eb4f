"""HIP graph capture of the one-call layer.  Every call of the library is a
sequence of kernel launches on the caller's stream with every data-dependent
size kept on the device, so a captured layer replays correctly: each replay
rebuilds the work tables and clears the fused decode queue's ticket and
counters with kernels of its own.  Checked per kernel family: three replays,
with eager work and host synchronisation between them, each bit-identical to
the eager call; then new input values written into the captured buffers,
and the replay bit-identical to an eager call on those values.  Calls go
through the C ABI."""
import numpy as np
import pytest

from moe_expert_layer_gate_amd import inputs as synth
from tests.gpu_util import say, small_cfg, torch_cuda

pytestmark = pytest.mark.gpu

CASES = {
    # bf16: large tiles, skinny fused decode queue (also in the masked layout)
    "bf16_large": (small_cfg(T=1500, H=512, E=16, E_L=4, e_lo=12, k=4, I=640,
                             logits="gumbel_zipf"), None, 31),
    "bf16_skinny": (small_cfg(T=60, H=384, E=16, E_L=8, k=4, I=384, logits="gumbel_zipf"),
                    None, 32),
    "bf16_skinny_masked": (small_cfg(T=60, H=384, E=16, E_L=8, k=4, I=384,
                                     logits="gumbel_zipf"), 64, 32),
    # block-FP8 (skinny routed experts, pipelined shared expert) and MXFP4
    "fp8_shared": (small_cfg(T=150, H=1024, E=64, E_L=16, e_lo=16, k=8, I=512, I_s=256,
                             fp8=True, logits="gumbel_zipf"), None, 33),
    "mx_decode": (small_cfg(T=16, H=1024, E=64, E_L=16, k=8, I=256, mx=True), None, 34),
    "mx_large": (small_cfg(T=1300, H=384, E=8, E_L=4, e_lo=2, k=2, I=640, I_s=256, mx=True),
                 None, 35),
}


def _bits(torch, t):
    return t.view(torch.int16)


@pytest.mark.parametrize("name", list(CASES))
def test_layer_graph_replays(name):
    torch = torch_cuda()
    from moe_expert_layer_gate_amd import device as dv
    from moe_expert_layer_gate_amd import moelayer as ml
    cfg, cap, seed = CASES[name]
    d = synth.make_inputs(cfg, seed, x_std=1.0, std=0.05)
    dev = dv.upload(d, cfg.fp8, mx=cfg.mx)
    p = ml.Problem.from_config(cfg, capacity=cap)
    W = dv.weights_of(dev, p.quantized)
    ws = dv.workspace(p)
    logits, x = dev["logits"].clone(), dev["x"].clone()
    y = torch.empty((p.T, p.H), dtype=torch.bfloat16, device="cuda")
    say("graph eager", name)
    ml.moe_layer(p, logits, x, W, y, ws)
    torch.cuda.synchronize()
    y_eager = y.clone()
    say("graph capture", name)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ml.moe_layer(p, logits, x, W, y, ws)
    torch.cuda.synchronize()
    for it in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        say("graph replay", name, it)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(torch, y), _bits(torch, y_eager)), f"replay {it}"
    # new values in the captured input buffers
    d2 = synth.make_inputs(cfg, seed + 100, x_std=1.0, std=0.05)
    logits.copy_(torch.from_numpy(d2["logits"]).cuda())
    x.copy_(dv.bf16_from_bits(d2["x"]))
    y2 = torch.empty_like(y)
    ml.moe_layer(p, logits, x, W, y2, dv.workspace(p))
    torch.cuda.synchronize()
    assert not torch.equal(_bits(torch, y2), _bits(torch, y_eager))
    say("graph replay new inputs", name)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch, y), _bits(torch, y2))
