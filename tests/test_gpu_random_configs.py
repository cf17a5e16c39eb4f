"""GPU parity on seeded random small configurations: element type (bf16,
block-FP8, MXFP4), MLP form (SwiGLU, GELU), expert layout (contiguous or
masked), shared expert, expert counts, top-k and sizes drawn so the rows per
local expert fall in every kernel family (skinny, pipelined / 128-row, large
tiles) with ragged segment ends and n-tile remainders.  Each case checks
routing and permutation bit for bit and every stage against the oracle (and,
masked, the output bit-identical to the contiguous layout).  Calls go through
the C ABI."""
import numpy as np
import pytest

from moe_expert_layer_gate_amd import inputs as synth
from tests.gpu_util import small_cfg, torch_cuda
from tests.test_gpu_layer import check_small_case
from tests.test_gpu_masked import check_masked

pytestmark = pytest.mark.gpu


def _draw_cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = {}
    for i in range(n):
        dtype = ("bf16", "fp8", "mx")[i % 3]
        E = int(rng.choice([4, 8, 16, 32, 64]))
        E_L = int(rng.choice([d for d in (1, 2, 4, 8, 16) if d <= E]))
        e_lo = int(rng.integers(0, E - E_L + 1))
        k = int(rng.integers(1, min(E, 8) + 1))
        H = int(rng.choice([128, 256, 384, 512]))
        I = int(rng.choice([128, 256, 384, 640]))
        rows = int(rng.choice([6, 24, 90, 300]))          # target rows per local expert
        kk = min(k, E_L)
        T = int(np.clip(rows * E_L / max(kk * E_L / E, 1e-9) / E_L, 1, 4000 // kk))
        I_s = int(rng.choice([0, 0, 128, 256]))
        act = "gelu" if dtype == "bf16" and rng.random() < 0.3 else "swiglu"
        logits = "gumbel_zipf" if rng.random() < 0.5 else "normal"
        cap = T + int(rng.integers(0, 9)) if rng.random() < 0.3 else None
        cfg = small_cfg(T=T, H=H, E=E, E_L=E_L, e_lo=e_lo, k=k, I=I, I_s=I_s,
                        fp8=dtype == "fp8", mx=dtype == "mx", act=act, logits=logits)
        name = (f"r{i:02d}_{dtype}_{act}_T{T}_H{H}_I{I}_E{E}_L{E_L}_k{k}"
                + (f"_s{I_s}" if I_s else "") + (f"_C{cap}" if cap else ""))
        cases[name] = (cfg, cap, 1000 + i)
    return cases


CASES = _draw_cases()


def _draw_tall_cases(n=4, seed=20261204):
    """bf16 cases with at least 1536 rows per local expert by the host's bound
    (T min(k, E_L) / E_L, or the capacity C in the masked layout), so the
    large-tile GEMMs run 384-row tiles: ragged T, small H and I."""
    rng = np.random.default_rng(seed)
    cases = {}
    for i in range(n):
        E = int(rng.choice([4, 8]))
        E_L = int(rng.choice([d for d in (1, 2, 4) if d <= E]))
        k = int(rng.integers(1, 3))
        kk = min(k, E_L)
        T = int(2048 * E_L / kk) + int(rng.integers(1, 700))
        H = int(rng.choice([128, 256]))
        I = int(rng.choice([128, 384]))
        act = "gelu" if i % 2 else "swiglu"
        cap = T + int(rng.integers(0, 9)) if i == n - 1 else None
        cfg = small_cfg(T=T, H=H, E=E, E_L=E_L, e_lo=int(rng.integers(0, E - E_L + 1)), k=k,
                        I=I, act=act, logits="gumbel_zipf")
        name = (f"tall{i}_{act}_T{T}_H{H}_I{I}_E{E}_L{E_L}_k{k}" + (f"_C{cap}" if cap else ""))
        cases[name] = (cfg, cap, 2000 + i)
    return cases


CASES.update(_draw_tall_cases())


@pytest.mark.parametrize("name", list(CASES))
def test_random_config(name):
    torch = torch_cuda()
    from moe_expert_layer_gate_amd import device as dv
    cfg, cap, seed = CASES[name]
    d = synth.make_inputs(cfg, seed, x_std=1.0, std=0.05)
    dev = dv.upload(d, cfg.fp8, mx=cfg.mx)
    if cap:
        check_masked(torch, name, cfg, cap, d, dev)
    else:
        check_small_case(name, cfg, d, dev)
