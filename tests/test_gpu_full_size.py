"""Every row at full size: the Qwen3-30B-A3B-shaped prefill, the
DeepSeek-V3-shaped EP8 shard in bf16, and the same shard in block-FP8 with
its shared expert, against the whole oracle on all tokens.

Page "OverlapAdvisor ...", section 6.1.2: every strategy is validated on
every measured configuration against a serial reference, at relative l2
below 1e-2 (BF16) and 5e-2 (FP8).  Checked here, on the staged calls through
the C ABI (which give the intermediate stages) and on the one-call layer:
  * routing ids, offsets, the permutation and the inverse map bit-exact;
  * every row of h, of y_perm (expert-major order) and of y, and of the
    shared expert's output, within the per-row gate (max over rows of
    ||got - ref|| / ||ref||: 2e-2 bf16, 6e-2 block-FP8, against the exact
    oracle -- for block-FP8 the oracle's dequantised weights, x and h not
    quantised);
  * the pages' global relative l2 of y below 1e-2 (bf16) / 5e-2 (FP8);
  * the one-call moe_layer bit-identical to the staged calls.
The oracle takes tens of seconds per workload on the host's cores."""
import numpy as np
import pytest

from moe_expert_layer_gate_amd import inputs as synth
from oracle import moe_oracle as O
from tests.gpu_util import (TOL_BF16, TOL_FP8, OracleWeights, global_rel, rel_rows_all, say,
                            torch_cuda)
from tests.test_gpu_layer import f64, h_values, run_layer, run_staged

pytestmark = pytest.mark.gpu

GLOBAL_BF16 = 1e-2
GLOBAL_FP8 = 5e-2


def _mods():
    from moe_expert_layer_gate_amd import device as dv
    from moe_expert_layer_gate_amd import moelayer as ml
    return ml, dv


def _rows_ok(name, got, ref, tol):
    e = rel_rows_all(got, ref)
    worst = int(np.argmax(e)) if e.size else -1
    print(f"  {name}: rows {e.size}, max {e.max() if e.size else 0:.3e} (row {worst}), "
          f"mean {e.mean() if e.size else 0:.3e}, global {global_rel(got, ref):.3e}", flush=True)
    assert e.size == 0 or e.max() <= tol, (name, worst, e[worst])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [2, 3, 4])
def test_every_row_full_size(cid):
    torch = torch_cuda()
    ml, dv = _mods()
    cfg = synth.config(cid)
    quant = cfg.fp8
    tol = TOL_FP8 if quant else TOL_BF16
    d = synth.make_inputs(cfg, cid)
    dev = dv.upload(d, cfg.fp8)
    p = ml.Problem.from_config(cfg)
    say("full size, every row: staged calls", cfg.name)
    st = run_staged(torch, p, dev)
    N = int(st["offsets"][-1].item())
    got = {"ids": st["ids"].cpu().numpy(), "offsets": st["offsets"].cpu().numpy(),
           "row_token": st["row_token"][:N].cpu().numpy(), "tsr": st["tsr"].cpu().numpy(),
           "h": h_values(st, p), "y_perm": f64(st["y_perm"][:N]), "y": f64(st["y"]),
           "shared": f64(st["shared"]) if st["shared"] is not None else None}
    y_bits = dv.bits_from_bf16(st["y"])
    del st
    say("full size, every row: one-call layer", cfg.name)
    y_layer = dv.bits_from_bf16(run_layer(torch, p, dev))
    np.testing.assert_array_equal(y_layer, y_bits)
    del dev
    torch.cuda.empty_cache()

    say("full size, every row: oracle on the host", cfg.name)
    ow = OracleWeights(d, cfg.fp8)
    ref = O.moe_layer(d["logits"], d["x"], ow.as_layer_dict(cfg.E_L), k=cfg.k, e_lo=cfg.e_lo,
                      E_L=cfg.E_L, fp8=cfg.fp8)
    np.testing.assert_array_equal(got["ids"], ref["ids"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["row_token"], ref["row_token"])
    np.testing.assert_array_equal(got["tsr"], ref["token_slot_row"])
    print(f"{cfg.name}: {N} local pairs, routing and permutation exact", flush=True)
    # h is stored in the GEMM activation format (bf16, or E4M3 with scales):
    # compared with the exact oracle's h at the gate of that format
    _rows_ok("h", got["h"], ref["h"], tol)
    _rows_ok("y_perm", got["y_perm"], ref["y_perm"], tol)
    if ref["shared"] is not None:
        _rows_ok("shared", got["shared"], ref["shared"], tol)
    _rows_ok("y", got["y"], ref["y"], tol)
    g = global_rel(got["y"], ref["y"])
    assert g < (GLOBAL_FP8 if quant else GLOBAL_BF16), g
