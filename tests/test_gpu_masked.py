"""GPU parity of the masked (fixed-capacity) layout against the oracle's
index_build_masked / moe_layer(capacity=...): counts, block starts, rows and
the inverse map bit-exact, rows that hold no pair untouched; FFN stages and
the output within the bf16 / block-FP8 gates; and the output bit-identical to
the contiguous layout's (a row's tile, and so its arithmetic, is the same in
both).  Decode-sized cases run the one-launch fused FFN.  Calls go through
the C ABI."""
import dataclasses

import numpy as np
import pytest

from moe_expert_layer_gate_amd import inputs as synth
from oracle import moe_oracle as O
from tests.gpu_util import (TOL_BF16, TOL_FP8, OracleWeights, rel_rows_all, say, small_cfg,
                            torch_cuda, unpanel)
from tests.test_gpu_layer import f64, run_gather_path, run_layer, run_staged
from tests.test_gpu_route_dispatch import run_dispatch

pytestmark = pytest.mark.gpu


def _mods():
    from moe_expert_layer_gate_amd import device as dv
    from moe_expert_layer_gate_amd import moelayer as ml
    return ml, dv


@pytest.mark.parametrize("T,E,k,e_lo,E_L,extra", [
    (64, 256, 8, 0, 32, 0),      # decode batch: one-block index build, capacity = T
    (1, 8, 2, 0, 8, 5),
    (200, 16, 4, 4, 8, 17),
    (777, 16, 4, 0, 16, 3),      # several 256-token blocks
    (300, 64, 8, 60, 4, 0)])
@pytest.mark.parametrize("fp8", [False, True])
def test_masked_dispatch(T, E, k, e_lo, E_L, extra, fp8):
    torch = torch_cuda()
    ml, dv = _mods()
    rng = np.random.default_rng(T * 7 + E_L)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    H = 256
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    C = T + extra
    p = ml.Problem(T=T, H=H, E=E, k=k, e_lo=e_lo, E_L=E_L, I=128, fp8=fp8, capacity=C)
    say("masked dispatch", T, E, k, e_lo, E_L, C, fp8)
    g = run_dispatch(torch, p, x, ids)
    r = O.index_build_masked(ids, e_lo, E_L, C)
    np.testing.assert_array_equal(g["counts"], r["counts"])
    np.testing.assert_array_equal(g["offsets"], r["offsets"])
    np.testing.assert_array_equal(g["tsr"], r["token_slot_row"])
    used = r["row_token"] >= 0
    np.testing.assert_array_equal(g["row_token"][used], r["row_token"][used])
    np.testing.assert_array_equal(g["row_slot"][used], r["row_slot"][used])
    assert (g["row_token"][~used] == -5).all() and (g["row_slot"][~used] == -5).all()
    if fp8:
        xp = g["x_perm"].cpu().numpy()
        qx, sx = O.quantize_rows_groups(O.bf16_to_f64(x), 128)
        np.testing.assert_array_equal(xp[used], qx[r["row_token"][used]])
        np.testing.assert_array_equal(g["x_perm_scale"].cpu().numpy()[used],
                                      sx[r["row_token"][used]])
    else:
        xp = dv.bits_from_bf16(g["x_perm"])
        np.testing.assert_array_equal(xp[used], x[r["row_token"][used]])
    assert not xp[~used].any()           # unused rows are never written


CASES = {
    # decode-like: a few rows per expert -> the fused one-launch FFN
    "decode_like": (small_cfg(T=64, H=512, E=64, E_L=16, e_lo=8, k=8, I=384), 64, 21),
    "decode_gelu": (small_cfg(T=48, H=384, E=32, E_L=16, k=4, I=256, act="gelu"), 60, 22),
    "pipelined": (small_cfg(T=300, H=256, E=8, E_L=8, k=2, I=384), 301, 23),
    "large_tiles": (small_cfg(T=1300, H=384, E=8, E_L=4, e_lo=2, k=2, I=384), 1300, 24),
    "fp8_shared": (small_cfg(T=150, H=512, E=32, E_L=8, e_lo=8, k=4, I=256, I_s=256,
                             fp8=True), 160, 25),
    # MXFP4 weights, decode-sized: the fused skinny MX kernel over the blocks
    "mx_decode": (small_cfg(T=64, H=512, E=64, E_L=16, e_lo=8, k=8, I=384, I_s=128,
                            mx=True), 64, 26),
    "mx_pipelined": (small_cfg(T=300, H=256, E=8, E_L=8, k=2, I=384, mx=True), 301, 27),
}


def check_masked(torch, name, cfg, C, d, dev):
    ml, dv = _mods()
    p = ml.Problem.from_config(cfg, capacity=C)
    say("masked layer", name)
    st = run_staged(torch, p, dev)
    quant = cfg.fp8 or cfg.mx
    ow = OracleWeights(d, cfg.fp8, cfg.mx)
    ref = O.moe_layer(d["logits"], d["x"], ow.as_layer_dict(cfg.E_L), k=cfg.k, e_lo=cfg.e_lo,
                      E_L=cfg.E_L, fp8=cfg.fp8, quantize_activations=quant,
                      activation=cfg.act, capacity=C, mx=cfg.mx)

    def ok(got, want):
        e = rel_rows_all(got, want)
        if e.size == 0:
            return True
        if not quant:
            return e.max() <= TOL_BF16
        return e.max() <= TOL_FP8 and np.percentile(e, 99) <= TOL_BF16

    np.testing.assert_array_equal(st["ids"].cpu().numpy(), ref["ids"])
    np.testing.assert_array_equal(st["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(st["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(st["tsr"].cpu().numpy(), ref["token_slot_row"])
    used = ref["row_token"] >= 0
    np.testing.assert_array_equal(st["row_token"].cpu().numpy()[used], ref["row_token"][used])
    if cfg.mx:
        # only the used rows: the others are never written (any bytes)
        h = O.mx_dequantize(st["h"].cpu().numpy()[used], st["h_scale"].cpu().numpy()[used],
                            "e4m3")
        assert ok(h, O.mx8_activation(ref["h"][used]))
    elif cfg.fp8:
        h = (O.e4m3_value(st["h"].cpu().numpy()[used]) *
             np.repeat(st["h_scale"].cpu().numpy()[used].astype(np.float64), 128, axis=1))
        assert ok(h, O.fp8_activation(ref["h"][used]))
    else:
        assert ok(f64(st["h"])[used], ref["h"][used])
    assert ok(f64(st["y_perm"])[used], ref["y_perm"][used])
    assert ok(f64(st["y"]), ref["y"])
    # one call, and the contiguous layout: the same bits
    y = run_layer(torch, p, dev, guard=2)
    np.testing.assert_array_equal(dv.bits_from_bf16(y), dv.bits_from_bf16(st["y"]))
    yc = run_layer(torch, dataclasses.replace(p, capacity=0), dev)
    np.testing.assert_array_equal(dv.bits_from_bf16(yc), dv.bits_from_bf16(st["y"]))
    if not quant:
        say("masked gather path", name)
        if cfg.I_s == 0:
            yg = run_gather_path(torch, p, dev)
            np.testing.assert_array_equal(dv.bits_from_bf16(yg), dv.bits_from_bf16(st["y"]))
        # panel weights and panel activations over the masked blocks
        say("masked panel layouts", name)
        devp = dv.upload(d, False, panel=True)
        pp = dataclasses.replace(p, layout=ml.LAYOUT_PANEL_WEIGHTS | ml.LAYOUT_PANEL_ACTS)
        sp = run_staged(torch, pp, devp)
        np.testing.assert_array_equal(dv.bits_from_bf16(sp["y"]), dv.bits_from_bf16(st["y"]))
        np.testing.assert_array_equal(dv.bits_from_bf16(sp["h"])[used],
                                      dv.bits_from_bf16(st["h"])[used])


@pytest.mark.parametrize("name", list(CASES))
def test_masked_layer(name):
    torch = torch_cuda()
    ml, dv = _mods()
    cfg, C, seed = CASES[name]
    d = synth.make_inputs(cfg, seed, x_std=1.0, std=0.05)
    dev = dv.upload(d, cfg.fp8, mx=cfg.mx)
    check_masked(torch, name, cfg, C, d, dev)


def test_masked_decode_workload_full_oracle():
    """The DeepSeek-V3 shard's decode batch (T = 64, E_L = 32, k = 8,
    H = 7168, I = 2048) in the masked layout with capacity T, against the
    whole oracle, and bit-identical to the contiguous layout."""
    torch = torch_cuda()
    ml, dv = _mods()
    cfg = synth.config(5)
    d = synth.make_inputs(cfg, cfg.T)
    dev = dv.upload(d, False)
    check_masked(torch, "decode workload", cfg, cfg.T, d, dev)
