"""Pins of the oracle's E4M3 format and block quantiser: values the OCP FP8
specification fixes, a brute-force nearest-code search with ties to even,
round trips, saturation and the scale rule amax -> 448."""
import os

import numpy as np
import pytest

from moe_expert_layer_gate_amd import inputs as synth
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_matches_spec_points():
    for line in open(os.path.join(GOLDEN, "e4m3_points.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        code, val = line.split()
        got = O.e4m3_value(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == np.signbit(float(val)), code


def brute_encode(v):
    """Scan every finite code; nearest value wins, an exact tie goes to the
    code whose mantissa LSB is 0; magnitudes above 448 give +-448."""
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = {c: float(O.e4m3_value(np.array([c], np.uint8))[0]) for c in codes}
    out = []
    for x in v:
        x = float(x)
        if abs(x) > 448:
            out.append(0x7E | (0x80 if x < 0 else 0))
            continue
        best = None
        for c in codes:
            if (vals[c] < 0) != (x < 0) and vals[c] != 0:
                continue
            d = abs(vals[c] - x)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1)):
                best = (d, c)
        c = best[1]
        if vals[c] == 0:   # zero keeps the sign of the input
            c = 0x80 if np.signbit(x) else 0x00
        out.append(c)
    return np.array(out, np.uint8)


def test_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(0)
    finite = O.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (finite[:-1] + finite[1:]) / 2          # exact ties
    v = np.concatenate([
        rng.standard_normal(3000) * 50, rng.standard_normal(1000) * 0.01,
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
        [0.0, -0.0, 447.9, 448.0, 463.9, 464.0, 470.0, 1e30, -1e30, 1e-30, -1e-30],
    ]).astype(np.float32)
    np.testing.assert_array_equal(O.e4m3_encode(v), brute_encode(v))


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_value(codes)), codes)


def test_saturation():
    v = np.array([448.0, 449.0, 500.0, 1e9, -448.0, -1e9], np.float32)
    np.testing.assert_array_equal(O.e4m3_encode(v), [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])


def test_block_quantiser_scale_rule():
    rng = np.random.default_rng(1)
    a = O.bf16_to_f64(synth.f32_to_bf16_bits(rng.standard_normal((300, 260)) * 0.02))
    q, s = O.quantize_blocks(a, 128, 128)
    assert s.shape == (3, 3) and s.dtype == np.float32
    for i in range(3):
        for j in range(3):
            blk = a[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            qb = q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            assert s[i, j] == np.float32(amax / np.float32(448))
            # the amax element lands on +-448 exactly (quotient rounds to 448)
            r, c = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert qb[r, c] & 0x7F == 0x7E
    deq = O.dequantize_blocks(q, s, 128, 128)
    # rounding error at most half a code spacing: relative 2^-4 for normals
    rel = np.abs(deq - a) / np.maximum(np.abs(a), 1e-30)
    big = np.abs(a) > np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:300, :260] * 2 ** -6
    assert rel[big].max() <= 2 ** -4 + 1e-12


def test_zero_block_scale_is_one():
    q, s = O.quantize_blocks(np.zeros((128, 128)), 128, 128)
    assert s[0, 0] == 1.0 and np.all(q == 0)


def test_row_groups_match_blocks_of_height_one():
    rng = np.random.default_rng(2)
    a = O.bf16_to_f64(synth.f32_to_bf16_bits(rng.standard_normal((7, 384))))
    q1, s1 = O.quantize_rows_groups(a, 128)
    q2, s2 = O.quantize_blocks(a, 1, 128)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)


def test_fp8_layer_close_to_bf16_layer():
    """Block-FP8 weights (dequantised) stay close to the bf16 weights they
    were made from: the per-row relative error of the layer output is a
    few percent at most."""
    cfg = synth.MoEConfig("t", T=32, H=256, E=8, E_L=8, e_lo=0, k=2, I=256)
    d = synth.make_inputs(cfg, 3)
    qd = {}
    for name in ("w13", "w2"):
        qs = [O.quantize_blocks(O.bf16_to_f64(m), 128, 128) for m in d[name]]
        qd[name + "_q"] = np.stack([q for q, _ in qs])
        qd[name + "_s"] = np.stack([s for _, s in qs])
    y16 = O.moe_layer(d["logits"], d["x"], d, k=2, e_lo=0, E_L=8)["y"]
    y8 = O.moe_layer(d["logits"], d["x"], qd, k=2, e_lo=0, E_L=8, fp8=True)["y"]
    rel = np.linalg.norm(y8 - y16, axis=1) / np.linalg.norm(y16, axis=1)
    assert rel.max() < 0.08


def _fp8_layer_inputs(cfg, seed, std, x_std):
    d = synth.make_inputs(cfg, seed, std=std, x_std=x_std)
    qd = {}
    for name in ("w13", "w2", "ws13", "ws2"):
        if name not in d:
            continue
        if d[name].ndim == 3:
            qs = [O.quantize_blocks(O.bf16_to_f64(m), 128, 128) for m in d[name]]
            qd[name + "_q"] = np.stack([q for q, _ in qs])
            qd[name + "_s"] = np.stack([s for _, s in qs])
        else:
            qd[name + "_q"], qd[name + "_s"] = O.quantize_blocks(O.bf16_to_f64(d[name]), 128, 128)
    return d, qd


def test_activation_quantisation_is_identity_on_representable_groups():
    """Groups whose values are E4M3 values times 2^j with amax 448 * 2^j
    (scale exactly 2^j) pass through unchanged."""
    rng = np.random.default_rng(5)
    vals = O.e4m3_value(np.array([c for c in range(0x7F)], np.uint8))
    a = rng.choice(vals, size=(6, 256)) * rng.choice([-1, 1], size=(6, 256))
    a[:, 0] = 448.0
    a[:, 128] = -448.0
    a *= np.exp2(rng.integers(-20, 5, size=(6, 1)))
    np.testing.assert_array_equal(O.fp8_activation(a), a)


def test_activation_quantisation_sits_before_each_gemm(monkeypatch):
    """With quantize_activations the layer passes exactly two kinds of
    arrays through the activation quantiser: the token activations x (all
    tokens, before the up GEMM) and each expert's h (before the down GEMM),
    never the outputs."""
    cfg = synth.MoEConfig("t", T=24, H=256, E=4, E_L=4, e_lo=0, k=2, I=384, I_s=128)
    d, qd = _fp8_layer_inputs(cfg, 8, std=0.05, x_std=1.0)
    seen = []
    real = O.fp8_activation
    monkeypatch.setattr(O, "fp8_activation", lambda a: (seen.append(np.array(a)), real(a))[1])
    out = O.moe_layer(d["logits"], d["x"], qd, k=2, e_lo=0, E_L=4, fp8=True,
                      quantize_activations=True)
    x = O.bf16_to_f64(d["x"])
    np.testing.assert_array_equal(seen[0], x)                       # x, whole batch, first
    h_shapes = [a.shape for a in seen[1:]]
    assert all(sh[1] in (384, 128) for sh in h_shapes)              # h widths (I or I_s)
    assert sum(sh[0] for sh in h_shapes if sh[1] == 384) == out["offsets"][-1]
    # the routed h seen are the layer's h rows, segment by segment
    np.testing.assert_array_equal(np.concatenate([a for a in seen[1:] if a.shape[1] == 384]),
                                  out["h"])
    # and those h come from the quantised x
    e0 = int(np.nonzero(out["counts"])[0][0])
    a0, b0 = out["offsets"][e0], out["offsets"][e0 + 1]
    w13 = O.dequantize_blocks(qd["w13_q"][e0], qd["w13_s"][e0], 128, 128)
    xq = real(x)[out["row_token"][a0:b0]]
    np.testing.assert_allclose(out["h"][a0:b0],
                               O.silu(xq @ w13[:384].T) * (xq @ w13[384:].T), rtol=1e-12)


@pytest.mark.parametrize("shared", [0, 128])
def test_quantised_activations_move_the_output_a_little(shared):
    cfg = synth.MoEConfig("t", T=40, H=256, E=8, E_L=8, e_lo=0, k=2, I=256, I_s=shared)
    d, qd = _fp8_layer_inputs(cfg, 7, std=0.05, x_std=1.0)
    a = O.moe_layer(d["logits"], d["x"], qd, k=2, e_lo=0, E_L=8, fp8=True)["y"]
    b = O.moe_layer(d["logits"], d["x"], qd, k=2, e_lo=0, E_L=8, fp8=True,
                    quantize_activations=True)["y"]
    rel = np.linalg.norm(a - b, axis=1) / np.linalg.norm(a, axis=1)
    assert 1e-3 < rel.min() and rel.max() < 0.12
    toks = [0, 17, 39]
    np.testing.assert_allclose(
        O.moe_layer_tokens(d["logits"], d["x"], qd, toks, k=2, e_lo=0, E_L=8, fp8=True,
                           quantize_activations=True), b[toks], rtol=1e-12, atol=1e-300)
