"""Pins of the oracle's standard (non-gated) GELU MLP (m = 1 first-layer
matrix): tabulated standard-normal values, two library routines (scipy's
normal distribution function, torch's exact GELU), the odd-part identity
gelu(a) - gelu(-a) = a, the tanh approximation being something else, a
dense reduction against torch, brute-force loops with math.erf, and the
layer against a dense all-experts reference with masked gates."""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.stats import norm

from moe_expert_layer_gate_amd import inputs as synth
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_cfg(T=40, H=48, E=8, E_L=8, e_lo=0, k=2, I=24, **kw):
    return synth.MoEConfig("t", T=T, H=H, E=E, E_L=E_L, e_lo=e_lo, k=k, I=I, act="gelu", **kw)


def test_gelu_tabulated_normal_distribution():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "normal_cdf_points.txt"))
            if l.strip() and not l.startswith("#")]
    z = np.array([float(r[0]) for r in rows])
    phi = np.array([float(r[1]) for r in rows])
    got = O.gelu(z)
    # four printed decimals of Phi: |gelu(z) - z Phi| <= 5e-5 |z|
    assert np.all(np.abs(got - z * phi) <= 5e-5 * np.abs(z) + 1e-300)
    assert O.gelu(np.array([0.0]))[0] == 0.0


def test_gelu_matches_library_routines():
    a = np.linspace(-12, 12, 4801)
    np.testing.assert_allclose(O.gelu(a), a * norm.cdf(a), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(O.gelu(a), F.gelu(torch.from_numpy(a), approximate="none").numpy(),
                               rtol=1e-13, atol=1e-15)


def test_gelu_odd_part_and_limits():
    a = np.linspace(-9, 9, 1801)
    # Phi(a) + Phi(-a) = 1  =>  gelu(a) - gelu(-a) = a
    np.testing.assert_allclose(O.gelu(a) - O.gelu(-a), a, atol=1e-15)
    assert abs(O.gelu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.gelu(np.array([-40.0]))[0]) < 1e-300


def test_gelu_is_exact_not_tanh_approximation():
    a = np.array([-2.0, -1.0, 1.5, 3.0])
    tanh_form = 0.5 * a * (1 + np.tanh(np.sqrt(2 / np.pi) * (a + 0.044715 * a ** 3)))
    assert np.max(np.abs(O.gelu(a) - tanh_form)) > 1e-4
    np.testing.assert_allclose(O.gelu(a), [a_ * 0.5 * (1 + math.erf(a_ / math.sqrt(2))) for a_ in a],
                               rtol=1e-15)


def test_expert_mlp_matches_torch_dense():
    rng = np.random.default_rng(2)
    H, I, n = 20, 12, 6
    x = rng.standard_normal((n, H))
    w1 = rng.standard_normal((I, H)) * 0.5
    w2 = rng.standard_normal((H, I)) * 0.5
    h, y = O.expert_ffn(x, w1, w2, activation="gelu")
    tx, t1, t2 = (torch.from_numpy(v) for v in (x, w1, w2))
    th = F.gelu(F.linear(tx, t1), approximate="none")
    np.testing.assert_allclose(h, th.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y, F.linear(th, t2).numpy(), rtol=1e-12, atol=1e-13)
    assert O.up_rows(I, "gelu") == I and O.up_rows(I, "swiglu") == 2 * I


def test_expert_mlp_brute_force_loops():
    rng = np.random.default_rng(3)
    H, I, n = 5, 4, 3
    x = rng.standard_normal((n, H))
    w1 = rng.standard_normal((I, H))
    w2 = rng.standard_normal((H, I))
    h, y = O.expert_ffn(x, w1, w2, activation="gelu")
    for r in range(n):
        hr = []
        for i in range(I):
            a = sum(x[r, c] * w1[i, c] for c in range(H))
            hr.append(a * 0.5 * math.erfc(-a / math.sqrt(2)))
        for o in range(H):
            want = sum(hr[i] * w2[o, i] for i in range(I))
            assert abs(y[r, o] - want) <= 1e-12 * (1 + abs(want))
        np.testing.assert_allclose(h[r], hr, rtol=1e-13)


def dense_masked_reference(d, k, e_lo, E_L):
    ids, w = O.route(d["logits"], k)
    T = ids.shape[0]
    G = np.zeros((T, E_L))
    for t in range(T):
        for s in range(k):
            e = ids[t, s] - e_lo
            if 0 <= e < E_L:
                G[t, e] = w[t, s]
    x = torch.from_numpy(O.bf16_to_f64(d["x"]))
    y = torch.zeros_like(x)
    for e in range(E_L):
        w1 = torch.from_numpy(O.bf16_to_f64(d["w13"][e]))
        w2 = torch.from_numpy(O.bf16_to_f64(d["w2"][e]))
        y += torch.from_numpy(G[:, e:e + 1]) * F.linear(F.gelu(F.linear(x, w1)), w2)
    return y.numpy()


@pytest.mark.parametrize("shape", [dict(), dict(E=16, E_L=4, e_lo=8, k=4)])
def test_gelu_layer_matches_dense_masked_reference(shape):
    cfg = small_cfg(**shape)
    d = synth.make_inputs(cfg, 5, std=0.3, x_std=1.0)
    assert d["w13"].shape == (cfg.E_L, cfg.I, cfg.H)
    out = O.moe_layer(d["logits"], d["x"], d, k=cfg.k, e_lo=cfg.e_lo, E_L=cfg.E_L,
                      activation="gelu")
    np.testing.assert_allclose(out["y"], dense_masked_reference(d, cfg.k, cfg.e_lo, cfg.E_L),
                               rtol=1e-10, atol=1e-12)
    # spot rows agree with the whole layer
    toks = np.array([0, 3, cfg.T - 1])
    yt = O.moe_layer_tokens(d["logits"], d["x"], d, toks, k=cfg.k, e_lo=cfg.e_lo, E_L=cfg.E_L,
                            activation="gelu")
    np.testing.assert_allclose(yt, out["y"][toks], rtol=1e-10, atol=1e-14)


def test_gelu_shared_expert_is_dense_mlp():
    cfg = small_cfg(T=24, E=8, E_L=4, e_lo=2, k=2, I_s=16)
    d = synth.make_inputs(cfg, 6, std=0.3, x_std=1.0)
    assert d["ws13"].shape == (cfg.I_s, cfg.H)
    with_s = O.moe_layer(d["logits"], d["x"], d, k=2, e_lo=2, E_L=4, activation="gelu")
    without = O.moe_layer(d["logits"], d["x"], {"w13": d["w13"], "w2": d["w2"]}, k=2, e_lo=2,
                          E_L=4, activation="gelu")
    x = torch.from_numpy(O.bf16_to_f64(d["x"]))
    sh = F.linear(F.gelu(F.linear(x, torch.from_numpy(O.bf16_to_f64(d["ws13"])))),
                  torch.from_numpy(O.bf16_to_f64(d["ws2"]))).numpy()
    np.testing.assert_allclose(with_s["y"] - without["y"], sh, rtol=1e-9, atol=1e-12)
