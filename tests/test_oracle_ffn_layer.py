"""Pins of the oracle's expert FFN and whole layer: tabulated SiLU values,
torch's library SiLU/linear, the E = 1 reduction to a dense SwiGLU FFN,
a gate/up asymmetry check, linearity, identity experts, a dense
all-experts reference with masked gates (independent of the permutation),
the shard-sum, row-independence and token-permutation invariants, and
brute-force loops on tiny shapes."""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from moe_expert_layer_gate_amd import inputs as synth
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_cfg(T=48, H=64, E=8, E_L=8, e_lo=0, k=2, I=32, **kw):
    return synth.MoEConfig("t", T=T, H=H, E=E, E_L=E_L, e_lo=e_lo, k=k, I=I, **kw)


def draw(cfg, seed, std=0.3, x_std=1.0):
    return synth.make_inputs(cfg, seed, std=std, x_std=x_std)


def test_silu_tabulated_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "silu_points.txt"))
            if l.strip() and not l.startswith("#")]
    a = np.array([float(r[0]) for r in rows])
    want = np.array([float(r[1]) for r in rows])
    np.testing.assert_allclose(O.silu(a), want, rtol=2e-15, atol=0)


def test_silu_matches_torch_library():
    a = np.linspace(-60, 60, 2001)
    np.testing.assert_allclose(O.silu(a), F.silu(torch.from_numpy(a)).numpy(),
                               rtol=1e-15, atol=1e-300)
    assert O.silu(np.array([-800.0]))[0] == 0.0


def test_expert_ffn_matches_torch_dense_swiglu():
    rng = np.random.default_rng(1)
    H, I, n = 24, 10, 7
    x = rng.standard_normal((n, H))
    w13 = rng.standard_normal((2 * I, H)) * 0.5
    w2 = rng.standard_normal((H, I)) * 0.5
    h, y = O.expert_ffn(x, w13, w2)
    tx, t13, t2 = (torch.from_numpy(v) for v in (x, w13, w2))
    g = F.linear(tx, t13[:I])
    u = F.linear(tx, t13[I:])
    th = F.silu(g) * u
    np.testing.assert_allclose(h, th.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y, F.linear(th, t2).numpy(), rtol=1e-12, atol=1e-13)


def test_gate_and_up_are_not_swapped():
    """x = e_0, gate column = [1, -1], up column = [1, 1], W2 = identity:
    y = [silu(1), silu(-1)].  With gate and up swapped the second entry
    would be -silu(1) instead."""
    H = I = 2
    x = np.array([[1.0, 0.0]])
    w13 = np.zeros((2 * I, H))
    w13[0, 0], w13[1, 0] = 1.0, -1.0      # gate rows
    w13[2, 0], w13[3, 0] = 1.0, 1.0       # up rows
    _, y = O.expert_ffn(x, w13, np.eye(2))
    np.testing.assert_allclose(y[0], [0.7310585786300049, -0.2689414213699951], rtol=1e-15)


def test_brute_force_loops_tiny():
    rng = np.random.default_rng(2)
    H, I, n = 5, 3, 4
    x = rng.standard_normal((n, H))
    w13 = rng.standard_normal((2 * I, H))
    w2 = rng.standard_normal((H, I))
    _, y = O.expert_ffn(x, w13, w2)
    import math
    for r in range(n):
        for o in range(H):
            acc = 0.0
            for i in range(I):
                g = sum(x[r, c] * w13[i, c] for c in range(H))
                u = sum(x[r, c] * w13[I + i, c] for c in range(H))
                acc += g / (1 + math.exp(-g)) * u * w2[o, i]
            assert abs(acc - y[r, o]) <= 1e-12 * (1 + abs(acc))


def test_single_expert_layer_is_dense_ffn():
    """E = 1, k = 1: every token goes to the one expert with weight 1."""
    cfg = small_cfg(T=20, H=32, E=1, E_L=1, k=1, I=16)
    d = draw(cfg, 3)
    out = O.moe_layer(d["logits"], d["x"], d, k=1, e_lo=0, E_L=1)
    x = torch.from_numpy(O.bf16_to_f64(d["x"]))
    w13 = torch.from_numpy(O.bf16_to_f64(d["w13"][0]))
    w2 = torch.from_numpy(O.bf16_to_f64(d["w2"][0]))
    ref = F.linear(F.silu(F.linear(x, w13[:16])) * F.linear(x, w13[16:]), w2)
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-15)


def test_linearity_in_w2_and_zero_w13():
    cfg = small_cfg()
    d = draw(cfg, 4)
    base = O.moe_layer(d["logits"], d["x"], d, k=2, e_lo=0, E_L=8)["y"]
    d2 = dict(d)
    # doubling a bf16 value is exact: add one to the exponent field
    d2["w2"] = (d["w2"].astype(np.uint32) + (1 << 7)).astype(np.uint16)
    d2["w2"][d["w2"] & 0x7FFF == 0] = d["w2"][d["w2"] & 0x7FFF == 0]
    np.testing.assert_allclose(O.moe_layer(d["logits"], d["x"], d2, k=2, e_lo=0, E_L=8)["y"],
                               2 * base, rtol=1e-13, atol=1e-300)
    d3 = dict(d)
    d3["w13"] = np.zeros_like(d["w13"])
    assert np.all(O.moe_layer(d["logits"], d["x"], d3, k=2, e_lo=0, E_L=8)["y"] == 0)


@pytest.mark.parametrize("e_lo,E_L", [(0, 16), (4, 8), (12, 4)])
def test_identity_experts_return_weighted_input(e_lo, E_L):
    """Dispatch then combine with identity experts (y_perm = x_perm) gives
    x times the sum of the token's local weights; x itself when every expert
    is local."""
    cfg = small_cfg(T=60, H=16, E=16, E_L=E_L, e_lo=e_lo, k=4)
    d = synth.make_inputs(cfg, 5, weights=False, x_std=1.0)
    ids, w = O.route(d["logits"], 4)
    L = O.index_build(ids, e_lo, E_L)
    x = O.bf16_to_f64(d["x"])
    y = O.combine(O.dispatch(x, L["row_token"]), L["token_slot_row"], w)
    local = (ids >= e_lo) & (ids < e_lo + E_L)
    np.testing.assert_allclose(y, x * (w * local).sum(1, keepdims=True), rtol=1e-14, atol=0)
    if E_L == 16:
        np.testing.assert_allclose(y, x, rtol=1e-14)


def dense_masked_reference(d, k, e_lo, E_L):
    """Every local expert on every token (torch, float64), weighted by a
    [T, E_L] gate matrix that is w_s where the token's slot s picked that
    expert and 0 elsewhere.  Uses no permutation at all."""
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
        w13 = torch.from_numpy(O.bf16_to_f64(d["w13"][e]))
        w2 = torch.from_numpy(O.bf16_to_f64(d["w2"][e]))
        I = w13.shape[0] // 2
        fe = F.linear(F.silu(F.linear(x, w13[:I])) * F.linear(x, w13[I:]), w2)
        y += torch.from_numpy(G[:, e:e + 1]) * fe
    return y.numpy()


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("shape", [dict(), dict(E=16, E_L=16, k=4),
                                   dict(E=16, E_L=4, e_lo=8, k=4), dict(E=8, E_L=8, k=8)])
def test_layer_matches_dense_masked_reference(seed, shape):
    cfg = small_cfg(**shape)
    d = draw(cfg, seed)
    out = O.moe_layer(d["logits"], d["x"], d, k=cfg.k, e_lo=cfg.e_lo, E_L=cfg.E_L)
    ref = dense_masked_reference(d, cfg.k, cfg.e_lo, cfg.E_L)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-10, atol=1e-12)


def test_tiny_workload_matches_dense_masked_reference():
    cfg = synth.config(1)
    d = synth.make_inputs(cfg, 1)
    out = O.moe_layer(d["logits"], d["x"], d, k=cfg.k, e_lo=0, E_L=cfg.E_L)
    ref = dense_masked_reference(d, cfg.k, 0, cfg.E_L)
    scale = np.abs(ref).max()
    np.testing.assert_allclose(out["y"], ref, rtol=1e-9, atol=1e-12 * scale)


def test_shard_sum_equals_whole_layer():
    """Summing the partial outputs of all expert-parallel shards gives the
    layer with every expert local (every expert covered exactly once)."""
    E, k = 16, 4
    full = small_cfg(T=40, H=32, E=E, E_L=E, k=k, I=16)
    d = draw(full, 7)
    whole = O.moe_layer(d["logits"], d["x"], d, k=k, e_lo=0, E_L=E)["y"]
    acc = np.zeros_like(whole)
    for e_lo in range(0, E, 4):
        dd = dict(d, w13=d["w13"][e_lo:e_lo + 4], w2=d["w2"][e_lo:e_lo + 4])
        acc += O.moe_layer(d["logits"], d["x"], dd, k=k, e_lo=e_lo, E_L=4)["y"]
    np.testing.assert_allclose(acc, whole, rtol=1e-12, atol=1e-15)


def test_replica_segments_are_independent():
    cfg = small_cfg(T=64, H=32, E=16, E_L=8, e_lo=0, k=4, I=16, replicas=4,
                    logits="gumbel_zipf")
    d = draw(cfg, 8)
    ro = d["replica_offsets"]
    assert ro[0] == 0 and ro[-1] == cfg.T and np.all(np.diff(ro) >= 0)
    whole = O.moe_layer(d["logits"], d["x"], d, k=4, e_lo=0, E_L=8)["y"]
    parts = [O.moe_layer(d["logits"][a:b], d["x"][a:b], d, k=4, e_lo=0, E_L=8)["y"]
             for a, b in zip(ro[:-1], ro[1:])]
    np.testing.assert_allclose(np.concatenate(parts), whole, rtol=1e-13, atol=1e-300)


def test_token_permutation_permutes_output():
    cfg = small_cfg(T=50, H=32, E=8, E_L=8, k=2, I=16)
    d = draw(cfg, 9)
    a = O.moe_layer(d["logits"], d["x"], d, k=2, e_lo=0, E_L=8)
    p = np.random.default_rng(0).permutation(cfg.T)
    b = O.moe_layer(d["logits"][p], d["x"][p], d, k=2, e_lo=0, E_L=8)
    np.testing.assert_array_equal(b["ids"], a["ids"][p])
    np.testing.assert_allclose(b["y"], a["y"][p], rtol=1e-13, atol=1e-300)


def test_spot_check_rows_equal_whole_layer():
    cfg = small_cfg(T=70, H=32, E=16, E_L=8, e_lo=4, k=4, I=16)
    d = draw(cfg, 10)
    whole = O.moe_layer(d["logits"], d["x"], d, k=4, e_lo=4, E_L=8)["y"]
    toks = [0, 5, 69, 33, 5]
    np.testing.assert_allclose(O.moe_layer_tokens(d["logits"], d["x"], d, toks, k=4, e_lo=4, E_L=8),
                               whole[toks], rtol=1e-13, atol=1e-300)


def test_tokens_without_local_slot_are_zero():
    cfg = small_cfg(T=30, H=16, E=16, E_L=1, e_lo=15, k=2, I=8)
    d = draw(cfg, 11)
    out = O.moe_layer(d["logits"], d["x"], d, k=2, e_lo=15, E_L=1)
    none = ~(out["ids"] == 15).any(1)
    assert none.any()
    assert np.all(out["y"][none] == 0)


def test_empty_batch_layer():
    cfg = small_cfg(T=0)
    d = draw(cfg, 0)
    out = O.moe_layer(d["logits"], d["x"], d, k=2, e_lo=0, E_L=8)
    assert out["y"].shape == (0, cfg.H) and out["offsets"][-1] == 0
    assert out["h"].shape == (0, cfg.I)


def test_no_local_rows_keeps_h_width():
    """Every pick lands off the shard: h is [0, I] (contiguous) or all-zero
    [E_L * capacity, I] (masked), and y is zero."""
    cfg = small_cfg(T=5, H=16, E=8, E_L=2, e_lo=6, k=2, I=12)
    d = draw(cfg, 3)
    d["logits"][:, 6:] = -1e4                         # experts 6 and 7 never picked
    out = O.moe_layer(d["logits"], d["x"], d, k=2, e_lo=6, E_L=2)
    assert out["offsets"][-1] == 0 and out["h"].shape == (0, cfg.I)
    assert np.all(out["y"] == 0)
    h, y = O.grouped_ffn_masked(np.zeros((2 * 4, cfg.H)), np.zeros(2, np.int64), 4,
                                d["w13"], d["w2"])
    assert h.shape == (8, cfg.I) and not h.any() and not y.any()


@pytest.mark.parametrize("e_lo,E_L", [(0, 8), (4, 2)])
def test_shared_expert_adds_dense_ffn_with_unit_weight(e_lo, E_L):
    cfg = small_cfg(T=24, H=32, E=8, E_L=E_L, e_lo=e_lo, k=2, I=16, I_s=24)
    d = draw(cfg, 12)
    with_s = O.moe_layer(d["logits"], d["x"], d, k=2, e_lo=e_lo, E_L=E_L)
    no_s = O.moe_layer(d["logits"], d["x"], {"w13": d["w13"], "w2": d["w2"]},
                       k=2, e_lo=e_lo, E_L=E_L)
    x = torch.from_numpy(O.bf16_to_f64(d["x"]))
    s13 = torch.from_numpy(O.bf16_to_f64(d["ws13"]))
    s2 = torch.from_numpy(O.bf16_to_f64(d["ws2"]))
    dense = F.linear(F.silu(F.linear(x, s13[:24])) * F.linear(x, s13[24:]), s2).numpy()
    np.testing.assert_allclose(with_s["y"] - no_s["y"], dense, rtol=1e-9, atol=1e-13)
    toks = [0, 7, 23]
    np.testing.assert_allclose(
        O.moe_layer_tokens(d["logits"], d["x"], d, toks, k=2, e_lo=e_lo, E_L=E_L),
        with_s["y"][toks], rtol=1e-13, atol=1e-300)
