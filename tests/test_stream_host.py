"""The library's streaming-FFN host logic against the oracle (no GPU): the
launch plan and the threshold bit-exact, argument checks of the streamed
layer, and its workspace covering every group size."""
import ctypes

import numpy as np
import pytest

from moe_expert_layer_gate_amd import inputs as synth
from moe_expert_layer_gate_amd import moelayer as ml
from oracle import streamffn as S


@pytest.mark.parametrize("seed", range(60))
def test_plan_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 40))
    rows = [int(v) for v in rng.integers(0, 3000, size=n)]
    if n and seed % 3 == 0:
        rows[int(rng.integers(0, n))] = 0
    for theta in (0, 1, int(rng.integers(0, 20000)), 10 ** 12):
        assert ml.stream_plan(rows, theta) == S.launch_groups(rows, theta)


def test_plan_rejects_negative_counts_and_theta():
    L = ml.lib()
    r = (ctypes.c_int64 * 3)(5, -1, 7)
    e = (ctypes.c_int32 * 3)()
    ng = ctypes.c_int32(-9)
    assert L.moe_stream_plan(r, 3, 10, e, ctypes.byref(ng)) == ml.MOE_ERR_INVALID_ARG
    r2 = (ctypes.c_int64 * 3)(5, 1, 7)
    assert L.moe_stream_plan(r2, 3, -1, e, ctypes.byref(ng)) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_stream_plan(None, 0, 10, None, ctypes.byref(ng)) == ml.MOE_OK and ng.value == 0


@pytest.mark.parametrize("seed", range(40))
def test_threshold_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 20))
    counts = [int(v) for v in rng.choice(1 << 16, size=n, replace=False)]
    tp = [float(v) for v in rng.random(n) * 1000]
    for rho in (0.0, 0.5, 0.9, 1.0, float(rng.random())):
        assert ml.stream_threshold(counts, tp, rho) == S.threshold(counts, tp, rho)


def test_threshold_invalid():
    assert ml.stream_threshold([], [], 0.9) == -1
    assert ml.stream_threshold([10], [1.0], 1.5) == -1
    assert ml.stream_threshold([10], [float("nan")], 0.9) == -1
    assert ml.stream_threshold([-3], [1.0], 0.9) == -1


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_streamed_workspace_covers_every_group_size(cid):
    """One slice must hold the layer's workspace for any group of up to the
    requested size, across the GEMM path changes."""
    cfg = synth.config(cid)
    p = ml.Problem.from_config(cfg)
    for max_g in sorted({1, 7, 33, 64, 300, 1024, cfg.T // 3, cfg.T}):
        if max_g > cfg.T:
            continue
        total = ml.workspace_bytes_streamed(p, max_g, 3)
        assert total > 0 and total % 3 == 0
        slice_ = total // 3
        for t in sorted({1, 2, 5, 31, 32, 33, 40, 63, 64, 65, 255, 256, 257, 300, 511, 513,
                         max_g // 2, max_g - 1, max_g}):
            if 1 <= t <= max_g:
                import dataclasses
                need = ml.workspace_bytes(dataclasses.replace(p, T=t))
                assert need <= slice_, (max_g, t, need, slice_)


def test_streamed_argument_checks():
    L = ml.lib()
    p = ml.Problem(T=100, H=256, E=8, k=2, e_lo=0, E_L=8, I=256)
    pc = p.c()
    w = ml.moe_weights(256, 256, None, None, None, None, None, None)
    streams = (ctypes.c_void_p * 2)(None, None)
    n = ml.workspace_bytes_streamed(p, 60, 2)
    assert n > 0
    assert ml.workspace_bytes_streamed(p, 101, 2) == 0      # longer than the batch
    assert ml.workspace_bytes_streamed(p, 60, 0) == 0
    assert ml.workspace_bytes_streamed(p, 60, 65) == 0

    def call(groups, ns=2, ws_bytes=n):
        g = (ctypes.c_int32 * len(groups))(*groups)
        return L.moe_layer_streamed(ctypes.byref(pc), 256, 256, ctypes.byref(w), 256, g,
                                    len(groups) - 1, streams, ns, 256, ws_bytes)
    assert call([0, 50, 40, 100]) == ml.MOE_ERR_INVALID_ARG     # decreasing
    assert call([0, 50, 99]) == ml.MOE_ERR_INVALID_ARG          # does not end at T
    assert call([1, 50, 100]) == ml.MOE_ERR_INVALID_ARG         # does not start at 0
    assert call([0, 40, 100], ns=0) == ml.MOE_ERR_INVALID_ARG
    assert call([0, 40, 100], ws_bytes=n // 2) == ml.MOE_ERR_WORKSPACE   # a 60-token group
    g = (ctypes.c_int32 * 3)(0, 40, 100)
    assert L.moe_layer_streamed(ctypes.byref(pc), 264, 256, ctypes.byref(w), 256, g, 2, streams,
                                2, 256, n) == ml.MOE_ERR_INVALID_ARG   # misaligned logits
    # an empty batch enqueues nothing
    p0 = ml.Problem(T=0, H=256, E=8, k=2, e_lo=0, E_L=8, I=256).c()
    g0 = (ctypes.c_int32 * 1)(0)
    n0 = ml.workspace_bytes_streamed(ml.Problem(T=0, H=256, E=8, k=2, e_lo=0, E_L=8, I=256), 0, 1)
    assert L.moe_layer_streamed(ctypes.byref(p0), 256, 256, ctypes.byref(w), 256, g0, 0, streams,
                                1, 256, n0) == ml.MOE_OK


@pytest.mark.parametrize("seed", range(5))
def test_synthetic_arrival_order_is_the_oracle_reading(seed):
    off = synth.replica_split(np.random.default_rng(seed), 16384, 8)
    assert synth.replica_arrival(off) == S.arrival_order(off)
    perm = synth.arrival_permutation(off)
    assert sorted(perm.tolist()) == list(range(16384))
