"""Host-side checks of the C ABI that need no GPU: the library loads, every
function include/moe_layer.h declares is exported, workspace sizing, status
names, and argument validation (which returns before anything is enqueued)."""
import ctypes
import os
import re

import pytest

from moe_expert_layer_gate_amd import inputs as synth
from moe_expert_layer_gate_amd import moelayer as ml

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z0-9_]+)\s*\(",
                             src, flags=re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_expected_calls():
    assert {"moe_route", "moe_dispatch", "moe_grouped_ffn", "moe_grouped_ffn_gather",
            "moe_combine", "moe_layer",
            "moe_quantize_fp8", "moe_pack_panel", "moe_workspace_bytes", "moe_status_str",
            "moe_abi_version"} <= declared_functions()


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(ml.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and the binding knows each of them
    assert declared_functions() <= set(ml.SIGNATURES)


def test_abi_version_and_status_strings():
    assert ml.lib().moe_abi_version() == 10
    assert ml.status_str(0) == "MOE_OK"
    assert ml.status_str(3) == "MOE_ERR_WORKSPACE"
    assert ml.status_str(99) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workspace_sizes(cid):
    p = ml.Problem.from_config(synth.config(cid))
    layer = ml.workspace_bytes(p, ml.STAGE_LAYER)
    disp = ml.workspace_bytes(p, ml.STAGE_DISPATCH)
    ffn = ml.workspace_bytes(p, ml.STAGE_FFN)
    assert layer > 0 and disp > 0 and ffn > 0
    assert layer > disp and layer > ffn
    # the layer workspace holds at least the expert outputs and h (the up GEMM
    # gathers its rows straight from the tokens; block-FP8 also holds the
    # tokens quantised once, T rows)
    beta = 1 if p.fp8 else 2
    assert layer >= p.n_cap * (2 * p.H + beta * p.I) + (p.T * p.H if p.fp8 else 0)
    assert ml.workspace_bytes(p, 7) == 0


@pytest.mark.parametrize("fmt", ["fp8", "mx"])
def test_quantised_layer_workspace_holds_the_tokens_once(fmt):
    """Block-FP8 and MX layers with a shared expert quantise the tokens once
    ([T, H] codes plus scales, read by the routed and the shared expert): the
    shared expert adds its own FFN scratch and its [T, H] bf16 output to the
    workspace, not a second copy of the quantised tokens."""
    kw = dict(T=4096, H=1024, E=16, k=4, e_lo=0, E_L=8, I=256, fp8=fmt == "fp8", mx=fmt == "mx")
    with_shared = ml.workspace_bytes(ml.Problem(I_s=256, **kw))
    without = ml.workspace_bytes(ml.Problem(I_s=0, **kw))
    q = ml.Problem(T=kw["T"], H=kw["H"], E=1, k=1, e_lo=0, E_L=1, I=256, fp8=kw["fp8"],
                   mx=kw["mx"])
    shared_ffn = ml.workspace_bytes(q, ml.STAGE_FFN)
    T, H = kw["T"], kw["H"]
    extra = with_shared - without
    assert extra >= shared_ffn - 256 + 2 * T * H
    # alignment of a few carved buffers at most; a second quantised copy of
    # the tokens would add T * H bytes more
    assert extra <= shared_ffn + 2 * T * H + 2048 < shared_ffn + 3 * T * H


def test_workspace_flags_argument_checks():
    p = ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256)
    pc = p.c()
    L = ml.lib()
    n = ml.workspace_bytes(p)
    # the dispatch stage has no FFN flags; null or misaligned flag pointer;
    # short workspace (all rejected before anything is enqueued)
    assert L.moe_workspace_flags(ctypes.byref(pc), ml.STAGE_DISPATCH, 256, n, 256,
                                 None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_flags(ctypes.byref(pc), ml.STAGE_LAYER, 256, n, None,
                                 None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_flags(ctypes.byref(pc), ml.STAGE_LAYER, 256, n, 258,
                                 None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_flags(ctypes.byref(pc), ml.STAGE_LAYER, 256, 16, 256,
                                 None) == ml.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("bad", [
    dict(T=-1), dict(E=0), dict(k=0), dict(k=9, E=8), dict(k=33, E=64), dict(E_L=0),
    dict(e_lo=6, E_L=4), dict(e_lo=-1), dict(H=100), dict(I=96), dict(I_s=64), dict(H=0),
    dict(E=2000, E_L=8), dict(layout=4), dict(layout=-1)])
def test_invalid_problems_rejected(bad):
    base = dict(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256, I_s=0, fp8=False)
    base.update(bad)
    p = ml.Problem(**base)
    assert ml.workspace_bytes(p) == 0
    pc = p.c()
    # validation fails before any pointer is looked at or anything enqueued
    assert ml.lib().moe_route(ctypes.byref(pc), 16, 16, 16, None) == ml.MOE_ERR_INVALID_ARG


def test_null_and_misaligned_pointers_rejected():
    p = ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256)
    pc = p.c()
    L = ml.lib()
    assert L.moe_route(ctypes.byref(pc), None, 256, 256, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_route(ctypes.byref(pc), 257, 256, 256, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, 256, 256, 256, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_combine(ctypes.byref(pc), 256, None, 256, None, 256, None) == ml.MOE_ERR_INVALID_ARG
    w = ml.moe_weights(None, 256, None, None, None, None, None, None)
    assert L.moe_layer(ctypes.byref(pc), 256, 256, ctypes.byref(w), 256, 256, 1 << 30,
                       None) == ml.MOE_ERR_INVALID_ARG
    w = ml.moe_weights(256, 256, None, None, None, None, None, None)
    assert L.moe_layer(ctypes.byref(pc), 256, 256, ctypes.byref(w), 256, 256, 16,
                       None) == ml.MOE_ERR_WORKSPACE
    assert L.moe_dispatch(ctypes.byref(pc), *([256] * 8), None, None, 0, None) == ml.MOE_ERR_WORKSPACE
    # fp8 needs its scale pointers
    pf = ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256, fp8=True).c()
    w = ml.moe_weights(256, 256, None, None, None, None, None, None)
    assert L.moe_layer(ctypes.byref(pf), 256, 256, ctypes.byref(w), 256, 256, 1 << 40,
                       None) == ml.MOE_ERR_INVALID_ARG
    # shared expert needs its weights
    ps = ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256, I_s=128).c()
    w = ml.moe_weights(256, 256, None, None, None, None, None, None)
    assert L.moe_layer(ctypes.byref(ps), 256, 256, ctypes.byref(w), 256, 256, 1 << 40,
                       None) == ml.MOE_ERR_INVALID_ARG


def test_empty_batch_enqueues_nothing():
    """T = 0 is valid and returns before any HIP call (so it runs without a GPU)."""
    p = ml.Problem(T=0, H=256, E=8, k=2, e_lo=0, E_L=8, I=256)
    pc = p.c()
    L = ml.lib()
    assert L.moe_route(ctypes.byref(pc), 256, 256, 256, None) == ml.MOE_OK
    w = ml.moe_weights(256, 256, None, None, None, None, None, None)
    n = ml.workspace_bytes(p)
    assert L.moe_layer(ctypes.byref(pc), 256, 256, ctypes.byref(w), 256, 256, n, None) == ml.MOE_OK


def test_quantize_argument_checks():
    L = ml.lib()
    assert L.moe_quantize_fp8(256, 1, 128, 100, 128, 256, 256, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_fp8(256, 1, 128, 128, 64, 256, 256, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_fp8(None, 1, 128, 128, 128, 256, 256, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_fp8(256, 0, 128, 128, 128, 256, 256, None) == ml.MOE_OK


def test_layout_checks():
    L = ml.lib()
    # no panel layouts for block-FP8
    pf = ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256, fp8=True,
                    layout=ml.LAYOUT_PANEL_WEIGHTS)
    assert ml.workspace_bytes(pf) == 0
    pc = pf.c()
    assert L.moe_route(ctypes.byref(pc), 16, 16, 16, None) == ml.MOE_ERR_UNSUPPORTED
    for lay in (ml.LAYOUT_PANEL_WEIGHTS, ml.LAYOUT_PANEL_ACTS, 3):
        p = ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256, layout=lay)
        assert ml.workspace_bytes(p) == ml.workspace_bytes(
            ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256))
    # panel activations need 64 N_cap < 2^31 (N_cap = T min(k, E_L))
    big = dict(T=1 << 22, H=128, E=8, k=8, e_lo=0, E_L=8, I=128)
    assert ml.workspace_bytes(ml.Problem(**big)) > 0
    pb = ml.Problem(**big, layout=ml.LAYOUT_PANEL_ACTS).c()
    assert L.moe_route(ctypes.byref(pb), 16, 16, 16, None) == ml.MOE_ERR_UNSUPPORTED


def test_pack_panel_argument_checks():
    L = ml.lib()
    assert L.moe_pack_panel(256, 1, 4, 48, 1 << 20, None) == ml.MOE_ERR_INVALID_ARG    # cols % 32
    assert L.moe_pack_panel(256, 1, 4, 0, 1 << 20, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel(None, 1, 4, 64, 1 << 20, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel(264, 1, 4, 64, 1 << 20, None) == ml.MOE_ERR_INVALID_ARG   # misaligned
    assert L.moe_pack_panel(256, 1, 4, 64, 512, None) == ml.MOE_ERR_INVALID_ARG       # overlap
    assert L.moe_pack_panel(256, -1, 4, 64, 1 << 20, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel(256, 1 << 20, 1 << 20, 64, 1 << 40, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel(256, 0, 4, 64, 1 << 20, None) == ml.MOE_OK
    assert L.moe_pack_panel(256, 3, 0, 64, 1 << 20, None) == ml.MOE_OK


def test_gather_ffn_argument_checks():
    L = ml.lib()
    p = ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256).c()
    w = ml.moe_weights(256, 256, None, None, None, None, None, None)
    n = ml.workspace_bytes(ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256), ml.STAGE_FFN)
    # x, x_scale, row_token, offsets, w, h, h_scale, y_perm, ws, ws_bytes, stream
    ok_args = [256, None, 256, 256, ctypes.byref(w), None, None, 256, 256, n, None]
    for i in (0, 2, 3, 7):      # x, row_token, offsets, y_perm
        bad = list(ok_args)
        bad[i] = None
        assert L.moe_grouped_ffn_gather(ctypes.byref(p), *bad) == ml.MOE_ERR_INVALID_ARG
    bad = list(ok_args)
    bad[9] = 16                 # workspace too small
    assert L.moe_grouped_ffn_gather(ctypes.byref(p), *bad) == ml.MOE_ERR_WORKSPACE
    # block-FP8: the token scales (and, with h, the h scales) are required
    pq = ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256, fp8=True)
    wq = ml.moe_weights(256, 256, None, None, 256, 256, None, None)
    nq = ml.workspace_bytes(pq, ml.STAGE_FFN)
    fq = [256, 256, 256, 256, ctypes.byref(wq), None, None, 256, 256, nq, None]
    pqc = pq.c()
    bad = list(fq)
    bad[1] = None
    assert L.moe_grouped_ffn_gather(ctypes.byref(pqc), *bad) == ml.MOE_ERR_INVALID_ARG
    bad = list(fq)
    bad[5] = 256                # h without h_scale
    assert L.moe_grouped_ffn_gather(ctypes.byref(pqc), *bad) == ml.MOE_ERR_INVALID_ARG
    p0q = ml.Problem(T=0, H=256, E=8, k=2, e_lo=0, E_L=8, I=256, fp8=True).c()
    assert L.moe_grouped_ffn_gather(ctypes.byref(p0q), *fq) == ml.MOE_OK
    # T = 0: nothing to do
    p0 = ml.Problem(T=0, H=256, E=8, k=2, e_lo=0, E_L=8, I=256).c()
    assert L.moe_grouped_ffn_gather(ctypes.byref(p0), *ok_args) == ml.MOE_OK
    # index-only dispatch (x_perm = NULL) still checks the other pointers
    pd = ml.Problem(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256)
    nd = ml.workspace_bytes(pd, ml.STAGE_DISPATCH)
    assert L.moe_dispatch(ctypes.byref(p), None, *([256] * 6), None, None, 256, nd,
                          None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch(ctypes.byref(p), *([256] * 6), 264, None, None, 256, nd,
                          None) == ml.MOE_ERR_INVALID_ARG   # misaligned token_slot_row


def test_activation_checks():
    L = ml.lib()
    base = dict(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256)
    assert ml.workspace_bytes(ml.Problem(**base, act="gelu")) > 0
    pc = ml.Problem(**base, act="gelu").c()
    pc.activation = 2
    assert L.moe_route(ctypes.byref(pc), 16, 16, 16, None) == ml.MOE_ERR_INVALID_ARG
    pf = ml.Problem(**base, fp8=True, act="gelu").c()     # the standard MLP is bf16 only
    assert L.moe_route(ctypes.byref(pf), 16, 16, 16, None) == ml.MOE_ERR_UNSUPPORTED


def test_capacity_checks():
    """Masked layout: capacity 0 (contiguous) or >= T; E_L * capacity rows."""
    L = ml.lib()
    base = dict(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256)
    for cap, want in ((-1, ml.MOE_ERR_INVALID_ARG), (15, ml.MOE_ERR_INVALID_ARG),
                      ((1 << 24) + 1, ml.MOE_ERR_INVALID_ARG)):
        pc = ml.Problem(**base, capacity=cap).c()
        assert L.moe_route(ctypes.byref(pc), 16, 16, 16, None) == want
        assert ml.workspace_bytes(ml.Problem(**base, capacity=cap)) == 0
    # E_L * capacity must stay below 2^31 rows
    pc = ml.Problem(**dict(base, E=1024, E_L=1024), capacity=1 << 21).c()
    assert L.moe_route(ctypes.byref(pc), 16, 16, 16, None) == ml.MOE_ERR_UNSUPPORTED
    # the buffers grow to E_L * capacity rows
    small = ml.workspace_bytes(ml.Problem(**base))
    masked = ml.workspace_bytes(ml.Problem(**base, capacity=64))
    assert masked > small
    p = ml.Problem(**base, capacity=64)
    assert p.n_cap == 8 * 64
    assert masked >= p.n_cap * (2 * p.H + 2 * p.I)
    # a capacity of exactly T is valid; T = 0 is always a no-op
    assert ml.workspace_bytes(ml.Problem(**base, capacity=16)) > 0
    p0 = ml.Problem(**dict(base, T=0), capacity=16).c()
    assert L.moe_route(ctypes.byref(p0), 16, 16, 16, None) == ml.MOE_OK


def test_mxfp4_checks():
    """MXFP4: panel weights but row-major activations, and the gated MLP
    only; scale pointers are required like block-FP8's; moe_quantize_mx and
    moe_pack_panel_mx argument checks."""
    L = ml.lib()
    base = dict(T=16, H=256, E=8, k=2, e_lo=0, E_L=8, I=256, mx=True)
    assert ml.workspace_bytes(ml.Problem(**base)) > 0
    assert ml.workspace_bytes(ml.Problem(**base, layout=ml.LAYOUT_PANEL_WEIGHTS)) == \
        ml.workspace_bytes(ml.Problem(**base))
    for bad, want in ((dict(layout=ml.LAYOUT_PANEL_ACTS), ml.MOE_ERR_UNSUPPORTED),
                      (dict(layout=3), ml.MOE_ERR_UNSUPPORTED),
                      (dict(act="gelu"), ml.MOE_ERR_UNSUPPORTED)):
        pc = ml.Problem(**base, **bad).c()
        assert L.moe_route(ctypes.byref(pc), 16, 16, 16, None) == want
    pc = ml.Problem(**base).c()
    pc.dtype = 3
    assert L.moe_route(ctypes.byref(pc), 16, 16, 16, None) == ml.MOE_ERR_INVALID_ARG
    # the gathering FFN needs the MX token scales
    p = ml.Problem(**base).c()
    w = ml.moe_weights(256, 256, None, None, 256, 256, None, None)
    n = ml.workspace_bytes(ml.Problem(**base), ml.STAGE_FFN)
    assert L.moe_grouped_ffn_gather(ctypes.byref(p), 256, None, 256, 256, ctypes.byref(w), None,
                                    None, 256, 256, n, None) == ml.MOE_ERR_INVALID_ARG
    # moe_grouped_ffn needs the activation scales
    assert L.moe_grouped_ffn(ctypes.byref(p), 256, None, 256, ctypes.byref(w), None, None, 256,
                             256, n, None) == ml.MOE_ERR_INVALID_ARG
    w0 = ml.moe_weights(256, 256, None, None, None, None, None, None)   # no weight scales
    assert L.moe_grouped_ffn(ctypes.byref(p), 256, 256, 256, ctypes.byref(w0), None, None, 256,
                             256, n, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_mx(256, 1, 4, 48, 0, 256, 256, None) == ml.MOE_ERR_INVALID_ARG   # cols % 32
    assert L.moe_quantize_mx(256, 1, 4, 64, 2, 256, 256, None) == ml.MOE_ERR_INVALID_ARG   # elem
    assert L.moe_quantize_mx(256, 1, 4, 64, 1, 256, 256, None) == ml.MOE_ERR_INVALID_ARG   # e4m3: cols % 128
    assert L.moe_quantize_mx(None, 1, 4, 64, 0, 256, 256, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_mx(256, 0, 4, 64, 0, 256, 256, None) == ml.MOE_OK
    # moe_pack_panel_mx: cols % 128, alignment, disjoint buffers
    a, b, c, d = 1 << 20, 2 << 20, 3 << 20, 4 << 20
    assert L.moe_pack_panel_mx(a, b, 1, 4, 64, c, d, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel_mx(a, b, 1, 4, 192, c, d, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel_mx(a, b, 1, 4, 1 << 21, c, d, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel_mx(a + 8, b, 1, 4, 128, c, d, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel_mx(None, b, 1, 4, 128, c, d, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel_mx(a, b, 1, 4, 128, a + 128, d, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel_mx(a, b, 1, 4, 128, c, c + 16, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel_mx(a, b, -1, 4, 128, c, d, None) == ml.MOE_ERR_INVALID_ARG
    assert L.moe_pack_panel_mx(a, b, 0, 4, 128, c, d, None) == ml.MOE_OK
    assert L.moe_pack_panel_mx(a, b, 3, 0, 128, c, d, None) == ml.MOE_OK
