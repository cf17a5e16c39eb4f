"""Helpers of the GPU parity tests: run the library's stages on seeded
inputs and compare with the oracle.  (Not a test module.)"""
from __future__ import annotations

import functools
import sys

import numpy as np
import pytest

from moe_expert_layer_gate_amd import inputs as synth
from oracle import moe_oracle as O

# Output gates: maximum over rows of ||y_t - y*_t|| / ||y*_t||.
TOL_BF16 = 2e-2
TOL_FP8 = 6e-2


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def rel_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """Max per-row relative l2 error.  Rows whose reference is exactly zero
    must come out exactly zero (returns inf otherwise)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.shape[0] == 0:
        return 0.0
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    zero = den == 0
    if np.any(num[zero] != 0):
        return float("inf")
    den = np.where(zero, 1.0, den)
    return float((num / den).max())


def rel_rows_all(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row relative l2 errors (rows whose reference is exactly zero: 0 if
    the row is exactly zero too, else inf)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    zero = den == 0
    out = num / np.where(zero, 1.0, den)
    out[zero & (num != 0)] = np.inf
    return out


def global_rel(got, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    d = np.linalg.norm(np.asarray(got, dtype=np.float64) - ref)
    n = np.linalg.norm(ref)
    return float(d / n) if n > 0 else float(d)


def unpanel(t, rows: int, cols: int):
    """A [rows, cols] matrix stored in panel layout ([cols/32][rows][32],
    element (r, c) at ((c // 32) * rows + r) * 32 + c % 32) -> row major."""
    return t.reshape(cols // 32, rows, 32).permute(1, 0, 2).reshape(rows, cols)


def small_cfg(**kw) -> synth.MoEConfig:
    base = dict(name="t", T=64, H=256, E=8, E_L=8, e_lo=0, k=2, I=256)
    base.update(kw)
    return synth.MoEConfig(**base)


class OracleWeights:
    """The oracle's own view of the weights, decoded per expert on demand
    (fp8 / MXFP4: quantised by the oracle itself from the bf16 draws), cached."""

    def __init__(self, d, fp8: bool, mx: bool = False):
        self.d, self.fp8, self.mx = d, fp8 or mx, mx

    @functools.lru_cache(maxsize=None)
    def _q(self, name, e):
        m = self.d[name] if e is None else self.d[name][e]
        if self.mx:
            return O.mx_quantize(O.bf16_to_f64(m), "e2m1")
        return O.quantize_blocks(O.bf16_to_f64(m), 128, 128)

    def codes(self, name, e=None):
        return self._q(name, e)

    @functools.lru_cache(maxsize=64)
    def w(self, name, e=None):
        if self.mx:
            q, s = self._q(name, e)
            return O.mx_dequantize(q, s, "e2m1")
        if self.fp8:
            q, s = self._q(name, e)
            return O.dequantize_blocks(q, s, 128, 128)
        m = self.d[name] if e is None else self.d[name][e]
        return O.bf16_to_f64(m)

    def as_layer_dict(self, E_L):
        """Weights dict in the form oracle.moe_layer expects."""
        if not self.fp8:
            out = {k: self.d[k] for k in ("w13", "w2", "ws13", "ws2") if k in self.d}
            return out
        out = {"w13_q": _ExpertView(self, "w13", 0, E_L), "w13_s": _ExpertView(self, "w13", 1, E_L),
               "w2_q": _ExpertView(self, "w2", 0, E_L), "w2_s": _ExpertView(self, "w2", 1, E_L)}
        if "ws13" in self.d:
            out["ws13_q"], out["ws13_s"] = self.codes("ws13")
            out["ws2_q"], out["ws2_s"] = self.codes("ws2")
        return out


class _ExpertView:
    """Indexable per-expert codes (part 0) or scales (part 1), quantised lazily."""

    def __init__(self, ow, name, part, n):
        self.ow, self.name, self.part, self.n = ow, name, part, n

    def __getitem__(self, e):
        return self.ow.codes(self.name, int(e))[self.part]

    def __len__(self):
        return self.n


def pack_e2m1(codes):
    """E2M1 codes [.., C] -> bytes [.., C/2], two per byte, low nibble first."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
