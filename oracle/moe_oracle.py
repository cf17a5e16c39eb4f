"""Plain, slow CPU oracle of one GPU's expert-parallel MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only the tests, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing).

Everything is computed in float64 from the exact values of the inputs
(bfloat16 bit patterns are decoded exactly; float32 logits widen exactly).
No rounding of the GPU path is emulated, except where a floating-point step
decides an integer: the FP8 quantiser divides in float32, as the GPU does,
because its output is an integer code.

Sources (page title, then section / equation):
* "OverlapAdvisor: Modeling and Adapting Computation-Communication Overlap
  for Distributed MoE Serving" (OverlapAdvisor below): section 2.1 (top-k
  experts per token; dispatch to experts, combine back to the origin),
  section 4.2.1 (permute groups tokens by expert, unpermute restores the
  order; SwiGLU between the GroupGEMMs), section 4.2.2 and Eq. 6-8 (m = 2
  first-layer matrices for a gated MLP), Table 6 (FP8 gated SwiGLU group),
  section 4.4 (BF16 checkpoints quantised to block-FP8 at load time).
* "CascadeEP: Asynchronous Expert Execution for MoE Prefill under Attention
  Imbalance" (CascadeEP below): Appendix C, "Grouped FFN invocations"
  (per-expert row offsets from the selected counts, groups aligned to the
  GEMM tile, activations packed with their quantisation metadata, an inverse
  map to (token, routing slot)) and "Output return and combine" (each routed
  contribution weighted by its routing coefficient exactly once, summed at
  the origin, plus the shared-expert output).
* "ExpertPlex" page, Eq. 3 (tile-aware token count: the sum over experts
  with tokens of ceil(m_e / M_t)).

Readings taken where the pages leave a step open (each is also listed with
the design notes of the repository):
* Gate: the pages name only "top-k".  The gate here is the softmax of the
  router logits restricted to the k selected experts (equivalently a softmax
  over all E renormalised over the k selected: the partition function
  cancels).  Selection is on the raw logits, ordered by (value descending,
  expert index ascending); -0.0 equals +0.0.
* Slots whose expert is not local still count in the renormalisation; the
  shard returns its partial sum, and the partial sums of all shards add up
  to the whole layer.
* Local experts are the contiguous range [e_lo, e_lo + E_L).
* Permutation: segments in ascending local expert; inside a segment rows in
  ascending token (a stable counting sort of token-major (token, slot) pairs).
* SwiGLU: h = silu(gate) * up with silu(a) = a / (1 + exp(-a)); rows
  0..I-1 of W13 are the gate projection and rows I..2I-1 the up projection.
* Standard (non-gated) MLP, the pages' BF16 group: one first-layer matrix
  (m = 1, OverlapAdvisor Eq. 8) and GELU between the GEMMs (OverlapAdvisor
  Table 6); the pages give no formula, and the plainest reading is the
  exact GELU, gelu(a) = a * Phi(a) = a (1 + erf(a / sqrt 2)) / 2 (not the
  tanh approximation).  W1 [I, H] takes the place of W13.
* FP8: OCP E4M3FN codes (largest finite 448, no infinities); per-block scale
  s = amax / 448 in float32 (s = 1 for an all-zero block); code =
  round-to-nearest-even(v / s) with the quotient formed in float32 and
  saturated to +-448.  Weights use 128 x 128 blocks of each [N, K] matrix,
  activations use groups of 128 consecutive hidden elements of one token.
  The oracle's FP8 layer uses the dequantised weights (code * scale) as the
  layer's parameters and does not quantise x or h.
* Shared expert: always on, weight 1, same SwiGLU form, added in combine.
* MXFP4 (CascadeEP section 4.1 names MXFP4 routed-expert weights; the
  format is the OCP MX one): E2M1 elements with one E8M0 scale per 32
  consecutive elements of a weight row (along K), converted with the MX
  rule (shared exponent floor(log2 amax) - 2, round to nearest even,
  saturate at 6).  The GEMM inputs that go with them are MXFP8 (E4M3, one
  E8M0 scale per 32 elements of a token row, shared exponent floor(log2
  amax) - 8), the MX form of the FP8 activations.  As for block-FP8, the
  dequantised weights are the layer's parameters.
* Masked (fixed-capacity) layout, the decode-time alternative to the
  contiguous one (the ExpertPlex page's masked grouped-GEMM layout; the
  OverlapAdvisor page's Table 7, where the low-latency dispatch feeds the
  GroupGEMM with no permute step, and Table 6 note b, low latency for small
  batches): the pages give no capacity rule.  Reading: local expert e owns
  the fixed row block [e*C, (e+1)*C) and its pairs fill the first counts[e]
  rows, ascending token as in the contiguous layout; C >= every count (C >=
  T always suffices, a token picks an expert at most once); unused rows
  hold no pair.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

__all__ = [
    "bf16_to_f64", "route", "index_build", "tile_count", "dispatch", "silu",
    "expert_ffn", "grouped_ffn", "combine", "moe_layer", "moe_layer_tokens",
    "index_build_masked", "grouped_ffn_masked",
    "e4m3_value", "e4m3_encode", "quantize_blocks", "quantize_rows_groups",
    "dequantize_blocks", "fp8_activation", "E4M3_MAX", "e2m1_value", "e2m1_encode",
    "e8m0_value", "mx_quantize", "mx_dequantize", "mx8_activation",
]


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16), as float64.  A
    bfloat16 is the upper half of a float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


E4M3_MAX = 448.0


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Value of OCP E4M3FN codes (uint8) as float64.

    Bit 7 sign, bits 6..3 biased exponent (bias 7), bits 2..0 mantissa.
    Exponent field 0 is subnormal (m * 2^-9); field 15 with mantissa 7 is
    NaN (the format has no infinities); everything else is (1 + m/8) *
    2^(field - 7).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(ef == 0, m * 2.0 ** -9,
                   (1.0 + m / 8.0) * np.exp2(ef.astype(np.float64) - 7.0))
    val = np.where((ef == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


# Value of every non-negative finite code 0x00..0x7E, increasing with the code.
_POS_VALUES = e4m3_value(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round float values to E4M3FN codes: nearest representable value, ties
    to the code with an even mantissa, magnitudes beyond 448 saturate to
    448.  NaN inputs are not allowed.

    Written from the format: within a binade [2^e, 2^(e+1)), e >= -6, the
    spacing is 2^(e-3); below 2^-6 (subnormals) it is 2^-9.  Dividing by a
    power of two is exact, so rint (ties to even) of |v| / spacing gives the
    rounded magnitude exactly.  A magnitude that rounds up into the next
    binade lands on its first value, which is also the right result.
    """
    v64 = np.asarray(v, dtype=np.float64)
    if np.isnan(v64).any():
        raise ValueError("NaN has no E4M3 code here")
    neg = np.signbit(v64)
    a = np.abs(v64)
    _, ex = np.frexp(a)                     # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)              # binade exponent, floored at min normal
    # rint(a / 2^(e-3)) * 2^(e-3); the scalings by powers of two are exact.
    q = np.ldexp(np.rint(np.ldexp(a, 3 - e)), e - 3)
    q = np.minimum(q, E4M3_MAX)
    # Code of the magnitude q: subnormals are q / 2^-9; a normal q = (1 + m/8)
    # 2^eq has code (eq + 7) * 8 + m = (eq + 6) * 8 + q * 2^(3 - eq).
    _, eq = np.frexp(q)
    eq = eq - 1
    mag = np.where(q < 2.0 ** -6, np.ldexp(q, 9), (eq + 6) * 8 + np.ldexp(q, 3 - eq))
    mag_code = mag.astype(np.uint8)
    assert np.all(_POS_VALUES[mag_code] == q)   # decodes back to q exactly
    # -0.0 keeps its sign bit (code 0x80), as the hardware's sign does.
    return mag_code | (neg.astype(np.uint8) << 7)


# MX formats (OCP Microscaling Formats (MX) v1.0): blocks of 32 elements along
# a row share one E8M0 scale 2^(e - 127); elements are E2M1 (MXFP4) or E4M3
# (MXFP8).  The pages name MXFP4 routed-expert weights only (CascadeEP
# section 4.1); the format itself comes from the public OCP specification.

MX_BLOCK = 32
E2M1_MAX = 6.0
_E2M1_EMAX = 2     # exponent of the largest normal E2M1 value (6 = 1.5 * 2^2)
_E4M3_EMAX = 8     # 448 = 1.75 * 2^8


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    """Value of 4-bit E2M1 codes (0..15): sign bit 3, exponent bits 2..1
    (bias 1), mantissa bit 0; exponent field 0 is subnormal (m * 0.5)."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.ldexp(1.0, e - 1))
    return np.where(s == 1, -mag, mag)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Round to E2M1 codes: nearest representable value, ties to the code
    with an even mantissa bit, magnitudes beyond 6 saturate to 6.  Within a
    binade [2^e, 2^(e+1)), e >= 0, the spacing is 2^(e-1); below 1 (the
    subnormal range) it is 0.5."""
    v64 = np.asarray(v, dtype=np.float64)
    if np.isnan(v64).any():
        raise ValueError("NaN has no E2M1 code")
    neg = np.signbit(v64)
    a = np.abs(v64)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, 0)
    q = np.minimum(np.ldexp(np.rint(np.ldexp(a, 1 - e)), e - 1), E2M1_MAX)
    # code of the magnitude: subnormal/zero q in {0, 0.5} -> 2q; normal
    # q = (1 + m/2) 2^eq -> (eq + 1) * 2 + m
    _, eq = np.frexp(q)
    eq = eq - 1
    mag = np.where(q < 1.0, 2.0 * q, (eq + 1) * 2 + (np.ldexp(q, -eq) - 1.0) * 2)
    mag_code = mag.astype(np.int64)
    assert np.all(e2m1_value(mag_code) == q)
    return (mag_code | (neg.astype(np.int64) << 3)).astype(np.uint8)


def e8m0_value(codes: np.ndarray) -> np.ndarray:
    """Value of E8M0 scale codes: 2^(code - 127) (code 255, NaN, is never
    produced here)."""
    c = np.asarray(codes, dtype=np.int64)
    if np.any(c == 255):
        raise ValueError("E8M0 NaN")
    return np.ldexp(1.0, c - 127)


def mx_quantize(a: np.ndarray, elem: str):
    """MX conversion of a [R, C] array (C % 32 == 0) along its rows, as the
    OCP MX specification defines it: per block of 32, shared exponent
    floor(log2(amax)) - emax_elem (clamped to the E8M0 range [-127, 127];
    an all-zero block takes -127), X = 2^shared; element = the element
    format's rounding of v / X (round to nearest even, saturating to its
    largest normal).  elem: "e2m1" (MXFP4) or "e4m3" (MXFP8).
    Returns (element codes uint8 [R, C], E8M0 codes uint8 [R, C/32])."""
    a = np.asarray(a, dtype=np.float64)
    R, C = a.shape
    assert C % MX_BLOCK == 0
    g = a.reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = np.abs(g).max(axis=2)
    emax = _E2M1_EMAX if elem == "e2m1" else _E4M3_EMAX
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.where(amax > 0, ex - 1 - emax, -127)
    shared = np.clip(shared, -127, 127)
    quot = np.ldexp(g, -shared[:, :, None])               # exact: a power of two
    enc = e2m1_encode if elem == "e2m1" else e4m3_encode
    codes = enc(quot).reshape(R, C)
    return codes, (shared + 127).astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, elem: str) -> np.ndarray:
    """code value * 2^(scale - 127) per block of 32 along the rows."""
    val = e2m1_value(codes) if elem == "e2m1" else e4m3_value(codes)
    R, C = val.shape
    x = np.repeat(e8m0_value(scales), MX_BLOCK, axis=1)
    return val * x


def quantize_blocks(a: np.ndarray, block_rows: int, block_cols: int):
    """Block-FP8 quantisation of a 2-D array of exact values (float64 holding
    float32-representable numbers, e.g. decoded bfloat16).

    Follows the block-FP8 scheme the OverlapAdvisor page names for its FP8
    experiment group (section 4.4, Table 6) and the packing of activations
    with their quantisation metadata in CascadeEP Appendix C: every
    block_rows x block_cols block gets one float32 scale s = amax / 448
    (s = 1 when the block is all zero) and codes e4m3(fp32(v) / s), the
    quotient rounded in float32.  Partial edge blocks are allowed.

    Returns (codes uint8 same shape, scales float32 [ceil(R/br), ceil(C/bc)]).
    """
    a = np.asarray(a, dtype=np.float64)
    R, C = a.shape
    nbr = -(-R // block_rows)
    nbc = -(-C // block_cols)
    # Pad to whole blocks with zeros (a zero never raises a block's amax).
    pad = np.zeros((nbr * block_rows, nbc * block_cols), dtype=np.float64)
    pad[:R, :C] = a
    blocks = pad.reshape(nbr, block_rows, nbc, block_cols)
    amax = np.abs(blocks).max(axis=(1, 3)).astype(np.float32)          # [nbr, nbc]
    scales = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32),
                      np.float32(1.0)).astype(np.float32)
    quot = blocks.astype(np.float32) / scales[:, None, :, None]        # IEEE float32 division
    codes = e4m3_encode(quot).reshape(nbr * block_rows, nbc * block_cols)[:R, :C]
    return np.ascontiguousarray(codes), scales


def quantize_rows_groups(a: np.ndarray, group: int = 128):
    """Per-row quantisation in groups of ``group`` consecutive columns (the
    activation layout: one scale per token per 128 hidden elements).
    Returns (codes [R, C], scales float32 [R, C / group])."""
    a = np.asarray(a, dtype=np.float64)
    R, C = a.shape
    assert C % group == 0
    g = a.reshape(R, C // group, group)
    amax = np.abs(g).max(axis=2).astype(np.float32)
    s = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32),
                 np.float32(1.0)).astype(np.float32)
    quot = g.astype(np.float32) / s[:, :, None]
    codes = e4m3_encode(quot).reshape(R, C)
    return codes, s


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray,
                      block_rows: int, block_cols: int) -> np.ndarray:
    """code value * block scale, as float64 (exact: a 4-bit significand
    times a float32 fits in float64)."""
    v = e4m3_value(codes)
    s = np.repeat(np.repeat(scales.astype(np.float64), block_rows, axis=0),
                  block_cols, axis=1)[: v.shape[0], : v.shape[1]]
    return v * s


# ----------------------------------------------------------------------------
# Gate
# ----------------------------------------------------------------------------

def route(logits: np.ndarray, k: int):
    """Top-k gate (OverlapAdvisor section 2.1: each token activates its top-k
    experts) with softmax weights renormalised over the selected experts.

    Selection: the k experts first in the order (logit descending, expert
    index ascending), slot s holding the s-th of them.  Weights:
    w_s = exp(l_s - l_0) / sum_j exp(l_j - l_0) over the selected slots.

    Returns (ids int32 [T, k], w float64 [T, k]).
    """
    lg = np.asarray(logits, dtype=np.float64) + 0.0   # -0.0 -> +0.0
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("k must be in [1, E]")
    if np.isnan(lg).any():
        raise ValueError("logits must not be NaN")
    # Stable sort of the negated logits keeps equal logits in index order.
    order = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    ids = order.astype(np.int32)
    sel = np.take_along_axis(lg, order, axis=1)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return ids, w


# ----------------------------------------------------------------------------
# Permutation (dispatch layout)
# ----------------------------------------------------------------------------

def index_build(ids: np.ndarray, e_lo: int, E_L: int) -> Dict[str, np.ndarray]:
    """Expert-major layout of the local (token, slot) pairs.

    CascadeEP Appendix C ("Grouped FFN invocations"): per-expert row offsets
    from the selected token counts, rows grouped contiguously by expert, and
    an inverse map from each row back to its token and routing slot.
    OverlapAdvisor section 4.2.1: permute groups tokens by expert.

    Pairs are enumerated token-major (t, then s); those with a local expert
    are stably sorted by local expert id, so a segment lists its tokens in
    ascending order.

    Returns counts [E_L], offsets [E_L + 1] (exclusive scan), row_token [N],
    row_slot [N] and token_slot_row [T, k] (-1 where the expert is not
    local), all int32; N = offsets[E_L].
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    loc = ids - e_lo
    is_local = (loc >= 0) & (loc < E_L)
    flat_loc = loc.reshape(-1)
    flat_ok = is_local.reshape(-1)
    pair = np.nonzero(flat_ok)[0]                   # token-major order
    keys = flat_loc[pair]
    order = np.argsort(keys, kind="stable")
    sorted_pairs = pair[order]
    counts = np.bincount(keys, minlength=E_L).astype(np.int32)
    offsets = np.zeros(E_L + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_token = (sorted_pairs // k).astype(np.int32)
    row_slot = (sorted_pairs % k).astype(np.int32)
    tsr = np.full(T * k, -1, dtype=np.int32)
    tsr[sorted_pairs] = np.arange(len(sorted_pairs), dtype=np.int32)
    return {"counts": counts, "offsets": offsets, "row_token": row_token,
            "row_slot": row_slot, "token_slot_row": tsr.reshape(T, k)}


def index_build_masked(ids: np.ndarray, e_lo: int, E_L: int,
                       capacity: int) -> Dict[str, np.ndarray]:
    """Masked (fixed-capacity) layout of the local (token, slot) pairs: the
    ExpertPlex page's masked grouped-GEMM layout, fed without a permute step
    (OverlapAdvisor Table 7, low-latency dispatch).

    Local expert e owns rows [e * capacity, (e + 1) * capacity); its pairs
    take the first counts[e] of them, tokens ascending.  Row r of that block
    is therefore the r-th token, in token order, that picked expert e.

    Returns counts [E_L], offsets [E_L + 1] (the block starts e * capacity),
    row_token and row_slot [E_L * capacity] (-1 in rows that hold no pair)
    and token_slot_row [T, k] (-1 where the expert is not local), int32.
    Raises ValueError if an expert has more pairs than ``capacity``.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    C = int(capacity)
    row_token = np.full(E_L * C, -1, dtype=np.int32)
    row_slot = np.full(E_L * C, -1, dtype=np.int32)
    tsr = np.full((T, k), -1, dtype=np.int32)
    counts = np.zeros(E_L, dtype=np.int32)
    for e in range(E_L):
        hit_t, hit_s = np.nonzero(ids == e_lo + e)    # row-major: tokens ascending
        n = len(hit_t)
        if n > C:
            raise ValueError(f"expert {e} has {n} pairs, capacity {C}")
        counts[e] = n
        rows = e * C + np.arange(n)
        row_token[rows] = hit_t
        row_slot[rows] = hit_s
        tsr[hit_t, hit_s] = rows
    offsets = (np.arange(E_L + 1) * C).astype(np.int32)
    return {"counts": counts, "offsets": offsets, "row_token": row_token,
            "row_slot": row_slot, "token_slot_row": tsr}


def tile_count(counts: np.ndarray, tile_m: int) -> int:
    """Tile-aware row count of the ExpertPlex page's Eq. 3: the number of
    tile_m-row tiles covering every expert that has tokens,
    sum over e with m_e > 0 of ceil(m_e / tile_m)."""
    c = np.asarray(counts, dtype=np.int64)
    return int(sum(-(-int(m) // tile_m) for m in c if m > 0))


def dispatch(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """Permute: row j of the expert-major activations is token row_token[j]
    (OverlapAdvisor section 4.2.1)."""
    return np.asarray(x)[np.asarray(row_token, dtype=np.int64)]


# ----------------------------------------------------------------------------
# Expert FFN
# ----------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    """SiLU (swish with unit slope): a * sigmoid(a) = a / (1 + exp(-a))."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def gelu(a: np.ndarray) -> np.ndarray:
    """Exact GELU: a * Phi(a), Phi the standard normal distribution
    function, written with the complementary error function:
    Phi(a) = (1 + erf(a / sqrt 2)) / 2 = erfc(-a / sqrt 2) / 2 (the erfc form
    keeps full relative precision in the negative tail)."""
    from scipy.special import erfc
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * a * erfc(-a / np.sqrt(2.0))


ACTIVATIONS = ("swiglu", "gelu")


def up_rows(I: int, activation: str = "swiglu") -> int:
    """Rows of an expert's first-layer weight: m * I, m = 2 first-layer
    matrices for the gated MLP, 1 for the standard one (OverlapAdvisor Eq. 8)."""
    return (2 if activation == "swiglu" else 1) * I


def expert_ffn(xr: np.ndarray, w13: np.ndarray, w2: np.ndarray, h_fn=None,
               activation: str = "swiglu"):
    """One expert's FFN on a block of rows.

    Gated SwiGLU (default): OverlapAdvisor section 4.2.2 (a gated MLP has
    m = 2 first-layer matrices), Eq. 8 (the up GroupGEMM has 2*m*H*I FLOPs
    per row, the down GroupGEMM 2*H*I), Table 6 (gated SwiGLU), section
    4.2.1 (the activation sits between the two GroupGEMMs).
    xr [n, H]; w13 [2I, H] (gate rows then up rows); w2 [H, I].

    Standard MLP (activation="gelu"): m = 1 (Eq. 8), Table 6 (BF16 standard
    MLP with GELU): h = gelu(xr @ w1.T) with w13 = w1 [I, H].

    ``h_fn``, if given, maps h before the down projection (the FP8 path's
    activation quantisation).
    Returns (h [n, I], y [n, H]) in float64.
    """
    if activation == "swiglu":
        I = w13.shape[0] // 2
        g = xr @ w13[:I].T
        u = xr @ w13[I:].T
        h = silu(g) * u
    elif activation == "gelu":
        h = gelu(xr @ w13.T)
    else:
        raise ValueError(activation)
    return h, (h if h_fn is None else h_fn(h)) @ w2.T


def grouped_ffn(x_perm: np.ndarray, offsets: np.ndarray, w13, w2, h_fn=None,
                activation: str = "swiglu"):
    """Grouped FFN over the expert-major rows: segment e
    [offsets[e], offsets[e+1]) runs through local expert e.  ``w13``/``w2``
    are callables or arrays indexed by the local expert giving float64
    weights.  Returns (h [N, I], y_perm [N, H])."""
    E_L = len(offsets) - 1
    get13 = w13 if callable(w13) else (lambda e: w13[e])
    get2 = w2 if callable(w2) else (lambda e: w2[e])
    N = int(offsets[-1])
    H = x_perm.shape[1]
    h_all = None
    y_perm = np.zeros((N, H), dtype=np.float64)
    for e in range(E_L):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        we13, we2 = get13(e), get2(e)
        if h_all is None:
            h_all = np.zeros((N, we2.shape[1]), dtype=np.float64)
        h, y = expert_ffn(x_perm[a:b], we13, we2, h_fn, activation)
        h_all[a:b] = h
        y_perm[a:b] = y
    if h_all is None:
        # no local rows: h is still [0, I], I read from the expert weights
        I = get2(0).shape[1] if E_L > 0 else 0
        h_all = np.zeros((N, I), dtype=np.float64)
    return h_all, y_perm


def grouped_ffn_masked(x_perm: np.ndarray, counts: np.ndarray, capacity: int,
                       w13, w2, h_fn=None, activation: str = "swiglu"):
    """Grouped FFN over the masked layout: rows [e * capacity,
    e * capacity + counts[e]) run through local expert e; the other rows of
    each block are not computed and stay zero.  Weights as in grouped_ffn.
    Returns (h [E_L * capacity, I], y_perm [E_L * capacity, H])."""
    E_L = len(counts)
    C = int(capacity)
    get13 = w13 if callable(w13) else (lambda e: w13[e])
    get2 = w2 if callable(w2) else (lambda e: w2[e])
    H = x_perm.shape[1]
    h_all = None
    y_perm = np.zeros((E_L * C, H), dtype=np.float64)
    for e in range(E_L):
        n = int(counts[e])
        if n == 0:
            continue
        we13, we2 = get13(e), get2(e)
        if h_all is None:
            h_all = np.zeros((E_L * C, we2.shape[1]), dtype=np.float64)
        a = e * C
        h, y = expert_ffn(x_perm[a:a + n], we13, we2, h_fn, activation)
        h_all[a:a + n] = h
        y_perm[a:a + n] = y
    if h_all is None:
        # every block empty: h keeps its [E_L * capacity, I] shape, all zero
        I = get2(0).shape[1] if E_L > 0 else 0
        h_all = np.zeros((E_L * C, I), dtype=np.float64)
    return h_all, y_perm


def combine(y_perm: np.ndarray, token_slot_row: np.ndarray, w: np.ndarray,
            shared: Optional[np.ndarray] = None, H: Optional[int] = None) -> np.ndarray:
    """Unpermute and weighted combine (CascadeEP Appendix C, "Output return
    and combine"; OverlapAdvisor section 4.2.1 unpermute): for every token,
    the sum over its local slots, in slot order, of the slot's routing
    weight times its expert output row, plus the shared-expert output.
    A token with no local slot gets 0 (plus the shared output)."""
    tsr = np.asarray(token_slot_row)
    T, k = tsr.shape
    if H is None:
        H = y_perm.shape[1]
    y = np.zeros((T, H), dtype=np.float64)
    for s in range(k):
        r = tsr[:, s]
        m = r >= 0
        y[m] += w[m, s][:, None] * y_perm[r[m]]
    if shared is not None:
        y += shared
    return y


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------

def _expert_weights(weights: dict, fp8: bool, mx: bool = False):
    """Float64 weight accessors.  bf16: the exact values.  fp8: the exact
    dequantisation (code * block scale) of the block-FP8 weights, which are
    the layer's parameters.  mx: the same for MXFP4 weights (E2M1 codes
    "w13_q"/"w2_q" and E8M0 scales "w13_s"/"w2_s" per 32 along K)."""
    if mx:
        return (lambda e: mx_dequantize(weights["w13_q"][e], weights["w13_s"][e], "e2m1"),
                lambda e: mx_dequantize(weights["w2_q"][e], weights["w2_s"][e], "e2m1"))
    if not fp8:
        return (lambda e: bf16_to_f64(weights["w13"][e]),
                lambda e: bf16_to_f64(weights["w2"][e]))
    return (lambda e: dequantize_blocks(weights["w13_q"][e], weights["w13_s"][e], 128, 128),
            lambda e: dequantize_blocks(weights["w2_q"][e], weights["w2_s"][e], 128, 128))


def _shared_weights(weights: dict, fp8: bool, mx: bool = False):
    if "ws13" not in weights and "ws13_q" not in weights:
        return None
    if mx:
        return (mx_dequantize(weights["ws13_q"], weights["ws13_s"], "e2m1"),
                mx_dequantize(weights["ws2_q"], weights["ws2_s"], "e2m1"))
    if not fp8:
        return bf16_to_f64(weights["ws13"]), bf16_to_f64(weights["ws2"])
    return (dequantize_blocks(weights["ws13_q"], weights["ws13_s"], 128, 128),
            dequantize_blocks(weights["ws2_q"], weights["ws2_s"], 128, 128))


def fp8_activation(a: np.ndarray) -> np.ndarray:
    """The value an activation row block carries after block-FP8 packing
    (CascadeEP Appendix C: activations packed with their quantisation
    metadata; OverlapAdvisor Table 6: FP8 activations): per token, per 128
    consecutive elements, dequantise(quantise(a))."""
    q, s = quantize_rows_groups(a, 128)
    return dequantize_blocks(q, s, 1, 128)


def mx8_activation(a: np.ndarray) -> np.ndarray:
    """The value an activation row block carries after MXFP8 packing (E4M3
    elements, one E8M0 scale per 32 consecutive elements of a token): the
    activation format that goes with MXFP4 weights here."""
    q, s = mx_quantize(a, "e4m3")
    return mx_dequantize(q, s, "e4m3")


def moe_layer(logits: np.ndarray, x_bits: np.ndarray, weights: dict, *,
              k: int, e_lo: int, E_L: int, fp8: bool = False,
              quantize_activations: bool = False,
              activation: str = "swiglu",
              capacity: Optional[int] = None,
              mx: bool = False) -> Dict[str, np.ndarray]:
    """The whole layer for one GPU's local experts, every stage kept.

    ``weights``: bf16 -> "w13" [E_L, m*I, H] (m = 2 for SwiGLU, 1 for the
    standard GELU MLP), "w2" [E_L, H, I] (bf16 bits),
    optional "ws13"/"ws2" (shared expert); fp8 -> the same names with
    suffixes "_q" (codes) and "_s" (128 x 128 block scales).

    ``quantize_activations`` (fp8 only) also passes the inputs of both
    GEMMs -- x and h -- through per-token 128-group block-FP8, as the FP8
    path of the pages does between its GEMMs (CascadeEP Appendix C, the
    activation and quantisation operations between the two expert GEMMs).
    The default leaves them exact: the reference the output gate measures.

    ``mx`` takes MXFP4 weights (see _expert_weights); with
    ``quantize_activations`` x and h then pass through MXFP8 (per-token
    blocks of 32 with E8M0 scales) instead of block-FP8.

    ``capacity`` (optional) runs the layer over the masked fixed-capacity
    layout (index_build_masked / grouped_ffn_masked) instead of the
    contiguous one; the stage arrays are then in that layout.

    Returns every stage: ids, w, counts, offsets, row_token, row_slot,
    token_slot_row, x_perm, h, y_perm, shared (or None) and y, as float64
    for the floating-point ones (h before its own quantisation).
    """
    ids, w = route(logits, k)
    masked = capacity is not None
    ix = index_build_masked(ids, e_lo, E_L, capacity) if masked else index_build(ids, e_lo, E_L)
    x = bf16_to_f64(x_bits)
    qa = (fp8 or mx) and quantize_activations
    act_q = mx8_activation if mx else fp8_activation
    xq = act_q(x) if qa else x
    if masked:                                   # unused rows of a block stay zero
        x_perm = np.zeros((len(ix["row_token"]), x.shape[1]), dtype=np.float64)
        used = ix["row_token"] >= 0
        x_perm[used] = dispatch(xq, ix["row_token"][used])
    else:
        x_perm = dispatch(xq, ix["row_token"])
    g13, g2 = _expert_weights(weights, fp8, mx)
    h_fn = act_q if qa else None
    if masked:
        h, y_perm = grouped_ffn_masked(x_perm, ix["counts"], capacity, g13, g2, h_fn, activation)
    else:
        h, y_perm = grouped_ffn(x_perm, ix["offsets"], g13, g2, h_fn, activation)
    sw = _shared_weights(weights, fp8, mx)
    shared = None
    if sw is not None:
        shared = expert_ffn(xq, sw[0], sw[1], h_fn, activation)[1]
    y = combine(y_perm, ix["token_slot_row"], w, shared, H=x.shape[1])
    out = dict(ix)
    out.update(ids=ids, w=w, x_perm=x_perm, h=h, y_perm=y_perm, shared=shared, y=y)
    return out


def moe_layer_tokens(logits: np.ndarray, x_bits: np.ndarray, weights: dict,
                     tokens, *, k: int, e_lo: int, E_L: int,
                     fp8: bool = False, quantize_activations: bool = False,
                     activation: str = "swiglu", mx: bool = False) -> np.ndarray:
    """Layer output rows for a few tokens only, one token at a time (for
    spot checks at sizes where the whole layer is too slow on the CPU).
    A token's output depends only on its own logits and activations, so
    this is the same definition restricted to those rows.  Returns float64
    [len(tokens), H]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    ids, w = route(logits[tokens], k)
    x = bf16_to_f64(x_bits[tokens])
    qa = (fp8 or mx) and quantize_activations
    act_q = mx8_activation if mx else fp8_activation
    if qa:
        x = act_q(x)                # per-token groups: same rows as for the whole batch
    h_fn = act_q if qa else None
    g13, g2 = _expert_weights(weights, fp8, mx)
    sw = _shared_weights(weights, fp8, mx)
    y = np.zeros_like(x)
    # Group the requested tokens by local expert so each expert's weights are
    # decoded once.
    by_expert: Dict[int, list] = {}
    for i in range(len(tokens)):
        for s in range(k):
            e = int(ids[i, s]) - e_lo
            if 0 <= e < E_L:
                by_expert.setdefault(e, []).append((i, s))
    contrib = np.zeros((len(tokens), k, x.shape[1]), dtype=np.float64)
    for e, lst in sorted(by_expert.items()):
        we13, we2 = g13(e), g2(e)
        rows = np.array([i for i, _ in lst])
        _, ye = expert_ffn(x[rows], we13, we2, h_fn, activation)
        for (i, s), yr in zip(lst, ye):
            contrib[i, s] = w[i, s] * yr
    for s in range(k):                       # slot order, as in combine()
        y += contrib[:, s]
    if sw is not None:
        y += expert_ffn(x, sw[0], sw[1], h_fn, activation)[1]
    return y
