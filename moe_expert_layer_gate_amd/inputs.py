"""Seeded synthetic inputs for the MoE layer: the one module that both the
CPU oracle's tests and the HIP path's tests and benchmark draw from.

It holds no arithmetic of the layer itself (no gating, no permutation, no
FFN, no quantisation).  It only draws random numbers and stores them in the
layer's input formats:

* router logits: float32 ``[T, E]``;
* activations and weights: bfloat16 bit patterns held in ``numpy.uint16``
  (an fp32 draw rounded to nearest-even on its upper 16 bits);
* a replica split of the token rows (metadata only; it changes no output).

Workload shapes follow the model shapes the OverlapAdvisor page lists for its
single-layer benchmarks (Figure 2 panels (a) and (b): DeepSeek-V3/R1 with
H=7168, I=2048, E=256, k=8 and Qwen3-30B-A3B with H=2048, I=768, E=128, k=8)
and the block-FP8 / gated-SwiGLU experiment group of its Table 6.

Each kind of input comes from its own numpy generator, seeded with a key
that starts ``[seed, n]``: n = 0 logits, 1 x, 2 routed weights (W13 then
W2), 3 shared weights, 4 replica shares.  So the weights of a seed do not
depend on T, and the logits do not depend on whether weights are drawn.
Weights and activations are N(0, std) with std = 0.02 unless a caller asks
for another spread (tests use larger spreads to drive SiLU out of its
linear region).
"""
from __future__ import annotations

import dataclasses
import os
from typing import List, Dict, Optional

import numpy as np

__all__ = ["MoEConfig", "CONFIGS", "config", "make_inputs", "f32_to_bf16_bits",
           "make_logits", "replica_split"]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One workload: the layer shape plus how its routing is drawn.

    Fields follow the pages' workload tuple (H, I, E, k, tokens) plus the
    local expert range of one expert-parallel rank.
    """
    name: str
    T: int            # tokens in the batch
    H: int            # hidden size
    E: int            # global experts
    E_L: int          # local experts on this GPU
    e_lo: int         # first local expert (global id)
    k: int            # experts per token
    I: int            # expert intermediate size
    I_s: int = 0      # shared-expert intermediate size (0 = no shared expert)
    fp8: bool = False  # block-FP8 weights and GEMM activations
    mx: bool = False   # MXFP4 weights, MXFP8 GEMM activations
    logits: str = "normal"     # "normal" | "gumbel_zipf"
    zipf_s: float = 1.1
    replicas: int = 0          # >0: Dirichlet(0.5) split of the rows over replicas
    std: float = 0.02
    act: str = "swiglu"        # "swiglu" (gated, m = 2) | "gelu" (standard MLP, m = 1)

    @property
    def m(self) -> int:
        """First-layer matrices per expert."""
        return 2 if self.act == "swiglu" else 1

    @property
    def dtype(self) -> str:
        return "mxfp4" if self.mx else "fp8_e4m3" if self.fp8 else "bf16"


CONFIGS: Dict[str, MoEConfig] = {
    # Tiny layer: every expert local.
    "tiny": MoEConfig("tiny", T=256, H=512, E=8, E_L=8, e_lo=0, k=2, I=1024),
    # Qwen3-30B-A3B-shaped prefill, all 128 experts local.
    "qwen3_30b_prefill": MoEConfig("qwen3_30b_prefill", T=8192, H=2048, E=128,
                                   E_L=128, e_lo=0, k=8, I=768),
    # DeepSeek-V3-shaped shard of an 8-way expert-parallel layer: 16384 tokens
    # arriving from 8 attention replicas, 32 of 256 experts local, Zipf(1.1)
    # expert popularity; the shard holds the most popular experts.
    "dsv3_ep8_prefill": MoEConfig("dsv3_ep8_prefill", T=16384, H=7168, E=256,
                                  E_L=32, e_lo=0, k=8, I=2048,
                                  logits="gumbel_zipf", replicas=8),
    # The same shard with block-FP8 weights/activations and one shared expert.
    "dsv3_ep8_prefill_fp8": MoEConfig("dsv3_ep8_prefill_fp8", T=16384, H=7168,
                                      E=256, E_L=32, e_lo=0, k=8, I=2048,
                                      I_s=2048, fp8=True, logits="gumbel_zipf",
                                      replicas=8),
    # Decode-sized batch on the same shard shape with uniform routing.
    "dsv3_ep8_decode": MoEConfig("dsv3_ep8_decode", T=64, H=7168, E=256, E_L=32,
                                 e_lo=0, k=8, I=2048),
    # The decode batch with block-FP8 weights and activations.
    "dsv3_ep8_decode_fp8": MoEConfig("dsv3_ep8_decode_fp8", T=64, H=7168, E=256, E_L=32,
                                     e_lo=0, k=8, I=2048, fp8=True),
    # The same shard with MXFP4 routed-expert weights (MXFP8 activations) and
    # its shared expert in the same format.
    "dsv3_ep8_prefill_mxfp4": MoEConfig("dsv3_ep8_prefill_mxfp4", T=16384, H=7168,
                                        E=256, E_L=32, e_lo=0, k=8, I=2048,
                                        I_s=2048, mx=True, logits="gumbel_zipf",
                                        replicas=8),
    # The decode batch with MXFP4 weights.
    "dsv3_ep8_decode_mxfp4": MoEConfig("dsv3_ep8_decode_mxfp4", T=64, H=7168, E=256, E_L=32,
                                       e_lo=0, k=8, I=2048, mx=True),
    # The Qwen3-30B-A3B prefill shape with a standard (non-gated) GELU MLP:
    # the pages' BF16 group runs its models with a standard MLP.
    "qwen3_30b_prefill_gelu": MoEConfig("qwen3_30b_prefill_gelu", T=8192, H=2048, E=128,
                                        E_L=128, e_lo=0, k=8, I=768, act="gelu"),
}
# Numbered aliases in the order the workloads are usually listed.
_ORDER = ["tiny", "qwen3_30b_prefill", "dsv3_ep8_prefill",
          "dsv3_ep8_prefill_fp8", "dsv3_ep8_decode"]


def config(name_or_index) -> MoEConfig:
    """Look a workload up by name or by 1-based position in the list above."""
    if isinstance(name_or_index, int):
        return CONFIGS[_ORDER[name_or_index - 1]]
    return CONFIGS[name_or_index]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns.  Inputs are finite, so the 32-bit sum cannot wrap."""
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= 16
    return u.astype(np.uint16)


_CHUNK = 1 << 24


def _normal_bf16(seed_key, shape, std: float) -> np.ndarray:
    """N(0, std) draws in float32, stored as bfloat16 bits.

    Element block c (of 2^24 elements, in C order) comes from the generator
    seeded ``seed_key + [c]``, so the blocks can be drawn on several threads
    and the result does not depend on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        s = c * _CHUNK
        m = min(_CHUNK, n - s)
        g = np.random.default_rng(list(seed_key) + [c])
        v = g.standard_normal(m, dtype=np.float32)
        v *= np.float32(std)
        out[s:s + m] = f32_to_bf16_bits(v)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        import concurrent.futures as cf
        workers = min(nchunks, os.cpu_count() or 1, 16)
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def make_logits(rng: np.random.Generator, cfg: MoEConfig) -> np.ndarray:
    """Router logits, float32 [T, E].

    "normal": i.i.d. N(0, 1).
    "gumbel_zipf": ln p_e + Gumbel(0, 1) with p_e proportional to
    (e + 1)^-s.  Taking the top k of such a row samples k experts without
    replacement with probability proportional to p (the Gumbel-top-k trick),
    so expert 0 is the most popular.  Computed in float64, stored float32.
    """
    if cfg.logits == "normal":
        return rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.logits == "gumbel_zipf":
        e = np.arange(cfg.E, dtype=np.float64)
        p = (e + 1.0) ** (-cfg.zipf_s)
        p /= p.sum()
        u = rng.random((cfg.T, cfg.E))  # in [0, 1)
        u = np.maximum(u, np.finfo(np.float64).tiny)
        g = -np.log(-np.log(u))
        return (np.log(p)[None, :] + g).astype(np.float32)
    raise ValueError(f"unknown logits kind {cfg.logits!r}")


def replica_split(rng: np.random.Generator, T: int, replicas: int) -> np.ndarray:
    """Row offsets [replicas + 1] of a replica-major split of T rows with
    shares ~ Dirichlet(0.5, ..., 0.5), rounded by largest remainder."""
    shares = rng.dirichlet(np.full(replicas, 0.5))
    raw = shares * T
    base = np.floor(raw).astype(np.int64)
    rem = T - int(base.sum())
    order = np.argsort(-(raw - base), kind="stable")
    base[order[:rem]] += 1
    return np.concatenate([[0], np.cumsum(base)]).astype(np.int64)


def replica_arrival(replica_offsets: np.ndarray) -> List[int]:
    """Arrival model of the synthetic prefill batches: a replica's attention
    time grows with its token count, so replicas arrive in ascending order of
    size (ties by index)."""
    off = np.asarray(replica_offsets, dtype=np.int64)
    sizes = (off[1:] - off[:-1]).tolist()
    return sorted(range(len(sizes)), key=lambda r: (sizes[r], r))


def arrival_permutation(replica_offsets: np.ndarray) -> np.ndarray:
    """Token permutation that puts the rows in arrival order (the order in
    which the destination receives them): the replicas' token ranges one
    after another in replica_arrival order."""
    off = np.asarray(replica_offsets, dtype=np.int64)
    return np.concatenate([np.arange(off[r], off[r + 1]) for r in replica_arrival(off)]
                          + [np.zeros(0, dtype=np.int64)])


def make_inputs(cfg: MoEConfig, seed: int, *, weights: bool = True,
                std: Optional[float] = None,
                x_std: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Draw one batch of inputs for ``cfg``.

    Returns a dict with
      logits  float32 [T, E]
      x       uint16 (bf16 bits) [T, H]
      w13     uint16 [E_L, m I, H]  SwiGLU (m = 2): rows 0..I-1 gate, I..2I-1 up;
                                    GELU (m = 1): the first-layer matrix
      w2      uint16 [E_L, H, I]
      ws13    uint16 [m I_s, H]     (only when I_s > 0)
      ws2     uint16 [H, I_s]       (only when I_s > 0)
      replica_offsets int64 [R + 1] (only when cfg.replicas > 0)
    ``weights=False`` skips the weight draws.
    """
    def stream(n: int) -> np.random.Generator:
        return np.random.default_rng([seed, n])

    w_std = cfg.std if std is None else std
    a_std = cfg.std if x_std is None else x_std
    out: Dict[str, np.ndarray] = {}
    out["logits"] = make_logits(stream(0), cfg)
    out["x"] = _normal_bf16([seed, 1], (cfg.T, cfg.H), a_std)
    if cfg.replicas > 0:
        out["replica_offsets"] = replica_split(stream(4), cfg.T, cfg.replicas)
    if not weights:
        return out
    out["w13"] = _normal_bf16([seed, 2, 0], (cfg.E_L, cfg.m * cfg.I, cfg.H), w_std)
    out["w2"] = _normal_bf16([seed, 2, 1], (cfg.E_L, cfg.H, cfg.I), w_std)
    if cfg.I_s > 0:
        out["ws13"] = _normal_bf16([seed, 3, 0], (cfg.m * cfg.I_s, cfg.H), w_std)
        out["ws2"] = _normal_bf16([seed, 3, 1], (cfg.H, cfg.I_s), w_std)
    return out
