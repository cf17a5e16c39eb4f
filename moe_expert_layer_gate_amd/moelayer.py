"""ctypes binding of libmoelayer.so (include/moe_layer.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Arrays are torch tensors on the GPU (torch provides device memory
and the current stream); the functions pass their data pointers, the problem
struct and the stream handle through, and raise MoEError on a non-OK status.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoelayer.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 = 0, 1, 2
MX_E2M1, MX_E4M3 = 0, 1
LAYOUT_PANEL_WEIGHTS, LAYOUT_PANEL_ACTS = 1, 2
ACT_SWIGLU, ACT_GELU = 0, 1
STAGE_LAYER, STAGE_DISPATCH, STAGE_FFN = 0, 1, 2

# Every function the header declares, with its ctypes signature.
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class moe_problem(ctypes.Structure):
    _fields_ = [("num_tokens", _i32), ("hidden", _i32), ("num_experts", _i32),
                ("top_k", _i32), ("expert_begin", _i32), ("num_local", _i32),
                ("inter", _i32), ("shared_inter", _i32), ("dtype", _i32),
                ("layout", _i32), ("activation", _i32), ("capacity", _i32)]


class moe_weights(ctypes.Structure):
    _fields_ = [("w13", _vp), ("w2", _vp), ("ws13", _vp), ("ws2", _vp),
                ("w13_scale", _vp), ("w2_scale", _vp), ("ws13_scale", _vp),
                ("ws2_scale", _vp)]


_P = ctypes.POINTER(moe_problem)
_W = ctypes.POINTER(moe_weights)
SIGNATURES = {
    "moe_route": (_i32, [_P, _vp, _vp, _vp, _vp]),
    "moe_dispatch": (_i32, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_grouped_ffn": (_i32, [_P, _vp, _vp, _vp, _W, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_grouped_ffn_gather": (_i32, [_P, _vp, _vp, _vp, _vp, _W, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_combine": (_i32, [_P, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_layer": (_i32, [_P, _vp, _vp, _W, _vp, _vp, _sz, _vp]),
    "moe_layer_static": (_i32, [_P, _vp, _vp, _W, _vp, _vp]),
    "moe_quantize_fp8": (_i32, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "moe_pack_panel": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "moe_pack_panel_mx": (_i32, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "moe_quantize_mx": (_i32, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "moe_workspace_bytes": (_sz, [_P, _i32]),
    "moe_workspace_flags": (_i32, [_P, _i32, _vp, _sz, _vp, _vp]),
    "moe_stream_threshold": (_i64, [_vp, _vp, _i32, ctypes.c_double]),
    "moe_stream_plan": (_i32, [_vp, _i32, _i64, _vp, _vp]),
    "moe_workspace_bytes_streamed": (_sz, [_P, _i32, _i32]),
    "moe_layer_streamed": (_i32, [_P, _vp, _vp, _W, _vp, _vp, _i32, _vp, _i32, _vp, _sz]),
    "moe_status_str": (ctypes.c_char_p, [_i32]),
    "moe_abi_version": (_i32, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m moe_expert_layer_gate_amd.build)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype, f.argtypes = res, args
        _lib = l
    return _lib


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status_str(status)}")
        self.status = status


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


@dataclasses.dataclass(frozen=True)
class Problem:
    """The workload tuple of one rank (mirrors moe_problem)."""
    T: int
    H: int
    E: int
    k: int
    e_lo: int
    E_L: int
    I: int
    I_s: int = 0
    fp8: bool = False
    layout: int = 0   # LAYOUT_* bits
    act: str = "swiglu"  # "swiglu" | "gelu"
    capacity: int = 0    # 0: contiguous segments; C >= T: masked fixed-capacity layout
    mx: bool = False     # MXFP4 weights, MXFP8 activations (fp8 must be False)

    @property
    def dtype(self) -> int:
        return MOE_MXFP4 if self.mx else MOE_FP8_E4M3 if self.fp8 else MOE_BF16

    @property
    def quantized(self) -> bool:
        """GEMM activations are quantised with per-row scales (fp8 or MX)."""
        return self.fp8 or self.mx

    def c(self) -> moe_problem:
        return moe_problem(self.T, self.H, self.E, self.k, self.e_lo, self.E_L, self.I,
                           self.I_s, self.dtype, self.layout,
                           ACT_GELU if self.act == "gelu" else ACT_SWIGLU, self.capacity)

    @property
    def m(self) -> int:
        """First-layer matrices per expert (2 gated, 1 standard)."""
        return 1 if self.act == "gelu" else 2

    @property
    def n_cap(self) -> int:
        """Rows of the permuted buffers."""
        if self.capacity > 0:
            return self.capacity * self.E_L
        return self.T * min(self.k, self.E_L)

    @classmethod
    def from_config(cls, cfg, T: Optional[int] = None, layout: int = 0,
                    capacity: Optional[int] = None) -> "Problem":
        return cls(T=cfg.T if T is None else T, H=cfg.H, E=cfg.E, k=cfg.k, e_lo=cfg.e_lo,
                   E_L=cfg.E_L, I=cfg.I, I_s=cfg.I_s, fp8=cfg.fp8, layout=layout, act=cfg.act,
                   mx=getattr(cfg, "mx", False),
                   capacity=getattr(cfg, "capacity", 0) if capacity is None else capacity)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status)


def weights_struct(w13, w2, ws13=None, ws2=None, w13_scale=None, w2_scale=None,
                   ws13_scale=None, ws2_scale=None) -> moe_weights:
    return moe_weights(_ptr(w13), _ptr(w2), _ptr(ws13), _ptr(ws2), _ptr(w13_scale),
                       _ptr(w2_scale), _ptr(ws13_scale), _ptr(ws2_scale))


def workspace_bytes(p: Problem, stage: int = STAGE_LAYER) -> int:
    pc = p.c()
    return int(lib().moe_workspace_bytes(ctypes.byref(pc), stage))


FLAG_WAIT_TIMEOUT = 1


def moe_workspace_flags(p: Problem, stage: int, ws, flags, stream=None) -> None:
    """Enqueue the copy of workspace ws's FFN flags into the device int32
    tensor `flags` (see moe_workspace_flags in the header)."""
    pc = p.c()
    _check("moe_workspace_flags", lib().moe_workspace_flags(
        ctypes.byref(pc), stage, _ptr(ws), ws.numel() * ws.element_size(), _ptr(flags),
        _stream(stream)))


def moe_route(p: Problem, logits, topk_ids, topk_w, stream=None) -> None:
    pc = p.c()
    _check("moe_route", lib().moe_route(ctypes.byref(pc), _ptr(logits), _ptr(topk_ids),
                                        _ptr(topk_w), _stream(stream)))


def moe_dispatch(p: Problem, x, topk_ids, counts, offsets, row_token, row_slot,
                 token_slot_row, x_perm, x_perm_scale, ws, stream=None) -> None:
    pc = p.c()
    _check("moe_dispatch", lib().moe_dispatch(
        ctypes.byref(pc), _ptr(x), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
        _ptr(row_token), _ptr(row_slot), _ptr(token_slot_row), _ptr(x_perm),
        _ptr(x_perm_scale), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn(p: Problem, x_perm, x_perm_scale, offsets, weights: moe_weights, h,
                    h_scale, y_perm, ws, stream=None) -> None:
    pc = p.c()
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        ctypes.byref(pc), _ptr(x_perm), _ptr(x_perm_scale), _ptr(offsets),
        ctypes.byref(weights), _ptr(h), _ptr(h_scale), _ptr(y_perm), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn_gather(p: Problem, x, x_scale, row_token, offsets, weights: moe_weights, h,
                           h_scale, y_perm, ws, stream=None) -> None:
    pc = p.c()
    _check("moe_grouped_ffn_gather", lib().moe_grouped_ffn_gather(
        ctypes.byref(pc), _ptr(x), _ptr(x_scale), _ptr(row_token), _ptr(offsets),
        ctypes.byref(weights), _ptr(h), _ptr(h_scale), _ptr(y_perm), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def moe_combine(p: Problem, y_perm, token_slot_row, topk_w, shared_out, y, stream=None) -> None:
    pc = p.c()
    _check("moe_combine", lib().moe_combine(
        ctypes.byref(pc), _ptr(y_perm), _ptr(token_slot_row), _ptr(topk_w), _ptr(shared_out),
        _ptr(y), _stream(stream)))


def moe_layer(p: Problem, logits, x, weights: moe_weights, y, ws, stream=None) -> None:
    pc = p.c()
    _check("moe_layer", lib().moe_layer(
        ctypes.byref(pc), _ptr(logits), _ptr(x), ctypes.byref(weights), _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


STATIC_SCRATCH_BYTES = 64 << 20


def moe_layer_static(p: Problem, logits, x, weights: moe_weights, y, stream=None) -> None:
    """moe_layer on the library's static per-device workspace (no workspace
    argument; see moe_layer_static in the header)."""
    pc = p.c()
    _check("moe_layer_static", lib().moe_layer_static(
        ctypes.byref(pc), _ptr(logits), _ptr(x), ctypes.byref(weights), _ptr(y),
        _stream(stream)))


def moe_quantize_fp8(src, batch: int, rows: int, cols: int, block_rows: int, codes, scales,
                     stream=None) -> None:
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(
        _ptr(src), batch, rows, cols, block_rows, _ptr(codes), _ptr(scales), _stream(stream)))


def moe_pack_panel(src, batch: int, rows: int, cols: int, dst, stream=None) -> None:
    _check("moe_pack_panel", lib().moe_pack_panel(
        _ptr(src), batch, rows, cols, _ptr(dst), _stream(stream)))


def moe_pack_panel_mx(codes, scales, batch: int, rows: int, cols: int, codes_dst, scales_dst,
                      stream=None) -> None:
    _check("moe_pack_panel_mx", lib().moe_pack_panel_mx(
        _ptr(codes), _ptr(scales), batch, rows, cols, _ptr(codes_dst), _ptr(scales_dst),
        _stream(stream)))


def stream_threshold(counts, throughput, rho: float) -> int:
    """moe_stream_threshold on host sequences (-1 if invalid)."""
    n = len(counts)
    c = (ctypes.c_int64 * max(n, 1))(*[int(v) for v in counts])
    t = (ctypes.c_double * max(n, 1))(*[float(v) for v in throughput])
    return int(lib().moe_stream_threshold(c, t, n, float(rho)))


def stream_plan(ready_rows, theta: int):
    """moe_stream_plan: the exclusive end arrival of each invocation."""
    n = len(ready_rows)
    r = (ctypes.c_int64 * max(n, 1))(*[int(v) for v in ready_rows])
    ends = (ctypes.c_int32 * max(n, 1))()
    ng = ctypes.c_int32(0)
    _check("moe_stream_plan", lib().moe_stream_plan(r, n, int(theta), ends, ctypes.byref(ng)))
    return [int(ends[i]) for i in range(ng.value)]


def workspace_bytes_streamed(p: Problem, max_group_tokens: int, n_streams: int) -> int:
    pc = p.c()
    return int(lib().moe_workspace_bytes_streamed(ctypes.byref(pc), int(max_group_tokens),
                                                  int(n_streams)))


def moe_layer_streamed(p: Problem, logits, x, weights: moe_weights, y, group_tokens, streams,
                       ws) -> None:
    """moe_layer over token groups [group_tokens[j], group_tokens[j+1]), group
    j on streams[j % len(streams)] (torch streams or raw handles)."""
    pc = p.c()
    g = (ctypes.c_int32 * len(group_tokens))(*[int(v) for v in group_tokens])
    hs = (ctypes.c_void_p * len(streams))(*[_stream(st) for st in streams])
    _check("moe_layer_streamed", lib().moe_layer_streamed(
        ctypes.byref(pc), _ptr(logits), _ptr(x), ctypes.byref(weights), _ptr(y), g,
        len(group_tokens) - 1, hs, len(streams), _ptr(ws), ws.numel() * ws.element_size()))


def moe_quantize_mx(src, batch: int, rows: int, cols: int, elem: int, codes, scales,
                    stream=None) -> None:
    _check("moe_quantize_mx", lib().moe_quantize_mx(
        _ptr(src), batch, rows, cols, elem, _ptr(codes), _ptr(scales), _stream(stream)))
