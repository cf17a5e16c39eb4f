"""Device-memory plumbing around the binding: upload seeded host inputs as
torch tensors, convert bf16 weights to block-FP8 with the library's own
quantiser, and size workspaces.  No step of the layer is computed here."""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch

from . import moelayer as ml


def bf16_from_bits(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor (no rounding)."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bits_from_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def workspace(p: ml.Problem, stage: int = ml.STAGE_LAYER, device="cuda") -> torch.Tensor:
    n = ml.workspace_bytes(p, stage)
    if n == 0:
        raise ValueError(f"invalid problem {p}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def quantize_fp8(w: torch.Tensor, block_rows: int = 128):
    """[B, R, C] or [R, C] bf16 -> (E4M3 codes uint8 same shape, fp32 scales
    [B, ceil(R/br), C/128]) using moe_quantize_fp8."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    B, R, C = w3.shape
    codes = torch.empty((B, R, C), dtype=torch.uint8, device=w.device)
    nrb = (R + block_rows - 1) // block_rows
    scales = torch.empty((B, nrb, C // 128), dtype=torch.float32, device=w.device)
    ml.moe_quantize_fp8(w3.contiguous(), B, R, C, block_rows, codes, scales)
    if squeeze:
        return codes[0], scales[0]
    return codes, scales


def quantize_mx4(w: torch.Tensor):
    """[B, R, C] or [R, C] bf16 -> (E2M1 codes uint8 [.., R, C/2], two per
    byte, E8M0 scales uint8 [.., R, C/32]) using moe_quantize_mx."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    B, R, C = w3.shape
    codes = torch.empty((B, R, C // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((B, R, C // 32), dtype=torch.uint8, device=w.device)
    ml.moe_quantize_mx(w3.contiguous(), B, R, C, ml.MX_E2M1, codes, scales)
    if squeeze:
        return codes[0], scales[0]
    return codes, scales


def pack_panel(w: torch.Tensor) -> torch.Tensor:
    """[B, R, C] or [R, C] bf16 -> the same values in panel layout
    ([B, C/32, R, 32]), made by moe_pack_panel; returned with w's shape."""
    w3 = w.unsqueeze(0) if w.dim() == 2 else w
    B, R, C = w3.shape
    out = torch.empty_like(w)
    ml.moe_pack_panel(w3.contiguous(), B, R, C, out)
    return out


def pack_panel_mx(codes: torch.Tensor, scales: torch.Tensor):
    """MXFP4 codes [B, R, C/2] and scales [B, R, C/32] (or without B) -> the
    MX panel layout ([B, C/128, R, 64] and [B, C/128, R, 4] bytes), made by
    moe_pack_panel_mx; returned with the inputs' shapes."""
    c3 = codes.unsqueeze(0) if codes.dim() == 2 else codes
    s3 = scales.unsqueeze(0) if scales.dim() == 2 else scales
    B, R, half = c3.shape
    oc, os_ = torch.empty_like(codes), torch.empty_like(scales)
    ml.moe_pack_panel_mx(c3.contiguous(), s3.contiguous(), B, R, 2 * half, oc, os_)
    return oc, os_


def upload(d: Dict[str, np.ndarray], fp8: bool, keep_bf16: bool = False,
           panel: bool = False, mx: bool = False) -> Dict[str, torch.Tensor]:
    """Move a make_inputs() batch to the GPU.  With fp8, the weights are
    converted to E4M3 + 128x128 block scales on the device (load-time
    conversion) and the bf16 copies are dropped unless keep_bf16.  With
    panel (bf16 or mx), the weights are repacked into panel layout at load
    time (use the problem's LAYOUT_PANEL_WEIGHTS bit with them).  With mx,
    the weights become MXFP4 (E2M1 codes and E8M0 scales, load-time
    conversion by the library)."""
    out: Dict[str, torch.Tensor] = {}
    out["logits"] = torch.from_numpy(d["logits"]).cuda()
    out["x"] = bf16_from_bits(d["x"])
    for name in ("w13", "w2", "ws13", "ws2"):
        if name not in d:
            continue
        wb = bf16_from_bits(d[name])
        if mx:
            out[name + "_q"], out[name + "_s"] = quantize_mx4(wb)
            if panel:
                out[name + "_q"], out[name + "_s"] = pack_panel_mx(out[name + "_q"],
                                                                   out[name + "_s"])
            if keep_bf16:
                out[name] = wb
            else:
                del wb
        elif fp8:
            q, s = quantize_fp8(wb, 128)
            out[name + "_q"], out[name + "_s"] = q, s
            if keep_bf16:
                out[name] = wb
            else:
                del wb
        elif panel:
            out[name] = pack_panel(wb)
            del wb
        else:
            out[name] = wb
    return out


def weights_of(dev: Dict[str, torch.Tensor], fp8: bool) -> ml.moe_weights:
    """The weights struct; quantised weights (block-FP8 or MXFP4, whichever
    upload made) when fp8 is set."""
    if fp8:
        return ml.weights_struct(dev["w13_q"], dev["w2_q"], dev.get("ws13_q"), dev.get("ws2_q"),
                                 dev["w13_s"], dev["w2_s"], dev.get("ws13_s"), dev.get("ws2_s"))
    return ml.weights_struct(dev["w13"], dev["w2"], dev.get("ws13"), dev.get("ws2"))
