"""Benchmark of the MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one moe_layer call -- route, dispatch, grouped SwiGLU FFN (and
shared expert), combine -- over one batch of the workload, with inputs
already resident in HBM.  Prints ONE JSON line: MoE-layer tokens/s as
`value`, the grouped FFN's TFLOP/s against the MFMA peak (or, for the
decode workload, its bytes/s against HBM) as `roofline`, and the CPU
oracle on a bounded sample of the same workload as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_30b_prefill")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens of the workload the CPU oracle runs on (0 = skip)")
    ap.add_argument("--ffn-reps", type=int, default=None)
    ap.add_argument("--layout", choices=("panel", "rows"), default="panel",
                    help="bf16 storage: panel = weights packed once at load time and panel "
                         "activations in the staged calls (moe_layer always keeps its own "
                         "activations in panel layout); rows = everything row major")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="finish with three 1 GiB device copies (a known-size reference "
                         "for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def sources_digest() -> str:
    """sha256 over the HIP library sources: identifies the kernels a stored
    traffic measurement belongs to."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_expert_layer_gate_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per grouped-FFN launch from the committed counter runs
    (profiles/grouped_ffn_<workload>.traffic.json), or None when the kernel
    sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"grouped_ffn_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("sources_sha256") != sources_digest():
        return None
    return rec.get("bytes_per_launch")


def gemm_rows(counts, fp8: bool, n_cap: int, E_L: int) -> int:
    """Token rows the GEMMs compute, padding included, under the library's
    tile choice: 128-row tiles for up to 256 rows per expert on average, else
    256-row tiles (bf16: a last remainder of 1..128 rows takes a 128-row wide
    tile)."""
    rows = 0
    for c in (int(x) for x in counts):
        if n_cap // E_L <= 256:
            rows += -(-c // 128) * 128
        elif fp8:
            rows += -(-c // 256) * 256
        else:
            rem = c % 256
            rows += c - rem + (256 if rem > 128 else 128 if rem else 0)
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_expert_layer_gate_amd import device as dv
    from moe_expert_layer_gate_amd import inputs as synth
    from moe_expert_layer_gate_amd import moelayer as ml

    cfg = synth.config(args.workload)
    seed = args.seed if args.seed is not None else 2
    dev_id = int(os.environ.get("LOCAL_RANK", "0"))
    torch.cuda.set_device(dev_id)
    d = synth.make_inputs(cfg, seed)
    panel = args.layout == "panel" and not cfg.fp8
    dev = dv.upload(d, cfg.fp8, panel=panel)   # load-time packing, outside any timing
    p = ml.Problem.from_config(cfg, layout=ml.LAYOUT_PANEL_WEIGHTS if panel else 0)
    # the staged calls run with the layouts moe_layer uses inside
    p_st = ml.Problem.from_config(
        cfg, layout=(ml.LAYOUT_PANEL_WEIGHTS | ml.LAYOUT_PANEL_ACTS) if panel else 0)
    W = dv.weights_of(dev, cfg.fp8)
    ws = dv.workspace(p)
    y = torch.empty((p.T, p.H), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        ml.moe_layer(p, dev["logits"], dev["x"], W, y, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = p.T * args.steps / elapsed

    # ---- staged calls: per-stage times and the grouped FFN on its own ----
    i32 = dict(dtype=torch.int32, device="cuda")
    N = p.n_cap
    ids = torch.empty((p.T, p.k), **i32)
    tw = torch.empty((p.T, p.k), dtype=torch.float32, device="cuda")
    counts, offsets = torch.empty(p.E_L, **i32), torch.empty(p.E_L + 1, **i32)
    rt, rs, tsr = torch.empty(N, **i32), torch.empty(N, **i32), torch.empty((p.T, p.k), **i32)
    if cfg.fp8:
        xp = torch.empty((N, p.H), dtype=torch.uint8, device="cuda")
        xs = torch.empty((N, p.H // 128), dtype=torch.float32, device="cuda")
    else:
        xp = torch.empty((N, p.H), dtype=torch.bfloat16, device="cuda")
        xs = None
    yp = torch.empty((N, p.H), dtype=torch.bfloat16, device="cuda")
    ws_d = dv.workspace(p, ml.STAGE_DISPATCH)
    ws_f = dv.workspace(p, ml.STAGE_FFN)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    stages = {"route": [], "dispatch": [], "grouped_ffn": [], "combine": []}
    for it in range(max(3, min(args.steps, 10))):
        e = [ev() for _ in range(5)]
        e[0].record(stream)
        ml.moe_route(p_st, dev["logits"], ids, tw, stream)
        e[1].record(stream)
        ml.moe_dispatch(p_st, dev["x"], ids, counts, offsets, rt, rs, tsr, xp, xs, ws_d, stream)
        e[2].record(stream)
        ml.moe_grouped_ffn(p_st, xp, xs, offsets, W, None, None, yp, ws_f, stream)
        e[3].record(stream)
        ml.moe_combine(p_st, yp, tsr, tw, None, y, stream)
        e[4].record(stream)
        torch.cuda.synchronize()
        if it == 0:
            continue  # first pass warms the staged buffers
        for name, a, b in zip(stages, e[:-1], e[1:]):
            stages[name].append(a.elapsed_time(b))
    stage_ms = {k: float(np.median(v)) for k, v in stages.items()}

    # The grouped FFN timed launch by launch on the stream it runs on.
    reps = args.ffn_reps or max(args.steps, 20)
    starts, ends = [ev() for _ in range(reps)], [ev() for _ in range(reps)]
    for i in range(reps):
        starts[i].record(stream)
        ml.moe_grouped_ffn(p_st, xp, xs, offsets, W, None, None, yp, ws_f, stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)]))

    n_pairs = int(offsets[-1].item())
    cnt = counts.cpu().numpy()
    flops = 6.0 * p.H * p.I * n_pairs
    dtype = "fp8" if cfg.fp8 else "bf16"
    beta_w = 1 if cfg.fp8 else 2
    active = int((cnt > 0).sum())
    ffn_tflops = flops / (ffn_ms * 1e-3) / 1e12
    padded_rows = gemm_rows(cnt, cfg.fp8, p.n_cap, p.E_L)

    traffic = stored_traffic(cfg.name)
    # Few rows per expert: the FFN streams weights and is bound by HBM.
    decode = n_pairs < 64 * max(active, 1)
    if decode:
        # weight streaming: every active expert's W13 and W2 once, plus the
        # permuted activations in and out of both GEMMs
        bytes_ = (active * 3 * p.H * p.I * beta_w
                  + n_pairs * (p.H * beta_w + 2 * p.I * beta_w + 2 * p.H))
        achieved = bytes_ / (ffn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": "moe_grouped_ffn (tile schedule + up GEMM/SwiGLU + down GEMM)",
                "work_per_launch": {"bytes": bytes_}, "avg_launch_ms": round(ffn_ms, 4)}
    else:
        peak = PEAK_TFLOPS[dtype]
        roof = {"bound": "mfma", "achieved": round(ffn_tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ffn_tflops / peak, 4), "traffic": traffic,
                "kernel": "moe_grouped_ffn (tile schedule + up GEMM/SwiGLU + down GEMM)",
                "work_per_launch": {"flops": flops}, "avg_launch_ms": round(ffn_ms, 4)}

    # ---- CPU baseline: the oracle on a bounded sample of the same workload ----
    cpu = None
    sample = args.cpu_sample_tokens
    if sample is None:
        sample = {"tiny": 256, "qwen3_30b_prefill": 4096, "dsv3_ep8_prefill": 128,
                  "dsv3_ep8_prefill_fp8": 64, "dsv3_ep8_decode": 64}.get(cfg.name, 256)
    if sample > 0:
        cpu = cpu_baseline(cfg, d, sample)

    out = {
        "metric": "MoE-layer tokens/s and grouped-FFN TFLOP/s (% MFMA peak) on 1 MI355X",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,0.02) activations/weights, generated routing logits)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "experts": cfg.E,
                   "local_experts": cfg.E_L, "expert_begin": cfg.e_lo, "top_k": cfg.k,
                   "inter": cfg.I, "shared_inter": cfg.I_s, "seed": seed,
                   "layout": "panel" if panel else "rows"},
        "grouped_ffn_tflops": round(ffn_tflops, 2),
        "grouped_ffn_frac_of_peak": round(ffn_tflops / PEAK_TFLOPS[dtype], 4),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "routing": {"local_pairs": n_pairs, "active_experts": active,
                    "rows_per_expert_max": int(cnt.max()), "rows_per_expert_mean": round(float(cnt.mean()), 1),
                    "gemm_rows_computed": padded_rows,
                    "padding_frac": round(padded_rows / max(n_pairs, 1) - 1.0, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


def cpu_baseline(cfg, d, sample):
    """The oracle, as it stands, on the first `sample` tokens."""
    import numpy as np

    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    T = min(sample, cfg.T)
    wd = d
    if cfg.fp8:
        wd = {}
        for name in ("w13", "w2"):
            qs = [O.quantize_blocks(O.bf16_to_f64(m), 128, 128) for m in d[name]]
            wd[name + "_q"] = np.stack([q for q, _ in qs])
            wd[name + "_s"] = np.stack([s for _, s in qs])
        for name in ("ws13", "ws2"):
            if name in d:
                wd[name + "_q"], wd[name + "_s"] = O.quantize_blocks(O.bf16_to_f64(d[name]), 128, 128)
    t0 = time.perf_counter()
    O.moe_layer(d["logits"][:T], d["x"][:T], wd, k=cfg.k, e_lo=cfg.e_lo, E_L=cfg.E_L, fp8=cfg.fp8)
    dt = time.perf_counter() - t0
    return {"value": round(T / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {T} of {cfg.T} tokens of {cfg.name}, whole layer (float64 numpy), "
                      f"{dt:.1f} s"}


if __name__ == "__main__":
    main()
