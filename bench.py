"""Benchmark of the MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: the DeepSeek-V3-shaped shard of an 8-way expert-parallel
layer (16384 tokens, hidden 7168, 32 of 256 experts local, top-8,
intermediate 2048, bf16), the largest configuration that runs on one GPU.

One step is one pass of the layer -- route, dispatch, grouped SwiGLU FFN (and
shared expert), combine -- over one batch of the workload, with inputs
already resident in HBM.  The timed region is K calls of the one-call
moe_layer between two synchronisations; `value` is tokens x K / wall time,
and HIP events around each call give the per-step median, min and mean.
The same kernels are then issued one library call per stage, so that the
grouped FFN's launches can be bracketed by HIP events on their stream: that
gives `stage_ms`, the small stages' GB/s, and the grouped FFN's TFLOP/s
against the MFMA peak (or, for few rows per expert, its bytes/s against HBM)
as `roofline`.  Decode-sized batches also report the whole layer's bytes/s
against HBM.  A working set below 512 MB (it would stay in the MALL between
back-to-back calls) is also timed call by call after a 512 MB write.  Prints
ONE JSON line, with the GPU's clock and power under load, the host, and the
CPU oracle on a bounded sample of the same workload as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense MFMA; the MX path runs E2M1 x E4M3 instructions, priced at the
# fp8 rate (the 10.1 PF fp4 figure needs both operands in fp4)
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 5000.0}
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 for the latency-bound tiny workload)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_ep8_prefill")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens of the workload the CPU oracle runs on (0 = skip)")
    ap.add_argument("--layout", choices=("panel", "rows"), default="panel",
                    help="panel = weights packed once at load time (bf16 and MXFP4) and, "
                         "bf16, panel activations in the staged calls (moe_layer always keeps "
                         "its own bf16 activations in panel layout); rows = everything row "
                         "major.  Block-FP8 is always row major")
    ap.add_argument("--masked", action="store_true",
                    help="masked fixed-capacity expert layout (capacity = tokens) instead of "
                         "contiguous segments")
    ap.add_argument("--stream", action="store_true",
                    help="also measure the streaming FFN (workloads with replicas): the FFN "
                         "throughput curve, the launch threshold at rho, and the streamed layer "
                         "against the one-call layer")
    ap.add_argument("--rho", type=float, default=0.90)
    ap.add_argument("--streams", type=int, default=2)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the HIP-graph replay and the clock/power sampling (for runs "
                         "under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="finish with three passes of an elementwise kernel over 1 GiB in "
                         "and 1 GiB out (a known-size reference for the FETCH_SIZE / WRITE_SIZE "
                         "counters)")
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


def gemm_rows(counts, fp8: bool, max_pairs: int, E_L: int, mx: bool = False) -> int:
    """Token rows the GEMMs compute, padding included, under the library's
    tile choice (from the most pairs per expert on average, T min(k, E_L) /
    E_L): bf16 32-row tiles up to 32; 128-row tiles up to 256; else 256-row
    tiles, 384-row from 1536 (bf16: a last remainder of 1..128 rows takes a
    128-row wide tile; block-FP8 takes 32-row tiles up to 32 too).
    MX: 32-row tiles up to 32, 128-row up to 256, else 256-row tiles."""
    rows = 0
    tall = max_pairs // E_L >= 1536
    for c in (int(x) for x in counts):
        if mx:
            r = max_pairs // E_L
            tm = 256 if r > 256 else 128 if r > 32 else 32
            rows += -(-c // tm) * tm
        elif max_pairs // E_L <= 32:
            rows += -(-c // 32) * 32
        elif max_pairs // E_L <= 256:
            rows += -(-c // 128) * 128
        elif fp8:
            rows += -(-c // 256) * 256
        else:
            bm = 384 if tall else 256
            rem = c % bm
            rows += c - rem + (bm if rem > 128 else 128 if rem else 0)
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs on one GPU per process "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_expert_layer_gate_amd import device as dv
    from moe_expert_layer_gate_amd import inputs as synth
    from moe_expert_layer_gate_amd import moelayer as ml

    cfg = synth.config(args.workload)
    seed = args.seed if args.seed is not None else 2
    if args.steps is None:
        args.steps = 200 if cfg.name == "tiny" else 20
    dev_id = int(os.environ.get("LOCAL_RANK", "0"))
    torch.cuda.set_device(dev_id)
    d = synth.make_inputs(cfg, seed)
    quant = cfg.fp8 or cfg.mx          # quantised GEMM activations with per-row scales
    panel = args.layout == "panel" and not cfg.fp8   # bf16 and MXFP4 weights
    dev = dv.upload(d, cfg.fp8, panel=panel, mx=cfg.mx)   # load-time conversion, untimed
    # Layouts of moe_layer's own path: panel weights as loaded, panel h (bf16;
    # MXFP4 activations stay row major).
    cap = cfg.T if args.masked else 0
    wlay = ml.LAYOUT_PANEL_WEIGHTS if panel else 0
    p = ml.Problem.from_config(
        cfg, layout=wlay | (ml.LAYOUT_PANEL_ACTS if panel and not quant else 0), capacity=cap)
    p_layer = ml.Problem.from_config(cfg, layout=ml.LAYOUT_PANEL_WEIGHTS if panel else 0,
                                     capacity=cap)
    W = dv.weights_of(dev, quant)
    stream = torch.cuda.current_stream()
    T, k, H, N = p.T, p.k, p.H, p.n_cap
    i32 = dict(dtype=torch.int32, device="cuda")
    ids = torch.empty((T, k), **i32)
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts, offsets = torch.empty(p.E_L, **i32), torch.empty(p.E_L + 1, **i32)
    rt, rs, tsr = torch.empty(N, **i32), torch.empty(N, **i32), torch.empty((T, k), **i32)
    yp = torch.empty((N, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws_d = dv.workspace(p, ml.STAGE_DISPATCH)
    ws_f = dv.workspace(p, ml.STAGE_FFN)
    if quant:
        # activation scales: fp32 per 128 (block-FP8) or E8M0 bytes per 32 (MX)
        sc = dict(dtype=torch.uint8, device="cuda") if cfg.mx else \
            dict(dtype=torch.float32, device="cuda")
        g = 32 if cfg.mx else 128
        # the tokens quantised once, gathered by the FFN
        xq = torch.empty((T, H), dtype=torch.uint8, device="cuda")
        xqs = torch.empty((T, H // g), **sc)
        if p.I_s:
            q = ml.Problem(T=T, H=H, E=1, k=1, e_lo=0, E_L=1, I=p.I_s, fp8=cfg.fp8, mx=cfg.mx,
                           layout=wlay)
            off2 = torch.tensor([0, T], **i32)
            sw = ml.weights_struct(dev["ws13_q"], dev["ws2_q"], None, None, dev["ws13_s"],
                                   dev["ws2_s"])
            shared = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
            ws_s = dv.workspace(q, ml.STAGE_FFN)

    seg = counts if cap else offsets   # segment table of the FFN calls (masked: counts)

    # One step: moe_layer's kernels, one library call per stage, so that the
    # grouped FFN's launches inside the timed region can be bracketed with
    # HIP events on the stream they run on.  bf16: route, index-only
    # dispatch, the FFN gathering its rows from x, combine.  block-FP8 and
    # MX: route, index-only dispatch and x quantised once, the FFN gathering
    # its rows from those codes, the shared expert on them, combine.
    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev else (lambda i: None)
        rec(0)
        ml.moe_route(p, dev["logits"], ids, tw, stream)
        rec(1)
        if not quant:
            ml.moe_dispatch(p, dev["x"], ids, counts, offsets, rt, rs, tsr, None, None, ws_d,
                            stream)
            rec(2)
            ml.moe_grouped_ffn_gather(p, dev["x"], None, rt, seg, W, None, None, yp, ws_f,
                                      stream)
            rec(3)
            sh = None
        else:
            ml.moe_dispatch(p, dev["x"], ids, counts, offsets, rt, rs, tsr, None, None, ws_d,
                            stream)
            if cfg.mx:
                ml.moe_quantize_mx(dev["x"], 1, T, H, ml.MX_E4M3, xq, xqs, stream)
            else:
                ml.moe_quantize_fp8(dev["x"], 1, T, H, 1, xq, xqs, stream)
            rec(2)
            ml.moe_grouped_ffn_gather(p, xq, xqs, rt, seg, W, None, None, yp, ws_f, stream)
            sh = None
            if p.I_s:
                ml.moe_grouped_ffn(q, xq, xqs, off2, sw, None, None, shared, ws_s, stream)
                sh = shared
            rec(3)
        ml.moe_combine(p, yp, tsr, tw, sh, y, stream)
        rec(4)

    # ---- the headline: the one-call moe_layer, K calls between two
    # synchronisations, each bracketed by HIP events on its stream ----
    ws_l = dv.workspace(p_layer)
    y_l = torch.empty_like(y)

    def layer():
        ml.moe_layer(p_layer, dev["logits"], dev["x"], W, y_l, ws_l, stream)

    for _ in range(args.warmup):
        layer()
    torch.cuda.synchronize()
    lev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        lev[i].record(stream)
        layer()
    lev[args.steps].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed
    layer_ms = [lev[i].elapsed_time(lev[i + 1]) for i in range(args.steps)]

    # A working set that fits the 256 MB MALL would be timed from the cache
    # by back-to-back calls: then each call is also timed alone after a
    # 512 MB write that evicts it (reported beside the headline).
    ws_bytes = sum(t_.numel() * t_.element_size() for t_ in dev.values()
                   if isinstance(t_, torch.Tensor))
    flushed = None
    if ws_bytes < (512 << 20) and not args.no_extras:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        fl = []
        for _ in range(min(args.steps, 50)):
            scratch.fill_(1)
            a_ = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            layer()
            b_.record(stream)
            torch.cuda.synchronize()
            fl.append(a_.elapsed_time(b_))
        del scratch
        flushed = {"median": round(float(np.median(fl)), 4), "min": round(float(np.min(fl)), 4),
                   "working_set_bytes": int(ws_bytes)}

    # ---- the same kernels one library call per stage, so that the grouped
    # FFN's launches can be bracketed by events on their stream ----
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    staged_tps = T * args.steps / (time.perf_counter() - t1)
    names = ("route", "dispatch", "grouped_ffn", "combine")
    per = {n: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, n in enumerate(names)}
    stage_ms = {n: float(np.median(v)) for n, v in per.items()}
    ffn_ms = float(np.mean(per["grouped_ffn"]))   # the FFN launches of the timed steps
    y_steps = y.clone()
    same = bool(torch.equal(y_l.view(torch.int16), y_steps.view(torch.int16)))

    # The one-call layer captured once in a HIP graph and replayed K times
    # (how a serving loop replays a step): no per-launch host work.  Same
    # output bits as the calls above.  The clock and power of the GPU are
    # sampled while it replays.
    graph_tps = same_graph = gpu = None
    if not args.no_extras:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            ml.moe_layer(p_layer, dev["logits"], dev["x"], W, y_l, ws_l)
        y_l.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same_graph = bool(torch.equal(y_l.view(torch.int16), y_steps.view(torch.int16)))
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_tps = T * args.steps / (time.perf_counter() - t2)
        gpu = gpu_under_load(lambda: graph.replay(), float(np.median(layer_ms)))

    cnt = counts.cpu().numpy()
    n_pairs = int(cnt.sum())
    # 2 m H I (up, m first-layer matrices) + 2 H I (down) per row (Eq. 8)
    mm = 2.0 * (p.m + 1)
    flops = mm * p.H * p.I * n_pairs + mm * p.H * p.I_s * p.T
    dtype = "mxfp4" if cfg.mx else "fp8" if cfg.fp8 else "bf16"
    # bytes per weight element (MXFP4: half a byte plus one E8M0 byte per 32)
    beta_w = 0.5 + 1 / 32 if cfg.mx else 1 if cfg.fp8 else 2
    beta_a = 1 + 1 / 32 if cfg.mx else 1 if cfg.fp8 else 2   # GEMM activation bytes
    active = int((cnt > 0).sum())
    ffn_tflops = flops / (ffn_ms * 1e-3) / 1e12
    padded_rows = gemm_rows(cnt, quant, p.T * min(p.k, p.E_L), p.E_L, cfg.mx)

    # HBM bytes of the small stages (what each must move at least) and their
    # rates over the stage's median time: route T E 4 + T k 8; dispatch (the
    # index build: ids in, row_token / row_slot / token_slot_row out, T k 16;
    # quantised paths also read x once and write its codes and scales);
    # combine N H 2 + T H 2 (+ the shared expert's T H 2) + T k 8.
    a_scale = (1 / 32 if cfg.mx else 4 / 128) if quant else 0
    stage_bytes = {
        "route": p.T * p.E * 4 + p.T * p.k * 8,
        "dispatch": p.T * p.k * 16 + (p.T * p.H * (2 + 1 + a_scale) if quant else 0),
        "combine": n_pairs * p.H * 2 + p.T * p.H * 2 * (2 if p.I_s else 1) + p.T * p.k * 8,
    }
    stage_rates = {n: round(b / (stage_ms[n] * 1e-3) / 1e9, 1) for n, b in stage_bytes.items()}

    traffic = stored_traffic(cfg.name + ("_masked" if cap else ""))
    act = "SwiGLU" if cfg.act == "swiglu" else "GELU"
    skinny = p.T * min(p.k, p.E_L) // p.E_L <= 32
    kernel = ((f"grouped FFN: work table + one launch of up GEMM/{act} and down GEMM" if skinny
               else f"grouped FFN: work table + up GEMM/{act} + down GEMM")
              + (" (+ shared expert: x quantisation and its FFN)" if p.I_s else ""))
    # Few rows per expert: the FFN streams weights and is bound by HBM.
    decode = n_pairs < 64 * max(active, 1)
    decode_layer = None
    if decode:
        # weight streaming: every active expert's W13 and W2 once, plus the
        # token rows in and out of both GEMMs
        bytes_ = int(active * (p.m + 1) * p.H * p.I * beta_w
                     + n_pairs * (p.H * beta_a + 2 * p.I * beta_a + 2 * p.H))
        achieved = bytes_ / (ffn_ms * 1e-3) / 1e9
        # the whole layer against HBM: those weights, x in, y out, the
        # logits and the index bytes, over the one-call layer's median step
        layer_bytes = int(active * (p.m + 1) * p.H * p.I * beta_w + 2 * p.T * p.H * 2
                          + p.T * p.E * 4 + p.T * p.k * 16)
        layer_gbs = layer_bytes / (float(np.median(layer_ms)) * 1e-3) / 1e9
        decode_layer = {"bytes": layer_bytes, "gbs": round(layer_gbs, 1),
                        "frac_hbm": round(layer_gbs / PEAK_HBM_GBS, 4)}
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": kernel, "work_per_launch": {"bytes": bytes_},
                "avg_launch_ms": round(ffn_ms, 4)}
    else:
        peak = PEAK_TFLOPS[dtype]
        roof = {"bound": "mfma", "achieved": round(ffn_tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ffn_tflops / peak, 4), "traffic": traffic,
                "kernel": kernel, "work_per_launch": {"flops": flops},
                "avg_launch_ms": round(ffn_ms, 4)}

    # ---- CPU baseline: the oracle on a bounded sample of the same workload ----
    cpu = None
    sample = args.cpu_sample_tokens
    if sample is None:
        # about 10-30 s of CPU work on the GPU host (the block-FP8 and MX oracles
        # dequantise every active expert's weights in float64 first: a fixed cost)
        sample = {"tiny": 256, "qwen3_30b_prefill": 8192, "dsv3_ep8_prefill": 16384,
                  "dsv3_ep8_prefill_fp8": 256, "dsv3_ep8_decode": 64,
                  "dsv3_ep8_prefill_mxfp4": 256, "dsv3_ep8_decode_mxfp4": 64,
                  "dsv3_ep8_decode_fp8": 64}.get(cfg.name, 256)
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
                   "mlp": "gated SwiGLU" if cfg.act == "swiglu" else "standard GELU",
                   "layout": "panel" if panel else "rows",
                   "expert_layout": f"masked (capacity {cap})" if cap else "contiguous"},
        "grouped_ffn_tflops": round(ffn_tflops, 2),
        "grouped_ffn_frac_of_peak": round(ffn_tflops / PEAK_TFLOPS[dtype], 4),
        # quantised paths: the same rate against the bf16 peak as well
        "grouped_ffn_frac_of_bf16_peak": round(ffn_tflops / PEAK_TFLOPS["bf16"], 4),
        "timed": "moe_layer, one call per step; value = tokens x steps / wall time "
                 "between synchronisations",
        "step_ms": {"median": round(float(np.median(layer_ms)), 4),
                    "min": round(float(np.min(layer_ms)), 4),
                    "mean": round(float(np.mean(layer_ms)), 4)},
        "step_ms_mall_flushed": flushed,
        "decode_layer_hbm": decode_layer,
        "stage_ms": {k2: round(v, 4) for k2, v in stage_ms.items()},
        "stage_gbs": stage_rates,
        "staged_calls": {"tokens_per_s": round(staged_tps, 1), "same_output_bits": same},
        "moe_layer_graph": ({"tokens_per_s": round(graph_tps, 1), "same_output_bits": same_graph}
                            if graph_tps else None),
        "gpu": gpu,
        "host": host_info(),
        "routing": {"local_pairs": n_pairs, "active_experts": active,
                    "rows_per_expert_max": int(cnt.max()), "rows_per_expert_mean": round(float(cnt.mean()), 1),
                    "gemm_rows_computed": padded_rows,
                    "padding_frac": round(padded_rows / max(n_pairs, 1) - 1.0, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.stream:
        out["streamffn"] = stream_bench(args, cfg, d, p_layer, W, dev)
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        # a plain elementwise kernel over 1 GiB in and 1 GiB out (three times):
        # the known-size reference of the FETCH_SIZE / WRITE_SIZE counters
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()


def host_info():
    """The host the CPU baseline runs on: logical CPUs, those this process
    may use, and the CPU model."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "cpu_model": model}


def _smi(args):
    """rocm-smi's JSON for the first card, or None."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", *args, "--json"], capture_output=True, text=True,
                           timeout=30)
        d = json.loads(r.stdout[r.stdout.index("{"):])
        return next(iter(d.values()))
    except Exception:
        return None


def _num(v):
    import re
    m = re.search(r"[-+]?[0-9]*\.?[0-9]+", str(v))
    return float(m.group(0)) if m else None


def gpu_under_load(replay, step_ms):
    """The GPU's name, power cap, and its graphics clock and socket power
    sampled by rocm-smi while `replay` keeps it busy (about two seconds of
    replays)."""
    import threading

    import torch
    props = torch.cuda.get_device_properties(0)
    out = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count, "power_cap_w": None,
           "sclk_mhz_under_load": None, "power_w_under_load": None}
    cap = _smi(["--showmaxpower"])
    if cap:
        out["power_cap_w"] = next((_num(v) for k, v in cap.items() if "Max" in k and "Power" in k),
                                  None)
    sample = {}

    def probe():
        time.sleep(0.5)
        sample.update(_smi(["--showclocks", "--showpower"]) or {})

    th = threading.Thread(target=probe)
    th.start()
    t_end = time.perf_counter() + 2.5
    n = max(1, int(50.0 / max(step_ms, 1e-3)))      # ~50 ms of GPU work per batch
    while th.is_alive() and time.perf_counter() < t_end + 30:
        for _ in range(n):
            replay()
        torch.cuda.synchronize()
    th.join()
    for k, v in sample.items():
        if "sclk" in k and "speed" in k:
            out["sclk_mhz_under_load"] = _num(v)
        if "Power" in k and "Max" not in k:
            out["power_w_under_load"] = _num(v)
    return out


def _time_ms(fn, reps):
    """Median wall time of fn() on the GPU, bracketed by synchronisations."""
    import torch
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        ts.append((time.perf_counter() - t0) * 1e3)
    return sorted(ts)[len(ts) // 2]


def stream_bench(args, cfg, d, p_layer, W, dev):
    """Streaming FFN on one GPU (CascadeEP section 3.2): the replicas' rows
    arrive in ascending order of size; the FFN throughput curve over
    arrival-order prefixes gives the launch threshold theta at rho; the
    threshold plan's invocations run as moe_layer_streamed on several streams
    and are timed against the one-call layer (synchronous) and one invocation
    per replica on one stream (asynchronous without threshold)."""
    import dataclasses

    import numpy as np
    import torch

    from moe_expert_layer_gate_amd import device as dv
    from moe_expert_layer_gate_amd import inputs as synth
    from moe_expert_layer_gate_amd import moelayer as ml

    if "replica_offsets" not in d:
        return {"error": "workload has no replica split"}
    off = d["replica_offsets"]
    perm = torch.from_numpy(synth.arrival_permutation(off)).cuda()
    logits = dev["logits"][perm].contiguous()
    x = dev["x"][perm].contiguous()
    T, k, H = p_layer.T, p_layer.k, p_layer.H
    sizes = [int(off[r + 1] - off[r]) for r in synth.replica_arrival(off)]
    bounds = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    i32 = dict(dtype=torch.int32, device="cuda")
    ids = torch.empty((T, k), **i32)
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ml.moe_route(p_layer, logits, ids, tw)
    loc = ((ids >= p_layer.e_lo) & (ids < p_layer.e_lo + p_layer.E_L)).sum(1).cpu().numpy()
    ready = [int(loc[bounds[i]:bounds[i + 1]].sum()) for i in range(len(sizes))]

    # FFN throughput against expert-token count (rows of one invocation)
    pf = dataclasses.replace(p_layer, layout=p_layer.layout | ml.LAYOUT_PANEL_ACTS) \
        if not p_layer.fp8 else p_layer
    curve = []
    t_pts = sorted({t for t in (256, 512, 1024, 2048, 3072, 4096, 6144, 8192, 12288, T) if t <= T})
    for tp in t_pts:
        q = dataclasses.replace(pf, T=tp)
        N = q.n_cap
        cnt, offs = torch.empty(q.E_L, **i32), torch.empty(q.E_L + 1, **i32)
        rt, rs, tsr = torch.empty(N, **i32), torch.empty(N, **i32), torch.empty((tp, k), **i32)
        yp = torch.empty((N, H), dtype=torch.bfloat16, device="cuda")
        ml.moe_dispatch(q, x, ids, cnt, offs, rt, rs, tsr, None, None,
                        dv.workspace(q, ml.STAGE_DISPATCH))
        wsf = dv.workspace(q, ml.STAGE_FFN)
        if q.fp8:   # the FFN gathers from the tokens quantised once
            xq = torch.empty((tp, H), dtype=torch.uint8, device="cuda")
            xqs = torch.empty((tp, H // 128), dtype=torch.float32, device="cuda")
            ml.moe_quantize_fp8(x, 1, tp, H, 1, xq, xqs)
            fn = lambda: ml.moe_grouped_ffn_gather(q, xq, xqs, rt, offs, W, None, None, yp, wsf)
        else:
            fn = lambda: ml.moe_grouped_ffn_gather(q, x, None, rt, offs, W, None, None, yp, wsf)
        fn()
        ms = _time_ms(fn, 7)
        pairs = int(cnt.sum().item())
        tfl = 2.0 * (q.m + 1) * H * q.I * pairs / (ms * 1e-3) / 1e12
        curve.append({"tokens": tp, "expert_tokens": pairs, "ffn_ms": round(ms, 4),
                      "tflops": round(tfl, 1)})
        del yp, rt, rs, tsr, wsf
    theta = ml.stream_threshold([c["expert_tokens"] for c in curve],
                                [c["tflops"] for c in curve], args.rho)
    ends = ml.stream_plan(ready, theta)
    groups = [0] + [int(bounds[e]) for e in ends]
    per_replica = [int(b) for b in bounds]

    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws_l = dv.workspace(p_layer)
    cur = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in range(max(1, args.streams))]

    def streamed(g, ns):
        gmax = max(b - a for a, b in zip(g[:-1], g[1:]))
        ws = torch.empty(ml.workspace_bytes_streamed(p_layer, gmax, ns), dtype=torch.uint8,
                         device="cuda")

        def run():
            for st in streams[:ns]:
                st.wait_stream(cur)
            ml.moe_layer_streamed(p_layer, logits, x, W, y, g, streams[:ns], ws)
            for st in streams[:ns]:
                cur.wait_stream(st)
        return run

    reps = max(5, args.steps // 2)
    sync_fn = lambda: ml.moe_layer(p_layer, logits, x, W, y, ws_l)
    runs = {"sync": sync_fn, f"stream_{len(streams)}": streamed(groups, len(streams)),
            "stream_1": streamed(groups, 1), "async_per_replica_1": streamed(per_replica, 1)}
    res = {}
    for name, fn in runs.items():
        fn()
        res[name] = round(_time_ms(fn, reps), 4)
    best = res[f"stream_{len(streams)}"]
    return {"rho": args.rho, "theta_expert_tokens": theta, "curve": curve,
            "arrival_replica_tokens": sizes, "arrival_expert_tokens": ready,
            "invocations_tokens": groups, "layer_ms": res,
            "retained_throughput": round(res["sync"] / best, 4),
            "retained_throughput_1_stream": round(res["sync"] / res["stream_1"], 4),
            "retained_throughput_async": round(res["sync"] / res["async_per_replica_1"], 4)}


def cpu_baseline(cfg, d, sample):
    """The oracle, as it stands, on the first `sample` tokens."""
    import numpy as np

    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import moe_oracle as O
    # every CPU this process may use (this host's share for the GPU), capped
    # by OMP_NUM_THREADS where the environment sets one
    ncpu = len(os.sched_getaffinity(0))
    want = min(ncpu, int(os.environ.get("OMP_NUM_THREADS", ncpu) or ncpu))
    limiter = threadpool_limits(limits=want)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    T = min(sample, cfg.T)
    wd = d
    if cfg.mx:
        wd = {}
        for name in ("w13", "w2"):
            qs = [O.mx_quantize(O.bf16_to_f64(m), "e2m1") for m in d[name]]
            wd[name + "_q"] = np.stack([q for q, _ in qs])
            wd[name + "_s"] = np.stack([s for _, s in qs])
        for name in ("ws13", "ws2"):
            if name in d:
                wd[name + "_q"], wd[name + "_s"] = O.mx_quantize(O.bf16_to_f64(d[name]), "e2m1")
    elif cfg.fp8:
        wd = {}
        for name in ("w13", "w2"):
            qs = [O.quantize_blocks(O.bf16_to_f64(m), 128, 128) for m in d[name]]
            wd[name + "_q"] = np.stack([q for q, _ in qs])
            wd[name + "_s"] = np.stack([s for _, s in qs])
        for name in ("ws13", "ws2"):
            if name in d:
                wd[name + "_q"], wd[name + "_s"] = O.quantize_blocks(O.bf16_to_f64(d[name]), 128, 128)
    t0 = time.perf_counter()
    O.moe_layer(d["logits"][:T], d["x"][:T], wd, k=cfg.k, e_lo=cfg.e_lo, E_L=cfg.E_L, fp8=cfg.fp8,
                mx=cfg.mx)
    dt = time.perf_counter() - t0
    limiter.restore_original_limits()
    host = host_info()
    return {"value": round(T / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {T} of {cfg.T} tokens of {cfg.name}, whole layer (float64 numpy, "
                      f"BLAS on {threads} threads), {dt:.1f} s",
            "nproc": host["nproc"], "cpu_model": host["cpu_model"]}


if __name__ == "__main__":
    main()
