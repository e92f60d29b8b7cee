#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

One step = one moe_forward call (router GEMM, top-K, dispatch, grouped gate_up GEMM with fused
SiLU*up, shared expert, grouped down GEMM, weighted gather combine with the final cast) over one
synthetic batch already resident in HBM.

Default workload: the 35B-A3B-shaped layer (D=2048, E=256, top-8, F=512, bf16) at the prefill
batch T=4096; the same layer's decode batch T=64 is timed next to it.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload a3b_prefill]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
# sources the grouped matrix-core GEMM is compiled from (a traffic record is only used if it was
# taken on exactly these)
_CSRC = os.path.join(ROOT, "mixture_experts_layer_renorm_amd", "csrc")
GEMM_SRCS = [os.path.join(_CSRC, f) for f in ("gemm_mfma.hip", "kernels.h", "silu.h")]


def gemm_source_sha256() -> str:
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="a3b_prefill")
    ap.add_argument("--decode-workload", default="a3b_decode")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mfma-workload", default="ds_sigmoid",
                    help="matrix-core-bound workload reported beside the main one")
    ap.add_argument("--no-mfma-workload", action="store_true")
    ap.add_argument("--no-granularity", action="store_true",
                    help="skip the granularity pair (128 experts x F=1536 x top-8 vs "
                         "64 x 3072 x top-4)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0)
    ap.add_argument("--atomic-combine", action="store_true",
                    help="time the fused fp32-atomic combine instead of the default gather")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one 1 GiB device-to-device copy (for PMC scaling)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (same SONAME)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e: int) -> None:
        self.lib.hipEventDestroy(e)


def run_workload(name, steps, warmup, atomic_combine, hip):
    import torch
    from mixture_experts_layer_renorm_amd import abi, costmodel
    from mixture_experts_layer_renorm_amd.synth import CONFIGS, make_layer

    cfg = CONFIGS[name]
    dev = "cuda"
    layer = make_layer(cfg, device=dev, seed=0)
    p = abi.make_problem(T=cfg.T, D=cfg.D, E=cfg.E, K=cfg.K, F=cfg.F, F_shared=cfg.F_shared,
                         shared_gated=cfg.shared_gated, scoring=cfg.scoring, dtype=cfg.torch_dtype,
                         atomic_combine=atomic_combine)
    weights = {"w_router": layer["w_router"], "logit_bias": layer["logit_bias"],
               "w_gate_up": layer["w_gate_up"], "w_down": layer["w_down"],
               "ws_gate_up": layer["ws_gate_up"], "ws_down": layer["ws_down"],
               "ws_gate": layer["w_shared_gate"]}
    routing = abi.alloc_routing(p, dev, logits=False)
    out = torch.empty((cfg.T, cfg.D), dtype=cfg.torch_dtype, device=dev)
    ws = abi.alloc_workspace(p, dev)
    x = layer["x"]

    for _ in range(warmup):
        abi.moe_forward(p, x, weights, routing, out, ws)
    torch.cuda.synchronize()

    # Timed region: the forward as a caller runs it, with one pair of HIP events on its stream
    # bracketing the routed gate_up launch(es) of each step (the roofline's kernel).
    n_ev = abi.MOE_STAGE_COUNT + 1
    gu_ev = [[hip.create(), hip.create()] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ev = [None] * n_ev
        ev[abi.MOE_STAGE_GATE_UP], ev[abi.MOE_STAGE_GATE_UP + 1] = gu_ev[k]
        abi.moe_forward_timed(p, x, weights, routing, out, ws, ev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gate_up_live_ms = sum(hip.elapsed_ms(a, b) for a, b in gu_ev) / steps
    for pair in gu_ev:
        for e in pair:
            hip.destroy(e)

    # Per-stage breakdown from a second pass with HIP events between the stages (each marker
    # adds a few microseconds, so these stages sum to more than the plain step).
    events = [[hip.create() for _ in range(n_ev)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        abi.moe_forward_timed(p, x, weights, routing, out, ws, events[k])
    torch.cuda.synchronize()

    stage_ms = [0.0] * abi.MOE_STAGE_COUNT
    for k in range(steps):
        for i in range(abi.MOE_STAGE_COUNT):
            stage_ms[i] += hip.elapsed_ms(events[k][i], events[k][i + 1]) / steps
    gpu_ms = hip.elapsed_ms(events[0][0], events[-1][-1]) / steps
    for row in events:
        for e in row:
            hip.destroy(e)

    counts = routing["expert_counts"].cpu()
    U = int((counts > 0).sum())
    nz = counts[counts > 0].float()
    ms_per_step = (t1 - t0) * 1e3 / steps
    A = cfg.T * cfg.K
    gu = costmodel.gate_up(cfg.T, cfg.D, cfg.F, cfg.K, U, cfg.dtype)
    dn = costmodel.down(cfg.T, cfg.D, cfg.F, cfg.K, U, cfg.dtype, cfg.dtype)
    lay = costmodel.layer(cfg.T, cfg.D, cfg.E, cfg.K, cfg.F, U, cfg.F_shared, cfg.shared_gated,
                          cfg.dtype, cfg.dtype)
    st = dict(zip(abi.MOE_STAGE_NAMES, stage_ms))
    res = {
        "workload": name, "plan": abi.describe_plan(p), "T": cfg.T, "D": cfg.D, "E": cfg.E,
        "K": cfg.K, "F": cfg.F, "F_shared": cfg.F_shared, "scoring": cfg.scoring, "dtype": cfg.dtype,
        "ms_per_step": ms_per_step, "gpu_ms_per_step_with_stage_markers": gpu_ms,
        "tokens_per_s": cfg.T / (ms_per_step / 1e3),
        "stage_ms": st, "U": U, "assignments": A,
        "t_e": {"min": int(nz.min()), "median": float(nz.median()), "max": int(nz.max())},
        "layer_tflops": lay["flops"] / (ms_per_step / 1e3) / 1e12,
        "layer_gbs": lay["bytes"] / (ms_per_step / 1e3) / 1e9,
        "gate_up": {"ms": gate_up_live_ms, "alg_bytes": gu["bytes"], "alg_flops": gu["flops"],
                    "gbs": gu["bytes"] / (gate_up_live_ms / 1e3) / 1e9,
                    "tflops": gu["flops"] / (gate_up_live_ms / 1e3) / 1e12},
        "down": {"ms": st["down"], "alg_bytes": dn["bytes"], "alg_flops": dn["flops"],
                 "gbs": dn["bytes"] / (st["down"] / 1e3) / 1e9,
                 "tflops": dn["flops"] / (st["down"] / 1e3) / 1e12},
        "expert_weight_gbs": (gu["weight_bytes"] + dn["weight_bytes"]) /
                             ((st["gate_up"] + st["down"]) / 1e3) / 1e9,
    }
    return res, layer, cfg


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def read_traffic(kernel_tag):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was taken on the
    current GEMM source (else None)."""
    path = os.path.join(PROFILES, f"{kernel_tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path, encoding="utf-8"):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256") != gemm_source_sha256():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, layer, min_seconds):
    """The float64 oracle, unmodified, on the same batch (host copies), repeated to >= min_seconds."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as O

    f32 = lambda t: None if t is None else t.detach().to("cpu", torch.float32).numpy()
    x = f32(layer["x"])
    wr = f32(layer["w_router"])
    wgu = f32(layer["w_gate_up"])
    wd = f32(layer["w_down"])
    bias = f32(layer["logit_bias"])
    kw = {}
    if cfg.F_shared:
        kw = {"ws_gate_up": f32(layer["ws_gate_up"]), "ws_down": f32(layer["ws_down"]),
              "w_shared_gate": f32(layer["w_shared_gate"])}
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    passes, tokens = 0, 0
    t0 = time.perf_counter()
    while True:
        O.moe_forward(x, wr, wgu, wd, cfg.K, cfg.scoring, logit_bias=bias, **kw)
        passes += 1
        tokens += cfg.T
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full {cfg.T}-token batch of the {cfg.name} layer, {passes} pass(es), "
                      f"{el:.1f} s, float64 NumPy oracle",
            "seconds": el}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this build measures one GPU only "
              "(no sharding or collectives are built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from mixture_experts_layer_renorm_amd import costmodel
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    hip = HipEvents()

    main_res, layer, cfg = run_workload(args.workload, args.steps, args.warmup,
                                        args.atomic_combine, hip)
    sys.stderr.write(json.dumps({"progress": "main workload timed",
                                 "ms_per_step": main_res["ms_per_step"]}) + "\n")
    decode = None
    if not args.no_decode:
        decode, _, _ = run_workload(args.decode_workload, args.steps, args.warmup,
                                    args.atomic_combine, hip)
        sys.stderr.write(json.dumps({"progress": "decode workload timed",
                                     "ms_per_step": decode["ms_per_step"]}) + "\n")
    mfma_bound = None
    if not args.no_mfma_workload and args.mfma_workload != args.workload:
        g, lay, _ = run_workload(args.mfma_workload, args.steps, args.warmup, args.atomic_combine,
                                 hip)
        del lay
        torch.cuda.empty_cache()
        pk = costmodel.MFMA_BF16_PEAK_TFLOPS
        mfma_bound = {
            "workload": args.mfma_workload, "plan": g["plan"], "T": g["T"], "U": g["U"],
            "t_e": g["t_e"], "ms_per_step": g["ms_per_step"], "tokens_per_s": g["tokens_per_s"],
            "gate_up_tflops": g["gate_up"]["tflops"], "gate_up_mfma_frac": g["gate_up"]["tflops"] / pk,
            "down_tflops": g["down"]["tflops"], "down_mfma_frac": g["down"]["tflops"] / pk,
            "layer_tflops": g["layer_tflops"], "layer_mfma_frac": g["layer_tflops"] / pk,
            "stage_ms": g["stage_ms"]}
        sys.stderr.write(json.dumps({"progress": f"{args.mfma_workload} timed",
                                     "ms_per_step": g["ms_per_step"]}) + "\n")
    granularity = None
    if not args.no_granularity:
        from mixture_experts_layer_renorm_amd.synth import GRANULARITY_PAIR
        granularity = {}
        for name in GRANULARITY_PAIR:
            g, lay, _ = run_workload(name, args.steps, args.warmup, args.atomic_combine, hip)
            del lay
            torch.cuda.empty_cache()
            granularity[name] = {
                "T": g["T"], "D": g["D"], "E": g["E"], "K": g["K"], "F": g["F"], "U": g["U"],
                "plan": g["plan"], "ms_per_step": g["ms_per_step"],
                "tokens_per_s": g["tokens_per_s"], "layer_tflops": g["layer_tflops"],
                "gate_up_tflops": g["gate_up"]["tflops"], "down_tflops": g["down"]["tflops"],
                "gate_up_mfma_frac": g["gate_up"]["tflops"] / costmodel.MFMA_BF16_PEAK_TFLOPS,
                "stage_ms": g["stage_ms"]}
            sys.stderr.write(json.dumps({"progress": f"{name} timed",
                                         "ms_per_step": g["ms_per_step"]}) + "\n")
    if args.copy_calibration:
        copy_calibration()

    gu = main_res["gate_up"]
    traffic = read_traffic(f"gate_up_{args.workload}")
    grouped = main_res["plan"].split("grouped gate_up/down: ")[1].split(";")[0]
    roofline = {"kernel": f"routed gate_up, {grouped} tiles, fused SiLU*up epilogue",
                "bound": "hbm", "achieved": gu["gbs"], "peak": costmodel.HBM_PEAK_GBS,
                "unit": "GB/s", "frac": gu["gbs"] / costmodel.HBM_PEAK_GBS, "traffic": traffic,
                "alg_bytes_per_launch": gu["alg_bytes"], "avg_launch_ms": gu["ms"],
                "mfma_tflops": gu["tflops"],
                "mfma_frac": gu["tflops"] / costmodel.MFMA_BF16_PEAK_TFLOPS}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, layer, args.cpu_min_seconds)
    del layer
    torch.cuda.empty_cache()

    line = {
        "metric": "MoE-layer tokens/s; grouped-GEMM TFLOP/s (% MFMA peak); decode HBM GB/s",
        "value": main_res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0, std) inputs and random-init weights of the layer's shapes)",
        "config": {"workload": f"{args.workload}: {cfg.description}", "T": cfg.T, "D": cfg.D,
                   "E": cfg.E, "K": cfg.K, "F": cfg.F, "combine":
                   "fused fp32 atomics" if args.atomic_combine else "gather (deterministic)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "grouped_gemm": {"gate_up_tflops": gu["tflops"],
                         "gate_up_mfma_frac": gu["tflops"] / costmodel.MFMA_BF16_PEAK_TFLOPS,
                         "down_tflops": main_res["down"]["tflops"],
                         "down_mfma_frac": main_res["down"]["tflops"] /
                                           costmodel.MFMA_BF16_PEAK_TFLOPS},
        "main": main_res,
        "decode": None if decode is None else {
            "workload": args.decode_workload, "tokens_per_s": decode["tokens_per_s"],
            "ms_per_step": decode["ms_per_step"], "U": decode["U"],
            "expert_weight_gbs": decode["expert_weight_gbs"],
            "expert_weight_hbm_frac": decode["expert_weight_gbs"] / costmodel.HBM_PEAK_GBS,
            "stage_ms": decode["stage_ms"]},
        "mfma_bound": mfma_bound,
        "granularity": granularity,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
