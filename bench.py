#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

One step = one moe_forward call (router GEMM, top-K, dispatch, grouped gate_up GEMM with fused
SiLU*up, shared expert, grouped down GEMM, weighted gather combine with the final cast) over one
synthetic batch already resident in HBM.

Headline workload: the DeepSeek-style sigmoid layer (T=16384, D=4096, E=256, top-6, F=2048, one
ungated shared expert F=2048, bf16), the largest of the layer configurations that fits one GPU.
Its dominant kernel, the routed gate_up GEMM, is bound by the matrix cores, so the roofline
object is TFLOP/s against the dense bf16 peak.  Every other configuration (tiny fp32, the
35B-A3B-shaped decode and prefill batches, the 397B-A17B-shaped layer, the skewed and fully
concentrated layers, the granularity pair) gets its own entry under "workloads".

Timing protocol, per workload: W warm-up steps, then K timed steps.  Before each step a 1 GiB
buffer is read once (evicts the L2s and the 256 MiB MALL, so weights come from HBM every step,
as they would between the layers of a model; a read leaves no dirty lines whose write-back
would fall into the next step); HIP events on the launch stream bracket each step, and
ms_per_step is the median over the K steps.  An event recorded between two launches idles the
GPU for ~5 us, so the routed gate_up's duration is taken from a second pass of K steps with
events right around that launch, and the per-stage times from a third.  The machine
peaks are measured live (a streaming read and a register-only MFMA loop) and reported beside
the published ones.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload ds_sigmoid]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
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

ALL_WORKLOADS = ("ds_sigmoid", "tiny", "a3b_decode", "a3b_prefill", "a17b", "skew", "skew_conc",
                 "gran_e128", "gran_e64")
FLUSH_BYTES = 1 << 30


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
    ap.add_argument("--workload", default="ds_sigmoid", help="headline workload")
    ap.add_argument("--workloads", default="all",
                    help="comma-separated list of the other workloads to time, 'all' or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-chunk", type=int, default=1024,
                    help="tokens per oracle call in the CPU baseline")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not read 1 GiB between steps (weights may stay in the MALL)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured machine peaks")
    ap.add_argument("--gemm-kernel", default="auto", choices=("auto", "tile32", "tile256", "mfma"),
                    help="force the grouped GEMM (moe_problem.gemm_kernel), for tuning")
    ap.add_argument("--dispatch-kernel", default="auto",
                    choices=("auto", "one_workgroup", "multi"),
                    help="force the dispatch kernel (moe_problem.dispatch_kernel), for tuning")
    ap.add_argument("--atomic-combine", action="store_true",
                    help="time the fused fp32-atomic combine instead of the default gather")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one 1 GiB device-to-device copy (for PMC scaling)")
    return ap.parse_args()


def progress(**kw):
    sys.stderr.write(json.dumps({"progress": kw}) + "\n")
    sys.stderr.flush()


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (same SONAME)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def record(self, e: int, stream: int) -> None:
        if self.lib.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e: int) -> None:
        self.lib.hipEventDestroy(e)


def measure_peaks(hip, reps=5):
    """Measured HBM read rate and bf16 MFMA rate on this GPU (median of `reps` timed launches,
    each long enough for the clock to settle under the load)."""
    import torch
    from mixture_experts_layer_renorm_amd import abi
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = 4 << 30  # far beyond the 256 MiB MALL
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(65536, dtype=torch.float32, device="cuda")
    waves, iters = 2048, 40000  # 8 waves per CU; 10.7 TFLOP per launch (about 5 ms)
    mfma_flops = waves * iters * 4 * 32768
    res = {}
    for name, launch, work in (
            ("hbm_read", lambda: abi.moe_peak_hbm_read(buf, sink), nbytes),
            ("mfma_bf16", lambda: abi.moe_peak_mfma_bf16(waves, iters, sink), mfma_flops)):
        launch()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a, b = hip.create(), hip.create()
            hip.record(a, stream)
            launch()
            hip.record(b, stream)
            torch.cuda.synchronize()
            times.append(hip.elapsed_ms(a, b))
            hip.destroy(a)
            hip.destroy(b)
        ms = statistics.median(times)
        res[name] = (ms, work / (ms / 1e3))
    del buf, sink
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": res["hbm_read"][1] / 1e9, "hbm_read_bytes": nbytes,
            "hbm_read_ms": res["hbm_read"][0],
            "mfma_bf16_tflops": res["mfma_bf16"][1] / 1e12, "mfma_bf16_ms": res["mfma_bf16"][0],
            "mfma_loop": f"{waves} waves x {iters} x 4 v_mfma_f32_32x32x16_bf16 on registers"}


def kernel_roofline(flops, nbytes, ms, mfma_peak_tflops, costmodel):
    """Achieved rate of one kernel against the roofline its intensity puts it under (the
    matrix-core peak of its dtype, or HBM)."""
    s = ms / 1e3
    tflops = flops / s / 1e12
    gbs = nbytes / s / 1e9
    ridge = mfma_peak_tflops * 1e12 / (costmodel.HBM_PEAK_GBS * 1e9)
    bound = "mfma" if flops / nbytes >= ridge else "hbm"
    frac = tflops / mfma_peak_tflops if bound == "mfma" else gbs / costmodel.HBM_PEAK_GBS
    return {"ms": ms, "alg_flops": flops, "alg_bytes": nbytes, "tflops": tflops, "gbs": gbs,
            "bound": bound, "frac": frac, "mfma_peak_tflops": mfma_peak_tflops}


def run_workload(name, steps, warmup, atomic_combine, flush, hip, gemm_kernel="auto",
                 dispatch_kernel="auto"):
    import torch
    from mixture_experts_layer_renorm_amd import abi, costmodel
    from mixture_experts_layer_renorm_amd.synth import CONFIGS, make_layer

    cfg = CONFIGS[name]
    dev = "cuda"
    layer = make_layer(cfg, device=dev, seed=0)
    p = abi.make_problem(T=cfg.T, D=cfg.D, E=cfg.E, K=cfg.K, F=cfg.F, F_shared=cfg.F_shared,
                         shared_gated=cfg.shared_gated, scoring=cfg.scoring, dtype=cfg.torch_dtype,
                         atomic_combine=atomic_combine, gemm_kernel=gemm_kernel,
                         dispatch_kernel=dispatch_kernel)
    weights = {"w_router": layer["w_router"], "logit_bias": layer["logit_bias"],
               "w_gate_up": layer["w_gate_up"], "w_down": layer["w_down"],
               "ws_gate_up": layer["ws_gate_up"], "ws_down": layer["ws_down"],
               "ws_gate": layer["w_shared_gate"]}
    routing = abi.alloc_routing(p, dev, logits=False)
    out = torch.empty((cfg.T, cfg.D), dtype=cfg.torch_dtype, device=dev)
    ws = abi.alloc_workspace(p, dev)
    x = layer["x"]
    stream = torch.cuda.current_stream().cuda_stream

    def do_flush(k):
        if flush is not None:
            abi.moe_peak_hbm_read(flush[0], flush[1])

    for k in range(warmup):
        do_flush(k)
        abi.moe_forward(p, x, weights, routing, out, ws)
    torch.cuda.synchronize()

    # Timed steps: events on the launch stream at each step's start and end only.  Every event
    # recorded between two launches leaves the GPU idle for ~5 us (kernel traces show the gap),
    # so the routed gate_up's duration comes from a second pass of the same steps with events
    # right around that launch (moe_forward_timed records them between the launches), and the
    # per-stage breakdown from a third with events between all stages.
    n_ev = abi.MOE_STAGE_COUNT + 1
    G = abi.MOE_STAGE_GATE_UP

    def timed_pass(slots):
        ev = [[hip.create() for _ in slots] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            do_flush(k)
            e = [None] * n_ev
            for slot, h in zip(slots, ev[k]):
                e[slot] = h
            abi.moe_forward_timed(p, x, weights, routing, out, ws, e)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [[hip.elapsed_ms(row[i], row[i + 1]) for i in range(len(slots) - 1)] for row in ev]
        for row in ev:
            for h in row:
                hip.destroy(h)
        return ms, wall

    ms_a, wall_a = timed_pass([0, n_ev - 1])
    step_ms = [m[0] for m in ms_a]
    ms_b, _ = timed_pass([0, G, G + 1, n_ev - 1])
    gu_ms = [m[1] for m in ms_b]
    step_ms_kernel_events = [sum(m) for m in ms_b]

    # Per-stage breakdown from a second pass with events between all stages (each boundary
    # costs a few microseconds, so these stages add up to slightly more than the plain step).
    events = [[hip.create() for _ in range(n_ev)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        do_flush(k)
        abi.moe_forward_timed(p, x, weights, routing, out, ws, events[k])
    torch.cuda.synchronize()
    stage_ms = {}
    for i, sname in enumerate(abi.MOE_STAGE_NAMES):
        stage_ms[sname] = statistics.median(
            hip.elapsed_ms(events[k][i], events[k][i + 1]) for k in range(steps))
    for row in events:
        for h in row:
            hip.destroy(h)

    counts = routing["expert_counts"].cpu()
    U = int((counts > 0).sum())
    nz = counts[counts > 0].float()
    ms = statistics.median(step_ms)
    dts = cfg.dtype
    gu = costmodel.gate_up(cfg.T, cfg.D, cfg.F, cfg.K, U, dts)
    dn = costmodel.down(cfg.T, cfg.D, cfg.F, cfg.K, U, dts, dts)
    lay = costmodel.layer(cfg.T, cfg.D, cfg.E, cfg.K, cfg.F, U, cfg.F_shared, cfg.shared_gated,
                          dts, dts)
    mfma_peak = (costmodel.MFMA_BF16_PEAK_TFLOPS if dts == "bf16"
                 else costmodel.MFMA_FP32_PEAK_TFLOPS) * 1e12
    t_mfma = lay["flops"] / mfma_peak
    t_hbm = lay["bytes"] / (costmodel.HBM_PEAK_GBS * 1e9)
    res = {
        "workload": name, "description": cfg.description, "plan": abi.describe_plan(p),
        "T": cfg.T, "D": cfg.D, "E": cfg.E, "K": cfg.K, "F": cfg.F, "F_shared": cfg.F_shared,
        "scoring": cfg.scoring, "dtype": dts,
        "ms_per_step": ms, "ms_per_step_mean": statistics.fmean(step_ms),
        "ms_per_step_min": min(step_ms), "ms_per_step_max": max(step_ms),
        "wall_ms_per_step_incl_flush": wall_a * 1e3 / steps,
        "ms_per_step_with_gate_up_events": statistics.median(step_ms_kernel_events),
        "tokens_per_s": cfg.T / (ms / 1e3),
        "U": U, "assignments": cfg.T * cfg.K,
        "t_e": {"min": int(nz.min()), "median": float(nz.median()), "max": int(nz.max())},
        "layer": {"alg_flops": lay["flops"], "alg_bytes": lay["bytes"],
                  "tflops": lay["flops"] / (ms / 1e3) / 1e12,
                  "gbs": lay["bytes"] / (ms / 1e3) / 1e9,
                  "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                  "roofline_ms": max(t_mfma, t_hbm) * 1e3,
                  "roofline_frac": max(t_mfma, t_hbm) / (ms / 1e3)},
        "gate_up": kernel_roofline(gu["flops"], gu["bytes"], statistics.median(gu_ms),
                                   mfma_peak / 1e12, costmodel),
        "down": kernel_roofline(dn["flops"], dn["bytes"], stage_ms["down"], mfma_peak / 1e12,
                                costmodel),
        "expert_weight_gbs": (gu["weight_bytes"] + dn["weight_bytes"]) /
                             ((statistics.median(gu_ms) + stage_ms["down"]) / 1e3) / 1e9,
        "stage_ms": stage_ms,
    }
    res["expert_weight_hbm_frac"] = res["expert_weight_gbs"] / costmodel.HBM_PEAK_GBS
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


def cpu_baseline(cfg, layer, min_seconds, chunk):
    """The float64 oracle, unmodified, on consecutive chunks of the same batch (host copies of
    the tokens; weights upcast expert by expert inside each call, as the oracle does), until at
    least min_seconds have passed."""
    import numpy as np  # noqa: F401
    import torch
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as O

    class Lazy:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return self.t[e].detach().to("cpu", torch.float64).numpy()

    f64 = lambda t: None if t is None else t.detach().to("cpu", torch.float64).numpy()
    wr = f64(layer["w_router"])
    bias = f64(layer["logit_bias"])
    kw = {}
    if cfg.F_shared:
        kw = {"ws_gate_up": f64(layer["ws_gate_up"]), "ws_down": f64(layer["ws_down"]),
              "w_shared_gate": f64(layer["w_shared_gate"])}
    info = threadpool_info()
    blas = [i for i in info if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    vendor = ",".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in blas})) or "?"
    tokens, calls = 0, 0
    t0 = time.perf_counter()
    while tokens < cfg.T:
        n = min(chunk, cfg.T - tokens)
        x = f64(layer["x"][tokens:tokens + n])
        O.moe_forward(x, wr, Lazy(layer["w_gate_up"]), Lazy(layer["w_down"]), cfg.K, cfg.scoring,
                      logit_bias=bias, **kw)
        tokens += n
        calls += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"tokens [0, {tokens}) of the {cfg.T}-token {cfg.name} batch in {calls} "
                      f"oracle call(s) of {chunk} tokens (each upcasts every hit expert's "
                      f"weights to float64), {el:.1f} s, float64 NumPy oracle",
            "seconds": el, "blas": vendor, "blas_threads": int(threads),
            "host_cpus_available": len(os.sched_getaffinity(0))}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this benchmark measures one GPU only "
              "(no sharding or collectives are built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from mixture_experts_layer_renorm_amd import costmodel
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    hip = HipEvents()
    if args.workloads == "all":
        others = [w for w in ALL_WORKLOADS if w != args.workload]
    elif args.workloads == "none":
        others = []
    else:
        others = [w for w in args.workloads.split(",") if w and w != args.workload]

    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks(hip)
        progress(step="peaks", **{k: v for k, v in peaks.items() if isinstance(v, float)})
    flush = None
    if not args.no_flush:
        flush = (torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda"),
                 torch.empty(2048, dtype=torch.float32, device="cuda"))

    main_res, layer, cfg = run_workload(args.workload, args.steps, args.warmup,
                                        args.atomic_combine, flush, hip, args.gemm_kernel,
                                        args.dispatch_kernel)
    progress(step=args.workload, ms_per_step=main_res["ms_per_step"])
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, layer, args.cpu_min_seconds, args.cpu_chunk)
        progress(step="cpu_baseline", tokens_per_s=cpu["value"])
    del layer
    torch.cuda.empty_cache()

    workloads = {args.workload: main_res}
    for name in others:
        r, lay, _ = run_workload(name, args.steps, args.warmup, args.atomic_combine, flush, hip,
                                 args.gemm_kernel, args.dispatch_kernel)
        del lay
        torch.cuda.empty_cache()
        workloads[name] = r
        progress(step=name, ms_per_step=r["ms_per_step"])
    if args.copy_calibration:
        copy_calibration()

    gu = main_res["gate_up"]
    grouped = main_res["plan"].split("grouped gate_up/down: ")[1].split(";")[0]
    if gu["bound"] == "mfma":
        achieved, peak, unit = gu["tflops"], costmodel.MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        measured_peak = peaks["mfma_bf16_tflops"] if peaks else None
    else:
        achieved, peak, unit = gu["gbs"], costmodel.HBM_PEAK_GBS, "GB/s"
        measured_peak = peaks["hbm_read_gbs"] if peaks else None
    roofline = {"kernel": f"routed gate_up ({grouped} tiles, fused SiLU*up epilogue)",
                "bound": gu["bound"], "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": read_traffic(f"gate_up_{args.workload}"),
                "alg_flops_per_launch": gu["alg_flops"], "alg_bytes_per_launch": gu["alg_bytes"],
                "avg_launch_ms": gu["ms"],
                "launch_ms_statistic": ("median of HIP events recorded right around the launch "
                                        "in a second pass of the timed steps"),
                "measured_peak": measured_peak,
                "frac_of_measured_peak": achieved / measured_peak if measured_peak else None}

    summary = {n: {"ms_per_step": r["ms_per_step"], "tokens_per_s": r["tokens_per_s"],
                   "layer_bound": r["layer"]["bound"],
                   "layer_roofline_frac": r["layer"]["roofline_frac"],
                   "gate_up_bound": r["gate_up"]["bound"], "gate_up_frac": r["gate_up"]["frac"],
                   "gate_up_tflops": r["gate_up"]["tflops"], "gate_up_gbs": r["gate_up"]["gbs"],
                   "expert_weight_hbm_frac": r["expert_weight_hbm_frac"]}
               for n, r in workloads.items()}
    line = {
        "metric": "MoE-layer tokens/s; grouped-GEMM TFLOP/s (% MFMA peak); decode HBM GB/s",
        "value": main_res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0, std) inputs and random-init weights of the layer's shapes)",
        "config": {"workload": f"{args.workload}: {cfg.description}", "T": cfg.T, "D": cfg.D,
                   "E": cfg.E, "K": cfg.K, "F": cfg.F, "F_shared": cfg.F_shared,
                   "scoring": cfg.scoring,
                   "combine": "fused fp32 atomics" if args.atomic_combine
                   else "gather (deterministic)",
                   "flush_between_steps": None if args.no_flush else "1 GiB read"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "peaks": {"spec_hbm_gbs": costmodel.HBM_PEAK_GBS,
                  "spec_mfma_bf16_tflops": costmodel.MFMA_BF16_PEAK_TFLOPS,
                  "measured": peaks},
        "summary": summary,
        "workloads": workloads,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
