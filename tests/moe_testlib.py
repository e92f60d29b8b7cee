"""Shared helpers for the test-suite: tensor <-> numpy conversion, lazy expert access for the
oracle, tolerances and the layer-to-argument plumbing.  Holds none of the method's arithmetic.
"""

from __future__ import annotations

import numpy as np
import torch

from mixture_experts_layer_renorm_amd import abi
from mixture_experts_layer_renorm_amd.synth import LayerConfig

# Tolerances (max-abs error over the output, relative to the oracle output's RMS).  The bf16
# bound is applied to the layer's fp32 result; a bf16 output may additionally differ by its own
# rounding (half a bf16 ulp of the value), which is checked separately.
TOL_BF16 = 2e-2
TOL_F32 = 1e-4
TOL_ROUTING_W = 1e-6


def f64(t) -> np.ndarray:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def i64(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


class LazyRows:
    """Indexable view of a [E, ...] tensor that converts one expert to float64 on demand."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, e):
        return f64(self.t[e])

    def __len__(self):
        return self.t.shape[0]


def problem_for(cfg: LayerConfig, T=None, out_dtype=None, atomic_combine=False,
                renormalize=True, gemm_kernel="auto", dispatch_kernel="auto"):
    dt = cfg.torch_dtype
    return abi.make_problem(T=cfg.T if T is None else T, D=cfg.D, E=cfg.E, K=cfg.K, F=cfg.F,
                            F_shared=cfg.F_shared, shared_gated=cfg.shared_gated,
                            scoring=cfg.scoring, dtype=dt,
                            out_dtype=dt if out_dtype is None else out_dtype,
                            atomic_combine=atomic_combine, renormalize=renormalize,
                            gemm_kernel=gemm_kernel, dispatch_kernel=dispatch_kernel)


def weights_for(layer) -> dict:
    return {"w_router": layer["w_router"], "logit_bias": layer["logit_bias"],
            "w_gate_up": layer["w_gate_up"], "w_down": layer["w_down"],
            "ws_gate_up": layer["ws_gate_up"], "ws_down": layer["ws_down"],
            "ws_gate": layer["w_shared_gate"]}


def oracle_args(cfg: LayerConfig, layer, token_ids=None):
    """Positional and keyword arguments for oracle.moe_forward on (a subset of) the layer."""
    x = layer["x"] if token_ids is None else layer["x"][token_ids]
    kw = {"scoring": cfg.scoring, "logit_bias": f64(layer["logit_bias"])}
    if cfg.F_shared:
        kw["ws_gate_up"] = f64(layer["ws_gate_up"])
        kw["ws_down"] = f64(layer["ws_down"])
        kw["w_shared_gate"] = f64(layer["w_shared_gate"]) if cfg.shared_gated else None
    return (f64(x), f64(layer["w_router"]), LazyRows(layer["w_gate_up"]),
            LazyRows(layer["w_down"]), cfg.K), kw


def rel_max_err(got, want) -> float:
    got, want = f64(got), f64(want)
    rms = float(np.sqrt(np.mean(want ** 2)))
    return float(np.max(np.abs(got - want))) / rms


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |v| (the largest error of a round-to-nearest bf16 value)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, np.finfo(np.float32).tiny)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))
