"""Seeded synthetic MoE layers: shapes, value distributions and the draw order.

This module holds no arithmetic of the method (no routing, no expert math).  It only draws
random tensors, so that the HIP path and the CPU oracle can be fed byte-identical inputs.

Recipe (every workload): one ``torch.Generator`` on the drawing device, seeded with ``seed``
(0 by default).  Tensors are drawn in the fixed order x, W_r, w_s, W_gate_up (expert by
expert), W_down (expert by expert), Ws_gate_up, Ws_down.  Each is drawn in float32 as
N(0, 1) * std and rounded to the layer dtype (round-to-nearest-even).  "N(0, s)" is read as
standard deviation s.  The skewed workloads add a fixed float32 logit bias on the hot experts
{0, 32, 64, ..., 224}.  Different devices give different (but equally seeded) streams; the
oracle always receives a copy of the tensors the GPU uses.

The shapes follow the pages' models: the 35B-A3B-shaped layer of "S23-J10" §2.1, the
397B-A17B-shaped layer of "MoE" §1.1, and the DeepSeek-style sigmoid layer of "S23-J10" §4
(V4-Flash expert 3·4096·2048, top-6, one shared expert) with the sigmoid gating of
"1.6 混合专家（MoE）" §四.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

SOFTMAX = "softmax"
SIGMOID = "sigmoid"


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    D: int
    E: int
    K: int
    F: int
    F_shared: int = 0
    shared_gated: bool = False
    scoring: str = SOFTMAX
    dtype: str = "bf16"               # "bf16" or "f32"
    std_x: float = 1.0
    std_router: float = 0.02
    std_shared_gate: float = 0.02
    std_expert: float = 0.02
    hot_bias: float = 0.0             # logit bias on the hot experts (0 = no bias tensor)
    hot_stride: int = 32              # hot experts are 0, stride, 2*stride, ... (8 of them)
    n_hot: int = 8
    description: str = ""

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def A(self) -> int:
        return self.T * self.K


_RSQRT_2048 = 1.0 / math.sqrt(2048.0)

CONFIGS: Dict[str, LayerConfig] = {
    "tiny": LayerConfig(
        "tiny", T=64, D=256, E=8, K=2, F=128, dtype="f32", std_router=0.02,
        description="tiny fp32 layer: T=64, D=256, E=8, top-2, F=128, softmax, no shared expert"),
    "a3b_decode": LayerConfig(
        "a3b_decode", T=64, D=2048, E=256, K=8, F=512, std_router=_RSQRT_2048,
        description="35B-A3B-shaped bf16 layer, decode batch T=64 (D=2048, E=256, top-8, F=512)"),
    "a3b_prefill": LayerConfig(
        "a3b_prefill", T=4096, D=2048, E=256, K=8, F=512, std_router=_RSQRT_2048,
        description="35B-A3B-shaped bf16 layer, prefill batch T=4096 (D=2048, E=256, top-8, F=512)"),
    "a17b": LayerConfig(
        "a17b", T=8192, D=4096, E=512, K=10, F=1024, F_shared=1024, shared_gated=True,
        description="397B-A17B-shaped bf16 layer, T=8192 (D=4096, E=512, top-10, F=1024, "
                    "one sigmoid-gated shared expert F=1024)"),
    "skew": LayerConfig(
        "skew", T=4096, D=2048, E=256, K=8, F=512, std_router=_RSQRT_2048, hot_bias=4.0,
        description="skewed routing on the 35B-A3B shapes, T=4096: +4.0 logit bias on 8 hot experts"),
    "skew_conc": LayerConfig(
        "skew_conc", T=4096, D=2048, E=256, K=8, F=512, std_router=_RSQRT_2048, hot_bias=30.0,
        description="fully concentrated routing on the 35B-A3B shapes, T=4096: +30 logit bias "
                    "on 8 hot experts, so every token picks the same 8 (U=8)"),
    "ds_sigmoid": LayerConfig(
        "ds_sigmoid", T=16384, D=4096, E=256, K=6, F=2048, F_shared=2048, shared_gated=False,
        scoring=SIGMOID,
        description="DeepSeek-style sigmoid-affinity bf16 layer, T=16384 (D=4096, E=256, top-6, "
                    "F=2048, one ungated shared expert F=2048)"),
    # granularity pair ("S23-J10" §4.1): halving E and K while doubling F keeps the routed
    # parameters (3·E·D·F) and the per-token expert FLOPs (6·K·D·F) equal; only the GEMM shapes
    # and the read pattern change.  D = 4096 is a stated choice (the page gives none).
    "gran_e128": LayerConfig(
        "gran_e128", T=4096, D=4096, E=128, K=8, F=1536,
        description="granularity pair, fine: 128 experts x F=1536, top-8 (D=4096, T=4096)"),
    "gran_e64": LayerConfig(
        "gran_e64", T=4096, D=4096, E=64, K=4, F=3072,
        description="granularity pair, coarse: 64 experts x F=3072, top-4 (D=4096, T=4096)"),
}

GRANULARITY_PAIR = ("gran_e128", "gran_e64")


def hot_experts(cfg: LayerConfig):
    return [i * cfg.hot_stride for i in range(cfg.n_hot) if i * cfg.hot_stride < cfg.E]


def _draw(shape, std, gen, device, dtype):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_layer(cfg: LayerConfig, device="cpu", seed: int = 0,
               T: Optional[int] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one seeded layer (inputs and weights) on ``device``.

    ``T`` overrides the token count (smaller parity cases reuse a workload's weights' recipe).
    Returns a dict of tensors; absent optional tensors are None.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = cfg.torch_dtype
    T = cfg.T if T is None else T
    D, E, F, Fs = cfg.D, cfg.E, cfg.F, cfg.F_shared

    x = _draw((T, D), cfg.std_x, gen, device, dt)
    w_router = _draw((E, D), cfg.std_router, gen, device, dt)
    w_shared_gate = (_draw((1, D), cfg.std_shared_gate, gen, device, dt)
                     if (Fs > 0 and cfg.shared_gated) else None)
    w_gate_up = torch.empty((E, 2 * F, D), dtype=dt, device=device)
    for e in range(E):
        w_gate_up[e] = _draw((2 * F, D), cfg.std_expert, gen, device, dt)
    w_down = torch.empty((E, D, F), dtype=dt, device=device)
    for e in range(E):
        w_down[e] = _draw((D, F), cfg.std_expert, gen, device, dt)
    ws_gate_up = _draw((2 * Fs, D), cfg.std_expert, gen, device, dt) if Fs > 0 else None
    ws_down = _draw((D, Fs), cfg.std_expert, gen, device, dt) if Fs > 0 else None
    logit_bias = None
    if cfg.hot_bias != 0.0:
        logit_bias = torch.zeros(E, dtype=torch.float32, device=device)
        logit_bias[hot_experts(cfg)] = cfg.hot_bias
    return {"x": x, "w_router": w_router, "w_shared_gate": w_shared_gate,
            "w_gate_up": w_gate_up, "w_down": w_down, "ws_gate_up": ws_gate_up,
            "ws_down": ws_down, "logit_bias": logit_bias}
