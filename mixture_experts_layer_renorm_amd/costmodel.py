"""Algorithmic work of the layer's kernels, for roofline reporting.

"Algorithmic" means what the method must move or compute, not what the kernels happen to do:
padding, re-reads and intermediate scratch traffic are not counted.  The weight term follows
the read model of "S23-J10" §3: every distinct expert hit by the batch is read once,
R = b_W·N_e·U, with N_e = 3·D·F ("S23-J10" §2).  FLOPs: 2 per multiply-add.

Per-kernel units (multiplied by the units one launch processes):
  gate_up : per hit expert 2F·D·b weight bytes; per token D·b input bytes (the row is needed
            once however many experts use it); per assignment F·b output bytes and 4·D·F FLOP.
  down    : per hit expert D·F·b weight bytes; per assignment F·b input bytes and 2·D·F FLOP;
            per token D·b_out output bytes.
  router  : E·D·b weight bytes, T·D·b input bytes, T·E·4 logit bytes; 2·T·D·E FLOP.
  shared  : 3·D·F_s·b weight bytes, T·D·b input, T·D·b_out output; 6·T·D·F_s FLOP.
"""

from __future__ import annotations

from typing import Dict

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix, published
MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X fp32 matrix, published


def _b(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def gate_up(T: int, D: int, F: int, K: int, U: int, dtype: str = "bf16") -> Dict[str, float]:
    b = _b(dtype)
    A = T * K
    return {"bytes": U * 2 * F * D * b + T * D * b + A * F * b, "flops": 4.0 * A * D * F,
            "weight_bytes": U * 2 * F * D * b}


def down(T: int, D: int, F: int, K: int, U: int, dtype: str = "bf16",
         out_dtype: str = "bf16") -> Dict[str, float]:
    b = _b(dtype)
    A = T * K
    return {"bytes": U * D * F * b + A * F * b + T * D * _b(out_dtype), "flops": 2.0 * A * D * F,
            "weight_bytes": U * D * F * b}


def router(T: int, D: int, E: int, dtype: str = "bf16", gated_shared: bool = False):
    b = _b(dtype)
    n = E + (1 if gated_shared else 0)
    return {"bytes": n * D * b + T * D * b + T * E * 4, "flops": 2.0 * T * D * n}


def shared(T: int, D: int, Fs: int, dtype: str = "bf16", out_dtype: str = "bf16"):
    b = _b(dtype)
    if Fs == 0:
        return {"bytes": 0, "flops": 0.0}
    return {"bytes": 3 * D * Fs * b + T * D * b + T * D * _b(out_dtype), "flops": 6.0 * T * D * Fs}


def layer(T: int, D: int, E: int, K: int, F: int, U: int, Fs: int = 0, gated_shared=False,
          dtype: str = "bf16", out_dtype: str = "bf16") -> Dict[str, float]:
    """Whole-layer algorithmic FLOPs and HBM bytes: weights of the hit experts, shared expert
    and router read once; x read once; the output written once; routing tables (T·K ids and
    weights) written once."""
    b = _b(dtype)
    flops = (router(T, D, E, dtype, gated_shared)["flops"] + 6.0 * T * K * D * F +
             shared(T, D, Fs, dtype)["flops"])
    nbytes = (3 * D * F * U * b + 3 * D * Fs * b + (E + (1 if gated_shared else 0)) * D * b +
              T * D * b + T * D * _b(out_dtype) + 8 * T * K)
    return {"flops": flops, "bytes": nbytes}
