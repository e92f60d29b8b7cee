"""Thin ctypes binding to libmoe.so (the C ABI of include/moe.h).

Every function here only marshals arguments: torch tensors become device pointers, Python
values become the C structs, the current HIP stream is passed along.  All computation happens
in the library's HIP kernels.  torch is used for device memory and streams only.

If libmoe.so has not been built, the first call raises immediately: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_SCORE_SOFTMAX = 0
MOE_SCORE_SIGMOID = 1
MOE_FLAG_ATOMIC_COMBINE = 1
MOE_FLAG_NO_RENORM = 2
MOE_GEMM_AUTO = 0
MOE_GEMM_TILE_32 = 1
MOE_GEMM_TILE_256 = 2
MOE_GEMM_MFMA_256 = 3
MOE_DISPATCH_AUTO = 0
MOE_DISPATCH_ONE_WORKGROUP = 1
MOE_DISPATCH_MULTI = 2
GEMM_KERNELS = {"auto": MOE_GEMM_AUTO, "tile32": MOE_GEMM_TILE_32, "tile256": MOE_GEMM_TILE_256,
                "mfma": MOE_GEMM_MFMA_256}
DISPATCH_KERNELS = {"auto": MOE_DISPATCH_AUTO, "one_workgroup": MOE_DISPATCH_ONE_WORKGROUP,
                    "multi": MOE_DISPATCH_MULTI}

SYMBOLS = ("moe_workspace_size", "moe_route", "moe_route_logits", "moe_dispatch",
           "moe_experts", "moe_combine", "moe_forward", "moe_forward_timed",
           "moe_status_string", "moe_last_error", "moe_describe_plan", "moe_update_select_bias",
           "moe_router_stats", "moe_peak_hbm_read", "moe_peak_mfma_bf16",
           "moe_forward_noalloc")
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_STAGE_NAMES = ("router", "topk", "dispatch", "gate_up", "shared", "down", "final")
MOE_STAGE_COUNT = len(MOE_STAGE_NAMES)
MOE_STAGE_GATE_UP = MOE_STAGE_NAMES.index("gate_up")

_DTYPE_CODE = {torch.float32: MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16}
_DTYPE_OF_CODE = {MOE_DTYPE_F32: torch.float32, MOE_DTYPE_BF16: torch.bfloat16}


class moe_problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("D", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("F", ctypes.c_int32), ("F_shared", ctypes.c_int32),
                ("shared_gated", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("capacity_factor", ctypes.c_float),
                ("min_capacity", ctypes.c_int32), ("gemm_kernel", ctypes.c_int32),
                ("dispatch_kernel", ctypes.c_int32)]


_WEIGHT_FIELDS = ("w_router", "logit_bias", "w_gate_up", "w_down", "ws_gate_up", "ws_down",
                  "ws_gate", "select_bias")
_FP32_WEIGHTS = ("logit_bias", "select_bias")
_ROUTING_FIELDS = ("logits", "topk_idx", "topk_w", "expert_counts", "expert_offsets", "perm",
                   "inv_perm", "shared_gate", "select_keys")


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


class moe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _ROUTING_FIELDS]


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """dlopen libmoe.so and declare the C signatures (no device is touched)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run `python -m mixture_experts_layer_renorm_amd.build`)")
    lib = ctypes.CDLL(path)
    P, vp, sz = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t
    prob = P(moe_problem)
    lib.moe_workspace_size.argtypes = [prob, P(ctypes.c_size_t)]
    lib.moe_route.argtypes = [prob, vp, P(moe_weights), P(moe_routing), vp, sz, vp]
    lib.moe_route_logits.argtypes = [prob, vp, vp, P(moe_routing), vp]
    lib.moe_update_select_bias.argtypes = [prob, vp, vp, ctypes.c_float, vp]
    lib.moe_router_stats.argtypes = [prob, vp, vp, vp, vp, sz, vp]
    lib.moe_dispatch.argtypes = [prob, vp, P(moe_routing), vp, vp, sz, vp]
    lib.moe_experts.argtypes = [prob, vp, vp, P(moe_weights), P(moe_routing), vp, vp, vp, sz, vp]
    lib.moe_combine.argtypes = [prob, vp, P(moe_routing), vp, vp, vp]
    lib.moe_forward.argtypes = [prob, vp, P(moe_weights), P(moe_routing), vp, vp, sz, vp]
    lib.moe_forward_timed.argtypes = [prob, vp, P(moe_weights), P(moe_routing), vp, vp, sz, vp,
                                      P(ctypes.c_void_p)]
    lib.moe_forward_noalloc.argtypes = [prob, vp, P(moe_weights), P(moe_routing), vp, vp]
    for n in ("moe_workspace_size", "moe_route", "moe_route_logits", "moe_dispatch",
              "moe_experts", "moe_combine", "moe_forward", "moe_forward_timed",
              "moe_update_select_bias", "moe_router_stats", "moe_forward_noalloc"):
        getattr(lib, n).restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_describe_plan.argtypes = [prob]
    lib.moe_describe_plan.restype = ctypes.c_char_p
    lib.moe_peak_hbm_read.argtypes = [vp, sz, vp, vp]
    lib.moe_peak_hbm_read.restype = ctypes.c_int
    lib.moe_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    lib.moe_peak_mfma_bf16.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != MOE_OK:
        lib = load_library()
        raise MoEError(status, f"{lib.moe_status_string(status).decode()}: "
                               f"{lib.moe_last_error().decode()}")


def make_problem(T: int, D: int, E: int, K: int, F: int, F_shared: int = 0,
                 shared_gated: bool = False, scoring: str = "softmax", dtype=torch.bfloat16,
                 out_dtype=None, atomic_combine: bool = False,
                 renormalize: bool = True, capacity_factor: float = 0.0,
                 min_capacity: int = 0, gemm_kernel: str = "auto",
                 dispatch_kernel: str = "auto") -> moe_problem:
    if scoring not in ("softmax", "sigmoid"):
        raise ValueError(f"scoring must be 'softmax' or 'sigmoid', got {scoring!r}")
    out_dtype = dtype if out_dtype is None else out_dtype
    flags = (MOE_FLAG_ATOMIC_COMBINE if atomic_combine else 0) | \
            (0 if renormalize else MOE_FLAG_NO_RENORM)
    return moe_problem(T=T, D=D, E=E, K=K, F=F, F_shared=F_shared,
                       shared_gated=1 if shared_gated else 0,
                       scoring=MOE_SCORE_SOFTMAX if scoring == "softmax" else MOE_SCORE_SIGMOID,
                       dtype=_DTYPE_CODE[dtype], out_dtype=_DTYPE_CODE[out_dtype], flags=flags,
                       capacity_factor=capacity_factor, min_capacity=min_capacity,
                       gemm_kernel=GEMM_KERNELS[gemm_kernel],
                       dispatch_kernel=DISPATCH_KERNELS[dispatch_kernel])


def problem_dtype(p: moe_problem) -> torch.dtype:
    return _DTYPE_OF_CODE[p.dtype]


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor or None")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    return t.data_ptr()


def _weights(p: moe_problem, w: Dict[str, Optional[torch.Tensor]]) -> moe_weights:
    dt = problem_dtype(p)
    out = moe_weights()
    for n in _WEIGHT_FIELDS:
        t = w.get(n)
        setattr(out, n, _ptr(t, n, torch.float32 if n in _FP32_WEIGHTS else dt))
    return out


_ROUTING_DTYPES = {"logits": torch.float32, "topk_idx": torch.int32, "topk_w": torch.float32,
                   "expert_counts": torch.int32, "expert_offsets": torch.int32,
                   "perm": torch.int32, "inv_perm": torch.int32, "shared_gate": torch.float32,
                   "select_keys": torch.float32}


def _routing(r: Optional[Dict[str, Optional[torch.Tensor]]]) -> Optional[moe_routing]:
    if r is None:
        return None
    out = moe_routing()
    for n in _ROUTING_FIELDS:
        setattr(out, n, _ptr(r.get(n), n, _ROUTING_DTYPES[n]))
    return out


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    return _ptr(ws, "workspace"), ws.numel() * ws.element_size()


# ---------------------------------------------------------------------- entry points ----

def describe_plan(p: moe_problem) -> str:
    """Names of the kernels moe_forward launches for p (tile shapes, combine mode)."""
    lib = load_library()
    text = lib.moe_describe_plan(ctypes.byref(p)).decode()
    if not text:
        raise MoEError(MOE_ERR_INVALID_ARG, lib.moe_last_error().decode())
    return text


def moe_workspace_size(p: moe_problem) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moe_route(p: moe_problem, x: torch.Tensor, weights: Dict, routing: Dict,
              workspace: torch.Tensor, stream=None) -> None:
    lib = load_library()
    w, r = _weights(p, weights), _routing(routing)
    wp, wb = _ws(workspace)
    _check(lib.moe_route(ctypes.byref(p), _ptr(x, "x", problem_dtype(p)), ctypes.byref(w),
                         ctypes.byref(r), wp, wb, _stream(stream)))


def moe_route_logits(p: moe_problem, logits: torch.Tensor, routing: Dict, stream=None,
                     select_bias: Optional[torch.Tensor] = None) -> None:
    lib = load_library()
    r = _routing(routing)
    _check(lib.moe_route_logits(ctypes.byref(p), _ptr(logits, "logits", torch.float32),
                                _ptr(select_bias, "select_bias", torch.float32),
                                ctypes.byref(r), _stream(stream)))


def moe_router_stats(p: moe_problem, logits: torch.Tensor, expert_counts: torch.Tensor,
                     workspace: torch.Tensor, stream=None) -> Dict[str, torch.Tensor]:
    """Router statistics; returns f [E], P [E] and the scalars aux, z, cv, max_over_mean as
    0-d fp32 device tensors (views of one [2E + 4] buffer)."""
    lib = load_library()
    E = p.E
    out = torch.empty(2 * E + 4, dtype=torch.float32, device=logits.device)
    wp, wb = _ws(workspace)
    _check(lib.moe_router_stats(ctypes.byref(p), _ptr(logits, "logits", torch.float32),
                                _ptr(expert_counts, "expert_counts", torch.int32),
                                _ptr(out, "stats", torch.float32), wp, wb, _stream(stream)))
    return {"f": out[:E], "P": out[E:2 * E], "aux": out[2 * E], "z": out[2 * E + 1],
            "cv": out[2 * E + 2], "max_over_mean": out[2 * E + 3]}


def moe_update_select_bias(p: moe_problem, expert_counts: torch.Tensor,
                           select_bias: torch.Tensor, gamma: float, stream=None) -> None:
    lib = load_library()
    _check(lib.moe_update_select_bias(ctypes.byref(p),
                                      _ptr(expert_counts, "expert_counts", torch.int32),
                                      _ptr(select_bias, "select_bias", torch.float32),
                                      ctypes.c_float(gamma), _stream(stream)))


def moe_dispatch(p: moe_problem, x: Optional[torch.Tensor], routing: Dict,
                 x_perm: Optional[torch.Tensor], workspace: torch.Tensor, stream=None) -> None:
    lib = load_library()
    r = _routing(routing)
    wp, wb = _ws(workspace)
    dt = problem_dtype(p)
    _check(lib.moe_dispatch(ctypes.byref(p), _ptr(x, "x", dt), ctypes.byref(r),
                            _ptr(x_perm, "x_perm", dt), wp, wb, _stream(stream)))


def moe_experts(p: moe_problem, x: Optional[torch.Tensor], x_perm: Optional[torch.Tensor],
                weights: Dict, routing: Dict, y_perm: torch.Tensor,
                y_shared: Optional[torch.Tensor], workspace: torch.Tensor, stream=None) -> None:
    lib = load_library()
    w, r = _weights(p, weights), _routing(routing)
    wp, wb = _ws(workspace)
    dt = problem_dtype(p)
    _check(lib.moe_experts(ctypes.byref(p), _ptr(x, "x", dt), _ptr(x_perm, "x_perm", dt),
                           ctypes.byref(w), ctypes.byref(r),
                           _ptr(y_perm, "y_perm", torch.float32),
                           _ptr(y_shared, "y_shared", torch.float32), wp, wb, _stream(stream)))


def moe_combine(p: moe_problem, y_perm: torch.Tensor, routing: Dict,
                y_shared: Optional[torch.Tensor], out: torch.Tensor, stream=None) -> None:
    lib = load_library()
    r = _routing(routing)
    _check(lib.moe_combine(ctypes.byref(p), _ptr(y_perm, "y_perm", torch.float32),
                           ctypes.byref(r), _ptr(y_shared, "y_shared", torch.float32),
                           _ptr(out, "out", _DTYPE_OF_CODE[p.out_dtype]), _stream(stream)))


def moe_forward(p: moe_problem, x: torch.Tensor, weights: Dict, routing: Optional[Dict],
                out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    lib = load_library()
    w, r = _weights(p, weights), _routing(routing)
    wp, wb = _ws(workspace)
    _check(lib.moe_forward(ctypes.byref(p), _ptr(x, "x", problem_dtype(p)), ctypes.byref(w),
                           ctypes.byref(r) if r is not None else None,
                           _ptr(out, "out", _DTYPE_OF_CODE[p.out_dtype]), wp, wb,
                           _stream(stream)))


def moe_forward_noalloc(p: moe_problem, x: torch.Tensor, weights: Dict, routing: Optional[Dict],
                        out: torch.Tensor, stream=None) -> None:
    """moe_forward on the library's fixed per-GPU scratch: no workspace, no allocation."""
    lib = load_library()
    w, r = _weights(p, weights), _routing(routing)
    _check(lib.moe_forward_noalloc(ctypes.byref(p), _ptr(x, "x", problem_dtype(p)),
                                   ctypes.byref(w), ctypes.byref(r) if r is not None else None,
                                   _ptr(out, "out", _DTYPE_OF_CODE[p.out_dtype]),
                                   _stream(stream)))


def moe_forward_timed(p: moe_problem, x: torch.Tensor, weights: Dict, routing: Optional[Dict],
                      out: torch.Tensor, workspace: torch.Tensor, events, stream=None) -> None:
    """moe_forward recording `events` (MOE_STAGE_COUNT + 1 raw hipEvent_t handles as ints;
    None entries are not recorded)."""
    lib = load_library()
    if len(events) != MOE_STAGE_COUNT + 1:
        raise ValueError(f"need {MOE_STAGE_COUNT + 1} events")
    w, r = _weights(p, weights), _routing(routing)
    wp, wb = _ws(workspace)
    ev = (ctypes.c_void_p * len(events))(*events)
    _check(lib.moe_forward_timed(ctypes.byref(p), _ptr(x, "x", problem_dtype(p)), ctypes.byref(w),
                                 ctypes.byref(r) if r is not None else None,
                                 _ptr(out, "out", _DTYPE_OF_CODE[p.out_dtype]), wp, wb,
                                 _stream(stream), ev))


def moe_peak_hbm_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Stream-read all of `buf` (a multiple of 64 KiB) once; sink: >= 2048 fp32."""
    lib = load_library()
    if sink.numel() < 2048:
        raise ValueError("sink must hold 2048 floats")
    st = lib.moe_peak_hbm_read(_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                               _ptr(sink, "sink", torch.float32), _stream(stream))
    if st != MOE_OK:
        raise MoEError(st, lib.moe_status_string(st).decode())


def moe_peak_mfma_bf16(waves: int, iters: int, sink: torch.Tensor, stream=None) -> None:
    """waves * iters * 4 bf16 MFMAs of 32x32x16 on registers; sink: >= waves fp32."""
    lib = load_library()
    if sink.numel() < waves:
        raise ValueError("sink must hold one float per wave")
    st = lib.moe_peak_mfma_bf16(waves, iters, _ptr(sink, "sink", torch.float32), _stream(stream))
    if st != MOE_OK:
        raise MoEError(st, lib.moe_status_string(st).decode())


# ------------------------------------------------------------- allocation helpers ----

def alloc_workspace(p: moe_problem, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_workspace_size(p), 16), dtype=torch.uint8, device=device)


def alloc_routing(p: moe_problem, device="cuda", logits: bool = True,
                  select_keys: bool = False) -> Dict[str, torch.Tensor]:
    T, E, K = p.T, p.E, p.K
    i32, f32 = torch.int32, torch.float32
    r = {"topk_idx": torch.empty((T, K), dtype=i32, device=device),
         "topk_w": torch.empty((T, K), dtype=f32, device=device),
         "expert_counts": torch.empty(E, dtype=i32, device=device),
         "expert_offsets": torch.empty(E + 1, dtype=i32, device=device),
         "perm": torch.empty(T * K, dtype=i32, device=device),
         "inv_perm": torch.empty(T * K, dtype=i32, device=device),
         "shared_gate": torch.empty(max(T, 1), dtype=f32, device=device)}
    if logits:
        r["logits"] = torch.empty((T, E), dtype=f32, device=device)
    if select_keys:
        r["select_keys"] = torch.empty((T, E), dtype=f32, device=device)
    return r
