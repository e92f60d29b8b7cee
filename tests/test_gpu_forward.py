"""End-to-end GPU parity of the layer (moe_forward and the staged API) against the CPU oracle.

Sizes are chosen so the float64 oracle finishes in seconds while the GPU path still spans
several tiles of both tile shapes and ragged tails.  Routing is compared bit-exactly on the
GPU's exported fp32 logits, and the oracle computes the expert outputs from those same logits
(the near-tie protocol: logits themselves are checked against the oracle's in
test_gpu_route.py).  Outputs: max |err| <= 2e-2·RMS (bf16 layers) or 1e-4·RMS (fp32 layers)
on the fp32 result; a bf16 output is additionally allowed its own rounding (half a bf16 ulp),
and with the (default) gather combine must equal the round-to-nearest-even of the fp32 result
bit for bit.
"""

import numpy as np
import pytest
import torch

from mixture_experts_layer_renorm_amd import abi
from mixture_experts_layer_renorm_amd.synth import CONFIGS, hot_experts, make_layer
from oracle import moe_oracle as O
from tests.moe_testlib import (TOL_BF16, TOL_F32, TOL_ROUTING_W, bf16_half_ulp, f64, i64,
                               oracle_args, problem_for, rel_max_err, weights_for)

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    # name: (workload, overrides, T)
    "tiny": ("tiny", {}, 64),
    "tiny_large_tiles": ("tiny", {}, 1000),
    "a3b_decode": ("a3b_decode", {}, 64),
    "a3b_E16": ("a3b_prefill", {"E": 16}, 600),
    "a3b_T1": ("a3b_prefill", {}, 1),
    "a17b_E32": ("a17b", {"E": 32}, 400),
    "ds_sigmoid_E16": ("ds_sigmoid", {"E": 16}, 333),
    "skew_E64": ("skew", {"E": 64, "hot_stride": 8}, 500),
    "skew_conc_E64": ("skew_conc", {"E": 64, "hot_stride": 8}, 300),
    # wide gated shared expert: its dense GEMMs fill the chip and run on the matrix-core GEMM
    # (dense tiles; the down GEMM writes fp32 rows, row-scaled by the gate with the atomic combine)
    "shared_wide": ("tiny", {"D": 256, "E": 4, "K": 2, "F": 256, "F_shared": 2048,
                             "shared_gated": True, "dtype": "bf16"}, 2048),
    # the same with an ungated shared expert and a sigmoid router, a ragged last 256-row tile of
    # the dense shared GEMMs, and D = 320 (a ragged last column tile and fp16 factor block)
    "shared_wide_sigmoid": ("tiny", {"D": 320, "E": 6, "K": 3, "F": 192, "F_shared": 2048,
                                     "shared_gated": False, "scoring": "sigmoid",
                                     "dtype": "bf16"}, 2000),
    # degenerate routings: every expert selected (dense mixture), a single expert
    "dense_K_eq_E": ("tiny", {"E": 8, "K": 8}, 77),
    "single_expert": ("tiny", {"E": 1, "K": 1, "dtype": "bf16"}, 50),
    # the largest E and K the library takes, with reduction lengths of one and two K steps
    "max_E_K": ("a3b_prefill", {"D": 128, "E": 1024, "K": 64, "F": 64}, 40),
    # reduction lengths that are not a multiple of the streaming ring, ragged N tiles
    "odd_k": ("a3b_prefill", {"D": 192, "F": 320, "E": 16}, 300),
    # expert outputs far above the fp16 range (|y| ~ 1e5): the fp16 rows of the default path
    # carry a power-of-two factor per row and 128-column block, so nothing overflows
    "huge_values": ("tiny", {"dtype": "bf16", "std_expert": 4.0, "D": 320}, 200),
    # batches of at most 64 tokens: reductions of exactly three K stages (the shortest that
    # carries the rings into the next tile) and of five, ragged N tiles, tiles over 32 rows
    "small_ragged": ("a3b_prefill", {"D": 192, "F": 320, "E": 4, "K": 2}, 61),
    # T = 64 with about 32 rows per expert: consecutive tiles alternate between one and two
    # 32-row halves
    "small_E8_T64": ("a3b_prefill", {"E": 8, "K": 4}, 64),
}


def _case(name):
    wl, over, T = CASES[name]
    cfg = CONFIGS[wl].with_(**over)
    layer = make_layer(cfg, device=DEV, T=T)
    return cfg, layer, T


def _forward(cfg, layer, T, out_dtype, atomic, gemm_kernel="auto"):
    p = problem_for(cfg, T=T, out_dtype=out_dtype, atomic_combine=atomic, gemm_kernel=gemm_kernel)
    r = abi.alloc_routing(p, DEV)
    out = torch.empty((T, cfg.D), dtype=out_dtype, device=DEV)
    abi.moe_forward(p, layer["x"], weights_for(layer), r, out, abi.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    return out, r


def _oracle(cfg, layer, logits):
    args, kw = oracle_args(cfg, layer)
    return O.moe_forward(*args, logits=f64(logits), **kw)


def _check_routing(cfg, r, ref):
    np.testing.assert_array_equal(i64(r["topk_idx"]), ref["topk_idx"])
    np.testing.assert_allclose(f64(r["topk_w"]), ref["topk_w"], rtol=0, atol=TOL_ROUTING_W)
    n = int(ref["offsets"][cfg.E])
    np.testing.assert_array_equal(i64(r["expert_counts"]), ref["counts"])
    np.testing.assert_array_equal(i64(r["expert_offsets"]), ref["offsets"])
    np.testing.assert_array_equal(i64(r["perm"])[:n], ref["perm"])
    np.testing.assert_array_equal(i64(r["inv_perm"]), ref["inv_perm"])


def _tol(cfg):
    return TOL_F32 if cfg.dtype == "f32" else TOL_BF16


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("atomic", [False, True])
def test_forward_matches_oracle(name, atomic):
    cfg, layer, T = _case(name)
    out32, r = _forward(cfg, layer, T, torch.float32, atomic)
    ref = _oracle(cfg, layer, r["logits"])
    _check_routing(cfg, r, ref)
    if cfg.shared_gated:
        np.testing.assert_allclose(f64(r["shared_gate"][:T]), ref["gate"], rtol=0, atol=1e-5)
    err = rel_max_err(out32, ref["out"])
    assert err <= _tol(cfg), f"{name}: max|err|/RMS = {err:.3e}"
    if cfg.dtype == "bf16":
        outb, rb = _forward(cfg, layer, T, torch.bfloat16, atomic)
        assert torch.equal(rb["topk_idx"], r["topk_idx"])
        if not atomic:
            assert torch.equal(outb, out32.to(torch.bfloat16))
        got = f64(outb)
        rms = float(np.sqrt(np.mean(ref["out"] ** 2)))
        bound = _tol(cfg) * rms + bf16_half_ulp(ref["out"])
        assert np.all(np.abs(got - ref["out"]) <= bound)


@pytest.mark.parametrize("name", ["tiny", "a3b_E16", "a17b_E32", "ds_sigmoid_E16", "a3b_decode"])
def test_staged_api_matches_oracle(name):
    cfg, layer, T = _case(name)
    p = problem_for(cfg, T=T, out_dtype=torch.float32)
    ws = abi.alloc_workspace(p, DEV)
    r = abi.alloc_routing(p, DEV)
    w = weights_for(layer)
    x = layer["x"]
    abi.moe_route(p, x, w, r, ws)
    x_perm = torch.empty((T * cfg.K, cfg.D), dtype=cfg.torch_dtype, device=DEV)
    abi.moe_dispatch(p, x, r, x_perm, ws)
    A = T * cfg.K
    y_perm = torch.empty((A, cfg.D), dtype=torch.float32, device=DEV)
    y_perm2 = torch.empty((A, cfg.D), dtype=torch.float32, device=DEV)
    y_shared = (torch.empty((T, cfg.D), dtype=torch.float32, device=DEV)
                if cfg.F_shared else None)
    abi.moe_experts(p, x, None, w, r, y_perm, y_shared, ws)       # rows gathered on load
    abi.moe_experts(p, None, x_perm, w, r, y_perm2, None, ws)     # rows from x_perm
    out = torch.empty((T, cfg.D), dtype=torch.float32, device=DEV)
    abi.moe_combine(p, y_perm, r, y_shared, out)
    torch.cuda.synchronize()
    ref = _oracle(cfg, layer, r["logits"])
    _check_routing(cfg, r, ref)
    assert torch.equal(y_perm, y_perm2)
    tol = _tol(cfg)
    assert rel_max_err(y_perm, ref["y_perm"]) <= tol
    if cfg.F_shared:
        assert rel_max_err(y_shared, ref["y_shared"]) <= tol
    assert rel_max_err(out, ref["out"]) <= tol


def test_deterministic_forward_is_bitwise_reproducible():
    cfg, layer, T = _case("a17b_E32")
    a, _ = _forward(cfg, layer, T, torch.bfloat16, False)
    b, _ = _forward(cfg, layer, T, torch.bfloat16, False)
    assert torch.equal(a, b)


def test_empty_batch_is_noop():
    cfg = CONFIGS["tiny"]
    p = problem_for(cfg, T=0)
    out = torch.full((1, cfg.D), 7.0, device=DEV)
    layer = make_layer(cfg, device=DEV, T=1)
    abi.moe_forward(p, layer["x"], weights_for(layer), None, out, abi.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_concentrated_routing_hits_eight_experts():
    cfg, layer, T = _case("skew_conc_E64")
    _, r = _forward(cfg, layer, T, torch.float32, True)
    counts = i64(r["expert_counts"])
    assert sorted(np.nonzero(counts)[0].tolist()) == hot_experts(cfg)
    assert np.all(counts[hot_experts(cfg)] == T)


GROUPED_TILES = ["tile32", "tile256", "mfma"]


@pytest.mark.parametrize("tile", GROUPED_TILES)
@pytest.mark.parametrize("name", ["a3b_E16", "a17b_E32", "skew_conc_E64", "ds_sigmoid_E16",
                                  "a3b_T1", "odd_k", "skew_E64"])
def test_every_grouped_tile_shape_matches_oracle(name, tile):
    """Every grouped GEMM the library has, forced through moe_problem.gemm_kernel on the same
    inputs: ragged groups, multi-tile experts and empty experts in all of them."""
    cfg, layer, T = _case(name)
    for atomic in (False, True):
        out32, r = _forward(cfg, layer, T, torch.float32, atomic, gemm_kernel=tile)
        ref = _oracle(cfg, layer, r["logits"])
        _check_routing(cfg, r, ref)
        err = rel_max_err(out32, ref["out"])
        assert err <= _tol(cfg), f"{name}/{tile}/atomic={atomic}: max|err|/RMS = {err:.3e}"


@pytest.mark.parametrize("name", ["ds_sigmoid_E16", "a3b_E16", "a3b_decode"])
def test_forward_with_select_bias(name):
    """moe_forward with a selection-only bias: routing bit-exact against the oracle fed the
    GPU's logits and the fp32 selection keys (score + bias) the GPU compared, output within the
    layer's tolerance."""
    cfg, layer, T = _case(name)
    g = torch.Generator(device="cpu").manual_seed(77)
    scale = 0.05 if cfg.scoring == "sigmoid" else 2.0 / cfg.E
    bias = (torch.randn(cfg.E, generator=g) * scale).to(torch.float32)
    p = problem_for(cfg, T=T, out_dtype=torch.float32)
    r = abi.alloc_routing(p, DEV, select_keys=True)
    out = torch.empty((T, cfg.D), dtype=torch.float32, device=DEV)
    w = weights_for(layer)
    w["select_bias"] = bias.to(DEV)
    abi.moe_forward(p, layer["x"], w, r, out, abi.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    args, kw = oracle_args(cfg, layer)
    ref = O.moe_forward(*args, logits=f64(r["logits"]), select_bias=f64(bias),
                        select_keys=f64(r["select_keys"]), **kw)
    _check_routing(cfg, r, ref)
    plain = O.topk_select(f64(r["logits"]), cfg.K)
    assert np.any(np.sort(ref["topk_idx"], 1) != np.sort(plain, 1))  # the bias mattered
    assert rel_max_err(out, ref["out"]) <= _tol(cfg)


@pytest.mark.parametrize("name,cf", [("tiny", 0.75), ("a3b_E16", 1.0), ("skew_E64", 1.25),
                                     ("a3b_decode", 2.0), ("a17b_E32", 0.5)])
@pytest.mark.parametrize("atomic", [False, True])
def test_forward_with_capacity(name, cf, atomic):
    """Token dropping: routing and the kept rows bit-exact against the oracle with the same
    capacity, dropped slots contributing nothing (a token with every slot dropped and no shared
    expert outputs exactly 0).  Output bound: 2e-2 (bf16) / 1e-4 (fp32) of the output RMS,
    applied token by token on each token's own output RMS (every case) and on the RMS of the
    whole capped output (every case but the skewed layer).  On the skewed layer dropping
    removes most hot-expert terms: the output RMS falls 2.4x while the tokens that kept their
    hot slots stay as large, so max|y|/RMS grows from about 7 to 13-19 and the rounding of H
    to bf16 alone (the intermediate precision of the pages' chain) reaches 2.3-3.2e-2 of that
    RMS in a float64 emulation of five draws, while staying within 0.9-1.1e-2 of each token's
    own RMS."""
    cfg, layer, T = _case(name)
    p = problem_for(cfg, T=T, out_dtype=torch.float32, atomic_combine=atomic)
    p.capacity_factor = cf
    r = abi.alloc_routing(p, DEV)
    out = torch.empty((T, cfg.D), dtype=torch.float32, device=DEV)
    abi.moe_forward(p, layer["x"], weights_for(layer), r, out, abi.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    C = O.expert_capacity(T * cfg.K, cfg.E, cf)
    args, kw = oracle_args(cfg, layer)
    ref = O.moe_forward(*args, logits=f64(r["logits"]), capacity=C, **kw)
    _check_routing(cfg, r, ref)
    assert int(ref["counts"].max()) <= C
    got, want = f64(out), ref["out"]
    err = rel_max_err(got, want)
    tok_rms = np.sqrt(np.mean(want ** 2, axis=1))
    live = tok_rms > 0
    per_tok = float(np.max(np.max(np.abs(got - want), axis=1)[live] / tok_rms[live]))
    print(f"{name} cf={cf} atomic={atomic}: max|err|/RMS(capped output) = {err:.3e}, "
          f"max over tokens of max|err_t|/RMS(y_t) = {per_tok:.3e}")
    assert per_tok <= _tol(cfg), f"{name}: per-token max|err_t|/RMS(y_t) = {per_tok:.3e}"
    if name != "skew_E64":
        assert err <= _tol(cfg), f"{name}: max|err|/RMS = {err:.3e}"
    all_dropped = np.all(ref["inv_perm"].reshape(T, cfg.K) < 0, axis=1)
    if not cfg.F_shared and all_dropped.any():
        assert np.all(f64(out)[all_dropped] == 0.0)
