"""Parity at the full sizes of the benchmark workloads, in the launch configuration bench.py
times (default flags: gather combine; output in the layer dtype).

  * Routing and dispatch are checked bit-exactly over the WHOLE batch: the oracle's top-K,
    weights, histogram, offsets and stable permutation are recomputed from the GPU's exported
    fp32 logits (the near-tie protocol; the logits themselves are checked against the oracle's
    router on a token sample).
  * Outputs, to the bf16 bound max|err| <= 2e-2 * RMS(oracle output) on the fp32 result (plus
    half a bf16 ulp on the bf16 output):
      - every token of the batch for the 35B-A3B-shaped decode and prefill batches, the skewed
        and concentrated layers and the granularity pair;
      - for the 397B-A17B-shaped and the sigmoid layers (8192 and 16384 tokens, 5.8 TFLOP of
        float64 work for the whole sigmoid batch), the tokens at the first and last row of every
        M tile of every expert (the tile map's own split of each expert's rows), every token of
        three chosen experts, the first and last row of every 256-row tile of the dense shared
        expert, and a seeded sample; plus those three experts' whole outputs through the staged
        API (moe_experts), row for row.
  * Properties that hold at any size are checked on the whole output: it is finite, and the
    bf16 output is exactly the round-to-nearest-even of the same call's fp32 result.
"""

import numpy as np
import pytest
import torch

from mixture_experts_layer_renorm_amd import abi
from mixture_experts_layer_renorm_amd.synth import CONFIGS, hot_experts, make_layer
from oracle import moe_oracle as O
from tests.moe_testlib import (TOL_BF16, TOL_ROUTING_W, bf16_half_ulp, f64, i64, oracle_args,
                               problem_for, rel_max_err, weights_for)

pytestmark = pytest.mark.gpu
DEV = "cuda"

WHOLE_BATCH = ("a3b_decode", "a3b_prefill", "skew", "skew_conc", "gran_e128", "gran_e64")
TILE_ROWS = ("a17b", "ds_sigmoid")
WORKLOADS = WHOLE_BATCH + TILE_ROWS
MTILE = 256   # rows per M tile of the grouped matrix-core GEMM (the tile map's bm)
DENSE_TILE = 256


@pytest.fixture(scope="module", params=list(WORKLOADS))
def run(request):
    name = request.param
    cfg = CONFIGS[name]
    print(f"\n[fullsize] {name}: T={cfg.T} D={cfg.D} E={cfg.E} K={cfg.K} F={cfg.F}", flush=True)
    layer = make_layer(cfg, device=DEV, seed=0)
    outs = {}
    for out_dtype in (cfg.torch_dtype, torch.float32):
        p = problem_for(cfg, T=cfg.T, out_dtype=out_dtype)
        r = abi.alloc_routing(p, DEV)
        out = torch.empty((cfg.T, cfg.D), dtype=out_dtype, device=DEV)
        abi.moe_forward(p, layer["x"], weights_for(layer), r, out, abi.alloc_workspace(p, DEV))
        torch.cuda.synchronize()
        outs[out_dtype] = (out, r)
    yield name, cfg, layer, outs
    del layer, outs
    torch.cuda.empty_cache()


def test_routing_and_dispatch_bit_exact_on_whole_batch(run):
    name, cfg, layer, outs = run
    out, r = outs[cfg.torch_dtype]
    logits = f64(r["logits"])
    idx, alpha = O.route(logits, cfg.K, cfg.scoring)
    np.testing.assert_array_equal(i64(r["topk_idx"]), idx)
    np.testing.assert_allclose(f64(r["topk_w"]), alpha, rtol=0, atol=TOL_ROUTING_W)
    d = O.dispatch(idx, cfg.E)
    np.testing.assert_array_equal(i64(r["expert_counts"]), d["counts"])
    np.testing.assert_array_equal(i64(r["expert_offsets"]), d["offsets"])
    np.testing.assert_array_equal(i64(r["perm"]), d["perm"])
    np.testing.assert_array_equal(i64(r["inv_perm"]), d["inv_perm"])
    assert int(d["offsets"][-1]) == cfg.T * cfg.K
    if name == "skew_conc":
        assert sorted(np.nonzero(d["counts"])[0].tolist()) == hot_experts(cfg)
    # the second call (fp32 output) routed identically
    assert torch.equal(outs[torch.float32][1]["topk_idx"], r["topk_idx"])


def test_router_logits_match_oracle_on_sample(run):
    name, cfg, layer, outs = run
    _, r = outs[cfg.torch_dtype]
    rng = np.random.RandomState(1)
    tok = np.sort(rng.choice(cfg.T, size=min(cfg.T, 64), replace=False))
    x = f64(layer["x"][tok])
    w = f64(layer["w_router"])
    ref = O.router_logits(x, w, f64(layer["logit_bias"]))
    got = f64(r["logits"])[tok]
    # fp32 accumulation of D products of exactly representable terms, plus the final rounding
    u = 2.0 ** -24
    bound = (cfg.D + 1) * u / (1 - (cfg.D + 1) * u) * (np.abs(x) @ np.abs(w).T) + 2 * u * np.abs(ref)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)


def _tile_rows(counts, offsets):
    """Positions of the first and last row of every M tile: an expert's c rows are split evenly
    over ceil(c / 256) tiles, the first c % n tiles one row longer (the tile map's rule)."""
    pos = []
    for e, c in enumerate(counts):
        c = int(c)
        if c == 0:
            continue
        n = -(-c // MTILE)
        base, extra = divmod(c, n)
        start = int(offsets[e])
        for q in range(n):
            rows = base + (1 if q < extra else 0)
            pos += [start, start + rows - 1]
            start += rows
    return np.asarray(pos, dtype=np.int64)


def _chosen_experts(counts):
    """Three experts: the largest group, the one whose tile rows are furthest from a multiple
    of 32 (the most padding in its last 32-row pair), and the smallest non-empty group."""
    nz = np.nonzero(counts)[0]
    big = int(nz[np.argmax(counts[nz])])
    small = int(nz[np.argmin(counts[nz])])

    def ragged(e):
        c = int(counts[e])
        n = -(-c // MTILE)
        return (-(c // n)) % 32
    rag = int(max(nz, key=lambda e: (ragged(e), -e)))
    return sorted({big, rag, small})


def _checked_tokens(name, cfg, r):
    if name in WHOLE_BATCH:
        return np.arange(cfg.T)
    counts, offsets, perm = i64(r["expert_counts"]), i64(r["expert_offsets"]), i64(r["perm"])
    tok = set((perm[_tile_rows(counts, offsets)] // cfg.K).tolist())
    for e in _chosen_experts(counts):
        tok |= set((perm[offsets[e]:offsets[e + 1]] // cfg.K).tolist())
    if cfg.F_shared:
        for m in range(0, cfg.T, DENSE_TILE):
            tok |= {m, min(m + DENSE_TILE, cfg.T) - 1}
    rng = np.random.RandomState(0)
    tok |= set(rng.choice(cfg.T, size=64, replace=False).tolist())
    return np.asarray(sorted(tok), dtype=np.int64)


def test_outputs_match_oracle(run):
    name, cfg, layer, outs = run
    out, r = outs[cfg.torch_dtype]
    out32, _ = outs[torch.float32]
    tok = _checked_tokens(name, cfg, r)
    print(f"[fullsize] {name}: oracle on {len(tok)} of {cfg.T} tokens", flush=True)
    args, kw = oracle_args(cfg, layer, token_ids=torch.as_tensor(tok, device=DEV))
    ref = O.moe_forward(*args, logits=f64(r["logits"])[tok], **kw)["out"]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err32 = float(np.max(np.abs(f64(out32)[tok] - ref))) / rms
    assert err32 <= TOL_BF16, f"{name}: fp32 result max|err|/RMS = {err32:.3e}"
    got = f64(out)[tok]
    assert np.all(np.abs(got - ref) <= TOL_BF16 * rms + bf16_half_ulp(ref))


@pytest.mark.parametrize("name", TILE_ROWS)
def test_whole_experts_through_staged_api(name):
    """Three experts' whole outputs (every row, every column) from moe_experts at the full batch,
    against the oracle's SwiGLU on the same gathered rows."""
    cfg = CONFIGS[name]
    layer = make_layer(cfg, device=DEV, seed=0)
    p = problem_for(cfg, T=cfg.T, out_dtype=torch.float32)
    ws = abi.alloc_workspace(p, DEV)
    r = abi.alloc_routing(p, DEV)
    w = weights_for(layer)
    abi.moe_route(p, layer["x"], w, r, ws)
    abi.moe_dispatch(p, None, r, None, ws)
    A = cfg.T * cfg.K
    y_perm = torch.empty((A, cfg.D), dtype=torch.float32, device=DEV)
    abi.moe_experts(p, layer["x"], None, w, r, y_perm, None, ws)
    torch.cuda.synchronize()
    counts, offsets, perm = i64(r["expert_counts"]), i64(r["expert_offsets"]), i64(r["perm"])
    for e in _chosen_experts(counts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = torch.as_tensor(perm[lo:hi] // cfg.K, device=DEV)
        want = O.swiglu(f64(layer["x"][rows]), f64(layer["w_gate_up"][e]), f64(layer["w_down"][e]))
        got = f64(y_perm[lo:hi])
        err = rel_max_err(got, want)
        print(f"[fullsize] {name}: expert {e} ({hi - lo} rows) max|err|/RMS = {err:.2e}",
              flush=True)
        assert err <= TOL_BF16, (e, hi - lo, err)
    del layer, y_perm, ws
    torch.cuda.empty_cache()


def test_whole_output_properties(run):
    name, cfg, layer, outs = run
    out, _ = outs[cfg.torch_dtype]
    out32, _ = outs[torch.float32]
    assert torch.isfinite(out32).all()
    # deterministic gather combine: the bf16 output is the RNE of the fp32 result, bit for bit
    assert torch.equal(out, out32.to(out.dtype))
