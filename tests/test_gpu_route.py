"""GPU parity of stage 1 (router GEMM, top-K, weights) against the CPU oracle.

Selection is compared bit-exactly on the same fp32 logits (the GPU's exported logits, or
logits constructed here); weights within 1e-6 absolute; the router GEMM's logits within the
worst-case fp32 summation bound of the float64 oracle logits.
"""

import numpy as np
import pytest
import torch

from mixture_experts_layer_renorm_amd import abi
from mixture_experts_layer_renorm_amd.synth import CONFIGS
from oracle import moe_oracle as O
from tests.moe_testlib import TOL_ROUTING_W, f64, i64, problem_for, weights_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _route_logits(logits: torch.Tensor, K: int, scoring="softmax", renormalize=True):
    T, E = logits.shape
    p = abi.make_problem(T=T, D=64, E=E, K=K, F=64, scoring=scoring, renormalize=renormalize)
    r = {"topk_idx": torch.empty((T, K), dtype=torch.int32, device=DEV),
         "topk_w": torch.empty((T, K), dtype=torch.float32, device=DEV)}
    abi.moe_route_logits(p, logits.contiguous(), r)
    torch.cuda.synchronize()
    return r["topk_idx"], r["topk_w"]


def _check_route(logits, K, scoring="softmax", renormalize=True, check_w=True):
    idx, w = _route_logits(logits, K, scoring, renormalize)
    L = f64(logits)
    want_idx = O.topk_select(L, K)
    np.testing.assert_array_equal(i64(idx), want_idx)
    if check_w:
        want_w = O.routing_weights(L, want_idx, scoring, renormalize)
        np.testing.assert_allclose(f64(w), want_w, rtol=0, atol=TOL_ROUTING_W)


@pytest.mark.parametrize("E,K", [(8, 2), (256, 8), (512, 10), (256, 6), (5, 2), (1000, 7),
                                 (64, 64), (8, 8), (1, 1), (130, 3), (1024, 64)])
@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_topk_random_logits(E, K, scoring):
    g = torch.Generator(device="cpu").manual_seed(E * 100 + K)
    T = 37 if E > 256 else 301  # ragged: not a multiple of the 4 tokens per work-group
    logits = (torch.randn((T, E), generator=g) * 2.0).to(DEV)
    _check_route(logits, K, scoring)


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_topk_no_renorm(scoring):
    g = torch.Generator(device="cpu").manual_seed(3)
    logits = torch.randn((129, 256), generator=g).to(DEV)
    _check_route(logits, 8, scoring, renormalize=False)


def test_topk_exact_ties_and_special_values():
    """Quantised logits force ties at the K boundary; ±0, ±inf and NaN rows follow the total order."""
    g = torch.Generator(device="cpu").manual_seed(4)
    q = torch.randint(-3, 4, (200, 64), generator=g).float() * 0.25
    rows = [
        [1.0] * 64,
        [-0.0 if i % 2 else 0.0 for i in range(64)],
        [float("nan") if i % 3 == 0 else float(i % 5) for i in range(64)],
        [float("inf") if i in (5, 9) else (-float("inf") if i % 2 else 0.5) for i in range(64)],
        [float("nan")] * 64,
        [3.0e38 if i == 63 else -3.0e38 for i in range(64)],
    ]
    logits = torch.cat([q, torch.tensor(rows)]).to(DEV)
    for K in (1, 2, 8, 13):
        idx, _ = _route_logits(logits, K)
        np.testing.assert_array_equal(i64(idx), O.topk_select(f64(logits), K))
    # weights are checked where they are finite
    _check_route(q.to(DEV), 8)


def test_worked_example_through_gpu():
    """E=5, k=2, sigmoid scores 0.90 (expert 2) and 0.60 (expert 5) give weights 0.60 and 0.40."""
    s = torch.tensor([[0.1, 0.9, 0.2, 0.3, 0.6]], dtype=torch.float64)
    logits = torch.log(s / (1 - s)).float().to(DEV)
    idx, w = _route_logits(logits, 2, "sigmoid")
    assert i64(idx).tolist() == [[1, 4]]
    np.testing.assert_allclose(f64(w)[0], [0.6, 0.4], rtol=0, atol=TOL_ROUTING_W)


def _fp32_logit_bound(X, W, logits64):
    """Worst-case error of the fp32 logits: a length-D dot product of exactly representable
    products accumulated in fp32 errs by at most γ_D·Σ|x_i w_i|, γ_D = D·u/(1-D·u), u = 2^-24
    (any summation order; one more term covers rounded fp32 products); adding a bias rounds
    once more (u·|r|)."""
    D = X.shape[1] + 1
    u = 2.0 ** -24
    gamma = D * u / (1 - D * u)
    return gamma * (np.abs(X) @ np.abs(W).T) + 2 * u * np.abs(logits64) + 1e-30


# bf16 batches of up to 1024 tokens take the split-K router (K slices summed by the top-K
# kernel: 8 slices at T=64, 4 for the gated 513-column a17b router at T=70, 1 past 256 blocks);
# larger bf16 batches with fewer than 32 output tiles take the tile GEMM with its reduction
# split into up to 8 slices (4 at T=1025 with a ragged last M tile, 2 for the gated
# 513-column a17b router at T=1100 and at T=3000 of the sigmoid layer, 1 at T=2000 of a17b),
# and from 32 tiles the matrix-core GEMM split into 8 slices (ragged last M tiles at T=8000 of
# the sigmoid layer and T=4000 of the gated a17b layer, whose gate logit the top-K kernel
# computes; the skewed layer's logit bias at T=8192); fp32 takes the unsplit tile GEMM.
@pytest.mark.parametrize("name,T", [("tiny", 64), ("a3b_prefill", 333), ("a17b", 70),
                                    ("skew", 200), ("ds_sigmoid", 90), ("a3b_decode", 64),
                                    ("a3b_prefill", 1), ("a17b", 1), ("a3b_prefill", 1024),
                                    ("a3b_prefill", 1025), ("a17b", 1100), ("a17b", 2000),
                                    ("skew", 4096), ("ds_sigmoid", 3000), ("ds_sigmoid", 8000),
                                    ("a17b", 4000), ("skew", 8192)])
def test_router_gemm_and_topk(name, T):
    cfg = CONFIGS[name]
    # only the router's tensors, drawn on the CPU at the workload's real widths
    g = torch.Generator(device="cpu").manual_seed(11)
    dt = cfg.torch_dtype
    x = (torch.randn((T, cfg.D), generator=g)).to(dt)
    wr = (torch.randn((cfg.E, cfg.D), generator=g) * cfg.std_router).to(dt)
    ws = (torch.randn((1, cfg.D), generator=g) * 0.02).to(dt) if cfg.shared_gated else None
    bias = None
    if cfg.hot_bias:
        bias = torch.zeros(cfg.E)
        bias[[i * cfg.hot_stride for i in range(cfg.n_hot)]] = cfg.hot_bias
    p = problem_for(cfg, T=T)
    plan = abi.describe_plan(p)
    tiles = -(-T // 256) * -(-cfg.E // 256)
    if cfg.dtype == "bf16" and T > 1024 and tiles >= 32:
        assert plan.startswith("router: mfma 256x256, 8 K slice(s)"), plan
    r = abi.alloc_routing(p, DEV)
    weights = {"w_router": wr.to(DEV), "logit_bias": None if bias is None else bias.to(DEV),
               "ws_gate": None if ws is None else ws.to(DEV)}
    ws_buf = abi.alloc_workspace(p, DEV)
    abi.moe_route(p, x.to(DEV), weights, r, ws_buf)
    torch.cuda.synchronize()
    X, W = f64(x), f64(wr)
    want_logits = O.router_logits(X, W, f64(bias))
    got_logits = f64(r["logits"])
    bound = _fp32_logit_bound(X, W, want_logits)
    assert np.all(np.abs(got_logits - want_logits) <= bound)
    # selection bit-exact on the GPU's own fp32 logits, weights within 1e-6
    want_idx = O.topk_select(got_logits, cfg.K)
    np.testing.assert_array_equal(i64(r["topk_idx"]), want_idx)
    want_w = O.routing_weights(got_logits, want_idx, cfg.scoring)
    np.testing.assert_allclose(f64(r["topk_w"]), want_w, rtol=0, atol=TOL_ROUTING_W)
    # tokens whose selection differs under the fp64 logits must be near-ties
    ref_idx = O.topk_select(want_logits, cfg.K)
    differ = np.nonzero(np.any(np.sort(ref_idx, 1) != np.sort(want_idx, 1), axis=1))[0]
    delta = np.max(bound, axis=1)
    for t in differ:
        srt = np.sort(want_logits[t])[::-1]
        assert srt[cfg.K - 1] - srt[cfg.K] <= 2 * delta[t]
    if ws is not None:
        # sigmoid is 1/4-Lipschitz: the gate errs by at most a quarter of its logit's bound
        Ws = f64(ws)
        want_g = O.shared_gate(X, Ws)
        gbound = 0.25 * _fp32_logit_bound(X, Ws, X @ Ws.T)[:, 0] + 1e-7
        assert np.all(np.abs(f64(r["shared_gate"]) - want_g) <= gbound)


@pytest.mark.parametrize("T,D,E,K,scoring,gated,bias", [(8200, 1024, 300, 5, "softmax", True, True),
                                                       (8192, 512, 1024, 8, "sigmoid", False, False)])
def test_matrix_core_router_partial_column_tiles(T, D, E, K, scoring, gated, bias):
    """The matrix-core router where E is not a multiple of its 256-column tiles: E = 300 (a
    second, mostly empty column tile, with a logit bias and the gate logit from the top-K
    kernel; 2 slices) and E = 1024 (four column tiles; top-K over 16 logits per lane)."""
    g = torch.Generator(device="cpu").manual_seed(E)
    x = torch.randn((T, D), generator=g).to(torch.bfloat16)
    wr = (torch.randn((E, D), generator=g) * D ** -0.5).to(torch.bfloat16)
    ws = (torch.randn((1, D), generator=g) * 0.02).to(torch.bfloat16) if gated else None
    lb = torch.randn(E, generator=g) * 0.5 if bias else None
    p = abi.make_problem(T=T, D=D, E=E, K=K, F=64, F_shared=64 if gated else 0,
                         shared_gated=gated, scoring=scoring)
    plan = abi.describe_plan(p)
    assert plan.startswith("router: mfma 256x256"), plan
    r = abi.alloc_routing(p, DEV)
    weights = {"w_router": wr.to(DEV), "logit_bias": None if lb is None else lb.to(DEV),
               "ws_gate": None if ws is None else ws.to(DEV)}
    abi.moe_route(p, x.to(DEV), weights, r, abi.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    X, W = f64(x), f64(wr)
    want_logits = O.router_logits(X, W, f64(lb))
    got_logits = f64(r["logits"])
    assert np.all(np.abs(got_logits - want_logits) <= _fp32_logit_bound(X, W, want_logits))
    want_idx = O.topk_select(got_logits, K)
    np.testing.assert_array_equal(i64(r["topk_idx"]), want_idx)
    np.testing.assert_allclose(f64(r["topk_w"]), O.routing_weights(got_logits, want_idx, scoring),
                               rtol=0, atol=TOL_ROUTING_W)
    if gated:
        Ws = f64(ws)
        gbound = 0.25 * _fp32_logit_bound(X, Ws, X @ Ws.T)[:, 0] + 1e-7
        assert np.all(np.abs(f64(r["shared_gate"]) - O.shared_gate(X, Ws)) <= gbound)


# ---- selection-only bias ("1.6 ..." §三): choose on score + bias, weight with the score ----

def select_key_bound(logits64, bias64, scoring, E):
    """Largest error of the GPU's fp32 key fl(score) + bias against the float64 score + bias.

    sigmoid: s = 1/(1 + e^-r) from a float32 exp (a few ulp), an add and a divide: relative
    error within 8u.  softmax: p = e^(r - m) / sum over E of e^(r_j - m): the subtraction errs
    by u|r - m| before the exp (relative u|r - m| after it), the exp by a few ulp, the float32
    sum over E terms by at most (E/64 + 6) u relative (lane sums of E/64 terms, then a 6-level
    butterfly), and the divide by u; with the largest |r_j - m| of the row, the relative error
    of p is within (2 |r - m| + 2 max|r_j - m| + E/64 + 16) u.  The final add of the bias rounds
    once more (u |key|), counted twice for slack."""
    u = 2.0 ** -24
    score = O.routing_scores(logits64, scoring)
    key = np.abs(score + bias64[None, :])
    if scoring == "sigmoid":
        rel = 8 * u
    else:
        z = logits64 - np.max(logits64, axis=1, keepdims=True)
        rel = (2 * np.abs(z) + 2 * np.max(np.abs(z), axis=1, keepdims=True) + E / 64 + 16) * u
    return rel * score + 2 * u * key + 1e-30


@pytest.mark.parametrize("E,K", [(8, 2), (256, 8), (256, 6), (64, 64), (130, 3), (1024, 16)])
@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("renormalize", [True, False])
def test_topk_select_bias(E, K, scoring, renormalize):
    """Routing with a selection-only bias is bit-exact: the oracle chooses on the fp32 keys
    (score + bias) the GPU compared, exported through select_keys, so both sides apply the same
    total order to the same values and no token may differ.  The keys themselves are checked
    against the float64 score + bias within their rounding bound, and the weights (unbiased
    scores of the chosen experts) within 1e-6."""
    g = torch.Generator().manual_seed(E * 7 + K)
    T = 700
    logits = torch.randn((T, E), generator=g) * 1.5
    # a bias comparable to the spread of the scores, so it really moves the choice
    scale = 0.05 if scoring == "sigmoid" else 2.0 / E
    bias = (torch.randn(E, generator=g) * scale).to(torch.float32)
    p = abi.make_problem(T=T, D=64, E=E, K=K, F=64, scoring=scoring, renormalize=renormalize)
    r = {"topk_idx": torch.empty((T, K), dtype=torch.int32, device=DEV),
         "topk_w": torch.empty((T, K), dtype=torch.float32, device=DEV),
         "select_keys": torch.empty((T, E), dtype=torch.float32, device=DEV)}
    abi.moe_route_logits(p, logits.to(DEV), r, select_bias=bias.to(DEV))
    torch.cuda.synchronize()
    L, b = f64(logits), f64(bias)
    keys = f64(r["select_keys"])
    got = i64(r["topk_idx"])
    want, want_w = O.route(L, K, scoring, renormalize, select_bias=b, select_keys=keys)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_allclose(f64(r["topk_w"]), want_w, rtol=0, atol=TOL_ROUTING_W)
    keys64 = O.routing_scores(L, scoring) + b[None, :]
    assert np.all(np.abs(keys - keys64) <= select_key_bound(L, b, scoring, E))
    # the bias moved the choice of many tokens away from the unbiased router's
    if K < E:
        assert np.mean(np.any(np.sort(got, 1) != np.sort(O.topk_select(L, K), 1), axis=1)) > 0.05


def test_select_keys_without_bias_are_the_logits():
    """Without a selection bias the key top-K compares is the logit itself."""
    g = torch.Generator().manual_seed(5)
    T, E, K = 99, 130, 5
    logits = torch.randn((T, E), generator=g)
    p = abi.make_problem(T=T, D=64, E=E, K=K, F=64)
    r = {"topk_idx": torch.empty((T, K), dtype=torch.int32, device=DEV),
         "topk_w": torch.empty((T, K), dtype=torch.float32, device=DEV),
         "select_keys": torch.empty((T, E), dtype=torch.float32, device=DEV)}
    abi.moe_route_logits(p, logits.to(DEV), r)
    torch.cuda.synchronize()
    assert torch.equal(r["select_keys"].cpu(), logits)


@pytest.mark.parametrize("E", [1, 7, 256, 1024])
def test_update_select_bias_bit_exact(E):
    g = torch.Generator().manual_seed(E)
    counts = torch.randint(0, 40, (E,), generator=g, dtype=torch.int32)
    if E >= 7:
        counts[3] = 0
        counts[:E // 2] = int(counts.sum()) // E  # some at the integer mean (maybe not exact)
    bias = (torch.randn(E, generator=g) * 0.1).to(torch.float32)
    p = abi.make_problem(T=1, D=64, E=E, K=1, F=64)
    b_dev = bias.to(DEV)
    abi.moe_update_select_bias(p, counts.to(DEV), b_dev, 1e-3)
    torch.cuda.synchronize()
    want = O.update_select_bias(counts.numpy(), bias.numpy(), 1e-3)
    assert np.array_equal(b_dev.cpu().numpy().view(np.uint32), want.view(np.uint32))


# ---- router statistics ("1.6 ..." §三 balance loss, §六 z-loss) ----

def _stats_check(got, want, E):
    np.testing.assert_allclose(f64(got["f"]), want["f"], rtol=1e-6, atol=0)
    # P: fp32 sums of positive terms in a fixed order (at most ~ 20 + T/64 additions deep)
    np.testing.assert_allclose(f64(got["P"]), want["P"], rtol=5e-5, atol=1e-9)
    for k, rtol in (("aux", 5e-5), ("z", 5e-5), ("cv", 1e-6), ("max_over_mean", 1e-6)):
        assert abs(float(got[k]) - want[k]) <= rtol * abs(want[k]) + 1e-9, (k, float(got[k]),
                                                                           want[k])


@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (333, 8, 2), (1000, 256, 8), (4096, 256, 8),
                                   (700, 1000, 7), (65, 64, 64)])
@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_router_stats_match_oracle(T, E, K, scoring):
    g = torch.Generator().manual_seed(T + E)
    logits = torch.randn((T, E), generator=g) * 2.0
    idx = O.topk_select(f64(logits), K)
    counts = torch.as_tensor(O.dispatch(idx, E)["counts"], dtype=torch.int32)
    p = abi.make_problem(T=T, D=64, E=E, K=K, F=64, scoring=scoring)
    got = abi.moe_router_stats(p, logits.to(DEV), counts.to(DEV), abi.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    _stats_check(got, O.router_stats(f64(logits), counts.numpy(), scoring), E)


def test_router_stats_from_a_forward_pass():
    """The statistics of a real batch: logits and counts exported by moe_forward on the skewed
    35B-A3B-shaped layer (most assignments on 8 hot experts)."""
    cfg = CONFIGS["skew"]
    from mixture_experts_layer_renorm_amd.synth import make_layer
    layer = make_layer(cfg, device=DEV, T=2048)
    p = problem_for(cfg, T=2048)
    r = abi.alloc_routing(p, DEV)
    ws = abi.alloc_workspace(p, DEV)
    out = torch.empty((2048, cfg.D), dtype=cfg.torch_dtype, device=DEV)
    abi.moe_forward(p, layer["x"], weights_for(layer), r, out, ws)
    got = abi.moe_router_stats(p, r["logits"], r["expert_counts"], ws)
    torch.cuda.synchronize()
    want = O.router_stats(f64(r["logits"]), i64(r["expert_counts"]), cfg.scoring)
    _stats_check(got, want, cfg.E)
    assert want["max_over_mean"] > 10  # the skew is visible in the loads
