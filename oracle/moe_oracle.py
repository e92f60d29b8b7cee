"""CPU oracle for the forward pass of a sparse Mixture-of-Experts feed-forward layer.

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, float64 restatement of what the
layer computes.  It exists to check the HIP path and nothing else: only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The
product path (``mixture_experts_layer_renorm_amd``) never imports it, and it imports nothing
from the product path.  It shares no code with the kernels.

Sources (the pages are cited by title and section):

* [MoE]        "MoE" (llm.rainlin.net, llm-inference) -- §2 Router (routing equations and the
               router module), §3 专家计算 (SwiGLU expert, routed-expert loop), §4 输出聚合
               (routed sum, gated shared expert, branch add).
* [Satori-1.6] "1.6 混合专家（MoE）：参数量与计算量的解耦" (llm.satori-ai.cn) -- §二 Top-k 门控公式
               (four gating steps and the E=5, k=2 worked example), §四 DeepSeekMoE
               (ungated shared-expert isolation, sigmoid gating).
* [S23-J10]    "S23-J10" (clxhxhhr.top) -- §2 (N_e = 3·d·f), §3 (F = 2·N_e·Σt_e, R = b_W·N_e·U,
               worked example 2-4), §4 (shared expert is a routing-independent cost),
               §4.1 (granularity invariance), §10 自测.
* [FFN-notes]  "Qwen3.8-Flash-Next 架构笔记 · 04 / FFN & MOE" (cbphcr.github.io) -- §1 (SwiGLU),
               §2 (MoE sum over the top-k set, without renormalisation).

Readings taken where the pages are silent (each is listed with its reason in the design doc):

* Selection key is the logit r (softmax and sigmoid are strictly increasing, so the top-K set
  of p equals the top-K set of r).  Total order: key descending, expert id ascending; -0.0 is
  +0.0; NaN ranks as -inf.  Slots are written in that order.
* Renormalisation has no epsilon ([MoE] §2 router module).
* Sigmoid scores are normalised by their plain sum over the selected set ([Satori-1.6] §二,
  worked example).
* SiLU(z) = z·sigmoid(z).
* An index outside [0, E) in a top-K table is a sentinel: skipped, not counted ([MoE] §3.2
  routed-expert loop skips the id equal to the expert count).
* Dispatch order inside one expert is ascending assignment id a = t·K + k.
* The layer output excludes the residual ([MoE] §4 block code returns without it).

Parity status of each public function (pins live in tests/test_oracle_pins.py):
every function below is pinned; none is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import Any, Dict, Optional, Sequence

import numpy as np

SCORING_SOFTMAX = "softmax"
SCORING_SIGMOID = "sigmoid"

__all__ = [
    "SCORING_SOFTMAX", "SCORING_SIGMOID",
    "as_f64", "router_logits", "shared_gate", "selection_keys", "topk_select",
    "routing_scores", "routing_weights", "topk_select_biased", "route", "update_select_bias",
    "router_stats", "expert_capacity",
    "dispatch", "silu", "sigmoid", "swiglu",
    "moe_forward", "moe_forward_dense_masked",
    "expert_params", "expert_flops", "expert_read_bytes", "layer_flops",
]


def as_f64(a: Any) -> np.ndarray:
    """Exact upcast of a float array (fp32 or already-widened bf16 values) to float64."""
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------------------------
# Stage 1: router.  [MoE] §2: flatten [B,S,D] to T tokens, project without bias to E logits.
# ---------------------------------------------------------------------------------------------

def router_logits(x: Any, w_router: Any, logit_bias: Optional[Any] = None) -> np.ndarray:
    """r = x · W_rᵀ  (+ an optional per-expert logit bias), in float64.  x [T,D], W_r [E,D].

    [MoE] §2 Router: r = x W_rᵀ ∈ R^{T×E}, a linear map with no bias term.  The optional bias
    is the skewed-routing workload's fixed per-expert shift of the logits before scoring.
    """
    r = as_f64(x) @ as_f64(w_router).T
    if logit_bias is not None:
        r = r + as_f64(logit_bias)[None, :]
    return r


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1/(1+e^{-z}) in float64, written to avoid overflow warnings."""
    z = as_f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def shared_gate(x: Any, w_shared_gate: Any) -> np.ndarray:
    """g_t = sigmoid(w_sᵀ x_t) for every token; w_s is the [1,D] (or [D]) gate projection.

    [MoE] §4 输出聚合: the shared expert's output is scaled by a scalar sigmoid gate computed
    from the same input token.
    """
    w = as_f64(w_shared_gate).reshape(-1)
    return sigmoid(as_f64(x) @ w)


# ---------------------------------------------------------------------------------------------
# Stage 1b: top-K selection and weights.  [MoE] §2; [Satori-1.6] §二 steps 2-3.
# ---------------------------------------------------------------------------------------------

def selection_keys(logits: Any) -> np.ndarray:
    """Canonical selection keys: NaN -> -inf, -0.0 -> +0.0, everything else unchanged."""
    k = as_f64(logits).copy()
    k[np.isnan(k)] = -np.inf
    k = k + 0.0  # -0.0 + 0.0 == +0.0 under round-to-nearest
    return k


def topk_select(logits: Any, K: int) -> np.ndarray:
    """Indices [T,K] (int32) of the K largest keys per row, in descending key order.

    [MoE] §2: I_t = TopK(p_t, K); [Satori-1.6] §二 step 2 keeps the K highest scores.  Ties are
    broken toward the lower expert id (the order is total, so the result is unique).
    """
    keys = selection_keys(logits)
    T, E = keys.shape
    if not 1 <= K <= E:
        raise ValueError(f"need 1 <= K <= E, got K={K}, E={E}")
    # A stable ascending sort of -key visits keys in descending order and keeps equal keys in
    # ascending id order.
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def routing_scores(logits: Any, scoring: str = SCORING_SOFTMAX) -> np.ndarray:
    """Scores [T,E] (float64): softmax probabilities over all E experts ([MoE] §2), or the
    per-expert sigmoid affinities ([Satori-1.6] §二 step 1, §四)."""
    r = as_f64(logits)
    if scoring == SCORING_SOFTMAX:
        m = np.max(np.where(np.isnan(r), -np.inf, r), axis=1, keepdims=True)
        e = np.exp(r - m)
        return e / np.sum(e, axis=1, keepdims=True)
    if scoring == SCORING_SIGMOID:
        return sigmoid(r)
    raise ValueError(f"unknown scoring {scoring!r}")


def routing_weights(logits: Any, idx: Any, scoring: str = SCORING_SOFTMAX,
                    renormalize: bool = True) -> np.ndarray:
    """Weights α [T,K] (float64) of the selected experts.

    softmax: p = softmax(r) over all E experts; α = p_e / Σ_{j∈I_t} p_j   ([MoE] §2).
    sigmoid: s = sigmoid(r); α = s_e / Σ_{j∈I_t} s_j   ([Satori-1.6] §二 step 3, worked example).
    renormalize=False keeps p_e (or s_e) unnormalised, the plain top-k sum of [FFN-notes] §2.
    """
    score = routing_scores(logits, scoring)
    idx = np.asarray(idx, dtype=np.int64)
    sel = np.take_along_axis(score, idx, axis=1)
    if renormalize:
        sel = sel / np.sum(sel, axis=1, keepdims=True)
    return sel


def topk_select_biased(logits: Any, K: int, scoring: str, select_bias: Any) -> np.ndarray:
    """Selection on s_e + b_e ([Satori-1.6] §三, DeepSeek-V3's auxiliary-loss-free balancing:
    a per-expert bias enters only the top-k choice, never the gating weight).

    s is the score of routing_scores (sigmoid affinity, or the softmax probability for a
    softmax router -- the page states the rule for affinities; applying it to probabilities is
    this oracle's reading).  Same total order as topk_select: key descending, id ascending;
    a NaN key ranks as -inf.
    """
    keys = routing_scores(logits, scoring) + as_f64(select_bias)[None, :]
    keys = selection_keys(keys)
    T, E = keys.shape
    if not 1 <= K <= E:
        raise ValueError(f"need 1 <= K <= E, got K={K}, E={E}")
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def route(logits: Any, K: int, scoring: str = SCORING_SOFTMAX,
          renormalize: bool = True, select_bias: Optional[Any] = None,
          select_keys: Optional[Any] = None):
    """(topk_idx [T,K] int32, topk_w [T,K] float64) from logits.

    With select_bias, the experts are chosen on score + bias and weighted with the unbiased
    scores ([Satori-1.6] §三).  select_keys [T,E], if given, are the score + bias values some
    other implementation compared (e.g. in float32): the choice is then the same total order
    (key descending, id ascending) applied to those keys, so the two choices can be compared bit
    for bit; the weights still come from the logits."""
    if select_keys is not None:
        if select_bias is None:
            raise ValueError("select_keys are only meaningful with a select_bias")
        idx = topk_select(select_keys, K)
    elif select_bias is None:
        idx = topk_select(logits, K)
    else:
        idx = topk_select_biased(logits, K, scoring, select_bias)
    return idx, routing_weights(logits, idx, scoring, renormalize)


def update_select_bias(counts: Any, select_bias: Any, gamma: float) -> np.ndarray:
    """One step of the bias feedback of [Satori-1.6] §三: an expert whose load is above the
    mean load has its bias lowered by gamma, one below the mean raised by gamma, and one at the
    mean keeps it.  The mean is Σ counts / E; the comparison is made exactly in integers
    (counts_e · E against Σ counts).  Arithmetic in float32, the bias's storage type (one
    rounding per expert), so the result is exact to compare."""
    c = np.asarray(counts, dtype=np.int64)
    b = np.asarray(select_bias, dtype=np.float32).copy()
    E = c.shape[0]
    total = int(c.sum())
    g = np.float32(gamma)
    for e in range(E):
        d = int(c[e]) * E - total
        if d > 0:
            b[e] = np.float32(b[e] - g)
        elif d < 0:
            b[e] = np.float32(b[e] + g)
    return b


def router_stats(logits: Any, counts: Any, scoring: str = SCORING_SOFTMAX) -> Dict[str, Any]:
    """Load-balance and stability statistics of one routed batch.

    f[i]  = t_i / Σ_j t_j, the fraction of the batch's dispatched assignments on expert i
            (the hard counts of [Satori-1.6] §三; Σ f = 1).
    P[i]  = mean over tokens of the router probability of expert i: the softmax probability
            ([Satori-1.6] §三); for a sigmoid router, the affinities normalised over all E
            experts of the token (this oracle's reading, so that Σ P = 1 as the page requires).
    aux   = N · Σ_i f_i P_i, the auxiliary balance loss before its weight α ([Satori-1.6] §三;
            1 when f and P are uniform, N when both sit on one expert).
    z     = mean over tokens of (log Σ_j exp r_tj)², the router z-loss before its weight
            ([Satori-1.6] §六).
    cv    = std(t) / mean(t) over the E experts, population standard deviation (the load
            coefficient of variation of the routing visualisation on the "Qwen3.6-27B" page,
            §五), and max_over_mean = max(t) / mean(t).
    """
    r = as_f64(logits)
    t = np.asarray(counts, dtype=np.float64)
    T, E = r.shape
    total = t.sum()
    f = t / total if total > 0 else np.zeros(E)
    m = np.max(r, axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.sum(np.exp(r - m), axis=1))
    if scoring == SCORING_SOFTMAX:
        prob = np.exp(r - lse[:, None])
    elif scoring == SCORING_SIGMOID:
        s = sigmoid(r)
        prob = s / np.sum(s, axis=1, keepdims=True)
    else:
        raise ValueError(f"unknown scoring {scoring!r}")
    P = prob.mean(axis=0)
    mean = total / E
    return {"f": f, "P": P, "aux": float(E * np.sum(f * P)), "z": float(np.mean(lse ** 2)),
            "cv": float(t.std() / mean) if mean > 0 else 0.0,
            "max_over_mean": float(t.max() / mean) if mean > 0 else 0.0}


# ---------------------------------------------------------------------------------------------
# Stage 2: dispatch.  [MoE] §3.2: group the assignments by expert so each hit expert runs once.
# ---------------------------------------------------------------------------------------------

def expert_capacity(A: int, E: int, capacity_factor: float, min_capacity: int = 0) -> int:
    """Rows one expert may take: the even share of the batch's A = T·K assignments times the
    capacity factor ([Satori-1.6] §三 专家容量, factor > 1 such as 1.25, leaving headroom for
    imbalance), rounded up, and at least min_capacity (the floor of the training configuration
    on the "Qwen3.6-27B" page, §四).  Counting assignments rather than tokens is this oracle's
    reading for top-K routing."""
    return max(int(min_capacity), math.ceil(capacity_factor * A / E))


def dispatch(topk_idx: Any, E: int, capacity: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Expert-contiguous grouping of the T·K assignments a = t·K + k.

    counts[e]  = number of assignments kept on expert e (ids outside [0,E) are sentinels,
                 skipped)
    offsets    = [0, cumsum(counts)]  (length E+1)
    perm[pos]  = assignment id at position pos of the grouped order; grouped by expert, ascending
                 assignment id within an expert (a stable counting sort by expert)
    inv_perm[a]= position of assignment a, or -1 for a skipped sentinel or a dropped assignment
    dropped    = number of assignments dropped for capacity

    capacity: if given, each expert keeps only its first `capacity` assignments in that order
    (earlier tokens first); the rest are dropped and, with no residual in the layer output,
    contribute nothing ([Satori-1.6] §三 token dropping).
    """
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)          # sentinels sort after every real expert
    order = np.argsort(key, kind="stable")
    raw = np.bincount(flat[valid], minlength=E).astype(np.int64)
    kept_parts = []
    start = 0
    for e in range(E):
        group = order[start:start + raw[e]]
        start += raw[e]
        kept_parts.append(group if capacity is None else group[:capacity])
    perm = np.concatenate(kept_parts) if kept_parts else np.zeros(0, dtype=np.int64)
    counts = np.array([len(g) for g in kept_parts], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    inv_perm = np.full(flat.shape[0], -1, dtype=np.int64)
    inv_perm[perm] = np.arange(perm.shape[0])
    return {"counts": counts, "offsets": offsets, "perm": perm, "inv_perm": inv_perm,
            "dropped": int(raw.sum() - counts.sum())}


# ---------------------------------------------------------------------------------------------
# Stage 3: SwiGLU experts.  [MoE] §3: E_e(x) = W_down(SiLU(W_gate x) ⊙ W_up x); [FFN-notes] §1.
# ---------------------------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z · sigmoid(z)."""
    z = as_f64(z)
    return z * sigmoid(z)


def swiglu(X: Any, w_gate_up: Any, w_down: Any) -> np.ndarray:
    """One SwiGLU expert on the rows of X [m,D].

    w_gate_up is [2F, D]: rows [0,F) are W_gate, rows [F,2F) are W_up (the fused projection of
    [MoE] §3.2, split in two halves).  w_down is [D, F].  Returns [m, D] float64.
    """
    X = as_f64(X)
    wgu = as_f64(w_gate_up)
    F = wgu.shape[0] // 2
    gate = X @ wgu[:F].T
    up = X @ wgu[F:].T
    h = silu(gate) * up
    return h @ as_f64(w_down).T


# ---------------------------------------------------------------------------------------------
# Stages 3-5 together: the layer.  [MoE] §3.2 loop, §4 aggregation; [Satori-1.6] §二, §四.
# ---------------------------------------------------------------------------------------------

def moe_forward(x: Any, w_router: Any, w_gate_up: Sequence[Any], w_down: Sequence[Any], K: int,
                scoring: str = SCORING_SOFTMAX, renormalize: bool = True,
                logit_bias: Optional[Any] = None,
                ws_gate_up: Optional[Any] = None, ws_down: Optional[Any] = None,
                w_shared_gate: Optional[Any] = None,
                logits: Optional[Any] = None,
                select_bias: Optional[Any] = None,
                select_keys: Optional[Any] = None,
                capacity: Optional[int] = None) -> Dict[str, Any]:
    """Forward pass of one MoE layer, float64, without the residual.

    x [T,D]; w_router [E,D]; w_gate_up[e] [2F,D] and w_down[e] [D,F] are indexed one expert at a
    time (any object with __getitem__ works, so large layers can be fetched lazily).
    ws_gate_up/ws_down: the always-on shared expert ([Satori-1.6] §四) or None.
    w_shared_gate: [1,D] sigmoid gate of the shared branch ([MoE] §4); None = ungated (g ≡ 1).
    logits: if given (e.g. fp32 logits exported by another implementation), routing is taken
    from them instead of being recomputed from x and w_router.
    select_bias: [E] selection-only bias ([Satori-1.6] §三), or None.
    select_keys: [T,E] score + bias values to choose on (see route), or None.
    capacity: rows per expert (see expert_capacity); dropped assignments contribute nothing.

    y_t = Σ_k α_{t,k} · E_{I_t[k]}(x_t) + g_t · E_s(x_t)
    """
    X = as_f64(x)
    T = X.shape[0]
    if logits is None:
        r = router_logits(X, w_router, logit_bias)
    else:
        r = as_f64(logits)
    E = r.shape[1]
    idx, alpha = route(r, K, scoring, renormalize, select_bias, select_keys)
    d = dispatch(idx, E, capacity)
    counts, offsets, perm, inv_perm = d["counts"], d["offsets"], d["perm"], d["inv_perm"]

    D = X.shape[1]
    y_perm = np.zeros((int(offsets[E]), D), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue  # experts with no rows are never evaluated
        rows = X[perm[lo:hi] // K]
        y_perm[lo:hi] = swiglu(rows, w_gate_up[e], w_down[e])

    y_routed = np.zeros((T, D), dtype=np.float64)
    for k in range(K):
        pos = inv_perm.reshape(T, K)[:, k]
        kept = pos >= 0
        y_routed[kept] += alpha[kept, k:k + 1] * y_perm[pos[kept]]

    out = y_routed.copy()
    y_shared = None
    gate = None
    if ws_gate_up is not None:
        y_shared = swiglu(X, ws_gate_up, ws_down)
        gate = shared_gate(X, w_shared_gate) if w_shared_gate is not None else np.ones(T)
        out = out + gate[:, None] * y_shared
    return {"logits": r, "topk_idx": idx, "topk_w": alpha, "counts": counts,
            "offsets": offsets, "perm": perm, "inv_perm": inv_perm, "y_perm": y_perm,
            "y_routed": y_routed, "y_shared": y_shared, "gate": gate, "out": out}


def moe_forward_dense_masked(x: Any, w_router: Any, w_gate_up: Sequence[Any],
                             w_down: Sequence[Any], K: int, scoring: str = SCORING_SOFTMAX,
                             renormalize: bool = True, logit_bias: Optional[Any] = None,
                             ws_gate_up: Optional[Any] = None, ws_down: Optional[Any] = None,
                             w_shared_gate: Optional[Any] = None) -> np.ndarray:
    """Brute force for tiny inputs: evaluate every expert on every token, then mask.

    M[t,e] = α_{t,e} if e ∈ I_t else 0; y = Σ_e M[:,e] · E_e(x) (+ gated shared branch).
    [Satori-1.6] §二 and [FFN-notes] §2 state the layer as this masked sum; the sparse path must
    give the same numbers without evaluating the unselected experts.
    """
    X = as_f64(x)
    r = router_logits(X, w_router, logit_bias)
    T, E = r.shape
    keys = selection_keys(r)
    M = np.zeros((T, E))
    for t in range(T):
        # independent selection: repeatedly take the best remaining (key, -id)
        remaining = list(range(E))
        chosen = []
        for _ in range(K):
            best = max(remaining, key=lambda e: (keys[t, e], -e))
            chosen.append(best)
            remaining.remove(best)
        if scoring == SCORING_SOFTMAX:
            finite = r[t][~np.isnan(r[t])]
            m = finite.max() if finite.size else 0.0
            p = np.array([math.exp(v - m) for v in r[t]])
            p = p / p.sum()
        else:
            p = np.array([1.0 / (1.0 + math.exp(-v)) if v >= 0 else
                          math.exp(v) / (1.0 + math.exp(v)) for v in r[t]])
        s = sum(p[e] for e in chosen) if renormalize else 1.0
        for e in chosen:
            M[t, e] = p[e] / s
    out = np.zeros_like(X)
    for e in range(E):
        out += M[:, e:e + 1] * swiglu(X, w_gate_up[e], w_down[e])
    if ws_gate_up is not None:
        g = shared_gate(X, w_shared_gate) if w_shared_gate is not None else np.ones(T)
        out += g[:, None] * swiglu(X, ws_gate_up, ws_down)
    return out


# ---------------------------------------------------------------------------------------------
# Analytic cost model.  [S23-J10] §2, §3, §4.
# ---------------------------------------------------------------------------------------------

def expert_params(d: int, f: int) -> int:
    """N_e = 3·d·f: gate, up and down projections of one SwiGLU expert ([S23-J10] §2)."""
    return 3 * d * f


def expert_flops(d: int, f: int, counts: Sequence[int]) -> int:
    """F_expert = 2·N_e·Σ_e t_e: each dispatched row costs 2 FLOP per expert parameter."""
    return 2 * expert_params(d, f) * int(np.sum(np.asarray(counts, dtype=np.int64)))


def expert_read_bytes(d: int, f: int, U: int, bytes_per_weight: int = 2) -> int:
    """R_expert = b_W·N_e·U: each distinct expert hit in the batch is read once ([S23-J10] §3)."""
    return bytes_per_weight * expert_params(d, f) * U


def layer_flops(d: int, f: int, counts: Sequence[int], m: int = 0, f_shared: int = 0) -> int:
    """2·m·N_s + 2·Σ_e t_e·N_e: the shared expert runs on all m tokens ([S23-J10] §4)."""
    return 2 * m * expert_params(d, f_shared) + expert_flops(d, f, counts)
