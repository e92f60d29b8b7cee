/*
 * moe.h -- C ABI of libmoe.so: forward pass of one sparse Mixture-of-Experts feed-forward layer
 * on an AMD Instinct MI355X (gfx950).
 *
 * The layer, for each of T tokens x_t (a row of x [T,D]):
 *   r_t  = W_r x_t (+ b)                                   router logits, E experts
 *   I_t  = the K experts with the largest r_t               top-K selection
 *   a_t,e = p_e / sum_{j in I_t} p_j                        renormalised weights
 *           (p = softmax(r_t) or p = sigmoid(r_t))
 *   y_t  = sum_{e in I_t} a_t,e * E_e(x_t) + g_t * E_s(x_t) routed sum + optional shared expert
 *   E_e(x) = W_down_e (SiLU(W_gate_e x) * W_up_e x)         SwiGLU expert, SiLU(z) = z*sigmoid(z)
 *   g_t  = sigmoid(w_s . x_t) (gated shared expert) or 1 (ungated)
 * Sources: "MoE" (llm.rainlin.net) §2 Router, §3 专家计算, §4 输出聚合; "1.6 混合专家（MoE）：参数量与
 * 计算量的解耦" (llm.satori-ai.cn) §二 Top-k 门控公式, §四 DeepSeekMoE (sigmoid scores, ungated
 * shared expert).  The residual add belongs to the enclosing decoder block and is not done here.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless stated; every buffer is owned by the caller.  The
 *    library never allocates, frees or synchronises, and keeps no mutable global state other
 *    than the thread-local text returned by moe_last_error().
 *  - All work is enqueued asynchronously on `stream` (NULL = the null stream).  Validation
 *    happens before any launch: an invalid call returns an error and enqueues nothing.
 *  - Device faults surface at the caller's next synchronisation.  A launch error is reported
 *    as MOE_ERR_HIP.
 *  - T == 0 is a no-op returning MOE_OK.
 *  - Every device pointer must be 16-byte aligned.  `out` must not alias `x`.
 *  - Matrices are row-major with the reduction dimension contiguous.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same object as hipStream_t. */
typedef struct ihipStream_t *moe_stream_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* NULL required pointer, misalignment, K > E, K < 1, ...         */
  MOE_ERR_UNSUPPORTED = -2, /* shape outside v1 limits (see moe_problem)                     */
  MOE_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than moe_workspace_size()           */
  MOE_ERR_HIP = -4          /* a HIP call or kernel launch failed                            */
} moe_status;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_SCORE_SOFTMAX = 0, /* p = softmax over all E logits, in fp32   ("MoE" §2)             */
  MOE_SCORE_SIGMOID = 1  /* p = per-expert sigmoid of the logit       ("1.6 ..." §二 step 1)  */
} moe_scoring;

enum {
  MOE_FLAG_ATOMIC_COMBINE = 1u, /* fuse the combine into the down GEMM with fp32 atomic
                                   adds into a [T,D] accumulator: no [T*K,D] buffer, but the
                                   summation order (and so the last bits) varies run to run.
                                   Default: each expert row is stored and a gather kernel sums
                                   each token's K rows in slot order (bitwise reproducible;
                                   measured faster on MI355X, whose device-scope float
                                   atomics do not resolve in the per-XCD L2)              */
  MOE_FLAG_NO_RENORM = 2u      /* a = p_e without renormalisation over I_t (the plain
                                  top-k sum of "Qwen3.8-Flash-Next 架构笔记 · 04" §2)       */
};

/* Kernel used for the routed (grouped) expert GEMMs.  AUTO: the matrix-core GEMM with
 * 256 x 256 tiles for bf16 layers whose operands fit its 32-bit offsets, else the tile GEMM
 * (256-row tiles when experts average more than 48 rows, 32-row tiles otherwise). */
typedef enum {
  MOE_GEMM_AUTO = 0,
  MOE_GEMM_TILE_32 = 1,   /* tile GEMM, 32 x 128 output tiles (any dtype)                     */
  MOE_GEMM_TILE_256 = 2,  /* tile GEMM, 256 x 128 output tiles (any dtype)                    */
  MOE_GEMM_MFMA_256 = 3   /* matrix-core GEMM, 256 x 256 tiles (bf16 layers only; otherwise
                             MOE_ERR_UNSUPPORTED)                                         */
} moe_gemm_kernel;

/* Dispatch implementation.  AUTO: one work-group for up to 8192 assignments and E <= 768,
 * else a histogram launch followed by a scan + scatter launch. */
typedef enum {
  MOE_DISPATCH_AUTO = 0,
  MOE_DISPATCH_ONE_WORKGROUP = 1, /* any T*K; E <= 768 (otherwise MOE_ERR_UNSUPPORTED)        */
  MOE_DISPATCH_MULTI = 2          /* count, then scan + scatter                               */
} moe_dispatch_kernel;

/* Problem statement (host struct, read during the call, not retained).
 * v1 limits: D, F and F_shared multiples of 64; 1 <= E <= 1024; 1 <= K <= min(E, 64);
 * T*K < 2^31. */
typedef struct {
  int64_t T;            /* tokens (batch x sequence flattened)                             */
  int32_t D;            /* hidden width                                                    */
  int32_t E;            /* routed experts                                                  */
  int32_t K;            /* experts per token                                               */
  int32_t F;            /* routed-expert intermediate width                                */
  int32_t F_shared;     /* shared-expert intermediate width, 0 = no shared expert          */
  int32_t shared_gated; /* 1: shared output scaled by sigmoid(w_s . x); 0: by 1            */
  int32_t scoring;      /* moe_scoring                                                     */
  int32_t dtype;        /* moe_dtype of x, the weights and the intermediate H              */
  int32_t out_dtype;    /* moe_dtype of `out`; accumulation is always fp32, and a bf16
                           output is the round-to-nearest-even of the fp32 result         */
  uint32_t flags;       /* MOE_FLAG_*                                                      */
  float capacity_factor;/* 0: dropless.  > 0: each expert keeps at most
                           C = max(min_capacity, ceil(capacity_factor * T*K / E)) rows
                           ("1.6 ..." §三 expert capacity; the ceiling is taken in double on
                           the host): its first C assignments in ascending a = t*K + k; the
                           others are dropped (inv_perm = -1, excluded from counts) and add
                           nothing to the output                                           */
  int32_t min_capacity; /* floor of C when capacity_factor > 0 (>= 0)                      */
  int32_t gemm_kernel;  /* moe_gemm_kernel: which GEMM runs the routed experts; 0 (AUTO) =
                           the library's choice.  A forced choice computes the same result
                           (within the layer's tolerance) with another tiling, for tests and
                           tuning; it is never read from the environment               */
  int32_t dispatch_kernel; /* moe_dispatch_kernel; 0 (AUTO) = the library's choice; forced
                              choices give bit-identical dispatch results              */
} moe_problem;

/* Weights, all in `dtype` except logit_bias (fp32).  Layouts follow the fused projections of
 * "MoE" §3.2: the gate and up projections of one expert are one [2F, D] matrix. */
typedef struct {
  const void *w_router;    /* [E, D]                                   required            */
  const float *logit_bias; /* [E] added to the logits before scoring, or NULL              */
  const void *w_gate_up;   /* [E, 2F, D]; rows [0,F) gate, rows [F,2F) up                  */
  const void *w_down;      /* [E, D, F]                                                    */
  const void *ws_gate_up;  /* [2*F_shared, D]  (shared expert; NULL iff F_shared == 0)     */
  const void *ws_down;     /* [D, F_shared]                                                */
  const void *ws_gate;     /* [1, D] shared-expert gate projection (required iff gated)    */
  const float *select_bias;/* [E] fp32 selection-only bias, or NULL ("1.6 ..." §三,
                              DeepSeek-V3's auxiliary-loss-free balancing): experts are
                              chosen on score + bias and weighted with the unbiased score,
                              where score = softmax probability or sigmoid affinity        */
} moe_weights;

/* Routing tensors.  Which fields are inputs and which are outputs depends on the call. */
typedef struct {
  float *logits;           /* [T, E] fp32 router logits (bias included)                    */
  int32_t *topk_idx;       /* [T, K] selected experts, slots in descending key order (the
                              logit; with a select_bias, score + bias), ties to the lower
                              expert id; ids outside [0,E) are skipped
                              by dispatch and combine (sentinels)                          */
  float *topk_w;           /* [T, K] fp32 weights a_t,e                                    */
  int32_t *expert_counts;  /* [E]   t_e = assignments routed to (and kept on) expert e     */
  int32_t *expert_offsets; /* [E+1] exclusive prefix sum of expert_counts                  */
  int32_t *perm;           /* [T*K] perm[pos] = assignment id a = t*K + k, grouped by
                              expert, ascending a within an expert (first offsets[E] valid) */
  int32_t *inv_perm;       /* [T*K] inv_perm[a] = pos, or -1 for a skipped sentinel or an
                              assignment dropped for capacity                              */
  float *shared_gate;      /* [T]   g_t = sigmoid(w_s . x_t)                               */
  float *select_keys;      /* [T, E] fp32: the value top-K compared for each expert -- the
                              logit r_te, or with a select_bias the fp32 score + bias
                              (NaN ranks as -inf, -0 as +0).  Output of moe_route,
                              moe_route_logits and moe_forward when non-NULL; with the
                              exported keys, a selection can be checked bit for bit          */
} moe_routing;

/* Host only.  Bytes of device workspace every entry point below accepts for problem `p`
 * (one size serves all of them).  Returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED for a
 * problem the library cannot run. */
int moe_workspace_size(const moe_problem *p, size_t *bytes);

/* Stage 1, router ("MoE" §2; "1.6 ..." §二 steps 1-3).
 * In: x [T,D], w->w_router, w->logit_bias, w->ws_gate (if F_shared > 0 and gated).
 * Out: r->topk_idx, r->topk_w (required); r->logits (optional, [T,E] fp32);
 *      r->shared_gate (optional, only written for a gated shared expert).
 * Logits are fp32 MFMA accumulations of the dtype inputs; selection compares these fp32
 * values exactly (a NaN logit ranks as -inf; -0 equals +0).  With w->select_bias the key is
 * the fp32 score + bias instead (the same total order on that key). */
int moe_route(const moe_problem *p, const void *x, const moe_weights *w, moe_routing *r,
              void *workspace, size_t workspace_bytes, moe_stream_t stream);

/* Stage 1 from given logits: top-K selection and weights only.
 * In: logits [T,E] fp32 (logit bias, if any, already included); select_bias [E] fp32 or
 * NULL (as moe_weights.select_bias).  Out: r->topk_idx, r->topk_w.
 * No workspace.  Used to check selection bit-exactly on shared logits. */
int moe_route_logits(const moe_problem *p, const float *logits, const float *select_bias,
                     moe_routing *r, moe_stream_t stream);

/* Router statistics of one routed batch ("1.6 ..." §三 auxiliary balance loss, §六 router
 * z-loss).  In: logits [T,E] fp32 (e.g. r->logits of moe_route / moe_forward, bias included),
 * expert_counts [E] int32 (the dispatch histogram).  Out: stats [2E + 4] fp32:
 *   stats[e]       f_e = t_e / sum(t), the fraction of dispatched assignments on expert e
 *   stats[E + e]   P_e = mean over tokens of the router probability of expert e (softmax; for a
 *                  sigmoid router the affinities normalised over the token's E experts)
 *   stats[2E]      E * sum_e f_e P_e (the balance loss before its weight; 1 when uniform)
 *   stats[2E + 1]  mean over tokens of (log sum_e exp r_te)^2 (the z-loss before its weight)
 *   stats[2E + 2]  population std / mean of the loads t_e;  stats[2E + 3]  max t_e / mean t_e
 * Deterministic (fixed-order reductions, no atomics).  Uses the workspace.  T = 0: no-op. */
int moe_router_stats(const moe_problem *p, const float *logits, const int32_t *expert_counts,
                     float *stats, void *workspace, size_t workspace_bytes, moe_stream_t stream);

/* One step of the selection-bias feedback ("1.6 ..." §三): with the loads t_e of a dispatch
 * (expert_counts [E] int32) and their mean m = sum(t) / E, select_bias[e] (fp32 [E], updated
 * in place) is lowered by gamma if t_e > m, raised by gamma if t_e < m, kept if t_e = m.
 * The comparison is exact (t_e * E against sum(t) in 64-bit integers); each update is one
 * fp32 add.  One work-group; no workspace.  MOE_ERR_INVALID_ARG for NULL or unaligned
 * pointers. */
int moe_update_select_bias(const moe_problem *p, const int32_t *expert_counts,
                           float *select_bias, float gamma, moe_stream_t stream);

/* Stage 2, dispatch ("MoE" §3.2: gather the tokens of each hit expert).
 * In: r->topk_idx.  Out: r->expert_counts, r->expert_offsets, r->perm, r->inv_perm (required).
 * x_perm: optional [T*K, D] dtype; row pos receives x[perm[pos] / K] (rows at and beyond
 * offsets[E] are left untouched).  NULL = experts gather rows from x on load instead.
 * x may be NULL when x_perm is NULL.  The result is bit-exact and deterministic. */
int moe_dispatch(const moe_problem *p, const void *x, moe_routing *r, void *x_perm,
                 void *workspace, size_t workspace_bytes, moe_stream_t stream);

/* Stage 3, experts ("MoE" §3): y_perm[pos] = E_e(x[perm[pos]/K]) for every valid pos of
 * expert e (unweighted), fp32.  In: x [T,D] (or x_perm if non-NULL), w, r->expert_offsets,
 * r->perm.  y_perm: [T*K, D] fp32, rows at and beyond offsets[E] untouched.
 * y_shared: [T, D] fp32 receives E_s(x_t) (ungated) when F_shared > 0, else ignored (may be
 * NULL; NULL with F_shared > 0 skips the shared expert). */
int moe_experts(const moe_problem *p, const void *x, const void *x_perm, const moe_weights *w,
                const moe_routing *r, float *y_perm, float *y_shared, void *workspace,
                size_t workspace_bytes, moe_stream_t stream);

/* Stage 4, combine ("MoE" §3.2 index_add, §4 branch add):
 * out[t] = sum_k topk_w[t,k] * y_perm[inv_perm[t*K+k]] + g_t * y_shared[t], summed in slot
 * order in fp32 and rounded once to out_dtype.  g_t = r->shared_gate[t] if gated, else 1.
 * y_shared NULL = no shared term.  Deterministic.  No workspace. */
int moe_combine(const moe_problem *p, const float *y_perm, const moe_routing *r,
                const float *y_shared, void *out, moe_stream_t stream);

/* The whole layer: router, dispatch, grouped gate_up GEMM with fused SiLU*up, grouped down
 * GEMM with fused weighted combine, shared expert, final cast.  out: [T, D] out_dtype.
 * r_opt may be NULL; each non-NULL field of *r_opt receives the corresponding intermediate.
 * By default the combine gathers each token's K expert rows in slot order (bitwise
 * reproducible); MOE_FLAG_ATOMIC_COMBINE selects the fused atomic epilogue instead. */
int moe_forward(const moe_problem *p, const void *x, const moe_weights *w, moe_routing *r_opt,
                void *out, void *workspace, size_t workspace_bytes, moe_stream_t stream);

/* Stage boundaries recorded by moe_forward_timed, in launch order. */
enum {
  MOE_STAGE_ROUTER = 0,   /* router GEMM (+ shared-gate column)                        */
  MOE_STAGE_TOPK = 1,     /* top-K selection and weights                               */
  MOE_STAGE_DISPATCH = 2, /* histogram, scan + tile map, stable scatter                */
  MOE_STAGE_GATE_UP = 3,  /* routed grouped gate_up GEMM with fused SiLU*up            */
  MOE_STAGE_SHARED = 4,   /* shared expert (atomic mode: or the accumulator zero-fill) */
  MOE_STAGE_DOWN = 5,     /* routed grouped down GEMM (+ fused combine in atomic mode)  */
  MOE_STAGE_FINAL = 6,    /* gather combine (default), or the final cast (atomic mode) */
  MOE_STAGE_COUNT = 7
};

/* moe_forward with timing: events[i] (a caller-created hipEvent_t, passed as void*) is
 * recorded on `stream` right before stage i is launched and events[MOE_STAGE_COUNT] after
 * the last one, so hipEventElapsedTime(events[i], events[i+1]) brackets stage i.  `events`
 * must hold MOE_STAGE_COUNT + 1 entries; a NULL entry is not recorded (so a caller can bracket
 * one stage with two events).  Same results and errors as moe_forward. */
int moe_forward_timed(const moe_problem *p, const void *x, const moe_weights *w,
                      moe_routing *r_opt, void *out, void *workspace, size_t workspace_bytes,
                      moe_stream_t stream, void *const *events);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_forward without a workspace argument.  Its
 * kernels use a fixed scratch array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends; the caller still passes inputs and outputs.
 * Same results and errors as moe_forward with a workspace, plus MOE_ERR_WORKSPACE (nothing
 * enqueued) when moe_workspace_size(p) exceeds the scratch size -- e.g. bf16 35B-A3B-shaped
 * batches (D=2048, E=256, K=8, F=512) fit up to a few hundred tokens.  The first call on a
 * device looks up that device's scratch address (no allocation).  Every call on one GPU shares
 * its scratch, which keeps the last call's contents (nothing in it needs to start at zero):
 * calls that may overlap on one GPU -- different streams, or several host threads -- race and
 * must be serialised by the caller.  Never allocates, frees or synchronises. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_problem *p, const void *x, const moe_weights *w,
                        moe_routing *r_opt, void *out, moe_stream_t stream);

/* Static text for a status code. */
const char *moe_status_string(int status);

/* Thread-local text naming the kernels moe_forward would launch for problem p (tile shapes
 * of the router, grouped and shared GEMMs; combine mode), e.g. for reports.  Returns "" and
 * sets moe_last_error() if p is invalid.  Valid until the next call on this thread. */
const char *moe_describe_plan(const moe_problem *p);

/* Thread-local detail about the last failed call on this thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
