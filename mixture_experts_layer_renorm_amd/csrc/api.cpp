// Host side of the C ABI declared in include/moe.h: argument validation, workspace layout and
// the order of kernel launches for each stage.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <climits>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "moe.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_HIP_TRY(expr, what)                     \
  do {                                              \
    hipError_t e_ = (expr);                         \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int dtype) { return dtype == MOE_DTYPE_BF16 ? 2 : 4; }

// The matrix-core GEMM addresses its operands with 32-bit byte offsets from a uniform base:
// the grouped GEMMs' token rows ([T*K, max(D, F)] at most, via x_perm or H) and one expert's
// weights must each span less than 4 GiB.
bool mfma_fits(const moe_problem* p) {
  const int64_t es = (int64_t)esize(p->dtype);
  const int64_t wide = p->D > p->F ? p->D : p->F;
  const int64_t lim = (int64_t)1 << 32;
  return p->dtype == MOE_DTYPE_BF16 && p->T * p->K * wide * es < lim &&
         (int64_t)2 * p->F * p->D * es < lim;
}

// The same limit for the shared expert's dense GEMMs: x [T, D], Hs [T, F_s] and the shared
// weights ([2 F_s, D], [D, F_s]).
bool mfma_fits_shared(const moe_problem* p) {
  const int64_t es = (int64_t)esize(p->dtype);
  const int64_t lim = (int64_t)1 << 32;
  return p->dtype == MOE_DTYPE_BF16 && p->T * p->D * es < lim && p->T * p->F_shared * es < lim &&
         (int64_t)2 * p->F_shared * p->D * es < lim;
}

int check_problem(const moe_problem* p) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "problem is NULL");
  if (p->T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
  if (p->E < 1) return fail(MOE_ERR_INVALID_ARG, "E < 1");
  if (p->K < 1 || p->K > p->E) return fail(MOE_ERR_INVALID_ARG, "need 1 <= K <= E (K=%d, E=%d)", p->K, p->E);
  if (p->D < 1 || p->F < 1 || p->F_shared < 0)
    return fail(MOE_ERR_INVALID_ARG, "D, F must be positive and F_shared >= 0");
  if (p->scoring != MOE_SCORE_SOFTMAX && p->scoring != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "unknown scoring %d", p->scoring);
  if (p->dtype != MOE_DTYPE_F32 && p->dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->out_dtype != MOE_DTYPE_F32 && p->out_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown out_dtype %d", p->out_dtype);
  if (p->shared_gated != 0 && p->shared_gated != 1)
    return fail(MOE_ERR_INVALID_ARG, "shared_gated must be 0 or 1");
  if (p->flags & ~(uint32_t)(MOE_FLAG_ATOMIC_COMBINE | MOE_FLAG_NO_RENORM))
    return fail(MOE_ERR_INVALID_ARG, "unknown flag bits 0x%x", p->flags);
  if (!(p->capacity_factor >= 0.0f) || p->capacity_factor > 1e6f)
    return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be in [0, 1e6]");
  if (p->min_capacity < 0) return fail(MOE_ERR_INVALID_ARG, "min_capacity < 0");
  if (p->D % 64 || p->F % 64 || p->F_shared % 64)
    return fail(MOE_ERR_UNSUPPORTED, "D, F and F_shared must be multiples of 64 (D=%d F=%d Fs=%d)",
                p->D, p->F, p->F_shared);
  if (p->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E > 1024");
  if (p->K > 64) return fail(MOE_ERR_UNSUPPORTED, "K > 64");
  if (p->T * (int64_t)p->K >= (int64_t)1 << 31) return fail(MOE_ERR_UNSUPPORTED, "T*K >= 2^31");
  if (p->T * (int64_t)p->D >= (int64_t)1 << 40) return fail(MOE_ERR_UNSUPPORTED, "T*D too large");
  if (p->gemm_kernel < MOE_GEMM_AUTO || p->gemm_kernel > MOE_GEMM_MFMA_256)
    return fail(MOE_ERR_INVALID_ARG, "unknown gemm_kernel %d", p->gemm_kernel);
  if (p->dispatch_kernel < MOE_DISPATCH_AUTO || p->dispatch_kernel > MOE_DISPATCH_MULTI)
    return fail(MOE_ERR_INVALID_ARG, "unknown dispatch_kernel %d", p->dispatch_kernel);
  if (p->gemm_kernel == MOE_GEMM_MFMA_256 && !mfma_fits(p))
    return fail(MOE_ERR_UNSUPPORTED,
                "gemm_kernel MFMA_256 needs a bf16 layer whose token rows and expert weights "
                "each span less than 4 GiB");
  if (!moe::dispatch_supported(p->E, p->dispatch_kernel))
    return fail(MOE_ERR_UNSUPPORTED, "dispatch_kernel ONE_WORKGROUP needs E <= %d",
                moe::kDispatchOneWgMaxE);
  return MOE_OK;
}

bool has_shared(const moe_problem* p) { return p->F_shared > 0; }

// Rows each expert may keep (INT32_MAX when dropless).
int32_t capacity(const moe_problem* p) {
  if (!(p->capacity_factor > 0.0f)) return INT32_MAX;
  const double c = std::ceil((double)p->capacity_factor * (double)(p->T * p->K) / p->E);
  const double lim = (double)INT32_MAX;
  const double v = c > lim ? lim : c;
  return v > p->min_capacity ? (int32_t)v : p->min_capacity;
}
bool gated(const moe_problem* p) { return p->F_shared > 0 && p->shared_gated; }

// Grouped (routed-expert) GEMMs, one tile map of M tiles of up to tile_bm rows.  bf16 layers
// run every expert group on the matrix-core GEMM (256 x 256 tiles, a partial tile computed in
// 32-row steps): at decode sizes its direct-to-LDS weight ring streams the weights at the
// speed of its load pattern, and groups of hundreds of rows keep the matrix cores busy.  fp32
// layers and operands past the 32-bit offsets use the tile GEMM.  moe_problem.gemm_kernel
// forces one of them (tests and tuning).
moe::TileCfg grouped_cfg(const moe_problem* p) {
  switch (p->gemm_kernel) {
    case MOE_GEMM_TILE_32: return moe::TILE_SMALL;
    case MOE_GEMM_TILE_256: return moe::TILE_LARGE;
    case MOE_GEMM_MFMA_256: return moe::TILE_MFMA;  // check_problem: bf16, fits
    default: break;
  }
  if (mfma_fits(p)) return moe::TILE_MFMA;
  const double mean = (double)(p->T * p->K) / p->E;
  return mean <= 48 ? moe::TILE_SMALL : moe::TILE_LARGE;
}

// Dense GEMMs: large tiles unless they would leave CUs idle.  The router (extra gate column,
// column bias) stays on the tile GEMM.
moe::TileCfg dense_cfg(int64_t M, int64_t N) {
  const int64_t bm = moe::tile_bm(moe::TILE_LARGE), bn = moe::tile_bn(moe::TILE_LARGE);
  const bool big = ((M + bm - 1) / bm) * ((N + bn - 1) / bn) >= moe::kCus;
  return big ? moe::TILE_LARGE : moe::TILE_SMALL;
}

// Router: bf16 batches of up to 1024 tokens use the split-K matrix-core router (partial sums
// reduced by the top-K kernel), which keeps the latency of a short batch low.  Longer bf16
// batches of at least 32 output tiles run on the matrix-core GEMM (dense 256 x 256 tiles;
// measured on MI355X: 8192 and 16384 tokens 50 us instead of 105 and 75; at 16 tiles, 4096
// tokens, it was slower than the tile GEMM, 26 vs 20 us) with the reduction split into
// up to 8 slices of at least 4 stages, until about one work-group per CU runs; the top-K
// kernel sums the slices in order and computes the shared-gate logit itself (a dot product of
// the token's row with the gate vector, so no extra output column is needed).  That needs E a
// multiple of 4 and 32-bit operand offsets; otherwise, and for fp32 layers, the tile GEMM
// runs: 32 x 128 tiles with the reduction split (up to 8 slices of at least 8 K steps) until
// two work-groups per CU run; when the 32-row tiles alone exceed that, 256 x 128 tiles split
// until they fill every CU, if they can (fp32 layers unsplit).
bool router_split(const moe_problem* p) { return p->dtype == MOE_DTYPE_BF16 && p->T <= 1024; }

struct RouterTiles {
  moe::TileCfg cfg;
  int ks;
};

bool router_mfma(const moe_problem* p) {
  const int64_t lim = (int64_t)1 << 32;
  const int64_t tiles = ((p->T + 255) / 256) * ((p->E + 255) / 256);
  return p->dtype == MOE_DTYPE_BF16 && p->T > 1024 && tiles >= 32 && p->E % 4 == 0 &&
         p->T * p->D * 2 < lim && (int64_t)p->E * p->D * 2 < lim &&
         p->T * p->E < ((int64_t)1 << 31);
}

RouterTiles router_tiles(const moe_problem* p) {
  const int64_t ncols = p->E + (gated(p) ? 1 : 0);
  if (p->dtype != MOE_DTYPE_BF16) return {dense_cfg(p->T, ncols), 1};
  if (router_mfma(p)) {
    const int64_t tiles = ((p->T + 255) / 256) * ((p->E + 255) / 256);
    const int ns = p->D / 64;  // 64-wide stages of the whole reduction
    int ks = 1;
    while (ks * 2 <= 8 && tiles * ks * 2 <= moe::kCus && ns % (ks * 2) == 0 && ns / (ks * 2) >= 4)
      ks *= 2;
    return {moe::TILE_MFMA, ks};
  }
  const int nk = p->D / 64;  // 64-wide K steps of bf16 rows
  const auto split = [&](int64_t tiles, int64_t slots) {
    int ks = 1;
    while (ks * 2 <= 8 && tiles * ks * 2 <= slots && nk % (ks * 2) == 0 && nk / (ks * 2) >= 8)
      ks *= 2;
    return ks;
  };
  const int64_t nt = (ncols + 127) / 128;
  const int64_t small = (p->T + 31) / 32 * nt, large = (p->T + 255) / 256 * nt;
  const int64_t slots = 2 * moe::kCus;  // 32-row tiles: two work-groups per CU
  if (small < slots) return {moe::TILE_SMALL, split(small, slots)};
  const int ks = split(large, moe::kCus);
  if (large * ks >= moe::kCus) return {moe::TILE_LARGE, ks};
  return {moe::TILE_SMALL, 1};
}

int router_ks(const moe_problem* p) {
  return router_split(p) ? moe::router_kslices(p->T, p->D, p->E, gated(p) ? 1 : 0)
                         : router_tiles(p).ks;
}

// The shared expert's two GEMMs: the matrix-core GEMM (dense 256 x 256 tiles) for bf16
// layers when they fill the chip and every operand fits its 32-bit offsets; the 64-bit tile
// GEMM otherwise.
moe::TileCfg shared_cfg(const moe_problem* p) {
  const moe::TileCfg c = dense_cfg(p->T, (int64_t)2 * p->F_shared);
  return c == moe::TILE_LARGE && mfma_fits_shared(p) ? moe::TILE_MFMA : c;
}

// Workspace layout: every region 256-byte aligned.
struct Layout {
  size_t logits, gate_logit, gate, topk_idx, topk_w, counts, offsets, perm, inv_perm, seg_counts,
      tiles, tile_count, H, Hs, acc, y_perm, y_shared, stats, total;
  int64_t max_mtiles;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Layout layout(const moe_problem* p) {
  Layout L{};
  const int64_t T = p->T, A = p->T * p->K, E = p->E, D = p->D;
  const size_t es = esize(p->dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.max_mtiles = (A + 31) / 32 + (E < A ? E : A);  // upper bound for the smallest BM (32)
  {  // router output: the split-K partial sums [ks][T][E + gated] (small batches) or
     // [ks][T][E] (tile GEMM; the gate logit's partials [ks][T] go to gate_logit)
    const size_t ks = (size_t)router_ks(p);
    const size_t b = ks * (size_t)T * (E + (gated(p) ? 1 : 0)) * 4;
    L.logits = take(b);
    L.gate_logit = take(ks * (size_t)T * 4);
  }
  L.gate = take((size_t)T * 4);
  L.topk_idx = take((size_t)A * 4);
  L.topk_w = take((size_t)A * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.perm = take((size_t)A * 4);
  L.inv_perm = take((size_t)A * 4);
  {  // per-segment histograms, then their sums per chunk of 4 segments
    const size_t nseg = (size_t)moe::dispatch_num_segments(A);
    L.seg_counts = take((nseg + (nseg + 3) / 4) * E * 4);
  }
  L.tiles = take((size_t)L.max_mtiles * moe::kTileStride * 4);
  L.tile_count = take(16);
  L.H = take((size_t)A * p->F * es);
  L.Hs = take((size_t)T * p->F_shared * es);
  if (p->flags & MOE_FLAG_ATOMIC_COMBINE) {
    L.acc = take(p->out_dtype == MOE_DTYPE_F32 ? 0 : (size_t)T * D * 4);
    L.y_perm = L.y_shared = 0;
  } else {
    L.acc = 0;
    // fp32 rows, or fp16 rows (256-byte aligned) followed by their fp32 block factors
    const size_t f32_rows = (size_t)A * D * 4;
    const size_t f16_rows = ((size_t)A * D * 2 + 255) / 256 * 256 +
                            (size_t)A * ((D + moe::kScaleCols - 1) / moe::kScaleCols) * 4;
    L.y_perm = take(f32_rows > f16_rows ? f32_rows : f16_rows);
    L.y_shared = take(has_shared(p) ? (size_t)T * D * 4 : 0);
  }
  L.stats = take((size_t)moe::stats_blocks(T) * (E + 1) * 4);
  L.total = off;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int check_ws(const moe_problem* p, void* ws, size_t bytes, Layout* L) {
  *L = layout(p);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  if (bytes < L->total)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", bytes, L->total);
  return MOE_OK;
}

#define MOE_CHECK_PTR(ptr, name)                                                    \
  do {                                                                              \
    if (!(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);                \
    if (!aligned16(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s not 16-byte aligned", name); \
  } while (0)
#define MOE_CHECK_OPT(ptr, name)                                                    \
  do {                                                                              \
    if ((ptr) && !aligned16(ptr))                                                   \
      return fail(MOE_ERR_INVALID_ARG, "%s not 16-byte aligned", name);              \
  } while (0)

// ---- stage bodies (arguments already validated) -----------------------------------------

// Router logits (and the shared-gate logit), left where launch_topk's arguments say.
hipError_t run_router(const moe_problem* p, const void* x, const moe_weights* w, float* part,
                      float* gate_logit, bool want_gate, moe::TopkArgs* ta, hipStream_t s) {
  const void* gate_w = want_gate ? w->ws_gate : nullptr;
  ta->T = p->T;
  ta->E = p->E;
  ta->K = p->K;
  ta->scoring = p->scoring;
  ta->renorm = !(p->flags & MOE_FLAG_NO_RENORM);
  ta->src = part;
  if (router_split(p)) {
    const int ks = router_ks(p);
    const int64_t ne = p->E + (gate_w ? 1 : 0);
    ta->ks = ks;
    ta->ld = ne;
    ta->slice_stride = p->T * ne;
    ta->gate_src = gate_w ? part + p->E : nullptr;
    ta->gate_ld = ne;
    ta->gate_slice_stride = p->T * ne;
    return moe::launch_router_bf16(x, w->w_router, gate_w, w->logit_bias, p->T, p->D, p->E, ks,
                                   part, s);
  }
  const size_t es = esize(p->dtype);
  moe::GemmParams g{};
  g.A = (const char*)x;
  g.lda_bytes = (int64_t)p->D * es;
  g.B = (const char*)w->w_router;
  g.ldb_bytes = (int64_t)p->D * es;
  g.B2 = (const char*)gate_w;
  g.N = p->E;
  g.Kdim = p->D;
  g.M = (int32_t)p->T;
  g.C = part;
  g.ldc = p->E;
  g.C2 = gate_w ? gate_logit : nullptr;
  g.col_bias = w->logit_bias;
  const RouterTiles rt = router_tiles(p);
  g.k_slices = rt.ks;
  g.c_slice_stride = p->T * p->E;
  g.c2_slice_stride = p->T;
  ta->ks = rt.ks;
  ta->ld = p->E;
  ta->slice_stride = p->T * p->E;
  ta->gate_src = gate_w ? gate_logit : nullptr;
  ta->gate_ld = 1;
  ta->gate_slice_stride = p->T;
  if (rt.cfg == moe::TILE_MFMA) {
    // no extra column: the top-K kernel takes the gate logit from x and the gate vector
    g.B2 = nullptr;
    g.C2 = nullptr;
    ta->gate_src = nullptr;
    ta->gate_x = gate_w ? (const __bf16*)x : nullptr;
    ta->gate_w = (const __bf16*)gate_w;
    ta->D = p->D;
  }
  const int bm = moe::tile_bm(rt.cfg);
  return moe::launch_gemm(p->dtype, rt.cfg, moe::EPI_STORE, g, (p->T + bm - 1) / bm, s);
}

// A grouped GEMM over the tile map.
hipError_t launch_grouped(const moe_problem* p, moe::TileCfg cfg, moe::Epilogue epi,
                          moe::GemmParams g, const int32_t* tiles, const int32_t* tile_count,
                          int64_t max_mtiles, hipStream_t s) {
  g.tiles = tiles;
  g.tile_count = tile_count;
  g.rows_bound = (int32_t)p->T;  // an expert receives at most one row per token
  return moe::launch_gemm(p->dtype, cfg, epi, g, max_mtiles, s);
}

hipError_t run_gate_up(const moe_problem* p, const void* x, const void* x_perm, const void* w_gu,
                       const int32_t* perm, const int32_t* tiles, const int32_t* tile_count,
                       int64_t max_mtiles, void* H, moe::TileCfg plan, hipStream_t s) {
  const size_t es = esize(p->dtype);
  moe::GemmParams g{};
  g.A = (const char*)(x_perm ? x_perm : x);
  g.lda_bytes = (int64_t)p->D * es;
  g.a_gather = x_perm ? nullptr : perm;
  g.a_div = p->K;
  g.B = (const char*)w_gu;
  g.b_group_bytes = (int64_t)2 * p->F * p->D * es;
  g.ldb_bytes = (int64_t)p->D * es;
  g.N = p->F;
  g.Kdim = p->D;
  g.C = H;
  g.ldc = p->F;
  return launch_grouped(p, plan, moe::EPI_SWIGLU, g, tiles, tile_count, max_mtiles, s);
}

hipError_t run_down(const moe_problem* p, const void* H, const void* w_d, const int32_t* tiles,
                    const int32_t* tile_count, int64_t max_mtiles, moe::TileCfg plan,
                    void* y_perm, float* acc, const int32_t* perm, const float* topk_w,
                    hipStream_t s, float* y_scale = nullptr) {
  const size_t es = esize(p->dtype);
  moe::GemmParams g{};
  g.A = (const char*)H;
  g.lda_bytes = (int64_t)p->F * es;
  g.B = (const char*)w_d;
  g.b_group_bytes = (int64_t)p->D * p->F * es;
  g.ldb_bytes = (int64_t)p->F * es;
  g.N = p->D;
  g.Kdim = p->F;
  if (y_perm) {
    g.C = y_perm;
    g.ldc = p->D;
    g.c_scale = y_scale;  // fp16 rows with block factors (see compact_rows)
    g.ldcs = (p->D + moe::kScaleCols - 1) / moe::kScaleCols;
    return launch_grouped(p, plan, moe::EPI_STORE, g, tiles, tile_count, max_mtiles, s);
  }
  g.acc_out = acc;
  g.ldo = p->D;
  g.perm = perm;
  g.topk_w = topk_w;
  g.topk = p->K;
  return launch_grouped(p, plan, moe::EPI_ATOMIC_COMBINE, g, tiles, tile_count, max_mtiles, s);
}

// Whether moe_forward keeps the routed expert rows (y_perm) as fp16 with a power-of-two factor
// per row and 128-column block instead of fp32: for bf16 layers whose grouped GEMM is the
// matrix-core kernel (the only one with that epilogue).  Half the bytes of the down GEMM's
// stores and of the combine's reads; the factor keeps every value below 2^15, so nothing
// overflows, and the 11-bit significand adds about 2^-12 of a block's largest value, far
// below the bf16 rounding of H.
bool compact_rows(const moe_problem* p, moe::TileCfg plan) {
  return p->dtype == MOE_DTYPE_BF16 && plan == moe::TILE_MFMA;
}

// Shared expert on all T tokens: Hs = SwiGLU gate/up of x; out = row_scale * (Hs Ws_downᵀ), as
// fp32 rows, or (out_scale, matrix-core GEMM only) fp16 rows with one power-of-two factor per
// row and 128-column block in out_scale [T, ceil(D / 128)].
hipError_t run_shared(const moe_problem* p, const void* x, const moe_weights* w, void* Hs,
                      void* out, const float* row_scale, hipStream_t s,
                      float* out_scale = nullptr) {
  const size_t es = esize(p->dtype);
  const moe::TileCfg cfg = shared_cfg(p);
  const int bm = moe::tile_bm(cfg);
  const int64_t mt = (p->T + bm - 1) / bm;
  moe::GemmParams g{};
  g.A = (const char*)x;
  g.lda_bytes = (int64_t)p->D * es;
  g.B = (const char*)w->ws_gate_up;
  g.ldb_bytes = (int64_t)p->D * es;
  g.N = p->F_shared;
  g.Kdim = p->D;
  g.M = (int32_t)p->T;
  g.C = Hs;
  g.ldc = p->F_shared;
  hipError_t e = moe::launch_gemm(p->dtype, cfg, moe::EPI_SWIGLU, g, mt, s);
  if (e != hipSuccess) return e;
  moe::GemmParams d{};
  d.A = (const char*)Hs;
  d.lda_bytes = (int64_t)p->F_shared * es;
  d.B = (const char*)w->ws_down;
  d.ldb_bytes = (int64_t)p->F_shared * es;
  d.N = p->D;
  d.Kdim = p->F_shared;
  d.M = (int32_t)p->T;
  d.C = out;
  d.ldc = p->D;
  d.row_scale = row_scale;
  d.c_scale = out_scale;
  d.ldcs = (p->D + moe::kScaleCols - 1) / moe::kScaleCols;
  return moe::launch_gemm(p->dtype, cfg, moe::EPI_STORE, d, mt, s);
}

int check_weights(const moe_problem* p, const moe_weights* w, bool router, bool experts) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (router) {
    MOE_CHECK_PTR(w->w_router, "w_router");
    MOE_CHECK_OPT(w->logit_bias, "logit_bias");
    MOE_CHECK_OPT(w->select_bias, "select_bias");
    if (gated(p)) MOE_CHECK_PTR(w->ws_gate, "ws_gate");
  }
  if (experts) {
    MOE_CHECK_PTR(w->w_gate_up, "w_gate_up");
    MOE_CHECK_PTR(w->w_down, "w_down");
    if (has_shared(p)) {
      MOE_CHECK_PTR(w->ws_gate_up, "ws_gate_up");
      MOE_CHECK_PTR(w->ws_down, "ws_down");
    }
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_describe_plan(const moe_problem* p) {
  static thread_local std::string text;
  text.clear();
  g_last_error.clear();
  if (check_problem(p)) return text.c_str();
  auto name = [](moe::TileCfg c) -> std::string {
    const char* kind = c == moe::TILE_MFMA ? "mfma " : "tile ";
    return std::string(kind) + std::to_string(moe::tile_bm(c)) + "x" +
           std::to_string(moe::tile_bn(c));
  };
  const std::string router =
      router_split(p)
          ? "split-K mfma 16x64, " + std::to_string(router_ks(p)) + " K slice(s)"
          : name(router_tiles(p).cfg) + ", " + std::to_string(router_tiles(p).ks) + " K slice(s)" +
                (router_tiles(p).cfg == moe::TILE_MFMA && gated(p) ? ", gate logit in top-K"
                                                                   : "");
  text = "router: " + router + "; dispatch: " +
         (moe::dispatch_fused(p->T * p->K, p->E, p->dispatch_kernel) ? "one work-group"
                                                                      : "count, then scan+scatter") +
         "; grouped gate_up/down: " + name(grouped_cfg(p));
  if (has_shared(p)) text += "; shared: " + name(shared_cfg(p));
  text += (p->flags & MOE_FLAG_ATOMIC_COMBINE)
              ? "; combine: fp32 atomics in the down epilogue"
              : compact_rows(p, grouped_cfg(p))
                    ? (has_shared(p) && shared_cfg(p) == moe::TILE_MFMA
                           ? "; combine: gather in slot order over fp16 rows with block factors "
                             "(routed and shared)"
                           : "; combine: gather in slot order over fp16 rows with block factors")
                    : "; combine: gather in slot order";
  return text.c_str();
}

int moe_workspace_size(const moe_problem* p, size_t* bytes) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout(p).total;
  return MOE_OK;
}

int moe_route(const moe_problem* p, const void* x, const moe_weights* w, moe_routing* r,
              void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  MOE_CHECK_PTR(x, "x");
  if ((st = check_weights(p, w, true, false))) return st;
  if (!r) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  MOE_CHECK_PTR(r->topk_idx, "topk_idx");
  MOE_CHECK_PTR(r->topk_w, "topk_w");
  MOE_CHECK_OPT(r->logits, "logits");
  MOE_CHECK_OPT(r->shared_gate, "shared_gate");
  MOE_CHECK_OPT(r->select_keys, "select_keys");
  Layout L;
  if ((st = check_ws(p, workspace, workspace_bytes, &L))) return st;
  hipStream_t s = (hipStream_t)stream;
  const bool want_gate = gated(p) && r->shared_gate;
  moe::TopkArgs ta{};
  MOE_HIP_TRY(run_router(p, x, w, at<float>(workspace, L.logits),
                         at<float>(workspace, L.gate_logit), want_gate, &ta, s),
              "router GEMM launch");
  ta.idx = r->topk_idx;
  ta.w = r->topk_w;
  ta.logits_out = r->logits;
  ta.keys_out = r->select_keys;
  ta.gate_out = want_gate ? r->shared_gate : nullptr;
  ta.sel_bias = w->select_bias;
  MOE_HIP_TRY(moe::launch_topk(ta, s), "top-K launch");
  return MOE_OK;
}

int moe_route_logits(const moe_problem* p, const float* logits, const float* select_bias,
                     moe_routing* r, moe_stream_t stream) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  MOE_CHECK_PTR(logits, "logits");
  MOE_CHECK_OPT(select_bias, "select_bias");
  if (!r) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  MOE_CHECK_PTR(r->topk_idx, "topk_idx");
  MOE_CHECK_PTR(r->topk_w, "topk_w");
  MOE_CHECK_OPT(r->select_keys, "select_keys");
  moe::TopkArgs ta{};
  ta.src = logits;
  ta.keys_out = r->select_keys;
  ta.ks = 1;
  ta.ld = p->E;
  ta.T = p->T;
  ta.E = p->E;
  ta.K = p->K;
  ta.scoring = p->scoring;
  ta.renorm = !(p->flags & MOE_FLAG_NO_RENORM);
  ta.idx = r->topk_idx;
  ta.w = r->topk_w;
  ta.sel_bias = select_bias;
  MOE_HIP_TRY(moe::launch_topk(ta, (hipStream_t)stream), "top-K launch");
  return MOE_OK;
}

int moe_router_stats(const moe_problem* p, const float* logits, const int32_t* expert_counts,
                     float* stats, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  MOE_CHECK_PTR(logits, "logits");
  MOE_CHECK_PTR(expert_counts, "expert_counts");
  MOE_CHECK_PTR(stats, "stats");
  Layout L;
  if ((st = check_ws(p, workspace, workspace_bytes, &L))) return st;
  float* part = at<float>(workspace, L.stats);
  float* zpart = part + moe::stats_blocks(p->T) * p->E;
  MOE_HIP_TRY(moe::launch_router_stats(logits, expert_counts, p->T, p->E, p->scoring, part, zpart,
                                       stats, (hipStream_t)stream),
              "router statistics launch");
  return MOE_OK;
}

int moe_update_select_bias(const moe_problem* p, const int32_t* expert_counts,
                           float* select_bias, float gamma, moe_stream_t stream) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  MOE_CHECK_PTR(expert_counts, "expert_counts");
  MOE_CHECK_PTR(select_bias, "select_bias");
  MOE_HIP_TRY(moe::launch_update_select_bias(expert_counts, p->E, select_bias, gamma,
                                             (hipStream_t)stream),
              "bias update launch");
  return MOE_OK;
}

int moe_dispatch(const moe_problem* p, const void* x, moe_routing* r, void* x_perm,
                 void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  if (!r) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  MOE_CHECK_PTR(r->topk_idx, "topk_idx");
  MOE_CHECK_PTR(r->expert_counts, "expert_counts");
  MOE_CHECK_PTR(r->expert_offsets, "expert_offsets");
  MOE_CHECK_PTR(r->perm, "perm");
  MOE_CHECK_PTR(r->inv_perm, "inv_perm");
  MOE_CHECK_OPT(x_perm, "x_perm");
  if (x_perm) MOE_CHECK_PTR(x, "x");
  Layout L;
  if ((st = check_ws(p, workspace, workspace_bytes, &L))) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t A = p->T * p->K;
  MOE_HIP_TRY(moe::launch_dispatch(r->topk_idx, A, p->E, at<int32_t>(workspace, L.seg_counts),
                                   r->expert_counts, r->expert_offsets, r->perm, r->inv_perm,
                                   capacity(p), p->dispatch_kernel, 0, nullptr, nullptr, s),
              "dispatch launch");
  if (x_perm)
    MOE_HIP_TRY(moe::launch_gather_rows(x, p->D, (int)esize(p->dtype), r->perm, r->expert_offsets,
                                        p->E, p->K, A, x_perm, s),
                "row gather launch");
  return MOE_OK;
}

int moe_experts(const moe_problem* p, const void* x, const void* x_perm, const moe_weights* w,
                const moe_routing* r, float* y_perm, float* y_shared, void* workspace,
                size_t workspace_bytes, moe_stream_t stream) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  if ((st = check_weights(p, w, false, true))) return st;
  if (!x && !x_perm) return fail(MOE_ERR_INVALID_ARG, "x and x_perm are both NULL");
  MOE_CHECK_OPT(x, "x");
  MOE_CHECK_OPT(x_perm, "x_perm");
  if (has_shared(p) && y_shared) MOE_CHECK_PTR(x, "x");
  if (!r) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  MOE_CHECK_PTR(r->expert_offsets, "expert_offsets");
  if (!x_perm) MOE_CHECK_PTR(r->perm, "perm");
  MOE_CHECK_PTR(y_perm, "y_perm");
  MOE_CHECK_OPT(y_shared, "y_shared");
  Layout L;
  if ((st = check_ws(p, workspace, workspace_bytes, &L))) return st;
  hipStream_t s = (hipStream_t)stream;
  const moe::TileCfg plan = grouped_cfg(p);
  int32_t* tiles = at<int32_t>(workspace, L.tiles);
  int32_t* tile_count = at<int32_t>(workspace, L.tile_count);
  MOE_HIP_TRY(moe::launch_tile_map(r->expert_offsets, p->E, moe::tile_bm(plan), tiles, tile_count,
                                   s),
              "tile map launch");
  void* H = at<void>(workspace, L.H);
  MOE_HIP_TRY(run_gate_up(p, x, x_perm, w->w_gate_up, r->perm, tiles, tile_count, L.max_mtiles, H,
                          plan, s),
              "gate_up GEMM launch");
  MOE_HIP_TRY(run_down(p, H, w->w_down, tiles, tile_count, L.max_mtiles, plan, y_perm, nullptr,
                       nullptr, nullptr, s),
              "down GEMM launch");
  if (has_shared(p) && y_shared)
    MOE_HIP_TRY(run_shared(p, x, w, at<void>(workspace, L.Hs), y_shared, nullptr, s),
                "shared expert launch");
  return MOE_OK;
}

int moe_combine(const moe_problem* p, const float* y_perm, const moe_routing* r,
                const float* y_shared, void* out, moe_stream_t stream) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  MOE_CHECK_PTR(y_perm, "y_perm");
  MOE_CHECK_PTR(out, "out");
  MOE_CHECK_OPT(y_shared, "y_shared");
  if (!r) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  MOE_CHECK_PTR(r->inv_perm, "inv_perm");
  MOE_CHECK_PTR(r->topk_w, "topk_w");
  const float* gate = nullptr;
  if (y_shared && gated(p)) {
    MOE_CHECK_PTR(r->shared_gate, "shared_gate");
    gate = r->shared_gate;
  }
  MOE_HIP_TRY(moe::launch_combine(y_perm, r->inv_perm, r->topk_w, has_shared(p) ? y_shared : nullptr,
                                  gate, p->T, p->K, p->D, out, p->out_dtype, (hipStream_t)stream),
              "combine launch");
  return MOE_OK;
}

}  // extern "C"

namespace {

int forward_impl(const moe_problem* p, const void* x, const moe_weights* w, moe_routing* r_opt,
                 void* out, void* workspace, size_t workspace_bytes, moe_stream_t stream,
                 void* const* events) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  MOE_CHECK_PTR(x, "x");
  MOE_CHECK_PTR(out, "out");
  if (out == x) return fail(MOE_ERR_INVALID_ARG, "out aliases x");
  if ((st = check_weights(p, w, true, true))) return st;
  moe_routing r{};
  if (r_opt) {
    r = *r_opt;
    MOE_CHECK_OPT(r.logits, "logits");
    MOE_CHECK_OPT(r.topk_idx, "topk_idx");
    MOE_CHECK_OPT(r.topk_w, "topk_w");
    MOE_CHECK_OPT(r.expert_counts, "expert_counts");
    MOE_CHECK_OPT(r.expert_offsets, "expert_offsets");
    MOE_CHECK_OPT(r.perm, "perm");
    MOE_CHECK_OPT(r.inv_perm, "inv_perm");
    MOE_CHECK_OPT(r.shared_gate, "shared_gate");
    MOE_CHECK_OPT(r.select_keys, "select_keys");
  }
  Layout L;
  if ((st = check_ws(p, workspace, workspace_bytes, &L))) return st;
  void* ws = workspace;
  if (!r.topk_idx) r.topk_idx = at<int32_t>(ws, L.topk_idx);
  if (!r.topk_w) r.topk_w = at<float>(ws, L.topk_w);
  if (!r.expert_counts) r.expert_counts = at<int32_t>(ws, L.counts);
  if (!r.expert_offsets) r.expert_offsets = at<int32_t>(ws, L.offsets);
  if (!r.perm) r.perm = at<int32_t>(ws, L.perm);
  if (!r.inv_perm) r.inv_perm = at<int32_t>(ws, L.inv_perm);
  if (!r.shared_gate) r.shared_gate = at<float>(ws, L.gate);

  hipStream_t s = (hipStream_t)stream;
  const int64_t A = p->T * p->K;
  const bool g = gated(p);
  float* gate_logit = at<float>(ws, L.gate_logit);
  auto mark = [&](int stage) -> hipError_t {
    return events && events[stage] ? hipEventRecord((hipEvent_t)events[stage], s) : hipSuccess;
  };

  // 1. router GEMM (+ shared-gate column) and top-K
  MOE_HIP_TRY(mark(MOE_STAGE_ROUTER), "event record");
  moe::TopkArgs ta{};
  MOE_HIP_TRY(run_router(p, x, w, at<float>(ws, L.logits), gate_logit, g, &ta, s),
              "router GEMM launch");
  MOE_HIP_TRY(mark(MOE_STAGE_TOPK), "event record");
  ta.idx = r.topk_idx;
  ta.w = r.topk_w;
  ta.logits_out = r.logits;  // only if the caller asked for them
  ta.keys_out = r.select_keys;
  ta.gate_out = g ? r.shared_gate : nullptr;
  ta.sel_bias = w->select_bias;
  MOE_HIP_TRY(moe::launch_topk(ta, s), "top-K launch");
  // 2. dispatch + tile map
  const moe::TileCfg plan = grouped_cfg(p);
  int32_t* tiles = at<int32_t>(ws, L.tiles);
  int32_t* tile_count = at<int32_t>(ws, L.tile_count);
  MOE_HIP_TRY(mark(MOE_STAGE_DISPATCH), "event record");
  MOE_HIP_TRY(moe::launch_dispatch(r.topk_idx, A, p->E, at<int32_t>(ws, L.seg_counts),
                                   r.expert_counts, r.expert_offsets, r.perm, r.inv_perm,
                                   capacity(p), p->dispatch_kernel, moe::tile_bm(plan), tiles,
                                   tile_count, s),
              "dispatch launch");
  // 3. routed gate_up with SiLU*up
  void* H = at<void>(ws, L.H);
  MOE_HIP_TRY(mark(MOE_STAGE_GATE_UP), "event record");
  MOE_HIP_TRY(run_gate_up(p, x, nullptr, w->w_gate_up, r.perm, tiles, tile_count, L.max_mtiles, H,
                          plan, s),
              "gate_up GEMM launch");
  const float* gate = g ? r.shared_gate : nullptr;
  if (!(p->flags & MOE_FLAG_ATOMIC_COMBINE)) {
    // 4. shared expert and routed down into row buffers, then the gather combine.  With fp16
    //    routed rows the shared rows are fp16 with block factors too when the matrix-core GEMM
    //    runs the shared expert (its epilogue makes them): half the bytes of the shared
    //    expert's store and of the combine's read of it
    float* y_perm = at<float>(ws, L.y_perm);
    void* y_shared = has_shared(p) ? at<void>(ws, L.y_shared) : nullptr;
    float* ys_scale = nullptr;
    if (y_shared && compact_rows(p, plan) && shared_cfg(p) == moe::TILE_MFMA)
      ys_scale = reinterpret_cast<float*>(static_cast<char*>(y_shared) +
                                          ((p->T * p->D * 2 + 255) / 256) * 256);
    MOE_HIP_TRY(mark(MOE_STAGE_SHARED), "event record");
    if (y_shared)
      MOE_HIP_TRY(run_shared(p, x, w, at<void>(ws, L.Hs), y_shared, nullptr, s, ys_scale),
                  "shared expert launch");
    MOE_HIP_TRY(mark(MOE_STAGE_DOWN), "event record");
    if (compact_rows(p, plan)) {
      // fp16 rows [A, D], then the fp32 block factors [A, ceil(D / kScaleCols)] (256-byte
      // aligned)
      const int nblk = (p->D + moe::kScaleCols - 1) / moe::kScaleCols;
      float* y_scale = reinterpret_cast<float*>(
          reinterpret_cast<char*>(y_perm) + ((A * p->D * 2 + 255) / 256) * 256);
      MOE_HIP_TRY(run_down(p, H, w->w_down, tiles, tile_count, L.max_mtiles, plan, y_perm,
                           nullptr, nullptr, nullptr, s, y_scale),
                  "down GEMM launch");
      MOE_HIP_TRY(mark(MOE_STAGE_FINAL), "event record");
      MOE_HIP_TRY(moe::launch_combine16(y_perm, y_scale, nblk, r.inv_perm, r.topk_w, y_shared,
                                        ys_scale, gate, p->T, p->K, p->D, out, p->out_dtype, s),
                  "combine launch");
    } else {
      MOE_HIP_TRY(run_down(p, H, w->w_down, tiles, tile_count, L.max_mtiles, plan, y_perm,
                           nullptr, nullptr, nullptr, s),
                  "down GEMM launch");
      MOE_HIP_TRY(mark(MOE_STAGE_FINAL), "event record");
      MOE_HIP_TRY(moe::launch_combine(y_perm, r.inv_perm, r.topk_w,
                                      static_cast<const float*>(y_shared), gate, p->T, p->K, p->D,
                                      out, p->out_dtype, s),
                  "combine launch");
    }
    MOE_HIP_TRY(mark(MOE_STAGE_COUNT), "event record");
    return MOE_OK;
  }
  // 4'. atomic mode: the shared branch initialises an fp32 accumulator (or it is zeroed), the
  //     down GEMM adds the weighted routed rows with atomics, then one cast to the output dtype.
  float* acc = p->out_dtype == MOE_DTYPE_F32 ? static_cast<float*>(out) : at<float>(ws, L.acc);
  MOE_HIP_TRY(mark(MOE_STAGE_SHARED), "event record");
  if (has_shared(p))
    MOE_HIP_TRY(run_shared(p, x, w, at<void>(ws, L.Hs), acc, gate, s), "shared expert launch");
  else
    MOE_HIP_TRY(moe::launch_zero(acc, p->T * p->D, s), "zero launch");
  MOE_HIP_TRY(mark(MOE_STAGE_DOWN), "event record");
  MOE_HIP_TRY(run_down(p, H, w->w_down, tiles, tile_count, L.max_mtiles, plan, nullptr, acc,
                       r.perm, r.topk_w, s),
              "down GEMM launch");
  MOE_HIP_TRY(mark(MOE_STAGE_FINAL), "event record");
  if (p->out_dtype != MOE_DTYPE_F32)
    MOE_HIP_TRY(moe::launch_cast(acc, out, p->T * p->D, p->out_dtype, s), "cast launch");
  MOE_HIP_TRY(mark(MOE_STAGE_COUNT), "event record");
  return MOE_OK;
}

// Scratch of moe_forward_noalloc: one copy per GPU (a device global lives in each device's
// copy of the code object).  In host code `scratch` names a host-side stand-in, not device
// memory, so it is never passed to a kernel or a copy: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  MOE_HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    MOE_HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const moe_problem* p, const void* x, const moe_weights* w,
                        moe_routing* r_opt, void* out, moe_stream_t stream) {
  g_last_error.clear();
  int st = check_problem(p);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  const size_t need = layout(p).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "problem needs %zu bytes of workspace, more than the %zu-byte scratch of "
                "moe_forward_noalloc (use moe_forward with a workspace)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return forward_impl(p, x, w, r_opt, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_forward(const moe_problem* p, const void* x, const moe_weights* w, moe_routing* r_opt,
                void* out, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  return forward_impl(p, x, w, r_opt, out, workspace, workspace_bytes, stream, nullptr);
}

int moe_forward_timed(const moe_problem* p, const void* x, const moe_weights* w,
                      moe_routing* r_opt, void* out, void* workspace, size_t workspace_bytes,
                      moe_stream_t stream, void* const* events) {
  if (!events) {
    g_last_error.clear();
    return fail(MOE_ERR_INVALID_ARG, "events is NULL");
  }
  return forward_impl(p, x, w, r_opt, out, workspace, workspace_bytes, stream, events);
}

}  // extern "C"
