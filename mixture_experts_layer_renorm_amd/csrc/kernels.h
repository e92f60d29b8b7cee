// Internal declarations shared by the HIP translation units and the host API layer.
// Nothing here is part of the public ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kXcds = 8;         // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kCus = 256;
constexpr int kTileStride = 8;   // int32 words per tile-map entry

// Reads a word that is the same for the whole work-group and is not written while the kernel
// runs (tile maps and counts, produced by an earlier launch) through the scalar cache.  Read
// with a vector load instead, the compiler's next wait on the vector-memory counter would also
// wait for every weight load in flight.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Grouped / dense GEMM description.  C[row, n] = sum_k A[row, k] * B[n, k]; rows come from
// per-group row ranges (tile map) or one dense range [0, M).
enum Epilogue : int {
  EPI_STORE = 0,           // fp32 store (+ column bias, x row scale); column N goes to C2
  EPI_SWIGLU = 1,          // H[row, n] = SiLU(C[row, n]) * C[row, F + n], stored in dtype
  EPI_ATOMIC_COMBINE = 2,  // out_acc[token(row), n] += w(row) * C[row, n]  (fp32 atomics)
};

// Columns per power-of-two factor of fp16 expert rows (GemmParams::c_scale, combine16).
constexpr int kScaleCols = 128;

struct GemmParams {
  // A operand: row r of the logical A matrix is A + arow(r) * lda_bytes.
  const char* A;
  int64_t lda_bytes;
  const int32_t* a_gather;  // if non-null: arow(pos) = a_gather[pos] / a_div
  int32_t a_div;
  // B operand: [groups][rows][Kdim]; group stride in bytes.
  const char* B;
  int64_t b_group_bytes;
  int64_t ldb_bytes;
  const char* B2;           // optional extra B row, output column N (router's shared-gate column)
  int32_t N;                // output columns per group (SWIGLU: F, B has 2F rows)
  int32_t Kdim;             // reduction length, elements
  // Tiles: map mode (tiles != null) or dense mode over M rows.
  const int32_t* tiles;
  const int32_t* tile_count;
  int32_t M;
  int32_t rows_bound;       // map mode: an upper bound on any tile's rows, or <= 0 if unknown
  // Epilogue operands.
  void* C;                  // STORE: fp32 [rows, ldc] (or fp16 with c_scale); SWIGLU: dtype
  int64_t ldc;
  float* c_scale;           // STORE, streaming and matrix-core GEMMs only: if set, C holds fp16
                            // values scaled by a power of two per block of kScaleCols columns
                            // of a row (block max < 2^15), and c_scale[row * ldcs + b] the
                            // factor that restores block b of row `row`
  int64_t ldcs;
  float* C2;                // STORE: column N (if B2) -> C2[row]
  const float* col_bias;    // STORE: + col_bias[n]
  int32_t k_slices;         // tile GEMM, dense STORE: split the reduction into this many
                            // equal slices (<= 1: none); slice z writes its partial sums to
                            // C + z * c_slice_stride and C2 + z * c2_slice_stride (col_bias
                            // in slice 0 only)
  int64_t c_slice_stride, c2_slice_stride;
  const float* row_scale;   // STORE: * row_scale[row]
  float* acc_out;           // ATOMIC: [tokens, ldo]
  int64_t ldo;
  const int32_t* perm;      // ATOMIC: assignment id of each row (position)
  const float* topk_w;      // ATOMIC: routing weight of each assignment id
  int32_t topk;             // ATOMIC: K (token = assignment id / K)
};

// Tile configurations (BM x BN output tiles).
enum TileCfg : int {
  TILE_SMALL = 0,       // tile GEMM, BM=32,  BN=128
  TILE_LARGE = 1,       // tile GEMM, BM=256, BN=128
  TILE_MFMA = 2,        // matrix-core GEMM, 256 x 256 tiles, bf16 only, no B2; col_bias and
                        // k_slices for dense fp32 rows only
};
int tile_bm(TileCfg cfg);
int tile_bn(TileCfg cfg);

// Matrix-core grouped or dense GEMM (256 x 256 tiles), bf16.
hipError_t launch_mfma_gemm(Epilogue epi, const GemmParams& p, int64_t max_mtiles,
                            hipStream_t stream);

// dtype: 0 = fp32, 1 = bf16.  Returns hipSuccess or the launch error.
hipError_t launch_gemm(int dtype, TileCfg cfg, Epilogue epi, const GemmParams& p, int64_t max_tiles,
                       hipStream_t stream);

// Router top-K.  The logit of (t, e) is the sum, in slice order, of src[q * slice_stride +
// t * ld + e] over q < ks (ks = 1: src is the logits matrix).  Writes idx/w [T, K]; optionally
// the summed logits [T, E] to logits_out, the selection keys [T, E] (the logit, or with
// sel_bias the fp32 score + bias) to keys_out, and sigmoid of the gate logit (same summation
// over gate_src[q * gate_slice_stride + t * gate_ld], or the dot product of gate_x[t] and
// gate_w when gate_x is set) to gate_out [T].
struct TopkArgs {
  const float* src;
  int ks;
  int64_t slice_stride;
  int64_t ld;
  int64_t T;
  int E, K, scoring, renorm;
  int32_t* idx;
  float* w;
  float* logits_out;
  float* keys_out;
  const float* gate_src;
  int64_t gate_ld;
  int64_t gate_slice_stride;
  float* gate_out;
  const __bf16* gate_x;   // if set (bf16 layers): the gate logit is x[t] . gate_w over D,
  const __bf16* gate_w;   // computed here instead of read from gate_src
  int D;
  const float* sel_bias;  // [E] or null: choose on score + bias, weight with the score
};
hipError_t launch_update_select_bias(const int32_t* counts, int E, float* bias, float gamma,
                                     hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

// Router logits from bf16 x [T, D] and W_r [E, D] (+ gate row [D]): K split into ks slices,
// part [ks][T][E + gated] fp32, bias added in slice 0.
int router_kslices(int64_t T, int D, int E, int gated);
hipError_t launch_router_bf16(const void* x, const void* w_router, const void* w_gate,
                              const float* bias, int64_t T, int D, int E, int ks, float* part,
                              hipStream_t stream);

// Dispatch.  path: 0 = automatic, 1 = one work-group, 2 = count then scan + scatter (the
// moe_dispatch_kernel values).
constexpr int kDispatchOneWgMaxE = 768;  // LDS of the one-work-group kernel: 17 ints per expert
int dispatch_segment_len(int64_t A);
int64_t dispatch_num_segments(int64_t A);
bool dispatch_supported(int E, int path);
// True when launch_dispatch runs as one work-group.
bool dispatch_fused(int64_t A, int E, int path);
// cap: rows each expert keeps (its first cap assignments in ascending id; the others get
// inv_perm = -1 and are not counted); INT32_MAX for none.  With tiles non-null, the tile map
// of the grouped GEMMs (M tiles of up to bm rows, one map entry each) goes to tiles and its
// size to tile_count[0].
hipError_t launch_dispatch(const int32_t* idx, int64_t A, int E, int32_t* seg_counts,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                           int cap, int path, int bm, int32_t* tiles, int32_t* tile_count,
                           hipStream_t stream);
// Tile map from offsets alone (staged API).
hipError_t launch_tile_map(const int32_t* offsets, int E, int bm, int32_t* tiles,
                           int32_t* tile_count, hipStream_t stream);
hipError_t launch_gather_rows(const void* x, int64_t D, int esize, const int32_t* perm,
                              const int32_t* offsets, int E, int K, int64_t A, void* x_perm,
                              hipStream_t stream);

// Router statistics: out [2E + 4] = f [E], P [E], N·Σ f P, z-loss, load CV, max/mean load.
// part [stats_blocks(T)][E] and zpart [stats_blocks(T)] are scratch.
int64_t stats_blocks(int64_t T);
hipError_t launch_router_stats(const float* logits, const int32_t* counts, int64_t T, int E,
                               int scoring, float* part, float* zpart, float* out,
                               hipStream_t stream);

__device__ __forceinline__ float wave_max_abs(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Power-of-two scale of one block of values for fp16 storage: s with max|v| * s < 2^15 (so
// no value overflows fp16) and its exact inverse.  max_abs = 0 gives s = 2^15.
__device__ __forceinline__ void f16_block_scale(float max_abs, float* s, float* inv) {
  int ex = 0;
  (void)frexpf(max_abs, &ex);  // max_abs = f * 2^ex with f in [0.5, 1)
  int e = 15 - ex;
  e = e < -126 ? -126 : (e > 126 ? 126 : e);
  *s = ldexpf(1.0f, e);
  *inv = ldexpf(1.0f, -e);
}

// Combine / finalize.
hipError_t launch_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w,
                          const float* y_shared, const float* gate, int64_t T, int K, int D,
                          void* out, int out_dtype, hipStream_t stream);
// The same combine over fp16 expert rows y16 [T*K, D] with block factors ysc [T*K, nblk]
// (nblk = ceil(D / kScaleCols)); each term is (topk_w * factor) * value, summed in slot order.
// The shared rows y_shared [T, D] are fp32, or fp16 with block factors ys_sc [T, nblk] when
// ys_sc is non-null.
hipError_t launch_combine16(const void* y16, const float* ysc, int nblk, const int32_t* inv_perm,
                            const float* topk_w, const void* y_shared, const float* ys_sc,
                            const float* gate, int64_t T, int K, int D, void* out, int out_dtype,
                            hipStream_t stream);
hipError_t launch_cast(const float* src, void* dst, int64_t n, int out_dtype, hipStream_t stream);
hipError_t launch_zero(float* dst, int64_t n, hipStream_t stream);

}  // namespace moe
