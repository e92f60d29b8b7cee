// Grouped / dense GEMM on gfx950 matrix cores, with the epilogues the MoE layer needs.
//
// One kernel template serves every contraction of the layer:
//   router      C = x W_rᵀ (+ the shared-gate column w_s), fp32 logits      ("MoE" §2 Router)
//   gate_up     H = SiLU(X_e W_gateᵀ) ⊙ (X_e W_upᵀ) per expert, rows gathered through the
//               dispatch permutation                                          ("MoE" §3 eq. E_e)
//   down        y = H W_downᵀ per expert; the epilogue scales each row by its routing weight
//               and adds it into the token's fp32 accumulator                 ("MoE" §3.2, §4)
//   shared      the same gate_up/down on all T tokens, gate applied as a row scale (§4)
//
// Design (gfx950, wave64):
//  * 256 threads = 4 waves arranged WM x WN over a BM x BN output tile.
//  * K advances 128 bytes of every row per step (64 bf16 or 32 fp32 elements).  Global loads are
//    16-byte vectors, staged through registers into a double-buffered LDS tile whose rows are
//    padded to 144 bytes, so the 16 rows read by one MFMA operand fetch hit distinct banks.
//  * bf16: v_mfma_f32_16x16x32_bf16 (lane l holds row l%16, k = 8*(l/16)..+7 of each operand;
//    result rows 4*(l/16)..+3, column l%16).  fp32: v_mfma_f32_16x16x4_f32, eight per 32-wide k
//    slice, the k order permuted identically for both operands.
//  * 16-row and 16-column sub-tiles that lie wholly outside the valid rows/columns are skipped,
//    so a group with 2 rows costs one 16-row MFMA slice, not BM.
//  * Persistent, XCD-aware schedule: work-group b runs on XCD b % 8; each XCD owns one
//    contiguous eighth of the logical tile sequence, which is ordered expert-major, then by
//    N tile, then by M tile.  Tiles that share an expert's weights or rows therefore run at the
//    same time on the same XCD and meet in its L2.
#include "kernels.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowBytes = 128;  // bytes of each row consumed per K step
constexpr int kPitch = 144;     // LDS bytes per staged row

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

template <typename T>
__device__ __forceinline__ T to_out(float v);
template <>
__device__ __forceinline__ float to_out<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 to_out<__bf16>(float v) { return (__bf16)v; }

template <typename T, int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(256) gemm_kernel(const GemmParams p) {
  static_assert(WM * WN == 4, "4 waves");
  constexpr int ACH = BM / 32;  // 16-byte chunks per thread per K step, A tile
  constexpr int BCH = BN / 32;  // same, B tile
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 16, NI = WTN / 16;
  constexpr bool kF32 = sizeof(T) == 4;
  constexpr int KE = kRowBytes / (int)sizeof(T);
  constexpr bool kSwiglu = EPI == EPI_SWIGLU;
  static_assert(!kSwiglu || (NI % 2 == 0), "SwiGLU pairs gate and up sub-tiles");

  __shared__ __attribute__((aligned(16))) char smem[2][(BM + BN) * kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lk = lane >> 4;
  const int crow = tid >> 3, ccol = (tid & 7) * 16;

  const int ncols = kSwiglu ? p.N : p.N + (p.B2 ? 1 : 0);
  constexpr int BNE = kSwiglu ? BN / 2 : BN;  // output columns per tile
  const int ntN = (ncols + BNE - 1) / BNE;
  const int mt_total = p.tiles ? *p.tile_count : (p.M + BM - 1) / BM;
  const int nt = mt_total * ntN;
  const int xcd = blockIdx.x % kXcds, per = gridDim.x / kXcds, jb = blockIdx.x / kXcds;
  const int lo = (int)((int64_t)nt * xcd / kXcds), hi = (int)((int64_t)nt * (xcd + 1) / kXcds);
  const int nk = p.Kdim / KE;

  for (int t = lo + jb; t < hi; t += per) {
    // ---- decode the logical tile: expert-major, then N tile, then M tile -------------------
    const int q = t / ntN;
    int first, cnt;
    if (p.tiles) {
      first = p.tiles[q * kTileStride + 4];
      cnt = p.tiles[q * kTileStride + 5];
    } else {
      first = 0;
      cnt = mt_total;
    }
    const int l = t - first * ntN;
    const int n_tile = l / cnt;
    const int m = first + l % cnt;
    int group, row_start, rows;
    if (p.tiles) {
      group = p.tiles[m * kTileStride + 0];
      row_start = p.tiles[m * kTileStride + 1];
      rows = p.tiles[m * kTileStride + 2];
    } else {
      group = 0;
      row_start = m * BM;
      rows = min(BM, p.M - row_start);
    }

    // ---- per-thread row pointers for the global->LDS copy -----------------------------------
    const char* aptr[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int r = min(crow + 32 * i, rows - 1);
      const int pos = row_start + r;
      const int64_t arow = p.a_gather ? (int64_t)(p.a_gather[pos] / p.a_div) : (int64_t)pos;
      aptr[i] = p.A + arow * p.lda_bytes + ccol;
    }
    const char* gbase = p.B + (int64_t)group * p.b_group_bytes;
    const char* bptr[BCH];
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int rb = crow + 32 * i;
      if (kSwiglu) {
        const int n = n_tile * (BN / 2) + (rb < BN / 2 ? rb : rb - BN / 2);
        const int64_t brow = n < p.N ? (int64_t)(rb < BN / 2 ? n : p.N + n) : 0;
        bptr[i] = gbase + brow * p.ldb_bytes + ccol;
      } else {
        const int n = n_tile * BN + rb;
        if (n < p.N)
          bptr[i] = gbase + (int64_t)n * p.ldb_bytes + ccol;
        else if (p.B2 && n == p.N)
          bptr[i] = p.B2 + ccol;
        else
          bptr[i] = gbase + ccol;
      }
    }

    // ---- which 16x16 sub-tiles of this wave hold any valid output ---------------------------
    bool mval[MI], nval[NI];
    int blds[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) mval[i] = wm * WTM + i * 16 < rows;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      if (kSwiglu) {
        const int jj = j < NI / 2 ? j : j - NI / 2;
        blds[j] = (j < NI / 2 ? 0 : BN / 2) + wn * (WTN / 2) + jj * 16;
        nval[j] = n_tile * (BN / 2) + wn * (WTN / 2) + jj * 16 < p.N;
      } else {
        blds[j] = wn * WTN + j * 16;
        nval[j] = n_tile * BN + blds[j] < ncols;
      }
    }

    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 ra[ACH], rb[BCH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[i] = *(const uint4*)(aptr[i]);
#pragma unroll
    for (int i = 0; i < BCH; ++i) rb[i] = *(const uint4*)(bptr[i]);
#pragma unroll
    for (int i = 0; i < ACH; ++i) *(uint4*)(&smem[0][(crow + 32 * i) * kPitch + ccol]) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i)
      *(uint4*)(&smem[0][(BM + crow + 32 * i) * kPitch + ccol]) = rb[i];
    __syncthreads();

    for (int ks = 0; ks < nk; ++ks) {
      const int cur = ks & 1;
      const bool more = ks + 1 < nk;
      if (more) {
        const int64_t off = (int64_t)(ks + 1) * kRowBytes;
#pragma unroll
        for (int i = 0; i < ACH; ++i) ra[i] = *(const uint4*)(aptr[i] + off);
#pragma unroll
        for (int i = 0; i < BCH; ++i) rb[i] = *(const uint4*)(bptr[i] + off);
      }
      const char* sa = smem[cur];
      const char* sb = smem[cur] + BM * kPitch;
      if constexpr (!kF32) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8 af[MI], bfr[NI];
#pragma unroll
          for (int i = 0; i < MI; ++i)
            af[i] = *(const bf16x8*)(sa + (wm * WTM + i * 16 + lr) * kPitch + s * 64 + lk * 16);
#pragma unroll
          for (int j = 0; j < NI; ++j)
            bfr[j] = *(const bf16x8*)(sb + (blds[j] + lr) * kPitch + s * 64 + lk * 16);
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
              if (mval[i] && nval[j])
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      } else {
        f32x4 af[MI][2], bfr[NI][2];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const char* src = sa + (wm * WTM + i * 16 + lr) * kPitch + lk * 32;
          af[i][0] = *(const f32x4*)src;
          af[i][1] = *(const f32x4*)(src + 16);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const char* src = sb + (blds[j] + lr) * kPitch + lk * 32;
          bfr[j][0] = *(const f32x4*)src;
          bfr[j][1] = *(const f32x4*)(src + 16);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
            if (mval[i] && nval[j]) {
#pragma unroll
              for (int qq = 0; qq < 8; ++qq)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][qq >> 2][qq & 3],
                                                                 bfr[j][qq >> 2][qq & 3],
                                                                 acc[i][j], 0, 0, 0);
            }
      }
      if (more) {
        char* dst = smem[cur ^ 1];
#pragma unroll
        for (int i = 0; i < ACH; ++i) *(uint4*)(&dst[(crow + 32 * i) * kPitch + ccol]) = ra[i];
#pragma unroll
        for (int i = 0; i < BCH; ++i)
          *(uint4*)(&dst[(BM + crow + 32 * i) * kPitch + ccol]) = rb[i];
      }
      __syncthreads();
    }

    // ---- epilogue --------------------------------------------------------------------------
    if constexpr (kSwiglu) {
      T* H = (T*)p.C;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if (!mval[i]) continue;
#pragma unroll
        for (int j = 0; j < NI / 2; ++j) {
          const int n = n_tile * (BN / 2) + wn * (WTN / 2) + j * 16 + lr;
          if (n >= p.N) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = wm * WTM + i * 16 + lk * 4 + r;
            if (row < rows) {
              const float g = acc[i][j][r], u = acc[i][j + NI / 2][r];
              H[(int64_t)(row_start + row) * p.ldc + n] = to_out<T>(silu_f(g) * u);
            }
          }
        }
      }
    } else if constexpr (EPI == EPI_STORE) {
      float* C = (float*)p.C;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if (!mval[i]) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * WTM + i * 16 + lk * 4 + r;
          if (row >= rows) continue;
          const int64_t grow = row_start + row;
          const float scale = p.row_scale ? p.row_scale[grow] : 1.0f;
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int n = n_tile * BN + wn * WTN + j * 16 + lr;
            const float v = acc[i][j][r];
            if (n < p.N) {
              const float b = p.col_bias ? p.col_bias[n] : 0.0f;
              C[grow * p.ldc + n] = (v + b) * scale;
            } else if (p.B2 && n == p.N) {
              p.C2[grow] = v;
            }
          }
        }
      }
    } else {  // EPI_ATOMIC_COMBINE
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if (!mval[i]) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * WTM + i * 16 + lk * 4 + r;
          if (row >= rows) continue;
          const int a = p.perm[row_start + row];
          const float w = p.topk_w[a];
          float* dst = p.acc_out + (int64_t)(a / p.topk) * p.ldo;
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int n = n_tile * BN + wn * WTN + j * 16 + lr;
            if (n < p.N) unsafeAtomicAdd(dst + n, w * acc[i][j][r]);
          }
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(Epilogue epi, const GemmParams& p, int64_t max_mtiles, int occupancy,
                      hipStream_t stream) {
  const int ncols = epi == EPI_SWIGLU ? p.N : p.N + (p.B2 ? 1 : 0);
  const int bne = epi == EPI_SWIGLU ? BN / 2 : BN;
  const int64_t ntN = (ncols + bne - 1) / bne;
  int64_t want = max_mtiles * ntN;
  int64_t cap = (int64_t)kCus * occupancy;
  int64_t grid = want < cap ? want : cap;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  dim3 g((unsigned)grid), b(256);
  switch (epi) {
    case EPI_STORE:
      hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_STORE>), g, b, 0, stream, p);
      break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_SWIGLU>), g, b, 0, stream, p);
      break;
    case EPI_ATOMIC_COMBINE:
      hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_ATOMIC_COMBINE>), g, b, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int tile_bm(TileCfg cfg) { return cfg == TILE_SMALL ? 32 : 128; }

hipError_t launch_gemm(int dtype, TileCfg cfg, Epilogue epi, const GemmParams& p,
                       int64_t max_mtiles, hipStream_t stream) {
  if (max_mtiles <= 0) return hipSuccess;
  // Occupancy from LDS: SMALL uses 2*(32+128)*144 B = 45 KiB (3 per CU), LARGE 108 KiB (1).
  if (dtype == 1) {
    if (cfg == TILE_SMALL) return launch_cfg<__bf16, 32, 128, 1, 4>(epi, p, max_mtiles, 3, stream);
    return launch_cfg<__bf16, 128, 256, 2, 2>(epi, p, max_mtiles, 1, stream);
  }
  if (cfg == TILE_SMALL) return launch_cfg<float, 32, 128, 1, 4>(epi, p, max_mtiles, 3, stream);
  return launch_cfg<float, 128, 256, 2, 2>(epi, p, max_mtiles, 1, stream);
}

}  // namespace moe
