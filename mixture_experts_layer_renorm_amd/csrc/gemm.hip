// Grouped / dense GEMM on gfx950 matrix cores, with the epilogues the MoE layer needs.
//
// One kernel template serves every contraction of the layer:
//   router      C = x W_rᵀ (+ the shared-gate column w_s), fp32 logits      ("MoE" §2 Router)
//   gate_up     H = SiLU(X_e W_gateᵀ) ⊙ (X_e W_upᵀ) per expert, rows gathered through the
//               dispatch permutation                                          ("MoE" §3 eq. E_e)
//   down        y = H W_downᵀ per expert, stored per position, or scaled by the routing weight
//               and added into the token's fp32 accumulator                  ("MoE" §3.2, §4)
//   shared      the same gate_up/down on all T tokens, gate applied as a row scale (§4)
//
// Design (gfx950, wave64):
//  * 256 threads = 4 waves arranged WM x WN over a BM x BN output tile.
//  * K advances 128 bytes of every row per step (64 bf16 or 32 fp32 elements).  Operands move
//    from HBM/L2 straight into LDS with global_load_lds_dwordx4 (16 bytes per lane, one 1 KiB
//    run of 8 rows per wave instruction), through a ring of S stages, so S-1 steps of loads are
//    in flight while one step is multiplied and no registers are spent on staging.  One bare
//    s_barrier per step (with explicit vmcnt/lgkmcnt waits) separates reuse of a stage.
//  * LDS rows are 128 bytes, unpadded; the eight 16-byte chunks of row r are stored XOR-swizzled
//    by (r >> 1) & 7, so the 16 rows read by one MFMA operand fetch fall in distinct banks.
//  * bf16: v_mfma_f32_16x16x32_bf16 (lane l holds row l%16, k = 8*(l/16)..+7 of each operand;
//    result rows 4*(l/16)..+3, column l%16).  fp32: v_mfma_f32_16x16x4_f32, eight per 32-wide k
//    slice, the k order permuted identically for both operands.
//  * Padding rows (a group's last tile) and padding columns are computed on clamped, valid
//    addresses and discarded by the epilogue.  The MFMA stream has no branches: guards around
//    sub-tiles would split it and force the accumulators out of the AGPRs.
//  * Persistent, XCD-aware schedule: work-group b runs on XCD b % 8; each XCD owns one
//    contiguous eighth of the logical tile sequence, which is ordered expert-major, then by
//    N tile, then by M tile.  Tiles that share an expert's weights or rows therefore run at the
//    same time on the same XCD and meet in its L2.
#include "kernels.h"
#include "silu.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowBytes = 128;  // bytes of each row consumed per K step (8 chunks of 16 B)

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector-memory operations and
// `lgkm` LDS/scalar operations of this wave are outstanding.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Work-group barrier with explicit waits and no memory fence: the caller states which of its
// own loads must have landed.  The empty asm statements keep the compiler from moving LDS
// reads or DMA issues across the barrier.
template <int VM, int LGKM>
__device__ __forceinline__ void barrier_after() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, LGKM));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


template <typename T>
__device__ __forceinline__ T to_out(float v);
template <>
__device__ __forceinline__ float to_out<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 to_out<__bf16>(float v) { return (__bf16)v; }

// One step of operand DMA: this lane's L 16-byte chunks, each wave instruction filling 1 KiB
// (8 staged rows) of the stage.
template <int L>
__device__ __forceinline__ void dma_step(const char* const* src, int64_t off, char* stage,
                                         int wave) {
#pragma unroll
  for (int i = 0; i < L; ++i)
    __builtin_amdgcn_global_load_lds(src[i] + off, stage + (4 * i + wave) * 1024, 16, 0, 0);
}

template <typename T, int BM, int BN, int WM, int WN, int S, int EPI>
__global__ void __launch_bounds__(256) gemm_kernel(const GemmParams p) {
  static_assert(WM * WN == 4, "4 waves");
  constexpr int ROWS = BM + BN;            // rows staged per step
  constexpr int L = ROWS / 32;             // 1 KiB DMA runs per wave per step
  constexpr int STAGE = ROWS * kRowBytes;  // bytes per stage
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 16, NI = WTN / 16;
  constexpr bool kF32 = sizeof(T) == 4;
  constexpr int KE = kRowBytes / (int)sizeof(T);
  constexpr bool kSwiglu = EPI == EPI_SWIGLU;
  static_assert(!kSwiglu || (NI % 2 == 0), "SwiGLU pairs gate and up sub-tiles");
  static_assert(BM % 32 == 0 && BN % 32 == 0, "whole 8-row runs per wave");
  static_assert(L * (S - 2) < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) char smem[S][STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lk = lane >> 4;
  // DMA: wave instruction i of a step fills staged rows [8*(4i+wave), +8); lane -> (row, chunk)
  const int drow = lane >> 3, dchunk = lane & 7;

  const int ncols = kSwiglu ? p.N : p.N + (p.B2 ? 1 : 0);
  constexpr int BNE = kSwiglu ? BN / 2 : BN;  // output columns per tile
  const int ntN = (ncols + BNE - 1) / BNE;
  const int mt_total = p.tiles ? load_uniform(p.tile_count, 0) : (p.M + BM - 1) / BM;
  // split-K (dense STORE only): logical tile t is reduction slice t % ks of output tile t / ks
  const int ks = (EPI == EPI_STORE && !p.tiles && p.k_slices > 1) ? p.k_slices : 1;
  const int nt = mt_total * ntN * ks;
  const int xcd = blockIdx.x % kXcds, per = gridDim.x / kXcds, jb = blockIdx.x / kXcds;
  const int lo = (int)((int64_t)nt * xcd / kXcds), hi = (int)((int64_t)nt * (xcd + 1) / kXcds);
  const int nk = p.Kdim / KE / ks;  // K steps per slice (the host makes ks divide them)

  // LDS rows of this wave's B sub-tiles (SwiGLU: gate j and up j sit NI/2 sub-tiles apart).
  int blds[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    if (kSwiglu) {
      const int jj = j < NI / 2 ? j : j - NI / 2;
      blds[j] = BM + (j < NI / 2 ? 0 : BN / 2) + wn * (WTN / 2) + jj * 16;
    } else {
      blds[j] = BM + wn * WTN + j * 16;
    }
  }

  for (int tk = lo + jb; tk < hi; tk += per) {
    // ---- decode the logical tile: expert-major, then N tile, then M tile -------------------
    const int kslice = tk % ks, t = tk / ks;
    const int64_t k0 = (int64_t)kslice * nk * kRowBytes;  // this slice's first byte of a row
    const int q = t / ntN;
    int first, cnt;
    if (p.tiles) {
      first = load_uniform(p.tiles, q * kTileStride + 4);
      cnt = load_uniform(p.tiles, q * kTileStride + 5);
    } else {
      first = 0;
      cnt = mt_total;
    }
    const int l = t - first * ntN;
    const int n_tile = l / cnt;
    const int m = first + l % cnt;
    int group, row_start, rows;
    if (p.tiles) {
      group = load_uniform(p.tiles, m * kTileStride + 0);
      row_start = load_uniform(p.tiles, m * kTileStride + 1);
      rows = load_uniform(p.tiles, m * kTileStride + 2);
    } else {
      group = 0;
      row_start = m * BM;
      rows = min(BM, p.M - row_start);
    }

    // ---- global source of every DMA this lane issues per step --------------------------------
    const char* gbase = p.B + (int64_t)group * p.b_group_bytes;
    const char* src[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int r = 8 * (4 * i + wave) + drow;  // staged row, A rows first
      const int chunk = dchunk ^ swz(r);        // logical 16-byte chunk stored at this slot
      const char* rowp;
      if (r < BM) {
        const int pos = row_start + min(r, rows - 1);
        const int64_t arow = p.a_gather ? (int64_t)(p.a_gather[pos] / p.a_div) : (int64_t)pos;
        rowp = p.A + arow * p.lda_bytes;
      } else {
        const int rb = r - BM;
        if (kSwiglu) {
          const int n = n_tile * (BN / 2) + (rb < BN / 2 ? rb : rb - BN / 2);
          const int64_t brow = n < p.N ? (int64_t)(rb < BN / 2 ? n : p.N + n) : 0;
          rowp = gbase + brow * p.ldb_bytes;
        } else {
          const int n = n_tile * BN + rb;
          if (n < p.N)
            rowp = gbase + (int64_t)n * p.ldb_bytes;
          else if (p.B2 && n == p.N)
            rowp = p.B2;
          else
            rowp = gbase;
        }
      }
      src[i] = rowp + chunk * 16;
    }

    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Every wave is done with the previous tile's stages and stores before new DMA starts.
    barrier_after<0, 0>();

#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (st < nk) dma_step<L>(src, k0 + (int64_t)st * kRowBytes, smem[st], wave);

    for (int kk = 0; kk < nk; ++kk) {
      // this wave's DMA for step kk has landed (later steps may still fly), earlier LDS reads
      // are complete; the barrier then publishes step kk and frees stage (kk - 1) % S
      if (kk + S - 2 < nk)
        barrier_after<L * (S - 2), 0>();
      else
        barrier_after<0, 0>();
      if (kk + S - 1 < nk)
        dma_step<L>(src, k0 + (int64_t)(kk + S - 1) * kRowBytes, smem[(kk + S - 1) % S], wave);

      const char* sm = smem[kk % S];
      if constexpr (!kF32) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8 af[MI], bfr[NI];
          const int c = s * 4 + lk;  // logical chunk: k = 32*s + 8*lk .. +7
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            const int r = wm * WTM + i * 16 + lr;
            af[i] = *(const bf16x8*)(sm + r * kRowBytes + ((c ^ swz(r)) << 4));
          }
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int r = blds[j] + lr;
            bfr[j] = *(const bf16x8*)(sm + r * kRowBytes + ((c ^ swz(r)) << 4));
          }
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      } else {
        f32x4 af[MI][2], bfr[NI][2];
        const int c0 = 2 * lk, c1 = 2 * lk + 1;  // k = 8*lk .. 8*lk+7
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int r = wm * WTM + i * 16 + lr;
          af[i][0] = *(const f32x4*)(sm + r * kRowBytes + ((c0 ^ swz(r)) << 4));
          af[i][1] = *(const f32x4*)(sm + r * kRowBytes + ((c1 ^ swz(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int r = blds[j] + lr;
          bfr[j][0] = *(const f32x4*)(sm + r * kRowBytes + ((c0 ^ swz(r)) << 4));
          bfr[j][1] = *(const f32x4*)(sm + r * kRowBytes + ((c1 ^ swz(r)) << 4));
        }
#pragma unroll
        for (int qq = 0; qq < 8; ++qq)
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][qq >> 2][qq & 3],
                                                               bfr[j][qq >> 2][qq & 3], acc[i][j],
                                                               0, 0, 0);
      }
    }

    // ---- epilogue --------------------------------------------------------------------------
    if constexpr (kSwiglu) {
      T* H = (T*)p.C;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NI / 2; ++j) {
          const int n = n_tile * (BN / 2) + wn * (WTN / 2) + j * 16 + lr;
          if (n >= p.N) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = wm * WTM + i * 16 + lk * 4 + r;
            if (row < rows) {
              const float g = acc[i][j][r], u = acc[i][j + NI / 2][r];
              H[(int64_t)(row_start + row) * p.ldc + n] = to_out<T>(silu_fast(g) * u);
            }
          }
        }
      }
    } else if constexpr (EPI == EPI_STORE) {
      float* C = (float*)p.C + kslice * p.c_slice_stride;
      float* C2 = p.C2 ? p.C2 + kslice * p.c2_slice_stride : nullptr;
      const float* col_bias = kslice == 0 ? p.col_bias : nullptr;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
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
              const float b = col_bias ? col_bias[n] : 0.0f;
              C[grow * p.ldc + n] = (v + b) * scale;
            } else if (p.B2 && n == p.N) {
              C2[grow] = v;
            }
          }
        }
      }
    } else {  // EPI_ATOMIC_COMBINE
#pragma unroll
      for (int i = 0; i < MI; ++i) {
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

template <typename T, int BM, int BN, int WM, int WN, int S>
hipError_t launch_cfg(Epilogue epi, const GemmParams& p, int64_t max_mtiles, int occupancy,
                      hipStream_t stream) {
  const int ncols = epi == EPI_SWIGLU ? p.N : p.N + (p.B2 ? 1 : 0);
  const int bne = epi == EPI_SWIGLU ? BN / 2 : BN;
  const int64_t ntN = (ncols + bne - 1) / bne;
  const int ks = (epi == EPI_STORE && !p.tiles && p.k_slices > 1) ? p.k_slices : 1;
  if (ks > 1 && (p.Kdim / (kRowBytes / (int)sizeof(T))) % ks != 0) return hipErrorInvalidValue;
  int64_t want = max_mtiles * ntN * ks;
  int64_t cap = (int64_t)kCus * occupancy;
  int64_t grid = want < cap ? want : cap;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  dim3 g((unsigned)grid), b(256);
  switch (epi) {
    case EPI_STORE:
      hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, S, EPI_STORE>), g, b, 0, stream, p);
      break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, S, EPI_SWIGLU>), g, b, 0, stream, p);
      break;
    case EPI_ATOMIC_COMBINE:
      hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, S, EPI_ATOMIC_COMBINE>), g, b, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int tile_bm(TileCfg cfg) { return cfg == TILE_SMALL ? 32 : 256; }
// Weight rows per tile (output columns; half of them for the fused gate/up epilogue).
int tile_bn(TileCfg cfg) { return cfg == TILE_MFMA ? 256 : 128; }

hipError_t launch_gemm(int dtype, TileCfg cfg, Epilogue epi, const GemmParams& p,
                       int64_t max_mtiles, hipStream_t stream) {
  if (max_mtiles <= 0) return hipSuccess;
  if (cfg == TILE_MFMA) {
    if (dtype != 1) return hipErrorInvalidValue;
    return launch_mfma_gemm(epi, p, max_mtiles, stream);
  }
  // Occupancy from LDS: SMALL stages 4 x 20 KiB (2 work-groups per CU), LARGE 3 x 48 KiB (1).
  // LARGE is 256 rows x 128 columns: one M tile holds every row of an expert with up to 256
  // tokens, so that expert's weights stream from HBM once.
  if (dtype == 1) {
    if (cfg == TILE_SMALL)
      return launch_cfg<__bf16, 32, 128, 1, 4, 4>(epi, p, max_mtiles, 2, stream);
    return launch_cfg<__bf16, 256, 128, 4, 1, 3>(epi, p, max_mtiles, 1, stream);
  }
  if (cfg == TILE_SMALL) return launch_cfg<float, 32, 128, 1, 4, 4>(epi, p, max_mtiles, 2, stream);
  return launch_cfg<float, 256, 128, 4, 1, 3>(epi, p, max_mtiles, 1, stream);
}

}  // namespace moe
