// Weight-streaming grouped GEMM for the routed experts (gfx950, bf16).
//
// At the token counts of the layer's workloads an expert sees a few to a few hundred rows, so
// the expert GEMMs are bound by reading the weights from HBM (read volume b_W·N_e·U:
// "S23-J10" §3), not by the matrix cores.  Under full load HBM latency is several
// microseconds, so what bounds throughput is how many weight bytes each CU keeps in flight.
// LDS (160 KiB) is too small for that; the register file (512 KiB per CU) is not:
//  * A work-group of 8 waves (two per SIMD) owns BN = 256 weight rows (output columns) of one
//    expert and up to BM of its token rows, so every weight byte is fetched from HBM once.  The
//    waves split the columns, 32 each, which keeps each wave's accumulators small.
//  * Each lane loads its weight fragments with plain 16-byte vector loads straight into
//    registers already in the MFMA operand layout (lane l: row l%16, k = 8*(l/16)..+7), P K-steps
//    (of 32) ahead, in a register ring: 16 KiB of weights per step, P = 8 steps (128 KiB) in
//    flight per CU.
//  * The token rows, shared by all waves, are loaded the same P steps ahead into registers and
//    written one step ahead of use into a double-buffered LDS tile of 64-byte rows whose 16-byte
//    chunks are XOR-swizzled by (row >> 1) & 3 (conflict-free for the 16-row operand fetches).
//  * Only ordinary vector loads are in flight, so the compiler's vmcnt accounting is exact
//    across the unrolled ring (mixing them with LDS DMA makes it fall back to vmcnt(0)).
//  * Epilogues: fused SiLU·up (gate_up; a wave's 64 columns are 32 gate/up pairs), fp32 row
//    store (down), or the weighted fp32 atomic combine (down, opt-in).
#include "kernels.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRow = 64;  // LDS bytes per token row per step (32 bf16)

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }

// Token-row chunk i of a thread exists unless it falls in the partial last round (known at
// compile time when CH is a multiple of the block size).
template <int CH, int NT, int LA>
__device__ __forceinline__ bool a_live(int tid, int i) {
  return CH % NT == 0 || i + 1 < LA || tid + NT * i < CH;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

template <int BM, int P, int EPI>
__global__ void __launch_bounds__(512) stream_kernel(const GemmParams p) {
  constexpr int NT = 512;          // threads: 8 waves
  constexpr int BN = 256;
  constexpr int MI = BM / 16;      // 16-row sub-tiles
  constexpr int NJ = 2;            // 16-column sub-tiles per wave
  constexpr int CH = BM * 4;       // 16-byte token-row chunks per step
  constexpr int LA = (CH + NT - 1) / NT;  // token-row loads per thread per step (last: partial)
  constexpr bool kSwiglu = EPI == EPI_SWIGLU;
  static_assert(CH % 64 == 0, "a wave loads whole chunk groups");

  __shared__ __attribute__((aligned(16))) char smem[2][BM * kRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lk = lane >> 4;
  // token-row chunk i of this thread: c = tid + 512 i -> row c >> 2, LDS slot c & 3 (chunks
  // beyond CH belong to no thread; the predicate is uniform per wave)
  const int aslot = tid & 3;

  constexpr int BNE = kSwiglu ? BN / 2 : BN;  // output columns per tile
  const int ntN = (p.N + BNE - 1) / BNE;
  const int mt_total = *p.tile_count;
  const int nt = mt_total * ntN;
  const int xcd = blockIdx.x % kXcds, per = gridDim.x / kXcds, jb = blockIdx.x / kXcds;
  const int lo = (int)((int64_t)nt * xcd / kXcds), hi = (int)((int64_t)nt * (xcd + 1) / kXcds);
  const int nk = p.Kdim / 32;

  for (int t = lo + jb; t < hi; t += per) {
    // ---- tile: expert-major, then N tile, then M tile ---------------------------------------
    const int q = t / ntN;
    const int first = p.tiles[q * kTileStride + 4];
    const int cnt = p.tiles[q * kTileStride + 5];
    const int l = t - first * ntN;
    const int n_tile = l / cnt;
    const int m = first + l % cnt;
    const int group = p.tiles[m * kTileStride + 0];
    const int row_start = p.tiles[m * kTileStride + 1];
    const int rows = p.tiles[m * kTileStride + 2];

    // token-row sources (logical chunk aslot ^ swz(row) lands in LDS slot aslot)
    const char* asrc[LA];
    int alds[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = min((tid + NT * i) >> 2, BM - 1);
      const int pos = row_start + min(r, rows - 1);
      const int64_t arow = p.a_gather ? (int64_t)(p.a_gather[pos] / p.a_div) : (int64_t)pos;
      asrc[i] = p.A + arow * p.lda_bytes + ((aslot ^ swz(r)) << 4);
      alds[i] = r * kRow + (aslot << 4);
    }
    // weight rows of this lane's column sub-tiles
    const char* gbase = p.B + (int64_t)group * p.b_group_bytes;
    const char* bsrc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int64_t wr;
      if (kSwiglu) {  // sub-tile 0: gate rows, sub-tile 1: the matching up rows
        const int n = n_tile * (BN / 2) + wave * 16 + lr;
        wr = n < p.N ? (j == 0 ? n : p.N + n) : 0;
      } else {
        const int n = n_tile * BN + wave * 32 + j * 16 + lr;
        wr = n < p.N ? n : 0;
      }
      bsrc[j] = gbase + wr * p.ldb_bytes + lk * 16;
    }

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 areg[P][LA], breg[P][NJ];
#pragma unroll
    for (int s = 0; s < P; ++s) {
      if (s < nk) {
        const int64_t off = (int64_t)s * kRow;
#pragma unroll
        for (int i = 0; i < LA; ++i)
          if (a_live<CH, NT, LA>(tid, i)) areg[s][i] = *(const bf16x8*)(asrc[i] + off);
#pragma unroll
        for (int j = 0; j < NJ; ++j) breg[s][j] = *(const bf16x8*)(bsrc[j] + off);
      }
    }
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int i = 0; i < LA; ++i)
      if (a_live<CH, NT, LA>(tid, i)) *(bf16x8*)(&smem[0][alds[i]]) = areg[0][i];
    __syncthreads();

    // One K step: multiply LDS buffer ks&1 by weight slot QQ, refill slot QQ with step ks+P,
    // stage the next step's token rows into the other LDS buffer.
#define MOE_STREAM_STEP(QQ, KS, ISSUE, STAGE_NEXT)                                          \
  {                                                                                        \
    const char* sm = smem[(KS) & 1];                                                       \
    bf16x8 af[MI];                                                                         \
    _Pragma("unroll") for (int i = 0; i < MI && i < 2; ++i) {                              \
      const int r = i * 16 + lr;                                                           \
      af[i] = *(const bf16x8*)(sm + r * kRow + ((lk ^ swz(r)) << 4));                      \
    }                                                                                      \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                       \
      if (i + 2 < MI) {                                                                    \
        const int r = (i + 2) * 16 + lr;                                                   \
        af[i + 2] = *(const bf16x8*)(sm + r * kRow + ((lk ^ swz(r)) << 4));                \
      }                                                                                    \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      _Pragma("unroll") for (int j = 0; j < NJ; ++j) acc[i][j] =                           \
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], breg[QQ][j], acc[i][j], 0, 0, 0); \
      __builtin_amdgcn_sched_barrier(0);                                                   \
    }                                                                                      \
    if (ISSUE) {                                                                           \
      const int64_t off = (int64_t)((KS) + P) * kRow;                                      \
      _Pragma("unroll") for (int i = 0; i < LA; ++i) if (a_live<CH, NT, LA>(tid, i)) areg[QQ][i] =  \
          *(const bf16x8*)(asrc[i] + off);                                                 \
      _Pragma("unroll") for (int j = 0; j < NJ; ++j) breg[QQ][j] =                         \
          *(const bf16x8*)(bsrc[j] + off);                                                 \
    }                                                                                      \
    if (STAGE_NEXT) {                                                                      \
      _Pragma("unroll") for (int i = 0; i < LA; ++i) if (a_live<CH, NT, LA>(tid, i))                \
          *(bf16x8*)(&smem[((KS) + 1) & 1][alds[i]]) = areg[((QQ) + 1) % P][i];            \
    }                                                                                      \
    __syncthreads();                                                                       \
  }

    // steady state: all P steps of a round issue step ks + P (needs ks + P < nk)
    int ks0 = 0;
    for (; ks0 + 2 * P <= nk; ks0 += P) {
#pragma unroll
      for (int qq = 0; qq < P; ++qq) MOE_STREAM_STEP(qq, ks0 + qq, true, true);
    }
    // the last P..2P-1 steps
#pragma unroll
    for (int qq = 0; qq < 2 * P; ++qq) {
      const int ks = ks0 + qq;
      if (ks < nk) MOE_STREAM_STEP(qq % P, ks, ks + P < nk, ks + 1 < nk);
    }
#undef MOE_STREAM_STEP

    // ---- epilogue ---------------------------------------------------------------------------
    if constexpr (kSwiglu) {
      __bf16* H = (__bf16*)p.C;
      const int n = n_tile * (BN / 2) + wave * 16 + lr;
      if (n < p.N) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = i * 16 + lk * 4 + r;
            if (row < rows)
              H[(int64_t)(row_start + row) * p.ldc + n] =
                  (__bf16)(silu_f(acc[i][0][r]) * acc[i][1][r]);
          }
      }
    } else if constexpr (EPI == EPI_STORE) {
      float* C = (float*)p.C;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = i * 16 + lk * 4 + r;
          if (row >= rows) continue;
          const int64_t grow = row_start + row;
          const float scale = p.row_scale ? p.row_scale[grow] : 1.0f;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int n = n_tile * BN + wave * 32 + j * 16 + lr;
            if (n < p.N) C[grow * p.ldc + n] = acc[i][j][r] * scale;
          }
        }
    } else {  // EPI_ATOMIC_COMBINE
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = i * 16 + lk * 4 + r;
          if (row >= rows) continue;
          const int a = p.perm[row_start + row];
          const float w = p.topk_w[a];
          float* dst = p.acc_out + (int64_t)(a / p.topk) * p.ldo;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int n = n_tile * BN + wave * 32 + j * 16 + lr;
            if (n < p.N) unsafeAtomicAdd(dst + n, w * acc[i][j][r]);
          }
        }
    }
  }
}

template <int BM, int P>
hipError_t launch_bm(Epilogue epi, const GemmParams& p, int64_t max_mtiles, int occupancy,
                     hipStream_t stream) {
  const int bne = epi == EPI_SWIGLU ? 128 : 256;
  const int64_t ntN = (p.N + bne - 1) / bne;
  const int64_t want = max_mtiles * ntN;
  const int64_t cap = (int64_t)kCus * occupancy;
  int64_t grid = want < cap ? want : cap;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  const dim3 g((unsigned)grid), b(512);
  switch (epi) {
    case EPI_SWIGLU:
      hipLaunchKernelGGL((stream_kernel<BM, P, EPI_SWIGLU>), g, b, 0, stream, p);
      break;
    case EPI_STORE:
      hipLaunchKernelGGL((stream_kernel<BM, P, EPI_STORE>), g, b, 0, stream, p);
      break;
    case EPI_ATOMIC_COMBINE:
      hipLaunchKernelGGL((stream_kernel<BM, P, EPI_ATOMIC_COMBINE>), g, b, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_gemm(TileCfg cfg, Epilogue epi, const GemmParams& p, int64_t max_mtiles,
                              hipStream_t stream) {
  if (max_mtiles <= 0) return hipSuccess;
  switch (cfg) {
    case TILE_STREAM_64:
      return launch_bm<64, 8>(epi, p, max_mtiles, 1, stream);
    case TILE_STREAM_192:
      return launch_bm<192, 6>(epi, p, max_mtiles, 1, stream);
    case TILE_STREAM_128:
      return launch_bm<128, 8>(epi, p, max_mtiles, 1, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
