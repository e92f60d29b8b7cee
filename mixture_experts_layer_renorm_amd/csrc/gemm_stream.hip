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

// One output tile; every field is uniform across the work-group.
struct StreamTile {
  int group, row_start, rows, n_tile;
};

// Logical tiles run expert-major, then N tile, then M tile: the m-tiles of one expert are
// entries [first, first + cnt) of the tile map and own logical tiles [first·ntN, (first+cnt)·ntN).
__device__ __forceinline__ StreamTile decode_tile(const GemmParams& p, int t, int ntN) {
  const int q = t / ntN;
  const int first = p.tiles[q * kTileStride + 4];
  const int cnt = p.tiles[q * kTileStride + 5];
  const int l = t - first * ntN;
  const int m = first + l % cnt;
  StreamTile s;
  s.n_tile = l / cnt;
  s.group = p.tiles[m * kTileStride + 0];
  s.row_start = p.tiles[m * kTileStride + 1];
  s.rows = p.tiles[m * kTileStride + 2];
  return s;
}

// Source row of tile row r (rows past the group's end repeat its last row; their results are
// discarded by the epilogue).
__device__ __forceinline__ int token_row(const GemmParams& p, const StreamTile& s, int r) {
  const int pos = s.row_start + min(r, s.rows - 1);
  return p.a_gather ? p.a_gather[pos] / p.a_div : pos;
}

template <int BM, int P, int EPI, bool CROSS>
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
  // Epilogue staging: output rows are assembled in LDS and leave as whole 16-byte chunks.
  constexpr int kEpRows = BM < 64 ? BM : 64;  // fp32 rows per store pass
  constexpr int kLdE = BN + 4;                // fp32 per staged row (padded against bank conflicts)
  constexpr int kLdH = BN / 2 + 8;            // bf16 per staged H row
  constexpr int kEpBytes = EPI == EPI_STORE    ? kEpRows * kLdE * 4
                           : EPI == EPI_SWIGLU ? BM * kLdH * 2
                                               : 16;
  __shared__ __attribute__((aligned(16))) char ep[kEpBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lk = lane >> 4;

  constexpr int BNE = kSwiglu ? BN / 2 : BN;  // output columns per tile
  const int ntN = (p.N + BNE - 1) / BNE;
  const int mt_total = *p.tile_count;
  const int nt = mt_total * ntN;
  const int xcd = blockIdx.x % kXcds, per = gridDim.x / kXcds, jb = blockIdx.x / kXcds;
  const int lo = (int)((int64_t)nt * xcd / kXcds), hi = (int)((int64_t)nt * (xcd + 1) / kXcds);
  const int nk = p.Kdim / 32;
  int t = lo + jb;
  if (t >= hi) return;

  // Token-row chunk i of this thread: c = tid + 512 i -> tile row c >> 2, LDS slot c & 3, which
  // holds logical chunk (c & 3) ^ swz(row) of the row's 64 bytes.
  int arow_t[LA], alds[LA], aoff[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = min((tid + NT * i) >> 2, BM - 1);
    arow_t[i] = r;
    alds[i] = r * kRow + ((tid & 3) << 4);
    aoff[i] = ((tid & 3) ^ swz(r)) << 4;
  }

  StreamTile cur = decode_tile(p, t, ntN);
  int arow[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) arow[i] = token_row(p, cur, arow_t[i]);

  // Loaders: byte offsets of this thread's token-row chunks in A (aoffs) and of its weight rows
  // in the current group (boffs, from the uniform base bbase); all operands are below 4 GiB, so
  // the loads take a scalar base plus a 32-bit lane offset.  With nk a multiple of P the ring
  // runs on across tiles: the last P steps of a tile fetch the first P steps of the next, and
  // the last step stages its first rows, so the next tile starts with its loads in flight while
  // this one's epilogue stores drain.
  uint32_t aoffs[LA], boffs[NJ];
  const char* bbase;
  bf16x8 areg[P][LA], breg[P][NJ];

#define MOE_STREAM_POINT(S)                                                                  \
  {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < LA; ++i) aoffs[i] =                                \
        (uint32_t)arow[i] * (uint32_t)p.lda_bytes + (uint32_t)aoff[i];                       \
    bbase = p.B + (int64_t)(S).group * p.b_group_bytes;                                      \
    _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                         \
      int wr;                                                                                \
      if (kSwiglu) { /* sub-tile 0: gate rows, sub-tile 1: the matching up rows */           \
        const int n = (S).n_tile * (BN / 2) + wave * 16 + lr;                                \
        wr = n < p.N ? (j == 0 ? n : p.N + n) : 0;                                           \
      } else {                                                                               \
        const int n = (S).n_tile * BN + wave * 32 + j * 16 + lr;                             \
        wr = n < p.N ? n : 0;                                                                \
      }                                                                                      \
      boffs[j] = (uint32_t)wr * (uint32_t)p.ldb_bytes + (uint32_t)(lk * 16);                 \
    }                                                                                        \
  }

  // Load K step STEP of the tile set up by MOE_STREAM_POINT into ring slot SLOT.
#define MOE_STREAM_LOAD(SLOT, STEP)                                                          \
  {                                                                                          \
    const uint32_t off_ = (uint32_t)(STEP) * kRow;                                           \
    _Pragma("unroll") for (int i = 0; i < LA; ++i) if (a_live<CH, NT, LA>(tid, i))           \
        areg[SLOT][i] = *(const bf16x8*)(p.A + (aoffs[i] + off_));                           \
    _Pragma("unroll") for (int j = 0; j < NJ; ++j) breg[SLOT][j] =                           \
        *(const bf16x8*)(bbase + (boffs[j] + off_));                                         \
  }

  MOE_STREAM_POINT(cur)
#pragma unroll
  for (int s_ = 0; s_ < P; ++s_)
    if (s_ < nk) MOE_STREAM_LOAD(s_, s_)

  // One K step: multiply LDS buffer ks&1 by weight slot QQ; if ISSUE, refill slot QQ with step
  // ISTEP of the tile behind (AS, BS); if STAGE_NEXT, stage slot QQ+1's token rows into the
  // other LDS buffer.
#define MOE_STREAM_STEP(QQ, KS, ISSUE, ISTEP, STAGE_NEXT)                                  \
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
    if (ISSUE) MOE_STREAM_LOAD(QQ, ISTEP)                                                  \
    if (STAGE_NEXT) {                                                                      \
      _Pragma("unroll") for (int i = 0; i < LA; ++i) if (a_live<CH, NT, LA>(tid, i))       \
          *(bf16x8*)(&smem[((KS) + 1) & 1][alds[i]]) = areg[((QQ) + 1) % P][i];            \
    }                                                                                      \
    __syncthreads();                                                                       \
  }

  bool staged = false;  // step 0 of the current tile already sits in LDS buffer 0
  for (;;) {
    if (!staged) {
#pragma unroll
      for (int i = 0; i < LA; ++i)
        if (a_live<CH, NT, LA>(tid, i)) *(bf16x8*)(&smem[0][alds[i]]) = areg[0][i];
      __syncthreads();
    }

    // the next tile and its token rows, fetched now so they have arrived before they are used
    const int tn = t + per;
    const bool more = tn < hi;
    StreamTile nxt = cur;
    if (more) {
      nxt = decode_tile(p, tn, ntN);
#pragma unroll
      for (int i = 0; i < LA; ++i) arow[i] = token_row(p, nxt, arow_t[i]);
    }

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (CROSS) {  // requires nk % P == 0
      // all rounds but the last refill from this tile; the last one from the next tile
      int ks0 = 0;
      for (; ks0 + P < nk; ks0 += P) {
#pragma unroll
        for (int qq = 0; qq < P; ++qq)
          MOE_STREAM_STEP(qq, ks0 + qq, true, ks0 + qq + P, true);
      }
      if (more) MOE_STREAM_POINT(nxt)
#pragma unroll
      for (int qq = 0; qq < P; ++qq)
        MOE_STREAM_STEP(qq, ks0 + qq, more, qq, (qq + 1 < P) || more);
      staged = true;
    } else {
      // steady state: all P steps of a round issue step ks + P (needs ks + P < nk)
      int ks0 = 0;
      for (; ks0 + 2 * P <= nk; ks0 += P) {
#pragma unroll
        for (int qq = 0; qq < P; ++qq)
          MOE_STREAM_STEP(qq, ks0 + qq, true, ks0 + qq + P, true);
      }
      // the last P..2P-1 steps
#pragma unroll
      for (int qq = 0; qq < 2 * P; ++qq) {
        const int ks = ks0 + qq;
        if (ks < nk) MOE_STREAM_STEP(qq % P, ks, ks + P < nk, ks + P, ks + 1 < nk);
      }
      // the next tile's loads go out before this tile's stores, so they overlap them
      if (more) {
        MOE_STREAM_POINT(nxt)
#pragma unroll
        for (int s_ = 0; s_ < P; ++s_)
          if (s_ < nk) MOE_STREAM_LOAD(s_, s_)
      }
      staged = false;
    }

    // ---- epilogue ---------------------------------------------------------------------------
    // Lane (lr, lk) holds rows i*16 + lk*4 + r of column sub-tile j in acc[i][j][r].  The lane
    // index is laundered through an empty asm so the store offsets below are computed here,
    // not hoisted out of the tile loop into registers the K loop needs.
    int etid = tid;
    asm volatile("" : "+v"(etid));
    const int elr = etid & 15, elk = (etid >> 4) & 3;
    if constexpr (kSwiglu) {
      __bf16* Eh = (__bf16*)ep;
      const int col = wave * 16 + elr;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if (i * 16 < cur.rows) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Eh[(i * 16 + elk * 4 + r) * kLdH + col] = (__bf16)(silu_f(acc[i][0][r]) * acc[i][1][r]);
        }
      }
      __syncthreads();
      constexpr int kCpr = BN / 2 / 8;  // 16-byte chunks per H row
      // tile origin (uniform) + 32-bit lane offsets
      char* Ht = (char*)p.C + ((int64_t)cur.row_start * p.ldc + cur.n_tile * (BN / 2)) * 2;
      const int ncols = min(BN / 2, p.N - cur.n_tile * (BN / 2));
#pragma unroll
      for (int m = 0; m < BM * kCpr / NT; ++m) {
        const int c = etid + NT * m;
        const int row = c / kCpr, ch = c % kCpr;
        if (row < cur.rows && ch * 8 < ncols)
          *(bf16x8*)(Ht + (uint32_t)(row * (int)p.ldc + ch * 8) * 2u) =
              *(const bf16x8*)(Eh + row * kLdH + ch * 8);
      }
      __syncthreads();
    } else if constexpr (EPI == EPI_STORE) {
      float* E = (float*)ep;
      // tile origin (uniform) + 32-bit lane offsets
      char* Ct = (char*)p.C + ((int64_t)cur.row_start * p.ldc + cur.n_tile * BN) * 4;
      const float* rs = p.row_scale ? p.row_scale + cur.row_start : nullptr;
      const int ncols = min(BN, p.N - cur.n_tile * BN);
      constexpr int kCpr = BN / 4;  // 16-byte chunks per fp32 row
#pragma unroll
      for (int q = 0; q < BM / kEpRows; ++q) {
        if (q * kEpRows < cur.rows) {
#pragma unroll
          for (int ii = 0; ii < kEpRows / 16; ++ii) {
            const int i = q * (kEpRows / 16) + ii;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                E[(ii * 16 + elk * 4 + r) * kLdE + wave * 32 + j * 16 + elr] = acc[i][j][r];
          }
          __syncthreads();
#pragma unroll
          for (int m = 0; m < kEpRows * kCpr / NT; ++m) {
            const int c = etid + NT * m;
            const int lrow = c / kCpr, col = (c % kCpr) * 4;
            const int row = q * kEpRows + lrow;
            if (row < cur.rows && col < ncols) {
              f32x4 v = *(const f32x4*)(E + lrow * kLdE + col);
              if (rs) v *= rs[row];
              *(f32x4*)(Ct + (uint32_t)(row * (int)p.ldc + col) * 4u) = v;
            }
          }
          __syncthreads();
        }
      }
    } else {  // EPI_ATOMIC_COMBINE
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = i * 16 + elk * 4 + r;
          if (row >= cur.rows) continue;
          const int a = p.perm[cur.row_start + row];
          const float w = p.topk_w[a];
          float* dst = p.acc_out + (int64_t)(a / p.topk) * p.ldo;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int n = cur.n_tile * BN + wave * 32 + j * 16 + elr;
            if (n < p.N) unsafeAtomicAdd(dst + n, w * acc[i][j][r]);
          }
        }
    }
    if (!more) break;
    cur = nxt;
    t = tn;
  }
#undef MOE_STREAM_STEP
#undef MOE_STREAM_POINT
#undef MOE_STREAM_LOAD
}

template <int BM, int P, int EPI>
hipError_t launch_epi(const GemmParams& p, dim3 g, hipStream_t stream) {
  if ((p.Kdim / 32) % P == 0)
    hipLaunchKernelGGL((stream_kernel<BM, P, EPI, true>), g, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((stream_kernel<BM, P, EPI, false>), g, dim3(512), 0, stream, p);
  return hipGetLastError();
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
  const dim3 g((unsigned)grid);
  switch (epi) {
    case EPI_SWIGLU:
      return launch_epi<BM, P, EPI_SWIGLU>(p, g, stream);
    case EPI_STORE:
      return launch_epi<BM, P, EPI_STORE>(p, g, stream);
    case EPI_ATOMIC_COMBINE:
      return launch_epi<BM, P, EPI_ATOMIC_COMBINE>(p, g, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_stream_gemm(TileCfg cfg, Epilogue epi, const GemmParams& p, int64_t max_mtiles,
                              hipStream_t stream) {
  if (max_mtiles <= 0) return hipSuccess;
  switch (cfg) {
    case TILE_STREAM_64:
      return launch_bm<64, 8>(epi, p, max_mtiles, 1, stream);
    case TILE_STREAM_192:
      return launch_bm<192, 4>(epi, p, max_mtiles, 1, stream);
    case TILE_STREAM_128:
      return launch_bm<128, 8>(epi, p, max_mtiles, 1, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
