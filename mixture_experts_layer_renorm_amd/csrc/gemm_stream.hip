// Weight-streaming grouped GEMM for the routed experts (gfx950, bf16).  It runs the groups of
// up to 192 rows under the split plan and the forced streaming plans; the default bf16 plan
// runs every group on the matrix-core GEMM (gemm_mfma.hip), which computes a partial tile in
// 32-row steps where this kernel always runs its BM rows.
//
// At the token counts of the layer's workloads an expert sees a few to a few hundred rows, so
// the expert GEMMs are bound by reading the weights from HBM (read volume b_W·N_e·U:
// "S23-J10" §3), not by the matrix cores.  The kernel is built so that the memory pipeline of
// each CU only carries what the product needs and always has enough of it in flight:
//  * A work-group of 8 waves (two per SIMD) owns BN = 256 weight rows (output columns) of one
//    expert and up to BM of its token rows, so every weight byte is fetched from HBM once.  The
//    waves split the columns, 32 each, which keeps each wave's accumulators small.
//  * A K step is 64 wide.  Each lane loads its weight fragments with plain 16-byte vector loads
//    straight into registers in the MFMA operand layout (lane l: row l%16, k = 8*(l/16)..+7 of
//    each 32-wide half); the two halves of a row's 128 bytes are requested back to back, so
//    the second hits the line the first brought into L1.  A register ring holds P steps
//    (P·32 KiB per CU) in flight.
//  * Token rows, shared by all waves, are loaded with the same step into registers and written
//    one step ahead of use into a double-buffered LDS tile of 128-byte rows whose 16-byte
//    chunks are XOR-swizzled by (row >> 1) & 7 (conflict-free for the 16-row operand
//    fetches).  Rows past the group's end are not fetched.
//  * Only ordinary vector loads are in flight and every path into the K loop starts with
//    none outstanding, so the compiler's load counts are exact across the ring.
//  * When the step count is a multiple of P the ring runs on across tiles: the last round of a
//    tile fetches the first P steps of the next, whose loads then overlap this tile's
//    epilogue.
//  * Epilogues: fused SiLU·up (gate_up; a wave's 32 columns are 16 gate/up pairs), row store
//    (down: fp32, or fp16 with one power-of-two factor per tile, so that max|v| < 2^15), both
//    staged in LDS and written as whole chunks, or the weighted fp32 atomic combine (down,
//    opt-in).
#include "kernels.h"
#include "silu.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kRow = 128;  // bytes per token row per K step (64 bf16)
// s_waitcnt immediate (gfx9 layout) that waits for vmcnt == 0 and leaves expcnt/lgkmcnt free.
constexpr int kWaitVmcnt0 = (7 << 4) | (15 << 8);

// 16-byte chunk swizzle of a 128-byte LDS row.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Token-row chunk i of a thread exists unless it falls in the partial last round (known at
// compile time when CH is a multiple of the block size).
template <int CH, int NT, int LA>
__device__ __forceinline__ bool a_live(int tid, int i) {
  return CH % NT == 0 || i + 1 < LA || tid + NT * i < CH;
}

// One output tile; every field is uniform across the work-group.
struct StreamTile {
  int group, row_start, rows, n_tile;
};

// Logical tiles run expert-major, then N tile, then M tile: the m-tiles of one expert are
// entries [first, first + cnt) of the tile map and own logical tiles [first·ntN, (first+cnt)·ntN).
__device__ __forceinline__ StreamTile decode_tile(const GemmParams& p, int t, int ntN) {
  const int q = t / ntN;
  const int first = load_uniform(p.tiles, q * kTileStride + 4);
  const int cnt = load_uniform(p.tiles, q * kTileStride + 5);
  const int l = t - first * ntN;
  const int m = first + l % cnt;
  StreamTile s;
  s.n_tile = l / cnt;
  s.group = load_uniform(p.tiles, m * kTileStride + 0);
  s.row_start = load_uniform(p.tiles, m * kTileStride + 1);
  s.rows = load_uniform(p.tiles, m * kTileStride + 2);
  return s;
}

// Source entry of tile row r: the gather-table entry (A row = entry / a_div) or the row itself.
// Rows past the group's end repeat its last row; their results are discarded by the epilogue.
// The division is left to the caller, so the gather load is not waited for until its row is
// needed.
__device__ __forceinline__ int token_src(const GemmParams& p, const StreamTile& s, int r) {
  const int pos = s.row_start + min(r, s.rows - 1);
  return p.a_gather ? p.a_gather[pos] : pos;
}

template <int BM, int P, int EPI, bool CROSS>
__global__ void __launch_bounds__(512) stream_kernel(const GemmParams p) {
  constexpr int NT = 512;          // threads: 8 waves
  constexpr int BN = 256;
  constexpr int MI = BM / 16;      // 16-row sub-tiles
  constexpr int NJ = 2;            // 16-column sub-tiles per wave
  constexpr int KH = 2;            // 32-wide MFMA halves of a K step
  constexpr int CH = BM * 8;       // 16-byte token-row chunks per step
  constexpr int LA = (CH + NT - 1) / NT;  // token-row loads per thread per step (last: partial)
  constexpr bool kSwiglu = EPI == EPI_SWIGLU;
  static_assert(BM % 16 == 0 && CH % 64 == 0, "whole 16-row sub-tiles, whole-wave chunk groups");

  __shared__ __attribute__((aligned(16))) char smem[2][BM * kRow];
  // Epilogue staging: output rows are assembled in LDS and leave as whole 16-byte chunks.
  constexpr int kEpRows = BM < 64 ? BM : 64;  // fp32 rows per store pass
  constexpr int kLdE = BN + 4;                // fp32 per staged row (padded against bank conflicts)
  constexpr int kLdH = BN / 2 + 8;            // bf16 per staged H row
  constexpr int kEpBytes = EPI == EPI_STORE    ? kEpRows * kLdE * 4
                           : EPI == EPI_SWIGLU ? BM * kLdH * 2
                                               : 16;
  __shared__ __attribute__((aligned(16))) char ep[kEpBytes];
  __shared__ float tmax[8];  // per-wave maxima of the fp16 row store

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lk = lane >> 4;

  constexpr int BNE = kSwiglu ? BN / 2 : BN;  // output columns per tile
  const int ntN = (p.N + BNE - 1) / BNE;
  const int mt_total = load_uniform(p.tile_count, 0);
  const int nt = mt_total * ntN;
  const int xcd = blockIdx.x % kXcds, per = gridDim.x / kXcds, jb = blockIdx.x / kXcds;
  const int lo = (int)((int64_t)nt * xcd / kXcds), hi = (int)((int64_t)nt * (xcd + 1) / kXcds);
  const int nk = p.Kdim / 64;
  int t = lo + jb;
  if (t >= hi) return;

  // Token-row chunk i of this thread: c = tid + 512 i -> tile row c >> 3, LDS slot c & 7, which
  // holds logical chunk (c & 7) ^ swz(row) of the row's 128 bytes.  A wave's chunks cover 8
  // consecutive rows starting at arow0[i] (uniform).
  int arow_t[LA], alds[LA], aoff[LA], arow0[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = min((tid + NT * i) >> 3, BM - 1);
    arow_t[i] = r;
    arow0[i] = (wave * 64 + NT * i) >> 3;
    alds[i] = r * kRow + ((tid & 7) << 4);
    aoff[i] = ((tid & 7) ^ swz(r)) << 4;
  }

  StreamTile cur = decode_tile(p, t, ntN);
  int arow[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) arow[i] = token_src(p, cur, arow_t[i]);

  // Loaders: byte offsets of this thread's token-row chunks in A (aoffs) and of its weight rows
  // in the current group (boffs, from the uniform base bbase); all operands are below 4 GiB, so
  // the loads take a scalar base plus a 32-bit lane offset.  ld_rows: rows of the tile being
  // fetched (chunk groups past it are skipped).
  uint32_t aoffs[LA], boffs[NJ];
  const char* bbase;
  int ld_rows;
  bf16x8 areg[P][LA], breg[P][NJ][KH];
  // token-row registers of skipped chunk groups keep whatever they held: start them defined
#pragma unroll
  for (int s_ = 0; s_ < P; ++s_)
#pragma unroll
    for (int i = 0; i < LA; ++i) areg[s_][i] = bf16x8{};

#define MOE_STREAM_POINT(S)                                                                  \
  {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < LA; ++i) {                                         \
      const int row_ = p.a_gather ? arow[i] / p.a_div : arow[i];                             \
      aoffs[i] = (uint32_t)row_ * (uint32_t)p.lda_bytes + (uint32_t)aoff[i];                 \
    }                                                                                        \
    bbase = p.B + (int64_t)(S).group * p.b_group_bytes;                                      \
    ld_rows = (S).rows;                                                                      \
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
    _Pragma("unroll") for (int i = 0; i < LA; ++i)                                           \
        if (a_live<CH, NT, LA>(tid, i) && arow0[i] < ld_rows)                                \
            areg[SLOT][i] = *(const bf16x8*)(p.A + (aoffs[i] + off_));                       \
    _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                           \
      _Pragma("unroll") for (int h = 0; h < KH; ++h) breg[SLOT][j][h] =                      \
          *(const bf16x8*)(bbase + (boffs[j] + off_ + h * 64));                              \
  }

  MOE_STREAM_POINT(cur)
#pragma unroll
  for (int s_ = 0; s_ < P; ++s_)
    if (s_ < nk) MOE_STREAM_LOAD(s_, s_)

  // One K step: multiply LDS buffer ks&1 by weight slot QQ (both 32-wide halves); if ISSUE,
  // refill slot QQ with step ISTEP of the tile set up by MOE_STREAM_POINT; if STAGE_NEXT,
  // stage slot QQ+1's token rows into the other LDS buffer.  Operand fragment u = h·MI + i is
  // read from LDS two ahead of its MFMAs.
#define MOE_STREAM_AFRAG(U)                                                                  \
  (*(const bf16x8*)(sm + ((U) % MI * 16 + lr) * kRow +                                      \
                    ((((U) / MI) * 4 + lk) ^ swz((U) % MI * 16 + lr)) * 16))
#define MOE_STREAM_STEP(QQ, KS, ISSUE, ISTEP, STAGE_NEXT)                                  \
  {                                                                                        \
    const char* sm = smem[(KS) & 1];                                                       \
    bf16x8 af[KH * MI];                                                                    \
    af[0] = MOE_STREAM_AFRAG(0);                                                           \
    af[1] = MOE_STREAM_AFRAG(1);                                                           \
    _Pragma("unroll") for (int u = 0; u < KH * MI; ++u) {                                  \
      if (u + 2 < KH * MI) af[u + 2] = MOE_STREAM_AFRAG(u + 2);                            \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      _Pragma("unroll") for (int j = 0; j < NJ; ++j) acc[u % MI][j] =                      \
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u], breg[QQ][j][u / MI],              \
                                                  acc[u % MI][j], 0, 0, 0);                \
      __builtin_amdgcn_sched_barrier(0);                                                   \
    }                                                                                      \
    if (ISSUE) MOE_STREAM_LOAD(QQ, ISTEP)                                                  \
    if (STAGE_NEXT) {                                                                      \
      _Pragma("unroll") for (int i = 0; i < LA; ++i) if (a_live<CH, NT, LA>(tid, i))       \
          *(bf16x8*)(&smem[((KS) + 1) & 1][alds[i]]) = areg[((QQ) + 1) % P][i];            \
    }                                                                                      \
    __syncthreads();                                                                       \
  }

  // Stage step 0 of the first tile.  Every tile then starts with nothing in flight (the
  // prologue's loads may have been issued in any order, and the epilogue drains below): the
  // compiler's load counts at the head of the K loop are only exact if every path into it
  // agrees, and otherwise every round would wait for the whole ring.
#pragma unroll
  for (int i = 0; i < LA; ++i)
    if (a_live<CH, NT, LA>(tid, i)) *(bf16x8*)(&smem[0][alds[i]]) = areg[0][i];
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  for (;;) {
    // the next tile and its token rows, fetched now so they have arrived before they are used
    const int tn = t + per;
    const bool more = tn < hi;
    StreamTile nxt = cur;
    if (more) {
      nxt = decode_tile(p, tn, ntN);
#pragma unroll
      for (int i = 0; i < LA; ++i) arow[i] = token_src(p, nxt, arow_t[i]);
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
            Eh[(i * 16 + elk * 4 + r) * kLdH + col] = (__bf16)(silu_fast(acc[i][0][r]) * acc[i][1][r]);
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
      // fp16 rows: one power-of-two factor for the tile, from its largest |value| (reduced
      // over the lane, the wave, then the 8 waves through LDS)
      float sc = 1.0f, inv = 1.0f;
      if (p.c_scale) {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[i][j][r]));
        mx = wave_max_abs(mx);
        if ((etid & 63) == 0) tmax[wave] = mx;
        __syncthreads();
        mx = tmax[0];
#pragma unroll
        for (int w = 1; w < 8; ++w) mx = fmaxf(mx, tmax[w]);
        f16_block_scale(mx, &sc, &inv);
      }
      // tile origin (uniform) + 32-bit lane offsets
      char* Ct = (char*)p.C + ((int64_t)cur.row_start * p.ldc + cur.n_tile * BN) * 4;
      char* Ch = (char*)p.C + ((int64_t)cur.row_start * p.ldc + cur.n_tile * BN) * 2;
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
            const int lrow = c / kCpr, col = (c % kCpr) * 4;  // one row per wave
            const int row = q * kEpRows + lrow;
            if (p.c_scale) {
              // fp16 with the tile's power-of-two factor
              const f32x4 v = *(const f32x4*)(E + lrow * kLdE + col);
              if (row < cur.rows) {
                if (col < ncols) {
                  const f16x4 h = {(_Float16)(v[0] * sc), (_Float16)(v[1] * sc),
                                   (_Float16)(v[2] * sc), (_Float16)(v[3] * sc)};
                  *(f16x4*)(Ch + (uint32_t)(row * (int)p.ldc + col) * 2u) = h;
                }
                // the tile's factor for each of its kScaleCols-column blocks that holds columns
                if ((etid & 63) < BN / kScaleCols && (etid & 63) * kScaleCols < ncols)
                  p.c_scale[(int64_t)(cur.row_start + row) * p.ldcs +
                            cur.n_tile * (BN / kScaleCols) + (etid & 63)] = inv;
              }
            } else if (row < cur.rows && col < ncols) {
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
    // Stores and loads retire out of order, so once the stores above are pending the compiler
    // can no longer count the loads in flight and would drain the whole ring at the head of
    // every round that follows.  One explicit drain here, when the next tile's first loads have
    // had the epilogue's duration to land, keeps its counts exact for the rest of the tile.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (!more) break;
    cur = nxt;
    t = tn;
    if constexpr (!CROSS) {  // stage the next tile's step 0 (its loads are in)
#pragma unroll
      for (int i = 0; i < LA; ++i)
        if (a_live<CH, NT, LA>(tid, i)) *(bf16x8*)(&smem[0][alds[i]]) = areg[0][i];
      __syncthreads();
    }
  }
#undef MOE_STREAM_STEP
#undef MOE_STREAM_AFRAG
#undef MOE_STREAM_POINT
#undef MOE_STREAM_LOAD
}

template <int BM, int P, int EPI>
hipError_t launch_epi(const GemmParams& p, dim3 g, hipStream_t stream) {
  if ((p.Kdim / 64) % P == 0)
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
      return launch_bm<64, 4>(epi, p, max_mtiles, 1, stream);
    case TILE_STREAM_192:
      return launch_bm<192, 2>(epi, p, max_mtiles, 1, stream);
    case TILE_STREAM_128:
      return launch_bm<128, 4>(epi, p, max_mtiles, 1, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
