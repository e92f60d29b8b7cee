// Matrix-core grouped / dense GEMM (gfx950, bf16): every routed expert group of a bf16 layer,
// and the shared expert, which sees every token.  Groups of hundreds of rows reuse each weight
// byte that many times ("S23-J10" §3: a group's intensity is about t_e FLOP per weight byte),
// so there the limit is the MFMA pipes; decode-sized groups are bound by streaming their
// weights, which the direct-to-LDS weight ring does at HBM speed.  The kernel:
//  * 8 waves (two per SIMD) over a 256 x 256 output tile, 4 row blocks x 2 column halves of
//    128; each wave owns MI x 8 MFMA tiles of 16 x 16 (v_mfma_f32_16x16x32_bf16), MI <= 4.
//    Per 32-wide K step a wave reads MI A and 8 B fragments from LDS for 8 MI MFMAs.  A tile
//    of r rows is computed in P = ceil(r / 32) pairs of 16-row MFMA tiles spread so that every
//    SIMD runs P sets of 8 MFMAs (see mfma_tile), so a partly filled tile costs in proportion
//    to its rows, to 32 rows.
//  * K advances 64 per stage (128 bytes of every row, so each row's line is requested once).
//    Both operands move from L2/HBM straight into LDS with global_load_lds_dwordx4 (no staging
//    registers), token rows in a 2-stage ring and weights, which stream from HBM, in a
//    3-stage ring (32 KiB per operand stage, 160 KiB of LDS).
//  * The fragments of each 32-wide K step are read from LDS while the MFMAs of the previous
//    one run (A fragments in place as their rows finish, B fragments into a second set), so
//    LDS latency is hidden inside the wave; one barrier per stage publishes the next stage
//    and frees the one just read.
//  * LDS rows are 128 bytes; the eight 16-byte chunks of row r are XOR-swizzled by
//    (r >> 1) & 7, which keeps the 16-row operand fetches conflict-free.
//  * Token rows are gathered through the dispatch permutation by the DMA addresses themselves.
//  * Persistent, XCD-aware schedule over logical tiles ordered expert-major, then N tile, then
//    M tile, so the tiles that share an expert's weights or rows meet in one XCD's L2.
//  * Epilogues are assembled in LDS (reusing the ring) and leave as whole chunks: fused
//    SiLU·up (a wave's 8 column tiles are 4 gate/up pairs), fp32 store with an optional row
//    scale, fp16 store with one power-of-two factor per tile, or the weighted fp32 atomic
//    combine.
#include "kernels.h"
#include "silu.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;       // tile rows (tokens)
constexpr int kBN = 256;       // tile weight rows (output columns; half of them for SwiGLU)
constexpr int kRow = 128;      // LDS bytes per staged row per stage (64 bf16: two MFMA K steps)
constexpr int kSA = 2, kSB = 3;             // ring depths: token rows (L2-resident), weights
constexpr int kAStage = kBM * kRow, kBStage = kBN * kRow;  // 32 KiB each
constexpr int kLds = kSA * kAStage + kSB * kBStage;       // 160 KiB

// s_waitcnt immediate (gfx9 layout): at most `vm` vector-memory and `lgkm` LDS/scalar
// operations of this wave outstanding.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

// Barrier with explicit waits and no memory fence; the empty asm statements keep the compiler
// from moving LDS accesses or DMA issues across it.
template <int VM, int LGKM>
__device__ __forceinline__ void barrier_after() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, LGKM));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Barrier for LDS traffic only: waits for this wave's LDS operations and leaves its
// vector-memory operations (stores, prefetches) in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One stage of one operand (up to 256 rows x 128 bytes) by one of NW waves: instruction i fills
// staged rows [8 (wave + NW i), +8), so the first N instructions of the 8 waves fill rows
// [0, 64 N); src holds the lane's 32-bit byte offsets from base.
template <int NW, int N = kBM / 8 / NW>
__device__ __forceinline__ void dma_operand(const char* base, const uint32_t* src, uint32_t off,
                                            char* stage, int wave) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_global_load_lds(base + (src[i] + off), stage + (wave + NW * i) * 1024, 16,
                                     0, 0);
}

// Fragment u of this wave in a stage: A fragments 0..7 (16 rows each) at la + 1024 u, B
// fragments at lb + boff(j).  Every fragment row has the same (row >> 1) & 3, so one swizzled
// lane offset per operand serves all of them and the rest is an immediate offset.
template <bool SWIGLU>
__device__ __forceinline__ int boff(int j) {
  return SWIGLU ? ((j < 4 ? 0 : kBN / 2) + (j & 3) * 16) * kRow : j * 16 * kRow;
}

template <int MI, bool SWIGLU>
__device__ __forceinline__ void read_frags(const char* la, const char* lb, bf16x8* af,
                                           bf16x8* bfr) {
#pragma unroll
  for (int i = 0; i < MI; ++i) af[i] = *(const bf16x8*)(la + i * 16 * kRow);
#pragma unroll
  for (int j = 0; j < 8; ++j) bfr[j] = *(const bf16x8*)(lb + boff<SWIGLU>(j));
}

// The 8·MI MFMAs of one 32-wide K step, reading the next step's fragments in between: one of
// the 8 next B fragments (into the other B set) after every MI MFMAs, A fragment i in place
// right after row i's 8 MFMAs.
template <int MI, bool SWIGLU>
__device__ __forceinline__ void mma_stage(f32x4 (*acc)[8], bf16x8* af, const bf16x8* bfr,
                                          const char* la_n, const char* lb_n, bf16x8* bfr_n) {
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      if ((i * 8 + j + 1) % MI == 0) {
        const int b = (i * 8 + j + 1) / MI - 1;
        bfr_n[b] = *(const bf16x8*)(lb_n + boff<SWIGLU>(b));
      }
    }
    af[i] = *(const bf16x8*)(la_n + i * 16 * kRow);
  }
}

constexpr int kNW = 8;                 // waves: 4 along M x 2 along N
constexpr int kNT = 64 * kNW;          // threads
constexpr int kDma = kBM / 8 / kNW;    // 1 KiB DMA instructions per wave per full operand stage

// First row of wave row block wm when blocks 0 and 1 hold mi_hi and blocks 2 and 3 mi_lo
// 16-row MFMA tiles.
__device__ __forceinline__ int block_row0(int wm, int mi_hi, int mi_lo) {
  return wm < 2 ? wm * 16 * mi_hi : 32 * mi_hi + (wm - 2) * 16 * mi_lo;
}

// One output tile.  Wave (wm, wn) owns MI x 8 MFMA tiles of 16 x 16: columns [128 wn, +128)
// and MI 16-row tiles starting at block_row0(wm).  A tile of `rows` rows is computed as
// P = ceil(rows / 32) pairs of 16-row tiles: row blocks 0 and 1 take mi_hi = ceil(P / 2) each,
// blocks 2 and 3 mi_lo = floor(P / 2).  The two waves that share a SIMD (waves w and w + 4)
// hold one block of each kind, so every SIMD runs P sets of 8 MFMAs per K step and a partly
// filled tile (a group's last one) costs in proportion to its rows, to 32 rows.  Only the
// token rows [0, 32 P) are fetched; MI is also this wave's count of 1 KiB token-row DMA
// instructions per stage.
template <int MI, int EPI>
__device__ __forceinline__ void mfma_tile(const GemmParams& p, char* smem, int tid, int wave,
                                          int group, int row_start, int rows, int n_tile,
                                          int ns, int mi_hi, int mi_lo) {
  constexpr bool kSwiglu = EPI == EPI_SWIGLU;
  constexpr int MIA = MI > 0 ? MI : 1;  // array extent
  static_assert(MI >= 0 && MI <= 4 && kDma == 4 && 4 * kDma < 64, "tile shape, vmcnt range");
  char* const sA = smem;                  // token-row ring, kSA stages
  char* const sB = smem + kSA * kAStage;  // weight ring, kSB stages
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lk = lane >> 4;

  // Lane offsets (within a stage) of this wave's first A and B fragment rows, for each 32-wide
  // half of the stage.  For SwiGLU the tile's first 128 B rows are gate rows and the next 128
  // the matching up rows, and a wave's column tiles j and j + 4 are a gate/up pair.
  const int wrow0 = block_row0(wm, mi_hi, mi_lo);
  const int la_row = (wrow0 + lr) * kRow;
  const int lb_row = ((kSwiglu ? wn * 64 : wn * 128) + lr) * kRow;
  const int ch0 = (lk ^ swz(lr)) << 4, ch1 = ((4 + lk) ^ swz(lr)) << 4;

  // ---- global source of each DMA chunk this lane issues per stage ----------------------------
  const char* gbase = p.B + (int64_t)group * p.b_group_bytes;
  uint32_t srcA[kDma], srcB[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int r = 8 * (wave + kNW * i) + (lane >> 3);  // staged row of either operand
    const int chunk = (lane & 7) ^ swz(r);            // logical chunk kept in this slot
    const int pos = row_start + min(r, rows - 1);
    const int arow = p.a_gather ? p.a_gather[pos] / p.a_div : pos;
    srcA[i] = (uint32_t)arow * (uint32_t)p.lda_bytes + chunk * 16;
    int brow;
    if (kSwiglu) {
      const int n = n_tile * (kBN / 2) + (r & (kBN / 2 - 1));
      brow = n < p.N ? (r < kBN / 2 ? n : p.N + n) : 0;
    } else {
      const int n = n_tile * kBN + r;
      brow = n < p.N ? n : 0;
    }
    srcB[i] = (uint32_t)brow * (uint32_t)p.ldb_bytes + chunk * 16;
  }

  f32x4 acc[MIA][8];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // every wave is done with the previous tile's LDS (epilogue staging) before new DMA lands
  barrier_after<0, 0>();
  // Ring schedule (per wave, in issue order): prologue A0 B0 A1 B1 B2, then before stage g+1
  // is used, A(g+2) B(g+3).  Token rows run two stages ahead, weights three, so up to 64 KiB
  // of weights per CU are in flight.  A stage of token rows is MI instructions per wave, one
  // of weights kDma; the waits below count exactly those.
  dma_operand<kNW, MI>(p.A, srcA, 0, sA, wave);
  dma_operand<kNW>(gbase, srcB, 0, sB, wave);
  if (ns > 1) {
    dma_operand<kNW, MI>(p.A, srcA, kRow, sA + kAStage, wave);
    dma_operand<kNW>(gbase, srcB, kRow, sB + kBStage, wave);
  }
  if (ns > 2) dma_operand<kNW>(gbase, srcB, 2 * kRow, sB + 2 * kBStage, wave);

  // stage 0 published, its first half's fragments read (A fragments are refilled in place,
  // B fragments alternate between two sets)
  bf16x8 af0[MIA], bf0[8], bf1[8];
  if (ns > 2)  // A1 B1 B2 were issued after B0 and may still fly
    barrier_after<MI + 2 * kDma, 0>();
  else
    barrier_after<0, 0>();
  if constexpr (MI > 0) read_frags<MI, kSwiglu>(sA + la_row + ch0, sB + lb_row + ch0, af0, bf0);

  // Stage g's MFMAs: first half (step 2g) while reading the second half's fragments from
  // the same stage; then publish stage g+1 (this wave's copies landed; every wave has read
  // all of stage g, so its buffers are free), refill them with A(g+2) and B(g+3), and run the
  // second half (step 2g+1) while reading stage g+1's first half.
  for (int g = 0; g < ns; ++g) {
    const char* ca = sA + (g % kSA) * kAStage;
    const char* cb = sB + (g % kSB) * kBStage;
    if constexpr (MI > 0)
      mma_stage<MI, kSwiglu>(acc, af0, bf0, ca + la_row + ch1, cb + lb_row + ch1, bf1);
    if (g + 1 < ns) {
      if (g + 2 < ns)  // B(g+2) went out after A(g+1) and may still fly
        barrier_after<kDma, 0>();
      else
        barrier_after<0, 0>();
      if (g + 2 < ns)
        dma_operand<kNW, MI>(p.A, srcA, (uint32_t)(g + 2) * kRow, sA + (g % kSA) * kAStage,
                             wave);
      if (g + 3 < ns)
        dma_operand<kNW>(gbase, srcB, (uint32_t)(g + 3) * kRow, sB + (g % kSB) * kBStage, wave);
    }
    // after the last stage these reads fetch unused leftovers
    const char* na = sA + ((g + 1) % kSA) * kAStage;
    const char* nb = sB + ((g + 1) % kSB) * kBStage;
    if constexpr (MI > 0)
      mma_stage<MI, kSwiglu>(acc, af0, bf1, na + la_row + ch0, nb + lb_row + ch0, bf0);
  }

  // ---- epilogue (staged in the ring's LDS) ---------------------------------------------------
  // Lane (lr, lk) holds rows wrow0 + 16 i + 4 lk + r of column tile j in acc[i][j][r].  The
  // thread index is laundered through an empty asm so the store offsets below are computed
  // here, not hoisted out of the tile loop into registers (and spilled).
  int etid = tid;
  asm volatile("" : "+v"(etid));
  const int elr = etid & 15, elk = (etid >> 4) & 3;
  barrier_after<0, 0>();  // all waves are done reading the ring
  if constexpr (kSwiglu) {
    // H tile: up to 256 rows x 128 columns of the layer dtype, 272-byte LDS rows
    constexpr int kLdH = kBN / 2 + 8;
    __bf16* Eh = (__bf16*)smem;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wrow0 + i * 16 + elk * 4 + r;
          const int col = wn * 64 + j * 16 + elr;
          Eh[row * kLdH + col] = (__bf16)(silu_fast(acc[i][j][r]) * acc[i][j + 4][r]);
        }
    barrier_after<0, 0>();
    constexpr int kCpr = kBN / 2 / 8;  // 16 chunks of 8 values per H row
    char* Ht = (char*)p.C + ((int64_t)row_start * p.ldc + n_tile * (kBN / 2)) * 2;
    const int ncols = min(kBN / 2, p.N - n_tile * (kBN / 2));
    const int nmm = (rows * kCpr + kNT - 1) / kNT;
    for (int mm = 0; mm < nmm; ++mm) {
      const int c = etid + kNT * mm;
      const int row = c / kCpr, ch = c % kCpr;
      if (row < rows && ch * 8 < ncols)
        *(bf16x8*)(Ht + (uint32_t)(row * (int)p.ldc + ch * 8) * 2u) =
            *(const bf16x8*)(Eh + row * kLdH + ch * 8);
    }
  } else if constexpr (EPI == EPI_STORE) {
    // fp32 tile in four passes, one per wave row block (up to 64 rows x 256 columns, 1040-byte
    // LDS rows), each written to LDS by the two waves that own it
    constexpr int kLdE = kBN + 4;
    float* E = (float*)smem;
    // fp16 rows: one power-of-two factor for the tile, from its largest |value| (reduced over
    // the lane, the wave, then the 8 waves through LDS past the staging area)
    float sc = 1.0f, inv = 1.0f;
    if (p.c_scale) {
      float* tmax = (float*)(smem + kLds - 64);
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[i][j][r]));
      mx = wave_max_abs(mx);
      if ((etid & 63) == 0) tmax[wave] = mx;
      barrier_after<0, 0>();
      mx = tmax[0];
#pragma unroll
      for (int w = 1; w < kNW; ++w) mx = fmaxf(mx, tmax[w]);
      f16_block_scale(mx, &sc, &inv);
    }
    char* Ct = (char*)p.C + ((int64_t)row_start * p.ldc + n_tile * kBN) * 4;
    char* Ch = (char*)p.C + ((int64_t)row_start * p.ldc + n_tile * kBN) * 2;
    const float* rs = p.row_scale ? p.row_scale + row_start : nullptr;
    const int ncols = min(kBN, p.N - n_tile * kBN);
    constexpr int kCpr = kBN / 4;  // 16-byte chunks per fp32 row
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int prow0 = block_row0(pass, mi_hi, mi_lo);
      const int pmi = pass < 2 ? mi_hi : mi_lo;
      if (pmi > 0 && prow0 < rows) {  // uniform
        if (wm == pass) {
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                E[(i * 16 + elk * 4 + r) * kLdE + wn * 128 + j * 16 + elr] = acc[i][j][r];
        }
        barrier_after<0, 0>();
        for (int mm = 0; mm < 2 * pmi; ++mm) {  // 16 pmi rows of kCpr chunks
          const int c = etid + kNT * mm;
          const int lrow = c / kCpr, col = (c % kCpr) * 4;  // one row per wave
          const int row = prow0 + lrow;
          if (p.c_scale) {
            // fp16 with the tile's power-of-two factor
            const f32x4 v = *(const f32x4*)(E + lrow * kLdE + col);
            if (row < rows) {
              if (col < ncols) {
                const f16x4 h = {(_Float16)(v[0] * sc), (_Float16)(v[1] * sc),
                                 (_Float16)(v[2] * sc), (_Float16)(v[3] * sc)};
                *(f16x4*)(Ch + (uint32_t)(row * (int)p.ldc + col) * 2u) = h;
              }
              if ((etid & 63) == 0) p.c_scale[(int64_t)(row_start + row) * p.ldcs + n_tile] = inv;
            }
          } else if (row < rows && col < ncols) {
            f32x4 v = *(const f32x4*)(E + lrow * kLdE + col);
            if (rs) v *= rs[row];
            *(f32x4*)(Ct + (uint32_t)(row * (int)p.ldc + col) * 4u) = v;
          }
        }
        barrier_after<0, 0>();
      }
    }
  } else {  // EPI_ATOMIC_COMBINE
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wrow0 + i * 16 + elk * 4 + r;
        if (row >= rows) continue;
        const int a = p.perm[row_start + row];
        const float w = p.topk_w[a];
        float* dst = p.acc_out + (int64_t)(a / p.topk) * p.ldo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n_tile * kBN + wn * 128 + j * 16 + elr;
          if (n < p.N) unsafeAtomicAdd(dst + n, w * acc[i][j][r]);
        }
      }
  }
}

// Logical tile t: expert-major, then N tile, then M tile (the m-tiles of one expert are
// entries [first, first + cnt) of the tile map and own logical tiles [first·ntN, (first+cnt)·ntN));
// dense mode (no tile map) has one group of mt_total M tiles.
__device__ __forceinline__ void decode_mtile(const GemmParams& p, int t, int ntN, int mt_total,
                                             int* group, int* row_start, int* rows,
                                             int* n_tile) {
  const int q = t / ntN;
  int first = 0, cnt = mt_total;
  if (p.tiles) {
    first = load_uniform(p.tiles, q * kTileStride + 4);
    cnt = load_uniform(p.tiles, q * kTileStride + 5);
  }
  const int l = t - first * ntN;
  *n_tile = l / cnt;
  const int m = first + l % cnt;
  if (p.tiles) {
    *group = load_uniform(p.tiles, m * kTileStride + 0);
    *row_start = load_uniform(p.tiles, m * kTileStride + 1);
    *rows = load_uniform(p.tiles, m * kTileStride + 2);
  } else {
    *group = 0;
    *row_start = m * kBM;
    *rows = min(kBM, p.M - m * kBM);
  }
}

template <int EPI>
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[kLds];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  constexpr int BNE = EPI == EPI_SWIGLU ? kBN / 2 : kBN;  // output columns per tile
  const int ntN = (p.N + BNE - 1) / BNE;
  const int mt_total = p.tiles ? load_uniform(p.tile_count, 0) : (p.M + kBM - 1) / kBM;
  const int nt = mt_total * ntN;
  const int xcd = blockIdx.x % kXcds, per = gridDim.x / kXcds, jb = blockIdx.x / kXcds;
  const int lo = (int)((int64_t)nt * xcd / kXcds), hi = (int)((int64_t)nt * (xcd + 1) / kXcds);
  const int ns = p.Kdim / 64;  // DMA stages (Kdim is a multiple of 64)

  for (int t = lo + jb; t < hi; t += per) {
    // ---- logical tile: expert-major, then N tile, then M tile -------------------------------
    const int q = t / ntN;
    int first = 0, cnt = mt_total;
    if (p.tiles) {
      first = load_uniform(p.tiles, q * kTileStride + 4);
      cnt = load_uniform(p.tiles, q * kTileStride + 5);
    }
    const int l = t - first * ntN;
    const int n_tile = l / cnt;
    const int m = first + l % cnt;
    int group = 0, row_start = m * kBM, rows = min(kBM, p.M - m * kBM);
    if (p.tiles) {
      group = load_uniform(p.tiles, m * kTileStride + 0);
      row_start = load_uniform(p.tiles, m * kTileStride + 1);
      rows = load_uniform(p.tiles, m * kTileStride + 2);
    }
    // 32-row pairs of MFMA row tiles that hold rows, split over the wave row blocks
    const int pairs = min(max((rows + 31) >> 5, 1), 8);
    const int mi_hi = (pairs + 1) >> 1, mi_lo = pairs >> 1;
    switch (wave < 4 ? mi_hi : mi_lo) {  // waves 0-3 hold row blocks 0 and 1
      case 0:
        mfma_tile<0, EPI>(p, smem, tid, wave, group, row_start, rows, n_tile, ns, mi_hi, mi_lo);
        break;
      case 1:
        mfma_tile<1, EPI>(p, smem, tid, wave, group, row_start, rows, n_tile, ns, mi_hi, mi_lo);
        break;
      case 2:
        mfma_tile<2, EPI>(p, smem, tid, wave, group, row_start, rows, n_tile, ns, mi_hi, mi_lo);
        break;
      case 3:
        mfma_tile<3, EPI>(p, smem, tid, wave, group, row_start, rows, n_tile, ns, mi_hi, mi_lo);
        break;
      default:
        mfma_tile<4, EPI>(p, smem, tid, wave, group, row_start, rows, n_tile, ns, mi_hi, mi_lo);
        break;
    }
  }
}

// ---- batches of at most 64 tokens (decode) -----------------------------------------------
// Every tile then has at most 64 rows, so a token-row stage takes 8 KiB, and the LDS holds the
// two rings (2 x 8 KiB of token rows, 3 x 32 KiB of weights) and a separate 48 KiB staging
// area for the epilogue.  The rings run on across the tiles of a work-group: the refills of a
// tile's last three stages fetch the next tile's first stages (global stage G = the work-group's
// stage count, ring slots G % 2 and G % 3), so the next tile starts with its prologue in LDS
// and the weight stream never stops for a tile's epilogue or its first loads.
constexpr int kSmallRows = 64;
constexpr int kSmallAStage = kSmallRows * kRow;             // 8 KiB
constexpr int kSmallStg = 2 * kSmallAStage + 3 * kBStage;  // staging area: [112 KiB, 160 KiB)

// The lane's DMA source offsets for one tile: token rows (gathered) and weight rows.
template <bool SWIGLU>
__device__ __forceinline__ void tile_sources(const GemmParams& p, int lane, int wave,
                                             int row_start, int rows, int n_tile, uint32_t* sa,
                                             uint32_t* sb) {
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int r = 8 * (wave + kNW * i) + (lane >> 3);  // staged row of either operand
    const int chunk = (lane & 7) ^ swz(r);            // logical chunk kept in this slot
    const int pos = row_start + min(r, rows - 1);
    const int arow = p.a_gather ? p.a_gather[pos] / p.a_div : pos;
    sa[i] = (uint32_t)arow * (uint32_t)p.lda_bytes + chunk * 16;
    int brow;
    if (SWIGLU) {
      const int n = n_tile * (kBN / 2) + (r & (kBN / 2 - 1));
      brow = n < p.N ? (r < kBN / 2 ? n : p.N + n) : 0;
    } else {
      const int n = n_tile * kBN + r;
      brow = n < p.N ? n : 0;
    }
    sb[i] = (uint32_t)brow * (uint32_t)p.ldb_bytes + chunk * 16;
  }
}

// Token-row DMA of one stage with a run-time count of instructions (0 or 1 here).
__device__ __forceinline__ void dma_rows_small(int n, const char* base, const uint32_t* src,
                                               uint32_t off, char* stage, int wave) {
  if (n > 0) dma_operand<kNW, 1>(base, src, off, stage, wave);
}

// One tile of a small batch.  MI (0 or 1) is this wave's count of 16-row MFMA tiles and of
// token-row DMA instructions per stage; nx_* describe the work-group's next tile (nx_group < 0:
// none), nx_mi this wave's MI there.  G0 is the global index of this tile's stage 0; `pre`:
// its stages 0-2 were issued by the previous tile.
template <int MI, int EPI>
__device__ __forceinline__ void small_tile(const GemmParams& p, char* smem, int tid, int wave,
                                           int group, int row_start, int rows, int n_tile,
                                           int ns, int mi_hi, int mi_lo, int G0, bool pre,
                                           int nx_group, int nx_row_start, int nx_rows,
                                           int nx_n_tile, int nx_mi) {
  constexpr bool kSwiglu = EPI == EPI_SWIGLU;
  static_assert(MI == 0 || MI == 1, "at most 64 rows: one 16-row MFMA tile per wave");
  char* const sA = smem;                      // token-row ring, 2 stages of 8 KiB
  char* const sB = smem + 2 * kSmallAStage;   // weight ring, 3 stages
  char* const stg = smem + kSmallStg;         // epilogue staging
  const auto a_at = [&](int G) { return sA + (G & 1) * kSmallAStage; };
  const auto b_at = [&](int G) { return sB + (G % 3) * kBStage; };
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lk = lane >> 4;
  const int wrow0 = block_row0(wm, mi_hi, mi_lo);
  const int la_row = (wrow0 + lr) * kRow;
  const int lb_row = ((kSwiglu ? wn * 64 : wn * 128) + lr) * kRow;
  const int ch0 = (lk ^ swz(lr)) << 4, ch1 = ((4 + lk) ^ swz(lr)) << 4;

  uint32_t srcA[kDma], srcB[kDma], nsA[kDma], nsB[kDma];
  tile_sources<kSwiglu>(p, lane, wave, row_start, rows, n_tile, srcA, srcB);
  const char* gbase = p.B + (int64_t)group * p.b_group_bytes;
  const bool nxt = nx_group >= 0;
  const char* nbase = p.B + (int64_t)(nxt ? nx_group : 0) * p.b_group_bytes;
  if (nxt) tile_sources<kSwiglu>(p, lane, wave, nx_row_start, nx_rows, nx_n_tile, nsA, nsB);

  f32x4 acc[1][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[0][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (!pre) {
    // first tile of the work-group: prologue A0 B0 A1 B1 B2
    barrier_after<0, 0>();
    dma_rows_small(MI, p.A, srcA, 0, a_at(G0), wave);
    dma_operand<kNW>(gbase, srcB, 0, b_at(G0), wave);
    if (ns > 1) {
      dma_rows_small(MI, p.A, srcA, kRow, a_at(G0 + 1), wave);
      dma_operand<kNW>(gbase, srcB, kRow, b_at(G0 + 1), wave);
    }
    if (ns > 2) dma_operand<kNW>(gbase, srcB, 2 * kRow, b_at(G0 + 2), wave);
    if (ns > 2)  // A1 B1 B2 were issued after B0 and may still fly
      barrier_after<MI + 2 * kDma, 0>();
    else
      barrier_after<0, 0>();
  } else {
    // stages 0-2 came with the previous tile's last refills: drain them and its stores
    barrier_after<0, 0>();
  }

  bf16x8 af0[1], bf0[8], bf1[8];
  if constexpr (MI > 0)
    read_frags<1, kSwiglu>(a_at(G0) + la_row + ch0, b_at(G0) + lb_row + ch0, af0, bf0);

  for (int g = 0; g < ns; ++g) {
    const int G = G0 + g;
    if constexpr (MI > 0)
      mma_stage<1, kSwiglu>(acc, af0, bf0, a_at(G) + la_row + ch1, b_at(G) + lb_row + ch1, bf1);
    // Publish stage g+1: this wave's copies landed (B(G+2), refilled one stage ago after
    // A(G+1), may still fly, unless nothing refilled it); every wave has read stage g, whose
    // slots take global stages G+2 (token rows) and G+3 (weights) of this tile or the next.
    if (g + 1 < ns) {
      if (g + 2 < ns || nxt || g == 0)
        barrier_after<kDma, 0>();
      else
        barrier_after<0, 0>();
    } else {
      lds_barrier();  // the last stage: nothing to wait for, the slots are free
    }
    if (g + 2 < ns)
      dma_rows_small(MI, p.A, srcA, (uint32_t)(g + 2) * kRow, a_at(G + 2), wave);
    else if (nxt)
      dma_rows_small(nx_mi, p.A, nsA, (uint32_t)(g + 2 - ns) * kRow, a_at(G + 2), wave);
    if (g + 3 < ns)
      dma_operand<kNW>(gbase, srcB, (uint32_t)(g + 3) * kRow, b_at(G + 3), wave);
    else if (nxt)
      dma_operand<kNW>(nbase, nsB, (uint32_t)(g + 3 - ns) * kRow, b_at(G + 3), wave);
    if constexpr (MI > 0) {
      if (g + 1 < ns)
        mma_stage<1, kSwiglu>(acc, af0, bf1, a_at(G + 1) + la_row + ch0, b_at(G + 1) + lb_row + ch0,
                              bf0);
      else
        mma_stage<1, kSwiglu>(acc, af0, bf1, a_at(G) + la_row + ch0, b_at(G) + lb_row + ch0, bf0);
    }
  }

  // ---- epilogue, staged in its own LDS area (only LDS barriers: the next tile's loads fly) --
  int etid = tid;
  asm volatile("" : "+v"(etid));
  const int elr = etid & 15, elk = (etid >> 4) & 3;
  if constexpr (kSwiglu) {
    constexpr int kLdH = kBN / 2 + 8;  // up to 64 rows x 128 columns, 272-byte rows
    __bf16* Eh = (__bf16*)stg;
    if constexpr (MI > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wrow0 + elk * 4 + r;
          const int col = wn * 64 + j * 16 + elr;
          Eh[row * kLdH + col] = (__bf16)(silu_fast(acc[0][j][r]) * acc[0][j + 4][r]);
        }
    }
    lds_barrier();
    constexpr int kCpr = kBN / 2 / 8;  // 16 chunks of 8 values per H row
    char* Ht = (char*)p.C + ((int64_t)row_start * p.ldc + n_tile * (kBN / 2)) * 2;
    const int ncols = min(kBN / 2, p.N - n_tile * (kBN / 2));
#pragma unroll
    for (int mm = 0; mm < kSmallRows * kCpr / kNT; ++mm) {
      const int c = etid + kNT * mm;
      const int row = c / kCpr, ch = c % kCpr;
      if (row < rows && ch * 8 < ncols)
        *(bf16x8*)(Ht + (uint32_t)(row * (int)p.ldc + ch * 8) * 2u) =
            *(const bf16x8*)(Eh + row * kLdH + ch * 8);
    }
  } else if constexpr (EPI == EPI_STORE) {
    constexpr int kLdE = kBN + 4;  // 16 rows x 256 columns per pass, 1040-byte rows
    float* E = (float*)stg;
    float sc = 1.0f, inv = 1.0f;
    if (p.c_scale) {
      float* tmax = (float*)(stg + 32 * 1024);
      float mx = 0.0f;
      if constexpr (MI > 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[0][j][r]));
      }
      mx = wave_max_abs(mx);
      if ((etid & 63) == 0) tmax[wave] = mx;
      lds_barrier();
      mx = tmax[0];
#pragma unroll
      for (int w = 1; w < kNW; ++w) mx = fmaxf(mx, tmax[w]);
      f16_block_scale(mx, &sc, &inv);
    }
    char* Ct = (char*)p.C + ((int64_t)row_start * p.ldc + n_tile * kBN) * 4;
    char* Ch = (char*)p.C + ((int64_t)row_start * p.ldc + n_tile * kBN) * 2;
    const float* rs = p.row_scale ? p.row_scale + row_start : nullptr;
    const int ncols = min(kBN, p.N - n_tile * kBN);
    constexpr int kCpr = kBN / 4;  // 16-byte chunks per fp32 row
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int prow0 = block_row0(pass, mi_hi, mi_lo);
      const int pmi = pass < 2 ? mi_hi : mi_lo;
      if (pmi > 0 && prow0 < rows) {  // uniform
        if constexpr (MI > 0) {
          if (wm == pass) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                E[(elk * 4 + r) * kLdE + wn * 128 + j * 16 + elr] = acc[0][j][r];
          }
        }
        lds_barrier();
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {  // 16 rows of kCpr chunks, one row per wave
          const int c = etid + kNT * mm;
          const int lrow = c / kCpr, col = (c % kCpr) * 4;
          const int row = prow0 + lrow;
          if (p.c_scale) {
            const f32x4 v = *(const f32x4*)(E + lrow * kLdE + col);
            if (row < rows) {
              if (col < ncols) {
                const f16x4 h = {(_Float16)(v[0] * sc), (_Float16)(v[1] * sc),
                                 (_Float16)(v[2] * sc), (_Float16)(v[3] * sc)};
                *(f16x4*)(Ch + (uint32_t)(row * (int)p.ldc + col) * 2u) = h;
              }
              if ((etid & 63) == 0) p.c_scale[(int64_t)(row_start + row) * p.ldcs + n_tile] = inv;
            }
          } else if (row < rows && col < ncols) {
            f32x4 v = *(const f32x4*)(E + lrow * kLdE + col);
            if (rs) v *= rs[row];
            *(f32x4*)(Ct + (uint32_t)(row * (int)p.ldc + col) * 4u) = v;
          }
        }
        lds_barrier();
      }
    }
  } else {  // EPI_ATOMIC_COMBINE
    if constexpr (MI > 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wrow0 + elk * 4 + r;
        if (row >= rows) continue;
        const int a = p.perm[row_start + row];
        const float w = p.topk_w[a];
        float* dst = p.acc_out + (int64_t)(a / p.topk) * p.ldo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n_tile * kBN + wn * 128 + j * 16 + elr;
          if (n < p.N) unsafeAtomicAdd(dst + n, w * acc[0][j][r]);
        }
      }
    }
  }
}

template <int EPI>
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_small_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[kLds];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int BNE = EPI == EPI_SWIGLU ? kBN / 2 : kBN;
  const int ntN = (p.N + BNE - 1) / BNE;
  const int mt_total = p.tiles ? load_uniform(p.tile_count, 0) : (p.M + kBM - 1) / kBM;
  const int nt = mt_total * ntN;
  const int xcd = blockIdx.x % kXcds, per = gridDim.x / kXcds, jb = blockIdx.x / kXcds;
  const int lo = (int)((int64_t)nt * xcd / kXcds), hi = (int)((int64_t)nt * (xcd + 1) / kXcds);
  const int ns = p.Kdim / 64;

  // The next tile's first three stages come with this tile's last three refills, which needs
  // three stages per tile; shorter reductions run each tile with its own prologue.
  const bool cross = ns >= 3;
  int G0 = 0;
  for (int t = lo + jb; t < hi; t += per) {
    int group, row_start, rows, n_tile;
    decode_mtile(p, t, ntN, mt_total, &group, &row_start, &rows, &n_tile);
    int nx_group = -1, nx_row_start = 0, nx_rows = 1, nx_n_tile = 0, nx_mi = 0;
    if (cross && t + per < hi) {
      decode_mtile(p, t + per, ntN, mt_total, &nx_group, &nx_row_start, &nx_rows, &nx_n_tile);
      nx_mi = wave < 4 ? 1 : (nx_rows > 32 ? 1 : 0);
    }
    const int mi_hi = 1, mi_lo = rows > 32 ? 1 : 0;  // rows <= 64 (the host guarantees it)
    const bool pre = cross && G0 > 0;
    if (wave < 4 || mi_lo)
      small_tile<1, EPI>(p, smem, tid, wave, group, row_start, rows, n_tile, ns, mi_hi, mi_lo, G0,
                         pre, nx_group, nx_row_start, nx_rows, nx_n_tile, nx_mi);
    else
      small_tile<0, EPI>(p, smem, tid, wave, group, row_start, rows, n_tile, ns, mi_hi, mi_lo, G0,
                         pre, nx_group, nx_row_start, nx_rows, nx_n_tile, nx_mi);
    G0 += ns;
  }
}

template <int EPI>
hipError_t launch_epi(const GemmParams& p, int64_t max_mtiles, hipStream_t stream) {
  constexpr int BNE = EPI == EPI_SWIGLU ? kBN / 2 : kBN;
  const int64_t ntN = (p.N + BNE - 1) / BNE;
  const int64_t want = max_mtiles * ntN;
  int64_t grid = want < kCus ? want : kCus;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  const bool small = p.tiles ? (p.rows_bound > 0 && p.rows_bound <= kSmallRows)
                             : p.M <= kSmallRows;
  if (small)
    hipLaunchKernelGGL((mfma_small_kernel<EPI>), dim3((unsigned)grid), dim3(kNT), 0, stream, p);
  else
    hipLaunchKernelGGL((mfma_kernel<EPI>), dim3((unsigned)grid), dim3(kNT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_gemm(Epilogue epi, const GemmParams& p, int64_t max_mtiles,
                            hipStream_t stream) {
  if (max_mtiles <= 0) return hipSuccess;
  if (p.B2 || p.col_bias) return hipErrorInvalidValue;  // router-only features
  switch (epi) {
    case EPI_SWIGLU:
      return launch_epi<EPI_SWIGLU>(p, max_mtiles, stream);
    case EPI_STORE:
      return launch_epi<EPI_STORE>(p, max_mtiles, stream);
    case EPI_ATOMIC_COMBINE:
      return launch_epi<EPI_ATOMIC_COMBINE>(p, max_mtiles, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
