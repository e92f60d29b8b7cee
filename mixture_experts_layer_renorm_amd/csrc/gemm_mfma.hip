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
//    3-stage ring (32 KiB per operand stage, 160 KiB of LDS; decode batches, whose tiles have
//    at most 64 rows, use 8 KiB token-row stages).
//  * The fragments of each 32-wide K step are read from LDS while the MFMAs of the previous
//    one run (A fragments in place as their rows finish, B fragments into a second set), so
//    LDS latency is hidden inside the wave; one barrier per stage publishes the next stage
//    and frees the one just read.
//  * LDS rows are 128 bytes; the eight 16-byte chunks of row r are XOR-swizzled by
//    (r >> 1) & 7, which keeps the 16-row operand fetches conflict-free.
//  * Token rows are gathered through the dispatch permutation by the DMA addresses themselves.
//    Weight DMAs are non-temporal (see kWeightAux).
//  * Persistent, XCD-aware schedule over logical tiles ordered expert-major, then N tile, then
//    M tile, so the tiles that share an expert's weights or rows meet in one XCD's L2.  With
//    three or more K stages the rings run on across a work-group's tiles: a tile's last
//    refills fetch the next tile's first stages.
//  * Epilogues store straight from the accumulators, which hold the transposed tile (weights
//    are the MFMA's first operand), so each lane owns consecutive columns of a row: 8 for the
//    fused SiLU·up (a wave's 8 column tiles are 4 gate/up pairs) and fp16 rows with a
//    power-of-two factor per row and 128-column block, whose weight rows are read in a paired
//    order (boff) so that each 16-byte store fills 64 bytes of a row (fp16 rows: neighbouring
//    lanes trade a chunk, and each store fills whole 128-byte lines); 4 for fp32 rows (optional
//    row scale) and the weighted fp32 atomic combine.  No LDS is involved, so the next tile's
//    loads fly meanwhile.
#include <type_traits>

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
constexpr int kBStage = kBN * kRow;        // 32 KiB weight stage (token-row stages: 32 or 8 KiB)

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

// Weight-row swizzle of the paired column layout (see boff): bits 1, 3 and 4 of the row, which
// tell apart the 16 rows that one fragment read takes (rows 8 q + s, q, s < 4, plus a multiple
// of 4 that only sets bit 2 or bits above 4), so that read is conflict-free as well.
__device__ __forceinline__ int swz_pair(int row) { return ((row >> 1) & 1) | (((row >> 3) & 3) << 1); }

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
template <int NW, int N = kBM / 8 / NW, int AUX = 0>
__device__ __forceinline__ void dma_operand(const char* base, const uint32_t* src, uint32_t off,
                                            char* stage, int wave) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_global_load_lds(base + (src[i] + off), stage + (wave + NW * i) * 1024, 16,
                                     0, AUX);
}

// Fragment u of this wave in a stage: A fragments 0..7 (16 rows each) at la + 1024 u, B
// fragments at lb + boff(j).  Every fragment row has the same swizzle, so one swizzled lane
// offset per operand serves all of them and the rest is an immediate offset.
//
// B column tiles: output columns of MFMA tile j, lane row c (c = 4 lk + r holds column 4 lk + r
// of the transposed accumulator).  Plain layout: columns 16 j + c.  Paired layout (PAIR): tiles
// 2m and 2m + 1 interleave in groups of 4, column 32 m + 8 (c / 4) + 4 (j & 1) + c % 4, so the
// lane with lk holds columns 32 m + 8 lk + [0, 8) across the pair: 16-byte stores of 8 bf16 or
// fp16 values, 64-byte row runs per store.  The lane's row offset is then 8 (lr / 4) + lr % 4
// and tile j adds 32 (j / 2) + 4 (j & 1).  For SwiGLU, tiles j and j + 4 are a gate/up pair
// (gate rows first, up rows from kBN / 2), with the same layout over j & 3.
template <bool SWIGLU, bool PAIR>
__device__ __forceinline__ int boff(int j) {
  const int jj = SWIGLU ? (j & 3) : j;
  const int col = PAIR ? 32 * (jj >> 1) + 4 * (jj & 1) : 16 * jj;
  return ((SWIGLU && j >= 4 ? kBN / 2 : 0) + col) * kRow;
}

template <int MI, bool SWIGLU, bool PAIR>
__device__ __forceinline__ void read_frags(const char* la, const char* lb, bf16x8* af,
                                           bf16x8* bfr) {
#pragma unroll
  for (int i = 0; i < MI; ++i) af[i] = *(const bf16x8*)(la + i * 16 * kRow);
#pragma unroll
  for (int j = 0; j < 8; ++j) bfr[j] = *(const bf16x8*)(lb + boff<SWIGLU, PAIR>(j));
}

// The 8·MI MFMAs of one 32-wide K step, reading the next step's fragments in between: one of
// the 8 next B fragments (into the other B set) after every MI MFMAs, A fragment i in place
// right after row i's 8 MFMAs.  The weight fragment goes in as the MFMA's first operand, so
// each 16 x 16 accumulator holds the transposed output tile: lane (lr, lk) gets token row lr,
// output columns 4 lk + [0, 4) (both operands have the same fragment layout, so the swap is
// free and lets the epilogue store 4 consecutive columns per lane).
// Instruction order inside one K step: after MFMA k, the LDS reads that bring the issued count
// to floor((k + 1) NR / NM), so the next step's fragments arrive spread over this step's MFMAs
// instead of in one burst near its end (measured on MI355X: the fused gate/up GEMM of the
// 397B-A17B-shaped and sigmoid layers 2.2% and 1.3% faster; the down GEMM, whose shorter
// reduction leaves less to overlap, 0.3-1.5% slower, so it keeps the compiler's order).
template <int NM, int NR, int K = 0>
__device__ __forceinline__ void interleave_reads() {
  if constexpr (K < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int before = K * NR / NM, after = (K + 1) * NR / NM;
    if constexpr (after > before)
      __builtin_amdgcn_sched_group_barrier(0x100, after - before, 0);  // LDS reads
    interleave_reads<NM, NR, K + 1>();
  }
}

template <int MI, bool SWIGLU, bool PAIR>
__device__ __forceinline__ void mma_stage(f32x4 (*acc)[8], bf16x8* af, const bf16x8* bfr,
                                          const char* la_n, const char* lb_n, bf16x8* bfr_n) {
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      if ((i * 8 + j + 1) % MI == 0) {
        const int b = (i * 8 + j + 1) / MI - 1;
        bfr_n[b] = *(const bf16x8*)(lb_n + boff<SWIGLU, PAIR>(b));
      }
    }
    af[i] = *(const bf16x8*)(la_n + i * 16 * kRow);
  }
  if constexpr (SWIGLU) interleave_reads<8 * MI, 8 + MI>();
}

constexpr int kNW = 8;                 // waves: 4 along M x 2 along N
constexpr int kNT = 64 * kNW;          // threads
constexpr int kDma = kBM / 8 / kNW;    // 1 KiB DMA instructions per wave per full operand stage
// Cache policy of the weight DMAs: non-temporal (gfx950 `nt`).  Each expert's weights are
// read by its M tiles at about the same time and then not again in the launch, so they should
// not push token rows, H and the expert rows the next kernels read out of L2 and the MALL
// (measured on MI355X: 35B-A3B decode 289 -> 271 us, prefill 435 -> 418 us, skewed 567 ->
// 532 us; the sigmoid and 397B-A17B layers' gate_up 1.7% and 2.7% faster).
constexpr int kWeightAux = 2;

// First row of wave row block wm when blocks 0 and 1 hold mi_hi and blocks 2 and 3 mi_lo
// 16-row MFMA tiles.
__device__ __forceinline__ int block_row0(int wm, int mi_hi, int mi_lo) {
  return wm < 2 ? wm * 16 * mi_hi : 32 * mi_hi + (wm - 2) * 16 * mi_lo;
}

// 32-row pairs of MFMA row tiles that hold `rows` rows, split over the wave row blocks: blocks
// 0 and 1 take mi_hi 16-row tiles each, blocks 2 and 3 mi_lo.
__device__ __forceinline__ void tile_mi(int rows, int* mi_hi, int* mi_lo) {
  const int pairs = min(max((rows + 31) >> 5, 1), 8);
  *mi_hi = (pairs + 1) >> 1;
  *mi_lo = pairs >> 1;
}

// A tile of a work-group's schedule: its group (expert), rows [row_start, + rows) and N tile.
struct TileMap {
  int group, row_start, rows, n_tile;
  uint32_t k0;  // first byte of each row this tile reduces over (split-K slice * slice bytes)
  int slice;
};

// Logical tile t: expert-major, then N tile, then M tile (the M tiles of one expert are
// entries [first, first + cnt) of the tile map and own logical tiles [first·ntN, (first+cnt)·ntN));
// dense mode (no tile map) has one group of mt_total M tiles.  Decoding takes two dependent
// rounds of scalar loads: the expert's entry (map_expert), then the M tile's (map_mtile).
// (Cutting dense mode into groups of a few M tiles, so that an XCD streams only its own token
// rows, made the dense shared expert about 1% faster but cost the grouped kernels scalar
// registers, and the sigmoid layer's routed gate_up 2.8%.)
__device__ __forceinline__ void map_expert(const GemmParams& p, int t, int ntN, int mt_total,
                                           int* first, int* cnt) {
  if (p.tiles) {
    const int q = t / ntN;
    *first = load_uniform(p.tiles, q * kTileStride + 4);
    *cnt = load_uniform(p.tiles, q * kTileStride + 5);
  } else {
    *first = 0;
    *cnt = mt_total;
  }
}

__device__ __forceinline__ void map_mtile(const GemmParams& p, int t, int ntN, int first, int cnt,
                                          TileMap& tile) {
  const int l = t - first * ntN;
  tile.n_tile = l / cnt;
  const int m = first + l % cnt;
  if (p.tiles) {
    tile.group = load_uniform(p.tiles, m * kTileStride + 0);
    tile.row_start = load_uniform(p.tiles, m * kTileStride + 1);
    tile.rows = load_uniform(p.tiles, m * kTileStride + 2);
  } else {
    tile.group = 0;
    tile.row_start = m * kBM;
    tile.rows = min(kBM, p.M - m * kBM);
  }
}

// Staged row r = 8 (wave + 8 i) + (lane >> 3) of DMA instruction i keeps logical chunk
// (lane & 7) ^ swz(r) in the lane's slot; swz depends on r mod 16 only, so one value serves
// every instruction of the wave.
__device__ __forceinline__ int lane_chunk(int lane, int wave) {
  return (lane & 7) ^ swz(8 * wave + (lane >> 3));
}

template <bool SWIGLU, bool PAIR>
__device__ __forceinline__ void weight_sources(const GemmParams& p, int lane, int wave,
                                               int n_tile, uint32_t* sb) {
  // staged row r = 8 (wave + 8 i) + (lane >> 3): bits 1, 3 and 4 do not depend on i either
  const int r0 = 8 * wave + (lane >> 3);
  const int chunk = (lane & 7) ^ (PAIR ? swz_pair(r0) : swz(r0));
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int r = 8 * (wave + kNW * i) + (lane >> 3);
    int brow;
    if (SWIGLU) {
      // the tile's first 128 staged rows are gate rows, the next 128 the matching up rows
      const int n = n_tile * (kBN / 2) + (r & (kBN / 2 - 1));
      brow = n < p.N ? (r < kBN / 2 ? n : p.N + n) : 0;
    } else {
      const int n = n_tile * kBN + r;
      brow = n < p.N ? n : 0;
    }
    sb[i] = (uint32_t)brow * (uint32_t)p.ldb_bytes + chunk * 16;
  }
}

// Token row of instruction i without a gather: position row_start + min(r, rows - 1).
__device__ __forceinline__ uint32_t row_source(const GemmParams& p, int lane, int wave,
                                               int row_start, int rows, int i) {
  const int r = 8 * (wave + kNW * i) + (lane >> 3);
  return (uint32_t)(row_start + min(r, rows - 1)) * (uint32_t)p.lda_bytes +
         lane_chunk(lane, wave) * 16;
}

// Gathered token rows in two steps, so that all loads of a tile go out together.  gather_issue
// reads the permutation entries of instruction i's 8 positions row_start + min(r0 + k,
// rows - 1) with scalar loads (uniform addresses: no vector load is left for the compiler to
// wait on, and a wait on the vector-memory counter would also wait for every DMA and store in
// flight); gather_source picks the lane's.
__device__ __forceinline__ void gather_issue(const GemmParams& p, int wave, int row_start,
                                             int rows, int i, int* v) {
  const int r0 = 8 * (wave + kNW * i);
  if (r0 + 8 <= rows) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load_uniform(p.a_gather, row_start + r0 + k);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load_uniform(p.a_gather, row_start + min(r0 + k, rows - 1));
  }
}

__device__ __forceinline__ uint32_t gather_source(const GemmParams& p, int lane, int wave,
                                                  const int* v) {
  // a tree of selects on the bits of q over values the compiler cannot trace back to the
  // loads (selects between loaded values become an indexed private array, i.e. scratch)
  int w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    w[k] = v[k];
    asm volatile("" : "+s"(w[k]));
  }
  const int q = lane >> 3;
  const bool b0 = q & 1, b1 = q & 2, b2 = q & 4;
  const int a01 = b0 ? w[1] : w[0], a23 = b0 ? w[3] : w[2];
  const int a45 = b0 ? w[5] : w[4], a67 = b0 ? w[7] : w[6];
  const int a03 = b1 ? a23 : a01, a47 = b1 ? a67 : a45;
  const int a = b2 ? a47 : a03;
  return (uint32_t)(a / p.a_div) * (uint32_t)p.lda_bytes + lane_chunk(lane, wave) * 16;
}

// Split-K (KS variant: dense fp32 rows, the router): the reduction is cut into p.k_slices
// equal slices and logical tile t covers slice t / (mt_total ntN) of output tile
// t % (mt_total ntN), so an XCD's share of the sequence mostly stays within one slice and its
// tiles share that slice of the weights.  Other variants have one slice at compile time.
template <bool KS>
__device__ __forceinline__ int k_slices(const GemmParams& p) {
  if constexpr (KS) return p.k_slices > 1 ? p.k_slices : 1;
  return 1;
}

template <bool KS>
__device__ __forceinline__ void load_map(const GemmParams& p, int t, int ntN, int mt_total,
                                         TileMap& tile) {
  int slice = 0;
  if constexpr (KS) {
    slice = t / (mt_total * ntN);
    t -= slice * mt_total * ntN;
  }
  int first, cnt;
  map_expert(p, t, ntN, mt_total, &first, &cnt);
  map_mtile(p, t, ntN, first, cnt, tile);
  tile.slice = slice;
  tile.k0 = KS ? (uint32_t)slice * (uint32_t)(p.Kdim / k_slices<KS>(p)) * 2u : 0u;  // bf16 bytes
}

// Every DMA source of a tile: weight rows, and token rows of the first NA instructions (the
// gathered ones in one round of loads).
template <bool SWIGLU, bool PAIR, int NA>
__device__ __forceinline__ void tile_sources(const GemmParams& p, int lane, int wave,
                                             const TileMap& tile, uint32_t* sa, uint32_t* sb) {
  weight_sources<SWIGLU, PAIR>(p, lane, wave, tile.n_tile, sb);
  if (p.a_gather) {
    int v[NA][8];
#pragma unroll
    for (int i = 0; i < NA; ++i) gather_issue(p, wave, tile.row_start, tile.rows, i, v[i]);
#pragma unroll
    for (int i = 0; i < NA; ++i) sa[i] = gather_source(p, lane, wave, v[i]);
  } else {
    // dense rows; a split-K tile starts its rows at byte k0 (0 without a split)
#pragma unroll
    for (int i = 0; i < NA; ++i)
      sa[i] = row_source(p, lane, wave, tile.row_start, tile.rows, i) + tile.k0;
#pragma unroll
    for (int i = 0; i < kDma; ++i) sb[i] += tile.k0;
  }
}

// Token-row DMA of one stage with a run-time count n <= MAXN of instructions per wave.
template <int MAXN>
__device__ __forceinline__ void dma_rows_n(int n, const char* base, const uint32_t* src,
                                           uint32_t off, char* stage, int wave) {
#pragma unroll
  for (int i = 0; i < MAXN; ++i)
    if (i < n)
      __builtin_amdgcn_global_load_lds(base + (src[i] + off), stage + (wave + kNW * i) * 1024, 16,
                                       0, 0);
}

// Epilogue straight from the accumulators.  The weight fragment is the MFMA's first operand,
// so lane (lr, lk) of MFMA tile (i, j) holds row wrow0 + 16 i + lr of the output tile and 4
// consecutive columns of its wave's column block (boff): in the plain layout columns
// 16 j + 4 lk + [0, 4) (fp32 rows and the atomic combine: 16-byte stores, 64-byte row runs),
// in the paired layout columns 32 m + 8 lk + [0, 8) over tiles j = 2m, 2m + 1 (bf16 H and
// fp16 rows: 16-byte stores, 64-byte row runs, half the store instructions).  L2 merges the
// runs into whole lines.  No LDS, no barrier.
template <int MI, int EPI, bool RS, bool PAIR, bool KS>
__device__ __forceinline__ void store_tile(const GemmParams& p, const f32x4 (*acc)[8], int lane,
                                           int wn, int wrow0, int row_start, int rows,
                                           int n_tile, int slice) {
  typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const int lr = lane & 15, lk = lane >> 4;
  if constexpr (EPI == EPI_SWIGLU) {
    static_assert(PAIR, "SwiGLU rows use the paired layout");
    // H: the tile's 128 columns; wave wn holds [64 wn, +64) as gate tiles j and up tiles j + 4,
    // 8 consecutive columns per lane
    const int ncols = min(kBN / 2, p.N - n_tile * (kBN / 2));
    __bf16* Ht = (__bf16*)p.C + (int64_t)row_start * p.ldc + n_tile * (kBN / 2);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = wrow0 + 16 * i + lr;
      if (row < rows) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int col = wn * 64 + 32 * m + 8 * lk;
          if (col < ncols) {
            bf16x8v h;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              h[r] = (__bf16)(silu_fast(acc[i][2 * m][r]) * acc[i][2 * m + 4][r]);
              h[4 + r] = (__bf16)(silu_fast(acc[i][2 * m + 1][r]) * acc[i][2 * m + 5][r]);
            }
            *(bf16x8v*)(Ht + (int64_t)row * p.ldc + col) = h;
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_STORE && PAIR) {
    // fp16 with a power-of-two factor per row of the wave's 128 columns, from the row's largest
    // |value| (the lane's 32 values, then the 4 lanes that share the row)
    static_assert(kScaleCols == kBN / 2 && !RS, "one fp16 factor block per wave column half");
    const int ncols = min(kBN, p.N - n_tile * kBN);
    const int c0 = wn * 128;  // this wave's columns [c0, c0 + 128) of the tile
    _Float16* Ch = (_Float16*)p.C + (int64_t)row_start * p.ldc + n_tile * kBN;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      float mx = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + 32 * (j >> 1) < ncols)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[i][j][r]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float sc, inv;
      f16_block_scale(mx, &sc, &inv);
      // Per 64-column span the lane holds two 8-column chunks of its row (pairs 2p and 2p + 1:
      // columns 8 lk and 32 + 8 lk of the span).  Lanes lr and lr ^ 1 (rows R, R + 1) trade one
      // chunk (DPP swap), so that one store writes row R's whole 128 bytes from the 8 lanes of
      // the two rows and the next store row R + 1's: every store fills whole lines.
      const int row = wrow0 + 16 * i + lr;
      const bool odd = lr & 1;
      const int row_a = row - (odd ? 1 : 0), row_b = row_a + 1;
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const int cs = c0 + 64 * sp;
        if (cs < ncols) {  // uniform
          f16x8 ca, cb;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ca[r] = (_Float16)(acc[i][4 * sp][r] * sc);
            ca[4 + r] = (_Float16)(acc[i][4 * sp + 1][r] * sc);
            cb[r] = (_Float16)(acc[i][4 * sp + 2][r] * sc);
            cb[4 + r] = (_Float16)(acc[i][4 * sp + 3][r] * sc);
          }
          // row R's lane sends its second chunk, row R + 1's lane its first
          typedef int i32x4 __attribute__((ext_vector_type(4)));
          const i32x4 snd = odd ? __builtin_bit_cast(i32x4, ca) : __builtin_bit_cast(i32x4, cb);
          i32x4 rcv;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            rcv[q] = __builtin_amdgcn_update_dpp(snd[q], snd[q], 0xB1, 0xf, 0xf, false);
          const f16x8 got = __builtin_bit_cast(f16x8, rcv);
          const f16x8 first = odd ? got : ca;   // row R, columns (odd ? 32 : 0) + 8 lk
          const f16x8 second = odd ? cb : got;  // row R + 1, the same columns
          const int col = cs + (odd ? 32 : 0) + 8 * lk;
          if (row_a < rows) *(f16x8*)(Ch + (int64_t)row_a * p.ldc + col) = first;
          if (row_b < rows) *(f16x8*)(Ch + (int64_t)row_b * p.ldc + col) = second;
        }
      }
      if (lane < 16 && row < rows && c0 < ncols)
        p.c_scale[(int64_t)(row_start + row) * p.ldcs + n_tile * (kBN / kScaleCols) + wn] = inv;
    }
  } else if constexpr (EPI == EPI_STORE) {
    // fp32, times row_scale[row] in the RS variant (its vector load is waited for at once,
    // which also waits for the next tile's first stages; the variant serves only the
    // row-scaled shared expert).  A split-K tile writes its partial sums to its slice's plane,
    // and slice 0 adds col_bias.
    static_assert(!PAIR, "fp32 rows use the plain layout");
    const int c4 = 4 * lk;
    const int ncols = min(kBN, p.N - n_tile * kBN);
    const int c0 = wn * 128;
    float* Ct = (float*)p.C + slice * p.c_slice_stride + (int64_t)row_start * p.ldc +
                n_tile * kBN;
    const float* bias = KS && slice == 0 && p.col_bias ? p.col_bias + n_tile * kBN : nullptr;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = wrow0 + 16 * i + lr;
      if (row < rows) {
        float s = 1.0f;
        if constexpr (RS) s = p.row_scale[row_start + row];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = c0 + 16 * j + c4;
          if (col < ncols) {
            f32x4 v = acc[i][j];
            if (bias) v += *(const f32x4*)(bias + col);
            if constexpr (RS) v *= s;
            *(f32x4*)(Ct + (int64_t)row * p.ldc + col) = v;
          }
        }
      }
    }
  } else {  // EPI_ATOMIC_COMBINE: the token's output row += routing weight * row
    static_assert(!PAIR, "the atomic combine uses the plain layout");
    const int c4 = 4 * lk;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = wrow0 + 16 * i + lr;
      if (row < rows) {
        const int a = p.perm[row_start + row];
        const float w = p.topk_w[a];
        const int n0 = n_tile * kBN + wn * 128;
        float* dst = p.acc_out + (int64_t)(a / p.topk) * p.ldo + n0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = 16 * j + c4 + r;
            if (n0 + n < p.N) unsafeAtomicAdd(dst + n, w * acc[i][j][r]);
          }
      }
    }
  }
}

// One output tile.  Wave (wm, wn) owns MI x 8 MFMA tiles of 16 x 16: columns [128 wn, +128)
// and MI 16-row tiles starting at block_row0(wm).  A tile of `rows` rows is computed as
// P = ceil(rows / 32) pairs of 16-row tiles (tile_mi): row blocks 0 and 1 take mi_hi =
// ceil(P / 2) each, blocks 2 and 3 mi_lo = floor(P / 2).  The two waves that share a SIMD
// (waves w and w + 4) hold one block of each kind, so every SIMD runs P sets of 8 MFMAs per K
// step and a partly filled tile (a group's last one) costs in proportion to its rows, to 32
// rows.  Only the token rows [0, 32 P) are fetched; MI is also this wave's count of 1 KiB
// token-row DMA instructions per stage.
//
// Rings: token rows in 2 stages of AROWS x 128 bytes, weights in 3 stages of 32 KiB.  Global
// stage G (the work-group's running count, this tile's stage 0 is G0) lives in slots G % 2 and
// G % 3.  When the reduction has at least 3 stages the rings run on across the work-group's
// tiles: the refills during a tile's last three stages fetch the next tile's stages 0-2 (nx_*
// describe it, nx_group < 0 if there is none, and nx_mi is this wave's MI there), and that
// tile then starts with them in flight or landed (`pre`), so the weight stream does not stop
// for an epilogue or a prologue.
template <int MI, int EPI, int AROWS, bool RS, bool PAIR, bool KS>
__device__ __forceinline__ void ring_tile(const GemmParams& p, char* smem, int tid, int wave,
                                          const TileMap& cur, int ns, int mi_hi, int mi_lo,
                                          int G0, bool pre, int tn, int ntN, int mt_total,
                                          TileMap& nx) {
  constexpr bool kSwiglu = EPI == EPI_SWIGLU;
  constexpr int kAS = AROWS * kRow;  // token-row stage bytes
  constexpr int kMaxMI = AROWS / 64;
  constexpr int MIA = MI > 0 ? MI : 1;  // array extent
  static_assert(MI >= 0 && MI <= kMaxMI && kSA == 2 && kSB == 3, "tile shape, ring depths");
  static_assert(kDma == 4 && 2 * kDma + kMaxMI < 64, "vmcnt range");
  char* const sA = smem;             // token-row ring
  char* const sB = smem + kSA * kAS;  // weight ring
  const auto a_at = [&](int G) { return sA + (G & 1) * kAS; };
  const auto b_at = [&](int G) { return sB + (G % 3) * kBStage; };
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lk = lane >> 4;

  // Lane offsets (within a stage) of this wave's first A and B fragment rows, for each 32-wide
  // half of the stage.  For SwiGLU the tile's first 128 B rows are gate rows and the next 128
  // the matching up rows, and a wave's column tiles j and j + 4 are a gate/up pair.
  const int wrow0 = block_row0(wm, mi_hi, mi_lo);
  const int la_row = (wrow0 + lr) * kRow;
  const int ch0 = (lk ^ swz(lr)) << 4, ch1 = ((4 + lk) ^ swz(lr)) << 4;
  // B: the lane's fragment row within its column tiles (boff) and that row's swizzle
  const int lrow = PAIR ? 8 * (lr >> 2) + (lr & 3) : lr;
  const int lb_row = ((kSwiglu ? wn * 64 : wn * 128) + lrow) * kRow;
  const int bsw = PAIR ? swz_pair(lrow) : swz(lrow);
  const int cb0 = (lk ^ bsw) << 4, cb1 = ((4 + lk) ^ bsw) << 4;

  const int rows = cur.rows;
  uint32_t srcA[kMaxMI], srcB[kDma], nsA[kMaxMI], nsB[kDma];
  tile_sources<kSwiglu, PAIR, kMaxMI>(p, lane, wave, cur, srcA, srcB);
  const char* gbase = p.B + (int64_t)cur.group * p.b_group_bytes;

  // The next tile (logical tile tn >= 0), whose first stages this tile's last refills fetch:
  // its map entry (returned in nx for the caller) and DMA sources.
  const bool nxt = tn >= 0;
  int nx_mi = 0;  // this wave's token-row DMA instructions per stage of the next tile
  if (nxt) {
    load_map<KS>(p, tn, ntN, mt_total, nx);
    tile_sources<kSwiglu, PAIR, kMaxMI>(p, lane, wave, nx, nsA, nsB);
    int nh, nl;
    tile_mi(nx.rows, &nh, &nl);
    nx_mi = wave < 4 ? nh : nl;
  }

  f32x4 acc[MIA][8];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (!pre) {
    // Prologue A0 B0 A1 B1 B2, once every wave is done reading the previous tile's ring.
    // Token rows run two stages ahead, weights three, so up to 64 KiB of weights per CU are
    // in flight; a stage of token rows is MI instructions per wave, one of weights kDma.
    lds_barrier();
    dma_operand<kNW, MI>(p.A, srcA, 0, a_at(G0), wave);
    dma_operand<kNW, kDma, kWeightAux>(gbase, srcB, 0, b_at(G0), wave);
    if (ns > 1) {
      dma_operand<kNW, MI>(p.A, srcA, kRow, a_at(G0 + 1), wave);
      dma_operand<kNW, kDma, kWeightAux>(gbase, srcB, kRow, b_at(G0 + 1), wave);
    }
    if (ns > 2) dma_operand<kNW, kDma, kWeightAux>(gbase, srcB, 2 * kRow, b_at(G0 + 2), wave);
    if (ns > 2)  // A1 B1 B2 were issued after B0 and may still fly
      barrier_after<MI + 2 * kDma, 0>();
    else
      barrier_after<0, 0>();
  } else {
    // Stages 0-2 went out with the previous tile's last refills, as B0 A0 B1 A1 B2, followed by
    // its stores.  Loads complete in order, so A0 and B0 have landed once at most the
    // 2 kDma + MI loads issued after A0 are outstanding (the stores are counted too, which
    // can only lengthen the wait).
    barrier_after<2 * kDma + MI, 0>();
  }

  // stage 0's first half's fragments (A fragments are refilled in place, B fragments alternate
  // between two sets)
  bf16x8 af0[MIA], bf0[8], bf1[8];
  if constexpr (MI > 0)
    read_frags<MI, kSwiglu, PAIR>(a_at(G0) + la_row + ch0, b_at(G0) + lb_row + cb0, af0, bf0);

  // Stage g's MFMAs: first half (step 2g) while reading the second half's fragments from the
  // same stage; then publish stage g+1 (this wave's copies landed; every wave has read all of
  // stage g, so its slots are free), refill them with token rows of stage g+2 and weights of
  // g+3 (this tile's or, in the last three stages, the next tile's), and run the second half
  // (step 2g+1) while reading stage g+1's first half.  ra and rb are the ring slots of stage
  // g (global stage G0 + g modulo 2 and 3).
  int ra = G0 & 1, rb = G0 % 3;
  int g = 0;
  for (; g + 3 < ns; ++g) {  // refills of this tile only
    const int ra1 = ra ^ 1, rb1 = rb == 2 ? 0 : rb + 1;
    if constexpr (MI > 0)
      mma_stage<MI, kSwiglu, PAIR>(acc, af0, bf0, sA + ra * kAS + la_row + ch1,
                             sB + rb * kBStage + lb_row + cb1, bf1);
    barrier_after<kDma, 0>();  // B(g+2) went out after A(g+1) and may still fly
    dma_operand<kNW, MI>(p.A, srcA, (uint32_t)(g + 2) * kRow, sA + ra * kAS, wave);
    dma_operand<kNW, kDma, kWeightAux>(gbase, srcB, (uint32_t)(g + 3) * kRow, sB + rb * kBStage, wave);
    if constexpr (MI > 0)
      mma_stage<MI, kSwiglu, PAIR>(acc, af0, bf1, sA + ra1 * kAS + la_row + ch0,
                             sB + rb1 * kBStage + lb_row + cb0, bf0);
    ra = ra1;
    rb = rb1;
  }
  for (; g < ns; ++g) {  // the last three stages
    const int ra1 = ra ^ 1, rb1 = rb == 2 ? 0 : rb + 1;
    if constexpr (MI > 0)
      mma_stage<MI, kSwiglu, PAIR>(acc, af0, bf0, sA + ra * kAS + la_row + ch1,
                             sB + rb * kBStage + lb_row + cb1, bf1);
    if (g + 1 < ns) {
      if (g + 2 < ns || nxt)  // B(g+2) went out after A(g+1) and may still fly
        barrier_after<kDma, 0>();
      else
        barrier_after<0, 0>();
    } else {
      lds_barrier();  // the last stage: nothing to wait for, the slots are free
    }
    if (g + 2 < ns)
      dma_operand<kNW, MI>(p.A, srcA, (uint32_t)(g + 2) * kRow, sA + ra * kAS, wave);
    else if (nxt)
      dma_rows_n<kMaxMI>(nx_mi, p.A, nsA, (uint32_t)(g + 2 - ns) * kRow, sA + ra * kAS, wave);
    if (nxt)  // g + 3 >= ns here: the next tile's weights
      dma_operand<kNW, kDma, kWeightAux>(p.B + (int64_t)nx.group * p.b_group_bytes, nsB,
                       (uint32_t)(g + 3 - ns) * kRow, sB + rb * kBStage, wave);
    if constexpr (MI > 0) {
      // after the last stage these reads fetch unused leftovers
      const int na = g + 1 < ns ? ra1 : ra, nb = g + 1 < ns ? rb1 : rb;
      mma_stage<MI, kSwiglu, PAIR>(acc, af0, bf1, sA + na * kAS + la_row + ch0,
                             sB + nb * kBStage + lb_row + cb0, bf0);
    }
    ra = ra1;
    rb = rb1;
  }

  // ---- epilogue from registers, while the next tile's first stages land ----------------------
  // The lane index is laundered through an empty asm so the store offsets are computed here,
  // not hoisted out of the tile loop into registers (and spilled).
  int elane = lane;
  asm volatile("" : "+v"(elane));
  if constexpr (MI > 0)
    store_tile<MI, EPI, RS, PAIR, KS>(p, acc, elane, wn, wrow0, cur.row_start, rows, cur.n_tile,
                                  cur.slice);
}

// Persistent, XCD-aware work-groups over the logical tiles: XCD x (work-groups b with
// b % 8 == x) takes the x-th eighth of the tiles, its work-groups striding through it.
// AROWS = 256 rows per token-row stage (any tile), or 64 when no tile has more than 64 rows
// (decode batches: 8 KiB stages); RS: the STORE epilogue multiplies by row_scale; PAIR: the
// paired column layout (SwiGLU and fp16 rows, see boff).
template <int EPI, int AROWS, bool RS, bool PAIR, bool KS>
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[kSA * AROWS * kRow + kSB * kBStage];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int BNE = EPI == EPI_SWIGLU ? kBN / 2 : kBN;  // output columns per tile
  const int ntN = (p.N + BNE - 1) / BNE;
  const int mt_total = p.tiles ? load_uniform(p.tile_count, 0) : (p.M + kBM - 1) / kBM;
  const int nt = mt_total * ntN * k_slices<KS>(p);
  const int xcd = blockIdx.x % kXcds, per = gridDim.x / kXcds, jb = blockIdx.x / kXcds;
  const int lo = (int)((int64_t)nt * xcd / kXcds), hi = (int)((int64_t)nt * (xcd + 1) / kXcds);
  const int ns = p.Kdim / 64 / k_slices<KS>(p);  // DMA stages per tile (host-checked divisor)

  // The next tile's stages 0-2 come with this tile's last three refills, which needs three
  // stages per tile; shorter reductions run each tile with its own prologue.  A tile's map
  // entry comes from the previous tile, which needed it for those refills (first tile: here).
  const bool cross = ns >= 3;
  int t = lo + jb;
  TileMap cur, nx;
  if (t < hi) load_map<KS>(p, t, ntN, mt_total, cur);
  int G0 = 0;
  for (; t < hi; t += per) {
    const int tn = cross && t + per < hi ? t + per : -1;
    int mi_hi, mi_lo;
    tile_mi(cur.rows, &mi_hi, &mi_lo);
    const bool pre = cross && G0 > 0;
    const auto run = [&](auto mi) {
      ring_tile<decltype(mi)::value, EPI, AROWS, RS, PAIR, KS>(p, smem, tid, wave, cur, ns, mi_hi, mi_lo,
                                                     G0, pre, tn, ntN, mt_total, nx);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    const int mi = wave < 4 ? mi_hi : mi_lo;  // waves 0-3 hold row blocks 0 and 1
    if constexpr (AROWS == 64) {
      if (mi == 0) run(I0{}); else run(I1{});
    } else {
      switch (mi) {
        case 0: run(I0{}); break;
        case 1: run(I1{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        default: run(std::integral_constant<int, 4>{}); break;
      }
    }
    G0 += ns;
    if (tn >= 0)
      cur = nx;
    else if (t + per < hi)
      load_map<KS>(p, t + per, ntN, mt_total, cur);
  }
}

constexpr int kSmallRows = 64;  // token-row stage rows of the decode-batch variant

template <int EPI>
hipError_t launch_epi(const GemmParams& p, int64_t max_mtiles, hipStream_t stream) {
  constexpr int BNE = EPI == EPI_SWIGLU ? kBN / 2 : kBN;
  const int64_t ntN = (p.N + BNE - 1) / BNE;
  const int64_t ks = (!p.tiles && p.k_slices > 1) ? p.k_slices : 1;
  const int64_t want = max_mtiles * ntN * ks;
  int64_t grid = want < kCus ? want : kCus;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  const bool small = p.tiles ? (p.rows_bound > 0 && p.rows_bound <= kSmallRows)
                             : p.M <= kSmallRows;
  const dim3 g((unsigned)grid), b(kNT);
  // layout and epilogue variants: SwiGLU and fp16 rows paired, fp32 rows (optionally
  // row-scaled, or split-K with a column bias) and the atomic combine plain
  const auto go = [&](auto rs, auto pair, auto ksplit) {
    constexpr bool RS = decltype(rs)::value, PAIR = decltype(pair)::value;
    constexpr bool KS = decltype(ksplit)::value;
    if (small)
      hipLaunchKernelGGL((mfma_kernel<EPI, kSmallRows, RS, PAIR, KS>), g, b, 0, stream, p);
    else
      hipLaunchKernelGGL((mfma_kernel<EPI, kBM, RS, PAIR, KS>), g, b, 0, stream, p);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if constexpr (EPI == EPI_SWIGLU) {
    go(F_{}, T_{}, F_{});
  } else if constexpr (EPI == EPI_STORE) {
    if (p.c_scale && p.row_scale) return hipErrorInvalidValue;  // no row-scaled fp16 rows
    if (p.c_scale)
      go(F_{}, T_{}, F_{});
    else if (p.row_scale)
      go(T_{}, F_{}, F_{});
    else if (p.k_slices > 1 || p.col_bias)
      go(F_{}, F_{}, T_{});
    else
      go(F_{}, F_{}, F_{});
  } else {
    go(F_{}, F_{}, F_{});
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_gemm(Epilogue epi, const GemmParams& p, int64_t max_mtiles,
                            hipStream_t stream) {
  if (max_mtiles <= 0) return hipSuccess;
  if (p.B2) return hipErrorInvalidValue;  // the extra weight row is the tile GEMM's
  // split-K and the column bias: dense fp32 rows only, whole 64-wide stages per slice, and
  // 4-column groups that stay inside a row (f32x4 stores and bias loads)
  const bool plain_f32 = epi == EPI_STORE && !p.c_scale && !p.row_scale && !p.tiles;
  if ((p.col_bias || p.k_slices > 1) && !(plain_f32 && p.N % 4 == 0 && p.ldc % 4 == 0))
    return hipErrorInvalidValue;
  if (p.k_slices > 1 && (p.Kdim % (64 * p.k_slices) != 0 || p.c_slice_stride % 4 != 0))
    return hipErrorInvalidValue;
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
