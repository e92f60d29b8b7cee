// Dispatch: per-expert histogram, prefix sum and a stable counting sort of the T*K assignments
// into expert-contiguous order ("MoE" §3.2: the tokens routed to each hit expert are gathered so
// that the expert runs once on all of them; "1.6 混合专家（MoE）" §二: route, group, compute,
// merge).
//
// The assignments a = t*K + k are cut into segments of 128, 256 or 512 consecutive ids (by
// batch size), one wave64 each (each lane prefetches its ids of the segment at once).
//   count        : each wave histograms its segment in LDS (atomics are fine: counts do not
//                  depend on order) and writes seg_counts[segment][E].
//   scan_scatter : every work-group re-derives the expert totals, offsets and its segments'
//                  first ranks from seg_counts (work-group 0 also writes counts and offsets,
//                  an extra last work-group the tile maps); then each wave re-reads its
//                  segment 64 ids at a time and
//                  places every assignment by its ballot-computed rank.  Segments, rounds and
//                  lanes all follow ascending a, so the sort is stable and the result
//                  bit-exact.
// Small batches take one work-group for the whole dispatch (dispatch_fused_kernel).
// Expert capacity ("1.6 混合专家（MoE）" §三): with a cap C, scan counts min(t_e, C) rows per
// expert (so offsets and tile maps cover only kept rows) and scatter drops every assignment
// whose rank q is C or more (inv_perm = -1): each expert keeps its first C assignments.
#include <type_traits>

#include "kernels.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;
// A segment is R rounds of 64 ids (one wave): R = 2, 4 or 8, the shortest that keeps the
// number of segments at or below kSegTarget.  Short segments spread the scatter over more
// work-groups; long ones keep the histograms that every scatter work-group sums few.  Measured
// on MI355X: 32768 assignments 19.3 -> 16.3 us with 128-id segments, while 98304 assignments
// went 20.5 -> 25.1 us with them (and 22.2 with 256-id ones), hence the bound.
constexpr int kSegTarget = 256;
constexpr int kMaxSegRounds = 8;
int seg_rounds(int64_t A) {
  for (int r = 2; r < kMaxSegRounds; r *= 2)
    if ((A + 64 * r - 1) / (64 * r) <= kSegTarget) return r;
  return kMaxSegRounds;
}
// Single-work-group dispatch up to this many assignments (its LDS holds 17 ints per expert).
constexpr int64_t kFusedMaxA = 8192;
constexpr int kFusedMaxE = kDispatchOneWgMaxE;

// One DPP step of a wave-wide inclusive sum: v plus the value CTRL brings from another lane;
// lanes with no source under CTRL, or in rows outside ROW_MASK, add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int add_dpp(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// Exclusive prefix sum over the wave's 64 lanes (lane order): shifts by 1, 2, 4 and 8 lanes
// within each row of 16, then the last lane of row 0 carried into rows 1 and 3 and that of
// row 1 into rows 2 and 3 (integer adds, so the grouping does not change the result).
__device__ __forceinline__ int wave_prefix_exclusive(int v) {
  int x = add_dpp<0x111, 0xf>(v);  // row_shr:1
  x = add_dpp<0x112, 0xf>(x);      // row_shr:2
  x = add_dpp<0x114, 0xf>(x);      // row_shr:4
  x = add_dpp<0x118, 0xf>(x);      // row_shr:8
  x = add_dpp<0x142, 0xa>(x);      // row_bcast:15 into rows 1 and 3
  x = add_dpp<0x143, 0xc>(x);      // row_bcast:31 into rows 2 and 3
  return x - v;
}

// Exclusive scan of one int per thread across an NT-thread block.  Returns the prefix and
// writes the block total to *total.  Every thread adds up the wave totals itself (the same
// LDS words for the whole wave), so no thread scans them for the others.
template <int NT>
__device__ int block_exclusive_scan(int v, int* scratch /* >= NT / 64 ints */, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ex = wave_prefix_exclusive(v);
  if (lane == 63) scratch[wave] = ex + v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int c = scratch[w];
    all += c;
    before += w < wave ? c : 0;
  }
  *total = all;
  __syncthreads();  // scratch is free for the next scan
  return ex + before;
}

// Two exclusive scans of one int each per thread across an NT-thread block, with one pair of
// barriers: *pv, *pu the prefixes of v and u, *tv, *tu their block totals.
template <int NT>
__device__ void block_exclusive_scan2(int v, int u, int* scratch /* >= 2 NT / 64 ints */, int* pv,
                                      int* pu, int* tv, int* tu) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ev = wave_prefix_exclusive(v), eu = wave_prefix_exclusive(u);
  if (lane == 63) {
    scratch[wave] = ev + v;
    scratch[W + wave] = eu + u;
  }
  __syncthreads();
  int bv = 0, bu = 0, av = 0, au = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int cv = scratch[w], cu = scratch[W + w];
    av += cv;
    au += cu;
    bv += w < wave ? cv : 0;
    bu += w < wave ? cu : 0;
  }
  *pv = ev + bv;
  *pu = eu + bu;
  *tv = av;
  *tu = au;
  __syncthreads();  // scratch is free again
}

// Work-group b counts segments 4 b .. 4 b + 3 (one per wave) and also writes their sum, the
// histogram of chunk b (kChunkSegs segments), so that the scatter work-groups can form the
// counts of all earlier segments from a quarter as many rows.
constexpr int kChunkSegs = 4;

template <int R>
__global__ void __launch_bounds__(256) count_kernel(const int32_t* __restrict__ idx, int64_t A,
                                                    int E, int64_t nseg,
                                                    int32_t* __restrict__ seg_counts,
                                                    int32_t* __restrict__ chunk_counts) {
  extern __shared__ int hist_all[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seg = (int64_t)blockIdx.x * kChunkSegs + wave;
  int* hist = hist_all + wave * E;
  for (int e = lane; e < E; e += 64) hist[e] = 0;
  if (seg < nseg) {  // whole wave
    const int64_t a0 = seg * (64 * R);
    int ev[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t a = a0 + r * 64 + lane;
      ev[r] = a < A ? idx[a] : -1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (ev[r] >= 0 && ev[r] < E) atomicAdd(&hist[ev[r]], 1);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
    for (int e = lane; e < E; e += 64) seg_counts[seg * E + e] = hist[e];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kChunkSegs; ++w) c += hist_all[w * E + e];
    chunk_counts[(int64_t)blockIdx.x * E + e] = c;
  }
}

// Builds the tile map from per-expert counts held in LDS.  One entry per M tile:
// {expert, first row position, rows, 0, first M tile of the expert, M tiles of the expert, 0,
// 0}.  An expert's rows are split evenly over its ceil(c / bm) M tiles (the first c % mt tiles
// one row more): its tiles then cost the same, run in step on one XCD and fetch each weight
// tile once into its L2 for all of them (a full tile and a short last one drift apart, and
// each streams the weights from memory by itself).  Splitting in whole 32-row pairs instead
// (390 rows as 224 + 166, 13 pairs, not 195 + 195, 14 pairs) saves MFMAs but lets the tiles
// drift by a pair in seven: measured on MI355X it made the sigmoid layer's grouped GEMMs 24%
// slower.
// The map entries of expert e: c rows from position off, in mt M tiles from map index first.
__device__ __forceinline__ void write_tiles(int e, int c, int mt, int first, int off,
                                            int32_t* tiles) {
  const int base_rows = mt > 0 ? c / mt : 0, extra = mt > 0 ? c % mt : 0;
  for (int q = 0; q < mt; ++q) {
    int32_t* ent = tiles + (int64_t)(first + q) * kTileStride;
    ent[0] = e;
    ent[1] = off + q * base_rows + min(q, extra);
    ent[2] = base_rows + (q < extra ? 1 : 0);
    ent[3] = 0;
    ent[4] = first;
    ent[5] = mt;
    ent[6] = 0;
    ent[7] = 0;
  }
}

template <int NT>
__device__ void build_tiles(const int* cnt_lds, const int* off_lds, int E, int bm, int* scratch,
                            int32_t* tiles, int32_t* tile_count) {
  int total = 0;
  for (int base = 0; base < E; base += NT) {
    const int e = base + threadIdx.x;
    const int c = e < E ? cnt_lds[e] : 0;
    const int mt = (c + bm - 1) / bm;
    int chunk_total;
    const int first = block_exclusive_scan<NT>(mt, scratch, &chunk_total) + total;
    if (e < E) write_tiles(e, c, mt, first, off_lds[e], tiles);
    total += chunk_total;
  }
  if (threadIdx.x == 0) tile_count[0] = total;
}

__global__ void __launch_bounds__(kScanThreads) tile_map_kernel(const int32_t* __restrict__ offsets,
                                                                int E, int bm,
                                                                int32_t* __restrict__ tiles,
                                                                int32_t* __restrict__ tile_count) {
  extern __shared__ int sm[];
  int* cnt = sm;
  int* off = sm + E;
  int* scratch = sm + 2 * E;
  for (int e = threadIdx.x; e < E; e += kScanThreads) {
    off[e] = offsets[e];
    cnt[e] = offsets[e + 1] - offsets[e];
  }
  __syncthreads();
  build_tiles<kScanThreads>(cnt, off, E, bm, scratch, tiles, tile_count);
}

// Scan and scatter in one launch.  Work-group b owns segments [8 b, 8 b + 8), one per wave.
// Every work-group first re-derives, from the per-segment histograms, each expert's total
// (capped at the capacity) and the first rank of its own segments within the expert; the
// histograms are a few KiB per hundred segments, read from L2 in one batch of loads.
// Work-group 0 also writes the counts and offsets; with a tile map, one more work-group (the
// last, which owns no segment) builds it.  Then each wave re-reads its segment 64 ids at a time: lanes
// holding the same expert find each other with one ballot per bit of the expert id, and a
// lane's rank among its lower-numbered peers plus its expert's running rank (in LDS) is its
// rank q within the expert; offsets[e] + q is its position, unless q reaches the capacity.
constexpr int kSSThreads = 512;
constexpr int kSSWaves = kSSThreads / 64;
constexpr int kSSBatch = 64;  // histogram rows loaded together
static_assert(kSSWaves % kChunkSegs == 0, "a scatter work-group owns whole count chunks");

template <int R>
__global__ void __launch_bounds__(kSSThreads) scan_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t A, int E, int nbits, int cap, int64_t nseg,
    const int32_t* __restrict__ seg_counts, const int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    const int bm, int32_t* __restrict__ tiles, int32_t* __restrict__ tile_count) {
  extern __shared__ int sm[];
  int* run = sm;                      // [kSSWaves][E]: next rank in each expert, per segment
  int* cnt = run + kSSWaves * E;      // [E] rows kept
  int* off = cnt + E;                 // [E]
  int* scratch = off + E;             // [32]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seg0 = (int64_t)blockIdx.x * kSSWaves;

  // per expert: the count of every chunk (their sum is the expert's total; the chunks before
  // this work-group's first give the count of all earlier segments), then this work-group's own
  // segments one by one.  Loads go out a batch at a time: clamped rows, no branch between them.
  const int64_t nchunk = (nseg + kChunkSegs - 1) / kChunkSegs;
  const int64_t chunk0 = seg0 / kChunkSegs;  // kSSWaves is a multiple of kChunkSegs
  for (int e = threadIdx.x; e < E; e += kSSThreads) {
    int acc = 0, before = 0;
    for (int64_t c0 = 0; c0 < nchunk; c0 += kSSBatch) {
      int v[kSSBatch];
#pragma unroll
      for (int u = 0; u < kSSBatch; ++u) {
        const int64_t c = c0 + u < nchunk ? c0 + u : nchunk - 1;
        v[u] = chunk_counts[c * E + e];
      }
#pragma unroll
      for (int u = 0; u < kSSBatch; ++u) {
        const int64_t c = c0 + u;
        const int x = c < nchunk ? v[u] : 0;
        acc += x;
        if (c < chunk0) before += x;
      }
    }
    int own[kSSWaves];
#pragma unroll
    for (int w = 0; w < kSSWaves; ++w) {
      const int64_t sg = seg0 + w < nseg ? seg0 + w : nseg - 1;
      own[w] = seg_counts[sg * E + e];
    }
#pragma unroll
    for (int w = 0; w < kSSWaves; ++w) {
      if (seg0 + w < nseg) run[w * E + e] = before;
      before += seg0 + w < nseg ? own[w] : 0;
    }
    cnt[e] = acc < cap ? acc : cap;
  }
  __syncthreads();
  int total = 0;
  for (int base = 0; base < E; base += kSSThreads) {
    const int ee = base + threadIdx.x;
    const int v = ee < E ? cnt[ee] : 0;
    int chunk_total;
    const int ex = block_exclusive_scan<kSSThreads>(v, scratch, &chunk_total) + total;
    if (ee < E) {
      off[ee] = ex;
      if (blockIdx.x == 0) {
        counts[ee] = v;
        offsets[ee] = ex;
      }
    }
    total += chunk_total;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) offsets[E] = total;
  __syncthreads();
  // the tile maps come from the extra last work-group, which owns no segment, so that no
  // scatter waits for them
  if (tiles && blockIdx.x == gridDim.x - 1) {
    build_tiles<kSSThreads>(cnt, off, E, bm, scratch, tiles, tile_count);
    return;
  }

  const int64_t seg = seg0 + wave;
  if (seg >= nseg) return;  // after every work-group barrier
  int* r = run + wave * E;
  const int64_t a0 = seg * (64 * R);
  int ev[R];
#pragma unroll
  for (int rd = 0; rd < R; ++rd) {
    const int64_t a = a0 + rd * 64 + lane;
    ev[rd] = a < A ? idx[a] : -1;
  }
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int rd = 0; rd < R; ++rd) {
    if (a0 + rd * 64 >= A) break;  // uniform: the rest of a short last segment is empty
    const int64_t a = a0 + rd * 64 + lane;
    const int e = ev[rd];
    const bool valid = e >= 0 && e < E;
    unsigned long long peers = __ballot(valid);
    for (int bt = 0; bt < nbits; ++bt) {
      const bool bit = (e >> bt) & 1;
      const unsigned long long m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & lt);
      const int base = r[e], first = off[e];  // both LDS reads in flight together
      const int q = base + rank;  // rank of this assignment within its expert
      if (q < cap) {
        const int pos = first + q;
        perm[pos] = (int32_t)a;
        inv_perm[a] = pos;
      } else {
        inv_perm[a] = -1;  // over capacity: dropped
      }
      if (rank == 0) r[e] = base + __popcll(peers);
    } else if (a < A) {
      inv_perm[a] = -1;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }
}

// Whole dispatch in one work-group, for batches whose launch latency would otherwise dominate:
// wave w owns the contiguous range [w*L, (w+1)*L) of assignment ids.  Count (LDS atomics into
// the wave's own histogram), exclusive prefix over waves per expert, expert offsets, tile maps,
// then the same ballot-ranked stable scatter as scan_scatter_kernel.  Wave ranges, rounds and lanes
// all follow ascending a, so the result equals the multi-kernel path's bit for bit.
constexpr int kFusedWaves = kScanThreads / 64;
constexpr int kFusedBatch = 8;  // 64-id rounds whose loads are issued together

static_assert(kFusedMaxA <= (int64_t)kFusedWaves * 64 * kFusedBatch,
              "automatic one-work-group batches fit one batch of ids per wave");
static_assert(kFusedMaxE <= kScanThreads, "one expert per thread in the scans");

__global__ void __launch_bounds__(kScanThreads) dispatch_fused_kernel(
    const int32_t* __restrict__ idx, int64_t A, int E, int nbits, int cap,
    int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    const int bm, int32_t* __restrict__ tiles, int32_t* __restrict__ tile_count) {
  extern __shared__ int sm[];
  int* hist = sm;                       // [kFusedWaves][E]: counts, then running ranks
  int* off = hist + kFusedWaves * E;    // [E]
  int* scratch = off + E;               // [2 kFusedWaves]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t L = ((A + kFusedWaves - 1) / kFusedWaves + 63) / 64 * 64;
  const int64_t a_begin = wave * L, a_end = min(A, a_begin + L);
  // The wave's ids, a batch of 64 * kFusedBatch at a time; the first batch is requested before
  // anything else.  When a wave's range is one batch (always, unless this path is forced for a
  // larger batch), the scatter reuses it instead of loading the ids again.
  const bool one_batch = L <= 64 * kFusedBatch;  // the same for every wave
  int ev[kFusedBatch];
  const auto load_ids = [&](int64_t b0) {
#pragma unroll
    for (int r = 0; r < kFusedBatch; ++r) {
      const int64_t a = b0 + r * 64 + lane;
      ev[r] = a < a_end ? idx[a] : -1;
    }
  };
  load_ids(a_begin);
  int* h = hist + wave * E;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  for (int64_t b0 = a_begin;;) {
#pragma unroll
    for (int r = 0; r < kFusedBatch; ++r)
      if (ev[r] >= 0 && ev[r] < E) atomicAdd(&h[ev[r]], 1);
    b0 += 64 * kFusedBatch;
    if (b0 >= a_end) break;
    load_ids(b0);
  }
  __syncthreads();
  // thread e: each wave's first position within expert e, the rows it keeps, their M tiles;
  // then the expert offsets and the tile map's first entries in one pair of scans
  const int e = threadIdx.x;
  int kept = 0;
  if (e < E) {
    int c[kFusedWaves];  // every wave's count read before the first running rank is written
#pragma unroll
    for (int w = 0; w < kFusedWaves; ++w) c[w] = hist[w * E + e];
    int run = 0;
#pragma unroll
    for (int w = 0; w < kFusedWaves; ++w) {
      hist[w * E + e] = run;
      run += c[w];
    }
    kept = run < cap ? run : cap;
  }
  const int mt = tiles ? (kept + bm - 1) / bm : 0;
  int first_row, first_tile, rows_total, tiles_total;
  block_exclusive_scan2<kScanThreads>(kept, mt, scratch, &first_row, &first_tile, &rows_total,
                                      &tiles_total);
  if (e < E) {
    off[e] = first_row;
    counts[e] = kept;
    offsets[e] = first_row;
    if (tiles) write_tiles(e, kept, mt, first_tile, first_row, tiles);
  }
  if (threadIdx.x == 0) {
    offsets[E] = rows_total;
    if (tiles) tile_count[0] = tiles_total;
  }
  __syncthreads();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t b0 = a_begin; b0 < a_end; b0 += 64 * kFusedBatch) {
    if (!one_batch) load_ids(b0);
#pragma unroll
    for (int r = 0; r < kFusedBatch; ++r) {
      if (b0 + r * 64 >= a_end) break;  // uniform: no id of this wave's range is left
      const int64_t a = b0 + r * 64 + lane;
      const int ee = ev[r];
      const bool valid = ee >= 0 && ee < E;
      unsigned long long peers = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (ee >> b) & 1;
        const unsigned long long m = __ballot(bit);
        peers &= bit ? m : ~m;
      }
      if (valid) {
        const int rank = __popcll(peers & lt);
        const int base = h[ee], first = off[ee];  // both LDS reads in flight together
        const int q = base + rank;  // rank within the expert
        if (q < cap) {
          const int pos = first + q;
          perm[pos] = (int32_t)a;
          inv_perm[a] = pos;
        } else {
          inv_perm[a] = -1;  // over capacity: dropped
        }
        if (rank == 0) h[ee] = base + __popcll(peers);
      } else if (a < a_end) {
        inv_perm[a] = -1;
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <typename V>
__global__ void __launch_bounds__(256) gather_rows_kernel(const V* __restrict__ x, int64_t vrow,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ offsets,
                                                          int E, int K, int64_t A,
                                                          V* __restrict__ x_perm) {
  const int64_t valid = offsets[E];
  for (int64_t pos = blockIdx.x; pos < valid; pos += gridDim.x) {
    const int64_t tok = perm[pos] / K;
    const V* src = x + tok * vrow;
    V* dst = x_perm + pos * vrow;
    for (int64_t c = threadIdx.x; c < vrow; c += blockDim.x) dst[c] = src[c];
  }
}

}  // namespace

int dispatch_segment_len(int64_t A) { return 64 * seg_rounds(A); }

bool dispatch_supported(int E, int path) { return path != 1 || E <= kFusedMaxE; }

bool dispatch_fused(int64_t A, int E, int path) {
  if (path == 1) return true;
  if (path == 2) return false;
  return A <= kFusedMaxA && E <= kFusedMaxE;
}

int64_t dispatch_num_segments(int64_t A) {
  const int64_t len = dispatch_segment_len(A);
  return (A + len - 1) / len;
}

hipError_t launch_dispatch(const int32_t* idx, int64_t A, int E, int32_t* seg_counts,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                           int cap, int path, int bm, int32_t* tiles, int32_t* tile_count,
                           hipStream_t stream) {
  const int64_t nseg = dispatch_num_segments(A);
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  if (dispatch_fused(A, E, path)) {
    const size_t lds = (size_t)((kFusedWaves + 1) * E + 2 * kFusedWaves) * sizeof(int);
    hipLaunchKernelGGL(dispatch_fused_kernel, dim3(1), dim3(kScanThreads), lds, stream, idx, A,
                       E, nbits, cap, counts, offsets, perm, inv_perm, bm, tiles, tile_count);
    return hipGetLastError();
  }
  const auto go = [&](auto rounds) -> hipError_t {
    constexpr int R = decltype(rounds)::value;
    const dim3 g((unsigned)((nseg + 3) / 4)), b(256);
    hipLaunchKernelGGL(count_kernel<R>, g, b, (size_t)4 * E * sizeof(int), stream, idx, A, E,
                       nseg, seg_counts, seg_counts + nseg * E);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t lds = (size_t)((kSSWaves + 2) * E + 32) * sizeof(int);
    const unsigned groups = (unsigned)((nseg + kSSWaves - 1) / kSSWaves) + (tiles ? 1 : 0);
    const int32_t* chunk_counts = seg_counts + nseg * E;
    hipLaunchKernelGGL(scan_scatter_kernel<R>, dim3(groups), dim3(kSSThreads), lds, stream, idx,
                       A, E, nbits, cap, nseg, seg_counts, chunk_counts, counts, offsets, perm,
                       inv_perm, bm, tiles, tile_count);
    return hipGetLastError();
  };
  switch (seg_rounds(A)) {
    case 2: return go(std::integral_constant<int, 2>{});
    case 4: return go(std::integral_constant<int, 4>{});
    default: return go(std::integral_constant<int, kMaxSegRounds>{});
  }
}

hipError_t launch_tile_map(const int32_t* offsets, int E, int bm, int32_t* tiles,
                           int32_t* tile_count, hipStream_t stream) {
  const size_t lds = (size_t)(2 * E + 32) * sizeof(int);
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(kScanThreads), lds, stream, offsets, E, bm,
                     tiles, tile_count);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, int64_t D, int esize, const int32_t* perm,
                              const int32_t* offsets, int E, int K, int64_t A, void* x_perm,
                              hipStream_t stream) {
  if (A <= 0) return hipSuccess;
  const int64_t row_bytes = D * esize;  // multiple of 128 (D % 64 == 0)
  const int64_t vrow = row_bytes / 16;
  const int64_t grid = A < 4096 ? A : 4096;
  hipLaunchKernelGGL(gather_rows_kernel<uint4>, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const uint4*)x, vrow, perm, offsets, E, K, A, (uint4*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
