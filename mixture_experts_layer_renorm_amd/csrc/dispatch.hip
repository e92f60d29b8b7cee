// Dispatch: per-expert histogram, prefix sum and a stable counting sort of the T*K assignments
// into expert-contiguous order ("MoE" §3.2: the tokens routed to each hit expert are gathered so
// that the expert runs once on all of them; "1.6 混合专家（MoE）" §二: route, group, compute,
// merge).
//
// The assignments a = t*K + k are cut into segments of 512 consecutive ids, one wave64 each
// (each lane prefetches its 8 ids of the segment at once).
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
#include <cstdlib>
#include <cstring>

#include "kernels.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kSegRounds = 8;                // 64-id rounds per segment
constexpr int kSegLen = 64 * kSegRounds;      // assignments per segment (one wave)
// Single-work-group dispatch up to this many assignments (its LDS holds 18 ints per expert).
constexpr int64_t kFusedMaxA = 8192;
constexpr int kFusedMaxE = 768;

__device__ __forceinline__ int wave_prefix_exclusive(int v, int lane) {
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x - v;
}

// Exclusive scan of one int per thread across an NT-thread block.  Returns the prefix and
// writes the block total to *total.
template <int NT>
__device__ int block_exclusive_scan(int v, int* scratch /* >= NT / 64 + 1 ints */, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ex = wave_prefix_exclusive(v, lane);
  if (lane == 63) scratch[wave] = ex + v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int c = scratch[w];
      scratch[w] = run;
      run += c;
    }
    scratch[NT / 64] = run;
  }
  __syncthreads();
  const int r = ex + scratch[wave];
  *total = scratch[NT / 64];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(256) count_kernel(const int32_t* __restrict__ idx, int64_t A,
                                                    int E, int64_t nseg,
                                                    int32_t* __restrict__ seg_counts) {
  extern __shared__ int hist_all[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seg = (int64_t)blockIdx.x * 4 + wave;
  if (seg >= nseg) return;  // whole wave; no block-wide barrier below
  int* hist = hist_all + wave * E;
  for (int e = lane; e < E; e += 64) hist[e] = 0;
  const int64_t a0 = seg * kSegLen;
  int ev[kSegRounds];
#pragma unroll
  for (int r = 0; r < kSegRounds; ++r) {
    const int64_t a = a0 + r * 64 + lane;
    ev[r] = a < A ? idx[a] : -1;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < kSegRounds; ++r)
    if (ev[r] >= 0 && ev[r] < E) atomicAdd(&hist[ev[r]], 1);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
  for (int e = lane; e < E; e += 64) seg_counts[seg * E + e] = hist[e];
}

// Builds the tile maps from per-expert counts held in LDS.  One entry per M tile:
// {expert, first row position, rows, 0, first M tile of the expert, M tiles of the expert};
// experts with more than ts.split rows go to map 1 (bm1-row tiles), the others to map 0.
// An expert's rows are split evenly over its ceil(c / bm) M tiles (the first c % mt tiles one
// row more): its tiles then cost the same, run in step on one XCD and fetch each weight tile
// once into its L2 for all of them (a full tile and a short last one drift apart, and each
// streams the weights from memory by itself).
template <int NT>
__device__ void build_tiles(const int* cnt_lds, const int* off_lds, int E, const TileSplit ts,
                            int* scratch, int32_t* tiles, int32_t* tile_count) {
  int32_t* maps[2] = {tiles, tiles + ts.map1_entries * kTileStride};
  const int bms[2] = {ts.bm0, ts.bm1};
  int total[2] = {0, 0};
  for (int base = 0; base < E; base += NT) {
    const int e = base + threadIdx.x;
    const int c = e < E ? cnt_lds[e] : 0;
    const int which = (ts.split >= 0 && c > ts.split) ? 1 : 0;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int bm = bms[m];
      const int mt = which == m ? (c + bm - 1) / bm : 0;
      int chunk_total;
      const int first = block_exclusive_scan<NT>(mt, scratch, &chunk_total) + total[m];
      const int base_rows = mt > 0 ? c / mt : 0, extra = mt > 0 ? c % mt : 0;
      for (int q = 0; q < mt; ++q) {
        int32_t* ent = maps[m] + (int64_t)(first + q) * kTileStride;
        ent[0] = e;
        ent[1] = off_lds[e] + q * base_rows + min(q, extra);
        ent[2] = base_rows + (q < extra ? 1 : 0);
        ent[3] = 0;
        ent[4] = first;
        ent[5] = mt;
        ent[6] = 0;
        ent[7] = 0;
      }
      total[m] += chunk_total;
    }
  }
  if (threadIdx.x == 0) {
    tile_count[0] = total[0];
    tile_count[1] = total[1];
  }
}

__global__ void __launch_bounds__(kScanThreads) tile_map_kernel(const int32_t* __restrict__ offsets,
                                                                int E, const TileSplit ts,
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
  build_tiles<kScanThreads>(cnt, off, E, ts, scratch, tiles, tile_count);
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

__global__ void __launch_bounds__(kSSThreads) scan_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t A, int E, int nbits, int cap, int64_t nseg,
    const int32_t* __restrict__ seg_counts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    const TileSplit ts, int32_t* __restrict__ tiles, int32_t* __restrict__ tile_count) {
  extern __shared__ int sm[];
  int* run = sm;                      // [kSSWaves][E]: next rank in each expert, per segment
  int* cnt = run + kSSWaves * E;      // [E] rows kept
  int* off = cnt + E;                 // [E]
  int* scratch = off + E;             // [32]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seg0 = (int64_t)blockIdx.x * kSSWaves;

  for (int e = threadIdx.x; e < E; e += kSSThreads) {
    int acc = 0;
    for (int64_t s0 = 0; s0 < nseg; s0 += kSSBatch) {
      int v[kSSBatch];
#pragma unroll
      for (int u = 0; u < kSSBatch; ++u) v[u] = s0 + u < nseg ? seg_counts[(s0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kSSBatch; ++u) {
        const int64_t sg = s0 + u;
        if (sg >= seg0 && sg < seg0 + kSSWaves) run[(sg - seg0) * E + e] = acc;
        acc += v[u];
      }
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
    build_tiles<kSSThreads>(cnt, off, E, ts, scratch, tiles, tile_count);
    return;
  }

  const int64_t seg = seg0 + wave;
  if (seg >= nseg) return;  // after every work-group barrier
  int* r = run + wave * E;
  const int64_t a0 = seg * kSegLen;
  int ev[kSegRounds];
#pragma unroll
  for (int rd = 0; rd < kSegRounds; ++rd) {
    const int64_t a = a0 + rd * 64 + lane;
    ev[rd] = a < A ? idx[a] : -1;
  }
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int rd = 0; rd < kSegRounds; ++rd) {
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
      const int base = r[e];
      const int q = base + rank;  // rank of this assignment within its expert
      if (q < cap) {
        const int pos = off[e] + q;
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

__global__ void __launch_bounds__(kScanThreads) dispatch_fused_kernel(
    const int32_t* __restrict__ idx, int64_t A, int E, int nbits, int cap,
    int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    const TileSplit ts, int32_t* __restrict__ tiles, int32_t* __restrict__ tile_count) {
  extern __shared__ int sm[];
  int* hist = sm;                       // [kFusedWaves][E]: counts, then running ranks
  int* cnt = hist + kFusedWaves * E;    // [E]
  int* off = cnt + E;                   // [E]
  int* scratch = off + E;               // [32]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t L = ((A + kFusedWaves - 1) / kFusedWaves + 63) / 64 * 64;
  const int64_t a_begin = wave * L, a_end = min(A, a_begin + L);
  int* h = hist + wave * E;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  for (int64_t b0 = a_begin; b0 < a_end; b0 += 64 * kFusedBatch) {
    int ev[kFusedBatch];
#pragma unroll
    for (int r = 0; r < kFusedBatch; ++r) {
      const int64_t a = b0 + r * 64 + lane;
      ev[r] = a < a_end ? idx[a] : -1;
    }
#pragma unroll
    for (int r = 0; r < kFusedBatch; ++r)
      if (ev[r] >= 0 && ev[r] < E) atomicAdd(&h[ev[r]], 1);
  }
  __syncthreads();
  // per expert: each wave's first position within the expert, and the expert's count
  for (int e = threadIdx.x; e < E; e += kScanThreads) {
    int run = 0;
    for (int w = 0; w < kFusedWaves; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    cnt[e] = run < cap ? run : cap;  // rows kept
  }
  __syncthreads();
  int total = 0;
  for (int base = 0; base < E; base += kScanThreads) {
    const int ee = base + threadIdx.x;
    const int v = ee < E ? cnt[ee] : 0;
    int chunk_total;
    const int ex = block_exclusive_scan<kScanThreads>(v, scratch, &chunk_total) + total;
    if (ee < E) {
      off[ee] = ex;
      counts[ee] = v;
      offsets[ee] = ex;
    }
    total += chunk_total;
  }
  if (threadIdx.x == 0) offsets[E] = total;
  __syncthreads();
  if (tiles) build_tiles<kScanThreads>(cnt, off, E, ts, scratch, tiles, tile_count);
  __syncthreads();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t b0 = a_begin; b0 < a_end; b0 += 64 * kFusedBatch) {
    int ev[kFusedBatch];
#pragma unroll
    for (int r = 0; r < kFusedBatch; ++r) {
      const int64_t a = b0 + r * 64 + lane;
      ev[r] = a < a_end ? idx[a] : -1;
    }
#pragma unroll
    for (int r = 0; r < kFusedBatch; ++r) {
      const int64_t a = b0 + r * 64 + lane;
      const int e = ev[r];
      const bool valid = e >= 0 && e < E;
      unsigned long long peers = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long m = __ballot(bit);
        peers &= bit ? m : ~m;
      }
      if (valid) {
        const int rank = __popcll(peers & lt);
        const int base = h[e];
        const int q = base + rank;  // rank within the expert
        if (q < cap) {
          const int pos = off[e] + q;
          perm[pos] = (int32_t)a;
          inv_perm[a] = pos;
        } else {
          inv_perm[a] = -1;  // over capacity: dropped
        }
        if (rank == 0) h[e] = base + __popcll(peers);
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

int dispatch_segment_len(int64_t) { return kSegLen; }

bool dispatch_fused(int64_t A, int E) {
  bool fused = A <= kFusedMaxA && E <= kFusedMaxE;
  if (const char* o = std::getenv("MOE_DISPATCH")) {
    if (!std::strcmp(o, "fused")) fused = E <= kFusedMaxE;
    if (!std::strcmp(o, "multi")) fused = false;
  }
  return fused;
}

int64_t dispatch_num_segments(int64_t A) { return (A + kSegLen - 1) / kSegLen; }

hipError_t launch_dispatch(const int32_t* idx, int64_t A, int E, int32_t* seg_counts,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                           int cap, const TileSplit& ts, int32_t* tiles, int32_t* tile_count,
                           hipStream_t stream) {
  const int64_t nseg = dispatch_num_segments(A);
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  if (dispatch_fused(A, E)) {
    const size_t lds = (size_t)((kFusedWaves + 2) * E + 32) * sizeof(int);
    hipLaunchKernelGGL(dispatch_fused_kernel, dim3(1), dim3(kScanThreads), lds, stream, idx, A,
                       E, nbits, cap, counts, offsets, perm, inv_perm, ts, tiles, tile_count);
    return hipGetLastError();
  }
  const dim3 g((unsigned)((nseg + 3) / 4)), b(256);
  hipLaunchKernelGGL(count_kernel, g, b, (size_t)4 * E * sizeof(int), stream, idx, A, E, nseg,
                     seg_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds = (size_t)((kSSWaves + 2) * E + 32) * sizeof(int);
  const unsigned groups = (unsigned)((nseg + kSSWaves - 1) / kSSWaves) + (tiles ? 1 : 0);
  hipLaunchKernelGGL(scan_scatter_kernel, dim3(groups), dim3(kSSThreads), lds, stream, idx, A, E, nbits, cap, nseg, seg_counts,
                     counts, offsets, perm, inv_perm, ts, tiles, tile_count);
  return hipGetLastError();
}

hipError_t launch_tile_map(const int32_t* offsets, int E, const TileSplit& ts, int32_t* tiles,
                           int32_t* tile_count, hipStream_t stream) {
  const size_t lds = (size_t)(2 * E + 32) * sizeof(int);
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(kScanThreads), lds, stream, offsets, E, ts,
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
