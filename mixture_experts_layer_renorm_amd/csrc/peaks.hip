// Machine-peak probes (include/moe_peaks.h): a streaming HBM read and a register-only MFMA
// loop.  They measure the two roofline ceilings of the layer's kernels on the running GPU, at
// the clock it holds under that load ("S23-J10" §3: a grouped GEMM over expert weights is bound
// by reading them when each expert sees few rows, by the matrix cores when it sees hundreds).
#include "moe_peaks.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kReadGroups = 8192;
constexpr int kReadThreads = 512;
constexpr int kReadDepth = 4;  // 16-byte loads in flight per lane

// Each work-group sweeps one contiguous chunk of the buffer (the fastest of the read patterns
// measured on MI355X: a grid-stride sweep reaches about 10% less).  The sink is written only
// if a work-group's loaded words XOR to a fixed value, which keeps every load alive.
__global__ void __launch_bounds__(kReadThreads) hbm_read_kernel(const uint4* __restrict__ buf,
                                                                int64_t n16,
                                                                float* __restrict__ sink) {
  const int64_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n16 ? lo + chunk : n16;
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)kReadDepth * kReadThreads) {
    uint4 v[kReadDepth];
#pragma unroll
    for (int k = 0; k < kReadDepth; ++k)
      v[k] = i + k * kReadThreads < hi ? buf[i + k * kReadThreads] : uint4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kReadDepth; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 2047] = 1.0f;
}

// Four independent 32 x 32 accumulators per wave, each updated by v_mfma_f32_32x32x16_bf16 on
// register operands: enough independent work per SIMD to keep the matrix unit issuing back to
// back (measured: 95-99% of the data-sheet rate at 1-4 waves per SIMD; fewer chains of the
// 16 x 16 x 32 instruction issue only about every other slot).
__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* __restrict__ sink) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)((float)((lane + j + iters) & 7) * 0.125f);
    b[j] = (__bf16)((float)((lane * 3 + j) & 7) * 0.0625f);
  }
  constexpr int kChains = 4;
  f32x16 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += acc[k][0] + acc[k][15];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_peak_hbm_read(const void* buf, size_t bytes, float* sink, moe_stream_t stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) ||
      (reinterpret_cast<uintptr_t>(sink) & 15) || bytes == 0 || bytes % 65536)
    return MOE_ERR_INVALID_ARG;
  // at least 64 KiB per work-group
  const size_t groups = bytes / 65536 < (size_t)moe::kReadGroups ? bytes / 65536
                                                                  : (size_t)moe::kReadGroups;
  hipLaunchKernelGGL(moe::hbm_read_kernel, dim3((unsigned)groups), dim3(moe::kReadThreads), 0,
                     (hipStream_t)stream, (const uint4*)buf, (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_peak_mfma_bf16(int waves, int iters, float* sink, moe_stream_t stream) {
  if (!sink || (reinterpret_cast<uintptr_t>(sink) & 15) || waves <= 0 || waves % 4 ||
      waves > 65536 || iters < 0)
    return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(moe::mfma_loop_kernel, dim3(waves / 4), dim3(256), 0, (hipStream_t)stream,
                     iters, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
