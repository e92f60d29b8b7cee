// Combine and output conversion ("MoE" §3.2: weighted rows are accumulated back at their
// tokens; §4: the routed and shared branches are added).
//
// combine : deterministic gather-sum.  One work-group per token: the K rows of the token's
//           expert outputs are read through inv_perm and summed in slot order in fp32, the
//           shared branch is added with its gate, and the sum is rounded once to the output
//           dtype.  16-byte loads along D.  combine16 reads the same rows stored as fp16 with
//           a power-of-two factor per 256-column block.
// cast    : fp32 accumulator -> output dtype (round to nearest even), for the atomic path.
// zero    : fill an fp32 accumulator with +0.0 (a kernel, not a memset node).
#include <type_traits>

#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ void store4(float* dst, float4 v) { *(float4*)dst = v; }
__device__ __forceinline__ void store4(__bf16* dst, float4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 o;
  o[0] = (__bf16)v.x;
  o[1] = (__bf16)v.y;
  o[2] = (__bf16)v.z;
  o[3] = (__bf16)v.w;
  *(bf16x4*)dst = o;
}

template <typename OUT>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ y_shared,
                                                      const float* __restrict__ gate, int64_t T,
                                                      int K, int D, OUT* __restrict__ out) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const float g = y_shared ? (gate ? gate[t] : 1.0f) : 0.0f;
    for (int d = threadIdx.x * 4; d < D; d += blockDim.x * 4) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < K; ++k) {
        const int pos = inv_perm[t * K + k];
        if (pos < 0) continue;  // sentinel assignment
        const float w = topk_w[t * K + k];
        const float4 v = *(const float4*)(y_perm + (int64_t)pos * D + d);
        acc.x += w * v.x;
        acc.y += w * v.y;
        acc.z += w * v.z;
        acc.w += w * v.w;
      }
      if (y_shared) {
        const float4 v = *(const float4*)(y_shared + t * D + d);
        acc.x += g * v.x;
        acc.y += g * v.y;
        acc.z += g * v.z;
        acc.w += g * v.w;
      }
      store4(out + t * D + d, acc);
    }
  }
}

__device__ __forceinline__ void store8(float* dst, const float* a) {
  *(float4*)dst = make_float4(a[0], a[1], a[2], a[3]);
  *(float4*)(dst + 4) = make_float4(a[4], a[5], a[6], a[7]);
}
__device__ __forceinline__ void store8(__bf16* dst, const float* a) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (__bf16)a[i];
  *(bf16x8*)dst = o;
}

// Gather-sum over fp16 expert rows with per-(row, kScaleCols-column block) factors: 8 columns per
// thread (one 16-byte load per slot), in slot order, then the shared branch -- fp32 rows, or
// (SH16) fp16 rows with the same kind of factors -- each term one fma, one rounding.  The slots
// are taken 8 at a time: their positions and weights are uniform loads, and the 8 row chunks
// and factors are all requested before the first is added, so each wave keeps 8 row loads in
// flight instead of one (the sum is still formed in slot order).
constexpr int kSlotBatch = 8;

template <typename OUT, bool SH16>
__global__ void __launch_bounds__(512) combine16_kernel(const _Float16* __restrict__ y16,
                                                        const float* __restrict__ ysc, int nblk,
                                                        const int32_t* __restrict__ inv_perm,
                                                        const float* __restrict__ topk_w,
                                                        const void* __restrict__ y_shared,
                                                        const float* __restrict__ ys_sc,
                                                        const float* __restrict__ gate, int64_t T,
                                                        int K, int D, OUT* __restrict__ out) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const float g = y_shared ? (gate ? gate[t] : 1.0f) : 0.0f;
    for (int d = threadIdx.x * 8; d < D; d += blockDim.x * 8) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      const int blk = d / kScaleCols;
      // the shared branch's row goes out with the first batch of slot loads
      float sh[8], gs = g;
      if (y_shared) {
        if constexpr (SH16) {
          gs = g * ys_sc[t * nblk + blk];
          const f16x8 v = *(const f16x8*)((const _Float16*)y_shared + t * D + d);
#pragma unroll
          for (int i = 0; i < 8; ++i) sh[i] = (float)v[i];
        } else {
          const float* ys = (const float*)y_shared;
          const float4 a = *(const float4*)(ys + t * D + d);
          const float4 b = *(const float4*)(ys + t * D + d + 4);
          sh[0] = a.x; sh[1] = a.y; sh[2] = a.z; sh[3] = a.w;
          sh[4] = b.x; sh[5] = b.y; sh[6] = b.z; sh[7] = b.w;
        }
      }
      for (int k0 = 0; k0 < K; k0 += kSlotBatch) {
        int pos[kSlotBatch];
        float w[kSlotBatch];
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u) {
          const int k = k0 + u;
          pos[u] = k < K ? inv_perm[t * K + k] : -1;
          w[u] = k < K ? topk_w[t * K + k] : 0.0f;
        }
        f16x8 v[kSlotBatch];
        float sc[kSlotBatch];
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u) {
          // a sentinel, dropped or past-K slot (pos < 0) reads row 0 and is not added: loads
          // without branches between them go out back to back
          const int64_t row = pos[u] < 0 ? 0 : pos[u];
          sc[u] = ysc[row * nblk + blk];
          v[u] = *(const f16x8*)(y16 + row * D + d);
        }
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u) {
          const float wu = w[u] * sc[u];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float a = __builtin_fmaf(wu, (float)v[u][i], acc[i]);
            acc[i] = pos[u] < 0 ? acc[i] : a;
          }
        }
      }
      if (y_shared) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(gs, sh[i], acc[i]);
      }
      store8(out + t * D + d, acc);
    }
  }
}

__global__ void __launch_bounds__(256) cast_bf16_kernel(const float* __restrict__ src,
                                                        __bf16* __restrict__ dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x)
    store4(dst + 4 * i, ((const float4*)src)[i]);
}

__global__ void __launch_bounds__(256) zero_kernel(float4* __restrict__ dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

unsigned grid_for(int64_t n4) {
  int64_t g = (n4 + 255) / 256;
  const int64_t cap = (int64_t)kCus * 8;
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w,
                          const float* y_shared, const float* gate, int64_t T, int K, int D,
                          void* out, int out_dtype, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t cap = (int64_t)kCus * 16;
  const dim3 g((unsigned)(T < cap ? T : cap)), b(256);
  if (out_dtype == 1)
    hipLaunchKernelGGL(combine_kernel<__bf16>, g, b, 0, stream, y_perm, inv_perm, topk_w, y_shared,
                       gate, T, K, D, (__bf16*)out);
  else
    hipLaunchKernelGGL(combine_kernel<float>, g, b, 0, stream, y_perm, inv_perm, topk_w, y_shared,
                       gate, T, K, D, (float*)out);
  return hipGetLastError();
}

hipError_t launch_combine16(const void* y16, const float* ysc, int nblk, const int32_t* inv_perm,
                            const float* topk_w, const void* y_shared, const float* ys_sc,
                            const float* gate, int64_t T, int K, int D, void* out, int out_dtype,
                            hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t cap = (int64_t)kCus * 16;
  // rows of 4096 or more columns: 512 threads, so one pass covers 4096 columns of each row
  // (measured 1-2% faster than two passes of 256 threads at D = 4096)
  const dim3 g((unsigned)(T < cap ? T : cap)), b(D >= 4096 ? 512 : 256);
  const auto go = [&](auto out_t, auto sh16) {
    using OUT = decltype(out_t);
    hipLaunchKernelGGL((combine16_kernel<OUT, decltype(sh16)::value>), g, b, 0, stream,
                       (const _Float16*)y16, ysc, nblk, inv_perm, topk_w, y_shared, ys_sc, gate, T,
                       K, D, (OUT*)out);
  };
  const bool sh16 = y_shared && ys_sc;
  if (out_dtype == 1) {
    if (sh16) go(__bf16{}, std::true_type{}); else go(__bf16{}, std::false_type{});
  } else {
    if (sh16) go(float{}, std::true_type{}); else go(float{}, std::false_type{});
  }
  return hipGetLastError();
}

hipError_t launch_cast(const float* src, void* dst, int64_t n, int out_dtype, hipStream_t stream) {
  if (n <= 0 || out_dtype != 1) return hipSuccess;
  const int64_t n4 = n / 4;  // n = T*D, D % 64 == 0
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for(n4)), dim3(256), 0, stream, src, (__bf16*)dst,
                     n4);
  return hipGetLastError();
}

hipError_t launch_zero(float* dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n4)), dim3(256), 0, stream, (float4*)dst, n4);
  return hipGetLastError();
}

}  // namespace moe
