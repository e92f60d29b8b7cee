// Router scoring, top-K selection and renormalisation ("MoE" §2 Router; "1.6 混合专家（MoE）"
// §二 Top-k 门控公式 steps 2-3).
//
// One wave64 per token.  Lane l holds logits l, l+64, ... as 64-bit keys
//   (order-preserving image of the fp32 logit) << 32 | (0xFFFFFFFF - expert id)
// so one unsigned max picks the largest logit and, among equal logits, the lowest id.  NaN is
// mapped to -inf's key and -0.0 to +0.0's key before packing.  K rounds of a butterfly max
// over the wave select the experts in descending order; the winner's key is cleared.
//
// Selection compares logits, not probabilities: softmax and sigmoid are strictly increasing,
// so the top-K set is the same, and the choice does not depend on exp/sigmoid rounding.
// Softmax weights use only the K selected logits: the full-E denominator cancels in
// p_e / sum_{j in I} p_j, leaving exp(r_e - r_max) / sum_{j in I} exp(r_j - r_max).
#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (v != v) u = 0xFF800000u;          // NaN ranks as -inf
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const unsigned long long o = __shfl_xor(v, m, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int NPL>  // logits held per lane: ceil(E / 64)
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int64_t T,
                                                   int E, int K, int scoring, int renorm,
                                                   int32_t* __restrict__ idx, float* __restrict__ w,
                                                   const float* __restrict__ gate_logit,
                                                   float* __restrict__ gate_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;

  unsigned long long key[NPL];
  float val[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      val[j] = row[e];
      key[j] = ((unsigned long long)order_key(val[j]) << 32) | (0xFFFFFFFFu - (uint32_t)e);
    } else {
      val[j] = 0.0f;
      key[j] = 0ull;  // below every real key
    }
  }

  // Slot k (k < K <= 64) is kept by lane k: its logit and expert id.
  float top = 0.0f, my_val = 0.0f;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    unsigned long long best = key[0];
#pragma unroll
    for (int j = 1; j < NPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const uint32_t e = 0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull);
    const float v = key_value((uint32_t)(best >> 32));
    if (k == 0) top = v;
    if ((int)(e & 63u) == lane) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (j == (int)(e >> 6)) key[j] = 0ull;
    }
    if (lane == k) {
      my_val = v;
      my_id = (int)e;
    }
  }

  float s = 0.0f;
  if (lane < K) s = scoring == 0 ? expf(my_val - top) : 1.0f / (1.0f + expf(-my_val));
  float denom;
  if (renorm) {
    denom = wave_sum(s);
  } else if (scoring == 0) {
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      if (lane + 64 * j < E) part += expf(val[j] - top);
    denom = wave_sum(part);
  } else {
    denom = 1.0f;
  }
  if (lane < K) {
    idx[t * K + lane] = my_id;
    w[t * K + lane] = s / denom;
  }
  if (gate_out && lane == 0) gate_out[t] = 1.0f / (1.0f + expf(-gate_logit[t]));
}

}  // namespace

hipError_t launch_topk(const float* logits, int64_t T, int E, int K, int scoring, int renorm,
                       int32_t* idx, float* w, const float* gate_logit, float* gate_out,
                       hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  dim3 g((unsigned)((T + 3) / 4)), b(256);
  const int npl = (E + 63) / 64;
#define MOE_TOPK_CASE(N)                                                                      \
  case N:                                                                                     \
    hipLaunchKernelGGL(topk_kernel<N>, g, b, 0, stream, logits, T, E, K, scoring, renorm, idx, \
                       w, gate_logit, gate_out);                                              \
    break;
  switch (npl) {
    MOE_TOPK_CASE(1)
    MOE_TOPK_CASE(2)
    MOE_TOPK_CASE(3)
    MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(5)
    MOE_TOPK_CASE(6)
    MOE_TOPK_CASE(7)
    MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(9)
    MOE_TOPK_CASE(10)
    MOE_TOPK_CASE(11)
    MOE_TOPK_CASE(12)
    MOE_TOPK_CASE(13)
    MOE_TOPK_CASE(14)
    MOE_TOPK_CASE(15)
    MOE_TOPK_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

}  // namespace moe
