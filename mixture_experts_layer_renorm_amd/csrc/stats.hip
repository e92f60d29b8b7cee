// Router statistics of one routed batch: the load fractions f_i and mean router probabilities
// P_i of the auxiliary balance loss and the loss itself, N·Σ f_i P_i ("1.6 混合专家（MoE）"
// §三), the router z-loss, the mean of the squared log-sum-exp of each token's logits (§六),
// and the coefficient of variation and max/mean ratio of the expert loads.
//
// Two deterministic passes (no floating-point atomics):
//   partial : a work-group of 4 waves takes 64 tokens, 16 per wave, one token at a time: the
//             wave holds the token's E logits (lane l: experts l, l+64, ...), reduces the max
//             and the sum of exponentials, and adds the token's probabilities into per-lane
//             column sums.  The four waves' sums are added in wave order into the block's
//             row of partial sums, and so are the squared log-sum-exps.
//   final   : one work-group adds the block rows in block order, divides by T, and computes
//             the load fractions and load statistics from the integer counts in float64.
#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// xor butterfly: every lane ends with the same value (each step adds the same two numbers)
__device__ __forceinline__ float wave_add(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ double wave_add_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

constexpr int kTokPerWave = 16;
constexpr int kTokPerBlock = 4 * kTokPerWave;

template <int NPL>
__global__ void __launch_bounds__(256) stats_partial_kernel(const float* __restrict__ logits,
                                                            int64_t T, int E, int scoring,
                                                            float* __restrict__ part,
                                                            float* __restrict__ zpart) {
  __shared__ float red[4][NPL * 64];
  __shared__ float zred[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerBlock + wave * kTokPerWave;
  float acc[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) acc[j] = 0.0f;
  float zacc = 0.0f;
  for (int i = 0; i < kTokPerWave; ++i) {
    const int64_t t = t0 + i;
    if (t >= T) break;
    const float* row = logits + t * E;
    float v[NPL];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? row[e] : -INFINITY;
      m = fmaxf(m, v[j]);
    }
    m = wave_max(m);
    float ex[NPL];
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      ex[j] = lane + 64 * j < E ? expf(v[j] - m) : 0.0f;
      s += ex[j];
    }
    s = wave_add(s);
    const float lse = m + logf(s);
    zacc += lse * lse;
    if (scoring == 0) {
#pragma unroll
      for (int j = 0; j < NPL; ++j) acc[j] += ex[j] / s;
    } else {
      float sg[NPL];
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        sg[j] = lane + 64 * j < E ? 1.0f / (1.0f + expf(-v[j])) : 0.0f;
        ss += sg[j];
      }
      ss = wave_add(ss);
#pragma unroll
      for (int j = 0; j < NPL; ++j) acc[j] += sg[j] / ss;
    }
  }
#pragma unroll
  for (int j = 0; j < NPL; ++j) red[wave][lane + 64 * j] = acc[j];
  if (lane == 0) zred[wave] = zacc;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    part[(int64_t)blockIdx.x * E + e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
  if (threadIdx.x == 0) zpart[blockIdx.x] = ((zred[0] + zred[1]) + zred[2]) + zred[3];
}

__global__ void __launch_bounds__(1024) stats_final_kernel(const float* __restrict__ part,
                                                           const float* __restrict__ zpart,
                                                           int nblk,
                                                           const int32_t* __restrict__ counts,
                                                           int64_t T, int E,
                                                           float* __restrict__ out) {
  __shared__ double dred[16];
  __shared__ long long ired[16], imax[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // load total and maximum
  long long tot = 0, mx = 0;
  for (int e = threadIdx.x; e < E; e += 1024) {
    const long long c = counts[e];
    tot += c;
    mx = c > mx ? c : mx;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    tot += __shfl_xor(tot, m, 64);
    const long long o = __shfl_xor(mx, m, 64);
    mx = o > mx ? o : mx;
  }
  if (lane == 0) {
    ired[wave] = tot;
    imax[wave] = mx;
  }
  __syncthreads();
  tot = 0;
  mx = 0;
  for (int w = 0; w < 16; ++w) {
    tot += ired[w];
    mx = imax[w] > mx ? imax[w] : mx;
  }
  const double mean = (double)tot / E;
  // per expert: P_e (block rows in block order), f_e; accumulate f·P and squared deviations
  double fp = 0.0, var = 0.0;
  for (int e = threadIdx.x; e < E; e += 1024) {
    float P = 0.0f;
    for (int b = 0; b < nblk; ++b) P += part[(int64_t)b * E + e];
    P = P / (float)T;
    const float f = tot > 0 ? (float)((double)counts[e] / (double)tot) : 0.0f;
    out[e] = f;
    out[E + e] = P;
    fp += (double)f * (double)P;
    const double d = (double)counts[e] - mean;
    var += d * d;
  }
  fp = wave_add_d(fp);
  var = wave_add_d(var);
  __syncthreads();  // ired/imax reads are done before dred is written
  if (lane == 0) dred[wave] = fp;
  __syncthreads();
  double sfp = 0.0;
  for (int w = 0; w < 16; ++w) sfp += dred[w];
  __syncthreads();
  if (lane == 0) dred[wave] = var;
  __syncthreads();
  if (threadIdx.x == 0) {
    double svar = 0.0;
    for (int w = 0; w < 16; ++w) svar += dred[w];
    double z = 0.0;
    for (int b = 0; b < nblk; ++b) z += (double)zpart[b];
    out[2 * E + 0] = (float)(E * sfp);
    out[2 * E + 1] = (float)(z / (double)T);
    out[2 * E + 2] = mean > 0 ? (float)(sqrt(svar / E) / mean) : 0.0f;
    out[2 * E + 3] = mean > 0 ? (float)((double)mx / mean) : 0.0f;
  }
}

}  // namespace

int64_t stats_blocks(int64_t T) { return (T + kTokPerBlock - 1) / kTokPerBlock; }

hipError_t launch_router_stats(const float* logits, const int32_t* counts, int64_t T, int E,
                               int scoring, float* part, float* zpart, float* out,
                               hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t nblk = stats_blocks(T);
  const dim3 g((unsigned)nblk), b(256);
  const int npl = (E + 63) / 64;
#define MOE_STATS_CASE(N)                                                                     \
  case N:                                                                                     \
    hipLaunchKernelGGL(stats_partial_kernel<N>, g, b, 0, stream, logits, T, E, scoring, part,  \
                       zpart);                                                                \
    break;
  switch (npl) {
    MOE_STATS_CASE(1)
    MOE_STATS_CASE(2)
    MOE_STATS_CASE(3)
    MOE_STATS_CASE(4)
    MOE_STATS_CASE(5)
    MOE_STATS_CASE(6)
    MOE_STATS_CASE(7)
    MOE_STATS_CASE(8)
    MOE_STATS_CASE(9)
    MOE_STATS_CASE(10)
    MOE_STATS_CASE(11)
    MOE_STATS_CASE(12)
    MOE_STATS_CASE(13)
    MOE_STATS_CASE(14)
    MOE_STATS_CASE(15)
    MOE_STATS_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_STATS_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(1024), 0, stream, part, zpart, (int)nblk,
                     counts, T, E, out);
  return hipGetLastError();
}

}  // namespace moe
