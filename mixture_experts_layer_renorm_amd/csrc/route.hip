// Router scoring, top-K selection and renormalisation ("MoE" §2 Router; "1.6 混合专家（MoE）"
// §二 Top-k 门控公式 steps 2-3).
//
// One wave64 per token.  Lane l holds logits l, l+64, ... as 32-bit keys, the
// order-preserving image of the fp32 logit (NaN mapped to -inf's key, -0.0 to +0.0's).  Each
// of K rounds takes the wave's largest key with a DPP max and then, with one ballot per held
// slot, the lowest expert id among the lanes holding it, so experts are selected in descending
// order with ties going to the lower id; the winner's key is cleared to 0, below every real
// key (padding slots past E hold 0 from the start).
//
// Selection compares logits, not probabilities: softmax and sigmoid are strictly increasing,
// so the top-K set is the same, and the choice does not depend on exp/sigmoid rounding.
// Softmax weights use only the K selected logits: the full-E denominator cancels in
// p_e / sum_{j in I} p_j, leaving exp(r_e - r_max) / sum_{j in I} exp(r_j - r_max).
#include <type_traits>

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

// One DPP step of a 32-bit wave max: v and the lane's DPP partner's value.  Lanes in rows
// outside ROW_MASK read 0, the identity of an unsigned max, so they keep their own value (and
// the move folds into a v_max_u32 with a DPP operand).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t max_dpp_u32(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
  return o > v ? o : v;
}

// Maximum over the wave, returned uniformly: DPP steps within quads (lane ^ 1, lane ^ 2), within
// rows of 16 (half-mirror, mirror), then row 0's and 1's maxima carried into rows 1 and 3 and
// row 1's into rows 2 and 3 (row broadcasts), leaving the wave's maximum in lane 63.  A max
// does not depend on the order of its operands, so this is exact.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_dpp_u32<0xB1, 0xf>(v);   // quad_perm [1, 0, 3, 2]
  v = max_dpp_u32<0x4E, 0xf>(v);   // quad_perm [2, 3, 0, 1]
  v = max_dpp_u32<0x141, 0xf>(v);  // row_half_mirror
  v = max_dpp_u32<0x140, 0xf>(v);  // row_mirror
  v = max_dpp_u32<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = max_dpp_u32<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

constexpr int kMaxSlices = 8;  // router K slices summed by the top-K kernel

// NPL: logits held per lane, ceil(E / 64); KSM: slices loaded per logit, a.ks rounded up to a
// power of two (the routers' slice counts are powers of two, so no slice is loaded twice)
template <int NPL, int KSM>
__global__ void __launch_bounds__(256) topk_kernel(const TopkArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int E = a.E, K = a.K;

  // logit e = the router's partial sums over K slices, added in slice order
  uint32_t key[NPL];
  float val[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    float v = 0.0f;
    if (e < E) {
      // all slices are loaded before the first add (clamped, always valid indices)
      const float* p0 = a.src + t * a.ld + e;
      float u[KSM];
#pragma unroll
      for (int q = 0; q < KSM; ++q) u[q] = p0[(q < a.ks ? q : a.ks - 1) * a.slice_stride];
      v = u[0];
#pragma unroll
      for (int q = 1; q < KSM; ++q)
        if (q < a.ks) v += u[q];
      if (a.logits_out) a.logits_out[t * E + e] = v;
    }
    val[j] = v;
    key[j] = e < E ? order_key(v) : 0u;  // 0: below every real key (-inf's is 0x007FFFFF)
    if (a.keys_out && !a.sel_bias && e < E) a.keys_out[t * E + e] = v;
  }

  // Selection-only bias: the key becomes score + bias (score = softmax probability over all
  // E experts, or the sigmoid affinity); the weights below use the unbiased score.
  float sc[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) sc[j] = 0.0f;
  if (a.sel_bias) {
    if (a.scoring == 0) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (lane + 64 * j < E) m = fmaxf(m, val[j]);
      m = wave_max_f(m);
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (lane + 64 * j < E) part += expf(val[j] - m);
      const float sum = wave_sum(part);
#pragma unroll
      for (int j = 0; j < NPL; ++j) sc[j] = expf(val[j] - m) / sum;
    } else {
#pragma unroll
      for (int j = 0; j < NPL; ++j) sc[j] = 1.0f / (1.0f + expf(-val[j]));
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      if (e < E) {
        const float kv = sc[j] + a.sel_bias[e];
        key[j] = order_key(kv);
        if (a.keys_out) a.keys_out[t * E + e] = kv;
      }
    }
  }

  // Slot k (k < K <= 64) is kept by lane k: its logit (or, with a bias, its score) and id.
  float top = 0.0f, my_val = 0.0f;
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t best = key[0];
#pragma unroll
    for (int j = 1; j < NPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u32(best);
    // the lowest id holding the best key: the first slot with a hit, its lowest lane
    int slot = 0;
    unsigned long long hit = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      if (hit == 0) {
        hit = __ballot(key[j] == best);
        slot = j;
      }
    }
    const int owner = __builtin_ctzll(hit);
    const uint32_t e = (uint32_t)(64 * slot + owner);
    const float v = key_value(best);
    if (k == 0) top = v;
    if (lane == owner) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (j == slot) key[j] = 0u;
    }
    float mv = v;
    if (a.sel_bias) {  // the selected expert's unbiased score, from the lane that holds it
      float own = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (j == slot) own = sc[j];
      mv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, own), owner));
    }
    if (lane == k) {
      my_val = mv;
      my_id = (int)e;
    }
  }

  float s = 0.0f, denom = 1.0f;
  if (a.sel_bias) {
    if (lane < K) s = my_val;  // the slot's unbiased score
    if (a.renorm) denom = wave_sum(s);
  } else {
    if (lane < K) s = a.scoring == 0 ? expf(my_val - top) : 1.0f / (1.0f + expf(-my_val));
    if (a.renorm) {
      denom = wave_sum(s);
    } else if (a.scoring == 0) {
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (lane + 64 * j < E) part += expf(val[j] - top);
      denom = wave_sum(part);
    }
  }
  if (lane < K) {
    a.idx[t * K + lane] = my_id;
    a.w[t * K + lane] = s / denom;
  }
  if (a.gate_out) {
    float g;
    if (a.gate_x) {
      // gate logit x[t] . w_s: lane l takes elements 8 l + 512 c, c = 0, 1, ...; each lane's
      // products in order, then a butterfly over the wave (a fixed order, so deterministic)
      typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
      const __bf16* xr = a.gate_x + t * a.D;
      float part = 0.0f;
      for (int d = 8 * lane; d < a.D; d += 512) {
        const bf16x8 xv = *(const bf16x8*)(xr + d);
        const bf16x8 wv = *(const bf16x8*)(a.gate_w + d);
#pragma unroll
        for (int i = 0; i < 8; ++i) part = __builtin_fmaf((float)xv[i], (float)wv[i], part);
      }
      g = wave_sum(part);
    } else {
      g = a.gate_src[t * a.gate_ld];
      for (int q = 1; q < a.ks; ++q) g += a.gate_src[q * a.gate_slice_stride + t * a.gate_ld];
    }
    if (lane == 0) a.gate_out[t] = 1.0f / (1.0f + expf(-g));
  }
}

// Router logits for bf16 operands, one K slice per blockIdx.z:
//   part[z][t][n] = sum over k in slice z of x[t, k] * W[n, k]  (+ bias[n] in slice 0)
// where W rows [0, E) are the router and row E (if gated) is the shared-expert gate vector.
// A work-group computes 16 tokens x 64 columns; its 4 waves take every fourth 32-wide K step
// of the slice and their sums are added in wave order through LDS.  Operands are read straight
// from global memory into registers in the MFMA operand layout (lane l: row l % 16,
// k = 8 (l / 16) .. +7 of a step).  Rows past T and columns past NE are computed on clamped,
// valid rows and not stored.  Built for small token counts, where the latency of a long K
// loop on few work-groups would dominate.
__global__ void __launch_bounds__(256) router_kernel(const __bf16* __restrict__ x,
                                                     const __bf16* __restrict__ wr,
                                                     const __bf16* __restrict__ wg,
                                                     const float* __restrict__ bias, int64_t T,
                                                     int D, int E, int NE, int kslice,
                                                     float* __restrict__ part) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ f32x4 red[3][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  const int64_t tok0 = (int64_t)blockIdx.x * 16;
  const int col0 = blockIdx.y * 64;
  const int z = blockIdx.z;
  const int64_t k0 = (int64_t)z * kslice + wave * 32 + lk * 8;
  const int64_t trow = tok0 + lr < T ? tok0 + lr : T - 1;
  const __bf16* ap = x + trow * D + k0;
  const __bf16* bp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = col0 + 16 * j + lr;
    bp[j] = (n < E ? wr + (int64_t)n * D : (n == E && wg) ? wg : wr) + k0;
  }
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int kw = kslice - wave * 32;  // this wave's steps: k = 0, 128, ... < kw
#pragma unroll 4
  for (int k = 0; k < kw; k += 128) {
    const bf16x8 av = *(const bf16x8*)(ap + k);
    bf16x8 bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = *(const bf16x8*)(bp[j] + k);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[j], acc[j], 0, 0, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wave - 1][j][lane] = acc[j];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += red[w][j][lane];
  // lane holds rows 4 (l / 16) + r, column l % 16 of each 16 x 16 sub-tile
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = col0 + 16 * j + lr;
    if (n >= NE) continue;
    const float b = (z == 0 && bias && n < E) ? bias[n] : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = tok0 + lk * 4 + r;
      if (t < T) part[((int64_t)z * T + t) * NE + n] = acc[j][r] + b;
    }
  }
}

// Selection-bias feedback: one work-group; the load total in 64-bit integers, then one fp32
// add per expert.
__global__ void __launch_bounds__(1024) update_bias_kernel(const int32_t* __restrict__ counts,
                                                           int E, float* __restrict__ bias,
                                                           float gamma) {
  __shared__ long long part[16];
  long long sum = 0;
  for (int e = threadIdx.x; e < E; e += 1024) sum += counts[e];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sum;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < 16; ++w) total += part[w];
  for (int e = threadIdx.x; e < E; e += 1024) {
    const long long d = (long long)counts[e] * E - total;
    if (d > 0) bias[e] = bias[e] - gamma;
    else if (d < 0) bias[e] = bias[e] + gamma;
  }
}

}  // namespace

hipError_t launch_update_select_bias(const int32_t* counts, int E, float* bias, float gamma,
                                     hipStream_t stream) {
  hipLaunchKernelGGL(update_bias_kernel, dim3(1), dim3(1024), 0, stream, counts, E, bias, gamma);
  return hipGetLastError();
}

int router_kslices(int64_t T, int D, int E, int gated) {
  const int64_t blocks = ((T + 15) / 16) * ((E + gated + 63) / 64);
  int ks = 1;
  // split K until about 256 work-groups run, keeping slices at least 256 wide
  while (ks * 2 <= kMaxSlices && blocks * ks * 2 <= 256 && D % (ks * 2 * 32) == 0 &&
         D / (ks * 2) >= 256)
    ks *= 2;
  return ks;
}

hipError_t launch_router_bf16(const void* x, const void* w_router, const void* w_gate,
                              const float* bias, int64_t T, int D, int E, int ks, float* part,
                              hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int NE = E + (w_gate ? 1 : 0);
  const dim3 g((unsigned)((T + 15) / 16), (unsigned)((NE + 63) / 64), (unsigned)ks), b(256);
  hipLaunchKernelGGL(router_kernel, g, b, 0, stream, (const __bf16*)x, (const __bf16*)w_router,
                     (const __bf16*)w_gate, bias, T, D, E, NE, D / ks, part);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  if (a.ks < 1 || a.ks > kMaxSlices) return hipErrorInvalidValue;
  dim3 g((unsigned)((a.T + 3) / 4)), b(256);
  const int npl = (a.E + 63) / 64;
  if (npl < 1 || npl > 16) return hipErrorInvalidValue;
  const auto go = [&](auto n) {
    constexpr int N = decltype(n)::value;
    if (a.ks == 1)
      hipLaunchKernelGGL((topk_kernel<N, 1>), g, b, 0, stream, a);
    else if (a.ks == 2)
      hipLaunchKernelGGL((topk_kernel<N, 2>), g, b, 0, stream, a);
    else if (a.ks <= 4)
      hipLaunchKernelGGL((topk_kernel<N, 4>), g, b, 0, stream, a);
    else
      hipLaunchKernelGGL((topk_kernel<N, 8>), g, b, 0, stream, a);
  };
  switch (npl) {
#define MOE_TOPK_CASE(N) \
  case N:                \
    go(std::integral_constant<int, N>{}); \
    break;
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
#undef MOE_TOPK_CASE
  }
  return hipGetLastError();
}

}  // namespace moe
