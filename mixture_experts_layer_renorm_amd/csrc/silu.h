// SiLU for the fused gate/up epilogues: silu(z) = z * sigmoid(z) = z / (1 + e^-z).
// Built on the hardware base-2 exponential and reciprocal (about 1 ulp each): the result is
// rounded to the layer dtype right after, so full-precision expf and IEEE division would only
// add latency to the epilogue.  Limits: z -> -inf gives -0, z -> +inf gives z, NaN stays NaN.
#pragma once

namespace moe {

__device__ __forceinline__ float silu_fast(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);  // e^-z
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace moe
