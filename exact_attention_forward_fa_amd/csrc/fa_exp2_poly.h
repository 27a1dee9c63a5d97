// fa_exp2_poly.h -- 2^x on the FMA pipe instead of the transcendental unit.
//
// The polynomial replacement of the exponential that "Dissecting the SM_120
// Microarchitecture" lists first among the remedies for the softmax-bound
// FlashAttention tile (section 11.2, Fig. 12).  Cody-Waite split x = n + f
// with n = rint(x), f in [-1/2, 1/2]; 2^f by a degree-3 polynomial fitted here
// by iterated weighted least squares for relative error on [-1/2, 1/2] (max
// 7.5e-5, below the bf16 rounding of P); 2^n by ldexp.  x is clamped at -160,
// so a masked score (-inf) gives exactly 0; NaN propagates.
//
// Host and device: the kernels use it, and a CPU test checks its error bound
// against exp2 over the whole range the softmax feeds it.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

__host__ __device__ __forceinline__ float exp2_poly(float x) {
  x = __builtin_elementwise_maximum(x, -160.f);
  const float n = __builtin_rintf(x);
  const float f = x - n;
  float p = __builtin_fmaf(0.05517605319619179f, f, 0.24261149764060974f);
  p = __builtin_fmaf(p, f, 0.6932601928710938f);
  p = __builtin_fmaf(p, f, 0.9999280571937561f);
  return __builtin_ldexpf(p, (int)n);
}

}  // namespace fa
