// The activation of the expert-side epilogue, shared by the epilogue kernel
// and the first expert matmul's fused form ("UMDK/CAM communication
// acceleration library deep analysis v2", section 4.8.1, the GMM1 epilogue
// PerTokenDequantSwiGLU):
//   g = (float(cg) * wg) * ts,  u = (float(cu) * wu) * ts,  a = (g / (1 + e^-g)) * u
// each operation rounded on its own in binary32 (every file that includes
// this is compiled with floating-point contraction off).
//
// e^x: Cody and Waite's reduction (Software Manual for the Elementary
// Functions, 1980) with ln 2 = C1 + C2, C1 = 355/512, then the degree-7
// Taylor polynomial of e^r in Horner form, then the scale by 2^k, all in
// binary32.
#pragma once

#include "device_util.h"

#pragma clang fp contract(off)

namespace moe {

// Arguments are clamped to [-104, 89] first; the method itself then gives
// +inf at 89 (k = 128 and p > 1) and +0 at -104 (p 2^-150 is below half the
// smallest subnormal), which are the results for every argument beyond.
// p * 2^k is one v_ldexp_f32: exact for a normal result, rounded once for a
// subnormal one or overflowing to +inf, as the two-multiply form
// (p * 2^(k+64)) * 2^-64 or (p * 2^127) * 2 would be.  (A subnormal e^-g never
// changes the activation anyway: 1 + e^-g rounds to 1 for e^-g < 2^-24.)
// Arguments must not be NaN (finite scales and accumulators give none).
__device__ __forceinline__ float exp_cw(float x) {
  const float xc = __builtin_amdgcn_fmed3f(x, -104.0f, 89.0f);
  const float kf = __builtin_rintf(xc * 1.44269502162933349609375f);  // x log2(e)
  float r = xc - kf * 0.693359375f;     // C1 = 355/512: k * C1 is exact
  r = r - kf * -2.12194440e-4f;         // C2 = ln 2 - C1
  float p = 1.0f / 5040.0f;
  p = p * r + 1.0f / 720.0f;
  p = p * r + 1.0f / 120.0f;
  p = p * r + 1.0f / 24.0f;
  p = p * r + 1.0f / 6.0f;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  return __builtin_amdgcn_ldexpf(p, static_cast<int>(kf));
}

__device__ __forceinline__ float swiglu(int32_t cg, int32_t cu, float wg, float wu, float ts) {
  float g = static_cast<float>(cg) * wg;
  g = g * ts;
  float u = static_cast<float>(cu) * wu;
  u = u * ts;
  const float e = exp_cw(-g);
  const float d = e + 1.0f;
  const float y = g / d;
  return y * u;
}

}  // namespace moe
