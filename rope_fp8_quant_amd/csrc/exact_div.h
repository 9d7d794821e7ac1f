// Correctly rounded m / 448 and 1 / s for the gfx950 kernels, without the
// compiler's general divide expansion (about ten instructions each):
//  * 448 = 7 * 2^6, and m / 448 stays an fp32 normal for every m >= 2^-116,
//    so RN(m / 448) = RN(m / 7) * 2^-6 exactly.  RN(m / 7) is the product by
//    RN(1/7) corrected once by its FMA remainder (the division-by-a-constant
//    form of the Markstein correction step).
//  * RN(1 / s) is v_rcp_f32's estimate after one Newton-Raphson step with an
//    FMA residual, for positive normal s below 2^126.
// Both hold for every input in those domains: tests/exact checks every
// positive normal fp32 on the host (the first) and on the GPU (both).
// Neither form is used for an amax that overflowed to +inf: the callers
// take the IEEE results there directly (inf / 448 = inf, 1 / inf = 0).
#ifndef ROPEQUANT_EXACT_DIV_H
#define ROPEQUANT_EXACT_DIV_H

__device__ __forceinline__ float div448(float m) {
  constexpr float kInv7 = 1.0f / 7.0f;
  const float q0 = m * kInv7;
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, 7.0f, m), kInv7, q0);
  return q * 0x1p-6f;
}

__device__ __forceinline__ float recip_scale(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  return __builtin_fmaf(y0, __builtin_fmaf(-s, y0, 1.0f), y0);
}

#endif  // ROPEQUANT_EXACT_DIV_H
