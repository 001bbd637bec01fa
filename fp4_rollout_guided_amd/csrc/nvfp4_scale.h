// Decoded NVFP4 block scales and the exact fast division of the libtrace
// kernels (gfx950): the decoded scale s = fl32(E4M3FN(byte) * ts) of a block
// with its reciprocals, and fl32(x / s) in four VALU operations, correctly
// rounded wherever the result can reach a rounding decision of the E2M1 grid.
// Used by the NVFP4 kernels (kernels.hip) and the diagnostics kernel
// (diag_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "fp4_block.h"

namespace trace_dev {

// Decoded block scale of one E4M3FN byte under tensor scale ts, with the
// reciprocals the fast division needs:
//   rhi = RN(1/s)                       (the Markstein correction step),
//   dhi = RD(1/s), dlo = RN((1 - s*dhi) * dhi) >= 0   (the first approximation;
//        both parts non-negative, so x*dhi + x*dlo carries the sign of x even
//        when x is a signed zero).
// 1 - s*dhi is exact because dhi is within one ulp of 1/s.  Scales outside
// [2^-96, 2^16] get dhi = NaN, so every quotient of the block is flagged and
// the exact fallback runs.  Zero-scale bytes get s = 1, rhi = dhi = dlo = 0,
// which maps every finite x to a zero of its own sign; rhi == 0 marks them.
struct alignas(16) ScaleEntry {
  float s, rhi, dhi, dlo;
};

__device__ __forceinline__ ScaleEntry make_scale_entry(uint32_t byte, float ts) {
  const float s = e4m3_decode(byte) * ts;
  if (s > 0.f && s <= 3.40282347e38f) {
    const float rhi = 1.0f / s;
    const float res = __builtin_fmaf(-s, rhi, 1.0f);  // exact: 1 - s*rhi
    const float dhi = res < 0.f ? __uint_as_float(__float_as_uint(rhi) - 1u) : rhi;
    const float dlo = __builtin_fmaf(-s, dhi, 1.0f) * dhi;
    const bool fast = (s >= 0x1p-96f) && (s <= 0x1p16f);
    return ScaleEntry{s, rhi, fast ? dhi : __uint_as_float(0x7fc00000u), dlo};
  }
  return ScaleEntry{1.f, 0.f, 0.f, 0.f};
}

// fl32(x / s).  q1 = RN(x*dhi + RN(x*dlo)) is within 0.5 ulp + 2^-23 ulp of
// x/s, hence faithful; r = s*q1 - x is then exact and RN(q1 - r*rhi) with
// rhi = RN(1/s) is the correctly rounded quotient (Markstein's theorem).
// This holds whenever the quotient can reach a rounding decision of the
// E2M1 grid (|x/s| >= 2^-3 with s >= 2^-96 puts x above 2^-99, where the
// remainder is representable).  Below that, a remainder that falls into the
// subnormal range perturbs q by at most 2^-150 / s, i.e. by a relative
// 2^-17 of |x/s| for every nonzero bf16 x when s <= 2^16: q keeps the sign
// of x, stays nonzero, and stays below every decision threshold.  A zero x
// gives a zero of the same sign.  NaN or infinite x, and quotients too large
// for binary32, make q1 NaN or infinite; the caller flags those.
template <bool kCheck>
__device__ __forceinline__ float div_fast(float x, const ScaleEntry& e, bool& bad) {
  const float q1 = __builtin_fmaf(x, e.dhi, x * e.dlo);
  if (kCheck) bad |= __builtin_amdgcn_class(q1, kBadClass);
  const float r = __builtin_fmaf(q1, e.s, -x);
  return __builtin_fmaf(-r, e.rhi, q1);
}

// The same with compile-time/uniform operands: fl32(a / d) for a >= 2^-100.
__device__ __forceinline__ float div_fast_u(float a, float d, float rhi, float rlo) {
  const float q1 = __builtin_fmaf(a, rhi, a * rlo);
  const float r = __builtin_fmaf(q1, d, -a);
  return __builtin_fmaf(-r, rhi, q1);
}

}  // namespace trace_dev
