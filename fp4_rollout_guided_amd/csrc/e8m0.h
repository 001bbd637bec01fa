// E8M0 block scales of the OCP Microscaling Formats (MX) v1.0 specification,
// shared by the MXFP4 (mx_kernels.hip) and MXFP8 (mx8_kernels.hip) kernels:
// byte b stands for 2^(b - 127), 0xFF is NaN.  A block's shared exponent is
// floor(log2(amax)) minus the exponent of the element format's largest
// normal, clamped to E8M0's range.  A lane owns one 16-element half of a
// 32-element block; lane pairs combine their halves' maxima (pair_swap, in
// fp4_block.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trace_dev {

constexpr uint32_t kE2M1Emax = 2;  // 6 = 1.5 * 2^2
constexpr uint32_t kE4M3Emax = 8;  // 448 = 1.75 * 2^8

// 2^(b - 127) for an E8M0 byte b in 0..254 (b = 0: the binary32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t b) { return __uint_as_float(b ? (b << 23) : 0x00400000u); }

// 2^(127 - b), exact for every b in 0..254 (b = 254: 2^-127).
__device__ __forceinline__ float e8m0_inverse(uint32_t b) {
  return __uint_as_float(b < 254u ? ((254u - b) << 23) : 0x00400000u);
}

// Scale byte of a block from its largest magnitude's bf16 bits (NaN
// excluded) for elements whose largest normal has exponent kEmax: the
// exponent field E gives floor(log2(amax)) = E - 127 for normal values; the
// byte 127 + clamp(E - 127 - kEmax, -127, 127) is then max(E, kEmax) - kEmax,
// which also covers zero and subnormal maxima (byte 0) and an infinite one
// (E = 255: byte 255 - kEmax).
template <uint32_t kEmax>
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  const uint32_t e = amax_bits >> 7;
  return (e < kEmax ? kEmax : e) - kEmax;
}

// Largest magnitude's bf16 bits over 16 elements, NaN excluded (a signed
// 16-bit maximum of m + 0x7f puts NaN halves below every other value).
__device__ __forceinline__ uint32_t half_amax_bits(const uint32_t (&w)[8]) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  s16x2_t best = {0, 0};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t m = (w[k] & 0x7fff7fffu) + 0x007f007fu;
    s16x2_t v;
    __builtin_memcpy(&v, &m, 4);
    best = __builtin_elementwise_max(best, v);
  }
  const int lo = best.x, hi = best.y;
  const int m = lo > hi ? lo : hi;
  return m > 0x7f ? (uint32_t)(m - 0x7f) : 0u;
}

}  // namespace trace_dev
