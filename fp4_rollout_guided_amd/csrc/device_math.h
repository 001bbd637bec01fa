// Device-side number-format helpers for the libtrace kernels (gfx950).
//
// Formats (NVFP4 as used by the rcap.io post "TRACE: Rollout-Guided
// Quantization-Aware Training for FP4"; the pages name the format, these are
// its parameters): bf16 activations, OCP E4M3FN block scales, IEEE fp32
// tensor scale, E2M1 codewords {0, .5, 1, 1.5, 2, 3, 4, 6} with sign.
//
// Every helper here is exact: it either performs one correctly rounded IEEE
// binary32 operation or an integer manipulation whose result is fixed by the
// format definitions.  The library is compiled with -ffp-contract=off and
// correctly rounded fp32 division, so `a / b` below is IEEE division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trace_dev {

constexpr int kBlock = 16;          // NVFP4 block length (elements)
constexpr float kTensorDiv = 2688.f; // 6 (E2M1 max) * 448 (E4M3FN max)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element j (0..15) of a block held as eight packed bf16 pairs.
__device__ __forceinline__ float block_elem(const uint32_t (&w)[8], int j) {
  return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
}

// bf16 round-to-nearest-even of a finite or infinite fp32 value.  Carrying
// into the exponent handles mantissa overflow, and values at or above the
// midpoint between the largest finite bf16 and 2^128 become infinity, as
// IEEE rounding requires.  NaN never reaches this helper.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP E4M3FN byte -> value.  Only 0x00..0x7E are scales; 0x7F (NaN) and the
// negative bytes make the block a zero-scale block, signalled by NaN.  The
// hardware conversion decodes the byte exactly (subnormals m * 2^-9, normals
// (1 + m/8) 2^(e-7)); a select replaces the other bytes, without a branch.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const float v = __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
  return b < 0x7fu ? v : __uint_as_float(0x7fc00000u);
}

// Non-negative fp32 (or NaN) -> E4M3FN byte, round to nearest even,
// saturating at 448 (0x7E); NaN -> 0.
__device__ __forceinline__ uint32_t e4m3_encode_sat(float v) {
  if (!(v < 448.f)) return (v >= 448.f) ? 0x7eu : 0u;
  if (v < 0x1p-6f) return (uint32_t)rintf(v * 512.f);  // subnormal grid m * 2^-9; 8 -> 0x08
  uint32_t u = __float_as_uint(v);
  u += 0x7ffffu + ((u >> 20) & 1u);                     // RNE to 3 mantissa bits
  const uint32_t code = (u >> 20) - (120u << 3);        // rebias exponent 127 -> 7
  return code < 0x7eu ? code : 0x7eu;
}

// E2M1 magnitude of index i in 0..7.
__device__ __forceinline__ float e2m1_mag(uint32_t i) {
  return i < 4 ? 0.5f * (float)i : (i < 6 ? (float)(i - 2) : (i == 6 ? 4.f : 6.f));
}

// Round-to-nearest-even index of a in [0, 6]: count the midpoints passed;
// at a midpoint the step is taken only toward an even index.
__device__ __forceinline__ uint32_t e2m1_rne_index(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.f);
}

// Index of the largest E2M1 magnitude <= a, a in [0, 6].
__device__ __forceinline__ uint32_t e2m1_floor_index(float a) {
  return (uint32_t)(a >= 0.5f) + (uint32_t)(a >= 1.f) + (uint32_t)(a >= 1.5f) +
         (uint32_t)(a >= 2.f) + (uint32_t)(a >= 3.f) + (uint32_t)(a >= 4.f) +
         (uint32_t)(a >= 6.f);
}

__device__ __forceinline__ bool is_nan_f(float f) { return !(f == f); }

}  // namespace trace_dev
