// libtrace MXFP8 kernels for gfx950: capture and the guided / RNE /
// full-information fake-quant forwards on the FP8 activation grid of the
// W4A8 setting (the rcap.io post's Ablations bullet: the method carries over
// to MXFP4 W4A8).  Format: the OCP Microscaling Formats (MX) v1.0 MXFP8 with
// E4M3 elements -- 32-element blocks, one E8M0 scale byte b per block
// standing for 2^(b - 127) (0xFF: a zero-scale block), shared exponent
// floor(log2(amax)) - 8, elements OCP E4M3FN bytes sign << 7 | magnitude
// code, magnitudes 0..448 increasing with the code.  The rule is the E2M1
// path's on this grid: z = clip(x / s, -448, 448); the cached bit is the
// magnitude code's last bit; the bracket endpoint with that parity is kept.
//
// Kernels (all grid-stride over 16-element halves of blocks):
//   mx8_capture_kernel       scale byte, parity bit-plane, optional codes
//   mx8_fakequant_kernel<M>  M = 0 RNE, 1 guided, 2 full information
//
// A lane owns one 16-element half (32 bytes of bf16 in, 16 bytes of codes,
// 2 bytes of bits or mask); lane pairs share a block's scale byte (one DPP
// move exchanges the halves' maxima).  The quotient by a power-of-two scale
// is a multiplication by its exact inverse, so x * 2^(127 - b) is the
// correctly rounded x / s.  Codes come from the hardware conversions:
// v_cvt_pk_fp8_f32 rounds to nearest even; v_cvt_sr_fp8_f32 with a zero
// random operand truncates, giving the floor code F of |z| and, on the
// predecessor of z toward zero, P: z is a codeword exactly when the two
// differ, and then they differ in their last bit (P = F - 1, or a NaN code
// with last bit 1 when z = +-0), so one bit per byte decides.  Four codes
// share a dword and the bracket choice runs on its byte lanes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "e8m0.h"
#include "fp4_block.h"
#include "launch.h"

namespace trace_dev {

constexpr uint32_t kLow = 0x01010101u;   // bit 0 of every byte
constexpr uint32_t kSign = 0x80808080u;  // bit 7 of every byte

// Quotients of one half under inverse scale inv; NaN quotients (a NaN
// element, or an infinity times the zero of a zero-scale block) become the
// zero the format gives them -- +0 for a NaN element, the element's signed
// zero otherwise -- and their elements are flagged in *nan_bits (a NaN
// element's mask bit is 0).
__device__ __forceinline__ void mx8_quotients(const uint32_t (&w)[8], float inv, float (&q)[16],
                                              uint32_t& nan_bits) {
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    q[j] = block_elem(w, j) * inv;
    bad |= __builtin_amdgcn_class(q[j], 0x003);  // signalling or quiet NaN
  }
  nan_bits = 0;
  if (bad) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float xv = block_elem(w, j);
      if (is_nan_f(q[j])) {
        q[j] = is_nan_f(xv) ? 0.f : copysignf(0.f, xv);
        nan_bits |= is_nan_f(xv) ? (1u << j) : 0u;
      }
    }
  }
}

// Clip-mask word: bit j set when |q_j| <= 448 (the sign bit of 448 - |q_j|
// is clear exactly then, infinities included).
__device__ __forceinline__ uint32_t mx8_keep_bits(const float (&q)[16]) {
  uint32_t clip = 0;
#pragma unroll
  for (int j = 15; j >= 0; --j) clip = __builtin_amdgcn_alignbit(clip, __float_as_uint(448.f - fabsf(q[j])), 31);
  return ~clip & 0xffffu;
}

// Round-to-nearest-even E4M3FN codes of the clipped quotients, dword k
// holding elements 4k..4k+3 (byte j = element 4k + j).
__device__ __forceinline__ void fp8_rne_codes(const float (&qc)[16], uint32_t (&C)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qc[4 * k], qc[4 * k + 1], 0, false);
    C[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qc[4 * k + 2], qc[4 * k + 3], (int)lo, true);
  }
}

// Toward-zero E4M3FN codes, same layout: the stochastic-rounding conversion
// with a zero random operand truncates.
__device__ __forceinline__ uint32_t fp8_rtz4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_sr_fp8_f32(a, 0, 0, 0);
  r = __builtin_amdgcn_cvt_sr_fp8_f32(b, 0, r, 1);
  r = __builtin_amdgcn_cvt_sr_fp8_f32(c, 0, r, 2);
  r = __builtin_amdgcn_cvt_sr_fp8_f32(d, 0, r, 3);
  return (uint32_t)r;
}

// Bit 0 of each of the 16 code bytes, gathered into a 16-bit word in
// element order.
__device__ __forceinline__ uint32_t fp8_parity_word(const uint32_t (&C)[4]) {
  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t t = C[k] & kLow;  // bits 0, 8, 16, 24
    t |= t >> 7;               // bits 0, 1 (and 16, 17)
    t |= t >> 14;              // bits 0..3
    word |= (t & 15u) << (4 * k);
  }
  return word;
}

// Cached bits 4k..4k+3 of a 16-bit word into bit 0 of the four bytes of a
// dword (the product places bit i at 8i; no two partial products meet).
__device__ __forceinline__ uint32_t fp8_spread4(uint32_t word, int k) {
  const uint32_t nib = (word >> (4 * k)) & 15u;
  return (nib * 0x00204081u) & kLow;
}

// Codes of q* for 16 quotients: RNE (kMode 0), guided by the cached bits
// (kMode 1; 16-bit word, bit j = element j) or full information (kMode 2;
// the rollout code bytes in roll, same layout as the output).
template <int kMode>
__device__ __forceinline__ void mx8_select_codes(const float (&qc)[16], uint32_t cached, uint4 roll,
                                                 uint32_t (&Q)[4]) {
  if (kMode == 0) {
    fp8_rne_codes(qc, Q);
    return;
  }
  const uint32_t R[4] = {roll.x, roll.y, roll.z, roll.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float pv[4];  // predecessors toward zero (a NaN for +-0)
#pragma unroll
    for (int j = 0; j < 4; ++j) pv[j] = __uint_as_float(__float_as_uint(qc[4 * k + j]) - 1u);
    const uint32_t F = fp8_rtz4(qc[4 * k], qc[4 * k + 1], qc[4 * k + 2], qc[4 * k + 3]);
    const uint32_t P = fp8_rtz4(pv[0], pv[1], pv[2], pv[3]);
    const uint32_t inside = ~(F ^ P) & kLow;  // bit 0 per byte: z strictly inside (F, F + 1)
    uint32_t up;
    if (kMode == 1) {
      up = (F ^ fp8_spread4(cached, k)) & inside;  // floor parity differs from the cached bit
    } else {
      // the upper endpoint is nearer the rollout codeword exactly when that
      // codeword has z's sign and a larger magnitude code (a NaN byte, 0x7F,
      // counts as beyond 448): (R | 0x80) - F_mag - 1 keeps bit 7 then
      const uint32_t gt = ((R[k] | kSign) - (F & ~kSign) - kLow) & kSign;
      const uint32_t same = ~(R[k] ^ F) & kSign;
      up = ((gt & same) >> 7) & inside;
    }
    Q[k] = F + up;  // magnitude code at most 0x7D below 448: no carry out of a byte
  }
}

// y for 16 codes: bf16_RNE(fl32(s * q)), 8 packed bf16 pairs.
__device__ __forceinline__ void fp8_decode_scaled(const uint32_t (&Q)[4], float s, uint32_t (&out)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)Q[k], false);  // elements 4k, 4k + 1
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)Q[k], true);   // elements 4k + 2, 4k + 3
    const bf16x2 p0 = __builtin_convertvector((f32x2){s * a.x, s * a.y}, bf16x2);
    const bf16x2 p1 = __builtin_convertvector((f32x2){s * b.x, s * b.y}, bf16x2);
    __builtin_memcpy(&out[2 * k], &p0, 4);
    __builtin_memcpy(&out[2 * k + 1], &p1, 4);
  }
}

// ---------------------------------------------------------------------------
// capture.  Lane pairs (h even, h + 1) hold one 32-element block; the even
// lane writes the scale byte.  The half count is even, so both lanes of a
// pair are always active together.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void mx8_capture_kernel(const uint4* __restrict__ x, uint64_t nhalves,
                                                               uint8_t* __restrict__ scales,
                                                               uint16_t* __restrict__ bits,
                                                               uint4* __restrict__ codes) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t h = (uint64_t)blockIdx.x * kThreads + threadIdx.x; h < nhalves; h += stride) {
    uint32_t w[8];
    load_block(x, h, w);
    const uint32_t a = half_amax_bits(w);
    const uint32_t b = pair_swap(a);
    const uint32_t sb = mx_scale_byte<kE4M3Emax>(a > b ? a : b);  // at most 247: always a valid scale
    float q[16];
    uint32_t nan_bits;
    mx8_quotients(w, e8m0_inverse(sb), q, nan_bits);
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = __builtin_amdgcn_fmed3f(q[j], -448.f, 448.f);
    uint32_t C[4];
    fp8_rne_codes(q, C);
    if ((h & 1) == 0) scales[h >> 1] = (uint8_t)sb;
    bits[h] = (uint16_t)fp8_parity_word(C);
    if (codes) codes[h] = make_uint4(C[0], C[1], C[2], C[3]);
  }
}

// ---------------------------------------------------------------------------
// fake-quant forward; kMode: 0 = RNE, 1 = guided, 2 = full information.
// ---------------------------------------------------------------------------
template <int kMode>
__global__ __launch_bounds__(kThreads) void mx8_fakequant_kernel(const uint4* __restrict__ x, uint64_t nhalves,
                                                                 const uint8_t* __restrict__ scales,
                                                                 const uint16_t* __restrict__ bits,
                                                                 const uint4* __restrict__ rcodes,
                                                                 uint4* __restrict__ y, uint16_t* __restrict__ mask,
                                                                 uint4* __restrict__ qcodes) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t h = (uint64_t)blockIdx.x * kThreads + threadIdx.x; h < nhalves; h += stride) {
    const uint32_t sbyte = scales[h >> 1];
    const uint32_t cached = kMode == 1 ? (uint32_t)bits[h] : 0u;
    const uint4 roll = kMode == 2 ? rcodes[h] : make_uint4(0u, 0u, 0u, 0u);
    uint32_t w[8];
    load_block(x, h, w);
    // a NaN scale byte makes a zero-scale block: multiplying by 0 maps every
    // finite x to a zero of its own sign, decoded with s = 1
    const bool valid = sbyte != 0xffu;
    const float inv = valid ? e8m0_inverse(sbyte) : 0.f;
    const float s = valid ? e8m0_value(sbyte) : 1.f;
    float q[16];
    uint32_t nan_bits;
    mx8_quotients(w, inv, q, nan_bits);
    const uint32_t keep = mx8_keep_bits(q) & ~nan_bits;
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = __builtin_amdgcn_fmed3f(q[j], -448.f, 448.f);
    uint32_t Q[4];
    mx8_select_codes<kMode>(q, cached, roll, Q);
    uint32_t out[8];
    fp8_decode_scaled(Q, s, out);
    store_block(y, h, out);
    mask[h] = (uint16_t)(valid ? keep : 0u);
    if (qcodes) qcodes[h] = make_uint4(Q[0], Q[1], Q[2], Q[3]);
  }
}

}  // namespace trace_dev

namespace trace_host {

using namespace trace_dev;

static unsigned mx8_grid(uint64_t nhalves) {
  const uint64_t g = (nhalves + kThreads - 1) / kThreads;
  return (unsigned)(g < kMaxGroups ? g : kMaxGroups);
}

hipError_t launch_mx8_capture(const uint16_t* x, uint64_t nblocks, uint8_t* scales, uint8_t* bits, uint8_t* codes,
                              hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const uint64_t nhalves = 2 * nblocks;
  hipLaunchKernelGGL(mx8_capture_kernel, dim3(mx8_grid(nhalves)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(x), nhalves, scales, reinterpret_cast<uint16_t*>(bits),
                     reinterpret_cast<uint4*>(codes));
  return hipGetLastError();
}

hipError_t launch_mx8_fakequant(int mode, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                                const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                                hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const uint64_t nhalves = 2 * nblocks;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint4* yv = reinterpret_cast<uint4*>(y);
  uint16_t* mv = reinterpret_cast<uint16_t*>(mask);
  uint4* qv = reinterpret_cast<uint4*>(qcodes);
  const dim3 grid(mx8_grid(nhalves)), block(kThreads);
  if (mode == 1)
    hipLaunchKernelGGL(mx8_fakequant_kernel<1>, grid, block, 0, stream, xv, nhalves, scales,
                       reinterpret_cast<const uint16_t*>(side), static_cast<const uint4*>(nullptr), yv, mv, qv);
  else if (mode == 2)
    hipLaunchKernelGGL(mx8_fakequant_kernel<2>, grid, block, 0, stream, xv, nhalves, scales,
                       static_cast<const uint16_t*>(nullptr), reinterpret_cast<const uint4*>(side), yv, mv, qv);
  else
    hipLaunchKernelGGL(mx8_fakequant_kernel<0>, grid, block, 0, stream, xv, nhalves, scales,
                       static_cast<const uint16_t*>(nullptr), static_cast<const uint4*>(nullptr), yv, mv, qv);
  return hipGetLastError();
}

}  // namespace trace_host
