// libtrace MXFP4 kernels for gfx950: capture and the guided / RNE /
// full-information fake-quant forwards on MXFP4 scales (the rcap.io post's
// Ablations bullet: the method carries over to MXFP4).  MXFP4 parameters
// from the OCP Microscaling Formats (MX) v1.0 specification: 32-element
// blocks, one E8M0 scale byte b per block standing for 2^(b - 127) (0xFF is
// NaN), E2M1 elements.  The block scale is 2^(floor(log2(amax)) - 2) clamped
// to E8M0's range; elements are rounded as on the NVFP4 path.
//
// One lane owns one 32-element block: 64 contiguous bytes of bf16 (four
// 128-bit loads), its scale byte, one 32-bit word of every bit-plane and 16
// bytes of codes; the block is processed as two 16-element halves with the
// machinery of fp4_block.h.  Dividing by a power of two is a multiplication
// by its exact inverse: x * 2^(127 - b) is the correctly rounded x / s, also
// where it underflows, so there is no division at all.  Blocks holding a NaN
// or an infinity, or whose quotients overflow, run the exact per-element
// fallback.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "fp4_block.h"
#include "launch.h"

namespace trace_dev {

// 2^(b - 127) for an E8M0 byte b in 0..254 (b = 0: the binary32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t b) { return __uint_as_float(b ? (b << 23) : 0x00400000u); }

// 2^(127 - b), exact for every b in 0..254 (b = 254: 2^-127).
__device__ __forceinline__ float e8m0_inverse(uint32_t b) {
  return __uint_as_float(b < 254u ? ((254u - b) << 23) : 0x00400000u);
}

// Scale byte of a block from its largest magnitude's bf16 bits (NaN
// excluded): the exponent field E gives floor(log2(amax)) = E - 127 for
// normal values; the byte 127 + clamp(E - 127 - 2, -127, 127) is then
// max(E, 2) - 2, which also covers zero and subnormal maxima (byte 0) and an
// infinite one (E = 255: byte 253).
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  const uint32_t e = amax_bits >> 7;
  return (e < 2u ? 2u : e) - 2u;
}

__device__ __forceinline__ void load_mx_block(const uint4* __restrict__ x, uint64_t b, uint32_t (&wa)[8],
                                              uint32_t (&wb)[8]) {
  load_block(x, 2 * b, wa);
  load_block(x, 2 * b + 1, wb);
}

// Largest magnitude's bf16 bits over 32 elements, NaN excluded (a signed
// 16-bit maximum of m + 0x7f puts NaN halves below every other value).
__device__ __forceinline__ uint32_t mx_amax_bits(const uint32_t (&wa)[8], const uint32_t (&wb)[8]) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  s16x2_t best = {0, 0};
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t m = ((k < 8 ? wa[k] : wb[k - 8]) & 0x7fff7fffu) + 0x007f007fu;
    s16x2_t v;
    __builtin_memcpy(&v, &m, 4);
    best = __builtin_elementwise_max(best, v);
  }
  const int lo = best.x, hi = best.y;
  const int m = lo > hi ? lo : hi;
  return m > 0x7f ? (uint32_t)(m - 0x7f) : 0u;
}

// ---------------------------------------------------------------------------
// exact fallbacks (IEEE division, one element at a time)
// ---------------------------------------------------------------------------
__device__ __noinline__ void mx_capture_block_exact(const uint4* __restrict__ x4, uint64_t b,
                                                    uint8_t* __restrict__ scales, uint32_t* __restrict__ bits,
                                                    uint4* __restrict__ codes) {
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 32 * b;
  uint32_t amax_bits = 0;
#pragma unroll 1
  for (int j = 0; j < 32; ++j) {
    const uint32_t m = x[j] & 0x7fffu;
    if (m <= 0x7f80u && m > amax_bits) amax_bits = m;  // NaN (m > 0x7f80) ignored
  }
  const uint32_t sb = mx_scale_byte(amax_bits);
  const float s = e8m0_value(sb);
  uint32_t bitword = 0;
  uint32_t cw[4] = {0, 0, 0, 0};
#pragma unroll 1
  for (int j = 0; j < 32; ++j) {
    const uint32_t code = exact_capture_code(__uint_as_float((uint32_t)x[j] << 16), s, true);
    bitword |= (code & 1u) << j;
    cw[j >> 3] |= code << (4 * (j & 7));
  }
  scales[b] = (uint8_t)sb;
  bits[b] = bitword;
  if (codes) codes[b] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
}

__device__ __noinline__ void mx_fakequant_block_exact(int mode, const uint4* __restrict__ x4, uint64_t b,
                                                      uint32_t sbyte, uint32_t cached, uint4 roll,
                                                      uint4* __restrict__ y4, uint32_t* __restrict__ mask,
                                                      uint4* __restrict__ qcodes) {
  const bool valid = sbyte != 0xffu;
  const float s = valid ? e8m0_value(sbyte) : 1.f;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 32 * b;
  uint16_t* y = reinterpret_cast<uint16_t*>(y4) + 32 * b;
  const uint32_t rw[4] = {roll.x, roll.y, roll.z, roll.w};
  uint32_t maskword = 0;
  uint32_t cw[4] = {0, 0, 0, 0};
#pragma unroll 1
  for (int j = 0; j < 32; ++j) {
    const uint32_t rc = (rw[j >> 3] >> (4 * (j & 7))) & 15u;
    uint32_t code, mk, ybits;
    exact_forward_element(mode, __uint_as_float((uint32_t)x[j] << 16), s, valid, (cached >> j) & 1u, rc, code, mk,
                          ybits);
    maskword |= mk << j;
    y[j] = (uint16_t)ybits;
    cw[j >> 3] |= code << (4 * (j & 7));
  }
  mask[b] = maskword;
  if (qcodes) qcodes[b] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
}

// ---------------------------------------------------------------------------
// capture
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void mx_capture_kernel(const uint4* __restrict__ x, uint64_t nblocks,
                                                              uint8_t* __restrict__ scales,
                                                              uint32_t* __restrict__ bits,
                                                              uint4* __restrict__ codes) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += stride) {
    uint32_t wa[8], wb[8];
    load_mx_block(x, b, wa, wb);
    const uint32_t sb = mx_scale_byte(mx_amax_bits(wa, wb));
    const float inv = e8m0_inverse(sb);
    bool bad = false;
    float q[16];
    uint32_t E0 = 0, O0 = 0, E1 = 0, O1 = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      q[j] = block_elem(wa, j) * inv;
      bad |= __builtin_amdgcn_class(q[j], kBadClass);
    }
    FP4_PACK8(FP4_RNE, E0, q, 0);
    FP4_PACK8(FP4_RNE, O0, q, 1);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      q[j] = block_elem(wb, j) * inv;
      bad |= __builtin_amdgcn_class(q[j], kBadClass);
    }
    FP4_PACK8(FP4_RNE, E1, q, 0);
    FP4_PACK8(FP4_RNE, O1, q, 1);
    if (bad) {
      mx_capture_block_exact(x, b, scales, bits, codes);
    } else {
      scales[b] = (uint8_t)sb;
      bits[b] = gather_parity(E0, O0) | (gather_parity(E1, O1) << 16);
      if (codes) {
        uint32_t c0, c1, c2, c3;
        interleave_codes(E0, O0, c0, c1);
        interleave_codes(E1, O1, c2, c3);
        codes[b] = make_uint4(c0, c1, c2, c3);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fake-quant forward; kMode: 0 = RNE, 1 = guided, 2 = full information
// ---------------------------------------------------------------------------
template <int kMode>
__global__ __launch_bounds__(kThreads) void mx_fakequant_kernel(const uint4* __restrict__ x, uint64_t nblocks,
                                                                const uint8_t* __restrict__ scales,
                                                                const uint32_t* __restrict__ bits,
                                                                const uint4* __restrict__ rcodes,
                                                                uint4* __restrict__ y, uint32_t* __restrict__ mask,
                                                                uint4* __restrict__ qcodes) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += stride) {
    const uint32_t sbyte = scales[b];
    const uint32_t cached = kMode == 1 ? bits[b] : 0u;
    const uint4 roll = kMode == 2 ? rcodes[b] : make_uint4(0u, 0u, 0u, 0u);
    uint32_t wa[8], wb[8];
    load_mx_block(x, b, wa, wb);
    // a NaN scale byte makes a zero-scale block: multiplying by 0 maps every
    // finite x to a zero of its own sign, decoded with s = 1
    const bool valid = sbyte != 0xffu;
    const float inv = valid ? e8m0_inverse(sbyte) : 0.f;
    const float s = valid ? e8m0_value(sbyte) : 1.f;
    bool bad = false;
    float q[16];
    uint32_t QE0, QO0, QE1, QO1;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      q[j] = block_elem(wa, j) * inv;
      bad |= __builtin_amdgcn_class(q[j], kBadClass);
    }
    const uint32_t keep0 = select_codes<kMode>(q, cached & 0xffffu, make_uint2(roll.x, roll.y), QE0, QO0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      q[j] = block_elem(wb, j) * inv;
      bad |= __builtin_amdgcn_class(q[j], kBadClass);
    }
    const uint32_t keep1 = select_codes<kMode>(q, cached >> 16, make_uint2(roll.z, roll.w), QE1, QO1);
    if (bad) {
      mx_fakequant_block_exact(kMode, x, b, sbyte, cached, roll, y, mask, qcodes);
    } else {
      uint32_t out[8];
      decode_block(QE0, QO0, s, out);
      store_block(y, 2 * b, out);
      decode_block(QE1, QO1, s, out);
      store_block(y, 2 * b + 1, out);
      mask[b] = valid ? (keep0 | (keep1 << 16)) : 0u;
      if (qcodes) {
        uint32_t c0, c1, c2, c3;
        interleave_codes(QE0, QO0, c0, c1);
        interleave_codes(QE1, QO1, c2, c3);
        qcodes[b] = make_uint4(c0, c1, c2, c3);
      }
    }
  }
}

}  // namespace trace_dev

namespace trace_host {

using namespace trace_dev;

static unsigned mx_grid(uint64_t nblocks) {
  const uint64_t g = (nblocks + kThreads - 1) / kThreads;
  return (unsigned)(g < kMaxGroups ? g : kMaxGroups);
}

hipError_t launch_mx_capture(const uint16_t* x, uint64_t nblocks, uint8_t* scales, uint8_t* bits, uint8_t* codes,
                             hipStream_t stream) {
  hipLaunchKernelGGL(mx_capture_kernel, dim3(mx_grid(nblocks)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(x), nblocks, scales, reinterpret_cast<uint32_t*>(bits),
                     reinterpret_cast<uint4*>(codes));
  return hipGetLastError();
}

hipError_t launch_mx_fakequant(int mode, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                               const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                               hipStream_t stream) {
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint4* yv = reinterpret_cast<uint4*>(y);
  uint32_t* mv = reinterpret_cast<uint32_t*>(mask);
  uint4* qv = reinterpret_cast<uint4*>(qcodes);
  const dim3 grid(mx_grid(nblocks)), block(kThreads);
  if (mode == 1)
    hipLaunchKernelGGL(mx_fakequant_kernel<1>, grid, block, 0, stream, xv, nblocks, scales,
                       reinterpret_cast<const uint32_t*>(side), static_cast<const uint4*>(nullptr), yv, mv, qv);
  else if (mode == 2)
    hipLaunchKernelGGL(mx_fakequant_kernel<2>, grid, block, 0, stream, xv, nblocks, scales,
                       static_cast<const uint32_t*>(nullptr), reinterpret_cast<const uint4*>(side), yv, mv, qv);
  else
    hipLaunchKernelGGL(mx_fakequant_kernel<0>, grid, block, 0, stream, xv, nblocks, scales,
                       static_cast<const uint32_t*>(nullptr), static_cast<const uint4*>(nullptr), yv, mv, qv);
  return hipGetLastError();
}

}  // namespace trace_host
