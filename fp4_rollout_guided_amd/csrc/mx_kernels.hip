// libtrace MXFP4 kernels for gfx950: capture and the guided / RNE /
// full-information fake-quant forwards on MXFP4 scales (the rcap.io post's
// Ablations bullet: the method carries over to MXFP4).  MXFP4 parameters
// from the OCP Microscaling Formats (MX) v1.0 specification: 32-element
// blocks, one E8M0 scale byte b per block standing for 2^(b - 127) (0xFF is
// NaN), E2M1 elements.  The block scale is 2^(floor(log2(amax)) - 2) clamped
// to E8M0's range; elements are rounded as on the NVFP4 path.
//
// A lane owns one 16-element half of a block -- the same 32 contiguous bytes
// of bf16, 16-bit bit-plane words and 8 bytes of codes as on the NVFP4 path
// -- and lane pairs share a block's scale: the pair exchanges its halves'
// maxima with one DPP move.  (A lane per 32-element block was measured ~15%
// slower: its 64-byte stride doubles the cache lines each load instruction
// touches.)  Dividing by a power of two is a multiplication
// by its exact inverse: x * 2^(127 - b) is the correctly rounded x / s, also
// where it underflows, so there is no division at all.  Blocks holding a NaN
// or an infinity, or whose quotients overflow, run the exact per-element
// fallback.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "e8m0.h"
#include "fp4_block.h"
#include "launch.h"

namespace trace_dev {

// ---------------------------------------------------------------------------
// exact fallbacks (IEEE division, one element at a time) for one lane's
// 16-element half of a block whose scale byte is already known
// ---------------------------------------------------------------------------
__device__ __noinline__ void mx_capture_half_exact(const uint4* __restrict__ x4, uint64_t h, uint32_t sb,
                                                   uint16_t* __restrict__ bits, uint2* __restrict__ codes) {
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 16 * h;
  const float s = e8m0_value(sb);
  uint32_t bitword = 0;
  uint64_t cw = 0;
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    const uint32_t code = exact_capture_code(__uint_as_float((uint32_t)x[j] << 16), s, true);
    bitword |= (code & 1u) << j;
    cw |= (uint64_t)code << (4 * j);
  }
  bits[h] = (uint16_t)bitword;
  if (codes) codes[h] = make_uint2((uint32_t)cw, (uint32_t)(cw >> 32));
}

__device__ __noinline__ void mx_fakequant_half_exact(int mode, const uint4* __restrict__ x4, uint64_t h,
                                                     uint32_t sbyte, uint32_t cached, uint2 roll,
                                                     uint4* __restrict__ y4, uint16_t* __restrict__ mask,
                                                     uint2* __restrict__ qcodes) {
  const bool valid = sbyte != 0xffu;
  const float s = valid ? e8m0_value(sbyte) : 1.f;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 16 * h;
  uint16_t* y = reinterpret_cast<uint16_t*>(y4) + 16 * h;
  uint32_t maskword = 0;
  uint64_t cw = 0;
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    const uint32_t rc = ((j < 8 ? roll.x : roll.y) >> (4 * (j & 7))) & 15u;
    uint32_t code, mk, ybits;
    exact_forward_element(mode, __uint_as_float((uint32_t)x[j] << 16), s, valid, (cached >> j) & 1u, rc, code, mk,
                          ybits);
    maskword |= mk << j;
    y[j] = (uint16_t)ybits;
    cw |= (uint64_t)code << (4 * j);
  }
  mask[h] = (uint16_t)maskword;
  if (qcodes) qcodes[h] = make_uint2((uint32_t)cw, (uint32_t)(cw >> 32));
}

// ---------------------------------------------------------------------------
// capture.  Lane pairs (h even, h + 1) hold one 32-element block: each lane
// loads its 16 elements (32 contiguous bytes), the pair exchanges its
// halves' maxima, and the even lane writes the scale byte.  The half count
// n/16 is even, so both lanes of a pair are always active together.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void mx_capture_kernel(const uint4* __restrict__ x, uint64_t nhalves,
                                                              uint8_t* __restrict__ scales,
                                                              uint16_t* __restrict__ bits,
                                                              uint2* __restrict__ codes) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t h = (uint64_t)blockIdx.x * kThreads + threadIdx.x; h < nhalves; h += stride) {
    uint32_t w[8];
    load_block(x, h, w);
    const uint32_t a = half_amax_bits(w);
    const uint32_t b = pair_swap(a);
    const uint32_t sb = mx_scale_byte<kE2M1Emax>(a > b ? a : b);
    const float inv = e8m0_inverse(sb);
    bool bad = false;
    float q[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      q[j] = block_elem(w, j) * inv;
      bad |= __builtin_amdgcn_class(q[j], kBadClass);
    }
    uint32_t E = 0, O = 0;
    FP4_PACK8(FP4_RNE, E, q, 0);
    FP4_PACK8(FP4_RNE, O, q, 1);
    if ((h & 1) == 0) scales[h >> 1] = (uint8_t)sb;
    if (bad) {
      mx_capture_half_exact(x, h, sb, bits, codes);
    } else {
      bits[h] = (uint16_t)gather_parity(E, O);
      if (codes) {
        uint32_t c0, c1;
        interleave_codes(E, O, c0, c1);
        codes[h] = make_uint2(c0, c1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fake-quant forward; kMode: 0 = RNE, 1 = guided, 2 = full information.  One
// lane per 16-element half; both lanes of a block read its scale byte.
// ---------------------------------------------------------------------------
template <int kMode>
__global__ __launch_bounds__(kThreads) void mx_fakequant_kernel(const uint4* __restrict__ x, uint64_t nhalves,
                                                                const uint8_t* __restrict__ scales,
                                                                const uint16_t* __restrict__ bits,
                                                                const uint2* __restrict__ rcodes,
                                                                uint4* __restrict__ y, uint16_t* __restrict__ mask,
                                                                uint2* __restrict__ qcodes) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t h = (uint64_t)blockIdx.x * kThreads + threadIdx.x; h < nhalves; h += stride) {
    const uint32_t sbyte = scales[h >> 1];
    const uint32_t cached = kMode == 1 ? (uint32_t)bits[h] : 0u;
    const uint2 roll = kMode == 2 ? rcodes[h] : make_uint2(0u, 0u);
    uint32_t w[8];
    load_block(x, h, w);
    // a NaN scale byte makes a zero-scale block: multiplying by 0 maps every
    // finite x to a zero of its own sign, decoded with s = 1
    const bool valid = sbyte != 0xffu;
    const float inv = valid ? e8m0_inverse(sbyte) : 0.f;
    const float s = valid ? e8m0_value(sbyte) : 1.f;
    bool bad = false;
    float q[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      q[j] = block_elem(w, j) * inv;
      bad |= __builtin_amdgcn_class(q[j], kBadClass);
    }
    uint32_t QE, QO;
    const uint32_t keep = select_codes<kMode>(q, cached, roll, QE, QO);
    if (bad) {
      mx_fakequant_half_exact(kMode, x, h, sbyte, cached, roll, y, mask, qcodes);
    } else {
      uint32_t out[8];
      decode_block(QE, QO, s, out);
      store_block(y, h, out);
      mask[h] = (uint16_t)(valid ? keep : 0u);
      if (qcodes) {
        uint32_t c0, c1;
        interleave_codes(QE, QO, c0, c1);
        qcodes[h] = make_uint2(c0, c1);
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
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const uint64_t nhalves = 2 * nblocks;
  hipLaunchKernelGGL(mx_capture_kernel, dim3(mx_grid(nhalves)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(x), nhalves, scales, reinterpret_cast<uint16_t*>(bits),
                     reinterpret_cast<uint2*>(codes));
  return hipGetLastError();
}

hipError_t launch_mx_fakequant(int mode, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                               const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                               hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const uint64_t nhalves = 2 * nblocks;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint4* yv = reinterpret_cast<uint4*>(y);
  uint16_t* mv = reinterpret_cast<uint16_t*>(mask);
  uint2* qv = reinterpret_cast<uint2*>(qcodes);
  const dim3 grid(mx_grid(nhalves)), block(kThreads);
  if (mode == 1)
    hipLaunchKernelGGL(mx_fakequant_kernel<1>, grid, block, 0, stream, xv, nhalves, scales,
                       reinterpret_cast<const uint16_t*>(side), static_cast<const uint2*>(nullptr), yv, mv, qv);
  else if (mode == 2)
    hipLaunchKernelGGL(mx_fakequant_kernel<2>, grid, block, 0, stream, xv, nhalves, scales,
                       static_cast<const uint16_t*>(nullptr), reinterpret_cast<const uint2*>(side), yv, mv, qv);
  else
    hipLaunchKernelGGL(mx_fakequant_kernel<0>, grid, block, 0, stream, xv, nhalves, scales,
                       static_cast<const uint16_t*>(nullptr), static_cast<const uint2*>(nullptr), yv, mv, qv);
  return hipGetLastError();
}

}  // namespace trace_host
