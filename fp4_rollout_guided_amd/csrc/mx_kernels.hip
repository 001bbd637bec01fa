// libtrace MXFP4 kernels for gfx950: capture and the guided / RNE /
// full-information fake-quant forwards on MXFP4 scales (the rcap.io post's
// Ablations bullet: the method carries over to MXFP4).  MXFP4 parameters
// from the OCP Microscaling Formats (MX) v1.0 specification: 32-element
// blocks, one E8M0 scale byte b per block standing for 2^(b - 127) (0xFF is
// NaN), E2M1 elements.  The block scale is 2^(floor(log2(amax)) - 2) clamped
// to E8M0's range; elements are rounded as on the NVFP4 path.
//
// In the capture a lane owns one 16-element half of a block (32 contiguous
// bytes of bf16, a 16-bit bit-plane word, 8 bytes of codes) and lane pairs
// share a block's scale: the pair exchanges its halves' maxima with one DPP
// move.  (A lane per 32-element block was measured ~15% slower: its 64-byte
// stride doubles the cache lines each load instruction touches.)  The
// forwards run one lane per 8-element vector (a quarter block: one 128-bit
// load, one byte of bits and of mask, one dword of codes), which streams
// faster still.  Dividing by a power of two is a multiplication
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
// elements (a capture half, a forward vector) whose scale byte is known
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

// The same for one 8-element vector g (elements 8g..8g+7) of the forward:
// cached = its 8 bits, roll = its rollout codes (element order).
__device__ __noinline__ void mx_fakequant_vec_exact(int mode, const uint4* __restrict__ x4, uint64_t g,
                                                    uint32_t sbyte, uint32_t cached, uint32_t roll,
                                                    uint4* __restrict__ y4, uint8_t* __restrict__ mask,
                                                    uint32_t* __restrict__ qcodes) {
  const bool valid = sbyte != 0xffu;
  const float s = valid ? e8m0_value(sbyte) : 1.f;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 8 * g;
  uint16_t* y = reinterpret_cast<uint16_t*>(y4) + 8 * g;
  uint32_t maskbyte = 0, cw = 0;
#pragma unroll 1
  for (int j = 0; j < 8; ++j) {
    uint32_t code, mk, ybits;
    exact_forward_element(mode, __uint_as_float((uint32_t)x[j] << 16), s, valid, (cached >> j) & 1u,
                          (roll >> (4 * j)) & 15u, code, mk, ybits);
    maskbyte |= mk << j;
    y[j] = (uint16_t)ybits;
    cw |= code << (4 * j);
  }
  mask[g] = (uint8_t)maskbyte;
  if (qcodes) qcodes[g] = cw;
}

// ---------------------------------------------------------------------------
// capture.  Lane pairs (h even, h + 1) hold one 32-element block: each lane
// loads its 16 elements (32 contiguous bytes), the pair exchanges its
// halves' maxima, and the even lane writes the scale byte.  The half count
// n/16 is even, so both lanes of a pair are always active together.
// ---------------------------------------------------------------------------
// kNT: the record is stored with the non-temporal hint (tensors past the
// last-level cache; the loads stay plain, as in the NVFP4 capture).
template <bool kNT>
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
    if ((h & 1) == 0) store_word<kNT>(&scales[h >> 1], (uint8_t)sb);
    if (bad) {
      mx_capture_half_exact(x, h, sb, bits, codes);
    } else {
      store_word<kNT>(&bits[h], (uint16_t)gather_parity(E, O));
      if (codes) {
        uint32_t c0, c1;
        interleave_codes(E, O, c0, c1);
        store_pair<kNT>(&codes[h], make_uint2(c0, c1));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fake-quant forward; kMode: 0 = RNE, 1 = guided, 2 = full information.  One
// lane per 8-element vector (one 128-bit load; a quarter of a block): a lane
// with one vector in flight streams faster than one moving 32 bytes.  The
// four lanes of a block read its scale byte.  kNT: x is loaded and every
// output stored with the non-temporal hint (tensors past the last-level
// cache).
// ---------------------------------------------------------------------------
template <int kMode, bool kNT>
__global__ __launch_bounds__(kThreads) void mx_fakequant_kernel(const uint4* __restrict__ x, uint64_t nvec,
                                                                const uint8_t* __restrict__ scales,
                                                                const uint8_t* __restrict__ bits,
                                                                const uint32_t* __restrict__ rcodes,
                                                                uint4* __restrict__ y, uint8_t* __restrict__ mask,
                                                                uint32_t* __restrict__ qcodes) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x; g < nvec; g += stride) {
    const uint32_t sbyte = scales[g >> 2];
    const uint32_t cached = kMode == 1 ? (uint32_t)bits[g] : 0u;
    const uint32_t roll = kMode == 2 ? rcodes[g] : 0u;
    const uint4 v = load_vec<kNT>(&x[g]);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    // a NaN scale byte makes a zero-scale block: multiplying by 0 maps every
    // finite x to a zero of its own sign, decoded with s = 1
    const bool valid = sbyte != 0xffu;
    const float inv = valid ? e8m0_inverse(sbyte) : 0.f;
    const float s = valid ? e8m0_value(sbyte) : 1.f;
    bool bad = false;
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      q[j] = half_elem(w, j) * inv;
      bad |= __builtin_amdgcn_class(q[j], kBadClass);
    }
    uint32_t Q;
    const uint32_t keep = select_codes8<kMode>(q, cached, roll, Q);
    if (bad) {
      mx_fakequant_vec_exact(kMode, x, g, sbyte, cached, roll, y, mask, qcodes);
    } else {
      uint32_t out[4];
      decode_half(Q, s, out);
      store_vec<kNT>(&y[g], make_uint4(out[0], out[1], out[2], out[3]));
      store_word<kNT>(&mask[g], (uint8_t)(valid ? keep : 0u));
      if (qcodes) store_word<kNT>(&qcodes[g], Q);
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
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint16_t* bv = reinterpret_cast<uint16_t*>(bits);
  uint2* cv = reinterpret_cast<uint2*>(codes);
  if (past_cache(nblocks * 64))
    hipLaunchKernelGGL(mx_capture_kernel<true>, dim3(mx_grid(nhalves)), dim3(kThreads), 0, stream, xv, nhalves,
                       scales, bv, cv);
  else
    hipLaunchKernelGGL(mx_capture_kernel<false>, dim3(mx_grid(nhalves)), dim3(kThreads), 0, stream, xv, nhalves,
                       scales, bv, cv);
  return hipGetLastError();
}

template <bool kNT>
static void launch_mx_fakequant_t(int mode, const uint4* xv, uint64_t nvec, const uint8_t* scales,
                                  const uint8_t* side, uint4* yv, uint8_t* mask, uint32_t* qv, hipStream_t stream) {
  const dim3 grid(mx_grid(nvec)), block(kThreads);
  if (mode == 1)
    hipLaunchKernelGGL((mx_fakequant_kernel<1, kNT>), grid, block, 0, stream, xv, nvec, scales, side,
                       static_cast<const uint32_t*>(nullptr), yv, mask, qv);
  else if (mode == 2)
    hipLaunchKernelGGL((mx_fakequant_kernel<2, kNT>), grid, block, 0, stream, xv, nvec, scales,
                       static_cast<const uint8_t*>(nullptr), reinterpret_cast<const uint32_t*>(side), yv, mask, qv);
  else
    hipLaunchKernelGGL((mx_fakequant_kernel<0, kNT>), grid, block, 0, stream, xv, nvec, scales,
                       static_cast<const uint8_t*>(nullptr), static_cast<const uint32_t*>(nullptr), yv, mask, qv);
}

hipError_t launch_mx_fakequant(int mode, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                               const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                               hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const uint64_t nvec = 4 * nblocks;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint4* yv = reinterpret_cast<uint4*>(y);
  uint32_t* qv = reinterpret_cast<uint32_t*>(qcodes);
  if (past_cache(nblocks * 64))
    launch_mx_fakequant_t<true>(mode, xv, nvec, scales, side, yv, mask, qv, stream);
  else
    launch_mx_fakequant_t<false>(mode, xv, nvec, scales, side, yv, mask, qv, stream);
  return hipGetLastError();
}

}  // namespace trace_host
