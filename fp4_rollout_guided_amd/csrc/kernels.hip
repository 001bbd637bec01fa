// libtrace kernels for gfx950: tensor amax, capture, guided / RNE fake-quant
// forward and STE backward.
//
// Work decomposition: one lane owns one 16-element NVFP4 block, i.e. 32
// contiguous bytes of bf16 (two 128-bit loads), its scale byte, and 16 bits of
// every bit-plane (one 16-bit store).  Blocks never span lanes, so the block
// amax needs no cross-lane traffic and every output byte has one writer.  A
// 256-lane workgroup covers 4096 consecutive elements: its bit-plane, mask and
// scale stores are whole 128-byte lines.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "launch.h"

namespace trace_dev {

constexpr int kThreads = 256;

__device__ __forceinline__ void load_block(const uint4* __restrict__ x, uint64_t b, uint32_t (&w)[8]) {
  const uint4 v0 = x[2 * b];
  const uint4 v1 = x[2 * b + 1];
  w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
  w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
}

__device__ __forceinline__ void store_block(uint4* __restrict__ y, uint64_t b, const uint32_t (&w)[8]) {
  y[2 * b] = make_uint4(w[0], w[1], w[2], w[3]);
  y[2 * b + 1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// ---------------------------------------------------------------------------
// tensor amax: per-workgroup maxima of the bf16 magnitude bits (NaN excluded),
// then one workgroup folds them and forms ts = fl32(amax / 2688).
// Integer maxima over magnitude bits order non-NaN bf16 values exactly as
// their absolute values.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[kThreads / 64];
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  if (threadIdx.x < 64) {
    v = threadIdx.x < kThreads / 64 ? red[threadIdx.x] : 0u;
    v = wave_max_u32(v);
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const uint4* __restrict__ x,
                                                                uint64_t nblocks,
                                                                uint32_t* __restrict__ partial) {
  uint32_t best = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += stride) {
    uint32_t w[8];
    load_block(x, b, w);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t lo = w[k] & 0x7fffu, hi = (w[k] >> 16) & 0x7fffu;
      if (lo <= 0x7f80u) best = max(best, lo);
      if (hi <= 0x7f80u) best = max(best, hi);
    }
  }
  best = block_max_u32(best);
  if (threadIdx.x == 0) partial[blockIdx.x] = best;
}

__global__ __launch_bounds__(kThreads) void amax_finalize_kernel(const uint32_t* __restrict__ partial,
                                                                 uint32_t count, float* __restrict__ ts_out) {
  uint32_t best = 0;
  for (uint32_t i = threadIdx.x; i < count; i += kThreads) best = max(best, partial[i]);
  best = block_max_u32(best);
  if (threadIdx.x == 0) *ts_out = __uint_as_float(best << 16) / kTensorDiv;
}

// ---------------------------------------------------------------------------
// capture
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void capture_kernel(const uint4* __restrict__ x, uint64_t nblocks,
                                                           const float* __restrict__ ts_ptr,
                                                           uint8_t* __restrict__ scales,
                                                           uint16_t* __restrict__ bits,
                                                           uint2* __restrict__ codes) {
  const uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nblocks) return;
  const float ts = *ts_ptr;
  uint32_t w[8];
  load_block(x, b, w);

  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    const float a = fabsf(block_elem(w, j));
    if (a > amax) amax = a;  // NaN compares false: ignored
  }
  uint32_t sb = 0;
  if (ts > 0.f && ts <= 3.40282347e38f) sb = e4m3_encode_sat((amax / 6.f) / ts);
  const float s = e4m3_decode(sb) * ts;
  const bool valid = s > 0.f && s <= 3.40282347e38f;

  uint32_t bitword = 0, c0 = 0, c1 = 0;
#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    const float xv = block_elem(w, j);
    uint32_t sign = __float_as_uint(xv) >> 31;
    uint32_t idx = 0;
    if (is_nan_f(xv)) {
      sign = 0;
    } else if (valid) {
      const float z = xv / s;
      idx = e2m1_rne_index(fminf(fabsf(z), 6.f));
    }
    bitword |= (idx & 1u) << j;
    const uint32_t code = (sign << 3) | idx;
    if (j < 8) c0 |= code << (4 * j); else c1 |= code << (4 * (j - 8));
  }
  scales[b] = (uint8_t)sb;
  bits[b] = (uint16_t)bitword;
  if (codes) codes[b] = make_uint2(c0, c1);
}

// ---------------------------------------------------------------------------
// fake-quant forward (guided or plain RNE) and STE backward
// ---------------------------------------------------------------------------
template <bool kGuided>
__global__ __launch_bounds__(kThreads) void fakequant_kernel(const uint4* __restrict__ x, uint64_t nblocks,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ ts_ptr,
                                                             const uint16_t* __restrict__ bits,
                                                             uint4* __restrict__ y,
                                                             uint16_t* __restrict__ mask,
                                                             uint2* __restrict__ qcodes) {
  const uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nblocks) return;
  const float ts = *ts_ptr;
  const float s = e4m3_decode(scales[b]) * ts;
  const bool valid = s > 0.f && s <= 3.40282347e38f;
  const uint32_t cached = kGuided ? (uint32_t)bits[b] : 0u;
  uint32_t w[8];
  load_block(x, b, w);

  uint32_t out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint32_t maskword = 0, c0 = 0, c1 = 0;
#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    const float xv = block_elem(w, j);
    uint32_t sign = __float_as_uint(xv) >> 31;
    uint32_t idx = 0, mk = 0;
    float yv;
    if (is_nan_f(xv)) {
      sign = 0;
      yv = 0.f;
    } else if (!valid) {
      yv = sign ? -0.f : 0.f;
    } else {
      const float zr = xv / s;
      mk = fabsf(zr) <= 6.f ? 1u : 0u;
      const float a = fminf(fabsf(zr), 6.f);
      if (kGuided) {
        const uint32_t lo = e2m1_floor_index(a);
        const bool exact = (a == e2m1_mag(lo));
        const uint32_t c = (cached >> j) & 1u;
        idx = (exact || ((lo & 1u) == c)) ? lo : lo + 1;
      } else {
        idx = e2m1_rne_index(a);
      }
      const float q = e2m1_mag(idx);
      yv = s * (sign ? -q : q);
    }
    maskword |= mk << j;
    out[j >> 1] |= bf16_rne_bits(yv) << (16 * (j & 1));
    const uint32_t code = (sign << 3) | idx;
    if (j < 8) c0 |= code << (4 * j); else c1 |= code << (4 * (j - 8));
  }
  store_block(y, b, out);
  mask[b] = (uint16_t)maskword;
  if (qcodes) qcodes[b] = make_uint2(c0, c1);
}

__global__ __launch_bounds__(kThreads) void ste_bwd_kernel(const uint4* __restrict__ g, uint64_t nblocks,
                                                           const uint16_t* __restrict__ mask,
                                                           uint4* __restrict__ gin) {
  const uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nblocks) return;
  const uint32_t m = mask[b];
  uint32_t w[8];
  load_block(g, b, w);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t keep = (((m >> (2 * k)) & 1u) ? 0x0000ffffu : 0u) |
                          (((m >> (2 * k + 1)) & 1u) ? 0xffff0000u : 0u);
    w[k] &= keep;
  }
  store_block(gin, b, w);
}

}  // namespace trace_dev

// ---------------------------------------------------------------------------
// launchers (host)
// ---------------------------------------------------------------------------
namespace trace_host {

using namespace trace_dev;

static unsigned grid_for(uint64_t nblocks) { return (unsigned)((nblocks + kThreads - 1) / kThreads); }

uint32_t amax_partial_count(uint64_t nblocks) {
  const uint64_t g = (nblocks + kThreads - 1) / kThreads;
  return (uint32_t)(g < kAmaxMaxGroups ? (g == 0 ? 1 : g) : kAmaxMaxGroups);
}

hipError_t launch_tensor_scale(const uint16_t* x, uint64_t nblocks, uint32_t* partial, float* ts_out,
                               hipStream_t stream) {
  const uint32_t groups = amax_partial_count(nblocks);
  if (nblocks > 0)
    hipLaunchKernelGGL(amax_partial_kernel, dim3(groups), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), nblocks, partial);
  hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(kThreads), 0, stream, partial,
                     nblocks > 0 ? groups : 0u, ts_out);
  return hipGetLastError();
}

hipError_t launch_capture(const uint16_t* x, uint64_t nblocks, const float* ts, uint8_t* scales,
                          uint8_t* bits, uint8_t* codes, hipStream_t stream) {
  hipLaunchKernelGGL(capture_kernel, dim3(grid_for(nblocks)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(x), nblocks, ts, scales,
                     reinterpret_cast<uint16_t*>(bits), reinterpret_cast<uint2*>(codes));
  return hipGetLastError();
}

hipError_t launch_fakequant(bool guided, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                            const float* ts, const uint8_t* bits, uint16_t* y, uint8_t* mask,
                            uint8_t* qcodes, hipStream_t stream) {
  if (guided)
    hipLaunchKernelGGL(fakequant_kernel<true>, dim3(grid_for(nblocks)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), nblocks, scales, ts,
                       reinterpret_cast<const uint16_t*>(bits), reinterpret_cast<uint4*>(y),
                       reinterpret_cast<uint16_t*>(mask), reinterpret_cast<uint2*>(qcodes));
  else
    hipLaunchKernelGGL(fakequant_kernel<false>, dim3(grid_for(nblocks)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), nblocks, scales, ts,
                       static_cast<const uint16_t*>(nullptr), reinterpret_cast<uint4*>(y),
                       reinterpret_cast<uint16_t*>(mask), reinterpret_cast<uint2*>(qcodes));
  return hipGetLastError();
}

hipError_t launch_ste_bwd(const uint16_t* g, const uint8_t* mask, uint64_t nblocks, uint16_t* gin,
                          hipStream_t stream) {
  hipLaunchKernelGGL(ste_bwd_kernel, dim3(grid_for(nblocks)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(g), nblocks,
                     reinterpret_cast<const uint16_t*>(mask), reinterpret_cast<uint4*>(gin));
  return hipGetLastError();
}

}  // namespace trace_host
