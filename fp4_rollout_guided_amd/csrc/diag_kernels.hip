// libtrace diagnostics kernel for gfx950: rollout / training agreement
// statistics of one NVFP4 site tensor.  The rcap.io post "TRACE:
// Rollout-Guided Quantization-Aware Training for FP4" rests on three facts
// about the sites where the two paths disagree: most mismatches are one
// adjacent codeword (bandwidth paragraph), such a mismatch is a value
// straddling a rounding midpoint (rounding-boundary paragraph), and the
// guided choice is never farther from the rollout codeword than plain
// rounding (rollout-guided rounding paragraph).  This kernel counts them on
// whole tensors:
//   mismatch_stats_kernel   per element, the training side's RNE, guided and
//                           full-information codes (the forwards' own code
//                           selection, fast path and exact fallback alike)
//                           against the rollout code, accumulated into a
//                           histogram of signed grid steps and four counters.
//
// One lane owns one 16-element block, as in the forwards.  Counts live in
// registers per lane (steps 0 and 1, the four counters) and in a
// workgroup-shared table (steps 2..14, rare); after the grid-stride loop each
// wave folds its registers with cross-lane adds, one lane per wave adds them
// to the shared table, and the workgroup adds the table to the 64-bit device
// counters with vector-memory atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "fp4_block.h"
#include "launch.h"
#include "nvfp4_scale.h"

namespace trace_dev {

constexpr int kStatWords = 20;  // see the layout in launch.h

__device__ __forceinline__ int signed_idx(uint32_t c) {
  const int m = (int)(c & 7u);
  return (c & 8u) ? -m : m;
}

// Twice the signed value of an E2M1 code: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
// become the integers 0, 1, 2, 3, 4, 6, 8, 12.
__device__ __forceinline__ int twice_value(uint32_t c) {
  const int m = (int)((0x0C08060403020100ull >> (8 * (c & 7u))) & 0xFFu);
  return (c & 8u) ? -m : m;
}

// RNE, guided and full-information codes of one block (element order, 4
// bits per element) by the definitions, for the lanes the fast path rejects.
__device__ __noinline__ void stats_block_exact(const uint4* __restrict__ x4, uint64_t b, uint32_t sbyte, float ts,
                                               uint32_t cached, uint2 roll, uint64_t (&cw)[3]) {
  const float s = e4m3_decode(sbyte) * ts;
  const bool valid = s > 0.f && s <= 3.40282347e38f;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 16 * b;
  cw[0] = cw[1] = cw[2] = 0;
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    const float xv = __uint_as_float((uint32_t)x[j] << 16);
    const uint32_t rc = ((j < 8 ? roll.x : roll.y) >> (4 * (j & 7))) & 15u;
#pragma unroll 1
    for (int mode = 0; mode < 3; ++mode) {
      uint32_t code, mk, ybits;
      exact_forward_element(mode, xv, s, valid, (cached >> j) & 1u, rc, code, mk, ybits);
      cw[mode] |= (uint64_t)code << (4 * j);
    }
  }
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  for (int off = 32; off > 0; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
  return v;
}

__global__ __launch_bounds__(kThreads) void mismatch_stats_kernel(const uint4* __restrict__ x, uint64_t nblocks,
                                                                  const uint8_t* __restrict__ scales,
                                                                  const float* __restrict__ ts_ptr,
                                                                  const uint16_t* __restrict__ bits,
                                                                  const uint2* __restrict__ rcodes,
                                                                  unsigned long long* __restrict__ stats) {
  __shared__ uint32_t table[kStatWords];
  if (threadIdx.x < kStatWords) table[threadIdx.x] = 0;
  __syncthreads();
  const float ts = *ts_ptr;
  // per-lane counts: steps 0, steps 1, straddle, crossed, recovered, violations, elements
  uint32_t n0 = 0, n1 = 0, nst = 0, ncr = 0, nrec = 0, nvio = 0, nel = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += stride) {
    const uint32_t sbyte = scales[b];
    const uint32_t cached = bits[b];
    const uint2 roll = rcodes[b];
    uint32_t w[8];
    load_block(x, b, w);
    const ScaleEntry e = make_scale_entry(sbyte, ts);
    bool bad = false;
    float q[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = div_fast<true>(block_elem(w, j), e, bad);
    uint64_t cw[3];
    if (bad) {
      stats_block_exact(x, b, sbyte, ts, cached, roll, cw);
    } else {
      uint32_t QE, QO, c0, c1;
      select_codes<0>(q, cached, roll, QE, QO);
      interleave_codes(QE, QO, c0, c1);
      cw[0] = ((uint64_t)c1 << 32) | c0;
      select_codes<1>(q, cached, roll, QE, QO);
      interleave_codes(QE, QO, c0, c1);
      cw[1] = ((uint64_t)c1 << 32) | c0;
      select_codes<2>(q, cached, roll, QE, QO);
      interleave_codes(QE, QO, c0, c1);
      cw[2] = ((uint64_t)c1 << 32) | c0;
    }
    const uint64_t rw = ((uint64_t)roll.y << 32) | roll.x;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t r = (uint32_t)(rw >> (4 * j)) & 15u;
      const uint32_t cn = (uint32_t)(cw[0] >> (4 * j)) & 15u;
      const uint32_t cg = (uint32_t)(cw[1] >> (4 * j)) & 15u;
      const uint32_t cf = (uint32_t)(cw[2] >> (4 * j)) & 15u;
      const int sr = signed_idx(r);
      const int d = sr - signed_idx(cn);
      const uint32_t steps = (uint32_t)(d < 0 ? -d : d);
      n0 += steps == 0;
      n1 += steps == 1;
      if (steps >= 2) atomicAdd(&table[steps], 1u);
      // the full-information code is the rollout's exactly when the rollout
      // codeword is an endpoint of the bracket
      const bool straddle = steps != 0 && signed_idx(cf) == sr;
      nst += straddle;
      ncr += steps == 1 && !straddle;
      nrec += steps != 0 && signed_idx(cg) == sr;
      const int vr = twice_value(r);
      const int dg = twice_value(cg) - vr, dn = twice_value(cn) - vr;
      nvio += (dg < 0 ? -dg : dg) > (dn < 0 ? -dn : dn);
    }
    nel += 16;
  }
  const uint32_t red[7] = {wave_sum_u32(n0), wave_sum_u32(n1), wave_sum_u32(nst), wave_sum_u32(ncr),
                           wave_sum_u32(nrec), wave_sum_u32(nvio), wave_sum_u32(nel)};
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&table[0], red[0]);
    atomicAdd(&table[1], red[1]);
    atomicAdd(&table[15], red[2]);
    atomicAdd(&table[16], red[3]);
    atomicAdd(&table[17], red[4]);
    atomicAdd(&table[18], red[5]);
    atomicAdd(&table[19], red[6]);
  }
  __syncthreads();
  if (threadIdx.x < kStatWords && table[threadIdx.x] != 0)
    atomicAdd(&stats[threadIdx.x], (unsigned long long)table[threadIdx.x]);
}

}  // namespace trace_dev

namespace trace_host {

using namespace trace_dev;

hipError_t launch_mismatch_stats(const uint16_t* x, uint64_t nblocks, const uint8_t* scales, const float* ts,
                                 const uint8_t* bits, const uint8_t* codes, uint64_t* stats, hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const uint64_t g = (nblocks + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(mismatch_stats_kernel, dim3((unsigned)(g < kMaxGroups ? g : kMaxGroups)), dim3(kThreads), 0,
                     stream, reinterpret_cast<const uint4*>(x), nblocks, scales, ts,
                     reinterpret_cast<const uint16_t*>(bits), reinterpret_cast<const uint2*>(codes),
                     reinterpret_cast<unsigned long long*>(stats));
  return hipGetLastError();
}

}  // namespace trace_host
