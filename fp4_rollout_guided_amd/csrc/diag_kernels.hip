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
// One lane owns one 16-element block, as in the forwards.  The four code
// words of a block (rollout, RNE, guided, full information; even and odd
// elements in separate dwords, eight nibbles each) are compared with
// nibble-parallel integer arithmetic: a code's signed grid index is shifted
// by 8 into a nibble 1..15 (both zeros map to 8), equality and one-step
// neighbours become per-nibble zero tests, and counts are population counts.
// That covers every element whose rollout and RNE codes are at most one step
// apart and whose guided and RNE codes are too; a block with any other
// element (a two-step mismatch, rare) is counted element by element.  Counts
// live in registers per lane (steps 0 and 1, the four counters) and in a
// workgroup-shared table (steps 2..14); after the grid-stride loop each wave
// folds its registers with cross-lane adds, one lane per wave adds them to
// the shared table, and the workgroup adds the table to the 64-bit device
// counters with vector-memory atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "device_math.h"
#include "fp4_block.h"
#include "launch.h"
#include "nvfp4_scale.h"

namespace trace_dev {

constexpr int kStatWords = 20;  // see the layout in launch.h

constexpr uint32_t kNib3 = 0x88888888u;  // bit 3 of every nibble
constexpr uint32_t kOnes = 0x11111111u;

// 8 + signed grid index of every code nibble (sign << 3 | magnitude index):
// 1..15, both zeros 8.  Positive codes give c ^ 8 = 8 + m; negative ones
// (c ^ 15) + 1 = 16 - c = 8 - m, the +1 staying inside the nibble.
__device__ __forceinline__ uint32_t offset_index(uint32_t c) {
  const uint32_t sb = c & kNib3;
  const uint32_t s1 = sb >> 3;                 // 1 in negative nibbles
  return (c ^ kNib3 ^ (sb - s1)) + s1;         // sb - s1 = 7 in negative nibbles
}

// Bit 3 of each nibble set where that nibble of x is zero.
__device__ __forceinline__ uint32_t zero_nibbles(uint32_t x) {
  return ~(((x & 0x77777777u) + 0x77777777u) | x) & kNib3;
}

// Per-nibble flags of one code dword pair; false when some element needs the
// per-element count.  One-step neighbours are tested by subtracting 1 from
// the larger side (offset indices are >= 1, so no nibble borrows).
struct NibbleStats {
  uint32_t same, one, straddle, crossed, recovered, violation;
};

__device__ __forceinline__ bool nibble_stats(uint32_t r, uint32_t n, uint32_t g, uint32_t f, NibbleStats& o) {
  const uint32_t ur = offset_index(r), un = offset_index(n), ug = offset_index(g), uf = offset_index(f);
  const uint32_t same = zero_nibbles(ur ^ un);               // rollout == RNE
  const uint32_t up = zero_nibbles(un ^ (ur - kOnes));       // rollout one step above RNE
  const uint32_t down = zero_nibbles(ur ^ (un - kOnes));     // rollout one step below RNE
  const uint32_t g_eq = zero_nibbles(ug ^ un);               // guided == RNE
  const uint32_t g_up = zero_nibbles(un ^ (ug - kOnes));     // guided one step above RNE
  const uint32_t g_down = zero_nibbles(ug ^ (un - kOnes));   // guided one step below RNE
  o.same = same;
  o.one = up | down;
  o.straddle = ~same & zero_nibbles(uf ^ ur) & kNib3;
  o.crossed = o.one & ~o.straddle;
  o.recovered = ~same & zero_nibbles(ug ^ ur) & kNib3;
  // guided and RNE adjacent: the guided value is farther from the rollout
  // codeword exactly when the rollout lies on the RNE side (or on it)
  o.violation = (g_up & (same | down)) | (g_down & (same | up));
  return ((same | o.one) & (g_eq | g_up | g_down)) == kNib3;
}

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

// Counts of one block by the definitions, one element at a time: steps of 2
// or more go to the shared table; the rest come back packed five bits each
// (steps 0, steps 1, straddle, crossed, recovered, violations).
// Arguments: the code dwords of the even (suffix 0) and odd (suffix 1) elements.
__device__ __noinline__ uint32_t count_block_slow(uint32_t r0, uint32_t r1, uint32_t n0, uint32_t n1, uint32_t g0,
                                                  uint32_t g1, uint32_t f0, uint32_t f1, uint32_t* table) {
  uint32_t packed = 0;
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    const bool odd = j >= 8;
    const int sh = 4 * (j & 7);
    const uint32_t cr = ((odd ? r1 : r0) >> sh) & 15u, cn = ((odd ? n1 : n0) >> sh) & 15u;
    const uint32_t cg = ((odd ? g1 : g0) >> sh) & 15u, cf = ((odd ? f1 : f0) >> sh) & 15u;
    const int sr = signed_idx(cr);
    const int d = sr - signed_idx(cn);
    const uint32_t steps = (uint32_t)(d < 0 ? -d : d);
    if (steps >= 2) atomicAdd(&table[steps], 1u);
    // the full-information code is the rollout's exactly when the rollout
    // codeword is an endpoint of the bracket
    const bool straddle = steps != 0 && signed_idx(cf) == sr;
    const int vr = twice_value(cr);
    const int dg = twice_value(cg) - vr, dn = twice_value(cn) - vr;
    packed += (uint32_t)(steps == 0) + ((uint32_t)(steps == 1) << 5) + ((uint32_t)straddle << 10) +
              ((uint32_t)(steps == 1 && !straddle) << 15) +
              ((uint32_t)(steps != 0 && signed_idx(cg) == sr) << 20) +
              ((uint32_t)((dg < 0 ? -dg : dg) > (dn < 0 ? -dn : dn)) << 25);
  }
  return packed;
}

// RNE, guided and full-information codes of one block (element order, 4
// bits per element) by the definitions, for the lanes the fast path rejects.
struct BlockCodes {
  uint64_t rne, guided, full;
};

__device__ __noinline__ BlockCodes stats_block_exact(const uint4* __restrict__ x4, uint64_t b, uint32_t sbyte,
                                                     float ts, uint32_t cached, uint2 roll) {
  const float s = e4m3_decode(sbyte) * ts;
  const bool valid = s > 0.f && s <= 3.40282347e38f;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 16 * b;
  uint64_t cw[3] = {0, 0, 0};
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    const float xv = __uint_as_float((uint32_t)x[j] << 16);
    const uint32_t rc = ((j < 8 ? roll.x : roll.y) >> (4 * (j & 7))) & 15u;
#pragma unroll 1
    for (int mode = 0; mode < 3; ++mode) {
      uint32_t code, mk, ybits;
      exact_forward_element(mode, xv, s, valid, (cached >> j) & 1u, rc, code, mk, ybits);
      const uint64_t c = (uint64_t)code << (4 * j);
      if (mode == 0) cw[0] |= c; else if (mode == 1) cw[1] |= c; else cw[2] |= c;
    }
  }
  return BlockCodes{cw[0], cw[1], cw[2]};
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
    // code dwords [even elements, odd elements]: rollout, RNE, guided, full information
    uint32_t r[2], cn[2], cg[2], cf[2];
    split_codes(roll.x, roll.y, r[0], r[1]);
    if (bad) {
      const BlockCodes c = stats_block_exact(x, b, sbyte, ts, cached, roll);
      split_codes((uint32_t)c.rne, (uint32_t)(c.rne >> 32), cn[0], cn[1]);
      split_codes((uint32_t)c.guided, (uint32_t)(c.guided >> 32), cg[0], cg[1]);
      split_codes((uint32_t)c.full, (uint32_t)(c.full >> 32), cf[0], cf[1]);
    } else {
      select_codes<0>(q, cached, roll, cn[0], cn[1]);
      select_codes<1>(q, cached, roll, cg[0], cg[1]);
      select_codes<2>(q, cached, roll, cf[0], cf[1]);
    }
    NibbleStats s0, s1;
    const bool ok0 = nibble_stats(r[0], cn[0], cg[0], cf[0], s0);
    const bool ok1 = nibble_stats(r[1], cn[1], cg[1], cf[1], s1);
    if (ok0 && ok1) {
      n0 += __builtin_popcount(s0.same) + __builtin_popcount(s1.same);
      n1 += __builtin_popcount(s0.one) + __builtin_popcount(s1.one);
      nst += __builtin_popcount(s0.straddle) + __builtin_popcount(s1.straddle);
      ncr += __builtin_popcount(s0.crossed) + __builtin_popcount(s1.crossed);
      nrec += __builtin_popcount(s0.recovered) + __builtin_popcount(s1.recovered);
      nvio += __builtin_popcount(s0.violation) + __builtin_popcount(s1.violation);
    } else {
      const uint32_t p = count_block_slow(r[0], r[1], cn[0], cn[1], cg[0], cg[1], cf[0], cf[1], table);
      n0 += p & 31u;
      n1 += (p >> 5) & 31u;
      nst += (p >> 10) & 31u;
      ncr += (p >> 15) & 31u;
      nrec += (p >> 20) & 31u;
      nvio += (p >> 25) & 31u;
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

// Workgroups of the statistics kernel resident at once on the current device
// (occupancy x compute units), cached per device.  Every workgroup ends with
// atomic adds to the same twenty counters, so the grid is held to one
// resident wave of workgroups that loop over the tensor: one workgroup per
// 256 blocks would queue ~10^5 atomics per counter at one L2 channel.
static uint32_t stats_resident_groups() {
  constexpr uint32_t kDefault = 1024;  // should the queries fail (the launch then reports the error)
  static std::atomic<uint32_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefault;
  uint32_t v = cache[dev].load(std::memory_order_relaxed);
  if (v) return v;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mismatch_stats_kernel, kThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu <= 0 ||
      cus <= 0)
    return kDefault;
  v = (uint32_t)per_cu * (uint32_t)cus;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_mismatch_stats(const uint16_t* x, uint64_t nblocks, const uint8_t* scales, const float* ts,
                                 const uint8_t* bits, const uint8_t* codes, uint64_t* stats, hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  uint64_t g = (nblocks + kThreads - 1) / kThreads;
  const uint64_t resident = stats_resident_groups();
  if (g > resident) g = resident;
  if (g > kMaxGroups) g = kMaxGroups;
  hipLaunchKernelGGL(mismatch_stats_kernel, dim3((unsigned)g), dim3(kThreads), 0,
                     stream, reinterpret_cast<const uint4*>(x), nblocks, scales, ts,
                     reinterpret_cast<const uint16_t*>(bits), reinterpret_cast<const uint2*>(codes),
                     reinterpret_cast<unsigned long long*>(stats));
  return hipGetLastError();
}

}  // namespace trace_host
