// libtrace NVFP4 kernels for gfx950: tensor amax, capture, guided / RNE /
// full-information fake-quant forward, STE backward, per-expert (row-group)
// variants of the tensor scale, capture and forwards, capture to and forward
// from b cached low bits, and the record gather.  The MXFP4 kernels are in
// mx_kernels.hip, the MXFP8 ones in mx8_kernels.hip and the agreement
// statistics in diag_kernels.hip; the block machinery they share is in
// fp4_block.h and the NVFP4 scale decode and exact division in
// nvfp4_scale.h.
//
// Work decomposition: in the capture and the low-bits forward one lane owns
// one 16-element NVFP4 block, i.e. 32 contiguous bytes of bf16 (two 128-bit
// loads), its scale byte, and 16 bits of every bit-plane (one 16-bit store).
// Blocks never span lanes, so the block amax needs no cross-lane traffic and
// every output byte has one writer.  The forwards (ungrouped, per-expert and
// on records read back in place) run one lane per half block (8 elements,
// one 128-bit load, one byte of mask, one dword of codes) and the STE
// backward one lane per 128-bit vector: a lane with one vector in flight
// streams ~5% faster there, and every load and store instruction covers
// whole lines, while the capture (a long dependent chain after its load) and
// the low-bits forward (more dependent loads) measured slower that way.  The
// grid covers the tensor once
// (one tile per workgroup); the kernels keep a grid-stride loop only for grids
// larger than the launch limit.  The two amax passes are the exceptions: the
// tensor amax loops a capped grid (one partial maximum per workgroup) and the
// per-row amax gives each row a workgroup (rows of 2048 elements or more) or
// a wave (narrower rows).
//
// Every kernel has an exact fast path and an exact fallback.  The fast path
// computes each quotient x / s with a double-word reciprocal and one
// remainder correction (4 VALU ops, correctly rounded when the operands are in
// range, see div_fast), and lets gfx950's FP4 / FP8 conversion instructions do
// the grid rounding (their rounding was checked exhaustively against the
// format definitions).  A lane whose block holds a NaN, an infinity, a
// subnormal quotient, or a scale outside the fast range runs the fallback,
// which evaluates the definitions directly with IEEE division.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "device_math.h"
#include "fp4_block.h"
#include "launch.h"
#include "nvfp4_scale.h"

namespace trace_dev {

// ---------------------------------------------------------------------------
// exact fallbacks: the definitions evaluated directly (IEEE division)
// ---------------------------------------------------------------------------

// These run only for the rare lanes the fast path rejects, so they favour a
// small register footprint (one element at a time, 16-bit accesses) over
// speed.  In-place use (y == x) is safe: each element is read before it is
// written and the fast path stored nothing for the lane.
// Bit planes of the b cached low bits: plane k of block b is word
// b + k * stride of the plane array (plane 0 is the parity plane).
struct Planes {
  uint32_t count;   // b
  uint64_t stride;  // words (16-bit) per plane = blocks
};

__device__ __noinline__ void capture_block_exact(const uint4* __restrict__ x4, uint64_t b, float ts,
                                                 uint8_t* __restrict__ scales, uint16_t* __restrict__ bits,
                                                 uint2* __restrict__ codes, Planes planes = Planes{1, 0}) {
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 16 * b;
  float amax = 0.f;
#pragma unroll 1
  for (int j = 0; j < kBlock; ++j) {
    const float a = fabsf(__uint_as_float((uint32_t)x[j] << 16));
    if (a > amax) amax = a;  // NaN compares false: ignored
  }
  uint32_t sb = 0;
  if (ts > 0.f && ts <= 3.40282347e38f) sb = e4m3_encode_sat((amax / 6.f) / ts);
  const float s = e4m3_decode(sb) * ts;
  const bool valid = s > 0.f && s <= 3.40282347e38f;
  uint32_t pw[4] = {0, 0, 0, 0};
  uint64_t cw = 0;
#pragma unroll 1
  for (int j = 0; j < kBlock; ++j) {
    const uint32_t code = exact_capture_code(__uint_as_float((uint32_t)x[j] << 16), s, valid);
    const uint32_t si = (code & 8u) ? ((16u - (code & 7u)) & 15u) : code;  // signed index, 4-bit two's complement
#pragma unroll
    for (int k = 0; k < 4; ++k) pw[k] |= ((si >> k) & 1u) << j;
    cw |= (uint64_t)code << (4 * j);
  }
  scales[b] = (uint8_t)sb;
#pragma unroll 1
  for (uint32_t k = 0; k < planes.count; ++k) bits[b + k * planes.stride] = (uint16_t)pw[k];
  if (codes) codes[b] = make_uint2((uint32_t)cw, (uint32_t)(cw >> 32));
}

// mode: 0 = RNE, 1 = guided by the cached bit (cached = 16-bit word),
// 2 = full information (rollout codes in roll_lo / roll_hi, element order).
// mode 3: b cached low bits, residues as even / odd nibble dwords in
// roll_lo / roll_hi, rule lb.
__device__ __noinline__ void fakequant_block_exact(int mode, const uint4* __restrict__ x4, uint64_t b,
                                                   uint32_t sbyte, float ts, uint32_t cached,
                                                   uint32_t roll_lo, uint32_t roll_hi,
                                                   uint4* __restrict__ y4, uint16_t* __restrict__ mask,
                                                   uint2* __restrict__ qcodes,
                                                   LowBitsRule lb = LowBitsRule{}) {
  const float s = e4m3_decode(sbyte) * ts;
  const bool valid = s > 0.f && s <= 3.40282347e38f;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 16 * b;
  uint16_t* y = reinterpret_cast<uint16_t*>(y4) + 16 * b;
  uint32_t maskword = 0;
  uint64_t cw = 0;
#pragma unroll 1
  for (int j = 0; j < kBlock; ++j) {
    const uint32_t rc = mode == 3 ? (((j & 1) ? roll_hi : roll_lo) >> (4 * (j >> 1))) & 15u
                                  : ((j < 8 ? roll_lo : roll_hi) >> (4 * (j & 7))) & 15u;
    uint32_t code, mk, ybits;
    exact_forward_element(mode, __uint_as_float((uint32_t)x[j] << 16), s, valid, (cached >> j) & 1u, rc, code, mk,
                          ybits, lb);
    maskword |= mk << j;
    y[j] = (uint16_t)ybits;
    cw |= (uint64_t)code << (4 * j);
  }
  mask[b] = (uint16_t)maskword;
  if (qcodes) qcodes[b] = make_uint2((uint32_t)cw, (uint32_t)(cw >> 32));
}

// The same for one half block h (elements 8h..8h+7) of the half-lane
// forward: cached = its 8 bits, roll = its rollout codes (element order).
__device__ __noinline__ void fakequant_half_exact(int mode, const uint4* __restrict__ x4, uint64_t h,
                                                  uint32_t sbyte, float ts, uint32_t cached, uint32_t roll,
                                                  uint4* __restrict__ y4, uint8_t* __restrict__ mask,
                                                  uint32_t* __restrict__ qcodes, LowBitsRule lb = LowBitsRule{}) {
  const float s = e4m3_decode(sbyte) * ts;
  const bool valid = s > 0.f && s <= 3.40282347e38f;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x4) + 8 * h;
  uint16_t* y = reinterpret_cast<uint16_t*>(y4) + 8 * h;
  uint32_t maskbyte = 0, cw = 0;
#pragma unroll 1
  for (int j = 0; j < 8; ++j) {
    uint32_t code, mk, ybits;
    exact_forward_element(mode, __uint_as_float((uint32_t)x[j] << 16), s, valid, (cached >> j) & 1u,
                          (roll >> (4 * j)) & 15u, code, mk, ybits, lb);
    maskbyte |= mk << j;
    y[j] = (uint16_t)ybits;
    cw |= code << (4 * j);
  }
  mask[h] = (uint8_t)maskbyte;
  if (qcodes) qcodes[h] = cw;
}

// ---------------------------------------------------------------------------
// tensor amax: per-workgroup maxima of the bf16 magnitude bits (NaN excluded),
// then one workgroup folds them and forms ts = fl32(amax / 2688).  Integer
// maxima over magnitude bits order non-NaN bf16 values as their absolute
// values do.  NaN halves (magnitude > 0x7f80) are mapped below every other
// value: m + 0x7f stays below 0x8000 exactly for non-NaN halves, so a signed
// 16-bit maximum of m + 0x7f ignores NaN.
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

typedef short s16x2 __attribute__((ext_vector_type(2)));

// The amax and STE kernels have no block structure, so their loads are fully
// coalesced: a 4096-element tile is 512 128-bit vectors and lane t takes
// vectors t and t + 256 (every load instruction covers 1 KiB contiguous).
// The workgroup's partial maximum (bf16 magnitude bits) over tiles g, g + G,
// g + 2G, ... of the tensor.  Tiles below nt_tiles are loaded with the
// non-temporal hint (see launch_tensor_scale).

template <bool kNT>
__device__ __forceinline__ void amax_accumulate(const uint4* __restrict__ x, uint64_t i, s16x2& best) {
  const u32x4* p = reinterpret_cast<const u32x4*>(x) + i;
  const u32x4 v = kNT ? __builtin_nontemporal_load(p) : *p;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t m = (v[k] & 0x7fff7fffu) + 0x007f007fu;  // no carry between halves
    s16x2 vv;
    __builtin_memcpy(&vv, &m, 4);
    best = __builtin_elementwise_max(best, vv);
  }
}

__device__ __forceinline__ uint32_t amax_partial_body(const uint4* __restrict__ x, uint64_t nblocks, uint64_t g,
                                                      uint64_t G, uint64_t nt_tiles = 0) {
  s16x2 best = {0, 0};  // holds max(m + 0x7f) over non-NaN halves, >= 0x7f once any was seen
  const uint64_t nvec = 2 * nblocks;
  for (uint64_t tile = g; tile * 512 < nvec; tile += G) {
    if (tile < nt_tiles) {  // below nt_tiles every tile is whole
#pragma unroll
      for (int h = 0; h < 2; ++h) amax_accumulate<true>(x, tile * 512 + 256 * h + threadIdx.x, best);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint64_t i = tile * 512 + 256 * h + threadIdx.x;
        if (i < nvec) amax_accumulate<false>(x, i, best);
      }
    }
  }
  const int lo = best.x, hi = best.y;
  const int m = lo > hi ? lo : hi;
  const uint32_t r = m > 0x7f ? (uint32_t)(m - 0x7f) : 0u;
  return block_max_u32(r);
}

__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const uint4* __restrict__ x,
                                                                uint64_t nblocks, uint64_t nt_tiles,
                                                                uint32_t* __restrict__ partial) {
  const uint32_t r = amax_partial_body(x, nblocks, blockIdx.x, gridDim.x, nt_tiles);
  if (threadIdx.x == 0) partial[blockIdx.x] = r;
}

// Maximum of words [begin, end) over a workgroup's lanes: every lane issues
// kFoldLoads loads before it waits for any (a loop of single loads waits one
// memory round trip per word).  Indices past the end read the last word
// again, which leaves the maximum unchanged and keeps the loads unconditional.
constexpr int kFoldLoads = 8;

__device__ __forceinline__ uint32_t fold_max_u32(const uint32_t* __restrict__ v, uint64_t begin, uint64_t end) {
  uint32_t best = 0;
  for (uint64_t base = begin; base < end; base += (uint64_t)kFoldLoads * kThreads) {
    uint32_t w[kFoldLoads];
#pragma unroll
    for (int u = 0; u < kFoldLoads; ++u) {
      const uint64_t i = base + (uint64_t)u * kThreads + threadIdx.x;
      w[u] = v[i < end ? i : end - 1];
    }
#pragma unroll
    for (int u = 0; u < kFoldLoads; ++u) best = max(best, w[u]);
  }
  return block_max_u32(best);
}

__global__ __launch_bounds__(kThreads) void amax_finalize_kernel(const uint32_t* __restrict__ partial,
                                                                 uint32_t count, float* __restrict__ ts_out) {
  const uint32_t best = fold_max_u32(partial, 0, count);
  if (threadIdx.x == 0) *ts_out = __uint_as_float(best << 16) / kTensorDiv;
}

// ---------------------------------------------------------------------------
// row groups (per-expert tensor scales of packed MoE rows): group g holds
// rows [off[g], off[g+1]).  Offsets are clamped to [0, rows] when read, so
// any offsets array (even a decreasing one) keeps every access in bounds;
// only nondecreasing offsets give a meaningful assignment.
// ---------------------------------------------------------------------------
struct RowGroups {
  const int64_t* off;  // int64[count + 1]
  uint32_t count;
  uint64_t rows;
  uint64_t bpr;        // 16-element blocks per row
  uint64_t per_block;  // count / blocks in 32.32 fixed point, below 2^32: the group a block
                       // would fall in if all groups were equal
};

__device__ __forceinline__ uint64_t group_row(const RowGroups& G, uint32_t g) {
  const int64_t o = G.off[g];
  return o < 0 ? 0 : ((uint64_t)o > G.rows ? G.rows : (uint64_t)o);
}

// Start of group g in blocks, with group 0 starting at 0 and group count
// (one past the last) at infinity.
__device__ __forceinline__ uint64_t group_start(const RowGroups& G, uint32_t g) {
  if (g == 0) return 0;
  if (g >= G.count) return ~0ull;
  return group_row(G, g) * G.bpr;
}

// Tensor scale of block b's group; b0 is the first block of the tile or
// segment (wave-uniform, b0 <= b).  The group of b0 is found with scalar
// work only: a guess that assumes equal groups (an integer multiply by the
// fixed-point count / blocks, no vector-to-scalar moves), checked against a
// window of three groups whose starts and scales come in one round of
// independent scalar loads (enough for balanced expert loads); otherwise by
// binary search.  Lanes past the next group start (a group boundary inside
// the tile, rare) walk on with per-lane loads.  Computing the guess from a
// lane's block instead (a readfirstlane and float arithmetic before the
// loads) made the per-expert capture 12% slower.  group_at does the
// uniform part (the group holding b0, its scale and where the following
// group starts), group_lane the per-lane one.
struct GroupAt {
  uint32_t lo;    // the group holding b0
  float t;        // its tensor scale
  uint64_t next;  // the block where the following group starts
};

__device__ __forceinline__ GroupAt group_at(const RowGroups& G, const float* __restrict__ ts, uint64_t b0) {
  const uint32_t g0 = (uint32_t)__umul64hi(b0, G.per_block << 32);  // floor(b0 * count / blocks), within 2
  const uint32_t guess = g0 < G.count - 1 ? g0 : G.count - 1;
  uint32_t lo = G.count;  // not found yet
  float t = 0.f;
  uint64_t next = 0;
  if (G.count >= 3) {
    // window: groups i, i + 1, i + 2 around the guess; offsets[i .. i + 3]
    // and ts[i .. i + 2] are in bounds and loaded unconditionally, together
    const uint32_t i = guess == 0 ? 0 : (guess - 1 > G.count - 3 ? G.count - 3 : guess - 1);
    int64_t ov[4];
    float tw[3];
#pragma unroll
    for (int j = 0; j < 4; ++j) ov[j] = G.off[i + j];
#pragma unroll
    for (int j = 0; j < 3; ++j) tw[j] = ts[i + j];
    uint64_t st[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t o = ov[j];
      const uint64_t row = o < 0 ? 0 : ((uint64_t)o > G.rows ? G.rows : (uint64_t)o);
      st[j] = i + j == 0 ? 0 : (i + j >= G.count ? ~0ull : row * G.bpr);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const bool in = st[j] <= b0 && b0 < st[j + 1];
      lo = in ? i + j : lo;
      t = in ? tw[j] : t;
      next = in ? st[j + 1] : next;
    }
  }
  if (lo == G.count) {  // unbalanced groups: binary search
    uint32_t l = 0, h = G.count;
    while (h - l > 1) {
      const uint32_t mid = (l + h) >> 1;
      if (group_row(G, mid) * G.bpr <= b0) l = mid; else h = mid;
    }
    lo = l;
    next = group_start(G, lo + 1);
    t = ts[lo];
  }
  // readfirstlane keeps the uniform value scalar (the compiler would otherwise
  // merge the loads with the per-lane load in group_lane into vector loads)
  return GroupAt{lo, __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(t))), next};
}

// Tensor scale of block b, at or after the block that A was found for.
__device__ __forceinline__ float group_lane(const RowGroups& G, const float* __restrict__ ts, const GroupAt& A,
                                            uint64_t b) {
  float t = A.t;
  if (b >= A.next) {
    uint32_t g = A.lo + 1;
    while (g + 1 < G.count && group_row(G, g + 1) * G.bpr <= b) ++g;
    t = ts[g];
  }
  return t;
}

__device__ __forceinline__ float group_tensor_scale(const RowGroups& G, const float* __restrict__ ts, uint64_t b0,
                                                   uint64_t b) {
  return group_lane(G, ts, group_at(G, ts, b0), b);
}


// Maximum over a wave of non-negative values by DPP (row shifts within each
// 16-lane row, then the row broadcasts of lanes 15 and 31); the result is
// valid in lane 63.  Lanes a shift reaches from outside their row read 0,
// which leaves a maximum of non-negative values unchanged.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));   // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));   // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));   // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));   // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}

// Magnitude-bit maximum of a 128-bit vector's halves folded into best (NaN
// halves map below every other value, as in amax_partial_body).
__device__ __forceinline__ void fold_vec_max(const uint4 v, s16x2& best) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t m = (w[k] & 0x7fff7fffu) + 0x007f007fu;
    s16x2 vv;
    __builtin_memcpy(&vv, &m, 4);
    best = __builtin_elementwise_max(best, vv);
  }
}

__device__ __forceinline__ uint32_t best_to_bits(s16x2 best) {
  const int lo = best.x, hi = best.y;
  const int m = lo > hi ? lo : hi;
  return m > 0x7f ? (uint32_t)(m - 0x7f) : 0u;
}

// Grouped tensor scale, pass 1: the magnitude-bit maximum of every row (NaN
// excluded as in amax_partial_kernel).  Rows of fewer than 256 vectors (2048
// elements): one wave per row, four loads in flight per lane.
__global__ __launch_bounds__(kThreads) void row_amax_kernel(const uint4* __restrict__ x, uint64_t rows,
                                                            uint64_t vec_per_row,
                                                            uint32_t* __restrict__ row_amax) {
  const uint32_t lane = threadIdx.x & 63;
  for (uint64_t r = (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < rows;
       r += (uint64_t)gridDim.x * (kThreads / 64)) {
    s16x2 best = {0, 0};
    for (uint64_t c0 = 0; c0 < vec_per_row; c0 += 4 * 64) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // four loads in flight before any is used
        // past the row's end: its last vector again (a repeat leaves the maximum unchanged)
        const uint64_t c = c0 + 64 * u + lane;
        v[u] = x[r * vec_per_row + (c < vec_per_row ? c : vec_per_row - 1)];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) fold_vec_max(v[u], best);
    }
    const uint32_t rmax = wave_max_dpp(best_to_bits(best));
    if (lane == 63) row_amax[r] = rmax;
  }
}

// Rows of 256 vectors or more: one workgroup per row, lane t loading vectors
// t, t + 256, ... of it.  On the 131072x2048 routed-expert site this streams
// 4-8% faster than a wave per row (one vector per lane in flight, the
// layout the streaming kernels favour): 88 against 91-93 us after a
// read-only pass, 114 against 122-126 us right after a 512 MB writer.
__global__ __launch_bounds__(kThreads) void row_amax_wg_kernel(const uint4* __restrict__ x, uint64_t rows,
                                                               uint64_t vec_per_row,
                                                               uint32_t* __restrict__ row_amax) {
  __shared__ uint32_t red[kThreads / 64];
  for (uint64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    s16x2 best = {0, 0};
    const uint4* row = x + r * vec_per_row;
    for (uint64_t c = threadIdx.x; c < vec_per_row; c += kThreads) fold_vec_max(row[c], best);
    const uint32_t wm = wave_max_dpp(best_to_bits(best));
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = wm;
    __syncthreads();
    if (threadIdx.x == 0) row_amax[r] = max(max(red[0], red[1]), max(red[2], red[3]));
    __syncthreads();  // red is rewritten for the next row
  }
}

// Grouped tensor scale, pass 2: one workgroup per group folds its rows' maxima.
__global__ __launch_bounds__(kThreads) void group_amax_finalize_kernel(const uint32_t* __restrict__ row_amax,
                                                                       RowGroups G, float* __restrict__ ts_out) {
  const uint32_t g = blockIdx.x;
  const uint64_t r0 = g == 0 ? 0 : group_row(G, g);
  const uint64_t r1 = g + 1 == G.count ? G.rows : group_row(G, g + 1);
  const uint32_t best = fold_max_u32(row_amax, r0, r1);
  if (threadIdx.x == 0) ts_out[g] = __uint_as_float(best << 16) / kTensorDiv;
}

// ---------------------------------------------------------------------------
// capture
// ---------------------------------------------------------------------------
// Per-tensor-scale constants of the capture: validity, the range in which the
// block-scale divisions are exact on the fast path, 1/ts as a double word,
// and the v1 bound beyond which the scale byte saturates.
struct CaptureScale {
  float ts, rthi, rtlo, lim;
  bool valid, slow;
};

__device__ __forceinline__ CaptureScale capture_scale(float ts) {
  CaptureScale c;
  c.ts = ts;
  c.valid = ts > 0.f && ts <= 3.40282347e38f;
  c.slow = c.valid && !(ts >= 0x1p-100f && ts <= 0x1p100f);
  c.rthi = 1.0f / (c.valid ? ts : 1.f);
  c.rtlo = __builtin_fmaf(-(c.valid ? ts : 1.f), c.rthi, 1.0f) * c.rthi;
  c.lim = 512.f * ts;  // v1 beyond lim gives v > 448: saturates
  return c;
}

// One block of the capture: scale byte, parity bits and (optionally) codes.
template <bool kPlanes, bool kNT>
__device__ __forceinline__ void capture_one(const uint4* __restrict__ x, uint64_t b, const uint32_t (&w)[8],
                                            const CaptureScale& cs, float r6hi, float r6lo,
                                            uint8_t* __restrict__ scales, uint16_t* __restrict__ bits,
                                            uint2* __restrict__ codes, Planes planes) {
  const float ts = cs.ts;
  // block amax on packed bf16 magnitudes
  u16x2 mx;
  {
    uint32_t m0 = w[0] & 0x7fff7fffu;
    __builtin_memcpy(&mx, &m0, 4);
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      const uint32_t mk = w[k] & 0x7fff7fffu;
      u16x2 v;
      __builtin_memcpy(&v, &mk, 4);
      mx = __builtin_elementwise_max(mx, v);
    }
  }
  const uint32_t amax_bits = mx.x > mx.y ? mx.x : mx.y;
  const float amax = __uint_as_float(amax_bits << 16);
  // a zero block, or amax >= 2^-100 (bf16 bits 0x0d80) keeps the two divisions
  // exact; a NaN or infinite element shows as amax_bits >= 0x7f80
  bool bad = cs.slow || (amax_bits - 1u) < 0x0d7fu || amax_bits >= 0x7f80u;

  const float v1 = __builtin_amdgcn_fmed3f(div_fast_u(amax, 6.0f, r6hi, r6lo), 0.f, cs.lim);
  const float v = div_fast_u(v1, ts, cs.rthi, cs.rtlo);
  uint32_t sb = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(v, 0.f, 448.f), 0.f, 0, false);
  sb = cs.valid ? sb : 0u;

  const ScaleEntry e = make_scale_entry(sb, ts);
  // The first approximation q1 = fma(x, dhi, x*dlo) is monotone in |x|
  // (dhi, dlo >= 0), so the block maximum's bounds every element's.  Below
  // 2^127 every quotient of the block is finite and Markstein's correction
  // applies; at or above it (a saturated scale byte under a small tensor
  // scale with a huge element: |x| / (448 ts) near binary32 overflow), and
  // for a scale outside the fast range (dhi NaN), the block takes the exact
  // path.  No per-element flag is needed.
  bad |= !(__builtin_fmaf(amax, e.dhi, amax * e.dlo) < 0x1p127f);

  float q[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) q[j] = div_fast<false>(block_elem(w, j), e, bad);

  uint32_t E = 0, O = 0;
  FP4_PACK8(FP4_RNE, E, q, 0);
  FP4_PACK8(FP4_RNE, O, q, 1);
  if (bad) {
    capture_block_exact(x, b, ts, scales, bits, codes, kPlanes ? planes : Planes{1, 0});
  } else {
    store_word<kNT>(&scales[b], (uint8_t)sb);
    if (kPlanes) {
      // plane k: bit k of each element's signed grid index (two's complement)
      const uint32_t SE = signed_index_nibbles(E), SO = signed_index_nibbles(O);
      store_word<kNT>(&bits[b], (uint16_t)gather_parity(SE, SO));
#pragma unroll
      for (uint32_t k = 1; k < 4; ++k)
        if (k < planes.count) store_word<kNT>(&bits[b + k * planes.stride], (uint16_t)gather_parity(SE >> k, SO >> k));
    } else {
      store_word<kNT>(&bits[b], (uint16_t)gather_parity(E, O));
    }
    if (codes) {
      uint32_t c0, c1;
      interleave_codes(E, O, c0, c1);
      store_pair<kNT>(&codes[b], make_uint2(c0, c1));
    }
  }
}

template <bool kGrouped, bool kPlanes, bool kNT>
__global__ __launch_bounds__(kThreads) void capture_kernel(const uint4* __restrict__ x, uint64_t nblocks,
                                                           const float* __restrict__ ts_ptr, RowGroups groups,
                                                           uint8_t* __restrict__ scales,
                                                           uint16_t* __restrict__ bits,
                                                           uint2* __restrict__ codes, Planes planes) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  // Tiles are taken from the tensor's end backwards: the tensor amax, which
  // reads the same tensor just before, leaves its last-read lines in the
  // 256 MB last-level cache, and the capture reaches them first.
  uint64_t b0 = (uint64_t)(gridDim.x - 1 - blockIdx.x) * kThreads;  // the tile's first block (uniform)
  uint64_t b = b0 + threadIdx.x;
  if (b >= nblocks) return;
  // The first block's loads go out before the tensor scale is read and its
  // reciprocal formed (a dependent scalar load and a division at kernel
  // entry): 2% faster right after the tensor amax of the same tensor.
  uint32_t w[8];
  load_block(x, b, w);
  __builtin_amdgcn_sched_barrier(0);
  const float r6hi = 1.0f / 6.0f;
  const float r6lo = __builtin_fmaf(-6.0f, r6hi, 1.0f) * r6hi;
  const CaptureScale cs0 = kGrouped ? CaptureScale{} : capture_scale(*ts_ptr);
  for (;;) {
    const CaptureScale cs = kGrouped ? capture_scale(group_tensor_scale(groups, ts_ptr, b0, b)) : cs0;
    capture_one<kPlanes, kNT>(x, b, w, cs, r6hi, r6lo, scales, bits, codes, planes);
    b += stride;
    b0 += stride;
    if (b >= nblocks) break;
    load_block(x, b, w);  // issued before the group search, whose latency it hides
  }
}

// ---------------------------------------------------------------------------
// batches of site tensors (the rollout side of one layer: its activation and
// KV sites in one tensor-scale pass and one capture launch).  Site k owns
// workgroups [wg_begin, wg_begin + wg_count) of the batch grid; a workgroup
// finds its site wave-uniformly from the kernel arguments.  Every site keeps
// its own tensor scale and record, so the results equal per-site calls.
// ---------------------------------------------------------------------------
struct BatchSite {
  const uint4* x;
  uint64_t nblocks;
  float* ts;          // the tensor scale pass writes it; the capture reads it
  uint8_t* scales;
  uint16_t* bits;
  uint2* codes;       // nullable
  uint32_t wg_begin;
  uint32_t wg_count;
  uint64_t nt_tiles;  // tensor scale pass: tiles below it are loaded with the non-temporal hint
  uint32_t nt;        // capture: the record is stored with the non-temporal hint
};

struct BatchSites {
  BatchSite site[trace_host::kMaxBatchSites];
  uint32_t count;
};

// The site whose workgroup range holds workgroup wg: the last site starting
// at or before it (sites without workgroups share their successor's start
// and are passed over).
__device__ __forceinline__ uint32_t batch_site_of(const BatchSites& B, uint32_t wg) {
  uint32_t k = 0;
#pragma unroll
  for (uint32_t i = 1; i < trace_host::kMaxBatchSites; ++i) k = (i < B.count && B.site[i].wg_begin <= wg) ? i : k;
  return k;
}

__global__ __launch_bounds__(kThreads) void amax_partial_batch_kernel(BatchSites B, uint32_t* __restrict__ partial) {
  const BatchSite& S = B.site[batch_site_of(B, blockIdx.x)];
  const uint32_t r = amax_partial_body(S.x, S.nblocks, blockIdx.x - S.wg_begin, S.wg_count, S.nt_tiles);
  if (threadIdx.x == 0) partial[blockIdx.x] = r;
}

// One workgroup per site: the site's tensor scale from its partial maxima (a
// site without workgroups, an empty tensor, gets 0).
__global__ __launch_bounds__(kThreads) void amax_finalize_batch_kernel(BatchSites B,
                                                                       const uint32_t* __restrict__ partial) {
  const BatchSite& S = B.site[blockIdx.x];
  const uint32_t best = fold_max_u32(partial, S.wg_begin, (uint64_t)S.wg_begin + S.wg_count);
  if (threadIdx.x == 0) *S.ts = __uint_as_float(best << 16) / kTensorDiv;
}

// One 256-block tile per workgroup.  The grid is walked from its end, across
// sites and within each site, so the capture first meets the lines the tensor
// scale pass read last.  Each site takes the record stores a capture of it
// alone would (non-temporal past the last-level cache's size).
__global__ __launch_bounds__(kThreads) void capture_batch_kernel(BatchSites B) {
  const uint32_t gw = gridDim.x - 1 - blockIdx.x;
  const BatchSite& S = B.site[batch_site_of(B, gw)];
  const uint64_t b = (uint64_t)(S.wg_count - 1 - (gw - S.wg_begin)) * kThreads + threadIdx.x;
  if (b >= S.nblocks) return;
  uint32_t w[8];
  load_block(S.x, b, w);
  const float r6hi = 1.0f / 6.0f;
  const float r6lo = __builtin_fmaf(-6.0f, r6hi, 1.0f) * r6hi;
  const CaptureScale cs = capture_scale(*S.ts);
  if (S.nt)
    capture_one<false, true>(S.x, b, w, cs, r6hi, r6lo, S.scales, S.bits, S.codes, Planes{1, 0});
  else
    capture_one<false, false>(S.x, b, w, cs, r6hi, r6lo, S.scales, S.bits, S.codes, Planes{1, 0});
}

// ---------------------------------------------------------------------------
// fake-quant forward (guided or plain RNE)
// ---------------------------------------------------------------------------
// One block of a fake-quant forward (the low-bits forward: one lane per
// block).
template <int kMode>
__device__ __forceinline__ void fakequant_one(const uint4* __restrict__ x, uint64_t b, const uint32_t (&w)[8],
                                              uint32_t sbyte, uint32_t cached, uint2 roll, float ts,
                                              uint4* __restrict__ y, uint16_t* __restrict__ mask,
                                              uint2* __restrict__ qcodes,
                                              const LowBitsRule& lb = LowBitsRule{}) {
  const ScaleEntry e = make_scale_entry(sbyte, ts);
  bool bad = false;  // set by a NaN / infinite quotient, or a scale outside the fast range (dhi NaN)

  float q[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) q[j] = div_fast<true>(block_elem(w, j), e, bad);

  uint32_t QE, QO;
  const uint32_t keep = select_codes<kMode>(q, cached, roll, QE, QO, lb);
  const uint32_t maskword = (e.rhi != 0.f) ? keep : 0u;

  if (bad) {
    fakequant_block_exact(kMode, x, b, sbyte, ts, cached, roll.x, roll.y, y, mask, qcodes, lb);
  } else {
    uint32_t out[8];
    decode_block(QE, QO, e.s, out);
    store_block(y, b, out);
    mask[b] = (uint16_t)maskword;
    if (qcodes) {
      uint32_t c0, c1;
      interleave_codes(QE, QO, c0, c1);
      qcodes[b] = make_uint2(c0, c1);
    }
  }
}

// One half block of a fake-quant forward.
template <int kMode, bool kNT>
__device__ __forceinline__ void fakequant_half(const uint4* __restrict__ x, uint64_t h, const uint32_t (&w)[4],
                                               uint32_t sbyte, uint32_t cached, uint32_t roll, float ts,
                                               uint4* __restrict__ y, uint8_t* __restrict__ mask,
                                               uint32_t* __restrict__ qcodes,
                                               const LowBitsRule& lb = LowBitsRule{}) {
  const ScaleEntry e = make_scale_entry(sbyte, ts);
  bool bad = false;  // set by a NaN / infinite quotient, or a scale outside the fast range (dhi NaN)

  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = div_fast<true>(half_elem(w, j), e, bad);

  uint32_t Q;
  const uint32_t keep = select_codes8<kMode>(q, cached, roll, Q, lb);
  const uint32_t maskbyte = (e.rhi != 0.f) ? keep : 0u;

  if (bad) {
    fakequant_half_exact(kMode, x, h, sbyte, ts, cached, roll, y, mask, qcodes, lb);
  } else {
    uint32_t out[4];
    decode_half(Q, e.s, out);
    store_vec<kNT>(&y[h], make_uint4(out[0], out[1], out[2], out[3]));
    store_word<kNT>(&mask[h], (uint8_t)maskbyte);
    if (qcodes) store_word<kNT>(&qcodes[h], Q);
  }
}

// The ungrouped forwards (kMode 0, 1, 2) with one lane per half block (8
// elements, one 128-bit load): ~5% faster than a lane per block, which the
// capture and the low-bits forward (more dependent loads) keep.  Both halves
// of a block read its scale byte.
template <int kMode, bool kNT>
__global__ __launch_bounds__(kThreads) void fakequant_half_kernel(const uint4* __restrict__ x, uint64_t nhalves,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ ts_ptr,
                                                             const uint8_t* __restrict__ bits,
                                                             const uint32_t* __restrict__ rcodes,
                                                             uint4* __restrict__ y,
                                                             uint8_t* __restrict__ mask,
                                                             uint32_t* __restrict__ qcodes) {
  const float ts = *ts_ptr;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t h = (uint64_t)blockIdx.x * kThreads + threadIdx.x; h < nhalves; h += stride) {
    const uint32_t sbyte = scales[h >> 1];
    const uint32_t cached = kMode == 1 ? (uint32_t)bits[h] : 0u;
    const uint32_t roll = kMode == 2 ? rcodes[h] : 0u;
    const uint4 v = load_vec<kNT>(&x[h]);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    fakequant_half<kMode, kNT>(x, h, w, sbyte, cached, roll, ts, y, mask, qcodes);
  }
}

// ---------------------------------------------------------------------------
// trainer-side forward on records read back in the trainer's row order:
// destination row r of x_train takes the record of source row row_index[r]
// (its scale bytes and cached bits or codes, and the tensor scale of its
// group), read in place; no gathered copy of the record is written first.
// An index outside [0, src_rows) gives zero-scale blocks.
// ---------------------------------------------------------------------------
struct GatherMap {
  const int64_t* row_index;  // int64[destination rows]
  uint64_t src_rows;
  uint64_t hpr;              // half blocks (8 elements) per row
  uint64_t inv;              // ceil(2^64 / hpr): h / hpr = mulhi(h, inv) for h * hpr < 2^64
};

// Tensor scale of the group holding source row s, in two steps so that a
// wave can issue the loads for several rows before it waits on any: the
// window (group_window_load) is three groups around a guess that assumes
// equal groups (the fixed-point count / blocks, as in group_at),
// whose four starts and three scales are loaded together, in bounds for any
// s; group_window_pick takes the group holding s from it, or, when s lies
// outside the window (unbalanced groups, or fewer than three), binary
// searches for the last group starting at or before s.  With a
// wave-uniform s the compiler issues scalar loads.
struct GroupWindow {
  uint32_t i;  // first group of the window
  int64_t ov[4];
  float tw[3];
};

__device__ __forceinline__ GroupWindow group_window_load(const RowGroups& G, const float* __restrict__ ts, uint64_t s) {
  GroupWindow w{};
  if (G.count >= 3) {
    const uint32_t g0 = (uint32_t)__umul64hi(s * G.bpr, G.per_block << 32);
    const uint32_t guess = g0 < G.count - 1 ? g0 : G.count - 1;
    w.i = guess == 0 ? 0 : (guess - 1 > G.count - 3 ? G.count - 3 : guess - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) w.ov[j] = G.off[w.i + j];
#pragma unroll
    for (int j = 0; j < 3; ++j) w.tw[j] = ts[w.i + j];
  }
  return w;
}

// For a row s in [0, rows), comparing s with a clamped offset equals
// comparing it with the raw offset as a signed number, so no clamping is
// needed here; group 0 starts at 0 and the last group has no end.
__device__ __forceinline__ float group_window_pick(const RowGroups& G, const float* __restrict__ ts,
                                                   const GroupWindow& w, uint64_t s) {
  const int64_t si = (int64_t)s;
  if (G.count >= 3) {
    float t = 0.f;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const bool in = (w.i + j == 0 || w.ov[j] <= si) && (w.i + j + 1 >= G.count || si < w.ov[j + 1]);
      t = in ? w.tw[j] : t;
      found |= in;
    }
    if (found) return t;
  }
  uint32_t l = 0, h = G.count;  // the last group starting at or before s
  while (h - l > 1) {
    const uint32_t mid = (l + h) >> 1;
    if (G.off[mid] <= si) l = mid; else h = mid;
  }
  return ts[l];
}

__device__ __forceinline__ uint64_t readfirstlane_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Each wave takes kGatherSegs segments of 64 consecutive half blocks of the
// destination (lane t: half t of every segment).  A half block's record
// bytes sit behind two dependent loads (its row's index, then the source
// row's bytes), so a wave issues all its x loads and row-index loads first,
// then all record loads (and group windows), before it computes.  On the
// 131072x2048 routed-expert site in a shuffled row order, after a read-only
// pass: one segment per wave 198-203 us, two 189-194, four 190-199, eight
// 210 (registers); the gather and then the forward take 204-222 us.
// kRows = 1 (half blocks per row a multiple of 64): every segment lies
// inside one row, so its row index, source row and group lookup are scalar
// work, and a segment in the same row as the previous one reuses them
// (per-expert scales on the 2048-wide site: 215-240 -> 187-188 us, with one
// scalar group window live at a time; two live at once spilled registers).
// kRows = 2 (rows of 64 half blocks or more, one tensor scale): a segment
// spans at most two rows; both are looked up as scalar work and each lane
// picks its own (131072x768 site: 89 -> 80 us, where the gather and then
// the forward take 84 us).  Per-expert scales stay per lane there: two
// scalar group windows per segment overflow the scalar registers (49-64
// spilled), and each scalar lookup is ~40 scalar instructions on a unit
// that serves all of a compute unit's waves (87 -> 95 us).  kRows = 0:
// each lane finds its own row.
#ifndef TRACE_GATHER_SEGS
#define TRACE_GATHER_SEGS 2
#endif
constexpr int kGatherSegs = TRACE_GATHER_SEGS;

template <int kMode, bool kGrouped, int kRows, bool kNT>
__global__ __launch_bounds__(kThreads) void fakequant_gathered_kernel(const uint4* __restrict__ x, uint64_t nhalves,
                                                                      GatherMap gm,
                                                                      const uint8_t* __restrict__ scales_src,
                                                                      const float* __restrict__ ts_ptr,
                                                                      RowGroups groups,
                                                                      const uint8_t* __restrict__ bits_src,
                                                                      const uint32_t* __restrict__ codes_src,
                                                                      uint4* __restrict__ y,
                                                                      uint8_t* __restrict__ mask,
                                                                      uint32_t* __restrict__ qcodes) {
  static_assert(!(kGrouped && kRows == 2), "per-expert scales take scalar lookups only for one row per segment");
  constexpr int K = kGatherSegs;
  const float ts0 = kGrouped ? 0.f : *ts_ptr;
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t per_wg = (uint64_t)kThreads * K;
  const uint64_t stride = (uint64_t)gridDim.x * per_wg;
  // the wave's first half block (wave-uniform)
  uint64_t base = readfirstlane_u64((uint64_t)blockIdx.x * per_wg + (uint64_t)(threadIdx.x >> 6) * 64 * K);
  for (; base < nhalves; base += stride) {
    uint4 v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint64_t h = base + 64 * k + lane;
      v[k] = h < nhalves ? load_vec<kNT>(&x[h]) : make_uint4(0u, 0u, 0u, 0u);
    }
    int64_t s[K];  // each lane's source row (-1: none)
    uint64_t c[K];  // each lane's half block within its row
    bool dup[K];    // kRows 1: the segment lies in the same row as the previous one
    // kRows 2: the segment's rows ra and ra + 1 (two: it reaches into the
    // second) and their source rows
    uint64_t ra[K];
    bool two[K];
    int64_t sa[K], sb[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint64_t h0 = base + 64 * k;  // the segment's first half block (wave-uniform)
      const uint64_t h = h0 + lane;
      const int p = k > 0 ? k - 1 : 0;
      dup[k] = false;
      if (kRows == 0) {
        const uint64_t r = __umul64hi(h, gm.inv);  // destination row
        c[k] = h - r * gm.hpr;
        s[k] = h < nhalves ? gm.row_index[r] : -1;
      } else if (kRows == 1) {
        // rows start at segment boundaries and nhalves is a multiple of 64:
        // a live segment has every lane live
        const bool live = h0 < nhalves;
        const uint64_t r = __umul64hi(h0, gm.inv);
        c[k] = h - r * gm.hpr;
        dup[k] = k > 0 && live && h0 - r * gm.hpr >= 64;
        s[k] = dup[k] ? s[p] : (live ? gm.row_index[r] : -1);
      } else {
        const bool live = h0 < nhalves;
        ra[k] = __umul64hi(h0, gm.inv);
        const uint64_t next = (ra[k] + 1) * gm.hpr;  // where the following row starts
        two[k] = live && next < h0 + 64 && next < nhalves;
        // reuse: the previous segment looked up this segment's first row as
        // its own first row, or as its second row
        const bool same_a = k > 0 && live && ra[p] == ra[k];
        const bool prev_b = k > 0 && live && two[p] && ra[p] + 1 == ra[k];
        sa[k] = !live ? -1 : (same_a ? sa[p] : (prev_b ? sb[p] : gm.row_index[ra[k]]));
        sb[k] = two[k] ? gm.row_index[ra[k] + 1] : sa[k];
        const bool second = h >= next;
        s[k] = h >= nhalves ? -1 : (second ? sb[k] : sa[k]);
        c[k] = h - (second ? next : ra[k] * gm.hpr);
      }
    }
    uint32_t sbyte[K], side[K];
    float ts[K];
    bool ok[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      ok[k] = s[k] >= 0 && (uint64_t)s[k] < gm.src_rows;
      sbyte[k] = 0;  // a row the rollout never produced: zero-scale blocks
      side[k] = 0;
      ts[k] = ts0;
      if (ok[k]) {
        const uint64_t sh = (uint64_t)s[k] * gm.hpr + c[k];  // the same half block of the source row
        sbyte[k] = scales_src[sh >> 1];
        if (kMode == 1) side[k] = bits_src[sh];
        if (kMode == 2) side[k] = codes_src[sh];
      }
    }
    if (kGrouped && kRows == 1) {
      // one scalar window at a time (two live at once spilled scalar
      // registers); where rows are 128 half blocks or longer the second
      // segment of a wave always reuses the first one's lookup
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (dup[k]) {
          ts[k] = ts[k > 0 ? k - 1 : 0];
        } else if (ok[k]) {
          const GroupWindow gw = group_window_load(groups, ts_ptr, (uint64_t)s[k]);
          ts[k] = group_window_pick(groups, ts_ptr, gw, (uint64_t)s[k]);
        }
      }
    } else if (kGrouped) {
      // per lane: every window is loaded before any is compared
      GroupWindow gw[K];
#pragma unroll
      for (int k = 0; k < K; ++k) gw[k] = group_window_load(groups, ts_ptr, ok[k] ? (uint64_t)s[k] : 0);
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (ok[k]) ts[k] = group_window_pick(groups, ts_ptr, gw[k], (uint64_t)s[k]);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint64_t h = base + 64 * k + lane;
      if (h < nhalves) {
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        fakequant_half<kMode, kNT>(x, h, w, sbyte[k], kMode == 1 ? side[k] : 0u, kMode == 2 ? side[k] : 0u, ts[k],
                                   y, mask, qcodes);
      }
    }
  }
}

// The per-expert forwards (one tensor scale per group of rows); kMode: 0 =
// RNE, 1 = guided by the cached bit, 2 = full information.  One lane per
// half block, as the ungrouped forwards: a wave takes kGroupedSegs segments
// of 64 consecutive half blocks, so every load and store instruction covers
// whole lines (a lane per block splits each line between two instructions,
// and with the non-temporal hint the second one misses: that layout ran the
// 131072x2048 routed-expert site at 201-202 us with plain accesses, 213-218
// us with the hint, against 184-185 us here, rep after rep; all three modes
// 6-13% faster, within 2% after a read-only pass and on 768-wide rows).  The
// group is found once per segment with scalar work, and a segment that
// starts before the current group's end reuses it; lanes past a group start
// walk on per lane.
constexpr int kGroupedSegs = 2;

template <int kMode, bool kNT>
__global__ __launch_bounds__(kThreads) void fakequant_grouped_half_kernel(const uint4* __restrict__ x,
                                                                          uint64_t nhalves,
                                                                          const uint8_t* __restrict__ scales,
                                                                          const float* __restrict__ ts_ptr,
                                                                          RowGroups groups,
                                                                          const uint8_t* __restrict__ bits,
                                                                          const uint32_t* __restrict__ rcodes,
                                                                          uint4* __restrict__ y,
                                                                          uint8_t* __restrict__ mask,
                                                                          uint32_t* __restrict__ qcodes) {
  constexpr int K = kGroupedSegs;
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t per_wg = (uint64_t)kThreads * K;
  const uint64_t stride = (uint64_t)gridDim.x * per_wg;
  // the wave's first half block (wave-uniform)
  uint64_t base = readfirstlane_u64((uint64_t)blockIdx.x * per_wg + (uint64_t)(threadIdx.x >> 6) * 64 * K);
  for (; base < nhalves; base += stride) {
    uint4 v[K];
    uint32_t sbyte[K], side[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint64_t h = base + 64 * k + lane;
      const bool live = h < nhalves;
      v[k] = live ? load_vec<kNT>(&x[h]) : make_uint4(0u, 0u, 0u, 0u);
      sbyte[k] = live ? (uint32_t)scales[h >> 1] : 0u;
      side[k] = !live ? 0u : (kMode == 1 ? (uint32_t)bits[h] : (kMode == 2 ? rcodes[h] : 0u));
    }
    float ts[K];
    GroupAt at = group_at(groups, ts_ptr, base >> 1);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint64_t b0 = (base + 64 * k) >> 1;  // the segment's first block (uniform)
      if (k > 0 && b0 >= at.next) at = group_at(groups, ts_ptr, b0);
      ts[k] = group_lane(groups, ts_ptr, at, (base + 64 * k + lane) >> 1);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint64_t h = base + 64 * k + lane;
      if (h < nhalves) {
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        fakequant_half<kMode, kNT>(x, h, w, sbyte[k], kMode == 1 ? side[k] : 0u, kMode == 2 ? side[k] : 0u, ts[k],
                                   y, mask, qcodes);
      }
    }
  }
}

// b cached low bits (kMode 3): the residues come from b bit-planes.
__global__ __launch_bounds__(kThreads) void lowbits_fakequant_kernel(const uint4* __restrict__ x, uint64_t nblocks,
                                                                     const uint8_t* __restrict__ scales,
                                                                     const float* __restrict__ ts_ptr,
                                                                     const uint16_t* __restrict__ planes, Planes pl,
                                                                     LowBitsRule lb, uint4* __restrict__ y,
                                                                     uint16_t* __restrict__ mask,
                                                                     uint2* __restrict__ qcodes) {
  const float ts0 = *ts_ptr;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += stride) {
    const uint32_t sbyte = scales[b];
    uint32_t pw[4] = {0, 0, 0, 0};
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k)
      if (k < pl.count) pw[k] = planes[b + k * pl.stride];
    uint32_t w[8];
    load_block(x, b, w);
    uint32_t RE, RO;
    residue_nibbles(pw, pl.count, RE, RO);
    fakequant_one<3>(x, b, w, sbyte, 0u, make_uint2(RE, RO), ts0, y, mask, qcodes, lb);
  }
}

// ---------------------------------------------------------------------------
// STE backward
// ---------------------------------------------------------------------------
// The tile of workgroup w among G: the hardware hands workgroup w to XCD
// w % 8, so in dispatch order each XCD streams every eighth tile.  Within
// each group of 8 * 256 workgroups this gives XCD x runs of 256 consecutive
// tiles instead; workgroups past the last whole group keep their own tile.
// A permutation of [0, G) for every G.
__device__ __forceinline__ uint32_t xcd_run_tile(uint32_t w, uint32_t G) {
  constexpr uint32_t kRun = 256, kGroup = 8 * kRun;
  if (w >= G - G % kGroup) return w;
  const uint32_t j = w / 8, x = w % 8;
  return ((j / kRun) * 8 + x) * kRun + j % kRun;
}

// One 128-bit vector (8 elements, whose mask bits are byte i of the mask)
// per lane: a lane with one load and one store in flight streams ~5% faster
// than a lane moving two vectors, for copies as for this kernel.  Tiles go to
// XCDs in runs (xcd_run_tile): on 20 layers of 262144x2048 in the step order
// 338-341 us against 346-348 us in dispatch order, with identical outputs.
// The forwards and the capture keep dispatch order (the same mapping left
// them level or slower).
template <bool kNT>
__global__ __launch_bounds__(kThreads) void ste_bwd_kernel(const uint4* __restrict__ g, uint64_t nblocks,
                                                           const uint16_t* __restrict__ mask16,
                                                           uint4* __restrict__ gin) {
  const uint8_t* mask = reinterpret_cast<const uint8_t*>(mask16);
  const uint64_t nvec = 2 * nblocks;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  const uint32_t tile = xcd_run_tile(blockIdx.x, gridDim.x);
  for (uint64_t i = (uint64_t)tile * kThreads + threadIdx.x; i < nvec; i += stride) {
    const uint32_t m = mask[i];
    const uint4 v = load_vec<kNT>(&g[i]);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t keep = (((m >> (2 * k)) & 1u) ? 0x0000ffffu : 0u) |
                            (((m >> (2 * k + 1)) & 1u) ? 0xffff0000u : 0u);
      w[k] &= keep;
    }
    store_vec<kNT>(&gin[i], make_uint4(w[0], w[1], w[2], w[3]));
  }
}

// ---------------------------------------------------------------------------
// record gather (trainer-side readback): destination row r <- source row
// row_index[r] of one record plane (bits, scale bytes or codes), moved in
// words of type V.  A workgroup covers whole rows: with wpr words per row,
// thread t copies word t % wpr of row t / wpr (rows_per_wg = 256 / wpr rows),
// or, for rows of 256 words or more, one row in 256-word strides.  An index
// outside [0, src_rows) writes a zero row (zero-scale blocks).
// ---------------------------------------------------------------------------
template <typename V>
__device__ __forceinline__ V zero_word() {
  V z;
  __builtin_memset(&z, 0, sizeof(V));
  return z;
}

template <typename V>
__global__ __launch_bounds__(kThreads) void gather_plane_kernel(const V* __restrict__ src, V* __restrict__ dst,
                                                                uint64_t src_rows, uint64_t dst_rows, uint32_t wpr,
                                                                uint32_t rows_per_wg,
                                                                const int64_t* __restrict__ row_index) {
  const uint32_t lr = wpr >= kThreads ? 0u : threadIdx.x / wpr;
  if (lr >= rows_per_wg) return;
  const uint32_t w0 = threadIdx.x - lr * (wpr >= kThreads ? 0u : wpr);
  const uint32_t wstep = wpr >= kThreads ? kThreads : wpr;
  for (uint64_t r = (uint64_t)blockIdx.x * rows_per_wg + lr; r < dst_rows; r += (uint64_t)gridDim.x * rows_per_wg) {
    const int64_t s = row_index[r];
    const bool ok = s >= 0 && (uint64_t)s < src_rows;
    for (uint32_t w = w0; w < wpr; w += wstep)
      dst[r * wpr + w] = ok ? src[(uint64_t)s * wpr + w] : zero_word<V>();
  }
}

// All planes of a record in one launch, when every plane moves in 16-byte
// words (row widths and base addresses multiples of 16): workgroups
// [first[k], first[k+1]) gather plane k, one pass over the destination rows
// each, so the planes' short transfers share one ramp-up and one drain.
// A lane moves the same word of kGatherRows rows, rpw rows apart: it issues
// their row-index loads, then their source loads, before it stores, so the
// two dependent loads per word overlap across the rows.
#ifndef TRACE_GATHER_ROWS
#define TRACE_GATHER_ROWS 4
#endif
constexpr int kGatherRows = TRACE_GATHER_ROWS;

struct GatherPlane {
  const uint4* src;
  uint4* dst;
  uint32_t wpr;    // 16-byte words per row
  uint32_t rpw;    // rows per workgroup and repetition (1 for rows of 256 words or more)
  uint32_t first;  // first workgroup of this plane
};
struct GatherPlanes {
  GatherPlane p[3];
  uint32_t count;
};

__global__ __launch_bounds__(kThreads) void gather_planes_kernel(GatherPlanes P, uint64_t src_rows,
                                                                 uint64_t dst_rows,
                                                                 const int64_t* __restrict__ row_index) {
  constexpr int J = kGatherRows;
  const uint32_t k = (P.count > 2 && blockIdx.x >= P.p[2].first) ? 2u
                     : (P.count > 1 && blockIdx.x >= P.p[1].first) ? 1u : 0u;
  const GatherPlane g = P.p[k];
  const uint32_t lr = g.wpr >= kThreads ? 0u : threadIdx.x / g.wpr;
  if (lr >= g.rpw) return;
  const uint64_t base = (uint64_t)(blockIdx.x - g.first) * g.rpw * J + lr;  // row of repetition 0
  const uint32_t w0 = threadIdx.x - lr * (g.wpr >= kThreads ? 0u : g.wpr);
  const uint32_t wstep = g.wpr >= kThreads ? kThreads : g.wpr;
  int64_t s[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint64_t r = base + (uint64_t)j * g.rpw;
    s[j] = r < dst_rows ? row_index[r] : -1;
  }
  for (uint32_t w = w0; w < g.wpr; w += wstep) {
    uint4 v[J];
#pragma unroll
    for (int j = 0; j < J; ++j)
      v[j] = (s[j] >= 0 && (uint64_t)s[j] < src_rows) ? g.src[(uint64_t)s[j] * g.wpr + w] : zero_word<uint4>();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint64_t r = base + (uint64_t)j * g.rpw;
      if (r < dst_rows) g.dst[r * g.wpr + w] = v[j];
    }
  }
}

}  // namespace trace_dev

// ---------------------------------------------------------------------------
// launchers (host)
// ---------------------------------------------------------------------------
namespace trace_host {

using namespace trace_dev;

static unsigned grid_for(uint64_t nblocks) {
  const uint64_t g = (nblocks + kThreads - 1) / kThreads;
  return (unsigned)(g < kMaxGroups ? g : kMaxGroups);
}

// MI355X's memory-side last-level cache.  A kernel whose input stream is
// larger moves it, and its outputs, with the non-temporal hint (load_vec,
// store_vec): the forwards and the STE backward read x and write y, the mask
// and gin that way, the capture writes its record that way (its loads stay
// plain: it reads the tensor amax's kept tail from the cache).  Measured on
// 20 layers of 262144x2048 in the step order (rollout side, then training
// side), with identical outputs: guided forward 376 -> 366 us, RNE 361 ->
// 341 us, STE backward 364 -> 345 us, and the tensor amax after a capture
// with a non-temporal record 172 -> 161 us; the step 29.3 -> 28.1 ms.
// Smaller tensors keep plain accesses (past_cache, launch.h).
constexpr uint64_t kLastLevelCacheBytes = 256ull << 20;

uint32_t amax_partial_count(uint64_t nblocks) {
  const uint64_t g = (nblocks + kThreads - 1) / kThreads;
  return (uint32_t)(g < kAmaxMaxGroups ? (g == 0 ? 1 : g) : kAmaxMaxGroups);
}

// The tensor amax streams the tensor with the non-temporal hint except its
// last kAmaxKeepBytes, which it reads last and leaves in the 256 MB
// last-level cache for the capture (which walks the same tensor from its
// end).  After a large writer, the cache's dirty lines are written back
// while the next kernel streams; non-temporal loads leave them to the
// capture.  Measured on 262144x2048 layers with each layer's kernels in
// turn, right after a 1 GiB plain writer: the amax 201.6 -> 189.0 us, the
// capture 194.8 -> 195.5 us, the step -0.7%; a smaller kept tail speeds the
// amax further but slows the capture by more (0 bytes: 158.7 / 222.5 us),
// and tensors of up to 256 MiB are unchanged.  In the phase-ordered step
// the amax follows the previous layer's capture, whose non-temporal record
// leaves no dirty lines, and runs at the read ceiling (~162 us).
constexpr uint64_t kAmaxKeepBytes = kLastLevelCacheBytes;

// Tiles (8 KiB) of an nblocks tensor that the tensor amax loads with the
// non-temporal hint: all but the kept tail, never the last (partial) tile.
static uint64_t amax_nt_tiles(uint64_t nblocks) {
  const uint64_t tiles = (nblocks + kThreads - 1) / kThreads;
  const uint64_t keep = kAmaxKeepBytes / (2 * 16 * kThreads);
  return tiles > keep ? tiles - keep : 0ull;
}

hipError_t launch_tensor_scale(const uint16_t* x, uint64_t nblocks, uint32_t* partial, float* ts_out,
                               hipStream_t stream) {
  const uint32_t groups = amax_partial_count(nblocks);
  if (nblocks > 0)
    hipLaunchKernelGGL(amax_partial_kernel, dim3(groups), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), nblocks, amax_nt_tiles(nblocks), partial);
  hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(kThreads), 0, stream, partial,
                     nblocks > 0 ? groups : 0u, ts_out);
  return hipGetLastError();
}

// Workgroups of each site in the batch tensor-scale pass: one per tile when
// all tiles fit in kAmaxMaxGroups, otherwise that budget shared in
// proportion to the sites' tiles (at least one workgroup per non-empty site).
static void batch_amax_split(const BatchSiteSpec* sites, uint32_t count, uint32_t* wg) {
  uint64_t total = 0;
  for (uint32_t i = 0; i < count; ++i) total += (sites[i].nblocks + kThreads - 1) / kThreads;
  for (uint32_t i = 0; i < count; ++i) {
    const uint64_t t = (sites[i].nblocks + kThreads - 1) / kThreads;
    uint64_t g = t;
    if (total > kAmaxMaxGroups && t > 0) {
      g = (uint64_t)kAmaxMaxGroups * t / total;
      g = g < 1 ? 1 : (g > t ? t : g);
    }
    wg[i] = (uint32_t)g;
  }
}

uint32_t batch_amax_partial_count(const BatchSiteSpec* sites, uint32_t count) {
  uint32_t wg[kMaxBatchSites];
  batch_amax_split(sites, count, wg);
  uint32_t total = 0;
  for (uint32_t i = 0; i < count; ++i) total += wg[i];
  return total;
}

static BatchSites batch_sites(const BatchSiteSpec* sites, uint32_t count, const uint32_t* wg) {
  BatchSites B{};
  B.count = count;
  uint32_t begin = 0;
  for (uint32_t i = 0; i < count; ++i) {
    B.site[i] = BatchSite{reinterpret_cast<const uint4*>(sites[i].x), sites[i].nblocks, sites[i].ts,
                          sites[i].scales, reinterpret_cast<uint16_t*>(sites[i].bits),
                          reinterpret_cast<uint2*>(sites[i].codes), begin, wg[i],
                          amax_nt_tiles(sites[i].nblocks), past_cache(sites[i].nblocks * 32) ? 1u : 0u};
    begin += wg[i];
  }
  return B;
}

hipError_t launch_tensor_scale_batch(const BatchSiteSpec* sites, uint32_t count, uint32_t* partial,
                                     hipStream_t stream) {
  if (count == 0) return hipSuccess;
  uint32_t wg[kMaxBatchSites];
  batch_amax_split(sites, count, wg);
  const BatchSites B = batch_sites(sites, count, wg);
  const uint32_t total = batch_amax_partial_count(sites, count);
  if (total > 0)
    hipLaunchKernelGGL(amax_partial_batch_kernel, dim3(total), dim3(kThreads), 0, stream, B, partial);
  hipLaunchKernelGGL(amax_finalize_batch_kernel, dim3(count), dim3(kThreads), 0, stream, B,
                     static_cast<const uint32_t*>(partial));
  return hipGetLastError();
}

hipError_t launch_capture_batch(const BatchSiteSpec* sites, uint32_t count, hipStream_t stream) {
  uint32_t wg[kMaxBatchSites];
  uint64_t total = 0;
  for (uint32_t i = 0; i < count; ++i) {
    const uint64_t t = (sites[i].nblocks + kThreads - 1) / kThreads;
    wg[i] = (uint32_t)(t < kMaxGroups ? t : kMaxGroups);
    total += t;
  }
  if (total == 0) return hipSuccess;  // an empty grid is not a valid launch
  if (total > kMaxGroups) {           // too many tiles for one grid: one launch per site
    for (uint32_t i = 0; i < count; ++i) {
      const hipError_t e = launch_capture(sites[i].x, sites[i].nblocks, sites[i].ts, nullptr, sites[i].scales,
                                          sites[i].bits, sites[i].codes, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const BatchSites B = batch_sites(sites, count, wg);
  hipLaunchKernelGGL(capture_batch_kernel, dim3((unsigned)total), dim3(kThreads), 0, stream, B);
  return hipGetLastError();
}

static RowGroups row_groups(const GroupSpec& g, uint64_t nblocks = 0) {
  // count / blocks in 32.32 fixed point, kept below 2^32 (more groups than
  // blocks: the guess is then off and the binary search finds the group)
  uint64_t fx = 0;
  if (nblocks) {
    const unsigned __int128 q = ((unsigned __int128)g.count << 32) / nblocks;
    fx = q < 0xffffffffull ? (uint64_t)q : 0xffffffffull;
  }
  return RowGroups{g.offsets, (uint32_t)g.count, g.rows, g.cols / 16, fx};
}

hipError_t launch_grouped_tensor_scale(const uint16_t* x, const GroupSpec& g, uint32_t* row_amax, float* ts_out,
                                       hipStream_t stream) {
  const uint64_t rows_per_group = kThreads / 64;
  const uint64_t wg = (g.rows + rows_per_group - 1) / rows_per_group;
  const uint64_t vpr = g.cols / 8;
  if (g.rows > 0 && vpr >= kThreads)
    hipLaunchKernelGGL(row_amax_wg_kernel, dim3((unsigned)(g.rows < kMaxGroups ? g.rows : kMaxGroups)),
                       dim3(kThreads), 0, stream, reinterpret_cast<const uint4*>(x), g.rows, vpr, row_amax);
  else if (g.rows > 0)  // every row gets its word, also rows of zero width
    hipLaunchKernelGGL(row_amax_kernel, dim3((unsigned)(wg < kMaxGroups ? wg : kMaxGroups)), dim3(kThreads), 0,
                       stream, reinterpret_cast<const uint4*>(x), g.rows, vpr, row_amax);
  hipLaunchKernelGGL(group_amax_finalize_kernel, dim3((unsigned)g.count), dim3(kThreads), 0, stream, row_amax,
                     row_groups(g), ts_out);
  return hipGetLastError();
}

template <bool kGrouped, bool kPlanes>
static void launch_capture_t(bool nt, const uint4* xv, uint64_t nblocks, const float* ts, const RowGroups& rg,
                             uint8_t* scales, uint16_t* bv, uint2* cv, const Planes& pl, hipStream_t stream) {
  const dim3 grid(grid_for(nblocks)), block(kThreads);
  if (nt)
    hipLaunchKernelGGL((capture_kernel<kGrouped, kPlanes, true>), grid, block, 0, stream, xv, nblocks, ts, rg,
                       scales, bv, cv, pl);
  else
    hipLaunchKernelGGL((capture_kernel<kGrouped, kPlanes, false>), grid, block, 0, stream, xv, nblocks, ts, rg,
                       scales, bv, cv, pl);
}

hipError_t launch_capture(const uint16_t* x, uint64_t nblocks, const float* ts, const GroupSpec* g,
                          uint8_t* scales, uint8_t* bits, uint8_t* codes, hipStream_t stream, uint32_t nplanes) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint16_t* bv = reinterpret_cast<uint16_t*>(bits);
  uint2* cv = reinterpret_cast<uint2*>(codes);
  const Planes pl{nplanes, nblocks};
  const bool nt = past_cache(nblocks * 32);
  if (g)
    launch_capture_t<true, false>(nt, xv, nblocks, ts, row_groups(*g, nblocks), scales, bv, cv, pl, stream);
  else if (nplanes > 1)
    launch_capture_t<false, true>(nt, xv, nblocks, ts, RowGroups{}, scales, bv, cv, pl, stream);
  else
    launch_capture_t<false, false>(nt, xv, nblocks, ts, RowGroups{}, scales, bv, cv, pl, stream);
  return hipGetLastError();
}

hipError_t launch_lowbits_fakequant(const uint16_t* x, uint64_t nblocks, const uint8_t* scales, const float* ts,
                                    const uint8_t* planes, uint32_t nplanes, uint16_t* y, uint8_t* mask,
                                    uint8_t* qcodes, hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  hipLaunchKernelGGL(lowbits_fakequant_kernel, dim3(grid_for(nblocks)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(x), nblocks, scales, ts,
                     reinterpret_cast<const uint16_t*>(planes), Planes{nplanes, nblocks},
                     LowBitsRule{(1u << nplanes) - 1u, 1u << (nplanes - 1)},
                     reinterpret_cast<uint4*>(y), reinterpret_cast<uint16_t*>(mask), reinterpret_cast<uint2*>(qcodes));
  return hipGetLastError();
}

// Per-expert forwards: one lane per half block, kGroupedSegs segments per wave.
template <bool kNT>
static void launch_fakequant_grouped_t(int mode, const uint4* xv, uint64_t nblocks, const uint8_t* scales,
                                       const float* ts, const RowGroups& rg, const uint8_t* side, uint4* yv,
                                       uint8_t* mask, uint32_t* qv, hipStream_t stream) {
  const uint64_t nhalves = 2 * nblocks;
  const dim3 grid(grid_for((nhalves + kGroupedSegs - 1) / kGroupedSegs)), block(kThreads);
  if (mode == 1)
    hipLaunchKernelGGL((fakequant_grouped_half_kernel<1, kNT>), grid, block, 0, stream, xv, nhalves, scales, ts, rg,
                       side, static_cast<const uint32_t*>(nullptr), yv, mask, qv);
  else if (mode == 2)
    hipLaunchKernelGGL((fakequant_grouped_half_kernel<2, kNT>), grid, block, 0, stream, xv, nhalves, scales, ts, rg,
                       static_cast<const uint8_t*>(nullptr), reinterpret_cast<const uint32_t*>(side), yv, mask, qv);
  else
    hipLaunchKernelGGL((fakequant_grouped_half_kernel<0, kNT>), grid, block, 0, stream, xv, nhalves, scales, ts, rg,
                       static_cast<const uint8_t*>(nullptr), static_cast<const uint32_t*>(nullptr), yv, mask, qv);
}

// Ungrouped forwards: one lane per half block (grid over 2 * nblocks lanes).
template <bool kNT>
static void launch_fakequant_half_t(int mode, const uint4* xv, uint64_t nblocks, const uint8_t* scales,
                                    const float* ts, const uint8_t* side, uint4* yv, uint8_t* mask, uint32_t* qv,
                                    hipStream_t stream) {
  const uint64_t nhalves = 2 * nblocks;
  const dim3 grid(grid_for(nhalves)), block(kThreads);
  if (mode == 1)
    hipLaunchKernelGGL((fakequant_half_kernel<1, kNT>), grid, block, 0, stream, xv, nhalves, scales, ts, side,
                       static_cast<const uint32_t*>(nullptr), yv, mask, qv);
  else if (mode == 2)
    hipLaunchKernelGGL((fakequant_half_kernel<2, kNT>), grid, block, 0, stream, xv, nhalves, scales, ts,
                       static_cast<const uint8_t*>(nullptr), reinterpret_cast<const uint32_t*>(side), yv, mask, qv);
  else
    hipLaunchKernelGGL((fakequant_half_kernel<0, kNT>), grid, block, 0, stream, xv, nhalves, scales, ts,
                       static_cast<const uint8_t*>(nullptr), static_cast<const uint32_t*>(nullptr), yv, mask, qv);
}

hipError_t launch_fakequant(int mode, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                            const float* ts, const GroupSpec* g, const uint8_t* side, uint16_t* y, uint8_t* mask,
                            uint8_t* qcodes, hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint4* yv = reinterpret_cast<uint4*>(y);
  uint32_t* q1 = reinterpret_cast<uint32_t*>(qcodes);
  const bool nt = past_cache(nblocks * 32);
  if (g && nt)
    launch_fakequant_grouped_t<true>(mode, xv, nblocks, scales, ts, row_groups(*g, nblocks), side, yv, mask, q1, stream);
  else if (g)
    launch_fakequant_grouped_t<false>(mode, xv, nblocks, scales, ts, row_groups(*g, nblocks), side, yv, mask, q1, stream);
  else if (nt)
    launch_fakequant_half_t<true>(mode, xv, nblocks, scales, ts, side, yv, mask, q1, stream);
  else
    launch_fakequant_half_t<false>(mode, xv, nblocks, scales, ts, side, yv, mask, q1, stream);
  return hipGetLastError();
}

template <int kMode, bool kGrouped, int kRows, bool kNT>
static void launch_gathered_rows(dim3 grid, const uint4* x, uint64_t nhalves, const GatherMap& gm,
                                 const uint8_t* scales_src, const float* ts, const RowGroups& rg,
                                 const uint8_t* side_src, uint4* y, uint8_t* mask, uint32_t* qcodes,
                                 hipStream_t stream) {
  const uint8_t* bits = kMode == 1 ? side_src : nullptr;
  const uint32_t* codes = kMode == 2 ? reinterpret_cast<const uint32_t*>(side_src) : nullptr;
  hipLaunchKernelGGL((fakequant_gathered_kernel<kMode, kGrouped, kRows, kNT>), grid, dim3(kThreads), 0, stream, x,
                     nhalves, gm, scales_src, ts, rg, bits, codes, y, mask, qcodes);
}

// The row mode: 1 when every 64-half segment lies inside one row, 2 when it
// spans at most two (one tensor scale only), else 0 (per lane).
template <int kMode, bool kGrouped, bool kNT>
static void launch_gathered_mode(dim3 grid, uint64_t hpr, const uint4* x, uint64_t nhalves, const GatherMap& gm,
                                 const uint8_t* scales_src, const float* ts, const RowGroups& rg,
                                 const uint8_t* side_src, uint4* y, uint8_t* mask, uint32_t* qcodes,
                                 hipStream_t stream) {
  if (hpr % 64 == 0)
    launch_gathered_rows<kMode, kGrouped, 1, kNT>(grid, x, nhalves, gm, scales_src, ts, rg, side_src, y, mask, qcodes,
                                                  stream);
  else if (!kGrouped && hpr >= 64)
    launch_gathered_rows<kMode, false, 2, kNT>(grid, x, nhalves, gm, scales_src, ts, rg, side_src, y, mask, qcodes,
                                               stream);
  else
    launch_gathered_rows<kMode, kGrouped, 0, kNT>(grid, x, nhalves, gm, scales_src, ts, rg, side_src, y, mask, qcodes,
                                                  stream);
}

template <int kMode, bool kGrouped>
static void launch_gathered_nt(bool nt, dim3 grid, uint64_t hpr, const uint4* x, uint64_t nhalves,
                               const GatherMap& gm, const uint8_t* scales_src, const float* ts, const RowGroups& rg,
                               const uint8_t* side_src, uint4* y, uint8_t* mask, uint32_t* qcodes,
                               hipStream_t stream) {
  if (nt)
    launch_gathered_mode<kMode, kGrouped, true>(grid, hpr, x, nhalves, gm, scales_src, ts, rg, side_src, y, mask,
                                                qcodes, stream);
  else
    launch_gathered_mode<kMode, kGrouped, false>(grid, hpr, x, nhalves, gm, scales_src, ts, rg, side_src, y, mask,
                                                 qcodes, stream);
}

hipError_t launch_gathered_fakequant(int mode, const uint16_t* x, uint64_t rows, uint64_t cols,
                                     const int64_t* row_index, uint64_t src_rows, const GroupSpec* g,
                                     const uint8_t* scales_src, const float* ts, const uint8_t* side_src, uint16_t* y,
                                     uint8_t* mask, uint8_t* qcodes, hipStream_t stream) {
  const uint64_t hpr = cols / 8, nhalves = rows * hpr;
  if (nhalves == 0) return hipSuccess;  // an empty grid is not a valid launch
  const unsigned __int128 two64 = (unsigned __int128)1 << 64;
  const GatherMap gm{row_index, src_rows, hpr, (uint64_t)((two64 + hpr - 1) / hpr)};
  const RowGroups rg = g ? row_groups(*g, g->rows * (g->cols / 16)) : RowGroups{};
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint4* yv = reinterpret_cast<uint4*>(y);
  uint32_t* qv = reinterpret_cast<uint32_t*>(qcodes);
  const dim3 grid(grid_for((nhalves + kGatherSegs - 1) / kGatherSegs));
  const bool nt = past_cache(nhalves * 16);
  if (mode == 0 && g)
    launch_gathered_nt<0, true>(nt, grid, hpr, xv, nhalves, gm, scales_src, ts, rg, side_src, yv, mask, qv, stream);
  else if (mode == 0)
    launch_gathered_nt<0, false>(nt, grid, hpr, xv, nhalves, gm, scales_src, ts, rg, side_src, yv, mask, qv, stream);
  else if (mode == 1 && g)
    launch_gathered_nt<1, true>(nt, grid, hpr, xv, nhalves, gm, scales_src, ts, rg, side_src, yv, mask, qv, stream);
  else if (mode == 1)
    launch_gathered_nt<1, false>(nt, grid, hpr, xv, nhalves, gm, scales_src, ts, rg, side_src, yv, mask, qv, stream);
  else if (g)
    launch_gathered_nt<2, true>(nt, grid, hpr, xv, nhalves, gm, scales_src, ts, rg, side_src, yv, mask, qv, stream);
  else
    launch_gathered_nt<2, false>(nt, grid, hpr, xv, nhalves, gm, scales_src, ts, rg, side_src, yv, mask, qv, stream);
  return hipGetLastError();
}

hipError_t launch_ste_bwd(const uint16_t* g, const uint8_t* mask, uint64_t nblocks, uint16_t* gin,
                          hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const dim3 grid(grid_for(2 * nblocks)), block(kThreads);
  const uint4* gv = reinterpret_cast<const uint4*>(g);
  const uint16_t* mv = reinterpret_cast<const uint16_t*>(mask);
  uint4* iv = reinterpret_cast<uint4*>(gin);
  if (past_cache(nblocks * 32))
    hipLaunchKernelGGL(ste_bwd_kernel<true>, grid, block, 0, stream, gv, nblocks, mv, iv);
  else
    hipLaunchKernelGGL(ste_bwd_kernel<false>, grid, block, 0, stream, gv, nblocks, mv, iv);
  return hipGetLastError();
}

template <typename V>
static void launch_gather_plane_t(const uint8_t* src, uint8_t* dst, uint64_t src_rows, uint64_t dst_rows,
                                  uint64_t row_bytes, const int64_t* row_index, hipStream_t stream) {
  const uint32_t wpr = (uint32_t)(row_bytes / sizeof(V));
  const uint32_t rpw = wpr >= (uint32_t)kThreads ? 1u : (uint32_t)kThreads / wpr;
  const uint64_t wg = (dst_rows + rpw - 1) / rpw;
  hipLaunchKernelGGL(gather_plane_kernel<V>, dim3((unsigned)(wg < kMaxGroups ? wg : kMaxGroups)), dim3(kThreads), 0,
                     stream, reinterpret_cast<const V*>(src), reinterpret_cast<V*>(dst), src_rows, dst_rows, wpr, rpw,
                     row_index);
}

// The widest word that divides the row and keeps both planes aligned.
static void launch_gather_plane(const uint8_t* src, uint8_t* dst, uint64_t src_rows, uint64_t dst_rows,
                                uint64_t row_bytes, const int64_t* row_index, hipStream_t stream) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | (uintptr_t)row_bytes;
  if ((a & 15) == 0)
    launch_gather_plane_t<uint4>(src, dst, src_rows, dst_rows, row_bytes, row_index, stream);
  else if ((a & 7) == 0)
    launch_gather_plane_t<uint2>(src, dst, src_rows, dst_rows, row_bytes, row_index, stream);
  else if ((a & 3) == 0)
    launch_gather_plane_t<uint32_t>(src, dst, src_rows, dst_rows, row_bytes, row_index, stream);
  else if ((a & 1) == 0)
    launch_gather_plane_t<uint16_t>(src, dst, src_rows, dst_rows, row_bytes, row_index, stream);
  else
    launch_gather_plane_t<uint8_t>(src, dst, src_rows, dst_rows, row_bytes, row_index, stream);
}

// One launch for every plane when all move in 16-byte words and one pass
// fits the grid limit; otherwise one launch per plane with its widest word.
static bool launch_gather_fused(const uint8_t* const (&src)[3], uint8_t* const (&dst)[3], const uint64_t (&row_bytes)[3],
                                uint32_t nplanes, uint64_t src_rows, uint64_t dst_rows, const int64_t* row_index,
                                hipStream_t stream) {
  GatherPlanes P{};
  uint64_t wg = 0;
  for (uint32_t k = 0; k < nplanes; ++k) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(src[k]) | reinterpret_cast<uintptr_t>(dst[k]) |
                        (uintptr_t)row_bytes[k];
    if ((a & 15) != 0) return false;
    const uint64_t wpr = row_bytes[k] / 16;
    const uint64_t rpw = wpr >= kThreads ? 1 : kThreads / wpr;
    if (wpr > 0xffffffffull) return false;
    P.p[k] = GatherPlane{reinterpret_cast<const uint4*>(src[k]), reinterpret_cast<uint4*>(dst[k]), (uint32_t)wpr,
                         (uint32_t)rpw, (uint32_t)wg};
    wg += (dst_rows + rpw * kGatherRows - 1) / (rpw * kGatherRows);
    if (wg > kMaxGroups) return false;
  }
  P.count = nplanes;
  hipLaunchKernelGGL(gather_planes_kernel, dim3((unsigned)wg), dim3(kThreads), 0, stream, P, src_rows, dst_rows,
                     row_index);
  return true;
}

hipError_t launch_gather_records(const uint8_t* bits_src, const uint8_t* scales_src, const uint8_t* codes_src,
                                 uint64_t src_rows, uint64_t cols, const int64_t* row_index, uint64_t dst_rows,
                                 uint8_t* bits_dst, uint8_t* scales_dst, uint8_t* codes_dst, hipStream_t stream) {
  if (dst_rows == 0 || cols == 0) return hipSuccess;  // nothing to move
  const uint8_t* const src[3] = {bits_src, scales_src, codes_src};
  uint8_t* const dst[3] = {bits_dst, scales_dst, codes_dst};
  const uint64_t row_bytes[3] = {cols / 8, cols / 16, cols / 2};
  if (launch_gather_fused(src, dst, row_bytes, codes_dst ? 3u : 2u, src_rows, dst_rows, row_index, stream))
    return hipGetLastError();
  launch_gather_plane(bits_src, bits_dst, src_rows, dst_rows, cols / 8, row_index, stream);
  launch_gather_plane(scales_src, scales_dst, src_rows, dst_rows, cols / 16, row_index, stream);
  if (codes_dst) launch_gather_plane(codes_src, codes_dst, src_rows, dst_rows, cols / 2, row_index, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// allocation-free tensor scale: the partial maxima live in the library's own
// device array instead of a caller's workspace
// ---------------------------------------------------------------------------
}  // namespace trace_host

// One partial maximum per workgroup of the capped tensor-scale grid.  Every
// GPU the library runs on holds its own copy until the process ends.  In
// host code this name is a host-side stand-in, never a device address: host
// code uses only the address hipGetSymbolAddress returns for the device.
static __device__ __align__(256) uint32_t scratch[trace_host::kAmaxMaxGroups];

namespace trace_host {

constexpr int kMaxDevices = 64;
static std::atomic<uint32_t*> g_scratch[kMaxDevices];

size_t noalloc_scratch_bytes() { return sizeof(uint32_t) * kAmaxMaxGroups; }

// The device address of `scratch` on the current device, looked up on the
// first call per device (with that device current) and kept.
static hipError_t scratch_on_current_device(uint32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint32_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    p = static_cast<uint32_t*>(a);
    g_scratch[dev].store(p, std::memory_order_release);  // a racing first call stores the same address
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_tensor_scale_noalloc(const uint16_t* x, uint64_t nblocks, float* ts_out, hipStream_t stream) {
  if (amax_partial_count(nblocks) > kAmaxMaxGroups) return hipErrorInvalidValue;  // cannot happen: the grid is capped
  if (stream) {  // the stream must run on the current device, whose copy of the array is used
    int cur = -1, sdev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != cur) return hipErrorInvalidDevice;
  }
  uint32_t* partial = nullptr;
  const hipError_t e = scratch_on_current_device(&partial);
  if (e != hipSuccess) return e;
  return launch_tensor_scale(x, nblocks, partial, ts_out, stream);
}

}  // namespace trace_host
