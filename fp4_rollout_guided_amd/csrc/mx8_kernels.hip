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
// Kernels (grid-stride):
//   mx8_capture_kernel       scale byte, parity bit-plane, optional codes;
//                            one lane per 16-element half block
//   mx8_fakequant_kernel<M>  M = 0 RNE, 1 guided, 2 full information; one
//                            lane per 8-element vector (a quarter block)
//
// In the capture a lane owns one 16-element half (32 bytes of bf16 in, 16
// bytes of codes, 2 bytes of bits); lane pairs share a block's scale byte
// (one DPP move exchanges the halves' maxima).  In the forwards a lane owns 8
// elements (16 bytes in and out, 8 code bytes, a byte of bits and of mask).
// The quotient by a power-of-two scale is a multiplication by its exact
// inverse, so x * 2^(127 - b) is the correctly rounded x / s.  Codes come from the hardware conversions:
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

// Element j of a lane's N elements held as N / 2 packed bf16 pairs.
template <int N>
__device__ __forceinline__ float lane_elem(const uint32_t (&w)[N / 2], int j) {
  return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
}

// Quotients of a lane's N elements under inverse scale inv; NaN quotients (a
// NaN element, or an infinity times the zero of a zero-scale block) become
// the zero the format gives them -- +0 for a NaN element, the element's
// signed zero otherwise -- and their elements are flagged in *nan_bits (a
// NaN element's mask bit is 0).
template <int N>
__device__ __forceinline__ void mx8_quotients(const uint32_t (&w)[N / 2], float inv, float (&q)[N],
                                              uint32_t& nan_bits) {
  bool bad = false;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    q[j] = lane_elem<N>(w, j) * inv;
    bad |= __builtin_amdgcn_class(q[j], 0x003);  // signalling or quiet NaN
  }
  nan_bits = 0;
  if (bad) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float xv = lane_elem<N>(w, j);
      if (is_nan_f(q[j])) {
        q[j] = is_nan_f(xv) ? 0.f : copysignf(0.f, xv);
        nan_bits |= is_nan_f(xv) ? (1u << j) : 0u;
      }
    }
  }
}

// Clip-mask word: bit j set when |q_j| <= 448 (the sign bit of 448 - |q_j|
// is clear exactly then, infinities included).
template <int N>
__device__ __forceinline__ uint32_t mx8_keep_bits(const float (&q)[N]) {
  uint32_t clip = 0;
#pragma unroll
  for (int j = N - 1; j >= 0; --j) clip = __builtin_amdgcn_alignbit(clip, __float_as_uint(448.f - fabsf(q[j])), 31);
  return ~clip & ((1u << N) - 1u);
}

// Round-to-nearest-even E4M3FN codes of the clipped quotients, dword k
// holding elements 4k..4k+3 (byte j = element 4k + j).
template <int N>
__device__ __forceinline__ void fp8_rne_codes(const float (&qc)[N], uint32_t (&C)[N / 4]) {
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
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

// Bit 0 of each of the N code bytes, gathered into an N-bit word in element
// order.
template <int N>
__device__ __forceinline__ uint32_t fp8_parity_word(const uint32_t (&C)[N / 4]) {
  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    uint32_t t = C[k] & kLow;  // bits 0, 8, 16, 24
    t |= t >> 7;               // bits 0, 1 (and 16, 17)
    t |= t >> 14;              // bits 0..3
    word |= (t & 15u) << (4 * k);
  }
  return word;
}

// Cached bits 4k..4k+3 of a bit word into bit 0 of the four bytes of a dword
// (the product places bit i at 8i; no two partial products meet).
__device__ __forceinline__ uint32_t fp8_spread4(uint32_t word, int k) {
  const uint32_t nib = (word >> (4 * k)) & 15u;
  return (nib * 0x00204081u) & kLow;
}

// Codes of q* for N quotients: RNE (kMode 0), guided by the cached bits
// (kMode 1; N-bit word, bit j = element j) or full information (kMode 2;
// the rollout code bytes in R, same layout as the output).
template <int kMode, int N>
__device__ __forceinline__ void mx8_select_codes(const float (&qc)[N], uint32_t cached, const uint32_t (&R)[N / 4],
                                                 uint32_t (&Q)[N / 4]) {
  if (kMode == 0) {
    fp8_rne_codes<N>(qc, Q);
    return;
  }
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
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

// y for N codes: bf16_RNE(fl32(s * q)), N / 2 packed bf16 pairs.
template <int N>
__device__ __forceinline__ void fp8_decode_scaled(const uint32_t (&Q)[N / 4], float s, uint32_t (&out)[N / 2]) {
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
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
// kNT: the record is stored with the non-temporal hint (tensors past the
// last-level cache; the loads stay plain, as in the NVFP4 capture).
template <bool kNT>
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
    mx8_quotients<16>(w, e8m0_inverse(sb), q, nan_bits);
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = __builtin_amdgcn_fmed3f(q[j], -448.f, 448.f);
    uint32_t C[4];
    fp8_rne_codes<16>(q, C);
    if ((h & 1) == 0) store_word<kNT>(&scales[h >> 1], (uint8_t)sb);
    store_word<kNT>(&bits[h], (uint16_t)fp8_parity_word<16>(C));
    if (codes) store_vec<kNT>(&codes[h], make_uint4(C[0], C[1], C[2], C[3]));
  }
}

// ---------------------------------------------------------------------------
// fake-quant forward; kMode: 0 = RNE, 1 = guided, 2 = full information.  One
// lane per 8-element vector (a quarter block: one 128-bit load of x, one
// byte of bits and of mask, 8 code bytes), which streams faster than a lane
// per 16-element half; the four lanes of a block read its scale byte.  kNT:
// x is loaded and every output stored with the non-temporal hint (tensors
// past the last-level cache).
// ---------------------------------------------------------------------------
template <int kMode, bool kNT>
__global__ __launch_bounds__(kThreads) void mx8_fakequant_kernel(const uint4* __restrict__ x, uint64_t nvec,
                                                                 const uint8_t* __restrict__ scales,
                                                                 const uint8_t* __restrict__ bits,
                                                                 const uint2* __restrict__ rcodes,
                                                                 uint4* __restrict__ y, uint8_t* __restrict__ mask,
                                                                 uint2* __restrict__ qcodes) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x; g < nvec; g += stride) {
    const uint32_t sbyte = scales[g >> 2];
    const uint32_t cached = kMode == 1 ? (uint32_t)bits[g] : 0u;
    const uint2 rv = kMode == 2 ? rcodes[g] : make_uint2(0u, 0u);
    const uint4 v = load_vec<kNT>(&x[g]);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    // a NaN scale byte makes a zero-scale block: multiplying by 0 maps every
    // finite x to a zero of its own sign, decoded with s = 1
    const bool valid = sbyte != 0xffu;
    const float inv = valid ? e8m0_inverse(sbyte) : 0.f;
    const float s = valid ? e8m0_value(sbyte) : 1.f;
    float q[8];
    uint32_t nan_bits;
    mx8_quotients<8>(w, inv, q, nan_bits);
    const uint32_t keep = mx8_keep_bits<8>(q) & ~nan_bits;
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_fmed3f(q[j], -448.f, 448.f);
    const uint32_t R[2] = {rv.x, rv.y};
    uint32_t Q[2];
    mx8_select_codes<kMode, 8>(q, cached, R, Q);
    uint32_t out[4];
    fp8_decode_scaled<8>(Q, s, out);
    store_vec<kNT>(&y[g], make_uint4(out[0], out[1], out[2], out[3]));
    store_word<kNT>(&mask[g], (uint8_t)(valid ? keep : 0u));
    if (qcodes) store_pair<kNT>(&qcodes[g], make_uint2(Q[0], Q[1]));
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
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint16_t* bv = reinterpret_cast<uint16_t*>(bits);
  uint4* cv = reinterpret_cast<uint4*>(codes);
  if (past_cache(nblocks * 64))
    hipLaunchKernelGGL(mx8_capture_kernel<true>, dim3(mx8_grid(nhalves)), dim3(kThreads), 0, stream, xv, nhalves,
                       scales, bv, cv);
  else
    hipLaunchKernelGGL(mx8_capture_kernel<false>, dim3(mx8_grid(nhalves)), dim3(kThreads), 0, stream, xv, nhalves,
                       scales, bv, cv);
  return hipGetLastError();
}

template <bool kNT>
static void launch_mx8_fakequant_t(int mode, const uint4* xv, uint64_t nvec, const uint8_t* scales,
                                   const uint8_t* side, uint4* yv, uint8_t* mask, uint2* qv, hipStream_t stream) {
  const dim3 grid(mx8_grid(nvec)), block(kThreads);
  if (mode == 1)
    hipLaunchKernelGGL((mx8_fakequant_kernel<1, kNT>), grid, block, 0, stream, xv, nvec, scales, side,
                       static_cast<const uint2*>(nullptr), yv, mask, qv);
  else if (mode == 2)
    hipLaunchKernelGGL((mx8_fakequant_kernel<2, kNT>), grid, block, 0, stream, xv, nvec, scales,
                       static_cast<const uint8_t*>(nullptr), reinterpret_cast<const uint2*>(side), yv, mask, qv);
  else
    hipLaunchKernelGGL((mx8_fakequant_kernel<0, kNT>), grid, block, 0, stream, xv, nvec, scales,
                       static_cast<const uint8_t*>(nullptr), static_cast<const uint2*>(nullptr), yv, mask, qv);
}

hipError_t launch_mx8_fakequant(int mode, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                                const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                                hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;  // an empty grid is not a valid launch
  const uint64_t nvec = 4 * nblocks;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint4* yv = reinterpret_cast<uint4*>(y);
  uint2* qv = reinterpret_cast<uint2*>(qcodes);
  if (past_cache(nblocks * 64))
    launch_mx8_fakequant_t<true>(mode, xv, nvec, scales, side, yv, mask, qv, stream);
  else
    launch_mx8_fakequant_t<false>(mode, xv, nvec, scales, side, yv, mask, qv, stream);
  return hipGetLastError();
}

}  // namespace trace_host
