// Format-independent block machinery of the libtrace kernels (gfx950): the
// hardware FP4 conversions, the bit-plane packing, the guided /
// full-information / low-bits code selection, the decode to bf16 and the
// exact per-element fallbacks, for two lane layouts:
//   - 8 elements (one 128-bit vector) per lane, codes as one dword of nibbles
//     in element order: the ungrouped NVFP4 forwards (half blocks,
//     kernels.hip) and the MXFP4 forwards (quarter blocks, mx_kernels.hip);
//   - 16 elements (two 128-bit vectors) per lane, codes as two dwords of
//     nibbles (even / odd elements): the NVFP4 capture, per-expert and
//     low-bits forwards (kernels.hip), the MXFP4 capture (a 32-element block
//     is two 16-element halves) and the diagnostics kernel (diag_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"

namespace trace_dev {

constexpr int kThreads = 256;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// v_cmp_class mask: signalling/quiet NaN and +-infinity.
constexpr int kBadClass = 0x001 | 0x002 | 0x004 | 0x200;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Loads and stores with an optional non-temporal hint (kNT).  A kernel whose
// input is larger than the 256 MB memory-side last-level cache cannot leave
// lines there for a consumer (the cache keeps only the stream's last
// quarter-gigabyte, which a consumer reading from the start has evicted
// again before it gets there), so such streams bypass it: the forwards and
// the STE backward read x and write their outputs with the hint, the capture
// writes its record with it.  The hint changes where lines are allocated,
// never the values.
template <bool kNT>
__device__ __forceinline__ uint4 load_vec(const uint4* __restrict__ p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  const u32x4 v = kNT ? __builtin_nontemporal_load(q) : *q;
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <bool kNT>
__device__ __forceinline__ void store_vec(uint4* __restrict__ p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  if (kNT)
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  else
    *reinterpret_cast<u32x4*>(p) = w;
}

template <bool kNT>
__device__ __forceinline__ void store_pair(uint2* __restrict__ p, uint2 v) {
  const u32x2 w = {v.x, v.y};
  if (kNT)
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
  else
    *reinterpret_cast<u32x2*>(p) = w;
}

template <bool kNT, typename T>
__device__ __forceinline__ void store_word(T* __restrict__ p, T v) {
  if (kNT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

template <bool kNT = false>
__device__ __forceinline__ void load_block(const uint4* __restrict__ x, uint64_t b, uint32_t (&w)[8]) {
  const uint4 v0 = load_vec<kNT>(x + 2 * b);
  const uint4 v1 = load_vec<kNT>(x + 2 * b + 1);
  w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
  w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
}

template <bool kNT = false>
__device__ __forceinline__ void store_block(uint4* __restrict__ y, uint64_t b, const uint32_t (&w)[8]) {
  store_vec<kNT>(y + 2 * b, make_uint4(w[0], w[1], w[2], w[3]));
  store_vec<kNT>(y + 2 * b + 1, make_uint4(w[4], w[5], w[6], w[7]));
}

// Toward-zero E2M1 codes of two values into byte SEL of acc: the stochastic-
// rounding conversion with a zero random operand truncates.  Issued as inline
// asm with acc tied to the destination: the compiler's builtin for this
// instruction does not keep the other bytes of the destination (the
// round-to-nearest builtin does).
template <int SEL>
__device__ __forceinline__ uint32_t fp4_rtz_at(uint32_t acc, float a, float b) {
  const f32x2 v = {a, b};
  asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, 0, 1.0 op_sel:[0,0,%2,%3]"
      : "+v"(acc)
      : "v"(v), "n"(SEL & 1), "n"(SEL >> 1));
  return acc;
}

// E2M1 codes (sign << 3 | index) of two values, written into byte `sel` of
// `acc`: round to nearest even (saturating at 6) or toward zero.
#define FP4_RNE(acc, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((acc), (a), (b), 1.0f, (sel))
#define FP4_RTZ(acc, a, b, sel) fp4_rtz_at<(sel)>((acc), (a), (b))
// Codes of the even (off = 0) or odd (off = 1) elements of a 16-value block,
// nibble k holding element 2k + off.  The byte selector must be a literal.
#define FP4_PACK8(CVT, dst, v, off)                 \
  do {                                              \
    dst = CVT(dst, (v)[0 + (off)], (v)[2 + (off)], 0);   \
    dst = CVT(dst, (v)[4 + (off)], (v)[6 + (off)], 1);   \
    dst = CVT(dst, (v)[8 + (off)], (v)[10 + (off)], 2);  \
    dst = CVT(dst, (v)[12 + (off)], (v)[14 + (off)], 3); \
  } while (0)

// The partner lane's value (lane ^ 1): a DPP quad permutation [1, 0, 3, 2].
// Both lanes of the pair must be active.
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

// ---------------------------------------------------------------------------
// 8-element half blocks (the NVFP4 kernels: one 128-bit vector of bf16 per
// lane, codes as one dword of nibbles in element order, nibble j = element j)
// ---------------------------------------------------------------------------

// Element j (0..7) of a half block held as four packed bf16 pairs.
__device__ __forceinline__ float half_elem(const uint32_t (&w)[4], int j) {
  return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
}

// Bit j of an 8-bit word to bit 0 of nibble j.
__device__ __forceinline__ uint32_t spread8(uint32_t x) {
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  return (x | (x << 3)) & 0x11111111u;
}

// Bit 0 of nibble j to bit j (the inverse of spread8).
__device__ __forceinline__ uint32_t gather8(uint32_t c) {
  c &= 0x11111111u;
  c = (c | (c >> 3)) & 0x03030303u;
  c = (c | (c >> 6)) & 0x000F000Fu;
  return (c | (c >> 12)) & 0xFFu;
}

// Largest magnitude's bf16 bits over a half block (NaN and infinity compare
// above every finite value: 0x7f80 and up).
__device__ __forceinline__ uint32_t half_max_bits(const uint32_t (&w)[4]) {
  uint32_t m0 = w[0] & 0x7fff7fffu;
  u16x2 mx;
  __builtin_memcpy(&mx, &m0, 4);
#pragma unroll
  for (int k = 1; k < 4; ++k) {
    const uint32_t mk = w[k] & 0x7fff7fffu;
    u16x2 v;
    __builtin_memcpy(&v, &mk, 4);
    mx = __builtin_elementwise_max(mx, v);
  }
  return mx.x > mx.y ? mx.x : mx.y;
}

// Bit 0 of the 16 nibbles of E (elements 0,2,..,14) and O (1,3,..,15),
// gathered into a 16-bit word in element order.
__device__ __forceinline__ uint32_t gather_parity(uint32_t E, uint32_t O) {
  const uint32_t X = ((O << 1) & 0x22222222u) | (E & ~0x22222222u);
  const uint32_t Y = ((X >> 2) & 0x0C0C0C0Cu) | (X & ~0x0C0C0C0Cu);
  const uint32_t Z = ((Y >> 4) & 0x00F000F0u) | (Y & ~0x00F000F0u);
  return __builtin_amdgcn_perm(Z, Z, 0x0C0C0200u);
}

// Inverse of gather_parity: bit j of a 16-bit word W to bit 0 of nibble j/2
// of the result (even j) or bit 1 of that nibble (odd j); other bits junk.
__device__ __forceinline__ uint32_t spread_bits(uint32_t W) {
  const uint32_t Z = __builtin_amdgcn_perm(W, W, 0x0C010C00u);
  const uint32_t Y = ((Z << 4) & 0x0F000F00u) | (Z & ~0x0F000F00u);
  return ((Y << 2) & 0x30303030u) | (Y & ~0x30303030u);
}

// y for elements 4K..4K+3 from byte K of the even / odd code dwords:
// bf16_RNE(fl32(s * q)) with q the decoded codeword (sign included).
template <int K>
__device__ __forceinline__ void decode_scaled_pair(uint32_t QE, uint32_t QO, float s, uint32_t (&out)[8]) {
  const f32x2 ge = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(QE, 1.0f, K);  // elements 4K, 4K+2
  const f32x2 go = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(QO, 1.0f, K);  // elements 4K+1, 4K+3
  const bf16x2 p0 = __builtin_convertvector((f32x2){s * ge.x, s * go.x}, bf16x2);
  const bf16x2 p1 = __builtin_convertvector((f32x2){s * ge.y, s * go.y}, bf16x2);
  __builtin_memcpy(&out[2 * K], &p0, 4);
  __builtin_memcpy(&out[2 * K + 1], &p1, 4);
}

// Element-order nibble codes from the even/odd nibble dwords.
__device__ __forceinline__ void interleave_codes(uint32_t E, uint32_t O, uint32_t& c0, uint32_t& c1) {
  c0 = 0; c1 = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t ce = (E >> (4 * k)) & 15u, co = (O >> (4 * k)) & 15u;
    const uint32_t pair = ce | (co << 4);
    if (k < 4) c0 |= pair << (8 * k); else c1 |= pair << (8 * (k - 4));
  }
}

// De-interleave element-order nibble codes (c0: elements 0..7, c1: 8..15)
// into even-element and odd-element nibble dwords.
__device__ __forceinline__ void split_codes(uint32_t c0, uint32_t c1, uint32_t& E, uint32_t& O) {
  uint32_t e0 = c0 & 0x0F0F0F0Fu, e1 = c1 & 0x0F0F0F0Fu;
  uint32_t o0 = (c0 >> 4) & 0x0F0F0F0Fu, o1 = (c1 >> 4) & 0x0F0F0F0Fu;
  e0 = (e0 | (e0 >> 4)) & 0x00FF00FFu;  // bytes 0, 2 hold nibble pairs
  e1 = (e1 | (e1 >> 4)) & 0x00FF00FFu;
  o0 = (o0 | (o0 >> 4)) & 0x00FF00FFu;
  o1 = (o1 | (o1 >> 4)) & 0x00FF00FFu;
  E = __builtin_amdgcn_perm(e1, e0, 0x06040200u);
  O = __builtin_amdgcn_perm(o1, o0, 0x06040200u);
}

// Codes of q* for the full-information rule from the floor codes F, the
// predecessor floor codes P (equal to F exactly when q is inside a bracket)
// and the rollout codes R, all packed 8 per dword: the upper endpoint F + 1
// is taken when q is inside a bracket and the rollout code has the same sign
// as F and a larger magnitude index.
__device__ __forceinline__ uint32_t full_info_select(uint32_t F, uint32_t P, uint32_t R) {
  uint32_t t = F ^ P;
  t |= t >> 2;
  t |= t >> 1;                                                    // bit 0 per nibble: exact
  const uint32_t gt = ((R | 0x88888888u) - (F & 0x77777777u) - 0x11111111u) & 0x88888888u;  // r_idx > f_idx
  const uint32_t same = ~(R ^ F) & 0x88888888u;
  return F + ((gt & same) >> 3 & ~t & 0x11111111u);
}

// The b-low-bits rule for one b.  For z >= 0 in the bracket (f, f + 1) and a
// rollout residue r, the rollout index is reconstructed as the one with
// residue r (mod 2^b) nearest to f + 1/2 among -7..7; the upper endpoint is
// taken when that index is at least f + 1.  With d = (r - f) mod 2^b this is
// exactly 1 <= d <= 2^(b-1) and d + f <= 7: offsets d above 2^(b-1) fall
// below the bracket, and an index past 7 does not exist, so the candidate
// 2^b lower (below the bracket) is the one taken -- or none, for the one
// residue no index has (8 when b = 4), which then keeps the endpoint nearer
// zero.  Negative z mirror: residue -r mod 2^b.
struct LowBitsRule {
  uint32_t mask;  // 2^b - 1
  uint32_t half;  // 2^(b-1)
};

__device__ __forceinline__ bool lowbits_up(uint32_t f, uint32_t sign, uint32_t r, const LowBitsRule& lb) {
  const uint32_t rp = ((r ^ (0u - sign)) + sign) & lb.mask;  // sign ? -r : r, modulo 2^b
  const uint32_t d = (rp - f) & lb.mask;
  return d >= 1u && d <= lb.half && d + f <= 7u;
}

// Codes of q* for the b-low-bits rule, 8 nibbles at a time: floor codes F,
// predecessor floor codes P (F == P inside a bracket) and residues R (b low
// bits of the rollout's signed grid index).  Inside a bracket the magnitude
// steps up from f to f + 1 when lowbits_up holds; computed on 8-bit lanes
// (4 elements per dword, values at most 15), each comparison the carry into
// bit 7 of a biased sum.
__device__ __forceinline__ uint32_t lowbits_select(uint32_t F, uint32_t P, uint32_t R, const LowBitsRule& lb) {
  uint32_t t = F ^ P;
  t |= t >> 2;
  t |= t >> 1;
  const uint32_t mb = lb.mask * 0x01010101u;
  const uint32_t le_half = (0x80u - (lb.half + 1u)) * 0x01010101u;
  uint32_t up = 0;
#pragma unroll
  for (int sh = 0; sh < 8; sh += 4) {
    const uint32_t fb = (F >> sh) & 0x0F0F0F0Fu, rb = (R >> sh) & 0x0F0F0F0Fu;
    const uint32_t sgn = (fb >> 3) & 0x01010101u;
    const uint32_t f = fb & 0x07070707u;
    const uint32_t sm = (sgn << 8) - sgn;                        // 0xFF in negative lanes
    const uint32_t rneg = 0x10101010u - rb;                      // 16 - r, no borrows (r <= 15)
    const uint32_t rp = ((rb & ~sm) | (rneg & sm)) & mb;
    const uint32_t d = ((rp + 0x10101010u) - f) & mb;            // (r' - f) mod 2^b, no borrows
    uint32_t u = (d + 0x7F7F7F7Fu) & 0x80808080u;               // d >= 1
    u &= ~(d + le_half) & 0x80808080u;                           // d <= 2^(b-1)
    u &= ~(d + f + 0x78787878u) & 0x80808080u;                   // d + f <= 7
    up |= (u >> 7) << sh;
  }
  return F + (up & ~t & 0x11111111u);
}

// Codes of q* for 16 quotients q (even / odd nibble dwords QE, QO) and the
// clip-mask bits (bit j set when |q_j| <= 6; NaN quotients are the caller's
// to flag).  kMode 0: round to nearest even; 1: guided by the cached bits
// (16-bit word, bit j = element j); 2: full information (rollout codes,
// element order, in roll.x / roll.y).
// kMode 3: b cached low bits; roll holds the residues as even / odd nibble
// dwords and lb the rule.
template <int kMode>
__device__ __forceinline__ uint32_t select_codes(const float (&q)[16], uint32_t cached, uint2 roll, uint32_t& QE,
                                                 uint32_t& QO, const LowBitsRule& lb = LowBitsRule{}) {
  // clip mask: sign bit of 6 - |q| is set exactly when |q| > 6
  uint32_t clip = 0;
#pragma unroll
  for (int j = 15; j >= 0; --j)
    clip = __builtin_amdgcn_alignbit(clip, __float_as_uint(6.0f - fabsf(q[j])), 31);

  float qc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) qc[j] = __builtin_amdgcn_fmed3f(q[j], -6.0f, 6.0f);

  QE = 0;
  QO = 0;
  if (kMode != 0) {
    // floor codes of q and of its predecessor toward zero: equal exactly when
    // q lies strictly inside a bracket, so the upper endpoint is floor + 1
    float pv[16];  // predecessors toward zero (a NaN for +-0, whose floor code differs)
#pragma unroll
    for (int j = 0; j < 16; ++j) pv[j] = __uint_as_float(__float_as_uint(qc[j]) - 1u);
    uint32_t FE = 0, FO = 0, PE = 0, PO = 0;
    FP4_PACK8(FP4_RTZ, FE, qc, 0);
    FP4_PACK8(FP4_RTZ, FO, qc, 1);
    FP4_PACK8(FP4_RTZ, PE, pv, 0);
    FP4_PACK8(FP4_RTZ, PO, pv, 1);
    if (kMode == 1) {
      const uint32_t C = spread_bits(cached);  // bit 0 / bit 1 of nibble k: cached bit of 2k / 2k+1
      uint32_t t = FE ^ PE;
      t |= t >> 2;
      t |= t >> 1;
      QE = FE + (~t & (FE ^ C) & 0x11111111u);
      t = FO ^ PO;
      t |= t >> 2;
      t |= t >> 1;
      QO = FO + (~t & (FO ^ (C >> 1)) & 0x11111111u);
    } else if (kMode == 2) {
      uint32_t RE, RO;
      split_codes(roll.x, roll.y, RE, RO);
      QE = full_info_select(FE, PE, RE);
      QO = full_info_select(FO, PO, RO);
    } else {
      QE = lowbits_select(FE, PE, roll.x, lb);
      QO = lowbits_select(FO, PO, roll.y, lb);
    }
  } else {
    FP4_PACK8(FP4_RNE, QE, qc, 0);
    FP4_PACK8(FP4_RNE, QO, qc, 1);
  }
  return ~clip & 0xffffu;
}

// Signed grid index of each code nibble (sign << 3 | index) as a 4-bit two's
// complement nibble: the index, or 16 - index for negative codes (0 for -0).
// Its low b bits are the b cached low bits.
__device__ __forceinline__ uint32_t signed_index_nibbles(uint32_t C) {
  const uint32_t i = C & 0x77777777u;
  const uint32_t sgn = (C >> 3) & 0x11111111u;
  const uint32_t m = (sgn << 4) - sgn;                       // 0xF in negative nibbles
  const uint32_t neg = (0x88888888u - i) ^ 0x88888888u;      // (16 - i) mod 16, no borrows (i <= 7)
  return (i & ~m) | (neg & m);
}

// Low-bit residues of 16 elements from b bit-plane words (bit j = element
// j), as even / odd nibble dwords.
__device__ __forceinline__ void residue_nibbles(const uint32_t (&pw)[4], uint32_t nplanes, uint32_t& RE,
                                                uint32_t& RO) {
  RE = 0;
  RO = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if ((uint32_t)k < nplanes) {
      const uint32_t sp = spread_bits(pw[k]);
      RE |= (sp & 0x11111111u) << k;
      RO |= ((sp >> 1) & 0x11111111u) << k;
    }
  }
}

// y (8 packed bf16 pairs) for 16 codes: bf16_RNE(fl32(s * q)).
__device__ __forceinline__ void decode_block(uint32_t QE, uint32_t QO, float s, uint32_t (&out)[8]) {
  decode_scaled_pair<0>(QE, QO, s, out);
  decode_scaled_pair<1>(QE, QO, s, out);
  decode_scaled_pair<2>(QE, QO, s, out);
  decode_scaled_pair<3>(QE, QO, s, out);
}

// Codes of q* for the 8 quotients of a half block, element order (nibble j =
// element j), and the clip-mask bits (bit j set when |q_j| <= 6).  kMode 0:
// round to nearest even; 1: guided by the cached bits (bit j = element j);
// 2: full information (rollout codes, same layout as the result); 3: b
// cached low bits (residue nibbles, same layout) with rule lb.
template <int kMode>
__device__ __forceinline__ uint32_t select_codes8(const float (&q)[8], uint32_t cached, uint32_t roll, uint32_t& Q,
                                                  const LowBitsRule& lb = LowBitsRule{}) {
  uint32_t clip = 0;
#pragma unroll
  for (int j = 7; j >= 0; --j)
    clip = __builtin_amdgcn_alignbit(clip, __float_as_uint(6.0f - fabsf(q[j])), 31);
  float qc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qc[j] = __builtin_amdgcn_fmed3f(q[j], -6.0f, 6.0f);
  if (kMode == 0) {
    Q = 0;
    Q = FP4_RNE(Q, qc[0], qc[1], 0);
    Q = FP4_RNE(Q, qc[2], qc[3], 1);
    Q = FP4_RNE(Q, qc[4], qc[5], 2);
    Q = FP4_RNE(Q, qc[6], qc[7], 3);
  } else {
    // floor codes of q and of its predecessor toward zero: equal exactly when
    // q lies strictly inside a bracket, so the upper endpoint is floor + 1
    float pv[8];  // predecessors toward zero (a NaN for +-0, whose floor code differs)
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[j] = __uint_as_float(__float_as_uint(qc[j]) - 1u);
    uint32_t F = 0, P = 0;
    F = FP4_RTZ(F, qc[0], qc[1], 0);
    F = FP4_RTZ(F, qc[2], qc[3], 1);
    F = FP4_RTZ(F, qc[4], qc[5], 2);
    F = FP4_RTZ(F, qc[6], qc[7], 3);
    P = FP4_RTZ(P, pv[0], pv[1], 0);
    P = FP4_RTZ(P, pv[2], pv[3], 1);
    P = FP4_RTZ(P, pv[4], pv[5], 2);
    P = FP4_RTZ(P, pv[6], pv[7], 3);
    if (kMode == 1) {
      uint32_t t = F ^ P;
      t |= t >> 2;
      t |= t >> 1;  // bit 0 per nibble: q is a codeword
      Q = F + (~t & (F ^ spread8(cached)) & 0x11111111u);
    } else if (kMode == 2) {
      Q = full_info_select(F, P, roll);
    } else {
      Q = lowbits_select(F, P, roll, lb);
    }
  }
  return ~clip & 0xffu;
}

template <int K>
__device__ __forceinline__ void decode_pair8(uint32_t Q, float s, uint32_t (&out)[4]) {
  const f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(Q, 1.0f, K);  // elements 2K, 2K + 1
  const bf16x2 p = __builtin_convertvector((f32x2){s * f.x, s * f.y}, bf16x2);
  __builtin_memcpy(&out[K], &p, 4);
}

// y for the 8 codes of a half block: bf16_RNE(fl32(s * q)), 4 packed pairs.
__device__ __forceinline__ void decode_half(uint32_t Q, float s, uint32_t (&out)[4]) {
  decode_pair8<0>(Q, s, out);
  decode_pair8<1>(Q, s, out);
  decode_pair8<2>(Q, s, out);
  decode_pair8<3>(Q, s, out);
}

// ---------------------------------------------------------------------------
// exact per-element definitions (IEEE division), for the fallbacks
// ---------------------------------------------------------------------------

// Capture code of one element under decoded scale s (valid: s is a positive
// finite number): sign(z) << 3 | E2M1 RNE index of min(|x / s|, 6); NaN -> 0.
__device__ __forceinline__ uint32_t exact_capture_code(float xv, float s, bool valid) {
  if (is_nan_f(xv)) return 0u;
  const uint32_t sign = __float_as_uint(xv) >> 31;
  const uint32_t idx = valid ? e2m1_rne_index(fminf(fabsf(xv / s), 6.f)) : 0u;
  return (sign << 3) | idx;
}

// Forward of one element: code of q*, clip-mask bit and y bits.
// mode 0: RNE; 1: guided by the cached bit cbit; 2: full information with
// rollout code rc; 3: b cached low bits with residue rc and rule lb.
__device__ __forceinline__ void exact_forward_element(int mode, float xv, float s, bool valid, uint32_t cbit,
                                                      uint32_t rc, uint32_t& code, uint32_t& mk, uint32_t& ybits,
                                                      const LowBitsRule& lb = LowBitsRule{}) {
  uint32_t sign = __float_as_uint(xv) >> 31;
  uint32_t idx = 0;
  mk = 0;
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
    if (mode == 1) {
      const uint32_t lo = e2m1_floor_index(a);
      const bool exact = (a == e2m1_mag(lo));
      idx = (exact || ((lo & 1u) == cbit)) ? lo : lo + 1;
    } else if (mode == 2) {
      // endpoint nearest to the rollout codeword: the upper one exactly when
      // the rollout code has z's sign and a larger magnitude index
      const uint32_t lo = e2m1_floor_index(a);
      const bool exact = (a == e2m1_mag(lo));
      idx = (!exact && (rc >> 3) == sign && (rc & 7u) > lo) ? lo + 1 : lo;
    } else if (mode == 3) {
      // rc: residue of the rollout's signed index; the table decides the step
      const uint32_t lo = e2m1_floor_index(a);
      const bool exact = (a == e2m1_mag(lo));
      idx = (!exact && lowbits_up(lo, sign, rc, lb)) ? lo + 1 : lo;
    } else {
      idx = e2m1_rne_index(a);
    }
    const float q = e2m1_mag(idx);
    yv = s * (sign ? -q : q);
  }
  code = (sign << 3) | idx;
  ybits = bf16_rne_bits(yv);
}

}  // namespace trace_dev
