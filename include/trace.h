/*
 * libtrace -- rollout-guided FP4 rounding (TRACE) for MI355X (gfx950).
 *
 * C ABI of the data-parallel hot path of TRACE's rollout-guided rounding as
 * described in the rcap.io post "TRACE: Rollout-Guided Quantization-Aware
 * Training for FP4" (2026-10-06):
 *
 *   rollout side  -- quantize each captured activation / KV site to NVFP4 and
 *                    keep a compact record: one mantissa bit per element plus
 *                    the scale metadata (bandwidth paragraph; the capture half
 *                    of the pseudo-code listing);
 *   training side -- recompute z = clip(x_train / s, -6, 6) with the cached
 *                    rollout scale, bracket z between two adjacent FP4
 *                    codewords, keep the one the cached bit points at, and
 *                    return s * q* through a straight-through estimator
 *                    (rollout-guided rounding paragraph; the QAT half of the
 *                    listing).
 *
 * NVFP4 parameters (the pages name the format, not its parameters): blocks of
 * 16 consecutive elements along the last dimension, one OCP E4M3FN scale byte
 * per block, one IEEE fp32 tensor scale ts = amax / (6 * 448), and E2M1
 * codewords {0, 0.5, 1, 1.5, 2, 3, 4, 6} with sign, reached by
 * round-to-nearest-even.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Tensors are flat, row-major, and live in device memory (hipMalloc'd or
 *   allocated by a framework on the same device).  bf16 values are passed as
 *   raw uint16_t bit patterns.  A site tensor of rows x cols elements needs
 *   cols % 16 == 0; blocks never cross rows.
 * - Record layout (the rollout -> trainer cache contract):
 *     scales : uint8_t[n/16], one E4M3FN byte per block, in block order;
 *     bits   : uint8_t[n/8], bit k of byte j is the parity bit of element
 *              8*j + k (bit 0 of its E2M1 code = parity of its signed grid
 *              index: the single low bit the post keeps per element);
 *     codes  : uint8_t[n/2], optional full 4-bit codes (sign << 3 | index),
 *              element 2*j in the low nibble of byte j;
 *     ts     : one IEEE fp32 tensor scale, in device memory.
 *   The caller indexes records by [trajectory, token, site]; one call handles
 *   one site tensor.
 * - Ownership: the caller owns every buffer.  The library allocates nothing,
 *   frees nothing, never synchronizes, and keeps no state between calls
 *   other than a thread-local copy of the last HIP error code and, per
 *   device, the resident-workgroup count of the agreement statistics kernel
 *   (one occupancy query, cached atomically) and the address of the 6 KiB
 *   device array of trace_tensor_scale_noalloc (below), whose contents are
 *   shared by that entry point's calls on the device.  It is safe to call
 *   from several host threads.
 * - Asynchrony: all device work is enqueued on `stream` (a hipStream_t; NULL
 *   is the default stream).  Outputs are valid once that stream reaches the
 *   point of the call.
 * - Errors: entry points return a trace_status.  Arguments are validated
 *   before any HIP call; on a validation error nothing is enqueued.
 *   n == 0 is a successful no-op that enqueues nothing and accepts NULL data
 *   pointers (trace_tensor_scale still writes ts = 0 to ts_out).
 * - Alignment: bf16 tensors need 16-byte alignment, bit-planes and masks
 *   2-byte alignment, code arrays 8-byte alignment; scale bytes have none.
 * - Aliasing: outputs must not overlap inputs, except exact in-place use
 *   where an entry point allows it.
 * - Caching: for a tensor larger than 256 MiB (MI355X's memory-side
 *   last-level cache) the forwards and the STE backward load it and store
 *   their outputs with the non-temporal hint, and the captures store their
 *   records with it, so those lines are not left in that cache for the next
 *   kernel; smaller tensors use plain accesses.  Values are unaffected.
 */
#ifndef LIBTRACE_TRACE_H
#define LIBTRACE_TRACE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRACE_ABI_VERSION 10

#if defined(__GNUC__)
#define TRACE_API __attribute__((visibility("default")))
#else
#define TRACE_API
#endif

typedef int trace_status;
enum {
  TRACE_OK = 0,
  TRACE_E_NULL = 1,  /* a required pointer is NULL                          */
  TRACE_E_SHAPE = 2, /* negative size, cols not a multiple of the block
                        length (16; 32 for MXFP4), size overflow, a group or
                        bit count out of range, or a workspace that is too
                        small                                               */
  TRACE_E_ALIGN = 3, /* a pointer is not aligned as stated above            */
  TRACE_E_ALIAS = 4, /* an output overlaps an input or another output       */
  TRACE_E_HIP = 5    /* a HIP runtime call or kernel launch failed;
                        trace_last_hip_error() returns its hipError_t       */
};

/* TRACE_ABI_VERSION of the built library. */
TRACE_API int trace_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
TRACE_API const char* trace_status_string(trace_status status);

/* hipError_t of the most recent TRACE_E_HIP returned on this host thread,
 * 0 if none. */
TRACE_API int trace_last_hip_error(void);

/*
 * Tensor scale of a rollout site tensor (NVFP4 second-level scale; "scale
 * metadata" in the bandwidth paragraph, scale_roll in the listing):
 *   ts = fl32(amax / 2688),  amax = max |x[i]| over the n elements, NaN
 *   ignored, 0 for n == 0 or an all-NaN tensor.
 *   x         : bf16[n] (device), n >= 0, n % 16 == 0.
 *   workspace : device scratch of at least
 *               trace_tensor_scale_workspace_bytes(n) bytes, 4-byte aligned,
 *               caller-owned; its contents are not preserved.
 *   ts_out    : one fp32 (device), written on `stream`.
 * The result is exact (a maximum and one correctly rounded division), so it
 * does not depend on the launch geometry.
 */
TRACE_API size_t trace_tensor_scale_workspace_bytes(int64_t n);
TRACE_API trace_status trace_tensor_scale(const uint16_t* x, int64_t n, void* workspace,
                                size_t workspace_bytes, float* ts_out,
                                void* stream);

/*
 * trace_tensor_scale without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same result, arguments and errors as
 * trace_tensor_scale minus the workspace.  The partial maxima go to a device
 * array inside the library of TRACE_NOALLOC_SCRATCH_BYTES (6 KiB), one copy
 * per GPU, held until the process ends; the call itself allocates nothing.
 * Its address is looked up on the first call on each device (that device
 * current).  Every tensor size is accepted (the partial-maximum grid is
 * capped at the array's 1536 words; a size needing more would be
 * TRACE_E_SHAPE).  `stream` must belong to the current device (else
 * TRACE_E_HIP with hipErrorInvalidDevice).  Each call writes every word it
 * reads, so nothing needs clearing between calls; but every call on one GPU
 * shares that GPU's array, so calls that overlap in time on one GPU (on
 * different streams, or from several host threads) race and may return a
 * wrong scale: order them on one stream.
 */
#define TRACE_NOALLOC_SCRATCH_BYTES 6144
TRACE_API trace_status trace_tensor_scale_noalloc(const uint16_t* x, int64_t n, float* ts_out,
                                                  void* stream);

/*
 * Rollout-side capture (fp4_quantize and low_bits(q_roll, b=1) in the
 * listing; the compact cache of the bandwidth paragraph).  Per 16-element
 * block b:
 *   amax_b = max |x| over the block (NaN ignored);
 *   scales[b] = E4M3FN_RNE_saturating(fl32(fl32(amax_b / 6) / ts)), 0 when ts
 *               is 0 or not finite;
 *   s = fl32(E4M3FN(scales[b]) * ts).
 * Per element: z = fl32(x / s); idx = E2M1 round-to-nearest-even index of
 * min(|z|, 6) (ties to the even index); code = sign(z) << 3 | idx;
 * bit = idx & 1.  In a block whose s is not a positive finite number, every
 * code is a zero with the input's sign.  NaN elements give code 0.
 *   x_roll : bf16[rows*cols] (device); ts : one fp32 (device), usually from
 *            trace_tensor_scale.
 *   scales : uint8[n/16], bits : uint8[n/8], codes : uint8[n/2] or NULL.
 */
TRACE_API trace_status trace_capture(const uint16_t* x_roll, int64_t rows, int64_t cols,
                           const float* ts, uint8_t* scales, uint8_t* bits,
                           uint8_t* codes, void* stream);

/*
 * The rollout side of several site tensors at once (a layer's activation and
 * KV sites: the listing captures every site, the bandwidth paragraph logs
 * every activation and KV entry).  Each site keeps its own tensor scale and
 * record; the results equal trace_tensor_scale and trace_capture called per
 * site, bit for bit.  The batch runs as one tensor-scale pass (two kernel
 * launches) and one capture launch instead of three launches per site,
 * which saves the fixed cost of filling and draining the GPU per launch on
 * small and medium sites.
 *   sites : host array of count descriptors, 0 <= count <= TRACE_MAX_BATCH_SITES
 *           (count == 0 is a successful no-op); per site:
 *     x, rows, cols : the site tensor as in trace_capture (bf16[rows*cols],
 *                     cols % 16 == 0, 16-byte aligned; NULL when empty);
 *     ts            : one fp32 (device): written by trace_tensor_scale_batch
 *                     (0 for an empty site), read by trace_capture_batch;
 *     scales, bits, codes : the record, as in trace_capture (codes may be
 *                     NULL); unused by trace_tensor_scale_batch.
 *   workspace : device scratch of at least
 *               trace_tensor_scale_batch_workspace_bytes(sites, count) bytes,
 *               4-byte aligned, caller-owned; its contents are not preserved.
 * No output may overlap any site's input or another output (sites may share
 * inputs, and trace_capture_batch's ts are inputs).  Errors as for the
 * per-site calls; nothing is enqueued unless every site is valid.
 */
#define TRACE_MAX_BATCH_SITES 8
typedef struct trace_site {
  const uint16_t* x;
  int64_t rows;
  int64_t cols;
  float* ts;
  uint8_t* scales;
  uint8_t* bits;
  uint8_t* codes;
} trace_site;
TRACE_API size_t trace_tensor_scale_batch_workspace_bytes(const trace_site* sites, int32_t count);
TRACE_API trace_status trace_tensor_scale_batch(const trace_site* sites, int32_t count, void* workspace,
                                                size_t workspace_bytes, void* stream);
TRACE_API trace_status trace_capture_batch(const trace_site* sites, int32_t count, void* stream);

/*
 * Training-side rollout-guided fake-quant forward (the QAT half of the
 * listing; rollout-guided rounding paragraph).  With the cached rollout
 * record (scales, ts, bits) of the same site:
 *   s = fl32(E4M3FN(scales[b]) * ts);  zr = fl32(x_train / s);
 *   mask = |zr| <= 6;  z = clip(zr, -6, 6);
 *   lo, hi = the E2M1 magnitudes enclosing |z| (equal when |z| is one);
 *   m = |z| if lo == hi, else the one of lo, hi whose index parity is the
 *       cached bit;  q* = copysign(m, z);  y = bf16_RNE(fl32(s * q*)).
 * Zero-scale blocks (s not a positive finite number; any scale byte >= 0x7F)
 * give y = +-0 with the input's sign and mask 0; NaN inputs give y = +0 and
 * mask 0.
 *   x_train : bf16[rows*cols]; scales/ts/bits : the capture record;
 *   y       : bf16[n]; may be exactly x_train (in place);
 *   mask    : uint8[n/8], clip mask for trace_ste_bwd (bit layout as bits);
 *   qcodes  : uint8[n/2] codes of q*, or NULL.
 */
TRACE_API trace_status trace_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                        int64_t cols, const uint8_t* scales,
                                        const float* ts, const uint8_t* bits,
                                        uint16_t* y, uint8_t* mask,
                                        uint8_t* qcodes, void* stream);

/*
 * Plain round-to-nearest-even fake-quant forward on the same scales, the
 * vanilla-QAT baseline the post compares against (the rounding that the
 * guided rule replaces): as trace_guided_fakequant_fwd with m = the E2M1
 * magnitude nearest to |z|, ties to the even index.  Same arguments minus
 * `bits`; y may be exactly x_train.
 */
TRACE_API trace_status trace_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                     int64_t cols, const uint8_t* scales,
                                     const float* ts, uint16_t* y,
                                     uint8_t* mask, uint8_t* qcodes,
                                     void* stream);

/*
 * Full-information guided fake-quant forward: the ablation reference that
 * caches the whole 4-bit rollout code instead of one bit (rcap.io post,
 * Ablations bullet; the rollout-guided rounding paragraph's rule with the
 * rollout codeword known).  As trace_guided_fakequant_fwd, except
 *   m = |z| if lo == hi, else the one of lo, hi whose signed value is nearest
 *       to the rollout's signed codeword (no ties are possible).
 * This choice is never farther from the rollout value than round-to-nearest.
 *   codes : uint8[n/2] rollout codes from trace_capture (element 2j in the
 *           low nibble of byte j), 8-byte aligned.
 * Other arguments, aliasing and errors as trace_guided_fakequant_fwd.
 */
TRACE_API trace_status trace_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                     int64_t cols, const uint8_t* scales,
                                                     const float* ts, const uint8_t* codes,
                                                     uint16_t* y, uint8_t* mask,
                                                     uint8_t* qcodes, void* stream);

/*
 * Straight-through-estimator backward (straight_through_estimator in the
 * listing): grad_in[i] = mask bit i ? grad_out[i] : +0.0 (0x0000).
 *   grad_out, grad_in : bf16[n]; grad_in may be exactly grad_out;
 *   mask : uint8[n/8] from a fake-quant forward; n % 16 == 0.
 */
TRACE_API trace_status trace_ste_bwd(const uint16_t* grad_out, const uint8_t* mask,
                           int64_t n, uint16_t* grad_in, void* stream);

/*
 * Trainer-side readback of compact records: the training engine reads the
 * rollout's per-site records back in its own row order (rcap.io post,
 * limitations list: a cache tier holds the records and the trainer reads
 * them back).  Destination row r receives source row row_index[r] of the
 * bit-plane, the scale bytes and, when both code pointers are given, the
 * 4-bit codes.  A row index outside [0, src_rows) produces an all-zero row:
 * scale byte 0, i.e. zero-scale blocks for the trainer.
 *   bits_src u8[src_rows*cols/8] (2-byte aligned), scales_src
 *   u8[src_rows*cols/16], codes_src u8[src_rows*cols/2] (8-byte aligned);
 *   the source pointers may be NULL when src_rows == 0;
 *   row_index int64[dst_rows] in device memory, 8-byte aligned;
 *   bits_dst, scales_dst, codes_dst sized for dst_rows (same alignments).
 *   Codes are gathered iff codes_dst is non-NULL; codes_src without
 *   codes_dst is TRACE_E_NULL.  cols % 16 == 0.  Outputs must not overlap
 *   inputs (no in-place gather).  dst_rows == 0 is a no-op.
 */
TRACE_API trace_status trace_gather_records(const uint8_t* bits_src, const uint8_t* scales_src,
                                            const uint8_t* codes_src, int64_t src_rows, int64_t cols,
                                            const int64_t* row_index, int64_t dst_rows,
                                            uint8_t* bits_dst, uint8_t* scales_dst,
                                            uint8_t* codes_dst, void* stream);

/*
 * Training-side forwards on records read back in the trainer's row order,
 * without a gathered copy of the record (rcap.io post, limitations list: a
 * cache tier holds the rollout's records and the training engine reads them
 * back).  The result equals trace_gather_records into the trainer's order
 * followed by the guided (full-information, RNE) forward, with each
 * destination row's tensor scale taken from its source row:
 *   destination row r of x_train (rows x cols) uses source row
 *   s = row_index[r] of the record (scales_src, bits_src or codes_src) of a
 *   src_rows x cols site, and tensor scale ts[0], or, with offsets, ts[g]
 *   for the group g of source rows [offsets[g], offsets[g+1]) holding s;
 *   an index outside [0, src_rows) gives zero-scale blocks (y = +-0 with
 *   the input's sign, mask 0), as a gathered all-zero record row would.
 *   row_index : int64[rows] in device memory, 8-byte aligned;
 *   offsets, groups : NULL and 0 for one tensor scale; otherwise the
 *               per-expert groups of the source rows, with the rules of the
 *               grouped entry points below (offsets[groups] = src_rows);
 *   scales_src u8[src_rows*cols/16]; bits_src u8[src_rows*cols/8];
 *   codes_src u8[src_rows*cols/2], 8-byte aligned (the RNE forward reads
 *   neither: the vanilla-QAT baseline on the same records); ts fp32[1 or groups];
 *   the record pointers may be NULL when src_rows == 0;
 *   y, mask, qcodes : as trace_guided_fakequant_fwd, in destination order;
 *   y may be exactly x_train.
 * Also TRACE_E_SHAPE when rows * (cols/8)^2 reaches 2^64.  rows == 0 is a
 * no-op.  Other errors as trace_guided_fakequant_fwd.
 */
TRACE_API trace_status trace_gathered_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                                           const int64_t* row_index, int64_t src_rows,
                                                           const int64_t* offsets, int64_t groups,
                                                           const uint8_t* scales_src, const float* ts,
                                                           const uint8_t* bits_src, uint16_t* y, uint8_t* mask,
                                                           uint8_t* qcodes, void* stream);
TRACE_API trace_status trace_gathered_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                                        const int64_t* row_index, int64_t src_rows,
                                                        const int64_t* offsets, int64_t groups,
                                                        const uint8_t* scales_src, const float* ts, uint16_t* y,
                                                        uint8_t* mask, uint8_t* qcodes, void* stream);
TRACE_API trace_status trace_gathered_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                                              const int64_t* row_index, int64_t src_rows,
                                                              const int64_t* offsets, int64_t groups,
                                                              const uint8_t* scales_src, const float* ts,
                                                              const uint8_t* codes_src, uint16_t* y, uint8_t* mask,
                                                              uint8_t* qcodes, void* stream);

/*
 * Per-expert tensor scales for packed MoE rows.  Only the routed experts (and
 * the KV cache) run in FP4 (rcap.io post, limitations list), and a
 * routed-expert site holds the rows of every expert back to back.  Reading
 * taken here: each expert's rows form a tensor of their own, with their own
 * amax and tensor scale, as a grouped FP4 GEMM quantizes them.  Group g holds
 * rows [offsets[g], offsets[g+1]) of the rows x cols site tensor.
 *   offsets : int64[groups + 1] in device memory, 8-byte aligned,
 *             offsets[0] = 0, offsets[groups] = rows, nondecreasing (empty
 *             groups allowed); 1 <= groups <= 2^20.  The library does not
 *             read the offsets on the host: offsets that break these rules
 *             still keep every access in bounds (values are clamped to
 *             [0, rows]) but assign rows to groups in an unspecified way.
 *   ts      : fp32[groups] in device memory, one tensor scale per group.
 * Every other argument, the record layout, aliasing (offsets and ts are
 * inputs) and the error rules are those of the ungrouped entry point.
 */

/* ts_out[g] = fl32(amax over the rows of group g / 2688); 0 for an empty
 * group.  workspace: trace_grouped_tensor_scale_workspace_bytes(rows) bytes
 * of device scratch (one word per row), 4-byte aligned; rows == 0 accepts a
 * NULL workspace and still writes ts_out. */
TRACE_API size_t trace_grouped_tensor_scale_workspace_bytes(int64_t rows);
TRACE_API trace_status trace_grouped_tensor_scale(const uint16_t* x, int64_t rows, int64_t cols,
                                                  const int64_t* offsets, int64_t groups,
                                                  void* workspace, size_t workspace_bytes,
                                                  float* ts_out, void* stream);

/* trace_capture with ts[group of the row] as each row's tensor scale. */
TRACE_API trace_status trace_grouped_capture(const uint16_t* x_roll, int64_t rows, int64_t cols,
                                             const int64_t* offsets, int64_t groups,
                                             const float* ts, uint8_t* scales, uint8_t* bits,
                                             uint8_t* codes, void* stream);

/* The three forwards with ts[group of the row]. */
TRACE_API trace_status trace_grouped_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                          int64_t cols, const int64_t* offsets,
                                                          int64_t groups, const uint8_t* scales,
                                                          const float* ts, const uint8_t* bits,
                                                          uint16_t* y, uint8_t* mask,
                                                          uint8_t* qcodes, void* stream);
TRACE_API trace_status trace_grouped_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                       int64_t cols, const int64_t* offsets,
                                                       int64_t groups, const uint8_t* scales,
                                                       const float* ts, uint16_t* y,
                                                       uint8_t* mask, uint8_t* qcodes,
                                                       void* stream);
TRACE_API trace_status trace_grouped_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                             int64_t cols, const int64_t* offsets,
                                                             int64_t groups, const uint8_t* scales,
                                                             const float* ts, const uint8_t* codes,
                                                             uint16_t* y, uint8_t* mask,
                                                             uint8_t* qcodes, void* stream);

/*
 * b cached low bits, b = 1..4 (low_bits(q_roll, b) in the listing, which the
 * post runs with b = 1: the single bit of the bandwidth paragraph).
 * Reading for b > 1: the b low bits of each codeword's signed grid index
 * (-7..7) in two's complement; for b = 1 this is the parity bit above.  The
 * record keeps them as b bit-planes of n/8 bytes each, back to back: plane k
 * holds bit k, in the bit-plane layout above, so plane 0 is the b = 1 record.
 * The training side reconstructs the rollout's signed index as the one with
 * that residue modulo 2^b nearest to the middle of z's bracket (among the
 * grid's 15 indices; the candidates are 2^b apart, so there is no tie) and
 * returns the bracket endpoint nearest to it; z itself when z is a
 * codeword.  A rollout codeword within the window of 2^b signed indices
 * around z's bracket is recovered exactly; b = 4 is full information.
 *   nbits  : b, 1..4 (else TRACE_E_SHAPE);
 *   planes : uint8[b * n/8], 2-byte aligned.
 * Other arguments, layouts, aliasing and errors as trace_capture /
 * trace_guided_fakequant_fwd.
 */
TRACE_API trace_status trace_capture_lowbits(const uint16_t* x_roll, int64_t rows, int64_t cols,
                                             const float* ts, int32_t nbits, uint8_t* scales,
                                             uint8_t* planes, uint8_t* codes, void* stream);
TRACE_API trace_status trace_lowbits_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                   int64_t cols, const uint8_t* scales,
                                                   const float* ts, int32_t nbits,
                                                   const uint8_t* planes, uint16_t* y,
                                                   uint8_t* mask, uint8_t* qcodes, void* stream);

/*
 * Agreement statistics of one site tensor between the rollout's codes and
 * the training side.  The post's premises: most mismatched sites differ by
 * one adjacent codeword (bandwidth paragraph), a one-codeword mismatch is a
 * value straddling a rounding midpoint (rounding-boundary paragraph), and
 * the guided choice is never farther from the rollout codeword than plain
 * rounding (rollout-guided rounding paragraph).  Per element, the RNE,
 * guided and full-information codes of x_train under the rollout record
 * (scales, ts, bits; as trace_guided_fakequant_fwd computes them) are
 * compared with the rollout code (codes, as trace_capture writes them), and
 * the counts are ADDED to stats (calls accumulate, e.g. over a layer sweep;
 * zero it before the first call):
 *   stats[k], k = 0..14 : elements whose rollout and RNE codes are k signed
 *                         grid steps apart (k = 0: agreement);
 *   stats[15] : straddles -- mismatches whose rollout codeword is an end of
 *               the bracket of x_train / s;
 *   stats[16] : crossed -- one-step mismatches that are not straddles;
 *   stats[17] : recovered -- mismatches where the guided code is the
 *               rollout's (equal to stats[15] when bits are the parity of
 *               codes);
 *   stats[18] : violations -- elements whose guided value is farther from
 *               the rollout value than the RNE value;
 *   stats[19] : elements counted.
 * Arguments: x_train bf16[rows*cols] (16-byte aligned), scales uint8[n/16],
 * ts device fp32[1], bits uint8[n/8] (2-byte aligned), codes uint8[n/2]
 * (8-byte aligned), stats uint64[20] device (8-byte aligned, must not overlap
 * an input).  Errors as trace_guided_fakequant_fwd; n == 0 is a no-op.
 */
TRACE_API trace_status trace_mismatch_stats(const uint16_t* x_train, int64_t rows, int64_t cols,
                                            const uint8_t* scales, const float* ts,
                                            const uint8_t* bits, const uint8_t* codes,
                                            uint64_t* stats, void* stream);

/*
 * MXFP4 variant.  The post reports that the method carries over to MXFP4
 * (rcap.io post, Ablations bullet) without giving the format's parameters;
 * they are the OCP Microscaling Formats (MX) v1.0 specification's:
 *   - blocks of 32 consecutive elements along the last dimension
 *     (cols % 32 == 0);
 *   - one E8M0 scale byte b per block, standing for s = 2^(b - 127); byte
 *     0xFF (NaN) makes a zero-scale block;
 *   - capture: b = 127 + clamp(floor(log2(amax)) - 2, -127, 127) with amax
 *     the block's largest magnitude (NaN ignored; an all-zero block gets
 *     b = 0; an infinite element counts as exponent 128, b = 253);
 *   - elements, parity bits, codes, the three forwards, the clip mask, zero
 *     scales and NaN handling: exactly as on the NVFP4 path above, with this
 *     s in place of fl32(E4M3FN(byte) * ts).  There is no tensor scale.
 * Layouts: scales uint8[n/32]; bits, mask, codes and qcodes as above (same
 * layouts and alignments).  The STE backward (trace_ste_bwd) takes the mask
 * unchanged.
 */
TRACE_API trace_status trace_mx_capture(const uint16_t* x_roll, int64_t rows, int64_t cols,
                                        uint8_t* scales, uint8_t* bits, uint8_t* codes,
                                        void* stream);
TRACE_API trace_status trace_mx_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                     int64_t cols, const uint8_t* scales,
                                                     const uint8_t* bits, uint16_t* y,
                                                     uint8_t* mask, uint8_t* qcodes,
                                                     void* stream);
TRACE_API trace_status trace_mx_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                  int64_t cols, const uint8_t* scales,
                                                  uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                                                  void* stream);
TRACE_API trace_status trace_mx_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                        int64_t cols, const uint8_t* scales,
                                                        const uint8_t* codes, uint16_t* y,
                                                        uint8_t* mask, uint8_t* qcodes,
                                                        void* stream);

/*
 * MXFP8 variant: the FP8 activation grid of the W4A8 setting.  The post
 * reports that the method carries over to MXFP4 W4A8 (rcap.io post,
 * Ablations bullet); in W4A8 the rounded activations are 8-bit.  Reading:
 * the OCP MX v1.0 format MXFP8 with E4M3 elements:
 *   - blocks of 32 consecutive elements along the last dimension
 *     (cols % 32 == 0), one E8M0 scale byte b each, s = 2^(b - 127); byte
 *     0xFF (NaN) makes a zero-scale block;
 *   - capture: b = 127 + clamp(floor(log2(amax)) - 8, -127, 127) (8: the
 *     exponent of E4M3's largest normal, 448), with amax as for MXFP4 (an
 *     infinite element gives b = 247);
 *   - elements: OCP E4M3FN bytes, sign << 7 | magnitude code; the code of
 *     z = clip(fl32(x / s), -448, 448) rounded to nearest even; the cached
 *     bit is the magnitude code's last bit, bit k of byte j of the
 *     bit-plane belonging to element 8j + k;
 *   - forwards: as on the NVFP4 path with this grid, clip bound 448 and mask
 *     |x / s| <= 448; full information takes the bracket endpoint nearest
 *     the rollout's signed codeword, a NaN rollout byte (0x7F / 0xFF)
 *     counting as +-480.
 * Layouts: scales uint8[n/32]; bits and mask uint8[n/8], 2-byte aligned;
 * codes, rollout codes and qcodes uint8[n] (one E4M3FN byte per element,
 * flat element order), 16-byte aligned.  Aliasing and errors as the MXFP4
 * entry points; y may alias x_train exactly.  The STE backward
 * (trace_ste_bwd) takes the mask unchanged.
 */
TRACE_API trace_status trace_mx8_capture(const uint16_t* x_roll, int64_t rows, int64_t cols,
                                         uint8_t* scales, uint8_t* bits, uint8_t* codes,
                                         void* stream);
TRACE_API trace_status trace_mx8_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                      int64_t cols, const uint8_t* scales,
                                                      const uint8_t* bits, uint16_t* y,
                                                      uint8_t* mask, uint8_t* qcodes,
                                                      void* stream);
TRACE_API trace_status trace_mx8_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                   int64_t cols, const uint8_t* scales,
                                                   uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                                                   void* stream);
TRACE_API trace_status trace_mx8_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows,
                                                         int64_t cols, const uint8_t* scales,
                                                         const uint8_t* codes, uint16_t* y,
                                                         uint8_t* mask, uint8_t* qcodes,
                                                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBTRACE_TRACE_H */
