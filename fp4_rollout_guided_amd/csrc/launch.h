// Internal host-side launchers (not part of the C ABI).  Arguments have been
// validated by api.cpp; sizes are in 16-element blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trace_host {

// Upper bound on amax partial workgroups (and on workspace words): six
// workgroups per compute unit.  On 128 MiB and 1 GiB tensors 1536 streamed
// 1-3% faster than 2048 (eight per compute unit, full residency); 1024 or
// fewer were slower, and larger grids lose more in the finalize than they gain.
#ifndef TRACE_AMAX_MAX_GROUPS
#define TRACE_AMAX_MAX_GROUPS 1536u
#endif
constexpr uint32_t kAmaxMaxGroups = TRACE_AMAX_MAX_GROUPS;
// Upper bound on the grid of the streaming kernels (one 4096-element tile per
// workgroup below it; workgroups loop over the tensor beyond it).  A grid
// that covers the tensor once streams faster than a persistent grid, whose
// loop makes each tile's loads wait behind the previous tile's stores.  A
// dispatch counts at most 2^32 - 1 work-items per dimension, so 256-thread
// workgroups cap the grid below 2^24; 2^22 groups cover 2^34 elements (32 GiB
// of bf16) in one pass.
#ifndef TRACE_MAX_GROUPS
#define TRACE_MAX_GROUPS (1u << 22)
#endif
constexpr uint32_t kMaxGroups = TRACE_MAX_GROUPS;
static_assert((uint64_t)TRACE_MAX_GROUPS * 256 <= 0xffffffffull, "grid exceeds 2^32 - 1 work-items");

// Tensors larger than MI355X's 256 MB memory-side last-level cache are
// streamed with the non-temporal hint: the kernels' instantiations with kNT
// set load x and store their outputs (the captures: their records) that
// way; smaller tensors keep plain accesses, so a consumer can still find
// their lines in the cache.  The test build that caps grids sets the
// threshold to 0, so that its tensors run the hinted instantiations.
#ifndef TRACE_NT_STREAM_BYTES
#define TRACE_NT_STREAM_BYTES (256ull << 20)
#endif
constexpr uint64_t kNTStreamBytes = TRACE_NT_STREAM_BYTES;
inline bool past_cache(uint64_t bytes) { return bytes > kNTStreamBytes; }

// Row groups with one tensor scale each: group g holds rows
// [offsets[g], offsets[g+1]) of a rows x cols site tensor (device int64[count + 1]).
constexpr uint32_t kMaxRowGroups = 1u << 20;
struct GroupSpec {
  const int64_t* offsets;
  uint64_t count;
  uint64_t rows;
  uint64_t cols;
};

uint32_t amax_partial_count(uint64_t nblocks);

// Batches of site tensors (tensor scale pass and capture over up to
// kMaxBatchSites sites in one launch each).
constexpr uint32_t kMaxBatchSites = 8;
struct BatchSiteSpec {
  const uint16_t* x;
  uint64_t nblocks;
  float* ts;
  uint8_t* scales;
  uint8_t* bits;
  uint8_t* codes;  // nullable
};
// Partial-maximum words the batch tensor scale pass needs (its workspace).
uint32_t batch_amax_partial_count(const BatchSiteSpec* sites, uint32_t count);
hipError_t launch_tensor_scale_batch(const BatchSiteSpec* sites, uint32_t count, uint32_t* partial,
                                     hipStream_t stream);
hipError_t launch_capture_batch(const BatchSiteSpec* sites, uint32_t count, hipStream_t stream);

hipError_t launch_tensor_scale(const uint16_t* x, uint64_t nblocks, uint32_t* partial, float* ts_out,
                               hipStream_t stream);
// The same with the library's per-device scratch array (noalloc_scratch_bytes()
// bytes) in place of a workspace; the stream must belong to the current device.
size_t noalloc_scratch_bytes();
hipError_t launch_tensor_scale_noalloc(const uint16_t* x, uint64_t nblocks, float* ts_out, hipStream_t stream);
// row_amax: u32[rows] workspace; ts_out: fp32[count]
hipError_t launch_grouped_tensor_scale(const uint16_t* x, const GroupSpec& g, uint32_t* row_amax, float* ts_out,
                                       hipStream_t stream);
// g == nullptr: one tensor scale ts[0]; otherwise ts[group of the row].
// nplanes > 1 (ungrouped only): bits holds nplanes bit-planes of n/8 bytes
// (the b cached low bits).
hipError_t launch_capture(const uint16_t* x, uint64_t nblocks, const float* ts, const GroupSpec* g,
                          uint8_t* scales, uint8_t* bits, uint8_t* codes, hipStream_t stream,
                          uint32_t nplanes = 1);
// b = nplanes cached low bits (1..4) in nplanes bit-planes of n/8 bytes.
hipError_t launch_lowbits_fakequant(const uint16_t* x, uint64_t nblocks, const uint8_t* scales, const float* ts,
                                    const uint8_t* planes, uint32_t nplanes, uint16_t* y, uint8_t* mask,
                                    uint8_t* qcodes, hipStream_t stream);
// mode 0: RNE; 1: guided, side = bit-plane (u8[n/8]); 2: full information,
// side = rollout codes (u8[n/2]).
hipError_t launch_fakequant(int mode, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                            const float* ts, const GroupSpec* g, const uint8_t* side, uint16_t* y, uint8_t* mask,
                            uint8_t* qcodes, hipStream_t stream);
// Forward on records read back in the trainer's row order: destination row r
// of the rows x cols x_train reads source row row_index[r] of the record
// (scales_src, and side_src = bits for mode 1 or codes for mode 2; mode 0,
// RNE, reads no side plane) of a
// src_rows x cols site; g == nullptr: one tensor scale ts[0], else g
// describes groups of the source rows (ts[group of the source row]).
// Requires rows * (cols / 8) * (cols / 8) < 2^64 (checked by the caller): the
// row of a half block is then one 64-bit multiply-high by ceil(2^64 / (cols / 8)).
hipError_t launch_gathered_fakequant(int mode, const uint16_t* x, uint64_t rows, uint64_t cols,
                                     const int64_t* row_index, uint64_t src_rows, const GroupSpec* g,
                                     const uint8_t* scales_src, const float* ts, const uint8_t* side_src, uint16_t* y,
                                     uint8_t* mask, uint8_t* qcodes, hipStream_t stream);
// MXFP4 (32-element blocks, E8M0 scales); sizes in 32-element blocks.
hipError_t launch_mx_capture(const uint16_t* x, uint64_t nblocks, uint8_t* scales, uint8_t* bits, uint8_t* codes,
                             hipStream_t stream);
hipError_t launch_mx_fakequant(int mode, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                               const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                               hipStream_t stream);
// MXFP8 (E4M3 elements, 32-element blocks, E8M0 scales); sizes in 32-element
// blocks; codes / rollout codes / qcodes: one byte per element.
hipError_t launch_mx8_capture(const uint16_t* x, uint64_t nblocks, uint8_t* scales, uint8_t* bits, uint8_t* codes,
                              hipStream_t stream);
hipError_t launch_mx8_fakequant(int mode, const uint16_t* x, uint64_t nblocks, const uint8_t* scales,
                                const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                                hipStream_t stream);
hipError_t launch_gather_records(const uint8_t* bits_src, const uint8_t* scales_src, const uint8_t* codes_src,
                                 uint64_t src_rows, uint64_t cols, const int64_t* row_index, uint64_t dst_rows,
                                 uint8_t* bits_dst, uint8_t* scales_dst, uint8_t* codes_dst, hipStream_t stream);
// Agreement statistics, added to stats (uint64[20]): [0..14] elements whose
// rollout and RNE codes are k signed grid steps apart, [15] straddles,
// [16] crossed one-step mismatches, [17] recovered mismatches, [18] guarantee
// violations, [19] elements.
hipError_t launch_mismatch_stats(const uint16_t* x, uint64_t nblocks, const uint8_t* scales, const float* ts,
                                 const uint8_t* bits, const uint8_t* codes, uint64_t* stats, hipStream_t stream);
hipError_t launch_ste_bwd(const uint16_t* g, const uint8_t* mask, uint64_t nblocks, uint16_t* gin,
                          hipStream_t stream);

}  // namespace trace_host
