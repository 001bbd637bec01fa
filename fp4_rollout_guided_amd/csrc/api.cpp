// C ABI of libtrace: argument validation and dispatch to the HIP launchers.
// Validation happens before any HIP call, so a rejected call enqueues
// nothing.  See include/trace.h for the contract of each entry point.
#include "trace.h"

#include <hip/hip_runtime.h>

#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

struct Range {
  uintptr_t lo;
  uint64_t len;
};

bool overlaps(Range a, Range b) {
  if (a.len == 0 || b.len == 0) return false;
  return a.lo < b.lo + b.len && b.lo < a.lo + a.len;
}

Range rng(const void* p, uint64_t len) { return Range{reinterpret_cast<uintptr_t>(p), len}; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// n = rows * cols with cols % 16 == 0 and 2n bytes addressable.
trace_status site_size(int64_t rows, int64_t cols, uint64_t* n_out) {
  if (rows < 0 || cols < 0 || (cols % 16) != 0) return TRACE_E_SHAPE;
  int64_t n = 0;
  if (__builtin_mul_overflow(rows, cols, &n) || n > (INT64_MAX / 4)) return TRACE_E_SHAPE;
  *n_out = (uint64_t)n;
  return TRACE_OK;
}

trace_status hip_status(hipError_t e) {
  if (e == hipSuccess) return TRACE_OK;
  g_last_hip_error = (int)e;
  return TRACE_E_HIP;
}

// Outputs must not overlap any input nor each other; `inplace_ok` lists an
// (output, input) pair that may coincide exactly.
trace_status check_alias(const Range* outs, int nout, const Range* ins, int nin, int inplace_out = -1,
                         int inplace_in = -1) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j) {
      if (i == inplace_out && j == inplace_in && outs[i].lo == ins[j].lo && outs[i].len == ins[j].len)
        continue;
      if (overlaps(outs[i], ins[j])) return TRACE_E_ALIAS;
    }
    for (int k = i + 1; k < nout; ++k)
      if (overlaps(outs[i], outs[k])) return TRACE_E_ALIAS;
  }
  return TRACE_OK;
}

}  // namespace

extern "C" {

int trace_abi_version(void) { return TRACE_ABI_VERSION; }

const char* trace_status_string(trace_status s) {
  switch (s) {
    case TRACE_OK: return "TRACE_OK";
    case TRACE_E_NULL: return "TRACE_E_NULL: a required pointer is NULL";
    case TRACE_E_SHAPE:
      return "TRACE_E_SHAPE: bad size or count (negative, cols not a multiple of the block length, overflow, "
             "group or bit count out of range, or workspace too small)";
    case TRACE_E_ALIGN: return "TRACE_E_ALIGN: misaligned pointer";
    case TRACE_E_ALIAS: return "TRACE_E_ALIAS: an output overlaps an input or another output";
    case TRACE_E_HIP: return "TRACE_E_HIP: HIP runtime or launch failure";
    default: return "TRACE: unknown status";
  }
}

int trace_last_hip_error(void) { return g_last_hip_error; }

size_t trace_tensor_scale_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  return (size_t)trace_host::amax_partial_count((uint64_t)n / 16) * sizeof(uint32_t);
}

trace_status trace_tensor_scale(const uint16_t* x, int64_t n, void* workspace, size_t workspace_bytes,
                                float* ts_out, void* stream) {
  if (!workspace || !ts_out || (n > 0 && !x)) return TRACE_E_NULL;
  if (n < 0 || (n % 16) != 0 || n > (INT64_MAX / 4)) return TRACE_E_SHAPE;
  if (workspace_bytes < trace_tensor_scale_workspace_bytes(n)) return TRACE_E_SHAPE;
  if (!aligned(x, 16) || !aligned(workspace, 4) || !aligned(ts_out, 4)) return TRACE_E_ALIGN;
  const uint64_t un = (uint64_t)n;
  const Range outs[2] = {rng(workspace, trace_tensor_scale_workspace_bytes(n)), rng(ts_out, 4)};
  const Range ins[1] = {rng(x, 2 * un)};
  if (trace_status st = check_alias(outs, 2, ins, 1)) return st;
  return hip_status(trace_host::launch_tensor_scale(x, un / 16, static_cast<uint32_t*>(workspace), ts_out,
                                                    static_cast<hipStream_t>(stream)));
}

static_assert(TRACE_NOALLOC_SCRATCH_BYTES == sizeof(uint32_t) * trace_host::kAmaxMaxGroups ||
                  trace_host::kAmaxMaxGroups < 1536u,
              "the allocation-free scratch size differs from the header");

trace_status trace_tensor_scale_noalloc(const uint16_t* x, int64_t n, float* ts_out, void* stream) {
  if (!ts_out || (n > 0 && !x)) return TRACE_E_NULL;
  if (n < 0 || (n % 16) != 0 || n > (INT64_MAX / 4)) return TRACE_E_SHAPE;
  if (trace_tensor_scale_workspace_bytes(n) > trace_host::noalloc_scratch_bytes()) return TRACE_E_SHAPE;
  if (!aligned(x, 16) || !aligned(ts_out, 4)) return TRACE_E_ALIGN;
  const Range outs[1] = {rng(ts_out, 4)};
  const Range ins[1] = {rng(x, 2 * (uint64_t)n)};
  if (trace_status st = check_alias(outs, 1, ins, 1)) return st;
  return hip_status(trace_host::launch_tensor_scale_noalloc(x, (uint64_t)n / 16, ts_out,
                                                            static_cast<hipStream_t>(stream)));
}

static_assert(TRACE_MAX_BATCH_SITES == trace_host::kMaxBatchSites, "batch size limits differ");

// Validates a batch and fills one launcher spec per site.  with_record: the
// capture batch (scales and bits required, codes optional) rather than the
// tensor scale pass (ts written).  extra: the workspace range of the tensor
// scale pass (an output), or an empty range.
static trace_status batch_specs(const trace_site* sites, int32_t count, bool with_record, Range extra,
                                trace_host::BatchSiteSpec* spec) {
  if (count < 0 || count > TRACE_MAX_BATCH_SITES) return TRACE_E_SHAPE;
  if (count > 0 && !sites) return TRACE_E_NULL;
  Range outs[3 * TRACE_MAX_BATCH_SITES + 1], ins[2 * TRACE_MAX_BATCH_SITES];
  int nout = 0, nin = 0;
  for (int32_t i = 0; i < count; ++i) {
    const trace_site& t = sites[i];
    uint64_t n = 0;
    if (trace_status st = site_size(t.rows, t.cols, &n)) return st;
    if ((n > 0 && !t.x) || (!t.ts && (n > 0 || !with_record))) return TRACE_E_NULL;
    if (with_record && n > 0 && (!t.scales || !t.bits)) return TRACE_E_NULL;
    if (!aligned(t.x, 16) || !aligned(t.ts, 4)) return TRACE_E_ALIGN;
    if (with_record && (!aligned(t.bits, 2) || (t.codes && !aligned(t.codes, 8)))) return TRACE_E_ALIGN;
    ins[nin++] = rng(t.x, 2 * n);
    if (with_record) {
      ins[nin++] = rng(t.ts, n > 0 ? 4 : 0);
      outs[nout++] = rng(t.scales, n / 16);
      outs[nout++] = rng(t.bits, n / 8);
      outs[nout++] = rng(t.codes, t.codes ? n / 2 : 0);
    } else {
      outs[nout++] = rng(t.ts, 4);
    }
    spec[i] = trace_host::BatchSiteSpec{t.x, n / 16, t.ts, with_record ? t.scales : nullptr,
                                        with_record ? t.bits : nullptr, with_record ? t.codes : nullptr};
  }
  outs[nout++] = extra;
  return check_alias(outs, nout, ins, nin);
}

// Row groups of a grouped call: 1 <= groups <= kMaxRowGroups and an
// 8-byte-aligned offsets array of groups + 1 entries.  Fills *spec.
static trace_status group_spec(const int64_t* offsets, int64_t groups, int64_t rows, int64_t cols,
                               trace_host::GroupSpec* spec) {
  if (!offsets) return TRACE_E_NULL;
  if (groups < 1 || groups > (int64_t)trace_host::kMaxRowGroups) return TRACE_E_SHAPE;
  if (!aligned(offsets, 8)) return TRACE_E_ALIGN;
  *spec = trace_host::GroupSpec{offsets, (uint64_t)groups, (uint64_t)rows, (uint64_t)cols};
  return TRACE_OK;
}

static trace_status capture(const uint16_t* x_roll, int64_t rows, int64_t cols, const int64_t* offsets,
                            int64_t groups, bool grouped, const float* ts, uint8_t* scales, uint8_t* bits,
                            uint8_t* codes, void* stream) {
  uint64_t n = 0;
  if (trace_status st = site_size(rows, cols, &n)) return st;
  trace_host::GroupSpec spec{};
  if (grouped)
    if (trace_status st = group_spec(offsets, groups, rows, cols, &spec)) return st;
  if (n == 0) return TRACE_OK;
  if (!x_roll || !ts || !scales || !bits) return TRACE_E_NULL;
  if (!aligned(x_roll, 16) || !aligned(ts, 4) || !aligned(bits, 2) || (codes && !aligned(codes, 8)))
    return TRACE_E_ALIGN;
  const uint64_t ts_len = 4 * (grouped ? spec.count : 1);
  const Range outs[3] = {rng(scales, n / 16), rng(bits, n / 8), rng(codes, codes ? n / 2 : 0)};
  const Range ins[3] = {rng(x_roll, 2 * n), rng(ts, ts_len), rng(offsets, grouped ? 8 * (spec.count + 1) : 0)};
  if (trace_status st = check_alias(outs, 3, ins, 3)) return st;
  return hip_status(trace_host::launch_capture(x_roll, n / 16, ts, grouped ? &spec : nullptr, scales, bits, codes,
                                               static_cast<hipStream_t>(stream)));
}

size_t trace_tensor_scale_batch_workspace_bytes(const trace_site* sites, int32_t count) {
  trace_host::BatchSiteSpec spec[TRACE_MAX_BATCH_SITES];
  if (batch_specs(sites, count, false, Range{0, 0}, spec) != TRACE_OK) return 0;
  return (size_t)trace_host::batch_amax_partial_count(spec, (uint32_t)count) * sizeof(uint32_t);
}

trace_status trace_tensor_scale_batch(const trace_site* sites, int32_t count, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  trace_host::BatchSiteSpec spec[TRACE_MAX_BATCH_SITES];
  if (trace_status st = batch_specs(sites, count, false, Range{0, 0}, spec)) return st;
  if (count == 0) return TRACE_OK;
  const size_t need = (size_t)trace_host::batch_amax_partial_count(spec, (uint32_t)count) * sizeof(uint32_t);
  if (need > 0 && !workspace) return TRACE_E_NULL;
  if (workspace_bytes < need) return TRACE_E_SHAPE;
  if (!aligned(workspace, 4)) return TRACE_E_ALIGN;
  if (trace_status st = batch_specs(sites, count, false, rng(workspace, need), spec)) return st;
  return hip_status(trace_host::launch_tensor_scale_batch(spec, (uint32_t)count, static_cast<uint32_t*>(workspace),
                                                          static_cast<hipStream_t>(stream)));
}

trace_status trace_capture_batch(const trace_site* sites, int32_t count, void* stream) {
  trace_host::BatchSiteSpec spec[TRACE_MAX_BATCH_SITES];
  if (trace_status st = batch_specs(sites, count, true, Range{0, 0}, spec)) return st;
  if (count == 0) return TRACE_OK;
  return hip_status(trace_host::launch_capture_batch(spec, (uint32_t)count, static_cast<hipStream_t>(stream)));
}

trace_status trace_capture(const uint16_t* x_roll, int64_t rows, int64_t cols, const float* ts,
                           uint8_t* scales, uint8_t* bits, uint8_t* codes, void* stream) {
  return capture(x_roll, rows, cols, nullptr, 0, false, ts, scales, bits, codes, stream);
}

trace_status trace_grouped_capture(const uint16_t* x_roll, int64_t rows, int64_t cols, const int64_t* offsets,
                                   int64_t groups, const float* ts, uint8_t* scales, uint8_t* bits,
                                   uint8_t* codes, void* stream) {
  return capture(x_roll, rows, cols, offsets, groups, true, ts, scales, bits, codes, stream);
}

// mode 0: RNE; 1: guided (side = bit-plane, n/8 bytes, 2-byte aligned);
// 2: full information (side = codes, n/2 bytes, 8-byte aligned).
static trace_status fakequant(int mode, const uint16_t* x, int64_t rows, int64_t cols, const int64_t* offsets,
                              int64_t groups, bool grouped, const uint8_t* scales, const float* ts,
                              const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes, void* stream) {
  uint64_t n = 0;
  if (trace_status st = site_size(rows, cols, &n)) return st;
  trace_host::GroupSpec spec{};
  if (grouped)
    if (trace_status st = group_spec(offsets, groups, rows, cols, &spec)) return st;
  if (n == 0) return TRACE_OK;
  if (!x || !scales || !ts || (mode != 0 && !side) || !y || !mask) return TRACE_E_NULL;
  const uint64_t side_len = mode == 1 ? n / 8 : (mode == 2 ? n / 2 : 0);
  const uintptr_t side_align = mode == 2 ? 8 : 2;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ts, 4) || !aligned(mask, 2) ||
      (mode != 0 && !aligned(side, side_align)) || (qcodes && !aligned(qcodes, 8)))
    return TRACE_E_ALIGN;
  const uint64_t ts_len = 4 * (grouped ? spec.count : 1);
  const Range outs[3] = {rng(y, 2 * n), rng(mask, n / 8), rng(qcodes, qcodes ? n / 2 : 0)};
  const Range ins[5] = {rng(x, 2 * n), rng(scales, n / 16), rng(ts, ts_len), rng(side, side_len),
                        rng(offsets, grouped ? 8 * (spec.count + 1) : 0)};
  if (trace_status st = check_alias(outs, 3, ins, 5, /*inplace_out=*/0, /*inplace_in=*/0)) return st;
  return hip_status(trace_host::launch_fakequant(mode, x, n / 16, scales, ts, grouped ? &spec : nullptr, side, y,
                                                 mask, qcodes, static_cast<hipStream_t>(stream)));
}

trace_status trace_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                        const uint8_t* scales, const float* ts, const uint8_t* bits,
                                        uint16_t* y, uint8_t* mask, uint8_t* qcodes, void* stream) {
  return fakequant(1, x_train, rows, cols, nullptr, 0, false, scales, ts, bits, y, mask, qcodes, stream);
}

trace_status trace_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                     const uint8_t* scales, const float* ts, uint16_t* y, uint8_t* mask,
                                     uint8_t* qcodes, void* stream) {
  return fakequant(0, x_train, rows, cols, nullptr, 0, false, scales, ts, nullptr, y, mask, qcodes, stream);
}

trace_status trace_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                           const uint8_t* scales, const float* ts, const uint8_t* codes,
                                           uint16_t* y, uint8_t* mask, uint8_t* qcodes, void* stream) {
  return fakequant(2, x_train, rows, cols, nullptr, 0, false, scales, ts, codes, y, mask, qcodes, stream);
}

trace_status trace_grouped_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                                const int64_t* offsets, int64_t groups, const uint8_t* scales,
                                                const float* ts, const uint8_t* bits, uint16_t* y, uint8_t* mask,
                                                uint8_t* qcodes, void* stream) {
  return fakequant(1, x_train, rows, cols, offsets, groups, true, scales, ts, bits, y, mask, qcodes, stream);
}

trace_status trace_grouped_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                             const int64_t* offsets, int64_t groups, const uint8_t* scales,
                                             const float* ts, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                                             void* stream) {
  return fakequant(0, x_train, rows, cols, offsets, groups, true, scales, ts, nullptr, y, mask, qcodes, stream);
}

trace_status trace_grouped_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                                   const int64_t* offsets, int64_t groups, const uint8_t* scales,
                                                   const float* ts, const uint8_t* codes, uint16_t* y,
                                                   uint8_t* mask, uint8_t* qcodes, void* stream) {
  return fakequant(2, x_train, rows, cols, offsets, groups, true, scales, ts, codes, y, mask, qcodes, stream);
}

// mode 0: RNE (no side plane); 1: guided (side = bit-plane of the source,
// src_n/8 bytes); 2: full information (side = codes of the source, src_n/2
// bytes, 8-byte aligned).
static trace_status gathered_fakequant(int mode, const uint16_t* x, int64_t rows, int64_t cols,
                                       const int64_t* row_index, int64_t src_rows, const int64_t* offsets,
                                       int64_t groups, const uint8_t* scales_src, const float* ts,
                                       const uint8_t* side_src, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                                       void* stream) {
  uint64_t n = 0, n_src = 0;
  if (trace_status st = site_size(rows, cols, &n)) return st;
  if (trace_status st = site_size(src_rows, cols, &n_src)) return st;
  const bool grouped = offsets != nullptr;
  if (!grouped && groups != 0) return TRACE_E_NULL;
  trace_host::GroupSpec spec{};
  if (grouped)
    if (trace_status st = group_spec(offsets, groups, src_rows, cols, &spec)) return st;
  if (n == 0) return TRACE_OK;
  uint64_t bound = 0;  // the kernel finds a half block's row with one multiply-high
  if (__builtin_mul_overflow(n / 8, (uint64_t)cols / 8, &bound)) return TRACE_E_SHAPE;
  if (!x || !row_index || !ts || !y || !mask || (n_src > 0 && (!scales_src || (mode != 0 && !side_src))))
    return TRACE_E_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ts, 4) || !aligned(mask, 2) || !aligned(row_index, 8) ||
      (mode == 2 && !aligned(side_src, 8)) || (qcodes && !aligned(qcodes, 8)))
    return TRACE_E_ALIGN;
  const uint64_t ts_len = 4 * (grouped ? spec.count : 1);
  const uint64_t side_len = mode == 1 ? n_src / 8 : (mode == 2 ? n_src / 2 : 0);
  const Range outs[3] = {rng(y, 2 * n), rng(mask, n / 8), rng(qcodes, qcodes ? n / 2 : 0)};
  const Range ins[6] = {rng(x, 2 * n),           rng(scales_src, n_src / 16),
                        rng(ts, ts_len),         rng(side_src, side_len),
                        rng(row_index, 8 * (uint64_t)rows), rng(offsets, grouped ? 8 * (spec.count + 1) : 0)};
  if (trace_status st = check_alias(outs, 3, ins, 6, /*inplace_out=*/0, /*inplace_in=*/0)) return st;
  return hip_status(trace_host::launch_gathered_fakequant(mode, x, (uint64_t)rows, (uint64_t)cols, row_index,
                                                          (uint64_t)src_rows, grouped ? &spec : nullptr, scales_src, ts,
                                                          side_src, y, mask, qcodes, static_cast<hipStream_t>(stream)));
}

trace_status trace_gathered_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                                 const int64_t* row_index, int64_t src_rows, const int64_t* offsets,
                                                 int64_t groups, const uint8_t* scales_src, const float* ts,
                                                 const uint8_t* bits_src, uint16_t* y, uint8_t* mask, uint8_t* qcodes,
                                                 void* stream) {
  return gathered_fakequant(1, x_train, rows, cols, row_index, src_rows, offsets, groups, scales_src, ts, bits_src, y,
                            mask, qcodes, stream);
}

trace_status trace_gathered_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                              const int64_t* row_index, int64_t src_rows, const int64_t* offsets,
                                              int64_t groups, const uint8_t* scales_src, const float* ts, uint16_t* y,
                                              uint8_t* mask, uint8_t* qcodes, void* stream) {
  return gathered_fakequant(0, x_train, rows, cols, row_index, src_rows, offsets, groups, scales_src, ts, nullptr, y,
                            mask, qcodes, stream);
}

trace_status trace_gathered_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                                    const int64_t* row_index, int64_t src_rows,
                                                    const int64_t* offsets, int64_t groups, const uint8_t* scales_src,
                                                    const float* ts, const uint8_t* codes_src, uint16_t* y,
                                                    uint8_t* mask, uint8_t* qcodes, void* stream) {
  return gathered_fakequant(2, x_train, rows, cols, row_index, src_rows, offsets, groups, scales_src, ts, codes_src, y,
                            mask, qcodes, stream);
}

size_t trace_grouped_tensor_scale_workspace_bytes(int64_t rows) {
  if (rows < 0) return 0;
  return (size_t)rows * sizeof(uint32_t);
}

trace_status trace_grouped_tensor_scale(const uint16_t* x, int64_t rows, int64_t cols, const int64_t* offsets,
                                        int64_t groups, void* workspace, size_t workspace_bytes, float* ts_out,
                                        void* stream) {
  uint64_t n = 0;
  if (trace_status st = site_size(rows, cols, &n)) return st;
  trace_host::GroupSpec spec{};
  if (trace_status st = group_spec(offsets, groups, rows, cols, &spec)) return st;
  if (!ts_out || (rows > 0 && !workspace) || (n > 0 && !x)) return TRACE_E_NULL;
  if (workspace_bytes < trace_grouped_tensor_scale_workspace_bytes(rows)) return TRACE_E_SHAPE;
  if (!aligned(x, 16) || !aligned(workspace, 4) || !aligned(ts_out, 4)) return TRACE_E_ALIGN;
  const Range outs[2] = {rng(workspace, trace_grouped_tensor_scale_workspace_bytes(rows)), rng(ts_out, 4 * spec.count)};
  const Range ins[2] = {rng(x, 2 * n), rng(offsets, 8 * (spec.count + 1))};
  if (trace_status st = check_alias(outs, 2, ins, 2)) return st;
  return hip_status(trace_host::launch_grouped_tensor_scale(x, spec, static_cast<uint32_t*>(workspace), ts_out,
                                                            static_cast<hipStream_t>(stream)));
}

trace_status trace_ste_bwd(const uint16_t* grad_out, const uint8_t* mask, int64_t n, uint16_t* grad_in,
                           void* stream) {
  if (n < 0 || (n % 16) != 0 || n > (INT64_MAX / 4)) return TRACE_E_SHAPE;
  if (n == 0) return TRACE_OK;
  if (!grad_out || !mask || !grad_in) return TRACE_E_NULL;
  if (!aligned(grad_out, 16) || !aligned(grad_in, 16) || !aligned(mask, 2)) return TRACE_E_ALIGN;
  const uint64_t un = (uint64_t)n;
  const Range outs[1] = {rng(grad_in, 2 * un)};
  const Range ins[2] = {rng(grad_out, 2 * un), rng(mask, un / 8)};
  if (trace_status st = check_alias(outs, 1, ins, 2, 0, 0)) return st;
  return hip_status(trace_host::launch_ste_bwd(grad_out, mask, un / 16, grad_in,
                                               static_cast<hipStream_t>(stream)));
}

trace_status trace_gather_records(const uint8_t* bits_src, const uint8_t* scales_src, const uint8_t* codes_src,
                                  int64_t src_rows, int64_t cols, const int64_t* row_index, int64_t dst_rows,
                                  uint8_t* bits_dst, uint8_t* scales_dst, uint8_t* codes_dst, void* stream) {
  uint64_t n_src = 0, n_dst = 0;
  if (trace_status st = site_size(src_rows, cols, &n_src)) return st;
  if (trace_status st = site_size(dst_rows, cols, &n_dst)) return st;
  if (n_dst == 0) return TRACE_OK;
  // codes are gathered iff codes_dst is given; an empty source needs no pointers
  if (codes_src && !codes_dst) return TRACE_E_NULL;
  if (!row_index || !bits_dst || !scales_dst || (n_src > 0 && (!bits_src || !scales_src || (codes_dst && !codes_src))))
    return TRACE_E_NULL;
  if (!aligned(row_index, 8) || !aligned(bits_dst, 2) || (bits_src && !aligned(bits_src, 2)) ||
      (codes_dst && (!aligned(codes_dst, 8) || (codes_src && !aligned(codes_src, 8)))))
    return TRACE_E_ALIGN;
  const Range outs[3] = {rng(bits_dst, n_dst / 8), rng(scales_dst, n_dst / 16), rng(codes_dst, codes_dst ? n_dst / 2 : 0)};
  const Range ins[4] = {rng(bits_src, n_src / 8), rng(scales_src, n_src / 16), rng(codes_src, codes_src ? n_src / 2 : 0),
                        rng(row_index, 8 * (uint64_t)dst_rows)};
  if (trace_status st = check_alias(outs, 3, ins, 4)) return st;
  return hip_status(trace_host::launch_gather_records(bits_src, scales_src, codes_src, (uint64_t)src_rows,
                                                      (uint64_t)cols, row_index, (uint64_t)dst_rows, bits_dst,
                                                      scales_dst, codes_dst, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// b cached low bits
// ---------------------------------------------------------------------------

trace_status trace_capture_lowbits(const uint16_t* x_roll, int64_t rows, int64_t cols, const float* ts,
                                   int32_t nbits, uint8_t* scales, uint8_t* planes, uint8_t* codes, void* stream) {
  uint64_t n = 0;
  if (trace_status st = site_size(rows, cols, &n)) return st;
  if (nbits < 1 || nbits > 4) return TRACE_E_SHAPE;
  if (n == 0) return TRACE_OK;
  if (!x_roll || !ts || !scales || !planes) return TRACE_E_NULL;
  if (!aligned(x_roll, 16) || !aligned(ts, 4) || !aligned(planes, 2) || (codes && !aligned(codes, 8)))
    return TRACE_E_ALIGN;
  const Range outs[3] = {rng(scales, n / 16), rng(planes, (uint64_t)nbits * (n / 8)), rng(codes, codes ? n / 2 : 0)};
  const Range ins[2] = {rng(x_roll, 2 * n), rng(ts, 4)};
  if (trace_status st = check_alias(outs, 3, ins, 2)) return st;
  return hip_status(trace_host::launch_capture(x_roll, n / 16, ts, nullptr, scales, planes, codes,
                                               static_cast<hipStream_t>(stream), (uint32_t)nbits));
}

trace_status trace_lowbits_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols, const uint8_t* scales,
                                         const float* ts, int32_t nbits, const uint8_t* planes, uint16_t* y,
                                         uint8_t* mask, uint8_t* qcodes, void* stream) {
  uint64_t n = 0;
  if (trace_status st = site_size(rows, cols, &n)) return st;
  if (nbits < 1 || nbits > 4) return TRACE_E_SHAPE;
  if (n == 0) return TRACE_OK;
  if (!x_train || !scales || !ts || !planes || !y || !mask) return TRACE_E_NULL;
  if (!aligned(x_train, 16) || !aligned(y, 16) || !aligned(ts, 4) || !aligned(mask, 2) || !aligned(planes, 2) ||
      (qcodes && !aligned(qcodes, 8)))
    return TRACE_E_ALIGN;
  const Range outs[3] = {rng(y, 2 * n), rng(mask, n / 8), rng(qcodes, qcodes ? n / 2 : 0)};
  const Range ins[4] = {rng(x_train, 2 * n), rng(scales, n / 16), rng(ts, 4),
                        rng(planes, (uint64_t)nbits * (n / 8))};
  if (trace_status st = check_alias(outs, 3, ins, 4, /*inplace_out=*/0, /*inplace_in=*/0)) return st;
  return hip_status(trace_host::launch_lowbits_fakequant(x_train, n / 16, scales, ts, planes, (uint32_t)nbits, y,
                                                         mask, qcodes, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// MXFP4
// ---------------------------------------------------------------------------

// n = rows * cols with cols % 32 == 0.
static trace_status mx_site_size(int64_t rows, int64_t cols, uint64_t* n_out) {
  if (cols % 32 != 0) return TRACE_E_SHAPE;
  return site_size(rows, cols, n_out);
}

trace_status trace_mx_capture(const uint16_t* x_roll, int64_t rows, int64_t cols, uint8_t* scales, uint8_t* bits,
                              uint8_t* codes, void* stream) {
  uint64_t n = 0;
  if (trace_status st = mx_site_size(rows, cols, &n)) return st;
  if (n == 0) return TRACE_OK;
  if (!x_roll || !scales || !bits) return TRACE_E_NULL;
  if (!aligned(x_roll, 16) || !aligned(bits, 2) || (codes && !aligned(codes, 8))) return TRACE_E_ALIGN;
  const Range outs[3] = {rng(scales, n / 32), rng(bits, n / 8), rng(codes, codes ? n / 2 : 0)};
  const Range ins[1] = {rng(x_roll, 2 * n)};
  if (trace_status st = check_alias(outs, 3, ins, 1)) return st;
  return hip_status(trace_host::launch_mx_capture(x_roll, n / 32, scales, bits, codes,
                                                  static_cast<hipStream_t>(stream)));
}

// mode 0: RNE; 1: guided (side = bit-plane, n/8 bytes, 2-byte aligned);
// 2: full information (side = codes, n/2 bytes, 8-byte aligned).
static trace_status mx_fakequant(int mode, const uint16_t* x, int64_t rows, int64_t cols, const uint8_t* scales,
                                 const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes, void* stream) {
  uint64_t n = 0;
  if (trace_status st = mx_site_size(rows, cols, &n)) return st;
  if (n == 0) return TRACE_OK;
  if (!x || !scales || (mode != 0 && !side) || !y || !mask) return TRACE_E_NULL;
  const uint64_t side_len = mode == 1 ? n / 8 : (mode == 2 ? n / 2 : 0);
  const uintptr_t side_align = mode == 2 ? 8 : 2;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(mask, 2) || (mode != 0 && !aligned(side, side_align)) ||
      (qcodes && !aligned(qcodes, 8)))
    return TRACE_E_ALIGN;
  const Range outs[3] = {rng(y, 2 * n), rng(mask, n / 8), rng(qcodes, qcodes ? n / 2 : 0)};
  const Range ins[3] = {rng(x, 2 * n), rng(scales, n / 32), rng(side, side_len)};
  if (trace_status st = check_alias(outs, 3, ins, 3, /*inplace_out=*/0, /*inplace_in=*/0)) return st;
  return hip_status(trace_host::launch_mx_fakequant(mode, x, n / 32, scales, side, y, mask, qcodes,
                                                    static_cast<hipStream_t>(stream)));
}

trace_status trace_mx_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                           const uint8_t* scales, const uint8_t* bits, uint16_t* y, uint8_t* mask,
                                           uint8_t* qcodes, void* stream) {
  return mx_fakequant(1, x_train, rows, cols, scales, bits, y, mask, qcodes, stream);
}

trace_status trace_mx_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols, const uint8_t* scales,
                                        uint16_t* y, uint8_t* mask, uint8_t* qcodes, void* stream) {
  return mx_fakequant(0, x_train, rows, cols, scales, nullptr, y, mask, qcodes, stream);
}

trace_status trace_mx_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                              const uint8_t* scales, const uint8_t* codes, uint16_t* y,
                                              uint8_t* mask, uint8_t* qcodes, void* stream) {
  return mx_fakequant(2, x_train, rows, cols, scales, codes, y, mask, qcodes, stream);
}

// ---------------------------------------------------------------------------
// agreement statistics
// ---------------------------------------------------------------------------

trace_status trace_mismatch_stats(const uint16_t* x_train, int64_t rows, int64_t cols, const uint8_t* scales,
                                  const float* ts, const uint8_t* bits, const uint8_t* codes, uint64_t* stats,
                                  void* stream) {
  uint64_t n = 0;
  if (trace_status st = site_size(rows, cols, &n)) return st;
  if (n == 0) return TRACE_OK;
  if (!x_train || !scales || !ts || !bits || !codes || !stats) return TRACE_E_NULL;
  if (!aligned(x_train, 16) || !aligned(ts, 4) || !aligned(bits, 2) || !aligned(codes, 8) || !aligned(stats, 8))
    return TRACE_E_ALIGN;
  const Range outs[1] = {rng(stats, 20 * sizeof(uint64_t))};
  const Range ins[5] = {rng(x_train, 2 * n), rng(scales, n / 16), rng(ts, 4), rng(bits, n / 8), rng(codes, n / 2)};
  if (trace_status st = check_alias(outs, 1, ins, 5)) return st;
  return hip_status(trace_host::launch_mismatch_stats(x_train, n / 16, scales, ts, bits, codes, stats,
                                                      static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// MXFP8 (the W4A8 setting's FP8 activation grid)
// ---------------------------------------------------------------------------

trace_status trace_mx8_capture(const uint16_t* x_roll, int64_t rows, int64_t cols, uint8_t* scales, uint8_t* bits,
                               uint8_t* codes, void* stream) {
  uint64_t n = 0;
  if (trace_status st = mx_site_size(rows, cols, &n)) return st;
  if (n == 0) return TRACE_OK;
  if (!x_roll || !scales || !bits) return TRACE_E_NULL;
  if (!aligned(x_roll, 16) || !aligned(bits, 2) || (codes && !aligned(codes, 16))) return TRACE_E_ALIGN;
  const Range outs[3] = {rng(scales, n / 32), rng(bits, n / 8), rng(codes, codes ? n : 0)};
  const Range ins[1] = {rng(x_roll, 2 * n)};
  if (trace_status st = check_alias(outs, 3, ins, 1)) return st;
  return hip_status(trace_host::launch_mx8_capture(x_roll, n / 32, scales, bits, codes,
                                                   static_cast<hipStream_t>(stream)));
}

// mode 0: RNE; 1: guided (side = bit-plane, n/8 bytes, 2-byte aligned);
// 2: full information (side = rollout codes, n bytes, 16-byte aligned).
static trace_status mx8_fakequant(int mode, const uint16_t* x, int64_t rows, int64_t cols, const uint8_t* scales,
                                  const uint8_t* side, uint16_t* y, uint8_t* mask, uint8_t* qcodes, void* stream) {
  uint64_t n = 0;
  if (trace_status st = mx_site_size(rows, cols, &n)) return st;
  if (n == 0) return TRACE_OK;
  if (!x || !scales || (mode != 0 && !side) || !y || !mask) return TRACE_E_NULL;
  const uint64_t side_len = mode == 1 ? n / 8 : (mode == 2 ? n : 0);
  const uintptr_t side_align = mode == 2 ? 16 : 2;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(mask, 2) || (mode != 0 && !aligned(side, side_align)) ||
      (qcodes && !aligned(qcodes, 16)))
    return TRACE_E_ALIGN;
  const Range outs[3] = {rng(y, 2 * n), rng(mask, n / 8), rng(qcodes, qcodes ? n : 0)};
  const Range ins[3] = {rng(x, 2 * n), rng(scales, n / 32), rng(side, side_len)};
  if (trace_status st = check_alias(outs, 3, ins, 3, /*inplace_out=*/0, /*inplace_in=*/0)) return st;
  return hip_status(trace_host::launch_mx8_fakequant(mode, x, n / 32, scales, side, y, mask, qcodes,
                                                     static_cast<hipStream_t>(stream)));
}

trace_status trace_mx8_guided_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                            const uint8_t* scales, const uint8_t* bits, uint16_t* y, uint8_t* mask,
                                            uint8_t* qcodes, void* stream) {
  return mx8_fakequant(1, x_train, rows, cols, scales, bits, y, mask, qcodes, stream);
}

trace_status trace_mx8_rne_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols, const uint8_t* scales,
                                         uint16_t* y, uint8_t* mask, uint8_t* qcodes, void* stream) {
  return mx8_fakequant(0, x_train, rows, cols, scales, nullptr, y, mask, qcodes, stream);
}

trace_status trace_mx8_full_info_fakequant_fwd(const uint16_t* x_train, int64_t rows, int64_t cols,
                                               const uint8_t* scales, const uint8_t* codes, uint16_t* y,
                                               uint8_t* mask, uint8_t* qcodes, void* stream) {
  return mx8_fakequant(2, x_train, rows, cols, scales, codes, y, mask, qcodes, stream);
}

}  // extern "C"
