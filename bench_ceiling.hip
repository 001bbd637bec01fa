// Practical HBM ceilings of this GPU for the access mixes of the libtrace
// kernels: a plain 128-bit copy (read + write, the layout of the STE
// backward: one vector per lane), the same copy with the non-temporal hint on
// its loads and stores (as the kernels stream tensors larger than the 256 MB
// last-level cache), a read-only stream and a write-only fill, each over
// 1 GiB buffers with one-shot grids, plus the runtime's device-to-device
// copy, and plain copies of 12 MiB to 192 MiB.
// Each is timed (median of 15 HIP-event-timed launches) in three settings:
// back to back, after a read-only pass over another 1 GiB buffer, and after
// a 1 GiB write to another buffer (whose dirty lines are then written back
// while the measured kernel streams).  Prints one JSON object.
//
// Built by fp4_rollout_guided_amd/build.py into _build/bench_ceiling; run by
// `python bench.py` (the "practical_ceiling" field) or on its own.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#define CHECK(call)                                                                  \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));              \
      exit(1);                                                                       \
    }                                                                                \
  } while (0)

// One 128-bit vector per lane: the fastest stream measured on this GPU (two or
// more vectors per lane copy 4-5 points of the 8 TB/s slower).
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ s, uint4* __restrict__ d, uint64_t n) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) d[i] = s[i];
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_nt_kernel(const u32x4* __restrict__ s, u32x4* __restrict__ d,
                                                      uint64_t n) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ s, uint32_t* __restrict__ out,
                                                   uint64_t n) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  if (i < n) {
    const uint4 v = s[i];
    acc = v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;  // data-dependent store keeps the loads
}

__global__ __launch_bounds__(256) void fill_kernel(uint4* __restrict__ d, uint64_t n) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) d[i] = make_uint4(1u, 2u, 3u, 4u);
}

struct Buffers {
  uint4 *src, *dst, *other;
  uint32_t* sink;
  uint64_t n;  // uint4 per buffer
};

enum Kind { kCopy, kCopyNT, kRead, kFill, kMemcpy };

static void launch(Kind k, const Buffers& b) {
  const dim3 blk(256);
  switch (k) {
    case kCopy: hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((b.n + 255) / 256)), blk, 0, 0, b.src, b.dst, b.n); break;
    case kCopyNT:
      hipLaunchKernelGGL(copy_nt_kernel, dim3((unsigned)((b.n + 255) / 256)), blk, 0, 0,
                         reinterpret_cast<const u32x4*>(b.src), reinterpret_cast<u32x4*>(b.dst), b.n);
      break;
    case kRead: hipLaunchKernelGGL(read_kernel, dim3((unsigned)((b.n + 255) / 256)), blk, 0, 0, b.src, b.sink, b.n); break;
    case kFill: hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((b.n + 255) / 256)), blk, 0, 0, b.dst, b.n); break;
    case kMemcpy: CHECK(hipMemcpyAsync(b.dst, b.src, b.n * 16, hipMemcpyDeviceToDevice, 0)); break;
  }
}

static void prepass(int mode, const Buffers& b) {
  if (mode == 1)
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)((b.n + 255) / 256)), dim3(256), 0, 0, b.other, b.sink, b.n);
  if (mode == 2) hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((b.n + 255) / 256)), dim3(256), 0, 0, b.other, b.n);
}

static double median_us(Kind k, int mode, const Buffers& b) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<float> t;
  for (int r = 0; r < 16; ++r) {
    prepass(mode, b);
    CHECK(hipEventRecord(e0, 0));
    launch(k, b);
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (r > 0) t.push_back(ms);  // the first launch warms up
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  std::sort(t.begin(), t.end());
  return 1e3 * t[t.size() / 2];
}

// A plain copy of `bytes` (read, and the same written) from b.src to b.dst:
// median of 15 launches, back to back (mode 0) or each after a read-only pass
// over the whole 1 GiB of b.other (mode 1).  Small copies show the fixed cost
// of filling and draining the chip that short kernels pay.
static double copy_size_us(uint64_t bytes, int mode, const Buffers& b) {
  const uint64_t n = bytes / 16;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<float> t;
  for (int r = 0; r < 16; ++r) {
    prepass(mode, b);
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, 0, b.src, b.dst, n);
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (r > 0) t.push_back(ms);
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  std::sort(t.begin(), t.end());
  return 1e3 * t[t.size() / 2];
}

int main() {
  const uint64_t bytes = 1ull << 30;
  Buffers b;
  b.n = bytes / 16;
  CHECK(hipMalloc(&b.src, bytes));
  CHECK(hipMalloc(&b.dst, bytes));
  CHECK(hipMalloc(&b.other, bytes));
  CHECK(hipMalloc(&b.sink, (b.n / 256 + 1) * sizeof(uint32_t)));
  CHECK(hipMemset(b.src, 1, bytes));
  CHECK(hipMemset(b.dst, 2, bytes));
  CHECK(hipMemset(b.other, 3, bytes));
  CHECK(hipDeviceSynchronize());
  const struct { const char* name; Kind k; double traffic; } tests[] = {
      {"copy", kCopy, 2.0 * bytes}, {"copy_nontemporal", kCopyNT, 2.0 * bytes}, {"read", kRead, 1.0 * bytes},
      {"fill", kFill, 1.0 * bytes},
      {"runtime_d2d_copy", kMemcpy, 2.0 * bytes}};
  const char* modes[] = {"back_to_back", "after_read_pass", "after_write_pass"};
  printf("{\"buffer_bytes\": %llu, \"peak_GB_s\": 8000", (unsigned long long)bytes);
  for (const auto& t : tests) {
    printf(", \"%s\": {", t.name);
    for (int m = 0; m < 3; ++m) {
      const double us = median_us(t.k, m, b);
      const double gbs = t.traffic / (us * 1e-6) / 1e9;
      printf("%s\"%s\": {\"us\": %.1f, \"GB_s\": %.1f, \"frac\": %.4f}", m ? ", " : "", modes[m], us, gbs,
             gbs / 8000.0);
    }
    printf("}");
  }
  // plain copies of 12 MiB to 192 MiB (the sizes of the smaller sites' streams)
  printf(", \"copy_by_size\": {");
  const uint64_t mib[] = {12, 24, 48, 96, 192};
  for (int i = 0; i < 5; ++i) {
    const uint64_t sz = mib[i] << 20;
    printf("%s\"%llu_MiB\": {", i ? ", " : "", (unsigned long long)mib[i]);
    for (int m = 0; m < 2; ++m) {
      const double us = copy_size_us(sz, m, b);
      const double gbs = 2.0 * sz / (us * 1e-6) / 1e9;
      printf("%s\"%s\": {\"us\": %.2f, \"GB_s\": %.1f, \"frac\": %.4f}", m ? ", " : "", modes[m], us, gbs,
             gbs / 8000.0);
    }
    printf("}");
  }
  printf("}}\n");
  CHECK(hipFree(b.src));
  CHECK(hipFree(b.dst));
  CHECK(hipFree(b.other));
  CHECK(hipFree(b.sink));
  return 0;
}
