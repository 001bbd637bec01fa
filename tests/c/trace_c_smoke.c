/* A C caller of libtrace: device buffers from hipMalloc, the default
 * stream, no PyTorch.  Reads a rows x cols site (x_roll, x_train, grad as
 * raw bf16 bit patterns) from an input file, runs the tensor scale, the
 * capture (with codes), the guided and RNE fake-quant forwards and the STE
 * backward through the C ABI, and writes every output to a file for the
 * GPU test to compare with the oracle.
 *
 *   trace_c_smoke IN_PATH OUT_PATH
 *
 * IN_PATH:  int64 rows, int64 cols, then uint16 x_roll[n], x_train[n], grad[n]
 * OUT_PATH: float ts, uint8 scales[n/16], bits[n/8], codes[n/2],
 *           uint16 y_g[n], uint8 mask_g[n/8], uint16 y_r[n],
 *           uint8 mask_r[n/8], uint16 grad_in[n]
 * Exit status 0 on success; otherwise a message on stderr names the call.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "trace.h"

static int fail(const char* what, const char* detail) {
  fprintf(stderr, "trace_c_smoke: %s: %s\n", what, detail);
  return 1;
}

#define HIP_OK(call)                                                  \
  do {                                                                \
    hipError_t e_ = (call);                                           \
    if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_)); \
  } while (0)

#define TRACE_OK_OR_FAIL(call)                                        \
  do {                                                                \
    trace_status s_ = (call);                                         \
    if (s_ != TRACE_OK) return fail(#call, trace_status_string(s_)); \
  } while (0)

static int read_all(FILE* f, void* p, size_t bytes) { return fread(p, 1, bytes, f) == bytes; }
static int write_all(FILE* f, const void* p, size_t bytes) { return fwrite(p, 1, bytes, f) == bytes; }

int main(int argc, char** argv) {
  if (argc != 3) return fail("usage", "trace_c_smoke IN_PATH OUT_PATH");
  if (trace_abi_version() != TRACE_ABI_VERSION) return fail("trace_abi_version", "library and header differ");
  FILE* in = fopen(argv[1], "rb");
  if (!in) return fail("fopen", argv[1]);
  int64_t rows = 0, cols = 0;
  if (!read_all(in, &rows, 8) || !read_all(in, &cols, 8)) return fail("read", "header");
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || rows > (1 << 20) || cols > (1 << 16))
    return fail("read", "rows / cols out of the range this program accepts");
  const size_t n = (size_t)rows * (size_t)cols;
  /* host buffers: three inputs, then the outputs in file order */
  uint16_t* h_in = (uint16_t*)malloc(3 * n * sizeof(uint16_t));
  if (!h_in) return fail("malloc", "inputs");
  if (!read_all(in, h_in, 3 * n * sizeof(uint16_t))) return fail("read", "inputs");
  fclose(in);

  uint16_t *d_xr, *d_xt, *d_g, *d_yg, *d_yr, *d_gin;
  uint8_t *d_sc, *d_bits, *d_codes, *d_mg, *d_mr;
  float* d_ts;
  void* d_ws;
  const size_t ws_bytes = trace_tensor_scale_workspace_bytes((int64_t)n);
  HIP_OK(hipMalloc((void**)&d_xr, 2 * n));
  HIP_OK(hipMalloc((void**)&d_xt, 2 * n));
  HIP_OK(hipMalloc((void**)&d_g, 2 * n));
  HIP_OK(hipMalloc((void**)&d_yg, 2 * n));
  HIP_OK(hipMalloc((void**)&d_yr, 2 * n));
  HIP_OK(hipMalloc((void**)&d_gin, 2 * n));
  HIP_OK(hipMalloc((void**)&d_sc, n / 16));
  HIP_OK(hipMalloc((void**)&d_bits, n / 8));
  HIP_OK(hipMalloc((void**)&d_codes, n / 2));
  HIP_OK(hipMalloc((void**)&d_mg, n / 8));
  HIP_OK(hipMalloc((void**)&d_mr, n / 8));
  HIP_OK(hipMalloc((void**)&d_ts, sizeof(float)));
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMemcpy(d_xr, h_in, 2 * n, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_xt, h_in + n, 2 * n, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_g, h_in + 2 * n, 2 * n, hipMemcpyHostToDevice));

  /* the path, on the default stream (NULL) */
  TRACE_OK_OR_FAIL(trace_tensor_scale(d_xr, (int64_t)n, d_ws, ws_bytes, d_ts, NULL));
  TRACE_OK_OR_FAIL(trace_capture(d_xr, rows, cols, d_ts, d_sc, d_bits, d_codes, NULL));
  TRACE_OK_OR_FAIL(trace_guided_fakequant_fwd(d_xt, rows, cols, d_sc, d_ts, d_bits, d_yg, d_mg, NULL, NULL));
  TRACE_OK_OR_FAIL(trace_rne_fakequant_fwd(d_xt, rows, cols, d_sc, d_ts, d_yr, d_mr, NULL, NULL));
  TRACE_OK_OR_FAIL(trace_ste_bwd(d_g, d_mg, (int64_t)n, d_gin, NULL));
  /* a rejected call enqueues nothing and says why */
  if (trace_capture(d_xr, rows, cols + 1, d_ts, d_sc, d_bits, NULL, NULL) != TRACE_E_SHAPE)
    return fail("trace_capture", "cols % 16 != 0 was not rejected");
  HIP_OK(hipDeviceSynchronize());

  float ts = 0.f;
  uint8_t* h8 = (uint8_t*)malloc(n);
  uint16_t* h16 = (uint16_t*)malloc(2 * n);
  if (!h8 || !h16) return fail("malloc", "outputs");
  FILE* out = fopen(argv[2], "wb");
  if (!out) return fail("fopen", argv[2]);
  HIP_OK(hipMemcpy(&ts, d_ts, sizeof(float), hipMemcpyDeviceToHost));
  if (!write_all(out, &ts, sizeof(float))) return fail("write", "ts");
  const struct { const void* d; size_t bytes; int wide; } outs[] = {
      {d_sc, n / 16, 0}, {d_bits, n / 8, 0}, {d_codes, n / 2, 0}, {d_yg, 2 * n, 1},
      {d_mg, n / 8, 0},  {d_yr, 2 * n, 1},   {d_mr, n / 8, 0},    {d_gin, 2 * n, 1}};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    void* h = outs[i].wide ? (void*)h16 : (void*)h8;
    HIP_OK(hipMemcpy(h, outs[i].d, outs[i].bytes, hipMemcpyDeviceToHost));
    if (!write_all(out, h, outs[i].bytes)) return fail("write", "outputs");
  }
  fclose(out);
  hipFree(d_xr); hipFree(d_xt); hipFree(d_g); hipFree(d_yg); hipFree(d_yr); hipFree(d_gin);
  hipFree(d_sc); hipFree(d_bits); hipFree(d_codes); hipFree(d_mg); hipFree(d_mr); hipFree(d_ts); hipFree(d_ws);
  free(h_in); free(h8); free(h16);
  printf("trace_c_smoke: %lld x %lld done, ts = %.9g\n", (long long)rows, (long long)cols, (double)ts);
  return 0;
}
