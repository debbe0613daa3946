// Host-only driver of the C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer:
// every argument check, the buffer sizes and workspace layouts of the named workloads, the
// status strings and error messages, and the report of a failed launch (the stub launchers
// fail with a HIP error).  Nothing runs on a GPU.  Exit status 0 and "sanitize driver ok" when
// every expectation holds.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "sla2.h"

static int g_fail = 0;

static void expect(bool ok, const char* what) {
  if (!ok) {
    printf("FAIL: %s (last error: %s)\n", what, sla2_last_error());
    ++g_fail;
  }
}

static sla2_params params(int B, int H, int N, int d, int topk, int dtype, int qk) {
  sla2_params p;
  p.B = B; p.H = H; p.N = N; p.d = d; p.block = 64; p.topk = topk; p.smooth_k = 1;
  p.dtype = dtype; p.qk_mode = qk; p.eps = 1e-5f;
  return p;
}

int main() {
  sla2_sizes sz;
  // named workloads: fp32 native, bf16 native, bf16 FP8 (C2, C3), low-bit P.V, backward shape
  const sla2_params ok[] = {params(1, 2, 1000, 64, 4, SLA2_F32, SLA2_QK_NATIVE),
                            params(1, 2, 32760, 128, 26, SLA2_BF16, SLA2_QK_NATIVE),
                            params(1, 12, 32760, 128, 15, SLA2_BF16, SLA2_QK_FP8_E4M3),
                            params(1, 40, 75600, 128, 35, SLA2_BF16, SLA2_QK_FP8_E4M3),
                            params(2, 3, 4097, 128, 7, SLA2_BF16, SLA2_QK_PV_FP8_E4M3),
                            params(1, 1, 262144, 128, 4096, SLA2_BF16, SLA2_QK_FP8_E4M3)};
  for (const sla2_params& p : ok) {
    expect(sla2_buffer_sizes(&p, &sz) == SLA2_OK, "sizes of a valid workload");
    expect(sz.workspace > 0 && sz.lut == (size_t)p.B * p.H * ((p.N + 63) / 64) * p.topk * 4, "lut size");
  }
  // every rejected parameter, with its status
  struct Bad { sla2_params p; int status; const char* what; };
  Bad bad[] = {
      {params(0, 1, 100, 128, 1, SLA2_BF16, 0), SLA2_ERR_INVALID_ARG, "B = 0"},
      {params(1, 1, 0, 128, 1, SLA2_BF16, 0), SLA2_ERR_INVALID_ARG, "N = 0"},
      {params(1, 1, 100, 96, 1, SLA2_F32, 0), SLA2_ERR_INVALID_ARG, "d = 96"},
      {params(1, 1, 100, 128, 1, 7, 0), SLA2_ERR_INVALID_ARG, "dtype 7"},
      {params(1, 1, 100, 128, 1, SLA2_BF16, 9), SLA2_ERR_INVALID_ARG, "qk_mode 9"},
      {params(1, 1, 100, 128, 0, SLA2_BF16, 0), SLA2_ERR_INVALID_ARG, "topk 0"},
      {params(1, 1, 100, 128, 3, SLA2_BF16, 0), SLA2_ERR_INVALID_ARG, "topk > T"},
      {params(1, 1, 262145, 128, 1, SLA2_BF16, 0), SLA2_ERR_UNSUPPORTED, "T > 4096"},
      {params(1 << 20, 1 << 10, 262144, 128, 1, SLA2_BF16, 0), SLA2_ERR_INVALID_ARG, "B*H*T overflow"},
      {params(1, 1, 100, 128, 1, SLA2_F32, SLA2_QK_FP8_E4M3), SLA2_ERR_UNSUPPORTED, "FP8 with fp32"},
      {params(1, 1, 100, 64, 1, SLA2_BF16, 0), SLA2_ERR_UNSUPPORTED, "bf16 with d = 64"},
  };
  for (Bad& b : bad) {
    expect(sla2_buffer_sizes(&b.p, &sz) == b.status, b.what);
    expect(strlen(sla2_last_error()) > 0, "message of a rejected call");
  }
  sla2_params pe = params(1, 1, 100, 128, 1, SLA2_BF16, 0);
  pe.block = 32;
  expect(sla2_buffer_sizes(&pe, &sz) == SLA2_ERR_INVALID_ARG, "block 32");
  pe = params(1, 1, 100, 128, 1, SLA2_BF16, 0);
  pe.eps = NAN;
  expect(sla2_buffer_sizes(&pe, &sz) == SLA2_ERR_INVALID_ARG, "eps NaN");
  pe.eps = 2.f;
  expect(sla2_buffer_sizes(&pe, &sz) == SLA2_ERR_INVALID_ARG, "eps 2");
  pe = params(1, 1, 100, 128, 1, SLA2_BF16, 0);
  pe.smooth_k = 2;
  expect(sla2_buffer_sizes(&pe, &sz) == SLA2_ERR_INVALID_ARG, "smooth_k 2");
  expect(sla2_buffer_sizes(nullptr, &sz) == SLA2_ERR_INVALID_ARG, "NULL params");

  // entry points: NULL tensors, then missing buffers, then a complete set (never dereferenced)
  const sla2_params p = params(1, 12, 32760, 128, 15, SLA2_BF16, SLA2_QK_FP8_E4M3);
  expect(sla2_route(&p, nullptr, nullptr) == SLA2_ERR_INVALID_ARG, "route without tensors");
  expect(sla2_linear_precompute(&p, nullptr, nullptr) == SLA2_ERR_INVALID_ARG, "precompute without tensors");
  expect(sla2_attention_fwd(&p, nullptr, nullptr) == SLA2_ERR_INVALID_ARG, "fwd without tensors");
  sla2_tensors t;
  memset(&t, 0, sizeof t);
  expect(sla2_route(&p, &t, nullptr) == SLA2_ERR_INVALID_ARG, "route with NULL buffers");
  expect(sla2_attention_bwd(&p, &t, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != SLA2_OK,
         "backward with NULL buffers");
  static char fake[256] __attribute__((aligned(256)));
  void** f = reinterpret_cast<void**>(&t);
  for (size_t i = 0; i < sizeof t / sizeof(void*); ++i) f[i] = fake;
  expect(sla2_route_soft(&p, &t, -1.f, (float*)fake, (float*)fake, nullptr) == SLA2_ERR_INVALID_ARG, "tau < 0");
  // a complete set gets through the checks to the (stub) launcher, whose HIP error is reported
  const int st = sla2_route(&p, &t, nullptr);
  expect(st == SLA2_ERR_HIP, "a failed launch reports SLA2_ERR_HIP");
  expect(std::string(sla2_last_error()).find("sla2_route") != std::string::npos, "message names the call");
  expect(sla2_linear_precompute(&p, &t, nullptr) == SLA2_ERR_HIP, "precompute launch failure");
  expect(sla2_attention_fwd(&p, &t, nullptr) == SLA2_ERR_HIP, "fwd launch failure");
  // a backward workspace off its 256-byte alignment is rejected before anything runs
  t.workspace_bwd = fake + 16;
  expect(sla2_attention_fwd(&p, &t, nullptr) == SLA2_ERR_INVALID_ARG, "misaligned backward workspace");

  for (int s : {(int)SLA2_OK, (int)SLA2_ERR_INVALID_ARG, (int)SLA2_ERR_UNSUPPORTED, (int)SLA2_ERR_HIP, 12345})
    expect(sla2_status_string(s) != nullptr && strlen(sla2_status_string(s)) > 0, "status string");
  if (g_fail == 0) printf("sanitize driver ok\n");
  return g_fail == 0 ? 0 : 1;
}
