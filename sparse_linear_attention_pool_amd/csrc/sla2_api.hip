// C entry points of libsla2: argument checks, buffer sizes, workspace layout, launches.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <string>

#include "sla2_internal.hpp"

// Scratch of sla2_route_noalloc: the router's fp64 block sums, key-mean partials, projected
// pooled rows and score keys, for callers that cannot allocate device memory.  Each GPU the library runs on
// holds its own copy until the process ends.  Host code never passes this name to a kernel (it
// is a host-side stand-in there): it looks up the device address once per device and uses that.
constexpr size_t kRouteScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kRouteScratchBytes];

namespace sla2 {
namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return SLA2_OK;
  return fail(SLA2_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_params(const sla2_params* p, Geometry* g) {
  if (p == nullptr) return fail(SLA2_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 1 || p->H < 1 || p->N < 1) return fail(SLA2_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (p->d != 64 && p->d != 128) return fail(SLA2_ERR_INVALID_ARG, "d must be 64 or 128 (got %d)", p->d);
  if (p->block != 64) return fail(SLA2_ERR_INVALID_ARG, "block must be 64 (got %d)", p->block);
  if (p->dtype != SLA2_F32 && p->dtype != SLA2_BF16) return fail(SLA2_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->qk_mode != SLA2_QK_NATIVE && p->qk_mode != SLA2_QK_FP8_E4M3 && p->qk_mode != SLA2_QK_PV_FP8_E4M3)
    return fail(SLA2_ERR_INVALID_ARG, "unknown qk_mode %d", p->qk_mode);
  if (p->smooth_k != 0 && p->smooth_k != 1) return fail(SLA2_ERR_INVALID_ARG, "smooth_k must be 0 or 1");
  if (!(p->eps >= 0.f) || p->eps > 1.f) return fail(SLA2_ERR_INVALID_ARG, "eps must be in [0, 1]");
  const long long T = ((long long)p->N + 63) / 64;
  if (T > 4096) return fail(SLA2_ERR_UNSUPPORTED, "at most 4096 blocks per sequence (N <= 262144)");
  if (p->topk < 1 || p->topk > T) return fail(SLA2_ERR_INVALID_ARG, "topk must be in [1, %lld] (got %d)", T, p->topk);
  if ((long long)p->B * p->H * T > 0x7fffffffLL) return fail(SLA2_ERR_INVALID_ARG, "B*H*T too large");
  if (p->qk_mode != SLA2_QK_NATIVE && p->dtype != SLA2_BF16)
    return fail(SLA2_ERR_UNSUPPORTED, "FP8 Q.K^T needs bf16 inputs");
  if (p->dtype == SLA2_BF16 && p->d != 128) return fail(SLA2_ERR_UNSUPPORTED, "bf16 kernels need d = 128");
  g->B = p->B;
  g->H = p->H;
  g->N = p->N;
  g->D = p->d;
  g->T = (int)T;
  g->topk = p->topk;
  g->P = (g->T + kChunk - 1) / kChunk;
  g->BH = p->B * p->H;
  g->smooth_k = p->smooth_k != 0;
  g->fp8 = p->qk_mode != SLA2_QK_NATIVE;
  g->pv8 = p->qk_mode == SLA2_QK_PV_FP8_E4M3;
  g->bf16 = p->dtype == SLA2_BF16;
  g->eps = p->eps;
  return SLA2_OK;
}

}  // namespace

// The router's part of the workspace (the first six regions of workspace_layout), used by
// sla2_route and sla2_route_soft only.  Returns its size in bytes.
size_t route_layout(const Geometry& g, Workspace* ws, char* base) {
  const size_t BH = g.BH, T = g.T, D = g.D, P32 = (g.T + 31) / 32;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return base ? base + o : nullptr;
  };
  Workspace w{};
  w.qsum = (double*)take(BH * T * D * sizeof(double));
  w.ksum = (double*)take(BH * T * D * sizeof(double));
  w.mu = (double*)take((BH * P32 * D + BH * D) * sizeof(double));
  w.qhat = (double*)take(BH * T * D * sizeof(double));
  w.khatT = (double*)take(BH * D * T * sizeof(double));
  w.keys = (uint64_t*)take(BH * T * T * sizeof(uint64_t));
  if (ws) *ws = w;
  return off;
}

size_t workspace_layout(const Geometry& g, Workspace* ws, char* base) {
  const size_t BH = g.BH, T = g.T, D = g.D, P = g.P;
  Workspace w;
  size_t off = route_layout(g, &w, base);
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return base ? base + o : nullptr;
  };
  w.hpart = (float*)take(BH * P * D * D * sizeof(float));
  w.zpart = (float*)take(BH * P * D * sizeof(float));
  w.vt = (uint16_t*)take(g.bf16 ? BH * T * D * 64 * (g.pv8 ? 1 : sizeof(uint16_t)) : 0);
  w.vexp = (uint8_t*)take(g.pv8 ? BH * T * D : 0);
  w.phik8 = (uint8_t*)take(g.bf16 ? BH * T * 64 * D : 0);
  w.zblk = (float*)take(g.bf16 ? BH * T * D * sizeof(float) : 0);
  w.zrout = (float*)take(g.bf16 ? BH * T * D * sizeof(float) : 0);
  w.hbf = (uint16_t*)take(g.bf16 ? BH * D * D * sizeof(uint16_t) : 0);
  if (ws) *ws = w;
  return off;
}

// Layout of the backward pass's scratch (sla2_sizes.workspace_bwd).
size_t bwd_workspace_layout(const Geometry& g, BwdWorkspace* ws, char* base) {
  const size_t BH = g.BH, T = g.T, D = g.D, N = g.N;
  const size_t pg = (g.T + kGChunk - 1) / kGChunk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return base ? base + o : nullptr;
  };
  BwdWorkspace w;
  w.os = (uint16_t*)take(BH * N * D * 2);
  w.ol = (uint16_t*)take(BH * N * D * 2);
  w.inv_den = (float*)take(BH * T * 64 * 4);
  w.q8t = (uint16_t*)take(BH * T * D * 64 * 2);
  w.phqdt = (uint16_t*)take(BH * T * D * 64 * 2);
  w.k8t = (uint16_t*)take(BH * T * D * 64 * 2);
  w.phkt = (uint16_t*)take(BH * T * D * 64 * 2);
  w.htimg = (uint16_t*)take(BH * D * D * 2);
  w.qrec = (float*)take(BH * T * kRec * 4);
  w.dden = (float*)take(BH * T * 64 * 4);
  w.inv = (int32_t*)take(BH * T * T * 4);
  w.inv_cnt = (int32_t*)take(BH * T * 4);
  w.dZ = (float*)take(BH * T * D * 4);
  w.gpart = (float*)take(BH * pg * D * D * 4);
  w.zpart = (float*)take(BH * pg * D * 4);
  w.g_tot = (float*)take(BH * D * D * 4);
  w.dZ_tot = (float*)take(BH * D * 4);
  w.dalpha_part = (float*)take(BH * T * D * 4);
  w.dkt = (float*)take(BH * T * 64 * D * 4);
  w.colsum_part = (float*)take(BH * T * D * 4);
  w.dk_mean = (float*)take(BH * D * 4);
  if (ws) *ws = w;
  return off;
}

namespace {

std::mutex g_scratch_mu;
constexpr int kMaxDevices = 256;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device ordinal, once looked up

// The device address of this GPU's copy of `scratch` (the current device's), looked up on the
// first call on that device.
int route_scratch(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(SLA2_ERR_UNSUPPORTED, "%s: device ordinal %d", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (ptr == nullptr) return fail(SLA2_ERR_HIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SLA2_OK;
}

}  // namespace

}  // namespace sla2

using namespace sla2;

namespace {

int fill_sizes(const Geometry& g, sla2_sizes* s) {
  const size_t BH = g.BH, T = g.T, D = g.D, N = g.N;
  const size_t es = g.bf16 ? 2 : 4;
  memset(s, 0, sizeof *s);
  s->q_pool = BH * T * D * 4;
  s->k_pool = BH * T * D * 4;
  s->k_mean = BH * D * 4;
  s->lut = BH * T * g.topk * 4;
  s->mask = BH * T * T;
  if (g.fp8) {
    s->q8 = BH * T * 64 * D;
    s->k8 = BH * T * 64 * D;
    s->q_scale = BH * T * 4;
    s->k_scale = BH * T * 4;
  }
  s->h = BH * T * D * D * es;
  s->z = BH * T * D * 4;
  s->h_sum = BH * D * D * 4;
  s->z_sum = BH * D * 4;
  s->o = BH * N * D * es;
  s->lse = BH * N * 4;
  s->workspace = workspace_layout(g, nullptr, nullptr);
  s->workspace_bwd = (g.bf16 && g.fp8 && !g.pv8 && g.D == 128) ? bwd_workspace_layout(g, nullptr, nullptr) : 0;
  return SLA2_OK;
}

#define REQUIRE(ptr, name) \
  if ((ptr) == nullptr) return fail(SLA2_ERR_INVALID_ARG, "%s: tensor '%s' is NULL", fn, name)

int prepare(const char* fn, const sla2_params* p, const sla2_tensors* t, Geometry* g, Workspace* ws) {
  const int st = check_params(p, g);
  if (st != SLA2_OK) return st;
  if (t == nullptr) return fail(SLA2_ERR_INVALID_ARG, "%s: tensors is NULL", fn);
  REQUIRE(t->workspace, "workspace");
  if (((uintptr_t)t->workspace & 255) != 0) return fail(SLA2_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  workspace_layout(*g, ws, (char*)t->workspace);
  return SLA2_OK;
}

}  // namespace

extern "C" {

int sla2_buffer_sizes(const sla2_params* p, sla2_sizes* out) {
  Geometry g;
  const int st = check_params(p, &g);
  if (st != SLA2_OK) return st;
  if (out == nullptr) return fail(SLA2_ERR_INVALID_ARG, "sla2_buffer_sizes: out is NULL");
  return fill_sizes(g, out);
}

int sla2_route(const sla2_params* p, const sla2_tensors* t, void* stream) {
  const char* fn = "sla2_route";
  Geometry g;
  Workspace ws;
  int st = prepare(fn, p, t, &g, &ws);
  if (st != SLA2_OK) return st;
  REQUIRE(t->q, "q");
  REQUIRE(t->k, "k");
  REQUIRE(t->q_pool, "q_pool");
  REQUIRE(t->k_pool, "k_pool");
  REQUIRE(t->k_mean, "k_mean");
  REQUIRE(t->lut, "lut");
  REQUIRE(t->mask, "mask");
  if (g.fp8) {
    REQUIRE(t->q8, "q8");
    REQUIRE(t->q_scale, "q_scale");
  }
  return hip_status(launch_route(g, *t, ws, (hipStream_t)stream), fn);
}

int sla2_route_noalloc(const sla2_params* p, const sla2_tensors* t, void* stream) {
  const char* fn = "sla2_route_noalloc";
  Geometry g;
  int st = check_params(p, &g);
  if (st != SLA2_OK) return st;
  if (t == nullptr) return fail(SLA2_ERR_INVALID_ARG, "%s: tensors is NULL", fn);
  const size_t need = route_layout(g, nullptr, nullptr);
  if (need > kRouteScratchBytes)
    return fail(SLA2_ERR_UNSUPPORTED,
                "%s: these sizes need %zu bytes of router scratch, more than the %zu this entry point holds "
                "(32 * d + 8 * ceil(N / 64) bytes per query block of every head); use sla2_route with a workspace",
                fn, need, kRouteScratchBytes);
  REQUIRE(t->q, "q");
  REQUIRE(t->k, "k");
  REQUIRE(t->q_pool, "q_pool");
  REQUIRE(t->k_pool, "k_pool");
  REQUIRE(t->k_mean, "k_mean");
  REQUIRE(t->lut, "lut");
  REQUIRE(t->mask, "mask");
  if (g.fp8) {
    REQUIRE(t->q8, "q8");
    REQUIRE(t->q_scale, "q_scale");
  }
  void* base = nullptr;
  st = route_scratch(fn, &base);
  if (st != SLA2_OK) return st;
  Workspace ws;
  route_layout(g, &ws, (char*)base);
  return hip_status(launch_route(g, *t, ws, (hipStream_t)stream), fn);
}

int sla2_route_soft(const sla2_params* p, const sla2_tensors* t, float tau, float* soft_mask, float* lambda,
                    void* stream) {
  const char* fn = "sla2_route_soft";
  Geometry g;
  Workspace ws;
  int st = prepare(fn, p, t, &g, &ws);
  if (st != SLA2_OK) return st;
  REQUIRE(t->q, "q");
  REQUIRE(t->k, "k");
  REQUIRE(t->q_pool, "q_pool");
  REQUIRE(t->k_pool, "k_pool");
  REQUIRE(t->k_mean, "k_mean");
  REQUIRE(t->lut, "lut");
  REQUIRE(t->mask, "mask");
  if (g.fp8) {
    REQUIRE(t->q8, "q8");
    REQUIRE(t->q_scale, "q_scale");
  }
  REQUIRE(soft_mask, "soft_mask");
  REQUIRE(lambda, "lambda");
  if (!(tau > 0.f) || !std::isfinite(tau)) return fail(SLA2_ERR_INVALID_ARG, "%s: tau must be positive and finite", fn);
  return hip_status(launch_route_soft(g, *t, ws, (double)tau, soft_mask, lambda, (hipStream_t)stream), fn);
}

int sla2_linear_precompute(const sla2_params* p, const sla2_tensors* t, void* stream) {
  const char* fn = "sla2_linear_precompute";
  Geometry g;
  Workspace ws;
  int st = prepare(fn, p, t, &g, &ws);
  if (st != SLA2_OK) return st;
  REQUIRE(t->k, "k");
  REQUIRE(t->v, "v");
  REQUIRE(t->k_mean, "k_mean");
  if (!g.bf16) {          // the fp32 forward reads the per-block statistics
    REQUIRE(t->h, "h");
    REQUIRE(t->z, "z");
  }
  REQUIRE(t->h_sum, "h_sum");
  REQUIRE(t->z_sum, "z_sum");
  if (g.fp8) {
    REQUIRE(t->k8, "k8");
    REQUIRE(t->k_scale, "k_scale");
  }
  return hip_status(launch_precompute(g, *t, ws, (hipStream_t)stream), fn);
}

int sla2_attention_fwd(const sla2_params* p, const sla2_tensors* t, void* stream) {
  const char* fn = "sla2_attention_fwd";
  Geometry g;
  Workspace ws;
  int st = prepare(fn, p, t, &g, &ws);
  if (st != SLA2_OK) return st;
  REQUIRE(t->q, "q");
  if (!g.bf16 || !g.fp8) REQUIRE(t->k, "k");
  REQUIRE(t->v, "v");
  REQUIRE(t->alpha, "alpha");
  REQUIRE(t->lut, "lut");
  if (!g.bf16) {
    REQUIRE(t->h, "h");
    REQUIRE(t->z, "z");
  }
  REQUIRE(t->h_sum, "h_sum");
  REQUIRE(t->z_sum, "z_sum");
  REQUIRE(t->o, "o");
  REQUIRE(t->k_mean, "k_mean");
  if (g.fp8) {
    REQUIRE(t->q8, "q8");
    REQUIRE(t->k8, "k8");
    REQUIRE(t->q_scale, "q_scale");
    REQUIRE(t->k_scale, "k_scale");
  }
  // a backward workspace makes this a training forward: it also stores what the backward reads
  BwdWorkspace bw;
  const bool keep = t->workspace_bwd != nullptr && g.bf16 && g.fp8 && !g.pv8 && g.D == 128;
  if (keep) {
    if (((uintptr_t)t->workspace_bwd & 255) != 0)
      return fail(SLA2_ERR_INVALID_ARG, "%s: workspace_bwd must be 256-byte aligned", fn);
    bwd_workspace_layout(g, &bw, (char*)t->workspace_bwd);
  }
  return hip_status(launch_fwd(g, *t, ws, keep ? &bw : nullptr, (hipStream_t)stream), fn);
}

int sla2_attention_bwd(const sla2_params* p, const sla2_tensors* t, const void* dout, void* dq, void* dk,
                       void* dv, float* dalpha, void* stream) {
  const char* fn = "sla2_attention_bwd";
  Geometry g;
  Workspace ws;
  int st = prepare(fn, p, t, &g, &ws);
  if (st != SLA2_OK) return st;
  if (!g.bf16 || !g.fp8 || g.pv8 || g.D != 128)
    return fail(SLA2_ERR_UNSUPPORTED, "%s: implemented for bf16 inputs with FP8 Q.K^T (bf16 P.V) and d = 128", fn);
  REQUIRE(t->q, "q");
  REQUIRE(t->k, "k");
  REQUIRE(t->v, "v");
  REQUIRE(t->alpha, "alpha");
  REQUIRE(t->k_mean, "k_mean");
  REQUIRE(t->lut, "lut");
  REQUIRE(t->mask, "mask");
  REQUIRE(t->q8, "q8");
  REQUIRE(t->q_scale, "q_scale");
  REQUIRE(t->k8, "k8");
  REQUIRE(t->k_scale, "k_scale");
  REQUIRE(t->h_sum, "h_sum");
  REQUIRE(t->z_sum, "z_sum");
  REQUIRE(t->lse, "lse");
  REQUIRE(t->workspace_bwd, "workspace_bwd");
  if (((uintptr_t)t->workspace_bwd & 255) != 0)
    return fail(SLA2_ERR_INVALID_ARG, "%s: workspace_bwd must be 256-byte aligned", fn);
  REQUIRE(dout, "dout");
  REQUIRE(dq, "dq");
  REQUIRE(dk, "dk");
  REQUIRE(dv, "dv");
  REQUIRE(dalpha, "dalpha");
  BwdWorkspace bw;
  bwd_workspace_layout(g, &bw, (char*)t->workspace_bwd);
  return hip_status(launch_bwd(g, *t, ws, bw, dout, dq, dk, dv, dalpha, (hipStream_t)stream), fn);
}

int sla2_selftest_mfma(int which, const void* a, const void* b, void* d, void* stream) {
  if (which < 0 || which > 4) return fail(SLA2_ERR_INVALID_ARG, "sla2_selftest_mfma: which must be 0 to 4");
  if (a == nullptr || b == nullptr || d == nullptr)
    return fail(SLA2_ERR_INVALID_ARG, "sla2_selftest_mfma: NULL operand");
  return hip_status(launch_selftest_mfma(which, a, b, d, (hipStream_t)stream), "sla2_selftest_mfma");
}

const char* sla2_status_string(int status) {
  switch (status) {
    case SLA2_OK: return "ok";
    case SLA2_ERR_INVALID_ARG: return "invalid argument";
    case SLA2_ERR_UNSUPPORTED: return "unsupported";
    case SLA2_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sla2_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
