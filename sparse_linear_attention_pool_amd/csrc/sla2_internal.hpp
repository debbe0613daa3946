// Host-side launch interface shared by the SLA2 translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sla2.h"

namespace sla2 {

// Key blocks summed into one partial of h_sum / z_sum by the precompute kernels.
// 13 key blocks per workgroup: the C2 head count and length (12 x 512 blocks) then fill the
// 512 workgroup slots of a 256-CU MI355X (two per CU) in one round, with no tail.
constexpr int kChunk = 13;

struct Geometry {
  int B, H, N, D, T, topk, P;   // P = ceil(T / kChunk)
  int BH;
  bool smooth_k, fp8, bf16;
  float eps;
};

// Views into the caller's workspace (layout fixed by workspace_layout()).
struct Workspace {
  double* qsum;    // [BH, T, D]  column sums of each Q block (fp64)
  double* ksum;    // [BH, T, D]  column sums of each K block
  double* mu;      // [BH, D]     token mean of K (fp64)
  double* qhat;    // [BH, T, D]  projected pooled Q
  double* khatT;   // [BH, D, T]  projected pooled K~, transposed
  float* hpart;    // [BH, P, D, D] chunk partials of h_sum (transposed like h)
  float* zpart;    // [BH, P, D]
  uint16_t* vt;    // bf16 modes: [BH, T, D, 64] V of each key block, transposed, keys permuted
  uint8_t* phik8;  // bf16 modes: [BH, T*64, D] e4m3 codes of 448 phi(K~) (pad rows 0); in each
                   // row, byte 32g + 8s + e holds feature 32s + 8g + e (g, s < 4, e < 8)
  float* zblk;     // bf16 modes: [BH, T, D] z_j of every key block
  float* zrout;    // bf16 modes: [BH, T, D] Z_R(i) = sum of z_j over the routed blocks of row i
  uint16_t* hbf;   // bf16 modes: [BH, D, D] h_sum (rows c, columns a) in bf16, 16-byte chunk k of
                   // row c stored at chunk k ^ (c % 16): the LDS image the forward epilogue uses
};

size_t workspace_layout(const Geometry& g, Workspace* ws, char* base);

// Views into the caller's backward workspace (layout fixed by bwd_workspace_layout()).
struct BwdWorkspace {
  uint16_t* dos;        // [BH, 64T, D] alpha * dO in bf16 (rows past N zero)
  uint16_t* dot;        // [BH, T, D, 64] dos transposed per block
  uint16_t* qt;         // [BH, T, D, 64] dequantised e4m3 Q, transposed per block
  uint16_t* kt;         // [BH, T, D, 64] dequantised e4m3 K~, transposed per block
  int32_t* inv;         // [BH, T, T] per key block: the query blocks routing to it, ascending
  int32_t* inv_cnt;     // [BH, T]
  float* dsum;          // [BH, 64T] rowsum(dO_s * O_s)
  float* dH;            // [BH, T, D, D] dH_i
  float* dZ;            // [BH, T, D]
  float* dH_tot;        // [BH, D, D]
  float* dZ_tot;        // [BH, D]
  float* dalpha_part;   // [BH, T, D]
  float* dkt;           // [BH, 64T, D] dK~ in fp32, before the key-smoothing correction
  float* colsum_part;   // [BH, ceil(N/256), D]
  float* dk_mean;       // [BH, D]
};

size_t bwd_workspace_layout(const Geometry& g, BwdWorkspace* ws, char* base);

hipError_t launch_route(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s);
hipError_t launch_route_soft(const Geometry& g, const sla2_tensors& t, const Workspace& ws, double tau,
                             float* soft_mask, float* lambda, hipStream_t s);
hipError_t launch_precompute(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s);
hipError_t launch_fwd(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s);
hipError_t launch_sum_parts(const float* parts, const float* zparts, int P, int D, int BH, float* out,
                            float* zout, hipStream_t s);
hipError_t launch_bwd(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const BwdWorkspace& bw,
                      const void* dout, void* dq, void* dk, void* dv, float* dalpha, hipStream_t s);
hipError_t launch_selftest_mfma(int which, const void* a, const void* b, void* d, hipStream_t s);

}  // namespace sla2
