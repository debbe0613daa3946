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
  bool pv8;                     // P.V in e4m3 as well (implies fp8)
  float eps;
};

// Views into the caller's workspace (layout fixed by workspace_layout()).
struct Workspace {
  double* qsum;    // [BH, T, D]  column sums of each Q block (fp64)
  double* ksum;    // [BH, T, D]  column sums of each K block
  double* mu;      // [BH, D]     token mean of K (fp64)
  double* qhat;    // [BH, T, D]  projected pooled Q
  double* khatT;   // [BH, D, T]  projected pooled K~, transposed
  uint64_t* keys;  // [BH, T, T]  block scores as order-preserving 64-bit keys
  float* hpart;    // [BH, P, D, D] chunk partials of h_sum (transposed like h)
  float* zpart;    // [BH, P, D]
  uint16_t* vt;    // bf16 modes: [BH, T, D, 64] V of each key block, transposed, keys permuted;
                   // with e4m3 P.V the same region holds [BH, T, D, 64] bytes: e4m3 codes of
                   // V * 2^-e, row c (a channel) holding key 16mt + 4g + rr at byte 16g + 4mt + rr
  uint8_t* vexp;   // e4m3 P.V only: [BH, T, D] the biased exponents e + 127 of the V scales,
                   // channel c = 16dt + f at byte 8f + dt
  uint8_t* phik8;  // bf16 modes: [BH, T*64, D] e4m3 codes of 448 phi(K~) (pad rows 0); in each
                   // row, byte 32g + 8s + e holds feature 32s + 8g + e (g, s < 4, e < 8)
  float* zblk;     // bf16 modes: [BH, T, D] z_j of every key block
  float* zrout;    // bf16 modes: [BH, T, D] Z_R(i) = sum of z_j over the routed blocks of row i
  uint16_t* hbf;   // bf16 modes: [BH, D, D] h_sum (rows c, columns a) in bf16, 16-byte chunk k of
                   // row c stored at chunk k ^ (c % 16): the LDS image the forward epilogue uses
};

size_t workspace_layout(const Geometry& g, Workspace* ws, char* base);
size_t route_layout(const Geometry& g, Workspace* ws, char* base);

// Views into the caller's backward workspace (layout fixed by bwd_workspace_layout()).  The
// first three are written by the forward pass when it is given the backward workspace.
struct BwdWorkspace {
  uint16_t* os;         // [BH, N, D] O_s of the forward (bf16)
  uint16_t* ol;         // [BH, N, D] O_l of the forward (bf16)
  float* inv_den;       // [BH, 64T] 1 / (phi(q).Z_i + eps) of the forward (0 with every block routed)
  uint16_t* q8t;        // [BH, T, D, 64] e4m3 values of the Q codes, transposed likewise
  uint16_t* phqdt;      // [BH, T, D, 64] phi(q) / den, transposed likewise
  uint16_t* k8t;        // [BH, T, D, 64] e4m3 values of the K~ codes, transposed likewise
  uint16_t* phkt;       // [BH, T, D, 64] phi(K~), transposed likewise (pad tokens 0)
  uint16_t* htimg;      // [BH, D, D] bf16 h_sum transposed (rows a), in its LDS layout
  float* qrec;          // [BH, T, 256] per query block: -lse log2(e) [64] (-inf past N), D_q[64], zeros
  float* dden;          // [BH, 64T]
  int32_t* inv;         // [BH, T, T] per key block: the query blocks routing to it, ascending
  int32_t* inv_cnt;     // [BH, T]
  float* dZ;            // [BH, T, D] dZ_i
  float* gpart;         // [BH, ceil(T/8), D, D] partials of G_tot
  float* zpart;         // [BH, ceil(T/8), D] partials of dZ_tot
  float* g_tot;         // [BH, D, D] sum over tokens of (phi(q)/den)^T dO
  float* dZ_tot;        // [BH, D]
  float* dalpha_part;   // [BH, T, D]
  float* dkt;           // [BH, 64T, D] dK~ in fp32, before the key-smoothing correction
  float* colsum_part;   // [BH, T, D] column sums of dK~ over each key block
  float* dk_mean;       // [BH, D]
};

// backward workspace geometry (the backward kernels and the layout below share it)
constexpr int kRec = 256;                 // floats per query block in the key side's record
constexpr int kGChunk = 8;                // query blocks per partial of G_tot
size_t bwd_workspace_layout(const Geometry& g, BwdWorkspace* ws, char* base);

hipError_t launch_route(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s);
hipError_t launch_route_soft(const Geometry& g, const sla2_tensors& t, const Workspace& ws, double tau,
                             float* soft_mask, float* lambda, hipStream_t s);
hipError_t launch_precompute(const Geometry& g, const sla2_tensors& t, const Workspace& ws, hipStream_t s);
hipError_t launch_fwd(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const BwdWorkspace* bw,
                      hipStream_t s);
hipError_t launch_sum_parts(const float* parts, const float* zparts, int P, int D, int BH, float* out,
                            float* zout, hipStream_t s);
hipError_t launch_bwd(const Geometry& g, const sla2_tensors& t, const Workspace& ws, const BwdWorkspace& bw,
                      const void* dout, void* dq, void* dk, void* dv, float* dalpha, hipStream_t s);
hipError_t launch_selftest_mfma(int which, const void* a, const void* b, void* d, hipStream_t s);

}  // namespace sla2
