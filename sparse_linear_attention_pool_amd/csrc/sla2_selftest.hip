// Diagnostic kernel: one wave runs one matrix-core instruction of the kind the kernels use, so
// that a test can pin the operand and scale lane layouts they assume (C = 0).
#include "sla2_device.hpp"
#include "sla2_internal.hpp"

namespace sla2 {

// which = 0: bf16 16x16x32; 1: e4m3 16x16x128; 2: fp64 16x16x4; 3: e4m3 16x16x128 with E8M0
// scales, lane l's scale words after the 64 x 32 code bytes of a and of b, byte 2 of the word
// selected for A (the form the low-bit P.V products use: op_sel picks the byte) and byte 0 for B;
// 4: the e4m3 decode the kernels use, lane l decoding the four code bytes of word l of a.
__global__ __launch_bounds__(64) void selftest_mfma_kernel(int which, const u32x4* a, const u32x4* b, float4* d) {
  const int l = threadIdx.x;
  f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
  if (which == 4) {
    r = e4m3_decode4(reinterpret_cast<const uint32_t*>(a)[l]);
    d[l] = make_float4(r[0], r[1], r[2], r[3]);
    return;
  }
  if (which == 2) {
    const f64x4 r64 = mfma_f64(reinterpret_cast<const double*>(a)[l], reinterpret_cast<const double*>(b)[l],
                               f64x4{0.0, 0.0, 0.0, 0.0});
    double* d64 = reinterpret_cast<double*>(d);
    d64[4 * l + 0] = r64[0];
    d64[4 * l + 1] = r64[1];
    d64[4 * l + 2] = r64[2];
    d64[4 * l + 3] = r64[3];
    return;
  }
  if (which == 0) {
    r = mfma_bf16(__builtin_bit_cast(bf16x8, a[l]), __builtin_bit_cast(bf16x8, b[l]), r);
  } else {
    const u32x4 a0 = a[2 * l], a1 = a[2 * l + 1], b0 = b[2 * l], b1 = b[2 * l + 1];
    const i32x8 ao = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8 bo = i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    if (which == 1) {
      r = mfma_fp8(ao, bo, r);
    } else {
      const int sa = reinterpret_cast<const int*>(a + 128)[l], sb = reinterpret_cast<const int*>(b + 128)[l];
      r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ao, bo, r, 0, 0, 2, sa, 0, sb);
    }
  }
  d[l] = make_float4(r[0], r[1], r[2], r[3]);
}

hipError_t launch_selftest_mfma(int which, const void* a, const void* b, void* d, hipStream_t s) {
  hipLaunchKernelGGL(selftest_mfma_kernel, dim3(1), dim3(64), 0, s, which, (const u32x4*)a, (const u32x4*)b,
                     (float4*)d);
  return hipGetLastError();
}

}  // namespace sla2
