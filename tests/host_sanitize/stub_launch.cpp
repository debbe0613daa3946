// Launchers with no GPU behind them, for the host-only sanitizer build of the C-ABI layer
// (sla2_api.hip): argument checks, buffer sizes and workspace layouts run for real; a call that
// gets through them reaches one of these, which touches nothing and reports the HIP error
// `kStubError`, so the driver also sees how a failed launch is reported.
#include "sla2_internal.hpp"

namespace sla2 {

constexpr hipError_t kStubError = hipErrorInvalidConfiguration;

hipError_t launch_route(const Geometry&, const sla2_tensors&, const Workspace&, hipStream_t) { return kStubError; }
hipError_t launch_route_soft(const Geometry&, const sla2_tensors&, const Workspace&, double, float*, float*,
                             hipStream_t) {
  return kStubError;
}
hipError_t launch_precompute(const Geometry&, const sla2_tensors&, const Workspace&, hipStream_t) { return kStubError; }
hipError_t launch_fwd(const Geometry&, const sla2_tensors&, const Workspace&, const BwdWorkspace*, hipStream_t) {
  return kStubError;
}
hipError_t launch_sum_parts(const float*, const float*, int, int, int, float*, float*, hipStream_t) { return kStubError; }
hipError_t launch_bwd(const Geometry&, const sla2_tensors&, const Workspace&, const BwdWorkspace&, const void*, void*,
                      void*, void*, float*, hipStream_t) {
  return kStubError;
}
hipError_t launch_selftest_mfma(int, const void*, const void*, void*, hipStream_t) { return kStubError; }

}  // namespace sla2
