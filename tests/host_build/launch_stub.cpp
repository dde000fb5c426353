// Host-only stand-ins for the kernel launchers, so that the C-ABI layer
// (fa_api.cpp) can be built with the host sanitizers and driven by the CPU
// ABI tests without a GPU or device code.  A call that passes validation
// reaches these and launches nothing; it is counted, so a test can tell that
// validation let a call through.
#include <hip/hip_runtime_api.h>

#include "fa_launch.h"

extern "C" int fa_stub_launches = 0;

namespace fa {

// The projection's two compiled tiles (features x tokens): the large one for
// grids of at least four workgroups per CU of a 256-CU device.
ProjTiling proj_tiling(int64_t M, int64_t ncol) {
  const int64_t large = ((ncol + 255) / 256) * ((M + 255) / 256);
  if (large >= 4 * 256) return {1, 256, 256};
  return {0, 128, 128};
}

hipError_t launch_fwd(Dtype, int, bool, const FwdParams&, hipStream_t) {
  ++fa_stub_launches;
  return hipSuccess;
}

hipError_t launch_qkv_proj(Dtype, const ProjParams&, hipStream_t) {
  ++fa_stub_launches;
  return hipSuccess;
}

hipError_t launch_bwd(Dtype, int, bool, const BwdParams& p, hipStream_t) {
  ++fa_stub_launches;
  return p.delta != nullptr ? hipSuccess : hipErrorInvalidValue;
}

// A stand-in address for the static workspace (never dereferenced here).
hipError_t bwd_scratch(hipStream_t, float** out) {
  static float stand_in[4];
  *out = stand_in;
  return hipSuccess;
}

}  // namespace fa
