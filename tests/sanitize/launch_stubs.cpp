// Host-only stand-ins for the kernel launchers and the one HIP runtime call
// of the C-ABI layer, so that its validation code can be built and run under
// AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a GPU.
// Each launcher records that it was reached and the arguments it got; none
// touches device memory.
#include <hip/hip_runtime_api.h>

#include "../../depth_wise_kv_amd/csrc/moda_internal.h"
#include "../../depth_wise_kv_amd/csrc/moda_small.h"

int g_stub_launches = 0;

extern "C" const char *hipGetErrorString(hipError_t e) {
  return e == hipSuccess ? "hipSuccess" : "stubbed HIP error";
}

namespace moda {

static hipError_t reached() {
  ++g_stub_launches;
  return hipSuccess;
}

hipError_t launch_fwd_mfma(const FwdArgs &a, int G, int waves, hipStream_t) {
  if (G < 1 || (waves != 4 && waves != 8 && waves != kFwdKeySplit) || a.T < 1)
    return hipErrorInvalidValue;
  return reached();
}
hipError_t launch_pack_mfma(const PackArgs &a, hipStream_t) {
  return a.nblk < 1 ? hipErrorInvalidValue : reached();
}
hipError_t launch_bwd(const BwdArgs &a, hipStream_t) {
  return a.T < 1 ? hipErrorInvalidValue : reached();
}
hipError_t launch_decode(const DecArgs &a, hipStream_t) {
  return a.nsplit < 1 ? hipErrorInvalidValue : reached();
}
hipError_t launch_append(const AppendArgs &a, bool, int row_bytes, hipStream_t) {
  return (a.n < 1 || row_bytes < 16) ? hipErrorInvalidValue : reached();
}
hipError_t launch_fwd_generic(const FwdArgs &a, bool, hipStream_t) {
  return a.T < 1 ? hipErrorInvalidValue : reached();
}
hipError_t launch_fwd_small(const FwdArgs &a, bool bf16, hipStream_t) {
  return !small_supported(bf16, a.d, a.Hq / a.Hkv) || a.T < 1 ? hipErrorInvalidValue : reached();
}
hipError_t launch_pack_generic(const PackArgs &a, bool, hipStream_t) {
  return a.T < 1 ? hipErrorInvalidValue : reached();
}
hipError_t decode_scratch(void **ptr) {
  *ptr = (void *)(uintptr_t)0x7f0000000000ull;  // a fake, 256-byte aligned device address
  return hipSuccess;
}

}  // namespace moda
