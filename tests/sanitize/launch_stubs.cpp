// Host-only stand-ins for the kernel launchers of libflashbev, for the sanitizer
// build of the C-ABI host layer (flashbev_api.cpp).  Each records that it was
// reached and returns what `stub_status` says, so the harness can check that
// invalid calls never reach a launcher and that a launcher's failure comes back
// as FBEV_ERR_DEVICE.  No device code; nothing here touches a GPU.
#include <hip/hip_runtime.h>

#include "../../camera_bev_view_amd/csrc/deform_agg.h"
#include "../../camera_bev_view_amd/csrc/kernels.h"
#include "../../camera_bev_view_amd/csrc/lift_splat.h"

int stub_launches = 0;
hipError_t stub_status = hipSuccess;

extern "C" const char* hipGetErrorString(hipError_t e) {
  return e == hipSuccess ? "no error" : "stub launch failure";
}
extern "C" hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
extern "C" hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) {
  *d = 0;
  return hipSuccess;
}

namespace fbev {
namespace {
hipError_t reached() {
  ++stub_launches;
  return stub_status;
}
}  // namespace

hipError_t launch_forward(const Problem&, float*, uint8_t*, hipStream_t) { return reached(); }
hipError_t launch_backward(const Problem&, const float*, float*, hipStream_t) { return reached(); }
hipError_t launch_forward_temporal(const Problem&, float*, uint8_t*, bool, int, const float*, const float*, int,
                                   hipStream_t) {
  return reached();
}
hipError_t launch_backward_temporal(const Problem&, const float*, float*, int, const float*, float*, int,
                                    hipStream_t) {
  return reached();
}
// the real size for one batch sample and a grid of at least 1792 units: 12 fp64 partial sums per camera and
// workgroup, 1792 workgroups
size_t camera_grad_workspace_bytes(const Problem& p) { return (size_t)8 * 12 * 1792 * (size_t)(p.N > 0 ? p.N : 1); }
hipError_t launch_camera_backward(const Problem&, const float*, float*, float*, float*, void*, hipStream_t) {
  return reached();
}
hipError_t camera_scratch(int device, void** ptr) {
  if (device != 0) return hipErrorInvalidDevice;
  *ptr = reinterpret_cast<void*>(0x20000);
  return hipSuccess;
}
hipError_t launch_lss_forward(LssArgs, hipStream_t) { return reached(); }
hipError_t launch_lss_backward(LssArgs, hipStream_t) { return reached(); }
hipError_t launch_deform_forward(const DeformArgs&, hipStream_t) { return reached(); }
size_t deform_backward_workspace_bytes(const DeformArgs& a) { return (size_t)64 * (size_t)(a.Q > 0 ? a.Q : 1); }
hipError_t launch_deform_backward(DeformArgs, void*, hipStream_t) { return reached(); }
}  // namespace fbev
