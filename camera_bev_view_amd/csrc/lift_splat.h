// Internal interface between the C-ABI host layer and the Lift-Splat kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace fbev {

// One Lift-Splat problem, validated by the host layer.  Per batch sample the
// pixel index is p = (n H + v) W + u; depth is [B, NHW, D] and context
// [B, NHW, C], both contiguous.
struct LssArgs {
  const float* depth;     // alpha, [B, N, H, W, D]
  const float* ctx;       // c, [B, N, H, W, C]
  const float* K;         // [B, N, 3, 3] intrinsics (feature-map pixels)
  const float* R;         // [B, N, 3, 3] ego -> camera rotation
  const float* t;         // [B, N, 3]
  const float* grad;      // backward: dL/dout [B, C, X, Y]
  float* out;             // forward: [B, C, X, Y]
  float* gdep;            // backward: [B, N, H, W, D]
  float* gctx;            // backward: [B, N, H, W, C]
  int B, N, H, W, C, D, X, Y;
  double dmin, dstep;     // bin k sits at camera depth dmin + k dstep
  double x_min, y_min, cdx, cdy;   // cell (i, j) covers [x_min + i cdx, +cdx) x [y_min + j cdy, +cdy)
  // set by the launcher
  int tiles_x, tiles_y, c_lo, Cg;
  double inv_cdx, inv_cdy;
  float f_dlo, f_dhi, f_dmin, f_inv_dstep, f_slack;   // fp32 constants of the candidate test
};

hipError_t launch_lss_forward(LssArgs a, hipStream_t stream);
hipError_t launch_lss_backward(LssArgs a, hipStream_t stream);

}  // namespace fbev
