// Temporal fusion of BEV maps for gfx950: the previous frame's BEV map brought
// into the current ego frame and stacked after the current transform's
// channels.
//
// The FlashBEV notes name a temporal fused view transform as future work
// ("Takeaway" item 4); the SparseDriveV2 notes ask that history be moved into
// the current ego frame (ego-motion compensation) before it is used, and the
// Lift-Splat-Shoot tutorial combines two BEV maps of one scene by stacking them
// in the same BEV space (the BEVFusion paragraph).  For current cell (i, j)
// with centre (x, y), the planar motion A maps it to (x', y') = A [x; y; 1] in
// the previous ego frame, at continuous index i' = (x' - x_min)/dx - 1/2,
// j' = (y' - y_min)/dy - 1/2 of the previous grid (same range and cells).
// Inside the closed box [0, X-1] x [0, Y-1] of cell centres the previous map
// is sampled bilinearly (the clamped tap at i' = X-1 has weight 0); outside,
// there is no history and the value is 0.
//
// bev_align_fwd: a thread per (cell, 8 channels): the source position in fp64
// once, then four taps per channel; workgroups are numbered so that each XCD
// takes a contiguous run of (cell block, channel chunk) units.
// bev_align_bwd: the adjoint as a gather, a thread per (previous cell q,
// 8 channels): the current cells whose sample can
// touch q lie in a small box around A^{-1}(q) (the inverse image of the open
// 2 x 2 square of q's taps); each is re-evaluated with the forward's own
// arithmetic and adds weight x upstream gradient when q is one of its taps.
// No atomics: the result is deterministic and every element is written once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bev_align.h"
#include "kernels.h"

namespace fbev {
namespace {

__global__ __launch_bounds__(kAlignBlock) void bev_align_fwd(AlignArgs a) { align_fwd_body(a, blockIdx.x, gridDim.x); }

__global__ __launch_bounds__(kAlignBlock) void bev_align_bwd(AlignArgs a) { align_bwd_body(a, blockIdx.x, gridDim.x); }

}  // namespace

hipError_t launch_align_forward(const Problem& p, const float* prev, int Cp, const float* ego, float* out, int c0,
                                hipStream_t stream) {
  if (p.B == 0 || Cp == 0 || p.X == 0 || p.Y == 0) return hipSuccess;
  AlignArgs a = align_args(p, Cp, ego, c0);
  a.src = prev;
  a.dst = out;
  const dim3 grid = align_grid(a);
  hipLaunchKernelGGL(bev_align_fwd, grid, dim3(kAlignBlock), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_align_backward(const Problem& p, const float* grad, int Cp, const float* ego, float* gprev, int c0,
                                 hipStream_t stream) {
  if (p.B == 0 || Cp == 0 || p.X == 0 || p.Y == 0) return hipSuccess;
  AlignArgs a = align_args(p, Cp, ego, c0);
  a.src = grad;
  a.dst = gprev;
  const dim3 grid = align_grid(a);
  hipLaunchKernelGGL(bev_align_bwd, grid, dim3(kAlignBlock), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fbev
