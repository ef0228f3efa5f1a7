// Internal interface between the C-ABI host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fbev {

constexpr int kMaxLevels = 4;

// Everything a launch needs, already validated by the host layer.
struct Problem {
  const void* feat;       // [B,N,P,C] channels-last (fp32 or bf16 bits); P pixels per camera
  const float* K;         // [B,N,3,3]
  const float* R;         // [B,N,3,3]
  const float* t;         // [B,N,3]
  int B, N, C, H, W;      // H, W: the level-0 map (the in-view test)
  int X, Y, Z;
  int out_ch;             // channels per batch sample of the output (forward) / upstream gradient (backward)
                          // tensor [B, out_ch, X, Y]; the transform's C channels come first
  double ox, dx, oy, dy, oz, dz;   // voxel centre i -> o + (i + 1/2) d
  int elem_bytes;         // 4 (fp32) or 2 (bf16)
  int vec_bytes;          // bytes one lane moves per tap: 16 or 4
  // feature levels: level l is lvl_H[l] x lvl_W[l] at pixel lvl_off[l] of a camera's
  // P = sum of H_l W_l pixels, level coordinate u_l = (u + 1/2) lvl_inv_r[l] - 1/2
  int L, P;
  int lvl_H[kMaxLevels], lvl_W[kMaxLevels], lvl_off[kMaxLevels];
  double lvl_inv_r[kMaxLevels];
};

hipError_t launch_forward(const Problem& p, float* out, uint8_t* counts, hipStream_t stream);
// The single-level forward over bin runs (sampling_vt_runs.hip): p.L == 1.
hipError_t launch_forward_runs(const Problem& p, float* out, uint8_t* counts, hipStream_t stream);
// The single-level backward over bin runs with a per-block counting sort (sampling_vt_runs.hip), onto a
// zero-filled dL/dF; for maps of at most 256 x 256 pixels.
bool backward_runs_supported(const Problem& p);
hipError_t launch_backward_runs(const Problem& p, const float* grad_out, float* grad_feat, hipStream_t stream);
hipError_t launch_backward(const Problem& p, const float* grad_out, float* grad_feat, hipStream_t stream);

// Camera gradients (single level, fp32 features): dL/dK, dL/dR [B,N,3,3] and
// dL/dt [B,N,3], fully overwritten; `work` holds camera_grad_workspace_bytes(p).
size_t camera_grad_workspace_bytes(const Problem& p);
hipError_t launch_camera_backward(const Problem& p, const float* grad_out, float* gK, float* gR, float* gt, void* work,
                                  hipStream_t stream);
// The allocation-free variant's device scratch: kCameraScratchBytes on every GPU, its device address for
// `device` looked up once (hipGetSymbolAddress with that device current) and kept for later calls.
constexpr size_t kCameraScratchBytes = (size_t)4 << 20;
hipError_t camera_scratch(int device, void** ptr);

// Temporal fusion: the previous BEV map prev [B, Cp, X, Y] resampled at the
// current cells mapped by the planar motion ego [B, 2, 3] (current ego x, y ->
// previous ego x, y) into channels [c0, c0 + Cp) of out [B, out_ch, X, Y]; and
// the adjoint, dL/dprev [B, Cp, X, Y] (fully overwritten) from channels
// [c0, c0 + Cp) of grad [B, out_ch, X, Y].  p supplies B, X, Y and the grid.
hipError_t launch_align_forward(const Problem& p, const float* prev, int Cp, const float* ego, float* out, int c0,
                                hipStream_t stream);
hipError_t launch_align_backward(const Problem& p, const float* grad, int Cp, const float* ego, float* gprev, int c0,
                                 hipStream_t stream);
// The temporal forward: the current frame's channels (when `current`: output channels or counts to
// write) and the aligned previous map after them, its resampling riding with the forward's last launch
// when the channel layout allows (a separate launch otherwise).
hipError_t launch_forward_temporal(const Problem& p, float* out, uint8_t* counts, bool current, int Cp,
                                   const float* prev, const float* ego, int c0, hipStream_t stream);
// The temporal backward: dL/dF of the current frame's channels and dL/dprev of the aligned previous
// map, in one launch after the zero-fill when both parts have work (separate launches otherwise).
hipError_t launch_backward_temporal(const Problem& p, const float* grad_out, float* grad_feat, int Cp, const float* ego,
                                    float* grad_prev, int c0, hipStream_t stream);

}  // namespace fbev
