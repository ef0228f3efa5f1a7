// Internal interface between the C-ABI host layer and the Deformable
// Aggregation kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace fbev {

// One problem, validated by the host layer.  Query q of sample b has anchor
// anchors[b,q,:], keypoint offsets offsets[b,q,k,:] and weights
// weights[b,q,n,k]; features are channels-last [B,N,H,W,C] fp32.
struct DeformArgs {
  const float* feat;
  const float* K;          // [B,N,3,3]
  const float* R;          // [B,N,3,3]
  const float* t;          // [B,N,3]
  const float* anchors;    // [B,Q,3]
  const float* offsets;    // [B,Q,Kp,3]
  const float* weights;    // [B,Q,N,Kp]
  const float* grad;       // backward: dL/dout [B,Q,C]
  float* out;              // forward: [B,Q,C]
  float* gfeat;            // backward: [B,N,H,W,C]
  float* gweights;         // backward: [B,Q,N,Kp]
  float* goffsets;         // backward: [B,Q,Kp,3]
  float* ganchors;         // backward: [B,Q,3] or NULL
  int B, N, C, H, W, Q, Kp;
  int q_stride;            // set by the backward's launcher
  int wq_n;                // waves per query in the backward (set by its launcher)
  // backward, dL/dF by gather (set by its launcher from the caller's workspace; entries NULL = none)
  int* pix_count;          // [B N H W] entries per pixel
  int* pix_first;          // [B N H W] first bucket slot of each pixel
  int* blk_sum;            // per scan block: sum of its counts
  int* q_count;            // [B Q] entries each query emitted
  int* entries;            // [B Q][cap] (pixel, rank within the pixel, merged weight bits)
  int2* bucket;            // entries by pixel: (b Q + q, weight bits)
  int cap;                 // entries per query at most (4 N Kp)
  int tab_max;             // hash-table slots per wave (set by the backward's launcher)
};

hipError_t launch_deform_forward(const DeformArgs& a, hipStream_t stream);
// Device workspace the backward needs for these sizes (0 when dL/dF has nothing to gather).
size_t deform_backward_workspace_bytes(const DeformArgs& a);
hipError_t launch_deform_backward(DeformArgs a, void* workspace, hipStream_t stream);

}  // namespace fbev
