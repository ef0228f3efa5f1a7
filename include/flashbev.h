/*
 * libflashbev -- exact dense Sampling-VT camera-to-BEV view transform, fused,
 * for AMD Instinct MI355X (gfx950).  Plain C ABI: no C++ types, no exceptions,
 * no framework types cross this boundary.
 *
 * The operation (FlashBEV reading notes, "Problem Setting", "Core Idea" and
 * "Method" items 1-4): for every batch sample b, BEV cell (x, y) and channel c,
 *
 *   out[b,c,x,y] = sum_z  mean_{n valid at (b,x,y,z)}  bilinear(F[b,n,:,:,c], u, v)
 *
 * where, for height bin z, the voxel centre p = (x_x, y_y, z_z) is projected
 * through camera n as [u, v, 1]^T ~ K_n (R_n p + t_n) (SparseDriveV2 notes,
 * "Deformable Aggregation", step 2) and camera n is valid when the depth
 * d = (K_n (R_n p + t_n))_3 > 0 and the point lands in the image.  A point
 * no camera sees contributes 0.  Nothing per (camera, height, channel) is
 * stored in device memory: projection, validity test, sampling, mean and
 * height sum happen in one kernel.
 *
 * Conventions (the pages leave these open; this library fixes them):
 *   - voxel centres of the half-open ranges: x_i = x_min + (i + 1/2)(x_max - x_min)/X,
 *     likewise y_j, z_k; out[b, c, i, j] has i along ego x, j along ego y;
 *   - (R, t) maps ego to camera coordinates, p_cam = R p + t;
 *   - integer (u, v) are pixel centres, u along W (columns), v along H (rows);
 *     "in the image" means 0 <= u <= W-1 and 0 <= v <= H-1 (closed), so every
 *     valid sample is a convex combination of existing pixels;
 *   - bilinear taps x0 = floor(u), x1 = min(x0 + 1, W - 1), likewise rows;
 *   - projection and the in-image test are evaluated in double precision;
 *     interpolation weights and accumulation are fp32.
 *
 * Memory: every pointer is caller-owned *device* memory unless stated.  The
 * library allocates no device memory and keeps no state beyond the calling
 * thread's last-error text.  All work is enqueued on `stream` (a hipStream_t;
 * NULL = the null stream) and calls return before it completes.
 *
 * Errors: arguments are validated on the host before anything is enqueued;
 * on a non-OK status nothing has been written.  FBEV_ERR_DEVICE reports a
 * launch error from the HIP runtime; fbev_last_error() gives the text.
 */
#ifndef FLASHBEV_H
#define FLASHBEV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FBEV_ABI_VERSION 8
#define FBEV_MAX_CAMERAS 64
#define FBEV_MAX_GRID 65536
#define FBEV_MAX_LEVELS 4
#define FBEV_MAX_KEYPOINTS 256

typedef enum {
  FBEV_OK = 0,
  FBEV_ERR_INVALID_ARGUMENT = 1, /* negative size, NULL pointer for a non-empty buffer, bad range, N > FBEV_MAX_CAMERAS,
                                    bad feature levels */
  FBEV_ERR_UNSUPPORTED = 2,      /* unknown dtype, odd C for bf16, misaligned features, per-sample features >= 2 GiB,
                                    cameras x levels > 64 */
  FBEV_ERR_DEVICE = 3            /* the HIP runtime reported an error when enqueueing */
} fbev_status;

typedef enum { FBEV_DTYPE_F32 = 0, FBEV_DTYPE_BF16 = 1 } fbev_dtype;

/* Feature maps are channels-last [B, N, H, W, C], contiguous. */
typedef struct {
  int32_t B, N, C, H, W;
} fbev_feat_desc;

/* BEV extent in metres, ego frame; each axis is the half-open [min, max). */
typedef struct {
  float x_min, x_max, y_min, y_max, z_min, z_max;
} fbev_range;

/*
 * Forward of the fused Sampling-VT (FlashBEV notes, "Method" items 1-2).
 *
 *   features : [B,N,H,W,C] of `dtype` (fp32, or bf16 bit patterns), device, read only.
 *              Must be 4-byte aligned; 16-byte alignment with C*elem_size a
 *              multiple of 16 takes the wide-load path.
 *   K        : [B,N,3,3] fp32 intrinsics (feature-map pixels), device.
 *   R, t     : [B,N,3,3] and [B,N,3] fp32 ego->camera extrinsics, device.
 *   bev_range, X, Y, Z : the voxel grid (X, Y, Z >= 0, each <= FBEV_MAX_GRID).
 *   out      : [B,C,X,Y] fp32, device; fully overwritten (zero where no camera
 *              sees any height bin, all zeros when Z == 0).
 *   counts   : [B,X,Y,Z] uint8 valid-camera counts, device, or NULL to skip.
 *
 * Sizes of zero are allowed and give the empty / all-zero result.  The result
 * is deterministic (fixed reduction order).
 */
fbev_status fbev_forward(const void* features, fbev_dtype dtype, fbev_feat_desc fd, const float* K,
                         const float* R, const float* t, fbev_range bev_range, int32_t X, int32_t Y,
                         int32_t Z, float* out, uint8_t* counts, void* stream);

/*
 * Gradient of fbev_forward with respect to the features (FlashBEV notes,
 * "Method" item 4: the fused operator keeps the forward/backward semantics
 * of the tensorized one).  The forward is linear in the features with the
 * validity mask, bilinear weights and camera counts fixed, so
 *
 *   dF[b,n,y,x,c] = sum over (cell, z) valid for n, and taps of that sample
 *                   landing on (y, x), of grad_out[b,c,cell] * w_tap / count.
 *
 *   grad_out      : [B,C,X,Y] fp32, device, read only.
 *   grad_features : [B,N,H,W,C] fp32, device; fully overwritten (zeroed on
 *                   `stream`, then accumulated with fp32 atomics, so the
 *                   bit pattern may vary from run to run within fp32
 *                   rounding).  Returned in fp32 also for bf16 forwards.
 * Other arguments as for fbev_forward; no feature values are needed.
 */
fbev_status fbev_backward(const float* grad_out, fbev_feat_desc fd, const float* K, const float* R,
                          const float* t, fbev_range bev_range, int32_t X, int32_t Y, int32_t Z,
                          float* grad_features, void* stream);

/*
 * Gradients of fbev_forward's output with respect to the cameras.  The
 * SparseDriveV2 notes ("Deformable Aggregation", pitfalls) ask for a
 * projection-and-sampling chain that gradients flow through; for
 * L = <grad_out, out> this returns dL/dK, dL/dR and dL/dt with the validity
 * mask and the camera counts held fixed (they are piecewise constant in the
 * cameras).  Per in-view sample of camera n at voxel centre p, with
 * h = K (R p + t), u = h_1 / h_3 and v = h_2 / h_3:
 *
 *   dL/du = <grad_out[b,:,cell], d sample / du> / count   (likewise v; inside
 *           the pixel square floor() picks, the sample is bilinear in u, v),
 *   dL/dP += [dL/du; dL/dv; -(u dL/du + v dL/dv)] [p; 1]^T / h_3,  P = K [R | t],
 *   dL/dK = dL/dP [R | t]^T,   [dL/dR | dL/dt] = K^T dL/dP.
 *
 * Every entry of K, R and t gets its partial derivative (R is not constrained
 * to a rotation).
 *
 *   grad_out   : [B,C,X,Y] fp32, device, read only.
 *   features   : [B,N,H,W,C] fp32, device, read only (4-byte aligned;
 *                16-byte alignment with C a multiple of 4 takes the wide path).
 *   grad_K, grad_R : [B,N,3,3] fp32, device; fully overwritten.
 *   grad_t     : [B,N,3] fp32, device; fully overwritten.
 *   workspace  : device scratch of at least the size that
 *                fbev_backward_cameras_workspace() reports for these sizes
 *                (may be NULL when that is 0); its contents are not needed
 *                before or after the call.  Calls that share a workspace must
 *                not overlap.
 * Other arguments as for fbev_forward; features are fp32 only.  A workspace
 * smaller than required gives FBEV_ERR_INVALID_ARGUMENT.  The result is deterministic: partial sums per workgroup are added in a
 * fixed order in fp64.  Zero sizes give zero (or empty) gradients.
 */
/*
 * Temporal fused view transform.  The FlashBEV notes name a temporal fused
 * transform as future work ("Takeaway" item 4); the SparseDriveV2 notes ask
 * that history be moved into the current ego frame before use (ego-motion
 * compensation), and the Lift-Splat-Shoot tutorial stacks two BEV maps of one
 * scene in the same BEV space (the BEVFusion paragraph).  This call writes
 *
 *   out[b, 0:C]      = fbev_forward(features, ...)[b]           (current frame)
 *   out[b, C:C+Cp]   = prev_bev[b] resampled at the current cells
 *
 * where current cell (i, j), centre (x, y), maps to (x', y') = A_b [x; y; 1]
 * in the previous ego frame, i.e. to the continuous cell index
 * i' = (x' - x_min)/dx - 1/2, j' = (y' - y_min)/dy - 1/2 of the previous map,
 * which lies on the same grid (bev_range, X, Y).  Inside the closed box
 * [0, X-1] x [0, Y-1] of cell centres the previous map is sampled bilinearly
 * (the clamped tap at i' = X-1 has weight 0); outside it the value is 0.
 *
 *   prev_bev : [B,Cp,X,Y] fp32, device, read only (NULL allowed when B*Cp*X*Y == 0).
 *   ego      : [B,2,3] fp32, device: A_b, current-ego (x, y) -> previous-ego
 *              (x, y) in metres (a rigid planar motion in practice).
 *   out      : [B,C+Cp,X,Y] fp32, device, fully overwritten.
 *   counts   : as for fbev_forward.
 * Other arguments as for fbev_forward.  Deterministic.  Cp < 0 or NULL
 * pointers for non-empty buffers -> FBEV_ERR_INVALID_ARGUMENT; X*Y >= 2^31 ->
 * FBEV_ERR_UNSUPPORTED.
 */
fbev_status fbev_forward_temporal(const void* features, fbev_dtype dtype, fbev_feat_desc fd, const float* K,
                                  const float* R, const float* t, fbev_range bev_range, int32_t X, int32_t Y,
                                  int32_t Z, const float* prev_bev, int32_t Cp, const float* ego, float* out,
                                  uint8_t* counts, void* stream);

/*
 * Gradients of fbev_forward_temporal: dL/dF from grad_out[:, 0:C] exactly as
 * fbev_backward, and dL/dprev_bev [B,Cp,X,Y] (fp32, device, fully overwritten,
 * deterministic) = the adjoint of the resampling: every current cell passes
 * grad_out[b, C + c, i, j] times its bilinear weights to its four taps.  The
 * adjoint is computed as a gather over the current cells whose sample can
 * reach a previous cell, within 16 cells per axis of the inverse-mapped cell.
 * A rigid motion stays inside that window whatever its turn when the cell
 * aspect ratio dx/dy lies in (1/15, 15); other grids give
 * FBEV_ERR_UNSUPPORTED when Cp > 0.  A non-rigid motion (ego is read on the
 * device, so the host cannot check it) whose inverse stretches the grid past
 * the window leaves those previous cells' gradient at 0.  No gradient with
 * respect to the ego motion.
 *   grad_out : [B,C+Cp,X,Y] fp32, device, read only.
 */
fbev_status fbev_backward_temporal(const float* grad_out, fbev_feat_desc fd, const float* K, const float* R,
                                   const float* t, fbev_range bev_range, int32_t X, int32_t Y, int32_t Z, int32_t Cp,
                                   const float* ego, float* grad_features, float* grad_prev, void* stream);

fbev_status fbev_backward_cameras_workspace(fbev_feat_desc fd, int32_t X, int32_t Y, int32_t Z, size_t* bytes);
fbev_status fbev_backward_cameras(const float* grad_out, const float* features, fbev_feat_desc fd, const float* K,
                                  const float* R, const float* t, fbev_range bev_range, int32_t X, int32_t Y,
                                  int32_t Z, float* grad_K, float* grad_R, float* grad_t, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * fbev_backward_cameras without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as
 * fbev_backward_cameras minus the workspace; this call allocates nothing.
 *
 * The partial sums live in a fixed device scratch of FBEV_NOALLOC_SCRATCH_BYTES
 * (4 MiB) that the library holds on every GPU it runs on until the process
 * ends; its address is looked up on the first call on each device.  Problems
 * that need more than that (what fbev_backward_cameras_workspace reports: at
 * most N * 172032 bytes for B <= 27, so up to 24 cameras always fit there)
 * return FBEV_ERR_UNSUPPORTED before anything is enqueued.  Every call on one GPU shares that GPU's scratch, and each
 * call overwrites all of it that it reads: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must be serialized
 * by the caller.  The scratch needs no clearing between calls.
 */
#define FBEV_NOALLOC_SCRATCH_BYTES (4 << 20)
fbev_status fbev_backward_cameras_noalloc(const float* grad_out, const float* features, fbev_feat_desc fd,
                                          const float* K, const float* R, const float* t, fbev_range bev_range,
                                          int32_t X, int32_t Y, int32_t Z, float* grad_K, float* grad_R,
                                          float* grad_t, void* stream);

/*
 * Multi-level (feature-pyramid) variants.  The pages name a multi-scale fused
 * view transform as the next step (FlashBEV notes, "Limitation" item 4 and
 * "Takeaway" item 4) and describe the FPN pyramid it would read
 * (SparseDriveV2 notes, "Multi-scale features": P2-P5 at growing strides);
 * they do not define the fused operator, so this library fixes it as the
 * single-level operator with each camera's sample replaced by the mean of its
 * L level samples:
 *   - level l is (H / r_l) x (W / r_l) with integer ratios r_l, r_0 = 1; K maps
 *     to level-0 pixels; validity and the camera count are decided at level 0
 *     exactly as in fbev_forward;
 *   - level l is sampled at u_l = (u + 1/2) / r_l - 1/2 (v likewise): a level
 *     pixel centre sits at the centre of the r_l x r_l level-0 block it covers;
 *     u_l, v_l are clamped to the level's pixel-centre box (border replication);
 *   - camera sample = (1/L) sum_l bilinear_l; then the valid-camera mean and
 *     the height sum as in fbev_forward.  L = 1 is fbev_forward.
 *
 *   features : [B, N, P, C] with P = sum_l (H/r_l)(W/r_l): per camera, level 0's
 *              pixels row-major, then level 1's, ... (dtype and alignment as for
 *              fbev_forward).  fd.H, fd.W describe level 0.
 *   L        : 1..FBEV_MAX_LEVELS levels, with N * L <= 64.
 *   ratios   : host array of L ratios (ratios[0] = 1, each divides H and W), read
 *              during the call only; may be NULL when L = 1.
 * Other arguments, outputs and errors as for fbev_forward.
 */
fbev_status fbev_forward_levels(const void* features, fbev_dtype dtype, fbev_feat_desc fd, int32_t L,
                                const int32_t* ratios, const float* K, const float* R, const float* t,
                                fbev_range bev_range, int32_t X, int32_t Y, int32_t Z, float* out, uint8_t* counts,
                                void* stream);

/*
 * Gradient of fbev_forward_levels with respect to the packed level features:
 * grad_features is [B, N, P, C] fp32 in the same packing, fully overwritten
 * (zeroed on `stream`, then accumulated with fp32 atomics).  The adjoint of the
 * level mean scales each level's taps by 1/L.  Other arguments as for
 * fbev_forward_levels and fbev_backward.
 */
fbev_status fbev_backward_levels(const float* grad_out, fbev_feat_desc fd, int32_t L, const int32_t* ratios,
                                 const float* K, const float* R, const float* t, fbev_range bev_range, int32_t X,
                                 int32_t Y, int32_t Z, float* grad_features, void* stream);

/*
 * Lift-Splat, the push view transform (Lift-Splat-Shoot tutorial, sections
 * "Lift" and "Splat").  Every feature-map pixel (n, v, u) carries a depth
 * distribution alpha over D bins and a context vector c of C channels; bin k
 * puts the point alpha_k * c on the pixel's ray at camera depth
 * d_k = d_min + k * d_step (the tutorial's nuScenes setting: [4, 45) at 1 m,
 * 41 bins at 4, 5, ..., 44).  The point moves to the ego frame,
 *   p = R_n^T (d_k K_n^-1 [u, v, 1]^T - t_n)     ((R, t) maps ego to camera),
 * and lands in BEV cell (i, j) = (floor((p_x - x_min) / dx), floor((p_y - y_min) / dy)),
 * dx = (x_max - x_min) / X, dy = (y_max - y_min) / Y, when 0 <= i < X and
 * 0 <= j < Y; there is no bound on p_z (each cell is a pillar) and
 * bev_range.z_min / z_max are not used.  Each cell sums its points:
 *
 *   out[b, c, i, j] = sum over (n, k, v, u) whose point lands in (i, j) of alpha[b,n,v,u,k] * ctx[b,n,v,u,c]
 *
 * The geometry and the cell index are evaluated in double precision; the
 * products and sums are fp32.  A point within rounding of a cell edge lands in
 * one of the two cells, never in both or neither.  No point, cell index or
 * sorted order is stored in device memory.
 *
 *   depth    : alpha, [B, N, H, W, D] fp32, device, read only (any values; a
 *              softmax output in the tutorial's network).
 *   context  : c, [B, N, H, W, C] fp32 (channels-last), device, read only.
 *   fd       : B, N, C (context channels), H, W of the feature map.
 *   D, d_min, d_step : the depth bins, 0 <= D <= FBEV_MAX_GRID, d_step > 0.
 *   K, R, t  : as for fbev_forward (K in feature-map pixels).
 *   out      : [B, C, X, Y] fp32, device, fully overwritten (zero where no
 *              point lands).  Deterministic.
 * Errors as for fbev_forward; FBEV_ERR_UNSUPPORTED when one sample's depth or
 * context has 2^31 elements or more.
 */
fbev_status fbev_lss_forward(const float* depth, const float* context, fbev_feat_desc fd, int32_t D, float d_min,
                             float d_step, const float* K, const float* R, const float* t, fbev_range bev_range,
                             int32_t X, int32_t Y, float* out, void* stream);

/*
 * Gradients of fbev_lss_forward.  With the geometry fixed the forward is
 * bilinear in (alpha, c) (tutorial, "Lift": the point features are the outer
 * product of the two), so for the point of bin k of pixel q landing in cell s:
 *
 *   grad_depth[b, q, k]   = <ctx[b, q, :], grad_out[b, :, s]>     (0 for points outside the grid)
 *   grad_context[b, q, c] = sum over q's landing points of alpha[b, q, k] * grad_out[b, c, s]
 *
 *   grad_out     : [B, C, X, Y] fp32, device, read only.
 *   depth, context : the forward's inputs (read only).
 *   grad_depth   : [B, N, H, W, D] fp32, device, fully overwritten.
 *   grad_context : [B, N, H, W, C] fp32, device, fully overwritten.
 * Both outputs are zeroed on `stream` and then accumulated with fp32 atomics:
 * grad_depth is deterministic for C <= 64 (one add per element), grad_context
 * sums one add per (pixel, 4 x 8 cell tile) in run-dependent order.  Pointers
 * whose buffer has no elements may be NULL.  Other arguments and errors as
 * for fbev_lss_forward.
 */
fbev_status fbev_lss_backward(const float* grad_out, const float* depth, const float* context, fbev_feat_desc fd,
                              int32_t D, float d_min, float d_step, const float* K, const float* R, const float* t,
                              fbev_range bev_range, int32_t X, int32_t Y, float* grad_depth, float* grad_context,
                              void* stream);

/*
 * Deformable Aggregation: multi-camera deformable sampling (SparseDriveV2
 * notes, "Deformable Aggregation", steps 1-3), the operator the FlashBEV
 * notes fuse for BEVFormer's spatial cross-attention.  For query q of batch
 * sample b with anchor a_q and keypoint offsets o_{q,k} (k < Kp):
 *
 *   p_{q,k} = a_q + o_{q,k}                                   (ego frame, metres)
 *   out[b, q, c] = sum_n sum_k  weights[b,q,n,k] * bilinear(F[b,n,:,:,c], u, v)   over (n, k) in view
 *
 * with [u, v, 1]^T ~ K_n (R_n p + t_n) and the in-view rule, pixel-centre
 * convention and bilinear taps of fbev_forward (depth > 0, closed box
 * [0, W-1] x [0, H-1]).  The weights are used as given (no renormalisation
 * over the pairs in view).  Projection and the in-view test in double
 * precision, interpolation and sums in fp32.
 *
 *   features : [B, N, H, W, C] fp32 channels-last, device, read only.
 *   K, R, t  : as for fbev_forward.
 *   anchors  : [B, Q, 3] fp32; offsets : [B, Q, Kp, 3] fp32; weights : [B, Q, N, Kp] fp32; device.
 *   Q, Kp    : queries per sample and keypoints per query (Kp <= FBEV_MAX_KEYPOINTS).
 *   out      : [B, Q, C] fp32, device, fully overwritten.  Deterministic.
 * Errors as for fbev_forward.
 */
fbev_status fbev_deform_forward(const float* features, fbev_feat_desc fd, const float* K, const float* R,
                                const float* t, const float* anchors, const float* offsets, const float* weights,
                                int32_t Q, int32_t Kp, float* out, void* stream);

/*
 * Gradients of fbev_deform_forward with the in-view mask held fixed (the page
 * asks for a sampling chain that gradients pass through):
 *   grad_features : [B,N,H,W,C] fp32 — each in-view sample adds w * tap weight * g
 *                   to its four taps.  Computed as a gather: a query's taps on one
 *                   pixel are merged, each (query, pixel) pair becomes an entry in the
 *                   pixel's bucket, and every element is the sum over its bucket
 *                   (written once; the order within a bucket varies run to run, so
 *                   the last bits may too).
 *   grad_weights  : [B,Q,N,Kp] fp32 — <sample, g> for pairs in view, 0 otherwise.
 *   grad_offsets  : [B,Q,Kp,3] fp32 — sum over cameras of w (<ds/du, g> du/dp + <ds/dv, g> dv/dp),
 *                   the bilinear sample's derivative inside its pixel square times the
 *                   projection's Jacobian du/dp = (P_1 - u P_3) / h_3 (P = K [R | t]).
 *   grad_anchors  : [B,Q,3] fp32 — the sum of grad_offsets over k; may be NULL.
 *   workspace     : device scratch of at least the size that
 *                   fbev_deform_backward_workspace() reports for these sizes (may be
 *                   NULL when that is 0), 16-byte aligned; its contents are not needed
 *                   before or after the call.  Calls that share a workspace must not
 *                   overlap.  It holds per-pixel counts and offsets and up to
 *                   4 N Kp entries of 20 bytes per query.
 * All outputs are fully overwritten; grad_out is [B,Q,C]; other arguments as
 * for fbev_deform_forward.  A workspace smaller than required gives
 * FBEV_ERR_INVALID_ARGUMENT; B N H W or B Q 4 N Kp of 2^31 or more gives
 * FBEV_ERR_UNSUPPORTED.
 */
fbev_status fbev_deform_backward_workspace(fbev_feat_desc fd, int32_t Q, int32_t Kp, size_t* bytes);
fbev_status fbev_deform_backward(const float* grad_out, const float* features, fbev_feat_desc fd, const float* K,
                                 const float* R, const float* t, const float* anchors, const float* offsets,
                                 const float* weights, int32_t Q, int32_t Kp, float* grad_features,
                                 float* grad_weights, float* grad_offsets, float* grad_anchors, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* fbev_status_string(fbev_status s);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* fbev_last_error(void);

/* FBEV_ABI_VERSION of the built library. */
int32_t fbev_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHBEV_H */
