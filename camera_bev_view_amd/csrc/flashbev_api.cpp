// C-ABI host layer of libflashbev: argument validation, launch-shape choice
// and error reporting.  Every check runs on the host before anything is
// enqueued, so a non-OK status means nothing was written.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <string>

#include "../../include/flashbev.h"
#include "kernels.h"
#include "lift_splat.h"
#include "deform_agg.h"

static_assert(fbev::kCameraScratchBytes == FBEV_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

namespace {

thread_local std::string g_last_error;

fbev_status fail(fbev_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

fbev_status fail(fbev_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool finite_range(float lo, float hi) { return std::isfinite(lo) && std::isfinite(hi) && hi > lo; }

// Validation of the sizes of a Sampling-VT problem (features and grid).
fbev_status check_sizes(const fbev_feat_desc& fd, int32_t X, int32_t Y, int32_t Z) {
  if (fd.B < 0 || fd.N < 0 || fd.C < 0 || fd.H < 0 || fd.W < 0)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "negative feature size (B=%d N=%d C=%d H=%d W=%d)", fd.B, fd.N, fd.C,
                fd.H, fd.W);
  if (X < 0 || Y < 0 || Z < 0) return fail(FBEV_ERR_INVALID_ARGUMENT, "negative grid size (X=%d Y=%d Z=%d)", X, Y, Z);
  if (X > FBEV_MAX_GRID || Y > FBEV_MAX_GRID || Z > FBEV_MAX_GRID)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "grid size above %d (X=%d Y=%d Z=%d)", FBEV_MAX_GRID, X, Y, Z);
  if (fd.N > FBEV_MAX_CAMERAS)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "N=%d cameras exceeds FBEV_MAX_CAMERAS=%d", fd.N, FBEV_MAX_CAMERAS);
  if (fd.H > FBEV_MAX_GRID || fd.W > FBEV_MAX_GRID)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "feature map %dx%d above %d", fd.H, fd.W, FBEV_MAX_GRID);
  return FBEV_OK;
}

// Shared validation of the geometry arguments; fills `p` on success.
fbev_status check_common(const fbev_feat_desc& fd, const float* K, const float* R, const float* t,
                         const fbev_range& r, int32_t X, int32_t Y, int32_t Z, fbev::Problem& p) {
  const fbev_status st = check_sizes(fd, X, Y, Z);
  if (st != FBEV_OK) return st;
  if (!finite_range(r.x_min, r.x_max) || !finite_range(r.y_min, r.y_max) || !finite_range(r.z_min, r.z_max))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "each BEV range axis needs finite min < max");
  if ((int64_t)fd.B * fd.N > 0 && (K == nullptr || R == nullptr || t == nullptr))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "K, R and t must be non-NULL when B*N > 0");
  p.K = K;
  p.R = R;
  p.t = t;
  p.B = fd.B;
  p.N = fd.N;
  p.C = fd.C;
  p.H = fd.H;
  p.W = fd.W;
  p.X = X;
  p.Y = Y;
  p.Z = Z;
  // voxel centre of index i: min + (i + 1/2) (max - min) / n, evaluated in double
  p.ox = (double)r.x_min;
  p.dx = ((double)r.x_max - (double)r.x_min) / (X > 0 ? X : 1);
  p.oy = (double)r.y_min;
  p.dy = ((double)r.y_max - (double)r.y_min) / (Y > 0 ? Y : 1);
  p.oz = (double)r.z_min;
  p.dz = ((double)r.z_max - (double)r.z_min) / (Z > 0 ? Z : 1);
  p.out_ch = fd.C;
  return FBEV_OK;
}

// Feature levels: level l is (H / r_l) x (W / r_l), packed after the earlier
// levels in each camera's pixel axis.  Fills the level fields of `p`.
fbev_status check_levels(const fbev_feat_desc& fd, int32_t L, const int32_t* ratios, fbev::Problem& p) {
  if (L < 1 || L > FBEV_MAX_LEVELS)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "L=%d feature levels outside [1, %d]", L, FBEV_MAX_LEVELS);
  if (L > 1 && ratios == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "ratios is NULL with L=%d levels", L);
  if ((int64_t)fd.N * L > 64)
    return fail(FBEV_ERR_UNSUPPORTED, "N*L = %d*%d cameras x levels exceeds 64", fd.N, L);
  int64_t P = 0;
  for (int l = 0; l < L; ++l) {
    const int r = (L == 1 && ratios == nullptr) ? 1 : ratios[l];
    if (l == 0 && r != 1) return fail(FBEV_ERR_INVALID_ARGUMENT, "ratios[0] must be 1 (got %d)", r);
    if (r < 1 || (fd.H > 0 && fd.H % r != 0) || (fd.W > 0 && fd.W % r != 0))
      return fail(FBEV_ERR_INVALID_ARGUMENT, "level %d ratio %d does not divide the %dx%d level-0 map", l, r, fd.H,
                  fd.W);
    p.lvl_H[l] = fd.H / r;
    p.lvl_W[l] = fd.W / r;
    p.lvl_off[l] = (int)P;
    p.lvl_inv_r[l] = 1.0 / (double)r;
    P += (int64_t)p.lvl_H[l] * p.lvl_W[l];
  }
  for (int l = L; l < fbev::kMaxLevels; ++l) {
    p.lvl_H[l] = p.lvl_H[0];
    p.lvl_W[l] = p.lvl_W[0];
    p.lvl_off[l] = 0;
    p.lvl_inv_r[l] = 1.0;
  }
  p.L = L;
  p.P = (int)P;
  return FBEV_OK;
}

fbev_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FBEV_OK;
  return fail(FBEV_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Temporal fusion arguments: Cp channels of the previous BEV map and the planar
// ego motion [B, 2, 3]; both pointers may be NULL when nothing would read them.
fbev_status check_temporal(const fbev_feat_desc& fd, int32_t X, int32_t Y, int32_t Cp, const void* prev,
                           const float* ego, const char* prev_name) {
  if (Cp < 0) return fail(FBEV_ERR_INVALID_ARGUMENT, "negative Cp=%d previous-map channels", Cp);
  const int64_t n_prev = (int64_t)fd.B * Cp * X * Y;
  if (n_prev > 0 && prev == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "%s is NULL", prev_name);
  if (n_prev > 0 && ego == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "ego is NULL");
  if ((int64_t)X * Y >= (int64_t)1 << 31)
    return fail(FBEV_ERR_UNSUPPORTED, "X*Y = %lld cells (limit 2^31 - 1)", (long long)X * Y);
  if ((int64_t)fd.C + Cp > INT32_MAX) return fail(FBEV_ERR_UNSUPPORTED, "C + Cp channels above 2^31 - 1");
  return FBEV_OK;
}

fbev_status forward_impl(const void* features, fbev_dtype dtype, fbev_feat_desc fd, int32_t L, const int32_t* ratios,
                         const float* K, const float* R, const float* t, fbev_range bev_range, int32_t X, int32_t Y,
                         int32_t Z, float* out, uint8_t* counts, void* stream, const float* prev = nullptr,
                         int32_t Cp = 0, const float* ego = nullptr) {
  fbev::Problem p{};
  fbev_status s = check_common(fd, K, R, t, bev_range, X, Y, Z, p);
  if (s != FBEV_OK) return s;
  s = check_levels(fd, L, ratios, p);
  if (s != FBEV_OK) return s;
  s = check_temporal(fd, X, Y, Cp, prev, ego, "prev_bev");
  if (s != FBEV_OK) return s;
  p.out_ch = fd.C + Cp;
  if (dtype != FBEV_DTYPE_F32 && dtype != FBEV_DTYPE_BF16)
    return fail(FBEV_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  const int es = (dtype == FBEV_DTYPE_F32) ? 4 : 2;
  const int64_t n_feat = (int64_t)fd.B * fd.N * p.P * fd.C;
  const int64_t n_out = (int64_t)fd.B * fd.C * X * Y;
  const int64_t n_prev = (int64_t)fd.B * Cp * X * Y;
  const int64_t n_cnt = (int64_t)fd.B * X * Y * Z;
  if (n_feat > 0 && features == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "features is NULL");
  if ((n_out > 0 || n_prev > 0) && out == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "out is NULL");
  if ((fd.C * es) % 4 != 0) return fail(FBEV_ERR_UNSUPPORTED, "bf16 features need an even C (got %d)", fd.C);
  const int64_t batch_bytes = (int64_t)fd.N * p.P * fd.C * es;
  if (batch_bytes >= (int64_t)1 << 31)
    return fail(FBEV_ERR_UNSUPPORTED, "one sample's features span %lld bytes (limit 2^31 - 1)",
                (long long)batch_bytes);
  const uintptr_t addr = reinterpret_cast<uintptr_t>(features);
  if (n_feat > 0 && (addr & 3) != 0) return fail(FBEV_ERR_UNSUPPORTED, "features must be 4-byte aligned");
  p.feat = features;
  p.elem_bytes = es;
  p.vec_bytes = ((fd.C * es) % 16 == 0 && (addr & 15) == 0) ? 16 : 4;
  const bool current = n_out > 0 || (counts != nullptr && n_cnt > 0);
  if (n_prev == 0) {
    if (!current) return FBEV_OK;
    return device_status(fbev::launch_forward(p, n_out > 0 ? out : nullptr, n_cnt > 0 ? counts : nullptr,
                                              static_cast<hipStream_t>(stream)),
                         "fbev_forward launch");
  }
  return device_status(fbev::launch_forward_temporal(p, out, n_cnt > 0 ? counts : nullptr, current, Cp, prev, ego,
                                                     fd.C, static_cast<hipStream_t>(stream)),
                       "fbev_forward_temporal launch");
}

fbev_status backward_impl(const float* grad_out, fbev_feat_desc fd, int32_t L, const int32_t* ratios, const float* K,
                          const float* R, const float* t, fbev_range bev_range, int32_t X, int32_t Y, int32_t Z,
                          float* grad_features, void* stream, int32_t Cp = 0, const float* ego = nullptr,
                          float* grad_prev = nullptr) {
  fbev::Problem p{};
  fbev_status s = check_common(fd, K, R, t, bev_range, X, Y, Z, p);
  if (s != FBEV_OK) return s;
  s = check_levels(fd, L, ratios, p);
  if (s != FBEV_OK) return s;
  s = check_temporal(fd, X, Y, Cp, grad_prev, ego, "grad_prev");
  if (s != FBEV_OK) return s;
  p.out_ch = fd.C + Cp;
  const int64_t n_feat = (int64_t)fd.B * fd.N * p.P * fd.C;
  const int64_t n_out = (int64_t)fd.B * fd.C * X * Y;
  const int64_t n_prev = (int64_t)fd.B * Cp * X * Y;
  if (n_feat > 0 && grad_features == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_features is NULL");
  if (((n_out > 0 && n_feat > 0) || n_prev > 0) && grad_out == nullptr)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  const int64_t batch_elems = (int64_t)fd.N * p.P * fd.C;
  if (batch_elems >= (int64_t)1 << 31)
    return fail(FBEV_ERR_UNSUPPORTED, "one sample's gradient spans %lld elements (limit 2^31 - 1)",
                (long long)batch_elems);
  // The resampling adjoint gathers, for each previous cell, the current cells within a window of
  // half-width |cos| + |sin| * (cell aspect) around the inverse-mapped centre (index units); a rigid
  // motion fits the window for every turn only when the cells' aspect ratio stays below 15.
  if (n_prev > 0 && (p.dx / p.dy >= 15.0 || p.dy / p.dx >= 15.0))
    return fail(FBEV_ERR_UNSUPPORTED, "cell aspect ratio dx/dy = %g: the previous-map gradient needs it in (1/15, 15)",
                p.dx / p.dy);
  p.feat = nullptr;
  p.elem_bytes = 4;
  p.vec_bytes = 4;
  if (n_prev == 0) {
    if (n_feat == 0) return FBEV_OK;
    return device_status(fbev::launch_backward(p, grad_out, grad_features, static_cast<hipStream_t>(stream)),
                         "fbev_backward launch");
  }
  return device_status(fbev::launch_backward_temporal(p, grad_out, n_feat > 0 ? grad_features : nullptr, Cp, ego,
                                                      grad_prev, fd.C, static_cast<hipStream_t>(stream)),
                       "fbev_backward_temporal launch");
}

// Camera gradients: the sizes of a single-level problem with fp32 features;
// fills the size fields of `p` (all the workspace size depends on).
fbev_status check_cameras(const fbev_feat_desc& fd, int32_t X, int32_t Y, int32_t Z, fbev::Problem& p) {
  fbev_status s = check_sizes(fd, X, Y, Z);
  if (s != FBEV_OK) return s;
  s = check_levels(fd, 1, nullptr, p);
  if (s != FBEV_OK) return s;
  p.B = fd.B;
  p.N = fd.N;
  p.C = fd.C;
  p.H = fd.H;
  p.W = fd.W;
  p.X = X;
  p.Y = Y;
  p.Z = Z;
  const int64_t batch_elems = (int64_t)fd.N * fd.H * fd.W * fd.C;
  if (batch_elems >= (int64_t)1 << 31)
    return fail(FBEV_ERR_UNSUPPORTED, "one sample's features span %lld elements (limit 2^31 - 1)",
                (long long)batch_elems);
  const int64_t units = (int64_t)X * ((Y + 31) / 32) * ((fd.C + 63) / 64);
  if (units >= (int64_t)1 << 31)
    return fail(FBEV_ERR_UNSUPPORTED, "%lld work units (x-rows x 32-cell tiles x 64-channel groups), limit 2^31 - 1",
                (long long)units);
  p.elem_bytes = 4;
  p.vec_bytes = 4;
  return FBEV_OK;
}

fbev_status cameras_workspace_impl(fbev_feat_desc fd, int32_t X, int32_t Y, int32_t Z, size_t* bytes) {
  if (bytes == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "bytes is NULL");
  fbev::Problem p{};
  const fbev_status s = check_cameras(fd, X, Y, Z, p);
  if (s != FBEV_OK) return s;
  *bytes = fbev::camera_grad_workspace_bytes(p);
  return FBEV_OK;
}

fbev_status backward_cameras_impl(const float* grad_out, const float* features, fbev_feat_desc fd, const float* K,
                                  const float* R, const float* t, fbev_range bev_range, int32_t X, int32_t Y,
                                  int32_t Z, float* grad_K, float* grad_R, float* grad_t, void* workspace,
                                  size_t workspace_bytes, void* stream, bool use_scratch = false) {
  fbev::Problem p{};
  fbev_status s = check_cameras(fd, X, Y, Z, p);
  if (s != FBEV_OK) return s;
  s = check_common(fd, K, R, t, bev_range, X, Y, Z, p);
  if (s != FBEV_OK) return s;
  const int64_t n_cam = (int64_t)fd.B * fd.N;
  if (n_cam == 0) return FBEV_OK;
  if (grad_K == nullptr || grad_R == nullptr || grad_t == nullptr)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_K, grad_R and grad_t must be non-NULL when B*N > 0");
  const int64_t n_feat = (int64_t)fd.B * fd.N * fd.H * fd.W * fd.C;
  const int64_t n_out = (int64_t)fd.B * fd.C * X * Y;
  if (n_feat > 0 && features == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "features is NULL");
  if (n_out > 0 && grad_out == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  const uintptr_t addr = reinterpret_cast<uintptr_t>(features);
  if (n_feat > 0 && (addr & 3) != 0) return fail(FBEV_ERR_UNSUPPORTED, "features must be 4-byte aligned");
  const size_t need = fbev::camera_grad_workspace_bytes(p);
  if (use_scratch) {
    if (need > fbev::kCameraScratchBytes)
      return fail(FBEV_ERR_UNSUPPORTED, "needs %zu bytes of scratch, the allocation-free variant holds %zu", need,
                  fbev::kCameraScratchBytes);
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      // the device the work is enqueued on: the stream's (the current device for the null stream)
      int dev = -1;
      hipError_t e = (stream != nullptr) ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                         : hipGetDevice(&dev);
      if (e == hipSuccess) e = fbev::camera_scratch(dev, &workspace);
      if (e != hipSuccess) return device_status(e, "fbev_backward_cameras_noalloc scratch lookup");
      workspace_bytes = fbev::kCameraScratchBytes;
    }
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 7) != 0)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "workspace must be 8-byte aligned");
  p.feat = features;
  return device_status(fbev::launch_camera_backward(p, grad_out, grad_K, grad_R, grad_t, workspace,
                                                    static_cast<hipStream_t>(stream)),
                       "fbev_backward_cameras launch");
}


// Lift-Splat arguments: depth [B,N,H,W,D] and context [B,N,H,W,C], the depth
// bins, the rig and the x-y extent of the BEV grid (its z fields are unused:
// a cell is a pillar).  Fills the geometry and size fields of `a`.
fbev_status check_lss(const fbev_feat_desc& fd, int32_t D, float d_min, float d_step, const float* K, const float* R,
                      const float* t, const fbev_range& r, int32_t X, int32_t Y, fbev::LssArgs& a) {
  if (fd.B < 0 || fd.N < 0 || fd.C < 0 || fd.H < 0 || fd.W < 0 || D < 0)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "negative size (B=%d N=%d C=%d H=%d W=%d D=%d)", fd.B, fd.N, fd.C, fd.H,
                fd.W, D);
  if (X < 0 || Y < 0) return fail(FBEV_ERR_INVALID_ARGUMENT, "negative grid size (X=%d Y=%d)", X, Y);
  if (X > FBEV_MAX_GRID || Y > FBEV_MAX_GRID || D > FBEV_MAX_GRID)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "size above %d (X=%d Y=%d D=%d)", FBEV_MAX_GRID, X, Y, D);
  if (fd.N > FBEV_MAX_CAMERAS)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "N=%d cameras exceeds FBEV_MAX_CAMERAS=%d", fd.N, FBEV_MAX_CAMERAS);
  if (fd.H > FBEV_MAX_GRID || fd.W > FBEV_MAX_GRID)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "feature map %dx%d above %d", fd.H, fd.W, FBEV_MAX_GRID);
  if (!finite_range(r.x_min, r.x_max) || !finite_range(r.y_min, r.y_max))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "the x and y BEV ranges need finite min < max");
  if (!std::isfinite(d_min) || !std::isfinite(d_step) || !(d_step > 0.0f))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "depth bins need a finite d_min and a finite d_step > 0");
  if ((int64_t)fd.B * fd.N > 0 && (K == nullptr || R == nullptr || t == nullptr))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "K, R and t must be non-NULL when B*N > 0");
  // the kernels find candidate bins in fp32: bin indices must stay far inside its precision
  const double span = (std::fabs((double)d_min) + std::fabs((double)d_min + (double)D * d_step)) / d_step;
  if (span >= (double)(1 << 20))
    return fail(FBEV_ERR_UNSUPPORTED, "depth bins of %g m at up to %g m: more than 2^20 steps from depth 0",
                (double)d_step, std::fabs((double)d_min) + (double)D * d_step);
  const int64_t pix = (int64_t)fd.N * fd.H * fd.W;
  const int64_t widest = fd.C > D ? fd.C : D;
  if (pix * widest >= (int64_t)1 << 31 || pix * 4 >= (int64_t)1 << 31)
    return fail(FBEV_ERR_UNSUPPORTED, "one sample's depth or context spans %lld elements (limit 2^31 - 1)",
                (long long)(pix * widest));
  a.K = K;
  a.R = R;
  a.t = t;
  a.B = fd.B;
  a.N = fd.N;
  a.H = fd.H;
  a.W = fd.W;
  a.C = fd.C;
  a.D = D;
  a.X = X;
  a.Y = Y;
  a.dmin = (double)d_min;
  a.dstep = (double)d_step;
  a.x_min = (double)r.x_min;
  a.y_min = (double)r.y_min;
  a.cdx = ((double)r.x_max - (double)r.x_min) / (X > 0 ? X : 1);
  a.cdy = ((double)r.y_max - (double)r.y_min) / (Y > 0 ? Y : 1);
  return FBEV_OK;
}

fbev_status lss_forward_impl(const float* depth, const float* context, fbev_feat_desc fd, int32_t D, float d_min,
                             float d_step, const float* K, const float* R, const float* t, fbev_range bev_range,
                             int32_t X, int32_t Y, float* out, void* stream) {
  fbev::LssArgs a{};
  fbev_status s = check_lss(fd, D, d_min, d_step, K, R, t, bev_range, X, Y, a);
  if (s != FBEV_OK) return s;
  const int64_t n_pix = (int64_t)fd.B * fd.N * fd.H * fd.W;
  const int64_t n_out = (int64_t)fd.B * fd.C * X * Y;
  if (n_out == 0) return FBEV_OK;
  if (out == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "out is NULL");
  if (n_pix * D > 0 && depth == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "depth is NULL");
  if (n_pix * fd.C > 0 && context == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "context is NULL");
  a.depth = depth;
  a.ctx = context;
  a.out = out;
  return device_status(fbev::launch_lss_forward(a, static_cast<hipStream_t>(stream)), "fbev_lss_forward launch");
}

fbev_status lss_backward_impl(const float* grad_out, const float* depth, const float* context, fbev_feat_desc fd,
                              int32_t D, float d_min, float d_step, const float* K, const float* R, const float* t,
                              fbev_range bev_range, int32_t X, int32_t Y, float* grad_depth, float* grad_context,
                              void* stream) {
  fbev::LssArgs a{};
  fbev_status s = check_lss(fd, D, d_min, d_step, K, R, t, bev_range, X, Y, a);
  if (s != FBEV_OK) return s;
  const int64_t n_pix = (int64_t)fd.B * fd.N * fd.H * fd.W;
  const int64_t n_out = (int64_t)fd.B * fd.C * X * Y;
  const bool want_d = n_pix * D > 0, want_c = n_pix * fd.C > 0;
  if (!want_d && !want_c) return FBEV_OK;
  if (want_d && grad_depth == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_depth is NULL");
  if (want_c && grad_context == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_context is NULL");
  // the gradient of one input needs the other one (the forward is bilinear in them)
  if (n_out > 0 && want_d && want_c && (depth == nullptr || context == nullptr))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "depth and context must be non-NULL");
  if (n_out > 0 && want_d && want_c && grad_out == nullptr)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  a.grad = grad_out;
  a.depth = depth;
  a.ctx = context;
  a.gdep = want_d ? grad_depth : nullptr;
  a.gctx = want_c ? grad_context : nullptr;
  return device_status(fbev::launch_lss_backward(a, static_cast<hipStream_t>(stream)), "fbev_lss_backward launch");
}


// Deformable Aggregation arguments: features [B,N,H,W,C] fp32, Q queries with
// anchors [B,Q,3], Kp keypoint offsets [B,Q,Kp,3] and weights [B,Q,N,Kp].
fbev_status check_deform(const fbev_feat_desc& fd, int32_t Q, int32_t Kp, const float* K, const float* R,
                         const float* t, fbev::DeformArgs& a, bool cams = true) {
  if (fd.B < 0 || fd.N < 0 || fd.C < 0 || fd.H < 0 || fd.W < 0 || Q < 0 || Kp < 0)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "negative size (B=%d N=%d C=%d H=%d W=%d Q=%d Kp=%d)", fd.B, fd.N, fd.C,
                fd.H, fd.W, Q, Kp);
  if (fd.N > FBEV_MAX_CAMERAS)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "N=%d cameras exceeds FBEV_MAX_CAMERAS=%d", fd.N, FBEV_MAX_CAMERAS);
  if (fd.H > FBEV_MAX_GRID || fd.W > FBEV_MAX_GRID)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "feature map %dx%d above %d", fd.H, fd.W, FBEV_MAX_GRID);
  if (Kp > FBEV_MAX_KEYPOINTS)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "Kp=%d keypoints exceeds FBEV_MAX_KEYPOINTS=%d", Kp, FBEV_MAX_KEYPOINTS);
  if (cams && (int64_t)fd.B * fd.N > 0 && (K == nullptr || R == nullptr || t == nullptr))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "K, R and t must be non-NULL when B*N > 0");
  const int64_t per_sample = (int64_t)fd.N * fd.H * fd.W * fd.C;
  if (per_sample >= (int64_t)1 << 31)
    return fail(FBEV_ERR_UNSUPPORTED, "one sample's features span %lld elements (limit 2^31 - 1)",
                (long long)per_sample);
  if ((int64_t)Q * fd.C >= (int64_t)1 << 40 || (int64_t)Q >= (int64_t)1 << 30)
    return fail(FBEV_ERR_UNSUPPORTED, "Q=%d queries too many", Q);
  a.K = K;
  a.R = R;
  a.t = t;
  a.B = fd.B;
  a.N = fd.N;
  a.C = fd.C;
  a.H = fd.H;
  a.W = fd.W;
  a.Q = Q;
  a.Kp = Kp;
  return FBEV_OK;
}

fbev_status deform_forward_impl(const float* features, fbev_feat_desc fd, const float* K, const float* R,
                                const float* t, const float* anchors, const float* offsets, const float* weights,
                                int32_t Q, int32_t Kp, float* out, void* stream) {
  fbev::DeformArgs a{};
  fbev_status s = check_deform(fd, Q, Kp, K, R, t, a);
  if (s != FBEV_OK) return s;
  const int64_t n_out = (int64_t)fd.B * Q * fd.C;
  if (n_out == 0) return FBEV_OK;
  if (out == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "out is NULL");
  if (anchors == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "anchors is NULL");
  const bool pairs = (int64_t)fd.N * Kp > 0;
  if (pairs && (offsets == nullptr || weights == nullptr))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "offsets and weights must be non-NULL when N*Kp > 0");
  if (pairs && (int64_t)fd.H * fd.W > 0 && features == nullptr)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "features is NULL");
  a.feat = features;
  a.anchors = anchors;
  a.offsets = offsets;
  a.weights = weights;
  a.out = out;
  return device_status(fbev::launch_deform_forward(a, static_cast<hipStream_t>(stream)), "fbev_deform_forward launch");
}

// The backward's dL/dF gather indexes pixels and entries (at most 4 N Kp per query) with 32 bits.
fbev_status check_deform_backward(const fbev_feat_desc& fd, int32_t Q, int32_t Kp, const float* K, const float* R,
                                  const float* t, fbev::DeformArgs& a, bool cams = true) {
  const fbev_status s = check_deform(fd, Q, Kp, K, R, t, a, cams);
  if (s != FBEV_OK) return s;
  const int64_t npix = (int64_t)fd.B * fd.N * fd.H * fd.W;
  if (npix >= (int64_t)1 << 31)
    return fail(FBEV_ERR_UNSUPPORTED, "%lld feature pixels (limit 2^31 - 1)", (long long)npix);
  const int64_t entries = (int64_t)fd.B * Q * 4 * fd.N * Kp;
  if (entries >= (int64_t)1 << 31)
    return fail(FBEV_ERR_UNSUPPORTED, "B*Q*4*N*Kp = %lld gradient entries (limit 2^31 - 1)", (long long)entries);
  return FBEV_OK;
}

fbev_status deform_workspace_impl(fbev_feat_desc fd, int32_t Q, int32_t Kp, size_t* bytes) {
  if (bytes == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "bytes is NULL");
  fbev::DeformArgs a{};
  const fbev_status s = check_deform_backward(fd, Q, Kp, nullptr, nullptr, nullptr, a, false);
  if (s != FBEV_OK) return s;
  *bytes = fbev::deform_backward_workspace_bytes(a);
  return FBEV_OK;
}

fbev_status deform_backward_impl(const float* grad_out, const float* features, fbev_feat_desc fd, const float* K,
                                 const float* R, const float* t, const float* anchors, const float* offsets,
                                 const float* weights, int32_t Q, int32_t Kp, float* grad_features,
                                 float* grad_weights, float* grad_offsets, float* grad_anchors, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  fbev::DeformArgs a{};
  fbev_status s = check_deform_backward(fd, Q, Kp, K, R, t, a);
  if (s != FBEV_OK) return s;
  const int64_t n_feat = (int64_t)fd.B * fd.N * fd.H * fd.W * fd.C;
  const int64_t n_q = (int64_t)fd.B * Q;
  const bool pairs = (int64_t)fd.N * Kp > 0;
  if (n_feat > 0 && grad_features == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_features is NULL");
  if (n_q > 0 && pairs && grad_weights == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_weights is NULL");
  if (n_q > 0 && Kp > 0 && grad_offsets == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "grad_offsets is NULL");
  if (n_q > 0) {
    if (anchors == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "anchors is NULL");
    if (Kp > 0 && offsets == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "offsets is NULL");
    if (pairs && weights == nullptr) return fail(FBEV_ERR_INVALID_ARGUMENT, "weights is NULL");
    if (pairs && fd.C > 0 && (int64_t)fd.H * fd.W > 0 && (features == nullptr || grad_out == nullptr))
      return fail(FBEV_ERR_INVALID_ARGUMENT, "features and grad_out must be non-NULL");
  }
  a.grad = grad_out;
  a.feat = features;
  a.anchors = anchors;
  a.offsets = offsets;
  a.weights = weights;
  a.gfeat = grad_features;
  a.gweights = grad_weights;
  a.goffsets = grad_offsets;
  a.ganchors = grad_anchors;
  const size_t need = fbev::deform_backward_workspace_bytes(a);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(FBEV_ERR_INVALID_ARGUMENT, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
    return fail(FBEV_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  return device_status(fbev::launch_deform_backward(a, workspace, static_cast<hipStream_t>(stream)),
                       "fbev_deform_backward launch");
}

}  // namespace

extern "C" {

fbev_status fbev_forward(const void* features, fbev_dtype dtype, fbev_feat_desc fd, const float* K, const float* R,
                         const float* t, fbev_range bev_range, int32_t X, int32_t Y, int32_t Z, float* out,
                         uint8_t* counts, void* stream) {
  return forward_impl(features, dtype, fd, 1, nullptr, K, R, t, bev_range, X, Y, Z, out, counts, stream);
}

fbev_status fbev_backward(const float* grad_out, fbev_feat_desc fd, const float* K, const float* R, const float* t,
                          fbev_range bev_range, int32_t X, int32_t Y, int32_t Z, float* grad_features,
                          void* stream) {
  return backward_impl(grad_out, fd, 1, nullptr, K, R, t, bev_range, X, Y, Z, grad_features, stream);
}

fbev_status fbev_forward_temporal(const void* features, fbev_dtype dtype, fbev_feat_desc fd, const float* K,
                                  const float* R, const float* t, fbev_range bev_range, int32_t X, int32_t Y,
                                  int32_t Z, const float* prev_bev, int32_t Cp, const float* ego, float* out,
                                  uint8_t* counts, void* stream) {
  return forward_impl(features, dtype, fd, 1, nullptr, K, R, t, bev_range, X, Y, Z, out, counts, stream, prev_bev, Cp,
                      ego);
}

fbev_status fbev_backward_temporal(const float* grad_out, fbev_feat_desc fd, const float* K, const float* R,
                                   const float* t, fbev_range bev_range, int32_t X, int32_t Y, int32_t Z, int32_t Cp,
                                   const float* ego, float* grad_features, float* grad_prev, void* stream) {
  return backward_impl(grad_out, fd, 1, nullptr, K, R, t, bev_range, X, Y, Z, grad_features, stream, Cp, ego,
                       grad_prev);
}

fbev_status fbev_forward_levels(const void* features, fbev_dtype dtype, fbev_feat_desc fd, int32_t L,
                                const int32_t* ratios, const float* K, const float* R, const float* t,
                                fbev_range bev_range, int32_t X, int32_t Y, int32_t Z, float* out, uint8_t* counts,
                                void* stream) {
  return forward_impl(features, dtype, fd, L, ratios, K, R, t, bev_range, X, Y, Z, out, counts, stream);
}

fbev_status fbev_backward_cameras_workspace(fbev_feat_desc fd, int32_t X, int32_t Y, int32_t Z, size_t* bytes) {
  return cameras_workspace_impl(fd, X, Y, Z, bytes);
}

fbev_status fbev_backward_cameras(const float* grad_out, const float* features, fbev_feat_desc fd, const float* K,
                                  const float* R, const float* t, fbev_range bev_range, int32_t X, int32_t Y,
                                  int32_t Z, float* grad_K, float* grad_R, float* grad_t, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return backward_cameras_impl(grad_out, features, fd, K, R, t, bev_range, X, Y, Z, grad_K, grad_R, grad_t, workspace,
                               workspace_bytes, stream);
}

fbev_status fbev_backward_cameras_noalloc(const float* grad_out, const float* features, fbev_feat_desc fd,
                                          const float* K, const float* R, const float* t, fbev_range bev_range,
                                          int32_t X, int32_t Y, int32_t Z, float* grad_K, float* grad_R,
                                          float* grad_t, void* stream) {
  return backward_cameras_impl(grad_out, features, fd, K, R, t, bev_range, X, Y, Z, grad_K, grad_R, grad_t, nullptr, 0,
                               stream, true);
}

fbev_status fbev_backward_levels(const float* grad_out, fbev_feat_desc fd, int32_t L, const int32_t* ratios,
                                 const float* K, const float* R, const float* t, fbev_range bev_range, int32_t X,
                                 int32_t Y, int32_t Z, float* grad_features, void* stream) {
  return backward_impl(grad_out, fd, L, ratios, K, R, t, bev_range, X, Y, Z, grad_features, stream);
}

fbev_status fbev_lss_forward(const float* depth, const float* context, fbev_feat_desc fd, int32_t D, float d_min,
                             float d_step, const float* K, const float* R, const float* t, fbev_range bev_range,
                             int32_t X, int32_t Y, float* out, void* stream) {
  return lss_forward_impl(depth, context, fd, D, d_min, d_step, K, R, t, bev_range, X, Y, out, stream);
}

fbev_status fbev_lss_backward(const float* grad_out, const float* depth, const float* context, fbev_feat_desc fd,
                              int32_t D, float d_min, float d_step, const float* K, const float* R, const float* t,
                              fbev_range bev_range, int32_t X, int32_t Y, float* grad_depth, float* grad_context,
                              void* stream) {
  return lss_backward_impl(grad_out, depth, context, fd, D, d_min, d_step, K, R, t, bev_range, X, Y, grad_depth,
                           grad_context, stream);
}

fbev_status fbev_deform_forward(const float* features, fbev_feat_desc fd, const float* K, const float* R,
                                const float* t, const float* anchors, const float* offsets, const float* weights,
                                int32_t Q, int32_t Kp, float* out, void* stream) {
  return deform_forward_impl(features, fd, K, R, t, anchors, offsets, weights, Q, Kp, out, stream);
}

fbev_status fbev_deform_backward_workspace(fbev_feat_desc fd, int32_t Q, int32_t Kp, size_t* bytes) {
  return deform_workspace_impl(fd, Q, Kp, bytes);
}

fbev_status fbev_deform_backward(const float* grad_out, const float* features, fbev_feat_desc fd, const float* K,
                                 const float* R, const float* t, const float* anchors, const float* offsets,
                                 const float* weights, int32_t Q, int32_t Kp, float* grad_features,
                                 float* grad_weights, float* grad_offsets, float* grad_anchors, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return deform_backward_impl(grad_out, features, fd, K, R, t, anchors, offsets, weights, Q, Kp, grad_features,
                              grad_weights, grad_offsets, grad_anchors, workspace, workspace_bytes, stream);
}

const char* fbev_status_string(fbev_status s) {
  switch (s) {
    case FBEV_OK: return "ok";
    case FBEV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FBEV_ERR_UNSUPPORTED: return "unsupported";
    case FBEV_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* fbev_last_error(void) { return g_last_error.c_str(); }

int32_t fbev_abi_version(void) { return FBEV_ABI_VERSION; }

}  // extern "C"
