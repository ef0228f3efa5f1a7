// Gradients of the dense Sampling-VT output with respect to the cameras
// (dL/dK, dL/dR, dL/dt) for gfx950.
//
// The sampling chain of the FlashBEV notes ("Method" items 1-4: projection,
// validity, bilinear sample, valid-camera mean, height sum) is differentiable
// in the cameras wherever the in-view mask and the counts do not change
// (SparseDriveV2 notes, "Deformable Aggregation" pitfalls: the projection and
// the sampling must let gradients through).  For an in-view sample of camera
// n at voxel centre p with h = P [p; 1], P = K [R | t], u = h_1 / h_3 and
// v = h_2 / h_3:
//
//   dL/du = <g_cell, d(sample)/du> / count,  dL/dv likewise,
//   d(sample)/du = (1 - b)(F01 - F00) + b (F11 - F10),
//   d(sample)/dv = (1 - a)(F10 - F00) + a (F11 - F01),
//   dL/dP_n += [dL/du; dL/dv; -(u dL/du + v dL/dv)] [p; 1]^T / h_3,
//
// and finally dL/dK = dL/dP [R | t]^T, dL/d[R | t] = K^T dL/dP.
//
// camera_grad_main: a workgroup walks units of 16 cells of one x-row and one
// 64-channel group (the tile's upstream gradient staged in LDS).  Per cell and
// pass, lane n * zpc + zl tests bin zc + zl against camera n (the layout of the
// forward's validity pass, so a lane's camera is the same in every pass and
// every cell); the in-view samples are compacted into a per-wave list, and for
// each of them the wave computes the four tap dot products <g_cell, F_tap> with
// lanes = (tap, 4-channel chunk) and a 16-lane DPP sum.  The owning lane turns
// them into dL/du, dL/dv and adds its 12 entries of dL/dP in registers.  At the
// end the lanes of one camera and the four waves are summed in a fixed order
// into the workgroup's slice of the workspace.  camera_grad_finish (a
// workgroup per camera, a wave per entry) sums the slices in a fixed order
// (fp64) and applies the chain through P: the result is deterministic.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"
#include "wave_ops.h"

namespace fbev {

// Device scratch of the allocation-free variant (fbev_backward_cameras_noalloc): the partial dL/dP
// slices of the main kernel.  Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, never the device memory: host code uses only the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kCameraScratchBytes];

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kBlock = kWave * kWaves;
constexpr int kTileY = 32;               // cells per unit (one x-row): 128-byte rows of the upstream gradient
constexpr int kCg = 64;                  // channels per unit
constexpr int kGLd = kCg + 4;            // padded LDS row of one cell's upstream gradient
constexpr int kRedLd = 13;               // padded LDS row of one lane's 12 partial sums
constexpr int kUnroll = 4;               // samples per gather step (the four-way row sum)
constexpr int kMaxGroups = 1792;         // workgroups of the main kernel per batch sample, at most
constexpr int kFinishPer = 28;           // workgroup slices each finishing lane adds
static_assert(kMaxGroups <= kFinishPer * kWave, "the finish reads every slice in one step");

typedef uint32_t u32x4 __attribute__((__vector_size__(16)));

__device__ __forceinline__ double recip(double x) {
  double r = __builtin_amdgcn_rcp(x);
  r = fma(r, fma(-x, r, 1.0), r);
  r = fma(r, fma(-x, r, 1.0), r);
  return r;
}

// Four row sums at once: d[q] holds lane j's part of value q (j = lane % 16);
// afterwards every lane of quad q of the row (j / 4 == q) holds the row's sum
// of value q.  Mirroring across the row and then across each half pairs every
// lane with three others so that the four lanes of a quad together cover the
// row; each step keeps half of the values (5 DPP adds instead of 16).
__device__ __forceinline__ float row_sum16_x4(const float (&d)[4], int j) {
  const bool lower = j < 8;
  const float a0 = (lower ? d[0] : d[2]) + dpp<kRowMirror>(lower ? d[2] : d[0]);
  const float a1 = (lower ? d[1] : d[3]) + dpp<kRowMirror>(lower ? d[3] : d[1]);
  const bool lo4 = (j & 7) < 4;
  float b = (lo4 ? a0 : a1) + dpp<kHalfMirror>(lo4 ? a1 : a0);
  b += dpp<kQuadSwap1>(b);
  b += dpp<kQuadSwap2>(b);
  return b;
}

struct CamGradArgs {
  Problem p;
  const float* grad;       // [B, C, X, Y]
  double* work;            // [B, N, 12, gx] partial dL/dP per workgroup
  float* gK;               // [B, N, 3, 3]
  float* gR;               // [B, N, 3, 3]
  float* gt;               // [B, N, 3]
  int gx;                  // workgroups per batch sample
  int tiles_y, groups, units;
};

// V = 4: lane chunk j holds channels 4j..4j+3 of the group (one 16-byte load
// per tap); V = 1: channels j, j+16, j+32, j+48 (four 4-byte loads).
template <int V>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(V == 4 ? 5 : 4))) void camera_grad_main(CamGradArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Problem& p = a.p;
  double* sP = reinterpret_cast<double*>(smem);                                   // [N][12]
  float* sG = reinterpret_cast<float*>(sP + 12 * p.N);                            // [kTileY][kGLd]
  float* sW = sG + kTileY * kGLd;                                                 // [kWaves][kWave * kRedLd]
  const int b = blockIdx.y;
  for (int e = threadIdx.x; e < p.N * 12; e += kBlock) {
    const int n = e / 12, r = (e % 12) >> 2, c = e & 3;
    const size_t bn = (size_t)b * p.N + n;
    double s = 0.0;
    for (int k = 0; k < 3; ++k)
      s = fma((double)p.K[bn * 9 + r * 3 + k], (double)(c < 3 ? p.R[bn * 9 + k * 3 + c] : p.t[bn * 3 + k]), s);
    sP[e] = s;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);
  float* wbuf = sW + wid * kWave * kRedLd;
  int* rec = reinterpret_cast<int*>(wbuf);                                        // [64][4] tap offsets of listed samples
  float* dots = wbuf + 4 * kWave;                                                 // [64][4] tap dot products
  const int tap = lane >> 4, j = lane & 15;

  // phase-A lane role: camera ln, bin zl of each pass
  const int zpc = kWave / p.N;
  const int ln = lane / zpc, zl = lane - ln * zpc;
  const bool lane_ok = lane < zpc * p.N;
  uint64_t bin_lanes = 0;
  for (int n = 0; n < p.N; ++n) bin_lanes |= 1ull << (n * zpc);
  bin_lanes <<= zl;
  const double* P = sP + (lane_ok ? ln : 0) * 12;
  const double Wm1 = (double)(p.W - 1), Hm1 = (double)(p.H - 1);
  const int HWC = p.H * p.W * p.C;
  const float* fb = static_cast<const float*>(p.feat) + (size_t)b * p.N * HWC;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(fb), 0,
                                                                      (int)(sizeof(float) * p.N * HWC), 0x00020000);
  float acc[12];
#pragma unroll
  for (int k = 0; k < 12; ++k) acc[k] = 0.f;

  // units dealt round-robin: neighbouring units run on different XCDs (keeping them on one XCD
  // halves the HBM traffic but concentrates each XCD's workgroups on the same image rows, which
  // measured slower)
  for (int u = blockIdx.x; u < a.units; u += a.gx) {
    const int grp = u % a.groups;
    const int rest = u / a.groups;
    const int ty = rest % a.tiles_y, x = rest / a.tiles_y;
    const int c0 = grp * kCg;
    const int Cg = min(kCg, p.C - c0);
    // the tile's upstream gradient, all loads issued before the first is used (element 0 stands in
    // for the ones outside the grid, whose values are then dropped)
    float gv[kTileY * kCg / kBlock];
#pragma unroll
    for (int i = 0; i < kTileY * kCg / kBlock; ++i) {
      const int e = threadIdx.x + i * kBlock;
      const int c = e / kTileY, cell = e - c * kTileY;
      const int y = ty * kTileY + cell;
      const bool ok = c < Cg && y < p.Y;
      gv[i] = a.grad[ok ? (((size_t)b * p.C + c0 + c) * p.X + x) * p.Y + y : 0];
    }
    __syncthreads();   // the camera table is staged; the previous unit's readers are done with sG
#pragma unroll
    for (int i = 0; i < kTileY * kCg / kBlock; ++i) {
      const int e = threadIdx.x + i * kBlock;
      const int c = e / kTileY, cell = e - c * kTileY;
      sG[cell * kGLd + c] = (c < Cg && ty * kTileY + cell < p.Y) ? gv[i] : 0.f;
    }
    __syncthreads();
    const double px = p.ox + ((double)x + 0.5) * p.dx;
    const double hA0 = fma(P[0], px, P[3]), hA1 = fma(P[4], px, P[7]), hA2 = fma(P[8], px, P[11]);
    const int jo = (4 * j < Cg) ? 4 * j : 0;             // this lane's channels; past the group it rereads c0
    for (int cell = wid; cell < kTileY; cell += kWaves) {
      const int y = ty * kTileY + cell;
      if (y >= p.Y) break;
      const double py = p.oy + ((double)y + 0.5) * p.dy;
      float g[4];
      if (V == 4) {
        const float4 gv = *reinterpret_cast<const float4*>(sG + cell * kGLd + 4 * j);
        g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) g[i] = sG[cell * kGLd + j + 16 * i];
      }
      for (int zc = 0; zc < p.Z; zc += zpc) {
        // ---- validity of (bin zc + zl, camera ln) by sign tests on h
        const int z = zc + zl;
        const bool in_range = lane_ok && z < p.Z;
        bool valid = false;
        double pz = 0.0, h0 = 0.0, h1 = 0.0, h2 = 1.0;
        if (in_range) {
          pz = p.oz + ((double)z + 0.5) * p.dz;
          h0 = fma(P[2], pz, fma(P[1], py, hA0));
          h1 = fma(P[6], pz, fma(P[5], py, hA1));
          h2 = fma(P[10], pz, fma(P[9], py, hA2));
          valid = (h2 > 0.0) && (h0 >= 0.0) && (fma(Wm1, h2, -h0) >= 0.0) && (h1 >= 0.0) && (fma(Hm1, h2, -h1) >= 0.0);
        }
        const uint64_t m = __ballot(valid);
        if (m == 0) continue;
        const int ns = (int)__builtin_popcountll(m);
        const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        float fa = 0.f, fbt = 0.f, rc = 0.f, ih = 0.f, uf = 0.f, vf = 0.f;
        if (valid) {
          const double r = recip(h2);
          const double uu = h0 * r, vv = h1 * r;
          const double fu = fmin(fmax(floor(uu), 0.0), Wm1);
          const double fv = fmin(fmax(floor(vv), 0.0), Hm1);
          const int x0 = (int)fu, y0 = (int)fv;
          fa = (float)(uu - fu);
          fbt = (float)(vv - fv);
          rc = __builtin_amdgcn_rcpf((float)__builtin_popcountll(m & bin_lanes));
          ih = (float)r;
          uf = (float)uu;
          vf = (float)vv;
          const int o00 = ln * HWC + (y0 * p.W + x0) * p.C + c0;
          const int ox = (x0 + 1 < p.W) ? p.C : 0, oy = (y0 + 1 < p.H) ? p.W * p.C : 0;
          *reinterpret_cast<int4*>(rec + 4 * rank) = make_int4(o00, o00 + ox, o00 + oy, o00 + ox + oy);
        }
        wave_lds_sync();
        // ---- tap dot products <g_cell, F_tap>, lanes = (tap, channel chunk)
        // All loads of a step are issued before any is used: past the list's end the last sample
        // is read again and channels past the group read channel c0, and both are dropped.
        for (int s0 = 0; s0 < ns; s0 += kUnroll) {
          float f[kUnroll][4];
          int offs[kUnroll];
#pragma unroll
          for (int i = 0; i < kUnroll; ++i) offs[i] = rec[4 * min(s0 + i, ns - 1) + tap];   // this lane's taps
#pragma unroll
          for (int i = 0; i < kUnroll; ++i) {
            const int off = offs[i];
            if (V == 4) {
              const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (off + jo), 0, 0);
#pragma unroll
              for (int k = 0; k < 4; ++k) f[i][k] = __uint_as_float(v[k]);
            } else {
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const int c = j + 16 * k;
                f[i][k] = fb[off + ((c < Cg) ? c : 0)];
              }
            }
          }
          float d[kUnroll];
#pragma unroll
          for (int i = 0; i < kUnroll; ++i) {
            d[i] = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) d[i] = fmaf(f[i][k], g[k], d[i]);   // g is 0 past the group's channels
          }
          const float sum = row_sum16_x4(d, j);                // sample s0 + j / 4 of this lane's tap row
          const int q = j >> 2;
          if ((j & 3) == 0 && s0 + q < ns) dots[(s0 + q) * 4 + tap] = sum;
        }
        wave_lds_sync();
        // ---- dL/du, dL/dv of the lane's sample and its 12 entries of dL/dP
        if (valid) {
          const float4 dd = *reinterpret_cast<const float4*>(dots + rank * 4);
          const float du = rc * ((1.f - fbt) * (dd.y - dd.x) + fbt * (dd.w - dd.z));
          const float dv = rc * ((1.f - fa) * (dd.z - dd.x) + fa * (dd.w - dd.y));
          const float al = du * ih, be = dv * ih, ga = -(du * uf + dv * vf) * ih;
          const float pt[4] = {(float)px, (float)py, (float)pz, 1.f};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc[k] = fmaf(al, pt[k], acc[k]);
            acc[4 + k] = fmaf(be, pt[k], acc[4 + k]);
            acc[8 + k] = fmaf(ga, pt[k], acc[8 + k]);
          }
        }
        wave_lds_sync();   // rec and dots are rewritten by the next pass
      }
    }
  }
  // ---- fixed-order sums: the lanes of each camera, then the four waves
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 12; ++k) wbuf[lane * kRedLd + k] = acc[k];
  __syncthreads();
  for (int e = threadIdx.x; e < p.N * 12; e += kBlock) {
    const int n = e / 12, k = e - n * 12;
    double s = 0.0;
    for (int w = 0; w < kWaves; ++w)
      for (int i = 0; i < zpc; ++i) s += (double)sW[w * kWave * kRedLd + (n * zpc + i) * kRedLd + k];
    a.work[((size_t)b * p.N * 12 + e) * a.gx + blockIdx.x] = s;
  }
}

// One workgroup per (camera, batch sample), one wave per entry of dL/dP: the
// entry is the sum of the workgroup slices (each lane a fixed strided subset,
// all loads in flight at once, then a fixed tree); then dL/dK = dL/dP [R | t]^T
// and dL/d[R | t] = K^T dL/dP.
__global__ __launch_bounds__(12 * kWave) void camera_grad_finish(CamGradArgs a) {
  __shared__ double sGP[12];
  const Problem& p = a.p;
  const int n = blockIdx.x, b = blockIdx.y;
  const size_t bn = (size_t)b * p.N + n;
  const int lane = threadIdx.x & (kWave - 1), e = threadIdx.x / kWave;
  const double* src = a.work + (bn * 12 + e) * a.gx;
  double v[kFinishPer];
#pragma unroll
  for (int k = 0; k < kFinishPer; ++k) {
    const int i = lane + k * kWave;
    v[k] = (i < a.gx) ? src[i] : 0.0;
  }
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kFinishPer; ++k) s += v[k];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) sGP[e] = s;
  __syncthreads();
  if (threadIdx.x >= 21) return;
  const int r = threadIdx.x;
  const double* G = sGP;                          // dL/dP, row-major 3 x 4
  const float* K = p.K + bn * 9;
  const float* R = p.R + bn * 9;
  const float* t = p.t + bn * 3;
  if (r < 9) {                                    // dL/dK_ik = sum_j dL/dP_ij M_kj, M = [R | t]
    const int ii = r / 3, k = r % 3;
    double w = G[ii * 4 + 3] * (double)t[k];
    for (int jj = 0; jj < 3; ++jj) w = fma(G[ii * 4 + jj], (double)R[k * 3 + jj], w);
    a.gK[bn * 9 + r] = (float)w;
  } else {                                        // dL/dM_ij = sum_k K_ki dL/dP_kj
    const int q = r - 9;
    const int ii = (q < 9) ? q / 3 : q - 9, jj = (q < 9) ? q % 3 : 3;
    double w = 0.0;
    for (int k = 0; k < 3; ++k) w = fma((double)K[k * 3 + ii], G[k * 4 + jj], w);
    if (q < 9) a.gR[bn * 9 + q] = (float)w;
    else a.gt[bn * 3 + (q - 9)] = (float)w;
  }
}

// Workgroups per batch sample: about one resident round of the chip in total
// (six or seven per CU), at least one so that the main kernel always writes
// the slices the finish reads.
int workgroups_per_sample(const Problem& p, int units) {
  const int cap = (p.B > 0 && kMaxGroups / p.B > 64) ? kMaxGroups / p.B : 64;
  return units < 1 ? 1 : (units < cap ? units : cap);
}

size_t work_bytes(const Problem& p, int gx) { return sizeof(double) * (size_t)p.B * p.N * 12 * (size_t)gx; }

void unit_counts(const Problem& p, int& tiles_y, int& groups, int& units) {
  tiles_y = (p.Y + kTileY - 1) / kTileY;
  groups = (p.C + kCg - 1) / kCg;
  const long long u = (p.Z > 0 && p.N > 0) ? (long long)p.X * tiles_y * groups : 0;
  units = (int)u;
}

}  // namespace

size_t camera_grad_workspace_bytes(const Problem& p) {
  if (p.B == 0 || p.N == 0) return 0;
  int tiles_y, groups, units;
  unit_counts(p, tiles_y, groups, units);
  return work_bytes(p, workgroups_per_sample(p, units));
}

hipError_t camera_scratch(int device, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex lock;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(lock);
  if (addr[device] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

hipError_t launch_camera_backward(const Problem& p, const float* grad_out, float* gK, float* gR, float* gt,
                                  void* work, hipStream_t stream) {
  if (p.B == 0 || p.N == 0) return hipSuccess;
  CamGradArgs a;
  a.p = p;
  a.grad = grad_out;
  a.gK = gK;
  a.gR = gR;
  a.gt = gt;
  unit_counts(p, a.tiles_y, a.groups, a.units);
  a.gx = workgroups_per_sample(p, a.units);
  a.work = static_cast<double*>(work);
  const size_t shmem = sizeof(double) * 12 * p.N + sizeof(float) * kTileY * kGLd +
                       sizeof(float) * kWaves * kWave * kRedLd;
  const dim3 grid((unsigned)a.gx, (unsigned)p.B);
  if (p.C % 4 == 0 && (reinterpret_cast<uintptr_t>(p.feat) & 15) == 0)
    hipLaunchKernelGGL(camera_grad_main<4>, grid, dim3(kBlock), shmem, stream, a);
  else
    hipLaunchKernelGGL(camera_grad_main<1>, grid, dim3(kBlock), shmem, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(camera_grad_finish, dim3((unsigned)p.N, (unsigned)p.B), dim3(12 * kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fbev
