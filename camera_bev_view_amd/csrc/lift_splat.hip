// Lift-Splat (the push view transform) for gfx950: forward sum-pooling of the
// lifted frustum points into BEV pillars, and its adjoint.
//
// The operator is the one the Lift-Splat-Shoot tutorial describes ("Lift",
// "Splat"): every feature-map pixel carries a depth distribution alpha over D
// bins and a context vector c; bin k places the point alpha_k * c on the
// pixel's ray at camera depth d_k = d_min + k d_step; the points move to the
// ego frame (p = R^T (d K^-1 [u, v, 1] - t)) and every BEV cell sums the
// points that fall in it, at any height.
//
// The tutorial implements the pooling as sort + prefix sum + differences at
// the cell boundaries (its cumsum trick), which needs the points, their cells
// and a sorted order in device memory.  Here the pooling runs the other way
// round, as a gather per BEV tile, with nothing stored: a workgroup owns a
// tile of cells, finds the rays that cross the tile's footprint (the ego x-y
// position of a ray's points is affine in the depth, so a two-slab test gives
// the depth interval inside the tile, and with it the candidate bins), and
// adds each candidate point whose cell is in the tile into a wave-private LDS
// copy of the tile (lanes = channels, one point per step: no atomics); the
// copies are summed and the tile leaves as coalesced rows of the [B,C,X,Y]
// output.  Each point is in exactly one cell, so each lands in exactly one
// workgroup.  The backward walks the same candidates against an LDS copy of
// the tile's upstream gradient: dL/dalpha_k of a point is one dot product
// over the channels (a wave reduction), dL/dc of a pixel sums alpha_k g over
// the pixel's points in the tile and leaves with one atomic per (pixel, tile)
// over consecutive channels.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lift_splat.h"

namespace fbev {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kBlock = kWave * kWaves;
constexpr int kTX = 4;                    // tile rows along x
constexpr int kTY = 8;                    // tile cells along y
constexpr int kCells = kTX * kTY;
constexpr int kCg = 64;                   // channels per group (one per lane)
constexpr int kLd = kCg + 1;              // padded LDS row of one cell's channels
constexpr int kCamD = 8;                  // doubles per camera: M rows x and y (3 each), origin x, y

__device__ __forceinline__ int xcd_tile(int bid, int nblk) {
  const int xcd = bid & 7, k = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  return (xcd < rem) ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per camera, in LDS: the x and y rows of M = R^T K^-1 and of the origin
// o = -R^T t, so the ego x-y of the point at camera depth d on pixel (u, v)'s
// ray is o + d M [u, v, 1] (tutorial, "Splat" step 1).
__device__ void stage_rays(double* sCam, const float* K, const float* R, const float* t, int b, int N) {
  for (int n = threadIdx.x; n < N; n += kBlock) {
    const size_t bn = (size_t)b * N + n;
    const float* Kn = K + bn * 9;
    const float* Rn = R + bn * 9;
    const float* tn = t + bn * 3;
    double k[9], ki[9];
    for (int i = 0; i < 9; ++i) k[i] = (double)Kn[i];
    // inverse by cofactors
    const double c00 = k[4] * k[8] - k[5] * k[7], c01 = k[5] * k[6] - k[3] * k[8], c02 = k[3] * k[7] - k[4] * k[6];
    const double det = k[0] * c00 + k[1] * c01 + k[2] * c02;
    const double id = 1.0 / det;
    ki[0] = c00 * id;
    ki[1] = (k[2] * k[7] - k[1] * k[8]) * id;
    ki[2] = (k[1] * k[5] - k[2] * k[4]) * id;
    ki[3] = c01 * id;
    ki[4] = (k[0] * k[8] - k[2] * k[6]) * id;
    ki[5] = (k[2] * k[3] - k[0] * k[5]) * id;
    ki[6] = c02 * id;
    ki[7] = (k[1] * k[6] - k[0] * k[7]) * id;
    ki[8] = (k[0] * k[4] - k[1] * k[3]) * id;
    double* c = sCam + n * kCamD;
    for (int r = 0; r < 2; ++r) {      // ego row r of R^T is column r of R
      for (int j = 0; j < 3; ++j) {
        double m = 0.0;
        for (int q = 0; q < 3; ++q) m = fma((double)Rn[q * 3 + r], ki[q * 3 + j], m);
        c[r * 3 + j] = m;
      }
      double o = 0.0;
      for (int q = 0; q < 3; ++q) o = fma(-(double)Rn[q * 3 + r], (double)tn[q], o);
      c[6 + r] = o;
    }
  }
}

// Depth interval [lo, hi) over which o + d * dir stays in the slab [a, b).
__device__ __forceinline__ void slab(double o, double dir, double a, double b, double& lo, double& hi) {
  if (dir > 0.0) {
    lo = fmax(lo, (a - o) / dir);
    hi = fmin(hi, (b - o) / dir);
  } else if (dir < 0.0) {
    lo = fmax(lo, (b - o) / dir);
    hi = fmin(hi, (a - o) / dir);
  } else if (!(o >= a && o < b)) {
    hi = -1.0;
    lo = 1.0;
  }
}

// Phase A (one pixel per lane): the candidate bins [k0, k0 + nb) of pixel p's
// ray for the tile footprint [xa, xb) x [ya, yb), widened by `pad` metres and
// by one bin on each side so that every bin whose point the cell test below
// puts in the tile is a candidate; nb = 0 when the ray misses the tile.  The
// ego x-y of the ray's point at depth d is (ox, oy) + d (rx, ry).
struct Ray {
  int n, k0, nb;
  double rx, ry;
};

__device__ __forceinline__ Ray ray_candidates(const double* sCam, const LssArgs& a, int p, double xa, double xb,
                                              double ya, double yb) {
  const int HW = a.H * a.W;
  Ray r;
  r.n = p / HW;
  const int rem = p - r.n * HW, v = rem / a.W, u = rem - v * a.W;
  const double* c = sCam + r.n * kCamD;
  r.rx = fma(c[0], (double)u, fma(c[1], (double)v, c[2]));
  r.ry = fma(c[3], (double)u, fma(c[4], (double)v, c[5]));
  double lo = a.dmin - a.dstep, hi = a.dmin + (double)a.D * a.dstep;
  slab(c[6], r.rx, xa, xb, lo, hi);
  slab(c[7], r.ry, ya, yb, lo, hi);
  r.k0 = 0;
  r.nb = 0;
  if (lo <= hi) {
    const int k0 = max(0, (int)fmax(ceil((lo - a.dmin) / a.dstep) - 1.0, -1.0));
    const int k1 = min(a.D - 1, (int)fmin(floor((hi - a.dmin) / a.dstep) + 1.0, (double)a.D));
    if (k0 <= k1) {
      r.k0 = k0;
      r.nb = k1 - k0 + 1;
    }
  }
  return r;
}

// Tile-local cell of the point at bin k on the ray (ox, oy) + d (rx, ry), or -1
// when the point is outside the tile or the grid.  The cell index is the
// floor of the offset from the grid's lower edge in cell units, evaluated in
// double precision like the rest of the geometry.
__device__ __forceinline__ int point_cell(const LssArgs& a, double ox, double oy, double rx, double ry, int k, int i0,
                                          int j0) {
  const double d = a.dmin + (double)k * a.dstep;
  const double px = fma(d, rx, ox), py = fma(d, ry, oy);
  const double fi = floor((px - a.x_min) / a.cdx), fj = floor((py - a.y_min) / a.cdy);
  const double ie = (double)min(i0 + kTX, a.X), je = (double)min(j0 + kTY, a.Y);
  if (!(fi >= (double)i0 && fi < ie && fj >= (double)j0 && fj < je)) return -1;
  return ((int)fi - i0) * kTY + ((int)fj - j0);
}

__device__ __forceinline__ int read_lane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float read_lane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double read_lane(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

constexpr int kGroup = 8;   // candidate rays whose loads one wave keeps in flight together

// One tile, both directions.  Forward: acc is this wave's private copy of the
// tile, [kCells][kLd], every in-tile point adds alpha_k c.  Backward: acc is
// the tile's upstream gradient (read only); every in-tile point gives
// dL/dalpha_k = <c, g[cell]> and adds alpha_k g[cell] to the pixel's dL/dc.
template <bool BWD>
__device__ __forceinline__ void splat_tile(const LssArgs& a, const double* sCam, float* acc, int b, int i0, int j0,
                                           int wid, int lane) {
  const double xa = a.x_min + (double)i0 * a.cdx, xb = a.x_min + (double)(i0 + kTX) * a.cdx;
  const double ya = a.y_min + (double)j0 * a.cdy, yb = a.y_min + (double)(j0 + kTY) * a.cdy;
  // a point the cell test puts in the tile is inside the footprint up to rounding
  const double pad = 1e-6 * fmax(a.cdx, a.cdy);
  const int npix = a.N * a.H * a.W;
  const bool ch = lane < a.Cg;
  const float* ctx_b = a.ctx + (size_t)b * npix * a.C + a.c_lo;
  const float* dep_b = a.depth + (size_t)b * npix * a.D;
  float* gctx_b = BWD ? a.gctx + (size_t)b * npix * a.C + a.c_lo : nullptr;
  float* gdep_b = BWD ? a.gdep + (size_t)b * npix * a.D : nullptr;

  for (int base = wid * kWave; base < npix; base += kBlock) {
    const int p = base + lane;
    Ray r = {0, 0, 0, 0.0, 0.0};
    if (p < npix) r = ray_candidates(sCam, a, p, xa - pad, xb + pad, ya - pad, yb + pad);
    uint64_t mask = __ballot(r.nb > 0);
    while (mask) {
      // Phase B: up to kGroup candidate rays; their context rows, depth bins and
      // bin cells are loaded / computed before any of them is consumed.
      int gp[kGroup], gk0[kGroup], gnb[kGroup], gn[kGroup];
      double grx[kGroup], gry[kGroup];
      float cv[kGroup], av[kGroup];
      int cell[kGroup];
      uint64_t in[kGroup];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        gnb[g] = 0;
        if (mask) {
          const int src = __builtin_ctzll(mask);
          mask &= mask - 1;
          gp[g] = read_lane(p, src);
          gk0[g] = read_lane(r.k0, src);
          gnb[g] = read_lane(r.nb, src);
          gn[g] = read_lane(r.n, src);
          grx[g] = read_lane(r.rx, src);
          gry[g] = read_lane(r.ry, src);
        }
      }
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        cv[g] = 0.f;
        av[g] = 0.f;
        cell[g] = -1;
        if (gnb[g] > 0) {
          if (ch) cv[g] = ctx_b[(size_t)gp[g] * a.C + lane];
          if (lane < gnb[g]) {
            av[g] = dep_b[(size_t)gp[g] * a.D + gk0[g] + lane];
            const double* c = sCam + gn[g] * kCamD;
            cell[g] = point_cell(a, c[6], c[7], grx[g], gry[g], gk0[g] + lane, i0, j0);
          }
        }
        in[g] = __ballot(cell[g] >= 0);
      }
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        if (gnb[g] == 0) continue;
        float dc = 0.f;
        bool any = false;
        for (int kb = 0;;) {
          float dav = 0.f;
          uint64_t m = in[g];
          any = any || m != 0;
          while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            const int ce = read_lane(cell[g], j);
            const float al = read_lane(av[g], j);
            float* row = acc + ce * kLd + lane;
            if (BWD) {
              const float gv = *row;
              const float da = wave_sum(cv[g] * gv);
              dav = (lane == j) ? da : dav;
              dc = fmaf(al, gv, dc);
            } else {
              *row = fmaf(al, cv[g], *row);
            }
          }
          // each point lies in one cell, so with one channel group this is the only add to its slot
          if (BWD && ((in[g] >> lane) & 1)) unsafeAtomicAdd(gdep_b + (size_t)gp[g] * a.D + gk0[g] + kb + lane, dav);
          // bins past the first 64 of this ray (long crossings at fine depth steps)
          kb += kWave;
          if (kb >= gnb[g]) break;
          av[g] = 0.f;
          cell[g] = -1;
          if (kb + lane < gnb[g]) {
            av[g] = dep_b[(size_t)gp[g] * a.D + gk0[g] + kb + lane];
            const double* c = sCam + gn[g] * kCamD;
            cell[g] = point_cell(a, c[6], c[7], grx[g], gry[g], gk0[g] + kb + lane, i0, j0);
          }
          in[g] = __ballot(cell[g] >= 0);
        }
        if (BWD && any && ch) unsafeAtomicAdd(gctx_b + (size_t)gp[g] * a.C + lane, dc);
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void lift_splat_fwd(LssArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* sCam = reinterpret_cast<double*>(smem);
  float* sAcc = reinterpret_cast<float*>(smem + sizeof(double) * kCamD * a.N);   // [kWaves][kCells][kLd]

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int jt = tile % a.tiles_y;
  const int r1 = tile / a.tiles_y;
  const int it = r1 % a.tiles_x;
  const int b = r1 / a.tiles_x;
  const int i0 = it * kTX, j0 = jt * kTY;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);

  stage_rays(sCam, a.K, a.R, a.t, b, a.N);
  for (int e = threadIdx.x; e < kWaves * kCells * kLd; e += kBlock) sAcc[e] = 0.f;
  __syncthreads();

  splat_tile<false>(a, sCam, sAcc + wid * kCells * kLd, b, i0, j0, wid, lane);
  __syncthreads();

  // sum the wave copies and store the tile: kTY consecutive y per (channel, x)
  const size_t cs = (size_t)a.X * a.Y;
  float* ob = a.out + ((size_t)b * a.C + a.c_lo) * cs;
  for (int e = threadIdx.x; e < a.Cg * kCells; e += kBlock) {
    const int c = e / kCells, cell = e - c * kCells;
    const int ci = cell / kTY, cj = cell - ci * kTY;
    if (i0 + ci < a.X && j0 + cj < a.Y) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += sAcc[(w * kCells + cell) * kLd + c];
      __builtin_nontemporal_store(s, ob + c * cs + (size_t)(i0 + ci) * a.Y + j0 + cj);
    }
  }
}

__global__ __launch_bounds__(kBlock) void lift_splat_bwd(LssArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* sCam = reinterpret_cast<double*>(smem);
  float* sG = reinterpret_cast<float*>(smem + sizeof(double) * kCamD * a.N);      // [kCells][kLd]

  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int jt = tile % a.tiles_y;
  const int r1 = tile / a.tiles_y;
  const int it = r1 % a.tiles_x;
  const int b = r1 / a.tiles_x;
  const int i0 = it * kTX, j0 = jt * kTY;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);

  stage_rays(sCam, a.K, a.R, a.t, b, a.N);
  {
    // the tile's upstream gradient; channels past Cg and cells past the grid read as 0
    const size_t cs = (size_t)a.X * a.Y;
    const float* gb = a.grad + ((size_t)b * a.C + a.c_lo) * cs;
    for (int e = threadIdx.x; e < kCg * kCells; e += kBlock) {
      const int c = e / kCells, cell = e - c * kCells;
      const int ci = cell / kTY, cj = cell - ci * kTY;
      sG[cell * kLd + c] = (c < a.Cg && i0 + ci < a.X && j0 + cj < a.Y)
                               ? __builtin_nontemporal_load(gb + c * cs + (size_t)(i0 + ci) * a.Y + j0 + cj)
                               : 0.f;
    }
  }
  __syncthreads();
  splat_tile<true>(a, sCam, sG, b, i0, j0, wid, lane);
}

__global__ void lss_fill_zero(float* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride) dst[k] = 0.f;
}

hipError_t fill(float* dst, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  const unsigned nb = (unsigned)(blocks < 2048 ? blocks : 2048);
  hipLaunchKernelGGL(lss_fill_zero, dim3(nb), dim3(256), 0, stream, dst, n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lss_forward(LssArgs a, hipStream_t stream) {
  a.tiles_x = (a.X + kTX - 1) / kTX;
  a.tiles_y = (a.Y + kTY - 1) / kTY;
  const long long tiles = (long long)a.B * a.tiles_x * a.tiles_y;
  if (tiles == 0 || a.C == 0) return hipSuccess;
  const size_t shmem = sizeof(double) * kCamD * a.N + sizeof(float) * kWaves * kCells * kLd;
  for (int c = 0; c < a.C; c += kCg) {
    a.c_lo = c;
    a.Cg = (a.C - c < kCg) ? a.C - c : kCg;
    hipLaunchKernelGGL(lift_splat_fwd, dim3((unsigned)tiles), dim3(kBlock), shmem, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_lss_backward(LssArgs a, hipStream_t stream) {
  const size_t npix = (size_t)a.B * a.N * a.H * a.W;
  hipError_t e = hipSuccess;
  if (a.gdep != nullptr) e = fill(a.gdep, npix * a.D, stream);
  if (e == hipSuccess && a.gctx != nullptr) e = fill(a.gctx, npix * a.C, stream);
  if (e != hipSuccess) return e;
  a.tiles_x = (a.X + kTX - 1) / kTX;
  a.tiles_y = (a.Y + kTY - 1) / kTY;
  const long long tiles = (long long)a.B * a.tiles_x * a.tiles_y;
  // with no depth bins or no channels both gradients are zero
  if (a.gdep == nullptr || a.gctx == nullptr || tiles == 0 || a.C == 0 || a.D == 0 || npix == 0) return hipSuccess;
  const size_t shmem = sizeof(double) * kCamD * a.N + sizeof(float) * kCells * kLd;
  for (int c = 0; c < a.C; c += kCg) {
    a.c_lo = c;
    a.Cg = (a.C - c < kCg) ? a.C - c : kCg;
    hipLaunchKernelGGL(lift_splat_bwd, dim3((unsigned)tiles), dim3(kBlock), shmem, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fbev
