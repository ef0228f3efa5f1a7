// Single-level fused Sampling-VT forward and backward for gfx950, organised around bin runs.
//
// The operator is the dense Sampling-VT of the FlashBEV reading notes ("Core
// Idea"; "Method" items 1-4): per BEV cell, project every height bin's voxel
// centre through every camera, keep the in-view samples, bilinearly sample,
// average over the valid cameras per bin and sum over the bins; nothing per
// (camera, bin, channel) is written to device memory.
//
// Bin runs.  For a fixed cell (x, y) and camera n, the homogeneous image
// coordinates h = P [x, y, z_k, 1] (P = K [R | t]) are affine in the bin index
// k, and each of the five in-view conditions of the SparseDriveV2 notes'
// projection rule ("Deformable Aggregation" step 2: depth h_3 > 0, and
// 0 <= u <= W-1, 0 <= v <= H-1 written as h_1 >= 0, (W-1) h_3 - h_1 >= 0,
// h_2 >= 0, (H-1) h_3 - h_2 >= 0) is a half-line in k.  So the bins camera n
// sees from a cell form one interval [lo, hi]: a "run".  The runs come from
// five fp64 multiplications per (cell, camera) by per-camera reciprocals, and
// the valid-camera count of bin k is the number of the cell's runs holding k.
// (This decides validity as the per-bin sign tests do except where a test's
// value is within rounding of zero, i.e. for a sample within ~1e-12 px of an
// image edge.)
//
// Per wave: eight consecutive cells of the flattened grid.  Phase A: lane = (cell,
// camera), the run, and an exclusive prefix of the run lengths, so the wave's
// samples have indices 0 .. T-1 in (cell, camera, bin) order.  Then rounds of
// 64 samples: phase B, lane = sample: its count, the exact projection (fp64
// reciprocal, two Newton steps), floor and fractions, the four taps with
// weights / count; pixel rows shared by consecutive bins of one run are merged
// (along a cell's vertical line the projected row is monotone, so a shared row
// is a run of consecutive samples; the first keeps it and takes the others'
// weights) and the kept taps compacted.  Phase C, the gather: lanes = (slot,
// chunk), a tap's channel group read as one coalesced channels-last row per
// 16-lane (or L-lane) slot, fp32 accumulation, and at a cell's last tap the
// slots are summed with lane swaps into the workgroup's output tile in LDS.
// The tile (32 consecutive cells of the flattened [X, Y] grid) leaves as full,
// aligned 128-byte lines of the [B, C, X, Y] output when X * Y is a multiple
// of 32.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bev_align.h"
#include "kernels.h"
#include "wave_ops.h"

namespace fbev {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kBlock = kWave * kWaves;
constexpr int kTileY = 32;               // cells per tile (flattened grid): one 128-byte output line per channel
constexpr int kCpw = kTileY / kWaves;    // cells per wave
constexpr int kOutLd = kCpw + 1;         // padded LDS row of a wave's output tile (one channel, its cells)
constexpr int kRound = kWave;            // samples per round, one per lane
constexpr int kOutOfRange = 0x7ffffff0;  // buffer offset the range check turns into a zero load

// Per camera, in LDS: P = K [R | t] (row-major 3 x 4), and for the five in-view
// conditions f_i(k) = alpha_i + beta_i k (alpha from the cell, beta per
// camera): beta_i and 1 / beta_i (0 when beta_i == 0).
struct CamRec {
  double P[12];
  double beta[5];
  double inv[5];
};

__device__ __forceinline__ double recip(double x) {
  double r = __builtin_amdgcn_rcp(x);
  r = fma(r, fma(-x, r, 1.0), r);
  r = fma(r, fma(-x, r, 1.0), r);
  return r;
}

// Camera table, staged by the whole workgroup: entry e = 12 n + 4 r + c of P = K [R | t] per thread (fp64
// from the fp32 inputs), then per camera the per-bin steps of the five condition forms (dz = bin height)
// and their reciprocals.  Ends with the workgroup barrier.
__device__ void stage_cameras(CamRec* cams, const Problem& p, int b) {
  for (int e = threadIdx.x; e < p.N * 12; e += blockDim.x) {
    const int n = e / 12, rc = e - n * 12, r = rc >> 2, col = rc & 3;
    const size_t bn = (size_t)b * p.N + n;
    const float* K = p.K + bn * 9 + r * 3;
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < 3; ++k)
      acc = fma((double)K[k], (double)(col < 3 ? p.R[bn * 9 + k * 3 + col] : p.t[bn * 3 + k]), acc);
    cams[n].P[rc] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < p.N * 5; e += blockDim.x) {
    const int n = e / 5, i = e - n * 5;
    const double* P = cams[n].P;
    const double s0 = P[2] * p.dz, s1 = P[6] * p.dz, s2 = P[10] * p.dz;
    const double be = (i == 0) ? s2                                       // depth
                    : (i == 1) ? s0                                       // u >= 0
                    : (i == 2) ? fma((double)(p.W - 1), s2, -s0)          // u <= W - 1
                    : (i == 3) ? s1                                       // v >= 0
                               : fma((double)(p.H - 1), s2, -s1);         // v <= H - 1
    cams[n].beta[i] = be;
    cams[n].inv[i] = (be != 0.0) ? 1.0 / be : 0.0;
  }
  __syncthreads();
}

// The bins [lo, hi] of camera `c` in view from the cell at (px, py); lo > hi when none.
__device__ __forceinline__ void bin_run(const CamRec& c, double px, double py, double z0, int Z, double Wm1,
                                        double Hm1, int& lo_out, int& hi_out) {
  const double h0 = fma(c.P[0], px, fma(c.P[1], py, fma(c.P[2], z0, c.P[3])));
  const double h1 = fma(c.P[4], px, fma(c.P[5], py, fma(c.P[6], z0, c.P[7])));
  const double h2 = fma(c.P[8], px, fma(c.P[9], py, fma(c.P[10], z0, c.P[11])));
  double alpha[5];
  alpha[0] = h2;
  alpha[1] = h0;
  alpha[2] = fma(Wm1, h2, -h0);
  alpha[3] = h1;
  alpha[4] = fma(Hm1, h2, -h1);
  double lo = 0.0, hi = (double)(Z - 1);
  bool none = false;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const double be = c.beta[i];
    // root of alpha + beta k, clamped far outside [0, Z) before any rounding to an integer
    const double root = fmin(fmax(-alpha[i] * c.inv[i], -2.0), (double)Z + 1.0);
    if (be > 0.0) {
      lo = fmax(lo, i == 0 ? floor(root) + 1.0 : ceil(root));      // depth: strictly positive
    } else if (be < 0.0) {
      hi = fmin(hi, i == 0 ? ceil(root) - 1.0 : floor(root));
    } else {
      none = none || (i == 0 ? !(alpha[i] > 0.0) : !(alpha[i] >= 0.0));
    }
  }
  if (none || lo > hi) {
    lo_out = 1;
    hi_out = 0;
  } else {
    lo_out = (int)lo;
    hi_out = (int)hi;
  }
}

struct Rec {
  int off;   // byte offset of the tap's pixel in the sample's features
  float w;   // bilinear weight / valid-camera count
};

typedef uint32_t u32x4 __attribute__((__vector_size__(16)));

// D consecutive dwords of one tap, accumulated into fp32 registers.
template <int D, bool BF16>
struct Lane {
  static constexpr int kVec = BF16 ? 2 * D : D;
  struct Raw {
    uint32_t d[D];
  };
  __device__ static Raw load(__amdgpu_buffer_rsrc_t rs, int off) {
    Raw r;
    int i = 0;
#pragma unroll
    for (; i + 4 <= D; i += 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 4 * i, 0, 0);
      r.d[i] = v[0];
      r.d[i + 1] = v[1];
      r.d[i + 2] = v[2];
      r.d[i + 3] = v[3];
    }
    if constexpr (D % 4 == 2) {
      typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 4 * i, 0, 0);
      r.d[i] = v[0];
      r.d[i + 1] = v[1];
      i += 2;
    }
#pragma unroll
    for (; i < D; ++i) r.d[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * i, 0, 0);
    return r;
  }
  __device__ static void fma_into(float* acc, const Raw& v, float w) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if constexpr (BF16) {
        acc[2 * i] = fmaf(w, __uint_as_float(v.d[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w, __uint_as_float(v.d[i] & 0xffff0000u), acc[2 * i + 1]);
      } else {
        acc[i] = fmaf(w, __uint_as_float(v.d[i]), acc[i]);
      }
    }
  }
};

struct RunArgs {
  Problem p;
  float* out;
  uint8_t* counts;
  int c_lo;          // first channel of this launch's group
  int Cg;            // channels of the group
  int ngroups;       // groups of Cg channels from c_lo taken by this launch in turn (the last one partial)
  int C_launch;      // channels of this launch (Cg when ngroups == 1)
  int tiles_pb;      // tiles per sample: ceil(X * Y / kTileY)
  int xcd_chunks;    // 1: each XCD takes a contiguous range of the tiles; 0: consecutive tiles on consecutive XCDs
  int write_counts;
};

// Sample descriptor: bin k (16 bits), camera n (6 bits), cell of the wave (up to 6 bits).
__device__ __forceinline__ int desc_pack(int k, int n, int cl) { return k | (n << 16) | (cl << 22); }

// The cells a wave works on: cell cl (0 <= cl < n) sits at position y0 + cl of rows of ny cells that start
// at grid row x0, shifted by yoff along y: a flat run of the [X, Y] grid (ny = Y, yoff = 0), or one row of
// a rectangular tile (y0 = 0, ny = tile width, yoff = the tile's first y).  Cells outside the grid have no
// samples.
struct CellSet {
  int x0, y0, ny, n, yoff;
  __device__ int x(int cl) const {
    int pos = y0 + cl, x = x0;
    while (pos >= ny) {
      pos -= ny;
      ++x;
    }
    return x;
  }
  __device__ int y(int cl) const {
    int pos = y0 + cl;
    while (pos >= ny) pos -= ny;
    return yoff + pos;
  }
};

// a / d for 0 <= a < 1024 and 1 <= d <= 64 by one multiply, given m = div_magic(d) (wave-uniform): the
// error a (m / 65536 - 1 / d) stays below 1024 / 65536 <= 1 / d, so the floor is exact.
__device__ __forceinline__ int div_magic(int d) { return uniform((65536 + d - 1) / d); }
__device__ __forceinline__ int div_small(int a, int m) { return (a * m) >> 16; }

template <class T>
__device__ __forceinline__ T level_of(const T (&a)[kMaxLevels], int l) {
  return l == 0 ? a[0] : l == 1 ? a[1] : l == 2 ? a[2] : a[3];
}

// Phase B for one sample: the four taps (byte offsets of their pixels, weights
// / count).  u, v are clamped to the pixel-centre box before the floor so that
// rounding at an edge never reaches outside the map; the clamped second tap at
// the last column / row repeats the first with weight 0.  With lvl_ir != 0 the
// taps are those of a coarser pyramid level of ratio 1 / lvl_ir: the point's
// level coordinate (u + 1/2) / r - 1/2, clamped to that level's box (the border
// rule of the level mean).
__device__ __forceinline__ void sample_taps(const CamRec& c, double px, double py, double pz, float rc, int H, int W,
                                            int pix_base, int pix_bytes, Rec (&t)[4], int& top, int& bot,
                                            int& xy, double lvl_ir = 0.0) {
  const double h0 = fma(c.P[0], px, fma(c.P[1], py, fma(c.P[2], pz, c.P[3])));
  const double h1 = fma(c.P[4], px, fma(c.P[5], py, fma(c.P[6], pz, c.P[7])));
  const double h2 = fma(c.P[8], px, fma(c.P[9], py, fma(c.P[10], pz, c.P[11])));
  const double r = recip(h2);
  double uu = h0 * r, vv = h1 * r;
  if (lvl_ir != 0.0) {
    // a coarser pyramid level (H, W its size): the level-0 point in that level's pixels
    uu = fma(uu + 0.5, lvl_ir, -0.5);
    vv = fma(vv + 0.5, lvl_ir, -0.5);
  }
  const double u = fmin(fmax(uu, 0.0), (double)(W - 1));
  const double v = fmin(fmax(vv, 0.0), (double)(H - 1));
  const double fu = floor(u), fv = floor(v);
  const int x0 = (int)fu, y0 = (int)fv;
  const float fa = (float)(u - fu), fb = (float)(v - fv);
  const int p00 = pix_base + y0 * W + x0;
  const int dxp = (x0 + 1 < W) ? 1 : 0;
  const int dyp = (y0 + 1 < H) ? W : 0;
  const float wa0 = (1.0f - fa) * rc, wa1 = fa * rc;
  const float wb0 = 1.0f - fb, wb1 = fb;
  t[0] = Rec{p00 * pix_bytes, wa0 * wb0};
  t[1] = Rec{(p00 + dxp) * pix_bytes, wa1 * wb0};
  t[2] = Rec{(p00 + dyp) * pix_bytes, wa0 * wb1};
  t[3] = Rec{(p00 + dyp + dxp) * pix_bytes, wa1 * wb1};
  top = p00;
  bot = dyp ? p00 + dyp : -1;      // no bottom row at the last image row (its weights are 0)
  xy = x0 | (y0 << 16);
}

// Phase A for the wave's cells: the run [lo, hi] of every (cell, virtual camera) pair, virtual camera
// vn = n L + l for camera n and pyramid level l (validity is decided at level 0, so a camera's levels share
// its run), cell-major, and the index of its first sample (sStart[npair] = the total); returns the wave's
// sample total.
template <bool ML>
__device__ int wave_runs(const CamRec* sCam, const Problem& p, const CellSet& cs, int* sRun, int* sStart,
                         int lane) {
  const int L = ML ? p.L : 1, NL = p.N * L, npair = cs.n * NL;
  const int mNL = ML ? div_magic(NL) : 0, mL = ML ? div_magic(L) : 0;
  const double z0 = p.oz + 0.5 * p.dz;
  const double Wm1 = (double)(p.W - 1), Hm1 = (double)(p.H - 1);
  int total = 0;
  for (int pb = 0; pb < npair; pb += kWave) {
    const int pi = pb + lane;
    const int cl = ML ? div_small(pi, mNL) : pi / (NL > 0 ? NL : 1);
    const int n = ML ? div_small(pi - cl * NL, mL) : pi - cl * NL;
    int lo = 1, hi = 0;
    if (pi < npair && cs.x(cl) < p.X && cs.y(cl) < p.Y) {
      const double px = p.ox + ((double)cs.x(cl) + 0.5) * p.dx;
      const double py = p.oy + ((double)cs.y(cl) + 0.5) * p.dy;
      bin_run(sCam[n], px, py, z0, p.Z, Wm1, Hm1, lo, hi);
    }
    const int len = max(hi - lo + 1, 0);
    const int incl = wave_scan_incl(len);
    if (pi < npair) {
      sRun[pi] = lo | (hi << 16);
      sStart[pi] = total + incl - len;
    }
    total += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  if (lane == 0) sStart[npair] = total;
  wave_lds_sync();
  return total;
}

// The descriptors of samples [r0, r0 + 64) of the wave: each run lane writes its bins in that range.
__device__ void emit_round(const int* sRun, const int* sStart, int npair, int N, int r0, int* sDesc, int lane) {
  for (int pb = 0; pb < npair; pb += kWave) {
    const int pi = pb + lane;
    if (pi < npair) {
      const int s0 = sStart[pi], s1 = sStart[pi + 1];
      const int lo = sRun[pi] & 0xffff;
      const int cl = pi / (N > 0 ? N : 1), n = pi - cl * N;
      const int j0 = max(s0, r0), j1 = min(s1, r0 + kRound);
      for (int j = j0; j < j1; ++j) sDesc[j - r0] = desc_pack(lo + (j - s0), n, cl);
    }
  }
}

// Phase B and the row merging for the round's samples (lane = sample, nsmp of them): the sample's four taps
// (Rec offsets = pixel index * pix_bytes) with weights / count, then rows shared with the neighbouring samples
// of the same run (same cell and camera, consecutive bins) merged: a row is kept by the first sample of the
// run that has it, which adds the weights of the following samples for as long as each of them has the row.
// On return tp holds the lane's (merged) taps, keep_top / keep_bot say which rows it keeps; sTap has been
// read by every lane (the caller may overwrite it after a wave sync).  The raw taps sit in sTap's space as
// offsets [4][kRound] then weights [4][kRound], so that lanes write and read consecutive words.
struct Sample {
  int cl, n, xy;              // cell of the wave, virtual camera (n L + level), top-left tap pixel (x | y << 16)
  bool keep_top, keep_bot;
  Rec tp[4];
};

template <bool ML>
__device__ Sample round_samples(const CamRec* sCam, const Problem& p, const CellSet& cs, const int* sRun,
                                const int* sDesc, Rec* sTap, int nsmp, int pix_bytes, int lane) {
  const int N = p.N, L = ML ? p.L : 1, NL = p.N * L;
  int* rOff = reinterpret_cast<int*>(sTap);
  float* rW = reinterpret_cast<float*>(sTap) + 4 * kRound;
  Sample sm;
  sm.cl = -1;
  sm.n = 0;
  sm.xy = 0;
  int dsc = 0, top = -1, bot = -1;
  if (lane < nsmp) {
    dsc = sDesc[lane];
    const int k = dsc & 0xffff, vn = (dsc >> 16) & 63, cl = dsc >> 22;
    const int n = ML ? div_small(vn, div_magic(L)) : vn, l = vn - n * L;
    int cnt = 0;
    for (int m = 0; m < N; ++m) {
      const int r = sRun[cl * NL + m * L];
      cnt += ((r & 0xffff) <= k && k <= (r >> 16)) ? 1 : 0;
    }
    const double px = p.ox + ((double)cs.x(cl) + 0.5) * p.dx;
    const double py = p.oy + ((double)cs.y(cl) + 0.5) * p.dy;
    const double pz = p.oz + ((double)k + 0.5) * p.dz;
    // the level mean's 1/L rides with the valid-camera count
    const float rc = __builtin_amdgcn_rcpf((float)(cnt * L));
    if (ML) {
      // level 0 is the map the run was decided on (lvl_H[0] = H, lvl_W[0] = W, lvl_off[0] = 0): no transform
      sample_taps(sCam[n], px, py, pz, rc, level_of(p.lvl_H, l), level_of(p.lvl_W, l),
                  n * p.P + level_of(p.lvl_off, l), pix_bytes, sm.tp, top, bot, sm.xy,
                  l == 0 ? 0.0 : level_of(p.lvl_inv_r, l));
    } else {
      sample_taps(sCam[n], px, py, pz, rc, p.H, p.W, n * p.P, pix_bytes, sm.tp, top, bot, sm.xy);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      rOff[t * kRound + lane] = sm.tp[t].off;
      rW[t * kRound + lane] = sm.tp[t].w;
    }
    sm.cl = cl;
    sm.n = vn;
  }
  const int run_id = dsc >> 16;
  const int prev_run = lane_prev(run_id, -1), prev_top = lane_prev(top, -2), prev_bot = lane_prev(bot, -2);
  const bool same_prev = lane > 0 && lane < nsmp && prev_run == run_id;
  bool keep_top = lane < nsmp, keep_bot = lane < nsmp && bot >= 0;
  if (same_prev) {
    keep_top = keep_top && top != prev_top && top != prev_bot;
    keep_bot = keep_bot && bot != prev_top && bot != prev_bot;
  }
  wave_lds_sync();
  if (keep_top || keep_bot) {
    Rec* tp = sm.tp;
    int ltop = keep_top ? lane + 1 : nsmp, lbot = keep_bot ? lane + 1 : nsmp;
    for (int j = lane + 1; j < nsmp; ++j) {
      const int dj = sDesc[j];
      if ((dj >> 16) != run_id) break;
      const Rec j0{rOff[j], rW[j]}, j2{rOff[2 * kRound + j], rW[2 * kRound + j]};
      const int jt = j0.off, jb = (j2.off != j0.off) ? j2.off : -1;
      const bool more_t = ltop == j && (jt == tp[0].off || jb == tp[0].off);
      const bool more_b = lbot == j && (jt == tp[2].off || jb == tp[2].off);
      if (more_t) {
        const bool from_top = jt == tp[0].off;
        tp[0].w += from_top ? j0.w : j2.w;
        tp[1].w += from_top ? rW[kRound + j] : rW[3 * kRound + j];
        ltop = j + 1;
      }
      if (more_b) {
        const bool from_top = jt == tp[2].off;
        tp[2].w += from_top ? j0.w : j2.w;
        tp[3].w += from_top ? rW[kRound + j] : rW[3 * kRound + j];
        lbot = j + 1;
      }
      if (!more_t && !more_b) break;
    }
  }
  sm.keep_top = keep_top;
  sm.keep_bot = keep_bot;
  return sm;
}

// Tap slots of one round: four per sample.
__host__ __device__ constexpr int tap_slots(int) { return 4 * kRound; }

// LDS of one wave (16-byte multiple) and of the output tile.
__host__ __device__ inline size_t wave_lds_bytes(int N, int S) {
  const size_t npair = (size_t)kCpw * N;
  const size_t b = sizeof(Rec) * tap_slots(S) + sizeof(int) * (kRound + 2 * kCpw + 2 * npair + 1);
  return (b + 15) & ~(size_t)15;
}

// U whole gather steps: the lane's tap of step u is rec[u S] (a record per slot); all U loads are issued
// before the first is used.
template <int U, int S, class Ln>
__device__ __forceinline__ void gather_steps(float* acc, const Rec* rec, __amdgpu_buffer_rsrc_t rs, int lane_off) {
  typename Ln::Raw v[U];
  float w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const Rec rr = rec[u * S];
    w[u] = rr.w;
    v[u] = Ln::load(rs, rr.off + lane_off);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) Ln::fma_into(acc, v[u], w[u]);
}

// K steps whose loads are all issued before the first is used, the last step masked: its slots past the
// cell's taps (rec + u S >= end) read outside the buffer with weight 0.
template <int K, int S, class Ln>
__device__ __forceinline__ void gather_last(float* acc, const Rec* rec, __amdgpu_buffer_rsrc_t rs, int lane_off,
                                            bool in_last) {
  typename Ln::Raw v[K];
  float w[K];
#pragma unroll
  for (int u = 0; u < K; ++u) {
    const Rec rr = rec[u * S];
    const bool in = u + 1 < K || in_last;
    w[u] = in ? rr.w : 0.f;
    v[u] = Ln::load(rs, in ? rr.off + lane_off : kOutOfRange);
  }
#pragma unroll
  for (int u = 0; u < K; ++u) Ln::fma_into(acc, v[u], w[u]);
}

// The kept taps [t, t1) of one cell into the lane's accumulators: whole groups of U steps of S taps while
// more than U steps remain, then the rest (1 to U steps, the last one masked) as one group, so that a cell
// of at most U steps costs one round trip to memory.
template <int U, int S, class Ln>
__device__ __forceinline__ void gather_cell(float* acc, const Rec* sTap, int t, int t1, int slot,
                                            __amdgpu_buffer_rsrc_t rs, int lane_off) {
  static_assert(U >= 1 && U <= 8, "one to eight steps in flight");
  for (; t + U * S < t1; t += U * S) gather_steps<U, S, Ln>(acc, sTap + t + slot, rs, lane_off);
  if (t >= t1) return;
  const int n = (t1 - t + S - 1) / S;                   // 1 .. U steps, wave-uniform
  const bool in_last = t + (n - 1) * S + slot < t1;
  const Rec* rec = sTap + t + slot;
  switch (n) {
    case 1: gather_last<1, S, Ln>(acc, rec, rs, lane_off, in_last); break;
    case 2: if constexpr (U >= 2) gather_last<2, S, Ln>(acc, rec, rs, lane_off, in_last); break;
    case 3: if constexpr (U >= 3) gather_last<3, S, Ln>(acc, rec, rs, lane_off, in_last); break;
    case 4: if constexpr (U >= 4) gather_last<4, S, Ln>(acc, rec, rs, lane_off, in_last); break;
    case 5: if constexpr (U >= 5) gather_last<5, S, Ln>(acc, rec, rs, lane_off, in_last); break;
    case 6: if constexpr (U >= 6) gather_last<6, S, Ln>(acc, rec, rs, lane_off, in_last); break;
    case 7: if constexpr (U >= 7) gather_last<7, S, Ln>(acc, rec, rs, lane_off, in_last); break;
    default: if constexpr (U >= 8) gather_last<8, S, Ln>(acc, rec, rs, lane_off, in_last); break;
  }
}

// Two channel groups of the same taps at once: K steps, each tap's record read once and both groups' loads
// (lane offsets off0, off1) issued before the first is used; the last step masked as in gather_last.
template <int K, int S, class Ln>
__device__ __forceinline__ void gather2_last(float* acc0, float* acc1, const Rec* rec, __amdgpu_buffer_rsrc_t rs,
                                             int off0, int off1, bool in_last) {
  typename Ln::Raw v0[K], v1[K];
  float w[K];
#pragma unroll
  for (int u = 0; u < K; ++u) {
    const Rec rr = rec[u * S];
    const bool in = u + 1 < K || in_last;
    w[u] = in ? rr.w : 0.f;
    v0[u] = Ln::load(rs, in ? rr.off + off0 : kOutOfRange);
    v1[u] = Ln::load(rs, in ? rr.off + off1 : kOutOfRange);
  }
#pragma unroll
  for (int u = 0; u < K; ++u) {
    Ln::fma_into(acc0, v0[u], w[u]);
    Ln::fma_into(acc1, v1[u], w[u]);
  }
}

// A cell's kept taps for two channel groups: groups of U steps, the last 1 to U steps (only the last masked) as one.
template <int U, int S, class Ln>
__device__ __forceinline__ void gather2_cell(float* acc0, float* acc1, const Rec* sTap, int t, int t1, int slot,
                                             __amdgpu_buffer_rsrc_t rs, int off0, int off1) {
  static_assert(U >= 1 && U <= 4, "one to four steps of two groups in flight");
  for (; t + U * S < t1; t += U * S) gather2_last<U, S, Ln>(acc0, acc1, sTap + t + slot, rs, off0, off1, true);
  if (t >= t1) return;
  const int n = (t1 - t + S - 1) / S;
  const bool in_last = t + (n - 1) * S + slot < t1;
  const Rec* rec = sTap + t + slot;
  switch (n) {
    case 1: gather2_last<1, S, Ln>(acc0, acc1, rec, rs, off0, off1, in_last); break;
    case 2: if constexpr (U >= 2) gather2_last<2, S, Ln>(acc0, acc1, rec, rs, off0, off1, in_last); break;
    case 3: if constexpr (U >= 3) gather2_last<3, S, Ln>(acc0, acc1, rec, rs, off0, off1, in_last); break;
    default: if constexpr (U >= 4) gather2_last<4, S, Ln>(acc0, acc1, rec, rs, off0, off1, in_last); break;
  }
}

// A cell's accumulators, complete: sum the S slots and park the channels in column `ct` of the output tile;
// the accumulators are cleared for the next cell.
template <int L, int kVec, bool kAdd = false>
__device__ __forceinline__ void flush_cell(float (&acc)[kVec], float* sOut, int ct, int lane, int Cg) {
  const int slot = lane / L, q = lane - slot * L;
  if constexpr (L == 16 && kVec % 4 == 0) {
    // reduce-scatter over the four slots: lane (row r, chunk q) ends with channel q kVec + 4 i + perm[r]
    const int rrow = lane >> 4;
#pragma unroll
    for (int i = 0; i < kVec; i += 4) {
      const float e01 = swap32_add(acc[i], acc[i + 1]);
      const float e23 = swap32_add(acc[i + 2], acc[i + 3]);
      const float s = swap16_add(e01, e23);
      const int ch = q * kVec + i + ((rrow & 1) ? 2 : 0) + (rrow >> 1);
      if (kAdd) {
        if (ch < Cg) sOut[ch * kOutLd + ct] += s;
      } else {
        sOut[ch * kOutLd + ct] = s;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      float s = row_sum_stride<L>(acc[i]);
      s = swap16_add(s, s);
      acc[i] = swap32_add(s, s);
    }
    if (slot == 0) {
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        const int ch = q * kVec + i;
        if (ch < Cg) {
          if (kAdd)
            sOut[ch * kOutLd + ct] += acc[i];
          else
            sOut[ch * kOutLd + ct] = acc[i];
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kVec; ++i) acc[i] = 0.f;
}
__host__ __device__ inline size_t out_tile_bytes(int Cg) {
  return (sizeof(float) * (size_t)(Cg > 0 ? Cg : 1) * kOutLd + 15) & ~(size_t)15;
}

// Occupancy request and gather depth (loads in flight per lane), chosen so that no layout spills:
// six waves per SIMD (80 VGPRs) up to 8 accumulated channels per lane, five (96) for 16.
template <int D, int L, bool BF16>
struct RunWaves {
  static constexpr int kVec = BF16 ? 2 * D : D;
  static constexpr bool kWide = D == 4 && L == 16;             // 16-byte lanes: 8 loads at 5 waves
  static constexpr int value = kWide ? 5 : (kVec <= 4 || (BF16 && kVec <= 8 && L == 16)) ? 6 : (kVec <= 8 ? 5 : 4);
  static constexpr int kLoads = kWide ? 8 : (D >= 3 || (BF16 && D >= 2)) ? 4 : 8;
};

// Forward.  L lanes cover one tap's channel group with D dwords each (L * D * 4 == group bytes);
// S = 64 / L taps per load instruction.  MG: the launch takes a.ngroups groups of a.Cg channels in turn over
// the same listed taps (the lanes past the last group's channels read nothing), each cell's sums added into
// the output tile at the end of its taps in a round.
template <int D, int L, bool BF16, bool ML, bool MG>
__device__ __forceinline__ void runs_fwd_body(const RunArgs& a, int blk, int nblk) {
  using Ln = Lane<D, BF16>;
  constexpr int kVec = Ln::kVec;
  constexpr int S = kWave / L;
  static_assert(S >= 4 && (S & 3) == 0, "lanes per tap divide the wave into at least four slots");
  constexpr int kU = RunWaves<D, L, BF16>::kLoads;       // loads in flight per lane in the gather
  extern __shared__ __align__(16) unsigned char smem[];
  const Problem& p = a.p;
  const int N = p.N, NL = ML ? p.N * p.L : p.N;    // cameras; virtual cameras (camera x pyramid level)
  const int npair = kCpw * NL;
  CamRec* sCam = reinterpret_cast<CamRec*>(smem);
  unsigned char* cur = smem + sizeof(CamRec) * N;
  const int wid = uniform(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  unsigned char* wbase = cur + (wave_lds_bytes(NL, S) + out_tile_bytes(a.C_launch)) * wid;
  float* sOut = reinterpret_cast<float*>(wbase + wave_lds_bytes(NL, S));  // [Cg][kOutLd] this wave's cells
  Rec* sTap = reinterpret_cast<Rec*>(wbase);                        // [tap_slots(S)] raw, then kept taps by step
  int* sDesc = reinterpret_cast<int*>(sTap + tap_slots(S));         // [kRound] the round's samples
  int* sCellLo = sDesc + kRound;                                    // [kCpw] first kept tap of the cell in the round
  int* sCellHi = sCellLo + kCpw;                                    // [kCpw] end | complete << 30, or -1
  int* sRun = sCellHi + kCpw;                                       // [npair] lo | hi << 16
  int* sStart = sRun + npair;                                       // [npair + 1] first sample index of each run

  // tile = kTileY consecutive cells of the flattened [X, Y] grid, so that every channel's part of the
  // output tile is one aligned 128-byte line when X * Y is a multiple of 32
  // Workgroup blk runs on XCD blk mod 8.  With several batch samples whose features together exceed an L2,
  // each XCD takes a contiguous range of the (sample, tile) sequence, so a sample's features stay in few L2s;
  // otherwise consecutive tiles go to consecutive XCDs, which spreads the dense tiles near the rig over all
  // of them (each XCD still works through a local window of the grid at a time).
  const int tile = a.xcd_chunks ? xcd_block(blk, nblk) : blk;
  const int b = tile / a.tiles_pb;
  const long long XY = (long long)p.X * p.Y;
  const long long f_wave = (long long)(tile - b * a.tiles_pb) * kTileY + wid * kCpw;

  stage_cameras(sCam, p, b);

  for (int e = lane; e < a.C_launch * kOutLd; e += kWave) sOut[e] = 0.f;   // cells with no sample stay 0
  const int ncell = (int)min((long long)kCpw, XY - f_wave);            // cells of this wave (may be <= 0)
  const int x_first = (int)(min(f_wave, XY) / p.Y), y_first = (int)(min(f_wave, XY) % p.Y);
  const CellSet cs{x_first, y_first, p.Y, kCpw, 0};

  // ---- phase A: runs of (cell, camera) pairs, cell-major, and their first sample indices
  const int total = wave_runs<ML>(sCam, p, cs, sRun, sStart, lane);

  // optional per-bin valid-camera counts (validation output)
  if (a.write_counts) {
    for (int e = lane; e < ncell * p.Z; e += kWave) {
      const int cl = e / p.Z, k = e - cl * p.Z;
      int cnt = 0;
      for (int n = 0; n < N; ++n) {
        const int r = sRun[cl * NL + n * (ML ? p.L : 1)];
        cnt += ((r & 0xffff) <= k && k <= (r >> 16)) ? 1 : 0;
      }
      a.counts[((size_t)b * XY + f_wave + cl) * p.Z + k] = (uint8_t)cnt;
    }
  }

  // gather lane roles
  const int slot = lane / L;
  const int q = lane - slot * L;
  const int lane_off = a.c_lo * p.elem_bytes + q * 4 * D;
  const size_t batch_bytes = (size_t)N * p.P * p.C * p.elem_bytes;
  const unsigned char* fbase = reinterpret_cast<const unsigned char*>(p.feat) + (size_t)b * batch_bytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(fbase), 0, (int)batch_bytes, 0x00020000);
  const int pix_bytes = p.C * p.elem_bytes;
  float acc[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) acc[i] = 0.f;

  for (int r0 = 0; r0 < total; r0 += kRound) {
    const int nsmp = min(kRound, total - r0);
    emit_round(sRun, sStart, npair, NL, r0, sDesc, lane);
    if (lane < kCpw) sCellHi[lane] = -1;
    wave_lds_sync();
    // ---- phase B: lane = sample; taps, count, row merging
    const Sample sm = round_samples<ML>(sCam, p, cs, sRun, sDesc, sTap, nsmp, pix_bytes, lane);
    const bool keep_top = sm.keep_top, keep_bot = sm.keep_bot;
    const int cl = sm.cl;
    const Rec* tp = sm.tp;
    const uint64_t mt = __ballot(keep_top), mb = __ballot(keep_bot);
    const int pos = 2 * (rank_below(mt) + rank_below(mb));
    const int nkept = 2 * ((keep_top ? 1 : 0) + (keep_bot ? 1 : 0));
    // per cell: its kept taps in this round, and whether its last sample is in this round
    const int next_cl = lane_next(cl, -1), prev_cl = lane_prev(cl, -1);   // every lane takes part
    const bool cell_first = lane < nsmp && (lane == 0 || prev_cl != cl);
    const bool cell_last = lane < nsmp && (lane == nsmp - 1 || next_cl != cl);
    wave_lds_sync();                                   // every lane has read the raw taps
    if (keep_top) {
      sTap[pos] = tp[0];
      sTap[pos + 1] = tp[1];
    }
    if (keep_bot) {
      sTap[pos + (keep_top ? 2 : 0)] = tp[2];
      sTap[pos + (keep_top ? 3 : 1)] = tp[3];
    }
    if (cell_first) sCellLo[cl] = pos;
    if (cell_last) {
      const bool fin = sStart[(cl + 1) * NL] <= r0 + kRound;
      sCellHi[cl] = (pos + nkept) | (fin ? (1 << 30) : 0);
    }
    wave_lds_sync();
    // ---- phase C: gather, cell by cell; a step takes S consecutive kept taps, kU steps in flight
    const int cl_first = __builtin_amdgcn_readfirstlane(cl), cl_last = __builtin_amdgcn_readlane(cl, nsmp - 1);
    if constexpr (MG) {
      // two channel groups (the launch's a.ngroups is 2): both groups' loads of a step issued together, so a cell
      // costs the round trips of one group; lanes past the second group's channels read outside the buffer (zeros)
      constexpr int kU2 = (kVec > 4 || L < 16) ? 2 : (kU > 4 ? 4 : kU);   // steps of both groups in flight, no spills
      const int g1_n = a.C_launch - a.Cg;
      const int off1 = (q * kVec < g1_n) ? lane_off + a.Cg * p.elem_bytes : 0x40000000;
      float acc1[kVec];
#pragma unroll
      for (int i = 0; i < kVec; ++i) acc1[i] = 0.f;
      for (int c = cl_first; c <= cl_last; ++c) {
        const int hi_raw = uniform(sCellHi[c]);
        if (hi_raw < 0) continue;
        const int t1 = hi_raw & ((1 << 30) - 1), t0 = uniform(sCellLo[c]);
        gather2_cell<kU2, S, Ln>(acc, acc1, sTap, t0, t1, slot, rs, lane_off, off1);
        flush_cell<L, kVec, true>(acc, sOut, c, lane, a.Cg);
        flush_cell<L, kVec, true>(acc1, sOut + a.Cg * kOutLd, c, lane, g1_n);
      }
    } else
    for (int c = cl_first; c <= cl_last; ++c) {
      const int hi_raw = uniform(sCellHi[c]);
      if (hi_raw < 0) continue;
      const int t1 = hi_raw & ((1 << 30) - 1);
      gather_cell<kU, S, Ln>(acc, sTap, uniform(sCellLo[c]), t1, slot, rs, lane_off);
      if (hi_raw >> 30) flush_cell<L, kVec>(acc, sOut, c, lane, a.Cg);
    }
    wave_lds_sync();
  }
  wave_lds_sync();

  // ---- write-out.  When the tile is 32 whole cells of one aligned 128-byte line per channel, the workgroup
  // writes it together after a barrier: each half-wave writes one channel's whole line (a lane per cell, read
  // from the four waves' LDS tiles) with non-temporal stores.  Otherwise each wave writes its own cells.
  const long long f_tile = f_wave - (long long)wid * kCpw;
  float* otile = a.out + ((size_t)b * p.out_ch + a.c_lo) * (size_t)XY + f_tile;
  const bool whole = f_tile + kTileY <= XY && (((uintptr_t)otile | ((size_t)XY * 4)) & 127) == 0;
  if (whole) {
    __syncthreads();
    const size_t wstride = wave_lds_bytes(NL, S) + out_tile_bytes(a.C_launch);
    const int cell = lane & 31, owner = cell / kCpw;
    const float* src = reinterpret_cast<const float*>(cur + wstride * owner + wave_lds_bytes(NL, S)) + (cell - owner * kCpw);
    for (int ch = 2 * wid + (lane >> 5); ch < a.C_launch; ch += 2 * kWaves)
      __builtin_nontemporal_store(src[ch * kOutLd], otile + (size_t)ch * XY + cell);
  } else if (ncell > 0) {
    const size_t c_stride = (size_t)XY;
    float* ob = a.out + ((size_t)b * p.out_ch + a.c_lo) * c_stride + f_wave;
    const bool vec = ncell == kCpw && (((uintptr_t)ob | (size_t)p.Y * 4) & 15) == 0;
    for (int e = lane; e < a.C_launch * 2; e += kWave) {
      const int ch = e >> 1, h = (e & 1) * 4;
      const float* src = sOut + ch * kOutLd + h;
      float* dst = ob + ch * c_stride + h;
      // plain stores: the L2 merges the four waves' quarters of a line before it writes the line back
      if (vec) {
        *reinterpret_cast<float4*>(dst) = make_float4(src[0], src[1], src[2], src[3]);
      } else {
        for (int k = 0; k < 4 && h + k < ncell; ++k) dst[k] = src[k];
      }
    }
  }
}

template <int D, int L, bool BF16, bool ML, bool MG>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(RunWaves<D, L, BF16>::value)))
void sampling_vt_runs_fwd(RunArgs a) {
  runs_fwd_body<D, L, BF16, ML, MG>(a, blockIdx.x, gridDim.x);
}

// The temporal forward in one launch: the Sampling-VT tiles (svt of them, padded to svt_pad, a multiple of 8,
// so that both parts keep their XCD numbering), then the previous map's resampling units, which the
// dispatcher hands out as the Sampling-VT workgroups end.
template <int D, int L, bool BF16>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(RunWaves<D, L, BF16>::value)))
void temporal_runs_fwd(RunArgs a, AlignArgs al, int svt, int svt_pad) {
  static_assert(kBlock == kAlignBlock, "one workgroup size for both parts");
  if ((int)blockIdx.x < svt_pad) {
    if ((int)blockIdx.x < svt) runs_fwd_body<D, L, BF16, false, false>(a, blockIdx.x, svt);
  } else {
    align_fwd_body(al, blockIdx.x - svt_pad, gridDim.x - svt_pad);
  }
}

// ---------------------------------------------------------------------------------------------------
// Backward (gradient with respect to the features; the map is linear in them).  One workgroup = an
// 8 x 8 block of cells and all channels (in groups of 64), eight waves, one x-row of 8 cells each.  The
// waves list their samples exactly as the forward does (runs, taps, merged rows), and every kept tap
// becomes an entry (pixel, cell, weight) of the workgroup.  A counting sort by pixel in LDS then makes
// every pixel's entries contiguous: the keys are a window per camera (the bounding box of the pixels
// that camera's taps reach), counts by integer LDS atomics, a block scan, and a scatter by atomic
// cursors.  The pixels are shared among the waves by entry count; each 16-lane group of a wave sums
// one pixel's entries, grad(cell) * weight with the grad rows read from the block's upstream-gradient
// tile in LDS (4 channels per lane), and each pixel leaves the workgroup as fp32 global atomics over
// its consecutive channels.  LDS float atomics are avoided: on this chip they are far slower than the
// integer ones.

constexpr int kBWaves = 8;
constexpr int kBThreads = kBWaves * kWave;
constexpr int kBTileX = kBWaves;           // tile rows along x, one per wave
constexpr int kBTileY = 8;                 // cells per row
constexpr int kBCells = kBTileX * kBTileY;
constexpr int kBCpw = kBTileY;             // cells per wave
constexpr int kBCg = 64;                   // channels per workgroup: 16 lanes x 4 per pixel
constexpr int kBgLd = kBCg + 4;            // upstream-gradient tile row (one cell's channels), 16-byte aligned

struct BwdRunArgs {
  Problem p;
  const float* grad;     // [B, out_ch, X, Y]
  float* dF;             // [B, N, P, C], zero-filled; atomically accumulated
  int tiles_x, tiles_y;
  int max_ent;           // entries held before a flush
  int max_keys;          // window counters per counting pass
  int xcd_chunks;        // 1: each XCD takes a contiguous range of the tiles; 0: consecutive tiles on consecutive XCDs
};

// Entry: pixel x (8 bits), row y (8 bits), camera n (6 bits), cell of the block (6 bits); and the weight.
__device__ __forceinline__ int ent_pack(int x, int y, int n, int cell) { return x | (y << 8) | (n << 16) | (cell << 22); }

// LDS carve-up of the backward (host and device agree on it).
struct BwdLds {
  size_t cam, g, box, win, misc, cnt, ent, sort, runs, total;
};
__host__ __device__ inline size_t bwd_round_bytes() {
  return (sizeof(Rec) * 4 * kRound + sizeof(int) * kRound + 15) & ~(size_t)15;
}
__host__ __device__ inline BwdLds bwd_lds(int N, int NL, int max_ent, int max_keys) {
  BwdLds l;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += (bytes + 15) & ~(size_t)15; return at; };
  l.cam = take(sizeof(CamRec) * N);
  l.g = take(sizeof(float) * kBCells * kBgLd);
  l.box = take(sizeof(int) * 4 * (NL > 0 ? NL : 1));
  l.win = take(sizeof(int) * 4 * (NL > 0 ? NL : 1));
  l.misc = take(sizeof(int) * 32);
  l.cnt = take(sizeof(int) * (max_keys + 1));
  l.ent = take(sizeof(int2) * max_ent);
  // the sorted entries share their space with the waves' per-round buffers (never live at the same time)
  const size_t sort_bytes = sizeof(int2) * max_ent, rounds = bwd_round_bytes() * kBWaves;
  l.sort = take(sort_bytes > rounds ? sort_bytes : rounds);
  l.runs = take(sizeof(int) * (2 * (size_t)kBCpw * NL + 1) * kBWaves);
  l.total = o;
  return l;
}

constexpr int kGPer = kBCells * kBCg / kBThreads;     // upstream-gradient tile values per thread

// Thread t's share of the block's upstream-gradient tile for channels [c_lo, c_lo + Cg): value i is channel
// c = e / kBCells of cell e mod kBCells, e = t + i kBThreads (zero past the group or the grid).
__device__ __forceinline__ void load_g_tile(const BwdRunArgs& a, int b, int x_tile, int y_tile, int c_lo, int Cg,
                                            float (&v)[kGPer]) {
  const Problem& p = a.p;
  const size_t c_stride = (size_t)p.X * p.Y;
  const float* gb = a.grad + ((size_t)b * p.out_ch + c_lo) * c_stride;
#pragma unroll
  for (int i = 0; i < kGPer; ++i) {
    const int e = threadIdx.x + i * kBThreads;
    const int c = e / kBCells, cl = e - c * kBCells;
    const int xx = x_tile + cl / kBTileY, yy = y_tile + cl % kBTileY;
    v[i] = (c < Cg && xx < p.X && yy < p.Y) ? __builtin_nontemporal_load(gb + c * c_stride + (size_t)xx * p.Y + yy)
                                            : 0.f;
  }
}

// Park a thread's share of a gradient tile in LDS.  Channel c = q + 16 r sits at 4 q + perm(r),
// perm = (0, 2, 1, 3), so that a lane's 16-byte read holds channels q, q + 32, q + 16, q + 48.
__device__ __forceinline__ void stage_g_tile(float* sG, const float (&v)[kGPer]) {
#pragma unroll
  for (int i = 0; i < kGPer; ++i) {
    const int e = threadIdx.x + i * kBThreads;
    const int c = e / kBCells, cl = e - c * kBCells;
    const int q = c & 15, r = c >> 4;
    sG[cl * kBgLd + 4 * q + ((r & 1) ? 2 : 0) + (r >> 1)] = v[i];
  }
}

// Sort the block's entries by pixel and add each pixel's sums to dF (one counting pass per window of
// max_keys keys), for every 64-channel group in turn: the sorted entries serve all groups.  With one group
// the caller has parked its gradient tile in LDS; with several, each group's tile is parked before its sums
// (the first group's from g0, the next group's loads issued while the current group is summed).  Called by
// the whole workgroup; ends with the entries and camera boxes cleared.
template <bool MG>
__device__ void bwd_flush(const BwdRunArgs& a, unsigned char* smem, const BwdLds& lay, int b, int x_tile,
                          int y_tile, const float (&g0)[kGPer]) {
  const Problem& p = a.p;
  const int N = p.N, NL = p.N;
  float* sG = reinterpret_cast<float*>(smem + lay.g);
  int* sBox = reinterpret_cast<int*>(smem + lay.box);
  int* sWin = reinterpret_cast<int*>(smem + lay.win);
  int* sMisc = reinterpret_cast<int*>(smem + lay.misc);
  int* sCnt = reinterpret_cast<int*>(smem + lay.cnt);
  const int2* sEnt = reinterpret_cast<const int2*>(smem + lay.ent);
  int2* sSort = reinterpret_cast<int2*>(smem + lay.sort);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);
  // the windows: lane n of wave 0 takes camera n's box, a wave scan places the windows one after another
  if (wid == 0) {
    int sz = 0, x_lo = 0, y_lo = 0, wdt = 0;
    if (lane < NL) {
      x_lo = sBox[4 * lane];
      y_lo = sBox[4 * lane + 2];
      const int x_hi = sBox[4 * lane + 1], y_hi = sBox[4 * lane + 3];
      if (x_lo <= x_hi) {
        wdt = x_hi - x_lo + 1;
        sz = wdt * (y_hi - y_lo + 1);
      }
    }
    const int incl = wave_scan_incl(sz);
    if (lane < NL) {
      sWin[4 * lane] = incl - sz;
      sWin[4 * lane + 1] = x_lo;
      sWin[4 * lane + 2] = y_lo;
      sWin[4 * lane + 3] = wdt;
    }
    if (lane == kWave - 1) sMisc[1] = incl;
  }
  __syncthreads();
  const int nkeys = sMisc[1], nent = sMisc[0];
  const size_t batch_elems = (size_t)N * p.P * p.C;
  float* db = a.dF + (size_t)b * batch_elems;
  const int ngroups = MG ? (p.C + kBCg - 1) / kBCg : 1;
  for (int k0 = 0; k0 < nkeys; k0 += a.max_keys) {
    const int kn = min(a.max_keys, nkeys - k0);
    for (int k = threadIdx.x; k <= kn; k += kBThreads) sCnt[k] = 0;
    __syncthreads();
    // counts per key of this pass
    for (int e = threadIdx.x; e < nent; e += kBThreads) {
      const int v = sEnt[e].x;
      const int x = v & 0xff, y = (v >> 8) & 0xff, n = (v >> 16) & 63;
      const int key = sWin[4 * n] + (y - sWin[4 * n + 2]) * sWin[4 * n + 3] + (x - sWin[4 * n + 1]) - k0;
      if (key >= 0 && key < kn) atomicAdd(&sCnt[key], 1);
    }
    __syncthreads();
    // exclusive scan of the counts (a chunk of keys per thread, then the chunk sums across the block); the
    // reduction's share of wave w is the keys from the first one that starts at or after w/8 of the pass's
    // entries (sMisc[24 + w]; kn where there is none)
    {
      const int per = (kn + kBThreads - 1) / kBThreads;
      const int c0 = min(kn, (int)threadIdx.x * per), c1 = min(kn, c0 + per);
      int run = 0;
      for (int k = c0; k < c1; ++k) run += sCnt[k];
      const int prev_cnt = (c0 > 0 && c0 < c1) ? sCnt[c0 - 1] : 0;
      const int incl = wave_scan_incl(run);
      if (lane == kWave - 1) sMisc[16 + wid] = incl;
      if (threadIdx.x < kBWaves) sMisc[24 + threadIdx.x] = threadIdx.x == 0 ? 0 : kn;
      __syncthreads();
      int base = incl - run, total = 0;
#pragma unroll
      for (int w = 0; w < kBWaves; ++w) {
        const int t = sMisc[16 + w];
        base += w < wid ? t : 0;
        total += t;
      }
      int prev_start = c0 > 0 ? base - prev_cnt : -1;
      for (int k = c0; k < c1; ++k) {
        const int c = sCnt[k];
        sCnt[k] = base;
#pragma unroll
        for (int w = 1; w < kBWaves; ++w) {
          const int lo = (int)(((long long)total * w) / kBWaves);
          if (prev_start < lo && base >= lo) sMisc[24 + w] = k;
        }
        prev_start = base;
        base += c;
      }
    }
    __syncthreads();
    // scatter by atomic cursors: afterwards sCnt[k] is the end of key k (and the start of key k + 1)
    for (int e = threadIdx.x; e < nent; e += kBThreads) {
      const int2 en = sEnt[e];
      const int x = en.x & 0xff, y = (en.x >> 8) & 0xff, n = (en.x >> 16) & 63;
      const int key = sWin[4 * n] + (y - sWin[4 * n + 2]) * sWin[4 * n + 3] + (x - sWin[4 * n + 1]) - k0;
      if (key >= 0 && key < kn) sSort[atomicAdd(&sCnt[key], 1)] = en;
    }
    __syncthreads();
    // per-pixel sums.  Wave w takes keys [sMisc[24 + w], sMisc[25 + w]): about an eighth of the entries.
    // Keys are taken 64 at a time, one per lane; the non-empty ones are compacted to the low lanes by a
    // forward lane permute, and each 16-lane group then sums one pixel: four pixels per step, each lane
    // holding 4 channels, its pixel's entries taken 4 at a time (grad rows from the block's tile in LDS).
    // With the tile's channel order, lane q of a group holds channels q, q + 32, q + 16 and q + 48, so the
    // pixel leaves the workgroup as four fp32 atomics over 16 consecutive channels each.  A pixel costs its
    // own entries plus a share of one step, whatever the spread of entries over pixels.
    float gn[kGPer];
    for (int gi = 0; gi < ngroups; ++gi) {
      const int c_lo = gi * kBCg, Cg = min(kBCg, p.C - c_lo);
      if (MG) {
        if (gi > 0) __syncthreads();               // the previous group's sums have read the tile
        if (gi == 0) {
          stage_g_tile(sG, g0);
        } else {
          stage_g_tile(sG, gn);
        }
        __syncthreads();
      }
      if (MG && gi + 1 < ngroups) load_g_tile(a, b, x_tile, y_tile, c_lo + kBCg, min(kBCg, p.C - c_lo - kBCg), gn);
      const int ka = sMisc[24 + wid], kb = wid + 1 < kBWaves ? sMisc[25 + wid] : kn;
      const int grp = lane >> 4, q = lane & 15;
      const float* gq = sG + 4 * q;
      for (int kc = ka; kc < kb; kc += kWave) {
        const int k = kc + lane;
        const int kend = k < kb ? sCnt[k] : 0;
        const int kbeg = (k < kb && k > 0) ? sCnt[k - 1] : 0;
        const bool some = kend > kbeg;
        const uint64_t todo = __ballot(some);
        const int nz = (int)__popcll(todo);
        if (nz == 0) continue;
        // lane j < nz holds the entry range of the j-th non-empty key (lanes with none write lane 63, which
        // is only read when all 64 keys are non-empty, and then no lane writes there but its own key's)
        const int dst = 4 * (some ? rank_below(todo) : kWave - 1);
        const int cbeg = __builtin_amdgcn_ds_permute(dst, kbeg);
        const int cend = __builtin_amdgcn_ds_permute(dst, kend);
        for (int s = 0; s < nz; s += 4) {
          // (the lane permutes run with every lane active: a lane permute reads 0 from an inactive lane)
          const int j = s + grp;
          const bool live = j < nz;
          const int jb = __builtin_amdgcn_ds_bpermute(4 * j, cbeg), je = __builtin_amdgcn_ds_bpermute(4 * j, cend);
          const int beg = live ? jb : 0;
          const int cnt = live ? je - jb : 0;
          const int last = max(cnt - 1, 0);
          // entries 4 at a time; the next four are read while the current ones' grad rows are summed
          int2 e[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) e[t] = sSort[beg + min(t, last)];
          const int v = e[0].x;
          float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
          for (int u0 = 0;;) {
            float4 gv[4];
            float w[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              gv[t] = *reinterpret_cast<const float4*>(gq + ((e[t].x >> 22) & 63) * kBgLd);
              w[t] = (u0 + t < cnt) ? __int_as_float(e[t].y) : 0.f;
            }
            // (read unconditionally, so that the waits for this step's grad rows need not cover them)
            const int un = u0 + 4;
            const bool more = __ballot(un < cnt) != 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) e[t] = sSort[beg + min(un + t, last)];
            __builtin_amdgcn_sched_barrier(0);        // keep those reads ahead of the sums
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              acc.x = fmaf(w[t], gv[t].x, acc.x);
              acc.y = fmaf(w[t], gv[t].y, acc.y);
              acc.z = fmaf(w[t], gv[t].z, acc.z);
              acc.w = fmaf(w[t], gv[t].w, acc.w);
            }
            if (!more) break;
            u0 = un;
          }
          if (cnt > 0) {
            const size_t pix = (size_t)((v >> 16) & 63) * p.P + (size_t)((v >> 8) & 0xff) * p.W + (v & 0xff);
            float* d = db + pix * p.C + c_lo + q;
            if (q < Cg) unsafeAtomicAdd(d, acc.x);
            if (q + 16 < Cg) unsafeAtomicAdd(d + 16, acc.z);
            if (q + 32 < Cg) unsafeAtomicAdd(d + 32, acc.y);
            if (q + 48 < Cg) unsafeAtomicAdd(d + 48, acc.w);
          }
        }
      }
    }
    __syncthreads();
  }
  // cleared for the next batch of entries
  for (int e = threadIdx.x; e < NL; e += kBThreads) {
    sBox[4 * e] = 0x7fffffff;
    sBox[4 * e + 1] = -1;
    sBox[4 * e + 2] = 0x7fffffff;
    sBox[4 * e + 3] = -1;
  }
  if (threadIdx.x == 0) {
    sMisc[0] = 0;
    sMisc[2] = 0x7fffffff;
    sMisc[3] = 0;
  }
  __syncthreads();
}

// MG: more than one 64-channel group.
template <bool MG>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(4))) void sampling_vt_runs_bwd(BwdRunArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Problem& p = a.p;
  const int N = p.N, NL = p.N;                      // single level: the virtual cameras are the cameras
  const BwdLds lay = bwd_lds(N, NL, a.max_ent, a.max_keys);
  CamRec* sCam = reinterpret_cast<CamRec*>(smem + lay.cam);
  int* sBox = reinterpret_cast<int*>(smem + lay.box);
  int* sMisc = reinterpret_cast<int*>(smem + lay.misc);
  int2* sEnt = reinterpret_cast<int2*>(smem + lay.ent);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);
  Rec* sTap = reinterpret_cast<Rec*>(smem + lay.sort + bwd_round_bytes() * wid);
  int* sDesc = reinterpret_cast<int*>(sTap + 4 * kRound);
  const int npair = kBCpw * NL;
  int* sRun = reinterpret_cast<int*>(smem + lay.runs) + (2 * npair + 1) * wid;
  int* sStart = sRun + npair;

  const int tile = a.xcd_chunks ? xcd_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int yt = tile % a.tiles_y;
  const int r1 = tile / a.tiles_y;
  const int xt = r1 % a.tiles_x;
  const int b = r1 / a.tiles_x;
  const int x_tile = xt * kBTileX, y_tile = yt * kBTileY;

  // boxes and the entry count start empty (visible after the camera staging's barrier)
  for (int e = threadIdx.x; e < NL; e += kBThreads) {
    sBox[4 * e] = 0x7fffffff;
    sBox[4 * e + 1] = -1;
    sBox[4 * e + 2] = 0x7fffffff;
    sBox[4 * e + 3] = -1;
  }
  if (threadIdx.x == 0) {
    sMisc[0] = 0;                    // entries reserved
    sMisc[2] = 0x7fffffff;           // first reservation that did not fit
    sMisc[3] = 0;                    // some wave stopped for want of room
  }
  stage_cameras(sCam, p, b);
  // the first channel group's upstream-gradient tile: its loads are issued once the camera table is staged
  // (vector loads complete in issue order, so loads issued earlier would hold up the staging's wait for the
  // camera entries), and it stays in registers, in flight during the listing, until the first flush needs it
  float gpre[kGPer];
  load_g_tile(a, b, x_tile, y_tile, 0, min(kBCg, p.C), gpre);
  // this wave's cells: x-row wid of the block, 8 cells; the waves go on without waiting for each other
  const CellSet cs{x_tile + wid, 0, kBTileY, kBCpw, y_tile};
  const int total = wave_runs<false>(sCam, p, cs, sRun, sStart, lane);
  bool g_staged = false;

  // The waves list their rounds without waiting for each other, each reserving room for a round's entries
  // with one LDS atomic; a round that does not fit stops its wave (it is listed again after the flush), and
  // every reservation after it fails too, so the entries written are those below the first failed one.  The
  // workgroup flushes when every wave has stopped or finished.
  int r0 = 0;
  for (;;) {
    while (r0 < total) {
      const int nsmp = min(kRound, total - r0);
      emit_round(sRun, sStart, npair, NL, r0, sDesc, lane);
      wave_lds_sync();
      const Sample sm = round_samples<false>(sCam, p, cs, sRun, sDesc, sTap, nsmp, 1, lane);
      const uint64_t mt = __ballot(sm.keep_top), mb = __ballot(sm.keep_bot);
      const int nk = 2 * ((int)__popcll(mt) + (int)__popcll(mb));
      int base = 0;
      if (lane == 0) base = atomicAdd(&sMisc[0], nk);
      base = __builtin_amdgcn_readfirstlane(base);
      if (base + nk > a.max_ent) {
        if (lane == 0) {
          atomicMin(&sMisc[2], base);
          sMisc[3] = 1;
        }
        break;
      }
      const int x0 = sm.xy & 0xffff, y0 = sm.xy >> 16;
      const int x1 = min(x0 + 1, p.W - 1), y1 = min(y0 + 1, p.H - 1);
      // each camera's pixel box grows by its samples' taps.  Along a run (one cell and camera, consecutive
      // bins, all in front of the camera) the projected u and v are monotone in the bin, so the run's taps lie
      // between those of its first and last samples: only the round's first and last sample of each run update
      // the box, by integer LDS atomics
      const int rid = sm.cl * 64 + sm.n;
      const int prev_rid = lane_prev(rid, -1), next_rid = lane_next(rid, -1);   // every lane takes part
      if (lane < nsmp && (lane == 0 || lane == nsmp - 1 || prev_rid != rid || next_rid != rid)) {
        atomicMin(&sBox[4 * sm.n], x0);
        atomicMax(&sBox[4 * sm.n + 1], x1);
        atomicMin(&sBox[4 * sm.n + 2], y0);
        atomicMax(&sBox[4 * sm.n + 3], y1);
      }
      const int pos = base + 2 * (rank_below(mt) + rank_below(mb));
      const int cell = wid * kBCpw + sm.cl;
      // the taps' pixels: top row (x0, y0), (x1, y0); bottom row one image row down
      if (sm.keep_top) {
        sEnt[pos] = make_int2(ent_pack(x0, y0, sm.n, cell), __float_as_int(sm.tp[0].w));
        sEnt[pos + 1] = make_int2(ent_pack(x1, y0, sm.n, cell), __float_as_int(sm.tp[1].w));
      }
      if (sm.keep_bot) {
        const int q = pos + (sm.keep_top ? 2 : 0);
        sEnt[q] = make_int2(ent_pack(x0, y1, sm.n, cell), __float_as_int(sm.tp[2].w));
        sEnt[q + 1] = make_int2(ent_pack(x1, y1, sm.n, cell), __float_as_int(sm.tp[3].w));
      }
      r0 += kRound;
    }
    __syncthreads();
    const bool again = sMisc[3] != 0;
    const int nent = min(sMisc[0], sMisc[2]);
    if (nent == 0 && !again) break;
    __syncthreads();                 // every wave has read the flags before the entry count changes
    if (threadIdx.x == 0) sMisc[0] = nent;
    if (!MG && !g_staged) {
      // one channel group: its tile is parked once, before the first flush (whose barriers publish it)
      stage_g_tile(reinterpret_cast<float*>(smem + lay.g), gpre);
      g_staged = true;
    }
    bwd_flush<MG>(a, smem, lay, b, x_tile, y_tile, gpre);
    if (!again) break;
  }
}

// Supported lane layouts (dwords per lane D, lanes per tap L): group bytes 4 L D.
#define FBEV_RUN_LAYOUTS(X)                                                                             \
  X(4, 16) X(8, 16) X(2, 16) X(1, 16) X(3, 16) X(4, 8) X(2, 8) X(1, 8) X(3, 8) X(4, 4) X(2, 4) X(1, 4)   \
  X(3, 4) X(4, 2) X(2, 2) X(1, 2) X(3, 2) X(4, 1) X(2, 1) X(1, 1) X(3, 1)

bool run_layout_supported(int D, int L) {
#define FBEV_IS(d, l) if (D == d && L == l) return true;
  FBEV_RUN_LAYOUTS(FBEV_IS)
#undef FBEV_IS
  return false;
}

template <bool BF16, bool ML>
bool dispatch_runs(int D, int L, const RunArgs& a, dim3 grid, size_t shmem, hipStream_t stream) {
  if (a.ngroups > 1) {
    // several channel groups in one launch: 16-byte lanes, 16 or 8 lanes per tap
    if (ML || D != 4 || (L != 16 && L != 8)) return false;
    if (L == 16)
      hipLaunchKernelGGL((sampling_vt_runs_fwd<4, 16, BF16, false, true>), grid, dim3(kBlock), shmem, stream, a);
    else
      hipLaunchKernelGGL((sampling_vt_runs_fwd<4, 8, BF16, false, true>), grid, dim3(kBlock), shmem, stream, a);
    return true;
  }
#define FBEV_CASE(d, l)                                                                                   \
  if (D == d && L == l) {                                                                                 \
    hipLaunchKernelGGL((sampling_vt_runs_fwd<d, l, BF16, ML, false>), grid, dim3(kBlock), shmem, stream, a); \
    return true;                                                                                          \
  }
  FBEV_RUN_LAYOUTS(FBEV_CASE)
#undef FBEV_CASE
  return false;
}

// Lane layout for a channel group of `bytes` per pixel: the widest L (lanes per tap) that divides it into
// a supported D (dwords per lane), trying 16-byte lanes first, then 8-byte, then 4-byte loads.  8- and
// 16-byte loads need `vec16` (16-byte aligned features and pixel rows); without it only D = 1 or 3.
void pick_run_layout(int bytes, bool vec16, int& D, int& L) {
  static const int kL[] = {16, 8, 4, 2, 1};
  for (int pass = 0; pass < 3; ++pass) {
    for (int l : kL) {
      if (bytes % (4 * l) != 0) continue;
      const int d = bytes / (4 * l);
      const bool wide = d % 4 == 0 || d % 4 == 2;            // takes a 16- or 8-byte load
      if (wide && !vec16) continue;
      if ((pass == 0 && d % 4 != 0) || (pass == 1 && d % 2 != 0)) continue;
      if (run_layout_supported(d, l)) {
        D = d;
        L = l;
        return;
      }
    }
  }
  D = 0;
  L = 0;
}

// Contiguous tile ranges per XCD (1), so that each XCD's L2 holds the features its part of the grid sees, unless
// a single sample's features exceed an L2 anyway (single level): then consecutive tiles go to consecutive
// XCDs (0), which spreads the dense tiles near the rig over all of them (400 x 400 bf16 map: 193 -> 188 us).
// On maps whose features fit an L2 the spread measured ~1% faster but fetched every feature line into all
// eight L2s (2.7x the fetched bytes on the nuScenes-shaped map), so they keep the ranges.
int xcd_chunks(const Problem& p) {
  const double feat_bytes = (double)p.B * p.N * p.P * p.C * p.elem_bytes;
  return (p.L == 1 && p.B == 1 && feat_bytes > 4.0 * (1 << 20)) ? 0 : 1;
}

}  // namespace

bool launch_forward_runs_temporal(const Problem& p, float* out, uint8_t* counts, const AlignArgs& al,
                                  hipStream_t stream, hipError_t& err) {
  // one launch of the 16-byte, 16-lane layout covering every channel, single level
  const int es = p.elem_bytes;
  if (p.L != 1 || p.vec_bytes != 16 || p.C <= 0 || p.C * es > 512) return false;
  int D = 0, L = 0;
  pick_run_layout(p.C * es, true, D, L);
  if (D != 4 || L != 16) return false;
  const long long tiles_pb = ((long long)p.X * p.Y + kTileY - 1) / kTileY;
  const long long svt = (long long)p.B * tiles_pb, svt_pad = (svt + 7) / 8 * 8;
  AlignArgs a2 = al;
  const long long align_blocks = align_grid(a2).x;
  if (svt == 0 || svt_pad + align_blocks >= (1ll << 31)) return false;
  RunArgs a;
  a.p = p;
  a.out = out;
  a.counts = counts;
  a.tiles_pb = (int)tiles_pb;
  a.xcd_chunks = xcd_chunks(p);
  a.c_lo = 0;
  a.Cg = p.C;
  a.ngroups = 1;
  a.C_launch = p.C;
  a.write_counts = counts != nullptr ? 1 : 0;
  const size_t shmem =
      sizeof(CamRec) * p.N + (out_tile_bytes(p.C) + wave_lds_bytes(p.N, kWave / L)) * kWaves;
  const dim3 grid((unsigned)(svt_pad + align_blocks)), block(kBlock);
  if (es == 2)
    hipLaunchKernelGGL((temporal_runs_fwd<4, 16, true>), grid, block, shmem, stream, a, a2, (int)svt, (int)svt_pad);
  else
    hipLaunchKernelGGL((temporal_runs_fwd<4, 16, false>), grid, block, shmem, stream, a, a2, (int)svt, (int)svt_pad);
  err = hipGetLastError();
  return true;
}

hipError_t launch_forward_runs(const Problem& p, float* out, uint8_t* counts, hipStream_t stream) {
  RunArgs a;
  a.p = p;
  a.out = out;
  a.counts = counts;
  const long long tiles_pb = ((long long)p.X * p.Y + kTileY - 1) / kTileY;
  const long long tiles = (long long)p.B * tiles_pb;
  if (tiles == 0) return hipSuccess;
  if (tiles >= (1ll << 31)) return hipErrorInvalidValue;
  a.tiles_pb = (int)tiles_pb;
  a.xcd_chunks = xcd_chunks(p);
  const int es = p.elem_bytes;
  const bool vec16 = p.vec_bytes == 16;
  // channel groups of at most 512 bytes per pixel (16 lanes x 8 dwords), each shrunk until its byte
  // size maps onto a supported lane layout
  const int max_group_ch = 512 / es;
  int c = 0;
  bool first = true;
  do {
    int Cg = p.C - c;
    if (Cg > max_group_ch) Cg = max_group_ch;
    int D = 0, L = 0;
    while (Cg > 0) {
      pick_run_layout(Cg * es, vec16, D, L);
      if (L > 0) break;
      --Cg;
    }
    if (Cg == 0) {
      if (p.C > 0) return hipErrorInvalidValue;      // unreachable for 4-byte-multiple channel rows
      D = 1;                                          // C == 0: counts only, no channel reads
      L = 16;
    }
    a.c_lo = c;
    a.Cg = Cg;
    a.ngroups = 1;
    a.C_launch = Cg;
    // the rest of the channels (at most one more group, 16-byte lanes) ride with this launch: the listing is
    // done once for both groups
    if (first && p.L == 1 && D == 4 && (L == 16 || L == 8) && vec16 && p.C > Cg && p.C <= 2 * Cg) {
      a.ngroups = 2;
      a.C_launch = p.C;
    }
    a.write_counts = (first && counts != nullptr) ? 1 : 0;
    const size_t shmem =
        sizeof(CamRec) * p.N + (out_tile_bytes(a.C_launch) + wave_lds_bytes(p.N * p.L, kWave / L)) * kWaves;
    const dim3 grid((unsigned)tiles);
    const bool ml = p.L > 1;
    const bool ok = (es == 2) ? (ml ? dispatch_runs<true, true>(D, L, a, grid, shmem, stream)
                                    : dispatch_runs<true, false>(D, L, a, grid, shmem, stream))
                              : (ml ? dispatch_runs<false, true>(D, L, a, grid, shmem, stream)
                                    : dispatch_runs<false, false>(D, L, a, grid, shmem, stream));
    if (!ok) return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    c += a.C_launch;
    first = false;
  } while (c < p.C);
  return hipSuccess;
}

bool backward_runs_supported(const Problem& p) {
  // pyramids stay on the hash-table backward: their fine level puts many distinct pixels under a tile, and
  // its 4 x 4 tiles measured faster there (142 against 416 us on the three-level workload)
  return p.L == 1 && p.W <= 256 && p.H <= 256 && p.N <= 64 && p.Z <= 65535;
}

hipError_t launch_backward_runs(const Problem& p, const float* grad_out, float* grad_feat, hipStream_t stream) {
  BwdRunArgs a;
  a.p = p;
  a.grad = grad_out;
  a.dF = grad_feat;
  a.tiles_x = (p.X + kBTileX - 1) / kBTileX;
  a.tiles_y = (p.Y + kBTileY - 1) / kBTileY;
  a.max_ent = 3072;                     // entries held before a flush (at least one round of a wave)
  a.max_keys = 2048;
  // contiguous tile ranges per XCD keep neighbouring tiles' atomics on the same pixels in one L2 (measured
  // faster on nuScenes-shaped and batched maps: 39.1 against 40.6 us, 238 against 251 us); a single sample
  // whose features exceed an L2 spreads its tiles over the XCDs instead (400 x 400 bf16 map: 830 -> 814 us)
  a.xcd_chunks = xcd_chunks(p);      // (single level here)
  const long long tiles = (long long)p.B * a.tiles_x * a.tiles_y;
  if (tiles == 0 || p.C == 0 || p.Z == 0 || p.N == 0) return hipSuccess;
  if (tiles >= (1ll << 31)) return hipErrorInvalidValue;
  const size_t shmem = bwd_lds(p.N, p.N, a.max_ent, a.max_keys).total;
  // one launch for all channels: the listing and the sort serve every 64-channel group
  if (p.C > kBCg)
    hipLaunchKernelGGL(sampling_vt_runs_bwd<true>, dim3((unsigned)tiles), dim3(kBThreads), shmem, stream, a);
  else
    hipLaunchKernelGGL(sampling_vt_runs_bwd<false>, dim3((unsigned)tiles), dim3(kBThreads), shmem, stream, a);
  return hipGetLastError();
}

}  // namespace fbev
