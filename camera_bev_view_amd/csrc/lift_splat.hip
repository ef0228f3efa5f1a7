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
#include "wave_ops.h"

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
constexpr int kCamD = 16;                 // doubles per camera: M rows x, y (3 each), origin x, y, BEV wedge (6)

// Per camera, in LDS: the x and y rows of M = R^T K^-1 and of the origin
// o = -R^T t, so the ego x-y of the point at camera depth d on pixel (u, v)'s
// ray is o + d M [u, v, 1] (tutorial, "Splat" step 1).
//
// Also the camera's BEV wedge, for culling whole cameras per tile: the ray
// directions (rx, ry) = M [u, v, 1] over the image form a parallelogram
// spanned by the four corner pixels' directions; when every corner is within
// 90 degrees of their mean, all of the camera's points at positive depth lie
// in the cone from o between the two angularly extreme corner directions, and
// within radius d_max * max |corner direction| of o.  Otherwise (or for depth
// bins at d <= 0) the camera is never culled.
__device__ void stage_rays(double* sCam, const float* K, const float* R, const float* t, int b, int N, int H, int W,
                           double dmin, double dmax) {
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
    double ex[4], ey[4], dot[4], crs[4], mx = 0.0, my = 0.0, r2 = 0.0;
    for (int q = 0; q < 4; ++q) {
      const double u = (q & 1) ? (double)(W - 1) : 0.0, v = (q & 2) ? (double)(H - 1) : 0.0;
      ex[q] = fma(c[0], u, fma(c[1], v, c[2]));
      ey[q] = fma(c[3], u, fma(c[4], v, c[5]));
      mx += ex[q];
      my += ey[q];
      r2 = fmax(r2, ex[q] * ex[q] + ey[q] * ey[q]);
    }
    const double rmax = sqrt(r2);
    bool ok = dmin > 0.0 && H > 0 && W > 0 && (mx != 0.0 || my != 0.0);
    for (int q = 0; q < 4; ++q) {
      dot[q] = ex[q] * mx + ey[q] * my;
      crs[q] = mx * ey[q] - my * ex[q];
      ok = ok && dot[q] > 0.0;
    }
    // order by the tangent of the angle from the mean direction, crs / dot, compared without dividing
    int qlo = 0, qhi = 0;
    for (int q = 1; q < 4; ++q) {
      if (crs[q] * dot[qlo] < crs[qlo] * dot[q]) qlo = q;
      if (crs[q] * dot[qhi] > crs[qhi] * dot[q]) qhi = q;
    }
    c[8] = ex[qlo];                   // right edge of the wedge (smallest angle)
    c[9] = ey[qlo];
    c[10] = ex[qhi];                  // left edge
    c[11] = ey[qhi];
    c[12] = dmax * rmax * (1.0 + 1e-9) + 1e-6;
    c[13] = ok ? 1.0 : 0.0;
  }
}

// Cameras with a point that may land in the footprint [xa, xb) x [ya, yb),
// widened by a margin far above rounding (one lane per camera).
__device__ __forceinline__ uint64_t visible_cameras(const double* sCam, int N, double xa, double xb, double ya,
                                                    double yb, int lane) {
  bool vis = false;
  if (lane < N) {
    const double* c = sCam + lane * kCamD;
    vis = true;
    if (c[13] != 0.0) {
      const double m = 1e-3 + 1e-9 * (fabs(xa) + fabs(xb) + fabs(ya) + fabs(yb) + fabs(c[6]) + fabs(c[7]));
      const double x0 = xa - m - c[6], x1 = xb + m - c[6], y0 = ya - m - c[7], y1 = yb + m - c[7];
      // right of the right edge: cross(aR, q) < 0 at every corner q of the box
      const double r00 = c[8] * y0 - c[9] * x0, r01 = c[8] * y1 - c[9] * x0;
      const double r10 = c[8] * y0 - c[9] * x1, r11 = c[8] * y1 - c[9] * x1;
      const bool right = fmax(fmax(r00, r01), fmax(r10, r11)) < 0.0;
      // left of the left edge: cross(q, aL) < 0 at every corner
      const double l00 = x0 * c[11] - y0 * c[10], l01 = x0 * c[11] - y1 * c[10];
      const double l10 = x1 * c[11] - y0 * c[10], l11 = x1 * c[11] - y1 * c[10];
      const bool left = fmax(fmax(l00, l01), fmax(l10, l11)) < 0.0;
      // beyond the farthest point: the box's nearest point to the origin
      const double nx = fmin(fmax(0.0, x0), x1), ny = fmin(fmax(0.0, y0), y1);
      const bool far = nx * nx + ny * ny > c[12] * c[12];
      vis = !(right || left || far);
    }
  }
  return __ballot(vis);
}

// Phase A (one pixel per lane): the candidate bins [k0, k0 + nb) of a pixel's
// ray for one tile.  The ego x-y of the ray's point at depth d is
// (ox, oy) + d (rx, ry).  Only a superset of the bins whose point lies in the
// tile is needed (membership is decided per point, below), so this runs in
// fp32: the slab edges, taken relative to the camera origin in double and
// rounded once, are pushed out by `pad`; the crossing depths, with a relative
// error of a few fp32 ulps, are widened by `slack`; and one more bin is added
// at each end.  A ray parallel to a slab gives +-inf crossings, which the
// min / max below treat as no bound (inside) or an empty interval (outside).
struct Ray {
  int k0, nb;
  double rx, ry;
};

struct TileCam {    // one (tile, camera) pair, uniform over the wave
  float ax0, ax1, ay0, ay1;   // slab edges minus the camera origin, padded
};

__device__ __forceinline__ Ray ray_candidates(const LssArgs& a, const double* c, const TileCam& tc, int u, int v) {
  Ray r;
  r.rx = fma(c[0], (double)u, fma(c[1], (double)v, c[2]));
  r.ry = fma(c[3], (double)u, fma(c[4], (double)v, c[5]));
  const float ix = __builtin_amdgcn_rcpf((float)r.rx), iy = __builtin_amdgcn_rcpf((float)r.ry);
  const float tx0 = tc.ax0 * ix, tx1 = tc.ax1 * ix, ty0 = tc.ay0 * iy, ty1 = tc.ay1 * iy;
  const float lo = fmaxf(fmaxf(a.f_dlo, fminf(tx0, tx1)), fminf(ty0, ty1)) - a.f_slack;
  const float hi = fminf(fminf(a.f_dhi, fmaxf(tx0, tx1)), fmaxf(ty0, ty1)) + a.f_slack;
  r.k0 = 0;
  r.nb = 0;
  if (lo <= hi) {
    // (lo - dmin) / dstep lies in [-1 - tiny, D + tiny] here
    const int k0 = max(0, (int)ceilf((lo - a.f_dmin) * a.f_inv_dstep) - 1);
    const int k1 = min(a.D - 1, (int)floorf((hi - a.f_dmin) * a.f_inv_dstep) + 1);
    if (k0 <= k1) {
      r.k0 = k0;
      r.nb = k1 - k0 + 1;
    }
  }
  return r;
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

constexpr int kGroup = 8;                 // candidates per phase-B group: lane = 8 * candidate + bin
constexpr int kSlots = kWave / kGroup;    // bins per candidate handled in the packed layout
constexpr int kListCap = 512;             // candidate list of one workgroup, in LDS
constexpr int kPart = kListCap / kWaves;  // each wave's part of the list; a round adds at most kWave to it
constexpr int kFlushMin = 4 * kWaves * kGroup;  // below this, keep collecting candidates before a flush

// The workgroup's candidate list in LDS, structure of arrays.
struct CandList {
  int* p;           // pixel index within the batch sample
  int* k0;          // first candidate bin
  int* nbn;         // nb | camera << 17
  double* rx;       // ray slope (ego x, y per metre of camera depth)
  double* ry;
};

// Tile-local cell of the point at camera depth d on the ray (ox, oy) + d (rx, ry),
// or -1 when the point is outside the tile or the grid: the floor of the offset
// from the grid's lower edge in cell units, in double precision; the same in
// every tile, so each point is counted by exactly one tile.
__device__ __forceinline__ int point_cell(const LssArgs& a, double ox, double oy, double rx, double ry, double d,
                                          int i0, int j0) {
  const double px = fma(d, rx, ox), py = fma(d, ry, oy);
  const double fi = floor((px - a.x_min) * a.inv_cdx), fj = floor((py - a.y_min) * a.inv_cdy);
  const double ie = (double)min(i0 + kTX, a.X), je = (double)min(j0 + kTY, a.Y);
  if (!(fi >= (double)i0 && fi < ie && fj >= (double)j0 && fj < je)) return -1;
  return ((int)fi - i0) * kTY + ((int)fj - j0);
}

// Phase B works on groups of kGroup list entries.  Packed layout: lane 8 g + j
// evaluates bin k0_g + j of the group's candidate g (one vector read of the
// list serves the whole group); lane 8 g also holds candidate g's pixel and
// bin count, which the consuming loop reads with v_readlane.  Bins past the
// first kSlots of a long crossing are taken 64 at a time when the candidate
// is consumed.
struct Group {
  int e0, cnt;            // entries [e0, min(e0 + kGroup, cnt)) of the list
  int cell, p, k, nb;     // packed lane: tile-local cell (-1: not in the tile), pixel, bin, candidate's bin count
  float al;               // packed lane: alpha of that bin
  uint64_t in, longs;     // packed lanes in the tile; bit 8 g: candidate g crosses more than kSlots bins
  float cv[kGroup];       // candidate g's context row (lane = channel)
};

__device__ __forceinline__ void fetch_group(const LssArgs& a, const double* sCam, const CandList& L, int e0, int cnt,
                                            int b, int i0, int j0, int lane, Group& G) {
  const int npix = a.N * a.H * a.W;
  const float* ctx_b = a.ctx + (size_t)b * npix * a.C + a.c_lo;
  const float* dep_b = a.depth + (size_t)b * npix * a.D;
  G.e0 = e0;
  G.cnt = cnt;
  const int e = e0 + (lane >> 3), j = lane & (kSlots - 1);
  G.cell = -1;
  G.p = 0;
  G.k = 0;
  G.nb = 0;
  G.al = 0.f;
  int n = 0;
  double rx = 0.0, ry = 0.0;
  if (e < cnt) {
    const int nbn = L.nbn[e];
    G.nb = nbn & 0x1FFFF;
    n = nbn >> 17;
    G.p = L.p[e];
    G.k = L.k0[e] + j;
    rx = L.rx[e];
    ry = L.ry[e];
  }
  // context rows first, so their latency overlaps the cell arithmetic below
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    G.cv[g] = 0.f;
    if (e0 + g < cnt && lane < a.Cg) G.cv[g] = ctx_b[(size_t)read_lane(G.p, kSlots * g) * a.C + lane];
  }
  if (j < G.nb) {
    G.al = dep_b[(size_t)G.p * a.D + G.k];
    const double* c = sCam + n * kCamD;
    G.cell = point_cell(a, c[6], c[7], rx, ry, a.dmin + (double)G.k * a.dstep, i0, j0);
  }
  G.in = __ballot(G.cell >= 0);
  G.longs = __ballot(j == 0 && G.nb > kSlots);
}

// Per-wave LDS scratch of the backward: product vectors of up to kDots points
// and the dot products of a group's packed points.
constexpr int kDots = 16;
constexpr int kPrdLd = kWave + 4;         // row stride: the 4-lane column reads below hit distinct banks
constexpr int kScratchFloats = kDots * kPrdLd + kWave;

// Dot products of the product rows [0, kDots) in sP: lane 4 r + s sums columns
// s, s + 4, ... of row r, then the four lanes of a row add up; the sums go
// to sDa[base + r].
__device__ __forceinline__ void flush_dots(float* sP, float* sDa, int base, int lane) {
  wave_lds_sync();
  const int r = lane >> 2, s = lane & 3;
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < kWave / 4; ++m) acc += sP[r * kPrdLd + s + 4 * m];
  acc = quad_sum(acc);
  if (s == 0) sDa[base + r] = acc;
  wave_lds_sync();
}

// Consume a fetched group.  Forward: tile[cell] += alpha_k c.  Backward: reads
// g = tile[cell], writes dL/dalpha_k = <c, g> and adds alpha_k g to dL/dc.
template <bool BWD>
__device__ __forceinline__ void consume_group(const LssArgs& a, const double* sCam, const CandList& L, const Group& G,
                                              float (&tile)[kCells], int b, int i0, int j0, int lane, float* scratch) {
  const int npix = a.N * a.H * a.W;
  const bool ch = lane < a.Cg;
  const float* dep_b = a.depth + (size_t)b * npix * a.D;
  const uint64_t in = G.in;
  float* sP = scratch;
  float* sDa = scratch + kDots * kPrdLd;
  int t = 0;                               // packed points consumed so far (backward)
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    if (G.e0 + g >= G.cnt) break;
    uint64_t m = (in >> (kSlots * g)) & ((1ull << kSlots) - 1);
    float dc = 0.f;
    const bool longer = (G.longs >> (kSlots * g)) & 1;
    const bool any = m != 0 || longer;
    while (m) {
      const int jj = kSlots * g + __builtin_ctzll(m);
      m &= m - 1;
      const int ce = read_lane(G.cell, jj);
      const float w = read_lane(G.al, jj);
      if (BWD) {
        const float gv = tile[ce];
        sP[(t & (kDots - 1)) * kPrdLd + lane] = G.cv[g] * gv;
        dc = fmaf(w, gv, dc);
        ++t;
        if ((t & (kDots - 1)) == 0) flush_dots(sP, sDa, t - kDots, lane);
      } else {
        tile[ce] = fmaf(w, G.cv[g], tile[ce]);
      }
    }
    if (longer) {
      // bins past the packed ones (a crossing longer than kSlots bins)
      const int e = G.e0 + g;
      const int nb = read_lane(G.nb, kSlots * g), gp = read_lane(G.p, kSlots * g);
      const int k0 = uniform(L.k0[e]), n = uniform(L.nbn[e] >> 17);
      const double* c = sCam + n * kCamD;
      const double rx = L.rx[e], ry = L.ry[e];
      for (int kb = kSlots; kb < nb; kb += kWave) {
        int ce2 = -1;
        float w2 = 0.f;
        const int k2 = k0 + kb + lane;
        if (kb + lane < nb) {
          w2 = dep_b[(size_t)gp * a.D + k2];
          ce2 = point_cell(a, c[6], c[7], rx, ry, a.dmin + (double)k2 * a.dstep, i0, j0);
        }
        uint64_t m2 = __ballot(ce2 >= 0);
        float dav2 = 0.f;
        while (m2) {
          const int jj = __builtin_ctzll(m2);
          m2 &= m2 - 1;
          const int ce = read_lane(ce2, jj);
          const float w = read_lane(w2, jj);
          if (BWD) {
            const float gv = tile[ce];
            const float da = wave_sum(G.cv[g] * gv);
            dav2 = (lane == jj) ? da : dav2;
            dc = fmaf(w, gv, dc);
          } else {
            tile[ce] = fmaf(w, G.cv[g], tile[ce]);
          }
        }
        if (BWD && ce2 >= 0) unsafeAtomicAdd(a.gdep + ((size_t)b * npix + gp) * a.D + k2, dav2);
      }
    }
    // one add per (pixel, tile) of this channel group's dL/dc
    if (BWD && any && ch && dc != 0.f) {
      const int gp = read_lane(G.p, kSlots * g);
      unsafeAtomicAdd(a.gctx + ((size_t)b * npix + gp) * a.C + a.c_lo + lane, dc);
    }
  }
  if (BWD && in != 0) {
    if (t & (kDots - 1)) flush_dots(sP, sDa, t & ~(kDots - 1), lane);
    // packed point of lane jj is the rank(jj)-th consumed; one point, one cell: the only add to its slot
    const int rank = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(in >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)in, 0u));
    if (G.cell >= 0) unsafeAtomicAdd(a.gdep + ((size_t)b * npix + G.p) * a.D + G.k, sDa[rank]);
    wave_lds_sync();
  }
}

// One tile, both directions; lanes are channels c_lo + lane.  Forward: tile[]
// is this wave's private copy of the tile in registers.  Backward: tile[]
// holds the tile's upstream gradient.  The cell index of a point is uniform
// over the wave, so tile[cell] is a register picked by a scalar index.
//
// Phase A: in each round every wave scans one 64-pixel chunk of one camera
// and appends the rays that may cross the tile to its own part of the
// workgroup's list; after the round's barrier every wave reads the four list
// lengths (published in a buffer of the round's parity, which no wave can
// overwrite before all have passed the next barrier), so all take the same
// decision.  Once enough candidates have gathered, phase B deals groups of
// kGroup entries of all four parts to the waves round-robin: a tile's work is
// spread over the four waves whichever cameras its rays come from.
template <bool BWD>
__device__ __forceinline__ void splat_tile(const LssArgs& a, const double* sCam, const CandList& L, int* sLen,
                                           float* scratch, float (&tile)[kCells], int b, int i0, int j0, int wid,
                                           int lane) {
  const double xa = a.x_min + (double)i0 * a.cdx, xb = a.x_min + (double)(i0 + kTX) * a.cdx;
  const double ya = a.y_min + (double)j0 * a.cdy, yb = a.y_min + (double)(j0 + kTY) * a.cdy;
  const int HW = a.H * a.W;
  const int nchunk = (HW + kWave - 1) / kWave;
  const uint64_t vis = visible_cameras(sCam, a.N, xa, xb, ya, yb, lane);
  const int total = __builtin_popcountll(vis) * nchunk;
  const float fiW = 1.0f / (float)a.W;
  int mine = 0;   // entries in this wave's part of the list
  for (int base = 0, round = 0; base < total; base += kWaves, ++round) {
    const int gi = base + wid;
    if (gi < total) {
      const int vi = uniform(gi / nchunk);
      uint64_t vm = vis;
      for (int x = 0; x < vi; ++x) vm &= vm - 1;
      const int n = __builtin_ctzll(vm);                        // the vi-th visible camera
      const int q = (gi - vi * nchunk) * kWave + lane;       // pixel within camera n
      const double* c = sCam + n * kCamD;
      // 1e-6 relative: far above the fp32 rounding of these differences and of the crossing depths
      const double pad = 1e-6 * (fabs(xa) + fabs(xb) + fabs(ya) + fabs(yb) + fabs(c[6]) + fabs(c[7]));
      TileCam tc;
      tc.ax0 = (float)(xa - pad - c[6]);
      tc.ax1 = (float)(xb + pad - c[6]);
      tc.ay0 = (float)(ya - pad - c[7]);
      tc.ay1 = (float)(yb + pad - c[7]);
      // v = q / W: the fp32 estimate is off by at most one, which the two steps fix
      int v = (int)(((float)q + 0.5f) * fiW);
      v -= (v * a.W > q);
      v += ((v + 1) * a.W <= q);
      const int u = q - v * a.W;
      Ray r = {0, 0, 0.0, 0.0};
      if (q < HW) r = ray_candidates(a, c, tc, u, v);
      const uint64_t mask = __ballot(r.nb > 0);
      if (r.nb > 0) {
        const int slot = wid * kPart + mine +
                         (int)__builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
        L.p[slot] = n * HW + q;
        L.k0[slot] = r.k0;
        L.nbn[slot] = r.nb | (n << 17);
        L.rx[slot] = r.rx;
        L.ry[slot] = r.ry;
      }
      mine += __builtin_popcountll(mask);
    }
    int* len = sLen + (round & 1) * kWaves;
    if (lane == 0) len[wid] = mine;
    __syncthreads();
    int cnt[kWaves], tot = 0, most = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      cnt[w] = uniform(len[w]);
      tot += cnt[w];
      most = max(most, cnt[w]);
    }
    const bool last = base + kWaves >= total;
    if (tot >= kFlushMin || most > kPart - kWave || (last && tot > 0)) {
      int first[kWaves + 1];
      first[0] = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) first[w + 1] = first[w] + (cnt[w] + kGroup - 1) / kGroup;
      // group gq of the flattened parts: part w, entries from e0 up to the part's end
      auto locate = [&](int gq, int& e0, int& end) {
        int w = 0;
#pragma unroll
        for (int x = 1; x < kWaves; ++x) w += (gq >= first[x]);
        e0 = w * kPart + (gq - first[w]) * kGroup;
        end = w * kPart + cnt[w];
      };
      const int ngroups = first[kWaves];
      for (int gq = wid; gq < ngroups; gq += kWaves) {
        Group G;
        int e0, end;
        locate(gq, e0, end);
        fetch_group(a, sCam, L, e0, end, b, i0, j0, lane, G);
        consume_group<BWD>(a, sCam, L, G, tile, b, i0, j0, lane, scratch);
      }
      __syncthreads();   // the list is read before the next appends overwrite it
      mine = 0;
    }
  }
}

__device__ __forceinline__ void decode_tile(const LssArgs& a, int& b, int& i0, int& j0) {
  const int tile = xcd_block(blockIdx.x, gridDim.x);
  const int jt = tile % a.tiles_y;
  const int r1 = tile / a.tiles_y;
  const int it = r1 % a.tiles_x;
  b = r1 / a.tiles_x;
  i0 = it * kTX;
  j0 = jt * kTY;
}

// LDS: cameras, then one region that holds the candidate list during the
// scan and (forward) the wave copies of the tile afterwards.
constexpr size_t kListBytes = (size_t)kListCap * (3 * sizeof(int) + 2 * sizeof(double));
constexpr size_t kAccBytes = (size_t)2 * kCells * kLd * sizeof(float);
constexpr size_t kRegionBytes = kListBytes > kAccBytes ? kListBytes : kAccBytes;
constexpr size_t kHeadBytes = 2 * kWaves * sizeof(int);           // 32: keeps the region 16-byte aligned
static_assert(kListBytes >= (size_t)kCells * kLd * sizeof(float), "the backward stages its gradient tile in the list region");
constexpr size_t kScratchBytes = (size_t)kWaves * kScratchFloats * sizeof(float);

__device__ __forceinline__ CandList carve_list(unsigned char* region) {
  CandList L;
  L.rx = reinterpret_cast<double*>(region);
  L.ry = L.rx + kListCap;
  L.p = reinterpret_cast<int*>(L.ry + kListCap);
  L.k0 = L.p + kListCap;
  L.nbn = L.k0 + kListCap;
  return L;
}

__global__ __launch_bounds__(kBlock) void lift_splat_fwd(LssArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* sLen = reinterpret_cast<int*>(smem);                         // [2][kWaves] list part lengths
  unsigned char* region = smem + kHeadBytes;
  double* sCam = reinterpret_cast<double*>(region + kRegionBytes);
  const CandList L = carve_list(region);
  int b, i0, j0;
  decode_tile(a, b, i0, j0);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);

  stage_rays(sCam, a.K, a.R, a.t, b, a.N, a.H, a.W, a.dmin, a.dmin + (double)(a.D - 1) * a.dstep);
  __syncthreads();

  float tile[kCells];
#pragma unroll
  for (int e = 0; e < kCells; ++e) tile[e] = 0.f;
  splat_tile<false>(a, sCam, L, sLen, nullptr, tile, b, i0, j0, wid, lane);
  // Sum the four wave copies in two steps through two LDS copies of the tile
  // (every flush ends with a barrier, so the list region is free again):
  // waves 0 and 1 store theirs, then waves 2 and 3 add theirs in.
  float* sAcc = reinterpret_cast<float*>(region);                    // [2][kCells][kLd]
  float* acc = sAcc + (wid & 1) * kCells * kLd;
  if (wid < 2) {
#pragma unroll
    for (int e = 0; e < kCells; ++e) acc[e * kLd + lane] = tile[e];
  }
  __syncthreads();
  if (wid >= 2) {
#pragma unroll
    for (int e = 0; e < kCells; ++e) acc[e * kLd + lane] += tile[e];
  }
  __syncthreads();

  // store the tile: kTY consecutive y per (channel, x)
  const size_t cs = (size_t)a.X * a.Y;
  float* ob = a.out + ((size_t)b * a.C + a.c_lo) * cs;
  for (int e = threadIdx.x; e < a.Cg * kCells; e += kBlock) {
    const int c = e / kCells, cell = e - c * kCells;
    const int ci = cell / kTY, cj = cell - ci * kTY;
    if (i0 + ci < a.X && j0 + cj < a.Y) {
      const float s = sAcc[cell * kLd + c] + sAcc[(kCells + cell) * kLd + c];
      __builtin_nontemporal_store(s, ob + c * cs + (size_t)(i0 + ci) * a.Y + j0 + cj);
    }
  }
}

__global__ __launch_bounds__(kBlock) void lift_splat_bwd(LssArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* sLen = reinterpret_cast<int*>(smem);
  unsigned char* region = smem + kHeadBytes;                         // kListBytes: no wave copies of the tile here
  float* sScr = reinterpret_cast<float*>(region + kListBytes);       // [kWaves][kScratchFloats]
  double* sCam = reinterpret_cast<double*>(region + kListBytes + kScratchBytes);
  const CandList L = carve_list(region);
  int b, i0, j0;
  decode_tile(a, b, i0, j0);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);

  // the tile's upstream gradient, staged through the list region with
  // coalesced row reads, then one register per cell in every wave (channels
  // past Cg and cells past the grid read as 0)
  float* sG = reinterpret_cast<float*>(region);                      // [kCells][kLd]
  {
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
  stage_rays(sCam, a.K, a.R, a.t, b, a.N, a.H, a.W, a.dmin, a.dmin + (double)(a.D - 1) * a.dstep);
  __syncthreads();
  float tile[kCells];
#pragma unroll
  for (int e = 0; e < kCells; ++e) tile[e] = sG[e * kLd + lane];
  __syncthreads();   // the region becomes the candidate list
  splat_tile<true>(a, sCam, L, sLen, sScr + wid * kScratchFloats, tile, b, i0, j0, wid, lane);
}

// Zeroes two buffers in one launch (the backward's two gradients): element k < n0 of the first, then
// the n1 elements of the second.
__global__ void lss_fill_zero(float* __restrict__ d0, size_t n0, float* __restrict__ d1, size_t n1) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n0 + n1; k += stride) {
    if (k < n0)
      d0[k] = 0.f;
    else
      d1[k - n0] = 0.f;
  }
}

hipError_t fill(float* d0, size_t n0, float* d1, size_t n1, hipStream_t stream) {
  const size_t n = n0 + n1;
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  const unsigned nb = (unsigned)(blocks < 2048 ? blocks : 2048);
  hipLaunchKernelGGL(lss_fill_zero, dim3(nb), dim3(256), 0, stream, d0, n0, d1, n1);
  return hipGetLastError();
}

}  // namespace

// fp32 constants of the candidate test (see ray_candidates)
void set_scan_constants(LssArgs& a) {
  const double dlo = a.dmin - a.dstep, dhi = a.dmin + (double)a.D * a.dstep;
  a.f_dlo = (float)dlo;
  a.f_dhi = (float)dhi;
  a.f_dmin = (float)a.dmin;
  a.f_inv_dstep = (float)(1.0 / a.dstep);
  // 1e-6 relative (about 17 fp32 ulps) of the largest depth the interval can hold
  a.f_slack = (float)(1e-6 * (fabs(dlo) + fabs(dhi)) + 1e-9);
  a.inv_cdx = 1.0 / a.cdx;
  a.inv_cdy = 1.0 / a.cdy;
}

hipError_t launch_lss_forward(LssArgs a, hipStream_t stream) {
  set_scan_constants(a);
  a.tiles_x = (a.X + kTX - 1) / kTX;
  a.tiles_y = (a.Y + kTY - 1) / kTY;
  const long long tiles = (long long)a.B * a.tiles_x * a.tiles_y;
  if (tiles == 0 || a.C == 0) return hipSuccess;
  const size_t shmem = kHeadBytes + kRegionBytes + sizeof(double) * kCamD * a.N;
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
  hipError_t e = fill(a.gdep, a.gdep != nullptr ? npix * a.D : 0, a.gctx, a.gctx != nullptr ? npix * a.C : 0, stream);
  if (e != hipSuccess) return e;
  set_scan_constants(a);
  a.tiles_x = (a.X + kTX - 1) / kTX;
  a.tiles_y = (a.Y + kTY - 1) / kTY;
  const long long tiles = (long long)a.B * a.tiles_x * a.tiles_y;
  // with no depth bins or no channels both gradients are zero
  if (a.gdep == nullptr || a.gctx == nullptr || tiles == 0 || a.C == 0 || a.D == 0 || npix == 0) return hipSuccess;
  const size_t shmem = kHeadBytes + kListBytes + kScratchBytes + sizeof(double) * kCamD * a.N;
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
