// Fused exact Sampling-VT for gfx950 (CDNA4): forward gather-reduction and
// its adjoint scatter.
//
// The operator is the one the FlashBEV reading notes describe ("Core Idea";
// "Method" items 1-4): each BEV output element depends only on its own cell,
// so voxel construction, projection, validity test, bilinear sampling, the
// valid-camera mean and the height sum can all run inside one kernel with
// nothing per (camera, height, channel) written to HBM.
//
// What differs from the thread-per-output design the notes describe (one
// thread per (b, x, y, c) that recomputes the geometry for every channel,
// "Method" items 2-3, flagged there as the cost that grows with C,
// "Limitation" item 2): the geometry is computed once per
// (cell, height bin, camera) and shared by all channels of the cell, and the
// expensive part of it (division, floor, weights) only for the samples that
// turn out to be in view.
//
// Geometry, per wavefront, in three phases over a batch of "items" (one item
// = one cell and a block of up to 64/N height bins):
//   A  validity: lane = (bin, camera).  The projective coordinates
//      h = P [p; 1] are affine in the voxel centre, and "depth > 0,
//      0 <= u <= W-1, 0 <= v <= H-1" equals five sign tests on h, so no
//      division is needed to decide validity.  One ballot gives every bin's
//      valid-camera count; valid lanes append a small descriptor to a
//      wave-private list in LDS.
//   B  taps: lane = one listed (valid) sample.  Divide in fp64 (reciprocal
//      estimate + two Newton steps), split into integer tap and fp32
//      fraction, and write the four (offset, weight / count) records.
//   C  gather (forward) or scatter (backward) over the records.
//
// Forward gather: lanes = (slot, q).  q selects D consecutive dwords of the
// pixel's channel group, so a tap is one coalesced channels-last read; the
// 64/L slots take different taps (and samples).  Accumulation is fp32 in
// registers; slots are summed with lane swaps, the cell's channels go to an
// LDS tile, and the tile leaves as coalesced rows of the [B,C,X,Y] output.
//
// Backward (gradient with respect to the features; the map is linear in
// them): one workgroup = a 4 x 4 block of cells and one group of <= 64
// channels.  Each tap's pixel is inserted into a workgroup-private hash table
// in LDS (integer compare-and-swap) and gets a rank within its pixel from an
// integer LDS atomic; a counting sort then makes every pixel's contributions
// contiguous.  Each 16-lane group of a wave sums one pixel's contributions
// (grad * weight / count, grad rows read from an LDS tile, 4 channels per
// lane), lane permutes transpose the four groups' sums, and each distinct
// pixel leaves the workgroup as one fp32 global atomic over its 64 consecutive
// channels.  A round ends when a wave's record buffer or the table is full;
// the remaining items go to the next round.  LDS float atomics are avoided on
// purpose: on this chip they are far slower than integer ones.

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
constexpr int kOutOfRange = 0x7ffffff0;  // buffer offset the range check turns into a zero load

// forward
constexpr int kTileY = 16;               // cells per workgroup (one x row)
constexpr int kTileLd = kTileY + 1;      // padded LDS row of the output tile
constexpr int kPend = 64;                // listed valid samples per wave (one per lane)
constexpr int kItems = 16;               // items per batch
constexpr int kRec = 4 * kPend;          // tap records per wave
constexpr int kUnroll = 4;               // loads in flight per lane and step

// backward
constexpr int kBwdTX = 4;                // tile rows along x
constexpr int kBwdTY = 4;                // tile cells along y
constexpr int kBwdCells = kBwdTX * kBwdTY;
static_assert(kBwdTX <= 4 && kBwdTY <= 8, "a cell's place in the tile packs into 2 + 3 bits");
constexpr int kBwdCg = 64;               // channels per group (one per lane)
constexpr int kBwdGLd = kBwdCg + 4;      // grad tile row: one cell's channels (16-byte aligned, padded)
constexpr int kSlotBits = 9;
constexpr int kSlots = 1 << kSlotBits;   // hash-table entries
constexpr int kFillMax = kSlots / 2;     // taken slots past which a round stops listing
constexpr int kProbes = 32;
constexpr int kOver = 16;                // per-wave queue of taps that found no table slot
constexpr int kBwdPend = 64;             // listed valid samples per wave
constexpr int kBwdRegion = 256;          // tap records per wave and round
constexpr int kRed = 8;                  // records per reduction step and lane group
static_assert(kBwdRegion >= 4 * kWave && kBwdPend == kWave, "an item of a full wave of valid samples fits an empty batch");

struct Rec {
  int off;   // forward: byte offset of the tap's pixel
  float w;   // bilinear weight / valid-camera count
};

// P_n = K_n [R_n | t_n] in double, 12 entries per camera, row-major 3x4.  Entry
// e = 12 n + 4 r + c is the dot product of row r of K_n with column c of [R_n | t_n].
struct CamEntry {
  float k[3], m[3];
};

__device__ __forceinline__ CamEntry cam_load(const float* K, const float* R, const float* t, int b, int N, int e) {
  const int n = e / 12, rc = e - n * 12, r = rc >> 2, c = rc & 3;
  const size_t bn = (size_t)b * N + n;
  CamEntry ce;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    ce.k[k] = K[bn * 9 + r * 3 + k];
    ce.m[k] = (c < 3) ? R[bn * 9 + k * 3 + c] : t[bn * 3 + k];
  }
  return ce;
}

__device__ __forceinline__ void cam_store(double* sP, int e, const CamEntry& ce) {
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < 3; ++k) acc = fma((double)ce.k[k], (double)ce.m[k], acc);
  sP[e] = acc;
}

__device__ void stage_cameras(double* sP, const float* K, const float* R, const float* t, int b, int N) {
  for (int e = threadIdx.x; e < N * 12; e += kBlock) cam_store(sP, e, cam_load(K, R, t, b, N, e));
}

// 1/x in double: hardware estimate plus two Newton steps.
__device__ __forceinline__ double recip(double x) {
  double r = __builtin_amdgcn_rcp(x);
  r = fma(r, fma(-x, r, 1.0), r);
  r = fma(r, fma(-x, r, 1.0), r);
  return r;
}

// Camera rows of one lane for phase A: h = A + Bc * py + Cc * pz with
// A = P[:,0] * px + P[:,3] (px is fixed for the item's cell).
struct LaneCam {
  double A[3], Bc[3], Cc[3];
};

__device__ __forceinline__ LaneCam lane_camera(const double* sP, int n, int N, double px) {
  LaneCam lc;
  const double* P = sP + (N > 0 ? n : 0) * 12;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    lc.A[i] = (N > 0) ? fma(P[4 * i], px, P[4 * i + 3]) : 0.0;
    lc.Bc[i] = (N > 0) ? P[4 * i + 1] : 0.0;
    lc.Cc[i] = (N > 0) ? P[4 * i + 2] : 0.0;
  }
  return lc;
}

// Phase A for one item: lane = n * zpc + zl (camera-major, so the listed
// samples of one camera come out in height order).  Validity by sign tests on
// h = P [p; 1] (SparseDriveV2 notes, "Deformable Aggregation" step 2:
// [u, v, 1]^T ~ K (R p + t); depth > 0 and the closed pixel-centre box),
// and one ballot for the valid-camera count of every bin (`bin_lanes` = the
// lanes of this lane's bin).
struct PassA {
  uint64_t mask;
  int z, cnt;
  bool writer;
};

__device__ __forceinline__ PassA validity_pass(const LaneCam& lc, double py, double oz, double dz, int zc, int zl,
                                               int n, bool lane_ok, int Z, int N, double Wm1, double Hm1,
                                               uint64_t bin_lanes) {
  PassA a;
  a.z = zc + zl;
  const bool in_range = lane_ok && a.z < Z;
  bool valid = false;
  if (in_range && N > 0) {
    const double pz = oz + ((double)a.z + 0.5) * dz;
    const double h2 = fma(lc.Cc[2], pz, fma(lc.Bc[2], py, lc.A[2]));
    const double h0 = fma(lc.Cc[0], pz, fma(lc.Bc[0], py, lc.A[0]));
    const double h1 = fma(lc.Cc[1], pz, fma(lc.Bc[1], py, lc.A[1]));
    valid = (h2 > 0.0) && (h0 >= 0.0) && (fma(Wm1, h2, -h0) >= 0.0) && (h1 >= 0.0) && (fma(Hm1, h2, -h1) >= 0.0);
  }
  a.mask = __ballot(valid);
  a.cnt = (in_range && N > 0) ? (int)__popcll(a.mask & bin_lanes) : 0;
  a.writer = in_range && n == 0;
  return a;
}

// Phase-A lane roles: lane = n * zpc + zl for N cameras and zpc = 64 / (N L)
// bins per item (an item's samples, one per feature level each, then fill at
// most one wave); bin_lanes = the lanes that hold bin zl.
struct LaneRole {
  int zpc, zl, ln;
  bool ok;
  uint64_t bin_lanes;
};

__device__ __forceinline__ LaneRole lane_role(int lane, int N, int L) {
  LaneRole r;
  const int Nn = (N > 0) ? N : 1;
  r.zpc = kWave / (Nn * L);
  r.ln = lane / r.zpc;
  r.zl = lane - r.ln * r.zpc;
  r.ok = lane < r.zpc * Nn;
  uint64_t g = 0;
  for (int n = 0; n < Nn; ++n) g |= 1ull << (n * r.zpc);
  r.bin_lanes = g << r.zl;
  return r;
}

// Merging of a listed sample's taps with those of its neighbours in the list.
// Samples of one cell and camera are listed in height order, and along the
// vertical line through a cell centre the image row of the projection is
// monotone, so consecutive samples often share a row of pixels (the same quad
// when they fall in the same pixel square).  Row r of sample s (top: taps 0-1,
// bottom: taps 2-3) is kept by s only when the previous listed sample of the
// same cell does not have that row; s then adds the weights of the row from the
// following samples, for as long as each of them has it.  Every tap's weight
// is counted exactly once, whatever the order of the rows.  raw[4 (t L + l) + k]
// holds the taps of listed sample t at feature level l (key = pixel or its byte
// offset), cell(t) = pend[t].y & 0xff; rows merge only within one level.
__device__ __forceinline__ bool row_of(const Rec* raw, int t, int key, float& wl, float& wr) {
  const Rec q0 = raw[4 * t], q2 = raw[4 * t + 2];
  if (q0.off == key) {
    wl += q0.w;
    wr += raw[4 * t + 1].w;
    return true;
  }
  if (q2.off == key) {
    wl += q2.w;
    wr += raw[4 * t + 3].w;
    return true;
  }
  return false;
}

__device__ __forceinline__ void merge_rows(const Rec* raw, const int2* pend, int s, int l, int L, int pending,
                                           Rec (&m)[4], bool& top, bool& bot) {
  const int v = s * L + l;                       // taps of (sample s, level l) start at raw[4 v]
  const int cell = pend[s].y & 0xff;
#pragma unroll
  for (int k = 0; k < 4; ++k) m[k] = raw[4 * v + k];
  top = true;
  bot = m[2].off != m[0].off;   // equal only at the clamped last row, whose weights are 0
  if (s > 0 && (pend[s - 1].y & 0xff) == cell) {
    const int pt = raw[4 * (v - L)].off, pb = raw[4 * (v - L) + 2].off;
    top = m[0].off != pt && m[0].off != pb;
    bot = bot && m[2].off != pt && m[2].off != pb;
  }
  if (top) {
    for (int t = s + 1; t < pending && (pend[t].y & 0xff) == cell; ++t)
      if (!row_of(raw, t * L + l, m[0].off, m[0].w, m[1].w)) break;
  }
  if (bot) {
    for (int t = s + 1; t < pending && (pend[t].y & 0xff) == cell; ++t)
      if (!row_of(raw, t * L + l, m[2].off, m[2].w, m[3].w)) break;
  }
}

// Phase B for one valid sample: exact division, taps and weights.
struct Taps {
  int pix[4];
  float w[4];
};

template <class T>
__device__ __forceinline__ T level_pick(const T (&a)[kMaxLevels], int l) {
  return l == 0 ? a[0] : l == 1 ? a[1] : l == 2 ? a[2] : a[3];
}

// Phase B for one valid sample at feature level `lvl`: exact division, the
// level's coordinates (u_l = (u + 1/2) / r_l - 1/2, clamped to the level's
// pixel-centre box), taps and weights; `rc` = 1 / (count * levels).
template <bool ML>
__device__ __forceinline__ Taps tap_geometry(const double* sP, int n, double px, double py, double pz, float rc,
                                             int lvl, const Problem& p) {
  const double* P = sP + n * 12;
  const double h0 = fma(P[0], px, fma(P[1], py, fma(P[2], pz, P[3])));
  const double h1 = fma(P[4], px, fma(P[5], py, fma(P[6], pz, P[7])));
  const double h2 = fma(P[8], px, fma(P[9], py, fma(P[10], pz, P[11])));
  const double r = recip(h2);
  double u = h0 * r, v = h1 * r;
  int H = p.H, W = p.W, base = n * p.P;
  if (ML && lvl > 0) {
    const double ir = level_pick(p.lvl_inv_r, lvl);
    H = level_pick(p.lvl_H, lvl);
    W = level_pick(p.lvl_W, lvl);
    base += level_pick(p.lvl_off, lvl);
    u = fma(u + 0.5, ir, -0.5);
    v = fma(v + 0.5, ir, -0.5);
  }
  // validity was decided in phase A at level 0; clamping guards rounding at the
  // edges there and is the border rule at coarser levels
  if (ML) {
    u = fmin(fmax(u, 0.0), (double)(W - 1));
    v = fmin(fmax(v, 0.0), (double)(H - 1));
  }
  const double fu = fmin(fmax(floor(u), 0.0), (double)(W - 1));
  const double fv = fmin(fmax(floor(v), 0.0), (double)(H - 1));
  const int x0 = (int)fu, y0 = (int)fv;
  const float fa = (float)(u - fu), fb = (float)(v - fv);
  Taps t;
  const int p00 = base + y0 * W + x0;
  const int dxp = (x0 + 1 < W) ? 1 : 0;      // the clamped tap has weight 0
  const int dyp = (y0 + 1 < H) ? W : 0;
  t.pix[0] = p00;
  t.pix[1] = p00 + dxp;
  t.pix[2] = p00 + dyp;
  t.pix[3] = p00 + dyp + dxp;
  const float wa0 = (1.0f - fa) * rc, wa1 = fa * rc;
  const float wb0 = 1.0f - fb, wb1 = fb;
  t.w[0] = wa0 * wb0;
  t.w[1] = wa1 * wb0;
  t.w[2] = wa0 * wb1;
  t.w[3] = wa1 * wb1;
  return t;
}

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

struct FwdArgs {
  Problem p;
  float* out;
  uint8_t* counts;
  int c_lo;          // first channel of this launch's group
  int merge;         // merge rows shared by consecutive samples of a cell (merge_rows)
  int Cg;            // channels of the group
  int tiles_y;       // ceil(Y / kTileY)
  int write_counts;
};

// Occupancy floor the forward asks the register allocator for: six waves per
// SIMD for single-level launches whose lanes accumulate at most 10 channels
// (they then fit without spilling), no constraint otherwise.
template <int D, bool BF16, bool ML>
struct FwdWaves {
  static constexpr int value = (!ML && (BF16 ? 2 * D : D) <= 10) ? 6 : 1;
};

// Forward kernel.  L lanes cover one tap's channel group with D dwords each
// (L * D * 4 == group bytes); S = 64 / L slots; T = S / 4 samples per step.
// One workgroup of the forward: tile `bid` of `nblk` (renumbered per XCD).
template <int D, int L, bool BF16, bool ML>
__device__ __forceinline__ void sampling_vt_fwd_tile(const FwdArgs& a, unsigned char* smem, int bid, int nblk) {
  using Ln = Lane<D, BF16>;
  constexpr int kVec = Ln::kVec;
  constexpr int S = kWave / L;
  static_assert(S >= 4 && (S & 3) == 0, "lanes per tap divide the wave");
  const Problem& p = a.p;
  double* sP = reinterpret_cast<double*>(smem);
  unsigned char* cur = smem + sizeof(double) * 12 * p.N;
  int2* sPend = reinterpret_cast<int2*>(cur);
  cur += sizeof(int2) * kPend * kWaves;
  Rec* sRec = reinterpret_cast<Rec*>(cur);
  cur += sizeof(Rec) * kRec * kWaves;
  int2* sItem = reinterpret_cast<int2*>(cur);
  cur += sizeof(int2) * kItems * kWaves;
  float* sOut = reinterpret_cast<float*>(cur);

  const int tile = xcd_block(bid, nblk);
  const int yt = tile % a.tiles_y;
  const int bx = tile / a.tiles_y;
  const int x = bx % p.X;
  const int b = bx / p.X;
  const int y_base = yt * kTileY;
  const int n_cells = min(kTileY, p.Y - y_base);

  stage_cameras(sP, p.K, p.R, p.t, b, p.N);
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);   // wave-uniform for the compiler too
  int2* pend = sPend + wid * kPend;
  Rec* rec = sRec + wid * kRec;
  int2* items = sItem + wid * kItems;

  // phase-A lane role
  const int nlev = ML ? p.L : 1;                  // feature levels (1 unless ML)
  const LaneRole role = lane_role(lane, p.N, nlev);
  const int zpc = role.zpc, zl = role.zl, ln = role.ln;
  const int vs = ML ? lane / nlev : lane, vl = lane - vs * nlev;  // phase-B lane role: (sample, level)
  const double px = p.ox + ((double)x + 0.5) * p.dx;
  const double Wm1 = (double)(p.W - 1), Hm1 = (double)(p.H - 1);

  // gather lane role
  const int slot = lane / L;
  const int q = lane - slot * L;
  const int lane_off = a.c_lo * p.elem_bytes + q * 4 * D;
  const size_t batch_bytes = (size_t)p.N * p.P * p.C * p.elem_bytes;
  const unsigned char* fbase = reinterpret_cast<const unsigned char*>(p.feat) + (size_t)b * batch_bytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(fbase), 0, (int)batch_bytes, 0x00020000);
  const int pix_bytes = p.C * p.elem_bytes;
  const int items_per_cell = (p.Z > 0) ? (p.Z + zpc - 1) / zpc : 1;

  // this wave's cells: wid, wid + 4, ...; items run over (cell, block of bins)
  const int my_cells = (n_cells > wid) ? (n_cells - wid + kWaves - 1) / kWaves : 0;
  const int total_items = my_cells * items_per_cell;
  float acc[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) acc[i] = 0.f;

  // phase-A camera rows of this lane's camera; re-read at the end of every batch so
  // they are not live through phases B and C
  LaneCam lc = lane_camera(sP, ln, p.N, px);
  int it = 0, ci = 0, zc = 0;                       // item counter, its cell and first bin
  while (it < total_items) {
    // ---- phase A: list the valid samples of as many items as fit (an item that
    // does not fit is left for the next batch and its validity pass repeated there)
    int pending = 0, nitems = 0;
    while (it < total_items && nitems < kItems) {
      const int cl = wid + ci * kWaves;
      const double py = p.oy + ((double)(y_base + cl) + 0.5) * p.dy;
      const PassA pa = validity_pass(lc, py, p.oz, p.dz, zc, zl, ln, role.ok, p.Z, p.N, Wm1, Hm1, role.bin_lanes);
      const int nv = (int)__popcll(pa.mask);
      if ((pending + nv) * nlev > kPend) break;
      if (a.write_counts && pa.writer)
        a.counts[(((size_t)b * p.X + x) * p.Y + y_base + cl) * p.Z + pa.z] = (uint8_t)pa.cnt;
      if ((pa.mask >> lane) & 1ull)
        pend[pending + rank_below(pa.mask)] = make_int2(pa.z, cl | (ln << 8) | (pa.cnt << 16));
      const bool last = (zc + zpc >= p.Z);
      if (lane == 0) items[nitems] = make_int2(pending | ((pending + nv) << 12) | (last ? (1 << 24) : 0), cl);
      pending += nv;
      ++nitems;
      ++it;
      zc += zpc;
      if (last) {
        zc = 0;
        ++ci;
      }
    }
    wave_lds_sync();
    // ---- phase B: taps of the listed samples (lane = (sample, feature level)),
    // then rows shared by consecutive samples of a cell merged and the kept taps
    // compacted
    const int nvirt = pending * nlev;
    if (lane < nvirt) {
      const int2 d = pend[vs];
      const int cl = d.y & 0xff, n = (d.y >> 8) & 0xff, cnt = d.y >> 16;
      const double py = p.oy + ((double)(y_base + cl) + 0.5) * p.dy;
      const double pz = p.oz + ((double)d.x + 0.5) * p.dz;
      const Taps tp = tap_geometry<ML>(sP, n, px, py, pz, __builtin_amdgcn_rcpf((float)(cnt * nlev)), vl, p);
#pragma unroll
      for (int k = 0; k < 4; ++k) rec[4 * lane + k] = Rec{tp.pix[k] * pix_bytes, tp.w[k]};
    }
    wave_lds_sync();
    {
      if (a.merge) {
        Rec m[4];
        bool top = false, bot = false;
        if (lane < nvirt) merge_rows(rec, pend, vs, vl, nlev, pending, m, top, bot);
        const uint64_t mt = __ballot(top), mb = __ballot(bot);
        const int pos = 2 * (rank_below(mt) + rank_below(mb));
        const int nrec = 2 * ((int)__popcll(mt) + (int)__popcll(mb));
        wave_lds_sync();                              // every lane has read the raw taps
        if (top) {
          rec[pos] = m[0];
          rec[pos + 1] = m[1];
        }
        if (bot) {
          rec[pos + (top ? 2 : 0)] = m[2];
          rec[pos + (top ? 3 : 1)] = m[3];
        }
        if (lane < nvirt) pend[lane].x = pos;        // first kept tap of (sample, level) number `lane`
        wave_lds_sync();
        // items: sample ranges -> ranges of kept taps
        if (lane < nitems) {
          const int i0 = items[lane].x;
          const int t0 = i0 & 0xfff, t1 = (i0 >> 12) & 0xfff;
          const int r0 = (t0 < pending) ? pend[t0 * nlev].x : nrec;
          const int r1 = (t1 < pending) ? pend[t1 * nlev].x : nrec;
          items[lane].x = r0 | (r1 << 12) | (i0 & (1 << 24));
        }
      } else if (lane < nitems) {
        // every tap kept: tap ranges are 4 L x the sample ranges
        const int i0 = items[lane].x;
        const int t0 = i0 & 0xfff, t1 = (i0 >> 12) & 0xfff;
        items[lane].x = (4 * nlev * t0) | ((4 * nlev * t1) << 12) | (i0 & (1 << 24));
      }
      wave_lds_sync();
    }
    // ---- phase C: gather, item by item; a step takes S consecutive kept taps
    for (int k = 0; k < nitems; ++k) {
      const int i0 = uniform(items[k].x);
      const int t0 = i0 & 0xfff, t1 = (i0 >> 12) & 0xfff;
      int jb = t0;
      for (; jb + S * kUnroll <= t1; jb += S * kUnroll) {
        typename Ln::Raw v[kUnroll];
        float w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const Rec rr = rec[jb + u * S + slot];
          w[u] = rr.w;
          v[u] = Ln::load(rs, rr.off + lane_off);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) Ln::fma_into(acc, v[u], w[u]);
      }
      if (jb < t1) {
        // last, partial step: taps past the item's end load nothing and weigh 0
        typename Ln::Raw v[kUnroll];
        float w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int j = jb + u * S + slot;
          const bool in = j < t1;
          const Rec rr = rec[min(j, kRec - 1)];
          w[u] = in ? rr.w : 0.f;
          v[u] = Ln::load(rs, in ? rr.off + lane_off : kOutOfRange);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) Ln::fma_into(acc, v[u], w[u]);
      }
      if ((i0 >> 24) & 1) {
        // last item of its cell: sum the slots and park the channels in the output tile
        const int cl = uniform(items[k].y);
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
          float s = row_sum_stride<L>(acc[i]);
          s = swap16_add(s, s);
          acc[i] = swap32_add(s, s);
        }
        if (slot == 0) {
#pragma unroll
          for (int i = 0; i < kVec; ++i) sOut[(q * kVec + i) * kTileLd + cl] = acc[i];
        }
#pragma unroll
        for (int i = 0; i < kVec; ++i) acc[i] = 0.f;
      }
    }
    lc = lane_camera(sP, ln, p.N, px);
    wave_lds_sync();
  }
  __syncthreads();

  // Coalesced write-out of the tile: rows of n_cells consecutive y per channel.
  {
    const size_t c_stride = (size_t)p.X * p.Y;
    float* ob = a.out + (((size_t)b * p.out_ch + a.c_lo) * p.X + x) * p.Y + y_base;
    const int yl = threadIdx.x & (kTileY - 1);
    if (yl < n_cells) {
      for (int c = threadIdx.x / kTileY; c < a.Cg; c += kBlock / kTileY)
        __builtin_nontemporal_store(sOut[c * kTileLd + yl], ob + c * c_stride + yl);
    }
  }
}

template <int D, int L, bool BF16, bool ML>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(FwdWaves<D, BF16, ML>::value)))
void sampling_vt_fwd(FwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  sampling_vt_fwd_tile<D, L, BF16, ML>(a, smem, blockIdx.x, gridDim.x);
}

// The temporal forward's last channel group in one launch: workgroups [0, tiles_pad) are the forward's
// tiles (padded to a multiple of 8, so both parts keep their XCD numbering), the rest resample the
// previous map into the output's last channels, filling the slots the forward's last tiles leave idle.
template <int D, int L, bool BF16>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(FwdWaves<D, BF16, false>::value)))
void temporal_fwd(FwdArgs a, AlignArgs al, int tiles, int tiles_pad, int align_blocks) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int v = blockIdx.x;
  if (v < tiles_pad) {
    if (v < tiles) sampling_vt_fwd_tile<D, L, BF16, false>(a, smem, v, tiles);
    return;
  }
  align_fwd_body(al, v - tiles_pad, align_blocks);
}

struct BwdArgs {
  Problem p;
  const float* grad;
  float* dF;
  int tiles_x, tiles_y;
};

// Hash-table slot of pixel `pix` (inserted if absent), or -1 when the probe
// sequence finds no room.  Integer compare-and-swap only; `fresh` is set when
// this call took a free slot.
__device__ __forceinline__ int table_slot(int* sTag, int pix, int& fresh) {
  uint32_t h = ((uint32_t)pix * 2654435761u) >> (32 - kSlotBits);
#pragma unroll 1
  for (int probe = 0; probe < kProbes; ++probe) {
    const int old = atomicCAS(&sTag[h], -1, pix);
    if (old == -1) ++fresh;
    if (old == -1 || old == pix) return (int)h;
    h = (h + 1) & (kSlots - 1);
  }
  return -1;
}

// One workgroup of the backward: tile `bid` of `nblk` (renumbered per XCD), channel group `group`.
template <bool ML>
__device__ __forceinline__ void sampling_vt_bwd_tile(const BwdArgs& a, unsigned char* smem, int bid, int nblk,
                                                     int group) {
  static_assert(kSlots == (1 << kSlotBits), "table size matches the hash width");
  static_assert(4 * kWaves * kBwdRegion < (1 << 16), "sorted positions and per-slot counts fit 16 bits");
  const Problem& p = a.p;
  double* sP = reinterpret_cast<double*>(smem);
  unsigned char* cur = smem + sizeof(double) * 12 * p.N;
  float* sG = reinterpret_cast<float*>(cur);                 // [kBwdCells][kBwdGLd] grad tile, channels last
  cur += sizeof(float) * kBwdCells * kBwdGLd;
  int2* sMeta = reinterpret_cast<int2*>(cur);                // occupied slots, compacted: (pixel, first | count << 16)
  cur += sizeof(int2) * kSlots;
  int* sTag = reinterpret_cast<int*>(cur);                   // pixel of each slot, -1 = free
  cur += sizeof(int) * kSlots;
  int* sCnt = reinterpret_cast<int*>(cur);                   // taps per slot; after the prefix sum, first sorted position
  cur += sizeof(int) * kSlots;
  int2* sPend = reinterpret_cast<int2*>(cur);                // [kWaves][kBwdPend] listed samples
  cur += sizeof(int2) * kBwdPend * kWaves;
  int2* sRegion = reinterpret_cast<int2*>(cur);              // [kWaves][kBwdRegion] (slot | rank << kSlotBits | cell << 24, w)
  cur += sizeof(int2) * kBwdRegion * kWaves;
  int2* sSorted = reinterpret_cast<int2*>(cur);              // [kWaves * kBwdRegion] (grad row offset, w)
  cur += sizeof(int2) * kBwdRegion * kWaves;
  int4* sOver = reinterpret_cast<int4*>(cur);                // [kWaves][kOver] (pix, cell, w)
  cur += sizeof(int4) * kOver * kWaves;
  int* sOverN = reinterpret_cast<int*>(cur);                 // [kWaves] queue lengths
  cur += sizeof(int) * kWaves;
  int* sFlag = reinterpret_cast<int*>(cur);                  // [0] more rounds, [1] occupied slots, [2] slots taken

  const int tile = xcd_block(bid, nblk);
  const int yt = tile % a.tiles_y;
  const int r1 = tile / a.tiles_y;
  const int xt = r1 % a.tiles_x;
  const int b = r1 / a.tiles_x;
  const int x_base = xt * kBwdTX, y_base = yt * kBwdTY;
  const int ncx = min(kBwdTX, p.X - x_base), ncy = min(kBwdTY, p.Y - y_base);
  const int n_cells = ncx * ncy;
  const int c_lo = group * kBwdCg;
  const int Cg = min(kBwdCg, p.C - c_lo);

  // grad tile [Cg][n_cells] (rows of ncy consecutive y): the loads are issued first and
  // the values parked in LDS only before the first reduction, so their latency overlaps
  // the set-up and the first listing
  constexpr int kGPer = kBwdCg * kBwdCells / kBlock;
  // camera entries first: waiting for them then leaves the grad loads in flight
  const bool cam0 = threadIdx.x < p.N * 12;
  CamEntry ce0;
  if (cam0) ce0 = cam_load(p.K, p.R, p.t, b, p.N, threadIdx.x);
  float gpre[kGPer];
  {
    const size_t c_stride = (size_t)p.X * p.Y;
    const float* gb = a.grad + (((size_t)b * p.out_ch + c_lo) * p.X + x_base) * p.Y + y_base;
#pragma unroll
    for (int i = 0; i < kGPer; ++i) {
      const int e = threadIdx.x + i * kBlock;
      const int c = e / n_cells, k = e - c * n_cells;
      const int dx = k / ncy, dy = k - dx * ncy;
      gpre[i] = (e < Cg * n_cells) ? __builtin_nontemporal_load(gb + c * c_stride + (size_t)dx * p.Y + dy) : 0.f;
    }
  }
  if (cam0) cam_store(sP, threadIdx.x, ce0);
  for (int e = threadIdx.x + kBlock; e < p.N * 12; e += kBlock) cam_store(sP, e, cam_load(p.K, p.R, p.t, b, p.N, e));
  for (int e = threadIdx.x; e < kSlots; e += kBlock) {
    sTag[e] = -1;
    sCnt[e] = 0;
  }
  if (threadIdx.x < kWaves) sOverN[threadIdx.x] = 0;
  if (threadIdx.x == 0) sFlag[2] = 0;
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);   // wave-uniform for the compiler too
  int2* region = sRegion + wid * kBwdRegion;
  int2* pend = sPend + wid * kBwdPend;
  // A multi-level backward takes the levels one after another inside each
  // workgroup (tap pass, merging and table as in a single-level backward, the
  // gradient tile and cameras staged once), and a tap's weight carries the 1/L
  // of the level mean.
  const int nlev = 1;
  const LaneRole role = lane_role(lane, p.N, 1);
  const int zpc = role.zpc, zl = role.zl, ln = role.ln;
  const int vs = lane;                               // phase-B lane role: one listed sample
  const float lmean = ML ? (float)p.L : 1.0f;
  const double Wm1 = (double)(p.W - 1), Hm1 = (double)(p.H - 1);
  const int items_per_cell = (p.Z > 0) ? (p.Z + zpc - 1) / zpc : 0;
  Rec* raw = reinterpret_cast<Rec*>(sSorted) + wid * kBwdRegion;   // raw taps while listing (sorted area is free then)
  const int my_cells = (n_cells > wid) ? (n_cells - wid + kWaves - 1) / kWaves : 0;
  const int total_items = my_cells * items_per_cell;
  const size_t batch_elems = (size_t)p.N * p.P * p.C;
  float* db = a.dF + (size_t)b * batch_elems + c_lo;
  const bool ch_lane = lane < Cg;
  // grad value of cell k, channel c of the group, from global memory (for taps that
  // found no table slot; such taps can be listed before the LDS tile is written)
  auto grad_at = [&](int k, int c) -> float {
    const int dx = k / ncy, dy = k - dx * ncy;
    return a.grad[(((size_t)b * p.out_ch + c_lo + c) * p.X + x_base + dx) * p.Y + y_base + dy];
  };

  bool grad_staged = false;
  for (int vl = 0; vl < (ML ? p.L : 1); ++vl) {      // feature level; each starts with a fresh table
  if (vl > 0) {
    for (int e = threadIdx.x; e < kSlots; e += kBlock) {
      sTag[e] = -1;
      sCnt[e] = 0;
    }
    if (threadIdx.x == 0) sFlag[2] = 0;
    __syncthreads();
  }
  int it = 0, ci = 0, zc = 0;                       // item counter, its cell and first bin
  int cdx = wid / ncy, cdy = wid - (wid / ncy) * ncy;   // the cell's place in the tile
  for (;;) {
    // ---- list taps in batches until this wave's region is full or the table is
    // loaded past kFillMax (the pixels of the remaining items go to a later round)
    int used = 0;
    // phase-A camera rows of this lane's camera, in registers for the round's items
    // (h = (P0 px + P3) + P1 py + P2 pz); re-read each round so they are not live
    // through the reduction
    double cp0[3], cp3[3];
    LaneCam lc;
    {
      const double* P = sP + (p.N > 0 ? ln : 0) * 12;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        cp0[i] = (p.N > 0) ? P[4 * i] : 0.0;
        lc.Bc[i] = (p.N > 0) ? P[4 * i + 1] : 0.0;
        lc.Cc[i] = (p.N > 0) ? P[4 * i + 2] : 0.0;
        cp3[i] = (p.N > 0) ? P[4 * i + 3] : 0.0;
      }
    }
    for (;;) {
      // phase A: valid samples of as many items as fit; an item that does not fit
      // is left for the next batch (or round) and its validity pass repeated there
      int pending = 0;
      bool round_full = uniform(sFlag[2]) > kFillMax;
      while (!round_full && it < total_items) {
        const int k = wid + ci * kWaves;               // cell within the tile
        const double px = p.ox + ((double)(x_base + cdx) + 0.5) * p.dx;
        const double py = p.oy + ((double)(y_base + cdy) + 0.5) * p.dy;
#pragma unroll
        for (int i = 0; i < 3; ++i) lc.A[i] = fma(cp0[i], px, cp3[i]);
        const PassA pa = validity_pass(lc, py, p.oz, p.dz, zc, zl, ln, role.ok, p.Z, p.N, Wm1, Hm1, role.bin_lanes);
        const int nv = (int)__popcll(pa.mask);
        if (used + 4 * nlev * (pending + nv) > kBwdRegion) {
          round_full = true;
          break;
        }
        if ((pending + nv) * nlev > kBwdPend) break;
        if ((pa.mask >> lane) & 1ull)
          pend[pending + rank_below(pa.mask)] =
              make_int2(pa.z, k | (ln << 8) | (pa.cnt << 16) | (cdx << 23) | (cdy << 25));
        pending += nv;
        ++it;
        zc += zpc;
        if (zc >= p.Z) {
          zc = 0;
          ++ci;
          cdy += kWaves;
          while (cdy >= ncy) {
            cdy -= ncy;
            ++cdx;
          }
        }
      }
      if (pending == 0) break;
      wave_lds_sync();
      // phase B: taps of the listed samples (lane = sample); rows shared by
      // consecutive samples of a cell are merged (merge_rows), and each kept tap
      // gets a table slot and a rank within it; a tap with no slot is queued for a
      // lanes-=-channels scatter (or, queue full, scattered by its lane)
      const int nvirt = pending * nlev;
      if (lane < nvirt) {
        const int2 d = pend[vs];
        const int n = (d.y >> 8) & 0xff, cnt = (d.y >> 16) & 0x7f;
        const int dx = (d.y >> 23) & 3, dy = (d.y >> 25) & 7;
        const double px = p.ox + ((double)(x_base + dx) + 0.5) * p.dx;
        const double py = p.oy + ((double)(y_base + dy) + 0.5) * p.dy;
        const double pz = p.oz + ((double)d.x + 0.5) * p.dz;
        const Taps tp = tap_geometry<ML>(sP, n, px, py, pz, __builtin_amdgcn_rcpf((float)cnt * lmean), vl, p);
#pragma unroll
        for (int t = 0; t < 4; ++t) raw[4 * lane + t] = Rec{tp.pix[t], tp.w[t]};
      }
      wave_lds_sync();
      int fresh = 0;
      int nrec;
      {
        Rec m[4];
        bool top = false, bot = false;
        if (lane < nvirt) merge_rows(raw, pend, vs, 0, 1, pending, m, top, bot);
        const uint64_t mt = __ballot(top), mb = __ballot(bot);
        const int pos = used + 2 * (rank_below(mt) + rank_below(mb));
        nrec = 2 * ((int)__popcll(mt) + (int)__popcll(mb));
        const int k = pend[min(vs, kBwdPend - 1)].y & 0xff;
        bool keep[4];
        int idx[4];
        keep[0] = keep[1] = top;
        keep[2] = keep[3] = bot;
        idx[0] = pos;
        idx[1] = pos + 1;
        idx[2] = pos + (top ? 2 : 0);
        idx[3] = pos + (top ? 3 : 1);
        // first probes of the kept taps issued together; collisions take the probe loop
        int sl4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sl4[t] = -3;
          if (keep[t]) {
            const int h = (int)(((uint32_t)m[t].off * 2654435761u) >> (32 - kSlotBits));
            const int old = atomicCAS(&sTag[h], -1, m[t].off);
            fresh += (old == -1);
            sl4[t] = (old == -1 || old == m[t].off) ? h : -2;
          }
        }
        int rk4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (sl4[t] == -2) sl4[t] = table_slot(sTag, m[t].off, fresh);
          rk4[t] = (sl4[t] >= 0) ? atomicAdd(&sCnt[sl4[t]], 1) : 0;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (!keep[t]) continue;
          const int sl = sl4[t];
          if (sl >= 0) {
            region[idx[t]] = make_int2(sl | (rk4[t] << kSlotBits) | (k << 24), __float_as_int(m[t].w));
          } else {
            region[idx[t]] = make_int2(-1, 0);
            fresh = kSlots;                            // table full: end the round after this batch
            const int qpos = atomicAdd(&sOverN[wid], 1);
            if (qpos < kOver) {
              sOver[wid * kOver + qpos] = make_int4(m[t].off, k, __float_as_int(m[t].w), 0);
            } else {
              for (int c = 0; c < Cg; ++c)
                unsafeAtomicAdd(db + (size_t)m[t].off * p.C + c, m[t].w * grad_at(k, c));
            }
          }
        }
      }
      if (fresh > 0) atomicAdd(&sFlag[2], fresh);
      used += nrec;
      wave_lds_sync();
      const int n_over = min(uniform(sOverN[wid]), kOver);
      if (n_over > 0) {
        for (int r = 0; r < n_over; ++r) {
          const int4 e = sOver[wid * kOver + r];
          if (ch_lane) unsafeAtomicAdd(db + (size_t)e.x * p.C + lane, __int_as_float(e.z) * grad_at(e.y, lane));
        }
        wave_lds_sync();
        if (lane == 0) sOverN[wid] = 0;
        wave_lds_sync();
      }
      if (round_full || it >= total_items) break;
    }
    if (!grad_staged) {
#pragma unroll
      for (int i = 0; i < kGPer; ++i) {
        const int e = threadIdx.x + i * kBlock;
        const int c = e / n_cells, k = e - c * n_cells;
        // channel c = q + 16 r of the group sits at 4 q + r, so a lane's 16-byte read holds q, q + 16, q + 32, q + 48
        if (e < Cg * n_cells) sG[k * kBwdGLd + 4 * (c & 15) + (c >> 4)] = gpre[i];
      }
      grad_staged = true;
    }
    __syncthreads();
    // ---- counting sort by slot: exclusive prefix sum of the per-slot counts and a
    // compact list of the occupied slots with their pixel and sorted range (wave 0)
    if (wid == 0) {
      constexpr int kPer = kSlots / kWave;
      int c4[kPer];
      int run = 0, mine = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        c4[i] = sCnt[lane * kPer + i];
        run += c4[i];
        mine += (c4[i] > 0);
      }
      int incl = run, inc = mine;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        const int oo = __shfl_up(inc, off);
        if (lane >= off) {
          incl += o;
          inc += oo;
        }
      }
      int first = incl - run, occ = inc - mine;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        sCnt[lane * kPer + i] = first;
        if (c4[i] > 0) sMeta[occ++] = make_int2(sTag[lane * kPer + i], first | (c4[i] << 16));
        first += c4[i];
      }
      if (lane == kWave - 1) sFlag[1] = inc;
      if (lane == 0) sFlag[0] = 0;
    }
    __syncthreads();
    for (int r = lane; r < used; r += kWave) {
      const int2 e = region[r];
      if (e.x >= 0) {
        const int sl = e.x & (kSlots - 1);
        sSorted[sCnt[sl] + ((e.x >> kSlotBits) & ((1 << (24 - kSlotBits)) - 1))] = make_int2((e.x >> 24) * kBwdGLd, e.y);
      }
    }
    if (it < total_items && lane == 0) atomicOr(&sFlag[0], 1);
    __syncthreads();
    // ---- per-pixel sums in registers, one global atomic per (pixel, channel).
    // lane = (group g, channel quad q): each 16-lane group sums one occupied slot,
    // kRed records per step, 4 channels per lane read as one 16-byte LDS load of
    // the record's grad row; four slots per wave at a time.
    {
      const int n_occ = sFlag[1];
      const int g = lane >> 4, c0 = 4 * (lane & 15);
      for (int kb = 4 * wid; kb < n_occ; kb += 4 * kWaves) {
        const int k = kb + g;
        const int2 m = (k < n_occ) ? sMeta[k] : make_int2(0, 0);
        const int first = m.y & 0xffff, count = m.y >> 16;
        const int2* srt = sSorted + first;
        const int last = max(count - 1, 0);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        // records of step j are read while step j - 8 is summed
        int2 e[kRed];
#pragma unroll
        for (int u = 0; u < kRed; ++u) e[u] = srt[min(u, last)];
        for (int j = 0; j < count; j += kRed) {
          float4 gv[kRed];
          float w[kRed];
#pragma unroll
          for (int u = 0; u < kRed; ++u) {
            gv[u] = *reinterpret_cast<const float4*>(sG + e[u].x + c0);
            w[u] = (j + u < count) ? __int_as_float(e[u].y) : 0.f;
          }
          if (j + kRed < count) {
#pragma unroll
            for (int u = 0; u < kRed; ++u) e[u] = srt[min(j + kRed + u, last)];
          }
#pragma unroll
          for (int u = 0; u < kRed; ++u) {
            acc.x = fmaf(w[u], gv[u].x, acc.x);
            acc.y = fmaf(w[u], gv[u].y, acc.y);
            acc.z = fmaf(w[u], gv[u].z, acc.z);
            acc.w = fmaf(w[u], gv[u].w, acc.w);
          }
        }
        // each group's slot leaves as four atomics over 16 consecutive channels each (lane q holds channels q,
        // q + 16, q + 32, q + 48): per instruction the wave covers 64-byte pieces of four pixels, which the
        // atomic units take faster than one pixel's 256 bytes
        if (k < n_occ && count > 0) {
          const int q = lane & 15;
          float* d = db + (size_t)m.x * p.C + q;
          if (q < Cg) unsafeAtomicAdd(d, acc.x);
          if (q + 16 < Cg) unsafeAtomicAdd(d + 16, acc.y);
          if (q + 32 < Cg) unsafeAtomicAdd(d + 32, acc.z);
          if (q + 48 < Cg) unsafeAtomicAdd(d + 48, acc.w);
        }
      }
    }
    const int more = sFlag[0];
    __syncthreads();
    if (!more) break;
    for (int e = threadIdx.x; e < kSlots; e += kBlock) {
      sTag[e] = -1;
      sCnt[e] = 0;
    }
    if (threadIdx.x == 0) sFlag[2] = 0;
    __syncthreads();
  }
  }   // levels
}

template <bool ML>
__global__ __launch_bounds__(kBlock) void sampling_vt_bwd(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  sampling_vt_bwd_tile<ML>(a, smem, blockIdx.x, gridDim.x, blockIdx.y);
}

// The temporal backward in one launch: workgroups [0, groups * tiles_pad) are the Sampling-VT backward's
// (channel group, tile) units, tiles padded to a multiple of 8 so that both parts keep their XCD
// numbering; the rest resample the previous map's gradient.  The dispatcher hands out workgroups in
// order, so the resampling units fill the slots that the backward's last tiles leave idle.
__global__ __launch_bounds__(kBlock) void temporal_bwd(BwdArgs a, AlignArgs al, int tiles, int tiles_pad,
                                                       int svt_blocks, int align_blocks) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int v = blockIdx.x;
  if (v < svt_blocks) {
    const int group = v / tiles_pad, t = v - group * tiles_pad;
    if (t < tiles) sampling_vt_bwd_tile<false>(a, smem, t, tiles, group);
    return;
  }
  align_bwd_body(al, v - svt_blocks, align_blocks);
}

__global__ void fill_zero_f32(float* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t n4 = ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) ? n / 4 : 0;
  float4* d4 = reinterpret_cast<float4*>(dst);
  for (size_t k = i; k < n4; k += stride) d4[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (size_t k = n4 * 4 + i; k < n; k += stride) dst[k] = 0.f;
}

template <int D, int L, bool BF16>
void launch_fwd_group(const FwdArgs& a, dim3 grid, size_t shmem, hipStream_t stream) {
  // single level only: this forward serves the temporal fusion; fbev_forward and the pyramids run the
  // bin-run forward (sampling_vt_runs.hip)
  hipLaunchKernelGGL((sampling_vt_fwd<D, L, BF16, false>), grid, dim3(kBlock), shmem, stream, a);
}

// Supported lane layouts (dwords per lane D, lanes per tap L).
#define FBEV_FWD_LAYOUTS(X)                                                                                  \
  X(1, 16) X(2, 16) X(3, 16) X(4, 16) X(5, 16) X(6, 16) X(8, 16) X(16, 16) X(1, 8) X(2, 8) X(3, 8) X(5, 8)     \
  X(6, 8) X(7, 8) X(1, 4) X(2, 4) X(3, 4) X(5, 4) X(6, 4) X(7, 4) X(1, 2) X(3, 2) X(5, 2) X(7, 2) X(1, 1)      \
  X(2, 1) X(3, 1) X(4, 1) X(5, 1) X(6, 1) X(7, 1)

bool layout_supported(int D, int L) {
#define FBEV_IS(d, l) if (D == d && L == l) return true;
  FBEV_FWD_LAYOUTS(FBEV_IS)
#undef FBEV_IS
  return false;
}

template <bool BF16>
bool dispatch_fwd(int D, int L, const FwdArgs& a, dim3 grid, size_t shmem, hipStream_t stream) {
#define FBEV_CASE(d, l) \
  if (D == d && L == l) { launch_fwd_group<d, l, BF16>(a, grid, shmem, stream); return true; }
  FBEV_FWD_LAYOUTS(FBEV_CASE)
#undef FBEV_CASE
  return false;
}

// Lane layout for a channel group of `bytes` per pixel: the widest L (lanes
// per tap) that divides it into a supported D (dwords per lane).
void pick_layout(int bytes, int& D, int& L) {
  static const int kL[] = {16, 8, 4, 2, 1};
  for (int l : kL) {
    if (bytes % (4 * l) != 0) continue;
    if (layout_supported(bytes / (4 * l), l)) {
      D = bytes / (4 * l);
      L = l;
      return;
    }
  }
  D = 0;
  L = 0;
}

}  // namespace

namespace {

// The temporal forward's last channel group with the resampling units appended (16 lanes per tap,
// D = 1, 2, 4 or 8 dwords per lane); false for other layouts, which then take separate launches.
template <bool BF16>
bool dispatch_temporal_fwd(int D, int L, const FwdArgs& a, const AlignArgs& al, int tiles, size_t shmem,
                           hipStream_t stream) {
  if (L != 16 || (D != 1 && D != 2 && D != 4 && D != 8)) return false;
  const int tiles_pad = (tiles + 7) / 8 * 8;
  const long long align_blocks = (long long)al.nblk * al.nchunk * al.B;
  if ((long long)tiles_pad + align_blocks >= (1ll << 31)) return false;
  const dim3 grid((unsigned)(tiles_pad + align_blocks));
  const int ab = (int)align_blocks;
  if (D == 1) hipLaunchKernelGGL((temporal_fwd<1, 16, BF16>), grid, dim3(kBlock), shmem, stream, a, al, tiles, tiles_pad, ab);
  if (D == 2) hipLaunchKernelGGL((temporal_fwd<2, 16, BF16>), grid, dim3(kBlock), shmem, stream, a, al, tiles, tiles_pad, ab);
  if (D == 4) hipLaunchKernelGGL((temporal_fwd<4, 16, BF16>), grid, dim3(kBlock), shmem, stream, a, al, tiles, tiles_pad, ab);
  if (D == 8) hipLaunchKernelGGL((temporal_fwd<8, 16, BF16>), grid, dim3(kBlock), shmem, stream, a, al, tiles, tiles_pad, ab);
  return true;
}

// The forward over all channel groups; with `al` the resampling of a temporal forward rides with the
// last group's launch when its layout allows (*al_done is set then).
hipError_t forward_groups(const Problem& p, float* out, uint8_t* counts, const AlignArgs* al, bool* al_done,
                          hipStream_t stream) {
  FwdArgs a;
  a.p = p;
  a.out = out;
  a.counts = counts;
  a.tiles_y = (p.Y + kTileY - 1) / kTileY;
  const long long tiles = (long long)p.B * p.X * a.tiles_y;
  if (tiles == 0) return hipSuccess;
  const int es = p.elem_bytes;
  // Merging shared pixel rows pays when a cell's height bins span more than one
  // item (many samples per cell and camera); with fewer bins its cost in the tap
  // pass outweighs the gather it saves.
  const int zpc = kWave / ((p.N > 0 ? p.N : 1) * p.L);
  const int merge = (p.Z > zpc) ? 1 : 0;
  // channel groups of at most 1 KiB per pixel (16 lanes x 16 dwords), each
  // shrunk until its byte size maps onto a supported lane layout
  const int max_group_ch = 1024 / es;
  int c = 0;
  bool first = true;
  do {
    int Cg = p.C - c;
    if (Cg > max_group_ch) Cg = max_group_ch;
    int D = 0, L = 0;
    while (Cg > 0) {
      pick_layout(Cg * es, D, L);
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
    a.merge = merge;
    a.write_counts = (first && counts != nullptr) ? 1 : 0;
    const size_t shmem = sizeof(double) * 12 * p.N + sizeof(int2) * kPend * kWaves + sizeof(Rec) * kRec * kWaves +
                         sizeof(int2) * kItems * kWaves + sizeof(float) * (size_t)(Cg > 0 ? Cg : 1) * kTileLd;
    const dim3 grid((unsigned)tiles);
    bool fused = false;
    if (al != nullptr && c + Cg >= p.C && tiles < (1ll << 31)) {
      fused = (es == 2) ? dispatch_temporal_fwd<true>(D, L, a, *al, (int)tiles, shmem, stream)
                        : dispatch_temporal_fwd<false>(D, L, a, *al, (int)tiles, shmem, stream);
      if (fused) *al_done = true;
    }
    const bool ok = fused || ((es == 2) ? dispatch_fwd<true>(D, L, a, grid, shmem, stream)
                                        : dispatch_fwd<false>(D, L, a, grid, shmem, stream));
    if (!ok) return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    c += Cg;
    first = false;
  } while (c < p.C);
  return hipSuccess;
}

}  // namespace

hipError_t launch_forward(const Problem& p, float* out, uint8_t* counts, hipStream_t stream) {
  return launch_forward_runs(p, out, counts, stream);
}

hipError_t launch_forward_temporal(const Problem& p, float* out, uint8_t* counts, bool current, int Cp,
                                   const float* prev, const float* ego, int c0, hipStream_t stream) {
  const bool previous = p.B > 0 && Cp > 0 && p.X > 0 && p.Y > 0;
  bool al_done = !previous;
  if (current) {
    AlignArgs al = align_args(p, Cp, ego, c0);
    al.src = prev;
    al.dst = out;
    align_grid(al);
    if (previous && p.C > 0) {
      hipError_t e = hipSuccess;
      if (launch_forward_runs_temporal(p, out, counts, al, stream, e)) return e;
    }
    const hipError_t e = forward_groups(p, p.C > 0 ? out : nullptr, counts, (previous && p.L == 1) ? &al : nullptr,
                                        &al_done, stream);
    if (e != hipSuccess) return e;
  }
  if (al_done) return hipSuccess;
  return launch_align_forward(p, prev, Cp, ego, out, c0, stream);
}

namespace {

size_t bwd_shmem(const Problem& p) {
  return sizeof(double) * 12 * p.N + sizeof(float) * kBwdCells * kBwdGLd + sizeof(int2) * kSlots +
         sizeof(int) * kSlots * 2 + sizeof(int2) * kBwdPend * kWaves + sizeof(int2) * kBwdRegion * kWaves * 2 +
         sizeof(int4) * kOver * kWaves + sizeof(int) * kWaves + sizeof(int) * 4;
}

// dL/dF := 0 on the stream (the backward then adds with atomics).
hipError_t zero_grad(const Problem& p, float* grad_feat, hipStream_t stream) {
  const size_t nF = (size_t)p.B * p.N * p.P * p.C;
  if (nF == 0) return hipSuccess;
  const size_t blocks = (nF / 4 + 255) / 256;
  const unsigned nb = (unsigned)(blocks < 2048 ? (blocks > 0 ? blocks : 1) : 2048);
  hipLaunchKernelGGL(fill_zero_f32, dim3(nb), dim3(256), 0, stream, grad_feat, nF);
  return hipGetLastError();
}

BwdArgs bwd_args(const Problem& p, const float* grad_out, float* grad_feat, long long& tiles) {
  BwdArgs a;
  a.p = p;
  a.grad = grad_out;
  a.dF = grad_feat;
  a.tiles_x = (p.X + kBwdTX - 1) / kBwdTX;
  a.tiles_y = (p.Y + kBwdTY - 1) / kBwdTY;
  tiles = (long long)p.B * a.tiles_x * a.tiles_y;
  return a;
}

}  // namespace

hipError_t launch_backward(const Problem& p, const float* grad_out, float* grad_feat, hipStream_t stream) {
  const size_t nF = (size_t)p.B * p.N * p.P * p.C;
  if (nF == 0) return hipSuccess;
  hipError_t e = zero_grad(p, grad_feat, stream);
  if (e != hipSuccess) return e;
  long long tiles = 0;
  const BwdArgs a = bwd_args(p, grad_out, grad_feat, tiles);
  if (tiles == 0 || p.Z == 0 || p.C == 0) return hipSuccess;
  if (backward_runs_supported(p)) return launch_backward_runs(p, grad_out, grad_feat, stream);
  const int groups = (p.C + kBwdCg - 1) / kBwdCg;
  const size_t shmem = bwd_shmem(p);
  if (p.L == 1) {
    hipLaunchKernelGGL(sampling_vt_bwd<false>, dim3((unsigned)tiles, (unsigned)groups), dim3(kBlock), shmem, stream,
                       a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(sampling_vt_bwd<true>, dim3((unsigned)tiles, (unsigned)groups), dim3(kBlock), shmem, stream, a);
  return hipGetLastError();
}

hipError_t launch_backward_temporal(const Problem& p, const float* grad_out, float* grad_feat, int Cp, const float* ego,
                                    float* grad_prev, int c0, hipStream_t stream) {
  const size_t nF = (size_t)p.B * p.N * p.P * p.C;
  long long tiles = 0;
  const BwdArgs a = bwd_args(p, grad_out, grad_feat, tiles);
  const bool current = nF > 0 && tiles > 0 && p.Z > 0 && p.C > 0;
  const bool previous = p.B > 0 && Cp > 0 && p.X > 0 && p.Y > 0;
  // one part alone, or a map the bin-run backward takes (faster alone than the hash-table backward fused with the
  // resampling): separate launches
  if (!current || !previous || p.L != 1 || backward_runs_supported(p)) {
    hipError_t e = launch_backward(p, grad_out, grad_feat, stream);
    if (e == hipSuccess && previous) e = launch_align_backward(p, grad_out, Cp, ego, grad_prev, c0, stream);
    return e;
  }
  hipError_t e = zero_grad(p, grad_feat, stream);
  if (e != hipSuccess) return e;
  AlignArgs al = align_args(p, Cp, ego, c0);
  al.src = grad_out;
  al.dst = grad_prev;
  const long long align_blocks = align_grid(al).x;
  const int groups = (p.C + kBwdCg - 1) / kBwdCg;
  const long long tiles_pad = (tiles + 7) / 8 * 8;
  const long long svt_blocks = groups * tiles_pad;
  if (svt_blocks + align_blocks >= (1ll << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(temporal_bwd, dim3((unsigned)(svt_blocks + align_blocks)), dim3(kBlock), bwd_shmem(p), stream, a,
                     al, (int)tiles, (int)tiles_pad, (int)svt_blocks, (int)align_blocks);
  return hipGetLastError();
}

}  // namespace fbev
