// Bilinear resampling of the previous frame's BEV map into the current ego
// frame, and its adjoint: the device bodies and launch geometry shared by the
// temporal kernels and by the fused temporal backward (which appends these
// units to the Sampling-VT backward's tiles in one launch).  The operator is
// described with the kernels that launch it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "wave_ops.h"

namespace fbev {

constexpr int kAlignBlock = 256;         // threads per workgroup of the resampling units
constexpr int kAlignChunk = 8;                // channels per thread
constexpr int kAlignMaxWin = 33;              // candidate cells per axis in the backward, at most

struct AlignArgs {
  const float* src;        // forward: prev [B, Cp, X, Y]; backward: grad [B, out_ch, X, Y]
  const float* ego;        // [B, 2, 3]
  float* dst;              // forward: out [B, out_ch, X, Y]; backward: dprev [B, Cp, X, Y]
  int B, X, Y, Cp, out_ch, c0;
  int nblk, nchunk;        // cell blocks per channel chunk, channel chunks
  double ox, dx, oy, dy;
};

// The planar motion of batch sample b in index units: i' = m00 i + m01 j + m02,
// j' = m10 i + m11 j + m12 (i, j integer cell indices of the current grid).
struct IndexMap {
  double m[6];
};

__device__ __forceinline__ IndexMap index_map(const AlignArgs& a, int b) {
  const float* A = a.ego + (size_t)b * 6;
  const double a00 = A[0], a01 = A[1], a02 = A[2], a10 = A[3], a11 = A[4], a12 = A[5];
  // x = ox + (i + 1/2) dx, y = oy + (j + 1/2) dy;  i' = (x' - ox) / dx - 1/2
  const double cx = a.ox + 0.5 * a.dx, cy = a.oy + 0.5 * a.dy;
  IndexMap im;
  im.m[0] = a00;
  im.m[1] = a01 * a.dy / a.dx;
  im.m[2] = (a00 * cx + a01 * cy + a02 - a.ox) / a.dx - 0.5;
  im.m[3] = a10 * a.dx / a.dy;
  im.m[4] = a11;
  im.m[5] = (a10 * cx + a11 * cy + a12 - a.oy) / a.dy - 0.5;
  return im;
}

// Source of current cell (i, j): in the box or not, first tap (i0, j0), steps
// to the second row / column (0 when clamped) and the bilinear weights.
struct Src {
  bool in;
  int i0, j0, di, dj;
  float w[4];   // (i0, j0), (i0, j0 + dj), (i0 + di, j0), (i0 + di, j0 + dj)
};

__device__ __forceinline__ Src source_of(const AlignArgs& a, const IndexMap& im, int i, int j) {
  Src s;
  const double si = fma(im.m[0], (double)i, fma(im.m[1], (double)j, im.m[2]));
  const double sj = fma(im.m[3], (double)i, fma(im.m[4], (double)j, im.m[5]));
  s.in = (si >= 0.0) && (si <= (double)(a.X - 1)) && (sj >= 0.0) && (sj <= (double)(a.Y - 1));
  const double fi = s.in ? floor(si) : 0.0, fj = s.in ? floor(sj) : 0.0;
  s.i0 = (int)fi;
  s.j0 = (int)fj;
  s.di = (s.i0 + 1 < a.X) ? 1 : 0;
  s.dj = (s.j0 + 1 < a.Y) ? 1 : 0;
  const float fa = s.in ? (float)(si - fi) : 0.f, fb = s.in ? (float)(sj - fj) : 0.f;
  s.w[0] = (1.f - fa) * (1.f - fb);
  s.w[1] = (1.f - fa) * fb;
  s.w[2] = fa * (1.f - fb);
  s.w[3] = fa * fb;
  return s;
}

__device__ __forceinline__ void align_fwd_body(const AlignArgs& a, int bid, int nblk) {
  const int u = xcd_block(bid, nblk);        // unit = (cell block, channel chunk, sample)
  const int blk = u % a.nblk, rest = u / a.nblk;
  const int chunk = rest % a.nchunk, b = rest / a.nchunk;
  const int XY = a.X * a.Y;
  const int q = blk * kAlignBlock + threadIdx.x;
  if (q >= XY) return;
  const int i = q / a.Y, j = q - i * a.Y;
  const IndexMap im = index_map(a, b);
  const Src s = source_of(a, im, i, j);
  const int c_begin = chunk * kAlignChunk;
  const int c_end = min(c_begin + kAlignChunk, a.Cp);
  const int t00 = s.i0 * a.Y + s.j0;
  const int t01 = t00 + s.dj, t10 = t00 + s.di * a.Y, t11 = t10 + s.dj;
  float v[kAlignChunk];
#pragma unroll
  for (int k = 0; k < kAlignChunk; ++k) {          // all taps of the chunk in flight before the first is used
    const int c = min(c_begin + k, c_end - 1);
    const float* pc = a.src + ((size_t)b * a.Cp + c) * XY;
    v[k] = s.w[0] * pc[t00] + s.w[1] * pc[t01] + s.w[2] * pc[t10] + s.w[3] * pc[t11];
  }
#pragma unroll
  for (int k = 0; k < kAlignChunk; ++k) {
    const int c = c_begin + k;
    if (c < c_end) a.dst[((size_t)b * a.out_ch + a.c0 + c) * XY + q] = s.in ? v[k] : 0.f;
  }
}

__device__ __forceinline__ void align_bwd_body(const AlignArgs& a, int bid, int nblk) {
  const int u = xcd_block(bid, nblk);        // unit = (cell block, channel chunk, sample)
  const int blk = u % a.nblk, rest = u / a.nblk;
  const int chunk = rest % a.nchunk, b = rest / a.nchunk;
  const int XY = a.X * a.Y;
  const int q = blk * kAlignBlock + threadIdx.x;
  if (q >= XY) return;
  const int qi = q / a.Y, qj = q - qi * a.Y;
  const IndexMap im = index_map(a, b);
  // cells (i, j) whose source lies in the open square (qi - 1, qi + 1) x (qj - 1, qj + 1):
  // (i, j) = M^{-1} ((si, sj) - m2), a box of half-widths r around M^{-1} ((qi, qj) - m2)
  const double det = im.m[0] * im.m[4] - im.m[1] * im.m[3];
  const double n00 = im.m[4] / det, n01 = -im.m[1] / det, n10 = -im.m[3] / det, n11 = im.m[0] / det;
  const double ci = n00 * (qi - im.m[2]) + n01 * (qj - im.m[5]);
  const double cj = n10 * (qi - im.m[2]) + n11 * (qj - im.m[5]);
  const double ri = fabs(n00) + fabs(n01) + 1e-6, rj = fabs(n10) + fabs(n11) + 1e-6;
  const bool ok = isfinite(ci) && isfinite(cj) && ri < 0.5 * (kAlignMaxWin - 1) && rj < 0.5 * (kAlignMaxWin - 1);
  const int i_lo = ok ? max(0, (int)ceil(ci - ri)) : 1, i_hi = ok ? min(a.X - 1, (int)floor(ci + ri)) : 0;
  const int j_lo = ok ? max(0, (int)ceil(cj - rj)) : 1, j_hi = ok ? min(a.Y - 1, (int)floor(cj + rj)) : 0;
  const int c_begin = chunk * kAlignChunk;
  const int c_end = min(c_begin + kAlignChunk, a.Cp);
  float acc[kAlignChunk];
#pragma unroll
  for (int k = 0; k < kAlignChunk; ++k) acc[k] = 0.f;
  for (int i = i_lo; i <= i_hi; ++i) {
    for (int j = j_lo; j <= j_hi; ++j) {
      const Src s = source_of(a, im, i, j);
      if (!s.in) continue;
      const int t00 = s.i0 * a.Y + s.j0;
      const int t01 = t00 + s.dj, t10 = t00 + s.di * a.Y, t11 = t10 + s.dj;
      // the taps can coincide at the last row / column (the clamped one weighs 0): add every match
      const float w = (t00 == q ? s.w[0] : 0.f) + (t01 == q ? s.w[1] : 0.f) + (t10 == q ? s.w[2] : 0.f) +
                      (t11 == q ? s.w[3] : 0.f);
      if (w == 0.f) continue;
      const int o = i * a.Y + j;
#pragma unroll
      for (int k = 0; k < kAlignChunk; ++k) {
        const int c = min(c_begin + k, c_end - 1);
        acc[k] = fmaf(w, a.src[((size_t)b * a.out_ch + a.c0 + c) * XY + o], acc[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kAlignChunk; ++k) {
    const int c = c_begin + k;
    if (c < c_end) a.dst[((size_t)b * a.Cp + c) * XY + q] = acc[k];
  }
}

inline AlignArgs align_args(const Problem& p, int Cp, const float* ego, int c0) {
  AlignArgs a;
  a.ego = ego;
  a.B = p.B;
  a.X = p.X;
  a.Y = p.Y;
  a.Cp = Cp;
  a.out_ch = p.out_ch;
  a.c0 = c0;
  a.ox = p.ox;
  a.dx = p.dx;
  a.oy = p.oy;
  a.dy = p.dy;
  return a;
}

inline dim3 align_grid(AlignArgs& a) {
  const long long XY = (long long)a.X * a.Y;
  a.nblk = (int)((XY + kAlignBlock - 1) / kAlignBlock);
  a.nchunk = (a.Cp + kAlignChunk - 1) / kAlignChunk;
  return dim3((unsigned)((long long)a.nblk * a.nchunk * a.B));
}

// The temporal forward's Sampling-VT part (the bin-run kernel) and the previous map's resampling `al` (its
// source, destination and motion set) in one launch; false, with nothing launched, where the bin-run forward
// would need several launches or another lane layout (err holds the launch's status otherwise).
bool launch_forward_runs_temporal(const Problem& p, float* out, uint8_t* counts, const AlignArgs& al,
                                  hipStream_t stream, hipError_t& err);

}  // namespace fbev
