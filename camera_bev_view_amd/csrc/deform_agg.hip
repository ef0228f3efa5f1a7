// Deformable Aggregation for gfx950: multi-camera deformable sampling fused
// into one kernel per direction.
//
// The operator is the one the SparseDriveV2 notes describe ("Deformable
// Aggregation", steps 1-3), which the FlashBEV notes carry over to BEVFormer's
// spatial cross-attention: query q has a 3D anchor a_q and K keypoint offsets;
// keypoint p = a_q + offset is projected into every camera
// ([u, v, 1]^T ~ K_i (R_i p + t_i)); where it is in view (depth > 0, inside
// the closed box of pixel centres) the camera's feature map is sampled
// bilinearly and weighted by the query's weight for (camera, keypoint); the
// query's output is the sum.  Nothing per (query, keypoint, camera) reaches
// device memory.
//
// Forward: a wave owns a (query, 64-channel block).  Phase A takes one
// (camera, keypoint) pair per lane: fp64 projection, sign tests for the in-view rule,
// then the four taps and their weights (bilinear x attention) for the pairs
// in view, compacted into a per-wave LDS list of tap records.  Phase C
// gathers with lanes = channels: each record is one coalesced row of the
// channels-last map, up to 8 in flight, accumulated in fp32; the query's row
// of [B, Q, C] leaves coalesced.
//
// Backward: the same phase A lists the in-view samples with their fractions
// and depths; a query's 64-channel blocks are spread over up to four waves of
// one workgroup.  (i) The feature gradient: all samples of a query scatter
// w x tap weight x g with the query's one g, so the pass's taps are merged per
// pixel in an LDS hash table (weights added) and each distinct pixel becomes
// one entry (pixel, rank, weight), the rank taken from the pixel's integer
// counter.  After the main kernel a scan of the counts gives every pixel a
// bucket, the entries are scattered into the buckets, and a gather kernel sums
// w x g over each pixel's bucket with lanes = channels and writes every element
// of dL/dF once: no floating-point atomics, no zero-fill of dL/dF.  Per sample,
// lanes = channels load the four taps once and give (ii) the wave's part of
// dL/dw = <sample, g> and (iii) of dL/du, dL/dv = w <dsample/du, g>,
// w <dsample/dv, g>, reduced twelve at a time (four samples) by lane swaps and
// DPP.  The parts are added in wave order; the keypoint gradient is then
// dL/du du/dp + dL/dv dv/dp with du/dp = (P_1 - u P_3) / h_3 (rows of the 3x3
// part of P = K [R | t]), summed over cameras per keypoint in LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "deform_agg.h"
#include "wave_ops.h"

namespace fbev {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kBlock = kWave * kWaves;
constexpr int kUnroll = 8;                // tap rows in flight per lane

struct TapRec {
  int off;      // element offset of the tap's channel row within the batch sample
  float w;      // bilinear weight x attention weight
};

// Twelve wave sums at once, v[3 i + j] = sum j (0..2) of sample i (0..3): each swap halves
// the values a lane carries, so afterwards the 16 lanes of row i hold sample i's sums z[0..2].
__device__ __forceinline__ void wave_sum_4x3(const float (&v)[12], float (&z)[3]) {
  float w[6];
#pragma unroll
  for (int k = 0; k < 6; ++k) w[k] = swap32_add(v[k], v[k + 6]);       // lower half: v[k], upper: v[k + 6]
#pragma unroll
  for (int k = 0; k < 3; ++k) z[k] = row_sum16(swap16_add(w[k], w[k + 3]));   // row r: v[k + 3 r]
}

// 1/x in double: hardware estimate and two Newton steps.
__device__ __forceinline__ double recip(double x) {
  double r = __builtin_amdgcn_rcp(x);
  r = fma(r, fma(-x, r, 1.0), r);
  r = fma(r, fma(-x, r, 1.0), r);
  return r;
}

// P = K [R | t] in fp64 for the N cameras of batch sample b, 12 doubles each
// (row-major 3 x 4), one camera per thread.
__device__ void stage_projections(double* sP, const float* K, const float* R, const float* t, int b, int N) {
  for (int n = threadIdx.x; n < N; n += kBlock) {
    const size_t bn = (size_t)b * N + n;
    double k[9], r[9], tt[3];
    for (int i = 0; i < 9; ++i) {
      k[i] = (double)K[bn * 9 + i];
      r[i] = (double)R[bn * 9 + i];
    }
    for (int i = 0; i < 3; ++i) tt[i] = (double)t[bn * 3 + i];
    double* P = sP + n * 12;
    for (int i = 0; i < 3; ++i) {
      for (int j = 0; j < 3; ++j) {
        double s = 0.0;
        for (int m = 0; m < 3; ++m) s = fma(k[i * 3 + m], r[m * 3 + j], s);
        P[i * 4 + j] = s;
      }
      double s = 0.0;
      for (int m = 0; m < 3; ++m) s = fma(k[i * 3 + m], tt[m], s);
      P[i * 4 + 3] = s;
    }
  }
}

// One (camera, keypoint) pair of a query: h = P [p; 1] and the in-view rule
// by sign tests (depth h_3 > 0 and 0 <= h_1 <= (W-1) h_3, 0 <= h_2 <= (H-1) h_3).
struct Proj {
  double h0, h1, h2;
  bool valid;
};

__device__ __forceinline__ Proj project_pair(const double* P, double px, double py, double pz, int H, int W) {
  Proj r;
  r.h0 = fma(P[0], px, fma(P[1], py, fma(P[2], pz, P[3])));
  r.h1 = fma(P[4], px, fma(P[5], py, fma(P[6], pz, P[7])));
  r.h2 = fma(P[8], px, fma(P[9], py, fma(P[10], pz, P[11])));
  r.valid = (r.h2 > 0.0) && (r.h0 >= 0.0) && (fma((double)(W - 1), r.h2, -r.h0) >= 0.0) && (r.h1 >= 0.0) &&
            (fma((double)(H - 1), r.h2, -r.h1) >= 0.0);
  return r;
}

// Taps of an in-view sample: x0 = floor(u), x1 = min(x0 + 1, W - 1) (the clamped
// tap has weight 0), likewise rows; fractions a = u - x0, b = v - y0.
struct Taps {
  int p00, dx, dy;   // element offset of tap (y0, x0); steps to x1 and y1 (0 when clamped)
  int pix, dxp, dyp; // the same as pixel indices within the batch sample (n H W + y W + x)
  float a, b;
  double u, v;
};

__device__ __forceinline__ Taps taps_of(const Proj& pr, int n, int H, int W, int C, size_t HWC) {
  Taps t;
  const double r = recip(pr.h2);
  t.u = pr.h0 * r;
  t.v = pr.h1 * r;
  const double fu = fmin(fmax(floor(t.u), 0.0), (double)(W - 1));
  const double fv = fmin(fmax(floor(t.v), 0.0), (double)(H - 1));
  const int x0 = (int)fu, y0 = (int)fv;
  t.a = (float)(t.u - fu);
  t.b = (float)(t.v - fv);
  t.pix = (n * H + y0) * W + x0;
  t.dxp = (x0 + 1 < W) ? 1 : 0;
  t.dyp = (y0 + 1 < H) ? W : 0;
  t.p00 = (int)((size_t)t.pix * C);
  t.dx = t.dxp * C;
  t.dy = t.dyp * C;
  return t;
}

constexpr int kVecSteps = 8;             // 16-byte gather: steps (four taps each) in flight per lane
constexpr int kOutOfRange = 0x7ffffff0;  // buffer offset the range check turns into a zero load

typedef uint32_t u32x4 __attribute__((__vector_size__(16)));

// K steps of the 16-byte gather, all loads issued before the first is used: lane (slot s, chunk j) takes tap
// t0 + 4 u + s of step u, channels 4 j .. 4 j + 3 of the lane's block; taps at or past ntaps, and lanes past
// the block's channels (lane_ok false), read nothing.
template <int K>
__device__ __forceinline__ void gather_vec(float (&acc)[4], const TapRec* rec, int t0, int ntaps, int slot,
                                           __amdgpu_buffer_rsrc_t rs, int lane_off, bool lane_ok) {
  u32x4 v[K];
  float w[K];
#pragma unroll
  for (int u = 0; u < K; ++u) {
    const int tap = t0 + 4 * u + slot;
    const bool in = tap < ntaps;
    const TapRec rr = rec[in ? tap : 0];
    w[u] = in ? rr.w : 0.f;
    v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (in && lane_ok) ? 4 * rr.off + lane_off : kOutOfRange, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < K; ++u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(w[u], __uint_as_float(v[u][i]), acc[i]);
  }
}

// Forward.  VEC: channels-last rows with C a multiple of 4 and 16-byte aligned, gathered with lanes =
// (tap slot, 4-channel chunk): a load instruction takes four taps' 64-channel blocks, whole groups of
// kVecSteps steps are issued before any is used (a query with up to 8 in-view pairs, 32 taps, costs one
// round trip), and the four slots are summed with lane swaps at the end.  Otherwise lanes = channels,
// one tap row per load, kUnroll in flight.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void deform_fwd(DeformArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* sP = reinterpret_cast<double*>(smem);                                   // [N][12]
  TapRec* sRec = reinterpret_cast<TapRec*>(smem + sizeof(double) * 12 * a.N);     // [kWaves][4 * kWave]
  const int b = blockIdx.y;
  stage_projections(sP, a.K, a.R, a.t, b, a.N);
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);
  TapRec* rec = sRec + wid * 4 * kWave;
  const int NK = a.N * a.Kp;
  const size_t HWC = (size_t)a.H * a.W * a.C;
  const float* fb = a.feat + (size_t)b * a.N * HWC;

  // this wave's unit: query q, channels [c0, c0 + 64)
  const int groups = (a.C + kWave - 1) / kWave;
  const int unit = blockIdx.x * kWaves + wid;
  if (unit >= a.Q * groups) return;                   // no barrier follows
  const int q = unit / groups;
  const int c0 = (unit - q * groups) * kWave;
  const size_t bq = (size_t)b * a.Q + q;
  const double ax = a.anchors[bq * 3], ay = a.anchors[bq * 3 + 1], az = a.anchors[bq * 3 + 2];
  const int c = c0 + lane;
  const bool ch = c < a.C;
  float acc = 0.f;
  // VEC lane roles: tap slot, and a 4-channel chunk of the block (lanes past the block's channels read nothing)
  const int slot = lane >> 4, jc = lane & 15;
  const bool ch4 = c0 + 4 * jc < a.C;
  const int lane_off = 4 * (c0 + 4 * jc);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(fb), 0, VEC ? (int)(sizeof(float) * a.N * HWC) : 0,
                                        0x00020000);
  float acc4[4] = {0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < NK; base += kWave) {
    // ---- phase A: pair idx = n * Kp + k on this lane
    const int idx = base + lane;
    bool valid = false;
    Taps tp;
    float wq = 0.f;
    if (idx < NK) {
      const int n = idx / a.Kp, k = idx - n * a.Kp;
      const float* o = a.offsets + (bq * a.Kp + k) * 3;
      wq = a.weights[bq * NK + idx];                 // loaded with the offsets: one round trip for both
      const Proj pr = project_pair(sP + n * 12, ax + (double)o[0], ay + (double)o[1], az + (double)o[2], a.H, a.W);
      valid = pr.valid;
      if (valid) tp = taps_of(pr, n, a.H, a.W, a.C, HWC);
    }
    const uint64_t m = __ballot(valid);
    const int cnt = (int)__builtin_popcountll(m);
    if (valid) {
      const int s = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
      const float wa0 = (1.f - tp.a) * wq, wa1 = tp.a * wq;
      rec[4 * s + 0] = TapRec{tp.p00, wa0 * (1.f - tp.b)};
      rec[4 * s + 1] = TapRec{tp.p00 + tp.dx, wa1 * (1.f - tp.b)};
      rec[4 * s + 2] = TapRec{tp.p00 + tp.dy, wa0 * tp.b};
      rec[4 * s + 3] = TapRec{tp.p00 + tp.dy + tp.dx, wa1 * tp.b};
    }
    wave_lds_sync();
    // ---- phase C: gather the listed taps
    const int ntaps = 4 * cnt;
    if constexpr (VEC) {
      for (int t0 = 0; t0 < ntaps; t0 += 4 * kVecSteps) {
        const int n = min(kVecSteps, (ntaps - t0 + 3) / 4);      // steps of this group, wave-uniform
        switch (n) {
          case 1: gather_vec<1>(acc4, rec, t0, ntaps, slot, rs, lane_off, ch4); break;
          case 2: gather_vec<2>(acc4, rec, t0, ntaps, slot, rs, lane_off, ch4); break;
          case 3: gather_vec<3>(acc4, rec, t0, ntaps, slot, rs, lane_off, ch4); break;
          case 4: gather_vec<4>(acc4, rec, t0, ntaps, slot, rs, lane_off, ch4); break;
          case 5: gather_vec<5>(acc4, rec, t0, ntaps, slot, rs, lane_off, ch4); break;
          case 6: gather_vec<6>(acc4, rec, t0, ntaps, slot, rs, lane_off, ch4); break;
          case 7: gather_vec<7>(acc4, rec, t0, ntaps, slot, rs, lane_off, ch4); break;
          default: gather_vec<8>(acc4, rec, t0, ntaps, slot, rs, lane_off, ch4); break;
        }
      }
    } else {
      for (int j = 0; j < ntaps; j += kUnroll) {
        float v[kUnroll], w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int jj = j + u;
          const bool in = jj < ntaps;
          const TapRec rr = rec[in ? jj : 0];
          w[u] = in ? rr.w : 0.f;
          v[u] = (in && ch) ? fb[(size_t)rr.off + c] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc = fmaf(w[u], v[u], acc);
      }
    }
    wave_lds_sync();   // the records are read before the next pass overwrites them
  }
  if constexpr (VEC) {
    // sum over the four slots: afterwards every lane holds its chunk's totals
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc4[i] = swap32_add(acc4[i], acc4[i]);
      acc4[i] = swap16_add(acc4[i], acc4[i]);
    }
    if (slot == 0 && ch4)
      *reinterpret_cast<float4*>(a.out + bq * a.C + c0 + 4 * jc) = make_float4(acc4[0], acc4[1], acc4[2], acc4[3]);
  } else {
    if (ch) a.out[bq * a.C + c] = acc;
  }
}

constexpr int kSampUnroll = 4;           // backward samples whose tap loads are in flight together (one per lane row)
constexpr int kVecSamples = 8;           // the same for the 16-byte tap loads (a multiple of four)
constexpr int kTabMinBits = 6;           // a pass uses 2^bits slots, at least 4/3 of its 4 cnt taps (at most 3/4 full)

// Per-wave LDS of the backward: the in-view samples of one pass.
struct SampleRec {
  int pix, dxp, dyp, idx; // taps as pixel indices (as in Taps); idx = n * Kp + k
  float a, b, w;
  int k;                  // keypoint
  double u, v, h2;
};

// Backward: a query's 64-channel blocks are spread over wq_n waves of one
// workgroup (qw_n = 4 / wq_n queries per workgroup).  Every wave lists the
// query's in-view samples itself; per sample it loads its channels of the four
// taps and forms its part of <sample, g>, <d sample/du, g>, <d sample/dv, g>;
// the query's first wave emits the merged dL/dF entries.  After a pass the parts are
// added in wave order (fixed), lane s of the query's first wave turns sample s's
// sums into dL/dw and its keypoint's gradient through the projection, and lane
// k adds the pass's contributions to keypoint k in sample order: dL/dw,
// dL/doffsets and dL/danchors are deterministic.
// Five waves per SIMD (at most 96 VGPRs): with the table sized to the pass bound, a dense workload's
// 27 KB of LDS then fits five workgroups per CU.
// Four row sums at once: d[q] holds lane j's part of value q (j = lane % 16); afterwards every lane of quad q
// of the row (j / 4 == q) holds the row's sum of value q (mirror across the row, then across each half, then
// two quad swaps: 5 DPP adds for four sums).
__device__ __forceinline__ float row_sums_x4(const float (&d)[4], int j) {
  const bool lower = j < 8;
  const float a0 = (lower ? d[0] : d[2]) + dpp<kRowMirror>(lower ? d[2] : d[0]);
  const float a1 = (lower ? d[1] : d[3]) + dpp<kRowMirror>(lower ? d[3] : d[1]);
  const bool lo4 = (j & 7) < 4;
  float b = (lo4 ? a0 : a1) + dpp<kHalfMirror>(lo4 ? a1 : a0);
  b += dpp<kQuadSwap1>(b);
  b += dpp<kQuadSwap2>(b);
  return b;
}

// VEC: the per-sample sums by 16-byte loads, lanes = (tap, 4-channel chunk): a lane forms the dot product of
// its tap's channels with g, the 16 lanes of a row sum it (four samples at a time), and the sample's three
// sums follow from its four tap dots: <sample, g> = sum of the bilinear weights times the dots, and the u and
// v derivatives are the dots' differences along x and y.  Otherwise lanes = channels, four tap loads each.
// W1: one wave per query (C <= 64), so the query's steps need only wave-level order: no workgroup barrier after
// the camera staging, and each wave goes at its own pace.
template <bool VEC, bool W1>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(5))) void deform_bwd(DeformArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* sP = reinterpret_cast<double*>(smem);                                             // [N][12]
  SampleRec* sS = reinterpret_cast<SampleRec*>(smem + sizeof(double) * 12 * a.N);           // [kWaves][kWave]
  float* sPart = reinterpret_cast<float*>(sS + kWaves * kWave);                             // [kWaves][kWave][4]
  int2* sTab = reinterpret_cast<int2*>(sPart + kWaves * kWave * 4);                         // [kWaves][tab_max]
  float* sG = reinterpret_cast<float*>(sTab + kWaves * a.tab_max);                           // [kWaves][Kp][3]
  const int b = blockIdx.y;
  stage_projections(sP, a.K, a.R, a.t, b, a.N);
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);
  const int wq_n = a.wq_n, qs = wid / wq_n, wq = wid - qs * wq_n;
  const int lead = qs * wq_n;                          // the query's first wave
  SampleRec* smp = sS + wid * kWave;
  int2* tab = sTab + wid * a.tab_max;                       // (pixel, merged weight bits); compacted in place
  float* con = sPart + wid * kWave * 4;                // keypoint contributions, over the parts once read
  const int NK = a.N * a.Kp;
  const size_t HWC = (size_t)a.H * a.W * a.C;
  const float* fb = a.feat + (size_t)b * a.N * HWC;
  const int pix_base = b * a.N * a.H * a.W;          // first pixel of this batch sample

  // queries visited in the order q = unit * stride mod Q (stride coprime to Q), which spreads the
  // waves that run at the same time over the image and so over the pixel counters' addresses
  const int unit = blockIdx.x * (kWaves / wq_n) + qs;
  const bool active = unit < a.Q;                     // inactive waves still take every barrier
  const int q = active ? (int)(((long long)unit * a.q_stride) % a.Q) : 0;
  const size_t bq = (size_t)b * a.Q + q;
  const double ax = a.anchors[bq * 3], ay = a.anchors[bq * 3 + 1], az = a.anchors[bq * 3 + 2];
  const float* gq = a.grad + bq * a.C;
  float* gk = sG + qs * a.Kp * 3;
  int ecount = 0;                                      // feature-gradient entries this query has emitted
  if (wq == 0)
    for (int e = lane; e < a.Kp * 3; e += kWave) gk[e] = 0.f;
  for (int base = 0; base < NK; base += kWave) {
    // ---- listing, as in the forward; out-of-view pairs get dL/dw = 0 (first wave of the query)
    const int idx = base + lane;
    bool valid = false;
    Proj pr;
    int n = 0;
    if (active && idx < NK) {
      n = idx / a.Kp;
      const int k = idx - n * a.Kp;
      const float* o = a.offsets + (bq * a.Kp + k) * 3;
      pr = project_pair(sP + n * 12, ax + (double)o[0], ay + (double)o[1], az + (double)o[2], a.H, a.W);
      valid = pr.valid;
      if (!valid && wq == 0) a.gweights[bq * NK + idx] = 0.f;
    }
    const uint64_t m = __ballot(valid);
    const int cnt = (int)__builtin_popcountll(m);
    if (valid) {
      const Taps tp = taps_of(pr, n, a.H, a.W, a.C, HWC);
      const int s = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
      smp[s] = SampleRec{tp.pix, tp.dxp, tp.dyp, idx, tp.a, tp.b, a.weights[bq * NK + idx], idx - n * a.Kp,
                         tp.u, tp.v, pr.h2};
    }
    // the table: 2^tb slots, the fewest (at least 64) that keep the pass's at most 4 cnt keys to 3/4 of them
    int tb = kTabMinBits;
    while ((1 << tb) * 3 < 16 * cnt) ++tb;
    const int tsize = 1 << tb;
    for (int e = lane; e < tsize; e += kWave) tab[e] = make_int2(-1, 0);
    wave_lds_sync();
    // ---- the pass's taps merged per pixel: every sample of a query scatters w x tap weight x g with
    // the same g, so taps on one pixel add their weights and leave as one dL/dF entry
    if (lane < cnt) {
      const SampleRec sr = smp[lane];
      const float wa0 = (1.f - sr.a) * sr.w, wa1 = sr.a * sr.w;
      const float wt[4] = {wa0 * (1.f - sr.b), wa1 * (1.f - sr.b), wa0 * sr.b, wa1 * sr.b};
      const int px[4] = {sr.pix, sr.pix + sr.dxp, sr.pix + sr.dyp, sr.pix + sr.dyp + sr.dxp};
      for (int t = 0; t < 4; ++t) {
        if (wt[t] == 0.f) continue;
        uint32_t h = ((uint32_t)px[t] * 2654435761u) >> (32 - tb);
        for (;;) {                                  // at most 4 cnt keys in 16 cnt / 3 slots or more: a free one exists
          const int old = atomicCAS(&tab[h].x, -1, px[t]);
          if (old == -1 || old == px[t]) break;
          h = (h + 1) & (tsize - 1);
        }
        atomicAdd(reinterpret_cast<float*>(&tab[h].y), wt[t]);
      }
    }
    wave_lds_sync();
    // compaction in place: an entry moves only to a lower slot, one the wave has already read
    int nu = 0;
    for (int e0 = 0; e0 < tsize; e0 += kWave) {
      const int2 ent = tab[e0 + lane];
      const uint64_t mk = __ballot(ent.x >= 0);
      if (ent.x >= 0)
        tab[nu + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(mk >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mk, 0u))] = ent;
      nu += (int)__builtin_popcountll(mk);
    }
    wave_lds_sync();
    // ---- per in-view sample: this wave's channels of the three sums, four samples at a time with
    // all their tap loads in flight (past the list's end the last sample is read again, unused)
    if constexpr (VEC) {
      const int trow = lane >> 4, jc = lane & 15;            // tap (x1 by bit 0, y1 by bit 1), channel chunk
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(fb), 0, (int)(sizeof(float) * a.N * HWC), 0x00020000);
      for (int s0 = 0; s0 < cnt; s0 += kVecSamples) {
        int off[kVecSamples];
#pragma unroll
        for (int i = 0; i < kVecSamples; ++i) {
          const SampleRec sr = smp[min(s0 + i, cnt - 1)];
          off[i] = (sr.pix + ((trow & 1) ? sr.dxp : 0) + ((trow & 2) ? sr.dyp : 0)) * a.C;
        }
        float d[kVecSamples];
#pragma unroll
        for (int i = 0; i < kVecSamples; ++i) d[i] = 0.f;
        for (int cb = wq * kWave; cb < a.C; cb += wq_n * kWave) {
          const int cc = cb + 4 * jc;
          const bool ok = cc < a.C;
          const float4 g4 = ok ? *reinterpret_cast<const float4*>(gq + cc) : make_float4(0.f, 0.f, 0.f, 0.f);
          u32x4 v[kVecSamples];
#pragma unroll
          for (int i = 0; i < kVecSamples; ++i)
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? 4 * (off[i] + cc) : kOutOfRange, 0, 0);
#pragma unroll
          for (int i = 0; i < kVecSamples; ++i) {
            d[i] = fmaf(g4.x, __uint_as_float(v[i][0]), d[i]);
            d[i] = fmaf(g4.y, __uint_as_float(v[i][1]), d[i]);
            d[i] = fmaf(g4.z, __uint_as_float(v[i][2]), d[i]);
            d[i] = fmaf(g4.w, __uint_as_float(v[i][3]), d[i]);
          }
        }
        const int qd = jc >> 2;
#pragma unroll
        for (int h = 0; h < kVecSamples; h += 4) {
          const float d4[4] = {d[h], d[h + 1], d[h + 2], d[h + 3]};
          const float dot = row_sums_x4(d4, jc);          // tap trow of sample s0 + h + jc / 4
          if ((jc & 3) == 0 && s0 + h + qd < cnt) sPart[(wid * kWave + s0 + h + qd) * 4 + trow] = dot;
        }
      }
      wave_lds_sync();
      // the sample's lane turns its four tap dots into the three sums (in place)
      if (lane < cnt) {
        const SampleRec sr = smp[lane];
        const float4 dt = *reinterpret_cast<const float4*>(sPart + (wid * kWave + lane) * 4);
        const float a0 = 1.f - sr.a, b0 = 1.f - sr.b;
        const float smpv = a0 * b0 * dt.x + sr.a * b0 * dt.y + a0 * sr.b * dt.z + sr.a * sr.b * dt.w;
        const float su = b0 * (dt.y - dt.x) + sr.b * (dt.w - dt.z);
        const float sv = a0 * (dt.z - dt.x) + sr.a * (dt.w - dt.y);
        *reinterpret_cast<float4*>(sPart + (wid * kWave + lane) * 4) = make_float4(smpv, su, sv, 0.f);
      }
    } else {
      for (int s0 = 0; s0 < cnt; s0 += kSampUnroll) {
        int p00[kSampUnroll], dx[kSampUnroll], dy[kSampUnroll];
        float fa[kSampUnroll], fbt[kSampUnroll];
  #pragma unroll
        for (int i = 0; i < kSampUnroll; ++i) {
          const SampleRec sr = smp[min(s0 + i, cnt - 1)];
          p00[i] = uniform(sr.pix) * a.C;
          dx[i] = uniform(sr.dxp) * a.C;
          dy[i] = uniform(sr.dyp) * a.C;
          fa[i] = sr.a;
          fbt[i] = sr.b;
        }
        float ds[kSampUnroll], du[kSampUnroll], dv[kSampUnroll];
  #pragma unroll
        for (int i = 0; i < kSampUnroll; ++i) ds[i] = du[i] = dv[i] = 0.f;
        for (int c = wq * kWave + lane; c < a.C; c += wq_n * kWave) {
          const float g = gq[c];
          float F[kSampUnroll][4];
  #pragma unroll
          for (int i = 0; i < kSampUnroll; ++i) {
            F[i][0] = fb[(size_t)p00[i] + c];
            F[i][1] = fb[(size_t)p00[i] + dx[i] + c];
            F[i][2] = fb[(size_t)p00[i] + dy[i] + c];
            F[i][3] = fb[(size_t)p00[i] + dy[i] + dx[i] + c];
          }
  #pragma unroll
          for (int i = 0; i < kSampUnroll; ++i) {
            const float a0 = 1.f - fa[i], b0 = 1.f - fbt[i];
            const float smpv = a0 * b0 * F[i][0] + fa[i] * b0 * F[i][1] + a0 * fbt[i] * F[i][2] + fa[i] * fbt[i] * F[i][3];
            const float su = b0 * (F[i][1] - F[i][0]) + fbt[i] * (F[i][3] - F[i][2]);
            const float sv = a0 * (F[i][2] - F[i][0]) + fa[i] * (F[i][3] - F[i][1]);
            ds[i] = fmaf(g, smpv, ds[i]);
            du[i] = fmaf(g, su, du[i]);
            dv[i] = fmaf(g, sv, dv[i]);
          }
        }
        float v[3 * kSampUnroll], z[3];
  #pragma unroll
        for (int i = 0; i < kSampUnroll; ++i) {
          v[3 * i] = ds[i];
          v[3 * i + 1] = du[i];
          v[3 * i + 2] = dv[i];
        }
        wave_sum_4x3(v, z);
        const int row = lane >> 4;
        if ((lane & 15) == 0 && s0 + row < cnt)
          *reinterpret_cast<float4*>(sPart + (wid * kWave + s0 + row) * 4) = make_float4(z[0], z[1], z[2], 0.f);
      }
    }
    // ---- the feature gradient: one entry (pixel, rank, merged weight) per merged pixel, the rank
    // taken from the pixel's counter; the gather kernels add w * g over each pixel's entries
    if (wq == 0 && a.entries != nullptr) {
      for (int e = lane; e < nu; e += kWave) {
        const int2 t = tab[e];
        const int gp = pix_base + t.x;
        const int rank = atomicAdd(a.pix_count + gp, 1);
        int* E = a.entries + ((size_t)bq * a.cap + ecount + e) * 3;
        E[0] = gp;
        E[1] = rank;
        E[2] = t.y;
      }
      ecount += nu;
    }
    if constexpr (W1) {
      wave_lds_sync();
    } else {
      __syncthreads();
    }
    // ---- the query's first wave: sums over its waves (wave order), dL/dw, keypoint contributions
    if (wq == 0 && lane < cnt) {
      float4 t = *reinterpret_cast<const float4*>(sPart + (lead * kWave + lane) * 4);
      for (int j = 1; j < wq_n; ++j) {
        const float4 o = *reinterpret_cast<const float4*>(sPart + ((lead + j) * kWave + lane) * 4);
        t.x += o.x;
        t.y += o.y;
        t.z += o.z;
      }
      const SampleRec sr = smp[lane];
      const int sn = sr.idx / a.Kp;
      a.gweights[bq * NK + sr.idx] = t.x;
      // keypoint gradient through the projection: du/dp = (P_1 - u P_3) / h_3, dv/dp likewise
      const double* P = sP + sn * 12;
      const double ih = recip(sr.h2);
      const double lu = (double)sr.w * t.y, lv = (double)sr.w * t.z;
      float c3[3];
      for (int r = 0; r < 3; ++r) {
        const double ju = (P[r] - sr.u * P[8 + r]) * ih, jv = (P[4 + r] - sr.v * P[8 + r]) * ih;
        c3[r] = (float)(lu * ju + lv * jv);
      }
      *reinterpret_cast<float4*>(con + lane * 4) = make_float4(c3[0], c3[1], c3[2], 0.f);   // this lane's parts are read
    }
    if (wq == 0) {
      wave_lds_sync();
      // lane k adds the contributions of this pass's samples of keypoint k, in sample order
      for (int kk = lane; kk < a.Kp; kk += kWave) {
        float gx = gk[kk * 3], gy = gk[kk * 3 + 1], gz = gk[kk * 3 + 2];
        for (int s = 0; s < cnt; ++s) {
          if (smp[s].k != kk) continue;
          const float4 c = *reinterpret_cast<const float4*>(con + s * 4);
          gx += c.x;
          gy += c.y;
          gz += c.z;
        }
        gk[kk * 3] = gx;
        gk[kk * 3 + 1] = gy;
        gk[kk * 3 + 2] = gz;
      }
    }
    // the sample lists and parts are rewritten by the next pass
    if constexpr (W1) {
      wave_lds_sync();
    } else {
      __syncthreads();
    }
  }
  // ---- the query's keypoint and anchor gradients (first wave)
  if (!active || wq != 0) return;                      // no barrier follows
  if (lane == 0 && a.entries != nullptr) a.q_count[bq] = ecount;
  float sx = 0.f, sy = 0.f, sz = 0.f;
  for (int k = lane; k < a.Kp; k += kWave) {
    const float gx = gk[k * 3], gy = gk[k * 3 + 1], gz = gk[k * 3 + 2];
    float* go = a.goffsets + (bq * a.Kp + k) * 3;
    go[0] = gx;
    go[1] = gy;
    go[2] = gz;
    sx += gx;
    sy += gy;
    sz += gz;
  }
  if (a.ganchors != nullptr) {
    sx = wave_sum(sx);
    sy = wave_sum(sy);
    sz = wave_sum(sz);
    if (lane == 0) {
      a.ganchors[bq * 3] = sx;
      a.ganchors[bq * 3 + 1] = sy;
      a.ganchors[bq * 3 + 2] = sz;
    }
  }
}

__global__ void deform_fill_zero(float* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride) dst[k] = 0.f;
}

// ---- dL/dF by gather: the per-pixel entry counts are scanned into bucket offsets, the entries
// scattered into their pixels' buckets, and every pixel's channels summed and written once.

constexpr int kScanThreads = 1024;                 // threads of a scan workgroup
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kScanPer = 16;                       // counts per thread in the scan kernels
constexpr int kScanBlock = kScanThreads * kScanPer;   // counts per scan workgroup

// Sum over the workgroup, returned to every thread (one barrier pair).
__device__ __forceinline__ int block_sum(int v, int* sW) {
  v = wave_sum(v);
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sW[wid] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < kScanWaves; ++w) t += sW[w];
  __syncthreads();
  return t;
}

// Per block of kScanBlock pixels: the sum of its entry counts.
__global__ __launch_bounds__(kScanThreads) void deform_scan_sums(const int* __restrict__ cnt, int n,
                                                                 int* __restrict__ bsum) {
  __shared__ int sW[kScanWaves];
  const int base = blockIdx.x * kScanBlock;
  int s = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    const int k = base + i * kScanThreads + threadIdx.x;
    s += (k < n) ? cnt[k] : 0;
  }
  s = block_sum(s, sW);
  if (threadIdx.x == 0) bsum[blockIdx.x] = s;
}

// Exclusive prefix sum of the counts: the preceding blocks' sums (bsum == NULL: added up from the
// counts themselves, for a few blocks), then a scan within the block (thread t owns kScanPer
// consecutive counts).
constexpr int kScanDirect = 16;                    // blocks at most for the one-launch scan
__global__ __launch_bounds__(kScanThreads) void deform_scan_apply(const int* __restrict__ cnt, int n,
                                                                  const int* __restrict__ bsum,
                                                                  int* __restrict__ first) {
  __shared__ int sW[kScanWaves];
  int pre = 0;
  if (bsum != nullptr) {
    for (int j = threadIdx.x; j < (int)blockIdx.x; j += kScanThreads) pre += bsum[j];
  } else {
#pragma unroll 8
    for (int j = threadIdx.x; j < (int)blockIdx.x * kScanBlock; j += kScanThreads) pre += cnt[j];
  }
  pre = block_sum(pre, sW);
  const int base = blockIdx.x * kScanBlock + threadIdx.x * kScanPer;
  int v[kScanPer];
  int own = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    v[i] = (base + i < n) ? cnt[base + i] : 0;
    own += v[i];
  }
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  int incl = own;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) sW[wid] = incl;
  __syncthreads();
  for (int w = 0; w < wid; ++w) pre += sW[w];
  int run = pre + incl - own;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    if (base + i < n) first[base + i] = run;
    run += v[i];
  }
}

// Entry (pixel p, rank r, w) of query bq into bucket slot first[p] + r; a wave per query.
__global__ __launch_bounds__(kBlock) void deform_scatter(DeformArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const size_t bq = (size_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  if (bq >= (size_t)a.B * a.Q) return;
  const int n = a.q_count[bq];
  const int* E = a.entries + bq * a.cap * 3;
  for (int e = lane; e < n; e += kWave)
    a.bucket[a.pix_first[E[3 * e]] + E[3 * e + 1]] = make_int2((int)bq, E[3 * e + 2]);
}

// One (pixel, 64-channel block) per wave: dL/dF[p, c] = sum over the pixel's entries of w * g[bq, c],
// the entries read as wave-uniform values, eight upstream rows in flight.  Every element is written.
constexpr int kGatherUnroll = 8;
__global__ __launch_bounds__(kBlock) void deform_gather(DeformArgs a, int npix) {
  const int lane = threadIdx.x & (kWave - 1);
  const int groups = (a.C + kWave - 1) / kWave;
  const long long unit = (long long)xcd_block(blockIdx.x, gridDim.x) * kWaves + threadIdx.x / kWave;
  if (unit >= (long long)npix * groups) return;
  const int p = (int)(unit / groups);
  const int c = (int)(unit - (long long)p * groups) * kWave + lane;
  const bool ch = c < a.C;
  const int n = uniform(a.pix_count[p]);
  const int2* bk = a.bucket + uniform(a.pix_first[p]);
  float acc = 0.f;
  for (int j = 0; j < n; j += kGatherUnroll) {
    float w[kGatherUnroll], v[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int2 e = bk[min(j + u, n - 1)];
      w[u] = (j + u < n) ? __int_as_float(e.y) : 0.f;
      v[u] = ch ? a.grad[(size_t)e.x * a.C + c] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) acc = fmaf(w[u], v[u], acc);
  }
  if (ch) a.gfeat[(size_t)p * a.C + c] = acc;
}

// The same for C % 4 == 0 with 16-byte aligned rows: lanes = (entry slot e, channel quad q), a wave covers up
// to 256 channels of its pixel as Qw quads (Qw = 16, 32 or 64, the power of two at or above the block's quads)
// and takes E = 64 / Qw entries per float4 load, eight loads in flight and the next step's entries read ahead;
// its E slots are summed by lane swaps at the end.  WP waves share a (pixel, 256-channel block): with WP = 4
// (pixels with a few hundred entries, as in the dense BEV form) the workgroup's waves take every fourth step of
// the pixel's entries and the first wave adds the others' sums in wave order; with WP = 1 a workgroup takes
// four pixels.
template <int Qw, int WP>
__global__ __launch_bounds__(kBlock) void deform_gather4(DeformArgs a, int npix) {
  static_assert(WP == 1 || WP == kWaves, "one wave or the whole workgroup per pixel");
  constexpr int E = kWave / Qw;
  constexpr int kStep = kGatherUnroll * E;
  __shared__ float4 sAcc[WP > 1 ? WP - 1 : 1][Qw];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = uniform(threadIdx.x / kWave);
  const int wp = wid % WP;                          // this wave's share of the pixel's entries
  const int e = lane / Qw, q = lane - e * Qw;
  const int groups = (a.C + 4 * kWave - 1) / (4 * kWave);
  const long long unit = (long long)xcd_block(blockIdx.x, gridDim.x) * (kWaves / WP) + wid / WP;
  if (unit >= (long long)npix * groups) return;      // (with WP > 1 the whole workgroup: no barrier follows)
  const int p = (int)(unit / groups);
  const int c = (int)(unit - (long long)p * groups) * 4 * kWave + 4 * q;
  const bool ch = c < a.C;
  const int n = uniform(a.pix_count[p]);
  const int2* bk = a.bucket + uniform(a.pix_first[p]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int j0 = wp * kStep;
  int2 en[kGatherUnroll];
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u) en[u] = (j0 < n) ? bk[min(j0 + u * E + e, n - 1)] : make_int2(0, 0);
  for (int j = j0; j < n; j += WP * kStep) {
    float4 v[kGatherUnroll];
    float w[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      w[u] = (j + u * E + e < n) ? __int_as_float(en[u].y) : 0.f;
      v[u] = ch ? *reinterpret_cast<const float4*>(a.grad + (size_t)en[u].x * a.C + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int jn = j + WP * kStep;
    if (jn < n) {
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) en[u] = bk[min(jn + u * E + e, n - 1)];
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      acc.x = fmaf(w[u], v[u].x, acc.x);
      acc.y = fmaf(w[u], v[u].y, acc.y);
      acc.z = fmaf(w[u], v[u].z, acc.z);
      acc.w = fmaf(w[u], v[u].w, acc.w);
    }
  }
  if constexpr (E == 4) {                           // slots in the four rows of 16 lanes
    acc.x = swap16_add(acc.x, acc.x);
    acc.y = swap16_add(acc.y, acc.y);
    acc.z = swap16_add(acc.z, acc.z);
    acc.w = swap16_add(acc.w, acc.w);
  }
  if constexpr (E >= 2) {                           // slots in the two half-waves
    acc.x = swap32_add(acc.x, acc.x);
    acc.y = swap32_add(acc.y, acc.y);
    acc.z = swap32_add(acc.z, acc.z);
    acc.w = swap32_add(acc.w, acc.w);
  }
  if constexpr (WP > 1) {
    if (wp > 0 && e == 0) sAcc[wp - 1][q] = acc;
    __syncthreads();
    if (wp == 0 && e == 0) {
#pragma unroll
      for (int w = 0; w < WP - 1; ++w) {
        const float4 o = sAcc[w][q];
        acc.x += o.x;
        acc.y += o.y;
        acc.z += o.z;
        acc.w += o.w;
      }
    }
  }
  if (wp == 0 && e == 0 && ch) *reinterpret_cast<float4*>(a.gfeat + (size_t)p * a.C + c) = acc;
}

}  // namespace

hipError_t launch_deform_forward(const DeformArgs& a, hipStream_t stream) {
  if (a.B == 0 || a.Q == 0 || a.C == 0) return hipSuccess;
  const long long units = (long long)a.Q * ((a.C + kWave - 1) / kWave);
  const dim3 grid((unsigned)((units + kWaves - 1) / kWaves), (unsigned)a.B);
  const size_t shmem = sizeof(double) * 12 * a.N + sizeof(TapRec) * 4 * kWave * kWaves;
  // the 16-byte gather needs 16-byte channel rows (C a multiple of 4, an aligned base) and buffer offsets
  // that fit 31 bits
  const bool vec = a.C % 4 == 0 && (reinterpret_cast<uintptr_t>(a.feat) & 15) == 0 &&
                   sizeof(float) * (double)a.N * a.H * a.W * a.C < (double)kOutOfRange;
  if (vec)
    hipLaunchKernelGGL(deform_fwd<true>, grid, dim3(kBlock), shmem, stream, a);
  else
    hipLaunchKernelGGL(deform_fwd<false>, grid, dim3(kBlock), shmem, stream, a);
  return hipGetLastError();
}

// A stride coprime to Q near Q times the golden ratio (1 when Q is small).
int query_stride(int Q) {
  if (Q < 64) return 1;
  auto gcd = [](long long x, long long y) { while (y) { const long long r = x % y; x = y; y = r; } return x; };
  long long s = (long long)(0.6180339887 * Q) | 1;
  while (gcd(s, Q) != 1) s += 2;
  return (int)(s % Q);
}

namespace {

// Workspace of the dL/dF gather: per-pixel counts and bucket offsets, scan block sums, per-query
// entry counts, the entries (at most 4 N Kp per query: 4 taps per (camera, keypoint) pair) and the
// buckets; each part 256-byte aligned.
struct WsLayout {
  size_t count, first, bsum, qcount, entries, bucket, total;
};

bool uses_gather(const DeformArgs& a) {
  return (size_t)a.B * a.N * a.H * a.W * a.C > 0 && (size_t)a.B * a.Q > 0 && a.N * a.Kp > 0;
}

WsLayout ws_layout(const DeformArgs& a) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t npix = (size_t)a.B * a.N * a.H * a.W;
  const size_t nblk = (npix + kScanBlock - 1) / kScanBlock;
  const size_t nq = (size_t)a.B * a.Q;
  const size_t ne = nq * 4 * (size_t)a.N * a.Kp;
  WsLayout L{};
  size_t o = 0;
  L.count = o;
  o = up(o + sizeof(int) * npix);
  L.first = o;
  o = up(o + sizeof(int) * npix);
  L.bsum = o;
  o = up(o + sizeof(int) * nblk);
  L.qcount = o;
  o = up(o + sizeof(int) * nq);
  L.entries = o;
  o = up(o + 3 * sizeof(int) * ne);
  L.bucket = o;
  o = up(o + sizeof(int2) * ne);
  L.total = o;
  return L;
}

}  // namespace

size_t deform_backward_workspace_bytes(const DeformArgs& a) { return uses_gather(a) ? ws_layout(a).total : 0; }

hipError_t launch_deform_backward(DeformArgs a, void* workspace, hipStream_t stream) {
  a.q_stride = query_stride(a.Q);
  const size_t npix = (size_t)a.B * a.N * a.H * a.W;
  const size_t nF = npix * a.C;
  const bool gather = uses_gather(a);
  a.entries = nullptr;
  if (gather) {
    const WsLayout L = ws_layout(a);
    unsigned char* w = static_cast<unsigned char*>(workspace);
    a.pix_count = reinterpret_cast<int*>(w + L.count);
    a.pix_first = reinterpret_cast<int*>(w + L.first);
    a.blk_sum = reinterpret_cast<int*>(w + L.bsum);
    a.q_count = reinterpret_cast<int*>(w + L.qcount);
    a.entries = reinterpret_cast<int*>(w + L.entries);
    a.bucket = reinterpret_cast<int2*>(w + L.bucket);
    a.cap = 4 * a.N * a.Kp;
  }
  // the counters start at zero; without entries to gather, dL/dF is zero
  float* zero = gather ? reinterpret_cast<float*>(a.pix_count) : a.gfeat;
  const size_t nz = gather ? npix : nF;
  if (nz > 0) {
    const size_t blocks = (nz + 255) / 256;
    hipLaunchKernelGGL(deform_fill_zero, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, stream, zero,
                       nz);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.B == 0 || a.Q == 0) return hipSuccess;
  // waves per query: one per 64-channel block, up to the workgroup's four (a power of two dividing four)
  const int blocks = (a.C + kWave - 1) / kWave;
  a.wq_n = blocks >= 3 ? 4 : (blocks == 2 ? 2 : 1);
  const int qw_n = kWaves / a.wq_n;
  const dim3 grid((unsigned)((a.Q + qw_n - 1) / qw_n), (unsigned)a.B);
  {  // the widest table a pass can need: at most 64 samples, and at most N Kp
    const int cmax = a.N * a.Kp < kWave ? a.N * a.Kp : kWave;
    int tb = kTabMinBits;
    while ((1 << tb) * 3 < 16 * cmax) ++tb;
    a.tab_max = 1 << tb;
  }
  const size_t shmem = sizeof(double) * 12 * a.N + sizeof(SampleRec) * kWave * kWaves +
                       sizeof(float) * 4 * kWave * kWaves + sizeof(int2) * a.tab_max * kWaves +
                       sizeof(float) * 3 * a.Kp * kWaves;
  // the 16-byte tap loads need 16-byte channel rows of the features and of the upstream gradient (C a
  // multiple of 4, aligned bases) and buffer offsets that fit 31 bits
  const bool vec = a.C % 4 == 0 && ((reinterpret_cast<uintptr_t>(a.feat) | reinterpret_cast<uintptr_t>(a.grad)) & 15) == 0 &&
                   sizeof(float) * (double)a.N * a.H * a.W * a.C < (double)kOutOfRange;
  if (a.wq_n == 1) {
    if (vec)
      hipLaunchKernelGGL((deform_bwd<true, true>), grid, dim3(kBlock), shmem, stream, a);
    else
      hipLaunchKernelGGL((deform_bwd<false, true>), grid, dim3(kBlock), shmem, stream, a);
  } else {
    if (vec)
      hipLaunchKernelGGL((deform_bwd<true, false>), grid, dim3(kBlock), shmem, stream, a);
    else
      hipLaunchKernelGGL((deform_bwd<false, false>), grid, dim3(kBlock), shmem, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !gather) return e;
  const int np = (int)npix;
  const unsigned nblk = (unsigned)((npix + kScanBlock - 1) / kScanBlock);
  if (nblk <= kScanDirect) {
    hipLaunchKernelGGL(deform_scan_apply, dim3(nblk), dim3(kScanThreads), 0, stream, a.pix_count, np, nullptr,
                       a.pix_first);
  } else {
    hipLaunchKernelGGL(deform_scan_sums, dim3(nblk), dim3(kScanThreads), 0, stream, a.pix_count, np, a.blk_sum);
    hipLaunchKernelGGL(deform_scan_apply, dim3(nblk), dim3(kScanThreads), 0, stream, a.pix_count, np, a.blk_sum,
                       a.pix_first);
  }
  const size_t nq = (size_t)a.B * a.Q;
  hipLaunchKernelGGL(deform_scatter, dim3((unsigned)((nq + kWaves - 1) / kWaves)), dim3(kBlock), 0, stream, a);
  const bool vec4 = a.C % 4 == 0 && ((reinterpret_cast<uintptr_t>(a.grad) | reinterpret_cast<uintptr_t>(a.gfeat)) & 15) == 0;
  if (vec4) {
    const size_t units = npix * ((a.C + 4 * kWave - 1) / (4 * kWave));
    // a workgroup per (pixel, block) when the pixels can hold a few hundred entries on average (the dense BEV
    // form: 123 against 127 us), else four per workgroup (the sparse queries: 38 against 39 us)
    const bool split = (double)a.B * a.Q * a.cap >= 512.0 * (double)npix;
    const dim3 g4((unsigned)(split ? units : (units + kWaves - 1) / kWaves));
#define FBEV_GATHER4(qw)                                                                   \
    if (split)                                                                             \
      hipLaunchKernelGGL((deform_gather4<qw, kWaves>), g4, dim3(kBlock), 0, stream, a, np); \
    else                                                                                   \
      hipLaunchKernelGGL((deform_gather4<qw, 1>), g4, dim3(kBlock), 0, stream, a, np);
    if (a.C <= 64) {
      FBEV_GATHER4(16)
    } else if (a.C <= 128) {
      FBEV_GATHER4(32)
    } else {
      FBEV_GATHER4(64)
    }
#undef FBEV_GATHER4
  } else {
    const size_t units = npix * blocks;
    hipLaunchKernelGGL(deform_gather, dim3((unsigned)((units + kWaves - 1) / kWaves)), dim3(kBlock), 0, stream, a,
                       np);
  }
  return hipGetLastError();
}

}  // namespace fbev
