// Wave-level helpers for the gfx950 kernels (64-lane wavefronts).
//
// Cross-lane sums use DPP row permutations (quad swaps, mirrors and rotations
// within a row of 16 lanes; plain VALU operands) and the gfx950 lane-swap
// instructions for the row pairs and the half-waves, never LDS permutes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fbev {

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Orders a wave's own LDS writes before its later reads (one wave, no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lanes below this one in mask.
__device__ __forceinline__ int rank_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// x of the lane that DPP control Ctrl names, within the lane's row of 16 (T: float or int).
template <int Ctrl, typename T>
__device__ __forceinline__ T dpp(T x) {
  static_assert(sizeof(T) == 4, "32-bit lanes");
  return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1, 0, 3, 2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2, 3, 0, 1]: lane ^ 2
constexpr int kHalfMirror = 0x141;    // lane j <-> 7 - j within each half-row
constexpr int kRowMirror = 0x140;     // lane j <-> 15 - j within the row
constexpr int kRowRor1 = 0x121;       // rotate the row by 1 lane
constexpr int kRowRor2 = 0x122;       // rotate the row by 2 lanes
constexpr int kRowRor4 = 0x124;       // rotate the row by 4 lanes
constexpr int kRowRor8 = 0x128;       // rotate the row by 8 lanes

constexpr int kRowShr1 = 0x111;       // lane j of the row takes lane j - 1 (none below lane 0 of the row)
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142;    // lane 15 of each row to every lane of the next row
constexpr int kRowBcast31 = 0x143;    // lane 31 to every lane of rows 2 and 3
constexpr int kWaveShl1 = 0x130;      // lane i takes lane i + 1 (none for lane 63)
constexpr int kWaveShr1 = 0x138;      // lane i takes lane i - 1 (none for lane 0)

// x of the lane that DPP control Ctrl names, or `none` where there is no such lane or its row is masked out.
template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ int dpp_or(int x, int none) {
  return __builtin_amdgcn_update_dpp(none, x, Ctrl, RowMask, 0xF, false);
}

// Inclusive prefix sum over the wave in lane order: shifts within each row of 16, then the row
// broadcasts carry each row's total into the rows above it (six DPP adds, no LDS).
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += dpp_or<kRowShr1>(v, 0);
  v += dpp_or<kRowShr2>(v, 0);
  v += dpp_or<kRowShr4>(v, 0);
  v += dpp_or<kRowShr8>(v, 0);
  v += dpp_or<kRowBcast15, 0xA>(v, 0);
  v += dpp_or<kRowBcast31, 0xC>(v, 0);
  return v;
}

// The value of the previous (next) lane of the wave, `none` for lane 0 (63).
__device__ __forceinline__ int lane_prev(int x, int none) { return dpp_or<kWaveShr1>(x, none); }
__device__ __forceinline__ int lane_next(int x, int none) { return dpp_or<kWaveShl1>(x, none); }

// Sum over the four lanes of a quad.
template <typename T>
__device__ __forceinline__ T quad_sum(T x) {
  x += dpp<kQuadSwap1>(x);
  return x + dpp<kQuadSwap2>(x);
}

// Sum over the 16 lanes of a row.
template <typename T>
__device__ __forceinline__ T row_sum16(T x) {
  x = quad_sum(x);
  x += dpp<kHalfMirror>(x);
  return x + dpp<kRowMirror>(x);
}

// Sum over the lanes of a row that agree modulo L (L = 1, 2, 4, 8 or 16): rotations by 8, 4, ...,
// L pair every lane with the others of its residue class.
template <int L, typename T>
__device__ __forceinline__ T row_sum_stride(T x) {
  static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16, "a power of two up to 16");
  if constexpr (L <= 8) x += dpp<kRowRor8>(x);
  if constexpr (L <= 4) x += dpp<kRowRor4>(x);
  if constexpr (L <= 2) x += dpp<kRowRor2>(x);
  if constexpr (L <= 1) x += dpp<kRowRor1>(x);
  return x;
}

// x + the register of the lane one row over (permlane16: rows 0 <-> 1, 2 <-> 3) or one
// half-wave over (permlane32), with x and y swapped in one instruction: the lanes of the
// rows (halves) that kept x hold x's pair sum, the others y's.
template <typename T>
__device__ __forceinline__ T swap16_add(T x, T y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y),
                                                  false, false);
  const uint32_t a = r[0], b = r[1];   // both halves as plain values before the casts
  return __builtin_bit_cast(T, a) + __builtin_bit_cast(T, b);
}
template <typename T>
__device__ __forceinline__ T swap32_add(T x, T y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y),
                                                  false, false);
  const uint32_t a = r[0], b = r[1];
  return __builtin_bit_cast(T, a) + __builtin_bit_cast(T, b);
}

// Sum over the wave, in every lane.
template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
  x = row_sum16(x);
  x = swap16_add(x, x);
  return swap32_add(x, x);
}

// Block bid of nblk renumbered so that the blocks the dispatcher sends to one XCD (bid mod 8,
// round-robin) take one contiguous range: neighbouring work shares that XCD's L2.
__device__ __forceinline__ int xcd_block(int bid, int nblk) {
  const int xcd = bid & 7, k = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  return (xcd < rem) ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
}

}  // namespace fbev
