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

// x of the lane that DPP control Ctrl names, within the lane's row of 16.
template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1, 0, 3, 2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2, 3, 0, 1]: lane ^ 2
constexpr int kHalfMirror = 0x141;    // lane j <-> 7 - j within each half-row
constexpr int kRowMirror = 0x140;     // lane j <-> 15 - j within the row
constexpr int kRowRor4 = 0x124;       // rotate the row by 4 lanes
constexpr int kRowRor8 = 0x128;       // rotate the row by 8 lanes

// Sum over the four lanes of a quad.
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  return x + dpp<kQuadSwap2>(x);
}

// Sum over the 16 lanes of a row.
__device__ __forceinline__ float row_sum16(float x) {
  x = quad_sum(x);
  x += dpp<kHalfMirror>(x);
  return x + dpp<kRowMirror>(x);
}

// Sum over the lanes of a row that agree modulo L (L = 1, 2, 4, 8 or 16): rotations by 8, 4, ...,
// L pair every lane with the others of its residue class.
template <int L>
__device__ __forceinline__ float row_sum_stride(float x) {
  static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16, "a power of two up to 16");
  if constexpr (L <= 8) x += dpp<kRowRor8>(x);
  if constexpr (L <= 4) x += dpp<kRowRor4>(x);
  if constexpr (L <= 2) x += dpp<0x122>(x);
  if constexpr (L <= 1) x += dpp<0x121>(x);
  return x;
}

// x + the register of the lane one row over (permlane16: rows 0 <-> 1, 2 <-> 3) or one
// half-wave over (permlane32), with x and y swapped in one instruction: the lanes of the
// rows (halves) that kept x hold x's pair sum, the others y's.
__device__ __forceinline__ float swap16_add(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_add(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the wave, in every lane.
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  x = swap16_add(x, x);
  return swap32_add(x, x);
}

}  // namespace fbev
