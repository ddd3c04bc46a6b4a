// Cross-lane exchanges for the 64-wide wavefront of gfx950.
//
// The row sums of a chunked tile (the Gated DeltaNet retrieval S^T k and the
// readout S^T q) reduce over the lane bits that carry the row block. The
// exchanges used, lowest row-block bit first:
//   lane bit 5  v_permlane32_swap  (a.hi <-> b.lo)
//   lane bit 4  v_permlane16_swap  (odd 16-lane rows of a <-> even rows of b)
//   lane bit 3  DPP row_ror:8      (lane l reads lane l^8 inside a 16-lane row)
//   lane bit 2  ds_swizzle xor 4
// The swaps move two registers in one instruction, so a "transposed" tree that
// halves the set of columns a lane carries at each level costs one exchange and
// one add per pair of columns.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsq {

__device__ __forceinline__ float dpp_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
}
// lane Q of each quad, broadcast to the four lanes of the quad
template <int Q>
__device__ __forceinline__ float dpp_quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Q * 0x55, 0xF, 0xF, true));
}
__device__ __forceinline__ float swz_xor(float v, int m) {
  // BitMode swizzle within 32 lanes: and 0x1F, or 0, xor m
  switch (m) {
    case 1: return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x041F));
    case 2: return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x081F));
    case 4: return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
    default: return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x201F));
  }
}

// max of |v[0..7]| in four v_max3/v_max with |.| source modifiers. The values
// are arithmetic results, so the canonicalising max the compiler would insert
// for fmaxf in IEEE mode is not needed.
__device__ __forceinline__ float absmax8(const float v[8]) {
  float m, n, p;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m) : "v"(v[0]), "v"(v[1]), "v"(v[2]));
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(n) : "v"(m), "v"(v[3]), "v"(v[4]));
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(p) : "v"(n), "v"(v[5]), "v"(v[6]));
  asm("v_max_f32_e64 %0, %1, |%2|" : "=v"(m) : "v"(p), "v"(v[7]));
  return m;
}

// signed extremes of v[0..7]
__device__ __forceinline__ float max8(const float v[8]) {
  float m, n, p;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(v[0]), "v"(v[1]), "v"(v[2]));
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(n) : "v"(m), "v"(v[3]), "v"(v[4]));
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(p) : "v"(n), "v"(v[5]), "v"(v[6]));
  asm("v_max_f32_e32 %0, %1, %2" : "=v"(m) : "v"(p), "v"(v[7]));
  return m;
}
__device__ __forceinline__ float min8(const float v[8]) {
  float m, n, p;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(v[0]), "v"(v[1]), "v"(v[2]));
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(n) : "v"(m), "v"(v[3]), "v"(v[4]));
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(p) : "v"(n), "v"(v[5]), "v"(v[6]));
  asm("v_min_f32_e32 %0, %1, %2" : "=v"(m) : "v"(p), "v"(v[7]));
  return m;
}

// clamp to [lo, hi] without the canonicalising max the compiler adds in IEEE mode
__device__ __forceinline__ float med3_nc(float v, float lo, float hi) {
  float m;
  asm("v_med3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(v), "v"(lo), "v"(hi));
  return m;
}

__device__ __forceinline__ float max_nc(float a, float b) {
  float m;
  asm("v_max_f32_e32 %0, %1, %2" : "=v"(m) : "v"(a), "v"(b));
  return m;
}
__device__ __forceinline__ float min_nc(float a, float b) {
  float m;
  asm("v_min_f32_e32 %0, %1, %2" : "=v"(m) : "v"(a), "v"(b));
  return m;
}

// max over the GL lanes of a scale group of values that are >= 0 (absolute
// values): their bit patterns order like the values, so an integer max does
// it, and the compiler folds each lane exchange (DPP) into the max itself.
// The groups are the low lane bits; after the quad steps every lane of a quad
// holds the quad's max, so the half-row and row mirrors complete 8 and 16.
template <int GL>
__device__ __forceinline__ float group_absmax(float m) {
  uint32_t u = __float_as_uint(m);
  if constexpr (GL >= 2) u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));
  if constexpr (GL >= 4) u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));
  if constexpr (GL >= 8) u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, false));
  if constexpr (GL >= 16) u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, false));
  return __uint_as_float(u);
}

// max over the GL lanes of a scale group (GL in 1, 2, 4, 8, 16: the low lane bits)
template <int GL>
__device__ __forceinline__ float group_max(float m) {
  if constexpr (GL >= 2) m = max_nc(m, dpp_xor1(m));
  if constexpr (GL >= 4) m = max_nc(m, dpp_xor2(m));
  if constexpr (GL >= 8) m = max_nc(m, swz_xor(m, 4));
  if constexpr (GL >= 16) m = max_nc(m, dpp_ror8(m));
  return m;
}

__device__ __forceinline__ float group_max_rt(float m, int gl) {
  if (gl >= 2) m = max_nc(m, dpp_xor1(m));
  if (gl >= 4) m = max_nc(m, dpp_xor2(m));
  if (gl >= 8) m = max_nc(m, swz_xor(m, 4));
  if (gl >= 16) m = max_nc(m, dpp_ror8(m));
  return m;
}

// (a, b) -> (a.lo | b.lo, a.hi | b.hi) over 32-lane halves; returns a' + b'.
__device__ __forceinline__ float swap32_add(float a, float b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __fadd_rn(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float swap16_add(float a, float b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __fadd_rn(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Transposed cascade over the NB row-block lane bits (5, 4, 3, 2 in that order)
// of 8 per-column lane values. Every addition joins two complete subtrees of
// the row order, so the result is the pairwise sum over all rows of the
// wavefront. On return v[0..(8 >> min(NB,3)) - 1] hold full sums; slot s of lane
// l holds column  s + 2*bit4(l) + 4*bit5(l)  (NB == 2), or
//                 bit3(l) + 2*bit4(l) + 4*bit5(l)  (NB >= 3).
template <int NB>
__device__ __forceinline__ void xtree(float v[8], int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = swap32_add(v[j], v[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) v[j] = swap16_add(v[j], v[j + 2]);
  if constexpr (NB >= 3) {
    const bool b3 = (lane & 8) != 0;
    const float keep = b3 ? v[1] : v[0];
    const float send = b3 ? v[0] : v[1];
    v[0] = __fadd_rn(keep, dpp_ror8(send));
  }
  if constexpr (NB >= 4) v[0] = __fadd_rn(v[0], swz_xor(v[0], 4));
}

// Sum of one value per row lane over the NB row-lane bits, in the order of
// xtree (lane bit 5 first, which carries the lowest row-block bit): the
// pairwise row order of the retrieval. Every lane gets the sum.
template <int NB>
__device__ __forceinline__ float row_lane_sum(float d) {
  d = __fadd_rn(d, __shfl_xor(d, 32, 64));
  if constexpr (NB >= 2) d = __fadd_rn(d, __shfl_xor(d, 16, 64));
  if constexpr (NB >= 3) d = __fadd_rn(d, dpp_ror8(d));
  if constexpr (NB >= 4) d = __fadd_rn(d, swz_xor(d, 4));
  return d;
}

// Column (0..7, inside the lane's column block) held in slot s after xtree.
template <int NB>
__device__ __forceinline__ int xtree_col(int s, int lane) {
  const int b4 = (lane >> 4) & 1, b5 = (lane >> 5) & 1;
  if constexpr (NB >= 3) return ((lane >> 3) & 1) + 2 * b4 + 4 * b5;
  return s + 2 * b4 + 4 * b5;
}

}  // namespace rsq
