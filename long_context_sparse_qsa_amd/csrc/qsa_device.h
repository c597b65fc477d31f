// Device helpers shared by the QSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kIndexDim = 128;
constexpr int kIndexHeads = 4;
constexpr int kBlockTokens = 4;
constexpr int kWave = 64;
constexpr int kMaxSegments = 16;

// Element types.  bf16 values are carried as raw 16-bit patterns.
struct F32 {
  using T = float;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float to_f(T x) { return x; }
  __device__ static __forceinline__ T from_f(float x) { return x; }
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round-to-nearest-even float32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct BF16 {
  using T = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float to_f(T x) { return bf16_bits_to_f32(x); }
  __device__ static __forceinline__ T from_f(float x) { return f32_to_bf16_bits(x); }
};

// Wave-wide reductions over 64 lanes through DPP moves (no LDS round
// trips): two quad permutations and the half-row and row mirrors combine
// each 16-lane row, row_bcast 15 and 31 carry rows 0-2 into row 3, and the
// last lane's value is returned (wave-uniform).  Every lane of the wave must
// be active.  Lanes a step does not update combine with the identity.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max_step(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), CTRL, ROWS,
                                                              0xF, false)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_sum_step(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_sum_step<0xB1, 0xF>(v);
  v = dpp_sum_step<0x4E, 0xF>(v);
  v = dpp_sum_step<0x141, 0xF>(v);
  v = dpp_sum_step<0x140, 0xF>(v);
  v = dpp_sum_step<0x142, 0xA>(v);
  v = dpp_sum_step<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Inclusive prefix sum over the 64 lanes of a wave, through DPP moves (no
// LDS round trips): row_shr 1, 2, 4, 8 scan each 16-lane row (a lane whose
// source lies outside its row adds the old value 0), then row_bcast 15 adds
// row 0's total to row 1 and row 2's to row 3, and row_bcast 31 adds the
// total of rows 0-1 to rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_add_step(uint32_t v) {
  return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int /*lane*/) {
  v = dpp_add_step<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add_step<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add_step<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add_step<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  return dpp_add_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
}

// Bitwise OR over the 64 lanes of a wave, through DPP moves: two quad
// permutations and the half-row and row mirrors give every lane its 16-lane
// row's OR, row_bcast 15 and 31 carry rows 0-2 into row 3, whose last lane is
// read (the result is wave-uniform).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_or_step(uint32_t v) {
  return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v = dpp_or_step<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_or_step<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_or_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_or_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_or_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_or_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// x plus the value of the lane whose index differs in bit 0 (XOR1) or bit 1,
// within a quad of lanes: one DPP quad permutation, no LDS round trip.
template <int XOR>
__device__ __forceinline__ float quad_xor_add(float x) {
  constexpr int kCtrl = XOR == 1 ? 0xB1 : 0x4E;  // quad_perm [1, 0, 3, 2] or [2, 3, 0, 1]
  static_assert(XOR == 1 || XOR == 2, "quad lanes");
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Make a value known to be wave-uniform visible as such to the compiler, so
// that loads addressed by it become scalar loads.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Pooled key element of one block: (((x0 + x1) + x2) + x3) * 0.25 in float32,
// fixed order, IEEE round-to-nearest-even, no contraction.
__device__ __forceinline__ float pool4(float x0, float x1, float x2, float x3) {
  float acc = __fadd_rn(x0, x1);
  acc = __fadd_rn(acc, x2);
  acc = __fadd_rn(acc, x3);
  return __fmul_rn(acc, 0.25f);
}

__device__ __forceinline__ int64_t clamp_nb(int64_t pos, int64_t nb_max) {
  int64_t nb = (pos + 1) / kBlockTokens;
  if (nb < 0) nb = 0;
  return nb < nb_max ? nb : nb_max;
}

}  // namespace qsa
