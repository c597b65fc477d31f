// Pieces of the top-k selection shared by the scoring kernel (which writes
// each row's score sample in its epilogue) and the selection kernels.
#pragma once

#include "qsa_device.h"

namespace qsa {
namespace sel {

constexpr int kDigitBits = 12;                 // top key bits per histogram bin
constexpr int kDigits = 1 << kDigitBits;       // 4,096 bins, 8 per octave of positive scores
constexpr int kDigitShift = 32 - kDigitBits;
constexpr int kCandMax = 4096;                 // candidate (key, id) pairs per row

// Per-row workspace record (32-bit words); nothing in it needs to start at
// any particular value:
//   0                 candidate count (zeroed by the sample producer)
//   1..7              reserved
//   8 ...             candidate keys [kCandMax], then candidate ids [kCandMax]
//   kSamples ...      one sampled score per 16-block group [ceil(nb_max / 16)]
struct RowWs {
  static constexpr int kCount = 0;
  static constexpr int kKeys = 8;
  static constexpr int kIds = kKeys + kCandMax;
  static constexpr int kSamples = kIds + kCandMax;
};
__host__ __device__ constexpr int64_t sample_groups(int64_t nb_max) { return (nb_max + 15) / 16; }
__host__ __device__ constexpr int64_t row_words(int64_t nb_max) {
  return (RowWs::kSamples + sample_groups(nb_max) + 63) / 64 * 64;  // 256-byte records
}

// The sample: exactly one block of every 16-block group, at a hashed offset,
// so a group's sample has a fixed slot (its group index).  The collect pass
// turns the samples into a conservative threshold (about 1.25 k + 256 blocks
// expected at or above it) and the finalize pass selects exactly.
__host__ __device__ constexpr uint32_t sample_offset(uint32_t group) { return (group * 2654435761u) >> 28; }
__host__ __device__ constexpr bool sampled(uint32_t block) { return (block & 15u) == sample_offset(block >> 4); }
__host__ __device__ constexpr uint32_t sample_target(uint32_t k) { return (k + k / 4) / 16u + 16u; }

// Order-preserving 32-bit key of a float32 score (-0 folded into +0).
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

}  // namespace sel
}  // namespace qsa
