// Pieces of the top-k selection shared by the scoring kernel (which writes
// each row's score sample in its epilogue) and the selection kernels.
#pragma once

#include "qsa_device.h"

namespace qsa {
namespace sel {

constexpr int kDigitBits = 12;                 // top key bits per histogram bin
constexpr int kDigits = 1 << kDigitBits;       // 4,096 bins, 8 per octave of positive scores
constexpr int kDigitShift = 32 - kDigitBits;
constexpr int kChunk = 4096;                   // blocks per collect workgroup
constexpr int kMaxChunks = 64;                 // rows of <= 262,144 blocks take the candidate path
constexpr int kCandMax = 4096;                 // candidates the finalize pass holds on chip

// Per-row workspace record (32-bit words, every part 256-byte aligned);
// nothing in it needs to start at any particular value:
//   [0, kCtlWords)       word kPathWord: how the last selection of the row went
//   cnt_off + c          candidate count of 4,096-block chunk c
//   key_off + c*kChunk   candidate keys of chunk c, ascending block order
//   id_off  + c*kChunk   their block ids
//   sample_off + g       sampled score of 16-block group g
constexpr int kCtlWords = 64;
constexpr int kPathWord = 0;
// Selection paths (a diagnostic: every path gives the same exact result).
enum SelPath : uint32_t {
  kPathAll = 1,         // at most k blocks: all kept
  kPathCandidates = 2,  // from the conservative candidates
  kPathExactChunks = 3, // exact whole-row select: more than kMaxChunks chunks
  kPathExactCount = 4,  // exact whole-row select: candidate count below k or above kCandMax
};
__host__ __device__ constexpr int64_t round64(int64_t x) { return (x + 63) / 64 * 64; }
__host__ __device__ constexpr int64_t n_chunks(int64_t nb_max) { return (nb_max + kChunk - 1) / kChunk; }
__host__ __device__ constexpr int64_t sample_groups(int64_t nb_max) { return (nb_max + 15) / 16; }
__host__ __device__ constexpr int64_t cnt_off(int64_t) { return kCtlWords; }
__host__ __device__ constexpr int64_t key_off(int64_t nb_max) { return cnt_off(nb_max) + round64(n_chunks(nb_max)); }
__host__ __device__ constexpr int64_t id_off(int64_t nb_max) { return key_off(nb_max) + round64(nb_max); }
__host__ __device__ constexpr int64_t sample_off(int64_t nb_max) { return id_off(nb_max) + round64(nb_max); }
__host__ __device__ constexpr int64_t row_words(int64_t nb_max) {
  return sample_off(nb_max) + round64(sample_groups(nb_max));
}

// The sample: exactly one block of every 16-block group, at a hashed
// offset, so a group's sample has a fixed slot (its group index).  The collect
// pass turns the samples into a conservative threshold (about 1.25 k + 256
// blocks expected at or above it) and the finalize pass selects exactly.
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
