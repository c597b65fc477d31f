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
//   [0, kCtlWords)       word kPathWord: how the last selection of the row went;
//                        word kArriveWord: chunk arrivals of the selection launch;
//                        word kThrWord: the row's candidate threshold digit
//   cnt_off + c          candidate count of 4,096-block chunk c
//   key_off + c*kChunk   candidate keys of chunk c, ascending block order
//   id_off  + c*kChunk   their block ids
//   sample_off + g       sampled score of 16-block group g
constexpr int kCtlWords = 64;
constexpr int kPathWord = 0;
// Arrival counter of the row's chunk workgroups in the selection launch:
// cleared by the pass that writes the row's sample, and by the last arrival.
constexpr int kArriveWord = 1;
// The row's candidate threshold digit, when a launch of its own computes it
// (many rows: the collect workgroups then read one word instead of the
// row's whole sample).
constexpr int kThrWord = 2;
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

// Memory-flat score -> top-k (many rows, no score matrix): per-call
// workspace, in 32-bit words.  Per row: its threshold digit, its candidate
// count (an atomic append counter), the path its selection took, its score
// sample (one per 16-block group) and kFlatCap candidate slots in no
// particular order, each slot a (key, block id) pair of two words.
constexpr int kFlatCap = 4096;
struct FlatLayout {
  int64_t thr, cnt, path, samples, pairs, total;
};
__host__ __device__ inline FlatLayout flat_layout(int64_t M, int64_t nb_max) {
  FlatLayout L;
  int64_t o = 0;
  L.thr = o;
  o += round64(M);
  L.cnt = o;
  o += round64(M);
  L.path = o;
  o += round64(M);
  L.samples = o;
  o += round64(M * sample_groups(nb_max));
  L.pairs = o;
  o += M * kFlatCap * 2;
  L.total = o;
  return L;
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


template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) sh[wave] = incl;
  __syncthreads();
  // every wave reads the wave totals itself (no second scan pass)
  uint32_t before = 0u, tot = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = sh[w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  total = tot;
  __syncthreads();  // sh is free for the next scan
  return before + incl - v;
}

// Counts in LDS, C copies per bin (cnt[bin * C + copy]; digit order
// ascending): find the digit where the count from the top reaches `want`.
// out3 = {digit, want - count above the digit, 0}; out3[2] = 1 when the
// total stays below `want`.  One wave does it, with no workgroup barrier
// inside: lane l sums the run of NBINS / 64 bins l-th from the top (its
// reads rotated by lane, so lanes spread over the banks), a wave scan finds
// the run that crosses `want`, and the lanes then take that run's bins one
// each.  The caller makes the counts visible first (a barrier); the function
// ends with one.
template <int NBINS, int C = 1>
__device__ void find_digit_desc(const uint32_t* cnt, uint32_t want, uint32_t* out3) {
  static_assert(NBINS % kWave == 0 && NBINS / kWave <= kWave, "one run of bins per lane");
  constexpr int R = NBINS / kWave;  // bins per lane
  constexpr int W = R * C;          // words per lane
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    const uint32_t* run = cnt + (NBINS - (l + 1) * R) * C;
    uint32_t c = 0u;
    if constexpr (W % 4 == 0) {
      constexpr int Q = W / 4;
#pragma unroll
      for (int j = 0; j < Q; ++j) {
        const uint4 x = reinterpret_cast<const uint4*>(run)[(j + l) % Q];
        c += (x.x + x.y) + (x.z + x.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < W; ++j) c += run[j];
    }
    const uint32_t incl = wave_incl_scan(c, l);
    // counts are non-negative: the first lane whose inclusive count reaches
    // want holds the digit
    const uint64_t hit = __ballot(incl >= want);
    if (hit == 0u) {
      if (l == 0) {
        out3[0] = 0u;
        out3[1] = want;
        out3[2] = 1u;
      }
    } else {
      const int L = __ffsll((unsigned long long)hit) - 1;
      const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(incl - c), L);  // L is wave-uniform
      const int top = NBINS - L * R - 1;  // the run's top bin
      uint32_t v = 0u;
      if (l < R) {
#pragma unroll
        for (int e = 0; e < C; ++e) v += cnt[(top - l) * C + e];
      }
      const uint32_t vi = wave_incl_scan(v, l);
      const uint64_t h2 = __ballot(l < R && above + vi >= want);
      if (l == __ffsll((unsigned long long)h2) - 1) {
        out3[0] = (uint32_t)(top - l);
        out3[1] = want - (above + vi - v);
        out3[2] = 0u;
      }
    }
  }
  __syncthreads();
}

// Exact top-k of a whole row: four 8-bit radix passes over all keys (16
// copies of each 256-bin histogram against atomic contention), then an
// order-preserving compaction in index order (ties go to the lower index).
// Src(i) gives block i's score; Sm provides hist16[4096], scan_sh
// and out3 in LDS.
struct ScoreArray {
  const float* __restrict__ s;
  __device__ __forceinline__ float operator()(int64_t i) const { return s[i]; }
};

template <int NT, class Src, class Sm>
__device__ void exact_select(const Src& src, int64_t nb, int k, int32_t* out, Sm& sm) {
  constexpr int kBins = 256, kCopies = 16;
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t prefix = 0, mask = 0, want = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < kBins * kCopies; i += NT) sm.hist16[i] = 0u;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < nb; i += NT) {
      const uint32_t u = order_key(src(i));
      if ((u & mask) == prefix) atomicAdd(&sm.hist16[((u >> shift) & 0xffu) * kCopies + (lane & (kCopies - 1))], 1u);
    }
    __syncthreads();
    find_digit_desc<kBins, kCopies>(sm.hist16, want, sm.out3);
    prefix |= sm.out3[0] << shift;
    mask |= 0xffu << shift;
    want = sm.out3[1];
    __syncthreads();
  }
  const uint32_t T = prefix, need = want;
  uint32_t base_out = 0, base_eq = 0;
  for (int64_t c0 = 0; c0 < nb; c0 += (int64_t)NT * 4) {
    const int64_t i0 = c0 + (int64_t)threadIdx.x * 4;
    uint32_t gt[4], eq[4], n_eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + e;
      const uint32_t u = i < nb ? order_key(src(i)) : 0u;
      gt[e] = (i < nb) && (u > T);
      eq[e] = (i < nb) && (u == T);
      n_eq += eq[e];
    }
    uint32_t tot_eq, tot_take;
    uint32_t eq_rank = base_eq + block_excl_scan<NT>(n_eq, sm.scan_sh, tot_eq);
    uint32_t take[4], n_take = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      take[e] = gt[e] || (eq[e] && eq_rank < need);
      eq_rank += eq[e];
      n_take += take[e];
    }
    uint32_t pos = base_out + block_excl_scan<NT>(n_take, sm.scan_sh, tot_take);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (take[e] && pos < (uint32_t)k) out[pos] = (int32_t)(i0 + e);
      pos += take[e];
    }
    base_out += tot_take;
    base_eq += tot_eq;
  }
}


// Thresholds come from a histogram of the sample over a window of 256
// digits: scores from 2^-16 to 2^16 at 8 bins per octave; lower digits share
// the first bin and higher ones the last.  A threshold is an estimate, so
// saturation only makes it more conservative (the selection is exact
// regardless).
constexpr int kWinBins = 256;
constexpr uint32_t kWinBase = 0x800u + (127u - 16u) * 8u;  // digit of 2^-16
__device__ __forceinline__ uint32_t win_bin(uint32_t key) {
  const uint32_t d = key >> kDigitShift;
  return d < kWinBase ? 0u : (d - kWinBase < (uint32_t)kWinBins ? d - kWinBase : (uint32_t)kWinBins - 1u);
}

}  // namespace sel
}  // namespace qsa
