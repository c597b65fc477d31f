// Top-k block selection (hipfire "QSA sparse attention ...", section 02:
// keep the top-scoring blocks within the token budget; section 03: a radix
// select follows the scoring; section 06: long score rows no longer fit the
// selector's on-chip memory).  Equal scores go to the lower block index.
//
// Scores map to order-preserving 32-bit keys (-0 folded into +0); the top 12
// key bits are a histogram digit (8 bins per octave of positive scores).  The
// work is spread over many compute units, with kernel boundaries (not fences)
// ordering the passes:
//
//  sample   (standalone selection only; the scoring kernel does the same in
//           its epilogue) one block of every 16-block group, at a hashed
//           offset, has its score copied to the group's slot in the row's
//           workspace record.
//  collect  one workgroup per 4,096-block chunk of a row histograms the row's
//           samples in LDS and walks the histogram from the top to the digit
//           B where the sample count reaches (1.25 k + 256) / 16: a
//           conservative threshold, about 1.25 k + 256 blocks are expected at
//           or above it.  The chunk's (key, id) pairs with digit >= B go to
//           the chunk's own slots in ascending block order (a block scan
//           places them; no atomics).
//  finalize one workgroup per row gathers the chunks' candidates (ascending
//           block order) and finds the k-th largest candidate key TK with
//           three histogram levels (12, 10 and 10 key bits; each level counts
//           only the candidates sharing the bits found so far).  Keys above TK
//           are kept, and of the keys equal to TK the first ones in block
//           order; a block scan writes the kept ids in ascending order.  A
//           candidate list shorter than k (the sample misled the threshold),
//           one longer than the on-chip list (massive ties) or a row of more
//           than 64 chunks takes an exact radix select over the whole row in
//           the same workgroup, so the result is exact in every case.
//
// Calls of 256 rows and more take a one-launch variant with one workgroup
// per row instead of collect + finalize (below).
//
// The workspace holds one record per row (sel::row_words); no part of it
// needs initialising.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "select_common.h"

namespace qsa {

namespace {

using sel::kCandMax;
using sel::kChunk;
using sel::kDigits;
using sel::kDigitShift;
using sel::kMaxChunks;
using sel::order_key;

constexpr int kBins = 256;
constexpr int kCopies = 16;
constexpr int kChunkThreads = 256;
constexpr int kChunkPer = kChunk / kChunkThreads;  // 16 consecutive scores per lane
constexpr int kFinThreads = 512;
constexpr int kFinPer = kCandMax / kFinThreads;    // 8 candidates per thread
constexpr int kLowBins = 1024;                     // 10-bit digits below the 12-bit one
using sel::kWinBase;
using sel::kWinBins;
using sel::win_bin;
static_assert(kChunkPer % 4 == 0, "float4 score loads");

using sel::block_excl_scan;
using sel::find_digit_desc;

struct FinSmem {
  uint32_t hist16[kBins * kCopies];  // exact-path radix passes; also the 12-bit digit histogram
  uint32_t h2[kLowBins];             // bits 19..10 of the cut-digit keys
  uint32_t h3[kLowBins];             // bits 9..0 of the cut keys
  uint32_t ck[kCandMax];             // candidate keys, ascending block order
  uint32_t ci[kCandMax];             // their block ids
  uint32_t coff[kMaxChunks + 1];     // chunk offsets into the candidate list
  uint32_t scan_sh[2 * (kFinThreads / kWave)];
  uint32_t out3[3];
  uint32_t cmax;                     // largest chunk count
};
static_assert(kDigits == kBins * kCopies, "the digit histogram reuses the radix histogram");

// Exact path over the whole row (select_common.h) reading the score array.
__device__ __forceinline__ void exact_row_select(const float* __restrict__ s, int64_t nb, int k, int32_t* out,
                                                 FinSmem& sm) {
  sel::exact_select<kFinThreads>(sel::ScoreArray{s}, nb, k, out, sm);
}

// ---------------------------------------------------------------- kernels

// Standalone selection: write each row's sampled scores (one per 16-block
// group) into the workspace.
__global__ void __launch_bounds__(kChunkThreads)
select_sample_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                     int64_t nb_max, uint32_t* __restrict__ ws) {
  const int m = blockIdx.y;
  const int64_t grp = (int64_t)blockIdx.x * kChunkThreads + threadIdx.x;
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  const int64_t b = grp * 16 + sel::sample_offset((uint32_t)grp);
  if (b < nb) reinterpret_cast<float*>(W)[sel::sample_off(nb_max) + grp] = scores[(int64_t)m * ld + b];
}

__global__ void __launch_bounds__(kChunkThreads)
select_collect_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                      int64_t nb_max, int k, uint32_t* __restrict__ ws) {
  __shared__ uint32_t h[kWinBins];
  __shared__ uint32_t scan_sh[2 * (kChunkThreads / kWave)];
  __shared__ uint32_t out3[3];
  const int m = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)c * kChunk;
  const float* __restrict__ s = scores + (int64_t)m * ld;
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  const float* __restrict__ smp = reinterpret_cast<const float*>(W + sel::sample_off(nb_max));
  const int64_t n_grp = sel::sample_groups(nb_max);

  // every load this pass needs is independent: issue them together
  const int64_t i0 = base + (int64_t)tid * kChunkPer;  // this lane's 16 consecutive blocks
  float4 sv[kChunkPer / 4];
#pragma unroll
  for (int q = 0; q < kChunkPer / 4; ++q) {
    const int64_t j = i0 + 4 * q;  // rows are padded to a multiple of 4 floats
    sv[q] = j < nb_max ? *reinterpret_cast<const float4*>(s + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  constexpr int kSampPer = kChunk / kChunkThreads;  // samples per lane per round
  float smpv[kSampPer];
#pragma unroll
  for (int e = 0; e < kSampPer; ++e) {
    const int64_t gi = (int64_t)e * kChunkThreads + tid;
    smpv[e] = gi < n_grp ? smp[gi] : 0.f;
  }
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  for (int i = tid; i < kWinBins; i += kChunkThreads) h[i] = 0u;
  if (nb <= k || base >= nb) return;  // every block kept, or a chunk the finalize pass does not read
  __syncthreads();
  // histogram of the row's samples (blocks < nb only)
#pragma unroll
  for (int e = 0; e < kSampPer; ++e) {
    const int64_t gi = (int64_t)e * kChunkThreads + tid;
    if (gi < n_grp && gi * 16 + sel::sample_offset((uint32_t)gi) < nb)
      atomicAdd(&h[win_bin(order_key(smpv[e]))], 1u);
  }
  for (int64_t g0 = kChunk; g0 < n_grp; g0 += kChunk) {  // rows of more than 65,536 blocks
    float v[kSampPer];
#pragma unroll
    for (int e = 0; e < kSampPer; ++e) {
      const int64_t gi = g0 + (int64_t)e * kChunkThreads + tid;
      v[e] = gi < n_grp ? smp[gi] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kSampPer; ++e) {
      const int64_t gi = g0 + (int64_t)e * kChunkThreads + tid;
      if (gi < n_grp && gi * 16 + sel::sample_offset((uint32_t)gi) < nb)
        atomicAdd(&h[win_bin(order_key(v[e]))], 1u);
    }
  }
  __syncthreads();
  // conservative threshold (not reached: every block is a candidate)
  find_digit_desc<kWinBins>(h, sel::sample_target((uint32_t)k), out3);
  // window bin 0 (or a target never reached): every block is a candidate
  const uint32_t B = (out3[2] || out3[0] == 0u) ? 0u : kWinBase + out3[0];

  uint32_t key[kChunkPer];
  uint32_t flags = 0u;
#pragma unroll
  for (int q = 0; q < kChunkPer / 4; ++q) {
    key[4 * q + 0] = order_key(sv[q].x);
    key[4 * q + 1] = order_key(sv[q].y);
    key[4 * q + 2] = order_key(sv[q].z);
    key[4 * q + 3] = order_key(sv[q].w);
  }
#pragma unroll
  for (int e = 0; e < kChunkPer; ++e)
    if (i0 + e < nb && (key[e] >> kDigitShift) >= B) flags |= 1u << e;
  // the chunk's candidates in ascending block order, in the chunk's own slots
  uint32_t total;
  uint32_t pos = block_excl_scan<kChunkThreads>((uint32_t)__popc(flags), scan_sh, total);
  uint32_t* K = W + sel::key_off(nb_max) + base;
  uint32_t* I = W + sel::id_off(nb_max) + base;
#pragma unroll
  for (int e = 0; e < kChunkPer; ++e) {
    if ((flags >> e) & 1u) {
      if (pos < (uint32_t)kChunk) {  // the chunk's own slots (a scan result never leaves them)
        K[pos] = key[e];
        I[pos] = (uint32_t)(i0 + e);
      }
      ++pos;
    }
  }
  if (tid == 0) W[sel::cnt_off(nb_max) + c] = total;
}

__global__ void __launch_bounds__(kFinThreads)
select_finalize_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                       int64_t nb_max, int k, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                       uint32_t* __restrict__ ws) {
  __shared__ FinSmem sm;
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const float* __restrict__ s = scores + (int64_t)m * ld;
  int32_t* __restrict__ out = sel + (int64_t)m * k;
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  // Every chunk count of the row is written by the collect pass whenever the
  // candidate path runs.  The counts and the first C slots of every chunk
  // (C = 4096 / the chunk count rounded up to a power of two) are loaded
  // before the row position arrives; only a chunk holding more than C
  // candidates costs a second round trip.
  const int64_t nch_max = sel::n_chunks(nb_max);
  const int nchm = (int)(nch_max < kMaxChunks ? nch_max : kMaxChunks);
  int lgc = 0;
  while ((1 << lgc) < nchm) ++lgc;
  const int lgC = 12 - lgc;  // log2 of C; kCandMax = 4096
  static_assert(kCandMax == 4096, "speculative slot split");
  const uint32_t* K = W + sel::key_off(nb_max);
  const uint32_t* I = W + sel::id_off(nb_max);
  uint32_t kk[kFinPer], ii[kFinPer];
#pragma unroll
  for (int e = 0; e < kFinPer; ++e) {
    const int q = e * kFinThreads + tid;
    const int c = q >> lgC;
    const int64_t slot = (int64_t)c * kChunk + (q & ((1 << lgC) - 1));
    const int64_t at = (c < nchm && slot < nb_max) ? slot : 0;
    kk[e] = K[at];
    ii[e] = I[at];
  }
  const uint32_t cnt_raw = (tid < kWave && tid < nchm) ? W[sel::cnt_off(nb_max) + tid] : 0u;
  if (nb <= k) {
    for (int i = tid; i < k; i += kFinThreads) out[i] = i < nb ? i : -1;
    if (tid == 0) {
      n_sel[m] = (int32_t)nb;
      W[sel::kPathWord] = sel::kPathAll;
    }
    return;
  }
  if (tid == 0) n_sel[m] = k;
  const int nch = (int)((nb + kChunk - 1) / kChunk);
  if (nch > kMaxChunks) {
    if (tid == 0) W[sel::kPathWord] = sel::kPathExactChunks;
    exact_row_select(s, nb, k, out, sm);
    return;
  }
  for (int i = tid; i < kDigits; i += kFinThreads) sm.hist16[i] = 0u;
  for (int i = tid; i < kLowBins; i += kFinThreads) {
    sm.h2[i] = 0u;
    sm.h3[i] = 0u;
  }
  if (tid < kWave) {  // chunk offsets (nch <= 64: one wave)
    const uint32_t cnt = tid < nch ? cnt_raw : 0u;
    const uint32_t incl = wave_incl_scan(cnt, lane);
    sm.coff[lane + 1] = incl;
    if (lane == 0) sm.coff[0] = 0u;
    const uint32_t mx = (uint32_t)wave_max((float)cnt);  // counts <= 4096: exact in float
    if (lane == 0) sm.cmax = mx;
  }
  __syncthreads();
  const uint32_t n_cand = sm.coff[nch];
  if (n_cand < (uint32_t)k || n_cand > (uint32_t)kCandMax) {
    if (tid == 0) W[sel::kPathWord] = sel::kPathExactCount;
    exact_row_select(s, nb, k, out, sm);
    return;
  }
  if (tid == 0) W[sel::kPathWord] = sel::kPathCandidates;

  // place the candidates in chunk order (= ascending block order)
  uint32_t vm = 0u;  // which of kk/ii hold a candidate
  if (sm.cmax <= (1u << lgC)) {
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      const int q = e * kFinThreads + tid;
      const int c = q >> lgC;
      const uint32_t j = (uint32_t)(q & ((1 << lgC) - 1));
      if (c < nch && j < sm.coff[c + 1] - sm.coff[c]) {
        const uint32_t i = sm.coff[c] + j;
        sm.ck[i] = kk[e];
        sm.ci[i] = ii[e];
        atomicAdd(&sm.hist16[kk[e] >> kDigitShift], 1u);
        vm |= 1u << e;
      }
    }
  } else {
    // a chunk overflowed its speculative share: gather by candidate index
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      const uint32_t i = (uint32_t)(e * kFinThreads + tid);
      // chunk of candidate i: the last c with coff[c] <= i
      int lo = 0, hi = nch;  // coff[lo] <= i < coff[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sm.coff[mid] <= i) lo = mid; else hi = mid;
      }
      const bool live = i < n_cand;
      const int64_t slot = live ? (int64_t)lo * kChunk + (i - sm.coff[lo]) : 0;
      kk[e] = K[slot];
      ii[e] = I[slot];
      vm |= live ? (1u << e) : 0u;
    }
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      const uint32_t i = (uint32_t)(e * kFinThreads + tid);
      if ((vm >> e) & 1u) {
        sm.ck[i] = kk[e];
        sm.ci[i] = ii[e];
        atomicAdd(&sm.hist16[kk[e] >> kDigitShift], 1u);
      }
    }
  }
  __syncthreads();
  // The k-th largest candidate key, 12 + 10 + 10 bits at a time; each level
  // histograms only the candidates that share the bits found so far, and the
  // search stops as soon as the cut bin is kept whole.  Then a key is kept if
  // (key >> shift) > prefix, or == prefix and (whole, or among the first
  // `need` such keys in block order).
  find_digit_desc<kDigits>(sm.hist16, (uint32_t)k, sm.out3);
  uint32_t prefix = sm.out3[0];
  uint32_t need = sm.out3[1];
  int shift = kDigitShift;
  bool whole = sm.hist16[prefix] == need;
  if (!whole) {
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      if (((vm >> e) & 1u) && (kk[e] >> kDigitShift) == prefix) atomicAdd(&sm.h2[(kk[e] >> 10) & (kLowBins - 1)], 1u);
    }
    __syncthreads();
    find_digit_desc<kLowBins>(sm.h2, need, sm.out3);
    const uint32_t d2 = sm.out3[0];
    prefix = (prefix << 10) | d2;
    need = sm.out3[1];
    shift = 10;
    whole = sm.h2[d2] == need;
  }
  if (!whole) {
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      if (((vm >> e) & 1u) && (kk[e] >> 10) == prefix) atomicAdd(&sm.h3[kk[e] & (kLowBins - 1)], 1u);
    }
    __syncthreads();
    find_digit_desc<kLowBins>(sm.h3, need, sm.out3);
    const uint32_t d3 = sm.out3[0];
    prefix = (prefix << 10) | d3;
    need = sm.out3[1];
    shift = 0;
    whole = sm.h3[d3] == need;
  }

  // keep flags over contiguous ranges of the (ascending) candidate list
  const uint32_t r0 = (uint32_t)tid * kFinPer;
  static_assert(kFinPer == 8, "two 16-byte LDS reads per thread");
  uint32_t key[kFinPer], cid[kFinPer];
  {
    const uint4 a0 = *reinterpret_cast<const uint4*>(&sm.ck[r0]);
    const uint4 a1 = *reinterpret_cast<const uint4*>(&sm.ck[r0 + 4]);
    const uint4 b0 = *reinterpret_cast<const uint4*>(&sm.ci[r0]);
    const uint4 b1 = *reinterpret_cast<const uint4*>(&sm.ci[r0 + 4]);
    key[0] = a0.x; key[1] = a0.y; key[2] = a0.z; key[3] = a0.w;
    key[4] = a1.x; key[5] = a1.y; key[6] = a1.z; key[7] = a1.w;
    cid[0] = b0.x; cid[1] = b0.y; cid[2] = b0.z; cid[3] = b0.w;
    cid[4] = b1.x; cid[5] = b1.y; cid[6] = b1.z; cid[7] = b1.w;
  }
  uint32_t keep = 0u, n_keep = 0u, tot;
  if (whole) {
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      const bool kp = r0 + e < n_cand && (key[e] >> shift) >= prefix;
      keep |= kp ? (1u << e) : 0u;
      n_keep += kp ? 1u : 0u;
    }
  } else {
    // equal keys straddle the cut: the first `need` of them in block order
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) n_eq += (r0 + e < n_cand && key[e] == prefix) ? 1u : 0u;
    uint32_t eq_rank = block_excl_scan<kFinThreads>(n_eq, sm.scan_sh, tot);
#pragma unroll
    for (int e = 0; e < kFinPer; ++e) {
      bool kp = r0 + e < n_cand && key[e] > prefix;
      if (r0 + e < n_cand && key[e] == prefix) kp = eq_rank++ < need;
      keep |= kp ? (1u << e) : 0u;
      n_keep += kp ? 1u : 0u;
    }
  }
  // kept candidates are already in ascending block order: compact them
  uint32_t pos = block_excl_scan<kFinThreads>(n_keep, sm.scan_sh, tot);
#pragma unroll
  for (int e = 0; e < kFinPer; ++e) {
    if ((keep >> e) & 1u) {
      if (pos < (uint32_t)k) out[pos] = (int32_t)cid[e];
      ++pos;
    }
  }
}

// ---------------------------------------------------------------- one workgroup per row
//
// For many rows (a workgroup per row fills the GPU) the collect and
// finalize passes run in one launch, one workgroup per row: every
// load is issued first (the row's sample and up to 65,536 scores, 16 bytes per
// load, 32 per thread); the sample's window histogram gives the threshold
// digit B as in the collect pass; each thread marks which of its loads hold a
// block at or above B, those loads go to a list, the workgroup re-reads them
// (cached) and appends their candidates (key, id) in LDS with their 12-bit
// digit counts; the 12/10/10-bit levels find the k-th key TK; keys above TK
// and the lowest-id keys equal to TK are marked in a bitmap of the row's
// blocks, which gives the kept ids in ascending order.  A candidate count
// outside [k, kCandMax], more keys equal to TK than the tie list holds, or a
// row longer than the bitmap take the exact whole-row select.  With few rows
// the two-pass path is faster: one compute unit streams a row at only
// ~40 GB/s (19 vs 13 us at 4 rows of 65,280 blocks), and a short row's
// zeroing and level passes outweigh the saved launch.
constexpr int kRowThreads = 512;
constexpr int kRowF4 = 32;                         // 16-byte score loads per thread per round
constexpr int kRoundBlocks = kRowThreads * kRowF4 * 4;  // 65,536
constexpr int kSmpPer = 8;                         // sample loads per thread per round (4,096 groups)
constexpr int kPairPer = sel::kCandMax / kRowThreads;  // listed loads per thread (8)
constexpr int kRowLowBins = 1024;                  // 10-bit digits below the 12-bit one
constexpr int kMaxTies = 512;                      // keys equal to TK ranked on chip
constexpr int64_t kRowMaxBlocks = (int64_t)kMaxChunks * kChunk;  // 262,144
constexpr int kBitWords = (int)(kRowMaxBlocks / 32);
constexpr int kSmpCopies = 16;                     // copies of the sample histogram against contention

struct RowSmem {
  uint32_t hist16[sel::kDigits];                  // the 12-bit digit histogram; the exact path's radix passes
  uint32_t smp_h[sel::kWinBins * kSmpCopies];   // the sample histogram
  uint32_t h2[kRowLowBins];                     // bits 19..10 of the cut-digit keys
  uint32_t h3[kRowLowBins];                     // bits 9..0 of the cut keys
  uint32_t ck[sel::kCandMax];                     // candidate keys (no particular order)
  uint32_t ci[sel::kCandMax];                     // their block ids
  uint32_t loads[sel::kCandMax];                  // 16-byte loads (index in the row) holding a candidate
  uint32_t bits[kBitWords];                  // kept blocks of the row
  uint32_t teq[kMaxTies];                    // ids of the keys equal to TK
  uint32_t scan_sh[2 * (kRowThreads / kWave)];
  uint32_t out3[3];
  uint32_t n_loads, n_cand, n_placed, n_eq;
};
static_assert(sizeof(RowSmem) <= 160 * 1024, "fits the LDS of one compute unit");

// 16-byte loads of one round: load j of thread t covers blocks
// 4 (r0 / 4 + j * kRowThreads + t) .. + 3 (rows are padded to 4 floats).
__device__ __forceinline__ void load_round(const float* __restrict__ s, int64_t nb_max, int64_t r0, int tid,
                                           float4 (&sv)[kRowF4]) {
#pragma unroll
  for (int j = 0; j < kRowF4; ++j) {
    const int64_t b = r0 + ((int64_t)j * kRowThreads + tid) * 4;
    sv[j] = b < nb_max ? *reinterpret_cast<const float4*>(s + b) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Which of the 4 blocks from b on are candidates: score >= f_min and block < nb.
__device__ __forceinline__ uint32_t cand4(const float4& v, float f_min, int64_t b, int64_t nb) {
  uint32_t m4 = (v.x >= f_min ? 1u : 0u) | (v.y >= f_min ? 2u : 0u) | (v.z >= f_min ? 4u : 0u) |
                (v.w >= f_min ? 8u : 0u);
  if (b + 4 > nb) m4 &= b >= nb ? 0u : (1u << (uint32_t)(nb - b)) - 1u;
  return m4;
}

// Wave-aggregated append: this lane's first slot of `n` in a list whose
// length counter lives in LDS.
__device__ __forceinline__ uint32_t wave_append(uint32_t n, uint32_t* counter) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t incl = wave_incl_scan(n, lane);
  const uint32_t wtot = (uint32_t)__shfl((int)incl, kWave - 1, kWave);
  uint32_t base = 0u;
  if (lane == 0 && wtot) base = atomicAdd(counter, wtot);
  return (uint32_t)__shfl((int)base, 0, kWave) + incl - n;
}

__global__ void __launch_bounds__(kRowThreads)
select_row_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                  int64_t nb_max, int k, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                  uint32_t* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char row_lds[];
  RowSmem& sm = *reinterpret_cast<RowSmem*>(row_lds);
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const float* __restrict__ s = scores + (int64_t)m * ld;
  int32_t* __restrict__ out = sel + (int64_t)m * k;
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  uint32_t* path = W + sel::kPathWord;
  const float* __restrict__ smp = reinterpret_cast<const float*>(W + sel::sample_off(nb_max));
  const int64_t n_grp = sel::sample_groups(nb_max);

  // every load of the first round at once: the position, the sample, the scores
  const int64_t p = row_pos[m];
  float smpv[kSmpPer];
#pragma unroll
  for (int e = 0; e < kSmpPer; ++e) {
    const int64_t gi = (int64_t)e * kRowThreads + tid;
    smpv[e] = gi < n_grp ? smp[gi] : 0.f;
  }
  float4 sv[kRowF4];
  load_round(s, nb_max, 0, tid, sv);
  const int64_t nb = clamp_nb(p, nb_max);
  if (nb <= k) {
    for (int i = tid; i < k; i += kRowThreads) out[i] = i < nb ? i : -1;
    if (tid == 0) {
      n_sel[m] = (int32_t)nb;
      *path = sel::kPathAll;
    }
    return;
  }
  if (tid == 0) n_sel[m] = k;
  if (nb > kRowMaxBlocks) {
    if (tid == 0) *path = sel::kPathExactChunks;
    sel::exact_select<kRowThreads>(sel::ScoreArray{s}, nb, k, out, sm);
    return;
  }
  const int bit_words = (int)((nb + 31) / 32);
  for (int i = tid; i < sel::kDigits; i += kRowThreads) {
    sm.hist16[i] = 0u;
    sm.smp_h[i] = 0u;
  }
  for (int i = tid; i < kRowLowBins; i += kRowThreads) {
    sm.h2[i] = 0u;
    sm.h3[i] = 0u;
  }
  for (int i = tid; i < bit_words; i += kRowThreads) sm.bits[i] = 0u;
  if (tid == 0) {
    sm.n_loads = 0u;
    sm.n_cand = 0u;
    sm.n_placed = 0u;
    sm.n_eq = 0u;
  }
  __syncthreads();

  // 1. the threshold digit B from the sample (blocks < nb only)
  for (int64_t g0 = 0; g0 < n_grp; g0 += (int64_t)kSmpPer * kRowThreads) {
    if (g0 > 0) {  // rows of more than 65,536 blocks
#pragma unroll
      for (int e = 0; e < kSmpPer; ++e) {
        const int64_t gi = g0 + (int64_t)e * kRowThreads + tid;
        smpv[e] = gi < n_grp ? smp[gi] : 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < kSmpPer; ++e) {
      const int64_t gi = g0 + (int64_t)e * kRowThreads + tid;
      if (gi < n_grp && gi * 16 + sel::sample_offset((uint32_t)gi) < nb)
        atomicAdd(&sm.smp_h[sel::win_bin(order_key(smpv[e])) * kSmpCopies + (tid & (kSmpCopies - 1))], 1u);
    }
  }
  __syncthreads();
  find_digit_desc<sel::kWinBins, kSmpCopies>(sm.smp_h, sel::sample_target((uint32_t)k), sm.out3);
  // window bin 0 (or a target never reached): every block is a candidate;
  // otherwise a block is one when its key's digit reaches B, i.e. its score
  // is at least the smallest positive float of digit B
  const uint32_t B = (sm.out3[2] || sm.out3[0] == 0u) ? 0u : sel::kWinBase + sm.out3[0];
  const float f_min = B == 0u ? -INFINITY : __uint_as_float((B << kDigitShift) & 0x7fffffffu);

  // 2. the 16-byte loads holding a candidate, round by round
  for (int64_t r0 = 0; r0 < nb; r0 += kRoundBlocks) {
    if (r0 > 0) load_round(s, nb_max, r0, tid, sv);
    uint32_t any = 0u, cnt = 0u;
#pragma unroll
    for (int j = 0; j < kRowF4; ++j) {
      const uint32_t m4 = cand4(sv[j], f_min, r0 + ((int64_t)j * kRowThreads + tid) * 4, nb);
      any |= (m4 != 0u ? 1u : 0u) << j;
      cnt += (uint32_t)__popc(m4);
    }
    wave_append(cnt, &sm.n_cand);
    uint32_t pos = wave_append((uint32_t)__popc(any), &sm.n_loads);
    while (any) {
      const int j = __ffs(any) - 1;
      any &= any - 1u;
      if (pos < (uint32_t)sel::kCandMax) sm.loads[pos] = (uint32_t)(r0 / 4 + (int64_t)j * kRowThreads + tid);
      ++pos;
    }
  }
  __syncthreads();
  const uint32_t n_cand = sm.n_cand;
  if (n_cand < (uint32_t)k || n_cand > (uint32_t)sel::kCandMax) {
    if (tid == 0) *path = sel::kPathExactCount;
    sel::exact_select<kRowThreads>(sel::ScoreArray{s}, nb, k, out, sm);
    return;
  }
  // 3. the listed loads again (cached now): their candidates into LDS, and
  // the candidates' 12-bit digit histogram (n_loads <= n_cand <= sel::kCandMax)
  const uint32_t n_loads = sm.n_loads;
  {
    uint32_t li[kPairPer];
    float4 lv[kPairPer];
#pragma unroll
    for (int e = 0; e < kPairPer; ++e) {
      const uint32_t i = (uint32_t)(e * kRowThreads + tid);
      li[e] = i < n_loads ? sm.loads[i] : 0u;
      lv[e] = *reinterpret_cast<const float4*>(s + 4 * (int64_t)li[e]);
    }
    uint32_t m4[kPairPer], cnt = 0u;
#pragma unroll
    for (int e = 0; e < kPairPer; ++e) {
      const uint32_t i = (uint32_t)(e * kRowThreads + tid);
      m4[e] = i < n_loads ? cand4(lv[e], f_min, 4 * (int64_t)li[e], nb) : 0u;
      cnt += (uint32_t)__popc(m4[e]);
    }
    uint32_t pos = wave_append(cnt, &sm.n_placed);
#pragma unroll
    for (int e = 0; e < kPairPer; ++e) {
      if ((uint32_t)(e * kRowThreads) >= n_loads) break;  // uniform
      const float c4[4] = {lv[e].x, lv[e].y, lv[e].z, lv[e].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (((m4[e] >> c) & 1u) && pos < (uint32_t)sel::kCandMax) {  // pos < n_cand: the same count as step 2
          const uint32_t key = order_key(c4[c]);
          sm.ck[pos] = key;
          sm.ci[pos] = 4u * li[e] + (uint32_t)c;
          atomicAdd(&sm.hist16[key >> kDigitShift], 1u);
          ++pos;
        }
      }
    }
  }
  __syncthreads();

  // 4. the k-th largest candidate key, 12 + 10 + 10 bits at a time; each
  // level counts only the candidates that share the bits found so far, and
  // the search stops once the cut bin is kept whole
  find_digit_desc<sel::kDigits>(sm.hist16, (uint32_t)k, sm.out3);
  uint32_t prefix = sm.out3[0];
  uint32_t need = sm.out3[1];
  int shift = kDigitShift;
  bool whole = sm.hist16[prefix] == need;
  if (!whole) {
    for (uint32_t i = tid; i < n_cand; i += kRowThreads) {
      const uint32_t key = sm.ck[i];
      if ((key >> kDigitShift) == prefix) atomicAdd(&sm.h2[(key >> 10) & (kRowLowBins - 1)], 1u);
    }
    __syncthreads();
    find_digit_desc<kRowLowBins>(sm.h2, need, sm.out3);
    const uint32_t d2 = sm.out3[0];
    prefix = (prefix << 10) | d2;
    need = sm.out3[1];
    shift = 10;
    whole = sm.h2[d2] == need;
  }
  if (!whole) {
    for (uint32_t i = tid; i < n_cand; i += kRowThreads) {
      const uint32_t key = sm.ck[i];
      if ((key >> 10) == prefix) atomicAdd(&sm.h3[key & (kRowLowBins - 1)], 1u);
    }
    __syncthreads();
    find_digit_desc<kRowLowBins>(sm.h3, need, sm.out3);
    const uint32_t d3 = sm.out3[0];
    prefix = (prefix << 10) | d3;
    need = sm.out3[1];
    shift = 0;
    whole = sm.h3[d3] == need;
  }
  // 5. kept: keys above the cut, the whole cut bin when it fits; otherwise
  // the keys equal to TK (shift is 0 then) go to the tie list
  for (uint32_t i = tid; i < n_cand; i += kRowThreads) {
    const uint32_t kh = sm.ck[i] >> shift;
    const uint32_t id = sm.ci[i];
    if (kh > prefix || (kh == prefix && whole)) {
      atomicOr(&sm.bits[id >> 5], 1u << (id & 31u));
    } else if (kh == prefix) {
      const uint32_t j = atomicAdd(&sm.n_eq, 1u);
      if (j < (uint32_t)kMaxTies) sm.teq[j] = id;
    }
  }
  __syncthreads();
  if (!whole) {
    const uint32_t n_eq = sm.n_eq;
    if (n_eq > (uint32_t)kMaxTies) {
      if (tid == 0) *path = sel::kPathExactTies;
      sel::exact_select<kRowThreads>(sel::ScoreArray{s}, nb, k, out, sm);
      return;
    }
    // equal keys: the `need` lowest block ids (ids are distinct)
    if ((uint32_t)tid < n_eq) {
      const uint32_t me = sm.teq[tid];
      uint32_t below = 0u;
      for (uint32_t j = 0; j < n_eq; ++j) below += sm.teq[j] < me ? 1u : 0u;
      if (below < need) atomicOr(&sm.bits[me >> 5], 1u << (me & 31u));
    }
    __syncthreads();
  }
  // 6. kept ids in ascending order: each thread owns a run of bitmap words
  const int per = (bit_words + kRowThreads - 1) / kRowThreads;
  const int w0 = tid * per;
  uint32_t mine = 0u;
  for (int w = w0; w < w0 + per && w < bit_words; ++w) mine += (uint32_t)__popc(sm.bits[w]);
  uint32_t total;
  uint32_t pos = block_excl_scan<kRowThreads>(mine, sm.scan_sh, total);
  for (int w = w0; w < w0 + per && w < bit_words; ++w) {
    uint32_t b = sm.bits[w];
    while (b) {
      const int bit = __ffs(b) - 1;
      b &= b - 1u;
      if (pos < (uint32_t)k) out[pos] = w * 32 + bit;
      ++pos;
    }
  }
  if (tid == 0) *path = sel::kPathCandidates;
}

hipError_t select_rows(const float* scores, int64_t ld, int M, const int64_t* row_pos, int64_t nb_max, int k,
                       int32_t* sel, int32_t* n_sel, uint32_t* W, hipStream_t stream) {
  hipLaunchKernelGGL(select_row_kernel, dim3((unsigned)M), dim3(kRowThreads), sizeof(RowSmem), stream, scores, ld,
                     row_pos, nb_max, k, sel, n_sel, W);
  return hipGetLastError();
}


hipError_t collect_finalize(const float* scores, int64_t ld, int M, const int64_t* row_pos, int64_t nb_max,
                            int k, int32_t* sel, int32_t* n_sel, uint32_t* W, hipStream_t stream) {
  if (nb_max > k) {
    const int64_t chunks = (nb_max + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(select_collect_kernel, dim3((unsigned)chunks, (unsigned)M), dim3(kChunkThreads), 0,
                       stream, scores, ld, row_pos, nb_max, k, W);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_finalize_kernel, dim3((unsigned)M), dim3(kFinThreads), 0, stream, scores, ld,
                     row_pos, nb_max, k, sel, n_sel, W);
  return hipGetLastError();
}

// The one-launch row selection for many rows (a workgroup per row fills the
// GPU: 143 vs 159 us for 2,048 prefill rows); the two-pass path otherwise
// (also for short rows: 12.5 vs 10.7 us for one row of 8,192 blocks).
bool row_select_fits(int M, int64_t /*nb_max*/) { return M >= 256; }

}  // namespace

size_t select_workspace_bytes(int max_M, int64_t nb_max, int /*k_blocks*/) {
  return (size_t)max_M * (size_t)sel::row_words(nb_max) * sizeof(uint32_t);
}

hipError_t launch_select_topk(const float* scores, int64_t ld, int M, const int64_t* row_pos,
                              int64_t nb_max, int k_blocks, int32_t* sel, int32_t* n_sel,
                              void* ws, size_t /*ws_bytes*/, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  uint32_t* W = static_cast<uint32_t*>(ws);
  if (nb_max > k_blocks) {
    const int64_t grid_x = (sel::sample_groups(nb_max) + kChunkThreads - 1) / kChunkThreads;
    hipLaunchKernelGGL(select_sample_kernel, dim3((unsigned)grid_x, (unsigned)M), dim3(kChunkThreads), 0,
                       stream, scores, ld, row_pos, nb_max, W);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (row_select_fits(M, nb_max)) return select_rows(scores, ld, M, row_pos, nb_max, k_blocks, sel, n_sel, W, stream);
  return collect_finalize(scores, ld, M, row_pos, nb_max, k_blocks, sel, n_sel, W, stream);
}

hipError_t launch_select_after_hist(const float* scores, int64_t ld, int M, const int64_t* row_pos,
                                   int64_t nb_max, int k_blocks, int32_t* sel, int32_t* n_sel,
                                   void* ws, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  uint32_t* W = static_cast<uint32_t*>(ws);
  if (row_select_fits(M, nb_max)) return select_rows(scores, ld, M, row_pos, nb_max, k_blocks, sel, n_sel, W, stream);
  return collect_finalize(scores, ld, M, row_pos, nb_max, k_blocks, sel, n_sel, W, stream);
}

}  // namespace qsa
