// Top-k block selection (hipfire "QSA sparse attention ...", section 02:
// keep the top-scoring blocks within the token budget; section 03: a radix
// select follows the scoring; section 06: long score rows no longer fit the
// selector's on-chip memory).  Equal scores go to the lower block index.
//
// Scores map to order-preserving 32-bit keys (-0 folded into +0); the top 12
// key bits are a histogram digit (8 bins per octave of positive scores).  The
// work is spread over many compute units:
//
//  sample   (standalone selection only; the scoring kernel does the same in
//           its epilogue) one block of every 16-block group, at a hashed
//           offset, has its score copied to the group's slot in the row's
//           workspace record, and the row's arrival counter is cleared.
//  collect  one workgroup per 4,096-block chunk of a row histograms the row's
//           samples in LDS and walks the histogram from the top to the digit
//           B where the sample count reaches (1.25 k + 256) / 16: a
//           conservative threshold, about 1.25 k + 256 blocks are expected at
//           or above it.  The chunk's (key, id) pairs with digit >= B go to
//           the chunk's own slots in ascending block order (a block scan
//           places them; no atomics).
//  finalize the last collect workgroup of a row to finish (an arrival counter
//           per row, after a device-wide release of every chunk's
//           candidates) gathers the chunks' candidates (ascending block
//           order) and finds the k-th largest candidate key TK with three
//           histogram levels (12, 10 and 10 key bits; each level counts only
//           the candidates sharing the bits found so far).  Keys above TK are
//           kept, and of the keys equal to TK the first ones in block order;
//           a block scan writes the kept ids in ascending order.  A candidate
//           list shorter than k (the sample misled the threshold), one longer
//           than the on-chip list (massive ties) or a row of more than 64
//           chunks takes an exact radix select over the whole row in the same
//           workgroup, so the result is exact in every case.
// Three forms, by size:
//  - rows of at most 8,192 blocks: one workgroup per row does it all
//    (select_row_kernel): the candidates never leave its LDS;
//  - up to 1,024 collect workgroups: collect and finalize are one launch, the
//    finalize of a row starting as soon as its chunks are collected, with no
//    kernel boundary in between (measured at the 262K verify: 11.7 us against
//    13.4 us as two launches);
//  - more (prefill): each row's threshold once (select_threshold_kernel),
//    then the collect pass reading it, then one finalize workgroup per row.
//
// The workspace holds one record per row (sel::row_words); no part of it
// needs initialising (the pass that writes the sample clears the arrival
// counter, and the finalizing workgroup clears it again after use).
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
constexpr int kSampleThreads = 256;
constexpr int kChunkThreads = 512;                 // the collect + finalize workgroup
constexpr int kChunkPer = kChunk / kChunkThreads;  // 8 consecutive scores per lane
constexpr int kFinThreads = kChunkThreads;
constexpr int kFinPer = kCandMax / kFinThreads;    // 8 candidates per thread
constexpr int kLowBins = 1024;                     // 10-bit digits below the 12-bit one
// Above this many collect workgroups (rows x chunks: prefill chunks) the
// finalize runs as a launch of its own: the fused kernel's LDS for the
// finalize halves how many collect workgroups fit on a compute unit, which
// costs more than the kernel boundary once the collect spans many waves of
// workgroups (measured: 2,048 rows, 0.49 ms fused against 0.21 ms).
constexpr int64_t kFusedMaxWorkgroups = 1024;
// Rows of at most this many blocks take the one-workgroup form (measured,
// sample + selection of one row: 9.3 against 11.1 us at 8,192 blocks; from
// 12,288 blocks on the chunked form is faster: one compute unit then streams
// the row too slowly).
constexpr int kRowPer = 16;
constexpr int64_t kRowMaxBlocks = kRowPer * kFinThreads;
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

// Words one workgroup writes and another reads within the same launch (the
// candidates and counts of the collect + finalize launch) travel through
// device-coherent accesses (relaxed agent-scope atomics: stores and loads
// that bypass the non-coherent part of each XCD's L2), so no cache-wide
// writeback or invalidate is needed to pass them between XCDs.
template <bool COH>
__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
template <bool COH>
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  if constexpr (COH) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *p = v;
  }
}

// ---------------------------------------------------------------- kernels

// Standalone selection: write each row's sampled scores (one per 16-block
// group) into the workspace and clear the row's arrival counter.
__global__ void __launch_bounds__(kSampleThreads)
select_sample_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                     int64_t nb_max, uint32_t* __restrict__ ws) {
  const int m = blockIdx.y;
  const int64_t grp = (int64_t)blockIdx.x * kSampleThreads + threadIdx.x;
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  const int64_t b = grp * 16 + sel::sample_offset((uint32_t)grp);
  if (b < nb) reinterpret_cast<float*>(W)[sel::sample_off(nb_max) + grp] = scores[(int64_t)m * ld + b];
  if (grp == 0) W[sel::kArriveWord] = 0u;
}

// The candidate threshold of a row: the digit B at which the row's sample
// reaches the target count, from a histogram of the sample in LDS (h, all
// threads).  0 when every block must be a candidate.
__device__ uint32_t row_threshold(const float* __restrict__ smp, int64_t n_grp, int64_t nb, int k,
                                  uint32_t* h, uint32_t* out3, const float (&smpv)[kChunk / kChunkThreads]) {
  constexpr int kSampPer = kChunk / kChunkThreads;  // samples per lane per round
  const int tid = threadIdx.x;
  // histogram of the row's samples (blocks < nb only)
#pragma unroll
  for (int e = 0; e < kSampPer; ++e) {
    const int64_t gi = (int64_t)e * kChunkThreads + tid;
    if (gi < n_grp && gi * 16 + sel::sample_offset((uint32_t)gi) < nb) atomicAdd(&h[win_bin(order_key(smpv[e]))], 1u);
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
      if (gi < n_grp && gi * 16 + sel::sample_offset((uint32_t)gi) < nb) atomicAdd(&h[win_bin(order_key(v[e]))], 1u);
    }
  }
  __syncthreads();
  // conservative threshold (not reached: every block is a candidate)
  find_digit_desc<kWinBins>(h, sel::sample_target((uint32_t)k), out3);
  // window bin 0 (or a target never reached): every block is a candidate
  return (out3[2] || out3[0] == 0u) ? 0u : kWinBase + out3[0];
}

// Exact selection among the candidates: sm.ck / sm.ci hold the candidate list
// (ascending block order, n_cand entries), sm.hist16 the count of each 12-bit
// digit, sm.h2 / sm.h3 are zero, and each thread holds candidates in kk (those
// flagged in vm) -- the caller has synchronised.  Writes the kept ids to out,
// ascending.
__device__ void select_from_candidates(FinSmem& sm, const uint32_t (&kk)[kFinPer], uint32_t vm, uint32_t n_cand,
                                       int k, int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
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

// Final selection of row m from its chunks' candidates (or, on the exact
// paths, from its scores): kept ids ascending into sel, the count into n_sel.
template <bool COH>
__device__ void finalize_row(const float* __restrict__ s, int64_t nb, int64_t nb_max, int k, int m,
                             int32_t* __restrict__ sel, int32_t* __restrict__ n_sel, uint32_t* __restrict__ W,
                             FinSmem& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  int32_t* __restrict__ out = sel + (int64_t)m * k;
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
    kk[e] = ld_u32<COH>(K + at);
    ii[e] = ld_u32<COH>(I + at);
  }
  const uint32_t cnt_raw = (tid < kWave && tid < nchm) ? ld_u32<COH>(W + sel::cnt_off(nb_max) + tid) : 0u;
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
      kk[e] = ld_u32<COH>(K + slot);
      ii[e] = ld_u32<COH>(I + slot);
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
  select_from_candidates(sm, kk, vm, n_cand, k, out);
}

// The candidate threshold of each row, once (many rows): one workgroup per
// row histograms the row's sample and stores the digit in the row's record,
// so that the row's chunk workgroups load one word instead of the sample.
__global__ void __launch_bounds__(kChunkThreads)
select_threshold_kernel(const int64_t* __restrict__ row_pos, int64_t nb_max, int k, uint32_t* __restrict__ ws) {
  __shared__ uint32_t h[kWinBins];
  __shared__ uint32_t out3[3];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  const float* __restrict__ smp = reinterpret_cast<const float*>(W + sel::sample_off(nb_max));
  const int64_t n_grp = sel::sample_groups(nb_max);
  constexpr int kSampPer = kChunk / kChunkThreads;
  float smpv[kSampPer];
#pragma unroll
  for (int e = 0; e < kSampPer; ++e) {
    const int64_t gi = (int64_t)e * kChunkThreads + tid;
    smpv[e] = gi < n_grp ? smp[gi] : 0.f;
  }
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  for (int i = tid; i < kWinBins; i += kChunkThreads) h[i] = 0u;
  if (nb <= k) return;  // uniform: the collect pass skips the row
  __syncthreads();
  const uint32_t B = row_threshold(smp, n_grp, nb, k, h, out3, smpv);
  if (tid == 0) W[sel::kThrWord] = B;
}

// Collect of one 4,096-block chunk of a row; with FUSED the last chunk of the
// row to finish also finalizes the row.
template <bool FUSED, bool PRE_THR = false>
__global__ void __launch_bounds__(kChunkThreads)
select_collect_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                      int64_t nb_max, int k, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                      uint32_t* __restrict__ ws) {
  __shared__ uint32_t h[kWinBins];
  __shared__ uint32_t scan_sh[2 * (kChunkThreads / kWave)];
  __shared__ uint32_t out3[3];
  __shared__ uint32_t last_sh;
  const int m = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)c * kChunk;
  const float* __restrict__ s = scores + (int64_t)m * ld;
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  const float* __restrict__ smp = reinterpret_cast<const float*>(W + sel::sample_off(nb_max));
  const int64_t n_grp = sel::sample_groups(nb_max);

  // every load this pass needs is independent: issue them together
  const int64_t i0 = base + (int64_t)tid * kChunkPer;  // this lane's consecutive blocks
  float4 sv[kChunkPer / 4];
#pragma unroll
  for (int q = 0; q < kChunkPer / 4; ++q) {
    const int64_t j = i0 + 4 * q;  // rows are padded to a multiple of 4 floats
    sv[q] = j < nb_max ? *reinterpret_cast<const float4*>(s + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  constexpr int kSampPer = kChunk / kChunkThreads;  // samples per lane per round
  float smpv[kSampPer];
  uint32_t thr = 0u;
  if constexpr (PRE_THR) {
    thr = W[sel::kThrWord];  // written by select_threshold_kernel
  } else {
#pragma unroll
    for (int e = 0; e < kSampPer; ++e) {
      const int64_t gi = (int64_t)e * kChunkThreads + tid;
      smpv[e] = gi < n_grp ? smp[gi] : 0.f;
    }
  }
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  if constexpr (!PRE_THR)
    for (int i = tid; i < kWinBins; i += kChunkThreads) h[i] = 0u;
  // every block kept, or a chunk the finalize pass does not read: nothing to collect
  const bool collect = !(nb <= k || base >= nb);
  if (collect) {
    uint32_t B = thr;
    if constexpr (!PRE_THR) {
      __syncthreads();
      B = row_threshold(smp, n_grp, nb, k, h, out3, smpv);
    }
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
          st_u32<FUSED>(K + pos, key[e]);
          st_u32<FUSED>(I + pos, (uint32_t)(i0 + e));
        }
        ++pos;
      }
    }
    if (tid == 0) st_u32<FUSED>(W + sel::cnt_off(nb_max) + c, total);
  }
  if constexpr (FUSED) {
    // Arrival: every wave waits until its coherent stores are complete, then
    // one lane counts the chunk in (a device-scope atomic); the chunk that
    // completes the count reads every chunk's candidates through coherent
    // loads.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(W + sel::kArriveWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_sh = old == gridDim.x - 1 ? 1u : 0u;
    }
    __syncthreads();
    if (!last_sh) return;
    // every chunk of the row has arrived: ready for the next call
    if (tid == 0) __hip_atomic_store(W + sel::kArriveWord, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __shared__ FinSmem sm;
    finalize_row<true>(s, nb, nb_max, k, m, sel, n_sel, W, sm);
  }
}

// Rows of at most kRowMaxBlocks blocks (decode at 32K context): one
// workgroup per row does the whole selection.  Its PER scores per lane and the
// row's sample arrive in one round trip, the threshold comes from the sample
// as in the collect pass, and the candidates go straight into LDS in
// ascending block order (a block scan), so none of them leaves the compute
// unit and no other workgroup is waited for.  Same paths and result as the
// collect + finalize form.
template <int PER>
__global__ void __launch_bounds__(kFinThreads)
select_row_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                  int64_t nb_max, int k, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                  uint32_t* __restrict__ ws) {
  static_assert(PER % 4 == 0 && PER <= 32, "float4 score loads, one flag bit per score");
  __shared__ FinSmem sm;
  __shared__ uint32_t h[kWinBins];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const float* __restrict__ s = scores + (int64_t)m * ld;
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  const float* __restrict__ smp = reinterpret_cast<const float*>(W + sel::sample_off(nb_max));
  const int64_t n_grp = sel::sample_groups(nb_max);
  int32_t* __restrict__ out = sel + (int64_t)m * k;

  // every load this pass needs, issued together
  const int64_t i0 = (int64_t)tid * PER;  // this lane's consecutive blocks
  float4 sv[PER / 4];
#pragma unroll
  for (int q = 0; q < PER / 4; ++q) {
    const int64_t j = i0 + 4 * q;  // rows are padded to a multiple of 4 floats
    sv[q] = j < nb_max ? *reinterpret_cast<const float4*>(s + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  constexpr int kSampPer = kChunk / kChunkThreads;  // row_threshold's register-held sample
  float smpv[kSampPer];
#pragma unroll
  for (int e = 0; e < kSampPer; ++e) {
    const int64_t gi = (int64_t)e * kChunkThreads + tid;
    smpv[e] = gi < n_grp ? smp[gi] : 0.f;
  }
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  if (nb <= k) {
    for (int i = tid; i < k; i += kFinThreads) out[i] = i < nb ? i : -1;
    if (tid == 0) {
      n_sel[m] = (int32_t)nb;
      W[sel::kPathWord] = sel::kPathAll;
    }
    return;
  }
  if (tid == 0) n_sel[m] = k;
  for (int i = tid; i < kWinBins; i += kFinThreads) h[i] = 0u;
  for (int i = tid; i < kDigits; i += kFinThreads) sm.hist16[i] = 0u;
  for (int i = tid; i < kLowBins; i += kFinThreads) {
    sm.h2[i] = 0u;
    sm.h3[i] = 0u;
  }
  __syncthreads();
  const uint32_t B = row_threshold(smp, n_grp, nb, k, h, sm.out3, smpv);
  uint32_t key[PER];
#pragma unroll
  for (int q = 0; q < PER / 4; ++q) {
    key[4 * q + 0] = order_key(sv[q].x);
    key[4 * q + 1] = order_key(sv[q].y);
    key[4 * q + 2] = order_key(sv[q].z);
    key[4 * q + 3] = order_key(sv[q].w);
  }
  uint32_t flags = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (i0 + e < nb && (key[e] >> kDigitShift) >= B) flags |= 1u << e;
  uint32_t total;
  uint32_t pos = block_excl_scan<kFinThreads>((uint32_t)__popc(flags), sm.scan_sh, total);
  if (total < (uint32_t)k || total > (uint32_t)kCandMax) {  // uniform
    if (tid == 0) W[sel::kPathWord] = sel::kPathExactCount;
    exact_row_select(s, nb, k, out, sm);
    return;
  }
  if (tid == 0) W[sel::kPathWord] = sel::kPathCandidates;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if ((flags >> e) & 1u) {  // pos < total <= kCandMax
      sm.ck[pos] = key[e];
      sm.ci[pos] = (uint32_t)(i0 + e);
      atomicAdd(&sm.hist16[key[e] >> kDigitShift], 1u);
      ++pos;
    }
  }
  __syncthreads();
  uint32_t kk[kFinPer];
  uint32_t vm = 0u;
#pragma unroll
  for (int e = 0; e < kFinPer; ++e) {
    const uint32_t i = (uint32_t)(e * kFinThreads + tid);  // < kCandMax
    kk[e] = sm.ck[i];
    vm |= i < total ? (1u << e) : 0u;
  }
  select_from_candidates(sm, kk, vm, total, k, out);
}

// Finalize pass of the two-launch form (one workgroup per row).
__global__ void __launch_bounds__(kFinThreads)
select_finalize_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                       int64_t nb_max, int k, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                       uint32_t* __restrict__ ws) {
  __shared__ FinSmem sm;
  const int m = blockIdx.x;
  finalize_row<false>(scores + (int64_t)m * ld, clamp_nb(row_pos[m], nb_max), nb_max, k, m, sel, n_sel,
               ws + (size_t)m * sel::row_words(nb_max), sm);
}

hipError_t collect_finalize(const float* scores, int64_t ld, int M, const int64_t* row_pos, int64_t nb_max,
                            int k, int32_t* sel, int32_t* n_sel, uint32_t* W, hipStream_t stream) {
  const int64_t chunks = (nb_max + kChunk - 1) / kChunk;
  if (nb_max > k && nb_max <= kRowMaxBlocks) {  // short rows: one workgroup per row
    hipLaunchKernelGGL(select_row_kernel<kRowPer>, dim3((unsigned)M), dim3(kFinThreads), 0, stream, scores, ld,
                       row_pos, nb_max, k, sel, n_sel, W);
  } else if (nb_max > k && M * chunks <= kFusedMaxWorkgroups) {  // collect, and the last chunk of each row finalizes it
    hipLaunchKernelGGL(select_collect_kernel<true>, dim3((unsigned)chunks, (unsigned)M), dim3(kChunkThreads), 0,
                       stream, scores, ld, row_pos, nb_max, k, sel, n_sel, W);
  } else if (nb_max > k) {  // many rows: thresholds, collect, then one finalize workgroup per row
    hipLaunchKernelGGL(select_threshold_kernel, dim3((unsigned)M), dim3(kChunkThreads), 0, stream, row_pos, nb_max, k,
                       W);
    hipLaunchKernelGGL((select_collect_kernel<false, true>), dim3((unsigned)chunks, (unsigned)M), dim3(kChunkThreads),
                       0, stream, scores, ld, row_pos, nb_max, k, sel, n_sel, W);
    hipLaunchKernelGGL(select_finalize_kernel, dim3((unsigned)M), dim3(kFinThreads), 0, stream, scores, ld,
                       row_pos, nb_max, k, sel, n_sel, W);
  } else {  // every row keeps all its blocks
    hipLaunchKernelGGL(select_finalize_kernel, dim3((unsigned)M), dim3(kFinThreads), 0, stream, scores, ld,
                       row_pos, nb_max, k, sel, n_sel, W);
  }
  return hipGetLastError();
}

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
    const int64_t grid_x = (sel::sample_groups(nb_max) + kSampleThreads - 1) / kSampleThreads;
    hipLaunchKernelGGL(select_sample_kernel, dim3((unsigned)grid_x, (unsigned)M), dim3(kSampleThreads), 0,
                       stream, scores, ld, row_pos, nb_max, W);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return collect_finalize(scores, ld, M, row_pos, nb_max, k_blocks, sel, n_sel, W, stream);
}

hipError_t launch_select_after_hist(const float* scores, int64_t ld, int M, const int64_t* row_pos,
                                   int64_t nb_max, int k_blocks, int32_t* sel, int32_t* n_sel,
                                   void* ws, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  return collect_finalize(scores, ld, M, row_pos, nb_max, k_blocks, sel, n_sel, static_cast<uint32_t*>(ws),
                          stream);
}

}  // namespace qsa
