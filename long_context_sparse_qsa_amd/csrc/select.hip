// Top-k block selection (hipfire "QSA sparse attention ...", section 02:
// keep the top-scoring blocks within the token budget; section 03: a radix
// select follows the scoring; section 06: long score rows no longer fit the
// selector's on-chip memory).  Equal scores go to the lower block index.
//
// Scores map to order-preserving 32-bit keys (-0 folded into +0); the top 12
// key bits are a histogram digit (8 bins per octave of positive scores).  The work is spread over many compute units, with kernel
// boundaries (not fences) ordering the passes:
//
//  sample   (standalone selection only; the scoring kernel does the same in
//           its epilogue) one block of every 16-block group, at a hashed
//           offset, has its score copied to the group's slot in the row's
//           workspace record.
//  collect  many workgroups per row histogram the row's samples in LDS and
//           walk the histogram from the top to the digit B where the sample
//           count reaches (1.25 k + 256) / 16: a conservative threshold, about
//           1.25 k + 256 blocks are expected at or above it.  Every (key, id)
//           with digit >= B goes to the row's candidate list (one atomic per
//           wave).
//  finalize one workgroup per row: an exact radix select over the candidate
//           keys gives the k-th key T and how many keys equal to T to keep;
//           those go to the lowest ids (a radix select on complemented ids).
//           Kept ids are set in an LDS bitmap that a prefix popcount writes
//           out in ascending order.  A candidate list shorter than k (the
//           sample misled the threshold), one that overflows (massive ties)
//           or a row beyond the bitmap takes an exact radix select over the
//           whole row in the same workgroup, so the result is exact in every
//           case.
//
// The workspace holds one record per row (sel::RowWs); no part of it needs
// initialising.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "select_common.h"

namespace qsa {

namespace {

using sel::kCandMax;
using sel::kDigits;
using sel::kDigitShift;
using sel::order_key;
using sel::RowWs;

constexpr int kBins = 256;
constexpr int kCopies = 16;
constexpr int kChunkThreads = 256;
constexpr int kChunkPer = 16;
constexpr int kChunk = kChunkThreads * kChunkPer;  // 4,096 scores per workgroup
constexpr int kFinThreads = 512;
constexpr int kBitmapWords = 8192;                 // 262,144 blocks

template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < NW ? sh[lane] : 0u;
    x = wave_incl_scan(x, lane);
    if (lane < NW) sh[NW + lane] = x;
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? sh[NW + wave - 1] : 0u;
  total = sh[2 * NW - 1];
  __syncthreads();
  return before + incl - v;
}

// Counts cnt[0..nbins) in LDS (digit order ascending): find the digit where
// the count from the top reaches `want`.  out3 = {digit, want - count above
// the digit, 0}; out3[2] = 1 when the total stays below `want`.
template <int NT>
__device__ void find_digit_desc(const uint32_t* cnt, int nbins, uint32_t want, uint32_t* scan_sh,
                                uint32_t* out3) {
  const int per = (nbins + NT - 1) / NT;
  const int hi = nbins - 1 - (int)threadIdx.x * per;
  uint32_t mine = 0;
  for (int j = 0; j < per; ++j)
    if (hi - j >= 0) mine += cnt[hi - j];
  if (threadIdx.x == 0) {
    out3[0] = 0u;
    out3[1] = want;
    out3[2] = 1u;
  }
  uint32_t tot;
  uint32_t above = block_excl_scan<NT>(mine, scan_sh, tot);
  for (int j = 0; j < per; ++j) {
    const int b = hi - j;
    if (b < 0) break;
    const uint32_t c = cnt[b];
    if (above < want && above + c >= want) {
      out3[0] = (uint32_t)b;
      out3[1] = want - above;
      out3[2] = 0u;
    }
    above += c;
  }
  __syncthreads();
}

struct FinSmem {
  uint32_t hist16[kBins * kCopies];
  uint32_t tot[kBins];
  uint32_t ck[kCandMax];
  uint32_t ci[kCandMax];
  uint32_t bm[kBitmapWords];
  uint32_t scan_sh[2 * (kFinThreads / kWave)];
  uint32_t out3[3];
  uint32_t n_eq;
};

// Radix select over LDS keys[0..n): the want-th largest key among all n,
// 8 bits per pass from bit 32 down.  out3 = {key T, keys == T to keep}.
__device__ void lds_radix_select(const uint32_t* keys, int n, uint32_t want, FinSmem& sm) {
  constexpr int NT = kFinThreads;
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t prefix = 0u, mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < kBins * kCopies; i += NT) sm.hist16[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t u = keys[i];
      if ((u & mask) == prefix) atomicAdd(&sm.hist16[((u >> shift) & 0xffu) * kCopies + (lane & (kCopies - 1))], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBins; i += NT) {
      uint32_t t = 0;
#pragma unroll
      for (int c = 0; c < kCopies; ++c) t += sm.hist16[i * kCopies + c];
      sm.tot[i] = t;
    }
    __syncthreads();
    find_digit_desc<NT>(sm.tot, kBins, want, sm.scan_sh, sm.out3);
    prefix |= sm.out3[0] << shift;
    mask |= 0xffu << shift;
    want = sm.out3[1];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    sm.out3[0] = prefix;
    sm.out3[1] = want;
  }
  __syncthreads();
}

// Kept ids, ascending, from the LDS bitmap.
__device__ void write_from_bitmap(const uint32_t* bm, int nwords, int32_t* out, int k, uint32_t* scan_sh) {
  constexpr int NT = kFinThreads;
  const int per = (nwords + NT - 1) / NT;
  const int w0 = threadIdx.x * per;
  uint32_t cnt = 0;
  for (int j = 0; j < per; ++j)
    if (w0 + j < nwords) cnt += __popc(bm[w0 + j]);
  uint32_t tot;
  uint32_t pos = block_excl_scan<NT>(cnt, scan_sh, tot);
  for (int j = 0; j < per; ++j) {
    const int w = w0 + j;
    if (w >= nwords) break;
    uint32_t bits = bm[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1u;
      if (pos < (uint32_t)k) out[pos] = w * 32 + b;
      ++pos;
    }
  }
}

// Exact path over the whole row: four 8-bit radix passes over all keys,
// then an order-preserving compaction in index order.
__device__ void exact_row_select(const float* __restrict__ s, int64_t nb, int k, int32_t* out, FinSmem& sm) {
  constexpr int NT = kFinThreads;
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t prefix = 0, mask = 0, want = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < kBins * kCopies; i += NT) sm.hist16[i] = 0u;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < nb; i += NT) {
      const uint32_t u = order_key(s[i]);
      if ((u & mask) == prefix) atomicAdd(&sm.hist16[((u >> shift) & 0xffu) * kCopies + (lane & (kCopies - 1))], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBins; i += NT) {
      uint32_t t = 0;
#pragma unroll
      for (int c = 0; c < kCopies; ++c) t += sm.hist16[i * kCopies + c];
      sm.tot[i] = t;
    }
    __syncthreads();
    find_digit_desc<NT>(sm.tot, kBins, want, sm.scan_sh, sm.out3);
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
      const uint32_t u = i < nb ? order_key(s[i]) : 0u;
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

// ---------------------------------------------------------------- kernels

// Standalone selection: write each row's sampled scores (one per 16-block
// group) into the workspace and zero the candidate counter.
__global__ void __launch_bounds__(kChunkThreads)
select_sample_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                     int64_t nb_max, uint32_t* __restrict__ ws) {
  const int m = blockIdx.y;
  const int64_t grp = (int64_t)blockIdx.x * kChunkThreads + threadIdx.x;
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  if (blockIdx.x == 0 && threadIdx.x == 0) W[RowWs::kCount] = 0u;
  const int64_t b = grp * 16 + sel::sample_offset((uint32_t)grp);
  if (b < nb) reinterpret_cast<float*>(W)[RowWs::kSamples + grp] = scores[(int64_t)m * ld + b];
}

__global__ void __launch_bounds__(kChunkThreads)
select_collect_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                      int64_t nb_max, int k, uint32_t* __restrict__ ws) {
  __shared__ uint32_t h[kDigits];
  __shared__ uint32_t scan_sh[2 * (kChunkThreads / kWave)];
  __shared__ uint32_t out3[3];
  const int m = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  const float* __restrict__ s = scores + (int64_t)m * ld;
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  const float* __restrict__ smp = reinterpret_cast<const float*>(W + RowWs::kSamples);
  // everything this pass reads is independent: issue it together
  const int64_t lim = nb_max - base;
  uint32_t key[kChunkPer];
#pragma unroll
  for (int e = 0; e < kChunkPer; ++e) {
    const int64_t j = (int64_t)e * kChunkThreads + threadIdx.x;
    key[e] = j < lim ? order_key(s[base + j]) : 0u;
  }
  const int64_t n_grp = sel::sample_groups(nb_max);
  constexpr int kSampPer = 16;  // samples per lane per round
  for (int i = threadIdx.x; i < kDigits; i += kChunkThreads) h[i] = 0u;
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  if (nb <= k || base >= nb) return;
  __syncthreads();
  // histogram of the row's samples (blocks < nb only)
  for (int64_t g0 = 0; g0 < n_grp; g0 += (int64_t)kChunkThreads * kSampPer) {
    float sv[kSampPer];
#pragma unroll
    for (int e = 0; e < kSampPer; ++e) {
      const int64_t gi = g0 + (int64_t)e * kChunkThreads + threadIdx.x;
      sv[e] = gi < n_grp ? smp[gi] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kSampPer; ++e) {
      const int64_t gi = g0 + (int64_t)e * kChunkThreads + threadIdx.x;
      if (gi < n_grp && gi * 16 + sel::sample_offset((uint32_t)gi) < nb)
        atomicAdd(&h[order_key(sv[e]) >> kDigitShift], 1u);
    }
  }
  __syncthreads();
  // conservative threshold (not reached: every block is a candidate)
  find_digit_desc<kChunkThreads>(h, kDigits, sel::sample_target((uint32_t)k), scan_sh, out3);
  const uint32_t B = out3[2] ? 0u : out3[0];

  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < kChunkPer; ++e) {
    const int64_t i = base + (int64_t)e * kChunkThreads + threadIdx.x;
    mine += (i < nb && (key[e] >> kDigitShift) >= B) ? 1u : 0u;
  }
  // one atomic per wave reserves its slots
  const uint32_t incl = wave_incl_scan(mine, lane);
  uint32_t wbase = 0;
  if (lane == kWave - 1 && incl) wbase = atomicAdd(&W[RowWs::kCount], incl);
  wbase = __shfl(wbase, kWave - 1, kWave);
  uint32_t p = wbase + incl - mine;
#pragma unroll
  for (int e = 0; e < kChunkPer; ++e) {
    const int64_t i = base + (int64_t)e * kChunkThreads + threadIdx.x;
    if (i < nb && (key[e] >> kDigitShift) >= B) {
      if (p < (uint32_t)kCandMax) {
        W[RowWs::kKeys + p] = key[e];
        W[RowWs::kIds + p] = (uint32_t)i;
      }
      ++p;
    }
  }
}

__global__ void __launch_bounds__(kFinThreads)
select_finalize_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ row_pos,
                       int64_t nb_max, int k, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                       uint32_t* __restrict__ ws) {
  __shared__ FinSmem sm;
  const int m = blockIdx.x;
  const float* __restrict__ s = scores + (int64_t)m * ld;
  int32_t* __restrict__ out = sel + (int64_t)m * k;
  uint32_t* W = ws + (size_t)m * sel::row_words(nb_max);
  const uint32_t n_cand = W[RowWs::kCount];
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  if (nb <= k) {
    for (int i = threadIdx.x; i < k; i += kFinThreads) out[i] = i < nb ? i : -1;
    if (threadIdx.x == 0) n_sel[m] = (int32_t)nb;
    return;
  }
  if (threadIdx.x == 0) n_sel[m] = k;
  const int nwords = (int)((nb + 31) / 32);
  if (n_cand < (uint32_t)k || n_cand > (uint32_t)kCandMax || nwords > kBitmapWords) {
    exact_row_select(s, nb, k, out, sm);
    return;
  }
  for (uint32_t i = threadIdx.x; i < n_cand; i += kFinThreads) {
    sm.ck[i] = W[RowWs::kKeys + i];
    sm.ci[i] = W[RowWs::kIds + i];
  }
  for (int i = threadIdx.x; i < nwords; i += kFinThreads) sm.bm[i] = 0u;
  if (threadIdx.x == 0) sm.n_eq = 0u;
  __syncthreads();

  lds_radix_select(sm.ck, (int)n_cand, (uint32_t)k, sm);
  const uint32_t T = sm.out3[0];
  const uint32_t need_t = sm.out3[1];
  uint32_t* eqk = sm.hist16;  // free after the radix passes
  for (uint32_t i = threadIdx.x; i < n_cand; i += kFinThreads) {
    const uint32_t kk = sm.ck[i];
    const uint32_t id = sm.ci[i];
    if ((int64_t)id >= nb) continue;  // never past the row (list written by this call's collect)
    if (kk > T) atomicOr(&sm.bm[id >> 5], 1u << (id & 31));
    else if (kk == T) eqk[atomicAdd(&sm.n_eq, 1u)] = ~id;
  }
  __syncthreads();
  const uint32_t n_eq = sm.n_eq;
  if (n_eq <= need_t) {
    for (uint32_t i = threadIdx.x; i < n_eq; i += kFinThreads) {
      const uint32_t id = ~eqk[i];
      atomicOr(&sm.bm[id >> 5], 1u << (id & 31));
    }
  } else {
    // the need_t lowest ids among equal keys = the largest complemented ids
    for (uint32_t i = threadIdx.x; i < n_eq; i += kFinThreads) sm.ck[i] = eqk[i];
    __syncthreads();
    lds_radix_select(sm.ck, (int)n_eq, need_t, sm);
    const uint32_t t_id = sm.out3[0];
    for (uint32_t i = threadIdx.x; i < n_eq; i += kFinThreads) {
      if (sm.ck[i] >= t_id) {
        const uint32_t id = ~sm.ck[i];
        atomicOr(&sm.bm[id >> 5], 1u << (id & 31));
      }
    }
  }
  __syncthreads();
  write_from_bitmap(sm.bm, nwords, out, k, sm.scan_sh);
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
