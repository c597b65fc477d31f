// Memory-flat score -> top-k for many rows of one sequence (hipfire "QSA
// sparse attention ...", section 02: keep the best blocks within the budget,
// ties to the lower index; section 06: the selector's on-chip memory no
// longer holds long score rows; the chunked-prefill page, section 1: the
// [rows x context] score buffer is the memory peak of a prefill chunk).
//
// No score matrix is written.  Four launches:
//  1. sample   the many-row matrix-core kernel scores only the sampled block
//              of every 16-block group (score_prefill.hip, sample-only mode);
//  2. thresh   one workgroup per row histograms its sample over the 256-digit
//              window and takes the conservative threshold digit B (about
//              1.25 k + 256 blocks expected at or above it); it also clears
//              the row's candidate counter;
//  3. emit     the full matrix-core scoring appends every block whose digit
//              reaches B to the row's candidate slots (unordered, at most
//              kFlatCap; score_prefill.hip, emit mode);
//  4. finalize one workgroup per row finds the k-th largest candidate key TK
//              (histogram levels of 12, 10 and 10 bits), keeps the keys
//              above TK and, of the keys equal to TK, those with the lowest
//              block ids, and writes the kept ids in ascending order through
//              a bitmap of the row's blocks in LDS.
// One threshold per row makes the candidates exactly the blocks with digit
// >= B, so when their number lies in [k, kFlatCap] every block at or above
// TK is among them and the result is exact.  Otherwise (a misleading sample,
// massive ties, more than 512 keys equal to TK, or a row longer than the
// LDS bitmap) the finalize workgroup selects exactly over the whole row,
// recomputing each score from the index query and the pooled keys in float32
// on the vector ALU: exact for those scores, slow, and rare.
//
// The chunked-prefill page (section 2.3) reaches a flat memory line by
// blocking the key axis and merging per-block top-k lists; a per-row
// threshold reaches it without holding a per-block top-k for every row of a
// scoring workgroup, and with the same exactness.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "select_common.h"

namespace qsa {

namespace {

using sel::block_excl_scan;
using sel::find_digit_desc;
using sel::kDigits;
using sel::kDigitShift;
using sel::kFlatCap;
using sel::order_key;

constexpr int kThrThreads = 256;
constexpr int kFinThreads = 512;
constexpr int kFinPer = kFlatCap / kFinThreads;  // 8 candidate slots per thread
constexpr int kSpecPer = 3;                        // slots per thread loaded with the count (1,536)
constexpr int kLowBins = 1024;
constexpr int kMaxTies = 512;                      // keys equal to TK ranked on chip
constexpr int64_t kBitmapBlocks = 262144;          // rows up to 1M tokens take the candidate path
constexpr int kBitWords = (int)(kBitmapBlocks / 32);
constexpr float kScoreScale = 0.08838834764831845f;  // 1/sqrt(128)
static_assert(kFlatCap == 4096 && kFinPer == 8, "8 slots per finalize thread");

enum FlatPath : uint32_t {
  kPathAll = 1,
  kPathCandidates = 2,
  kPathExactLong = 3,   // the row is longer than the bitmap
  kPathExactCount = 4,  // candidate count below k or above kFlatCap
  kPathExactTies = 5,   // more than kMaxTies keys equal to TK
};

// Row threshold: histogram of the row's sample over the 256-digit window.
__global__ void __launch_bounds__(kThrThreads)
flat_threshold_kernel(const int64_t* __restrict__ row_pos, int64_t nb_max, int k, uint32_t* __restrict__ ws,
                      int M) {
  __shared__ uint32_t h[sel::kWinBins];
  __shared__ uint32_t out3[3];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const sel::FlatLayout L = sel::flat_layout(M, nb_max);
  const int64_t n_grp = sel::sample_groups(nb_max);
  const float* __restrict__ smp = reinterpret_cast<const float*>(ws + L.samples) + (int64_t)m * n_grp;
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  for (int i = tid; i < sel::kWinBins; i += kThrThreads) h[i] = 0u;
  __syncthreads();
  for (int64_t g = tid; g < n_grp; g += kThrThreads)
    if (g * 16 + sel::sample_offset((uint32_t)g) < nb) atomicAdd(&h[sel::win_bin(order_key(smp[g]))], 1u);
  __syncthreads();
  find_digit_desc<sel::kWinBins>(h, sel::sample_target((uint32_t)k), out3);
  if (tid == 0) {
    // window bin 0 (or a target never reached): every block is a candidate
    ws[L.thr + m] = (out3[2] || out3[0] == 0u) ? 0u : sel::kWinBase + out3[0];
    ws[L.cnt + m] = 0u;
  }
}

struct FlatSmem {
  uint32_t hist16[256 * 16];  // the 12-bit digit histogram; the exact path's radix passes
  uint32_t h2[kLowBins];
  uint32_t h3[kLowBins];
  uint32_t bits[kBitWords];   // kept blocks of the row
  uint32_t teq[kMaxTies];     // ids of the keys equal to TK
  float q[kIndexHeads * kIndexDim];
  uint32_t scan_sh[2 * (kFinThreads / kWave)];
  uint32_t out3[3];
  uint32_t n_eq;
};
static_assert(sizeof(FlatSmem) <= 160 * 1024, "fits the LDS of one compute unit");

// Score of block i recomputed in float32 (exact path of a failed row).
struct RecomputedScore {
  const float* q;  // LDS [4][128]
  const float* __restrict__ pooled;
  __device__ __forceinline__ float operator()(int64_t i) const {
    const float4* p = reinterpret_cast<const float4*>(pooled + i * kIndexDim);
    float a[kIndexHeads] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int d4 = 0; d4 < kIndexDim / 4; ++d4) {
      const float4 x = p[d4];
#pragma unroll
      for (int h = 0; h < kIndexHeads; ++h) {
        const float* qh = q + h * kIndexDim + 4 * d4;
        a[h] = fmaf(qh[0], x.x, a[h]);
        a[h] = fmaf(qh[1], x.y, a[h]);
        a[h] = fmaf(qh[2], x.z, a[h]);
        a[h] = fmaf(qh[3], x.w, a[h]);
      }
    }
    return (((fmaxf(a[0], 0.f) + fmaxf(a[1], 0.f)) + fmaxf(a[2], 0.f)) + fmaxf(a[3], 0.f)) * kScoreScale;
  }
};

__device__ void flat_exact(const uint16_t* __restrict__ idx_q_row, const float* __restrict__ pooled, int64_t nb,
                           int k, int32_t* out, FlatSmem& sm) {
  for (int i = threadIdx.x; i < kIndexHeads * kIndexDim; i += kFinThreads)
    sm.q[i] = __uint_as_float((uint32_t)idx_q_row[i] << 16);
  __syncthreads();
  sel::exact_select<kFinThreads>(RecomputedScore{sm.q, pooled}, nb, k, out, sm);
}

__global__ void __launch_bounds__(kFinThreads)
flat_finalize_kernel(const uint16_t* __restrict__ idx_q, const int64_t* __restrict__ row_pos,
                     const float* __restrict__ pooled, int64_t nb_max, int k, int32_t* __restrict__ sel,
                     int32_t* __restrict__ n_sel, uint32_t* __restrict__ ws, int M) {
  extern __shared__ __align__(16) unsigned char flat_lds[];
  FlatSmem& sm = *reinterpret_cast<FlatSmem*>(flat_lds);
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const sel::FlatLayout L = sel::flat_layout(M, nb_max);
  int32_t* __restrict__ out = sel + (int64_t)m * k;
  const uint16_t* q_row = idx_q + (int64_t)m * kIndexHeads * kIndexDim;
  // The first kSpecPer slots per thread and the count are loaded at once
  // (a row usually holds about 1.25 k + 256 candidates, well within them);
  // the other slots only when the count reaches past them.
  const uint2* P = reinterpret_cast<const uint2*>(ws + L.pairs) + (int64_t)m * kFlatCap;
  uint32_t kk[kFinPer], ii[kFinPer];
#pragma unroll
  for (int e = 0; e < kSpecPer; ++e) {
    const uint2 kv = P[e * kFinThreads + tid];
    kk[e] = kv.x;
    ii[e] = kv.y;
  }
  const uint32_t n_cand = ws[L.cnt + m];
#pragma unroll
  for (int e = kSpecPer; e < kFinPer; ++e) {
    kk[e] = 0u;
    ii[e] = 0u;
  }
  if (n_cand > (uint32_t)(kSpecPer * kFinThreads) && n_cand <= (uint32_t)kFlatCap) {  // uniform
#pragma unroll
    for (int e = kSpecPer; e < kFinPer; ++e) {
      const uint2 kv = P[e * kFinThreads + tid];
      kk[e] = kv.x;
      ii[e] = kv.y;
    }
  }
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  uint32_t* path = ws + L.path + m;
  if (nb <= k) {
    for (int i = tid; i < k; i += kFinThreads) out[i] = i < nb ? i : -1;
    if (tid == 0) {
      n_sel[m] = (int32_t)nb;
      *path = kPathAll;
    }
    return;
  }
  if (tid == 0) n_sel[m] = k;
  if (nb > kBitmapBlocks || n_cand < (uint32_t)k || n_cand > (uint32_t)kFlatCap) {
    if (tid == 0) *path = nb > kBitmapBlocks ? kPathExactLong : kPathExactCount;
    flat_exact(q_row, pooled, nb, k, out, sm);
    return;
  }
  for (int i = tid; i < kDigits; i += kFinThreads) sm.hist16[i] = 0u;
  for (int i = tid; i < kLowBins; i += kFinThreads) {
    sm.h2[i] = 0u;
    sm.h3[i] = 0u;
  }
  const int bit_words = (int)((nb + 31) / 32);
  for (int i = tid; i < bit_words; i += kFinThreads) sm.bits[i] = 0u;
  if (tid == 0) sm.n_eq = 0u;
  __syncthreads();
  uint32_t vm = 0u;  // which of kk/ii are live candidates
#pragma unroll
  for (int e = 0; e < kFinPer; ++e) {
    if ((uint32_t)(e * kFinThreads + tid) < n_cand) {
      atomicAdd(&sm.hist16[kk[e] >> kDigitShift], 1u);
      vm |= 1u << e;
    }
  }
  __syncthreads();
  // The k-th largest candidate key, 12 + 10 + 10 bits at a time; each level
  // counts only the candidates that share the bits found so far, and the
  // search stops once the cut bin is kept whole.
  find_digit_desc<kDigits>(sm.hist16, (uint32_t)k, sm.out3);
  uint32_t prefix = sm.out3[0];
  uint32_t need = sm.out3[1];
  int shift = kDigitShift;
  bool whole = sm.hist16[prefix] == need;
  if (!whole) {
#pragma unroll
    for (int e = 0; e < kFinPer; ++e)
      if (((vm >> e) & 1u) && (kk[e] >> kDigitShift) == prefix) atomicAdd(&sm.h2[(kk[e] >> 10) & (kLowBins - 1)], 1u);
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
    for (int e = 0; e < kFinPer; ++e)
      if (((vm >> e) & 1u) && (kk[e] >> 10) == prefix) atomicAdd(&sm.h3[kk[e] & (kLowBins - 1)], 1u);
    __syncthreads();
    find_digit_desc<kLowBins>(sm.h3, need, sm.out3);
    const uint32_t d3 = sm.out3[0];
    prefix = (prefix << 10) | d3;
    need = sm.out3[1];
    shift = 0;
    whole = sm.h3[d3] == need;
  }
  // Kept: keys above the cut, the whole cut bin when it fits; otherwise the
  // keys equal to TK (shift is 0 then) go to the tie list.
#pragma unroll
  for (int e = 0; e < kFinPer; ++e) {
    if (!((vm >> e) & 1u)) continue;
    const uint32_t kh = kk[e] >> shift;
    if (kh > prefix || (kh == prefix && whole)) {
      atomicOr(&sm.bits[ii[e] >> 5], 1u << (ii[e] & 31u));
    } else if (kh == prefix) {
      const uint32_t j = atomicAdd(&sm.n_eq, 1u);
      if (j < (uint32_t)kMaxTies) sm.teq[j] = ii[e];
    }
  }
  __syncthreads();
  const uint32_t n_eq = sm.n_eq;
  if (!whole) {
    if (n_eq > (uint32_t)kMaxTies) {
      if (tid == 0) *path = kPathExactTies;
      flat_exact(q_row, pooled, nb, k, out, sm);
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
  // kept ids in ascending order: each thread owns a run of bitmap words
  const int per = (bit_words + kFinThreads - 1) / kFinThreads;
  const int w0 = tid * per;
  uint32_t mine = 0u;
  for (int w = w0; w < w0 + per && w < bit_words; ++w) mine += (uint32_t)__popc(sm.bits[w]);
  uint32_t total;
  uint32_t pos = block_excl_scan<kFinThreads>(mine, sm.scan_sh, total);
  for (int w = w0; w < w0 + per && w < bit_words; ++w) {
    uint32_t b = sm.bits[w];
    while (b) {
      const int bit = __ffs(b) - 1;
      b &= b - 1u;
      if (pos < (uint32_t)k) out[pos] = w * 32 + bit;
      ++pos;
    }
  }
  if (tid == 0) *path = kPathCandidates;
}

}  // namespace

size_t score_select_workspace_bytes(int max_M, int64_t nb_max, int /*k_blocks*/) {
  return (size_t)sel::flat_layout(max_M, nb_max).total * sizeof(uint32_t);
}

hipError_t launch_score_select_flat(const void* idx_q, int M, const int64_t* row_pos, const float* pooled,
                                    int64_t nb_max, int k_blocks, int32_t* sel, int32_t* n_sel, void* ws,
                                    hipStream_t stream) {
  if (M == 0) return hipSuccess;
  uint32_t* W = static_cast<uint32_t*>(ws);
  if (nb_max > k_blocks) {
    hipError_t e = launch_score_prefill_flat(idx_q, M, row_pos, pooled, nb_max, k_blocks, W, false, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(flat_threshold_kernel, dim3((unsigned)M), dim3(kThrThreads), 0, stream, row_pos, nb_max,
                       k_blocks, W, M);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_score_prefill_flat(idx_q, M, row_pos, pooled, nb_max, k_blocks, W, true, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(flat_finalize_kernel, dim3((unsigned)M), dim3(kFinThreads), sizeof(FlatSmem), stream,
                     static_cast<const uint16_t*>(idx_q), row_pos, pooled, nb_max, k_blocks, sel, n_sel, W, M);
  return hipGetLastError();
}

}  // namespace qsa
