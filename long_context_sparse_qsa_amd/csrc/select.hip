// Top-k block selection (hipfire "QSA sparse attention ...", section 02:
// keep the top-scoring blocks within the token budget; section 03: a radix
// select follows the scoring).  Equal scores go to the lower block index.
//
// One workgroup of 1024 lanes per row.  Scores are mapped to order-preserving
// 32-bit keys (-0 first folded into +0).  Four 8-bit radix passes find the
// exact k-th largest key T and how many blocks equal to T still have to be
// taken.  A final pass compacts, in index order, every block with key > T
// and the first `need` blocks with key == T, which leaves the kept list
// sorted ascending with no sort.  Histograms live in LDS, replicated 16
// times (lane % 16 picks the copy) so that lanes hitting one bin do not
// serialise on one address.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 256;
constexpr int kCopies = 16;
constexpr int kPerThread = 4;  // consecutive elements per lane in the compaction pass

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;  // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive scan over the workgroup; `total` receives the workgroup sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < kWaves ? sh[lane] : 0u;
    x = wave_incl_scan(x, lane);
    if (lane < kWaves) sh[kWaves + lane] = x;
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? sh[kWaves + wave - 1] : 0u;
  total = sh[2 * kWaves - 1];
  __syncthreads();
  return before + incl - v;
}

__global__ void __launch_bounds__(kThreads)
select_radix_kernel(const float* __restrict__ scores, int64_t ld,
                    const int64_t* __restrict__ row_pos, int64_t nb_max, int k,
                    int32_t* __restrict__ sel, int32_t* __restrict__ n_sel) {
  __shared__ uint32_t hist[kCopies][kBins];
  __shared__ uint32_t scan_sh[2 * kWaves];
  __shared__ uint32_t pick[2];

  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int64_t nb = clamp_nb(row_pos[m], nb_max);
  const float* __restrict__ s = scores + (int64_t)m * ld;
  int32_t* __restrict__ out = sel + (int64_t)m * k;

  if (nb <= k) {
    for (int i = tid; i < k; i += kThreads) out[i] = i < nb ? i : -1;
    if (tid == 0) n_sel[m] = (int32_t)nb;
    return;
  }

  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kCopies * kBins; i += kThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    uint32_t* my = hist[lane & (kCopies - 1)];
    for (int64_t i = tid; i < nb; i += kThreads) {
      const uint32_t u = order_key(s[i]);
      if ((u & mask) == prefix) atomicAdd(&my[(u >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns bins 4l..4l+3; find the bin where the count from the top
      // reaches `remaining`.
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t t = 0;
#pragma unroll
        for (int cp = 0; cp < kCopies; ++cp) t += hist[cp][4 * lane + j];
        c[j] = t;
      }
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      // suffix sum over lanes above this one
      uint32_t suf = mine;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_down(suf, off, kWave);
        if (lane + off < kWave) suf += t;
      }
      uint32_t above = suf - mine;  // blocks in bins of higher lanes
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < remaining && above + c[j] >= remaining) {
          pick[0] = (uint32_t)(4 * lane + j);
          pick[1] = remaining - above;
        }
        above += c[j];
      }
    }
    __syncthreads();
    prefix |= pick[0] << shift;
    mask |= 0xffu << shift;
    remaining = pick[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need = remaining;  // blocks with key == T still to take (>= 1)

  uint32_t base_out = 0, base_eq = 0;
  for (int64_t c0 = 0; c0 < nb; c0 += (int64_t)kThreads * kPerThread) {
    const int64_t i0 = c0 + (int64_t)tid * kPerThread;
    uint32_t gt[kPerThread], eq[kPerThread];
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int64_t i = i0 + e;
      const uint32_t u = i < nb ? order_key(s[i]) : 0u;
      gt[e] = (i < nb) && (u > T);
      eq[e] = (i < nb) && (u == T);
      n_eq += eq[e];
    }
    uint32_t tot_eq;
    uint32_t eq_rank = base_eq + block_excl_scan(n_eq, scan_sh, tot_eq);
    uint32_t take[kPerThread];
    uint32_t n_take = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      take[e] = gt[e] || (eq[e] && eq_rank < need);
      eq_rank += eq[e];
      n_take += take[e];
    }
    uint32_t tot_take;
    uint32_t pos = base_out + block_excl_scan(n_take, scan_sh, tot_take);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (take[e] && pos < (uint32_t)k) out[pos] = (int32_t)(i0 + e);
      pos += take[e];
    }
    base_out += tot_take;
    base_eq += tot_eq;
  }
  if (tid == 0) n_sel[m] = k;
}

}  // namespace

size_t select_workspace_bytes(int /*max_M*/, int64_t /*nb_max*/, int /*k_blocks*/) { return 0; }

hipError_t launch_select_topk(const float* scores, int64_t ld, int M, const int64_t* row_pos,
                              int64_t nb_max, int k_blocks, int32_t* sel, int32_t* n_sel,
                              void* /*ws*/, size_t /*ws_bytes*/, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(select_radix_kernel, dim3(M), dim3(kThreads), 0, stream, scores, ld, row_pos,
                     nb_max, k_blocks, sel, n_sel);
  return hipGetLastError();
}

}  // namespace qsa
