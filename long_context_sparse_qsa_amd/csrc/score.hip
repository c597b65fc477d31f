// Block scoring (hipfire "QSA sparse attention ...", section 02: four
// index-query heads score every pooled block as the sum of their ReLU'd dot
// products times 1/sqrt(128); section 03: a few-row variant for decode and
// verify and a 16-row variant for prefill).
//
// Few-row variant (this file): the pass streams the float32 pooled keys
// (512 B per block) once for a group of up to 8 rows that share one
// sequence, so it is bound by HBM bandwidth.  One wave owns 64 consecutive
// blocks.  The tile is read from HBM in four 32-dimension slabs with fully
// coalesced 16-byte loads (each slab row is one 128-byte line), transposed
// through LDS so that each lane holds one block, and the next slab's loads
// are issued before the current slab is consumed.  The index queries are
// wave-uniform, so they live in scalar registers and every multiply-add is a
// single VALU op with a scalar operand.  Accumulation is float32.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kTile = 64;          // blocks per wave
constexpr int kSlab = 32;          // dimensions per slab
constexpr int kSlabs = kIndexDim / kSlab;
constexpr int kPad = 4;            // LDS row padding (floats): conflict-free 16 B reads
constexpr int kRow = kSlab + kPad;
constexpr float kScoreScale = 0.08838834764831845f;  // 1/sqrt(128)

// Four consecutive index-query values (wave-uniform address: scalar loads).
template <class EQ>
__device__ __forceinline__ void load_q4(const typename EQ::T* __restrict__ q, float* v);
template <>
__device__ __forceinline__ void load_q4<F32>(const float* __restrict__ q, float* v) {
  const float4 x = *reinterpret_cast<const float4*>(q);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
template <>
__device__ __forceinline__ void load_q4<BF16>(const uint16_t* __restrict__ q, float* v) {
  const uint2 x = *reinterpret_cast<const uint2*>(q);
  v[0] = __uint_as_float(x.x << 16);
  v[1] = __uint_as_float(x.x & 0xffff0000u);
  v[2] = __uint_as_float(x.y << 16);
  v[3] = __uint_as_float(x.y & 0xffff0000u);
}

template <class EQ, int MR>
__global__ void __launch_bounds__(kWave)
score_fewrow_kernel(const typename EQ::T* __restrict__ idx_q, int M,
                    const int64_t* __restrict__ row_pos, const int32_t* __restrict__ row_seq,
                    const float* __restrict__ pooled, int n_seq, int64_t capacity,
                    int64_t nb_max, float* __restrict__ scores, int64_t ld) {
  __shared__ float4 lds4[2][kTile * kRow / 4];
  const int lane = threadIdx.x;
  const int m0 = blockIdx.y * MR;
  const int rows = min(MR, M - m0);

  int64_t nb_r[MR];
  int64_t nb_hi = 0;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    nb_r[r] = r < rows ? clamp_nb(row_pos[m0 + r], nb_max) : 0;
    nb_hi = nb_r[r] > nb_hi ? nb_r[r] : nb_hi;
  }
  const int64_t b0 = (int64_t)blockIdx.x * kTile;
  if (b0 >= nb_hi) return;
  const int s = row_seq ? row_seq[m0] : 0;
  if (s < 0 || s >= n_seq) return;
  const float* __restrict__ P = pooled + (int64_t)s * (capacity / kBlockTokens) * kIndexDim;
  const typename EQ::T* __restrict__ Q = idx_q + (int64_t)m0 * kIndexHeads * kIndexDim;

  // Slab loads: float4 number f = j*64 + lane covers row f/8, column (f%8)*4.
  float4 pre[8];
  auto load_slab = [&](int c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = j * kWave + lane;
      const int r = f >> 3;
      const int64_t b = b0 + r;
      if (b < nb_hi) {
        pre[j] = *reinterpret_cast<const float4*>(P + b * kIndexDim + c * kSlab + (f & 7) * 4);
      } else {
        pre[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = j * kWave + lane;
      lds4[buf][(f >> 3) * (kRow / 4) + (f & 7)] = pre[j];
    }
  };

  float acc[MR][kIndexHeads];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int h = 0; h < kIndexHeads; ++h) acc[r][h] = 0.f;

  load_slab(0);
#pragma unroll 1
  for (int c = 0; c < kSlabs; ++c) {
    const int buf = c & 1;
    store_slab(buf);
    __syncthreads();
    if (c + 1 < kSlabs) load_slab(c + 1);
#pragma unroll 1
    for (int d4 = 0; d4 < kSlab / 4; ++d4) {
      const float4 p = lds4[buf][lane * (kRow / 4) + d4];
      const int dim0 = c * kSlab + d4 * 4;
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const int rr = r < rows ? r : 0;  // rows past the group end reuse row 0 (not stored)
#pragma unroll
        for (int h = 0; h < kIndexHeads; ++h) {
          float qv[4];
          load_q4<EQ>(Q + (rr * kIndexHeads + h) * kIndexDim + dim0, qv);
          float a = acc[r][h];
          a = fmaf(p.x, qv[0], a);
          a = fmaf(p.y, qv[1], a);
          a = fmaf(p.z, qv[2], a);
          a = fmaf(p.w, qv[3], a);
          acc[r][h] = a;
        }
      }
    }
  }

  const int64_t b = b0 + lane;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    if (r < rows && b < nb_r[r]) {
      float sum = fmaxf(acc[r][0], 0.f);
#pragma unroll
      for (int h = 1; h < kIndexHeads; ++h) sum += fmaxf(acc[r][h], 0.f);
      scores[(int64_t)(m0 + r) * ld + b] = sum * kScoreScale;
    }
  }
}

template <class EQ, int MR>
hipError_t launch_fewrow(const void* idx_q, int M, const int64_t* row_pos, const int32_t* row_seq,
                         const float* pooled, int n_seq, int64_t capacity, int64_t nb_max,
                         float* scores, int64_t ld, hipStream_t stream) {
  const int64_t tiles = (nb_max + kTile - 1) / kTile;
  if (tiles == 0) return hipSuccess;
  dim3 grid((unsigned)tiles, (unsigned)((M + MR - 1) / MR)), block(kWave);
  hipLaunchKernelGGL((score_fewrow_kernel<EQ, MR>), grid, block, 0, stream,
                     static_cast<const typename EQ::T*>(idx_q), M, row_pos, row_seq, pooled,
                     n_seq, capacity, nb_max, scores, ld);
  return hipGetLastError();
}

template <class EQ>
hipError_t dispatch_rows(const void* idx_q, int M, const int64_t* row_pos, const int32_t* row_seq,
                         const float* pooled, int n_seq, int64_t capacity, int64_t nb_max,
                         float* scores, int64_t ld, hipStream_t stream) {
  // Rows of different sequences read different pooled keys: score them one
  // by one.  Rows of one sequence share each pooled read in groups of <= 8.
  const int mr = row_seq ? 1 : (M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8);
  switch (mr) {
    case 1: return launch_fewrow<EQ, 1>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, stream);
    case 2: return launch_fewrow<EQ, 2>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, stream);
    case 4: return launch_fewrow<EQ, 4>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, stream);
    default: return launch_fewrow<EQ, 8>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, stream);
  }
}

}  // namespace

hipError_t launch_score_blocks(const void* idx_q, int dtype, int M, const int64_t* row_pos,
                               const int32_t* row_seq, const float* pooled, int n_seq,
                               int64_t capacity, int64_t nb_max, float* scores, int64_t ld,
                               hipStream_t stream) {
  if (M == 0 || nb_max == 0) return hipSuccess;
  if (dtype == QSA_BF16)
    return dispatch_rows<BF16>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, stream);
  return dispatch_rows<F32>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, stream);
}

}  // namespace qsa
