// Block scoring, many-row variant (hipfire "QSA sparse attention ...",
// section 03: a few-row variant for decode and verify and a 16-row variant
// for prefill; section 02 defines the score: four index-query heads, sum of
// their ReLU'd dot products with a pooled block key, times 1/sqrt(128)).
//
// Prefill chunks score thousands of rows of one sequence against the same
// pooled keys, a dense contraction: (rows x 4 heads) x 128 dims against
// blocks.  It runs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16) with
// float32 accumulation.  Index queries are bf16 already.  Each float32
// pooled key x is split into three bf16 planes, hi = bf16(x), mid =
// bf16(x - hi), lo = bf16(x - hi - mid), whose sum is x (24 significand
// bits); bf16 x bf16 products are exact in float32, so the three-plane sum
// matches a float32 dot product to float32 accumulation error, at three bf16
// matrix ops per float32 one (the bf16 rate is 16 times the float32 rate).
//
// Workgroup tile: 64 consecutive blocks x 128 rows.  The tile's pooled keys
// are loaded once (coalesced), split into planes and staged in LDS with
// padded 272-byte rows (A-operand reads are then free of bank conflicts).
// Each of the 4 waves owns 32 rows = 8 column groups of (4 rows x 4 heads)
// whose index-query operands stay in VGPRs; per 16-block group it runs
// 8 groups x 4 k-steps x 3 planes MFMAs, then ReLU's, sums the 4 heads with
// two lane shuffles and stores the scores.  Blocks at or past a row's own
// block count are not stored.  With a selection workspace the epilogue
// also stores the score sample of every 16-block group (as the few-row
// variant does).
//
// Two more modes serve the memory-flat score -> top-k (no score matrix):
//  - sample only: the tile's 64 A rows are the sampled blocks of 64
//    consecutive 16-block groups, and their scores go to the rows' samples;
//  - emit: after the full scoring, each row keeps only its blocks whose
//    score digit reaches the row's threshold.  A wave counts its rows'
//    candidates over the tile (ballots), reserves space with one atomic add
//    per row (all issued together, one round trip) and appends the (key,
//    block) pairs to the row's candidate slots in no particular order; slots
//    past the capacity are dropped (the count still records them, which
//    sends the row to the exact selection).
#include "qsa_device.h"
#include "qsa_internal.h"
#include "select_common.h"

namespace qsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum PfMode { kPfScores = 0, kPfScoresSample = 1, kPfSampleOnly = 2, kPfEmit = 3 };

// Memory-flat workspace views of one call (select_common.h, FlatLayout).
struct FlatArgs {
  const uint32_t* thr;
  uint32_t* cnt;
  float* samples;
  uint32_t* keys;
  uint32_t* ids;
  int64_t n_grp;
  int k;
};

constexpr int kPfWaves = 4;
constexpr int kPfRowsPerWave = 32;
constexpr int kPfRows = kPfWaves * kPfRowsPerWave;  // 128 rows per workgroup
constexpr int kPfCg = kPfRowsPerWave / 4;           // 8 column groups per wave
constexpr int kPfBlocks = 64;                       // blocks per workgroup
constexpr int kPfGroups = kPfBlocks / 16;           // 16-block MFMA row groups
constexpr int kPfKs = kIndexDim / 32;               // 4 k-steps of 32 dims
constexpr int kPfRowWords = kIndexDim / 2 + 4;      // bf16 plane row + 16 B pad, in 32-bit words
constexpr float kScoreScale = 0.08838834764831845f; // 1/sqrt(128)

// Three bf16 planes of a float32 value (round to nearest even each time).
__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(x);
  const float r1 = x - __uint_as_float(hi << 16);
  mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f32_to_bf16_bits(r2);
}

template <int MODE>
__global__ void __launch_bounds__(kWave * kPfWaves, 2)
score_prefill_kernel(const uint16_t* __restrict__ idx_q, int M, const int64_t* __restrict__ row_pos,
                     const float* __restrict__ pooled, int64_t nb_max, float* __restrict__ scores,
                     int64_t ld, uint32_t* __restrict__ ws, FlatArgs fa) {
  __shared__ __align__(16) uint32_t planes[3][kPfBlocks * kPfRowWords];
  __shared__ int64_t nb_sh[kPfRows];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int64_t b0 = (int64_t)blockIdx.x * kPfBlocks;  // first block (sample only: first sample group)
  const int r0 = blockIdx.y * kPfRows;

  // ---- loads: the tile's pooled keys (coalesced), this wave's index-query
  // operands, the tile's row positions
  constexpr int kF4 = kPfBlocks * kIndexDim / 4 / (kWave * kPfWaves);  // 8 float4 per thread
  float4 pk[kF4];
#pragma unroll
  for (int i = 0; i < kF4; ++i) {
    const int idx = tid + i * kWave * kPfWaves;  // float4 index inside the tile
    int64_t b = b0 + idx / (kIndexDim / 4);
    if constexpr (MODE == kPfSampleOnly) b = b * 16 + sel::sample_offset((uint32_t)b);  // the group's sampled block
    const int64_t bl = b < nb_max ? b : nb_max - 1;  // past the last block: re-read it, never stored
    pk[i] = *reinterpret_cast<const float4*>(pooled + bl * kIndexDim + (idx % (kIndexDim / 4)) * 4);
  }
  // B operand of column group cg: column n16 = (row 4 cg + n16 / 4, head n16 % 4),
  // k-step s: dims 32 s + 8 g4 .. + 7
  uint4 bq[kPfCg][kPfKs];
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg) {
    int r = r0 + wave * kPfRowsPerWave + 4 * cg + (n16 >> 2);
    r = r < M ? r : M - 1;
    const uint16_t* src = idx_q + ((int64_t)r * kIndexHeads + (n16 & 3)) * kIndexDim + 8 * g4;
#pragma unroll
    for (int s = 0; s < kPfKs; ++s) bq[cg][s] = *reinterpret_cast<const uint4*>(src + 32 * s);
  }
  __shared__ uint32_t thr_sh[kPfRows];
  if (tid < kPfRows) {
    const int r = r0 + tid;
    nb_sh[tid] = r < M ? clamp_nb(row_pos[r], nb_max) : 0;
    if constexpr (MODE == kPfEmit) thr_sh[tid] = r < M ? fa.thr[r] : 0u;
  }
  // ---- split into planes, stage in LDS
#pragma unroll
  for (int i = 0; i < kF4; ++i) {
    const int idx = tid + i * kWave * kPfWaves;
    const int blk = idx / (kIndexDim / 4);
    const int d4 = idx % (kIndexDim / 4);
    uint32_t h[4], md[4], lo[4];
    split3(pk[i].x, h[0], md[0], lo[0]);
    split3(pk[i].y, h[1], md[1], lo[1]);
    split3(pk[i].z, h[2], md[2], lo[2]);
    split3(pk[i].w, h[3], md[3], lo[3]);
    const int w = blk * kPfRowWords + d4 * 2;  // 4 bf16 = 2 words
    *reinterpret_cast<uint2*>(&planes[0][w]) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    *reinterpret_cast<uint2*>(&planes[1][w]) = make_uint2(md[0] | (md[1] << 16), md[2] | (md[3] << 16));
    *reinterpret_cast<uint2*>(&planes[2][w]) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
  }
  __syncthreads();

  int64_t nb_row[kPfCg];
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg) nb_row[cg] = nb_sh[wave * kPfRowsPerWave + 4 * cg + (n16 >> 2)];
  const int64_t rw = sel::row_words(nb_max);
  const int64_t smp_off = sel::sample_off(nb_max);

  // emit mode: the key of the lane's block in every (16-block group, column
  // group), which of them are candidates, and the candidates of the lane's
  // row so far (the 16-block groups are unrolled so the keys stay in VGPRs)
  uint32_t ekey[kPfGroups][kPfCg];
  uint32_t eflag = 0u;
  uint32_t run[kPfCg];
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg) run[cg] = 0u;
  const uint64_t rmask = 0x000F000F000F000Full << (4 * (n16 >> 2));  // the lane's row in a ballot
  (void)ekey;

#pragma unroll
  for (int bg = 0; bg < kPfGroups; ++bg) {
    f32x4_t acc[kPfCg];
#pragma unroll
    for (int cg = 0; cg < kPfCg; ++cg) acc[cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kPfKs; ++s) {
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        // A operand: block bg*16 + n16, dims 32 s + 8 g4 .. + 7 of plane pl
        const uint4 a = *reinterpret_cast<const uint4*>(
            &planes[pl][(bg * 16 + n16) * kPfRowWords + (32 * s + 8 * g4) / 2]);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
        for (int cg = 0; cg < kPfCg; ++cg)
          acc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bq[cg][s]), acc[cg],
                                                           0, 0, 0);
      }
    }
    // acc[cg][v] = D[4 g4 + v][n16]: block b0 + 16 bg + 4 g4 + v, column n16
    const int64_t bb = b0 + bg * 16 + 4 * g4;
#pragma unroll
    for (int cg = 0; cg < kPfCg; ++cg) {
      float sv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = fmaxf(acc[cg][v], 0.f);
        x += __shfl_xor(x, 1, kWave);
        x += __shfl_xor(x, 2, kWave);
        sv[v] = x * kScoreScale;
      }
      const int r = r0 + wave * kPfRowsPerWave + 4 * cg + (n16 >> 2);
      // sample-only and emit: lane t = n16 % 4 of the row's quad takes slot t
      const int t = n16 & 3;
      const float xt = t == 0 ? sv[0] : (t == 1 ? sv[1] : (t == 2 ? sv[2] : sv[3]));
      if constexpr (MODE == kPfScores || MODE == kPfScoresSample) {
        if ((n16 & 3) == 0 && r < M) {
          float* dst = scores + (int64_t)r * ld + bb;
          if (bb + 3 < nb_row[cg]) {
            *reinterpret_cast<float4*>(dst) = make_float4(sv[0], sv[1], sv[2], sv[3]);
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (bb + v < nb_row[cg]) dst[v] = sv[v];
          }
          if constexpr (MODE == kPfScoresSample) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (bb + v < nb_row[cg] && sel::sampled((uint32_t)(bb + v)))
                reinterpret_cast<float*>(ws)[(size_t)r * rw + smp_off + ((bb + v) >> 4)] = sv[v];
          }
        }
      }
      if constexpr (MODE == kPfSampleOnly) {  // slot = sample group bb + t
        const int64_t g = bb + t;
        if (r < M && g < fa.n_grp && g * 16 + sel::sample_offset((uint32_t)g) < nb_row[cg])
          fa.samples[(int64_t)r * fa.n_grp + g] = xt;
      }
      if constexpr (MODE == kPfEmit) {  // slot = block bb + t
        const uint32_t key = sel::order_key(xt);
        const int rl = wave * kPfRowsPerWave + 4 * cg + (n16 >> 2);
        const bool c = r < M && bb + t < nb_row[cg] && nb_row[cg] > fa.k &&
                       (key >> sel::kDigitShift) >= thr_sh[rl];
        ekey[bg][cg] = key;
        eflag |= c ? 1u << (bg * kPfCg + cg) : 0u;
        run[cg] += (uint32_t)__popcll(__ballot(c) & rmask);
      }
    }
  }

  if constexpr (MODE == kPfEmit) {
    // reserve each row's slots: one atomic per row, all in flight together
    uint32_t base[kPfCg];
#pragma unroll
    for (int cg = 0; cg < kPfCg; ++cg) {
      const int r = r0 + wave * kPfRowsPerWave + 4 * cg + (n16 >> 2);
      uint32_t b = 0u;
      if (g4 == 0 && (n16 & 3) == 0 && r < M && run[cg] > 0u) b = atomicAdd(fa.cnt + r, run[cg]);
      base[cg] = b;
    }
    const uint64_t lane_lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int cg = 0; cg < kPfCg; ++cg) {
      const int r = r0 + wave * kPfRowsPerWave + 4 * cg + (n16 >> 2);
      uint32_t pos = (uint32_t)__shfl((int)base[cg], n16 & ~3, kWave);  // from lane 4 (n16 / 4)
#pragma unroll
      for (int bg = 0; bg < kPfGroups; ++bg) {
        const bool c = (eflag >> (bg * kPfCg + cg)) & 1u;
        const uint64_t mk = __ballot(c) & rmask;
        const uint32_t p = pos + (uint32_t)__popcll(mk & lane_lt);
        if (c && p < (uint32_t)sel::kFlatCap) {
          fa.keys[(int64_t)r * sel::kFlatCap + p] = ekey[bg][cg];
          fa.ids[(int64_t)r * sel::kFlatCap + p] = (uint32_t)(b0 + bg * 16 + 4 * g4 + (n16 & 3));
        }
        pos += (uint32_t)__popcll(mk);
      }
    }
  }
}

}  // namespace

hipError_t launch_score_prefill(const void* idx_q, int M, const int64_t* row_pos, const float* pooled,
                                int64_t nb_max, float* scores, int64_t ld, uint32_t* sel_ws,
                                hipStream_t stream) {
  if (M == 0 || nb_max == 0) return hipSuccess;
  dim3 grid((unsigned)((nb_max + kPfBlocks - 1) / kPfBlocks), (unsigned)((M + kPfRows - 1) / kPfRows));
  const FlatArgs none{};
  if (sel_ws)
    hipLaunchKernelGGL(score_prefill_kernel<kPfScoresSample>, grid, dim3(kWave * kPfWaves), 0, stream,
                       static_cast<const uint16_t*>(idx_q), M, row_pos, pooled, nb_max, scores, ld, sel_ws, none);
  else
    hipLaunchKernelGGL(score_prefill_kernel<kPfScores>, grid, dim3(kWave * kPfWaves), 0, stream,
                       static_cast<const uint16_t*>(idx_q), M, row_pos, pooled, nb_max, scores, ld, nullptr, none);
  return hipGetLastError();
}

hipError_t launch_score_prefill_flat(const void* idx_q, int M, const int64_t* row_pos, const float* pooled,
                                     int64_t nb_max, int k_blocks, uint32_t* ws, bool emit, hipStream_t stream) {
  if (M == 0 || nb_max == 0) return hipSuccess;
  const sel::FlatLayout L = sel::flat_layout(M, nb_max);
  FlatArgs fa;
  fa.thr = ws + L.thr;
  fa.cnt = ws + L.cnt;
  fa.samples = reinterpret_cast<float*>(ws + L.samples);
  fa.keys = ws + L.keys;
  fa.ids = ws + L.ids;
  fa.n_grp = sel::sample_groups(nb_max);
  fa.k = k_blocks;
  const unsigned gy = (unsigned)((M + kPfRows - 1) / kPfRows);
  if (emit) {
    dim3 grid((unsigned)((nb_max + kPfBlocks - 1) / kPfBlocks), gy);
    hipLaunchKernelGGL(score_prefill_kernel<kPfEmit>, grid, dim3(kWave * kPfWaves), 0, stream,
                       static_cast<const uint16_t*>(idx_q), M, row_pos, pooled, nb_max, nullptr, 0, nullptr, fa);
  } else {
    dim3 grid((unsigned)((fa.n_grp + kPfBlocks - 1) / kPfBlocks), gy);
    hipLaunchKernelGGL(score_prefill_kernel<kPfSampleOnly>, grid, dim3(kWave * kPfWaves), 0, stream,
                       static_cast<const uint16_t*>(idx_q), M, row_pos, pooled, nb_max, nullptr, 0, nullptr, fa);
  }
  return hipGetLastError();
}

}  // namespace qsa
