// Block scoring, many-row variant (hipfire "QSA sparse attention ...",
// section 03: a few-row variant for decode and verify and a 16-row variant
// for prefill; section 02 defines the score: four index-query heads, sum of
// their ReLU'd dot products with a pooled block key, times 1/sqrt(128)).
//
// Prefill chunks score thousands of rows of one sequence against the same
// pooled keys, a dense contraction: (rows x 4 heads) x 128 dims against
// blocks.  It runs on the bf16 matrix cores with float32 accumulation, on
// v_mfma_f32_32x32x16_bf16 (on this chip it sustains twice the rate of the
// 16x16x32 form).  Index queries are bf16 already.  Each float32 pooled key
// x is split into three bf16 planes, hi = bf16(x), mid = bf16(x - hi), lo =
// bf16(x - hi - mid), whose sum is x (24 significand bits); bf16 x bf16
// products are exact in float32, so the three-plane sum matches a float32
// dot product to float32 accumulation error, at three bf16 matrix ops per
// float32 one.
//
// Operands: A = 32 (row, head) pairs (8 rows x 4 heads) x 16 dims of index
// queries, B = 16 dims x 32 blocks of one pooled plane.  An output lane then
// holds, for its block, the 4 heads of each of its rows in consecutive
// accumulator registers, so the ReLU'd head sum needs no lane exchange.
//
// Work: tiles of 64 consecutive blocks x 128 rows.  A workgroup (8 waves,
// 16 rows each, one workgroup per compute unit) keeps its rows' index-query
// operands in VGPRs and walks a contiguous run of block tiles.  LDS holds
// two tiles' planes (padded 272-byte rows): while a tile is multiplied, the
// next one is split and staged and the one after it is loading.  Per
// 32-block group a wave runs 2 row groups x 8 k-steps x 3 planes MFMAs; the
// group's epilogue runs next to the following group's matrix work (two
// accumulator sets alternate).  Blocks at or past a row's own block count
// are not stored: stores go through buffer views of the wave's rows, and a
// masked lane's offset lies past the view, which the hardware drops.
//
// Modes:
//  - scores (and, with a selection workspace, the score sample of every
//    16-block group, as the few-row variant stores it);
//  - sample only (memory-flat selection): the tile's 64 B columns are the
//    sampled blocks of 64 consecutive 16-block groups, and their scores go
//    to the rows' samples;
//  - emit (memory-flat selection): each row keeps only its blocks whose
//    score digit reaches the row's threshold.  Per 32-block group a wave
//    counts its rows' candidates (ballots), reserves space with one atomic
//    add per row (all issued together; the result is used a group of matrix
//    work later) and appends the (key, block) pairs to the row's candidate
//    slots in no particular order; slots past the capacity are dropped (the
//    count still records them, which sends the row to the exact selection).
//    The epilogue takes no branch (ballots of the comparisons, a lane write
//    for the counts, buffer atomics and stores whose masked lanes fall
//    outside the view), so the whole tile stays one block of straight-line
//    code and the compiler interleaves the epilogue with the matrix work; a
//    branch per output row, as a conditional store makes, cuts the loop into
//    small blocks that the scheduler cannot overlap.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "select_common.h"

namespace qsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));

enum PfMode { kPfScores = 0, kPfScoresSample = 1, kPfSampleOnly = 2, kPfEmit = 3 };

// Memory-flat workspace views of one call (select_common.h, FlatLayout).
struct FlatArgs {
  const uint32_t* thr;
  uint32_t* cnt;
  float* samples;
  uint32_t* pairs;
  int64_t n_grp;
  int k;
};

constexpr int kPfWaves = 8;
constexpr int kPfRowsPerWave = 16;
constexpr int kPfRows = kPfWaves * kPfRowsPerWave;  // 128 rows per workgroup
constexpr int kPfCg = kPfRowsPerWave / 8;           // 2 groups of 8 rows (32 (row, head) pairs) per wave
constexpr int kPfBlocks = 64;                       // blocks per tile
constexpr int kPfBg = kPfBlocks / 32;               // 32-block MFMA column groups per tile
constexpr int kPfKs = kIndexDim / 16;               // 8 k-steps of 16 dims
constexpr int kPfRowWords = kIndexDim / 2 + 4;      // bf16 plane row + 16 B pad, in 32-bit words
constexpr int kPfSlots = 256;                       // workgroups in flight: 1 per compute unit
constexpr int kXcds = 8;                            // accelerator dies (each with its own L2)
constexpr int kPfF4 = kPfBlocks * kIndexDim / 4 / (kWave * kPfWaves);  // 4 float4 per thread per tile
constexpr float kScoreScale = 0.08838834764831845f; // 1/sqrt(128)
constexpr int kBufferWord3 = 0x00020000;            // raw buffer view (gfx9 family)
constexpr int kBufferDrop = (int)0x80000000u;       // an offset past any view: the store is dropped
constexpr int64_t kPfMaxView = (int64_t)1 << 31;    // bytes of a buffer view

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two float32 values to packed bf16 (first in the low half), rounded to
// nearest even by the hardware conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Three bf16 planes of two float32 values, packed in pairs: hi = bf16(x),
// mid = bf16(x - hi), lo = bf16(x - hi - mid).  Each difference is exact in
// float32 (it keeps at most 16, then 8, significant bits), so hi + mid + lo
// = x whenever 2^-110 <= |x| <= the largest finite bf16 (about 3.39e38).
// Below 2^-110 the lo plane would need bits finer than bf16's subnormal
// spacing (2^-133) and the last bits of x are lost; above the bf16 range hi
// overflows.  Pooled keys (averages of unit-scale values) sit far inside.
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  const float ra = a - __uint_as_float(hi << 16);
  const float rb = b - __uint_as_float(hi & 0xffff0000u);
  mid = pack_bf16x2(ra, rb);
  lo = pack_bf16x2(ra - __uint_as_float(mid << 16), rb - __uint_as_float(mid & 0xffff0000u));
}

// max(x, 0) on the bit pattern: a float with the sign bit set is a negative
// integer (one instruction; -0 gives +0).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// The pooled keys of tile t (coalesced: float4 idx of the tile per thread
// and step); in sample-only mode the tile's blocks are the sampled blocks of
// 64 consecutive 16-block groups.
template <int MODE>
__device__ __forceinline__ void load_tile(const float* __restrict__ pooled, int64_t nb_max, int64_t t, int tid,
                                          float4 (&pk)[kPfF4]) {
#pragma unroll
  for (int i = 0; i < kPfF4; ++i) {
    const int idx = tid + i * kWave * kPfWaves;
    int64_t b = t * kPfBlocks + idx / (kIndexDim / 4);
    if constexpr (MODE == kPfSampleOnly) b = b * 16 + sel::sample_offset((uint32_t)b);
    const int64_t bl = b < nb_max ? b : nb_max - 1;  // past the last block: re-read it, never stored
    pk[i] = *reinterpret_cast<const float4*>(pooled + bl * kIndexDim + (idx % (kIndexDim / 4)) * 4);
  }
}

// Splits a tile's pooled keys (as load_tile leaves them) into the three
// planes and stages them in LDS.
__device__ __forceinline__ void stage_tile(const float4 (&pk)[kPfF4], int tid, uint32_t (*planes)[kPfBlocks * kPfRowWords]) {
#pragma unroll
  for (int i = 0; i < kPfF4; ++i) {
    const int idx = tid + i * kWave * kPfWaves;
    const int blk = idx / (kIndexDim / 4);
    const int d4 = idx % (kIndexDim / 4);
    uint2 hi, md, lo;
    split3_pair(pk[i].x, pk[i].y, hi.x, md.x, lo.x);
    split3_pair(pk[i].z, pk[i].w, hi.y, md.y, lo.y);
    const int w = blk * kPfRowWords + d4 * 2;  // 4 bf16 = 2 words
    *reinterpret_cast<uint2*>(&planes[0][w]) = hi;
    *reinterpret_cast<uint2*>(&planes[1][w]) = md;
    *reinterpret_cast<uint2*>(&planes[2][w]) = lo;
  }
}

// One 32-block group's matrix work: acc[cg] += A(row group cg) x B(group
// bg of the staged tile), over 8 k-steps x 3 planes.
__device__ __forceinline__ void group_mfma(const uint32_t (*planes)[kPfBlocks * kPfRowWords], int bg, int j32, int h,
                                           const uint4 (&aq)[kPfCg][kPfKs], f32x16_t (&acc)[kPfCg]) {
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[cg][e] = 0.f;
  // B operand of step i = (k-step s, plane pl): block bg*32 + j32, dims
  // 16 s + 8 h .. + 7 of plane pl; step i + 1's is read before step i's
  // matrix instructions issue, so the LDS latency overlaps them
  const uint32_t* bsrc = &planes[0][(bg * 32 + j32) * kPfRowWords + 4 * h];
  auto bload = [&](int i) {
    const int s = i / 3, pl = i % 3;
    return *reinterpret_cast<const uint4*>(bsrc + pl * (kPfBlocks * kPfRowWords) + 8 * s);
  };
  uint4 bv = bload(0);
#pragma unroll
  for (int i = 0; i < kPfKs * 3; ++i) {
    const uint4 bn = i + 1 < kPfKs * 3 ? bload(i + 1) : bv;
#pragma unroll
    for (int cg = 0; cg < kPfCg; ++cg)
      acc[cg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aq[cg][i / 3]),
                                                       __builtin_bit_cast(bf16x8_t, bv), acc[cg], 0, 0, 0);
    bv = bn;
  }
}

// Epilogue of one 32-block group in the score-writing modes: the lane's
// block b, rows 8 cg + 2q + h of the wave (acc[cg][4q + hd] = head hd), all
// stores through the wave's buffer views (masked lanes dropped, no branch).
template <bool HIST>
__device__ __forceinline__ void group_store(const f32x16_t (&acc)[kPfCg], int64_t b, bool valid, int h,
                                            const int (&nbq)[kPfCg][4], __amdgpu_buffer_rsrc_t srs,
                                            __amdgpu_buffer_rsrc_t wrs, int64_t ld, int64_t rw, int64_t smp_off) {
  const bool smp = sel::sampled((uint32_t)b);
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float x = relu(acc[cg][4 * q]) + relu(acc[cg][4 * q + 1]);
      x += relu(acc[cg][4 * q + 2]) + relu(acc[cg][4 * q + 3]);
      x *= kScoreScale;
      const int rr = 8 * cg + 2 * q + h;
      const bool keep = valid && b < nbq[cg][q];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), srs, keep ? (int)((rr * ld + b) * 4) : kBufferDrop,
                                            0, 0);
      if constexpr (HIST)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), wrs,
                                              keep && smp ? (int)((rr * rw + smp_off + (b >> 4)) * 4) : kBufferDrop,
                                              0, 0);
    }
  }
}

// Sample-only mode's epilogue of one 32-block group: column b is sample
// group b (its sampled block), whose score goes to the row's sample slot
// through the wave's buffer view of the sample rows.
__device__ __forceinline__ void group_sample(const f32x16_t (&acc)[kPfCg], int64_t b, bool valid, int h,
                                             const int (&nbq)[kPfCg][4], __amdgpu_buffer_rsrc_t srs, int64_t n_grp) {
  const int64_t blk = b * 16 + sel::sample_offset((uint32_t)b);
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float x = relu(acc[cg][4 * q]) + relu(acc[cg][4 * q + 1]);
      x += relu(acc[cg][4 * q + 2]) + relu(acc[cg][4 * q + 3]);
      x *= kScoreScale;
      const int rr = 8 * cg + 2 * q + h;
      const bool keep = valid && b < n_grp && blk < nbq[cg][q];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), srs, keep ? (int)((rr * n_grp + b) * 4) : kBufferDrop,
                                            0, 0);
    }
  }
}

// Emit mode's record of one 32-block group: the keys of the lane's 8
// outputs (row group cg, row pair q) and (lane L < 16) the candidate count
// of row L of the wave.  Whether an output is a candidate is recomputed from
// its key where it is needed.
struct EmitRec {
  u32x8_t key;  // a vector value, not an array, so the record stays in registers
  uint32_t run;
};

// Order key of a score of this kernel: the scores are sums of ReLU'd terms
// (never negative, never -0), where the order key (select_common.h) is the
// bit pattern with the sign bit set.
__device__ __forceinline__ uint32_t nonneg_key(float x) { return __float_as_uint(x) | 0x80000000u; }

// Emit mode's candidate test: block b is visible to the row (b < nbe,
// unsigned; nbe is 0 for rows that keep all their blocks and b is -1, above
// every nbe, for a group that holds no blocks of this workgroup) and its
// key's digit reaches the row's threshold digit (key >= thk, the digit
// shifted into place).  The ballot is taken of each comparison on its own
// (each is the comparison's own result).
__device__ __forceinline__ uint64_t cand_ballot(bool vis, bool reach) {
  return __builtin_amdgcn_ballot_w64(vis) & __builtin_amdgcn_ballot_w64(reach);
}

// v_writelane (the compiler's intrinsic, which has no builtin here): lane
// `lane` of the result is the wave-uniform x, the other lanes are v's.
extern "C" __device__ int qsa_writelane_i32(int x, int lane, int v) __asm("llvm.amdgcn.writelane.i32");

// Emit mode's epilogue of one 32-block group: keys, and each row's
// candidate count by ballot.  Branch-free, so the compiler can interleave it
// with the matrix instructions.
__device__ __forceinline__ void group_emit(const f32x16_t (&acc)[kPfCg], int b, const int (&nbe)[kPfCg][4],
                                           const uint32_t (&thk)[kPfCg][4], EmitRec& rec) {
  int run = 0;
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float x = relu(acc[cg][4 * q]) + relu(acc[cg][4 * q + 1]);
      x += relu(acc[cg][4 * q + 2]) + relu(acc[cg][4 * q + 3]);
      x *= kScoreScale;
      const uint32_t key = nonneg_key(x);
      rec.key[cg * 4 + q] = key;
      const uint64_t m = cand_ballot((uint32_t)b < (uint32_t)nbe[cg][q], key >= thk[cg][q]);
      run = qsa_writelane_i32(__popc((uint32_t)m), 8 * cg + 2 * q, run);              // row 8 cg + 2q
      run = qsa_writelane_i32(__popc((uint32_t)(m >> 32)), 8 * cg + 2 * q + 1, run);  // row 8 cg + 2q + 1
    }
  }
  rec.run = (uint32_t)run;
}

// Emit mode: appends a finished group's candidates (lane block b) to their
// rows' slots from the bases its reservation returned (lane L < 16: row L's
// base).  prs views the wave's 16 rows of (key, id) slots; a candidate's
// slot is its row's base plus the number of candidates of the same row in
// lower lanes.  Stores of non-candidates and of slots past kFlatCap go to
// an offset outside the view and are dropped, so no branch is taken.
__device__ __forceinline__ void scatter_emit(const EmitRec& rec, uint32_t base, int b, int h,
                                             const int (&nbe)[kPfCg][4], const uint32_t (&thk)[kPfCg][4],
                                             __amdgpu_buffer_rsrc_t prs) {
  const uint32_t lower = h ? 0u : ~0u;  // the lower half's ballot bits count for lanes below 32 only
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rw8 = 8 * cg + 2 * q + h;
      const uint32_t key = rec.key[cg * 4 + q];
      const bool vis = (uint32_t)b < (uint32_t)nbe[cg][q], reach = key >= thk[cg][q];
      const uint64_t m = cand_ballot(vis, reach);
      // rank among the lane's half (row) of the ballot: the upper lanes
      // count no lower-half bits (lanes below 32 see no upper-half bits)
      const uint32_t rank =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m & lower, 0u));
      const uint32_t p = (uint32_t)__builtin_amdgcn_ds_bpermute(rw8 * 4, (int)base) + rank;
      const bool keep = vis & reach & (p < (uint32_t)sel::kFlatCap);
      const u32x2_t v = {key, (uint32_t)b};
      __builtin_amdgcn_raw_buffer_store_b64(v, prs, keep ? (int)((rw8 * sel::kFlatCap + (int)p) * 8) : kBufferDrop,
                                            0, 0);
    }
  }
}

// The score-writing modes and the emit mode, software-pipelined: each
// 32-block group's matrix work is issued next to the previous group's
// epilogue (and, for a tile's second group, next to the staging of the
// following tile), so the vector ALU and memory work hides behind the
// matrix instructions.  Two accumulator sets alternate: accA takes a tile's
// first group, accB its second, whose epilogue runs during the next tile's
// first group.  The two LDS buffers are separate arrays and the tile loop is
// unrolled by two, so the compiler sees that staging and matrix reads never
// touch the same words.  In emit mode a tile's slot reservation (one atomic
// per row) is issued once its second group is done and consumed a group of
// matrix work later, so the atomics' round trip hides behind it too.
template <int MODE>
__global__ void __launch_bounds__(kWave * kPfWaves, 1)
score_prefill_pipe_kernel(const uint16_t* __restrict__ idx_q, int M, const int64_t* __restrict__ row_pos,
                          const float* __restrict__ pooled, int64_t nb_max, float* __restrict__ scores, int64_t ld,
                          uint32_t* __restrict__ ws, FlatArgs fa, int n_rt, int64_t n_tiles, int n_chunks) {
  constexpr bool HIST = MODE == kPfScoresSample;
  constexpr bool EMIT = MODE == kPfEmit;
  constexpr bool SAMPLE = MODE == kPfSampleOnly;
  __shared__ __align__(16) uint32_t planes0[3][kPfBlocks * kPfRowWords];
  __shared__ __align__(16) uint32_t planes1[3][kPfBlocks * kPfRowWords];
  __shared__ int nb_sh[kPfRows];
  __shared__ uint32_t thr_sh[kPfRows];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int j32 = lane & 31;
  const int h = lane >> 5;
  int rt, chunk;
  if (n_chunks % kXcds == 0) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    rt = slot % n_rt;
    chunk = (slot / n_rt) * kXcds + xcd;
  } else {
    rt = blockIdx.x % n_rt;
    chunk = blockIdx.x / n_rt;
  }
  const int64_t t_begin = n_tiles * chunk / n_chunks;
  const int64_t t_end = n_tiles * (chunk + 1) / n_chunks;
  if (t_begin >= t_end) return;
  const int r0 = rt * kPfRows;
  // the selection that consumes the sample counts its chunks in from zero
  if (HIST && chunk == 0 && tid < kPfRows && r0 + tid < M)
    ws[(size_t)(r0 + tid) * sel::row_words(nb_max) + sel::kArriveWord] = 0u;

  uint4 aq[kPfCg][kPfKs];
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg) {
    int r = r0 + wave * kPfRowsPerWave + 8 * cg + (j32 >> 2);
    r = r < M ? r : M - 1;
    const uint16_t* src = idx_q + ((int64_t)r * kIndexHeads + (j32 & 3)) * kIndexDim + 8 * h;
#pragma unroll
    for (int s = 0; s < kPfKs; ++s) aq[cg][s] = *reinterpret_cast<const uint4*>(src + 16 * s);
  }
  float4 pk[kPfF4];
  load_tile<MODE>(pooled, nb_max, t_begin, tid, pk);  // after the queries: its wait covers them
  if (tid < kPfRows) {
    const int r = r0 + tid;
    nb_sh[tid] = r < M ? (int)clamp_nb(row_pos[r], nb_max) : 0;  // nb_max < 2^31 (launcher)
    if constexpr (EMIT) thr_sh[tid] = r < M ? fa.thr[r] : 0u;
  }
  const int64_t rw = sel::row_words(nb_max);
  const int64_t smp_off = sel::sample_off(nb_max);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform
  const int64_t wrow0 = r0 + wave_u * kPfRowsPerWave;
  // score rows (sample-only mode: sample rows; emit mode: none, the views
  // are empty and unused)
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      EMIT ? nullptr : SAMPLE ? static_cast<void*>(fa.samples + wrow0 * fa.n_grp) : scores + wrow0 * ld, 0,
      EMIT ? 0 : SAMPLE ? (int)(kPfRowsPerWave * fa.n_grp * 4) : (int)(kPfRowsPerWave * ld * 4), kBufferWord3);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      EMIT || !ws ? nullptr : reinterpret_cast<float*>(ws) + wrow0 * rw, 0,
      EMIT || !ws ? 0 : (int)(kPfRowsPerWave * rw * 4), kBufferWord3);

  stage_tile(pk, tid, planes0);
  load_tile<MODE>(pooled, nb_max, t_begin + 1 < t_end ? t_begin + 1 : t_end - 1, tid, pk);
  __syncthreads();
  // each (row group, row pair)'s visible block count; in emit mode 0 for
  // rows that keep all their blocks (they have no candidates), and the
  // row's threshold digit shifted into key position
  int nbq[kPfCg][4];
  uint32_t thk[kPfCg][4];
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = wave * kPfRowsPerWave + 8 * cg + 2 * q + h;
      const int nb = nb_sh[rr];
      nbq[cg][q] = EMIT && nb <= fa.k ? 0 : nb;
      thk[cg][q] = EMIT ? thr_sh[rr] << sel::kDigitShift : 0u;
    }

  f32x16_t accA[kPfCg], accB[kPfCg];
#pragma unroll
  for (int cg = 0; cg < kPfCg; ++cg)
#pragma unroll
    for (int e = 0; e < 16; ++e) accB[cg][e] = 0.f;
  // emit mode: each group's record is reserved right after its epilogue and
  // scattered after the next group's matrix work (recA: a tile's first
  // group, recB: its second)
  EmitRec recA{}, recB{};
  uint32_t baseA = 0u;
  // the wave's rows' candidate counters and (key, id) slots; rows past M
  // are outside both views
  const int64_t wrows = EMIT ? (M - wrow0 < 0 ? 0 : M - wrow0 < kPfRowsPerWave ? M - wrow0 : kPfRowsPerWave) : 0;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(EMIT ? fa.cnt + wrow0 : nullptr, 0,
                                                                       (int)(wrows * 4), kBufferWord3);
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      EMIT ? fa.pairs + wrow0 * sel::kFlatCap * 2 : nullptr, 0, (int)(wrows * sel::kFlatCap * 8), kBufferWord3);
  // reserve a finished record's slots: one atomic per row (lane L < 16: row
  // L; the other lanes' atomics are dropped and return zero)
  auto reserve = [&](const EmitRec& rec) -> uint32_t {
    const bool act = lane < kPfRowsPerWave && rec.run > 0u;
    return (uint32_t)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32((int)rec.run, crs, act ? lane * 4 : kBufferDrop,
                                                                   0, 0);
  };
  // one tile: matrix reads from cur_planes, staging (of tile t+1) into nxt
  auto tile = [&](int64_t t, const uint32_t (*cur_planes)[kPfBlocks * kPfRowWords],
                  uint32_t (*nxt)[kPfBlocks * kPfRowWords]) {
    const int64_t b0 = t * kPfBlocks;
    group_mfma(cur_planes, 0, j32, h, aq, accA);
    uint32_t baseB = 0u;
    // emit mode: the lane's blocks of the previous tile's groups, or none
    // (-1) on the run's first tile (nb_max <= 2^30: the entry point)
    const int bpA = t > t_begin ? (int)b0 - kPfBlocks + j32 : -1;
    const int bpB = t > t_begin ? (int)b0 - 32 + j32 : -1;
    if constexpr (EMIT) {
      group_emit(accB, bpB, nbq, thk, recB);  // previous tile, group 1
      baseB = reserve(recB);
      scatter_emit(recA, baseA, bpA, h, nbq, thk, prs);
    } else if constexpr (SAMPLE) {
      group_sample(accB, b0 - 32 + j32, t > t_begin, h, nbq, srs, fa.n_grp);
    } else {
      group_store<HIST>(accB, b0 - 32 + j32, t > t_begin, h, nbq, srs, wrs, ld, rw, smp_off);
    }
    group_mfma(cur_planes, 1, j32, h, aq, accB);
    if constexpr (EMIT) {
      group_emit(accA, (int)b0 + j32, nbq, thk, recA);
      baseA = reserve(recA);
      scatter_emit(recB, baseB, bpB, h, nbq, thk, prs);
    } else if constexpr (SAMPLE) {
      group_sample(accA, b0 + j32, true, h, nbq, srs, fa.n_grp);
    } else {
      group_store<HIST>(accA, b0 + j32, true, h, nbq, srs, wrs, ld, rw, smp_off);
    }
    stage_tile(pk, tid, nxt);  // tile t+1 (past the run: the last tile again, never read)
    load_tile<MODE>(pooled, nb_max, t + 2 < t_end ? t + 2 : t_end - 1, tid, pk);
    __syncthreads();
  };
  int64_t t = t_begin;
  for (; t + 1 < t_end; t += 2) {
    tile(t, planes0, planes1);
    tile(t + 1, planes1, planes0);
  }
  if (t < t_end) {
    tile(t, planes0, planes1);
    ++t;
  }
  // last tile, group 1
  if constexpr (EMIT) {
    const int bl = (int)(t * kPfBlocks) - kPfBlocks + j32;
    scatter_emit(recA, baseA, bl, h, nbq, thk, prs);
    group_emit(accB, bl + 32, nbq, thk, recB);
    const uint32_t base = reserve(recB);
    scatter_emit(recB, base, bl + 32, h, nbq, thk, prs);
  } else if constexpr (SAMPLE) {
    group_sample(accB, t * kPfBlocks - 32 + j32, true, h, nbq, srs, fa.n_grp);
  } else {
    group_store<HIST>(accB, t * kPfBlocks - 32 + j32, true, h, nbq, srs, wrs, ld, rw, smp_off);
  }
}

// Grid of the persistent form: row tiles x runs of block tiles, about
// kPfSlots workgroups in all.
struct PfGrid {
  int n_rt;
  int64_t n_tiles;
  int n_chunks;
  unsigned wgs() const { return (unsigned)(n_rt * n_chunks); }
};
PfGrid pf_grid(int M, int64_t n_cols) {
  PfGrid g;
  g.n_rt = (M + kPfRows - 1) / kPfRows;
  g.n_tiles = (n_cols + kPfBlocks - 1) / kPfBlocks;
  int64_t want = (kPfSlots + g.n_rt - 1) / g.n_rt;
  if (want >= kXcds) want -= want % kXcds;  // a multiple of the XCD count where possible
  g.n_chunks = (int)(want < g.n_tiles ? want : g.n_tiles);
  if (g.n_chunks < 1) g.n_chunks = 1;
  return g;
}

}  // namespace

bool prefill_views_fit(int64_t nb_max, int64_t ld) {
  return (int64_t)kPfRowsPerWave * ld * 4 < kPfMaxView &&
         (int64_t)kPfRowsPerWave * sel::row_words(nb_max) * 4 < kPfMaxView;
}

hipError_t launch_score_prefill(const void* idx_q, int M, const int64_t* row_pos, const float* pooled,
                                int64_t nb_max, float* scores, int64_t ld, uint32_t* sel_ws,
                                hipStream_t stream) {
  if (M == 0 || nb_max == 0) return hipSuccess;
  if (!prefill_views_fit(nb_max, ld)) return hipErrorInvalidValue;
  const PfGrid g = pf_grid(M, nb_max);
  const FlatArgs none{};
  if (sel_ws)
    hipLaunchKernelGGL(score_prefill_pipe_kernel<kPfScoresSample>, dim3(g.wgs()), dim3(kWave * kPfWaves), 0, stream,
                       static_cast<const uint16_t*>(idx_q), M, row_pos, pooled, nb_max, scores, ld, sel_ws, none,
                       g.n_rt, g.n_tiles, g.n_chunks);
  else
    hipLaunchKernelGGL(score_prefill_pipe_kernel<kPfScores>, dim3(g.wgs()), dim3(kWave * kPfWaves), 0, stream,
                       static_cast<const uint16_t*>(idx_q), M, row_pos, pooled, nb_max, scores, ld, nullptr, none,
                       g.n_rt, g.n_tiles, g.n_chunks);
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
  fa.pairs = ws + L.pairs;
  fa.n_grp = sel::sample_groups(nb_max);
  fa.k = k_blocks;
  if (emit) {
    const PfGrid g = pf_grid(M, nb_max);
    hipLaunchKernelGGL(score_prefill_pipe_kernel<kPfEmit>, dim3(g.wgs()), dim3(kWave * kPfWaves), 0, stream,
                       static_cast<const uint16_t*>(idx_q), M, row_pos, pooled, nb_max, nullptr, 0, nullptr, fa,
                       g.n_rt, g.n_tiles, g.n_chunks);
  } else {
    const PfGrid g = pf_grid(M, fa.n_grp);
    hipLaunchKernelGGL(score_prefill_pipe_kernel<kPfSampleOnly>, dim3(g.wgs()), dim3(kWave * kPfWaves), 0, stream,
                       static_cast<const uint16_t*>(idx_q), M, row_pos, pooled, nb_max, nullptr, 0, nullptr, fa,
                       g.n_rt, g.n_tiles, g.n_chunks);
  }
  return hipGetLastError();
}

}  // namespace qsa
