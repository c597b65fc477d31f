// Block scoring (hipfire "QSA sparse attention ...", section 02: four
// index-query heads score every pooled block as the sum of their ReLU'd dot
// products times 1/sqrt(128); section 03: a few-row variant for decode and
// verify and a 16-row variant for prefill).
//
// Few-row variant (this file).  The pass streams the float32 pooled keys
// (512 B per block) once for a group of up to 8 rows of one sequence, so HBM
// bandwidth bounds it.  The contraction itself -- (rows x 4 heads) x 128
// dims against 16 blocks at a time -- runs on the float32 matrix cores
// (v_mfma_f32_16x16x4_f32): A = 16 blocks x 4 dims of pooled keys, B = 4
// dims x 16 (row, head) columns of index queries, float32 accumulation.  On
// the vector ALU the same work at 4 rows would need ~3.4 us of pure FMA
// issue for 4.2 us of HBM time at peak; on the matrix cores it needs half
// that and leaves the VALU free, so the pass stays memory bound.
//
// Data flow per wave: groups of 16 consecutive blocks.  Lane l reads 16
// bytes of block (l % 16) at dimension 16c + 4(l / 16), for c = 0..7: each
// load instruction covers 64 contiguous bytes of 16 blocks, and every pooled
// byte is read once.  The dimension order inside the MFMA k-axis is a
// permutation (dims 16c + 4(l/16) + t for the t-th of 4 MFMAs of chunk c);
// the index-query operand is loaded with the same permutation, so the sum
// is unchanged.  All of a wave's loads are issued before the first MFMA.
// Output D[i][j] (i = block, j = row*4 + head) is ReLU'd and summed over the
// 4 heads with two DPP quad permutations inside each group of 4 lanes.
//
// With HIST, the epilogue also feeds the top-k selection: the score of one
// block per 16-block group (at a hashed offset) is stored in the row's sample
// slots in the selection workspace (plain stores, no atomics).
//
// With APPEND the launch also does the index-key append of the new tokens
// (one sequence) in two extra columns of workgroups: one writes their keys to
// the cache and pools every block they complete, as the append kernel does;
// the other scores those blocks for its row group, pooling each in registers
// from the same four keys (new ones from the call, earlier ones from the
// cache, which this launch does not write there) and running the scoring
// waves' exact MFMA sequence on it, so every score is bit-identical to an
// append followed by a plain scoring launch.  The scoring waves skip those
// blocks' stores; they learn which blocks they are from one position per
// lane, loaded with the index queries ahead of the pooled stream.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "append_common.h"
#include "select_common.h"

namespace qsa {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroupBlocks = 16;   // blocks per MFMA row group
constexpr int kChunks = kIndexDim / 16;  // 8 chunks of 16 dims
constexpr int kGroupsPerWave = 2;
// Waves per workgroup (the kernels' WPG): 4 for long rows of one
// sequence, 1 for rows of at most 16,384 blocks or rows of different
// sequences, so that short rows spread over more compute units (measured:
// decode at 32K context 4.3 us with 2 waves, 4.15 with 1, 6.0 with 4;
// batched decode 28.0 against 27.4 us with 1; the 262K verify's launch is
// 0.15 us faster with 2 but its step no faster).
constexpr int kWavesLong = 4;
constexpr int kWavesShort = 1;
constexpr int64_t kShortRowBlocks = 16384;
constexpr int kBlocksPerWave = kGroupBlocks * kGroupsPerWave;
constexpr float kScoreScale = 0.08838834764831845f;  // 1/sqrt(128)
constexpr int kBufferWord3 = 0x00020000;            // raw buffer view (gfx9 family)
constexpr int kBufferDrop = (int)0x80000000u;       // an offset past any view: the store is dropped
constexpr int64_t kMaxView = (int64_t)1 << 31;      // bytes of a buffer view

// Index-query elements as loaded (4 per lane per chunk) and as MFMA operands.
template <class EQ> struct QRaw;
template <> struct QRaw<F32> { using T = uint4; };
template <> struct QRaw<BF16> { using T = uint2; };
template <class EQ>
__device__ __forceinline__ typename QRaw<EQ>::T load_q_raw(const typename EQ::T* __restrict__ q) {
  return *reinterpret_cast<const typename QRaw<EQ>::T*>(q);
}
template <class EQ>
__device__ __forceinline__ float4 q_to_f4(typename QRaw<EQ>::T x);
template <>
__device__ __forceinline__ float4 q_to_f4<F32>(uint4 x) {
  return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
}
template <>
__device__ __forceinline__ float4 q_to_f4<BF16>(uint2 x) {
  return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                     __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
}

// A wave-uniform pointer, held in scalar registers.
__device__ __forceinline__ float* scalar_ptr(float* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return reinterpret_cast<float*>(((uint64_t)hi << 32) | lo);
}

// Raw query words ANDed with an all-ones or all-zeros mask: a dead row's
// operand becomes +0 in either format without a branch.
__device__ __forceinline__ uint4 mask_raw(uint4 x, uint32_t m) { return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m); }
__device__ __forceinline__ uint2 mask_raw(uint2 x, uint32_t m) { return make_uint2(x.x & m, x.y & m); }

// The append folded into the launch (one sequence).
struct AppendArgs {
  const void* new_idx;  // [n_new][128] in the query dtype
  const int64_t* pos;   // [n_new]
  void* cache;          // [capacity][128]
  float* pooled;        // the pooled keys the scoring reads (written for completed blocks)
  int n_new;
  int64_t capacity;
};

// A new token at position p completes a block whose score this launch
// writes from the keys rather than from the pooled stream.
__device__ __forceinline__ bool completes_scored_block(int64_t p, int64_t capacity, int64_t nb_max) {
  return p >= 0 && p < capacity && (p & 3) == 3 && (p >> 2) < nb_max;
}

// Index-query operand of a row group, as loaded: column i16 = (row 4 st +
// i16 / 4, head i16 % 4) of set st, dims 16c + 4 kq .. + 3.
template <class EQ, int NSET>
__device__ __forceinline__ void load_q_operand(const typename EQ::T* __restrict__ idx_q, int m0, int rows, int i16,
                                               int kq, typename QRaw<EQ>::T (&qraw)[NSET][kChunks]) {
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const int r = st * 4 + (i16 >> 2);
    const int h = i16 & 3;
    const typename EQ::T* qsrc = idx_q + ((int64_t)(m0 + (r < rows ? r : 0)) * kIndexHeads + h) * kIndexDim + 4 * kq;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) qraw[st][c] = load_q_raw<EQ>(qsrc + 16 * c);
  }
}

template <class EQ, int NSET>
__device__ __forceinline__ void q_operand(const typename QRaw<EQ>::T (&qraw)[NSET][kChunks], int rows, int i16,
                                          float4 (&bq)[NSET][kChunks]) {
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const uint32_t live = st * 4 + (i16 >> 2) < rows ? ~0u : 0u;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) bq[st][c] = q_to_f4<EQ>(mask_raw(qraw[st][c], live));
  }
}

// The scoring waves' index-query operand, read as one contiguous span and
// redistributed through a wave-private LDS copy.  A row group's queries are
// contiguous in memory ([4 NSET rows][4 heads][128]), so a wave reads the
// span 16 bytes per lane and instruction (4 instructions for 4 bf16 rows);
// read directly in the operand layout, each of 8 instructions per lane would
// touch 16 partial cache lines, and those requests, repeated by every wave
// of the launch, delay the pooled stream queued behind them.  Rows of the
// span past M re-read the group's first row (their columns are zeroed).
template <class EQ, int NSET>
struct QSpan {
  static constexpr int kRowBytes = kIndexHeads * kIndexDim * (int)sizeof(typename EQ::T);
  static constexpr int kU4 = NSET * 4 * kRowBytes / (kWave * 16);  // 16-byte loads per lane
  static constexpr int kWords = NSET * 4 * kRowBytes / 4;          // LDS words per wave
};
template <class EQ, int NSET>
__device__ __forceinline__ void load_q_span(const typename EQ::T* __restrict__ idx_q, int M, int m0, int lane,
                                            uint4 (&qv)[QSpan<EQ, NSET>::kU4]) {
  using S = QSpan<EQ, NSET>;
  const unsigned char* base = reinterpret_cast<const unsigned char*>(idx_q) + (int64_t)m0 * S::kRowBytes;
#pragma unroll
  for (int u = 0; u < S::kU4; ++u) {
    const int o = (u * kWave + lane) * 16;
    const int r = o / S::kRowBytes;
    qv[u] = *reinterpret_cast<const uint4*>(base + (m0 + r < M ? o : o % S::kRowBytes));
  }
}
template <class EQ, int NSET>
__device__ __forceinline__ void stage_q_span(const uint4 (&qv)[QSpan<EQ, NSET>::kU4], uint32_t* __restrict__ qst,
                                             int lane) {
#pragma unroll
  for (int u = 0; u < QSpan<EQ, NSET>::kU4; ++u) *reinterpret_cast<uint4*>(qst + (u * kWave + lane) * 4) = qv[u];
}
template <class EQ, int NSET>
__device__ __forceinline__ void q_operand_lds(const uint32_t* __restrict__ qst, int rows, int i16, int kq,
                                              float4 (&bq)[NSET][kChunks]) {
  __builtin_amdgcn_wave_barrier();
  // every piece read before any is used: one LDS round trip
  typename QRaw<EQ>::T raw[NSET][kChunks];
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const int r = st * 4 + (i16 >> 2);
    const int e0 = (r * kIndexHeads + (i16 & 3)) * kIndexDim + 4 * kq;  // element index of dims 4 kq .. + 3
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      raw[st][c] = *reinterpret_cast<const typename QRaw<EQ>::T*>(qst + (e0 + 16 * c) * (int)sizeof(typename EQ::T) / 4);
  }
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const uint32_t live = st * 4 + (i16 >> 2) < rows ? ~0u : 0u;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) bq[st][c] = q_to_f4<EQ>(mask_raw(raw[st][c], live));
  }
}

// Scores of one 16-block group against every column set: sv[st][v] is the
// score of block 4 kq + v of the group for row 4 st + i16 / 4 (the 4 heads'
// ReLU'd dot products summed by two DPP quad permutations, then scaled).
template <int NSET>
__device__ __forceinline__ void group_scores(const float4 (&a)[kChunks], const float4 (&bq)[NSET][kChunks],
                                             float (&sv)[NSET][4]) {
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c].x, bq[st][c].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c].y, bq[st][c].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c].z, bq[st][c].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c].w, bq[st][c].w, acc, 0, 0, 0);
    }
    // acc[v] = D[4*kq + v][i16]: block 4kq + v of the group, column i16
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float x = quad_xor_add<2>(quad_xor_add<1>(fmaxf(acc[v], 0.f)));
      sv[st][v] = x * kScoreScale;
    }
  }
}

// The folded append's second extra workgroup of each row group: scores of
// the blocks the new tokens complete, one block per wave at a time.  The
// block's pooled key is built in every A row and goes through the scoring
// waves' MFMA sequence (an output element depends only on its own A row and
// B column), so the score equals theirs on the stored pooled key.
template <class EQ, int NSET, int RPG, bool HIST, int WPG>
__device__ void score_fresh_blocks(const typename EQ::T* __restrict__ idx_q, int M,
                                   const int64_t* __restrict__ row_pos, int64_t nb_max, float* __restrict__ scores,
                                   int64_t ld, uint32_t* __restrict__ ws, int64_t rw, int64_t smp_off,
                                   const AppendArgs& ap) {
  using T = typename EQ::T;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int i16 = lane & 15;
  const int kq = lane >> 4;
  const int m0 = blockIdx.y * RPG;
  const int rows = min(RPG, M - m0);
  // positions of tokens i-3..i in one vector load: lane j % 4 loads token
  // i-3+j (index clamped into the call); issued first, so the wave's first
  // block needs one round trip for positions and one for its keys
  auto load_pos4 = [&](int i) -> int64_t {
    int il = i - (kBlockTokens - 1) + (lane & 3);
    il = il < 0 ? 0 : (il < ap.n_new ? il : ap.n_new - 1);
    return ap.pos[il];
  };
  int i = __builtin_amdgcn_readfirstlane(wave);
  int64_t pl = load_pos4(i);
  typename QRaw<EQ>::T qraw[NSET][kChunks];
  load_q_operand<EQ, NSET>(idx_q, m0, rows, i16, kq, qraw);
  int64_t nb_row[NSET];
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const int r = st * 4 + (i16 >> 2);
    nb_row[st] = r < rows ? clamp_nb(row_pos[m0 + r], nb_max) : 0;
  }
  float4 bq[NSET][kChunks];
  q_operand<EQ, NSET>(qraw, rows, i16, bq);
  const T* nw = static_cast<const T*>(ap.new_idx);
  const T* ca = static_cast<const T*>(ap.cache);
  for (; i < ap.n_new; i += WPG) {
    const int64_t cur = pl;
    pl = load_pos4(i + WPG);  // the wave's next token, in flight meanwhile
    int64_t pw[kBlockTokens];  // wave-uniform copies
#pragma unroll
    for (int j = 0; j < kBlockTokens; ++j) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)cur, j);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)cur >> 32), j);
      pw[j] = (int64_t)(((uint64_t)hi << 32) | lo);
    }
    const int64_t p = pw[kBlockTokens - 1];
    // key rows: from this call when the token is in it, else from the cache
    // (the append kernel's rule)
    const T* krow[kBlockTokens];
#pragma unroll
    for (int j = 0; j < kBlockTokens; ++j) {
      const int back = kBlockTokens - 1 - j;
      const int ij = i - back;
      const bool here = back == 0 || (ij >= 0 && pw[j] == p - back);
      krow[j] = here ? nw + (int64_t)ij * kIndexDim : ca + (p - back) * kIndexDim;
    }
    if (!completes_scored_block(p, ap.capacity, nb_max)) continue;
    const int64_t b = p >> 2;
    // the block's pooled key in every A row (all loads in flight together)
    typename QRaw<EQ>::T kraw[kChunks][kBlockTokens];
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
#pragma unroll
      for (int j = 0; j < kBlockTokens; ++j) kraw[c][j] = load_q_raw<EQ>(krow[j] + 16 * c + 4 * kq);
    __builtin_amdgcn_sched_barrier(0);  // keep every key load ahead of the first use
    float4 a[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      float4 x[kBlockTokens];
#pragma unroll
      for (int j = 0; j < kBlockTokens; ++j) x[j] = q_to_f4<EQ>(kraw[c][j]);
      a[c] = make_float4(pool4(x[0].x, x[1].x, x[2].x, x[3].x), pool4(x[0].y, x[1].y, x[2].y, x[3].y),
                         pool4(x[0].z, x[1].z, x[2].z, x[3].z), pool4(x[0].w, x[1].w, x[2].w, x[3].w));
    }
    float sv[NSET][4];
    group_scores<NSET>(a, bq, sv);
    const int64_t bb = (b & ~(int64_t)15) + 4 * kq;
#pragma unroll
    for (int st = 0; st < NSET; ++st) {
      const int r = st * 4 + (i16 >> 2);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if ((i16 & 3) == 0 && r < rows && bb + v == b && b < nb_row[st]) {
          scores[(int64_t)(m0 + r) * ld + b] = sv[st][v];
          if (HIST && sel::sampled((uint32_t)b))
            reinterpret_cast<float*>(ws)[(size_t)(m0 + r) * rw + smp_off + (b >> 4)] = sv[st][v];
        }
      }
    }
  }
}

template <class EQ, int NSET, int RPG, bool HIST, bool APPEND, int WPG>
__global__ void __launch_bounds__(kWave * WPG)
score_fewrow_kernel(const typename EQ::T* __restrict__ idx_q, int M,
                    const int64_t* __restrict__ row_pos, const int32_t* __restrict__ row_seq,
                    const float* __restrict__ pooled, int n_seq, int64_t capacity,
                    int64_t nb_max, float* __restrict__ scores, int64_t ld, uint32_t* __restrict__ ws,
                    int64_t rw, int64_t smp_off, AppendArgs ap) {
  static_assert(RPG <= 4 * NSET, "rows per group exceed the column sets");
  int bx = blockIdx.x;
  if constexpr (APPEND) {
    // the grid's two extra first columns (dispatched first, so that their
    // dependent loads start before the pooled stream fills the memory
    // queues): the append (row group 0's workgroup writes the cache rows and
    // the completed blocks' pooled keys) and the completed blocks' scores
    // (every row group's)
    if (bx < 2) {
      if (bx == 1) {
        score_fresh_blocks<EQ, NSET, RPG, HIST, WPG>(idx_q, M, row_pos, nb_max, scores, ld, ws, rw, smp_off, ap);
      } else if (blockIdx.y == 0) {
        for (int e = threadIdx.x; e < ap.n_new * kIndexDim; e += kWave * WPG)
          append_token_dim<EQ>(static_cast<const typename EQ::T*>(ap.new_idx), ap.pos, nullptr,
                               static_cast<typename EQ::T*>(ap.cache), ap.pooled, 1, ap.capacity, e / kIndexDim,
                               e % kIndexDim);
      }
      return;
    }
    bx -= 2;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m0 = blockIdx.y * RPG;
  const int rows = min(RPG, M - m0);
  // the selection that consumes the sample counts its chunks in from zero
  if (HIST && bx == 0 && (int)threadIdx.x < rows)
    ws[(size_t)(m0 + threadIdx.x) * rw + sel::kArriveWord] = 0u;

  // Everything is loaded up front.  The row positions (wave-uniform) and the
  // index-query operand are small and cached; issued before the pooled
  // stream, their waits leave the pooled loads in flight.  The pooled loads
  // depend only on nb_max (the host bound), not on the row positions.
  // (a wave past nb_max issues its clamped loads and leaves below: no
  // early branch holds the argument loads back)
  const int64_t wave_b0 = (int64_t)bx * (WPG * kBlocksPerWave) + wave * kBlocksPerWave;
  const int i16 = lane & 15;   // A row (block in group) / B column
  const int kq = lane >> 4;    // k slot 0..3
  int64_t pos_r[RPG];
#pragma unroll
  for (int r = 0; r < RPG; ++r) pos_r[r] = row_pos[m0 + (r < rows ? r : 0)];
  __shared__ __align__(16) uint32_t qstage[WPG][QSpan<EQ, NSET>::kWords];
  uint4 qv[QSpan<EQ, NSET>::kU4];
  load_q_span<EQ, NSET>(idx_q, M, m0, lane, qv);
  stage_q_span<EQ, NSET>(qv, qstage[wave], lane);
  // folded append: one new token's position per lane (lanes past the count
  // repeat the last; 1 <= n_new <= 64)
  int64_t new_p = -1;
  if constexpr (APPEND) new_p = ap.pos[lane < ap.n_new ? lane : ap.n_new - 1];
  // rows of several sequences come one per row group; a group of several
  // rows is one sequence's, so only the one-row kernel looks its sequence up
  const int s = (RPG == 1 && row_seq) ? row_seq[m0] : 0;
  const bool seq_ok = s >= 0 && s < n_seq;
  const float* __restrict__ P = pooled + (int64_t)(seq_ok ? s : 0) * (capacity / kBlockTokens) * kIndexDim;

  // Pooled loads: all groups, all chunks, unconditional (blocks past nb_max
  // re-read the last block; their scores are never stored).
  float4 a[kGroupsPerWave][kChunks];
#pragma unroll
  for (int g = 0; g < kGroupsPerWave; ++g) {
    const int64_t b = wave_b0 + g * kGroupBlocks + i16;
    const float* src = P + (b < nb_max ? b : nb_max - 1) * kIndexDim + 4 * kq;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) a[g][c] = *reinterpret_cast<const float4*>(src + 16 * c);
  }

  int64_t nb_r[RPG];
  int64_t nb_hi = 0;
#pragma unroll
  for (int r = 0; r < RPG; ++r) {
    nb_r[r] = r < rows ? clamp_nb(pos_r[r], nb_max) : 0;
    nb_hi = nb_r[r] > nb_hi ? nb_r[r] : nb_hi;
  }
  const bool active = wave_b0 < nb_hi && seq_ok;
  if (!active) return;

  float4 bq[NSET][kChunks];
  q_operand_lds<EQ, NSET>(qstage[wave], rows, i16, kq, bq);
  int64_t nb_row[NSET];
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const int r = st * 4 + (i16 >> 2);
    int64_t n = 0;
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr) n = (r == rr) ? nb_r[rr] : n;  // no dynamic register indexing
    nb_row[st] = n;
  }

  // blocks of this wave whose scores the fresh-block workgroup writes
  uint32_t fresh = 0u;
  static_assert(kBlocksPerWave <= 32, "one mask bit per block of the wave");
  if constexpr (APPEND) {
    const int64_t rel = (new_p >> 2) - wave_b0;
    fresh = completes_scored_block(new_p, ap.capacity, nb_max) && rel >= 0 && rel < kBlocksPerWave
                ? 1u << rel : 0u;
    fresh = wave_or(fresh);
  }

  // Stores through buffer views of each column set's 4 rows (scores and,
  // with HIST, the rows' workspace records), a masked lane's offset past the
  // view: no branch, so the epilogue is one straight-line block.  Lane
  // (kq, i16) stores block 4 kq + i16 % 4 of the group for row i16 / 4 of the
  // set (the head sum left every head lane of a row with all four scores).
  // Views over 2^31 bytes (rows of more than 2^27 blocks) take the branching
  // form below.
  // (readfirstlane: the compiler then keeps the test and the views scalar)
  const bool views = __builtin_amdgcn_readfirstlane(4 * ld * 4 < kMaxView && (!HIST || 4 * rw * 4 < kMaxView)) != 0;
  __amdgpu_buffer_rsrc_t srs[NSET], wrs[NSET];
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const int rs = rows - 4 * st < 0 ? 0 : (rows - 4 * st < 4 ? rows - 4 * st : 4);  // live rows of the set
    srs[st] = __builtin_amdgcn_make_buffer_rsrc(scalar_ptr(scores + (int64_t)(m0 + 4 * st) * ld), 0,
                                                __builtin_amdgcn_readfirstlane(views ? (int)(rs * ld * 4) : 0),
                                                kBufferWord3);
    wrs[st] = __builtin_amdgcn_make_buffer_rsrc(
        scalar_ptr(HIST ? reinterpret_cast<float*>(ws) + (int64_t)(m0 + 4 * st) * rw : nullptr), 0,
        __builtin_amdgcn_readfirstlane(HIST && views ? (int)(rs * rw * 4) : 0), kBufferWord3);
  }
  const int hd = i16 & 3;

  // group by group, so that the first group's matrix work and stores
  // proceed while the second group's pooled loads are still arriving
#pragma unroll
  for (int g = 0; g < kGroupsPerWave; ++g) {
    float sv[NSET][4];
    group_scores<NSET>(a[g], bq, sv);
    const int64_t bb = wave_b0 + g * kGroupBlocks + 4 * kq;
    if (views) {
      const int64_t b = bb + hd;
      const bool fr = (fresh >> (g * kGroupBlocks + 4 * kq + hd)) & 1u;
      const bool smp = sel::sampled((uint32_t)b);
#pragma unroll
      for (int st = 0; st < NSET; ++st) {
        const int rr = i16 >> 2;  // row of the set
        // score hd of the four, picked with bit masks (a select chain here
        // compiles to branches)
        const uint32_t m1 = 0u - (uint32_t)(hd & 1), m2 = 0u - (uint32_t)(hd >> 1);
        const uint32_t x01 = (__float_as_uint(sv[st][0]) & ~m1) | (__float_as_uint(sv[st][1]) & m1);
        const uint32_t x23 = (__float_as_uint(sv[st][2]) & ~m1) | (__float_as_uint(sv[st][3]) & m1);
        const uint32_t x = (x01 & ~m2) | (x23 & m2);
        const bool keep = st * 4 + rr < rows && b < nb_row[st] && !fr;
        __builtin_amdgcn_raw_buffer_store_b32(x, srs[st], keep ? (int)((rr * ld + b) * 4) : kBufferDrop, 0, 0);
        if constexpr (HIST)
          __builtin_amdgcn_raw_buffer_store_b32(x, wrs[st],
                                                keep && smp ? (int)((rr * rw + smp_off + (b >> 4)) * 4) : kBufferDrop,
                                                0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      continue;
    }
#pragma unroll
    for (int st = 0; st < NSET; ++st) {
      const int r = st * 4 + (i16 >> 2);
      if ((i16 & 3) != 0 || r >= rows) continue;
      float* dst = scores + (int64_t)(m0 + r) * ld;
      // the lane's 4 consecutive blocks in one 16-byte store when all four
      // are stored here (every span but a row's last and a fresh block's)
      const uint32_t fr = (fresh >> (g * kGroupBlocks + 4 * kq)) & 0xfu;
      if (bb + 3 < nb_row[st] && fr == 0u) {
        *reinterpret_cast<float4*>(dst + bb) = make_float4(sv[st][0], sv[st][1], sv[st][2], sv[st][3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (bb + v < nb_row[st] && !((fr >> v) & 1u)) dst[bb + v] = sv[st][v];
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool keep = bb + v < nb_row[st] && !((fr >> v) & 1u);
        // one sampled block per 16-block group: its score goes to the group's slot
        if (HIST && keep && sel::sampled((uint32_t)(bb + v)))
          reinterpret_cast<float*>(ws)[(size_t)(m0 + r) * rw + smp_off + ((bb + v) >> 4)] = sv[st][v];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <class EQ, int NSET, int RPG, bool HIST, int WPG>
hipError_t launch_fewrow_wpg(const void* idx_q, int M, const int64_t* row_pos, const int32_t* row_seq,
                             const float* pooled, int n_seq, int64_t capacity, int64_t nb_max,
                             float* scores, int64_t ld, uint32_t* ws, const AppendArgs* ap, hipStream_t stream) {
  constexpr int kBlocksPerWG = WPG * kBlocksPerWave;
  const int64_t wgs = (nb_max + kBlocksPerWG - 1) / kBlocksPerWG;
  if (wgs == 0) return hipSuccess;
  dim3 grid((unsigned)wgs, (unsigned)((M + RPG - 1) / RPG));
  if (ap)
    hipLaunchKernelGGL((score_fewrow_kernel<EQ, NSET, RPG, HIST, true, WPG>), dim3(grid.x + 2, grid.y),
                       dim3(kWave * WPG), 0, stream, static_cast<const typename EQ::T*>(idx_q), M, row_pos, row_seq, pooled, n_seq,
                       capacity, nb_max, scores, ld, ws, sel::row_words(nb_max), sel::sample_off(nb_max), *ap);
  else
    hipLaunchKernelGGL((score_fewrow_kernel<EQ, NSET, RPG, HIST, false, WPG>), grid, dim3(kWave * WPG), 0,
                       stream, static_cast<const typename EQ::T*>(idx_q), M, row_pos, row_seq, pooled, n_seq,
                       capacity, nb_max, scores, ld, ws, sel::row_words(nb_max), sel::sample_off(nb_max),
                       AppendArgs{});
  return hipGetLastError();
}

template <class EQ, int NSET, int RPG, bool HIST>
hipError_t launch_fewrow(const void* idx_q, int M, const int64_t* row_pos, const int32_t* row_seq,
                         const float* pooled, int n_seq, int64_t capacity, int64_t nb_max,
                         float* scores, int64_t ld, uint32_t* ws, const AppendArgs* ap, hipStream_t stream) {
  if (RPG == 1 || nb_max <= kShortRowBlocks)
    return launch_fewrow_wpg<EQ, NSET, RPG, HIST, kWavesShort>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity,
                                                               nb_max, scores, ld, ws, ap, stream);
  return launch_fewrow_wpg<EQ, NSET, RPG, HIST, kWavesLong>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity,
                                                            nb_max, scores, ld, ws, ap, stream);
}

template <class EQ, bool HIST>
hipError_t dispatch_rows(const void* idx_q, int M, const int64_t* row_pos, const int32_t* row_seq,
                         const float* pooled, int n_seq, int64_t capacity, int64_t nb_max,
                         float* scores, int64_t ld, uint32_t* ws, const AppendArgs* ap, hipStream_t stream) {
  // Rows of different sequences read different pooled keys: one row per
  // group.  Rows of one sequence share each pooled read, 4 or 8 at a time;
  // many bf16 rows go to the matrix-core many-row kernel.
  if (row_seq) return launch_fewrow<EQ, 1, 1, HIST>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, ws, ap, stream);
  if (EQ::kBytes == 2 && M >= kPrefillMinRows)  // (the append is never folded into this path)
    return launch_score_prefill(idx_q, M, row_pos, pooled, nb_max, scores, ld, ws, stream);
  if (M <= 4) return launch_fewrow<EQ, 1, 4, HIST>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, ws, ap, stream);
  return launch_fewrow<EQ, 2, 8, HIST>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, ws, ap, stream);
}

}  // namespace

hipError_t launch_score_blocks(const void* idx_q, int dtype, int M, const int64_t* row_pos,
                               const int32_t* row_seq, const float* pooled, int n_seq,
                               int64_t capacity, int64_t nb_max, float* scores, int64_t ld,
                               uint32_t* sel_ws, hipStream_t stream) {
  if (M == 0 || nb_max == 0) return hipSuccess;
  if (sel_ws) {
    if (dtype == QSA_BF16)
      return dispatch_rows<BF16, true>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, sel_ws, nullptr, stream);
    return dispatch_rows<F32, true>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, sel_ws, nullptr, stream);
  }
  if (dtype == QSA_BF16)
    return dispatch_rows<BF16, false>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, nullptr, nullptr, stream);
  return dispatch_rows<F32, false>(idx_q, M, row_pos, row_seq, pooled, n_seq, capacity, nb_max, scores, ld, nullptr, nullptr, stream);
}

bool append_folds_into_scoring(int dtype, int M, int n_new, int64_t nb_max) {
  return M > 0 && nb_max > 0 && n_new > 0 && n_new <= kMaxFoldedTokens && !(dtype == QSA_BF16 && M >= kPrefillMinRows);
}

hipError_t launch_append_score(const void* new_idx, int n_new, const int64_t* new_pos, void* idx_cache,
                               float* pooled, int64_t capacity, const void* idx_q, int dtype, int M,
                               const int64_t* row_pos, int64_t nb_max, float* scores, int64_t ld,
                               uint32_t* sel_ws, hipStream_t stream) {
  if (!append_folds_into_scoring(dtype, M, n_new, nb_max)) {  // two launches
    hipError_t e = launch_append_pool(new_idx, dtype, n_new, new_pos, nullptr, idx_cache, pooled, 1, capacity, stream);
    if (e != hipSuccess) return e;
    return launch_score_blocks(idx_q, dtype, M, row_pos, nullptr, pooled, 1, capacity, nb_max, scores, ld, sel_ws,
                               stream);
  }
  const AppendArgs ap{new_idx, new_pos, idx_cache, pooled, n_new, capacity};
  if (dtype == QSA_BF16) {
    if (sel_ws)
      return dispatch_rows<BF16, true>(idx_q, M, row_pos, nullptr, pooled, 1, capacity, nb_max, scores, ld, sel_ws, &ap, stream);
    return dispatch_rows<BF16, false>(idx_q, M, row_pos, nullptr, pooled, 1, capacity, nb_max, scores, ld, nullptr, &ap, stream);
  }
  if (sel_ws)
    return dispatch_rows<F32, true>(idx_q, M, row_pos, nullptr, pooled, 1, capacity, nb_max, scores, ld, sel_ws, &ap, stream);
  return dispatch_rows<F32, false>(idx_q, M, row_pos, nullptr, pooled, 1, capacity, nb_max, scores, ld, nullptr, &ap, stream);
}

}  // namespace qsa
