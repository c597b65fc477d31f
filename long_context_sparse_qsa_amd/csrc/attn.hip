// Gathered grouped-query attention over the kept rows (hipfire "QSA sparse
// attention ...", section 02: attention reads only the selected rows plus the
// incomplete tail; section 03: one workgroup per KV group of 12 query heads
// reads each selected K/V row once for the whole group) and the log-sum-exp
// merge of split partials (MTPLX PR #610, "What changes": float32 partials,
// merged by log-sum-exp, rounded once; rows with no visible key give zeros).
//
// Two kernels compute the attention, one grid of (row, KV head, split)
// workgroups each; split partials (output normalised by its own sum, and its
// lse) go to the workspace and attn_combine_kernel merges them (a single split
// writes the output directly).
//
// attn_mfma_kernel (bf16, fp8 E4M3 or Q8_0 K/V with bf16 queries): W waves
// per workgroup, each owning one 16-token slice of every tile of 16 W tokens,
// with its own online softmax (no workgroup barrier in the slice loop).  QK
// and P.V run on the matrix cores with the group's 12 query heads as one
// operand; K rows are loaded straight into the other operand's layout, V is
// staged through LDS as 4-token quads per dim, and the next slice's loads are
// in flight during the current slice's softmax and P.V.  The W wave partials
// are merged by log-sum-exp in LDS.  The plan (attn_plan) picks W, the tiles a
// split walks and the split count.
//
// attn_decode_kernel (float32 K/V): 4 waves over 64-token tiles on the vector
// ALU.  Each lane resolves 8 of the tile's tokens to K/V rows through the
// segment table and stages them in LDS once for all 12 query heads; QK with
// wave w on heads 3w..3w+2 (lane = token, the query row in scalar
// registers), an online softmax with base-2 exponentials, and P.V with lane =
// (dims, 6 heads), all in float32.
//
// Every independent load (row position, kept count, the kept block ids of
// the split, the segment table, the queries) is issued at once: memory round
// trips bound both kernels at decode sizes.
#include <mutex>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kGroup = 12;          // query heads per KV head
constexpr int kTileTok = 64;        // tokens per tile
constexpr int kThreads = 256;
constexpr int kHeadsPerWaveQK = kGroup / (kThreads / kWave);  // 3
constexpr int kHeadHalves = 2;      // PV: heads split in two halves of 6
constexpr int kHeadsPV = kGroup / kHeadHalves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 16-byte load through a global (not generic) pointer: generic loads may
// alias LDS, which would keep them ordered behind the staging writes.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16(const unsigned char* p) {
  typedef __attribute__((address_space(1))) const u32x4_t GU4;
  const u32x4_t v = *(GU4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 8-byte load through a global pointer (see ldg16).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ldg8(const unsigned char* p) {
  typedef __attribute__((address_space(1))) const u32x2_t GU2;
  const u32x2_t v = *(GU2*)(p);
  return make_uint2(v.x, v.y);
}

struct KvArgs {
  const int32_t* seq_seg_begin;
  const int64_t* seg_start;
  const int64_t* seg_len;
  const int64_t* seg_cap;
  const void* const* k_seg;
  const void* const* v_seg;
  const uint16_t* const* k_scale;  // fp8 / Q8_0 K/V: f16 scales per segment
  const uint16_t* const* v_scale;
  int n_seq;
  int n_seg_total;
};

struct SegDesc {
  int64_t lo, hi, cap;
  const unsigned char* k;
  const unsigned char* v;
  const uint16_t* ks;  // fp8 K/V only
  const uint16_t* vs;
};

// Element-type specific constants of the tile loop.
template <class E, int D>
struct Tile {
  static constexpr int kRowBytes = D * E::kBytes;
  static constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per row
  static constexpr int kKStride = kRowBytes + 16;       // padded K row in LDS
  static constexpr int kElemsPerChunk = 16 / E::kBytes;
  static constexpr int kDimsPerThread = D / (kThreads / kHeadHalves);  // PV dims per lane
  static constexpr int kItems = (kTileTok / 2) * kChunks;  // (token pair, chunk) staging items
  static constexpr int kItemsPerThread = kItems / kThreads;
};

// bf16 words (x of token t, y of token t+1) -> interleaved pairs per dim.
__device__ __forceinline__ void interleave(uint4 a, uint4 b, uint4& lo, uint4& hi) {
  // out word 2e   = (a.e low,  b.e low)  : dims 2e of the chunk
  // out word 2e+1 = (a.e high, b.e high) : dims 2e+1
  lo.x = __builtin_amdgcn_perm(b.x, a.x, 0x05040100u);
  lo.y = __builtin_amdgcn_perm(b.x, a.x, 0x07060302u);
  lo.z = __builtin_amdgcn_perm(b.y, a.y, 0x05040100u);
  lo.w = __builtin_amdgcn_perm(b.y, a.y, 0x07060302u);
  hi.x = __builtin_amdgcn_perm(b.z, a.z, 0x05040100u);
  hi.y = __builtin_amdgcn_perm(b.z, a.z, 0x07060302u);
  hi.z = __builtin_amdgcn_perm(b.w, a.w, 0x05040100u);
  hi.w = __builtin_amdgcn_perm(b.w, a.w, 0x07060302u);
}

template <class E, int D>
__global__ void __launch_bounds__(kThreads, 2)
attn_decode_kernel(const typename E::T* __restrict__ q, int M, int hq, float scale_log2,
                   const int64_t* __restrict__ row_pos, const int32_t* __restrict__ row_seq,
                   KvArgs kv, const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
                   int k_blocks, int tiles_per_split, int splits,
                   typename E::T* __restrict__ out, float* __restrict__ lse_out,
                   float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  using TT = Tile<E, D>;
  using T = typename E::T;
  constexpr bool kBf = (E::kBytes == 2);
  __shared__ __align__(16) unsigned char k_lds[kTileTok * TT::kKStride];
  __shared__ __align__(16) unsigned char v_lds[kTileTok * TT::kRowBytes];
  __shared__ __align__(16) uint32_t p_lds[kTileTok * kGroup];  // bf16: [32 pairs][12]; fp32: [64][12]
  __shared__ __align__(16) unsigned char q_lds[kGroup * TT::kRowBytes];  // the group's 12 query rows
  __shared__ float alpha_lds[kGroup];
  __shared__ float m_lds[kGroup], l_lds[kGroup];
  __shared__ SegDesc segs[kMaxSegments];
  __shared__ uint32_t valid_lds[kTileTok];
  __shared__ int nseg_sh;

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int m = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid / kWave);
  const int tok_begin = split * tiles_per_split * kTileTok;
  const int32_t* __restrict__ srow = sel + (int64_t)m * k_blocks;

  // ---- independent loads, issued together
  const int64_t p = row_pos[m];
  const int ns_raw = n_sel[m];
  const int sq_raw = row_seq ? row_seq[m] : 0;
  // kept block ids this lane's staging rows may need (speculative: every id
  // read lies inside the row's k_blocks entries)
  constexpr int kRows = TT::kItemsPerThread * 2;  // staging rows per lane per tile
  int32_t bid[kRows];
#pragma unroll
  for (int it = 0; it < TT::kItemsPerThread; ++it) {
    const int pair = (tid + it * kThreads) / TT::kChunks;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = tok_begin + 2 * pair + u;
      bid[it * 2 + u] = (j >> 2) < k_blocks ? srow[j >> 2] : -1;
    }
  }
  // the group's query rows, staged once (loads issued before the LDS writes)
  const unsigned char* qbytes = reinterpret_cast<const unsigned char*>(q + ((int64_t)m * hq + (int64_t)g * kGroup) * D);
  constexpr int kQChunks = kGroup * TT::kChunks;
  constexpr int kQPer = (kQChunks + kThreads - 1) / kThreads;
  uint4 qv[kQPer];
#pragma unroll
  for (int e = 0; e < kQPer; ++e) {
    const int i = tid + e * kThreads;
    qv[e] = ldg16(qbytes + (i < kQChunks ? i : 0) * 16);
  }
  // this sequence's segment descriptors (loads before any LDS write)
  int si_lo = 0, nseg_all = 0;
  if (kv.n_seq == 1) {
    // one sequence: its segments are entries 0 .. n_seg_total-1
    nseg_all = kv.n_seg_total < kMaxSegments ? kv.n_seg_total : kMaxSegments;
  } else {
    const bool seq_ok = sq_raw >= 0 && sq_raw < kv.n_seq;
    const int sq = seq_ok ? sq_raw : 0;
    int s_begin = kv.seq_seg_begin[sq], s_end = kv.seq_seg_begin[sq + 1];
    s_begin = s_begin < 0 ? 0 : s_begin;
    s_end = s_end > kv.n_seg_total ? kv.n_seg_total : s_end;
    si_lo = s_begin;
    nseg_all = (seq_ok && s_end > s_begin) ? min(s_end - s_begin, kMaxSegments) : 0;
  }
  SegDesc mine{};
  if (tid < nseg_all) {
    const int si = si_lo + tid;
    const int64_t st = kv.seg_start[si];
    mine.lo = st;
    mine.hi = st + kv.seg_len[si];
    mine.cap = kv.seg_cap[si];
    mine.k = static_cast<const unsigned char*>(kv.k_seg[si]);
    mine.v = static_cast<const unsigned char*>(kv.v_seg[si]);
  }
#pragma unroll
  for (int e = 0; e < kQPer; ++e) {
    const int i = tid + e * kThreads;
    if (i < kQChunks) *reinterpret_cast<uint4*>(q_lds + i * 16) = qv[e];
  }
  if (tid < nseg_all) segs[tid] = mine;
  if (tid == 0) nseg_sh = nseg_all;

  // Row geometry.
  const int64_t n_vis = p + 1 > 0 ? p + 1 : 0;
  const int64_t nb = n_vis / kBlockTokens;
  const int tail = (int)(n_vis - nb * kBlockTokens);
  int ns = ns_raw < 0 ? 0 : ns_raw;
  ns = ns > k_blocks ? k_blocks : ns;
  ns = (int64_t)ns > nb ? (int)nb : ns;
  const int total = ns * kBlockTokens + tail;

  // Running softmax state of this wave's QK heads (identical in all lanes).
  float m_run[kHeadsPerWaveQK], l_run[kHeadsPerWaveQK];
#pragma unroll
  for (int hh = 0; hh < kHeadsPerWaveQK; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
  }
  constexpr int DPT = TT::kDimsPerThread;
  const int dg = tid % (kThreads / kHeadHalves);
  const int half = tid / (kThreads / kHeadHalves);
  float acc[kHeadsPV][DPT];
#pragma unroll
  for (int h = 0; h < kHeadsPV; ++h)
#pragma unroll
    for (int d = 0; d < DPT; ++d) acc[h][d] = 0.f;

  __syncthreads();
  const int nseg = nseg_sh;
  // the first segment's descriptor, wave-uniform: held in scalar registers
  SegDesc seg0;
  {
    const SegDesc d0 = segs[0];
    auto u64 = [](uint64_t x) -> uint64_t {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
      return ((uint64_t)hi << 32) | lo;
    };
    seg0.lo = (int64_t)u64((uint64_t)d0.lo);
    seg0.hi = (int64_t)u64((uint64_t)d0.hi);
    seg0.cap = (int64_t)u64((uint64_t)d0.cap);
    seg0.k = reinterpret_cast<const unsigned char*>(u64(reinterpret_cast<uint64_t>(d0.k)));
    seg0.v = reinterpret_cast<const unsigned char*>(u64(reinterpret_cast<uint64_t>(d0.v)));
    seg0.ks = reinterpret_cast<const uint16_t*>(u64(reinterpret_cast<uint64_t>(d0.ks)));
    seg0.vs = reinterpret_cast<const uint16_t*>(u64(reinterpret_cast<uint64_t>(d0.vs)));
  }

  for (int t = 0; t < tiles_per_split; ++t) {
    const int j0 = tok_begin + t * kTileTok;
    if (j0 >= total) break;

    // 1. resolve this lane's staging rows, then issue all their loads at once
    int64_t tokv[kRows];
#pragma unroll
    for (int it = 0; it < TT::kItemsPerThread; ++it) {
      const int pair = (tid + it * kThreads) / TT::kChunks;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = it * 2 + u;
        const int j = j0 + 2 * pair + u;
        int64_t tok = -1;
        if (j < total) {
          if (j < ns * kBlockTokens) {
            const int64_t b = bid[i];
            if (b >= 0 && b < nb) tok = b * kBlockTokens + (j & 3);
          } else {
            tok = nb * kBlockTokens + (j - ns * kBlockTokens);
          }
        }
        tokv[i] = tok;
      }
    }
    const unsigned char* kp[kRows];
    const unsigned char* vp[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      kp[i] = qbytes;  // any readable address; masked below
      vp[i] = qbytes;
    }
    uint32_t okm = 0u;
    static_assert(kThreads % TT::kChunks == 0, "a lane keeps one chunk column");
    const int c_lane = tid % TT::kChunks;  // every item of a lane has the same chunk
    for (int si = 0; si < nseg; ++si) {  // uniform loop, one LDS broadcast per segment
      const SegDesc sd = segs[si];
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        const int64_t rel = tokv[i] - sd.lo;
        const bool hit = tokv[i] >= 0 && rel >= 0 && tokv[i] < sd.hi && rel < sd.cap && !((okm >> i) & 1u);
        const int64_t off = ((int64_t)g * sd.cap + rel) * TT::kRowBytes + c_lane * 16;
        kp[i] = hit ? sd.k + off : kp[i];
        vp[i] = hit ? sd.v + off : vp[i];
        okm |= hit ? (1u << i) : 0u;
      }
    }
    uint4 kk[kRows], vv[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      kk[i] = ldg16(kp[i]);
      vv[i] = ldg16(vp[i]);
    }
    // next tile's block ids, in flight during this tile's compute
    if (t + 1 < tiles_per_split) {
#pragma unroll
      for (int it = 0; it < TT::kItemsPerThread; ++it) {
        const int pair = (tid + it * kThreads) / TT::kChunks;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = j0 + kTileTok + 2 * pair + u;
          bid[it * 2 + u] = (j >> 2) < k_blocks ? srow[j >> 2] : -1;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < TT::kItemsPerThread; ++it) {
      const int item = tid + it * kThreads;
      const int pair = item / TT::kChunks;
      const int c = item % TT::kChunks;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = it * 2 + u;
        const bool ok = (okm >> i) & 1u;
        if (!ok) {
          kk[i] = make_uint4(0, 0, 0, 0);
          vv[i] = make_uint4(0, 0, 0, 0);
        }
        if (c == 0) valid_lds[2 * pair + u] = ok ? 1u : 0u;
        *reinterpret_cast<uint4*>(k_lds + (2 * pair + u) * TT::kKStride + c * 16) = kk[i];
      }
      if constexpr (kBf) {
        // pair-interleaved V: word (pair, dim) = (V[2 pair][dim], V[2 pair + 1][dim])
        uint4 lo, hi;
        interleave(vv[it * 2], vv[it * 2 + 1], lo, hi);
        uint4* dst = reinterpret_cast<uint4*>(v_lds + (pair * D + c * TT::kElemsPerChunk) * 4);
        dst[0] = lo;
        dst[1] = hi;
      } else {
        *reinterpret_cast<uint4*>(v_lds + (2 * pair) * TT::kRowBytes + c * 16) = vv[it * 2];
        *reinterpret_cast<uint4*>(v_lds + (2 * pair + 1) * TT::kRowBytes + c * 16) = vv[it * 2 + 1];
      }
    }
    __syncthreads();

    // 2. QK for heads 3w..3w+2, lane = token
    float sc[kHeadsPerWaveQK];
#pragma unroll
    for (int hh = 0; hh < kHeadsPerWaveQK; ++hh) sc[hh] = 0.f;
    const unsigned char* kl = k_lds + lane * TT::kKStride;
    const unsigned char* qw = q_lds + (wave * kHeadsPerWaveQK) * TT::kRowBytes;
#pragma unroll 4
    for (int c = 0; c < TT::kChunks; ++c) {
      const uint4 kv4 = *reinterpret_cast<const uint4*>(kl + c * 16);
#pragma unroll
      for (int hh = 0; hh < kHeadsPerWaveQK; ++hh) {
        const uint4 q4 = *reinterpret_cast<const uint4*>(qw + hh * TT::kRowBytes + c * 16);  // broadcast
        float a = sc[hh];
        if constexpr (kBf) {
          a = dot2_bf16(q4.x, kv4.x, a);
          a = dot2_bf16(q4.y, kv4.y, a);
          a = dot2_bf16(q4.z, kv4.z, a);
          a = dot2_bf16(q4.w, kv4.w, a);
        } else {
          a = fmaf(__uint_as_float(q4.x), __uint_as_float(kv4.x), a);
          a = fmaf(__uint_as_float(q4.y), __uint_as_float(kv4.y), a);
          a = fmaf(__uint_as_float(q4.z), __uint_as_float(kv4.z), a);
          a = fmaf(__uint_as_float(q4.w), __uint_as_float(kv4.w), a);
        }
        sc[hh] = a;
      }
    }
    const bool valid = valid_lds[lane] != 0u;

    // 3. online softmax
#pragma unroll
    for (int hh = 0; hh < kHeadsPerWaveQK; ++hh) {
      const float s2 = valid ? sc[hh] * scale_log2 : -INFINITY;
      const float tmax = wave_max(s2);
      const float m_new = fmaxf(m_run[hh], tmax);
      const float alpha = (m_run[hh] == m_new) ? 1.f : exp2f(m_run[hh] - m_new);
      float pv = (s2 == -INFINITY) ? 0.f : exp2f(s2 - m_new);
      const int h = wave * kHeadsPerWaveQK + hh;
      if constexpr (kBf) {
        // the PV dot2 consumes bf16 probabilities: normalise by the same values
        const uint32_t pb = f32_to_bf16_bits(pv);
        pv = __uint_as_float(pb << 16);
        const uint32_t nb16 = __shfl_xor(pb, 1, kWave);
        if ((lane & 1) == 0) p_lds[(lane >> 1) * kGroup + h] = pb | (nb16 << 16);
      } else {
        p_lds[lane * kGroup + h] = __float_as_uint(pv);
      }
      l_run[hh] = l_run[hh] * alpha + wave_sum(pv);
      m_run[hh] = m_new;
      if (lane == 0) alpha_lds[h] = alpha;
    }
    __syncthreads();

    // 4. PV
#pragma unroll
    for (int h = 0; h < kHeadsPV; ++h) {
      const float a = alpha_lds[half * kHeadsPV + h];
#pragma unroll
      for (int d = 0; d < DPT; ++d) acc[h][d] *= a;
    }
    const int rows = min(kTileTok, total - j0);
    if constexpr (kBf) {
      const int pairs = (rows + 1) >> 1;
      for (int pr = 0; pr < pairs; ++pr) {
        uint32_t w[DPT];
        if constexpr (DPT == 2) {
          const uint2 x = *reinterpret_cast<const uint2*>(v_lds + (pr * D + dg * 2) * 4);
          w[0] = x.x;
          w[1] = x.y;
        } else {
          w[0] = *reinterpret_cast<const uint32_t*>(v_lds + (pr * D + dg) * 4);
        }
        const uint32_t* pp = &p_lds[pr * kGroup + half * kHeadsPV];
#pragma unroll
        for (int h = 0; h < kHeadsPV; ++h) {
          const uint32_t pw = pp[h];
#pragma unroll
          for (int d = 0; d < DPT; ++d) acc[h][d] = dot2_bf16(pw, w[d], acc[h][d]);
        }
      }
    } else {
      for (int r = 0; r < rows; ++r) {
        float vv[DPT];
        const float* vp = reinterpret_cast<const float*>(v_lds + r * TT::kRowBytes) + dg * DPT;
#pragma unroll
        for (int d = 0; d < DPT; ++d) vv[d] = vp[d];
        const float* pr = reinterpret_cast<const float*>(&p_lds[r * kGroup + half * kHeadsPV]);
#pragma unroll
        for (int h = 0; h < kHeadsPV; ++h) {
          const float w = pr[h];
#pragma unroll
          for (int d = 0; d < DPT; ++d) acc[h][d] = fmaf(w, vv[d], acc[h][d]);
        }
      }
    }
    __syncthreads();
  }

  // Publish the softmax state, then write the partial (or final) output.
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < kHeadsPerWaveQK; ++hh) {
      m_lds[wave * kHeadsPerWaveQK + hh] = m_run[hh];
      l_lds[wave * kHeadsPerWaveQK + hh] = l_run[hh];
    }
  }
  __syncthreads();
  // bf16 PV dims: lane dg owns dims 2dg, 2dg+1 (DPT 2) or dg (DPT 1)
#pragma unroll
  for (int h6 = 0; h6 < kHeadsPV; ++h6) {
    const int h = half * kHeadsPV + h6;
    const float l = l_lds[h];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse = l > 0.f ? (m_lds[h] + log2f(l)) * kLn2 : -INFINITY;
    const int64_t head = (int64_t)m * hq + (int64_t)g * kGroup + h;
    if (splits == 1) {
      T* o = out + head * D + dg * DPT;
#pragma unroll
      for (int d = 0; d < DPT; ++d) o[d] = E::from_f(acc[h6][d] * inv);
      if (dg == 0) lse_out[head] = lse;
    } else {
      float* o = ws_o + (head * splits + split) * D + dg * DPT;
#pragma unroll
      for (int d = 0; d < DPT; ++d) o[d] = acc[h6][d] * inv;
      if (dg == 0) {  // no rounding here: the two lse values of a partial agree
        ws_lse[2 * (head * splits + split)] = lse;
        ws_lse[2 * (head * splits + split) + 1] = lse;
      }
    }
  }
}

// bf16 K/V: matrix-core kernel.  Grid and split plan as above; inside a
// workgroup each wave owns one 16-token slice of every 64-token tile and
// keeps its own online softmax state, so the tile loop has no workgroup
// barrier:
//   1. lanes resolve the slice's 16 tokens (lane % 16) to K and V rows; every
//      load of the slice is issued before any is used;
//   2. QK on v_mfma_f32_16x16x32_bf16: A = the group's 12 query heads (rows
//      12..15 zero) staged once in LDS in operand layout and read back per
//      slice (16 bytes per lane and k-step: no VGPRs held), B = the 16 tokens' K
//      rows loaded straight into the operand layout (lane: token lane % 16,
//      8 consecutive dims per k-step);
//   3. online softmax per head over the 16 lanes that hold a head's tokens
//      (base-2 exponentials, bf16-rounded probabilities packed in token
//      pairs into a wave-private LDS region); a running maximum moves only
//      when a logit exceeds it by more than kMaxSlack, and each lane sums
//      its own tokens' probabilities, added over the row after the loop;
//   4. PV on v_mfma_f32_16x16x16_bf16, D/16 instructions per slice: A = the
//      probabilities (12 heads x 16 tokens, read back from LDS in operand
//      layout), B = V staged in LDS as 4-token quads per dim (lane group g
//      reads tokens 4g .. 4g+3 of its dim in one 8-byte load); the output
//      lane holds heads 4 g .. 4 g + 3, the heads of its softmax state, so
//      the online rescale needs no lane exchange.
// At the end the wave partials are merged by log-sum-exp in LDS.
//
// F8: K/V are E4M3 codes with an f16 scale per KV head and token (the fp8
// state of the hipfire page, section 03).  Rows are D bytes; a lane reads
// 16 contiguous K bytes per pair of k-steps, so k-step s of lane quad g4
// covers dims 64 (s / 2) + 16 g4 + 8 (s % 2) .. + 7, and the query operand is
// loaded with the same dim permutation (the dot product is unchanged).  The
// codes become bf16 exactly; token t's logits are multiplied by its K scale,
// and its softmax weight by its V scale before the bf16 rounding that PV
// consumes (the normaliser sums the unscaled weights).  V goes to LDS as
// bf16 quads like the bf16 path.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));  // 4 bf16 operand of the 16x16x16 MFMA
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two float32 values to packed bf16 (first in the low half), rounded to
// nearest even by the hardware conversion.
typedef __bf16 bf16x2e_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2e_t));
}

// E4M3 codes -> bf16.  Every E4M3 value (4 significant bits, exponents
// 2^-9 .. 2^8) is exact in bf16; gfx950 converts two codes to a bf16 pair
// in one instruction (its scale operand 1: no scaling).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HI));
}
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                    fp8x2_to_bf16x2<true>(w1));
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ const unsigned char* shfl_ptr(const unsigned char* p, int src) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, kWave);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, kWave);
  return reinterpret_cast<const unsigned char*>(((uint64_t)hi << 32) | lo);
}

// Lane exchange inside a 16-lane row through the DPP modifier (no LDS
// traffic): quad_perm [1,0,3,2] and [2,3,0,1] (xor 1, xor 2), then
// row_half_mirror and row_mirror, which after the quad steps pair every
// lane with the other quad, then the other half.  Every lane of the row
// ends with the same bits (each step adds two equal-order operands).
template <int CTRL>
__device__ __forceinline__ int dpp_row(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);  // full-row patterns: every source lane exists
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// larger of two finite or -inf values (a compare and a select: no NaN
// canonicalisation, which fmaxf needs around lane exchanges)
__device__ __forceinline__ float max2(float a, float b) { return b > a ? b : a; }
template <int CTRL>
__device__ __forceinline__ float row_max_step(float x) {
  return max2(x, __int_as_float(dpp_row<CTRL>(__float_as_int(x))));
}
// max / sum over the 16 lanes of a row (lanes 16r .. 16r+15)
__device__ __forceinline__ float row16_max(float x) {
  x = row_max_step<kDppXor1>(x);
  x = row_max_step<kDppXor2>(x);
  x = row_max_step<kDppHalfMirror>(x);
  return row_max_step<kDppMirror>(x);
}
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(dpp_row<kDppXor1>(__float_as_int(x)));
  x += __int_as_float(dpp_row<kDppXor2>(__float_as_int(x)));
  x += __int_as_float(dpp_row<kDppHalfMirror>(__float_as_int(x)));
  return x + __int_as_float(dpp_row<kDppMirror>(__float_as_int(x)));
}

constexpr int kMaxWaves = 8;  // waves (16-token slices) per workgroup
// How far (log2 units) a logit may exceed its head's running maximum before
// the maximum moves: probabilities stay below 2^8, and rounding them to bf16
// keeps the same relative error whatever maximum they are taken against.
constexpr float kMaxSlack = 8.f;

// Where a masked token's K and V are read from: a row of zeros (its logit is
// replaced by -inf, and a zero V row adds nothing to P.V), so V needs no
// masking after the load.  Also its fp8 scales (0).
__device__ __align__(16) const unsigned char kZeroRow[512] = {};

// Word offset, inside a V quad row, of piece k (dims 8 u8 + 2k, + 1; 16
// bytes) of 8-dim unit u8.  The pieces of a unit are rotated by (u8 / 4) % 4
// so that the staging writes (one unit per lane, 64 bytes apart) spread over
// the LDS banks; the readers use the same map.
__device__ __forceinline__ constexpr int vslot(int u8, int k) { return 16 * u8 + 4 * ((k + (u8 >> 2)) & 3); }

// Dynamic LDS of the matrix-core kernel, in 32-bit words.  Phase 1, per wave:
// V of its 16-token slice as [token quad q][dim] -> 4 bf16 (tokens 4q ..
// 4q+3 of the dim, 8 bytes; quad rows padded), the PV B operand of lane
// group q; then the bf16 probabilities as [quad q][token parity p][head]
// words (tokens 4q+2p, 4q+2p+1 of the head), the A operand.  Phase 2 (merge,
// reusing the same memory): every wave's partial output, then the softmax
// states and the per-head merge weights.
template <int D>
struct MfmaLds {
  static constexpr int kQuadWords = 2 * D + 32;  // one token quad of V (+ pad)
  static constexpr int kPWords = 4 * 2 * 16;     // probabilities, heads 0..15
  static constexpr int kWaveWords = 4 * kQuadWords + kPWords;
  // the QK A operand (query heads), shared by the workgroup's waves: 16 bytes
  // per lane and k-step, after the wave regions
  static constexpr int kQWords = (D / 32) * kWave * 4;
  static constexpr int qop(int W) { return W * kWaveWords; }
  static constexpr int acc(int w) { return w * kGroup * D; }
  static constexpr int m(int W, int w) { return W * kGroup * D + w * kGroup; }
  static constexpr int l(int W, int w) { return W * kGroup * D + W * kGroup + w * kGroup; }
  static constexpr int l32(int W, int w) { return W * kGroup * D + 2 * W * kGroup + w * kGroup; }
  static constexpr int wt(int W, int h) { return W * kGroup * D + 3 * W * kGroup + h * kMaxWaves; }
  // per head: lse of the rounded normaliser (merge weights), lse of the float32 one (reported)
  static constexpr int lse(int W) { return W * kGroup * D + 3 * W * kGroup + kGroup * kMaxWaves; }
  static constexpr size_t bytes(int W) {
    return 4 * (size_t)(qop(W) + kQWords > lse(W) + 2 * kGroup ? qop(W) + kQWords : lse(W) + 2 * kGroup);
  }
};

// K/V formats of the matrix-core kernel: bf16, fp8 E4M3 codes with one f16
// scale per row, Q8_0 int8 codes with one f16 scale per 32 values.
constexpr int kKvBf16 = 0, kKvFp8 = 1, kKvQ8 = 2;

// Byte i of w as a signed integer, in float32: one conversion that reads the
// byte with sign extension (the compiler's sub-dword operand select).
__device__ __forceinline__ float sbyte_f(uint32_t w, int i) { return (float)(int)(int8_t)(uint8_t)(w >> (8 * i)); }
// Four signed bytes (one word) -> four bf16 values, exactly (|c| <= 128 fits
// bf16's 8-bit significand): the high halves of the float32 conversions.
__device__ __forceinline__ uint2 s8x4_to_bf16x4(uint32_t w) {
  const float a = sbyte_f(w, 0), b = sbyte_f(w, 1), c = sbyte_f(w, 2), d = sbyte_f(w, 3);
  return make_uint2(__builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u),
                    __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x07060302u));
}
// Four signed bytes times a scale -> four bf16 values: the float32 product
// (one rounding of the exact c sc), then the packed hardware conversion
// (rounded to nearest even).
__device__ __forceinline__ uint2 s8x4_scaled_bf16x4(uint32_t w, float sc) {
  const float a = sbyte_f(w, 0) * sc, b = sbyte_f(w, 1) * sc;
  const float c = sbyte_f(w, 2) * sc, d = sbyte_f(w, 3) * sc;
  return make_uint2(bf16x2_bits(a, b), bf16x2_bits(c, d));
}

template <int D, int NW, int KVF>
__global__ void __launch_bounds__(kWave * NW, NW < 8 ? 8 / NW : 1)  // at least 8 waves per CU: registers for 2 per SIMD
attn_mfma_kernel(const uint16_t* __restrict__ q, int M, int hq, float scale_log2,
                 const int64_t* __restrict__ row_pos, const int32_t* __restrict__ row_seq,
                 KvArgs kv, const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
                 int k_blocks, int tiles_per_split, int splits,
                 uint16_t* __restrict__ out, float* __restrict__ lse_out,
                 float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  constexpr int KS = D / 32;               // QK k-steps
  constexpr int NT = D / 16;               // PV output tiles of 16 dims
  constexpr bool F8 = KVF == kKvFp8;
  constexpr bool Q8 = KVF == kKvQ8;
  constexpr bool B8 = F8 || Q8;            // one byte per K/V value
  constexpr int kRowBytes = B8 ? D : D * 2;
  constexpr int QB = D / 32;               // Q8_0 scale blocks per row (= QK k-steps)
  constexpr int VCH = kRowBytes / 16;      // 16-byte chunks per V row
  constexpr int VITEMS = 4 * VCH;          // (token quad, chunk) V staging items
  constexpr int VIT = (VITEMS + kWave - 1) / kWave;  // per lane
  constexpr int KL = B8 ? KS / 2 : KS;     // 16-byte K registers per lane (Q8: two 8-byte loads each)
  static_assert(kRowBytes <= (int)sizeof(kZeroRow), "zero row shorter than a K/V row");
  using Lds = MfmaLds<D>;
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ SegDesc segs[kMaxSegments];
  __shared__ int nseg_sh;

  constexpr int nw = NW;  // waves = 16-token slices per tile
  constexpr int tile = 16 * nw;
  const int g = blockIdx.x;  // grid (KV head, row, split)
  const int m = blockIdx.y;
  const int split = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid / kWave);
  const int n16 = lane & 15;   // token of the slice (QK operand and softmax row position)
  const int g4 = lane >> 4;    // k-slice of the operands / head quad of the scores
  const int tok_begin = split * tiles_per_split * tile;
  const int32_t* __restrict__ srow = sel + (int64_t)m * k_blocks;

  // ---- independent loads, issued together
  const int64_t p = row_pos[m];
  const int ns_raw = n_sel[m];
  const int sq_raw = row_seq ? row_seq[m] : 0;
  int32_t bid;
  {
    const int j = tok_begin + wave * 16 + n16;
    bid = (j >> 2) < k_blocks ? srow[j >> 2] : -1;
  }
  // query operand, staged once in LDS for all waves: chunk i is k-step i / 64
  // of lane i % 64, i.e. head (i % 64) % 16 (heads 12..15 are zero), dims
  // 32 s + 8 g .. + 7 for lane group g (fp8: the permuted dims below)
  constexpr int kQChunks = KS * kWave;
  constexpr int kQPer = (kQChunks + kWave * NW - 1) / (kWave * NW);
  uint4 qraw[kQPer];
#pragma unroll
  for (int e = 0; e < kQPer; ++e) {
    const int i = tid + kWave * NW * e;
    const int ic = i < kQChunks ? i : 0;
    const int s = ic / kWave, h = ic & 15, gq = (ic % kWave) >> 4;
    const int dim = F8 ? 64 * (s >> 1) + 16 * gq + 8 * (s & 1) : 32 * s + 8 * gq;
    qraw[e] = ldg16(reinterpret_cast<const unsigned char*>(
                        q + ((int64_t)m * hq + (int64_t)g * kGroup + (h < kGroup ? h : 0)) * D) +
                    dim * 2);
  }
  int si_lo = 0, nseg_all = 0;
  if (kv.n_seq == 1) {
    nseg_all = kv.n_seg_total < kMaxSegments ? kv.n_seg_total : kMaxSegments;
  } else {
    const bool seq_ok = sq_raw >= 0 && sq_raw < kv.n_seq;
    const int sq = seq_ok ? sq_raw : 0;
    int s_begin = kv.seq_seg_begin[sq], s_end = kv.seq_seg_begin[sq + 1];
    s_begin = s_begin < 0 ? 0 : s_begin;
    s_end = s_end > kv.n_seg_total ? kv.n_seg_total : s_end;
    si_lo = s_begin;
    nseg_all = (seq_ok && s_end > s_begin) ? min(s_end - s_begin, kMaxSegments) : 0;
  }
  SegDesc mine{};
  if (tid < nseg_all) {
    const int si = si_lo + tid;
    const int64_t st = kv.seg_start[si];
    mine.lo = st;
    mine.hi = st + kv.seg_len[si];
    mine.cap = kv.seg_cap[si];
    mine.k = static_cast<const unsigned char*>(kv.k_seg[si]);
    mine.v = static_cast<const unsigned char*>(kv.v_seg[si]);
    if constexpr (B8) {
      mine.ks = kv.k_scale[si];
      mine.vs = kv.v_scale[si];
    }
  }
  if (tid < nseg_all) segs[tid] = mine;
  if (tid == 0) nseg_sh = nseg_all;
  uint4* qop = reinterpret_cast<uint4*>(lds + Lds::qop(nw));
#pragma unroll
  for (int e = 0; e < kQPer; ++e) {
    const int i = tid + kWave * NW * e;
    if (i < kQChunks) qop[i] = (i & 15) < kGroup ? qraw[e] : make_uint4(0, 0, 0, 0);
  }
  // k-step s of this lane's query operand (read per slice: no VGPRs held)
  auto qa = [&](int s) { return __builtin_bit_cast(bf16x8_t, qop[s * kWave + lane]); };

  const int64_t n_vis = p + 1 > 0 ? p + 1 : 0;
  const int64_t nb = n_vis / kBlockTokens;
  const int tail = (int)(n_vis - nb * kBlockTokens);
  int ns = ns_raw < 0 ? 0 : ns_raw;
  ns = ns > k_blocks ? k_blocks : ns;
  ns = (int64_t)ns > nb ? (int)nb : ns;
  const int total = ns * kBlockTokens + tail;
  __syncthreads();
  const int nseg = nseg_sh;
  // the first segment's descriptor, wave-uniform: held in scalar registers
  SegDesc seg0;
  {
    const SegDesc d0 = segs[0];
    auto u64 = [](uint64_t x) -> uint64_t {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
      return ((uint64_t)hi << 32) | lo;
    };
    seg0.lo = (int64_t)u64((uint64_t)d0.lo);
    seg0.hi = (int64_t)u64((uint64_t)d0.hi);
    seg0.cap = (int64_t)u64((uint64_t)d0.cap);
    seg0.k = reinterpret_cast<const unsigned char*>(u64(reinterpret_cast<uint64_t>(d0.k)));
    seg0.v = reinterpret_cast<const unsigned char*>(u64(reinterpret_cast<uint64_t>(d0.v)));
    seg0.ks = reinterpret_cast<const uint16_t*>(u64(reinterpret_cast<uint64_t>(d0.ks)));
    seg0.vs = reinterpret_cast<const uint16_t*>(u64(reinterpret_cast<uint64_t>(d0.vs)));
  }

  // running maxima of heads 4 g4 + v (identical over the 16 lanes of a row)
  // and this lane's share of their normalisers (its tokens' probabilities;
  // summed over the row after the loop): l_part sums the bf16-rounded
  // probabilities that P.V consumes (the output is normalised by it, so its
  // weights sum to one), l_full the float32 probabilities (the reported lse
  // comes from it, free of the bf16 rounding)
  float m_run[4], l_part[4], l_full[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    m_run[v] = -INFINITY;
    l_part[v] = 0.f;
    l_full[v] = 0.f;
  }
  // PV accumulators: pacc[n][r] = O[head 4 g4 + r][dim 16 n + n16] (heads
  // 12..15 of lane group 3 are padding)
  f32x4_t pacc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) pacc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t* vl = lds + wave * Lds::kWaveWords;
  uint32_t* pl = vl + 4 * Lds::kQuadWords;

  // Slice pipeline: slice t+1's K loads are issued right after slice t's QK
  // and its V loads right after slice t's V staging, into the same
  // registers, so they are in flight during slice t's softmax and P.V.
  struct SliceAddr {
    const unsigned char* kr;
    const unsigned char* vr;
    const uint16_t* ksp;
    const uint16_t* vsp;
    int ok;
  };
  // 1. token of this lane's position in slice t (block id bidv) -> K/V rows;
  // with live false every token is masked
  auto resolve_slice = [&](int t, int32_t bidv, bool live) -> SliceAddr {
    const int j = tok_begin + t * tile + wave * 16 + n16;
    int64_t tok = -1;
    if (live && j < total) {
      if (j < ns * kBlockTokens) {
        if (bidv >= 0 && bidv < nb) tok = (int64_t)bidv * kBlockTokens + (j & 3);
      } else {
        tok = nb * kBlockTokens + (j - ns * kBlockTokens);
      }
    }
    // a masked token reads the zero row
    const unsigned char* zr = kZeroRow;
    SliceAddr a{zr, zr, reinterpret_cast<const uint16_t*>(zr), reinterpret_cast<const uint16_t*>(zr), 0};
    auto resolve = [&](const SegDesc& sd) {
      const int64_t rel = tok - sd.lo;
      const bool hit = tok >= 0 && rel >= 0 && tok < sd.hi && rel < sd.cap && !a.ok;
      const int64_t row = (int64_t)g * sd.cap + rel;
      a.kr = hit ? sd.k + row * kRowBytes : a.kr;
      a.vr = hit ? sd.v + row * kRowBytes : a.vr;
      if constexpr (F8) {
        a.ksp = hit ? sd.ks + row : a.ksp;
        a.vsp = hit ? sd.vs + row : a.vsp;
      } else if constexpr (Q8) {
        a.ksp = hit ? sd.ks + row * QB : a.ksp;
        a.vsp = hit ? sd.vs + row * QB : a.vsp;
      }
      a.ok |= hit ? 1 : 0;
    };
    if (nseg == 1) {
      resolve(seg0);  // one segment (the common case): its descriptor stays in registers
    } else {
      for (int si = 0; si < nseg; ++si) resolve(segs[si]);
    }
    return a;
  };
  // block id of the lane's token in slice t (index clamped, so the load is
  // unconditional; resolve_slice reads it only for tokens of the first ns
  // blocks, ns <= k_blocks, so the value is used raw: no select waits on it)
  auto block_id = [&](int t) -> int32_t {
    const int jb = (tok_begin + t * tile + wave * 16 + n16) >> 2;
    return srow[jb < k_blocks ? jb : k_blocks - 1];
  };
  uint4 kb[KL];  // K operand rows: all k-steps
  uint32_t ks_bits = 0, vs_bits = 0;
  uint4 ksq = make_uint4(0, 0, 0, 0);  // Q8: the lane's token's K scales, one f16 per k-step
  auto load_k = [&](const SliceAddr& a) {
    if constexpr (Q8) {  // k-step s = dims 32 s + 8 g4 .. + 7 = scale block s
#pragma unroll
      for (int s = 0; s < KL; ++s) {
        const uint2 lo = ldg8(a.kr + 64 * s + 8 * g4);
        const uint2 hi = ldg8(a.kr + 64 * s + 32 + 8 * g4);
        kb[s] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
      if constexpr (QB == 8) {
        ksq = ldg16(reinterpret_cast<const unsigned char*>(a.ksp));
      } else {
        const uint2 q2 = ldg8(reinterpret_cast<const unsigned char*>(a.ksp));
        ksq = make_uint4(q2.x, q2.y, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KL; ++s) kb[s] = ldg16(a.kr + (F8 ? 64 * s + 16 * g4 : (32 * s + 8 * g4) * 2));
    }
    if constexpr (F8) {
      ks_bits = *a.ksp;
      vs_bits = *a.vsp;
    }
  };
  // V items: (token quad vq, chunk c) of the slice; lanes past the item
  // count (fp8 at head_dim 128) load a valid chunk and write nothing
  uint4 vt[VIT][4];
  uint32_t vsc[VIT][4];  // Q8: each staged chunk's V scale (f16 bits)
  auto load_v = [&](const SliceAddr& a) {
#pragma unroll
    for (int u = 0; u < VIT; ++u) {
      const int item = (lane + kWave * u) % VITEMS;
      const int vq = item / VCH;
      const int c = item % VCH;
#pragma unroll
      for (int e = 0; e < 4; ++e) vt[u][e] = ldg16(shfl_ptr(a.vr, 4 * vq + e) + c * 16);
      if constexpr (Q8) {  // chunk c = dims 16 c .. 16 c + 15: scale block c / 2
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vsc[u][e] = *reinterpret_cast<const uint16_t*>(
              shfl_ptr(reinterpret_cast<const unsigned char*>(a.vsp), 4 * vq + e) + (c >> 1) * 2);
      }
    }
  };
  SliceAddr cur = resolve_slice(0, bid, true);
  int32_t bid_n = block_id(1);  // slice 1
  load_k(cur);
  // K before V, as in the loop body: the loop head then waits for K only
  __builtin_amdgcn_sched_barrier(0);
  load_v(cur);

  for (int t = 0; t < tiles_per_split; ++t) {
    const int j0 = tok_begin + t * tile + wave * 16;
    if (j0 >= total) break;  // wave-uniform: the loop has no workgroup barrier
    const int ok = cur.ok;
    // 2. QK: sacc[v] = q[head 4 g4 + v] . K[token n16] (a masked token's
    // logit is replaced below: its K needs no mask)
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (Q8) {
      // per k-step partial products, each scaled by the token's block scale
      const uint32_t ksw[4] = {ksq.x, ksq.y, ksq.z, ksq.w};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint32_t w0 = (s & 1) ? kb[s >> 1].z : kb[s >> 1].x;
        const uint32_t w1 = (s & 1) ? kb[s >> 1].w : kb[s >> 1].y;
        const uint2 b0 = s8x4_to_bf16x4(w0), b1 = s8x4_to_bf16x4(w1);
        const uint4 bq = make_uint4(b0.x, b0.y, b1.x, b1.y);
        const f32x4_t part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa(s), __builtin_bit_cast(bf16x8_t, bq),
                                                                     f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float sc = f16_bits_to_f32((ksw[s >> 1] >> (16 * (s & 1))) & 0xffffu);
#pragma unroll
        for (int v = 0; v < 4; ++v) sacc[v] = fmaf(sc, part[v], sacc[v]);
      }
    } else if constexpr (F8) {
#pragma unroll
      for (int s = 0; s < KL; ++s) {
        const uint4 lo = fp8x8_to_bf16x8(kb[s].x, kb[s].y);
        const uint4 hi = fp8x8_to_bf16x8(kb[s].z, kb[s].w);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa(2 * s), __builtin_bit_cast(bf16x8_t, lo), sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa(2 * s + 1), __builtin_bit_cast(bf16x8_t, hi), sacc, 0, 0,
                                                       0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa(s), __builtin_bit_cast(bf16x8_t, kb[s]), sacc, 0, 0, 0);
    }
    // fp8: this lane's token scales (0 for a masked token)
    const float k_sc = F8 ? (ok ? f16_bits_to_f32(ks_bits) : 0.f) : 1.f;
    const float v_sc = F8 ? (ok ? f16_bits_to_f32(vs_bits) : 0.f) : 1.f;
    // next slice of this split: its rows and K loads.  Past the split's last
    // slice every token is masked and the loads read the zero row: the loads
    // stay unconditional, so every path through the loop has the same loads
    // in flight and each wait counts only the loads it needs.
    const bool more = t + 1 < tiles_per_split;
    const SliceAddr nxt = resolve_slice(t + 1, bid_n, more);
    load_k(nxt);
    bid_n = block_id(t + 2);

    // 3. online softmax per head over the row's 16 tokens (base-2 logits).
    // A head's running maximum moves only when the row's maximum exceeds it
    // by more than kMaxSlack (always on a wave's first slice, rarely after),
    // so the accumulator rescale below is usually skipped.
    float alpha[4];
    uint32_t pw[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float s2 = ok ? (F8 ? sacc[v] * k_sc : sacc[v]) * scale_log2 : -INFINITY;
      const float rmax = row16_max(s2);
      const float m_new = rmax > m_run[v] + kMaxSlack ? rmax : m_run[v];
      alpha[v] = (m_run[v] == m_new) ? 1.f : __builtin_amdgcn_exp2f(m_run[v] - m_new);
      const float pv = (s2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s2 - m_new);
      // PV consumes bf16 (rounded to nearest even): normalise by the same
      // values; fp8: V's scale joins the PV weight (the high half)
      const uint32_t both = bf16x2_bits(pv, F8 ? pv * v_sc : pv);
      l_part[v] = l_part[v] * alpha[v] + __uint_as_float(both << 16);
      l_full[v] = l_full[v] * alpha[v] + pv;
      m_run[v] = m_new;
      const uint32_t pbv = both >> 16;
      pw[v] = pbv | ((uint32_t)dpp_row<kDppXor1>((int)pbv) << 16);
    }
    // probabilities of token pair n16/2 (quad n16/4, parity (n16/2)%2),
    // heads 4 g4 .. 4 g4 + 3
    if ((n16 & 1) == 0 && g4 < 3)
      *reinterpret_cast<uint4*>(pl + (n16 >> 2) * 32 + ((n16 >> 1) & 1) * 16 + 4 * g4) =
          make_uint4(pw[0], pw[1], pw[2], pw[3]);
    // V as [quad][dim] -> 4 tokens: per dim the words (t0, t1) and (t2, t3)
#pragma unroll
    for (int u = 0; u < VIT; ++u) {
      if (VITEMS % kWave != 0 && lane + kWave * u >= VITEMS) continue;
      const int item = lane + kWave * u;
      const int vq = item / VCH;
      const int c = item % VCH;
      const uint4* t = vt[u];  // a masked token's row is the zero row
      // one 8-dim unit u8 (dims 8 u8 .. + 7): tokens' words -> 8 dims x
      // (t0 t1, t2 t3); its four 16-byte pieces are rotated by vslot
      auto put8 = [&](uint4 a, uint4 b, uint4 cc, uint4 d, uint32_t* quad, int u8) {
        uint4 lo01, hi01, lo23, hi23;
        interleave(a, b, lo01, hi01);
        interleave(cc, d, lo23, hi23);
        const uint4 piece[4] = {make_uint4(lo01.x, lo23.x, lo01.y, lo23.y), make_uint4(lo01.z, lo23.z, lo01.w, lo23.w),
                                make_uint4(hi01.x, hi23.x, hi01.y, hi23.y), make_uint4(hi01.z, hi23.z, hi01.w, hi23.w)};
#pragma unroll
        for (int k = 0; k < 4; ++k) *reinterpret_cast<uint4*>(quad + vslot(u8, k)) = piece[k];
      };
      uint32_t* quad = vl + vq * Lds::kQuadWords;
      if constexpr (Q8) {  // 16 codes per token: dims 16 c .. 16 c + 15, times the token's block scale
        uint4 lo8[4], hi8[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sc = f16_bits_to_f32(vsc[u][e]);
          const uint2 a0 = s8x4_scaled_bf16x4(t[e].x, sc), a1 = s8x4_scaled_bf16x4(t[e].y, sc);
          const uint2 a2 = s8x4_scaled_bf16x4(t[e].z, sc), a3 = s8x4_scaled_bf16x4(t[e].w, sc);
          lo8[e] = make_uint4(a0.x, a0.y, a1.x, a1.y);
          hi8[e] = make_uint4(a2.x, a2.y, a3.x, a3.y);
        }
        put8(lo8[0], lo8[1], lo8[2], lo8[3], quad, 2 * c);
        put8(hi8[0], hi8[1], hi8[2], hi8[3], quad, 2 * c + 1);
      } else if constexpr (F8) {  // 16 codes per token: dims 16 c .. 16 c + 15
        put8(fp8x8_to_bf16x8(t[0].x, t[0].y), fp8x8_to_bf16x8(t[1].x, t[1].y), fp8x8_to_bf16x8(t[2].x, t[2].y),
             fp8x8_to_bf16x8(t[3].x, t[3].y), quad, 2 * c);
        put8(fp8x8_to_bf16x8(t[0].z, t[0].w), fp8x8_to_bf16x8(t[1].z, t[1].w), fp8x8_to_bf16x8(t[2].z, t[2].w),
             fp8x8_to_bf16x8(t[3].z, t[3].w), quad, 2 * c + 1);
      } else {  // 8 dims per chunk: dims 8 c .. 8 c + 7
        put8(t[0], t[1], t[2], t[3], quad, c);
      }
    }
    load_v(nxt);  // the V registers are free again
    cur = nxt;
    // (on a wave's first slice the accumulators are still zero: nothing to rescale)
    if (t > 0 && __ballot(alpha[0] != 1.f || alpha[1] != 1.f || alpha[2] != 1.f || alpha[3] != 1.f)) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) pacc[n][r] *= alpha[r];  // the lane's heads are its softmax heads
    }
    __builtin_amdgcn_wave_barrier();
    // 4. PV on v_mfma_f32_16x16x16_bf16: A = P (head n16, tokens 4 g4 .. + 3),
    // B = V (tokens 4 g4 .. + 3, dim 16 n + n16)
    const uint2 pa = n16 < kGroup ? make_uint2(pl[g4 * 32 + n16], pl[g4 * 32 + 16 + n16]) : make_uint2(0, 0);
    const s16x4_t pa4 = __builtin_bit_cast(s16x4_t, pa);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int dim = 16 * n + n16;
      const uint2 vb2 =
          *reinterpret_cast<const uint2*>(vl + g4 * Lds::kQuadWords + vslot(dim >> 3, (dim & 7) >> 1) + 2 * (dim & 1));
      pacc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa4, __builtin_bit_cast(s16x4_t, vb2), pacc[n], 0, 0, 0);
    }
    // interleave the B reads (paired 8-byte reads) with the matrix
    // instructions, a few reads ahead, instead of holding all D/16 operands
    // in registers at once
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < NT / 2 - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_wave_barrier();
  }

  float l_run[4], l_f32[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    l_run[v] = row16_sum(l_part[v]);
    l_f32[v] = row16_sum(l_full[v]);
  }
  // ---- merge the wave partials (log2 domain)
  __syncthreads();  // every wave is done with its V / P region
  float* fl = reinterpret_cast<float*>(lds);
  if (g4 < 3) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < NT; ++n) fl[Lds::acc(wave) + (4 * g4 + r) * D + 16 * n + n16] = pacc[n][r];
  }
  if (n16 == 0 && g4 < 3) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      fl[Lds::m(nw, wave) + 4 * g4 + v] = m_run[v];
      fl[Lds::l(nw, wave) + 4 * g4 + v] = l_run[v];
      fl[Lds::l32(nw, wave) + 4 * g4 + v] = l_f32[v];
    }
  }
  __syncthreads();
  if (tid < kGroup) {  // per-head merge weights, once
    const int h = tid;
    // every wave's (m, l, l32) read in one batch, the weights written in one
    float mw[nw], lw[nw], l32w[nw];
#pragma unroll
    for (int w = 0; w < nw; ++w) {
      mw[w] = fl[Lds::m(nw, w) + h];
      lw[w] = fl[Lds::l(nw, w) + h];
      l32w[w] = fl[Lds::l32(nw, w) + h];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < nw; ++w) mx = fmaxf(mx, mw[w]);
    float f[nw];
    float L = 0.f, L32 = 0.f;
#pragma unroll
    for (int w = 0; w < nw; ++w) {
      f[w] = (mx == -INFINITY || mw[w] == -INFINITY) ? 0.f : exp2f(mw[w] - mx);
      L += lw[w] * f[w];
      L32 += l32w[w] * f[w];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int w = 0; w < nw; ++w) fl[Lds::wt(nw, h) + w] = f[w] * inv;
    fl[Lds::lse(nw) + 2 * h] = L > 0.f ? (mx + log2f(L)) * kLn2 : -INFINITY;
    fl[Lds::lse(nw) + 2 * h + 1] = L32 > 0.f ? (mx + log2f(L32)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  // 4 consecutive dims of one head per thread and step: 16-byte LDS reads
  // and stores
  for (int o = 4 * tid; o < kGroup * D; o += 4 * kWave * nw) {
    const int h = o / D;
    const int d = o % D;
    const float* wt = fl + Lds::wt(nw, h);
    f32x4_t O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < nw; ++w) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(fl + Lds::acc(w) + o);
      const float ww = wt[w];
#pragma unroll
      for (int r = 0; r < 4; ++r) O[r] = fmaf(a[r], ww, O[r]);
    }
    const int64_t head = (int64_t)m * hq + (int64_t)g * kGroup + h;
    if (splits == 1) {
      *reinterpret_cast<uint2*>(out + head * D + d) =
          make_uint2((uint32_t)f32_to_bf16_bits(O[0]) | ((uint32_t)f32_to_bf16_bits(O[1]) << 16),
                     (uint32_t)f32_to_bf16_bits(O[2]) | ((uint32_t)f32_to_bf16_bits(O[3]) << 16));
      if (d == 0) lse_out[head] = fl[Lds::lse(nw) + 2 * h + 1];
    } else {
      *reinterpret_cast<f32x4_t*>(ws_o + (head * splits + split) * D + d) = O;
      if (d == 0) *reinterpret_cast<f32x2_t*>(ws_lse + 2 * (head * splits + split)) =
          f32x2_t{fl[Lds::lse(nw) + 2 * h], fl[Lds::lse(nw) + 2 * h + 1]};
    }
  }
}

// Merge split partials by log-sum-exp.  One workgroup per (row, head), one
// thread per output dimension.  Each thread's partial outputs (up to
// kRegSplits) are loaded at once, and every wave loads all the splits' lse
// pairs (lane i holds splits i and 64 + i): each wave finds the maximum,
// the weights and their sums itself (DPP reductions) and reads the weights
// out of its lanes, so the merge takes one memory round trip and no
// workgroup barrier.  A partial carries two lse values:
// that of the normaliser its output was divided by (the sum of the
// bf16-rounded probabilities P.V consumed), which weighs the outputs so that
// the merge equals one normalisation over all tokens, and that of the
// float32 probabilities, which gives the reported lse.  (They coincide for
// float32 K/V.)
constexpr int kRegSplits = 72;

// NS: the splits one thread holds in registers (the launch picks the
// smallest multiple of 8 up to 72 that covers the plan, so no load is spent on
// padding); more splits than 72 take plain loops.
template <class E, int D, int NS>
__global__ void __launch_bounds__(D)
attn_combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse, int splits,
                    typename E::T* __restrict__ out, float* __restrict__ lse_out) {
  static_assert(D >= NS && NS <= kRegSplits && kRegSplits <= 2 * kWave, "split lse pairs: two per lane");
  const int64_t head = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const float* __restrict__ L = ws_lse + 2 * head * splits;  // (weighting, reported) per split
  const float* __restrict__ O = ws_o + head * splits * D + tid;
  if (splits > NS) {  // long budgets: plain loops
    float mx = -INFINITY, tot = 0.f, tot32 = 0.f, o = 0.f;
    for (int i = 0; i < splits; ++i) mx = fmaxf(mx, L[2 * i]);
    if (mx != -INFINITY) {
      for (int i = 0; i < splits; ++i) {
        const float li = L[2 * i], l32 = L[2 * i + 1];
        const float w = li == -INFINITY ? 0.f : expf(li - mx);
        tot += w;
        tot32 += l32 == -INFINITY ? 0.f : expf(l32 - mx);
        o = fmaf(w, O[(int64_t)i * D], o);
      }
    }
    const bool empty = (mx == -INFINITY) || tot == 0.f;
    out[head * D + tid] = E::from_f(empty ? 0.f : o / tot);
    if (tid == 0) lse_out[head] = empty ? -INFINITY : mx + logf(tot32);
    return;
  }
  constexpr int kHalves = NS > kWave ? 2 : 1;
  float ov[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) ov[i] = O[(int64_t)(i < splits ? i : splits - 1) * D];  // masked by w = 0
  f32x2_t lp[kHalves];
#pragma unroll
  for (int hv = 0; hv < kHalves; ++hv) {
    const int i = lane + kWave * hv;
    lp[hv] = i < splits ? *reinterpret_cast<const f32x2_t*>(L + 2 * i) : f32x2_t{-INFINITY, -INFINITY};
  }
  float mx = lp[0].x;
#pragma unroll
  for (int hv = 1; hv < kHalves; ++hv) mx = fmaxf(mx, lp[hv].x);
  mx = wave_max(mx);
  const bool empty = (mx == -INFINITY);
  float w[kHalves];
  float tot = 0.f, tot32 = 0.f;
#pragma unroll
  for (int hv = 0; hv < kHalves; ++hv) {
    w[hv] = (empty || lp[hv].x == -INFINITY) ? 0.f : expf(lp[hv].x - mx);
    const float w32 = (empty || lp[hv].y == -INFINITY) ? 0.f : expf(lp[hv].y - mx);
    tot += wave_sum(w[hv]);
    tot32 += wave_sum(w32);
  }
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i)  // every partial is finite
    o = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[i / kWave]), i % kWave)), ov[i], o);
  const bool none = empty || tot == 0.f;
  out[head * D + tid] = E::from_f(none ? 0.f : o / tot);
  if (tid == 0) lse_out[head] = none ? -INFINITY : mx + logf(tot32);
}

template <class E, int D, int KVF = kKvBf16>
hipError_t launch_typed(const void* q, int M, int hq, int hkv, float scale,
                        const int64_t* row_pos, const int32_t* row_seq, const KvArgs& kv,
                        const int32_t* sel, const int32_t* n_sel, int k_blocks, void* out,
                        float* lse, void* ws, hipStream_t stream) {
  constexpr bool kMfma = (E::kBytes == 2);
  const AttnPlan plan = kMfma ? attn_plan(M, hkv, k_blocks) : attn_plan_valu(M, hkv, k_blocks);
  float* ws_o = static_cast<float*>(ws);
  float* ws_lse = ws_o ? ws_o + (size_t)M * hq * plan.splits * D : nullptr;  // 2 per partial
  dim3 grid(plan.splits, hkv, M), block(kWave * plan.waves);
  if constexpr (kMfma) {
    grid = dim3(hkv, M, plan.splits);
    const size_t lds = MfmaLds<D>::bytes(plan.waves);
#define QSA_MFMA_LAUNCH(W)                                                                              \
  case W:                                                                                             \
    hipLaunchKernelGGL((attn_mfma_kernel<D, W, KVF>), grid, block, lds, stream,                       \
                       static_cast<const uint16_t*>(q), M, hq, scale * kLog2e, row_pos, row_seq, kv,  \
                       sel, n_sel, k_blocks, plan.tiles_per_split, plan.splits,                       \
                       static_cast<uint16_t*>(out), lse, ws_o, ws_lse);                               \
    break;
    switch (plan.waves) {
      QSA_MFMA_LAUNCH(3)
      QSA_MFMA_LAUNCH(4)
      QSA_MFMA_LAUNCH(5)
      QSA_MFMA_LAUNCH(6)
      QSA_MFMA_LAUNCH(7)
      QSA_MFMA_LAUNCH(8)
      default: return hipErrorInvalidConfiguration;
    }
#undef QSA_MFMA_LAUNCH
  } else {
    hipLaunchKernelGGL((attn_decode_kernel<E, D>), grid, block, 0, stream,
                       static_cast<const typename E::T*>(q), M, hq, scale * kLog2e, row_pos, row_seq,
                       kv, sel, n_sel, k_blocks, plan.tiles_per_split, plan.splits,
                       static_cast<typename E::T*>(out), lse, ws_o, ws_lse);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  const dim3 cgrid((unsigned)M * hq), cblock(D);
  typename E::T* o = static_cast<typename E::T*>(out);
  // the smallest multiple of 8 register-held splits that covers the plan
#define QSA_COMBINE(NS)                                                                                  \
  case NS / 8:                                                                                          \
    hipLaunchKernelGGL((attn_combine_kernel<E, D, NS>), cgrid, cblock, 0, stream, ws_o, ws_lse, plan.splits, o, \
                       lse);                                                                            \
    break;
  switch (plan.splits <= kRegSplits ? (plan.splits + 7) / 8 : kRegSplits / 8) {
    QSA_COMBINE(8)
    QSA_COMBINE(16)
    QSA_COMBINE(24)
    QSA_COMBINE(32)
    QSA_COMBINE(40)
    QSA_COMBINE(48)
    QSA_COMBINE(56)
    QSA_COMBINE(64)
    default:  // more than 64 splits (the kernel loops past kRegSplits)
      hipLaunchKernelGGL((attn_combine_kernel<E, D, kRegSplits>), cgrid, cblock, 0, stream, ws_o, ws_lse,
                         plan.splits, o, lse);
  }
#undef QSA_COMBINE
  return hipGetLastError();
}

}  // namespace

// Compute units of a gfx950 device (MI350X / MI355X).
constexpr long kCUs = 256;

// Matrix-core kernel: a workgroup holds `waves` 16-token slices of a tile.
// The fewest waves, from 3 up to 8, with which every (row, KV head, split)
// workgroup has a compute unit of its own: a second workgroup on a unit
// slows both more than another wave does.  Three waves serve one or two rows
// (measured, M = 1 at a 2,051-token budget: 10.2 us with 3 waves and 43
// splits, 10.5 with 4 and 33, 17.3 with 2 and 65: past that the combine's
// partials cost more than the shorter tiles save).  When even 8
// waves cannot fit, several tiles per workgroup: up to 4 units' worth of
// one-tile workgroups, 4 waves walking as many tiles as keep the grid to one
// workgroup per unit; beyond that (prefill) 8 waves walking as many tiles as
// keep it to 4 workgroups per unit.
AttnPlan attn_plan(int M, int hkv, int k_blocks) {
  const int max_tokens = k_blocks * kBlockTokens + (kBlockTokens - 1);
  const int slices = (max_tokens + 15) / 16;
  const long rows = (long)M * hkv;
  AttnPlan p;
  int w = 3;
  while (w < kMaxWaves && rows * ((slices + w - 1) / w) > kCUs) ++w;
  const int tiles = (slices + w - 1) / w;
  p.waves = w;
  p.tile_tokens = 16 * w;
  p.tiles_per_split = 1;
  if (rows * tiles > 4 * kCUs) {  // many rows (prefill): a few workgroups per compute unit, long walks
    long want = 4 * kCUs / rows;
    if (want < 1) want = 1;
    p.tiles_per_split = (int)((tiles + want - 1) / want);
  } else if (rows * tiles > kCUs) {
    // more one-tile workgroups than compute units: walk several tiles per
    // split so that the grid is one round of workgroups, not two or three
    // rounds of short ones, with 4 waves (one per SIMD: a walk's slices are
    // latency-bound, a SIMD of its own shortens each).  Measured, 16 rows of
    // batched decode: 23.1 us against 35.2 us for one-tile splits; 8 waves
    // with 3 tiles per split 24.4 us, 4 waves with 3, 4, 5 or 9 tiles 26.0,
    // 23.1, 23.2, 30.4 us; 3 or 5 waves walking 23.7 and 23.0 us against
    // 22.8 with 4.
    p.waves = 4;
    p.tile_tokens = 64;
    const int tiles4 = (slices + 3) / 4;
    long want = kCUs / rows;
    if (want < 1) want = 1;
    p.tiles_per_split = (int)((tiles4 + want - 1) / want);
    p.splits = (tiles4 + p.tiles_per_split - 1) / p.tiles_per_split;
    return p;
  }
  p.splits = (tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

// Vector kernel: 4-wave workgroups over 64-token tiles, about 512 of them.
AttnPlan attn_plan_valu(int M, int hkv, int k_blocks) {
  const int max_tokens = k_blocks * kBlockTokens + (kBlockTokens - 1);
  const int max_tiles = (max_tokens + kTileTok - 1) / kTileTok;
  const long target_wg = 512;
  long want = (target_wg + (long)M * hkv - 1) / ((long)M * hkv);
  if (want < 1) want = 1;
  if (want > max_tiles) want = max_tiles;
  AttnPlan p;
  p.tile_tokens = kTileTok;
  p.waves = kThreads / kWave;
  p.tiles_per_split = (max_tiles + (int)want - 1) / (int)want;
  p.splits = (max_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

size_t attn_workspace_bytes(int max_M, int hq, int head_dim, int k_blocks) {
  size_t best = 0;
  const int hkv = hq / kGroup > 0 ? hq / kGroup : 1;
  // partial count M * splits(M) is not monotone in M; take the maximum over
  // both kernels' plans.
  for (int m = 1; m <= max_M; ++m) {
    const AttnPlan pl[2] = {attn_plan(m, hkv, k_blocks), attn_plan_valu(m, hkv, k_blocks)};
    for (const AttnPlan& p : pl) {
      if (p.splits == 1) continue;
      const size_t need = (size_t)m * hq * p.splits * (head_dim + 2) * sizeof(float);
      best = need > best ? need : best;
    }
  }
  return best;
}

hipError_t launch_gathered_attn(const void* q, int dtype, int M, int hq, int hkv, int head_dim,
                                float scale, const int64_t* row_pos, const int32_t* row_seq,
                                const qsa_kv_segments* kv, const int32_t* sel,
                                const int32_t* n_sel, int k_blocks, void* out, float* lse,
                                void* ws, size_t /*ws_bytes*/, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  KvArgs a;
  a.seq_seg_begin = kv->seq_seg_begin;
  a.seg_start = kv->seg_start;
  a.seg_len = kv->seg_len;
  a.seg_cap = kv->seg_cap;
  a.k_seg = kv->k_seg;
  a.v_seg = kv->v_seg;
  a.k_scale = kv->k_scale_seg;
  a.v_scale = kv->v_scale_seg;
  a.n_seq = kv->n_seq;
  a.n_seg_total = kv->n_seg_total;
  if (kv->kv_format == QSA_KV_FP8_E4M3) {  // bf16 queries (validated by the caller)
    if (head_dim == 256)
      return launch_typed<BF16, 256, kKvFp8>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
    return launch_typed<BF16, 128, kKvFp8>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
  }
  if (kv->kv_format == QSA_KV_Q8_0) {  // bf16 queries (validated by the caller)
    if (head_dim == 256)
      return launch_typed<BF16, 256, kKvQ8>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
    return launch_typed<BF16, 128, kKvQ8>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
  }
  if (dtype == QSA_BF16) {
    if (head_dim == 256)
      return launch_typed<BF16, 256>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
    return launch_typed<BF16, 128>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
  }
  // float32 K/V is served at head_dim 128 (validated by the caller)
  return launch_typed<F32, 128>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the split-K partials live in a file-scope device
// array instead of a caller workspace.  Its host-side name is only a stand-in:
// each device's copy has its own address, taken once per device with
// hipGetSymbolAddress (with that device current) and kept here; kernels get
// that address, never the symbol.  Nothing in the array needs a starting
// value (every partial is written before it is read), and every call on one
// device shares that device's copy.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace qsa
