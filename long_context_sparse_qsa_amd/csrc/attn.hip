// Gathered grouped-query attention over the kept rows (hipfire "QSA sparse
// attention ...", section 02: attention reads only the selected rows plus the
// incomplete tail; section 03: one workgroup per KV group of 12 query heads
// reads each selected K/V row once for the whole group) and the log-sum-exp
// merge of split partials (MTPLX PR #610, "What changes": float32 partials,
// merged by log-sum-exp, rounded once; rows with no visible key give zeros).
//
// Decode / verify kernel: one workgroup (4 waves) per (row, KV head, split).
// A split walks 64-token tiles of the row's token list (kept blocks in
// ascending order, then the tail).  Per tile:
//   1. 64 lanes resolve their token to a K/V row through the sequence's
//      segment table (segments may cut a 4-token block anywhere);
//   2. the K and V rows (512 B each at head_dim 256, bf16) are staged into
//      LDS with 16-byte loads, once for all 12 query heads;
//   3. QK: wave w handles heads 3w..3w+2, lane = token; the query row is
//      wave-uniform (scalar registers) and bf16 pairs go through the packed
//      dot2 instruction with float32 accumulation;
//   4. online softmax (base-2 exponentials of logits pre-scaled by log2 e);
//   5. PV: lane = (dim group, 6 heads), probabilities broadcast from LDS.
// Split partials (normalised output + lse) go to the workspace and a second
// kernel merges them; with a single split the output is written directly.
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

struct KvArgs {
  const int32_t* seq_seg_begin;
  const int64_t* seg_start;
  const int64_t* seg_len;
  const int64_t* seg_cap;
  const void* const* k_seg;
  const void* const* v_seg;
  int n_seq;
  int n_seg_total;
};

// Element-type specific pieces of the tile loop.
template <class E, int D>
struct Tile {
  using T = typename E::T;
  static constexpr int kRowBytes = D * E::kBytes;
  static constexpr int kChunks = kRowBytes / 16;       // 16-byte chunks per row
  static constexpr int kKStride = kRowBytes + 16;      // padded K row in LDS
  static constexpr int kElemsPerChunk = 16 / E::kBytes;
  static constexpr int kDimsPerThread = D / (kThreads / kHeadHalves);  // PV dims per lane
};

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
  __shared__ __align__(16) unsigned char k_lds[kTileTok * TT::kKStride];
  __shared__ __align__(16) unsigned char v_lds[kTileTok * TT::kRowBytes];
  __shared__ __align__(16) float p_lds[kTileTok][kGroup];
  __shared__ float alpha_lds[kGroup];
  __shared__ float m_lds[kGroup], l_lds[kGroup];
  __shared__ const unsigned char* krow[kTileTok];
  __shared__ const unsigned char* vrow[kTileTok];
  __shared__ int64_t seg_lo[kMaxSegments], seg_hi[kMaxSegments], seg_cap[kMaxSegments];
  __shared__ const unsigned char* seg_k[kMaxSegments];
  __shared__ const unsigned char* seg_v[kMaxSegments];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int m = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid / kWave);

  // Row geometry.
  const int64_t p = row_pos[m];
  const int64_t n_vis = p + 1 > 0 ? p + 1 : 0;
  const int64_t nb = n_vis / kBlockTokens;
  const int tail = (int)(n_vis - nb * kBlockTokens);
  int ns = n_sel[m];
  ns = ns < 0 ? 0 : ns;
  ns = ns > k_blocks ? k_blocks : ns;
  ns = (int64_t)ns > nb ? (int)nb : ns;
  const int total = ns * kBlockTokens + tail;

  // Segment table of this row's sequence.
  int sq = row_seq ? row_seq[m] : 0;
  const bool seq_ok = sq >= 0 && sq < kv.n_seq;
  sq = seq_ok ? sq : 0;
  int s_begin = kv.seq_seg_begin[sq], s_end = kv.seq_seg_begin[sq + 1];
  s_begin = s_begin < 0 ? 0 : s_begin;
  s_end = s_end > kv.n_seg_total ? kv.n_seg_total : s_end;
  const int nseg = (seq_ok && s_end > s_begin) ? min(s_end - s_begin, kMaxSegments) : 0;
  if (tid < nseg) {
    const int si = s_begin + tid;
    const int64_t st = kv.seg_start[si];
    seg_lo[tid] = st;
    seg_hi[tid] = st + kv.seg_len[si];
    seg_cap[tid] = kv.seg_cap[si];
    seg_k[tid] = static_cast<const unsigned char*>(kv.k_seg[si]);
    seg_v[tid] = static_cast<const unsigned char*>(kv.v_seg[si]);
  }

  // Running softmax state of this wave's QK heads (identical in all lanes).
  float m_run[kHeadsPerWaveQK], l_run[kHeadsPerWaveQK];
#pragma unroll
  for (int hh = 0; hh < kHeadsPerWaveQK; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
  }
  // PV accumulators: lane owns dims [dg*DPT, dg*DPT+DPT) of heads half*6..half*6+5.
  constexpr int DPT = TT::kDimsPerThread;
  const int dg = tid % (kThreads / kHeadHalves);
  const int half = tid / (kThreads / kHeadHalves);
  float acc[kHeadsPV][DPT];
#pragma unroll
  for (int h = 0; h < kHeadsPV; ++h)
#pragma unroll
    for (int d = 0; d < DPT; ++d) acc[h][d] = 0.f;

  const T* __restrict__ qrow = q + ((int64_t)m * hq + (int64_t)g * kGroup) * D;
  const int32_t* __restrict__ srow = sel + (int64_t)m * k_blocks;
  __syncthreads();

  const int tok_begin = split * tiles_per_split * kTileTok;
  for (int t = 0; t < tiles_per_split; ++t) {
    const int j0 = tok_begin + t * kTileTok;
    if (j0 >= total) break;

    // 1. resolve tokens
    if (tid < kTileTok) {
      const int j = j0 + tid;
      const unsigned char* kr = nullptr;
      const unsigned char* vr = nullptr;
      if (j < total) {
        int64_t tok = -1;
        if (j < ns * kBlockTokens) {
          const int64_t b = srow[j >> 2];
          if (b >= 0 && b < nb) tok = b * kBlockTokens + (j & 3);
        } else {
          tok = nb * kBlockTokens + (j - ns * kBlockTokens);
        }
        if (tok >= 0) {
          for (int si = 0; si < nseg; ++si) {
            if (tok >= seg_lo[si] && tok < seg_hi[si] && tok - seg_lo[si] < seg_cap[si]) {
              const int64_t off = ((int64_t)g * seg_cap[si] + (tok - seg_lo[si])) * TT::kRowBytes;
              kr = seg_k[si] + off;
              vr = seg_v[si] + off;
              break;
            }
          }
        }
      }
      krow[tid] = kr;
      vrow[tid] = vr;
    }
    __syncthreads();

    // 2. stage K and V rows (zeros for missing rows)
    for (int idx = tid; idx < kTileTok * TT::kChunks; idx += kThreads) {
      const int r = idx / TT::kChunks;
      const int c = idx % TT::kChunks;
      const unsigned char* kr = krow[r];
      const unsigned char* vr = vrow[r];
      uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
      if (kr) {
        kv4 = *reinterpret_cast<const uint4*>(kr + c * 16);
        vv4 = *reinterpret_cast<const uint4*>(vr + c * 16);
      }
      *reinterpret_cast<uint4*>(k_lds + r * TT::kKStride + c * 16) = kv4;
      *reinterpret_cast<uint4*>(v_lds + r * TT::kRowBytes + c * 16) = vv4;
    }
    __syncthreads();

    // 3. QK for heads 3w..3w+2, lane = token
    float sc[kHeadsPerWaveQK];
#pragma unroll
    for (int hh = 0; hh < kHeadsPerWaveQK; ++hh) sc[hh] = 0.f;
    const unsigned char* kl = k_lds + lane * TT::kKStride;
    const T* __restrict__ qw = qrow + (wave * kHeadsPerWaveQK) * D;
#pragma unroll 4
    for (int c = 0; c < TT::kChunks; ++c) {
      const uint4 kk = *reinterpret_cast<const uint4*>(kl + c * 16);
#pragma unroll
      for (int hh = 0; hh < kHeadsPerWaveQK; ++hh) {
        const T* qc = qw + hh * D + c * TT::kElemsPerChunk;
        if constexpr (E::kBytes == 2) {
          const uint32_t* q32 = reinterpret_cast<const uint32_t*>(qc);
          float a = sc[hh];
          a = dot2_bf16(q32[0], kk.x, a);
          a = dot2_bf16(q32[1], kk.y, a);
          a = dot2_bf16(q32[2], kk.z, a);
          a = dot2_bf16(q32[3], kk.w, a);
          sc[hh] = a;
        } else {
          float a = sc[hh];
          a = fmaf(qc[0], __uint_as_float(kk.x), a);
          a = fmaf(qc[1], __uint_as_float(kk.y), a);
          a = fmaf(qc[2], __uint_as_float(kk.z), a);
          a = fmaf(qc[3], __uint_as_float(kk.w), a);
          sc[hh] = a;
        }
      }
    }
    const bool valid = krow[lane] != nullptr;

    // 4. online softmax
#pragma unroll
    for (int hh = 0; hh < kHeadsPerWaveQK; ++hh) {
      const float s2 = valid ? sc[hh] * scale_log2 : -INFINITY;
      const float tmax = wave_max(s2);
      const float m_new = fmaxf(m_run[hh], tmax);
      const float alpha = (m_run[hh] == m_new) ? 1.f : exp2f(m_run[hh] - m_new);
      const float pv = (s2 == -INFINITY) ? 0.f : exp2f(s2 - m_new);
      l_run[hh] = l_run[hh] * alpha + wave_sum(pv);
      m_run[hh] = m_new;
      const int h = wave * kHeadsPerWaveQK + hh;
      p_lds[lane][h] = pv;
      if (lane == 0) alpha_lds[h] = alpha;
    }
    __syncthreads();

    // 5. PV
#pragma unroll
    for (int h = 0; h < kHeadsPV; ++h) {
      const float a = alpha_lds[half * kHeadsPV + h];
#pragma unroll
      for (int d = 0; d < DPT; ++d) acc[h][d] *= a;
    }
    const int rows = min(kTileTok, total - j0);
    for (int r = 0; r < rows; ++r) {
      float vv[DPT];
      const unsigned char* vp = v_lds + r * TT::kRowBytes + dg * DPT * E::kBytes;
      if constexpr (E::kBytes == 2) {
        if constexpr (DPT == 2) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(vp);
          vv[0] = __uint_as_float(w << 16);
          vv[1] = __uint_as_float(w & 0xffff0000u);
        } else {
          vv[0] = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(vp));
        }
      } else {
#pragma unroll
        for (int d = 0; d < DPT; ++d) vv[d] = reinterpret_cast<const float*>(vp)[d];
      }
      const float* pr = &p_lds[r][half * kHeadsPV];
#pragma unroll
      for (int h = 0; h < kHeadsPV; ++h) {
        const float w = pr[h];
#pragma unroll
        for (int d = 0; d < DPT; ++d) acc[h][d] = fmaf(w, vv[d], acc[h][d]);
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
      if (dg == 0) ws_lse[head * splits + split] = lse;
    }
  }
}

// Merge split partials by log-sum-exp.  One workgroup per (row, head).
template <class E, int D>
__global__ void __launch_bounds__(D)
attn_combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse, int splits,
                    typename E::T* __restrict__ out, float* __restrict__ lse_out) {
  extern __shared__ float w_lds[];  // [splits]
  __shared__ float red[D / kWave];
  __shared__ float mx_sh, tot_sh;
  const int64_t head = blockIdx.x;
  const int tid = threadIdx.x;
  const float* L = ws_lse + head * splits;
  float mx = -INFINITY;
  for (int i = tid; i < splits; i += D) {
    const float v = L[i];
    w_lds[i] = v;
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = mx;
  __syncthreads();
  if (tid == 0) {
    float a = red[0];
    for (int i = 1; i < D / kWave; ++i) a = fmaxf(a, red[i]);
    mx_sh = a;
  }
  __syncthreads();
  mx = mx_sh;
  const bool empty = (mx == -INFINITY);
  float tot = 0.f;
  for (int i = tid; i < splits; i += D) {
    const float w = (empty || w_lds[i] == -INFINITY) ? 0.f : expf(w_lds[i] - mx);
    w_lds[i] = w;
    tot += w;
  }
  tot = wave_sum(tot);
  __syncthreads();
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = tot;
  __syncthreads();
  if (tid == 0) {
    float a = 0.f;
    for (int i = 0; i < D / kWave; ++i) a += red[i];
    tot_sh = a;
  }
  __syncthreads();
  tot = tot_sh;
  float o = 0.f;
  const float* O = ws_o + head * splits * D + tid;
  for (int i = 0; i < splits; ++i) {
    const float w = w_lds[i];
    if (w != 0.f) o = fmaf(w, O[(int64_t)i * D], o);
  }
  o = (empty || tot == 0.f) ? 0.f : o / tot;
  out[head * D + tid] = E::from_f(o);
  if (tid == 0) lse_out[head] = empty ? -INFINITY : mx + logf(tot);
}

template <class E, int D>
hipError_t launch_typed(const void* q, int M, int hq, int hkv, float scale,
                        const int64_t* row_pos, const int32_t* row_seq, const KvArgs& kv,
                        const int32_t* sel, const int32_t* n_sel, int k_blocks, void* out,
                        float* lse, void* ws, hipStream_t stream) {
  const AttnPlan plan = attn_plan(M, hkv, k_blocks);
  float* ws_o = static_cast<float*>(ws);
  float* ws_lse = ws_o ? ws_o + (size_t)M * hq * plan.splits * D : nullptr;
  dim3 grid(plan.splits, hkv, M), block(kThreads);
  hipLaunchKernelGGL((attn_decode_kernel<E, D>), grid, block, 0, stream,
                     static_cast<const typename E::T*>(q), M, hq, scale * kLog2e, row_pos, row_seq,
                     kv, sel, n_sel, k_blocks, plan.tiles_per_split, plan.splits,
                     static_cast<typename E::T*>(out), lse, ws_o, ws_lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  hipLaunchKernelGGL((attn_combine_kernel<E, D>), dim3((unsigned)M * hq), dim3(D),
                     plan.splits * sizeof(float), stream, ws_o, ws_lse, plan.splits,
                     static_cast<typename E::T*>(out), lse);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int M, int hkv, int k_blocks) {
  const int max_tokens = k_blocks * kBlockTokens + (kBlockTokens - 1);
  const int max_tiles = (max_tokens + kTileTok - 1) / kTileTok;
  const long target_wg = 512;
  long want = (target_wg + (long)M * hkv - 1) / ((long)M * hkv);
  if (want < 1) want = 1;
  if (want > max_tiles) want = max_tiles;
  AttnPlan p;
  p.tile_tokens = kTileTok;
  p.tiles_per_split = (max_tiles + (int)want - 1) / (int)want;
  p.splits = (max_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

size_t attn_workspace_bytes(int max_M, int hq, int head_dim, int k_blocks) {
  size_t best = 0;
  // partial count M * splits(M) is not monotone in M; take the maximum.
  for (int m = 1; m <= max_M; ++m) {
    const AttnPlan p = attn_plan(m, hq / kGroup > 0 ? hq / kGroup : 1, k_blocks);
    if (p.splits == 1) continue;
    const size_t need = (size_t)m * hq * p.splits * (head_dim + 1) * sizeof(float);
    best = need > best ? need : best;
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
  a.n_seq = kv->n_seq;
  a.n_seg_total = kv->n_seg_total;
  if (dtype == QSA_BF16) {
    if (head_dim == 256)
      return launch_typed<BF16, 256>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
    return launch_typed<BF16, 128>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
  }
  if (head_dim == 256)
    return launch_typed<F32, 256>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
  return launch_typed<F32, 128>(q, M, hq, hkv, scale, row_pos, row_seq, a, sel, n_sel, k_blocks, out, lse, ws, stream);
}

}  // namespace qsa
