// The index-key append and 4-token pooling of one (token, dimension) pair
// (hipfire "QSA sparse attention ...", section 02: one index key per token;
// every 4 consecutive keys are averaged into a pooled block key), shared by
// the append kernel and the scoring launch that folds the append in.
#pragma once

#include "qsa_device.h"

namespace qsa {

// Writes new token i's key element d to the cache and, when the token
// completes a block (position 4b+3), the block's pooled element d.  The
// block's earlier keys come from this call when they are in it -- a
// sequence's tokens are consecutive in new_idx and in ascending position
// order -- else from the cache, which this call does not write there.
template <class E>
__device__ __forceinline__ void append_token_dim(const typename E::T* __restrict__ new_idx,
                                                 const int64_t* __restrict__ pos, const int32_t* __restrict__ seq,
                                                 typename E::T* __restrict__ cache, float* __restrict__ pooled,
                                                 int n_seq, int64_t capacity, int i, int d) {
  using T = typename E::T;
  const int64_t p = pos[i];
  const int s = seq ? seq[i] : 0;
  if (p < 0 || p >= capacity || s < 0 || s >= n_seq) return;
  const int64_t seq_base = (int64_t)s * capacity;
  const T x = new_idx[(int64_t)i * kIndexDim + d];
  cache[(seq_base + p) * kIndexDim + d] = x;
  if ((p & 3) != 3) return;
  float v[kBlockTokens];
#pragma unroll
  for (int j = 0; j < kBlockTokens; ++j) {
    const int back = kBlockTokens - 1 - j;  // tokens before the completing one
    const int64_t pj = p - back;
    const int ij = i - back;
    bool here = (back == 0);
    if (!here && ij >= 0) here = (pos[ij] == pj) && ((seq ? seq[ij] : 0) == s);
    const T xj = here ? new_idx[(int64_t)ij * kIndexDim + d] : cache[(seq_base + pj) * kIndexDim + d];
    v[j] = E::to_f(xj);
  }
  pooled[((int64_t)s * (capacity / kBlockTokens) + (p >> 2)) * kIndexDim + d] = pool4(v[0], v[1], v[2], v[3]);
}

}  // namespace qsa
