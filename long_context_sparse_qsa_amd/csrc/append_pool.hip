// Index-key append and 4-token pooling (hipfire "QSA sparse attention ...",
// section 02: one 128-wide index key per token; every 4 consecutive keys are
// averaged into one pooled block key).  The write is in place (MTPLX PR #482,
// section 3, optimization 1).
//
// One workgroup of 128 lanes per new token, one lane per index dimension:
// a row of 128 keys is 256 B (bf16) or 512 B (fp32), written coalesced.  The
// token that completes a block (position 4b+3) also pools it; the three
// earlier keys come from this call when they are in it (the caller lists a
// sequence's tokens consecutively in ascending order), else from the cache,
// so no workgroup reads a row another workgroup of this launch writes.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "append_common.h"

namespace qsa {

template <class E>
__global__ void __launch_bounds__(kIndexDim)
append_pool_kernel(const typename E::T* __restrict__ new_idx, int n_new,
                   const int64_t* __restrict__ pos, const int32_t* __restrict__ seq,
                   typename E::T* __restrict__ cache, float* __restrict__ pooled,
                   int n_seq, int64_t capacity) {
  append_token_dim<E>(new_idx, pos, seq, cache, pooled, n_seq, capacity, blockIdx.x, threadIdx.x);
}

hipError_t launch_append_pool(const void* new_idx, int dtype, int n_new, const int64_t* pos,
                              const int32_t* seq, void* idx_cache, float* pooled, int n_seq,
                              int64_t capacity, hipStream_t stream) {
  if (n_new == 0) return hipSuccess;
  dim3 grid(n_new), block(kIndexDim);
  if (dtype == QSA_BF16) {
    hipLaunchKernelGGL(append_pool_kernel<BF16>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(new_idx), n_new, pos, seq,
                       static_cast<uint16_t*>(idx_cache), pooled, n_seq, capacity);
  } else {
    hipLaunchKernelGGL(append_pool_kernel<F32>, grid, block, 0, stream,
                       static_cast<const float*>(new_idx), n_new, pos, seq,
                       static_cast<float*>(idx_cache), pooled, n_seq, capacity);
  }
  return hipGetLastError();
}

}  // namespace qsa
