// Host-side launchers of the QSA kernels (internal; the public ABI is qsa.h).
// Each launcher assumes its arguments were validated by qsa_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qsa.h"

namespace qsa {

hipError_t launch_append_pool(const void* new_idx, int dtype, int n_new, const int64_t* pos,
                              const int32_t* seq, void* idx_cache, float* pooled, int n_seq,
                              int64_t capacity, hipStream_t stream);

// With sel_ws non-null the scoring epilogue also builds the per-row key
// histograms the selection consumes (see select.hip).
hipError_t launch_score_blocks(const void* idx_q, int dtype, int M, const int64_t* row_pos,
                               const int32_t* row_seq, const float* pooled, int n_seq,
                               int64_t capacity, int64_t nb_max, float* scores, int64_t ld,
                               uint32_t* sel_ws, hipStream_t stream);

// qsa_append_pool followed by qsa_score_blocks (one sequence) in one launch
// when the few-row kernel scores and at most kMaxFoldedTokens tokens are
// appended; otherwise the two launches.
constexpr int kMaxFoldedTokens = 64;
bool append_folds_into_scoring(int dtype, int M, int n_new, int64_t nb_max);
hipError_t launch_append_score(const void* new_idx, int n_new, const int64_t* new_pos, void* idx_cache,
                               float* pooled, int64_t capacity, const void* idx_q, int dtype, int M,
                               const int64_t* row_pos, int64_t nb_max, float* scores, int64_t ld,
                               uint32_t* sel_ws, hipStream_t stream);

// Many-row scoring (bf16 index queries, one sequence): the bf16 matrix-core
// kernel with three-plane pooled keys (score_prefill.hip).
constexpr int kPrefillMinRows = 64;
// The many-row kernel stores through buffer views of 16 score rows and 16
// selection-workspace rows, each under 2 GiB: false when ld or nb_max is
// too large for them.
bool prefill_views_fit(int64_t nb_max, int64_t ld);
hipError_t launch_score_prefill(const void* idx_q, int M, const int64_t* row_pos, const float* pooled,
                                int64_t nb_max, float* scores, int64_t ld, uint32_t* sel_ws,
                                hipStream_t stream);

// Memory-flat score -> top-k (select_flat.hip; its scoring modes in
// score_prefill.hip).
hipError_t launch_score_prefill_flat(const void* idx_q, int M, const int64_t* row_pos, const float* pooled,
                                     int64_t nb_max, int k_blocks, uint32_t* ws, bool emit, hipStream_t stream);
size_t score_select_workspace_bytes(int max_M, int64_t nb_max, int k_blocks);
hipError_t launch_score_select_flat(const void* idx_q, int M, const int64_t* row_pos, const float* pooled,
                                    int64_t nb_max, int k_blocks, int32_t* sel, int32_t* n_sel, void* ws,
                                    hipStream_t stream);

size_t select_workspace_bytes(int max_M, int64_t nb_max, int k_blocks);
// Standalone selection: histogram, collect and finalize passes.
hipError_t launch_select_topk(const float* scores, int64_t ld, int M, const int64_t* row_pos,
                              int64_t nb_max, int k_blocks, int32_t* sel, int32_t* n_sel,
                              void* ws, size_t ws_bytes, hipStream_t stream);
// Selection after a histogram-building scoring pass: collect and finalize.
hipError_t launch_select_after_hist(const float* scores, int64_t ld, int M, const int64_t* row_pos,
                                   int64_t nb_max, int k_blocks, int32_t* sel, int32_t* n_sel,
                                   void* ws, hipStream_t stream);

// Split plan of the gathered attention for M rows (same on every call with
// the same arguments, so results are reproducible bit for bit).
struct AttnPlan {
  int tile_tokens;     // tokens per inner tile
  int splits;          // split-K parts per (row, KV head)
  int tiles_per_split; // tiles walked by one workgroup
  int waves;           // waves per workgroup
};
// bf16 K/V (matrix-core kernel) and float32 K/V (vector kernel) plans.
AttnPlan attn_plan(int M, int hkv, int k_blocks);
AttnPlan attn_plan_valu(int M, int hkv, int k_blocks);
size_t attn_workspace_bytes(int max_M, int hq, int head_dim, int k_blocks);

// fp8 K/V cache writes (kv_fp8.hip).
hipError_t launch_quantize_kv_fp8(const void* src, int n_head, int n_tok, int head_dim, int64_t src_head_stride,
                                  uint8_t* dst, uint16_t* dst_scale, int64_t dst_head_stride,
                                  hipStream_t stream);

// The allocation-free attention entry point keeps its split-K partials in a
// file-scope device array of this many bytes (attn.hip); noalloc_scratch
// returns the current device's copy of it (its address is looked up once per
// device).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(void** ptr);

// Q8_0 K/V cache writes (kv_q8.hip).
hipError_t launch_quantize_kv_q8(const void* src, int n_head, int n_tok, int head_dim, int64_t src_head_stride,
                                 int8_t* dst, uint16_t* dst_scale, int64_t dst_head_stride, hipStream_t stream);

hipError_t launch_gathered_attn(const void* q, int dtype, int M, int hq, int hkv, int head_dim,
                                float scale, const int64_t* row_pos, const int32_t* row_seq,
                                const qsa_kv_segments* kv, const int32_t* sel,
                                const int32_t* n_sel, int k_blocks, void* out, float* lse,
                                void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace qsa
