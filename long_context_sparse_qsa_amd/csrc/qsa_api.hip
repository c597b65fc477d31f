// C ABI of the QSA layer path: host-side validation, reason strings and
// dispatch to the kernels.  Nothing here allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "qsa_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return QSA_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QSA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

bool dtype_ok(int32_t dt) { return dt == QSA_F32 || dt == QSA_BF16; }

}  // namespace

extern "C" {

int qsa_append_pool(const void* new_idx, int32_t dtype, int32_t n_new, const int64_t* pos,
                    const int32_t* seq, void* idx_cache, float* pooled, int32_t n_seq,
                    int64_t capacity, qsa_stream_t stream) {
  if (!dtype_ok(dtype)) return fail(QSA_ERR_ARG, "qsa_append_pool: dtype %d is not QSA_F32 or QSA_BF16", dtype);
  if (n_new < 0) return fail(QSA_ERR_ARG, "qsa_append_pool: n_new = %d < 0", n_new);
  if (n_seq < 1) return fail(QSA_ERR_ARG, "qsa_append_pool: n_seq = %d < 1", n_seq);
  if (capacity <= 0 || capacity % QSA_BLOCK_TOKENS != 0)
    return fail(QSA_ERR_ARG, "qsa_append_pool: capacity %lld must be a positive multiple of 4",
                (long long)capacity);
  if (n_new == 0) return ok();
  if (!new_idx || !pos || !idx_cache || !pooled)
    return fail(QSA_ERR_ARG, "qsa_append_pool: null pointer (new_idx, pos, idx_cache or pooled)");
  return launch_status(qsa::launch_append_pool(new_idx, dtype, n_new, pos, seq, idx_cache, pooled,
                                               n_seq, capacity, (hipStream_t)stream),
                       "qsa_append_pool");
}

int qsa_score_blocks(const void* idx_q, int32_t dtype, int32_t M, const int64_t* row_pos,
                     const int32_t* row_seq, const float* pooled, int32_t n_seq, int64_t capacity,
                     int64_t nb_max, float* scores, int64_t ld, void* sel_workspace,
                     size_t sel_workspace_bytes, qsa_stream_t stream) {
  if (!dtype_ok(dtype)) return fail(QSA_ERR_ARG, "qsa_score_blocks: dtype %d is not QSA_F32 or QSA_BF16", dtype);
  if (M < 0) return fail(QSA_ERR_ARG, "qsa_score_blocks: M = %d < 0", M);
  if (n_seq < 1) return fail(QSA_ERR_ARG, "qsa_score_blocks: n_seq = %d < 1", n_seq);
  if (capacity <= 0 || capacity % QSA_BLOCK_TOKENS != 0)
    return fail(QSA_ERR_ARG, "qsa_score_blocks: capacity %lld must be a positive multiple of 4",
                (long long)capacity);
  if (nb_max < 0 || nb_max > capacity / QSA_BLOCK_TOKENS)
    return fail(QSA_ERR_ARG, "qsa_score_blocks: nb_max %lld outside [0, capacity/4 = %lld]",
                (long long)nb_max, (long long)(capacity / QSA_BLOCK_TOKENS));
  if (ld < nb_max) return fail(QSA_ERR_ARG, "qsa_score_blocks: ld %lld < nb_max %lld", (long long)ld, (long long)nb_max);
  if (ld % 4 != 0 || ((uintptr_t)scores & 15u) != 0)
    return fail(QSA_ERR_ARG, "qsa_score_blocks: scores must be 16-byte aligned with ld a multiple of 4 (ld %lld)",
                (long long)ld);
  if (dtype == QSA_BF16 && M >= qsa::kPrefillMinRows && row_seq == nullptr && !qsa::prefill_views_fit(nb_max, ld))
    return fail(QSA_ERR_UNSUPPORTED,
                "qsa_score_blocks: %d bf16 rows with ld %lld, nb_max %lld: the many-row kernel needs 64 * ld and 64 * "
                "(selection-workspace words per row) under 2 GiB",
                M, (long long)ld, (long long)nb_max);
  if (sel_workspace && sel_workspace_bytes < qsa::select_workspace_bytes(M, nb_max, 1))
    return fail(QSA_ERR_WORKSPACE, "qsa_score_blocks: selection workspace %zu B < %zu B needed",
                sel_workspace_bytes, qsa::select_workspace_bytes(M, nb_max, 1));
  if (M == 0 || nb_max == 0) return ok();
  if (!idx_q || !row_pos || !pooled || !scores)
    return fail(QSA_ERR_ARG, "qsa_score_blocks: null pointer (idx_q, row_pos, pooled or scores)");
  if ((uintptr_t)idx_q & 15u) return fail(QSA_ERR_ARG, "qsa_score_blocks: idx_q must be 16-byte aligned");
  return launch_status(qsa::launch_score_blocks(idx_q, dtype, M, row_pos, row_seq, pooled, n_seq,
                                                capacity, nb_max, scores, ld,
                                                static_cast<uint32_t*>(sel_workspace), (hipStream_t)stream),
                       "qsa_score_blocks");
}

int qsa_append_score(const void* new_idx, int32_t n_new, const int64_t* new_pos, void* idx_cache,
                     float* pooled, int64_t capacity, const void* idx_q, int32_t dtype, int32_t M,
                     const int64_t* row_pos, int64_t nb_max, float* scores, int64_t ld,
                     void* sel_workspace, size_t sel_workspace_bytes, qsa_stream_t stream) {
  if (!dtype_ok(dtype)) return fail(QSA_ERR_ARG, "qsa_append_score: dtype %d is not QSA_F32 or QSA_BF16", dtype);
  if (n_new < 0) return fail(QSA_ERR_ARG, "qsa_append_score: n_new = %d < 0", n_new);
  if (M < 0) return fail(QSA_ERR_ARG, "qsa_append_score: M = %d < 0", M);
  if (capacity <= 0 || capacity % QSA_BLOCK_TOKENS != 0)
    return fail(QSA_ERR_ARG, "qsa_append_score: capacity %lld must be a positive multiple of 4", (long long)capacity);
  if (nb_max < 0 || nb_max > capacity / QSA_BLOCK_TOKENS)
    return fail(QSA_ERR_ARG, "qsa_append_score: nb_max %lld outside [0, capacity/4 = %lld]", (long long)nb_max,
                (long long)(capacity / QSA_BLOCK_TOKENS));
  if (ld < nb_max) return fail(QSA_ERR_ARG, "qsa_append_score: ld %lld < nb_max %lld", (long long)ld, (long long)nb_max);
  if (ld % 4 != 0 || ((uintptr_t)scores & 15u) != 0)
    return fail(QSA_ERR_ARG, "qsa_append_score: scores must be 16-byte aligned with ld a multiple of 4 (ld %lld)",
                (long long)ld);
  if (dtype == QSA_BF16 && M >= qsa::kPrefillMinRows && !qsa::prefill_views_fit(nb_max, ld))
    return fail(QSA_ERR_UNSUPPORTED,
                "qsa_append_score: %d bf16 rows with ld %lld, nb_max %lld: the many-row kernel needs 64 * ld and 64 * "
                "(selection-workspace words per row) under 2 GiB",
                M, (long long)ld, (long long)nb_max);
  if (sel_workspace && sel_workspace_bytes < qsa::select_workspace_bytes(M, nb_max, 1))
    return fail(QSA_ERR_WORKSPACE, "qsa_append_score: selection workspace %zu B < %zu B needed",
                sel_workspace_bytes, qsa::select_workspace_bytes(M, nb_max, 1));
  if (n_new > 0 && (!new_idx || !new_pos || !idx_cache || !pooled))
    return fail(QSA_ERR_ARG, "qsa_append_score: null pointer (new_idx, new_pos, idx_cache or pooled)");
  if (M > 0 && nb_max > 0 && (!idx_q || !row_pos || !pooled || !scores))
    return fail(QSA_ERR_ARG, "qsa_append_score: null pointer (idx_q, row_pos, pooled or scores)");
  if ((uintptr_t)idx_q & 15u) return fail(QSA_ERR_ARG, "qsa_append_score: idx_q must be 16-byte aligned");
  return launch_status(qsa::launch_append_score(new_idx, n_new, new_pos, idx_cache, pooled, capacity, idx_q, dtype,
                                                M, row_pos, nb_max, scores, ld,
                                                static_cast<uint32_t*>(sel_workspace), (hipStream_t)stream),
                       "qsa_append_score");
}

size_t qsa_select_workspace_bytes(int32_t max_M, int64_t nb_max, int32_t k_blocks) {
  if (max_M <= 0 || nb_max < 0 || k_blocks <= 0) return 0;
  return qsa::select_workspace_bytes(max_M, nb_max, k_blocks);
}

int qsa_select_topk(const float* scores, int64_t ld, int32_t M, const int64_t* row_pos,
                    int64_t nb_max, int32_t k_blocks, int32_t* sel, int32_t* n_sel,
                    void* workspace, size_t workspace_bytes, int32_t prepared, qsa_stream_t stream) {
  if (M < 0) return fail(QSA_ERR_ARG, "qsa_select_topk: M = %d < 0", M);
  if (k_blocks < 1 || k_blocks > QSA_MAX_K_BLOCKS)
    return fail(QSA_ERR_ARG, "qsa_select_topk: k_blocks %d outside [1, %d]", k_blocks, QSA_MAX_K_BLOCKS);
  if (nb_max < 0) return fail(QSA_ERR_ARG, "qsa_select_topk: nb_max %lld < 0", (long long)nb_max);
  if (ld < nb_max) return fail(QSA_ERR_ARG, "qsa_select_topk: ld %lld < nb_max %lld", (long long)ld, (long long)nb_max);
  if (ld % 4 != 0 || ((uintptr_t)scores & 15u) != 0)
    return fail(QSA_ERR_ARG, "qsa_select_topk: scores must be 16-byte aligned with ld a multiple of 4 (ld %lld)",
                (long long)ld);
  const size_t need = qsa::select_workspace_bytes(M, nb_max, k_blocks);
  if (workspace_bytes < need || (need && !workspace))
    return fail(QSA_ERR_WORKSPACE, "qsa_select_topk: workspace %zu B < %zu B needed", workspace_bytes, need);
  if (M == 0) return ok();
  if (!row_pos || !sel || !n_sel || (nb_max > 0 && !scores))
    return fail(QSA_ERR_ARG, "qsa_select_topk: null pointer (scores, row_pos, sel or n_sel)");
  if (prepared != 0 && prepared != 1) return fail(QSA_ERR_ARG, "qsa_select_topk: prepared = %d is not 0 or 1", prepared);
  if (prepared)
    return launch_status(qsa::launch_select_after_hist(scores, ld, M, row_pos, nb_max, k_blocks, sel, n_sel,
                                                       workspace, (hipStream_t)stream),
                         "qsa_select_topk");
  return launch_status(qsa::launch_select_topk(scores, ld, M, row_pos, nb_max, k_blocks, sel, n_sel,
                                               workspace, workspace_bytes, (hipStream_t)stream),
                       "qsa_select_topk");
}

size_t qsa_attn_workspace_bytes(int32_t max_M, int32_t hq, int32_t head_dim, int32_t k_blocks) {
  if (max_M <= 0 || hq <= 0 || head_dim <= 0 || k_blocks <= 0 || k_blocks > QSA_MAX_K_BLOCKS) return 0;
  return qsa::attn_workspace_bytes(max_M, hq, head_dim, k_blocks);
}

int qsa_attn_plan(int32_t M, int32_t hkv, int32_t k_blocks, int32_t dtype, int32_t* plan) {
  if (M < 1 || hkv < 1) return fail(QSA_ERR_ARG, "qsa_attn_plan: M %d and hkv %d must be >= 1", M, hkv);
  if (k_blocks < 1 || k_blocks > QSA_MAX_K_BLOCKS)
    return fail(QSA_ERR_ARG, "qsa_attn_plan: k_blocks %d outside [1, %d]", k_blocks, QSA_MAX_K_BLOCKS);
  if (!dtype_ok(dtype)) return fail(QSA_ERR_ARG, "qsa_attn_plan: dtype %d is not QSA_F32 or QSA_BF16", dtype);
  if (!plan) return fail(QSA_ERR_ARG, "qsa_attn_plan: plan is NULL");
  const qsa::AttnPlan p = dtype == QSA_BF16 ? qsa::attn_plan(M, hkv, k_blocks) : qsa::attn_plan_valu(M, hkv, k_blocks);
  plan[0] = p.waves;
  plan[1] = p.tile_tokens;
  plan[2] = p.tiles_per_split;
  plan[3] = p.splits;
  return ok();
}

}  // extern "C"

namespace {

// Checks shared by qsa_gathered_attn and its allocation-free variant; the
// workspace is checked by each caller.
int check_attn_args(const char* fn, const void* q, int32_t dtype, int32_t M, int32_t hq, int32_t hkv,
                    int32_t head_dim, float scale, const int64_t* row_pos, const qsa_kv_segments* kv,
                    const int32_t* sel, const int32_t* n_sel, int32_t k_blocks, void* out, float* lse) {
  if (!dtype_ok(dtype)) return fail(QSA_ERR_ARG, "%s: dtype %d is not QSA_F32 or QSA_BF16", fn, dtype);
  if (M < 0) return fail(QSA_ERR_ARG, "%s: M = %d < 0", fn, M);
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
    return fail(QSA_ERR_ARG, "%s: hq %d must be a positive multiple of hkv %d", fn, hq, hkv);
  if (hq / hkv != 12)
    return fail(QSA_ERR_UNSUPPORTED, "%s: %d query heads per KV head; this build serves 12", fn, hq / hkv);
  if (head_dim != 128 && head_dim != 256)
    return fail(QSA_ERR_UNSUPPORTED, "%s: head_dim %d; this build serves 128 and 256", fn, head_dim);
  if (dtype == QSA_F32 && head_dim != 128)
    return fail(QSA_ERR_UNSUPPORTED, "%s: float32 K/V is served at head_dim 128 only", fn);
  if (!(scale == scale) || isinf(scale)) return fail(QSA_ERR_ARG, "%s: scale is not finite", fn);
  if (k_blocks < 1 || k_blocks > QSA_MAX_K_BLOCKS)
    return fail(QSA_ERR_ARG, "%s: k_blocks %d outside [1, %d]", fn, k_blocks, QSA_MAX_K_BLOCKS);
  if (!kv) return fail(QSA_ERR_ARG, "%s: kv is NULL", fn);
  if (kv->n_seq < 1 || kv->n_seg_total < kv->n_seq)
    return fail(QSA_ERR_ARG, "%s: kv n_seq %d / n_seg_total %d invalid", fn, kv->n_seq, kv->n_seg_total);
  if (kv->max_seg_per_seq < 1 || kv->max_seg_per_seq > QSA_MAX_SEGMENTS)
    return fail(QSA_ERR_UNSUPPORTED, "%s: max_seg_per_seq %d outside [1, %d]", fn, kv->max_seg_per_seq,
                QSA_MAX_SEGMENTS);
  if (!kv->seq_seg_begin || !kv->seg_start || !kv->seg_len || !kv->seg_cap || !kv->k_seg || !kv->v_seg)
    return fail(QSA_ERR_ARG, "%s: null pointer in the kv segment table", fn);
  if (kv->kv_format != QSA_KV_SAME && kv->kv_format != QSA_KV_FP8_E4M3 && kv->kv_format != QSA_KV_Q8_0)
    return fail(QSA_ERR_ARG, "%s: kv_format %d is not QSA_KV_SAME, QSA_KV_FP8_E4M3 or QSA_KV_Q8_0", fn,
                kv->kv_format);
  if (kv->kv_format != QSA_KV_SAME) {
    const char* what = kv->kv_format == QSA_KV_FP8_E4M3 ? "fp8" : "Q8_0";
    if (dtype != QSA_BF16) return fail(QSA_ERR_UNSUPPORTED, "%s: %s K/V is served with bf16 queries only", fn, what);
    if (!kv->k_scale_seg || !kv->v_scale_seg)
      return fail(QSA_ERR_ARG, "%s: %s K/V needs k_scale_seg and v_scale_seg", fn, what);
  }
  if (M > 0 && (!q || !row_pos || !sel || !n_sel || !out || !lse))
    return fail(QSA_ERR_ARG, "%s: null pointer (q, row_pos, sel, n_sel, out or lse)", fn);
  if (M > 0 && ((uintptr_t)out & 15u))
    return fail(QSA_ERR_ARG, "%s: out must be 16-byte aligned", fn);
  if (M > 0 && ((uintptr_t)q & 15u))
    return fail(QSA_ERR_ARG, "%s: q must be 16-byte aligned", fn);
  return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_gathered_attn(const void* q, int32_t dtype, int32_t M, int32_t hq, int32_t hkv,
                      int32_t head_dim, float scale, const int64_t* row_pos,
                      const int32_t* row_seq, const qsa_kv_segments* kv, const int32_t* sel,
                      const int32_t* n_sel, int32_t k_blocks, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, qsa_stream_t stream) {
  const char* fn = "qsa_gathered_attn";
  int r = check_attn_args(fn, q, dtype, M, hq, hkv, head_dim, scale, row_pos, kv, sel, n_sel, k_blocks, out, lse);
  if (r != QSA_OK) return r;
  const size_t need = qsa::attn_workspace_bytes(M, hq, head_dim, k_blocks);
  if (M > 0 && (workspace_bytes < need || (need && !workspace)))
    return fail(QSA_ERR_WORKSPACE, "%s: workspace %zu B < %zu B needed", fn, workspace_bytes, need);
  if (M == 0) return ok();
  if ((uintptr_t)workspace & 15u) return fail(QSA_ERR_ARG, "%s: out and workspace must be 16-byte aligned", fn);
  return launch_status(qsa::launch_gathered_attn(q, dtype, M, hq, hkv, head_dim, scale, row_pos, row_seq, kv, sel,
                                                 n_sel, k_blocks, out, lse, workspace, workspace_bytes,
                                                 (hipStream_t)stream),
                       fn);
}

int qsa_gathered_attn_noalloc(const void* q, int32_t dtype, int32_t M, int32_t hq, int32_t hkv,
                              int32_t head_dim, float scale, const int64_t* row_pos, const int32_t* row_seq,
                              const qsa_kv_segments* kv, const int32_t* sel, const int32_t* n_sel,
                              int32_t k_blocks, void* out, float* lse, qsa_stream_t stream) {
  const char* fn = "qsa_gathered_attn_noalloc";
  int r = check_attn_args(fn, q, dtype, M, hq, hkv, head_dim, scale, row_pos, kv, sel, n_sel, k_blocks, out, lse);
  if (r != QSA_OK) return r;
  if (M == 0) return ok();
  const size_t need = qsa::attn_workspace_bytes(M, hq, head_dim, k_blocks);
  if (need > qsa::kNoAllocScratchBytes)
    return fail(QSA_ERR_UNSUPPORTED,
                "%s: %d rows x %d heads at head_dim %d, budget %d blocks need %zu B of split partials, above the "
                "%zu B static scratch",
                fn, M, hq, head_dim, k_blocks, need, qsa::kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = qsa::noalloc_scratch(&ws);
    if (e != hipSuccess) return fail(QSA_ERR_LAUNCH, "%s: static scratch address: %s", fn, hipGetErrorString(e));
  }
  return launch_status(qsa::launch_gathered_attn(q, dtype, M, hq, hkv, head_dim, scale, row_pos, row_seq, kv, sel,
                                                 n_sel, k_blocks, out, lse, ws, need, (hipStream_t)stream),
                       fn);
}

int qsa_score_select(const void* idx_q, int32_t M, const int64_t* row_pos, const float* pooled,
                     int64_t nb_max, int32_t k_blocks, int32_t* sel, int32_t* n_sel,
                     void* workspace, size_t workspace_bytes, qsa_stream_t stream) {
  if (M < 0) return fail(QSA_ERR_ARG, "qsa_score_select: M = %d < 0", M);
  if (nb_max < 0 || nb_max > QSA_SCORE_SELECT_MAX_BLOCKS)
    return fail(QSA_ERR_ARG, "qsa_score_select: nb_max %lld outside [0, %lld]", (long long)nb_max,
                (long long)QSA_SCORE_SELECT_MAX_BLOCKS);
  if (k_blocks < 1 || k_blocks > QSA_MAX_K_BLOCKS)
    return fail(QSA_ERR_ARG, "qsa_score_select: k_blocks %d outside [1, %d]", k_blocks, QSA_MAX_K_BLOCKS);
  const size_t need = qsa::score_select_workspace_bytes(M, nb_max, k_blocks);
  if (M > 0 && (workspace_bytes < need || !workspace))
    return fail(QSA_ERR_WORKSPACE, "qsa_score_select: workspace %zu B < %zu B needed", workspace_bytes, need);
  if (M == 0) return ok();
  if (((uintptr_t)workspace & 15u) != 0) return fail(QSA_ERR_ARG, "qsa_score_select: workspace must be 16-byte aligned");
  if (!idx_q || !row_pos || !sel || !n_sel || (nb_max > 0 && !pooled))
    return fail(QSA_ERR_ARG, "qsa_score_select: null pointer (idx_q, row_pos, pooled, sel or n_sel)");
  if ((uintptr_t)idx_q & 15u) return fail(QSA_ERR_ARG, "qsa_score_select: idx_q must be 16-byte aligned");
  return launch_status(qsa::launch_score_select_flat(idx_q, M, row_pos, pooled, nb_max, k_blocks, sel, n_sel,
                                                     workspace, (hipStream_t)stream),
                       "qsa_score_select");
}

size_t qsa_score_select_workspace_bytes(int32_t max_M, int64_t nb_max, int32_t k_blocks) {
  if (max_M <= 0 || nb_max < 0) return 0;
  return qsa::score_select_workspace_bytes(max_M, nb_max, k_blocks);
}

int qsa_quantize_kv_fp8(const void* src, int32_t n_head, int32_t n_tok, int32_t head_dim,
                        int64_t src_head_stride, void* dst, uint16_t* dst_scale,
                        int64_t dst_head_stride, qsa_stream_t stream) {
  if (n_head < 0 || n_tok < 0)
    return fail(QSA_ERR_ARG, "qsa_quantize_kv_fp8: n_head %d / n_tok %d < 0", n_head, n_tok);
  if (head_dim != 128 && head_dim != 256)
    return fail(QSA_ERR_UNSUPPORTED, "qsa_quantize_kv_fp8: head_dim %d; this build serves 128 and 256", head_dim);
  if (src_head_stride < n_tok || dst_head_stride < n_tok)
    return fail(QSA_ERR_ARG, "qsa_quantize_kv_fp8: head strides %lld / %lld below n_tok %d",
                (long long)src_head_stride, (long long)dst_head_stride, n_tok);
  if ((int64_t)n_head * n_tok == 0) return ok();
  if (!src || !dst || !dst_scale) return fail(QSA_ERR_ARG, "qsa_quantize_kv_fp8: null pointer (src, dst or dst_scale)");
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u) || ((uintptr_t)dst_scale & 1u))
    return fail(QSA_ERR_ARG, "qsa_quantize_kv_fp8: src and dst must be 16-byte aligned, dst_scale 2-byte aligned");
  return launch_status(qsa::launch_quantize_kv_fp8(src, n_head, n_tok, head_dim, src_head_stride,
                                                   static_cast<uint8_t*>(dst), dst_scale, dst_head_stride,
                                                   (hipStream_t)stream),
                       "qsa_quantize_kv_fp8");
}

int qsa_quantize_kv_q8_0(const void* src, int32_t n_head, int32_t n_tok, int32_t head_dim,
                         int64_t src_head_stride, void* dst, uint16_t* dst_scale,
                         int64_t dst_head_stride, qsa_stream_t stream) {
  if (n_head < 0 || n_tok < 0)
    return fail(QSA_ERR_ARG, "qsa_quantize_kv_q8_0: n_head %d / n_tok %d < 0", n_head, n_tok);
  if (head_dim != 128 && head_dim != 256)
    return fail(QSA_ERR_UNSUPPORTED, "qsa_quantize_kv_q8_0: head_dim %d; this build serves 128 and 256", head_dim);
  if (src_head_stride < n_tok || dst_head_stride < n_tok)
    return fail(QSA_ERR_ARG, "qsa_quantize_kv_q8_0: head strides %lld / %lld below n_tok %d",
                (long long)src_head_stride, (long long)dst_head_stride, n_tok);
  if ((int64_t)n_head * n_tok == 0) return ok();
  if (!src || !dst || !dst_scale) return fail(QSA_ERR_ARG, "qsa_quantize_kv_q8_0: null pointer (src, dst or dst_scale)");
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u) || ((uintptr_t)dst_scale & 1u))
    return fail(QSA_ERR_ARG, "qsa_quantize_kv_q8_0: src and dst must be 16-byte aligned, dst_scale 2-byte aligned");
  return launch_status(qsa::launch_quantize_kv_q8(src, n_head, n_tok, head_dim, src_head_stride,
                                                  static_cast<int8_t*>(dst), dst_scale, dst_head_stride,
                                                  (hipStream_t)stream),
                       "qsa_quantize_kv_q8_0");
}

int qsa_device_check(void) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QSA_ERR_DEVICE, "qsa_device_check: no HIP device: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess)
    return fail(QSA_ERR_DEVICE, "qsa_device_check: hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(QSA_ERR_DEVICE, "qsa_device_check: device %d is %s; this library is built for gfx950",
                dev, prop.gcnArchName);
  return ok();
}

const char* qsa_last_error(void) { return g_err; }

const char* qsa_version(void) { return "qsa-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
