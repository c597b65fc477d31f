/*
 * qsa.h -- C ABI of the QSA (Qwen Sparse Attention) per-layer path for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (hipfire page "QSA sparse attention and the VMM KV backend",
 * section 02 "How QSA chooses what to read"): every token of a QSA layer
 * writes one 128-wide index key beside its K/V; each run of 4 consecutive
 * index keys is averaged into one pooled block key; for each query row, 4
 * index-query heads score every causally visible pooled block as the sum of
 * their ReLU'd dot products times 1/sqrt(128); the best-scoring blocks inside
 * a 2,048-token budget (512 blocks) are kept together with the incomplete
 * block at the end; grouped-query attention then reads only those rows.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or synchronises; all work is enqueued on
 *    `stream` (NULL = the null stream) and is safe to capture in a HIP graph.
 *  - Sizes and shapes are host scalars.  Host-side validation runs before any
 *    enqueue: a failed check returns a negative qsa_status, launches nothing
 *    and records a reason readable through qsa_last_error().
 *  - Values that live in device memory (positions, selections, segment
 *    tables) are the caller's contract.  Kernels clamp every index they
 *    derive from them, so a broken contract gives unspecified results but
 *    never an out-of-bounds access.
 *  - A query row at absolute position p sees tokens 0..p (inclusive).  It has
 *    nb(p) = (p+1)/4 complete blocks and a tail of (p+1)%4 tokens.
 *  - Layouts are dense row-major; "[a][b]" means b is contiguous.
 *  - bf16 is IEEE bfloat16 (upper half of a float32), round-to-nearest-even
 *    wherever the library rounds.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type (hipStream_t) without pulling in HIP headers. */
typedef struct ihipStream_t* qsa_stream_t;

#define QSA_INDEX_DIM 128       /* width of an index key and of an index-query head */
#define QSA_INDEX_HEADS 4       /* index-query heads per query row */
#define QSA_BLOCK_TOKENS 4      /* tokens per pooled block */
#define QSA_MAX_K_BLOCKS 1024   /* largest supported budget, in blocks */
#define QSA_MAX_SEGMENTS 16     /* K/V segments per sequence */
#define QSA_SCORE_SELECT_MAX_BLOCKS ((int64_t)1 << 30) /* largest nb_max of qsa_score_select */

typedef enum {
  QSA_OK = 0,
  QSA_ERR_ARG = -1,          /* bad pointer, size or shape */
  QSA_ERR_UNSUPPORTED = -2,  /* valid request this build does not serve */
  QSA_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  QSA_ERR_LAUNCH = -4,       /* the HIP runtime refused a launch */
  QSA_ERR_DEVICE = -5        /* current device is not gfx950 */
} qsa_status;

typedef enum { QSA_F32 = 0, QSA_BF16 = 1 } qsa_dtype;

/* K/V storage formats (qsa_kv_segments.kv_format).  QSA_KV_FP8_E4M3 is the
 * fp8 state of the hipfire page, section 03 ("State formats"): E4M3 K and V
 * (OCP E4M3FN: bias 7, largest finite 448, no infinities) with one f16 scale
 * per KV head and token; a row's values are code * scale.  QSA_KV_Q8_0 is
 * the q8 state of the same table: Q8_0 K and V, int8 codes with one f16
 * scale per 32 consecutive values of a row (34 bytes per 32 values); value
 * = code * the scale of its block. */
#define QSA_KV_SAME 0      /* K/V in the query dtype */
#define QSA_KV_FP8_E4M3 1  /* E4M3 codes + f16 scales; queries bf16 */
#define QSA_KV_Q8_0 2      /* Q8_0: int8 codes + one f16 scale per 32 values; queries bf16 */

/*
 * qsa_append_pool -- write index keys in place and pool completed blocks.
 *
 * Page: hipfire "QSA sparse attention ...", section 02 (one index key per
 * token; every 4 consecutive keys averaged into a pooled block key).  The
 * write is in place and never reallocates (MTPLX PR #482, section 3,
 * optimization 1: the verify's KV write goes in place).
 *
 *  new_idx   [n_new][128] dtype          index keys of the new tokens
 *  dtype     QSA_F32 or QSA_BF16         dtype of new_idx and idx_cache
 *  n_new     >= 0                        tokens appended (0: no-op)
 *  pos       int64 [n_new]               absolute position of each new token
 *  seq       int32 [n_new] or NULL       sequence of each token (NULL: all 0)
 *  idx_cache [n_seq][capacity][128] dtype  per-token index keys (written)
 *  pooled    float32 [n_seq][capacity/4][128]  pooled block keys (written)
 *  n_seq     >= 1; capacity > 0, multiple of 4
 *
 * Every new token's key is copied to idx_cache[seq][pos].  Every block b
 * whose last token 4b+3 is among the new tokens gets
 *   pooled[seq][b] = (((x0 + x1) + x2) + x3) * 0.25
 * in float32 (round-to-nearest-even, no fused multiply-add), x_i being the
 * keys of tokens 4b+i, taken from this call when present, else from
 * idx_cache.  Contract: within one call, the tokens of one sequence are
 * consecutive in new_idx and in ascending position order.  Tokens whose
 * pos or seq is out of range are skipped.
 *
 * Rollback (a speculative verify whose tokens are partly rejected) needs no
 * call and no snapshot: the caller lowers its length.  Rows past the length
 * are never read, and a block's pooled key is rebuilt from its four cached
 * keys whenever its last token is written again, so appending from the
 * trimmed length gives the same bytes as if the rejected tokens had never
 * been written.
 */
int qsa_append_pool(const void* new_idx, int32_t dtype, int32_t n_new,
                    const int64_t* pos, const int32_t* seq,
                    void* idx_cache, float* pooled,
                    int32_t n_seq, int64_t capacity, qsa_stream_t stream);

/*
 * qsa_score_blocks -- score every causally visible pooled block.
 *
 * Page: hipfire "QSA sparse attention ...", section 02 (four index-query
 * heads, sum of ReLU'd dot products, scaled by 1/sqrt(128)) and section 03
 * (a few-row variant for <= 8 rows and a 16-row variant for prefill).
 *
 *  idx_q    [M][4][128] dtype           index queries of the rows, 16-byte
 *                                       aligned
 *  M        >= 0 rows (0: no-op)
 *  row_pos  int64 [M]                    absolute position of each row
 *  row_seq  int32 [M] or NULL            sequence of each row (NULL: all 0;
 *                                        rows then share one read of pooled)
 *  pooled   float32 [n_seq][capacity/4][128]
 *  nb_max   >= 0, <= capacity/4          host bound on nb(row_pos[m])
 *  scores   float32 [M][ld], ld >= nb_max, ld a multiple of 4, 16-byte
 *           aligned (written)
 *
 * scores[m][b] = (sum_h max(0, idx_q[m][h] . pooled[seq][b])) / sqrt(128)
 * for b < min(nb(row_pos[m]), nb_max), accumulated in float32.  Entries past
 * a row's block count are left untouched.
 *
 * 64 or more bf16 rows of one sequence (row_seq NULL) take the many-row
 * kernel, which needs 64 * ld bytes and 64 * (selection-workspace bytes per
 * row, about 8 * nb_max) under 2 GiB; larger shapes give QSA_ERR_UNSUPPORTED.
 *
 *  sel_workspace  NULL, or a qsa_select_topk workspace: the scoring pass then
 *                 also stores the score sample the selection starts from, and
 *                 the following qsa_select_topk on these scores may be called
 *                 with prepared = 1 (it skips its own sampling pass).
 */
int qsa_score_blocks(const void* idx_q, int32_t dtype, int32_t M,
                     const int64_t* row_pos, const int32_t* row_seq,
                     const float* pooled, int32_t n_seq, int64_t capacity,
                     int64_t nb_max, float* scores, int64_t ld,
                     void* sel_workspace, size_t sel_workspace_bytes, qsa_stream_t stream);

/*
 * qsa_append_score -- qsa_append_pool followed by qsa_score_blocks for one
 * sequence, in one launch where possible.
 *
 * Pages: as qsa_append_pool and qsa_score_blocks (hipfire "QSA sparse
 * attention ...", section 02).  One launch instead of two when the few-row
 * scoring kernel serves the rows (fewer than 64 bf16 rows, or float32) and
 * 1..64 tokens are appended: one workgroup writes the new keys and pools the
 * blocks they complete, and the scoring of such a block pools it in
 * registers from the same keys.  Otherwise the two launches.  Results are
 * bit-identical to the two calls.
 *
 *  new_idx, n_new, new_pos   as qsa_append_pool's new_idx, n_new, pos (seq NULL)
 *  idx_cache, pooled         [capacity][128] dtype, float32 [capacity/4][128]
 *  capacity                  > 0, multiple of 4
 *  idx_q, dtype, M, row_pos  as qsa_score_blocks (row_seq NULL, n_seq 1)
 *  nb_max, scores, ld        as qsa_score_blocks
 *  sel_workspace, ..._bytes  as qsa_score_blocks
 * Errors: those of either call.
 */
int qsa_append_score(const void* new_idx, int32_t n_new, const int64_t* new_pos, void* idx_cache,
                     float* pooled, int64_t capacity, const void* idx_q, int32_t dtype, int32_t M,
                     const int64_t* row_pos, int64_t nb_max, float* scores, int64_t ld,
                     void* sel_workspace, size_t sel_workspace_bytes, qsa_stream_t stream);

/*
 * qsa_select_topk -- keep the best blocks of each row within the budget.
 *
 * Page: hipfire "QSA sparse attention ...", section 02 (top-scoring blocks
 * within a 2,048-token budget, 512 blocks; the incomplete tail block is kept
 * in addition) and section 03 (a radix select follows the scoring).
 *
 *  scores    float32 [M][ld]            as written by qsa_score_blocks (same
 *                                       ld and alignment rules)
 *  row_pos   int64 [M]; nb_max as for qsa_score_blocks
 *  k_blocks  1..QSA_MAX_K_BLOCKS        budget in blocks (512 = 2,048 tokens)
 *  sel       int32 [M][k_blocks]        kept block ids, ascending; unused
 *                                       entries are set to -1 (written)
 *  n_sel     int32 [M]                  min(k_blocks, nb) (written)
 *  workspace / workspace_bytes          >= qsa_select_workspace_bytes(...);
 *                                       needs no initialisation.  Calls
 *                                       sharing a workspace must not overlap
 *                                       in time.
 *  prepared  0, or 1 when qsa_score_blocks stored the sample of these
 *            scores into this workspace (same M, row_pos and nb_max)
 *
 * When nb <= k_blocks every block is kept.  Otherwise the k_blocks largest
 * scores are kept; equal scores go to the lower block index.  The tail
 * tokens 4*nb..p are not listed; every attention call adds them.  Scores are
 * compared as float32 with -0 equal to +0.
 */
int qsa_select_topk(const float* scores, int64_t ld, int32_t M,
                    const int64_t* row_pos, int64_t nb_max, int32_t k_blocks,
                    int32_t* sel, int32_t* n_sel,
                    void* workspace, size_t workspace_bytes, int32_t prepared,
                    qsa_stream_t stream);

/* K/V of a batch of sequences, each held as 1..QSA_MAX_SEGMENTS segments.
 * Segments follow MTPLX PR #610 ("How it works": one immutable segment per
 * finished turn plus a growing tail; attention reads all segments in one
 * launch).  Every array below is DEVICE memory owned by the caller; the
 * struct itself is read on the host during the call only. */
typedef struct qsa_kv_segments {
  int32_t n_seq;                /* sequences described (>= 1) */
  int32_t n_seg_total;          /* segments over all sequences (>= n_seq) */
  int32_t max_seg_per_seq;      /* host bound, 1..QSA_MAX_SEGMENTS */
  int32_t kv_format;            /* QSA_KV_SAME or QSA_KV_FP8_E4M3 */
  const int32_t* seq_seg_begin; /* int32 [n_seq+1]: sequence s owns segments
                                   seq_seg_begin[s] .. seq_seg_begin[s+1]-1 */
  const int64_t* seg_start;     /* int64 [n_seg_total]: first logical token held */
  const int64_t* seg_len;       /* int64 [n_seg_total]: tokens held */
  const int64_t* seg_cap;       /* int64 [n_seg_total]: token stride between KV heads */
  const void* const* k_seg;     /* [n_seg_total] -> K [hkv][seg_cap][head_dim] dtype
                                   (QSA_KV_FP8_E4M3: uint8 codes) */
  const void* const* v_seg;     /* [n_seg_total] -> V, same layout */
  const uint16_t* const* k_scale_seg; /* QSA_KV_FP8_E4M3: [n_seg_total] -> f16 bits
                                   [hkv][seg_cap], the scale of each K row;
                                   QSA_KV_Q8_0: -> f16 bits [hkv][seg_cap][head_dim/32],
                                   the scale of each 32-value block; else NULL */
  const uint16_t* const* v_scale_seg; /* the same for V */
} qsa_kv_segments;

/*
 * qsa_gathered_attn -- grouped-query attention over the kept rows only.
 *
 * Pages: hipfire "QSA sparse attention ...", section 02 (full attention over
 * the selected rows plus the tail, at most 2,048 + 3 tokens per query) and
 * section 03 (one workgroup per KV group of query heads reads each selected
 * K/V row once for the whole group; gathered prefill tiles on matrix
 * cores); MTPLX PR #610 ("What changes": partials merged by log-sum-exp in
 * float32, rounded once; rows with no visible key give zeros, not NaN).
 *
 *  q          [M][hq][head_dim] dtype   query rows, 16-byte aligned
 *  M >= 0; hq, hkv with hq % hkv == 0 and hq/hkv == 12; head_dim 128 or 256
 *  scale      softmax scale (finite), usually 1/sqrt(head_dim)
 *  row_pos    int64 [M]; row_seq int32 [M] or NULL (all sequence 0)
 *  kv         K/V segment table of the sequences
 *  sel/n_sel  as written by qsa_select_topk; k_blocks its budget
 *  out        [M][hq][head_dim] dtype   (written; 16-byte aligned)
 *  lse        float32 [M][hq]           natural-log sum of exp of the
 *                                       scaled logits; -inf for a row with no
 *                                       visible token (written)
 *  workspace / workspace_bytes          >= qsa_attn_workspace_bytes(...),
 *                                       16-byte aligned
 *
 * Row m reads tokens 4b..4b+3 of every kept block b plus its tail tokens
 * 4*nb..p; query head h uses KV head h / (hq/hkv).  Logits, softmax and
 * partial outputs are float32; the output is rounded once to dtype.
 *
 * With kv->kv_format == QSA_KV_FP8_E4M3 (dtype QSA_BF16 only) K and V are
 * E4M3 codes with f16 row scales (see qsa_quantize_kv_fp8): a logit is
 * scale_k(t) * (q . code_k(t)) * scale, and token t's softmax weight is
 * multiplied by scale_v(t) before it meets V's codes (rounded to bf16 as the
 * weights of the bf16 path are).  With QSA_KV_Q8_0 (dtype QSA_BF16 only) K
 * and V are Q8_0 (see qsa_quantize_kv_q8_0): a logit is the sum over the
 * row's 32-value blocks j of scale_k(t, j) * (q_j . code_k(t)_j), times
 * scale; V values are code * scale_v(t, j) rounded to bf16 before P.V.
 */
int qsa_gathered_attn(const void* q, int32_t dtype, int32_t M, int32_t hq, int32_t hkv,
                      int32_t head_dim, float scale,
                      const int64_t* row_pos, const int32_t* row_seq,
                      const qsa_kv_segments* kv,
                      const int32_t* sel, const int32_t* n_sel, int32_t k_blocks,
                      void* out, float* lse,
                      void* workspace, size_t workspace_bytes, qsa_stream_t stream);

/*
 * qsa_gathered_attn_noalloc -- qsa_gathered_attn without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, results and errors are those of qsa_gathered_attn (same kernels,
 * same split plan, bit-identical outputs).  The split-K partials live in a
 * static device array of 16 MiB that the library holds on each device it runs
 * on until the process ends; its address is looked up on the first call on a
 * device.  Calls whose partials would need more (qsa_attn_workspace_bytes(M,
 * hq, head_dim, k_blocks) > 16 MiB) return QSA_ERR_UNSUPPORTED and launch
 * nothing; every shape this build serves needs at most 12.1 MiB (the split
 * plans keep at most 1,024 partial workgroups of 12 heads).  Nothing is
 * allocated or freed.  Every call on one device shares that device's array:
 * calls that overlap in time on one device (different streams, or host
 * threads) race and must be serialised by the caller.
 */
int qsa_gathered_attn_noalloc(const void* q, int32_t dtype, int32_t M, int32_t hq, int32_t hkv,
                              int32_t head_dim, float scale,
                              const int64_t* row_pos, const int32_t* row_seq,
                              const qsa_kv_segments* kv,
                              const int32_t* sel, const int32_t* n_sel, int32_t k_blocks,
                              void* out, float* lse, qsa_stream_t stream);

/*
 * qsa_score_select -- scores and top-k selection of many rows of one
 * sequence without a score matrix (memory-flat prefill).
 *
 * Pages: hipfire "QSA sparse attention ...", section 02 (score and keep the
 * best blocks within the budget, ties to the lower index) and section 06
 * (long score rows outgrow the selector's on-chip memory); the chunked-
 * prefill page, section 1 (the [rows x context] score buffer is a prefill
 * chunk's memory peak).  Same result as qsa_score_blocks followed by
 * qsa_select_topk on the many-row path, without writing the M x nb_max
 * scores: a sampled threshold per row, candidates above it appended during
 * scoring, an exact selection among them.
 *
 *  idx_q     bf16 [M][4][128]            index queries (one sequence), 16-byte
 *                                        aligned
 *  M >= 0; row_pos int64 [M]; pooled float32 [nb_max][128] (the sequence's
 *  pooled keys, e.g. the first sequence of qsa_append_pool's buffer)
 *  nb_max    >= max blocks of any row (a host bound), at most
 *            QSA_SCORE_SELECT_MAX_BLOCKS (2^30 blocks: block ids are held in
 *            32-bit signed lanes)
 *  k_blocks  1..QSA_MAX_K_BLOCKS
 *  sel       int32 [M][k_blocks], ascending block ids, -1 padded (written)
 *  n_sel     int32 [M] = min(k_blocks, nb) (written)
 *  workspace / workspace_bytes  >= qsa_score_select_workspace_bytes(M, nb_max,
 *            k_blocks), 16-byte aligned; needs no initialisation.  For each
 *            row m, 32-bit word 2 * round64(M) + m (round64: up to a multiple
 *            of 64) tells how the row was selected (a diagnostic): 1 all
 *            blocks kept, 2 from the candidates, 3/4/5 by an exact whole-row
 *            select over scores recomputed in float32 (row longer than
 *            262,144 blocks; candidate count outside [k, 4096]; more than 512
 *            keys equal to the k-th).
 *
 * The scores are the many-row kernel's (bf16 matrix cores, float32 pooled
 * keys as three bf16 planes); rows that take the exact path use float32
 * vector arithmetic instead, so their scores may differ in the last bits.
 * Workspace: about 4 B per 16 blocks plus 32 KiB per row, against 4 B per
 * block per row for the score matrix.
 */
int qsa_score_select(const void* idx_q, int32_t M, const int64_t* row_pos, const float* pooled,
                     int64_t nb_max, int32_t k_blocks, int32_t* sel, int32_t* n_sel,
                     void* workspace, size_t workspace_bytes, qsa_stream_t stream);
size_t qsa_score_select_workspace_bytes(int32_t max_M, int64_t nb_max, int32_t k_blocks);

/*
 * qsa_quantize_kv_fp8 -- write K or V rows into an fp8 (E4M3 + f16 scale)
 * cache.
 *
 * Page: hipfire "QSA sparse attention ...", section 03, "State formats"
 * (fp8 state: E4M3 K/V with an f16 scale per head and token, index keys
 * staying bf16).  The page gives the format only; the rule here:
 *   scale = f16(amax / 448), amax the row's largest magnitude, the quotient
 *   in float32 and rounded to nearest even (an f16 overflow clamps to
 *   65504); code = E4M3 value nearest to the float32 quotient x / scale,
 *   ties to the even code, magnitudes above 448 saturating to 448, the sign
 *   bit copied from x; a row whose scale rounds to zero gets zero codes.
 *
 *  src       bf16 rows: row (h, t) at src + (h * src_head_stride + t) * head_dim
 *  n_head, n_tok >= 0   rows written: n_head * n_tok
 *  head_dim  128 or 256
 *  dst       uint8 codes: row (h, t) at dst + (h * dst_head_stride + t) * head_dim
 *  dst_scale f16 bits: scale of row (h, t) at dst_scale[h * dst_head_stride + t]
 *  src_head_stride >= n_tok, dst_head_stride >= n_tok (in rows)
 * src and dst 16-byte aligned, dst_scale 2-byte aligned; the caller owns
 * every buffer.  Typical use: the new tokens' K of one layer, [hkv][T][D],
 * written at token t0 of a segment [hkv][cap][D]: dst = seg + t0 * head_dim,
 * dst_scale = seg_scale + t0, dst_head_stride = cap.  In place, nothing
 * allocated.  NaN or infinite inputs give undefined codes.
 */
int qsa_quantize_kv_fp8(const void* src, int32_t n_head, int32_t n_tok, int32_t head_dim,
                        int64_t src_head_stride, void* dst, uint16_t* dst_scale,
                        int64_t dst_head_stride, qsa_stream_t stream);

/*
 * qsa_quantize_kv_q8_0 -- write K or V rows into a Q8_0 cache (int8 codes,
 * one f16 scale per 32 consecutive values of a row).
 *
 * Page: hipfire "QSA sparse attention ...", section 03, "State formats" (the
 * opt-in q8 state: Q8_0 K/V with bf16 index keys, 1,408 bytes per token and
 * layer).  The page names the format only; the rule here, per 32-value
 * block of a row:
 *   scale = f16(amax / 127), amax the block's largest magnitude, the quotient
 *   in float32 and rounded to nearest even (an f16 overflow clamps to
 *   65504); code = the integer nearest to the float32 quotient x / scale,
 *   ties to even, clamped to [-127, 127]; a block whose scale rounds to zero
 *   gets zero codes.
 *
 *  src       bf16 rows: row (h, t) at src + (h * src_head_stride + t) * head_dim
 *  n_head, n_tok >= 0   rows written: n_head * n_tok
 *  head_dim  128 or 256
 *  dst       int8 codes: row (h, t) at dst + (h * dst_head_stride + t) * head_dim
 *  dst_scale f16 bits: block j of row (h, t) at
 *            dst_scale[(h * dst_head_stride + t) * (head_dim / 32) + j]
 *  src_head_stride >= n_tok, dst_head_stride >= n_tok (in rows)
 * src and dst 16-byte aligned, dst_scale 2-byte aligned; the caller owns
 * every buffer.  In place, nothing allocated.  NaN or infinite inputs give
 * undefined codes.  The attention reads a Q8_0 segment's scale rows with
 * 16-byte (head_dim 256) or 8-byte (head_dim 128) loads: a segment's scale
 * buffer must start 16-byte aligned.
 */
int qsa_quantize_kv_q8_0(const void* src, int32_t n_head, int32_t n_tok, int32_t head_dim,
                         int64_t src_head_stride, void* dst, uint16_t* dst_scale,
                         int64_t dst_head_stride, qsa_stream_t stream);

/* Workspace bytes qsa_select_topk needs for up to max_M rows of up to
 * nb_max blocks (0 means no workspace is needed).  The workspace is one
 * record per row, of qsa_select_workspace_bytes(1, nb_max, k_blocks) bytes;
 * after a selection, 32-bit word 0 of row m's record tells how row m was
 * selected (a diagnostic; every path gives the same exact result): 1 all
 * blocks kept, 2 from the conservative candidates, 3 or 4 by the exact
 * whole-row select (more than 64 chunks of 4,096 blocks; a candidate count
 * below k_blocks or above 4,096). */
size_t qsa_select_workspace_bytes(int32_t max_M, int64_t nb_max, int32_t k_blocks);

/* Workspace bytes qsa_gathered_attn needs for up to max_M rows (split-K
 * partials).  Reserve it once at load; it never grows (hipfire page,
 * section 03: scratch reserved at load never grows under a captured graph). */
size_t qsa_attn_workspace_bytes(int32_t max_M, int32_t hq, int32_t head_dim, int32_t k_blocks);

/* The split plan qsa_gathered_attn uses for M rows (host-only query, no
 * device work; the plan depends only on these arguments, so results are
 * reproducible bit for bit).  Page: hipfire "QSA sparse attention ...",
 * section 03 (one workgroup per KV group; gathered prefill tiles).
 *  plan  int32 [4] (host memory, written): waves per workgroup, tokens per
 *        tile, tiles walked by one workgroup, split-K parts per (row, KV head)
 * Errors: QSA_ERR_ARG for M < 1, hkv < 1, k_blocks outside
 * [1, QSA_MAX_K_BLOCKS], an unknown dtype or a NULL plan. */
int qsa_attn_plan(int32_t M, int32_t hkv, int32_t k_blocks, int32_t dtype, int32_t* plan);

/* Checks that the current HIP device is gfx950 and that the kernels load.
 * QSA_OK, or QSA_ERR_DEVICE with a reason. */
int qsa_device_check(void);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char* qsa_last_error(void);

/* Library version string. */
const char* qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
