/*
 * qsa_probe.h -- measurement kernels beside the QSA library (libqsa_probe.so).
 *
 * Not part of the QSA path: these kernels move bytes in the access patterns
 * the path's kernels use, with no arithmetic, so that a benchmark can state
 * what the memory system delivers for each pattern on this chip.  They back
 * the bounds quoted for the scoring pass (one launch that streams the
 * pooled keys once), the gathered attention (4-token K/V rows at random
 * selected blocks) and the kernel boundaries of a layer step (an empty
 * launch inside a HIP graph).
 *
 * Conventions as in qsa.h: device pointers owned by the caller, host-side
 * validation first (a negative status, nothing launched, a reason in
 * qsa_probe_last_error()), all work on `stream`.
 */
#ifndef QSA_PROBE_H_
#define QSA_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* qsa_stream_t;

/* Contiguous read of `bytes` (a multiple of wg_bytes; buf 16-byte aligned) in
 * one launch: each workgroup of 256 lanes issues all of its loads at once
 * (16 bytes per lane and load), `wg_bytes` per workgroup (16, 32 or 64
 * KiB).  The loaded words are folded into a value that is stored to sink[0]
 * only if it equals an impossible constant, so the loads cannot be removed;
 * sink must hold one float. */
int qsa_probe_read(const void* buf, int64_t bytes, int32_t wg_bytes, float* sink, qsa_stream_t stream);

/* Gather of n_chunk chunks of 2,048 bytes (a block of 4 bf16 K or V rows at
 * head_dim 256): chunk i is read from buf + 2048 * chunk_id[i].  Ids are
 * device values; the kernel clamps each into [0, buf_bytes / 2048), so any
 * id reads inside buf.  512 chunks per workgroup (ids staged in LDS first,
 * then 16 loads of 16 bytes in flight per lane); n_chunk must be a multiple
 * of 512, buf 16-byte aligned and at least 2,048 bytes.  sink as above. */
int qsa_probe_gather(const void* buf, int64_t buf_bytes, const int32_t* chunk_id, int64_t n_chunk, float* sink,
                     qsa_stream_t stream);

/* An empty kernel of `workgroups` workgroups of 64 lanes (1 .. 65,535): the
 * cost of one more launch in a graph of dependent launches. */
int qsa_probe_empty(int32_t workgroups, qsa_stream_t stream);

const char* qsa_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_PROBE_H_ */
