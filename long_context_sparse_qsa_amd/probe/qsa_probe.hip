// Measurement kernels (libqsa_probe.so): the memory patterns of the QSA
// path's kernels with the arithmetic taken out.  Built beside libqsa.so,
// loaded only by the benchmark; the QSA library does not depend on them.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "qsa_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunkBytes = 2048;
constexpr int kGatherPer = 512;  // chunks per gather workgroup
constexpr int kInFlight = 16;    // gather loads per lane in flight
constexpr float kNever = 1234.5f;

thread_local char g_err[256];

int fail(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return -1;
}

int launched(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_err, sizeof(g_err), "%s: launch failed: %s", fn, hipGetErrorString(e));
    return -4;
  }
  g_err[0] = 0;
  return 0;
}

// Workgroup w reads bytes [w * wg_bytes, (w + 1) * wg_bytes): PER loads of
// 16 bytes per lane, all issued before the first use.
template <int PER>
__global__ void __launch_bounds__(kThreads) read_kernel(const uint4* __restrict__ buf, float* sink) {
  const uint4* b = buf + (int64_t)blockIdx.x * PER * kThreads + threadIdx.x;
  uint4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) v[u] = b[u * kThreads];
  uint32_t x = 0u;
#pragma unroll
  for (int u = 0; u < PER; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (__uint_as_float(x) == kNever) sink[0] = 1.f;
}

// Workgroup w reads chunks chunk_id[512 w .. 512 w + 511]: the ids go to LDS
// first, then 2 chunks per 256 lanes and pass, 16 passes in flight.
__global__ void __launch_bounds__(kThreads) gather_kernel(const uint4* __restrict__ buf, int64_t n_chunks_buf,
                                                         const int32_t* __restrict__ chunk_id, float* sink) {
  __shared__ int32_t ids[kGatherPer];
  const int32_t* src = chunk_id + (int64_t)blockIdx.x * kGatherPer;
  for (int i = threadIdx.x; i < kGatherPer; i += kThreads) {
    const int32_t c = src[i];
    ids[i] = c < 0 ? 0 : (c >= n_chunks_buf ? (int32_t)(n_chunks_buf - 1) : c);
  }
  __syncthreads();
  constexpr int kU4 = kChunkBytes / 16;  // 128 uint4 per chunk
  const int half = threadIdx.x / kU4;    // which of the pass's 2 chunks
  const int e = threadIdx.x % kU4;
  uint32_t x = 0u;
  for (int c0 = 0; c0 < kGatherPer; c0 += 2 * kInFlight) {
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = buf[(int64_t)ids[c0 + 2 * u + half] * kU4 + e];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) x ^= v[u].x ^ v[u].w;
  }
  if (__uint_as_float(x) == kNever) sink[0] = 1.f;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

int qsa_probe_read(const void* buf, int64_t bytes, int32_t wg_bytes, float* sink, qsa_stream_t stream) {
  if (!buf || !sink) return fail("qsa_probe_read: null pointer");
  if ((uintptr_t)buf & 15u) return fail("qsa_probe_read: buf must be 16-byte aligned");
  if (wg_bytes < 16384 || wg_bytes > 65536 || wg_bytes % 4096)
    return fail("qsa_probe_read: wg_bytes %d not a multiple of 4 KiB in [16 KiB, 64 KiB]", wg_bytes);
  if (bytes <= 0 || bytes % wg_bytes)
    return fail("qsa_probe_read: bytes %lld not a positive multiple of wg_bytes", (long long)bytes);
  const dim3 grid((unsigned)(bytes / wg_bytes));
  const uint4* b = static_cast<const uint4*>(buf);
  hipStream_t s = (hipStream_t)stream;
  switch (wg_bytes / 4096) {
    case 4: hipLaunchKernelGGL(read_kernel<4>, grid, dim3(kThreads), 0, s, b, sink); break;
    case 8: hipLaunchKernelGGL(read_kernel<8>, grid, dim3(kThreads), 0, s, b, sink); break;
    case 16: hipLaunchKernelGGL(read_kernel<16>, grid, dim3(kThreads), 0, s, b, sink); break;
    default: return fail("qsa_probe_read: wg_bytes %d: 16, 32 or 64 KiB", wg_bytes);
  }
  return launched("qsa_probe_read");
}

int qsa_probe_gather(const void* buf, int64_t buf_bytes, const int32_t* chunk_id, int64_t n_chunk, float* sink,
                     qsa_stream_t stream) {
  if (!buf || !chunk_id || !sink) return fail("qsa_probe_gather: null pointer");
  if ((uintptr_t)buf & 15u) return fail("qsa_probe_gather: buf must be 16-byte aligned");
  if (buf_bytes < kChunkBytes) return fail("qsa_probe_gather: buf_bytes %lld below one chunk", (long long)buf_bytes);
  if (n_chunk <= 0 || n_chunk % kGatherPer)
    return fail("qsa_probe_gather: n_chunk %lld not a positive multiple of %d", (long long)n_chunk, kGatherPer);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(n_chunk / kGatherPer)), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(buf), buf_bytes / kChunkBytes, chunk_id, sink);
  return launched("qsa_probe_gather");
}

int qsa_probe_empty(int32_t workgroups, qsa_stream_t stream) {
  if (workgroups < 1 || workgroups > 65535) return fail("qsa_probe_empty: workgroups %d outside [1, 65535]", workgroups);
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)workgroups), dim3(64), 0, (hipStream_t)stream);
  return launched("qsa_probe_empty");
}

const char* qsa_probe_last_error(void) { return g_err; }

}  // extern "C"
