// Q8_0 K/V cache writes (hipfire "QSA sparse attention ...", section 03,
// "State formats": the opt-in q8 state keeps K and V as Q8_0 -- blocks of 32
// signed 8-bit integers with one f16 scale, 34 bytes per 32 values -- and
// the index keys in bf16).
//
// One wave per (head, token) row: each lane holds head_dim / 64 consecutive
// elements, so a 32-value block is 8 lanes (head_dim 256) or 16 lanes
// (head_dim 128) and its largest magnitude comes from a reduction over
// them.  The block's scale is f16(amax / 127) and every element becomes the
// integer nearest to x / scale (ties to even), clamped to [-127, 127].
// Bytes moved per row: 2 D read, D + D / 16 written.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kRowsPerWG = 4;
constexpr int kQ8Block = 32;
constexpr float kQ8Max = 127.f;
constexpr uint16_t kF16MaxBits = 0x7bffu;  // 65504

template <int D>
__global__ void __launch_bounds__(kWave * kRowsPerWG)
quantize_kv_q8_kernel(const uint16_t* __restrict__ src, int n_head, int n_tok, int64_t src_hs,
                      int8_t* __restrict__ dst, uint16_t* __restrict__ dst_scale, int64_t dst_hs) {
  constexpr int PER = D / kWave;             // 4 (D = 256) or 2 (D = 128) elements per lane
  constexpr int LANES = kQ8Block / PER;      // lanes per 32-value block
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWG + threadIdx.x / kWave;
  if (row >= (int64_t)n_head * n_tok) return;  // wave-uniform
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t h = row / n_tok;
  const int64_t t = row - h * n_tok;
  const uint16_t* s = src + (h * src_hs + t) * D + PER * lane;
  float x[PER];
  if constexpr (PER == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(s);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(s);
    x[0] = __uint_as_float(w << 16);
    x[1] = __uint_as_float(w & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) amax = fmaxf(amax, fabsf(x[i]));
  // over the block's lanes through DPP moves: after the quad steps the
  // half-row mirror joins the two quads of 8 lanes and the row mirror the two
  // halves of 16 (a max needs no particular pairing)
  static_assert(LANES == 8 || LANES == 16, "a 32-value block is 8 or 16 lanes");
  amax = dpp_max_step<0xB1, 0xF>(amax);
  amax = dpp_max_step<0x4E, 0xF>(amax);
  amax = dpp_max_step<0x141, 0xF>(amax);
  if constexpr (LANES == 16) amax = dpp_max_step<0x140, 0xF>(amax);
  const _Float16 s16 = (_Float16)(amax / kQ8Max);  // float32 quotient, round to nearest even
  uint16_t sbits = __builtin_bit_cast(uint16_t, s16);
  if ((sbits & 0x7fffu) == 0x7c00u) sbits = kF16MaxBits;  // f16 overflow clamps to 65504
  const float sf = (float)__builtin_bit_cast(_Float16, sbits);
  uint32_t packed = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    float c = sf > 0.f ? __builtin_rintf(x[i] / sf) : 0.f;  // nearest integer, ties to even
    c = fminf(fmaxf(c, -kQ8Max), kQ8Max);
    packed |= ((uint32_t)(int32_t)c & 0xffu) << (8 * i);
  }
  int8_t* d = dst + (h * dst_hs + t) * D + PER * lane;
  if constexpr (PER == 4) {
    *reinterpret_cast<uint32_t*>(d) = packed;
  } else {
    *reinterpret_cast<uint16_t*>(d) = (uint16_t)packed;
  }
  if (lane % LANES == 0) dst_scale[(h * dst_hs + t) * (D / kQ8Block) + lane / LANES] = sbits;
}

}  // namespace

hipError_t launch_quantize_kv_q8(const void* src, int n_head, int n_tok, int head_dim, int64_t src_head_stride,
                                 int8_t* dst, uint16_t* dst_scale, int64_t dst_head_stride, hipStream_t stream) {
  const int64_t rows = (int64_t)n_head * n_tok;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + kRowsPerWG - 1) / kRowsPerWG));
  const uint16_t* s = static_cast<const uint16_t*>(src);
  if (head_dim == 256)
    hipLaunchKernelGGL(quantize_kv_q8_kernel<256>, grid, dim3(kWave * kRowsPerWG), 0, stream, s, n_head, n_tok,
                       src_head_stride, dst, dst_scale, dst_head_stride);
  else
    hipLaunchKernelGGL(quantize_kv_q8_kernel<128>, grid, dim3(kWave * kRowsPerWG), 0, stream, s, n_head, n_tok,
                       src_head_stride, dst, dst_scale, dst_head_stride);
  return hipGetLastError();
}

}  // namespace qsa
