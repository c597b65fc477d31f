// fp8 K/V cache writes (hipfire "QSA sparse attention ...", section 03,
// "State formats": the fp8 state keeps K and V as E4M3 with one f16 scale
// per KV head and token; index keys stay bf16).
//
// One wave per (head, token) row: each lane holds head_dim / 64 elements,
// the row's largest magnitude comes from a wave reduction, the scale is
// f16(amax / 448) and every element is encoded as the E4M3 value nearest to
// x / scale (ties to the even code, saturating at 448).  The encoder works
// on the float32 bit pattern, so the codes do not depend on any conversion
// mode of the hardware.  Bytes moved per row: 2 D read, D + 2 written.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kRowsPerWG = 4;
constexpr float kE4m3Max = 448.f;
constexpr uint16_t kF16MaxBits = 0x7bffu;  // 65504

// E4M3 (OCP FN: bias 7, largest finite 448) code of a finite float32.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (!(a < kE4m3Max)) {
    code = 0x7eu;  // 448 and above saturate
  } else if (a < 0.015625f) {
    // below the smallest normal 2^-6: multiples of 2^-9 (an exact scaling),
    // rounded to the nearest even integer; 8 is the smallest normal (code 8)
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    // keep 3 mantissa bits, rounding to nearest even on the 20 dropped bits;
    // a carry moves into the exponent
    const uint32_t b = __float_as_uint(a);
    const uint32_t r = b + 0x7ffffu + ((b >> 20) & 1u);
    code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);  // exponent bias 127 -> 7
    code = code > 0x7eu ? 0x7eu : code;                   // rounding up past 448 saturates
  }
  return sign | code;
}

template <int D>
__global__ void __launch_bounds__(kWave * kRowsPerWG)
quantize_kv_fp8_kernel(const uint16_t* __restrict__ src, int n_head, int n_tok, int64_t src_hs,
                       uint8_t* __restrict__ dst, uint16_t* __restrict__ dst_scale, int64_t dst_hs) {
  constexpr int PER = D / kWave;  // 4 (D = 256) or 2 (D = 128) elements per lane
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
  amax = wave_max(amax);
  const _Float16 s16 = (_Float16)(amax / kE4m3Max);  // float32 quotient, round to nearest even
  uint16_t sbits = __builtin_bit_cast(uint16_t, s16);
  if ((sbits & 0x7fffu) == 0x7c00u) sbits = kF16MaxBits;  // f16 overflow clamps to 65504
  const float sf = (float)__builtin_bit_cast(_Float16, sbits);
  uint32_t packed = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t c = sf > 0.f ? e4m3_code(x[i] / sf) : 0u;
    packed |= c << (8 * i);
  }
  uint8_t* d = dst + (h * dst_hs + t) * D + PER * lane;
  if constexpr (PER == 4) {
    *reinterpret_cast<uint32_t*>(d) = packed;
  } else {
    *reinterpret_cast<uint16_t*>(d) = (uint16_t)packed;
  }
  if (lane == 0) dst_scale[h * dst_hs + t] = sbits;
}

}  // namespace

hipError_t launch_quantize_kv_fp8(const void* src, int n_head, int n_tok, int head_dim, int64_t src_head_stride,
                                  uint8_t* dst, uint16_t* dst_scale, int64_t dst_head_stride,
                                  hipStream_t stream) {
  const int64_t rows = (int64_t)n_head * n_tok;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + kRowsPerWG - 1) / kRowsPerWG));
  const uint16_t* s = static_cast<const uint16_t*>(src);
  if (head_dim == 256)
    hipLaunchKernelGGL(quantize_kv_fp8_kernel<256>, grid, dim3(kWave * kRowsPerWG), 0, stream, s, n_head, n_tok,
                       src_head_stride, dst, dst_scale, dst_head_stride);
  else
    hipLaunchKernelGGL(quantize_kv_fp8_kernel<128>, grid, dim3(kWave * kRowsPerWG), 0, stream, s, n_head, n_tok,
                       src_head_stride, dst, dst_scale, dst_head_stride);
  return hipGetLastError();
}

}  // namespace qsa
