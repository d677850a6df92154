// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// fp64 -> fp16 bits, round to nearest even, saturating at 65504 (v >= 0 expected;
// negative and NaN inputs give 0).
__device__ __forceinline__ uint16_t f64_to_f16_rne_sat(double v) {
  if (!(v > 0.0)) return 0;
  if (v >= 65520.0) return 0x7BFF;
  int e;
  frexp(v, &e);        // v = m 2^e, m in [0.5, 1): unbiased exponent e-1
  int E = e - 1;
  if (E < -14) E = -14;  // subnormal range shares the 2^-24 spacing
  // scaling by the power-of-two spacing is exact; rint rounds half to even
  const double r = ldexp(rint(ldexp(v, 10 - E)), E - 10);
  return __half_as_ushort(__float2half((float)r));  // r is an fp16 value: exact
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// number of codebook boundaries strictly below y/n (n > 0), as t_k * n < y
__device__ __forceinline__ int cell_index(const Codebook &cb, float y, float n) {
  int idx = 0;
#pragma unroll
  for (int k = 0; k < kMaxCentroids - 1; ++k)
    if (k < cb.L - 1) idx += (cb.t[k] * n < y) ? 1 : 0;
  return idx;
}

// Walsh subset masks (odd-size subsets of the index bits), enumeration order shared with the host
__host__ __device__ constexpr int walsh_count(int b) { return 1 << (b - 1); }

// Walsh planes of index bit-plane words: the odd-size subsets of the bits, XORed (a symmetric codebook
// is an odd function of the index bits, so c[idx] = sum_S beta_S prod_{p in S} (2 bit_p - 1))
template <int B>
__device__ __forceinline__ void walsh_planes(const uint32_t *w, uint32_t *out) {
  if constexpr (B == 1) {
    out[0] = w[0];
  } else if constexpr (B == 2) {
    out[0] = w[0]; out[1] = w[1];
  } else if constexpr (B == 3) {
    out[0] = w[0]; out[1] = w[1]; out[2] = w[2]; out[3] = w[0] ^ w[1] ^ w[2];
  } else {
    out[0] = w[0]; out[1] = w[1]; out[2] = w[2]; out[3] = w[3];
    out[4] = w[0] ^ w[1] ^ w[2]; out[5] = w[0] ^ w[1] ^ w[3];
    out[6] = w[0] ^ w[2] ^ w[3]; out[7] = w[1] ^ w[2] ^ w[3];
  }
}

__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
// integer min/max (the generic device min/max overloads may go through floating point)
__host__ __device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ __forceinline__ int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }
__host__ __device__ __forceinline__ int imin32(int a, int b) { return a < b ? a : b; }

}  // namespace tq
