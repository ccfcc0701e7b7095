// nvfp4_device.hpp -- NVFP4 block encoding shared by the standalone quantiser
// (nvfp4.hip) and the fused decode epilogue (attn_kernels.hpp): the "FP4
// quantization" item of the feature list on the page
// "NVFP4-1.1_RAW_CUDA_CPP_APPROACH.md", with the block recipe of include/fmha.h.
//
// Codecs are written from the format definitions (OCP 8-bit Floating Point
// Specification, E4M3FN; OCP Microscaling Formats v1.0, E2M1), with
// round-to-nearest-even:
//   * E4M3: below 2^-6 the grid is m * 2^-9 (m = 0..7), so the code is
//     rint(x * 2^9); above, the float's 23-bit mantissa is rounded to 3 bits
//     (round half to even on the dropped 20 bits, carries run into the
//     exponent) and the exponent is re-biased from 127 to 7.  x >= 448
//     saturates to 0x7E.
//   * E2M1: the magnitude grid {0, .5, 1, 1.5, 2, 3, 4, 6} split at its
//     midpoints; at a midpoint the even code wins, which decides whether the
//     comparison is strict.
// Every fp32 operation below is one IEEE binary32 operation: the including
// translation units are built with correctly rounded fp32 division and fp32
// denormals kept, and no expression here has a multiply feeding an add that
// contraction could fuse.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

__device__ inline uint32_t e4m3_encode(float x) {
  if (!(x > 0.0f)) return 0u;
  if (x >= 448.0f) return 0x7Eu;
  if (x < 0.015625f) {  // 2^-6: subnormal grid m * 2^-9 (m = 8 is the first normal)
    return (uint32_t)__builtin_rintf(x * 512.0f);
  }
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;  // 8-bit exp, 3-bit mantissa
  const uint32_t c = r - ((127u - 7u) << 3);
  return c > 0x7Eu ? 0x7Eu : c;
}

__device__ inline float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
}

__device__ inline uint32_t e2m1_encode(float q) {
  const float a = fabsf(q);
  const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
  return mag | ((__builtin_bit_cast(uint32_t, q) >> 28) & 8u);
}

// Block scale of a 16-element block with max |x| = ab under the global scale
// g: s = E4M3((ab / 6) / g) and the decode step t = value(s) * g (s = 0 and
// t = 0 when g is not positive).
__device__ inline uint32_t nvfp4_block_scale(float ab, float g, float& t) {
  t = 0.0f;
  if (!(g > 0.0f)) return 0u;
  const float sixth = ab / 6.0f;
  const float sf = sixth / g;
  const uint32_t s = e4m3_encode(sf);
  t = e4m3_value(s) * g;
  return s;
}

// E2M1 code of x / t (0 when the block scale is 0 or t underflowed).
__device__ inline uint32_t nvfp4_code(float x, uint32_t s, float t) {
  return (s != 0u && t > 0.0f) ? e2m1_encode(x / t) : 0u;
}

}  // namespace fmha
