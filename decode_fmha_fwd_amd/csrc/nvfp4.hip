// nvfp4.hip -- NVFP4 quantisation of a bf16 matrix (the "FP4 quantization"
// item of the feature list on the page "NVFP4-1.1_RAW_CUDA_CPP_APPROACH.md"),
// and the C ABI entry nvfp4_quantize (see include/fmha.h for the recipe).
//
// This translation unit is compiled with fp contraction off, correctly rounded
// fp32 division and fp32 denormals kept, because every step decides integer
// codes: each arithmetic operation below is one IEEE binary32 operation.
//
// The block codecs live in nvfp4_device.hpp (shared with the fused decode
// epilogue).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/fmha.h"
#include "fmha_device.hpp"
#include "nvfp4_device.hpp"
#include "host_common.hpp"

namespace fmha {
namespace {

__global__ void zero_f32_kernel(float* p) { *p = 0.0f; }

// max |x| over n bf16 values (n a multiple of 8), folded into *amax with an
// integer atomic on the non-negative float bits.
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x, long long n8,
                                                   float* amax) {
  float m = 0.0f;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (long long)gridDim.x * blockDim.x) {
    const u32x4 v = *(const u32x4*)(x + i * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      m = fmaxf(m, fabsf(bf16_bits_to_float(v[w] & 0xFFFFu)));
      m = fmaxf(m, fabsf(bf16_bits_to_float(v[w] >> 16)));
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomic_max_nonneg(amax, m);
}

// One thread per block of 16 elements.
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x,
                                                       long long nblocks,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       float* __restrict__ global_scale,
                                                       const float* __restrict__ amax_p) {
  const long long blk = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const float amax = *amax_p;
  const float g = amax / 2688.0f;
  if (blk == 0) *global_scale = g;
  if (blk >= nblocks) return;
  const u32x4 v0 = *(const u32x4*)(x + blk * 16);
  const u32x4 v1 = *(const u32x4*)(x + blk * 16 + 8);
  float xs[16];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    xs[2 * w] = bf16_bits_to_float(v0[w] & 0xFFFFu);
    xs[2 * w + 1] = bf16_bits_to_float(v0[w] >> 16);
    xs[8 + 2 * w] = bf16_bits_to_float(v1[w] & 0xFFFFu);
    xs[8 + 2 * w + 1] = bf16_bits_to_float(v1[w] >> 16);
  }
  float ab = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) ab = fmaxf(ab, fabsf(xs[e]));
  float t;
  const uint32_t s = nvfp4_block_scale(ab, g, t);
  scales[blk] = (uint8_t)s;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) lo |= nvfp4_code(xs[e], s, t) << (4 * e);
#pragma unroll
  for (int e = 0; e < 8; ++e) hi |= nvfp4_code(xs[8 + e], s, t) << (4 * e);
  *(u32x2*)(codes + blk * 8) = u32x2{lo, hi};
}

}  // namespace
}  // namespace fmha

using namespace fmha;

extern "C" {

size_t nvfp4_quantize_workspace_size(long long rows, int cols) {
  (void)rows;
  (void)cols;
  return 256;
}

fmha_status nvfp4_quantize(const void* x, long long rows, int cols, uint8_t* codes,
                           uint8_t* scales, float* global_scale, const float* amax_in,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !codes || !scales || !global_scale)
    return fail(FMHA_ERR_NULL, "x, codes, scales and global_scale must be non-null");
  if (rows < 1 || cols < 16 || cols % 16 != 0)
    return fail(FMHA_ERR_SHAPE, "need rows >= 1 and cols a positive multiple of 16");
  if (rows > (1LL << 40) / cols) return fail(FMHA_ERR_SHAPE, "tensor too large");
  if (!aligned16(x) || ((uintptr_t)codes & 7u) || ((uintptr_t)global_scale & 3u) ||
      (amax_in && ((uintptr_t)amax_in & 3u)))
    return fail(FMHA_ERR_ALIGN,
                "x must be 16-byte aligned, codes 8-byte, global_scale and amax_in 4-byte");
  const hipStream_t st = (hipStream_t)stream;
  const long long n = rows * (long long)cols;
  const float* amax = amax_in;
  if (!amax) {
    if (!workspace || workspace_bytes < nvfp4_quantize_workspace_size(rows, cols))
      return fail(FMHA_ERR_WORKSPACE, "workspace of %zu bytes needed",
                  nvfp4_quantize_workspace_size(rows, cols));
    if ((uintptr_t)workspace & 3u) return fail(FMHA_ERR_ALIGN, "workspace must be 4-byte aligned");
    float* ws = (float*)workspace;
    hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(1), 0, st, ws);
    fmha_status s = check_launch("amax reset launch");
    if (s != FMHA_OK) return s;
    const long long n8 = n / 8;
    long long grid = (n8 + 255) / 256;
    if (grid > 2048) grid = 2048;
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)x,
                       n8, ws);
    s = check_launch("amax kernel launch");
    if (s != FMHA_OK) return s;
    amax = ws;
  }
  const long long nblocks = n / 16;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)x, nblocks, codes, scales, global_scale, amax);
  return check_launch("quantize kernel launch");
}

}  // extern "C"
