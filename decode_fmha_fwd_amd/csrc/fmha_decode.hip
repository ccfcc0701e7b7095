// fmha_decode.hip -- instantiations and launchers of the split-KV decode
// attention kernels (16-row waves) and of the log-sum-exp combine kernel.
#include <hip/hip_runtime.h>

#include "decode_launch.hpp"

namespace fmha {

using decode_detail::launch_attn_cs;

fmha_status launch_decode(int D, int Dv, DecodeCfg c, const AttnParams& p, dim3 grid,
                          bool causal, bool split, bool kv_shared, hipStream_t st) {
  // Q/K head dim 576, V/O head dim 512: a latent of 512 plus 64 more key
  // dims.  V inside the K rows: one 4-deep ring of 32-key K tiles (144 KB);
  // separate V: 2-deep K and V rings (136 KB).
  if (D == 576 && Dv == 512) {
    if (kv_shared)
      return launch_attn_cs<576, 16, 4, 32, 4, 4, true, false, 512>(p, grid, causal, split, st);
    return launch_attn_cs<576, 16, 4, 32, 2, 2, false, false, 512>(p, grid, causal, split, st);
  }
  if (Dv != D)
    return fail(FMHA_ERR_HEAD_DIM, "decode: head dims D=%d, Dv=%d not built", D, Dv);
  // V aliasing K at head dim 512: one 5-deep ring of 32-key tiles (160 KB)
  if (D == 512 && kv_shared)
    return launch_attn_cs<512, 16, 4, 32, 5, 5, true>(p, grid, causal, split, st);
  // (head dims 64 and 128 also come with split groups; see decode_groups_built)
  if (D == 64 && c.nw == 1)
    return launch_attn_cs<64, 16, 1, 32, 3, 3, false, false, 64, true>(p, grid, causal, split, st);
  if (D == 64 && c.nw == 4)
    return launch_attn_cs<64, 16, 4, 64, 3, 3, false, false, 64, true>(p, grid, causal, split, st);
  // (head dim 128, one wave: a 3-deep K ring, 40 KB, four workgroups per CU --
  // 2048 workgroups of the MHA decode then run in exactly two rounds)
  if (D == 128 && c.nw == 1)
    return launch_attn_cs<128, 16, 1, 32, 3, 2, false, false, 128, true>(p, grid, causal, split, st);
  if (D == 128 && c.nw == 4)
    return launch_attn_cs<128, 16, 4, 64, 2, 2, false, false, 128, true>(p, grid, causal, split, st);
  if (D == 512) return launch_attn_cs<512, 16, 4, 32, 3, 2>(p, grid, causal, split, st);
  return fail(FMHA_ERR_HEAD_DIM, "fmha_decode_splitkv: head dim %d not built", D);
}

fmha_status launch_combine(int D, const float* op, const float* lp, uint16_t* o, float* lse,
                           float* amax, uint8_t* codes, uint8_t* scales, const float* gscale,
                           long long nrows, int nsplit, hipStream_t st) {
  const int rows_per_block = 4;
  dim3 grid((unsigned)((nrows + rows_per_block - 1) / rows_per_block));
  switch (D) {
    case 64:
      hipLaunchKernelGGL(lse_combine_kernel<64>, grid, dim3(256), 0, st, op, lp, o, lse, amax,
                         codes, scales, gscale, nrows, nsplit);
      break;
    case 128:
      hipLaunchKernelGGL(lse_combine_kernel<128>, grid, dim3(256), 0, st, op, lp, o, lse, amax,
                         codes, scales, gscale, nrows, nsplit);
      break;
    case 512:
      hipLaunchKernelGGL(lse_combine_kernel<512>, grid, dim3(256), 0, st, op, lp, o, lse, amax,
                         codes, scales, gscale, nrows, nsplit);
      break;
    default:
      return fail(FMHA_ERR_HEAD_DIM, "combine: head dim %d not built", D);
  }
  return check_launch("combine kernel launch");
}

}  // namespace fmha
