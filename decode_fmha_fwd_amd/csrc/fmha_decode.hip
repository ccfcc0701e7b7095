// fmha_decode.hip -- instantiations and launchers of the split-KV decode
// attention kernels (16-row waves; configurations in with_decode_cfg) and of
// the log-sum-exp combine kernel.
#include <hip/hip_runtime.h>

#include "decode_launch.hpp"

namespace fmha {

using decode_detail::launch_attn_cs;

fmha_status launch_decode(int D, int Dv, DecodeCfg c, const AttnParams& p, dim3 grid,
                          bool causal, bool split, bool kv_shared, hipStream_t st) {
  const fmha_status s = with_decode_cfg(D, Dv, c, kv_shared, [&](auto cfg) {
    using C = decltype(cfg);
    return launch_attn_cs<C::D, C::MT, C::NW, C::KT, C::KS, C::VS, C::KVS, false, C::DV,
                          C::GROUPS>(p, grid, causal, split, st);
  });
  if (s == FMHA_ERR_HEAD_DIM)
    return fail(s, "fmha_decode_splitkv: head dims D=%d, Dv=%d not built", D, Dv);
  return s;
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
