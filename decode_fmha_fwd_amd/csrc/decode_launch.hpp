// decode_launch.hpp -- launch helpers of the decode attention kernel, shared by
// the translation units that instantiate it (contiguous and paged K/V).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_kernels.hpp"
#include "host_common.hpp"
#include "launch.hpp"

namespace fmha {
namespace decode_detail {

template <int D, int MT, int NW, int KT, int KS, int VS, bool C, bool S, bool KVS, bool PG,
          int DV>
fmha_status launch_attn(const AttnParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, MT, NW, KT, KS, VS, C, S, KVS, PG, DV>), grid,
                     dim3(NW * 64), 0, st, p);
  return check_launch("attention kernel launch");
}

// The four (causal, split) instantiations of one tile configuration.
template <int D, int MT, int NW, int KT, int KS, int VS, bool KVS = false, bool PG = false,
          int DV = D>
fmha_status launch_attn_cs(const AttnParams& p, dim3 grid, bool causal, bool split,
                           hipStream_t st) {
  if (causal)
    return split ? launch_attn<D, MT, NW, KT, KS, VS, true, true, KVS, PG, DV>(p, grid, st)
                 : launch_attn<D, MT, NW, KT, KS, VS, true, false, KVS, PG, DV>(p, grid, st);
  return split ? launch_attn<D, MT, NW, KT, KS, VS, false, true, KVS, PG, DV>(p, grid, st)
               : launch_attn<D, MT, NW, KT, KS, VS, false, false, KVS, PG, DV>(p, grid, st);
}

}  // namespace decode_detail
}  // namespace fmha
