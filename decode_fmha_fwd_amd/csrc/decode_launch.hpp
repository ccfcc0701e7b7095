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
          int DV, bool G = false>
fmha_status launch_attn(const AttnParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, MT, NW, KT, KS, VS, C, S, KVS, PG, DV, G>), grid,
                     dim3(NW * 64), 0, st, p);
  return check_launch("attention kernel launch");
}

// The four (causal, split) instantiations of one tile configuration, plus the
// two with split groups (p.splits_per_wg > 1) where GROUPS is set.
template <int D, int MT, int NW, int KT, int KS, int VS, bool KVS = false, bool PG = false,
          int DV = D, bool GROUPS = false>
fmha_status launch_attn_cs(const AttnParams& p, dim3 grid, bool causal, bool split,
                           hipStream_t st) {
  if (split && p.splits_per_wg > 1) {
    if constexpr (GROUPS) {
      return causal ? launch_attn<D, MT, NW, KT, KS, VS, true, true, KVS, PG, DV, true>(p, grid, st)
                    : launch_attn<D, MT, NW, KT, KS, VS, false, true, KVS, PG, DV, true>(p, grid, st);
    } else {
      return fail(FMHA_ERR_ARG, "split groups are not built for head dim %d", D);
    }
  }
  if (causal)
    return split ? launch_attn<D, MT, NW, KT, KS, VS, true, true, KVS, PG, DV>(p, grid, st)
                 : launch_attn<D, MT, NW, KT, KS, VS, true, false, KVS, PG, DV>(p, grid, st);
  return split ? launch_attn<D, MT, NW, KT, KS, VS, false, true, KVS, PG, DV>(p, grid, st)
               : launch_attn<D, MT, NW, KT, KS, VS, false, false, KVS, PG, DV>(p, grid, st);
}

}  // namespace decode_detail
}  // namespace fmha
