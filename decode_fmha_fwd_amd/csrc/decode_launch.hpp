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
fmha_status launch_attn(const AttnParams& p0, dim3 grid, hipStream_t st) {
  auto kernel = attn_fwd_kernel<D, MT, NW, KT, KS, VS, C, S, KVS, PG, DV, G>;
  AttnParams p = p0;
  p.part_lds_bytes = 0;
  if constexpr (G) {
    // Split groups combining in the workgroup keep the partials in dynamic
    // LDS when that still leaves every workgroup of the grid resident at once
    // (the static LDS of the kernel plus the partials, per CU).
    if (p.combine_in_wg) {
      static const size_t stat = [&] {
        hipFuncAttributes a{};
        return hipFuncGetAttributes(&a, (const void*)kernel) == hipSuccess ? a.sharedSizeBytes
                                                                          : (size_t)0;
      }();
      const size_t rows = (size_t)(NW * MT < p.rows_per_kv ? NW * MT : p.rows_per_kv);
      const size_t bytes = rows * (size_t)p.nsplit * (DV + 1) * sizeof(float);
      const size_t per_cu = 160 * 1024;
      if (stat > 0 && bytes <= 48 * 1024 &&
          (long long)grid.x <= (long long)(per_cu / (stat + bytes)) * num_cus())
        p.part_lds_bytes = (int)bytes;
    }
  }
  hipLaunchKernelGGL(kernel, grid, dim3(NW * 64), (size_t)p.part_lds_bytes, st, p);
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
