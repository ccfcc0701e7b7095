// fmha_prefill.hip -- instantiations and launchers of the prefill attention
// kernels (4 waves x 32 query rows, 64-key tiles; configurations in
// with_fwd_cfg).  Built with MFMA accumulators in ordinary VGPRs (no AGPR
// copies).
#include <hip/hip_runtime.h>

#include "attn_kernels.hpp"
#include "host_common.hpp"
#include "launch.hpp"

namespace fmha {

fmha_status launch_fwd(int D, int Dv, const AttnParams& p, dim3 grid, bool causal,
                       hipStream_t st) {
  const fmha_status s = with_fwd_cfg(D, Dv, [&](auto cfg) {
    using C = decltype(cfg);
    if (causal)
      hipLaunchKernelGGL((attn_fwd_kernel<C::D, C::MT, C::NW, C::KT, C::KS, C::VS, true, false,
                                          false, false, C::DV>),
                         grid, dim3(C::NW * 64), 0, st, p);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<C::D, C::MT, C::NW, C::KT, C::KS, C::VS, false, false,
                                          false, false, C::DV>),
                         grid, dim3(C::NW * 64), 0, st, p);
    return check_launch("attention kernel launch");
  });
  if (s == FMHA_ERR_HEAD_DIM)
    return fail(s, "fmha_fwd: head dims D=%d, Dv=%d not built", D, Dv);
  return s;
}

}  // namespace fmha
