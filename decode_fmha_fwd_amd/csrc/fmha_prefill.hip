// fmha_prefill.hip -- instantiations and launchers of the prefill attention
// kernels (4 waves x 32 query rows, 64-key tiles; configurations in
// with_fwd_cfg: the pipelined kernel of prefill_kernel.hpp or attn_fwd_kernel).  Built with MFMA accumulators in ordinary VGPRs (no AGPR
// copies).
#include <hip/hip_runtime.h>

#include "prefill_kernel.hpp"
#include "host_common.hpp"
#include "launch.hpp"

namespace fmha {

fmha_status launch_fwd(int D, int Dv, const AttnParams& p, bool causal, hipStream_t st) {
  const int cus = num_cus();
  const fmha_status s = with_fwd_cfg(D, Dv, [&](auto cfg) {
    using C = decltype(cfg);
    if (causal)
      launch_prefill_cfg<C, true, false>(p, cus, st);
    else
      launch_prefill_cfg<C, false, false>(p, cus, st);
    return check_launch("attention kernel launch");
  });
  if (s == FMHA_ERR_HEAD_DIM)
    return fail(s, "fmha_fwd: head dims D=%d, Dv=%d not built", D, Dv);
  return s;
}

}  // namespace fmha
