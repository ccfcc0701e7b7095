// fmha_debug.hip -- the test-only instantiations of the attention kernels
// with DBG_S set: the prefill configurations of with_fwd_cfg and the
// one-split decode configurations of with_decode_cfg, non-causal, each
// storing its raw score tiles (fmha_debug_qk_scores).  The template
// arguments come from the same tables the production launches use, so the
// QK block under test is the one those kernels run.
#include <hip/hip_runtime.h>

#include "prefill_kernel.hpp"
#include "host_common.hpp"
#include "launch.hpp"

namespace fmha {

fmha_status launch_debug_scores(int D, int Dv, DecodeCfg c, const AttnParams& p, dim3 grid,
                                bool decode, bool kv_shared, hipStream_t st) {
  fmha_status s;
  if (!decode) {
    s = with_fwd_cfg(D, Dv, [&](auto cfg) {
      using C = decltype(cfg);
      launch_prefill_cfg<C, false, true>(p, num_cus(), st);
      return check_launch("debug score launch (prefill)");
    });
  } else if (decode_wide_takes(D, Dv, p.Sk, kv_shared)) {
    s = launch_decode_wide(D, Dv, p, grid, false, false, true, st);
  } else {
    s = with_decode_cfg(D, Dv, c, kv_shared, [&](auto cfg) {
      using C = decltype(cfg);
      hipLaunchKernelGGL((attn_fwd_kernel<C::D, C::MT, C::NW, C::KT, C::KS, C::VS, false, false,
                                          C::KVS, false, C::DV, false, true>),
                         grid, dim3(C::NW * 64), 0, st, p);
      return check_launch("debug score launch (decode)");
    });
  }
  if (s == FMHA_ERR_HEAD_DIM)
    return fail(s, "fmha_debug_qk_scores: head dims D=%d, Dv=%d not built", D, Dv);
  return s;
}

}  // namespace fmha
