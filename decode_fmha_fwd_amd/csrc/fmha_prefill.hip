// fmha_prefill.hip -- instantiations and launchers of the prefill attention
// kernels (4 waves x 32 query rows, 64-key tiles) and of the QK test hook.
// Built with MFMA accumulators in ordinary VGPRs (no AGPR copies).
#include <hip/hip_runtime.h>

#include "attn_kernels.hpp"
#include "host_common.hpp"
#include "launch.hpp"

namespace fmha {
namespace {

template <int D, int MT, int NW, int KT, int KS, int VS, bool C, bool S>
fmha_status launch_attn(const AttnParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, MT, NW, KT, KS, VS, C, S>), grid, dim3(NW * 64), 0, st,
                     p);
  return check_launch("attention kernel launch");
}

template <int D, int MT, int NW, int KT, int KS, int VS>
fmha_status launch_attn_cs(const AttnParams& p, dim3 grid, bool causal, bool split,
                           hipStream_t st) {
  if (causal)
    return split ? launch_attn<D, MT, NW, KT, KS, VS, true, true>(p, grid, st)
                 : launch_attn<D, MT, NW, KT, KS, VS, true, false>(p, grid, st);
  return split ? launch_attn<D, MT, NW, KT, KS, VS, false, true>(p, grid, st)
               : launch_attn<D, MT, NW, KT, KS, VS, false, false>(p, grid, st);
}

}  // namespace

// Prefill: 4 waves of 32 rows = 128 query rows per workgroup, 64-key tiles in
// a 3-stage LDS ring (2 stages at head dim 128).
fmha_status launch_fwd(int D, const AttnParams& p, dim3 grid, bool causal, hipStream_t st) {
  switch (D) {
    case 16: return launch_attn_cs<16, 32, 4, 64, 3, 3>(p, grid, causal, false, st);
    case 32: return launch_attn_cs<32, 32, 4, 64, 3, 3>(p, grid, causal, false, st);
    case 64: return launch_attn_cs<64, 32, 4, 64, 3, 3>(p, grid, causal, false, st);
    case 128: return launch_attn_cs<128, 32, 4, 64, 2, 2>(p, grid, causal, false, st);
  }
  return fail(FMHA_ERR_HEAD_DIM, "fmha_fwd: head dim %d not built", D);
}

fmha_status launch_debug_scores(const uint16_t* q, const uint16_t* k, float* s_out, int Sq,
                                int Sk, int D, float scale, hipStream_t st) {
  switch (D) {
    case 16: hipLaunchKernelGGL(qk_scores_debug_kernel<16>, dim3(1), dim3(256), 0, st, q, k, s_out, Sq, Sk, scale); break;
    case 32: hipLaunchKernelGGL(qk_scores_debug_kernel<32>, dim3(1), dim3(256), 0, st, q, k, s_out, Sq, Sk, scale); break;
    case 64: hipLaunchKernelGGL(qk_scores_debug_kernel<64>, dim3(1), dim3(256), 0, st, q, k, s_out, Sq, Sk, scale); break;
    case 128: hipLaunchKernelGGL(qk_scores_debug_kernel<128>, dim3(1), dim3(256), 0, st, q, k, s_out, Sq, Sk, scale); break;
    default: return fail(FMHA_ERR_HEAD_DIM, "debug scores support D in {16,32,64,128}");
  }
  return check_launch("debug score kernel launch");
}

}  // namespace fmha
