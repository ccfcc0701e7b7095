// fmha_prefill.hip -- instantiations and launchers of the prefill attention
// kernels (4 waves x 32 query rows, 64-key tiles) and of the QK test hook.
// Built with MFMA accumulators in ordinary VGPRs (no AGPR copies).
#include <hip/hip_runtime.h>

#include "attn_kernels.hpp"
#include "host_common.hpp"
#include "launch.hpp"

namespace fmha {
namespace {

template <int D, int MT, int NW, int KT, int KS, int VS, bool C, int DV>
fmha_status launch_attn(const AttnParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, MT, NW, KT, KS, VS, C, false, false, false, DV>), grid,
                     dim3(NW * 64), 0, st, p);
  return check_launch("attention kernel launch");
}

template <int D, int MT, int NW, int KT, int KS, int VS, int DV = D>
fmha_status launch_attn_c(const AttnParams& p, dim3 grid, bool causal, hipStream_t st) {
  return causal ? launch_attn<D, MT, NW, KT, KS, VS, true, DV>(p, grid, st)
                : launch_attn<D, MT, NW, KT, KS, VS, false, DV>(p, grid, st);
}

}  // namespace

// Prefill: 4 waves of 32 rows = 128 query rows per workgroup, 64-key tiles in
// 2-stage LDS rings at head dims 64 and 128 (3 stages at 16 and 32; at 64 the
// 2-stage rings, 32 KB, measured 1-2 % faster than 3 stages, 48 KB, and
// 4 stages 5-8 % slower).  Q/K head dim 192 with V/O head dim 128: 2-stage K
// (24 KB tiles) and V (16 KB) rings, 80 KB.
fmha_status launch_fwd(int D, int Dv, const AttnParams& p, dim3 grid, bool causal,
                       hipStream_t st) {
  if (D == 192 && Dv == 128) return launch_attn_c<192, 32, 4, 64, 2, 2, 128>(p, grid, causal, st);
  if (Dv != D) return fail(FMHA_ERR_HEAD_DIM, "fmha_fwd: head dims D=%d, Dv=%d not built", D, Dv);
  switch (D) {
    case 16: return launch_attn_c<16, 32, 4, 64, 3, 3>(p, grid, causal, st);
    case 32: return launch_attn_c<32, 32, 4, 64, 3, 3>(p, grid, causal, st);
    case 64: return launch_attn_c<64, 32, 4, 64, 2, 2>(p, grid, causal, st);
    case 128: return launch_attn_c<128, 32, 4, 64, 2, 2>(p, grid, causal, st);
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
