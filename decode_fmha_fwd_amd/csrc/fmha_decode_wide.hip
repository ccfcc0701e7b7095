// fmha_decode_wide.hip -- instantiations and launcher of the wide-head
// split-KV decode with V inside the K rows (decode_wide.hpp), including its
// test-only score-storing build.
#include <hip/hip_runtime.h>

#include "decode_wide.hpp"
#include "host_common.hpp"
#include "launch.hpp"

namespace fmha {
namespace {

template <int D, int DV, bool C, bool S, bool DBG = false>
fmha_status go(const AttnParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_wide_kernel<D, DV, C, S, DBG>), grid, dim3(kWideThreads), 0, st, p);
  return check_launch(DBG ? "debug score launch (wide decode)" : "wide decode launch");
}

template <int D, int DV>
fmha_status launch_dims(const AttnParams& p, dim3 grid, bool causal, bool split, bool dbg,
                        hipStream_t st) {
  if (dbg) return go<D, DV, false, false, true>(p, grid, st);
  if (causal) return split ? go<D, DV, true, true>(p, grid, st) : go<D, DV, true, false>(p, grid, st);
  return split ? go<D, DV, false, true>(p, grid, st) : go<D, DV, false, false>(p, grid, st);
}

}  // namespace

bool decode_wide_takes(int D, int Dv, int Sk, bool kv_shared) {
  return kv_shared && ((D == 512 && Dv == 512) || (D == 576 && Dv == 512)) &&
         decode_wide_fits(Sk, D);
}

fmha_status launch_decode_wide(int D, int Dv, const AttnParams& p, dim3 grid, bool causal,
                               bool split, bool dbg, hipStream_t st) {
  if (D == 512 && Dv == 512) return launch_dims<512, 512>(p, grid, causal, split, dbg, st);
  if (D == 576 && Dv == 512) return launch_dims<576, 512>(p, grid, causal, split, dbg, st);
  return fail(FMHA_ERR_HEAD_DIM, "wide decode: head dims D=%d, Dv=%d not built", D, Dv);
}

}  // namespace fmha
