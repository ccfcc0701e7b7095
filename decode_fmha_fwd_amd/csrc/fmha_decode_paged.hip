// fmha_decode_paged.hip -- the split-KV decode reading K and V from a paged
// cache: the tile configurations of fmha_decode.hip with PAGED set.
#include "decode_launch.hpp"

namespace fmha {

using decode_detail::launch_attn_cs;

fmha_status launch_decode_paged(int D, DecodeCfg c, const AttnParams& p, dim3 grid, bool causal,
                                bool split, hipStream_t st) {
  if (D == 64 && c.nw == 1)
    return launch_attn_cs<64, 16, 1, 32, 3, 3, false, true, 64, true>(p, grid, causal, split, st);
  if (D == 64 && c.nw == 4)
    return launch_attn_cs<64, 16, 4, 64, 3, 3, false, true, 64, true>(p, grid, causal, split, st);
  if (D == 128 && c.nw == 1)
    return launch_attn_cs<128, 16, 1, 32, 2, 2, false, true, 128, true>(p, grid, causal, split, st);
  if (D == 128 && c.nw == 4)
    return launch_attn_cs<128, 16, 4, 64, 2, 2, false, true, 128, true>(p, grid, causal, split, st);
  if (D == 512) return launch_attn_cs<512, 16, 4, 32, 3, 2, false, true>(p, grid, causal, split, st);
  return fail(FMHA_ERR_HEAD_DIM, "fmha_decode_paged: head dim %d not built", D);
}

}  // namespace fmha
