// buffer_copy.hpp -- asynchronous global->LDS tile copies through buffer
// loads with the LDS bit (buffer_load_dwordx4 ... lds), shared by the
// pipelined prefill kernel and the wide-head decode kernel.
//
// A buffer descriptor bounds every copy: loads at or past its byte count
// return zeros without touching memory, so rows past the keys a workgroup
// may see, and whole tiles past the last, need no clamping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.hpp"

namespace fmha {

// One 16-byte-per-lane buffer load into LDS (buffer_load_dwordx4 ... lds):
// lane l's 16 bytes at byte voff of the raw buffer [base, base + bytes) land
// at lds + 16 l; loads at or past `bytes` return zeros (the range check is on
// the lane offset).  The descriptor (word 3: the gfx9 raw-buffer format) is
// built from scalar values that stay the same through a row block, so it is
// hoisted out of the tile loop.  Only the device pass sees the body: in the
// host pass a kernel template that calls these builtins loses the host stubs
// of its later instantiations.
// AUX: the cache-policy operand (2 = non-temporal, for data read once).
template <int AUX = 0>
__device__ inline void buffer_load_lds16(const void* base, uint32_t bytes, FMHA_LDS void* lds,
                                         uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, AUX);
#else
  (void)base, (void)bytes, (void)lds, (void)voff;
#endif
}

// Copies of one [KT][W] bf16 tile into a swizzled LDS tile with buffer loads:
// copy j of wave w fills LDS slots [(j*NW + w)*64, +64) (16 bytes each); a
// lane fetches the global chunk that belongs in its slot, so 8 lanes read one
// 128-byte row segment.  voff: the lane's byte offset within the tile.
// (NW: the waves that share the copies; AUX: as for buffer_load_lds16)
template <int W, int NW, int KT, int AUX = 0>
struct BufTileCopy {
  static constexpr int kLoads = KT * W * 2 / (NW * 64 * 16);
  static_assert(kLoads >= 1 && kLoads * NW * 64 * 16 == KT * W * 2, "tile splits over copies");
  uint32_t voff[kLoads];

  __device__ inline void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int byte = ((j * NW + wave) * 64 + lane) * 16;
      const int row = byte / (W * 2);
      const int pchunk = (byte - row * W * 2) >> 4;
      voff[j] = (uint32_t)(row * W * 2 + ((pchunk ^ swz<W / 8>(row)) << 4));
    }
  }
  // rows: the cache rows of one (batch, KV head), `bytes` of them readable
  // (rows past them read as zeros); tile_bytes: the byte offset of the
  // tile's first row; lds: the stage base.
  __device__ inline void issue(const uint16_t* rows, uint32_t bytes, uint32_t tile_bytes,
                               FMHA_LDS char* lds, int wave_u) const {
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      buffer_load_lds16<AUX>(rows, bytes, (FMHA_LDS void*)(lds + (j * NW + wave_u) * 64 * 16),
                             tile_bytes + voff[j]);
  }
};

}  // namespace fmha
