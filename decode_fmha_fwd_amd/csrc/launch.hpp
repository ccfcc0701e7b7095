// launch.hpp -- the parameter block of the attention kernels and the host
// launchers each kernel translation unit provides to the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fmha.h"

namespace fmha {

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;          // bf16 output (no split)
  float* lse;           // fp32 [rows] or null (no split)
  float* o_part;        // fp32 [rows][nsplit][Dv] (split)
  float* lse_part;      // fp32 [rows][nsplit]   (split)
  float* o_amax;        // optional running max |O| (no split)
  uint8_t* fp4_codes;   // optional fused NVFP4 output: codes [rows][Dv/2] (no split)
  uint8_t* fp4_scales;  //   E4M3 block scales [rows][Dv/16]
  const float* fp4_gscale;  //   the caller's global scale (1 float, device)
  int B;
  int Hkv;
  int Sq;
  int Sk;
  int rows_per_kv;      // (Hq / Hkv) * Sq query rows share one KV head
  int n_row_blocks;     // ceil(rows_per_kv / (NW * MT))
  int nsplit;           // key ranges per (batch, KV head)
  int split_len;        // keys per range, a multiple of KT
  int splits_per_wg;    // consecutive splits one workgroup takes (split groups), >= 1
  int combine_in_wg;    // split groups holding every split: the kernel combines them
  float scale_log2;     // scale * log2(e)
  // Paged KV cache (decode only).  K and V are [num_pages][Hkv][page_size][D];
  // key j of batch b sits in page block_table[b * bt_stride + j / page_size].
  const int* seqlens;      // keys per batch [B] (clamped to [0, Sk], Sk = bt_stride * page_size)
  const int* block_table;  // page ids [B][bt_stride] (clamped to [0, num_pages))
  int bt_stride;
  int page_shift;          // log2(page_size); page_size is a power of two >= 64
  int num_pages;
};

// Tile configuration of the decode kernel for a head dim and a row count.
struct DecodeCfg {
  int nw;          // waves per workgroup (16 query rows each)
  int kt;          // keys per tile
  int wgs_per_cu;  // workgroups one CU holds at once (LDS-limited)
};

// One-wave workgroups when the rows of a KV head fit in one 16-row wave (many
// small workgroups keep enough loads in flight per CU); four waves otherwise.
// Head dim 512 (and 576 with V/O at 512): four waves sharing 32-key tiles in
// rings that take most of the CU's 160 KB of LDS.
// Must match the instantiations in fmha_decode.hip.
inline DecodeCfg decode_cfg(int D, int rows_per_kv) {
  if (D >= 512) return {4, 32, 1};
  if (rows_per_kv <= 16) return {1, 32, D == 64 ? 6 : 4};
  return {4, 64, D == 64 ? 3 : 2};
}

// Decode configurations built with split groups (one workgroup streaming
// several consecutive splits): head dims 64 and 128, two separate rings, a
// contiguous or a paged cache.
inline bool decode_groups_built(int D, int Dv, bool kv_shared) {
  return Dv == D && (D == 64 || D == 128) && !kv_shared;
}

// fmha_prefill.hip: 128-row prefill workgroups (4 waves x 32 rows).
fmha_status launch_fwd(int D, int Dv, const AttnParams& p, dim3 grid, bool causal,
                       hipStream_t st);
fmha_status launch_debug_scores(const uint16_t* q, const uint16_t* k, float* s_out, int Sq,
                                int Sk, int D, float scale, hipStream_t st);

// fmha_decode.hip: split-KV decode (16-row waves) and the log-sum-exp combine.
// D: head dim of Q/K, Dv: of V/O; kv_shared: V is the first Dv columns of the
// K rows (p.v == p.k).
fmha_status launch_decode(int D, int Dv, DecodeCfg c, const AttnParams& p, dim3 grid,
                          bool causal, bool split, bool kv_shared, hipStream_t st);
// The same decode reading K/V from a paged cache (p.seqlens, p.block_table set).
fmha_status launch_decode_paged(int D, DecodeCfg c, const AttnParams& p, dim3 grid, bool causal,
                                bool split, hipStream_t st);
fmha_status launch_combine(int D, const float* o_part, const float* lse_part, uint16_t* o,
                           float* lse, float* o_amax, uint8_t* fp4_codes, uint8_t* fp4_scales,
                           const float* fp4_gscale, long long nrows, int nsplit,
                           hipStream_t st);

}  // namespace fmha
