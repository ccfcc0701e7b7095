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
  int part_lds_bytes;   // with combine_in_wg: > 0 when the partials stay in dynamic LDS
                        // (that many bytes, [rows of the workgroup][nsplit][Dv + 1] fp32)
  float scale_log2;     // scale * log2(e)
  // Paged KV cache (decode only).  K and V are [num_pages][Hkv][page_size][D];
  // key j of batch b sits in page block_table[b * bt_stride + j / page_size].
  const int* seqlens;      // keys per batch [B] (clamped to [0, Sk], Sk = bt_stride * page_size)
  const int* block_table;  // page ids [B][bt_stride] (clamped to [0, num_pages))
  int bt_stride;
  int page_shift;          // log2(page_size); page_size is a power of two >= 64
  int num_pages;
  int rb_per_wg;        // prefill: row blocks per workgroup (1, or 2 paired)
  // Test builds (DBG_S) only: raw score tiles times s_dbg_scale, [rows][Sk].
  float* s_dbg;
  float s_dbg_scale;
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
// Must match the configurations of with_decode_cfg below.
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

// Compile-time tile configuration of one attention kernel instantiation.
// PIPE (prefill): the software-pipelined kernel of prefill_kernel.hpp (its
// own fixed tiling) instead of attn_fwd_kernel.
template <int D_, int MT_, int NW_, int KT_, int KS_, int VS_, bool KVS_ = false, int DV_ = D_,
          bool GROUPS_ = false, bool PIPE_ = false>
struct TileCfg {
  static constexpr int D = D_, MT = MT_, NW = NW_, KT = KT_, KS = KS_, VS = VS_, DV = DV_;
  static constexpr bool KVS = KVS_, GROUPS = GROUPS_, PIPE = PIPE_;
};

// The prefill kernel configurations (4 waves x 32 query rows, 64-key tiles):
// calls f(TileCfg<...>{}) for the (D, Dv) pair and returns its status, or
// FMHA_ERR_HEAD_DIM.  Head dim 64: the pipelined kernel (4 waves x 32 rows,
// 4-deep K and V rings, 64 KB, two workgroups per CU; 8 waves per workgroup
// measured 7 % slower on the causal B4 H16 S2048 prefill).  attn_fwd_kernel elsewhere: 2-stage
// LDS rings at head dim 128 (3 stages at 16 and 32); Q/K head dim 192 with
// V/O head dim 128: 2-stage K (24 KB tiles) and V (16 KB) rings, 80 KB.
template <class F>
fmha_status with_fwd_cfg(int D, int Dv, F&& f) {
  if (D == 192 && Dv == 128) return f(TileCfg<192, 32, 4, 64, 2, 2, false, 128>{});
  if (Dv == D) {
    switch (D) {
      case 16: return f(TileCfg<16, 32, 4, 64, 3, 3>{});
      case 32: return f(TileCfg<32, 32, 4, 64, 3, 3>{});
      case 64: return f(TileCfg<64, 32, 4, 64, 4, 4, false, 64, false, true>{});
      case 128: return f(TileCfg<128, 32, 4, 64, 2, 2>{});
    }
  }
  return FMHA_ERR_HEAD_DIM;
}

// The contiguous-cache decode kernel configurations (16-row waves), chosen by
// head dims, the row-count configuration c and whether V is the first Dv
// columns of the K rows (kv_shared); FMHA_ERR_HEAD_DIM if none is built.
//   576 / 512, V inside the K rows: one 4-deep ring of 32-key K tiles (144 KB);
//   576 / 512, separate V: 2-deep K and V rings (136 KB).
//   512, V aliasing K: one 5-deep ring of 32-key tiles (160 KB).
//   64 and 128 also come with split groups (GROUPS; see decode_groups_built);
//   128 with one wave: a 3-deep K ring, 40 KB, four workgroups per CU (2048
//   workgroups of the MHA decode then run in exactly two rounds).
template <class F>
fmha_status with_decode_cfg(int D, int Dv, DecodeCfg c, bool kv_shared, F&& f) {
  if (D == 576 && Dv == 512) {
    if (kv_shared) return f(TileCfg<576, 16, 4, 32, 4, 4, true, 512>{});
    return f(TileCfg<576, 16, 4, 32, 2, 2, false, 512>{});
  }
  if (Dv != D) return FMHA_ERR_HEAD_DIM;
  if (D == 512 && kv_shared) return f(TileCfg<512, 16, 4, 32, 5, 5, true>{});
  if (D == 64 && c.nw == 1) return f(TileCfg<64, 16, 1, 32, 3, 3, false, 64, true>{});
  if (D == 64 && c.nw == 4) return f(TileCfg<64, 16, 4, 64, 3, 3, false, 64, true>{});
  if (D == 128 && c.nw == 1) return f(TileCfg<128, 16, 1, 32, 3, 2, false, 128, true>{});
  if (D == 128 && c.nw == 4) return f(TileCfg<128, 16, 4, 64, 2, 2, false, 128, true>{});
  if (D == 512) return f(TileCfg<512, 16, 4, 32, 3, 2>{});
  return FMHA_ERR_HEAD_DIM;
}

// Compute units of the current device (cached).
int num_cus();

// fmha_prefill.hip: 128-row prefill workgroups (4 waves x 32 rows); the
// launcher sizes the grid (p.n_row_blocks row blocks of each unit).
fmha_status launch_fwd(int D, int Dv, const AttnParams& p, bool causal, hipStream_t st);

// fmha_decode.hip: split-KV decode (16-row waves) and the log-sum-exp combine.
// D: head dim of Q/K, Dv: of V/O; kv_shared: V is the first Dv columns of the
// K rows (p.v == p.k).
fmha_status launch_decode(int D, int Dv, DecodeCfg c, const AttnParams& p, dim3 grid,
                          bool causal, bool split, bool kv_shared, hipStream_t st);
// fmha_decode_wide.hip: the decode for V inside the K rows at head dims
// 512/512 and 576/512 (4 waves, each holding half of the head dims; no amax
// or NVFP4 epilogue).  decode_wide_takes: whether it serves such a call;
// dbg: the test-only score-storing build (non-causal, one split).
bool decode_wide_takes(int D, int Dv, int Sk, bool kv_shared);
fmha_status launch_decode_wide(int D, int Dv, const AttnParams& p, dim3 grid, bool causal,
                               bool split, bool dbg, hipStream_t st);
// The same decode reading K/V from a paged cache (p.seqlens, p.block_table set).
fmha_status launch_decode_paged(int D, DecodeCfg c, const AttnParams& p, dim3 grid, bool causal,
                                bool split, hipStream_t st);
// fmha_debug.hip: the same prefill (decode = false) or one-split decode
// kernels built with DBG_S (p.s_dbg, p.s_dbg_scale set), non-causal.
// (prefill: the grid is sized by the launcher as for launch_fwd)
fmha_status launch_debug_scores(int D, int Dv, DecodeCfg c, const AttnParams& p, dim3 grid,
                                bool decode, bool kv_shared, hipStream_t st);
fmha_status launch_combine(int D, const float* o_part, const float* lse_part, uint16_t* o,
                           float* lse, float* o_amax, uint8_t* fp4_codes, uint8_t* fp4_scales,
                           const float* fp4_gscale, long long nrows, int nsplit,
                           hipStream_t st);

}  // namespace fmha
