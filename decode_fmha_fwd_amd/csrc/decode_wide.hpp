// decode_wide.hpp -- split-KV decode for wide heads whose V lives in the K
// rows: V aliasing K at head dim 512, or V the first 512 columns of 576-wide
// K rows.  Each key row crosses HBM once and feeds both products.
//
// The arithmetic is that of attn_fwd_kernel (the feature list on the page
// "NVFP4-1.1_RAW_CUDA_CPP_APPROACH.md": QK on the matrix cores, online softmax
// with O rescale over KV tiles, PV, the correction epilogue, key ranges split
// over workgroups and merged by the combine kernel; head dim 512 is one of the
// blockers that page lists).  What differs is how a workgroup shares it out.
//
// Work split: a workgroup owns 64 query rows of one (batch, KV head, split)
// and runs 8 waves, four row groups of 16 rows times two halves.  Wave (g, h)
// computes the QK partial of rows 16g..16g+15 over half h of the Q/K head dim,
// and the PV product of the same rows for half h of the V/O columns.  The two
// waves of a row group add their QK partials through LDS (own + partner:
// float addition commutes, so both hold bit-identical scores) and run the
// same softmax, so each keeps half of Q and half of O in registers (96 VGPRs
// of state).  Two waves then share a SIMD and hide each other's LDS and MFMA
// latencies, where one 16-row wave holding all of Q and O (over 450
// registers) sat alone on its SIMD with every latency exposed.
//
// Per 32-key tile: barrier (the tile has landed; everyone is past the
// previous tile), QK partial with the copies of the tile three ahead (into
// the freed stage) spread between its LDS reads, partial to LDS, barrier,
// partner's partial and the first V^T reads from LDS, mask, softmax, PV.
// The ring is 4 tiles deep (128 KB at head dim 512, 144 KB at 576) plus
// 16 KB for the partials.  All 8 waves share the copies, buffer loads
// bounded by the split's key range (rows past it read as zeros, whole tiles
// past it cost no memory traffic).
#pragma once

#include <climits>

#include "attn_kernels.hpp"
#include "buffer_copy.hpp"

namespace fmha {

// 16-byte LDS write from inline asm (a compiler-visible LDS access after the
// asynchronous copies would make the compiler wait for every copy in flight).
template <uint32_t OFF>
__device__ inline void lds_write_b128_imm(uint32_t lds_addr, f32x4 v) {
  static_assert(OFF < 65536u, "DS offset field is 16 bits");
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(lds_addr), "v"(v), "i"(OFF));
}

// Whether the wide decode can take a call: its copy offsets are 32-bit byte
// offsets within one (batch, KV head) row range, tiles a few past the end
// included.
inline bool decode_wide_fits(int Sk, int D) {
  return ((long long)Sk + 256) * D * 2 < (1LL << 32);
}

// DBG_S (test builds only): as in attn_fwd_kernel, the summed score tiles
// times p.s_dbg_scale go to p.s_dbg [rows][Sk] before masking, and the
// kernel writes no output.
template <int D, int DV, bool CAUSAL, bool SPLIT, bool DBG_S = false>
__global__ __launch_bounds__(512) void decode_wide_kernel(AttnParams p) {
  using M = Mfma<16>;
  using Acc = M::Acc;
  constexpr int KT = 32;         // keys per tile
  constexpr int KST = 4;         // ring depth
  constexpr int DH = D / 2;      // Q/K head-dim columns of one wave
  constexpr int DVH = DV / 2;    // V/O columns of one wave
  constexpr int KSTEPS = DH / M::kK;
  constexpr int DBLK = DVH / 16;
  constexpr int KTILE = KT * D;  // elements of a tile
  // Tile copies: the tile's 1 KB chunks (64 lanes x 16 bytes) go round-robin
  // over the 8 waves, copy j of wave w being chunk 8 j + w (4 copies per
  // wave at head dim 512; at 576, 36 chunks: 5 for waves 0..3, 4 for 4..7).
  constexpr int kChunks = KT * D * 2 / 1024;
  constexpr int kMaxCopies = (kChunks + 7) / 8;
  static_assert(kChunks * 1024 == KT * D * 2, "a tile is whole 1 KB chunks");
  static_assert(DH % M::kK == 0 && DVH % 16 == 0 && DV <= D, "head-dim halves in whole steps");

  __shared__ __attribute__((aligned(16))) uint16_t ksm[KST][KTILE];
  // per wave: its QK partial, two 16-byte words per lane, lane-contiguous
  __shared__ __attribute__((aligned(16))) float xbuf[8][2][64][4];

  const int lane = threadIdx.x & 63;
  // (wave-uniform in scalar registers: branches on h are scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave & 3;  // row group: waves w and w + 4 share a SIMD
  const int h = wave >> 2;  // head-dim half
  const int qcol = lane & 15;
  const int kg = lane >> 4;

  // 1-D grid, row block slowest (as attn_fwd_kernel, without split groups)
  const int n_units = p.nsplit * p.Hkv * p.B;
  const int rb_rank = blockIdx.x / n_units;
  const int unit = blockIdx.x - rb_rank * n_units;
  const int rb = CAUSAL ? p.n_row_blocks - 1 - rb_rank : rb_rank;
  const int split = unit % p.nsplit;
  const int bk = unit / p.nsplit;
  const int kvh = bk % p.Hkv;
  const int b = bk / p.Hkv;
  const long long bh_kv = (long long)b * p.Hkv + kvh;
  const long long row_base = bh_kv * p.rows_per_kv;
  const int Sk = p.Sk;

  const int r_wg0 = rb * 64;
  const int r_wave0 = r_wg0 + rg * 16;
  const int my_r = r_wave0 + qcol;
  const bool row_ok = my_r < p.rows_per_kv;
  const int my_rc = row_ok ? my_r : p.rows_per_kv - 1;
  const int diag = Sk - p.Sq;  // causal: key j visible to row i iff j <= i + diag

  const int kbeg = split * p.split_len;
  int kend = min(Sk, kbeg + p.split_len);
  int wave_min_last = INT_MAX, wave_max_last = INT_MAX;
  if (CAUSAL) {
    const int r_end = min(p.rows_per_kv, r_wg0 + 64) - 1;
    const int i_last = (r_wg0 / p.Sq == r_end / p.Sq) ? r_end % p.Sq : p.Sq - 1;
    kend = min(kend, i_last + diag + 1);
    if (r_wave0 < p.rows_per_kv) {
      const int rw_end = min(p.rows_per_kv, r_wave0 + 16) - 1;
      const bool one_head = (r_wave0 / p.Sq == rw_end / p.Sq);
      wave_min_last = (one_head ? r_wave0 % p.Sq : 0) + diag;
      wave_max_last = (one_head ? rw_end % p.Sq : p.Sq - 1) + diag;
    } else {
      wave_min_last = wave_max_last = -1;
    }
  }
  const int my_last = CAUSAL ? (my_rc % p.Sq) + diag : INT_MAX;
  const int ntiles = (kend > kbeg) ? (kend - kbeg + KT - 1) / KT : 0;

  // The split's key rows, bounded: reads past kend return zeros.
  const uint16_t* kbase = p.k + ((long long)bh_kv * Sk + kbeg) * D;
  const uint32_t kbytes = (uint32_t)max(kend - kbeg, 0) * (uint32_t)(D * 2);
  FMHA_LDS char* ring = (FMHA_LDS char*)&ksm[0][0];
  const int n_copies = (kChunks - wave + 7) / 8;  // this wave's copies per tile
  uint32_t cvoff[kMaxCopies];  // a lane's byte offset in the tile, swizzled
#pragma unroll
  for (int j = 0; j < kMaxCopies; ++j) {
    const int byte = (8 * j + wave) * 1024 + lane * 16;
    const int row = byte / (D * 2);
    const int pchunk = (byte - row * D * 2) >> 4;
    cvoff[j] = (uint32_t)(row * D * 2 + ((pchunk ^ swz<D / 8>(row)) << 4));
  }
  // copies [J0, J1) of this wave for tile t
  auto issue = [&](int t, auto j0_c, auto j1_c) {
    static_for<decltype(j0_c)::value, decltype(j1_c)::value>([&](auto j_c) {
      constexpr int J = decltype(j_c)::value;
      if (J < kMaxCopies - 1 || 8 * J + wave < kChunks)
        buffer_load_lds16<2>(kbase, kbytes, (FMHA_LDS void*)(ring + (t & 3) * (KTILE * 2) +
                                                              (8 * J + wave) * 1024),
                             (uint32_t)t * (uint32_t)(KT * D * 2) + cvoff[J]);
    });
  };
  using C0 = std::integral_constant<int, 0>;
  using CAll = std::integral_constant<int, kMaxCopies>;

  // Prologue: tile 0, then this wave's half of the Q^T fragments, then tiles
  // 1 and 2.  The wait for Q (it is needed from the first tile on) then
  // covers only tile 0 besides, which the first tile needs as well.
  issue(0, C0{}, CAll{});
  u32x4 qf[KSTEPS];
  {
    const uint16_t* qrow = p.q + (row_base + my_rc) * D + h * DH + 8 * kg;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *(const u32x4*)(qrow + s * M::kK);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) asm volatile("; q ready" : "+v"(qf[s]));
  }
  issue(1, C0{}, CAll{});
  issue(2, C0{}, CAll{});

  // Per-lane LDS offsets (bytes).  The swizzle repeats every 2^KSW chunks of a
  // row and every 16 rows, so whole periods of columns and whole 16-key
  // blocks are instruction immediates.
  constexpr int KSW = CPR_LOG2<D / 8>::value;
  constexpr int KPER_RAW = (1 << KSW) / (M::kK / 8);  // k-steps per swizzle period
  constexpr int KPER = KPER_RAW < 1 ? 1 : (KPER_RAW > KSTEPS ? KSTEPS : KPER_RAW);
  constexpr int VPER_RAW = (1 << KSW) / 2;            // 16-column blocks per period
  constexpr int VPER = VPER_RAW > DBLK ? DBLK : VPER_RAW;
  uint32_t koff[KPER];
#pragma unroll
  for (int s = 0; s < KPER; ++s) koff[s] = 2u * tile_off<D>(qcol, h * DH + s * M::kK + 8 * kg);
  uint32_t voff[VPER];
  {
    // V^T through transpose reads: k-slots 0..3 <-> keys 4g + 0..3, 4..7 <->
    // keys 16 + 4g + 0..3 (g = lane / 16), matching the S^T register layout
    const int grp = lane >> 4, tj = (lane >> 2) & 3, ta = lane & 3;
#pragma unroll
    for (int db = 0; db < VPER; ++db)
      voff[db] = 2u * tile_off<D>(4 * grp + tj, h * DVH + db * 16 + 4 * ta);
  }
  const uint32_t k_lds = lds_addr((const FMHA_LDS void*)&ksm[0][0]);
  const uint32_t x_own = lds_addr((const FMHA_LDS void*)&xbuf[wave][0][lane][0]);
  const uint32_t x_par = lds_addr((const FMHA_LDS void*)&xbuf[wave ^ 4][0][lane][0]);

  Acc oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = Acc{};
  float m_run = kNegBig;
  float l_run = 0.0f;

  for (int t = 0; t < ntiles; ++t) {
    const int t0 = kbeg + t * KT;
    // Tile t has landed (t+1 and t+2 may still fly), every wave is past its
    // reads of tile t-1 and of the partials, and then everyone's copies of
    // tile t are visible.
    if (n_copies == kMaxCopies)
      wait_vmcnt<2 * kMaxCopies>();
    else
      wait_vmcnt<2 * (kMaxCopies - 1)>();
    wait_lgkmcnt0();
    lds_barrier();
    // (the copies of tile t+3, into the stage of tile t-1, are spread over
    // the QK block below)
    const uint32_t kst = k_lds + (uint32_t)(t & 3) * (uint32_t)(KTILE * 2);
    // causal: a tile past the last visible key of both waves' rows
    const bool skip = CAUSAL && t0 > wave_max_last;

    Acc s_own[2];
    if (!skip) {
      // ---- partial S^T = K_h Q_h^T, K read one chunk of QCH steps ahead;
      // even and odd steps in two accumulators ----
      constexpr int QCH = 3;
      constexpr int NQC = (KSTEPS + QCH - 1) / QCH;
      u32x4 kf[NQC][2][QCH];
      Acc sa[2] = {Acc{}, Acc{}}, sb[2] = {Acc{}, Acc{}};
      auto read_k = [&](auto c_c) {
        constexpr int C = decltype(c_c)::value;
        static_for<0, 2 * QCH>([&](auto j_c) {
          constexpr int J = decltype(j_c)::value;
          constexpr int kb = J / QCH, i = J % QCH, s = C * QCH + i;
          if constexpr (s < KSTEPS) {
            constexpr uint32_t imm = 2u * (kb * 16 * D + (s / KPER) * KPER * M::kK);
            kf[C][kb][i] = lds_read_b128_imm<imm>(kst + koff[s % KPER]);
          }
        });
      };
      read_k(std::integral_constant<int, 0>{});
      static_for<0, NQC>([&](auto c_c) {
        constexpr int C = decltype(c_c)::value;
        issue(t + 3, std::integral_constant<int, C * kMaxCopies / NQC>{},
              std::integral_constant<int, (C + 1) * kMaxCopies / NQC>{});
        if constexpr (C + 1 < NQC) read_k(std::integral_constant<int, C + 1>{});
        constexpr int rest = KSTEPS - (C + 1) * QCH;
        constexpr int kNext = (C + 1 < NQC) ? 2 * (rest < QCH ? rest : QCH) : 0;
        lds_wait<kNext>();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < QCH; ++i)
            if (C * QCH + i < KSTEPS) lds_tie(kf[C][kb][i]);
#pragma unroll
        for (int i = 0; i < QCH; ++i)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int s = C * QCH + i;
            if (s < KSTEPS) {
              const bf16x8 a = __builtin_bit_cast(bf16x8, kf[C][kb][i]);
              const bf16x8 q = __builtin_bit_cast(bf16x8, qf[s]);
              if (s & 1)
                sb[kb] = M::run(a, q, sb[kb]);
              else
                sa[kb] = M::run(a, q, sa[kb]);
            }
          }
      });
      s_own[0] = sa[0] + sb[0];
      s_own[1] = sa[1] + sb[1];
      lds_write_b128_imm<0>(x_own, s_own[0]);
      lds_write_b128_imm<1024>(x_own, s_own[1]);
    } else {
      issue(t + 3, C0{}, CAll{});
    }
    wait_lgkmcnt0();
    lds_barrier();
    if (skip) continue;

    // ---- S = own + partner partial; the first V^T reads of the PV block go
    // out with the partner read, so they land during the softmax ----
    constexpr int RA = 6;  // 16-column blocks of V^T read ahead (two reads each)
    u32x4 vfrag[DBLK];
    auto read_v = [&](auto u_c) {
      constexpr int U = decltype(u_c)::value;
      constexpr uint32_t lo = 2u * ((U / VPER) * VPER * 16);
      constexpr uint32_t hi = lo + 2u * 16 * D;  // keys 16..31
      const u32x2 a = lds_read_tr16_imm<lo>(kst + voff[U % VPER]);
      const u32x2 c = lds_read_tr16_imm<hi>(kst + voff[U % VPER]);
      vfrag[U] = u32x4{a[0], a[1], c[0], c[1]};
    };
    Acc sc[2];
    {
      u32x4 pa = lds_read_b128_imm<0>(x_par);
      u32x4 pb = lds_read_b128_imm<1024>(x_par);
      static_for<0, RA>([&](auto u_c) { read_v(u_c); });
      lds_wait_tied<2 * RA + 1>(pa);
      sc[0] = s_own[0] + __builtin_bit_cast(f32x4, pa);
      lds_wait_tied<2 * RA>(pb);
      sc[1] = s_own[1] + __builtin_bit_cast(f32x4, pb);
    }
    if constexpr (DBG_S) {
      if (h == 0 && row_ok) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = t0 + kb * 16 + acc_row<16>(lane, r);
            if (key < kend)
              p.s_dbg[(row_base + my_r) * (long long)Sk + key] = sc[kb][r] * p.s_dbg_scale;
          }
      }
    }

    // ---- mask the ragged end and the causal diagonal ----
    if ((t0 + KT > kend) || (CAUSAL && t0 + KT - 1 > wave_min_last)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = t0 + kb * 16 + acc_row<16>(lane, r);
          if (key >= kend || key > my_last) sc[kb][r] = -__builtin_inff();
        }
    }

    // ---- online softmax (base 2) with lazy rescaling ----
    float mloc = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, sc[kb][r]);
    mloc = group_max<16>(mloc) * p.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mloc > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) oacc[i] *= alpha;
    }
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = fast_exp2(__builtin_fmaf(sc[kb][r], p.scale_log2, -m_run));
        sc[kb][r] = pv;
        psum += pv;
      }
    l_run += psum;

    // ---- O_h^T += V_h^T P^T: one 32-deep MFMA per 16-column block ----
    u32x4 pw;
    pw[0] = pack_bf16x2(sc[0][0], sc[0][1]);
    pw[1] = pack_bf16x2(sc[0][2], sc[0][3]);
    pw[2] = pack_bf16x2(sc[1][0], sc[1][1]);
    pw[3] = pack_bf16x2(sc[1][2], sc[1][3]);
    const bf16x8 pbf = __builtin_bit_cast(bf16x8, pw);
    static_for<0, DBLK>([&](auto u_c) {
      constexpr int U = decltype(u_c)::value;
      if constexpr (U + RA < DBLK) read_v(std::integral_constant<int, U + RA>{});
      constexpr int pending = 2 * ((DBLK - 1 - U) < RA ? (DBLK - 1 - U) : RA);
      lds_wait_tied<pending>(vfrag[U]);
      oacc[U] = M::run(__builtin_bit_cast(bf16x8, vfrag[U]), pbf, oacc[U]);
    });
  }
  // the copies past the last tile (zeros) land before the LDS is released
  wait_vmcnt<0>();

  if constexpr (DBG_S) return;

  // ---- epilogue: this wave's half of O / l; lse from half 0 ----
  const float l_tot = group_sum<16>(l_run);
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l_tot;
  const float lse_val = empty ? -__builtin_inff() : (m_run + __log2f(l_tot)) * kLn2;
  if (row_ok) {
    const long long row = row_base + my_r;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int d0 = h * DVH + db * 16 + 4 * kg;
      const float o0 = oacc[db][0] * inv, o1 = oacc[db][1] * inv;
      const float o2 = oacc[db][2] * inv, o3 = oacc[db][3] * inv;
      if constexpr (SPLIT) {
        *(f32x4*)(p.o_part + (row * p.nsplit + split) * DV + d0) = f32x4{o0, o1, o2, o3};
      } else {
        *(u32x2*)(p.o + row * DV + d0) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
      }
    }
    if (h == 0 && kg == 0) {
      if constexpr (SPLIT) {
        p.lse_part[row * p.nsplit + split] = lse_val;
      } else {
        if (p.lse) p.lse[row] = lse_val;
      }
    }
  }
}

}  // namespace fmha
