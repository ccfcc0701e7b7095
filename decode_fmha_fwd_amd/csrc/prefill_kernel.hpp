// prefill_kernel.hpp -- the software-pipelined prefill attention kernel for
// gfx950 (32-row waves, 64-key tiles, head dim 64).
//
// What it computes is the attention of attn_kernels.hpp (the feature list on
// the page "NVFP4-1.1_RAW_CUDA_CPP_APPROACH.md": QK product, in-kernel softmax
// with O rescale over several KV tiles, PV product, correction epilogue); how
// it is scheduled differs:
//
//   * One workgroup = NW waves x 32 query rows that share a KV head (NW = 4:
//     64 KB of LDS, two workgroups per CU, two waves per SIMD; eight-wave
//     workgroups filling a CU alone measured 7 % slower).  Row blocks are
//     paired heaviest with lightest (see the grid below), and the waves'
//     priority falls with their workgroup's progress, so the two workgroups
//     of a CU finish close together (see progress() below).
//   * Software pipeline across KV tiles inside each wave: iteration j issues
//     the QK product of tile j+1 and the PV product of tile j-1 on the matrix
//     cores while the VALU computes the softmax of tile j.  The three are
//     independent, so a wave keeps the matrix cores fed by itself instead of
//     serialising QK -> softmax -> PV.
//   * The exponentials are taken against the running maximum m without first
//     computing the tile's maximum.  Because p = 2^(s c - m) <= (the lane's
//     sum of p), a wave-wide test of the lane sums against a bound catches
//     every tile that could overflow (and the first tile, where m is still
//     the "no score yet" stand-in); only those take the exact path, which
//     computes the row maximum, rescales O and l and recomputes P.  The final
//     O / l and the log-sum-exp do not depend on which m was subtracted.
//   * K and V tiles stream into 4-deep LDS rings through buffer loads with
//     the LDS bit (buffer_load_dwordx4 ... lds): one descriptor per row block
//     bounds the copies, a copy's lane offset is a fixed per-lane value plus
//     the tile's offset, and rows past the end of the keys read as zeros
//     (masked anyway).
//   * K operand reads, V transpose reads and their waits are inline asm, as in
//     attn_kernels.hpp, so the compiler never drains the copy ring to order a
//     plain LDS read after the asynchronous copies; the build checks the
//     assembly for any use of such a read's result before its wait.
#pragma once

#include <climits>
#include <type_traits>

#include "attn_kernels.hpp"
#include "buffer_copy.hpp"

namespace fmha {

// Bound on a lane's sum of p over one tile for the unchecked exponentials
// (2^16: at most ~16 log2 units above the running maximum).
constexpr float kPsumLimit = 65536.0f;

template <int D, int DV, int NW, bool CAUSAL, bool DBG_S = false>
__global__ __launch_bounds__(NW * 64)
void prefill_kernel(AttnParams p) {
  constexpr int MT = 32, KT = 64, KBLK = KT / MT;
  constexpr int KSTEPS = D / 16, DBLK = DV / 32, NPV = 2 * KBLK;
  // 4-deep K and V rings: iteration j reads K(j+1) and V(j-1) while K(j+3)
  // and V(j+1) are copied in, and K(j) stays resident through iteration j
  // (the fast path's fallback recomputes its scores).
  constexpr int KST = 4, VST = 4;
  // Tile t sits in ring stage (t - 1) & 3, so that iteration 1, where the
  // steady-state loop starts, has phase 0 (see the loop below).
  auto stage_of = [](int t) { return (t + 3) & 3; };
  constexpr int KTILE = KT * D, VTILE = KT * DV;
  using M = Mfma<32>;
  using Acc = f32x16;
  using CopyK = BufTileCopy<D, NW, KT>;
  using CopyV = BufTileCopy<DV, NW, KT>;
  constexpr int nK = CopyK::kLoads, nV = CopyV::kLoads;
  static_assert(D % 32 == 0 && DV % 32 == 0, "head dims in whole 32-wide blocks");
  static_assert((KST & (KST - 1)) == 0 && (VST & (VST - 1)) == 0, "ring depths: powers of two");

  // V ring first, then the K ring (byte offsets below 64 KiB throughout).
  __shared__ __attribute__((aligned(16))) uint16_t vsm[VST][VTILE];
  __shared__ __attribute__((aligned(16))) uint16_t ksm[KST][KTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Grid: row-block slot slowest, then the (batch, KV head) unit.  With one
  // row block per workgroup, slot s takes the s-th longest (causal) row
  // block, so the longest are dispatched first.  With two (p.rb_per_wg == 2,
  // when the grid would take two or more rounds of the GPU's workgroup
  // slots), slot s takes row blocks n-1-s and s of its unit one after the
  // other: under a causal mask every pair then costs the same (n + 1 tiles
  // of 128 rows), and the workgroups of one round stay resident until all
  // are done, with no dispatch gap between rounds.  A unit's row blocks sit
  // on one XCD (the unit count is a multiple of 8 in the usual shapes and
  // workgroups go round-robin over the 8 XCDs), so their K/V re-reads share
  // its L2.
  const int n_units = p.Hkv * p.B;
  const int slot = blockIdx.x / n_units;
  const int unit = blockIdx.x - slot * n_units;
  const int kvh = unit % p.Hkv;
  const int b = unit / p.Hkv;
  const long long bh_kv = (long long)b * p.Hkv + kvh;
  const int Sk = p.Sk;
  const long long row_base = bh_kv * p.rows_per_kv;
  const bool paired = p.rb_per_wg == 2;
  const int n_blocks = (paired && p.n_row_blocks - 1 - slot != slot) ? 2 : 1;

  // Progress-based wave priority.  Two workgroups share a CU, and the issue
  // arbiter favours the older one's waves at equal priority, so it pulls ahead
  // and the other finishes alone, one wave per SIMD.  Every wave starts at
  // priority 3 and steps down as its workgroup passes 1/2, 4/5 and 19/20 of
  // its tiles: the workgroup that is behind wins the arbitration until it has
  // caught up (measured 1-3 % faster, outputs bit-identical).
  auto tiles_of = [&](int blk) {
    const int rb = paired ? (blk == 0 ? p.n_row_blocks - 1 - slot : slot)
                          : (CAUSAL ? p.n_row_blocks - 1 - slot : slot);
    const int r_wg0 = rb * (NW * MT);
    int kend = Sk;
    if (CAUSAL) {
      const int diag = Sk - p.Sq;
      const int r_end = min(p.rows_per_kv, r_wg0 + NW * MT) - 1;
      const int i_last = (r_wg0 / p.Sq == r_end / p.Sq) ? r_end % p.Sq : p.Sq - 1;
      kend = min(kend, i_last + diag + 1);
    }
    return (kend + KT - 1) / KT;
  };
  int total_tiles = 0;
  for (int b2 = 0; b2 < n_blocks; ++b2) total_tiles += tiles_of(b2);
  total_tiles = max(total_tiles, 1);
  int done_tiles = 0, prio = 3;
  __builtin_amdgcn_s_setprio(3);
  auto progress = [&](int n) {
    done_tiles += n;
    const int lv = 3 - (20 * done_tiles >= 10 * total_tiles) -
                   (20 * done_tiles >= 16 * total_tiles) - (20 * done_tiles >= 19 * total_tiles);
    if (lv < prio) {
      prio = lv;
      if (lv == 2) __builtin_amdgcn_s_setprio(2);
      else if (lv == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
  };
  for (int blk = 0; blk < n_blocks; ++blk) {
    const int rb = paired ? (blk == 0 ? p.n_row_blocks - 1 - slot : slot)
                          : (CAUSAL ? p.n_row_blocks - 1 - slot : slot);
    if (blk > 0) {  // every wave is past its reads of the previous row block
      wait_lgkmcnt0();
      lds_barrier();
    }

    const int r_wg0 = rb * (NW * MT);
    const int r_wave0 = r_wg0 + wave * MT;
    const int qcol = lane % MT;
    const int kg = lane / MT;
    const int my_r = r_wave0 + qcol;
    const bool row_ok = my_r < p.rows_per_kv;
    const int my_rc = row_ok ? my_r : p.rows_per_kv - 1;
    const int diag = Sk - p.Sq;

    int kend = Sk;
    int wave_min_last = INT_MAX;  // smallest last-visible key over the wave's rows
    if (CAUSAL) {
      const int r_end = min(p.rows_per_kv, r_wg0 + NW * MT) - 1;
      const int i_last = (r_wg0 / p.Sq == r_end / p.Sq) ? r_end % p.Sq : p.Sq - 1;
      kend = min(kend, i_last + diag + 1);
      if (r_wave0 < p.rows_per_kv) {
        const int rw_end = min(p.rows_per_kv, r_wave0 + MT) - 1;
        const bool one_head = (r_wave0 / p.Sq == rw_end / p.Sq);
        wave_min_last = (one_head ? r_wave0 % p.Sq : 0) + diag;
      } else {
        wave_min_last = -1;
      }
    }
    const int my_last = CAUSAL ? (my_rc % p.Sq) + diag : INT_MAX;
    const int ntiles = (kend + KT - 1) / KT;
    // the leading tiles this wave needs no mask on
    int n_clean = kend / KT;
    if (r_wave0 >= p.rows_per_kv) n_clean = 0;
    else if (CAUSAL) n_clean = min(kend, wave_min_last + 1) / KT;

    // ---- copies ----
    CopyK ck;
    CopyV cv;
    ck.init(wave, lane);
    cv.init(wave, lane);
    const uint16_t* kbase = p.k + bh_kv * (long long)Sk * D;
    const uint16_t* vbase = p.v + bh_kv * (long long)Sk * DV;
    // A tile's copies read the keys below kend only (no row of the workgroup
    // sees a later one): rows from kend on, and whole tiles past the last,
    // read as zeros without touching memory.  Every iteration issues the same
    // copies, so every wait below is a constant count.
    // (the host keeps a head's K and V rows below 4 GiB, so the 32-bit buffer
    // offsets of every tile, and of the zero-filled tiles past the keys, fit)
    // (stage: t's ring stage, t & 3, passed in so that a compile-time
    // constant reaches the LDS destination)
    auto issue_k = [&](int t, int stage) {
      ck.issue(kbase, (uint32_t)kend * (D * 2), (uint32_t)t * (KT * D * 2),
               (FMHA_LDS char*)&ksm[stage][0], wave);
    };
    auto issue_v = [&](int t, int stage) {
      cv.issue(vbase, (uint32_t)kend * (DV * 2), (uint32_t)t * (KT * DV * 2),
               (FMHA_LDS char*)&vsm[stage][0], wave);
    };

    // Q first (the compiler's wait for it then leaves the copies in flight),
    // then the prologue copies K0 V0 K1 K2; iteration j issues K(j+3), V(j+1)
    bf16x8 qf[KSTEPS];
    load_q_frags<D, MT>(p.q + (row_base + my_rc) * D, kg, qf);
    issue_k(0, stage_of(0));
    issue_v(0, stage_of(0));
    issue_k(1, stage_of(1));
    issue_k(2, stage_of(2));

    // per-lane LDS offsets (constant over the loop; see attn_kernels.hpp)
    constexpr int KSW = CPR_LOG2<D / 8>::value;
    constexpr int KPER_RAW = (1 << KSW) / 2;
    constexpr int KPER = KPER_RAW < 1 ? 1 : (KPER_RAW > KSTEPS ? KSTEPS : KPER_RAW);
    constexpr int VSW = CPR_LOG2<DV / 8>::value;
    constexpr int VPER_RAW = (1 << VSW) / 4;
    constexpr int VPER = VPER_RAW < 1 ? 1 : (VPER_RAW > DBLK ? DBLK : VPER_RAW);
    uint32_t koff[KPER];
#pragma unroll
    for (int s = 0; s < KPER; ++s) koff[s] = 2u * tile_off<D>(lane % MT, s * 16 + 8 * kg);
    uint32_t voff0[VPER], voff1[VPER];
    {
      const int grp = lane >> 4, tj = (lane >> 2) & 3, ta = lane & 3;
#pragma unroll
      for (int db = 0; db < VPER; ++db) {
        const int col = db * 32 + 16 * (grp & 1) + 4 * ta;
        const int row1 = 4 * (grp >> 1) + tj;
        voff0[db] = 2u * tile_off<DV>(row1, col);
        voff1[db] = 2u * tile_off<DV>(row1 + 8, col);
      }
    }
    const uint32_t k_lds = lds_addr((const FMHA_LDS void*)&ksm[0][0]);
    const uint32_t v_lds = lds_addr((const FMHA_LDS void*)&vsm[0][0]);

    Acc oacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = Acc{};
    float m_run = kNegBig;
    float l_run = 0.0f;
    const float c = p.scale_log2;

    Acc sbuf[2][KBLK];      // raw scores of tiles j (cur) and j+1 (next)
    u32x4 pbuf[2][NPV];     // packed bf16 P of tiles j and j-1

    // QK product of tile t into S: K fragments read from LDS (asm) two
    // contraction steps ahead of the MFMAs that use them.
    auto qk = [&](int t, Acc (&S)[KBLK]) {
      const uint32_t kst = k_lds + (uint32_t)stage_of(t) * (KTILE * 2);
      constexpr int KRA = KSTEPS < 2 ? KSTEPS : 2;  // steps read ahead
      u32x4 kf[KSTEPS][KBLK];
      auto read = [&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        static_for<0, KBLK>([&](auto kb_c) {
          constexpr int kb = decltype(kb_c)::value;
          constexpr uint32_t imm = 2u * (kb * MT * D + (s / KPER) * KPER * 16);
          kf[s][kb] = lds_read_b128_imm<imm>(kst + koff[s % KPER]);
        });
      };
      static_for<0, KRA>([&](auto s_c) { read(s_c); });
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) S[kb] = Acc{};
      static_for<0, KSTEPS>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        // reads issued after step s's: those of steps s+1 .. min(s+KRA-1, last)
        constexpr int ahead = (KSTEPS - 1 - s) < (KRA - 1) ? (KSTEPS - 1 - s) : (KRA - 1);
        lds_wait<ahead * KBLK>();
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) lds_tie(kf[s][kb]);
        if constexpr (s + KRA < KSTEPS) read(std::integral_constant<int, s + KRA>{});
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb)
          S[kb] = M::run(__builtin_bit_cast(bf16x8, kf[s][kb]), qf[s], S[kb]);
      });
    };

    // PV product of tile t with packed P: V^T through transpose reads (asm),
    // RA units (one MFMA each) ahead of the MFMAs.
    auto pv = [&](int t, const u32x4 (&P)[NPV]) {
      const uint32_t vst = v_lds + (uint32_t)stage_of(t) * (VTILE * 2);
      constexpr int NU = NPV * DBLK;
      constexpr int RA = NU < 4 ? NU : 4;
      u32x4 vfrag[NU];
      auto read = [&](auto u_c) {
        constexpr int U = decltype(u_c)::value;
        constexpr int step = U / DBLK, db = U % DBLK;
        constexpr uint32_t imm = step * (16u * DV * 2) + (uint32_t)(db / VPER) * VPER * MT * 2;
        const u32x2 lo = lds_read_tr16_imm<imm>(vst + voff0[db % VPER]);
        const u32x2 hi = lds_read_tr16_imm<imm>(vst + voff1[db % VPER]);
        vfrag[U] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      static_for<0, RA>([&](auto u_c) { read(u_c); });
      static_for<0, NU>([&](auto u_c) {
        constexpr int U = decltype(u_c)::value;
        constexpr int ahead = (NU - 1 - U) < (RA - 1) ? (NU - 1 - U) : (RA - 1);
        lds_wait_tied<2 * ahead>(vfrag[U]);
        if constexpr (U + RA < NU) read(std::integral_constant<int, U + RA>{});
        oacc[U % DBLK] = M::run(__builtin_bit_cast(bf16x8, vfrag[U]),
                                __builtin_bit_cast(bf16x8, P[U / DBLK]), oacc[U % DBLK]);
      });
    };

    // Softmax of one tile's scores S (already masked): P (packed bf16), the
    // running m / l updated; O rescaled when the exact path moves m.
    auto pack = [&](const Acc (&pv_)[KBLK], u32x4 (&P)[NPV]) {
#pragma unroll
      for (int step = 0; step < NPV; ++step) {
        const int kb = step >> 1, t2 = step & 1;
        P[step] = u32x4{pack_bf16x2(pv_[kb][8 * t2 + 0], pv_[kb][8 * t2 + 1]),
                        pack_bf16x2(pv_[kb][8 * t2 + 2], pv_[kb][8 * t2 + 3]),
                        pack_bf16x2(pv_[kb][8 * t2 + 4], pv_[kb][8 * t2 + 5]),
                        pack_bf16x2(pv_[kb][8 * t2 + 6], pv_[kb][8 * t2 + 7])};
      }
    };
    // Exact softmax of a tile (masked tiles, the first tile, and the fallback
    // of the fast path): the tile's row maximum first; m moves (and O, l are
    // rescaled) when some row's maximum exceeds it; P computed in place.
    auto softmax_exact = [&](Acc (&S)[KBLK], u32x4 (&P)[NPV]) {
      float mloc = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, S[kb][r]);
      mloc = group_max<MT>(mloc) * c;
      if (__builtin_amdgcn_ballot_w64(mloc > m_run) != 0) {
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DBLK; ++i) oacc[i] *= alpha;
      }
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          S[kb][r] = fast_exp2(__builtin_fmaf(S[kb][r], c, -m_run));
          ps += S[kb][r];
        }
      pack(S, P);
      l_run += ps;
    };
    // Fast softmax of an unmasked tile against the running maximum, P computed
    // in place (the raw scores are consumed); false when some lane's sum of p
    // is beyond kPsumLimit (or not finite): the caller then recomputes the
    // scores and takes the exact path.
    auto softmax_fast = [&](Acc (&S)[KBLK], u32x4 (&P)[NPV]) {
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          S[kb][r] = fast_exp2(__builtin_fmaf(S[kb][r], c, -m_run));
          ps += S[kb][r];
        }
      pack(S, P);
      if (__builtin_amdgcn_ballot_w64(!(ps <= kPsumLimit)) != 0) return false;
      l_run += ps;
      return true;
    };

    // Causal diagonal and ragged end: key t0 + (its row in the tile) is
    // visible iff it is <= lim, the lane row's last visible key (kend - 1 at
    // most); the row of accumulator register r of key block kb is a constant
    // plus 4 (lane / 32), so one compare per score.
    const int lim = min(my_last, kend - 1) - 4 * kg;
    auto mask = [&](Acc (&S)[KBLK], int t) {
      const int d = lim - t * KT;
      static_for<0, KBLK * 16>([&](auto i_c) {
        constexpr int kb = decltype(i_c)::value / 16, r = decltype(i_c)::value % 16;
        constexpr int row = kb * MT + 8 * (r >> 2) + (r & 3);
        if (row > d) S[kb][r] = -__builtin_inff();
      });
    };

    // The steady-state iteration at head dim 64 written as eight chunks, each
    // two MFMAs (QK of tile j+1 and PV of tile j-1 alternately) plus the fast
    // softmax of four scores of tile j, with scheduling barriers between the
    // chunks so the compiler keeps the interleave: a wave then issues its VALU
    // work while its own MFMAs run.  The LDS reads of each chunk's operands are
    // issued a chunk ahead (in-order lgkmcnt waits below).  Returns false when
    // the fast softmax's bound test fails (as softmax_fast).
    // MASK: tile j crosses the causal diagonal or the ragged end; each score
    // past the lane row's last visible key gets p = 0 (see mask()).
    // PH: the phase (j - 1) & 3 when known at compile time (the ring stages
    // then travel as instruction immediates), else negative (stages from j at
    // run time).  Stage of tile j + 1: PH + 1; of tile j - 1: PH - 1 (mod 4).
    auto full_interleaved = [&](auto mask_c, auto ph_c, int j, Acc (&Sn)[KBLK],
                                const u32x4 (&Pp)[NPV], Acc (&Sc)[KBLK], u32x4 (&Pc)[NPV]) {
      constexpr bool MASK = decltype(mask_c)::value;
      constexpr int PH = decltype(ph_c)::value;
      const int d = lim - j * KT;
      static_assert(KSTEPS == 4 && KBLK == 2 && DBLK == 2, "the chunk plan is for D = DV = 64");
      constexpr uint32_t kimm0 = PH >= 0 ? (uint32_t)((PH + 1) & 3) * (KTILE * 2) : 0u;
      constexpr uint32_t vimm0 = PH >= 0 ? (uint32_t)((PH + 3) & 3) * (VTILE * 2) : 0u;
      const uint32_t kst = k_lds + (PH >= 0 ? 0u : (uint32_t)stage_of(j + 1) * (KTILE * 2));
      const uint32_t vst = v_lds + (PH >= 0 ? 0u : (uint32_t)stage_of(j - 1) * (VTILE * 2));
      u32x4 kf[KSTEPS][KBLK];
      u32x4 vfrag[8];
      auto read_k = [&](auto s_c) {
        constexpr int s_ = decltype(s_c)::value;
        static_for<0, KBLK>([&](auto kb_c) {
          constexpr int kb = decltype(kb_c)::value;
          constexpr uint32_t imm = kimm0 + 2u * (kb * MT * D + (s_ / KPER) * KPER * 16);
          kf[s_][kb] = lds_read_b128_imm<imm>(kst + koff[s_ % KPER]);
        });
      };
      auto read_v = [&](auto u_c) {
        constexpr int U = decltype(u_c)::value;
        constexpr int step = U / DBLK, db = U % DBLK;
        constexpr uint32_t imm =
            vimm0 + step * (16u * DV * 2) + (uint32_t)(db / VPER) * VPER * MT * 2;
        const u32x2 lo = lds_read_tr16_imm<imm>(vst + voff0[db % VPER]);
        const u32x2 hi = lds_read_tr16_imm<imm>(vst + voff1[db % VPER]);
        vfrag[U] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) Sn[kb] = Acc{};
      float ps = 0.0f;
      read_k(std::integral_constant<int, 0>{});
      read_v(std::integral_constant<int, 0>{});
      read_v(std::integral_constant<int, 1>{});
      static_for<0, 8>([&](auto c_c) {
        constexpr int C = decltype(c_c)::value;
        if constexpr (C % 2 == 0) {  // QK step C/2 (V reads of the next PV pair after it)
          constexpr int s_ = C / 2;
          lds_wait<4>();  // the two V reads issued after K(s_) may fly
#pragma unroll
          for (int kb = 0; kb < KBLK; ++kb) lds_tie(kf[s_][kb]);
          if constexpr (s_ + 1 < KSTEPS) read_k(std::integral_constant<int, s_ + 1>{});
#pragma unroll
          for (int kb = 0; kb < KBLK; ++kb)
            Sn[kb] = M::run(__builtin_bit_cast(bf16x8, kf[s_][kb]), qf[s_], Sn[kb]);
        } else {  // PV units C-1, C
          constexpr int U = C - 1;
          lds_wait<(C < 7 ? 2 : 0)>();
          lds_tie(vfrag[U]);
          lds_tie(vfrag[U + 1]);
          if constexpr (U + 2 < 8) {
            read_v(std::integral_constant<int, U + 2>{});
            read_v(std::integral_constant<int, U + 3>{});
          }
          oacc[U % DBLK] = M::run(__builtin_bit_cast(bf16x8, vfrag[U]),
                                  __builtin_bit_cast(bf16x8, Pp[U / DBLK]), oacc[U % DBLK]);
          oacc[(U + 1) % DBLK] = M::run(__builtin_bit_cast(bf16x8, vfrag[U + 1]),
                                        __builtin_bit_cast(bf16x8, Pp[(U + 1) / DBLK]),
                                        oacc[(U + 1) % DBLK]);
        }
        // softmax of scores Sc[C / 4][4 (C % 4) .. +3] -> two packed pairs of P
        constexpr int kb = C / 4, r0 = 4 * (C % 4);
        constexpr int step = 2 * kb + (C % 4) / 2, i0 = 2 * (C % 2);
        float e[4];
        static_for<0, 4>([&](auto r_c) {
          constexpr int r = decltype(r_c)::value;
          e[r] = fast_exp2(__builtin_fmaf(Sc[kb][r0 + r], c, -m_run));
          if constexpr (MASK) {
            constexpr int row = kb * MT + 8 * ((r0 + r) >> 2) + ((r0 + r) & 3);
            if (row > d) e[r] = 0.0f;
          }
          ps += e[r];
        });
        Pc[step][i0] = pack_bf16x2(e[0], e[1]);
        Pc[step][i0 + 1] = pack_bf16x2(e[2], e[3]);
        __builtin_amdgcn_sched_barrier(0);
      });
      if (__builtin_amdgcn_ballot_w64(!(ps <= kPsumLimit)) != 0) return false;
      l_run += ps;
      return true;
    };

    auto dbg_store = [&](const Acc (&S)[KBLK], int t) {
      if constexpr (DBG_S) {
        if (row_ok) {
#pragma unroll
          for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = t * KT + kb * MT + acc_row<MT>(lane, r);
              if (key < kend)
                p.s_dbg[(row_base + my_r) * (long long)Sk + key] = S[kb][r] * p.s_dbg_scale;
            }
        }
      }
    };

    // ---- prologue: S(0) ----
    if (ntiles > 0) {
      wait_vmcnt<nV + 2 * nK>();  // K0 landed (V0, K1, K2 may fly)
      lds_barrier();
      qk(0, sbuf[0]);
      dbg_store(sbuf[0], 0);
    }

    // ---- main loop: iteration j = softmax(j) || QK(j+1) || PV(j-1) ----
    // Iteration j keeps S(j) in sbuf[j & 1] and P(j) in pbuf[j & 1]; the loops
    // below fix the parity at compile time everywhere, so no register copies
    // are needed between iterations.
    auto sync = [&](auto ph_c, int j) {
      constexpr int PH = decltype(ph_c)::value;  // as for full_interleaved
      // K(j+1) and V(j-1) landed (the copies of iteration j-1 may still fly;
      // at j = 0, K(2) may), and every wave is past its reads of iteration j-1
      if (j == 0) wait_vmcnt<nK>();
      else wait_vmcnt<nK + nV>();
      wait_lgkmcnt0();
      lds_barrier();
      issue_k(j + 3, PH >= 0 ? (PH + 3) & 3 : stage_of(j + 3));
      issue_v(j + 1, PH >= 0 ? (PH + 1) & 3 : stage_of(j + 1));
    };
    // (the PV product of tile j-1 precedes the softmax of tile j in program
    // order: an exact-path rescale of O must apply to it, its P having been
    // taken against the old maximum; the fast path's VALU work does not depend
    // on it and interleaves with both products)
    // MASK: the tile crosses the causal diagonal or the ragged end.  The last
    // iteration's QK(j+1) reads a zero-filled stage (its copy lay past the
    // keys) and is discarded.
    // ph_c: the phase (j - 1) & 3 (0 .. 3) when known at compile time, else
    // -2 or -1: stages from j at run time, register buffers of parity 0 or 1
    // (the buffer parity, which selects registers, is always a constant; it
    // is j & 1 except where the masked iterations below renumber it).
    auto full_iter = [&](auto ph_c, auto mask_c, int j) {
      constexpr int PH = decltype(ph_c)::value;
      constexpr int PAR = PH >= 0 ? ((PH + 1) & 1) : PH + 2;
      constexpr bool MASK = decltype(mask_c)::value;
      sync(ph_c, j);
      bool ok;
      if constexpr (D == 64 && DV == 64) {
        ok = full_interleaved(mask_c, ph_c, j, sbuf[PAR ^ 1], pbuf[PAR ^ 1], sbuf[PAR],
                              pbuf[PAR]);
      } else {
        qk(j + 1, sbuf[PAR ^ 1]);
        pv(j - 1, pbuf[PAR ^ 1]);
        if constexpr (MASK) {
          mask(sbuf[PAR], j);
          softmax_exact(sbuf[PAR], pbuf[PAR]);
          ok = true;
        } else {
          ok = softmax_fast(sbuf[PAR], pbuf[PAR]);
        }
      }
      if (!ok) {
        qk(j, sbuf[PAR]);  // K(j) is still in its ring stage
        if constexpr (MASK) mask(sbuf[PAR], j);
        softmax_exact(sbuf[PAR], pbuf[PAR]);
      }
      if (j + 1 < ntiles) dbg_store(sbuf[PAR ^ 1], j + 1);
    };
    // Iteration 0: no PV product yet, and the first tile always takes the
    // exact softmax (the running maximum starts as the "no score yet"
    // stand-in).  Every wave runs it (a tile past a wave's last visible key is
    // masked whole and adds nothing).
    if (ntiles > 0) {
      sync(std::integral_constant<int, -2>{}, 0);
      if (1 < ntiles) {
        qk(1, sbuf[1]);
        dbg_store(sbuf[1], 1);
      }
      if (0 >= n_clean) mask(sbuf[0], 0);
      softmax_exact(sbuf[0], pbuf[0]);
    }
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    using Ph0 = std::integral_constant<int, 0>;
    using Ph1 = std::integral_constant<int, 1>;
    using Ph2 = std::integral_constant<int, 2>;
    using Ph3 = std::integral_constant<int, 3>;
    // Iterations 1 .. jm-1 need no mask: four at a time from j = 1 (phase 0)
    // with every ring stage a compile-time constant, then up to three more
    // (phases 0, 1, 2).  Iterations jm .. ntiles-1 (the causal diagonal and
    // the ragged end, a few per row block) run with stages computed from j;
    // they start with S(jm) in sbuf[0] and P(jm-1) in pbuf[1] (copied there
    // when jm is odd), then alternate buffer parities.
    const int jm = max(1, min(ntiles, n_clean));
    int j = 1;
    for (; j + 4 <= jm; j += 4) {
      full_iter(Ph0{}, NoMask{}, j);
      full_iter(Ph1{}, NoMask{}, j + 1);
      full_iter(Ph2{}, NoMask{}, j + 2);
      full_iter(Ph3{}, NoMask{}, j + 3);
      progress(4);
    }
    if (j < jm) full_iter(Ph0{}, NoMask{}, j++);
    if (j < jm) full_iter(Ph1{}, NoMask{}, j++);
    if (j < jm) full_iter(Ph2{}, NoMask{}, j++);
    if (j < ntiles && (j & 1)) {  // renumber: S(j) -> sbuf[0], P(j-1) -> pbuf[1]
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) sbuf[0][kb] = sbuf[1][kb];
#pragma unroll
      for (int st = 0; st < NPV; ++st) pbuf[1][st] = pbuf[0][st];
    }
    const int jpar = j & 1;  // j's parity where the masked iterations start
    for (; j < ntiles; j += 2) {
      full_iter(std::integral_constant<int, -2>{}, Mask{}, j);
      if (j + 1 < ntiles) full_iter(std::integral_constant<int, -1>{}, Mask{}, j + 1);
      progress(2);
    }
    // every copy landed and every wave past its reads of the rings (the
    // epilogue below reuses the K ring)
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    lds_barrier();
    // the last tile's PV product
    if (ntiles > 0) {
      // P(ntiles-1): in pbuf[(ntiles-1) & 1], or, when the masked iterations
      // renumbered the buffers (started at an odd j), in the other one
      const int jl = ntiles - 1;
      const bool renumbered = jm < ntiles && jpar;
      if (((jl & 1) ^ (renumbered ? 1 : 0)) != 0) pv(jl, pbuf[1]);
      else pv(jl, pbuf[0]);
    }

    // ---- epilogue: O / l, log-sum-exp ----
    if constexpr (!DBG_S) {
    const float l_tot = group_sum<MT>(l_run);
    const bool empty = !(l_tot > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / l_tot;
    const float lse_val = empty ? -__builtin_inff() : (m_run + __log2f(l_tot)) * kLn2;
    // O leaves the accumulators one row per lane in 8-byte pieces (a store
    // straight from them would write 16 bytes of each of 32 rows per
    // instruction); the wave's 32 rows go row-major through LDS first and
    // then out as whole 128-byte rows, 8 rows per store (measured 2-4 %
    // faster, same bits).  The K ring is idle here: every wave has passed the
    // barrier above after its last K read of this row block, and the next
    // row block's copies start after the barrier at its top.
    static_assert(DV == 64 && NW * MT * DV <= KST * KTILE, "O staging in the K ring");
    FMHA_LDS uint16_t* ost = (FMHA_LDS uint16_t*)&ksm[0][0] + wave * (MT * DV);
    // (the lane index laundered through an empty asm, so the compiler does
    // not hoist these addresses out of the row-block loop and hold them in
    // registers through the main loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int oc = ln & 31, og = ln >> 5;  // = qcol, kg
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const uint32_t w0 = pack_bf16x2(oacc[db][4 * qd + 0] * inv, oacc[db][4 * qd + 1] * inv);
        const uint32_t w1 = pack_bf16x2(oacc[db][4 * qd + 2] * inv, oacc[db][4 * qd + 3] * inv);
        // 16-byte chunk db*4+qd of row qcol (columns 8 (db*4+qd) + 4 kg ..),
        // chunks XOR-swizzled by the row so the row-major reads below are
        // free of bank conflicts
        const int cs = (db * 4 + qd) ^ (oc & 7);
        *(FMHA_LDS u32x2*)(ost + oc * DV + cs * 8 + 4 * og) = u32x2{w0, w1};
      }
    }
#pragma unroll
    for (int i = 0; i < MT / 8; ++i) {  // (LDS accesses of one wave stay in order)
      const int row = 8 * i + (ln >> 3), c = ln & 7;
      const u32x4 val = *(FMHA_LDS u32x4*)(ost + row * DV + ((c ^ (row & 7)) * 8));
      // (written through: 1.5-3 % faster than leaving 16 MB of O dirty in
      // the L2s for the write-back at the kernel's end; same bits)
      if (r_wave0 + row < p.rows_per_kv)
        global_store_b128_stream(p.o + (row_base + r_wave0 + row) * DV + c * 8, val);
    }
    if (row_ok && kg == 0 && p.lse) p.lse[row_base + my_r] = lse_val;
    }
  }  // row blocks of this workgroup
}

// Launch of one prefill configuration C (a TileCfg of with_fwd_cfg) over
// p.n_row_blocks row blocks of each of the Hkv * B units; sets the row blocks
// per workgroup of the pipelined kernel (p.rb_per_wg) and the grid.
// cus: compute units of the device.
template <class C, bool CAUSAL, bool DBG_S>
inline void launch_prefill_cfg(AttnParams p, int cus, hipStream_t st) {
  const long long units = (long long)p.Hkv * p.B;
  if constexpr (C::PIPE) {
    // row blocks of NW * 32 rows; pairs when the single-block grid takes two
    // or more rounds of the GPU's workgroup slots (8 waves per CU)
    p.n_row_blocks = (p.rows_per_kv + C::NW * 32 - 1) / (C::NW * 32);
    const long long wg_slots = (long long)cus * (8 / C::NW);
    const bool pair = p.n_row_blocks >= 2 && units * p.n_row_blocks >= 2 * wg_slots;
    p.rb_per_wg = pair ? 2 : 1;
    const long long slots = pair ? (p.n_row_blocks + 1) / 2 : p.n_row_blocks;
    hipLaunchKernelGGL((prefill_kernel<C::D, C::DV, C::NW, CAUSAL, DBG_S>),
                       dim3((unsigned)(slots * units)), dim3(C::NW * 64), 0, st, p);
  } else {
    p.rb_per_wg = 1;
    hipLaunchKernelGGL((attn_fwd_kernel<C::D, C::MT, C::NW, C::KT, C::KS, C::VS, CAUSAL, false,
                                        false, false, C::DV, false, DBG_S>),
                       dim3((unsigned)(p.n_row_blocks * units)), dim3(C::NW * 64), 0, st, p);
  }
}

}  // namespace fmha
