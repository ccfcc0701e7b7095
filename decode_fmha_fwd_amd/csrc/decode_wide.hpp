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
// and runs 4 waves, two row groups of 32 rows times two halves.  Wave (g, h)
// computes the QK partial of rows 32g..32g+31 over half h of the Q/K head dim
// (32x32x16 MFMAs, S^T = K Q^T), and the PV product of the same rows for half
// h of the V/O columns (O^T += V^T P^T, V^T through LDS transpose reads).
// The two waves of a row group add their QK partials through LDS (own +
// partner: float addition commutes, so both hold bit-identical scores) and
// run the same softmax.  32-row waves read each K and V^T byte of a tile from
// LDS twice per workgroup where 16-row waves read it four times, and each
// wave keeps only half of Q and of O in registers.
//
// Software pipeline, one barrier per 32-key tile: iteration t adds the
// partials of S(t), then issues the QK partial of tile t+1 with the softmax
// of S(t) interleaved between its MFMAs, then the PV product of tile t, and
// writes its partial of S(t+1) for the partner.  The LDS reads of K(t+1) and
// V^T(t) stream a fixed number ahead of the MFMAs that use them, and the
// copies of tile t+3 (into the stage of tile t-1) are spread over the
// iteration.  LDS: a 4-deep ring of 32-key tiles (128 KB at head dim 512,
// 144 KB at 576) and the partials (16 KB, double-buffered where the ring
// leaves room; a single buffer takes a second barrier before it is
// rewritten).  All 4 waves share the copies, buffer loads bounded by the
// split's key range (rows past it read as zeros, whole tiles past it cost no
// memory traffic).
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

// acc <- alpha acc for an MFMA accumulator held in AGPRs: the multiply is
// inline asm on AGPR operands, so the (rare) rescale of the output does not
// make the compiler keep the accumulators in VGPRs and copy them back and
// forth around every MFMA.
__device__ inline void scale_acc_agpr(f32x16& acc, float alpha) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = acc[i];
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(t)
        : "v"(alpha));
    acc[i] = x;
  }
}

// Threads per workgroup of the wide decode (4 waves).
constexpr int kWideThreads = 256;

// The read stream of one iteration of the wide decode: kq K reads (one per
// QK step), then two transpose reads per PV unit; MFMA m (QK steps first,
// then PV units) needs reads up to this index.
constexpr int wide_last_read(int m, int kq) { return m < kq ? m : kq + 2 * (m - kq) + 1; }
constexpr int wide_min(int a, int b) { return a < b ? a : b; }

// DBG_S (test builds only): as in attn_fwd_kernel, the summed score tiles
// times p.s_dbg_scale go to p.s_dbg [rows][Sk] before masking, and the
// kernel writes no output.
template <int D, int DV, bool CAUSAL, bool SPLIT, bool DBG_S = false>
__global__ __launch_bounds__(kWideThreads) void decode_wide_kernel(AttnParams p) {
  using M = Mfma<32>;
  using Acc = M::Acc;
  constexpr int KT = 32;           // keys per tile (one 32-key block)
  constexpr int KST = 4;           // ring depth
  constexpr int DH = D / 2;        // Q/K head-dim columns of one wave
  constexpr int DVH = DV / 2;      // V/O columns of one wave
  constexpr int KSTEPS = DH / 16;  // QK MFMAs per tile
  constexpr int DBLK = DVH / 32;   // 32-column blocks of O^T
  constexpr int NU = 2 * DBLK;     // PV MFMAs per tile (two 16-key steps per block)
  constexpr int KTILE = KT * D;    // elements of a tile
  // Tile copies: the tile's 1 KB chunks (64 lanes x 16 bytes) go round-robin
  // over the 4 waves, copy j of wave w being chunk 4 j + w.
  constexpr int kChunks = KT * D * 2 / 1024;
  constexpr int kMaxCopies = (kChunks + 3) / 4;
  constexpr int kRingBytes = KST * KTILE * 2;
  constexpr int kXBytes = 4 * 4 * 64 * 16;  // partials: 4 waves x 4 words x 64 lanes
  constexpr int NXB = (kRingBytes + 2 * kXBytes <= 160 * 1024) ? 2 : 1;
  static_assert(kChunks * 1024 == KT * D * 2, "a tile is whole 1 KB chunks");
  static_assert(DH % 16 == 0 && DVH % 32 == 0 && DV <= D, "head-dim halves in whole blocks");
  static_assert(KSTEPS >= 16, "the softmax is spread over 16 QK steps");
  static_assert(kRingBytes + NXB * kXBytes <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(16))) uint16_t ksm[KST][KTILE];
  // per buffer and wave: its QK partial, four 16-byte words per lane, each
  // word lane-contiguous
  __shared__ __attribute__((aligned(16))) float xbuf[NXB][4][4][64][4];

  const int lane = threadIdx.x & 63;
  // (wave-uniform in scalar registers: branches on it are scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave & 1;  // row group
  const int h = wave >> 1;  // head-dim half
  const int qcol = lane & 31;
  const int kg = lane >> 5;

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
  const int r_wave0 = r_wg0 + rg * 32;
  const int my_r = r_wave0 + qcol;
  const bool row_ok = my_r < p.rows_per_kv;
  const int my_rc = row_ok ? my_r : p.rows_per_kv - 1;
  const int diag = Sk - p.Sq;  // causal: key j visible to row i iff j <= i + diag

  const int kbeg = split * p.split_len;
  int kend = min(Sk, kbeg + p.split_len);
  if (CAUSAL) {
    const int r_end = min(p.rows_per_kv, r_wg0 + 64) - 1;
    const int i_last = (r_wg0 / p.Sq == r_end / p.Sq) ? r_end % p.Sq : p.Sq - 1;
    kend = min(kend, i_last + diag + 1);
  }
  const int my_last = CAUSAL ? (my_rc % p.Sq) + diag : INT_MAX;
  const int ntiles = (kend > kbeg) ? (kend - kbeg + KT - 1) / KT : 0;
  // Tiles [0, n_clean) need a mask for no row: they end at or before kend and
  // before every row's last visible key (row i sees keys up to i + diag,
  // so at least up to diag).  Decode rows are few, so at most the last tile
  // or two of a causal range need the mask.
  const int lim_all = CAUSAL ? min(diag, kend - 1) : kend - 1;
  const int n_clean = max(lim_all - kbeg + 1, 0) / KT;

  // ---- copies: the split's key rows, bounded (reads past kend return zeros)
  const uint16_t* kbase = p.k + ((long long)bh_kv * Sk + kbeg) * D;
  const uint32_t kbytes = (uint32_t)max(kend - kbeg, 0) * (uint32_t)(D * 2);
  FMHA_LDS char* ring = (FMHA_LDS char*)&ksm[0][0];
  const int n_copies = (kChunks - wave + 3) / 4;  // this wave's copies per tile
  uint32_t cvoff[kMaxCopies];  // a lane's byte offset in the tile, swizzled
#pragma unroll
  for (int j = 0; j < kMaxCopies; ++j) {
    const int byte = (4 * j + wave) * 1024 + lane * 16;
    const int row = byte / (D * 2);
    const int pchunk = (byte - row * D * 2) >> 4;
    cvoff[j] = (uint32_t)(row * D * 2 + ((pchunk ^ swz<D / 8>(row)) << 4));
  }
  // copy j of this wave for tile t
  auto issue_one = [&](int t, auto j_c) {
    constexpr int J = decltype(j_c)::value;
    if (J < kMaxCopies - 1 || 4 * J + wave < kChunks)
      buffer_load_lds16<2>(kbase, kbytes,
                           (FMHA_LDS void*)(ring + (t & 3) * (KTILE * 2) + (4 * J + wave) * 1024),
                           (uint32_t)t * (uint32_t)(KT * D * 2) + cvoff[J]);
  };
  auto issue_all = [&](int t) {
    static_for<0, kMaxCopies>([&](auto j_c) { issue_one(t, j_c); });
  };

  // Prologue: tile 0, then this wave's half of the Q^T fragments, then tiles
  // 1 and 2.  The wait for Q then covers tile 0 besides, which is needed
  // first anyway.
  issue_all(0);
  u32x4 qf[KSTEPS];
  {
    const uint16_t* qrow = p.q + (row_base + my_rc) * D + h * DH + 8 * kg;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *(const u32x4*)(qrow + s * 16);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) asm volatile("; q ready" : "+v"(qf[s]));
  }
  issue_all(1);
  issue_all(2);

  // ---- per-lane LDS offsets (bytes).  The swizzle repeats every 2^KSW
  // chunks of a row and every 16 rows, so whole periods of columns and whole
  // 16-key steps are instruction immediates.
  constexpr int KSW = CPR_LOG2<D / 8>::value;
  constexpr int KPER_RAW = (1 << KSW) / 2;  // 16-column k-steps per swizzle period
  constexpr int KPER = KPER_RAW < 1 ? 1 : (KPER_RAW > KSTEPS ? KSTEPS : KPER_RAW);
  constexpr int VPER_RAW = (1 << KSW) / 4;  // 32-column blocks per period
  constexpr int VPER = VPER_RAW < 1 ? 1 : (VPER_RAW > DBLK ? DBLK : VPER_RAW);
  uint32_t koff[KPER];
#pragma unroll
  for (int s = 0; s < KPER; ++s) koff[s] = 2u * tile_off<D>(qcol, h * DH + s * 16 + 8 * kg);
  uint32_t voff0[VPER], voff1[VPER];
  {
    // V^T through transpose reads: k-slots 0..3 <-> keys 16 step + 4 kg +
    // 0..3, 4..7 <-> keys 16 step + 8 + 4 kg + 0..3, matching the S^T
    // register layout of the P operand
    const int grp = lane >> 4, tj = (lane >> 2) & 3, ta = lane & 3;
#pragma unroll
    for (int db = 0; db < VPER; ++db) {
      const int col = h * DVH + db * 32 + 16 * (grp & 1) + 4 * ta;
      const int row1 = 4 * (grp >> 1) + tj;
      voff0[db] = 2u * tile_off<D>(row1, col);
      voff1[db] = 2u * tile_off<D>(row1 + 8, col);
    }
  }
  const uint32_t k_lds = lds_addr((const FMHA_LDS void*)&ksm[0][0]);
  const uint32_t x_own = lds_addr((const FMHA_LDS void*)&xbuf[0][wave][0][lane][0]);
  const uint32_t x_par = lds_addr((const FMHA_LDS void*)&xbuf[0][wave ^ 2][0][lane][0]);

  Acc oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = Acc{};
  float m_run = kNegBig;
  // Two row sums of P.  O is divided by the sum of the bf16-rounded P, the
  // very weights it accumulates, so its weights sum to one; the matrix cores
  // take it, an extra MFMA per 16-key step with an all-ones A operand leaving
  // every register of lane l with its row's sum.  The log-sum-exp needs the
  // sum of the unrounded p (with a few dominant keys the bf16 rounding moves
  // it by up to 2-3e-3): the lane's fp32 partial sum, l_run.  (Dividing O by
  // l_run instead raised its error to 2.3e-2 on such inputs.)
  Acc lacc = Acc{};
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  float l_run = 0.0f;
  const float c = p.scale_log2;
  Acc s_own = Acc{};  // this wave's QK partial of the tile the next iteration takes

  // This wave's partial of S^T to the partials buffer xb.
  auto write_partial = [&](const Acc& s, int xb) {
    const uint32_t a = x_own + (uint32_t)xb * kXBytes;
    lds_write_b128_imm<0>(a, f32x4{s[0], s[1], s[2], s[3]});
    lds_write_b128_imm<1024>(a, f32x4{s[4], s[5], s[6], s[7]});
    lds_write_b128_imm<2048>(a, f32x4{s[8], s[9], s[10], s[11]});
    lds_write_b128_imm<3072>(a, f32x4{s[12], s[13], s[14], s[15]});
  };

  // ---- prologue QK: this wave's partial of S^T(0) ----
  if (ntiles > 0) {
    wait_lgkmcnt0();
    lds_barrier();  // everyone's copies of tile 0 have landed (each waited for its own)
    constexpr int RA = 8;
    u32x4 kf[KSTEPS];
    auto read = [&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      kf[s] = lds_read_b128_imm<2u * ((s / KPER) * KPER * 16)>(k_lds + koff[s % KPER]);
    };
    static_for<0, RA>([&](auto s_c) { read(s_c); });
    Acc sa = Acc{}, sb = Acc{};
    static_for<0, KSTEPS>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      constexpr int ahead = (KSTEPS - 1 - s) < (RA - 1) ? (KSTEPS - 1 - s) : (RA - 1);
      lds_wait_tied<ahead>(kf[s]);
      if constexpr (s + RA < KSTEPS) read(std::integral_constant<int, s + RA>{});
      if constexpr (s & 1)
        sb = M::run(__builtin_bit_cast(bf16x8, kf[s]), __builtin_bit_cast(bf16x8, qf[s]), sb);
      else
        sa = M::run(__builtin_bit_cast(bf16x8, kf[s]), __builtin_bit_cast(bf16x8, qf[s]), sa);
    });
    s_own = sa + sb;
    write_partial(s_own, 0);
  }

  // ---- iteration t: S(t) from the partials, softmax, PV(t); with NEXT also
  // the QK partial of tile t+1 and the copies of tile t+3; with MASK the
  // ragged end and the causal diagonal ----
  auto iteration = [&](int t, auto next_c, auto mask_c) {
    constexpr bool NEXT = decltype(next_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    const int t0 = kbeg + t * KT;
    // Tile t+1 has landed (t+2 may still fly); every wave has written its
    // partial of S(t) and is past its reads of tile t-1 and of the partials
    // it read last.
    if constexpr (NEXT) {
      if (n_copies == kMaxCopies)
        wait_vmcnt<kMaxCopies>();
      else
        wait_vmcnt<kMaxCopies - 1>();
    }
    wait_lgkmcnt0();
    lds_barrier();
    const int xb = (NXB == 2) ? (t & 1) : 0;
    const uint32_t vst = k_lds + (uint32_t)(t & 3) * (uint32_t)(KTILE * 2);
    const uint32_t kst = k_lds + (uint32_t)((t + 1) & 3) * (uint32_t)(KTILE * 2);

    // The LDS read stream of the iteration: K(t+1) for QK steps 0..KSTEPS-1
    // (with NEXT), then the two transpose reads of each PV unit; the MFMA
    // stream: QK steps, then PV units.  Reads go WIN ahead of their MFMA.
    constexpr int KQ = NEXT ? KSTEPS : 0;
    constexpr int NR = KQ + 2 * NU;
    constexpr int NM = KQ + NU;
    constexpr int WIN = 8;
    constexpr int HEAD = wide_min(WIN + 1, NR);
    u32x4 kf[KSTEPS];
    u32x2 vlo[NU], vhi[NU];
    auto read = [&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      if constexpr (i < KQ) {
        kf[i] = lds_read_b128_imm<2u * ((i / KPER) * KPER * 16)>(kst + koff[i % KPER]);
      } else {
        constexpr int U = (i - KQ) / 2, half = (i - KQ) % 2;
        constexpr int step = U / DBLK, db = U % DBLK;
        constexpr uint32_t imm = step * (16u * D * 2) + (uint32_t)(db / VPER) * VPER * 64u;
        if constexpr (half == 0)
          vlo[U] = lds_read_tr16_imm<imm>(vst + voff0[db % VPER]);
        else
          vhi[U] = lds_read_tr16_imm<imm>(vst + voff1[db % VPER]);
      }
    };

    // partner's partial of S^T(t), then the head of the read stream
    Acc sc;
    {
      const uint32_t a = x_par + (uint32_t)xb * kXBytes;
      u32x4 x0 = lds_read_b128_imm<0>(a);
      u32x4 x1 = lds_read_b128_imm<1024>(a);
      u32x4 x2 = lds_read_b128_imm<2048>(a);
      u32x4 x3 = lds_read_b128_imm<3072>(a);
      static_for<0, HEAD>([&](auto i_c) { read(i_c); });
      lds_wait_tied<HEAD + 3>(x0);
      lds_wait_tied<HEAD + 2>(x1);
      lds_wait_tied<HEAD + 1>(x2);
      lds_wait_tied<HEAD>(x3);
      const f32x4 p0 = __builtin_bit_cast(f32x4, x0), p1 = __builtin_bit_cast(f32x4, x1);
      const f32x4 p2 = __builtin_bit_cast(f32x4, x2), p3 = __builtin_bit_cast(f32x4, x3);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = s_own[r] + p0[r];
        sc[4 + r] = s_own[4 + r] + p1[r];
        sc[8 + r] = s_own[8 + r] + p2[r];
        sc[12 + r] = s_own[12 + r] + p3[r];
      }
    }
    if constexpr (DBG_S) {
      if (h == 0 && row_ok) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t0 + acc_row<32>(lane, r);
          if (key < kend) p.s_dbg[(row_base + my_r) * (long long)Sk + key] = sc[r] * p.s_dbg_scale;
        }
      }
    }
    // ragged end and causal diagonal: key t0 + acc_row(lane, r) is visible
    // iff it is at most min(my_last, kend - 1); the row of register r is a
    // constant plus 4 kg, so one compare per score.  (A row with no visible
    // key in the tile gets p = 0 throughout.)
    if constexpr (MASK) {
      const int d = min(my_last, kend - 1) - t0 - 4 * kg;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > d) sc[r] = -__builtin_inff();
    }

    // Softmax of S(t), in 16 slices placed between the MFMAs (base 2, lazy
    // rescale: m moves only when a row's tile maximum exceeds it by more than
    // kRescaleSlack).
    float mloc = -__builtin_inff();
    u32x4 pw[2];
    auto slice = [&](auto k_c) {
      constexpr int k = decltype(k_c)::value;
      if constexpr (k == 0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) mloc = fmaxf(mloc, sc[r]);
      } else if constexpr (k == 1) {
#pragma unroll
        for (int r = 8; r < 16; ++r) mloc = fmaxf(mloc, sc[r]);
      } else if constexpr (k == 2) {
        mloc = group_max<32>(mloc) * c;
        if (__builtin_amdgcn_ballot_w64(mloc > m_run + kRescaleSlack) != 0) {
          const float m_new = fmaxf(m_run, mloc);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          // (the compiler puts no wait states between an MFMA and inline asm
          // reading its result; the last MFMAs into lacc and oacc were issued
          // in the previous iteration, before its last PV MFMAs, the barrier
          // and the partial reads: far more than the 18 wait states an MFMA
          // result needs)
          l_run *= alpha;
          scale_acc_agpr(lacc, alpha);
#pragma unroll
          for (int i = 0; i < DBLK; ++i) scale_acc_agpr(oacc[i], alpha);
        }
      } else if constexpr (k <= 10) {
        constexpr int r0 = 2 * (k - 3);
#pragma unroll
        for (int r = r0; r < r0 + 2; ++r) {
          sc[r] = fast_exp2(__builtin_fmaf(sc[r], c, -m_run));
          l_run += sc[r];
        }
      } else if constexpr (k <= 14) {
        // P as the B operand: k-slots 0..7 of 16-key step w/2 hold the S^T
        // registers 8 (w/2) + 0..7
        constexpr int w = k - 11;
        pw[w >> 1][2 * (w & 1)] = pack_bf16x2(sc[4 * w + 0], sc[4 * w + 1]);
        pw[w >> 1][2 * (w & 1) + 1] = pack_bf16x2(sc[4 * w + 2], sc[4 * w + 3]);
      }
    };
    if constexpr (!NEXT) static_for<0, 16>([&](auto k_c) { slice(k_c); });

    Acc sa = Acc{}, sb = Acc{};
    static_for<0, NM>([&](auto m_c) {
      constexpr int m = decltype(m_c)::value;
      // keep the reads up to WIN past the last one this MFMA needs in flight
      constexpr int need = wide_last_read(m, KQ);
      constexpr int prev_issued =
          (m == 0) ? HEAD : wide_min(wide_last_read(m - 1, KQ) + 1 + WIN, NR);
      constexpr int issued = wide_min(need + 1 + WIN, NR);
      static_for<prev_issued, issued>([&](auto i_c) { read(i_c); });
      if constexpr (m < KQ) {
        lds_wait_tied<issued - 1 - need>(kf[m]);
        if constexpr (m & 1)
          sb = M::run(__builtin_bit_cast(bf16x8, kf[m]), __builtin_bit_cast(bf16x8, qf[m]), sb);
        else
          sa = M::run(__builtin_bit_cast(bf16x8, kf[m]), __builtin_bit_cast(bf16x8, qf[m]), sa);
        if constexpr (m < 16) slice(std::integral_constant<int, m>{});
      } else {
        constexpr int U = m - KQ;
        lds_wait<issued - 1 - need>();
        lds_tie(vlo[U]);
        lds_tie(vhi[U]);
        const u32x4 vf = u32x4{vlo[U][0], vlo[U][1], vhi[U][0], vhi[U][1]};
        oacc[U % DBLK] = M::run(__builtin_bit_cast(bf16x8, vf),
                                __builtin_bit_cast(bf16x8, pw[U / DBLK]), oacc[U % DBLK]);
        if constexpr (U % DBLK == 0)  // the (bf16) row sums of this 16-key step
          lacc = M::run(__builtin_bit_cast(bf16x8, ones), __builtin_bit_cast(bf16x8, pw[U / DBLK]),
                        lacc);
        // this wave's partial of S^T(t+1) for the partner, once the QK chain
        // has had a few MFMAs' time to finish
        if constexpr (NEXT && U == 3) {
          s_own = sa + sb;
          if constexpr (NXB == 1) lds_barrier();  // every wave has read the buffer
          write_partial(s_own, (NXB == 2) ? ((t + 1) & 1) : 0);
        }
      }
      // copies of tile t+3, one after every other MFMA
      if constexpr (NEXT && (m & 1) && (m >> 1) < kMaxCopies)
        issue_one(t + 3, std::integral_constant<int, (m >> 1)>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  int t = 0;
  for (; t + 1 < ntiles && t < n_clean; ++t) iteration(t, std::true_type{}, std::false_type{});
  for (; t + 1 < ntiles; ++t) iteration(t, std::true_type{}, std::true_type{});
  if (ntiles > 0) iteration(ntiles - 1, std::false_type{}, std::true_type{});
  // the copies past the last tile (zeros) land before the LDS is released
  wait_vmcnt<0>();

  if constexpr (DBG_S) return;

  // ---- epilogue: this wave's half of O / l; lse from half 0 ----
  const float l_bf = lacc[0];                 // divides O
  const float l_tot = group_sum<32>(l_run);  // gives the log-sum-exp
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l_bf;
  const float lse_val = empty ? -__builtin_inff() : (m_run + __log2f(l_tot)) * kLn2;
  if constexpr (SPLIT) {
    // The accumulators hold one row per lane, so stores straight from them
    // write 32 bytes of each of 32 rows per instruction.  The wave's 32
    // partial rows (its half of the columns, fp32) go row-major through the
    // ring, idle now, and out as whole 1 KB row halves (2-3 % faster at head
    // dim 512, same bits).  Chunks are XOR-swizzled by the row so that both
    // the writes and the row-major reads are free of bank conflicts.
    static_assert(4 * 32 * DVH * 4 <= KST * KTILE * 2 && DVH == 256, "partials staging in the ring");
    wait_lgkmcnt0();
    lds_barrier();  // every wave past its last ring read
    FMHA_LDS float* st = (FMHA_LDS float*)&ksm[0][0] + wave * (32 * DVH);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int c = db * 8 + 2 * qd + kg;  // 16-byte chunk of the row half
        *(FMHA_LDS f32x4*)(st + qcol * DVH + ((c ^ qcol) * 4)) =
            f32x4{oacc[db][4 * qd + 0] * inv, oacc[db][4 * qd + 1] * inv,
                  oacc[db][4 * qd + 2] * inv, oacc[db][4 * qd + 3] * inv};
      }
    }
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {  // (LDS accesses of one wave stay in order)
      const f32x4 val = *(FMHA_LDS f32x4*)(st + i * DVH + ((lane ^ i) * 4));
      if (r_wave0 + i < p.rows_per_kv)
        *(f32x4*)(p.o_part + ((row_base + r_wave0 + i) * p.nsplit + split) * DV + h * DVH +
                  4 * lane) = val;
    }
    if (row_ok && h == 0 && kg == 0) p.lse_part[(row_base + my_r) * p.nsplit + split] = lse_val;
    return;
  }
  if (row_ok) {
    const long long row = row_base + my_r;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = h * DVH + db * 32 + 8 * qd + 4 * kg;
        const float o0 = oacc[db][4 * qd + 0] * inv, o1 = oacc[db][4 * qd + 1] * inv;
        const float o2 = oacc[db][4 * qd + 2] * inv, o3 = oacc[db][4 * qd + 3] * inv;
        *(u32x2*)(p.o + row * DV + d0) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
      }
    }
    if (h == 0 && kg == 0 && p.lse) p.lse[row] = lse_val;
  }
}

}  // namespace fmha
