// attn_kernels.hpp -- the fused attention kernel (prefill and split-KV decode)
// and the log-sum-exp combine kernel for gfx950.
//
// The parts follow the feature list on the page
// "NVFP4-1.1_RAW_CUDA_CPP_APPROACH.md": QK product on the matrix cores, an
// in-kernel softmax that rescales the output accumulator when the running
// maximum moves, a loop over several KV tiles, the PV product, a correction
// epilogue that divides by the softmax sum, and (on that page, "multi-CTA")
// several workgroups per row over disjoint key ranges, merged by a separate
// combine kernel.
//
// Design (gfx950, not a translation of the pages' Blackwell kernel):
//   * A workgroup of NW waves owns NW*MT query rows that share one KV head
//     (MT = 32 or 16 rows per wave).  Rows are the flattened (grouped head,
//     position) pairs of that KV head, so GQA decode packs all Hq/Hkv heads of
//     a KV head into one workgroup and each K/V byte is read once.
//   * K and V tiles of KT keys stream from HBM straight into rings of KST and
//     VST LDS tiles with asynchronous global->LDS copies (no registers, issued
//     KST-1 / VST-1 tiles ahead, one barrier per tile); 16-byte chunks are
//     XOR-swizzled by row so MFMA operand reads are free of bank conflicts.
//   * Scores are computed transposed, S^T = K * Q^T (K is the A operand, Q^T
//     the B operand held in registers), so each lane owns ONE query row and a
//     set of keys: row max and row sum are in-lane plus one or two lane swaps.
//   * The output is accumulated transposed too, O^T += V^T * P^T: the
//     probabilities stay in registers in exactly the layout the MFMA B operand
//     wants (keys are assigned to k-slots to match), and V^T comes from the LDS
//     tile through the gfx950 transpose read ds_read_b64_tr_b16.
//   * Online softmax in base 2: m is kept in units of log2, p = exp2(s*c - m)
//     with c = scale*log2(e) folded into one FMA; the output rescale factor is
//     exp2(m_old - m_new).
//   * Every LDS read of the tile loop (K operand reads and V transpose reads)
//     is issued from inline asm and waited for with explicit lgkmcnt waits: a
//     compiler-visible LDS read placed after asynchronous global->LDS copies
//     makes the compiler drain every copy in flight (vmcnt(0)) first, which
//     would serialise the ring.  The build scans the generated assembly to
//     prove no result of such a read is touched before its wait.
#pragma once

#include <climits>
#include <type_traits>
#include <utility>

#include "fmha_device.hpp"
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace fmha {


// Chunk-index bits the swizzle permutes for rows of CPR 16-byte chunks: 4 when
// a row is a whole number of 256-byte bank windows, else the bits of the
// row's offset within a window that the row index does not already vary (a
// 576-wide row, 72 chunks, starts each odd row half a window further on, so
// three bits are left).  CPR is a multiple of 2^bits, so an XORed chunk stays
// inside its row.
template <int CPR>
struct CPR_LOG2 {
  static constexpr int value =
      (CPR % 16 == 0) ? 4 : (CPR % 8 == 0 ? 3 : (CPR % 4 == 0 ? 2 : 1));
};

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// XOR swizzle of the 16-byte chunk index within a K/V row.  With 64 LDS
// banks of 4 bytes, a 16-byte read is served 16 lanes at a time and an 8-byte
// read 32 lanes at a time.  The K operand reads (16 lanes: one chunk of 16
// consecutive rows) and the V transpose reads (32 lanes: 4 or 8 consecutive
// rows, a 32- or 64-byte column band) both hit distinct banks when the chunk
// index is XORed with the bit-reversed low row bits: rows that share a bank
// window (256 bytes = 256/(2D) rows) are spread by the reversal's high bits,
// and neighbouring rows of a transpose read by its low bits.
template <int CPR>
__device__ inline int swz(int row) {
  constexpr int K = CPR_LOG2<CPR>::value;
  const unsigned x = (unsigned)(row >> (4 - K)) & ((1u << K) - 1u);
  return (int)(__builtin_bitreverse32(x) >> (32 - K));
}

// Element offset of (row, col) in a swizzled [rows][D] bf16 tile.
template <int D>
__device__ inline int tile_off(int row, int col) {
  constexpr int CPR = D / 8;
  return row * D + (((col >> 3) ^ swz<CPR>(row)) << 3) + (col & 7);
}

// Q^T fragments, the B operand of S^T = K Q^T: for contraction step s the
// lane holds Q[row][s*kK + 8*kg + 0..7] (zeros past D).
template <int D, int MT>
__device__ inline void load_q_frags(const uint16_t* qrow, int kg,
                                    bf16x8 (&qf)[(D + Mfma<MT>::kK - 1) / Mfma<MT>::kK]) {
  constexpr int KSTEPS = (D + Mfma<MT>::kK - 1) / Mfma<MT>::kK;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int d0 = s * Mfma<MT>::kK + 8 * kg;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (d0 < D) raw = *(const u32x4*)(qrow + d0);
    qf[s] = __builtin_bit_cast(bf16x8, raw);
  }
}

// Copies one K or V tile (KT rows of W bf16 taken at column col0 of rows that
// are `stride` elements apart; rows clamped to the last key for a ragged tail)
// into a swizzled LDS tile with asynchronous global->LDS copies.  Each wave
// issues kLoads copies of 64 lanes x BYTES; copy j of wave w fills the
// contiguous LDS slots [(j*NW + w)*64, +64) and every lane fetches the global
// bytes that belong in its slot, so 8 lanes read one 128-byte row segment and
// the swizzle costs nothing on the HBM side.
template <int W, int NW, int KT, bool NT>
struct TileCopy {
  static constexpr int kTileBytes = KT * W * 2;
  static constexpr int kBytes = (kTileBytes >= NW * 64 * 16) ? 16 : 4;
  static constexpr int kLoads = kTileBytes / (NW * 64 * kBytes);
  static_assert(kLoads >= 1 && kLoads * NW * 64 * kBytes == kTileBytes,
                "tile must split evenly over the workgroup's copies");

  // Copies [J0, J1) of the tile (all of them by default).
  template <int J0 = 0, int J1 = kLoads>
  __device__ static inline void issue(const uint16_t* base, int stride, int col0, int t0, int Sk,
                                      FMHA_LDS char* lds, int wave, int lane) {
    constexpr int CPR = W / 8;
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const int slot = (j * NW + wave) * 64 + lane;
      const int byte = slot * kBytes;
      const int row = byte / (W * 2);
      const int inrow = byte - row * (W * 2);
      const int pchunk = inrow >> 4;
      const int lchunk = pchunk ^ swz<CPR>(row);
      const long long key = min(t0 + row, Sk - 1);
      const uint16_t* g = base + key * stride + col0 + lchunk * 8 + ((inrow & 15) >> 1);
      dma_to_lds<kBytes, NT>(g, (FMHA_LDS void*)(lds + (j * NW + wave) * 64 * kBytes));
    }
  }
};

// s_waitcnt vmcnt(<= n) for a run-time n in [0, N]: waits for the largest
// immediate not above n (waiting for fewer outstanding copies is always safe).
template <int N>
__device__ inline void wait_vmcnt_at_most(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vmcnt<N>();
      return;
    }
    wait_vmcnt_at_most<N - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// Lazy rescaling threshold (log2 units): the running maximum only moves when
// a tile's maximum exceeds it by more than this, so most tiles skip the O
// rescale; probabilities then stay below 2^kRescaleSlack, harmless in fp32
// and bf16.  The final O / l and LSE are exact whichever maximum is used.
constexpr float kRescaleSlack = 8.0f;

// The combine of one wave's rows inside the attention kernel, for a split
// group holding every split of its (batch, KV head): the arithmetic of
// lse_combine_kernel row for row, so the output is bit-identical to the
// split kernel followed by that kernel.  DV/4 lanes serve a row (4 outputs
// each), 64/(DV/4) rows at a time; the combine kernel's 64 lanes, each with
// the splits s = lane mod 64, are emulated by 64/(DV/4) "virtual lanes" per
// lane, whose sums meet in the same tree order as its cross-lane butterfly.
// PP: pointer to the partials (global, or LDS); prow0: the partial row of
// output row row0.
__device__ inline f32x4 load_f32x4(const float* p) { return *(const f32x4*)p; }
__device__ inline f32x4 load_f32x4(const FMHA_LDS float* p) { return *(const FMHA_LDS f32x4*)p; }
template <int DV, class PP>
__device__ inline void combine_wave_rows(PP o_part, PP lse_part, long long prow0, uint16_t* o,
                                         float* lse, long long row0, int nrows, int nsplit,
                                         int lane) {
  static_assert(DV == 64 || DV == 128, "in-workgroup combine: head dims 64 and 128");
  constexpr int VL = DV / 4;   // lanes per row
  constexpr int G = 64 / VL;   // rows per pass, and virtual lanes per lane
  const int li = lane % VL;
  for (int r0 = 0; r0 < nrows; r0 += G) {
    const int r = r0 + lane / VL;
    const bool ok = r < nrows;
    const long long row = row0 + (ok ? r : 0);  // idle lanes repeat row0 (in bounds)
    const long long prow = prow0 + (ok ? r : 0);
    const PP lp = lse_part + prow * nsplit;
    float m = -__builtin_inff();
    for (int s = li; s < nsplit; s += VL) m = fmaxf(m, lp[s]);
#pragma unroll
    for (int msk = 1; msk < VL; msk <<= 1) m = fmaxf(m, xor_lane(m, msk));
    if (m == -__builtin_inff()) {
      if (ok) {
        *(u32x2*)(o + row * DV + 4 * li) = u32x2{0u, 0u};
        if (li == 0 && lse) lse[row] = -__builtin_inff();
      }
      continue;
    }
    // virtual lane k * VL + li holds the splits s = k * VL + li (mod 64)
    float part[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      part[k] = 0.0f;
      for (int s = k * VL + li; s < nsplit; s += 64) part[k] += __expf(lp[s] - m);
#pragma unroll
      for (int msk = 1; msk < VL; msk <<= 1) part[k] += xor_lane(part[k], msk);
    }
    // the butterfly's levels at lane masks VL .. 32
#pragma unroll
    for (int w = 1; w < G; w <<= 1)
#pragma unroll
      for (int k = 0; k < G; k += 2 * w) part[k] = part[k] + part[k + w];
    const float L = m + __logf(part[0]);
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const PP op = o_part + prow * nsplit * DV + 4 * li;
    int s = 0;
    for (; s + 4 <= nsplit; s += 4) {  // four splits' loads in flight, summed in order
      f32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = load_f32x4(op + (long long)(s + u) * DV);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = __expf(lp[s + u] - L);
        acc += w * x[u];
      }
    }
    for (; s < nsplit; ++s) {
      const float w = __expf(lp[s] - L);
      acc += w * load_f32x4(op + (long long)s * DV);
    }
    if (ok) {
      *(u32x2*)(o + row * DV + 4 * li) =
          u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      if (li == 0 && lse) lse[row] = L;
    }
  }
}


// KST / VST: depth of the K and V rings (VST <= KST <= VST + 1).  V is read
// after K within a tile, so with one K stage more than V stages the extra
// look-ahead costs a K tile of LDS rather than a K and a V tile.
//
// KVS (V aliasing K, p.v == p.k): one ring of KST K tiles; the PV product
// reads V^T from the same LDS tile the QK product read K from, so every key
// row crosses HBM once (VST must equal KST).
//
// PAGED: K and V come from a paged cache ([num_pages][Hkv][page_size][D], a
// block table per batch, a key count per batch); a key tile never straddles
// two pages (page_size is a multiple of KT) and a head's rows of a page are
// contiguous, so each tile is one contiguous read after one table lookup,
// done a tile ahead of its copies.
//
// DV: head dim of V and O (D: of Q and K).  With a shared ring (KVS) V is the
// first DV columns of each K row.
//
// GROUP (with SPLIT): a workgroup takes p.splits_per_wg consecutive splits of
// its (batch, KV head).  Their key ranges are contiguous, so one copy stream
// runs through all of them; at every split boundary the softmax state is
// written out as that split's partial and reset, which is the arithmetic of
// one workgroup per split, without a short-lived workgroup per split.
//
// DBG_S (test builds only): after the QK block of every tile, the raw score
// tile times p.s_dbg_scale is stored to p.s_dbg [rows][Sk] (before masking and
// softmax), and the kernel writes no output.  Everything else -- copies, ring,
// LDS reads, MFMA chains -- is the code of the kernel without the flag.
template <int D, int MT, int NW, int KT, int KST, int VST, bool CAUSAL, bool SPLIT,
          bool KVS = false, bool PAGED = false, int DV = D, bool GROUP = false,
          bool DBG_S = false>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(AttnParams p) {
  using M = Mfma<MT>;
  using Acc = typename M::Acc;
  // Decode reads every K/V byte once: stream it non-temporally.  Prefill
  // re-reads K/V from L2 for every row block of a head: keep it cached.
  constexpr bool kStream = (MT == 16);
  using CopyK = TileCopy<D, NW, KT, kStream>;
  using CopyV = TileCopy<DV, NW, KT, kStream>;
  constexpr int VW = KVS ? D : DV;                 // row width of the LDS tile V^T is read from
  constexpr int KSTEPS = (D + M::kK - 1) / M::kK;  // QK contraction steps
  constexpr int KBLK = KT / MT;                    // MT-key blocks per tile
  constexpr int DBLK = (DV + MT - 1) / MT;         // MT-wide head-dim blocks of O^T
  constexpr int ROWS_WG = NW * MT;
  // PV instructions per d-block: 16 keys each for 32-row waves, 32 keys each
  // for 16-row waves (a 16-key tile fills half of one; the other half gets P = 0).
  constexpr int NPV = (MT == 32) ? 2 * KBLK : (KBLK + 1) / 2;
  constexpr int KTILE = KT * D;   // elements of a K tile
  constexpr int VTILE = KT * VW;  // elements of the tile V^T is read from
  constexpr int nK = CopyK::kLoads, nV = KVS ? 0 : CopyV::kLoads;  // copies per wave per tile
  constexpr int kPerTile = nK + nV;
  static_assert(!KVS || KST == VST, "a shared K/V ring has one depth");
  static_assert(DV <= D || !KVS, "V inside the K rows needs DV <= D");
  static_assert(DV == D || DV % MT == 0, "a separate V width in whole MT-wide blocks");
  static_assert(!GROUP || SPLIT, "split groups write split partials");
  static_assert(!(KVS && PAGED), "a paged cache keeps K and V apart");
  static_assert(KT % MT == 0, "KT must be a multiple of MT");
  static_assert(MT == 32 || KT == 16 || KT % 32 == 0, "16-row waves: 16 keys or whole 32s");
  static_assert(D % 16 == 0 && D >= 16, "head dim must be a multiple of 16");
  static_assert(VST >= 2 && KST <= 6 && (KST == VST || KST == VST + 1), "ring depths");
  // copies of this wave that may still be in flight when a tile is needed
  constexpr int kMaxPending = (KST == VST) ? (KST - 2) * kPerTile
                                           : nK + (VST - 2) * kPerTile;
  static_assert(kMaxPending < 64, "vmcnt range");
  constexpr int LCM = (KST == VST) ? KST : KST * VST;  // loop unroll: both stages constant

  // V ring first in LDS so that every V transpose read can carry its full LDS
  // offset as an instruction immediate (< 64 KiB); then the K ring.
  __shared__ __attribute__((aligned(16))) uint16_t vsm[KVS ? 1 : VST][KVS ? 8 : VTILE];
  __shared__ __attribute__((aligned(16))) uint16_t ksm[KST][KTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // 1-D grid, row block slowest: with a causal mask the longest row blocks of
  // every head are dispatched first, and since the (batch, KV head, split)
  // count is a multiple of 8 in the usual shapes, all row blocks of one head
  // land on the same XCD (blocks go round-robin over the 8 XCDs) and share its
  // L2 for their K/V re-reads.
  const int spw = GROUP ? p.splits_per_wg : 1;     // splits per workgroup
  const int nsg = (p.nsplit + spw - 1) / spw;        // split groups per (b, KV head)
  const int n_units = nsg * p.Hkv * p.B;
  const int rb_rank = blockIdx.x / n_units;
  const int unit = blockIdx.x - rb_rank * n_units;
  const int rb = CAUSAL ? p.n_row_blocks - 1 - rb_rank : rb_rank;
  const int split0 = (unit % nsg) * spw;             // first split of this workgroup
  const int nspl = min(spw, p.nsplit - split0);      // its splits
  const int bk = unit / nsg;
  const int kvh = bk % p.Hkv;
  const int b = bk / p.Hkv;

  const long long bh_kv = (long long)b * p.Hkv + kvh;
  // Keys of this batch: Sk, or its own count in a paged cache (at most Sk,
  // the table's reach).
  const int Sk = PAGED ? min(max(p.seqlens[b], 0), p.Sk) : p.Sk;
  const long long row_base = bh_kv * p.rows_per_kv;  // flat (b, h, i) id of row 0

  const int r_wg0 = rb * ROWS_WG;
  const int r_wave0 = r_wg0 + wave * MT;
  const int qcol = lane % MT;  // the query row this lane owns
  const int kg = lane / MT;    // contraction lane group
  const int my_r = r_wave0 + qcol;
  const bool row_ok = my_r < p.rows_per_kv;
  const int my_rc = row_ok ? my_r : p.rows_per_kv - 1;
  const int diag = Sk - p.Sq;  // causal: key j visible to row i iff j <= i + diag

  // Key range of this workgroup (its splits, back to back).
  const int kbeg = split0 * p.split_len;
  int kend = min(Sk, kbeg + nspl * p.split_len);
  int wave_min_last = INT_MAX;  // smallest last-visible key over the wave's rows
  int wave_max_last = INT_MAX;  // largest
  if (CAUSAL) {
    const int r_end = min(p.rows_per_kv, r_wg0 + ROWS_WG) - 1;
    const int i_last = (r_wg0 / p.Sq == r_end / p.Sq) ? r_end % p.Sq : p.Sq - 1;
    kend = min(kend, i_last + diag + 1);
    if (r_wave0 < p.rows_per_kv) {
      const int rw_end = min(p.rows_per_kv, r_wave0 + MT) - 1;
      const bool one_head = (r_wave0 / p.Sq == rw_end / p.Sq);
      wave_min_last = (one_head ? r_wave0 % p.Sq : 0) + diag;
      wave_max_last = (one_head ? rw_end % p.Sq : p.Sq - 1) + diag;
    } else {
      wave_min_last = wave_max_last = -1;
    }
  }
  const int my_last = CAUSAL ? (my_rc % p.Sq) + diag : INT_MAX;
  const int ntiles = (kend > kbeg) ? (kend - kbeg + KT - 1) / KT : 0;

  // Where the rows of key tile `it` of a cache start, the index of its first
  // key relative to that, and the key count its ragged end is clamped to.
  struct TileSrc {
    const uint16_t* base;
    int t0, lim;
  };
  // Page of key tile `it` in a paged cache (tiles past the range still get an
  // in-bounds page: the table slot and the page id are clamped).  The table
  // is read through the constant address space (it is read-only while the
  // kernel runs), so a uniform index makes a scalar load; a vector load would
  // queue in the vector-memory counter behind the tile copies in flight, and
  // the wait for its value would drain the whole copy ring every tile.
  using ConstInt = const __attribute__((address_space(4))) int;
  auto page_of = [&](int it) {
    if constexpr (PAGED) {
      const int slot = min(max(kbeg + it * KT, 0) >> p.page_shift, p.bt_stride - 1);
      ConstInt* table = (ConstInt*)p.block_table;
      return min(max(table[(long long)b * p.bt_stride + slot], 0), p.num_pages - 1);
    } else {
      return 0;
    }
  };
  // (w: row width of the cache, D for K and DV for V)
  auto tile_src = [&](const uint16_t* cache, int w, int it, int page) {
    const int k0 = kbeg + it * KT;
    if constexpr (PAGED) {
      const long long row = (((long long)page * p.Hkv + kvh) << p.page_shift) +
                            (k0 & ((1 << p.page_shift) - 1));
      return TileSrc{cache + row * w, 0, Sk - k0};
    } else {
      return TileSrc{cache + bh_kv * p.Sk * w, k0, Sk};
    }
  };
  auto issue_k = [&](TileSrc src, int stage, auto j0_c, auto j1_c) {
    CopyK::template issue<decltype(j0_c)::value, decltype(j1_c)::value>(
        src.base, D, 0, src.t0, src.lim, (FMHA_LDS char*)&ksm[stage][0], wave, lane);
  };
  auto issue_v = [&](TileSrc src, int stage, auto j0_c, auto j1_c) {
    if constexpr (!KVS)
      CopyV::template issue<decltype(j0_c)::value, decltype(j1_c)::value>(
          src.base, DV, 0, src.t0, src.lim, (FMHA_LDS char*)&vsm[stage][0], wave, lane);
  };
  using All0 = std::integral_constant<int, 0>;
  using AllK = std::integral_constant<int, nK>;
  using AllV = std::integral_constant<int, CopyV::kLoads>;
  // Copies of this wave issued after both K(it) and V(it) (see the issue
  // order: prologue V0 K0 V1 K1 ..., then per tile V(it+VST-1), K(it+KST-1)).
  auto pending_after = [&](int it) {
    int n = 0;
    if constexpr (KST == VST) {
#pragma unroll
      for (int j = 1; j <= KST - 2; ++j)
        if (it + j < ntiles) n += kPerTile;
    } else {
      if (it + 1 < ntiles) n += nK;
#pragma unroll
      for (int j = 1; j <= VST - 2; ++j) {
        if (it + j < ntiles) n += nV;
        if (it + j + 1 < ntiles) n += nK;
      }
    }
    return n;
  };

  // Prologue: the first tiles in flight before Q is even loaded.
#pragma unroll
  for (int s = 0; s < KST - 1; ++s) {
    if (s < VST - 1 && s < ntiles) issue_v(tile_src(p.v, DV, s, page_of(s)), s, All0{}, AllV{});
    if (s < ntiles) issue_k(tile_src(p.k, D, s, page_of(s)), s, All0{}, AllK{});
  }

  bf16x8 qf[KSTEPS];
  load_q_frags<D, MT>(p.q + (row_base + my_rc) * D, kg, qf);

  Acc oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = Acc{};
  float m_run = kNegBig;
  float l_run = 0.0f;

  // Per-lane LDS offsets, fixed for the whole loop: the swizzle depends only on
  // the low 4 row bits, so moving by whole 16-row blocks or by whole swizzle
  // periods of head-dim columns adds a constant that the instructions carry as
  // an immediate.
  constexpr int KSW = CPR_LOG2<D / 8>::value;          // swizzled chunk-index bits
  constexpr int KPER_RAW = (1 << KSW) / (M::kK / 8);   // K-read column period in k-steps
  constexpr int KPER = KPER_RAW < 1 ? 1 : (KPER_RAW > KSTEPS ? KSTEPS : KPER_RAW);
  constexpr int VSW = CPR_LOG2<VW / 8>::value;          // the same for the V^T tile
  constexpr int VPER_RAW = (1 << VSW) / (MT / 8);      // V-read column period in d-blocks
  constexpr int VPER = VPER_RAW < 1 ? 1 : (VPER_RAW > DBLK ? DBLK : VPER_RAW);
  constexpr int VROWS = (MT == 32) ? 2 : 1;            // distinct row phases of a V read pair
  uint32_t koff[KPER];  // bytes
#pragma unroll
  for (int s = 0; s < KPER; ++s) {
    const int col = s * M::kK + 8 * kg;
    koff[s] = 2u * tile_off<D>(lane % MT, col < D ? col : 0);
  }
  const uint32_t k_lds = lds_addr((const FMHA_LDS void*)&ksm[0][0]);
  uint32_t voff[VROWS][VPER];  // bytes
  {
    const int grp = lane >> 4, tj = (lane >> 2) & 3, ta = lane & 3;
#pragma unroll
    for (int db = 0; db < VPER; ++db) {
      int col = (MT == 32) ? db * 32 + 16 * (grp & 1) + 4 * ta : db * 16 + 4 * ta;
      if (col >= DV) col -= DV;  // head dims past DV (16 with 32-wide blocks): discarded
      // MT = 32: k-slots 0..3 <-> keys 16*step + 4h + 0..3, 4..7 <-> 16*step + 8 + 4h + 0..3
      // MT = 16: k-slots 0..3 <-> keys 32*step + 4g + 0..3, 4..7 <-> 32*step + 16 + 4g + 0..3
      const int row1 = (MT == 32) ? 4 * (grp >> 1) + tj : 4 * grp + tj;
      voff[0][db] = 2u * tile_off<VW>(row1, col);
      if constexpr (VROWS == 2) voff[VROWS - 1][db] = 2u * tile_off<VW>(row1 + 8, col);
    }
  }
  const uint32_t v_lds = KVS ? lds_addr((const FMHA_LDS void*)&ksm[0][0])
                             : lds_addr((const FMHA_LDS void*)&vsm[0][0]);

  // Pages of the tiles the current tile issues copies for (paged cache).
  int page_v = page_of(VST - 1), page_k = page_of(KST - 1);

  auto tile = [&](auto u_c, int it) {
    constexpr int U = decltype(u_c)::value;  // it % LCM
    constexpr int KSG = U % KST, STG = U % VST;  // (equal with a shared ring)
    const int t0 = kbeg + it * KT;
    // Sources of the tiles this one issues copies for; their pages were looked
    // up a tile ahead (below), so the scalar loads have landed by now.
    const TileSrc v_next = tile_src(p.v, DV, it + VST - 1, page_v);
    const TileSrc k_next = tile_src(p.k, D, it + KST - 1, page_k);
    // This wave's copies of tile `it` have landed (later tiles may still fly),
    // every wave is past its reads of tile it-1, and then everyone's copies of
    // tile `it` are visible.
    wait_vmcnt_at_most<kMaxPending>(pending_after(it));
    wait_lgkmcnt0();
    lds_barrier();
    if constexpr (PAGED) {
      page_v = page_of(it + VST);
      page_k = page_of(it + KST);
    }
    // Decode spreads the copies for later tiles through this tile's work,
    // V's over the QK steps and K's over the PV steps (same order and count
    // as issuing them all here), so the memory pipeline is fed while the wave
    // computes instead of the wave stalling on one long burst of issues into
    // a full memory queue.  Prefill (copies from L2) issues them here.
    constexpr bool kSpread = (MT == 16);
    const bool more_v = it + VST - 1 < ntiles, more_k = it + KST - 1 < ntiles;
    const int v_stage = (U + VST - 1) % VST, k_stage = (U + KST - 1) % KST;
    if constexpr (!kSpread) {
      if (more_v) issue_v(v_next, v_stage, All0{}, AllV{});
      if (more_k) issue_k(k_next, k_stage, All0{}, AllK{});
    }

    // Causal: a tile entirely past this wave's last visible key adds nothing.
    if (CAUSAL && t0 > wave_max_last) {
      if constexpr (kSpread) {
        if (more_v) issue_v(v_next, v_stage, All0{}, AllV{});
        if (more_k) issue_k(k_next, k_stage, All0{}, AllK{});
      }
      return;
    }

    // ---- S^T = K Q^T ----
    // K fragments are read in chunks of QCH contraction steps, one chunk ahead
    // of the MFMAs that use it (bounded register footprint at large D, and
    // more points at which decode can slot in its copies; one step at a time
    // for 32-row waves, whose register budget sets how many waves share a
    // SIMD).
    constexpr int QCH = (MT == 32) ? 1 : (KSTEPS < 2 ? KSTEPS : 2);
    constexpr int NQC = (KSTEPS + QCH - 1) / QCH;
    // Byte offset of this tile's K stage: an instruction immediate when the
    // whole ring fits the 16-bit DS offset, else added once per tile.
    constexpr uint32_t kStageBytes = (uint32_t)KSG * KTILE * 2;
    constexpr bool kStageImm = (uint32_t)KST * KTILE * 2 <= 65536u;
    const uint32_t kst = k_lds + (kStageImm ? 0u : kStageBytes);
    u32x4 kf[NQC][KBLK][QCH];
    auto read_k = [&](auto c_c) {
      constexpr int C = decltype(c_c)::value;
      static_for<0, KBLK * QCH>([&](auto j_c) {
        constexpr int J = decltype(j_c)::value;
        constexpr int kb = J / QCH, i = J % QCH, s = C * QCH + i;
        if constexpr (s < KSTEPS) {
          constexpr uint32_t imm = (kStageImm ? kStageBytes : 0u) +
                                   2u * (kb * MT * D + (s / KPER) * KPER * M::kK);
          kf[C][kb][i] = lds_read_b128_imm<imm>(kst + koff[s % KPER]);
        }
      });
    };
    // Long contractions alternate between two accumulators per key block
    // (even and odd steps), so back-to-back MFMAs of one block do not wait on
    // each other's result: with one key block per tile, and for the shared
    // K/V ring, whose tiles stream in half the time so the MFMA latency shows
    // (measured: -15 % there, +8 % on the two-ring wide head).
    constexpr bool kTwoChains = (KBLK == 1 && KSTEPS >= 4) || (KVS && KSTEPS >= 8);
    Acc sacc[KBLK], sodd[KBLK];
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb) sacc[kb] = sodd[kb] = Acc{};
    read_k(std::integral_constant<int, 0>{});
    static_for<0, NQC>([&](auto c_c) {
      constexpr int C = decltype(c_c)::value;
      if (kSpread && more_v)  // V copies [C*L/NQC, (C+1)*L/NQC)
        issue_v(v_next, v_stage, std::integral_constant<int, C * CopyV::kLoads / NQC>{},
                std::integral_constant<int, (C + 1) * CopyV::kLoads / NQC>{});
      if constexpr (C + 1 < NQC) read_k(std::integral_constant<int, C + 1>{});
      // chunk C has landed once at most the next chunk's reads are in flight
      constexpr int kNext = (C + 1 < NQC) ? KBLK * ((KSTEPS - (C + 1) * QCH) < QCH
                                                        ? (KSTEPS - (C + 1) * QCH)
                                                        : QCH)
                                          : 0;
      lds_wait<kNext>();
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int i = 0; i < QCH; ++i)
          if (C * QCH + i < KSTEPS) lds_tie(kf[C][kb][i]);
#pragma unroll
      for (int i = 0; i < QCH; ++i)
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) {
          const int s = C * QCH + i;
          if (s < KSTEPS) {
            if (kTwoChains && (s & 1))
              sodd[kb] = M::run(__builtin_bit_cast(bf16x8, kf[C][kb][i]), qf[s], sodd[kb]);
            else
              sacc[kb] = M::run(__builtin_bit_cast(bf16x8, kf[C][kb][i]), qf[s], sacc[kb]);
          }
        }
    });
    if constexpr (kTwoChains) {
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) sacc[kb] += sodd[kb];
    }
    if constexpr (DBG_S) {
      if (row_ok) {
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
          for (int r = 0; r < M::kRegs; ++r) {
            const int key = t0 + kb * MT + acc_row<MT>(lane, r);
            if (key < kend)
              p.s_dbg[(row_base + my_r) * (long long)p.Sk + key] = sacc[kb][r] * p.s_dbg_scale;
          }
      }
    }

    // ---- mask the ragged end and the causal diagonal ----
    const bool need_mask = (t0 + KT > kend) || (CAUSAL && t0 + KT - 1 > wave_min_last);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < M::kRegs; ++r) {
          const int key = t0 + kb * MT + acc_row<MT>(lane, r);
          if (key >= kend || key > my_last) sacc[kb][r] = -__builtin_inff();
        }
    }

    // ---- online softmax (base 2) with lazy rescaling ----
    float mloc = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
      for (int r = 0; r < M::kRegs; ++r) mloc = fmaxf(mloc, sacc[kb][r]);
    mloc = group_max<MT>(mloc) * p.scale_log2;
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
    for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
      for (int r = 0; r < M::kRegs; ++r) {
        const float pv = fast_exp2(__builtin_fmaf(sacc[kb][r], p.scale_log2, -m_run));
        sacc[kb][r] = pv;
        psum += pv;
      }
    l_run += psum;

    // ---- O^T += V^T P^T ----
    // P as the B operand: k-slot e of a lane group holds the key that the S^T
    // register layout put there (the key <-> k-slot map is noted at voff).
    bf16x8 pb[NPV];
#pragma unroll
    for (int step = 0; step < NPV; ++step) {
      u32x4 pw;
      if constexpr (MT == 32) {
        const int kb = step >> 1, t2 = step & 1;
        pw[0] = pack_bf16x2(sacc[kb][8 * t2 + 0], sacc[kb][8 * t2 + 1]);
        pw[1] = pack_bf16x2(sacc[kb][8 * t2 + 2], sacc[kb][8 * t2 + 3]);
        pw[2] = pack_bf16x2(sacc[kb][8 * t2 + 4], sacc[kb][8 * t2 + 5]);
        pw[3] = pack_bf16x2(sacc[kb][8 * t2 + 6], sacc[kb][8 * t2 + 7]);
      } else {
        pw[0] = pack_bf16x2(sacc[2 * step][0], sacc[2 * step][1]);
        pw[1] = pack_bf16x2(sacc[2 * step][2], sacc[2 * step][3]);
        if (2 * step + 1 < KBLK) {
          pw[2] = pack_bf16x2(sacc[2 * step + 1][0], sacc[2 * step + 1][1]);
          pw[3] = pack_bf16x2(sacc[2 * step + 1][2], sacc[2 * step + 1][3]);
        } else {  // a 16-key tile on the 32-deep MFMA: the upper k-slots get P = 0
          pw[2] = pw[3] = 0u;
        }
      }
      pb[step] = __builtin_bit_cast(bf16x8, pw);
    }
    // V^T as the A operand through transpose reads, RA units (one MFMA each)
    // ahead of the MFMAs.
    constexpr int NU = NPV * DBLK;
    constexpr int RA = NU < 4 ? NU : 4;
    constexpr bool kVStageImm = (uint32_t)VST * VTILE * 2 <= 65536u;  // (KVS: VST == KST)
    const uint32_t vst = v_lds + (kVStageImm ? 0u : (uint32_t)STG * VTILE * 2);
    u32x4 vfrag[NU];
    auto issue_v = [&](auto u_c) {
      constexpr int U = decltype(u_c)::value;
      constexpr int step = U / DBLK, db = U % DBLK;
      // stage offset: an instruction immediate when the V ring fits the 16-bit
      // DS offset, else folded into the per-tile base vst
      constexpr uint32_t stage_bytes = kVStageImm ? (uint32_t)STG * VTILE * 2 : 0u;
      constexpr uint32_t row_step = (MT == 32) ? 16u * VW * 2 : 32u * VW * 2;
      constexpr uint32_t col_step = (uint32_t)(db / VPER) * VPER * MT * 2;
      constexpr uint32_t imm1 = stage_bytes + step * row_step + col_step;
      // (a half-filled 32-deep step re-reads its own rows for the zero-P half)
      constexpr uint32_t imm2 = imm1 + ((MT == 32 || KT == 16) ? 0u : 16u * VW * 2);
      const uint32_t a1 = vst + voff[0][db % VPER];
      const u32x2 lo = lds_read_tr16_imm<imm1>(a1);
      const uint32_t a2 = vst + voff[VROWS - 1][db % VPER];
      const u32x2 hi = lds_read_tr16_imm<imm2>(a2);
      vfrag[U] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    static_for<0, RA>([&](auto u_c) { issue_v(u_c); });
    static_for<0, NU>([&](auto u_c) {
      constexpr int U = decltype(u_c)::value;
      if (kSpread && more_k)  // K copies [U*L/NU, (U+1)*L/NU)
        issue_k(k_next, k_stage, std::integral_constant<int, U * nK / NU>{},
                std::integral_constant<int, (U + 1) * nK / NU>{});
      if constexpr (U + RA < NU) issue_v(std::integral_constant<int, U + RA>{});
      constexpr int pending = 2 * ((NU - 1 - U) < RA ? (NU - 1 - U) : RA);
      lds_wait_tied<pending>(vfrag[U]);
      oacc[U % DBLK] =
          M::run(__builtin_bit_cast(bf16x8, vfrag[U]), pb[U / DBLK], oacc[U % DBLK]);
    });
  };

  // Split groups that combine in the workgroup may keep their partials in
  // dynamic LDS instead of the workspace (the launch sizes it, when it leaves
  // the workgroups of the grid resident at once): [row of the workgroup]
  // [split][DV], then the lse values [row][split], for the first
  // min(NW * MT, rows_per_kv) rows.  Through global memory the partial stores
  // write 64 bytes of each of 16 rows per instruction between the splits'
  // tiles, and the partials stay dirty in the L2s for the kernel-end
  // write-back.
  extern __shared__ __attribute__((aligned(16))) float part_lds[];
  const bool plds = GROUP && p.part_lds_bytes > 0;
  const int prows = min(ROWS_WG, p.rows_per_kv);

  // The split-s partial of this workgroup's rows: fp32 O / l and its lse.
  auto write_partial = [&](int s) {
    const float l_tot = group_sum<MT>(l_run);
    const bool empty = !(l_tot > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / l_tot;
    const float lse_val = empty ? -__builtin_inff() : (m_run + __log2f(l_tot)) * kLn2;
    if (plds) {
      if (row_ok) {
        const int lr = my_r - r_wg0;
        const uint32_t base = lds_addr((const FMHA_LDS void*)part_lds);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
#pragma unroll
          for (int qd = 0; qd < M::kRegs / 4; ++qd) {
            const int d0 = (MT == 32) ? db * 32 + 8 * qd + 4 * kg : db * 16 + 4 * kg;
            if (d0 >= DV) continue;
            lds_write_b128_asm(base + 4u * (uint32_t)((lr * p.nsplit + s) * DV + d0),
                               f32x4{oacc[db][4 * qd + 0] * inv, oacc[db][4 * qd + 1] * inv,
                                     oacc[db][4 * qd + 2] * inv, oacc[db][4 * qd + 3] * inv});
          }
        }
        if (kg == 0)
          lds_write_b32_asm(base + 4u * (uint32_t)(prows * p.nsplit * DV + lr * p.nsplit + s),
                            lse_val);
      }
      return;
    }
    if (row_ok) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
#pragma unroll
        for (int qd = 0; qd < M::kRegs / 4; ++qd) {
          const int d0 = (MT == 32) ? db * 32 + 8 * qd + 4 * kg : db * 16 + 4 * kg;
          if (d0 >= DV) continue;
          float* dst = p.o_part + ((row_base + my_r) * p.nsplit + s) * DV + d0;
          *(f32x4*)dst = f32x4{oacc[db][4 * qd + 0] * inv, oacc[db][4 * qd + 1] * inv,
                               oacc[db][4 * qd + 2] * inv, oacc[db][4 * qd + 3] * inv};
        }
      }
      if (kg == 0) p.lse_part[(row_base + my_r) * p.nsplit + s] = lse_val;
    }
  };
  auto reset_state = [&]() {
    m_run = kNegBig;
    l_run = 0.0f;
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = Acc{};
  };
  const int tps = p.split_len / KT;  // tiles per split
  int s_done = 0;                    // splits of the group written so far
  for (int it0 = 0; it0 < ntiles; it0 += LCM) {
    static_for<0, LCM>([&](auto u_c) {
      constexpr int U = decltype(u_c)::value;
      const int it = it0 + U;
      if (it < ntiles) {
        tile(u_c, it);
        if constexpr (GROUP) {
          if ((it + 1) % tps == 0 && it + 1 < ntiles) {  // the last tile of a split
            write_partial(split0 + s_done);
            ++s_done;
            reset_state();
          }
        }
      }
    });
  }

  if constexpr (DBG_S) return;

  // ---- epilogue: O / l, log-sum-exp ----
  if constexpr (SPLIT) {
    if constexpr (GROUP) {
      // the split holding the last tile, then any later split of the group
      // with no visible key (lse = -inf, O = 0)
      for (int j = s_done; j < nspl; ++j) {
        write_partial(split0 + j);
        reset_state();
      }
      if constexpr (DV == 64 || DV == 128) {
        if (p.combine_in_wg) {  // every split of the unit is here: combine in place
          __syncthreads();      // the partial stores of every lane are visible
          const int nr = min(MT, p.rows_per_kv - r_wave0);
          if (nr > 0) {
            if (plds) {
              const FMHA_LDS float* pl = (const FMHA_LDS float*)part_lds;
              combine_wave_rows<DV>(pl, pl + prows * p.nsplit * DV, (long long)(r_wave0 - r_wg0),
                                    p.o, p.lse, row_base + r_wave0, nr, p.nsplit, lane);
            } else {
              combine_wave_rows<DV>((const float*)p.o_part, (const float*)p.lse_part,
                                    row_base + r_wave0, p.o, p.lse, row_base + r_wave0, nr,
                                    p.nsplit, lane);
            }
          }
        }
      }
    } else {
      write_partial(split0);
    }
    return;
  }
  const float l_tot = group_sum<MT>(l_run);
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l_tot;
  const float lse_val = empty ? -__builtin_inff() : (m_run + __log2f(l_tot)) * kLn2;

  float amax = 0.0f;
  // 32-row waves (prefill) with whole 64-column blocks: O leaves the
  // accumulators one row per lane in 8-byte pieces, so a store straight from
  // them writes 16 bytes of each of 32 rows.  The wave's rows go row-major
  // through the K ring, idle after the barrier below, and out as whole rows,
  // 64 lanes x 16 bytes per store, written through (O is not left dirty in
  // the L2s for the write-back at the kernel's end); 16-byte chunks
  // XOR-swizzled by the row.
  constexpr int OCH = DV / 8;  // 16-byte chunks per O row
  constexpr bool kStageO = !SPLIT && MT == 32 && DV % 64 == 0 && OCH <= 64 &&
                           NW * MT * DV <= KST * KTILE;
  if constexpr (kStageO) {
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    lds_barrier();  // every wave past its last ring read
    FMHA_LDS uint16_t* ost = (FMHA_LDS uint16_t*)&ksm[0][0] + wave * (MT * DV);
    // (the lane index laundered through an empty asm, so that the compiler
    // does not hoist these addresses out and hold them through the loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int oc = ln % MT, og = ln / MT;  // = qcol, kg
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const float o0 = oacc[db][4 * qd + 0] * inv, o1 = oacc[db][4 * qd + 1] * inv;
        const float o2 = oacc[db][4 * qd + 2] * inv, o3 = oacc[db][4 * qd + 3] * inv;
        const uint32_t w0 = pack_bf16x2(o0, o1), w1 = pack_bf16x2(o2, o3);
        const int cs = (db * 4 + qd) ^ (oc & (OCH - 1));
        *(FMHA_LDS u32x2*)(ost + oc * DV + cs * 8 + 4 * og) = u32x2{w0, w1};
        if (p.o_amax && row_ok) {
          amax = fmaxf(amax, fabsf(bf16_bits_to_float(w0 & 0xFFFF)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_float(w0 >> 16)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_float(w1 & 0xFFFF)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_float(w1 >> 16)));
        }
      }
    }
    if (p.o) {
      constexpr int RPI = 64 / OCH;  // rows per store
#pragma unroll
      for (int i = 0; i < MT / RPI; ++i) {  // (LDS accesses of one wave stay in order)
        const int row = RPI * i + ln / OCH, ch = ln % OCH;
        const u32x4 val = *(FMHA_LDS u32x4*)(ost + row * DV + ((ch ^ (row & (OCH - 1))) * 8));
        if (r_wave0 + row < p.rows_per_kv)
          global_store_b128_stream(p.o + (row_base + r_wave0 + row) * DV + ch * 8, val);
      }
    }
    if (row_ok && kg == 0 && p.lse) p.lse[row_base + my_r] = lse_val;
  } else if (row_ok) {
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int qd = 0; qd < M::kRegs / 4; ++qd) {
        const int d0 = (MT == 32) ? db * 32 + 8 * qd + 4 * kg : db * 16 + 4 * kg;
        if (d0 >= DV) continue;
        const float o0 = oacc[db][4 * qd + 0] * inv, o1 = oacc[db][4 * qd + 1] * inv;
        const float o2 = oacc[db][4 * qd + 2] * inv, o3 = oacc[db][4 * qd + 3] * inv;
        const uint32_t w0 = pack_bf16x2(o0, o1), w1 = pack_bf16x2(o2, o3);
        if (p.o) *(u32x2*)(p.o + (row_base + my_r) * DV + d0) = u32x2{w0, w1};
        if (p.o_amax) {
          amax = fmaxf(amax, fabsf(bf16_bits_to_float(w0 & 0xFFFF)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_float(w0 >> 16)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_float(w1 & 0xFFFF)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_float(w1 >> 16)));
        }
      }
    }
    if (kg == 0 && p.lse) p.lse[row_base + my_r] = lse_val;
  }
  if (p.o_amax) {
    amax = wave_max(amax);
    if (lane == 0) atomic_max_nonneg(p.o_amax, amax);
  }

  // Fused NVFP4 output (16-row waves): the 16-element block of head dims
  // [16 db, 16 db + 16) of this lane's row is spread over the four lanes kg
  // = 0..3 (4 values each), so its max |x| is a reduction over those lanes.
  // The values quantised are O rounded to bf16, exactly what the standalone
  // quantiser would read back.  All lanes take part in the reductions.
  if constexpr (!SPLIT && MT == 16) {
    if (p.fp4_codes) {
      const float g = *p.fp4_gscale;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const uint32_t w0 = pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv);
        const uint32_t w1 = pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv);
        const float x0 = bf16_bits_to_float(w0 & 0xFFFFu), x1 = bf16_bits_to_float(w0 >> 16);
        const float x2 = bf16_bits_to_float(w1 & 0xFFFFu), x3 = bf16_bits_to_float(w1 >> 16);
        const float ab =
            group_max<16>(fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3))));
        float t;
        const uint32_t sc = nvfp4_block_scale(ab, g, t);
        const uint32_t c = nvfp4_code(x0, sc, t) | (nvfp4_code(x1, sc, t) << 4) |
                           (nvfp4_code(x2, sc, t) << 8) | (nvfp4_code(x3, sc, t) << 12);
        if (row_ok) {
          const long long r = row_base + my_r;
          *(uint16_t*)(p.fp4_codes + r * (DV / 2) + db * 8 + 2 * kg) = (uint16_t)c;
          if (kg == 0) p.fp4_scales[r * (DV / 16) + db] = (uint8_t)sc;
        }
      }
    }
  }
}

// Log-sum-exp combine of split results: one wave per query row.
//   m = max_s lse_s;  LSE = m + log sum_s exp(lse_s - m);
//   O = sum_s exp(lse_s - LSE) * O_s  -> bf16.
// Splits with lse_s = -inf (no visible key) weigh 0.  The split weights are
// computed once, one split per lane (64 splits per pass), and broadcast with
// v_readlane; the partial rows are then read 16 bytes per lane, several
// splits ahead of the accumulation.
template <int D>
__global__ __launch_bounds__(256) void lse_combine_kernel(const float* __restrict__ o_part,
                                                          const float* __restrict__ lse_part,
                                                          uint16_t* __restrict__ o,
                                                          float* __restrict__ lse,
                                                          float* __restrict__ o_amax,
                                                          uint8_t* __restrict__ fp4_codes,
                                                          uint8_t* __restrict__ fp4_scales,
                                                          const float* __restrict__ fp4_gscale,
                                                          long long nrows, int nsplit) {
  static_assert(D % 64 == 0, "combine expects D a multiple of 64");
  // lanes that own 4 consecutive outputs each; the rest idle in the sum
  constexpr int VL = D / 4 < 64 ? D / 4 : 64;   // active lanes
  constexpr int NV = D / (4 * VL);               // float4 groups per active lane
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const float* lp = lse_part + row * nsplit;

  float m = -__builtin_inff();
  for (int s = lane; s < nsplit; s += 64) m = fmaxf(m, lp[s]);
  m = wave_max(m);
  float amax = 0.0f;
  if (m == -__builtin_inff()) {
    if (o)
      for (int e = lane; e < D; e += 64) o[row * D + e] = 0;
    if (fp4_codes) {
      for (int e = lane; e < D / 2; e += 64) fp4_codes[row * (D / 2) + e] = 0;
      for (int e = lane; e < D / 16; e += 64) fp4_scales[row * (D / 16) + e] = 0;
    }
    if (lane == 0 && lse) lse[row] = -__builtin_inff();
  } else {
    float sum = 0.0f;
    for (int s = lane; s < nsplit; s += 64) sum += __expf(lp[s] - m);
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) sum += xor_lane(sum, msk);
    const float L = m + __logf(sum);
    f32x4 acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float* op = o_part + row * nsplit * D + 4 * (lane < VL ? lane : 0);  // idle lanes: in bounds
    for (int s0 = 0; s0 < nsplit; s0 += 64) {
      // this lane's split weight, then broadcast split by split
      const int sl = s0 + lane;
      const float wl = sl < nsplit ? __expf(lp[sl] - L) : 0.0f;
      const int n = nsplit - s0 < 64 ? nsplit - s0 : 64;
      int s = 0;
      for (; s + 4 <= n; s += 4) {
        f32x4 x[4][NV];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < NV; ++v)
            x[u][v] = lane < VL ? *(const f32x4*)(op + (long long)(s0 + s + u) * D + v * 4 * VL)
                                : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s + u));
#pragma unroll
          for (int v = 0; v < NV; ++v) acc[v] += w * x[u][v];
        }
      }
      for (; s < n; ++s) {
        const float w =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s));
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (lane < VL) acc[v] += w * *(const f32x4*)(op + (long long)(s0 + s) * D + v * 4 * VL);
      }
    }
    if (lane < VL) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint32_t w0 = pack_bf16x2(acc[v][0], acc[v][1]);
        const uint32_t w1 = pack_bf16x2(acc[v][2], acc[v][3]);
        if (o) *(u32x2*)(o + row * D + v * 4 * VL + 4 * lane) = u32x2{w0, w1};
        amax = fmaxf(amax, fabsf(bf16_bits_to_float(w0 & 0xFFFF)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_float(w0 >> 16)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_float(w1 & 0xFFFF)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_float(w1 >> 16)));
      }
    }
    if (lane == 0 && lse) lse[row] = L;
    // Fused NVFP4 output: a 16-element block is 4 consecutive lanes here (4
    // values each); every lane takes part in the reduction, idle lanes with 0.
    if (fp4_codes) {
      const float g = *fp4_gscale;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint32_t w0 = pack_bf16x2(acc[v][0], acc[v][1]);
        const uint32_t w1 = pack_bf16x2(acc[v][2], acc[v][3]);
        const float x0 = bf16_bits_to_float(w0 & 0xFFFFu), x1 = bf16_bits_to_float(w0 >> 16);
        const float x2 = bf16_bits_to_float(w1 & 0xFFFFu), x3 = bf16_bits_to_float(w1 >> 16);
        float ab = fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3)));
        ab = fmaxf(ab, xor_lane(ab, 1));
        ab = fmaxf(ab, xor_lane(ab, 2));
        float t;
        const uint32_t sc = nvfp4_block_scale(ab, g, t);
        const uint32_t c = nvfp4_code(x0, sc, t) | (nvfp4_code(x1, sc, t) << 4) |
                           (nvfp4_code(x2, sc, t) << 8) | (nvfp4_code(x3, sc, t) << 12);
        if (lane < VL) {
          const int d0 = v * 4 * VL + 4 * lane;
          *(uint16_t*)(fp4_codes + row * (D / 2) + d0 / 2) = (uint16_t)c;
          if ((lane & 3) == 0) fp4_scales[row * (D / 16) + d0 / 16] = (uint8_t)sc;
        }
      }
    }
  }
  if (o_amax) {
    amax = wave_max(amax);
    if (lane == 0) atomic_max_nonneg(o_amax, amax);
  }
}

}  // namespace fmha
