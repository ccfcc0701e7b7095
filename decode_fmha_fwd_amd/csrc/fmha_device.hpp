// fmha_device.hpp -- gfx950 device primitives for the attention kernels:
// MFMA tile wrappers, bf16 packing, exp2, wavefront cross-lane reductions and
// the LDS transpose read used to feed V to the matrix cores.
//
// Register layouts of the two bf16 MFMA shapes used here (lane = 0..63):
//   v_mfma_f32_32x32x16_bf16  A[32 x 16] * B[16 x 32] -> C[32 x 32]
//     A: lane holds A[lane % 32][8*(lane / 32) + e], e = 0..7
//     B: lane holds B[8*(lane / 32) + e][lane % 32]
//     C: lane holds C[8*(r / 4) + 4*(lane / 32) + r % 4][lane % 32], r = 0..15
//   v_mfma_f32_16x16x32_bf16  A[16 x 32] * B[32 x 16] -> C[16 x 16]
//     A: lane holds A[lane % 16][8*(lane / 16) + e]
//     B: lane holds B[8*(lane / 16) + e][lane % 16]
//     C: lane holds C[4*(lane / 16) + r][lane % 16], r = 0..3
// Because a contraction index may be permuted freely as long as A and B agree,
// the kernels choose which key or head-dim element sits in each k-slot.
//
// ds_read_b64_tr_b16 (LDS transpose read), per group of 16 lanes: source lane
// 4*j + a supplies the address of four consecutive bf16 elements; destination
// lane 4*a + e receives, for j = 0..3, element e of source lane 4*j + a.
// Pointing source lane (j, a) at row (r0 + j), columns (c0 + 4a .. c0 + 4a + 3)
// of a row-major tile therefore gives lane (4a + e) the column c0 + 4a + e of
// rows r0 .. r0 + 3: a column read, which is what an MFMA operand that
// contracts over rows needs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

#define FMHA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no score seen yet": exp2(x - kNegBig) never becomes
// NaN the way (-inf) - (-inf) would for a row whose first tile is masked.
constexpr float kNegBig = -1.0e30f;

template <int MT> struct Mfma;

template <> struct Mfma<32> {
  using Acc = f32x16;
  static constexpr int kRegs = 16;
  static constexpr int kK = 16;          // contraction length per instruction
  static constexpr int kKGroups = 2;     // lane groups that split the contraction
  __device__ static inline Acc run(bf16x8 a, bf16x8 b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<16> {
  using Acc = f32x4;
  static constexpr int kRegs = 4;
  static constexpr int kK = 32;
  static constexpr int kKGroups = 4;
  __device__ static inline Acc run(bf16x8 a, bf16x8 b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// Row index (within an MT-row block) of accumulator register r in this lane.
template <int MT> __device__ inline int acc_row(int lane, int r);
template <> __device__ inline int acc_row<32>(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
template <> __device__ inline int acc_row<16>(int lane, int r) { return 4 * (lane >> 4) + r; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) packed low/high into one
// dword: a single v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ inline float bf16_bits_to_float(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane exchange of one float with lane ^ mask (mask 16 or 32).
__device__ inline float xor_lane(float v, int mask) {
  int lane = __lane_id();
  int src = lane ^ mask;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

// Symmetric exchange across lane halves without the LDS crossbar (gfx950
// v_permlane{16,32}_swap, lane layout checked on the GPU): with both operands
// holding v, the swap leaves in every lane its own value and its partner's
// (lane ^ 16, resp. lane ^ 32), so a commutative op on the pair is the
// pairwise reduction.
template <int HALF>
__device__ inline void swap_halves(float v, float& x, float& y) {
  const unsigned a = __builtin_bit_cast(unsigned, v);
  unsigned r0, r1;
  if constexpr (HALF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  x = __builtin_bit_cast(float, r0);
  y = __builtin_bit_cast(float, r1);
}
template <int HALF>
__device__ inline float pair_max(float v) {
  float x, y;
  swap_halves<HALF>(v, x, y);
  return fmaxf(x, y);
}
template <int HALF>
__device__ inline float pair_sum(float v) {
  float x, y;
  swap_halves<HALF>(v, x, y);
  return x + y;
}

// Reductions over the lanes that hold the same query column of an MT-wide
// MFMA output (lanes that differ only in bits above log2(MT)).
template <int MT> __device__ inline float group_max(float v);
template <> __device__ inline float group_max<32>(float v) { return pair_max<32>(v); }
template <> __device__ inline float group_max<16>(float v) { return pair_max<32>(pair_max<16>(v)); }
template <int MT> __device__ inline float group_sum(float v);
template <> __device__ inline float group_sum<32>(float v) { return pair_sum<32>(v); }
template <> __device__ inline float group_sum<16>(float v) { return pair_sum<32>(pair_sum<16>(v)); }

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, xor_lane(v, m));
  return v;
}

// The LDS transpose read of four bf16 (see the header comment), issued from
// inline asm: the compiler cannot tell which LDS bytes a transpose-read
// builtin touches, so it would wait for every outstanding global->LDS copy
// (vmcnt(0)) before each one, serialising the prefetch ring; from asm it
// inserts nothing, and the caller must wait (lds_wait_tied) before using the
// result.  A constant LDS byte offset is folded into the instruction
// (offset < 64 KiB).
template <uint32_t OFF>
__device__ inline u32x2 lds_read_tr16_imm(uint32_t lds_addr) {
  static_assert(OFF < 65536u, "DS offset field is 16 bits");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFF));
  return r;
}

// 16-byte global store that writes through the caches to memory and does not
// keep the line (nt sc0 sc1: non-temporal, system scope).  For output read by
// no later part of the kernel: written back during the kernel instead of by
// the cache write-back at its end.  (gfx950 has no builtin that sets these
// bits on a store; a plain store from asm, nothing waits on it.)
__device__ inline void global_store_b128_stream(void* dst, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off nt sc0 sc1" ::"v"(dst), "v"(v) : "memory");
}

// LDS writes issued from inline asm: a compiler-visible LDS access while
// asynchronous global->LDS copies are in flight makes the compiler wait for
// all of them first (vmcnt(0)); these write a region no copy targets.  The
// caller waits (lgkmcnt) before anything reads what they wrote.
__device__ inline void lds_write_b128_asm(uint32_t lds_addr, f32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(lds_addr), "v"(v) : "memory");
}
__device__ inline void lds_write_b32_asm(uint32_t lds_addr, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr), "v"(v) : "memory");
}

// 16-byte LDS read issued from inline asm, with a constant byte offset
// folded into the instruction, for the same reason as the transpose reads: a
// compiler-visible LDS read after asynchronous global->LDS copies makes the
// compiler wait for every copy in flight (vmcnt(0)) first.
template <uint32_t OFF>
__device__ inline u32x4 lds_read_b128_imm(uint32_t lds_addr) {
  static_assert(OFF < 65536u, "DS offset field is 16 bits");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFF));
  return r;
}

// s_waitcnt lgkmcnt(N) with no register tie; follow it with lds_tie on each
// result it covers.
template <int N>
__device__ inline void lds_wait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
}

// Marks r as produced here (after a preceding lds_wait), so no use of r can be
// scheduled before that wait.
template <typename T>
__device__ inline void lds_tie(T& r) {
  asm volatile("" : "+v"(r));
}

// s_waitcnt lgkmcnt(N) tied to a register tuple, so the compiler cannot use
// the tuple before the wait.  LDS operations complete in order, so waiting for
// at most N outstanding means everything issued before the last N is done.
template <int N, typename T>
__device__ inline void lds_wait_tied(T& r) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}

__device__ inline uint32_t lds_addr(const FMHA_LDS void* p) { return (uint32_t)(size_t)p; }

__device__ inline u32x4 lds_read_b128(const FMHA_LDS void* p) {
  return *(const FMHA_LDS u32x4*)p;
}

__device__ inline void lds_write_b128(FMHA_LDS void* p, u32x4 v) { *(FMHA_LDS u32x4*)p = v; }

// Asynchronous global -> LDS copy of 16 (or 4) bytes per lane
// (global_load_lds_dwordx4 / _dword): lane l's bytes land at lds_base +
// BYTES*l, where lds_base is the same for every lane of the wave (it goes
// to M0).  Completion is tracked by vmcnt like any global load; the compiler
// does not order LDS reads after these writes, so callers wait explicitly
// (wait_vmcnt) and then barrier before reading what other waves copied.
// NT selects the non-temporal cache policy (the "nt" bit): data read once
// (decode K/V) streams through without displacing reusable lines; measured
// here it raises streaming throughput of these copies by about 10%.
template <int BYTES, bool NT>
__device__ inline void dma_to_lds(const void* g, FMHA_LDS void* lds_base) {
  static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword copies");
  const __attribute__((address_space(1))) void* gp = (const __attribute__((address_space(1))) void*)g;
  constexpr int kAux = NT ? 2 : 0;  // cache-policy operand: bit 1 = nt
  if constexpr (BYTES == 16) {
    __builtin_amdgcn_global_load_lds(gp, lds_base, 16, 0, kAux);
  } else {
    __builtin_amdgcn_global_load_lds(gp, lds_base, 4, 0, kAux);
  }
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt split over bits 3:0 and 15:14;
// expcnt and lgkmcnt left at their maxima, i.e. not waited for).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0): all of this wave's LDS reads and writes have finished.
__device__ inline void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier that orders LDS accesses in the compiler without the
// memory-model fences of __syncthreads (whose release fence would also wait
// for every outstanding LDS copy, defeating the prefetch).  Callers wait for
// their own outstanding LDS traffic first.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Float bits of a non-negative float order like unsigned integers, so a
// max over magnitudes can use an integer atomic.
__device__ inline void atomic_max_nonneg(float* addr, float v) {
  atomicMax((unsigned int*)addr, __builtin_bit_cast(unsigned int, v));
}

}  // namespace fmha
