// fmha_api.cpp -- the C ABI of libfmha.so for attention (see include/fmha.h):
// argument validation, kernel selection, workspace layout and launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/fmha.h"
#include "fmha_device.hpp"
#include "host_common.hpp"
#include "launch.hpp"

namespace fmha {

namespace {
thread_local char g_last_error[512] = "";
}

fmha_status fail(fmha_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

fmha_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FMHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return FMHA_OK;
}

namespace {

constexpr size_t kAlign = 256;
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool decode_dim_ok(int D) { return D == 64 || D == 128 || D == 512; }
// (Q/K head dim, V/O head dim) pairs the decode kernels are built for.
bool decode_dims_ok(int D, int Dv) { return (Dv == D && decode_dim_ok(D)) || (D == 576 && Dv == 512); }
bool fwd_dim_ok(int D) { return D == 16 || D == 32 || D == 64 || D == 128; }

fmha_status check_common(const void* q, const void* k, const void* v, const void* o, int B,
                         int Hq, int Hkv, int Sq, int Sk, float scale, int causal) {
  if (!q || !k || !v || !o) return fail(FMHA_ERR_NULL, "q, k, v and o must be non-null");
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1)
    return fail(FMHA_ERR_SHAPE, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Sq=%d Sk=%d)", B, Hq, Hkv,
                Sq, Sk);
  if (Hq % Hkv != 0) return fail(FMHA_ERR_GQA, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (causal != 0 && causal != 1) return fail(FMHA_ERR_ARG, "causal must be 0 or 1");
  if (causal && Sq > Sk)
    return fail(FMHA_ERR_SHAPE, "causal attention needs Sq <= Sk (Sq=%d Sk=%d)", Sq, Sk);
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return fail(FMHA_ERR_ARG, "scale must be positive and finite");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(FMHA_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  return FMHA_OK;
}

bool sizes_fit(long long B, long long Hq, long long Hkv, long long Sq, long long Sk, long long D) {
  // 64-bit element offsets are used throughout; keep every tensor below 2^61 elements.
  return B * Hq * Sq * D < (1LL << 61) && B * Hkv * Sk * D < (1LL << 61);
}

// The kernels index a 1-D grid with 32-bit ints.
bool grid_fits(long long row_blocks, long long splits, long long Hkv, long long B) {
  return row_blocks * splits * Hkv * B < (1LL << 31);
}

}  // namespace

int num_cus() {
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return n > 0 ? n : 256;
  }();
  return cus;
}

namespace {

// Clears the amax accumulator of a decode call (a kernel on the call's stream,
// so the whole call can be captured in a graph).
__global__ void clear_f32_kernel(float* p) { *p = 0.0f; }

// Keys per split: equal ranges rounded up to the KV tile.
int split_len_for(int Sk, int nsplit, int kt) {
  int len = (Sk + nsplit - 1) / nsplit;
  return (len + kt - 1) / kt * kt;
}

}  // namespace

int default_splits(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || Hq % Hkv) return 1;
  const int rows = (Hq / Hkv) * Sq;
  const DecodeCfg c = decode_cfg(D, rows);
  const long long n_rb = (rows + 16 * c.nw - 1) / (16 * c.nw);
  const long long units = (long long)B * Hkv * n_rb;
  // Fill every workgroup slot of the GPU once; keep at least 4 tiles per split.
  const long long want_wgs = (long long)c.wgs_per_cu * num_cus();
  int ns = 1;
  while ((long long)ns * units < want_wgs && ns < 1024 && Sk / (2 * ns) >= 4 * c.kt) ns *= 2;
  return ns;
}

}  // namespace fmha

using namespace fmha;

extern "C" {

const char* fmha_status_string(fmha_status s) {
  switch (s) {
    case FMHA_OK: return "ok";
    case FMHA_ERR_NULL: return "null pointer";
    case FMHA_ERR_SHAPE: return "invalid shape";
    case FMHA_ERR_HEAD_DIM: return "unsupported head dimension";
    case FMHA_ERR_GQA: return "Hq is not a multiple of Hkv";
    case FMHA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FMHA_ERR_WORKSPACE: return "workspace missing or too small";
    case FMHA_ERR_HIP: return "HIP error";
    case FMHA_ERR_ARG: return "invalid argument";
  }
  return "unknown status";
}

const char* fmha_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

// (Q/K head dim, V/O head dim) pairs the prefill kernels are built for.
bool fwd_dims_ok(int D, int Dv) { return (Dv == D && fwd_dim_ok(D)) || (D == 192 && Dv == 128); }

fmha_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int Hq, int Hkv, int Sq, int Sk, int D, int Dv, float scale, int causal,
                     void* stream) {
  fmha_status s = check_common(q, k, v, o, B, Hq, Hkv, Sq, Sk, scale, causal);
  if (s != FMHA_OK) return s;
  if (lse && !aligned16(lse)) return fail(FMHA_ERR_ALIGN, "lse must be 16-byte aligned");
  if (!fwd_dims_ok(D, Dv))
    return fail(FMHA_ERR_HEAD_DIM,
                "prefill supports D = Dv in {16,32,64,128} and (D, Dv) = (192, 128), got (%d, %d)",
                D, Dv);
  if (!sizes_fit(B, Hq, Hkv, Sq, Sk, D > Dv ? D : Dv))
    return fail(FMHA_ERR_SHAPE, "tensor too large");
  // the prefill kernels address one head's K/V rows with 32-bit byte offsets
  // (up to three tiles past the last key)
  if (((long long)Sk + 4 * 64) * (D > Dv ? D : Dv) * 2 >= (1LL << 32))
    return fail(FMHA_ERR_SHAPE, "Sk * head dim too large for the prefill (K/V rows of one head "
                "must stay below 4 GiB)");
  AttnParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.B = B;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.rows_per_kv = (Hq / Hkv) * Sq;
  p.n_row_blocks = (p.rows_per_kv + 127) / 128;
  p.nsplit = 1;
  p.split_len = (Sk + 63) / 64 * 64;
  p.splits_per_wg = 1;
  p.scale_log2 = scale * kLog2e;
  if (!grid_fits(p.n_row_blocks, 1, Hkv, B)) return fail(FMHA_ERR_SHAPE, "grid too large");
  return launch_fwd(D, Dv, p, causal != 0, (hipStream_t)stream);
}

}  // namespace

extern "C" {

fmha_status fmha_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int Hq, int Hkv, int Sq, int Sk, int D, float scale, int causal,
                     void* stream) {
  g_last_error[0] = 0;
  if (D == 192) return fail(FMHA_ERR_HEAD_DIM, "D = 192 needs Dv: use fmha_fwd_dv");
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, D, scale, causal, stream);
}

fmha_status fmha_fwd_dv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int Hq, int Hkv, int Sq, int Sk, int D, int Dv, float scale, int causal,
                        void* stream) {
  g_last_error[0] = 0;
  if (k == v && Dv != D)  // the decode reads that as V inside the K rows
    return fail(FMHA_ERR_ARG, "fmha_fwd_dv: V inside the K rows (v == k) is built for the decode only");
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, Dv, scale, causal, stream);
}

int fmha_decode_default_splits(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
  return default_splits(B, Hq, Hkv, Sq, Sk, D);
}

size_t fmha_decode_splitkv_dv_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                             int Dv, int num_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || Hq % Hkv || !decode_dims_ok(D, Dv) ||
      num_splits < 0 || num_splits > 1024)
    return 0;
  int ns = num_splits ? num_splits : default_splits(B, Hq, Hkv, Sq, Sk, D);
  if (ns <= 1) return 0;
  const size_t rows = (size_t)B * Hq * Sq;
  return round_up(rows * ns * Dv * sizeof(float), kAlign) +
         round_up(rows * ns * sizeof(float), kAlign);
}

size_t fmha_decode_splitkv_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                          int num_splits) {
  if (!decode_dim_ok(D)) return 0;
  return fmha_decode_splitkv_dv_workspace_size(B, Hq, Hkv, Sq, Sk, D, D, num_splits);
}

}  // extern "C"

namespace {

// A paged K/V cache: per-batch key counts and a block table (device arrays).
struct PagedDesc {
  const int* seqlens;
  const int* block_table;
  int bt_stride;
  int page_shift;
  int num_pages;
};

// Split-KV decode; with fp4_codes set, the output epilogue (attention kernel
// without splits, combine kernel with) also writes the NVFP4 encoding of O
// for the caller's global scale, and o may be null.  With pg set, K and V are
// paged caches and Sk is the table's reach.
fmha_status decode_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int Hq, int Hkv, int Sq, int Sk, int D, int Dv, float scale, int causal,
                        int num_splits, void* workspace, size_t workspace_bytes, float* o_amax,
                        uint8_t* fp4_codes, uint8_t* fp4_scales, const float* fp4_gscale,
                        const PagedDesc* pg, void* stream) {
  // o is optional only for the fused NVFP4 output; q stands in for its checks
  fmha_status s = check_common(q, k, v, (o || !fp4_codes) ? o : q, B, Hq, Hkv, Sq, Sk, scale,
                               causal);
  if (s != FMHA_OK) return s;
  if (lse && !aligned16(lse)) return fail(FMHA_ERR_ALIGN, "lse must be 16-byte aligned");
  if (o_amax && ((uintptr_t)o_amax & 3)) return fail(FMHA_ERR_ALIGN, "o_amax must be 4-byte aligned");
  if (!decode_dims_ok(D, Dv))
    return fail(FMHA_ERR_HEAD_DIM,
                "decode supports D = Dv in {64,128,512} and (D, Dv) = (576, 512), got (%d, %d)",
                D, Dv);
  if (Dv != D && (pg || fp4_codes || o_amax))
    return fail(FMHA_ERR_HEAD_DIM, "Dv != D is built for the plain split-KV decode only");
  if (num_splits < 0 || num_splits > 1024)
    return fail(FMHA_ERR_ARG, "num_splits must be in 0..1024, got %d", num_splits);
  if (!sizes_fit(B, Hq, Hkv, Sq, Sk, D > Dv ? D : Dv))
    return fail(FMHA_ERR_SHAPE, "tensor too large");

  const int rows_per_kv = (Hq / Hkv) * Sq;
  const DecodeCfg c = decode_cfg(D, rows_per_kv);
  int ns = num_splits ? num_splits : default_splits(B, Hq, Hkv, Sq, Sk, D);
  const int split_len = split_len_for(Sk, ns, c.kt);
  const int ns_eff = (Sk + split_len - 1) / split_len;  // trailing empty ranges dropped

  AttnParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.o_amax = o_amax;
  p.fp4_codes = fp4_codes;
  p.fp4_scales = fp4_scales;
  p.fp4_gscale = fp4_gscale;
  p.B = B;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.rows_per_kv = rows_per_kv;
  p.n_row_blocks = (rows_per_kv + 16 * c.nw - 1) / (16 * c.nw);
  p.nsplit = ns_eff;
  p.split_len = split_len;
  p.splits_per_wg = 1;
  p.scale_log2 = scale * kLog2e;
  if (pg) {
    p.seqlens = pg->seqlens;
    p.block_table = pg->block_table;
    p.bt_stride = pg->bt_stride;
    p.page_shift = pg->page_shift;
    p.num_pages = pg->num_pages;
  }
  const hipStream_t st = (hipStream_t)stream;
  if (!grid_fits(p.n_row_blocks, ns_eff, Hkv, B)) return fail(FMHA_ERR_SHAPE, "grid too large");
  if (o_amax) {
    hipLaunchKernelGGL(clear_f32_kernel, dim3(1), dim3(1), 0, st, o_amax);
    s = check_launch("amax clear launch");
    if (s != FMHA_OK) return s;
  }

  // V aliasing K (the same buffer): at head dim 512, or with V the first Dv
  // columns of the K rows, each key row is then streamed from HBM once and
  // serves both products
  const bool kv_shared = !pg && (k == v) && (D == 512 || Dv < D);
  // (the wide-head kernel for V inside the K rows has no amax or NVFP4 epilogue)
  const bool wide = !pg && !o_amax && !fp4_codes && decode_wide_takes(D, Dv, Sk, kv_shared);
  auto attention = [&](dim3 grid, bool split) {
    if (pg) return launch_decode_paged(D, c, p, grid, causal != 0, split, st);
    if (wide) return launch_decode_wide(D, Dv, p, grid, causal != 0, split, false, st);
    return launch_decode(D, Dv, c, p, grid, causal != 0, split, kv_shared, st);
  };
  if (ns_eff <= 1) {
    dim3 grid((unsigned)p.n_row_blocks * Hkv * B);
    return attention(grid, false);
  }

  const size_t need = fmha_decode_splitkv_dv_workspace_size(B, Hq, Hkv, Sq, Sk, D, Dv, ns);
  if (!workspace || workspace_bytes < need)
    return fail(FMHA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(FMHA_ERR_ALIGN, "workspace must be 16-byte aligned");
  const size_t rows = (size_t)B * Hq * Sq;
  p.o_part = (float*)workspace;
  p.lse_part = (float*)((char*)workspace + round_up(rows * ns * Dv * sizeof(float), kAlign));
  // Split groups: when the (row block, batch, KV head) units alone give every
  // CU at least two workgroups and all fit the GPU's workgroup slots at once,
  // one workgroup streams all splits of its unit back to back (the same
  // partials, no short-lived workgroups).  Measured on the GQA decode (512
  // units, 16 splits): 169 us against 178 us contiguous, 176 against 180 us
  // from a shuffled page pool; with 1 unit per CU or fewer the split
  // parallelism is needed, and partial groups measured slower.
  if (decode_groups_built(D, Dv, kv_shared)) {
    const long long units = (long long)p.n_row_blocks * Hkv * B;
    if (units >= 2LL * num_cus() && units <= (long long)c.wgs_per_cu * num_cus())
      p.splits_per_wg = ns_eff;
  }
  // A workgroup holding every split of its unit combines them itself (the
  // combine kernel's arithmetic; the amax fold and the NVFP4 output stay with
  // that kernel): one launch fewer.
  p.combine_in_wg = (p.splits_per_wg == ns_eff && !o_amax && !fp4_codes) ? 1 : 0;
  const int nsg = (ns_eff + p.splits_per_wg - 1) / p.splits_per_wg;
  dim3 grid((unsigned)p.n_row_blocks * nsg * Hkv * B);
  s = attention(grid, true);
  if (s != FMHA_OK || p.combine_in_wg) return s;
  return launch_combine(Dv, p.o_part, p.lse_part, (uint16_t*)o, lse, o_amax, fp4_codes,
                        fp4_scales, fp4_gscale, (long long)rows, ns_eff, st);
}

}  // namespace

extern "C" {

fmha_status fmha_decode_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                                int causal, int num_splits, void* workspace,
                                size_t workspace_bytes, float* o_amax, void* stream) {
  g_last_error[0] = 0;
  if (D == 576) return fail(FMHA_ERR_HEAD_DIM, "D = 576 needs Dv: use fmha_decode_splitkv_dv");
  return decode_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, D, scale, causal, num_splits,
                     workspace, workspace_bytes, o_amax, nullptr, nullptr, nullptr, nullptr,
                     stream);
}

}  // extern "C"

namespace {

// Split partials of fmha_decode_splitkv_noalloc: a fixed device array, one
// copy per GPU, held until the process ends.  Its name is a host-side
// stand-in in host code; kernels get the device address that
// hipGetSymbolAddress returns for the current device (scratch_ptr).
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (with that device current); null after a HIP error (recorded).
void* scratch_ptr() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(FMHA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(FMHA_ERR_HIP, "device %d out of the supported range", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(FMHA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

fmha_status fmha_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                        float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                        float scale, int causal, int num_splits, float* o_amax,
                                        void* stream) {
  g_last_error[0] = 0;
  // host-only checks first: nothing touches the device before they pass
  fmha_status s = check_common(q, k, v, o, B, Hq, Hkv, Sq, Sk, scale, causal);
  if (s != FMHA_OK) return s;
  if (!decode_dim_ok(D))
    return fail(FMHA_ERR_HEAD_DIM, "fmha_decode_splitkv_noalloc: D in {64, 128, 512}, got %d", D);
  if (num_splits < 0 || num_splits > 1024)
    return fail(FMHA_ERR_ARG, "num_splits must be in 0..1024, got %d", num_splits);
  const size_t need = fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, num_splits);
  if (need > kScratchBytes)
    return fail(FMHA_ERR_WORKSPACE,
                "fmha_decode_splitkv_noalloc: the split partials need %zu bytes, more than the "
                "%zu bytes of its fixed scratch; use fewer splits or fmha_decode_splitkv",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_ptr();
    if (!ws) return FMHA_ERR_HIP;
  }
  return decode_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, D, scale, causal, num_splits, ws,
                     need > 0 ? kScratchBytes : 0, o_amax, nullptr, nullptr, nullptr, nullptr,
                     stream);
}

fmha_status fmha_decode_splitkv_dv(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                   int Dv, float scale, int causal, int num_splits,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return decode_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, Dv, scale, causal, num_splits,
                     workspace, workspace_bytes, nullptr, nullptr, nullptr, nullptr, nullptr,
                     stream);
}

fmha_status fmha_decode_splitkv_nvfp4(const void* q, const void* k, const void* v, void* o,
                                      float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                      float scale, int causal, int num_splits, void* workspace,
                                      size_t workspace_bytes, const float* global_scale,
                                      uint8_t* codes, uint8_t* scales, void* stream) {
  g_last_error[0] = 0;
  if (!global_scale || !codes || !scales)
    return fail(FMHA_ERR_NULL, "global_scale, codes and scales must be non-null");
  if (((uintptr_t)codes & 7u) || ((uintptr_t)global_scale & 3u))
    return fail(FMHA_ERR_ALIGN, "codes must be 8-byte aligned and global_scale 4-byte");
  if (D == 576) return fail(FMHA_ERR_HEAD_DIM, "the fused NVFP4 decode is built for D = Dv");
  return decode_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, D, scale, causal, num_splits,
                     workspace, workspace_bytes, nullptr, codes, scales, global_scale, nullptr,
                     stream);
}

fmha_status fmha_decode_paged(const void* q, const void* k_cache, const void* v_cache, void* o,
                              float* lse, int B, int Hq, int Hkv, int Sq, const int* seqlens_k,
                              const int* block_table, int max_pages_per_seq, int page_size,
                              int num_pages, int D, float scale, int causal, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!seqlens_k || !block_table)
    return fail(FMHA_ERR_NULL, "seqlens_k and block_table must be non-null");
  if (((uintptr_t)seqlens_k & 3u) || ((uintptr_t)block_table & 3u))
    return fail(FMHA_ERR_ALIGN, "seqlens_k and block_table must be 4-byte aligned");
  if (page_size < 64 || page_size > (1 << 24) || (page_size & (page_size - 1)))
    return fail(FMHA_ERR_ARG, "page_size must be a power of two in [64, 2^24], got %d",
                page_size);
  if (max_pages_per_seq < 1 || (long long)max_pages_per_seq * page_size > (1LL << 30))
    return fail(FMHA_ERR_ARG, "max_pages_per_seq * page_size must be in [page_size, 2^30]");
  if (num_pages < 1) return fail(FMHA_ERR_ARG, "num_pages must be >= 1, got %d", num_pages);
  if (Hkv >= 1 && decode_dim_ok(D) &&
      (long long)num_pages * page_size * Hkv * D >= (1LL << 61))
    return fail(FMHA_ERR_SHAPE, "cache too large");
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  const PagedDesc pg{seqlens_k, block_table, max_pages_per_seq, shift, num_pages};
  if (D == 576) return fail(FMHA_ERR_HEAD_DIM, "the paged decode is built for D = Dv");
  return decode_impl(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Sq, max_pages_per_seq * page_size,
                     D, D, scale, causal, num_splits, workspace, workspace_bytes, nullptr, nullptr,
                     nullptr, nullptr, &pg, stream);
}

fmha_status fmha_debug_qk_scores(const void* q, const void* k, const void* v, float* s_out,
                                 int B, int Hq, int Hkv, int Sq, int Sk, int D, int Dv,
                                 float scale, int decode, void* stream) {
  g_last_error[0] = 0;
  if (!s_out) return fail(FMHA_ERR_NULL, "s_out must be non-null");
  fmha_status s = check_common(q, k, v, s_out, B, Hq, Hkv, Sq, Sk, scale, 0);
  if (s != FMHA_OK) return s;
  if (decode != 0 && decode != 1) return fail(FMHA_ERR_ARG, "decode must be 0 or 1");
  if (decode ? !decode_dims_ok(D, Dv) : !fwd_dims_ok(D, Dv))
    return fail(FMHA_ERR_HEAD_DIM, "debug scores: head dims D=%d, Dv=%d not built", D, Dv);
  if (!decode && k == v && Dv != D)
    return fail(FMHA_ERR_ARG, "debug scores: V inside the K rows is built for the decode only");
  if ((long long)B * Hq * Sq * Sk >= (1LL << 31))
    return fail(FMHA_ERR_SHAPE, "debug scores: s_out larger than 2^31 elements");
  const int rows_per_kv = (Hq / Hkv) * Sq;
  const DecodeCfg c = decode ? decode_cfg(D, rows_per_kv) : DecodeCfg{4, 64, 3};
  const int rows_wg = decode ? 16 * c.nw : 128;
  AttnParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.B = B;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.rows_per_kv = rows_per_kv;
  p.n_row_blocks = (rows_per_kv + rows_wg - 1) / rows_wg;
  p.nsplit = 1;
  p.split_len = (Sk + c.kt - 1) / c.kt * c.kt;
  p.splits_per_wg = 1;
  p.scale_log2 = scale * kLog2e;
  p.s_dbg = s_out;
  p.s_dbg_scale = scale;
  if (!grid_fits(p.n_row_blocks, 1, Hkv, B)) return fail(FMHA_ERR_SHAPE, "grid too large");
  const bool kv_shared = decode && (k == v) && (D == 512 || Dv < D);
  dim3 grid((unsigned)p.n_row_blocks * Hkv * B);
  return launch_debug_scores(D, Dv, c, p, grid, decode != 0, kv_shared, (hipStream_t)stream);
}

}  // extern "C"
