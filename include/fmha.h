/*
 * fmha.h -- C ABI of libfmha.so: fused multi-head attention forward, split-KV
 * decode with a log-sum-exp combine, and an NVFP4 output quantiser, as
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The page "NVFP4-1.1_RAW_CUDA_CPP_APPROACH.md" (its
 * seven-point feature list) names the parts of the fused kernel: a QK matrix
 * product, an in-kernel softmax with rescaling of the output accumulator, a
 * loop over several KV tiles, a PV product, a correction epilogue and an FP4
 * quantisation of the output; the same page names multi-CTA (split-KV) work
 * and head dimension 512 among the goals.  Written out:
 *
 *     S[i, j] = scale * sum_d Q[i, d] * K[j, d]       (bf16 inputs, fp32 sum)
 *     P[i, j] = exp(S[i, j] - LSE[i]),   LSE[i] = log sum_{j visible} exp(S[i, j])
 *     O[i, :] = sum_{j visible} P[i, j] * V[j, :]
 *
 * The page "CURRENT ISSUE: UMMA QK GEMM -- 4x Scaling Bug" (section "The 4x
 * Bug") is the reminder that S must equal the scalar dot product times
 * `scale`, with no other factor.
 *
 * Conventions shared by every call:
 *   - bf16 tensors are raw 16-bit patterns (uint16), row-major, last index
 *     fastest, in the (batch, head, sequence, head_dim) order used for Q on the
 *     page "nvfp4-megamoe-kernel/CURRENT_ISSUE.md" (Q viewed as (B, H, 1, HD),
 *     batch stride H*HD):
 *         q [B, Hq, Sq, D]   k [B, Hkv, Sk, D]   v [B, Hkv, Sk, D]
 *         o [B, Hq, Sq, D]   lse [B, Hq, Sq] (fp32, natural log)
 *   - Grouped heads: query head h reads KV head h / (Hq / Hkv).
 *   - Causal mask, aligned to the bottom-right corner: key j is visible to query
 *     row i iff j <= i + (Sk - Sq).  Masked keys are left out entirely.
 *   - All pointers are DEVICE pointers owned by the caller and must be 16-byte
 *     aligned; the library never allocates device memory and never
 *     synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and runs asynchronously.
 *   - Every argument is checked on the host before anything is launched; on
 *     any error nothing is written and a non-zero fmha_status comes back.
 *     After each launch the HIP launch status is checked (FMHA_ERR_HIP).
 *   - Thread-safe: the only library state is a per-thread error string and a
 *     cached device-property query.
 */
#ifndef FMHA_H
#define FMHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FMHA_OK = 0,
    FMHA_ERR_NULL = 1,       /* a required pointer is NULL                          */
    FMHA_ERR_SHAPE = 2,      /* a size < 1, causal with Sq > Sk, cols % 16 != 0 ... */
    FMHA_ERR_HEAD_DIM = 3,   /* head dimension not built for this entry point       */
    FMHA_ERR_GQA = 4,        /* Hq is not a multiple of Hkv                         */
    FMHA_ERR_ALIGN = 5,      /* a pointer is not 16-byte aligned                    */
    FMHA_ERR_WORKSPACE = 6,  /* workspace missing or smaller than the size query    */
    FMHA_ERR_HIP = 7,        /* a HIP launch or runtime call failed                 */
    FMHA_ERR_ARG = 8         /* another argument out of range (scale <= 0 or NaN,
                                num_splits < 0, ...)                               */
} fmha_status;

/*
 * Fused attention forward (prefill and general Sq).
 *   q, k, v: bf16, layouts above.  o: bf16 [B, Hq, Sq, D] output.
 *   lse: fp32 [B, Hq, Sq] output, or NULL to skip it.
 *   D in {16, 32, 64, 128}.  scale > 0 (e.g. 1/sqrt(D) rounded to fp32).
 *   causal: 0 or 1 (causal requires Sq <= Sk).
 * One workgroup computes a 128-row tile of query rows against all visible KV
 * tiles with an online softmax (the feature list's "softmax with O rescale"
 * over "multi-KV-tile" loops), then normalises and stores O and LSE.
 */
fmha_status fmha_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale, int causal,
                     void* stream);

/*
 * Attention forward with a V/O head dimension Dv different from the Q/K head
 * dimension D (the workload list names the V head dimension apart from the
 * Q/K one).  The built pair is D = 192, Dv = 128 (128 content dimensions plus
 * 64 more key dimensions in Q and K).  Everything else is fmha_fwd:
 *   q [B, Hq, Sq, D], k [B, Hkv, Sk, D], v [B, Hkv, Sk, Dv], o [B, Hq, Sq, Dv],
 *   lse [B, Hq, Sq] or NULL.
 *   (D, Dv): (192, 128), or D == Dv in {16, 32, 64, 128} (then exactly
 *   fmha_fwd).  Anything else: FMHA_ERR_HEAD_DIM.  v must be its own tensor:
 *   the K buffer passed as V with Dv != D (the decode's "V inside the K
 *   rows") is rejected with FMHA_ERR_ARG.
 */
fmha_status fmha_fwd_dv(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Sq, int Sk, int D, int Dv, float scale,
                        int causal, void* stream);

/*
 * Bytes of device workspace fmha_decode_splitkv needs for these sizes and this
 * number of splits (0 = the library's choice, see fmha_decode_default_splits).
 * Returns 0 when no workspace is needed (one split) or the sizes are invalid.
 */
size_t fmha_decode_splitkv_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                          int num_splits);

/*
 * Split-KV decode (small Sq, e.g. 1): the keys of each (batch, KV head) are cut
 * into num_splits contiguous ranges (equal lengths rounded up to the KV tile;
 * trailing splits may be empty).  One workgroup handles all query rows that
 * share a KV head (the Hq/Hkv grouped heads times Sq) over one range, or over
 * all ranges of its (batch, KV head) back to back when those units alone fill
 * the GPU, and writes an fp32 partial output and its log-sum-exp per range to
 * the workspace; a second kernel combines them:  LSE = m + log sum_s exp(lse_s - m),  m = max_s lse_s,
 * O = sum_s exp(lse_s - LSE) * O_s  (a workgroup that holds all ranges of its
 * (batch, KV head) combines them itself, with the same arithmetic, unless
 * o_amax is given).  With one split the first kernel writes O and LSE
 * directly and no workspace is used.
 *   D in {64, 128, 512}; the Sq*Hq/Hkv rows of a KV head are taken in
 *   blocks of 16 or 64 (one workgroup each).
 *   num_splits: 0 = heuristic, otherwise 1..1024.
 *   workspace / workspace_bytes: device buffer of at least
 *     fmha_decode_splitkv_workspace_size(...) bytes (may be NULL when that is 0).
 *   o_amax: NULL, or a device fp32 that receives max|O| over the bf16 O the
 *     call writes (the call clears it first, with a kernel on `stream`); this
 *     folds the NVFP4 quantiser's tensor-wide amax into the decode, so
 *     nvfp4_quantize(..., amax_in = o_amax, ...) needs no amax pass.
 */
fmha_status fmha_decode_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                                int causal, int num_splits, void* workspace,
                                size_t workspace_bytes, float* o_amax, void* stream);

/*
 * fmha_decode_splitkv for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, with the split partials in a fixed scratch
 * array inside the library instead of a caller workspace.  Nothing is
 * allocated and no workspace is passed; inputs and outputs are the caller's,
 * as for fmha_decode_splitkv (same arguments without workspace /
 * workspace_bytes, same results bit for bit).
 *   Limit: fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D,
 *     num_splits) must not exceed 64 MiB (67108864 bytes); a larger request
 *     returns FMHA_ERR_WORKSPACE before anything is launched (choose fewer
 *     splits, or use fmha_decode_splitkv).  One split needs no scratch.
 *   The scratch is 64 MiB of device memory on every GPU the library runs on,
 *     held until the process ends; its address is looked up once per device
 *     (the first call on that device, with it current).  Every call on one
 *     GPU shares that GPU's scratch, so calls that overlap on one GPU (on
 *     different streams, or from different threads without ordering) race
 *     and may produce wrong results; calls ordered on one stream are safe.
 *     Each call writes every partial it reads, so no clearing is needed.
 */
fmha_status fmha_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                        float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                        float scale, int causal, int num_splits, float* o_amax,
                                        void* stream);

/* The split count used when num_splits == 0. */
int fmha_decode_default_splits(int B, int Hq, int Hkv, int Sq, int Sk, int D);

/*
 * Split-KV decode with a V/O head dimension Dv different from the Q/K head
 * dimension D.  The page "NVFP4-1.1_RAW_CUDA_CPP_APPROACH.md" singles out head
 * dimension 512 among its goals, and the workload list names the V head
 * dimension apart from the Q/K one; the built pair is the shared-latent shape
 * D = 576, Dv = 512 (a 512-wide latent that serves as V plus 64 more key
 * dimensions).  The arithmetic is that of fmha_decode_splitkv:
 *     S[i, j] = scale * sum_{d < D} Q[i, d] * K[j, d],   O[i, :] = sum_j P[i, j] * V[j, :Dv]
 *   q [B, Hq, Sq, D], k [B, Hkv, Sk, D], o [B, Hq, Sq, Dv], lse [B, Hq, Sq].
 *   v: either a separate bf16 [B, Hkv, Sk, Dv] tensor, or the very pointer
 *     passed as k, which makes V the first Dv columns of each K row (row
 *     stride D): each key row then crosses HBM once and serves both products.
 *   (D, Dv): (576, 512), or D == Dv in {64, 128, 512} (then exactly
 *     fmha_decode_splitkv).  Anything else: FMHA_ERR_HEAD_DIM.
 *   workspace_bytes >= fmha_decode_splitkv_dv_workspace_size(...) (fp32
 *     partials of width Dv).  num_splits, causal, scale, errors and the
 *     execution model: as fmha_decode_splitkv.
 */
size_t fmha_decode_splitkv_dv_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                             int Dv, int num_splits);
fmha_status fmha_decode_splitkv_dv(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                   int Dv, float scale, int causal, int num_splits,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace nvfp4_quantize needs (room for one fp32 amax).
 */
size_t nvfp4_quantize_workspace_size(long long rows, int cols);

/*
 * NVFP4 quantisation of a bf16 matrix x [rows, cols], cols % 16 == 0 (the
 * feature list's last item, "FP4 quantization" of the output).  Recipe, every
 * step one correctly rounded fp32 operation:
 *   amax = max |x| (over the whole tensor, or *amax_in when given);
 *   g = amax / 2688  (2688 = 6 * 448)                      -> *global_scale
 *   per block of 16 contiguous elements of a row:
 *     s = E4M3((amax_block / 6) / g)     (OCP E4M3FN, nearest-even, saturating)
 *     t = value(s) * g
 *     code = E2M1(x / t)                 (OCP E2M1, nearest-even, saturating;
 *                                         bit 3 = sign of x / t)
 *   codes [rows, cols/2]: byte = code[2k+1] << 4 | code[2k];
 *   scales [rows, cols/16]: one E4M3 byte per block, row-major.
 * amax == 0 (or g underflowing to 0) gives g = 0 and all codes and scales 0; a
 * block with s == 0 (or t underflowing to 0) gets all codes 0.
 *   amax_in: NULL, or a device fp32 holding max|x| (e.g. the o_amax of
 *     fmha_decode_splitkv), which skips the amax pass.
 *   workspace: at least nvfp4_quantize_workspace_size() bytes (used only when
 *     amax_in is NULL).
 */
fmha_status nvfp4_quantize(const void* x, long long rows, int cols, uint8_t* codes,
                           uint8_t* scales, float* global_scale, const float* amax_in,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split-KV decode with the NVFP4 quantisation fused into its output epilogue,
 * for callers that already hold the global scale g (e.g. from a previous step
 * or a calibration pass), so no tensor-wide amax pass is needed: the "FP4
 * quantization" item of the feature list done inside the kernel.  Everything
 * else is as fmha_decode_splitkv.  The values quantised are O rounded to bf16,
 * so codes and scales equal nvfp4_quantize of that O with this g; the per-block
 * recipe (s, t, codes, packing, zero cases) is nvfp4_quantize's with
 * g = *global_scale instead of amax / 2688.  The epilogue that produces the
 * final O does the encoding: the attention kernel without splits, the combine
 * kernel with them.
 *   o: bf16 [B, Hq, Sq, D] output, or NULL to skip writing it.
 *   global_scale: device fp32 (read, not written).
 *   codes: [B*Hq*Sq, D/2] bytes, 8-byte aligned; scales: [B*Hq*Sq, D/16] bytes.
 */
fmha_status fmha_decode_splitkv_nvfp4(const void* q, const void* k, const void* v, void* o,
                                      float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                      float scale, int causal, int num_splits, void* workspace,
                                      size_t workspace_bytes, const float* global_scale,
                                      uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Split-KV decode over a paged, variable-length KV cache: the arithmetic,
 * splits and combine of fmha_decode_splitkv, with K and V read through a block
 * table instead of from one contiguous [B, Hkv, Sk, D] tensor each (the cache
 * layout of a serving loop; the paging itself is not one of the pages' items).
 *   k_cache, v_cache: bf16 [num_pages, Hkv, page_size, D] (head-major pages:
 *     a head's keys of one page are contiguous), 16-byte aligned.
 *   seqlens_k: device int32 [B], the number of keys of each batch; values are
 *     clamped to [0, max_pages_per_seq * page_size].  A batch with no keys (or,
 *     causal, a query row that sees none) gets O = 0 and LSE = -inf.
 *   block_table: device int32 [B, max_pages_per_seq]; key j of batch b, KV
 *     head h, is row j % page_size of head h of page block_table[b][j / page_size].  Page ids are
 *     clamped to [0, num_pages), so a bad entry reads a wrong page, never
 *     outside the cache; only the pages of the first ceil(seqlens_k[b] /
 *     page_size) entries of a row are read (later entries of the row may be
 *     looked up ahead, never followed).  Neither array may change while the
 *     call runs.
 *   page_size: a power of two, at least 64 (a key tile never straddles pages).
 *   causal: bottom-right aligned per batch (row i sees keys j <= i + len_b - Sq).
 *   Sk for the split choice and the workspace is max_pages_per_seq * page_size:
 *     workspace_bytes >= fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq,
 *     max_pages_per_seq * page_size, D, num_splits).
 *   D, num_splits, q, o, lse: as fmha_decode_splitkv (no o_amax).
 * Errors (nothing launched): FMHA_ERR_NULL for a null pointer, FMHA_ERR_ARG
 * for a page size, page count or table width out of range, and the checks of
 * fmha_decode_splitkv.  seqlens_k and block_table stay on the device; their
 * values are not checked on the host.
 */
fmha_status fmha_decode_paged(const void* q, const void* k_cache, const void* v_cache, void* o,
                              float* lse, int B, int Hq, int Hkv, int Sq, const int* seqlens_k,
                              const int* block_table, int max_pages_per_seq, int page_size,
                              int num_pages, int D, float scale, int causal, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test hook: the raw scores S = scale * Q K^T of every (query row, key) pair,
 * computed by the QK block of the attention kernel itself -- the global->LDS
 * copy ring, the inline-asm LDS reads of K and the MFMA accumulation chains
 * of the production kernel, built with a flag that stores each score tile as
 * it leaves that block (before masking and softmax) and skips the outputs.
 * The page "CURRENT ISSUE: UMMA QK GEMM -- 4x Scaling Bug" (sections "The 4x
 * Bug" and "How to fix") is why: its MMA result differed from the scalar dot
 * product by a factor of 4; on integer-valued inputs every partial sum here is
 * exact, so S must equal scale * <q, k> bit for bit.
 *   decode = 0: the prefill kernel fmha_fwd / fmha_fwd_dv would launch for
 *     (D, Dv) (32-row waves, 32x32x16 MFMAs); decode = 1: the one-split
 *     kernel fmha_decode_splitkv / _dv would launch (16-row waves, 16x16x32
 *     MFMAs), with v == k selecting the shared-ring form where that exists --
 *     at (512, 512) and (576, 512) the wide-head decode (32-row waves, each
 *     with half of the head dims, 32x32x16 MFMAs; the score of a pair is the
 *     sum of its two halves' partials, as in that kernel).
 *   q, k, v: as for those calls; non-causal.
 *   s_out: fp32 [B * Hq * Sq, Sk] (row = (b * Hq + h) * Sq + i), every entry
 *     written; B * Hq * Sq * Sk < 2^31.
 * Errors: the argument checks of the matching call, FMHA_ERR_HEAD_DIM for a
 * (D, Dv) pair that path is not built for.
 */
fmha_status fmha_debug_qk_scores(const void* q, const void* k, const void* v, float* s_out,
                                 int B, int Hq, int Hkv, int Sq, int Sk, int D, int Dv,
                                 float scale, int decode, void* stream);

const char* fmha_status_string(fmha_status s);

/* Detail for the calling thread's last non-OK return ("" if none). */
const char* fmha_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FMHA_H */
