/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the fused
 * multi-head attention forward / split-KV decode path and its NVFP4 output
 * quantiser.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * What the pages fix, and what is read into them:
 *   - "NVFP4-1.1_RAW_CUDA_CPP_APPROACH.md", the seven-point feature list: a
 *     QK matrix product, an in-kernel softmax whose running state rescales
 *     the output accumulator, a loop over several KV tiles, a PV product, a
 *     correction epilogue and an FP4 quantisation of the output.  The pages
 *     never write the formula; a tiled online softmax reaches, up to rounding
 *     order, the plain softmax-attention result, so that plain definition is
 *     what is written out here (two passes over a materialised row, fp64).
 *   - "CURRENT ISSUE: UMMA QK GEMM -- 4x Scaling Bug", section "The 4x Bug":
 *     the QK product must equal the scalar dot product with no stray factor;
 *     here the dot product IS the scalar loop.
 *   - The FP4 recipe (e2m1 values in blocks of 16 along a row, an E4M3 scale
 *     per block, one fp32 per-tensor scale amax/(6*448), round to nearest
 *     even) is not spelled out on the pages beyond "FP4 quantization for
 *     NVFP4"; the formats are the OCP ones (OCP 8-bit Floating Point
 *     Specification for E4M3FN, OCP Microscaling Formats v1.0 for E2M1).
 *
 * Precision: attention in fp64 from the exact bf16 inputs; the quantiser in
 * IEEE fp32, one rounded operation at a time (built with -ffp-contract=off,
 * no fast-math), because it decides integer codes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* bf16 <-> binary64                                                   */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a binary64 straight to bf16 (8 significant bits, binary32 exponent
 * range), round-to-nearest, ties to even, overflow to infinity -- in one
 * rounding (no detour through binary32, which could round twice). */
uint16_t oracle_double_to_bf16(double x)
{
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    frexp(a, &e);            /* a in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < -126) ex = -126; /* below the normal range the spacing is fixed */
    double quantum = ldexp(1.0, ex - 7);
    double r = nearbyint(a / quantum) * quantum; /* default mode: ties to even */
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    float rf = (float)r;     /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* O1: attention, the plain definition                                 */
/* ------------------------------------------------------------------ */

/* Layouts (row-major, last index fastest), as on the first page's Q load
 * (Q viewed as (B, H, 1, HD) with a batch stride of H*HD):
 *   q [B, Hq, Sq, D], k [B, Hkv, Sk, D], v [B, Hkv, Sk, Dv]   (bf16 bits)
 * Query head h reads KV head h / (Hq / Hkv).
 * Causal visibility (aligned to the bottom-right corner): key j is visible to
 * query row i iff j <= i + (Sk - Sq).  Masked keys are excluded outright.
 *
 * rows: flat row ids r = (b*Hq + h)*Sq + i to evaluate (NULL: all of them,
 * in order).  Outputs: o[nrows, Dv] (unrounded fp64) and lse[nrows] =
 * natural log of the sum of exp(score) over visible keys.  A row with no
 * visible key gets o = 0 and lse = -inf.
 *
 * kv_begin/kv_end restrict the keys to [kv_begin, kv_end) before the mask,
 * which is how one split of a split-KV decode is described. */
static void attention_row(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          int Hq, int Hkv, int Sq, int Sk, int D, int Dv,
                          double scale, int causal, int kv_begin, int kv_end,
                          long long r, double *s, double *o_row, double *lse_out)
{
    long long i = r % Sq;
    long long bh = r / Sq;
    long long h = bh % Hq;
    long long b = bh / Hq;
    long long kvh = h / (Hq / Hkv);
    const uint16_t *qi = q + ((b * Hq + h) * Sq + i) * (long long)D;
    const uint16_t *kb = k + (b * Hkv + kvh) * (long long)Sk * D;
    const uint16_t *vb = v + (b * Hkv + kvh) * (long long)Sk * Dv;

    /* pass 1: scores of the visible keys and their maximum */
    long long last = causal ? i + (Sk - Sq) : (long long)Sk - 1;
    int n = 0;
    double m = -INFINITY;
    for (long long j = kv_begin; j < kv_end; ++j) {
        if (j > last) break;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += oracle_bf16_to_double(qi[d]) * oracle_bf16_to_double(kb[j * D + d]);
        s[n] = scale * dot;
        if (s[n] > m) m = s[n];
        ++n;
    }
    for (int d = 0; d < Dv; ++d) o_row[d] = 0.0;
    if (n == 0) { *lse_out = -INFINITY; return; }

    /* pass 2: exponentials, their sum, and the weighted sum of V rows */
    double l = 0.0;
    for (int t = 0; t < n; ++t) {
        double e = exp(s[t] - m);
        l += e;
        const uint16_t *vj = vb + (long long)(kv_begin + t) * Dv;
        for (int d = 0; d < Dv; ++d) o_row[d] += e * oracle_bf16_to_double(vj[d]);
    }
    for (int d = 0; d < Dv; ++d) o_row[d] /= l;
    *lse_out = m + log(l);
}

static int shape_ok(int B, int Hq, int Hkv, int Sq, int Sk, int D, int Dv)
{
    return B >= 1 && Hq >= 1 && Hkv >= 1 && Sq >= 1 && Sk >= 0 && D >= 1 && Dv >= 1 &&
           Hq % Hkv == 0;
}

int oracle_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D, int Dv,
                     double scale, int causal,
                     long long nrows, const long long *rows,
                     double *o, double *lse, int nthreads)
{
    if (!q || !k || !v || !o || !lse) return 1;
    if (!shape_ok(B, Hq, Hkv, Sq, Sk, D, Dv)) return 2;
    long long total = (long long)B * Hq * Sq;
    if (!rows) nrows = total;
    for (long long t = 0; t < (rows ? nrows : 0); ++t)
        if (rows[t] < 0 || rows[t] >= total) return 2;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
#pragma omp for schedule(dynamic, 1)
        for (long long t = 0; t < nrows; ++t) {
            long long r = rows ? rows[t] : t;
            if (!s) {
#pragma omp atomic write
                err = 3;
                continue;
            }
            attention_row(q, k, v, Hq, Hkv, Sq, Sk, D, Dv, scale, causal, 0, Sk, r, s,
                          o + t * Dv, lse + t);
        }
        free(s);
    }
    return err;
}

/* ------------------------------------------------------------------ */
/* O2: split-KV, then the log-sum-exp combine                          */
/* ------------------------------------------------------------------ */

/* Split s covers keys [s*chunk, min(Sk, (s+1)*chunk)).  For each split the
 * split-normalised output and its log-sum-exp are formed as in O1 over that
 * key range only (empty split: o = 0, lse = -inf).
 * o_part[nrows, nsplit, Dv], lse_part[nrows, nsplit]. */
int oracle_attention_splits(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            int B, int Hq, int Hkv, int Sq, int Sk, int D, int Dv,
                            double scale, int causal, int nsplit, int chunk,
                            double *o_part, double *lse_part, int nthreads)
{
    if (!q || !k || !v || !o_part || !lse_part) return 1;
    if (!shape_ok(B, Hq, Hkv, Sq, Sk, D, Dv) || nsplit < 1 || chunk < 1) return 2;
    long long nrows = (long long)B * Hq * Sq;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (long long r = 0; r < nrows; ++r)
            for (int sp = 0; sp < nsplit; ++sp) {
                if (!s) {
#pragma omp atomic write
                    err = 3;
                    continue;
                }
                long long b0 = (long long)sp * chunk;
                long long b1 = b0 + chunk;
                if (b0 > Sk) b0 = Sk;
                if (b1 > Sk) b1 = Sk;
                attention_row(q, k, v, Hq, Hkv, Sq, Sk, D, Dv, scale, causal, (int)b0,
                              (int)b1, r, s, o_part + (r * nsplit + sp) * Dv,
                              lse_part + r * nsplit + sp);
            }
        free(s);
    }
    return err;
}

/* Combine per row: m* = max_s lse_s; lse = m* + ln sum_s exp(lse_s - m*);
 * o = sum_s exp(lse_s - lse) * o_s.  Splits with lse_s = -inf weigh 0; a row
 * whose splits are all empty gets o = 0, lse = -inf. */
int oracle_combine(const double *o_part, const double *lse_part, long long nrows,
                   int nsplit, int Dv, double *o, double *lse)
{
    if (!o_part || !lse_part || !o || !lse) return 1;
    if (nrows < 0 || nsplit < 1 || Dv < 1) return 2;
    for (long long r = 0; r < nrows; ++r) {
        const double *ls = lse_part + r * nsplit;
        double m = -INFINITY;
        for (int s = 0; s < nsplit; ++s)
            if (ls[s] > m) m = ls[s];
        for (int d = 0; d < Dv; ++d) o[r * Dv + d] = 0.0;
        if (m == -INFINITY) { lse[r] = -INFINITY; continue; }
        double sum = 0.0;
        for (int s = 0; s < nsplit; ++s) sum += exp(ls[s] - m);
        double L = m + log(sum);
        for (int s = 0; s < nsplit; ++s) {
            double w = exp(ls[s] - L);
            for (int d = 0; d < Dv; ++d) o[r * Dv + d] += w * o_part[(r * nsplit + s) * Dv + d];
        }
        lse[r] = L;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O3: NVFP4 quantiser, IEEE binary32 one step at a time               */
/* ------------------------------------------------------------------ */

/* Value of an OCP E4M3FN code (sign 1, exponent 4 with bias 7, mantissa 3;
 * no infinities; 0x7F/0xFF are NaN; exponent field 0 is subnormal m*2^-9). */
double oracle_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest E4M3FN code to a non-negative x, ties to the code whose lowest bit
 * is 0 (round half to even), saturating to the largest finite value 448
 * (code 0x7E).  Written as a search over the 127 finite non-negative codes. */
uint8_t oracle_e4m3_encode(float x)
{
    if (!(x > 0.0f)) return 0;          /* zero (and the never-used negatives/NaN) */
    if ((double)x >= 448.0) return 0x7E;
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs((double)x - oracle_e4m3_value((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
    }
    return (uint8_t)best;
}

/* E2M1 magnitudes for codes 0..7 (OCP MX: sign, 2 exponent bits with bias 1,
 * 1 mantissa bit). */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(uint8_t c)
{
    double m = kE2M1[c & 7];
    return (c & 8) ? -m : m;
}

/* Nearest E2M1 code to q (round half to even among the 8 magnitudes,
 * saturating to 6); bit 3 carries the sign of q, so a negative q that rounds
 * to magnitude 0 encodes as 0x8. */
uint8_t oracle_e2m1_encode(float q)
{
    uint8_t sign = signbit(q) ? 8 : 0;
    double a = fabs((double)q);
    if (isnan(q)) return 0;
    if (a >= 6.0) return sign | 7;
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(a - kE2M1[c]);
        if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
    }
    return sign | (uint8_t)best;
}

/* The per-block part of the NVFP4 recipe for a given global scale g: per
 * 16-element block along a row of the bf16 matrix x[rows, cols]
 * (cols % 16 == 0): s = E4M3((amax_b / 6) / g), t = value(s) * g, and for
 * each element code = E2M1(x / t);
 *   codes[r, c/2] = code[c+1] << 4 | code[c]   (low nibble = even element),
 *   scales[r, c/16] = s.
 * g <= 0 gives all scales and codes 0; a block with s == 0, or with t
 * underflowing to 0, gets all codes 0.  Every arithmetic step is one
 * correctly rounded binary32 operation.  (The tensor-wide recipe below uses
 * g = amax / 2688; a caller that already holds g, e.g. from an earlier step,
 * quantises with it directly.) */
int oracle_nvfp4_quantize_with_scale(const uint16_t *x, long long rows, int cols, float g,
                                     uint8_t *codes, uint8_t *scales)
{
    if (!x || !codes || !scales) return 1;
    if (rows < 0 || cols < 16 || cols % 16) return 2;
    int nb = cols / 16;
    for (long long r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const uint16_t *blk = x + r * cols + b * 16;
            uint8_t *cb = codes + r * (cols / 2) + b * 8;
            float ab = 0.0f;
            for (int e = 0; e < 16; ++e) {
                float a = fabsf((float)oracle_bf16_to_double(blk[e]));
                if (a > ab) ab = a;
            }
            uint8_t s = 0;
            volatile float t = 0.0f;
            if (g > 0.0f) {
                volatile float sixth = ab / 6.0f;
                volatile float sf = sixth / g;
                s = oracle_e4m3_encode(sf);
                t = (float)oracle_e4m3_value(s) * g;
            }
            scales[r * nb + b] = s;
            for (int e = 0; e < 16; e += 2) {
                uint8_t c0 = 0, c1 = 0;
                if (s != 0 && t > 0.0f) {
                    volatile float q0 = (float)oracle_bf16_to_double(blk[e]) / t;
                    volatile float q1 = (float)oracle_bf16_to_double(blk[e + 1]) / t;
                    c0 = oracle_e2m1_encode(q0);
                    c1 = oracle_e2m1_encode(q1);
                }
                cb[e / 2] = (uint8_t)((c1 << 4) | c0);
            }
        }
    }
    return 0;
}

/* Quantise a bf16 matrix x[rows, cols] (cols % 16 == 0) to NVFP4:
 *   amax = max |x| over the whole tensor; g = amax / 2688 (2688 = 6*448);
 *   then the per-block recipe above with that g; *gscale = g.
 * amax == 0 (or g underflowing to 0) gives g = 0 and all scales and codes 0. */
int oracle_nvfp4_quantize(const uint16_t *x, long long rows, int cols,
                          uint8_t *codes, uint8_t *scales, float *gscale)
{
    if (!x || !codes || !scales || !gscale) return 1;
    if (rows < 0 || cols < 16 || cols % 16) return 2;
    float amax = 0.0f;
    for (long long i = 0; i < rows * cols; ++i) {
        float a = fabsf((float)oracle_bf16_to_double(x[i]));
        if (a > amax) amax = a;
    }
    volatile float g = amax / 2688.0f;
    *gscale = g;
    return oracle_nvfp4_quantize_with_scale(x, rows, cols, g, codes, scales);
}

/* ------------------------------------------------------------------ */
/* Array forms of the codecs (for exhaustive tests)                    */
/* ------------------------------------------------------------------ */

void oracle_double_to_bf16_array(const double *x, long long n, uint16_t *out)
{
    for (long long i = 0; i < n; ++i) out[i] = oracle_double_to_bf16(x[i]);
}

void oracle_bf16_to_double_array(const uint16_t *h, long long n, double *out)
{
    for (long long i = 0; i < n; ++i) out[i] = oracle_bf16_to_double(h[i]);
}

void oracle_e4m3_encode_array(const float *x, long long n, uint8_t *out)
{
    for (long long i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

void oracle_e2m1_encode_array(const float *x, long long n, uint8_t *out)
{
    for (long long i = 0; i < n; ++i) out[i] = oracle_e2m1_encode(x[i]);
}

/* Threads the OpenMP loops above will use (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
