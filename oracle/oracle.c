/*
 * oracle.c -- plain, slow, fp64 CPU reference for the decode-context-parallel
 * (DCP) LSE merge and for the per-shard MLA decode partials that feed it.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only callers.  The product library
 * (the HIP code under context_lse_merge_amd/) never links, loads or calls this
 * file, and this file includes none of its headers: the two share no code.
 *
 * Every value is widened to double before any arithmetic; bf16 inputs are
 * decoded here, bit by bit, by this file's own routine.  No blocking, no
 * fusion and no reordering beyond the definitions below.  OpenMP only spreads
 * independent output rows over threads; each row's arithmetic is the same
 * sequential loop whatever the thread count.
 *
 * What is computed, and where the pages fix it:
 *
 *  merge  -- "[DCP] Run fi_a2a on FlashInfer's fused all-to-all + LSE reduce"
 *            (sglang PR #40539), Motivation: the received head partials are
 *            combined by an LSE-weighted merge.  Modifications: the [B, H, D]
 *            attention output is read as [B, H/cp, cp, D] and its LSE as
 *            [B, H/cp, cp]; head h belongs to shard h // (H/cp), so shard s of
 *            local head j is head s*(H/cp) + j.  Accuracy Tests: FlashMLA's
 *            [B, H, 1] LSE layout is accepted as well; both LSE bases (2, e).
 *            "[Attention] Add direct symmetric-memory DCP A2A" (vLLM PR
 *            #48897), commit message: the combine weights received states by
 *            their LSE in FP32; port commit: an empty shard publishes
 *            LSE = -inf, its payload is not written, and zero-weight sources
 *            are skipped.  "[DCP] Optimize shared Output, Query, and
 *            Indexer/Top-K via peer memory" (sglang PR #32851), commit log:
 *            a row that selected no token weighs in with exp2 of -inf, i.e.
 *            zero, and its merged result must be zero rather than NaN.
 *            The pages name the merge but never print its formula; it is the
 *            split-softmax identity
 *                M   = max_s lse_s
 *                w_s = base^(lse_s - M)            (0 for lse_s = -inf)
 *                S   = sum_s w_s
 *                out = sum_s (w_s / S) * O_s
 *                L   = M + log_base(S)
 *            which the tests pin against brute-force softmax attention.
 *
 *  attention partials -- the producer behind the merge: each DCP shard runs
 *            MLA decode attention over its own slice of the latent KV cache
 *            (PR #32851 commit log: KV tokens are owned by DCP ranks; the
 *            backend returns the LSE with the output).  In the MLA absorbed
 *            form the value is the first 512 latent columns of the cached row
 *            (PR #48897 review thread: head_dim = kv_lora_rank = 512), and the
 *            query/key dot product runs over all 576 columns (512 latent +
 *            64 rope).  For one query row and a token set T:
 *                z_t = scale * <q, k_t>
 *                lse = ln sum_{t in T} exp(z_t)     (times log2 e in base 2)
 *                O   = sum_{t in T} softmax(z)_t * v_t
 *            An empty token set gives lse = -inf and O = 0.
 *
 *  variable-length partials -- the same per query token b over its own
 *            cache of L_b = seq_lens[b] tokens ("[Attention] Add direct
 *            symmetric-memory DCP A2A", vLLM PR #48897, amended port commit:
 *            the decode seq_lens decide which KV shards are empty; an empty
 *            shard publishes -inf).  Shard s owns either a contiguous slice
 *            [floor(s L/cp), floor((s+1) L/cp)) or, with the latent KV spread
 *            over the DCP ranks in interleaved order ("[DCP] Optimize shared Output,
 *            Query, and Indexer/Top-K via peer memory", sglang PR #32851,
 *            commit log), the tokens t < L with t mod cp = s.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* LSE bases and layouts, as the oracle numbers them. */
#define ORACLE_BASE_E 0
#define ORACLE_BASE_2 1
#define ORACLE_LSE_BHC 0 /* [B, H/cp, cp] contiguous: element (b, j, s)        */
#define ORACLE_LSE_BH1 1 /* [B, H, 1] contiguous: element (b, s*(H/cp) + j)    */

#define ORACLE_BF16 0
#define ORACLE_F16 1
#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* bf16 is the upper half of an IEEE binary32: widen the 16 bits into the top
 * of a 32-bit word and reinterpret.  Exact for every finite value, infinity
 * and NaN. */
double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void oracle_decode_bf16(const uint16_t* src, double* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_bf16_to_f64(src[i]);
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent field 0 holds zero and the subnormals, fraction * 2^-24; field 31
 * holds infinity (fraction 0) and NaN; otherwise the value is
 * (1024 + fraction) * 2^(exponent - 25).  Every value is exact in double. */
double oracle_f16_to_f64(uint16_t bits) {
    const int sign = (bits >> 15) & 1;
    const int expo = (bits >> 10) & 0x1F;
    const int frac = bits & 0x3FF;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac == 0 ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

void oracle_decode_f16(const uint16_t* src, double* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f16_to_f64(src[i]);
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Offset of LSE element (b, j, s) in a contiguous array of the given layout. */
static int64_t lse_offset(int layout, int64_t b, int64_t j, int64_t s, int64_t h_local, int64_t cp) {
    if (layout == ORACLE_LSE_BHC) return (b * h_local + j) * cp + s;
    return b * (h_local * cp) + s * h_local + j; /* BH1: head s*H_local + j */
}

/*
 * LSE-weighted merge over cp shards, all in double.
 *   O       [B, H, D] contiguous; shard s of local head j is head s*H_local + j
 *   lse     contiguous, layout ORACLE_LSE_BHC or ORACLE_LSE_BH1
 *   out     [B, H_local, D]      merged output
 *   out_lse [B, H_local]         merged LSE, same base as the input (nullable)
 *   out_abs [B, H_local, D]      sum_s (w_s/S) |O_s|, the magnitude the
 *                                rounding tolerance is scaled by (nullable)
 * An empty shard (lse = -inf) is never read.  An all-empty row gives out = 0
 * and L = -inf.
 */
int oracle_merge_f64(const double* O, const double* lse, int64_t B, int64_t H, int64_t cp, int64_t D,
                     int lse_layout, int lse_mode, double* out, double* out_lse, double* out_abs,
                     int nthreads) {
    if (B < 0 || H <= 0 || cp <= 0 || D <= 0 || H % cp != 0) return ORACLE_BAD_ARG;
    if (lse_layout != ORACLE_LSE_BHC && lse_layout != ORACLE_LSE_BH1) return ORACLE_BAD_ARG;
    if (lse_mode != ORACLE_BASE_E && lse_mode != ORACLE_BASE_2) return ORACLE_BAD_ARG;
    const int64_t h_local = H / cp;
    set_threads(nthreads);

#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < B * h_local; ++row) {
        const int64_t b = row / h_local;
        const int64_t j = row % h_local;
        double* w = (double*)malloc((size_t)cp * sizeof(double));

        double M = -INFINITY;
        for (int64_t s = 0; s < cp; ++s) {
            double x = lse[lse_offset(lse_layout, b, j, s, h_local, cp)];
            if (x > M) M = x;
        }

        double* o_row = out + row * D;
        double* a_row = out_abs ? out_abs + row * D : NULL;
        if (M == -INFINITY) {
            for (int64_t d = 0; d < D; ++d) {
                o_row[d] = 0.0;
                if (a_row) a_row[d] = 0.0;
            }
            if (out_lse) out_lse[row] = -INFINITY;
            free(w);
            continue;
        }

        double S = 0.0;
        for (int64_t s = 0; s < cp; ++s) {
            double x = lse[lse_offset(lse_layout, b, j, s, h_local, cp)];
            if (x == -INFINITY) {
                w[s] = 0.0;
            } else if (lse_mode == ORACLE_BASE_E) {
                w[s] = exp(x - M);
            } else {
                w[s] = exp2(x - M);
            }
            S += w[s];
        }

        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t s = 0; s < cp; ++s) {
                if (w[s] == 0.0) continue; /* empty shard: payload never read */
                double o = O[(b * H + s * h_local + j) * D + d];
                acc += (w[s] / S) * o;
                acc_abs += (w[s] / S) * fabs(o);
            }
            o_row[d] = acc;
            if (a_row) a_row[d] = acc_abs;
        }
        if (out_lse) out_lse[row] = M + (lse_mode == ORACLE_BASE_E ? log(S) : log2(S));
        free(w);
    }
    return ORACLE_OK;
}

/* Same merge on the product's input types: 16-bit O (raw bits, decoded by
 * `decode`) and fp32 LSE.  Both are widened exactly to double first. */
static int merge_16bit(void (*decode)(const uint16_t*, double*, int64_t), const uint16_t* O, const float* lse,
                       int64_t B, int64_t H, int64_t cp, int64_t D, int lse_layout, int lse_mode, double* out,
                       double* out_lse, double* out_abs, int nthreads) {
    if (B < 0 || H <= 0 || cp <= 0 || D <= 0 || H % cp != 0) return ORACLE_BAD_ARG;
    const int64_t n_o = B * H * D, n_l = B * H;
    double* Od = (double*)malloc((size_t)(n_o > 0 ? n_o : 1) * sizeof(double));
    double* Ld = (double*)malloc((size_t)(n_l > 0 ? n_l : 1) * sizeof(double));
    if (!Od || !Ld) {
        free(Od);
        free(Ld);
        return ORACLE_BAD_ARG;
    }
    decode(O, Od, n_o);
    for (int64_t i = 0; i < n_l; ++i) Ld[i] = (double)lse[i];
    int rc = oracle_merge_f64(Od, Ld, B, H, cp, D, lse_layout, lse_mode, out, out_lse, out_abs, nthreads);
    free(Od);
    free(Ld);
    return rc;
}

int oracle_merge_bf16(const uint16_t* O, const float* lse, int64_t B, int64_t H, int64_t cp, int64_t D,
                      int lse_layout, int lse_mode, double* out, double* out_lse, double* out_abs,
                      int nthreads) {
    return merge_16bit(oracle_decode_bf16, O, lse, B, H, cp, D, lse_layout, lse_mode, out, out_lse, out_abs,
                       nthreads);
}

int oracle_merge_f16(const uint16_t* O, const float* lse, int64_t B, int64_t H, int64_t cp, int64_t D,
                     int lse_layout, int lse_mode, double* out, double* out_lse, double* out_abs,
                     int nthreads) {
    return merge_16bit(oracle_decode_f16, O, lse, B, H, cp, D, lse_layout, lse_mode, out, out_lse, out_abs,
                       nthreads);
}

/*
 * Softmax attention of one query row over KV rows [t0, t1): the definition,
 * in two passes (max, then exponentials).  q has dqk columns, each kv row has
 * kv_stride elements of which the first dqk are the key and the first dv the
 * value.  Writes o[dv] and returns the natural-log LSE (-inf for t0 == t1).
 */
typedef double (*decode16_fn)(uint16_t);

static decode16_fn decoder(int dtype) { return dtype == ORACLE_F16 ? oracle_f16_to_f64 : oracle_bf16_to_f64; }

static double attend_row(decode16_fn dec, const uint16_t* q, const uint16_t* kv, int64_t kv_stride, int64_t t0,
                         int64_t t1, int64_t dqk, int64_t dv, double scale, double* qd, double* o) {
    for (int64_t d = 0; d < dv; ++d) o[d] = 0.0;
    if (t1 <= t0) return -INFINITY;
    for (int64_t d = 0; d < dqk; ++d) qd[d] = dec(q[d]);

    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        const uint16_t* k = kv + t * kv_stride;
        double z = 0.0;
        for (int64_t d = 0; d < dqk; ++d) z += qd[d] * dec(k[d]);
        z *= scale;
        if (z > m) m = z;
    }
    double l = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        const uint16_t* k = kv + t * kv_stride;
        double z = 0.0;
        for (int64_t d = 0; d < dqk; ++d) z += qd[d] * dec(k[d]);
        z *= scale;
        double p = exp(z - m);
        l += p;
        for (int64_t d = 0; d < dv; ++d) o[d] += p * dec(k[d]);
    }
    for (int64_t d = 0; d < dv; ++d) o[d] /= l;
    return m + log(l);
}

/* Shard s of a T-token cache split into cp contiguous shards covers
 * [floor(s*T/cp), floor((s+1)*T/cp)). */
static void shard_bounds(int64_t T, int64_t cp, int64_t s, int64_t* t0, int64_t* t1) {
    *t0 = (s * T) / cp;
    *t1 = ((s + 1) * T) / cp;
}

/*
 * Per-shard decode partials for the query rows listed in `rows` (each row is
 * b*hq + h; NULL means all B*hq rows in order).
 *   q        [B, hq, dqk] contiguous 16-bit bits (dtype ORACLE_BF16 or ORACLE_F16)
 *   kv       [T, dqk] contiguous 16-bit bits of the same type (value = first dv columns)
 *   o_part   [n_rows, cp, dv]
 *   lse_part [n_rows, cp]     base-e, or times log2 e for base 2
 */
int oracle_attention_partials(const uint16_t* q, const uint16_t* kv, int64_t B, int64_t hq, int64_t T,
                              int64_t dqk, int64_t dv, int64_t cp, double scale, int lse_mode, int dtype,
                              const int64_t* rows, int64_t n_rows, double* o_part, double* lse_part,
                              int nthreads) {
    if (B < 0 || hq <= 0 || T < 0 || dqk <= 0 || dv <= 0 || dv > dqk || cp <= 0) return ORACLE_BAD_ARG;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F16) return ORACLE_BAD_ARG;
    const decode16_fn dec = decoder(dtype);
    if (lse_mode != ORACLE_BASE_E && lse_mode != ORACLE_BASE_2) return ORACLE_BAD_ARG;
    if (!rows) n_rows = B * hq;
    set_threads(nthreads);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t r = rows ? rows[i] : i;
        double* qd = (double*)malloc((size_t)dqk * sizeof(double));
        for (int64_t s = 0; s < cp; ++s) {
            int64_t t0, t1;
            shard_bounds(T, cp, s, &t0, &t1);
            double lse =
                attend_row(dec, q + r * dqk, kv, dqk, t0, t1, dqk, dv, scale, qd, o_part + (i * cp + s) * dv);
            if (lse_mode == ORACLE_BASE_2) lse *= M_LOG2E;
            lse_part[i * cp + s] = lse;
        }
        free(qd);
    }
    return ORACLE_OK;
}

/*
 * Softmax attention of one query row over the cache rows t0, t0 + step, ...
 * (n rows): the definition, as attend_row but over a strided token set.
 */
static double attend_rows_strided(decode16_fn dec, const uint16_t* q, const uint16_t* kv, int64_t kv_stride,
                                  int64_t t0, int64_t step, int64_t n, int64_t dqk, int64_t dv, double scale,
                                  double* qd, double* o) {
    for (int64_t d = 0; d < dv; ++d) o[d] = 0.0;
    if (n <= 0) return -INFINITY;
    for (int64_t d = 0; d < dqk; ++d) qd[d] = dec(q[d]);
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t* k = kv + (t0 + i * step) * kv_stride;
        double z = 0.0;
        for (int64_t d = 0; d < dqk; ++d) z += qd[d] * dec(k[d]);
        z *= scale;
        if (z > m) m = z;
    }
    double l = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t* k = kv + (t0 + i * step) * kv_stride;
        double z = 0.0;
        for (int64_t d = 0; d < dqk; ++d) z += qd[d] * dec(k[d]);
        z *= scale;
        double p = exp(z - m);
        l += p;
        for (int64_t d = 0; d < dv; ++d) o[d] += p * dec(k[d]);
    }
    for (int64_t d = 0; d < dv; ++d) o[d] /= l;
    return m + log(l);
}

/*
 * Per-shard partials with one cache per query token.
 *   q         [B, hq, dqk] contiguous 16-bit bits
 *   kv        token b's cache row t at kv + (b*kv_sb + t)*dqk (kv_sb in rows;
 *             0 lets every token share one cache), 16-bit bits
 *   seq_lens  [B]: token b attends over its rows t < seq_lens[b]
 *   interleaved  0: shard s owns [floor(s L/cp), floor((s+1) L/cp));
 *                1: shard s owns the rows t < L with t mod cp == s
 *   o_part [n_rows, cp, dv], lse_part [n_rows, cp] as oracle_attention_partials.
 */
int oracle_attention_partials_varlen(const uint16_t* q, const uint16_t* kv, int64_t B, int64_t hq, int64_t kv_sb,
                                     const int32_t* seq_lens, int interleaved, int64_t dqk, int64_t dv, int64_t cp,
                                     double scale, int lse_mode, int dtype, const int64_t* rows, int64_t n_rows,
                                     double* o_part, double* lse_part, int nthreads) {
    if (B < 0 || hq <= 0 || kv_sb < 0 || dqk <= 0 || dv <= 0 || dv > dqk || cp <= 0) return ORACLE_BAD_ARG;
    if (lse_mode != ORACLE_BASE_E && lse_mode != ORACLE_BASE_2) return ORACLE_BAD_ARG;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F16) return ORACLE_BAD_ARG;
    for (int64_t b = 0; b < B; ++b)
        if (seq_lens[b] < 0) return ORACLE_BAD_ARG;
    const decode16_fn dec = decoder(dtype);
    if (!rows) n_rows = B * hq;
    set_threads(nthreads);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t r = rows ? rows[i] : i;
        const int64_t b = r / hq;
        const int64_t L = seq_lens[b];
        const uint16_t* cache = kv + b * kv_sb * dqk;
        double* qd = (double*)malloc((size_t)dqk * sizeof(double));
        for (int64_t s = 0; s < cp; ++s) {
            int64_t t0, step, n;
            if (interleaved) {
                t0 = s;
                step = cp;
                n = L > s ? (L - s + cp - 1) / cp : 0;
            } else {
                int64_t t1;
                shard_bounds(L, cp, s, &t0, &t1);
                step = 1;
                n = t1 - t0;
            }
            double lse = attend_rows_strided(dec, q + r * dqk, cache, dqk, t0, step, n, dqk, dv, scale, qd,
                                             o_part + (i * cp + s) * dv);
            if (lse_mode == ORACLE_BASE_2) lse *= M_LOG2E;
            lse_part[i * cp + s] = lse;
        }
        free(qd);
    }
    return ORACLE_OK;
}

/* Full (unsharded) decode attention over all T rows: the brute-force answer
 * the merged partials must reproduce.  o [n_rows, dv], lse [n_rows]. */
int oracle_attention_full(const uint16_t* q, const uint16_t* kv, int64_t B, int64_t hq, int64_t T, int64_t dqk,
                          int64_t dv, double scale, int lse_mode, int dtype, const int64_t* rows, int64_t n_rows,
                          double* o, double* lse, int nthreads) {
    if (B < 0 || hq <= 0 || T < 0 || dqk <= 0 || dv <= 0 || dv > dqk) return ORACLE_BAD_ARG;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F16) return ORACLE_BAD_ARG;
    const decode16_fn dec = decoder(dtype);
    if (lse_mode != ORACLE_BASE_E && lse_mode != ORACLE_BASE_2) return ORACLE_BAD_ARG;
    if (!rows) n_rows = B * hq;
    set_threads(nthreads);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t r = rows ? rows[i] : i;
        double* qd = (double*)malloc((size_t)dqk * sizeof(double));
        double l = attend_row(dec, q + r * dqk, kv, dqk, 0, T, dqk, dv, scale, qd, o + i * dv);
        if (lse_mode == ORACLE_BASE_2) l *= M_LOG2E;
        lse[i] = l;
        free(qd);
    }
    return ORACLE_OK;
}
