/*
 * dsv4_oracle.c -- plain, slow CPU oracle for the CSA/HCA compressed-attention
 * hot path.  TEST INFRASTRUCTURE ONLY: nothing in the product library links,
 * includes or calls this file; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no code, header, table or
 * constant with the HIP path.
 *
 * Every floating-point result is accumulated in fp64.  The only places where
 * fp32 appears are the storage-quantisation decisions (scale and scaled value
 * before rounding to a code), which are taken in the same fp32 precision the
 * kernels use, so that a stored code is a function of the stored inputs and
 * not of the arithmetic that decides it.
 *
 * Sources (pages as published; sections named, statements paraphrased):
 *  [V]  vastsailsolution.com article on the DeepSeek-V4 report, sections
 *       "CSA -- compressed sparse attention", "HCA -- heavily compressed
 *       attention" and the paragraphs after them on the sliding window, the
 *       attention sink, partial RoPE, mixed-precision KV and the two caches.
 *  [R]  rqlyzj.com "three paradigm innovations" article, section 01 (the
 *       folded million-token context: thinner vs shorter KV, overlap, indexer).
 *  [X]  xiaoyuzhoufm.com podcast summary, section 1.1 (hybrid attention; CSA
 *       applies DSA over the compressed entries; both have an SWA branch).
 *  [H]  hwcomputing.csdn.net "DeepSeek V4 底层逻辑全解析", section 二
 *       (CSA three steps with overlap and Top-512/1024; HCA m'=128 dense).
 *
 * Parity status: every function below is pinned by a CPU test (closed forms,
 * library routines on special cases, brute force on tiny inputs) except the
 * composition at full production shapes, which is "parity unpinned" beyond
 * those pins.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* Threads the parallel loops use (for reporting the CPU baseline). */
ORC_API int orc_num_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* Storage number formats.                                                   */
/* [V] (partial RoPE + mixed precision paragraph): the RoPE dimensions of a  */
/* KV entry are kept in BF16 and all other dimensions in FP8.  FP8 is read   */
/* as OCP E4M3 (4 exponent bits, bias 7, 3 mantissa bits, no infinities,     */
/* largest finite value 448).                                                */
/* ------------------------------------------------------------------------ */

/* Value of an E4M3 code, straight from the format definition. */
ORC_API double orc_e4m3_decode(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);          /* subnormal: m/8 * 2^-6 */
    else v = ldexp((double)(8 + m), e - 10);       /* (1 + m/8) * 2^(e-7)   */
    return sign ? -v : v;
}

/* Round an fp32 value to the nearest E4M3 code (ties to even mantissa),
 * saturating to +-448.  Codes are monotone in magnitude, so the code is the
 * number of representable steps of size ulp(a) below a, offset by the binade.
 */
ORC_API uint8_t orc_e4m3_encode(float y) {
    if (isnan(y)) return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    if (a >= 448.0) return sign | 0x7E;
    int e;                              /* a = f * 2^e with f in [0.5, 1) */
    frexp(a, &e);
    int unb = e - 1;                    /* unbiased exponent of a         */
    if (a == 0.0 || unb < -6) unb = -6; /* subnormal range shares ulp 2^-9 */
    double q = rint(ldexp(a, 3 - unb)); /* a / ulp, ulp = 2^(unb-3)       */
    /* normal binade unb: code = (unb+7)<<3 | (q-8) = 8*(unb+6) + q; q == 16
     * lands on the first code of the next binade, q <= 8 in the subnormal
     * range is the code itself. */
    int code = 8 * (unb + 6) + (int)q;
    if (code > 0x7E) code = 0x7E;
    return sign | (uint8_t)code;
}

/* Round an fp32 value to bfloat16 (nearest, ties to even) and return it. */
ORC_API float orc_bf16_round(float x) {
    if (isnan(x)) return x;
    uint32_t u;
    memcpy(&u, &x, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;
    float r;
    memcpy(&r, &u, 4);
    return r;
}

/* ------------------------------------------------------------------------ */
/* FP4 of the indexer's query and key activations.  [R] section on FP4 QAT:  */
/* the lightning indexer's QK activations are cached, loaded and multiplied  */
/* in FP4; [X] 2.1: FP4 on the CSA indexer path; [H] 二, CSA step 2: the      */
/* indexer scores in low precision (FP4).  The pages name no FP4 layout.     */
/* Reading: OCP Microscaling MXFP4 -- blocks of 32 consecutive values share  */
/* one power-of-two scale 2^x (an E8M0 byte, x in [-127, 127]) and each      */
/* value is an E2M1 code: sign, 2 exponent bits (bias 1), 1 mantissa bit,    */
/* magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (no infinities, no NaN).            */
/* ------------------------------------------------------------------------ */

/* Value of an E2M1 code (low 4 bits), straight from the format definition. */
ORC_API double orc_e2m1_decode(uint8_t c) {
    int sign = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

/* Nearest E2M1 code of y, ties to even mantissa, saturating to +-6 (the
 * microscaling conversion rule for values past the largest magnitude).  As
 * for E4M3: inside binade [2^u, 2^(u+1)) the step is 2^(u-1); below 1 the
 * subnormal step 0.5 continues the first binade's. */
ORC_API uint8_t orc_e2m1_encode(float y) {
    uint8_t sign = signbit(y) ? 8 : 0;
    double a = fabs((double)y);
    if (!(a < 6.0)) return sign | 7;
    int e;                              /* a = f * 2^e with f in [0.5, 1) */
    frexp(a, &e);
    int unb = e - 1;                    /* floor(log2 a)                  */
    if (a == 0.0 || unb < 0) unb = 0;
    double q = rint(ldexp(a, 1 - unb)); /* a / step, step = 2^(unb-1)     */
    return sign | (uint8_t)(2 * unb + (int)q);
}

/* Shared exponent x of a block with largest magnitude amax: the microscaling
 * rule x = floor(log2 amax) - 2 (2 = exponent of E2M1's largest magnitude),
 * clamped to the E8M0 range; an all-zero block takes the smallest scale. */
ORC_API int orc_mx_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    int e;
    frexp((double)amax, &e);
    int x = (e - 1) - 2;
    return x < -127 ? -127 : (x > 127 ? 127 : x);
}

/* MXFP8 (OCP microscaling, E4M3 elements) of the indexer path's activations
 * [X 2.1, R FP4 QAT section: the indexer path runs in low precision; the
 * activations of its projections are read as FP8 with the same block-scale
 * scheme as the FP4 rows]: blocks of 32 consecutive values share 2^x with
 * x = floor(log2 amax) - 8 (8 = the exponent of E4M3's largest value 448),
 * clamped to [-127, 127]; each value is RNE(v / 2^x) in E4M3, saturating to
 * +-448.  Returns the represented values. */
ORC_API void orc_mxfp8_rows(const double *x, long rows, int n, double *out) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r)
        for (int b0 = 0; b0 < n; b0 += 32) {
            const int nb = n - b0 < 32 ? n - b0 : 32;
            float amax = 0.0f;
            for (int i = 0; i < nb; ++i) amax = fmaxf(amax, fabsf((float)x[r * n + b0 + i]));
            int e = -127;
            if (amax > 0.0f) {
                int ex;
                frexp((double)amax, &ex);
                e = (ex - 1) - 8;
                e = e < -127 ? -127 : (e > 127 ? 127 : e);
            }
            for (int i = 0; i < nb; ++i) {
                const float y = ldexpf((float)x[r * n + b0 + i], -e);
                out[r * n + b0 + i] = ldexp(orc_e4m3_decode(orc_e4m3_encode(y)), e);
            }
        }
}

/* Store one vector of n values the way the cache holds it and return the
 * value the cache then represents (fp64, exact).
 *   mode 0 : fp32 storage (each value rounded to fp32).
 *   mode 1 : the first n_fp8 values as E4M3 codes sharing one fp32 scale,
 *            the remaining n - n_fp8 values as bf16.
 *   mode 2 : (indexer rows) MXFP4, blocks of 32 consecutive values, each
 *            with its shared exponent from its own largest magnitude.
 * Scale rule (one reading of "FP8" in [V]): scale = amax / 448 with
 * code = E4M3(x * (448 / amax)); both quotients and the product are fp32
 * operations, the precision in which the kernels take the same decision.
 * A block whose amax is zero (or below 1e-30) uses scale 1.
 */
ORC_API void orc_store_vec(const double *x, int n, int n_fp8, int mode, double *out) {
    if (mode == 0) {
        for (int i = 0; i < n; ++i) out[i] = (double)(float)x[i];
        return;
    }
    if (mode == 2) {                    /* MXFP4: all n values, blocks of 32 */
        for (int b0 = 0; b0 < n; b0 += 32) {
            const int nb = n - b0 < 32 ? n - b0 : 32;
            float amax = 0.0f;
            for (int i = 0; i < nb; ++i) amax = fmaxf(amax, fabsf((float)x[b0 + i]));
            const int e = orc_mx_exponent(amax);
            for (int i = 0; i < nb; ++i) {
                const float y = ldexpf((float)x[b0 + i], -e);   /* exact: a power of two */
                out[b0 + i] = ldexp(orc_e2m1_decode(orc_e2m1_encode(y)), e);
            }
        }
        return;
    }
    float amax = 0.0f;
    for (int i = 0; i < n_fp8; ++i) {
        float a = fabsf((float)x[i]);
        if (a > amax || isnan(a)) amax = a;
    }
    float scale = 1.0f, inv = 1.0f;
    if (amax >= 1e-30f) {
        scale = amax / 448.0f;
        inv = 448.0f / amax;
    }
    for (int i = 0; i < n_fp8; ++i) {
        float y = (float)x[i] * inv;
        out[i] = orc_e4m3_decode(orc_e4m3_encode(y)) * (double)scale;
    }
    for (int i = n_fp8; i < n; ++i) out[i] = (double)orc_bf16_round((float)x[i]);
}

ORC_API void orc_store_rows(const double *x, long rows, int n, int n_fp8, int mode, double *out) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) orc_store_vec(x + r * n, n, n_fp8, mode, out + r * n);
}

/* ------------------------------------------------------------------------ */
/* RoPE on a slice of d_r values (the last d_r dims of a head vector).       */
/* [V]: RoPE is applied only to the last 64 dimensions of queries and KV.    */
/* Reading: pairs (2i, 2i+1) rotated by angle pos * base^(-2i/d_r).          */
/* ------------------------------------------------------------------------ */
ORC_API void orc_rope(double *x, int d_r, double pos, double base) {
    for (int i = 0; i < d_r / 2; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)d_r);
        double ang = pos * theta;
        double c = cos(ang), s = sin(ang);
        double a = x[2 * i], b = x[2 * i + 1];
        x[2 * i] = a * c - b * s;
        x[2 * i + 1] = a * s + b * c;
    }
}

/* Rotate the last d_r dims of each row r of x (rows x d) by position pos[r]. */
ORC_API void orc_rope_rows(double *x, long rows, int d, int d_r, const double *pos, double base) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) orc_rope(x + r * d + (d - d_r), d_r, pos[r], base);
}

/* ------------------------------------------------------------------------ */
/* Block compressor.  [R] section 01 and [V] CSA: the tokens of a block are  */
/* mixed by learned importance weights into one entry (no decompression).   */
/* Reading: per channel c, the weights are a softmax over the block's tokens */
/* of the gate logits gate[s][c]; the entry is the weighted sum of kv[s][c]. */
/* ------------------------------------------------------------------------ */
ORC_API void orc_gated_pool(const double *kv, const double *gate, int ntok, int dim, double *out) {
    for (int c = 0; c < dim; ++c) {
        double m = -INFINITY;
        for (int s = 0; s < ntok; ++s) if (gate[s * dim + c] > m) m = gate[s * dim + c];
        double den = 0.0, num = 0.0;
        for (int s = 0; s < ntok; ++s) {
            double a = exp(gate[s * dim + c] - m);
            den += a;
            num += a * kv[s * dim + c];
        }
        out[c] = num / den;
    }
}

/* Pool many entries at once.  Entry e pools tokens first[e] .. first[e]+cnt[e]-1
 * of the token arrays (kv, gate: ntok_total x dim). */
ORC_API void orc_pool_entries(const double *kv, const double *gate, int dim,
                              const long *first, const int *cnt, long n_entries, double *out) {
#pragma omp parallel for schedule(static)
    for (long e = 0; e < n_entries; ++e)
        orc_gated_pool(kv + first[e] * dim, gate + first[e] * dim, cnt[e], dim, out + e * dim);
}

/* ------------------------------------------------------------------------ */
/* Lightning-indexer score.  [V] CSA + [X] 1.1: the query is projected into  */
/* several index heads, passed through ReLU against the compressed index     */
/* keys; CSA applies DSA over the entries.  Reading (DSA form):              */
/*   I[j] = sum_h w[h] * max(0, q[h] . k[j]).                                */
/* ------------------------------------------------------------------------ */
ORC_API void orc_index_scores(const double *q, const double *w, int H, int D,
                              const double *keys, long N, double *scores) {
#pragma omp parallel for schedule(static)
    for (long j = 0; j < N; ++j) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h) {
            double dot = 0.0;
            for (int t = 0; t < D; ++t) dot += q[h * D + t] * keys[j * D + t];
            acc += w[h] * (dot > 0.0 ? dot : 0.0);
        }
        scores[j] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Top-k selector.  [V] CSA / [H] step 2: keep the k best-scoring entries.   */
/* Reading: order by (score descending, index ascending), NaN below every    */
/* number; keep the first min(k, N); emit them in ascending index order and  */
/* pad with -1.                                                              */
/* ------------------------------------------------------------------------ */
typedef struct { double s; long j; } orc_pair;

static int orc_pair_cmp(const void *pa, const void *pb) {
    const orc_pair *a = (const orc_pair *)pa, *b = (const orc_pair *)pb;
    int an = isnan(a->s), bn = isnan(b->s);
    if (an != bn) return an ? 1 : -1;
    if (!an && a->s != b->s) return a->s > b->s ? -1 : 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int orc_long_cmp(const void *pa, const void *pb) {
    long a = *(const long *)pa, b = *(const long *)pb;
    return (a > b) - (a < b);
}

ORC_API void orc_topk(const double *scores, long N, int k, int32_t *out) {
    long take = N < k ? N : k;
    orc_pair *p = (orc_pair *)malloc(sizeof(orc_pair) * (N > 0 ? N : 1));
    long *sel = (long *)malloc(sizeof(long) * (take > 0 ? take : 1));
    for (long j = 0; j < N; ++j) { p[j].s = scores[j]; p[j].j = j; }
    qsort(p, N, sizeof(orc_pair), orc_pair_cmp);
    for (long i = 0; i < take; ++i) sel[i] = p[i].j;
    qsort(sel, take, sizeof(long), orc_long_cmp);
    for (long i = 0; i < k; ++i) out[i] = i < take ? (int32_t)sel[i] : -1;
    free(p);
    free(sel);
}

/* ------------------------------------------------------------------------ */
/* Single-KV-head attention with a per-head sink.                            */
/* [V] CSA/HCA: MQA over the selected (or all) entries plus the window; the  */
/* sink paragraph: each head has a learnable sink logit added only to the    */
/* softmax denominator, so a head may attend to nothing.  One record serves  */
/* as both key and value.                                                    */
/*   l_i = tau * q_h . v_i ;  M = max(z_h, max_i l_i)                        */
/*   o_h = sum_i e^(l_i - M) v_i / (e^(z_h - M) + sum_i e^(l_i - M))         */
/* sink_mass (optional) receives e^(z_h - M) / denominator per head.         */
/* ------------------------------------------------------------------------ */
ORC_API void orc_attend(const double *q, const double *sinks, int H, int d, double tau,
                        const double *recs, long n, double *out, double *sink_mass) {
#pragma omp parallel for schedule(static)
    for (int h = 0; h < H; ++h) {
        double *lg = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
        double M = sinks[h];
        for (long i = 0; i < n; ++i) {
            double dot = 0.0;
            for (int t = 0; t < d; ++t) dot += q[(long)h * d + t] * recs[i * d + t];
            lg[i] = tau * dot;
            if (lg[i] > M) M = lg[i];
        }
        double *o = out + (long)h * d;
        for (int t = 0; t < d; ++t) o[t] = 0.0;
        if (M == -INFINITY) {           /* nothing to attend and an empty sink */
            if (sink_mass) sink_mass[h] = 0.0;
            free(lg);
            continue;
        }
        double den = exp(sinks[h] - M);
        for (long i = 0; i < n; ++i) {
            double p = exp(lg[i] - M);
            den += p;
            for (int t = 0; t < d; ++t) o[t] += p * recs[i * d + t];
        }
        for (int t = 0; t < d; ++t) o[t] /= den;
        if (sink_mass) sink_mass[h] = exp(sinks[h] - M) / den;
        free(lg);
    }
}

/* ------------------------------------------------------------------------ */
/* Grouped output projection.  [R] section on depth compensation: the 128   */
/* heads' outputs (128 x 512 = 65536 dims) are not projected to the model   */
/* width in one matrix; the heads are split into 16 groups, each group's    */
/* output is first condensed into a short group summary, and the 16         */
/* summaries are projected to the model width.  Reading: two linear maps,   */
/*   y[g] = W1[g] . o[g]   (o[g]: the group's heads concatenated, gd dims;  */
/*                          y[g]: r dims), stored as bf16 (the operand of   */
/*                          the second product),                           */
/*   out  = W2 . concat_g y[g]   (hidden dims).                             */
/* Sums in fp64; y rounded to bf16 through fp32, the precision in which the  */
/* kernels take the same rounding decision.                                  */
/* ------------------------------------------------------------------------ */
ORC_API void orc_out_proj(const double *o, long T, int G, int gd, int r, const double *w1,
                          const double *w2, int hidden, double *y_out, double *out) {
#pragma omp parallel for schedule(dynamic)
    for (long t = 0; t < T; ++t) {
        double *y = y_out + t * (long)G * r;
        for (int g = 0; g < G; ++g)
            for (int j = 0; j < r; ++j) {
                const double *w = w1 + ((long)g * r + j) * gd;
                const double *x = o + t * (long)G * gd + (long)g * gd;
                double acc = 0.0;
                for (int i = 0; i < gd; ++i) acc += w[i] * x[i];
                y[(long)g * r + j] = (double)orc_bf16_round((float)acc);
            }
        for (int n = 0; n < hidden; ++n) {
            const double *w = w2 + (long)n * G * r;
            double acc = 0.0;
            for (int k = 0; k < G * r; ++k) acc += w[k] * y[k];
            out[t * (long)hidden + n] = acc;
        }
    }
}
