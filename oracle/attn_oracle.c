/*
 * Oracle for exact scaled-dot-product attention, fp64, CPU only.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may build, load or call this file. The product path (the
 * HIP library) never touches it, and this file shares no code, header, table
 * or constant with that library.
 *
 * What it computes is the plain definition of softmax attention, one query
 * row at a time, with the whole row of scores held in memory:
 *   - "Standard attention" as the cookbook notebook's SDPA reference layer
 *     computes it (hassan11196 llm-systems-cookbook, "FlashAttention-2 in an
 *     attention layer": shape algebra section and the SDPAAttention layer),
 *     the result FlashAttention-2 reaches exactly ("no algorithmic change --
 *     same math", infra.bea.ai FlashAttention V2 guide, introduction).
 *   - The score of key j for query i is scale * (q_i . k_j), the scale applied
 *     after the dot product and before masking (cookbook Triton kernel body).
 *   - Causal masking keeps key j for query i iff j <= i (cookbook Triton kernel,
 *     the offs_m >= cur_n mask; queries and keys have the same length).
 *   - Softmax is the two-pass form: m = max_j s_j, e_j = exp(s_j - m),
 *     l = sum_j e_j; o_i = (sum_j e_j v_j) / l.
 *   - lse_i = m + log(l), natural log (the per-row logsumexp that the
 *     FlashAttention-2 epilogue writes, jared-hpc Lecture 6 reading task;
 *     m and l are the running max and sum of the online softmax in the
 *     infra.bea.ai guide, "Optimization 2: Delay Rescaling").
 *
 * Inputs are the exact fp64 values the GPU receives (fp16/bf16 widened by the
 * caller). Every sum runs in a fixed order with one fp64 accumulator; the
 * file is compiled without -ffast-math, so exp and log are libm's.
 *
 * Layout: q, k, v, o are contiguous (B, H, S, D) row-major: element
 * (b, h, s, d) sits at ((b*H + h)*S + s)*D + d. lse is contiguous (B, H, S).
 */
#include <math.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One output row: query row i of head (b, h). `scores` holds S doubles. */
static void oracle_one_row(const double *q, const double *k, const double *v,
                           long H, long S, long D, long b, long h, long i,
                           int causal, double scale, double *scores,
                           double *o_row, double *lse_out) {
    const long head = (b * H + h) * S * D;
    const double *qi = q + head + i * D;
    const long n_keys = causal ? i + 1 : S; /* keys j in [0, n_keys) */

    /* scores s_j = scale * (q_i . k_j) */
    for (long j = 0; j < n_keys; ++j) {
        const double *kj = k + head + j * D;
        double dot = 0.0;
        for (long d = 0; d < D; ++d) dot += qi[d] * kj[d];
        scores[j] = scale * dot;
    }

    /* pass 1: row max */
    double m = -INFINITY;
    for (long j = 0; j < n_keys; ++j)
        if (scores[j] > m) m = scores[j];

    /* pass 2: e_j = exp(s_j - m), l = sum e_j (e_j kept in `scores`) */
    double l = 0.0;
    for (long j = 0; j < n_keys; ++j) {
        scores[j] = exp(scores[j] - m);
        l += scores[j];
    }

    /* o_i = sum_j e_j v_j / l */
    for (long d = 0; d < D; ++d) o_row[d] = 0.0;
    for (long j = 0; j < n_keys; ++j) {
        const double *vj = v + head + j * D;
        const double e = scores[j];
        for (long d = 0; d < D; ++d) o_row[d] += e * vj[d];
    }
    for (long d = 0; d < D; ++d) o_row[d] /= l;

    *lse_out = m + log(l);
}

static int oracle_check_args(const void *q, const void *k, const void *v,
                             const void *o, const void *lse, long B, long H,
                             long S, long D) {
    if (!q || !k || !v || !o || !lse) return 1;
    if (B < 1 || H < 1 || S < 1 || D < 1) return 2;
    return 0;
}

/*
 * Full attention: o (B, H, S, D) and lse (B, H, S), fp64.
 * Returns 0 on success, 1 for a null pointer, 2 for a non-positive size,
 * 3 when the per-thread score buffer cannot be allocated.
 */
int oracle_attention_f64(const double *q, const double *k, const double *v,
                         double *o, double *lse, long B, long H, long S,
                         long D, int causal, double scale, int nthreads) {
    int err = oracle_check_args(q, k, v, o, lse, B, H, S, D);
    if (err) return err;
    const long n_rows = B * H * S;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)S);
        if (!scores) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
            for (long r = 0; r < n_rows; ++r) {
                const long i = r % S, bh = r / S;
                oracle_one_row(q, k, v, H, S, D, bh / H, bh % H, i, causal,
                               scale, scores, o + r * D, lse + r);
            }
            free(scores);
        }
    }
    return failed ? 3 : 0;
}

/*
 * Selected rows only: rows[t] is a flat row index (b*H + h)*S + i. Writes
 * o_rows (n_rows, D) and lse_rows (n_rows). Same return codes as above, plus
 * 4 when a row index is out of range.
 */
int oracle_attention_rows_f64(const double *q, const double *k,
                              const double *v, const long *rows, long n_rows,
                              double *o_rows, double *lse_rows, long B, long H,
                              long S, long D, int causal, double scale,
                              int nthreads) {
    int err = oracle_check_args(q, k, v, o_rows, lse_rows, B, H, S, D);
    if (err) return err;
    if (n_rows < 0 || (n_rows > 0 && !rows)) return 1;
    for (long t = 0; t < n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= B * H * S) return 4;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)S);
        if (!scores) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
            for (long t = 0; t < n_rows; ++t) {
                const long r = rows[t], i = r % S, bh = r / S;
                oracle_one_row(q, k, v, H, S, D, bh / H, bh % H, i, causal,
                               scale, scores, o_rows + t * D, lse_rows + t);
            }
            free(scores);
        }
    }
    return failed ? 3 : 0;
}

/*
 * Attention of Sq query rows against Sk key rows per head: the decoding
 * (KV-cache) form that the infra.bea.ai FlashAttention V2 guide lists as
 * served by a FlashDecoding variant ("When V2 Is Used vs Not" table).
 *
 * q and o are contiguous (B, H, Sq, D); k and v are contiguous (B, H, Sk, D);
 * lse is contiguous (B, H, Sq). The queries are the last Sq positions of a
 * sequence whose Sk keys are all present (the cache includes the new rows),
 * so query i sits at position Sk - Sq + i. Causal masking then keeps key j
 * for query i iff j <= i + (Sk - Sq): the same "key not after the query"
 * rule as the cookbook kernel's causal mask, with queries and keys counted
 * from the same sequence start. With Sq = Sk this is the square case above.
 * Scores, softmax and lse are as above.
 */
static void oracle_one_row_kv(const double *q, const double *k, const double *v,
                              long H, long Sq, long Sk, long D, long b, long h,
                              long i, int causal, double scale, double *scores,
                              double *o_row, double *lse_out) {
    const double *qi = q + ((b * H + h) * Sq + i) * D;
    const long kv_head = (b * H + h) * Sk * D;
    const long n_keys = causal ? i + (Sk - Sq) + 1 : Sk; /* keys j in [0, n_keys) */

    for (long j = 0; j < n_keys; ++j) {
        const double *kj = k + kv_head + j * D;
        double dot = 0.0;
        for (long d = 0; d < D; ++d) dot += qi[d] * kj[d];
        scores[j] = scale * dot;
    }
    double m = -INFINITY;
    for (long j = 0; j < n_keys; ++j)
        if (scores[j] > m) m = scores[j];
    double l = 0.0;
    for (long j = 0; j < n_keys; ++j) {
        scores[j] = exp(scores[j] - m);
        l += scores[j];
    }
    for (long d = 0; d < D; ++d) o_row[d] = 0.0;
    for (long j = 0; j < n_keys; ++j) {
        const double *vj = v + kv_head + j * D;
        const double e = scores[j];
        for (long d = 0; d < D; ++d) o_row[d] += e * vj[d];
    }
    for (long d = 0; d < D; ++d) o_row[d] /= l;
    *lse_out = m + log(l);
}

/*
 * Returns 0 on success, 1 for a null pointer, 2 for a non-positive size or
 * (causal) Sq > Sk, which would leave the first queries without any key,
 * 3 when a score buffer cannot be allocated.
 */
int oracle_attention_kv_f64(const double *q, const double *k, const double *v,
                            double *o, double *lse, long B, long H, long Sq,
                            long Sk, long D, int causal, double scale,
                            int nthreads) {
    if (!q || !k || !v || !o || !lse) return 1;
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1) return 2;
    if (causal && Sq > Sk) return 2;
    const long n_rows = B * H * Sq;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)Sk);
        if (!scores) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
            for (long r = 0; r < n_rows; ++r) {
                const long i = r % Sq, bh = r / Sq;
                oracle_one_row_kv(q, k, v, H, Sq, Sk, D, bh / H, bh % H, i, causal,
                                  scale, scores, o + r * D, lse + r);
            }
            free(scores);
        }
    }
    return failed ? 3 : 0;
}

/*
 * Tolerance of the FP8 attention path: a forward error bound, per output,
 * for attention computed with FP8 products and P rounded to e4m3, next to
 * the exact result on the same (dequantized) inputs. This is not part of
 * the definition of attention; it is the arithmetic's worst case, which the
 * tests hold the FP8 path to element by element.
 *
 * The FP8 path (infra.bea.ai FlashAttention V2 guide, "FlashAttention-3
 * and Beyond", the FP8 direction) computes, with t_j = log2(e) s_j the
 * base-2 logits of one query row:
 *   - s~_j from a product whose sum is off by at most
 *     eps_sum * |scale| * A_j, A_j = sum_d |q_d k_jd| (the matrix-core
 *     instruction's measured bound, the fp32 rounding of c and of the FMA
 *     with the reference max folded in as 2^-21 (|t_j| + |t_max|));
 *   - P8_j = e4m3(2^(t~_j - m + p_exp)) for a reference max m of at most
 *     max_j t~_j, so every P8_j is Z w_j (1 + gamma_j) + sigma_j with
 *     Z = 2^p_exp sum_k 2^(t_k - m) >= 2^(p_exp - Delta_max) / w_max,
 *     |gamma_j| <= g_j = 2^Delta_j (1 + 2^-20)(1 + 2^-4) - 1 (e4m3 keeps
 *     3 mantissa bits: half an ulp is 2^-4 of the value; 2^-20 covers exp2)
 *     and |sigma_j| <= 2^-10 (half the spacing of e4m3's subnormals);
 *   - O = (sum P8_j v_j + E_pv) / (sum P8_j + E_l), both sums from FP8
 *     products, |E_pv| <= eps_sum sum P8_j |v_jd|, |E_l| <= eps_sum sum P8_j,
 *     fp32 accumulation across key tiles (at most n steps of 2^-24), then
 *     rounded once to the output type (half an ulp: u_out of the value);
 *   - lse = ln2 (m + log2 l - p_exp), l the fp32 sum of the unrounded P.
 * Since sum_j w_j (v_jd - O_d) = 0, the numerator's error against O_d L is
 * sum_j (P8_j - Z w_j)(v_jd - O_d), which gives, in units of Z,
 *   |dO_d| <= [sum_j w_j g_j |v_jd - O_d| + zeta 2^-10 sum_j |v_jd - O_d|
 *              + eps_sum (sum_j (w_j (1 + g_j) + zeta 2^-10) |v_jd|
 *                         + |O_d| L_max) + 2n 2^-24 L_max max|v|]
 *             / (L_min - eps_sum L_max)
 * with zeta = w_max 2^(Delta_max - p_exp) >= 1 / Z,
 * L_max = sum_j w_j (1 + g_j) + n zeta 2^-10, L_min = sum_j w_j (1 - g_j)
 * - n zeta 2^-10; then bound_o = that + u_out (|O_d| + that). And
 *   |dlse| <= ln(sum_j w_j 2^Delta_j (1 + 2^-22)) + (2n + 4) 2^-24
 *             + 2^-21 (|lse| + p_exp + 1).
 * Delta_j = log2(e) (eps_sum |scale| A_j) + 2^-21 (|t_j| + |t_max|).
 *
 * Writes o and lse (the plain definition, as oracle_attention_f64 computes
 * them) and bound_o (B, H, S, D), bound_lse (B, H, S). Returns the codes of
 * oracle_attention_f64, plus 5 when L_min - eps_sum L_max is not positive
 * for some row (no bound).
 */
static int oracle_fp8_bound_row(const double *q, const double *k, const double *v,
                                long H, long S, long D, long b, long h, long row,
                                int causal, double scale, double eps_sum,
                                double p_exp, double u_out, double *s,
                                double *a, double *o_row, double *lse_out,
                                double *bo_row, double *bl_out) {
    const long hoff = ((b * H + h) * S) * D;
    const double *qrow = q + hoff + row * D;
    const long nk = causal ? (row + 1) : S;
    const double log2e = 1.4426950408889634074;
    double m = -INFINITY;
    for (long j = 0; j < nk; ++j) {
        const double *krow = k + hoff + j * D;
        double dot = 0.0, absdot = 0.0;
        for (long d = 0; d < D; ++d) {
            dot += qrow[d] * krow[d];
            absdot += fabs(qrow[d] * krow[d]);
        }
        s[j] = scale * dot;
        a[j] = fabs(scale) * absdot;
        if (s[j] > m) m = s[j];
    }
    const double t_max = m * log2e;
    /* weights w_j = e_j / ell, O, lse; then Delta_j and g_j (kept in a[]) */
    double ell = 0.0;
    for (long j = 0; j < nk; ++j) {
        s[j] = exp(s[j] - m);
        ell += s[j];
    }
    for (long d = 0; d < D; ++d) o_row[d] = 0.0;
    for (long j = 0; j < nk; ++j) {
        const double *vrow = v + hoff + j * D;
        for (long d = 0; d < D; ++d) o_row[d] += s[j] * vrow[d];
    }
    for (long d = 0; d < D; ++d) o_row[d] /= ell;
    *lse_out = m + log(ell);
    double w_max = 0.0, delta_max = 0.0, lse_sum = 0.0, lmin = 0.0, lmax = 0.0;
    for (long j = 0; j < nk; ++j) {
        const double w = s[j] / ell;
        /* t_j from w: t_j = t_max + log2(e_j) */
        const double t_j = t_max + log2(s[j] > 0.0 ? s[j] : 1e-300);
        const double delta = log2e * eps_sum * a[j] + ldexp(fabs(t_j) + fabs(t_max), -21);
        const double g = exp2(delta) * (1.0 + ldexp(1.0, -20)) * (1.0 + ldexp(1.0, -4)) - 1.0;
        if (w > w_max) w_max = w;
        if (delta > delta_max) delta_max = delta;
        lse_sum += w * exp2(delta) * (1.0 + ldexp(1.0, -22));
        lmin += w * (1.0 - g);
        lmax += w * (1.0 + g);
        s[j] = w;
        a[j] = g;
    }
    const double zeta = w_max * exp2(delta_max - p_exp);
    const double sub = ldexp(1.0, -10);
    lmin -= (double)nk * zeta * sub;
    lmax += (double)nk * zeta * sub;
    const double den = lmin - eps_sum * lmax;
    double vmax = 0.0;
    for (long j = 0; j < nk; ++j) {
        const double *vrow = v + hoff + j * D;
        for (long d = 0; d < D; ++d)
            if (fabs(vrow[d]) > vmax) vmax = fabs(vrow[d]);
    }
    for (long d = 0; d < D; ++d) {
        double dev_w = 0.0, dev = 0.0, mag = 0.0;
        for (long j = 0; j < nk; ++j) {
            const double vjd = v[hoff + j * D + d];
            const double e = fabs(vjd - o_row[d]);
            dev_w += s[j] * a[j] * e;
            dev += e;
            mag += (s[j] * (1.0 + a[j]) + zeta * sub) * fabs(vjd);
        }
        const double num = dev_w + zeta * sub * dev + eps_sum * (mag + fabs(o_row[d]) * lmax) +
                           2.0 * (double)nk * ldexp(1.0, -24) * lmax * vmax;
        const double pre = num / den;
        bo_row[d] = pre + u_out * (fabs(o_row[d]) + pre);
    }
    *bl_out = log(lse_sum) + (2.0 * (double)nk + 4.0) * ldexp(1.0, -24) +
              ldexp(fabs(*lse_out) + p_exp + 1.0, -21);
    return den > 0.0 ? 0 : 5;
}

int oracle_attention_fp8_bound_f64(const double *q, const double *k, const double *v,
                                   double *o, double *lse, double *bound_o,
                                   double *bound_lse, long B, long H, long S, long D,
                                   int causal, double scale, double eps_sum,
                                   double p_exp, double u_out, int nthreads) {
    int err = oracle_check_args(q, k, v, o, lse, B, H, S, D);
    if (err) return err;
    if (!bound_o || !bound_lse) return 1;
    const long n_rows = B * H * S;
    int failed = 0, nobound = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed, nobound)
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)S);
        double *a = (double *)malloc(sizeof(double) * (size_t)S);
        if (!s || !a) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
            for (long r = 0; r < n_rows; ++r) {
                const long i = r % S, bh = r / S;
                nobound |= oracle_fp8_bound_row(q, k, v, H, S, D, bh / H, bh % H, i, causal,
                                                scale, eps_sum, p_exp, u_out, s, a, o + r * D,
                                                lse + r, bound_o + r * D, bound_lse + r) != 0;
            }
        }
        free(s);
        free(a);
    }
    return failed ? 3 : nobound ? 5 : 0;
}

/* Number of threads an OpenMP region would use by default (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
