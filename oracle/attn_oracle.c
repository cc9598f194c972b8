/*
 * attn_oracle.c -- the CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference that the HIP kernels are checked against.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the GPU library, and the
 * GPU library never calls it.
 *
 * Everything is computed in IEEE double precision from the exact input
 * values (bf16 and fp32 inputs arrive widened to float, which is exact).
 * No blocking, tiling, online rescaling or reordering beyond the plain
 * definition: each score row is materialised in full, masked, soft-maxed
 * and used to mix the values.  Built without -ffast-math.
 *
 * Sources (the pages the method is taken from):
 *  - "Attention Engineering: From MHA to GQA, MLA & FlashAttention",
 *    section 2, equation "Grouped-Query Attention Formulation":
 *    O = softmax(Q K^T / sqrt(d_h) + M) V per query head, with the query
 *    heads of group g sharing K_g and V_g.
 *  - "2.4 Multi-Head Attention, MQA, GQA & MLA", section "Implementing the
 *    MHA -> GQA conversion": query head j reads KV group floor(j / n_rep).
 *  - "Attention deep dive (MHA -> MQA -> GQA -> FlashAttention)", section 6
 *    "Sliding-window attention": key j is visible to query i iff
 *    (j <= i) and (i - j < W).
 *  - "Attention Engineering ...", section 4, the FlashAttention-2 recurrence
 *    and its epilogue: the per-row log-sum-exp L = m + log(l).
 *  - "Attention deep dive ...", section 5 "The KV cache": at decode the one
 *    new query attends to every cached key (cached + new), so no causal
 *    mask applies inside the cache.
 *  - "Attention Engineering ...", section 3, equation "Complete MLA
 *    Attention Score": s = (q_absorbed . c + q_R . k_R) / sqrt(d_h + d_R),
 *    and the absorbed output sum_s alpha_s c_s before W_UV.
 *
 * Conventions (readings where the pages leave a step open):
 *  - the caller passes the softmax scale (1/sqrt(d_h) for plain attention,
 *    1/sqrt(d_h + d_R) for MLA); it multiplies the dot product before the
 *    mask and the softmax;
 *  - a masked entry is excluded from the softmax (a select, not an added
 *    -inf), so a non-finite value at a masked key never reaches the result;
 *  - a row with no visible key has output 0 and log-sum-exp -inf;
 *  - the log-sum-exp is the natural logarithm.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Visibility of key j to query i for the prefill mask.  Causal: j <= i.
 * Window W > 0: additionally i - j < W ("Attention deep dive", section 6). */
static int prefill_visible(long i, long j, int causal, int window)
{
    if (causal && j > i) return 0;
    if (window > 0 && i - j >= window) return 0;
    return 1;
}

/* softmax over the visible entries of s[0..n), then out[d] = sum_j p_j v_j[d].
 * v_row(j) points at the value row of key j (stride vstride floats).
 * `sink` (-INFINITY for none) is an extra logit in the softmax denominator
 * with no value row ("Attention Engineering ...", section 5, failure mode
 * 2: a learnable scalar sink logit in the denominator).
 * Writes out[0..dv) and *lse. */
static void softmax_weights(const double *s, const unsigned char *vis, long n,
                            double *p, double *lse, double sink)
{
    double m = -INFINITY;
    long any = 0;
    for (long j = 0; j < n; ++j)
        if (vis[j]) { if (!any || s[j] > m) m = s[j]; any = 1; }
    if (sink != -INFINITY && (!any || sink > m)) m = sink;
    if (!any) {
        for (long j = 0; j < n; ++j) p[j] = 0.0;
        *lse = sink;
        return;
    }
    double l = sink != -INFINITY ? exp(sink - m) : 0.0;
    for (long j = 0; j < n; ++j) {
        p[j] = vis[j] ? exp(s[j] - m) : 0.0;
        l += p[j];
    }
    for (long j = 0; j < n; ++j) p[j] /= l;
    *lse = m + log(l);
}

static void softmax_mix(const double *s, const unsigned char *vis, long n,
                        const float *v, long vstride, int dv,
                        double *out, double *lse, double *p, double sink)
{
    softmax_weights(s, vis, n, p, lse, sink);
    for (int d = 0; d < dv; ++d) out[d] = 0.0;
    for (long j = 0; j < n; ++j) {
        if (!vis[j]) continue;
        const float *vr = v + j * vstride;
        for (int d = 0; d < dv; ++d) out[d] += p[j] * (double)vr[d];
    }
}

/* the same with double value rows */
static void softmax_mix_d(const double *s, const unsigned char *vis, long n,
                          const double *v, long vstride, int dv,
                          double *out, double *lse, double *p, double sink)
{
    softmax_weights(s, vis, n, p, lse, sink);
    for (int d = 0; d < dv; ++d) out[d] = 0.0;
    for (long j = 0; j < n; ++j) {
        if (!vis[j]) continue;
        const double *vr = v + j * vstride;
        for (int d = 0; d < dv; ++d) out[d] += p[j] * vr[d];
    }
}

/*
 * Prefill forward.  q:[B,hq,T,d]  k,v:[B,hkv,T,d]  (row-major, float).
 * rows: optional list of n_rows query positions to evaluate (NULL = all T,
 * in order).  o:[B,hq,n_rows,d]  lse:[B,hq,n_rows] (may be NULL).
 * Query head h reads KV head h / (hq / hkv).
 * Returns 0, or -1 for an invalid shape.
 */
int oracle_prefill(const float *q, const float *k, const float *v,
                   double *o, double *lse,
                   int B, int T, int hq, int hkv, int d,
                   int causal, int window, double scale,
                   const int *rows, int n_rows, const float *sinks)
{
    if (B < 0 || T < 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv) return -1;
    if (!rows) n_rows = T;
    const int G = hq / hkv;
    const long units = (long)B * hq * n_rows;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (T > 0 ? T : 1));
        double *p = (double *)malloc(sizeof(double) * (T > 0 ? T : 1));
        unsigned char *vis = (unsigned char *)malloc(T > 0 ? T : 1);
#pragma omp for schedule(dynamic, 16)
        for (long u = 0; u < units; ++u) {
            const long r = u % n_rows;
            const long h = (u / n_rows) % hq;
            const long b = u / ((long)n_rows * hq);
            const long i = rows ? rows[r] : r;
            const long g = h / G;
            const float *qi = q + (((b * hq + h) * T) + i) * d;
            const float *kb = k + ((b * hkv + g) * (long)T) * d;
            const float *vb = v + ((b * hkv + g) * (long)T) * d;
            /* full score row, then the mask */
            for (long j = 0; j < T; ++j) {
                double acc = 0.0;
                const float *kj = kb + j * d;
                for (int t = 0; t < d; ++t) acc += (double)qi[t] * (double)kj[t];
                s[j] = acc * scale;
                vis[j] = (unsigned char)prefill_visible(i, j, causal, window);
            }
            double l_out;
            softmax_mix(s, vis, T, vb, d, d, o + u * d, &l_out, p,
                        sinks ? (double)sinks[h] : -INFINITY);
            if (lse) lse[u] = l_out;
        }
        free(s); free(p); free(vis);
    }
    return 0;
}

/*
 * Prefill backward: the gradients of the prefill forward above with respect
 * to q, k and v, given the gradient dO of its output.
 *
 * The pages keep only the per-row log-sum-exp of the forward for the
 * backward pass and have it recompute the scores ("Attention Engineering
 * ...", section 4, the text after the FlashAttention-2 recurrence;
 * "Attention, Worked Out by Hand (Part 2)", section 2).  The gradient itself
 * is the chain rule applied to the plain forward, with every score row
 * materialised (P_ij the softmax weight of visible key j in row i, 0 for a
 * masked key):
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 * where for K and V the sums over i also run over the query heads of the
 * group that shares them.  With a sink logit per query head (sinks may be
 * NULL) P_ij is the weight under the sink-augmented denominator; the sink
 * has no value row, so the formulas are otherwise unchanged.  The sink's
 * own gradient (dsinks may be NULL) is the derivative of the loss through
 * the denominator alone: with P_i = exp(sink - lse_i) the sink's weight in
 * row i, dsink = -sum over the head's rows of P_i sum_j P_ij dP_ij.
 *
 * Two plain passes: the first goes over query rows (log-sum-exp, the row
 * dot product sum_j P_ij dP_ij, and dQ_i); the second over keys of each
 * K/V head (dK_j, dV_j), recomputing P_ij = exp(s_ij - lse_i).
 * q, dout:[B,hq,T,d]  k,v:[B,hkv,T,d]  (float);  dq:[B,hq,T,d],
 * dk,dv:[B,hkv,T,d] (double).  Returns 0, or -1 for an invalid shape.
 */
int oracle_prefill_backward(const float *q, const float *k, const float *v,
                            const float *dout, double *dq, double *dk, double *dv,
                            int B, int T, int hq, int hkv, int d,
                            int causal, int window, double scale, const float *sinks,
                            double *dsinks)
{
    if (B < 0 || T < 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv) return -1;
    const int G = hq / hkv;
    const long rows = (long)B * hq * T;
    double *lse = (double *)malloc(sizeof(double) * (rows > 0 ? rows : 1));
    double *rdot = (double *)malloc(sizeof(double) * (rows > 0 ? rows : 1));
    double *sgrad = (double *)malloc(sizeof(double) * (rows > 0 ? rows : 1));
    if (!lse || !rdot || !sgrad) { free(lse); free(rdot); free(sgrad); return -1; }
    /* pass 1: one query row at a time */
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (T > 0 ? T : 1));
        double *dp = (double *)malloc(sizeof(double) * (T > 0 ? T : 1));
        unsigned char *vis = (unsigned char *)malloc(T > 0 ? T : 1);
#pragma omp for schedule(dynamic, 16)
        for (long u = 0; u < rows; ++u) {
            const long i = u % T;
            const long h = (u / T) % hq;
            const long b = u / ((long)T * hq);
            const long g = h / G;
            const float *qi = q + u * d;
            const float *doi = dout + u * d;
            const float *kb = k + ((b * hkv + g) * (long)T) * d;
            const float *vb = v + ((b * hkv + g) * (long)T) * d;
            double m = -INFINITY;
            int any = 0;
            for (long j = 0; j < T; ++j) {
                vis[j] = (unsigned char)prefill_visible(i, j, causal, window);
                s[j] = 0.0;
                dp[j] = 0.0;
                if (!vis[j]) continue;
                double acc = 0.0, accv = 0.0;
                for (int t = 0; t < d; ++t) {
                    acc += (double)qi[t] * (double)kb[j * d + t];
                    accv += (double)doi[t] * (double)vb[j * d + t];
                }
                s[j] = acc * scale;
                dp[j] = accv;
                if (!any || s[j] > m) m = s[j];
                any = 1;
            }
            double *dqi = dq + u * d;
            for (int t = 0; t < d; ++t) dqi[t] = 0.0;
            if (!any) { lse[u] = -INFINITY; rdot[u] = 0.0; sgrad[u] = 0.0; continue; }
            /* a sink logit only adds a term to the denominator (no value row) */
            const double sk = sinks ? (double)sinks[h] : -INFINITY;
            if (sk > m) m = sk;
            double l = sk != -INFINITY ? exp(sk - m) : 0.0;
            for (long j = 0; j < T; ++j)
                if (vis[j]) l += exp(s[j] - m);
            const double L = m + log(l);
            double rd = 0.0;
            for (long j = 0; j < T; ++j)
                if (vis[j]) rd += exp(s[j] - L) * dp[j];
            lse[u] = L;
            rdot[u] = rd;
            sgrad[u] = sk != -INFINITY ? -exp(sk - L) * rd : 0.0;
            for (long j = 0; j < T; ++j) {
                if (!vis[j]) continue;
                const double ds = exp(s[j] - L) * (dp[j] - rd);
                for (int t = 0; t < d; ++t) dqi[t] += scale * ds * (double)kb[j * d + t];
            }
        }
        free(s); free(dp); free(vis);
    }
    if (dsinks)
        for (long h = 0; h < hq; ++h) {
            double acc = 0.0;
            for (long b = 0; b < B; ++b)
                for (long i = 0; i < T; ++i) acc += sgrad[(b * hq + h) * (long)T + i];
            dsinks[h] = acc;
        }
    /* pass 2: one key of one K/V head at a time, over the group's query rows */
    const long keys = (long)B * hkv * T;
#pragma omp parallel for schedule(dynamic, 16)
    for (long u = 0; u < keys; ++u) {
        const long j = u % T;
        const long g = (u / T) % hkv;
        const long b = u / ((long)T * hkv);
        const float *kj = k + u * d;
        const float *vj = v + u * d;
        double *dkj = dk + u * d;
        double *dvj = dv + u * d;
        for (int t = 0; t < d; ++t) { dkj[t] = 0.0; dvj[t] = 0.0; }
        for (long h = g * G; h < (g + 1) * G; ++h) {
            for (long i = 0; i < T; ++i) {
                if (!prefill_visible(i, j, causal, window)) continue;
                const long r = ((b * hq + h) * (long)T) + i;
                const float *qi = q + r * d;
                const float *doi = dout + r * d;
                double acc = 0.0, accv = 0.0;
                for (int t = 0; t < d; ++t) {
                    acc += (double)qi[t] * (double)kj[t];
                    accv += (double)doi[t] * (double)vj[t];
                }
                const double p = exp(acc * scale - lse[r]);
                const double ds = p * (accv - rdot[r]);
                for (int t = 0; t < d; ++t) {
                    dvj[t] += p * (double)doi[t];
                    dkj[t] += scale * ds * (double)qi[t];
                }
            }
        }
    }
    free(lse); free(rdot); free(sgrad);
    return 0;
}

/*
 * Single-token decode against a KV cache.
 * q:[B,hq,d]  kc,vc:[B,hkv,S_max,d]  seq_lens[B] (valid cached length of
 * sequence b, already including the current token).  The query is the
 * token at position len-1; it sees cache positions j < len, and with a
 * window W > 0 only those with (len-1) - j < W.
 * o:[B,hq,d]  lse:[B,hq] (may be NULL).
 */
int oracle_decode(const float *q, const float *kc, const float *vc,
                  const int *seq_lens, double *o, double *lse,
                  int B, int S_max, int hq, int hkv, int d,
                  int window, double scale, const float *sinks)
{
    if (B < 0 || S_max < 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv) return -1;
    const int G = hq / hkv;
    const long units = (long)B * hq;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (S_max > 0 ? S_max : 1));
        double *p = (double *)malloc(sizeof(double) * (S_max > 0 ? S_max : 1));
        unsigned char *vis = (unsigned char *)malloc(S_max > 0 ? S_max : 1);
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            const long h = u % hq, b = u / hq, g = h / G;
            long len = seq_lens[b];
            if (len < 0) len = 0;
            if (len > S_max) len = S_max;
            const long i = len - 1;
            const float *qi = q + (b * hq + h) * (long)d;
            const float *kb = kc + ((b * hkv + g) * (long)S_max) * d;
            const float *vb = vc + ((b * hkv + g) * (long)S_max) * d;
            for (long j = 0; j < len; ++j) {
                double acc = 0.0;
                const float *kj = kb + j * d;
                for (int t = 0; t < d; ++t) acc += (double)qi[t] * (double)kj[t];
                s[j] = acc * scale;
                vis[j] = (unsigned char)(window <= 0 || i - j < window);
            }
            double l_out;
            softmax_mix(s, vis, len, vb, d, d, o + u * d, &l_out, p,
                        sinks ? (double)sinks[h] : -INFINITY);
            if (lse) lse[u] = l_out;
        }
        free(s); free(p); free(vis);
    }
    return 0;
}

/*
 * MLA absorbed-latent decode.
 * q:[B,H,dc+dr]: per head the absorbed content query (first dc entries)
 *   followed by the rotated decoupled query (last dr entries).
 * cache:[B,S_max,dc+dr]: per token the latent c (first dc) followed by the
 *   shared rotated key k_R (last dr).
 * s_j = scale * (q[0:dc] . c_j + q[dc:] . kR_j); o = sum_j softmax_j c_j,
 * i.e. the latent context before the W_UV up-projection.
 * o:[B,H,dc]  lse:[B,H] (may be NULL).
 */
int oracle_mla_decode(const float *q, const float *cache, const int *seq_lens,
                      double *o, double *lse,
                      int B, int S_max, int H, int dc, int dr, double scale,
                      const float *sinks)
{
    if (B < 0 || S_max < 0 || H <= 0 || dc <= 0 || dr < 0) return -1;
    const int dk = dc + dr;
    const long units = (long)B * H;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (S_max > 0 ? S_max : 1));
        double *p = (double *)malloc(sizeof(double) * (S_max > 0 ? S_max : 1));
        unsigned char *vis = (unsigned char *)malloc(S_max > 0 ? S_max : 1);
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            const long b = u / H;
            long len = seq_lens[b];
            if (len < 0) len = 0;
            if (len > S_max) len = S_max;
            const float *qh = q + u * (long)dk;
            const float *cb = cache + b * (long)S_max * dk;
            for (long j = 0; j < len; ++j) {
                const float *cj = cb + j * dk;
                double content = 0.0, rope = 0.0;
                for (int t = 0; t < dc; ++t) content += (double)qh[t] * (double)cj[t];
                for (int t = 0; t < dr; ++t) rope += (double)qh[dc + t] * (double)cj[dc + t];
                s[j] = (content + rope) * scale;
                vis[j] = 1;
            }
            double l_out;
            softmax_mix(s, vis, len, cb, dk, dc, o + u * dc, &l_out, p,
                        sinks ? (double)sinks[u % H] : -INFINITY);
            if (lse) lse[u] = l_out;
        }
        free(s); free(p); free(vis);
    }
    return 0;
}

/*
 * Merge of partial attention results over disjoint key sets.
 * Each part s carries a normalised output O_s (over its own keys) and its
 * log-sum-exp L_s.  The union's result follows from the FlashAttention-2
 * state ("Attention Engineering ...", section 4): L = log sum_s exp(L_s),
 * O = sum_s exp(L_s - L) O_s.  Parts with L_s = -inf (no keys) drop out.
 * parts_o:[n_parts,dv]  parts_lse:[n_parts]  ->  o:[dv], *lse.
 */
void oracle_merge_partials(const double *parts_o, const double *parts_lse,
                           int n_parts, int dv, double *o, double *lse)
{
    double m = -INFINITY;
    for (int s = 0; s < n_parts; ++s)
        if (parts_lse[s] > m) m = parts_lse[s];
    for (int t = 0; t < dv; ++t) o[t] = 0.0;
    if (m == -INFINITY) { *lse = -INFINITY; return; }
    double z = 0.0;
    for (int s = 0; s < n_parts; ++s)
        if (parts_lse[s] != -INFINITY) z += exp(parts_lse[s] - m);
    const double L = m + log(z);
    for (int s = 0; s < n_parts; ++s) {
        if (parts_lse[s] == -INFINITY) continue;
        const double w = exp(parts_lse[s] - L);
        for (int t = 0; t < dv; ++t) o[t] += w * parts_o[(long)s * dv + t];
    }
    *lse = L;
}

/* Threads the OpenMP regions above use (0 leaves the runtime default). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * FP8 KV cache.
 *
 * Format: OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); no infinities; the
 * all-ones magnitude 0x7f is NaN; the largest finite value is 448.  This is
 * the FP8 type of the pages' per-tile quantisation ("Flash Attention 3 and
 * Multi-Headed Latent Attention", the FP8 attention section: the scale is
 * the tile's absolute maximum over 448, the E4M3 maximum) and of the
 * quantised caches the pages name ("Attention deep dive ...", section 5,
 * production-engine notes; "2.4 Multi-Head Attention, MQA, GQA & MLA": an
 * fp8 cache stacks with GQA).
 *
 * Tile of the cache (reading): 32 consecutive positions of one K/V head of
 * one sequence, all d_h values of each; one fp32 scale per tile and per
 * tensor (K and V separately).  scale = amax / 448 (fp32 division; 1 for an
 * all-zero tile), code = nearest E4M3 value of x / scale (fp32 division),
 * ties to the even code, magnitudes above 448 saturated to 448.
 *
 * Non-finite input (reading): E4M3 has no infinities; its only non-finite
 * value is NaN (codes 0x7f and 0xff).  A NaN or an infinity is stored as
 * that NaN code with the input's sign bit, so it stays non-finite when the
 * cache is read back.  The scale is a statistic of the values the type can
 * hold, so amax runs over the tile's finite values only: a non-finite entry
 * leaves the codes of its finite neighbours unchanged.
 */
static double fp8_value(unsigned code)
{
    const unsigned e = (code >> 3) & 15u, m = code & 7u;
    const double sgn = (code & 0x80u) ? -1.0 : 1.0;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) return sgn * ldexp((double)m / 8.0, -6);
    return sgn * ldexp(1.0 + (double)m / 8.0, (int)e - 7);
}

double oracle_fp8_e4m3_value(int code) { return fp8_value((unsigned)code & 0xffu); }

/* nearest finite E4M3 code to v, ties to the even code, saturating;
 * NaN and +-infinity give the NaN code with v's sign */
static unsigned char fp8_encode(float v)
{
    if (isnan(v) || isinf(v)) return (unsigned char)(signbit(v) ? 0xffu : 0x7fu);
    const double a = fabs((double)v);
    unsigned best = 0;
    double best_err = INFINITY;
    for (unsigned c = 0; c < 127u; ++c) {        /* every finite non-negative code */
        const double err = fabs(fp8_value(c) - a);
        if (err < best_err || (err == best_err && (c & 1u) == 0u)) {
            best = c;
            best_err = err;
        }
    }
    if (a >= 448.0) best = 126u;                 /* saturate */
    return (unsigned char)(best | (signbit(v) ? 0x80u : 0u));
}

int oracle_fp8_e4m3_encode(float v) { return (int)fp8_encode(v); }

/* One tile of n values: scale = amax / 448 over its finite values (1 when
 * that is 0), codes = E4M3 of x / scale. */
static float quantize_block(const float *x, long n, unsigned char *codes)
{
    float amax = 0.0f;
    for (long i = 0; i < n; ++i) {
        const float a = fabsf(x[i]);
        if (isfinite(a) && a > amax) amax = a;
    }
    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (long i = 0; i < n; ++i)
        codes[i] = fp8_encode(isfinite(x[i]) ? x[i] / sc : x[i]);
    return sc;
}

/* x:[B,hkv,S,d] float -> codes:[B,hkv,S,d], scales:[B,hkv,ceil(S/32)] */
int oracle_quantize_kv_fp8(const float *x, unsigned char *codes, float *scales,
                           int B, int hkv, int S, int d)
{
    if (B < 0 || hkv <= 0 || S < 0 || d <= 0) return -1;
    const long nt = (S + 31) / 32;
    const long tiles = (long)B * hkv * nt;
#pragma omp parallel for schedule(static)
    for (long u = 0; u < tiles; ++u) {
        const long t = u % nt, bg = u / nt;
        const long r0 = t * 32, r1 = (r0 + 32 < S) ? r0 + 32 : S;
        const long off = (bg * (long)S + r0) * d;
        scales[u] = quantize_block(x + off, (r1 - r0) * d, codes + off);
    }
    return 0;
}

/*
 * Decode against an FP8 cache: the plain decode (see oracle_decode) on the
 * dequantised values code * scale of the cache tile, in double.
 * k8, v8:[B,hkv,S_max,d] codes; ks, vs:[B,hkv,ceil(S_max/32)] scales.
 */
int oracle_decode_fp8(const float *q, const unsigned char *k8, const unsigned char *v8,
                      const float *ks, const float *vs, const int *seq_lens,
                      double *o, double *lse, int B, int S_max, int hq, int hkv, int d,
                      int window, double scale, const float *sinks)
{
    if (B < 0 || S_max < 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv) return -1;
    const int G = hq / hkv;
    const long nt = (S_max + 31) / 32;
    const long units = (long)B * hq;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (S_max > 0 ? S_max : 1));
        double *p = (double *)malloc(sizeof(double) * (S_max > 0 ? S_max : 1));
        unsigned char *vis = (unsigned char *)malloc(S_max > 0 ? S_max : 1);
        double *vdq = (double *)malloc(sizeof(double) * ((long)(S_max > 0 ? S_max : 1) * d));
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            const long h = u % hq, b = u / hq, g = h / G;
            long len = seq_lens[b];
            if (len < 0) len = 0;
            if (len > S_max) len = S_max;
            const long i = len - 1;
            const float *qi = q + (b * hq + h) * (long)d;
            const long bg = b * hkv + g;
            const unsigned char *kb = k8 + (bg * (long)S_max) * d;
            const unsigned char *vb = v8 + (bg * (long)S_max) * d;
            for (long j = 0; j < len; ++j) {
                const double ksc = (double)ks[bg * nt + j / 32];
                const double vsc = (double)vs[bg * nt + j / 32];
                double acc = 0.0;
                for (int t = 0; t < d; ++t)
                    acc += (double)qi[t] * (fp8_value(kb[j * d + t]) * ksc);
                s[j] = acc * scale;
                vis[j] = (unsigned char)(window <= 0 || i - j < window);
                for (int t = 0; t < d; ++t) vdq[j * d + t] = fp8_value(vb[j * d + t]) * vsc;
            }
            double l_out;
            softmax_mix_d(s, vis, len, vdq, d, d, o + u * d, &l_out, p,
                          sinks ? (double)sinks[h] : -INFINITY);
            if (lse) lse[u] = l_out;
        }
        free(s); free(p); free(vis); free(vdq);
    }
    return 0;
}

/*
 * MLA absorbed decode in FP8: the pages' FP8 attention ("Flash Attention 3
 * and Multi-Headed Latent Attention", the FP8 attention section and the
 * FA3FP8BlockProcessor listing: q, k, v and p quantised to E4M3 per tile
 * with scale = amax / 448, both products on FP8 operands, the results
 * dequantised by the scales) applied to the MLA decode of "Attention
 * Engineering ...", section 3, as that page's combined FA3 + MLA kernel box
 * suggests.  Steps, per sequence b and head h:
 *
 *  1. the query row (576 values) is one tile: sq = amax / 448, q8 = E4M3(q /
 *     sq) -- the quantiser above on a one-row tile;
 *  2. the cache holds codes c8 with one scale sc per 32 tokens (the FP8 cache
 *     quantiser above with h_kv = 1); the value of token j is the first d_c
 *     entries of its dequantised row, so k and v share their codes and scale;
 *  3. s_j = scale * sq * sc_j * sum_d q8[d] c8_j[d] (exact dequantised
 *     product), in natural units;
 *  4. the weight of token j in the value product carries its tile's value
 *     scale: y_j = s_j log2(e) + log2(sc_j).  The keys of the sequence are
 *     taken in chunks of `split` tokens and each chunk in compute tiles of
 *     `tile` tokens in order.  The chunk keeps a reference R (-inf at the
 *     start); before a tile's weights are taken, if the tile's max of y
 *     exceeds R, R moves to that max plus MLA_FP8_HEADROOM (5, in log2
 *     units), so later tiles may rise by up to 2^5 before R has to move
 *     again;
 *  5. p is quantised to E4M3 against that reference: P8_j = E4M3(min(448,
 *     448 * 2^(y_j - R))) with the value scale folded in -- the pages' p /
 *     (amax / 448) with amax bounded by 2^R (every y_j <= R, so no weight
 *     passes 448); when R moves, the chunk's accumulated numerator and
 *     denominator are rescaled by 2^(R_old - R_new);
 *  6. the numerator N = sum_j P8_j * c8_j[0:d_c] (exact), the denominator the
 *     unquantised l = sum_j 2^(s_j log2(e) - R) (the page normalises the
 *     softmax before quantising p); the chunk's output N / (448 l) and
 *     log-sum-exp (R + log2 l) ln 2;
 *  7. chunks merge by their log-sum-exp (oracle_merge_partials), with the
 *     sink logit as one more part of zero output.
 * q:[B,H,dc+dr] float (bf16 values); c8:[B,S_max,dc+dr] codes; cs:[B,
 * ceil(S_max/32)] scales; o:[B,H,dc]; lse:[B,H].  split and tile are
 * positive multiples of 32, tile divides split.
 */
#define MLA_FP8_HEADROOM 5.0

int oracle_mla_decode_fp8(const float *q, const unsigned char *c8, const float *cs,
                          const int *seq_lens, double *o, double *lse,
                          int B, int S_max, int H, int dc, int dr, double scale,
                          const float *sinks, int split, int tile)
{
    if (B < 0 || S_max < 0 || H <= 0 || dc <= 0 || dr < 0 || split <= 0 || tile <= 0 ||
        split % 32 || tile % 32 || split % tile) return -1;
    const int dk = dc + dr;
    double val[256];                   /* fp8_value of every code, looked up below */
    for (int c = 0; c < 256; ++c) val[c] = fp8_value((unsigned)c);
    const long nt = (S_max + 31) / 32;
    const long units = (long)B * H;
    const double log2e = 1.0 / log(2.0);
#pragma omp parallel
    {
        unsigned char *q8 = (unsigned char *)malloc(dk);
        double *num = (double *)malloc(sizeof(double) * dc);
        double *y = (double *)malloc(sizeof(double) * (tile > 0 ? tile : 1));
        double *sn = (double *)malloc(sizeof(double) * (tile > 0 ? tile : 1));
        const long max_parts = S_max / split + 2;
        double *part_o = (double *)malloc(sizeof(double) * max_parts * dc);
        double *part_l = (double *)malloc(sizeof(double) * max_parts);
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            const long b = u / H, h = u % H;
            long len = seq_lens[b];
            if (len < 0) len = 0;
            if (len > S_max) len = S_max;
            const double sq = (double)quantize_block(q + u * dk, dk, q8);
            int np = 0;
            for (long c0 = 0; c0 < len; c0 += split) {
                const long c1 = c0 + split < len ? c0 + split : len;
                double R = -INFINITY, l = 0.0;
                for (int d = 0; d < dc; ++d) num[d] = 0.0;
                for (long t0 = c0; t0 < c1; t0 += tile) {
                    const long t1 = t0 + tile < c1 ? t0 + tile : c1;
                    double tmax = -INFINITY;
                    for (long j = t0; j < t1; ++j) {
                        const unsigned char *row = c8 + ((size_t)b * S_max + j) * dk;
                        const double sc = (double)cs[b * nt + j / 32];
                        double acc = 0.0;
                        for (int d = 0; d < dk; ++d) acc += val[q8[d]] * val[row[d]];
                        sn[j - t0] = scale * sq * sc * acc;
                        y[j - t0] = sn[j - t0] * log2e + log2(sc);
                        if (y[j - t0] > tmax) tmax = y[j - t0];
                    }
                    if (tmax > R) {                 /* move the reference, rescale */
                        const double Rn = tmax + MLA_FP8_HEADROOM;
                        const double f = R == -INFINITY ? 0.0 : exp2(R - Rn);
                        for (int d = 0; d < dc; ++d) num[d] *= f;
                        l *= f;
                        R = Rn;
                    }
                    for (long j = t0; j < t1; ++j) {
                        const unsigned char *row = c8 + ((size_t)b * S_max + j) * dk;
                        double w = 448.0 * exp2(y[j - t0] - R);
                        if (w > 448.0) w = 448.0;
                        const double pq = val[fp8_encode((float)w)];
                        for (int d = 0; d < dc; ++d) num[d] += pq * val[row[d]];
                        l += exp2(sn[j - t0] * log2e - R);
                    }
                }
                for (int d = 0; d < dc; ++d) part_o[(long)np * dc + d] = num[d] / (448.0 * l);
                part_l[np] = (R + log2(l)) * log(2.0);
                ++np;
            }
            if (sinks && sinks[h] != -INFINITY) {
                for (int d = 0; d < dc; ++d) part_o[(long)np * dc + d] = 0.0;
                part_l[np++] = (double)sinks[h];
            }
            double l_out;
            oracle_merge_partials(part_o, part_l, np, dc, o + u * dc, &l_out);
            if (lse) lse[u] = l_out;
        }
        free(q8); free(num); free(y); free(sn); free(part_o); free(part_l);
    }
    return 0;
}

/*
 * Prefill with FP8 attention: the pages' FP8 recipe ("Flash Attention 3 and
 * Multi-Headed Latent Attention", the FP8 attention section: q, k and v
 * quantised to E4M3 per tile with scale amax / 448, both products on FP8
 * operands, p quantised before the second) on the prefill forward above,
 * with the steps and readings of oracle_mla_decode_fp8:
 *  - q, k and v arrive as codes with one scale per 32 positions of a head
 *    (the cache quantiser's tiles): qs[b,h,i/32], ks / vs[b,g,j/32];
 *  - s_ij = scale * qs_i * ks_j * (q8_i . k8_j) (exact dequantised product);
 *  - the weight of key j carries its value scale: y_ij = s_ij log2(e) +
 *    log2(vs_j);
 *  - row i takes its visible keys in tiles of `tile` keys aligned at
 *    multiples of `tile`, in increasing order; its reference R (-inf at the
 *    start) moves to a tile's max of y plus MLA_FP8_HEADROOM when the tile
 *    exceeds it, rescaling what was accumulated by 2^(R_old - R_new);
 *  - P8_ij = E4M3(min(448, 448 * 2^(y_ij - R))); numerator sum_j P8_ij v8_j,
 *    unquantised denominator l = sum_j 2^(s_ij log2(e) - R); o = num / (448
 *    l), lse = (R + log2 l) ln 2; a sink logit joins as in the plain prefill.
 * q8:[B,hq,T,d] qs:[B,hq,ceil(T/32)]  k8,v8:[B,hkv,T,d] ks,vs:[B,hkv,ceil(T/32)]
 * row_list: optional n_rows query positions (NULL = all T, in order);
 * o:[B,hq,n_rows,d]  lse:[B,hq,n_rows] (may be NULL).
 */
int oracle_prefill_fp8(const unsigned char *q8, const float *qs, const unsigned char *k8,
                       const float *ks, const unsigned char *v8, const float *vs,
                       double *o, double *lse, int B, int T, int hq, int hkv, int d,
                       int causal, int window, double scale, const float *sinks, int tile,
                       const int *row_list, int n_rows)
{
    if (B < 0 || T < 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv || tile <= 0 || tile % 32)
        return -1;
    if (!row_list) n_rows = T;
    const int G = hq / hkv;
    const long nt = (T + 31) / 32;
    const long rows = (long)B * hq * n_rows;
    const double log2e = 1.0 / log(2.0);
    double val[256];
    for (int c = 0; c < 256; ++c) val[c] = fp8_value((unsigned)c);
#pragma omp parallel
    {
        double *num = (double *)malloc(sizeof(double) * d);
        double *sn = (double *)malloc(sizeof(double) * tile);
        double *y = (double *)malloc(sizeof(double) * tile);
        unsigned char *vis = (unsigned char *)malloc(tile);
#pragma omp for schedule(dynamic, 16)
        for (long u = 0; u < rows; ++u) {
            const long r = u % n_rows, h = (u / n_rows) % hq, b = u / ((long)n_rows * hq);
            const long i = row_list ? row_list[r] : r;
            const long g = h / G, bg = b * hkv + g;
            const unsigned char *qi = q8 + (((b * hq + h) * (long)T) + i) * d;
            const double sq = (double)qs[(b * hq + h) * nt + i / 32];
            double R = -INFINITY, l = 0.0;
            for (int e = 0; e < d; ++e) num[e] = 0.0;
            for (long t0 = 0; t0 < T; t0 += tile) {
                double tmax = -INFINITY;
                int any = 0;
                for (long j = t0; j < t0 + tile; ++j) {
                    vis[j - t0] = (unsigned char)(j < T && prefill_visible(i, j, causal, window));
                    if (!vis[j - t0]) continue;
                    any = 1;
                    const unsigned char *kj = k8 + (bg * (long)T + j) * d;
                    double acc = 0.0;
                    for (int e = 0; e < d; ++e) acc += val[qi[e]] * val[kj[e]];
                    sn[j - t0] = scale * sq * (double)ks[bg * nt + j / 32] * acc;
                    y[j - t0] = sn[j - t0] * log2e + log2((double)vs[bg * nt + j / 32]);
                    if (y[j - t0] > tmax) tmax = y[j - t0];
                }
                if (!any) continue;
                if (tmax > R) {
                    const double Rn = tmax + MLA_FP8_HEADROOM;
                    const double f = R == -INFINITY ? 0.0 : exp2(R - Rn);
                    for (int e = 0; e < d; ++e) num[e] *= f;
                    l *= f;
                    R = Rn;
                }
                for (long j = t0; j < t0 + tile; ++j) {
                    if (!vis[j - t0]) continue;
                    double w = 448.0 * exp2(y[j - t0] - R);
                    if (w > 448.0) w = 448.0;
                    const double pq = val[fp8_encode((float)w)];
                    const unsigned char *vj = v8 + (bg * (long)T + j) * d;
                    for (int e = 0; e < d; ++e) num[e] += pq * val[vj[e]];
                    l += exp2(sn[j - t0] * log2e - R);
                }
            }
            double *orow = o + u * d;
            double L = l > 0.0 ? (R + log2(l)) * log(2.0) : -INFINITY;
            for (int e = 0; e < d; ++e) orow[e] = l > 0.0 ? num[e] / (448.0 * l) : 0.0;
            if (sinks && sinks[h] != -INFINITY) {       /* merge with the sink's empty part */
                const double sk = (double)sinks[h];
                const double M = L > sk ? L : sk;
                const double Ln = M + log(exp(L - M) + exp(sk - M));
                const double f = L == -INFINITY ? 0.0 : exp(L - Ln);
                for (int e = 0; e < d; ++e) orow[e] *= f;
                L = Ln;
            }
            if (lse) lse[u] = L;
        }
        free(num); free(sn); free(y); free(vis);
    }
    return 0;
}

/*
 * Rotary position embedding ("Attention Engineering: From MHA to GQA, MLA &
 * FlashAttention", section 1, the complex-plane derivation and the
 * relative-distance identity): the rotated dimensions of a row are taken in
 * pairs (x_{2j}, x_{2j+1}), j = 0 .. rope_dim/2 - 1, each a complex number
 * rotated by the angle m * theta_j at token position m, with
 * theta_j = base^(-2j / rope_dim):
 *   x'_{2j}   = x_{2j} cos(m theta_j) - x_{2j+1} sin(m theta_j)
 *   x'_{2j+1} = x_{2j} sin(m theta_j) + x_{2j+1} cos(m theta_j).
 * The rotated dimensions are [rope_offset, rope_offset + rope_dim) of each
 * row (the whole head for GQA; the decoupled 64-d tail for MLA); the others
 * are copied.  x:[B, H, T, row] float; positions: [B, T] int or NULL (then
 * m = t); out:[B, H, T, row] double.
 */
int oracle_rope(const float *x, const int *positions, double *out, int B, int H, int T,
                int row, int rope_offset, int rope_dim, double base)
{
    if (B < 0 || H < 0 || T < 0 || row <= 0 || rope_dim < 0 || rope_dim % 2 ||
        rope_offset < 0 || rope_offset + rope_dim > row || !(base > 0.0)) return -1;
    const long rows = (long)B * H * T;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const long t = r % T, b = r / ((long)H * T);
        const double m = positions ? (double)positions[b * T + t] : (double)t;
        const float *xr = x + r * row;
        double *orow = out + r * row;
        for (int e = 0; e < row; ++e) orow[e] = (double)xr[e];
        for (int j = 0; j < rope_dim / 2; ++j) {
            const double theta = pow(base, -2.0 * j / rope_dim);
            const double c = cos(m * theta), s = sin(m * theta);
            const double a = xr[rope_offset + 2 * j], bb = xr[rope_offset + 2 * j + 1];
            orow[rope_offset + 2 * j] = a * c - bb * s;
            orow[rope_offset + 2 * j + 1] = a * s + bb * c;
        }
    }
    return 0;
}

