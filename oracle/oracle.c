/*
 * oracle.c - plain CPU reference of the speculative-decoding verification pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU library shares
 * no code with it: no headers, helpers, tables or constants.
 *
 * What it computes, and where the pages define it:
 *
 *  - GGUF block decode (Q8_0, Q4_K, Q6_K).  The pages name these formats and
 *    defer their definition to ggml ("How Kinetic is fast", References; the
 *    OpenJet page, "One GPU launch for a speculative cycle", says the
 *    projections keep the GGUF representations).  The bit layouts below are
 *    the public ggml ones.  Fidelity to real GGUF files: parity unpinned (no
 *    GGUF file or ggml source is available); the layouts are pinned by
 *    hand-built golden blocks instead.
 *  - Activation quantiser Q8A32 (int8 activations, OpenJet page, same
 *    section): per 32-element block, amax, d = amax/127, q = round-half-away
 *    (x * (1/d)) clamped to [-127, 127], and exact int sums per 16.  This
 *    decides integers from floats, so it runs in fp32, the precision the GPU
 *    kernel uses.
 *  - Projection Y = W * A for M positions sharing one weight read (OpenJet
 *    page, "The bottleneck" and "One GPU launch..."; Kinetic page, "RAD-1").
 *    Integer block sums are exact (int64); each block term and the row sum
 *    are fp64 and the row sum is sequential in block order.  T = sum |term|
 *    is returned beside it: it bounds the rounding any summation order adds.
 *  - Head argmax (ties to the lowest index), greedy acceptance (Kinetic page,
 *    "Why the output does not change": keep a guess only when it is the top
 *    token), rejection acceptance (micrologics page, "Mathematical Integrity:
 *    Rejection Sampling for LLMs", the alpha and p' equations), and sampling
 *    against a certain one-token drafter (Kinetic page, same section).  All
 *    probabilities are fp64; sampling is the inverse CDF in index order.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_Q8_0 8
#define OR_Q4_K 12
#define OR_Q6_K 14

/* ------------------------------------------------------------------ */
/* fp16 -> double, exact (subnormals included).                        */
/* ------------------------------------------------------------------ */
double or_half(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = m ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------------ */
/* Block decoders.  Each writes integer quants for K elements of one   */
/* row plus the block scales, exactly as stored.                       */
/* ------------------------------------------------------------------ */

/* Q8_0: 34 bytes per 32 elements: fp16 d, int8 q[32].  w = d * q. */
void or_decode_q8_0(const uint8_t *row, int64_t K, int32_t *q, double *d) {
    for (int64_t b = 0; b < K / 32; b++) {
        const uint8_t *blk = row + b * 34;
        d[b] = or_half(rd16(blk));
        for (int i = 0; i < 32; i++) q[b * 32 + i] = (int8_t)blk[2 + i];
    }
}

/* Q4_K: 144 bytes per 256 elements: fp16 d, fp16 dmin, 12 bytes holding
 * eight 6-bit scales and eight 6-bit mins, 128 bytes of 4-bit quants.
 * Sub-block j (32 elements): w = d * sc[j] * q - dmin * m[j], q in [0,15].
 * Outputs: q[K], d[K/256], dmin[K/256], sc[K/32], m[K/32]. */
void or_decode_q4_k(const uint8_t *row, int64_t K, int32_t *q, double *d, double *dmin,
                    int32_t *sc, int32_t *m) {
    for (int64_t s = 0; s < K / 256; s++) {
        const uint8_t *blk = row + s * 144;
        const uint8_t *scl = blk + 4;
        const uint8_t *qs = blk + 16;
        d[s] = or_half(rd16(blk));
        dmin[s] = or_half(rd16(blk + 2));
        for (int j = 0; j < 8; j++) {
            int a, b;
            if (j < 4) {
                a = scl[j] & 63;
                b = scl[j + 4] & 63;
            } else {
                a = (scl[j + 4] & 15) | ((scl[j - 4] >> 6) << 4);
                b = (scl[j + 4] >> 4) | ((scl[j] >> 6) << 4);
            }
            sc[s * 8 + j] = a;
            m[s * 8 + j] = b;
        }
        /* 64-element chunk c uses bytes qs[32c .. 32c+31]: the low nibbles
         * hold sub-block 2c, the high nibbles sub-block 2c+1. */
        for (int c = 0; c < 4; c++)
            for (int i = 0; i < 32; i++) {
                uint8_t byte = qs[32 * c + i];
                q[s * 256 + 64 * c + i] = byte & 15;
                q[s * 256 + 64 * c + 32 + i] = byte >> 4;
            }
    }
}

/* Q6_K: 210 bytes per 256 elements: ql[128] low 4 bits, qh[64] high 2 bits,
 * int8 scales[16] (one per 16 elements), fp16 d.
 * w = d * scales[e/16] * (q - 32), q in [0,63].
 * Outputs: q[K] (0..63), d[K/256], sc[K/16]. */
void or_decode_q6_k(const uint8_t *row, int64_t K, int32_t *q, double *d, int32_t *sc) {
    for (int64_t s = 0; s < K / 256; s++) {
        const uint8_t *blk = row + s * 210;
        const uint8_t *ql = blk, *qh = blk + 128;
        const int8_t *scl = (const int8_t *)(blk + 192);
        d[s] = or_half(rd16(blk + 208));
        for (int k = 0; k < 16; k++) sc[s * 16 + k] = scl[k];
        for (int e = 0; e < 256; e++) {
            int h = e / 128, r = e % 128, g = r / 32, l = r % 32;
            uint8_t lb = ql[64 * h + l + 32 * (g % 2)];
            int lo = (g < 2) ? (lb & 15) : (lb >> 4);
            int hi = (qh[32 * h + l] >> (2 * g)) & 3;
            q[s * 256 + e] = lo | (hi << 4);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Activation quantiser Q8A32 (fp32 decisions).                        */
/* x[M][K] (optionally times gamma[K], one fp32 rounding per element)  */
/* -> q int8 [M][K], d fp32 [M][K/32], s16 int32 [M][K/16];            */
/* sumsq[M] (fp64, may be NULL) = sum of x^2 (before gamma).           */
/* ------------------------------------------------------------------ */
void or_quantize_act(const float *x, const float *gamma, int32_t M, int64_t K, int8_t *q,
                     float *d, int32_t *s16, double *sumsq) {
    for (int32_t mi = 0; mi < M; mi++) {
        const float *xr = x + (int64_t)mi * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; k++) ss += (double)xr[k] * (double)xr[k];
        if (sumsq) sumsq[mi] = ss;
        for (int64_t b = 0; b < K / 32; b++) {
            float v[32];
            float amax = 0.0f;
            for (int i = 0; i < 32; i++) {
                float t = xr[b * 32 + i];
                if (gamma) t = t * gamma[b * 32 + i];
                v[i] = t;
                float a = fabsf(t);
                if (a > amax) amax = a;
            }
            float dd = amax / 127.0f;
            float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
            d[(int64_t)mi * (K / 32) + b] = dd;
            int32_t s0 = 0, s1 = 0;
            for (int i = 0; i < 32; i++) {
                float r = roundf(v[i] * id);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                int8_t qi = (int8_t)r;
                q[(int64_t)mi * K + b * 32 + i] = qi;
                if (i < 16) s0 += qi; else s1 += qi;
            }
            s16[(int64_t)mi * (K / 16) + 2 * b] = s0;
            s16[(int64_t)mi * (K / 16) + 2 * b + 1] = s1;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Projection: y[m][n] = scale[m] * sum_b t_b, fp64, block order.      */
/* ------------------------------------------------------------------ */

/* Row kernel: exact integer block sums, fp64 terms.  bsum (may be NULL)
 * receives the integer sum of every 32-element block for this row and
 * each position: Q8_0 sum q_w q_a; Q4_K sum q q_a (0..15 quants);
 * Q6_K sum (q-32) q_a per 16-element half folded with the two int8 scales
 * sc0*S0 + sc1*S1. */
static void row_dot(int qtype, const uint8_t *wrow, int64_t K, const int8_t *qa,
                    const float *da, int32_t M, double *y, double *T, int64_t ystride,
                    int64_t *bsum, int64_t bstride,
                    int32_t *wq, double *wd, double *wd2, int32_t *wsc, int32_t *wm) {
    int64_t nb = K / 32;
    if (qtype == OR_Q8_0) or_decode_q8_0(wrow, K, wq, wd);
    else if (qtype == OR_Q4_K) or_decode_q4_k(wrow, K, wq, wd, wd2, wsc, wm);
    else or_decode_q6_k(wrow, K, wq, wd, wsc);
    for (int32_t mi = 0; mi < M; mi++) {
        const int8_t *a = qa + (int64_t)mi * K;
        const float *ad = da + (int64_t)mi * nb;
        double acc = 0.0, tabs = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            double t;
            int64_t bs;
            if (qtype == OR_Q8_0) {
                int64_t S = 0;
                for (int i = 0; i < 32; i++) S += (int64_t)wq[b * 32 + i] * a[b * 32 + i];
                bs = S;
                t = wd[b] * (double)ad[b] * (double)S;
            } else if (qtype == OR_Q4_K) {
                int64_t S = 0, A = 0;
                for (int i = 0; i < 32; i++) {
                    S += (int64_t)wq[b * 32 + i] * a[b * 32 + i];
                    A += a[b * 32 + i];
                }
                bs = S;
                int64_t sb = b / 8;
                /* d*sc*S and dmin*m*A are exact in fp64 (at most 11+6+16
                 * and 11+6+13 significant bits). */
                double dq = wd[sb] * (double)wsc[b] * (double)S;
                double mq = wd2[sb] * (double)wm[b] * (double)A;
                t = (double)ad[b] * (dq - mq);
            } else {
                int64_t S0 = 0, S1 = 0;
                for (int i = 0; i < 16; i++) {
                    S0 += (int64_t)(wq[b * 32 + i] - 32) * a[b * 32 + i];
                    S1 += (int64_t)(wq[b * 32 + 16 + i] - 32) * a[b * 32 + 16 + i];
                }
                int64_t I = (int64_t)wsc[2 * b] * S0 + (int64_t)wsc[2 * b + 1] * S1;
                bs = I;
                t = wd[b / 8] * (double)ad[b] * (double)I;
            }
            if (bsum) bsum[mi * bstride + b] = bs;
            acc += t;
            tabs += fabs(t);
        }
        y[mi * ystride] = acc;
        if (T) T[mi * ystride] = tabs;
    }
}

typedef struct {
    int qtype;
    const uint8_t *W;
    int64_t N, K, rb;
    const int8_t *qa;
    const float *da;
    int32_t M;
    const double *scale;
    const int32_t *row_ids;
    double *y, *T;
    int64_t *bsum;
    int64_t r0, r1;
} mv_job;

static int64_t row_bytes_of(int qtype, int64_t K) {
    if (qtype == OR_Q8_0) return K / 32 * 34;
    if (qtype == OR_Q4_K) return K / 256 * 144;
    return K / 256 * 210;
}

static void *mv_worker(void *p) {
    mv_job *j = (mv_job *)p;
    int32_t *wq = (int32_t *)malloc(sizeof(int32_t) * j->K);
    double *wd = (double *)malloc(sizeof(double) * (j->K / 32 + 1));
    double *wd2 = (double *)malloc(sizeof(double) * (j->K / 256 + 1));
    int32_t *wsc = (int32_t *)malloc(sizeof(int32_t) * (j->K / 16 + 1));
    int32_t *wm = (int32_t *)malloc(sizeof(int32_t) * (j->K / 32 + 1));
    int64_t nb = j->K / 32;
    for (int64_t n = j->r0; n < j->r1; n++) {
        int64_t src = j->row_ids ? j->row_ids[n] : n;
        row_dot(j->qtype, j->W + src * j->rb, j->K, j->qa, j->da, j->M, j->y + n,
                j->T ? j->T + n : NULL, j->N,
                j->bsum ? j->bsum + n * nb : NULL, j->N * nb,
                wq, wd, wd2, wsc, wm);
        if (j->scale)
            for (int32_t mi = 0; mi < j->M; mi++) {
                j->y[mi * j->N + n] *= j->scale[mi];
                if (j->T) j->T[mi * j->N + n] *= fabs(j->scale[mi]);
            }
    }
    free(wq); free(wd); free(wd2); free(wsc); free(wm);
    return NULL;
}

/*
 * y[M][N] (fp64) = scale[m] * (W_dequant . A_dequant) for rows n of W, or
 * rows row_ids[n] when row_ids is given (a restricted head).  T[M][N] gets
 * scale * sum|t_b| (may be NULL).  bsum[M][N][K/32] (may be NULL) gets the
 * exact integer block sums described at row_dot.  Rows are split over
 * nthreads threads; every row's arithmetic is independent of the split.
 */
int or_matvec(int qtype, const uint8_t *W, int64_t N, int64_t K, const int32_t *row_ids,
              const int8_t *qa, const float *da, int32_t M, const double *scale, double *y,
              double *T, int64_t *bsum, int32_t nthreads) {
    if (qtype != OR_Q8_0 && qtype != OR_Q4_K && qtype != OR_Q6_K) return -4;
    if (K % (qtype == OR_Q8_0 ? 32 : 256)) return -2;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (N < nthreads) nthreads = (int32_t)(N > 0 ? N : 1);
    pthread_t th[256];
    mv_job jobs[256];
    int64_t rb = row_bytes_of(qtype, K);
    for (int t = 0; t < nthreads; t++) {
        mv_job j = {qtype, W, N, K, rb, qa, da, M, scale, row_ids, y, T, bsum,
                    N * t / nthreads, N * (t + 1) / nthreads};
        jobs[t] = j;
    }
    for (int t = 1; t < nthreads; t++) pthread_create(&th[t], NULL, mv_worker, &jobs[t]);
    mv_worker(&jobs[0]);
    for (int t = 1; t < nthreads; t++) pthread_join(th[t], NULL);
    return 0;
}

/* ------------------------------------------------------------------ */
/* RMS factor of a producer output: r = 1/sqrt(sum y^2 / n + eps).     */
/* ------------------------------------------------------------------ */
double or_rms_factor(double sumsq, int64_t n, double eps) {
    return 1.0 / sqrt(sumsq / (double)n + eps);
}

/* ------------------------------------------------------------------ */
/* Argmax per row, ties to the lowest index.                           */
/* ------------------------------------------------------------------ */
void or_argmax(const double *logits, int32_t M, int64_t V, int64_t *idx) {
    for (int32_t mi = 0; mi < M; mi++) {
        const double *z = logits + (int64_t)mi * V;
        int64_t best = 0;
        for (int64_t j = 1; j < V; j++)
            if (z[j] > z[best]) best = j;
        idx[mi] = best;
    }
}

/* ------------------------------------------------------------------ */
/* Greedy acceptance.  Row i's top token judges draft i; the first     */
/* mismatch is replaced by the top token, and if every draft matches   */
/* row K supplies one more token.                                      */
/* out[0] = n accepted drafts; out[1..n+1] = emitted tokens.           */
/* ------------------------------------------------------------------ */
void or_accept_greedy(const int64_t *top, const int32_t *drafts, int32_t K, int32_t *out) {
    int32_t n = 0;
    while (n < K && drafts[n] == top[n]) {
        out[1 + n] = drafts[n];
        n++;
    }
    out[1 + n] = (int32_t)top[n];
    out[0] = n;
}

/* ------------------------------------------------------------------ */
/* Rejection acceptance, fp64.                                          */
/*   p_i = softmax(z_i / temperature); e_ij = exp((z_ij - max_i)/T),    */
/*   S_i = sum_j e_ij (sequential), p_ij = e_ij / S_i.                  */
/* General drafter (q != NULL, q[K][V]): accept x_i iff                 */
/*   u[i][0] * q_i(x_i) < p_i(x_i)   (u < min(1, p/q) without division);*/
/*   on rejection r_j = max(0, p_ij - q_ij), R = sum r, emit the        */
/*   smallest j with cumsum_j(r) > u[i][1] * R, and stop.  If R == 0     */
/*   (possible only through rounding) sample from p_i instead.  If all  */
/*   K are accepted, the bonus is the smallest j with                   */
/*   cumsum_j(e_K) > u[K][1] * S_K.                                     */
/* Certain drafter (q == NULL): for i = 0..K, t_i = smallest j with     */
/*   cumsum_j(e_i) > u[i][0] * S_i; if i < K and t_i == x_i accept and   */
/*   go on, else emit t_i and stop.  One uniform per emitted token, in  */
/*   order, so the tokens equal plain sampling with the same uniforms.  */
/* margin (may be NULL, [K+1]) receives, for each decision taken, its   */
/* distance to the decision boundary relative to the scale it was taken */
/* at; a value below ~1e-10 means another summation order could flip it.*/
/* ------------------------------------------------------------------ */
static int64_t inv_cdf(const double *w, int64_t V, double thr, double *margin) {
    double c = 0.0;
    for (int64_t j = 0; j < V; j++) {
        double prev = c;
        c += w[j];
        if (c > thr) {
            if (margin) {
                double a = fabs(c - thr), b = fabs(thr - prev);
                *margin = (a < b ? a : b);
            }
            return j;
        }
    }
    /* thr >= total: only reachable through rounding; take the last
     * index with nonzero weight. */
    for (int64_t j = V - 1; j >= 0; j--)
        if (w[j] > 0.0) {
            if (margin) *margin = 0.0;
            return j;
        }
    if (margin) *margin = 0.0;
    return 0;
}

int or_accept_rejection(const float *logits, int64_t V, const float *q, const int32_t *drafts,
                        int32_t K, const double *u, double temperature, int32_t *out,
                        double *margin) {
    if (!(temperature > 0.0)) return -1;
    double *e = (double *)malloc(sizeof(double) * V);
    double *r = (double *)malloc(sizeof(double) * V);
    int32_t n = 0;
    int done = 0;
    for (int32_t i = 0; i <= K && !done; i++) {
        const float *z = logits + (int64_t)i * V;
        double zmax = -INFINITY;
        for (int64_t j = 0; j < V; j++)
            if ((double)z[j] > zmax) zmax = z[j];
        double S = 0.0;
        for (int64_t j = 0; j < V; j++) {
            e[j] = exp(((double)z[j] - zmax) / temperature);
            S += e[j];
        }
        double mg = 0.0;
        if (q == NULL) {
            int64_t t = inv_cdf(e, V, u[2 * i] * S, &mg);
            if (margin) margin[i] = mg / S;
            if (i < K && t == drafts[i]) {
                out[1 + n++] = drafts[i];
                continue;
            }
            out[1 + n] = (int32_t)t;
            done = 1;
        } else if (i < K) {
            const float *qi = q + (int64_t)i * V;
            int32_t x = drafts[i];
            double px = e[x] / S;
            double lhs = u[2 * i] * (double)qi[x];
            if (lhs < px) {
                if (margin) margin[i] = fabs(px - lhs) / (px > lhs ? px : lhs);
                out[1 + n++] = x;
                continue;
            }
            double R = 0.0;
            for (int64_t j = 0; j < V; j++) {
                double d = e[j] / S - (double)qi[j];
                r[j] = d > 0.0 ? d : 0.0;
                R += r[j];
            }
            double accm = (px == lhs) ? 0.0 : fabs(px - lhs) / (px > lhs ? px : lhs);
            int64_t t;
            if (R > 0.0) {
                t = inv_cdf(r, V, u[2 * i + 1] * R, &mg);
                mg /= R;
            } else {
                t = inv_cdf(e, V, u[2 * i + 1] * S, &mg);
                mg /= S;
            }
            if (margin) margin[i] = accm < mg ? accm : mg;
            out[1 + n] = (int32_t)t;
            done = 1;
        } else {
            int64_t t = inv_cdf(e, V, u[2 * i + 1] * S, &mg);
            if (margin) margin[i] = mg / S;
            out[1 + n] = (int32_t)t;
            done = 1;
        }
    }
    out[0] = n;
    free(e);
    free(r);
    return 0;
}
