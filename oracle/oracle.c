/*
 * CPU fp64 oracle for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the GPU library: it is a plain, slow, obviously correct statement
 * of what the fused kernel must compute.
 *
 * Definition followed (MUSA SDK guide "FlashAttention optimization", section
 * "Problems of standard self-attention": the attention formula and the
 * three-step standard implementation; the same three steps open the pwwt.cn
 * Triton tutorial, section 1):
 *
 *   S = scale * Q K^T              (one N-vector of scores per query row)
 *   P = softmax(S) row by row      (the safe form that subtracts the row max,
 *                                   MUSA guide "online softmax numerical
 *                                   stability"; tutorial section 2.3)
 *   O = P V
 *   LSE = m + ln(sum_j exp(s_j - m))   natural log of the row's partition sum
 *
 * A second entry point runs the blockwise online-softmax recurrences (MUSA
 * guide, "online softmax core idea" recurrences and the FlashAttention formula
 * steps 1-4, a-f) for one head, recording the running max m and running sum l
 * after every key block.  Tests use it only to show that the recurrences reach
 * the three-step result.
 *
 * A third entry point, oracle_attention_bwd, gives the gradients of O with respect
 * to Q, K and V (the backward pass, by the chain rule; see its comment).
 *
 * Inputs are the storage bits the GPU receives (fp32, IEEE binary16 or
 * bfloat16), widened exactly to double.  All arithmetic is double.
 * Parity pins: see tests/test_oracle.py (brute force, closed forms, library
 * routines, invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* storage dtype codes (same integer values the C boundary uses) */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* ---- exact widening of the storage formats to double ---------------------- */

static double widen_f16(uint16_t h)
{
    /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits */
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(f | 0x400), e - 25); /* (1.f) * 2^(e-15) */
    return sign ? -mag : mag;
}

static double widen_bf16(uint16_t b)
{
    /* bfloat16 is the upper half of a binary32 */
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

static double elem(const void *base, int dtype, int64_t idx)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[idx];
    case ORC_F16: return widen_f16(((const uint16_t *)base)[idx]);
    default: return widen_bf16(((const uint16_t *)base)[idx]);
    }
}

/* widen one head's [N, d] slice into a double buffer */
static void widen_head(const void *src, int dtype, int64_t head, int64_t N, int64_t d, double *dst)
{
    int64_t base = head * N * d;
    for (int64_t t = 0; t < N * d; ++t)
        dst[t] = elem(src, dtype, base + t);
}

/*
 * One query row through the three standard steps.
 *   qrow: d doubles; Kd, Vd: [N, d] doubles of the same head
 *   s_out: N doubles receiving the scaled scores (may be NULL)
 *   p_out: N doubles receiving the probabilities (must hold N doubles)
 *   o_out: d doubles; *lse_out: natural-log partition sum
 */
static void row_three_step(const double *qrow, const double *Kd, const double *Vd, int64_t N,
                           int64_t d, double scale, double *s_out, double *p_out, double *o_out,
                           double *lse_out)
{
    /* step 1: s_j = scale * <q, k_j> */
    for (int64_t j = 0; j < N; ++j) {
        const double *kr = Kd + j * d;
        double acc = 0.0;
        for (int64_t t = 0; t < d; ++t)
            acc += qrow[t] * kr[t];
        p_out[j] = scale * acc;
        if (s_out)
            s_out[j] = p_out[j];
    }
    /* step 2: safe softmax: m = max s, z = sum exp(s - m), p = exp(s - m) / z */
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j)
        if (p_out[j] > m)
            m = p_out[j];
    double z = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        p_out[j] = exp(p_out[j] - m);
        z += p_out[j];
    }
    for (int64_t j = 0; j < N; ++j)
        p_out[j] /= z;
    /* step 3: o = sum_j p_j v_j */
    for (int64_t t = 0; t < d; ++t)
        o_out[t] = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        const double *vr = Vd + j * d;
        double pj = p_out[j];
        for (int64_t t = 0; t < d; ++t)
            o_out[t] += pj * vr[t];
    }
    *lse_out = m + log(z);
}

static int check_common(const void *q, const void *k, const void *v, int dtype, int64_t B,
                        int64_t H, int64_t N, int64_t d)
{
    if (!q || !k || !v)
        return -1;
    if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16)
        return -2;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
        return -3;
    return 0;
}

/*
 * Attention forward for a set of query rows.
 *   q, k, v: storage bits, contiguous [B, H, N, d]
 *   rows:    global row indices r = (b*H + h)*N + i, ascending (NULL = every row)
 *   o:       [nrows, d] doubles;  lse: [nrows] doubles
 * Returns 0, or a negative code for invalid arguments.
 */
int oracle_attention(const void *q, const void *k, const void *v, int dtype, int64_t B,
                     int64_t H, int64_t N, int64_t d, double scale, const int64_t *rows,
                     int64_t nrows, double *o, double *lse)
{
    int rc = check_common(q, k, v, dtype, B, H, N, d);
    if (rc)
        return rc;
    int64_t total = B * H * N;
    if (!rows)
        nrows = total;
    if (nrows < 0 || !o || !lse)
        return -4;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t g = rows ? rows[r] : r;
        if (g < 0 || g >= total || (r > 0 && rows && rows[r] < rows[r - 1]))
            return -5;
    }
    double *Kd = (double *)malloc(sizeof(double) * N * d);
    double *Vd = (double *)malloc(sizeof(double) * N * d);
    if (!Kd || !Vd) {
        free(Kd);
        free(Vd);
        return -6;
    }
    int64_t r0 = 0;
    while (r0 < nrows) {
        int64_t head = (rows ? rows[r0] : r0) / N;
        int64_t r1 = r0;
        while (r1 < nrows && (rows ? rows[r1] : r1) / N == head)
            ++r1;
        /* widen this head's K and V once, then run its rows in parallel */
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < N; ++j) {
            for (int64_t t = 0; t < d; ++t) {
                Kd[j * d + t] = elem(k, dtype, (head * N + j) * d + t);
                Vd[j * d + t] = elem(v, dtype, (head * N + j) * d + t);
            }
        }
        int fail = 0;
#pragma omp parallel reduction(| : fail)
        {
            double *qrow = (double *)malloc(sizeof(double) * d);
            double *prow = (double *)malloc(sizeof(double) * N);
            if (!qrow || !prow)
                fail = 1;
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = r0; r < r1; ++r) {
                if (fail)
                    continue;
                int64_t g = rows ? rows[r] : r;
                for (int64_t t = 0; t < d; ++t)
                    qrow[t] = elem(q, dtype, g * d + t);
                row_three_step(qrow, Kd, Vd, N, d, scale, NULL, prow, o + r * d, lse + r);
            }
            free(qrow);
            free(prow);
        }
        if (fail) {
            free(Kd);
            free(Vd);
            return -6;
        }
        r0 = r1;
    }
    free(Kd);
    free(Vd);
    return 0;
}

/*
 * All three steps of one head, exposing S and P.  Small N only (N*N doubles).
 *   head: b*H + h;  s, p: [N, N];  o: [N, d];  lse: [N]
 */
int oracle_head_steps(const void *q, const void *k, const void *v, int dtype, int64_t B,
                      int64_t H, int64_t N, int64_t d, double scale, int64_t head, double *s,
                      double *p, double *o, double *lse)
{
    int rc = check_common(q, k, v, dtype, B, H, N, d);
    if (rc)
        return rc;
    if (head < 0 || head >= B * H || !s || !p || !o || !lse)
        return -4;
    double *Qd = (double *)malloc(sizeof(double) * N * d);
    double *Kd = (double *)malloc(sizeof(double) * N * d);
    double *Vd = (double *)malloc(sizeof(double) * N * d);
    if (!Qd || !Kd || !Vd) {
        free(Qd);
        free(Kd);
        free(Vd);
        return -6;
    }
    widen_head(q, dtype, head, N, d, Qd);
    widen_head(k, dtype, head, N, d, Kd);
    widen_head(v, dtype, head, N, d, Vd);
    for (int64_t i = 0; i < N; ++i)
        row_three_step(Qd + i * d, Kd, Vd, N, d, scale, s + i * N, p + i * N, o + i * d, lse + i);
    free(Qd);
    free(Kd);
    free(Vd);
    return 0;
}

/*
 * Blockwise online softmax for one head, in the order the FlashAttention
 * formula gives it.  For every query row i:
 *   m = -inf, l = 0, O = 0
 *   for each key block j (block keys; the last block may be shorter):
 *     S_ij  = scale * q_i K_j^T
 *     m_ij  = max(m, rowmax(S_ij))
 *     l     = exp(m - m_ij) * l + rowsum(exp(S_ij - m_ij))
 *     O     = exp(m - m_ij) * O + exp(S_ij - m_ij) V_j
 *     m     = m_ij
 *   O = O / l,  LSE = m + ln l
 * m_trace, l_trace: [N, nblocks] doubles receiving (m, l) after each block
 * (either may be NULL).
 */
int oracle_online_head(const void *q, const void *k, const void *v, int dtype, int64_t B,
                       int64_t H, int64_t N, int64_t d, double scale, int64_t head, int64_t block,
                       double *o, double *lse, double *m_trace, double *l_trace)
{
    int rc = check_common(q, k, v, dtype, B, H, N, d);
    if (rc)
        return rc;
    if (head < 0 || head >= B * H || block <= 0 || !o || !lse)
        return -4;
    int64_t nblocks = (N + block - 1) / block;
    double *Qd = (double *)malloc(sizeof(double) * N * d);
    double *Kd = (double *)malloc(sizeof(double) * N * d);
    double *Vd = (double *)malloc(sizeof(double) * N * d);
    double *sblk = (double *)malloc(sizeof(double) * block);
    if (!Qd || !Kd || !Vd || !sblk) {
        free(Qd);
        free(Kd);
        free(Vd);
        free(sblk);
        return -6;
    }
    widen_head(q, dtype, head, N, d, Qd);
    widen_head(k, dtype, head, N, d, Kd);
    widen_head(v, dtype, head, N, d, Vd);
    for (int64_t i = 0; i < N; ++i) {
        const double *qi = Qd + i * d;
        double *Oi = o + i * d;
        double m = -INFINITY, l = 0.0;
        for (int64_t t = 0; t < d; ++t)
            Oi[t] = 0.0;
        for (int64_t jb = 0; jb < nblocks; ++jb) {
            int64_t j0 = jb * block;
            int64_t nb = (j0 + block <= N) ? block : N - j0;
            double bmax = -INFINITY;
            for (int64_t u = 0; u < nb; ++u) {
                const double *kr = Kd + (j0 + u) * d;
                double acc = 0.0;
                for (int64_t t = 0; t < d; ++t)
                    acc += qi[t] * kr[t];
                sblk[u] = scale * acc;
                if (sblk[u] > bmax)
                    bmax = sblk[u];
            }
            double m_ij = m > bmax ? m : bmax;
            double alpha = exp(m - m_ij); /* exp(-inf) = 0 on the first block */
            double rowsum = 0.0;
            for (int64_t u = 0; u < nb; ++u)
                rowsum += exp(sblk[u] - m_ij);
            l = alpha * l + rowsum;
            for (int64_t t = 0; t < d; ++t)
                Oi[t] *= alpha;
            for (int64_t u = 0; u < nb; ++u) {
                double pu = exp(sblk[u] - m_ij);
                const double *vr = Vd + (j0 + u) * d;
                for (int64_t t = 0; t < d; ++t)
                    Oi[t] += pu * vr[t];
            }
            m = m_ij;
            if (m_trace)
                m_trace[i * nblocks + jb] = m;
            if (l_trace)
                l_trace[i * nblocks + jb] = l;
        }
        for (int64_t t = 0; t < d; ++t)
            Oi[t] /= l;
        lse[i] = m + log(l);
    }
    free(Qd);
    free(Kd);
    free(Vd);
    free(sblk);
    return 0;
}

/*
 * Attention backward: the gradients of O with respect to Q, K and V for an upstream
 * gradient dO.  The Triton tutorial (sections 2.4 and 4.4) states the method - P is not
 * kept; the backward pass recomputes it from the forward pass's inputs and statistics
 * and applies the chain rule - without writing the rule out.  Written out for
 * O = softmax(scale Q K^T) V (LSE is an auxiliary output and receives no gradient):
 *
 *   P     = softmax(scale Q K^T)                 row by row, the three standard steps
 *   dV    = P^T dO
 *   dP    = dO V^T
 *   dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)      the Jacobian of each row's softmax
 *   dQ    = scale dS K
 *   dK    = scale dS^T Q
 *
 *   dout:  float32 [B, H, N, d] (the gradient of the float32 output O)
 *   heads: indices b*H + h to compute, ascending (NULL = every head), nheads of them
 *   dq, dk, dv: doubles [nheads, N, d]
 * Returns 0, or a negative code for invalid arguments.  Cost B*H*N^2*d: small inputs,
 * or a few heads.
 */
int oracle_attention_bwd(const void *q, const void *k, const void *v, const float *dout,
                         int dtype, int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                         const int64_t *heads, int64_t nheads, double *dq, double *dk,
                         double *dv)
{
    int rc = check_common(q, k, v, dtype, B, H, N, d);
    if (rc)
        return rc;
    if (!heads)
        nheads = B * H;
    if (!dout || !dq || !dk || !dv || nheads < 0)
        return -4;
    for (int64_t x = 0; x < nheads; ++x) {
        int64_t hd = heads ? heads[x] : x;
        if (hd < 0 || hd >= B * H || (x > 0 && heads && heads[x] <= heads[x - 1]))
            return -5;
    }
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
    for (int64_t x = 0; x < nheads; ++x) {
        const int64_t head = heads ? heads[x] : x;
        double *Qd = (double *)malloc(sizeof(double) * N * d);
        double *Kd = (double *)malloc(sizeof(double) * N * d);
        double *Vd = (double *)malloc(sizeof(double) * N * d);
        double *dOd = (double *)malloc(sizeof(double) * N * d);
        double *prow = (double *)malloc(sizeof(double) * N);
        double *dprow = (double *)malloc(sizeof(double) * N);
        double *orow = (double *)malloc(sizeof(double) * d);
        if (!Qd || !Kd || !Vd || !dOd || !prow || !dprow || !orow) {
            fail = 1;
        } else {
            widen_head(q, dtype, head, N, d, Qd);
            widen_head(k, dtype, head, N, d, Kd);
            widen_head(v, dtype, head, N, d, Vd);
            for (int64_t t = 0; t < N * d; ++t)
                dOd[t] = (double)dout[head * N * d + t];
            double *dQh = dq + x * N * d, *dKh = dk + x * N * d, *dVh = dv + x * N * d;
            for (int64_t t = 0; t < N * d; ++t)
                dQh[t] = dKh[t] = dVh[t] = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                const double *qi = Qd + i * d, *gi = dOd + i * d;
                double lse;
                row_three_step(qi, Kd, Vd, N, d, scale, NULL, prow, orow, &lse); /* P row i */
                /* dP_ij = <dO_i, v_j> and the row term sum_k P_ik dP_ik */
                double Di = 0.0;
                for (int64_t j = 0; j < N; ++j) {
                    const double *vj = Vd + j * d;
                    double acc = 0.0;
                    for (int64_t t = 0; t < d; ++t)
                        acc += gi[t] * vj[t];
                    dprow[j] = acc;
                    Di += prow[j] * acc;
                }
                for (int64_t j = 0; j < N; ++j) {
                    const double ds = prow[j] * (dprow[j] - Di);
                    const double *kj = Kd + j * d;
                    double *dkj = dKh + j * d, *dvj = dVh + j * d;
                    for (int64_t t = 0; t < d; ++t) {
                        dQh[i * d + t] += scale * ds * kj[t];
                        dkj[t] += scale * ds * qi[t];
                        dvj[t] += prow[j] * gi[t];
                    }
                }
            }
        }
        free(Qd);
        free(Kd);
        free(Vd);
        free(dOd);
        free(prow);
        free(dprow);
        free(orow);
    }
    return fail ? -6 : 0;
}

/* number of OpenMP threads a parallel region of this library will use */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
