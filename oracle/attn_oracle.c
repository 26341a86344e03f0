/*
 * attn_oracle.c -- plain fp64 CPU reference for exact scaled-dot-product
 * attention.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark load it; the GPU library never does, and
 * this file shares no code with it.
 *
 * What it computes is the plain definition of attention, not the tiled
 * method: the pages describe FlashAttention as an exact algorithm that only
 * reorganises where the softmax(Q K^T * scale) V product is computed
 * («Что такое memory-efficient attention для long context на 8x H100?»,
 * section 2, "FlashAttention-3: IO-aware attention", and «Оптимизация
 * внимания Flash», "When to use alternatives": the speed-up comes without
 * loss of accuracy).  So the oracle materialises each query row's scores and
 * softmax weights in fp64 and never tiles, fuses or reorders anything.
 *
 * Definition followed, for every batch b, query head h and query row i
 * («Оптимизация внимания Flash», Workflow 1, Step 2 and Step 4: standard
 * attention is softmax(q k^T / sqrt(d_k)) v; Workflow 2, Steps 2-3: causal
 * flag, (left, right) sliding window, automatic scale, fewer K/V heads):
 *
 *   g      = h / (H / H_kv)                      K/V head shared by h
 *   V(i)   = { j : j <= i if causal;
 *                  i - j <= window and (causal or j - i <= window)
 *                  if window >= 0 }
 *   s_ij   = scale * sum_c q[b,h,i,c] * k[b,g,j,c]          (j in V(i))
 *   m_i    = max_j s_ij
 *   l_i    = sum_j exp(s_ij - m_i)
 *   O[i,:] = sum_j exp(s_ij - m_i) * v[b,g,j,:] / l_i
 *   lse_i  = m_i + ln(l_i)                        (natural-log logsumexp)
 *
 * Inputs are 16-bit float bit patterns (IEEE binary16 or bfloat16), or OCP
 * fp8 E4M3 patterns in the low byte of 16-bit words, decoded exactly to
 * double.  The scale is the fp32 value the GPU receives, widened.
 * Outputs are fp64 and are not rounded.
 *
 * Readings of points the pages leave open (each one also listed in the
 * design notes): layout [B,H,L,d] for q/out and [B,H_kv,L,d] for k/v; head
 * h reads K/V head h / (H/H_kv) (contiguous groups); the window is inclusive
 * on both sides with right = 0 when causal; scale <= 0 or NaN selects
 * 1/sqrt(d) rounded to fp32.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1, ORACLE_F8E4M3 = 2 };

/* IEEE-754 binary16: sign bit, 5-bit exponent with bias 15, 10-bit fraction.
 * Exponent 0 encodes zero/subnormals (fraction * 2^-24), exponent 31 encodes
 * infinities (fraction 0) and NaNs. */
double oracle_f16_to_f64(uint16_t bits)
{
    int sign = bits >> 15;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25); /* 1.frac * 2^(expo-15) */
    return sign ? -mag : mag;
}

/* bfloat16 is the upper 16 bits of an IEEE-754 binary32 value. */
double oracle_bf16_to_f64(uint16_t bits)
{
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn", the float8_e4m3fn type of «Оптимизация внимания
 * Flash», Workflow 3, Step 3): sign bit, 4-bit exponent with bias 7, 3-bit
 * fraction.  Exponent 0 encodes zero/subnormals (fraction * 2^-9); there are
 * no infinities, and S.1111.111 is NaN (the largest finite value is 448).
 * The byte is the low 8 bits of `bits`. */
double oracle_f8e4m3_to_f64(uint16_t bits)
{
    int sign = (bits >> 7) & 1;
    int expo = (bits >> 3) & 0xf;
    int frac = bits & 0x7;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -9);
    else if (expo == 15 && frac == 7)
        mag = NAN;
    else
        mag = ldexp((double)(8 + frac), expo - 10); /* 1.frac * 2^(expo-7) */
    return sign ? -mag : mag;
}

static double decode(uint16_t bits, int dtype)
{
    if (dtype == ORACLE_F8E4M3)
        return oracle_f8e4m3_to_f64(bits);
    return dtype == ORACLE_BF16 ? oracle_bf16_to_f64(bits) : oracle_f16_to_f64(bits);
}

void oracle_decode(const uint16_t *src, double *dst, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = decode(src[i], dtype);
}

/* The automatic scale 1/sqrt(d) («Оптимизация внимания Flash», Workflow 2,
 * Step 2: softmax_scale=None means auto-scale), as the fp32 nearest to it. */
float oracle_resolve_scale(float scale, int d)
{
    if (!(scale > 0.0f))
        return (float)(1.0 / sqrt((double)d));
    return scale;
}

/* Is key j visible from query i?  Causal: no key after the query.  Window:
 * at most `window` keys before the query and, when not causal, at most
 * `window` keys after it («Оптимизация внимания Flash», Workflow 2, Step 3,
 * sliding-window attention). */
int oracle_visible(int64_t i, int64_t j, int causal, int window)
{
    if (causal && j > i)
        return 0;
    if (window >= 0) {
        if (i - j > window)
            return 0;
        if (!causal && j - i > window)
            return 0;
    }
    return 1;
}

/* The K/V head read by query head h: query heads form H_kv contiguous groups
 * of H/H_kv heads, each sharing one K/V head («Оптимизация внимания Flash»,
 * Workflow 2, Step 3, multi-query attention with fewer K/V heads). */
int oracle_kv_head(int h, int H, int H_kv)
{
    return h / (H / H_kv);
}

/* Does flat query row r = (b*H + h)*L + i belong to batch `b` and read K/V
 * head `g`? */
static int reads_kv_head(int64_t r, int b, int g, int H, int H_kv, int L)
{
    int64_t bh = r / L;
    return bh / H == b && oracle_kv_head((int)(bh % H), H, H_kv) == g;
}

/* One query row i of the definition: its scores s_ij of the visible keys,
 * their maximum m, l = sum_j exp(s_ij - m), and acc = sum_j exp(s_ij - m) v_j
 * (so O_i = acc / l).  qd: the row's decoded q; kd, vd: the decoded K/V head.
 * If dod (the row's decoded upstream gradient) is not NULL, also
 * D = dO_i . O_i for the backward pass, and rho = sqrt(sum_c (dO_ic O_ic)^2),
 * the root-sum-square of D's terms.  If acc_abs is not NULL it receives
 * sum_j exp(s_ij - m) |v_jc| (the same weights, absolute values), and aux
 * (2 doubles) the number of visible keys and max_j scale * sum_c |q_c k_jc|.
 * Returns 0, or -2 if the row sees no key. */
static int row_softmax(const double *qd, const double *dod, const double *kd, const double *vd,
                       int64_t i, int L, int d, int causal, int window, double sc,
                       double *s, double *acc, double *m_out, double *l_out, double *D_out,
                       double *rho_out, double *acc_abs, double *aux)
{
    double m = -INFINITY, sabs = 0.0;
    int64_t count = 0;
    for (int64_t j = 0; j < L; ++j) {
        if (!oracle_visible(i, j, causal, window))
            continue;
        double dot = 0.0, dot_abs = 0.0;
        for (int c = 0; c < d; ++c) {
            dot += qd[c] * kd[j * d + c];
            dot_abs += fabs(qd[c] * kd[j * d + c]);
        }
        s[j] = sc * dot;
        if (s[j] > m)
            m = s[j];
        if (sc * dot_abs > sabs)
            sabs = sc * dot_abs;
        ++count;
    }
    if (count == 0)
        return -2;
    double l = 0.0;
    for (int c = 0; c < d; ++c) {
        acc[c] = 0.0;
        if (acc_abs)
            acc_abs[c] = 0.0;
    }
    for (int64_t j = 0; j < L; ++j) {
        if (!oracle_visible(i, j, causal, window))
            continue;
        double p = exp(s[j] - m);
        l += p;
        for (int c = 0; c < d; ++c) {
            acc[c] += p * vd[j * d + c];
            if (acc_abs)
                acc_abs[c] += p * fabs(vd[j * d + c]);
        }
    }
    *m_out = m;
    *l_out = l;
    if (aux) {
        aux[0] = (double)count;
        aux[1] = sabs;
    }
    if (dod) {
        double D = 0.0, R = 0.0;
        for (int c = 0; c < d; ++c) {
            D += dod[c] * (acc[c] / l);
            R += (dod[c] * (acc[c] / l)) * (dod[c] * (acc[c] / l));
        }
        *D_out = D;
        *rho_out = sqrt(R);
    }
    return 0;
}

/*
 * Exact attention for a set of query rows.
 *
 * q: [B,H,L,d], k and v: [B,H_kv,L,d], 16-bit patterns of `dtype`.
 * rows: flat row ids r = (b*H + h)*L + i, or NULL for all B*H*L rows in
 *   order (then n_rows is ignored).
 * out: [n_rows, d] fp64, lse: [n_rows] fp64 (row order of `rows`).
 * oabs: NULL, or [n_rows, d] fp64 receiving sum_j P_ij |v_jc| with P_ij the
 *   softmax weights of the row (what a relative error of each weight can move
 *   out[i,c] by, used by tests to bound 16-bit weight rounding).
 * row_aux: NULL, or [n_rows, 2] fp64 receiving, per row, the number of
 *   visible keys and max_j scale * sum_c |q_ic k_jc| (the size an absolute
 *   error of the score sums can reach).
 * threads <= 0 uses OpenMP's default.
 * Returns 0, or -1 for bad arguments, or -2 if a row has no visible key.
 */
int oracle_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype,
                int B, int H, int H_kv, int L, int d, int causal, int window,
                float scale, const int64_t *rows, int64_t n_rows, double *out,
                double *lse, double *oabs, double *row_aux, int threads)
{
    if (B < 0 || H <= 0 || H_kv <= 0 || L < 0 || d <= 0 || H % H_kv != 0 || window < -1)
        return -1;
    if (rows == NULL)
        n_rows = (int64_t)B * H * L;
    if (n_rows == 0)
        return 0;
    const double sc = (double)oracle_resolve_scale(scale, d);
    const int64_t head_elems = (int64_t)L * d;
    if (threads <= 0)
        threads = omp_get_max_threads();

    double *kd = malloc(sizeof(double) * (size_t)head_elems);
    double *vd = malloc(sizeof(double) * (size_t)head_elems);
    if (!kd || !vd) {
        free(kd);
        free(vd);
        return -1;
    }
    int status = 0;

    /* One K/V head at a time: decode it, then every requested row of every
     * query head that reads it. */
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < H_kv; ++g) {
            int64_t kv_base = ((int64_t)b * H_kv + g) * head_elems;
            int any = 0;
            for (int64_t t = 0; t < n_rows && !any; ++t)
                any = reads_kv_head(rows ? rows[t] : t, b, g, H, H_kv, L);
            if (!any)
                continue;
            oracle_decode(k + kv_base, kd, head_elems, dtype);
            oracle_decode(v + kv_base, vd, head_elems, dtype);

#pragma omp parallel num_threads(threads)
            {
                double *s = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
                double *qd = malloc(sizeof(double) * (size_t)d);
                double *acc = malloc(sizeof(double) * (size_t)d);
                double *acc_abs = malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 8)
                for (int64_t t = 0; t < n_rows; ++t) {
                    int64_t r = rows ? rows[t] : t;
                    if (!reads_kv_head(r, b, g, H, H_kv, L))
                        continue;
                    int64_t i = r % L;
                    oracle_decode(q + r * d, qd, d, dtype);

                    double m, l;
                    if (row_softmax(qd, NULL, kd, vd, i, L, d, causal, window, sc, s, acc, &m, &l,
                                    NULL, NULL, oabs ? acc_abs : NULL, row_aux ? row_aux + 2 * t : NULL) != 0) {
#pragma omp atomic write
                        status = -2;
                        continue;
                    }
                    for (int c = 0; c < d; ++c) {
                        out[t * d + c] = acc[c] / l;
                        if (oabs)
                            oabs[t * d + c] = acc_abs[c] / l;
                    }
                    lse[t] = m + log(l);
                }
                free(s);
                free(qd);
                free(acc);
                free(acc_abs);
            }
        }
    }
    free(kd);
    free(vd);
    return status;
}

/*
 * Gradients of exact attention: the backward pass.
 *
 * The pages recommend FlashAttention for training as well as inference
 * («Оптимизация внимания Flash», introduction) and list the backward pass as
 * unmeasured in their benchmark («ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Сравнить Hyena vs
 * FlashAttention на 128k», stage 5); they give no formula for it.  The
 * backward pass is therefore the gradient of the forward definition above:
 * for an upstream gradient dO of the output, with P_ij = exp(s_ij - m_i) / l_i
 * the softmax weight of a visible pair,
 *
 *   dv_j  = sum over query heads h reading g, and rows i that see j, of P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = dO_i . O_i                 (= sum_j P_ij dP_ij)
 *   dS_ij = P_ij (dP_ij - D_i)         (the softmax Jacobian applied to dP)
 *   dq_i  = scale * sum_j dS_ij k_j
 *   dk_j  = scale * sum over the same (h, i) of dS_ij q_i
 *
 * A K/V head receives the gradients of every query head that reads it.
 * Everything is fp64 from the exactly decoded 16-bit inputs; nothing is tiled
 * or reordered beyond recomputing a row's statistics where they are needed.
 */

/*
 * q, dout: [B,H,L,d]; k, v: [B,H_kv,L,d]; 16-bit patterns of `dtype`.
 * q_rows: flat ids (b*H + h)*L + i of the dq rows wanted, or NULL for all
 *   (then n_q_rows is ignored); dq: [n_q_rows, d].
 * kv_rows: flat ids (b*H_kv + g)*L + j of the dk/dv rows wanted, or NULL for
 *   all; dk, dv: [n_kv_rows, d].
 * dq_abs, dk_abs, dv_abs: NULL, or arrays shaped like dq, dk, dv that receive
 *   the sum of the absolute values of the terms whose sum is each gradient
 *   element (scale * sum_j |dS_ij k_j|, scale * sum |dS_ij q_i|,
 *   sum |P_ij dO_i|): the size a rounding error relative to each term can
 *   reach, used by tests to bound 16-bit arithmetic.
 * dq_dsens, dk_dsens: NULL, or arrays shaped like dq, dk that receive the
 *   sensitivity of each element to the row terms D: scale * rho_i *
 *   sum_j P_ij |k_j| and scale * sum_i P_ij rho_i |q_i|, with rho_i the
 *   root-sum-square of the terms of D_i.  If every D_i moves by at most
 *   eps * rho_i, dq and dk move by at most eps times these.
 * Returns 0, -1 for bad arguments or no memory, -2 if a row has no visible key.
 */
int oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                    int dtype, int B, int H, int H_kv, int L, int d, int causal, int window,
                    float scale, const int64_t *q_rows, int64_t n_q_rows, const int64_t *kv_rows,
                    int64_t n_kv_rows, double *dq, double *dk, double *dv, double *dq_abs,
                    double *dk_abs, double *dv_abs, double *dq_dsens, double *dk_dsens,
                    int threads)
{
    if (B < 0 || H <= 0 || H_kv <= 0 || L < 0 || d <= 0 || H % H_kv != 0 || window < -1)
        return -1;
    if (q_rows == NULL)
        n_q_rows = (int64_t)B * H * L;
    if (kv_rows == NULL)
        n_kv_rows = (int64_t)B * H_kv * L;
    if (n_q_rows == 0 && n_kv_rows == 0)
        return 0;
    const double sc = (double)oracle_resolve_scale(scale, d);
    const int group = H / H_kv;
    const int64_t head_elems = (int64_t)L * d;
    const int64_t group_rows = (int64_t)group * L;
    if (threads <= 0)
        threads = omp_get_max_threads();

    double *kd = malloc(sizeof(double) * (size_t)head_elems);
    double *vd = malloc(sizeof(double) * (size_t)head_elems);
    double *qd = malloc(sizeof(double) * (size_t)(group_rows * d));
    double *dod = malloc(sizeof(double) * (size_t)(group_rows * d));
    double *m = malloc(sizeof(double) * (size_t)group_rows);
    double *l = malloc(sizeof(double) * (size_t)group_rows);
    double *Dr = malloc(sizeof(double) * (size_t)group_rows);
    double *rho = malloc(sizeof(double) * (size_t)group_rows);
    char *needed = malloc((size_t)group_rows);
    int status = 0;
    if (!kd || !vd || !qd || !dod || !m || !l || !Dr || !rho || !needed)
        status = -1;

    for (int b = 0; b < B && status == 0; ++b) {
        for (int g = 0; g < H_kv && status == 0; ++g) {
            const int h0 = g * group;  /* first query head reading g */
            const int64_t kv_base = ((int64_t)b * H_kv + g) * L;

            /* which rows of this (b, g) are wanted */
            int any = 0;
            memset(needed, 0, (size_t)group_rows);
            for (int64_t t = 0; t < n_q_rows; ++t) {
                int64_t r = q_rows ? q_rows[t] : t;
                int64_t bh = r / L;
                if (bh / H == b && oracle_kv_head((int)(bh % H), H, H_kv) == g) {
                    needed[(bh % H - h0) * L + r % L] = 1;
                    any = 1;
                }
            }
            /* every row that sees a wanted key needs its statistics too */
            for (int64_t t = 0; t < n_kv_rows; ++t) {
                int64_t r = kv_rows ? kv_rows[t] : t;
                if (r / L != (int64_t)b * H_kv + g)
                    continue;
                any = 1;
                int64_t j = r % L;
                for (int hh = 0; hh < group; ++hh)
                    for (int64_t i = 0; i < L; ++i)
                        if (oracle_visible(i, j, causal, window))
                            needed[hh * L + i] = 1;
            }
            if (!any)
                continue;

            oracle_decode(k + kv_base * d, kd, head_elems, dtype);
            oracle_decode(v + kv_base * d, vd, head_elems, dtype);
            const int64_t q_base = ((int64_t)b * H + h0) * L;
            oracle_decode(q + q_base * d, qd, group_rows * d, dtype);
            oracle_decode(dout + q_base * d, dod, group_rows * d, dtype);

            /* 1. row statistics */
#pragma omp parallel num_threads(threads)
            {
                double *s = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
                double *acc = malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 8)
                for (int64_t r = 0; r < group_rows; ++r) {
                    if (!needed[r])
                        continue;
                    if (row_softmax(qd + r * d, dod + r * d, kd, vd, r % L, L, d, causal, window, sc,
                                  s, acc, &m[r], &l[r], &Dr[r], &rho[r], NULL, NULL) != 0) {
#pragma omp atomic write
                        status = -2;
                    }
                }
                free(s);
                free(acc);
            }
            if (status != 0)
                break;

            /* 2. dq_i = scale * sum_j dS_ij k_j */
#pragma omp parallel num_threads(threads)
            {
                double *acc = malloc(sizeof(double) * (size_t)d);
                double *acc_abs = malloc(sizeof(double) * (size_t)d);
                double *acc_P = malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 8)
                for (int64_t t = 0; t < n_q_rows; ++t) {
                    int64_t r = q_rows ? q_rows[t] : t;
                    int64_t bh = r / L;
                    if (bh / H != b || oracle_kv_head((int)(bh % H), H, H_kv) != g)
                        continue;
                    const int64_t gr = (bh % H - h0) * L + r % L;  /* row within the group */
                    const int64_t i = r % L;
                    const double *qi = qd + gr * d, *doi = dod + gr * d;
                    for (int c = 0; c < d; ++c)
                        acc[c] = acc_abs[c] = acc_P[c] = 0.0;
                    for (int64_t j = 0; j < L; ++j) {
                        if (!oracle_visible(i, j, causal, window))
                            continue;
                        double dot = 0.0, dP = 0.0;
                        for (int c = 0; c < d; ++c) {
                            dot += qi[c] * kd[j * d + c];
                            dP += doi[c] * vd[j * d + c];
                        }
                        double P = exp(sc * dot - m[gr]) / l[gr];
                        double dS = P * (dP - Dr[gr]);
                        for (int c = 0; c < d; ++c) {
                            acc[c] += dS * kd[j * d + c];
                            acc_abs[c] += fabs(dS * kd[j * d + c]);
                            acc_P[c] += P * fabs(kd[j * d + c]);
                        }
                    }
                    for (int c = 0; c < d; ++c) {
                        dq[t * d + c] = sc * acc[c];
                        if (dq_abs)
                            dq_abs[t * d + c] = sc * acc_abs[c];
                        if (dq_dsens)
                            dq_dsens[t * d + c] = sc * rho[gr] * acc_P[c];
                    }
                }
                free(acc);
                free(acc_abs);
                free(acc_P);
            }

            /* 3. dv_j = sum P_ij dO_i and dk_j = scale * sum dS_ij q_i over the
             *    group's query heads and the rows that see j */
#pragma omp parallel num_threads(threads)
            {
                double *ak = malloc(sizeof(double) * (size_t)d);
                double *av = malloc(sizeof(double) * (size_t)d);
                double *ak_abs = malloc(sizeof(double) * (size_t)d);
                double *av_abs = malloc(sizeof(double) * (size_t)d);
                double *ak_P = malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 8)
                for (int64_t t = 0; t < n_kv_rows; ++t) {
                    int64_t r = kv_rows ? kv_rows[t] : t;
                    if (r / L != (int64_t)b * H_kv + g)
                        continue;
                    const int64_t j = r % L;
                    const double *kj = kd + j * d, *vj = vd + j * d;
                    for (int c = 0; c < d; ++c)
                        ak[c] = av[c] = ak_abs[c] = av_abs[c] = ak_P[c] = 0.0;
                    for (int hh = 0; hh < group; ++hh) {
                        for (int64_t i = 0; i < L; ++i) {
                            if (!oracle_visible(i, j, causal, window))
                                continue;
                            const int64_t gr = hh * L + i;
                            const double *qi = qd + gr * d, *doi = dod + gr * d;
                            double dot = 0.0, dP = 0.0;
                            for (int c = 0; c < d; ++c) {
                                dot += qi[c] * kj[c];
                                dP += doi[c] * vj[c];
                            }
                            double P = exp(sc * dot - m[gr]) / l[gr];
                            double dS = P * (dP - Dr[gr]);
                            for (int c = 0; c < d; ++c) {
                                av[c] += P * doi[c];
                                ak[c] += dS * qi[c];
                                av_abs[c] += fabs(P * doi[c]);
                                ak_abs[c] += fabs(dS * qi[c]);
                                ak_P[c] += P * rho[gr] * fabs(qi[c]);
                            }
                        }
                    }
                    for (int c = 0; c < d; ++c) {
                        dv[t * d + c] = av[c];
                        dk[t * d + c] = sc * ak[c];
                        if (dk_abs) {
                            dv_abs[t * d + c] = av_abs[c];
                            dk_abs[t * d + c] = sc * ak_abs[c];
                        }
                        if (dk_dsens)
                            dk_dsens[t * d + c] = sc * ak_P[c];
                    }
                }
                free(ak);
                free(av);
                free(ak_abs);
                free(av_abs);
                free(ak_P);
            }
        }
    }
    free(kd);
    free(vd);
    free(qd);
    free(dod);
    free(m);
    free(l);
    free(Dr);
    free(rho);
    free(needed);
    return status;
}
