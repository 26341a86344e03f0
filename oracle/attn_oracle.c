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
 * Inputs are 16-bit float bit patterns (IEEE binary16 or bfloat16), decoded
 * exactly to double.  The scale is the fp32 value the GPU receives, widened.
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

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

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

static double decode(uint16_t bits, int dtype)
{
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

/*
 * Exact attention for a set of query rows.
 *
 * q: [B,H,L,d], k and v: [B,H_kv,L,d], 16-bit patterns of `dtype`.
 * rows: flat row ids r = (b*H + h)*L + i, or NULL for all B*H*L rows in
 *   order (then n_rows is ignored).
 * out: [n_rows, d] fp64, lse: [n_rows] fp64 (row order of `rows`).
 * threads <= 0 uses OpenMP's default.
 * Returns 0, or -1 for bad arguments, or -2 if a row has no visible key.
 */
int oracle_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype,
                int B, int H, int H_kv, int L, int d, int causal, int window,
                float scale, const int64_t *rows, int64_t n_rows, double *out,
                double *lse, int threads)
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
#pragma omp for schedule(dynamic, 8)
                for (int64_t t = 0; t < n_rows; ++t) {
                    int64_t r = rows ? rows[t] : t;
                    if (!reads_kv_head(r, b, g, H, H_kv, L))
                        continue;
                    int64_t i = r % L;
                    oracle_decode(q + r * d, qd, d, dtype);

                    /* scores of the visible keys, and their maximum */
                    double m = -INFINITY;
                    int64_t count = 0;
                    for (int64_t j = 0; j < L; ++j) {
                        if (!oracle_visible(i, j, causal, window))
                            continue;
                        double dot = 0.0;
                        for (int c = 0; c < d; ++c)
                            dot += qd[c] * kd[j * d + c];
                        s[j] = sc * dot;
                        if (s[j] > m)
                            m = s[j];
                        ++count;
                    }
                    if (count == 0) {
#pragma omp atomic write
                        status = -2;
                        continue;
                    }

                    /* softmax weights, their sum, and the weighted sum of values */
                    double l = 0.0;
                    for (int c = 0; c < d; ++c)
                        acc[c] = 0.0;
                    for (int64_t j = 0; j < L; ++j) {
                        if (!oracle_visible(i, j, causal, window))
                            continue;
                        double p = exp(s[j] - m);
                        l += p;
                        for (int c = 0; c < d; ++c)
                            acc[c] += p * vd[j * d + c];
                    }
                    for (int c = 0; c < d; ++c)
                        out[t * d + c] = acc[c] / l;
                    lse[t] = m + log(l);
                }
                free(s);
                free(qd);
                free(acc);
            }
        }
    }
    free(kd);
    free(vd);
    return status;
}
