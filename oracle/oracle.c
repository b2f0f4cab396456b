/*
 * CPU oracle for the batch-1 decode matrix-vector product y = W . x.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the GPU library, and the library
 * never loads it.
 *
 * What it computes (the pages describe the operation, not a formula):
 *  - MiniCPM-V 4.6 on Orange Pi AIPro (Ascend 310B) post, baseline paragraph:
 *    at decode M = 1, so every linear layer is a vector-matrix product; the
 *    closing paragraph says each step reads the FP16 weights once and is bound
 *    by memory bandwidth.  Here W is [N, K] row-major, x is [K], and
 *    y[n] = sum_k W[n,k] * x[k].
 *  - Same post, second change: the wide lm_head is cut into slices whose
 *    results are reduced.  A split of the k-sum changes only the summation
 *    order, so the oracle is the unsplit definition.
 *  - Same post, closing paragraph, and the vLLM Arm CPU optimisation post,
 *    "INT8 W8A8" and "INT8 W4A8" sections: 8-bit and 4-bit weights whose
 *    dequantisation is fused into the product.  The oracle dequantises
 *    explicitly, element by element, and forms the same sum.
 *  - EdgeFM summary, section 2C (speculative decoding): a verify block is M
 *    rows checked against the same W; each output row is the M = 1 product of
 *    its own activation row.
 *
 * Arithmetic: every fp16 value is decoded from its bit pattern to an exact
 * double; products of two fp16 values (at most 22 significant bits) and of a
 * 4-bit integer with an fp16 scale are exact in double; sums are taken in
 * increasing k in double.  The int8 product is summed exactly in int64.
 * Rows are independent, so the OpenMP split over rows leaves every result
 * bit-identical at any thread count.  Build: gcc -O2 -fopenmp
 * -ffp-contract=off (no fused multiply-add, no fast-math).
 *
 *  - Same MiniCPM-V post, second change, read with its host reduce: the
 *    next token is the argmax of the lm_head logits (orc_argmax_f32).
 *
 * Status codes: 0 ok, 1 an fp16 input is Inf or NaN, 2 bad shape,
 * 3 an int8 accumulator leaves the int32 range.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

#define ORC_OK 0
#define ORC_ERR_NONFINITE 1
#define ORC_ERR_SHAPE 2
#define ORC_ERR_RANGE 3

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent field 0 encodes the subnormals m * 2^-24; fields 1..30
 * encode (1024 + m) * 2^(e - 25); field 31 is Inf/NaN and is rejected. */
static int f16_value(uint16_t h, double *out)
{
    unsigned sign = h >> 15;
    unsigned e = (h >> 10) & 31u;
    unsigned m = h & 1023u;
    double v;
    if (e == 31u)
        return ORC_ERR_NONFINITE;
    if (e == 0u)
        v = ldexp((double)m, -24);
    else
        v = ldexp((double)(1024u + m), (int)e - 25);
    *out = sign ? -v : v;
    return ORC_OK;
}

/* Canonical int4 layout: element k of a row is the 4-bit field at bits
 * [4*(k%8), 4*(k%8)+3] of word k/8 of that row; q in 0..15. */
static int q4_canonical(const uint32_t *row_words, int64_t k)
{
    uint32_t word = row_words[k / 8];
    return (int)((word >> (4 * (k % 8))) & 15u);
}

static void note_error(int *shared, int code)
{
    if (code != ORC_OK) {
#pragma omp atomic write
        *shared = code;
    }
}

int orc_f16_decode(const uint16_t *h, int64_t n, double *out)
{
    int err = ORC_OK;
    for (int64_t i = 0; i < n; ++i) {
        int e = f16_value(h[i], &out[i]);
        if (e != ORC_OK)
            err = e;
    }
    return err;
}

/* y[n] = sum_k W[n,k] x[k];  A[n] = sum_k |W[n,k] x[k]| (for the tolerance). */
int orc_gemv_f16(const uint16_t *W, const uint16_t *x, int64_t N, int64_t K,
                 double *y, double *A)
{
    if (N < 0 || K < 0)
        return ORC_ERR_SHAPE;
    int err = ORC_OK;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!xd)
        return ORC_ERR_SHAPE;
    note_error(&err, orc_f16_decode(x, K, xd));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t *row = W + n * K;
        double s = 0.0, a = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double w;
            int e = f16_value(row[k], &w);
            if (e != ORC_OK)
                note_error(&err, e);
            double p = w * xd[k];
            s += p;
            a += fabs(p);
        }
        y[n] = s;
        if (A)
            A[n] = a;
    }
    free(xd);
    return err;
}

/* acc[n] = sum_k Wq[n,k] xq[k] exactly (int64, must fit int32);
 * y[n] = acc[n] * w_scale[n] * x_scale in double;
 * A[n] = w_scale[n] * x_scale * sum_k |Wq[n,k] xq[k]|. */
int orc_gemv_w8a8(const int8_t *Wq, const float *w_scale, const int8_t *xq,
                  float x_scale, int64_t N, int64_t K,
                  int32_t *acc, double *y, double *A)
{
    if (N < 0 || K < 0)
        return ORC_ERR_SHAPE;
    int err = ORC_OK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const int8_t *row = Wq + n * K;
        int64_t s = 0, a = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t p = (int64_t)row[k] * (int64_t)xq[k];
            s += p;
            a += p < 0 ? -p : p;
        }
        if (s > INT32_MAX || s < INT32_MIN)
            note_error(&err, ORC_ERR_RANGE);
        double scale = (double)w_scale[n] * (double)x_scale;
        if (acc)
            acc[n] = (int32_t)s;
        y[n] = (double)s * scale;
        if (A)
            A[n] = (double)a * fabs(scale);
    }
    return err;
}

/* Canonical int4 layout: element k of row n is the 4-bit field at bits
 * [4*(k%8), 4*(k%8)+3] of word Wc[n, k/8]; its value is q - 8 with q in 0..15
 * (zero-point 8), times the fp16 scale s4[n, k/group].
 * Y[m,n] = sum_k (q[n,k] - 8) * s4[n,k/group] * X[m,k];  A the matching sum
 * of magnitudes. */
int orc_gemv_w4a16(const uint32_t *Wc, const uint16_t *s4, const uint16_t *X,
                   int64_t M, int64_t N, int64_t K, int64_t group,
                   double *Y, double *A)
{
    if (M < 0 || N < 0 || K < 0 || group <= 0 || K % 8 || K % group)
        return ORC_ERR_SHAPE;
    int err = ORC_OK;
    int64_t words = K / 8, groups = K / group;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!xd)
        return ORC_ERR_SHAPE;
    note_error(&err, orc_f16_decode(X, M * K, xd));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int q = q4_canonical(Wc + n * words, k);
                double scale;
                int e = f16_value(s4[n * groups + k / group], &scale);
                if (e != ORC_OK)
                    note_error(&err, e);
                double w = (double)(q - 8) * scale;
                double p = w * xd[m * K + k];
                s += p;
                a += fabs(p);
            }
            Y[m * N + n] = s;
            if (A)
                A[m * N + n] = a;
        }
    }
    free(xd);
    return err;
}

/* Dynamic per-token activation quantisation for the 4-bit-weight x 8-bit-
 * activation product (vLLM Arm CPU optimisation post, INT8 W4A8 section:
 * 4-bit weights, 8-bit activations).  The pages fix no quantiser; the
 * reading used here is symmetric per token in fp32:
 *   amax = max_k |x_k|,  s_x = amax / 127  (fp32, round to nearest even),
 *   xq_k = clamp(rint(x_k / s_x), -127, 127)  (fp32 division, ties to even),
 *   and amax == 0 gives s_x = 0, xq = 0.
 * Every step is a single IEEE fp32 operation, so any IEEE implementation
 * that performs the same operations gets the same xq bit for bit. */
int orc_quantize_x_i8(const uint16_t *x, int64_t K, int8_t *xq, float *s_x)
{
    if (K < 0)
        return ORC_ERR_SHAPE;
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        double v;
        int e = f16_value(x[k], &v);
        if (e != ORC_OK)
            return e;
        float a = fabsf((float)v);          /* fp16 -> fp32 is exact */
        if (a > amax)
            amax = a;
    }
    volatile float s = amax / 127.0f;      /* volatile: keep exactly these fp32 operations */
    *s_x = s;
    for (int64_t k = 0; k < K; ++k) {
        double v;
        f16_value(x[k], &v);
        if (amax == 0.0f) {
            xq[k] = 0;
            continue;
        }
        volatile float t = (float)v / s;
        float r = rintf(t);
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        xq[k] = (int8_t)r;
    }
    return ORC_OK;
}

/* 4-bit weights (canonical words, zero-point 8, fp16 group scales as in
 * orc_gemv_w4a16) times 8-bit activations xq with scale s_x:
 *   y[n] = s_x * sum_k (q[n,k] - 8) * s4[n, k/group] * xq[k]   in double,
 *   A[n] = s_x * sum_k |(q[n,k] - 8) * s4[n, k/group] * xq[k]|. */
int orc_gemv_w4a8(const uint32_t *Wc, const uint16_t *s4, const int8_t *xq, float s_x,
                  int64_t N, int64_t K, int64_t group, double *y, double *A)
{
    if (N < 0 || K < 0 || group <= 0 || K % 8 || K % group)
        return ORC_ERR_SHAPE;
    int err = ORC_OK;
    int64_t words = K / 8, groups = K / group;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double s = 0.0, a = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            int q = q4_canonical(Wc + n * words, k);
            double scale;
            int e = f16_value(s4[n * groups + (k / group)], &scale);
            if (e != ORC_OK)
                note_error(&err, e);
            double p = (double)(q - 8) * scale * (double)xq[k];
            s += p;
            a += fabs(p);
        }
        y[n] = s * (double)s_x;
        if (A)
            A[n] = a * fabs((double)s_x);
    }
    return err;
}

/* One decode step of a causal depthwise 1-D convolution (MiniCPM-V 4.6 on
 * Orange Pi AIPro post, third change: the causal-conv1d of each decode step,
 * replaced there by a vectorised step kernel).  The page gives no formula;
 * the reading used here is the usual decode-time update of a short causal
 * convolution over each channel's last W inputs:
 *   window_c = (state[c][0], ..., state[c][W-2], x[c])   (oldest first)
 *   pre_c    = bias[c] + sum_j w[c][j] * window_c[j]
 *   out[c]   = silu ? pre_c / (1 + exp(-pre_c)) : pre_c
 *   state[c] <- (window_c[1], ..., window_c[W-1])        (x[c] appended)
 * x, state, bias and out are fp32, w is fp16 [C, W] (decoded exactly);
 * products and sums are exact or rounded once in fp64.  A[c] = |bias[c]| +
 * sum_j |w[c][j] * window_c[j]| is returned for the tolerance.
 * bias may be NULL (zero). */
int orc_causal_conv1d_step(const float *x, const uint16_t *w, const float *bias, float *state,
                           int64_t C, int64_t W, int silu, double *out, double *A)
{
    if (C < 0 || W < 2)
        return ORC_ERR_SHAPE;
    int err = ORC_OK;
    for (int64_t c = 0; c < C; ++c) {
        double pre = bias ? (double)bias[c] : 0.0;
        double a = fabs(pre);
        for (int64_t j = 0; j < W; ++j) {
            double wv;
            int e = f16_value(w[c * W + j], &wv);
            if (e != ORC_OK)
                err = e;
            double win = j < W - 1 ? (double)state[c * (W - 1) + j] : (double)x[c];
            pre += wv * win;
            a += fabs(wv * win);
        }
        for (int64_t j = 0; j + 1 < W - 1; ++j)
            state[c * (W - 1) + j] = state[c * (W - 1) + j + 1];
        state[c * (W - 1) + W - 2] = x[c];
        out[c] = silu ? pre / (1.0 + exp(-pre)) : pre;
        if (A)
            A[c] = a;
    }
    return err;
}

/* A decode step's linears feed each other through fp16 activations: the
 * output of one linear, rounded to fp16, is the input of a later one
 * (EdgeFM summary, section 2C: the decode iteration replayed as one
 * execution graph; the AIPro post's step is a sequence of such products).
 * orc_round_f16 rounds each double to the nearest IEEE binary16 value, ties
 * to the even significand, overflow to +-Inf, keeping subnormals; returns
 * the bit patterns.  NaN input is rejected. */
int orc_round_f16(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        double a = v[i];
        if (isnan(a))
            return ORC_ERR_NONFINITE;
        uint16_t sign = signbit(a) ? 0x8000u : 0u;
        a = fabs(a);
        /* the grid spacing at a: 2^(e - 10) for normals, 2^-24 below 2^-14 */
        int e;
        if (a < ldexp(1.0, -14))
            e = -14;
        else {
            frexp(a, &e);
            e -= 1;                                   /* a in [2^e, 2^(e+1)) */
        }
        double q = ldexp(a, 10 - e);                  /* significand in units of the grid */
        double r = nearbyint(q);                      /* default rounding: ties to even */
        double mag = ldexp(r, e - 10);
        uint16_t bits;
        if (mag >= 65520.0 || isinf(a))               /* 65504 + half a step rounds up to Inf */
            bits = 0x7C00u;
        else if (mag < ldexp(1.0, -14))               /* subnormal (or zero): m * 2^-24 */
            bits = (uint16_t)ldexp(mag, 24);
        else {
            int me;
            double f = frexp(mag, &me);               /* mag = f * 2^me, f in [0.5, 1) */
            uint16_t mant = (uint16_t)(ldexp(f, 11) - 1024.0);
            bits = (uint16_t)(((me - 1 + 15) << 10) | mant);
        }
        out[i] = (uint16_t)(sign | bits);
    }
    return ORC_OK;
}

/* Greedy decoding's token choice over the lm_head logits (MiniCPM-V 4.6 on
 * Orange Pi AIPro post, second change: the lm_head's sliced results are
 * reduced, there on the host, to pick the next token).  The token is the
 * index of the largest logit.  The pages fix no rule for ties or NaN; the
 * reading used here: values compare as IEEE numbers (so -0 equals +0), a NaN
 * is below every number, and among equal values (or among NaNs) the lowest
 * index wins.  n must be positive. */
int orc_argmax_f32(const float *y, int64_t n, int64_t *idx)
{
    if (n <= 0)
        return ORC_ERR_SHAPE;
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i) {
        if (isnan(y[i]))
            continue;
        if (isnan(y[best]) || y[i] > y[best])
            best = i;
    }
    *idx = best;
    return ORC_OK;
}

/* Top-k of the logits (the token choice of the same post's second change,
 * widened from the single largest logit to the k largest, as samplers that
 * draw from the best k candidates need).  The order is the greedy token's:
 * larger values first (IEEE comparison, so -0 equals +0), a NaN below every
 * number, and among equal values (or among NaNs) the lower index first.
 * idx receives the first k indices of all n indices sorted by that order. */
static const float *topk_values;

static int topk_before(int64_t a, int64_t b)
{
    const float va = topk_values[a], vb = topk_values[b];
    const int na = isnan(va), nb = isnan(vb);
    if (na != nb)
        return nb;                      /* the number comes before the NaN */
    if (!na && va != vb)
        return va > vb;
    return a < b;
}

static int topk_compare(const void *pa, const void *pb)
{
    const int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    if (a == b)
        return 0;
    return topk_before(a, b) ? -1 : 1;
}

int orc_topk_f32(const float *y, int64_t n, int64_t k, int64_t *idx)
{
    if (n <= 0 || k <= 0 || k > n)
        return ORC_ERR_SHAPE;
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!order)
        return ORC_ERR_SHAPE;
    for (int64_t i = 0; i < n; ++i)
        order[i] = i;
    topk_values = y;
    qsort(order, (size_t)n, sizeof(int64_t), topk_compare);
    for (int64_t i = 0; i < k; ++i)
        idx[i] = order[i];
    free(order);
    return ORC_OK;
}

void orc_set_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
}

int orc_max_threads(void)
{
    return omp_get_max_threads();
}
