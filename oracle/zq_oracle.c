/*
 * zq_oracle.c -- plain, slow, obviously-correct CPU oracle for the fused
 * quantized linear layer of ZeroQuant.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the HIP library never calls it.
 *
 * Sources (web pages on ZeroQuant, arXiv 2206.01861):
 *   [SUM]  "ZeroQuant: Efficient and Affordable Post-Training Quantization for
 *          Large-Scale Transformers" -- long-form summary page (paper-graph-ui).
 *          Sections used: 3.4 "Group-wise Weight Quantization" (paper Sec. 4.1,
 *          Eq. (2)), 3.4 "Token-wise Activation Quantization" (paper Sec. 4.1),
 *          3.4 "Quantization-Optimized Transformer Kernels" (paper Sec. 4.3,
 *          App. D, Fig. 2).
 *
 * Precision: the quantizer decides integer codes, so it runs in fp32 exactly
 * as the kernel does (IEEE division, round-half-to-even).  LayerNorm
 * statistics and the dequantization epilogue run in fp64.  The integer GEMM
 * accumulates in int64 and reports whether any sum leaves the int32 range.
 *
 * Every function here has a pin in the CPU test suite (closed forms,
 * invariants, brute force, library routines); none is "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary64, written from the format's definition:     */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent field 0 */
/* holds subnormals with quantum 2^-24.  Conversion to binary16 rounds to    */
/* nearest, ties to even, in a single step.                                  */
/* ------------------------------------------------------------------------ */
double zqo_half_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);
    return sign ? -v : v;
}

uint16_t zqo_double_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    int e2;
    int ex;
    double quantum, n;
    if (isnan(v))
        return 0x7e00;
    if (isinf(v))
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    frexp(a, &e2);          /* a in [2^(e2-1), 2^e2) */
    ex = e2 - 1;            /* a in [2^ex, 2^(ex+1)) */
    if (ex < -14)
        ex = -14;           /* below the normal range the quantum stays 2^-24 */
    quantum = ldexp(1.0, ex - 10);
    n = rint(a / quantum);  /* division by a power of two is exact; RNE */
    if (ex == -14 && n < 1024.0)
        return sign | (uint16_t)n;  /* subnormal or zero */
    if (n == 2048.0) {              /* rounded up into the next binade */
        n = 1024.0;
        ex += 1;
    }
    if (ex > 15)
        return sign | 0x7c00;       /* overflow: infinity */
    return sign | (uint16_t)((ex + 15) << 10) | (uint16_t)(n - 1024.0);
}

void zqo_half_to_double_array(const uint16_t *h, size_t n, double *out)
{
    size_t i;
    for (i = 0; i < n; i++)
        out[i] = zqo_half_to_double(h[i]);
}

void zqo_double_to_half_array(const double *v, size_t n, uint16_t *out)
{
    size_t i;
    for (i = 0; i < n; i++)
        out[i] = zqo_double_to_half(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Symmetric uniform quantizer, [SUM] 3.4 "Group-wise Weight Quantization",  */
/* Eq. (2): x_q = round(clamp(x / S)), dequantized as x_q * S.  The pages     */
/* print S = max|x| and also say x/S is first normalised to [-1, 1] and then  */
/* scaled to the integer range; the plain reading that satisfies both is     */
/* S = max|x| / qmax with qmax = 2^(bit-1) - 1 (127 for 8 bits, 7 for 4).     */
/* The clamp bound is +-qmax (symmetric); |x/S| never exceeds qmax by more   */
/* than fp32 rounding, so the lower bound -2^(bit-1) of Eq. (2) is never hit. */
/* Rounding is to nearest with ties to even.  An all-zero unit gets S = 0    */
/* and all-zero codes.                                                        */
/* The unit is n contiguous fp16 values: one token row for activations, one  */
/* group of whole weight rows for weights.  Returns S.                        */
/* ------------------------------------------------------------------------ */
static void quantize_with_scale(const uint16_t *v, size_t n, float s, int qmax,
                                int8_t *q);

static float quantize_unit(const uint16_t *v, size_t n, int qmax, int8_t *q)
{
    float amax = 0.0f;
    float s;
    size_t i;
    for (i = 0; i < n; i++) {
        float a = fabsf((float)zqo_half_to_double(v[i]));
        if (a > amax)
            amax = a;
    }
    s = amax / (float)qmax;
    quantize_with_scale(v, n, s, qmax, q);
    return s;
}

/* Eq. (2) with a given scale S (the clamp applies to values beyond the     */
/* range S was taken from).                                                  */
static void quantize_with_scale(const uint16_t *v, size_t n, float s, int qmax,
                                int8_t *q)
{
    size_t i;
    for (i = 0; i < n; i++) {
        float x, r;
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        x = (float)zqo_half_to_double(v[i]) / s;  /* fp32 IEEE division */
        if (x > (float)qmax)
            x = (float)qmax;
        if (x < -(float)qmax)
            x = -(float)qmax;
        r = rintf(x);                              /* ties to even */
        q[i] = (int8_t)r;
    }
}

/* ------------------------------------------------------------------------ */
/* Group-wise weight quantization, [SUM] 3.4 "Group-wise Weight              */
/* Quantization" (paper Sec. 4.1): W[N][K] (row n = output channel, K        */
/* contiguous) is split into groups of G contiguous rows along the output    */
/* dimension; group g = rows [g*G, (g+1)*G) gets its own S_g.                 */
/* bits = 8 -> qmax 127; bits = 4 -> qmax 7.  Codes are written unpacked to  */
/* q[N][K] (int8) and scales to sw[N/G].  Returns 0, or -1 on bad arguments. */
/* ------------------------------------------------------------------------ */
int zqo_quantize_weights(const uint16_t *w, int N, int K, int G, int bits,
                         int8_t *q, float *sw)
{
    int g, qmax;
    if (N <= 0 || K <= 0 || G <= 0 || N % G != 0)
        return -1;
    if (bits == 8)
        qmax = 127;
    else if (bits == 4)
        qmax = 7;
    else
        return -1;
#pragma omp parallel for schedule(dynamic)
    for (g = 0; g < N / G; g++) {
        size_t off = (size_t)g * G * K;
        sw[g] = quantize_unit(w + off, (size_t)G * K, qmax, q + off);
    }
    return 0;
}

/* W4 storage: two's-complement nibbles, two per byte along K; the low      */
/* nibble holds the even k.  The pages describe no INT4 layout, so this one  */
/* is a stated convention.  K must be even.                                  */
void zqo_pack_w4(const int8_t *q, int N, int K, uint8_t *packed)
{
    int n, j;
    for (n = 0; n < N; n++)
        for (j = 0; j < K / 2; j++) {
            int lo = q[(size_t)n * K + 2 * j] & 0xF;
            int hi = q[(size_t)n * K + 2 * j + 1] & 0xF;
            packed[(size_t)n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
}

void zqo_unpack_w4(const uint8_t *packed, int N, int K, int8_t *q)
{
    int n, j;
    for (n = 0; n < N; n++)
        for (j = 0; j < K / 2; j++) {
            int b = packed[(size_t)n * (K / 2) + j];
            int lo = b & 0xF;
            int hi = (b >> 4) & 0xF;
            if (lo >= 8)
                lo -= 16;
            if (hi >= 8)
                hi -= 16;
            q[(size_t)n * K + 2 * j] = (int8_t)lo;
            q[(size_t)n * K + 2 * j + 1] = (int8_t)hi;
        }
}

/* ------------------------------------------------------------------------ */
/* LayerNorm producing the fp16 activation that the fused kernel quantizes,  */
/* [SUM] 3.4 "Quantization-Optimized Transformer Kernels" (paper App. D,     */
/* Fig. 2: X -> LN + Quantize -> GeMM + Dequantize).  The pages do not spell */
/* out LayerNorm; the plain definition is used: per token, mean and biased   */
/* variance over the K features, h = (x - mean) / sqrt(var + eps) * gamma +   */
/* beta, evaluated in fp64 and rounded once to fp16.  gamma / beta may be    */
/* NULL (1 and 0).                                                            */
/* ------------------------------------------------------------------------ */
void zqo_layernorm(const uint16_t *x, const uint16_t *gamma,
                   const uint16_t *beta, float eps, int M, int K, uint16_t *h)
{
    int t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < M; t++) {
        const uint16_t *row = x + (size_t)t * K;
        double mean = 0.0, var = 0.0, denom;
        int k;
        for (k = 0; k < K; k++)
            mean += zqo_half_to_double(row[k]);
        mean /= K;
        for (k = 0; k < K; k++) {
            double d = zqo_half_to_double(row[k]) - mean;
            var += d * d;
        }
        var /= K;
        denom = sqrt(var + (double)eps);
        for (k = 0; k < K; k++) {
            double g = gamma ? zqo_half_to_double(gamma[k]) : 1.0;
            double b = beta ? zqo_half_to_double(beta[k]) : 0.0;
            double v = (zqo_half_to_double(row[k]) - mean) / denom * g + b;
            h[(size_t)t * K + k] = zqo_double_to_half(v);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Token-wise dynamic activation quantization, [SUM] 3.4 "Token-wise         */
/* Activation Quantization" (paper Sec. 4.1): one scale per row of the      */
/* (batch*seqlen) x hidden activation, computed at run time from that row    */
/* alone, then Eq. (2) with qmax = 127.                                      */
/* ------------------------------------------------------------------------ */
void zqo_quant_tokens(const uint16_t *h, int M, int K, int8_t *q, float *sx)
{
    int t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < M; t++)
        sx[t] = quantize_unit(h + (size_t)t * K, (size_t)K, 127,
                              q + (size_t)t * K);
}

/* ------------------------------------------------------------------------ */
/* Static per-tensor activation quantization, the prior-PTQ scheme that      */
/* [SUM] 3.4 "Token-wise Activation Quantization" contrasts with token-wise  */
/* scales (paper App. B.1): the range is calibrated offline as a moving      */
/* average over calibration batches,                                          */
/*   x_max = m * x_max + (1 - m) * max(batch),  x_min likewise (m = 0.95),   */
/* and frozen; S = max(|x_min|, |x_max|), read as for the token scale with    */
/* qmax: S = max(|x_min|, |x_max|) / 127.  Readings where the pages are      */
/* silent: the first batch initializes (x_min, x_max); the state and the      */
/* update are fp32, each product and the sum rounded separately.             */
/* state = {x_min, x_max}; x is n fp16 values (one calibration batch).       */
/* ------------------------------------------------------------------------ */
void zqo_calibrate_minmax(const uint16_t *x, size_t n, float momentum,
                          int first, float *state)
{
    float mn = INFINITY, mx = -INFINITY;
    size_t i;
    for (i = 0; i < n; i++) {
        float v = (float)zqo_half_to_double(x[i]);
        if (v < mn)
            mn = v;
        if (v > mx)
            mx = v;
    }
    if (first) {
        state[0] = mn;
        state[1] = mx;
    } else {
        float w = 1.0f - momentum;
        float a0 = momentum * state[0], b0 = w * mn;
        float a1 = momentum * state[1], b1 = w * mx;
        state[0] = a0 + b0;
        state[1] = a1 + b1;
    }
}

/* Eq. (2) over the whole tensor with the frozen scale; returns S. */
float zqo_quant_static(const uint16_t *x, size_t n, const float *state,
                       int8_t *q)
{
    float s = fmaxf(fabsf(state[0]), fabsf(state[1])) / 127.0f;
    quantize_with_scale(x, n, s, 127, q);
    return s;
}

/* ------------------------------------------------------------------------ */
/* INT8 x INT8 GEMM with integer accumulation, [SUM] 3.4 "Quantization-      */
/* Optimized Transformer Kernels" (paper Sec. 4.3): acc[t][n] =              */
/* sum_k qx[t][k] * qw[n][k].  Summed in int64; returns the number of       */
/* results that do not fit int32 (0 means every acc is exact in int32).     */
/* ------------------------------------------------------------------------ */
long zqo_gemm_i32(const int8_t *qx, const int8_t *qw, int M, int N, int K,
                  int32_t *acc)
{
    long overflow = 0;
    long idx;
    long total = (long)M * N;
#pragma omp parallel for schedule(static) reduction(+ : overflow)
    for (idx = 0; idx < total; idx++) {
        int t = (int)(idx / N), n = (int)(idx % N);
        const int8_t *a = qx + (size_t)t * K;
        const int8_t *b = qw + (size_t)n * K;
        int64_t s = 0;
        int k;
        for (k = 0; k < K; k++)
            s += (int64_t)a[k] * (int64_t)b[k];
        if (s > INT32_MAX || s < INT32_MIN)
            overflow++;
        acc[idx] = (int32_t)s;
    }
    return overflow;
}

/* ------------------------------------------------------------------------ */
/* Dequantization epilogue, [SUM] 3.4 "Quantization-Optimized Transformer    */
/* Kernels" (paper App. D): each int32 result is turned back into a real    */
/* value with the scale of its token and the scale of its weight group,     */
/* then (plain reading of the fusion with bias-add and GeLU) the bias is    */
/* added and an optional exact-erf GeLU applied.  fp64 throughout; z is the */
/* unrounded value, y its fp16 rounding.  act: 0 = none, 1 = GeLU.          */
/* bias may be NULL.                                                         */
/* ------------------------------------------------------------------------ */
void zqo_epilogue(const int32_t *acc, const float *sx, const float *sw, int G,
                  const uint16_t *bias, int act, int M, int N, double *z,
                  uint16_t *y)
{
    long idx;
    long total = (long)M * N;
#pragma omp parallel for schedule(static)
    for (idx = 0; idx < total; idx++) {
        int t = (int)(idx / N), n = (int)(idx % N);
        double v = (double)acc[idx] * (double)sx[t] * (double)sw[n / G];
        if (bias)
            v += zqo_half_to_double(bias[n]);
        if (act == 1)
            v = 0.5 * v * (1.0 + erf(v / sqrt(2.0)));
        if (z)
            z[idx] = v;
        if (y)
            y[idx] = zqo_double_to_half(v);
    }
}

/* ------------------------------------------------------------------------ */
/* W8A16 linear: INT8 group-wise weights with FP16 activations, the mixed    */
/* scheme of [SUM] Sec. 5 "Experimental Analysis" (Table 4: W8A16, INT8      */
/* weights and FP16 activations; Table 8: GPT-NeoX20B keeps the             */
/* self-attention input activations in FP16 while its weights are INT8).    */
/* Plain definition: each                                                    */
/* weight is dequantized, w[n][k] = sw[n/G] * q[n][k], and                   */
/*   z[t][n] = act( sum_k x[t][k] * w[n][k] + bias[n] ),  y = fp16(z).       */
/* fp64 throughout (every product of a binary16 value and a dequantized      */
/* weight is exact in fp64).  act: 0 = none, 1 = exact-erf GeLU; bias may    */
/* be NULL.                                                                  */
/* ------------------------------------------------------------------------ */
void zqo_gemm_w8a16(const uint16_t *x, const int8_t *q, const float *sw, int G,
                    const uint16_t *bias, int act, int M, int N, int K,
                    double *z, uint16_t *y)
{
    long idx;
    long total = (long)M * N;
#pragma omp parallel for schedule(static)
    for (idx = 0; idx < total; idx++) {
        int t = (int)(idx / N), n = (int)(idx % N);
        const uint16_t *a = x + (size_t)t * K;
        const int8_t *b = q + (size_t)n * K;
        double s = 0.0;
        int k;
        for (k = 0; k < K; k++) {
            double w = (double)sw[n / G] * (double)b[k];
            s += zqo_half_to_double(a[k]) * w;
        }
        if (bias)
            s += zqo_half_to_double(bias[n]);
        if (act == 1)
            s = 0.5 * s * (1.0 + erf(s / sqrt(2.0)));
        if (z)
            z[idx] = s;
        if (y)
            y[idx] = zqo_double_to_half(s);
    }
}

/* Threads the OpenMP loops above use (reported with CPU timings). */
int zqo_threads(void)
{
    return omp_get_max_threads();
}

/* Sets the thread count of later OpenMP loops (CPU timings only; the
 * results do not depend on it: every loop writes disjoint outputs). */
void zqo_set_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : 1);
}
