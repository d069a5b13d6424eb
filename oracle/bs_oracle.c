/*
 * CPU oracle for the block-scaled low-precision linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or constant with
 * the HIP library; every number format is decoded here from its bit layout
 * and every sum is taken in fp64, in the order the definitions state.
 *
 * What it computes (sources are the five web pages bundled as the
 * reference; each function names the page and section it follows):
 *
 *   - per-token activation quantization to e4m3fn with one fp32 scale per
 *     row (the "(q_fp8, scale)" pairs of the sly-radiance README, fused
 *     norm/quant section; constants amax/448, round-to-nearest-even and
 *     saturation are the workload's own definition);
 *   - Y = dequant(A) . dequant(W)^T (+ bias) with e4m3 weights carrying one
 *     E8M0 scale per 32x32 block, row-major [N/32, K/32]
 *     (vLLM DeepSeek-V4 AMD mono runner page, AttnWeights: the fused
 *     q/kv projection's [2048, 7168] e4m3 weight carries a [64, 224] uint8
 *     E8M0 grid, one byte per 32x32 block);
 *   - the same with fp4 e2m1 weights packed two per byte and one E8M0 scale
 *     per row per 32 along K, [N, K/32] (same page, MonoLayerWeights.check:
 *     the routed experts' fp4x2 weights and their uint8 scale rows);
 *   - the optional bias / tanh-GELU epilogue (flash-rt groot_n17 frontend,
 *     module docstring: bias and bias+GELU fused into the FP8 GEMM epilogue;
 *     the tanh GELU is the cortiq vit.rs ACT_SRC shader, act == 2 branch).
 *
 * Parallelism: OpenMP over output elements; each output is computed by one
 * thread in one fixed order, so results are bit-identical for any thread
 * count (the cortiq dit.rs page makes the same argument for its row split).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>

#define OR_EPI_NONE 0
#define OR_EPI_BIAS 1
#define OR_EPI_BIAS_GELU_TANH 2

/* ---------------------------------------------------------------- codecs */

/* e4m3fn (OCP 8-bit float, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, NaN only at S.1111.111). The pages name the dtype
 * torch.float8_e4m3fn (vLLM DeepSeek-V4 mono runner, AttnWeights). */
double or_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);            /* subnormal: m/8 * 2^(1-7) */
    else
        mag = ldexp((double)(8 + m), e - 10);  /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* e2m1 (OCP 4-bit float: 2 exponent bits with bias 1, 1 mantissa bit, no
 * NaN or infinity). The dtype is torch.float4_e2m1fn_x2 on the mono runner
 * page (MonoLayerWeights.check). `c` is one nibble. */
double or_e2m1_value(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double mag = (e == 0) ? 0.5 * m                        /* m/2 * 2^(1-1) */
                          : ldexp((double)(2 + m), e - 2); /* (1 + m/2) * 2^(e-1) */
    return s ? -mag : mag;
}

/* E8M0: an unsigned biased exponent, value 2^(s-127); 255 encodes NaN. */
double or_e8m0_value(uint8_t s)
{
    if (s == 255)
        return NAN;
    return ldexp(1.0, (int)s - 127);
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double or_bf16_value(uint16_t b)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)b << 16;
    return (double)v.f;
}

/* Round a real number held exactly in a double to the nearest binary32
 * (the C cast rounds to nearest-even). */
static float to_f32(double x) { return (float)x; }

/* Nearest e4m3fn code to `v`, ties to the code with the even mantissa bit,
 * magnitudes above the largest finite value (448) saturate to it, and the
 * sign of v (also of -0 and of negatives that round to zero) goes to bit 7.
 * The search walks the 127 non-negative finite codes, which are increasing
 * in value, and decides between the two neighbours of |v| by comparing |v|
 * with their midpoint, which is exact in fp64 (both neighbours have 4-bit
 * significands). `v` must be finite. */
uint8_t or_e4m3_encode(double v)
{
    double a = fabs(v);
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    uint8_t lo, code;
    double mid;
    if (a >= 448.0)
        return sign | 0x7E;
    lo = 0;
    while (lo < 0x7E && or_e4m3_value((uint8_t)(lo + 1)) <= a)
        ++lo;
    /* now value(lo) <= a < value(lo + 1) and lo < 0x7E */
    mid = 0.5 * (or_e4m3_value(lo) + or_e4m3_value((uint8_t)(lo + 1)));
    if (a < mid)
        code = lo;
    else if (a > mid)
        code = (uint8_t)(lo + 1);
    else
        code = (lo & 1) ? (uint8_t)(lo + 1) : lo;
    return sign | code;
}

/* Nearest e2m1 code (nibble) with the same rules; saturates at 6. */
uint8_t or_e2m1_encode(double v)
{
    double a = fabs(v);
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    uint8_t lo, code;
    double mid;
    if (a >= 6.0)
        return sign | 0x7;
    lo = 0;
    while (lo < 0x7 && or_e2m1_value((uint8_t)(lo + 1)) <= a)
        ++lo;
    mid = 0.5 * (or_e2m1_value(lo) + or_e2m1_value((uint8_t)(lo + 1)));
    if (a < mid)
        code = lo;
    else if (a > mid)
        code = (uint8_t)(lo + 1);
    else
        code = (lo & 1) ? (uint8_t)(lo + 1) : lo;
    return sign | code;
}

/* ------------------------------------------------------------ quantizer */

/* Per-token quantization of bf16 activations [M, K] (row stride ldx
 * elements) to e4m3fn codes [M, K] (row stride ldq bytes) and one fp32
 * scale per row, the "(q_fp8, scale)" pair the sly-radiance README's fused
 * producers hand to its W4A8 GEMM (fused norm/quant rows of its table):
 *     amax  = max_k |x[m,k]|
 *     s[m]  = fl32(amax / 448)
 *     q     = enc(fl32(x / s[m]))           (enc: nearest, ties even, saturate)
 * A row of zeros gets s = 0 and signed-zero codes. Dividing two binary32
 * values in fp64 and rounding the quotient to binary32 gives the correctly
 * rounded binary32 quotient (53 >= 2*24 + 2). */
void or_quant_rows(const uint16_t *x, int64_t ldx, int64_t M, int64_t K,
                   uint8_t *q, int64_t ldq, float *s)
{
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * ldx;
        uint8_t *qr = q + m * ldq;
        double amax = 0.0;
        float sc;
        int64_t k;
        for (k = 0; k < K; ++k) {
            double a = fabs(or_bf16_value(xr[k]));
            if (a > amax)
                amax = a;
        }
        sc = to_f32(amax / 448.0);
        s[m] = sc;
        for (k = 0; k < K; ++k) {
            double xv = or_bf16_value(xr[k]);
            if (sc == 0.0f)
                qr[k] = signbit(xv) ? 0x80 : 0x00;
            else
                qr[k] = or_e4m3_encode((double)to_f32(xv / (double)sc));
        }
    }
}

/* Quantization with a given (static, per-tensor) scale, the flash-rt
 * groot_n17 frontend's calibrated activation scales (its host "alphas" are
 * act_scale x w_scale): q = enc(fl32(x / s)) for every element, s > 0
 * finite. Values beyond 448 s saturate. */
void or_quant_rows_static(const uint16_t *x, int64_t ldx, int64_t M, int64_t K, float sc,
                          uint8_t *q, int64_t ldq)
{
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t k;
        for (k = 0; k < K; ++k)
            q[m * ldq + k] = or_e4m3_encode((double)to_f32(or_bf16_value(x[m * ldx + k]) / (double)sc));
    }
}

/* ------------------------------------------------------ fused producers */

/* Nearest bfloat16 to a real number held exactly in a double, as bits:
 * ties to the even significand, magnitudes that round past the largest
 * finite value become infinity, the sign is kept (also for zero results).
 * bfloat16 has binary32's exponent range and 8 significand bits, so its
 * spacing is 2^(e-7) in the binade [2^e, 2^(e+1)) for e >= -126 and 2^-133
 * below 2^-126. |v| / spacing is exact in fp64 (a power-of-two scaling),
 * rint() rounds it to the nearest integer with ties to even, and the
 * rounded value times the spacing is a bfloat16 value (or 2^128), which
 * the binary32 cast holds exactly. `v` must be finite. */
static uint16_t bf16_round(double v)
{
    union { float f; uint32_t u; } c;
    double a = fabs(v), ulp, r;
    if (a == 0.0) {
        ulp = 1.0;
    } else if (a < ldexp(1.0, -126)) {
        ulp = ldexp(1.0, -133);
    } else {
        int e2;
        frexp(a, &e2);                 /* a = f * 2^e2, f in [0.5, 1) */
        ulp = ldexp(1.0, (e2 - 1) - 7);
    }
    r = rint(a / ulp) * ulp;
    c.f = r >= ldexp(1.0, 128) ? INFINITY : (float)r;
    return (uint16_t)((c.u >> 16) | (signbit(v) ? 0x8000u : 0u));
}

uint16_t or_bf16_round(double v) { return bf16_round(v); }

/* RMSNorm with an optional residual add in front, the input side of the
 * sly-radiance README's fused add_rms_quant producer (fused norm/quant rows
 * of its file table: the new residual and the "(q_fp8, scale)" pair come
 * out of one kernel). Per row m, with bf16 inputs x, res and weight w:
 *     r[k]  = bf16(x[k] + res[k])          (r = x when res is NULL)
 *     ms    = (sum_k r[k]^2) / K            fp64, summed in k order
 *     inv   = 1 / sqrt(ms + eps)            fp64
 *     h[k]  = bf16(fl32(fl32(r[k] * inv) * w[k]))
 *     (q, s) = the per-token quantizer applied to the row h.
 * The norm is the cortiq dit.rs page's rms_norm (mean of squares and the
 * reciprocal root in fp64, the normalized value rounded to fp32, then the
 * fp32 weight multiply); h is rounded to bf16 as the unfused chain's norm
 * output would be before the quantizer reads it. The sum x + res of two
 * bf16 values is exact in fp64. Outputs: r into res_out (when res is
 * given), h into h_out, codes and scales as or_quant_rows. */
void or_add_rms_norm_quant(const uint16_t *x, int64_t ldx, const uint16_t *res, int64_t ldr,
                           const uint16_t *w, double eps, int64_t M, int64_t K,
                           uint16_t *res_out, int64_t ldro, uint16_t *h_out, int64_t ldh,
                           uint8_t *q, int64_t ldq, float *s)
{
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * ldx;
        uint16_t *hr = h_out + m * ldh;
        double ss = 0.0, inv;
        int64_t k;
        for (k = 0; k < K; ++k) {
            double r = or_bf16_value(xr[k]);
            if (res) {
                uint16_t rb = bf16_round(r + or_bf16_value(res[m * ldr + k]));
                res_out[m * ldro + k] = rb;
                r = or_bf16_value(rb);
            }
            ss += r * r;
        }
        inv = 1.0 / sqrt(ss / (double)K + eps);
        for (k = 0; k < K; ++k) {
            double r = or_bf16_value(res ? res_out[m * ldro + k] : xr[k]);
            float n32 = to_f32(r * inv);
            float h32 = n32 * (float)or_bf16_value(w[k]);     /* binary32 multiply */
            hr[k] = bf16_round((double)h32);
        }
    }
    or_quant_rows(h_out, ldh, M, K, q, ldq, s);
}

/* SiLU(gate) * up, the input side of the sly-radiance README's fused
 * silu_mul_quant producer (same rows of its table; the gated MLP's act_fn).
 * gu is [M, 2I] bf16 with the gate in columns [0, I) and up in [I, 2I).
 *     sg[k] = fl32(g / (1 + exp(-g)))      fp64 inside, g = gu[m, k]
 *     a[k]  = bf16(fl32(sg[k] * u))          u = gu[m, I + k], binary32 multiply
 *     (q, s) = the per-token quantizer applied to the row a.
 * silu and the gate-times-up product follow the cortiq dit.rs page's
 * silu() and SwiGLU loop (binary32 values); silu is evaluated in fp64 and
 * rounded once to binary32 (exp in fp64 is within an ulp on any platform,
 * where binary32 expf implementations differ). Outputs a into a_out and the
 * codes and scales as or_quant_rows. */
void or_silu_mul_quant(const uint16_t *gu, int64_t ldgu, int64_t M, int64_t I,
                       uint16_t *a_out, int64_t lda, uint8_t *q, int64_t ldq, float *s)
{
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t k;
        for (k = 0; k < I; ++k) {
            double g = or_bf16_value(gu[m * ldgu + k]);
            double u = or_bf16_value(gu[m * ldgu + I + k]);
            float sg = to_f32(g / (1.0 + exp(-g)));
            float a32 = sg * (float)u;                      /* binary32 multiply */
            a_out[m * lda + k] = bf16_round((double)a32);
        }
    }
    or_quant_rows(a_out, lda, M, I, q, ldq, s);
}

/* ------------------------------------------------------------- epilogue */

/* tanh-approximated GELU: 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))),
 * the act == 2 branch of the cortiq vit.rs bias/activation shader, taken
 * here in fp64 with sqrt(2/pi) at full precision and without the shader's
 * +-15 clamp on the tanh argument (tanh is +-1 to fp64 precision there). */
double or_gelu_tanh(double v)
{
    const double pi = acos(-1.0);
    const double c = sqrt(2.0 / pi);
    return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
}

static double epilogue(double pre, int epi)
{
    return epi == OR_EPI_BIAS_GELU_TANH ? or_gelu_tanh(pre) : pre;
}

/* ---------------------------------------------------------------- GEMMs */

/* One output of the block-scaled e4m3 GEMM Y = dequant(A) dequant(W)^T
 * (+ bias), the y = x . W^T linear layer (cortiq dit.rs, Proj::matmat doc
 * comment). `a` is one row of e4m3 codes [K], `w` one row of W [K], `ws`
 * that row's block-row of E8M0 scales [K/32] (the grid is [N/32, K/32]
 * with one scale per 32x32 block). In fp64:
 *   acc   = sum_kb 2^(ws[kb]-127) * sum_{k in block kb} a[k] w[k]
 *   pre   = a_scale * acc (+ bias)
 *   out   = pre, or GELU_tanh(pre)
 *   absum = a_scale * sum_kb 2^(ws[kb]-127) * sum_k |a[k] w[k]|           */
static void one_bs_fp8(const uint8_t *a, float a_scale, const uint8_t *w,
                       const uint8_t *ws, const uint16_t *bias_n, int epi,
                       int64_t K, double *out, double *absum)
{
    double acc = 0.0, abs_acc = 0.0, pre;
    int64_t kb, k;
    for (kb = 0; kb < K / 32; ++kb) {
        double blk = 0.0, blk_abs = 0.0, sc = or_e8m0_value(ws[kb]);
        for (k = kb * 32; k < kb * 32 + 32; ++k) {
            double p = or_e4m3_value(a[k]) * or_e4m3_value(w[k]);
            blk += p;
            blk_abs += fabs(p);
        }
        acc += sc * blk;
        abs_acc += sc * blk_abs;
    }
    pre = (double)a_scale * acc;
    if (epi >= OR_EPI_BIAS)
        pre += or_bf16_value(*bias_n);
    *out = epilogue(pre, epi);
    *absum = fabs((double)a_scale) * abs_acc;
}

/* One output of the MXFP4-weight GEMM (A8W4 on the mono runner page,
 * MonoLayerWeights.check): `w` is one row of fp4 e2m1 codes packed two per
 * byte [K/2], element k in byte k/2, low nibble for even k; `ws` is that
 * row's E8M0 scales [K/32], one per 32 consecutive k.
 *   w[k] = e2m1(nibble_k) * 2^(ws[k/32]-127); the rest as one_bs_fp8.     */
static void one_mxfp4(const uint8_t *a, float a_scale, const uint8_t *w,
                      const uint8_t *ws, const uint16_t *bias_n, int epi,
                      int64_t K, double *out, double *absum)
{
    double acc = 0.0, abs_acc = 0.0, pre;
    int64_t kb, k;
    for (kb = 0; kb < K / 32; ++kb) {
        double blk = 0.0, blk_abs = 0.0, sc = or_e8m0_value(ws[kb]);
        for (k = kb * 32; k < kb * 32 + 32; ++k) {
            uint8_t byte = w[k / 2];
            uint8_t nib = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
            double p = or_e4m3_value(a[k]) * or_e2m1_value(nib);
            blk += p;
            blk_abs += fabs(p);
        }
        acc += sc * blk;
        abs_acc += sc * blk_abs;
    }
    pre = (double)a_scale * acc;
    if (epi >= OR_EPI_BIAS)
        pre += or_bf16_value(*bias_n);
    *out = epilogue(pre, epi);
    *absum = fabs((double)a_scale) * abs_acc;
}

/* Whole GEMMs. A e4m3 [M, K] (row stride lda), a_scale fp32 [M],
 * W [N, K] e4m3 (row stride ldw) with WS [N/32, K/32], or W [N, K/2] fp4x2
 * (row stride ldw bytes) with WS [N, K/32]; bias bf16 [N] for epi >= 1.
 * out and absum are [M, N] row-major. K and N are multiples of 32. */
void or_gemm_bs_fp8(const uint8_t *a, int64_t lda, const float *a_scale,
                    const uint8_t *w, int64_t ldw, const uint8_t *ws,
                    const uint16_t *bias, int epi,
                    int64_t M, int64_t N, int64_t K,
                    double *out, double *absum)
{
    int64_t idx;
#pragma omp parallel for schedule(dynamic, 64)
    for (idx = 0; idx < M * N; ++idx) {
        int64_t m = idx / N, n = idx % N;
        one_bs_fp8(a + m * lda, a_scale[m], w + n * ldw, ws + (n / 32) * (K / 32),
                   bias ? bias + n : NULL, epi, K, out + idx, absum + idx);
    }
}

void or_gemm_mxfp4_w4a8(const uint8_t *a, int64_t lda, const float *a_scale,
                        const uint8_t *w, int64_t ldw, const uint8_t *ws,
                        const uint16_t *bias, int epi,
                        int64_t M, int64_t N, int64_t K,
                        double *out, double *absum)
{
    int64_t idx;
#pragma omp parallel for schedule(dynamic, 64)
    for (idx = 0; idx < M * N; ++idx) {
        int64_t m = idx / N, n = idx % N;
        one_mxfp4(a + m * lda, a_scale[m], w + n * ldw, ws + n * (K / 32),
                  bias ? bias + n : NULL, epi, K, out + idx, absum + idx);
    }
}

/* One output of the MXFP4 x MXFP4 GEMM (W4A4): activations and weights both
 * fp4 e2m1 packed two per byte with one E8M0 scale per row per 32 along K
 * (sly-radiance README: MXFP4 W4A4 is the base path its W4A8 kernel takes
 * over from; the per-32 scale rule is OCP MX's, as for the weights). In fp64:
 *   acc   = sum_kb 2^(sa[kb]-127) 2^(sw[kb]-127) sum_{k in block kb} a[k] w[k]
 *   pre   = acc (+ bias); out = pre or GELU_tanh(pre)
 *   absum = sum_kb 2^(sa[kb]-127) 2^(sw[kb]-127) sum_k |a[k] w[k]|         */
static double e2m1_at(const uint8_t *packed, int64_t k)
{
    uint8_t byte = packed[k / 2];
    return or_e2m1_value((k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15));
}

static void one_w4a4(const uint8_t *a, const uint8_t *as, const uint8_t *w, const uint8_t *ws,
                     const uint16_t *bias_n, int epi, int64_t K, double *out, double *absum)
{
    double acc = 0.0, abs_acc = 0.0, pre;
    int64_t kb, k;
    for (kb = 0; kb < K / 32; ++kb) {
        double blk = 0.0, blk_abs = 0.0;
        double sc = or_e8m0_value(as[kb]) * or_e8m0_value(ws[kb]);
        for (k = kb * 32; k < kb * 32 + 32; ++k) {
            double p = e2m1_at(a, k) * e2m1_at(w, k);
            blk += p;
            blk_abs += fabs(p);
        }
        acc += sc * blk;
        abs_acc += sc * blk_abs;
    }
    pre = acc;
    if (epi >= OR_EPI_BIAS)
        pre += or_bf16_value(*bias_n);
    *out = epilogue(pre, epi);
    *absum = abs_acc;
}

void or_gemm_mxfp4_w4a4(const uint8_t *a, int64_t lda, const uint8_t *a_scale,
                        const uint8_t *w, int64_t ldw, const uint8_t *ws,
                        const uint16_t *bias, int epi, int64_t M, int64_t N, int64_t K,
                        double *out, double *absum)
{
    int64_t idx;
#pragma omp parallel for schedule(dynamic, 64)
    for (idx = 0; idx < M * N; ++idx) {
        int64_t m = idx / N, n = idx % N;
        one_w4a4(a + m * lda, a_scale + m * (K / 32), w + n * ldw, ws + n * (K / 32),
                 bias ? bias + n : NULL, epi, K, out + idx, absum + idx);
    }
}

void or_gemm_mxfp4_w4a4_sampled(const uint8_t *a, int64_t lda, const uint8_t *a_scale,
                                const uint8_t *w, int64_t ldw, const uint8_t *ws,
                                const uint16_t *bias, int epi, int64_t K, int64_t count,
                                const int64_t *ms, const int64_t *ns, double *out, double *absum)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        one_w4a4(a + m * lda, a_scale + m * (K / 32), w + n * ldw, ws + n * (K / 32),
                 bias ? bias + n : NULL, epi, K, out + i, absum + i);
    }
}

/* Grouped (MoE) W4A8 GEMM: token rows grouped by expert, rows
 * [off[e], off[e+1]) of A use expert e's MXFP4 weights (mono runner page,
 * MonoLayerWeights.check: the routed experts' w13 [experts, 2 inter,
 * hidden / 2] fp4x2 with uint8 scales [experts * 2 inter, hidden / 32]).
 * For t in expert e's rows, n < N:
 *   y[t, n] = one_mxfp4(a[t], a_scale[t], W_e[n], S_e[n], bias_e[n])
 * W_e = w + e * w_estride (bytes), S_e = ws + e * N * (K / 32),
 * bias_e = bias + e * N (or none). out/absum are [T, N]. */
void or_gemm_mxfp4_w4a8_grouped(const uint8_t *a, int64_t lda, const float *a_scale,
                                const int32_t *off, int64_t E,
                                const uint8_t *w, int64_t ldw, int64_t w_estride,
                                const uint8_t *ws, const uint16_t *bias, int epi,
                                int64_t T, int64_t N, int64_t K, double *out, double *absum)
{
    int64_t idx;
    (void)T;
#pragma omp parallel for schedule(dynamic, 64)
    for (idx = 0; idx < (int64_t)off[E] * N; ++idx) {
        int64_t t = idx / N, n = idx % N, e = 0;
        while (off[e + 1] <= t)
            ++e;
        one_mxfp4(a + t * lda, a_scale[t], w + e * w_estride + n * ldw,
                  ws + (e * N + n) * (K / 32), bias ? bias + e * N + n : NULL, epi, K,
                  out + idx, absum + idx);
    }
}

/* One output of the row-wise scaled e4m3 GEMM: per-token activation scale
 * times per-output-channel weight scale (sly-radiance README, lm_head row of
 * its file table: the head's weight quantized to fp8 per output channel and
 * run as a row-wise scaled GEMM with per-token fp8 activations). In fp64:
 *   acc   = sum_k a[k] w[k]
 *   pre   = a_scale * w_scale * acc (+ bias)
 *   out   = pre, or GELU_tanh(pre)
 *   absum = |a_scale * w_scale| * sum_k |a[k] w[k]|                        */
static void one_rowwise(const uint8_t *a, float a_scale, const uint8_t *w, float w_scale,
                        const uint16_t *bias_n, int epi, int64_t K, double *out, double *absum)
{
    double acc = 0.0, abs_acc = 0.0, pre;
    int64_t k;
    for (k = 0; k < K; ++k) {
        double p = or_e4m3_value(a[k]) * or_e4m3_value(w[k]);
        acc += p;
        abs_acc += fabs(p);
    }
    pre = (double)a_scale * (double)w_scale * acc;
    if (epi >= OR_EPI_BIAS)
        pre += or_bf16_value(*bias_n);
    *out = epilogue(pre, epi);
    *absum = fabs((double)a_scale * (double)w_scale) * abs_acc;
}

void or_gemm_fp8_rowwise(const uint8_t *a, int64_t lda, const float *a_scale,
                         const uint8_t *w, int64_t ldw, const float *w_scale,
                         const uint16_t *bias, int epi, int64_t M, int64_t N, int64_t K,
                         double *out, double *absum)
{
    int64_t idx;
#pragma omp parallel for schedule(dynamic, 64)
    for (idx = 0; idx < M * N; ++idx) {
        int64_t m = idx / N, n = idx % N;
        one_rowwise(a + m * lda, a_scale[m], w + n * ldw, w_scale[n], bias ? bias + n : NULL,
                    epi, K, out + idx, absum + idx);
    }
}

void or_gemm_fp8_rowwise_sampled(const uint8_t *a, int64_t lda, const float *a_scale,
                                 const uint8_t *w, int64_t ldw, const float *w_scale,
                                 const uint16_t *bias, int epi, int64_t K, int64_t count,
                                 const int64_t *ms, const int64_t *ns, double *out, double *absum)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        one_rowwise(a + m * lda, a_scale[m], w + n * ldw, w_scale[n], bias ? bias + n : NULL,
                    epi, K, out + i, absum + i);
    }
}

/* The same for a list of sampled outputs (ms[i], ns[i]), for problems too
 * large to evaluate whole; out and absum are [count]. */
void or_gemm_bs_fp8_sampled(const uint8_t *a, int64_t lda, const float *a_scale,
                            const uint8_t *w, int64_t ldw, const uint8_t *ws,
                            const uint16_t *bias, int epi, int64_t K,
                            int64_t count, const int64_t *ms, const int64_t *ns,
                            double *out, double *absum)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        one_bs_fp8(a + m * lda, a_scale[m], w + n * ldw, ws + (n / 32) * (K / 32),
                   bias ? bias + n : NULL, epi, K, out + i, absum + i);
    }
}

void or_gemm_mxfp4_w4a8_sampled(const uint8_t *a, int64_t lda, const float *a_scale,
                                const uint8_t *w, int64_t ldw, const uint8_t *ws,
                                const uint16_t *bias, int epi, int64_t K,
                                int64_t count, const int64_t *ms, const int64_t *ns,
                                double *out, double *absum)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        one_mxfp4(a + m * lda, a_scale[m], w + n * ldw, ws + n * (K / 32),
                  bias ? bias + n : NULL, epi, K, out + i, absum + i);
    }
}

/* --------------------------------------------------- weight preparation */

/* e4m3 weight codes from real values: one enc() per element (offline weight
 * preparation; the workloads draw weight values and encode them). */
void or_encode_e4m3(const float *v, int64_t count, uint8_t *q)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i)
        q[i] = or_e4m3_encode((double)v[i]);
}

/* MXFP4 weight quantization of real values [N, K] (row-major, K % 32 == 0)
 * by the OCP Microscaling v1.0 conversion, per group of 32 consecutive k:
 *   shared exponent X = floor(log2(amax)) - 2   (2 = e2m1's largest exponent)
 *   scale byte       = X + 127, clamped to [0, 254]
 *   element          = enc_e2m1(v / 2^(byte-127))   (nearest, ties even,
 *                                                    saturating at 6)
 * A group of zeros gets scale byte 0 and zero codes. Output: packed
 * [N, K/2] (low nibble = even k) and scales [N, K/32]. The sly-radiance
 * README's checkpoints are MXFP4 produced this way offline; the conversion
 * rule itself is the OCP specification's. */
void or_quant_mxfp4_weights(const float *v, int64_t N, int64_t K,
                            uint8_t *packed, uint8_t *scales)
{
    int64_t n, KB = K / 32;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        int64_t kb, k;
        for (kb = 0; kb < KB; ++kb) {
            const float *g = v + n * K + kb * 32;
            double amax = 0.0, unit;
            int X, byte;
            for (k = 0; k < 32; ++k)
                if (fabs((double)g[k]) > amax)
                    amax = fabs((double)g[k]);
            if (amax == 0.0) {
                byte = 0;
            } else {
                int e2;
                frexp(amax, &e2);          /* amax = f * 2^e2, f in [0.5, 1) */
                X = (e2 - 1) - 2;          /* floor(log2 amax) - emax(e2m1) */
                byte = X + 127;
                if (byte < 0) byte = 0;
                if (byte > 254) byte = 254;
            }
            scales[n * KB + kb] = (uint8_t)byte;
            unit = ldexp(1.0, byte - 127);
            for (k = 0; k < 32; k += 2) {
                uint8_t lo = or_e2m1_encode((double)g[k] / unit);
                uint8_t hi = or_e2m1_encode((double)g[k + 1] / unit);
                packed[n * (K / 2) + kb * 16 + k / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/* MXFP4 quantization of bf16 activation rows [M, K] (row stride ldx
 * elements): the OCP MX conversion above applied to each row's values
 * (bf16 values are exact in binary32). Output packed [M, K/2] (low nibble =
 * even k) and scales [M, K/32]. */
void or_quant_mxfp4_rows(const uint16_t *x, int64_t ldx, int64_t M, int64_t K,
                         uint8_t *packed, uint8_t *scales)
{
    int64_t m;
    for (m = 0; m < M; ++m) {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        int64_t k;
        for (k = 0; k < K; ++k)
            row[k] = (float)or_bf16_value(x[m * ldx + k]);
        or_quant_mxfp4_weights(row, 1, K, packed + m * (K / 2), scales + m * (K / 32));
        free(row);
    }
}

/* Threads the OpenMP runtime will use (for reporting). */
/* Threads of the parallel loops from now on (the benchmark's single-core
 * baseline); n >= 1. */
void or_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

int or_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
