/*
 * CPU oracle for the fused residual-add + norm + projection path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Everything is computed in IEEE double precision with plain loops, in the
 * order the method states its steps, except where the pages fix the
 * precision: the normalised value that feeds the product is formed in single
 * precision from single-precision statistics, as the LayerNorm + QKV sketch
 * [D] declares them (R11), and then rounded to the activation dtype: a fused
 * kernel feeds the matrix unit in that dtype ("reading A").  The unrounded
 * double-precision normalised row is available too ("reading B",
 * rounded = 0).  Weights are used exactly as stored (int8 weights through
 * their documented dequantisation).
 *
 * Sources (web pages on TensorRT-LLM; cited by title and section):
 *  [D] "TensorRT-LLM 深度工程实践：从模型到生产级推理服务", §2.3 跨算子融合,
 *      sketch "LayerNorm + QKV Projection 融合" (per-token mean and variance,
 *      reciprocal square root of variance plus eps, scale by gamma and shift
 *      by beta, then the Q, K and V products written straight out) and sketch
 *      "GEMM + 激活融合（SwiGLU）" (SiLU of the gate product times the up
 *      product, activation and multiply kept in registers).
 *  [D2] same page, §2.2 图构建与算子映射: QKV projection = one matmul followed
 *      by reshape and GQA grouping of the heads.
 *  [I] "2. TensorRT-LLM 简介", 核心原理: the graph-optimisation layer fuses
 *      QKV, fuses residual + LayerNorm, and matches precision per op.
 *  [F] "TRT-LLM deep dive" (lib.uml.com.cn), 构建阶段详解 §3 Layer Fusion
 *      figure: Add -> (Mul/Bias) -> LayerNorm -> GELU collapsed into one
 *      kernel; 面试视角: LayerNorm + Linear + GELU as a single kernel.
 *
 * Readings of points the pages leave open (each repeated where it is used):
 *  R1 residual add h = x + r, exact; the stored residual stream is
 *     h_out = RNE_act(h).
 *  R2 RMSNorm n = h / sqrt(mean(h^2) + eps) * gamma (no mean, no beta).
 *  R3 LayerNorm uses the biased (1/K) variance; gamma scales the normalised
 *     value and beta is added last, the order the sketch [D] uses.
 *  R4 QKV columns are three contiguous blocks Q | K | V; q, k, v are stored
 *     token-major [M, heads, head_dim].
 *  R5 SwiGLU: the weight holds the gate rows [0, F) then the up rows [F, 2F);
 *     out = SiLU(gate) * up with SiLU(g) = g / (1 + exp(-g)).
 *  R6 GELU is the tanh approximation
 *     0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))).
 *  R7 bias (when given) is added to the accumulator before the activation.
 *  R8 int8 weights: w = RNE_bf16(RNE_f32(q * s)) with s the fp32 scale of the
 *     output row; both roundings are part of the definition.
 *  R9 int4 weights (4-bit weights with 16-bit activations, symmetric, one
 *     scale per group of 128 consecutive k, no zero point: [Q] below): the
 *     [N, K] weight is stored as [N, K/2] bytes, element k of a row in the
 *     low nibble of byte k/2 for even k and in the high nibble for odd k,
 *     each nibble a two's-complement integer in [-8, 7]; the scales are
 *     [N, K/128] fp32; w = RNE_bf16(RNE_f32(q * s[row][k/128])), the two
 *     roundings of R8.  A zero product is +0: the value is exactly zero (the
 *     format defines no signed zero; only a zero scale with a negative q
 *     could give an IEEE -0).
 *  R10 FP8 W8A8 ([Q]: the full-FP8 configuration, whose activation range is
 *     taken from the data at run time rather than from a calibration): the
 *     weights are E4M3 codes [N, K] with one fp32 scale per output row,
 *     w = e4m3(code) * s[row] (exact in double); the activations are
 *     quantised per token at run time from the single-precision normalised
 *     row n32 of R11, in single precision: amax = max_k |n32[k]|,
 *     s_a = fp32(amax / 448), t = fp32(n32 * fp32(448 / amax)) clamped to
 *     [-448, 448], code = E4M3 nearest of t (ties to the even code), a =
 *     e4m3(code) * s_a; a row with amax = 0 quantises to zeros.  The product
 *     then uses a and w as above.  E4M3 here is the OCP 8-bit format with
 *     1 sign, 4 exponent (bias 7) and 3 mantissa bits: exponent field 0
 *     holds the subnormals m * 2^-9, there are no infinities, S.1111.111 is
 *     NaN and 448 is the largest finite value.
 *  R11 precision of the normalisation (the sketch [D] holds the mean, the
 *     variance and the reciprocal root as float and forms the normalised
 *     value from them before storing it as half): the row statistics are
 *     accumulated in double and rounded once to fp32, mu32 = fp32(mean) and
 *     rs32 = fp32(1 / sqrt(var + eps)) (RMS: mean(h^2) for var, mu32 = 0);
 *     h32 = fp32(x + r); the normalised value is then evaluated in fp32 as
 *       RMS:   n32 = fp32(fp32(h32 * rs32) * gamma)
 *       LAYER: n32 = fma32(fp32(fp32(h32 - mu32) * rs32), gamma, beta or 0)
 *       NONE:  n32 = h32
 *     and the GEMM operand is a = RNE_act(n32).  Every rounding that decides
 *     a stored value (the activation dtype, an E4M3 code) thus starts from a
 *     value both implementations compute with the same single-precision
 *     operations; the double-precision n of R2 / R3 stays the reference that
 *     n32 is pinned to.
 *  R12 MXFP4 weights with 16-bit activations ([Q]: the W4A16_FP4
 *     configuration; [B]: microscaling, 32 FP4 elements sharing one 8-bit
 *     scale): the [N, K] weight is stored as [N, K/2] bytes of E2M1 codes,
 *     element k of a row in the low nibble of byte k/2 for even k and in the
 *     high nibble for odd k, with [N, K/32] E8M0 scales, one per row and
 *     block of 32 consecutive k.  E2M1 is 1 sign, 2 exponent (bias 1) and
 *     1 mantissa bit: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}, no infinities or NaN,
 *     code 8 is -0; E8M0 is an unsigned exponent, 2^(s - 127), s = 255 NaN
 *     (out of contract).  w = e2m1(code) * 2^(s - 127), exact in double; the
 *     GEMM operand is RNE_bf16(w), w itself for every s up to 252 (larger
 *     scales can overflow bf16 to +-inf).  Activations stay bf16 (the
 *     sixteen-bit half of W4A16), normalised and rounded as R11.
 *  [B] same page, §7.1 FP4 精度与第五代 Tensor Core: two-level (block and
 *      element) quantisation; MXFP4, each 32 FP4 elements sharing one 8-bit
 *      scale.
 *  [Q] "TensorRT-LLM 深度工程实践…", §3.3 FP4/FP8 动态量化加速: the W4A16
 *      (AWQ/GPTQ) configuration with group size 128 and no zero point, and
 *      the W8A8 FP8 configuration with online activation ranges.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_I8 = 3, OR_I4 = 4, OR_E4M3 = 5, OR_MXFP4 = 6 };
enum { OR_E4M3_MAX = 448 };
enum { OR_I4_GROUP = 128 };
enum { OR_MX_BLOCK = 32 };
enum { OR_NORM_NONE = 0, OR_NORM_RMS = 1, OR_NORM_LAYER = 2 };
enum { OR_ACT_NONE = 0, OR_ACT_SWIGLU = 1, OR_ACT_GELU_TANH = 2 };

/* ---------------------------------------------------------------------------
 * Number formats.  A binary floating-point format is described by its
 * significand precision p (bits, implicit bit included), the exponent of its
 * smallest normal number, and its largest finite value.
 * ------------------------------------------------------------------------- */
static void fmt_params(int dtype, int *p, int *emin, double *maxv) {
    switch (dtype) {
    case OR_F16:  *p = 11; *emin = -14;  *maxv = 65504.0; break;
    case OR_BF16: *p = 8;  *emin = -126; *maxv = ldexp(255.0, 120); break; /* (2-2^-7)*2^127 */
    default:      *p = 24; *emin = -126; *maxv = ldexp(16777215.0, 104); break; /* (2-2^-23)*2^127 */
    }
}

/* Round v to the nearest value of the format, ties to even; values beyond the
 * largest finite number (after rounding) become +-inf.  Works directly from
 * the double, so there is no double rounding. */
double or_round(double v, int dtype) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    int p, emin; double maxv;
    fmt_params(dtype, &p, &emin, &maxv);
    int e2;
    (void)frexp(v, &e2);          /* v = f * 2^e2, 0.5 <= |f| < 1 */
    int lead = e2 - 1;            /* exponent of the leading bit */
    if (lead < emin) lead = emin; /* subnormal range: fixed quantum */
    int qexp = lead - (p - 1);    /* weight of the last significand bit */
    double scaled = ldexp(v, -qexp);         /* exact (power-of-two scaling) */
    double r = nearbyint(scaled);            /* default mode: ties to even */
    double out = ldexp(r, qexp);
    if (fabs(out) > maxv) out = copysign(INFINITY, v);
    return out;
}

/* Decode one stored element to double. */
double or_load(const void *ptr, int dtype, int64_t i) {
    switch (dtype) {
    case OR_F32: return (double)((const float *)ptr)[i];
    case OR_I8:  return (double)((const int8_t *)ptr)[i];
    case OR_BF16: {
        uint32_t b = ((const uint16_t *)ptr)[i];
        uint32_t u = b << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    case OR_F16: {
        uint16_t b = ((const uint16_t *)ptr)[i];
        int sign = (b >> 15) & 1, ex = (b >> 10) & 31, man = b & 1023;
        double mag;
        if (ex == 0)       mag = ldexp((double)man, -24);              /* subnormal */
        else if (ex == 31) mag = man ? NAN : INFINITY;
        else               mag = ldexp((double)(1024 + man), ex - 25); /* 1.man * 2^(ex-15) */
        return sign ? -mag : mag;
    }
    }
    return NAN;
}

void or_decode_array(const void *in, int dtype, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_load(in, dtype, i);
}

void or_round_array(const double *in, double *out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_round(in[i], dtype);
}

/* bf16 bit pattern of a double that is already exactly a bf16 value. */
static uint16_t bf16_bits_of(double v) {
    float f = (float)v;   /* exact: v is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------------------
 * Activations (R5, R6).
 * ------------------------------------------------------------------------- */
double or_silu(double g) { return g / (1.0 + exp(-g)); }

double or_gelu_tanh(double y) {
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * y * (1.0 + tanh(c * (y + 0.044715 * y * y * y)));
}

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * int8 weight dequantisation (R8): w = RNE_bf16(RNE_f32(q * s)).
 * q * s is exact in double (8-bit times 24-bit significands).
 * ------------------------------------------------------------------------- */
int or_dequant_i8(const int8_t *q, const float *s, int64_t N, int64_t K,
                  double *w_out, uint16_t *bits_out) {
    for (int64_t j = 0; j < N; ++j) {
        for (int64_t k = 0; k < K; ++k) {
            double prod = (double)q[j * K + k] * (double)s[j];
            double w = or_round(or_round(prod, OR_F32), OR_BF16);
            if (w_out) w_out[j * K + k] = w;
            if (bits_out) bits_out[j * K + k] = bf16_bits_of(w);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * int4 weight dequantisation (R9): element k of row j is the nibble
 * (byte k/2 of the row) >> (4 (k mod 2)), read as a 4-bit two's-complement
 * integer, times the scale of its group k / 128; then the two roundings of
 * R8.  q * s is exact in double (4-bit times 24-bit significands).
 * ------------------------------------------------------------------------- */
int or_i4_value(const uint8_t *row, int64_t k) {
    int nib = (row[k / 2] >> (4 * (int)(k % 2))) & 0xF;
    return nib >= 8 ? nib - 16 : nib;
}

int or_dequant_i4(const uint8_t *q, const float *s, int64_t N, int64_t K,
                  double *w_out, uint16_t *bits_out) {
    if (K % OR_I4_GROUP != 0) return -1;
    const int64_t G = K / OR_I4_GROUP;
    for (int64_t j = 0; j < N; ++j) {
        const uint8_t *row = q + j * (K / 2);
        for (int64_t k = 0; k < K; ++k) {
            double prod = (double)or_i4_value(row, k) * (double)s[j * G + k / OR_I4_GROUP];
            double w = or_round(or_round(prod, OR_F32), OR_BF16);
            if (w == 0.0) w = 0.0;   /* +0 (R9) */
            if (w_out) w_out[j * K + k] = w;
            if (bits_out) bits_out[j * K + k] = bf16_bits_of(w);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * MXFP4 weights (R12): E2M1 element codes with one E8M0 scale per block of 32
 * consecutive k of a row.
 * ------------------------------------------------------------------------- */
double or_e2m1_value(int code) {
    code &= 0xF;
    const int e = (code >> 1) & 3, m = code & 1;
    /* subnormal (e = 0): m * 0.5; normal: (1 + m/2) 2^(e-1) = (2 + m) 2^(e-2) */
    const double v = e == 0 ? 0.5 * m : ldexp(2.0 + m, e - 2);
    return (code & 8) ? -v : v;
}

double or_e8m0_value(int s) {
    s &= 0xFF;
    return s == 255 ? NAN : ldexp(1.0, s - 127);
}

int or_mxfp4_code(const uint8_t *row, int64_t k) {
    return (row[k >> 1] >> ((k & 1) << 2)) & 0xF;   /* even k: low nibble */
}

int or_dequant_mxfp4(const uint8_t *q, const uint8_t *s, int64_t N, int64_t K,
                     double *w_out, uint16_t *bits_out) {
    if (K % OR_MX_BLOCK != 0) return -1;
    const int64_t G = K / OR_MX_BLOCK;
    for (int64_t j = 0; j < N; ++j) {
        const uint8_t *row = q + j * (K / 2);
        for (int64_t k = 0; k < K; ++k) {
            /* exact product (2-bit significand times a power of two), then the
             * bf16 operand */
            const double prod = or_e2m1_value(or_mxfp4_code(row, k)) * or_e8m0_value(s[j * G + k / OR_MX_BLOCK]);
            const double w = or_round(prod, OR_BF16);
            if (w_out) w_out[j * K + k] = w;
            if (bits_out) bits_out[j * K + k] = bf16_bits_of(w);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * E4M3 (R10).
 * ------------------------------------------------------------------------- */
/* value of an E4M3 code (NaN for S.1111.111) */
double or_e4m3_value(int code) {
    code &= 0xFF;
    const int e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    /* normal: (1 + m/8) 2^(e-7) = (8 + m) 2^(e-10); subnormal: m 2^-9 */
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return (code & 0x80) ? -v : v;
}

/* nearest E4M3 code of t, ties to the even code; magnitudes beyond 448 are
 * taken as 448 (the quantiser clamps before it rounds) */
int or_e4m3_encode(double t) {
    const int sign = signbit(t) ? 0x80 : 0;
    double a = fabs(t);
    if (a > (double)OR_E4M3_MAX) a = (double)OR_E4M3_MAX;
    if (a < ldexp(1.0, -6))                       /* below the smallest normal: */
        return sign | (int)nearbyint(ldexp(a, 9)); /* a multiple of 2^-9; 8 is the smallest normal */
    int e;
    const double f = frexp(a, &e);                /* a = f 2^e, f in [0.5, 1) */
    double q = nearbyint(16.0 * f - 8.0);         /* 3 mantissa bits, exact argument */
    int field = e - 1 + 7;
    if (q == 8.0) { q = 0.0; field += 1; }
    return sign | (field << 3) | (int)q;
}

/* per-token quantisation of the rows of n [M, K] (R10), in single
 * precision: each value is taken as fp32 (the rows are the fp32 values n32 of
 * R11, or activations of a 16-bit dtype, both exact in fp32); codes (or NULL),
 * a = e4m3(code) * s_a (or NULL; may be n itself) and s_a [M] (or NULL) */
int or_quant_rows_e4m3(const double *n, int64_t M, int64_t K, uint8_t *codes, double *a,
                       double *s_out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k)
            if (fabsf((float)n[m * K + k]) > amax) amax = fabsf((float)n[m * K + k]);
        const float s = amax / (float)OR_E4M3_MAX;
        const float inv = amax > 0.0f ? (float)OR_E4M3_MAX / amax : 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float t = (float)n[m * K + k] * inv;
            if (t > (float)OR_E4M3_MAX) t = (float)OR_E4M3_MAX;
            if (t < -(float)OR_E4M3_MAX) t = -(float)OR_E4M3_MAX;
            const int c = or_e4m3_encode((double)t);
            if (codes) codes[m * K + k] = (uint8_t)c;
            if (a) a[m * K + k] = or_e4m3_value(c) * (double)s;
        }
        if (s_out) s_out[m] = (double)s;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Residual add and row normalisation, one token row at a time ([D], [I]).
 *  h = x + r                                        (R1; r may be NULL)
 *  RMS:   n = h / sqrt(sum(h^2)/K + eps) * gamma    (R2)
 *  LAYER: mu = sum(h)/K, var = sum((h-mu)^2)/K,
 *         n = (h - mu) / sqrt(var + eps) * gamma + beta   (R3; beta may be NULL)
 *  NONE:  n = h
 * Outputs (each may be NULL): h_out = RNE_act(h), n_out = n (double),
 * n32_out = the single-precision normalised value of R11 (as double),
 * a_out = RNE_act(n32).
 * ------------------------------------------------------------------------- */
int or_add_norm(const void *x, const void *r, const void *gamma, const void *beta,
                int act, int norm, double eps, int64_t M, int64_t K,
                double *h_out, double *n_out, double *n32_out, double *a_out) {
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *h = (double *)malloc(sizeof(double) * (size_t)K);
        if (!h) { bad = 1; continue; }
        for (int64_t k = 0; k < K; ++k) {
            double hv = or_load(x, act, m * K + k);
            if (r) hv += or_load(r, act, m * K + k);
            h[k] = hv;
            if (h_out) h_out[m * K + k] = or_round(hv, act);
        }
        double mu = 0.0, inv = 1.0;
        if (norm == OR_NORM_RMS) {
            double ss = 0.0;
            for (int64_t k = 0; k < K; ++k) ss += h[k] * h[k];
            inv = 1.0 / sqrt(ss / (double)K + eps);
        } else if (norm == OR_NORM_LAYER) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += h[k];
            mu = s / (double)K;
            double vs = 0.0;
            for (int64_t k = 0; k < K; ++k) vs += (h[k] - mu) * (h[k] - mu);
            inv = 1.0 / sqrt(vs / (double)K + eps);
        }
        /* R11: the statistics rounded once to single precision */
        const float mu32 = (float)mu, rs32 = (float)inv;
        for (int64_t k = 0; k < K; ++k) {
            double n;
            const float h32 = (float)h[k];
            float n32;
            if (norm == OR_NORM_RMS) {
                n = h[k] * inv * or_load(gamma, act, k);
                const float t = h32 * rs32;
                n32 = t * (float)or_load(gamma, act, k);
            } else if (norm == OR_NORM_LAYER) {
                n = (h[k] - mu) * inv * or_load(gamma, act, k);
                if (beta) n += or_load(beta, act, k);
                const float d = h32 - mu32;
                const float t = d * rs32;
                n32 = fmaf(t, (float)or_load(gamma, act, k), beta ? (float)or_load(beta, act, k) : 0.0f);
            } else {
                n = h[k];
                n32 = h32;
            }
            if (n_out) n_out[m * K + k] = n;
            if (n32_out) n32_out[m * K + k] = (double)n32;
            if (a_out) a_out[m * K + k] = or_round((double)n32, act);
        }
        free(h);
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------------
 * The projection product acc[m, j] = sum_k a[m, k] * w[j, k]  ([D]).
 * w is [N, K] with K contiguous, in its stored dtype; int8, int4 and E4M3
 * weights go through the dequantisations above (R8, R9, R10; w_scale is [N]
 * or [N, K/128]).  Each weight row is decoded once into a double buffer and then
 * used for every token row.
 * ------------------------------------------------------------------------- */
int or_matmul_nt(const double *a, const void *w, int wdtype, const void *w_scale_v,
                 int64_t M, int64_t K, int64_t N, double *acc) {
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j) {
        double *wr = (double *)malloc(sizeof(double) * (size_t)K);
        if (!wr) { bad = 1; continue; }
        const float *w_scale = (const float *)w_scale_v;
        if (wdtype == OR_MXFP4) {
            if (or_dequant_mxfp4((const uint8_t *)w + j * (K / 2), (const uint8_t *)w_scale_v + j * (K / OR_MX_BLOCK),
                                 1, K, wr, NULL))
                bad = 1;
        } else if (wdtype == OR_I8)
            or_dequant_i8((const int8_t *)w + j * K, w_scale + j, 1, K, wr, NULL);
        else if (wdtype == OR_E4M3)
            for (int64_t k = 0; k < K; ++k)
                wr[k] = or_e4m3_value(((const uint8_t *)w)[j * K + k]) * (double)w_scale[j];
        else if (wdtype == OR_I4) {
            if (or_dequant_i4((const uint8_t *)w + j * (K / 2), w_scale + j * (K / OR_I4_GROUP), 1, K, wr, NULL))
                bad = 1;
        } else
            for (int64_t k = 0; k < K; ++k) wr[k] = or_load(w, wdtype, j * K + k);
        for (int64_t m = 0; m < M; ++m) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += a[m * K + k] * wr[k];
            acc[m * N + j] = s;
        }
        free(wr);
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------------
 * Full calls.
 * ------------------------------------------------------------------------- */
/* the GEMM A operand: the single-precision normalised rows (R11) rounded to
 * the activation dtype (reading A) or quantised per token for E4M3 weights
 * (R10), or the unrounded double-precision rows (reading B) */
static double *prologue(const void *x, const void *r, const void *gamma, const void *beta,
                        int act, int norm, double eps, int64_t M, int64_t K,
                        double *h_out, int rounded, int wdtype) {
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!a) return NULL;
    const int fp8 = rounded && wdtype == OR_E4M3;
    int rc = !rounded ? or_add_norm(x, r, gamma, beta, act, norm, eps, M, K, h_out, a, NULL, NULL)
           : fp8      ? or_add_norm(x, r, gamma, beta, act, norm, eps, M, K, h_out, NULL, a, NULL)
                      : or_add_norm(x, r, gamma, beta, act, norm, eps, M, K, h_out, NULL, NULL, a);
    if (!rc && fp8) rc = or_quant_rows_e4m3(a, M, K, NULL, a, NULL);
    if (rc) { free(a); return NULL; }
    return a;
}

/* residual add + norm -> QKV product -> (+bias) -> split into q, k, v.
 * q: [M, H, D], k and v: [M, Hkv, D]; column c of the product is
 * q[m, c / D, c % D] for c < H*D, then k, then v (R4, [D2]). */
int or_add_norm_qkv(const void *x, const void *r, const void *gamma, const void *beta,
                    int act, int norm, double eps,
                    const void *w, int wdtype, const void *w_scale, const void *bias,
                    int64_t M, int64_t K, int64_t H, int64_t Hkv, int64_t D,
                    double *q, double *k, double *v, double *h_out, int rounded) {
    int64_t N = (H + 2 * Hkv) * D, nq = H * D, nkv = Hkv * D;
    double *a = prologue(x, r, gamma, beta, act, norm, eps, M, K, h_out, rounded, wdtype);
    double *acc = (double *)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
    if (!a || !acc) { free(a); free(acc); return -1; }
    if (or_matmul_nt(a, w, wdtype, w_scale, M, K, N, acc)) { free(a); free(acc); return -1; }
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < N; ++c) {
            double y = acc[m * N + c];
            if (bias) y += or_load(bias, act, c);
            if (c < nq)            q[m * nq + c] = y;
            else if (c < nq + nkv) k[m * nkv + (c - nq)] = y;
            else                   v[m * nkv + (c - nq - nkv)] = y;
        }
    }
    free(a);
    free(acc);
    return 0;
}

/* (residual add + norm ->) gate/up or up product -> (+bias) -> activation.
 * SWIGLU: w is [2F, K] (gate rows then up rows), out[m, j] = SiLU(g) * u (R5).
 * GELU_TANH / NONE: w is [F, K], out = GELU(acc + b) or acc + b (R6, R7, [F]). */
int or_gateup_act(const void *x, const void *r, const void *gamma, const void *beta,
                  int act, int norm, double eps,
                  const void *w, int wdtype, const void *w_scale, const void *bias,
                  int64_t M, int64_t K, int64_t F, int actfn,
                  double *out, double *h_out, int rounded) {
    int64_t N = actfn == OR_ACT_SWIGLU ? 2 * F : F;
    double *a = prologue(x, r, gamma, beta, act, norm, eps, M, K, h_out, rounded, wdtype);
    double *acc = (double *)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
    if (!a || !acc) { free(a); free(acc); return -1; }
    if (or_matmul_nt(a, w, wdtype, w_scale, M, K, N, acc)) { free(a); free(acc); return -1; }
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < F; ++j) {
            double y;
            if (actfn == OR_ACT_SWIGLU) {
                double g = acc[m * N + j], u = acc[m * N + F + j];
                if (bias) { g += or_load(bias, act, j); u += or_load(bias, act, F + j); }
                y = or_silu(g) * u;
            } else {
                y = acc[m * N + j];
                if (bias) y += or_load(bias, act, j);
                if (actfn == OR_ACT_GELU_TANH) y = or_gelu_tanh(y);
            }
            out[m * F + j] = y;
        }
    }
    free(a);
    free(acc);
    return 0;
}

/* Down projection with the residual add ([T] below):
 * out[m, c] = residual[m, c] + bias[c] + sum_k a[m, k] * w[c, k], in double.
 * a is [M, K] in the activation dtype and used as stored (no norm, no
 * rounding: it is already an activation-dtype tensor; with E4M3 weights it
 * is quantised per token, R10); w is [N, K] as for the other products (R8,
 * R9, R10); residual and bias may be NULL.
 * [T] "TensorRT-LLM 深度工程实践…", §4.1: the MLP's gate/up projection
 *     followed by the down projection; "TRT-LLM deep dive", 构建阶段详解 §3:
 *     the Add folded into the neighbouring kernel. */
int or_down_residual(const void *a, int act, const void *w, int wdtype, const void *w_scale,
                     const void *bias, const void *residual, int64_t M, int64_t K, int64_t N,
                     double *out) {
    double *ad = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!ad) return -1;
    or_decode_array(a, act, M * K, ad);
    if (wdtype == OR_E4M3) or_quant_rows_e4m3(ad, M, K, NULL, ad, NULL);   /* R10 */
    if (or_matmul_nt(ad, w, wdtype, w_scale, M, K, N, out)) { free(ad); return -1; }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < N; ++c) {
            if (bias) out[m * N + c] += or_load(bias, act, c);
            if (residual) out[m * N + c] += or_load(residual, act, m * N + c);
        }
    free(ad);
    return 0;
}
