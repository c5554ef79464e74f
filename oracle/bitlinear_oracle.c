/*
 * CPU oracle of the BitNet b1.58 BitLinear forward -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct reference of what the GPU library computes.
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this code; the product path never does.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * Sources (web pages), cited by title and section:
 *   [P4] "BitNet b1.58 in Production: 1-Bit LLMs and Energy Benchmarks",
 *        section "The Mathematical Mechanism", items 1-4 (weight quantization,
 *        activation quantization, integer addition kernel, de-quantization),
 *        and its "bit_linear.py" listing (weight_quant / activation_quant /
 *        BitLinear.forward), used only where the items leave a step open.
 *   [P5] "BitNet 1-bit LLM Inference Framework: Running Large Language Models
 *        on CPU", section "How the LUT Kernel Works" (2-bit code assignment
 *        00 = 0, 01 = +1, 10 = -1, four weights per byte).
 *
 * Readings where the pages leave a choice open (all documented with the tests):
 *   - gamma is one scalar per weight matrix: the mean of |W| accumulated in
 *     binary64, divided by n*k in binary64, rounded once to binary32;
 *   - the weight epsilon is additive, 1e-5, added in binary32 to gamma;
 *   - "Round" is round-half-to-even (the listing's torch.round);
 *   - weights: round then clip to [-1, 1]; activations: round then clip to
 *     [-127, 127] with Q_b = 2^(8-1) - 1 = 127;
 *   - activation scale per token: a' = max(max_k |x|, 1e-8), s = 127 / a'
 *     (one binary32 divide), code = clip(round(x * s)) (one binary32 multiply);
 *   - de-quantization y = acc * gamma * a' / 127 evaluated in binary64 and
 *     rounded once to binary32.
 *
 * Beyond the four steps (the steps on either side of the contraction):
 *   [P4] the "bit_linear.py" listing normalises the BitLinear input with
 *        nn.RMSNorm(in_features) before activation_quant;
 *   [P5] "BitNet 1-bit LLM Inference Framework", section "A Deep Look at the
 *        BitNet Architecture", the ffn of the transformer block:
 *        down_proj(silu(gate_proj(x)) * up_proj(x)).
 * Readings taken there:
 *   - RMSNorm, in the listing's order: r = 1 / sqrt(mean_k x^2 + eps) per
 *     token (binary64, rounded once to binary32), x_norm = (x * r) * w with
 *     an optional per-channel gain w (binary32), and then the per-token
 *     absmax rule of O5 on x_norm.  An all-zero x_norm gives codes 0 and
 *     a' = 1e-8;
 *   - SwiGLU: h = silu(g) * u = g * u / (1 + exp(-g)) in binary64, rounded
 *     once to binary32, from the two de-quantized BitLinear outputs;
 *   - h is requantized for the next BitLinear from binary32 with the same
 *     per-token rule as the bf16 activations.
 *
 * Variant modes (each its own functions, V1-V3 below):
 *   V1 [P5] "BitNet 1-bit LLM Inference Framework", the BitLinear class
 *      under "The Core Structure of BitNet b1.58": one activation scale per
 *      tensor, Q_b = 2^7 = 128, codes in
 *      [-128, 127] (clamp, then round), de-quantization by gamma * g / 2^7.
 *      The same listing's weight epsilon (1e-8) is not taken: the variant
 *      changes the activation side only, weights follow O1-O3;
 *   V2 [P2] "BitNet-2B-4T: Inside the 2B-Parameter, 4T-Token 1-Bit LLM",
 *      section "Weight Representation: Ternary + Scale, Not Pure Binary":
 *      one FP16 scale per output channel.  Reading: the scale is that row's
 *      absmean (as gamma, per row), rounded to binary32 then to binary16, and
 *      the row is ternarized and de-quantized with the stored value;
 *   V3 [P1] "BitNet's 1-Bit Transformer: Architecture Breakdown", section
 *      "Binary Weight Matrices with Learnable Scaling": W_bit = s * sign(W),
 *      s one learned scalar per layer (an input here).  Reading: sign(0) is
 *      +1; the activations take the main path's per-token int8 codes.
 *
 * Build: gcc -O2 -fopenmp -fno-fast-math -ffp-contract=off (see build.py).
 * OpenMP is used over independent output rows only.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* helpers                                                             */
/* ------------------------------------------------------------------ */

/* bf16 bit pattern -> binary32 (exact: bf16 is the top half of binary32). */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 value to the nearest integer, ties to even, written out
 * from the definition (no dependence on the FPU rounding mode).  Valid for
 * |t| < 2^23, where t - floor(t) is exact; larger binary32 values are
 * already integers. */
static double round_half_even(float t)
{
    double td = (double)t;
    if (fabs(td) >= 8388608.0) /* 2^23: already an integer */
        return td;
    double fl = floor(td);
    double frac = td - fl; /* exact */
    if (frac > 0.5)
        return fl + 1.0;
    if (frac < 0.5)
        return fl;
    /* exact tie: pick the even neighbour */
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

static double clip(double v, double lo, double hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

/* ------------------------------------------------------------------ */
/* O1: absmean weight scale gamma  [P4, Mathematical Mechanism, item 1] */
/* ------------------------------------------------------------------ */

/* Sum of |W| over all n*k weights in binary64.  Each row is summed left to
 * right, then the row sums are added in row order, so the result does not
 * depend on the thread count. */
double oracle_abs_sum(const float *w, int64_t n, int64_t k, double *row_sums)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        double s = 0.0;
        const float *row = w + r * k;
        for (int64_t c = 0; c < k; ++c)
            s += fabs((double)row[c]);
        row_sums[r] = s;
    }
    double total = 0.0;
    for (r = 0; r < n; ++r)
        total += row_sums[r];
    return total;
}

/* gamma = (1 / (n m)) * sum |W_ij| ; binary64 mean, rounded once to binary32. */
float oracle_gamma_from_sum(double abs_sum, int64_t n, int64_t k)
{
    double mean = abs_sum / ((double)n * (double)k);
    return (float)mean;
}

/* ------------------------------------------------------------------ */
/* O2-O3: ternary RoundClip  [P4, Mathematical Mechanism, item 1]      */
/* ------------------------------------------------------------------ */

/* q = Clip(Round(W / (gamma + eps)), -1, 1) with eps = 1e-5 added in binary32
 * and one IEEE binary32 divide per weight. */
static int8_t ternary_code(float w, float denom)
{
    const float t = w / denom;
    return (int8_t)clip(round_half_even(t), -1.0, 1.0);
}

void oracle_ternarize(const float *w, int64_t n, int64_t k, float gamma, int8_t *q)
{
    const float denom = gamma + 1e-5f;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        for (int64_t c = 0; c < k; ++c)
            q[r * k + c] = ternary_code(w[r * k + c], denom);
    }
}

/* ------------------------------------------------------------------ */
/* O4: canonical 2-bit packing  [P5, How the LUT Kernel Works]          */
/* ------------------------------------------------------------------ */

/* Row-major; row r occupies ceil(k/4) bytes; weight c of the row sits in byte
 * c/4 at bits 2*(c%4) .. 2*(c%4)+1 (least significant first).  Codes:
 * 00 = 0, 01 = +1, 10 = -1; padding fields are 00. */
void oracle_pack_canonical(const int8_t *q, int64_t n, int64_t k, uint8_t *out)
{
    const int64_t kb = (k + 3) / 4;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t j = 0; j < kb; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                int64_t c = 4 * j + i;
                unsigned code = 0;
                if (c < k) {
                    int8_t v = q[r * k + c];
                    code = (v == 1) ? 1u : (v == -1) ? 2u : 0u;
                }
                byte |= code << (2 * i);
            }
            out[r * kb + j] = (uint8_t)byte;
        }
    }
}

/* Inverse of oracle_pack_canonical.  Returns 0, or -1 if any field inside
 * the k valid columns holds the unused code 11, or -2 if a padding field is
 * not 00. */
int oracle_unpack_canonical(const uint8_t *in, int64_t n, int64_t k, int8_t *q)
{
    const int64_t kb = (k + 3) / 4;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t j = 0; j < kb; ++j) {
            unsigned byte = in[r * kb + j];
            for (int i = 0; i < 4; ++i) {
                int64_t c = 4 * j + i;
                unsigned code = (byte >> (2 * i)) & 3u;
                if (c >= k) {
                    if (code != 0)
                        return -2;
                    continue;
                }
                if (code == 3)
                    return -1;
                q[r * k + c] = (int8_t)(code == 1 ? 1 : (code == 2 ? -1 : 0));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O5: per-token absmax int8 activation quantization                    */
/*     [P4, Mathematical Mechanism, item 2]                             */
/* ------------------------------------------------------------------ */

/* x: bf16 bits [m][k]; xq: int8 [m][k]; amax: [m] receives a' (the clamped
 * per-token max used by both quantization and de-quantization). */
void oracle_quant_act(const uint16_t *x, int64_t m, int64_t k, int8_t *xq, float *amax)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        float a = 0.0f;
        for (int64_t c = 0; c < k; ++c) {
            float v = fabsf(bf16_to_f32(x[r * k + c]));
            if (v > a)
                a = v;
        }
        if (a < 1e-8f)
            a = 1e-8f;
        const float s = 127.0f / a;
        for (int64_t c = 0; c < k; ++c) {
            float t = bf16_to_f32(x[r * k + c]) * s;
            xq[r * k + c] = (int8_t)clip(round_half_even(t), -127.0, 127.0);
        }
        amax[r] = a;
    }
}

/* Same rule from binary32 activations (x: fp32 [m][k]). */
void oracle_quant_act_f32(const float *x, int64_t m, int64_t k, int8_t *xq, float *amax)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        float a = 0.0f;
        for (int64_t c = 0; c < k; ++c) {
            float v = fabsf(x[r * k + c]);
            if (v > a)
                a = v;
        }
        if (a < 1e-8f)
            a = 1e-8f;
        const float s = 127.0f / a;
        for (int64_t c = 0; c < k; ++c) {
            float t = x[r * k + c] * s;
            xq[r * k + c] = (int8_t)clip(round_half_even(t), -127.0, 127.0);
        }
        amax[r] = a;
    }
}

/* ------------------------------------------------------------------ */
/* RMSNorm ahead of the activation quantization                        */
/*   [P4, "bit_linear.py": x_norm = rms_norm(x); activation_quant(x_norm)]*/
/* ------------------------------------------------------------------ */

/* The listing's order, value by value: first the normalised input
 *   r = 1 / sqrt(mean_k x^2 + eps)   (mean square in binary64, r rounded once
 *                                     to binary32),
 *   x_norm = (x * r) * w              (two binary32 multiplies; w = 1 when
 *                                     the gain is NULL),
 * then O5's per-token absmax rule applied to x_norm:
 *   a' = max(max_k |x_norm|, 1e-8), s = 127 / a' (binary32 divide),
 *   code = Clip(Round(x_norm * s), -127, 127).
 * x: bf16 bits [m][k]; xq: int8 [m][k]; amax: [m] receives a'.  rms_out (may
 * be NULL) receives r; xnorm_out (may be NULL) receives x_norm, fp32 [m][k]. */
void oracle_rmsnorm_quant_act(const uint16_t *x, const float *w, float eps, int64_t m, int64_t k,
                              int8_t *xq, float *amax, float *rms_out, float *xnorm_out)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        /* nn.RMSNorm: the mean of the squares, then its reciprocal root */
        double ss = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            const double xv = (double)bf16_to_f32(x[r * k + c]);
            ss += xv * xv;
        }
        const float rr = (float)(1.0 / sqrt(ss / (double)k + (double)eps));
        if (rms_out)
            rms_out[r] = rr;
        /* the normalised token, then activation_quant of it */
        float a = 0.0f;
        for (int64_t c = 0; c < k; ++c) {
            float xn = bf16_to_f32(x[r * k + c]) * rr;
            if (w)
                xn = xn * w[c];
            if (xnorm_out)
                xnorm_out[r * k + c] = xn;
            if (fabsf(xn) > a)
                a = fabsf(xn);
        }
        if (a < 1e-8f)
            a = 1e-8f;
        const float s = 127.0f / a;
        for (int64_t c = 0; c < k; ++c) {
            float xn = bf16_to_f32(x[r * k + c]) * rr;
            if (w)
                xn = xn * w[c];
            xq[r * k + c] = (int8_t)clip(round_half_even(xn * s), -127.0, 127.0);
        }
        amax[r] = a;
    }
}

/* ------------------------------------------------------------------ */
/* O6: ternary x int8 contraction  [P4, Mathematical Mechanism, item 3] */
/* ------------------------------------------------------------------ */

/* acc[i][j] = sum_k xq[i][k] * q[j][k]: the plain integer dot product of a
 * token's codes with a weight row whose entries are -1, 0 or +1, so every
 * term is the code itself, zero, or its negation and no real multiplication
 * is needed.  The terms are summed in int64, in column order, and the sum is
 * checked against |acc| <= qmax * k (127 * k; 128 * k for the V1 codes,
 * which reach -128) before it is stored as int32.
 * Returns 0, or -1 if the bound (or int32 range) is violated, or -2 if a
 * weight is not in {-1, 0, 1}. */
static int64_t ternary_dot(const int8_t *a, const int8_t *w, int64_t k, int *bad)
{
    int64_t s = 0;
    for (int64_t c = 0; c < k; ++c) {
        if (w[c] < -1 || w[c] > 1)
            *bad |= 2;
        s += (int64_t)a[c] * (int64_t)w[c];
    }
    return s;
}

static int contract_bounded(const int8_t *xq, const int8_t *q, int64_t m, int64_t n, int64_t k,
                            int64_t qmax, int32_t *acc)
{
    int bad = 0;
    const int64_t bound = qmax * k;
    int64_t i;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (i = 0; i < m * n; ++i) {
        const int64_t row = i / n, col = i % n;
        const int64_t s = ternary_dot(xq + row * k, q + col * k, k, &bad);
        if (s > bound || s < -bound || s > INT32_MAX || s < INT32_MIN)
            bad |= 1;
        acc[i] = (int32_t)s;
    }
    if (bad & 2)
        return -2;
    return (bad & 1) ? -1 : 0;
}

int oracle_contract(const int8_t *xq, const int8_t *q, int64_t m, int64_t n, int64_t k,
                    int32_t *acc)
{
    return contract_bounded(xq, q, m, n, k, 127, acc);
}

/* Same contraction for an explicit list of (row, col) output positions, for
 * sampled checks of shapes too large to contract in full. */
int oracle_contract_pairs(const int8_t *xq, const int8_t *q_rows, int64_t k,
                          const int64_t *row_of_pair, const int64_t *qrow_of_pair,
                          int64_t npairs, int32_t *acc)
{
    int bad = 0;
    const int64_t bound = 127 * k;
    int64_t p;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (p = 0; p < npairs; ++p) {
        const int64_t s = ternary_dot(xq + row_of_pair[p] * k, q_rows + qrow_of_pair[p] * k, k, &bad);
        if (s > bound || s < -bound)
            bad |= 1;
        acc[p] = (int32_t)s;
    }
    if (bad & 2)
        return -2;
    return (bad & 1) ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* O7: de-quantization  [P4, Mathematical Mechanism, item 4]            */
/* ------------------------------------------------------------------ */

/* y[i][j] = acc[i][j] * (gamma * a'_i / 127), evaluated in binary64 and
 * rounded once to binary32. */
void oracle_dequant(const int32_t *acc, int64_t m, int64_t n, float gamma, const float *amax,
                    float *y)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j)
            y[i * n + j] =
                (float)((double)acc[i * n + j] * (double)gamma * (double)amax[i] / 127.0);
    }
}

/* ------------------------------------------------------------------ */
/* SwiGLU between gate+up and down  [P5, Deep Look: the block's ffn]    */
/* ------------------------------------------------------------------ */

/* h[i] = silu(g[i]) * u[i] with silu(g) = g / (1 + exp(-g)), in binary64,
 * rounded once to binary32.  g, u, h: fp32, count values each. */
void oracle_swiglu(const float *g, const float *u, int64_t count, float *h)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i) {
        const double gd = (double)g[i];
        h[i] = (float)(gd * (double)u[i] / (1.0 + exp(-gd)));
    }
}

/* ================================================================== */
/* Variant modes the pages describe beside the main path               */
/* ================================================================== */

/* ------------------------------------------------------------------ */
/* V1: per-tensor activation quantization, Q_b = 128                    */
/*   [P5, "BitNet 1-bit LLM Inference Framework", "A Deep Look at the    */
/*    BitNet Architecture", "The Core Structure of BitNet b1.58": the    */
/*    BitLinear class's activation_quantize and its de-quantization]    */
/* ------------------------------------------------------------------ */

/* One scale for the whole [m][k] tensor: g = max |x| over every element;
 * each code is the binary32 value (x * 128) / (g + 1e-8) (one multiply, one
 * IEEE divide; 1e-8 added to g in binary32), clamped to [-128, 127] first
 * and then rounded half to even.  gx receives g itself (the listing returns
 * the max, without the epsilon, as the de-quantization scale). */
void oracle_quant_act_tensor(const uint16_t *x, int64_t m, int64_t k, int8_t *xq, float *gx)
{
    float g = 0.0f;
    for (int64_t i = 0; i < m * k; ++i) {
        const float v = fabsf(bf16_to_f32(x[i]));
        if (v > g)
            g = v;
    }
    const float d = g + 1e-8f;
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < m * k; ++i) {
        const float t = (bf16_to_f32(x[i]) * 128.0f) / d;
        xq[i] = (int8_t)round_half_even((float)clip((double)t, -128.0, 127.0));
    }
    *gx = g;
}

/* y = acc * gamma * g / 2^7 (the listing's de-quantization), binary64,
 * rounded once to binary32. */
void oracle_dequant_tensor(const int32_t *acc, int64_t m, int64_t n, float gamma, float gx, float *y)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < m * n; ++i)
        y[i] = (float)((double)acc[i] * (double)gamma * (double)gx / 128.0);
}

/* Contraction of codes in [-128, 127] (the V1 range): as oracle_contract,
 * with the bound |acc| <= 128 * k. */
int oracle_contract_q128(const int8_t *xq, const int8_t *q, int64_t m, int64_t n, int64_t k,
                         int32_t *acc)
{
    return contract_bounded(xq, q, m, n, k, 128, acc);
}

/* ------------------------------------------------------------------ */
/* V2: per-output-channel FP16 scales                                  */
/*   [P2, "BitNet-2B-4T: Inside the 2B-Parameter, 4T-Token 1-Bit LLM",   */
/*    "Weight Representation: Ternary + Scale, Not Pure Binary": W_bit   */
/*    times s with one FP16 scale per output channel]                    */
/* ------------------------------------------------------------------ */

/* Ties-to-even rounding of a binary64 value below 2^52 (written out from
 * the definition, as round_half_even). */
static double rne_double(double v)
{
    const double below = floor(v);
    const double rest = v - below; /* exact */
    if (rest != 0.5)
        return rest < 0.5 ? below : below + 1.0;
    return fmod(below, 2.0) != 0.0 ? below + 1.0 : below; /* tie: even neighbour */
}

/* IEEE 754 binary16 encoding of a binary32 value, round to nearest, ties to
 * even: 1 sign, 5 exponent (bias 15) and 10 fraction bits; subnormals are
 * multiples of 2^-24; magnitudes from 65520 (halfway between the largest
 * finite 65504 and 2^16) round to infinity. */
uint16_t oracle_f32_to_f16(float f)
{
    const uint16_t sign = signbit(f) ? 0x8000u : 0u;
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    const double a = fabs((double)f);
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7C00u);
    if (a < 6.103515625e-05) { /* below 2^-14: subnormal quantum 2^-24 */
        const double q = rne_double(a * 16777216.0);
        return (uint16_t)(sign | (uint16_t)q); /* q = 1024 encodes 2^-14 itself */
    }
    int e;
    (void)frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): unbiased exponent e - 1 */
    e -= 1;
    double q = rne_double(ldexp(a, 10 - e)); /* 1024 .. 2048 */
    if (q >= 2048.0) {
        q = 1024.0;
        e += 1;
    }
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0));
}

/* Decode binary16 bits (exact in binary32). */
float oracle_f16_to_f32(uint16_t h)
{
    const int e = (h >> 10) & 31;
    const int frac = h & 1023;
    double v;
    if (e == 31)
        v = frac ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)frac, -24);
    else
        v = ldexp((double)(frac + 1024), e - 25);
    return (float)((h & 0x8000u) ? -v : v);
}

/* Reading: the scale of output channel r is that row's absmean (the main
 * path's gamma rule applied to one row: binary64 sum left to right, divided
 * by k, rounded once to binary32), stored as binary16. */
void oracle_row_scales(const float *w, int64_t n, int64_t k, uint16_t *s16)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        double s = 0.0;
        for (int64_t c = 0; c < k; ++c)
            s += fabs((double)w[r * k + c]);
        s16[r] = oracle_f32_to_f16((float)(s / (double)k));
    }
}

/* Row r is ternarized with its stored scale: q = Clip(Round(W / (s_r + 1e-5)),
 * -1, 1), s_r the binary16 value widened to binary32, eps added in binary32,
 * one binary32 divide per weight. */
void oracle_ternarize_rows(const float *w, int64_t n, int64_t k, const uint16_t *s16, int8_t *q)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        const float denom = oracle_f16_to_f32(s16[r]) + 1e-5f;
        for (int64_t c = 0; c < k; ++c)
            q[r * k + c] = ternary_code(w[r * k + c], denom);
    }
}

/* y[i][j] = acc[i][j] * s_j * a'_i / 127 (binary64, rounded once). */
void oracle_dequant_rows(const int32_t *acc, int64_t m, int64_t n, const uint16_t *s16,
                         const float *amax, float *y)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j)
            y[i * n + j] = (float)((double)acc[i * n + j] * (double)oracle_f16_to_f32(s16[j]) *
                                   (double)amax[i] / 127.0);
    }
}

/* ------------------------------------------------------------------ */
/* V3: binary +-1 weights with a per-layer scale                        */
/*   [P1, "BitNet's 1-Bit Transformer: Architecture Breakdown", "Binary  */
/*    Weight Matrices with Learnable Scaling": W_bit = s * sign(W)]      */
/* ------------------------------------------------------------------ */

/* b = sign(W) with zero taken as +1 (a reading: one bit per weight leaves no
 * code for 0), i.e. -1 exactly where W < 0.  The scale s is learned, not
 * derived from W; it enters only the de-quantization (oracle_dequant with
 * gamma = s). */
void oracle_binarize(const float *w, int64_t n, int64_t k, int8_t *b)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n * k; ++i)
        b[i] = (int8_t)(w[i] < 0.0f ? -1 : 1);
}

/* Number of OpenMP threads the oracle runs with (reported by the benchmark). */
int oracle_num_threads(void)
{
    int t = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        t = omp_get_num_threads();
    }
#endif
    return t;
}
