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
 *        00 = 0, 01 = +1, 10 = -1; conditional add / skip / subtract loop),
 *        and section "The Difference in How Computation Works" (mask form).
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
 *   - RMSNorm: r = 1 / sqrt(mean_k x^2 + eps) per token (binary64), times an
 *     optional per-channel gain w.  Absmax quantization is invariant under a
 *     positive per-token factor, so the codes are those of v = x * w (one
 *     binary32 multiply) and r is carried by the scale instead:
 *     a' = max(max_k |v| * r, 1e-8) (binary64 product, rounded once).  An
 *     all-zero v gives codes 0 and a' = 1e-8;
 *   - SwiGLU: h = silu(g) * u = g * u / (1 + exp(-g)) in binary64, rounded
 *     once to binary32, from the two de-quantized BitLinear outputs;
 *   - h is requantized for the next BitLinear from binary32 with the same
 *     per-token rule as the bf16 activations.
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
void oracle_ternarize(const float *w, int64_t n, int64_t k, float gamma, int8_t *q)
{
    const float denom = gamma + 1e-5f;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        for (int64_t c = 0; c < k; ++c) {
            float t = w[r * k + c] / denom;
            q[r * k + c] = (int8_t)clip(round_half_even(t), -1.0, 1.0);
        }
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

/* x: bf16 bits [m][k]; w: per-channel gain [k] (NULL: all ones); eps added to
 * the mean square.  Codes quantize v = x * w; the factor r = 1/sqrt(mean x^2 +
 * eps), which cancels in the codes, is folded into a'.  rms_out (may be NULL)
 * receives r rounded to binary32. */
void oracle_rmsnorm_quant_act(const uint16_t *x, const float *w, float eps, int64_t m, int64_t k,
                              int8_t *xq, float *amax, float *rms_out)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < m; ++r) {
        double ss = 0.0;
        float a = 0.0f;
        for (int64_t c = 0; c < k; ++c) {
            const float xv = bf16_to_f32(x[r * k + c]);
            ss += (double)xv * (double)xv;
            const float v = fabsf(w ? xv * w[c] : xv);
            if (v > a)
                a = v;
        }
        const double rr = 1.0 / sqrt(ss / (double)k + (double)eps);
        if (rms_out)
            rms_out[r] = (float)rr;
        if (a == 0.0f) {
            for (int64_t c = 0; c < k; ++c)
                xq[r * k + c] = 0;
            amax[r] = 1e-8f;
            continue;
        }
        const float s = 127.0f / a;
        for (int64_t c = 0; c < k; ++c) {
            const float xv = bf16_to_f32(x[r * k + c]);
            const float v = w ? xv * w[c] : xv;
            xq[r * k + c] = (int8_t)clip(round_half_even(v * s), -127.0, 127.0);
        }
        float ap = (float)((double)a * rr);
        amax[r] = ap < 1e-8f ? 1e-8f : ap;
    }
}

/* ------------------------------------------------------------------ */
/* O6: ternary x int8 contraction by add / skip / subtract              */
/*     [P4, Mathematical Mechanism, item 3; P5, How the LUT Kernel Works]*/
/* ------------------------------------------------------------------ */

/* acc[i][j] = sum_k xq[i][k] * q[j][k], computed as: +x where the weight is
 * +1, nothing where it is 0, -x where it is -1.  The sum is kept in int64 and
 * checked against the bound |acc| <= 127 * k before it is stored as int32.
 * Returns 0, or -1 if the bound (or int32 range) is violated, or -2 if a
 * weight is not in {-1, 0, 1}. */
int oracle_contract(const int8_t *xq, const int8_t *q, int64_t m, int64_t n, int64_t k,
                    int32_t *acc)
{
    int bad = 0;
    const int64_t bound = 127 * k;
    int64_t i;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (i = 0; i < m * n; ++i) {
        const int64_t row = i / n, col = i % n;
        const int8_t *a = xq + row * k;
        const int8_t *w = q + col * k;
        int64_t s = 0;
        for (int64_t c = 0; c < k; ++c) {
            if (w[c] == 1)
                s += a[c];
            else if (w[c] == -1)
                s -= a[c];
            else if (w[c] != 0)
                bad |= 2;
        }
        if (s > bound || s < -bound || s > INT32_MAX || s < INT32_MIN)
            bad |= 1;
        acc[i] = (int32_t)s;
    }
    if (bad & 2)
        return -2;
    return (bad & 1) ? -1 : 0;
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
        const int8_t *a = xq + row_of_pair[p] * k;
        const int8_t *w = q_rows + qrow_of_pair[p] * k;
        int64_t s = 0;
        for (int64_t c = 0; c < k; ++c) {
            if (w[c] == 1)
                s += a[c];
            else if (w[c] == -1)
                s -= a[c];
            else if (w[c] != 0)
                bad |= 2;
        }
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
