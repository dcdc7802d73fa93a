/*
 * Layerwise QK-Norm oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library. The product
 * (the HIP library and its Python binding) never calls it, and the two share
 * no code: this file includes nothing from the product tree.
 *
 * What it computes (one RMSNorm per token and per tensor, applied to the FULL
 * projected vector of width H):
 *
 *   RMSNorm(x) = x / sqrt( (1/H) * sum_{j=1..H} x_j^2 + eps ) (.) gamma
 *
 * Source: "SwiftQK: Fast and Communication-Efficient Tensor Parallelism for
 * Query-Key Normalization", Section II-A, Eq. (1) (the letter's rendering is
 * garbled); the same Eq. (1) in the reading notes "SwiftQK：当归一化层成为张量
 * 并行的瓶颈", Section 2, which prints it cleanly. The letter states that the
 * sharded computation preserves the global normalization semantics
 * (Section III-A, Section V) and measures precision against an FP64 RMSNorm
 * of the gathered vector (Section IV-C); this file is that FP64 RMSNorm.
 *
 * The per-shard partial sums of squares (Algorithm 1, Phase A; the notes'
 * worked example, Eqs. (3)-(4)) are provided for the split API:
 *
 *   p[k][t] = sum_{j in shard k} x[t][j]^2,   shard k = columns [k*H/N, (k+1)*H/N)
 *
 * The contiguous equal split is the column-parallel split of the projection
 * (letter, Section II-B) and is the split of the notes' worked example
 * (Section 4b: the first GPU holds the first four elements).
 *
 * Decoding of stored inputs is exact: a bf16 value is the upper 16 bits of
 * an IEEE binary32 value; binary32 -> binary64 is exact. eps is received as
 * binary32 (the value the GPU library receives) and promoted exactly.
 *
 * FP8 activations (the letter evaluates FP8-E4M3 next to BF16 and accumulates
 * in FP32 for both, Section IV-C): an E4M3 code is decoded exactly from the
 * OCP 8-bit floating point format (OFP8, revision 1.0), E4M3 encoding:
 * sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
 * holds zero and subnormals m * 2^-9; no infinities; S.1111.111 is NaN, so
 * the largest finite magnitude is S.1111.110 = 448. With E4M3 activations the
 * scale gamma is bf16 (the format of the layer's weights).
 *
 * No blocking, fusion or reordering: each sum is a plain left-to-right loop
 * in binary64 (relative error <= H * 2^-53).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double decode_bf16(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double decode_f32(float v)
{
    return (double)v;
}

static double decode_e4m3(uint8_t code)
{
    const int sign = code >> 7;
    const int expo = (code >> 3) & 15;
    const int mant = code & 7;
    double mag;
    if (expo == 15 && mant == 7)
        mag = NAN;
    else if (expo == 0)
        mag = ldexp((double)mant, -9);                 /* subnormal: m/8 * 2^(1-7) */
    else
        mag = ldexp(1.0 + (double)mant / 8.0, expo - 7);
    return sign ? -mag : mag;
}

/* input format codes: 0 = bf16 (uint16_t bit patterns), 1 = fp32,
 * 2 = E4M3 codes (uint8_t); the scale gamma is bf16 for format 2 and has the
 * format of x otherwise */
static double load(const void* base, int dtype, int64_t i)
{
    if (dtype == 0)
        return decode_bf16(((const uint16_t*)base)[i]);
    if (dtype == 2)
        return decode_e4m3(((const uint8_t*)base)[i]);
    return decode_f32(((const float*)base)[i]);
}

static int gamma_format(int dtype)
{
    return dtype == 2 ? 0 : dtype;
}

static int format_ok(int dtype)
{
    return dtype == 0 || dtype == 1 || dtype == 2;
}

/*
 * RMSNorm of T rows of width H (row-major, row stride H).
 *   x      [T][H]  input values (bf16 bits, fp32 or E4M3 codes)
 *   gamma  [H]     scale (format of x; bf16 bits when x is E4M3)
 *   eps            binary32 epsilon, promoted exactly
 * Outputs (any may be NULL):
 *   y      [T][H]  x / sqrt(S/H + eps) * gamma, unrounded binary64
 *   sumsq  [T]     S = sum_j x_j^2
 *   rinv   [T]     1 / sqrt(S/H + eps)
 * Returns 0, or -1 on a bad argument.
 */
int oracle_rmsnorm(const void* x, const void* gamma, int dtype, int64_t T, int64_t H,
                   float eps, double* y, double* sumsq, double* rinv)
{
    if (!x || (y && !gamma) || T < 0 || H < 1 || !format_ok(dtype))
        return -1;
    const double e = (double)eps;
    for (int64_t t = 0; t < T; ++t) {
        double S = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = load(x, dtype, t * H + j);
            S += v * v;
        }
        double denom = sqrt(S / (double)H + e);
        if (sumsq)
            sumsq[t] = S;
        if (rinv)
            rinv[t] = 1.0 / denom;
        if (y) {
            for (int64_t j = 0; j < H; ++j) {
                double v = load(x, dtype, t * H + j);
                double g = load(gamma, gamma_format(dtype), j);
                y[t * H + j] = v / denom * g;
            }
        }
    }
    return 0;
}

/*
 * Per-shard partial sums of squares, shard-major: p[k*T + t] for k = 0..N-1.
 * Requires H % N == 0 (equal contiguous shards). Returns 0, or -1.
 */
int oracle_shard_sumsq(const void* x, int dtype, int64_t T, int64_t H, int n_shards,
                       double* p)
{
    if (!x || !p || T < 0 || H < 1 || n_shards < 1 || H % n_shards != 0 || !format_ok(dtype))
        return -1;
    const int64_t W = H / n_shards;
    for (int k = 0; k < n_shards; ++k) {
        for (int64_t t = 0; t < T; ++t) {
            double s = 0.0;
            for (int64_t j = k * W; j < (k + 1) * W; ++j) {
                double v = load(x, dtype, t * H + j);
                s += v * v;
            }
            p[(int64_t)k * T + t] = s;
        }
    }
    return 0;
}

/* Exact value of each of n E4M3 codes (for the tests of the decoder). */
int oracle_decode_e4m3(const uint8_t* codes, int64_t n, double* out)
{
    if (!codes || !out || n < 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = decode_e4m3(codes[i]);
    return 0;
}

/*
 * LayerNorm of T rows of width H (the extension of the method to a norm with
 * two additive statistics, reading notes Section 5e: mean and variance of the
 * whole vector, from sum x and sum x^2 of every shard):
 *
 *   mu = (1/H) sum_j x_j,   var = (1/H) sum_j (x_j - mu)^2,
 *   y_j = (x_j - mu) / sqrt(var + eps) * gamma_j + beta_j
 *
 * computed here by the definition, two passes in binary64 (mean, then the
 * centred sum of squares), not by the sum / sum-of-squares identity.
 *   x      [T][H]  input values (format as for oracle_rmsnorm)
 *   gamma  [H]     scale, beta [H] shift (NULL = no shift), format of x
 * Outputs (any may be NULL): y [T][H] unrounded, mean [T], rstd [T] = 1/sqrt(var+eps).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_layernorm(const void* x, const void* gamma, const void* beta, int dtype, int64_t T,
                     int64_t H, float eps, double* y, double* mean, double* rstd)
{
    if (!x || (y && !gamma) || T < 0 || H < 1 || !format_ok(dtype))
        return -1;
    const double e = (double)eps;
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int64_t j = 0; j < H; ++j)
            s += load(x, dtype, t * H + j);
        const double mu = s / (double)H;
        double c = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            const double d = load(x, dtype, t * H + j) - mu;
            c += d * d;
        }
        const double denom = sqrt(c / (double)H + e);
        if (mean)
            mean[t] = mu;
        if (rstd)
            rstd[t] = 1.0 / denom;
        if (y) {
            for (int64_t j = 0; j < H; ++j) {
                const double v = load(x, dtype, t * H + j);
                const double g = load(gamma, gamma_format(dtype), j);
                const double b = beta ? load(beta, gamma_format(dtype), j) : 0.0;
                y[t * H + j] = (v - mu) / denom * g + b;
            }
        }
    }
    return 0;
}

/*
 * The two additive statistics of every shard, shard-major:
 *   sums[k*T + t] = sum_{j in shard k} x[t][j],  sumsq[k*T + t] = sum x[t][j]^2.
 * Requires H % N == 0. Returns 0, or -1.
 */
int oracle_shard_stats(const void* x, int dtype, int64_t T, int64_t H, int n_shards,
                       double* sums, double* sumsq)
{
    if (!x || !sums || !sumsq || T < 0 || H < 1 || n_shards < 1 || H % n_shards != 0 ||
        !format_ok(dtype))
        return -1;
    const int64_t W = H / n_shards;
    for (int k = 0; k < n_shards; ++k) {
        for (int64_t t = 0; t < T; ++t) {
            double a = 0.0, b = 0.0;
            for (int64_t j = k * W; j < (k + 1) * W; ++j) {
                const double v = load(x, dtype, t * H + j);
                a += v;
                b += v * v;
            }
            sums[(int64_t)k * T + t] = a;
            sumsq[(int64_t)k * T + t] = b;
        }
    }
    return 0;
}

/*
 * Headwise RMSNorm: one factor per attention head instead of one per vector
 * (letter, Section II-A: headwise QK-Norm normalises each head on its own).
 * Row t of x holds n_heads heads of head_dim columns; head h is columns
 * [h*D, (h+1)*D) and gamma [D] scales every head alike:
 *
 *   y[t][h*D + j] = x[t][h*D + j] / sqrt((1/D) sum_{i<D} x[t][h*D + i]^2 + eps) * gamma[j]
 *
 *   x [T][n_heads*D], gamma [D]; y [T][n_heads*D] unrounded, rinv [T][n_heads]
 *   (either may be NULL). Returns 0, or -1 on a bad argument.
 */
int oracle_headwise(const void* x, const void* gamma, int dtype, int64_t T, int64_t n_heads,
                    int64_t D, float eps, double* y, double* rinv)
{
    if (!x || (y && !gamma) || T < 0 || n_heads < 1 || D < 1 || !format_ok(dtype))
        return -1;
    const double e = (double)eps;
    const int64_t H = n_heads * D;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < n_heads; ++h) {
            double S = 0.0;
            for (int64_t i = 0; i < D; ++i) {
                const double v = load(x, dtype, t * H + h * D + i);
                S += v * v;
            }
            const double denom = sqrt(S / (double)D + e);
            if (rinv)
                rinv[t * n_heads + h] = 1.0 / denom;
            if (y) {
                for (int64_t j = 0; j < D; ++j) {
                    const double v = load(x, dtype, t * H + h * D + j);
                    const double g = load(gamma, gamma_format(dtype), j);
                    y[t * H + h * D + j] = v / denom * g;
                }
            }
        }
    }
    return 0;
}
