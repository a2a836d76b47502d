/*
 * Seeded synthetic inputs for the QAM-W weight codec: weight matrices shaped
 * like LLM projections, per-input-channel scales and training points drawn
 * from the unit circular Gaussian.
 *
 * This module only produces inputs.  It holds none of the codec's arithmetic
 * and is shared, as a data source, by the CPU oracle and the GPU library.
 *
 * Every value is a pure function of (seed, stream id, counter), so any subset
 * of rows can be generated on its own and in any thread order.
 *
 * Random numbers: the splitmix64 output mixer (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; constants as
 * published by Vigna) applied to a Weyl sequence.  Gaussians: Box-Muller
 * (cosine branch).  The logarithm and cosine are written here from their
 * series using only +, -, *, / and sqrt, so the bytes do not depend on the
 * C library.  Build with -ffp-contract=off.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define SX_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t sx_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t sid) { return sx_mix(seed * SX_GOLDEN + sid); }

uint64_t synth_u64(uint64_t key, uint64_t i) { return sx_mix(key + (i + 1) * SX_GOLDEN); }

/* U in [0, 1) with 53 random bits. */
double synth_uniform(uint64_t key, uint64_t i) { return (double)(synth_u64(key, i) >> 11) * 0x1p-53; }

/* Natural log for x in [2^-53, 1]: x = m * 2^e with m in [sqrt(1/2), sqrt(2)),
 * ln m = 2 atanh(t), t = (m-1)/(m+1), |t| < 0.172, series to t^23. */
static double sx_log(double x)
{
    uint64_t bits;
    memcpy(&bits, &x, 8);
    int e = (int)((bits >> 52) & 0x7ff) - 1023;
    bits = (bits & 0x000fffffffffffffULL) | 0x3ff0000000000000ULL;
    double m;
    memcpy(&m, &bits, 8);
    if (m > 1.4142135623730951) {
        m = m * 0.5;
        e += 1;
    }
    double t = (m - 1.0) / (m + 1.0);
    double t2 = t * t;
    double s = 1.0 / 23.0;
    for (int k = 21; k >= 1; k -= 2) s = s * t2 + 1.0 / (double)k;
    return 2.0 * t * s + (double)e * 0.6931471805599453;
}

/* cos(2 pi v) for v in [0, 1): quadrant from 4v (exact), then Taylor series
 * of sin / cos on [0, pi/2). */
static double sx_cos2pi(double v)
{
    double v4 = v * 4.0;
    int q = (int)v4;
    double f = v4 - (double)q;
    double th = f * 1.5707963267948966;
    double th2 = th * th;
    double c = 1.0, ct = 1.0, s = th, st = th;
    for (int k = 1; k <= 13; ++k) {
        ct = -ct * th2 / (double)((2 * k - 1) * (2 * k));
        c = c + ct;
        st = -st * th2 / (double)((2 * k) * (2 * k + 1));
        s = s + st;
    }
    switch (q & 3) {
    case 0: return c;
    case 1: return -s;
    case 2: return -c;
    default: return s;
    }
}

/* Standard normal number q of the stream: Box-Muller on uniforms 2q, 2q+1. */
double synth_gauss(uint64_t key, uint64_t q)
{
    double u1 = synth_uniform(key, 2 * q);
    double u2 = synth_uniform(key, 2 * q + 1);
    double rad = sqrt(-2.0 * sx_log(1.0 - u1));
    return rad * sx_cos2pi(u2);
}

static inline uint16_t sx_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Rows [row0, row0 + nrows) of a d_out x d_in weight matrix, row-major,
 * element (i, j) built from normals with counters (i*d_in + j)*n_norm + t.
 *   dist 0: scale * N(0,1)
 *   dist 1: scale * Student-t(nu): g0 / sqrt((g1^2 + ... + g_nu^2) / nu)
 * Columns with outlier_mask[j] != 0 are multiplied by outlier_factor.
 * Computed in double, rounded to float (RNE), then to bf16 (RNE) when
 * out_bf16 != 0 (out is then uint16 bit patterns). */
void synth_weights(uint64_t seed, uint64_t sid, int64_t row0, int64_t nrows, int32_t d_in,
                   int32_t dist, int32_t nu, double scale, const uint8_t* outlier_mask,
                   double outlier_factor, int32_t out_bf16, void* out)
{
    uint64_t key = synth_key(seed, sid);
    int64_t n_norm = (dist == 1) ? (int64_t)nu + 1 : 1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = row0 + r;
        for (int32_t j = 0; j < d_in; ++j) {
            uint64_t q0 = (uint64_t)((i * d_in + j) * n_norm);
            double g = synth_gauss(key, q0);
            if (dist == 1) {
                double acc = 0.0;
                for (int t = 1; t <= nu; ++t) {
                    double h = synth_gauss(key, q0 + (uint64_t)t);
                    acc = acc + h * h;
                }
                g = g / sqrt(acc / (double)nu);
            }
            double v = scale * g;
            if (outlier_mask && outlier_mask[j]) v = v * outlier_factor;
            float f = (float)v;
            if (out_bf16)
                ((uint16_t*)out)[r * d_in + j] = sx_f32_to_bf16(f);
            else
                ((float*)out)[r * d_in + j] = f;
        }
    }
}

/* n_out distinct columns of [0, d_in): the first n_out entries of a partial
 * Fisher-Yates shuffle driven by the stream. */
void synth_outlier_columns(uint64_t seed, uint64_t sid, int32_t d_in, int32_t n_out, int32_t* cols)
{
    uint64_t key = synth_key(seed, sid);
    int32_t* perm = cols; /* caller buffer has d_in entries */
    for (int32_t j = 0; j < d_in; ++j) perm[j] = j;
    for (int32_t t = 0; t < n_out; ++t) {
        uint64_t span = (uint64_t)(d_in - t);
        int32_t r = t + (int32_t)(synth_u64(key, (uint64_t)t) % span);
        int32_t tmp = perm[t];
        perm[t] = perm[r];
        perm[r] = tmp;
    }
}

/* s_j = fl32(sqrt(|g_j|) + 0.1). */
void synth_channel_scale(uint64_t seed, uint64_t sid, int32_t d_in, float* s)
{
    uint64_t key = synth_key(seed, sid);
    for (int32_t j = 0; j < d_in; ++j) {
        double g = synth_gauss(key, (uint64_t)j);
        s[j] = (float)(sqrt(fabs(g)) + 0.1);
    }
}

/* n points of the unit circular Gaussian, fp32, x and y interleaved. */
void synth_points(uint64_t seed, uint64_t sid, int64_t n, float* xy)
{
    uint64_t key = synth_key(seed, sid);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        xy[2 * i] = (float)synth_gauss(key, (uint64_t)(2 * i));
        xy[2 * i + 1] = (float)synth_gauss(key, (uint64_t)(2 * i + 1));
    }
}
