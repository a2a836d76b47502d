/*
 * CPU oracle for the QAM-W weight codec -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow implementation written to be checked by eye against the paper
 * "QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard Rotation
 * and Activation-Aware Scaling" (Sharma and Dobek):
 *   - explicit b x b Hadamard matrices (no fast transform),
 *   - brute-force nearest-codeword search over every codeword,
 *   - double precision everywhere the paper does not fix a precision.
 * Only tests/, the package smoke check and the benchmark's CPU-baseline leg
 * use it; the GPU library shares no code with it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (no FMA contraction, IEEE
 * single and double operations, round-to-nearest-even).
 *
 * Readings where the paper is silent (each is also listed in the design
 * notes of the repository):
 *   R1 sign mask: the functions below take it as bits, eps_j = -1 where bit j is
 *      set; the bits are drawn from a 64-bit seed by oracle_sign_mask (section
 *      3.3 only calls the mask deterministic): eps_j = -1 when the top bit of
 *      the (j+1)-th output of the splitmix64 generator started at the seed is
 *      set.  Rotation y = blockdiag(H_b) (eps . u), H_b in Sylvester order.
 *   R2 sigma_k: mean |z_k| over the non-zero, finite rows among those passed
 *      (the caller passes the first min(d_out, 1024) rows), in double, then
 *      divided by sqrt(pi/2) and rounded to float; fallback 1/sqrt(d_in).
 *   R3 pairs p_k = fl32(y_2k / sigma_k), fl32(y_2k+1 / sigma_k), division in
 *      double; distances in float, each operation rounded:
 *      D = fl32(fl32(dx*dx) + fl32(dy*dy)), dx = fl32(px - cx); ties go to
 *      the lowest codeword index.
 *   R4 row norm stored as f16(fl32(r)) with round-to-nearest-even; the row
 *      is normalized by the double r.  A row with r == 0 is a zero row: norm
 *      0 and every index 0.
 *   R5 packing: bit t of index k is stream bit k*B + t, stream bit q is bit
 *      q%8 of byte q/8 (LSB first); each row starts on a 16-byte boundary.
 *   R6 channel scale: multiplied in before the norm at encode, divided out
 *      after the inverse rotation at decode.
 *   R7 Lloyd on a sample of points: first K points as the start, empty cells
 *      keep their centroid, sums kept as 64-bit integers of x*2^32 so that
 *      the result does not depend on summation order.
 *   R8 polar baseline (section 3.5): the magnitude quantizer is the Na-level
 *      Lloyd-Max quantizer of the unit Rayleigh density r exp(-r^2/2), started
 *      from the conditional means of Na equal-probability intervals and
 *      iterated (thresholds at the midpoints of adjacent levels, levels at the
 *      conditional means of their intervals, integrals in closed form) until
 *      no level moves by more than 1e-15 of itself, at most 10000 times.  A
 *      pair's magnitude index is the number of thresholds t with
 *      fl64(px^2 + py^2) > fl64(t^2) (the squares of the float pair are exact
 *      in double; ties go to the lower level).  Its phase index is
 *      floor(atan2(py, px) * Np / (2 pi) + 1/2) mod Np, the bin centred on
 *      2 pi j / Np; a pair at the origin (either sign of zero) has phase
 *      index 0, since the sign of a zero out of the transform depends on the
 *      order of its additions, which the method leaves open.  The pair's
 *      B = Ba + Bp bit index is ia + Na * ip, and the
 *      decoder is the QAM-W decoder with the table
 *      c[ia + Na ip] = fl32(a_ia cos(2 pi ip / Np)), fl32(a_ia sin(2 pi ip / Np)).
 *   R10 scalar (d = 1) ablation (section 2, the PolarQuant comparison): the
 *      same front end, then each coordinate of the scaled pair is coded alone
 *      with the L = 2^b level Lloyd-Max quantizer of the standard normal
 *      density (the law of each coordinate of a unit circular Gaussian pair),
 *      b bits per coordinate, B = 2b per pair.  The start is the conditional
 *      means of L equal-probability cells, whose edges are the normal
 *      quantiles found by bisection; the iteration and its stopping rule are
 *      those of R8.  A coordinate's index is the number of thresholds t with
 *      t < fl64(p) (ties to the lower level); the pair's index is ix + L iy,
 *      and the decoder is the QAM-W decoder with the product table
 *      c[ix + L iy] = (fl32(a_ix), fl32(a_iy)).
 *   R11 activation-aware channel scale (section 1 and the summary of the
 *      AWQ-style scaling): s_j = fl32(r_j^alpha), r_j the RMS of input channel j
 *      over the calibration activations, sqrt(sum_t x_tj^2 / T) in fp64; a
 *      channel that is zero over the batch gets s_j = 1 (its weights never
 *      reach the output, any positive scale serves).  The pages state s_j only
 *      up to a constant; a global factor cancels between the row norm and the
 *      decoder's division by s, so the constant 1 is taken.
 */
#include "qamw_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_PI 3.14159265358979323846

/* ------------------------------------------------------------------------
 * Number formats.  A finite x is rounded to the nearest value with
 * `mant_bits` fraction bits and minimum normal exponent `emin`, ties to even,
 * by scaling with powers of two (exact) and rint() in the default
 * round-to-nearest-even mode.
 * ------------------------------------------------------------------------ */
static double round_to_format(double x, int mant_bits, int emin)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(fabs(x), &e); /* |x| = f * 2^e, f in [0.5, 1): leading bit weight 2^(e-1) */
    int lead = e - 1;
    if (lead < emin) lead = emin; /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, lead - mant_bits);
    return rint(x / quantum) * quantum;
}

/* IEEE binary16: 10 fraction bits, emin -14, largest finite 65504. */
uint16_t oracle_f16_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    double x = fabs((double)f);
    if (isnan(f)) return 0x7e00;
    double r = isinf(f) ? INFINITY : round_to_format(x, 10, -14);
    if (r > 65504.0) return (uint16_t)(sign | 0x7c00u);
    if (r == 0.0) return sign;
    int e;
    double fr = frexp(r, &e); /* r = fr * 2^e */
    int lead = e - 1;
    if (lead < -14) { /* subnormal: r = m * 2^-24 */
        uint16_t m = (uint16_t)ldexp(r, 24);
        return (uint16_t)(sign | m);
    }
    uint16_t m = (uint16_t)(ldexp(fr, 11) - 1024.0);
    return (uint16_t)(sign | ((uint16_t)(lead + 15) << 10) | m);
}

float oracle_f32_from_f16(uint16_t h)
{
    int sign = (h >> 15) & 1, ex = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (ex == 0) v = ldexp((double)m, -24);
    else if (ex == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1024.0 + m, ex - 25);
    return (float)(sign ? -v : v);
}

/* bfloat16: 7 fraction bits, the exponent range of float. */
uint16_t oracle_bf16_from_f32(float f)
{
    if (isnan(f)) return 0x7fc0;
    double r = round_to_format((double)f, 7, -126);
    float fr;
    if (fabs(r) > 3.3895313892515355e38) /* beyond the largest finite bf16 */
        fr = (r > 0) ? INFINITY : -INFINITY;
    else
        fr = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &fr, 4);
    if (f == 0.0f) memcpy(&u, &f, 4); /* keep the sign of zero */
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------
 * Rotation (paper section 3.3, Lemma 1 in section 4): sign-masked block
 * Hadamard.  H_b[i][k] = (-1)^popcount(i & k) / sqrt(b), Sylvester order.
 * ------------------------------------------------------------------------ */
void oracle_hadamard(int32_t b, double* H)
{
    double scale = 1.0 / sqrt((double)b);
    for (int i = 0; i < b; ++i)
        for (int k = 0; k < b; ++k) H[(size_t)i * b + k] = (__builtin_popcount(i & k) & 1) ? -scale : scale;
}

/* Section 3.3: the largest power of two dividing d_in, at most 1024. */
int32_t oracle_default_block(int32_t d_in)
{
    if (d_in <= 0) return 0;
    int32_t b = 1;
    while (b < 1024 && d_in % (2 * b) == 0) b *= 2;
    return b;
}

/* Section 3.7, eq. 3: B bits per pair (two weights) plus 16 bits per row. */
double oracle_bpw(int32_t d_in, int32_t bits) { return bits / 2.0 + 16.0 / d_in; }

/* Section 3.7: row-level packing and alignment (reading R5). */
size_t oracle_row_stride(int32_t d_in, int32_t bits)
{
    size_t used = ((size_t)(d_in / 2) * (size_t)bits + 7) / 8;
    return (used + 15) / 16 * 16;
}

/* ------------------------------------------------------------------------
 * The sign mask (section 3.3, reading R1).  splitmix64 (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014, with
 * the constants of Vigna's reference code): the state advances by the golden
 * gamma 0x9E3779B97F4A7C15 and each output is the new state passed through the
 * finalizer below, all modulo 2^64.
 * ------------------------------------------------------------------------ */
void oracle_splitmix64(uint64_t seed, int64_t n, uint64_t* out)
{
    uint64_t state = seed;
    for (int64_t t = 0; t < n; ++t) {
        state += 0x9E3779B97F4A7C15ULL;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
        out[t] = z ^ (z >> 31);
    }
}

/* Bit j % 32 of word j / 32 is set when eps_j = -1, i.e. when output j + 1 of
 * the generator started at `seed` has its top bit set (0 <= j < d_in). */
void oracle_sign_mask(uint64_t seed, int32_t d_in, uint32_t* bits)
{
    int32_t nw = (d_in + 31) / 32;
    for (int32_t w = 0; w < nw; ++w) bits[w] = 0;
    uint64_t* z = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)(d_in > 0 ? d_in : 1));
    oracle_splitmix64(seed, d_in, z);
    for (int32_t j = 0; j < d_in; ++j)
        if (z[j] >> 63) bits[j >> 5] |= 1u << (j & 31);
    free(z);
}

static double eps_of(const uint32_t* sign_bits, int j)
{
    return ((sign_bits[j >> 5] >> (j & 31)) & 1u) ? -1.0 : 1.0;
}

static double weight_at(const void* w, int w_bf16, int64_t row, int64_t ld, int j)
{
    if (w_bf16) {
        uint32_t u = (uint32_t)((const uint16_t*)w)[row * ld + j] << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    return (double)((const float*)w)[row * ld + j];
}

static int check_block(int32_t d_in, int32_t block)
{
    if (d_in <= 0 || (d_in & 1) || block < 2 || block > 1024 || (block & (block - 1)) || d_in % block)
        return -1;
    return 0;
}

static int32_t scale_flags(const float* s, int32_t d_in)
{
    for (int j = 0; j < d_in; ++j)
        if (!(s[j] > 0.0f)) return ORACLE_FLAG_BAD_SCALE;
    return 0;
}

/* Section 3.1 steps 1-2 for one row: a = w . s (channel scale, section 3.8),
 * r = ||a||_2, u = a / r, y = R_fwd u = blockdiag(H_b) (eps . u).
 * Returns the flags of the row; y is left zero for a zero row. */
static int32_t front_end_row(const void* w, int w_bf16, int64_t row, int32_t d_in, int64_t ld,
                             const float* s, const uint32_t* sign_bits, int32_t block,
                             const double* H, double* a, double* y, double* r_out)
{
    int32_t flags = 0;
    for (int j = 0; j < d_in; ++j) {
        a[j] = weight_at(w, w_bf16, row, ld, j) * (double)s[j];
        if (!isfinite(a[j])) flags |= ORACLE_FLAG_NONFINITE;
    }
    double r2 = 0.0;
    for (int j = 0; j < d_in; ++j) r2 += a[j] * a[j];
    double r = sqrt(r2);
    if (!isfinite(r)) flags |= ORACLE_FLAG_NONFINITE;
    *r_out = r;
    for (int j = 0; j < d_in; ++j) y[j] = 0.0;
    if (r == 0.0 || !isfinite(r)) return flags;
    for (int j = 0; j < d_in; ++j) a[j] = eps_of(sign_bits, j) * (a[j] / r); /* v = eps . u */
    for (int t = 0; t < d_in / block; ++t) {
        const double* v = a + (size_t)t * block;
        double* yt = y + (size_t)t * block;
        for (int i = 0; i < block; ++i) {
            double acc = 0.0;
            for (int k = 0; k < block; ++k) acc += H[(size_t)i * block + k] * v[k];
            yt[i] = acc;
        }
    }
    return flags;
}

int oracle_front_end(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                     const float* s, const uint32_t* sign_bits, int32_t block, double* y, double* r,
                     int32_t* status)
{
    if (check_block(d_in, block) || ld < d_in || n_rows < 0) return -1;
    double* H = malloc(sizeof(double) * (size_t)block * block);
    oracle_hadamard(block, H);
    int32_t flags = scale_flags(s, d_in);
#pragma omp parallel for schedule(dynamic, 4) reduction(| : flags)
    for (int64_t i = 0; i < n_rows; ++i) {
        double* a = malloc(sizeof(double) * (size_t)d_in);
        flags |= front_end_row(w, w_bf16, i, d_in, ld, s, sign_bits, block, H, a, y + i * d_in, r + i);
        free(a);
    }
    free(H);
    if (status) *status |= flags;
    return 0;
}

/* Section 3.4, eq. 1: sigma_k = mean(|z_k|) / sqrt(pi/2) over at most 1024
 * unit-normalized rows (reading R2). */
int oracle_calibrate(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                     const float* s, const uint32_t* sign_bits, int32_t block, float* sigma,
                     int32_t* status)
{
    if (check_block(d_in, block) || n_rows < 0) return -1;
    double* y = malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1) * d_in);
    double* r = malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1));
    int rc = oracle_front_end(w, w_bf16, n_rows, d_in, ld, s, sign_bits, block, y, r, status);
    if (rc) {
        free(y);
        free(r);
        return rc;
    }
    int n_pairs = d_in / 2;
    double* sum = calloc((size_t)n_pairs, sizeof(double));
    int64_t n_nz = 0;
    for (int64_t i = 0; i < n_rows; ++i) {
        if (!(r[i] > 0.0) || !isfinite(r[i])) continue;
        ++n_nz;
        const double* yi = y + i * d_in;
        for (int k = 0; k < n_pairs; ++k) sum[k] += sqrt(yi[2 * k] * yi[2 * k] + yi[2 * k + 1] * yi[2 * k + 1]);
    }
    double rayleigh_mean = sqrt(ORACLE_PI / 2.0); /* E|z| = sigma sqrt(pi/2) */
    for (int k = 0; k < n_pairs; ++k) {
        double m = (n_nz > 0) ? sum[k] / (double)n_nz : 0.0;
        sigma[k] = (m > 0.0) ? (float)(m / rayleigh_mean) : (float)(1.0 / sqrt((double)d_in));
    }
    free(sum);
    free(y);
    free(r);
    return 0;
}

/* Section 3.6: the Euclidean-nearest codeword, by trying every codeword
 * (reading R3 for the float distance and the tie rule). */
int32_t oracle_nearest(float px, float py, const float* cb, int32_t K, float* dist)
{
    int32_t best = 0;
    float best_d = INFINITY;
    for (int32_t j = 0; j < K; ++j) {
        float dx = px - cb[2 * j];
        float dy = py - cb[2 * j + 1];
        float dx2 = dx * dx;
        float dy2 = dy * dy;
        float d = dx2 + dy2;
        if (d < best_d) {
            best_d = d;
            best = j;
        }
    }
    if (dist) *dist = best_d;
    return best;
}

void oracle_nearest_many(const float* p, int64_t n, const float* cb, int32_t K, int32_t* idx, float* dist)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) idx[i] = oracle_nearest(p[2 * i], p[2 * i + 1], cb, K, dist ? dist + i : NULL);
}

/* Section 3.1 step 6: bit-packed index stream (reading R5). */
void oracle_pack_row(const int32_t* idx, int32_t n_pairs, int32_t bits, uint8_t* out, size_t stride)
{
    memset(out, 0, stride);
    for (int32_t k = 0; k < n_pairs; ++k)
        for (int32_t t = 0; t < bits; ++t)
            if ((idx[k] >> t) & 1) {
                size_t q = (size_t)k * bits + t;
                out[q / 8] |= (uint8_t)(1u << (q % 8));
            }
}

void oracle_unpack_row(const uint8_t* in, int32_t n_pairs, int32_t bits, int32_t* idx)
{
    for (int32_t k = 0; k < n_pairs; ++k) {
        int32_t v = 0;
        for (int32_t t = 0; t < bits; ++t) {
            size_t q = (size_t)k * bits + t;
            v |= ((in[q / 8] >> (q % 8)) & 1) << t;
        }
        idx[k] = v;
    }
}

/* ------------------------------------------------------------------------
 * Section 3.5: the polar baseline (reading R8). */

/* Integrals of the unit Rayleigh density over [a, b] (b may be infinite):
 * mass = exp(-a^2/2) - exp(-b^2/2);
 * first moment = a exp(-a^2/2) - b exp(-b^2/2) + sqrt(pi/2) (erf(b/sqrt2) - erf(a/sqrt2)). */
static double rayleigh_mass(double a, double b)
{
    return exp(-0.5 * a * a) - (isinf(b) ? 0.0 : exp(-0.5 * b * b));
}
static double rayleigh_moment(double a, double b)
{
    double hi = isinf(b) ? 0.0 : b * exp(-0.5 * b * b);
    double eb = isinf(b) ? 1.0 : erf(b / sqrt(2.0));
    return a * exp(-0.5 * a * a) - hi + sqrt(0.5 * ORACLE_PI) * (eb - erf(a / sqrt(2.0)));
}

int oracle_rayleigh_lloyd_max(int32_t ba, double* levels, double* thresholds)
{
    if (ba < 0 || ba > 8) return -1;
    int32_t na = 1 << ba;
    /* start: conditional means of na equal-probability intervals, edges at the
     * quantiles sqrt(-2 ln(1 - i/na)) */
    for (int i = 0; i < na; ++i) {
        double a = sqrt(-2.0 * log(1.0 - (double)i / na));
        double b = (i + 1 == na) ? INFINITY : sqrt(-2.0 * log(1.0 - (double)(i + 1) / na));
        levels[i] = rayleigh_moment(a, b) / rayleigh_mass(a, b);
    }
    for (int it = 0; it < 10000; ++it) {
        for (int i = 0; i + 1 < na; ++i) thresholds[i] = 0.5 * (levels[i] + levels[i + 1]);
        int moved = 0;
        for (int i = 0; i < na; ++i) {
            double a = (i == 0) ? 0.0 : thresholds[i - 1];
            double b = (i + 1 == na) ? INFINITY : thresholds[i];
            double v = rayleigh_moment(a, b) / rayleigh_mass(a, b);
            if (fabs(v - levels[i]) > 1e-15 * levels[i]) moved = 1;
            levels[i] = v;
        }
        if (!moved) break;
    }
    for (int i = 0; i + 1 < na; ++i) thresholds[i] = 0.5 * (levels[i] + levels[i + 1]);
    return 0;
}

int32_t oracle_polar_index(float px, float py, int32_t ba, int32_t bp, const double* thresholds)
{
    int32_t na = 1 << ba, np_ = 1 << bp;
    double r2 = (double)px * px + (double)py * py;
    int32_t ia = 0;
    for (int i = 0; i + 1 < na; ++i)
        if (r2 > thresholds[i] * thresholds[i]) ia = i + 1;
    int32_t ip = 0;
    if (r2 > 0.0) {
        double th = atan2((double)py, (double)px);
        ip = (int32_t)floor(th * np_ / (2.0 * ORACLE_PI) + 0.5);
        ip = ((ip % np_) + np_) % np_;
    }
    return ia + na * ip;
}

void oracle_polar_table(int32_t ba, int32_t bp, const double* levels, float* cb)
{
    int32_t na = 1 << ba, np_ = 1 << bp;
    for (int ip = 0; ip < np_; ++ip) {
        double th = 2.0 * ORACLE_PI * ip / np_;
        for (int ia = 0; ia < na; ++ia) {
            cb[2 * (ia + na * ip)] = (float)(levels[ia] * cos(th));
            cb[2 * (ia + na * ip) + 1] = (float)(levels[ia] * sin(th));
        }
    }
}

/* Section 2 (the scalar ablation, reading R10): integrals of the standard
 * normal density phi over [a, b] (either end may be infinite):
 * mass = Phi(b) - Phi(a); first moment = phi(a) - phi(b). */
static double normal_pdf(double x)
{
    return isinf(x) ? 0.0 : exp(-0.5 * x * x) / sqrt(2.0 * ORACLE_PI);
}
static double normal_cdf(double x)
{
    return 0.5 * erfc(-x / sqrt(2.0));
}

int oracle_gauss_lloyd_max(int32_t b, double* levels, double* thresholds)
{
    if (b < 1 || b > 8) return -1;
    int32_t L = 1 << b;
    /* cell edges at the quantiles Phi^-1(i / L), by bisection to the last bit */
    double* q = malloc(sizeof(double) * (size_t)(L + 1));
    q[0] = -INFINITY;
    q[L] = INFINITY;
    for (int i = 1; i < L; ++i) {
        double lo = -40.0, hi = 40.0, target = (double)i / L;
        for (;;) {
            double mid = 0.5 * (lo + hi);
            if (mid <= lo || mid >= hi) break;
            if (normal_cdf(mid) < target) lo = mid; else hi = mid;
        }
        q[i] = 0.5 * (lo + hi);
    }
    for (int i = 0; i < L; ++i)
        levels[i] = (normal_pdf(q[i]) - normal_pdf(q[i + 1])) / (normal_cdf(q[i + 1]) - normal_cdf(q[i]));
    free(q);
    for (int it = 0; it < 10000; ++it) {
        for (int i = 0; i + 1 < L; ++i) thresholds[i] = 0.5 * (levels[i] + levels[i + 1]);
        int moved = 0;
        for (int i = 0; i < L; ++i) {
            double a = (i == 0) ? -INFINITY : thresholds[i - 1];
            double c = (i + 1 == L) ? INFINITY : thresholds[i];
            double v = (normal_pdf(a) - normal_pdf(c)) / (normal_cdf(c) - normal_cdf(a));
            if (fabs(v - levels[i]) > 1e-15 * fabs(levels[i])) moved = 1;
            levels[i] = v;
        }
        if (!moved) break;
    }
    for (int i = 0; i + 1 < L; ++i) thresholds[i] = 0.5 * (levels[i] + levels[i + 1]);
    return 0;
}

int32_t oracle_scalar_index(float p, int32_t b, const double* thresholds)
{
    int32_t L = 1 << b, ix = 0;
    for (int i = 0; i + 1 < L; ++i)
        if ((double)p > thresholds[i]) ix = i + 1;
    return ix;
}

void oracle_scalar_table(int32_t b, const double* levels, float* cb)
{
    int32_t L = 1 << b;
    for (int iy = 0; iy < L; ++iy)
        for (int ix = 0; ix < L; ++ix) {
            cb[2 * (ix + L * iy)] = (float)levels[ix];
            cb[2 * (ix + L * iy) + 1] = (float)levels[iy];
        }
}

/* Section 3.1, steps 1-6, for every row passed in; step 5 is the nearest
 * codeword of cb (QAM-W, section 3.6) or, when thresholds is given, the polar
 * index (section 3.5, reading R8) with bits = ba + bp. */
static int encode_rows(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                       const float* s, const uint32_t* sign_bits, int32_t block, const float* cb,
                       int32_t bits, const double* thresholds, int32_t ba, int32_t scalar, const float* sigma,
                       uint16_t* norm16, uint8_t* codes, int32_t* idx_out, float* p_out, int32_t* status)
{
    if (check_block(d_in, block) || ld < d_in || n_rows < 0 || bits < 1 || bits > 16) return -1;
    int32_t K = 1 << bits, n_pairs = d_in / 2;
    size_t stride = oracle_row_stride(d_in, bits);
    double* H = malloc(sizeof(double) * (size_t)block * block);
    oracle_hadamard(block, H);
    int32_t flags = scale_flags(s, d_in);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : flags)
    for (int64_t i = 0; i < n_rows; ++i) {
        double* a = malloc(sizeof(double) * (size_t)d_in);
        double* y = malloc(sizeof(double) * (size_t)d_in);
        int32_t* idx = malloc(sizeof(int32_t) * (size_t)n_pairs);
        double r;
        int32_t f = front_end_row(w, w_bf16, i, d_in, ld, s, sign_bits, block, H, a, y, &r);
        for (int k = 0; k < n_pairs; ++k) idx[k] = 0;
        uint16_t nh = 0;
        if (r > 0.0 && isfinite(r)) {
            for (int k = 0; k < n_pairs; ++k) {
                /* steps 3-4: pair z_k = y_2k + i y_2k+1, divide by sigma_k */
                float px = (float)(y[2 * k] / (double)sigma[k]);
                float py = (float)(y[2 * k + 1] / (double)sigma[k]);
                if (p_out) {
                    p_out[i * d_in + 2 * k] = px;
                    p_out[i * d_in + 2 * k + 1] = py;
                }
                if (scalar) /* step 5, one scalar quantizer per coordinate (reading R10) */
                    idx[k] = oracle_scalar_index(px, bits / 2, thresholds) +
                             (oracle_scalar_index(py, bits / 2, thresholds) << (bits / 2));
                else
                idx[k] = thresholds ? oracle_polar_index(px, py, ba, bits - ba, thresholds) /* step 5 */
                                    : oracle_nearest(px, py, cb, K, NULL);
            }
            nh = oracle_f16_from_f32((float)r); /* section 3.2: 16-bit row norm */
            if ((nh & 0x7fffu) == 0x7c00u) f |= ORACLE_FLAG_NORM_RANGE;
        } else if (p_out) {
            for (int j = 0; j < d_in; ++j) p_out[i * d_in + j] = 0.0f;
        }
        norm16[i] = nh;
        if (idx_out)
            for (int k = 0; k < n_pairs; ++k) idx_out[i * n_pairs + k] = idx[k];
        oracle_pack_row(idx, n_pairs, bits, codes + (size_t)i * stride, stride);
        flags |= f;
        free(a);
        free(y);
        free(idx);
    }
    free(H);
    if (status) *status |= flags;
    return 0;
}

int oracle_encode(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                  const float* s, const uint32_t* sign_bits, int32_t block, const float* cb,
                  int32_t bits, const float* sigma, uint16_t* norm16, uint8_t* codes,
                  int32_t* idx_out, float* p_out, int32_t* status)
{
    return encode_rows(w, w_bf16, n_rows, d_in, ld, s, sign_bits, block, cb, bits, NULL, 0, 0, sigma, norm16,
                       codes, idx_out, p_out, status);
}

int oracle_encode_polar(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                        const float* s, const uint32_t* sign_bits, int32_t block, int32_t ba, int32_t bp,
                        const double* thresholds, const float* sigma, uint16_t* norm16, uint8_t* codes,
                        int32_t* idx_out, float* p_out, int32_t* status)
{
    if (ba < 1 || bp < 1 || ba + bp > 16) return -1;
    return encode_rows(w, w_bf16, n_rows, d_in, ld, s, sign_bits, block, NULL, ba + bp, thresholds, ba, 0, sigma,
                       norm16, codes, idx_out, p_out, status);
}

int oracle_encode_scalar(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                         const float* s, const uint32_t* sign_bits, int32_t block, int32_t b,
                         const double* thresholds, const float* sigma, uint16_t* norm16, uint8_t* codes,
                         int32_t* idx_out, float* p_out, int32_t* status)
{
    if (b < 1 || b > 8) return -1;
    return encode_rows(w, w_bf16, n_rows, d_in, ld, s, sign_bits, block, NULL, 2 * b, thresholds, 0, 1, sigma,
                       norm16, codes, idx_out, p_out, status);
}

/* Section 3.2: unpack, look up, rescale by sigma_k, reassemble pairs, apply
 * R_inv = R_fwd^T = diag(eps) blockdiag(H_b)^T, multiply by the stored row
 * norm; then remove the channel scale (reading R6).  BF16 output is the
 * round-to-nearest-even of the float result (section 1: dequantize to BF16
 * before the matrix product). */
int oracle_decode(const uint8_t* codes, const uint16_t* norm16, int64_t n_rows, int32_t d_in,
                  const float* sigma, const float* cb, int32_t bits, const float* s,
                  const uint32_t* sign_bits, int32_t block, float* out_f32, uint16_t* out_bf16,
                  double* out_f64)
{
    if (check_block(d_in, block) || n_rows < 0 || bits < 1 || bits > 16) return -1;
    int32_t n_pairs = d_in / 2;
    size_t stride = oracle_row_stride(d_in, bits);
    double* H = malloc(sizeof(double) * (size_t)block * block);
    oracle_hadamard(block, H);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_rows; ++i) {
        int32_t* idx = malloc(sizeof(int32_t) * (size_t)n_pairs);
        double* x = malloc(sizeof(double) * (size_t)d_in);
        double* v = malloc(sizeof(double) * (size_t)d_in);
        oracle_unpack_row(codes + (size_t)i * stride, n_pairs, bits, idx);
        double rn = (double)oracle_f32_from_f16(norm16[i]);
        for (int k = 0; k < n_pairs; ++k) {
            x[2 * k] = (double)sigma[k] * (double)cb[2 * idx[k]];
            x[2 * k + 1] = (double)sigma[k] * (double)cb[2 * idx[k] + 1];
        }
        for (int t = 0; t < d_in / block; ++t)
            for (int jj = 0; jj < block; ++jj) {
                double acc = 0.0;
                for (int k = 0; k < block; ++k) acc += H[(size_t)k * block + jj] * x[(size_t)t * block + k];
                v[(size_t)t * block + jj] = acc;
            }
        for (int j = 0; j < d_in; ++j) {
            double wj = (rn == 0.0) ? 0.0 : ((rn * eps_of(sign_bits, j)) * v[j]) / (double)s[j];
            float f = (float)wj;
            if (out_f64) out_f64[i * d_in + j] = wj;
            if (out_f32) out_f32[i * d_in + j] = f;
            if (out_bf16) out_bf16[i * d_in + j] = oracle_bf16_from_f32(f);
        }
        free(idx);
        free(x);
        free(v);
    }
    free(H);
    return 0;
}

/* Section 1 (the matrix product that follows dequantization): y = x W^T for
 * M activation rows x (fp32, leading dimension ld_x), with W the decoder's
 * output before any rounding (the fp64 values of oracle_decode):
 *   y[m * n_rows + i] = sum over j of x[m][j] * w_ij, summed in order in fp64. */
int oracle_qgemm(const float* x, int32_t M, int64_t ld_x, const uint8_t* codes, const uint16_t* norm16,
                 int64_t n_rows, int32_t d_in, const float* sigma, const float* cb, int32_t bits,
                 const float* s, const uint32_t* sign_bits, int32_t block, double* y)
{
    if (M < 0 || ld_x < d_in || n_rows < 0) return -1;
    const int64_t chunk = 256;
    double* w = malloc(sizeof(double) * (size_t)chunk * (size_t)d_in);
    float* f32 = malloc(sizeof(float) * (size_t)chunk * (size_t)d_in);
    uint16_t* b16 = malloc(sizeof(uint16_t) * (size_t)chunk * (size_t)d_in);
    size_t stride = oracle_row_stride(d_in, bits);
    int rc = 0;
    for (int64_t i0 = 0; i0 < n_rows && rc == 0; i0 += chunk) {
        int64_t n = n_rows - i0 < chunk ? n_rows - i0 : chunk;
        rc = oracle_decode(codes + (size_t)i0 * stride, norm16 + i0, n, d_in, sigma, cb, bits, s, sign_bits,
                           block, f32, b16, w);
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            for (int32_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int32_t j = 0; j < d_in; ++j) acc += (double)x[(size_t)m * ld_x + j] * w[(size_t)i * d_in + j];
                y[(size_t)m * n_rows + i0 + i] = acc;
            }
    }
    free(w);
    free(f32);
    free(b16);
    return rc;
}

/* Activation-aware channel scale (reading R11): x is T x d_in (fp32 values,
 * leading dimension ld); rms (may be NULL) receives r_j. */
int oracle_act_scale(const float* x, int64_t T, int32_t d_in, int64_t ld, double alpha, float* scale, double* rms)
{
    if (T < 1 || d_in < 1 || ld < d_in) return -1;
    for (int32_t j = 0; j < d_in; ++j) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double v = (double)x[t * ld + j];
            acc += v * v;
        }
        double r = sqrt(acc / (double)T);
        if (rms) rms[j] = r;
        scale[j] = r > 0.0 ? (float)pow(r, alpha) : 1.0f;
    }
    return 0;
}

/* Section 3.6, eq. 2: Lloyd iterations for the 2D codebook on samples of the
 * unit circular Gaussian (reading R7).  e_trace[t] = sum over points of
 * llrint(D * 2^32) for the assignment of iteration t (modulo 2^64). */
int oracle_lloyd(const float* pts, int64_t n, int32_t bits, int32_t iters, const float* init,
                 float* cb, int64_t* e_trace, int32_t* status)
{
    if (bits < 1 || bits > 16 || iters < 0) return -1;
    int32_t K = 1 << bits;
    if (n < K) return -1;
    int lg = 0;
    while (((int64_t)1 << lg) < n) ++lg;
    double limit = ldexp(1.0, 31 - lg);
    if (limit > 4096.0) limit = 4096.0;
    for (int32_t j = 0; j < 2 * K; ++j) cb[j] = init ? init[j] : pts[j];
    int32_t* idx = malloc(sizeof(int32_t) * (size_t)n);
    float* dist = malloc(sizeof(float) * (size_t)n);
    int64_t* sx = malloc(sizeof(int64_t) * (size_t)K);
    int64_t* sy = malloc(sizeof(int64_t) * (size_t)K);
    int64_t* cnt = malloc(sizeof(int64_t) * (size_t)K);
    int32_t flags = 0;
    for (int32_t it = 0; it < iters; ++it) {
        oracle_nearest_many(pts, n, cb, K, idx, dist);
        for (int32_t j = 0; j < K; ++j) sx[j] = sy[j] = cnt[j] = 0;
        uint64_t e = 0;
        for (int64_t i = 0; i < n; ++i) {
            float x = pts[2 * i], y = pts[2 * i + 1];
            if (!(fabsf(x) < limit) || !(fabsf(y) < limit)) {
                flags |= ORACLE_FLAG_POINT_RANGE;
                continue;
            }
            int32_t j = idx[i];
            sx[j] += llrint((double)x * 4294967296.0);
            sy[j] += llrint((double)y * 4294967296.0);
            cnt[j] += 1;
            e += (uint64_t)llrint((double)dist[i] * 4294967296.0);
        }
        if (e_trace) e_trace[it] = (int64_t)e;
        for (int32_t j = 0; j < K; ++j)
            if (cnt[j] > 0) { /* centroid condition; an empty cell keeps its codeword */
                cb[2 * j] = (float)(((double)sx[j] * 0x1p-32) / (double)cnt[j]);
                cb[2 * j + 1] = (float)(((double)sy[j] * 0x1p-32) / (double)cnt[j]);
            }
    }
    free(idx);
    free(dist);
    free(sx);
    free(sy);
    free(cnt);
    if (status) *status |= flags;
    return 0;
}
