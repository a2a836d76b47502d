// GPU form of the seeded weight generator of synth.c (test and benchmark inputs only).
//
// The same recipe, written again for the device so that a 12.7 G-weight stack can be drawn in
// HBM from its seeds in seconds: splitmix64 counters, Box-Muller normals with the logarithm and
// cosine evaluated from the series of synth.c (+, -, *, / and sqrt only, each rounded once:
// built with -ffp-contract=off), Student-t as g0 / sqrt(sum g_t^2 / nu), fp64 -> fp32 -> bf16
// with round-to-nearest-even.  Every element is a pure function of (seed, stream, row, column),
// so the bytes equal those of synth.c; a GPU test compares the two.
//
// This file holds no part of the codec; it is not linked into libqamw.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ uint64_t mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ double uniform(uint64_t key, uint64_t i) {
    return (double)(mix(key + (i + 1) * kGolden) >> 11) * 0x1p-53;
}

// natural log on [2^-53, 1]: mantissa in [sqrt(1/2), sqrt(2)), 2 atanh(t) series to t^23
__device__ double log_series(double x) {
    uint64_t bits = __double_as_longlong(x);
    int e = (int)((bits >> 52) & 0x7ff) - 1023;
    bits = (bits & 0x000fffffffffffffull) | 0x3ff0000000000000ull;
    double m = __longlong_as_double(bits);
    if (m > 1.4142135623730951) {
        m = m * 0.5;
        e += 1;
    }
    const double t = (m - 1.0) / (m + 1.0);
    const double t2 = t * t;
    double s = 1.0 / 23.0;
    for (int k = 21; k >= 1; k -= 2) s = s * t2 + 1.0 / (double)k;
    return 2.0 * t * s + (double)e * 0.6931471805599453;
}

// cos(2 pi v) for v in [0, 1): quadrant, then the Taylor series of sin / cos on [0, pi/2)
__device__ double cos2pi_series(double v) {
    const double v4 = v * 4.0;
    const int q = (int)v4;
    const double f = v4 - (double)q;
    const double th = f * 1.5707963267948966;
    const double th2 = th * th;
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

__device__ double gauss(uint64_t key, uint64_t q) {
    const double u1 = uniform(key, 2 * q);
    const double u2 = uniform(key, 2 * q + 1);
    const double rad = __builtin_sqrt(-2.0 * log_series(1.0 - u1));
    return rad * cos2pi_series(u2);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(256) void k_synth_weights(uint64_t key, int64_t row0, int64_t nrows, int32_t d_in,
                                                       int32_t dist, int32_t nu, double scale,
                                                       const uint8_t* __restrict__ mask, double factor,
                                                       int32_t out_bf16, void* __restrict__ out) {
    const int64_t n = nrows * (int64_t)d_in;
    const int64_t n_norm = dist == 1 ? (int64_t)nu + 1 : 1;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = e / d_in;
        const int32_t j = (int32_t)(e - r * d_in);
        const int64_t i = row0 + r;
        const uint64_t q0 = (uint64_t)((i * d_in + j) * n_norm);
        double g = gauss(key, q0);
        if (dist == 1) {
            double acc = 0.0;
            for (int t = 1; t <= nu; ++t) {
                const double h = gauss(key, q0 + (uint64_t)t);
                acc = acc + h * h;
            }
            g = g / __builtin_sqrt(acc / (double)nu);
        }
        double v = scale * g;
        if (mask && mask[j]) v = v * factor;
        const float f = (float)v;
        if (out_bf16)
            reinterpret_cast<uint16_t*>(out)[e] = f32_to_bf16(f);
        else
            reinterpret_cast<float*>(out)[e] = f;
    }
}

}  // namespace

extern "C" {

// Rows [row0, row0 + nrows) of the matrix synth_weights of synth.c generates for (seed, sid), into
// device memory (row-major, d_in per row; uint16 bf16 bit patterns when out_bf16).  d_mask: d_in
// device bytes (outlier columns) or NULL.  Returns 0, or -1 for bad arguments / a failed launch.
int synth_weights_device(uint64_t seed, uint64_t sid, int64_t row0, int64_t nrows, int32_t d_in, int32_t dist,
                         int32_t nu, double scale, const uint8_t* d_mask, double factor, int32_t out_bf16,
                         void* d_out, void* stream) {
    if (nrows < 0 || d_in <= 0 || row0 < 0 || !d_out) return -1;
    if (nrows == 0) return 0;
    const uint64_t key = mix(seed * kGolden + sid);   // synth_key of synth.c (host evaluation)
    const int64_t n = nrows * (int64_t)d_in;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_synth_weights, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, key, row0, nrows,
                       d_in, dist, nu, scale, d_mask, factor, out_bf16, d_out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
