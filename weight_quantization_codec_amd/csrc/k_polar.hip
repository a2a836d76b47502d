// Codebook of the polar baseline (paper section 3.5): magnitude levels of the Na-level
// Lloyd-Max quantizer of the unit Rayleigh density f(r) = r exp(-r^2/2) (the modulus of a
// circular standard Gaussian pair), its thresholds, and the Na x Np product table that the QAM-W
// decoder reads (entry ia + Na ip = level ia at angle 2 pi ip / Np).
//
// One workgroup, one thread per level.  Lloyd-Max alternates the two optimality conditions of a
// scalar quantizer: thresholds at the midpoints of adjacent levels, levels at the conditional
// means of their cells.  With F(r) = exp(-r^2/2):
//   mass(a, b)   = F(a) - F(b)
//   moment(a, b) = int_a^b r^2 exp(-r^2/2) dr = a F(a) - b F(b) + sqrt(pi/2) (erfc(a/sqrt2) - erfc(b/sqrt2))
// (integration by parts; erfc keeps the top cell's difference free of cancellation).  The start is
// the conditional means of Na equal-probability cells (edges at the quantiles
// sqrt(-2 ln(1 - i/Na))), and the iteration stops when no level moves by more than 1e-15 of
// itself, or after 10000 rounds.
#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

namespace {

constexpr int kPolarIters = 10000;
constexpr int kScalarMaxB = 6;   // 2b <= 12 index bits

__device__ inline double ray_F(double r) { return __builtin_isinf(r) ? 0.0 : exp(-0.5 * r * r); }

__device__ inline double ray_cell_mean(double a, double b) {
    const double rs2 = 0.70710678118654752440;   // 1/sqrt(2)
    const double sq_half_pi = 1.25331413731550025121;   // sqrt(pi/2)
    const double fa = ray_F(a), fb = ray_F(b);
    const double bfb = __builtin_isinf(b) ? 0.0 : b * fb;
    const double tail = erfc(a * rs2) - (__builtin_isinf(b) ? 0.0 : erfc(b * rs2));
    return (a * fa - bfb + sq_half_pi * tail) / (fa - fb);
}

__global__ __launch_bounds__(256) void k_polar_codebook(int ba, int bp, double* __restrict__ levels,
                                                        double* __restrict__ thr, float* __restrict__ cb) {
    __shared__ double lv[1 << kPolarMaxBa];
    __shared__ double th[1 << kPolarMaxBa];
    const int na = 1 << ba, i = threadIdx.x;
    const bool mine = i < na;
    const double inf = __builtin_huge_val();
    if (mine) {
        const double a = sqrt(-2.0 * log1p(-(double)i / (double)na));
        const double b = i + 1 == na ? inf : sqrt(-2.0 * log1p(-(double)(i + 1) / (double)na));
        lv[i] = ray_cell_mean(a, b);
    }
    __syncthreads();
    for (int it = 0; it < kPolarIters; ++it) {
        if (i + 1 < na) th[i] = 0.5 * (lv[i] + lv[i + 1]);
        __syncthreads();
        bool moved = false;
        double v = 0.0;
        if (mine) {
            const double a = i == 0 ? 0.0 : th[i - 1];
            const double b = i + 1 == na ? inf : th[i];
            v = ray_cell_mean(a, b);
            moved = fabs(v - lv[i]) > 1e-15 * lv[i];
        }
        // every thread has read lv for the thresholds (barrier above) and reads only th here
        if (mine) lv[i] = v;
        if (!__syncthreads_or(moved)) break;
    }
    if (i + 1 < na) th[i] = 0.5 * (lv[i] + lv[i + 1]);
    __syncthreads();
    if (mine) levels[i] = lv[i];
    if (i + 1 < na) thr[i] = th[i];
    const int np = 1 << bp, n = na * np;
    for (int k = i; k < n; k += blockDim.x) {
        const int ia = k & (na - 1), ip = k >> ba;
        const double f = 2.0 * (double)ip / (double)np;   // the angle / pi, exact
        cb[2 * k] = (float)(lv[ia] * cospi(f));
        cb[2 * k + 1] = (float)(lv[ia] * sinpi(f));
    }
}

// Polar indices of n pairs (grid-stride; the tables are built per workgroup).
__global__ __launch_bounds__(256) void k_polar_index(const float2* __restrict__ pts, int64_t n, int ba, int bp,
                                                     const double* __restrict__ thr, int32_t* __restrict__ out,
                                                     int32_t* __restrict__ status) {
    extern __shared__ __align__(16) char smem[];
    PolarLds pl = polar_lds_carve(smem, ba, bp);
    const bool bad = polar_lds_fill(pl, thr, threadIdx.x, blockDim.x);
    __syncthreads();
    if (bad && blockIdx.x == 0) flag_status(status, 16);
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
        const float2 q = pts[k];
        float x[1] = {q.x}, y[1] = {q.y};
        int r[1];
        polar_batch<1>(x, y, pl, r);
        out[k] = r[0];
    }
}

// Scalar (d = 1) ablation (paper section 2): the L-level Lloyd-Max quantizer of the standard
// normal density, for each coordinate of a pair, and the L x L product table (entry ix + L iy =
// (a_ix, a_iy)).  Start: the conditional means of L equal-probability cells, whose edges are the
// quantiles Phi^-1(i / L) found by bisection to the last bit; then the Lloyd-Max rounds of
// k_polar_codebook.  With phi the density and Phi the distribution function, a cell's mean is
// (phi(a) - phi(c)) / (Phi(c) - Phi(a)); the mass is taken from the nearer tail (erfc), free of
// cancellation.
__device__ inline double nrm_pdf(double x) {
    return __builtin_isinf(x) ? 0.0 : exp(-0.5 * x * x) * 0.39894228040143267794;   // 1/sqrt(2 pi)
}
__device__ inline double nrm_cdf(double x) { return 0.5 * erfc(-x * 0.70710678118654752440); }
__device__ inline double nrm_mass(double a, double c) {
    const double rs2 = 0.70710678118654752440;
    if (a >= 0.0) return 0.5 * (erfc(a * rs2) - (__builtin_isinf(c) ? 0.0 : erfc(c * rs2)));
    return 0.5 * ((__builtin_isinf(c) ? 2.0 : erfc(-c * rs2)) - erfc(-a * rs2));
}
__device__ inline double nrm_cell_mean(double a, double c) { return (nrm_pdf(a) - nrm_pdf(c)) / nrm_mass(a, c); }

__global__ __launch_bounds__(256) void k_scalar_codebook(int b, double* __restrict__ levels, double* __restrict__ thr,
                                                         float* __restrict__ cb) {
    __shared__ double lv[1 << kScalarMaxB];
    __shared__ double th[1 << kScalarMaxB];
    __shared__ double q[(1 << kScalarMaxB) + 1];
    const int L = 1 << b, i = threadIdx.x;
    const bool mine = i < L;
    const double inf = __builtin_huge_val();
    if (i <= L) {
        double e = i == 0 ? -inf : inf;
        if (i > 0 && i < L) {
            double lo = -40.0, hi = 40.0;
            const double target = (double)i / (double)L;
            for (;;) {
                const double mid = 0.5 * (lo + hi);
                if (mid <= lo || mid >= hi) break;
                if (nrm_cdf(mid) < target) lo = mid; else hi = mid;
            }
            e = 0.5 * (lo + hi);
        }
        q[i] = e;
    }
    __syncthreads();
    if (mine) lv[i] = nrm_cell_mean(q[i], q[i + 1]);
    __syncthreads();
    for (int it = 0; it < kPolarIters; ++it) {
        if (i + 1 < L) th[i] = 0.5 * (lv[i] + lv[i + 1]);
        __syncthreads();
        bool moved = false;
        double v = 0.0;
        if (mine) {
            const double a = i == 0 ? -inf : th[i - 1];
            const double c = i + 1 == L ? inf : th[i];
            v = nrm_cell_mean(a, c);
            moved = fabs(v - lv[i]) > 1e-15 * fabs(lv[i]);
        }
        if (mine) lv[i] = v;
        if (!__syncthreads_or(moved)) break;
    }
    if (i + 1 < L) th[i] = 0.5 * (lv[i] + lv[i + 1]);
    __syncthreads();
    if (mine) levels[i] = lv[i];
    if (i + 1 < L) thr[i] = th[i];
    for (int k = i; k < L * L; k += blockDim.x) {
        cb[2 * k] = (float)lv[k & (L - 1)];
        cb[2 * k + 1] = (float)lv[k >> b];
    }
}

}  // namespace

hipError_t launch_scalar_codebook(int b, double* levels, double* thr, float* cb, hipStream_t st) {
    hipLaunchKernelGGL(k_scalar_codebook, dim3(1), dim3(256), 0, st, b, levels, thr, cb);
    return hipGetLastError();
}

hipError_t launch_polar_index(const float* pts, int64_t n, int ba, int bp, const double* thr, int32_t* out,
                              int32_t* status, hipStream_t st) {
    const int64_t blocks = (n + 255) / 256;
    const int grid = (int)(blocks < 2048 ? blocks : 2048);
    hipLaunchKernelGGL(k_polar_index, dim3(grid), dim3(256), polar_lds_bytes(bp), st,
                       reinterpret_cast<const float2*>(pts), n, ba, bp, thr, out, status);
    return hipGetLastError();
}

hipError_t launch_polar_codebook(int ba, int bp, double* levels, double* thr, float* cb, hipStream_t st) {
    hipLaunchKernelGGL(k_polar_codebook, dim3(1), dim3(256), 0, st, ba, bp, levels, thr, cb);
    return hipGetLastError();
}

}  // namespace qamw
