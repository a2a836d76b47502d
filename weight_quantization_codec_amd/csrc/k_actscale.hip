// Activation-aware channel scale (the AWQ-style per-channel scaling of the paper: s_j proportional to
// r_j^alpha, r_j the RMS of input channel j over calibration activations).
//
// k_act_partial: fp64 sums of squares of 4 consecutive columns per thread over one chunk of rows
// (grid: column blocks x row chunks; the chunking depends on T only, so the result is
// deterministic).  k_act_finish: per column, the chunks in order, r = sqrt(sum / T), and
// s = fl32(r^alpha) (1 for a channel that is zero over the batch).  HBM-bound: one read of X.
#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

namespace {

constexpr int kActCols = 4;
constexpr int kActThreads = 256;
constexpr int kActMaxChunks = 64;
constexpr int kActUnroll = 8;

template <bool BF, bool VEC>
__global__ __launch_bounds__(kActThreads) void k_act_partial(const void* __restrict__ x, int64_t T, int d_in,
                                                             int64_t ld, int64_t rows_per,
                                                             double* __restrict__ partial) {
    const int j0 = (blockIdx.x * kActThreads + threadIdx.x) * kActCols;
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * rows_per;
    const int64_t t1 = t0 + rows_per < T ? t0 + rows_per : T;
    double acc[kActCols] = {0.0, 0.0, 0.0, 0.0};
    // the kActCols values of row t (zeros past d_in)
    auto load_row = [&](int64_t t, float (&v)[kActCols]) {
        if constexpr (BF) {
            const uint16_t* row = reinterpret_cast<const uint16_t*>(x) + t * ld;
            if constexpr (VEC) {   // 8-byte aligned and d_in a multiple of 4
                const uint2 q = *reinterpret_cast<const uint2*>(row + j0);
                v[0] = __uint_as_float(q.x << 16);
                v[1] = __uint_as_float(q.x & 0xFFFF0000u);
                v[2] = __uint_as_float(q.y << 16);
                v[3] = __uint_as_float(q.y & 0xFFFF0000u);
            } else {
#pragma unroll
                for (int k = 0; k < kActCols; ++k) v[k] = j0 + k < d_in ? bf16_bits_to_float(row[j0 + k]) : 0.0f;
            }
        } else {
            const float* row = reinterpret_cast<const float*>(x) + t * ld;
            if constexpr (VEC) {   // 16-byte aligned and d_in a multiple of 4
                const float4 q = *reinterpret_cast<const float4*>(row + j0);
                v[0] = q.x;
                v[1] = q.y;
                v[2] = q.z;
                v[3] = q.w;
            } else {
#pragma unroll
                for (int k = 0; k < kActCols; ++k) v[k] = j0 + k < d_in ? row[j0 + k] : 0.0f;
            }
        }
    };
    if (j0 < d_in) {
        int64_t t = t0;
        // eight rows at a time, every load issued before the sums (rows are added in order)
        for (; t + kActUnroll <= t1; t += kActUnroll) {
            float v[kActUnroll][kActCols];
#pragma unroll
            for (int u = 0; u < kActUnroll; ++u) load_row(t + u, v[u]);
#pragma unroll
            for (int u = 0; u < kActUnroll; ++u)
#pragma unroll
                for (int k = 0; k < kActCols; ++k) acc[k] += (double)v[u][k] * (double)v[u][k];
        }
        for (; t < t1; ++t) {
            float v[kActCols];
            load_row(t, v);
#pragma unroll
            for (int k = 0; k < kActCols; ++k) acc[k] += (double)v[k] * (double)v[k];
        }
    }
#pragma unroll
    for (int k = 0; k < kActCols; ++k)
        if (j0 + k < d_in) partial[(size_t)c * d_in + j0 + k] = acc[k];
}

__global__ __launch_bounds__(256) void k_act_finish(const double* __restrict__ partial, int n_chunks, int64_t T,
                                                    int d_in, double alpha, float* __restrict__ scale,
                                                    double* __restrict__ rms) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= d_in) return;
    double sum = 0.0;
    int c = 0;
    for (; c + kActUnroll <= n_chunks; c += kActUnroll) {   // loads first, then the sums in order
        double v[kActUnroll];
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u) v[u] = partial[(size_t)(c + u) * d_in + j];
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u) sum += v[u];
    }
    for (; c < n_chunks; ++c) sum += partial[(size_t)c * d_in + j];
    const double r = sqrt(sum / (double)T);
    if (rms) rms[j] = r;
    scale[j] = r > 0.0 ? (float)pow(r, alpha) : 1.0f;
}

}  // namespace

int act_chunks(int64_t T) {
    // rows per chunk at least 16, at most kActMaxChunks chunks
    int64_t c = (T + 15) / 16;
    return (int)(c < kActMaxChunks ? (c > 0 ? c : 1) : kActMaxChunks);
}

hipError_t launch_act_scale(const void* x, int x_bf16, int64_t T, int d_in, int64_t ld, double alpha, float* scale,
                            double* rms, double* partial, hipStream_t st) {
    const int n_chunks = act_chunks(T);
    const int64_t rows_per = (T + n_chunks - 1) / n_chunks;
    const dim3 grid((d_in + kActThreads * kActCols - 1) / (kActThreads * kActCols), n_chunks);
    const size_t esz = x_bf16 ? 2 : 4;
    const bool vec = (d_in % kActCols == 0) && (((uintptr_t)x % (esz * kActCols)) == 0) &&
                     (((size_t)ld * esz) % (esz * kActCols) == 0);
    if (x_bf16) {
        if (vec)
            hipLaunchKernelGGL((k_act_partial<true, true>), grid, dim3(kActThreads), 0, st, x, T, d_in, ld, rows_per, partial);
        else
            hipLaunchKernelGGL((k_act_partial<true, false>), grid, dim3(kActThreads), 0, st, x, T, d_in, ld, rows_per, partial);
    } else {
        if (vec)
            hipLaunchKernelGGL((k_act_partial<false, true>), grid, dim3(kActThreads), 0, st, x, T, d_in, ld, rows_per, partial);
        else
            hipLaunchKernelGGL((k_act_partial<false, false>), grid, dim3(kActThreads), 0, st, x, T, d_in, ld, rows_per, partial);
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(k_act_finish, dim3((d_in + 255) / 256), dim3(256), 0, st, partial, n_chunks, T, d_in, alpha,
                       scale, rms);
    return hipGetLastError();
}

}  // namespace qamw
