// Lloyd training of the 2D codebook (paper section 3.6, eq. 2: Lloyd iterations on the unit
// circular Gaussian, here on a seeded sample of it).
//
// Per iteration two kernels on the caller's stream:
//   assign  -> every point to its nearest codeword (fp32 distance, ties to the lowest index),
//              sums of round(x * 2^32), round(y * 2^32), counts and round(D * 2^32) privatized
//              per workgroup in LDS (64-bit integer atomics) and flushed with global atomics;
//   update  -> c_j = fl32((S_j * 2^-32) / N_j) for non-empty cells, records the distortion
//              sum, and clears the accumulators for the next iteration.
// Integer sums do not depend on the order of the atomics, so the codebook is bit-identical
// from run to run and to a sequential computation.
#include <cmath>

#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

struct LloydAcc {
    unsigned long long sx[4096];
    unsigned long long sy[4096];
    unsigned long long cnt[4096];
    unsigned long long e;
};

size_t lloyd_workspace(int bits) {
    (void)bits;
    return sizeof(LloydAcc);
}

namespace {

__global__ __launch_bounds__(256) void k_lloyd_init(const float* src, float* cb, int K,
                                                    LloydAcc* acc) {
    int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < K) {
        float2 c = reinterpret_cast<const float2*>(src)[j];
        reinterpret_cast<float2*>(cb)[j] = c;
        acc->sx[j] = 0;
        acc->sy[j] = 0;
        acc->cnt[j] = 0;
    }
    if (j == 0) acc->e = 0;
}

__device__ __forceinline__ unsigned long long fx32(double v) {
    // round(v * 2^32) to nearest, ties to even, as a two's-complement 64-bit pattern
    return (unsigned long long)(long long)__builtin_rint(v * 4294967296.0);
}

__global__ __launch_bounds__(256) void k_lloyd_assign(const float* __restrict__ pts, int64_t n,
                                                      const float* __restrict__ cb, int K, float limit,
                                                      LloydAcc* __restrict__ acc, int32_t* status) {
    extern __shared__ __align__(16) char smem[];
    float2* scb = reinterpret_cast<float2*>(smem);
    unsigned long long* lsx = reinterpret_cast<unsigned long long*>(smem + (size_t)K * sizeof(float2));
    unsigned long long* lsy = lsx + K;
    unsigned int* lcnt = reinterpret_cast<unsigned int*>(lsy + K);
    __shared__ unsigned long long le;
    for (int j = threadIdx.x; j < K; j += blockDim.x) {
        scb[j] = reinterpret_cast<const float2*>(cb)[j];
        lsx[j] = 0;
        lsy[j] = 0;
        lcnt[j] = 0;
    }
    if (threadIdx.x == 0) le = 0;
    __syncthreads();
    unsigned long long e_local = 0;
    int32_t flags = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float2 p = reinterpret_cast<const float2*>(pts)[i];
        float bd = __builtin_inff();
        int bj = 0;
        for (int j = 0; j < K; ++j) eval_cw(p.x, p.y, scb[j], j, bd, bj);
        if (fabsf(p.x) < limit && fabsf(p.y) < limit) {
            atomicAdd(&lsx[bj], fx32((double)p.x));
            atomicAdd(&lsy[bj], fx32((double)p.y));
            atomicAdd(&lcnt[bj], 1u);
            e_local += fx32((double)bd);
        } else {
            flags |= 8;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) e_local += __shfl_xor(e_local, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) atomicAdd(&le, e_local);
    __syncthreads();
    for (int j = threadIdx.x; j < K; j += blockDim.x) {
        if (lcnt[j]) {
            atomicAdd(&acc->sx[j], lsx[j]);
            atomicAdd(&acc->sy[j], lsy[j]);
            atomicAdd(&acc->cnt[j], (unsigned long long)lcnt[j]);
        }
    }
    if (threadIdx.x == 0) atomicAdd(&acc->e, le);
    flag_status(status, flags);
}

__global__ __launch_bounds__(256) void k_lloyd_update(float* __restrict__ cb, int K, LloydAcc* __restrict__ acc,
                                                      int64_t* trace, int it) {
    int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < K) {
        unsigned long long c = acc->cnt[j];
        if (c > 0) {
            double sx = (double)(long long)acc->sx[j] * 0x1p-32;
            double sy = (double)(long long)acc->sy[j] * 0x1p-32;
            reinterpret_cast<float2*>(cb)[j] = make_float2((float)(sx / (double)c), (float)(sy / (double)c));
        }
        acc->sx[j] = 0;
        acc->sy[j] = 0;
        acc->cnt[j] = 0;
    }
    if (j == 0) {
        if (trace) trace[it] = (int64_t)acc->e;
        acc->e = 0;
    }
}

}  // namespace

hipError_t launch_lloyd(const float* pts, int64_t n, int bits, int iters, const float* init, float* cb,
                        int64_t* trace, int32_t* status, void* ws, hipStream_t st) {
    const int K = 1 << bits;
    LloydAcc* acc = reinterpret_cast<LloydAcc*>(ws);
    int lg = 0;
    while (((int64_t)1 << lg) < n) ++lg;
    double lim = std::ldexp(1.0, 31 - lg);   // keeps n * |x| * 2^32 below 2^63
    if (lim > 4096.0) lim = 4096.0;
    const float limit = (float)lim;
    hipLaunchKernelGGL(k_lloyd_init, dim3((K + 255) / 256), dim3(256), 0, st, init ? init : pts, cb, K, acc);
    const size_t smem = (size_t)K * (sizeof(float2) + 2 * sizeof(unsigned long long) + sizeof(unsigned int));
    int64_t blocks = (n + 255) / 256;
    const int per_cu = (int)((160 * 1024) / (smem + 64));
    int64_t cap = 256 * (per_cu < 1 ? 1 : (per_cu > 8 ? 8 : per_cu));
    if (blocks > cap) blocks = cap;
    allow_lds(k_lloyd_assign, smem);
    for (int it = 0; it < iters; ++it) {
        hipLaunchKernelGGL(k_lloyd_assign, dim3((unsigned)blocks), dim3(256), smem, st, pts, n, cb, K, limit, acc,
                           status);
        hipLaunchKernelGGL(k_lloyd_update, dim3((K + 255) / 256), dim3(256), 0, st, cb, K, acc, trace, it);
    }
    return hipGetLastError();
}

}  // namespace qamw
