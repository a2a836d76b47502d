// Search index for the nearest-codeword step (paper section 3.6: each normalized pair maps to
// its Euclidean-nearest codebook entry).
//
// A uniform G x G grid covers [-R, R]^2, R = 1.3 * max_j max(|c_jx|, |c_jy|).  For a cell Q
// (widened by 1e-3 of a cell on each side to absorb the fp32 rounding of the cell lookup),
//   U_Q = min_j maxdist^2(Q, c_j)            (every point of Q has a codeword within sqrt(U_Q)),
//   cand(Q) = { j : mindist^2(Q, c_j) <= U_Q * (1 + 1e-5) }   in increasing j,
// computed in double.  A codeword outside cand(Q) is farther than the nearest one by more than
// the relative error of the fp32 distance (about 2.4e-7), so the fp32 argmin over cand(Q), with
// ties to the lowest index, equals the argmin over all K codewords.  Cells with more than
// kIndexCap-1 candidates are marked as overflow and searched exhaustively.
#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

__global__ __launch_bounds__(256) void k_index_header(const float* __restrict__ cb, int K, int G, int bits,
                                                      IndexHeader* hdr) {
    __shared__ float red[256];
    float m = 0.f;
    for (int j = threadIdx.x; j < K; j += blockDim.x) {
        float2 c = reinterpret_cast<const float2*>(cb)[j];
        m = fmaxf(m, fmaxf(fabsf(c.x), fabsf(c.y)));   // NaN codewords are ignored by fmaxf
    }
    red[threadIdx.x] = m;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        float R = 1.3f * red[0];
        if (!(R >= 1e-3f) || !(R < 1e30f)) R = 1.0f;
        hdr->K = K;
        hdr->G = G;
        hdr->cap = kIndexCap;
        hdr->bits = bits;
        hdr->R = R;
        hdr->inv_h = (float)G / (2.0f * R);
        hdr->ready = 1;
        hdr->max_count = 0;
    }
}

__global__ __launch_bounds__(256) void k_index_cells(const float* __restrict__ cb, int K, IndexHeader* hdr,
                                                     uint16_t* __restrict__ slots) {
    extern __shared__ float2 scb[];
    for (int j = threadIdx.x; j < K; j += blockDim.x) scb[j] = reinterpret_cast<const float2*>(cb)[j];
    __syncthreads();
    const int G = hdr->G;
    const int cell = blockIdx.x * blockDim.x + threadIdx.x;
    if (cell >= G * G) return;
    const int cx = cell % G, cy = cell / G;
    const double R = (double)hdr->R;
    const double h = 1.0 / (double)hdr->inv_h;
    const double d = 1e-3 * h;
    const double x0 = cx * h - R - d, x1 = (cx + 1) * h - R + d;
    const double y0 = cy * h - R - d, y1 = (cy + 1) * h - R + d;
    double U = 1e300;
    for (int j = 0; j < K; ++j) {
        double px = scb[j].x, py = scb[j].y;
        double ax = fmax(fabs(px - x0), fabs(px - x1));
        double ay = fmax(fabs(py - y0), fabs(py - y1));
        U = fmin(U, ax * ax + ay * ay);
    }
    const double lim = U * (1.0 + 1e-5);
    uint16_t* s = slots + (size_t)cell * kIndexCap;
    int n = 0;
    for (int j = 0; j < K; ++j) {
        double px = scb[j].x, py = scb[j].y;
        double dx = fmax(fmax(x0 - px, px - x1), 0.0);
        double dy = fmax(fmax(y0 - py, py - y1), 0.0);
        if (dx * dx + dy * dy <= lim) {
            if (n + 1 < kIndexCap) s[n + 1] = (uint16_t)j;
            ++n;
        }
    }
    s[0] = (n + 1 < kIndexCap) ? (uint16_t)n : kCellOverflow;
    for (int t = (n + 1 < kIndexCap ? n + 1 : kIndexCap); t < kIndexCap; ++t) s[t] = 0;
    atomicMax(&hdr->max_count, n);
}

int index_grid_size(int bits) {
    // about two cells per codeword spacing at the centre of a Gaussian-trained codebook
    double K = (double)(1 << bits);
    int G = 16;
    while (G < 256 && G < 5.6 * __builtin_sqrt(K)) G *= 2;
    return G;
}

hipError_t launch_index_build(const float* cb, int bits, void* index, hipStream_t st) {
    const int K = 1 << bits;
    const int G = index_grid_size(bits);
    IndexHeader* hdr = reinterpret_cast<IndexHeader*>(index);
    uint16_t* slots = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(index) + kIndexHeaderBytes);
    hipLaunchKernelGGL(k_index_header, dim3(1), dim3(256), 0, st, cb, K, G, bits, hdr);
    const int cells = G * G;
    hipLaunchKernelGGL(k_index_cells, dim3((cells + 255) / 256), dim3(256), K * sizeof(float2), st, cb, K, hdr,
                       slots);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_nearest(const float* __restrict__ pts, int64_t n, const float* __restrict__ cb,
                                                 int K, const IndexHeader* __restrict__ hdr,
                                                 const uint16_t* __restrict__ slots, int32_t* __restrict__ out) {
    extern __shared__ float2 scb[];
    for (int j = threadIdx.x; j < K; j += blockDim.x) scb[j] = reinterpret_cast<const float2*>(cb)[j];
    __syncthreads();
    const IndexHeader ih = *hdr;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float2 p = reinterpret_cast<const float2*>(pts)[i];
        out[i] = nearest_indexed(p.x, p.y, scb, K, ih, slots);
    }
}

hipError_t launch_nearest(const float* pts, int64_t n, const float* cb, int bits, const void* index, int32_t* out,
                          hipStream_t st) {
    const int K = 1 << bits;
    const IndexHeader* hdr = reinterpret_cast<const IndexHeader*>(index);
    const uint16_t* slots =
        reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(index) + kIndexHeaderBytes);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(k_nearest, dim3((unsigned)blocks), dim3(256), K * sizeof(float2), st, pts, n, cb, K, hdr,
                       slots, out);
    return hipGetLastError();
}

}  // namespace qamw
