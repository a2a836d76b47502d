// Search index for the nearest-codeword step (paper section 3.6: each normalized pair maps to
// its Euclidean-nearest codebook entry), built on the GPU once per codebook.
//
// Grid.  A G x G grid over [-Rg, Rg]^2, Rg = 2.5 max_j max(|c_jx|, |c_jy|), whose cell edges sit
// at quantiles of the codeword coordinates (both axes share one set of edges): a point is
// located by a uniform fine bin (W bins over [-Rg, Rg]) and a table fine bin -> cell, so that
// cells are equally fine, relative to the codeword spacing, wherever the codebook is dense or
// sparse (G = 2.12 sqrt(K): a few cells per codeword, short candidate lists).
//
// Candidates.  Codeword j is listed for cell Q when its Voronoi region, widened to absorb fp32
// distance rounding, meets Q widened by 1e-3 of a fine bin (the lookup's own rounding):
//   1. prefilter: mindist^2(Q, c_j) <= U_Q (1 + 1e-5), U_Q = min_k maxdist^2(Q, c_k);
//   2. clip Q by the half-planes |p - c_j|^2 - |p - c_k|^2 <= 1e-6 (maxdist^2(Q, c_j) +
//      maxdist^2(Q, c_k)) for every other prefiltered k (double precision); j stays if the
//      polygon is not empty.
// The fp32 distance fl(fl(dx*dx) + fl(dy*dy)) is within 2.4e-7 relative of the exact one, so a
// codeword outside the list can neither beat nor tie the listed ones in fp32: the fp32 argmin
// over the list, ties to the lowest index (lists are in increasing index order), equals the
// argmin over all K codewords.  Points outside the grid use a scan in decreasing |c| that stops
// once |p| - |c| exceeds the distance to a known codeword (plus a 1e-5 margin); with Rg at 2.5
// times the codebook's extent such points do not occur for calibrated data (a Gaussian
// coordinate beyond 9 sigma), so that path only has to be correct, not fast.
#include <cmath>

#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

namespace {

constexpr int kIxGroup = 16;   // lanes per candidate polygon (at most that many vertices)

struct CellBox {
    double x0, x1, y0, y1;
};

__device__ CellBox cell_box(const IndexHeader& ih, const uint16_t* __restrict__ lo, int cell) {
    const int cx = cell % ih.G, cy = cell / ih.G;
    const double w = 1.0 / (double)ih.inv_w;   // the lookup bins by fp32 (p + R) * inv_w
    const double d = 1e-3 * w;
    CellBox q;
    q.x0 = -(double)ih.R + lo[cx] * w - d;
    q.x1 = -(double)ih.R + lo[cx + 1] * w + d;
    q.y0 = -(double)ih.R + lo[cy] * w - d;
    q.y1 = -(double)ih.R + lo[cy + 1] * w + d;
    return q;
}

__device__ __forceinline__ double maxd2(const CellBox& q, double px, double py) {
    double ax = fmax(fabs(px - q.x0), fabs(px - q.x1));
    double ay = fmax(fabs(py - q.y0), fabs(py - q.y1));
    return ax * ax + ay * ay;
}

__device__ __forceinline__ double mind2(const CellBox& q, double px, double py) {
    double dx = fmax(fmax(q.x0 - px, px - q.x1), 0.0);
    double dy = fmax(fmax(q.y0 - py, py - q.y1), 0.0);
    return dx * dx + dy * dy;
}

// Is codeword j a candidate of the (non-empty) cell box q?  pre[] holds the prefiltered set.
// Whether the Voronoi region of codeword j, widened by a margin, meets the cell box q: the box is
// clipped (Sutherland-Hodgman, double precision) by the half-plane |p - c_j|^2 - |p - c_k|^2 <= m of
// every other prefiltered codeword k, and the region meets the cell when something is left.  Each
// group of kIxGroup lanes tests its own candidate j (j < 0: none), its polygon's vertex l in lane l
// of the group: a clip tests each vertex and the next one, counts the vertices each lane emits (the
// vertex if inside, the crossing point if the edge crosses the line), places them by a ballot
// prefix count within the group and moves them through the group's part of the wavefront's LDS
// buffer.  The loop is uniform over the wavefront: a group that has its answer clips nothing
// further.  A polygon that would need more than kIxGroup vertices counts as meeting the cell (an
// extra list entry costs search time only).  Returns the answer of the lane's group.
__device__ bool voronoi_meets_group(const CellBox& q, const float2* __restrict__ cb, int j, const uint16_t* pre,
                                   int npre, double2* wbuf, int lane) {
    constexpr int kHalf = kIxGroup;   // lanes of a group
    const int h = lane / kHalf, gl = lane % kHalf;
    const uint64_t hmask = (~0ull >> (kWave - kHalf)) << (h * kHalf);
    double2* hb = wbuf + h * kHalf;
    double px = gl == 1 || gl == 2 ? q.x1 : q.x0;
    double py = gl >= 2 ? q.y1 : q.y0;
    int n = 4;
    bool done = j < 0, res = false;   // uniform within each group
    const int jj = j < 0 ? 0 : j;
    const double cjx = cb[jj].x, cjy = cb[jj].y;
    const double mj = maxd2(q, cjx, cjy);
    const double nj = cjx * cjx + cjy * cjy;
    for (int t = 0; t < npre; ++t) {
        if (__ballot(!done) == 0) break;   // every group has its answer
        const int k = pre[t];
        const double ckx = cb[k].x, cky = cb[k].y;
        const double m = 1e-6 * (mj + maxd2(q, ckx, cky));
        // |p-cj|^2 - |p-ck|^2 <= m   <=>   2 (ck - cj).p <= |ck|^2 - |cj|^2 + m
        double ax = 2.0 * (ckx - cjx), ay = 2.0 * (cky - cjy), b = (ckx * ckx + cky * cky) - nj + m;
        if (done || k == jj) {   // no clip for this group: every vertex stays
            ax = 0.0;
            ay = 0.0;
            b = 1.0;
        }
        const double tol = 1e-12 * (fabs(b) + 1.0);
        const int nx = gl + 1 == n ? 0 : gl + 1;
        const double px2 = __shfl(px, h * kHalf + nx, kWave), py2 = __shfl(py, h * kHalf + nx, kWave);
        const double s1 = ax * px + ay * py - b;
        const double s2 = ax * px2 + ay * py2 - b;
        const bool live = gl < n;
        const bool in1 = live && s1 <= tol;
        const bool cross = live && (s1 <= tol) != (s2 <= tol);
        const uint64_t ba = __ballot(in1) & hmask, bc = __ballot(cross) & hmask;
        const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ba >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ba, 0u)) +
                          (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bc >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bc, 0u));
        const int m2 = __popcll(ba) + __popcll(bc);
        if (!done && m2 > kHalf) {
            done = true;
            res = true;
        }
        if (!done && in1) hb[below] = make_double2(px, py);
        if (!done && cross) {
            const double tt = s1 / (s1 - s2);
            hb[below + (in1 ? 1 : 0)] = make_double2(px + tt * (px2 - px), py + tt * (py2 - py));
        }
        wave_lds_sync();
        if (!done) {
            n = m2;
            if (gl < n) {
                const double2 v = hb[gl];
                px = v.x;
                py = v.y;
            }
        }
        wave_lds_sync();   // read before the next clip overwrites the buffer
        if (!done && n == 0) {
            done = true;
            res = false;
        }
    }
    if (!done) res = n > 0;
    return res;
}

// ---------------------------------------------------------------------------------------------
// 1. Header, fine-bin table and cell edges (one workgroup).
__global__ __launch_bounds__(1024) void k_ix_grid(const float* __restrict__ cb, int K, int G, int W, int bits,
                                                  char* __restrict__ index) {
    __shared__ float red[1024];
    __shared__ int hist[kIndexFineMax];
    IndexHeader* hdr = reinterpret_cast<IndexHeader*>(index);
    uint8_t* fine = reinterpret_cast<uint8_t*>(index + kIndexFineOff);
    uint16_t* lo = reinterpret_cast<uint16_t*>(index + kIndexEdgeOff);
    const int tid = threadIdx.x;
    float m = 0.f;
    for (int j = tid; j < K; j += blockDim.x) {
        float2 c = reinterpret_cast<const float2*>(cb)[j];
        m = fmaxf(m, fmaxf(fabsf(c.x), fabsf(c.y)));   // NaN codewords are ignored by fmaxf
    }
    red[tid] = m;
    for (int b = tid; b < W; b += blockDim.x) hist[b] = 0;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
        __syncthreads();
    }
    float R = 2.5f * red[0];
    if (!(R >= 1e-3f) || !(R < 1e30f)) R = 1.0f;
    const float inv_w = (float)W / (2.0f * R);
    for (int j = tid; j < 2 * K; j += blockDim.x) {
        float v = cb[j];
        int b = (int)((v + R) * inv_w);
        b = b < 0 ? 0 : (b >= W ? W - 1 : b);
        if (v == v) atomicAdd(&hist[b], 1);
    }
    __syncthreads();
    if (tid == 0) {
        // fine bin b -> cell min(G-1, C(b) * G / (2K)), C(b) = coordinates in bins before b
        int c = 0, prev = -1;
        for (int b = 0; b < W; ++b) {
            int cell = (int)(((int64_t)c * G) / (2 * K));
            if (cell > G - 1) cell = G - 1;
            fine[b] = (uint8_t)cell;
            for (int e = prev + 1; e <= cell; ++e) lo[e] = (uint16_t)b;   // first fine bin of each cell
            prev = cell;
            c += hist[b];
        }
        for (int e = prev + 1; e <= G; ++e) lo[e] = (uint16_t)W;
        hdr->K = K;
        hdr->G = G;
        hdr->W = W;
        hdr->bits = bits;
        hdr->R = R;
        hdr->inv_w = inv_w;
        hdr->n_entries = 0;
        hdr->overflow = 0;
    }
}

// 2./4. Candidate lists: one workgroup per cell.  pass 0 counts, pass 1 writes the list in
// increasing codeword order at the cell's offset.
// LDS of k_ix_cells: the codebook (K float2), the prefiltered list (K uint16), one 64-vertex buffer
// per wavefront (kIxGroup vertices per lane group, 16-byte aligned), and a K-bit set of the
// codewords whose regions meet the cell.
constexpr int kIxCellsThreads = 256;
__host__ __device__ inline size_t ix_cells_wbuf_off(int K) { return ((size_t)K * 10 + 15) / 16 * 16; }
__host__ __device__ inline size_t ix_cells_bits_off(int K) {
    return ix_cells_wbuf_off(K) + (size_t)(kIxCellsThreads / kWave) * kWave * 16;
}
__host__ __device__ inline size_t ix_cells_lds(int K) { return ix_cells_bits_off(K) + (size_t)(K + 31) / 32 * 4; }

__global__ __launch_bounds__(kIxCellsThreads) void k_ix_cells(const float* __restrict__ cb, int K, char* __restrict__ index,
                                                  int pass) {
    extern __shared__ __align__(16) char smem[];
    float2* scb = reinterpret_cast<float2*>(smem);
    uint16_t* pre = reinterpret_cast<uint16_t*>(smem + (size_t)K * sizeof(float2));
    double2* wbuf = reinterpret_cast<double2*>(smem + ix_cells_wbuf_off(K)) + (threadIdx.x / kWave) * kWave;
    uint32_t* meets = reinterpret_cast<uint32_t*>(smem + ix_cells_bits_off(K));   // K bits
    __shared__ double redU[256];
    __shared__ int npre, wbase;
    __shared__ int scan[256];
    const IndexHeader ih = *reinterpret_cast<const IndexHeader*>(index);
    const uint16_t* lo = reinterpret_cast<const uint16_t*>(index + kIndexEdgeOff);
    uint32_t* offs = reinterpret_cast<uint32_t*>(index + kIndexOffsOff);
    uint16_t* ent = reinterpret_cast<uint16_t*>(index + kIndexEntOff);
    const int cell = blockIdx.x, tid = threadIdx.x;
    if (pass && reinterpret_cast<const uint8_t*>(index + kIndexOvfOff)[cell]) return;   // uniform per block
    for (int j = tid; j < K; j += blockDim.x) scb[j] = reinterpret_cast<const float2*>(cb)[j];
    for (int w = tid; w < (K + 31) / 32; w += blockDim.x) meets[w] = 0u;
    if (tid == 0) {
        npre = 0;
        wbase = 0;
    }
    const int cx = cell % ih.G, cy = cell / ih.G;
    const bool empty = lo[cx] == lo[cx + 1] || lo[cy] == lo[cy + 1];
    __syncthreads();
    const CellBox q = cell_box(ih, lo, cell);
    double U = 1e300;
    for (int j = tid; j < K; j += blockDim.x) U = fmin(U, maxd2(q, scb[j].x, scb[j].y));
    redU[tid] = U;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) redU[tid] = fmin(redU[tid], redU[tid + s]);
        __syncthreads();
    }
    const double lim = redU[0] * (1.0 + 1e-5);
    // prefilter (order within pre[] does not matter)
    for (int j = tid; j < K; j += blockDim.x) {
        if (!empty && mind2(q, scb[j].x, scb[j].y) <= lim) {
            int at = atomicAdd(&npre, 1);
            pre[at] = (uint16_t)j;
        }
    }
    __syncthreads();
    const int np = npre;
    // the prefiltered codewords whose regions meet the cell
    {
        const int lane = tid & (kWave - 1);
        const int nw = blockDim.x / kWave;
        // kWave / kIxGroup candidates per wavefront at a time, one per lane group
        constexpr int kPer = kWave / kIxGroup;
        for (int i0 = kPer * __builtin_amdgcn_readfirstlane(tid / kWave); i0 < np; i0 += kPer * nw) {
            const int i = i0 + lane / kIxGroup;
            const int j = i < np ? pre[i] : -1;
            const bool hit = voronoi_meets_group(q, scb, j, pre, np, wbuf, lane);
            if (hit && j >= 0 && lane % kIxGroup == 0) atomicOr(&meets[j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();
    uint32_t count = 0;
    const uint32_t base = pass ? offs[cell] : 0u;
    // candidates in increasing j: chunks of 256 codewords, ordered by a workgroup prefix sum
    for (int j0 = 0; j0 < K; j0 += blockDim.x) {
        const int j = j0 + tid;
        int is = 0;
        if (!empty && j < K) is = (int)((meets[j >> 5] >> (j & 31)) & 1u);
        scan[tid] = is;
        __syncthreads();
        for (int s = 1; s < 256; s <<= 1) {
            int v = (tid >= s) ? scan[tid - s] : 0;
            __syncthreads();
            scan[tid] += v;
            __syncthreads();
        }
        const int total = scan[255];
        if (pass && is) ent[base + count + scan[tid] - 1] = (uint16_t)j;
        count += total;
        __syncthreads();
    }
    if (tid == 0 && !pass) offs[cell] = count;   // counts; turned into offsets by k_ix_scan
}

// 3. Exclusive prefix sum of the counts (one workgroup); cells beyond the entry budget are
// marked as overflow (count 0, searched exhaustively).
__global__ __launch_bounds__(1024) void k_ix_scan(char* __restrict__ index, int max_entries) {
    IndexHeader* hdr = reinterpret_cast<IndexHeader*>(index);
    uint32_t* offs = reinterpret_cast<uint32_t*>(index + kIndexOffsOff);
    uint8_t* ovf = reinterpret_cast<uint8_t*>(index + kIndexOvfOff);
    if (threadIdx.x != 0) return;
    const int cells = hdr->G * hdr->G;
    uint32_t acc = 0;
    int over = 0;
    for (int c = 0; c < cells; ++c) {
        uint32_t n = offs[c];
        offs[c] = acc;
        if (acc + n > (uint32_t)max_entries || n > kIndexCellCap) {
            ovf[c] = 1;
            ++over;
        } else {
            ovf[c] = 0;
            acc += n;
        }
    }
    offs[cells] = acc;
    hdr->n_entries = (int)acc;
    hdr->overflow = over;
}

// 5. Codewords in decreasing |c| (ties: lower index first), for points outside the grid.
__global__ __launch_bounds__(256) void k_ix_order(const float* __restrict__ cb, int K, char* __restrict__ index) {
    uint16_t* order = reinterpret_cast<uint16_t*>(index + kIndexOrderOff);
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K) return;
    const float2 cj = reinterpret_cast<const float2*>(cb)[j];
    const double nj = __builtin_sqrt((double)cj.x * cj.x + (double)cj.y * cj.y);
    int rank = 0;
    for (int k = 0; k < K; ++k) {
        const float2 ck = reinterpret_cast<const float2*>(cb)[k];
        const double nk = __builtin_sqrt((double)ck.x * ck.x + (double)ck.y * ck.y);
        rank += (nk > nj || (nk == nj && k < j)) ? 1 : 0;
    }
    order[rank] = (uint16_t)j;
}

// 6. The LDS image (layout of search_image_layout): codebook, fine-bin table, list offsets as
// u16 (clamped to the entries kept), lists as byte offsets 8 j, then zeros.
__global__ __launch_bounds__(256) void k_ix_image(const float* __restrict__ cb, int K, char* __restrict__ index) {
    const IndexHeader& ih = *reinterpret_cast<const IndexHeader*>(index);
    const SearchImageLayout l = search_image_layout(K, ih.G);
    char* img = index + kIndexImgOff;
    const uint32_t* offs = reinterpret_cast<const uint32_t*>(index + kIndexOffsOff);
    const uint16_t* ent = reinterpret_cast<const uint16_t*>(index + kIndexEntOff);
    const uint8_t* fine = reinterpret_cast<const uint8_t*>(index + kIndexFineOff);
    const uint32_t ne = (uint32_t)min(ih.n_entries, index_lds_entries(K));
    const int cells = ih.G * ih.G;
    const int stride = gridDim.x * blockDim.x;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < (int)(l.bytes / 2); i += stride) {
        const size_t byte = (size_t)i * 2;   // one u16 of the image per step
        uint16_t v = 0;
        if (byte < l.fine) {
            v = reinterpret_cast<const uint16_t*>(cb)[i];
        } else if (byte < l.offs) {
            const size_t b = byte - l.fine;
            if (b + 1 < (size_t)kIndexFine) v = (uint16_t)(fine[b] | (fine[b + 1] << 8));
        } else if (byte < l.ent) {
            const size_t c = (byte - l.offs) / 2;
            if (c <= (size_t)cells) v = (uint16_t)min(offs[c], ne);
        } else {
            const size_t e = (byte - l.ent) / 2;
            if (e < ne) v = (uint16_t)(8u * ent[e]);
        }
        reinterpret_cast<uint16_t*>(img)[i] = v;
    }
}

}  // namespace

int index_grid_size(int bits) {
    // G = 2.12 sqrt(K): about 4.5 cells per codeword, so a point's list holds 2.5 codewords on
    // average and at most about 7 (Gaussian-trained codebooks); K = 4096 uses G = 64 to keep the
    // LDS image (codebook, offsets, lists) below about 90 KiB.
    const int K = 1 << bits;
    if (K >= 4096) return 64;
    int G = (int)std::lround(2.12 * std::sqrt((double)K));
    return G < 4 ? 4 : (G > kIndexGMax ? kIndexGMax : G);
}

size_t index_bytes_for(int bits) {
    return kIndexImgOff + search_lds_bytes(1 << bits, index_grid_size(bits));
}

hipError_t launch_index_build(const float* cb, int bits, void* index, hipStream_t st) {
    const int K = 1 << bits;
    const int G = index_grid_size(bits);
    char* ix = reinterpret_cast<char*>(index);
    hipLaunchKernelGGL(k_ix_grid, dim3(1), dim3(1024), 0, st, cb, K, G, kIndexFine, bits, ix);
    const size_t smem = ix_cells_lds(K);
    allow_lds(k_ix_cells, smem);
    hipLaunchKernelGGL(k_ix_cells, dim3(G * G), dim3(kIxCellsThreads), smem, st, cb, K, ix, 0);
    hipLaunchKernelGGL(k_ix_scan, dim3(1), dim3(64), 0, st, ix, index_lds_entries(K));
    hipLaunchKernelGGL(k_ix_cells, dim3(G * G), dim3(kIxCellsThreads), smem, st, cb, K, ix, 1);
    hipLaunchKernelGGL(k_ix_order, dim3((K + 255) / 256), dim3(256), 0, st, cb, K, ix);
    hipLaunchKernelGGL(k_ix_image, dim3(64), dim3(256), 0, st, cb, K, ix);
    return hipGetLastError();
}

namespace {

__global__ __launch_bounds__(256) void k_nearest(const float* __restrict__ pts, int64_t n, const float* __restrict__ cb,
                                                 int K, int G, const char* __restrict__ index,
                                                 int32_t* __restrict__ out) {
    extern __shared__ __align__(16) char smem[];
    const IndexHeader ih = *reinterpret_cast<const IndexHeader*>(index);
    if (!index_header_ok(ih, K, G)) {   // an index of another codebook size: every answer is -1
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
            out[i] = -1;
        return;
    }
    SearchLds s = search_lds_carve(smem, K, ih, index);
    search_lds_fill(s, index, K, threadIdx.x, blockDim.x);
    __syncthreads();
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float2 p = reinterpret_cast<const float2*>(pts)[i];
        out[i] = nearest_lds(p.x, p.y, s);
    }
}

}  // namespace

hipError_t launch_nearest(const float* pts, int64_t n, const float* cb, int bits, const void* index, int32_t* out,
                          hipStream_t st) {
    const int K = 1 << bits;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) return hipSuccess;
    const int G = index_grid_size(bits);
    const size_t smem = search_lds_bytes(K, G);
    allow_lds(k_nearest, smem);
    hipLaunchKernelGGL(k_nearest, dim3((unsigned)blocks), dim3(256), smem, st, pts, n, cb, K, G,
                       reinterpret_cast<const char*>(index), out);
    return hipGetLastError();
}

}  // namespace qamw
