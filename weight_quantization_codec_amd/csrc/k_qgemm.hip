// Fused dequantize-and-multiply (paper section 1: the matrix product that follows the decoder)
// for M activation rows:  y[m][i] = sum_j x[m][j] w^_ij,  w^ the decoder's output before rounding.
//
// W^ is never formed.  With D = diag(eps_j / s_j) and the block transform H = blockdiag(H_b)/sqrt(b)
// symmetric, row i of W^ is f16(norm_i) D H z_i with z_i,2k = sigma_k c[idx_ik].x (and .y), so
//   sum_j x_j w^_ij = f16(norm_i) sum_k (c[idx_ik] . u_k),   u_k = sigma_k (H D x)_(2k, 2k+1).
// k_qgemm_rotate forms u once per activation row (fp64, rounded to fp32 once); k_qgemm then costs
// one codebook lookup per weight pair and two FMAs per pair and activation row, reading only the
// packed codes (B/16 bytes per weight) from HBM.
//
// k_qgemm: 16 wavefronts per workgroup share an LDS copy of the codebook and of u for up to four
// activation rows (an "m-tile") over up to four passes of 2048 pairs.  A wavefront owns a row at a
// time; in a pass lane l owns the 32 consecutive pairs l*32 .. l*32 + 31, whose 32 B code bits start
// on a dword boundary, so its B dwords come in with dword-aligned buffer loads and the indices come
// out with shifts.  The work items (row, pass) of a wavefront are prefetched one ahead.  Rows wider
// than the LDS tile are split over the grid's z dimension; a second kernel adds the partial sums in
// a fixed order and applies the norm.
#include <hip/hip_fp16.h>

#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQgThreads = 1024;        // 16 wavefronts
constexpr int kQgPass = 2048;           // pairs per pass: 64 lanes x 32
constexpr int kQgPadLanes = kWave + 1;  // u tile row pitch (float2): conflict-free reads, 2-way writes
constexpr int kQgMaxTile = 4;           // m-tile rows x passes held in LDS

// ---------------------------------------------------------------------------- activation rotation
// u[m][j] (fp32, pairs interleaved) = sigma_(j/2) * (blockdiag(H_b) (eps . x_m / s))_j / sqrt(b), the
// transform as unnormalized fp64 butterflies in LDS.  Workgroup: T = max(b, 256) columns of one
// activation row (whole blocks); columns past d_in carry zeros.
//   frag == 0: u row-major, M x d_in.
//   frag == 1: the operand order of k_qgemm_mfma, for 16 rows (rows m >= M are zeros) and the
//              columns padded to whole chunks of 64 pairs (zeros): u of pair k = 64 c + 32 h + s,
//              component e, row m goes to ((c * 8 + s / 4) * 64 + (2 h + e) * 16 + m) * 4 + s % 4.
__global__ __launch_bounds__(1024) void k_qgemm_rotate(const void* __restrict__ x, int x_bf16, int64_t ld_x, int M,
                                                       int d_in, int cols, int b, const float* __restrict__ s,
                                                       uint64_t sign_seed,
                                                       const float* __restrict__ sigma, float* __restrict__ u,
                                                       int frag) {
    extern __shared__ double buf[];
    const int m = blockIdx.y;
    const int tid = threadIdx.x;
    const int col = blockIdx.x * blockDim.x + tid;
    double v = 0.0;
    if (col < d_in && m < M) {
        const float xv = x_bf16 ? bf16_bits_to_float(reinterpret_cast<const uint16_t*>(x)[(size_t)m * ld_x + col])
                                : reinterpret_cast<const float*>(x)[(size_t)m * ld_x + col];
        const double sc = s ? (double)s[col] : 1.0;
        const bool neg = eps_negative(sign_seed, (uint32_t)col);
        v = (neg ? -(double)xv : (double)xv) / sc;
    }
    buf[tid] = v;
    for (int h = 1; h < b; h <<= 1) {
        __syncthreads();
        const double a = buf[tid], c = buf[tid ^ h];
        __syncthreads();
        buf[tid] = (tid & h) ? c - a : a + c;
    }
    __syncthreads();
    if (col >= cols) return;
    const float r = col < d_in ? (float)(buf[tid] * (1.0 / __builtin_sqrt((double)b)) * (double)sigma[col >> 1]) : 0.0f;
    if (!frag) {
        u[(size_t)m * d_in + col] = r;
    } else {
        const int k = col >> 1, e = col & 1;
        const int c = k >> 6, h = (k >> 5) & 1, st = k & 31;
        u[(((size_t)c * 8 + (st >> 2)) * kWave + (2 * h + e) * 16 + m) * 4 + (st & 3)] = r;
    }
}

// ---------------------------------------------------------------------------- the product
// N consecutive dwords from byte offset off of a buffer (dword-aligned; dwords past the descriptor's
// size read as 0).
template <int N>
__device__ __forceinline__ void qg_load(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t (&d)[N]) {
#pragma unroll
    for (int c = 0; c + 4 <= N; c += 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 4 * c, 0, 0);
        d[c] = v[0];
        d[c + 1] = v[1];
        d[c + 2] = v[2];
        d[c + 3] = v[3];
    }
    constexpr int c = N / 4 * 4;
    if constexpr (N - c == 3) {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rs, off + 4 * c, 0, 0);
        d[c] = v[0];
        d[c + 1] = v[1];
        d[c + 2] = v[2];
    } else if constexpr (N - c == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 4 * c, 0, 0);
        d[c] = v[0];
        d[c + 1] = v[1];
    } else if constexpr (N - c == 1) {
        d[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * c, 0, 0);
    }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);   // v_cvt_pk_bf16_f32: round to nearest even
}

// Sum over the wavefront (fp32, fixed order), returned to every lane: DPP moves within rows of 16,
// then the row broadcasts into lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dppf(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_sum_f(float v) {
    v += dppf<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v += dppf<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v += dppf<0x141, 0xF>(v);   // row_half_mirror
    v += dppf<0x140, 0xF>(v);   // row_mirror
    v += dppf<0x142, 0xA>(v);   // row_bcast:15
    v += dppf<0x143, 0xC>(v);   // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

template <int BITS, int MT>
__global__ __launch_bounds__(kQgThreads) void k_qgemm(QgemmArgs a) {
    extern __shared__ __align__(16) char smem[];
    const int K = 1 << BITS;
    float2* cb_l = reinterpret_cast<float2*>(smem);
    float2* u_l = reinterpret_cast<float2*>(smem + (size_t)K * sizeof(float2));
    // the wavefront index as a scalar: rows and buffer descriptors derived from it stay uniform
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave),
              nw = blockDim.x / kWave;
    const int m0 = blockIdx.y * MT;                          // first activation row of the m-tile
    const int pass0 = blockIdx.z * a.pps;                    // first pass of this split
    const int np_here = min(a.pps, a.n_pass - pass0);        // passes in this split (>= 1)

    constexpr uint32_t mask = (1u << BITS) - 1u;
    const int rstride = gridDim.x * nw;
    // work items of this wavefront: (row, pass) for rows wave0, wave0 + rstride, ...
    int row = blockIdx.x * nw + wave, p = 0;
    auto codes_rsrc = [&](int r) {
        const bool ok = r < a.d_out;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(a.codes + (size_t)(ok ? r : 0) * a.stride), (short)0,
                                                 ok ? (int)a.stride : 0, 0x00020000);
    };
    auto lane_off = [&](int pp) { return (uint32_t)(((pass0 + pp) * kWave + lane) * BITS) * 4u; };
    // the first work item's codes are in flight while the LDS tables fill
    uint32_t nxt[BITS];
    if (row < a.d_out) qg_load<BITS>(codes_rsrc(row), lane_off(0), nxt);

    // codebook and the u tile: u_l[((p * MT + m) * 32 + t) * 65 + l] = u pair (pass0 + p) * 2048 + l * 32 + t
    // every load of a thread issued before its stores: at most K / 1024 <= 4 codebook entries and
    // kQgMaxTile * 2048 / 1024 = 8 u values per thread
    {
        float2 cv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = threadIdx.x + j * kQgThreads;
            cv[j] = k < K ? reinterpret_cast<const float2*>(a.cb)[k] : make_float2(0.0f, 0.0f);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = threadIdx.x + j * kQgThreads;
            if (k < K) cb_l[k] = cv[j];
        }
    }
    const int tile = np_here * MT * kQgPass;
    {
        float2 uv[kQgMaxTile * kQgPass / kQgThreads];
#pragma unroll
        for (int j = 0; j < kQgMaxTile * kQgPass / kQgThreads; ++j) {
            const int q = threadIdx.x + j * kQgThreads;
            const int p = q / (MT * kQgPass), r = q - p * (MT * kQgPass);
            const int m = r / kQgPass, kk = r - m * kQgPass;     // kk = l * 32 + t: consecutive global pairs
            const int k = (pass0 + p) * kQgPass + kk;
            uv[j] = make_float2(0.0f, 0.0f);
            if (q < tile && m0 + m < a.M && k < a.n_pairs)
                uv[j] = reinterpret_cast<const float2*>(a.u)[(size_t)(m0 + m) * a.n_pairs + k];
        }
#pragma unroll
        for (int j = 0; j < kQgMaxTile * kQgPass / kQgThreads; ++j) {
            const int q = threadIdx.x + j * kQgThreads;
            const int p = q / (MT * kQgPass), r = q - p * (MT * kQgPass);
            const int m = r / kQgPass, kk = r - m * kQgPass;
            if (q < tile) u_l[((p * MT + m) * 32 + (kk & 31)) * kQgPadLanes + (kk >> 5)] = uv[j];
        }
    }
    __syncthreads();

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    while (row < a.d_out) {
        uint32_t d[BITS];
#pragma unroll
        for (int c = 0; c < BITS; ++c) d[c] = nxt[c];
        // the next work item, in flight while this one computes
        int nrow = row, np2 = p + 1;
        if (np2 == np_here) {
            np2 = 0;
            nrow = row + rstride;
        }
        if (nrow < a.d_out) qg_load<BITS>(codes_rsrc(nrow), lane_off(np2), nxt);
        const float2* ut = u_l + (size_t)(p * MT) * 32 * kQgPadLanes + lane;
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const int off = t * BITS, w = off >> 5, sh = off & 31;
            const uint32_t v = (sh + BITS <= 32) ? (d[w] >> sh) : __builtin_amdgcn_alignbit(d[w + 1], d[w], sh);
            const float2 c = cb_l[v & mask];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float2 uu = ut[(m * 32 + t) * kQgPadLanes];
                acc[m] = __builtin_fmaf(c.x, uu.x, acc[m]);
                acc[m] = __builtin_fmaf(c.y, uu.y, acc[m]);
            }
        }
        if (p + 1 == np_here) {   // the row is done: reduce and store
            const float nrm = __half2float(__ushort_as_half(a.norm[row]));
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float sum = wave_sum_f(acc[m]);
                acc[m] = 0.0f;
                if (lane == m && m0 + m < a.M) {
                    if (a.partial) {
                        a.partial[((size_t)blockIdx.z * a.M + (m0 + m)) * a.d_out + row] = sum;
                    } else if (a.y_bf16) {
                        const float yv = sum * nrm;
                        reinterpret_cast<uint16_t*>(a.y)[(size_t)(m0 + m) * a.ld_y + row] = f32_to_bf16_rne(yv);
                    } else {
                        reinterpret_cast<float*>(a.y)[(size_t)(m0 + m) * a.ld_y + row] = sum * nrm;
                    }
                }
            }
        }
        row = nrow;
        p = np2;
    }
}

// The product on the matrix cores: v_mfma_f32_16x16x4f32, D[16 x 16] += A[16 x 4] B[4 x 16] in fp32,
// with A = 16 weight rows x 4 of their rotated-domain values (codebook components) and B = the same
// 4 values of u for 16 activation rows.  Lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and
// holds D[4 (l / 16) + v][l % 16] (v = 0..3).  The 4 k-slots of a step are (pair s, x), (pair s, y),
// (pair 32 + s, x), (pair 32 + s, y) of a chunk of 64 pairs, so lane (r, q) reads the codes of row
// r for pairs 32 (q / 2) .. + 31 of the chunk: 32 B bits, dword-aligned, as in k_qgemm.
// Workgroup: one tile of 16 rows, kQmWaves wavefronts taking the chunks c = w, w + kQmWaves, ...;
// their partial D are added in LDS in wavefront order.
constexpr int kQmWaves = 4;

template <int BITS>
__global__ __launch_bounds__(kQmWaves * kWave) void k_qgemm_mfma(QgemmArgs a) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    extern __shared__ __align__(16) char smem[];
    const int K = 1 << BITS;
    float* cbf = reinterpret_cast<float*>(smem);                                   // K x 2
    f32x4* part = reinterpret_cast<f32x4*>(smem + (size_t)K * sizeof(float2));     // kQmWaves x 64
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    {   // the codebook: every load issued before the stores (K / 2 <= 2048 float4)
        typedef float f4 __attribute__((ext_vector_type(4)));
        constexpr int kPer = (2048 + kQmWaves * kWave - 1) / (kQmWaves * kWave);   // float4 per thread
        const f4* src = reinterpret_cast<const f4*>(a.cb);
        f4* dst = reinterpret_cast<f4*>(cbf);
        const int n4 = K / 2;   // K >= 2
        f4 v[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int t = threadIdx.x + j * kQmWaves * kWave;
            v[j] = t < n4 ? src[t] : f4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int t = threadIdx.x + j * kQmWaves * kWave;
            if (t < n4) dst[t] = v[j];
        }
    }
    __syncthreads();
    const int r = lane & 15, q = lane >> 4, h = q >> 1, e = q & 1;
    const float* cbe = cbf + e;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    const int n_chunks = (a.n_pairs + 63) / 64;
    const int n_tiles = (a.d_out + 15) / 16;
    const f32x4* uf = reinterpret_cast<const f32x4*>(a.u);
    for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        // one descriptor for the tile's rows (a descriptor must be uniform over the wavefront); a row
        // past the end lies past the descriptor's range and reads zeros
        const int row0 = tile * 16;
        const int nrows = a.d_out - row0 < 16 ? a.d_out - row0 : 16;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.codes + (size_t)row0 * a.stride), (short)0, nrows * (int)a.stride, 0x00020000);
        const uint32_t row_off = (uint32_t)r * (uint32_t)a.stride;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};   // even and odd steps
        int c = wave;
        uint32_t nd[BITS];
        f32x4 nu[8];
        auto load = [&](int cc) {
            qg_load<BITS>(rs, row_off + (uint32_t)((2 * cc + h) * BITS) * 4u, nd);
#pragma unroll
            for (int j = 0; j < 8; ++j) nu[j] = uf[((size_t)cc * 8 + j) * kWave + lane];
        };
        if (c < n_chunks) load(c);
        for (; c < n_chunks; c += kQmWaves) {
            uint32_t d[BITS];
            f32x4 uu[8];
#pragma unroll
            for (int j = 0; j < BITS; ++j) d[j] = nd[j];
#pragma unroll
            for (int j = 0; j < 8; ++j) uu[j] = nu[j];
            if (c + kQmWaves < n_chunks) load(c + kQmWaves);
#pragma unroll
            for (int st = 0; st < 32; ++st) {
                const int off = st * BITS, w = off >> 5, sh = off & 31;
                const uint32_t v = (sh + BITS <= 32) ? (d[w] >> sh) : __builtin_amdgcn_alignbit(d[w + 1], d[w], sh);
                const float av = cbe[2 * (v & mask)];
                if (st & 1)
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av, uu[st >> 2][st & 3], acc1, 0, 0, 0);
                else
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, uu[st >> 2][st & 3], acc, 0, 0, 0);
            }
        }
        acc[0] += acc1[0];
        acc[1] += acc1[1];
        acc[2] += acc1[2];
        acc[3] += acc1[3];
        part[wave * kWave + lane] = acc;
        __syncthreads();
        if (wave == 0) {
            f32x4 sum = part[lane];
#pragma unroll
            for (int w2 = 1; w2 < kQmWaves; ++w2) {
                const f32x4 p2 = part[w2 * kWave + lane];
                sum[0] += p2[0];
                sum[1] += p2[1];
                sum[2] += p2[2];
                sum[3] += p2[3];
            }
            const int m = lane & 15;
#pragma unroll
            for (int v2 = 0; v2 < 4; ++v2) {
                const int orow = tile * 16 + 4 * q + v2;
                if (m < a.M && orow < a.d_out) {
                    const float yv = sum[v2] * __half2float(__ushort_as_half(a.norm[orow]));
                    if (a.y_bf16)
                        reinterpret_cast<uint16_t*>(a.y)[(size_t)m * a.ld_y + orow] = f32_to_bf16_rne(yv);
                    else
                        reinterpret_cast<float*>(a.y)[(size_t)m * a.ld_y + orow] = yv;
                }
            }
        }
        __syncthreads();   // part is reused by the next tile
    }
}

// y[m][i] = f16(norm_i) * sum over splits z (in order) of partial[z][m][i].
__global__ __launch_bounds__(256) void k_qgemm_reduce(QgemmArgs a, int splits) {
    const int64_t n = (int64_t)a.M * a.d_out;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n; q += (int64_t)gridDim.x * blockDim.x) {
        const int m = (int)(q / a.d_out), i = (int)(q - (int64_t)m * a.d_out);
        float sum = 0.0f;
        for (int z = 0; z < splits; ++z) sum += a.partial[((size_t)z * a.M + m) * a.d_out + i];
        const float yv = sum * __half2float(__ushort_as_half(a.norm[i]));
        if (a.y_bf16)
            reinterpret_cast<uint16_t*>(a.y)[(size_t)m * a.ld_y + i] = f32_to_bf16_rne(yv);
        else
            reinterpret_cast<float*>(a.y)[(size_t)m * a.ld_y + i] = yv;
    }
}

template <int BITS>
hipError_t qgemm_B(QgemmArgs a, const QgemmPlan& pl, hipStream_t st) {
    const size_t smem = qgemm_lds_bytes(BITS, pl.mt, pl.pps);
    const dim3 grid(pl.grid_x, pl.mtiles, pl.splits);
    a.pps = pl.pps;
    a.n_pass = pl.n_pass;
    switch (pl.mt) {
    case 1:
        allow_lds(k_qgemm<BITS, 1>, smem);
        hipLaunchKernelGGL((k_qgemm<BITS, 1>), grid, dim3(kQgThreads), smem, st, a);
        break;
    case 2:
        allow_lds(k_qgemm<BITS, 2>, smem);
        hipLaunchKernelGGL((k_qgemm<BITS, 2>), grid, dim3(kQgThreads), smem, st, a);
        break;
    default:
        allow_lds(k_qgemm<BITS, 4>, smem);
        hipLaunchKernelGGL((k_qgemm<BITS, 4>), grid, dim3(kQgThreads), smem, st, a);
        break;
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    if (pl.splits > 1) {
        const int64_t n = (int64_t)a.M * a.d_out;
        const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
        hipLaunchKernelGGL(k_qgemm_reduce, dim3(blocks), dim3(256), 0, st, a, pl.splits);
    }
    return hipGetLastError();
}

}  // namespace

size_t qgemm_lds_bytes(int bits, int mt, int pps) {
    return (size_t)(1 << bits) * sizeof(float2) + (size_t)pps * mt * 32 * kQgPadLanes * sizeof(float2);
}

QgemmPlan qgemm_plan(int M, int d_out, int d_in) {
    QgemmPlan pl{};
    const int n_pairs = d_in / 2;
    pl.n_pass = (n_pairs + kQgPass - 1) / kQgPass;
    pl.mt = M <= 1 ? 1 : (M == 2 ? 2 : 4);
    pl.mtiles = M > 0 ? (M + pl.mt - 1) / pl.mt : 1;
    pl.pps = kQgMaxTile / pl.mt;
    if (pl.pps > pl.n_pass) pl.pps = pl.n_pass;
    if (pl.pps < 1) pl.pps = 1;
    pl.splits = (pl.n_pass + pl.pps - 1) / pl.pps;
    const int rows_per_wg = kQgThreads / kWave;
    const int need = (d_out + rows_per_wg - 1) / rows_per_wg;
    int gx = 256 / (pl.mtiles * pl.splits);
    if (gx < 1) gx = 1;
    pl.grid_x = gx < need ? gx : need;
    return pl;
}

// Below this many activation rows the VALU kernel runs, from it on the matrix-core kernel (which
// costs the same for any M <= 16; measured crossover on the 4096 x 4096 and 13B shapes).
constexpr int kQgMfmaMinM = 6;

size_t qgemm_workspace(int M, int d_out, int d_in) {
    const QgemmPlan pl = qgemm_plan(M, d_out, d_in);
    const size_t u = ((size_t)M * d_in * sizeof(float) + 255) / 256 * 256;
    const size_t part = pl.splits > 1 ? (size_t)pl.splits * M * d_out * sizeof(float) : 0;
    const size_t n_chunks = ((size_t)d_in / 2 + 63) / 64;
    const size_t frag = n_chunks * 8 * kWave * 4 * sizeof(float);   // 16 rows x 128 columns per chunk
    return M >= kQgMfmaMinM ? frag : u + part;   // the launcher takes the same branch
}

template <int BITS>
hipError_t qgemm_mfma_B(const QgemmArgs& a, hipStream_t st) {
    const size_t smem = (size_t)(1 << BITS) * sizeof(float2) + (size_t)kQmWaves * kWave * 4 * sizeof(float);
    const int n_tiles = (a.d_out + 15) / 16;
    const int grid = n_tiles < 2048 ? n_tiles : 2048;
    allow_lds(k_qgemm_mfma<BITS>, smem);
    hipLaunchKernelGGL(k_qgemm_mfma<BITS>, dim3(grid), dim3(kQmWaves * kWave), smem, st, a);
    return hipGetLastError();
}

hipError_t launch_qgemm(const QgemmArgs& a0, const QgemmRotateArgs& r, hipStream_t st) {
    QgemmArgs a = a0;
    const bool mfma = a.M >= kQgMfmaMinM;
    // activation rotation
    const int T = r.block > 256 ? r.block : 256;
    const int cols = mfma ? (r.d_in / 2 + 63) / 64 * 128 : r.d_in;
    hipLaunchKernelGGL(k_qgemm_rotate, dim3((cols + T - 1) / T, mfma ? 16 : a.M), dim3(T), (size_t)T * sizeof(double),
                       st, r.x, r.x_bf16, r.ld_x, a.M, r.d_in, cols, r.block, r.scale, r.sign_seed, r.sigma, a.u,
                       mfma ? 1 : 0);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
#define QAMW_QG(b) \
    case b: return mfma ? qgemm_mfma_B<b>(a, st) : qgemm_B<b>(a, pl, st);
    const QgemmPlan pl = qgemm_plan(a.M, a.d_out, r.d_in);
    if (pl.splits <= 1) a.partial = nullptr;
    switch (a.bits) {
        QAMW_QG(1) QAMW_QG(2) QAMW_QG(3) QAMW_QG(4) QAMW_QG(5) QAMW_QG(6)
        QAMW_QG(7) QAMW_QG(8) QAMW_QG(9) QAMW_QG(10) QAMW_QG(11) QAMW_QG(12)
    default: return hipErrorInvalidValue;
    }
#undef QAMW_QG
}

}  // namespace qamw
