// QAM-W encoder (paper section 3.1) with pair calibration (section 3.4) and the
// activation-aware channel scale (section 3.8).
//
// One workgroup owns one row at a time (rows strided over the grid) and keeps the row in
// registers from the single HBM read to the packed codes:
//   load  -> a_j = w_ij * s_j * eps_j (double, exact), partial sum of a_j^2
//   FWHT  -> unnormalized Sylvester transform of each block, double butterflies in registers,
//            one LDS exchange per wavefront (layout in qamw_device.hpp)
//   norm  -> r = sqrt(sum a^2) over the workgroup (wave shuffles + one barrier)
//   pairs -> p_k = fl32(t_2k * (1/sqrt(b)) / r / sigma_k), nearest codeword via the grid index
//   pack  -> indices through LDS, one 32-bit word per thread, coalesced stores; f16(fl32(r)).
// The calibration kernel runs the same front end on rows 0 .. min(d_out, 1024) - 1 and sums
// |z_k| per pair in double; a finishing kernel adds the per-group sums in a fixed order.
#include <hip/hip_fp16.h>

#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

namespace {

constexpr int kMaxWaves = 16;
constexpr int kCalibMaxGroups = 256;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ double eps_of(const uint32_t* sign, int j) {
    return (sign && ((sign[j >> 5] >> (j & 31)) & 1u)) ? -1.0 : 1.0;
}

// Column of register m of this lane in the final (phase B) layout.
template <int L>
__device__ __forceinline__ int col_B(int tid, int m) {
    using Lo = Layout<L>;
    if constexpr (Lo::two_phase) {
        return (tid / Lo::lanes) * Lo::b + Lo::jB(tid % Lo::lanes, m);
    } else {
        return tid * Lo::E + m;
    }
}

// Raw bits of the E consecutive weights a lane reads from one row (bf16: two per dword).
template <int E, bool BF>
struct RawW {
    static constexpr int N = BF ? E / 2 : E;
    uint32_t u[N];
};

template <int E, bool BF>
__device__ __forceinline__ void load_raw(const void* w, bool vec, int64_t off, RawW<E, BF>& r) {
    if constexpr (BF) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(w) + off;
        if (vec) {
#pragma unroll
            for (int v = 0; v < E / 8; ++v) {
                uint4 q = reinterpret_cast<const uint4*>(p)[v];
                r.u[4 * v] = q.x;
                r.u[4 * v + 1] = q.y;
                r.u[4 * v + 2] = q.z;
                r.u[4 * v + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int m = 0; m < E / 2; ++m) r.u[m] = (uint32_t)p[2 * m] | ((uint32_t)p[2 * m + 1] << 16);
        }
    } else {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(w) + off;
        if (vec) {
#pragma unroll
            for (int v = 0; v < E / 4; ++v) {
                uint4 q = reinterpret_cast<const uint4*>(p)[v];
                r.u[4 * v] = q.x;
                r.u[4 * v + 1] = q.y;
                r.u[4 * v + 2] = q.z;
                r.u[4 * v + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int m = 0; m < E; ++m) r.u[m] = p[m];
        }
    }
}

// a_j = w_j * s_j * eps_j in double (exact), accumulating sum a_j^2.
template <int E, bool BF>
__device__ __forceinline__ void scale_raw(const RawW<E, BF>& r, const double (&cf)[E], double (&x)[E], double& ss,
                                          int32_t& flags) {
#pragma unroll
    for (int m = 0; m < E; ++m) {
        float f;
        if constexpr (BF)
            f = __uint_as_float((m & 1) ? (r.u[m >> 1] & 0xFFFF0000u) : (r.u[m >> 1] << 16));
        else
            f = __uint_as_float(r.u[m]);
        double a = (double)f * cf[m];
        if (!__builtin_isfinite(a)) flags |= 1;
        x[m] = a;
        ss += a * a;
    }
}

// Front end for one row given its raw weights: x <- unnormalized transform (phase B layout);
// returns sum a^2 over the whole row (fixed shuffle tree, then wavefronts in order).
template <int L, bool BF>
__device__ __forceinline__ double front_end(const RawW<Layout<L>::E, BF>& raw, bool active, int tid,
                                            const double (&cf)[Layout<L>::E], double (&x)[Layout<L>::E],
                                            double* red, double* xb, int nwaves, int32_t& flags) {
    using Lo = Layout<L>;
    constexpr int E = Lo::E;
    double ss = 0.0;
    if (active) {
        scale_raw<E, BF>(raw, cf, x, ss, flags);
    } else {
#pragma unroll
        for (int m = 0; m < E; ++m) x[m] = 0.0;
    }
    ss = wave_sum(ss);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
    if constexpr (Lo::two_phase) {
#pragma unroll
        for (int r = 0; r < Lo::e; ++r) butterfly<E>(x, r);
        exchange_AB<L>(x, xb, tid & (kWave - 1));
#pragma unroll
        for (int r = 1; r < Lo::e; ++r)
            if (L - Lo::e + r >= Lo::e) butterfly<E>(x, r);
    } else {
#pragma unroll
        for (int r = 0; r < L; ++r) butterfly<E>(x, r);
    }
    __syncthreads();
    double r2 = 0.0;
    for (int v = 0; v < nwaves; ++v) r2 += red[v];
    return r2;
}

template <int L, int MAXT, bool BF>
__global__ __launch_bounds__(MAXT) void k_calibrate(CalibArgs a) {
    using Lo = Layout<L>;
    constexpr int E = Lo::E, NP = E / 2;
    extern __shared__ __align__(16) char smem[];
    double* red = reinterpret_cast<double*>(smem);
    double* xb = red + kMaxWaves + (threadIdx.x / kWave) * Lo::xbuf;
    const int tid = threadIdx.x, nwaves = blockDim.x / kWave;
    const int units = a.d_in / E;
    const bool active = tid < units;
    const bool vec = (((uintptr_t)a.w & 15) == 0) && (((a.ld * (BF ? 2 : 4)) & 15) == 0);
    double cf[E];
#pragma unroll
    for (int m = 0; m < E; ++m) {
        int j = min(tid * E + m, a.d_in - 1);
        cf[m] = (a.scale ? (double)a.scale[j] : 1.0) * eps_of(a.sign, j);
    }
    const double inv_sqrt_b = 1.0 / __builtin_sqrt((double)Lo::b);
    double acc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = 0.0;
    int nz = 0;
    int32_t flags = 0;
    RawW<E, BF> nxt;
    int row = blockIdx.x;
    if (active && row < a.n_rows) load_raw<E, BF>(a.w, vec, (int64_t)row * a.ld + (int64_t)tid * E, nxt);
    for (; row < a.n_rows; row += gridDim.x) {
        const RawW<E, BF> cur = nxt;
        if (active && row + (int)gridDim.x < a.n_rows)
            load_raw<E, BF>(a.w, vec, (int64_t)(row + gridDim.x) * a.ld + (int64_t)tid * E, nxt);
        double x[E];
        double r2 = front_end<L, BF>(cur, active, tid, cf, x, red, xb, nwaves, flags);
        double r = __builtin_sqrt(r2);
        if (r > 0.0 && __builtin_isfinite(r)) {
            ++nz;
            double hr = inv_sqrt_b / r;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                double y0 = x[2 * i] * hr, y1 = x[2 * i + 1] * hr;
                acc[i] += __builtin_sqrt(y0 * y0 + y1 * y1);
            }
        }
        __syncthreads();   // red[] is rewritten by the next row
    }
    if (active) {
        double* part = a.partial + (size_t)blockIdx.x * (a.d_in / 2);
#pragma unroll
        for (int i = 0; i < NP; ++i) part[col_B<L>(tid, 2 * i) / 2] = acc[i];
    }
    if (tid == 0) a.nz[blockIdx.x] = nz;
}

// sigma_k from the per-group sums: each pair's groups are split over 4 threads, every thread adds
// its groups in increasing order, and the 4 partial sums are added in a fixed order.
__global__ __launch_bounds__(256) void k_calibrate_finish(const double* __restrict__ partial,
                                                          const int32_t* __restrict__ nzs, int n_groups, int n_pairs,
                                                          int d_in, float* __restrict__ sigma) {
    __shared__ double part[4][64];
    const int kl = threadIdx.x & 63, quarter = threadIdx.x >> 6;
    const int k = blockIdx.x * 64 + kl;
    double s = 0.0;
    if (k < n_pairs) {
        const int per = (n_groups + 3) / 4;
        const int g0 = quarter * per, g1 = min(n_groups, g0 + per);
        int g = g0;
        for (; g + 8 <= g1; g += 8) {
            double v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = partial[(size_t)(g + t) * n_pairs + k];
#pragma unroll
            for (int t = 0; t < 8; ++t) s += v[t];
        }
        for (; g < g1; ++g) s += partial[(size_t)g * n_pairs + k];
    }
    part[quarter][kl] = s;
    __syncthreads();
    if (quarter != 0 || k >= n_pairs) return;
    int64_t n = 0;
    for (int g = 0; g < n_groups; ++g) n += nzs[g];
    double tot = ((part[0][kl] + part[1][kl]) + part[2][kl]) + part[3][kl];
    double m = (n > 0) ? tot / (double)n : 0.0;
    const double rayleigh_mean = __builtin_sqrt(3.14159265358979323846 / 2.0);   // E|z| = sigma sqrt(pi/2)
    sigma[k] = (m > 0.0) ? (float)(m / rayleigh_mean) : (float)(1.0 / __builtin_sqrt((double)d_in));
}

template <int L, int MAXT, bool BF>
__global__ __launch_bounds__(MAXT) void k_encode(EncodeArgs a) {
    using Lo = Layout<L>;
    constexpr int E = Lo::E, NP = E / 2;
    extern __shared__ __align__(16) char smem[];
    const int K = 1 << a.bits;
    const int tid = threadIdx.x, nwaves = blockDim.x / kWave;
    const char* index = reinterpret_cast<const char*>(a.index);
    const IndexHeader ih = *reinterpret_cast<const IndexHeader*>(index);
    const SearchLds sl = search_lds_carve(smem, K, ih);
    double* red = reinterpret_cast<double*>(smem + search_lds_bytes(K, ih.G));
    double* xb_all = red + kMaxWaves;
    double* xb = xb_all + (tid / kWave) * Lo::xbuf;
    uint16_t* idxrow = reinterpret_cast<uint16_t*>(xb_all + (Lo::two_phase ? nwaves * Lo::xbuf : 0));
    search_lds_fill(sl, a.cb, K, index, tid, blockDim.x);

    const int units = a.d_in / E, n_pairs = a.d_in / 2;
    const bool active = tid < units;
    const bool vec = (((uintptr_t)a.w & 15) == 0) && (((a.ld * (BF ? 2 : 4)) & 15) == 0);
    int32_t flags = 0;
    double cf[E];
#pragma unroll
    for (int m = 0; m < E; ++m) {
        int j = min(tid * E + m, a.d_in - 1);
        float s = a.scale ? a.scale[j] : 1.0f;
        if (active && !(s > 0.0f)) flags |= 2;
        cf[m] = (double)s * eps_of(a.sign, j);
        pin_reg(cf[m]);
    }
    double isg[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        isg[i] = 1.0 / (double)a.sigma[min(col_B<L>(tid, 2 * i) / 2, n_pairs - 1)];
        pin_reg(isg[i]);
    }
    if (blockIdx.x != 0) flags &= ~2;   // report a bad scale once
    const double inv_sqrt_b = 1.0 / __builtin_sqrt((double)Lo::b);
    const int bits = a.bits;
    const int nwords = (int)(a.stride / 4);

    RawW<E, BF> nxt;
    int row = blockIdx.x;
    if (active && row < a.d_out) load_raw<E, BF>(a.w, vec, (int64_t)row * a.ld + (int64_t)tid * E, nxt);
    __syncthreads();

    for (; row < a.d_out; row += gridDim.x) {
        const RawW<E, BF> cur = nxt;
        if (active && row + (int)gridDim.x < a.d_out)   // prefetch the next row while this one is encoded
            load_raw<E, BF>(a.w, vec, (int64_t)(row + gridDim.x) * a.ld + (int64_t)tid * E, nxt);
        double x[E];
        int32_t rf = 0;
        double r2 = front_end<L, BF>(cur, active, tid, cf, x, red, xb, nwaves, rf);
        double r = __builtin_sqrt(r2);
        bool nonzero = r > 0.0 && __builtin_isfinite(r);
        if (!__builtin_isfinite(r)) rf |= 1;
        if (active) {
            if (nonzero) {
                const double hr = inv_sqrt_b / r;
                float px[NP], py[NP];
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    double g = isg[i] * hr;
                    px[i] = (float)(x[2 * i] * g);
                    py[i] = (float)(x[2 * i + 1] * g);
                }
                int idx[NP];
                nearest_lds_batch<NP>(px, py, sl, index, idx);
#pragma unroll
                for (int i = 0; i < NP; ++i) idxrow[col_B<L>(tid, 2 * i) / 2] = (uint16_t)idx[i];
            } else {
#pragma unroll
                for (int i = 0; i < NP; ++i) idxrow[col_B<L>(tid, 2 * i) / 2] = 0;
            }
        }
        if (tid == 0) {
            uint16_t nh = 0;
            if (nonzero) {
                __half hv = __float2half_rn((float)r);
                nh = __half_as_ushort(hv);
                if ((nh & 0x7FFF) == 0x7C00) rf |= 4;
            }
            a.norm[row] = nh;
        }
        flags |= rf;
        __syncthreads();
        uint32_t* crow = reinterpret_cast<uint32_t*>(a.codes + (size_t)row * a.stride);
        for (int wd = tid; wd < nwords; wd += blockDim.x) {
            const int bit0 = wd * 32;
            const int k0 = bit0 / bits;
            const int k1 = min((bit0 + 31) / bits, n_pairs - 1);
            uint32_t v = 0;
            for (int k = k0; k <= k1; ++k) {
                uint32_t val = idxrow[k];
                int pos = k * bits - bit0;
                v |= (pos >= 0) ? (val << pos) : (val >> (-pos));
            }
            crow[wd] = v;
        }
    }
    flag_status(a.status, flags);
}

template <int L>
size_t encode_smem(int K, int nwaves, int d_in) {
    using Lo = Layout<L>;
    int bits = 0;
    while ((1 << bits) < K) ++bits;
    return search_lds_bytes(K, index_grid_size(bits)) + kMaxWaves * sizeof(double) +
           (Lo::two_phase ? (size_t)nwaves * Lo::xbuf * sizeof(double) : 0) + (size_t)(d_in / 2) * sizeof(uint16_t);
}

template <int L>
size_t calib_smem(int nwaves) {
    using Lo = Layout<L>;
    return kMaxWaves * sizeof(double) + (Lo::two_phase ? (size_t)nwaves * Lo::xbuf * sizeof(double) : 0);
}

template <int L, bool BF>
hipError_t encode_LB(const EncodeArgs& a, hipStream_t st) {
    using Lo = Layout<L>;
    int threads = ((a.d_in / Lo::E) + kWave - 1) / kWave * kWave;
    int nwaves = threads / kWave;
    size_t smem = encode_smem<L>(1 << a.bits, nwaves, a.d_in);
    int blocks_per_cu = (int)((160 * 1024) / smem);
    if (blocks_per_cu < 1) return hipErrorInvalidConfiguration;
    if (blocks_per_cu * nwaves > 32) blocks_per_cu = 32 / nwaves;
    if (blocks_per_cu < 1) blocks_per_cu = 1;
    int grid = 256 * blocks_per_cu;
    if (grid > a.d_out) grid = a.d_out;
    if (grid < 1) return hipSuccess;
    if (threads <= 512) {
        allow_lds(k_encode<L, 512, BF>, smem);
        hipLaunchKernelGGL((k_encode<L, 512, BF>), dim3(grid), dim3(threads), smem, st, a);
    } else if constexpr (L <= 7) {
        allow_lds(k_encode<L, 1024, BF>, smem);
        hipLaunchKernelGGL((k_encode<L, 1024, BF>), dim3(grid), dim3(threads), smem, st, a);
    } else {
        return hipErrorInvalidConfiguration;
    }
    return hipGetLastError();
}

template <int L, bool BF>
hipError_t calibrate_LB(const CalibArgs& a, float* sigma, hipStream_t st) {
    using Lo = Layout<L>;
    int threads = ((a.d_in / Lo::E) + kWave - 1) / kWave * kWave;
    int nwaves = threads / kWave;
    if (a.n_groups > 0) {
        if (threads <= 512) {
            allow_lds(k_calibrate<L, 512, BF>, calib_smem<L>(nwaves));
            hipLaunchKernelGGL((k_calibrate<L, 512, BF>), dim3(a.n_groups), dim3(threads), calib_smem<L>(nwaves), st,
                               a);
        } else if constexpr (L <= 7) {
            allow_lds(k_calibrate<L, 1024, BF>, calib_smem<L>(nwaves));
            hipLaunchKernelGGL((k_calibrate<L, 1024, BF>), dim3(a.n_groups), dim3(threads), calib_smem<L>(nwaves), st,
                               a);
        } else {
            return hipErrorInvalidConfiguration;
        }
    }
    int n_pairs = a.d_in / 2;
    hipLaunchKernelGGL(k_calibrate_finish, dim3((n_pairs + 63) / 64), dim3(256), 0, st, a.partial, a.nz,
                       a.n_groups, n_pairs, a.d_in, sigma);
    return hipGetLastError();
}

template <int L>
hipError_t encode_L(const EncodeArgs& a, hipStream_t st) {
    return a.w_bf16 ? encode_LB<L, true>(a, st) : encode_LB<L, false>(a, st);
}

template <int L>
hipError_t calibrate_L(const CalibArgs& a, float* sigma, hipStream_t st) {
    return a.w_bf16 ? calibrate_LB<L, true>(a, sigma, st) : calibrate_LB<L, false>(a, sigma, st);
}

}  // namespace

int lane_elems(int L) {
    switch (L) {
    case 1: return Layout<1>::E;
    case 2: return Layout<2>::E;
    case 3: return Layout<3>::E;
    case 4: return Layout<4>::E;
    case 5: return Layout<5>::E;
    case 6: return Layout<6>::E;
    case 7: return Layout<7>::E;
    case 8: return Layout<8>::E;
    case 9: return Layout<9>::E;
    case 10: return Layout<10>::E;
    default: return 0;
    }
}

size_t encode_lds_bytes(int L, int bits, int d_in) {
    const int E = lane_elems(L);
    if (E <= 0) return 0;
    const int nwaves = ((d_in / E) + kWave - 1) / kWave;
    const size_t xb = (L > 4) ? (size_t)nwaves * (kWave * (E / 2) + kWave) * sizeof(double) : 0;
    return search_lds_bytes(1 << bits, index_grid_size(bits)) + kMaxWaves * sizeof(double) + xb +
           (size_t)(d_in / 2) * sizeof(uint16_t);
}

int calib_groups(int n_rows) { return n_rows < kCalibMaxGroups ? n_rows : kCalibMaxGroups; }

size_t calib_workspace(int d_out, int d_in) {
    int n_cal = d_out < 1024 ? d_out : 1024;
    int g = calib_groups(n_cal);
    size_t part = (size_t)(g > 0 ? g : 1) * (size_t)(d_in / 2) * sizeof(double);
    return part + 256 + (size_t)kCalibMaxGroups * sizeof(int32_t);
}

#define QAMW_DISPATCH_L(L, CALL) \
    switch (L) {                 \
    case 1: CALL(1);             \
    case 2: CALL(2);             \
    case 3: CALL(3);             \
    case 4: CALL(4);             \
    case 5: CALL(5);             \
    case 6: CALL(6);             \
    case 7: CALL(7);             \
    case 8: CALL(8);             \
    case 9: CALL(9);             \
    case 10: CALL(10);           \
    default: return hipErrorInvalidValue; \
    }

hipError_t launch_encode(const EncodeArgs& a, int L, hipStream_t st) {
#define QAMW_ENC(l) return encode_L<l>(a, st)
    QAMW_DISPATCH_L(L, QAMW_ENC)
#undef QAMW_ENC
}

hipError_t launch_calibrate(const CalibArgs& a, int L, float* sigma, hipStream_t st) {
#define QAMW_CAL(l) return calibrate_L<l>(a, sigma, st)
    QAMW_DISPATCH_L(L, QAMW_CAL)
#undef QAMW_CAL
}

}  // namespace qamw
