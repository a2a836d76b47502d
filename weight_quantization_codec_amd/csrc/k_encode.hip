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
constexpr size_t kGroupCountBytes = 64;   // the encoder's per-row-group counters (R <= 16)
constexpr int kCalibMaxGroups = 256;

// Sum over the wavefront in a fixed order, the same value returned to every lane.  DPP moves
// (32-bit halves of the double) within rows of 16 lanes, then the row broadcasts into lane 63:
// no LDS traffic and a short dependent chain.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_term(double x) {
    // lanes of rows outside ROW_MASK get 0 (the `old` operand)
    const int lo = __builtin_amdgcn_update_dpp(0, (int)__double2loint(x), CTRL, ROW_MASK, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)__double2hiint(x), CTRL, ROW_MASK, 0xF, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_sum(double v) {
    v += dpp_term<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]: pairs
    v += dpp_term<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]: quads
    v += dpp_term<0x141, 0xF>(v);   // row_half_mirror: 8 lanes
    v += dpp_term<0x140, 0xF>(v);   // row_mirror: rows of 16
    v += dpp_term<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_term<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3: lane 63 holds the total
    const int lo = __builtin_amdgcn_readlane((int)__double2loint(v), kWave - 1);
    const int hi = __builtin_amdgcn_readlane((int)__double2hiint(v), kWave - 1);
    return __hiloint2double(hi, lo);
}

// Square root of q >= 0 for normal or zero q: the hardware reciprocal square root refined by one
// Newton step (error about one fp64 ulp, against about 2^-29 for the bare estimate), times q.
__device__ __forceinline__ double sqrt_pos(double q) {
    const double r = __builtin_amdgcn_rsq(q);
    const double h = 0.5 * q * r;                          // q r / 2
    const double rr = __builtin_fma(r, __builtin_fma(-h, r, 0.5), r);   // r (1.5 - q r^2 / 2)
    return q > 0.0 ? q * rr : 0.0;
}

// The sign mask of columns 0 .. d_in - 1 as bits in LDS, one 64-bit word per 64 columns, drawn
// once per workgroup: thread t takes columns t, t + blockDim.x, ..., so a wavefront's 64
// consecutive columns come out of one ballot (a lane of the encoder would otherwise draw all E of
// its columns, and every row group the same ones).  The caller synchronizes the workgroup before
// the words are read.
__device__ __forceinline__ void sign_words(uint64_t seed, int d_in, uint64_t* words) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int c0 = (int)threadIdx.x - lane; c0 < d_in; c0 += (int)blockDim.x) {
        const int j = c0 + lane;
        const uint64_t m = __builtin_amdgcn_ballot_w64(j < d_in && eps_negative(seed, (uint32_t)j));
        if (lane == 0) words[c0 / kWave] = m;
    }
}

// s_j * eps_j of the E consecutive columns tid*E .. tid*E + E - 1 of a lane (phase A), exact in
// fp32: the scales with 16-byte buffer loads, the signs from the words of sign_words (E divides
// 64, so a lane's columns sit in one word).  Columns at or past d_in get a scale of 1 and no sign.
// bad is set when a scale of the lane is not > 0 (NaN included).
template <int E>
__device__ __forceinline__ void load_cf(const float* scale, const uint64_t* words, int tid, int d_in, float (&cf)[E],
                                        bool& bad) {
    static_assert(kWave % E == 0, "a lane's columns sit in one sign word");
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int j0 = tid * E;
    if (scale) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)scale, (short)0, d_in * 4, 0x00020000);
#pragma unroll
        for (int v = 0; v < E / 4; ++v) {
            const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(j0 + 4 * v) * 4u, 0, 0);
#pragma unroll
            for (int k = 0; k < 4; ++k) cf[4 * v + k] = __uint_as_float(q[k]);
        }
    } else {
#pragma unroll
        for (int m = 0; m < E; ++m) cf[m] = 1.0f;
    }
#pragma unroll
    for (int m = 0; m < E; ++m) {
        if (j0 + m >= d_in) cf[m] = 1.0f;
        bad |= !(cf[m] > 0.0f);
    }
    const uint64_t sw = j0 < d_in ? words[j0 / kWave] >> (j0 % kWave) : 0;
#pragma unroll
    for (int m = 0; m < E; ++m)
        if ((sw >> m) & 1) cf[m] = -cf[m];
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

// a_j = w_j * s_j * eps_j in double (exact), accumulating sum a_j^2.  A non-finite a_j makes the
// row's sum of squares non-finite (|a_j| < 2^256, so a_j^2 cannot overflow), so the row norm
// alone tells whether the row has a non-finite weight.
template <int E, bool BF>
__device__ __forceinline__ void scale_raw(const RawW<E, BF>& r, const double (&cf)[E], double (&x)[E], double& ss) {
#pragma unroll
    for (int m = 0; m < E; ++m) {
        float f;
        if constexpr (BF)
            f = __uint_as_float((m & 1) ? (r.u[m >> 1] & 0xFFFF0000u) : (r.u[m >> 1] << 16));
        else
            f = __uint_as_float(r.u[m]);
        double a = (double)f * cf[m];   // exact: two 24-bit significands
        x[m] = a;
        ss = __builtin_fma(a, a, ss);   // the order of the row's sum is the kernel's own anyway
    }
}

// Front end for one row given its raw weights: x <- unnormalized transform (phase B layout);
// returns sum a^2 over the whole row (fixed shuffle tree, then wavefronts in order).  With SPLIT
// the LDS transpose runs for lanes 0-31 and then for lanes 32-63 (a block's lanes never straddle
// the two), so the wavefront's exchange buffer covers 32 lanes: half the LDS.
// With a group counter (gcnt) the wavefronts of the row wait only for each other: each publishes
// its partial sum and adds 1 to the group's LDS counter, which reaches nwaves * (pass + 1) once the
// whole row's partials of this pass are in; otherwise the workgroup synchronizes.
template <int L, bool BF, bool SPLIT = false, bool B2 = false>
__device__ __forceinline__ double front_end(const RawW<Layout<L>::E, BF>& raw, bool active, int tid,
                                            const double (&cf)[Layout<L>::E], double (&x)[Layout<L>::E],
                                            double* red, double* xb, int nwaves, int* gcnt = nullptr,
                                            int target = 0) {
    using Lo = Layout<L>;
    constexpr int E = Lo::E;
    double ss = 0.0;
    if (active) {
        scale_raw<E, BF>(raw, cf, x, ss);
    } else {
#pragma unroll
        for (int m = 0; m < E; ++m) x[m] = 0.0;
    }
    ss = wave_sum(ss);
    if ((tid & (kWave - 1)) == 0) {
        red[tid / kWave] = ss;
        if (gcnt) __hip_atomic_fetch_add(gcnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if constexpr (B2) {
        // the outer stage of a 256-column block on the 128-column layout: in phase A lane q of the
        // block holds elements 16 q + m, so element bit 7 is lane bit 3 (row_ror:8 within rows of 16
        // lanes is lane ^ 8); the stages commute, so this one runs first.  The lower half-block adds
        // its partner's element, the upper one subtracts its own from the partner's.
        static_assert(L == 7, "256-column blocks run on the 128-column layout");
        const double sgn = ((tid >> 3) & 1) ? -1.0 : 1.0;
#pragma unroll
        for (int m = 0; m < Layout<L>::E; ++m) {
            const int lo = __builtin_amdgcn_update_dpp(0, (int)__double2loint(x[m]), 0x128, 0xF, 0xF, false);
            const int hi = __builtin_amdgcn_update_dpp(0, (int)__double2hiint(x[m]), 0x128, 0xF, 0xF, false);
            x[m] = __builtin_fma(x[m], sgn, __hiloint2double(hi, lo));
        }
    }
    if constexpr (Lo::two_phase) {
        // The stages commute: stage 0 (element bit 0) runs last, in phase B, so the two halves
        // (bit 0 = 0 or 1) stay apart until then and each half is exchanged while the other one
        // is transformed.
        if constexpr (SPLIT) {
            // Two rounds per half through a buffer of 32 lanes' size: round r carries the elements
            // of the lanes whose top q bit is r, and every lane reads in both rounds.  The round-1
            // writers send the values they held before round 0 (`pre`).
            const ExchangeHalf<L> ex(xb, tid & (kWave - 1));
            double pre[E];
#pragma unroll
            for (int r = 1; r < Lo::e; ++r) butterfly_half<E>(x, r, 0);
            if (!ex.top) ex.write(x, 0);
#pragma unroll
            for (int r = 1; r < Lo::e; ++r) butterfly_half<E>(x, r, 1);
#pragma unroll
            for (int m = 0; m < E; ++m) pre[m] = x[m];
            wave_lds_sync();
            ex.read(x, 0, 0);
            wave_lds_sync();
            if (ex.top) ex.write(pre, 0);
            wave_lds_sync();
            ex.read(x, 0, 1);
#pragma unroll
            for (int m = 0; m < E; ++m) pre[m] = x[m];
            wave_lds_sync();
            if (!ex.top) ex.write(pre, 1);
#pragma unroll
            for (int r = 1; r < Lo::e; ++r)
                if (L - Lo::e + r >= Lo::e) butterfly_half<E>(x, r, 0);
            wave_lds_sync();
            ex.read(x, 1, 0);
            wave_lds_sync();
            if (ex.top) ex.write(pre, 1);
            wave_lds_sync();
            ex.read(x, 1, 1);
            wave_lds_sync();
        } else {
            const Exchange<L> ex(xb, tid & (kWave - 1));
#pragma unroll
            for (int r = 1; r < Lo::e; ++r) butterfly_half<E>(x, r, 0);
            ex.write(x, 0);
#pragma unroll
            for (int r = 1; r < Lo::e; ++r) butterfly_half<E>(x, r, 1);
            wave_lds_sync();
            ex.read(x, 0);
            wave_lds_sync();   // half 0 read before half 1 overwrites the buffer
            ex.write(x, 1);
#pragma unroll
            for (int r = 1; r < Lo::e; ++r)
                if (L - Lo::e + r >= Lo::e) butterfly_half<E>(x, r, 0);
            wave_lds_sync();
            ex.read(x, 1);
            wave_lds_sync();
        }
#pragma unroll
        for (int r = 1; r < Lo::e; ++r)
            if (L - Lo::e + r >= Lo::e) butterfly_half<E>(x, r, 1);
        butterfly<E>(x, 0);
    } else {
#pragma unroll
        for (int r = 0; r < L; ++r) butterfly<E>(x, r);
    }
    if (gcnt) {
        while (__hip_atomic_load(gcnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
            __builtin_amdgcn_s_sleep(1);
    } else {
        __syncthreads();
    }
    double r2 = 0.0;
    for (int v = 0; v < nwaves; ++v) r2 += red[v];
    return r2;
}

// Pair calibration, first pass.  A workgroup runs R rows at a time (R groups of T lanes, T =
// lanes per row); group g takes rows base + g for base = R * blockIdx.x, R * (blockIdx.x +
// gridDim.x), ...  Every group runs every pass (rows past the end are zero), so the barriers in
// the front end are reached by the whole workgroup.  At the end the groups' |z_k| sums are added
// in group order and written as the workgroup's partial sums.
// The calibration's lane layout: 256-column blocks of bf16 rows on the 128-column one, as in the
// encoder (one DPP stage for the outer butterfly; see enc_b2 below).
template <int L, bool BF>
__host__ __device__ constexpr int cal_layout() { return (L == 8 && BF) ? 7 : L; }

template <int L, int MAXT, bool BF>
__global__ __launch_bounds__(MAXT) void k_calibrate(CalibArgs a, int T, int R) {
    constexpr int LL = cal_layout<L, BF>();
    using Lo = Layout<LL>;
    constexpr int E = Lo::E, NP = E / 2;
    extern __shared__ __align__(16) char smem[];
    const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / T);
    const int tid = threadIdx.x - grp * T, nwaves = T / kWave;
    double* red = reinterpret_cast<double*>(smem) + grp * kMaxWaves;
    double* xb_all = reinterpret_cast<double*>(smem) + R * kMaxWaves;
    double* xb = xb_all + (threadIdx.x / kWave) * Lo::xbuf;
    const int units = a.d_in / E;
    const bool active = tid < units;
    const bool vec = (((uintptr_t)a.w & 15) == 0) && (((a.ld * (BF ? 2 : 4)) & 15) == 0);
    RawW<E, BF> nxt;
    const int rstride = gridDim.x * R;
    int base = blockIdx.x * R;
    if (active && base + grp < a.n_rows) load_raw<E, BF>(a.w, vec, (int64_t)(base + grp) * a.ld + (int64_t)tid * E, nxt);
    double cf[E];   // s_j * eps_j (exact in fp32; scales are checked by the encoder)
    {
        // the sign words in the exchange buffers, free until the first front end
        uint64_t* words = reinterpret_cast<uint64_t*>(xb_all);
        sign_words(a.sign_seed, a.d_in, words);
        __syncthreads();
        float cf32[E];
        bool bad_scale = false;
        load_cf<E>(a.scale, words, tid, a.d_in, cf32, bad_scale);
#pragma unroll
        for (int m = 0; m < E; ++m) cf[m] = (double)cf32[m];
        __syncthreads();
    }
    const double inv_sqrt_b = 1.0 / __builtin_sqrt((double)(1 << L));
    double acc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = 0.0;
    int nz = 0;
    for (; base < a.n_rows; base += rstride) {
        const int row = base + grp;
        const bool rv = row < a.n_rows;
        double x[E];
        double r2 = front_end<LL, BF, false, (LL != L)>(nxt, active && rv, tid, cf, x, red, xb, nwaves);
        if (active && row + rstride < a.n_rows)
            load_raw<E, BF>(a.w, vec, (int64_t)(row + rstride) * a.ld + (int64_t)tid * E, nxt);
        double r = __builtin_sqrt(r2);
        if (rv && r > 0.0 && __builtin_isfinite(r)) {
            ++nz;
            double hr = inv_sqrt_b / r;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                double y0 = x[2 * i] * hr, y1 = x[2 * i + 1] * hr;
                acc[i] += sqrt_pos(y0 * y0 + y1 * y1);
            }
        }
        __syncthreads();   // red[] and the exchange buffers are rewritten by the next pass
    }
    // groups' sums in group order, through LDS (the exchange buffers are free now)
    double* comb = xb_all;
    for (int g = 0; g < R; ++g) {
        if (grp == g && active) {
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int k = col_B<LL>(tid, 2 * i) / 2;
                comb[k] = (g == 0) ? acc[i] : comb[k] + acc[i];
            }
        }
        __syncthreads();
    }
    // rows with a non-zero norm: one count per group (lane 0 of its first wave), added in order
    __shared__ int nz_grp[8];
    if (tid == 0) nz_grp[grp] = nz;
    __syncthreads();
    if (grp == 0 && active) {
        double* part = a.partial + (size_t)blockIdx.x * (a.d_in / 2);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int k = col_B<LL>(tid, 2 * i) / 2;
            part[k] = comb[k];
        }
    }
    if (threadIdx.x == 0) {
        int n = 0;
        for (int g = 0; g < R; ++g) n += nz_grp[g];
        a.nz[blockIdx.x] = n;
    }
}

// sigma_k from the per-group sums.  A block of 1024 threads owns kFinishPairs pairs; each pair's
// groups are split into kFinishParts contiguous runs, one per thread, every thread adds its run in
// increasing group order, and the run sums are added in run order, so the result does not depend
// on scheduling.  The count of non-zero rows is reduced by the whole block.
constexpr int kFinishParts = 32;
constexpr int kFinishPairs = 1024 / kFinishParts;
__global__ __launch_bounds__(1024) void k_calibrate_finish(const double* __restrict__ partial,
                                                           const int32_t* __restrict__ nzs, int n_groups, int n_pairs,
                                                           int d_in, float* __restrict__ sigma) {
    __shared__ double part[kFinishParts][kFinishPairs];
    __shared__ int64_t nzw[1024 / kWave];
    const int kl = threadIdx.x % kFinishPairs, q = threadIdx.x / kFinishPairs;
    const int k = blockIdx.x * kFinishPairs + kl;
    // rows counted by the groups (each thread at most one group per pass)
    int64_t nn = 0;
    for (int g = threadIdx.x; g < n_groups; g += blockDim.x) nn += nzs[g];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nn += __shfl_xor(nn, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) nzw[threadIdx.x / kWave] = nn;
    double s = 0.0;
    if (k < n_pairs) {
        const int per = (n_groups + kFinishParts - 1) / kFinishParts;
        const int g0 = q * per, g1 = min(n_groups, g0 + per);
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
    part[q][kl] = s;
    __syncthreads();
    if (q != 0 || k >= n_pairs) return;
    int64_t n = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) n += nzw[w];
    double tot = part[0][kl];
#pragma unroll
    for (int r = 1; r < kFinishParts; ++r) tot += part[r][kl];
    double m = (n > 0) ? tot / (double)n : 0.0;
    const double rayleigh_mean = __builtin_sqrt(3.14159265358979323846 / 2.0);   // E|z| = sigma sqrt(pi/2)
    sigma[k] = (m > 0.0) ? (float)(m / rayleigh_mean) : (float)(1.0 / __builtin_sqrt((double)d_in));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw weights of one row for a lane through a buffer descriptor: a row past the end has a
// descriptor covering no bytes and reads zeros, so the prefetch never branches.  Requires the
// 16-byte vector path (row starts 16-byte aligned).
template <int E, bool BF>
__device__ __forceinline__ void load_raw_buf(const void* w, int64_t ld, int d_in, int d_out, int row, int tid,
                                             RawW<E, BF>& r) {
    constexpr int ESZ = BF ? 2 : 4;
    const bool ok = row < d_out;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(w) + (size_t)(ok ? row : 0) * (size_t)ld * ESZ), (short)0,
        ok ? d_in * ESZ : 0, 0x00020000);
    const uint32_t off = (uint32_t)tid * (uint32_t)(E * ESZ);
#pragma unroll
    for (int v = 0; v < RawW<E, BF>::N / 4; ++v) {
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u * v, 0, 0);
        r.u[4 * v] = q[0];
        r.u[4 * v + 1] = q[1];
        r.u[4 * v + 2] = q[2];
        r.u[4 * v + 3] = q[3];
    }
}

// The same through 2- or 4-byte loads, for rows that are not 16-byte aligned.
template <int E, bool BF>
__device__ __forceinline__ void load_raw_buf_unaligned(const void* w, int64_t ld, int d_in, int d_out, int row,
                                                       int tid, RawW<E, BF>& r) {
    constexpr int ESZ = BF ? 2 : 4;
    const bool ok = row < d_out;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(w) + (size_t)(ok ? row : 0) * (size_t)ld * ESZ), (short)0,
        ok ? d_in * ESZ : 0, 0x00020000);
    const uint32_t off = (uint32_t)tid * (uint32_t)(E * ESZ);
    if constexpr (BF) {
#pragma unroll
        for (int m = 0; m < E / 2; ++m) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 4u * m, 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 4u * m + 2u, 0, 0);
            r.u[m] = lo | (hi << 16);
        }
    } else {
#pragma unroll
        for (int m = 0; m < E; ++m) r.u[m] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4u * m, 0, 0);
    }
}

template <int E, bool BF, bool VEC>
__device__ __forceinline__ void load_row_raw(const void* w, int64_t ld, int d_in, int d_out, int row, int tid,
                                             RawW<E, BF>& r) {
    if constexpr (VEC)
        load_raw_buf<E, BF>(w, ld, d_in, d_out, row, tid, r);
    else
        load_raw_buf_unaligned<E, BF>(w, ld, d_in, d_out, row, tid, r);
}

// Encoder.  A workgroup runs R rows at a time (R groups of T lanes, T = lanes per row) over one
// LDS image of the codebook and its search index; group g takes rows base + g for base = R *
// blockIdx.x, R * (blockIdx.x + gridDim.x), ...  Every group runs every pass (a row past the end
// is all zero and writes nothing), so the workgroup barriers are reached by all threads.
// Per pass: front end (scale, norm, transform), pairs, lockstep search in batches of four pairs
// per lane, indices to LDS, then each wavefront packs and stores its part of the row.
constexpr int kSearchBatch = 4;
constexpr int kSearchCap = 3;   // lockstep steps before a longer list goes to the queue
constexpr int kPolarBatch = 1;   // pairs per polar batch: more spill registers

// LDS bytes per wavefront of the encoder.  A wavefront's lanes cover 32 E consecutive pairs of
// the row, so it packs and stores its own part of the row: its buffer holds the exchange during
// the front end and then the wavefront's 32 E indices (u16) followed by the search queue and then
// by their packed words (4 E bits bytes, a multiple of 16).
__host__ __device__ inline size_t encode_wave_bytes(int E, bool two_phase, int bits) {
    const size_t xch = two_phase ? (size_t)(32 * (E / 2) + 32) * sizeof(double) : 0;   // the split transpose
    const size_t pack = (size_t)64 * E + (size_t)4 * E * bits;
    const size_t queue = (size_t)64 * E + search_queue_bytes();   // the search queue after the indices
    const size_t m = xch > pack ? xch : pack;
    return m > queue ? m : queue;
}

// 256-column blocks of aligned bf16 rows (the QAM-W search) run on the 128-column lane layout:
// H_256 = [[H_128, H_128], [H_128, -H_128]] in Sylvester order, so each half-block is transformed as
// a 128-column block and one more stage combines the halves, which lanes 8 apart hold with the same
// element positions.  That layout has 16 elements per lane instead of 32: half the registers, so
// twice the wavefronts per CU.
template <int L, bool BF, bool VEC, bool POLAR>
__host__ __device__ constexpr bool enc_b2() { return L == 8 && BF && VEC && !POLAR; }
template <int L, bool BF, bool VEC, bool POLAR>
__host__ __device__ constexpr int enc_layout() { return enc_b2<L, BF, VEC, POLAR>() ? 7 : L; }

template <int L, int MAXT, bool BF, bool VEC, bool ISG_LDS, bool POLAR>
__global__ __launch_bounds__(MAXT) void k_encode(EncodeArgs a, int T, int R) {
    constexpr bool kB2 = enc_b2<L, BF, VEC, POLAR>();
    constexpr int LL = enc_layout<L, BF, VEC, POLAR>();   // the lane layout's block
    using Lo = Layout<LL>;
    constexpr int E = Lo::E, NP = E / 2;
    extern __shared__ __align__(16) char smem[];
    const int K = 1 << a.bits;
    const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / T);
    const int tid = threadIdx.x - grp * T, nwaves = T / kWave;
    // the quantizer's tables: the QAM-W search image (section 3.6) or the polar tables (3.5)
    const char* index = reinterpret_cast<const char*>(a.index);
    SearchLds sl{};
    PolarLds pl{};
    size_t front;
    if constexpr (POLAR) {
        pl = polar_lds_carve(smem, a.ba, a.bits - a.ba);
        front = polar_lds_bytes(a.bits - a.ba);
    } else {
        const IndexHeader ih = *reinterpret_cast<const IndexHeader*>(index);
        if (!index_header_ok(ih, K, a.index_g)) {   // uniform over the grid: no workgroup goes on
            if (blockIdx.x == 0 && threadIdx.x == 0) flag_status(a.status, kFlagBadIndex);
            return;
        }
        sl = search_lds_carve(smem, K, ih, index);
        front = search_lds_bytes(K, ih.G);
    }
    // norm partials, double-buffered by pass parity ([2][R][kMaxWaves]): a wavefront may reach
    // the next pass's front end while others still read this pass's partials
    double* red_all = reinterpret_cast<double*>(smem + front);
    const int wave_bytes = (int)encode_wave_bytes(E, Lo::two_phase, a.bits);
    char* wbuf = reinterpret_cast<char*>(red_all + 2 * R * kMaxWaves) + (threadIdx.x / kWave) * wave_bytes;
    double* xb = reinterpret_cast<double*>(wbuf);
    const int n_pairs = a.d_in / 2;
    const int lane = threadIdx.x & (kWave - 1);
    // this wavefront's indices and packed words (after the front end, in its exchange buffer)
    uint16_t* widx = reinterpret_cast<uint16_t*>(wbuf);
    uint32_t* wstage = reinterpret_cast<uint32_t*>(wbuf + 64 * E);
    // this lane's pairs k = col_B(tid, 2i)/2 are base + i * (lanes per block): one base address
    uint16_t* idx_l = widx + (Lo::two_phase ? ((unsigned)lane / Lo::lanes) * (Lo::b / 2) + (unsigned)lane % Lo::lanes
                                            : (unsigned)lane * NP);
    const int units = a.d_in / E;
    const bool active = tid < units;
    const int rstride = gridDim.x * R;
    int base = blockIdx.x * R;

    // Every VMEM access of the row loop is unconditional (out-of-range lanes and rows use offsets
    // or descriptors outside their buffers: loads return 0, stores are dropped), so the wait for
    // the prefetched row can leave the previous row's stores in flight.
    RawW<E, BF> nxt;
    load_row_raw<E, BF, VEC>(a.w, a.ld, a.d_in, a.d_out, base + grp, tid, nxt);
    int32_t flags = 0;
    if constexpr (POLAR) {
        if (polar_lds_fill(pl, a.thr, threadIdx.x, blockDim.x) && blockIdx.x == 0) flags |= 16;
    } else {
        search_lds_fill(sl, index, K, threadIdx.x, blockDim.x);
    }

    double cf[E];   // s_j * eps_j (exact in fp32), held as doubles: converted once, not per row
    {
        // the sign words in the wavefronts' buffers, free until the first front end (after the
        // barrier that ends the set-up)
        uint64_t* words = reinterpret_cast<uint64_t*>(red_all + 2 * R * kMaxWaves);
        sign_words(a.sign_seed, a.d_in, words);
        __syncthreads();
        float cf32[E];
        bool bad_scale = false;
        load_cf<E>(a.scale, words, tid, a.d_in, cf32, bad_scale);
        if (active && bad_scale && blockIdx.x == 0) flags |= 2;   // reported once
#pragma unroll
        for (int m = 0; m < E; ++m) cf[m] = (double)cf32[m];
    }
#pragma unroll
    for (int m = 0; m < E; ++m) pin_reg(cf[m]);
    // 1 / sigma_k of the lane's pairs: in registers, or (ISG_LDS, which frees 16 VGPRs) in LDS,
    // the same for every group (it depends on the lane's columns only), as double2 [NP/2][T] so
    // that a wavefront's reads are consecutive
    double2 isg_reg[NP / 2];
    double2* isg_lds = reinterpret_cast<double2*>(reinterpret_cast<char*>(red_all + 2 * R * kMaxWaves) +
                                                  (size_t)(blockDim.x / kWave) * wave_bytes);
    // per row group, the count of wavefronts that have published their pass's norm partial
    int* gcnt = reinterpret_cast<int*>(reinterpret_cast<char*>(isg_lds) + (ISG_LDS ? (size_t)T * NP * sizeof(double) : 0)) + grp;
    if (tid == 0) *gcnt = 0;
#pragma unroll
    for (int i = 0; i < NP / 2; ++i) {
        const double i0 = 1.0 / (double)a.sigma[min(col_B<LL>(tid, 4 * i) / 2, n_pairs - 1)];
        const double i1 = 1.0 / (double)a.sigma[min(col_B<LL>(tid, 4 * i + 2) / 2, n_pairs - 1)];
        if constexpr (ISG_LDS) {
            if (grp == 0) isg_lds[i * T + tid] = make_double2(i0, i1);
        } else {
            isg_reg[i] = make_double2(i0, i1);
            pin_reg(isg_reg[i].x);
            pin_reg(isg_reg[i].y);
        }
    }
    const double inv_sqrt_b = 1.0 / __builtin_sqrt((double)(1 << L));
    const int bits = a.bits;
    const __amdgpu_buffer_rsrc_t nrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.norm, (short)0, a.d_out * 2, 0x00020000);
    __syncthreads();

    const uint32_t wave_byte0 = (uint32_t)(tid / kWave) * (uint32_t)(4 * E * a.bits);   // the wavefront's part of the row
    for (int pass = 0; base < a.d_out; base += rstride, ++pass) {
        const int row = base + grp;
        const bool rv = row < a.d_out;
        double x[E];
        int32_t rf = 0;
        double* red = red_all + ((pass & 1) * R + grp) * kMaxWaves;
        // lanes past the row (whole blocks of their own) and rows past the matrix loaded zeros,
        // so the front end runs on every lane: nothing of theirs is stored or searched
        const double r2 = front_end<LL, BF, true, kB2>(nxt, true, tid, cf, x, red, xb, nwaves, gcnt, nwaves * (pass + 1));
        // the next row, in flight during the search and the packing (its registers were free
        // during the front end)
        load_row_raw<E, BF, VEC>(a.w, a.ld, a.d_in, a.d_out, row + rstride, tid, nxt);
        const double r = __builtin_sqrt(r2);
        const bool nonzero = r > 0.0 && __builtin_isfinite(r);
        if (rv && !__builtin_isfinite(r)) rf |= 1;
        float px[NP], py[NP];
        if (active) {
            const double hr = inv_sqrt_b / r;
#pragma unroll
            for (int i = 0; i < NP; i += 2) {
                const double2 isg = ISG_LDS ? isg_lds[(i / 2) * T + tid] : isg_reg[i / 2];
                const double g0 = isg.x * hr, g1 = isg.y * hr;
                px[i] = (float)(x[2 * i] * g0);
                py[i] = (float)(x[2 * i + 1] * g0);
                px[i + 1] = (float)(x[2 * i + 2] * g1);
                py[i + 1] = (float)(x[2 * i + 3] * g1);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NP; ++i) px[i] = py[i] = 0.0f;
        }
        // Searches capped at kSearchCap lockstep steps; the longer lists go to the wavefront's queue
        // (after the indices, where the packed words go later) and are finished one per lane.  Pairs
        // past the row (inactive lanes) and zero rows get index 0, so the row's padding bits are 0.
        const SearchQueue sq = search_queue_at(wbuf + 64 * E);
        const uint32_t slot_l = (uint32_t)(idx_l - widx);
        constexpr uint32_t kSlotStep = Lo::two_phase ? Lo::lanes : 1;
        int qn = 0;   // entries in the queue (uniform over the wavefront)
#pragma unroll
        for (int h = 0; h < NP / kSearchBatch; ++h) {
            float bx[kSearchBatch], by[kSearchBatch];
            int bi[kSearchBatch];
            SearchCont st[kSearchBatch];
#pragma unroll
            for (int i = 0; i < kSearchBatch; ++i) {
                bx[i] = px[h * kSearchBatch + i];
                by[i] = py[h * kSearchBatch + i];
                bi[i] = 0;
                st[i] = SearchCont{0.0f, 0u, 0u};
            }
            if (active && nonzero) {
                if constexpr (POLAR) {
#pragma unroll
                    for (int g = 0; g < kSearchBatch; g += kPolarBatch) {
                        float gx[kPolarBatch], gy[kPolarBatch];
                        int gi[kPolarBatch];
#pragma unroll
                        for (int i = 0; i < kPolarBatch; ++i) {
                            gx[i] = bx[g + i];
                            gy[i] = by[g + i];
                        }
                        polar_batch<kPolarBatch>(gx, gy, pl, gi);
#pragma unroll
                        for (int i = 0; i < kPolarBatch; ++i) bi[g + i] = gi[i];
                    }
                } else {
                    // the unrolled walk for aligned bf16 rows, except with E = 16 and 1/sigma in
                    // registers: there, and for fp32 or unaligned rows, its extra registers spill
                    nearest_lds_capped<kSearchBatch, kSearchCap, (BF && VEC && (ISG_LDS || E > 16))>(bx, by, sl, bi, st);
                }
            }
#pragma unroll
            for (int i = 0; i < kSearchBatch; ++i) idx_l[(h * kSearchBatch + i) * kSlotStep] = (uint16_t)bi[i];
            if constexpr (!POLAR) {
#pragma unroll
                for (int i = 0; i < kSearchBatch; ++i) {
                    const bool want = st[i].open();
                    const uint64_t m = __builtin_amdgcn_ballot_w64(want);
                    const int c = __builtin_popcountll(m);
                    if (c == 0) continue;
                    if (qn + c > kSearchQueue) {   // full: finish what it holds first
                        wave_lds_sync();
                        search_finish(sq, qn, sl, widx, lane);
                        wave_lds_sync();
                        qn = 0;
                    }
                    if (want) {
                        const int pos =
                            qn + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                        sq.x[pos] = bx[i];
                        sq.y[pos] = by[i];
                        sq.bd[pos] = st[i].bd;
                        sq.a[pos] = (st[i].bo_next & 0xFFFFu) | ((slot_l + (uint32_t)(h * kSearchBatch + i) * kSlotStep) << 16);
                        sq.b[pos] = (st[i].bo_next >> 16) | (st[i].end << 16);
                    }
                    qn += c;
                }
            }
        }
        if constexpr (!POLAR) {
            if (qn > 0) {
                wave_lds_sync();   // the queue and the provisional indices are written
                search_finish(sq, qn, sl, widx, lane);
            }
        }
        {   // the norm, stored by lane 0 of the group
            uint16_t nh = 0;
            if (nonzero) {
                __half hv = __float2half_rn((float)r);
                nh = __half_as_ushort(hv);
                if (tid == 0 && (nh & 0x7FFF) == 0x7C00) rf |= 4;
            }
            __builtin_amdgcn_raw_buffer_store_b16(nh, nrs, tid == 0 ? (uint32_t)row * 2u : kNoByte, 0, 0);
        }
        if (rv) flags |= rf;
        wave_lds_sync();
        // pack (LSB first): the wavefront's 32 E indices make E * bits words; lane l packs indices
        // NP l .. NP l + NP - 1 (bits NP l bits onwards), eight at a time: the eight indices form a
        // run of 8 bits <= 96 bits (bits <= 12), which, shifted to its offset within its first word,
        // covers at most four words; each non-zero word is OR-ed into LDS (a run's first and last
        // words are shared with its neighbours).  A zero word is skipped, so no word past the
        // wavefront's part is touched.
        for (int wd = lane; wd < E * bits; wd += kWave) wstage[wd] = 0;
        wave_lds_sync();
#pragma unroll 1
        for (int v = 0; v < NP / 8; ++v) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(widx + NP * lane + 8 * v);
            // index i of the eight starts at bit i * bits of the run (a uniform choice between the
            // run's low 64 bits, lo, and its bits from 32 on, hi)
            uint64_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint64_t id = (q[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                const int p = i * bits;
                if (p < 32)
                    lo |= id << p;
                else
                    hi |= id << (p - 32);
            }
            const uint32_t r0 = (uint32_t)lo, r1 = (uint32_t)(lo >> 32) | (uint32_t)hi, r2 = (uint32_t)(hi >> 32);
            const uint32_t o = (uint32_t)((lane * NP + 8 * v) * bits), nb = o & 31u;
            uint32_t* wp = wstage + (o >> 5);
            const uint64_t s01 = (((uint64_t)r1 << 32) | r0) << nb;
            const uint32_t w2 = (uint32_t)(((((uint64_t)r2 << 32) | r1) << nb) >> 32);
            const uint32_t w3 = (uint32_t)(((uint64_t)r2 << nb) >> 32);
            if ((uint32_t)s01) __hip_atomic_fetch_or(wp, (uint32_t)s01, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if ((uint32_t)(s01 >> 32))
                __hip_atomic_fetch_or(wp + 1, (uint32_t)(s01 >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (w2) __hip_atomic_fetch_or(wp + 2, w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (w3) __hip_atomic_fetch_or(wp + 3, w3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        wave_lds_sync();
        // 16-byte stores of the wavefront's 4 E bits bytes: E bits / 4 chunks, lane c storing
        // chunks c, c + 64, ...; chunks past the row stride are dropped by the descriptor
        const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.codes + (size_t)(rv ? row : 0) * a.stride), (short)0, rv ? (int)a.stride : 0, 0x00020000);
        const int nchunks = E * bits / 4;
        constexpr int NCH = (E * 4 + kWave - 1) / kWave;   // bits <= 16
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int c = lane + u * kWave;
            const u32x4 q = *reinterpret_cast<const u32x4*>(wstage + 4 * min(c, nchunks - 1));
            __builtin_amdgcn_raw_buffer_store_b128(q, crs, c < nchunks ? wave_byte0 + (uint32_t)c * 16u : kNoByte, 0, 0);
        }
        wave_lds_sync();   // the staged words are read before the next front end reuses the buffer
    }
    flag_status(a.status, flags);
}

// LDS of the encoder: search image, R * kMaxWaves norm partials, and one region holding either
// the exchange buffers (one per wavefront) or the R groups' indices and packed words.
template <int L>
size_t encode_smem(size_t front, int bits, int R, int nwaves_total, bool isg_lds) {
    using Lo = Layout<L>;
    const size_t isg = isg_lds ? (size_t)(nwaves_total / R) * kWave * (Lo::E / 2) * sizeof(double) : 0;
    return front + (size_t)2 * R * kMaxWaves * sizeof(double) +
           (size_t)nwaves_total * encode_wave_bytes(Lo::E, Lo::two_phase, bits) + isg + kGroupCountBytes;
}

// LDS of the quantizer's tables
inline size_t encode_front_bytes(const EncodeArgs& a) {
    return a.thr ? polar_lds_bytes(a.bits - a.ba) : search_lds_bytes(1 << a.bits, index_grid_size(a.bits));
}

// R * kMaxWaves norm partials, then the exchange buffers (at least d_in/2 doubles: they also
// hold the groups' combined sums at the end).
template <int L>
size_t calib_smem(int R, int nwaves) {
    using Lo = Layout<L>;
    const size_t xb = Lo::two_phase ? (size_t)nwaves * Lo::xbuf * sizeof(double) : 0;
    const size_t comb = (size_t)nwaves * kWave * (Lo::E / 2) * sizeof(double);
    return (size_t)R * kMaxWaves * sizeof(double) + (xb > comb ? xb : comb);
}

// Launch with one workgroup per resident slot: the occupancy the kernel reaches with this LDS and
// its register count (rows are strided over the grid, so a second wave of workgroups would only
// add a tail).
template <int L, int MT, bool BF, bool VEC, bool ISG, bool POLAR>
hipError_t encode_launch(const EncodeArgs& a, int R, int threads, size_t smem, int T, hipStream_t st) {
    auto kern = k_encode<L, MT, BF, VEC, ISG, POLAR>;
    allow_lds(kern, smem);
    // the last answer of the occupancy query, per instantiation and host thread
    static thread_local int c_threads = -1, c_per_cu = 1;
    static thread_local size_t c_smem = 0;
    if (threads != c_threads || smem != c_smem) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, smem) != hipSuccess || per_cu < 1)
            per_cu = 1;
        c_threads = threads;
        c_smem = smem;
        c_per_cu = per_cu;
    }
    const int per_cu = c_per_cu;
    const int need = (a.d_out + R - 1) / R;
    const int grid = 256 * per_cu < need ? 256 * per_cu : need;
    if (grid < 1) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), smem, st, a, T, R);
    return hipGetLastError();
}

template <int L, bool BF, bool VEC, bool POLAR>
hipError_t encode_LBVP(const EncodeArgs& a, hipStream_t st) {
    constexpr int LL = enc_layout<L, BF, VEC, POLAR>();   // the kernel's lane layout
    using Lo = Layout<LL>;
    const int T = ((a.d_in / Lo::E) + kWave - 1) / kWave * kWave;
    if (T > 1024 || (T > 512 && LL > 7)) return hipErrorInvalidConfiguration;
    const size_t front = encode_front_bytes(a);
    if constexpr (LL <= 7) {
        // up to 1024 threads with 1 / sigma in LDS (128 VGPRs, four wavefronts per SIMD)
        int R = 1024 / T;
        if (R > 4) R = 4;
        if (R > a.d_out) R = a.d_out > 0 ? a.d_out : 1;
        while (R > 1 && encode_smem<LL>(front, a.bits, R, R * T / kWave, true) > kLdsBytes) --R;
        const int threads = R * T;
        const size_t smem = encode_smem<LL>(front, a.bits, R, threads / kWave, true);
        if (smem <= kLdsBytes) return encode_launch<L, 1024, BF, VEC, true, POLAR>(a, R, threads, smem, T, st);
    }
    // 1 / sigma in registers
    constexpr int kMax = LL <= 7 ? 768 : 512;
    int R = T >= kMax ? 1 : kMax / T;
    if (R > 4) R = 4;
    if (R > a.d_out) R = a.d_out > 0 ? a.d_out : 1;
    while (R > 1 && encode_smem<LL>(front, a.bits, R, R * T / kWave, false) > kLdsBytes) --R;
    const int threads = R * T;
    const size_t smem = encode_smem<LL>(front, a.bits, R, threads / kWave, false);
    if (smem > kLdsBytes) return hipErrorInvalidConfiguration;
    if (threads <= 512) return encode_launch<L, 512, BF, VEC, false, POLAR>(a, R, threads, smem, T, st);
    if constexpr (LL <= 7) {
        if (threads <= 768) return encode_launch<L, 768, BF, VEC, false, POLAR>(a, R, threads, smem, T, st);
        return encode_launch<L, 1024, BF, VEC, false, POLAR>(a, R, threads, smem, T, st);
    }
    return hipErrorInvalidConfiguration;
}

template <int L, bool BF, bool VEC>
hipError_t encode_LBV(const EncodeArgs& a, hipStream_t st) {
    return a.thr ? encode_LBVP<L, BF, VEC, true>(a, st) : encode_LBVP<L, BF, VEC, false>(a, st);
}

template <int L, bool BF>
hipError_t encode_LB(const EncodeArgs& a, hipStream_t st) {
    const bool vec = (((uintptr_t)a.w & 15) == 0) && (((a.ld * (BF ? 2 : 4)) & 15) == 0);
    return vec ? encode_LBV<L, BF, true>(a, st) : encode_LBV<L, BF, false>(a, st);
}

template <int L, bool BF>
hipError_t calibrate_LB(const CalibArgs& a, float* sigma, hipStream_t st) {
    constexpr int LL = cal_layout<L, BF>();   // the kernel's lane layout
    using Lo = Layout<LL>;
    constexpr int kMax = LL <= 7 ? 1024 : 512;
    const int T = ((a.d_in / Lo::E) + kWave - 1) / kWave * kWave;
    if (T > kMax) return hipErrorInvalidConfiguration;
    int R = kMax / T;
    if (R > 4) R = 4;
    int groups = 0;
    if (a.n_rows > 0) {
        if (R > a.n_rows) R = a.n_rows;
        groups = (a.n_rows + R - 1) / R;
        if (groups > a.n_groups) groups = a.n_groups;   // the workspace holds n_groups partial rows
        const int threads = R * T;
        const size_t smem = calib_smem<LL>(R, threads / kWave);
        if (threads <= 512) {
            allow_lds(k_calibrate<L, 512, BF>, smem);
            hipLaunchKernelGGL((k_calibrate<L, 512, BF>), dim3(groups), dim3(threads), smem, st, a, T, R);
        } else if constexpr (LL <= 7) {
            allow_lds(k_calibrate<L, 1024, BF>, smem);
            hipLaunchKernelGGL((k_calibrate<L, 1024, BF>), dim3(groups), dim3(threads), smem, st, a, T, R);
        } else {
            return hipErrorInvalidConfiguration;
        }
    }
    int n_pairs = a.d_in / 2;
    hipLaunchKernelGGL(k_calibrate_finish, dim3((n_pairs + kFinishPairs - 1) / kFinishPairs), dim3(1024), 0, st, a.partial, a.nz,
                       groups, n_pairs, a.d_in, sigma);
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

size_t encode_lds_bytes(int L, int bits, int d_in, int polar_bp) {
    const int E = lane_elems(L);
    if (E <= 0) return 0;
    const int nwaves = ((d_in / E) + kWave - 1) / kWave;
    const size_t front = polar_bp >= 1 ? polar_lds_bytes(polar_bp) : search_lds_bytes(1 << bits, index_grid_size(bits));
    return front + 2 * kMaxWaves * sizeof(double) + (size_t)nwaves * encode_wave_bytes(E, L > 4, bits) +
           kGroupCountBytes;
}

namespace {
// Bit j % 32 of word j / 32 is set when eps_j = -1 (the mask the kernels draw from the seed).
__global__ __launch_bounds__(256) void k_sign_mask(uint64_t seed, int d_in, uint32_t* __restrict__ out) {
    const int w = blockIdx.x * blockDim.x + threadIdx.x;
    if (w * 32 >= d_in) return;
    uint32_t v = 0;
    for (int t = 0; t < 32 && w * 32 + t < d_in; ++t)
        if (eps_negative(seed, (uint32_t)(w * 32 + t))) v |= 1u << t;
    out[w] = v;
}
}  // namespace

hipError_t launch_sign_mask(uint64_t seed, int d_in, uint32_t* bits, hipStream_t st) {
    const int words = (d_in + 31) / 32;
    hipLaunchKernelGGL(k_sign_mask, dim3((words + 255) / 256), dim3(256), 0, st, seed, d_in, bits);
    return hipGetLastError();
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
