// QAM-W decoder (paper section 3.2), output dequantized to BF16 or fp32 (section 1: the
// weights are dequantized to BF16 before the matrix product).
//
// HBM-bound streaming kernel: per weight it reads B/16 bytes of codes (plus 2/d_in of norm)
// and writes 2 (BF16) or 4 (fp32) bytes.  One workgroup covers a whole row with one lane per
// E consecutive columns and walks rows strided over the grid; per-column constants stay in
// registers across rows:
//   unpack -> B-bit fields from 32-bit buffer loads (funnel shifts)
//   lookup -> LDS table of (c_x + c_y, c_x - c_y) in double = the first butterfly stage,
//             times sigma_k * f16(norm) / sqrt(b)
//   FWHT   -> remaining stages in double (register butterflies, one LDS exchange per wave)
//   scale  -> * eps_j / s_j, round to fp32 (RNE), then to BF16 (RNE, v_cvt_pk_bf16_f32)
// The transform runs in double so that every output, even one near zero, is within one BF16
// ulp of the exactly rounded result.
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

namespace {

template <int L>
__device__ __forceinline__ int dcol_B(int tid, int m) {
    using Lo = Layout<L>;
    if constexpr (Lo::two_phase) {
        return (tid / Lo::lanes) * Lo::b + Lo::jB(tid % Lo::lanes, m);
    } else {
        return tid * Lo::E + m;
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values to a BF16 pair (RNE), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Cache policy of the output stores: non-temporal.  The decoded matrix is written once and
// streamed; on gfx950 this raises the sustained rate of the mixed code-read / output-write
// traffic from about 4.5 to about 6 TB/s (measured with 1 KiB-contiguous 16-byte stores).
constexpr int kStoreNT = 2;


__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* codes, size_t stride, int row) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(codes + (size_t)row * stride), (short)0, (int)stride,
                                             0x00020000);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* out, int64_t ld, int esz, int d_in, int row) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(reinterpret_cast<char*>(out) + (size_t)row * ld * esz), (short)0,
                                             d_in * esz, 0x00020000);
}

// Reciprocal of a positive double within about one ulp: hardware estimate and two Newton steps.
__device__ __forceinline__ double recip(double v) {
    double r = __builtin_amdgcn_rcp(v);
    r = r * (2.0 - v * r);
    return r * (2.0 - v * r);
}

// Per-wavefront LDS staging.  One buffer serves, in turn, the row's packed codes (loaded with
// coalesced 16-byte loads), the transform exchange, and the output (stored with 16-byte stores,
// each instruction writing 1 KiB of consecutive bytes).  Output dword k lives at k + 4*(k/32)
// (padding keeps 16-byte alignment and spreads the scattered writes over the banks).
template <int L>
struct DecWave {
    using Lo = Layout<L>;
    static constexpr int E = Lo::E, NP = E / 2;
    static constexpr int out_f32 = kWave * E;                      // output dwords, fp32
    static constexpr int out_pad = out_f32 + 4 * (out_f32 / 32);
    static constexpr int nload = (E * 12 / 4 + kWave - 1) / kWave;  // 16-byte code loads per lane
    static constexpr int code_dw = 4 * kWave * nload;               // staged code dwords (all lanes)
    static constexpr int xch_dw = Lo::two_phase ? 2 * Lo::xbuf : 0;
    static constexpr int dwords = (out_pad > code_dw ? (out_pad > xch_dw ? out_pad : xch_dw)
                                                     : (code_dw > xch_dw ? code_dw : xch_dw));
    __device__ static constexpr int pad(int k) { return k + 4 * (k >> 5); }
};

// The dwords that hold NP consecutive fields of BITS bits, whatever the bit phase of the first.
template <int NP, int BITS>
struct LaneCodes {
    static constexpr int NA = (NP * BITS + 31) / 32;   // dwords of the fields once aligned
    static constexpr int ND = NA + 1;                  // dwords to load
};

// N consecutive dwords from byte offset off of a buffer (dword-aligned; dwords past the
// descriptor's size read as 0, each dword checked on its own).
template <int N>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t* d) {
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

// The NP fields of a lane from its loaded dwords; s0 = bit phase of the first field.
template <int NP, int BITS>
__device__ __forceinline__ void unpack_lane(const uint32_t (&dw)[LaneCodes<NP, BITS>::ND], uint32_t s0,
                                            int (&idx)[NP]) {
    constexpr int NA = LaneCodes<NP, BITS>::NA;
    uint32_t al[NA];
#pragma unroll
    for (int t = 0; t < NA; ++t) al[t] = __builtin_amdgcn_alignbit(dw[t + 1], dw[t], s0);
    constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int off = i * BITS, w = off >> 5, sh = off & 31;
        const uint32_t v = (sh + BITS <= 32) ? (al[w] >> sh) : __builtin_amdgcn_alignbit(al[w + 1], al[w], sh);
        idx[i] = (int)(v & mask);
    }
}

template <int L, int BITS>
__device__ __forceinline__ void unpack_staged(const uint32_t* wb, int lane, int bits, int (&idx)[Layout<L>::E / 2]) {
    constexpr int NP = Layout<L>::E / 2;
    const uint32_t bp0 = (uint32_t)(lane * NP) * (uint32_t)bits;
    if constexpr (BITS > 0) {
        constexpr int NA = (NP * BITS + 31) / 32;
        const uint32_t d0 = bp0 >> 5, s0 = bp0 & 31;
        uint32_t dw[NA + 1];
#pragma unroll
        for (int t = 0; t <= NA; ++t) dw[t] = wb[d0 + t];
        uint32_t al[NA];
#pragma unroll
        for (int t = 0; t < NA; ++t) al[t] = __builtin_amdgcn_alignbit(dw[t + 1], dw[t], s0);
        constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int off = i * BITS, w = off >> 5, sh = off & 31;
            uint32_t v = (sh + BITS <= 32) ? (al[w] >> sh) : __builtin_amdgcn_alignbit(al[w + 1], al[w], sh);
            idx[i] = (int)(v & mask);
        }
    } else {
        const uint32_t mask = (1u << bits) - 1u;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const uint32_t bp = bp0 + (uint32_t)(i * bits);
            const uint32_t d = bp >> 5;
            idx[i] = (int)(__builtin_amdgcn_alignbit(wb[d + 1], wb[d], bp & 31) & mask);
        }
    }
}

// A workgroup decodes R rows at a time (R groups of T lanes, T = lanes per row) and walks rows
// strided over the grid with the next row's codes in flight.  Memory accesses never branch:
// idle lanes and rows past the end load and store through offsets or descriptors outside their
// buffers (loads return 0, stores are dropped), so the wait for the prefetched row can leave the
// previous row's stores in flight.  A row with a zero norm takes a branch that is uniform over
// its group and writes +0.
//
// With a compile-time field width each lane loads the dwords holding its own fields straight
// into registers; otherwise the group stages the row's codes in LDS.  The output leaves through
// the wave's LDS buffer: 16-byte stores, each instruction writing 1 KiB of consecutive bytes.
template <int L, int BITS, int MAXT, bool OBF>
__global__ __launch_bounds__(MAXT) void k_decode(DecodeArgs a, int T, int R) {
    using Lo = Layout<L>;
    using DW = DecWave<L>;
    constexpr int E = Lo::E, NP = E / 2;
    constexpr int ESZ = OBF ? 2 : 4;
    constexpr bool kLaneLoads = BITS > 0;
    extern __shared__ __align__(16) char smem[];
    const int bits = BITS > 0 ? BITS : a.bits;
    const int K = 1 << bits;
    double2* tab = reinterpret_cast<double2*>(smem);
    uint32_t* wb = reinterpret_cast<uint32_t*>(smem + (size_t)K * sizeof(double2)) + (threadIdx.x / kWave) * DW::dwords;
    double* xb = reinterpret_cast<double*>(wb);

    // which of the R concurrent rows; uniform per wavefront (T is a multiple of 64), and saying so
    // keeps buffer descriptors and row indices in scalar registers
    const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / T);
    const int tid = threadIdx.x - grp * T;     // lane within the row
    const int lane = threadIdx.x & (kWave - 1);
    const int wave_in_row = tid / kWave;
    const bool active = tid < a.d_in / E;
    const int rstride = gridDim.x * R;

    // this wave's code span: E*bits dwords from dword wave_in_row*E*bits of the row; this lane's
    // fields start at bit bp0 of the span
    const int span_dw = E * bits;
    const uint32_t bp0 = (uint32_t)(lane * NP) * (uint32_t)bits;
    const uint32_t s0 = bp0 & 31u;
    constexpr int ND = kLaneLoads ? LaneCodes<NP, (BITS > 0 ? BITS : 1)>::ND : 4 * DW::nload;
    uint32_t lane_off = active ? (uint32_t)(wave_in_row * span_dw * 4) + (bp0 >> 5) * 4u : 0x7FFFFF00u;
    uint32_t coff[DW::nload];
#pragma unroll
    for (int c = 0; c < DW::nload; ++c) {
        const int d = 4 * (lane + c * kWave);
        coff[c] = d < span_dw ? (uint32_t)((wave_in_row * span_dw + d) * 4) : 0x7FFFFFF0u;
    }

    const __amdgpu_buffer_rsrc_t nrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.norm, (short)0, a.d_out * 2, 0x00020000);
    auto load_row = [&](int r, uint32_t (&dst)[ND]) {
        const bool ok = r < a.d_out;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.codes + (size_t)(ok ? r : 0) * a.stride), (short)0, ok ? (int)a.stride : 0, 0x00020000);
        if constexpr (kLaneLoads) {
            load_dwords<ND>(rs, lane_off, dst);
        } else {
#pragma unroll
            for (int c = 0; c < DW::nload; ++c) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, coff[c], 0, 0);
#pragma unroll
                for (int k = 0; k < 4; ++k) dst[4 * c + k] = v[k];
            }
        }
    };
    // Row norms come in batches of 64: lane l holds the norm of the group's row r0 + l * rstride
    // (0 past the end), and pass n of the batch reads lane n.  A batch is loaded (and waited for)
    // once per 64 passes, so no pass waits on a norm load issued in that pass.
    auto load_norms = [&](int r0) {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
            nrs, ((uint32_t)r0 + (uint32_t)lane * (uint32_t)rstride) * 2u, 0, 0);
    };

    int row = blockIdx.x * R + grp;
    uint32_t nxt[ND];
    load_row(row, nxt);
    uint32_t nbatch = load_norms(row);

    // ---- once per workgroup: codebook table, sigma of this lane's pairs, eps_j / s_j of its columns
    {   // table entry j = (c_x + c_y, c_x - c_y), exact in double; two codewords per 16-byte load
        const __amdgpu_buffer_rsrc_t crs =
            __builtin_amdgcn_make_buffer_rsrc((void*)a.cb, (short)0, K * 8, 0x00020000);
        for (int j = 2 * (int)threadIdx.x; j < K; j += 2 * (int)blockDim.x) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(crs, (uint32_t)j * 8u, 0, 0);
            const double x0 = __uint_as_float(v[0]), y0 = __uint_as_float(v[1]);
            const double x1 = __uint_as_float(v[2]), y1 = __uint_as_float(v[3]);
            tab[j] = make_double2(x0 + y0, x0 - y0);
            tab[j + 1] = make_double2(x1 + y1, x1 - y1);
        }
    }
    float sg[NP];   // kept in fp32 (half the registers); widened exactly where used
    {
        const __amdgpu_buffer_rsrc_t srs =
            __builtin_amdgcn_make_buffer_rsrc((void*)a.sigma, (short)0, (a.d_in / 2) * 4, 0x00020000);
#pragma unroll
        for (int c = 0; c < NP / 4; ++c) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(srs, (uint32_t)(tid * NP + 4 * c) * 4u, 0, 0);
#pragma unroll
            for (int k = 0; k < 4; ++k) sg[4 * c + k] = __uint_as_float(v[k]);
        }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) pin_reg(sg[i]);
    // eps_j / s_j: the workgroup computes a chunk of columns into LDS (the staging buffers, not yet
    // in use), four columns per thread, and each lane copies the columns it owns.  Chunks hold
    // whole column groups (a lane's columns never straddle two chunks).
    double cf[E];
#pragma unroll
    for (int m = 0; m < E; ++m) cf[m] = 1.0;
    {
        double* cfl = reinterpret_cast<double*>(smem + (size_t)K * sizeof(double2));
        constexpr int CB = Lo::b > E ? Lo::b : E;
        const int chunk = (int)(blockDim.x / kWave) * DW::dwords / 2 / CB * CB;
        const int my0 = Lo::two_phase ? (tid / Lo::lanes) * Lo::b : tid * E;   // first column of the group
        const __amdgpu_buffer_rsrc_t srs =
            __builtin_amdgcn_make_buffer_rsrc((void*)a.scale, (short)0, a.scale ? a.d_in * 4 : 0, 0x00020000);
        for (int c0 = 0; c0 < a.d_in; c0 += chunk) {
            const int n = min(chunk, a.d_in - c0);
            for (int j = 4 * (int)threadIdx.x; j < n; j += 4 * (int)blockDim.x) {
                const int col = c0 + j;   // a multiple of 4
                double r[4] = {1.0, 1.0, 1.0, 1.0};
                if (a.scale) {
                    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(srs, (uint32_t)col * 4u, 0, 0);
#pragma unroll
                    for (int u = 0; u < 4; ++u) r[u] = recip((double)__uint_as_float(v[u]));
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (eps_negative(a.sign_seed, (uint32_t)(col + u))) r[u] = -r[u];
                if (j + 4 <= n) {
                    *reinterpret_cast<double2*>(cfl + j) = make_double2(r[0], r[1]);
                    *reinterpret_cast<double2*>(cfl + j + 2) = make_double2(r[2], r[3]);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (j + u < n) cfl[j + u] = r[u];
                }
            }
            __syncthreads();
            if (my0 >= c0 && my0 < c0 + n) {
#pragma unroll
                for (int m = 0; m < E; m += 2) {
                    const int col = dcol_B<L>(tid, m);   // even; col + 1 is element m + 1
                    if (col < a.d_in) {
                        const double2 v = *reinterpret_cast<const double2*>(cfl + (col - c0));
                        cf[m] = v.x;
                        cf[m + 1] = v.y;
                    }
                }
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int m = 0; m < E; ++m) pin_reg(cf[m]);
    const double inv_sqrt_b = 1.0 / __builtin_sqrt((double)Lo::b);
    // Output, staged: chunk c of this wave covers dwords [256 c, 256 c + 256) of the wave's span;
    // element m of this lane goes to dword pad(kb + o(m)) of the wave buffer, kb per lane and o(m)
    // a compile-time offset.  kb's place within its 32-dword group plus o(m)'s never crosses a
    // group, so pad(kb + o) = pad(kb) + o + 4*(o/32): one base register.
    constexpr int out_dw = kWave * E * ESZ / 4;
    constexpr int nchunk = out_dw / 256;
    const uint32_t wave_byte0 = (uint32_t)(wave_in_row * out_dw * 4);
    uint32_t* stg;
    {
        const unsigned ul = (unsigned)lane;
        unsigned kb;
        if constexpr (Lo::two_phase) {
            const unsigned beta = ul / Lo::lanes, q = ul % Lo::lanes;
            kb = OBF ? beta * (Lo::b / 2) + q : beta * Lo::b + 2 * q;
        } else {
            kb = OBF ? ul * (E / 2) : ul * E;
        }
        stg = wb + DW::pad((int)kb);
    }
    __syncthreads();

    int npass = 0;
    for (; row < a.d_out; row += rstride) {
        if (npass == kWave) {
            nbatch = load_norms(row);
            pin_reg(nbatch);   // waited for here, not at the reads of later passes
            npass = 0;
        }
        const uint16_t nh = (uint16_t)__builtin_amdgcn_readlane(nbatch, npass);
        ++npass;
        const float rn = __half2float(__ushort_as_half(nh));
        // this lane's fields, then the next row's codes into the same registers
        int idx[NP];
        if constexpr (kLaneLoads) {
            unpack_lane<NP, (BITS > 0 ? BITS : 1)>(nxt, s0, idx);
        } else {
#pragma unroll
            for (int c = 0; c < DW::nload; ++c)
                *reinterpret_cast<u32x4*>(wb + 4 * (lane + c * kWave)) =
                    u32x4{nxt[4 * c], nxt[4 * c + 1], nxt[4 * c + 2], nxt[4 * c + 3]};
            wave_lds_sync();
            unpack_staged<L, BITS>(wb, lane, bits, idx);
            wave_lds_sync();
        }
        load_row(row + rstride, nxt);   // keep the next row in flight
        uint32_t ow[E * ESZ / 4];       // output dwords of this lane, in m order
        if (rn != 0.0f) {
            double x[E];
            const double g = (double)rn * inv_sqrt_b;
            // all NP table reads in flight at once, then one wait
            double2 t[NP];
#pragma unroll
            for (int i = 0; i < NP; ++i) t[i] = tab[idx[i]];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const double sc = (double)sg[i] * g;
                x[2 * i] = t[i].x * sc;
                x[2 * i + 1] = t[i].y * sc;
            }
            // Stage 0 is in the table; the other stages never mix the halves (element bit 0 = 0
            // or 1), so each half is exchanged while the other one is transformed: the LDS
            // latency of one half hides behind the arithmetic of the other.
            float f[E];   // x * eps / s, rounded to fp32
            if constexpr (Lo::two_phase) {
                const Exchange<L> ex(xb, lane);
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
#pragma unroll
                for (int m = 0; m < E; m += 2) f[m] = (float)(x[m] * cf[m]);
                wave_lds_sync();
                ex.read(x, 1);
                wave_lds_sync();
#pragma unroll
                for (int r = 1; r < Lo::e; ++r)
                    if (L - Lo::e + r >= Lo::e) butterfly_half<E>(x, r, 1);
#pragma unroll
                for (int m = 1; m < E; m += 2) f[m] = (float)(x[m] * cf[m]);
            } else {
#pragma unroll
                for (int r = 1; r < L; ++r) butterfly<E>(x, r);
#pragma unroll
                for (int m = 0; m < E; ++m) f[m] = (float)(x[m] * cf[m]);
            }
            // round to the output type
#pragma unroll
            for (int m = 0; m < E; m += 2) {
                if constexpr (OBF) {
                    ow[m / 2] = pack_bf16x2(f[m], f[m + 1]);
                } else {
                    ow[m] = __float_as_uint(f[m]);
                    ow[m + 1] = __float_as_uint(f[m + 1]);
                }
            }
        } else {   // a zero row decodes to +0
#pragma unroll
            for (int k = 0; k < E * ESZ / 4; ++k) ow[k] = 0u;
        }
        const bool rv = row < a.d_out;
        const __amdgpu_buffer_rsrc_t ors = out_rsrc(a.out, a.ld, ESZ, rv ? a.d_in : 0, rv ? row : 0);
        // stage in wave order, then 16-byte stores
#pragma unroll
        for (int m = 0; m < E; m += 2) {
            if constexpr (OBF) {
                const int o = Lo::two_phase ? (m >> 1) * Lo::lanes : m / 2;
                stg[o + 4 * (o >> 5)] = ow[m / 2];
            } else {
                const int o = Lo::two_phase ? (m >> 1) * 2 * Lo::lanes : m;
                stg[o + 4 * (o >> 5)] = ow[m];
                stg[o + 1 + 4 * ((o + 1) >> 5)] = ow[m + 1];
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int c = 0; c < nchunk; ++c) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(wb + DW::pad(256 * c + 4 * lane));
            const uint32_t off = wave_byte0 + (uint32_t)(c * 1024 + 16 * lane);
            if constexpr (L >= 3) {   // d_in is a multiple of b >= 8: rows are whole 16-byte chunks
                __builtin_amdgcn_raw_buffer_store_b128(v, ors, off, 0, kStoreNT);
            } else {
                __builtin_amdgcn_raw_buffer_store_b32(v[0], ors, off, 0, kStoreNT);
                __builtin_amdgcn_raw_buffer_store_b32(v[1], ors, off + 4, 0, kStoreNT);
                __builtin_amdgcn_raw_buffer_store_b32(v[2], ors, off + 8, 0, kStoreNT);
                __builtin_amdgcn_raw_buffer_store_b32(v[3], ors, off + 12, 0, kStoreNT);
            }
        }
        wave_lds_sync();   // the wave buffer is rewritten by the next pass
    }
}

template <int L>
size_t decode_smem(int K, int nwaves) {
    return (size_t)K * sizeof(double2) + (size_t)nwaves * DecWave<L>::dwords * sizeof(uint32_t);
}

template <int L, int BITS, bool OBF>
hipError_t decode_LBO(const DecodeArgs& a, hipStream_t st) {
    using Lo = Layout<L>;
    constexpr int kMax = L <= 7 ? 1024 : 512;   // rows of more than 512 lanes exist only for E = 16
    const int T = ((a.d_in / Lo::E) + kWave - 1) / kWave * kWave;
    if (T > kMax) return hipErrorInvalidConfiguration;
    int R = kMax / T;
    if (R > 4) R = 4;
    if (R > a.d_out) R = a.d_out > 0 ? a.d_out : 1;
    while (R > 1 && decode_smem<L>(1 << a.bits, R * T / kWave) > kLdsBytes) --R;
    const int threads = R * T;
    const size_t smem = decode_smem<L>(1 << a.bits, threads / kWave);
    if (smem > kLdsBytes) return hipErrorInvalidConfiguration;
    int per_cu = (int)(kLdsBytes / smem);
    if (per_cu * (threads / kWave) > 32) per_cu = 32 / (threads / kWave);
    if (per_cu < 1) per_cu = 1;
    int grid = 256 * per_cu;
    const int need = (a.d_out + R - 1) / R;
    if (grid > need) grid = need;
    if (grid < 1) return hipSuccess;
    if (threads <= 512) {
        allow_lds(k_decode<L, BITS, 512, OBF>, smem);
        hipLaunchKernelGGL((k_decode<L, BITS, 512, OBF>), dim3(grid), dim3(threads), smem, st, a, T, R);
    } else if constexpr (L <= 7) {
        allow_lds(k_decode<L, BITS, 1024, OBF>, smem);
        hipLaunchKernelGGL((k_decode<L, BITS, 1024, OBF>), dim3(grid), dim3(threads), smem, st, a, T, R);
    } else {
        return hipErrorInvalidConfiguration;
    }
    return hipGetLastError();
}

template <int L, int BITS>
hipError_t decode_LB(const DecodeArgs& a, hipStream_t st) {
    return a.out_bf16 ? decode_LBO<L, BITS, true>(a, st) : decode_LBO<L, BITS, false>(a, st);
}

template <int L>
hipError_t decode_L(const DecodeArgs& a, hipStream_t st) {
    switch (a.bits) {
    case 7: return decode_LB<L, 7>(a, st);
    case 8: return decode_LB<L, 8>(a, st);
    case 11: return decode_LB<L, 11>(a, st);
    default: return decode_LB<L, 0>(a, st);
    }
}

}  // namespace

size_t decode_lds_bytes(int L, int bits, int d_in) {
    const int E = lane_elems(L);
    if (E <= 0) return 0;
    const int nwaves = ((d_in / E) + kWave - 1) / kWave;
    switch (L) {
    case 1: return decode_smem<1>(1 << bits, nwaves);
    case 2: return decode_smem<2>(1 << bits, nwaves);
    case 3: return decode_smem<3>(1 << bits, nwaves);
    case 4: return decode_smem<4>(1 << bits, nwaves);
    case 5: return decode_smem<5>(1 << bits, nwaves);
    case 6: return decode_smem<6>(1 << bits, nwaves);
    case 7: return decode_smem<7>(1 << bits, nwaves);
    case 8: return decode_smem<8>(1 << bits, nwaves);
    case 9: return decode_smem<9>(1 << bits, nwaves);
    case 10: return decode_smem<10>(1 << bits, nwaves);
    default: return 0;
    }
}

hipError_t launch_decode(const DecodeArgs& a, int L, hipStream_t st) {
    if (decode128_supported(a, L)) return launch_decode128(a, L, st);
    switch (L) {
    case 1: return decode_L<1>(a, st);
    case 2: return decode_L<2>(a, st);
    case 3: return decode_L<3>(a, st);
    case 4: return decode_L<4>(a, st);
    case 5: return decode_L<5>(a, st);
    case 6: return decode_L<6>(a, st);
    case 7: return decode_L<7>(a, st);
    case 8: return decode_L<8>(a, st);
    case 9: return decode_L<9>(a, st);
    case 10: return decode_L<10>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qamw
