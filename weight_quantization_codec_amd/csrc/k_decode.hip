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
// strided over the grid with the next row's codes in flight.  Every lane runs the same
// instruction stream: idle lanes load and store through buffer descriptors with offsets beyond
// their bounds (loads then return 0, stores are dropped), and rows with a zero norm select +0
// after the arithmetic, so the compiler never has to wait for this row's stores.
template <int L, int BITS, int MAXT, bool OBF>
__global__ __launch_bounds__(MAXT) void k_decode(DecodeArgs a, int T, int R) {
    using Lo = Layout<L>;
    using DW = DecWave<L>;
    constexpr int E = Lo::E, NP = E / 2;
    constexpr int ESZ = OBF ? 2 : 4;
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
    const uint16_t* __restrict__ norms = a.norm;
    const int rstride = gridDim.x * R;

    // this wave's code span: E*bits dwords from dword wave_in_row*E*bits of the row
    const int span_dw = E * bits;
    uint32_t coff[DW::nload];
#pragma unroll
    for (int c = 0; c < DW::nload; ++c) {
        const int d = 4 * (lane + c * kWave);
        coff[c] = d < span_dw ? (uint32_t)((wave_in_row * span_dw + d) * 4) : 0x7FFFFFF0u;
    }

    int row = blockIdx.x * R + grp;
    u32x4 nxt[DW::nload];
    uint16_t nh_next = 0;
    if (row < a.d_out) {
        nh_next = norms[row];
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.codes, a.stride, row);
#pragma unroll
        for (int c = 0; c < DW::nload; ++c) nxt[c] = __builtin_amdgcn_raw_buffer_load_b128(rs, coff[c], 0, 0);
    }

    for (int j = threadIdx.x; j < K; j += blockDim.x) {
        float2 c = reinterpret_cast<const float2*>(a.cb)[j];
        tab[j] = make_double2((double)c.x + (double)c.y, (double)c.x - (double)c.y);   // exact in double
    }
    double sg[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        sg[i] = (double)a.sigma[min(tid * NP + i, a.d_in / 2 - 1)];
        pin_reg(sg[i]);
    }
    double cf[E];
#pragma unroll
    for (int m = 0; m < E; ++m) {
        int j = min(dcol_B<L>(tid, m), a.d_in - 1);
        double e = (a.sign && ((a.sign[j >> 5] >> (j & 31)) & 1u)) ? -1.0 : 1.0;
        cf[m] = e * recip(a.scale ? (double)a.scale[j] : 1.0);
        pin_reg(cf[m]);
    }
    // output: chunk c of this wave covers dwords [256 c, 256 c + 256) of the wave's span
    constexpr int out_dw = kWave * E * ESZ / 4;
    constexpr int nchunk = out_dw / 256;
    const uint32_t wave_byte0 = (uint32_t)(wave_in_row * out_dw * 4);
    const double inv_sqrt_b = 1.0 / __builtin_sqrt((double)Lo::b);
    __syncthreads();

    for (; row < a.d_out; row += rstride) {
        const uint16_t nh = nh_next;
        u32x4 cur[DW::nload];
#pragma unroll
        for (int c = 0; c < DW::nload; ++c) cur[c] = nxt[c];
        const int rnext = row + rstride;
        if (rnext < a.d_out) {   // keep the next row's codes in flight
            nh_next = norms[rnext];
            const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.codes, a.stride, rnext);
#pragma unroll
            for (int c = 0; c < DW::nload; ++c) nxt[c] = __builtin_amdgcn_raw_buffer_load_b128(rs, coff[c], 0, 0);
        }
        const float rn = __half2float(__ushort_as_half(nh));
        const bool zero_row = rn == 0.0f;
        // codes -> LDS -> fields of this lane
#pragma unroll
        for (int c = 0; c < DW::nload; ++c) *reinterpret_cast<u32x4*>(wb + 4 * (lane + c * kWave)) = cur[c];
        wave_lds_sync();
        double x[E];
        {
            int idx[NP];
            unpack_staged<L, BITS>(wb, lane, bits, idx);
            const double g = (double)rn * inv_sqrt_b;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                double2 t = tab[idx[i]];
                double sc = sg[i] * g;
                x[2 * i] = t.x * sc;
                x[2 * i + 1] = t.y * sc;
            }
        }
        wave_lds_sync();
        if constexpr (Lo::two_phase) {
#pragma unroll
            for (int r = 1; r < Lo::e; ++r) butterfly<E>(x, r);
            exchange_AB<L>(x, xb, lane);
#pragma unroll
            for (int r = 1; r < Lo::e; ++r)
                if (L - Lo::e + r >= Lo::e) butterfly<E>(x, r);
        } else {
#pragma unroll
            for (int r = 1; r < L; ++r) butterfly<E>(x, r);
        }
        // scale, round, and stage the output in wave order
#pragma unroll
        for (int m = 0; m < E; m += 2) {
            float v0 = (float)(x[m] * cf[m]);
            float v1 = (float)(x[m + 1] * cf[m + 1]);
            const int e = dcol_B<L>(lane, m);   // element index within the wave's span
            if constexpr (OBF) {
                __hip_bfloat162 p = __float22bfloat162_rn(make_float2(v0, v1));
                uint32_t u = *reinterpret_cast<uint32_t*>(&p);
                wb[DW::pad(e >> 1)] = zero_row ? 0u : u;   // a zero row decodes to +0
            } else {
                wb[DW::pad(e)] = zero_row ? 0u : __float_as_uint(v0);
                wb[DW::pad(e + 1)] = zero_row ? 0u : __float_as_uint(v1);
            }
        }
        wave_lds_sync();
        const __amdgpu_buffer_rsrc_t ors = out_rsrc(a.out, a.ld, ESZ, a.d_in, row);
#pragma unroll
        for (int c = 0; c < nchunk; ++c) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(wb + DW::pad(256 * c + 4 * lane));
            const uint32_t off = wave_byte0 + (uint32_t)(c * 1024 + 16 * lane);
            if constexpr (L >= 3) {   // d_in is a multiple of b >= 8: rows are whole 16-byte chunks
                __builtin_amdgcn_raw_buffer_store_b128(v, ors, off, 0, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b32(v[0], ors, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(v[1], ors, off + 4, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(v[2], ors, off + 8, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(v[3], ors, off + 12, 0, 0);
            }
        }
        wave_lds_sync();
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

hipError_t launch_decode(const DecodeArgs& a, int L, hipStream_t st) {
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
