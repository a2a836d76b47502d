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

// Code words of one lane for one row: the NP fields of `bits` bits starting at stream bit
// `bitpos`.  BITS > 0 makes the field width a compile-time constant so that every shift is static;
// the dwords are loaded first (so that the next row can be prefetched) and unpacked later.
template <int NP, int BITS>
struct CodeWords {
    static constexpr int NA = BITS > 0 ? (NP * BITS + 31) / 32 : 1;
    uint32_t dw[NA + 1];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* codes, size_t stride, int row) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(codes + (size_t)row * stride), (short)0, (int)stride,
                                             0x00020000);
}

template <int NP, int BITS>
__device__ __forceinline__ void load_codes(__amdgpu_buffer_rsrc_t rs, uint32_t bitpos, CodeWords<NP, BITS>& c) {
    if constexpr (BITS > 0) {
        const uint32_t d0 = bitpos >> 5;
#pragma unroll
        for (int t = 0; t <= CodeWords<NP, BITS>::NA; ++t)
            c.dw[t] = __builtin_amdgcn_raw_buffer_load_b32(rs, (d0 + t) * 4, 0, 0);
    }
}

template <int NP, int BITS>
__device__ __forceinline__ void unpack_codes(const CodeWords<NP, BITS>& c, __amdgpu_buffer_rsrc_t rs, uint32_t bitpos,
                                             int bits, int (&idx)[NP]) {
    if constexpr (BITS > 0) {
        constexpr int NA = CodeWords<NP, BITS>::NA;
        const uint32_t s0 = bitpos & 31;
        uint32_t al[NA];
#pragma unroll
        for (int t = 0; t < NA; ++t) al[t] = __builtin_amdgcn_alignbit(c.dw[t + 1], c.dw[t], s0);
        constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int off = i * BITS, w = off >> 5, sh = off & 31;
            uint32_t v = (sh + BITS <= 32) ? (al[w] >> sh) : __builtin_amdgcn_alignbit(al[w + 1], al[w], sh);
            idx[i] = (int)(v & mask);
        }
    } else {
        const uint32_t mask = (bits >= 32) ? 0xFFFFFFFFu : ((1u << bits) - 1u);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            uint32_t bp = bitpos + (uint32_t)(i * bits);
            uint32_t d = bp >> 5;
            uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(rs, d * 4, 0, 0);
            uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(rs, (d + 1) * 4, 0, 0);
            idx[i] = (int)(__builtin_amdgcn_alignbit(hi, lo, bp & 31) & mask);
        }
    }
}

template <int L, int BITS, int MAXT>
__global__ __launch_bounds__(MAXT) void k_decode(DecodeArgs a) {
    using Lo = Layout<L>;
    constexpr int E = Lo::E, NP = E / 2;
    extern __shared__ __align__(16) char smem[];
    const int bits = BITS > 0 ? BITS : a.bits;
    const int K = 1 << bits;
    const int tid = threadIdx.x;
    double2* tab = reinterpret_cast<double2*>(smem);
    double* xb = reinterpret_cast<double*>(smem + (size_t)K * sizeof(double2)) + (tid / kWave) * Lo::xbuf;

    const int units = a.d_in / E;
    const bool active = tid < units;
    const uint32_t bitpos = (uint32_t)(tid * NP) * (uint32_t)bits;

    // first row's codes in flight while the tables are set up
    int row = blockIdx.x;
    CodeWords<NP, BITS> nxt;
    uint16_t nh_next = 0;
    if (row < a.d_out) {
        nh_next = a.norm[row];
        if (active) load_codes<NP, BITS>(row_rsrc(a.codes, a.stride, row), bitpos, nxt);
    }

    for (int j = tid; j < K; j += blockDim.x) {
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
        cf[m] = e * (1.0 / (a.scale ? (double)a.scale[j] : 1.0));
        pin_reg(cf[m]);
    }
    const double inv_sqrt_b = 1.0 / __builtin_sqrt((double)Lo::b);
    __syncthreads();

    for (; row < a.d_out; row += gridDim.x) {
        const uint16_t nh = nh_next;
        const CodeWords<NP, BITS> cur = nxt;
        const int rnext = row + (int)gridDim.x;
        if (rnext < a.d_out) {   // prefetch the next row
            nh_next = a.norm[rnext];
            if (active) load_codes<NP, BITS>(row_rsrc(a.codes, a.stride, rnext), bitpos, nxt);
        }
        const float rn = __half2float(__ushort_as_half(nh));
        char* orow = reinterpret_cast<char*>(a.out) + (size_t)row * a.ld * (a.out_bf16 ? 2 : 4);
        if (rn == 0.0f) {
            if (active) {
#pragma unroll
                for (int m = 0; m < E; m += 2) {
                    int c = dcol_B<L>(tid, m);
                    if (a.out_bf16)
                        *reinterpret_cast<uint32_t*>(orow + (size_t)c * 2) = 0u;
                    else
                        *reinterpret_cast<float2*>(orow + (size_t)c * 4) = make_float2(0.f, 0.f);
                }
            }
            continue;
        }
        double x[E];
        if (active) {
            int idx[NP];
            unpack_codes<NP, BITS>(cur, row_rsrc(a.codes, a.stride, row), bitpos, bits, idx);
            const double g = (double)rn * inv_sqrt_b;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                double2 t = tab[idx[i]];
                double s = sg[i] * g;
                x[2 * i] = t.x * s;
                x[2 * i + 1] = t.y * s;
            }
        } else {
#pragma unroll
            for (int m = 0; m < E; ++m) x[m] = 0.0;
        }
        if constexpr (Lo::two_phase) {
#pragma unroll
            for (int r = 1; r < Lo::e; ++r) butterfly<E>(x, r);
            exchange_AB<L>(x, xb, tid & (kWave - 1));
#pragma unroll
            for (int r = 1; r < Lo::e; ++r)
                if (L - Lo::e + r >= Lo::e) butterfly<E>(x, r);
        } else {
#pragma unroll
            for (int r = 1; r < L; ++r) butterfly<E>(x, r);
        }
        if (active) {
#pragma unroll
            for (int m = 0; m < E; m += 2) {
                int c = dcol_B<L>(tid, m);
                float v0 = (float)(x[m] * cf[m]);
                float v1 = (float)(x[m + 1] * cf[m + 1]);
                if (a.out_bf16) {
                    __hip_bfloat162 p = __float22bfloat162_rn(make_float2(v0, v1));
                    *reinterpret_cast<__hip_bfloat162*>(orow + (size_t)c * 2) = p;
                } else {
                    *reinterpret_cast<float2*>(orow + (size_t)c * 4) = make_float2(v0, v1);
                }
            }
        }
    }
}

template <int L>
size_t decode_smem(int K, int nwaves) {
    using Lo = Layout<L>;
    return (size_t)K * sizeof(double2) + (Lo::two_phase ? (size_t)nwaves * Lo::xbuf * sizeof(double) : 0);
}

template <int L, int BITS>
hipError_t decode_LB(const DecodeArgs& a, hipStream_t st) {
    constexpr bool kWide = L <= 7;   // rows of more than 512 lanes exist only for E = 16
    using Lo = Layout<L>;
    int threads = ((a.d_in / Lo::E) + kWave - 1) / kWave * kWave;
    int nwaves = threads / kWave;
    size_t smem = decode_smem<L>(1 << a.bits, nwaves);
    int blocks_per_cu = (int)((160 * 1024) / smem);
    if (blocks_per_cu < 1) return hipErrorInvalidConfiguration;
    if (blocks_per_cu * nwaves > 32) blocks_per_cu = 32 / nwaves;
    if (blocks_per_cu < 1) blocks_per_cu = 1;
    int grid = 256 * blocks_per_cu;
    if (grid > a.d_out) grid = a.d_out;
    if (grid < 1) return hipSuccess;
    if (threads <= 512) {
        allow_lds(k_decode<L, BITS, 512>, smem);
        hipLaunchKernelGGL((k_decode<L, BITS, 512>), dim3(grid), dim3(threads), smem, st, a);
    } else if constexpr (kWide) {
        allow_lds(k_decode<L, BITS, 1024>, smem);
        hipLaunchKernelGGL((k_decode<L, BITS, 1024>), dim3(grid), dim3(threads), smem, st, a);
    } else {
        return hipErrorInvalidConfiguration;
    }
    return hipGetLastError();
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
