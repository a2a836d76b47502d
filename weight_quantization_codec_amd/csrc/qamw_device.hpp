// Device helpers shared by the QAM-W kernels (gfx950, wave64).
//
// Transform layout.  A Hadamard block of b = 2^L elements is spread over b/E lanes of one
// wavefront, E = 2^e elements per lane, in two register layouts:
//   phase A: lane q of the block holds elements q*E + m (m = 0..E-1, contiguous), so the
//            butterflies along element bits 0..e-1 are register-local;
//   phase B: lane q holds element j(q, m) = (m & 1) | (q << 1) | ((m >> 1) << (L - e + 1)),
//            so element bit 0 and bits L-e+1 .. L-1 are register-local.
// One exchange through LDS (per wavefront, no workgroup barrier) moves a block from phase A
// to phase B; with e = max(4, ceil((L+1)/2)) the two phases cover all L bits.  Element bit 0
// stays in registers in both layouts, so the (y_2k, y_2k+1) pairs of the paper (section 3.1
// step 3) are always held by one lane.  Blocks of b <= 16 fit in one lane (phase A only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qamw {

constexpr int kWave = 64;
constexpr int kIndexHeaderBytes = 256;
constexpr int kIndexCap = 32;         // uint16 slots per grid cell: [0] = count, then candidates
constexpr uint16_t kCellOverflow = 0xFFFF;

struct IndexHeader {
    int32_t K;
    int32_t G;       // grid is G x G cells over [-R, R]^2
    int32_t cap;
    int32_t bits;
    float R;
    float inv_h;     // G / (2R)
    int32_t ready;
    int32_t max_count;
};

template <int L>
struct Layout {
    static constexpr int b = 1 << L;
    static constexpr int e = (L <= 4) ? 4 : ((L + 2) / 2 < 4 ? 4 : (L + 2) / 2);
    static constexpr int E = 1 << e;
    static constexpr bool two_phase = L > 4;
    static constexpr int lanes = two_phase ? (b / E) : 1;   // lanes per block (two-phase)
    static constexpr int half = E / 2;                       // doubles per lane per exchange half
    // doubles per wavefront for one exchange half, padded by one double per lane run
    static constexpr int xbuf = kWave * half + kWave;
    __device__ static constexpr int jB(int q, int m) {
        return (m & 1) | (q << 1) | ((m >> 1) << (L - e + 1));
    }
};

template <int E>
__device__ __forceinline__ void butterfly(double (&x)[E], int rbit) {
#pragma unroll
    for (int m = 0; m < E; ++m) {
        if (!(m & (1 << rbit))) {
            double a = x[m], c = x[m | (1 << rbit)];
            x[m] = a + c;
            x[m | (1 << rbit)] = a - c;
        }
    }
}

// Make LDS writes of this wavefront visible to its other lanes before the reads that follow.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Phase A -> phase B for one wavefront.  `xb` is the wavefront's exchange buffer
// (Layout<L>::xbuf doubles).  lane = lane id in the wavefront.
template <int L>
__device__ __forceinline__ void exchange_AB(double (&x)[Layout<L>::E], double* xb, int lane) {
    using Lo = Layout<L>;
    constexpr int E = Lo::E, H = Lo::half;
    const int beta = lane / Lo::lanes, q = lane % Lo::lanes;
    const int base = beta * (Lo::b / 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // write: element q*E + 2i + h  ->  compact index c = base + q*H + i
#pragma unroll
        for (int i = 0; i < H; ++i) {
            int c = base + q * H + i;
            xb[c + c / H] = x[2 * i + h];
        }
        wave_lds_sync();
        // read: element j = h | (q << 1) | (i << (L-e+1))  ->  c = base + q + (i << (L-e))
#pragma unroll
        for (int i = 0; i < H; ++i) {
            int c = base + q + (i << (L - Lo::e));
            x[2 * i + h] = xb[c + c / H];
        }
        wave_lds_sync();
    }
}

// Exact nearest codeword (fp32 distance fl(fl(dx*dx) + fl(dy*dy)), ties to the lowest index)
// of (px, py) among the candidates of its grid cell; points outside the grid, non-finite
// points and overflowing cells search all K codewords.
__device__ __forceinline__ void eval_cw(float px, float py, float2 c, int j, float& bd, int& bj) {
    float dx = px - c.x;
    float dy = py - c.y;
    float d = dx * dx + dy * dy;   // built with -ffp-contract=off: three rounded operations
    if (d < bd) {
        bd = d;
        bj = j;
    }
}

__device__ __forceinline__ int nearest_indexed(float px, float py, const float2* __restrict__ cb, int K,
                                               const IndexHeader& ih, const uint16_t* __restrict__ slots) {
    float bd = __builtin_inff();
    int bj = 0;
    bool inside = fabsf(px) < ih.R && fabsf(py) < ih.R;
    int n = 0;
    const uint16_t* list = nullptr;
    if (inside) {
        int cx = min((int)((px + ih.R) * ih.inv_h), ih.G - 1);
        int cy = min((int)((py + ih.R) * ih.inv_h), ih.G - 1);
        list = slots + (size_t)(cy * ih.G + cx) * ih.cap;
        uint4 head = *reinterpret_cast<const uint4*>(list);
        n = head.x & 0xFFFF;
        if (n == kCellOverflow) {
            inside = false;
        } else {
            // first seven candidates come with the count
            uint32_t w[4] = {head.x, head.y, head.z, head.w};
#pragma unroll
            for (int t = 1; t < 8; ++t) {
                if (t <= n) {
                    int j = (w[t >> 1] >> ((t & 1) * 16)) & 0xFFFF;
                    eval_cw(px, py, cb[j], j, bd, bj);
                }
            }
            for (int t0 = 8; t0 <= n; t0 += 8) {
                uint4 v = *reinterpret_cast<const uint4*>(list + t0);
                uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    if (t0 + t <= n) {
                        int j = (u[t >> 1] >> ((t & 1) * 16)) & 0xFFFF;
                        eval_cw(px, py, cb[j], j, bd, bj);
                    }
                }
            }
        }
    }
    if (!inside) {
        for (int j = 0; j < K; ++j) eval_cw(px, py, cb[j], j, bd, bj);
    }
    return bj;
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ void flag_status(int32_t* status, int32_t f) {
    if (status && f) atomicOr(status, f);
}

}  // namespace qamw
