// Fused dequantize-and-multiply (paper section 1: the matrix product that follows the decoder)
// for M <= 16 activation rows:  y[m][i] = sum_j x[m][j] w^_ij,  w^ the decoder's output before rounding.
//
// W^ is never formed.  With D = diag(eps_j / s_j) and the block transform H = blockdiag(H_b)/sqrt(b)
// symmetric, row i of W^ is f16(norm_i) D H z_i with z_i,2k = sigma_k c[idx_ik].x (and .y), so
//   sum_j x_j w^_ij = f16(norm_i) sum_k (c[idx_ik] . u_k),   u_k = sigma_k (H D x)_(2k, 2k+1).
// k_qgemm_rotate_mx forms u once per call (fp64, rounded to fp32 once); k_qgemm_mx then reads only
// the packed codes (B/16 bytes per weight) from HBM and costs one codebook lookup per weight pair,
// the sums c[idx] . u running on the matrix cores.
#include <hip/hip_fp16.h>

#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);   // v_cvt_pk_bf16_f32: round to nearest even
}

// ---------------------------------------------------------------------------- bf16-piece operands
// k_qgemm_mx multiplies on v_mfma_f32_16x16x32_bf16.  Its operands are fp32 values written as sums of
// bf16 pieces, each piece the bf16 rounding of what the pieces before it leave: a codebook
// component c = c1 + c2 (|c - c1 - c2| <= 2^-18 |c|) and an activation value u = u1 + u2 (+ u3),
// |u - u1 - u2| <= 2^-18 |u|, three pieces exact.  Products of pieces are exact in fp32.
// The 16 B columns hold (activation row, u piece): for M <= 5 column 3 m + p with pieces p = 0..2
// (np = 3) and one operand group; for M <= 8 column 2 m + p, np = 2; for M <= 16 two operand
// groups, rows 8 g .. 8 g + 7, column 2 (m - 8 g) + p.  An A operand (c1 or c2) times such a B
// gives every piece product c_i u_p in one instruction; the sum over the pieces of a row is taken
// at the end.
struct QxMode {
    int ng, np, w32;   // operand groups, u pieces, 32-row tiles (k_qgemm_mx32)
};
// Above 8 rows: 32-row tiles once the 16-row tiles would take more than one round of the 256
// compute units (measured: on 4096 rows the 32-row tiles were 37% slower, half empty; from 5120
// rows on they were equal or up to 20% faster), two operand groups of 16-row tiles below.
__device__ __host__ __forceinline__ QxMode qx_mode(int M, int d_out) {
    if (M > 8) return d_out > 16 * 256 ? QxMode{1, 2, 1} : QxMode{2, 2, 0};
    return QxMode{1, M <= 5 ? 3 : 2, 0};
}
// pairs per chunk
__device__ __host__ __forceinline__ int qx_chunk(QxMode md) { return md.w32 ? 64 : 128; }
// Operand lane order (one chunk = 128 pairs, 8 steps of 16 pairs): lane l = 16 q + j holds, for
// step s, the k-slots of pairs 128 c + 32 q + 4 s + (0..3), components (x, y) in the low and high
// halves of each dword.  A: j = weight row of the tile; B: j = column.  The B operand of (chunk c,
// step s, group g) is 64 lanes x 4 dwords at entry ((c * 8 + s) * ng + g) * 64 + lane; the dword
// of pair k, piece p of activation row m:
// With 32-row tiles (k_qgemm_mx32, v_mfma_f32_32x32x16_bf16) a chunk is 64 pairs: lane l = 32 q + j
// holds the k-slots of pairs 64 c + 32 q + 4 s + (0..3), B column j = 2 m + p, at entry (c * 8 + s) *
// 64 + lane.
__device__ __forceinline__ size_t qx_dword(QxMode md, int m, int k, int p) {
    if (md.w32) {
        const int c = k >> 6, kk = k & 63, q = kk >> 5, t = kk & 31;
        return ((size_t)(c * 8 + (t >> 2)) * kWave + q * 32 + 2 * m + p) * 4 + (t & 3);
    }
    const int g = md.ng == 2 ? m >> 3 : 0, mm = md.ng == 2 ? m & 7 : m;
    const int c = k >> 7, kk = k & 127, q = kk >> 5, t = kk & 31;
    const size_t entry = ((size_t)(c * 8 + (t >> 2)) * md.ng + g) * kWave + q * 16 + md.np * mm + p;
    return entry * 4 + (t & 3);
}

// The rotation for k_qgemm_mx: u[m][j] = sigma_(j/2) (blockdiag(H_b) (eps . x_m / s))_j / sqrt(b) as
// unnormalized fp64 butterflies, rounded to fp32 once, written as bf16 pieces in the B operand order.  Workgroup: T =
// max(256, b / 2) threads, thread t holding pair t of 2 T columns of activation row blockIdx.y
// (whole blocks; columns past d_in are zeros, columns past `cols` are not written).  Butterflies:
// distance 1 in registers, 2 .. 64 between lanes of a wavefront through its own LDS slice (no
// barrier), 128 .. 512 across wavefronts (one barrier each); two LDS buffers alternate.
__global__ __launch_bounds__(512) void k_qgemm_rotate_mx(const void* __restrict__ x, int x_bf16, int64_t ld_x,
                                                         QxMode md, int d_in, int cols, int b,
                                                         const float* __restrict__ s, uint64_t sign_seed,
                                                         const float* __restrict__ sigma, uint32_t* __restrict__ uf) {
    __shared__ double2 ex[2][512];
    const int m = blockIdx.y, t = threadIdx.x;
    const int k = blockIdx.x * blockDim.x + t;   // the thread's pair
    double v[2] = {0.0, 0.0};
    double sg = 0.0;
    if (2 * k < d_in) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int col = 2 * k + i;
            const float xv = x_bf16 ? bf16_bits_to_float(reinterpret_cast<const uint16_t*>(x)[(size_t)m * ld_x + col])
                                    : reinterpret_cast<const float*>(x)[(size_t)m * ld_x + col];
            const double sc = s ? (double)s[col] : 1.0;
            v[i] = (eps_negative(sign_seed, (uint32_t)col) ? -(double)xv : (double)xv) / sc;
        }
        sg = (double)sigma[k];
    }
    // element i of the block: i ^ h is its partner; with bit h set it becomes partner - self,
    // else self + partner
    {
        const double a0 = v[0], a1 = v[1];
        v[0] = a0 + a1;
        v[1] = a0 - a1;
    }
    int buf = 0;
    for (int h = 2; h < b; h <<= 1, buf ^= 1) {
        const int dt = h >> 1;   // partner thread t ^ dt
        ex[buf][t] = make_double2(v[0], v[1]);
        if (dt < kWave) wave_lds_sync(); else __syncthreads();
        const double2 p = ex[buf][t ^ dt];
        const bool hi = (t & dt) != 0;
        v[0] = hi ? p.x - v[0] : v[0] + p.x;
        v[1] = hi ? p.y - v[1] : v[1] + p.y;
    }
    if (2 * k >= cols) return;
    float rx = 0.0f, ry = 0.0f;
    if (2 * k < d_in) {
        const double rs = 1.0 / __builtin_sqrt((double)b);
        rx = (float)(v[0] * rs * sg);
        ry = (float)(v[1] * rs * sg);
    }
    uint32_t* dst = uf + qx_dword(md, m, k, 0);   // piece p: 4 p dwords further
    for (int p = 0; p < md.np; ++p) {   // r = piece 0 + piece 1 (+ piece 2) + what is left
        const uint32_t px = f32_to_bf16_rne(rx), py = f32_to_bf16_rne(ry);
        rx -= __uint_as_float(px << 16);
        ry -= __uint_as_float(py << 16);
        dst[4 * p] = px | (py << 16);
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

// The product on the matrix cores in bf16 pieces: v_mfma_f32_16x16x32_bf16, D[16 x 16] += A[16 x 32]
// B[32 x 16], fp32 accumulation.  A = 16 weight rows x 16 pairs of codebook pieces (gathered from
// an LDS table of {c1, c2} per codeword, 8 B), B = the u pieces of those 16 pairs for the 16 columns of
// qx_mode.  Lane l = 16 q + j supplies A row j and B column j for the k-slots of its 4 pairs of
// the step, and holds D[4 q + v][j] (v = 0..3).  Per step and operand group: one instruction with
// A = c1, one with A = c2.
// Workgroup: one tile of 16 weight rows, WAVES wavefronts taking the chunks w, w + WAVES, ...
// (lane (j, q) reads the codes of row j for pairs 32 q .. 32 q + 31 of the chunk: BITS dwords,
// dword-aligned); each wavefront loads the next chunk's codes and B operands while it works on the
// current one.  The partial D of the wavefronts are added in LDS in wavefront order, then the
// pieces of each column.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Wavefronts per workgroup: 4, or 8 for rows of 40 chunks and more (measured on the 4096², 5120²,
// 13824 x 5120 and 5120 x 13824 products at M = 1, 4 and 16: 4 was up to 7% faster on the shorter
// rows, 8 up to 4% on the longest).
constexpr int kQxLongRow = 40;
constexpr int kComputeUnits = 256;   // MI355X

size_t qx_lds_bytes(int bits, int ng, int waves) {
    return (size_t)(1 << bits) * sizeof(uint2) + (size_t)waves * ng * kWave * sizeof(f32x4) +
           (size_t)ng * 256 * sizeof(float);
}

__device__ __forceinline__ f32x4 qx_mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// A operands (c1 and c2 pieces) of step s from the chunk's code dwords d (s a constant after
// unrolling, so the shifts and dword indices are too).  One 8-byte LDS read per codeword: the
// reads land at random addresses, and their cost goes by the instruction more than by its width.
template <int BITS>
__device__ __forceinline__ void qx_gather(const uint2* __restrict__ cb_l, const uint32_t (&d)[BITS], int s, u32x4& a1,
                                          u32x4& a2) {
    constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int off = (4 * s + e) * BITS, w = off >> 5, sh = off & 31;
        const uint32_t v = ((sh + BITS <= 32) ? (d[w] >> sh) : __builtin_amdgcn_alignbit(d[w + 1], d[w], sh)) & mask;
        const uint2 ent = cb_l[v];
        a1[e] = ent.x;
        a2[e] = ent.y;
    }
}

// Steps S0 .. S0 + NS - 1 of a chunk: NG = 1, operand b[s - S0 + BO]; NG = 2, b[2 (s - S0)] and
// b[2 (s - S0) + 1].  The gathers of a step are issued before the products of the step before it.
template <int BITS, int NG, int S0, int NS, int BO>
__device__ __forceinline__ void qx_steps(const uint2* __restrict__ cb_l, const uint32_t (&d)[BITS], const u32x4 (&b)[8],
                                         f32x4 (&acc)[2 * NG]) {
    u32x4 a1[2], a2[2];
    qx_gather<BITS>(cb_l, d, S0, a1[0], a2[0]);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
        if (t + 1 < NS) qx_gather<BITS>(cb_l, d, S0 + t + 1, a1[(t + 1) & 1], a2[(t + 1) & 1]);
        if constexpr (NG == 1) {
            acc[0] = qx_mfma(a1[t & 1], b[BO + t], acc[0]);
            acc[1] = qx_mfma(a2[t & 1], b[BO + t], acc[1]);
        } else {
            acc[0] = qx_mfma(a1[t & 1], b[2 * t], acc[0]);
            acc[1] = qx_mfma(a2[t & 1], b[2 * t], acc[1]);
            acc[2] = qx_mfma(a1[t & 1], b[2 * t + 1], acc[2]);
            acc[3] = qx_mfma(a2[t & 1], b[2 * t + 1], acc[3]);
        }
    }
}

template <int BITS, int NG, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(NG == 1 ? 4 : 3)))
void k_qgemm_mx(QgemmArgs a, int full, int tail_h) {
    constexpr int kQxWaves = WAVES;
    extern __shared__ __align__(16) char smem[];
    constexpr int K = 1 << BITS;
    constexpr int kThreads = kQxWaves * kWave;
    constexpr uint32_t kOut = 0xFFFFF000u;   // an offset past every descriptor's range: reads zeros
    uint2* cb_l = reinterpret_cast<uint2*>(smem);                                            // K x {c1, c2}
    f32x4* part = reinterpret_cast<f32x4*>(smem + (size_t)K * sizeof(uint2));               // waves x NG x 64
    float* dsum = reinterpret_cast<float*>(part + kQxWaves * NG * kWave);                   // NG x 16 x 16
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int j = lane & 15, q = lane >> 4;
    const QxMode md = qx_mode(a.M, a.d_out);
    const int n_chunks = (a.n_pairs + 127) / 128;
    // workgroups below `full` own 16 rows, the rest `tail_h` rows each (rows past d_out: none)
    const int tile = blockIdx.x;
    const int row0 = tile < full ? tile * 16 : full * 16 + (tile - full) * tail_h;
    const int h = tile < full ? 16 : tail_h;
    const int nrows = a.d_out - row0 < h ? a.d_out - row0 : h;

    // Every global load goes through a buffer descriptor, unconditionally (offsets past the range
    // read zeros), so that the loop has no branches around loads and the waits count exactly.
    // The codebook's loads come first, then the first chunk's: waiting for the former does not wait
    // for the latter.
    constexpr int kCbPer = (K + kThreads - 1) / kThreads;
    const __amdgpu_buffer_rsrc_t cbr =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.cb, (short)0, K * (int)sizeof(float2), 0x00020000);
    u32x2 cv[kCbPer];
#pragma unroll
    for (int t = 0; t < kCbPer; ++t)
        cv[t] = __builtin_amdgcn_raw_buffer_load_b64(cbr, (uint32_t)(threadIdx.x + t * kThreads) * 8u, 0, 0);
    // codes of the tile's rows through one descriptor (rows past the end read zeros)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.codes + (size_t)row0 * a.stride), (short)0, nrows * (int)a.stride, 0x00020000);
    const uint32_t row_off = (uint32_t)j * (uint32_t)a.stride;
    const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.u, (short)0, n_chunks * 8 * NG * kWave * (int)sizeof(u32x4), 0x00020000);
    // B columns that carry data; the other lanes read zeros without touching memory
    const int cols0 = md.ng == 2 ? 16 : md.np * a.M;
    const int cols1 = md.ng == 2 ? 2 * (a.M - 8) : 0;
    const bool on0 = j < cols0, on1 = j < cols1;
    // a B block: 8 operands (NG = 1: the 8 steps of a chunk; NG = 2: 4 steps x 2 groups, half a chunk)
    auto load_b = [&](int blk, bool ok, u32x4 (&dst)[8]) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const bool on = (NG == 2 && (t & 1)) ? on1 : on0;
            const uint32_t off = ok && on ? (uint32_t)(((blk * 8 + t) * kWave + lane) * (int)sizeof(u32x4)) : kOut;
            dst[t] = __builtin_amdgcn_raw_buffer_load_b128(ur, off, 0, 0);
        }
    };
    auto load_codes = [&](int c, bool ok, uint32_t (&dst)[BITS]) {
        qg_load<BITS>(rs, ok ? row_off + (uint32_t)((4 * c + q) * BITS) * 4u : kOut, dst);
    };
    // two register sets for the codes (and, NG = 1, the B operands): a chunk's loads are issued
    // into one set while the other is in use, with no copies between them
    uint32_t d0[BITS], d1[BITS];
    u32x4 b0[8], b1[8];
    int c = wave;
    load_codes(c, c < n_chunks, d0);
    load_b(c * NG, c < n_chunks, b0);
#pragma unroll
    for (int t = 0; t < kCbPer; ++t) {
        const int k = threadIdx.x + t * kThreads;
        const float x = __uint_as_float(cv[t][0]), y = __uint_as_float(cv[t][1]);
        const uint32_t x1 = f32_to_bf16_rne(x), y1 = f32_to_bf16_rne(y);
        const uint32_t x2 = f32_to_bf16_rne(x - __uint_as_float(x1 << 16));
        const uint32_t y2 = f32_to_bf16_rne(y - __uint_as_float(y1 << 16));
        if (K % kThreads == 0 || k < K) cb_l[k] = make_uint2(x1 | (y1 << 16), x2 | (y2 << 16));
    }
    __syncthreads();

    f32x4 acc[2 * NG];
#pragma unroll
    for (int t = 0; t < 2 * NG; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // one chunk: NG = 1, operands in b, the next chunk's loads into (dn, bn); NG = 2, the chunk's first
    // half in b0, its second half loaded into b1, the next chunk's first half into b0 once free
    auto chunk = [&](int cc, uint32_t (&d)[BITS], u32x4 (&b)[8], uint32_t (&dn)[BITS], u32x4 (&bn)[8]) {
        const bool more = cc + kQxWaves < n_chunks;
        if constexpr (NG == 1) {
            load_codes(cc + kQxWaves, more, dn);
            load_b(cc + kQxWaves, more, bn);
            __builtin_amdgcn_sched_barrier(0);
            qx_steps<BITS, 1, 0, 8, 0>(cb_l, d, b, acc);
        } else {
            load_b(2 * cc + 1, true, b1);
            load_codes(cc + kQxWaves, more, dn);
            __builtin_amdgcn_sched_barrier(0);
            qx_steps<BITS, 2, 0, 4, 0>(cb_l, d, b0, acc);
            __builtin_amdgcn_sched_barrier(0);
            load_b(2 * (cc + kQxWaves), more, b0);
            __builtin_amdgcn_sched_barrier(0);
            qx_steps<BITS, 2, 4, 4, 0>(cb_l, d, b1, acc);
        }
    };
    for (; c < n_chunks; c += 2 * kQxWaves) {
        chunk(c, d0, b0, d1, b1);
        if (c + kQxWaves >= n_chunks) break;
        chunk(c + kQxWaves, d1, b1, d0, b0);
    }
    // wavefront partials: D = (c1 + c2) u per group
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        f32x4 v = acc[2 * g];
        v[0] += acc[2 * g + 1][0];
        v[1] += acc[2 * g + 1][1];
        v[2] += acc[2 * g + 1][2];
        v[3] += acc[2 * g + 1][3];
        part[(wave * NG + g) * kWave + lane] = v;
    }
    __syncthreads();
    if (threadIdx.x < NG * kWave) {   // sum over the wavefronts in order; D[4 q + v][j] to dsum
        const int g = threadIdx.x / kWave;
        f32x4 sum = part[g * kWave + lane];
        for (int w = 1; w < kQxWaves; ++w) {
            const f32x4 p2 = part[(w * NG + g) * kWave + lane];
            sum[0] += p2[0];
            sum[1] += p2[1];
            sum[2] += p2[2];
            sum[3] += p2[3];
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) dsum[(g * 16 + 4 * q + v) * 16 + j] = sum[v];
    }
    __syncthreads();
    if (threadIdx.x < a.M * 16) {   // y[m][row0 + i] = f16(norm) * sum over the pieces p of column (m, p)
        const int m = threadIdx.x >> 4, i = threadIdx.x & 15;
        const int g = md.ng == 2 ? m >> 3 : 0, mm = md.ng == 2 ? m & 7 : m;
        const float* dr = dsum + (g * 16 + i) * 16 + md.np * mm;
        float yv = dr[0] + dr[1];
        if (md.np == 3) yv += dr[2];
        if (i < nrows) {
            yv *= __half2float(__ushort_as_half(a.norm[row0 + i]));
            if (a.y_bf16)
                reinterpret_cast<uint16_t*>(a.y)[(size_t)m * a.ld_y + row0 + i] = f32_to_bf16_rne(yv);
            else
                reinterpret_cast<float*>(a.y)[(size_t)m * a.ld_y + row0 + i] = yv;
        }
    }
}

// 9 to 16 activation rows: v_mfma_f32_32x32x16_bf16, D[32 x 32] += A[32 x 16] B[16 x 32], a tile of
// 32 weight rows, so that each B operand (the u pieces, 2 KB per 16 pairs at 16 rows) serves twice
// the weight rows of the 16-row layout.  Lane l = 32 q + j supplies A row j and B column j = 2 m + p
// for the k-slots of its 4 pairs of the step (pairs 64 c + 32 q + 4 s + (0..3) of a 64-pair chunk:
// lane (j, q) reads row j's codes for 32 pairs, BITS dwords, dword-aligned) and holds D[8 (v / 4) +
// 4 q + v % 4][j] (v = 0..15).  Otherwise as k_qgemm_mx with one operand group.
typedef float f32x16 __attribute__((ext_vector_type(16)));
size_t qx32_lds_bytes(int bits, int waves) {
    return (size_t)(1 << bits) * sizeof(uint2) + (size_t)waves * kWave * sizeof(f32x16) + 32 * 32 * sizeof(float);
}
__device__ __forceinline__ f32x16 qx_mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

template <int BITS, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(3)))
void k_qgemm_mx32(QgemmArgs a, int full, int tail_h) {
    extern __shared__ __align__(16) char smem[];
    constexpr int K = 1 << BITS;
    constexpr int kThreads = WAVES * kWave;
    constexpr uint32_t kOut = 0xFFFFF000u;
    uint2* cb_l = reinterpret_cast<uint2*>(smem);                                  // K x {c1, c2}
    f32x4* part = reinterpret_cast<f32x4*>(smem + (size_t)K * sizeof(uint2));     // waves x 64 lanes x 4
    float* dsum = reinterpret_cast<float*>(part + WAVES * kWave * 4);              // 32 x 32
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int j = lane & 31, q = lane >> 5;
    const int n_chunks = (a.n_pairs + 63) / 64;
    const int tile = blockIdx.x;
    const int row0 = tile < full ? tile * 32 : full * 32 + (tile - full) * tail_h;
    const int h = tile < full ? 32 : tail_h;
    const int nrows = a.d_out - row0 < h ? a.d_out - row0 : h;

    constexpr int kCbPer = (K + kThreads - 1) / kThreads;
    const __amdgpu_buffer_rsrc_t cbr =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.cb, (short)0, K * (int)sizeof(float2), 0x00020000);
    u32x2 cv[kCbPer];
#pragma unroll
    for (int t = 0; t < kCbPer; ++t)
        cv[t] = __builtin_amdgcn_raw_buffer_load_b64(cbr, (uint32_t)(threadIdx.x + t * kThreads) * 8u, 0, 0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.codes + (size_t)row0 * a.stride), (short)0, nrows * (int)a.stride, 0x00020000);
    const uint32_t row_off = (uint32_t)j * (uint32_t)a.stride;
    const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.u, (short)0, n_chunks * 8 * kWave * (int)sizeof(u32x4), 0x00020000);
    const bool on = j < 2 * a.M;   // B columns that carry data
    auto load_b = [&](int c, bool ok, u32x4 (&dst)[8]) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t off = ok && on ? (uint32_t)(((c * 8 + t) * kWave + lane) * (int)sizeof(u32x4)) : kOut;
            dst[t] = __builtin_amdgcn_raw_buffer_load_b128(ur, off, 0, 0);
        }
    };
    auto load_codes = [&](int c, bool ok, uint32_t (&dst)[BITS]) {
        qg_load<BITS>(rs, ok ? row_off + (uint32_t)((2 * c + q) * BITS) * 4u : kOut, dst);
    };
    uint32_t d0[BITS], d1[BITS];
    u32x4 b0[8], b1[8];
    int c = wave;
    load_codes(c, c < n_chunks, d0);
    load_b(c, c < n_chunks, b0);
#pragma unroll
    for (int t = 0; t < kCbPer; ++t) {
        const int k = threadIdx.x + t * kThreads;
        const float x = __uint_as_float(cv[t][0]), y = __uint_as_float(cv[t][1]);
        const uint32_t x1 = f32_to_bf16_rne(x), y1 = f32_to_bf16_rne(y);
        const uint32_t x2 = f32_to_bf16_rne(x - __uint_as_float(x1 << 16));
        const uint32_t y2 = f32_to_bf16_rne(y - __uint_as_float(y1 << 16));
        if (K % kThreads == 0 || k < K) cb_l[k] = make_uint2(x1 | (y1 << 16), x2 | (y2 << 16));
    }
    __syncthreads();

    f32x16 acc = {};   // c1 and c2 products into one accumulator (two would spill)
    auto chunk = [&](int cc, uint32_t (&d)[BITS], u32x4 (&b)[8], uint32_t (&dn)[BITS], u32x4 (&bn)[8]) {
        const bool more = cc + WAVES < n_chunks;
        load_codes(cc + WAVES, more, dn);
        load_b(cc + WAVES, more, bn);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 a1[2], a2[2];
        qx_gather<BITS>(cb_l, d, 0, a1[0], a2[0]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t + 1 < 8) qx_gather<BITS>(cb_l, d, t + 1, a1[(t + 1) & 1], a2[(t + 1) & 1]);
            acc = qx_mfma32(a1[t & 1], b[t], acc);
            acc = qx_mfma32(a2[t & 1], b[t], acc);
        }
    };
    for (; c < n_chunks; c += 2 * WAVES) {
        chunk(c, d0, b0, d1, b1);
        if (c + WAVES >= n_chunks) break;
        chunk(c + WAVES, d1, b1, d0, b0);
    }
    // wavefront partials D = (c1 + c2) u, then the sum over the wavefronts in order
#pragma unroll
    for (int v = 0; v < 4; ++v)
        part[(wave * kWave + lane) * 4 + v] = f32x4{acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]};
    __syncthreads();
    if (threadIdx.x < kWave) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            f32x4 sum = part[lane * 4 + v];
            for (int w = 1; w < WAVES; ++w) {
                const f32x4 p2 = part[(w * kWave + lane) * 4 + v];
                sum[0] += p2[0];
                sum[1] += p2[1];
                sum[2] += p2[2];
                sum[3] += p2[3];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) dsum[(8 * v + 4 * q + r) * 32 + j] = sum[r];
        }
    }
    __syncthreads();
    for (int o = threadIdx.x; o < a.M * 32; o += kThreads) {   // y[m][row0 + i] = f16(norm) (piece 0 + piece 1)
        const int m = o >> 5, i = o & 31;
        if (i < nrows) {
            const float yv = (dsum[i * 32 + 2 * m] + dsum[i * 32 + 2 * m + 1]) *
                             __half2float(__ushort_as_half(a.norm[row0 + i]));
            if (a.y_bf16)
                reinterpret_cast<uint16_t*>(a.y)[(size_t)m * a.ld_y + row0 + i] = f32_to_bf16_rne(yv);
            else
                reinterpret_cast<float*>(a.y)[(size_t)m * a.ld_y + row0 + i] = yv;
        }
    }
}

}  // namespace

size_t qgemm_workspace(int M, int d_out, int d_in) {   // the B operands of k_qgemm_mx
    const QxMode md = qx_mode(M, d_out);
    const int ch = qx_chunk(md);
    return (size_t)((d_in / 2 + ch - 1) / ch) * 8 * md.ng * kWave * sizeof(u32x4);
}

namespace {
// Tiles of at most T rows over the compute units: whole rounds of T-row tiles, then one round of
// shorter tiles for the rows left over, so that no unit takes two full tiles while others take
// one; fewer rows than one round fills are spread over a round of shorter tiles.
struct QxTiling {
    int full, tail_h, n_wg;
};
QxTiling qx_tiling(int d_out, int T) {
    QxTiling t{0, 1, 0};
    const int rounds = d_out / (kComputeUnits * T);
    t.full = rounds * kComputeUnits;
    const int rest = d_out - t.full * T;
    t.tail_h = (rest + kComputeUnits - 1) / kComputeUnits;
    if (t.tail_h < 1) t.tail_h = 1;
    t.n_wg = t.full + (rest + t.tail_h - 1) / t.tail_h;
    return t;
}

template <int BITS, int NG, int WAVES>
hipError_t qgemm_mx_launch(const QgemmArgs& a, hipStream_t st) {
    const size_t smem = qx_lds_bytes(BITS, NG, WAVES);
    allow_lds(k_qgemm_mx<BITS, NG, WAVES>, smem);
    const QxTiling t = qx_tiling(a.d_out, 16);
    hipLaunchKernelGGL((k_qgemm_mx<BITS, NG, WAVES>), dim3(t.n_wg), dim3(WAVES * kWave), smem, st, a, t.full,
                       t.tail_h);
    return hipGetLastError();
}

template <int BITS, int WAVES>
hipError_t qgemm_mx32_launch(const QgemmArgs& a, hipStream_t st) {
    const size_t smem = qx32_lds_bytes(BITS, WAVES);
    allow_lds(k_qgemm_mx32<BITS, WAVES>, smem);
    const QxTiling t = qx_tiling(a.d_out, 32);
    hipLaunchKernelGGL((k_qgemm_mx32<BITS, WAVES>), dim3(t.n_wg), dim3(WAVES * kWave), smem, st, a, t.full, t.tail_h);
    return hipGetLastError();
}

template <int BITS>
hipError_t qgemm_mx_B(const QgemmArgs& a, hipStream_t st) {
    const QxMode md = qx_mode(a.M, a.d_out);
    if (md.w32) {
        const bool wide32 = (a.n_pairs + 63) / 64 >= 2 * kQxLongRow;
        return wide32 ? qgemm_mx32_launch<BITS, 8>(a, st) : qgemm_mx32_launch<BITS, 4>(a, st);
    }
    const bool two = md.ng == 2, wide = (a.n_pairs + 127) / 128 >= kQxLongRow;
    if (two) return wide ? qgemm_mx_launch<BITS, 2, 8>(a, st) : qgemm_mx_launch<BITS, 2, 4>(a, st);
    return wide ? qgemm_mx_launch<BITS, 1, 8>(a, st) : qgemm_mx_launch<BITS, 1, 4>(a, st);
}

}  // namespace

hipError_t launch_qgemm(const QgemmArgs& a, const QgemmRotateArgs& r, hipStream_t st) {
    const QxMode md = qx_mode(a.M, a.d_out);
    const int ch = qx_chunk(md);
    const int cols = (r.d_in / 2 + ch - 1) / ch * ch * 2;   // whole chunks
    const int T = r.block / 2 > 256 ? r.block / 2 : 256;   // threads: pairs per workgroup
    hipLaunchKernelGGL(k_qgemm_rotate_mx, dim3((cols / 2 + T - 1) / T, a.M), dim3(T), 0, st, r.x, r.x_bf16, r.ld_x, md,
                       r.d_in, cols, r.block, r.scale, r.sign_seed, r.sigma, reinterpret_cast<uint32_t*>(a.u));
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
#define QAMW_QX(b) \
    case b: return qgemm_mx_B<b>(a, st);
    switch (a.bits) {
        QAMW_QX(1) QAMW_QX(2) QAMW_QX(3) QAMW_QX(4) QAMW_QX(5) QAMW_QX(6)
        QAMW_QX(7) QAMW_QX(8) QAMW_QX(9) QAMW_QX(10) QAMW_QX(11) QAMW_QX(12)
    default: return hipErrorInvalidValue;
    }
#undef QAMW_QX
}

}  // namespace qamw
