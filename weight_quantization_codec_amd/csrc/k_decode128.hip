// QAM-W decoder for Hadamard blocks of 128 columns (paper section 3.2; section 1: the weights
// are dequantized to BF16 before the matrix product).  Block 128 is the block of the attention,
// 13B-layer and 40-layer workloads; other block sizes use k_decode (k_decode.hip).
//
// Work split.  A workgroup owns a span of NBW consecutive 128-column blocks and walks tiles of
// R = 16 / NBW rows, one tile per wavefront at a time: lane = (slot, q), slot = lane & 15 picks
// (row rr = slot / NBW, block bb = slot % NBW) of the tile, q = lane >> 4 the quarter of the
// block.  A lane's columns never change, so eps_j / s_j and sigma_k are set up once per
// workgroup (a few columns and pairs per thread) and handed out through LDS.
//
// Transform (all in double).  The lane starts with elements 32 q + m (m = 0..31) of its row's
// block: element bits 0-4 in register bits 0-4, element bits 5-6 in lane bits 4-5.
//   stage 0      folded into the LDS table (c_x + c_y, c_x - c_y)
//   stage 1      with the pair scaling sigma_k f16(norm) / sqrt(128): per two pairs, two products
//                and four fused multiply-adds
//   stages 2-4   register butterflies
//   element bit 5 <-> register bit 4 by v_permlane16_swap (lane bit 4), then stage 5
//   element bit 6 <-> register bit 3 by v_permlane32_swap (lane bit 5), then stage 6
// The lane then holds element bits 0-2 in register bits 0-2 (bits 3 and 4 of the element are
// lane bits 5 and 4, bits 5 and 6 register bits 4 and 3): eight consecutive columns per group
// of eight registers.
//
// Output.  The tile goes through the wavefront's LDS staging area so that every store
// instruction writes whole 128-byte lines (1 KB of one row when NBW = 4): stores of 64-byte
// pieces cost HBM write efficiency (measured: about 3.3 against 5.4 TB/s for the same traffic).
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include "qamw_device.hpp"
#include "qamw_launch.hpp"

namespace qamw {

namespace {

// Two launch shapes.  4 wavefronts per workgroup with sigma_k in registers (158-164 VGPRs, three
// wavefronts per SIMD, three workgroups per CU): the matrices of the 13B shapes and grouped
// launches.  8 wavefronts with sigma_k in LDS (at most 128 VGPRs, four per SIMD, two workgroups
// per CU): a lone small matrix, where more wavefronts with fewer tiles each overlap better.
template <int W>
struct D128Shape {
    static constexpr int waves = W;
    static constexpr int threads = kWave * W;
    static constexpr bool sg_lds = W == 8;
    static constexpr int wg_per_cu = W == 8 ? 2 : 3;
};
constexpr bool kD128CfLds = true;   // eps_j / s_j from LDS (frees 32 registers per lane)


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) const double lds_double;

// Cache policy of the output stores: non-temporal (the decoded matrix is written once).
constexpr int kStoreNT128 = 2;

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Exchange between lanes l and l ^ 16 (bit 4 = 0: keeps a, receives the partner's a into b;
// bit 4 = 1: keeps b, receives the partner's b into a), and the same between l and l ^ 32.
__device__ __forceinline__ void swap_lanes16(double& a, double& b) {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)__double2loint(a), (uint32_t)__double2loint(b), false,
                                                     false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)__double2hiint(a), (uint32_t)__double2hiint(b), false,
                                                     false);
    a = __hiloint2double((int)hi[0], (int)lo[0]);
    b = __hiloint2double((int)hi[1], (int)lo[1]);
}
__device__ __forceinline__ void swap_lanes32(double& a, double& b) {
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)__double2loint(a), (uint32_t)__double2loint(b), false,
                                                     false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)__double2hiint(a), (uint32_t)__double2hiint(b), false,
                                                     false);
    a = __hiloint2double((int)hi[0], (int)lo[0]);
    b = __hiloint2double((int)hi[1], (int)lo[1]);
}

// Dwords holding a lane's 16 fields of BITS bits: its first field starts at bit 16 q BITS of
// the block, i.e. at bit 16 (q BITS mod 2) of its first dword.
template <int BITS>
struct Lane128 {
    static constexpr int ND = (BITS & 1) ? (BITS + 1) / 2 : BITS / 2;   // dwords loaded
    static constexpr int NA = (16 * BITS + 31) / 32;                     // dwords once aligned
};

// N consecutive dwords at byte offset off of a buffer; dwords past the descriptor's range read 0.
template <int N>
__device__ __forceinline__ void load_dw(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t (&d)[N]) {
#pragma unroll
    for (int c = 0; c + 4 <= N; c += 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 4 * c, 0, 0);
        d[c] = v[0];
        d[c + 1] = v[1];
        d[c + 2] = v[2];
        d[c + 3] = v[3];
    }
    constexpr int c = N / 4 * 4;
    if constexpr (N - c >= 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 4 * c, 0, 0);
        d[c] = v[0];
        d[c + 1] = v[1];
    }
    if constexpr (N - c == 3) d[c + 2] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * c + 8, 0, 0);
    if constexpr (N - c == 1) d[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * c, 0, 0);
}

// LDS byte offsets (x 16: the table's entries are 16 bytes) of the lane's 16 codewords.
template <int BITS>
__device__ __forceinline__ void unpack128(const uint32_t (&dw)[Lane128<BITS>::ND], uint32_t s0, uint32_t (&addr)[16]) {
    constexpr int ND = Lane128<BITS>::ND, NA = Lane128<BITS>::NA;
    uint32_t al[NA];
#pragma unroll
    for (int t = 0; t < NA; ++t) al[t] = __builtin_amdgcn_alignbit(t + 1 < ND ? dw[t + 1] : 0u, dw[t], s0);
    constexpr uint32_t mask = ((1u << BITS) - 1u) << 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int off = i * BITS, w = off >> 5, sh = off & 31;
        uint32_t v;
        if (sh >= 4)
            v = __builtin_amdgcn_alignbit(w + 1 < NA ? al[w + 1] : 0u, al[w], sh - 4);
        else if (w > 0)
            v = __builtin_amdgcn_alignbit(al[w], al[w - 1], 28 + sh);
        else
            v = al[0] << (4 - sh);
        addr[i] = v & mask;
    }
}

// LDS of a workgroup beyond the codebook table (bytes):
//   cf    eps_j / s_j (fp32) of the span's 128 NBW columns   (kept when CF_LDS, else set-up only)
//   sg    sigma_k / sqrt(128) (double) of its 64 NBW pairs  (kept when SG_LDS, else set-up only)
//   stage per wavefront, one tile: R rows x NBW blocks x 128 columns, each block padded by 16 bytes
template <int NBW, bool OBF, bool CF_LDS, bool SG_LDS, int WAVES>
struct Smem128 {
    static constexpr int R = 16 / NBW;
    static constexpr int ESZ = OBF ? 2 : 4;
    static constexpr int BLKP = 128 * ESZ + 16;          // bytes per staged block (padded)
    static constexpr int ROWP = NBW * BLKP;              // bytes per staged row
    static constexpr int STAGE = R * ROWP;               // bytes per wavefront
    static constexpr int CF = 128 * NBW * 4;
    static constexpr int SG = 64 * NBW * 8;
    static constexpr int setup = CF + SG;
    static constexpr int keep = SG_LDS ? CF + SG : (CF_LDS ? CF : 0);   // persists past the set-up
    static constexpr int body = keep + WAVES * STAGE;
    static constexpr int bytes = setup > body ? setup : body;
};

// A launch decodes b.n matrices; matrix m owns workgroups b.it[m].wg0 .. + n_wg - 1.  Within it a
// workgroup w takes the NBW-block span (w / 8) % n_span and the tile groups listed below, wavefront
// v of the workgroup taking tile 4 group + v.
template <int BITS, bool OBF, int NBW, bool CF_LDS, bool SG_LDS, int NI, int L, int WAVES>
__global__ __launch_bounds__(kWave * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES == 8 ? 4 : 3)))
void k_decode128(const Decode128Batch<NI> b) {
    static_assert(L == 7 || (L == 8 && NBW >= 2), "blocks of 256 columns are two 128-column blocks of one span");
    int m = 0;
    if constexpr (NI > 1) {
        for (int i = 1; i < b.n; ++i) m = (int)blockIdx.x >= b.it[i].wg0 ? i : m;
    }
    const Decode128Item& a = b.it[m];
    using SM = Smem128<NBW, OBF, CF_LDS, SG_LDS, WAVES>;
    constexpr int R = SM::R, ESZ = SM::ESZ;
    constexpr int K = 1 << BITS;
    extern __shared__ __align__(16) char smem[];
    double2* tab = reinterpret_cast<double2*>(smem);
    char* area = smem + (size_t)K * sizeof(double2);
    float* cf_l = reinterpret_cast<float*>(area);
    double* sg_l = reinterpret_cast<double*>(area + SM::CF);
    const int wave_in = threadIdx.x / kWave;
    char* stage = area + SM::keep + wave_in * SM::STAGE;
    const int lane = threadIdx.x & (kWave - 1);
    // Workgroups are dealt to the eight XCDs round-robin (blockIdx % 8).  The spans of one group of
    // tiles go to one XCD, so the code lines that two neighbouring spans share hit the same L2.
    const int n_span = a.nb / NBW;
    const int wg = (int)blockIdx.x - a.wg0, xcd = wg & 7, j = wg >> 3;   // wg0 is a multiple of 8
    const int span = j % n_span;
    const int group = (j / n_span) * 8 + xcd;
    const int col0 = 128 * NBW * span;   // first column of the span

    const int slot = lane & 15, q = lane >> 4;
    const int rr = slot / NBW, bb = slot % NBW;
    const int l4 = q & 1, l5 = q >> 1;

    // ---- this lane's codes: bits 16 q BITS .. of block span * NBW + bb of its row.  Codes, norms
    // and output go through buffer descriptors covering exactly their d_out rows: a row past the
    // end reads zeros and its stores are dropped, and every offset advances by a constant per pass.
    constexpr int ND = Lane128<BITS>::ND;
    const uint32_t s0 = (uint32_t)(16 * (q * BITS & 1));
    const int n_tiles = (a.d_out + R - 1) / R;
    const int n_groups_launched = a.n_wg / n_span;   // a multiple of 8
    int tile = WAVES * group + wave_in;
    const uint32_t tile_step = (uint32_t)(WAVES * n_groups_launched);
    const __amdgpu_buffer_rsrc_t crs =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.codes, (short)0, (int)((size_t)a.d_out * a.stride), 0x00020000);
    const __amdgpu_buffer_rsrc_t nrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.norm, (short)0, a.d_out * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        a.out, (short)0, (int)((size_t)a.d_out * (size_t)a.ld * ESZ), 0x00020000);
    const uint32_t row0 = (uint32_t)(R * tile + rr);
    uint32_t c_off = row0 * (uint32_t)a.stride + (uint32_t)((NBW * span + bb) * (8 * BITS) + 4 * ((q * BITS) >> 1));
    uint32_t n_off = row0 * 2u;
    const uint32_t c_step = (uint32_t)R * tile_step * (uint32_t)a.stride, n_step = (uint32_t)R * tile_step * 2u;
    // Two code buffers in turn: the next tile's codes and norm are loaded while this tile is
    // transformed, and no copy between the buffers (which would wait for the loads to land ahead
    // of this tile's stores, and so for the previous tile's stores too) is needed.  The first
    // tile's are requested before the set-up, whose latency they share.
    uint32_t dwA[ND], dwB[ND];
    uint32_t nhA, nhB;
    load_dw<ND>(crs, c_off, dwA);
    nhA = __builtin_amdgcn_raw_buffer_load_b16(nrs, n_off, 0, 0);

    // ---- set-up: codebook table (stage 0), eps_j / s_j of the span's columns, sigma of its pairs.
    // Fixed trip counts: every thread's loads are in flight at once.
    {
        constexpr int T = kWave * WAVES;
        constexpr int NE = (K + T - 1) / T, NC = (128 * NBW + T - 1) / T, NS = (64 * NBW + T - 1) / T;
        const int t = (int)threadIdx.x;
        // without a scale the descriptor has no records and its loads read 0
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)a.scale, (short)0, a.scale ? (int)((col0 + 128 * NBW) * 4) : 0, 0x00020000);
        const bool has_scale = a.scale != nullptr;
        float2 c[NE];
        uint32_t sv[NC];
        float sgv[NS];
#pragma unroll
        for (int e = 0; e < NE; ++e)
            if (K % T == 0 || e * T + t < K) c[e] = reinterpret_cast<const float2*>(b.cb)[e * T + t];
#pragma unroll
        for (int e = 0; e < NC; ++e)
            sv[e] = __builtin_amdgcn_raw_buffer_load_b32(srs, (uint32_t)(col0 + e * T + t) * 4u, 0, 0);
#pragma unroll
        for (int e = 0; e < NS; ++e)
            if ((64 * NBW) % T == 0 || e * T + t < 64 * NBW) sgv[e] = a.sigma[col0 / 2 + e * T + t];
#pragma unroll
        for (int e = 0; e < NE; ++e)
            if (K % T == 0 || e * T + t < K)
                tab[e * T + t] = make_double2((double)c[e].x + (double)c[e].y, (double)c[e].x - (double)c[e].y);
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            const int j = e * T + t;
            if ((128 * NBW) % T == 0 || j < 128 * NBW) {
                double v = has_scale ? 1.0 / (double)__uint_as_float(sv[e]) : 1.0;
                if (eps_negative(a.sign_seed, (uint32_t)(col0 + j))) v = -v;
                cf_l[j] = (float)v;
            }
        }
#pragma unroll
        for (int e = 0; e < NS; ++e)
            if ((64 * NBW) % T == 0 || e * T + t < 64 * NBW)
                sg_l[e * T + t] = (double)sgv[e] * (L == 7 ? 0.088388347648318440550 : 0.0625);   // sigma_k / sqrt(b)
    }
    __syncthreads();
    // phase-A pairs of the lane: 16 q + i of block bb
    const double* sg_lane = sg_l + 64 * bb + 16 * q;
    double sg[SG_LDS ? 1 : 16];
    if constexpr (!SG_LDS) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sg[i] = sg_lane[i];
#pragma unroll
        for (int i = 0; i < 16; ++i) pin_reg(sg[i]);
    }
    // final-layout columns of the lane, register r: element (r & 7) + 8 l5 + 16 l4 + 32 (r >> 4 & 1)
    // + 64 (r >> 3 & 1) of block bb; run u = r >> 3 starts at cf_run(u)
    const int cf_lane = 128 * bb + 8 * l5 + 16 * l4;
    float cf[CF_LDS ? 1 : 32];
    if constexpr (!CF_LDS) {
#pragma unroll
        for (int r = 0; r < 32; ++r) cf[r] = cf_l[cf_lane + (r & 7) + 32 * ((r >> 4) & 1) + 64 * ((r >> 3) & 1)];
#pragma unroll
        for (int r = 0; r < 32; ++r) pin_reg(cf[r]);
    }
    __syncthreads();   // the set-up area becomes staging space

    // staging: writes of run u of this lane; store pieces p = 64 k + lane of the tile, row p / PPR
    constexpr int PPR = NBW * 128 * ESZ / 16;     // 16-byte pieces per tile row
    constexpr int NST = R * PPR / kWave;          // store instructions per tile
    constexpr int PPB = 128 * ESZ / 16;           // pieces per block
    char* const wr = stage + rr * SM::ROWP + bb * SM::BLKP + (8 * l5 + 16 * l4) * ESZ;
    const uint32_t ldE = (uint32_t)a.ld * ESZ;
    uint32_t o_off = (uint32_t)(R * tile) * ldE + (uint32_t)col0 * ESZ +
                     (uint32_t)(lane / PPR) * ldE + (uint32_t)(lane % PPR) * 16u;   // piece 0 of this lane
    const uint32_t o_step = (uint32_t)R * tile_step * ldE;
    auto do_tile = [&](const uint32_t (&dw)[ND], const uint32_t nhv) {
        const uint16_t nh = (uint16_t)nhv;
        uint32_t addr[16];
        unpack128<BITS>(dw, s0, addr);
        // the 16 table reads in flight together (the table sits at LDS address 0), then one wait
        double2 t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const lds_double* ent = reinterpret_cast<const lds_double*>((size_t)addr[i]);
            t[i].x = ent[0];
            t[i].y = ent[1];
        }
        __builtin_amdgcn_sched_barrier(0);
        const double g = (double)__half2float(__ushort_as_half(nh));
        double x[32];
        // stages 0 (table) and 1 with the pair scaling
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            double si, sj;
            if constexpr (SG_LDS) {
                const double2 v = *reinterpret_cast<const double2*>(sg_lane + i);
                si = v.x * g;
                sj = v.y * g;
            } else {
                si = sg[i] * g;
                sj = sg[i + 1] * g;
            }
            const double pT = t[i + 1].x * sj, pD = t[i + 1].y * sj;
            x[2 * i] = __builtin_fma(t[i].x, si, pT);
            x[2 * i + 2] = __builtin_fma(t[i].x, si, -pT);
            x[2 * i + 1] = __builtin_fma(t[i].y, si, pD);
            x[2 * i + 3] = __builtin_fma(t[i].y, si, -pD);
        }
        butterfly<32>(x, 2);
        butterfly<32>(x, 3);
        butterfly<32>(x, 4);
#pragma unroll
        for (int j = 0; j < 16; ++j) swap_lanes16(x[j], x[j + 16]);   // register bit 4 <- element bit 5
        butterfly<32>(x, 4);                                          // stage 5
#pragma unroll
        for (int j = 0; j < 32; ++j)
            if (!(j & 8)) swap_lanes32(x[j], x[j + 8]);               // register bit 3 <- element bit 6
        butterfly<32>(x, 3);                                          // stage 6
        if constexpr (L == 8) {
            // b = 256: the two 128-column halves of the block are blocks bb and bb ^ 1 of the span, in
            // lanes l and l ^ 1 with the same element positions: the last stage (element bit 7) adds
            // the partner's element (lower half) or subtracts this lane's from it (upper half)
            const double sgn = (bb & 1) ? -1.0 : 1.0;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const int lo = __builtin_amdgcn_update_dpp(0, (int)__double2loint(x[j]), 0xB1, 0xF, 0xF, false);
                const int hi = __builtin_amdgcn_update_dpp(0, (int)__double2hiint(x[j]), 0xB1, 0xF, 0xF, false);
                x[j] = __builtin_fma(x[j], sgn, __hiloint2double(hi, lo));   // quad_perm [1,0,3,2]: lane ^ 1
            }
        }
        // eps_j / s_j, fp32 rounding, output type; staged run by run.  fma(x, c, +0) is x c rounded
        // once, except that a zero product is +0: a zero row (norm 0) decodes to +0.
        f32x4 cfv[CF_LDS ? 8 : 1];
        if constexpr (CF_LDS) {   // all eight reads in flight before the first use
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e0 = 32 * (u >> 1) + 64 * (u & 1);
                cfv[2 * u] = *reinterpret_cast<const f32x4*>(cf_l + cf_lane + e0);
                cfv[2 * u + 1] = *reinterpret_cast<const f32x4*>(cf_l + cf_lane + e0 + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e0 = 32 * (u >> 1) + 64 * (u & 1);   // the run's first element offset
            float f[8];
            if constexpr (CF_LDS) {
#pragma unroll
                for (int v = 0; v < 8; ++v) f[v] = __builtin_fmaf((float)x[8 * u + v], cfv[2 * u + v / 4][v % 4], 0.0f);
            } else {
#pragma unroll
                for (int v = 0; v < 8; ++v) f[v] = __builtin_fmaf((float)x[8 * u + v], cf[8 * u + v], 0.0f);
            }
            if constexpr (OBF) {
                const u32x4 o = {pk_bf16(f[0], f[1]), pk_bf16(f[2], f[3]), pk_bf16(f[4], f[5]), pk_bf16(f[6], f[7])};
                *reinterpret_cast<u32x4*>(wr + e0 * ESZ) = o;
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4 o = {__float_as_uint(f[4 * h]), __float_as_uint(f[4 * h + 1]),
                                     __float_as_uint(f[4 * h + 2]), __float_as_uint(f[4 * h + 3])};
                    *reinterpret_cast<u32x4*>(wr + e0 * ESZ + 16 * h) = o;
                }
            }
        }
        wave_lds_sync();
        // whole lines out: piece p = 64 k + lane of the tile is row p / PPR, byte 16 (p % PPR) of the
        // span (PPR divides 64 or 64 divides PPR: the row's lane part is in o_off, its k part k_off)
#pragma unroll
        for (int k = 0; k < NST; ++k) {
            const int p = k * kWave + lane;
            const int prow = p / PPR, o = p % PPR;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + prow * SM::ROWP + (o / PPB) * SM::BLKP +
                                                             16 * (o % PPB));
            const uint32_t k_off = (uint32_t)((k * kWave) / PPR) * ldE + (uint32_t)((k * kWave) % PPR) * 16u;
            // the whole offset in the VGPR: the descriptor's range check then covers the row
            __builtin_amdgcn_raw_buffer_store_b128(v, ors, o_off + k_off, 0, kStoreNT128);
        }
        o_off += o_step;
        wave_lds_sync();   // the staging area is rewritten by the next tile
    };
    auto next = [&](uint32_t (&dw)[ND], uint32_t& nhv) {
        c_off += c_step;
        n_off += n_step;
        load_dw<ND>(crs, c_off, dw);
        nhv = __builtin_amdgcn_raw_buffer_load_b16(nrs, n_off, 0, 0);
    };
    if (tile >= n_tiles) return;
    // The first tile is peeled: the loop is entered, as it is repeated, with one tile's codes in
    // flight behind the previous tile's stores, so its wait counts need not cover those stores.
    next(dwB, nhB);
    do_tile(dwA, nhA);
    for (tile += (int)tile_step; tile < n_tiles; tile += (int)tile_step) {
        next(dwA, nhA);
        do_tile(dwB, nhB);
        tile += (int)tile_step;
        if (tile >= n_tiles) break;
        next(dwB, nhB);
        do_tile(dwA, nhA);
    }
}

template <int BITS, bool OBF, int NBW, int NI, int L, int W>
hipError_t launch128(const Decode128Batch<NI>& bt, int n_wg, hipStream_t st) {
    using S = D128Shape<W>;
    auto kern = k_decode128<BITS, OBF, NBW, kD128CfLds, S::sg_lds, NI, L, W>;
    const size_t smem = ((size_t)1 << BITS) * 16 + Smem128<NBW, OBF, kD128CfLds, S::sg_lds, W>::bytes;
    allow_lds(kern, smem);
    hipLaunchKernelGGL(kern, dim3(n_wg), dim3(S::threads), smem, st, bt);
    return hipGetLastError();
}

template <int NI, int WV, bool OBF>
hipError_t dispatch128_o(const Decode128Batch<NI>& bt, int bits, int nbw, int L, int n_wg, hipStream_t st) {
#define QAMW_D128_CASE(B, W, LL) \
    if (bits == B && nbw == W && L == LL) return launch128<B, OBF, W, NI, LL, WV>(bt, n_wg, st);
    QAMW_D128_CASE(7, 1, 7) QAMW_D128_CASE(7, 2, 7) QAMW_D128_CASE(7, 4, 7)
    QAMW_D128_CASE(8, 1, 7) QAMW_D128_CASE(8, 2, 7) QAMW_D128_CASE(8, 4, 7)
    QAMW_D128_CASE(11, 1, 7) QAMW_D128_CASE(11, 2, 7) QAMW_D128_CASE(11, 4, 7)
    if constexpr (WV == 4 && OBF) {   // 256-column blocks: BF16 out, 4 wavefronts (the rest spill)
        QAMW_D128_CASE(7, 2, 8) QAMW_D128_CASE(7, 4, 8)
        QAMW_D128_CASE(8, 2, 8) QAMW_D128_CASE(8, 4, 8)
        QAMW_D128_CASE(11, 2, 8) QAMW_D128_CASE(11, 4, 8)
    }
#undef QAMW_D128_CASE
    return hipErrorInvalidValue;
}

template <int NI, int WV>
hipError_t dispatch128(const Decode128Batch<NI>& bt, int bits, int nbw, int L, bool obf, int n_wg, hipStream_t st) {
    if constexpr (WV == 8) {   // BF16 output only (fp32 output spills at 8 wavefronts)
        return obf ? dispatch128_o<NI, 8, true>(bt, bits, nbw, L, n_wg, st) : hipErrorInvalidValue;
    } else {
        return obf ? dispatch128_o<NI, 4, true>(bt, bits, nbw, L, n_wg, st)
                   : dispatch128_o<NI, 4, false>(bt, bits, nbw, L, n_wg, st);
    }
}

// span width in 128-column blocks: 4 (1 KB of BF16 per row per store instruction) when the row
// allows; at least 2 for 256-column Hadamard blocks (nb is even there)
int span_blocks(int nb) { return nb % 4 == 0 ? 4 : (nb % 2 == 0 ? 2 : 1); }

// The matrix's descriptor and workgroup count (a multiple of 8: one per XCD for every tile group).
Decode128Item make_item(const DecodeArgs& d, int wg0, int waves) {
    Decode128Item it{};
    it.codes = d.codes;
    it.norm = d.norm;
    it.sigma = d.sigma;
    it.scale = d.scale;
    it.out = d.out;
    it.sign_seed = d.sign_seed;
    it.stride = (uint32_t)d.stride;
    it.d_out = d.d_out;
    it.ld = (uint32_t)d.ld;
    it.nb = d.d_in / 128;
    const int nbw = span_blocks(it.nb);
    const int R = 16 / nbw;
    const int n_span = it.nb / nbw;
    const int n_tiles = (d.d_out + R - 1) / R;
    const int n_groups = (n_tiles + waves - 1) / waves;   // a tile per wavefront
    // about 12 (4 wavefronts per workgroup) or 16 (8) wavefronts per CU are resident: aim at that
    // many workgroups, the tiles spread evenly over them; groups per span in multiples of 8 (one
    // per XCD)
    int per_span = 256 * (waves == 8 ? D128Shape<8>::wg_per_cu : D128Shape<4>::wg_per_cu) / n_span;
    if (per_span < 8) per_span = 8;
    if (per_span > n_groups) per_span = n_groups;
    const int iters = (n_groups + per_span - 1) / per_span;
    per_span = (n_groups + iters - 1) / iters;
    per_span = (per_span + 7) / 8 * 8;
    it.wg0 = wg0;
    it.n_wg = n_tiles == 0 ? 0 : n_span * per_span;
    return it;
}

}  // namespace

bool decode128_supported(const DecodeArgs& d, int L) {
    // buffer offsets are 32-bit: codes and output below 2 GiB
    const size_t esz = d.out_bf16 ? 2 : 4;
    // b = 256 with fp32 output goes to k_decode (this kernel would spill there)
    return (L == 7 || (L == 8 && d.out_bf16)) && (d.bits == 7 || d.bits == 8 || d.bits == 11) &&
           d.d_in % (1 << L) == 0 &&
           (size_t)d.d_out * d.stride < ((size_t)1 << 31) && (size_t)d.d_out * (size_t)d.ld * esz < ((size_t)1 << 31);
}

hipError_t launch_decode128(const DecodeArgs& d, int L, hipStream_t st) {
    Decode128Batch<1> bt{};
    bt.cb = d.cb;
    bt.n = 1;
    // the 8-wavefront shape when it gives each workgroup at most two tile groups (a small matrix)
    const Decode128Item i8 = make_item(d, 0, 8);
    const int n_span = i8.nb / span_blocks(i8.nb);
    const int R = 16 / span_blocks(i8.nb);
    const int groups8 = ((d.d_out + R - 1) / R + 7) / 8;
    const bool small = L == 7 && d.out_bf16 && i8.n_wg > 0 && (groups8 + i8.n_wg / n_span - 1) / (i8.n_wg / n_span) <= 2;
    bt.it[0] = small ? i8 : make_item(d, 0, 4);
    if (bt.it[0].n_wg == 0) return hipSuccess;
    const int nbw = span_blocks(bt.it[0].nb);
    return small ? dispatch128<1, 8>(bt, d.bits, nbw, L, d.out_bf16 != 0, bt.it[0].n_wg, st)
                 : dispatch128<1, 4>(bt, d.bits, nbw, L, d.out_bf16 != 0, bt.it[0].n_wg, st);
}

hipError_t launch_decode128_many(const DecodeArgs* d, const int* L, int n, hipStream_t st) {
    // consecutive matrices of one span width and block size share a launch, at most kDecodeBatch
    Decode128Batch<kDecodeBatch> bt{};
    int i = 0;
    while (i < n) {
        const int nbw = span_blocks(d[i].d_in / 128), li = L[i];
        bt.cb = d[i].cb;
        bt.n = 0;
        int wg = 0;
        for (; i < n && bt.n < kDecodeBatch && span_blocks(d[i].d_in / 128) == nbw && L[i] == li; ++i) {
            const Decode128Item it = make_item(d[i], wg, 4);
            if (it.n_wg == 0) continue;
            bt.it[bt.n++] = it;
            wg += it.n_wg;
        }
        if (bt.n == 0) continue;
        const hipError_t e = dispatch128<kDecodeBatch, 4>(bt, d[0].bits, nbw, li, d[0].out_bf16 != 0, wg, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qamw
