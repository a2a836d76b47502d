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

// A buffer offset past the byte range of every buffer descriptor the library builds (those cover
// fewer than 2^31 bytes), with room for small offsets to be added without wrapping: loads through
// it return 0 and stores are dropped.
constexpr uint32_t kNoByte = 0x80000000u;

// Search-index layout (bytes from the start of the index buffer written by qamw_codebook_index).
constexpr int kIndexFine = 2048;                          // W: fine bins per axis
constexpr int kIndexFineMax = 2048;
constexpr int kIndexGMax = 128;                           // cells per axis, at most
constexpr int kIndexCellCap = 64;                         // longer lists: cell searched exhaustively
constexpr int kIndexListPad = kIndexCellCap + 8;          // LDS entries after the lists (over-reads)
constexpr int kIndexMaxEntries = 40960;                   // candidate-list capacity (u16 entries)
constexpr int kIndexHeaderBytes = 256;
constexpr int kIndexFineOff = 256;                                    // u8[W]      fine bin -> cell
constexpr int kIndexEdgeOff = kIndexFineOff + kIndexFine;             // u16[G+1]   first fine bin of each cell
constexpr int kIndexOvfOff = kIndexEdgeOff + 512;                     // u8[G*G]    overflow flags
constexpr int kIndexOrderOff = kIndexOvfOff + kIndexGMax * kIndexGMax; // u16[K]     codewords by decreasing norm
constexpr int kIndexOffsOff = kIndexOrderOff + 8192;                  // u32[G*G+1] list offsets
constexpr int kIndexEntOff = kIndexOffsOff + 4 * kIndexGMax * kIndexGMax + 256;   // u16[] candidate lists

struct IndexHeader {
    int32_t K;
    int32_t G;        // grid is G x G cells over [-R, R]^2
    int32_t W;        // fine bins per axis
    int32_t bits;
    float R;
    float inv_w;      // W / (2R)
    int32_t n_entries;
    int32_t overflow; // cells searched exhaustively
};

// Candidate-list entries kept in LDS for a K-entry codebook.  With G = 2.12 sqrt(K) cells per
// axis a Gaussian-trained codebook lists about 11.5 K entries (2.5 per point on average);
// K = 4096 uses a coarser grid (G = 64, about 5 K entries) to stay within LDS.  A codebook that
// needs more gets exhaustive cells instead (at the far end of the grid's scan order).
__host__ __device__ constexpr int index_lds_entries(int K) {
    return K >= 4096 ? 22528 : (12 * K < 64 ? 64 : 12 * K);
}

__host__ __device__ constexpr size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

// An index buffer fits the codebook size it is used with: built for K codewords on a G x G grid
// (G as the host computes it for that K), so the LDS image the kernels size and fill matches.
__host__ __device__ inline bool index_header_ok(const IndexHeader& ih, int K, int G) {
    return ih.K == K && ih.G == G && ih.W == kIndexFine && ih.n_entries >= 0;
}

// LDS image of the codebook and its index used by the search.
struct SearchLds {
    float2* cb;
    uint32_t cb_lds;   // LDS byte address of cb (the lists hold cb_lds + 8 j)
    const uint16_t* order;   // codewords by decreasing norm (global memory: exterior points only)
    uint8_t* fine;
    uint16_t* offs;
    uint16_t* ent;     // candidate lists: LDS byte addresses cb_lds + 8 j of the codewords
    float R, inv_w;
    int W, G, K;
};

// The candidate lists in LDS hold the LDS byte addresses of their codewords (the image starts
// low in LDS and K <= 4096, so they fit in 16 bits) and are followed by kIndexListPad entries
// naming codeword 0, so a list can be read past its end.
__host__ __device__ inline size_t search_lds_bytes(int K, int G) {
    return align16((size_t)K * 8) + align16(kIndexFine) + align16((size_t)(G * G + 1) * 2) +
           align16((size_t)(index_lds_entries(K) + kIndexListPad) * 2);
}

// Byte offsets of the sections of the LDS image: codebook, fine-bin table, list offsets (u16),
// lists.  The search index holds a ready-made copy of this image (lists as byte offsets 8 j)
// at kIndexImgOff, so a workgroup fills its LDS with a plain 16-byte copy.
struct SearchImageLayout {
    size_t cb, fine, offs, ent, bytes;
};
__host__ __device__ inline SearchImageLayout search_image_layout(int K, int G) {
    SearchImageLayout l;
    l.cb = 0;
    l.fine = l.cb + align16((size_t)K * 8);
    l.offs = l.fine + align16(kIndexFine);
    l.ent = l.offs + align16((size_t)(G * G + 1) * 2);
    l.bytes = search_lds_bytes(K, G);
    return l;
}
constexpr size_t kIndexImgOff = ((size_t)kIndexEntOff + (size_t)kIndexMaxEntries * 2 + 255) / 256 * 256;

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

// Keep a value in a register: the empty asm hides how it was computed, so the compiler cannot
// rematerialize it (e.g. redo a division) inside a loop.
template <typename T>
__device__ __forceinline__ void pin_reg(T& v) {
    asm volatile("" : "+v"(v));
}

// Sign mask of the rotation (paper section 3.3: a deterministic sign per input column, shared by
// every row).  eps_j = -1 exactly when the top bit of the (j+1)-th output of the splitmix64
// generator started at `seed` is set; that output is the published splitmix64 finalizer (Steele,
// Lea and Flood, OOPSLA 2014; the constants of Vigna's reference code) applied to
// seed + (j+1) * 0x9E3779B97F4A7C15, all arithmetic modulo 2^64.  The last xor-shift of the
// finalizer leaves the top bit unchanged, so it is not computed.
__host__ __device__ __forceinline__ bool eps_negative(uint64_t seed, uint32_t j) {
    uint64_t z = seed + (uint64_t)(j + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (z >> 63) != 0;
}

// Make LDS writes of this wavefront visible to its other lanes before the reads that follow.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Butterflies on index bit rbit over the elements whose bit 0 is h (rbit >= 1 keeps the two
// halves apart).
template <int E>
__device__ __forceinline__ void butterfly_half(double (&x)[E], int rbit, int h) {
#pragma unroll
    for (int m = 0; m < E; ++m) {
        if ((m & 1) == h && !(m & (1 << rbit))) {
            double a = x[m], c = x[m | (1 << rbit)];
            x[m] = a + c;
            x[m | (1 << rbit)] = a - c;
        }
    }
}

// Phase A -> phase B for one wavefront, one half (the elements with bit 0 = h) at a time.
// `xb` is the wavefront's exchange buffer (Layout<L>::xbuf doubles, one half).
// Compact index c of a (block-local) element sits at c + c/H (one pad double per H).  The lanes
// of a block divide H, so both address streams are one per-lane base plus compile-time offsets:
//   write: element q*E + 2i + h -> c = base + q*H + i,        c/H = base/H + q
//   read : element h | (q<<1) | (i<<(L-e+1)) -> c = base + q + i*lanes, c/H = base/H + i*lanes/H
template <int L>
struct Exchange {
    using Lo = Layout<L>;
    static constexpr int H = Lo::half, NL = Lo::lanes;
    static_assert(H % NL == 0, "lanes of a block must divide E/2");
    double* wr;
    double* rd;
    __device__ Exchange(double* xb, int lane) {
        const unsigned beta = (unsigned)lane / NL, q = (unsigned)lane % NL;
        const unsigned base = beta * (Lo::b / 2);
        wr = xb + (base + base / H + q * (H + 1));
        rd = xb + (base + base / H + q);
    }
    __device__ __forceinline__ void write(const double (&x)[Lo::E], int h) const {
#pragma unroll
        for (int i = 0; i < H; ++i) wr[i] = x[2 * i + h];
    }
    __device__ __forceinline__ void read(double (&x)[Lo::E], int h) const {
#pragma unroll
        for (int i = 0; i < H; ++i) x[2 * i + h] = rd[i * NL + (i * NL) / H];
    }
};

// The same transpose through a buffer of half the size, in two rounds that every lane of the
// wavefront reads in.  Reader slot i of lane q takes source lane (q + i*lanes) / H, which has its top
// q bit clear exactly for i < H/2: round r moves the elements of the source lanes whose top q bit is r
// (they write all H of theirs) into reader slots r*H/2 .. r*H/2 + H/2 - 1.  Only the writes depend on
// the lane, so no register has to be merged between lanes that read and lanes that did not.
// Round-compact index of a block's element: writer ql = q mod lanes/2, element i -> beta*HB + ql*H + i;
// reader slot r*H/2 + j -> beta*HB + q + j*lanes; stored at c + c/H (one pad double per H).
//   write: c/H = beta*lanes/2 + ql;  read: c/H = beta*lanes/2 + (j*lanes)/H.
// A wavefront's buffer holds 32*(H + 1) doubles.
template <int L>
struct ExchangeHalf {
    using Lo = Layout<L>;
    static constexpr int H = Lo::half, NL = Lo::lanes, HB = NL / 2 * H;
    static_assert(H % NL == 0 && NL % 2 == 0, "lanes of a block must be even and divide E/2");
    double* wr;
    double* rd;
    bool top;   // the lane's top q bit: it writes in round 1
    __device__ ExchangeHalf(double* xb, int lane) {
        const unsigned beta = (unsigned)lane / NL, q = (unsigned)lane % NL, ql = q % (NL / 2);
        top = q >= (unsigned)(NL / 2);
        wr = xb + (beta * (HB + NL / 2) + ql * (H + 1));
        rd = xb + (beta * (HB + NL / 2) + q);
    }
    // this lane's H elements of half h (x[2 i + h]), from `src` (the values before round 0's reads)
    __device__ __forceinline__ void write(const double (&src)[Lo::E], int h) const {
#pragma unroll
        for (int i = 0; i < H; ++i) wr[i] = src[2 * i + h];
    }
    // reader slots r*H/2 .. r*H/2 + H/2 - 1 of half h
    __device__ __forceinline__ void read(double (&x)[Lo::E], int h, int r) const {
#pragma unroll
        for (int j = 0; j < H / 2; ++j) x[2 * (r * (H / 2) + j) + h] = rd[j * NL + (j * NL) / H];
    }
};

template <int L>
__device__ __forceinline__ void exchange_AB(double (&x)[Layout<L>::E], double* xb, int lane) {
    const Exchange<L> ex(xb, lane);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        ex.write(x, h);
        wave_lds_sync();
        ex.read(x, h);
        wave_lds_sync();
    }
}

// Exact nearest codeword (fp32 distance fl(fl(dx*dx) + fl(dy*dy)), ties to the lowest index).
__device__ __forceinline__ float dist_f32(float px, float py, float2 c) {
    float dx = px - c.x;
    float dy = py - c.y;
    return dx * dx + dy * dy;   // built with -ffp-contract=off: three rounded operations
}

__device__ __forceinline__ void eval_cw(float px, float py, float2 c, int j, float& bd, int& bj) {
    float d = dist_f32(px, py, c);
    if (d < bd) {
        bd = d;
        bj = j;
    }
}

__device__ inline SearchLds search_lds_carve(char* smem, int K, const IndexHeader& ih, const char* index) {
    const SearchImageLayout l = search_image_layout(K, ih.G);
    SearchLds s;
    s.cb = reinterpret_cast<float2*>(smem + l.cb);
    s.cb_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);   // LDS offset
    s.order = reinterpret_cast<const uint16_t*>(index + kIndexOrderOff);
    s.fine = reinterpret_cast<uint8_t*>(smem + l.fine);
    s.offs = reinterpret_cast<uint16_t*>(smem + l.offs);
    s.ent = reinterpret_cast<uint16_t*>(smem + l.ent);
    s.R = ih.R;
    s.inv_w = ih.inv_w;
    s.W = ih.W;
    s.G = ih.G;
    s.K = K;
    return s;
}

// Copy the index's LDS image into LDS (16-byte copies, four in flight per thread).  The image's
// lists hold byte offsets 8 j; when the image does not start at LDS address 0 they are rebased
// after a barrier.  The caller synchronizes afterwards.
__device__ inline void search_lds_fill(const SearchLds& s, const char* __restrict__ index, int K, int tid,
                                       int nthreads) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const IndexHeader& ih = *reinterpret_cast<const IndexHeader*>(index);
    const SearchImageLayout l = search_image_layout(K, ih.G);
    const int n16 = (int)(l.bytes / 16);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(index + kIndexImgOff);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(s.cb);
    int i = tid;
    for (; i + 3 * nthreads < n16; i += 4 * nthreads) {
        const u32x4_t v0 = src[i], v1 = src[i + nthreads], v2 = src[i + 2 * nthreads], v3 = src[i + 3 * nthreads];
        dst[i] = v0;
        dst[i + nthreads] = v1;
        dst[i + 2 * nthreads] = v2;
        dst[i + 3 * nthreads] = v3;
    }
    for (; i < n16; i += nthreads) dst[i] = src[i];
    if (s.cb_lds != 0) {
        __syncthreads();
        const int ne = min(ih.n_entries, index_lds_entries(K)) + kIndexListPad;
        for (int e = tid; e < ne; e += nthreads) s.ent[e] = (uint16_t)(s.ent[e] + s.cb_lds);
    }
}

// True when any active lane of the wavefront has a non-zero value.
__device__ __forceinline__ bool wave_any(uint32_t v) { return __builtin_amdgcn_ballot_w64(v != 0) != 0; }

// Points outside the grid: scan codewords by decreasing norm, stopping once |p| - |c| exceeds
// sqrt(D_a (1 + 1e-5)) for a known codeword a -- no later codeword can then beat or tie a.
__device__ __forceinline__ int nearest_exterior(float px, float py, const SearchLds& s) {
    const float lim_in = s.R * 0.999f;
    const float qx = fminf(fmaxf(px, -lim_in), lim_in), qy = fminf(fmaxf(py, -lim_in), lim_in);
    const int bx = min((int)((qx + s.R) * s.inv_w), s.W - 1), by = min((int)((qy + s.R) * s.inv_w), s.W - 1);
    const int cell = s.fine[by] * s.G + s.fine[bx];
    const int a = (s.offs[cell + 1] > s.offs[cell]) ? (int)((s.ent[s.offs[cell]] - s.cb_lds) >> 3) : 0;
    const float da = dist_f32(px, py, s.cb[a]);
    const double pn = __builtin_sqrt((double)px * px + (double)py * py);
    const double lim = pn - __builtin_sqrt((double)da * (1.0 + 1e-5));
    const double lim2 = lim > 0.0 ? lim * lim : -1.0;
    float bd = __builtin_inff();
    int bj = s.K;
    for (int t = 0; t < s.K; ++t) {
        const int j = s.order[t];
        const float2 c = s.cb[j];
        if ((double)c.x * c.x + (double)c.y * c.y < lim2) break;   // |c| < lim, exact squares in double
        const float d = dist_f32(px, py, c);
        if (d < bd || (d == bd && j < bj)) {
            bd = d;
            bj = j;
        }
    }
    return bj;
}

// The slow cases of one point: outside the grid, non-finite, or in a cell searched exhaustively.
__device__ __forceinline__ int nearest_slow(float px, float py, const SearchLds& s) {
    if (fabsf(px) < s.R && fabsf(py) < s.R) {   // exhaustive cell (its list did not fit)
        float bd = __builtin_inff();
        int bj = 0;
        for (int j = 0; j < s.K; ++j) eval_cw(px, py, s.cb[j], j, bd, bj);
        return bj;
    }
    if (!(__builtin_isfinite(px) && __builtin_isfinite(py))) return 0;   // every distance is NaN or inf
    return nearest_exterior(px, py, s);
}

__device__ __forceinline__ int nearest_lds(float px, float py, const SearchLds& s) {
    if (fabsf(px) < s.R && fabsf(py) < s.R) {
        const int bx = min((int)((px + s.R) * s.inv_w), s.W - 1);
        const int by = min((int)((py + s.R) * s.inv_w), s.W - 1);
        const int cell = s.fine[by] * s.G + s.fine[bx];
        const int o0 = s.offs[cell], o1 = s.offs[cell + 1];
        if (o1 > o0) {
            float bd = __builtin_inff();
            int bj = 0;
            for (int o = o0; o < o1; ++o) {
                const int j = (int)((s.ent[o] - s.cb_lds) >> 3);
                eval_cw(px, py, s.cb[j], j, bd, bj);
            }
            return bj;
        }
    }
    return nearest_slow(px, py, s);
}

// Codeword at LDS byte address `addr`.
typedef float lds_f2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 cw_at(uint32_t addr) {
    const lds_f2 v = *(const __attribute__((address_space(3))) lds_f2*)(size_t)addr;
    return make_float2(v.x, v.y);
}

// NP points searched in lockstep, at most S steps.  Step t evaluates entry o_i + t of every point's
// list.  The loop runs until the longest list of the wavefront is done or S steps have run (a
// uniform loop) and reads shorter lists past their end, into the following cells' lists and the
// zero padding: that is harmless, because a list holds every codeword that can be nearest or tied
// anywhere in its cell, so an extra codeword can neither be strictly closer nor tie with a lower
// index than the answer (lists are in increasing index order and only a strictly smaller distance
// replaces the best).  A point whose list is longer than S leaves its state in `st` (best distance
// and codeword address, next entry and end of its list) for search_finish, which evaluates the
// rest of the list in the same order.  Points outside the grid, in exhaustive cells or non-finite
// take the single-point path afterwards, one point slot at a time (a uniform loop, so the slow
// path exists once in the code); their answer is final.
struct SearchCont {
    float bd;
    uint32_t bo_next;   // LDS byte address of the best codeword so far | list entry to evaluate next << 16
    uint32_t end;       // one past the list's last entry (end > next: the list is not finished)
    __device__ bool open() const { return end > (bo_next >> 16); }
};

template <int NP, int S, bool UNROLL = true>
__device__ __forceinline__ void nearest_lds_capped(const float (&px)[NP], const float (&py)[NP], const SearchLds& s,
                                                   int (&out)[NP], SearchCont (&st)[NP]) {
    float bd[NP];
    uint32_t bo[NP], o0[NP], o1[NP];
    uint32_t slow = 0;
    int steps = 0;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        bd[i] = __builtin_inff();
        bo[i] = s.cb_lds;
        int a0 = 0, a1 = 0;   // empty: points outside the grid take the slow path
        if (fabsf(px[i]) < s.R && fabsf(py[i]) < s.R) {
            const int bx = min((int)((px[i] + s.R) * s.inv_w), s.W - 1);
            const int by = min((int)((py[i] + s.R) * s.inv_w), s.W - 1);
            const int cell = s.fine[by] * s.G + s.fine[bx];
            a0 = s.offs[cell];
            a1 = s.offs[cell + 1];
        }
        if (a1 <= a0) {   // outside the grid, non-finite, or exhaustive cell
            slow |= 1u << i;
            a0 = 0;
            a1 = 0;
        }
        o0[i] = (uint32_t)a0;
        o1[i] = (uint32_t)a1;
        steps = max(steps, a1 - a0);
    }
    if (steps > S) steps = S;
    auto step = [&](int t) {
        uint32_t ad[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) ad[i] = s.ent[o0[i] + t];
        float2 c[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) c[i] = cw_at(ad[i]);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const float d = dist_f32(px[i], py[i], c[i]);
            if (d < bd[i]) {
                bd[i] = d;
                bo[i] = ad[i];
            }
        }
    };
    if constexpr (UNROLL) {
        // unrolled: a step's list reads are one base address per pair plus a constant offset, and
        // no pointer increments or loop-carried copies remain (more code and live registers)
#pragma unroll
        for (int t = 0; t < S; ++t) {
            if (!wave_any((uint32_t)(t < steps))) break;
            step(t);
        }
    } else {
        for (int t = 0; wave_any((uint32_t)(t < steps)); ++t) step(t);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        out[i] = (int)((bo[i] - s.cb_lds) >> 3);
        st[i].bd = bd[i];
        st[i].bo_next = bo[i] | ((o0[i] + S) << 16);
        st[i].end = o1[i];   // slow points have an empty list: end 0 <= next
    }
    if (wave_any(slow)) {
#pragma unroll 1
        for (int i = 0; i < NP; ++i) {
            if (!wave_any(slow & (1u << i))) continue;
            float qx = px[0], qy = py[0];
#pragma unroll
            for (int k = 1; k < NP; ++k) {
                qx = (i == k) ? px[k] : qx;
                qy = (i == k) ? py[k] : qy;
            }
            int r = 0;
            if (slow & (1u << i)) r = nearest_slow(qx, qy, s);
#pragma unroll
            for (int k = 0; k < NP; ++k)
                if (i == k && (slow & (1u << i))) out[k] = r;
        }
    }
}

// Queue of unfinished searches of one wavefront (kSearchQueue entries, structure of arrays in LDS):
// the point, the best distance so far, the best codeword's LDS address with the index slot the
// answer goes to, and the rest of the list.
constexpr int kSearchQueue = 64;
struct SearchQueue {
    float* x;
    float* y;
    float* bd;
    uint32_t* a;   // bo | slot << 16
    uint32_t* b;   // next | end << 16
};
__host__ __device__ constexpr size_t search_queue_bytes() { return (size_t)kSearchQueue * 5 * sizeof(uint32_t); }
__device__ __forceinline__ SearchQueue search_queue_at(char* p) {
    SearchQueue q;
    q.x = reinterpret_cast<float*>(p);
    q.y = q.x + kSearchQueue;
    q.bd = q.y + kSearchQueue;
    q.a = reinterpret_cast<uint32_t*>(q.bd + kSearchQueue);
    q.b = q.a + kSearchQueue;
    return q;
}

// Finishes the n queued searches, one per lane (n <= the wavefront size), and writes each answer
// to idx[slot].  Called by the whole wavefront; the queue's entries are visible (wave_lds_sync).
__device__ __forceinline__ void search_finish(const SearchQueue& q, int n, const SearchLds& s, uint16_t* idx,
                                              int lane) {
    const bool mine = lane < n;
    float x = 0.0f, y = 0.0f, bd = 0.0f;
    uint32_t a = 0, b = 0;
    if (mine) {
        x = q.x[lane];
        y = q.y[lane];
        bd = q.bd[lane];
        a = q.a[lane];
        b = q.b[lane];
    }
    uint32_t bo = a & 0xFFFFu;
    const uint32_t next = b & 0xFFFFu;
    const int rem = mine ? (int)((b >> 16) - next) : 0;
    for (int t = 0; wave_any((uint32_t)(t < rem)); ++t) {
        const uint32_t ad = s.ent[next + t];   // past its end for the shorter lists: harmless
        const float d = dist_f32(x, y, cw_at(ad));
        if (d < bd) {
            bd = d;
            bo = ad;
        }
    }
    if (mine) idx[a >> 16] = (uint16_t)((bo - s.cb_lds) >> 3);
}

// ----------------------------------------------------------------------------- polar baseline
// Paper section 3.5: the pair is coded as a magnitude level (Na = 2^ba levels) times a phase bin
// (Np = 2^bp bins centred on 2 pi j / Np); the index is ia + Na * ip.  Both parts are found by a
// guess and an exact check, so the dependent chain is short:
//   magnitude  ia = #{i : t2[i] < fl64(x^2 + y^2)}.  A grid of kPolarGrid cells over
//              r in [0, 1.5 t_max) gives a lower bound (the count below the edge of the cell under
//              the one r falls in), and a scan of t2 upwards finishes it (cells hold at most one
//              Lloyd-Max threshold for ba <= 8, so the scan takes one or two steps).
//   phase      the pair is rotated by a multiple of pi/2 into the first quadrant (exact); a fp32
//              arctangent gives the bin m0 to within one; the fp64 cross products with the two
//              bin edges around m0 decide the bin exactly (up to rounding at an edge).
// In LDS:
//   t2[i]   = fl64(t_i^2), the Na - 1 squared thresholds;
//   mg[g]   = #{i : t_i < g w}, w = 1.5 t_max / kPolarGrid;
//   edge[k] = (cos, sin) of the bin edge (2k + 1) pi / Np, k = 0 .. Np/4 - 1 (first quadrant).
constexpr int kPolarMaxBa = 8;
constexpr int kPolarGrid = 1024;

struct PolarLds {
    double* t2;
    uint16_t* mg;
    double2* edge;
    int ba, bp;
    float inv_w;   // kPolarGrid / (1.5 t_max)
};

__host__ __device__ inline size_t polar_lds_bytes(int bp) {
    const int nq = bp >= 2 ? (1 << bp) / 4 : 1;
    return (size_t)(1 << kPolarMaxBa) * sizeof(double) + (size_t)kPolarGrid * sizeof(uint16_t) +
           (size_t)nq * 2 * sizeof(double);
}

__device__ inline PolarLds polar_lds_carve(char* smem, int ba, int bp) {
    PolarLds p;
    p.t2 = reinterpret_cast<double*>(smem);
    p.mg = reinterpret_cast<uint16_t*>(smem + (size_t)(1 << kPolarMaxBa) * sizeof(double));
    p.edge = reinterpret_cast<double2*>(smem + (size_t)(1 << kPolarMaxBa) * sizeof(double) +
                                        (size_t)kPolarGrid * sizeof(uint16_t));
    p.ba = ba;
    p.bp = bp;
    p.inv_w = 0.0f;
    return p;
}

// Fill the tables and p.inv_w (all threads of the workgroup take part; a barrier must follow).
// Returns true in some thread when the thresholds are not finite, non-negative and non-decreasing.
__device__ inline bool polar_lds_fill(PolarLds& p, const double* __restrict__ thr, int tid, int nthreads) {
    const int na = 1 << p.ba;
    bool bad = false;
    for (int i = tid; i < na - 1; i += nthreads) {
        const double t = thr[i];
        p.t2[i] = t * t;
        bad |= !(t >= 0.0 && t <= __builtin_huge_val());
        if (i + 1 < na - 1) bad |= !(t <= thr[i + 1]);
    }
    double rmax = 1.5 * thr[na - 2];
    if (!(rmax > 1e-30 && rmax < 1e30)) rmax = 1.0;   // degenerate thresholds (flagged): any grid is valid
    const double w = rmax / kPolarGrid;
    p.inv_w = (float)(kPolarGrid / rmax);
    for (int g = tid; g < kPolarGrid; g += nthreads) {
        const double e = g * w;
        int c = 0;   // #{t_i < e}, binary search over the sorted thresholds
        for (int step = na >> 1; step >= 1; step >>= 1)
            if (thr[c + step - 1] < e) c += step;
        p.mg[g] = (uint16_t)c;
    }
    if (p.bp >= 2) {
        const int np = 1 << p.bp, nq = np / 4;
        for (int k = tid; k < nq; k += nthreads) {
            const double f = (double)(2 * k + 1) / (double)np;   // exact
            p.edge[k] = make_double2(cospi(f), sinpi(f));
        }
    }
    return bad;
}

// atan(t) for t in [0, 1] to about 3e-5: t times a least-squares fit of atan(t)/t in t^2
__device__ __forceinline__ float atan_unit(float t) {
    const float s = t * t;
    float q = 0.0245979764f;
    q = q * s - 0.0935131311f;
    q = q * s + 0.186332226f;
    q = q * s - 0.331977546f;
    q = q * s + 0.999985754f;
    return q * t;
}

// Polar indices of NB pairs.  A pair at the origin (or NaN) gets phase 0; an infinite component is
// taken as the direction it points.
template <int NB>
__device__ __forceinline__ void polar_batch(const float (&px)[NB], const float (&py)[NB], const PolarLds& p,
                                            int (&out)[NB]) {
    const int na = 1 << p.ba;
    int ia[NB];
    bool zero[NB], big[NB];
    {
        double r2[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const double x = px[i], y = py[i];
            r2[i] = x * x + y * y;   // both products exact
            zero[i] = !(r2[i] > 0.0);   // the origin, or NaN
            big[i] = __builtin_isinf(r2[i]);
            const float gf = __builtin_amdgcn_sqrtf((float)r2[i]) * p.inv_w;
            // one cell below the cell of r: a lower bound however fp32 rounds (NaN -> cell 0)
            const int g = gf >= 1.0f ? (int)__builtin_fminf(gf, (float)kPolarGrid) - 1 : 0;
            ia[i] = p.mg[g];
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
            while (ia[i] < na - 1 && p.t2[ia[i]] < r2[i]) ++ia[i];
    }
    // the pair, with an infinite component taken as the direction it points (r2 infinite)
    float fx[NB], fy[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        fx[i] = px[i];
        fy[i] = py[i];
        if (big[i]) {
            fx[i] = __builtin_isinf(fx[i]) ? __builtin_copysignf(1.0f, fx[i]) : __builtin_copysignf(0.0f, fx[i]);
            fy[i] = __builtin_isinf(fy[i]) ? __builtin_copysignf(1.0f, fy[i]) : __builtin_copysignf(0.0f, fy[i]);
        }
    }
    int ip[NB];
    if (p.bp == 1) {   // two bins, centred on 0 and pi: the edge is the y axis (theta = -pi/2 goes to 0)
#pragma unroll
        for (int i = 0; i < NB; ++i) ip[i] = (fx[i] > 0.0f || (fx[i] == 0.0f && fy[i] < 0.0f)) ? 0 : 1;
    } else {
        const int nq = (1 << p.bp) >> 2;
        const float bins_per_rad = (float)(1 << p.bp) * 0.159154943f;   // Np / (2 pi)
        double2 elo[NB], ehi[NB];
        int m0[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const float x = fx[i], y = fy[i];
            // quadrant q: theta in [q pi/2, (q+1) pi/2) (mod 2 pi); (fx, fy) becomes the pair rotated
            // by -q pi/2 (exact), and ip starts at q Np/4
            int q;
            if (x > 0.0f && y >= 0.0f) {
                q = 0; fx[i] = x; fy[i] = y;
            } else if (x <= 0.0f && y > 0.0f) {
                q = 1; fx[i] = y; fy[i] = -x;
            } else if (x < 0.0f && y <= 0.0f) {
                q = 2; fx[i] = -x; fy[i] = -y;
            } else {
                q = 3; fx[i] = -y; fy[i] = x;
            }
            ip[i] = q * nq;
            const float u = fx[i], v = fy[i];
            float lo = __builtin_fminf(u, v), hi = __builtin_fmaxf(u, v);
            // the fp32 reciprocal flushes denormal inputs and results, which would throw the guess
            // off by more than a bin: an exact power-of-two scale keeps hi in [2^-49, 2^28]
            const float sc = hi < 0x1p-100f ? 0x1p100f : (hi > 0x1p100f ? 0x1p-100f : 1.0f);
            lo *= sc;
            hi *= sc;
            const float tq = hi > 0.0f ? __builtin_fminf(lo * __builtin_amdgcn_rcpf(hi), 1.0f) : 0.0f;
            const float at = atan_unit(tq);
            const float phi = v > u ? 1.57079633f - at : at;
            const float mf = phi * bins_per_rad + 0.5f;
            const int m = mf >= 1.0f ? (int)__builtin_fminf(mf, (float)nq) : 0;   // NaN -> 0
            m0[i] = m;
            elo[i] = p.edge[m > 0 ? m - 1 : 0];
            ehi[i] = p.edge[m < nq ? m : nq - 1];
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const double u = fx[i], v = fy[i];
            // the true bin is m0 - 1, m0 or m0 + 1: below the edge of m0, or on or past the next one
            const bool dec = m0[i] > 0 && elo[i].x * v - elo[i].y * u < 0.0;
            const bool inc = m0[i] < nq && ehi[i].x * v - ehi[i].y * u >= 0.0;
            ip[i] = (ip[i] + m0[i] - (dec ? 1 : 0) + (inc ? 1 : 0)) & ((1 << p.bp) - 1);
        }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) out[i] = ia[i] + ((zero[i] ? 0 : ip[i]) << p.ba);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// QAMW_FLAG_BAD_INDEX of qamw.h: the search index was built for another codebook size.
constexpr int32_t kFlagBadIndex = 32;

__device__ __forceinline__ void flag_status(int32_t* status, int32_t f) {
    if (status && f) atomicOr(status, f);
}

}  // namespace qamw
