// Host-side launchers of the QAM-W kernels.  Arguments are validated by the C ABI layer
// (qamw_api.cpp) before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qamw {

// Let `kernel` use more than the default 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU).
template <typename K>
inline void allow_lds(K kernel, size_t bytes) {
    if (bytes > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)bytes);
}

int index_grid_size(int bits);
size_t index_bytes_for(int bits);
hipError_t launch_index_build(const float* cb, int bits, void* index, hipStream_t st);
hipError_t launch_nearest(const float* pts, int64_t n, const float* cb, int bits, const void* index, int32_t* out,
                          hipStream_t st);

struct EncodeArgs {
    const void* w;
    int w_bf16;
    int d_out, d_in;
    int64_t ld;
    const float* scale;        // may be null (all ones)
    uint64_t sign_seed;        // sign mask eps_j (eps_negative)
    const float* sigma;        // d_in/2
    const float* cb;
    int bits;
    const void* index;
    int index_g;               // grid size the index of a 2^bits codebook has (checked on the device)
    const double* thr;         // polar baseline: ba bits of magnitude (thresholds) and bits - ba of phase
    int ba;
    uint16_t* norm;
    uint8_t* codes;
    size_t stride;
    int32_t* status;
};

struct CalibArgs {
    const void* w;
    int w_bf16;
    int n_rows, d_in;
    int64_t ld;
    const float* scale;
    uint64_t sign_seed;
    double* partial;           // [n_groups][d_in/2]
    int32_t* nz;               // [n_groups]
    int n_groups;
};

struct DecodeArgs {
    const uint8_t* codes;
    size_t stride;
    const uint16_t* norm;
    const float* sigma;
    const float* cb;
    int bits;
    const float* scale;
    uint64_t sign_seed;
    int d_out, d_in;
    void* out;
    int out_bf16;
    int64_t ld;
};

// Elements per lane of the transform layout for block size 2^L.
int lane_elems(int L);
// LDS bytes of the encoder for one row group; polar_bp >= 1 for the polar quantizer, else the
// QAM-W search image.
size_t encode_lds_bytes(int L, int bits, int d_in, int polar_bp);
constexpr size_t kLdsBytes = 160 * 1024;   // LDS per CU on gfx950
int calib_groups(int n_rows);
size_t calib_workspace(int d_out, int d_in);

hipError_t launch_calibrate(const CalibArgs& a, int L, float* sigma_out, hipStream_t st);
hipError_t launch_encode(const EncodeArgs& a, int L, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int L, hipStream_t st);
// Smallest LDS the decoder needs for a row of d_in columns (one row per workgroup).
size_t decode_lds_bytes(int L, int bits, int d_in);

// The decoder for 128-column blocks (k_decode128.hip): workgroups own spans of column blocks and
// walk tiles of rows.
// One matrix of a 128-column decode launch: its workgroups are wg0 .. wg0 + n_wg - 1 of the grid
// (wg0 and n_wg multiples of 8).
struct Decode128Item {
    const uint8_t* codes;
    const uint16_t* norm;
    const float* sigma;
    const float* scale;
    void* out;
    uint64_t sign_seed;
    uint32_t stride;   // bytes per code row
    int32_t d_out;
    uint32_t ld;       // output elements per row
    int32_t nb;        // column blocks per row
    int32_t wg0, n_wg;
};
// Matrices per launch of a grouped decode: the descriptors travel as kernel arguments (4 KiB).
constexpr int kDecodeBatch = 48;
template <int NI>
struct Decode128Batch {
    const float* cb;
    int32_t n;
    Decode128Item it[NI];
};
bool decode128_supported(const DecodeArgs& a, int L);
hipError_t launch_decode128(const DecodeArgs& a, int L, hipStream_t st);
// Decodes that share codebook, bits and output type, each accepted by decode128_supported (with the
// log2 block sizes L[i]), as launches of up to kDecodeBatch matrices.
hipError_t launch_decode128_many(const DecodeArgs* a, const int* L, int n, hipStream_t st);
hipError_t launch_sign_mask(uint64_t seed, int d_in, uint32_t* bits, hipStream_t st);
hipError_t launch_polar_codebook(int ba, int bp, double* levels, double* thr, float* cb, hipStream_t st);
hipError_t launch_scalar_codebook(int b, double* levels, double* thr, float* cb, hipStream_t st);
int act_chunks(int64_t T);
hipError_t launch_act_scale(const void* x, int x_bf16, int64_t T, int d_in, int64_t ld, double alpha, float* scale,
                            double* rms, double* partial, hipStream_t st);
hipError_t launch_polar_index(const float* pts, int64_t n, int ba, int bp, const double* thr, int32_t* out,
                              int32_t* status, hipStream_t st);

// Fused dequantize-and-multiply (k_qgemm.hip).
struct QgemmArgs {
    const uint8_t* codes;
    size_t stride;
    const uint16_t* norm;
    const float* cb;
    int bits;
    float* u;            // workspace: the rotated, sigma-scaled activations as bf16-piece B operands
    int M, n_pairs, d_out;
    void* y;
    int y_bf16;
    int64_t ld_y;
};
struct QgemmRotateArgs {
    const void* x;
    int x_bf16;
    int64_t ld_x;
    int d_in, block;
    const float* scale;
    uint64_t sign_seed;
    const float* sigma;
};
size_t qgemm_workspace(int M, int d_out, int d_in);
hipError_t launch_qgemm(const QgemmArgs& a, const QgemmRotateArgs& r, hipStream_t st);

struct LloydAcc;   // device accumulators, defined in k_lloyd.hip
size_t lloyd_workspace(int bits);
hipError_t launch_lloyd(const float* pts, int64_t n, int bits, int iters, const float* init, float* cb,
                        int64_t* trace, int32_t* status, void* ws, hipStream_t st);

}  // namespace qamw
