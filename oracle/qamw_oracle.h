/*
 * CPU oracle for the QAM-W weight codec -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the package's smoke check and bench.py's cpu_baseline leg may
 * call this library.  The GPU library never includes, links or calls it.
 *
 * Source: "QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
 * Rotation and Activation-Aware Scaling" (Sharma and Dobek, arXiv 2605.26339),
 * sections 3.1-3.8.  Every function names the passage it follows.
 *
 * Conventions: all pointers are host pointers owned by the caller; per-row
 * arrays hold exactly the rows passed in, in order.  Functions return 0 on
 * success and -1 on a bad argument; data faults are OR-ed into *status.
 */
#ifndef QAMW_ORACLE_H
#define QAMW_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORACLE_FLAG_NONFINITE = 1,
    ORACLE_FLAG_BAD_SCALE = 2,
    ORACLE_FLAG_NORM_RANGE = 4,
    ORACLE_FLAG_POINT_RANGE = 8
};

uint16_t oracle_f16_from_f32(float f);
float oracle_f32_from_f16(uint16_t h);
uint16_t oracle_bf16_from_f32(float f);

/* section 3.3, the deterministic sign mask (reading R1): splitmix64 outputs and the mask bits */
void oracle_splitmix64(uint64_t seed, int64_t n, uint64_t* out);
void oracle_sign_mask(uint64_t seed, int32_t d_in, uint32_t* bits);
void oracle_hadamard(int32_t b, double* H);
int32_t oracle_default_block(int32_t d_in);
double oracle_bpw(int32_t d_in, int32_t bits);
size_t oracle_row_stride(int32_t d_in, int32_t bits);

int oracle_front_end(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                     const float* s, const uint32_t* sign_bits, int32_t block, double* y, double* r,
                     int32_t* status);
int oracle_calibrate(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                     const float* s, const uint32_t* sign_bits, int32_t block, float* sigma,
                     int32_t* status);
int32_t oracle_nearest(float px, float py, const float* cb, int32_t K, float* dist);
void oracle_nearest_many(const float* p, int64_t n, const float* cb, int32_t K, int32_t* idx,
                         float* dist);
void oracle_pack_row(const int32_t* idx, int32_t n_pairs, int32_t bits, uint8_t* out, size_t stride);
void oracle_unpack_row(const uint8_t* in, int32_t n_pairs, int32_t bits, int32_t* idx);
int oracle_encode(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                  const float* s, const uint32_t* sign_bits, int32_t block, const float* cb,
                  int32_t bits, const float* sigma, uint16_t* norm16, uint8_t* codes,
                  int32_t* idx_out, float* p_out, int32_t* status);
int oracle_decode(const uint8_t* codes, const uint16_t* norm16, int64_t n_rows, int32_t d_in,
                  const float* sigma, const float* cb, int32_t bits, const float* s,
                  const uint32_t* sign_bits, int32_t block, float* out_f32, uint16_t* out_bf16,
                  double* out_f64);
int oracle_lloyd(const float* pts, int64_t n, int32_t bits, int32_t iters, const float* init,
                 float* cb, int64_t* e_trace, int32_t* status);
/* section 1: the product after dequantization, y = x W^T in fp64 */
int oracle_qgemm(const float* x, int32_t M, int64_t ld_x, const uint8_t* codes, const uint16_t* norm16,
                 int64_t n_rows, int32_t d_in, const float* sigma, const float* cb, int32_t bits,
                 const float* s, const uint32_t* sign_bits, int32_t block, double* y);
/* section 3.5, the polar baseline (reading R8) */
int oracle_rayleigh_lloyd_max(int32_t ba, double* levels, double* thresholds);
int32_t oracle_polar_index(float px, float py, int32_t ba, int32_t bp, const double* thresholds);
void oracle_polar_table(int32_t ba, int32_t bp, const double* levels, float* cb);
int oracle_encode_polar(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                        const float* s, const uint32_t* sign_bits, int32_t block, int32_t ba, int32_t bp,
                        const double* thresholds, const float* sigma, uint16_t* norm16, uint8_t* codes,
                        int32_t* idx_out, float* p_out, int32_t* status);
/* the activation-aware channel scale (reading R11) */
int oracle_act_scale(const float* x, int64_t T, int32_t d_in, int64_t ld, double alpha, float* scale, double* rms);
/* section 2, the scalar (d = 1) ablation (reading R10) */
int oracle_gauss_lloyd_max(int32_t b, double* levels, double* thresholds);
int32_t oracle_scalar_index(float p, int32_t b, const double* thresholds);
void oracle_scalar_table(int32_t b, const double* levels, float* cb);
int oracle_encode_scalar(const void* w, int32_t w_bf16, int64_t n_rows, int32_t d_in, int64_t ld,
                         const float* s, const uint32_t* sign_bits, int32_t block, int32_t b,
                         const double* thresholds, const float* sigma, uint16_t* norm16, uint8_t* codes,
                         int32_t* idx_out, float* p_out, int32_t* status);

#ifdef __cplusplus
}
#endif
#endif
