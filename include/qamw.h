/*
 * qamw.h -- C ABI of libqamw.so, the QAM-W weight codec on AMD Instinct MI355X (gfx950).
 *
 * QAM-W is defined in "QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
 * Rotation and Activation-Aware Scaling" (Sharma and Dobek, arXiv 2605.26339), section 3.
 * Each entry point below names the passage that defines the operation it computes.
 *
 * General conventions
 *   - Pointers prefixed d_ are device pointers (HBM of the current HIP device), owned by the
 *     caller, and must stay valid until the work queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void*; NULL selects the default stream.  Every call
 *     only queues work on that stream and never synchronizes with the host.
 *   - The library keeps no state between calls and allocates no device memory: scratch lives
 *     in the caller's workspace (sizes from the *_workspace / qamw_index_bytes helpers).  The one
 *     exception is qamw_qgemm_noalloc, whose workspace is a static array of the library on each
 *     device (QAMW_QGEMM_NOALLOC_BYTES, held until the process ends).
 *   - Return value: QAMW_OK, or a negative QAMW_ERR_* code computed by host code before any
 *     launch (bad argument, unsupported shape, short workspace) or from a failed launch.
 *     Nothing is queued when an argument error is returned.
 *   - Data faults found while running (non-finite weights, non-positive scale, row norm out
 *     of f16 range, training point out of range) are OR-ed as QAMW_FLAG_* bits into *d_status
 *     when d_status is not NULL; outputs for the affected rows/points are then unspecified.
 *   - Matrices are row-major: element (i, j) of W is at d_w[i * ld_w + j].
 *   - Concurrent calls on different streams are safe when they use different workspaces.
 */
#ifndef QAMW_H
#define QAMW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { QAMW_F32 = 0, QAMW_BF16 = 1 } qamw_dtype;

enum {
    QAMW_OK = 0,
    QAMW_ERR_ARG = -1,         /* invalid argument (shape, pointer, range)                   */
    QAMW_ERR_UNSUPPORTED = -2, /* valid by the paper but outside what the kernels implement  */
    QAMW_ERR_WORKSPACE = -3,   /* workspace / index buffer smaller than required             */
    QAMW_ERR_HIP = -4          /* a HIP launch failed                                        */
};

enum {
    QAMW_FLAG_NONFINITE = 1,   /* w_ij * s_j or the row norm is not finite                    */
    QAMW_FLAG_BAD_SCALE = 2,   /* some s_j <= 0 or NaN                                        */
    QAMW_FLAG_NORM_RANGE = 4,  /* the row norm overflows f16                                  */
    QAMW_FLAG_POINT_RANGE = 8, /* a training point is non-finite or out of the fixed-point range */
    QAMW_FLAG_BAD_THRESHOLDS = 16, /* polar thresholds not finite, >= 0 and non-decreasing       */
    QAMW_FLAG_BAD_INDEX = 32   /* the search index was built for another codebook size: nothing
                                  was encoded                                                 */
};

/* Section 3.3: the rotation's sign mask is deterministic and shared by every row.  It is drawn from
 * a 64-bit seed: eps_j = -1 exactly when the top bit of the (j+1)-th output of the splitmix64
 * generator started at the seed is set, i.e. of mix(seed + (j+1) * 0x9E3779B97F4A7C15) with the
 * published splitmix64 finalizer mix(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 * z *= 0x94D049BB133111EB; z ^= z >> 31 (arithmetic modulo 2^64).  Encoder and decoder must be
 * given the same seed.  QAMW_DEFAULT_SIGN_SEED is the value used when the caller has no other. */
#define QAMW_DEFAULT_SIGN_SEED 0x51414D57ull

/* Most rows a matrix may have in qamw_encode, qamw_encode_polar, qamw_decode and qamw_qgemm
 * (QAMW_ERR_UNSUPPORTED above): the kernels address the d_out row norms through 32-bit byte
 * ranges. */
#define QAMW_MAX_ROWS ((1 << 30) - 1)

/* Bytes per row of the packed index stream: ceil((d_in/2) * bits / 8) rounded up to 16.
 * Index k of a row occupies stream bits k*bits .. k*bits+bits-1, least significant first;
 * stream bit q is bit q%8 of byte q/8; padding bytes are zero.
 * (Section 3.1 step 6 and section 3.7: bit-packed indices with row-level alignment.)
 * Returns 0 for invalid arguments. */
size_t qamw_row_stride(int32_t d_in, int32_t bits);

/* Section 3.3: the block size used when `block` is 0 -- the largest power of two dividing
 * d_in, at most 1024.  Returns 0 when d_in <= 0. */
int32_t qamw_default_block(int32_t d_in);

/* Size of the search index that qamw_codebook_index writes for a 2^bits-entry codebook. */
size_t qamw_index_bytes(int32_t bits);

/* Workspace bytes for qamw_encode on a d_out x d_in matrix (calibration partial sums). */
size_t qamw_encode_workspace(int32_t d_out, int32_t d_in, int32_t bits);

/* Workspace bytes for qamw_codebook_train. */
size_t qamw_train_workspace(int64_t n_points, int32_t bits);

/* Section 3.6, eq. 2: train the single 2D codebook C = {c_0 .. c_{K-1}}, K = 2^bits, by Lloyd
 * iterations on samples of the unit circular Gaussian.
 *   d_points   n_points x 2 fp32, (x, y) interleaved.  n_points >= K.
 *   iters      number of Lloyd iterations (>= 0).
 *   d_init     K x 2 fp32 starting codebook, or NULL to start from the first K points.
 *   d_codebook K x 2 fp32 output (may alias d_init).
 *   d_err_trace NULL or iters int64 entries: entry t = sum over points of round(D * 2^32)
 *              (modulo 2^64) for the assignment of iteration t, D the squared distance to the
 *              assigned codeword; MSE_t = entry / 2^32 / n_points.
 * Each iteration assigns every point to its nearest codeword (fp32 distance
 * fl(fl(dx*dx) + fl(dy*dy)), dx = fl(px - cx); ties to the lowest index), sums the assigned
 * points as 64-bit integers of round(x * 2^32), and moves each non-empty codeword to
 * fl32((sum * 2^-32) / count); an empty cell keeps its codeword.  Integer sums make the result
 * independent of thread order.  Points that are non-finite or have |x| or |y| >=
 * min(2^(31 - ceil(log2 n_points)), 4096) are skipped and set QAMW_FLAG_POINT_RANGE.
 * Limits: 1 <= bits <= 12. */
int qamw_codebook_train(const float* d_points, int64_t n_points, int32_t bits, int32_t iters,
                        const float* d_init, float* d_codebook, int64_t* d_err_trace,
                        int32_t* d_status, void* d_ws, size_t ws_bytes, void* stream);

/* Build the nearest-codeword search index of a codebook (section 3.6: encoding maps each
 * normalized pair to its Euclidean-nearest entry).  The index is a uniform grid over the
 * codebook's extent; each cell lists, in increasing order, every codeword that can be the
 * nearest (or tied nearest) to a point of the cell, with a margin that covers fp32 rounding,
 * so searching a cell's list returns exactly what a search over all K codewords returns.
 * The index also holds a copy of the codebook, laid out with the grid as the encoder loads it
 * into LDS; qamw_encode searches that copy, so d_codebook passed to qamw_encode must be the
 * codebook the index was built from.
 *   d_index  device buffer of at least qamw_index_bytes(bits) bytes; it stays valid for this
 *            codebook until the codebook changes.  Limits: 1 <= bits <= 12. */
int qamw_codebook_index(const float* d_codebook, int32_t bits, void* d_index, size_t index_bytes,
                        void* stream);

/* Section 3.6: nearest codeword of n 2D points (fp32, interleaved), written to d_idx (int32),
 * using an index from qamw_codebook_index.  Same distance and tie rule as above.  An index built
 * for another codebook size gives -1 for every point. */
int qamw_nearest(const float* d_points, int64_t n, const float* d_codebook, int32_t bits,
                 const void* d_index, int32_t* d_idx, void* stream);

/* Section 3.1 (encoder) with section 3.4 (pair calibration) and section 3.8 (activation-aware
 * per-channel scale).  For every row i of W:
 *   a_j = w_ij * s_j (double), r = ||a||_2; r == 0 gives a zero row (norm 0, all indices 0);
 *   y = blockdiag(H_b) (eps . a / r), H_b the Sylvester-ordered Hadamard matrix / sqrt(b),
 *   eps the sign mask of sign_seed (section 3.3, QAMW_DEFAULT_SIGN_SEED above);
 *   p_k = (fl32(y_2k / sigma_k), fl32(y_2k+1 / sigma_k)), idx_k = nearest codeword;
 *   norm_i = f16(fl32(r)) round-to-nearest-even (section 3.2: 16-bit row norm);
 *   indices packed as in qamw_row_stride.
 * Arguments:
 *   d_w, w_dtype   weights (QAMW_F32 or QAMW_BF16), d_out x d_in, leading dimension ld_w >= d_in;
 *                  0 <= d_out <= QAMW_MAX_ROWS.
 *   d_scale        d_in fp32 channel scales s_j > 0, or NULL for all ones.
 *   block          Hadamard block size b: a power of two in [2, 1024] dividing d_in, or 0 for
 *                  qamw_default_block(d_in).  d_in must be even.  The kernels give each lane E
 *                  consecutive columns (E = 16 for b <= 128, 32 for b = 256 or 512, 64 for
 *                  b = 1024): d_in must be a multiple of E and d_in / E at most 1024 (E = 16)
 *                  or 512 (E = 32, 64), i.e. d_in <= 16384, 16384 and 32768; otherwise
 *                  QAMW_ERR_UNSUPPORTED.  At b = 1024 with bits >= 11 the decoder's LDS bounds
 *                  d_in to 28672; encode and decode reject wider rows alike
 *                  (QAMW_ERR_UNSUPPORTED), so whatever is encoded can be decoded.
 *   sign_seed      seed of the sign mask.
 *   d_codebook, bits, d_index   K = 2^bits codebook and its index; 1 <= bits <= 12.  The index
 *                  argument is not in the problem statement of the pages: it is built once per
 *                  codebook by qamw_codebook_index (tens of milliseconds) and serves every matrix
 *                  coded with that codebook.  An index of another codebook size sets
 *                  QAMW_FLAG_BAD_INDEX and nothing is written.
 *   d_sigma_in     d_in/2 fp32 per-pair scales to use, or NULL to calibrate (eq. 1):
 *                  sigma_k = fl32(mean |z_k| / sqrt(pi/2)), mean in double over the non-zero
 *                  finite rows among rows 0 .. min(d_out, 1024) - 1; 1/sqrt(d_in) when there
 *                  is no such row or the mean is 0.
 *   d_sigma_out    d_in/2 fp32 output of the sigma used (written when calibrating; when
 *                  d_sigma_in is given it may be NULL or receives a copy).
 *   d_norm_f16     d_out uint16 (IEEE binary16 bit patterns).
 *   d_codes        d_out x qamw_row_stride(d_in, bits) bytes.
 *   d_ws, ws_bytes at least qamw_encode_workspace(d_out, d_in, bits) bytes. */
int qamw_encode(const void* d_w, qamw_dtype w_dtype, int32_t d_out, int32_t d_in, int64_t ld_w,
                const float* d_scale, int32_t block, uint64_t sign_seed,
                const float* d_codebook, int32_t bits, const void* d_index,
                const float* d_sigma_in, float* d_sigma_out, uint16_t* d_norm_f16, uint8_t* d_codes,
                int32_t* d_status, void* d_ws, size_t ws_bytes, void* stream);

/* Section 3.2 (decoder) and section 1 (dequantize to BF16 before the matrix product):
 * unpack the indices, look up c[idx_k], rescale by sigma_k, apply R_inv = diag(eps)
 * blockdiag(H_b), multiply by the stored f16 row norm and divide by s_j:
 *   w^_ij = f16(norm_i) * eps_j * (H_b x)_j / s_j,  x_2k = sigma_k c_x[idx_k], x_2k+1 = sigma_k c_y[idx_k]
 * computed in double and rounded to fp32 (QAMW_F32) or to fp32 then BF16 with
 * round-to-nearest-even (QAMW_BF16).  A zero norm gives a row of +0.
 * Arguments mirror qamw_encode (sign_seed must be the encoder's); d_out_w is d_out x d_in with
 * leading dimension ld_out >= d_in (ld_out even).  Same block / d_in / d_out / bits limits as
 * qamw_encode: every matrix qamw_encode accepts can be decoded. */
int qamw_decode(const uint8_t* d_codes, const uint16_t* d_norm_f16, const float* d_sigma,
                const float* d_codebook, int32_t bits, const float* d_scale,
                int32_t d_out, int32_t d_in, int32_t block, uint64_t sign_seed,
                void* d_out_w, qamw_dtype out_dtype, int64_t ld_out, void* stream);

/* One matrix of qamw_decode_many: the per-matrix arguments of qamw_decode. */
typedef struct {
    const uint8_t* d_codes;
    const uint16_t* d_norm_f16;
    const float* d_sigma;
    const float* d_scale;     /* NULL for all ones */
    int32_t d_out;
    int32_t d_in;
    uint64_t sign_seed;
    void* d_out_w;
    int64_t ld_out;
} qamw_decode_job;

/* Section 3.2 and section 1 for the matrices of a model (the pages quantize every linear layer with
 * the one codebook): each job is decoded exactly as qamw_decode decodes it, with the shared
 * d_codebook, bits, block and out_dtype.  Jobs at block 128 (block 0 with 128 the default counts)
 * and bits 7, 8 or 11 are decoded by grouped launches of up to 48 matrices each, which start one
 * matrix while the previous one finishes; other jobs get a launch each.  The results equal those
 * of qamw_decode bit for bit.
 *   jobs     host array of n_jobs entries, read during the call only; n_jobs >= 0 (0 is a no-op).
 * Every job is checked as qamw_decode checks its arguments before anything is queued: the first
 * failing job's error is returned and nothing is queued.  Outputs must not overlap each other or
 * any input (the jobs run concurrently). */
int qamw_decode_many(const qamw_decode_job* jobs, int32_t n_jobs, const float* d_codebook, int32_t bits,
                     int32_t block, qamw_dtype out_dtype, void* stream);

/* Section 3.3: the sign mask of a seed as bits, for callers and tests that need eps itself: bit
 * j % 32 of d_bits[j / 32] is set when eps_j = -1 (j < d_in); the bits of the last word past d_in
 * are 0.  d_bits: (d_in + 31) / 32 device words.  d_in >= 0 (0 is a no-op). */
int qamw_sign_mask(uint64_t sign_seed, int32_t d_in, uint32_t* d_bits, void* stream);

/* Section 1 (the matrix product that follows dequantization), fused: for M activation rows
 *   y[m][i] = sum_j x[m][j] w^_ij
 * with w^ the qamw_decode weights before any rounding (f16(norm_i) eps_j (H_b x_i)_j / s_j, the
 * decoder's arguments as there), computed without forming W^: the activation is rotated instead,
 * u = sigma . blockdiag(H_b)(eps . x / s) (fp64, rounded to fp32 once), and
 *   y[m][i] = f16(norm_i) * sum_k (c[idx_ik].x u_m,2k + c[idx_ik].y u_m,2k+1)
 * on the matrix cores (v_mfma_f32_16x16x32_bf16; from 9 rows on matrices of more than 4096 rows,
 * v_mfma_f32_32x32x16_bf16) with each fp32 operand written as a sum of bf16
 * pieces: c = c1 + c2 (within 2^-18 |c|), u = u1 + u2 + u3 (exact) for M <= 5, u1 + u2 (within
 * 2^-18 |u|) above; piece products are exact and the sums run in fp32, per-wavefront partials
 * added in a fixed order, so results do not depend on timing.  The error against the exact product
 * is at most (2^-16.9 + (6 d_in + 16) 2^-24) times f16(norm_i) sum_k |c[idx_ik].x u_m,2k| +
 * |c.y u_m,2k+1| (measured: below 3e-6 of that sum).
 * Arguments:
 *   d_x, x_dtype, M, ld_x   M x d_in activations (QAMW_F32 or QAMW_BF16), row m at d_x + m ld_x.
 *                           1 <= M <= 16 (QAMW_ERR_UNSUPPORTED above; M = 0 is a no-op).
 *   d_codes ... block       as qamw_decode (any block size 2..1024 dividing d_in; bits <= 12;
 *                           d_out <= QAMW_MAX_ROWS; d_in <= QAMW_QGEMM_MAX_COLS, else
 *                           QAMW_ERR_UNSUPPORTED).
 *   d_y, y_dtype, ld_y      M x d_out outputs, y[m][i] at d_y + m ld_y (ld_y >= d_out); BF16 is the
 *                           fp32 result rounded to nearest even.
 *   d_ws, ws_bytes          at least qamw_qgemm_workspace(M, d_out, d_in) bytes, 256-byte aligned. */
#define QAMW_QGEMM_MAX_COLS (1 << 24)
size_t qamw_qgemm_workspace(int32_t M, int32_t d_out, int32_t d_in);
int qamw_qgemm(const void* d_x, qamw_dtype x_dtype, int32_t M, int64_t ld_x, const uint8_t* d_codes,
               const uint16_t* d_norm_f16, const float* d_sigma, const float* d_codebook, int32_t bits,
               const float* d_scale, int32_t d_out, int32_t d_in, int32_t block, uint64_t sign_seed,
               void* d_y, qamw_dtype y_dtype, int64_t ld_y, void* d_ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory or pass a workspace -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: qamw_qgemm without the d_ws /
 * ws_bytes arguments, same result bit for bit.  Its workspace is an array of
 * QAMW_QGEMM_NOALLOC_BYTES bytes that the library holds on each device from its first call there
 * until the process ends; the call itself allocates nothing.  Shapes whose qamw_qgemm_workspace
 * exceeds that size return QAMW_ERR_WORKSPACE (4 MiB covers d_in <= 65536 at any M <= 16).
 * `stream` must belong to the current device (NULL: its default stream); otherwise, or when the
 * array's address cannot be obtained, QAMW_ERR_HIP.  All calls on a device share its array: calls
 * that may run at the same time on one device (different streams, threads without ordering) race
 * on it and their results are undefined; calls queued on one stream are safe. */
#define QAMW_QGEMM_NOALLOC_BYTES (4u << 20)
int qamw_qgemm_noalloc(const void* d_x, qamw_dtype x_dtype, int32_t M, int64_t ld_x, const uint8_t* d_codes,
                       const uint16_t* d_norm_f16, const float* d_sigma, const float* d_codebook, int32_t bits,
                       const float* d_scale, int32_t d_out, int32_t d_in, int32_t block, uint64_t sign_seed,
                       void* d_y, qamw_dtype y_dtype, int64_t ld_y, void* stream);

/* Section 3.5 (the polar baseline QAM-W is compared with): a pair is coded as a magnitude level
 * times a phase.  The magnitude quantizer is the Na = 2^ba level Lloyd-Max quantizer of the unit
 * Rayleigh density r exp(-r^2/2) (the modulus of a circular standard Gaussian pair, the
 * distribution the rotated, sigma-scaled pairs follow by section 3.4): started from the
 * conditional means of Na equal-probability cells, thresholds at midpoints of adjacent levels and
 * levels at the conditional means of their cells, in fp64, until no level moves by more than
 * 1e-15 of itself or for 10000 rounds.  The phase has Np = 2^bp uniform bins centred on
 * 2 pi j / Np.  Writes, on the stream:
 *   d_levels      Na doubles, increasing;
 *   d_thresholds  Na - 1 doubles, t_i = (a_i + a_i+1) / 2;
 *   d_codebook    Na * Np interleaved fp32 pairs, entry ia + Na ip =
 *                 (fl32(a_ia cos(2 pi ip / Np)), fl32(a_ia sin(2 pi ip / Np))): the table that
 *                 qamw_decode reads with bits = ba + bp.
 * Limits: 1 <= ba <= 8, bp >= 1, ba + bp <= 12 (QAMW_ERR_UNSUPPORTED above, QAMW_ERR_ARG for
 * ba or bp < 1 or ba + bp > 16).  Device pointers, 8-byte aligned, owned by the caller. */
int qamw_polar_codebook(int32_t ba, int32_t bp, double* d_levels, double* d_thresholds, float* d_codebook,
                        void* stream);

/* Section 3.5: polar indices of n 2D points (fp32, interleaved) into d_idx (int32): the index
 * ia + Na ip that qamw_encode_polar gives a scaled pair (rule below), with the thresholds of
 * qamw_polar_codebook.  Limits as qamw_polar_codebook; d_status (may be NULL) receives
 * QAMW_FLAG_BAD_THRESHOLDS. */
int qamw_polar_index(const float* d_points, int64_t n, int32_t ba, int32_t bp, const double* d_thresholds,
                     int32_t* d_idx, int32_t* d_status, void* stream);

/* Section 3.5: the encoder of qamw_encode (same front end, calibration, norms, packing,
 * arguments and limits) with the polar quantizer in place of the nearest-codeword search.  With
 * p the scaled pair:
 *   ia = #{i : fl64(t_i^2) < fl64(px^2 + py^2)}                 (the nearest level)
 *   ip = floor(atan2(py, px) Np / (2 pi) + 1/2) mod Np          (the nearest bin centre),
 *        0 for a pair at the origin, decided up to rounding at a bin edge
 *   index = ia + Na ip, packed with bits = ba + bp.
 * d_thresholds: Na - 1 device doubles, finite, >= 0 and non-decreasing (as qamw_polar_codebook
 * writes them); otherwise QAMW_FLAG_BAD_THRESHOLDS is set and the indices are unspecified.
 * Decode with qamw_decode, the table of qamw_polar_codebook and bits = ba + bp. */
int qamw_encode_polar(const void* d_w, qamw_dtype w_dtype, int32_t d_out, int32_t d_in, int64_t ld_w,
                      const float* d_scale, int32_t block, uint64_t sign_seed, int32_t ba, int32_t bp,
                      const double* d_thresholds, const float* d_sigma_in, float* d_sigma_out,
                      uint16_t* d_norm_f16, uint8_t* d_codes, int32_t* d_status, void* d_ws, size_t ws_bytes,
                      void* stream);

/* The activation-aware per-channel scale (the AWQ-style scaling of the paper, motivated by the
 * layer-output trace identity ||X dW^T||_F^2 = Tr(dW X^T X dW^T)): from T calibration activation
 * rows X (T x d_in, QAMW_F32 or QAMW_BF16, leading dimension ld_x >= d_in),
 *   r_j = sqrt(sum_t x_tj^2 / T)   (fp64, fixed-order chunked sums: deterministic)
 *   s_j = fl32(r_j^alpha), or 1 for a channel that is zero over the batch,
 * written to d_scale (d_in fp32, the d_scale of qamw_encode / qamw_decode / qamw_qgemm) and, when
 * d_rms is not NULL, r to d_rms (d_in doubles).  The pages give s only up to a constant factor; a
 * global factor cancels between the row norm and the decoder's division, so none is applied.
 * alpha must be finite (the paper uses 0.3).  d_ws: at least qamw_act_scale_workspace(T, d_in)
 * bytes, 8-byte aligned.  T >= 1, d_in >= 1, else QAMW_ERR_ARG. */
size_t qamw_act_scale_workspace(int64_t T, int32_t d_in);
int qamw_act_scale(const void* d_x, qamw_dtype x_dtype, int64_t T, int32_t d_in, int64_t ld_x, double alpha,
                   float* d_scale, double* d_rms, void* d_ws, size_t ws_bytes, void* stream);

/* Section 2 (the scalar, d = 1, ablation that the paper names as its first follow-up): the same front
 * end, with each coordinate of the scaled pair coded alone by the L = 2^b level Lloyd-Max quantizer of
 * the standard normal density (the law of each coordinate of a unit circular Gaussian pair).  The
 * start is the conditional means of L equal-probability cells (edges at the normal quantiles, by
 * bisection); the rounds and the stopping rule are those of qamw_polar_codebook.  Writes:
 *   d_levels      L doubles, increasing (symmetric about 0);
 *   d_thresholds  L - 1 doubles, midpoints of adjacent levels;
 *   d_codebook    L * L interleaved fp32 pairs, entry ix + L iy = (fl32(a_ix), fl32(a_iy)): the
 *                 product table.  Nearest-codeword search over it (qamw_codebook_index +
 *                 qamw_encode with bits = 2b) gives each coordinate its nearest level (ties between
 *                 levels within fp32 rounding of the distance), and qamw_decode decodes it.
 * Limits: 1 <= b <= 6 (QAMW_ERR_UNSUPPORTED for 7 and 8, QAMW_ERR_ARG otherwise).  Device pointers,
 * 8-byte aligned, owned by the caller. */
int qamw_scalar_codebook(int32_t b, double* d_levels, double* d_thresholds, float* d_codebook, void* stream);

/* Human-readable text for a return code. */
const char* qamw_status_string(int code);

#ifdef __cplusplus
}
#endif
#endif /* QAMW_H */
