// C ABI of libqamw.so (declared in include/qamw.h).  Every argument is checked here, in host
// code, before anything is queued; then the kernels are launched on the caller's stream.
#include <mutex>
#include <vector>
#include <cmath>

#include "qamw.h"
#include "qamw_device.hpp"
#include "qamw_launch.hpp"

using namespace qamw;

namespace {

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int log2i(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Resolve and check the Hadamard block size; returns L = log2(b) or a negative error.
int check_shape(int32_t d_in, int32_t block) {
    if (d_in <= 0 || (d_in & 1)) return QAMW_ERR_ARG;
    int32_t b = block == 0 ? qamw_default_block(d_in) : block;
    if (b < 2 || b > 1024 || !is_pow2(b) || d_in % b) return QAMW_ERR_ARG;
    int L = log2i(b);
    int E = lane_elems(L);
    // one lane per E columns (whole lanes only), one workgroup per row: at most 1024 lanes (512
    // when E >= 32)
    if (E <= 0 || d_in % E || d_in / E > (E >= 32 ? 512 : 1024)) return QAMW_ERR_UNSUPPORTED;
    return L;
}

int check_bits(int32_t bits) {
    if (bits < 1 || bits > 16) return QAMW_ERR_ARG;
    if (bits > 12) return QAMW_ERR_UNSUPPORTED;
    return QAMW_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? QAMW_OK : QAMW_ERR_HIP; }

}  // namespace

namespace {

// The encoder common to QAM-W and the polar baseline: thr == nullptr selects the QAM-W search
// (d_codebook, d_index), else the polar quantizer (ba magnitude bits, thresholds thr).
int encode_common(const void* d_w, qamw_dtype w_dtype, int32_t d_out, int32_t d_in, int64_t ld_w,
                  const float* d_scale, int32_t block, uint64_t sign_seed, const float* d_codebook,
                  int32_t bits, const void* d_index, const double* thr, int32_t ba, const float* d_sigma_in,
                  float* d_sigma_out, uint16_t* d_norm_f16, uint8_t* d_codes, int32_t* d_status, void* d_ws,
                  size_t ws_bytes, void* stream) {
    if (d_out < 0 || (w_dtype != QAMW_F32 && w_dtype != QAMW_BF16)) return QAMW_ERR_ARG;
    if (d_out > QAMW_MAX_ROWS) return QAMW_ERR_UNSUPPORTED;
    int L = check_shape(d_in, block);
    if (L < 0) return L;
    int rc = check_bits(bits);
    if (rc) return rc;
    if (ld_w < d_in) return QAMW_ERR_ARG;
    if (encode_lds_bytes(L, bits, d_in, thr ? bits - ba : -1) > kLdsBytes) return QAMW_ERR_UNSUPPORTED;
    // whatever is encoded can be decoded: the decoder's limit applies here too
    if (decode_lds_bytes(L, bits, d_in) > kLdsBytes) return QAMW_ERR_UNSUPPORTED;
    if (!d_sigma_in && !d_sigma_out) return QAMW_ERR_ARG;
    if (d_out > 0 && (!d_w || !d_norm_f16 || !d_codes)) return QAMW_ERR_ARG;
    if (d_out > 0 && !thr && (!d_codebook || !d_index || !aligned(d_codebook, 8) || !aligned(d_index, 16)))
        return QAMW_ERR_ARG;
    if (d_out > 0 && thr && !aligned(thr, 8)) return QAMW_ERR_ARG;
    if (d_out > 0 && (!aligned(d_codes, 4) || !aligned(d_w, w_dtype == QAMW_BF16 ? 2 : 4) || !aligned(d_norm_f16, 2)))
        return QAMW_ERR_ARG;
    const bool calibrate = d_sigma_in == nullptr;
    if (calibrate && (!d_ws || !aligned(d_ws, 16) || ws_bytes < qamw_encode_workspace(d_out, d_in, bits)))
        return QAMW_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const float* sigma = d_sigma_in;
    if (calibrate) {
        CalibArgs c{};
        c.w = d_w;
        c.w_bf16 = w_dtype == QAMW_BF16;
        c.n_rows = d_out < 1024 ? d_out : 1024;
        c.d_in = d_in;
        c.ld = ld_w;
        c.scale = d_scale;
        c.sign_seed = sign_seed;
        c.n_groups = calib_groups(c.n_rows);
        const size_t part_bytes = (size_t)(c.n_groups > 0 ? c.n_groups : 1) * (size_t)(d_in / 2) * sizeof(double);
        c.partial = reinterpret_cast<double*>(d_ws);
        c.nz = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(d_ws) + (part_bytes + 255) / 256 * 256);
        hipError_t e = launch_calibrate(c, L, d_sigma_out, st);
        if (e != hipSuccess) return QAMW_ERR_HIP;
        sigma = d_sigma_out;
    } else if (d_sigma_out && d_sigma_out != d_sigma_in) {
        if (hipMemcpyAsync(d_sigma_out, d_sigma_in, sizeof(float) * (size_t)(d_in / 2), hipMemcpyDeviceToDevice, st) !=
            hipSuccess)
            return QAMW_ERR_HIP;
    }
    if (d_out == 0) return QAMW_OK;
    EncodeArgs a{};
    a.w = d_w;
    a.w_bf16 = w_dtype == QAMW_BF16;
    a.d_out = d_out;
    a.d_in = d_in;
    a.ld = ld_w;
    a.scale = d_scale;
    a.sign_seed = sign_seed;
    a.sigma = sigma;
    a.cb = d_codebook;
    a.bits = bits;
    a.index = d_index;
    a.index_g = index_grid_size(bits);
    a.thr = thr;
    a.ba = ba;
    a.norm = d_norm_f16;
    a.codes = d_codes;
    a.stride = qamw_row_stride(d_in, bits);
    a.status = d_status;
    return hip_rc(launch_encode(a, L, st));
}

}  // namespace

namespace {
int check_polar_bits(int32_t ba, int32_t bp) {
    if (ba < 1 || bp < 1 || ba + bp > 16) return QAMW_ERR_ARG;
    if (ba > kPolarMaxBa || ba + bp > 12) return QAMW_ERR_UNSUPPORTED;
    return QAMW_OK;
}
}  // namespace

extern "C" {

size_t qamw_row_stride(int32_t d_in, int32_t bits) {
    if (d_in <= 0 || (d_in & 1) || bits < 1 || bits > 16) return 0;
    size_t used = ((size_t)(d_in / 2) * (size_t)bits + 7) / 8;
    return (used + 15) / 16 * 16;
}

int32_t qamw_default_block(int32_t d_in) {
    if (d_in <= 0) return 0;
    int32_t b = 1;
    while (b < 1024 && d_in % (2 * b) == 0) b *= 2;
    return b;
}

size_t qamw_index_bytes(int32_t bits) {
    if (check_bits(bits) != QAMW_OK) return 0;
    return index_bytes_for(bits);
}

size_t qamw_encode_workspace(int32_t d_out, int32_t d_in, int32_t bits) {
    if (d_out < 0 || d_in <= 0 || (d_in & 1) || check_bits(bits) != QAMW_OK) return 0;
    return calib_workspace(d_out, d_in);
}

size_t qamw_train_workspace(int64_t n_points, int32_t bits) {
    if (n_points < 0 || check_bits(bits) != QAMW_OK) return 0;
    return lloyd_workspace(bits);
}

int qamw_codebook_train(const float* d_points, int64_t n_points, int32_t bits, int32_t iters, const float* d_init,
                        float* d_codebook, int64_t* d_err_trace, int32_t* d_status, void* d_ws, size_t ws_bytes,
                        void* stream) {
    int rc = check_bits(bits);
    if (rc) return rc;
    if (iters < 0 || !d_points || !d_codebook || n_points < ((int64_t)1 << bits)) return QAMW_ERR_ARG;
    if (!aligned(d_points, 8) || !aligned(d_codebook, 8) || (d_init && !aligned(d_init, 8))) return QAMW_ERR_ARG;
    if (!d_ws || !aligned(d_ws, 16) || ws_bytes < qamw_train_workspace(n_points, bits)) return QAMW_ERR_WORKSPACE;
    return hip_rc(launch_lloyd(d_points, n_points, bits, iters, d_init, d_codebook, d_err_trace, d_status, d_ws,
                               (hipStream_t)stream));
}

int qamw_codebook_index(const float* d_codebook, int32_t bits, void* d_index, size_t index_bytes, void* stream) {
    int rc = check_bits(bits);
    if (rc) return rc;
    if (!d_codebook || !aligned(d_codebook, 8)) return QAMW_ERR_ARG;
    if (!d_index || !aligned(d_index, 16) || index_bytes < qamw_index_bytes(bits)) return QAMW_ERR_WORKSPACE;
    return hip_rc(launch_index_build(d_codebook, bits, d_index, (hipStream_t)stream));
}

int qamw_nearest(const float* d_points, int64_t n, const float* d_codebook, int32_t bits, const void* d_index,
                 int32_t* d_idx, void* stream) {
    int rc = check_bits(bits);
    if (rc) return rc;
    if (n < 0) return QAMW_ERR_ARG;
    if (n == 0) return QAMW_OK;
    if (!d_points || !d_codebook || !d_index || !d_idx || !aligned(d_points, 8) || !aligned(d_codebook, 8) ||
        !aligned(d_index, 16))
        return QAMW_ERR_ARG;
    return hip_rc(launch_nearest(d_points, n, d_codebook, bits, d_index, d_idx, (hipStream_t)stream));
}

int qamw_encode(const void* d_w, qamw_dtype w_dtype, int32_t d_out, int32_t d_in, int64_t ld_w, const float* d_scale,
                int32_t block, uint64_t sign_seed, const float* d_codebook, int32_t bits, const void* d_index,
                const float* d_sigma_in, float* d_sigma_out, uint16_t* d_norm_f16, uint8_t* d_codes,
                int32_t* d_status, void* d_ws, size_t ws_bytes, void* stream) {
    return encode_common(d_w, w_dtype, d_out, d_in, ld_w, d_scale, block, sign_seed, d_codebook, bits, d_index,
                         nullptr, 0, d_sigma_in, d_sigma_out, d_norm_f16, d_codes, d_status, d_ws, ws_bytes, stream);
}

size_t qamw_qgemm_workspace(int32_t M, int32_t d_out, int32_t d_in) {
    if (M < 0 || d_out < 0 || d_in <= 0 || (d_in & 1)) return 0;
    return qgemm_workspace(M, d_out, d_in);
}

}  // extern "C"

namespace {

// The library's own workspace for qamw_qgemm_noalloc: one array per device, held until the process
// ends.  Host code never uses the name itself (on the host it only stands for the symbol): the
// device address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[QAMW_QGEMM_NOALLOC_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The array's address on the device of `stream` (which must be the current device), or nullptr.
void* scratch_address(hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    if (stream) {
        int sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// The checks of qamw_qgemm except the workspace's; QAMW_OK with *run = false when there is nothing
// to do.
int qgemm_check(const void* d_x, qamw_dtype x_dtype, int32_t M, int64_t ld_x, const uint8_t* d_codes,
                const uint16_t* d_norm_f16, const float* d_sigma, const float* d_codebook, int32_t bits, int32_t d_out,
                int32_t d_in, int32_t block, void* d_y, qamw_dtype y_dtype, int64_t ld_y, bool* run) {
    *run = false;
    if (M < 0 || d_out < 0 || (x_dtype != QAMW_F32 && x_dtype != QAMW_BF16) ||
        (y_dtype != QAMW_F32 && y_dtype != QAMW_BF16))
        return QAMW_ERR_ARG;
    if (d_out > QAMW_MAX_ROWS) return QAMW_ERR_UNSUPPORTED;
    if (d_in <= 0 || (d_in & 1)) return QAMW_ERR_ARG;
    const int32_t b = block == 0 ? qamw_default_block(d_in) : block;
    if (b < 2 || b > 1024 || !is_pow2(b) || d_in % b) return QAMW_ERR_ARG;
    int rc = check_bits(bits);
    if (rc) return rc;
    if (M > 16) return QAMW_ERR_UNSUPPORTED;
    // the product addresses a tile's codes and the B operands through 32-bit buffer offsets
    if (d_in > QAMW_QGEMM_MAX_COLS) return QAMW_ERR_UNSUPPORTED;
    if (ld_x < d_in || ld_y < d_out) return QAMW_ERR_ARG;
    if (M == 0 || d_out == 0) return QAMW_OK;
    if (!d_x || !d_codes || !d_norm_f16 || !d_sigma || !d_codebook || !d_y) return QAMW_ERR_ARG;
    if (!aligned(d_x, x_dtype == QAMW_BF16 ? 2 : 4) || !aligned(d_y, y_dtype == QAMW_BF16 ? 2 : 4) ||
        !aligned(d_codes, 4) || !aligned(d_codebook, 8) || !aligned(d_norm_f16, 2))
        return QAMW_ERR_ARG;
    *run = true;
    return QAMW_OK;
}

// Queues the product with its workspace at d_ws (checked by the caller).
int qgemm_run(const void* d_x, qamw_dtype x_dtype, int32_t M, int64_t ld_x, const uint8_t* d_codes,
              const uint16_t* d_norm_f16, const float* d_sigma, const float* d_codebook, int32_t bits,
              const float* d_scale, int32_t d_out, int32_t d_in, int32_t block, uint64_t sign_seed, void* d_y,
              qamw_dtype y_dtype, int64_t ld_y, void* d_ws, hipStream_t stream) {
    QgemmArgs a{};
    a.codes = d_codes;
    a.stride = qamw_row_stride(d_in, bits);
    a.norm = d_norm_f16;
    a.cb = d_codebook;
    a.bits = bits;
    a.u = reinterpret_cast<float*>(d_ws);
    a.M = M;
    a.n_pairs = d_in / 2;
    a.d_out = d_out;
    a.y = d_y;
    a.y_bf16 = y_dtype == QAMW_BF16;
    a.ld_y = ld_y;
    QgemmRotateArgs r{};
    r.x = d_x;
    r.x_bf16 = x_dtype == QAMW_BF16;
    r.ld_x = ld_x;
    r.d_in = d_in;
    r.block = block == 0 ? qamw_default_block(d_in) : block;
    r.scale = d_scale;
    r.sign_seed = sign_seed;
    r.sigma = d_sigma;
    return hip_rc(launch_qgemm(a, r, stream));
}

}  // namespace

extern "C" {

int qamw_qgemm(const void* d_x, qamw_dtype x_dtype, int32_t M, int64_t ld_x, const uint8_t* d_codes,
               const uint16_t* d_norm_f16, const float* d_sigma, const float* d_codebook, int32_t bits,
               const float* d_scale, int32_t d_out, int32_t d_in, int32_t block, uint64_t sign_seed,
               void* d_y, qamw_dtype y_dtype, int64_t ld_y, void* d_ws, size_t ws_bytes, void* stream) {
    bool run = false;
    const int rc = qgemm_check(d_x, x_dtype, M, ld_x, d_codes, d_norm_f16, d_sigma, d_codebook, bits, d_out, d_in,
                               block, d_y, y_dtype, ld_y, &run);
    if (rc || !run) return rc;
    if (!d_ws || !aligned(d_ws, 256) || ws_bytes < qamw_qgemm_workspace(M, d_out, d_in)) return QAMW_ERR_WORKSPACE;
    return qgemm_run(d_x, x_dtype, M, ld_x, d_codes, d_norm_f16, d_sigma, d_codebook, bits, d_scale, d_out, d_in,
                     block, sign_seed, d_y, y_dtype, ld_y, d_ws, (hipStream_t)stream);
}

int qamw_qgemm_noalloc(const void* d_x, qamw_dtype x_dtype, int32_t M, int64_t ld_x, const uint8_t* d_codes,
                       const uint16_t* d_norm_f16, const float* d_sigma, const float* d_codebook, int32_t bits,
                       const float* d_scale, int32_t d_out, int32_t d_in, int32_t block, uint64_t sign_seed,
                       void* d_y, qamw_dtype y_dtype, int64_t ld_y, void* stream) {
    bool run = false;
    const int rc = qgemm_check(d_x, x_dtype, M, ld_x, d_codes, d_norm_f16, d_sigma, d_codebook, bits, d_out, d_in,
                               block, d_y, y_dtype, ld_y, &run);
    if (rc || !run) return rc;
    if (qamw_qgemm_workspace(M, d_out, d_in) > QAMW_QGEMM_NOALLOC_BYTES) return QAMW_ERR_WORKSPACE;
    void* ws = scratch_address((hipStream_t)stream);
    if (!ws) return QAMW_ERR_HIP;
    // nothing in the workspace has to start at zero: every word the product reads was written
    // earlier in the same call
    return qgemm_run(d_x, x_dtype, M, ld_x, d_codes, d_norm_f16, d_sigma, d_codebook, bits, d_scale, d_out, d_in,
                     block, sign_seed, d_y, y_dtype, ld_y, ws, (hipStream_t)stream);
}

int qamw_polar_codebook(int32_t ba, int32_t bp, double* d_levels, double* d_thresholds, float* d_codebook,
                        void* stream) {
    int rc = check_polar_bits(ba, bp);
    if (rc) return rc;
    if (!d_levels || !d_thresholds || !d_codebook || !aligned(d_levels, 8) || !aligned(d_thresholds, 8) ||
        !aligned(d_codebook, 8))
        return QAMW_ERR_ARG;
    return hip_rc(launch_polar_codebook(ba, bp, d_levels, d_thresholds, d_codebook, (hipStream_t)stream));
}

size_t qamw_act_scale_workspace(int64_t T, int32_t d_in) {
    if (T < 1 || d_in < 1) return 0;
    return (size_t)act_chunks(T) * (size_t)d_in * sizeof(double);
}

int qamw_act_scale(const void* d_x, qamw_dtype x_dtype, int64_t T, int32_t d_in, int64_t ld_x, double alpha,
                   float* d_scale, double* d_rms, void* d_ws, size_t ws_bytes, void* stream) {
    if (T < 1 || d_in < 1 || ld_x < d_in || (x_dtype != QAMW_F32 && x_dtype != QAMW_BF16) || !std::isfinite(alpha))
        return QAMW_ERR_ARG;
    if (!d_x || !d_scale || !aligned(d_x, x_dtype == QAMW_BF16 ? 2 : 4) || !aligned(d_scale, 4) ||
        (d_rms && !aligned(d_rms, 8)))
        return QAMW_ERR_ARG;
    if (!d_ws || !aligned(d_ws, 8) || ws_bytes < qamw_act_scale_workspace(T, d_in)) return QAMW_ERR_WORKSPACE;
    return hip_rc(launch_act_scale(d_x, x_dtype == QAMW_BF16, T, d_in, ld_x, alpha, d_scale, d_rms,
                                   reinterpret_cast<double*>(d_ws), (hipStream_t)stream));
}

int qamw_scalar_codebook(int32_t b, double* d_levels, double* d_thresholds, float* d_codebook, void* stream) {
    if (b < 1 || b > 8) return QAMW_ERR_ARG;
    if (b > 6) return QAMW_ERR_UNSUPPORTED;
    if (!d_levels || !d_thresholds || !d_codebook || !aligned(d_levels, 8) || !aligned(d_thresholds, 8) ||
        !aligned(d_codebook, 8))
        return QAMW_ERR_ARG;
    return hip_rc(launch_scalar_codebook(b, d_levels, d_thresholds, d_codebook, (hipStream_t)stream));
}

int qamw_polar_index(const float* d_points, int64_t n, int32_t ba, int32_t bp, const double* d_thresholds,
                     int32_t* d_idx, int32_t* d_status, void* stream) {
    int rc = check_polar_bits(ba, bp);
    if (rc) return rc;
    if (n < 0) return QAMW_ERR_ARG;
    if (n == 0) return QAMW_OK;
    if (!d_points || !d_thresholds || !d_idx || !aligned(d_points, 8) || !aligned(d_thresholds, 8) ||
        !aligned(d_idx, 4))
        return QAMW_ERR_ARG;
    return hip_rc(launch_polar_index(d_points, n, ba, bp, d_thresholds, d_idx, d_status, (hipStream_t)stream));
}

int qamw_encode_polar(const void* d_w, qamw_dtype w_dtype, int32_t d_out, int32_t d_in, int64_t ld_w,
                      const float* d_scale, int32_t block, uint64_t sign_seed, int32_t ba, int32_t bp,
                      const double* d_thresholds, const float* d_sigma_in, float* d_sigma_out,
                      uint16_t* d_norm_f16, uint8_t* d_codes, int32_t* d_status, void* d_ws, size_t ws_bytes,
                      void* stream) {
    int rc = check_polar_bits(ba, bp);
    if (rc) return rc;
    if (!d_thresholds) return QAMW_ERR_ARG;
    return encode_common(d_w, w_dtype, d_out, d_in, ld_w, d_scale, block, sign_seed, nullptr, ba + bp, nullptr,
                         d_thresholds, ba, d_sigma_in, d_sigma_out, d_norm_f16, d_codes, d_status, d_ws, ws_bytes,
                         stream);
}

}  // extern "C"

namespace {

// The checks of qamw_decode; fills *a and *L (log2 of the block) when the call is valid.
int decode_check(const uint8_t* d_codes, const uint16_t* d_norm_f16, const float* d_sigma, const float* d_codebook,
                 int32_t bits, const float* d_scale, int32_t d_out, int32_t d_in, int32_t block, uint64_t sign_seed,
                 void* d_out_w, qamw_dtype out_dtype, int64_t ld_out, qamw::DecodeArgs* a, int* L) {
    using namespace qamw;
    if (d_out < 0 || (out_dtype != QAMW_F32 && out_dtype != QAMW_BF16)) return QAMW_ERR_ARG;
    if (d_out > QAMW_MAX_ROWS) return QAMW_ERR_UNSUPPORTED;
    *L = check_shape(d_in, block);
    if (*L < 0) return *L;
    int rc = check_bits(bits);
    if (rc) return rc;
    if (ld_out < d_in || (ld_out & 1)) return QAMW_ERR_ARG;
    if (decode_lds_bytes(*L, bits, d_in) > kLdsBytes) return QAMW_ERR_UNSUPPORTED;
    if (d_out == 0) {
        a->d_out = 0;
        return QAMW_OK;
    }
    if (!d_codes || !d_norm_f16 || !d_sigma || !d_codebook || !d_out_w) return QAMW_ERR_ARG;
    if (!aligned(d_codebook, 8) || !aligned(d_codes, 4) || !aligned(d_norm_f16, 2) ||
        !aligned(d_out_w, out_dtype == QAMW_BF16 ? 4 : 8))
        return QAMW_ERR_ARG;
    *a = DecodeArgs{};
    a->codes = d_codes;
    a->stride = qamw_row_stride(d_in, bits);
    a->norm = d_norm_f16;
    a->sigma = d_sigma;
    a->cb = d_codebook;
    a->bits = bits;
    a->scale = d_scale;
    a->sign_seed = sign_seed;
    a->d_out = d_out;
    a->d_in = d_in;
    a->out = d_out_w;
    a->out_bf16 = out_dtype == QAMW_BF16;
    a->ld = ld_out;
    return QAMW_OK;
}

}  // namespace

extern "C" {

int qamw_decode(const uint8_t* d_codes, const uint16_t* d_norm_f16, const float* d_sigma, const float* d_codebook,
                int32_t bits, const float* d_scale, int32_t d_out, int32_t d_in, int32_t block, uint64_t sign_seed,
                void* d_out_w, qamw_dtype out_dtype, int64_t ld_out, void* stream) {
    DecodeArgs a{};
    int L = 0;
    const int rc = decode_check(d_codes, d_norm_f16, d_sigma, d_codebook, bits, d_scale, d_out, d_in, block, sign_seed,
                                d_out_w, out_dtype, ld_out, &a, &L);
    if (rc || d_out == 0) return rc;
    return hip_rc(launch_decode(a, L, (hipStream_t)stream));
}

int qamw_decode_many(const qamw_decode_job* jobs, int32_t n_jobs, const float* d_codebook, int32_t bits,
                     int32_t block, qamw_dtype out_dtype, void* stream) {
    if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return QAMW_ERR_ARG;
    std::vector<DecodeArgs> args;
    std::vector<int> ls;
    args.reserve((size_t)n_jobs);
    ls.reserve((size_t)n_jobs);
    for (int i = 0; i < n_jobs; ++i) {   // every job is checked before anything is queued
        const qamw_decode_job& j = jobs[i];
        DecodeArgs a{};
        int L = 0;
        const int rc = decode_check(j.d_codes, j.d_norm_f16, j.d_sigma, d_codebook, bits, j.d_scale, j.d_out, j.d_in,
                                    block, j.sign_seed, j.d_out_w, out_dtype, j.ld_out, &a, &L);
        if (rc) return rc;
        if (j.d_out == 0) continue;
        args.push_back(a);
        ls.push_back(L);
    }
    const hipStream_t st = (hipStream_t)stream;
    size_t i = 0;
    while (i < args.size()) {
        if (!decode128_supported(args[i], ls[i])) {
            const int rc = hip_rc(launch_decode(args[i], ls[i], st));
            if (rc) return rc;
            ++i;
            continue;
        }
        size_t k = i;   // a run of jobs the grouped 128-column decoder takes
        while (k < args.size() && decode128_supported(args[k], ls[k])) ++k;
        const int rc = hip_rc(launch_decode128_many(args.data() + i, ls.data() + i, (int)(k - i), st));
        if (rc) return rc;
        i = k;
    }
    return QAMW_OK;
}

int qamw_sign_mask(uint64_t sign_seed, int32_t d_in, uint32_t* d_bits, void* stream) {
    if (d_in < 0) return QAMW_ERR_ARG;
    if (d_in == 0) return QAMW_OK;
    if (!d_bits || !aligned(d_bits, 4)) return QAMW_ERR_ARG;
    return hip_rc(launch_sign_mask(sign_seed, d_in, d_bits, (hipStream_t)stream));
}

const char* qamw_status_string(int code) {
    switch (code) {
    case QAMW_OK: return "ok";
    case QAMW_ERR_ARG: return "invalid argument";
    case QAMW_ERR_UNSUPPORTED: return "unsupported shape or codebook size";
    case QAMW_ERR_WORKSPACE: return "workspace or index buffer too small";
    case QAMW_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

}  // extern "C"
