// C ABI of the unified-FP8 linear layer: host-side validation and dispatch.
//
// Every entry point checks its arguments on the host first and returns a
// status without touching the device when they are invalid; only then does it
// enqueue kernels on the caller's stream.  No memory is allocated and no state
// is kept between calls.
#include "../../include/fp8w8a8.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "kernels.hpp"

namespace {

constexpr int64_t kMaxDim = INT32_MAX;  // kernels index rows and columns with 32-bit ints
constexpr size_t kAlign = 256;          // workspace sub-buffer alignment
constexpr int64_t kMaxTiles = INT32_MAX - 8;  // launch grids count output tiles in 32 bits

// Output tiles of 128 x 128 (no GEMM kernel uses smaller tiles along both axes
// with one workgroup each), bounded so every grid and tile index fits 32 bits.
bool tiles_ok(int64_t row_tiles, int64_t N) { return row_tiles * ((N + 127) / 128) <= kMaxTiles; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// a * b without int64 overflow (a, b >= 0)
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

fp8_status_t check_dims(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return FP8_ERR_INVALID_ARGUMENT;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8_ERR_UNSUPPORTED;
    if (K % 16 != 0) return FP8_ERR_UNSUPPORTED;
    if (!tiles_ok((M + 127) / 128, N)) return FP8_ERR_UNSUPPORTED;
    return FP8_OK;
}

// A row-major matrix argument: rows x cols elements of `elem` bytes, stride
// ld.  Input operands are read in 16-byte pieces, so their row stride must be
// a multiple of 16 bytes (strided_ok = false); the BF16 output may have any
// row stride (strided_ok = true).
fp8_status_t check_matrix(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t elem,
                          bool strided_ok = false) {
    if (rows > 0 && cols > 0 && p == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (rows > 0 && ld < cols) return FP8_ERR_INVALID_ARGUMENT;
    int64_t span, bytes;
    if (!mul_ok(rows, ld, &span) || !mul_ok(span, elem, &bytes)) return FP8_ERR_INVALID_ARGUMENT;
    if (rows > 0 && cols > 0) {
        if (!aligned16(p)) return FP8_ERR_UNSUPPORTED;
        if (!strided_ok && (ld * elem) % 16 != 0) return FP8_ERR_UNSUPPORTED;
    }
    return FP8_OK;
}

fp8_status_t check_vector(const void* p, int64_t n) {
    if (n > 0 && p == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (n > 0 && !aligned16(p)) return FP8_ERR_UNSUPPORTED;
    return FP8_OK;
}

#define FP8_TRY(expr)                          \
    do {                                       \
        fp8_status_t s_ = (expr);              \
        if (s_ != FP8_OK) return s_;           \
    } while (0)

static_assert(FP8_KV_E4M3 == fp8k::kKvE4M3 && FP8_KV_E5M2 == fp8k::kKvE5M2, "KV format ids");
static_assert(FP8_KV_F32 == fp8k::kKvF32 && FP8_KV_BF16 == fp8k::kKvBF16 && FP8_KV_F16 == fp8k::kKvF16, "KV dtype ids");

// KV batch extents: C channels in groups of 4 (one 32-bit word of codes).
fp8_status_t check_kv_dims(int64_t T, int64_t C) {
    if (T < 0 || C < 0) return FP8_ERR_INVALID_ARGUMENT;
    if (T > kMaxDim || C > kMaxDim) return FP8_ERR_UNSUPPORTED;
    if (C % 4 != 0) return FP8_ERR_UNSUPPORTED;
    return FP8_OK;
}

fp8_status_t check_kv_format(fp8_kv_format_t fmt) {
    return (fmt == FP8_KV_E4M3 || fmt == FP8_KV_E5M2) ? FP8_OK : FP8_ERR_INVALID_ARGUMENT;
}

// Element size of a KV row type, 0 when the type is unknown.
int64_t kv_elem_bytes(fp8_kv_dtype_t t) {
    switch (t) {
        case FP8_KV_F32: return 4;
        case FP8_KV_BF16:
        case FP8_KV_F16: return 2;
    }
    return 0;
}

// Element size of a KV row type and the channel rule that goes with it:
// 16-bit rows are read 8 channels (16 bytes) per thread, so C % 8 == 0.
fp8_status_t kv_row_type(fp8_kv_dtype_t t, int64_t C, int64_t* eb) {
    *eb = kv_elem_bytes(t);
    if (*eb == 0) return FP8_ERR_INVALID_ARGUMENT;
    if (*eb == 2 && C % 8 != 0) return FP8_ERR_UNSUPPORTED;
    return FP8_OK;
}

fp8_status_t from_hip(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_DEVICE; }

// Bytes the GEMM path itself needs for an M x N x K problem: the skinny
// kernel's fp32 split-k partial sums when it splits k, else none.
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
    return M <= fp8k::kSkinnyMaxM ? round_up(fp8k::gemm_skinny_ws_bytes(M, N, K), kAlign) : 0;
}

// Bytes the fused path stages its activation codes and scales in.
size_t fused_stage_bytes(int64_t M, int64_t K) {
    return round_up((size_t)M * (size_t)K, kAlign) + round_up((size_t)M * sizeof(float), kAlign);
}

// BF16 output to y, or (y32 != nullptr) the fp32 value before rounding to y32.
fp8_status_t gemm_dispatch(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw, int64_t ldw,
                           const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int64_t M, int64_t N, int64_t K,
                           void* ws, hipStream_t stream) {
    if (M <= fp8k::kSkinnyMaxM)
        return from_hip(fp8k::launch_gemm_skinny(qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, ws, stream));
    if (K % 128 == 0)
        return from_hip(fp8k::launch_gemm_mfma(qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, stream));
    return from_hip(fp8k::launch_gemm_tiled(qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, stream));
}

// Bytes of the fp32 output staged by the FP8-output GEMM.
size_t fp8out_stage_bytes(int64_t M, int64_t N) { return round_up((size_t)M * (size_t)N * sizeof(float), kAlign); }

}  // namespace

extern "C" {

const char* fp8_status_string(fp8_status_t status) {
    switch (status) {
        case FP8_OK: return "FP8_OK";
        case FP8_ERR_INVALID_ARGUMENT: return "FP8_ERR_INVALID_ARGUMENT";
        case FP8_ERR_UNSUPPORTED: return "FP8_ERR_UNSUPPORTED";
        case FP8_ERR_WORKSPACE: return "FP8_ERR_WORKSPACE";
        case FP8_ERR_DEVICE: return "FP8_ERR_DEVICE";
    }
    return "FP8_ERR_UNKNOWN";
}

size_t fp8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_dims(M, N, K) == FP8_ERR_INVALID_ARGUMENT) return SIZE_MAX;
    int64_t mk;
    if (!mul_ok(M, K, &mk)) return SIZE_MAX;
    return fused_stage_bytes(M, K) + gemm_ws_bytes(M, N, K);
}

size_t fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_dims(M, N, K) == FP8_ERR_INVALID_ARGUMENT) return SIZE_MAX;
    return gemm_ws_bytes(M, N, K);
}

size_t fp8_fp8out_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_dims(M, N, K) == FP8_ERR_INVALID_ARGUMENT) return SIZE_MAX;
    int64_t mn;
    if (!mul_ok(M, N, &mn) || mn > INT64_MAX / 8) return SIZE_MAX;
    return fp8out_stage_bytes(M, N) + gemm_ws_bytes(M, N, K);
}

size_t fp8_grouped_workspace_bytes(int64_t T, int64_t R, int64_t E, int64_t N, int64_t K) {
    if (T < 0 || R < 0 || E < 0 || N < 0 || K < 0) return SIZE_MAX;
    return 0;
}

fp8_status_t fp8_quantize_per_token(const float* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* q,
                                    int64_t ldq, float* scales, hipStream_t stream) {
    FP8_TRY(check_dims(rows, 1, K));
    FP8_TRY(check_matrix(x, rows, K, ldx, 4));
    FP8_TRY(check_matrix(q, rows, K, ldq, 1));
    FP8_TRY(check_vector(scales, rows));
    if (rows == 0) return FP8_OK;
    return from_hip(fp8k::launch_quantize_rows(x, ldx, q, ldq, scales, rows, K, stream));
}

fp8_status_t fp8_quantize_static(const float* x, int64_t rows, int64_t K, int64_t ldx, const float* scale,
                                 uint8_t* q, int64_t ldq, float* scales_out, hipStream_t stream) {
    FP8_TRY(check_dims(rows, 1, K));
    FP8_TRY(check_matrix(x, rows, K, ldx, 4));
    FP8_TRY(check_matrix(q, rows, K, ldq, 1));
    FP8_TRY(check_vector(scales_out, rows));
    if (rows > 0 && scale == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (rows > 0 && (reinterpret_cast<uintptr_t>(scale) & 3u) != 0) return FP8_ERR_UNSUPPORTED;
    if (rows == 0) return FP8_OK;
    return from_hip(fp8k::launch_quantize_static(x, ldx, scale, q, ldq, scales_out, rows, K, stream));
}

fp8_status_t fp8_quantize_per_token_clipped(const float* x, int64_t rows, int64_t K, int64_t ldx, const float* clip,
                                            uint8_t* q, int64_t ldq, float* scales, hipStream_t stream) {
    FP8_TRY(check_dims(rows, 1, K));
    FP8_TRY(check_matrix(x, rows, K, ldx, 4));
    FP8_TRY(check_matrix(q, rows, K, ldq, 1));
    FP8_TRY(check_vector(scales, rows));
    if (rows > 0 && clip == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (rows > 0 && (reinterpret_cast<uintptr_t>(clip) & 3u) != 0) return FP8_ERR_UNSUPPORTED;
    if (rows == 0) return FP8_OK;
    return from_hip(fp8k::launch_quantize_clipped(x, ldx, clip, q, ldq, scales, rows, K, stream));
}

size_t fp8_calibrate_workspace_bytes(void) { return fp8k::kCalibrateWsBytes; }

fp8_status_t fp8_calibrate_percentile(const float* x, int64_t n, int64_t num, int64_t den, float* value_out,
                                      float* scale_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (n <= 0 || num <= 0 || den <= 0 || num > den) return FP8_ERR_INVALID_ARGUMENT;
    if (n > (int64_t)UINT32_MAX) return FP8_ERR_UNSUPPORTED;  // 32-bit histogram bins
    if (x == nullptr || value_out == nullptr || ws == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(x) & 3u) != 0 || (reinterpret_cast<uintptr_t>(value_out) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(scale_out) & 3u) != 0)
        return FP8_ERR_UNSUPPORTED;
    if (!aligned16(ws)) return FP8_ERR_UNSUPPORTED;
    if (ws_bytes < fp8k::kCalibrateWsBytes) return FP8_ERR_WORKSPACE;
    // nearest rank: ceil(num * n / den), exact in 128-bit integers
    const unsigned __int128 prod = (unsigned __int128)num * (unsigned __int128)n;
    int64_t rank = (int64_t)((prod + (unsigned __int128)(den - 1)) / (unsigned __int128)den);
    if (rank < 1) rank = 1;
    if (rank > n) rank = n;
    return from_hip(fp8k::launch_calibrate_percentile(x, n, rank, value_out, scale_out, ws, stream));
}

fp8_status_t fp8_quantize_mx(const float* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                             uint8_t* scales, hipStream_t stream) {
    FP8_TRY(check_dims(rows, 1, K));
    if (K % 128 != 0) return FP8_ERR_UNSUPPORTED;
    FP8_TRY(check_matrix(x, rows, K, ldx, 4));
    FP8_TRY(check_matrix(q, rows, K, ldq, 1));
    FP8_TRY(check_matrix(scales, K / 128, 4 * rows, 4 * rows, 1, true));
    if (rows == 0 || K == 0) return FP8_OK;
    return from_hip(fp8k::launch_quantize_mx(x, ldx, q, ldq, scales, rows, K, stream));
}

// The block-scaled GEMM's workspace: the skinny kernel's split-K partial
// sums (M <= 64); none for the MFMA kernel.
static size_t mx_ws_bytes(int64_t M, int64_t N, int64_t K) { return gemm_ws_bytes(M, N, K); }

size_t fp8_mx_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_dims(M, N, K) != FP8_OK || K % 128 != 0) return SIZE_MAX;
    return mx_ws_bytes(M, N, K);
}

fp8_status_t fp8_gemm_mx(const uint8_t* qa, int64_t lda, const uint8_t* sa, const uint8_t* qw, int64_t ldw,
                         const uint8_t* sw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
    FP8_TRY(check_dims(M, N, K));
    if (K % 128 != 0) return FP8_ERR_UNSUPPORTED;
    FP8_TRY(check_matrix(qa, M, K, lda, 1));
    FP8_TRY(check_matrix(qw, N, K, ldw, 1));
    FP8_TRY(check_matrix(y, M, N, ldy, 2, true));
    // block scales: unit-stride rows of K / 32 bytes, read as 32-bit words
    if (M > 0 && N > 0 && K > 0) {
        if (qa == nullptr || qw == nullptr || sa == nullptr || sw == nullptr) return FP8_ERR_INVALID_ARGUMENT;
        if ((reinterpret_cast<uintptr_t>(sa) & 3u) != 0 || (reinterpret_cast<uintptr_t>(sw) & 3u) != 0)
            return FP8_ERR_UNSUPPORTED;
    }
    const size_t need = mx_ws_bytes(M, N, K);
    if (ws_bytes < need) return FP8_ERR_WORKSPACE;
    if (need > 0 && ws == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (need > 0 && !aligned16(ws)) return FP8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8_OK;
    if (M <= fp8k::kSkinnyMaxM)
        return from_hip(fp8k::launch_gemm_skinny_mx(qa, lda, sa, qw, ldw, sw, y, ldy, M, N, K, ws, stream));
    return from_hip(fp8k::launch_gemm_mfma_mx(qa, lda, sa, qw, ldw, sw, y, ldy, M, N, K, stream));
}

size_t fp8_kv_scales_workspace_bytes(int64_t T, int64_t C) {
    if (check_kv_dims(T, C) != FP8_OK) return SIZE_MAX;
    return round_up(fp8k::kv_scales_ws_bytes(T, C), kAlign);
}

fp8_status_t fp8_kv_channel_scales(const void* kv, fp8_kv_dtype_t kv_dtype, int64_t T, int64_t C, int64_t ldkv,
                                   fp8_kv_format_t fmt, float* scales, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
    FP8_TRY(check_kv_dims(T, C));
    FP8_TRY(check_kv_format(fmt));
    int64_t eb = 0;
    FP8_TRY(kv_row_type(kv_dtype, C, &eb));
    FP8_TRY(check_matrix(kv, T, C, ldkv, eb));
    FP8_TRY(check_vector(scales, C));
    if (C == 0) return FP8_OK;
    const size_t need = round_up(fp8k::kv_scales_ws_bytes(T, C), kAlign);
    if (ws_bytes < need) return FP8_ERR_WORKSPACE;
    if (ws == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (!aligned16(ws)) return FP8_ERR_UNSUPPORTED;
    return from_hip(fp8k::launch_kv_channel_scales(kv, (int)kv_dtype, T, C, ldkv, (int)fmt, scales, ws, stream));
}

fp8_status_t fp8_kv_quantize_paged(const void* kv, fp8_kv_dtype_t kv_dtype, int64_t T, int64_t C, int64_t ldkv,
                                   const float* scales, fp8_kv_format_t fmt, const int32_t* slot_mapping,
                                   uint8_t* cache, int64_t num_slots, hipStream_t stream) {
    FP8_TRY(check_kv_dims(T, C));
    FP8_TRY(check_kv_format(fmt));
    int64_t eb = 0;
    FP8_TRY(kv_row_type(kv_dtype, C, &eb));
    if (num_slots < 0) return FP8_ERR_INVALID_ARGUMENT;
    if (num_slots > kMaxDim) return FP8_ERR_UNSUPPORTED;
    FP8_TRY(check_matrix(kv, T, C, ldkv, eb));
    FP8_TRY(check_vector(scales, T > 0 ? C : 0));
    FP8_TRY(check_matrix(cache, num_slots, C, C, 1, true));
    if (T > 0 && slot_mapping == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (T > 0 && (reinterpret_cast<uintptr_t>(slot_mapping) & 3u) != 0) return FP8_ERR_UNSUPPORTED;
    if (T == 0 || C == 0 || num_slots == 0) return FP8_OK;
    return from_hip(fp8k::launch_kv_quantize_paged(kv, (int)kv_dtype, T, C, ldkv, scales, (int)fmt, slot_mapping,
                                                   cache, num_slots, stream));
}

fp8_status_t fp8_kv_dequantize_paged(const uint8_t* cache, int64_t num_slots, const int32_t* slot_mapping,
                                     int64_t T, int64_t C, const float* scales, fp8_kv_format_t fmt, void* out,
                                     fp8_kv_dtype_t out_dtype, int64_t ldo, hipStream_t stream) {
    FP8_TRY(check_kv_dims(T, C));
    FP8_TRY(check_kv_format(fmt));
    int64_t eb = 0;
    FP8_TRY(kv_row_type(out_dtype, C, &eb));
    if (num_slots < 0) return FP8_ERR_INVALID_ARGUMENT;
    if (num_slots > kMaxDim) return FP8_ERR_UNSUPPORTED;
    FP8_TRY(check_matrix(cache, num_slots, C, C, 1, true));
    FP8_TRY(check_matrix(out, T, C, ldo, eb));
    FP8_TRY(check_vector(scales, T > 0 ? C : 0));
    if (T > 0 && slot_mapping == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (T > 0 && (reinterpret_cast<uintptr_t>(slot_mapping) & 3u) != 0) return FP8_ERR_UNSUPPORTED;
    if (T == 0 || C == 0) return FP8_OK;
    return from_hip(fp8k::launch_kv_dequantize_paged(cache, num_slots, slot_mapping, T, C, scales, (int)fmt, out,
                                                     (int)out_dtype, ldo, stream));
}

fp8_status_t fp8_gemm_scaled(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw,
                             int64_t ldw, const float* s_ch, uint16_t* y, int64_t ldy, int64_t M, int64_t N,
                             int64_t K, void* ws, size_t ws_bytes, hipStream_t stream) {
    FP8_TRY(check_dims(M, N, K));
    FP8_TRY(check_matrix(qa, M, K, lda, 1));
    FP8_TRY(check_matrix(qw, N, K, ldw, 1));
    FP8_TRY(check_vector(s_tok, M));
    FP8_TRY(check_vector(s_ch, N));
    FP8_TRY(check_matrix(y, M, N, ldy, 2, true));
    // operands are read only when the output is non-empty
    if (M > 0 && N > 0 && K > 0 && (qa == nullptr || qw == nullptr)) return FP8_ERR_INVALID_ARGUMENT;
    const size_t need = gemm_ws_bytes(M, N, K);
    if (ws_bytes < need) return FP8_ERR_WORKSPACE;
    if (need > 0 && ws == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (need > 0 && !aligned16(ws)) return FP8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8_OK;
    return gemm_dispatch(qa, lda, s_tok, qw, ldw, s_ch, y, nullptr, ldy, M, N, K, ws, stream);
}

fp8_status_t fp8_quant_gemm_fused(const float* x, int64_t ldx, const uint8_t* qw, int64_t ldw,
                                  const float* s_ch, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                  uint8_t* qa_out, float* s_tok_out, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
    FP8_TRY(check_dims(M, N, K));
    FP8_TRY(check_matrix(x, M, K, ldx, 4));
    FP8_TRY(check_matrix(qw, N, K, ldw, 1));
    FP8_TRY(check_vector(s_ch, N));
    FP8_TRY(check_matrix(y, M, N, ldy, 2, true));
    if (qa_out) FP8_TRY(check_matrix(qa_out, M, K, K, 1));
    if (s_tok_out) FP8_TRY(check_vector(s_tok_out, M));
    if (M > 0 && N > 0 && K > 0 && qw == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    const size_t need = fp8_workspace_bytes(M, N, K);
    if (ws_bytes < need) return FP8_ERR_WORKSPACE;
    if (need > 0 && ws == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (need > 0 && !aligned16(ws)) return FP8_ERR_UNSUPPORTED;
    if (M == 0) return FP8_OK;
    if (N > 0 && fp8k::gemm_skinny_fused_fits(M, N, K))
        return from_hip(fp8k::launch_gemm_skinny_fused(x, ldx, qw, ldw, s_ch, y, ldy, M, N, K, qa_out, s_tok_out,
                                                       stream));
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint8_t* qa = qa_out ? qa_out : base;
    float* s_tok = s_tok_out ? s_tok_out : reinterpret_cast<float*>(base + round_up((size_t)M * (size_t)K, kAlign));
    FP8_TRY(from_hip(fp8k::launch_quantize_rows(x, ldx, qa, K, s_tok, M, K, stream)));
    if (N == 0) return FP8_OK;
    return gemm_dispatch(qa, K, s_tok, qw, ldw, s_ch, y, nullptr, ldy, M, N, K, base + fused_stage_bytes(M, K),
                         stream);
}

fp8_status_t fp8_gemm_scaled_fp8out(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw,
                                    int64_t ldw, const float* s_ch, uint8_t* q_out, int64_t ldq, float* s_out,
                                    float* y32_out, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
    FP8_TRY(check_dims(M, N, K));
    if (N % 16 != 0) return FP8_ERR_UNSUPPORTED;  // output rows are quantized in 16-byte pieces
    FP8_TRY(check_matrix(qa, M, K, lda, 1));
    FP8_TRY(check_matrix(qw, N, K, ldw, 1));
    FP8_TRY(check_vector(s_tok, M));
    FP8_TRY(check_vector(s_ch, N));
    FP8_TRY(check_matrix(q_out, M, N, ldq, 1));
    FP8_TRY(check_vector(s_out, M));
    if (y32_out) FP8_TRY(check_matrix(y32_out, M, N, N, 4));
    if (M > 0 && N > 0 && K > 0 && (qa == nullptr || qw == nullptr)) return FP8_ERR_INVALID_ARGUMENT;
    int64_t mn;
    if (!mul_ok(M, N, &mn) || mn > INT64_MAX / 8) return FP8_ERR_INVALID_ARGUMENT;
    const size_t stage = y32_out ? 0 : fp8out_stage_bytes(M, N);
    const size_t need = stage + gemm_ws_bytes(M, N, K);
    if (ws_bytes < need) return FP8_ERR_WORKSPACE;
    if (need > 0 && ws == nullptr) return FP8_ERR_INVALID_ARGUMENT;
    if (need > 0 && !aligned16(ws)) return FP8_ERR_UNSUPPORTED;
    if (M == 0) return FP8_OK;
    float* y32 = y32_out ? y32_out : static_cast<float*>(ws);
    if (N > 0)
        FP8_TRY(gemm_dispatch(qa, lda, s_tok, qw, ldw, s_ch, nullptr, y32, N, M, N, K,
                              static_cast<uint8_t*>(ws) + stage, stream));
    return from_hip(fp8k::launch_quantize_rows(y32, N, q_out, ldq, s_out, M, N, stream));
}

fp8_status_t fp8_gemm_grouped_scaled(const uint8_t* qa, const float* s_tok, const int32_t* row_token,
                                     const int32_t* expert_offsets, const uint8_t* qw, const float* s_ch,
                                     uint16_t* y, int64_t T, int64_t R, int64_t E, int64_t N, int64_t K,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
    (void)ws;
    FP8_TRY(check_dims(T, N, K));
    if (R < 0 || E < 0) return FP8_ERR_INVALID_ARGUMENT;
    if (R > kMaxDim || E > 1024) return FP8_ERR_UNSUPPORTED;
    if (!tiles_ok((R + 127) / 128 + E, N)) return FP8_ERR_UNSUPPORTED;
    if (R > 0 && E == 0) return FP8_ERR_INVALID_ARGUMENT;
    if (R > 0 && T == 0) return FP8_ERR_INVALID_ARGUMENT;
    FP8_TRY(check_matrix(qa, T, K, K, 1));
    FP8_TRY(check_vector(s_tok, T));
    FP8_TRY(check_vector(row_token, R));
    FP8_TRY(check_vector(expert_offsets, R > 0 ? E + 1 : 0));
    int64_t en;
    if (!mul_ok(E, N, &en)) return FP8_ERR_INVALID_ARGUMENT;
    FP8_TRY(check_matrix(qw, en, K, K, 1));
    FP8_TRY(check_vector(s_ch, en));
    FP8_TRY(check_matrix(y, R, N, N, 2, true));
    if (R > 0 && N > 0 && K > 0 && (qa == nullptr || qw == nullptr)) return FP8_ERR_INVALID_ARGUMENT;
    if (ws_bytes < fp8_grouped_workspace_bytes(T, R, E, N, K)) return FP8_ERR_WORKSPACE;
    if (R == 0 || N == 0) return FP8_OK;
    if (K % 128 == 0)
        return from_hip(fp8k::launch_gemm_grouped_mfma(qa, s_tok, row_token, expert_offsets, qw, s_ch, y, T, R, E,
                                                       N, K, stream));
    return from_hip(fp8k::launch_gemm_grouped(qa, s_tok, row_token, expert_offsets, qw, s_ch, y, T, R, E, N, K,
                                              stream));
}

fp8_status_t fp8_stream_read(const void* p, size_t bytes, int32_t workgroups, int32_t nontemporal, uint32_t* sink,
                             hipStream_t stream) {
    if (bytes % 16 != 0 || workgroups < 1 || workgroups > (1 << 20)) return FP8_ERR_INVALID_ARGUMENT;
    if (bytes > 0 && (p == nullptr || sink == nullptr)) return FP8_ERR_INVALID_ARGUMENT;
    if (bytes > 0 && (!aligned16(p) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)) return FP8_ERR_UNSUPPORTED;
    if (bytes == 0) return FP8_OK;
    return from_hip(fp8k::launch_stream_read(p, bytes, workgroups, nontemporal != 0, sink, stream));
}

}  // extern "C"
