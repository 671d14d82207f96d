// Launchers of the gfx950 kernels (internal to the library; the C ABI in
// include/fp8w8a8.h validates arguments before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8k {

// Per-row absmax quantization (quantize.hip).
hipError_t launch_quantize_rows(const float* x, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                                int64_t rows, int64_t K, hipStream_t stream);
// Static per-tensor scale *scale (device, floored at 1e-12) for every row;
// scales[r] receives it for each row.
hipError_t launch_quantize_static(const float* x, int64_t ldx, const float* scale, uint8_t* q, int64_t ldq,
                                  float* scales, int64_t rows, int64_t K, hipStream_t stream);
// Per-row absmax scale with the absmax clipped at *clip (device).
hipError_t launch_quantize_clipped(const float* x, int64_t ldx, const float* clip, uint8_t* q, int64_t ldq,
                                   float* scales, int64_t rows, int64_t K, hipStream_t stream);
// Nearest-rank percentile of |x| over n values (calibrate.hip): value_out =
// the rank-th smallest |x| (1 <= rank <= n); scale_out (nullable) =
// max(fl32(value / 448), 1e-12f).  ws: kCalibrateWsBytes bytes.
constexpr size_t kCalibrateWsBytes = 2048;
hipError_t launch_calibrate_percentile(const float* x, int64_t n, int64_t rank, float* value_out, float* scale_out,
                                       void* ws, hipStream_t stream);

// FP8 KV-cache codec (kv_cache.hip).  fmt: kKvE4M3 or kKvE5M2; element
// types of the KV rows and of the read back: kKvF32, kKvBF16, kKvF16.
// C % 4 == 0, row strides in elements with 16-byte aligned rows, scales
// 16-byte aligned.
constexpr int kKvE4M3 = 0;
constexpr int kKvE5M2 = 1;
constexpr int kKvF32 = 0;
constexpr int kKvBF16 = 1;
constexpr int kKvF16 = 2;
// Row chunks of the per-channel maximum pass; its fp32 partials take
// kv_scales_ws_bytes(T, C) bytes of workspace (16-byte aligned).
struct KvChunks {
    int rows_per_chunk, chunks;
};
KvChunks kv_amax_chunks(int64_t T, int64_t C, int quads);
size_t kv_scales_ws_bytes(int64_t T, int64_t C);
hipError_t launch_kv_channel_scales(const void* kv, int dtype, int64_t T, int64_t C, int64_t ldkv, int fmt,
                                    float* scales, void* ws, hipStream_t stream);
hipError_t launch_kv_quantize_paged(const void* kv, int dtype, int64_t T, int64_t C, int64_t ldkv, const float* scales,
                                    int fmt, const int32_t* slot, uint8_t* cache, int64_t num_slots,
                                    hipStream_t stream);
hipError_t launch_kv_dequantize_paged(const uint8_t* cache, int64_t num_slots, const int32_t* slot, int64_t T,
                                      int64_t C, const float* scales, int fmt, void* out, int out_dtype, int64_t ldo,
                                      hipStream_t stream);

// The dense GEMM launchers write BF16 y, or, when y32 is not null, the fp32
// value acc * (s_tok * s_ch) before rounding to y32 (same row stride ldy).

// Block-scaled quantization (block_scale.hip): K % 128 == 0; scales are
// chunk-major exponent bytes: word [K / 128][rows], byte j = block 4c + j.
hipError_t launch_quantize_mx(const float* x, int64_t ldx, uint8_t* q, int64_t ldq, uint8_t* scales, int64_t rows,
                              int64_t K, hipStream_t stream);

// Block ("MX") scales of both GEMM operands: exponent bytes, 2^(c - 127),
// one per 32 k of a row, chunk-major: 32-bit word [K / 128][rows] holds a
// row's 4 bytes of one 128-k chunk.  sa covers M rows, sw N rows.
struct MxScales {
    const uint8_t* sa;
    const uint8_t* sw;
};

// Largest M the skinny (decode) kernel takes.
constexpr int64_t kSkinnyMaxM = 64;

// Skinny-M scaled GEMM, M <= kSkinnyMaxM (gemm_skinny.hip).  Shapes with few
// weight rows and long k split k across workgroups; they need
// gemm_skinny_ws_bytes(M, N, K) bytes of workspace in ws (fp32 partial sums,
// fully overwritten by every call, no zero fill needed).
struct SkinnyPlan {
    int mt, nt, splits, split_chunks;
};
SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K);
size_t gemm_skinny_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_skinny(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw,
                              int64_t ldw, const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int64_t M, int64_t N,
                              int64_t K, void* ws, hipStream_t stream);

// Block-scaled skinny GEMM (K % 128 == 0): y = bf16_rne(sum over blocks of
// 2^(sa + sw - 254) * block dot); same plan and workspace as above.
hipError_t launch_gemm_skinny_mx(const uint8_t* qa, int64_t lda, const uint8_t* sa, const uint8_t* qw, int64_t ldw,
                                 const uint8_t* sw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws,
                                 hipStream_t stream);

// Block-scaled MFMA GEMM for M > kSkinnyMaxM, K % 128 == 0 (gemm_mfma.hip).
hipError_t launch_gemm_mfma_mx(const uint8_t* qa, int64_t lda, const uint8_t* sa, const uint8_t* qw, int64_t ldw,
                               const uint8_t* sw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream);

// Quantize + skinny GEMM in one kernel, for M <= kSkinnyFusedMaxM rows whose
// codes fit in kSkinnyFusedLds bytes of LDS and N <= 8192 (gemm_skinny.hip).  qa_out and
// s_tok_out may be null; when given they receive the codes and scales.
constexpr int64_t kSkinnyFusedMaxM = 16;
constexpr int64_t kSkinnyFusedLds = 64 * 1024 + 16 * 16;
bool gemm_skinny_fused_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_skinny_fused(const float* x, int64_t ldx, const uint8_t* qw, int64_t ldw, const float* s_ch,
                                    uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, uint8_t* qa_out,
                                    float* s_tok_out, hipStream_t stream);

// LDS-tiled MFMA scaled GEMM for larger M (gemm_tiled.hip).
hipError_t launch_gemm_tiled(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw,
                             int64_t ldw, const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int64_t M, int64_t N,
                             int64_t K, hipStream_t stream);

// Two-stage DMA-fed MFMA GEMM, K % 128 == 0 (gemm_mfma.hip).
hipError_t launch_gemm_mfma(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw, int64_t ldw,
                            const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int64_t M, int64_t N, int64_t K,
                            hipStream_t stream);

// Grouped (MoE) variant of the two-stage kernel, K % 128 == 0 (gemm_mfma.hip).
hipError_t launch_gemm_grouped_mfma(const uint8_t* qa, const float* s_tok, const int32_t* row_token,
                                    const int32_t* offsets, const uint8_t* qw, const float* s_ch, uint16_t* y,
                                    int64_t T, int64_t R, int64_t E, int64_t N, int64_t K, hipStream_t stream);

// Grouped (MoE) scaled GEMM, any K % 16 == 0 (gemm_tiled.hip).
hipError_t launch_gemm_grouped(const uint8_t* qa, const float* s_tok, const int32_t* row_token,
                               const int32_t* offsets, const uint8_t* qw, const float* s_ch, uint16_t* y,
                               int64_t T, int64_t R, int64_t E, int64_t N, int64_t K, hipStream_t stream);

// Plain streaming read of `bytes` bytes (multiple of 16, p 16-byte aligned)
// by about `workgroups` workgroups of 256 threads (stream_read.hip); sink: one
// uint32 that is written only when the folded data equals a magic value.
hipError_t launch_stream_read(const void* p, size_t bytes, int workgroups, bool nontemporal, uint32_t* sink,
                              hipStream_t stream);

}  // namespace fp8k
