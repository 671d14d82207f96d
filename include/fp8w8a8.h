/*
 * fp8w8a8.h -- C ABI of the MI355X (gfx950) unified-FP8 linear layer.
 *
 * The operation (from the FP8 inference pages this library implements):
 *   - activations are quantized per token to OCP FP8 E4M3 with a dynamic
 *     scale s_tok = max(fl32(rowmax|x| / 448), 1e-12f), codes enc(fl32(x/s))
 *     rounded to nearest even and saturating at +-448
 *     (Llama 3 FP8 page, §1.1 range and §3.1 absmax/448 conversion;
 *      DeepSeek V4 950 page, §2.4 per-token activation scales computed on the
 *      fly, §3.1 step 3; FP8 deployment page, §2.3 clamp to +-448);
 *   - weights arrive pre-quantized to E4M3 with one scale per output channel
 *     (same conversion, applied offline to each row of W[N,K]);
 *   - the GEMM multiplies E4M3 by E4M3 with FP32 accumulation
 *     (DeepSeek V4 950 page, §2.3) and a dequantizing epilogue writes
 *     y[m,n] = bf16_rne(acc[m,n] * (s_tok[m] * s_ch[n])).
 *
 * Layouts (row-major, unit stride along the last dimension):
 *   x      fp32  [M, K]  row stride ldx >= K      activations
 *   qa     u8    [M, K]  row stride lda >= K      activation codes
 *   qw     u8    [N, K]  row stride ldw >= K      weight codes (nn.Linear [out, in])
 *   s_tok  fp32  [M]     per-token scales
 *   s_ch   fp32  [N]     per-output-channel scales
 *   y      bf16  [M, N]  row stride ldy >= N      stored as uint16 bit patterns
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers the caller owns; buffers must stay alive
 *     until the work enqueued on `stream` completes.  The library allocates
 *     no memory and keeps no state between calls: it is re-entrant.
 *   - Every call is asynchronous on `stream` (0 = the default stream).
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and no buffer is touched.
 *       FP8_ERR_INVALID_ARGUMENT  null pointer with a non-empty extent,
 *                                 negative extent, leading dimension below the
 *                                 row length, or a size that overflows int64;
 *       FP8_ERR_UNSUPPORTED       K not a multiple of 16, an extent above
 *                                 2^31 - 1, an output with more than
 *                                 2^31 - 9 tiles of 128 x 128 (for the
 *                                 grouped GEMM: (ceil(R/128) + E) row tiles
 *                                 times ceil(N/128)), a pointer not 16-byte
 *                                 aligned, or
 *                                 an input row stride (x, qa, qw) that is not
 *                                 a multiple of 16 bytes (y may have any
 *                                 row stride ldy >= N);
 *       FP8_ERR_WORKSPACE         ws_bytes below the documented requirement;
 *       FP8_ERR_DEVICE            the HIP runtime reported a launch error.
 *   - An empty problem (M == 0, R == 0 or N == 0) is a no-op returning FP8_OK.
 *     K == 0 is valid for the GEMMs (y = 0) and for the quantizer (scales are
 *     the 1e-12 floor).
 *   - Inputs are assumed finite (E4M3 operand codes 0x7F / 0xFF are NaN).
 *   - ws is caller-owned device scratch, 16-byte aligned when it is needed;
 *     its contents on entry do not matter and are undefined after the call.
 *     Calls that share a workspace must not run concurrently.
 */
#ifndef FP8W8A8_H
#define FP8W8A8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8_OK = 0,
    FP8_ERR_INVALID_ARGUMENT = 1,
    FP8_ERR_UNSUPPORTED = 2,
    FP8_ERR_WORKSPACE = 3,
    FP8_ERR_DEVICE = 4
} fp8_status_t;

/*
 * Per-row absmax quantization to E4M3 (Llama 3 FP8 page, §3.1; applied per
 * token to activations, DeepSeek V4 950 page §2.4, and per output channel to
 * weights, the offline conversion of the same page's §3.1).
 *   scales[r] = max(fl32(max_k |x[r,k]|) / 448), 1e-12f)
 *   q[r,k]    = E4M3 code of fl32(x[r,k] / scales[r]), RNE, saturating +-448
 * x: fp32 [rows, K], stride ldx; q: u8 [rows, K], stride ldq; scales: [rows].
 * No workspace.
 */
fp8_status_t fp8_quantize_per_token(const float* x, int64_t rows, int64_t K, int64_t ldx,
                                    uint8_t* q, int64_t ldq, float* scales,
                                    hipStream_t stream);

/*
 * Static (calibrated, per-tensor) activation quantization (DeepSeek V4 950
 * page, §3.1: the static part of the activation scale is computed offline
 * from calibration data; §2.4: per-tensor scales):
 *   s          = max(*scale, 1e-12f)          (scale: one fp32 on the device)
 *   q[r,k]     = E4M3 code of fl32(x[r,k] / s), RNE, saturating +-448
 *   scales_out[r] = s for every row (so the GEMM can take it as s_tok)
 * Unlike the absmax scale, a static scale lets quotients exceed 448: they
 * saturate (the clip of §4.2 of the same page).  No workspace.
 */
fp8_status_t fp8_quantize_static(const float* x, int64_t rows, int64_t K, int64_t ldx,
                                 const float* scale, uint8_t* q, int64_t ldq, float* scales_out,
                                 hipStream_t stream);

/*
 * Per-token quantization with a static clip (the hybrid per-token + per-tensor
 * activation scale of the DeepSeek V4 950 page, §2.4 and §3.1; values above a
 * calibrated percentile clipped, §4.2):
 *   scales[r] = max(fl32(min(max_k |x[r,k]|, *clip) / 448), 1e-12f)
 *   q[r,k]    = E4M3 code of fl32(x[r,k] / scales[r]), RNE, saturating +-448
 * clip: one fp32 on the device (e.g. the P99.99 of |x| from
 * fp8_calibrate_percentile).  No workspace.
 */
fp8_status_t fp8_quantize_per_token_clipped(const float* x, int64_t rows, int64_t K, int64_t ldx,
                                            const float* clip, uint8_t* q, int64_t ldq, float* scales,
                                            hipStream_t stream);

/*
 * Calibration percentile (DeepSeek V4 950 page, §3.1 step 1 and 3, §4.2):
 * the nearest-rank percentile num/den of |x| over the n values of x (any
 * layout, fp32, device): *value_out = the r-th smallest |x| with
 * r = ceil(num * n / den) (clamped to [1, n]); scale_out (nullable) receives
 * the static scale max(fl32(*value_out / 448), 1e-12f).  E.g. num/den =
 * 999/1000 for P99.9.  0 < num <= den, 1 <= n <= 2^32 - 1.  ws: at least
 * fp8_calibrate_workspace_bytes() bytes, 16-byte aligned.  The inputs are
 * assumed finite.
 */
fp8_status_t fp8_calibrate_percentile(const float* x, int64_t n, int64_t num, int64_t den,
                                      float* value_out, float* scale_out,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes fp8_calibrate_percentile needs (host only). */
size_t fp8_calibrate_workspace_bytes(void);

/*
 * Scaled FP8 GEMM with BF16 output (DeepSeek V4 950 page, §2.3 FP8 inputs
 * with FP32 accumulation; §2.4 per-token x per-channel scales):
 *   y[m,n] = bf16_rne( (sum_k e4m3(qa[m,k]) * e4m3(qw[n,k])) * (s_tok[m] * s_ch[n]) )
 * Skinny M (decode, M <= 64) streams W once from HBM; larger M runs the
 * LDS-tiled MFMA kernel.  ws: device scratch of at least
 * fp8_gemm_workspace_bytes(M, N, K) bytes (may be NULL when that is 0).  Skinny
 * shapes with more than 16 rows, few weight rows and long K split K across
 * workgroups and keep fp32 partial sums there (added in a fixed order, so
 * results are reproducible).
 */
fp8_status_t fp8_gemm_scaled(const uint8_t* qa, int64_t lda, const float* s_tok,
                             const uint8_t* qw, int64_t ldw, const float* s_ch,
                             uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Quantize-then-GEMM in one call: the unified FP8 dataflow with no separate
 * cast step exposed to the caller (DeepSeek V4 950 page, §1.3 and §2.3).
 * Equivalent to fp8_quantize_per_token(x) followed by fp8_gemm_scaled.
 * qa_out [M, K] (stride K) and s_tok_out [M] are optional (NULL allowed);
 * when given they receive the activation codes and scales.  ws must hold at
 * least fp8_workspace_bytes(M, N, K) bytes.
 * For M <= 16 rows with M * (K + 16) <= 65792 and ceil(K / 256) <= 16
 * (M <= 8) or <= 8 (M <= 16), and 0 < N <= 8192, the call runs as one kernel
 * that quantizes x in each workgroup's prologue (ws is then not touched); the
 * codes, scales and y are the same bytes either way.
 */
fp8_status_t fp8_quant_gemm_fused(const float* x, int64_t ldx, const uint8_t* qw, int64_t ldw,
                                  const float* s_ch, uint16_t* y, int64_t ldy,
                                  int64_t M, int64_t N, int64_t K,
                                  uint8_t* qa_out, float* s_tok_out,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * FP8-output scaled GEMM: the dataflow of the DeepSeek V4 950 page, §2.3
 * (FP8 inputs, FP32 accumulation, the output converted back to FP8 for the
 * next layer), with the output re-quantized per token like the activations:
 *   y32[m,n]  = fl32( (sum_k e4m3(qa[m,k]) * e4m3(qw[n,k])) * (s_tok[m] * s_ch[n]) )
 *               (the fp32 value fp8_gemm_scaled rounds to BF16)
 *   s_out[m]  = max(fl32(max_n |y32[m,n]| / 448), 1e-12f)
 *   q_out[m,n] = E4M3 code of fl32(y32[m,n] / s_out[m]), RNE, saturating +-448
 * so q_out / s_out can feed the next layer's qa / s_tok directly.
 * q_out: u8 [M, N], stride ldq; s_out: fp32 [M].  y32_out (fp32 [M, N],
 * stride N) is optional: when given it receives y32 and serves as the
 * staging buffer, else y32 is staged in ws.  N must be a multiple of 16
 * (FP8_ERR_UNSUPPORTED otherwise).  ws must hold at least
 * fp8_fp8out_workspace_bytes(M, N, K) bytes (M * N * 4 fewer when y32_out is
 * given).  The FP32 accumulation order is the GEMM kernels' own, so a code can
 * differ from one computed from the exact sum where y32 lies within rounding
 * error of an E4M3 rounding boundary; the codes are exactly those of
 * fp8_quantize_per_token applied to y32.
 */
fp8_status_t fp8_gemm_scaled_fp8out(const uint8_t* qa, int64_t lda, const float* s_tok,
                                    const uint8_t* qw, int64_t ldw, const float* s_ch,
                                    uint8_t* q_out, int64_t ldq, float* s_out, float* y32_out,
                                    int64_t M, int64_t N, int64_t K,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Grouped (MoE expert) scaled FP8 GEMM (DeepSeek V4 950 page, §2.3 item 5:
 * expert computation entirely in FP8; §2.4 per-channel scales per expert).
 * Routed rows are sorted by expert: rows [expert_offsets[e], expert_offsets[e+1])
 * belong to expert e, and routed row r reads token row_token[r]:
 *   y[r,n] = bf16_rne( (sum_k e4m3(qa[t,k]) * e4m3(qw[e,n,k])) * (s_tok[t] * s_ch[e,n]) ),
 *   t = row_token[r]
 * qa: u8 [T, K] (stride K); s_tok: [T]; row_token: int32 [R] (device);
 * expert_offsets: int32 [E+1] (device), non-decreasing, offsets[0] = 0,
 * offsets[E] = R; qw: u8 [E, N, K]; s_ch: fp32 [E, N]; y: bf16 [R, N] (stride N).
 * The routing arrays are read on the device and not validated there: offsets
 * that are not non-decreasing in [0, R], or tokens outside [0, T), are
 * undefined behaviour.  E <= 1024.  ws must hold at least
 * fp8_grouped_workspace_bytes(...) bytes (currently 0: ws may be NULL).
 */
fp8_status_t fp8_gemm_grouped_scaled(const uint8_t* qa, const float* s_tok,
                                     const int32_t* row_token, const int32_t* expert_offsets,
                                     const uint8_t* qw, const float* s_ch, uint16_t* y,
                                     int64_t T, int64_t R, int64_t E, int64_t N, int64_t K,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Allocation-free fused call, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and kernels as fp8_quant_gemm_fused,
 * without ws: the scratch (staged activation codes and scales, split-K
 * partial sums) is a static device array of FP8_NOALLOC_SCRATCH_BYTES that
 * each GPU the library runs on holds until the process ends.  The call
 * allocates nothing; its device address is looked up once per device on the
 * first call there.  Limits and errors: FP8_ERR_WORKSPACE when
 * fp8_workspace_bytes(M, N, K) exceeds FP8_NOALLOC_SCRATCH_BYTES (e.g. up to
 * M * K ~ 72 MiB of staged codes: the 8192 x 8192 x 8192 prefill fits);
 * FP8_ERR_INVALID_ARGUMENT when `stream` belongs to another device than the
 * calling thread's current one; otherwise as fp8_quant_gemm_fused.  All calls
 * on one GPU share the array (nothing in it needs to start at zero): calls
 * that overlap on one GPU race and must be serialized by the caller.
 */
#define FP8_NOALLOC_SCRATCH_BYTES (72u << 20)
fp8_status_t fp8_quant_gemm_fused_noalloc(const float* x, int64_t ldx, const uint8_t* qw, int64_t ldw,
                                          const float* s_ch, uint16_t* y, int64_t ldy,
                                          int64_t M, int64_t N, int64_t K,
                                          uint8_t* qa_out, float* s_tok_out, hipStream_t stream);

/* Workspace bytes fp8_gemm_scaled_fp8out needs (host only; SIZE_MAX for
 * invalid sizes). */
size_t fp8_fp8out_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Workspace bytes fp8_quant_gemm_fused needs for this shape: the staged
 * activation codes and scales (M * K + 4 * M bytes, each rounded up to 256)
 * plus what the GEMM needs (host-only, pure; SIZE_MAX for invalid sizes).
 * The one-kernel fused path touches none of it, but callers size ws with
 * this value whatever path the shape takes. */
size_t fp8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Workspace bytes fp8_gemm_scaled needs for this shape: the skinny kernel's
 * fp32 split-K partial sums when the shape splits K, else 0 (host-only,
 * pure; SIZE_MAX for invalid sizes). */
size_t fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Workspace bytes fp8_gemm_grouped_scaled needs (host-only, pure). */
size_t fp8_grouped_workspace_bytes(int64_t T, int64_t R, int64_t E, int64_t N, int64_t K);

/*
 * Block-scaled ("MX") quantization (per-group/block scales: DeepSeek V4 950
 * page, §2.4 and §4.2; MXFP8 block scaling: FP8 deployment page, §7.1):
 * every 32 consecutive elements of a row (block b = k / 32) share a
 * power-of-two scale, kept as its exponent byte c (scale 2^(c - 127)):
 *   v      = max(fl32(max_{k in block} |x[r,k]| / 448), 1e-12f)
 *   e      = the smallest integer with 2^e >= v     (so nothing clips)
 *   q[r,k] = E4M3 code of x[r,k] * 2^-e, RNE
 * x: fp32 [rows, K], stride ldx; q: u8 [rows, K], stride ldq.
 * Scale layout (chunk-major, the order the GEMM kernels fetch it): u8
 * [K/128][rows][4]; byte j of row r in chunk c is the exponent byte of block
 * 4c + j, i.e. scales[(c * rows + r) * 4 + j] = e(r, 4c + j) + 127.
 * K must be a multiple of 128 (else FP8_ERR_UNSUPPORTED); the other
 * conventions as for fp8_quantize_per_token.  No workspace.
 */
fp8_status_t fp8_quantize_mx(const float* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                             uint8_t* scales, hipStream_t stream);

/*
 * Block-scaled FP8 GEMM with BF16 output (block scales applied inside the K
 * loop by gfx950's block-scaled MFMA; FP32 accumulation, DeepSeek V4 950
 * page, §2.3):
 *   y[m,n] = bf16_rne( sum_b 2^(ea(m,b) + ew(n,b) - 254)
 *                          * sum_{k in block b} e4m3(qa[m,k]) * e4m3(qw[n,k]) )
 * qa u8 [M, K] (lda), qw u8 [N, K] (ldw); sa u8 [K/128][M][4] and sw u8
 * [K/128][N][4] hold the exponent bytes ea, ew in the chunk-major layout
 * fp8_quantize_mx writes (4-byte aligned); y bf16 [M, N] (ldy).  K must be
 * a multiple of 128 (K == 0 gives y = 0).  ws: at least
 * fp8_mx_workspace_bytes(M, N, K) bytes, 16-byte aligned (decode shapes that
 * split K keep fp32 partial sums there; may be NULL when that is 0; contents
 * on entry do not matter).
 */
fp8_status_t fp8_gemm_mx(const uint8_t* qa, int64_t lda, const uint8_t* sa, const uint8_t* qw, int64_t ldw,
                         const uint8_t* sw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Workspace bytes fp8_gemm_mx needs (host only; SIZE_MAX for invalid sizes). */
size_t fp8_mx_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * FP8 KV cache (DeepSeek V4 950 page, §2.1: E5M2 for the KV cache, §2.2:
 * one scale per latent dimension, paged blocks; 512K-context page, §3.3:
 * block pool with per-request block tables, per-channel FP8 scales; FP8
 * deployment page, §2.3: the E4M3 KV variant and its absmax/448 scale).
 *
 * A KV batch is T token rows of C channels (e.g. the K and V heads of one
 * layer side by side, or one latent vector): kv [T, C] of fp32, bf16 or
 * fp16 elements (kv_dtype; 16-bit values convert to fp32 exactly, and all
 * arithmetic below is on that fp32 value), row stride ldkv elements.  The cache is a pool of num_slots rows of C codes (u8 [num_slots, C],
 * unit-stride rows of exactly C bytes); slot_mapping int32 [T] names each
 * token's row, physical block * block size + offset in the block, as the
 * caller's block table resolves it.  fmt picks the code format; scales are
 * fp32 [C], one per channel, floored at 1e-12f wherever they are used.
 * C must be a multiple of 4 (of 8 for bf16 / fp16 rows, which are read
 * 8 channels at a time); kv and out rows 16-byte aligned (row stride
 * times element size a multiple of 16 bytes); kv, scales, cache, out
 * 16-byte aligned (else FP8_ERR_UNSUPPORTED).  T, C, num_slots <= 2^31 - 1.
 * Inputs are assumed finite.
 */
typedef enum { FP8_KV_E4M3 = 0, FP8_KV_E5M2 = 1 } fp8_kv_format_t;
typedef enum { FP8_KV_F32 = 0, FP8_KV_BF16 = 1, FP8_KV_F16 = 2 } fp8_kv_dtype_t;

/*
 * Per-channel scales of a KV batch (the online calibration of the Llama 3
 * FP8 page, §3.2, per channel):
 *   scales[c] = max(fl32(max_t |kv[t,c]| / fmt_max), 1e-12f),
 * fmt_max = 448 (E4M3) or 57344 (E5M2).  T == 0 gives the floor.  ws: at
 * least fp8_kv_scales_workspace_bytes(T, C) bytes, 16-byte aligned.
 */
fp8_status_t fp8_kv_channel_scales(const void* kv, fp8_kv_dtype_t kv_dtype, int64_t T, int64_t C, int64_t ldkv,
                                   fp8_kv_format_t fmt, float* scales, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Workspace bytes fp8_kv_channel_scales needs (host only; SIZE_MAX for
 * invalid sizes). */
size_t fp8_kv_scales_workspace_bytes(int64_t T, int64_t C);

/*
 * Quantize a KV batch into its cache slots:
 *   cache[slot_mapping[t], c] = enc_fmt(fl32(kv[t,c] / scales[c]))
 * rounded to nearest even and saturating at the format's largest finite
 * value (+-448 or +-57344).  Tokens whose slot is outside [0, num_slots)
 * (padding carries -1) are skipped; cache rows no token names are left
 * as they were.  Two tokens naming the same slot race (one of them wins).
 * No workspace.
 */
fp8_status_t fp8_kv_quantize_paged(const void* kv, fp8_kv_dtype_t kv_dtype, int64_t T, int64_t C, int64_t ldkv,
                                   const float* scales, fp8_kv_format_t fmt, const int32_t* slot_mapping,
                                   uint8_t* cache, int64_t num_slots, hipStream_t stream);

/*
 * Read a sequence's rows back out of the cache:
 *   out[t,c] = round_out(fl32(dec_fmt(cache[slot_mapping[t], c]) * scales[c]))
 * out [T, C] of out_dtype elements (fp32: the product itself; bf16 / fp16:
 * rounded to nearest even), row stride ldo elements; a slot outside
 * [0, num_slots) gives a row of +0.  No workspace.
 */
fp8_status_t fp8_kv_dequantize_paged(const uint8_t* cache, int64_t num_slots, const int32_t* slot_mapping,
                                     int64_t T, int64_t C, const float* scales, fp8_kv_format_t fmt, void* out,
                                     fp8_kv_dtype_t out_dtype, int64_t ldo, hipStream_t stream);

/*
 * HBM read ceiling (a measurement utility beside the layer, not part of it):
 * reads the `bytes` bytes at p once with plain 16-byte vector loads
 * (nontemporal loads when `nontemporal` != 0) from about `workgroups`
 * workgroups of 256 threads, each streaming a contiguous share, 8 loads in
 * flight per thread -- the request size and depth of the decode kernels, so
 * its rate is the weight-streaming ceiling those kernels are measured against
 * (DeepSeek V4 950 page, §1.2: decode time is the time to move the weights).
 * The data is folded into one 32-bit value per thread, stored to *sink only
 * when it equals 0x9E3779B9 (so the loads cannot be dropped).  bytes % 16 ==
 * 0, 1 <= workgroups <= 2^20, p 16-byte aligned, sink 4-byte aligned.
 */
fp8_status_t fp8_stream_read(const void* p, size_t bytes, int32_t workgroups, int32_t nontemporal, uint32_t* sink,
                             hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fp8_status_string(fp8_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* FP8W8A8_H */
