/*
 * CPU oracle for the unified-FP8 (W8A8) linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, plain reference the
 * HIP path is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no code, headers, tables or constants with the HIP library.
 *
 * Sources (web pages on FP8 LLM inference; cited by page and section):
 *   [DSV4]  "DeepSeek V4 950: unified low-precision dataflow" (2kiu.com),
 *           §1.2 (decode is bandwidth bound), §2.1 (E4M3 vs E5M2),
 *           §2.3 (FP8 in, FP32 accumulate), §2.4 (per-channel weight and
 *           per-token activation scales), §3.1 (scales computed on the fly).
 *   [L3]    "Llama 3 FP8 deployment and long context" (dpshk.com),
 *           §1.1 (E4M3 largest value 448, smallest non-zero 2^-9),
 *           §3.1 (weight-conversion snippet: per-output-channel absmax/448,
 *           clamped below at 1e-12, cast to float8_e4m3fn),
 *           §4.1 (scan quantized tensors for NaN/Inf).
 *   [DEPLOY] "FP8 mixed-precision inference deployment" (ybb.press),
 *           §1.1 (E4M3 range +-448, E5M2 range +-57344), §2.3 (clamp to
 *           +-448; the KV-cache scale sketch).
 *   [SP512K] "512K context on 8 x H20" (hotelren.com), §3.3 (paged KV cache
 *           in FP8 with per-channel scales).
 * Block scales: [DSV4] §2.4 (per-group/block scales: one scale per small
 * block of a tensor) and §4.2 (per-group where activation ranges jump);
 * [DEPLOY] §7.1 (MXFP8: FP8 elements with a shared scale per block).
 *
 * Readings where the pages leave a step open (all float arithmetic below is
 * IEEE binary32/binary64 with round-to-nearest-even; build without
 * fast-math and without FP contraction):
 *   - E4M3 is the OCP "fn" variant: bias 7, no infinities, S.1111.111 is NaN,
 *     largest finite S.1111.110 = 448, smallest subnormal 2^-9.
 *   - Encoding rounds to nearest, ties to the even code, and saturates to
 *     +-448 (infinities included); NaN keeps its sign as S.1111.111.
 *   - The scale is the dequantization multiplier s = max(fl32(amax/448), 1e-12f)
 *     for activation rows and weight rows alike; codes are enc(fl32(x / s))
 *     with a correctly rounded division.
 *   - The GEMM is sum_k dec(a)*dec(w) accumulated in binary64, which is exact
 *     here (every product is a multiple of 2^-18 and |sum| < 2^35 for
 *     K <= 28672), times (double)s_tok * (double)s_ch.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- codec -- */

/* Value of an E4M3 code ([L3] §1.1; [DSV4] §2.1): sign s, exponent field E
 * (4 bits, bias 7), mantissa field m (3 bits).  E = 0 is subnormal m * 2^-9. */
double oracle_e4m3_decode(uint8_t code) {
    int s = (code >> 7) & 1;
    int E = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (E == 15 && m == 7) return NAN;
    if (E == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, E - 7);
    return s ? -mag : mag;
}

/* Round a non-negative double to an integer, ties to even. */
static double round_half_even(double q) {
    double f = floor(q);
    double d = q - f;
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* fp32 -> E4M3 code: round to nearest even on the E4M3 grid, saturate to
 * +-448 ([DEPLOY] §2.3 clamp), NaN -> S.1111.111. */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int ex = e2 - 1;        /* a in [2^ex, 2^(ex+1)) */
    if (ex < -6) {
        /* below the smallest normal 2^-6: grid step 2^-9, codes 0..8
           (8 * 2^-9 = 2^-6 is code 0x08, the smallest normal) */
        double r = round_half_even(ldexp(a, 9));
        return (uint8_t)(sign | (int)r);
    }
    /* binade [2^ex, 2^(ex+1)): 8 steps of 2^(ex-3) */
    double r = round_half_even(ldexp(a, 3 - ex)); /* in [8, 16] */
    if (r == 16.0) { ex += 1; r = 8.0; }
    int E = ex + 7, m = (int)r - 8;
    return (uint8_t)(sign | (E << 3) | m);
}

/* Element-wise encode of an array (the codec above, applied n times). */
void oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

/* Value of an E5M2 code ([DSV4] §2.1: 5 exponent bits, 2 mantissa bits,
 * range +-57344; [DEPLOY] §1.1): exponent field E (bias 15), mantissa m.
 * E = 31 holds infinity (m = 0) and NaN (m != 0); E = 0 is subnormal
 * m * 2^-16. */
double oracle_e5m2_decode(uint8_t code) {
    int s = (code >> 7) & 1;
    int E = (code >> 2) & 31;
    int m = code & 3;
    double mag;
    if (E == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
    if (E == 0)
        mag = ldexp((double)m, -16);
    else
        mag = ldexp(1.0 + (double)m / 4.0, E - 15);
    return s ? -mag : mag;
}

/* fp32 -> E5M2 code: round to nearest even on the E5M2 grid, saturate to
 * +-57344 (the KV cache keeps finite values; the same clamp as for E4M3),
 * NaN -> S.11111.11. */
uint8_t oracle_e5m2_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 57344.0) return (uint8_t)(sign | 0x7B);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;
    if (ex < -14) {
        /* below the smallest normal 2^-14: grid step 2^-16, codes 0..4 */
        double r = round_half_even(ldexp(a, 16));
        return (uint8_t)(sign | (int)r);
    }
    /* binade [2^ex, 2^(ex+1)): 4 steps of 2^(ex-2) */
    double r = round_half_even(ldexp(a, 2 - ex)); /* in [4, 8] */
    if (r == 8.0) { ex += 1; r = 4.0; }
    int E = ex + 15, m = (int)r - 4;
    return (uint8_t)(sign | (E << 2) | m);
}

void oracle_e5m2_encode_array(const float* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e5m2_encode(v[i]);
}

/* ------------------------------------------------------------ quantizer -- */

/* Per-row absmax quantization, the [L3] §3.1 conversion applied to any
 * row-major matrix: rows of W (per output channel) or rows of X (per token,
 * computed on the fly as [DSV4] §2.4 and §3.1 describe).
 *   scale[r] = max(fl32(max_k |x[r,k]|) / 448), 1e-12f)
 *   q[r,k]   = enc(fl32(x[r,k] / scale[r]))                                 */
void oracle_quantize_rows(const float* x, int64_t rows, int64_t K, int64_t ldx,
                          uint8_t* q, int64_t ldq, float* scales) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * ldx;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(xr[k]);
            if (a > amax) amax = a;
        }
        float s = amax / 448.0f;
        if (s < 1e-12f) s = 1e-12f;
        scales[r] = s;
        for (int64_t k = 0; k < K; ++k) {
            float t = xr[k] / s;
            q[r * ldq + k] = oracle_e4m3_encode(t);
        }
    }
}

/* Static (calibrated, per-tensor) quantization: one scale s for the whole
 * tensor, computed offline from a percentile of |x| over calibration data
 * ([DSV4] §3.1: P99.9 of the activation magnitudes instead of the maximum;
 * §4.2: values beyond the range clipped).  Quotients above 448 saturate, the
 * clamp of [DEPLOY] §2.3:
 *   q[r,k] = enc(fl32(x[r,k] / s))                                          */
void oracle_quantize_static(const float* x, int64_t rows, int64_t K, int64_t ldx, float s,
                            uint8_t* q, int64_t ldq) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) q[r * ldq + k] = oracle_e4m3_encode(x[r * ldx + k] / s);
}

/* Per-token quantization with a static clip (the per-token + per-tensor
 * hybrid of [DSV4] §2.4; outliers above a calibrated percentile clipped,
 * §4.2):
 *   scale[r] = max(fl32(min(max_k |x[r,k]|, clip) / 448), 1e-12f)
 *   q[r,k]   = enc(fl32(x[r,k] / scale[r]))                                 */
void oracle_quantize_rows_clipped(const float* x, int64_t rows, int64_t K, int64_t ldx, float clip,
                                  uint8_t* q, int64_t ldq, float* scales) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * ldx;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(xr[k]);
            if (a > amax) amax = a;
        }
        if (clip < amax) amax = clip;
        float s = amax / 448.0f;
        if (s < 1e-12f) s = 1e-12f;
        scales[r] = s;
        for (int64_t k = 0; k < K; ++k) q[r * ldq + k] = oracle_e4m3_encode(xr[k] / s);
    }
}

/* ----------------------------------------------------------- KV cache -- */

/* Per-channel KV scales ([DSV4] §2.2: one scale per latent dimension;
 * [SP512K] §3.3 and [DEPLOY] §2.3: per-channel scales):
 *   scale[c] = max(fl32(max_t |kv[t,c]| / fmt_max), 1e-12f),
 * fmt_max = 448 (E4M3) or 57344 (E5M2, the KV format of [DSV4] §2.1).    */
void oracle_kv_channel_scales(const float* kv, int64_t T, int64_t C, int64_t ld, int fmt, float* scales) {
    const float fmax = fmt == 1 ? 57344.0f : 448.0f;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        float amax = 0.0f;
        for (int64_t t = 0; t < T; ++t) {
            float a = fabsf(kv[t * ld + c]);
            if (a > amax) amax = a;
        }
        float s = amax / fmax;
        if (s < 1e-12f) s = 1e-12f;
        scales[c] = s;
    }
}

/* Quantize T tokens of KV into a paged cache of num_slots rows: token t goes
 * to cache row slot[t] (a block index times the block size plus the offset
 * in the block, as the block table of [SP512K] §3.3 resolves it).  A slot
 * outside [0, num_slots) (padding tokens carry -1) skips the token.  The
 * scale is floored at 1e-12f as everywhere else.
 *   cache[slot[t], c] = enc_fmt(fl32(kv[t,c] / scale[c]))                 */
void oracle_kv_quantize(const float* kv, int64_t T, int64_t C, int64_t ld, const float* scales, int fmt,
                        const int32_t* slot, uint8_t* cache, int64_t num_slots) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        if (slot[t] < 0 || slot[t] >= num_slots) continue;
        for (int64_t c = 0; c < C; ++c) {
            float s = scales[c] < 1e-12f ? 1e-12f : scales[c];
            float q = kv[t * ld + c] / s;
            cache[(int64_t)slot[t] * C + c] = fmt == 1 ? oracle_e5m2_encode(q) : oracle_e4m3_encode(q);
        }
    }
}

/* Read back: out[t,c] = fl32(dec_fmt(cache[slot[t], c]) * scale[c]) with the
 * same floored scale; a slot outside [0, num_slots) gives a row of zeros.  */
void oracle_kv_dequantize(const uint8_t* cache, int64_t num_slots, const int32_t* slot, int64_t T, int64_t C,
                          const float* scales, int fmt, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < C; ++c) {
            if (slot[t] < 0 || slot[t] >= num_slots) {
                out[t * C + c] = 0.0f;
                continue;
            }
            uint8_t code = cache[(int64_t)slot[t] * C + c];
            float s = scales[c] < 1e-12f ? 1e-12f : scales[c];
            float d = (float)(fmt == 1 ? oracle_e5m2_decode(code) : oracle_e4m3_decode(code));
            out[t * C + c] = d * s;
        }
}

/* --------------------------------------------------------------- GEMM ---- */

static double g_dec[256];
static int g_dec_ready = 0;

static void dec_table(void) {
    if (g_dec_ready) return;
    for (int c = 0; c < 256; ++c) g_dec[c] = oracle_e4m3_decode((uint8_t)c);
    g_dec_ready = 1;
}

void oracle_init(void) { dec_table(); }

/* One output element of the scaled FP8 GEMM ([DSV4] §2.3: FP8 operands,
 * wide accumulation; scales of §2.4 applied after the sum):
 *   D = sum_k dec(a[k]) * dec(w[k])        (binary64, exact)
 *   A = sum_k |dec(a[k]) * dec(w[k])|
 *   ref = D * (s_tok * s_ch),  absref = A * (s_tok * s_ch)                    */
static void dot_one(const uint8_t* a, const uint8_t* w, int64_t K, double st, double sc,
                    double* ref, double* absref) {
    double D = 0.0, A = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = g_dec[a[k]] * g_dec[w[k]];
        D += p;
        A += fabs(p);
    }
    double s = st * sc;
    *ref = D * s;
    *absref = A * s;
}

/* Full reference: ref[m,n], absref[m,n] for qa [M,K] (lda), qw [N,K] (ldw). */
void oracle_gemm_ref(const uint8_t* qa, int64_t lda, const float* s_tok,
                     const uint8_t* qw, int64_t ldw, const float* s_ch,
                     int64_t M, int64_t N, int64_t K, double* ref, double* absref) {
    dec_table();
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            dot_one(qa + m * lda, qw + n * ldw, K, (double)s_tok[m], (double)s_ch[n],
                    ref + m * N + n, absref + m * N + n);
}

/* Reference at the listed (m, n) pairs only. */
void oracle_gemm_ref_sampled(const uint8_t* qa, int64_t lda, const float* s_tok,
                             const uint8_t* qw, int64_t ldw, const float* s_ch, int64_t K,
                             const int64_t* ms, const int64_t* ns, int64_t count,
                             double* ref, double* absref) {
    dec_table();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        dot_one(qa + ms[i] * lda, qw + ns[i] * ldw, K, (double)s_tok[ms[i]], (double)s_ch[ns[i]],
                ref + i, absref + i);
}

/* Grouped (MoE) reference ([DSV4] §2.3 item 5 and §2.4: experts run in FP8
 * with per-channel weight scales of their own).  Routed row r belongs to the
 * expert e with offsets[e] <= r < offsets[e+1]; it reads token row_token[r]:
 *   y[r,n] = (sum_k dec(qa[tok,k]) * dec(qw[e,n,k])) * s_tok[tok] * s_ch[e,n]
 * Evaluated at the listed (r, n) pairs.  Returns -1 if a row has no expert. */
int oracle_grouped_ref_sampled(const uint8_t* qa, const float* s_tok, const int32_t* row_token,
                               const int32_t* offsets, int64_t E, const uint8_t* qw,
                               const float* s_ch, int64_t N, int64_t K,
                               const int64_t* rs, const int64_t* ns, int64_t count,
                               double* ref, double* absref) {
    dec_table();
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t i = 0; i < count; ++i) {
        int64_t r = rs[i], e = -1;
        for (int64_t j = 0; j < E; ++j)
            if (offsets[j] <= r && r < offsets[j + 1]) { e = j; break; }
        if (e < 0) { bad = 1; ref[i] = NAN; absref[i] = NAN; continue; }
        int64_t t = row_token[r];
        dot_one(qa + t * K, qw + (e * N + ns[i]) * K, K, (double)s_tok[t],
                (double)s_ch[e * N + ns[i]], ref + i, absref + i);
    }
    return bad ? -1 : 0;
}

/* ----------------------------------------------------------- BF16 -------- */

/* ------------------------------------------------------ block scales -- */

/* Block-scaled ("MX") quantization.  Every 32 consecutive elements of a row
 * share one scale that is a power of two, stored as its exponent byte
 * (E8M0: code c means 2^(c - 127)).  Readings: the block is 32 elements
 * (the open MX format; [DEPLOY] §7.1 says 16); the scale is the pages'
 * absmax/448 scale ([L3] §3.1, 1e-12 floor) rounded up to a power of two,
 *   v = max(fl32(amax / 448), 1e-12f),  e = smallest integer with 2^e >= v,
 * so |x| / 2^e <= 448 and no element of the block is clipped; the codes are
 * enc(x / 2^e) (a division by a power of two, exact unless the quotient is
 * an fp32 subnormal, where it rounds once like any IEEE division).        */
static int mx_exponent(float v) {
    int e2;
    double m = frexp((double)v, &e2); /* v = m * 2^e2, m in [0.5, 1) */
    return m == 0.5 ? e2 - 1 : e2;
}

uint8_t oracle_mx_scale_code(float amax) {
    float v = amax / 448.0f;
    if (v < 1e-12f) v = 1e-12f;
    return (uint8_t)(mx_exponent(v) + 127);
}

/* x [rows, K] (K % 32 == 0) -> codes q [rows, K] (ldq), scale codes
 * sc [rows, K / 32] (row-major, no padding). */
void oracle_quantize_mx(const float* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                        uint8_t* sc) {
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = x + r * ldx + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i)
                if (fabsf(xb[i]) > amax) amax = fabsf(xb[i]);
            const uint8_t c = oracle_mx_scale_code(amax);
            const double scale = ldexp(1.0, (int)c - 127);
            sc[r * nb + b] = c;
            for (int i = 0; i < 32; ++i) q[r * ldq + 32 * b + i] = oracle_e4m3_encode((float)((double)xb[i] / scale));
        }
}

/* Block-scaled GEMM reference at the listed (m, n) pairs:
 *   ref = sum_k dec(a[m,k]) dec(w[n,k]) 2^(sa[m,k/32] - 127) 2^(sw[n,k/32] - 127)
 *   absref = the same sum of magnitudes.  Each block's sum is exact in
 * binary64; adding the scaled block sums rounds only in binary64 (relative
 * error about 2^-53 of absref).  sa [M, K/32], sw [N, K/32]. */
static void mx_dot(const uint8_t* a, const uint8_t* sa, const uint8_t* w, const uint8_t* sw, int64_t K, double* ref,
                   double* absref) {
    double D = 0.0, A = 0.0;
    for (int64_t b = 0; b < K / 32; ++b) {
        double d = 0.0, ab = 0.0;
        for (int i = 0; i < 32; ++i) {
            double p = g_dec[a[32 * b + i]] * g_dec[w[32 * b + i]];
            d += p;
            ab += fabs(p);
        }
        double s = ldexp(1.0, (int)sa[b] + (int)sw[b] - 254);
        D += d * s;
        A += ab * s;
    }
    *ref = D;
    *absref = A;
}

void oracle_gemm_mx_ref_sampled(const uint8_t* qa, int64_t lda, const uint8_t* sa, const uint8_t* qw, int64_t ldw,
                                const uint8_t* sw, int64_t K, const int64_t* ms, const int64_t* ns, int64_t count,
                                double* ref, double* absref) {
    dec_table();
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        mx_dot(qa + ms[i] * lda, sa + ms[i] * nb, qw + ns[i] * ldw, sw + ns[i] * nb, K, ref + i, absref + i);
}

/* Nearest bfloat16 (1-8-7 format) of a double, ties to even, as bits.  Used
 * only to report how many GPU outputs equal the correctly rounded reference. */
uint16_t oracle_bf16_from_double(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0);
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;
    if (ex < -126) ex = -126;                 /* subnormal range: fixed step */
    double r = round_half_even(ldexp(a, 7 - ex));
    double mag = ldexp(r, ex - 7);
    if (mag >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float f = (float)mag;                     /* exact: mag has <= 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return (uint16_t)(sign | (bits >> 16));
}

void oracle_bf16_from_double_array(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_double(v[i]);
}

/* Nearest IEEE binary16 (1-5-10 format, exponent bias 15) of a double, ties
 * to even, as bits: the 16-bit read back of the KV cache ([SP512K] §3.3: the
 * cache holds FP8 in place of FP16 KV).  Normal values in [2^e, 2^(e+1)),
 * e in [-14, 15], have 10 fraction bits; below 2^-14 the grid step is 2^-24
 * (subnormals); a value that rounds to 2^16 or beyond (|v| >= 65520) is
 * infinite; NaN keeps its sign with the quiet bit set. */
uint16_t oracle_fp16_from_double(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00);
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7C00);
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;                          /* a in [2^ex, 2^(ex+1)) */
    if (ex < -14) {
        /* subnormal range: integer multiples of 2^-24, codes 0 .. 0x400
           (0x400 * 2^-24 = 2^-14 is the smallest normal, exponent field 1) */
        double r = round_half_even(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)r);
    }
    double r = round_half_even(ldexp(a, 10 - ex)); /* significand in [1024, 2048] */
    if (r == 2048.0) { ex += 1; r = 1024.0; }
    if (ex > 15) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | ((ex + 15) << 10) | ((int)r - 1024));
}

void oracle_fp16_from_double_array(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp16_from_double(v[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
