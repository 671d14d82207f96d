/*
 * Check of the division method the GPU quantizer uses: for a row scale s and
 * an element x it forms r = RN(1/s), q0 = RN(x * r), d = q0 * s - x (one FMA,
 * exact) and q = RN(q0 - d * r) (one FMA); with the residual in that order
 * x = -0 gives -0 (d = +0, q = -0 - 0), so no sign fix-up follows.  The claim
 * checked here is q == RN(x / s) bit for bit,
 * except for subnormal x (see agree() below), where the E4M3 code is the
 * same signed zero either way; the reference quotient is binary64 division
 * rounded to binary32, which is correctly rounded because 53 >= 2 * 24 + 2.
 *
 * Cases: random scales over the whole range a row scale can take
 * (1e-12 .. FLT_MAX / 448) with random |x| <= 448 s or <= 57344 s; any
 * finite x (quotients that overflow included); and, for a list of scales,
 * every x within a few ulps of (midpoint between two consecutive E4M3 or
 * E5M2 magnitudes) * s and of (FP8 magnitude) * s -- the quotients where a
 * one-ulp error would change the code.
 */
#include <math.h>
#include <stdint.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static uint64_t sm64(uint64_t* st) {
    uint64_t z = (*st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* The first quotient is clamped to +-2^20 (a med3 on the GPU) so that an
 * fp32 overflow of x * r cannot turn the residual into inf - inf = NaN; a
 * clamped quotient is far beyond every FP8 code's range and still saturates. */
static float method(float x, float s) {
    const float r = (float)(1.0 / (double)s);
    const float q0 = fminf(fmaxf(x * r, -0x1p20f), 0x1p20f);
    const float d = fmaf(q0, s, -x);
    return fmaf(d, -r, q0);
}

static float exact(float x, float s) { return (float)((double)x / (double)s); }

static int same(float a, float b) {
    union { float f; uint32_t u; } ua = {a}, ub = {b};
    return ua.u == ub.u;
}

/* The method equals IEEE division bit for bit, except where the residual
 * x - q0 * s underflows (x itself subnormal): there both quotients are far
 * below 2^-11, where every E4M3 code is the signed zero, and the signs agree. */
static int agree(float q, float ref) {
    if (same(q, ref)) return 1;
    return fabsf(q) < 0x1p-11f && fabsf(ref) < 0x1p-11f && signbit(q) == signbit(ref);
}

/* random scale in [1e-12, FLT_MAX / 448]: log-uniform exponent, random significand */
static float rand_scale(uint64_t* st) {
    const double lo = log2(1e-12), hi = log2((double)FLT_MAX / 448.0);
    const double u = (double)(sm64(st) >> 11) * 0x1.0p-53;
    float s = (float)exp2(lo + (hi - lo) * u);
    union { float f; uint32_t u; } b = {s};
    b.u = (b.u & 0xFF800000u) | (uint32_t)(sm64(st) & 0x7FFFFFu);
    s = b.f;
    if (s < 1e-12f) s = 1e-12f;
    if (s > FLT_MAX / 448.0f) s = FLT_MAX / 448.0f;
    return s;
}

/* Any finite x and any scale: below 2^20 the quotient is IEEE's (agree());
 * at or above it, both quotients are beyond 2^17 -- past both FP8 formats'
 * saturation points -- with the same sign. */
uint64_t pin_div_any_x(uint64_t n, uint64_t seed, float* bad_x, float* bad_s) {
    uint64_t bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t t = 0; t < (int64_t)(n >> 12); ++t) {
        uint64_t st = seed * 0x9E3779B97F4A7C15ull + (uint64_t)t;
        const float s = rand_scale(&st);
        for (int i = 0; i < 4096; ++i) {
            union { float f; uint32_t u; } b;
            do { b.u = (uint32_t)sm64(&st); } while (!isfinite(b.f));
            const float x = b.f;
            const float q = method(x, s), ref = exact(x, s);
            int ok;
            if (fabsf(ref) < 0x1p20f)
                ok = agree(q, ref);
            else
                ok = fabsf(q) >= 0x1p17f && signbit(q) == signbit(ref);
            if (!ok) {
                ++bad;
                *bad_x = x;
                *bad_s = s;
            }
        }
    }
    return bad;
}

uint64_t pin_div_random(uint64_t n, uint64_t seed, float* bad_x, float* bad_s) {
    uint64_t bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t t = 0; t < (int64_t)(n >> 12); ++t) {
        uint64_t st = seed * 0x100000001B3ull + (uint64_t)t;
        const float s = rand_scale(&st);
        for (int i = 0; i < 4096; ++i) {
            /* |x| <= 448 s (E4M3 rows) or <= 57344 s (E5M2 KV channels): a
             * random magnitude fraction with random exponent depth */
            const double frac = (double)(sm64(&st) >> 11) * 0x1.0p-53;
            const int depth = (int)(sm64(&st) % 40);
            const double top = (t & 1) ? 57344.0 : 448.0;
            float x = (float)(top * (double)s * frac * exp2(-depth));
            if (sm64(&st) & 1) x = -x;
            if (!agree(method(x, s), exact(x, s))) {
                ++bad;
                *bad_x = x;
                *bad_s = s;
            }
        }
    }
    return bad;
}

/* E4M3 finite magnitudes (exponent bias 7, 3 mantissa bits, subnormals below 2^-6). */
static int e4m3_mags(double* out) {
    int n = 0;
    for (int code = 0; code <= 0x7E; ++code) {
        const int e = code >> 3, m = code & 7;
        out[n++] = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    }
    return n;
}

/* E5M2 finite magnitudes (exponent bias 15, 2 mantissa bits, subnormals below 2^-14). */
static int e5m2_mags(double* out) {
    int n = 0;
    for (int code = 0; code <= 0x7B; ++code) {
        const int e = code >> 2, m = code & 3;
        out[n++] = e == 0 ? ldexp((double)m, -16) : ldexp(1.0 + m / 4.0, e - 15);
    }
    return n;
}

/* fmt 0: E4M3 boundaries, 1: E5M2 boundaries. */
uint64_t pin_div_boundaries(const float* scales, int n_scales, int ulps, int fmt, uint64_t* checked) {
    double mags[127];
    const int nm = fmt == 1 ? e5m2_mags(mags) : e4m3_mags(mags);
    double pts[2 * 127];
    int np = 0;
    for (int i = 0; i < nm; ++i) pts[np++] = mags[i];
    for (int i = 0; i + 1 < nm; ++i) pts[np++] = 0.5 * (mags[i] + mags[i + 1]);
    uint64_t bad = 0, cnt = 0;
#pragma omp parallel for reduction(+ : bad, cnt) schedule(static)
    for (int k = 0; k < n_scales; ++k) {
        const float s = scales[k];
        for (int p = 0; p < np; ++p) {
            const float x0 = (float)(pts[p] * (double)s);
            float lo = x0, hi = x0;
            for (int u = 0; u < ulps; ++u) {
                lo = nextafterf(lo, 0.0f);
                hi = nextafterf(hi, INFINITY);
            }
            for (float x = lo;; x = nextafterf(x, INFINITY)) {
                for (int sg = 0; sg < 2; ++sg) {
                    const float xs = sg ? -x : x;
                    cnt += 1;
                    if (!agree(method(xs, s), exact(xs, s))) bad += 1;
                }
                if (x == hi) break;
            }
        }
    }
    *checked = cnt;
    return bad;
}
