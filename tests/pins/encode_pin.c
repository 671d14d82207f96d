/*
 * Exhaustive pin of an fp32 -> FP8 encoder (E4M3 or E5M2): for every one of
 * the 2^32 fp32 bit patterns, the encoder's code must be the brute-force
 * answer:
 *   - NaN input   -> S.1111111 (sign kept);
 *   - otherwise   -> the finite FP8 value nearest to |v| (values above the
 *                    largest finite one saturate to it), ties to the even
 *                    code, sign of v attached (so -0 and tiny negatives give
 *                    0x80).
 * Finite non-negative codes are 0x00 .. nmag-1 in increasing order in both
 * formats (127 of them in E4M3, 124 in E5M2, whose 0x7C is infinity).
 * The finite magnitudes come from the caller (a table decoded by an
 * independent library), so this file holds no E4M3 arithmetic of its own.
 * Nearest is found by binary search over the sorted magnitudes and decided
 * by an exact comparison with the midpoint of the two neighbours.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdatomic.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef uint8_t (*enc_fn)(float);

static uint8_t brute(float v, const double* mags, int nmag) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= mags[nmag - 1]) return (uint8_t)(sign | (nmag - 1));
    int lo = 0, hi = nmag - 1;           /* mags[lo] <= a < mags[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (mags[mid] <= a) lo = mid; else hi = mid;
    }
    double midpt = 0.5 * (mags[lo] + mags[hi]);  /* exact in binary64 */
    int code;
    if (a < midpt) code = lo;
    else if (a > midpt) code = hi;
    else code = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | code);
}

/* Checks patterns [start, end).  `mags` holds the nmag non-negative finite
 * magnitudes in code order.  Returns the mismatch count; the first
 * mismatching pattern goes to *first_bad. */
uint64_t pin_encode_range_n(enc_fn enc, const double* mags, int nmag, uint64_t start, uint64_t end,
                            uint32_t* first_bad) {
    uint64_t bad = 0;
    uint64_t first = UINT64_MAX;
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad) reduction(min : first)
    for (uint64_t u = start; u < end; ++u) {
        uint32_t bits = (uint32_t)u;
        float v;
        memcpy(&v, &bits, 4);
        if (enc(v) != brute(v, mags, nmag)) {
            bad += 1;
            if (u < first) first = u;
        }
    }
    *first_bad = (first == UINT64_MAX) ? 0 : (uint32_t)first;
    return bad;
}

uint64_t pin_encode_range(enc_fn enc, const double* mags, uint64_t start, uint64_t end, uint32_t* first_bad) {
    return pin_encode_range_n(enc, mags, 127, start, end, first_bad);
}

/* The brute-force answer for one value (used to cross-check single cases). */
uint8_t pin_encode_one_n(const double* mags, int nmag, float v) { return brute(v, mags, nmag); }
uint8_t pin_encode_one(const double* mags, float v) { return brute(v, mags, 127); }
