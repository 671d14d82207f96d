// Device helpers shared by the gfx950 kernels of the FP8 W8A8 linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Largest finite OCP E4M3 value and the scale floor (Llama 3 FP8 page, §1.1
// range; §3.1 absmax/448 conversion clamped below at 1e-12).
constexpr float kE4M3Max = 448.0f;
constexpr float kScaleFloor = 1e-12f;

// Two fp32 -> OCP E4M3 codes in bytes [2*HI, 2*HI+1] of `old`.  The clamp to
// +-448 first (FP8 deployment page, §2.3) makes the conversion saturating;
// the hardware convert rounds to nearest even (MODE register default).
template <bool HI>
__device__ __forceinline__ int cvt2_e4m3(float a, float b, int old) {
    a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
    b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Four fp32 -> four E4M3 codes packed little-endian in a 32-bit word.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
    int w = cvt2_e4m3<false>(a, b, 0);
    w = cvt2_e4m3<true>(c, d, w);
    return (uint32_t)w;
}

// fp32 -> bf16 bits, round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bf16_rne_bits(lo) | (bf16_rne_bits(hi) << 16);
}

// D += A * B on a 16x16x128 FP8 (E4M3 x E4M3) tile, FP32 accumulate.
// A: 16 rows x 128 k, B: 128 k x 16 columns; each lane supplies 32 bytes of
// its row (A) or column (B).  The k order inside the 32 bytes is the same for
// A and B, so any fixed assignment of k indices to (lane group, byte) that
// both operands share gives the dot product.  D: lane l holds column l % 16,
// rows 4 * (l / 16) + {0, 1, 2, 3}.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i join(const v4i& lo, const v4i& hi) {
    v8i r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Cross-lane max over a wave of 64.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Per-token quantization steps shared by the quantizer and the fused decode
// GEMM (Llama 3 FP8 page, §3.1): running |x| maximum, the row scale
// s = max(fl32(amax / 448), 1e-12f) and the codes E4M3(fl32(x / s)).
__device__ __forceinline__ float absmax4(float m, const float4& v) {
    return fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ float row_scale(float amax) {
    float s = __fdiv_rn(amax, kE4M3Max);
    return s < kScaleFloor ? kScaleFloor : s;
}

// A row's scale and its correctly rounded reciprocal.
struct RowScale {
    float s, r;
};

__device__ __forceinline__ RowScale make_row_scale(float amax) {
    const float s = row_scale(amax);
    return RowScale{s, __fdiv_rn(1.0f, s)};
}

// fl32(x / s) from r = RN(1 / s): q0 = RN(x r) is within one ulp of x / s,
// the residual q0 s - x is exact in one FMA, and RN(q0 - residual * r) is
// then the correctly rounded quotient (Markstein's division theorem; a
// reciprocal and two FMAs instead of a full IEEE division per element).  The
// residual is taken as q0 s - x and subtracted, not as x - q0 s and added:
// for x = -0 the former is +0 and q0 - (+0) r = -0, so signed zeros come out
// right with no extra instruction (the other order gives +0 there).  Where x
// is subnormal the residual can lose bits, but the quotient is then below
// 2^-11, whose E4M3 code is the signed zero either way (E5M2's smallest step
// is 2^-16, so there too), and its sign is still that of x.
// q0 is clamped to +-2^20: when x * r overflows fp32 (a static or stale
// scale far below |x| / 448) the residual would otherwise be inf - inf; a
// clamped quotient is past every FP8 code and still saturates.  A CPU test
// checks all of this against IEEE division on random, overflowing and
// FP8-boundary quotients.
__device__ __forceinline__ float div_by_scale(float x, const RowScale& rs) {
    const float q0 = __builtin_amdgcn_fmed3f(x * rs.r, -1048576.0f, 1048576.0f);
    const float d = __builtin_fmaf(q0, rs.s, -x);
    return __builtin_fmaf(d, -rs.r, q0);
}

__device__ __forceinline__ uint32_t cast4(const float4& v, const RowScale& rs) {
    return cvt4_e4m3(div_by_scale(v.x, rs), div_by_scale(v.y, rs), div_by_scale(v.z, rs), div_by_scale(v.w, rs));
}

__device__ __forceinline__ v4i load16(const uint8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// Kernels that take more than 64 KB of dynamic LDS need this opt-in before launch.
#define FP8K_SET_LDS(KERNEL, BYTES) \
    hipFuncSetAttribute(reinterpret_cast<const void*>(&KERNEL), hipFuncAttributeMaxDynamicSharedMemorySize, (BYTES))

}  // namespace fp8k
