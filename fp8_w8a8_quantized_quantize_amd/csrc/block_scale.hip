// Block-scaled ("MX") quantization to OCP E4M3 on gfx950.
//
// Every 32 consecutive elements of a row share one power-of-two scale 2^e,
// stored as its exponent byte e + 127 (per-group/block scales of the
// DeepSeek V4 950 page, §2.4 and §4.2; MXFP8 block scaling of the FP8
// deployment page, §7.1, with the 32-element blocks of the open MX format,
// which are also the blocks gfx950's block-scaled MFMA applies).  The scale
// is the absmax/448 scale of the Llama 3 FP8 page, §3.1 (1e-12 floor),
// rounded up to a power of two: v = max(fl32(amax / 448), 1e-12f) and e the
// smallest integer with 2^e >= v, so every |x| / 2^e <= 448 and nothing is
// clipped; codes are E4M3(x * 2^-e), rounded to nearest even.
//
// Scales are stored chunk-major: for each 128-element chunk of K, one 32-bit
// word per row holding the exponent bytes of its 4 blocks (word [chunk][row],
// byte j = block 4 * chunk + j), the order in which the GEMM kernels fetch
// them (a chunk's words for consecutive rows are contiguous).
//
// One float4 per thread; the 8 threads of a block reduce their maxima with
// three butterfly steps.  The stream is read once (nontemporal loads for
// large inputs, as in the per-token quantizer).
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

constexpr int kMxThreads = 256;

__device__ __forceinline__ float4 mx_load(const float4* p, bool nt) {
    if (nt) {
        const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
        return make_float4(t[0], t[1], t[2], t[3]);
    }
    return *p;
}

// Items are the float4 of the matrix in row-major order, K4 = K / 4 per row
// (a multiple of 8, so the 8 lanes of a block always share a row and are
// active together).
template <bool NT>
__global__ __launch_bounds__(kMxThreads) void quantize_mx_kernel(const float* __restrict__ x, int64_t ldx,
                                                                  uint8_t* __restrict__ q, int64_t ldq,
                                                                  uint8_t* __restrict__ sc, int64_t rows,
                                                                  int64_t K4, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * kMxThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kMxThreads) {
        const int64_t row = i / K4;
        const int64_t c4 = i - row * K4;
        const float4 v = mx_load(reinterpret_cast<const float4*>(x + row * ldx) + c4, NT);
        float amax = absmax4(0.0f, v);
        amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
        // v = max(fl32(amax / 448), 1e-12f) is a normal float: e is its
        // exponent, plus one unless v is a power of two
        const uint32_t bits = __float_as_uint(fmaxf(__fdiv_rn(amax, kE4M3Max), kScaleFloor));
        const int e = (int)(bits >> 23) - 127 + ((bits & 0x7FFFFFu) != 0u);
        const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-39, 120]
        *reinterpret_cast<uint32_t*>(q + row * ldq + 4 * c4) = cvt4_e4m3(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
        // chunk-major: byte j of word [chunk][row] is block 4 * chunk + j
        if ((c4 & 7) == 0) sc[((c4 >> 5) * rows + row) * 4 + ((c4 >> 3) & 3)] = (uint8_t)(e + 127);
    }
}

hipError_t launch_quantize_mx(const float* x, int64_t ldx, uint8_t* q, int64_t ldq, uint8_t* scales, int64_t rows,
                              int64_t K, hipStream_t stream) {
    const int64_t K4 = K / 4;
    const int64_t total = rows * K4;
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + kMxThreads - 1) / kMxThreads;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    if (rows >= 512)
        hipLaunchKernelGGL(quantize_mx_kernel<true>, dim3((unsigned)blocks), dim3(kMxThreads), 0, stream, x, ldx, q,
                           ldq, scales, rows, K4, total);
    else
        hipLaunchKernelGGL(quantize_mx_kernel<false>, dim3((unsigned)blocks), dim3(kMxThreads), 0, stream, x, ldx, q,
                           ldq, scales, rows, K4, total);
    return hipGetLastError();
}

}  // namespace fp8k
