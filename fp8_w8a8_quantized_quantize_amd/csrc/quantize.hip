// Per-row absmax quantization to OCP E4M3 on gfx950.
//
// One row per workgroup of 256 threads (4 waves).  A row is read from HBM
// once: rows with K <= 32768 stay in registers between the absmax pass and
// the cast pass (all of a row's loads are in flight at once, which is what
// makes the few-row decode case fast); longer rows are re-read for the cast,
// from L2.  The absmax is
// a wave64 butterfly max (order independent, so it is exact) followed by a
// 4-entry LDS reduction.  Scale and codes follow the Llama 3 FP8 page, §3.1:
// s = max(fl32(amax / 448), 1e-12f), code = E4M3(fl32(x / s)) with an IEEE
// correctly rounded division, round to nearest even, saturation at +-448.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

constexpr int kQThreads = 256;

__device__ __forceinline__ float block_max_256(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) red[w] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();  // red may be rewritten by the next row
    return r;
}

__device__ __forceinline__ float absmax4(float m, const float4& v) {
    return fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ float row_scale(float amax) {
    float s = __fdiv_rn(amax, kE4M3Max);
    return s < kScaleFloor ? kScaleFloor : s;
}

__device__ __forceinline__ uint32_t cast4(const float4& v, float s) {
    return cvt4_e4m3(__fdiv_rn(v.x, s), __fdiv_rn(v.y, s), __fdiv_rn(v.z, s), __fdiv_rn(v.w, s));
}

// Row held in registers: VPT float4 per thread, K4 = K / 4 <= 256 * VPT.
template <int VPT>
__global__ __launch_bounds__(kQThreads) void quantize_rows_regs(const float* __restrict__ x, int64_t ldx,
                                                                 uint8_t* __restrict__ q, int64_t ldq,
                                                                 float* __restrict__ scales, int64_t rows,
                                                                 int K4) {
    __shared__ float red[4];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float4* xr = reinterpret_cast<const float4*>(x + r * ldx);
        float4 v[VPT];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = i * kQThreads + threadIdx.x;
            if (j < K4) {
                v[i] = xr[j];
                amax = absmax4(amax, v[i]);
            }
        }
        amax = block_max_256(amax, red);
        const float s = row_scale(amax);
        if (threadIdx.x == 0) scales[r] = s;
        uint32_t* qr = reinterpret_cast<uint32_t*>(q + r * ldq);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = i * kQThreads + threadIdx.x;
            if (j < K4) qr[j] = cast4(v[i], s);
        }
    }
}

// Any K: absmax pass, then a second (L2-resident) pass for the cast.
__global__ __launch_bounds__(kQThreads) void quantize_rows_loop(const float* __restrict__ x, int64_t ldx,
                                                                 uint8_t* __restrict__ q, int64_t ldq,
                                                                 float* __restrict__ scales, int64_t rows,
                                                                 int64_t K4) {
    __shared__ float red[4];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float4* xr = reinterpret_cast<const float4*>(x + r * ldx);
        float amax = 0.0f;
        for (int64_t j = threadIdx.x; j < K4; j += kQThreads) amax = absmax4(amax, xr[j]);
        amax = block_max_256(amax, red);
        const float s = row_scale(amax);
        if (threadIdx.x == 0) scales[r] = s;
        uint32_t* qr = reinterpret_cast<uint32_t*>(q + r * ldq);
        for (int64_t j = threadIdx.x; j < K4; j += kQThreads) qr[j] = cast4(xr[j], s);
    }
}

hipError_t launch_quantize_rows(const float* x, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                                int64_t rows, int64_t K, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const int64_t K4 = K / 4;
    const unsigned grid = (unsigned)(rows < (1 << 20) ? rows : (1 << 20));
    const dim3 block(kQThreads);
    if (K4 <= 256 * 1)
        hipLaunchKernelGGL(quantize_rows_regs<1>, dim3(grid), block, 0, stream, x, ldx, q, ldq, scales, rows, (int)K4);
    else if (K4 <= 256 * 2)
        hipLaunchKernelGGL(quantize_rows_regs<2>, dim3(grid), block, 0, stream, x, ldx, q, ldq, scales, rows, (int)K4);
    else if (K4 <= 256 * 4)
        hipLaunchKernelGGL(quantize_rows_regs<4>, dim3(grid), block, 0, stream, x, ldx, q, ldq, scales, rows, (int)K4);
    else if (K4 <= 256 * 8)
        hipLaunchKernelGGL(quantize_rows_regs<8>, dim3(grid), block, 0, stream, x, ldx, q, ldq, scales, rows, (int)K4);
    else if (K4 <= 256 * 16)
        hipLaunchKernelGGL(quantize_rows_regs<16>, dim3(grid), block, 0, stream, x, ldx, q, ldq, scales, rows, (int)K4);
    else if (K4 <= 256 * 32)
        hipLaunchKernelGGL(quantize_rows_regs<32>, dim3(grid), block, 0, stream, x, ldx, q, ldq, scales, rows, (int)K4);
    else
        hipLaunchKernelGGL(quantize_rows_loop, dim3(grid), block, 0, stream, x, ldx, q, ldq, scales, rows, K4);
    return hipGetLastError();
}

}  // namespace fp8k
