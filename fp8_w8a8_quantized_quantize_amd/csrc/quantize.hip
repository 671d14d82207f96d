// Per-row absmax quantization to OCP E4M3 on gfx950.
//
// One row per workgroup (256 threads, or 1024 when there are few rows).  A
// row is read from HBM once: up to 32 (256 threads) or 16 (1024 threads)
// float4 per thread stay in registers between the absmax pass and the cast
// pass, with all of a row's loads in flight at once; longer rows are re-read
// for the cast, from L2.  The absmax is a wave64 butterfly max (order
// independent, so it is exact) followed by a per-wave LDS reduction.  Scale
// and codes follow the Llama 3 FP8 page, §3.1: s = max(fl32(amax / 448),
// 1e-12f) and code = E4M3(fl32(x / s)) rounded to nearest even and saturated
// at +-448; the quotient is formed from the correctly rounded reciprocal of s
// and two FMAs, which gives the IEEE quotient (div_by_scale in
// device_common.hpp).
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

// Block sizes: 256 threads per row when there are many rows, 1024 when there
// are fewer rows than twice the CU count (decode batches), so a few long rows
// still keep many loads in flight per CU.
constexpr int kQThreads = 256;
constexpr int kQThreadsWide = 1024;
constexpr int64_t kQWideRowsBelow = 512;

template <int T>
__device__ __forceinline__ float block_max(float v, float* red) {
    constexpr int W = T / kWave;
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < W; ++i) r = fmaxf(r, red[i]);
    __syncthreads();  // red may be rewritten by the next row
    return r;
}

// Row held in registers: VPT float4 per thread, K4 = K / 4 <= T * VPT.
template <int VPT, int T>
__global__ __launch_bounds__(T) void quantize_rows_regs(const float* __restrict__ x, int64_t ldx,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ scales, int64_t rows, int K4) {
    __shared__ float red[T / kWave];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float4* xr = reinterpret_cast<const float4*>(x + r * ldx);
        float4 v[VPT];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = i * T + threadIdx.x;
            if (j < K4) {
                v[i] = xr[j];
                amax = absmax4(amax, v[i]);
            }
        }
        amax = block_max<T>(amax, red);
        const RowScale rs = make_row_scale(amax);
        if (threadIdx.x == 0) scales[r] = rs.s;
        uint32_t* qr = reinterpret_cast<uint32_t*>(q + r * ldq);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = i * T + threadIdx.x;
            if (j < K4) qr[j] = cast4(v[i], rs);
        }
    }
}

// Any K: absmax pass, then a second (L2-resident) pass for the cast.
template <int T>
__global__ __launch_bounds__(T) void quantize_rows_loop(const float* __restrict__ x, int64_t ldx,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ scales, int64_t rows, int64_t K4) {
    __shared__ float red[T / kWave];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float4* xr = reinterpret_cast<const float4*>(x + r * ldx);
        float amax = 0.0f;
        for (int64_t j = threadIdx.x; j < K4; j += T) amax = absmax4(amax, xr[j]);
        amax = block_max<T>(amax, red);
        const RowScale rs = make_row_scale(amax);
        if (threadIdx.x == 0) scales[r] = rs.s;
        uint32_t* qr = reinterpret_cast<uint32_t*>(q + r * ldq);
        for (int64_t j = threadIdx.x; j < K4; j += T) qr[j] = cast4(xr[j], rs);
    }
}

template <int T>
static void launch_rows(const float* x, int64_t ldx, uint8_t* q, int64_t ldq, float* scales, int64_t rows,
                        int64_t K4, hipStream_t stream) {
    const dim3 grid((unsigned)(rows < (1 << 20) ? rows : (1 << 20))), block(T);
    const int k4 = (int)K4;
    if (K4 <= T * 1)
        hipLaunchKernelGGL((quantize_rows_regs<1, T>), grid, block, 0, stream, x, ldx, q, ldq, scales, rows, k4);
    else if (K4 <= T * 2)
        hipLaunchKernelGGL((quantize_rows_regs<2, T>), grid, block, 0, stream, x, ldx, q, ldq, scales, rows, k4);
    else if (K4 <= T * 4)
        hipLaunchKernelGGL((quantize_rows_regs<4, T>), grid, block, 0, stream, x, ldx, q, ldq, scales, rows, k4);
    else if (K4 <= T * 8)
        hipLaunchKernelGGL((quantize_rows_regs<8, T>), grid, block, 0, stream, x, ldx, q, ldq, scales, rows, k4);
    else if (K4 <= T * 16)
        hipLaunchKernelGGL((quantize_rows_regs<16, T>), grid, block, 0, stream, x, ldx, q, ldq, scales, rows, k4);
    else if (T == kQThreads && K4 <= T * 32)
        hipLaunchKernelGGL((quantize_rows_regs<32, kQThreads>), grid, block, 0, stream, x, ldx, q, ldq, scales, rows,
                           k4);
    else
        hipLaunchKernelGGL((quantize_rows_loop<T>), grid, block, 0, stream, x, ldx, q, ldq, scales, rows, K4);
}

hipError_t launch_quantize_rows(const float* x, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                                int64_t rows, int64_t K, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (rows < kQWideRowsBelow)
        launch_rows<kQThreadsWide>(x, ldx, q, ldq, scales, rows, K / 4, stream);
    else
        launch_rows<kQThreads>(x, ldx, q, ldq, scales, rows, K / 4, stream);
    return hipGetLastError();
}

}  // namespace fp8k
