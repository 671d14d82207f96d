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

// A row held in registers is read from HBM exactly once: nontemporal loads
// keep it from displacing cache lines that are still useful.
__device__ __forceinline__ float4 load_nt(const float4* p) {
    const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}

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

// The row scale of each mode: the per-token absmax scale (MODE 0), one static
// per-tensor scale *param for every row (MODE 1: no absmax is taken), or the
// per-token absmax scale with the absmax clipped at *param (MODE 2).
template <int MODE>
__device__ __forceinline__ RowScale mode_scale(float amax, const float* param) {
    if constexpr (MODE == 1) {
        const float s = fmaxf(*param, kScaleFloor);
        return RowScale{s, __fdiv_rn(1.0f, s)};
    } else if constexpr (MODE == 2) {
        return make_row_scale(fminf(amax, *param));
    } else {
        return make_row_scale(amax);
    }
}

// Row held in registers: VPT float4 per thread, K4 = K / 4 <= T * VPT.
template <int VPT, int T, int MODE>
__global__ __launch_bounds__(T) void quantize_rows_regs(const float* __restrict__ x, int64_t ldx,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ scales, int64_t rows, int K4,
                                                        const float* __restrict__ param) {
    __shared__ float red[T / kWave];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float4* xr = reinterpret_cast<const float4*>(x + r * ldx);
        float4 v[VPT];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = i * T + threadIdx.x;
            if (j < K4) {
                // many rows (256-thread blocks): a stream read once, kept out of
                // the caches; decode batches keep plain loads (measured faster)
                if constexpr (T == kQThreads)
                    v[i] = load_nt(xr + j);
                else
                    v[i] = xr[j];
                if constexpr (MODE != 1) amax = absmax4(amax, v[i]);
            }
        }
        if constexpr (MODE != 1) amax = block_max<T>(amax, red);
        const RowScale rs = mode_scale<MODE>(amax, param);
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
template <int T, int MODE>
__global__ __launch_bounds__(T) void quantize_rows_loop(const float* __restrict__ x, int64_t ldx,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ scales, int64_t rows, int64_t K4,
                                                        const float* __restrict__ param) {
    __shared__ float red[T / kWave];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float4* xr = reinterpret_cast<const float4*>(x + r * ldx);
        float amax = 0.0f;
        if constexpr (MODE != 1) {
            for (int64_t j = threadIdx.x; j < K4; j += T) amax = absmax4(amax, xr[j]);
            amax = block_max<T>(amax, red);
        }
        const RowScale rs = mode_scale<MODE>(amax, param);
        if (threadIdx.x == 0) scales[r] = rs.s;
        uint32_t* qr = reinterpret_cast<uint32_t*>(q + r * ldq);
        for (int64_t j = threadIdx.x; j < K4; j += T) qr[j] = cast4(xr[j], rs);
    }
}

template <int T, int MODE>
static void launch_rows(const float* x, int64_t ldx, uint8_t* q, int64_t ldq, float* scales, int64_t rows,
                        int64_t K4, const float* param, hipStream_t stream) {
    const dim3 grid((unsigned)(rows < (1 << 20) ? rows : (1 << 20))), block(T);
    const int k4 = (int)K4;
#define FP8K_Q_REGS(V) \
    hipLaunchKernelGGL((quantize_rows_regs<V, T, MODE>), grid, block, 0, stream, x, ldx, q, ldq, scales, rows, k4, param)
    if (K4 <= T * 1)
        FP8K_Q_REGS(1);
    else if (K4 <= T * 2)
        FP8K_Q_REGS(2);
    else if (K4 <= T * 4)
        FP8K_Q_REGS(4);
    else if (K4 <= T * 8)
        FP8K_Q_REGS(8);
    else if (K4 <= T * 16)
        FP8K_Q_REGS(16);
    else if (T == kQThreads && K4 <= T * 32)
        hipLaunchKernelGGL((quantize_rows_regs<32, kQThreads, MODE>), grid, block, 0, stream, x, ldx, q, ldq, scales,
                           rows, k4, param);
    else
        hipLaunchKernelGGL((quantize_rows_loop<T, MODE>), grid, block, 0, stream, x, ldx, q, ldq, scales, rows, K4,
                           param);
#undef FP8K_Q_REGS
}

template <int MODE>
static hipError_t launch_mode(const float* x, int64_t ldx, uint8_t* q, int64_t ldq, float* scales, int64_t rows,
                              int64_t K, const float* param, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (rows < kQWideRowsBelow)
        launch_rows<kQThreadsWide, MODE>(x, ldx, q, ldq, scales, rows, K / 4, param, stream);
    else
        launch_rows<kQThreads, MODE>(x, ldx, q, ldq, scales, rows, K / 4, param, stream);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const float* x, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                                int64_t rows, int64_t K, hipStream_t stream) {
    return launch_mode<0>(x, ldx, q, ldq, scales, rows, K, nullptr, stream);
}

hipError_t launch_quantize_static(const float* x, int64_t ldx, const float* scale, uint8_t* q, int64_t ldq,
                                  float* scales, int64_t rows, int64_t K, hipStream_t stream) {
    return launch_mode<1>(x, ldx, q, ldq, scales, rows, K, scale, stream);
}

hipError_t launch_quantize_clipped(const float* x, int64_t ldx, const float* clip, uint8_t* q, int64_t ldq,
                                   float* scales, int64_t rows, int64_t K, hipStream_t stream) {
    return launch_mode<2>(x, ldx, q, ldq, scales, rows, K, clip, stream);
}

}  // namespace fp8k
