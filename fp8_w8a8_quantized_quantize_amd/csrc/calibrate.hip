// Calibration of a static activation scale (DeepSeek V4 950 page, §3.1 and
// §4.2: the static part of the activation scale comes from the P99.9
// percentile of |x| over calibration data instead of the maximum, so that rare
// outliers do not shrink everyone's precision; values beyond the range are
// clipped).
//
// The percentile is the nearest-rank one: the rank-th smallest |x|.  It is
// found exactly by a four-pass radix select on the magnitude bits (for
// non-negative floats the bit pattern orders like the value): each pass
// histograms one byte of the keys that share the bytes chosen so far (LDS
// histograms per workgroup, added into a 256-bin global histogram), then one
// workgroup picks the byte whose cumulative count reaches the remaining rank.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

namespace {

struct SelectState {
    uint32_t hist[256];
    uint32_t prefix;  // key bytes chosen so far
    uint32_t pad;
    unsigned long long rank;  // rank still to find among keys that match prefix
};
static_assert(sizeof(SelectState) <= kCalibrateWsBytes, "calibration workspace");

__global__ __launch_bounds__(256) void select_init(SelectState* st, unsigned long long rank) {
    st->hist[threadIdx.x] = 0u;
    if (threadIdx.x == 0) {
        st->prefix = 0u;
        st->pad = 0u;
        st->rank = rank;
    }
}

__global__ __launch_bounds__(256) void select_hist(const float* __restrict__ x, int64_t n, SelectState* st,
                                                   int shift) {
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0u;
    __syncthreads();
    const uint32_t prefix = st->prefix;
    const uint32_t hi = shift >= 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const uint32_t key = __float_as_uint(x[i]) & 0x7FFFFFFFu;
        if (((key ^ prefix) & hi) == 0u) atomicAdd(&h[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t c = h[threadIdx.x];
    if (c != 0u) atomicAdd(&st->hist[threadIdx.x], c);
}

// One workgroup of 256 threads: inclusive prefix sum of the histogram, the
// byte whose range holds the remaining rank, then the histogram is cleared
// for the next pass.
__global__ __launch_bounds__(256) void select_pick(SelectState* st, int shift) {
    __shared__ unsigned long long c[256];
    const int t = threadIdx.x;
    const unsigned long long v = st->hist[t];
    c[t] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const unsigned long long add = t >= off ? c[t - off] : 0ull;
        __syncthreads();
        c[t] += add;
        __syncthreads();
    }
    const unsigned long long rank = st->rank;
    const unsigned long long incl = c[t], excl = incl - v;
    __syncthreads();
    if (v != 0ull && excl < rank && rank <= incl) {
        st->prefix |= (uint32_t)t << shift;
        st->rank = rank - excl;
    }
    st->hist[t] = 0u;
}

__global__ void select_finish(const SelectState* st, float* value_out, float* scale_out) {
    const float v = __uint_as_float(st->prefix);
    *value_out = v;
    if (scale_out != nullptr) scale_out[0] = fmaxf(__fdiv_rn(v, kE4M3Max), kScaleFloor);
}

}  // namespace

hipError_t launch_calibrate_percentile(const float* x, int64_t n, int64_t rank, float* value_out, float* scale_out,
                                       void* ws, hipStream_t stream) {
    SelectState* st = static_cast<SelectState*>(ws);
    hipLaunchKernelGGL(select_init, dim3(1), dim3(256), 0, stream, st, (unsigned long long)rank);
    const int64_t blocks64 = (n + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 2048 ? blocks64 : 2048);
    for (int shift = 24; shift >= 0; shift -= 8) {
        hipLaunchKernelGGL(select_hist, dim3(blocks), dim3(256), 0, stream, x, n, st, shift);
        hipLaunchKernelGGL(select_pick, dim3(1), dim3(256), 0, stream, st, shift);
    }
    hipLaunchKernelGGL(select_finish, dim3(1), dim3(1), 0, stream, st, value_out, scale_out);
    return hipGetLastError();
}

}  // namespace fp8k
