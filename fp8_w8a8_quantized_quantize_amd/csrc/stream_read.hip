// HBM read ceiling: a plain streaming read of a buffer, the yardstick for the
// weight-streaming decode GEMMs (DeepSeek V4 950 page, §1.2: decode time is
// the time to move the weights).  Measurement utility; not on the layer's path.
//
// Workgroup b of G reads a contiguous share of the buffer with 16-byte loads,
// UNROLL loads in flight per thread (the same request size and depth the
// decode kernels use), and folds the data into one 32-bit value per thread.
// The value is stored only when it equals kMagic, so the loads cannot be
// dropped and the kernel writes (almost) nothing.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

namespace {
constexpr uint32_t kMagic = 0x9E3779B9u;
constexpr int kThreads = 256;
constexpr int kUnroll = 8;
}  // namespace

template <bool NONTEMPORAL>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const v4i* __restrict__ p, int64_t n16,
                                                              int64_t per_wg, uint32_t* __restrict__ sink) {
    const int64_t begin = (int64_t)blockIdx.x * per_wg;
    const int64_t end = min(begin + per_wg, n16);
    uint32_t acc = 0;
    int64_t i = begin + threadIdx.x;
    // full rounds: kUnroll loads of 16 bytes per thread issued back to back
    for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
        v4i v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = NONTEMPORAL ? __builtin_nontemporal_load(p + i + u * kThreads) : p[i + u * kThreads];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    }
    for (; i < end; i += kThreads) {
        const v4i v = p[i];
        acc ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
    }
    if (acc == kMagic) sink[0] = acc;
}

hipError_t launch_stream_read(const void* p, size_t bytes, int workgroups, bool nontemporal, uint32_t* sink,
                              hipStream_t stream) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0 || workgroups <= 0) return hipSuccess;
    // a share per workgroup, rounded up to whole rounds of the block
    const int64_t round = (int64_t)kThreads * kUnroll;
    int64_t per = (n16 + workgroups - 1) / workgroups;
    per = (per + round - 1) / round * round;
    const unsigned grid = (unsigned)((n16 + per - 1) / per);
    const v4i* src = static_cast<const v4i*>(p);
    if (nontemporal)
        hipLaunchKernelGGL(stream_read_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, src, n16, per, sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, src, n16, per, sink);
    return hipGetLastError();
}

}  // namespace fp8k
