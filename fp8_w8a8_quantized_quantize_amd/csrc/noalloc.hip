// Allocation-free form of the fused quantize + GEMM call, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It runs exactly the kernels of
// fp8_quant_gemm_fused; the scratch those kernels use (the staged activation
// codes and scales, the skinny GEMM's split-K partial sums) lives in one
// file-scope device array instead of a caller-given workspace.
//
// The array is a static __device__ object, so each GPU the library runs on
// holds its own copy (FP8_NOALLOC_SCRATCH_BYTES) until the process ends.  In
// host code its name is only a host-side stand-in: the device address comes
// from hipGetSymbolAddress, taken once per device (with that device current)
// on the first call there, and only that address is handed to the kernels.
// Every call on one GPU shares the array; nothing in it has to start at zero
// (every kernel that reads it first writes what it reads in the same call),
// and calls that overlap on one GPU race on it.
#include "../../include/fp8w8a8.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

static_assert(FP8_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

__device__ __align__(256) uint8_t scratch[FP8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once.
fp8_status_t scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8_ERR_DEVICE;
    if (dev >= kMaxDevices) return FP8_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return FP8_ERR_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FP8_OK;
}

}  // namespace

extern "C" fp8_status_t fp8_quant_gemm_fused_noalloc(const float* x, int64_t ldx, const uint8_t* qw, int64_t ldw,
                                                     const float* s_ch, uint16_t* y, int64_t ldy, int64_t M,
                                                     int64_t N, int64_t K, uint8_t* qa_out, float* s_tok_out,
                                                     hipStream_t stream) {
    // sizes first (host only): SIZE_MAX for invalid sizes, above the array's
    // size for problems too large for it
    const size_t need = fp8_workspace_bytes(M, N, K);
    if (need == SIZE_MAX) return M < 0 || N < 0 || K < 0 ? FP8_ERR_INVALID_ARGUMENT : FP8_ERR_UNSUPPORTED;
    if (need > (size_t)FP8_NOALLOC_SCRATCH_BYTES) return FP8_ERR_WORKSPACE;
    // the stream must belong to the current device, whose copy of the array is used
    if (stream != nullptr) {
        int cur = -1, sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess)
            return FP8_ERR_DEVICE;
        if (cur != sdev) return FP8_ERR_INVALID_ARGUMENT;
    }
    void* ws = nullptr;
    const fp8_status_t st = scratch_on_current_device(&ws);
    if (st != FP8_OK) return st;
    return fp8_quant_gemm_fused(x, ldx, qw, ldw, s_ch, y, ldy, M, N, K, qa_out, s_tok_out, ws,
                                (size_t)FP8_NOALLOC_SCRATCH_BYTES, stream);
}
