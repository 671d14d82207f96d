// FP8 KV-cache codec on gfx950: per-channel scales, quantize into paged
// cache blocks, and read back.
//
// The cache keeps K/V rows in FP8, E5M2 by default for its wider range
// (DeepSeek V4 950 page, §2.1) or E4M3, with one scale per channel (per
// latent dimension in §2.2 of the same page; per channel on the 512K-context
// page, §3.3, and the FP8 deployment page, §2.3).  Rows live in fixed-size
// blocks of a shared pool; a per-token slot index (physical block times block
// size plus offset, resolved from the request's block table) says where each
// token's row goes (512K-context page, §3.3).
//
// All three kernels are HBM-bound streams.  A thread owns four adjacent
// channels (one float4 of a row, one 32-bit word of codes) and walks down a
// range of rows, so a wave touches 1 KB of fp32 or 256 B of codes per row,
// contiguous, and the per-channel scale and its reciprocal are formed once
// per thread, not per element.  The fp32 stream that is read once (the
// batch) and the one that is written once (the read back) go through
// nontemporal loads and stores: measured on MI355X they lift the batch read
// from about 5.4 to 6.4 TB/s and the read back from 4.6 to 6.7 TB/s.
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

constexpr float kE5M2Max = 57344.0f;  // largest finite E5M2 value
constexpr int kKvThreads = 256;       // 4 channels per thread: 1024 channels per workgroup
constexpr int kKvUnroll = 8;          // rows in flight per thread (maximum pass, read back)
constexpr int kKvQuantUnroll = 16;    // rows in flight per thread (quantize)

__device__ __forceinline__ float4 load_nt(const float4* p) {
    const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}

__device__ __forceinline__ void store_nt(const float4& v, float4* p) {
    const v4f t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<v4f*>(p));
}

// Two fp32 -> FP8 codes in bytes [2*HI, 2*HI+1] of `old`, clamped to the
// format's largest finite value first so the conversion saturates; the
// hardware convert rounds to nearest even.
template <int FMT, bool HI>
__device__ __forceinline__ int kv_cvt2(float a, float b, int old) {
    constexpr float m = FMT == kKvE5M2 ? kE5M2Max : kE4M3Max;
    a = __builtin_amdgcn_fmed3f(a, -m, m);
    b = __builtin_amdgcn_fmed3f(b, -m, m);
    if constexpr (FMT == kKvE5M2)
        return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
    else
        return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Four codes (bytes, little-endian) -> four exact fp32 values.
template <int FMT>
__device__ __forceinline__ float4 kv_decode4(uint32_t w) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    v2f lo, hi;
    if constexpr (FMT == kKvE5M2) {
        lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
    } else {
        lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    }
    return make_float4(lo[0], lo[1], hi[0], hi[1]);
}

__device__ __forceinline__ float4 abs_max4(float4 m, const float4& v) {
    return make_float4(fmaxf(m.x, fabsf(v.x)), fmaxf(m.y, fabsf(v.y)), fmaxf(m.z, fabsf(v.z)), fmaxf(m.w, fabsf(v.w)));
}

// Column |x| maxima of one chunk of rows: grid.x spans the channel groups,
// grid.y the row chunks.  The partial of chunk k for channel group g goes to
// part[g * chunks + k], so the reduction reads each group's partials
// contiguously.
__global__ __launch_bounds__(kKvThreads) void kv_amax_partial(const float* __restrict__ kv, int64_t ld4, int T,
                                                              int C4, int rows_per_chunk, int chunks,
                                                              float4* __restrict__ part) {
    const int g = blockIdx.x * kKvThreads + threadIdx.x;
    if (g >= C4) return;
    const int r0 = blockIdx.y * rows_per_chunk;
    const int r1 = min(T, r0 + rows_per_chunk);
    const float4* p = reinterpret_cast<const float4*>(kv) + g;
    float4 m = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int r = r0;
    for (; r + kKvUnroll <= r1; r += kKvUnroll) {
        float4 v[kKvUnroll];
#pragma unroll
        for (int i = 0; i < kKvUnroll; ++i) v[i] = load_nt(p + (int64_t)(r + i) * ld4);
#pragma unroll
        for (int i = 0; i < kKvUnroll; ++i) m = abs_max4(m, v[i]);
    }
    for (; r < r1; ++r) m = abs_max4(m, load_nt(p + (int64_t)r * ld4));
    part[(int64_t)g * chunks + blockIdx.y] = m;
}

// One wave per channel group: the 64 lanes stride over the chunks' partials,
// a butterfly max joins them, and lane 0 writes the four scales
// max(fl32(amax / fmt_max), 1e-12f).
template <int FMT>
__global__ __launch_bounds__(kKvThreads) void kv_scale_finish(const float4* __restrict__ part, int chunks, int C4,
                                                              float4* __restrict__ scales) {
    const int g = blockIdx.x * (kKvThreads / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (g >= C4) return;  // whole waves leave together: g is uniform in a wave
    const float4* p = part + (int64_t)g * chunks;
    float4 m = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int k = lane; k < chunks; k += kWave) {
        const float4 v = p[k];
        m = make_float4(fmaxf(m.x, v.x), fmaxf(m.y, v.y), fmaxf(m.z, v.z), fmaxf(m.w, v.w));
    }
    m = make_float4(wave_max(m.x), wave_max(m.y), wave_max(m.z), wave_max(m.w));
    if (lane == 0) {
        constexpr float fm = FMT == kKvE5M2 ? kE5M2Max : kE4M3Max;
        float4 s = make_float4(__fdiv_rn(m.x, fm), __fdiv_rn(m.y, fm), __fdiv_rn(m.z, fm), __fdiv_rn(m.w, fm));
        s.x = fmaxf(s.x, kScaleFloor);
        s.y = fmaxf(s.y, kScaleFloor);
        s.z = fmaxf(s.z, kScaleFloor);
        s.w = fmaxf(s.w, kScaleFloor);
        scales[g] = s;
    }
}

__device__ __forceinline__ RowScale channel_scale(float s) {
    s = fmaxf(s, kScaleFloor);
    return RowScale{s, __fdiv_rn(1.0f, s)};
}

template <int FMT>
__device__ __forceinline__ uint32_t kv_encode4(const float4& v, const RowScale (&rs)[4]) {
    int w = kv_cvt2<FMT, false>(div_by_scale(v.x, rs[0]), div_by_scale(v.y, rs[1]), 0);
    w = kv_cvt2<FMT, true>(div_by_scale(v.z, rs[2]), div_by_scale(v.w, rs[3]), w);
    return (uint32_t)w;
}

// Rows [r0, r1) of the batch into their cache slots.  Tokens whose slot is
// outside [0, num_slots) are skipped.
template <int FMT>
__global__ __launch_bounds__(kKvThreads) void kv_quantize_paged(const float* __restrict__ kv, int64_t ld4,
                                                                const float* __restrict__ scales,
                                                                const int32_t* __restrict__ slot,
                                                                uint8_t* __restrict__ cache, int64_t num_slots, int T,
                                                                int C4, int rows_per_block) {
    const int g = blockIdx.x * kKvThreads + threadIdx.x;
    if (g >= C4) return;
    const float4 s4 = reinterpret_cast<const float4*>(scales)[g];
    const RowScale rs[4] = {channel_scale(s4.x), channel_scale(s4.y), channel_scale(s4.z), channel_scale(s4.w)};
    const int r0 = blockIdx.y * rows_per_block;
    const int r1 = min(T, r0 + rows_per_block);
    const float4* p = reinterpret_cast<const float4*>(kv) + g;
    uint32_t* out = reinterpret_cast<uint32_t*>(cache) + g;
    const int64_t c4 = C4;
    int r = r0;
    for (; r + kKvQuantUnroll <= r1; r += kKvQuantUnroll) {
        float4 v[kKvQuantUnroll];
        int sl[kKvQuantUnroll];
#pragma unroll
        for (int i = 0; i < kKvQuantUnroll; ++i) {
            sl[i] = slot[r + i];
            v[i] = load_nt(p + (int64_t)(r + i) * ld4);
        }
#pragma unroll
        for (int i = 0; i < kKvQuantUnroll; ++i)
            if (sl[i] >= 0 && sl[i] < num_slots) out[(int64_t)sl[i] * c4] = kv_encode4<FMT>(v[i], rs);
    }
    for (; r < r1; ++r) {
        const int s = slot[r];
        if (s >= 0 && s < num_slots) out[(int64_t)s * c4] = kv_encode4<FMT>(load_nt(p + (int64_t)r * ld4), rs);
    }
}

// out[t, :] = decoded cache row slot[t] times the channel scales; a slot
// outside [0, num_slots) reads as code 0, so its row is all +0.
template <int FMT>
__global__ __launch_bounds__(kKvThreads) void kv_dequantize_paged(const uint8_t* __restrict__ cache, int64_t num_slots,
                                                                  const int32_t* __restrict__ slot,
                                                                  const float* __restrict__ scales,
                                                                  float* __restrict__ outp, int64_t ldo4, int T,
                                                                  int C4, int rows_per_block) {
    const int g = blockIdx.x * kKvThreads + threadIdx.x;
    if (g >= C4) return;
    float4 s = reinterpret_cast<const float4*>(scales)[g];
    s = make_float4(fmaxf(s.x, kScaleFloor), fmaxf(s.y, kScaleFloor), fmaxf(s.z, kScaleFloor), fmaxf(s.w, kScaleFloor));
    const int r0 = blockIdx.y * rows_per_block;
    const int r1 = min(T, r0 + rows_per_block);
    const uint32_t* in = reinterpret_cast<const uint32_t*>(cache) + g;
    float4* out = reinterpret_cast<float4*>(outp) + g;
    const int64_t c4 = C4;
    int r = r0;
    for (; r + kKvUnroll <= r1; r += kKvUnroll) {
        uint32_t w[kKvUnroll];
#pragma unroll
        for (int i = 0; i < kKvUnroll; ++i) {
            const int sl = slot[r + i];
            w[i] = (sl >= 0 && sl < num_slots) ? in[(int64_t)sl * c4] : 0u;
        }
#pragma unroll
        for (int i = 0; i < kKvUnroll; ++i) {
            const float4 d = kv_decode4<FMT>(w[i]);
            store_nt(make_float4(d.x * s.x, d.y * s.y, d.z * s.z, d.w * s.w), out + (int64_t)(r + i) * ldo4);
        }
    }
    for (; r < r1; ++r) {
        const int sl = slot[r];
        const uint32_t w = (sl >= 0 && sl < num_slots) ? in[(int64_t)sl * c4] : 0u;
        const float4 d = kv_decode4<FMT>(w);
        store_nt(make_float4(d.x * s.x, d.y * s.y, d.z * s.z, d.w * s.w), out + (int64_t)r * ldo4);
    }
}

// ---------------------------------------------------------------- host ----

namespace {

// Grid sizes, from a sweep on MI355X over a 32768 x 2048 batch: the maximum
// pass is fastest with one workgroup per CU, each streaming long column
// ranges (42 us vs 54 us at 4 per CU); quantize and read back with about 8
// per CU.
constexpr int64_t kKvAmaxBlocks = 256;
constexpr int64_t kKvTargetBlocks = 2048;
constexpr int64_t kKvMinRows = 16;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Row ranges per workgroup so the grid has about `target` workgroups and no
// workgroup takes fewer than kKvMinRows rows (or all of them).
int64_t rows_per_block(int64_t T, int64_t col_blocks, int64_t target) {
    int64_t row_blocks = ceil_div(target, col_blocks);
    row_blocks = std::min<int64_t>(row_blocks, std::max<int64_t>(1, ceil_div(T, kKvMinRows)));
    return std::max<int64_t>(1, ceil_div(T, row_blocks));
}

}  // namespace

KvChunks kv_amax_chunks(int64_t T, int64_t C) {
    const int64_t col_blocks = ceil_div(C / 4, kKvThreads);
    const int64_t rpc = rows_per_block(T, std::max<int64_t>(col_blocks, 1), kKvAmaxBlocks);
    return KvChunks{(int)rpc, (int)std::max<int64_t>(1, ceil_div(T, rpc))};
}

size_t kv_scales_ws_bytes(int64_t T, int64_t C) { return (size_t)kv_amax_chunks(T, C).chunks * (size_t)C * 4; }

hipError_t launch_kv_channel_scales(const float* kv, int64_t T, int64_t C, int64_t ldkv, int fmt, float* scales,
                                    void* ws, hipStream_t stream) {
    const int C4 = (int)(C / 4);
    const KvChunks ch = kv_amax_chunks(T, C);
    float4* part = static_cast<float4*>(ws);
    const dim3 g1((unsigned)ceil_div(C4, kKvThreads), (unsigned)ch.chunks);
    hipLaunchKernelGGL(kv_amax_partial, g1, dim3(kKvThreads), 0, stream, kv, ldkv / 4, (int)T, C4, ch.rows_per_chunk,
                       ch.chunks, part);
    const dim3 g2((unsigned)ceil_div(C4, kKvThreads / kWave));
    if (fmt == kKvE5M2)
        hipLaunchKernelGGL(kv_scale_finish<kKvE5M2>, g2, dim3(kKvThreads), 0, stream, part, ch.chunks, C4,
                           reinterpret_cast<float4*>(scales));
    else
        hipLaunchKernelGGL(kv_scale_finish<kKvE4M3>, g2, dim3(kKvThreads), 0, stream, part, ch.chunks, C4,
                           reinterpret_cast<float4*>(scales));
    return hipGetLastError();
}

hipError_t launch_kv_quantize_paged(const float* kv, int64_t T, int64_t C, int64_t ldkv, const float* scales, int fmt,
                                    const int32_t* slot, uint8_t* cache, int64_t num_slots, hipStream_t stream) {
    const int C4 = (int)(C / 4);
    const int64_t cb = ceil_div(C4, kKvThreads);
    const int64_t rpb = rows_per_block(T, cb, kKvTargetBlocks);
    const dim3 grid((unsigned)cb, (unsigned)ceil_div(T, rpb));
    if (fmt == kKvE5M2)
        hipLaunchKernelGGL(kv_quantize_paged<kKvE5M2>, grid, dim3(kKvThreads), 0, stream, kv, ldkv / 4, scales, slot,
                           cache, num_slots, (int)T, C4, (int)rpb);
    else
        hipLaunchKernelGGL(kv_quantize_paged<kKvE4M3>, grid, dim3(kKvThreads), 0, stream, kv, ldkv / 4, scales, slot,
                           cache, num_slots, (int)T, C4, (int)rpb);
    return hipGetLastError();
}

hipError_t launch_kv_dequantize_paged(const uint8_t* cache, int64_t num_slots, const int32_t* slot, int64_t T,
                                      int64_t C, const float* scales, int fmt, float* out, int64_t ldo,
                                      hipStream_t stream) {
    const int C4 = (int)(C / 4);
    const int64_t cb = ceil_div(C4, kKvThreads);
    const int64_t rpb = rows_per_block(T, cb, kKvTargetBlocks);
    const dim3 grid((unsigned)cb, (unsigned)ceil_div(T, rpb));
    if (fmt == kKvE5M2)
        hipLaunchKernelGGL(kv_dequantize_paged<kKvE5M2>, grid, dim3(kKvThreads), 0, stream, cache, num_slots, slot,
                           scales, out, ldo / 4, (int)T, C4, (int)rpb);
    else
        hipLaunchKernelGGL(kv_dequantize_paged<kKvE4M3>, grid, dim3(kKvThreads), 0, stream, cache, num_slots, slot,
                           scales, out, ldo / 4, (int)T, C4, (int)rpb);
    return hipGetLastError();
}

}  // namespace fp8k
