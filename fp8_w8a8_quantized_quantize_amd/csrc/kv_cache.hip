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
// channels (16 bytes of an fp32 row or 8 of a bf16 / fp16 row, one 32-bit word
// of codes) and walks down a range of rows, so a wave touches contiguous
// memory per row, and the per-channel scale and its reciprocal are formed
// once per thread, not per element.  KV rows may arrive as fp32, bf16 or
// fp16 (the pages convert FP16 KV to FP8; 512K-context page, §3.3); a
// 16-bit value converts to fp32 exactly, so the codes depend only on the
// value.  The read back is written as fp32, bf16 or fp16, rounded to
// nearest even from the fp32 product.  The fp32 stream that is read once (the
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

typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_to_float(uint32_t h) {
    _Float16 f;
    const uint16_t b = (uint16_t)h;
    __builtin_memcpy(&f, &b, 2);
    return (float)f;
}

__device__ __forceinline__ uint32_t float_to_half_bits(float x) {
    const _Float16 f = (_Float16)x;  // round to nearest even
    uint16_t b;
    __builtin_memcpy(&b, &f, 2);
    return b;
}

// Quads (4 consecutive channels) per thread: one 16-byte load covers 4
// fp32 or 8 bf16 / fp16 channels.
template <int DT>
constexpr int kv_quads() {
    return DT == kKvF32 ? 1 : 2;
}

// The 4 * Q elements of a KV row at element offset `e` from `base`, as fp32
// quads; DT: kKvF32, kKvBF16 or kKvF16.  Read once: nontemporal.
template <int DT>
__device__ __forceinline__ void kv_load(const void* base, int64_t e, float4 (&v)[kv_quads<DT>()]) {
    if constexpr (DT == kKvF32) {
        v[0] = load_nt(reinterpret_cast<const float4*>(static_cast<const float*>(base) + e));
    } else {
        const v4u w = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(static_cast<const uint16_t*>(base) + e));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t a = w[2 * q], b = w[2 * q + 1];
            if constexpr (DT == kKvBF16)
                v[q] = make_float4(__uint_as_float(a << 16), __uint_as_float(a & 0xFFFF0000u), __uint_as_float(b << 16),
                                   __uint_as_float(b & 0xFFFF0000u));
            else
                v[q] = make_float4(half_to_float(a & 0xFFFFu), half_to_float(a >> 16), half_to_float(b & 0xFFFFu),
                                   half_to_float(b >> 16));
        }
    }
}

// 4 * Q fp32 values to consecutive output elements (written once).
template <int DT>
__device__ __forceinline__ void kv_store(void* base, int64_t e, const float4 (&v)[kv_quads<DT>()]) {
    if constexpr (DT == kKvF32) {
        store_nt(v[0], reinterpret_cast<float4*>(static_cast<float*>(base) + e));
    } else {
        v4u w;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if constexpr (DT == kKvBF16) {
                w[2 * q] = pack_bf16x2(v[q].x, v[q].y);
                w[2 * q + 1] = pack_bf16x2(v[q].z, v[q].w);
            } else {
                w[2 * q] = float_to_half_bits(v[q].x) | (float_to_half_bits(v[q].y) << 16);
                w[2 * q + 1] = float_to_half_bits(v[q].z) | (float_to_half_bits(v[q].w) << 16);
            }
        }
        __builtin_nontemporal_store(w, reinterpret_cast<v4u*>(static_cast<uint16_t*>(base) + e));
    }
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

// Column |x| maxima of one chunk of rows.  grid.x spans the channel groups,
// kWave quads per workgroup, grid.y the row chunks; each of the workgroup's
// waves takes one contiguous slice of the chunk's rows (more loads in flight
// per CU than one wave per column range), and LDS joins the slices.  The
// partial of chunk k for quad G (channels 4G .. 4G + 3) goes to
// part[G * chunks + k], so the reduction reads each quad's partials
// contiguously.
template <int DT>
__global__ __launch_bounds__(kKvThreads) void kv_amax_partial(const void* __restrict__ kv, int64_t ld, int T,
                                                              int CQ, int rows_per_chunk, int chunks,
                                                              float4* __restrict__ part) {
    constexpr int Q = kv_quads<DT>();
    constexpr int S = kKvThreads / kWave;  // row slices, one per wave
    __shared__ float4 red[S - 1][Q][kWave];
    const int lane = threadIdx.x % kWave;
    const int w = threadIdx.x / kWave;
    const int g = blockIdx.x * kWave + lane;  // channels [4Qg, 4Qg + 4Q)
    const bool live = g < CQ;
    const int r0 = blockIdx.y * rows_per_chunk;
    const int n = max(0, min(T - r0, rows_per_chunk));
    const int per = (n + S - 1) / S;
    const int r1 = r0 + min(n, (w + 1) * per);
    const int64_t e0 = 4 * Q * (int64_t)g;
    float4 m[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) m[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (live) {
        int r = r0 + min(n, w * per);
        for (; r + kKvUnroll <= r1; r += kKvUnroll) {
            float4 v[kKvUnroll][Q];
#pragma unroll
            for (int i = 0; i < kKvUnroll; ++i) kv_load<DT>(kv, (int64_t)(r + i) * ld + e0, v[i]);
#pragma unroll
            for (int i = 0; i < kKvUnroll; ++i)
#pragma unroll
                for (int q = 0; q < Q; ++q) m[q] = abs_max4(m[q], v[i][q]);
        }
        for (; r < r1; ++r) {
            float4 v[Q];
            kv_load<DT>(kv, (int64_t)r * ld + e0, v);
#pragma unroll
            for (int q = 0; q < Q; ++q) m[q] = abs_max4(m[q], v[q]);
        }
    }
    if (w > 0) {
#pragma unroll
        for (int q = 0; q < Q; ++q) red[w - 1][q][lane] = m[q];
    }
    __syncthreads();
    if (w == 0 && live) {
#pragma unroll
        for (int k = 0; k < S - 1; ++k)
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const float4 o = red[k][q][lane];
                m[q] = make_float4(fmaxf(m[q].x, o.x), fmaxf(m[q].y, o.y), fmaxf(m[q].z, o.z), fmaxf(m[q].w, o.w));
            }
#pragma unroll
        for (int q = 0; q < Q; ++q) part[((int64_t)Q * g + q) * chunks + blockIdx.y] = m[q];
    }
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

// fl32(d * s) per element.  The product must be rounded to fp32 before any
// narrowing store: left to itself the compiler fuses the multiply and the
// fp16 conversion into one mixed-precision FMA (a single rounding, and
// -0 * s + 0 = +0), which changes fp16 results; the empty asm pins each
// product in a register as an fp32 value.
__device__ __forceinline__ float4 scale4(const float4& d, const float4& s) {
    float4 p = make_float4(d.x * s.x, d.y * s.y, d.z * s.z, d.w * s.w);
    asm volatile("" : "+v"(p.x), "+v"(p.y), "+v"(p.z), "+v"(p.w));
    return p;
}

// Rows [r0, r1) of the batch into their cache slots.  Tokens whose slot is
// outside [0, num_slots) are skipped.
template <int FMT, int DT>
__global__ __launch_bounds__(kKvThreads) void kv_quantize_paged(const void* __restrict__ kv, int64_t ld,
                                                                const float* __restrict__ scales,
                                                                const int32_t* __restrict__ slot,
                                                                uint8_t* __restrict__ cache, int64_t num_slots, int T,
                                                                int CQ, int rows_per_block) {
    constexpr int Q = kv_quads<DT>();
    constexpr int U = kKvQuantUnroll / Q;  // rows in flight: 16 (fp32) or 8 (16-bit, 16 channels each)
    const int g = blockIdx.x * kKvThreads + threadIdx.x;
    if (g >= CQ) return;
    RowScale rs[Q][4];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const float4 s4 = reinterpret_cast<const float4*>(scales)[Q * g + q];
        rs[q][0] = channel_scale(s4.x);
        rs[q][1] = channel_scale(s4.y);
        rs[q][2] = channel_scale(s4.z);
        rs[q][3] = channel_scale(s4.w);
    }
    const int r0 = blockIdx.y * rows_per_block;
    const int r1 = min(T, r0 + rows_per_block);
    const int64_t e0 = 4 * Q * (int64_t)g;
    const int64_t C = 4 * Q * (int64_t)CQ;  // cache row length in bytes
    auto encode = [&](const float4 (&v)[Q], uint32_t (&w)[Q]) {
#pragma unroll
        for (int q = 0; q < Q; ++q) w[q] = kv_encode4<FMT>(v[q], rs[q]);
    };
    auto put = [&](int s, const uint32_t (&w)[Q]) {
        uint8_t* dst = cache + (int64_t)s * C + e0;
        if constexpr (Q == 1)
            *reinterpret_cast<uint32_t*>(dst) = w[0];
        else
            *reinterpret_cast<v2u*>(dst) = v2u{w[0], w[1]};
    };
    int r = r0;
    for (; r + U <= r1; r += U) {
        float4 v[U][Q];
        int sl[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            sl[i] = slot[r + i];
            kv_load<DT>(kv, (int64_t)(r + i) * ld + e0, v[i]);
        }
        // Every row is encoded, and only the store depends on its slot: were
        // the encode left inside the slot test, the compiler would sink a
        // row's load into that branch, and the wait for that load (the last
        // one issued) would also wait for all the others.
        uint32_t w[U][Q];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            encode(v[i], w[i]);
#pragma unroll
            for (int q = 0; q < Q; ++q) asm volatile("" : "+v"(w[i][q]));
        }
#pragma unroll
        for (int i = 0; i < U; ++i)
            if (sl[i] >= 0 && sl[i] < num_slots) put(sl[i], w[i]);
    }
    for (; r < r1; ++r) {
        const int s = slot[r];
        if (s >= 0 && s < num_slots) {
            float4 v[Q];
            uint32_t w[Q];
            kv_load<DT>(kv, (int64_t)r * ld + e0, v);
            encode(v, w);
            put(s, w);
        }
    }
}

// out[t, :] = decoded cache row slot[t] times the channel scales; a slot
// outside [0, num_slots) reads as code 0, so its row is all +0.
template <int FMT, int DT>
__global__ __launch_bounds__(kKvThreads) void kv_dequantize_paged(const uint8_t* __restrict__ cache, int64_t num_slots,
                                                                  const int32_t* __restrict__ slot,
                                                                  const float* __restrict__ scales,
                                                                  void* __restrict__ out, int64_t ldo, int T,
                                                                  int CQ, int rows_per_block) {
    constexpr int Q = kv_quads<DT>();
    const int g = blockIdx.x * kKvThreads + threadIdx.x;
    if (g >= CQ) return;
    float4 s[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const float4 t = reinterpret_cast<const float4*>(scales)[Q * g + q];
        s[q] = make_float4(fmaxf(t.x, kScaleFloor), fmaxf(t.y, kScaleFloor), fmaxf(t.z, kScaleFloor),
                           fmaxf(t.w, kScaleFloor));
    }
    const int r0 = blockIdx.y * rows_per_block;
    const int r1 = min(T, r0 + rows_per_block);
    const int64_t e0 = 4 * Q * (int64_t)g;
    const int64_t C = 4 * Q * (int64_t)CQ;
    auto fetch = [&](int r, uint32_t (&w)[Q]) {
        const int sl = slot[r];
        const bool ok = sl >= 0 && sl < num_slots;
        const uint8_t* src = cache + (int64_t)(ok ? sl : 0) * C + e0;
        if constexpr (Q == 1) {
            w[0] = ok ? *reinterpret_cast<const uint32_t*>(src) : 0u;
        } else {
            const v2u t = ok ? *reinterpret_cast<const v2u*>(src) : v2u{0u, 0u};
            w[0] = t[0];
            w[1] = t[1];
        }
    };
    auto emit = [&](int r, const uint32_t (&w)[Q]) {
        float4 o[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) o[q] = scale4(kv_decode4<FMT>(w[q]), s[q]);
        kv_store<DT>(out, (int64_t)r * ldo + e0, o);
    };
    int r = r0;
    for (; r + kKvUnroll <= r1; r += kKvUnroll) {
        uint32_t w[kKvUnroll][Q];
#pragma unroll
        for (int i = 0; i < kKvUnroll; ++i) fetch(r + i, w[i]);
#pragma unroll
        for (int i = 0; i < kKvUnroll; ++i) emit(r + i, w[i]);
    }
    for (; r < r1; ++r) {
        uint32_t w[Q];
        fetch(r, w);
        emit(r, w);
    }
}

// ---------------------------------------------------------------- host ----

namespace {

// Grid sizes, from a sweep on MI355X over a 32768 x 2048 batch: the maximum
// pass is fastest with one workgroup per CU, each streaming long column
// ranges (42 us vs 54 us at 4 per CU); quantize and read back with about 8
// per CU.
constexpr int64_t kKvAmaxBlocks = 1024;
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

// Row chunks of the channel-maxima pass for rows read `quads` channel quads
// per thread (1 for fp32, 2 for 16-bit elements).
KvChunks kv_amax_chunks(int64_t T, int64_t C, int quads) {
    const int64_t col_blocks = ceil_div(C / 4 / quads, kWave);
    const int64_t rpc = rows_per_block(T, std::max<int64_t>(col_blocks, 1), kKvAmaxBlocks);
    return KvChunks{(int)rpc, (int)std::max<int64_t>(1, ceil_div(T, rpc))};
}

// Sized for the element type with the most chunks (the 16-bit one).
size_t kv_scales_ws_bytes(int64_t T, int64_t C) { return (size_t)kv_amax_chunks(T, C, 2).chunks * (size_t)C * 4; }

// Dispatch on the element type (DT) and the code format (FMT).
#define FP8K_KV_DT(dt, CALL)                 \
    switch (dt) {                            \
        case kKvBF16: CALL(kKvBF16); break;  \
        case kKvF16: CALL(kKvF16); break;    \
        default: CALL(kKvF32); break;        \
    }

hipError_t launch_kv_channel_scales(const void* kv, int dtype, int64_t T, int64_t C, int64_t ldkv, int fmt,
                                    float* scales, void* ws, hipStream_t stream) {
    const int C4 = (int)(C / 4);
    const KvChunks ch = kv_amax_chunks(T, C, dtype == kKvF32 ? 1 : 2);
    float4* part = static_cast<float4*>(ws);
#define FP8K_KV_AMAX(D)                                                                                              \
    {                                                                                                                \
        const int cq = C4 / kv_quads<D>();                                                                           \
        const dim3 g1((unsigned)ceil_div(cq, kWave), (unsigned)ch.chunks);                                           \
        hipLaunchKernelGGL(kv_amax_partial<D>, g1, dim3(kKvThreads), 0, stream, kv, ldkv, (int)T, cq, ch.rows_per_chunk, \
                           ch.chunks, part);                                                                         \
    }
    FP8K_KV_DT(dtype, FP8K_KV_AMAX)
#undef FP8K_KV_AMAX
    const dim3 g2((unsigned)ceil_div(C4, kKvThreads / kWave));
    if (fmt == kKvE5M2)
        hipLaunchKernelGGL(kv_scale_finish<kKvE5M2>, g2, dim3(kKvThreads), 0, stream, part, ch.chunks, C4,
                           reinterpret_cast<float4*>(scales));
    else
        hipLaunchKernelGGL(kv_scale_finish<kKvE4M3>, g2, dim3(kKvThreads), 0, stream, part, ch.chunks, C4,
                           reinterpret_cast<float4*>(scales));
    return hipGetLastError();
}

hipError_t launch_kv_quantize_paged(const void* kv, int dtype, int64_t T, int64_t C, int64_t ldkv, const float* scales,
                                    int fmt, const int32_t* slot, uint8_t* cache, int64_t num_slots,
                                    hipStream_t stream) {
    const int C4 = (int)(C / 4);
#define FP8K_KV_Q(D)                                                                                                   \
    {                                                                                                                  \
        const int cq = C4 / kv_quads<D>();                                                                             \
        const int64_t cb = ceil_div(cq, kKvThreads);                                                                   \
        const int64_t rpb = rows_per_block(T, cb, kKvTargetBlocks);                                                    \
        const dim3 grid((unsigned)cb, (unsigned)ceil_div(T, rpb));                                                     \
        if (fmt == kKvE5M2)                                                                                            \
            hipLaunchKernelGGL((kv_quantize_paged<kKvE5M2, D>), grid, dim3(kKvThreads), 0, stream, kv, ldkv, scales,    \
                               slot, cache, num_slots, (int)T, cq, (int)rpb);                                          \
        else                                                                                                           \
            hipLaunchKernelGGL((kv_quantize_paged<kKvE4M3, D>), grid, dim3(kKvThreads), 0, stream, kv, ldkv, scales,    \
                               slot, cache, num_slots, (int)T, cq, (int)rpb);                                          \
    }
    FP8K_KV_DT(dtype, FP8K_KV_Q)
#undef FP8K_KV_Q
    return hipGetLastError();
}

hipError_t launch_kv_dequantize_paged(const uint8_t* cache, int64_t num_slots, const int32_t* slot, int64_t T,
                                      int64_t C, const float* scales, int fmt, void* out, int out_dtype, int64_t ldo,
                                      hipStream_t stream) {
    const int C4 = (int)(C / 4);
#define FP8K_KV_DQ(D)                                                                                                  \
    {                                                                                                                  \
        const int cq = C4 / kv_quads<D>();                                                                             \
        const int64_t cb = ceil_div(cq, kKvThreads);                                                                   \
        const int64_t rpb = rows_per_block(T, cb, kKvTargetBlocks);                                                    \
        const dim3 grid((unsigned)cb, (unsigned)ceil_div(T, rpb));                                                     \
        if (fmt == kKvE5M2)                                                                                            \
            hipLaunchKernelGGL((kv_dequantize_paged<kKvE5M2, D>), grid, dim3(kKvThreads), 0, stream, cache, num_slots,  \
                               slot, scales, out, ldo, (int)T, cq, (int)rpb);                                          \
        else                                                                                                           \
            hipLaunchKernelGGL((kv_dequantize_paged<kKvE4M3, D>), grid, dim3(kKvThreads), 0, stream, cache, num_slots,  \
                               slot, scales, out, ldo, (int)T, cq, (int)rpb);                                          \
    }
    FP8K_KV_DT(out_dtype, FP8K_KV_DQ)
#undef FP8K_KV_DQ
    return hipGetLastError();
}
#undef FP8K_KV_DT

}  // namespace fp8k
