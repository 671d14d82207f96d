// Skinny-M (decode) scaled FP8 GEMM on gfx950: y[M,N] = epi(qa[M,K] . qw[N,K]^T), M <= 64.
//
// Decode is bound by streaming the weights from HBM (DeepSeek V4 950 page,
// §1.2: every generated token moves the layer's weights; FP8 halves the bytes
// moved).  The kernel therefore reads every weight byte exactly once, straight
// into registers in the MFMA operand layout (no LDS staging for W), keeps
// several 128-byte k chunks per row in flight, and spends MFMA slots freely
// (M = 8 uses half of a 16-wide tile).
//
// Work split: a workgroup of KW waves owns NT x 16 weight rows; its waves take
// interleaved 128-byte k chunks (wave w: chunks w, w+KW, ...) and are summed in
// LDS in a fixed wave order at the end, so results are bit-reproducible.
// Measured on MI355X: the activation fragments (re-read from L2 for every
// 16 * NT weight rows) are what limits M = 64; larger NT cuts them.
// MFMA A operand = 16 weight rows, B operand = 16 activation rows, so each
// lane of the 16x16 result holds 4 consecutive output columns of one token
// row (one 8-byte BF16 store).
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

// Keeps the compiler's scheduler from moving any instruction across this
// point: each step's loads are issued right after the step they replace is
// consumed, in program order (the order they return in), and the next step's
// operand selects cannot be hoisted above this step's MFMAs (a hoisted select
// would wait for loads that are meant to stay in flight).
__device__ __forceinline__ void issue_order_fence() { __builtin_amdgcn_sched_barrier(0); }

// Lane `lane` supplies bytes [16g, 16g+16) and [64+16g, 64+16g+16) of a
// 128-byte k chunk (g = lane / 16) for A and B alike.
//
// Split K (part != nullptr): workgroup (x, z) covers the k chunks
// [z * split_chunks, (z + 1) * split_chunks) and writes its fp32 sums to
// part[z][m][n] (row stride N); skinny_splitk_reduce adds the splits in order
// z = 0, 1, ... and applies the epilogue.
//
// Block-scaled operands (MX = true): every 32 k of a row carry a power-of-two
// scale (exponent byte), chunk-major in mx.sa / mx.sw (32-bit word
// [chunk][row]); the hardware's block-scaled MFMA applies them, so there are
// no s_tok / s_ch and y = bf16_rne(acc).  In this lane layout the scale that
// lane group g supplies covers k [32g, 32g + 32) of the 128-byte chunk
// (measured on gfx950), so each lane passes byte g of its row's chunk word.
// K must be a multiple of 128.
template <int MT, int NT, int KW, int DEPTH, bool MX>
__global__ __launch_bounds__(KW * 64) void gemm_skinny_kernel(
    const uint8_t* __restrict__ qa, int64_t lda, const float* __restrict__ s_tok,
    const uint8_t* __restrict__ qw, int64_t ldw, const float* __restrict__ s_ch,
    uint16_t* __restrict__ y, float* __restrict__ y32, int64_t ldy, int M, int N, int K, float* __restrict__ part,
    int split_chunks, MxScales mx) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * (NT * 16);
    const int c0 = blockIdx.z * split_chunks;
    const int nchunks = min((K + 127) >> 7, c0 + split_chunks) - c0;
    // Chunk order of a wave: interleaved (wave w: chunks w, w + KW, ...) for
    // one activation tile, whose one-kernel fused variant must add in the same
    // order; with more tiles (M > 16), one contiguous range per wave, which
    // streams a 235 MB weight matrix markedly faster (measured on MI355X with
    // the same loads and no arithmetic: 44 vs 52 us for 128-row workgroups).
    constexpr bool CONTIG = MT > 1;
    const int per = (nchunks + KW - 1) / KW;
    const int cw0 = CONTIG ? c0 + wave * per : c0 + wave;
    const int steps = CONTIG ? max(0, min(nchunks - wave * per, per))
                             : (nchunks > wave ? (nchunks - wave + KW - 1) / KW : 0);
    auto chunk_of = [&](int s) { return CONTIG ? cw0 + s : cw0 + KW * s; };

    const uint8_t* wrow[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = n0 + 16 * j + r16;
        wrow[j] = qw + (int64_t)(n < N ? n : 0) * ldw;
    }
    const uint8_t* xrow[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = 16 * i + r16;
        xrow[i] = qa + (int64_t)(m < M ? m : 0) * lda;
    }
    constexpr int SD = MX ? DEPTH : 1;  // scale words in flight
    const uint8_t* wsrow[NT];
    const uint8_t* xsrow[MT];
    if constexpr (MX) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int n = n0 + 16 * j + r16;
            wsrow[j] = mx.sw + 4 * (int64_t)(n < N ? n : 0);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int m = 16 * i + r16;
            xsrow[i] = mx.sa + 4 * (int64_t)(m < M ? m : 0);
        }
    }

    v4f acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    v4i wb[DEPTH][NT][2];
    v4i xb[DEPTH][MT][2];
    uint32_t wsc[SD][NT], xsc[SD][MT];  // block scales of the chunk (MX)
    const v4i zero = v4i{0, 0, 0, 0};

    // Loads are issued raw and consumed DEPTH steps later; the operand
    // selects that zero a partial last k chunk happen at the point of use and
    // a scheduling barrier closes every step, so the compiler waits for exactly
    // the loads of the step being consumed while the next DEPTH - 1 steps stay
    // in flight (vector loads return in order: a select hoisted next to a load
    // would make the wave wait for everything issued before it).  Offsets past
    // K read the row's first bytes (K >= 16 whenever a step runs).  Rows past
    // N or M read row 0: they only feed output elements that are never stored.
    auto load_step = [&](int s, int d) {
        const int kb = chunk_of(s) * 128;
        const int o0 = kb + 16 * g < K ? kb + 16 * g : 0;
        const int o1 = kb + 64 + 16 * g < K ? kb + 64 + 16 * g : 0;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            wb[d][j][0] = load16(wrow[j] + o0);
            wb[d][j][1] = load16(wrow[j] + o1);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            xb[d][i][0] = load16(xrow[i] + o0);
            xb[d][i][1] = load16(xrow[i] + o1);
        }
        if constexpr (MX) {
            const int64_t chunk = kb >> 7;  // the chunk's word of 4 block scales (K % 128 == 0)
#pragma unroll
            for (int j = 0; j < NT; ++j)
                wsc[d][j] = *reinterpret_cast<const uint32_t*>(wsrow[j] + chunk * 4 * (int64_t)N);
#pragma unroll
            for (int i = 0; i < MT; ++i)
                xsc[d][i] = *reinterpret_cast<const uint32_t*>(xsrow[i] + chunk * 4 * (int64_t)M);
        }
    };

    if (steps > 0) {
        // (unconditional, so the compiler knows the return order exactly;
        // steps beyond the last repeat it and are never consumed)
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load_step(min(d, steps - 1), d);
        issue_order_fence();
        for (int s0 = 0; s0 < steps; s0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int s = s0 + d;
                const int kb = chunk_of(s) * 128;
                const bool ok0 = s < steps && kb + 16 * g < K;
                const bool ok1 = s < steps && kb + 64 + 16 * g < K;
                v8i xf[MT];
#pragma unroll
                for (int i = 0; i < MT; ++i) xf[i] = join(ok0 ? xb[d][i][0] : zero, ok1 ? xb[d][i][1] : zero);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const v8i a = join(ok0 ? wb[d][j][0] : zero, ok1 ? wb[d][j][1] : zero);
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        if constexpr (MX)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                a, xf[i], acc[i][j], 0, 0, 0, (int)((wsc[d % SD][j] >> (8 * g)) & 0xFFu), 0,
                                (int)((xsc[d % SD][i] >> (8 * g)) & 0xFFu));
                        else
                            acc[i][j] = mfma_16x16x128_e4m3(a, xf[i], acc[i][j]);
                    }
                }
                if (s + DEPTH < steps) load_step(s + DEPTH, d);
                issue_order_fence();
            }
        }
    }

    // Sum the KW partial tiles in wave order 0..KW-1, then the epilogue
    // y = bf16_rne(acc * (s_tok[m] * s_ch[n])).
    __shared__ v4f red[KW][MT * NT][64];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) red[wave][i * NT + j][lane] = acc[i][j];
    __syncthreads();
    for (int t = wave; t < MT * NT; t += KW) {
        v4f sum = red[0][t][lane];
#pragma unroll
        for (int w = 1; w < KW; ++w) sum += red[w][t][lane];
        const int i = t / NT, j = t % NT;
        const int m = 16 * i + r16;
        const int nb = n0 + 16 * j + 4 * g;
        if (m >= M || nb >= N) continue;
        if (part != nullptr) {
            float* pr = part + ((int64_t)blockIdx.z * M + m) * N;
            if (nb + 3 < N && (N & 3) == 0) {
                *reinterpret_cast<float4*>(pr + nb) = make_float4(sum[0], sum[1], sum[2], sum[3]);
            } else {
                for (int v = 0; v < 4 && nb + v < N; ++v) pr[nb + v] = sum[v];
            }
            continue;
        }
        if constexpr (MX) {  // block scales already applied: y = bf16_rne(acc)
            uint16_t* yr = y + (int64_t)m * ldy;
            if (nb + 3 < N && (ldy & 3) == 0) {
                uint2 o;
                o.x = pack_bf16x2(sum[0], sum[1]);
                o.y = pack_bf16x2(sum[2], sum[3]);
                *reinterpret_cast<uint2*>(yr + nb) = o;
            } else {
                for (int v = 0; v < 4 && nb + v < N; ++v) yr[nb + v] = (uint16_t)bf16_rne_bits(sum[v]);
            }
            continue;
        }
        const float st = s_tok[m];
        if (y32 != nullptr) {  // fp32 output: acc * (s_tok * s_ch), unrounded
            float* yr = y32 + (int64_t)m * ldy;
            if (nb + 3 < N && (ldy & 3) == 0) {
                const float4 sc = *reinterpret_cast<const float4*>(s_ch + nb);
                *reinterpret_cast<float4*>(yr + nb) =
                    make_float4(sum[0] * (st * sc.x), sum[1] * (st * sc.y), sum[2] * (st * sc.z), sum[3] * (st * sc.w));
            } else {
                for (int v = 0; v < 4 && nb + v < N; ++v) yr[nb + v] = sum[v] * (st * s_ch[nb + v]);
            }
            continue;
        }
        uint16_t* yr = y + (int64_t)m * ldy;
        if (nb + 3 < N && (ldy & 3) == 0) {
            const float4 sc = *reinterpret_cast<const float4*>(s_ch + nb);
            uint2 o;
            o.x = pack_bf16x2(sum[0] * (st * sc.x), sum[1] * (st * sc.y));
            o.y = pack_bf16x2(sum[2] * (st * sc.z), sum[3] * (st * sc.w));
            *reinterpret_cast<uint2*>(yr + nb) = o;
        } else {
            for (int v = 0; v < 4 && nb + v < N; ++v)
                yr[nb + v] = (uint16_t)bf16_rne_bits(sum[v] * (st * s_ch[nb + v]));
        }
    }
}

// Fused per-token quantization + skinny GEMM for a few rows whose codes fit in
// LDS and whose fp32 values fit in 16 float4 registers per lane: M <= 8 rows
// of K <= 4096 (wave w holds row w) or M <= 16 rows of K <= 2048 (wave w holds
// rows w and w + 8).  Every workgroup issues its loads of x first and its
// first DEPTH steps of weight loads right after them (vector loads complete in
// issue order, so the quantization can start while the weight stream is in
// flight), quantizes the whole activation matrix itself exactly as the
// stand-alone quantizer does, into an LDS copy of the codes, and then runs the
// weight-streaming loop above with the activation fragments read from LDS.
// Workgroup 0 also writes the codes and scales to qa_out / s_tok_out when
// those are given.
constexpr int kFusedRowPad = 16;          // bytes after each LDS code row (bank spread)
constexpr int kFusedRegVec = 16;          // float4 registers per lane for x
constexpr int kFusedWaves = 8;

template <int NT, int KW, int DEPTH>
__global__ __launch_bounds__(KW * 64) void gemm_skinny_fused_kernel(
    const float* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ qw, int64_t ldw,
    const float* __restrict__ s_ch, uint16_t* __restrict__ y, int64_t ldy, int M, int N, int K,
    uint8_t* __restrict__ qa_out, float* __restrict__ s_tok_out) {
    extern __shared__ __align__(16) uint8_t fused_smem[];
    __shared__ float s_tok_sh[16];
    __shared__ v4f red[KW][NT][64];
    static_assert(KW == kFusedWaves, "one or two rows per wave cover M <= 16");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * (NT * 16);
    const int nchunks = (K + 127) >> 7;
    const int steps = nchunks > wave ? (nchunks - wave + KW - 1) / KW : 0;
    const int ldq = K + kFusedRowPad;
    uint8_t* xq = fused_smem;

    // ---- x loads, then the first weight steps.  Everything up to the first
    // use of x is unconditional (indexes are clamped instead), so the compiler
    // knows that the x loads return first and waits for them alone.
    // Register e holds row wave + KW * slot(e), float4 index lane + 64 * idx(e):
    // one row per wave: slot = 0, idx = e; two rows: slot = e / 8, idx = e % 8.
    // A wave without a row, or an index past the row, re-reads a valid float4
    // that is then ignored.
    const int K4 = K >> 2;
    const bool two = M > KW;
    const uint8_t* wrow[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = n0 + 16 * j + r16;
        wrow[j] = qw + (int64_t)(n < N ? n : 0) * ldw;
    }
    v4f acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    v4i wb[DEPTH][NT][2];
    const v4i zero = v4i{0, 0, 0, 0};
    auto load_w = [&](int s, v4i (&wd)[NT][2]) {
        const int kb = (wave + KW * s) * 128;
        const int o0 = kb + 16 * g < K ? kb + 16 * g : 0;
        const int o1 = kb + 64 + 16 * g < K ? kb + 64 + 16 * g : 0;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            wd[j][0] = load16(wrow[j] + o0);
            wd[j][1] = load16(wrow[j] + o1);
        }
    };

    RowScale sc0 = make_row_scale(0.0f), sc1 = sc0;  // K == 0: the scale is the floor
    if (K4 > 0) {
        float4 v[kFusedRegVec];
#pragma unroll
        for (int e = 0; e < kFusedRegVec; ++e) {
            const int slot = two ? (e >> 3) : 0;
            const int idx = two ? (e & 7) : e;
            const int mr = wave + KW * slot;
            const int m = mr < M ? mr : 0;
            const int j = min(lane + 64 * idx, K4 - 1);
            v[e] = reinterpret_cast<const float4*>(x + (int64_t)m * ldx)[j];
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load_w(d, wb[d]);  // past the last step: never consumed
        issue_order_fence();

        // ---- quantize x into LDS
        float amax0 = 0.0f, amax1 = 0.0f;
#pragma unroll
        for (int e = 0; e < kFusedRegVec; ++e) {
            const bool second = two && e >= 8;
            const int idx = two ? (e & 7) : e;
            const bool ok = wave + (second ? KW : 0) < M && lane + 64 * idx < K4;
            const float a = absmax4(0.0f, v[e]);
            if (second)
                amax1 = fmaxf(amax1, ok ? a : 0.0f);
            else
                amax0 = fmaxf(amax0, ok ? a : 0.0f);
        }
        sc0 = make_row_scale(wave_max(amax0));
        sc1 = make_row_scale(wave_max(amax1));
        const bool keep = blockIdx.x == 0;
#pragma unroll
        for (int e = 0; e < kFusedRegVec; ++e) {
            const bool second = two && e >= 8;
            const int idx = two ? (e & 7) : e;
            const int m = wave + (second ? KW : 0);
            const int j = lane + 64 * idx;
            if (m < M && j < K4) {
                const uint32_t c = cast4(v[e], second ? sc1 : sc0);
                reinterpret_cast<uint32_t*>(xq + m * ldq)[j] = c;
                if (keep && qa_out) reinterpret_cast<uint32_t*>(qa_out + (int64_t)m * K)[j] = c;
            }
        }
    }
    if (lane == 0) {
        const bool keep = blockIdx.x == 0 && s_tok_out != nullptr;
        if (wave < M) {
            s_tok_sh[wave] = sc0.s;
            if (keep) s_tok_out[wave] = sc0.s;
        }
        if (wave + KW < M) {
            s_tok_sh[wave + KW] = sc1.s;
            if (keep) s_tok_out[wave + KW] = sc1.s;
        }
    }
    __syncthreads();

    // ---- weight stream, activation fragments from LDS -----------------------
    // (rows past M read row 0 of the LDS copy: their outputs are never stored;
    // offsets past K read the row start and are zeroed)
    const uint8_t* xs = xq + (r16 < M ? r16 : 0) * ldq;
    if (steps > 0) {
        for (int s0 = 0; s0 < steps; s0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int s = s0 + d;
                const int kb = (wave + KW * s) * 128;
                const bool ok0 = s < steps && kb + 16 * g < K;
                const bool ok1 = s < steps && kb + 64 + 16 * g < K;
                const v4i xa = *reinterpret_cast<const v4i*>(xs + (ok0 ? kb + 16 * g : 0));
                const v4i xc = *reinterpret_cast<const v4i*>(xs + (ok1 ? kb + 64 + 16 * g : 0));
                const v8i b = join(ok0 ? xa : zero, ok1 ? xc : zero);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[j] = mfma_16x16x128_e4m3(join(ok0 ? wb[d][j][0] : zero, ok1 ? wb[d][j][1] : zero), b, acc[j]);
                if (s + DEPTH < steps) load_w(s + DEPTH, wb[d]);
                issue_order_fence();
            }
        }
    }

    // ---- sum the KW partial tiles in wave order, scale, store ---------------
#pragma unroll
    for (int j = 0; j < NT; ++j) red[wave][j][lane] = acc[j];
    __syncthreads();
    for (int j = wave; j < NT; j += KW) {
        v4f sum = red[0][j][lane];
#pragma unroll
        for (int w = 1; w < KW; ++w) sum += red[w][j][lane];
        const int m = r16;
        const int nb = n0 + 16 * j + 4 * g;
        if (m >= M || nb >= N) continue;
        const float st = s_tok_sh[m];
        uint16_t* yr = y + (int64_t)m * ldy;
        if (nb + 3 < N && (ldy & 3) == 0) {
            const float4 sc = *reinterpret_cast<const float4*>(s_ch + nb);
            uint2 o;
            o.x = pack_bf16x2(sum[0] * (st * sc.x), sum[1] * (st * sc.y));
            o.y = pack_bf16x2(sum[2] * (st * sc.z), sum[3] * (st * sc.w));
            *reinterpret_cast<uint2*>(yr + nb) = o;
        } else {
            for (int v = 0; v < 4 && nb + v < N; ++v)
                yr[nb + v] = (uint16_t)bf16_rne_bits(sum[v] * (st * s_ch[nb + v]));
        }
    }
}

// y[m, n] = bf16_rne((part[0][m][n] + part[1][m][n] + ...) * (s_tok[m] * s_ch[n])),
// the splits added in order; one thread per 4 consecutive outputs.
__global__ __launch_bounds__(256) void skinny_splitk_reduce(const float* __restrict__ part, int splits, int M, int N,
                                                           const float* __restrict__ s_tok,
                                                           const float* __restrict__ s_ch, uint16_t* __restrict__ y,
                                                           float* __restrict__ y32, int64_t ldy) {
    const int n4 = (N + 3) >> 2;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)M * n4) return;
    const int m = (int)(t / n4);
    const int nb = (int)(t - (int64_t)m * n4) * 4;
    const int64_t plane = (int64_t)M * N;
    const float* p = part + (int64_t)m * N + nb;
    const bool unit = s_tok == nullptr;  // block-scaled sums: no epilogue scales
    const float st = unit ? 1.0f : s_tok[m];
    if (nb + 3 < N && (N & 3) == 0 && (ldy & 3) == 0) {
        float4 a = *reinterpret_cast<const float4*>(p);
        for (int z = 1; z < splits; ++z) {
            const float4 b = *reinterpret_cast<const float4*>(p + z * plane);
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        const float4 sc = unit ? make_float4(1.0f, 1.0f, 1.0f, 1.0f) : *reinterpret_cast<const float4*>(s_ch + nb);
        if (y32 != nullptr) {
            *reinterpret_cast<float4*>(y32 + (int64_t)m * ldy + nb) =
                make_float4(a.x * (st * sc.x), a.y * (st * sc.y), a.z * (st * sc.z), a.w * (st * sc.w));
            return;
        }
        uint16_t* yr = y + (int64_t)m * ldy;
        uint2 o;
        o.x = pack_bf16x2(a.x * (st * sc.x), a.y * (st * sc.y));
        o.y = pack_bf16x2(a.z * (st * sc.z), a.w * (st * sc.w));
        *reinterpret_cast<uint2*>(yr + nb) = o;
    } else {
        for (int v = 0; v < 4 && nb + v < N; ++v) {
            float a = p[v];
            for (int z = 1; z < splits; ++z) a += p[z * plane + v];
            const float sc = unit ? 1.0f : s_ch[nb + v];
            if (y32 != nullptr)
                y32[(int64_t)m * ldy + nb + v] = a * (st * sc);
            else
                y[(int64_t)m * ldy + nb + v] = (uint16_t)bf16_rne_bits(a * (st * sc));
        }
    }
}

template <int MT, int NT, int KW, bool MX>
static void launch_cfg(dim3 grid, hipStream_t stream, const uint8_t* qa, int64_t lda, const float* s_tok,
                       const uint8_t* qw, int64_t ldw, const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int M,
                       int N, int K, float* part, int split_chunks, MxScales mx) {
    // The block-scaled MFMA keeps its operands in VGPRs (the plain one also
    // reads AGPRs), so the MX kernels keep fewer steps in flight to stay
    // within the register file without spills (checked in the compiler's
    // register report for every instantiation).
    constexpr int DEPTH = MX ? (MT * NT == 1 ? 4 : ((NT == 8 ? MT == 1 : MT * NT <= 6) ? 2 : 1))
                             : ((MT * NT <= 2) ? 4 : 2);
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, NT, KW, DEPTH, MX>), grid, dim3(KW * 64), 0, stream, qa, lda, s_tok,
                       qw, ldw, s_ch, y, y32, ldy, M, N, K, part, split_chunks, mx);
}

template <int MT, bool MX>
static void launch_mt(int nt, dim3 grid, hipStream_t stream, const uint8_t* qa, int64_t lda, const float* s_tok,
                      const uint8_t* qw, int64_t ldw, const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int M,
                      int N, int K, float* part, int split_chunks, MxScales mx) {
    switch (nt) {
        case 8: launch_cfg<MT, 8, 4, MX>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, part, split_chunks, mx); break;
        case 7: launch_cfg<MT, 7, 4, MX>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, part, split_chunks, mx); break;
        case 6: launch_cfg<MT, 6, 4, MX>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, part, split_chunks, mx); break;
        case 5: launch_cfg<MT, 5, 4, MX>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, part, split_chunks, mx); break;
        case 4: launch_cfg<MT, 4, 8, MX>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, part, split_chunks, mx); break;
        case 2: launch_cfg<MT, 2, 8, MX>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, part, split_chunks, mx); break;
        default: launch_cfg<MT, 1, 8, MX>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, part, split_chunks, mx); break;
    }
}

// Weight rows per workgroup (16 * nt) and the number of k splits.  The
// activation fragments are re-read from L2 once per 16 * nt weight rows, so
// larger nt means less L2 traffic; the grid should still hold about one
// workgroup per CU (measured on MI355X: 256 workgroups of 4 waves, one per
// CU, beat partial second rounds).  One activation tile (M <= 16): the largest
// nt <= 4 that leaves >= 224 workgroups, never split (the one-kernel fused
// path must produce the same bits).  More tiles: when nt = 8 (4 waves)
// leaves >= 224 workgroups, the smallest nt in 5..8 that still leaves at most
// 256 (the 70B gate/up shape: nt = 7 gives exactly 256 workgroups and
// measured 50.7 us against 55.7 us for nt = 8's 224); when it leaves at most
// 128, k is split into floor(256 / workgroups) parts (each keeping at least
// two 128-byte chunks per wave); in between, nt = 4 (8 waves).  Split
// workgroups write fp32 partial sums to the workspace, which a second kernel
// adds up in a fixed order.
SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K) {
    SkinnyPlan p{};
    p.mt = (int)((M + 15) / 16);
    p.splits = 1;
    const int64_t chunks = (K + 127) / 128;
    p.split_chunks = (int)chunks;
    auto groups = [&](int nt) { return (N + 16 * nt - 1) / (16 * nt); };
    auto spread = [&](int nt_max) {
        for (int c = nt_max; c >= 1; c >>= 1)
            if (groups(c) >= 224) return c;
        return 1;
    };
    if (p.mt == 1) {
        p.nt = spread(4);
        return p;
    }
    const int64_t g8 = groups(8);
    if (g8 >= 224) {
        p.nt = 8;
        for (int c = 7; c >= 5 && groups(c) <= 256; --c) p.nt = c;
        return p;
    }
    if (g8 > 128) {
        p.nt = 4;
        return p;
    }
    int64_t splits = 256 / g8;
    const int64_t max_splits = chunks / (2 * 4);
    if (splits > max_splits) splits = max_splits;
    if (splits > 16) splits = 16;
    if (splits <= 1) {
        p.nt = spread(8);
        return p;
    }
    p.nt = 8;
    p.split_chunks = (int)((chunks + splits - 1) / splits);
    p.splits = (int)((chunks + p.split_chunks - 1) / p.split_chunks);
    return p;
}

size_t gemm_skinny_ws_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || M > kSkinnyMaxM) return 0;
    const SkinnyPlan p = skinny_plan(M, N, K);
    return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

template <bool MX>
static hipError_t launch_skinny_any(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw,
                                    int64_t ldw, const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int64_t M,
                                    int64_t N, int64_t K, void* ws, MxScales mx, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    SkinnyPlan p = skinny_plan(M, N, K);
    // MX: 4 activation tiles with nt = 4 (8 waves, 256 VGPRs each) would
    // spill; take nt = 8 (4 waves) there (same splits: none on this branch).
    // The shallower MX prefetch also measured slower with nt = 5..7 than
    // with nt = 8 (70B gate/up: 62.8 vs 60.8 us), so MX keeps nt = 8.
    if (MX && p.mt == 4 && p.nt == 4) p.nt = 8;
    if (MX && p.nt >= 5 && p.nt <= 7) p.nt = 8;
    float* part = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    const dim3 grid((unsigned)((N + 16 * p.nt - 1) / (16 * p.nt)), 1, (unsigned)p.splits);
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (p.mt) {
        case 1: launch_mt<1, MX>(p.nt, grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, m, n, k, part, p.split_chunks, mx); break;
        case 2: launch_mt<2, MX>(p.nt, grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, m, n, k, part, p.split_chunks, mx); break;
        case 3: launch_mt<3, MX>(p.nt, grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, m, n, k, part, p.split_chunks, mx); break;
        default: launch_mt<4, MX>(p.nt, grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, m, n, k, part, p.split_chunks, mx); break;
    }
    if (part != nullptr) {
        const int64_t threads = M * ((N + 3) / 4);
        hipLaunchKernelGGL(skinny_splitk_reduce, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, part,
                           p.splits, m, n, MX ? nullptr : s_tok, MX ? nullptr : s_ch, y, y32, ldy);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_skinny(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw,
                              int64_t ldw, const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int64_t M, int64_t N,
                              int64_t K, void* ws, hipStream_t stream) {
    return launch_skinny_any<false>(qa, lda, s_tok, qw, ldw, s_ch, y, y32, ldy, M, N, K, ws, MxScales{}, stream);
}

hipError_t launch_gemm_skinny_mx(const uint8_t* qa, int64_t lda, const uint8_t* sa, const uint8_t* qw, int64_t ldw,
                                 const uint8_t* sw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws,
                                 hipStream_t stream) {
    return launch_skinny_any<true>(qa, lda, nullptr, qw, ldw, nullptr, y, nullptr, ldy, M, N, K, ws,
                                   MxScales{sa, sw}, stream);
}

// The one-kernel path pays for every workgroup reading all of x (fp32) from
// L2.  Measured on MI355X against quantize + GEMM in HIP graphs: it wins by
// 1-1.5 us for N = 4096 and 8192 and loses for N = 14336 (17.6 vs 16.9 us)
// and 28672 (29.5 vs 27.1 us), so wider outputs take the two-kernel path.
constexpr int64_t kFusedMaxN = 8192;

bool gemm_skinny_fused_fits(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > kSkinnyFusedMaxM || M * (K + kFusedRowPad) > kSkinnyFusedLds) return false;
    if (N > kFusedMaxN) return false;
    const int64_t vec_per_row = (K / 4 + 63) / 64;
    return vec_per_row <= (M > kFusedWaves ? kFusedRegVec / 2 : kFusedRegVec);
}

template <int NT, int KW>
static hipError_t launch_fused_cfg(dim3 grid, size_t lds, hipStream_t stream, const float* x, int64_t ldx,
                             const uint8_t* qw, int64_t ldw, const float* s_ch, uint16_t* y, int64_t ldy, int M,
                             int N, int K, uint8_t* qa_out, float* s_tok_out) {
    constexpr int DEPTH = NT <= 2 ? 4 : 2;
    const hipError_t e = FP8K_SET_LDS((gemm_skinny_fused_kernel<NT, KW, DEPTH>), (int)kSkinnyFusedLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_skinny_fused_kernel<NT, KW, DEPTH>), grid, dim3(KW * 64), lds, stream, x, ldx, qw, ldw,
                       s_ch, y, ldy, M, N, K, qa_out, s_tok_out);
    return hipGetLastError();
}

hipError_t launch_gemm_skinny_fused(const float* x, int64_t ldx, const uint8_t* qw, int64_t ldw, const float* s_ch,
                                    uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, uint8_t* qa_out,
                                    float* s_tok_out, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (!gemm_skinny_fused_fits(M, N, K)) return hipErrorInvalidValue;
    // the same weight-rows-per-workgroup rule as the unfused M <= 16 case
    int nt = 1;
    for (int c = 4; c >= 1; c >>= 1)
        if ((N + 16 * c - 1) / (16 * c) >= 224) {
            nt = c;
            break;
        }
    const dim3 grid((unsigned)((N + 16 * nt - 1) / (16 * nt)));
    const size_t lds = (size_t)(M * (K + kFusedRowPad));
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (nt) {
        case 4: return launch_fused_cfg<4, 8>(grid, lds, stream, x, ldx, qw, ldw, s_ch, y, ldy, m, n, k, qa_out, s_tok_out);
        case 2: return launch_fused_cfg<2, 8>(grid, lds, stream, x, ldx, qw, ldw, s_ch, y, ldy, m, n, k, qa_out, s_tok_out);
        default: return launch_fused_cfg<1, 8>(grid, lds, stream, x, ldx, qw, ldw, s_ch, y, ldy, m, n, k, qa_out, s_tok_out);
    }
}

}  // namespace fp8k
