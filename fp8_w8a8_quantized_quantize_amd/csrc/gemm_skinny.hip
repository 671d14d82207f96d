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

// Lane `lane` supplies bytes [16g, 16g+16) and [64+16g, 64+16g+16) of a
// 128-byte k chunk (g = lane / 16) for A and B alike.
template <int MT, int NT, int KW, int DEPTH>
__global__ __launch_bounds__(KW * 64) void gemm_skinny_kernel(
    const uint8_t* __restrict__ qa, int64_t lda, const float* __restrict__ s_tok,
    const uint8_t* __restrict__ qw, int64_t ldw, const float* __restrict__ s_ch,
    uint16_t* __restrict__ y, int64_t ldy, int M, int N, int K) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * (NT * 16);
    const int nchunks = (K + 127) >> 7;
    const int steps = nchunks > wave ? (nchunks - wave + KW - 1) / KW : 0;

    const uint8_t* wrow[NT];
    bool wok[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = n0 + 16 * j + r16;
        wok[j] = n < N;
        wrow[j] = qw + (int64_t)(wok[j] ? n : 0) * ldw;
    }
    const uint8_t* xrow[MT];
    bool xok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = 16 * i + r16;
        xok[i] = m < M;
        xrow[i] = qa + (int64_t)(xok[i] ? m : 0) * lda;
    }

    v4f acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    v4i wb[DEPTH][NT][2];
    v4i xb[DEPTH][MT][2];
    const v4i zero = v4i{0, 0, 0, 0};

    auto load_step = [&](int s, v4i (&wd)[NT][2], v4i (&xd)[MT][2]) {
        const int kb = (wave + KW * s) * 128;
        const bool ok0 = kb + 16 * g < K;
        const bool ok1 = kb + 64 + 16 * g < K;
        // out-of-range chunks read the row's first 16 bytes (K >= 16 whenever
        // a step runs) and are replaced by zeros
        const int o0 = ok0 ? kb + 16 * g : 0;
        const int o1 = ok1 ? kb + 64 + 16 * g : 0;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            v4i a = load16(wrow[j] + o0);
            v4i b = load16(wrow[j] + o1);
            wd[j][0] = (ok0 && wok[j]) ? a : zero;
            wd[j][1] = (ok1 && wok[j]) ? b : zero;
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            v4i a = load16(xrow[i] + o0);
            v4i b = load16(xrow[i] + o1);
            xd[i][0] = (ok0 && xok[i]) ? a : zero;
            xd[i][1] = (ok1 && xok[i]) ? b : zero;
        }
    };

#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (d < steps) load_step(d, wb[d], xb[d]);

    for (int s0 = 0; s0 < steps; s0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int s = s0 + d;
            if (s < steps) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const v8i a = join(wb[d][j][0], wb[d][j][1]);
#pragma unroll
                    for (int i = 0; i < MT; ++i) acc[i][j] = mfma_16x16x128_e4m3(a, join(xb[d][i][0], xb[d][i][1]), acc[i][j]);
                }
                if (s + DEPTH < steps) load_step(s + DEPTH, wb[d], xb[d]);
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
        const float st = s_tok[m];
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

template <int MT, int NT, int KW>
static void launch_cfg(dim3 grid, hipStream_t stream, const uint8_t* qa, int64_t lda, const float* s_tok,
                       const uint8_t* qw, int64_t ldw, const float* s_ch, uint16_t* y, int64_t ldy, int M, int N,
                       int K) {
    constexpr int DEPTH = (MT * NT <= 2) ? 4 : (MT * NT <= 16 ? 2 : 1);
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, NT, KW, DEPTH>), grid, dim3(KW * 64), 0, stream, qa, lda, s_tok, qw,
                       ldw, s_ch, y, ldy, M, N, K);
}

template <int MT>
static void launch_mt(int nt, dim3 grid, hipStream_t stream, const uint8_t* qa, int64_t lda, const float* s_tok,
                      const uint8_t* qw, int64_t ldw, const float* s_ch, uint16_t* y, int64_t ldy, int M, int N,
                      int K) {
    switch (nt) {
        case 8: launch_cfg<MT, 8, 4>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, ldy, M, N, K); break;
        case 4: launch_cfg<MT, 4, 8>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, ldy, M, N, K); break;
        case 2: launch_cfg<MT, 2, 8>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, ldy, M, N, K); break;
        default: launch_cfg<MT, 1, 8>(grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, ldy, M, N, K); break;
    }
}

hipError_t launch_gemm_skinny(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw,
                              int64_t ldw, const float* s_ch, uint16_t* y, int64_t ldy, int64_t M, int64_t N,
                              int64_t K, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int mt = (int)((M + 15) / 16);
    // Weight rows per workgroup (16 * NT): as many as still leave >= 224
    // workgroups (the activation fragments are re-read from L2 once per
    // 16 * NT weight rows, so larger NT means less L2 traffic), up to 8 tiles
    // when M needs 3-4 activation tiles and 4 otherwise.  Waves per
    // workgroup that split K: 8, or 4 with NT = 8 (register budget).
    const int nt_max = mt >= 3 ? 8 : 4;
    int nt = 1;
    for (int c = nt_max; c >= 1; c >>= 1)
        if ((N + 16 * c - 1) / (16 * c) >= 224) {
            nt = c;
            break;
        }
    const dim3 grid((unsigned)((N + 16 * nt - 1) / (16 * nt)));
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (mt) {
        case 1: launch_mt<1>(nt, grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, ldy, m, n, k); break;
        case 2: launch_mt<2>(nt, grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, ldy, m, n, k); break;
        case 3: launch_mt<3>(nt, grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, ldy, m, n, k); break;
        default: launch_mt<4>(nt, grid, stream, qa, lda, s_tok, qw, ldw, s_ch, y, ldy, m, n, k); break;
    }
    return hipGetLastError();
}

}  // namespace fp8k
