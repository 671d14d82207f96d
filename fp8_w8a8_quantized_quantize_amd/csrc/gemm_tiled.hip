// LDS-tiled, double-buffered FP8 MFMA GEMM on gfx950 (prefill-shaped M and
// the grouped MoE expert GEMM), FP32 accumulation and a fused s_tok*s_ch
// dequantizing BF16 epilogue (DeepSeek V4 950 page, §2.3 and §2.4).
//
// Tile: BN weight rows x BM activation rows, k step 128 bytes.  Four waves in
// a WN x WM grid, each owning an (FN*16) x (FM*16) sub-tile of 16x16x128 MFMA
// tiles (MFMA A = weight rows, B = activation rows).  Per k step the
// workgroup copies a BN x 128 and a BM x 128 byte tile HBM/L2 -> registers ->
// LDS (one buffer being filled while the other feeds the MFMAs); 16-byte
// chunks are XOR-swizzled by row (chunk c of row r sits at c ^ (r & 7)) so the
// fragment reads (16 rows x one chunk per 16 lanes) hit distinct banks.
//
// Dense launches remap workgroup ids so that consecutive tiles land on the
// same XCD (the hardware deals workgroups round-robin over the 8 XCDs, each
// with its own L2) and walk the output in groups of GROUP_M tile rows, so the
// k slices of a few activation tiles and many weight tiles are shared in L2.
//
// Grouped launches: routed rows are sorted by expert; every workgroup derives
// its (expert, row tile, column tile) from the expert offsets on the device,
// gathers its activation rows through row_token, and uses the expert's weight
// matrix and channel scales.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

constexpr int kBK = 128;
constexpr int kThreads = 256;

struct TiledArgs {
    const uint8_t* qa;
    int64_t lda;
    const float* s_tok;
    const uint8_t* qw;
    int64_t ldw;
    const float* s_ch;
    uint16_t* y;
    float* y32;  // when set (dense only): fp32 output instead of y, row stride ldy
    int64_t ldy;
    int M, N, K;
    int tiles_m, tiles_n;
    // grouped only
    const int32_t* row_token;
    const int32_t* offsets;
    int E;
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// Inclusive prefix over experts of (row tiles x column tiles); finds the
// expert owning `tile`.  Runs on wave 0; results go to LDS.
template <int BM>
__device__ void find_expert(const TiledArgs& p, int tile, int* sh) {
    // sh[0] = expert or -1, sh[1] = first tile of that expert
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int carry = 0;
        int found_e = -1, found_base = 0;
        for (int e0 = 0; e0 < p.E; e0 += 64) {
            const int e = e0 + lane;
            int cnt = 0;
            if (e < p.E) {
                const int rows = p.offsets[e + 1] - p.offsets[e];
                cnt = ((rows + BM - 1) / BM) * p.tiles_n;
            }
            int incl = cnt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(incl, off, 64);
                if (lane >= off) incl += v;
            }
            const int excl = carry + incl - cnt;
            const bool hit = (e < p.E) && cnt > 0 && tile >= excl && tile < excl + cnt;
            const unsigned long long mask = __ballot(hit);
            if (mask) {
                const int src = __ffsll((long long)mask) - 1;
                found_e = __shfl(e, src, 64);
                found_base = __shfl(excl, src, 64);
                break;
            }
            carry += __shfl(incl, 63, 64);
        }
        if (lane == 0) {
            sh[0] = found_e;
            sh[1] = found_base;
        }
    }
    __syncthreads();
}

template <int BN, int BM, int WN, int WM, int GROUP_M, bool GROUPED>
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled_kernel(TiledArgs p) {
    static_assert(WN * WM == 4, "four waves");
    constexpr int FN = BN / WN / 16;
    constexpr int FM = BM / WM / 16;
    constexpr int WCH = BN * 8 / kThreads;  // 16-byte weight chunks per thread per k step
    constexpr int XCH = BM * 8 / kThreads;  // activation chunks per thread per k step
    constexpr int STAGE = (BN + BM) * kBK;  // bytes per LDS stage
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
    __shared__ int sh[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % WN, wm = wave / WN;
    const int r16 = lane & 15, g = lane >> 4;

    // ---- which output tile ------------------------------------------------
    int tile_m, tile_n, expert = 0, row_begin = 0, rows_valid;
    if constexpr (!GROUPED) {
        const int total = p.tiles_m * p.tiles_n;
        int t = blockIdx.x;
        if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);  // XCD-contiguous
        const int per_group = GROUP_M * p.tiles_n;
        const int grp = t / per_group;
        const int first_m = grp * GROUP_M;
        const int gsz = min(p.tiles_m - first_m, GROUP_M);
        const int in = t - grp * per_group;
        tile_m = first_m + in % gsz;
        tile_n = in / gsz;
        rows_valid = p.M - tile_m * BM;
    } else {
        find_expert<BM>(p, blockIdx.x, sh);
        expert = sh[0];
        if (expert < 0) return;  // beyond the last tile (uniform over the block)
        const int local = blockIdx.x - sh[1];
        row_begin = p.offsets[expert];
        const int rows_e = p.offsets[expert + 1] - row_begin;
        const int mt_e = (rows_e + BM - 1) / BM;
        tile_m = local % mt_e;
        tile_n = local / mt_e;
        rows_valid = rows_e - tile_m * BM;
    }
    const int n0 = tile_n * BN;
    const int m0 = tile_m * BM;
    const uint8_t* qw = p.qw;
    const float* s_ch = p.s_ch;
    if constexpr (GROUPED) {
        qw += (int64_t)expert * p.N * p.K;
        s_ch += (int64_t)expert * p.N;
    }

    // ---- per-thread global sources for the LDS fill -----------------------
    // chunk id = tid + 256 * i -> row id / 8, 16-byte column id % 8
    const int ccol = tid & 7;
    const int crow = tid >> 3;  // + 32 * i
    const uint8_t* wsrc[WCH];
    bool wvalid[WCH];
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
        const int n = n0 + crow + 32 * i;
        wvalid[i] = n < p.N;
        wsrc[i] = qw + (int64_t)(wvalid[i] ? n : 0) * (GROUPED ? p.K : p.ldw);
    }
    const uint8_t* xsrc[XCH];
    bool xvalid[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int ml = crow + 32 * i;
        xvalid[i] = ml < rows_valid;
        int64_t row;
        if constexpr (GROUPED)
            row = xvalid[i] ? p.row_token[row_begin + m0 + ml] : 0;
        else
            row = xvalid[i] ? m0 + ml : 0;
        xsrc[i] = p.qa + row * (GROUPED ? p.K : p.lda);
    }

    v4i wreg[WCH], xreg[XCH];
    const v4i zero = v4i{0, 0, 0, 0};
    auto gload = [&](int k0) {
        // chunks beyond K read the row's first 16 bytes and are zeroed
        const bool kok = k0 + ccol * 16 < p.K;
        const int ko = kok ? k0 + ccol * 16 : 0;
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            v4i v = load16(wsrc[i] + ko);
            wreg[i] = (kok && wvalid[i]) ? v : zero;
        }
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            v4i v = load16(xsrc[i] + ko);
            xreg[i] = (kok && xvalid[i]) ? v : zero;
        }
    };
    auto lstore = [&](uint8_t* st) {
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const int r = crow + 32 * i;
            *reinterpret_cast<v4i*>(st + r * kBK + swz(r, ccol) * 16) = wreg[i];
        }
        uint8_t* xs = st + BN * kBK;
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int r = crow + 32 * i;
            *reinterpret_cast<v4i*>(xs + r * kBK + swz(r, ccol) * 16) = xreg[i];
        }
    };

    v4f acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    const int ktiles = (p.K + kBK - 1) / kBK;
    if (ktiles > 0) {
        gload(0);
        lstore(lds);
    }
    __syncthreads();

    const int wrow0 = wn * (BN / WN);
    const int xrow0 = wm * (BM / WM);
    for (int kt = 0; kt < ktiles; ++kt) {
        uint8_t* cur = lds + (kt & 1) * STAGE;
        if (kt + 1 < ktiles) gload((kt + 1) * kBK);
        const uint8_t* ws = cur;
        const uint8_t* xs = cur + BN * kBK;
        v8i bf[FM];
#pragma unroll
        for (int b = 0; b < FM; ++b) {
            const int r = xrow0 + b * 16 + r16;
            const v4i lo = *reinterpret_cast<const v4i*>(xs + r * kBK + swz(r, g) * 16);
            const v4i hi = *reinterpret_cast<const v4i*>(xs + r * kBK + swz(r, 4 + g) * 16);
            bf[b] = join(lo, hi);
        }
#pragma unroll
        for (int a = 0; a < FN; ++a) {
            const int r = wrow0 + a * 16 + r16;
            const v4i lo = *reinterpret_cast<const v4i*>(ws + r * kBK + swz(r, g) * 16);
            const v4i hi = *reinterpret_cast<const v4i*>(ws + r * kBK + swz(r, 4 + g) * 16);
            const v8i af = join(lo, hi);
#pragma unroll
            for (int b = 0; b < FM; ++b) acc[a][b] = mfma_16x16x128_e4m3(af, bf[b], acc[a][b]);
        }
        if (kt + 1 < ktiles) lstore(lds + ((kt + 1) & 1) * STAGE);
        __syncthreads();
    }

    // ---- epilogue: y = bf16_rne(acc * (s_tok * s_ch)) ----------------------
    // 8-byte stores and 16-byte scale loads need 4-element aligned rows
    const bool vec_store = GROUPED ? (p.N & 3) == 0 : (p.ldy & 3) == 0;
#pragma unroll
    for (int b = 0; b < FM; ++b) {
        const int ml = xrow0 + b * 16 + r16;
        if (ml >= rows_valid) continue;
        int64_t yrow;
        float st;
        if constexpr (GROUPED) {
            yrow = row_begin + m0 + ml;
            st = p.s_tok[p.row_token[yrow]];
        } else {
            yrow = m0 + ml;
            st = p.s_tok[yrow];
        }
        uint16_t* yr = p.y + yrow * (GROUPED ? (int64_t)p.N : p.ldy);
#pragma unroll
        for (int a = 0; a < FN; ++a) {
            const int nb = n0 + wrow0 + a * 16 + 4 * g;
            if (nb >= p.N) continue;
            const v4f s = acc[a][b];
            if (!GROUPED && p.y32 != nullptr) {
                float* yr32 = p.y32 + yrow * p.ldy;
                for (int v = 0; v < 4 && nb + v < p.N; ++v) yr32[nb + v] = s[v] * (st * s_ch[nb + v]);
                continue;
            }
            if (nb + 3 < p.N && vec_store) {
                const float4 sc = *reinterpret_cast<const float4*>(s_ch + nb);
                uint2 o;
                o.x = pack_bf16x2(s[0] * (st * sc.x), s[1] * (st * sc.y));
                o.y = pack_bf16x2(s[2] * (st * sc.z), s[3] * (st * sc.w));
                *reinterpret_cast<uint2*>(yr + nb) = o;
            } else {
                for (int v = 0; v < 4 && nb + v < p.N; ++v)
                    yr[nb + v] = (uint16_t)bf16_rne_bits(s[v] * (st * s_ch[nb + v]));
            }
        }
    }
}

hipError_t launch_gemm_tiled(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw,
                             int64_t ldw, const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int64_t M, int64_t N,
                             int64_t K, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    constexpr int BN = 256, BM = 256;
    TiledArgs p{};
    p.qa = qa; p.lda = lda; p.s_tok = s_tok; p.qw = qw; p.ldw = ldw; p.s_ch = s_ch; p.y = y; p.y32 = y32; p.ldy = ldy;
    p.M = (int)M; p.N = (int)N; p.K = (int)K;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
    hipLaunchKernelGGL((gemm_tiled_kernel<BN, BM, 2, 2, 4, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm_grouped(const uint8_t* qa, const float* s_tok, const int32_t* row_token,
                               const int32_t* offsets, const uint8_t* qw, const float* s_ch, uint16_t* y,
                               int64_t T, int64_t R, int64_t E, int64_t N, int64_t K, hipStream_t stream) {
    (void)T;
    if (R <= 0 || N <= 0 || E <= 0) return hipSuccess;
    constexpr int BN = 256, BM = 128;
    TiledArgs p{};
    p.qa = qa; p.lda = K; p.s_tok = s_tok; p.qw = qw; p.ldw = K; p.s_ch = s_ch; p.y = y; p.ldy = N;
    p.M = (int)R; p.N = (int)N; p.K = (int)K;
    p.tiles_n = (int)((N + BN - 1) / BN);
    p.tiles_m = 0;
    p.row_token = row_token; p.offsets = offsets; p.E = (int)E;
    // upper bound of sum_e ceil(rows_e / BM) is ceil(R / BM) + E
    const int64_t grid = ((R + BM - 1) / BM + E) * p.tiles_n;
    hipLaunchKernelGGL((gemm_tiled_kernel<BN, BM, 2, 2, 1, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fp8k
