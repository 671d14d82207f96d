// Multi-stage FP8 MFMA GEMM for gfx950 fed by direct global->LDS loads
// (prefill-shaped M and the grouped MoE expert GEMM), FP32 accumulation and
// the s_tok*s_ch dequantizing BF16 epilogue (DeepSeek V4 950 page, §2.3 and
// §2.4; FP8 x FP8 with FP32 accumulation, precision/hardware page §2.3).
//
// Tile: BN weight rows (MFMA A operand) x BM activation rows (MFMA B operand),
// 64 bytes of K per stage, STAGES stages in LDS.  Four waves in a 2 x 2 grid,
// each owning (BN/2) x (BM/2) outputs as 32x32x64 FP8 MFMA tiles with 16
// accumulators per lane.
//
// Data movement: global_load_lds_dwordx4 writes each wave's 1 KB of a stage
// straight into LDS (no VGPR staging, no ds_write).  One DMA instruction
// covers 16 rows x 64 bytes; lane l fetches row l/4, 16-byte piece
// (l % 4) ^ swz(row), so the LDS image holds piece c of row r at position
// c ^ swz(r).  swz(r) = ((r >> 1) ^ (r >> 2)) & 3 keeps the fragment reads
// (32 rows x one 16-byte piece per wave read) free of bank conflicts for both
// 8-lane/128-byte and 16-lane/256-byte LDS service groups.
//
// Pipeline per K step k (one barrier), STAGES-1 stages in flight:
//   wait (vmcnt) for this wave's DMA of stage k; barrier (every wave's part of
//   stage k has landed and every wave has finished reading stage k-1);
//   issue the DMA of stage k+STAGES-1 into stage k-1's buffer;
//   read the fragments of stage k and run its MFMAs.
// The compiler does not track DMA-written LDS, so the waits are explicit
// (s_waitcnt vmcnt with the number of younger DMA instructions) and compiler
// memory fences keep LDS reads on their side of each wait and barrier.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

typedef float v16f __attribute__((ext_vector_type(16)));

namespace {

constexpr int kDK = 64;       // K bytes per stage
constexpr int kThreadsM = 256;

__device__ __forceinline__ v16f mfma_32x32x64_e4m3(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ int dswz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt vmcnt(n) for n = 8 * outstanding stages (n <= 63).
template <int PER_STAGE>
__device__ __forceinline__ void wait_dma(int outstanding_stages) {
    compiler_fence();
    switch (outstanding_stages) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER_STAGE) : "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER_STAGE) : "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER_STAGE) : "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * PER_STAGE) : "memory"); break;
    }
    compiler_fence();
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes
// land at lds + 16 * i (lds is wave-uniform).
__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have completed.
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void block_barrier() {
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// One 32-row MFMA operand fragment from a stage tile of 64-byte rows:
// lane l supplies row row0 + l % 32, pieces g and 2 + g (g = l / 32).
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int g) {
    const int s = dswz(row);
    const v4i lo = *reinterpret_cast<const v4i*>(tile + row * kDK + ((g ^ s) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(tile + row * kDK + (((2 + g) ^ s) << 4));
    return join(lo, hi);
}

}  // namespace

// Dynamic LDS of the kernels below (the stage ring).
extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

struct MfmaArgs {
    const uint8_t* qa;
    int64_t lda;
    const float* s_tok;
    const uint8_t* qw;
    int64_t ldw;
    const float* s_ch;
    uint16_t* y;
    int64_t ldy;
    int M, N, K;
    int tiles_m, tiles_n;
    const int32_t* row_token;  // grouped only
    const int32_t* offsets;
    int E;
};

// Expert owning grouped tile `tile` (prefix over experts of row tiles x
// column tiles, computed by wave 0).  sh[0] = expert or -1, sh[1] = its first tile.
template <int BM>
__device__ void find_expert_tile(const MfmaArgs& p, int tile, int* sh) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int carry = 0, found_e = -1, found_base = 0;
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

template <int BN, int BM, int STAGES, int GROUP_M, bool GROUPED>
__global__ __launch_bounds__(kThreadsM, 1) void gemm_mfma_kernel(MfmaArgs p) {
    constexpr int FN = BN / 64;                 // 32-row weight fragments per wave
    constexpr int FM = BM / 64;                 // 32-row activation fragments per wave
    constexpr int DA = BN / 64;                 // DMA instructions per wave per stage, weights
    constexpr int DB = BM / 64;                 // ... activations
    constexpr int PER_STAGE = DA + DB;
    constexpr int STAGE = (BN + BM) * kDK;
    static_assert(STAGES >= 2 && STAGES <= 5, "stages");
    __shared__ int sh[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1, wm = wave >> 1;
    const int r32 = lane & 31, g = lane >> 5;

    // ---- output tile ------------------------------------------------------
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
        find_expert_tile<BM>(p, blockIdx.x, sh);
        expert = sh[0];
        if (expert < 0) return;  // past the last tile (uniform over the block)
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
    int64_t ldw = p.ldw, lda = p.lda;
    if constexpr (GROUPED) {
        qw += (int64_t)expert * p.N * p.K;
        s_ch += (int64_t)expert * p.N;
    }

    // ---- per-lane DMA sources ----------------------------------------------
    // instruction j of this wave covers tile rows (wave * D + j) * 16 .. +15
    const uint8_t* asrc[DA];
    const uint8_t* bsrc[DB];
#pragma unroll
    for (int j = 0; j < DA; ++j) {
        const int row = (wave * DA + j) * 16 + (lane >> 2);
        const int n = min(n0 + row, p.N - 1);  // rows past N feed discarded columns
        asrc[j] = qw + (int64_t)n * ldw + (((lane & 3) ^ dswz(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < DB; ++j) {
        const int row = (wave * DB + j) * 16 + (lane >> 2);
        const int ml = min(row, rows_valid - 1);  // rows past the tile feed discarded rows
        int64_t src_row;
        if constexpr (GROUPED)
            src_row = p.row_token[row_begin + m0 + ml];
        else
            src_row = m0 + ml;
        bsrc[j] = p.qa + src_row * lda + (((lane & 3) ^ dswz(row)) << 4);
    }

    auto issue_stage = [&](int kt) {
        uint8_t* base = smem + (kt % STAGES) * STAGE;
        const int koff = kt * kDK;
#pragma unroll
        for (int j = 0; j < DA; ++j)
            dma16(asrc[j] + koff, base + (wave * DA + j) * 1024);
#pragma unroll
        for (int j = 0; j < DB; ++j)
            dma16(bsrc[j] + koff, base + BN * kDK + (wave * DB + j) * 1024);
    };

    v16f acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

    const int KT = p.K / kDK;
    const int arow0 = wn * (BN / 2) + r32;
    const int brow0 = wm * (BM / 2) + r32;
    v8i fa[FN], fb[FM];

    auto read_stage = [&](int kt, v8i (&ra)[FN], v8i (&rb)[FM]) {
        const uint8_t* base = smem + (kt % STAGES) * STAGE;
#pragma unroll
        for (int b = 0; b < FM; ++b) rb[b] = read_frag(base + BN * kDK, brow0 + b * 32, g);
#pragma unroll
        for (int a = 0; a < FN; ++a) ra[a] = read_frag(base, arow0 + a * 32, g);
    };
    auto mma_stage = [&](const v8i (&ra)[FN], const v8i (&rb)[FM]) {
#pragma unroll
        for (int a = 0; a < FN; ++a)
#pragma unroll
            for (int b = 0; b < FM; ++b) acc[a][b] = mfma_32x32x64_e4m3(ra[a], rb[b], acc[a][b]);
    };

    // prologue: stages 0 .. STAGES-2 in flight
    if (KT > 0) {
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < KT) issue_stage(s);
    }
    for (int k = 0; k < KT; ++k) {
        // this wave's DMA of stage k has landed; the barrier makes every
        // wave's part visible and guarantees stage k-1 is no longer read
        wait_dma<PER_STAGE>(min(KT - 1, k + STAGES - 2) - k);
        block_barrier();
        if (k + STAGES - 1 < KT) issue_stage(k + STAGES - 1);  // into stage k-1's buffer
        read_stage(k, fa, fb);
        mma_stage(fa, fb);
        wait_lds_reads();  // reads of stage k done before the next barrier
    }

    // ---- epilogue: y = bf16_rne(acc * (s_tok * s_ch)) ----------------------
    // lane l of a 32x32 tile: column (activation row) l % 32, weight rows
    // 8 * (v / 4) + 4 * (l / 32) + v % 4 for accumulator v.
    const bool vec_store = GROUPED ? (p.N & 3) == 0 : (p.ldy & 3) == 0;
#pragma unroll
    for (int b = 0; b < FM; ++b) {
        const int ml = wm * (BM / 2) + b * 32 + r32;
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
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nb = n0 + wn * (BN / 2) + a * 32 + 8 * q + 4 * g;
                if (nb >= p.N) continue;
                const float c0 = acc[a][b][4 * q + 0], c1 = acc[a][b][4 * q + 1];
                const float c2 = acc[a][b][4 * q + 2], c3 = acc[a][b][4 * q + 3];
                if (nb + 3 < p.N && vec_store) {
                    const float4 sc = *reinterpret_cast<const float4*>(s_ch + nb);
                    uint2 o;
                    o.x = pack_bf16x2(c0 * (st * sc.x), c1 * (st * sc.y));
                    o.y = pack_bf16x2(c2 * (st * sc.z), c3 * (st * sc.w));
                    *reinterpret_cast<uint2*>(yr + nb) = o;
                } else {
                    const float cv[4] = {c0, c1, c2, c3};
                    for (int v = 0; v < 4 && nb + v < p.N; ++v)
                        yr[nb + v] = (uint16_t)bf16_rne_bits(cv[v] * (st * s_ch[nb + v]));
                }
            }
        }
    }
}

// The kernels use more than 64 KB of dynamic LDS, which needs an opt-in.
#define FP8K_SET_LDS(KERNEL, BYTES) \
    hipFuncSetAttribute(reinterpret_cast<const void*>(&KERNEL), hipFuncAttributeMaxDynamicSharedMemorySize, (BYTES))

hipError_t launch_gemm_mfma(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw, int64_t ldw,
                            const float* s_ch, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                            hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    constexpr int BN = 256, BM = 256, ST = 4;
    constexpr int LDS = ST * (BN + BM) * kDK;
    MfmaArgs p{};
    p.qa = qa; p.lda = lda; p.s_tok = s_tok; p.qw = qw; p.ldw = ldw; p.s_ch = s_ch; p.y = y; p.ldy = ldy;
    p.M = (int)M; p.N = (int)N; p.K = (int)K;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    hipError_t e = FP8K_SET_LDS((gemm_mfma_kernel<BN, BM, ST, 4, false>), LDS);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
    hipLaunchKernelGGL((gemm_mfma_kernel<BN, BM, ST, 4, false>), dim3(grid), dim3(kThreadsM), LDS, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm_grouped_mfma(const uint8_t* qa, const float* s_tok, const int32_t* row_token,
                                    const int32_t* offsets, const uint8_t* qw, const float* s_ch, uint16_t* y,
                                    int64_t T, int64_t R, int64_t E, int64_t N, int64_t K, hipStream_t stream) {
    (void)T;
    if (R <= 0 || N <= 0 || E <= 0) return hipSuccess;
    constexpr int BN = 256, BM = 128, ST = 4;
    constexpr int LDS = ST * (BN + BM) * kDK;
    MfmaArgs p{};
    p.qa = qa; p.lda = K; p.s_tok = s_tok; p.qw = qw; p.ldw = K; p.s_ch = s_ch; p.y = y; p.ldy = N;
    p.M = (int)R; p.N = (int)N; p.K = (int)K;
    p.tiles_n = (int)((N + BN - 1) / BN);
    p.row_token = row_token; p.offsets = offsets; p.E = (int)E;
    hipError_t e = FP8K_SET_LDS((gemm_mfma_kernel<BN, BM, ST, 1, true>), LDS);
    if (e != hipSuccess) return e;
    const int64_t grid = ((R + BM - 1) / BM + E) * p.tiles_n;
    hipLaunchKernelGGL((gemm_mfma_kernel<BN, BM, ST, 1, true>), dim3((unsigned)grid), dim3(kThreadsM), LDS, stream, p);
    return hipGetLastError();
}

}  // namespace fp8k
