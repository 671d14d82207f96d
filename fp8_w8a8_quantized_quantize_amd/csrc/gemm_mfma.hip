// Two-stage FP8 MFMA GEMM for gfx950 fed by direct global->LDS loads
// (prefill-shaped M and the grouped MoE expert GEMM), FP32 accumulation and
// the s_tok*s_ch dequantizing BF16 epilogue (DeepSeek V4 950 page, §2.3 and
// §2.4; FP8 x FP8 with FP32 accumulation, precision/hardware page §2.3).
//
// Tile: BN weight rows (MFMA A operand) x BM activation rows (MFMA B operand),
// 128 bytes of K per stage, two stages in LDS.  WN x WM waves, each owning
// BN/WN weight rows times every WM-th 32-row block of activation rows
// ((BN/WN) x (BM/WM) outputs) as 32x32x64 FP8 MFMA tiles (16 accumulators per
// lane per tile); a stage is consumed as two 64-wide K halves.  The launchers
// use 2 x 2 waves of 128 x 128: measured on MI355X, 2 x 4 waves (two per SIMD,
// which doubles the LDS read rate a CU reaches) lose more to the 50% larger
// LDS read volume of 128 x 64 wave tiles and to register spills.
//
// Data movement: global_load_lds_dwordx4 writes a stage straight into LDS
// (no VGPR staging, no ds_write).  One DMA instruction covers 8 rows x 128
// bytes -- whole cache lines, which the L2->CU path delivers markedly faster
// than half lines; lane l fetches row l / 8, 16-byte piece (l % 8) ^ swz(row),
// so the LDS image holds piece c of row r at position c ^ swz(r).
// swz(r) = (r ^ (r >> 3)) & 7 keeps the fragment reads (32 rows x one piece
// per read) free of bank conflicts for 8-lane/128-byte and 16-lane/256-byte
// LDS service groups alike.
//
// Pipeline, step s (stage s in LDS, its first-half fragments in registers):
//   first-half MFMAs of stage s, refilling each fragment register with the
//   second half as soon as its last first-half MFMA has issued;
//   wait (vmcnt) for this wave's DMA of stage s+1 and (lgkmcnt) for its reads
//   of stage s; barrier: stage s+1 is complete in LDS and nobody reads stage
//   s any more -> the DMA of stage s+2 may go into stage s's buffer;
//   second-half MFMAs of stage s, each followed by one DMA instruction of
//   stage s+2, refilling the registers with the first half of stage s+1.
// Scheduling hints alternate MFMAs and LDS reads within each half (measured
// on MI355X: about 8% faster than letting them bunch).
// One barrier per 32 MFMAs, LDS reads overlapped with MFMAs, a whole step of
// MFMA time to hide each stage's load.  The compiler does not track
// DMA-written LDS, so the waits are explicit and compiler memory fences keep
// LDS reads on their side of each wait and barrier.
//
// The output tile leaves through LDS (scaled, BF16, swizzled) so that the
// global stores are 16-byte row-contiguous; the tile's scales are staged in
// LDS at the start.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8k {

typedef float v16f __attribute__((ext_vector_type(16)));

namespace {

constexpr int kBK = 128;      // K bytes per stage

__device__ __forceinline__ v16f mfma_32x32x64_e4m3(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same MFMA with block scales: the exponent byte that lane (r, g)
// passes scales k [32g, 32g + 32) of the 64-k half for row r of its operand
// (the fragment layout of read_frag below; measured on gfx950).
__device__ __forceinline__ v16f mfma_32x32x64_e4m3_mx(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ int dswz(int row) { return (row ^ (row >> 3)) & 7; }

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

// One 32-row MFMA operand fragment from a stage tile of 128-byte rows, K half
// h: lane l supplies row row0 + l % 32, pieces 4h + g and 4h + 2 + g
// (g = l / 32).  A and B fragments use the same piece order, so every k pairs
// with itself in the dot product.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int h, int g) {
    const int s = dswz(row);
    const v4i lo = *reinterpret_cast<const v4i*>(tile + row * kBK + (((4 * h + g) ^ s) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(tile + row * kBK + (((4 * h + 2 + g) ^ s) << 4));
    return join(lo, hi);
}

// Scheduling hint for a half step (MF MFMAs and the RD LDS reads that refill
// the fragments): spread the reads evenly between the MFMAs instead of letting
// them bunch after them.
template <int MF, int RD>
__device__ __forceinline__ void interleave_mfma_reads() {
    constexpr int base = RD / MF, extra = RD % MF;
#pragma unroll
    for (int i = 0; i < extra; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, base + 1, 0);  // LDS reads
    }
#pragma unroll
    for (int i = extra; i < MF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (base > 0) __builtin_amdgcn_sched_group_barrier(0x100, base, 0);
    }
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
    float* y32;  // when set: fp32 output (unrounded acc * s_tok * s_ch) instead of y, row stride ldy
    int64_t ldy;
    int M, N, K;
    int tiles_m, tiles_n;
    const int32_t* row_token;  // grouped only
    const int32_t* offsets;
    int E;
    MxScales mx;  // block-scaled operands (MX kernels only)
};

// Number of output tiles of expert e (row tiles x column tiles).
template <int BM>
__device__ __forceinline__ int expert_tiles(const MfmaArgs& p, int e) {
    const int rows = p.offsets[e + 1] - p.offsets[e];
    return ((rows + BM - 1) / BM) * p.tiles_n;
}

// Grouped tile of workgroup b, computed by wave 0: sh[0] = expert (or -1 when
// b has no tile), sh[1] = the tile's index inside that expert.
//
// The real tiles, numbered expert by expert, are cut into 8 contiguous ranges,
// one per XCD (workgroups are dealt to the XCDs round-robin, b % 8), so the
// tiles that share an expert's weights run side by side on one XCD and read
// those weights through one L2.
template <int BM>
__device__ void find_expert_tile(const MfmaArgs& p, int b, int* sh) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int total = 0;
        for (int e0 = 0; e0 < p.E; e0 += 64) {
            int cnt = (e0 + lane < p.E) ? expert_tiles<BM>(p, e0 + lane) : 0;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
            total += cnt;
        }
        const int x = b & 7, j = b >> 3;
        const int tile = (int)(((int64_t)x * total) >> 3) + j;
        const int end = (int)(((int64_t)(x + 1) * total) >> 3);
        int carry = 0, found_e = -1, found_local = 0;
        for (int e0 = 0; e0 < p.E && tile < end; e0 += 64) {
            const int e = e0 + lane;
            const int cnt = (e < p.E) ? expert_tiles<BM>(p, e) : 0;
            int incl = cnt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(incl, off, 64);
                if (lane >= off) incl += v;
            }
            const int excl = carry + incl - cnt;
            const bool hit = cnt > 0 && tile >= excl && tile < excl + cnt;
            const unsigned long long mask = __ballot(hit);
            if (mask) {
                const int src = __ffsll((long long)mask) - 1;
                found_e = __shfl(e, src, 64);
                found_local = tile - __shfl(excl, src, 64);
                break;
            }
            carry += __shfl(incl, 63, 64);
        }
        if (lane == 0) {
            sh[0] = found_e;
            sh[1] = found_local;
        }
    }
    __syncthreads();
}

// MX = true: block-scaled operands (dense only).  A stage also carries the
// tile rows' 4 block-scale bytes (one 32-bit word per row, fetched by two more
// DMA instructions per wave into a ring of their own); a lane reads its
// fragment rows' words for stage s + 1 after the barrier of step s and passes
// byte 2h + g for K half h; the tile scales of the epilogue are 1.  The
// scales are chunk-major (word [kt][row]), so a stage's words for
// consecutive rows are contiguous: a row-major [row][kt] order made every
// lane of a scale DMA touch its own cache line (measured: 23 % slower on
// 8192^3).
// SKIP (dense): compile the K loop for 1-4 live activation fragments, as the
// grouped kernel always does; the launcher takes it only when the whole grid
// is one row of tiles with at most 192 real rows (M in 65..192), because the
// extra instantiations cost the full-tile loop about 1 % (measured on 8192^3).
template <int BN, int BM, int WN, int WM, int GROUP_M, bool GROUPED, bool MX = false, bool SKIP = false>
__global__ __launch_bounds__(64 * WN * WM, 1) void gemm_mfma_kernel(MfmaArgs p) {
    static_assert(!(MX && GROUPED), "block scales: dense GEMM only");
    constexpr int NW = WN * WM;                 // waves: WN along the weight rows, WM along the activations
    constexpr int NTH = 64 * NW;
    constexpr int FN = BN / (32 * WN);          // 32-row weight fragments per wave
    constexpr int FM = BM / (32 * WM);          // 32-row activation fragments per wave
    constexpr int DA = BN / (8 * NW);           // DMA instructions per wave per stage, weights
    constexpr int DB = BM / (8 * NW);           // ... activations
    constexpr int DS = MX ? (BN + BM) / (64 * NW) : 0;  // ... block-scale words (64 rows each)
    constexpr int PER_STAGE = DA + DB + DS;
    constexpr int STAGE = (BN + BM) * kBK;
    constexpr int SRING = 2 * STAGE + 4 * (BN + BM);    // block-scale ring: 2 x (BN + BM) words
    static_assert(DA * 8 * NW == BN && DB * 8 * NW == BM, "whole DMA instructions per wave");
    static_assert(!MX || DS * 64 * NW == BN + BM, "whole scale DMA instructions per wave");
    static_assert(BM * BN * 2 <= 2 * STAGE, "the BF16 output tile must fit in the ring");
    int* sh = reinterpret_cast<int*>(smem + 2 * STAGE + 4 * (BN + BM));  // grouped tile lookup
    // Grouped: the weight tile's lines of stage s + 3 are touched into L2
    // during step s (one 4-byte DMA per row into a dummy LDS slot), so the
    // stage's own DMA one step later finds them there: expert weights stream
    // from HBM, whose latency one step of MFMAs does not always cover.
    constexpr bool PF = GROUPED;
    static_assert(!PF || BN == 64 * NW, "one prefetch row per lane");
    uint8_t* pf_lds = smem + 2 * STAGE + 4 * (BN + BM) + 16;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wm = wave / WN;
    const int r32 = lane & 31, g = lane >> 5;

    // ---- output tile ------------------------------------------------------
    int tile_m, tile_n, expert = 0, row_begin = 0, rows_valid;
    if constexpr (!GROUPED) {
        // Workgroups are dealt round-robin to the 8 XCDs (blockIdx % 8).  When
        // the tile grid splits evenly, XCD x owns a 2 x 4 block of the grid
        // (half the activation tiles, a quarter of the weight tiles), so each
        // XCD's L2 sees only its share of both operands; inside it, tiles go
        // in groups of GROUP_M activation rows.
        int sub_m = p.tiles_m, sub_n = p.tiles_n, off_m = 0, off_n = 0;
        int t = blockIdx.x;
        if ((p.tiles_m & 1) == 0 && (p.tiles_n & 3) == 0) {
            const int x = t & 7;
            t >>= 3;
            sub_m = p.tiles_m >> 1;
            sub_n = p.tiles_n >> 2;
            off_m = (x >> 2) * sub_m;
            off_n = (x & 3) * sub_n;
        }
        const int per_group = GROUP_M * sub_n;
        const int grp = t / per_group;
        const int first_m = grp * GROUP_M;
        const int gsz = min(sub_m - first_m, GROUP_M);
        const int in = t - grp * per_group;
        tile_m = off_m + first_m + in % gsz;
        tile_n = off_n + in / gsz;
        rows_valid = p.M - tile_m * BM;
    } else {
        find_expert_tile<BM>(p, blockIdx.x, sh);
        expert = sh[0];
        if (expert < 0) return;  // no tile for this workgroup (uniform over the block)
        const int local = sh[1];
        row_begin = p.offsets[expert];
        const int rows_e = p.offsets[expert + 1] - row_begin;
        const int mt_e = (rows_e + BM - 1) / BM;
        // inside the expert: groups of GROUP_M row tiles, row tiles fastest
        const int per_group = GROUP_M * p.tiles_n;
        const int grp = local / per_group;
        const int first_m = grp * GROUP_M;
        const int gsz = min(mt_e - first_m, GROUP_M);
        const int in = local - grp * per_group;
        tile_m = first_m + in % gsz;
        tile_n = in / gsz;
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

    // ---- tile scales -> LDS (used by the epilogue) ------------------------
    constexpr int RING = 2 * STAGE;
    float* s_ch_t = reinterpret_cast<float*>(smem + RING);
    float* s_tok_t = s_ch_t + BN;
    for (int i = tid; i < BN; i += NTH) s_ch_t[i] = MX ? 1.0f : s_ch[min(n0 + i, p.N - 1)];
    for (int i = tid; i < BM; i += NTH) {
        const int ml = min(i, rows_valid - 1);
        if constexpr (MX)
            s_tok_t[i] = 1.0f;
        else if constexpr (GROUPED)
            s_tok_t[i] = p.s_tok[p.row_token[row_begin + m0 + ml]];
        else
            s_tok_t[i] = p.s_tok[m0 + ml];
    }

    // ---- per-lane DMA sources ----------------------------------------------
    // Instruction j of this wave covers tile rows (wave * D + j) * 8 .. +7;
    // lane l takes row l / 8 of those and the piece (l % 8) ^ swz(row).
    const int lrow = lane >> 3;
    const int lpos = lane & 7;
    const uint8_t* bsrc[DB];
#pragma unroll
    for (int j = 0; j < DB; ++j) {
        const int row = (wave * DB + j) * 8 + lrow;
        const int ml = min(row, rows_valid - 1);  // rows past the tile feed discarded rows
        int64_t src_row;
        if constexpr (GROUPED)
            src_row = p.row_token[row_begin + m0 + ml];
        else
            src_row = m0 + ml;
        bsrc[j] = p.qa + src_row * lda + ((lpos ^ dswz(row)) << 4);
    }
    const int nlast = p.N - 1;
    const uint8_t* pf_src = qw + (int64_t)min(n0 + wave * 64 + lane, nlast) * ldw;
    auto prefetch_a = [&](int kt) {
        if constexpr (PF) __builtin_amdgcn_global_load_lds(pf_src + kt * kBK, pf_lds, 4, 0, 0);
    };
    // Block-scale DMA (MX): instruction j of this wave fetches the stage's
    // scale words of tile rows (wave * DS + j) * 64 + lane, weight rows first.
    const uint8_t* ssrc[DS + 1];
    int64_t sstep[DS + 1];  // bytes between consecutive stages' words of a row
    if constexpr (MX) {
#pragma unroll
        for (int j = 0; j < DS; ++j) {
            const int r = (wave * DS + j) * 64 + lane;
            ssrc[j] = r < BN ? p.mx.sw + 4 * (int64_t)min(n0 + r, nlast)
                             : p.mx.sa + 4 * (int64_t)(m0 + min(r - BN, rows_valid - 1));
            sstep[j] = 4 * (int64_t)(r < BN ? p.N : p.M);
        }
    }
    auto issue_scale = [&](int kt, int slot, int j) {
        __builtin_amdgcn_global_load_lds(ssrc[j] + kt * sstep[j],
                                         smem + SRING + slot * 4 * (BN + BM) + (wave * DS + j) * 256, 4, 0, 0);
    };

    // DMA instruction j (0 .. PER_STAGE - 1) of stage kt into ring slot `slot`.
    auto issue_one = [&](int kt, int slot, int j) {
        uint8_t* base = smem + slot * STAGE;
        const int koff = kt * kBK;
        if (j >= DA + DB) {
            if constexpr (MX) issue_scale(kt, slot, j - DA - DB);
        } else if (j < DA) {
            const int row = (wave * DA + j) * 8 + lrow;
            const int n = min(n0 + row, nlast);  // rows past N feed discarded columns
            dma16(qw + (int64_t)n * ldw + koff + ((lpos ^ dswz(row)) << 4), base + (wave * DA + j) * 1024);
        } else {
            const int jb = j - DA;
            dma16(bsrc[jb] + koff, base + BN * kBK + (wave * DB + jb) * 1024);
        }
    };
    // Stage kt goes to ring slot `slot` (0 or 1).
    auto issue_stage = [&](int kt, int slot) {
        uint8_t* base = smem + slot * STAGE;
        const int koff = kt * kBK;
#pragma unroll
        for (int j = 0; j < DA; ++j) {
            const int row = (wave * DA + j) * 8 + lrow;
            const int n = min(n0 + row, nlast);  // rows past N feed discarded columns
            dma16(qw + (int64_t)n * ldw + koff + ((lpos ^ dswz(row)) << 4), base + (wave * DA + j) * 1024);
        }
#pragma unroll
        for (int j = 0; j < DB; ++j) dma16(bsrc[j] + koff, base + BN * kBK + (wave * DB + j) * 1024);
        if constexpr (MX) {
#pragma unroll
            for (int j = 0; j < DS; ++j) issue_scale(kt, slot, j);
        }
    };

    v16f acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

    const int KT = p.K / kBK;
    const int arow0 = wn * (BN / WN) + r32;
    // Activation fragment b of wave (wn, wm) covers tile rows
    // (b * WM + wm) * 32 .. + 31: the waves along M take alternate 32-row
    // blocks, so a partly filled tile leaves them equal shares of real rows.
    const int brow0 = wm * 32 + r32;
    auto read_a = [&](int slot, int h, int a) { return read_frag(smem + slot * STAGE, arow0 + a * 32, h, g); };
    auto read_b = [&](int slot, int h, int b) {
        return read_frag(smem + slot * STAGE + BN * kBK, brow0 + b * (32 * WM), h, g);
    };

    // Block scales (MX): the word of 4 exponent bytes of each of the lane's
    // fragment rows; sc_* for the stage being computed, nx_* for the next.
    constexpr int SF = MX ? 1 : 0;
    uint32_t sc_a[FN * SF + 1], sc_b[FM * SF + 1], nx_a[FN * SF + 1], nx_b[FM * SF + 1];
    auto read_scales = [&](int slot, uint32_t (&wa)[FN * SF + 1], uint32_t (&wb)[FM * SF + 1]) {
        if constexpr (MX) {
            const uint32_t* base = reinterpret_cast<const uint32_t*>(smem + SRING + slot * 4 * (BN + BM));
#pragma unroll
            for (int a = 0; a < FN; ++a) wa[a] = base[arow0 + a * 32];
#pragma unroll
            for (int b = 0; b < FM; ++b) wb[b] = base[BN + brow0 + b * (32 * WM)];
        }
    };
    auto next_scales = [&]() {
        if constexpr (MX) {
#pragma unroll
            for (int a = 0; a < FN; ++a) sc_a[a] = nx_a[a];
#pragma unroll
            for (int b = 0; b < FM; ++b) sc_b[b] = nx_b[b];
        }
    };
    // exponent byte for K half h of the current stage
    auto sbyte = [&](uint32_t w, int h) { return (int)__builtin_amdgcn_ubfe(w, 16 * h + 8 * g, 8); };
    auto mma = [&](const v8i& x, const v8i& w2, const v16f& c, int a, int b, int h) {
        if constexpr (MX)
            return mfma_32x32x64_e4m3_mx(x, w2, c, sbyte(sc_a[a], h), sbyte(sc_b[b], h));
        else
            return mfma_32x32x64_e4m3(x, w2, c);
    };
    // scale-word LDS instructions per step: the rows are 32 words apart, so
    // the compiler pairs the reads into ds_read2_b32
    constexpr int SR = MX ? (FN + FM) / 2 : 0;

    // The K loop for FA active activation fragments per wave (FA <= FM).  A
    // wave whose last fragments cover only rows past the tile's real rows
    // (the last row tile of an expert, or of a short M) skips their MFMAs and LDS reads; its
    // DMA share, waits and barriers are the same for every FA, so the waves
    // of one workgroup stay in step whatever their FA.
    auto k_loop = [&](auto fa_count) {
        constexpr int FA = decltype(fa_count)::value;
        v8i fa[FN], fb[FA];
        if (KT > 0) {
            // prologue: stages 0 and 1 in flight, stage 0 landed everywhere,
            // its first-half fragments in registers
            issue_stage(0, 0);
            if (KT > 1) issue_stage(1, 1);
            if (PF && KT > 2) prefetch_a(2);
            if (PF && KT > 2) {
                static_assert(PER_STAGE + 1 <= 63, "vmcnt field");
                compiler_fence();
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER_STAGE + 1) : "memory");
                compiler_fence();
            } else {
                wait_dma<PER_STAGE>(KT > 1 ? 1 : 0);
            }
            block_barrier();
            read_scales(0, sc_a, sc_b);
#pragma unroll
            for (int b = 0; b < FA; ++b) fb[b] = read_b(0, 0, b);
#pragma unroll
            for (int a = 0; a < FN; ++a) fa[a] = read_a(0, 0, a);
        }
        // Steps with a stage s+2 to load: no branches in the body, the DMA
        // instructions of stage s+2 dealt round-robin to the second-half MFMAs
        // (in program order they must precede the LDS reads that follow them,
        // which keeps them spread out instead of in one burst after the barrier).
        int s = 0;
        for (; s + 2 < KT; ++s) {
            const int cur = s & 1;
#pragma unroll
            for (int a = 0; a < FN; ++a) {
#pragma unroll
                for (int b = 0; b < FA; ++b) {
                    acc[a][b] = mma(fa[a], fb[b], acc[a][b], a, b, 0);
                    if (a == FN - 1) fb[b] = read_b(cur, 1, b);
                }
                fa[a] = read_a(cur, 1, a);
            }
            interleave_mfma_reads<FN * FA, 2 * (FN + FA)>();
            // this wave's part of stage s+1 landed (with prefetching, the
            // touch of stage s+2, issued after it, may still be in flight)
            if constexpr (PF) {
                compiler_fence();
                asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
                compiler_fence();
            } else {
                wait_dma<PER_STAGE>(0);
            }
            wait_lds_reads();        // ... and its reads of stage s are done
            block_barrier();
            read_scales(cur ^ 1, nx_a, nx_b);
#pragma unroll
            for (int a = 0; a < FN; ++a) {
#pragma unroll
                for (int b = 0; b < FA; ++b) {
                    acc[a][b] = mma(fa[a], fb[b], acc[a][b], a, b, 1);
#pragma unroll
                    for (int j = a * FA + b; j < PER_STAGE; j += FN * FA) issue_one(s + 2, cur, j);
                    if (a == FN - 1) fb[b] = read_b(cur ^ 1, 0, b);
                }
                fa[a] = read_a(cur ^ 1, 0, a);
            }
            interleave_mfma_reads<FN * FA, 2 * (FN + FA) + SR>();
            if (PF && s + 3 < KT) prefetch_a(s + 3);  // issued last: the next step waits for all but it
            next_scales();
        }
        // The last two steps (nothing left to load).
        for (; s < KT; ++s) {
            const int cur = s & 1;
            const bool more = s + 1 < KT;
            // first K half of stage s; refill with the second half
#pragma unroll
            for (int a = 0; a < FN; ++a) {
#pragma unroll
                for (int b = 0; b < FA; ++b) {
                    acc[a][b] = mma(fa[a], fb[b], acc[a][b], a, b, 0);
                    if (a == FN - 1) fb[b] = read_b(cur, 1, b);
                }
                fa[a] = read_a(cur, 1, a);
            }
            interleave_mfma_reads<FN * FA, 2 * (FN + FA)>();
            if (more) {
                wait_dma<PER_STAGE>(0);
                wait_lds_reads();
                block_barrier();
                read_scales(cur ^ 1, nx_a, nx_b);
            }
            // second K half of stage s; refill with the first half of stage s+1
            // (the last step re-reads its own slot, unused)
            const int nxt = more ? cur ^ 1 : cur;
#pragma unroll
            for (int a = 0; a < FN; ++a) {
#pragma unroll
                for (int b = 0; b < FA; ++b) {
                    acc[a][b] = mma(fa[a], fb[b], acc[a][b], a, b, 1);
                    if (a == FN - 1) fb[b] = read_b(nxt, 0, b);
                }
                fa[a] = read_a(nxt, 0, a);
            }
            interleave_mfma_reads<FN * FA, 2 * (FN + FA)>();
            if (more) next_scales();
        }
    };
    // Fragments holding at least one real row (at least 1, so that every wave
    // runs the loop body; a wave with none computes one discarded fragment).
    const int fa_live = min(FM, max(1, (rows_valid - wm * 32 + 32 * WM - 1) / (32 * WM)));
    if constexpr ((GROUPED || SKIP) && FM == 4 && !MX) {
        switch (fa_live) {
            case 1: k_loop(std::integral_constant<int, 1>{}); break;
            case 2: k_loop(std::integral_constant<int, 2>{}); break;
            case 3: k_loop(std::integral_constant<int, 3>{}); break;
            default: k_loop(std::integral_constant<int, 4>{}); break;
        }
    } else {
        (void)fa_live;
        k_loop(std::integral_constant<int, FM>{});
    }

    // ---- epilogue: y = bf16_rne(acc * (s_tok * s_ch)) ----------------------
    // The scaled BF16 tile is staged in LDS (the stage ring is free now) as
    // [BM rows][BN columns] with 16-byte chunks XOR-swizzled by row, then
    // written out with 16-byte row-contiguous stores.
    // Accumulator layout of a 32x32 MFMA tile: lane l holds activation row
    // l % 32 and weight columns 8 * (v / 4) + 4 * (l / 32) + v % 4, v = 0..15.
    if constexpr (!GROUPED) {
        if (p.y32 != nullptr) {
            // fp32 output straight from the accumulators: lane l holds 4
            // consecutive columns per group q (one 16-byte store when aligned).
            const bool vec = (p.ldy & 3) == 0;
#pragma unroll
            for (int b = 0; b < FM; ++b) {
                const int ml = (b * WM + wm) * 32 + r32;
                if (ml >= rows_valid) continue;
                const float st = s_tok_t[ml];
                float* yr = p.y32 + (int64_t)(m0 + ml) * p.ldy;
#pragma unroll
                for (int a = 0; a < FN; ++a) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nl = wn * (BN / WN) + a * 32 + 8 * q + 4 * g;
                        const int n = n0 + nl;
                        if (n >= p.N) continue;
                        const float4 sc4 = *reinterpret_cast<const float4*>(s_ch_t + nl);
                        const float o0 = acc[a][b][4 * q + 0] * (st * sc4.x), o1 = acc[a][b][4 * q + 1] * (st * sc4.y);
                        const float o2 = acc[a][b][4 * q + 2] * (st * sc4.z), o3 = acc[a][b][4 * q + 3] * (st * sc4.w);
                        if (vec && n + 3 < p.N) {
                            *reinterpret_cast<float4*>(yr + n) = make_float4(o0, o1, o2, o3);
                        } else {
                            if (n < p.N) yr[n] = o0;
                            if (n + 1 < p.N) yr[n + 1] = o1;
                            if (n + 2 < p.N) yr[n + 2] = o2;
                            if (n + 3 < p.N) yr[n + 3] = o3;
                        }
                    }
                }
            }
            return;
        }
    }
    wait_lds_reads();
    block_barrier();
    uint8_t* ct = smem;
    constexpr int CH = BN / 8;  // 16-byte chunks per tile row
#pragma unroll
    for (int b = 0; b < FM; ++b) {
        const int ml = (b * WM + wm) * 32 + r32;
        const float st = s_tok_t[ml];
#pragma unroll
        for (int a = 0; a < FN; ++a) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * (BN / WN) + a * 32 + 8 * q + 4 * g;
                const float4 sc4 = *reinterpret_cast<const float4*>(s_ch_t + nl);
                const float sc[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
                uint2 o;
                o.x = pack_bf16x2(acc[a][b][4 * q + 0] * (st * sc[0]), acc[a][b][4 * q + 1] * (st * sc[1]));
                o.y = pack_bf16x2(acc[a][b][4 * q + 2] * (st * sc[2]), acc[a][b][4 * q + 3] * (st * sc[3]));
                const int chunk = (nl >> 3) ^ (ml & (CH - 1) & 31);
                *reinterpret_cast<uint2*>(ct + ml * (BN * 2) + chunk * 16 + (nl & 7) * 2) = o;
            }
        }
    }
    block_barrier();
    const bool vec_store = GROUPED ? (p.N & 7) == 0 : (p.ldy & 7) == 0;
    const int64_t ldy = GROUPED ? (int64_t)p.N : p.ldy;
#pragma unroll 4
    for (int id = tid; id < BM * CH; id += NTH) {
        const int row = id / CH, c = id % CH;
        if (row >= rows_valid) continue;
        const int n = n0 + c * 8;
        if (n >= p.N) continue;
        const int chunk = c ^ (row & (CH - 1) & 31);
        const v4i val = *reinterpret_cast<const v4i*>(ct + row * (BN * 2) + chunk * 16);
        const int64_t yrow = GROUPED ? (int64_t)row_begin + m0 + row : (int64_t)m0 + row;
        uint16_t* dst = p.y + yrow * ldy + n;
        if (vec_store && n + 8 <= p.N) {
            __builtin_nontemporal_store(val, reinterpret_cast<v4i*>(dst));  // written once, read by the next layer
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < p.N) dst[e] = (uint16_t)((uint32_t)val[e >> 1] >> ((e & 1) * 16));
        }
    }
}

hipError_t launch_gemm_mfma(const uint8_t* qa, int64_t lda, const float* s_tok, const uint8_t* qw, int64_t ldw,
                            const float* s_ch, uint16_t* y, float* y32, int64_t ldy, int64_t M, int64_t N, int64_t K,
                            hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    constexpr int BN = 256, BM = 256, WN = 2, WM = 2;
    constexpr int LDS = 2 * (BN + BM) * kBK + 4 * (BN + BM);  // ring + tile scales
    MfmaArgs p{};
    p.qa = qa; p.lda = lda; p.s_tok = s_tok; p.qw = qw; p.ldw = ldw; p.s_ch = s_ch; p.y = y; p.y32 = y32; p.ldy = ldy;
    p.M = (int)M; p.N = (int)N; p.K = (int)K;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
    if (M <= BM - 64) {
        // one row of tiles whose last 32-row fragments are empty for both waves along M
        hipError_t e = FP8K_SET_LDS((gemm_mfma_kernel<BN, BM, WN, WM, 4, false, false, true>), LDS);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((gemm_mfma_kernel<BN, BM, WN, WM, 4, false, false, true>), dim3(grid), dim3(64 * WN * WM), LDS,
                           stream, p);
        return hipGetLastError();
    }
    hipError_t e = FP8K_SET_LDS((gemm_mfma_kernel<BN, BM, WN, WM, 4, false>), LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_mfma_kernel<BN, BM, WN, WM, 4, false>), dim3(grid), dim3(64 * WN * WM), LDS, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm_mfma_mx(const uint8_t* qa, int64_t lda, const uint8_t* sa, const uint8_t* qw, int64_t ldw,
                               const uint8_t* sw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    constexpr int BN = 256, BM = 256, WN = 2, WM = 2;
    // ring + tile scales (ones) + block-scale ring
    constexpr int LDS = 2 * (BN + BM) * kBK + 4 * (BN + BM) + 2 * 4 * (BN + BM);
    MfmaArgs p{};
    p.qa = qa; p.lda = lda; p.qw = qw; p.ldw = ldw; p.y = y; p.ldy = ldy;
    p.M = (int)M; p.N = (int)N; p.K = (int)K;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    p.mx = MxScales{sa, sw};
    hipError_t e = FP8K_SET_LDS((gemm_mfma_kernel<BN, BM, WN, WM, 4, false, true>), LDS);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
    hipLaunchKernelGGL((gemm_mfma_kernel<BN, BM, WN, WM, 4, false, true>), dim3(grid), dim3(64 * WN * WM), LDS, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm_grouped_mfma(const uint8_t* qa, const float* s_tok, const int32_t* row_token,
                                    const int32_t* offsets, const uint8_t* qw, const float* s_ch, uint16_t* y,
                                    int64_t T, int64_t R, int64_t E, int64_t N, int64_t K, hipStream_t stream) {
    (void)T;
    if (R <= 0 || N <= 0 || E <= 0) return hipSuccess;
    constexpr int BN = 256, BM = 256, WN = 2, WM = 2;
    constexpr int LDS = 2 * (BN + BM) * kBK + 4 * (BN + BM) + 16 + 256;  // ring + tile scales + tile lookup + prefetch slot
    MfmaArgs p{};
    p.qa = qa; p.lda = K; p.s_tok = s_tok; p.qw = qw; p.ldw = K; p.s_ch = s_ch; p.y = y; p.ldy = N;
    p.M = (int)R; p.N = (int)N; p.K = (int)K;
    p.tiles_n = (int)((N + BN - 1) / BN);
    p.row_token = row_token; p.offsets = offsets; p.E = (int)E;
    constexpr int GM = 4;
    hipError_t e = FP8K_SET_LDS((gemm_mfma_kernel<BN, BM, WN, WM, GM, true>), LDS);
    if (e != hipSuccess) return e;
    // sum over experts of ceil(rows_e / BM) <= ceil(R / BM) + E; each of the 8
    // XCD ranges holds at most ceil(total / 8) tiles
    const int64_t tiles_max = ((R + BM - 1) / BM + E) * p.tiles_n;
    const int64_t grid = 8 * ((tiles_max + 7) / 8);
    hipLaunchKernelGGL((gemm_mfma_kernel<BN, BM, WN, WM, GM, true>), dim3((unsigned)grid), dim3(64 * WN * WM), LDS, stream,
                       p);
    return hipGetLastError();
}

}  // namespace fp8k
