// The projection GEMM of the self-attention block (CDNA4, gfx950).
#pragma once

#include "common.hpp"

namespace regen {

// ---------------------------------------------------------------------------
// gemm_nt_kernel: a linear layer without bias, C = A B^T: A [M][K] (row stride
// lda), B [N][K] (row stride ldb: the [out][in] weight of the layer), C [M][N]
// (row stride ldc); bf16 in, fp32 accumulation, bf16 out (RNE). K % 64 == 0.
// A workgroup of 4 waves computes a 128 x 128 tile (64 x 64 per wave, 2 x 2
// MFMA blocks) or a 64 x 64 quarter tile (32 x 32 per wave), with K steps of
// 64 through double-buffered LDS filled by LDS-DMA copies (128-byte rows,
// chunk ^ ((row >> 1) & 7)). Rows past M or N read as zero (buffer
// resources) and are not stored.
// ---------------------------------------------------------------------------
constexpr int kGemmTile = 128, kGemmBK = 64;
constexpr int kGemmTileBytes = kGemmTile * kGemmBK * 2;

// Copies of the first 32 RUNS rows x 64 k of a tile (RUNS runs of 1 KiB per
// wave; RUNS = 4: all 128 rows, RUNS = 2: 64 rows).
template <int RUNS>
__device__ __forceinline__ void gemm_issue(__amdgpu_buffer_rsrc_t rs, int ld, int row0, int k0,
                                           char* lds, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < RUNS; ++i) {
        const int run = i * 4 + wave;
        const int p = run * 64 + lane;  // chunk position in the tile
        const int r = p >> 3, pc = p & 7;
        const int c = pc ^ ((r >> 1) & 7);  // the logical chunk stored at pc
        g2lds16(rs, (uint32_t)(((long long)(row0 + r) * ld + k0 + c * 8) * 2), lds + run * 1024);
    }
}

// One (2 WT) x (2 WT) output tile at (m0, n0), WT x WT per wave (WT = 64 or
// 32). The MFMA computes the tile transposed (B rows as its first operand), so
// that a lane ends up with 4 consecutive columns of one output row: 8-byte
// stores.
template <int WT>
__device__ __forceinline__ void gemm_tile(__amdgpu_buffer_rsrc_t ra, int lda,
                                          __amdgpu_buffer_rsrc_t rb, int ldb,
                                          uint16_t* __restrict__ C, int ldc, int M, int N, int K,
                                          int m0, int n0, char (*smem)[2][kGemmTileBytes]) {
    constexpr int NB = WT / 32, RUNS = WT / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[NB][NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    gemm_issue<RUNS>(ra, lda, m0, 0, smem[0][0], wave, lane);
    gemm_issue<RUNS>(rb, ldb, n0, 0, smem[0][1], wave, lane);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int nk = K / kGemmBK;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            gemm_issue<RUNS>(ra, lda, m0, (kt + 1) * kGemmBK, smem[buf ^ 1][0], wave, lane);
            gemm_issue<RUNS>(rb, ldb, n0, (kt + 1) * kGemmBK, smem[buf ^ 1][1], wave, lane);
        }
        const char* as = smem[buf][0];
        const char* bs = smem[buf][1];
#pragma unroll
        for (int kk = 0; kk < kGemmBK / 16; ++kk) {
            bf16x8 a[NB], b[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(as + swz_off<128>(wm * WT + i * 32 + col, kk * 2 + half));
#pragma unroll
            for (int j = 0; j < NB; ++j)
                b[j] = *reinterpret_cast<const bf16x8*>(bs + swz_off<128>(wn * WT + j * 32 + col, kk * 2 + half));
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
        }
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    // Lane (col, half) holds C[m][n] for m = its row col of the block and
    // n = 8 g + 4 half + e (g, e < 4) of the block's 32 columns.
    const bool st8 = (ldc & 3) == 0;  // 8-byte aligned runs of 4
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int m = m0 + wm * WT + i * 32 + col;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WT + j * 32 + g * 8 + half * 4;
                const f32x16& v = acc[i][j];
                uint16_t* cp = C + (long long)m * ldc + n;
                if (st8 && n + 3 < N) {
                    *reinterpret_cast<uint2*>(cp) = make_uint2(pack_bf16(v[g * 4], v[g * 4 + 1]),
                                                               pack_bf16(v[g * 4 + 2], v[g * 4 + 3]));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) cp[e] = (uint16_t)(pack_bf16(v[g * 4 + e], 0.0f) & 0xffffu);
                }
            }
    }
}

// The 128 x 128 tiles are numbered in groups of 8 tile rows (column-major
// inside a group), so that workgroups running together share A and B tiles
// in L2. Workgroups [0, nfull) take tiles [0, nfull), remapped so that each
// XCD walks one contiguous range of them. When the tile count leaves a last
// round that would keep only a few CUs busy, the host makes nfull the tiles
// of the full rounds, and workgroups nfull.. take each remaining tile as four
// 64 x 64 quarters, spreading that round over four times as many CUs.
__global__ __launch_bounds__(256) void gemm_nt_kernel(const uint16_t* __restrict__ A, int lda,
                                                      const uint16_t* __restrict__ B, int ldb,
                                                      uint16_t* __restrict__ C, int ldc, int M,
                                                      int N, int K, int nfull) {
    __shared__ __attribute__((aligned(1024))) char smem[2][2][kGemmTileBytes];  // [buffer][A, B]
    constexpr int GM = 8;
    const int mt = (M + kGemmTile - 1) / kGemmTile, nt = (N + kGemmTile - 1) / kGemmTile;
    const int bid = blockIdx.x;
    const int t = bid < nfull ? xcd_remap(bid, nfull) : nfull + (bid - nfull) / 4;
    const int first = (t / (GM * nt)) * GM;
    const int gm = min(mt - first, GM);
    const int r = t - first * nt;
    int m0 = (first + r % gm) * kGemmTile, n0 = (r / gm) * kGemmTile;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)((long long)M * lda * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (uint32_t)((long long)N * ldb * 2));
    if (bid < nfull) {
        gemm_tile<64>(ra, lda, rb, ldb, C, ldc, M, N, K, m0, n0, smem);
    } else {
        const int quarter = (bid - nfull) & 3;
        m0 += (quarter >> 1) * 64;
        n0 += (quarter & 1) * 64;
        gemm_tile<32>(ra, lda, rb, ldb, C, ldc, M, N, K, m0, n0, smem);
    }
}

// ---------------------------------------------------------------------------
// gemm_nt256_kernel: the same product for large outputs, persistent. G
// workgroups of 8 waves (one per CU: 128 KiB of LDS). The output is cut into
// 256 x 256 tiles (64 x 128 per wave, 2 x 4 MFMA blocks, K steps of 64,
// double-buffered LDS-DMA copies as above); workgroup p computes tiles
// p, p + G, ... of the first `rounds` G tiles, then the remaining tiles as
// 128 x 64 eighths (32 x 32 per wave) when they fit in one round, else as
// 128 x 128 quarters (32 x 64 per wave), quarter q to workgroup q mod G.
// Tiles are numbered in groups of 4 tile rows as in gemm_nt_kernel, and the
// workgroups of one XCD take consecutive numbers. A tile's C goes out
// through LDS in whole rows (16-byte chunks, a row of a wave's block per 8
// or 16 lanes) wherever the tile lies within N and rows are 16-byte aligned.
// ---------------------------------------------------------------------------
constexpr int kGemmBig = 256;
constexpr int kGemmBigSmem = 2 * 2 * kGemmBig * kGemmBK * 2;  // [buffer][A, B] at 256 rows

// Copies of ROWS rows x 64 k of a tile (ROWS / 8 runs of 1 KiB over 8 waves).
template <int ROWS>
__device__ __forceinline__ void gemm8_issue(__amdgpu_buffer_rsrc_t rs, int ld, int row0, int k0, char* lds,
                                            int wave, int lane) {
#pragma unroll
    for (int i = 0; i < ROWS / 64; ++i) {
        const int run = i * 8 + wave;
        const int p = run * 64 + lane;
        const int r = p >> 3, pc = p & 7;
        const int c = pc ^ ((r >> 1) & 7);
        g2lds16(rs, (uint32_t)(((long long)(row0 + r) * ld + k0 + c * 8) * 2), lds + run * 1024);
    }
}

// One (4 WTM) x (2 WTN) tile at (m0, n0) by 8 waves (WTM x WTN each), K
// steps through STAGES LDS buffers (STAGES * SBYTES <= 128 KiB): two for
// the full tiles, more for the small tiles of a last round, whose steps are
// too short to hide a copy's latency behind one step of work. Ends with
// every wave past its last read of `smem`.
template <int WTM, int WTN, int STAGES = 2>
__device__ __forceinline__ void gemm8_tile(__amdgpu_buffer_rsrc_t ra, int lda, __amdgpu_buffer_rsrc_t rb,
                                           int ldb, uint16_t* __restrict__ C, int ldc, int M, int N, int K,
                                           int m0, int n0, char* smem) {
    constexpr int TM = 4 * WTM, TN = 2 * WTN, NBM = WTM / 32, NBN = WTN / 32;
    constexpr int ABYTES = TM * kGemmBK * 2, SBYTES = (TM + TN) * kGemmBK * 2;
    static_assert(STAGES >= 2 && STAGES * SBYTES <= kGemmBigSmem, "LDS stages");
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[NBM][NBN];
#pragma unroll
    for (int i = 0; i < NBM; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = K / kGemmBK;
    auto mma_step = [&](const char* as, const char* bs) {
#pragma unroll
        for (int kk = 0; kk < kGemmBK / 16; ++kk) {
            bf16x8 a[NBM], b[NBN];
#pragma unroll
            for (int i = 0; i < NBM; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(as + swz_off<128>(wm * WTM + i * 32 + col, kk * 2 + half));
#pragma unroll
            for (int j = 0; j < NBN; ++j)
                b[j] = *reinterpret_cast<const bf16x8*>(bs + swz_off<128>(wn * WTN + j * 32 + col, kk * 2 + half));
#pragma unroll
            for (int i = 0; i < NBM; ++i)
#pragma unroll
                for (int j = 0; j < NBN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
        }
    };
    if constexpr (STAGES > 2) {
        // Copies run STAGES - 1 steps ahead. Step kt: wait for this wave's
        // copies of step kt (those of the later steps already issued may stay
        // in flight: CP copies per step per wave), barrier (every wave's
        // copies of kt have landed and every wave is past step kt - 1, whose
        // buffer the copies of step kt + STAGES - 1 now reuse), compute.
        constexpr int CP = TM / 64 + TN / 64;
        for (int s = 0; s < STAGES - 1 && s < nk; ++s) {
            gemm8_issue<TM>(ra, lda, m0, s * kGemmBK, smem + s * SBYTES, wave, lane);
            gemm8_issue<TN>(rb, ldb, n0, s * kGemmBK, smem + s * SBYTES + ABYTES, wave, lane);
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int later = min(STAGES - 2, nk - 1 - kt);  // steps issued after kt
            static_assert(STAGES <= 5 && 3 * CP < 64, "wait counts below");
            if (later >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_only(3 * CP));
            else if (later == 2) __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * CP));
            else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_only(CP));
            else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            __builtin_amdgcn_s_barrier();
            if (kt + STAGES - 1 < nk) {
                char* nxt = smem + ((kt + STAGES - 1) % STAGES) * SBYTES;
                gemm8_issue<TM>(ra, lda, m0, (kt + STAGES - 1) * kGemmBK, nxt, wave, lane);
                gemm8_issue<TN>(rb, ldb, n0, (kt + STAGES - 1) * kGemmBK, nxt + ABYTES, wave, lane);
            }
            const char* cur = smem + (kt % STAGES) * SBYTES;
            mma_step(cur, cur + ABYTES);
        }
        __syncthreads();
    } else {
        gemm8_issue<TM>(ra, lda, m0, 0, smem, wave, lane);
        gemm8_issue<TN>(rb, ldb, n0, 0, smem + ABYTES, wave, lane);
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            char* cur = smem + (kt & 1) * SBYTES;
            if (kt + 1 < nk) {
                char* nxt = smem + ((kt + 1) & 1) * SBYTES;
                gemm8_issue<TM>(ra, lda, m0, (kt + 1) * kGemmBK, nxt, wave, lane);
                gemm8_issue<TN>(rb, ldb, n0, (kt + 1) * kGemmBK, nxt + ABYTES, wave, lane);
            }
            mma_step(cur, cur + ABYTES);
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }
    if (n0 + TN <= N && (ldc & 7) == 0) {  // uniform
        // C through LDS (free now: every wave is past its last operand
        // read): each wave writes its WTM x WTN block in bf16 row-major into
        // its own part of smem (16-byte chunks XOR-swizzled by row), reads
        // it back as whole row chunks and stores it so that each store
        // instruction writes whole rows (at WTN = 128 two 128-byte lines
        // per row). The L2 then takes whole lines rather than 8-byte pieces
        // from 32 rows per instruction, which made writing C cost about
        // twice as much.
        constexpr int CPR = WTN / 8, RPI = 64 / CPR;  // 16-byte chunks per row, rows per store
        static_assert(8 * WTM * WTN * 2 <= kGemmBigSmem && RPI * CPR == 64, "C staging");
        char* ws = smem + wave * (WTM * WTN * 2);
#pragma unroll
        for (int i = 0; i < NBM; ++i)
#pragma unroll
            for (int j = 0; j < NBN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int r = i * 32 + col, c = j * 4 + g;
                    const f32x16& v = acc[i][j];
                    *reinterpret_cast<uint2*>(ws + r * (WTN * 2) + (c ^ (r & (CPR - 1))) * 16 + half * 8) =
                        make_uint2(pack_bf16(v[g * 4], v[g * 4 + 1]), pack_bf16(v[g * 4 + 2], v[g * 4 + 3]));
                }
        // A wave's LDS accesses complete in order: its reads below see its
        // writes above.
#pragma unroll
        for (int k = 0; k < WTM / RPI; ++k) {
            const int r = k * RPI + lane / CPR, c = lane % CPR;
            const uint4 x = *reinterpret_cast<const uint4*>(ws + r * (WTN * 2) + (c ^ (r & (CPR - 1))) * 16);
            const int m = m0 + wm * WTM + r;
            if (m < M) *reinterpret_cast<uint4*>(C + (long long)m * ldc + n0 + wn * WTN + c * 8) = x;
        }
        // Every wave is done reading smem before the next tile's copies
        // refill it (the stores need not have completed: no vmcnt wait).
        __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
        __builtin_amdgcn_s_barrier();
        return;
    }
    const bool st8 = (ldc & 3) == 0;
#pragma unroll
    for (int i = 0; i < NBM; ++i) {
        const int m = m0 + wm * WTM + i * 32 + col;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NBN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WTN + j * 32 + g * 8 + half * 4;
                const f32x16& v = acc[i][j];
                uint16_t* cp = C + (long long)m * ldc + n;
                if (st8 && n + 3 < N) {
                    *reinterpret_cast<uint2*>(cp) = make_uint2(pack_bf16(v[g * 4], v[g * 4 + 1]),
                                                               pack_bf16(v[g * 4 + 2], v[g * 4 + 3]));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) cp[e] = (uint16_t)(pack_bf16(v[g * 4 + e], 0.0f) & 0xffffu);
                }
            }
    }
}

__global__ __launch_bounds__(512) void gemm_nt256_kernel(const uint16_t* __restrict__ A, int lda,
                                                         const uint16_t* __restrict__ B, int ldb,
                                                         uint16_t* __restrict__ C, int ldc, int M, int N,
                                                         int K, int rounds) {
    __shared__ __attribute__((aligned(1024))) char smem[kGemmBigSmem];
    constexpr int GM = 4;
    const int G = gridDim.x;
    const int pid = xcd_remap(blockIdx.x, G);
    const int mt = (M + kGemmBig - 1) / kGemmBig, nt = (N + kGemmBig - 1) / kGemmBig;
    const int tiles = mt * nt;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)((long long)M * lda * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (uint32_t)((long long)N * ldb * 2));
    auto origin = [&](int t, int* m0, int* n0) {
        const int first = (t / (GM * nt)) * GM;
        const int gm = min(mt - first, GM);
        const int r = t - first * nt;
        *m0 = (first + r % gm) * kGemmBig;
        *n0 = (r / gm) * kGemmBig;
    };
    for (int k = 0; k < rounds; ++k) {
        int m0, n0;
        origin(k * G + pid, &m0, &n0);
        gemm8_tile<64, 128>(ra, lda, rb, ldb, C, ldc, M, N, K, m0, n0, smem);
    }
    const int done = rounds * G, left = tiles - done;
    if (left * 8 <= G) {
        // Eighths (128 x 64, 32 x 32 per wave) when they fit in one round.
        if (pid < left * 8) {
            int m0, n0;
            origin(done + pid / 8, &m0, &n0);
            gemm8_tile<32, 32, 4>(ra, lda, rb, ldb, C, ldc, M, N, K, m0 + ((pid & 7) >> 2) * 128,
                               n0 + (pid & 3) * 64, smem);
        }
        return;
    }
    for (int qd = pid; qd < left * 4; qd += G) {
        int m0, n0;
        origin(done + qd / 4, &m0, &n0);
        gemm8_tile<32, 64, 4>(ra, lda, rb, ldb, C, ldc, M, N, K, m0 + ((qd & 3) >> 1) * 128,
                           n0 + (qd & 1) * 128, smem);
    }
}

}  // namespace regen
