// A measurement aid of regen_attn (CDNA4, gfx950): the GPU core clock while
// every SIMD runs back-to-back bf16 MFMAs, the load the attention kernel puts
// on the chip. Kernel times divided into flops give TFLOP/s; to compare a
// kernel with the MFMA peak of the clock the chip actually ran at (the peak
// 256 CU x 4096 flop/clk x 2.4 GHz assumes the top clock) one needs that
// clock, which varies from machine to machine under this load.
#pragma once

#include "common.hpp"

namespace regen {

// clock_probe_kernel: grid = one workgroup of 8 waves per CU (two waves per
// SIMD, as in attn_fwd_kernel). Every wave runs `iters` rounds of four
// independent v_mfma_f32_32x32x16_bf16; wave 0 of workgroup 0 reads the core
// cycle counter (s_memtime) and the constant-rate counter around its loop:
// out[0..1] = cycles at start / end, out[2..3] = constant-rate ticks at
// start / end. out[4] is written only if the accumulators sum to an
// impossible value (keeps the MFMAs from being optimised away).
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void clock_probe_kernel(
    long long* __restrict__ out, int iters, float seed) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(lane + i));
        b[i] = (__bf16)(seed * (float)(lane - i));
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    __syncthreads();
    const long long t0 = __clock64(), w0 = wall_clock64();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    // The counters are read once the last MFMA has finished.
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    const long long t1 = __clock64(), w1 = wall_clock64();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        out[0] = t0;
        out[1] = t1;
        out[2] = w0;
        out[3] = w1;
    }
    if (s == 1234567.0f) out[4] = 1;
}

}  // namespace regen
