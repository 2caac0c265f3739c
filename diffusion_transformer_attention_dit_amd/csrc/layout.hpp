// The on-device half of a Ulysses all-to-all for regen_attn (CDNA4, gfx950).
#pragma once

#include "common.hpp"

namespace regen {

// ---------------------------------------------------------------------------
// block_transpose_kernel: the on-device half of a Ulysses all-to-all (blog summary,
// "Methodology - deep read", USP paragraph: Ulysses turns sequence shards
// into head shards). A block transpose src [A][B][E] -> dst [B][A][E] of
// E-byte blocks, 16 bytes per thread, writes in destination order:
//   pack   [Nl][G][H/G][D] -> [G][Nl][H/G][D]  (A = Nl, B = G)
//   unpack [G][Nl][H/G][D] -> [Nl][G][H/G][D]  (A = G, B = Nl)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void block_transpose_kernel(const uint4* __restrict__ src,
                                                              uint4* __restrict__ dst, long long A,
                                                              long long B, long long E16) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= A * B * E16) return;
    const long long e = i % E16, ba = i / E16;
    const long long a = ba % A, b = ba / A;
    dst[i] = src[(a * B + b) * E16 + e];
}

}  // namespace regen
