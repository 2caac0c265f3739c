// Cross-attention of regen_attn to a short conditioning context (CDNA4,
// gfx950). A DiT block attends to the conditioning encoders' tokens besides
// its own (blog summary, "Methodology - deep read", names the decoder's CLIP
// and T5 conditioning encoders); with a context of at most kCrossMaxKeys
// tokens the whole context of one head fits in LDS, so each workgroup copies
// it there once and its waves stream query rows against it with no barrier
// between them. Reading Q and writing O from and to HBM is the floor.
#pragma once

#include "attention.hpp"

namespace regen {

constexpr int kCrossMaxKeys = 256;  // longest context held in LDS

// ---------------------------------------------------------------------------
// cross_attn_kernel: grid G, NW * 64 threads.
//   q, o    : bf16, row m of head h at element h * qh + m * qn of q and
//             h * oh + m * on of o (head-major or token-major); Q is not
//             rotated, only scaled by c2 and rounded to bf16
//   k, v    : the Nk <= kCrossMaxKeys context keys and values, bf16, key n
//             of head h at element h * kh + n * kn (not rotated)
//   lse     : [heads][Nq] fp32 log-sum-exp of each row's scores, or null
// A unit is 32 query rows of one head (one wave's share), units numbered
// head-major. Each workgroup takes a contiguous range of units (below): for
// each head in that range it copies the head's context to LDS in the
// Kr / Vt fragment layout of rope_k_vt_kernel, in tiles of 32 keys (K
// gathered by the copies themselves, V copied row by row and transposed in
// LDS), then its waves take the head's units in turn, each unit
// independently: Q to registers (the next unit's Q loads in flight while
// one computes), S^T = K Q^T and online softmax over the key tiles
// exactly as in attn_fwd_kernel, O^T = V^T P^T, O / l stored.
// ---------------------------------------------------------------------------
template <int D, int NW, bool LSE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void cross_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Nq, int Nk, long long qh, long long qn_stride,
    long long kh, long long kn_stride, long long oh, long long on_stride, int heads,
    float c2 /* sm_scale * log2(e) */) {
    static_assert(D == 64 || D == 128, "head_dim");
    constexpr int BN = 32;  // keys per tile
    constexpr int KBYTES = BN * D * 2, VBYTES = D * BN * 2;  // LDS bytes of a K / Vt tile
    constexpr int TBYTES = KBYTES + VBYTES;
    constexpr float kLazy = 8.0f;  // rescale only when the max grows by > 2^8
    __shared__ __attribute__((aligned(1024))) char smem[(kCrossMaxKeys / BN) * TBYTES];

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int upH = (Nq + 31) / 32;  // units per head
    // Workgroup p's units: with at least as many workgroups as heads, head h
    // gets workgroups [h G / heads, (h + 1) G / heads) and each of them an
    // equal share of the head's units, so that no workgroup builds two
    // contexts; with fewer, workgroup p takes whole heads
    // [p heads / G, (p + 1) heads / G). Consecutive workgroups share an XCD.
    const int G = gridDim.x;
    const int pid = xcd_remap(blockIdx.x, G);
    long long u_begin, u_end;
    if (G >= heads) {
        int h = (int)(((long long)pid * heads) / G);
        while (h + 1 < heads && ((long long)(h + 1) * G) / heads <= pid) ++h;
        while (((long long)h * G) / heads > pid) --h;
        const int b0 = (int)(((long long)h * G) / heads), n = (int)(((long long)(h + 1) * G) / heads) - b0;
        u_begin = (long long)h * upH + (long long)upH * (pid - b0) / n;
        u_end = (long long)h * upH + (long long)upH * (pid - b0 + 1) / n;
    } else {
        u_begin = (long long)upH * (((long long)pid * heads) / G);
        u_end = (long long)upH * (((long long)(pid + 1) * heads) / G);
    }
    const int nkv = (Nk + BN - 1) / BN;
    const uint32_t kv_bytes = (uint32_t)(((long long)(Nk - 1) * kn_stride + D) * 2);
    constexpr int NKF = KBYTES / 1024, NVF = VBYTES / 1024;  // 1 KiB fragments per K / Vt tile

    // Every load and store below is a buffer access, issued whether or not
    // its row exists: rows past Nq (and units past the segment) get offsets
    // outside the resource, so loads return zero and stores are dropped
    // without touching memory. The counts of memory operations between two
    // points are then fixed, and each wait below names exactly what it needs.
    constexpr int QL = D / 16;  // Q loads per unit
    // O of a unit goes out through LDS as whole rows when the context leaves
    // room past it for every wave's 32 x D block (head_dim 128: contexts of
    // up to 96 keys), else from the accumulators as 32 bytes of each of the
    // 32 rows per store (store_o_rows), which the memory side takes at a
    // higher cost. Either way a unit's O is D / 16 stores of 16 bytes per lane.
    constexpr int OROW = D * 2 + 16;   // LDS bytes per staged O row (padded)
    constexpr int OBYTES = 32 * OROW;  // a unit's O block in LDS
    constexpr int ST = D / 16 + (LSE ? 1 : 0);  // stores per unit
    static_assert(32 * D * 2 / 1024 == D / 16, "stores per unit on both paths");
    static_assert(NW * OBYTES <= (kCrossMaxKeys / BN) * TBYTES, "O staging area");
    const bool o_lds = nkv * TBYTES + NW * OBYTES <= (kCrossMaxKeys / BN) * TBYTES;  // uniform
    constexpr uint32_t kOut = 0x80000000u;     // past every resource (the host keeps them < 2^31 bytes)
    const uint32_t q_bytes = (uint32_t)(((long long)(Nq - 1) * qn_stride + D) * 2);
    const uint32_t o_bytes = (uint32_t)(((long long)(Nq - 1) * on_stride + D) * 2);
    // This lane's half-row of the Q rows of unit uu (zero past Nq or when
    // uu is not below `end`).
    auto load_q = [&](uint4 (&qr)[D / 16], __amdgpu_buffer_rsrc_t qrs, int h, long long uu, long long end) {
        const int row = (int)(uu - (long long)h * upH) * 32 + col;
        const uint32_t off = (uu < end && row < Nq) ? (uint32_t)(((long long)row * qn_stride + half * 8) * 2) : kOut;
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(qrs, off + kb * 32, 0, 0);
            qr[kb] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    // Q scaled by sm_scale log2(e) and rounded: Q K^T comes out in the exp2
    // domain.
    auto scale_q = [&](const uint4 (&qr)[D / 16], bf16x8 (&qf)[D / 16]) {
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
            const uint32_t src[4] = {qr[kb].x, qr[kb].y, qr[kb].z, qr[kb].w};
            uint32_t dst[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) dst[p] = pack_bf16(bf_lo(src[p]) * c2, bf_hi(src[p]) * c2);
            qf[kb] = __builtin_bit_cast(bf16x8, make_uint4(dst[0], dst[1], dst[2], dst[3]));
        }
    };

    // One unit: 32 query rows of head h against the context in LDS.
    auto unit = [&](const bf16x8 (&qf)[D / 16], __amdgpu_buffer_rsrc_t ors, __amdgpu_buffer_rsrc_t lrs, int h,
                    long long uu) {
        const int qrow = (int)(uu - (long long)h * upH) * 32 + col;
        f32x16 acc[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
        float m_run = 0.0f;  // reference row max (exp2 domain); -m_run seeds S
        f32x16 negm;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = 0.0f;
        float l0 = 0.0f, l1 = 0.0f;  // this lane's partial row sums

        for (int j = 0; j < nkv; ++j) {
            const char* ks = smem + j * TBYTES;
            // Fragments: 0..NK-1 the Kr tile, then the Vt tile, 1 KiB each,
            // lane l's part at 16 l (the layout of rope_k_vt_kernel, for
            // BN-key tiles).
            constexpr int KB = D / 16, NK = (BN / 32) * KB, QB16 = BN / 16, NV = (D / 32) * QB16;
            auto frag = [&](int f) -> bf16x8 {
                return *reinterpret_cast<const bf16x8*>(ks + f * 1024 + lane * 16);
            };
            f32x16 s[BN / 32];
#pragma unroll
            for (int f = 0; f < NK; ++f) {
                const int kk = f % (BN / 32), kb = f / (BN / 32);
                s[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(f), qf[kb], kb == 0 ? negm : s[kk], 0,
                                                                0, 0);
            }
            // Keys past the context get -inf.
            if (j == nkv - 1 && (Nk % BN) != 0) {
#pragma unroll
                for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = j * BN + kk * 32 + (i / 4) * 8 + half * 4 + (i % 4);
                        if (key >= Nk) s[kk][i] = -INFINITY;
                    }
            }
            // Row max: in-lane, then with lane ^ 32.
            float mp[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int i = (kk == 0 ? 4 : 0); i < 16; ++i)
                    mp[i & 3] = __builtin_elementwise_maximum(mp[i & 3], s[kk][i]);
            float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mp[0], mp[1]),
                                                     __builtin_elementwise_maximum(mp[2], mp[3]));
            {
                auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false,
                                                           false);
                mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            // Lazy rescale (see attn_fwd_kernel); tile 0 sets the reference.
            if (j == 0 || mx > kLazy) {
                if (j != 0) {
                    const float alpha = __builtin_amdgcn_exp2f(-mx);
                    l0 *= alpha;
                    l1 *= alpha;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
                }
                m_run += mx;
#pragma unroll
                for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[kk][i] -= mx;
#pragma unroll
                for (int i = 0; i < 16; ++i) negm[i] = -m_run;
            }
            // P = exp2(s) in bf16; the row sum adds the rounded values.
            bf16x8 pk[BN / 16];
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    uint32_t w4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float e0 = __builtin_amdgcn_exp2f(s[kk][hb * 8 + 2 * e]);
                        const float e1 = __builtin_amdgcn_exp2f(s[kk][hb * 8 + 2 * e + 1]);
                        w4[e] = pack_bf16(e0, e1);
                        if (e & 1)
                            l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w4[e]), ones, l1, false);
                        else
                            l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w4[e]), ones, l0, false);
                    }
                    pk[kk * 2 + hb] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
                }
            // O^T += V^T P^T.
#pragma unroll
            for (int g = 0; g < NV; ++g) {
                const int db = g / QB16, kq = g % QB16;
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(NK + g), pk[kq], acc[db], 0, 0, 0);
            }
        }

        // O = O^T / l in bf16; lse = ln 2 (m + log2 l).
        const float l_half = l0 + l1;
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_half), __float_as_uint(l_half), false,
                                                   false);
        const float l_row = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const float inv = 1.0f / l_row;
        if (o_lds) {
            // This wave's block of the LDS area past the context: O written
            // in the accumulator layout (rows padded by 16 bytes, so that the
            // 32 rows of one write spread over the banks while every address
            // stays a lane base plus a constant), read back as whole rows
            // (the wave's LDS accesses complete in order) and stored CPR
            // lanes per row.
            constexpr int CPR = D / 8, RPI = 64 / CPR;
            char* ws = smem + (kCrossMaxKeys / BN) * TBYTES - (NW - wave) * OBYTES;
            char* wl = ws + col * OROW + half * 8;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    uint2 w2;
                    w2.x = pack_bf16(acc[db][g4 * 4 + 0] * inv, acc[db][g4 * 4 + 1] * inv);
                    w2.y = pack_bf16(acc[db][g4 * 4 + 2] * inv, acc[db][g4 * 4 + 3] * inv);
                    *reinterpret_cast<uint2*>(wl + (db * 4 + g4) * 16) = w2;
                }
            const int row0 = qrow - col;
            const char* rl = ws + (lane / CPR) * OROW + (lane % CPR) * 16;
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const int r = k * RPI + lane / CPR, c = lane % CPR;
                const uint4 x = *reinterpret_cast<const uint4*>(rl + k * RPI * OROW);
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 w4 = {x.x, x.y, x.z, x.w};
                const uint32_t off =
                    row0 + r < Nq ? (uint32_t)(((long long)(row0 + r) * on_stride + c * 8) * 2) : kOut;
                __builtin_amdgcn_raw_buffer_store_b128(w4, ors, off, 0, 0);
            }
        } else {
            const uint32_t ooff = qrow < Nq ? (uint32_t)((long long)qrow * on_stride * 2) : kOut;
            store_o_rows<D>(acc, inv, half, [&](int d0, uint4 w) {
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 w4 = {w.x, w.y, w.z, w.w};
                __builtin_amdgcn_raw_buffer_store_b128(w4, ors, ooff + d0 * 2, 0, 0);
            });
        }
        if (LSE) {
            const uint32_t loff = (qrow < Nq && half == 0) ? (uint32_t)qrow * 4 : kOut;
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint((m_run + log2f(l_row)) * 0.69314718055994531f), lrs, loff, 0, 0);
        }
    };

    for (long long u0 = u_begin; u0 < u_end;) {
        const int h = (int)(u0 / upH);
        const long long seg_end = min(u_end, (long long)(h + 1) * upH);
        // Head h's context: tile j's Kr at byte j * TBYTES, its Vt after it.
        // Every wave must be done with the previous head's before it goes.
        if (u0 != u_begin) __syncthreads();
        {
            // Keys past Nk have offsets past the resources: they read as zero.
            const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + h * kh, kv_bytes);
            const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + h * kh, kv_bytes);
            // Kr fragment f = (BN / 32) kb + kk of tile j, straight from the
            // rows: lane (c, g) gets key BN j + 32 kk + c, head dims
            // 16 kb + 8 g ..
            for (int F = wave; F < nkv * NKF; F += NW) {
                const int j = F / NKF, f = F % NKF;
                const int key = j * BN + (f % (BN / 32)) * 32 + col;
                g2lds16(krs, (uint32_t)(((long long)key * kn_stride + (f / (BN / 32)) * 16 + half * 8) * 2),
                        smem + j * TBYTES + f * 1024);
            }
            // V rows as they are into tile j's Vt area (row r at byte 2 D r),
            // transposed in place below.
            for (int R = wave; R < nkv * NVF; R += NW) {
                const int j = R / NVF, p = (R % NVF) * 64 + lane;  // 16-byte chunk p of the tile
                const int key = j * BN + p / (D / 8);
                g2lds16(vrs, (uint32_t)(((long long)key * kn_stride + (p % (D / 8)) * 8) * 2),
                        smem + j * TBYTES + KBYTES + (R % NVF) * 1024);
            }
        }
        // This wave's units u0 + wave + i NW, one ahead: the next unit's Q
        // loads go out as soon as a unit's Q is in registers, so the stores
        // of the first units overlap the loads of the later ones (requesting
        // two units' Q up front had every wave's loads ahead of any store).
        // The first unit's loads go out behind the context copies, whose wait
        // leaves them outstanding (the counter retires in issue order).
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + h * qh, q_bytes);
        const __amdgpu_buffer_rsrc_t ors = make_rsrc(o + h * oh, o_bytes);
        const __amdgpu_buffer_rsrc_t lrs =
            make_rsrc(LSE ? static_cast<const void*>(lse + (size_t)h * Nq) : static_cast<const void*>(o),
                      LSE ? (uint32_t)Nq * 4 : 0u);
        long long u = u0 + wave;
        uint4 qa[D / 16], qb[D / 16];
        load_q(qa, qrs, h, u, seg_end);
        __builtin_amdgcn_s_waitcnt(vmcnt_only(QL));
        __syncthreads();
        // Vt fragment 4 db + kq of tile j from the raw rows: lane (c, g)
        // holds head dim 32 db + c of the keys in slots 8 g .. 8 g + 7 of key
        // group kq, slot 8 g + i holding key 16 kq + 8 (i / 4) + 4 g + i % 4
        // of the tile (the P^T operand order). Tile by tile, every read of a
        // tile's rows before any write of its fragments.
        for (int j = 0; j < nkv; ++j) {
            constexpr int PER = (NVF + NW - 1) / NW;  // fragments of a tile per wave, at most
            char* vt_tile = smem + j * TBYTES + KBYTES;
            uint4 vf[PER];
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int g4 = i * NW + wave, kq = g4 % (BN / 16);
                if (g4 >= NVF) break;
                const char* raw = vt_tile + ((g4 / (BN / 16)) * 32 + col) * 2;
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k0 = kq * 16 + (e / 2) * 8 + half * 4 + (e % 2) * 2;
                    const uint32_t lo = *reinterpret_cast<const uint16_t*>(raw + k0 * 2 * D);
                    const uint32_t hi = *reinterpret_cast<const uint16_t*>(raw + (k0 + 1) * 2 * D);
                    w[e] = lo | (hi << 16);
                }
                vf[i] = make_uint4(w[0], w[1], w[2], w[3]);
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (i * NW + wave < NVF)
                    *reinterpret_cast<uint4*>(vt_tile + (i * NW + wave) * 1024 + lane * 16) = vf[i];
        }
        __syncthreads();

        // Outstanding operations (oldest first) at each wait: behind qa, the
        // last pass's stores of B (none on the first pass, whose context
        // copies were awaited above); behind qb, A's stores.
        bool first = true;
        for (; u < seg_end; u += 2 * NW) {
            bf16x8 qf[D / 16];
            if (first) __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            else __builtin_amdgcn_s_waitcnt(vmcnt_only(ST));
            scale_q(qa, qf);
            load_q(qb, qrs, h, u + NW, seg_end);
            unit(qf, ors, lrs, h, u);
            if (u + NW >= seg_end) break;
            __builtin_amdgcn_s_waitcnt(vmcnt_only(ST));
            scale_q(qb, qf);
            load_q(qa, qrs, h, u + 2 * NW, seg_end);
            unit(qf, ors, lrs, h, u + NW);
            first = false;
        }
        u0 = seg_end;
    }
}

}  // namespace regen
