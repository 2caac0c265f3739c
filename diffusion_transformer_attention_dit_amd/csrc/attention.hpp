// The attention kernels of regen_attn for CDNA4 (gfx950). One attention
// call runs the first two, and the third when the schedule split tiles:
//
//  1. rope_k_vt_kernel (HBM-bound pass over K and V): applies the 3D rotary
//     embedding to K and rounds it to bf16 into Kr, and writes V transposed
//     into Vt. Both are stored as the MFMA operand fragments the attention
//     kernel reads, in lane order, so that a tile is copied to LDS as
//     contiguous 1 KiB runs and every operand read is one LDS address plus a
//     constant.
//  2. attn_fwd_kernel (MFMA-bound): flash-style exact attention, persistent
//     (one round of resident workgroups, see Sched). Each wave owns 32 query
//     rows, rotates its Q rows while loading them (RoPE on load), then
//     streams K/V blocks through double-buffered LDS and keeps the online
//     softmax (running max, running sum) in registers.
//  3. merge_kernel: finishes query tiles whose key blocks were split over
//     several workgroups.
// merge_parts_kernel combines results over disjoint key sets (the Ring
// step).
//
// The attention is the one ReGenVC's decoder transformer evaluates over the
// window's latent tokens (arXiv 2607.28144, blog summary "Methodology - deep
// read", USP paragraph), kept exact as "Technical innovations" requires; the
// blocked, online-softmax evaluation follows FlashAttention/FlashAttention-2
// (index page, "Builds on") but is laid out here for 64-lane wavefronts and
// 32x32x16 bf16 MFMA.
//
// Attention is computed transposed, S^T = K Q^T, so that a lane's results
// all belong to ONE query (its column c in the MFMA layout of common.hpp)
// and 16 keys: the row max and row
// sum are in-lane reductions plus one exchange with lane l ^ 32
// (v_permlane32_swap), and the O^T = V^T P^T product consumes the
// probabilities straight from registers as its B operand. The key order that
// the B operand then implies (slot 8g + j <-> key 8(j/4) + 4g + j%4 inside
// each group of 16) is baked into Vt by rope_k_vt_kernel.
#pragma once

#include "common.hpp"

namespace regen {

constexpr int kPrepKeys = 128;  // workspace padding unit (keys)
constexpr int kPrepBlock = 64;  // keys per rope_k_vt block: one Kr / Vt tile
constexpr int kPrepDims = 64;   // head dims per rope_k_vt block (32: 15% slower at 12 x 10920)
constexpr int kTabLds = 3072;   // (cos, sin) entries the attention kernel keeps in LDS

// Rotary geometry: latent grid, pairs per axis, offsets of each axis' table
// in the (cos, sin) table. Entry off[a] + pos * pairs[a] + j holds
// (cos, sin) of pos * base^(-j / pairs[a]).
struct RopeGeom {
    int T, H, W;
    int pairs[3];
    int off[3];
};

// (cos, sin) for rotary pair i of a token at (t, h, w).
__device__ __forceinline__ float2 rope_cs(const float2* __restrict__ tab, const RopeGeom& g,
                                          int i, int t, int h, int w) {
    int idx;
    if (i < g.pairs[0]) {
        idx = g.off[0] + t * g.pairs[0] + i;
    } else if (i < g.pairs[0] + g.pairs[1]) {
        idx = g.off[1] + h * g.pairs[1] + (i - g.pairs[0]);
    } else {
        idx = g.off[2] + w * g.pairs[2] + (i - g.pairs[0] - g.pairs[1]);
    }
    return tab[idx];
}

// rope_table_kernel: the (cos, sin) table of geometry g, computed on the
// device in fp64 and stored as fp32: entry off[a] + pos * pairs[a] + j holds
// the angle pos * base^(-j / pairs[a]) of pair j of axis a (every angle 0
// when rope == 0). Grid ceil(entries / 256), 256 threads.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, RopeGeom g, double base,
                                                        int rope, int entries) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= entries) return;
    const int a = i < g.off[1] ? 0 : (i < g.off[2] ? 1 : 2);
    const int r = i - g.off[a], pos = r / g.pairs[a], j = r % g.pairs[a];
    const double theta = pow(base, -double(j) / double(g.pairs[a]));
    const double phi = double(pos) * theta;
    tab[i] = rope ? make_float2(float(cos(phi)), float(sin(phi))) : make_float2(1.0f, 0.0f);
}

// Rotate the 4 pairs held in one 16-byte chunk (8 bf16, pairs i0..i0+3),
// scale by `mul` and round to bf16.
__device__ __forceinline__ uint4 rope_chunk(uint4 in, const float2* __restrict__ tab,
                                            const RopeGeom& g, int i0, int t, int h, int w,
                                            float mul = 1.0f) {
    uint32_t src[4] = {in.x, in.y, in.z, in.w};
    uint32_t dst[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float2 cs = rope_cs(tab, g, i0 + p, t, h, w);
        float x = bf_lo(src[p]), y = bf_hi(src[p]);
        float xr = x * cs.x - y * cs.y;
        float yr = x * cs.y + y * cs.x;
        dst[p] = pack_bf16(xr * mul, yr * mul);
    }
    return make_uint4(dst[0], dst[1], dst[2], dst[3]);
}

// ---------------------------------------------------------------------------
// rope_k_vt_kernel: K rotation + V transpose. Grid (Npad / 64, heads, D / 64),
// 256 threads.
//   k, v : bf16, key n of head h at element h * sh + n * sn (head-major
//          [heads][N][D]: sh = N D, sn = D; token-major [N][heads][D]:
//          sh = D, sn = heads D), key n being token n_off + n of the grid.
//   Kr, Vt : [heads][Npad/64] tiles of 64 keys, 64 D bf16 each, a tile
//        being a run of 1 KiB MFMA A-operand fragments; lane l = 32 g + c of
//        a fragment holds bytes 16 l .. 16 l + 15:
//        Kr fragment f = 2 kb + kk: key 32 kk + c of the tile, head dims
//          16 kb + 8 g .. + 7, rotated;
//        Vt fragment 4 db + kq: head dim 32 db + c of the 8 keys in slots
//          8 g .. 8 g + 7 of the tile's key group kq (16 keys), slot 8 g + j
//          holding key 8 (j / 4) + 4 g + j % 4 of the group.
//        Keys >= N are zero.
// ---------------------------------------------------------------------------
// NT: the Kr / Vt stores are nontemporal (whole lines). For a short call
// (few blocks per CU) that made the pass 15% faster; for a long one 8%
// slower, so the host picks it by grid size.
template <int D, bool NT = false>
__global__ __launch_bounds__(256) void rope_k_vt_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ kr,
    uint16_t* __restrict__ vt, const float2* __restrict__ tab, RopeGeom geo, int N, int Npad,
    int n_off, long long sh, long long sn, int* __restrict__ cnt) {
    const int hd = blockIdx.y;
    // The attention kernel that follows on the stream claims leftover
    // pieces from this counter.
    if (cnt != nullptr && (blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) *cnt = 0;
    const int n0 = blockIdx.x * kPrepBlock;
    const int z = blockIdx.z;  // head dims kPrepDims z .. of the tile
    const int HW = geo.H * geo.W;

    // Rows are staged through LDS so that both the reads of K and V (whole
    // 128-byte row halves) and the writes of Kr and Vt (whole 1 KiB
    // fragments) are contiguous. LDS rows are XOR-swizzled by 16-byte chunk.
    // A block takes 64 of the head dims: the Kr fragments of 16-dim blocks
    // 4 z .. 4 z + 3 and the Vt fragments of 32-dim blocks 2 z, 2 z + 1 are
    // the tile's fragments 8 z .. 8 z + 7 of each, so the grid has D / 64
    // blocks per tile and twice as many blocks reach the memory system at
    // D = 128 (a short call, such as three heads, does not fill the chip
    // with one block per tile).
    constexpr int DH = kPrepDims;         // head dims per block
    constexpr int CPR = DH / 8;           // 16-byte chunks per staged row
    constexpr int PER = kPrepBlock * CPR / 256;
    constexpr int NF = DH / 8;            // 1 KiB fragments of Kr (and of Vt) per block
    static_assert(D % DH == 0 && NF * 64 == PER * 256, "fragments per block");
    __shared__ uint4 kl[kPrepBlock * CPR];
    __shared__ uint4 vl[kPrepBlock * CPR];
    const int tid = threadIdx.x;
    auto sw = [](int r, int c) { return r * CPR + (c ^ (r & (CPR - 1))); };

    uint4 kin[PER], vin[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int cid = i * 256 + tid, r = cid / CPR, c = z * CPR + cid % CPR, n = n0 + r;
        kin[i] = make_uint4(0, 0, 0, 0);
        vin[i] = make_uint4(0, 0, 0, 0);
        if (n < N) {
            kin[i] = *reinterpret_cast<const uint4*>(k + hd * sh + n * sn + c * 8);
            vin[i] = *reinterpret_cast<const uint4*>(v + hd * sh + n * sn + c * 8);
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int cid = i * 256 + tid, r = cid / CPR, cl = cid % CPR, n = n0 + r;
        uint4 out = make_uint4(0, 0, 0, 0);
        if (n < N) {
            const int ng = n_off + n;  // token index on the grid
            const int t = ng / HW, h = (ng / geo.W) % geo.H, w = ng % geo.W;
            out = rope_chunk(kin[i], tab, geo, (z * CPR + cl) * 4, t, h, w);
        }
        kl[sw(r, cl)] = out;
        vl[sw(r, cl)] = vin[i];
    }
    __syncthreads();

    // Tile fragment 8 z + F of Kr (f = 2 kb + kk): lane (c, g) holds key
    // 32 kk + c, head dims 16 kb + 8 g .. + 7. Tile fragment 8 z + F of Vt
    // (4 db + kq): lane (c, g) holds head dim 32 db + c of the keys in slots
    // 8 g .. 8 g + 7 of key group kq.
    const int lane = tid & 63, c = lane & 31, g = lane >> 5;
    uint16_t* kdst = kr + ((size_t)hd * Npad + n0) * D + z * NF * 512;
    uint16_t* vdst = vt + ((size_t)hd * Npad + n0) * D + z * NF * 512;
    const uint16_t* vl16 = reinterpret_cast<const uint16_t*>(vl);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int F = i * 4 + (tid >> 6);
        {
            const int r = (F % 2) * 32 + c;
            const uint4 kv = kl[sw(r, (F / 2) * 2 + g)];
            if constexpr (NT) {
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 kn = {kv.x, kv.y, kv.z, kv.w};
                __builtin_nontemporal_store(kn, reinterpret_cast<u32x4*>(kdst + F * 512 + lane * 8));
            } else {
                *reinterpret_cast<uint4*>(kdst + F * 512 + lane * 8) = kv;
            }
        }
        {
            const int dl = (F / 4) * 32 + c;  // head dim 64 z + dl
            const int rb = (F % 4) * 16 + 4 * g;
            uint32_t w4[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r0 = rb + (m / 2) * 8 + (m % 2) * 2, r1 = r0 + 1;
                const uint32_t lo = vl16[sw(r0, dl >> 3) * 8 + (dl & 7)];
                const uint32_t hi = vl16[sw(r1, dl >> 3) * 8 + (dl & 7)];
                w4[m] = lo | (hi << 16);
            }
            if constexpr (NT) {
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 vn = {w4[0], w4[1], w4[2], w4[3]};
                __builtin_nontemporal_store(vn, reinterpret_cast<u32x4*>(vdst + F * 512 + lane * 8));
            } else {
                *reinterpret_cast<uint4*>(vdst + F * 512 + lane * 8) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            }
        }
    }
}

// Rows of O from the P V accumulators of one wave: acc[db] holds O^T for 32
// head dims x 32 rows, lane (col, half) having row col's head dims
// 32 db + 8 g + 4 half .. + 3 (g < 4). Each pair of 8-dim chunks (2 gp,
// 2 gp + 1) is exchanged with lane ^ 32 (two v_permlane32_swap), so that
// lane (col, half) ends up with all 8 dims of chunk 2 gp + 1 - half and
// stores 16 bytes: a store instruction writes 32 contiguous bytes of each of
// the 32 rows rather than 16, which the memory side takes at less cost.
// put(d0, w) stores the 16 bytes w at head dim d0 of this lane's row; every
// lane of the wave must take part (the swaps read lane ^ 32).
template <int D, typename Put>
__device__ __forceinline__ void store_o_rows(const f32x16 (&acc)[D / 32], float scale, int half, Put&& put) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            const int g = 2 * gp;
            const uint32_t a0 = pack_bf16(acc[db][g * 4 + 0] * scale, acc[db][g * 4 + 1] * scale);
            const uint32_t a1 = pack_bf16(acc[db][g * 4 + 2] * scale, acc[db][g * 4 + 3] * scale);
            const uint32_t b0 = pack_bf16(acc[db][g * 4 + 4] * scale, acc[db][g * 4 + 5] * scale);
            const uint32_t b1 = pack_bf16(acc[db][g * 4 + 6] * scale, acc[db][g * 4 + 7] * scale);
            // [0]: b with lanes 32.. taken from a of lanes ..31; [1]: a with
            // lanes ..31 taken from b of lanes 32..
            const auto s0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
            put(db * 32 + (g + 1 - half) * 8, make_uint4(s0[0], s1[0], s0[1], s1[1]));
        }
}

// Issue the copies of K tile j and Vt tile j into LDS buffer (ks, vs). Both
// are stored in HBM as runs of 1 KiB MFMA operand fragments in lane order,
// which land unchanged in LDS: run r of a tile goes to byte 1024 r of the
// buffer, every wave copying RUNS / NW whole runs of each.
template <int D, int BN, int NW>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                           int j, char* ks, char* vs, int wave, int lane) {
    constexpr int RUNS = BN * D * 2 / 1024;  // 1 KiB runs per tile (same for K and V)
    static_assert(RUNS % NW == 0, "runs per wave");
    const uint32_t tile_off = (uint32_t)j * (RUNS * 1024);
#pragma unroll
    for (int i = 0; i < RUNS / NW; ++i) {
        const int run = i * NW + wave;
        const uint32_t voff = (uint32_t)(run * 1024 + lane * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            krs, (__attribute__((address_space(3))) void*)(ks + run * 1024), 16, voff, tile_off, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vrs, (__attribute__((address_space(3))) void*)(vs + run * 1024), 16, voff, tile_off, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// Work schedule. A "unit" is one (query tile, key block) pair: query tile t
// (BM = 32 NW rows of one head; tiles numbered head-major) against key
// block b (BN keys); unit index x = t * nkv + b. P persistent workgroups
// (one full round of resident slots) first make `full` passes over whole
// tiles, pass i giving tile i * P + p to workgroup p, so the workgroups that
// share an XCD sweep the same head's keys together. The `rem` leftover
// tiles (tiles >= full * P) are then cut stream-K style: their units are
// split into Prem = min(P, leftover units) equal contiguous ranges, one per
// workgroup p < Prem, so every slot ends with the same amount of work and no
// range is empty. A leftover tile whose units span several workgroups is
// finished by the merge kernel from the per-workgroup partial results
// (unnormalised O, running max m, row sum l), combined exactly as in
// blockwise softmax.
// ---------------------------------------------------------------------------
struct Sched {
    int n_qtiles;   // query tiles per head
    int nkv;        // key blocks per tile
    int P;          // persistent workgroups
    int full;       // whole-tile passes
    int Prem;       // workgroups sharing the leftover units, >= 1
    int rem_units;  // units of the leftover tiles (rem * nkv)
    int rem_q;      // rem_units / Prem
    int rem_r;      // rem_units % Prem
    int dyn;        // leftover tiles cut into pieces claimed at run time (below)
    int ppt;        // pieces per leftover tile (dyn)
    int npieces;    // leftover tiles x ppt (dyn)
};
// With dyn, the leftover tiles are not split statically: piece i (of tile
// full P + i / ppt, key blocks [j nkv / ppt, (j + 1) nkv / ppt) for
// j = i % ppt) goes to whichever workgroup claims it next from a counter,
// near the end of its whole tiles. The XCDs of one GPU run at different
// clocks, so the workgroups of the fast ones take the pieces while the slow
// ones finish their tiles. Every piece writes partial slot i and the merge
// folds a tile's pieces in order, so the result does not depend on which
// workgroup took which piece.
__host__ __device__ __forceinline__ void piece_segment(const Sched& sc, int i, int* t, int* kv0, int* kv1) {
    const int r = i / sc.ppt, j = i - r * sc.ppt;
    *t = sc.full * sc.P + r;
    *kv0 = (j * sc.nkv) / sc.ppt;
    *kv1 = ((j + 1) * sc.nkv) / sc.ppt;
}
// Every unit index (heads * n_qtiles * nkv) fits in 31 bits (the host checks
// this), so the schedule runs in 32-bit integer arithmetic.

// Start (offset into the leftover units) of workgroup p's leftover range,
// p <= Prem: floor(p * rem_units / Prem), split so that no product leaves
// 32 bits (p * rem_q <= rem_units, p * rem_r < Prem^2). Ranges are non-empty
// because rem_units >= Prem.
__host__ __device__ __forceinline__ int rem_begin(const Sched& sc, int p) {
    return p * sc.rem_q + (p * sc.rem_r) / sc.Prem;
}
// The workgroup whose leftover range holds leftover unit y (the largest p
// with rem_begin(p) <= y). Used by the merge only; 64-bit products.
__host__ __device__ __forceinline__ int rem_owner(const Sched& sc, int y) {
    return (int)(((long long)(y + 1) * sc.Prem - 1) / sc.rem_units);
}
// Partial-result slot of workgroup p for leftover tile t: the first tile of
// its range uses 2p, a later (necessarily its last) tile uses 2p + 1.
__host__ __device__ __forceinline__ int partial_slot(const Sched& sc, int p, int t) {
    const int x0 = sc.full * sc.P * sc.nkv + rem_begin(sc, p);
    return (t == x0 / sc.nkv) ? 2 * p : 2 * p + 1;
}

// Segment k of workgroup p's work: tile *t, key blocks [*kv0, *kv1).
// Returns false past the last segment.
__host__ __device__ __forceinline__ bool get_segment(const Sched& sc, int p, int k, int* t, int* kv0,
                                                     int* kv1) {
    if (k < sc.full) {
        *t = k * sc.P + p;
        *kv0 = 0;
        *kv1 = sc.nkv;
        return true;
    }
    if (sc.dyn || p >= sc.Prem) return false;
    const int base = sc.full * sc.P * sc.nkv;
    const int a = base + rem_begin(sc, p), b = base + rem_begin(sc, p + 1);
    const int x = (k == sc.full) ? a : (a / sc.nkv + (k - sc.full)) * sc.nkv;
    if (x >= b) return false;
    *t = x / sc.nkv;
    *kv0 = x - *t * sc.nkv;
    const int left = b - x;
    *kv1 = (left < sc.nkv - *kv0) ? *kv0 + left : sc.nkv;
    return true;
}

// ---------------------------------------------------------------------------
// attn_fwd_kernel: attention, persistent. Grid P, NW * 64 threads.
//   q, o    : bf16, row m of head h at element h * qh + m * qn of q and
//             h * oh + m * on of o (head-major, token-major or a strided
//             token-major view), row m being token q_off + m
//   Kr, Vt  : the Nk keys prepared by rope_k_vt_kernel (Npad rows per head)
//   lse     : [heads][Nq] fp32 log-sum-exp of each row's scores, or null
//   part_o  : [2P][BM][D] bf16 O / l of split tiles (normalised over the
//             segment's own keys)
//   part_ml : [2P][BM][2] fp32 (m, l) of split tiles
//   cnt     : with sc.dyn, the piece counter, zero at entry
// ---------------------------------------------------------------------------
template <int D, int BN, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vt, uint16_t* __restrict__ o, float* __restrict__ lse,
    const float2* __restrict__ tab, RopeGeom geo, int Nq, int Nk, int Npad, int q_off,
    long long qh, long long qn_stride, long long oh, long long on_stride, Sched sc,
    float c2 /* sm_scale * log2(e) */, int rotate_q, uint16_t* __restrict__ part_o,
    float* __restrict__ part_ml, int* __restrict__ cnt) {
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(BN == 64, "key tile: the Kr / Vt fragment layout holds 64-key tiles");
    constexpr int BM = NW * 32;
    constexpr int KBYTES = BN * D * 2, VBYTES = D * BN * 2;  // LDS bytes of a K / Vt tile
    constexpr float kLazy = 8.0f;  // rescale only when the max grows by > 2^8

    __shared__ __attribute__((aligned(1024))) char smem[2 * (KBYTES + VBYTES)];
    // The next segment's Q rows, copied during the current segment: row r at
    // byte r * 2 D, 16-byte chunk c stored at position c ^ (r % (D / 8)).
    __shared__ __attribute__((aligned(1024))) char qsm[BM * D * 2];
    // The (cos, sin) table, when it fits: Q rows are rotated from LDS, with no
    // global load waiting behind the K / V copies in flight.
    __shared__ float2 tabsm[kTabLds];
    __shared__ int claimed;  // the piece a workgroup claimed for its next segment

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;

    // Consecutive logical workgroups (hence consecutive tiles of one head)
    // share an XCD and its L2.
    const int pid = xcd_remap(blockIdx.x, gridDim.x);
    int t, kv0, kv1;
    if (!get_segment(sc, pid, 0, &t, &kv0, &kv1)) return;  // uniform; no barrier reached yet

    const uint32_t head_bytes = (uint32_t)Npad * D * 2;
    const int HW = geo.H * geo.W;
    const int tab_n = geo.off[2] + geo.W * geo.pairs[2];  // table entries
    const bool tab_lds = rotate_q && tab_n <= kTabLds;    // uniform
    if (tab_lds)  // read after the barrier before the first segment's Q
        for (int i = tid; i < tab_n; i += NW * 64) tabsm[i] = tab[i];

    // Buffer resources over the Kr rows and Vt blocks of tile tt's head.
    auto head_rsrc = [&](int tt, __amdgpu_buffer_rsrc_t* krs, __amdgpu_buffer_rsrc_t* vrs) {
        const int h = tt / sc.n_qtiles;
        *krs = make_rsrc(kr + (size_t)h * Npad * D, head_bytes);
        *vrs = make_rsrc(vt + (size_t)h * Npad * D, head_bytes);
    };
    // Copies of the BM Q rows of tile tt into qsm (this wave's share of the
    // 1 KiB runs). The resource covers the tile's rows below Nq only, so
    // rows past the end read as zero. Used when a tile's rows span < 2^31
    // bytes (uniform).
    constexpr int QCPR = D / 8;  // 16-byte chunks per Q row
    const bool q_lds = (long long)qn_stride * 2 * BM < (1LL << 31);
    auto issue_q = [&](int tt) {
        const int h = tt / sc.n_qtiles, qtt = tt - h * sc.n_qtiles;
        const int rows = min(BM, Nq - qtt * BM);
        const __amdgpu_buffer_rsrc_t qrs =
            make_rsrc(q + h * qh + (long long)qtt * BM * qn_stride,
                      (uint32_t)(((long long)(rows - 1) * qn_stride + D) * 2));
        constexpr int RUNS = BM * D * 2 / 1024;
        static_assert(RUNS % NW == 0, "Q runs per wave");
#pragma unroll
        for (int i = 0; i < RUNS / NW; ++i) {
            const int run = i * NW + wave;
            const int p = run * 64 + lane;  // chunk position in qsm
            const int r = p / QCPR, c = (p % QCPR) ^ (r % QCPR);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                qrs, (__attribute__((address_space(3))) void*)(qsm + run * 1024), 16,
                (uint32_t)(((long long)r * qn_stride + c * 8) * 2), 0, 0, 0);
        }
    };

    __amdgpu_buffer_rsrc_t krs, vrs;
    head_rsrc(t, &krs, &vrs);
    if (q_lds) issue_q(t);
    issue_tile<D, BN, NW>(krs, vrs, kv0, smem, smem + KBYTES, wave, lane);
    int buf = 0;
    bool more = true;

    int piece = -1;  // the current segment's piece (dyn leftover), else -1
    for (int k = 0; more; ++k) {
        // ---- segment k: tile t, key blocks [kv0, kv1) ----
        int nt_ = 0, nkv0 = 0, nkv1 = 0, npiece = -1;
        // The next segment is a claimed piece: it is claimed once this one's
        // key blocks are done (below), so the claim reflects how far this
        // workgroup actually got.
        const bool next_dyn = sc.dyn && k + 1 >= sc.full;  // uniform
        more = next_dyn ? false : get_segment(sc, pid, k + 1, &nt_, &nkv0, &nkv1);
        __amdgpu_buffer_rsrc_t nkrs = krs, nvrs = vrs;  // the next segment's head
        if (more) head_rsrc(nt_, &nkrs, &nvrs);
        const int hd = t / sc.n_qtiles, qt = t - hd * sc.n_qtiles;
        const int qrow = qt * BM + wave * 32 + col;

        // Q: load this lane's half-rows, rotate them (RoPE on load) and fold
        // in the softmax scale and log2(e), so that Q K^T comes out in the
        // exp2 domain.
        if (k == 0) {  // the first tile's Q rows, the table and the first K / V tile
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        bf16x8 qf[D / 16];
        {
            const int qn = qrow < Nq ? qrow : 0;
            const int qg = q_off + qn;  // token index on the grid
            const int tt = qg / HW, hh = (qg / geo.W) % geo.H, ww = qg % geo.W;
            const int lr = wave * 32 + col;
            char* qrow_sm = qsm + lr * D * 2;
            if (!q_lds) {
                // Rows too far apart for one buffer resource: each wave
                // stages its own rows (zero past the end) into the same LDS
                // layout; the wave's LDS accesses complete in order.
                const uint16_t* qp = q + hd * qh + (long long)qn * qn_stride + half * 8;
#pragma unroll
                for (int kb = 0; kb < D / 16; ++kb) {
                    const uint4 x = qrow < Nq ? *reinterpret_cast<const uint4*>(qp + kb * 16) : make_uint4(0, 0, 0, 0);
                    *reinterpret_cast<uint4*>(qrow_sm + ((kb * 2 + half) ^ (lr % QCPR)) * 16) = x;
                }
            }
            // Every chunk is requested before any is used; rows past the end
            // are zero in LDS.
            uint4 xq[D / 16];
#pragma unroll
            for (int kb = 0; kb < D / 16; ++kb)
                xq[kb] = *reinterpret_cast<const uint4*>(qrow_sm + ((kb * 2 + half) ^ (lr % QCPR)) * 16);
            // One instance per table location, so that the LDS one reads
            // through LDS addresses (a generic pointer would wait on every
            // outstanding global copy too).
            auto rotate = [&](const float2* tb) {
#pragma unroll
                for (int kb = 0; kb < D / 16; ++kb)
                    qf[kb] = __builtin_bit_cast(bf16x8, rope_chunk(xq[kb], tb, geo, kb * 8 + half * 4, tt, hh, ww, c2));
            };
            if (tab_lds) {
                rotate(tabsm);
            } else if (rotate_q) {
                rotate(tab);
            } else {  // unrotated (cross-attention): scale and round only
#pragma unroll
                for (int kb = 0; kb < D / 16; ++kb) {
                    const uint32_t src[4] = {xq[kb].x, xq[kb].y, xq[kb].z, xq[kb].w};
                    uint32_t dst[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) dst[p] = pack_bf16(bf_lo(src[p]) * c2, bf_hi(src[p]) * c2);
                    qf[kb] = __builtin_bit_cast(bf16x8, make_uint4(dst[0], dst[1], dst[2], dst[3]));
                }
            }
        }

        f32x16 acc[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
        // Running reference value of the row max (exp2 domain); -m_run fills
        // every slot of negm, the accumulator input of each key block's first
        // S MFMA, so the products come out already shifted: s = S - m_run.
        float m_run = 0.0f;
        f32x16 negm;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = 0.0f;
        float l0 = 0.0f, l1 = 0.0f;  // this lane's partial row sums

        for (int b = kv0; b < kv1; ++b) {
            const char* ks = smem + buf * (KBYTES + VBYTES);
            // The next segment's Q rows, once every wave has read this
            // segment's (the first block's barrier); they land with this
            // block's copies.
            if (q_lds && more && b == kv0 + 1) issue_q(nt_);
            {
                char* nks = smem + (buf ^ 1) * (KBYTES + VBYTES);
                if (b + 1 < kv1)
                    issue_tile<D, BN, NW>(krs, vrs, b + 1, nks, nks + KBYTES, wave, lane);
                else if (more)
                    issue_tile<D, BN, NW>(nkrs, nvrs, nkv0, nks, nks + KBYTES, wave, lane);
            }

            // MFMA A operands come from LDS through a ring of RING fragments
            // read ahead of their use; fragment f sits at byte 1024 f of the
            // buffer, lane l's part at 16 l. Fragments 0..NK-1 are the K tile
            // (head-dim block kb major, key block kk minor, so consecutive S
            // MFMAs feed different accumulators), NK..NK+NV-1 the Vt tile
            // (head-dim block db, key block kq). LDS read bandwidth is close to what the
            // S products need while all waves run them at once, so the first
            // Vt fragments are requested after the S products, to land during
            // the softmax.
            constexpr int KB = D / 16, NK = (BN / 32) * KB, QB16 = BN / 16, NV = (D / 32) * QB16;
            constexpr int RING = 8, DB = D / 32;
            // The P V products run key group by key group (c = kq DB + db), so
            // that each group's P is needed only by its own DB products.
            auto vfrag = [](int c) { return (c % DB) * QB16 + c / DB; };
            auto frag = [&](int f) -> bf16x8 {
                return *reinterpret_cast<const bf16x8*>(ks + f * 1024 + lane * 16);
            };
            bf16x8 fr[RING];
#pragma unroll
            for (int f = 0; f < RING; ++f) fr[f] = frag(f);

            // S^T = K Q^T - m_run for this block: BN keys x 32 queries. The
            // wave issuing these MFMAs gets issue priority, so the other wave
            // on its SIMD runs its softmax meanwhile rather than both waves
            // reaching the softmax together.
            __builtin_amdgcn_s_setprio(2);
            f32x16 s[BN / 32];
#pragma unroll
            for (int f = 0; f < NK; ++f) {
                const int kk = f % (BN / 32), kb = f / (BN / 32);
                s[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % RING], qf[kb],
                                                                kb == 0 ? negm : s[kk], 0, 0, 0);
                if (f + RING < NK) fr[f % RING] = frag(f + RING);
            }
#pragma unroll
            for (int c = 0; c < RING; ++c) fr[(NK + c) % RING] = frag(NK + vfrag(c));

            __builtin_amdgcn_s_setprio(0);
            // Keys past the end of the sequence get -inf (never zero-padding).
            // The number of this lane's valid keys is made opaque to the
            // compiler, which would otherwise hoist the 32 comparisons out of
            // the loop and keep their lane masks in 64 scalar registers.
            if (b == sc.nkv - 1 && (Nk % BN) != 0) {
                int left = Nk - b * BN - half * 4;  // keys of this lane's row left in the block
                __asm__ volatile("" : "+v"(left));
#pragma unroll
                for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (kk * 32 + (i / 4) * 8 + (i % 4) >= left) s[kk][i] = -INFINITY;
            }

            // Row max of s: in-lane over this lane's keys (4 independent
            // chains), then with lane ^ 32, which holds the row's other keys.
            float mp[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
                for (int i = (kk == 0 ? 4 : 0); i < 16; ++i) mp[i & 3] = __builtin_elementwise_maximum(mp[i & 3], s[kk][i]);
            float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mp[0], mp[1]),
                                                     __builtin_elementwise_maximum(mp[2], mp[3]));
            {
                auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                           false, false);
                mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            // Lazy rescale: keep the reference m_run unless the row max passes
            // it by more than kLazy, so P = exp2(s) stays <= 2^kLazy; the final
            // O / l is exact for any such reference. The segment's first block
            // always sets it.
            const bool first = (b == kv0);
            if (first || mx > kLazy) {
                if (!first) {
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

            // P = exp2(s), rounded to bf16 for the second product; the row sum
            // accumulates the rounded values (v_dot2 with ones). Key group kq
            // (16 keys) of P is computed while the products of group kq - 1
            // run.
            bf16x8 pk[BN / 16];
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
            auto make_p = [&](int kq) {
                const int kk = kq / 2, hb = kq % 2;
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
                pk[kq] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
            };

            // O^T += V^T P^T.
            make_p(0);
#pragma unroll
            for (int kq = 0; kq < QB16; ++kq) {
                if (kq + 1 < QB16) make_p(kq + 1);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int c = kq * DB + db;
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[(NK + c) % RING], pk[kq], acc[db], 0, 0, 0);
                    if (c + RING < NV) fr[(NK + c) % RING] = frag(NK + vfrag(c + RING));
                }
            }

            // The next block's copies must have landed (this wave's: vmcnt;
            // the others': the barrier) before anyone reads them, and every
            // wave must be done with this buffer before it is refilled.
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            buf ^= 1;
        }

        if (next_dyn) {
            // Claim the next piece; its Q rows and first K/V block go to LDS
            // now (the buffer after this segment's last block is free).
            if (tid == 0)
                claimed = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            npiece = claimed;
            more = npiece < sc.npieces;
            if (more) {
                piece_segment(sc, npiece, &nt_, &nkv0, &nkv1);
                head_rsrc(nt_, &nkrs, &nvrs);
                if (q_lds) issue_q(nt_);
                char* nks = smem + buf * (KBYTES + VBYTES);
                issue_tile<D, BN, NW>(nkrs, nvrs, nkv0, nks, nks + KBYTES, wave, lane);
                __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __syncthreads();
        }
        if (q_lds && more && kv1 - kv0 == 1 && !next_dyn) {
            // A one-block segment: copy the next Q rows now and wait.
            issue_q(nt_);
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }

        // ---- segment epilogue ----
        const float l_half = l0 + l1;
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_half), __float_as_uint(l_half),
                                                   false, false);
        const float l_row = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const float inv = 1.0f / l_row;
        if (kv0 == 0 && kv1 == sc.nkv) {
            // Whole tile here: O = O^T / l, bf16; lse = ln 2 (m + log2 l).
            // Both lanes of a row (col, 0 / 1) are active together.
            if (qrow < Nq) {
                if (lse != nullptr && half == 0)
                    lse[(size_t)hd * Nq + qrow] = (m_run + log2f(l_row)) * 0.69314718055994531f;
                uint16_t* op = o + hd * oh + qrow * on_stride;
                store_o_rows<D>(acc, inv, half,
                                [&](int d0, uint4 w) { *reinterpret_cast<uint4*>(op + d0) = w; });
            }
        } else {
            // Part of a tile: leave (O / l in bf16, m, l) for the merge.
            const int slot = piece >= 0 ? piece : partial_slot(sc, pid, t);
            const int r = wave * 32 + col;
            uint16_t* po = part_o + ((size_t)slot * BM + r) * D;
            store_o_rows<D>(acc, inv, half, [&](int d0, uint4 w) { *reinterpret_cast<uint4*>(po + d0) = w; });
            if (half == 0)
                *reinterpret_cast<float2*>(part_ml + ((size_t)slot * BM + r) * 2) = make_float2(m_run, l_row);
        }
        t = nt_;
        kv0 = nkv0;
        kv1 = nkv1;
        piece = npiece;
        krs = nkrs;
        vrs = nvrs;
    }
}

// ---------------------------------------------------------------------------
// merge_kernel: merge of split leftover tiles. Grid (rem tiles, BM / RPB),
// 256 threads. A tile held whole by one workgroup returns at once. For row r
// over the segments s holding it (segment s left O_s / l_s in bf16):
//   M = max_s m_s,  O = sum_s 2^(m_s - M) l_s (O_s / l_s) / sum_s 2^(m_s - M) l_s,
//   lse = ln 2 (M + log2 sum_s 2^(m_s - M) l_s).
// MW = 4 (tiles split many ways): four waves per row (RPB = 1), D/64 head
// dims per lane; wave w folds segments w, w + 4, ... in one pass with a
// running maximum, then the four partial results are folded the same way.
// MW = 1 (tiles split a few ways): 16 lanes per row, D/16 head dims per lane
// (8- or 16-byte loads), four rows per wave (RPB = 16); each lane folds all
// of its row's segments.
// ---------------------------------------------------------------------------
template <int D, int NW, int MW>
__global__ __launch_bounds__(256) void merge_kernel(uint16_t* __restrict__ o, float* __restrict__ lse,
                                                    const uint16_t* __restrict__ part_o,
                                                    const float* __restrict__ part_ml, int N,
                                                    Sched sc, long long oh, long long on_stride) {
    constexpr int BM = NW * 32;
    static_assert(MW == 1 || MW == 4, "waves per row");
    constexpr int LPR = MW == 4 ? 64 : 16;    // lanes per row (of one wave)
    constexpr int DPL = D / LPR;              // head dims per lane
    constexpr int RPB = MW == 4 ? 1 : 16;     // rows per block
    const int t = sc.full * sc.P + blockIdx.x;
    const int y0 = blockIdx.x * sc.nkv;  // leftover unit offsets of tile t
    // Parts p0 .. p1: workgroups (static split) or pieces (dyn), in order.
    const int p0 = sc.dyn ? blockIdx.x * sc.ppt : rem_owner(sc, y0);
    const int p1 = sc.dyn ? p0 + sc.ppt - 1 : rem_owner(sc, y0 + sc.nkv - 1);
    if (p0 == p1) return;  // uniform over the block
    const int hd = t / sc.n_qtiles, qt = t % sc.n_qtiles;
    const int wv = threadIdx.x >> 6;
    const int lane = threadIdx.x & (LPR - 1);
    const int r = MW == 4 ? blockIdx.y : blockIdx.y * RPB + (threadIdx.x >> 4);
    const int w = MW == 4 ? wv : 0;
    const int qrow = qt * BM + r;
    if (qrow >= N) return;  // uniform over the block when MW == 4

    // Partial slots: every workgroup after p0 starts its range inside tile
    // t, so t is its first leftover tile (slot 2p); p0's range starts in t
    // only if its first unit is t's first unit.
    const int slot0 = sc.dyn ? p0 : partial_slot(sc, p0, t);
    float M = -INFINITY, L = 0.0f, acc[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;
#pragma unroll 4
    for (int p = p0 + w; p <= p1; p += MW) {
        const int slot = sc.dyn ? p : (p == p0 ? slot0 : 2 * p);
        const float2 ml = *reinterpret_cast<const float2*>(part_ml + ((size_t)slot * BM + r) * 2);
        const uint16_t* po = part_o + ((size_t)slot * BM + r) * D + lane * DPL;
        float x[DPL];
        if constexpr (DPL == 1) {
            x[0] = __uint_as_float((uint32_t)po[0] << 16);
        } else {
            uint32_t w[DPL / 2];
            if constexpr (DPL == 8) {
                const uint4 v = *reinterpret_cast<const uint4*>(po);
                w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
            } else if constexpr (DPL == 4) {
                const uint2 v = *reinterpret_cast<const uint2*>(po);
                w[0] = v.x; w[1] = v.y;
            } else {
                w[0] = *reinterpret_cast<const uint32_t*>(po);
            }
#pragma unroll
            for (int i = 0; i < DPL / 2; ++i) {
                x[2 * i] = bf_lo(w[i]);
                x[2 * i + 1] = bf_hi(w[i]);
            }
        }
        const float Mn = fmaxf(M, ml.x);
        const float a = __builtin_amdgcn_exp2f(M - Mn), b = __builtin_amdgcn_exp2f(ml.x - Mn) * ml.y;
        L = L * a + b;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[i] = acc[i] * a + b * x[i];
        M = Mn;
    }
    float Mt = M, Lt = L, at[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) at[i] = acc[i];
    if constexpr (MW > 1) {
        __shared__ float sm_ml[MW][2];
        __shared__ float sm_o[MW][D];
        if (lane == 0) {
            sm_ml[w][0] = M;
            sm_ml[w][1] = L;
        }
#pragma unroll
        for (int i = 0; i < DPL; ++i) sm_o[w][lane * DPL + i] = acc[i];
        __syncthreads();
        if (w != 0) return;
        Mt = sm_ml[0][0];
#pragma unroll
        for (int v = 1; v < MW; ++v) Mt = fmaxf(Mt, sm_ml[v][0]);
        Lt = 0.0f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) at[i] = 0.0f;
#pragma unroll
        for (int v = 0; v < MW; ++v) {
            const float b = __builtin_amdgcn_exp2f(sm_ml[v][0] - Mt);  // 0 for a wave with no segment
            Lt += b * sm_ml[v][1];
#pragma unroll
            for (int i = 0; i < DPL; ++i) at[i] += b * sm_o[v][lane * DPL + i];
        }
    }
    const float inv = 1.0f / Lt;
    if (lse != nullptr && lane == 0) lse[(size_t)hd * N + qrow] = (Mt + log2f(Lt)) * 0.69314718055994531f;
    uint16_t* op = o + hd * oh + qrow * on_stride + lane * DPL;
    uint32_t pk[DPL > 1 ? DPL / 2 : 1];
#pragma unroll
    for (int i = 0; i < DPL / 2; ++i) pk[i] = pack_bf16(at[2 * i] * inv, at[2 * i + 1] * inv);
    if constexpr (DPL == 8) {
        *reinterpret_cast<uint4*>(op) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else if constexpr (DPL == 4) {
        *reinterpret_cast<uint2*>(op) = make_uint2(pk[0], pk[1]);
    } else if constexpr (DPL == 2) {
        *reinterpret_cast<uint32_t*>(op) = pk[0];
    } else {
        *op = (uint16_t)(pack_bf16(at[0] * inv, 0.0f) & 0xffffu);
    }
}

// ---------------------------------------------------------------------------
// merge_parts_kernel: combine attention results over disjoint key sets (Ring-style key
// splitting keeps attention exact this way). Part i holds O_i [rows][D] bf16,
// normalised over its own keys, and lse_i [rows] fp32; over the union of the
// key sets
//     lse = log sum_i e^{lse_i},   O = sum_i e^{lse_i - lse} O_i.
// D/8 lanes per row (8 head dims, 16 bytes each), 256 threads per block. A
// row whose parts are all -inf (no keys anywhere) gets O = 0, lse = -inf.
// ---------------------------------------------------------------------------
constexpr int kMaxMergeParts = 8;
struct MergeParts {
    const uint16_t* o[kMaxMergeParts];
    const float* lse[kMaxMergeParts];
};

template <int D>
__global__ __launch_bounds__(256) void merge_parts_kernel(MergeParts parts, int nparts,
                                                          long long rows,
                                                          uint16_t* __restrict__ o,
                                                          float* __restrict__ lse) {
    constexpr int LPR = D / 8;  // lanes per row
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long row = gid / LPR;
    const int c = (int)(gid % LPR);
    if (row >= rows) return;
    constexpr float kLog2e = 1.4426950408889634f;
    float li[kMaxMergeParts];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxMergeParts; ++i) {
        li[i] = (i < nparts) ? parts.lse[i][row] : -INFINITY;
        m = fmaxf(m, li[i]);
    }
    uint16_t* op = o + row * D + c * 8;
    if (m == -INFINITY) {
        *reinterpret_cast<uint4*>(op) = make_uint4(0, 0, 0, 0);
        if (lse != nullptr && c == 0) lse[row] = -INFINITY;
        return;
    }
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxMergeParts; ++i) {
        if (i >= nparts) break;
        const float w = __builtin_amdgcn_exp2f((li[i] - m) * kLog2e);
        z += w;
        const uint4 x = *reinterpret_cast<const uint4*>(parts.o[i] + row * D + c * 8);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w * bf_lo(xs[e]);
            acc[2 * e + 1] += w * bf_hi(xs[e]);
        }
    }
    const float inv = 1.0f / z;
    *reinterpret_cast<uint4*>(op) =
        make_uint4(pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv),
                   pack_bf16(acc[4] * inv, acc[5] * inv), pack_bf16(acc[6] * inv, acc[7] * inv));
    if (lse != nullptr && c == 0) lse[row] = m + logf(z);
}

}  // namespace regen
