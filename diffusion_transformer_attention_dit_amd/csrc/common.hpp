// Device helpers shared by the regen_attn kernels (CDNA4, gfx950): bf16
// packing, buffer resources, LDS-DMA copies, the XOR swizzle of LDS tiles and
// the XCD-aware block numbering.
//
// MFMA v_mfma_f32_32x32x16_bf16 operand layout (lane l, c = l % 32,
// g = l / 32): A supplies row c, k = 8g..8g+7; B supplies column c,
// k = 8g..8g+7; the 16 fp32 results of lane l are D[row = 8(i/4) + 4g + i%4]
// [column c], i = 0..15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace regen {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (round-to-nearest-even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 left at their maximum).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// ... and for lgkmcnt <= n only (vmcnt and expcnt at their maximum).
constexpr int lgkmcnt_only(int n) { return 15 | (3 << 14) | (7 << 4) | ((n & 15) << 8); }

// Logical block id with consecutive ids on one XCD. Blocks are dispatched
// round-robin over the 8 XCDs (block b runs on XCD b % 8); this maps each
// XCD's blocks onto one contiguous range of logical ids, so that the blocks
// sharing an XCD's L2 work on neighbouring data (the same head's K/V in
// attention, neighbouring output tiles in the GEMM).
__device__ __forceinline__ int xcd_remap(int b, int G) {
    const int per = G / 8, rem = G % 8, x = b % 8, loc = b / 8;
    return (x < rem) ? x * (per + 1) + loc : rem * (per + 1) + (x - rem) * per + loc;
}

// Byte offset of 16-byte chunk c of row r in an LDS tile whose rows are RB
// bytes (128 or 256) and stored unpadded. Chunks are XOR-swizzled by row so
// that the MFMA operand reads (32 rows, one chunk column) are free of bank
// conflicts; the swizzle is its own inverse.
template <int RB>
__device__ __forceinline__ int swz_off(int r, int c) {
    static_assert(RB == 128 || RB == 256, "row bytes");
    const int pc = (RB == 256) ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
    return r * RB + pc * 16;
}

// Buffer resource over `bytes` bytes at `base` (raw, untyped 32-bit data
// format); accesses past `bytes` read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// One wave-wide 16-byte-per-lane copy global -> LDS without registers
// (buffer_load_dwordx4 ... lds): lane i's 16 bytes, read at byte `voff` of
// the resource, land at lds_wave_base + 16 i. The MUBUF form is used rather
// than the global (FLAT) one so that LDS reads issued while copies are in
// flight keep precise, in-order wait counts.
__device__ __forceinline__ void g2lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                        void* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base,
                                             16, voff, 0, 0, 0);
}

}  // namespace regen
