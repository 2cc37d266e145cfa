// rda_lds.h -- LDS helpers shared by the chunk kernels: LDS-DMA issue and
// waits, the swizzled 256-byte token rows of K / Q tiles, the transposing
// 8-byte read, and the exchange buffers that hold ready bf16 hi/lo MFMA
// B operands.
#pragma once

#include "rda_device.h"

namespace rda {

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS-DMA: lane L's 16 (4) bytes from `src` land at lds_dst + 16 L (4 L).
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 4, 0, 0);
}

// Wait until at most kN vector memory operations of this wave are in flight
// (they complete in issue order); expcnt and lgkmcnt are left at their maxima.
template <int kN>
__device__ __forceinline__ void wait_vm() {
    static_assert(kN >= 0 && kN < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((kN & 15) | ((kN >> 4) << 14) | 0x0F70);
}

// Row r of a K or Q tile in LDS (64 rows of 256 bytes) keeps 16-byte granule
// j at position j ^ swz(r).  Sixteen consecutive rows read at one granule
// (row operands) and eight consecutive rows read at two adjacent granules
// (transposing reads) both land on distinct granules, i.e. distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// Row r of a swizzled tile as an MFMA A operand in natural k order: lane
// (g, c) gets elements 32m + 8g .. +7 (one 16-byte granule).
__device__ __forceinline__ bf16x8 row_op(const uint16_t* T, int r, int m, int g) {
    const unsigned char* row = reinterpret_cast<const unsigned char*>(T) + r * 256;
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const u32x4*>(row + 16 * ((4 * m + g) ^ swz(r))));
}

// ds_read_b64_tr_b16: within each 16-lane group, output lane i receives
// element i % 4 of the 8 bytes that source lane 4e + i / 4 addresses.
__device__ __forceinline__ u32x2 tr_read(const void* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

// Exchange buffers hold ready 16-byte B operands: entry [blk][hl][lane] is
// key (or token) block blk in bf16 hi (hl = 0) or lo (hl = 1), whose low 8
// bytes come from D tile 2 blk and high 8 bytes from tile 2 blk + 1, each
// written by the wave that owns that tile.
__device__ __forceinline__ void put_half(u32x4 (*X)[2][64], int tile, int l, u32x2 hi, u32x2 lo) {
    reinterpret_cast<u32x2*>(&X[tile >> 1][0][l])[tile & 1] = hi;
    reinterpret_cast<u32x2*>(&X[tile >> 1][1][l])[tile & 1] = lo;
}

// A D tile's 4 values of this lane, split into bf16 hi/lo, into its half.
__device__ __forceinline__ void publish4(u32x4 (*X)[2][64], int tile, int l, f32x4 v) {
    uint32_t h01, l01, h23, l23;
    split_pk(v[0], v[1], h01, l01);
    split_pk(v[2], v[3], h23, l23);
    put_half(X, tile, l, u32x2{h01, h23}, u32x2{l01, l23});
}

__device__ __forceinline__ bf16x8 ldsop(const u32x4 (*X)[2][64], int blk, int hl, int l) {
    return __builtin_bit_cast(bf16x8, X[blk][hl][l]);
}

// Products of a hi/lo A operand with a hi/lo B operand into three
// accumulators: hi*hi, hi*lo, lo*hi (lo*lo is below fp32 resolution).
__device__ __forceinline__ void mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4& p0,
                                     f32x4& p1, f32x4& p2) {
    p0 = mfma_bf16(ah, bh, p0);
    p1 = mfma_bf16(ah, bl, p1);
    p2 = mfma_bf16(al, bh, p2);
}

}  // namespace rda
