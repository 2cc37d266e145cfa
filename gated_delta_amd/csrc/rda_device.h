// rda_device.h -- small device helpers for the gfx950 kernels: vector types,
// bf16 conversion and hi/lo splitting, 16-lane DPP reductions, input loads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(uint32_t(h) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): the pair carries ~16
// mantissa bits, so an MFMA product of pairs (hi*hi + hi*lo + lo*hi) is
// accurate to ~2^-16 relative.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Split two fp32 values into packed bf16 hi and lo pairs (element 0 in the
// low half): hi = bf16(x), lo = bf16(x - hi), both round-to-nearest-even.
// Compiles to two v_cvt_pk_bf16_f32 plus four VALU ops for the pair.
__device__ __forceinline__ void split_pk(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const f32x2 v = {x0, x1};
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    const f32x2 hf = {__uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(v - hf, bf16x2));
}

// Sum over each 16-lane row of the wavefront with DPP (every lane of the
// row receives the row's sum): xor 1, xor 2 (quad permutes), then the half-
// and full-row mirrors pair up quads and half rows.
__device__ __forceinline__ float dpp_sum16(float x) {
    int v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false)); // row_half_mirror
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false)); // row_mirror
    return x;
}

// Largest of x over each 16-lane row (every lane of the row gets it).
__device__ __forceinline__ uint32_t dpp_umax16(uint32_t x) {
    x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0xB1, 0xF, 0xF, false)));
    x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x4E, 0xF, 0xF, false)));
    x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x141, 0xF, 0xF, false)));
    x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x140, 0xF, 0xF, false)));
    return x;
}

// Bitwise or of x over each group of 4 lanes.
__device__ __forceinline__ uint32_t dpp_or4(uint32_t x) {
    x |= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0xB1, 0xF, 0xF, false));
    x |= uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x4E, 0xF, 0xF, false));
    return x;
}

// Index of this lane's wavefront in the workgroup, as a wave-uniform scalar.
// Branches on it then compile to scalar branches: an MFMA placed under a
// per-lane EXEC mask would still execute for every lane (MFMA ignores EXEC),
// so wave-role conditions around matrix code must never be lane-divergent.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// A float that every lane of the wave holds alike, moved to a scalar
// register (its bits, not a conversion).
__device__ __forceinline__ float uniform_f32(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// D += A * B on v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16, c = l % 16:
// A lane holds row c, k = 8g .. 8g+7; B lane holds column c, the same k;
// D lane holds rows 4g .. 4g+3 of column c).
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D += A * B on v_mfma_f32_16x16x4_f32 (A lane: row c, k = g; B: column c, k = g).
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Split 8 fp32 values into bf16 hi and lo vectors (paired conversions).
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t a, b;
        split_pk(x[2 * p], x[2 * p + 1], a, b);
        h[p] = a;
        l[p] = b;
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Load 4 consecutive input elements as fp32 (bf16 bits or fp32).
__device__ __forceinline__ void load4_bf16(const uint16_t* p, float out[4]) {
    u16x4 h = *reinterpret_cast<const u16x4*>(p);
    out[0] = bf16_bits_to_f32(h[0]);
    out[1] = bf16_bits_to_f32(h[1]);
    out[2] = bf16_bits_to_f32(h[2]);
    out[3] = bf16_bits_to_f32(h[3]);
}

__device__ __forceinline__ void load4_f32(const float* p, float out[4]) {
    f32x4 x = *reinterpret_cast<const f32x4*>(p);
    out[0] = x[0];
    out[1] = x[1];
    out[2] = x[2];
    out[3] = x[3];
}

template <typename T>
__device__ __forceinline__ void load4(const T* p, float out[4]);
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float out[4]) { load4_bf16(p, out); }
template <>
__device__ __forceinline__ void load4<float>(const float* p, float out[4]) { load4_f32(p, out); }

template <typename T>
__device__ __forceinline__ float load1(const T* p);
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }

}  // namespace rda
