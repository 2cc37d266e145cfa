// rda_solve.h -- pieces shared by the chunk preps: the unit-lower-triangular
// solve T = (I + L)^-1 of a 64 x 64 fp32 matrix in LDS, and the packing of a
// 64 x 64 fp32 matrix as the walks' bf16 hi/lo MFMA A operands.
#pragma once

#include "rda_device.h"
#include "rda_internal.h"

namespace rda {

constexpr int kFS = 68;    // fp32 64x64 matrix row stride in LDS

// Pack rows of a 64 x 64 fp32 matrix (columns scaled by `colscale` when
// given) as bf16 hi/lo A operands for the walk: slot (row tile w, token
// block m, lane) holds row 16w + (lane % 16), columns {32m + 4g + i,
// 32m + 16 + 4g + i} with g = lane / 16; hi at [(w*2+m)*2][lane], lo after it.
__device__ __forceinline__ void pack_rows(const float* M, const float* colscale, bf16x8* dst,
                                          int tid) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
        const int slot = tid + 256 * qq;
        const int lp = slot & 63, m = (slot >> 6) & 1, wp = slot >> 7;
        const int r = 16 * wp + (lp & 15), c0 = 32 * m + 4 * (lp >> 4);
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(M + r * kFS + c0);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(M + r * kFS + c0 + 16);
        float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        if (colscale) {
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(colscale + c0);
            const f32x4 s1 = *reinterpret_cast<const f32x4*>(colscale + c0 + 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[j] *= s0[j];
                x[4 + j] *= s1[j];
            }
        }
        bf16x8 hi, lo;
        split8(x, hi, lo);
        const int base = ((wp * 2 + m) * 2) * 64 + lp;
        dst[base] = hi;
        dst[base + 64] = lo;
    }
}

// Step m of the column-oriented substitution in a 16 x 16 diagonal block:
// x_r -= L_rm x_m on every lane, with x_m taken from lane m of the same
// 16-lane row (DPP row_newbcast:m), then steps m + 1 .. 14.
template <int kM>
__device__ __forceinline__ void substitute_col_step(float (&x)[4], const float (&Lrow)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float xm = __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(x[j]), 0x150 + kM, 0xF, 0xF, false));
        x[j] -= Lrow[kM] * xm;
    }
    if constexpr (kM < 14) substitute_col_step<kM + 1>(x, Lrow);
}

// T = (I + L)^-1 for the strictly lower L in Ls (row stride kFS; Ts must
// hold zeros above the diagonal); one call by every wavefront of the
// workgroup (w = wave, g = lane / 16, c = lane % 16), of which waves 0-3 do
// the work; Rs is 3 x 256 floats of scratch.  Ends with a workgroup barrier.
__device__ __forceinline__ void solve_unit_lower(const float* Ls, float* Ts, float* Rs, int w,
                                                 int g, int c) {
    // (a) diagonal 16x16 blocks, one wavefront per block: lane (g, r = c)
    //     holds row r of columns 4g .. 4g+3, starting from the identity.
    //     Column-oriented forward substitution: once x_m is final, every row
    //     r > m takes x_r -= L_rm x_m, x_m broadcast inside each 16-lane row
    //     by DPP; L is zero on and above the diagonal, so rows r <= m are
    //     left unchanged without a branch.
    if (w < 4) {
        const int base = 16 * w, r = c;
        float Lrow[16];
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(Ls + (base + r) * kFS + base + 4 * m4);
#pragma unroll
            for (int e = 0; e < 4; ++e) Lrow[4 * m4 + e] = v[e];
        }
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = r == 4 * g + j ? 1.f : 0.f;
        substitute_col_step<0>(x, Lrow);
        *reinterpret_cast<f32x4*>(Ts + (base + r) * kFS + base + 4 * g) = f32x4{x[0], x[1], x[2], x[3]};
    }
    __syncthreads();
    // (b) off-diagonal blocks, block row by block row, on fp32 MFMA:
    //     T_ij = -T_ii * sum_{m=j}^{i-1} L_im T_mj.
    for (int bi = 1; bi < 4; ++bi) {
        if (w < bi) {
            const int bj = w;
            f32x4 acc = zero4();
            for (int m = bj; m < bi; ++m) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const float av = Ls[(16 * bi + c) * kFS + 16 * m + 4 * s4 + g];
                    const float bv = Ts[(16 * m + 4 * s4 + g) * kFS + 16 * bj + c];
                    acc = mfma_f32(av, bv, acc);
                }
            }
            float* R = Rs + 256 * w;
#pragma unroll
            for (int i = 0; i < 4; ++i) R[(4 * g + i) * 16 + c] = acc[i];
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): R visible to this wavefront
            f32x4 acc2 = zero4();
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const float av = Ts[(16 * bi + c) * kFS + 16 * bi + 4 * s4 + g];
                const float bv = R[(4 * s4 + g) * 16 + c];
                acc2 = mfma_f32(av, bv, acc2);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) Ts[(16 * bi + 4 * g + i) * kFS + 16 * bj + c] = -acc2[i];
        }
        __syncthreads();
    }
}

}  // namespace rda
