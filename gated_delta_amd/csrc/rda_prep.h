// rda_prep.h -- the per-(chunk, head) factors of the chunked prefill for bf16
// inputs, as a device function: the prep kernel runs one item per 256-thread
// workgroup, and the walk kernel's prep workgroups run four at a time (four
// 256-thread groups, each with its own PrepLds) on the CUs the walk leaves
// idle.  The chunk algebra is stated at the top of rda_prefill.hip; the
// layout of the factors at the top of rda_internal.h.
//
// One item: T_b = (I + L)^-1 diag(b), L = strict-lower(diag(b) K K^T .
// Gamma_ij), and A = lower(Q K^T . Gamma_ij), both packed as the walk's bf16
// hi/lo MFMA A operands, and the gates (gamma, gamma_C / gamma, gamma_C, the
// running log gate).  LDS holds the K and Q tiles (16-byte granules swizzled
// per row, loaded with LDS-DMA) and, once the Gram products are in
// registers, L and T in the same bytes.  A is produced directly in its
// packed layout: the transposed tile (K_j Q_i^T) leaves each lane exactly
// the 4 + 4 entries of its operand slot.  The triangular solve runs in fp32:
// the four 16 x 16 diagonal blocks by forward substitution with one lane
// per column, the off-diagonal blocks by block substitution on fp32 MFMA.
#pragma once

#include "rda_internal.h"
#include "rda_lds.h"
#include "rda_solve.h"

namespace rda {

struct PrepLds {
    union {
        struct {
            uint16_t K[kC * kD];   // 64 token rows x 256 B, granule j of row r at j ^ swz(r)
            uint16_t Q[kC * kD];
        } in;
        struct {
            float L[kC * kFS];
            float T[kC * kFS];
        } mat;
    } u;
    float la[64], bb[64], gg[64], gam[64];
    float R[3][256];   // off-diagonal solve scratch, one 16 x 16 block per wave
};

static_assert(sizeof(PrepLds) <= 40 * 1024, "four workgroups per CU");

// One item by one 256-thread group: `tid` 0..255 and `w` = tid / 64 (a
// wave-uniform value).  With valid false the group loads and stores nothing
// but passes the same workgroup barriers (the walk's prep workgroups run
// four groups in step).
__device__ __forceinline__ void prep_item(const PrepItemArgs& A, int chunk, int h, int t0, int len,
                                          bool valid, PrepLds& S, int tid, int w) {
    const uint16_t* __restrict__ q = A.q;
    const uint16_t* __restrict__ k = A.k;
    const float* __restrict__ a = A.a;
    const float* __restrict__ b = A.b;
    const int H = A.H;
    const int l = tid & 63, g = l >> 4, c = l & 15;
    unsigned char* F = A.factors + (size_t(chunk) * H + h) * kChunkHeadBytes;

    // ---- K and Q tiles by LDS-DMA (rows past the end duplicate the last
    // row: only finite values are needed there, b = 0 zeroes their effect)
    if (valid) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 4 * w + i;
            const int r = 4 * n + (l >> 4);
            const int rr = r < len ? r : len - 1;
            const int j = (l & 15) ^ swz(r);
            const size_t off = (size_t(t0 + rr) * H + h) * kD + 8 * j;
            dma16(k + off, reinterpret_cast<char*>(S.u.in.K) + 1024 * n);
            dma16(q + off, reinterpret_cast<char*>(S.u.in.Q) + 1024 * n);
        }
    }
    if (w == 0) {
        // gates: log a (clamped far below any fp32-visible decay), prefix sum;
        // rows past the chunk's end act as a = 1, b = 0 (inert)
        float lav = 0.f, bv = 0.f;
        if (valid && l < len) {
            const size_t th = size_t(t0 + l) * H + h;
            lav = fmaxf(logf(a[th]), -100.f);
            bv = b[th];
        }
        float sum = lav;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(sum, off, 64);
            if (l >= off) sum += o;
        }
        S.la[l] = lav;
        S.bb[l] = bv;
        S.gg[l] = sum;
        S.gam[l] = expf(sum);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's tile blocks have landed
    __syncthreads();

    // ---- Gram products.  Wave w: L tiles (ti, w) for ti >= w, and the
    // transposed A tiles (tj, w) for tj <= w, i.e. A's row tile w.  The decay
    // weights e^{g_i - g_j} (exponent <= 0 where used) take the hardware
    // exponential (a few 1e-7 relative), 20 per lane instead of the full
    // libm sequence.
    float Lv[4][4];
    {
        bf16x8 kw[4], qw[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            kw[m] = row_op(S.u.in.K, 16 * w + c, m, g);
            qw[m] = row_op(S.u.in.Q, 16 * w + c, m, g);
        }
        f32x4 at[4];
        const float gi = S.gg[16 * w + c];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 kt[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) kt[m] = row_op(S.u.in.K, 16 * t + c, m, g);
            const f32x4 gr = *reinterpret_cast<const f32x4*>(S.gg + 16 * t + 4 * g);
            if (t >= w) {   // L tile (t, w): rows 16t + 4g + e, column 16w + c
                f32x4 d = zero4();
#pragma unroll
                for (int m = 0; m < 4; ++m) d = mfma_bf16(kt[m], kw[m], d);
                const f32x4 br = *reinterpret_cast<const f32x4*>(S.bb + 16 * t + 4 * g);
                const int s = 16 * w + c;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * t + 4 * g + e;
                    Lv[t][e] = r > s ? br[e] * d[e] * __expf(gr[e] - gi) : 0.f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) Lv[t][e] = 0.f;
            }
            if (t <= w) {   // transposed A tile (t, w): A[16w + c][16t + 4g + e]
                f32x4 d = zero4();
#pragma unroll
                for (int m = 0; m < 4; ++m) d = mfma_bf16(kt[m], qw[m], d);
                const int i = 16 * w + c;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * t + 4 * g + e;
                    at[t][e] = j <= i ? d[e] * __expf(gi - gr[e]) : 0.f;
                }
            } else {
                at[t] = zero4();
            }
        }
        // A slots (w, m): row 16w + c, tokens {32m + 4g + e, 32m + 16 + 4g + e};
        // slots (w < 2, m = 1) are zero and never read, so they are not written
        bf16x8* P = reinterpret_cast<bf16x8*>(F + kOffA);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (!valid || m > (w >> 1)) break;
            const float x8[8] = {at[2 * m][0],     at[2 * m][1],     at[2 * m][2],
                                 at[2 * m][3],     at[2 * m + 1][0], at[2 * m + 1][1],
                                 at[2 * m + 1][2], at[2 * m + 1][3]};
            bf16x8 hi, lo;
            split8(x8, hi, lo);
            P[((w * 2 + m) * 2) * 64 + l] = hi;
            P[((w * 2 + m) * 2 + 1) * 64 + l] = lo;
        }
    }
    __syncthreads();   // every K, Q read is done: the tiles' bytes become L and T
    float* Ls = S.u.mat.L;
    float* Ts = S.u.mat.T;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (t < w) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) Ls[(16 * t + 4 * g + e) * kFS + 16 * w + c] = Lv[t][e];
    }
    __syncthreads();

    // ---- T = (I + L)^-1: the four 16 x 16 diagonal blocks by column-oriented
    // forward substitution (one wave per block), the off-diagonal blocks by
    // block substitution on fp32 MFMA (ends with a workgroup barrier) ---------
    solve_unit_lower(Ls, Ts, &S.R[0][0], w, g, c);

    // ---- T_b = T diag(b) packed (slot (w, m): row 16w + lane % 16, tokens
    // {32m + 4g + e, 32m + 16 + 4g + e}); T is zero above the diagonal
    {
        bf16x8* P = reinterpret_cast<bf16x8*>(F + kOffTb);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (!valid || m > (w >> 1)) break;   // zero slot, never read
            const int r = 16 * w + c, c0 = 32 * m + 4 * g;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(Ts + r * kFS + c0);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(Ts + r * kFS + c0 + 16);
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(S.bb + c0);
            const f32x4 s1 = *reinterpret_cast<const f32x4*>(S.bb + c0 + 16);
            float x8[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x8[e] = c0 + e <= r ? x0[e] * s0[e] : 0.f;
                x8[4 + e] = c0 + 16 + e <= r ? x1[e] * s1[e] : 0.f;
            }
            bf16x8 hi, lo;
            split8(x8, hi, lo);
            P[((w * 2 + m) * 2) * 64 + l] = hi;
            P[((w * 2 + m) * 2 + 1) * 64 + l] = lo;
        }
    }
    if (valid && tid < 64) {
        float* G = reinterpret_cast<float*>(F + kOffG);
        G[kGGam + tid] = S.gam[tid];
        G[kGScale + tid] = expf(S.gg[63] - S.gg[tid]);
        G[kGLog + tid] = S.gg[tid];
        if (tid == 0) G[kGC] = S.gam[63];
    }
}

}  // namespace rda
