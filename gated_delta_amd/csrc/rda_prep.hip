// rda_prep.hip -- per-chunk factors of the chunked RDA prefill for bf16
// inputs on gfx950 (the chunk algebra is stated at the top of
// rda_prefill.hip).  One 4-wave workgroup per (chunk, head) writes, in the
// layout the walk streams:
//   T_b = (I + L)^-1 diag(b),  L = strict-lower(diag(b) K K^T . Gamma_ij)
//   A   = lower(Q K^T . Gamma_ij)
// both as bf16 hi/lo MFMA A operands, and the gates (gamma, gamma_C / gamma,
// gamma_C, the running log gate).
//
// LDS holds the K and Q tiles (16-byte granules swizzled per row, loaded
// with LDS-DMA) and, once the Gram products are in registers, L and T in the
// same bytes; 38 KiB in all, so four workgroups share a CU and hide each
// other's latency.  A is produced directly in its packed layout: the
// transposed tile (K_j Q_i^T) leaves each lane exactly the 4 + 4 entries of
// its operand slot.  The triangular solve runs in fp32: the four 16 x 16
// diagonal blocks by forward substitution with one lane per column (no
// cross-lane reductions), the off-diagonal blocks by block substitution on
// fp32 MFMA.
#include "rda_device.h"
#include "rda_internal.h"

namespace rda {

namespace {

constexpr int kFS = 68;   // fp32 64 x 64 matrix row stride (floats): spreads LDS banks

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

__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

typedef __attribute__((address_space(3))) void lds_void;

// Row r of a swizzled tile, natural k order: lane (g, c) gets elements
// 32m + 8g .. +7 (one 16-byte granule).
__device__ __forceinline__ bf16x8 row_op(const uint16_t* T, int r, int m, int g) {
    const unsigned char* row = reinterpret_cast<const unsigned char*>(T) + r * 256;
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const u32x4*>(row + 16 * ((4 * m + g) ^ swz(r))));
}

// Step m of the column-oriented substitution in a 16 x 16 diagonal block:
// x_r -= L_rm x_m on every lane, with x_m taken from lane m of the same
// 16-lane row (DPP row_newbcast:m), then steps m + 1 .. 14.
template <int kM>
__device__ __forceinline__ void substitute_step(float (&x)[4], const float (&Lrow)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float xm = __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(x[j]), 0x150 + kM, 0xF, 0xF, false));
        x[j] -= Lrow[kM] * xm;
    }
    if constexpr (kM < 14) substitute_step<kM + 1>(x, Lrow);
}

__global__ __launch_bounds__(256) void prep_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ a,
    const float* __restrict__ b, int H, const int32_t* __restrict__ rec,
    const int32_t* __restrict__ num_chunks, unsigned char* __restrict__ factors,
    int32_t single_T, int32_t* __restrict__ rec_out, int32_t* __restrict__ seq_off_out,
    int32_t* __restrict__ num_out) {
    __shared__ __attribute__((aligned(16))) PrepLds S;
    const int chunk = blockIdx.x / H;
    const int h = blockIdx.x - chunk * H;
    int t0, len;
    if (single_T >= 0) {
        // one sequence of single_T tokens and no offsets: every chunk record
        // is plain arithmetic (the grid holds exactly ceil(single_T / 64)
        // chunks), and the head-0 workgroups also write the chunk table the
        // walk reads, so that no table kernel runs for this case
        t0 = kC * chunk;
        len = single_T - t0 < kC ? single_T - t0 : kC;
        if (h == 0 && threadIdx.x < 4) {
            const int32_t field[4] = {0, t0, len, chunk};
            rec_out[4 * chunk + threadIdx.x] = field[threadIdx.x];
            if (chunk == 0) {
                const int32_t nch = int32_t(gridDim.x / H);
                if (threadIdx.x == 0) seq_off_out[0] = 0;
                if (threadIdx.x == 1) seq_off_out[1] = nch;
                if (threadIdx.x == 2) num_out[0] = nch;
            }
        }
    } else {
        if (chunk >= num_chunks[0]) return;
        t0 = rec[4 * chunk + 1];
        len = rec[4 * chunk + 2];
    }
    const int tid = threadIdx.x;
    const int w = wave_id(), l = tid & 63, g = l >> 4, c = l & 15;
    unsigned char* F = factors + (size_t(chunk) * H + h) * kChunkHeadBytes;

    // ---- K and Q tiles by LDS-DMA (rows past the end duplicate the last
    // row: only finite values are needed there, b = 0 zeroes their effect)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = 4 * w + i;
        const int r = 4 * n + (l >> 4);
        const int rr = r < len ? r : len - 1;
        const int j = (l & 15) ^ swz(r);
        const size_t off = (size_t(t0 + rr) * H + h) * kD + 8 * j;
        __builtin_amdgcn_global_load_lds(k + off, (lds_void*)(reinterpret_cast<char*>(S.u.in.K) + 1024 * n),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(q + off, (lds_void*)(reinterpret_cast<char*>(S.u.in.Q) + 1024 * n),
                                         16, 0, 0);
    }
    if (w == 0) {
        // gates: log a (clamped far below any fp32-visible decay), prefix sum;
        // rows past the chunk's end act as a = 1, b = 0 (inert)
        float lav = 0.f, bv = 0.f;
        if (l < len) {
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
            if (m > (w >> 1)) break;
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

    // ---- T = (I + L)^-1 -------------------------------------------------------
    // (a) diagonal block w, all 64 lanes: lane (g, r = c) holds row r of
    //     columns 4g .. 4g+3, starting from the identity.  Column-oriented
    //     forward substitution: once x_m is final, every row r > m takes
    //     x_r -= L_rm x_m, with x_m broadcast inside each 16-lane row by DPP
    //     (row_newbcast).  L is zero on and above the diagonal, so rows
    //     r <= m are left unchanged without a branch.
    {
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
        substitute_step<0>(x, Lrow);
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
            float* R = S.R[w];
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

    // ---- T_b = T diag(b) packed (slot (w, m): row 16w + lane % 16, tokens
    // {32m + 4g + e, 32m + 16 + 4g + e}); T is zero above the diagonal
    {
        bf16x8* P = reinterpret_cast<bf16x8*>(F + kOffTb);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (m > (w >> 1)) break;   // zero slot, never read
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
    if (tid < 64) {
        float* G = reinterpret_cast<float*>(F + kOffG);
        G[kGGam + tid] = S.gam[tid];
        G[kGScale + tid] = expf(S.gg[63] - S.gg[tid]);
        G[kGLog + tid] = S.gg[tid];
        if (tid == 0) G[kGC] = S.gam[63];
    }
}

}  // namespace

hipError_t launch_prep_bf16(const uint16_t* q, const uint16_t* k, const float* a, const float* b,
                            int32_t heads, int32_t max_chunks, const int32_t* rec,
                            const int32_t* num_chunks, unsigned char* factors, int32_t single_T,
                            int32_t* rec_out, int32_t* seq_off_out, int32_t* num_out,
                            hipStream_t stream) {
    if (single_T >= 0) max_chunks = (single_T + kC - 1) / kC;
    const unsigned grid = unsigned(int64_t(max_chunks) * heads);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(prep_bf16_kernel, dim3(grid), dim3(256), 0, stream, q, k, a, b, heads, rec,
                       num_chunks, factors, single_T, rec_out, seq_off_out, num_out);
    return hipGetLastError();
}

}  // namespace rda
