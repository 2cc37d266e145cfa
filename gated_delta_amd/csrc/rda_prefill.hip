// rda_prefill.hip -- chunked prefill of the RDA gated delta rule on gfx950.
//
// The recurrence (decay, error of the value against the decayed state's
// prediction for the key, beta-weighted write, read-out after the update; the
// "Raon-1 nano" teardown, section "The other 1.5B: a hybrid built to forget")
// is evaluated in chunks of C = 64 tokens.  With S the state entering a chunk
// (rows = value channels), g_i the in-chunk running sum of log a and
// gamma_i = exp(g_i):
//
//   L     = strict-lower( diag(b) K K^T * Gamma ),  Gamma_ij = exp(g_i - g_j)
//   T     = (I + L)^-1
//   W     = T diag(b gamma) K ,   U' = T diag(b) V
//   A     = lower( Q K^T * Gamma )
//   Q'    = diag(gamma) Q - A W ,  O' = A U'
//   U     = U' - W S^T                      (the errors each token writes)
//   O     = O' + Q' S^T
//   S_out = gamma_C S + U^T diag(gamma_C / gamma) K
//
// which reproduces the token-by-token recurrence exactly in real arithmetic.
// Everything not involving S is independent per chunk: the PREP kernel
// computes it for all (chunk, head) pairs in parallel and stores W, Q', U',
// O', K and the decay factors in MFMA-ready packed layouts.  The WALK kernel
// then runs the S-dependent part, chunk after chunk, with the state held in
// MFMA accumulator registers: each workgroup owns 16 value channels of one
// (sequence, head) (rows of S evolve independently, so the 8 slices need no
// communication).  Per chunk a walk workgroup does two dependent MFMA GEMMs:
//   X  = [W ; Q'] S_slice^T   (128 x 16, K = 128)
//   S_slice^T = gamma_C S_slice^T + K^T (diag(gamma_C / gamma) U)   (K = 64)
//
// Precision: q, k, v enter MFMA as exact bf16 (fp32 inputs as bf16 hi + lo).
// Every computed fp32 operand (T, A, W, Q', S, U) is fed as a bf16 hi + lo
// pair, and products take hi*hi + hi*lo + lo*hi, i.e. ~2^-16 relative
// accuracy with fp32 accumulation.  The triangular solve and all gate
// arithmetic run in fp32; decay factors are formed only as exp of
// differences g_i - g_j <= 0, so nothing overflows.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (lane l, g = l / 16,
// c = l % 16): A[16 x 32] lane holds row c, k = 8g .. 8g+7; B[32 x 16] lane
// holds column c, k = 8g .. 8g+7; D[16 x 16] lane holds rows 4g .. 4g+3 of
// column c.  Products pair A and B elements held by the same lane group in
// the same register slot, so any permutation of k applied to both operands
// gives the same result.  The kernels use the permutation
//   block m of 32:  lane group g holds k = 32m + 4g + i and 32m + 16 + 4g + i
// which is exactly the union of D-layout rows of tiles 2m and 2m + 1: an
// accumulator tile pair is then a ready B operand with no data movement.
#include "rda_device.h"
#include "rda_internal.h"

namespace rda {

namespace {

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 x) { return __builtin_bit_cast(bf16x8, x); }

// Split 8 fp32 values into bf16 hi and lo vectors.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
    u16x8 h, l;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint16_t a, b;
        split_bf16(x[j], a, b);
        h[j] = a;
        l[j] = b;
    }
    hi = as_bf16x8(h);
    lo = as_bf16x8(l);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// PREP: one 256-thread workgroup per (chunk, head).
// ---------------------------------------------------------------------------
constexpr int kTS = 136;   // bf16 tile row stride (elements): 272 B, spreads LDS banks
constexpr int kFS = 68;    // fp32 64x64 matrix row stride
constexpr int kXS = 132;   // fp32 64x128 staging row stride
constexpr int kTileB = kC * kTS * 2;   // 17408 B
constexpr int kMatB = kC * kFS * 4;    // 17408 B

// LDS layout (bytes).  Ks and Ls are adjacent so the fp32 64 x 128 staging
// buffer Xs can reuse both once K and L are dead.
constexpr int kSmK = 0;
constexpr int kSmL = kSmK + kTileB;
constexpr int kSmQ = kSmL + kMatB;
constexpr int kSmV = kSmQ + kTileB;
constexpr int kSmA = kSmV + kTileB;
constexpr int kSmT = kSmA + kMatB;
constexpr int kSmG = kSmT + kMatB;           // la, bb, gg, gam, bgam: 5 x 64 floats
constexpr int kSmR = kSmG + 5 * 64 * 4;      // 3 x 16x16 fp32 solve scratch
constexpr int kSmLo = kSmR + 3 * 256 * 4;    // lo planes of K, Q, V (fp32 inputs only)
constexpr int kPrepSmemBf16 = kSmLo;
constexpr int kPrepSmemSplit = kSmLo + 3 * kTileB;
static_assert(kC * kXS * 4 <= kTileB + kMatB, "staging buffer must fit over K and L");

template <bool kSplit>
struct PrepIn;
template <>
struct PrepIn<false> { using T = uint16_t; };
template <>
struct PrepIn<true> { using T = float; };

// Stage one [64 x 128] token tile of head h into LDS as bf16 (hi, and lo for
// fp32 inputs).  Rows >= len are zero.
template <bool kSplit>
__device__ __forceinline__ void stage_tile(const typename PrepIn<kSplit>::T* __restrict__ src,
                                           int64_t t0, int len, int H, int h, uint16_t* hi,
                                           uint16_t* lo, int tid) {
    if constexpr (!kSplit) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int p = tid + 256 * qq;
            const int r = p >> 4, c8 = (p & 15) * 8;
            u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
            if (r < len)
                x = *reinterpret_cast<const u16x8*>(src + ((t0 + r) * H + h) * kD + c8);
            *reinterpret_cast<u16x8*>(hi + r * kTS + c8) = x;
        }
    } else {
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
            const int p = tid + 256 * qq;
            const int r = p >> 5, c4 = (p & 31) * 4;
            f32x4 x = zero4();
            if (r < len)
                x = *reinterpret_cast<const f32x4*>(src + ((t0 + r) * H + h) * kD + c4);
            u16x4 xh, xl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint16_t a, b;
                split_bf16(x[j], a, b);
                xh[j] = a;
                xl[j] = b;
            }
            *reinterpret_cast<u16x4*>(hi + r * kTS + c4) = xh;
            *reinterpret_cast<u16x4*>(lo + r * kTS + c4) = xl;
        }
    }
}

// 8 bf16 of column `col` for rows r0 .. r0+7 of a row-major bf16 tile.
__device__ __forceinline__ bf16x8 column8(const uint16_t* tile, int r0, int col) {
    u16x8 x;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = tile[(r0 + j) * kTS + col];
    return as_bf16x8(x);
}

// Column `col`, rows {r0 + i, r0 + 16 + i : i < 4} (the permuted token order).
__device__ __forceinline__ bf16x8 column8_perm(const uint16_t* tile, int r0, int col) {
    u16x8 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = tile[(r0 + i) * kTS + col];
        x[4 + i] = tile[(r0 + 16 + i) * kTS + col];
    }
    return as_bf16x8(x);
}

template <bool kSplit>
__global__ __launch_bounds__(256) void prep_kernel(
    const typename PrepIn<kSplit>::T* __restrict__ q, const typename PrepIn<kSplit>::T* __restrict__ k,
    const typename PrepIn<kSplit>::T* __restrict__ v, const float* __restrict__ a,
    const float* __restrict__ b, int H, const int32_t* __restrict__ rec,
    const int32_t* __restrict__ num_chunks, unsigned char* __restrict__ factors) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kSplit ? kPrepSmemSplit : kPrepSmemBf16];
    const int chunk = blockIdx.x / H;
    const int h = blockIdx.x - chunk * H;
    if (chunk >= num_chunks[0]) return;
    const int64_t t0 = rec[4 * chunk + 1];
    const int len = rec[4 * chunk + 2];

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;

    uint16_t* Ks = reinterpret_cast<uint16_t*>(smem + kSmK);
    uint16_t* Qs = reinterpret_cast<uint16_t*>(smem + kSmQ);
    uint16_t* Vs = reinterpret_cast<uint16_t*>(smem + kSmV);
    uint16_t* Kl = reinterpret_cast<uint16_t*>(smem + kSmLo);
    uint16_t* Ql = Kl + kC * kTS;
    uint16_t* Vl = Ql + kC * kTS;
    float* Ls = reinterpret_cast<float*>(smem + kSmL);
    float* As = reinterpret_cast<float*>(smem + kSmA);
    float* Ts = reinterpret_cast<float*>(smem + kSmT);
    float* Xs = reinterpret_cast<float*>(smem + kSmK);   // aliases Ks + Ls
    float* la = reinterpret_cast<float*>(smem + kSmG);
    float* bb = la + 64;
    float* gg = bb + 64;
    float* gam = gg + 64;
    float* bgam = gam + 64;
    float* Rs = reinterpret_cast<float*>(smem + kSmR);

    unsigned char* F = factors + (size_t(chunk) * H + h) * kChunkHeadBytes;

    // ---- stage inputs; zero T and the upper blocks of A -------------------
    stage_tile<kSplit>(k, t0, len, H, h, Ks, Kl, tid);
    stage_tile<kSplit>(q, t0, len, H, h, Qs, Ql, tid);
    stage_tile<kSplit>(v, t0, len, H, h, Vs, Vl, tid);
    for (int e = tid; e < kC * kFS; e += 256) {
        Ts[e] = 0.f;
        As[e] = 0.f;
    }
    if (w == 0) {
        // gates: log a (clamped far below any fp32-visible decay), prefix sum
        float lav = 0.f, bv = 0.f;
        if (l < len) {
            const size_t th = size_t(t0 + l) * H + h;
            lav = fmaxf(logf(a[th]), -100.f);
            bv = b[th];
        }
        float s = lav;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(s, off, 64);
            if (l >= off) s += o;
        }
        la[l] = lav;
        bb[l] = bv;
        gg[l] = s;
        const float gm = expf(s);
        gam[l] = gm;
        bgam[l] = bv * gm;
    }
    __syncthreads();

    // ---- Gram tiles: L = strict-lower(diag(b) K K^T . Gamma), A = lower(Q K^T . Gamma)
    {
        const int8_t tri[10][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1},
                                   {2, 2}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};
        for (int task = w; task < 20; task += 4) {
            const bool isq = task >= 10;
            const int ti = tri[isq ? task - 10 : task][0];
            const int tj = tri[isq ? task - 10 : task][1];
            const uint16_t* X = isq ? Qs : Ks;
            const uint16_t* Xl = isq ? Ql : Kl;
            f32x4 acc = zero4();
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int kk = 32 * m + 8 * g;
                const bf16x8 ah = *reinterpret_cast<const bf16x8*>(X + (16 * ti + c) * kTS + kk);
                const bf16x8 bh = *reinterpret_cast<const bf16x8*>(Ks + (16 * tj + c) * kTS + kk);
                acc = mfma_bf16(ah, bh, acc);
                if constexpr (kSplit) {
                    const bf16x8 al = *reinterpret_cast<const bf16x8*>(Xl + (16 * ti + c) * kTS + kk);
                    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(Kl + (16 * tj + c) * kTS + kk);
                    acc = mfma_bf16(ah, bl, acc);
                    acc = mfma_bf16(al, bh, acc);
                }
            }
            const int s_ = 16 * tj + c;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * ti + 4 * g + i;
                if (isq) {
                    As[r * kFS + s_] = r >= s_ ? acc[i] * expf(gg[r] - gg[s_]) : 0.f;
                } else {
                    Ls[r * kFS + s_] = r > s_ ? bb[r] * acc[i] * expf(gg[r] - gg[s_]) : 0.f;
                }
            }
        }
    }
    __syncthreads();

    // ---- T = (I + L)^-1 ------------------------------------------------------
    // (a) diagonal 16x16 blocks by forward substitution, one wavefront per block:
    //     lane (column c, part g) keeps x[m] for m = g (mod 4); each row step
    //     sums its part of L[r][m] x[m] and reduces across the four parts.
    {
        const int base = 16 * w;
        float xs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float part = 0.f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int m = 4 * qq + g;
                if (m < r) part += Ls[(base + r) * kFS + base + m] * xs[qq];
            }
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            const float x = (r == c ? 1.f : 0.f) - part;
            if ((r & 3) == g) {
                xs[r >> 2] = x;
                Ts[(base + r) * kFS + base + c] = x;
            }
        }
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

    // ---- W = T diag(b gamma) K  (wave w: key tiles 2w, 2w+1; all token tiles)
    f32x4 accW[4][2];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) accW[ti][0] = accW[ti][1] = zero4();
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int r0 = 32 * m + 8 * g;
        bf16x8 bkh[2], bkl[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            bkh[jj] = column8(Ks, r0, 16 * (2 * w + jj) + c);
            if constexpr (kSplit) bkl[jj] = column8(Kl, r0, 16 * (2 * w + jj) + c);
        }
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(bgam + r0);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(bgam + r0 + 4);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const f32x4 t0v = *reinterpret_cast<const f32x4*>(Ts + (16 * ti + c) * kFS + r0);
            const f32x4 t1v = *reinterpret_cast<const f32x4*>(Ts + (16 * ti + c) * kFS + r0 + 4);
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[j] = t0v[j] * s0[j];
                x[4 + j] = t1v[j] * s1[j];
            }
            bf16x8 ah, al;
            split8(x, ah, al);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                accW[ti][jj] = mfma_bf16(ah, bkh[jj], accW[ti][jj]);
                accW[ti][jj] = mfma_bf16(al, bkh[jj], accW[ti][jj]);
                if constexpr (kSplit) accW[ti][jj] = mfma_bf16(ah, bkl[jj], accW[ti][jj]);
            }
        }
    }

    // ---- K^T packed for the walk's state update (reads Ks before it is reused)
    {
        uint16_t* Kt = reinterpret_cast<uint16_t*>(F + kOffK);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int slot = tid + 256 * qq;
            const int lp = slot & 63, mp = (slot >> 6) & 1, kt = slot >> 7;
            const int col = 16 * kt + (lp & 15), r0 = 32 * mp + 4 * (lp >> 4);
            *reinterpret_cast<bf16x8*>(Kt + slot * 8) = column8_perm(Ks, r0, col);
            if constexpr (kSplit)
                *reinterpret_cast<bf16x8*>(Kt + kC * kD + slot * 8) = column8_perm(Kl, r0, col);
        }
    }

    // ---- Q' = diag(gamma) Q - A W -------------------------------------------
    f32x4 accQ[4][2];
    {
        bf16x8 bwh[2][2], bwl[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = accW[2 * m][jj][i];
                    x[4 + i] = accW[2 * m + 1][jj][i];
                }
                split8(x, bwh[m][jj], bwl[m][jj]);
            }
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            accQ[ti][0] = accQ[ti][1] = zero4();
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const float* arow = As + (16 * ti + c) * kFS + 32 * m + 4 * g;
                const f32x4 a0 = *reinterpret_cast<const f32x4*>(arow);
                const f32x4 a1 = *reinterpret_cast<const f32x4*>(arow + 16);
                float x[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                bf16x8 ah, al;
                split8(x, ah, al);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    accQ[ti][jj] = mfma_bf16(ah, bwh[m][jj], accQ[ti][jj]);
                    accQ[ti][jj] = mfma_bf16(ah, bwl[m][jj], accQ[ti][jj]);
                    accQ[ti][jj] = mfma_bf16(al, bwh[m][jj], accQ[ti][jj]);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * ti + 4 * g + i, kc = 16 * (2 * w + jj) + c;
                    float qv = bf16_bits_to_f32(Qs[r * kTS + kc]);
                    if constexpr (kSplit) qv += bf16_bits_to_f32(Ql[r * kTS + kc]);
                    accQ[ti][jj][i] = gam[r] * qv - accQ[ti][jj][i];
                }
        }
    }
    __syncthreads();   // every wavefront is done with Ks and Ls

    // ---- pack W and Q' for the walk through the fp32 staging buffer ----------
#pragma unroll
    for (int which = 0; which < 2; ++which) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Xs[(16 * ti + 4 * g + i) * kXS + 16 * (2 * w + jj) + c] =
                        which == 0 ? accW[ti][jj][i] : accQ[ti][jj][i];
        __syncthreads();
        uint16_t* P = reinterpret_cast<uint16_t*>(F + (which == 0 ? kOffW : kOffQ));
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int slot = tid + 256 * qq;   // (w', m, lane)
            const int lp = slot & 63, m = (slot >> 6) & 3, wp = slot >> 8;
            const float* row = Xs + (16 * wp + (lp & 15)) * kXS + 32 * m + 4 * (lp >> 4);
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(row);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(row + 16);
            float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            bf16x8 hi, lo;
            split8(x, hi, lo);
            const int base = ((wp * 4 + m) * 2) * 64 + lp;
            *reinterpret_cast<bf16x8*>(P + base * 8) = hi;
            *reinterpret_cast<bf16x8*>(P + (base + 64) * 8) = lo;
        }
        __syncthreads();
    }

    // ---- U' = T diag(b) V and O' = A U'  (wave w: value tiles 2w, 2w+1) -------
    {
        f32x4 accU[4][2];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) accU[ti][0] = accU[ti][1] = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int r0 = 32 * m + 8 * g;
            bf16x8 bvh[2], bvl[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                bvh[jj] = column8(Vs, r0, 16 * (2 * w + jj) + c);
                if constexpr (kSplit) bvl[jj] = column8(Vl, r0, 16 * (2 * w + jj) + c);
            }
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(bb + r0);
            const f32x4 s1 = *reinterpret_cast<const f32x4*>(bb + r0 + 4);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const f32x4 t0v = *reinterpret_cast<const f32x4*>(Ts + (16 * ti + c) * kFS + r0);
                const f32x4 t1v = *reinterpret_cast<const f32x4*>(Ts + (16 * ti + c) * kFS + r0 + 4);
                float x[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = t0v[j] * s0[j];
                    x[4 + j] = t1v[j] * s1[j];
                }
                bf16x8 ah, al;
                split8(x, ah, al);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    accU[ti][jj] = mfma_bf16(ah, bvh[jj], accU[ti][jj]);
                    accU[ti][jj] = mfma_bf16(al, bvh[jj], accU[ti][jj]);
                    if constexpr (kSplit) accU[ti][jj] = mfma_bf16(ah, bvl[jj], accU[ti][jj]);
                }
            }
        }
        f32x4* Up = reinterpret_cast<f32x4*>(F + kOffU);
        f32x4* Op = reinterpret_cast<f32x4*>(F + kOffO);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) Up[((2 * w + jj) * 4 + ti) * 64 + l] = accU[ti][jj];

        bf16x8 buh[2][2], bul[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = accU[2 * m][jj][i];
                    x[4 + i] = accU[2 * m + 1][jj][i];
                }
                split8(x, buh[m][jj], bul[m][jj]);
            }
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            f32x4 accO[2] = {zero4(), zero4()};
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const float* arow = As + (16 * ti + c) * kFS + 32 * m + 4 * g;
                const f32x4 a0 = *reinterpret_cast<const f32x4*>(arow);
                const f32x4 a1 = *reinterpret_cast<const f32x4*>(arow + 16);
                float x[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                bf16x8 ah, al;
                split8(x, ah, al);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    accO[jj] = mfma_bf16(ah, buh[m][jj], accO[jj]);
                    accO[jj] = mfma_bf16(ah, bul[m][jj], accO[jj]);
                    accO[jj] = mfma_bf16(al, buh[m][jj], accO[jj]);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) Op[((2 * w + jj) * 4 + ti) * 64 + l] = accO[jj];
        }
    }

    // ---- decay factors gamma_C / gamma_i = exp(g_C - g_i), and gamma_C --------
    if (tid < 64) {
        float* gs = reinterpret_cast<float*>(F + kOffG);
        gs[tid] = expf(gg[63] - gg[tid]);
        if (tid == 0) gs[64] = gam[63];
    }
}

// ---------------------------------------------------------------------------
// WALK: one 256-thread workgroup per (sequence, head, 16-channel value slice).
// ---------------------------------------------------------------------------
struct WalkOps {
    bf16x8 wh[4], wl[4], qh[4], ql[4];   // A operands of [W ; Q'], k-blocks 0..3
    f32x4 up, op;                        // U', O' for this lane's 4 tokens
    bf16x8 kt[2][2];                     // K^T A operands: key tile 2w+j, token block m
    bf16x8 ktl[2][2];                    // lo planes (fp32 inputs only)
    f32x4 gs;                            // gamma_C / gamma for this lane's 4 tokens
    float gC;
    int t0, len;
};

template <bool kSplit>
__device__ __forceinline__ void walk_load(WalkOps& o, const unsigned char* __restrict__ factors,
                                          const int32_t* __restrict__ rec, int chunk, int H, int h,
                                          int s, int w, int l) {
    const unsigned char* F = factors + (size_t(chunk) * H + h) * kChunkHeadBytes;
    const bf16x8* Wp = reinterpret_cast<const bf16x8*>(F + kOffW);
    const bf16x8* Qp = reinterpret_cast<const bf16x8*>(F + kOffQ);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int base = ((w * 4 + m) * 2) * 64 + l;
        o.wh[m] = Wp[base];
        o.wl[m] = Wp[base + 64];
        o.qh[m] = Qp[base];
        o.ql[m] = Qp[base + 64];
    }
    o.up = reinterpret_cast<const f32x4*>(F + kOffU)[(s * 4 + w) * 64 + l];
    o.op = reinterpret_cast<const f32x4*>(F + kOffO)[(s * 4 + w) * 64 + l];
    const bf16x8* Kt = reinterpret_cast<const bf16x8*>(F + kOffK);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            o.kt[j][m] = Kt[((2 * w + j) * 2 + m) * 64 + l];
            if constexpr (kSplit) o.ktl[j][m] = Kt[1024 + ((2 * w + j) * 2 + m) * 64 + l];
        }
    const float* gs = reinterpret_cast<const float*>(F + kOffG);
    o.gs = *reinterpret_cast<const f32x4*>(gs + 16 * w + 4 * (l >> 4));
    o.gC = gs[64];
    o.t0 = rec[4 * chunk + 1];
    o.len = rec[4 * chunk + 2];
}

template <bool kSplit>
__global__ __launch_bounds__(256) void walk_kernel(int N, int H, const int32_t* __restrict__ rec,
                                                   const int32_t* __restrict__ seq_off,
                                                   const int32_t* __restrict__ num_chunks,
                                                   const unsigned char* __restrict__ factors,
                                                   const float* __restrict__ S0,
                                                   float* __restrict__ o,
                                                   float* __restrict__ S_final) {
    // XCD-aware mapping: the 8 value slices of one (sequence, head) share the
    // same blockIdx.x % 8, hence the same XCD and L2, which holds the chunk
    // factors all 8 of them read.
    const int id = blockIdx.x;
    const int xcd = id & 7, rest = id >> 3;
    const int s = rest & 7, pg = rest >> 3;
    const int p = pg * 8 + xcd;
    if (p >= N * H) return;
    const int n = p / H, h = p - n * H;

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;

    __shared__ __attribute__((aligned(16))) bf16x8 Sx[4][2][64];   // state B operands
    __shared__ __attribute__((aligned(16))) u16x4 Ux[4][2][64];    // scaled U (hi, lo)

    // state: lane holds S^T[k = 32w + 16j + 4g + i][v = 16s + c], i.e.
    // S[v][k .. k+3], a 16-byte run of one state row
    const size_t srow = ((size_t(n) * H + h) * kD + 16 * s + c) * kD;
    f32x4 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        acc[j] = S0 ? *reinterpret_cast<const f32x4*>(S0 + srow + 32 * w + 16 * j + 4 * g) : zero4();

    const int nch = num_chunks[0];
    int c_begin = seq_off[n], c_end = seq_off[n + 1];
    if (c_end > nch) c_end = nch;

    WalkOps cur, nxt;
    if (c_begin < c_end) walk_load<kSplit>(nxt, factors, rec, c_begin, H, h, s, w, l);
    for (int ch = c_begin; ch < c_end; ++ch) {
        cur = nxt;
        if (ch + 1 < c_end) walk_load<kSplit>(nxt, factors, rec, ch + 1, H, h, s, w, l);

        // 1. this wave's state k-block -> hi/lo B operand in LDS
        {
            float x[8] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3],
                          acc[1][0], acc[1][1], acc[1][2], acc[1][3]};
            bf16x8 hi, lo;
            split8(x, hi, lo);
            Sx[w][0][l] = hi;
            Sx[w][1][l] = lo;
        }
        __syncthreads();

        // 2. X = [W ; Q'] S^T for this wave's token tile
        f32x4 xw = zero4(), xq = zero4();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x8 bh = Sx[m][0][l], bl = Sx[m][1][l];
            xw = mfma_bf16(cur.wh[m], bh, xw);
            xq = mfma_bf16(cur.qh[m], bh, xq);
            xw = mfma_bf16(cur.wh[m], bl, xw);
            xq = mfma_bf16(cur.qh[m], bl, xq);
            xw = mfma_bf16(cur.wl[m], bh, xw);
            xq = mfma_bf16(cur.ql[m], bh, xq);
        }

        // 3. outputs and the scaled errors
        u16x4 uh, ul;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 16 * w + 4 * g + i;
            const float u = cur.up[i] - xw[i];
            const float ov = cur.op[i] + xq[i];
            if (tok < cur.len) o[((size_t(cur.t0) + tok) * H + h) * kD + 16 * s + c] = ov;
            uint16_t hb, lb;
            split_bf16(u * cur.gs[i], hb, lb);
            uh[i] = hb;
            ul[i] = lb;
        }
        Ux[w][0][l] = uh;
        Ux[w][1][l] = ul;
        __syncthreads();

        // 4. S^T = gamma_C S^T + K^T U~  (this wave's two key tiles)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc[j] *= cur.gC;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const u16x4 h0 = Ux[2 * m][0][l], h1 = Ux[2 * m + 1][0][l];
                const u16x4 l0 = Ux[2 * m][1][l], l1 = Ux[2 * m + 1][1][l];
                const bf16x8 bh = as_bf16x8(u16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]});
                const bf16x8 bl = as_bf16x8(u16x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]});
                acc[j] = mfma_bf16(cur.kt[j][m], bh, acc[j]);
                acc[j] = mfma_bf16(cur.kt[j][m], bl, acc[j]);
                if constexpr (kSplit) acc[j] = mfma_bf16(cur.ktl[j][m], bh, acc[j]);
            }
        }
    }
    if (S_final) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            *reinterpret_cast<f32x4*>(S_final + srow + 32 * w + 16 * j + 4 * g) = acc[j];
    }
}

}  // namespace

hipError_t launch_prep(const void* q, const void* k, const void* v, rda_dtype dt, const float* a,
                       const float* b, int32_t heads, int32_t max_chunks, const int32_t* rec,
                       const int32_t* num_chunks, unsigned char* factors, hipStream_t stream) {
    const unsigned grid = unsigned(int64_t(max_chunks) * heads);
    if (grid == 0) return hipSuccess;
    if (dt == RDA_BF16) {
        hipLaunchKernelGGL(prep_kernel<false>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), a, b, heads, rec, num_chunks, factors);
    } else {
        hipLaunchKernelGGL(prep_kernel<true>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), a, b, heads, rec, num_chunks, factors);
    }
    return hipGetLastError();
}

hipError_t launch_walk(rda_dtype dt, int32_t num_seqs, int32_t heads, const int32_t* rec,
                       const int32_t* seq_off, const int32_t* num_chunks,
                       const unsigned char* factors, const float* S0, float* o, float* S_final,
                       hipStream_t stream) {
    const int64_t pairs = int64_t(num_seqs) * heads;
    const unsigned grid = unsigned(64 * ((pairs + 7) / 8));
    if (dt == RDA_BF16) {
        hipLaunchKernelGGL(walk_kernel<false>, dim3(grid), dim3(256), 0, stream, num_seqs, heads,
                           rec, seq_off, num_chunks, factors, S0, o, S_final);
    } else {
        hipLaunchKernelGGL(walk_kernel<true>, dim3(grid), dim3(256), 0, stream, num_seqs, heads,
                           rec, seq_off, num_chunks, factors, S0, o, S_final);
    }
    return hipGetLastError();
}

}  // namespace rda
