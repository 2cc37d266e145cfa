// rda_prefill_diag.hip -- chunked prefill of the gated delta rule with a
// per-key-channel (diagonal) decay, on gfx950.
//
// The decay alpha_t in (0,1]^dk scales column j of the state by alpha_tj
// before the error is taken (the Raon-1 mini vLLM article calls RDA a
// modification of Kimi Delta Attention, whose decay is per channel; the
// tiny-model card prints a low-rank decay projection whose output has the
// heads' key width).  Per chunk of C = 64 tokens, with S the entering state,
// G_i the in-chunk running sum of log alpha (a vector over key channels) and
// e^{G_i - G_j} taken per channel:
//
//   L_ij  = b_i sum_c k_ic k_jc e^{G_ic - G_jc}   (j < i),   T = (I + L)^-1
//   A_ij  = sum_c q_ic k_jc e^{G_ic - G_jc}       (j <= i),  T_b = T diag(b)
//   E     = V - (K . e^G) S^T                     (errors against the decayed state)
//   U     = T_b E
//   O     = (Q . e^G) S^T + A U
//   S_out = S diag(e^{G_C}) + U^T (K . e^{G_C - G})
//
// with . the elementwise product row by row.  This reduces to the scalar
// chunk algebra when alpha is equal on every channel, and reproduces the
// token-by-token recurrence in real arithmetic.
//
// PREP (parallel over chunk x head, 16 waves): G, the three decayed operands
// K e^G, Q e^G and (K e^{G_C - G})^T packed as bf16 hi/lo MFMA operands,
// L and A, the solve, T_b and A packed.  L and A are built from 16 x 16
// sub-blocks on MFMA, each factored through a reference token r so that no
// factor can overflow: a block of sub-chunk I against an earlier sub-chunk J
// uses r = the last token of J, so e^{G_i - G_r} <= 1 and e^{G_r - G_j} <= 1;
// a diagonal block uses r = its first token, so e^{G_i - G_r} <= 1 and
// e^{G_r - G_j} >= 1 is at most the decay across the block -- when that
// exceeds e^60 on some channel (possible only for decays below e^-3.75 per
// token), the block is computed elementwise with exact exponents instead.
//
// WALK (sequential over the chunks of a sequence): one 8-wave workgroup per
// (sequence, head, 16-channel value slice).  Wave w keeps the state's key
// tile w (16 keys x 16 values) in an MFMA accumulator.  Every operand comes
// pre-packed from the prep, so each wave loads its MFMA operands straight
// into registers, two chunks ahead; LDS only carries the state, the errors
// and U between waves.  Per chunk, wave tt = w % 4:
//   P1  every wave publishes its state tile (bf16 hi/lo B operand)
//   P2  waves 0-3: Y = (K e^G)[tt] S^T, E = V - Y published;
//       waves 4-7: Z = (Q e^G)[tt] S^T
//   P3  waves 0-3: U = T_b[tt] E, published
//   P4  every wave: S^T = diag(e^{G_C}) S^T + (K e^{G_C - G})^T U for its
//       key tile; waves 4-7: O = Z + A[tt] U, stored
// Three barriers per chunk.  Products of computed operands take hi*hi +
// hi*lo + lo*hi (about 2^-16 relative) with fp32 accumulation.
#include "rda_device.h"
#include "rda_internal.h"
#include "rda_solve.h"

namespace rda {
namespace {

constexpr int kKS = 136;                // bf16 K / Q tile row stride in the prep
constexpr int kGS = 129;                // fp32 G row stride in the prep
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kSpanMax = 60.f * kLog2e;   // largest diagonal-block span in log2 units

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

struct PrepDiagLds {
    uint16_t K[kC][kKS];
    uint16_t Q[kC][kKS];
    float G[kC][kGS];        // running sum of log2(alpha) per key channel
    float Gtot[8][kD];       // each eighth of the chunk's own sum per channel
    float L[kC * kFS];
    float A[kC * kFS];
    float T[kC * kFS];
    float bb[kC];
    float R[3 * 256];
    int exact[4];            // diagonal block J needs the elementwise form
};

// 8 values of a row of X . 2^(GL[row] - GL[ref]) at the permuted keys of k
// block m (32m + 4g + i and 32m + 16 + 4g + i), as bf16 hi / lo
__device__ __forceinline__ void scaled_keys(const PrepDiagLds& S, const uint16_t (*X)[kKS], int row,
                                            int ref, int m, int g, bool ref_minus_row,
                                            bf16x8& hi, bf16x8& lo) {
    float v[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 32 * m + 16 * hh + 4 * g + i;
            const float d = ref_minus_row ? S.G[ref][key] - S.G[row][key]
                                          : S.G[row][key] - S.G[ref][key];
            v[4 * hh + i] = bf16_bits_to_f32(X[row][key]) * exp2_hw(d);
        }
    split8(v, hi, lo);
}

constexpr int kPrepThreads = 1024;
constexpr int64_t kPrepDiagGrid = 256;

__global__ __launch_bounds__(kPrepThreads) void prep_diag_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ b, int H, const int32_t* __restrict__ rec,
    const int32_t* __restrict__ num_chunks, unsigned char* __restrict__ factors) {
    __shared__ __attribute__((aligned(16))) PrepDiagLds S;
    // Persistent: the workgroup takes items (chunk, head) blockIdx.x,
    // blockIdx.x + gridDim.x, ... and loads the next item's inputs into
    // registers while it works on the current one (one workgroup fills a CU,
    // so nothing else would hide that load's latency).
    const int total = num_chunks[0] * H;
    int item = blockIdx.x;
    if (item >= total) return;

    // K, Q rows, b, and alpha for (channel, eighth of 8 tokens) of one item;
    // rows past the chunk's end read as zero keys, b = 0 and alpha = 1
    u16x8 xk, xq;
    float bv, al[8];
    auto load_item = [&](int it) {
        const int tid = threadIdx.x;
        const int sr = tid >> 4, sc8 = (tid & 15) * 8;
        const int ch = tid & 127, qt = tid >> 7;
        const int ck = it / H, hh = it - ck * H;
        const int64_t s0 = rec[4 * ck + 1];
        const int n = rec[4 * ck + 2];
        xk = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        xq = xk;
        if (sr < n) {
            xk = *reinterpret_cast<const u16x8*>(k + ((s0 + sr) * H + hh) * kD + sc8);
            xq = *reinterpret_cast<const u16x8*>(q + ((s0 + sr) * H + hh) * kD + sc8);
        }
        bv = tid < n ? b[(s0 + tid) * H + hh] : 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int row = 8 * qt + r;
            al[r] = row < n ? alpha[((s0 + row) * H + hh) * kD + ch] : 1.f;
        }
    };
    load_item(item);
    for (;;) {
    // the lane's indices, opaque to the compiler on every item, so that
    // nothing derived from them is kept live across items
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int w = wave_id(), l = tid & 63, g = l >> 4, c = l & 15;
    const int sr = tid >> 4, sc8 = (tid & 15) * 8;
    const int ch = tid & 127, qt = tid >> 7;
    const int chunk = item / H;
    const int h = item - chunk * H;
    unsigned char* F = factors + (size_t(chunk) * H + h) * kDiagChunkHeadBytes;
    const int next = item + int(gridDim.x);
    // ---- stage K, Q (rows past the chunk's end are zero), b; zero T and A;
    //      G = running sum of log2(alpha) per channel, each eighth of the
    //      chunk first on its own, then offset by the eighths before it
    *reinterpret_cast<u16x8*>(&S.K[sr][sc8]) = xk;
    *reinterpret_cast<u16x8*>(&S.Q[sr][sc8]) = xq;
    if (tid < kC) S.bb[tid] = bv;
    for (int e = tid; e < kC * kFS; e += kPrepThreads) {
        S.T[e] = 0.f;
        S.A[e] = 0.f;
    }
    {
        float run[8];
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            // beyond any fp32-visible decay; keeps G finite
            acc += fmaxf(__builtin_amdgcn_logf(al[r]), -1000.f);
            run[r] = acc;
        }
        S.Gtot[qt][ch] = acc;
        // this item's inputs are in LDS or registers: the next item's loads go out now
        if (next < total) load_item(next);
        __syncthreads();
        float base = 0.f;
        for (int p = 0; p < qt; ++p) base += S.Gtot[p][ch];
#pragma unroll
        for (int r = 0; r < 8; ++r) S.G[8 * qt + r][ch] = qt > 0 ? run[r] + base : run[r];
    }
    __syncthreads();
    // diagonal block w: is the decay across it within e^60 on every channel?
    if (w < 4) {
        float span = 0.f;
        for (int ch = l; ch < kD; ch += 64)
            span = fmaxf(span, S.G[16 * w][ch] - S.G[16 * w + 15][ch]);
        for (int off = 32; off > 0; off >>= 1) span = fmaxf(span, __shfl_xor(span, off, 64));
        if (l == 0) S.exact[w] = span > kSpanMax ? 1 : 0;
    }

    // the exact-path flags are read by every Gram task
    __syncthreads();

    // ---- L and A from 16 x 16 sub-blocks: one task per block (I >= J) forms
    //      both, sharing the scaled key rows of block J --------------------
    if (w < 10) {
        const int I = (w >= 1) + (w >= 3) + (w >= 6);
        const int J = w - I * (I + 1) / 2;
        f32x4 accL = zero4(), accA = zero4();
        if (I > J || !S.exact[J]) {
            const int ref = I > J ? 16 * J + 15 : 16 * J;
            f32x4 l0 = zero4(), l1 = zero4(), l2 = zero4();
            f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4();
#pragma unroll 2
            for (int m = 0; m < 4; ++m) {
                bf16x8 bh, bl, xh, xl;
                scaled_keys(S, S.K, 16 * J + c, ref, m, g, true, bh, bl);
                scaled_keys(S, S.K, 16 * I + c, ref, m, g, false, xh, xl);
                l0 = mfma_bf16(xh, bh, l0);
                l1 = mfma_bf16(xh, bl, l1);
                l2 = mfma_bf16(xl, bh, l2);
                scaled_keys(S, S.Q, 16 * I + c, ref, m, g, false, xh, xl);
                a0 = mfma_bf16(xh, bh, a0);
                a1 = mfma_bf16(xh, bl, a1);
                a2 = mfma_bf16(xl, bh, a2);
            }
            accL = l0 + l1 + l2;
            accA = a0 + a1 + a2;
        } else {
            // exact: every factor e^{G_i - G_j} <= 1 formed on its own
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ri = 16 * I + 4 * g + i, sj = 16 * J + c;
                float sl = 0.f, sa = 0.f;
                if (ri >= sj)
                    for (int key = 0; key < kD; ++key) {
                        const float kj = bf16_bits_to_f32(S.K[sj][key]) *
                                         exp2_hw(S.G[ri][key] - S.G[sj][key]);
                        sl = fmaf(bf16_bits_to_f32(S.K[ri][key]), kj, sl);
                        sa = fmaf(bf16_bits_to_f32(S.Q[ri][key]), kj, sa);
                    }
                accL[i] = sl;
                accA[i] = sa;
            }
        }
        const int sj = 16 * J + c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ri = 16 * I + 4 * g + i;
            S.A[ri * kFS + sj] = ri >= sj ? accA[i] : 0.f;
            S.L[ri * kFS + sj] = ri > sj ? S.bb[ri] * accL[i] : 0.f;
        }
    } else {
        // ---- the other 6 waves meanwhile: decayed operands, packed for the
        //      walk (global stores only, so no barrier between the two) ----
        bf16x8* Kt = reinterpret_cast<bf16x8*>(F + kDOffKt);
        bf16x8* Qt = reinterpret_cast<bf16x8*>(F + kDOffQt);
        bf16x8* Kh = reinterpret_cast<bf16x8*>(F + kDOffKh);
        for (int idx = tid - 640; idx < 1024; idx += 384) {
            // (K e^G), (Q e^G): slot (token tile tt, key block m): row 16tt + lane % 16
            const int lp = idx & 63, m = (idx >> 6) & 3, tt = idx >> 8, gp = lp >> 4;
            const int row = 16 * tt + (lp & 15);
            float vk[8], vq[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 32 * m + 16 * hh + 4 * gp + i;
                    const float e = exp2_hw(S.G[row][key]);
                    vk[4 * hh + i] = bf16_bits_to_f32(S.K[row][key]) * e;
                    vq[4 * hh + i] = bf16_bits_to_f32(S.Q[row][key]) * e;
                }
            bf16x8 hk, lk, hq, lq;
            split8(vk, hk, lk);
            split8(vq, hq, lq);
            const int base = ((tt * 4 + m) * 2) * 64 + lp;
            Kt[base] = hk;
            Kt[base + 64] = lk;
            Qt[base] = hq;
            Qt[base + 64] = lq;
        }
        for (int idx = tid - 640; idx < 1024; idx += 384) {
            // (K e^{G_C - G})^T: slot (key tile kt, token block m): key 16kt + lane % 16
            const int lp = idx & 63, m = (idx >> 6) & 1, kt = idx >> 7, gp = lp >> 4;
            const int key = 16 * kt + (lp & 15);
            const float gc = S.G[kC - 1][key];
            float v[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = 32 * m + 16 * hh + 4 * gp + i;
                    v[4 * hh + i] = bf16_bits_to_f32(S.K[tok][key]) * exp2_hw(gc - S.G[tok][key]);
                }
            bf16x8 hi, lo;
            split8(v, hi, lo);
            const int base = ((kt * 2 + m) * 2) * 64 + lp;
            Kh[base] = hi;
            Kh[base + 64] = lo;
        }
        for (int e = tid - 640; e < kD; e += 384)
            reinterpret_cast<float*>(F + kDOffGC)[e] = exp2_hw(S.G[kC - 1][e]);
    }
    __syncthreads();

    // ---- T = (I + L)^-1, then T_b and A packed -------------------------------
    solve_unit_lower(S.L, S.T, S.R, w, g, c);
    if (tid < 256) pack_rows(S.T, S.bb, reinterpret_cast<bf16x8*>(F + kDOffTb), tid);
    else if (tid < 512) pack_rows(S.A, nullptr, reinterpret_cast<bf16x8*>(F + kDOffA), tid - 256);
    if (next >= total) break;
    item = next;
    __syncthreads();   // T, A and the staged rows are rewritten next
    }
}

// ---------------------------------------------------------------------------
// WALK
// ---------------------------------------------------------------------------
constexpr int kDWaves = 8;

// One wave's operands of one chunk.
struct DiagOps {
    bf16x8 xa[4][2];   // (K e^G) (waves 0-3) or (Q e^G) (waves 4-7), token tile tt: [key block][hi/lo]
    bf16x8 fa[2][2];   // T_b (waves 0-3) or A (waves 4-7), token tile tt: [token block][hi/lo]
    bf16x8 kh[2][2];   // (K e^{G_C - G})^T, key tile w: [token block][hi/lo]
    f32x4 gc;          // e^{G_C} of keys 16w + 4g .. +3
    uint16_t vraw[4];  // V at tokens 16tt + 4g + i, value 16s + c (waves 0-3), bf16 bits:
                       // widened where used, so the prefetch is never waited on here
    int t0, len;
};

// The chunks of one sequence are consecutive and full but for the last, so
// a chunk's first token and length follow from the first chunk's start and
// the sequence's end without a dependent load in the chunk loop.
struct DiagCtx {
    const uint16_t* v;
    const unsigned char* factors;
    int H, h, s, w, l;
    int c_begin, t_begin, t_end;
};

__device__ __forceinline__ const unsigned char* diag_factors(const DiagCtx& x, int chunk) {
    return x.factors + (size_t(chunk) * x.H + x.h) * kDiagChunkHeadBytes;
}

__device__ __forceinline__ void load_xa(DiagOps& o, const DiagCtx& x, int chunk) {
    const bf16x8* P =
        reinterpret_cast<const bf16x8*>(diag_factors(x, chunk) + (x.w < 4 ? kDOffKt : kDOffQt));
    const int tt = x.w & 3;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int base = ((tt * 4 + m) * 2) * 64 + x.l;
        o.xa[m][0] = P[base];
        o.xa[m][1] = P[base + 64];
    }
}

__device__ __forceinline__ void load_fa(DiagOps& o, const DiagCtx& x, int chunk) {
    const bf16x8* P =
        reinterpret_cast<const bf16x8*>(diag_factors(x, chunk) + (x.w < 4 ? kDOffTb : kDOffA));
    const int tt = x.w & 3;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int base = ((tt * 2 + m) * 2) * 64 + x.l;
        o.fa[m][0] = P[base];
        o.fa[m][1] = P[base + 64];
    }
}

__device__ __forceinline__ void load_kh(DiagOps& o, const DiagCtx& x, int chunk) {
    const unsigned char* F = diag_factors(x, chunk);
    const bf16x8* P = reinterpret_cast<const bf16x8*>(F + kDOffKh);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int base = ((x.w * 2 + m) * 2) * 64 + x.l;
        o.kh[m][0] = P[base];
        o.kh[m][1] = P[base + 64];
    }
    o.gc = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(F + kDOffGC) +
                                           16 * x.w + 4 * (x.l >> 4));
}

__device__ __forceinline__ void load_rec_v(DiagOps& o, const DiagCtx& x, int chunk) {
    o.t0 = x.t_begin + kC * (chunk - x.c_begin);
    o.len = min(kC, x.t_end - o.t0);
    // every wave loads (output waves do not use it): the same loads in the same
    // order in every wave keeps the compiler's load counting exact
    const int tt = x.w & 3, g = x.l >> 4, c = x.l & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * tt + 4 * g + i;
        const int rr = r < o.len ? r : o.len - 1;   // rows past the end: any valid row
        o.vraw[i] = x.v[((size_t(o.t0) + rr) * x.H + x.h) * kD + 16 * x.s + c];
    }
}

// the order of the in-loop refills, so the pending loads at the loop head are
// the same on entry and on the back edge
__device__ __forceinline__ void load_all(DiagOps& o, const DiagCtx& x, int chunk) {
    load_xa(o, x, chunk);
    load_fa(o, x, chunk);
    load_kh(o, x, chunk);
    load_rec_v(o, x, chunk);
}

struct DiagLds {
    u32x4 Sx[4][2][64];   // state tiles (hi/lo) as B operands, key blocks 0..3
    u32x4 Ex[2][2][64];   // E (hi/lo), token blocks 0, 1
    u32x4 Ux[2][2][64];   // U (hi/lo)
};

__device__ __forceinline__ void put_half(u32x4 (*X)[2][64], int tile, int l, u32x2 hi, u32x2 lo) {
    u32x2* hp = reinterpret_cast<u32x2*>(&X[tile >> 1][0][l]) + (tile & 1);
    u32x2* lp = reinterpret_cast<u32x2*>(&X[tile >> 1][1][l]) + (tile & 1);
    *hp = hi;
    *lp = lo;
}

__device__ __forceinline__ void publish4(u32x4 (*X)[2][64], int tile, int l, f32x4 v) {
    uint32_t h01, l01, h23, l23;
    split_pk(v[0], v[1], h01, l01);
    split_pk(v[2], v[3], h23, l23);
    put_half(X, tile, l, u32x2{h01, h23}, u32x2{l01, l23});
}

__device__ __forceinline__ bf16x8 ldsop(u32x4 (*X)[2][64], int blk, int hl, int l) {
    return __builtin_bit_cast(bf16x8, X[blk][hl][l]);
}

// hi*hi + hi*lo + lo*hi over `nb` k blocks: A from registers, B from LDS
template <int nb>
__device__ __forceinline__ f32x4 prod3(const bf16x8 (*a)[2], u32x4 (*B)[2][64], int l) {
    f32x4 p0 = zero4(), p1 = zero4(), p2 = zero4();
#pragma unroll
    for (int m = 0; m < nb; ++m) {
        const bf16x8 bh = ldsop(B, m, 0, l), bl = ldsop(B, m, 1, l);
        p0 = mfma_bf16(a[m][0], bh, p0);
        p1 = mfma_bf16(a[m][0], bl, p1);
        p2 = mfma_bf16(a[m][1], bh, p2);
    }
    return p0 + p1 + p2;
}

// One chunk; `cur` holds its operands and is refilled with chunk `next`
// as each part is consumed.  Without outputs (kOut false) the output waves
// only carry their state tiles; zero_v takes every value as zero (the walk
// then applies the chunks' transition alone).
template <bool kOut>
__device__ __forceinline__ void diag_step(DiagOps& cur, f32x4& acc, const DiagCtx& x, int next,
                                          DiagLds& S, float* __restrict__ o, bool zero_v) {
    const int w = x.w, l = x.l, g = l >> 4, c = l & 15, tt = w & 3;
    const bool state = w < 4;
    // P1
    publish4(S.Sx, w, l, acc);
    __syncthreads();
    // P2
    f32x4 yz = zero4();
    if (kOut || state) yz = prod3<4>(cur.xa, S.Sx, l);
    if (state) {
        const f32x4 vv = zero_v ? zero4()
                                : f32x4{bf16_bits_to_f32(cur.vraw[0]), bf16_bits_to_f32(cur.vraw[1]),
                                        bf16_bits_to_f32(cur.vraw[2]),
                                        bf16_bits_to_f32(cur.vraw[3])};
        publish4(S.Ex, tt, l, vv - yz);
    }
    load_xa(cur, x, next);
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch here: never sink it to its use
    __syncthreads();
    // P3
    if (state) publish4(S.Ux, tt, l, prod3<2>(cur.fa, S.Ex, l));
    __syncthreads();
    // P4
    const f32x4 upd = prod3<2>(cur.kh, S.Ux, l);
    acc = acc * cur.gc + upd;
    if (kOut && !state) {
        const f32x4 ov = yz + prod3<2>(cur.fa, S.Ux, l);
        const int t0 = cur.t0, len = cur.len;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 16 * tt + 4 * g + i;
            if (tok < len) o[((size_t(t0) + tok) * x.H + x.h) * kD + 16 * x.s + c] = ov[i];
        }
    }
    load_fa(cur, x, next);
    load_kh(cur, x, next);
    load_rec_v(cur, x, next);
    __builtin_amdgcn_sched_barrier(0);
}

template <bool kOut>
__global__ __launch_bounds__(kDWaves * 64) void walk_diag_kernel(
    const uint16_t* __restrict__ v, int N, int H, const int32_t* __restrict__ rec,
    const int32_t* __restrict__ seq_off, const int32_t* __restrict__ num_chunks,
    const unsigned char* __restrict__ factors, float* __restrict__ o, WalkJob j0, WalkJob j1,
    int seg_chunks) {
    // Jobs split the grid in halves.  Within a job the mapping is XCD-aware:
    // the 8 value slices of one (sequence, head) share the same
    // blockIdx.x % 8, hence one XCD and its L2, which holds the chunk
    // operands all 8 of them read.
    const int per_job = 64 * ((N * H + 7) / 8);
    const int job = blockIdx.x >= per_job ? 1 : 0;
    const WalkJob J = job ? j1 : j0;
    const int id = blockIdx.x - job * per_job;
    const int xcd = id & 7, rest = id >> 3;
    const int s = rest & 7, pg = rest >> 3;
    const int p = pg * 8 + xcd;
    if (p >= N * H) return;
    const int n = p / H, h = p - n * H;
    const int tid = threadIdx.x;
    const int w = wave_id(), l = tid & 63, g = l >> 4, c = l & 15;
    __shared__ __attribute__((aligned(16))) DiagLds lds;

    // sequence n's chunks: from the table, or the n-th run of seg_chunks
    const int nch = num_chunks[0];
    int c_begin, c_end;
    if (seg_chunks > 0) {
        c_begin = n * seg_chunks < nch ? n * seg_chunks : nch;
        c_end = c_begin + seg_chunks < nch ? c_begin + seg_chunks : nch;
    } else {
        c_begin = seq_off[n];
        c_end = seq_off[n + 1] < nch ? seq_off[n + 1] : nch;
    }
    int t_begin = 0, t_end = 0;
    if (c_begin < c_end) {
        t_begin = rec[4 * c_begin + 1];
        t_end = rec[4 * (c_end - 1) + 1] + rec[4 * (c_end - 1) + 2];
    }
    const DiagCtx x{v, factors, H, h, s, w, l, c_begin, t_begin, t_end};

    // state: lane holds S^T[key 16w + 4g + i][value 16s + c] = S[value][key .. key+3]
    const size_t srow = ((size_t(n) * H + h) * kD + 16 * s + c) * kD + 16 * w + 4 * g;
    f32x4 acc = zero4();
    if (J.identity) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = 16 * w + 4 * g + i == 16 * s + c ? 1.f : 0.f;
    } else if (J.S0) {
        acc = *reinterpret_cast<const f32x4*>(J.S0 + srow);
    }
    const bool zero_v = J.zero_v != 0;
    if (c_begin < c_end) {
        // two operand sets in turn, a pair of chunks per iteration (no exit
        // between the two steps, so the loads pending at the loop head are
        // the same on every path and the compiler's waits stay exact), and
        // an odd last chunk after the loop
        DiagOps A, B;
        const int last = c_end - 1;
        load_all(A, x, c_begin);
        load_all(B, x, c_begin + 1 < c_end ? c_begin + 1 : last);
        int ch = c_begin;
        for (; ch + 1 < c_end; ch += 2) {
            diag_step<kOut>(A, acc, x, ch + 2 < c_end ? ch + 2 : last, lds, o, zero_v);
            diag_step<kOut>(B, acc, x, ch + 3 < c_end ? ch + 3 : last, lds, o, zero_v);
        }
        if (ch < c_end) diag_step<kOut>(A, acc, x, last, lds, o, zero_v);
    }
    if (J.S_final) *reinterpret_cast<f32x4*>(J.S_final + srow) = acc;
}

}  // namespace

hipError_t launch_prep_diag(const uint16_t* q, const uint16_t* k, const float* alpha,
                            const float* b, int32_t heads, int32_t max_chunks, const int32_t* rec,
                            const int32_t* num_chunks, unsigned char* factors,
                            hipStream_t stream) {
    // one persistent workgroup per CU at most (each holds a CU's LDS)
    const int64_t items = int64_t(max_chunks) * heads;
    const unsigned pgrid = unsigned(items < kPrepDiagGrid ? items : kPrepDiagGrid);
    if (pgrid == 0) return hipSuccess;
    hipLaunchKernelGGL(prep_diag_kernel, dim3(pgrid), dim3(kPrepThreads), 0, stream, q, k, alpha,
                       b, heads, rec, num_chunks, factors);
    return hipGetLastError();
}

hipError_t launch_walk_diag(const uint16_t* v, int32_t num_seqs, int32_t heads,
                            const int32_t* rec, const int32_t* seq_off,
                            const int32_t* num_chunks, const unsigned char* factors, float* o,
                            const WalkJob* jobs, int32_t num_jobs, int32_t seg_chunks,
                            bool outputs, hipStream_t stream) {
    const int64_t pairs = int64_t(num_seqs) * heads;
    const unsigned wgrid = unsigned(num_jobs * 64 * ((pairs + 7) / 8));
    const WalkJob none{nullptr, nullptr, 0, 0};
    const WalkJob j1 = num_jobs > 1 ? jobs[1] : none;
    if (outputs)
        hipLaunchKernelGGL(walk_diag_kernel<true>, dim3(wgrid), dim3(kDWaves * 64), 0, stream, v,
                           num_seqs, heads, rec, seq_off, num_chunks, factors, o, jobs[0], j1,
                           seg_chunks);
    else
        hipLaunchKernelGGL(walk_diag_kernel<false>, dim3(wgrid), dim3(kDWaves * 64), 0, stream,
                           v, num_seqs, heads, rec, seq_off, num_chunks, factors, o, jobs[0], j1,
                           seg_chunks);
    return hipGetLastError();
}

hipError_t launch_prefill_diag(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const float* alpha, const float* b, int32_t num_seqs,
                               int32_t heads, int32_t max_chunks, const int32_t* rec,
                               const int32_t* seq_off, const int32_t* num_chunks,
                               unsigned char* factors, const float* S0, float* o,
                               float* S_final, hipStream_t stream) {
    const hipError_t err =
        launch_prep_diag(q, k, alpha, b, heads, max_chunks, rec, num_chunks, factors, stream);
    if (err != hipSuccess) return err;
    const WalkJob job{S0, S_final, 0, 0};
    return launch_walk_diag(v, num_seqs, heads, rec, seq_off, num_chunks, factors, o, &job, 1, 0,
                            true, stream);
}

}  // namespace rda
