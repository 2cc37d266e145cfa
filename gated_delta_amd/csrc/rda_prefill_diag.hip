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
// WALK (sequential over the chunks of a sequence): one 16-wave workgroup per
// (sequence, head, 16-channel value slice).  Compute wave w (0..7) keeps
// the state's key tile w (16 keys x 16 values) in an MFMA accumulator; eight
// loader waves stream every operand the prep packed into LDS with LDS-DMA,
// so the compute waves issue no global loads.  The chunk's operands do not
// fit twice in LDS (130 KiB), so they are held once, in three parts that
// are each streamed for the next chunk right after the barrier that ends
// their last read: the decayed K and Q tiles and V after barrier B, T_b
// after barrier C, (K e^{G_C - G})^T, A and e^{G_C} after the next chunk's
// barrier A.  Loaders 0 and 1 also touch the factor lines four chunks ahead
// so that they sit in L2 when the DMA asks for them.  Per chunk, wave
// tt = w % 4:
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
#include "rda_lds.h"
#include "rda_solve.h"

namespace rda {
namespace {

// K / Q tile row stride in the prep (elements): 136 bf16 or 132 fp32, both
// 4 banks apart from row to row
template <typename TIn>
constexpr int kKS = sizeof(TIn) == 2 ? 136 : 132;
constexpr int kGS = 129;                // fp32 G row stride in the prep
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kSpanMax = 60.f * kLog2e;   // largest diagonal-block span in log2 units

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// an input element as fp32 (bf16 bits, or fp32 as it is)
__device__ __forceinline__ float in_f32(uint16_t x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ float in_f32(float x) { return x; }

// K and Q staged in their input type: bf16 (124.5 KiB in all) or fp32
// (156.5 KiB), so that fp32 inputs enter every product at full precision
template <typename TIn>
struct PrepDiagLds {
    TIn K[kC][kKS<TIn>];
    TIn Q[kC][kKS<TIn>];
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
template <typename TIn>
__device__ __forceinline__ void scaled_keys(const PrepDiagLds<TIn>& S, const TIn (*X)[kKS<TIn>],
                                            int row, int ref, int m, int g, bool ref_minus_row,
                                            bf16x8& hi, bf16x8& lo) {
    float v[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 32 * m + 16 * hh + 4 * g + i;
            const float d = ref_minus_row ? S.G[ref][key] - S.G[row][key]
                                          : S.G[row][key] - S.G[ref][key];
            v[4 * hh + i] = in_f32(X[row][key]) * exp2_hw(d);
        }
    split8(v, hi, lo);
}

constexpr int kPrepThreads = 1024;
constexpr int64_t kPrepDiagGrid = 256;

static_assert(sizeof(PrepDiagLds<float>) <= 160 * 1024, "LDS budget of one workgroup");

// 8 consecutive input elements of a row, as loaded (bf16 bits or fp32)
template <typename TIn>
struct Row8;
template <>
struct Row8<uint16_t> {
    u16x8 d;
    __device__ __forceinline__ void zero() { d = u16x8{0, 0, 0, 0, 0, 0, 0, 0}; }
    __device__ __forceinline__ void load(const uint16_t* p) { d = *reinterpret_cast<const u16x8*>(p); }
    __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<u16x8*>(p) = d; }
};
template <>
struct Row8<float> {
    f32x4 d0, d1;
    __device__ __forceinline__ void zero() { d0 = zero4(); d1 = zero4(); }
    __device__ __forceinline__ void load(const float* p) {
        d0 = *reinterpret_cast<const f32x4*>(p);
        d1 = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ void store(float* p) const {
        *reinterpret_cast<f32x4*>(p) = d0;
        *reinterpret_cast<f32x4*>(p + 4) = d1;
    }
};

// The prep of items (chunk, head) first, first + stride, ... below `total`
// (item = chunk * H + head) by one 1024-thread workgroup, which loads the
// next item's inputs into registers while it works on the current one (one
// workgroup fills a CU, so nothing else would hide that load's latency).
template <typename TIn>
__device__ __forceinline__ void prep_diag_items(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ b, int H, const int32_t* __restrict__ rec, int first, int stride,
    int total, unsigned char* __restrict__ factors, PrepDiagLds<TIn>& S) {
    int item = first;
    if (item >= total) return;

    // K, Q rows, b, and alpha for (channel, eighth of 8 tokens) of one item;
    // rows past the chunk's end read as zero keys, b = 0 and alpha = 1
    Row8<TIn> xk, xq;
    float bv, al[8];
    auto load_item = [&](int it) {
        const int tid = threadIdx.x;
        const int sr = tid >> 4, sc8 = (tid & 15) * 8;
        const int ch = tid & 127, qt = tid >> 7;
        const int ck = it / H, hh = it - ck * H;
        const int64_t s0 = rec[4 * ck + 1];
        const int n = rec[4 * ck + 2];
        xk.zero();
        xq.zero();
        if (sr < n) {
            xk.load(k + ((s0 + sr) * H + hh) * kD + sc8);
            xq.load(q + ((s0 + sr) * H + hh) * kD + sc8);
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
    const int next = item + stride;
    // ---- stage K, Q (rows past the chunk's end are zero), b; zero T and A;
    //      G = running sum of log2(alpha) per channel, each eighth of the
    //      chunk first on its own, then offset by the eighths before it
    xk.store(&S.K[sr][sc8]);
    xq.store(&S.Q[sr][sc8]);
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
                        const float kj = in_f32(S.K[sj][key]) *
                                         exp2_hw(S.G[ri][key] - S.G[sj][key]);
                        sl = fmaf(in_f32(S.K[ri][key]), kj, sl);
                        sa = fmaf(in_f32(S.Q[ri][key]), kj, sa);
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
                    vk[4 * hh + i] = in_f32(S.K[row][key]) * e;
                    vq[4 * hh + i] = in_f32(S.Q[row][key]) * e;
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
                    v[4 * hh + i] = in_f32(S.K[tok][key]) * exp2_hw(gc - S.G[tok][key]);
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

// Persistent: workgroup i takes items i, i + gridDim.x, ... of the first
// item_end items (item_end < 0: all of them).
template <typename TIn>
__global__ __launch_bounds__(kPrepThreads) void prep_diag_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ b, int H, const int32_t* __restrict__ rec,
    const int32_t* __restrict__ num_chunks, unsigned char* __restrict__ factors, int item_end) {
    __shared__ __attribute__((aligned(16))) PrepDiagLds<TIn> S;
    int total = num_chunks[0] * H;
    if (item_end >= 0 && item_end < total) total = item_end;
    prep_diag_items<TIn>(q, k, alpha, b, H, rec, int(blockIdx.x), int(gridDim.x), total, factors,
                         S);
}

// ---------------------------------------------------------------------------
// WALK
// ---------------------------------------------------------------------------
constexpr int kDCompute = 8;                          // compute waves
constexpr int kDLoaders = 8;                          // loader waves
constexpr int kDThreads = (kDCompute + kDLoaders) * 64;
constexpr int kDPfAhead = 4;                          // L2 touch distance (chunks)

// One chunk's operands in LDS, in three parts with lifetimes of their own,
// each streamed for the next chunk right after the barrier that ends its
// last read:
//   XA  the decayed K and Q tiles and this slice's V columns: read in P2,
//       streamed after barrier B;
//   FT  T_b: read in P3, streamed after barrier C;
//   FK  (K e^{G_C - G})^T, A and e^{G_C}: read in P4, streamed after the next
//       chunk's barrier A.
// The packed operands keep the prep's layout: 1 KiB blocks of one 16-byte
// MFMA operand per lane.
template <typename TIn>
struct DiagStage {
    u32x4 Kt[32][64];    // (K e^G): [(token tile * 4 + key block) * 2 + hi/lo][lane]
    u32x4 Qt[32][64];    // (Q e^G), the same
    TIn V[kC * 16];      // this slice's 16 value channels, one row per token
    u32x4 Tb[16][64];    // T_b: [(token tile * 2 + token block) * 2 + hi/lo][lane]
    u32x4 Kh[32][64];    // (K e^{G_C - G})^T: [(key tile * 2 + token block) * 2 + hi/lo][lane]
    u32x4 Am[16][64];    // A, as T_b
    float GC[kD];        // e^{G_C} per key
};

template <typename TIn>
struct DiagLds {
    DiagStage<TIn> st;
    u32x4 Sx[4][2][64];  // state tiles (hi/lo) as B operands, key blocks 0..3
    u32x4 Ex[2][2][64];  // E (hi/lo), token blocks 0, 1
    u32x4 Ux[2][2][64];  // U (hi/lo)
    float sink[64];      // landing words of the L2 touches
};
static_assert(sizeof(DiagLds<float>) <= 160 * 1024, "LDS budget of one workgroup");

// The chunks of one sequence are consecutive and full but for the last, so
// a chunk's first token and length follow from the first chunk's start and
// the sequence's end.
template <typename TIn>
struct DiagCtx {
    const TIn* v;
    const unsigned char* factors;
    int H, h, s, l;
    int c_begin, t_begin, t_end;
};

template <typename TIn>
__device__ __forceinline__ const unsigned char* diag_factors(const DiagCtx<TIn>& x, int chunk) {
    return x.factors + (size_t(chunk) * x.H + x.h) * kDiagChunkHeadBytes;
}

// ---- loader waves ------------------------------------------------------------
// Blocks per chunk, by part: XA = K e^G (32), Q e^G (32, with outputs only),
// V (2 bf16 or 4 fp32 blocks of 32 or 16 token rows); FT = T_b (16); FK =
// (K e^{G_C - G})^T (32), A (16, with outputs only), e^{G_C} (half a block).
// Loader i issues the blocks i, i + 8, ... of each part.
template <typename TIn>
constexpr int kVBlocks = sizeof(TIn) == 2 ? 2 : 4;
template <bool kOut, typename TIn>
constexpr int kXABlocks = (kOut ? 64 : 32) + kVBlocks<TIn>;
constexpr int kFTBlocks = 16;
template <bool kOut>
constexpr int kFKBlocks = (kOut ? 48 : 32) + 1;

constexpr int loader_share(int n, int i) { return i < n ? (n - i + 7) / 8 : 0; }

template <bool kOut, typename TIn>
__device__ __forceinline__ void issue_xa_block(const DiagCtx<TIn>& x, int chunk, int j,
                                               DiagStage<TIn>& st) {
    const int L = x.l;
    const unsigned char* F = diag_factors(x, chunk);
    constexpr int kQ = kOut ? 32 : 0;
    if (j < 32) {
        dma16(F + kDOffKt + 1024 * j + 16 * L, reinterpret_cast<char*>(st.Kt) + 1024 * j);
    } else if (j < 32 + kQ) {
        dma16(F + kDOffQt + 1024 * (j - 32) + 16 * L,
              reinterpret_cast<char*>(st.Qt) + 1024 * (j - 32));
    } else {
        // V rows: 16 bytes per lane, 2 (bf16) or 4 (fp32) lanes per row; rows
        // past the chunk's end duplicate its last row (only finite values are
        // needed there: T_b is zero on those rows and columns)
        const int n = j - 32 - kQ;
        constexpr int kLanesPerRow = int(sizeof(TIn));   // a row is 16 values: 32 or 64 bytes
        constexpr int kRows = 64 / kLanesPerRow;         // rows per block: 32 or 16
        const int t0 = x.t_begin + kC * (chunk - x.c_begin);
        const int len = min(kC, x.t_end - t0);
        const int r = kRows * n + L / kLanesPerRow;
        const int rr = r < len ? r : len - 1;
        const TIn* src = x.v + (size_t(t0 + rr) * x.H + x.h) * kD + 16 * x.s +
                         (16 / int(sizeof(TIn))) * (L % kLanesPerRow);
        dma16(src, reinterpret_cast<char*>(st.V) + 1024 * n);
    }
}

template <bool kOut, typename TIn>
__device__ __forceinline__ void issue_fk_block(const DiagCtx<TIn>& x, int chunk, int j,
                                               DiagStage<TIn>& st) {
    const int L = x.l;
    const unsigned char* F = diag_factors(x, chunk);
    constexpr int kA = kOut ? 16 : 0;
    if (j < 32) {
        dma16(F + kDOffKh + 1024 * j + 16 * L, reinterpret_cast<char*>(st.Kh) + 1024 * j);
    } else if (j < 32 + kA) {
        dma16(F + kDOffA + 1024 * (j - 32) + 16 * L,
              reinterpret_cast<char*>(st.Am) + 1024 * (j - 32));
    } else if (L < 32) {
        dma16(F + kDOffGC + 16 * L, st.GC);   // 128 floats: lanes 0..31
    }
}

template <int kI, bool kOut, typename TIn>
__device__ __forceinline__ void issue_xa(const DiagCtx<TIn>& x, int chunk, DiagStage<TIn>& st) {
#pragma unroll
    for (int j = kI; j < kXABlocks<kOut, TIn>; j += kDLoaders) issue_xa_block<kOut>(x, chunk, j, st);
}
template <int kI, typename TIn>
__device__ __forceinline__ void issue_ft(const DiagCtx<TIn>& x, int chunk, DiagStage<TIn>& st) {
    const unsigned char* F = diag_factors(x, chunk);
#pragma unroll
    for (int j = kI; j < kFTBlocks; j += kDLoaders)
        dma16(F + kDOffTb + 1024 * j + 16 * x.l, reinterpret_cast<char*>(st.Tb) + 1024 * j);
}
template <int kI, bool kOut, typename TIn>
__device__ __forceinline__ void issue_fk(const DiagCtx<TIn>& x, int chunk, DiagStage<TIn>& st) {
#pragma unroll
    for (int j = kI; j < kFKBlocks<kOut>; j += kDLoaders) issue_fk_block<kOut>(x, chunk, j, st);
}

// Touch this slice's eighth of a chunk's factor lines (the 8 slices of a
// head share them through their XCD's L2): lines s + 8 u, u in 64 kHalf ..
// 64 kHalf + 63, one per lane.
template <int kHalf, typename TIn>
__device__ __forceinline__ void touch_diag(const DiagCtx<TIn>& x, int chunk, float* sink) {
    const int u = 64 * kHalf + x.l;
    dma4(diag_factors(x, chunk) + 128 * (x.s + 8 * u), sink);
}

// Before each barrier a loader waits until only what it issued after the
// part read next may still be in flight (loads complete in issue order):
// loaders 0 and 1 also issue one L2 touch right after each XA part.
template <int kI, bool kOut, typename TIn>
__device__ void diag_loader(const DiagCtx<TIn>& x, int c0, int c_end, DiagLds<TIn>& S) {
    constexpr int kT = kI < 2 ? 1 : 0;
    constexpr int nXA = loader_share(kXABlocks<kOut, TIn>, kI);
    constexpr int nFT = loader_share(kFTBlocks, kI);
    constexpr int nFK = loader_share(kFKBlocks<kOut>, kI);
    const int last = c_end - 1;
    auto cl = [last](int c) { return c < last ? c : last; };
    if constexpr (kI < 2) {
#pragma unroll
        for (int d = 1; d < kDPfAhead; ++d) touch_diag<kI>(x, cl(c0 + d), S.sink);
    }
    issue_xa<kI, kOut>(x, c0, S.st);
    if constexpr (kI < 2) touch_diag<kI>(x, cl(c0 + kDPfAhead), S.sink);
    issue_ft<kI>(x, c0, S.st);
    for (int c = c0; c < c_end; ++c) {
        wait_vm<kT + nFT>();               // XA(c) has landed
        __builtin_amdgcn_s_barrier();      // A
        issue_fk<kI, kOut>(x, c, S.st);    // FK was last read in the previous P4
        wait_vm<nFK>();                    // FT(c) has landed
        __builtin_amdgcn_s_barrier();      // B
        issue_xa<kI, kOut>(x, cl(c + 1), S.st);
        if constexpr (kI < 2) touch_diag<kI>(x, cl(c + 1 + kDPfAhead), S.sink);
        wait_vm<nXA + kT>();               // FK(c) has landed
        __builtin_amdgcn_s_barrier();      // C
        issue_ft<kI>(x, cl(c + 1), S.st);
    }
    wait_vm<0>();   // nothing may land in LDS after the workgroup ends
}

// ---- compute waves -------------------------------------------------------------

// hi*hi + hi*lo + lo*hi over `nb` k blocks: A operands from the packed stage
// blocks P[(base + m) * 2 + hl], B operands from an exchange buffer
template <int nb>
__device__ __forceinline__ f32x4 prod3(const u32x4 (*P)[64], int base, u32x4 (*B)[2][64], int l) {
    bf16x8 a[nb][2];
#pragma unroll
    for (int m = 0; m < nb; ++m) {
        a[m][0] = __builtin_bit_cast(bf16x8, P[(base + m) * 2][l]);
        a[m][1] = __builtin_bit_cast(bf16x8, P[(base + m) * 2 + 1][l]);
    }
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

// One chunk.  Wave w keeps the state's key tile w (16 keys x 16 values) in
// an MFMA accumulator; waves 0-3 also take token tile w through the errors
// and U, waves 4-7 token tile w - 4 through the outputs.  Without outputs
// (kOut false) the output waves only carry their state tiles; zero_v takes
// every value as zero (the walk then applies the chunks' transition alone).
template <bool kOut, typename TIn>
__device__ __forceinline__ void diag_step(const DiagCtx<TIn>& x, int w, int t0, int len,
                                          DiagLds<TIn>& S, f32x4& acc, float* __restrict__ o,
                                          bool zero_v) {
    const int l = x.l, g = l >> 4, c = l & 15, tt = w & 3;
    const bool state = w < 4;
    // P1
    publish4(S.Sx, w, l, acc);
    __syncthreads();   // A
    // P2
    f32x4 yz = zero4();
    if (state) {
        yz = prod3<4>(S.st.Kt, tt * 4, S.Sx, l);
        f32x4 vv = zero4();
        if (!zero_v) {
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[i] = in_f32(S.st.V[(16 * tt + 4 * g + i) * 16 + c]);
        }
        publish4(S.Ex, tt, l, vv - yz);
    } else if (kOut) {
        yz = prod3<4>(S.st.Qt, tt * 4, S.Sx, l);
    }
    __syncthreads();   // B
    // P3
    if (state) publish4(S.Ux, tt, l, prod3<2>(S.st.Tb, tt * 2, S.Ex, l));
    __syncthreads();   // C
    // P4
    const f32x4 upd = prod3<2>(S.st.Kh, w * 2, S.Ux, l);
    const f32x4 gc = *reinterpret_cast<const f32x4*>(S.st.GC + 16 * w + 4 * g);
    acc = acc * gc + upd;
    if (kOut && !state) {
        const f32x4 ov = yz + prod3<2>(S.st.Am, tt * 2, S.Ux, l);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 16 * tt + 4 * g + i;
            if (tok < len) o[((size_t(t0) + tok) * x.H + x.h) * kD + 16 * x.s + c] = ov[i];
        }
    }
}

// A walk launch's LDS: the walk's, or (its prep workgroups) the prep's.
template <typename TIn>
union DiagWalkOrPrepLds {
    DiagLds<TIn> walk;
    PrepDiagLds<TIn> prep;
};

template <bool kOut, typename TIn>
__global__ __launch_bounds__(kDThreads) void walk_diag_kernel(
    const TIn* __restrict__ v, int N, int H, const int32_t* __restrict__ rec,
    const int32_t* __restrict__ seq_off, const int32_t* __restrict__ num_chunks,
    unsigned char* __restrict__ factors, float* __restrict__ o, WalkJob j0, WalkJob j1,
    int seg_chunks, DiagSide X) {
    __shared__ __attribute__((aligned(16))) DiagWalkOrPrepLds<TIn> shm;
    if (int(blockIdx.x) >= X.walk_blocks) {
        // the prep of later chunks, on the CUs the walk leaves idle
        prep_diag_items<TIn>(static_cast<const TIn*>(X.q), static_cast<const TIn*>(X.k),
                             X.alpha, X.b, H, rec,
                             X.item_lo + int(blockIdx.x) - X.walk_blocks, X.prep_blocks,
                             X.item_hi, factors, shm.prep);
        return;
    }
    DiagLds<TIn>& lds = shm.walk;
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
    if (X.c_hi > 0) {   // one sequence walked over chunks [c_lo, c_hi) only
        c_begin = X.c_lo < nch ? X.c_lo : nch;
        c_end = X.c_hi < nch ? X.c_hi : nch;
    }
    int t_begin = 0, t_end = 0;
    if (c_begin < c_end) {
        t_begin = rec[4 * c_begin + 1];
        t_end = rec[4 * (c_end - 1) + 1] + rec[4 * (c_end - 1) + 2];
    }
    const DiagCtx<TIn> x{v, factors, H, h, s, l, c_begin, t_begin, t_end};

    if (w >= kDCompute) {
        if (c_begin < c_end) {
            switch (w - kDCompute) {
                case 0: diag_loader<0, kOut>(x, c_begin, c_end, lds); break;
                case 1: diag_loader<1, kOut>(x, c_begin, c_end, lds); break;
                case 2: diag_loader<2, kOut>(x, c_begin, c_end, lds); break;
                case 3: diag_loader<3, kOut>(x, c_begin, c_end, lds); break;
                case 4: diag_loader<4, kOut>(x, c_begin, c_end, lds); break;
                case 5: diag_loader<5, kOut>(x, c_begin, c_end, lds); break;
                case 6: diag_loader<6, kOut>(x, c_begin, c_end, lds); break;
                default: diag_loader<7, kOut>(x, c_begin, c_end, lds); break;
            }
        }
        return;
    }

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
    for (int ch = c_begin; ch < c_end; ++ch) {
        const int t0 = t_begin + kC * (ch - c_begin);
        diag_step<kOut>(x, w, t0, min(kC, t_end - t0), lds, acc, o, zero_v);
    }
    if (J.S_final) *reinterpret_cast<f32x4*>(J.S_final + srow) = acc;
}

}  // namespace

hipError_t launch_prep_diag(const void* q, const void* k, rda_dtype dt, const float* alpha,
                            const float* b, int32_t heads, int32_t max_chunks, const int32_t* rec,
                            const int32_t* num_chunks, unsigned char* factors,
                            hipStream_t stream, int32_t item_end) {
    // one persistent workgroup per CU at most (each holds a CU's LDS)
    int64_t items = int64_t(max_chunks) * heads;
    if (item_end >= 0 && item_end < items) items = item_end;
    const unsigned pgrid = unsigned(items < kPrepDiagGrid ? items : kPrepDiagGrid);
    if (pgrid == 0) return hipSuccess;
    if (dt == RDA_BF16)
        hipLaunchKernelGGL(prep_diag_kernel<uint16_t>, dim3(pgrid), dim3(kPrepThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), alpha,
                           b, heads, rec, num_chunks, factors, item_end);
    else
        hipLaunchKernelGGL(prep_diag_kernel<float>, dim3(pgrid), dim3(kPrepThreads), 0, stream,
                           static_cast<const float*>(q), static_cast<const float*>(k), alpha, b,
                           heads, rec, num_chunks, factors, item_end);
    return hipGetLastError();
}

template <bool kOut, typename TIn>
static void launch_walk_diag_t(const void* v, int32_t num_seqs, int32_t heads, const int32_t* rec,
                               const int32_t* seq_off, const int32_t* num_chunks,
                               unsigned char* factors, float* o, WalkJob j0, WalkJob j1,
                               int32_t seg_chunks, unsigned grid, const DiagSide& X,
                               hipStream_t stream) {
    hipLaunchKernelGGL((walk_diag_kernel<kOut, TIn>), dim3(grid), dim3(kDThreads), 0, stream,
                       static_cast<const TIn*>(v), num_seqs, heads, rec, seq_off, num_chunks,
                       factors, o, j0, j1, seg_chunks, X);
}

hipError_t launch_walk_diag(const void* v, rda_dtype dt, int32_t num_seqs, int32_t heads,
                            const int32_t* rec, const int32_t* seq_off,
                            const int32_t* num_chunks, unsigned char* factors, float* o,
                            const WalkJob* jobs, int32_t num_jobs, int32_t seg_chunks,
                            bool outputs, hipStream_t stream, const DiagSide* side) {
    const int64_t pairs = int64_t(num_seqs) * heads;
    const unsigned wgrid = unsigned(num_jobs * 64 * ((pairs + 7) / 8));
    DiagSide X{};
    if (side) X = *side;
    X.walk_blocks = int(wgrid);
    const unsigned grid = wgrid + unsigned(side ? side->prep_blocks : 0);
    const WalkJob none{nullptr, nullptr, 0, 0};
    const WalkJob j1 = num_jobs > 1 ? jobs[1] : none;
    if (dt == RDA_BF16) {
        if (outputs)
            launch_walk_diag_t<true, uint16_t>(v, num_seqs, heads, rec, seq_off, num_chunks,
                                               factors, o, jobs[0], j1, seg_chunks, grid, X,
                                               stream);
        else
            launch_walk_diag_t<false, uint16_t>(v, num_seqs, heads, rec, seq_off, num_chunks,
                                                factors, o, jobs[0], j1, seg_chunks, grid, X,
                                                stream);
    } else {
        if (outputs)
            launch_walk_diag_t<true, float>(v, num_seqs, heads, rec, seq_off, num_chunks, factors,
                                            o, jobs[0], j1, seg_chunks, grid, X, stream);
        else
            launch_walk_diag_t<false, float>(v, num_seqs, heads, rec, seq_off, num_chunks,
                                             factors, o, jobs[0], j1, seg_chunks, grid, X,
                                             stream);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_diag(const void* q, const void* k, const void* v, rda_dtype dt,
                               const float* alpha, const float* b, int32_t num_seqs,
                               int32_t heads, int32_t max_chunks, const int32_t* rec,
                               const int32_t* seq_off, const int32_t* num_chunks,
                               unsigned char* factors, const float* S0, float* o,
                               float* S_final, hipStream_t stream) {
    const hipError_t err =
        launch_prep_diag(q, k, dt, alpha, b, heads, max_chunks, rec, num_chunks, factors, stream);
    if (err != hipSuccess) return err;
    const WalkJob job{S0, S_final, 0, 0};
    return launch_walk_diag(v, dt, num_seqs, heads, rec, seq_off, num_chunks, factors, o, &job, 1,
                            0, true, stream);
}

}  // namespace rda
