// rda_prefill.hip -- chunked prefill of the RDA gated delta rule on gfx950.
//
// The recurrence (decay, the residual e = v - S'k of the decayed state at
// the key, the rank-one write b e k^T, read-out after the update; the
// "Raon-1 nano" teardown, section "The other 1.5B: a hybrid built to forget")
// is evaluated in chunks of C = 64 tokens.  With S the state entering a chunk
// (rows = value channels), g_i the in-chunk running sum of log a,
// gamma_i = exp(g_i), Gamma = diag(gamma) and Gamma_ij = exp(g_i - g_j):
//
//   L     = strict-lower( diag(b) K K^T . Gamma_ij ),   T = (I + L)^-1
//   T_b   = T diag(b)
//   A     = lower( Q K^T . Gamma_ij )
//   U     = T_b V - T_b Gamma (K S^T)             (the errors each token writes)
//   O     = Gamma (Q S^T) + A U                   (outputs of the chunk's tokens)
//   S_out = gamma_C S + U^T diag(gamma_C / gamma) K
//
// This is the WY / UT-transform form of the gated delta rule (W = T_b Gamma K
// is never formed: the walk multiplies through T_b instead; the bf16 walk
// applies T_b once, to E = V - Gamma (K S^T), while the fp32 walk below forms
// T_b V and T_b Gamma Y separately), and it reproduces the token-by-token
// recurrence exactly in real arithmetic.
//
// PREP (parallel over chunk x head): gates, Gram tiles K K^T and Q K^T on
// MFMA, the unit-lower-triangular solve for T in fp32, then T_b and A packed
// as bf16 hi/lo MFMA operands (33 KiB per chunk-head in the workspace; the
// bf16 kernels skip the slots that are zero, 25 KiB in use).
// WALK (sequential over the chunks of a sequence): one workgroup per
// (sequence, head, 16-channel value slice); the fp32 state slice lives in
// MFMA accumulators, and each chunk costs three dependent MFMA stages
// (Y = K S^T, the T_b product, the S update) over the raw bf16 q, k, v tiles
// and the two packed 64 x 64 factors.  Rows of S evolve independently, so the 8
// slices of a head need no communication.
//
// Precision: q, k, v enter MFMA as exact bf16 (fp32 inputs as bf16 hi + lo).
// Every computed fp32 operand (T_b, A, S, Gamma Y, U) is fed as a bf16 hi +
// lo pair, and products take hi*hi + hi*lo + lo*hi, i.e. ~2^-16 relative
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
#include <type_traits>

#include "rda_device.h"
#include "rda_internal.h"
#include "rda_lds.h"
#include "rda_out.h"
#include "rda_solve.h"

namespace rda {

namespace {

// ---------------------------------------------------------------------------
// PREP: one 256-thread workgroup per (chunk, head).
// ---------------------------------------------------------------------------
constexpr int kTS = 136;   // bf16 tile row stride (elements): 272 B, spreads LDS banks
constexpr int kTileB = kC * kTS * 2;   // 17408 B
constexpr int kMatB = kC * kFS * 4;    // 17408 B

constexpr int kSmK = 0;
constexpr int kSmQ = kSmK + kTileB;
constexpr int kSmL = kSmQ + kTileB;
constexpr int kSmA = kSmL + kMatB;
constexpr int kSmT = kSmA + kMatB;
constexpr int kSmG = kSmT + kMatB;           // la, bb, gg, gam: 4 x 64 floats
constexpr int kSmR = kSmG + 4 * 64 * 4;      // 3 x 16x16 fp32 solve scratch
constexpr int kSmLo = kSmR + 3 * 256 * 4;    // lo planes of K, Q (fp32 inputs only)
constexpr int kPrepSmemBf16 = kSmLo;
constexpr int kPrepSmemSplit = kSmLo + 2 * kTileB;

template <bool kSplit>
struct PrepIn;
template <>
struct PrepIn<false> { using T = uint16_t; };
template <>
struct PrepIn<true> { using T = float; };

// One [64 x 128] token tile of head h as this thread's share of loads (8
// bf16 or 4 fp32 elements per load), every load issued before any is used:
// rows past the chunk's end read its last row and are zeroed when stored.
template <bool kSplit>
struct TileLoads {
    using V = typename std::conditional<kSplit, f32x4, u16x8>::type;
    static constexpr int kN = kSplit ? 8 : 4;   // loads per thread
    V x[kN];
};

template <bool kSplit>
__device__ __forceinline__ void load_tile(const typename PrepIn<kSplit>::T* __restrict__ src,
                                          int64_t t0, int len, int H, int h, int tid,
                                          TileLoads<kSplit>& L) {
#pragma unroll
    for (int qq = 0; qq < TileLoads<kSplit>::kN; ++qq) {
        const int p = tid + 256 * qq;
        const int r = kSplit ? p >> 5 : p >> 4;
        const int col = kSplit ? (p & 31) * 4 : (p & 15) * 8;
        const int rr = r < len ? r : len - 1;
        L.x[qq] = *reinterpret_cast<const typename TileLoads<kSplit>::V*>(
            src + ((t0 + rr) * H + h) * kD + col);
    }
}

// Store a loaded tile into LDS as bf16 (hi, and lo for fp32 inputs); rows
// >= len are zero.
template <bool kSplit>
__device__ __forceinline__ void store_tile(const TileLoads<kSplit>& L, int len, uint16_t* hi,
                                           uint16_t* lo, int tid) {
#pragma unroll
    for (int qq = 0; qq < TileLoads<kSplit>::kN; ++qq) {
        const int p = tid + 256 * qq;
        if constexpr (!kSplit) {
            const int r = p >> 4, c8 = (p & 15) * 8;
            const u16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
            *reinterpret_cast<u16x8*>(hi + r * kTS + c8) = r < len ? L.x[qq] : zero;
        } else {
            const int r = p >> 5, c4 = (p & 31) * 4;
            const f32x4 x = r < len ? L.x[qq] : zero4();
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

template <bool kSplit>
__global__ __launch_bounds__(256) void prep_kernel(
    const typename PrepIn<kSplit>::T* __restrict__ q, const typename PrepIn<kSplit>::T* __restrict__ k,
    const float* __restrict__ a, const float* __restrict__ b, int H, const int32_t* __restrict__ rec,
    const int32_t* __restrict__ num_chunks, unsigned char* __restrict__ factors, int32_t single_T,
    int32_t* __restrict__ rec_out, int32_t* __restrict__ seq_off_out, int32_t* __restrict__ num_out) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kSplit ? kPrepSmemSplit : kPrepSmemBf16];
    const int chunk = blockIdx.x / H;
    const int h = blockIdx.x - chunk * H;
    const int tid = threadIdx.x;
    int64_t t0;
    int len;
    if (single_T >= 0) {
        // one sequence of single_T tokens and no offsets: the records are
        // plain arithmetic, and the head-0 workgroups write the table
        const int nch = (single_T + kC - 1) / kC;
        if (chunk >= nch) return;
        t0 = int64_t(kC) * chunk;
        len = single_T - int(t0) < kC ? single_T - int(t0) : kC;
        if (h == 0) prep_table_entry(chunk, int(t0), len, nch, tid, rec_out, seq_off_out, num_out);
    } else {
        if (chunk >= num_chunks[0]) return;
        t0 = rec[4 * chunk + 1];
        len = rec[4 * chunk + 2];
    }

    const int w = wave_id(), l = tid & 63, g = l >> 4, c = l & 15;

    uint16_t* Ks = reinterpret_cast<uint16_t*>(smem + kSmK);
    uint16_t* Qs = reinterpret_cast<uint16_t*>(smem + kSmQ);
    uint16_t* Kl = reinterpret_cast<uint16_t*>(smem + kSmLo);
    uint16_t* Ql = Kl + kC * kTS;
    float* Ls = reinterpret_cast<float*>(smem + kSmL);
    float* As = reinterpret_cast<float*>(smem + kSmA);
    float* Ts = reinterpret_cast<float*>(smem + kSmT);
    float* la = reinterpret_cast<float*>(smem + kSmG);
    float* bb = la + 64;
    float* gg = bb + 64;
    float* gam = gg + 64;
    float* Rs = reinterpret_cast<float*>(smem + kSmR);

    unsigned char* F = factors + (size_t(chunk) * H + h) * kChunkHeadBytes;

    // ---- stage inputs; zero T and A (their upper triangles stay zero) ------
    {
        TileLoads<kSplit> lk, lq;
        load_tile<kSplit>(k, t0, len, H, h, tid, lk);
        load_tile<kSplit>(q, t0, len, H, h, tid, lq);
        store_tile<kSplit>(lk, len, Ks, Kl, tid);
        store_tile<kSplit>(lq, len, Qs, Ql, tid);
    }
    for (int e = tid; e < kC * kFS; e += 256) {
        Ts[e] = 0.f;
        As[e] = 0.f;
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
        la[l] = lav;
        bb[l] = bv;
        gg[l] = sum;
        gam[l] = expf(sum);
    }
    __syncthreads();

    // ---- Gram tiles: L = strict-lower(diag(b) K K^T . Gamma), A = lower(Q K^T . Gamma).
    //      Wave w: the L tiles (t, w) for t >= w and the transposed A tiles
    //      (t, w) for t <= w, i.e. A's row tile w, with its own K and Q rows
    //      read once and K rows 16t.. for each t (fp32 inputs: hi*hi + hi*lo +
    //      lo*hi).  A transposed tile leaves each lane 4 consecutive entries
    //      of one row of A.
    {
        auto rowop = [&](const uint16_t* X, int r, int m) {
            return *reinterpret_cast<const bf16x8*>(X + r * kTS + 32 * m + 8 * g);
        };
        bf16x8 kwh[4], kwl[4], qwh[4], qwl[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            kwh[m] = rowop(Ks, 16 * w + c, m);
            qwh[m] = rowop(Qs, 16 * w + c, m);
            if constexpr (kSplit) {
                kwl[m] = rowop(Kl, 16 * w + c, m);
                qwl[m] = rowop(Ql, 16 * w + c, m);
            }
        }
        const int s = 16 * w + c;   // key token of the L tiles, query token of the A tiles
        const float gs = gg[s];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 kth[4], ktl[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                kth[m] = rowop(Ks, 16 * t + c, m);
                if constexpr (kSplit) ktl[m] = rowop(Kl, 16 * t + c, m);
            }
            if (t >= w) {   // L tile (t, w): rows 16t + 4g + e, column s
                f32x4 d = zero4();
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    d = mfma_bf16(kth[m], kwh[m], d);
                    if constexpr (kSplit) {
                        d = mfma_bf16(kth[m], kwl[m], d);
                        d = mfma_bf16(ktl[m], kwh[m], d);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * t + 4 * g + e;
                    Ls[r * kFS + s] = r > s ? bb[r] * d[e] * __expf(gg[r] - gs) : 0.f;
                }
            }
            if (t <= w) {   // transposed A tile (t, w): A[s][16t + 4g + e]
                f32x4 d = zero4();
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    d = mfma_bf16(kth[m], qwh[m], d);
                    if constexpr (kSplit) {
                        d = mfma_bf16(kth[m], qwl[m], d);
                        d = mfma_bf16(ktl[m], qwh[m], d);
                    }
                }
                f32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * t + 4 * g + e;
                    out[e] = j <= s ? d[e] * __expf(gs - gg[j]) : 0.f;
                }
                *reinterpret_cast<f32x4*>(As + s * kFS + 16 * t + 4 * g) = out;
            }
        }
    }
    __syncthreads();

    // ---- T = (I + L)^-1 ------------------------------------------------------
    solve_unit_lower(Ls, Ts, Rs, w, g, c);

    // ---- outputs: T_b = T diag(b) and A as packed hi/lo operands; gates ----
    pack_rows(Ts, bb, reinterpret_cast<bf16x8*>(F + kOffTb), tid);
    pack_rows(As, nullptr, reinterpret_cast<bf16x8*>(F + kOffA), tid);
    if (tid < 64) {
        float* G = reinterpret_cast<float*>(F + kOffG);
        G[kGGam + tid] = gam[tid];
        G[kGScale + tid] = expf(gg[63] - gg[tid]);
        G[kGLog + tid] = gg[tid];
        if (tid == 0) G[kGC] = gam[63];
    }
}

// ---------------------------------------------------------------------------
// WALK: one workgroup per (sequence, head, 16-channel value slice), 8 waves.
//
// Wave w owns the 16 x 16 tile of S^T with keys 16w .. 16w+15 (an MFMA
// accumulator).  Waves 0..3 ("state waves") carry the state-critical chain,
// waves 4..7 ("output waves") the outputs; token tile tt = w % 4.  Per chunk:
//   P1  every wave publishes its state tile (bf16 hi/lo) to LDS; state waves
//       store their 16 rows of the K tile and V slice, output waves their 16
//       rows of the Q tile (all loaded a chunk ahead with coalesced loads).
//   P2  state waves: Y = K S^T for token tile tt, Gamma Y (hi/lo) to LDS, and
//       U' = T_b V;  output waves: Z = Q S^T.  Every wave also fetches its K^T
//       operand for P4 with transposing LDS reads.
//   P3  state waves: X = T_b (Gamma Y), U = U' - X, and U and
//       U~ = diag(gamma_C / gamma) U (hi/lo) to LDS.
//   P4  every wave: S^T = gamma_C S^T + K^T U~ for its key tile;
//       output waves: O = Gamma Z + A U, stored.
// Three barriers per chunk.  Global operands of the chunk after next are
// loaded as soon as the current chunk has consumed them (two operand sets,
// ping-pong), with unconditional, clamped, in-bounds addresses so the
// compiler's load counters stay exact.
// ---------------------------------------------------------------------------
constexpr int kWalkWaves = 8;
constexpr int kWalkThreads = kWalkWaves * 64;
constexpr int kKS = 136;   // LDS K / Q tile row stride (bf16 elements)
constexpr int kVS = 20;    // LDS V slice row stride (bf16 elements)

// (bf16 inputs take the walk in rda_walk.hip; this one serves fp32 inputs,
// fed to MFMA as bf16 hi + lo planes)
template <typename TIn>
struct WalkIn;
template <>
struct WalkIn<float> { static constexpr bool kSplit = true; };

// Global operands of one chunk for one wave (state-independent).
template <bool kSplit>
struct WalkOps {
    // raw rows 16tt + 4i + l/16 (i < 4), elements 8(l%16) .. +7 of the K
    // tile (state waves) or Q tile (output waves): 8 bf16, or 8 floats for
    // fp32 inputs.  Masking and conversion happen at staging time so that the
    // loads are never waited on where they are issued.
    u32x4 rows[4][kSplit ? 2 : 1];
    u32x4 vrow;                   // V slice: row 16tt + l/4, channels 4(l%4) .. +3 (state waves)
    bf16x8 ah[2], al[2];          // T_b (state waves) or A (output waves), token blocks 0, 1
    f32x4 gam;                    // gamma of this lane's 4 tokens (16tt + 4g + i)
    f32x4 gs;                     // gamma_C / gamma of the same tokens (state waves)
    float gC;                     // gamma_C
    int t0, len;                  // first token and valid length of the chunk
};

template <typename TIn>
struct WalkCtx {
    const TIn* q;
    const TIn* k;
    const TIn* v;
    const unsigned char* factors;
    const int32_t* rec;
    int H, h, s, w, l;
};

template <typename TIn>
__device__ __forceinline__ const unsigned char* chunk_factors(const WalkCtx<TIn>& x, int chunk) {
    return x.factors + (size_t(chunk) * x.H + x.h) * kChunkHeadBytes;
}

// Coalesced rows of the K (state waves) or Q (output waves) tile: instruction
// i covers rows 16tt + 4i .. +3 (256 contiguous bytes each for bf16).  Rows
// past the chunk's end read a valid row; stage_rows zeroes them.
template <typename TIn>
__device__ __forceinline__ void load_rows(WalkOps<WalkIn<TIn>::kSplit>& o, const WalkCtx<TIn>& x,
                                          int chunk) {
    const int t0 = x.rec[4 * chunk + 1], len = x.rec[4 * chunk + 2];
    const TIn* src = x.w < 4 ? x.k : x.q;
    const int tt = x.w & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * tt + 4 * i + (x.l >> 4);
        const TIn* p = src + ((size_t(t0) + (r < len ? r : len - 1)) * x.H + x.h) * kD + 8 * (x.l & 15);
        o.rows[i][0] = *reinterpret_cast<const u32x4*>(p);
        if constexpr (WalkIn<TIn>::kSplit) o.rows[i][1] = *reinterpret_cast<const u32x4*>(p + 4);
    }
}

// V slice rows (state waves); stage_rows zeroes rows past the chunk's end
template <typename TIn>
__device__ __forceinline__ void load_v(WalkOps<WalkIn<TIn>::kSplit>& o, const WalkCtx<TIn>& x,
                                       int chunk) {
    const int t0 = x.rec[4 * chunk + 1], len = x.rec[4 * chunk + 2];
    const int r = 16 * (x.w & 3) + (x.l >> 2);
    const TIn* p = x.v + ((size_t(t0) + (r < len ? r : len - 1)) * x.H + x.h) * kD + 16 * x.s +
                   4 * (x.l & 3);
    if constexpr (!WalkIn<TIn>::kSplit) {
        const u32x2 d = *reinterpret_cast<const u32x2*>(p);
        o.vrow = u32x4{d[0], d[1], 0u, 0u};
    } else {
        o.vrow = *reinterpret_cast<const u32x4*>(p);
    }
}

// T_b (state waves) or A (output waves) rows of the token tile, and gates
template <typename TIn>
__device__ __forceinline__ void load_f(WalkOps<WalkIn<TIn>::kSplit>& o, const WalkCtx<TIn>& x,
                                       int chunk) {
    const unsigned char* F = chunk_factors(x, chunk);
    const int tt = x.w & 3;
    const bf16x8* P = reinterpret_cast<const bf16x8*>(F + (x.w < 4 ? kOffTb : kOffA));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int base = ((tt * 2 + m) * 2) * 64 + x.l;
        o.ah[m] = P[base];
        o.al[m] = P[base + 64];
    }
    const float* G = reinterpret_cast<const float*>(F + kOffG);
    o.gam = *reinterpret_cast<const f32x4*>(G + kGGam + 16 * tt + 4 * (x.l >> 4));
    o.gs = *reinterpret_cast<const f32x4*>(G + kGScale + 16 * tt + 4 * (x.l >> 4));
    o.gC = G[kGC];
}

template <typename TIn>
__device__ __forceinline__ void load_rec(WalkOps<WalkIn<TIn>::kSplit>& o, const WalkCtx<TIn>& x,
                                         int chunk) {
    o.t0 = x.rec[4 * chunk + 1];
    o.len = x.rec[4 * chunk + 2];
}

template <typename TIn>
__device__ __forceinline__ void load_all(WalkOps<WalkIn<TIn>::kSplit>& o, const WalkCtx<TIn>& x,
                                         int chunk) {
    load_rec(o, x, chunk);
    load_rows(o, x, chunk);
    if (x.w < 4) load_v(o, x, chunk);
    load_f(o, x, chunk);
}

// LDS exchange buffers hold ready 16-byte B operands: entry [blk][hl][lane]
// is key (or token) block blk, whose low 8 bytes come from tile 2 blk and
// high 8 bytes from tile 2 blk + 1, each written by the wave owning it.
// Transposed operand from a row-major bf16 LDS tile (row stride `stride`):
// lane (g = l/16, c = l%16) receives column col0 + c of rows
// {r0 + i, r0 + 16 + i : i < 4} with r0 = 32m + 4g (the permuted token order).
// ds_read_b64_tr_b16: within a 16-lane group, output lane i, element e is
// element i%4 of the 8 bytes addressed by source lane 4e + i/4, so source
// lane j points at row r0 + j/4, columns col0 + 4(j%4) .. +3.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int stride, int r0, int col0,
                                             int l) {
    const int j = l & 15;
    const uint16_t* p0 = tile + (r0 + (j >> 2)) * stride + col0 + 4 * (j & 3);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 16 * stride));
    return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, a)[0],
                                             __builtin_bit_cast(u32x2, a)[1],
                                             __builtin_bit_cast(u32x2, b)[0],
                                             __builtin_bit_cast(u32x2, b)[1]});
}

// A operand from a row-major bf16 LDS tile: row r, keys {32m + 4g + i,
// 32m + 16 + 4g + i : i < 4} (the permuted key order of the state operand).
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* tile, int r, int m, int g) {
    const uint16_t* p = tile + r * kKS + 32 * m + 4 * g;
    const u32x2 a = *reinterpret_cast<const u32x2*>(p);
    const u32x2 b = *reinterpret_cast<const u32x2*>(p + 16);
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

template <bool kSplit>
struct WalkLds {
    u32x4 Sx[4][2][64];   // state tiles (hi/lo) as B operands, key blocks 0..3
    u32x4 Yx[2][2][64];   // Gamma Y (hi/lo), token blocks 0, 1
    u32x4 Ux[2][2][64];   // U (hi/lo)
    u32x4 Uy[2][2][64];   // U~ (hi/lo)
    uint16_t K[2][kSplit ? 2 : 1][kC][kKS];   // K tile by chunk parity (hi, lo planes)
    uint16_t Q[kSplit ? 2 : 1][kC][kKS];      // Q tile
    uint16_t V[kSplit ? 2 : 1][kC][kVS];      // V slice
};

// P1 staging of this wave's tile rows into LDS (bf16 hi, and lo for fp32
// inputs); rows at or past `len` are stored as zeros.
template <bool kSplit>
__device__ __forceinline__ void stage_rows(const WalkOps<kSplit>& cur, uint16_t (*T)[kC][kKS],
                                           int tt, int l, int len) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * tt + 4 * i + (l >> 4);
        const bool valid = r < len;
        if constexpr (!kSplit) {
            *reinterpret_cast<u32x4*>(&T[0][r][8 * (l & 15)]) =
                valid ? cur.rows[i][0] : u32x4{0u, 0u, 0u, 0u};
        } else {
            const f32x4 d0 = __builtin_bit_cast(f32x4, cur.rows[i][0]);
            const f32x4 d1 = __builtin_bit_cast(f32x4, cur.rows[i][1]);
            float v8[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
            if (!valid)
#pragma unroll
                for (int j = 0; j < 8; ++j) v8[j] = 0.f;
            bf16x8 hi, lo;
            split8(v8, hi, lo);
            *reinterpret_cast<bf16x8*>(&T[0][r][8 * (l & 15)]) = hi;
            *reinterpret_cast<bf16x8*>(&T[1][r][8 * (l & 15)]) = lo;
        }
    }
}

template <bool kSplit>
__device__ __forceinline__ void stage_v(const WalkOps<kSplit>& cur, uint16_t (*V)[kC][kVS], int tt,
                                        int l, int len) {
    const int vr = 16 * tt + (l >> 2), vc = 4 * (l & 3);
    const bool valid = vr < len;
    if constexpr (!kSplit) {
        *reinterpret_cast<u32x2*>(&V[0][vr][vc]) =
            valid ? u32x2{cur.vrow[0], cur.vrow[1]} : u32x2{0u, 0u};
    } else {
        const f32x4 d = __builtin_bit_cast(f32x4, cur.vrow);
        uint32_t h01, l01, h23, l23;
        split_pk(valid ? d[0] : 0.f, valid ? d[1] : 0.f, h01, l01);
        split_pk(valid ? d[2] : 0.f, valid ? d[3] : 0.f, h23, l23);
        *reinterpret_cast<u32x2*>(&V[0][vr][vc]) = u32x2{h01, h23};
        *reinterpret_cast<u32x2*>(&V[1][vr][vc]) = u32x2{l01, l23};
    }
}

template <typename TIn, int kPar>
__device__ __forceinline__ void state_step(WalkOps<WalkIn<TIn>::kSplit>& cur, f32x4& acc,
                                           const WalkCtx<TIn>& x, int next,
                                           WalkLds<WalkIn<TIn>::kSplit>& S) {
    constexpr bool kSplit = WalkIn<TIn>::kSplit;
    const int w = x.w, l = x.l, g = l >> 4, c = l & 15, tt = w & 3;
    // P1
    publish4(S.Sx, w, l, acc);
    stage_rows<kSplit>(cur, S.K[kPar], tt, l, cur.len);
    stage_v<kSplit>(cur, S.V, tt, l, cur.len);
    __syncthreads();
    // P2: operands from LDS first, then Y = K S^T
    bf16x8 kt[2][kSplit ? 2 : 1], vb[2][kSplit ? 2 : 1], ka[4][kSplit ? 2 : 1];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int pl = 0; pl < (kSplit ? 2 : 1); ++pl) {
            kt[m][pl] = tr_operand(&S.K[kPar][pl][0][0], kKS, 32 * m + 4 * g, 16 * w, l);
            vb[m][pl] = tr_operand(&S.V[pl][0][0], kVS, 32 * m + 4 * g, 0, l);
        }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int pl = 0; pl < (kSplit ? 2 : 1); ++pl)
            ka[m][pl] = row_operand(&S.K[kPar][pl][0][0], 16 * tt + c, m, g);
    f32x4 y;
    {
        f32x4 p0 = zero4(), p1 = zero4(), p2 = zero4();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x8 bh = ldsop(S.Sx, m, 0, l), bl = ldsop(S.Sx, m, 1, l);
            p0 = mfma_bf16(ka[m][0], bh, p0);
            p1 = mfma_bf16(ka[m][0], bl, p1);
            if constexpr (kSplit) p2 = mfma_bf16(ka[m][kSplit ? 1 : 0], bh, p2);
        }
        y = p0 + p1 + p2;
    }
    publish4(S.Yx, tt, l, y * cur.gam);
    f32x4 up;
    {
        f32x4 p0 = zero4(), p1 = zero4(), p2 = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            p0 = mfma_bf16(cur.ah[m], vb[m][0], p0);
            p1 = mfma_bf16(cur.al[m], vb[m][0], p1);
            if constexpr (kSplit) p2 = mfma_bf16(cur.ah[m], vb[m][kSplit ? 1 : 0], p2);
        }
        up = p0 + p1 + p2;
    }
    load_rows(cur, x, next);
    load_v(cur, x, next);
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch here: never sink it to its use
    __syncthreads();
    // P3: X = T_b (Gamma Y), U = U' - X, publish U and U~
    {
        f32x4 p0 = zero4(), p1 = zero4(), p2 = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x8 bh = ldsop(S.Yx, m, 0, l), bl = ldsop(S.Yx, m, 1, l);
            p0 = mfma_bf16(cur.ah[m], bh, p0);
            p1 = mfma_bf16(cur.ah[m], bl, p1);
            p2 = mfma_bf16(cur.al[m], bh, p2);
        }
        const f32x4 u = up - (p0 + p1 + p2);
        publish4(S.Ux, tt, l, u);
        publish4(S.Uy, tt, l, u * cur.gs);
    }
    const float gC = cur.gC;
    load_f(cur, x, next);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // P4: S^T = gamma_C S^T + K^T U~
    {
        acc *= gC;
        f32x4 lo = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x8 ubh = ldsop(S.Uy, m, 0, l), ubl = ldsop(S.Uy, m, 1, l);
            acc = mfma_bf16(kt[m][0], ubh, acc);
            lo = mfma_bf16(kt[m][0], ubl, lo);
            if constexpr (kSplit) lo = mfma_bf16(kt[m][kSplit ? 1 : 0], ubh, lo);
        }
        acc += lo;
    }
    load_rec(cur, x, next);
    __builtin_amdgcn_sched_barrier(0);
}

template <typename TIn, int kPar>
__device__ __forceinline__ void output_step(WalkOps<WalkIn<TIn>::kSplit>& cur, f32x4& acc,
                                            const WalkCtx<TIn>& x, int next,
                                            WalkLds<WalkIn<TIn>::kSplit>& S,
                                            const OutSink& out) {
    constexpr bool kSplit = WalkIn<TIn>::kSplit;
    const int w = x.w, l = x.l, g = l >> 4, c = l & 15, tt = w & 3;
    // P1
    publish4(S.Sx, w, l, acc);
    stage_rows<kSplit>(cur, S.Q, tt, l, cur.len);
    __syncthreads();
    // P2: Z = Q S^T; K^T operand for P4
    bf16x8 kt[2][kSplit ? 2 : 1], qa[4][kSplit ? 2 : 1];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int pl = 0; pl < (kSplit ? 2 : 1); ++pl)
            kt[m][pl] = tr_operand(&S.K[kPar][pl][0][0], kKS, 32 * m + 4 * g, 16 * w, l);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int pl = 0; pl < (kSplit ? 2 : 1); ++pl)
            qa[m][pl] = row_operand(&S.Q[pl][0][0], 16 * tt + c, m, g);
    f32x4 z;
    {
        f32x4 p0 = zero4(), p1 = zero4(), p2 = zero4();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x8 bh = ldsop(S.Sx, m, 0, l), bl = ldsop(S.Sx, m, 1, l);
            p0 = mfma_bf16(qa[m][0], bh, p0);
            p1 = mfma_bf16(qa[m][0], bl, p1);
            if constexpr (kSplit) p2 = mfma_bf16(qa[m][kSplit ? 1 : 0], bh, p2);
        }
        z = p0 + p1 + p2;
    }
    load_rows(cur, x, next);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // P3: nothing for output waves
    __syncthreads();
    // P4: state update for key tile w, then O = Gamma Z + A U
    {
        const float gC = cur.gC;
        acc *= gC;
        f32x4 lo = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x8 ubh = ldsop(S.Uy, m, 0, l), ubl = ldsop(S.Uy, m, 1, l);
            acc = mfma_bf16(kt[m][0], ubh, acc);
            lo = mfma_bf16(kt[m][0], ubl, lo);
            if constexpr (kSplit) lo = mfma_bf16(kt[m][kSplit ? 1 : 0], ubh, lo);
        }
        acc += lo;
    }
    {
        f32x4 p0 = zero4(), p1 = zero4(), p2 = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x8 bh = ldsop(S.Ux, m, 0, l), bl = ldsop(S.Ux, m, 1, l);
            p0 = mfma_bf16(cur.ah[m], bh, p0);
            p1 = mfma_bf16(cur.ah[m], bl, p1);
            p2 = mfma_bf16(cur.al[m], bh, p2);
        }
        const f32x4 ov = z * cur.gam + (p0 + p1 + p2);
        store_out_tile(out, ov, cur.t0, 16 * tt, cur.len, x.H, x.h, x.s, g, c);
    }
    load_f(cur, x, next);
    load_rec(cur, x, next);
    __builtin_amdgcn_sched_barrier(0);
}

template <typename TIn, bool kState>
__device__ __forceinline__ void walk_loop(f32x4& acc, const WalkCtx<TIn>& x, int c_begin,
                                          int c_end, WalkLds<WalkIn<TIn>::kSplit>& S,
                                          const OutSink& out) {
    WalkOps<WalkIn<TIn>::kSplit> A, B;
    const int last = c_end - 1;
    load_all(A, x, c_begin);
    load_all(B, x, c_begin + 1 < c_end ? c_begin + 1 : last);
    for (int ch = c_begin; ch < c_end; ch += 2) {
        if constexpr (kState) state_step<TIn, 0>(A, acc, x, ch + 2 < c_end ? ch + 2 : last, S);
        else output_step<TIn, 0>(A, acc, x, ch + 2 < c_end ? ch + 2 : last, S, out);
        if (ch + 1 >= c_end) break;
        if constexpr (kState) state_step<TIn, 1>(B, acc, x, ch + 3 < c_end ? ch + 3 : last, S);
        else output_step<TIn, 1>(B, acc, x, ch + 3 < c_end ? ch + 3 : last, S, out);
    }
}

template <typename TIn>
__global__ __launch_bounds__(kWalkThreads) void walk_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, int N, int H,
    const int32_t* __restrict__ rec, const int32_t* __restrict__ seq_off,
    const int32_t* __restrict__ num_chunks, const unsigned char* __restrict__ factors,
    const float* __restrict__ S0, OutSink out, float* __restrict__ S_final) {
    // XCD-aware mapping: the 8 value slices of one (sequence, head) share the
    // same blockIdx.x % 8, hence the same XCD and L2, which holds the chunk's
    // K, Q and factors that all 8 of them read.
    const int id = blockIdx.x;
    const int xcd = id & 7, rest = id >> 3;
    const int s = rest & 7, pg = rest >> 3;
    const int p = pg * 8 + xcd;
    if (p >= N * H) return;
    const int n = p / H, h = p - n * H;

    const int tid = threadIdx.x;
    const int w = wave_id(), l = tid & 63, g = l >> 4, c = l & 15;

    __shared__ __attribute__((aligned(16))) WalkLds<WalkIn<TIn>::kSplit> lds;

    const int nch = num_chunks[0];
    const int c_begin = seq_off[n];
    const int c_end = seq_off[n + 1] < nch ? seq_off[n + 1] : nch;
    const WalkCtx<TIn> x{q, k, v, factors, rec, H, h, s, w, l};

    // state: lane holds S^T[k = 16w + 4g + i][v = 16s + c] = S[v][k .. k+3]
    const size_t srow = ((size_t(n) * H + h) * kD + 16 * s + c) * kD + 16 * w + 4 * g;
    f32x4 acc = S0 ? *reinterpret_cast<const f32x4*>(S0 + srow) : zero4();
    if (c_begin < c_end) {
        if (w < 4) walk_loop<TIn, true>(acc, x, c_begin, c_end, lds, out);
        else walk_loop<TIn, false>(acc, x, c_begin, c_end, lds, out);
    }
    if (S_final) *reinterpret_cast<f32x4*>(S_final + srow) = acc;
}

}  // namespace

hipError_t launch_prep(const void* q, const void* k, rda_dtype dt, const float* a,
                       const float* b, int32_t heads, int32_t max_chunks, const int32_t* rec,
                       const int32_t* num_chunks, unsigned char* factors, hipStream_t stream,
                       int32_t single_T, int32_t* rec_out, int32_t* seq_off_out,
                       int32_t* num_out) {
    const unsigned grid = unsigned(int64_t(max_chunks) * heads);
    if (grid == 0) return hipSuccess;
    if (dt == RDA_BF16) {
        return launch_prep_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), a,
                                b, heads, max_chunks, rec, num_chunks, factors, single_T, rec_out,
                                seq_off_out, num_out, stream);
    } else {
        hipLaunchKernelGGL(prep_kernel<true>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const float*>(q), static_cast<const float*>(k), a, b,
                           heads, rec, num_chunks, factors, single_T, rec_out, seq_off_out,
                           num_out);
    }
    return hipGetLastError();
}

hipError_t launch_walk(const void* q, const void* k, const void* v, rda_dtype dt,
                       int32_t num_seqs, int32_t heads, const int32_t* rec,
                       const int32_t* seq_off, const int32_t* num_chunks,
                       const unsigned char* factors, const float* S0, OutSink out,
                       float* S_final, hipStream_t stream) {
    const int64_t pairs = int64_t(num_seqs) * heads;
    const unsigned grid = unsigned(64 * ((pairs + 7) / 8));
    if (dt == RDA_BF16) {
        const WalkJob job{S0, S_final, 0, 0};
        return launch_walk_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                static_cast<const uint16_t*>(v), num_seqs, heads, rec, seq_off,
                                num_chunks, factors, out, &job, 1, 0, true, stream);
    } else {
        hipLaunchKernelGGL(walk_kernel<float>, dim3(grid), dim3(kWalkThreads), 0, stream,
                           static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), num_seqs, heads, rec, seq_off,
                           num_chunks, factors, S0, out, S_final);
    }
    return hipGetLastError();
}

}  // namespace rda
