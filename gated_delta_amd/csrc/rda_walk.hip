// rda_walk.hip -- the sequential chunk walk of the chunked RDA prefill for
// bf16 inputs on gfx950 (the chunk algebra and the operand conventions are
// those stated at the top of rda_prefill.hip; T_b, A and the gates come from
// the prep kernel).
//
// One workgroup per (sequence, head, 16-channel value slice), three roles:
//   state waves 0..3   carry the recurrence.  Wave w owns S^T for key block
//                      w (key tiles 2w, 2w+1, MFMA accumulators) and token
//                      tile w of the chunk-local products.  Per chunk:
//     P1  publish its S^T block (bf16 hi/lo) as ready B operands, keys in
//         natural order so that K and Q rows are single 16-byte reads
//     P2  Y = K S^T, publish E = V - Gamma Y (the chunk's errors before the
//         solve)
//     P3  U = T_b E; publish U and U~ = diag(gamma_C/gamma) U
//     P4  S^T = gamma_C S^T + K^T U~
//   output waves 4..7  produce the outputs of token tile tt = w - 4:
//     P2, P3  Z = Q S^T (key blocks 0-1 before the second barrier, 2-3 after
//             it, which spreads their LDS reads over two windows)
//     P4      O = Gamma Z + A U, stored
//   loader waves 8..15 stream each chunk's operands -- the K and Q tiles, the
//                      packed T_b and A factors, the gates and this slice's V
//                      columns -- into a two-stage LDS ring with LDS-DMA
//                      (global_load_lds_dwordx4), and touch the lines of
//                      chunks further ahead so that they sit in L2 when the
//                      DMA asks for them.
// A chunk's DMA goes out in one burst as soon as its stage is free (after
// the third barrier of the chunk two before it); the factor slots that are
// zero are not streamed.
// The compute waves issue no global loads at all (a wave stalls when it
// issues a memory instruction into a full queue, and any such stall would
// land on the recurrence), and the output work runs beside the recurrence on
// the other wave slots instead of lengthening it.
//
// The same kernel serves the segmented form of the state pass: a launch may
// carry two jobs over the same chunks that differ only in the starting state
// (taken from S0, zero, or the identity), in whether the values count (a job
// with zero values walks the state's own transition), and in where the final
// state goes;
// the sequences may be equal runs of chunks of one sequence (segments); and
// the instantiation without outputs streams neither Q nor A and leaves its
// output waves idle at the barriers.
//
// A launch may also walk only a range of one sequence's chunks (from a saved
// state, to a saved state) and carry prep workgroups after the walk's, which
// run the prep of later chunks (rda_prep.h) on the CUs the walk leaves free;
// nothing in the launch waits on them.
//
// Past the end of a chunk (len < 64) the loaders duplicate the last valid
// token row instead of zeroing: T_b has zero rows and columns there (b = 0),
// so U and U~ vanish on those rows and no duplicate reaches S or a stored
// output; they only need to be finite, which copies of real rows are.
#include "rda_internal.h"
#include "rda_lds.h"
#include "rda_norm.h"
#include "rda_out.h"
#include "rda_prep.h"

namespace rda {

namespace {

constexpr int kStateWaves = 4;
constexpr int kOutWaves = 4;
constexpr int kLoaders = 8;
constexpr int kLoader0 = kStateWaves + kOutWaves;   // wave index of the first loader
constexpr int kThreads = (kStateWaves + kOutWaves + kLoaders) * 64;
constexpr int kPfAhead = 4;                          // L2 touch distance (chunks)

// One chunk's operands in LDS (68608 bytes, every part whole 1 KiB DMA blocks).
struct Stage {
    uint16_t K[kC * kD];   // 64 token rows x 256 B; 16-byte granules swizzled per row
    uint16_t Q[kC * kD];
    u32x4 Tb[16][64];      // T_b packed: [(tile * 2 + block) * 2 + hi/lo][lane]
    u32x4 Am[16][64];      // A, same packing
    uint16_t V[kC * 16];   // this slice's 16 value channels, 32 B per token row
    float G[256];          // gamma, gamma_C / gamma, gamma_C, running log gate
};

struct Lds {
    Stage st[2];
    u32x4 Sx[4][2][64];    // S^T key block m hi/lo; lane (g, c): keys 32m + 8g .. +7, column c
    u32x4 Ex[2][2][64];    // E token block (tiles 2m, 2m+1) hi/lo
    u32x4 Ux[2][2][64];    // U
    u32x4 Uy[2][2][64];    // U~
    float sink[64];        // landing words of the L2 touches
};

static_assert(sizeof(Stage) == 67 * 1024, "stage is whole 1 KiB DMA blocks");
static_assert(sizeof(Lds) <= 160 * 1024, "LDS budget of one workgroup");

// A launch may also carry prep workgroups (after the walk's), each running
// four prep items at a time in four 256-thread groups: the walk's LDS or
// four PrepLds.
union WalkOrPrepLds {
    Lds walk;
    PrepLds prep[4];
};
static_assert(sizeof(WalkOrPrepLds) == sizeof(Lds), "prep groups fit in the walk's LDS");

struct Ctx {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const unsigned char* factors;
    const int32_t* rec;
    int H, h, s, l;
};

__device__ __forceinline__ const unsigned char* chunk_factors(const Ctx& x, int chunk) {
    return x.factors + (size_t(chunk) * x.H + x.h) * kChunkHeadBytes;
}

__device__ __forceinline__ const uint16_t* token_row(const uint16_t* base, const Ctx& x,
                                                     int t0, int r) {
    return base + (size_t(t0 + r) * x.H + x.h) * kD;
}

// ---- loader waves -------------------------------------------------------------
// The chunk's operands are 67 DMA blocks of 1 KiB: K 0..15, Q 16..31, T_b
// 32..47, A 48..63, V 64..65, G 66.  Loader i owns the blocks i, i + 8, ...
// (9 or 8 of them, fewer the unread factor blocks); loaders 0 and 1 also
// touch one line set each for L2.

__device__ __forceinline__ void issue_block(const Ctx& x, int t0, int len,
                                            const unsigned char* F, int blk, Stage& st) {
    const int L = x.l;
    if (blk < 32) {   // K or Q tile block: rows 4n .. 4n+3
        const int n = blk & 15;
        const int r = 4 * n + (L >> 4);
        const int rr = r < len ? r : len - 1;
        const int j = (L & 15) ^ swz(r);
        const uint16_t* src = blk < 16 ? x.k : x.q;
        uint16_t* dst = blk < 16 ? st.K : st.Q;
        dma16(token_row(src, x, t0, rr) + 8 * j, reinterpret_cast<char*>(dst) + 1024 * n);
    } else if (blk < 64) {   // T_b then A: contiguous 32 KiB in the factors
        dma16(F + kOffTb + 1024 * (blk - 32) + 16 * L,
              reinterpret_cast<char*>(st.Tb) + 1024 * (blk - 32));
    } else if (blk < 66) {   // V slice rows 32n .. 32n+31
        const int n = blk - 64;
        const int r = 32 * n + (L >> 1);
        const int rr = r < len ? r : len - 1;
        dma16(token_row(x.v, x, t0, rr) + 16 * x.s + 8 * (L & 1),
              reinterpret_cast<char*>(st.V) + 1024 * n);
    } else {
        dma16(F + kOffG + 16 * L, st.G);
    }
}

// Touch this slice's share of a chunk's 128-byte lines, one line per lane.
// Half kHalf of the shared lines (K, Q, T_b, A: 512 lines, every eighth
// one for this slice), plus (half 1) a quarter of the V lines that this
// slice shares with the three other slices of its 64-channel group.
template <int kHalf>
__device__ __forceinline__ void touch_chunk(const Ctx& x, int chunk, float* sink) {
    const int t0 = x.rec[4 * chunk + 1], len = x.rec[4 * chunk + 2];
    const int L = x.l;
    const unsigned char* F = chunk_factors(x, chunk);
    const void* a;
    const int u = 32 * kHalf + (L & 31);   // this slice's shared line index, 0..63
    const int i = x.s + 8 * u;             // shared line, 0..511
    if (kHalf == 1 && L >= 32) {
        const int r = 4 * (L & 15) + (x.s & 3);
        const int rr = r < len ? r : len - 1;
        a = token_row(x.v, x, t0, rr) + 64 * (x.s >> 2);
    } else if (i < 256) {
        const int r = (i & 127) >> 1;
        const int rr = r < len ? r : len - 1;
        a = token_row(i < 128 ? x.k : x.q, x, t0, rr) + 64 * (i & 1);
    } else {
        a = F + kOffTb + 128 * (i - 256);   // T_b then A: contiguous 32 KiB
    }
    dma4(a, sink);
}

// Blocks of the packed factors that no wave reads: slots (tile, block 1) of
// token tiles 0 and 1, whose operands are zero (both factors are lower
// triangular).  They are neither written by the prep kernel nor streamed.
// Without outputs the Q tile (blocks 16..31) and A (48..63) are not read
// either.
template <bool kOut>
constexpr bool unread_block(int blk) {
    const int slot = (blk - 32) & 15;   // (tile * 2 + block) * 2 + hi/lo
    if (!kOut && ((blk >= 16 && blk < 32) || (blk >= 48 && blk < 64))) return true;
    return blk >= 32 && blk < 64 && ((slot >> 1) & 1) == 1 && (slot >> 2) < 2;
}

// Number of blocks loader kI issues per chunk.
template <int kI, bool kOut>
constexpr int loader_blocks() {
    int n = 0;
    for (int blk = kI; blk < 67; blk += 8) n += unread_block<kOut>(blk) ? 0 : 1;
    return n;
}

// Loader kI's blocks of `chunk`, in three groups of ascending block number
// (the compiler keeps the order inside each group; left free to interleave
// all of them, it produced an order measured slower).
template <int kI, int kGroup, bool kOut>
__device__ __forceinline__ void issue_group(const Ctx& x, int chunk, Stage& st) {
    const int t0 = x.rec[4 * chunk + 1], len = x.rec[4 * chunk + 2];
    const unsigned char* F = chunk_factors(x, chunk);
#pragma unroll
    for (int q = 3 * kGroup; q < 3 * kGroup + 3; ++q) {
        const int blk = kI + 8 * q;
        if (blk < 67 && !unread_block<kOut>(blk)) issue_block(x, t0, len, F, blk, st);
    }
}

template <int kI, bool kOut>
__device__ __forceinline__ void issue_chunk(const Ctx& x, int chunk, Stage& st) {
    issue_group<kI, 0, kOut>(x, chunk, st);
    issue_group<kI, 1, kOut>(x, chunk, st);
    issue_group<kI, 2, kOut>(x, chunk, st);
}

// A chunk's blocks go out at once, right after the third barrier of the
// chunk two before it (its stage is free from then on), followed by one L2
// touch from loaders 0 and 1.  Before a chunk's first barrier each loader
// waits until only the blocks of the chunk after it (and that touch) may
// still be in flight: loads complete in issue order.  (Spreading the blocks
// over the three barrier windows instead was measured slightly slower.)
template <int kI, bool kOut>
__device__ void loader(const Ctx& x, int c0, int c_end, Lds& S) {
    constexpr int kPending = loader_blocks<kI, kOut>() + (kI < 2 ? 1 : 0);
    const int last = c_end - 1;
    auto cl = [last](int c) { return c < last ? c : last; };
    if constexpr (kI < 2) {
#pragma unroll
        for (int d = 1; d < kPfAhead; ++d) touch_chunk<kI>(x, cl(c0 + d), S.sink);
    }
    issue_chunk<kI, kOut>(x, c0, S.st[0]);
    issue_chunk<kI, kOut>(x, cl(c0 + 1), S.st[1]);
    if constexpr (kI < 2) touch_chunk<kI>(x, cl(c0 + kPfAhead), S.sink);
    for (int c = c0; c < c_end; ++c) {
        wait_vm<kPending>();
        __builtin_amdgcn_s_barrier();   // A
        __builtin_amdgcn_s_barrier();   // B
        __builtin_amdgcn_s_barrier();   // C: chunk c's stage is free
        issue_chunk<kI, kOut>(x, cl(c + 2), S.st[(c - c0) & 1]);
        if constexpr (kI < 2) touch_chunk<kI>(x, cl(c + 2 + kPfAhead), S.sink);
    }
    wait_vm<0>();   // nothing may land in LDS after the workgroup ends
}

// ---- LDS operand helpers -----------------------------------------------------------

// Transposed operand of the swizzled K tile: lane (g, c) receives column
// 16 kt + c of rows {32m + 4g + i, 32m + 16 + 4g + i : i < 4} (the permuted
// token order of the packed factors and of the exchanged U~).
// ds_read_b64_tr_b16 gives output lane i of a 16-lane group element i % 4 of
// the 8 bytes that source lane 4e + i / 4 addresses, so source lane j points
// at row r0 + j / 4, columns 16 kt + 4 (j % 4) .. +3.
__device__ __forceinline__ bf16x8 tr_op(const uint16_t* T, int m, int kt, int l) {
    const int g = l >> 4, j = l & 15;
    const int r = 32 * m + 4 * g + (j >> 2);
    const int gran = 2 * kt + ((j >> 1) & 1), hb = 8 * (j & 1);
    const unsigned char* base = reinterpret_cast<const unsigned char*>(T);
    const u32x2 a = tr_read(base + r * 256 + 16 * (gran ^ swz(r)) + hb);
    const u32x2 b = tr_read(base + (r + 16) * 256 + 16 * (gran ^ swz(r + 16)) + hb);
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// This slice's V in accumulator layout for token tile t: lane (g, c) gets
// channel c of tokens 16t + 4g + i, i < 4 (one transposing read).
__device__ __forceinline__ u32x2 tr_vd(const uint16_t* V, int t, int l) {
    const int g = l >> 4, j = l & 15;
    return tr_read(reinterpret_cast<const unsigned char*>(V) + (16 * t + 4 * g + (j >> 2)) * 32 +
                   8 * (j & 3));
}

__device__ __forceinline__ bf16x8 packed(const u32x4 (*P)[64], int tile, int m, int hl, int l) {
    return __builtin_bit_cast(bf16x8, P[(tile * 2 + m) * 2 + hl][l]);
}

// ---- state waves -------------------------------------------------------------------

__device__ __forceinline__ void state_step(const Ctx& x, int w, const Stage& st, Lds& S,
                                           f32x4& s0, f32x4& s1, bool zero_v) {
    const int l = x.l, g = l >> 4, c = l & 15;
    const int nb = (w >> 1) + 1;   // token blocks at or below token tile w
    // P1: publish S^T block w in natural key order: tile 2w (keys 32w + 4g + e)
    // -> lane c + 16 (g / 2), tile 2w + 1 -> lane c + 16 (2 + g / 2), 8-byte half g % 2
    {
        const int lane0 = c + 16 * (g >> 1), lane1 = lane0 + 32, half = g & 1;
        uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
        split_pk(s0[0], s0[1], h0, l0);
        split_pk(s0[2], s0[3], h1, l1);
        split_pk(s1[0], s1[1], h2, l2);
        split_pk(s1[2], s1[3], h3, l3);
        reinterpret_cast<u32x2*>(&S.Sx[w][0][lane0])[half] = u32x2{h0, h1};
        reinterpret_cast<u32x2*>(&S.Sx[w][1][lane0])[half] = u32x2{l0, l1};
        reinterpret_cast<u32x2*>(&S.Sx[w][0][lane1])[half] = u32x2{h2, h3};
        reinterpret_cast<u32x2*>(&S.Sx[w][1][lane1])[half] = u32x2{l2, l3};
    }
    __syncthreads();   // A
    // P2: Y = K S^T (token tile w), publish E = V - Gamma Y
    f32x4 gs;
    float gC;
    {
        bf16x8 sh[4], sl[4], ka[4];
        const f32x4 gam = *reinterpret_cast<const f32x4*>(st.G + kGGam + 16 * w + 4 * g);
        gs = *reinterpret_cast<const f32x4*>(st.G + kGScale + 16 * w + 4 * g);
        gC = st.G[kGC];
        const u32x2 vv = tr_vd(st.V, w, l);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            sh[m] = ldsop(S.Sx, m, 0, l);
            sl[m] = ldsop(S.Sx, m, 1, l);
            ka[m] = row_op(st.K, 16 * w + c, m, g);
        }
        f32x4 y0 = zero4(), y1 = zero4();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            y0 = mfma_bf16(ka[m], sh[m], y0);
            y1 = mfma_bf16(ka[m], sl[m], y1);
        }
        const f32x4 vf = zero_v ? zero4()
                                : f32x4{__uint_as_float(vv[0] << 16),
                                        __uint_as_float(vv[0] & 0xffff0000u),
                                        __uint_as_float(vv[1] << 16),
                                        __uint_as_float(vv[1] & 0xffff0000u)};
        publish4(S.Ex, w, l, vf - (y0 + y1) * gam);
    }
    __syncthreads();   // B
    // P3: U = T_b E (T_b is lower triangular: blocks m <= w / 2); K^T
    // operands for P4
    bf16x8 kt[2][2];
    {
        bf16x8 eh[2], el[2], th[2], tl[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (m >= nb) break;
            eh[m] = ldsop(S.Ex, m, 0, l);
            el[m] = ldsop(S.Ex, m, 1, l);
            th[m] = packed(st.Tb, w, m, 0, l);
            tl[m] = packed(st.Tb, w, m, 1, l);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int m = 0; m < 2; ++m) kt[j][m] = tr_op(st.K, m, 2 * w + j, l);
        f32x4 p0 = zero4(), p1 = zero4(), p2 = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (m >= nb) break;
            mma3(th[m], tl[m], eh[m], el[m], p0, p1, p2);
        }
        const f32x4 u = p0 + p1 + p2;
        publish4(S.Ux, w, l, u);
        publish4(S.Uy, w, l, u * gs);
    }
    __syncthreads();   // C
    // P4: S^T = gamma_C S^T + K^T U~
    {
        bf16x8 uh[2], ul[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            uh[m] = ldsop(S.Uy, m, 0, l);
            ul[m] = ldsop(S.Uy, m, 1, l);
        }
        f32x4 a0 = s0 * gC, a1 = s1 * gC, b0 = zero4(), b1 = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            a0 = mfma_bf16(kt[0][m], uh[m], a0);
            b0 = mfma_bf16(kt[0][m], ul[m], b0);
            a1 = mfma_bf16(kt[1][m], uh[m], a1);
            b1 = mfma_bf16(kt[1][m], ul[m], b1);
        }
        s0 = a0 + b0;
        s1 = a1 + b1;
    }
}

// ---- output waves ------------------------------------------------------------------

__device__ __forceinline__ void output_step(const Ctx& x, int tt, int ch, const Stage& st, Lds& S,
                                            const OutSink& out) {
    const int l = x.l, g = l >> 4, c = l & 15;
    const int nb = (tt >> 1) + 1;
    const int t0 = x.rec[4 * ch + 1], len = x.rec[4 * ch + 2];
    __syncthreads();   // A
    // Z = Q S^T, key blocks 0 and 1 before barrier B and blocks 2 and 3 (and
    // the A operands) after it, which spreads the output waves' LDS reads
    // over both windows in which the published S and this stage are valid
    f32x4 z0 = zero4(), z1 = zero4();
    bf16x8 ah[2], al[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (half == 1) __syncthreads();   // B
        bf16x8 sh[2], sl[2], qa[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int m = 2 * half + i;
            sh[i] = ldsop(S.Sx, m, 0, l);
            sl[i] = ldsop(S.Sx, m, 1, l);
            qa[i] = row_op(st.Q, 16 * tt + c, m, g);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            z0 = mfma_bf16(qa[i], sh[i], z0);
            z1 = mfma_bf16(qa[i], sl[i], z1);
        }
    }
    const f32x4 gam = *reinterpret_cast<const f32x4*>(st.G + kGGam + 16 * tt + 4 * g);
    const f32x4 z = (z0 + z1) * gam;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        if (m >= nb) break;
        ah[m] = packed(st.Am, tt, m, 0, l);
        al[m] = packed(st.Am, tt, m, 1, l);
    }
    __syncthreads();   // C
    // P4: O = Gamma Z + A U
    {
        bf16x8 xh[2], xl[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (m >= nb) break;
            xh[m] = ldsop(S.Ux, m, 0, l);
            xl[m] = ldsop(S.Ux, m, 1, l);
        }
        f32x4 p0 = zero4(), p1 = zero4(), p2 = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (m >= nb) break;
            mma3(ah[m], al[m], xh[m], xl[m], p0, p1, p2);
        }
        const f32x4 ov = z + (p0 + p1 + p2);
        store_out_tile(out, ov, t0, 16 * tt, len, x.H, x.h, x.s, g, c);
    }
}

// The prep workgroups of a launch: prep items [item_lo, item_hi) (item =
// chunk * H + head) of one sequence of single_T tokens without offsets, four
// consecutive items per round, writing their chunks' table entries too.
__device__ void prep_role(const WalkSide& X, PrepLds (&S)[4]) {
    const int sub = wave_id() >> 2;          // which of the four groups
    const int w = wave_id() & 3;             // wave within the group
    const int tid = threadIdx.x & 255;
    const int nprep = X.prep_blocks;
    const int wg = int(blockIdx.x) - X.walk_blocks;
    const int H = X.args.H;
    for (int base = X.item_lo + 4 * wg; base < X.item_hi; base += 4 * nprep) {
        const int item = base + sub;
        const bool valid = item < X.item_hi;
        const int chunk = valid ? item / H : 0;
        const int h = valid ? item - chunk * H : 0;
        const int t0 = kC * chunk;
        const int len = valid ? min(kC, X.single_T - t0) : 1;
        if (valid && h == 0)
            prep_table_entry(chunk, t0, len, X.nch, tid, X.rec_out, X.seq_off_out, X.num_out);
        prep_item(X.args, chunk, h, t0, len, valid, S[sub], tid, w);
        __syncthreads();   // this round's LDS is rewritten by the next
    }
}

// The norm workgroups of a launch: 64 rows at a time, 16 lanes per row,
// over rows [row_lo, row_hi) of the 16-bit form.
template <typename TG, typename TO, int kAct>
__device__ void norm_rows(const WalkNorm& N, int wg, int nwg) {
    const int c = threadIdx.x & 15, grp = threadIdx.x >> 4;
    for (int64_t base = N.row_lo + 64 * int64_t(wg); base < N.row_hi; base += 64 * int64_t(nwg)) {
        const int64_t r0 = base + grp;
        norm_gate_row<TG, TO, kAct, true>(nullptr, N.y, static_cast<const TG*>(N.g), N.w, N.eps,
                                          min(r0, N.row_hi - 1), r0 < N.row_hi,
                                          static_cast<TO*>(N.out), c);
    }
}

template <int kAct>
__device__ void norm_rows_act(const WalkNorm& N, int wg, int nwg) {
    if (N.g16 && N.o16) norm_rows<uint16_t, uint16_t, kAct>(N, wg, nwg);
    else if (N.g16) norm_rows<uint16_t, float, kAct>(N, wg, nwg);
    else if (N.o16) norm_rows<float, uint16_t, kAct>(N, wg, nwg);
    else norm_rows<float, float, kAct>(N, wg, nwg);
}

__device__ void norm_role(const WalkSide& X) {
    const int wg = int(blockIdx.x) - X.walk_blocks - X.prep_blocks;
    const WalkNorm& N = X.norm;
    if (N.act == RDA_GATE_SIGMOID) norm_rows_act<RDA_GATE_SIGMOID>(N, wg, N.blocks);
    else if (N.act == RDA_GATE_SILU) norm_rows_act<RDA_GATE_SILU>(N, wg, N.blocks);
    else norm_rows_act<RDA_GATE_NONE>(N, wg, N.blocks);
}

template <bool kOut>
__global__ __launch_bounds__(kThreads) void walk_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int N, int H, const int32_t* __restrict__ rec,
    const int32_t* __restrict__ seq_off, const int32_t* __restrict__ num_chunks,
    const unsigned char* __restrict__ factors, OutSink out, WalkJob j0, WalkJob j1,
    int seg_chunks, WalkSide X) {
    __shared__ __attribute__((aligned(16))) WalkOrPrepLds shm;
    if (int(blockIdx.x) >= X.walk_blocks + X.prep_blocks) {
        norm_role(X);
        return;
    }
    if (int(blockIdx.x) >= X.walk_blocks) {
        prep_role(X, shm.prep);
        return;
    }
    Lds& lds = shm.walk;
    // Jobs split the grid in halves.  Within a job the mapping is XCD-aware:
    // the 8 value slices of one (sequence, head) share blockIdx.x % 8, hence
    // one XCD and its L2, which then holds the chunk's K, Q and factors once
    // for all of them.
    const int per_job = 64 * ((N * H + 7) / 8);
    const int job = blockIdx.x >= per_job ? 1 : 0;
    const WalkJob J = job ? j1 : j0;
    const int id = blockIdx.x - job * per_job;
    const int xcd = id & 7, rest = id >> 3;
    const int s = rest & 7, pg = rest >> 3;
    const int p = pg * 8 + xcd;
    if (p >= N * H) return;
    const int n = p / H, h = p - n * H;

    const int w = wave_id(), l = threadIdx.x & 63, g = l >> 4, c = l & 15;
    const int nch = num_chunks[0];
    // sequence n's chunks: from the table, or the n-th run of seg_chunks
    int c0, c_end;
    if (seg_chunks > 0) {
        c0 = n * seg_chunks < nch ? n * seg_chunks : nch;
        c_end = c0 + seg_chunks < nch ? c0 + seg_chunks : nch;
    } else {
        c0 = seq_off[n];
        c_end = seq_off[n + 1] < nch ? seq_off[n + 1] : nch;
    }
    if (X.c_hi > 0) {   // one sequence walked over chunks [c_lo, c_hi) only
        c0 = X.c_lo < nch ? X.c_lo : nch;
        c_end = X.c_hi < nch ? X.c_hi : nch;
    }
    const Ctx x{q, k, v, factors, rec, H, h, s, l};

    if (w >= kLoader0) {
        if (c0 < c_end) {
            switch (w - kLoader0) {
                case 0: loader<0, kOut>(x, c0, c_end, lds); break;
                case 1: loader<1, kOut>(x, c0, c_end, lds); break;
                case 2: loader<2, kOut>(x, c0, c_end, lds); break;
                case 3: loader<3, kOut>(x, c0, c_end, lds); break;
                case 4: loader<4, kOut>(x, c0, c_end, lds); break;
                case 5: loader<5, kOut>(x, c0, c_end, lds); break;
                case 6: loader<6, kOut>(x, c0, c_end, lds); break;
                default: loader<7, kOut>(x, c0, c_end, lds); break;
            }
        }
        return;
    }
    if (w >= kStateWaves) {
        for (int ch = c0; ch < c_end; ++ch) {
            if constexpr (kOut) {
                output_step(x, w - kStateWaves, ch, lds.st[(ch - c0) & 1], lds, out);
            } else {
                __syncthreads();   // A
                __syncthreads();   // B
                __syncthreads();   // C
            }
        }
        return;
    }
    // lane holds S^T[k = 16 kt + 4g + e][v = 16s + c] = S[v][k] for kt = 2w, 2w+1
    const size_t srow = ((size_t(n) * H + h) * kD + 16 * s + c) * kD + 32 * w + 4 * g;
    f32x4 s0 = zero4(), s1 = zero4();
    if (J.identity) {
        const int vrow = 16 * s + c, key = 32 * w + 4 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s0[e] = key + e == vrow ? 1.f : 0.f;
            s1[e] = key + 16 + e == vrow ? 1.f : 0.f;
        }
    } else if (J.S0) {
        s0 = *reinterpret_cast<const f32x4*>(J.S0 + srow);
        s1 = *reinterpret_cast<const f32x4*>(J.S0 + srow + 16);
    }
    const bool zero_v = J.zero_v != 0;
    for (int ch = c0; ch < c_end; ++ch)
        state_step(x, w, lds.st[(ch - c0) & 1], lds, s0, s1, zero_v);
    if (J.S_final) {
        *reinterpret_cast<f32x4*>(J.S_final + srow) = s0;
        *reinterpret_cast<f32x4*>(J.S_final + srow + 16) = s1;
    }
}

}  // namespace

hipError_t launch_walk_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            int32_t num_seqs, int32_t heads, const int32_t* rec,
                            const int32_t* seq_off, const int32_t* num_chunks,
                            const unsigned char* factors, OutSink out, const WalkJob* jobs,
                            int32_t num_jobs, int32_t seg_chunks, bool outputs,
                            hipStream_t stream, const WalkSide* extra) {
    const int64_t pairs = int64_t(num_seqs) * heads;
    const unsigned walk_grid = unsigned(num_jobs * 64 * ((pairs + 7) / 8));
    WalkSide X{};
    if (extra) X = *extra;
    X.walk_blocks = int(walk_grid);
    const unsigned grid =
        walk_grid + unsigned(extra ? extra->prep_blocks + extra->norm.blocks : 0);
    const WalkJob none{nullptr, nullptr, 0, 0};
    const WalkJob j1 = num_jobs > 1 ? jobs[1] : none;
    if (outputs)
        hipLaunchKernelGGL(walk_bf16_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, q, k, v,
                           num_seqs, heads, rec, seq_off, num_chunks, factors, out, jobs[0], j1,
                           seg_chunks, X);
    else
        hipLaunchKernelGGL(walk_bf16_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, q, k,
                           v, num_seqs, heads, rec, seq_off, num_chunks, factors, out, jobs[0], j1,
                           seg_chunks, X);
    return hipGetLastError();
}

}  // namespace rda
