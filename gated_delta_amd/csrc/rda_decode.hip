// rda_decode.hip -- one decode step of the RDA gated delta rule, in place.
//
// Per (batch, head) the state S [128 x 128] fp32 (row i = value channel,
// column j = key channel) is read once and written once.  The recurrent
// step -- decay, the residual e = v - S'k of the decayed state at the key,
// the rank-one write b e k^T, read-out with the updated state -- is
// the one the "Raon-1 nano" teardown (section "The other 1.5B: a hybrid
// built to forget") describes.  Because each row of S is updated
// independently, one pass suffices: for row i,
//
//     (Sk)_i = S_i . k,   (Sq)_i = S_i . q,   kappa = k . q
//     e_i    = v_i - a (Sk)_i
//     S'_i   = a S_i + b e_i k
//     o_i    = S'_i . q = a (Sq)_i + b e_i kappa
//
// Decode is bound by HBM: 128 KiB of state traffic per (batch, head) against
// ~0.9 flop per byte.  Mapping: two 256-thread workgroups per (batch, head),
// each owning 64 rows of the state; 16 lanes own one row (each lane 8
// columns: 4 in each 64-column half, so every load instruction of a
// wavefront reads four 256-byte runs), a lane holds 4 rows, i.e. the
// workgroup's 32 KiB of state is in flight at once.  (One workgroup per
// (batch, head) holding all 64 KiB was measured 11 % slower: fewer, larger
// workgroups leave a ragged last round; quarters were in between.)  Row dot
// products are 16-lane DPP reductions.
#include "rda_device.h"
#include "rda_internal.h"
#include "rda_lds.h"
#include "rda_prologue_math.h"

namespace rda {

// The single-pass update of one lane's 4 state rows (rows rbase + 4p, p < 4,
// columns 4c.. and 64+4c..) for one token: the dot products, the error, the
// in-place state write and this row set's outputs (lane c < 4 returns the
// output of row rbase + 4c).  Shared by the decode step kernels so that they
// give the same bits.
// Every multiply-add is an explicit fmaf and the compiler may fuse nothing
// else, so each kernel that inlines this runs the same IEEE operations.
__device__ __forceinline__ float decode_rows(const f32x4 (&s)[4][2], const float (&kx)[8],
                                             const float (&qx)[8], float av, float bv,
                                             const float (&vr)[4], int c, float* __restrict__ Sb,
                                             int rbase) {
#pragma clang fp contract(off)
    float kap = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) kap = fmaf(kx[j], qx[j], kap);
    kap = dpp_sum16(kap);

    float o_mine = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sk = fmaf(s[p][1][j], kx[4 + j], fmaf(s[p][0][j], kx[j], sk));
            sq = fmaf(s[p][1][j], qx[4 + j], fmaf(s[p][0][j], qx[j], sq));
        }
        sk = dpp_sum16(sk);
        sq = dpp_sum16(sq);
        const float e = fmaf(-av, sk, vr[p]);
        const float be = bv * e;
        const float orow = fmaf(av, sq, be * kap);
        if (c == p) o_mine = orow;
        f32x4 n0, n1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            n0[j] = fmaf(av, s[p][0][j], be * kx[j]);
            n1[j] = fmaf(av, s[p][1][j], be * kx[4 + j]);
        }
        const int row = rbase + 4 * p;
        *reinterpret_cast<f32x4*>(Sb + row * kD + 4 * c) = n0;
        *reinterpret_cast<f32x4*>(Sb + row * kD + 64 + 4 * c) = n1;
    }
    return o_mine;
}

template <typename TIn>
__global__ __launch_bounds__(256) void decode_step_kernel(const TIn* __restrict__ q,
                                                          const TIn* __restrict__ k,
                                                          const TIn* __restrict__ v,
                                                          const float* __restrict__ a,
                                                          const float* __restrict__ b,
                                                          float* __restrict__ S,
                                                          float* __restrict__ o) {
    const int64_t bh = blockIdx.x >> 1;
    const int half = blockIdx.x & 1;
    const int t = threadIdx.x;
    const int w = wave_id();      // wavefront 0..3 -> rows 64 half + 16w .. +15
    const int g = (t >> 4) & 3;   // 16-lane group within the wavefront
    const int c = t & 15;         // lane within the group -> columns 4c.., 64+4c..
    float* __restrict__ Sb = S + bh * (kD * kD);

    // all state loads first: 8 rows x 2 float4 per lane
    f32x4 s[4][2];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = 64 * half + 16 * w + 4 * p + g;
        s[p][0] = *reinterpret_cast<const f32x4*>(Sb + row * kD + 4 * c);
        s[p][1] = *reinterpret_cast<const f32x4*>(Sb + row * kD + 64 + 4 * c);
    }
    float kx[8], qx[8];
    load4<TIn>(k + bh * kD + 4 * c, kx);
    load4<TIn>(k + bh * kD + 64 + 4 * c, kx + 4);
    load4<TIn>(q + bh * kD + 4 * c, qx);
    load4<TIn>(q + bh * kD + 64 + 4 * c, qx + 4);
    const float av = a[bh];
    const float bv = b[bh];
    float vr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) vr[p] = load1<TIn>(v + bh * kD + 64 * half + 16 * w + 4 * p + g);

    const float o_mine = decode_rows(s, kx, qx, av, bv, vr, c, Sb, 64 * half + 16 * w + g);
    if (c < 4) o[bh * kD + 64 * half + 16 * w + 4 * c + g] = o_mine;
}

// Several tokens per (batch, head) in one pass: the state is read once,
// carried in registers through the tokens in order (the per-row update of
// the one-token kernel above, token after token, in the same layout), and
// written at most once.  `n_acc` tokens (the per-sequence accept count,
// clamped to [0, tokens]) are committed: the state after the first n_acc
// tokens goes to S_out.  With kOut the outputs of all `tokens` tokens are
// produced, so a verify of drafted tokens and the commit of its accepted
// prefix share one pass when the count is known; otherwise a read-only
// verify (S_out = nullptr) is followed by a commit-only pass (kOut = false:
// stops after n_acc tokens and never reads q).  Token t of sequence n, head
// h sits at row (n * tokens + t) * heads + h of q, k, v, a, b and o, the
// packed layout of equal-length sequences.  The next token's inputs are
// loaded, unconverted, before the current token's arithmetic.
//
// Variants measured on the decode batch (256 x 16 states, 1-8 tokens) and
// not kept: 8 lanes per row with 2 rows per lane (fewer DPP steps, but more
// registers: slower); a lazily applied decay (state held as alpha * Sh, one
// FMA per element and token: no faster, and a branch per row); the token
// inputs staged once per workgroup through LDS (a barrier per token costs
// more than the repeated loads it saves).

// Four input elements as loaded (bf16 bits or fp32), widened at use.
template <typename TIn>
struct Raw4;
template <>
struct Raw4<uint16_t> {
    u32x2 d;
    __device__ __forceinline__ void load(const uint16_t* p) { d = *reinterpret_cast<const u32x2*>(p); }
    __device__ __forceinline__ void widen(float out[4]) const {
        out[0] = __uint_as_float(d[0] << 16);
        out[1] = __uint_as_float(d[0] & 0xffff0000u);
        out[2] = __uint_as_float(d[1] << 16);
        out[3] = __uint_as_float(d[1] & 0xffff0000u);
    }
};
template <>
struct Raw4<float> {
    f32x4 d;
    __device__ __forceinline__ void load(const float* p) { d = *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ void widen(float out[4]) const {
        out[0] = d[0];
        out[1] = d[1];
        out[2] = d[2];
        out[3] = d[3];
    }
};

template <typename TIn, bool kOut, bool kDiag>
__global__ __launch_bounds__(256) void decode_tokens_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, int32_t tokens, int32_t heads,
    const float* S_in, float* S_out, const int32_t* __restrict__ accept, float* __restrict__ o) {
    const int64_t bh = blockIdx.x >> 1;
    const int half = blockIdx.x & 1;
    const int64_t seq = bh / heads;
    const int64_t h = bh - seq * heads;
    const int t = threadIdx.x;
    const int w = wave_id();
    const int g = (t >> 4) & 3;
    const int c = t & 15;
    const int rbase = 64 * half + 16 * w + g;
    int n_acc = tokens;
    if (accept) n_acc = min(max(accept[seq], 0), tokens);
    const int n_run = kOut ? tokens : n_acc;
    const float* Si = S_in + bh * (kD * kD);
    f32x4 s[4][2];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = rbase + 4 * p;
        s[p][0] = *reinterpret_cast<const f32x4*>(Si + row * kD + 4 * c);
        s[p][1] = *reinterpret_cast<const f32x4*>(Si + row * kD + 64 + 4 * c);
    }
    float* So = S_out ? S_out + bh * (kD * kD) : nullptr;
    auto store_state = [&]() {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = rbase + 4 * p;
            *reinterpret_cast<f32x4*>(So + row * kD + 4 * c) = s[p][0];
            *reinterpret_cast<f32x4*>(So + row * kD + 64 + 4 * c) = s[p][1];
        }
    };
    if (So && n_acc == 0) store_state();
    if (n_run == 0) return;
    struct Tok {
        Raw4<TIn> k[2], q[kOut ? 2 : 1];
        float vr[4], av, bv;
        f32x4 al[kDiag ? 2 : 1];   // per-channel decay of this lane's 8 columns
    };
    auto load_tok = [&](int tok, Tok& x) {
        const int64_t r = (seq * tokens + tok) * heads + h;
        x.k[0].load(k + r * kD + 4 * c);
        x.k[1].load(k + r * kD + 64 + 4 * c);
        if (kOut) {
            x.q[0].load(q + r * kD + 4 * c);
            x.q[1].load(q + r * kD + 64 + 4 * c);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) x.vr[p] = load1<TIn>(v + r * kD + rbase + 4 * p);
        if constexpr (kDiag) {
            x.al[0] = *reinterpret_cast<const f32x4*>(a + r * kD + 4 * c);
            x.al[1] = *reinterpret_cast<const f32x4*>(a + r * kD + 64 + 4 * c);
            x.av = 1.f;
        } else {
            x.av = a[r];
        }
        x.bv = b[r];
    };
    auto step = [&](int tok, const Tok& x) {
        float kx[8], qx[8];
        x.k[0].widen(kx);
        x.k[1].widen(kx + 4);
        if (kOut) {
            x.q[0].widen(qx);
            x.q[1].widen(qx + 4);
        }
        // the decayed state's products: per-channel decay folds into k and q
        // (S diag(alpha) k = S (alpha . k)); the scalar one scales the sums
        float ak[8], aq[8], dj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            dj[j] = kDiag ? x.al[j >> 2][j & 3] : x.av;
            ak[j] = kDiag ? dj[j] * kx[j] : kx[j];
            aq[j] = kDiag && kOut ? dj[j] * qx[j] : qx[j];
        }
        float kap = 0.f;
        if (kOut) {
            float k0 = 0.f, k1 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                k0 = fmaf(kx[j], qx[j], k0);
                k1 = fmaf(kx[4 + j], qx[4 + j], k1);
            }
            kap = dpp_sum16(k0 + k1);
        }
        float o_mine = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float sk0 = 0.f, sk1 = 0.f, sq0 = 0.f, sq1 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sk0 = fmaf(s[p][0][j], ak[j], sk0);
                sk1 = fmaf(s[p][1][j], ak[4 + j], sk1);
                if (kOut) {
                    sq0 = fmaf(s[p][0][j], aq[j], sq0);
                    sq1 = fmaf(s[p][1][j], aq[4 + j], sq1);
                }
            }
            const float sk = dpp_sum16(sk0 + sk1);
            const float e = x.vr[p] - (kDiag ? sk : x.av * sk);
            const float be = x.bv * e;
            if (kOut) {
                const float sq = dpp_sum16(sq0 + sq1);
                const float orow = (kDiag ? sq : x.av * sq) + be * kap;
                if (c == p) o_mine = orow;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[p][0][j] = fmaf(dj[j], s[p][0][j], be * kx[j]);
                s[p][1][j] = fmaf(dj[4 + j], s[p][1][j], be * kx[4 + j]);
            }
        }
        if (kOut && c < 4) o[((seq * tokens + tok) * heads + h) * kD + rbase + 4 * c] = o_mine;
        if (So && tok + 1 == n_acc) store_state();
    };
    // two input buffers used in turn (no copies between tokens); the last
    // load of a run re-reads its own token (in bounds, unused)
    Tok xa, xb;
    load_tok(0, xa);
    for (int tok = 0;;) {
        load_tok(min(tok + 1, n_run - 1), xb);
        step(tok, xa);
        if (++tok == n_run) break;
        load_tok(min(tok + 1, n_run - 1), xa);
        step(tok, xb);
        if (++tok == n_run) break;
    }
}

// One decode step with a per-key-channel decay alpha [batch, H, 128]: the
// same layout and single pass as decode_step_kernel, with column j of the
// state scaled by alpha_j: for row i,
//     (S'k)_i = sum_j S_ij alpha_j k_j,   (S'q)_i = sum_j S_ij alpha_j q_j
//     e_i = v_i - (S'k)_i,   S_ij <- alpha_j S_ij + b e_i k_j
//     o_i = (S'q)_i + b e_i (k . q)
template <typename TIn>
__global__ __launch_bounds__(256) void decode_diag_kernel(const TIn* __restrict__ q,
                                                          const TIn* __restrict__ k,
                                                          const TIn* __restrict__ v,
                                                          const float* __restrict__ alpha,
                                                          const float* __restrict__ b,
                                                          float* __restrict__ S,
                                                          float* __restrict__ o) {
    const int64_t bh = blockIdx.x >> 1;
    const int half = blockIdx.x & 1;
    const int t = threadIdx.x;
    const int w = wave_id();
    const int g = (t >> 4) & 3;
    const int c = t & 15;
    float* __restrict__ Sb = S + bh * (kD * kD);
    f32x4 s[4][2];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = 64 * half + 16 * w + 4 * p + g;
        s[p][0] = *reinterpret_cast<const f32x4*>(Sb + row * kD + 4 * c);
        s[p][1] = *reinterpret_cast<const f32x4*>(Sb + row * kD + 64 + 4 * c);
    }
    float kx[8], qx[8];
    load4<TIn>(k + bh * kD + 4 * c, kx);
    load4<TIn>(k + bh * kD + 64 + 4 * c, kx + 4);
    load4<TIn>(q + bh * kD + 4 * c, qx);
    load4<TIn>(q + bh * kD + 64 + 4 * c, qx + 4);
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(alpha + bh * kD + 4 * c);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(alpha + bh * kD + 64 + 4 * c);
    const float ax[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const float bv = b[bh];
    float vr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) vr[p] = load1<TIn>(v + bh * kD + 64 * half + 16 * w + 4 * p + g);
    float ak[8], aq[8], kap = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ak[j] = ax[j] * kx[j];
        aq[j] = ax[j] * qx[j];
        kap += kx[j] * qx[j];
    }
    kap = dpp_sum16(kap);
    float o_mine = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sk = fmaf(s[p][0][j], ak[j], fmaf(s[p][1][j], ak[4 + j], sk));
            sq = fmaf(s[p][0][j], aq[j], fmaf(s[p][1][j], aq[4 + j], sq));
        }
        sk = dpp_sum16(sk);
        sq = dpp_sum16(sq);
        const float be = bv * (vr[p] - sk);
        const float orow = sq + be * kap;
        if (c == p) o_mine = orow;
        f32x4 n0, n1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            n0[j] = fmaf(ax[j], s[p][0][j], be * kx[j]);
            n1[j] = fmaf(ax[4 + j], s[p][1][j], be * kx[4 + j]);
        }
        const int row = 64 * half + 16 * w + 4 * p + g;
        *reinterpret_cast<f32x4*>(Sb + row * kD + 4 * c) = n0;
        *reinterpret_cast<f32x4*>(Sb + row * kD + 64 + 4 * c) = n1;
    }
    if (c < 4) o[bh * kD + 64 * half + 16 * w + 4 * c + g] = o_mine;
}

// ---------------------------------------------------------------------------
// One decode step with the block's prologue in front, one 512-thread
// workgroup per (batch, head).  Lanes 0..383 load the short convolution's
// operands for one channel each of q, k, v (lane 128x + ch: tensor x,
// channel ch) -- its weights, its history slots and the raw token -- and then
// every lane sends out its state loads (the decode step's layout: wave w
// holds rows 16w + 4p + g).  The convolution lanes run the taps in the
// prologue's order and the activation, leave the fp32 result in LDS and move
// their channel's history on by one token.  After a barrier lane groups 0
// and 1 of wave 0 take the L2 scales of q and k in the prologue kernel's
// lane layout (a lane 8 channels, 4c.. and 64+4c..) and leave q and k in
// bf16 in LDS; after a second barrier every wave reads them, rounds its rows
// of the gated v to bf16 and runs the decode step's single pass over its
// rows (decode_rows).  The result is that of rda_prologue (one-token layout)
// followed by rda_decode_step, bit for bit (the per-channel arithmetic is
// the shared code of rda_prologue_math.h), and q, k, v, a, b never reach
// memory.  A lane reads its channel's history slots before it writes the
// shifted ones, and no other lane touches them, so the history may be
// updated in place.
//
// That the history may be updated in place is what fixes one workgroup per
// (batch, head): both halves of the state need every q and k channel, hence
// the whole q / k history.  The gates go to scalar registers, which keeps
// the kernel at 64 registers, 8 waves per SIMD: 4 workgroups, as many state
// bytes in flight per CU as the plain decode step.  On 256 x 16 states this
// step takes 87 us against 80.5 us for the plain decode step, which moves
// 3.5 % fewer bytes (no history read and written); 6 waves per SIMD measure
// the same.  Measured and not kept: lane groups 0-2 of wave 0 running the
// prologue 8 channels per lane and loading their state only after it (93
// us, as long as rda_prologue followed by rda_decode_step), every lane group
// running the whole prologue for itself (173 us), a ninth wave for the
// prologue (94 us), persistent workgroups with the prologue one item ahead
// in a second LDS buffer (100 us), and the gates in vector registers, which
// spills a state load at 8 waves per SIMD (101 us).
template <int K, int kAct>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(8)))
void decode_prologue_kernel(const DecodePrologueArgs P) {
    __shared__ __attribute__((aligned(16))) float u[4][kD];        // q, k, v; row 3 unused
    __shared__ __attribute__((aligned(16))) uint16_t qk[2][kD];    // q, k in bf16
    const int64_t bh = blockIdx.x;
    const int64_t n = bh / P.H;
    const int h = int(bh - n * P.H);
    const int t = threadIdx.x;
    const int w = wave_id();      // 0..7
    const int g = (t >> 4) & 3;
    const int c = t & 15;
    const int rbase = 16 * w + g;
    float* __restrict__ Sb = P.S + bh * (kD * kD);

    // the convolution's loads first (waves 6, 7 load v's channels again and
    // keep nothing: all of this stays straight-line code), so that it waits
    // for them alone (loads return in order)
    const bool conv = t < 3 * kD;
    const int xr = __builtin_amdgcn_readfirstlane(t >> 7);   // 3 in waves 6, 7
    const int x = xr < 3 ? xr : 2;
    const uint32_t ch = uint32_t(t) & (kD - 1);
    const uint32_t hd = uint32_t(P.H) * kD;
    // history slots of tensor x for this (sequence, head): [N][3][K-1][H][128]
    const size_t hslots = (size_t(n) * 3 + x) * (K - 1) * hd + size_t(h) * kD;
    const float* wb = P.w + (size_t(x) * P.H + h) * kD * K;
    const uint16_t* xb = (x == 0 ? P.x[0] : x == 1 ? P.x[1] : P.x[2]) + bh * kD;
    float wt[K];
    uint32_t win[K];   // taps 0 .. K-2 from the history, tap K-1 the current token
#pragma unroll
    for (int i = 0; i < K; ++i) wt[i] = wb[ch * K + i];
    win[K - 1] = xb[ch];
    // without a history the taps read the current token and are masked to
    // zero further down (no branch)
    const uint32_t keep = P.hin ? 0xffffu : 0u;
    {
        const uint16_t* hb = P.hin ? P.hin + hslots : xb;
        const uint32_t hstep = P.hin ? hd : 0u;
#pragma unroll
        for (int i = 0; i < K - 1; ++i) win[i] = hb[ch + uint32_t(i) * hstep];
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s[4][2];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = rbase + 4 * p;
        s[p][0] = *reinterpret_cast<const f32x4*>(Sb + row * kD + 4 * c);
        s[p][1] = *reinterpret_cast<const f32x4*>(Sb + row * kD + 64 + 4 * c);
    }
    float acc[1] = {0.f};
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const float xv[1] = {__uint_as_float((i < K - 1 ? win[i] & keep : win[i]) << 16)};
        const float wv[1] = {wt[i]};
        conv_tap(acc, wv, xv);
    }
    conv_activation<kAct>(acc);
    u[xr][ch] = acc[0];
    if (conv && P.hout) {
        // the history moves on by one token: slot m takes the old slot m + 1,
        // the newest slot the current raw token (read above by this lane)
        uint16_t* ho = P.hout + hslots;
#pragma unroll
        for (int m = 0; m < K - 1; ++m)
            ho[ch + uint32_t(m) * hd] = uint16_t(m + 1 < K - 1 ? win[m + 1] & keep : win[m + 1]);
    }
    const float br = P.beta[bh];
    // the gates are the same in every lane: kept in scalar registers
    const float av = uniform_f32(floored_decay(P.glog[bh], P.floor_log));
    const float bv = uniform_f32(erase_gate(br));
    const float vg = uniform_f32(write_gate(br, P.delta ? P.delta[bh] : 0.f));
    __syncthreads();

    // q and k as rda_prologue leaves them: times their L2 scale, rounded to bf16
    const int ch0 = 4 * c, ch1 = 64 + 4 * c;
    if (w == 0 && g < 2) {
        float a8[8];
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(&u[g][ch0]);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(&u[g][ch1]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a8[e] = x0[e];
            a8[4 + e] = x1[e];
        }
        const float sc = l2_scale(a8, P.l2eps);
        *reinterpret_cast<u32x2*>(&qk[g][ch0]) =
            u32x2{pack_bf16(a8[0] * sc, a8[1] * sc), pack_bf16(a8[2] * sc, a8[3] * sc)};
        *reinterpret_cast<u32x2*>(&qk[g][ch1]) =
            u32x2{pack_bf16(a8[4] * sc, a8[5] * sc), pack_bf16(a8[6] * sc, a8[7] * sc)};
    }
    __syncthreads();

    // every wave: q and k from LDS; its rows of v times the write gate, in bf16
    float kx[8], qx[8], vr[4];
    {
        const u32x2 kr[2] = {*reinterpret_cast<const u32x2*>(&qk[1][ch0]),
                             *reinterpret_cast<const u32x2*>(&qk[1][ch1])};
        const u32x2 qr[2] = {*reinterpret_cast<const u32x2*>(&qk[0][ch0]),
                             *reinterpret_cast<const u32x2*>(&qk[0][ch1])};
        widen8(kr, kx);
        widen8(qr, qx);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            vr[p] = __uint_as_float(pack_bf16(u[2][rbase + 4 * p] * vg, 0.f) << 16);
    }
    const float o_mine = decode_rows(s, kx, qx, av, bv, vr, c, Sb, rbase);
    if (c < 4) P.o[bh * kD + rbase + 4 * c] = o_mine;
}

hipError_t launch_decode_prologue(const DecodePrologueArgs& P, int32_t batch, int32_t K,
                                  int32_t act, hipStream_t stream) {
    const unsigned grid = unsigned(int64_t(batch) * P.H);
    if (grid == 0) return hipSuccess;
#define RDA_DP_LAUNCH(KW)                                                                         \
    if (act == RDA_CONV_ACT_SILU)                                                                 \
        hipLaunchKernelGGL((decode_prologue_kernel<KW, RDA_CONV_ACT_SILU>), dim3(grid), dim3(512), \
                           0, stream, P);                                                         \
    else                                                                                          \
        hipLaunchKernelGGL((decode_prologue_kernel<KW, RDA_CONV_ACT_NONE>), dim3(grid), dim3(512), \
                           0, stream, P);
    switch (K) {
        case 1: RDA_DP_LAUNCH(1) break;
        case 2: RDA_DP_LAUNCH(2) break;
        case 3: RDA_DP_LAUNCH(3) break;
        default: RDA_DP_LAUNCH(4) break;
    }
#undef RDA_DP_LAUNCH
    return hipGetLastError();
}

hipError_t launch_decode_diag(const void* q, const void* k, const void* v, rda_dtype dt,
                              const float* alpha, const float* b, int32_t batch, int32_t heads,
                              float* S, float* o, hipStream_t stream) {
    const unsigned grid = unsigned(2 * int64_t(batch) * heads);
    if (grid == 0) return hipSuccess;
    if (dt == RDA_BF16)
        hipLaunchKernelGGL(decode_diag_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), alpha, b, S, o);
    else
        hipLaunchKernelGGL(decode_diag_kernel<float>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), alpha, b, S, o);
    return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, rda_dtype dt,
                         const float* a, const float* b, int32_t batch, int32_t heads,
                         float* S, float* o, hipStream_t stream) {
    const unsigned grid = unsigned(2 * int64_t(batch) * heads);
    if (grid == 0) return hipSuccess;
    if (dt == RDA_BF16) {
        hipLaunchKernelGGL(decode_step_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), a, b, S, o);
    } else {
        hipLaunchKernelGGL(decode_step_kernel<float>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), a, b, S, o);
    }
    return hipGetLastError();
}

template <typename TIn, bool kDiag>
void launch_tokens_t(const void* q, const void* k, const void* v, const float* a,
                     const float* b, int32_t tokens, int32_t heads, const float* S_in,
                     float* S_out, const int32_t* accept, float* o, unsigned grid,
                     hipStream_t stream) {
    const TIn* qt = static_cast<const TIn*>(q);
    const TIn* kt = static_cast<const TIn*>(k);
    const TIn* vt = static_cast<const TIn*>(v);
    if (o)
        hipLaunchKernelGGL((decode_tokens_kernel<TIn, true, kDiag>), dim3(grid), dim3(256), 0,
                           stream, qt, kt, vt, a, b, tokens, heads, S_in, S_out, accept, o);
    else
        hipLaunchKernelGGL((decode_tokens_kernel<TIn, false, kDiag>), dim3(grid), dim3(256), 0,
                           stream, qt, kt, vt, a, b, tokens, heads, S_in, S_out, accept, o);
}

hipError_t launch_decode_tokens(const void* q, const void* k, const void* v, rda_dtype dt,
                                const float* a, const float* b, int32_t batch, int32_t tokens,
                                int32_t heads, const float* S_in, float* S_out,
                                const int32_t* accept, float* o, bool diag, hipStream_t stream) {
    const unsigned grid = unsigned(2 * int64_t(batch) * heads);
    if (grid == 0) return hipSuccess;
    if (dt == RDA_BF16) {
        if (diag) launch_tokens_t<uint16_t, true>(q, k, v, a, b, tokens, heads, S_in, S_out, accept, o, grid, stream);
        else launch_tokens_t<uint16_t, false>(q, k, v, a, b, tokens, heads, S_in, S_out, accept, o, grid, stream);
    } else {
        if (diag) launch_tokens_t<float, true>(q, k, v, a, b, tokens, heads, S_in, S_out, accept, o, grid, stream);
        else launch_tokens_t<float, false>(q, k, v, a, b, tokens, heads, S_in, S_out, accept, o, grid, stream);
    }
    return hipGetLastError();
}

}  // namespace rda
