// rda_prologue.hip -- the steps of the RDA block between its projections and
// the recurrence, in one pass: the causal short convolution of q, k and v
// over a few tokens (with the raw history of earlier calls), an optional SiLU,
// the L2 normalisation of q and k, the write gate on v, b = sigmoid(beta_raw)
// and the floored decay a = exp(max(g_log, floor)).
//
// The Raon-1 nano teardown keeps a short convolution window per layer beside
// the recurrent state (section "The cache is small if the runtime keeps it
// small") and describes the decoupled gates -- erase with beta =
// sigmoid(beta_raw), a separate write gate sigmoid(beta_raw + delta) /
// sigmoid(beta_raw) scaling the value -- and the decay bounded below by -5 in
// log space (section "The other 1.5B: a hybrid built to forget"); the Raon-1
// mini vLLM article applies the write gate after the convolution, so the
// history holds raw tokens, and keeps that history in bf16.
//
// Mapping.  A workgroup takes one tensor (q, k or v), 16 heads and TT
// consecutive tokens; each of its 16-lane groups takes one head, a lane 8
// channels (4c..4c+3 and 64+4c..64+4c+3), so at every token position the
// workgroup reads the 16 heads' contiguous 4 KiB.  A lane loads its conv
// weights once and the raw window of its tokens once (TT tokens plus the
// K-1 before them), so the only HBM traffic is the raw tokens in, the bf16
// results out and the history where a sequence starts; the rows a window
// shares with the neighbouring workgroup come from L2.  TT is 8 when that
// still gives 512 workgroups, else 1 (a decode batch).  Where a
// sequence starts inside a token's window the history of that sequence
// replaces the raw tokens before it; a block whose tokens and windows all
// lie inside one sequence, away from the last K-1 tokens of a sequence whose
// history is kept, takes a plain path without those per-token lookups and
// branches, and its per-token gates are computed once per token by one lane
// each (16384 x 16: 83 us against 103).  The q and k norms are 16-lane DPP
// reductions.  The arithmetic (about 160 VALU instructions per token and
// lane, a third of them the SiLU's exp and reciprocal) is of the same order
// as the memory time, and the two overlap only in part.  Measured and not
// kept: one head per workgroup, reading 256-byte slices of each token's row
// (1.3x slower); each raw position widened once into a rolling or a full
// fp32 window (more registers: 1.1x slower).
#include <cmath>

#include "rda_device.h"
#include "rda_internal.h"
#include "rda_prologue_math.h"

namespace rda {
namespace {

// Sequence of token t: index n, first token s, end e (all clamped, so
// malformed offsets stay in bounds).
struct Seq {
    int32_t n, s, e;
};

__device__ __forceinline__ Seq seq_of(const PrologueArgs& P, int32_t t, int32_t n_hint) {
    Seq q;
    if (!P.cu) {
        q.n = t / P.L;
        q.s = q.n * P.L;
        q.e = q.s + P.L;
        return q;
    }
    int32_t n = n_hint;
    while (n + 1 < P.N && P.cu[n + 1] <= t) ++n;
    q.n = n;
    q.s = min(max(P.cu[n], 0), P.T);
    q.e = min(max(P.cu[n + 1], q.s), P.T);
    return q;
}

// first sequence whose end is past t (binary search over the offsets)
__device__ __forceinline__ int32_t find_seq(const PrologueArgs& P, int32_t t) {
    if (!P.cu) return t / P.L;
    int32_t lo = 0, hi = P.N - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (P.cu[mid + 1] <= t) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

template <int K, int kAct, int kTT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void prologue_kernel(const PrologueArgs P) {
    const int x = blockIdx.z;        // 0 = q, 1 = k, 2 = v
    const int lane = threadIdx.x;
    const int grp = lane >> 4;
    const int c = lane & 15;
    const int h = int(blockIdx.y) * 16 + grp;
    // XCD-aware order: workgroups are dealt to the 8 XCDs in turn, so within
    // each run of 8 x 16 token blocks XCD id % 8 takes 16 consecutive blocks,
    // and the block that re-reads a window's first K-1 positions is mostly
    // served by the same L2, while the 8 XCDs still sweep neighbouring
    // memory together (dealing each XCD one contiguous eighth of all blocks
    // removed the re-reads too, but was 10 % slower); blocks past the last
    // full run keep their order
    constexpr int32_t kS = 16;
    const int32_t nb = int32_t(gridDim.x), bid = int32_t(blockIdx.x), xcd = bid & 7;
    const int32_t full = nb / (8 * kS) * (8 * kS);
    int32_t tb = bid;
    if (bid < full) {
        const int32_t k = bid >> 3;
        tb = (k / kS) * (8 * kS) + xcd * kS + (k % kS);
    }
    const int32_t t_first = tb * kTT;
    if (h >= P.H) return;            // a whole 16-lane group: no DPP partner left behind
    const size_t hd = size_t(P.H) * kD;
    const int ch0 = 4 * c, ch1 = 64 + 4 * c;

    // conv weights of this lane's channels, [3][H][128][K]
    float wt[K][8];
    const float* wb = P.w + (size_t(x) * P.H + h) * kD * K;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < K; ++i) {
            wt[i][j] = wb[(ch0 + j) * K + i];
            wt[i][4 + j] = wb[(ch1 + j) * K + i];
        }

    // raw window: positions t_first - (K-1) .. t_first + kTT - 1
    constexpr int R = kTT + K - 1;
    u32x2 raw[R][2];
    const uint16_t* xb = P.x[x] + size_t(h) * kD;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int32_t p = t_first - (K - 1) + r;
        if (p >= 0 && p < P.T) {
            raw[r][0] = *reinterpret_cast<const u32x2*>(xb + size_t(p) * hd + ch0);
            raw[r][1] = *reinterpret_cast<const u32x2*>(xb + size_t(p) * hd + ch1);
        } else {
            raw[r][0] = u32x2{0u, 0u};
            raw[r][1] = u32x2{0u, 0u};
        }
    }

    int32_t n_hint = find_seq(P, t_first);
    {
        // The common block: its tokens and their windows inside one
        // sequence, and (with a history out) none of them among the
        // sequence's last K-1 tokens, whose raw values become the history.
        // Then every tap reads the raw window and nothing else is written:
        // the same arithmetic without the per-token lookups and branches.
        const Seq s0 = seq_of(P, t_first, n_hint);
        const int32_t t_last = min(t_first + kTT, P.T) - 1;
        const bool plain = t_first - (K - 1) >= s0.s && t_last < s0.e &&
                           (!P.hout || K == 1 || t_last < s0.e - (K - 1));
        if (plain) {
            // the per-token gates, lane c of each group taking token c of
            // the block (the same arithmetic as the token loop's, once per
            // token instead of once per token and lane): a and b by the q
            // workgroups, the write gate by the v workgroups, handed to the
            // group's lanes per token
            const bool gl = c < kTT && t_first + c <= t_last;
            const int32_t tg = gl ? t_first + c : t_last;   // a token of the block either way
            const size_t thg = size_t(tg) * P.H + h;
            float vgate = 0.f;
            if (x == 0 && gl) {
                P.b[thg] = erase_gate(P.beta[thg]);
                P.a[thg] = floored_decay(P.glog[thg], P.floor_log);
            }
            if (x == 2) vgate = write_gate(P.beta[thg], P.delta ? P.delta[thg] : 0.f);
#pragma unroll
            for (int j = 0; j < kTT; ++j) {
                const int32_t t = t_first + j;
                if (t > t_last) break;
                float acc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    float xv[8];
                    widen8(raw[j + i], xv);
                    conv_tap(acc, wt[i], xv);
                }
                conv_activation<kAct>(acc);
                const size_t th = size_t(t) * P.H + h;
                const float scale = x < 2 ? l2_scale(acc, P.l2eps)
                                          : __shfl(vgate, (lane & ~15) + j, 64);
                uint16_t* ob = P.out[x] + th * kD;
                *reinterpret_cast<u32x2*>(ob + ch0) = u32x2{pack_bf16(acc[0] * scale, acc[1] * scale),
                                                            pack_bf16(acc[2] * scale, acc[3] * scale)};
                *reinterpret_cast<u32x2*>(ob + ch1) = u32x2{pack_bf16(acc[4] * scale, acc[5] * scale),
                                                            pack_bf16(acc[6] * scale, acc[7] * scale)};
            }
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < kTT; ++j) {
        const int32_t t = t_first + j;
        if (t >= P.T) break;

        const Seq sq = seq_of(P, t, n_hint);
        n_hint = sq.n;
        // history slots of this sequence and tensor: [N][3][K-1][H][128]
        const size_t hslot0 = (size_t(sq.n) * 3 + x) * (K - 1);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int i = 0; i < K; ++i) {
            const int32_t p = t - (K - 1) + i;
            float xv[8];
            if (p >= sq.s) {
                widen8(raw[j + i], xv);
            } else if (P.hin) {
                const int m = min(max(p - sq.s + (K - 1), 0), K - 2);
                const uint16_t* hp = P.hin + (hslot0 + m) * hd + size_t(h) * kD;
                u32x2 hr[2];
                hr[0] = *reinterpret_cast<const u32x2*>(hp + ch0);
                hr[1] = *reinterpret_cast<const u32x2*>(hp + ch1);
                widen8(hr, xv);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) xv[e] = 0.f;
            }
            conv_tap(acc, wt[i], xv);
        }
        conv_activation<kAct>(acc);
        const size_t th = size_t(t) * P.H + h;
        float scale;
        if (x < 2) {
            scale = l2_scale(acc, P.l2eps);
        } else {
            const float br = P.beta[th];
            const float dl = P.delta ? P.delta[th] : 0.f;
            scale = write_gate(br, dl);
        }
        uint16_t* ob = P.out[x] + th * kD;
        *reinterpret_cast<u32x2*>(ob + ch0) =
            u32x2{pack_bf16(acc[0] * scale, acc[1] * scale), pack_bf16(acc[2] * scale, acc[3] * scale)};
        *reinterpret_cast<u32x2*>(ob + ch1) =
            u32x2{pack_bf16(acc[4] * scale, acc[5] * scale), pack_bf16(acc[6] * scale, acc[7] * scale)};
        if (x == 0 && c == 0) {
            P.b[th] = erase_gate(P.beta[th]);
            P.a[th] = floored_decay(P.glog[th], P.floor_log);
        }
        if (P.hout && K > 1 && t < sq.e) {
            // a sequence shorter than K-1 keeps the newest slots of its old
            // history, moved down by its length; copied in ascending slot
            // order before the new slot is written, so a history updated in
            // place (one token per sequence) reads every old slot first
            const int32_t len = sq.e - sq.s;
            if (t == sq.s && len < K - 1) {
                for (int m = 0; m < K - 1 - len; ++m) {
                    u32x2 v0 = u32x2{0u, 0u}, v1 = u32x2{0u, 0u};
                    if (P.hin) {
                        const uint16_t* src = P.hin + (hslot0 + m + len) * hd + size_t(h) * kD;
                        v0 = *reinterpret_cast<const u32x2*>(src + ch0);
                        v1 = *reinterpret_cast<const u32x2*>(src + ch1);
                    }
                    uint16_t* dst = P.hout + (hslot0 + m) * hd + size_t(h) * kD;
                    *reinterpret_cast<u32x2*>(dst + ch0) = v0;
                    *reinterpret_cast<u32x2*>(dst + ch1) = v1;
                }
            }
            // the sequence's last K-1 raw tokens become its history
            if (t >= sq.e - (K - 1)) {
                const int m = t - sq.e + (K - 1);
                uint16_t* hp = P.hout + (hslot0 + m) * hd + size_t(h) * kD;
                *reinterpret_cast<u32x2*>(hp + ch0) = raw[j + K - 1][0];
                *reinterpret_cast<u32x2*>(hp + ch1) = raw[j + K - 1][1];
            }
        }
    }
}

// Sequences without tokens keep their history (zeros without a history in):
// one thread per 8 bytes of the history out.
__global__ __launch_bounds__(256) void history_keep_kernel(const PrologueArgs P, int32_t slots) {
    const size_t per_seq = size_t(3) * slots * P.H * kD / 4;   // 8-byte units
    const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= per_seq * P.N) return;
    const int32_t n = int32_t(i / per_seq);
    int32_t len;
    if (P.cu) {
        const int32_t s = min(max(P.cu[n], 0), P.T);
        len = min(max(P.cu[n + 1], s), P.T) - s;
    } else {
        len = P.L;
    }
    if (len != 0) return;
    u32x2 v = u32x2{0u, 0u};
    if (P.hin) v = reinterpret_cast<const u32x2*>(P.hin)[i];
    reinterpret_cast<u32x2*>(P.hout)[i] = v;
}

template <int K, int kTT>
void launch_kt(const PrologueArgs& P, int32_t act, hipStream_t stream) {
    const dim3 grid(unsigned((int64_t(P.T) + kTT - 1) / kTT), unsigned((P.H + 15) / 16), 3);
    if (act == RDA_CONV_ACT_SILU)
        hipLaunchKernelGGL((prologue_kernel<K, RDA_CONV_ACT_SILU, kTT>), grid, dim3(256), 0,
                           stream, P);
    else
        hipLaunchKernelGGL((prologue_kernel<K, RDA_CONV_ACT_NONE, kTT>), grid, dim3(256), 0,
                           stream, P);
}

template <int K>
void launch_k(const PrologueArgs& P, int32_t act, hipStream_t stream) {
    // 8 tokens per lane group while that leaves at least 512 workgroups (2
    // per CU), else one (a decode batch): measured on 16384 x 16 and 2048 x
    // 16 tokens 8 is best (1, 2 and 4 were 1.3-1.9x slower), on 256 x 16
    // one-token sequences 1 is (8 was 2.5x slower)
    const int64_t per_tt = int64_t(3) * ((P.H + 15) / 16);
    if (per_tt * ((int64_t(P.T) + 7) / 8) >= 512) launch_kt<K, 8>(P, act, stream);
    else launch_kt<K, 1>(P, act, stream);
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& P, int32_t K, int32_t act, hipStream_t stream) {
    if (P.T > 0) {
        switch (K) {
            case 1: launch_k<1>(P, act, stream); break;
            case 2: launch_k<2>(P, act, stream); break;
            case 3: launch_k<3>(P, act, stream); break;
            default: launch_k<4>(P, act, stream); break;
        }
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // empty sequences exist only with offsets, or when there are no tokens
    if (P.hout && K > 1 && (P.cu || P.T == 0)) {
        const size_t units = size_t(P.N) * 3 * (K - 1) * P.H * kD / 4;
        hipLaunchKernelGGL(history_keep_kernel, dim3(unsigned((units + 255) / 256)), dim3(256), 0,
                           stream, P, K - 1);
    }
    return hipGetLastError();
}

}  // namespace rda
