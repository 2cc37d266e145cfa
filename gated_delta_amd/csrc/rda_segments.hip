// rda_segments.hip -- the combine step of the segmented state pass.
//
// The walk over one segment is affine in its starting state: per value row,
// s_end = s_start M + e with M the segment's key-space transition and e the
// end state reached from zero.  The first pass walks every segment twice in
// one launch: from zero (E = the e rows) and from the identity with every
// value taken as zero (that walk applies the transition alone, so it ends at
// M).  This kernel chains the segments, S_in[p + 1] = S_in[p] M_p + E_p,
// giving the state each segment starts from (for the pass that writes the
// outputs) and the final state.  Rows of the state never mix, so one
// workgroup owns 16 value rows of one head for every segment and no
// workgroup waits on another.  M_p (64 KiB) is brought into LDS by LDS-DMA
// one step ahead, into the other of two buffers; the products run on fp32
// MFMA (full fp32 arithmetic).
#include "rda_device.h"
#include "rda_internal.h"
#include "rda_lds.h"

namespace rda {

namespace {

// One workgroup owns 16 value rows of one head; wave w computes output
// columns 32w .. 32w + 31 (two 16 x 16 tiles) on fp32 MFMA (16 x 16 x 4).
// The rows of S_in[p] are the A operand, held in registers: lane (g, c)
// keeps S[row c][4 ks + g] for ks = 0 .. 31.  M_p is the B operand, read from
// LDS, where row r keeps its 16-byte granule q at position q ^ 4 (r mod 4):
// the 64 lanes of one B read (rows 4 ks + g, 16 consecutive columns) then
// hit 64 distinct banks.
constexpr int kRows = 16;
constexpr int kSx = kD + 4;   // row stride (floats) of the staged rows: spreads banks

struct CombineLds {
    float M[2][kD * kD];    // M_p, double-buffered, granules swizzled per row
    float Sx[kRows * kSx];  // the new rows, from accumulator to operand layout
};

static_assert(sizeof(CombineLds) <= 160 * 1024, "LDS budget of one workgroup");

__device__ __forceinline__ int mswz(int r) { return 4 * (r & 3); }

// A barrier that orders LDS only: the step's global stores of the new rows
// stay in flight across it (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Half kHalf of M_p into LDS: wave w moves the 1 KiB blocks w + 4 i (rows
// 2 blk, 2 blk + 1) for i in that half, each lane fetching the granule that
// lands at its slot.
template <int kHalf>
__device__ __forceinline__ void dma_matrix(const float* src, float* dst, int w, int l) {
#pragma unroll
    for (int i = 8 * kHalf; i < 8 * kHalf + 8; ++i) {
        const int blk = w + 4 * i;
        const int r = 2 * blk + (l >> 5), pq = l & 31;
        __builtin_amdgcn_global_load_lds(src + r * kD + 4 * (pq ^ mswz(r)),
                                         (lds_void*)(reinterpret_cast<char*>(dst) + 1024 * blk),
                                         16, 0, 0);
    }
}

__device__ __forceinline__ float mat(const float* M, int r, int col) {
    return M[r * kD + 4 * ((col >> 2) ^ mswz(r)) + (col & 3)];
}

__global__ __launch_bounds__(256) void segment_combine_kernel(const float* S0,
                                                              const float* __restrict__ E,
                                                              const float* __restrict__ Mt,
                                                              float* __restrict__ S_in,
                                                              float* S_final, int P, int H) {
    __shared__ __attribute__((aligned(16))) CombineLds L;
    // the 8 row blocks of a head share blockIdx.x % 8, hence one XCD and its
    // L2, which then fetches each M_p once for all of them (the grid holds 8
    // heads per 64 workgroups; those past the last head exit)
    const int h = (blockIdx.x >> 6) * 8 + (blockIdx.x & 7);
    const int rb = (blockIdx.x >> 3) & 7;
    if (h >= H) return;
    const int w = wave_id(), l = threadIdx.x & 63, g = l >> 4, c = l & 15;
    const size_t head = size_t(h) * kD * kD;
    const size_t seg = size_t(H) * kD * kD;
    const size_t rows = head + size_t(rb) * kRows * kD;   // this block's first row
    const int steps = S_final ? P : P - 1;   // the last step only feeds S_final

    if (steps > 0) {
        dma_matrix<0>(Mt + head, L.M[0], w, l);
        dma_matrix<1>(Mt + head, L.M[0], w, l);
    }
    // S_in[0] = S0 (or zero): the operand registers, and (wave w's columns)
    // the copy in S_in
    float aS[kD / 4];
#pragma unroll
    for (int ks = 0; ks < kD / 4; ++ks) aS[ks] = S0 ? S0[rows + size_t(c) * kD + 4 * ks + g] : 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t idx = rows + size_t(4 * g + e) * kD + 32 * w + 16 * u + c;
            S_in[idx] = S0 ? S0[idx] : 0.f;
        }
    // E_p's values at this lane's outputs, loaded one step ahead like M_p
    auto load_e = [&](int p, f32x4 (&ev)[2]) {
        const float* Ep = E + p * seg;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ev[u][e] = Ep[rows + size_t(4 * g + e) * kD + 32 * w + 16 * u + c];
    };
    f32x4 ev_next[2];
    if (steps > 0) load_e(0, ev_next);
    for (int p = 0; p < steps; ++p) {
        // this wave's part of M_p and its E_p values (issued before M_p) have
        // landed once at most the 8 row stores issued after them are in
        // flight; after the barrier, all of M_p has
        wait_vm<8>();
        lds_barrier();
        const f32x4 ev[2] = {ev_next[0], ev_next[1]};
        if (p + 1 < steps) load_e(p + 1, ev_next);
        else load_e(p, ev_next);   // a fixed count of loads keeps the waits exact
        __builtin_amdgcn_sched_barrier(0);   // issue them here, not after the products
        // the next step's matrix, one step ahead, in two halves issued before
        // the two halves of the products (the last step fetches its own again,
        // unread: a fixed count of loads keeps the waits exact)
        const int pn = p + 1 < steps ? p + 1 : p;
        const float* Mnext = Mt + pn * seg + head;
        float* Mbuf = L.M[(p + 1) & 1];
        const float* M = L.M[p & 1];
        f32x4 acc0 = zero4(), acc1 = zero4();
        // half of the B operands read at once, then their products (read
        // one at a time, every product waits out the LDS latency)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (half == 0) dma_matrix<0>(Mnext, Mbuf, w, l);
            else dma_matrix<1>(Mnext, Mbuf, w, l);
            float b0[16], b1[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 4 * (16 * half + i) + g;
                b0[i] = mat(M, r, 32 * w + c);
                b1[i] = mat(M, r, 32 * w + 16 + c);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc0 = mfma_f32(aS[16 * half + i], b0[i], acc0);
                acc1 = mfma_f32(aS[16 * half + i], b1[i], acc1);
            }
        }
        const f32x4 n0 = acc0 + ev[0], n1 = acc1 + ev[1];
        float* dst = p + 1 < P ? S_in + (p + 1) * seg : S_final;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 4 * g + e;
            L.Sx[row * kSx + 32 * w + c] = n0[e];
            L.Sx[row * kSx + 32 * w + 16 + c] = n1[e];
            dst[rows + size_t(row) * kD + 32 * w + c] = n0[e];
            dst[rows + size_t(row) * kD + 32 * w + 16 + c] = n1[e];
        }
        lds_barrier();   // the new rows are staged
#pragma unroll
        for (int ks = 0; ks < kD / 4; ++ks) aS[ks] = L.Sx[c * kSx + 4 * ks + g];
    }
    __builtin_amdgcn_s_waitcnt(0);   // nothing may land in LDS after the workgroup ends
}

}  // namespace

hipError_t launch_segment_combine(const float* S0, const float* E, const float* M, float* S_in,
                                  float* S_final, int32_t P, int32_t heads, hipStream_t stream) {
    const unsigned grid = unsigned(64 * ((heads + 7) / 8));
    if (grid == 0 || P <= 0) return hipSuccess;
    hipLaunchKernelGGL(segment_combine_kernel, dim3(grid), dim3(256), 0, stream, S0, E, M, S_in,
                       S_final, P, heads);
    return hipGetLastError();
}

}  // namespace rda
