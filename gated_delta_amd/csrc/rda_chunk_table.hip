// rda_chunk_table.hip -- the 64-token chunk table of a packed varlen batch.
//
// From cu_seqlens[N+1] (token offsets of N packed sequences) build
//   seq_off[n]  = sum_{m<n} ceil(len_m / 64)         (first chunk of sequence n)
//   rec[c]      = (n, first token, valid length, chunk index within n)
//   num_chunks  = seq_off[N]
// Integer work only; the result is exact.  Offsets are clamped into
// [0, total_tokens] and chunk indices are capped at max_chunks, so malformed
// offsets can never make this or any later kernel index out of bounds.
// One 1024-thread workgroup: a block-wide scan over tiles of sequences, then
// a strided pass that writes each chunk's record (binary search on seq_off).
#include "rda_internal.h"

namespace rda {

namespace {

__device__ __forceinline__ int32_t clampi(int32_t x, int32_t lo, int32_t hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

__device__ __forceinline__ void seq_range(const int32_t* cu, int32_t n, int32_t T, int32_t& s0,
                                          int32_t& len) {
    if (cu) {
        s0 = clampi(cu[n], 0, T);
        const int32_t s1 = clampi(cu[n + 1], 0, T);
        len = s1 > s0 ? s1 - s0 : 0;
    } else {
        s0 = 0;
        len = T;
    }
}

constexpr int kTableThreads = 1024;

__global__ __launch_bounds__(kTableThreads) void chunk_table_kernel(
    const int32_t* __restrict__ cu, int32_t N, int32_t T, int32_t max_chunks,
    int32_t* __restrict__ rec, int32_t* __restrict__ seq_off, int32_t* __restrict__ num_chunks) {
    __shared__ int64_t scan[kTableThreads];
    __shared__ int64_t carry_s;
    const int tid = threadIdx.x;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int32_t base = 0; base < N; base += kTableThreads) {
        const int32_t n = base + tid;
        int64_t cnt = 0;
        if (n < N) {
            int32_t s0, len;
            seq_range(cu, n, T, s0, len);
            cnt = (int64_t(len) + kC - 1) / kC;
        }
        scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < kTableThreads; off <<= 1) {
            const int64_t add = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        const int64_t carry = carry_s;
        if (n < N) {
            const int64_t excl = carry + scan[tid] - cnt;
            seq_off[n] = int32_t(excl < max_chunks ? excl : max_chunks);
        }
        __syncthreads();
        if (tid == 0) carry_s = carry + scan[kTableThreads - 1];
        __syncthreads();
    }
    const int64_t total = carry_s;
    const int32_t nch = int32_t(total < max_chunks ? total : max_chunks);
    if (tid == 0) {
        seq_off[N] = nch;
        num_chunks[0] = nch;
    }
    __syncthreads();
    for (int32_t c = tid; c < max_chunks; c += kTableThreads) {
        int32_t r0 = -1, r1 = 0, r2 = 0, r3 = 0;
        if (c < nch) {
            // last n in [0, N) with seq_off[n] <= c
            int32_t lo = 0, hi = N;  // invariant: seq_off[lo] <= c < seq_off[hi]
            while (hi - lo > 1) {
                const int32_t mid = (lo + hi) >> 1;
                if (seq_off[mid] <= c) lo = mid;
                else hi = mid;
            }
            int32_t s0, len;
            seq_range(cu, lo, T, s0, len);
            const int32_t j = c - seq_off[lo];
            const int32_t start = s0 + j * kC;
            const int32_t rem = s0 + len - start;
            r0 = lo;
            r1 = start;
            r2 = rem < kC ? rem : kC;
            r3 = j;
        }
        rec[4 * c + 0] = r0;
        rec[4 * c + 1] = r1;
        rec[4 * c + 2] = r2;
        rec[4 * c + 3] = r3;
    }
}

}  // namespace

hipError_t launch_chunk_table(const int32_t* cu, int32_t num_seqs, int32_t total_tokens,
                              int32_t max_chunks, int32_t* rec, int32_t* seq_off,
                              int32_t* num_chunks, hipStream_t stream) {
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kTableThreads), 0, stream, cu, num_seqs,
                       total_tokens, max_chunks, rec, seq_off, num_chunks);
    return hipGetLastError();
}

}  // namespace rda
