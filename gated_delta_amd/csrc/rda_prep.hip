// rda_prep.hip -- the prep kernel of the chunked RDA prefill for bf16 inputs
// on gfx950: one 4-wave workgroup per (chunk, head) runs prep_item
// (rda_prep.h); 38 KiB of LDS, so four workgroups share a CU and hide each
// other's latency.
#include "rda_prep.h"

namespace rda {

namespace {

__global__ __launch_bounds__(256) void prep_bf16_kernel(PrepItemArgs A,
                                                        const int32_t* __restrict__ rec,
                                                        const int32_t* __restrict__ num_chunks,
                                                        int32_t single_T, int32_t chunk_begin,
                                                        int32_t nch_total,
                                                        int32_t* __restrict__ rec_out,
                                                        int32_t* __restrict__ seq_off_out,
                                                        int32_t* __restrict__ num_out) {
    __shared__ __attribute__((aligned(16))) PrepLds S;
    const int H = A.H;
    const int chunk = chunk_begin + int(blockIdx.x) / H;
    const int h = int(blockIdx.x) - (chunk - chunk_begin) * H;
    const int tid = threadIdx.x;
    int t0, len;
    if (single_T >= 0) {
        // one sequence of single_T tokens and no offsets: every chunk record
        // is plain arithmetic, and the head-0 workgroups also write the chunk
        // table the walk reads, so that no table kernel runs for this case
        t0 = kC * chunk;
        len = single_T - t0 < kC ? single_T - t0 : kC;
        if (h == 0) prep_table_entry(chunk, t0, len, nch_total, tid, rec_out, seq_off_out, num_out);
    } else {
        if (chunk >= num_chunks[0]) return;
        t0 = rec[4 * chunk + 1];
        len = rec[4 * chunk + 2];
    }
    prep_item(A, chunk, h, t0, len, true, S, tid, wave_id());
}

}  // namespace

hipError_t launch_prep_bf16(const uint16_t* q, const uint16_t* k, const float* a, const float* b,
                            int32_t heads, int32_t max_chunks, const int32_t* rec,
                            const int32_t* num_chunks, unsigned char* factors, int32_t single_T,
                            int32_t* rec_out, int32_t* seq_off_out, int32_t* num_out,
                            hipStream_t stream, int32_t chunk_begin, int32_t chunk_count) {
    int32_t nch_total = max_chunks;
    if (single_T >= 0) {
        nch_total = (single_T + kC - 1) / kC;
        if (chunk_count < 0) chunk_count = nch_total - chunk_begin;
    } else {
        chunk_begin = 0;
        chunk_count = max_chunks;
    }
    const unsigned grid = unsigned(int64_t(chunk_count) * heads);
    if (grid == 0) return hipSuccess;
    const PrepItemArgs A{q, k, a, b, heads, factors};
    hipLaunchKernelGGL(prep_bf16_kernel, dim3(grid), dim3(256), 0, stream, A, rec, num_chunks,
                       single_T, chunk_begin, nch_total, rec_out, seq_off_out, num_out);
    return hipGetLastError();
}

}  // namespace rda
