// rda_epilogue.hip -- the output norm and gate of the RDA block as a pass
// of its own over the mixer's output rows (the row math is in rda_norm.h),
// from fp32 o or from the 16-bit form a fused prefill's walk leaves, to bf16
// or fp32.  The pass is bound by HBM: per row it reads 512 B of fp32 o (or
// 256 B of the 16-bit form) and 256 B of bf16 gate and writes 256 B of bf16,
// against ~6 flops per channel.  A 256-thread workgroup takes 16 rows, 16
// lanes per row.  Measured on 262144 rows: 2, 4 or 8 rows per lane group, 8
// contiguous channels per lane (16-byte gate loads and output stores) and
// non-temporal hints were all within 1 us of this form or slower.
#include "rda_norm.h"

namespace rda {
namespace {

constexpr int kRowsPerBlock = 16;

// kEnc: the rows come in the 16-bit form of a fused prefill (oe) instead of
// fp32 (o).
template <typename TG, typename TO, int kAct, bool kEnc>
__global__ __launch_bounds__(256) void norm_gate_kernel(const float* o,
                                                        const uint16_t* __restrict__ oe,
                                                        const TG* __restrict__ g,
                                                        const float* __restrict__ w, float eps,
                                                        int64_t rows, TO* out) {
    const int t = threadIdx.x;
    const int64_t r0 = int64_t(blockIdx.x) * 16 + (t >> 4);
    // the tail re-reads the last row, unused
    norm_gate_row<TG, TO, kAct, kEnc>(o, oe, g, w, eps, min(r0, rows - 1), r0 < rows, out,
                                      t & 15);
}

template <typename TG, typename TO, bool kEnc>
void launch_act(const float* o, const uint16_t* oe, const void* g, const float* w, float eps,
                int32_t act, int64_t rows, void* out, unsigned grid, hipStream_t stream) {
    const TG* gt = static_cast<const TG*>(g);
    TO* ot = static_cast<TO*>(out);
    if (act == RDA_GATE_SIGMOID)
        hipLaunchKernelGGL((norm_gate_kernel<TG, TO, RDA_GATE_SIGMOID, kEnc>), dim3(grid),
                           dim3(256), 0, stream, o, oe, gt, w, eps, rows, ot);
    else if (act == RDA_GATE_SILU)
        hipLaunchKernelGGL((norm_gate_kernel<TG, TO, RDA_GATE_SILU, kEnc>), dim3(grid),
                           dim3(256), 0, stream, o, oe, gt, w, eps, rows, ot);
    else
        hipLaunchKernelGGL((norm_gate_kernel<TG, TO, RDA_GATE_NONE, kEnc>), dim3(grid),
                           dim3(256), 0, stream, o, oe, gt, w, eps, rows, ot);
}

template <bool kEnc>
void launch_dtypes(const float* o, const uint16_t* oe, const void* g, rda_dtype g_dtype,
                   const float* w, float eps, int32_t act, int64_t rows, void* out,
                   rda_dtype out_dtype, unsigned grid, hipStream_t stream) {
    const bool g16 = g_dtype == RDA_BF16, o16 = out_dtype == RDA_BF16;
    if (g16 && o16)
        launch_act<uint16_t, uint16_t, kEnc>(o, oe, g, w, eps, act, rows, out, grid, stream);
    else if (g16)
        launch_act<uint16_t, float, kEnc>(o, oe, g, w, eps, act, rows, out, grid, stream);
    else if (o16)
        launch_act<float, uint16_t, kEnc>(o, oe, g, w, eps, act, rows, out, grid, stream);
    else
        launch_act<float, float, kEnc>(o, oe, g, w, eps, act, rows, out, grid, stream);
}

}  // namespace

int64_t norm_gate_blocks(int64_t rows) { return (rows + kRowsPerBlock - 1) / kRowsPerBlock; }

hipError_t launch_norm_gate(const float* o, const void* g, rda_dtype g_dtype, const float* w,
                            float eps, int32_t act, int64_t rows, void* out, rda_dtype out_dtype,
                            hipStream_t stream, const uint16_t* o_enc) {
    const unsigned grid = unsigned(norm_gate_blocks(rows));
    if (grid == 0) return hipSuccess;
    if (o_enc)
        launch_dtypes<true>(nullptr, o_enc, g, g_dtype, w, eps, act, rows, out, out_dtype, grid,
                            stream);
    else
        launch_dtypes<false>(o, nullptr, g, g_dtype, w, eps, act, rows, out, out_dtype, grid,
                             stream);
    return hipGetLastError();
}

}  // namespace rda
