// rda_epilogue.hip -- the output epilogue of the RDA block: per output row of
// one head (128 value channels), an RMS normalisation with epsilon and a
// per-channel weight, times an activation of the output gate, written as
// bf16 (or fp32).  The tiny-random/raon-1-mini model card, section "Printing
// the model", lists the block's o_norm (an RMS norm over the head dimension,
// eps 1e-5) and the g_proj projection that produces the gate; the gate's
// activation is a parameter (sigmoid, SiLU or none).
//
//     y_c = o_c / sqrt(mean_c'(o_c'^2) + eps) * w_c * act(g_c)
//
// The pass is bound by HBM: per row it reads 512 B of fp32 o and 256 B of
// bf16 gate and writes 256 B of bf16, against ~6 flops per channel.
// Mapping: 16 lanes per row, each lane channels 4c..4c+3 and 64+4c..64+4c+3,
// so every load and store instruction of a 16-lane group covers one
// contiguous run (256 B of o, 128 B of gate or output); a 256-thread
// workgroup takes 16 rows.  The row's sum of squares is a 16-lane DPP
// reduction.  Every lane loads its elements before storing and stores only
// those elements, so an fp32 output may overwrite o in place.  Measured on
// 262144 rows: 2, 4 or 8 rows per lane group, 8 contiguous channels per lane
// (16-byte gate loads and output stores) and non-temporal hints were all
// within 1 us of this form or slower.
#include "rda_device.h"
#include "rda_internal.h"

namespace rda {
namespace {

constexpr int kRowsPerGroup = 1;
constexpr int kRowsPerBlock = 16 * kRowsPerGroup;

template <typename TG>
__device__ __forceinline__ void load_gate(const TG* p, float out[4]);
template <>
__device__ __forceinline__ void load_gate<uint16_t>(const uint16_t* p, float out[4]) {
    const u32x2 d = *reinterpret_cast<const u32x2*>(p);
    out[0] = __uint_as_float(d[0] << 16);
    out[1] = __uint_as_float(d[0] & 0xffff0000u);
    out[2] = __uint_as_float(d[1] << 16);
    out[3] = __uint_as_float(d[1] & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load_gate<float>(const float* p, float out[4]) {
    const f32x4 d = *reinterpret_cast<const f32x4*>(p);
    for (int j = 0; j < 4; ++j) out[j] = d[j];
}

template <typename TO>
__device__ __forceinline__ void store_out(TO* p, const float y[4]);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, const float y[4]) {
    // round to nearest even (v_cvt_pk_bf16_f32)
    const f32x2 lo = {y[0], y[1]}, hi = {y[2], y[3]};
    u32x2 d;
    d[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
    d[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
    *reinterpret_cast<u32x2*>(p) = d;
}
template <>
__device__ __forceinline__ void store_out<float>(float* p, const float y[4]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
}

// Four channels 4c' .. 4c' + 3 of the 16-bit form a fused prefill's walk
// leaves (OutSink): lane c of a row's 16 holds places 4 (c % 4) .. +3 of
// slice c / 4 (or 4 + c / 4), so the four lanes of a quad hold one slice, and
// its first two lanes the 8 places that carry the exponent code.
__device__ __forceinline__ void load_enc(const uint16_t* p, int c, f32x4& out) {
    const u32x2 d = *reinterpret_cast<const u32x2*>(p);
    const uint32_t hv[4] = {d[0] & 0xffffu, d[0] >> 16, d[1] & 0xffffu, d[1] >> 16};
    uint32_t bits = 0;
    if ((c & 3) < 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bits |= (hv[e] & 1u) << (4 * (c & 3) + e);
    }
    const int E = int(dpp_or4(bits));
#pragma unroll
    for (int e = 0; e < 4; ++e)
        out[e] = E ? __builtin_amdgcn_ldexpf(float(__builtin_bit_cast(_Float16, uint16_t(hv[e]))),
                                             E - 126)
                   : 0.f;
}

template <int kAct>
__device__ __forceinline__ float gate_act(float x) {
    if (kAct == RDA_GATE_NONE) return 1.f;
    // sigmoid on the hardware's exp2 (one instruction, about 1 ulp)
    const float sig = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
    return kAct == RDA_GATE_SIGMOID ? sig : x * sig;
}

// kEnc: the rows come in the 16-bit form of a fused prefill (oe) instead of
// fp32 (o).
template <typename TG, typename TO, int kAct, bool kEnc>
__global__ __launch_bounds__(256) void norm_gate_kernel(const float* o,
                                                        const uint16_t* __restrict__ oe,
                                                        const TG* __restrict__ g,
                                                        const float* __restrict__ w, float eps,
                                                        int64_t rows, TO* out) {
    const int t = threadIdx.x;
    const int c = t & 15;
    const int64_t r0 = (int64_t(blockIdx.x) * 16 + (t >> 4)) * kRowsPerGroup;
    float wx[8];
    if (w) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + 4 * c);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + 64 + 4 * c);
        for (int j = 0; j < 4; ++j) {
            wx[j] = w0[j];
            wx[4 + j] = w1[j];
        }
    } else {
        for (int j = 0; j < 8; ++j) wx[j] = 1.f;
    }
    // all loads of the group's rows first
    f32x4 ox[kRowsPerGroup][2];
    float gx[kRowsPerGroup][8];
#pragma unroll
    for (int i = 0; i < kRowsPerGroup; ++i) {
        const int64_t r = min(r0 + i, rows - 1);   // the tail re-reads the last row, unused
        if constexpr (kEnc) {
            load_enc(oe + r * kD + 4 * c, c, ox[i][0]);
            load_enc(oe + r * kD + 64 + 4 * c, c, ox[i][1]);
        } else {
            ox[i][0] = *reinterpret_cast<const f32x4*>(o + r * kD + 4 * c);
            ox[i][1] = *reinterpret_cast<const f32x4*>(o + r * kD + 64 + 4 * c);
        }
        if (kAct != RDA_GATE_NONE) {
            load_gate<TG>(g + r * kD + 4 * c, gx[i]);
            load_gate<TG>(g + r * kD + 64 + 4 * c, gx[i] + 4);
        }
    }
#pragma unroll
    for (int i = 0; i < kRowsPerGroup; ++i) {
        float ss = 0.f;
        for (int j = 0; j < 4; ++j) {
            ss = fmaf(ox[i][0][j], ox[i][0][j], ss);
            ss = fmaf(ox[i][1][j], ox[i][1][j], ss);
        }
        ss = dpp_sum16(ss);
        const float inv = __builtin_amdgcn_rsqf(ss * (1.f / kD) + eps);
        float y[8];
        for (int j = 0; j < 4; ++j) {
            y[j] = ox[i][0][j] * inv * wx[j];
            y[4 + j] = ox[i][1][j] * inv * wx[4 + j];
        }
        if (kAct != RDA_GATE_NONE)
            for (int j = 0; j < 8; ++j) y[j] *= gate_act<kAct>(gx[i][j]);
        if (r0 + i < rows) {
            store_out<TO>(out + (r0 + i) * kD + 4 * c, y);
            store_out<TO>(out + (r0 + i) * kD + 64 + 4 * c, y + 4);
        }
    }
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
