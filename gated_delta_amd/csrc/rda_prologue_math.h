// rda_prologue_math.h -- the per-channel arithmetic of the RDA block's
// prologue, shared by the prologue kernel and the decode step that runs the
// prologue itself, so that both give the same bits: the causal short
// convolution over K raw tokens, the optional SiLU, the q / k L2 scale, the
// write gate on v, the erase strength b and the floored decay a.
//
// The Raon-1 nano teardown keeps a short convolution window beside the
// recurrent state (section "The cache is small if the runtime keeps it
// small") and gives the gates: b = sigmoid(beta_raw) erases, a write gate
// sigmoid(beta_raw + delta) / sigmoid(beta_raw) scales the value, and the
// decay is bounded below in log space (section "The other 1.5B: a hybrid
// built to forget").
//
// Every multiply-add here is an explicit fmaf and the compiler may fuse
// nothing else (fp contract off), so every kernel that inlines these runs
// the same IEEE operations and gives the same bits.
#pragma once

#include "rda_device.h"

namespace rda {

// Widen two 4-element bf16 runs (this lane's channels 4c.., 64+4c..) to fp32.
__device__ __forceinline__ void widen8(const u32x2 r[2], float out[8]) {
    for (int h = 0; h < 2; ++h) {
        out[4 * h + 0] = __uint_as_float(r[h][0] << 16);
        out[4 * h + 1] = __uint_as_float(r[h][0] & 0xffff0000u);
        out[4 * h + 2] = __uint_as_float(r[h][1] << 16);
        out[4 * h + 3] = __uint_as_float(r[h][1] & 0xffff0000u);
    }
}

// Two fp32 values to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
    const f32x2 v = {x0, x1};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// e^x and ln(x) on the hardware's exp2 / log2 (one instruction each, about
// 1 ulp; the results here end in bf16 or feed gates)
__device__ __forceinline__ float hw_exp(float x) {
#pragma clang fp contract(off)
    return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}
__device__ __forceinline__ float hw_log(float x) {
#pragma clang fp contract(off)
    return __builtin_amdgcn_logf(x) * 0.693147180559945309f;
}

// softplus(y) = ln(1 + e^y), without overflow for large |y|
__device__ __forceinline__ float softplus(float y) {
#pragma clang fp contract(off)
    return fmaxf(y, 0.f) + hw_log(1.f + hw_exp(-fabsf(y)));
}

// One tap of the convolution for n channels: acc += w * x, taps in order
// oldest first (tap K-1 multiplies the current token).
template <int N>
__device__ __forceinline__ void conv_tap(float (&acc)[N], const float (&w)[N],
                                         const float (&x)[N]) {
#pragma unroll
    for (int e = 0; e < N; ++e) acc[e] = fmaf(w[e], x[e], acc[e]);
}

// y * sigmoid(y) for each channel, with the activation selected at compile time.
template <int kAct, int N>
__device__ __forceinline__ void conv_activation(float (&acc)[N]) {
#pragma clang fp contract(off)
    if (kAct == RDA_CONV_ACT_SILU) {
#pragma unroll
        for (int e = 0; e < N; ++e) acc[e] = acc[e] * __builtin_amdgcn_rcpf(1.f + hw_exp(-acc[e]));
    }
}

// 1 / sqrt(sum of squares + eps) of a head's 128 channels held 8 per lane
// by a 16-lane group (channels 4c.., 64+4c..): every lane of the group gets it.
__device__ __forceinline__ float l2_scale(const float (&acc)[8], float eps) {
#pragma clang fp contract(off)
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(acc[e], acc[e], ss);
    return __builtin_amdgcn_rsqf(dpp_sum16(ss) + eps);
}

// sigmoid(beta + delta) / sigmoid(beta) = exp(softplus(-beta) - softplus(-beta - delta)),
// which no ratio of two tiny sigmoids can overflow
__device__ __forceinline__ float write_gate(float beta, float delta) {
#pragma clang fp contract(off)
    return hw_exp(softplus(-beta) - softplus(-beta - delta));
}

// erase strength b = sigmoid(beta_raw)
__device__ __forceinline__ float erase_gate(float beta) {
#pragma clang fp contract(off)
    return __builtin_amdgcn_rcpf(1.f + hw_exp(-beta));
}

// decay a = exp(max(g_log, floor)) (floor = -inf: no floor)
__device__ __forceinline__ float floored_decay(float g_log, float floor_log) {
#pragma clang fp contract(off)
    return hw_exp(fmaxf(g_log, floor_log));
}

}  // namespace rda
