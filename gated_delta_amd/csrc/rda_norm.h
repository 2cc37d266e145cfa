// rda_norm.h -- one row of the RDA block's output norm and gate, shared by
// the output norm kernel and the walk launches that run it beside the walk:
// per row of one head (128 channels) an RMS normalisation with epsilon and a
// per-channel weight, times an activation of the output gate.  The
// tiny-random/raon-1-mini model card, section "Printing the model", lists
// the block's o_norm (an RMS norm over the head dimension, eps 1e-5) and the
// g_proj projection that produces the gate; the gate's activation is a
// parameter (sigmoid, SiLU or none).
//
//     y_c = o_c / sqrt(mean_c'(o_c'^2) + eps) * w_c * act(g_c)
//
// 16 lanes per row (one DPP row), each lane channels 4c..4c+3 and
// 64+4c..64+4c+3, so every load and store instruction of a 16-lane group
// covers one contiguous run; the row's sum of squares is a 16-lane DPP
// reduction.  The input is fp32 o or the 16-bit form a fused prefill's walk
// leaves (OutSink).
#pragma once

#include "rda_device.h"
#include "rda_internal.h"

namespace rda {

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

// Row r of the output norm and gate by the 16 lanes of one DPP row (lane c
// of the 16; every lane must call it).  kEnc: the row comes in the 16-bit
// form (oe) instead of fp32 (o).  Stores only when `store`; every lane loads
// before it stores and stores only its own elements, so an fp32 output may
// overwrite o in place.
template <typename TG, typename TO, int kAct, bool kEnc>
__device__ __forceinline__ void norm_gate_row(const float* o, const uint16_t* __restrict__ oe,
                                              const TG* __restrict__ g,
                                              const float* __restrict__ w, float eps, int64_t r,
                                              bool store, TO* out, int c) {
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
    f32x4 ox[2];
    float gx[8];
    if constexpr (kEnc) {
        load_enc(oe + r * kD + 4 * c, c, ox[0]);
        load_enc(oe + r * kD + 64 + 4 * c, c, ox[1]);
    } else {
        ox[0] = *reinterpret_cast<const f32x4*>(o + r * kD + 4 * c);
        ox[1] = *reinterpret_cast<const f32x4*>(o + r * kD + 64 + 4 * c);
    }
    if (kAct != RDA_GATE_NONE) {
        load_gate<TG>(g + r * kD + 4 * c, gx);
        load_gate<TG>(g + r * kD + 64 + 4 * c, gx + 4);
    }
    float ss = 0.f;
    for (int j = 0; j < 4; ++j) {
        ss = fmaf(ox[0][j], ox[0][j], ss);
        ss = fmaf(ox[1][j], ox[1][j], ss);
    }
    ss = dpp_sum16(ss);
    const float inv = __builtin_amdgcn_rsqf(ss * (1.f / kD) + eps);
    float y[8];
    for (int j = 0; j < 4; ++j) {
        y[j] = ox[0][j] * inv * wx[j];
        y[4 + j] = ox[1][j] * inv * wx[4 + j];
    }
    if (kAct != RDA_GATE_NONE)
        for (int j = 0; j < 8; ++j) y[j] *= gate_act<kAct>(gx[j]);
    if (store) {
        store_out<TO>(out + r * kD + 4 * c, y);
        store_out<TO>(out + r * kD + 64 + 4 * c, y + 4);
    }
}

}  // namespace rda
