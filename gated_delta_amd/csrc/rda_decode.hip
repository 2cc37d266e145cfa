// rda_decode.hip -- one decode step of the RDA gated delta rule, in place.
//
// Per (batch, head) the state S [128 x 128] fp32 (row i = value channel,
// column j = key channel) is read once and written once.  The recurrent
// step -- decay, error of the value against the decayed state's prediction
// for the key, beta-weighted write, read-out with the updated state -- is
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

namespace rda {

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

    float kap = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) kap += kx[j] * qx[j];
    kap = dpp_sum16(kap);

    float o_mine = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sk += s[p][0][j] * kx[j] + s[p][1][j] * kx[4 + j];
            sq += s[p][0][j] * qx[j] + s[p][1][j] * qx[4 + j];
        }
        sk = dpp_sum16(sk);
        sq = dpp_sum16(sq);
        const float e = vr[p] - av * sk;
        const float be = bv * e;
        const float orow = av * sq + be * kap;
        if (c == p) o_mine = orow;
        f32x4 n0, n1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            n0[j] = av * s[p][0][j] + be * kx[j];
            n1[j] = av * s[p][1][j] + be * kx[4 + j];
        }
        const int row = 64 * half + 16 * w + 4 * p + g;
        *reinterpret_cast<f32x4*>(Sb + row * kD + 4 * c) = n0;
        *reinterpret_cast<f32x4*>(Sb + row * kD + 64 + 4 * c) = n1;
    }
    if (c < 4) o[bh * kD + 64 * half + 16 * w + 4 * c + g] = o_mine;
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

}  // namespace rda
