// rda_out.h -- the stores of a prefill walk's outputs, shared by the walks
// for bf16 and fp32 inputs.  A walk's output wave holds one MFMA accumulator
// tile: lane (g, c) has value channel 16 s + c (slice s of the head) of the
// chunk's token rows r0 + 4 g + i, i < 4.  The outputs go either to fp32
// rows or to the 16-bit form the fused output norm reads (OutSink): per
// token, the 16 lanes of row g find the slice's largest magnitude (its
// exponent E sets a power-of-two scale, exact in fp32), convert the scaled
// values to fp16 and carry E in the lowest bits of the first 8 of them, so
// the form needs no store besides the values.  A slice's scale keeps its values in fp16's
// normal range whatever the outputs' magnitude, and fp16's 10 remaining
// significand bits keep the norm pass's one bf16 rounding the dominant
// error.
#pragma once

#include "rda_device.h"
#include "rda_internal.h"

namespace rda {

// ov: the tile; row0 = the chunk's first token, r0 = first row of the tile
// within the chunk, len = the chunk's valid rows; H, h, s: heads, head, slice.
// Every lane of the wave must call it (the slice maxima reduce across lanes).
__device__ __forceinline__ void store_out_tile(const OutSink& sk, const f32x4& ov, int row0,
                                               int r0, int len, int H, int h, int s, int g,
                                               int c) {
    if (sk.o) {
        float* orow = sk.o + (size_t(row0 + r0 + 4 * g) * H + h) * kD + 16 * s + c;
        const size_t tstride = size_t(H) * kD;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (r0 + 4 * g + e < len) orow[e * tstride] = ov[e];
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t mx = dpp_umax16(__float_as_uint(ov[e]) & 0x7fffffffu);
        const int E = int(mx >> 23);   // biased exponent of the slice's largest |o|
        const float yv = E ? __builtin_amdgcn_ldexpf(ov[e], 126 - E) : 0.f;
        const uint32_t hb = __builtin_bit_cast(uint16_t, _Float16(yv));
        const uint32_t code = c < 8 ? (hb & ~1u) | ((uint32_t(E) >> c) & 1u) : hb;
        if (r0 + 4 * g + e < len)
            sk.y[(size_t(row0 + r0 + 4 * g + e) * H + h) * kD + 16 * s + c] = uint16_t(code);
    }
}

}  // namespace rda
