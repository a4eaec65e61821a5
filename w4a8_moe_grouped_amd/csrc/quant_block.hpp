// quant_block.hpp -- one 256-thread block of the dynamic per-token-per-128
// fp8 activation quantisation (shared by the quantiser and the fused
// align + quantise launch).
//
// Rule (DeepGEMM PR #53, commit note dropping the UE8M0 activation scale:
// fp32 per-token scales, amax clamped before the reciprocal 448/amax;
// SGLang PR #37796, part-1 notes on the fp8 KV write: saturate to +-448
// before the e4m3 cast):
//   amax_c = max(max|x|, 1e-10f); inv = 448/amax_c; scale = amax_c/448;
//   code = e4m3_rne(clamp(x*inv, +-448)).
//
// One 128-wide block of a row is handled by 16 lanes, 8 consecutive elements
// each (one 16-byte load of bf16); a 256-thread block covers 16 of them.
#pragma once

#include "common.hpp"

namespace w4a8 {

// MODE 0: canonical codes + scales (the public export)
// MODE 1: K-interleaved codes + {512*s, -8*s*sum(dec)} (the GEMM operand)
// fixed_scale: null for the dynamic rule; else a static per-tensor scale s
// (the input scales SGLang PR #7762 loads with the weights): inv = 1/s
// rounded once to fp32, and s is every block's scale.
template <int MODE>
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                            int64_t ldx, uint8_t* __restrict__ q,
                                            float* __restrict__ scales, float2* __restrict__ side,
                                            int64_t block, const float* __restrict__ fixed_scale)
{
    const int64_t G = K / kGroup;
    const int64_t gid = block * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    if (gid >= M * G)
        return;  // uniform over each 16-lane segment
    const int64_t m = gid / G, g = gid - m * G;

    const v4i raw = ldg16_nt(x + m * ldx + g * kGroup + sub * 8);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32((uint16_t)((uint32_t)raw[i] & 0xFFFFu));
        v[2 * i + 1] = bf16_to_f32((uint16_t)((uint32_t)raw[i] >> 16));
    }
    float inv, scale;
    if (fixed_scale != nullptr) {
        scale = *fixed_scale;
        inv = recip_static(scale);
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(v[i]));
        amax = group_max<16>(amax);
        const float amax_c = clamp_amax(amax);
        inv = recip448(amax_c);
        scale = scale_of(amax_c);
    }

    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        c[i] = cvt_e4m3x2(v[2 * i] * inv, v[2 * i + 1] * inv);
    uint32_t d0 = c[0] | (c[1] << 16), d1 = c[2] | (c[3] << 16);

    if (MODE == 1) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float2 f = dec_e4m3x2(c[i]);
            s += f.x + f.y;
        }
        s = group_sum<16>(s);
        uint32_t lo, hi;
        interleave8(d0, d1, lo, hi);
        d0 = lo;
        d1 = hi;
        if (sub == 0)
            side[m * G + g] = make_float2(512.0f * scale, -8.0f * (scale * s));
    } else {
        if (sub == 0)
            scales[m * G + g] = scale;
    }
    const int pos = MODE == 1 ? fp8_group_pos(sub) : sub * 8;
    uint2* dst = (uint2*)(q + m * K + g * kGroup + pos);
    *dst = make_uint2(d0, d1);
}

} // namespace w4a8
