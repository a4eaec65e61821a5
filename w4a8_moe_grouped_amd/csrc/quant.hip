// quant.hip -- dynamic per-token-per-128 fp8 activation quantisation.
//
// Rule (DeepGEMM PR #53, commit note dropping the UE8M0 activation scale:
// fp32 per-token scales, amax clamped before the reciprocal 448/amax;
// SGLang PR #37796, part-1 notes on the fp8 KV write: saturate to +-448
// before the e4m3 cast):
//   amax_c = max(max|x|, 1e-10f); inv = 448/amax_c; scale = amax_c/448;
//   code = e4m3_rne(clamp(x*inv, +-448)).
//
// One 128-wide block is handled by 16 lanes, 8 consecutive elements each
// (one 16-byte load of bf16); a 256-thread block covers 16 blocks.  The
// kernel is HBM-bound: 2 bytes read and ~1 byte written per element.
#include "common.hpp"
#include "internal.hpp"

namespace w4a8 {

// MODE 0: canonical codes + scales (the public export)
// MODE 1: K-interleaved codes + {512*s, -8*s*sum(dec)} (fp8 GEMM operand)
// MODE 2: codes in the order k0,k4,k1,k5,k2,k6,k3,k7 per 8-group (fp8_group_pos
//         placement) + {s, 0} (the f16 GEMM operand, converted in registers)
template <int MODE>
__global__ __launch_bounds__(256) void quant_bf16_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                         int64_t K, int64_t ldx,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scales,
                                                         float2* __restrict__ side)
{
    const int64_t G = K / kGroup;
    const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
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
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
    amax = group_max<16>(amax);
    const float amax_c = clamp_amax(amax);
    const float inv = recip448(amax_c);
    const float scale = scale_of(amax_c);

    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        c[i] = cvt_e4m3x2(v[2 * i] * inv, v[2 * i + 1] * inv);
    uint32_t d0 = c[0] | (c[1] << 16), d1 = c[2] | (c[3] << 16);

    if (MODE == 2) {
        // fp8 codes for the f16 gate_up path: inside the 8-group the order is
        // k0,k4,k1,k5 | k2,k6,k3,k7 (pairs converted to f16 with one
        // instruction line up with the int4 -> f16 unpack)
        const uint32_t p0 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
        const uint32_t p1 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
        *(uint2*)(q + m * K + g * kGroup + fp8_group_pos(sub)) = make_uint2(p0, p1);
        if (sub == 0)
            side[m * G + g] = make_float2(scale, 0.0f);
        return;
    }
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

hipError_t launch_quant_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                             float* scales, float2* side, int mode, hipStream_t s)
{
    const int64_t blocks = (M * (K / kGroup) + 15) / 16;
    if (blocks == 0)
        return hipSuccess;
    if (mode == 0)
        hipLaunchKernelGGL(quant_bf16_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, x, M, K,
                           ldx, q, scales, side);
    else if (mode == 1)
        hipLaunchKernelGGL(quant_bf16_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, x, M, K,
                           ldx, q, scales, side);
    else
        hipLaunchKernelGGL(quant_bf16_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, x, M, K,
                           ldx, q, scales, side);
    return hipGetLastError();
}

// Canonical codes + fp32 scales (the public quantiser's output) -> the GEMM
// operand form: K-interleaved codes and {c1, c0} = {512*s, -8*s*sum(dec)}.
__global__ __launch_bounds__(256) void prep_codes_kernel(const uint8_t* __restrict__ q,
                                                         const float* __restrict__ scales,
                                                         int64_t M, int64_t K,
                                                         uint8_t* __restrict__ q_il,
                                                         float2* __restrict__ side)
{
    const int64_t G = K / kGroup;
    const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    if (gid >= M * G)
        return;
    const int64_t m = gid / G, g = gid - m * G;
    const uint2 d = *(const uint2*)(q + m * K + g * kGroup + sub * 8);
    float s = 0.0f;
    const uint32_t w[4] = {d.x & 0xFFFFu, d.x >> 16, d.y & 0xFFFFu, d.y >> 16};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float2 f = dec_e4m3x2(w[i]);
        s += f.x + f.y;
    }
    s = group_sum<16>(s);
    uint32_t lo, hi;
    interleave8(d.x, d.y, lo, hi);
    *(uint2*)(q_il + m * K + g * kGroup + fp8_group_pos(sub)) = make_uint2(lo, hi);
    if (sub == 0) {
        const float sc = scales[m * G + g];
        side[m * G + g] = make_float2(512.0f * sc, -8.0f * (sc * s));
    }
}

hipError_t launch_prep_codes(const uint8_t* q, const float* scales, int64_t M, int64_t K,
                             uint8_t* q_il, float2* side, hipStream_t s)
{
    const int64_t blocks = (M * (K / kGroup) + 15) / 16;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(prep_codes_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q, scales, M, K,
                       q_il, side);
    return hipGetLastError();
}

} // namespace w4a8
