// quant.hip -- per-token-per-128 fp8 activation quantisation, dynamic or with
// a static per-tensor scale (the rules and the block layout are in
// quant_block.hpp).  HBM-bound: 2 bytes read and ~1 byte written per element.
#include "common.hpp"
#include "internal.hpp"
#include "quant_block.hpp"

namespace w4a8 {

template <int MODE>
__global__ __launch_bounds__(256) void quant_bf16_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                         int64_t K, int64_t ldx,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scales,
                                                         float2* __restrict__ side,
                                                         const float* __restrict__ fixed_scale)
{
    quant_block<MODE>(x, M, K, ldx, q, scales, side, blockIdx.x, fixed_scale);
}

hipError_t launch_quant_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                             float* scales, float2* side, int mode, const float* fixed_scale,
                             hipStream_t s)
{
    const int64_t blocks = (M * (K / kGroup) + 15) / 16;
    if (blocks == 0)
        return hipSuccess;
    if (mode == 0)
        hipLaunchKernelGGL(quant_bf16_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, x, M, K,
                           ldx, q, scales, side, fixed_scale);
    else
        hipLaunchKernelGGL(quant_bf16_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, x, M, K,
                           ldx, q, scales, side, fixed_scale);
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
