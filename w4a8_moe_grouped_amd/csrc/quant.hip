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

} // namespace w4a8
