// combine.hip -- un-permute and weighted sum of the expert outputs.
//
// SGLang PR #7762 ("Kernel": the post-reorder after the grouped GEMM) and
// DeepGEMM PR #53 ("Changes": ... L2 GEMM -> combine):
//   out[t, n] = bf16( sum_{j < topk, src2dst[t*topk+j] >= 0} w[t, j] * y2[src2dst[t*topk+j], n] )
// with j ascending; a token with no local pair gets +0.  One thread owns 8
// consecutive columns of one token (two 16-byte loads per pair, one 16-byte
// store); HBM-bound.
#include "common.hpp"
#include "internal.hpp"

namespace w4a8 {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y2,
                                                      const int32_t* __restrict__ src2dst,
                                                      const float* __restrict__ topk_w,
                                                      int64_t topk, int64_t H,
                                                      uint16_t* __restrict__ out)
{
    // 1-D grid: xb workgroups per token (grid.y would cap T at 65535)
    const int64_t xb = (H / 8 + 255) / 256;
    const int64_t t = (int64_t)blockIdx.x / xb;
    const int64_t col = (((int64_t)blockIdx.x - t * xb) * 256 + threadIdx.x) * 8;
    if (col >= H)
        return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t j = 0; j < topk; ++j) {
        const int32_t p = src2dst[t * topk + j];
        if (p < 0)
            continue;
        const float w = topk_w[t * topk + j];
        const float4* src = (const float4*)(y2 + (int64_t)p * H + col);
        const float4 u = src[0], v = src[1];
        acc[0] = fmaf(w, u.x, acc[0]);
        acc[1] = fmaf(w, u.y, acc[1]);
        acc[2] = fmaf(w, u.z, acc[2]);
        acc[3] = fmaf(w, u.w, acc[3]);
        acc[4] = fmaf(w, v.x, acc[4]);
        acc[5] = fmaf(w, v.y, acc[5]);
        acc[6] = fmaf(w, v.z, acc[6]);
        acc[7] = fmaf(w, v.w, acc[7]);
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
    *(uint4*)(out + t * H + col) = o;
}

hipError_t launch_combine(const float* y2, const int32_t* src2dst, const float* topk_w,
                          int64_t T, int64_t topk, int64_t H, uint16_t* out, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    dim3 grid((unsigned)((H / 8 + 255) / 256 * T));
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, y2, src2dst, topk_w, topk, H, out);
    return hipGetLastError();
}

} // namespace w4a8
