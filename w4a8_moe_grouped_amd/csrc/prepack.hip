// prepack.hip -- one-time re-layout of the int4 weights and their scales into
// the order the GEMM kernels consume (the load-time weight processing SGLang
// PR #7762 does in process_weights_after_loading; the layout is MI355X's own).
//
// Weights [E, N, K/2] -> [E][N/16][G][16][64 B]: the 16 rows of a fragment and
// one 128-K group form one contiguous 1 KB block, so a wave's 64 lanes read
// 1 KB in one load (row-major weights give 16 separate 64-byte pieces 3.5 KB
// apart).  Scales [E, N, G] -> [E][N/16][ceil(G/4)][16][4]: a 16-byte block of
// 4 groups per row, zero past the last group.  Pure data movement.
#include "common.hpp"
#include "internal.hpp"

namespace w4a8 {

// one thread per 16-byte chunk of the packed weights
__global__ __launch_bounds__(256) void prepack_weights_kernel(const uint8_t* __restrict__ w,
                                                              int64_t E, int64_t N, int64_t K,
                                                              uint8_t* __restrict__ wp)
{
    const int64_t G = K / kGroup;
    const int64_t chunks = E * N * G * 4;  // 16-byte chunks
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= chunks)
        return;
    // packed order: e, n/16, g, n%16, quarter
    const int64_t qtr = i & 3;
    int64_t rest = i >> 2;
    const int64_t r = rest % 16;
    rest /= 16;
    const int64_t g = rest % G;
    rest /= G;
    const int64_t nf = rest % (N / 16);
    const int64_t e = rest / (N / 16);
    const int64_t n = nf * 16 + r;
    const v4i v = *(const v4i*)(w + (e * N + n) * (K / 2) + g * 64 + qtr * 16);
    *(v4i*)(wp + i * 16) = v;
}

// one thread per packed scale
__global__ __launch_bounds__(256) void prepack_scales_kernel(const float* __restrict__ ws, int64_t E,
                                                             int64_t N, int64_t K,
                                                             float* __restrict__ sp)
{
    const int64_t G = K / kGroup, G4 = packed_groups4(G);
    const int64_t total = E * N * G4 * 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total)
        return;
    const int64_t j = i & 3;
    int64_t rest = i >> 2;
    const int64_t r = rest % 16;
    rest /= 16;
    const int64_t b = rest % G4;
    rest /= G4;
    const int64_t nf = rest % (N / 16);
    const int64_t e = rest / (N / 16);
    const int64_t g = b * 4 + j;
    sp[i] = g < G ? ws[(e * N + nf * 16 + r) * G + g] : 0.0f;
}

hipError_t launch_prepack(const uint8_t* w, const float* ws, int64_t E, int64_t N, int64_t K,
                          uint8_t* wp, float* sp, hipStream_t s)
{
    const int64_t G = K / kGroup;
    const int64_t chunks = E * N * G * 4;
    const int64_t scales = E * N * packed_groups4(G) * 4;
    if (chunks > 0)
        hipLaunchKernelGGL(prepack_weights_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                           s, w, E, N, K, wp);
    if (scales > 0)
        hipLaunchKernelGGL(prepack_scales_kernel, dim3((unsigned)((scales + 255) / 256)), dim3(256), 0,
                           s, ws, E, N, K, sp);
    return hipGetLastError();
}

} // namespace w4a8
