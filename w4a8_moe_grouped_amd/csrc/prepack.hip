// prepack.hip -- one-time re-layout of the int4 weights and their scales into
// the order the GEMM kernels consume (the load-time weight processing SGLang
// PR #7762 does in process_weights_after_loading; the layout is MI355X's own).
//
// Weights [E, N, K/2] -> [E][N/16][G][16][64 B]: the 16 rows of a fragment and
// one 128-K group form one contiguous 1 KB block, so a wave's 64 lanes read
// 1 KB in one load (row-major weights give 16 separate 64-byte pieces 3.5 KB
// apart).  Scales [E, N, G] -> [E][N/16][ceil(G/4)][16][4]: a 16-byte block of
// 4 groups per row, zero past the last group.  Pure data movement.  fp4
// weights (DeepGEMM PR #53, Changes: packed FP4 E2M1 with per-32-K UE8M0
// scales) take the same blocks, with the UE8M0 bytes [E, N, K/32] moved as
// [E, N, G] dwords, and the nibble reorder for the gate_up GEMM.
#include "common.hpp"
#include "internal.hpp"

namespace w4a8 {

// nibbles of one dword k0..k7 (low nibble first) -> k0,k2,k4,k6,k1,k3,k5,k7
__device__ __forceinline__ uint32_t interleave_nibbles(uint32_t x)
{
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int src = i < 4 ? 2 * i : 2 * (i - 4) + 1;
        r |= ((x >> (4 * src)) & 0xFu) << (4 * i);
    }
    return r;
}

// one thread per 16-byte chunk of the packed weights; SHUFFLE reorders the
// nibbles of each dword (fp4 weights of the gate_up GEMM)
template <bool SHUFFLE>
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
    v4i v = *(const v4i*)(w + (e * N + n) * (K / 2) + g * 64 + qtr * 16);
    if (SHUFFLE) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = (int)interleave_nibbles((uint32_t)v[j]);
    }
    *(v4i*)(wp + i * 16) = v;
}

// one thread per packed 4-byte scale element: an fp32 scale, the dword of
// four UE8M0 bytes, or (BF16) a bf16 scale widened to fp32, which is exact
template <bool BF16>
__global__ __launch_bounds__(256) void prepack_scales_kernel(const void* __restrict__ wsv, int64_t E,
                                                             int64_t N, int64_t K,
                                                             uint32_t* __restrict__ sp)
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
    const int64_t src = (e * N + nf * 16 + r) * G + g;
    uint32_t v = 0u;
    if (g < G)
        v = BF16 ? (uint32_t)((const uint16_t*)wsv)[src] << 16 : ((const uint32_t*)wsv)[src];
    sp[i] = v;
}

hipError_t launch_prepack(const uint8_t* w, const void* ws, int64_t E, int64_t N, int64_t K,
                          bool shuffle_nibbles, bool bf16_scales, uint8_t* wp, void* sp, hipStream_t s)
{
    const int64_t G = K / kGroup;
    const int64_t chunks = E * N * G * 4;
    const int64_t scales = E * N * packed_groups4(G) * 4;
    const dim3 wgrid((unsigned)((chunks + 255) / 256));
    if (chunks > 0 && shuffle_nibbles)
        hipLaunchKernelGGL(prepack_weights_kernel<true>, wgrid, dim3(256), 0, s, w, E, N, K, wp);
    else if (chunks > 0)
        hipLaunchKernelGGL(prepack_weights_kernel<false>, wgrid, dim3(256), 0, s, w, E, N, K, wp);
    const dim3 sgrid((unsigned)((scales + 255) / 256));
    if (scales > 0 && bf16_scales)
        hipLaunchKernelGGL(prepack_scales_kernel<true>, sgrid, dim3(256), 0, s, ws, E, N, K, (uint32_t*)sp);
    else if (scales > 0)
        hipLaunchKernelGGL(prepack_scales_kernel<false>, sgrid, dim3(256), 0, s, ws, E, N, K, (uint32_t*)sp);
    return hipGetLastError();
}

} // namespace w4a8
