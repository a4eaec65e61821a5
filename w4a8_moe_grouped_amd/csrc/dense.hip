// dense.hip -- the dense W4AFP8 linear (w4a8_gemm): out = bf16(A * W^T) with
// per-128-K promotion of both scales (SGLang PR #7762, "Model Info": dense
// layers next to the MoE; the chunk-size thread: groups of 128 along K).
//
// Shape of the work: M is small next to N * K (one token batch through one
// projection), so a workgroup owns every one of up to 128 rows, 64 weight
// rows and one slice of K; slices of K run in parallel workgroups and their
// fp32 partial sums are added in slice order by split_reduce_kernel (one
// bf16 rounding).  Each wave holds one 16-row weight fragment against the
// 128 rows (eight 16 x 16 tiles of v_mfma_f32_16x16x128_f8f6f4).
//
// Operands as w4a8_quantize_act writes them and as the caller stores the
// weights: canonical e4m3 codes [M, K] with fp32 scales [M, K/128], packed
// int4 [N, K/2] with fp32 scales [N, K/128].  No re-layout pass:
//  * a lane's 32 K-positions of a group are K [32q, 32q + 32) in natural
//    order on both sides (which positions a lane holds only has to agree
//    between A and B, the MFMA sums over all of them);
//  * weight nibble v (two's complement) becomes the e4m3 code of v * 2^-9:
//    |v| <= 7 are the subnormal codes |v|, -8 is 2^-6 = code 0x08, with the
//    sign bit -- exact, and no bias to remove afterwards;
//  * y += w_scale * (a_scale * 2^9 * raw) per group.
//
// Pipeline: the activation chunks of a group (128 rows x 128 B) and the
// wave's weight fragment (16 rows x 64 B) go straight from global memory
// into LDS (buffer_load ... lds), DW groups in flight in a ring of DW + 1
// stages, one explicit vmcnt wait and one barrier per group.  The scales of
// the whole slice are copied into LDS before the ring starts.
#include "common.hpp"
#include "internal.hpp"
#include "lds_direct.hpp"

namespace w4a8 {

namespace {

constexpr int kDRows = 128;                  // rows per workgroup
constexpr int kDCols = 64;                   // weight rows per workgroup (4 waves x 16)
constexpr int kDW = 4;                       // groups in flight
constexpr int kDStages = kDW + 1;
constexpr int kDAct = kDRows * kGroup;       // 16 KB of activation codes per stage
constexpr int kDWgt = kDCols * kGroup / 2;   // 4 KB of packed weights per stage
constexpr int kDStage = kDAct + kDWgt;
constexpr int kDMaxSplitGroups = 16;         // groups per K slice (scales staged in LDS)
constexpr int kDActLoads = kDAct / (1024 * 4);  // 16-byte direct loads per wave per group (4)
constexpr int kDLoads = kDActLoads + 1;         // + the wave's weight fragment

// four nibbles (one per byte, two's complement) -> e4m3 codes of v * 2^-9
__device__ __forceinline__ uint32_t int4_to_e4m3(uint32_t b)
{
    const uint32_t s = (b >> 3) & 0x01010101u;  // sign per byte
    const uint32_t m = s * 0x0Fu;               // 0x0F in negative bytes
    const uint32_t mag = (b ^ m) + s;           // |v| (16 - n for n >= 8), at most 8
    return mag | (s << 7);
}

// 16 packed bytes (32 nibbles, k even in the low nibble) -> 32 e4m3 codes in
// natural K order
__device__ __forceinline__ v8i unpack_int4_signed(const v4i& w)
{
    v8i r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = (uint32_t)w[i];
        const uint32_t lo = int4_to_e4m3(x & 0x0F0F0F0Fu);         // k0, k2, k4, k6
        const uint32_t hi = int4_to_e4m3((x >> 4) & 0x0F0F0F0Fu);  // k1, k3, k5, k7
        r[2 * i] = (int)__builtin_amdgcn_perm(hi, lo, 0x05010400u);     // k0, k1, k2, k3
        r[2 * i + 1] = (int)__builtin_amdgcn_perm(hi, lo, 0x07030602u); // k4, k5, k6, k7
    }
    return r;
}

// activation row r, 16-byte chunk c (0..7) of a group -> its LDS slot (the
// XOR spreads one chunk column over the banks)
__device__ __forceinline__ int act_slot(int r, int c)
{
    return r * 8 + (c ^ (r & 7));
}

}  // namespace

// grid: (ceil(N / 64), ceil(M / 128), splits).  SPLIT: write fp32 partials of
// slice blockIdx.z at out_f32 + z * M * N, else bf16 results.
template <bool SPLIT>
__global__ __launch_bounds__(256) void dense_gemm_kernel(const uint8_t* __restrict__ a,
                                                         const float* __restrict__ sa, int64_t M,
                                                         int64_t K, const uint8_t* __restrict__ w,
                                                         const float* __restrict__ sw, int64_t N,
                                                         int32_t split_groups,
                                                         float* __restrict__ out_f32,
                                                         uint16_t* __restrict__ out_bf16)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[kDStages * kDStage];
    __shared__ float s_sa[kDMaxSplitGroups][kDRows];
    __shared__ float s_sw[kDMaxSplitGroups][kDCols];

    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Gt = (int)(K / kGroup);
    const int gbase = (int)blockIdx.z * split_groups;
    const int G = min(split_groups, Gt - gbase);
    const int64_t m0 = (int64_t)blockIdx.y * kDRows;
    const int64_t n0 = (int64_t)blockIdx.x * kDCols;
    const int rows = (int)min((int64_t)kDRows, M - m0);

    // scales of the slice (rows / weight rows past the end read a valid row)
    for (int i = tid; i < G * kDRows; i += 256) {
        const int g = i / kDRows, r = i - g * kDRows;
        s_sa[g][r] = sa[(m0 + min(r, rows - 1)) * Gt + gbase + g];
    }
    for (int i = tid; i < G * kDCols; i += 256) {
        const int g = i / kDCols, c = i - g * kDCols;
        s_sw[g][c] = sw[min(n0 + c, N - 1) * Gt + gbase + g];
    }

    // per-lane global offsets of the direct loads (group 0 of the slice;
    // the group advance goes in the scalar offset)
    const v4i ra = sgpr_rsrc(a, (uint32_t)(M * K));
    const v4i rw = sgpr_rsrc(w, (uint32_t)(N * (K / 2)));
    uint32_t va[kDActLoads];
#pragma unroll
    for (int j = 0; j < kDActLoads; ++j) {
        const int slot = (wave * kDActLoads + j) * 64 + lane;
        const int r = slot >> 3, c = (slot & 7) ^ (r & 7);
        va[j] = (uint32_t)((m0 + min(r, rows - 1)) * K + (int64_t)gbase * kGroup + 16 * c);
    }
    // the wave's fragment: lane (c16, q) takes packed bytes [16q, 16q + 16) of
    // weight row n0 + 16 wave + c16 (K [32q, 32q + 32) of the group)
    const uint32_t vw =
        (uint32_t)(min(n0 + 16 * wave + c16, N - 1) * (K / 2) + (int64_t)gbase * (kGroup / 2) + 16 * q);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)s_stage;
    auto issue = [&](int g, int st) {  // group g of the slice into stage st
        const uint32_t base = lds0 + (uint32_t)(st * kDStage);
#pragma unroll
        for (int j = 0; j < kDActLoads; ++j)
            lds_load16(ra, base + (uint32_t)((wave * kDActLoads + j) * 1024), va[j], (uint32_t)g * kGroup);
        lds_load16(rw, base + (uint32_t)(kDAct + wave * 1024), vw, (uint32_t)g * (kGroup / 2));
    };

    float acc[kDRows / 16][4];
#pragma unroll
    for (int s = 0; s < kDRows / 16; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc[s][r] = 0.0f;

#pragma unroll
    for (int g = 0; g < kDW; ++g)
        issue(g < G ? g : G - 1, g);

    for (int g = 0; g < G; ++g) {
        // group g landed (the DW - 1 batches behind it may still fly; a
        // refill past the last group reloads it, so the count is uniform)
        wait_vmcnt<kDLoads * (kDW - 1)>();
        barrier();
        const uint8_t* st = s_stage + (g % kDStages) * kDStage;
        const v4i wq = *(const v4i*)(st + kDAct + wave * 1024 + 16 * lane);
        const v8i b = unpack_int4_signed(wq);
        const float swv = s_sw[g][16 * wave + c16];
#pragma unroll
        for (int s = 0; s < kDRows / 16; ++s) {
            const int r = 16 * s + c16;
            const v4i a0 = *(const v4i*)(st + 16 * act_slot(r, 2 * q));
            const v4i a1 = *(const v4i*)(st + 16 * act_slot(r, 2 * q + 1));
            const v8i av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const v4f raw = mfma16x16x128(av, b, v4f{0.0f, 0.0f, 0.0f, 0.0f});
            const float4 sa4 = *(const float4*)&s_sa[g][16 * s + 4 * q];
            const float sar[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)  // raw counts units of 2^-9 * a_code
                acc[s][i] = fmaf(swv, raw[i] * (sar[i] * 512.0f), acc[s][i]);
        }
        // the stage of group g - 1 is free (every wave passed this group's
        // barrier after reading it): refill it with group g + DW
        issue(g + kDW < G ? g + kDW : G - 1, (g + kDW) % kDStages);
    }
    wait_vmcnt<0>();  // no direct load may land after the workgroup's LDS is freed

    const int64_t n = n0 + 16 * wave + c16;
    if (n >= N)
        return;
#pragma unroll
    for (int s = 0; s < kDRows / 16; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * s + 4 * q + i;
            if (r < rows) {
                if (SPLIT)
                    out_f32[(int64_t)blockIdx.z * M * N + (m0 + r) * N + n] = acc[s][i];
                else
                    out_bf16[(m0 + r) * N + n] = f32_to_bf16(acc[s][i]);
            }
        }
}

// Partial sums of the K slices -> bf16: out[i] = bf16(sum over slices z
// ascending of part[z][i]), one rounding; four elements per thread (16-byte
// loads when M * N % 4 == 0, else element by element).
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int32_t splits,
                                                           int64_t MN, uint16_t* __restrict__ out)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN)
        return;
    if ((MN & 3) == 0) {
        float4 acc = *(const float4*)(part + i);
        for (int z = 1; z < splits; ++z) {
            const float4 v = *(const float4*)(part + (int64_t)z * MN + i);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
        o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
        *(uint2*)(out + i) = o;
        return;
    }
    for (int64_t k = i; k < i + 4 && k < MN; ++k) {
        float acc = part[k];
        for (int z = 1; z < splits; ++z)
            acc += part[(int64_t)z * MN + k];
        out[k] = f32_to_bf16(acc);
    }
}

hipError_t launch_split_reduce(const float* part, int32_t splits, int64_t M, int64_t N, uint16_t* out,
                               hipStream_t s)
{
    const int64_t MN = M * N;
    if (MN == 0)
        return hipSuccess;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((MN + 1023) / 1024)), dim3(256), 0, s, part,
                       splits, MN, out);
    return hipGetLastError();
}

int dense_max_split_groups()
{
    return kDMaxSplitGroups;
}

hipError_t launch_dense_gemm(const uint8_t* a, const float* sa, int64_t M, int64_t K, const uint8_t* w,
                             const float* sw, int64_t N, int32_t split_groups, float* part,
                             uint16_t* out, hipStream_t s)
{
    const int64_t G = K / kGroup;
    if (split_groups < 1 || split_groups > kDMaxSplitGroups)
        return hipErrorInvalidValue;
    const int64_t splits = (G + split_groups - 1) / split_groups;
    const dim3 grid((unsigned)((N + kDCols - 1) / kDCols), (unsigned)((M + kDRows - 1) / kDRows),
                    (unsigned)splits);
    if (splits > 1)
        hipLaunchKernelGGL(dense_gemm_kernel<true>, grid, dim3(256), 0, s, a, sa, M, K, w, sw, N,
                           split_groups, part, nullptr);
    else
        hipLaunchKernelGGL(dense_gemm_kernel<false>, grid, dim3(256), 0, s, a, sa, M, K, w, sw, N,
                           split_groups, nullptr, out);
    return hipGetLastError();
}

}  // namespace w4a8
