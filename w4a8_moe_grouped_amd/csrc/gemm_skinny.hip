// gemm_skinny.hip -- grouped W4A8 GEMM for few rows per expert (decode).
//
// y[p, n] = sum_g w_scale[n, g] * a_scale[p, g] * sum_{k in g} a[p, k] * w[n, k]
// over the rows p of one m-block of one expert (SGLang PR #7762: w4a8
// grouped GEMM over expert segments, weight groups of 128 along K; DeepGEMM
// PR #53 "Changes": small batches put the tokens on the narrow side of the
// MMA -- the swapAB idea).
//
// Work decomposition: a workgroup (4 waves) owns one m-block of BM = 16*NT
// rows of one expert and 256 weight rows (4 waves x 4 fragments of 16).  The
// rows sit on the A side of v_mfma_f32_16x16x128_f8f6f4 and the weight rows
// on the B side, so every weight byte is loaded from HBM exactly once per
// m-block, straight into VGPRs (16 bytes per lane, no LDS), through a ring of
// D groups in flight.  One MFMA covers one 128-group, so the per-group scale
// promotion is exact: acc += w_scale * fma(raw, c1, c0) (see common.hpp).
//
// Epilogues:
//   EPI_F32      out_f32[p, n]                       (down GEMM)
//   EPI_BF16     out_bf16[p, n]                      (dense linear)
//   EPI_SWIGLU_Q the tile holds gate rows i and up rows I+i of one 128-block
//                of i: h = silu(gate) * up, then fp8 requant of the block
//                (DeepGEMM PR #53 "Changes": SwiGLU -> per-token FP8 requant;
//                SGLang PR #7762: SiLU-and-Mul between the grouped GEMMs).
#include "common.hpp"
#include "internal.hpp"

#include <type_traits>

namespace w4a8 {

constexpr int kNF = 4;  // weight fragments (16 rows) per wave
constexpr int kWaves = 4;

template <int NT, int EPI, int D, bool F16>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs a)
{
    constexpr int BM = 16 * NT;
    constexpr int ESZ = F16 ? 2 : 1;   // activation element size
    constexpr int AV = F16 ? 4 : 2;    // 16-byte activation loads per lane per group
    extern __shared__ float4 lds_side4[];  // [G][BM] float2 {c1, c0}, 16-byte aligned
    float2* lds_side = (float2*)lds_side4;
    __shared__ int s_rows[BM];
    __shared__ float s_red[kWaves][BM];
    __shared__ float s_red2[kWaves][BM];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[EPI == EPI_SWIGLU_Q ? BM * kGroup : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, q = lane >> 4, c16 = lane & 15;
    const int64_t K = a.K, N = a.N, G = K / kGroup;

    int e, row0, rows;
    if (a.offsets != nullptr) {
        if ((int)blockIdx.y >= *a.num_blocks)
            return;
        e = a.block_expert[blockIdx.y];
        row0 = a.block_row[blockIdx.y];
        rows = min(BM, a.offsets[e + 1] - row0);
    } else {
        e = 0;
        row0 = (int)blockIdx.y * BM;
        if (row0 >= a.dense_rows)
            return;
        rows = min(BM, a.dense_rows - row0);
    }

    for (int i = tid; i < BM; i += 256)
        s_rows[i] = i < rows ? (a.sorted != nullptr ? a.sorted[row0 + i] / a.topk : row0 + i) : -1;
    __syncthreads();
    for (int i = tid; i < G * BM; i += 256) {
        const int g = i / BM, c = i - g * BM;
        const int r = s_rows[c];
        lds_side[i] = r >= 0 ? a.act_side[(int64_t)r * G + g] : make_float2(0.0f, 0.0f);
    }
    __syncthreads();

    // weight rows of this lane (one per fragment)
    int64_t nrow[kNF];
    bool nvalid[kNF];
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
        int64_t n;
        if (EPI == EPI_SWIGLU_Q)
            n = (f >= 2 ? a.I : 0) + (int64_t)blockIdx.x * kGroup + 32 * wave + 16 * (f & 1) + c16;
        else
            n = (int64_t)blockIdx.x * 256 + 64 * wave + 16 * f + c16;
        nvalid[f] = n < N;
        nrow[f] = nvalid[f] ? n : N - 1;
    }
    const uint8_t* wbase = a.w + (int64_t)e * a.w_estride;
    const float* sbase = a.ws + (int64_t)e * a.s_estride;
    const uint8_t* wp[kNF];
    const float* sp[kNF];
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
        wp[f] = wbase + nrow[f] * (K / 2) + 16 * q;
        sp[f] = sbase + nrow[f] * G;
    }
    const uint8_t* ap[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        int r = s_rows[16 * t + c16];
        if (r < 0)
            r = s_rows[0];
        // the lane's 16-byte chunks are q, 4+q, 8+q, 12+q (f16) or q, 4+q (fp8)
        ap[t] = a.act + (int64_t)r * K * ESZ + 16 * q;
    }

    // The f16 (gate_up) path promotes in fp64: each group's MFMA sum is the
    // correctly rounded fp32 value of an exact dot product, and keeping the
    // running sum in fp64 leaves y within ~2^-25 of the exact result, so the
    // SwiGLU + fp8 requant that follows almost never lands on another code.
    // The fp8 path promotes in fp32.
    using Acc = typename std::conditional<F16, double, float>::type;
    Acc acc[kNF][NT][4];
#pragma unroll
    for (int f = 0; f < kNF; ++f)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[f][t][r] = 0;

    // Ring of D groups in flight.  The loop runs over ceil(G/D)*D groups with
    // no branches: a refill past the last group reloads group G-1 (in bounds,
    // never used), and a padding group g >= G gets weight scale 0.
    // Weight scales: with G % 4 == 0 (and D == 4) one float4 per fragment
    // covers a whole turn of the ring, loaded one turn ahead.
    const bool sw4 = (G % 4 == 0) && (D == 4);
    v4i wb[D][kNF];
    v4i ab[D][NT][AV];
    float sb[D][kNF];
    float4 sw_cur[kNF], sw_next[kNF];

    auto load_group = [&](int s, int64_t g) {
#pragma unroll
        for (int f = 0; f < kNF; ++f) {
            wb[s][f] = ldg16(wp[f] + g * 64);
            if (!sw4)
                sb[s][f] = sp[f][g];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < AV; ++v)
                ab[s][t][v] = ldg16(ap[t] + g * kGroup * ESZ + 64 * v);
    };
    auto load_sw4 = [&](int64_t g4) {  // groups g4..g4+3, g4 % 4 == 0, g4 + 3 < G
#pragma unroll
        for (int f = 0; f < kNF; ++f)
            sw_next[f] = *(const float4*)(sp[f] + g4);
    };

    if (sw4) {
        load_sw4(0);
#pragma unroll
        for (int f = 0; f < kNF; ++f)
            sw_cur[f] = sw_next[f];
    }
#pragma unroll
    for (int s = 0; s < D; ++s)
        load_group(s, s < G ? s : G - 1);
    __builtin_amdgcn_sched_barrier(0);

    const int64_t Gr = (G + D - 1) / D * D;
    for (int64_t g0 = 0; g0 < Gr; g0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int64_t g = g0 + s;
            const int64_t gl = g < G ? g : G - 1;  // side data row (padding groups: any valid one)
            const bool live = g < G;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float4* sd = (const float4*)&lds_side[gl * BM + 16 * t + 4 * q];
                const float4 s01 = sd[0], s23 = sd[1];
                const float c1[4] = {s01.x, s01.z, s23.x, s23.z};
                const float c0[4] = {s01.y, s01.w, s23.y, s23.w};
                v8i at;
                v8h ah[4];
                if (F16) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        ah[c] = __builtin_bit_cast(v8h, ab[s][t][c]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        at[i] = ab[s][t][0][i];
                        at[4 + i] = ab[s][t][1][i];
                    }
                }
#pragma unroll
                for (int f = 0; f < kNF; ++f) {
                    float swsel;
                    if (sw4)
                        swsel = s == 0 ? sw_cur[f].x : s == 1 ? sw_cur[f].y : s == 2 ? sw_cur[f].z : sw_cur[f].w;
                    else
                        swsel = sb[s][f];
                    const float swf = live ? swsel : 0.0f;
                    v4f raw = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                    if (F16) {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            raw = mfma16x16x32_f16(ah[c], unpack_int4_f16((uint32_t)wb[s][f][c]), raw);
                        // c0 == 0 on this path; sw * c1 is exact in fp64
                        const double swd = (double)swf;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[f][t][r] = fma((double)raw[r], swd * (double)c1[r], (double)acc[f][t][r]);
                    } else {
                        raw = mfma16x16x128(at, unpack_int4_u(wb[s][f]), raw);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[f][t][r] = fmaf(swf, fmaf(raw[r], c1[r], c0[r]), (float)acc[f][t][r]);
                    }
                }
            }
            // keep the refill here, D groups ahead of its use: without the
            // barrier the scheduler sinks each load next to its consumer and
            // only one load stays in flight
            __builtin_amdgcn_sched_barrier(0);
            const int64_t gn = g + D < G ? g + D : G - 1;
            load_group(s, gn);
            if (sw4 && s == 0)
                load_sw4(g0 + D + 3 < G ? g0 + D : G - 4);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (sw4) {
#pragma unroll
            for (int f = 0; f < kNF; ++f)
                sw_cur[f] = sw_next[f];
        }
    }

    // ---- epilogues ----  output element (row 16t+4q+r of the block, weight row nrow[f])
    if (EPI == EPI_F32 || EPI == EPI_BF16) {
#pragma unroll
        for (int f = 0; f < kNF; ++f) {
            if (!nvalid[f])
                continue;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * t + 4 * q + r;
                    if (row < rows) {
                        const int64_t o = (int64_t)(row0 + row) * N + nrow[f];
                        if (EPI == EPI_F32)
                            a.out_f32[o] = (float)acc[f][t][r];
                        else
                            a.out_bf16[o] = f32_to_bf16((float)acc[f][t][r]);
                    }
                }
        }
        return;
    }

    if (EPI == EPI_SWIGLU_Q) {
        // h for i_local = 32*wave + 16*j + c16, j = 0, 1
        float h[2][NT][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // SwiGLU in fp64, one rounding to fp32 (as the definition)
                    const double gt = (double)acc[j][t][r], up = (double)acc[j + 2][t][r];
                    h[j][t][r] = (float)(gt / (1.0 + exp(-gt)) * up);
                }
        // amax per row over the 128 i's: in-lane (j), 16 lanes (c16), 4 waves (LDS)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float m = fmaxf(fabsf(h[0][t][r]), fabsf(h[1][t][r]));
                m = group_max<16>(m);
                if (c16 == 0)
                    s_red[wave][16 * t + 4 * q + r] = m;
            }
        __syncthreads();
        float inv[NT][4], scl[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * t + 4 * q + r;
                const float m = fmaxf(fmaxf(s_red[0][row], s_red[1][row]),
                                      fmaxf(s_red[2][row], s_red[3][row]));
                const float amax_c = clamp_amax(m);
                inv[t][r] = recip448(amax_c);
                scl[t][r] = scale_of(amax_c);
            }
        // codes, sum of decoded codes, and the interleaved byte position of each i
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * t + 4 * q + r;
                const uint32_t cc = cvt_e4m3x2(h[0][t][r] * inv[t][r], h[1][t][r] * inv[t][r]);
                const float2 dv = dec_e4m3x2(cc);
                float sum = group_sum<16>(dv.x + dv.y);
                if (c16 == 0)
                    s_red2[wave][row] = sum;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int il = 32 * wave + 16 * j + c16;
                    const int b = il & 7;
                    const int pos = fp8_group_pos(il >> 3) + ((b & 1) ? 4 + (b >> 1) : (b >> 1));
                    s_q[row * kGroup + pos] = (uint8_t)((cc >> (8 * j)) & 0xFFu);
                }
            }
        __syncthreads();
        const int64_t GI = a.I / kGroup;
        for (int i = tid; i < BM * 8; i += 256) {
            const int row = i >> 3, chunk = i & 7;
            if (row < rows) {
                const int64_t p = row0 + row;
                *(v4i*)(a.out_q + p * a.I + (int64_t)blockIdx.x * kGroup + chunk * 16) =
                    *(const v4i*)(s_q + row * kGroup + chunk * 16);
            }
        }
        for (int row = tid; row < BM; row += 256) {
            if (row < rows) {
                const float sum = s_red2[0][row] + s_red2[1][row] + s_red2[2][row] + s_red2[3][row];
                const float m = fmaxf(fmaxf(s_red[0][row], s_red[1][row]),
                                      fmaxf(s_red[2][row], s_red[3][row]));
                const float sc = scale_of(clamp_amax(m));
                a.out_side[(int64_t)(row0 + row) * GI + blockIdx.x] =
                    make_float2(512.0f * sc, -8.0f * (sc * sum));
            }
        }
    }
}

template <int NT, int EPI, int D, bool F16>
static hipError_t launch_one(const GemmArgs& a, hipStream_t s)
{
    const int64_t G = a.K / kGroup;
    const size_t lds = (size_t)G * 16 * NT * sizeof(float2);
    dim3 grid;
    if (EPI == EPI_SWIGLU_Q)
        grid.x = (unsigned)(a.I / kGroup);
    else
        grid.x = (unsigned)((a.N + 255) / 256);
    grid.y = (unsigned)a.max_blocks;
    grid.z = 1;
    if (grid.x == 0 || grid.y == 0)
        return hipSuccess;
    hipLaunchKernelGGL((gemm_skinny_kernel<NT, EPI, D, F16>), grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

size_t skinny_lds_bytes(int64_t K, int block_m)
{
    return (size_t)(K / kGroup) * (size_t)block_m * sizeof(float2);
}

hipError_t launch_gemm_skinny(const GemmArgs& a, int epilogue, int block_m, hipStream_t s)
{
    // gate_up (SwiGLU epilogue) runs on the exact f16 path, the others on fp8
#define W4A8_SKINNY(NT, D)                                                         \
    switch (epilogue) {                                                            \
    case EPI_F32: return launch_one<NT, EPI_F32, D, false>(a, s);                  \
    case EPI_BF16: return launch_one<NT, EPI_BF16, D, false>(a, s);                \
    default: return launch_one<NT, EPI_SWIGLU_Q, D, true>(a, s);                   \
    }
    if (block_m <= 16) {
        W4A8_SKINNY(1, 4)
    } else if (block_m <= 32) {
        W4A8_SKINNY(2, 3)
    } else {
        W4A8_SKINNY(4, 2)
    }
#undef W4A8_SKINNY
}

} // namespace w4a8
