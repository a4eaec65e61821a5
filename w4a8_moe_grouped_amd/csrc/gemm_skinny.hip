// gemm_skinny.hip -- grouped W4A8 GEMM for few rows per expert (decode).
//
// y[p, n] = sum_g w_scale[n, g] * a_scale[p, g] * sum_{k in g} a[p, k] * w[n, k]
// over the rows p of one m-block of one expert (SGLang PR #7762: w4a8
// grouped GEMM over expert segments, weight groups of 128 along K; DeepGEMM
// PR #53 "Changes": small batches put the tokens on the narrow side of the
// MMA -- the swapAB idea).
//
// Work decomposition: a workgroup (4 waves) owns one m-block of BM = 16*NT
// rows of one expert and 64*NF weight rows (4 waves x NF fragments of 16).  The
// rows sit on the A side of v_mfma_f32_16x16x128_f8f6f4 and the weight rows
// on the B side, so every weight byte is loaded from HBM exactly once per
// m-block, straight into VGPRs (16 bytes per lane, no LDS), through a ring of
// D groups in flight.  The block's activation rows ride in the same ring,
// either per wave in VGPRs or once per workgroup into LDS (SHARED, below).
// One MFMA covers one 128-group, so the per-group scale promotion is exact:
// acc += w_scale * fma(raw, c1, c0) (see common.hpp).
//
// Epilogues:
//   EPI_F32      out_f32[p, n]                       (down GEMM)
//   EPI_SWIGLU_Q the tile holds gate rows i and up rows I+i of one 128-block
//                of i: h = silu(gate) * up, then fp8 requant of the block
//                (DeepGEMM PR #53 "Changes": SwiGLU -> per-token FP8 requant;
//                SGLang PR #7762: SiLU-and-Mul between the grouped GEMMs).
#include "common.hpp"
#include "internal.hpp"
#include "lds_direct.hpp"

#include <type_traits>


namespace w4a8 {

constexpr int kWaves = 4;
// 16-row m-blocks: ring depth, and weight fragments per wave of the down GEMM
// (128 weight rows per workgroup: see launch_nt)
constexpr int kDW16 = 4;
constexpr int kDownNF16 = 2;


// NF: weight fragments (16 rows) per wave.  FP4: prepacked fp4 e2m1 weights
// with UE8M0 scale dwords (DeepGEMM PR #53, Changes): the f16 path converts
// them exactly with the lane's relative block scale, the fp8 path hands them
// to the scaled MFMA with the lane's block scale.
//
// SG: the finer activation-scale recipes of DeepGEMM PR #53 (one dynamic scale
// per 64 or 32 K of the down GEMM's input instead of 128).  The SwiGLU
// epilogue then emits SG-blocks, and the down GEMM splits each 128-K group into
// 128/SG lane-masked MFMAs, each promoted with its own block scale.
// One workgroup's work: m-block `by` of the block list, weight block `bx`.
template <int NT, int EPI, int DW, bool F16, bool SW4, bool PK, bool FP4, int NF, int SG>
__device__ __forceinline__ void skinny_body(const GemmArgs& a, const int by, const int bx)
{
    constexpr int kNF = NF;
    static_assert(SG == 128 || SG == 64 || SG == 32, "activation block of 128, 64 or 32 K");
    constexpr int ASPG = EPI == EPI_F32 ? 128 / SG : 1;       // A-side scale blocks per group
    constexpr int OSPG = EPI == EPI_SWIGLU_Q ? 128 / SG : 1;  // requant blocks per 128 i
    static_assert(EPI != EPI_SWIGLU_Q || NF == 4, "the SwiGLU tile pairs 2 gate and 2 up fragments");
    static_assert(!FP4 || PK, "fp4 weights are read in the prepacked layout only");
    constexpr int BM = 16 * NT;
    extern __shared__ float4 lds_side4[];  // [G * ASPG][BM] float2 {c1, c0}, 16-byte aligned
    float2* lds_side = (float2*)lds_side4;
    __shared__ float s_red[kWaves][BM];
    __shared__ float s_red2[kWaves][BM];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[EPI == EPI_SWIGLU_Q ? BM * kGroup : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, q = lane >> 4, c16 = lane & 15;
    const int64_t K = a.K, N = a.N;
    const int G = (int)(K / kGroup);

    int e, row0, rows;
    if (a.offsets != nullptr) {
        if (by >= *a.num_blocks)
            return;
        e = a.block_expert[by];
        row0 = a.block_row[by];
        rows = min(BM, a.offsets[e + 1] - row0);
    } else {
        e = 0;
        row0 = by * BM;
        if (row0 >= a.dense_rows)
            return;
        rows = min(BM, a.dense_rows - row0);
    }
    auto act_row = [&](int i) {  // activation row of block row i (padding rows reuse row 0)
        const int ii = i < rows ? i : 0;
        return a.sorted != nullptr ? a.sorted[row0 + ii] / a.topk : row0 + ii;
    };

    // weight rows of this lane (one per fragment)
    int64_t nrow[kNF];
    bool nvalid[kNF];
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
        int64_t n;
        if (EPI == EPI_SWIGLU_Q)
            n = (f >= 2 ? a.I : 0) + (int64_t)bx * kGroup + 32 * wave + 16 * (f & 1) + c16;
        else
            n = (int64_t)bx * (64 * NF) + 16 * NF * wave + 16 * f + c16;
        nvalid[f] = n < N;
        nrow[f] = nvalid[f] ? n : N - 1;
    }
    // Streaming loads go through buffer resources: a per-lane 32-bit offset
    // (row and quarter) and the per-group advance in a scalar offset.  The
    // activation operand is fp8 on both paths (one byte per element); the
    // lane's two 16-byte chunks of a group are q and 4+q (fp8_group_pos).
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w + (int64_t)e * a.w_estride, (uint32_t)(N * (K / 2)));
    const int64_t PG4 = packed_groups4(G);  // 4-group scale blocks per row (prepacked)
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(a.ws + (int64_t)e * a.s_estride, (uint32_t)(PK ? N * PG4 * 16 : N * G * 4));
    uint32_t vw[kNF], vs[kNF];
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
        // (prepacked: the rows of a fragment are 16-aligned, nrow % 16 == c16
        // except for clamped rows, which read a valid row of no consequence)
        vw[f] = PK ? (uint32_t)(((nrow[f] >> 4) * G * 16 + (nrow[f] & 15)) * 64 + 16 * q)
                   : (uint32_t)(nrow[f] * (K / 2) + 16 * q);
        vs[f] = PK ? (uint32_t)(((nrow[f] >> 4) * PG4 * 16 + (nrow[f] & 15)) * 16)
                   : (uint32_t)(nrow[f] * G * 4);
    }
    // Activation rows of a group (BM x 128 bytes), two ways:
    //  * SHARED: loaded once per workgroup straight into LDS (kAPer loads of
    //    kALane bytes per lane and wave) and read from there by all four
    //    waves.  Byte b of a buffer is byte b % 16 of slot b / 16, and slot s
    //    holds chunk (s % 8) ^ (row % 8) of row s / 8 (the XOR keeps the
    //    readers' 16-byte reads on distinct banks); a ring of DW + 1 buffers,
    //    one per group in flight plus the one being read, and a workgroup
    //    barrier per group.
    //  * otherwise every wave loads all BM rows into its registers through
    //    the ring, 2 x 16 bytes per lane and row slice.
    // Sharing cuts the L2-to-CU traffic of the activations by 4x; the barrier
    // makes the waves run in step.  Measured per fused call (32 of 256
    // experts, top-8): the 16-row down GEMM 45.7 -> 43.0 us, 128 tokens
    // (32-row blocks) 180.7 -> 172.3 us; the 16-row gate_up GEMM (heavier
    // per group, two waves per SIMD) 86.1 -> 88.6 us and 64-row blocks (one
    // wave per SIMD) 231 -> 249 us at 256 tokens lose, so they keep the
    // per-wave loads.
    constexpr bool SHARED = NT == 2 || (NT == 1 && EPI == EPI_F32);
    constexpr int kABytes = BM * kGroup;
    constexpr int kALane = kABytes >= 16 * 64 * kWaves ? 16 : 4;  // bytes per lane per load
    constexpr int kAPer = SHARED ? kABytes / (kALane * 64 * kWaves) : 0;  // loads per wave per group
    static_assert(!SHARED || kAPer * kALane * 64 * kWaves == kABytes, "the waves cover the rows exactly");
    constexpr int kABuf = DW + 1;
    __shared__ __attribute__((aligned(16))) uint8_t s_act[SHARED ? kABuf * kABytes : 16];
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // M0 operands must be wave-uniform
    const v4i ras = sgpr_rsrc(a.act, (uint32_t)(a.act_rows * K));
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.act, (uint32_t)(a.act_rows * K));
    const uint32_t s_act_lds = (uint32_t)(uintptr_t)(lds_ptr_t)s_act;
    uint32_t va[SHARED ? kAPer : NT];
    if constexpr (SHARED) {
#pragma unroll
        for (int j = 0; j < kAPer; ++j) {
            const int b = (wave + kWaves * j) * 64 * kALane + kALane * lane;  // LDS byte of the lane
            const int sl = b >> 4, row = sl >> 3;
            va[j] = (uint32_t)((int64_t)act_row(row) * K + 16 * ((sl & 7) ^ (row & 7)) + (b & 15));
        }
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            va[t] = (uint32_t)((int64_t)act_row(16 * t + c16) * K + 16 * q);
    }

    // Side data of the block's rows for every group, staged in LDS: its loads
    // are issued first, the ring's behind them, so waiting for the side data
    // does not wait for the ring.
    constexpr int kSidePer = 8;  // side loads per thread held in registers
    float2 side_v[kSidePer];
    const int nside = G * ASPG * BM;
    const bool side_in_regs = nside <= 256 * kSidePer;
    auto side_of = [&](int i) {
        const int gb = i / BM, c = i - gb * BM;
        return c < rows ? a.act_side[(int64_t)act_row(c) * (G * ASPG) + gb] : make_float2(0.0f, 0.0f);
    };
    if (side_in_regs) {
#pragma unroll
        for (int j = 0; j < kSidePer; ++j) {
            const int i = tid + 256 * j;
            if (i < nside)
                side_v[j] = side_of(i);
        }
    }

    // STAGED (16-row blocks of the down and dense GEMMs whose rows fit the
    // stage capacity the launch set aside; at decode a block holds 1-6 real
    // rows): the block's activation rows over the whole K are loaded once,
    // straight into LDS, before the ring starts, and every group reads them
    // from there: no activation loads and no barriers inside the K loop.  Row
    // stride K + 16 bytes, so the 16 rows' reads of one column spread over the
    // banks.  Other blocks take the loop below with the rows shared per group;
    // the choice is per workgroup and the two K loops are separate instances.
    // Measured per fused call (32 of 256 experts, 64 tokens, median of 7
    // interleaved runs): down 42.4 -> 40.9 us; the same for the 16-row gate_up
    // (K = 7168, 9 rows of capacity) measured 80.2 -> 81.0 us and is not used.
    constexpr bool kStage = NT == 1 && SG == 128 && EPI != EPI_SWIGLU_Q;
    const bool staged = kStage && rows <= a.stage_rows;
    const int64_t KS = K + 16;
    uint8_t* const stage = (uint8_t*)lds_side4 + ((int64_t)nside * 8 + 15) / 16 * 16;
    if (kStage && staged) {
        const uint32_t st_lds = (uint32_t)(uintptr_t)(lds_ptr_t)stage;
        const int per_row = (int)(K / 1024);  // 1 KB pieces (K % 1024 == 0 when stage_rows > 0)
        const int npieces = rows * per_row;
        for (int p = wave_s; p < npieces; p += kWaves) {
            const int r = p / per_row, j = p - r * per_row;
            lds_load16(ras, st_lds + (uint32_t)(r * KS + j * 1024), (uint32_t)(16 * lane),
                       (uint32_t)((int64_t)act_row(r) * K + j * 1024));
        }
    }

    // Promotion in fp32 on both paths.  On the f16 (gate_up) path each group's
    // MFMA sum is the correctly rounded fp32 value of an exact dot product, so
    // y carries only the fp32 roundings of the running sum, and the SwiGLU +
    // fp8 requant that follows lands on another code than the exact result's
    // for a few in 10^5 elements.  (An fp64 running sum removes even those,
    // at a VALU cost this HBM-bound kernel shows in its time.)
    float acc[kNF][NT][4];
#pragma unroll
    for (int f = 0; f < kNF; ++f)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[f][t][r] = 0;

    // Weight bytes are read once per m-block and go through the caches with
    // the non-temporal policy, which leaves L2 to the activations, scales and
    // side data that every workgroup of the expert re-reads (measured per
    // fused call, 32 of 256 experts: 64 tokens 137.9 -> 129.0 us, 128 tokens
    // 167.8 -> 159.1 us; the same policy on the weight scales measured
    // slower at 128 tokens).
    //
    // One ring of DW groups in flight for the weights and activations of a
    // group.  Vector-memory loads retire in issue order, so loads consumed at
    // different distances would make the nearest one drain the rest; the ring
    // keeps one common distance.  The loop runs over whole turns without
    // branches: a refill past the last group reloads group G-1 (never used)
    // and a padding group gets weight scale 0.
    //
    // Weight scales: with SW4 (G % 4 == 0) one float4 per fragment carries a
    // block of 4 groups, a quarter of the memory instructions of one float per
    // group.  The next block's float4 is issued at the first group of a block,
    // before that group's ring refill, so it retires no later than the
    // weights it is consumed with; the banks swap at the block boundary.  The
    // loop is unrolled over U = 4 groups (DW divides 4) so that slots and
    // lanes of the float4 are static.  Otherwise one float per group rides in
    // the ring slot.
    static_assert(!SW4 || 4 % DW == 0, "float4 scales need DW to divide 4");
    constexpr int U = SW4 ? 4 : DW;
    // (always_inline: not inlined, the lambda took the fp4 down instance from
    // 100 to 156 VGPRs)
    auto k_loop = [&](auto staged_tag) __attribute__((always_inline)) {
    constexpr bool ST = decltype(staged_tag)::value;
    v4i wb[DW][kNF];
    float sb[SW4 ? 1 : DW][kNF];
    float4 sc4[SW4 ? kNF : 1], sn4[SW4 ? kNF : 1];
    v4i ab[SHARED || ST ? 1 : DW][NT][2];
    // SHARED: the loads issued after a group's activation chunks up to its
    // consumption (the count of the explicit wait before the group's
    // barrier): the group's weight (and scale) loads, the DW - 1 groups
    // behind it and, in the first DW groups of a turn of U, the next scale
    // block issued at the turn's start.  The direct-to-LDS loads are inline
    // assembly the compiler does not count, so its own waits for the weights
    // only ever wait longer than needed.
    constexpr int kWLoads = SW4 ? kNF : 2 * kNF;
    constexpr int kAfter = kWLoads + (DW - 1) * (kAPer + kWLoads);
    auto load_group = [&](int s, int g, int buf) {
        if constexpr (SHARED && !ST) {
            // activation chunks first, so that the wait for them has the same
            // count on every group
#pragma unroll
            for (int j = 0; j < kAPer; ++j) {
                const uint32_t d = s_act_lds + (uint32_t)(buf * kABytes + (wave_s + kWaves * j) * 64 * kALane);
                if (kALane == 16)
                    lds_load16(ras, d, va[j], (uint32_t)g * kGroup);
                else
                    lds_load4(ras, d, va[j], (uint32_t)g * kGroup);
            }
        }
#pragma unroll
        for (int f = 0; f < kNF; ++f) {
            // prepacked: a group's 1 KB per fragment is contiguous, streamed
            // with the non-temporal policy; canonical rows: each lane's 16 B
            // lies in a 128-byte line shared with the next group, which
            // default loads keep in L2 for it (decode 187.7 -> 172.3 us per call)
            wb[s][f] = PK ? bload16_nt(rw, vw[f], (uint32_t)g * 1024u) : bload16(rw, vw[f], (uint32_t)g * 64u);
            if (!SW4)
                sb[s][f] = bload4f(rs, vs[f], PK ? (uint32_t)(g >> 2) * 256u + (uint32_t)(g & 3) * 4u
                                                  : (uint32_t)g * 4u);
        }
        if constexpr (!SHARED && !ST) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int v = 0; v < 2; ++v)
                    ab[s][t][v] = bload16(ra, va[t], (uint32_t)g * kGroup + 64u * v);
        }
    };
    auto load_scales4 = [&](float4 (&dst)[SW4 ? kNF : 1], int blk) {  // groups 4blk..4blk+3
        if (SW4) {
#pragma unroll
            for (int f = 0; f < kNF; ++f)
                dst[f] = __builtin_bit_cast(float4, bload16(rs, vs[f], (uint32_t)blk * (PK ? 256u : 16u)));
        }
    };
    __builtin_amdgcn_sched_barrier(0);
    load_scales4(sc4, 0);
#pragma unroll
    for (int s = 0; s < DW; ++s)
        load_group(s, s < G ? s : G - 1, s);
    __builtin_amdgcn_sched_barrier(0);

    if (side_in_regs) {
#pragma unroll
        for (int j = 0; j < kSidePer; ++j) {
            const int i = tid + 256 * j;
            if (i < nside)
                lds_side[i] = side_v[j];
        }
    } else {
        for (int i = tid; i < nside; i += 256)
            lds_side[i] = side_of(i);
    }
    // STAGED: the rows have landed (loads after them: the first scale block
    // and the ring); the barrier below publishes them
    if constexpr (ST)
        wait_vmcnt<(SW4 ? kNF : 0) + DW * kWLoads>();
    __syncthreads();

    const int G4 = G / 4;
    const int Gr = (G + U - 1) / U * U;
    for (int g0 = 0; g0 < Gr; g0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u;
            const int s = u % DW;  // ring slot
            const int gl = g < G ? g : G - 1;  // side data row (padding groups: any valid one)
            if (SW4 && u == 0) {
                // next block's scales, ahead of this turn's refills (the last
                // block reloads itself; never used)
                __builtin_amdgcn_sched_barrier(0);
                load_scales4(sn4, g0 / 4 + 1 < G4 ? g0 / 4 + 1 : G4 - 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            // SHARED: group g's activation chunks have landed in LDS (each wave
            // waits for its own; the barrier publishes them and orders every
            // wave's reads of group g - 1, whose buffer the refill below
            // overwrites, before that refill)
            const uint8_t* sa = s_act + (g % kABuf) * kABytes;
            if constexpr (ST)  // keep each group's LDS reads in its group (no hoisting across groups)
                asm volatile("" ::: "memory");
            if constexpr (SHARED && !ST) {
                __builtin_amdgcn_sched_barrier(0);
                if (SW4 && u < DW)
                    wait_vmcnt<kAfter + (SW4 ? kNF : 0)>();
                else
                    wait_vmcnt<kAfter>();
                barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
            auto act16 = [&](int t, int v) {  // the lane's chunk 4v + q of row 16t + c16
                if constexpr (ST)  // (padding rows read row 0)
                    return *(const v4i*)(stage + (16 * t + c16 < rows ? 16 * t + c16 : 0) * KS +
                                         (int64_t)gl * kGroup + 16 * (4 * v + q));
                else if constexpr (SHARED)
                    return *(const v4i*)(sa + 16 * ((16 * t + c16) * 8 + ((4 * v + q) ^ (c16 & 7))));
                else
                    return ab[s][t][v];
            };
            // int4: the weight scale (0 on padding groups); fp4: the bits of
            // the group's UE8M0 dword
            float swf[kNF];
#pragma unroll
            for (int f = 0; f < kNF; ++f) {
                float v;
                if (SW4) {
                    const float4 v4 = sc4[f];
                    v = u == 0 ? v4.x : u == 1 ? v4.y : u == 2 ? v4.z : v4.w;
                } else {
                    v = sb[s][f];
                }
                swf[f] = (FP4 || g < G) ? v : 0.0f;
            }
            if constexpr (F16 && NT == 2) {
                // two slices: 32-K step outer, slices inner, so that each
                // step's weight fragments are converted once for both slices
                // and only one step's f16 fragments are live (with the ring of
                // 2 groups this instance fits two waves per SIMD; for four
                // slices the per-slice order below measured faster)
                float conv[kNF], wsc[kNF];
                if (FP4) {
#pragma unroll
                    for (int f = 0; f < kNF; ++f) {
                        const Fp4GroupScale fs = fp4_group_scale(__builtin_bit_cast(uint32_t, swf[f]), q);
                        conv[f] = fs.conv;
                        wsc[f] = g < G ? fs.promote : 0.0f;
                    }
                }
                v4f raws[NT][kNF];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    v8h bc[kNF];
#pragma unroll
                    for (int f = 0; f < kNF; ++f) {
                        const uint32_t x = (uint32_t)wb[s][f][c];
                        bc[f] = FP4 ? fp4x8_to_f16(x, conv[f])
                                    : fp8x8_to_f16(xor_and_or<0x08080808u, 0x0F0F0F0Fu, 0u>(x),
                                                   xor_and_or<0x08080808u, 0x0F0F0F0Fu, 0u>(x >> 4));
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        if (t > 0 && 16 * t >= rows)
                            continue;
                        const v4i ac = act16(t, c >> 1);
                        const v8h ah = fp8x8_to_f16((uint32_t)ac[2 * (c & 1)], (uint32_t)ac[2 * (c & 1) + 1]);
#pragma unroll
                        for (int f = 0; f < kNF; ++f)
                            raws[t][f] = mfma16x16x32_f16(ah, bc[f], c == 0 ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : raws[t][f]);
                    }
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if (t > 0 && 16 * t >= rows)
                        continue;
                    const float4* sd = (const float4*)&lds_side[gl * BM + 16 * t + 4 * q];
                    const float4 s01 = sd[0], s23 = sd[1];
                    const float c1[4] = {s01.x, s01.z, s23.x, s23.z};
                    const float c0[4] = {s01.y, s01.w, s23.y, s23.w};
#pragma unroll
                    for (int f = 0; f < kNF; ++f)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (FP4)  // y += 2^(e_max - 136) * (raw * 512 sa)
                                acc[f][t][r] = fmaf(raws[t][f][r] * c1[r], wsc[f], acc[f][t][r]);
                            else
                                acc[f][t][r] = fmaf(swf[f], fmaf(raws[t][f][r], c1[r], c0[r]), acc[f][t][r]);
                        }
                }
            } else
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                // 16-row slices past the block's last row: nothing to compute
                // (slice 0 always holds a row)
                if (t > 0 && 16 * t >= rows)
                    continue;
                const float4* sd = (const float4*)&lds_side[gl * BM + 16 * t + 4 * q];
                const float4 s01 = sd[0], s23 = sd[1];
                const float c1[4] = {s01.x, s01.z, s23.x, s23.z};
                const float c0[4] = {s01.y, s01.w, s23.y, s23.w};
                uint32_t at[8];
                const v4i a0 = act16(t, 0), a1 = act16(t, 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    at[i] = (uint32_t)a0[i];
                    at[4 + i] = (uint32_t)a1[i];
                }
                // all MFMAs of the step first, each fragment into its own
                // accumulator, so they issue back to back; then the promotion
                v4f raw[kNF];
                float wsc[kNF];  // fp4 gate_up: promotion scale 2^(e_max - 136), 0 on padding groups
                if (F16 && FP4) {
                    v8h ah[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        ah[c] = fp8x8_to_f16(at[2 * c], at[2 * c + 1]);
                    float conv[kNF];
#pragma unroll
                    for (int f = 0; f < kNF; ++f) {
                        const Fp4GroupScale fs = fp4_group_scale(__builtin_bit_cast(uint32_t, swf[f]), q);
                        conv[f] = fs.conv;
                        wsc[f] = g < G ? fs.promote : 0.0f;
                        raw[f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int f = 0; f < kNF; ++f)
                            raw[f] = mfma16x16x32_f16(ah[c], fp4x8_to_f16((uint32_t)wb[s][f][c], conv[f]), raw[f]);
                } else if (F16) {
                    // fp8 codes -> exact f16: the lane's 8-group c is dwords
                    // 2c, 2c+1 of both operands (k0,k2,k4,k6 | k1,k3,k5,k7)
                    v8h ah[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        ah[c] = fp8x8_to_f16(at[2 * c], at[2 * c + 1]);
                    v8i b8[kNF];
#pragma unroll
                    for (int f = 0; f < kNF; ++f) {
                        b8[f] = unpack_int4_u(wb[s][f]);
                        raw[f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int f = 0; f < kNF; ++f)
                            raw[f] = mfma16x16x32_f16(
                                ah[c], fp8x8_to_f16((uint32_t)b8[f][2 * c], (uint32_t)b8[f][2 * c + 1]), raw[f]);
                } else if (ASPG > 1) {
                    // finer activation scales: one masked MFMA per SG-block of
                    // the group, each promoted with its own {c1, c0}.  The
                    // lane's A dwords hold K (real order) of one 32-block q
                    // (int4 operand order) or of [16q, 16q+16) and
                    // [64+16q, 64+16q+16) (fp4, natural order).
                    v8i b8[kNF];
                    int eq[kNF];
#pragma unroll
                    for (int f = 0; f < kNF; ++f) {
                        if (FP4)
                            eq[f] = (int)((__builtin_bit_cast(uint32_t, swf[f]) >> (8 * q)) & 0xFFu);
                        else
                            b8[f] = unpack_int4_u(wb[s][f]);
                    }
#pragma unroll
                    for (int b = 0; b < ASPG; ++b) {
                        const float4* sdb = (const float4*)&lds_side[(gl * ASPG + b) * BM + 16 * t + 4 * q];
                        const float4 b01 = sdb[0], b23 = sdb[1];
                        const float c1b[4] = {b01.x, b01.z, b23.x, b23.z};
                        const float c0b[4] = {b01.y, b01.w, b23.y, b23.w};
                        v8i av;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int kb = FP4 ? (i < 4 ? 16 * q : 64 + 16 * q) : 32 * q;
                            av[i] = kb / SG == b ? (int)at[i] : 0;
                        }
#pragma unroll
                        for (int f = 0; f < kNF; ++f) {
                            const v4f rb = FP4 ? mfma16x16x128_fp4(av, wb[s][f], eq[f])
                                               : mfma16x16x128(av, b8[f], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                if (FP4)
                                    acc[f][t][r] = fmaf(rb[r], g < G ? c1b[r] * 0x1p-9f : 0.0f, acc[f][t][r]);
                                else
                                    acc[f][t][r] = fmaf(swf[f], fmaf(rb[r], c1b[r], c0b[r]), acc[f][t][r]);
                            }
                        }
                    }
                    continue;
                } else {
                    v8i av;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        av[i] = (int)at[i];
#pragma unroll
                    for (int f = 0; f < kNF; ++f)
                        raw[f] = FP4 ? mfma16x16x128_fp4(av, wb[s][f],
                                                         (int)((__builtin_bit_cast(uint32_t, swf[f]) >> (8 * q)) & 0xFFu))
                                     : mfma16x16x128(av, unpack_int4_u(wb[s][f]), v4f{0.0f, 0.0f, 0.0f, 0.0f});
                }
                if (FP4 && F16) {
                    // y += 2^(e_max - 136) * (raw * 512 sa)
#pragma unroll
                    for (int f = 0; f < kNF; ++f)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[f][t][r] = fmaf(raw[f][r] * c1[r], wsc[f], acc[f][t][r]);
                } else if (FP4) {
                    // the weight scales are inside raw: y += sa * raw, sa = c1 * 2^-9
                    float sa[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sa[r] = g < G ? c1[r] * 0x1p-9f : 0.0f;
#pragma unroll
                    for (int f = 0; f < kNF; ++f)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[f][t][r] = fmaf(raw[f][r], sa[r], acc[f][t][r]);
                } else {
#pragma unroll
                    for (int f = 0; f < kNF; ++f)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[f][t][r] = fmaf(swf[f], fmaf(raw[f][r], c1[r], c0[r]), acc[f][t][r]);
                }
            }
            // keep the refill here, DW groups ahead of its use: without the
            // barrier the scheduler sinks each load next to its consumer and
            // only one load stays in flight
            __builtin_amdgcn_sched_barrier(0);
            load_group(s, g + DW < G ? g + DW : G - 1, (g + DW) % kABuf);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (SW4) {
#pragma unroll
            for (int f = 0; f < kNF; ++f)
                sc4[f] = sn4[f];
        }
    }
    // the last turns' refills (never read) land before the block's LDS is freed
    if constexpr (SHARED && !ST)
        wait_vmcnt<0>();
    };
    if constexpr (kStage) {
        if (staged)
            k_loop(std::true_type{});
        else
            k_loop(std::false_type{});
    } else {
        k_loop(std::false_type{});
    }

    // ---- epilogues ----  output element (row 16t+4q+r of the block, weight row nrow[f])
    if (EPI == EPI_F32) {
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
                        a.out_f32[(int64_t)(row0 + row) * N + nrow[f]] = acc[f][t][r];
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
        // a static requant scale (per tensor) replaces each row's amax / 448.
        // The requant blocks are SG i's: waves [ob*SG/32, (ob+1)*SG/32) of
        // block ob (a wave's 32 i's never straddle two blocks).
        const float* fixed = a.requant_scale;
        constexpr int kWB = SG / 32;  // waves per requant block
        auto block_amax = [&](int ob, int row) {
            float m = s_red[ob * kWB][row];
#pragma unroll
            for (int w = 1; w < kWB; ++w)
                m = fmaxf(m, s_red[ob * kWB + w][row]);
            return m;
        };
        auto block_sum = [&](int ob, int row) {
            float sm = s_red2[ob * kWB][row];
#pragma unroll
            for (int w = 1; w < kWB; ++w)
                sm += s_red2[ob * kWB + w][row];
            return sm;
        };
        float inv[NT][4], scl[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * t + 4 * q + r;
                const float amax_c = clamp_amax(block_amax(wave / kWB, row));
                inv[t][r] = fixed ? recip_static(*fixed) : recip448(amax_c);
                scl[t][r] = fixed ? *fixed : scale_of(amax_c);
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
                    // int4 down GEMM: the interleaved operand order; fp4: natural K order
                    const int il = 32 * wave + 16 * j + c16;
                    const int b = il & 7;
                    const int pos = FP4 ? il : fp8_group_pos(il >> 3) + ((b & 1) ? 4 + (b >> 1) : (b >> 1));
                    s_q[row * kGroup + pos] = (uint8_t)((cc >> (8 * j)) & 0xFFu);
                }
            }
        __syncthreads();
        const int64_t GI = a.I / SG;  // requant blocks per row
        for (int i = tid; i < BM * 8; i += 256) {
            const int row = i >> 3, chunk = i & 7;
            if (row < rows) {
                const int64_t p = row0 + row;
                *(v4i*)(a.out_q + p * a.I + (int64_t)bx * kGroup + chunk * 16) =
                    *(const v4i*)(s_q + row * kGroup + chunk * 16);
            }
        }
        for (int i = tid; i < BM * OSPG; i += 256) {
            const int row = i / OSPG, ob = i - row * OSPG;
            if (row < rows) {
                const float sum = block_sum(ob, row);
                const float sc = fixed ? *fixed : scale_of(clamp_amax(block_amax(ob, row)));
                a.out_side[(int64_t)(row0 + row) * GI + (int64_t)bx * OSPG + ob] =
                    make_float2(512.0f * sc, -8.0f * (sc * sum));
            }
        }
    }
}

template <int NT, int EPI, int DW, bool F16, bool SW4, bool PK, bool FP4, int NF, int SG>
__global__ __launch_bounds__(256, NT == 2 ? 2 : 1) void gemm_skinny_kernel(GemmArgs a)
{
    if (path_not_taken(a))
        return;
    skinny_body<NT, EPI, DW, F16, SW4, PK, FP4, NF, SG>(a, (int)blockIdx.y, (int)blockIdx.x);
}

// Two m-block lists in one launch (per-expert block heights): grid.y rows
// [0, nb2) run list a2's 32-row blocks, the rest list a1's 16-row blocks
// (workgroups are dispatched in grid order, so the longer ones start first
// and the short ones fill in around them); each list has its own
// weight-block count along grid.x (gx1, gx2).  Two waves per SIMD, as each
// instance alone.
template <int EPI, bool F16, bool SW4, bool PK, bool FP4, int NF1, int NF2>
__global__ __launch_bounds__(256, 2) void gemm_skinny_two_lists_kernel(GemmArgs a1, GemmArgs a2, int nb2,
                                                                       int gx1, int gx2)
{
    if (path_not_taken(a1))
        return;
    const int by = (int)blockIdx.y, bx = (int)blockIdx.x;
    if (by < nb2) {
        if (bx < gx2)
            skinny_body<2, EPI, 2, F16, false, PK, FP4, NF2, 128>(a2, by, bx);
    } else if (bx < gx1) {
        skinny_body<1, EPI, kDW16, F16, SW4, PK, FP4, NF1, 128>(a1, by - nb2, bx);
    }
}

// Dynamic LDS of one workgroup (side data of the block's rows for every
// group; for 16-row down blocks also the whole-K activation rows of up to
// a.stage_rows rows, which this sets).
template <int NT, int EPI, int DW, int SG>
static size_t skinny_lds(GemmArgs& a)
{
    const int64_t G = a.K / kGroup;
    const size_t side = (size_t)G * (EPI == EPI_F32 ? 128 / SG : 1) * 16 * NT * sizeof(float2);
    // 16-row blocks of the down GEMM: LDS for the whole-K activation rows of
    // up to stage_rows rows (1 KB pieces, so K % 1024 == 0), within a quarter
    // of the CU's LDS (the down instance runs four workgroups per CU) less
    // the side data, the shared-rows ring of the fallback loop (static LDS)
    // and 4 KB of other static LDS
    a.stage_rows = 0;
    if (NT == 1 && SG == 128 && EPI != EPI_SWIGLU_Q && a.K % 1024 == 0) {
        const int64_t ring = EPI == EPI_F32 ? (DW + 1) * 16 * kGroup : 0;
        const int64_t share = 160 * 1024 / 4 - 4096 - (int64_t)side - ring;
        const int64_t r = share / (a.K + 16);
        a.stage_rows = (int32_t)(r < 16 ? (r > 0 ? r : 0) : 16);
    }
    return side + (a.stage_rows > 0 ? 16 + (size_t)a.stage_rows * (size_t)(a.K + 16) : 0);
}

template <int NT, int EPI, int DW, bool F16, bool SW4, bool PK, bool FP4, int NF = 4, int SG = 128>
static hipError_t launch_one(const GemmArgs& a0, hipStream_t s)
{
    GemmArgs a = a0;
    const size_t lds = skinny_lds<NT, EPI, DW, SG>(a);
    dim3 grid;
    if (EPI == EPI_SWIGLU_Q)
        grid.x = (unsigned)(a.I / kGroup);
    else
        grid.x = (unsigned)((a.N + 64 * NF - 1) / (64 * NF));
    grid.y = (unsigned)a.max_blocks;
    grid.z = 1;
    if (grid.x == 0 || grid.y == 0)
        return hipSuccess;
    hipLaunchKernelGGL((gemm_skinny_kernel<NT, EPI, DW, F16, SW4, PK, FP4, NF, SG>), grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

// gate_up (SwiGLU epilogue) runs on the exact f16 path, the others on fp8;
// ring depth per m-block height.  The down GEMM of 16-row m-blocks takes
// 128 weight rows per workgroup: its K is short, so a workgroup lives briefly,
// and twice as many smaller ones leave less of the machine idle in the last
// round of workgroups.  32-row m-blocks run two waves per SIMD: a ring of 2
// groups and one scale load per group (the float4 scale blocks would not fit
// the register budget); measured against one wave per SIMD with a ring of 3,
// 128 tokens on 32 of 256 experts: 202 -> 181 us per fused call.
template <int NT, int DW, bool PK, bool FP4, int SG>
static hipError_t launch_nt(const GemmArgs& a, int epilogue, hipStream_t s)
{
    const bool g4 = (a.K / kGroup) % 4 == 0;
    constexpr int NFD = NT == 1 ? kDownNF16 : 4;
    switch (epilogue) {
    case EPI_F32:
        return g4 && NT != 2 ? launch_one<NT, EPI_F32, DW, false, 4 % DW == 0, PK, FP4, NFD, SG>(a, s)
                  : launch_one<NT, EPI_F32, DW, false, false, PK, FP4, NFD, SG>(a, s);
    default:
        return g4 && NT != 2 ? launch_one<NT, EPI_SWIGLU_Q, DW, true, 4 % DW == 0, PK, FP4, 4, SG>(a, s)
                  : launch_one<NT, EPI_SWIGLU_Q, DW, true, false, PK, FP4, 4, SG>(a, s);
    }
}

// the finer activation recipes (sub_group 64 or 32) run on prepacked weights
template <int NT, int DW, bool FP4>
static hipError_t launch_packed(const GemmArgs& a, int epilogue, hipStream_t s)
{
    switch (a.sub_group) {
    case 128: return launch_nt<NT, DW, true, FP4, 128>(a, epilogue, s);
    case 64: return launch_nt<NT, DW, true, FP4, 64>(a, epilogue, s);
    case 32: return launch_nt<NT, DW, true, FP4, 32>(a, epilogue, s);
    default: return hipErrorInvalidValue;
    }
}

template <int NT, int DW>
static hipError_t launch_layout(const GemmArgs& a, int epilogue, hipStream_t s)
{
    if (a.packed)
        return a.fp4 ? launch_packed<NT, DW, true>(a, epilogue, s) : launch_packed<NT, DW, false>(a, epilogue, s);
    if (a.fp4 || a.sub_group != 128)
        return hipErrorInvalidValue;
    return launch_nt<NT, DW, false, false, 128>(a, epilogue, s);
}

hipError_t launch_gemm_skinny(const GemmArgs& a, int epilogue, int block_m, hipStream_t s)
{
    if (block_m <= 16)
        return launch_layout<1, kDW16>(a, epilogue, s);
    if (block_m <= 32)
        return launch_layout<2, 2>(a, epilogue, s);
    return launch_layout<4, 2>(a, epilogue, s);
}

template <int EPI, bool PK, bool FP4, bool SW4>
static hipError_t launch_two_lists_t(const GemmArgs& a10, const GemmArgs& a20, hipStream_t s)
{
    constexpr bool F16 = EPI == EPI_SWIGLU_Q;
    constexpr int NF1 = EPI == EPI_F32 ? kDownNF16 : 4;
    GemmArgs a1 = a10, a2 = a20;
    const size_t l1 = skinny_lds<1, EPI, kDW16, 128>(a1);
    const size_t l2 = skinny_lds<2, EPI, 2, 128>(a2);
    const int gx1 = EPI == EPI_SWIGLU_Q ? (int)(a1.I / kGroup) : (int)((a1.N + 64 * NF1 - 1) / (64 * NF1));
    const int gx2 = EPI == EPI_SWIGLU_Q ? (int)(a2.I / kGroup) : (int)((a2.N + 255) / 256);
    const dim3 grid((unsigned)(gx1 > gx2 ? gx1 : gx2), (unsigned)(a1.max_blocks + a2.max_blocks));
    if (grid.x == 0 || grid.y == 0)
        return hipSuccess;
    hipLaunchKernelGGL((gemm_skinny_two_lists_kernel<EPI, F16, SW4, PK, FP4, NF1, 4>), grid, dim3(256),
                       l1 > l2 ? l1 : l2, s, a1, a2, (int)a2.max_blocks, gx1, gx2);
    return hipGetLastError();
}

template <int EPI, bool PK, bool FP4>
static hipError_t launch_two_lists_e(const GemmArgs& a1, const GemmArgs& a2, hipStream_t s)
{
    // float4 scale blocks for the 16-row instance when G % 4 == 0 (as launch_nt)
    if ((a1.K / kGroup) % 4 == 0 && 4 % kDW16 == 0)
        return launch_two_lists_t<EPI, PK, FP4, true>(a1, a2, s);
    return launch_two_lists_t<EPI, PK, FP4, false>(a1, a2, s);
}

hipError_t launch_gemm_skinny_two_lists(const GemmArgs& a1, const GemmArgs& a2, int epilogue, hipStream_t s)
{
    if (a1.sub_group != 128 || a2.sub_group != 128 || (a1.fp4 && !a1.packed))
        return hipErrorInvalidValue;
    const bool f32 = epilogue == EPI_F32;
    if (a1.fp4)
        return f32 ? launch_two_lists_e<EPI_F32, true, true>(a1, a2, s)
                   : launch_two_lists_e<EPI_SWIGLU_Q, true, true>(a1, a2, s);
    if (a1.packed)
        return f32 ? launch_two_lists_e<EPI_F32, true, false>(a1, a2, s)
                   : launch_two_lists_e<EPI_SWIGLU_Q, true, false>(a1, a2, s);
    return f32 ? launch_two_lists_e<EPI_F32, false, false>(a1, a2, s)
               : launch_two_lists_e<EPI_SWIGLU_Q, false, false>(a1, a2, s);
}

} // namespace w4a8
