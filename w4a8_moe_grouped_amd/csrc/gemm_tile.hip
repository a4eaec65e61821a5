// gemm_tile.hip -- grouped W4A8 GEMM for many rows per expert (prefill).
//
// y[p, n] = sum_g w_scale[n, g] * a_scale[p, g] * sum_{k in g} a[p, k] * w[n, k]
// over the rows p of one m-block of one expert (SGLang PR #7762: grouped
// GEMM over expert segments with 128-wide weight groups along K; DeepGEMM
// PR #53 "Changes": large batches are MMA-bound, so a block tile reuses each
// weight byte across many token rows).
//
// Work decomposition.  A workgroup of 8 waves owns a tile of 160 rows (one
// m-block) x 256 weight rows and walks K one 128-group at a time.  Waves sit
// on a 2 x 4 grid, each with an 80 x 64 register tile (5 x 4 fragments of
// 16 x 16); the two row halves go to waves 0-3 and 4-7, so that each SIMD
// holds one wave of each half.  A wave whose half holds no row of the
// m-block skips the K loop.  160 rows: with ~130 rows per local expert (a
// 4096-token batch over 256 experts, top-8) every expert's rows fit one
// m-block, where 128-row blocks leave a nearly empty second block for half of
// the experts.  For every group the workgroup copies, straight from global memory into LDS
// (buffer_load ... lds, no register staging), the 160 activation rows (fp8
// codes, gathered through the permutation), their {c1, c0} side data, the
// 256 packed int4 (or fp4) weight rows and their scales: 38 KB per stage, 4
// stages in flight.  Stage slots are XOR-swizzled so that the 16-byte
// fragment reads hit distinct LDS banks.
//
// MFMAs: the down GEMM runs on v_mfma_f32_16x16x128_f8f6f4 with the weights
// turned into u * 2^-9 fp8 codes (u = nibble ^ 8, see common.hpp); gate_up runs
// the same operands converted exactly to f16 through
// v_mfma_f32_16x16x32_f16, whose fp32 sum of each 32-wide step is exact to
// rounding (the fp8 form truncates, and the requantised SwiGLU output of
// gate_up is sensitive to that).  Either way one group's raw sum is promoted
// as y += w_scale * fma(raw, c1, c0).  With prepacked fp4 weights (FP4;
// DeepGEMM PR #53, Changes: FP4 E2M1 with per-32-K UE8M0 scales) gate_up
// converts the nibbles to f16 at the lane's relative block scale and promotes
// with 2^(e_max - 136), and the down GEMM hands them to the scaled fp8 x fp4
// MFMA with the lane's block exponent, promoting with the activation scale
// alone.
//
// Tile order: tiles are numbered expert by expert, weight block by weight
// block, m-block fastest (the m-blocks of one expert share its weight panel
// while they run), and the numbering is cut into 8 contiguous ranges, one per
// XCD (workgroups are dealt to the XCDs round robin), so that the panel and the
// activation rows of an expert stay in one XCD's L2.
//
// Epilogues:
//   TILE_DOWN    out_f32[p, n]
//   TILE_GATEUP  the tile holds gate rows i and up rows I+i of one 128-block of
//                i: h = silu(gate) * up (fp64, rounded once to fp32), then the
//                fp8 requant of the block (DeepGEMM PR #53 "Changes": SwiGLU ->
//                per-token FP8 requant).
#include <type_traits>

#include "w4a8.h"
#include "common.hpp"
#include "internal.hpp"
#include "lds_direct.hpp"


namespace w4a8 {

namespace {

constexpr int kTBM = kTileRows;    // rows per tile
constexpr int kHalf = kTBM / 2;    // rows per wave (two row halves)
constexpr int kSlices = kHalf / 16;
constexpr int kTBN = 256;          // weight rows per tile
constexpr int kTThreads = 512;
constexpr int kStages = 4;
static_assert(kHalf % 16 == 0, "row halves are whole 16-row slices");

constexpr int kAOff = 0;
constexpr int kBOff = kAOff + kTBM * kGroup;         // 20 KB of activation codes
constexpr int kSideOff = kBOff + kTBN * kGroup / 2;  // 16 KB of packed weights
constexpr int kSwOff = kSideOff + kTBM * 8;          // {c1, c0} per row
constexpr int kStageBytes = kSwOff + kTBN * 4;       // weight scale per weight row
constexpr int kSmemBytes = kStages * kStageBytes;
static_assert(kSmemBytes + 64 <= 160 * 1024, "stages exceed the LDS of a CU");

// Direct loads per stage, in 64-lane wave loads: 16-byte chunks of the
// activation rows and of the weight rows, dwords of the side data and of the
// weight scales.  Wave w issues activation loads w, w + 8, w + 16 (those
// below kALoads) and weight loads w, w + 8; waves 0-3 load the weight
// scales, waves 4-7 the side data (wave 4 also its fifth load).
constexpr int kALoads = kTBM * kGroup / 16 / 64;        // 20
constexpr int kBLoads = kTBN * kGroup / 2 / 16 / 64;    // 16
constexpr int kSideLoads = kTBM * 2 / 64;               // 5
static_assert(kALoads > 16 && kALoads <= 24 && kBLoads == 16 && kSideLoads == 5,
              "the load assignment below is written for a 160 x 256 tile");

// 16-byte slot of (activation row, chunk 0..7) and of (weight row, chunk 0..3)
__device__ __forceinline__ int a_slot(int row, int chunk)
{
    return row * 8 + (chunk ^ (row & 7));
}
__device__ __forceinline__ int b_slot(int wrow, int chunk)
{
    return wrow * 4 + (chunk ^ ((wrow >> 1) & 3));
}

}  // namespace

// One tile: rows [row0, row0 + kTBM) of m-block L's expert x weight block nb.
template <int MODE, bool PK, bool FP4>
__device__ __forceinline__ void tile_body(const GemmArgs& a, const int L, uint8_t* smem, int* s_expert_p)
{
    static_assert(!FP4 || PK, "fp4 weights are read in the prepacked layout only");
    int& s_expert = *s_expert_p;
    const int tid = threadIdx.x;
    // the wave index in an SGPR: LDS destinations of the direct loads go
    // through M0 and must be provably wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, q = lane >> 4, c16 = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t K = a.K, N = a.N;
    const int G = (int)(K / kGroup);
    const int E = a.num_experts;
    const int nbn = MODE == TILE_GATEUP ? (int)(a.I / kGroup) : (int)((N + kTBN - 1) / kTBN);

    if (tid == 0)
        s_expert = -1;
    __syncthreads();
    for (int e = tid; e < E; e += kTThreads) {
        const int b0 = a.block_start[e], b1 = a.block_start[e + 1];
        if (L >= b0 * nbn && L < b1 * nbn)  // exactly one expert owns tile L
            s_expert = e;
    }
    __syncthreads();
    const int e = __builtin_amdgcn_readfirstlane(s_expert);
    if (e < 0)
        return;
    const int bs = a.block_start[e];
    const int nbe = a.block_start[e + 1] - bs;
    if (nbe <= 0)
        return;
    const int local = L - bs * nbn;
    const int nb = local / nbe;
    const int blk = bs + (local - nb * nbe);
    const int row0 = a.block_row[blk];
    const int rows = min(kTBM, a.offsets[e + 1] - row0);

    auto act_row = [&](int i) {  // activation row of tile row i (padding rows reuse row 0)
        const int ii = i < rows ? i : 0;
        return a.sorted != nullptr ? a.sorted[row0 + ii] / a.topk : row0 + ii;
    };
    auto weight_row = [&](int wrow) -> int64_t {  // weight row of tile weight row wrow
        int64_t n;
        if (MODE == TILE_GATEUP)
            n = (wrow >= 128 ? a.I : 0) + (int64_t)nb * kGroup + (wrow & 127);
        else
            n = (int64_t)nb * kTBN + wrow;
        return n < N ? n : N - 1;
    };

    // ---- this thread's share of every stage's loads ----
    const v4i ra = sgpr_rsrc(a.act, (uint32_t)(a.act_rows * K));
    const v4i rsd = sgpr_rsrc(a.act_side, (uint32_t)(a.act_rows * G * 8));
    const v4i rw = sgpr_rsrc(a.w + (int64_t)e * a.w_estride, (uint32_t)(N * (K / 2)));
    const int64_t G4 = packed_groups4(G);
    const v4i rws = sgpr_rsrc(a.ws + (int64_t)e * a.s_estride, (uint32_t)(PK ? N * G4 * 16 : N * G * 4));
    // load L covers 16-byte slots [64 L, 64 L + 64) of its region
    uint32_t va[3] = {0u, 0u, 0u}, vb[2], vx[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int s = (wave + 8 * j) * 64 + lane;
        const int r = min(s >> 3, kTBM - 1), ca = (s & 7) ^ (r & 7);
        va[j] = (uint32_t)((int64_t)act_row(r) * K + 16 * ca);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int s = (wave + 8 * j) * 64 + lane;
        const int wr = s >> 2, cb = (s & 3) ^ ((wr >> 1) & 3);
        const int64_t n = weight_row(wr);
        vb[j] = PK ? (uint32_t)(((n >> 4) * G * 16 + (n & 15)) * 64 + 16 * cb)
                   : (uint32_t)(n * (K / 2) + 16 * cb);
    }
    if (wave < 4) {  // weight scales: one per weight row
        const int64_t n = weight_row(wave * 64 + lane);
        vx[0] = PK ? (uint32_t)(((n >> 4) * G4 * 16 + (n & 15)) * 16) : (uint32_t)(n * G * 4);
    } else {  // side data: dword d = 2 * row + component
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int d = min((wave - 4 + 4 * j) * 64 + lane, 2 * kTBM - 1);
            vx[j] = (uint32_t)(((int64_t)act_row(d >> 1) * G) * 8 + 4 * (d & 1));
        }
    }
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    auto issue = [&](int g, int st) {
        const uint32_t base = smem_lds + (uint32_t)(st * kStageBytes);
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (wave + 8 * j < kALoads)
                lds_load16(ra, base + kAOff + (uint32_t)(wave + 8 * j) * 1024u, va[j], (uint32_t)g * kGroup);
        const uint32_t gw = (uint32_t)g * (PK ? 1024u : 64u);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            lds_load16(rw, base + kBOff + (uint32_t)(wave + 8 * j) * 1024u, vb[j], gw);
        if (wave < 4) {
            lds_load4(rws, base + kSwOff + wave * 256, vx[0],
                      PK ? (uint32_t)(g >> 2) * 256u + (uint32_t)(g & 3) * 4u : (uint32_t)g * 4u);
        } else {
            lds_load4(rsd, base + kSideOff + (wave - 4) * 256, vx[0], (uint32_t)g * 8u);
            if (wave == 4)
                lds_load4(rsd, base + kSideOff + 4 * 256, vx[1], (uint32_t)g * 8u);
        }
    };
    // this wave's loads per stage: waves 0-4 issue 6, waves 5-7 issue 5
    const bool six_loads = wave <= 4;

    // weight rows of this lane's fragments (tile-local)
    int wrow_f[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
        wrow_f[f] = MODE == TILE_GATEUP ? (f >= 2 ? 128 : 0) + 32 * wn + 16 * (f & 1) + c16
                                        : 64 * wn + 16 * f + c16;

    // A wave computes the 16-row slices of its half that hold a row of the
    // m-block: the K loop and the epilogue below are instantiated for every
    // slice count and chosen once per tile (a branch per slice inside the
    // loop measured slower: it splits the MFMA/VALU schedule); a wave whose
    // half holds no row only loads and meets the barriers.  The compute also
    // stays behind a run-time test of that: without the branch the compiler
    // schedules the five-slice loop as straight-line code and spills.
    const int nsl = min(kSlices, max(0, (rows - kHalf * wm + 15) / 16));
    const bool wave_idle = nsl == 0;


    // this wave's loads of group h landed (the younger groups in flight may
    // stay so: loads retire in order)
    auto wait_group = [&](int h) {
        const int behind = min(kStages - 2, G - 1 - h);
        if (behind >= 2) {
            if (six_loads)
                wait_vmcnt<12>();
            else
                wait_vmcnt<10>();
        } else if (behind == 1) {
            if (six_loads)
                wait_vmcnt<6>();
            else
                wait_vmcnt<5>();
        } else {
            wait_vmcnt<0>();
        }
    };
    // LDS fragment reads: the weight fragments of a stage, and the activation
    // fragment + side data of one 16-row slice m
    auto read_b = [&](const uint8_t* base, v4i (&wb)[4], float (&sw)[4]) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            wb[f] = *(const v4i*)(base + kBOff + 16 * b_slot(wrow_f[f], q));
            sw[f] = *(const float*)(base + kSwOff + 4 * wrow_f[f]);
        }
    };
    auto read_a = [&](const uint8_t* base, int m, v4i& a0, v4i& a1) {
        const int trow = kHalf * wm + 16 * m;
        a0 = *(const v4i*)(base + kAOff + 16 * a_slot(trow + c16, q));
        a1 = *(const v4i*)(base + kAOff + 16 * a_slot(trow + c16, 4 + q));
    };
    // {c1, c0} of the lane's four rows 4q + r of slice m
    auto read_side = [&](const uint8_t* base, int m, float4& s01, float4& s23) {
        const float4* sd = (const float4*)(base + kSideOff + 8 * (kHalf * wm + 16 * m + 4 * q));
        s01 = sd[0];
        s23 = sd[1];
    };

    // Software pipeline.  Stages: groups g+1..g+3 are in flight while group g
    // is computed.  Registers: the operand fragments of the next slice (and,
    // across the group boundary, of the next group) are read while the
    // current one runs its MFMAs, so LDS latency hides behind them.  The side
    // data is needed only after a slice's MFMAs: gate_up (16 MFMAs per slice,
    // no registers to spare) reads it as the slice starts, the down GEMM (4
    // MFMAs per slice) with the next slice's fragments.
    constexpr bool kSidePre = MODE == TILE_DOWN;
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < G)
            issue(s, s);
    wait_group(0);
    barrier();
    if (kStages - 1 < G)
        issue(kStages - 1, kStages - 1);

    // the K loop and the epilogue of a wave that computes NSL slices
    auto kloop = [&](auto nsl_c) {
        constexpr int NSL = decltype(nsl_c)::value;
        float acc[NSL > 0 ? NSL : 1][4][4];
#pragma unroll
        for (int m = 0; m < NSL; ++m)
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[m][f][r] = 0;
        v4i wb[4], a0 = {}, a1 = {};
        float sw[4];
        float4 s01 = {}, s23 = {};  // prefetched side data (down GEMM)
        if (NSL > 0 && !wave_idle) {
            read_b(smem, wb, sw);
            read_a(smem, 0, a0, a1);
            if (kSidePre)
                read_side(smem, 0, s01, s23);
        }

        for (int g = 0; g < G; ++g) {
            const uint8_t* base = smem + (g % kStages) * kStageBytes;
            if (NSL > 0 && !wave_idle) {
                // int4: weight scales; fp4: gate_up promotion scales 2^(e_max - 136)
                float swc[4];
                int eq[4];  // fp4 down: the lane's UE8M0 byte
                v8i b8[4];
                v8h bh[MODE == TILE_GATEUP ? 4 : 1][4];
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const uint32_t sd = __builtin_bit_cast(uint32_t, sw[f]);
                    if (FP4 && MODE == TILE_GATEUP) {
                        const Fp4GroupScale fs = fp4_group_scale(sd, q);
                        swc[f] = fs.promote;
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            bh[f][c] = fp4x8_to_f16((uint32_t)wb[f][c], fs.conv);
                    } else if (FP4) {
                        eq[f] = (int)((sd >> (8 * q)) & 0xFFu);
                    } else {
                        swc[f] = sw[f];
                        b8[f] = unpack_int4_u(wb[f]);
                        if (MODE == TILE_GATEUP) {
#pragma unroll
                            for (int c = 0; c < 4; ++c)
                                bh[f][c] = fp8x8_to_f16((uint32_t)b8[f][2 * c], (uint32_t)b8[f][2 * c + 1]);
                        }
                    }
                }
                // the slices that hold rows (padding rows among them are
                // computed and dropped at the store)
#pragma unroll
                for (int m = 0; m < NSL; ++m) {
                    const v4i ca0 = a0, ca1 = a1;
                    float4 cs01 = s01, cs23 = s23;
                    if (!kSidePre)
                        read_side(base, m, cs01, cs23);
                    if (m + 1 < NSL) {
                        read_a(base, m + 1, a0, a1);
                        if (kSidePre)
                            read_side(base, m + 1, s01, s23);
                    }
                    v4f raw[4];
                    if (MODE == TILE_GATEUP) {
#pragma unroll
                        for (int f = 0; f < 4; ++f)
                            raw[f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                        // one 32-K step at a time: its converted fragment feeds
                        // the four MFMAs right away
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const v4i& src = c < 2 ? ca0 : ca1;
                            const v8h ah = fp8x8_to_f16((uint32_t)src[2 * (c & 1)], (uint32_t)src[2 * (c & 1) + 1]);
#pragma unroll
                            for (int f = 0; f < 4; ++f)
                                raw[f] = mfma16x16x32_f16(ah, bh[f][c], raw[f]);
                        }
                    } else {
                        const v8i av = {ca0[0], ca0[1], ca0[2], ca0[3], ca1[0], ca1[1], ca1[2], ca1[3]};
#pragma unroll
                        for (int f = 0; f < 4; ++f)
                            raw[f] = FP4 ? mfma16x16x128_fp4(av, wb[f], eq[f])
                                         : mfma16x16x128(av, b8[f], v4f{0.0f, 0.0f, 0.0f, 0.0f});
                    }
                    const float c1[4] = {cs01.x, cs01.z, cs23.x, cs23.z};
                    const float c0[4] = {cs01.y, cs01.w, cs23.y, cs23.w};
#pragma unroll
                    for (int f = 0; f < 4; ++f)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (FP4 && MODE == TILE_GATEUP)  // y += 2^(e_max - 136) * (raw * 512 sa)
                                acc[m][f][r] = fmaf(raw[f][r] * c1[r], swc[f], acc[m][f][r]);
                            else if (FP4)  // weight scales inside raw: y += sa * raw
                                acc[m][f][r] = fmaf(raw[f][r], c1[r] * 0x1p-9f, acc[m][f][r]);
                            else
                                acc[m][f][r] = fmaf(swc[f], fmaf(raw[f][r], c1[r], c0[r]), acc[m][f][r]);
                        }
                }
            }
            if (g + 1 < G) {
                wait_group(g + 1);
                // everyone's loads of group g+1 landed, and every wave's reads of
                // stage g are complete: refill it with group g+4
                barrier();
                if (g + kStages < G)
                    issue(g + kStages, g % kStages);
                if (NSL > 0 && !wave_idle) {
                    const uint8_t* nbase = smem + ((g + 1) % kStages) * kStageBytes;
                    read_b(nbase, wb, sw);
                    read_a(nbase, 0, a0, a1);
                    if (kSidePre)
                        read_side(nbase, 0, s01, s23);
                }
            }
        }

        // ---- epilogues: element (tile row 80wm + 16m + 4q + r, fragment f) ----
        if (MODE == TILE_DOWN) {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int64_t n = (int64_t)nb * kTBN + wrow_f[f];
                if (n >= N)
                    continue;
#pragma unroll
                for (int m = 0; m < NSL; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = kHalf * wm + 16 * m + 4 * q + r;
                        if (row < rows)
                            a.out_f32[(int64_t)(row0 + row) * N + n] = (float)acc[m][f][r];
                    }
            }
            return;
        }

        // TILE_GATEUP: fragments f and f + 2 hold gate and up of i = 32wn + 16f + c16
        barrier();  // every wave is done with the stages (no load is in flight)
        float* s_red = (float*)smem;                        // [4][kTBM] amax per wave column
        float* s_sum = s_red + 4 * kTBM;                    // [4][kTBM] sum of decoded codes
        uint8_t* s_q = (uint8_t*)(s_sum + 4 * kTBM);        // [kTBM][128] codes
        float h[NSL > 0 ? NSL : 1][2][4];
#pragma unroll
        for (int m = 0; m < NSL; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const double gt = (double)acc[m][j][r], up = (double)acc[m][j + 2][r];
                    h[m][j][r] = (float)(gt / (1.0 + exp(-gt)) * up);
                }
#pragma unroll
        for (int m = 0; m < NSL; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float mx = fmaxf(fabsf(h[m][0][r]), fabsf(h[m][1][r]));
                mx = group_max<16>(mx);
                if (c16 == 0)
                    s_red[wn * kTBM + kHalf * wm + 16 * m + 4 * q + r] = mx;
            }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < NSL; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = kHalf * wm + 16 * m + 4 * q + r;
                const float mx = fmaxf(fmaxf(s_red[row], s_red[kTBM + row]),
                                       fmaxf(s_red[2 * kTBM + row], s_red[3 * kTBM + row]));
                const float inv = a.requant_scale ? recip_static(*a.requant_scale) : recip448(clamp_amax(mx));
                const uint32_t cc = cvt_e4m3x2(h[m][0][r] * inv, h[m][1][r] * inv);
                const float2 dv = dec_e4m3x2(cc);
                const float sum = group_sum<16>(dv.x + dv.y);
                if (c16 == 0)
                    s_sum[wn * kTBM + row] = sum;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // int4 down GEMM: the interleaved operand order; fp4: natural K order
                    const int il = 32 * wn + 16 * j + c16;
                    const int b = il & 7;
                    const int pos = FP4 ? il : fp8_group_pos(il >> 3) + ((b & 1) ? 4 + (b >> 1) : (b >> 1));
                    s_q[row * kGroup + pos] = (uint8_t)((cc >> (8 * j)) & 0xFFu);
                }
            }
        __syncthreads();
        const int64_t GI = a.I / kGroup;
        for (int i = tid; i < kTBM * 8; i += kTThreads) {
            const int row = i >> 3, chunk = i & 7;
            if (row < rows)
                *(v4i*)(a.out_q + (int64_t)(row0 + row) * a.I + (int64_t)nb * kGroup + chunk * 16) =
                    *(const v4i*)(s_q + row * kGroup + chunk * 16);
        }
        if (tid < kTBM && tid < rows) {
            const int row = tid;
            const float sum = s_sum[row] + s_sum[kTBM + row] + s_sum[2 * kTBM + row] + s_sum[3 * kTBM + row];
            const float mx = fmaxf(fmaxf(s_red[row], s_red[kTBM + row]),
                                   fmaxf(s_red[2 * kTBM + row], s_red[3 * kTBM + row]));
            const float sc = a.requant_scale ? *a.requant_scale : scale_of(clamp_amax(mx));
            a.out_side[(int64_t)(row0 + row) * GI + nb] = make_float2(512.0f * sc, -8.0f * (sc * sum));
        }
    };
    static_assert(kSlices == 5, "one K-loop instance per slice count 0..5");
    switch (nsl) {
    case 0: kloop(std::integral_constant<int, 0>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    default: kloop(std::integral_constant<int, 5>{}); break;
    }
}

// Persistent: each workgroup walks the tiles of its XCD's range.
template <int MODE, bool PK, bool FP4>
__device__ __forceinline__ void tile_phase(const GemmArgs& a, uint8_t* smem, int* s_expert)
{
    const int nbn = MODE == TILE_GATEUP ? (int)(a.I / kGroup) : (int)((a.N + kTBN - 1) / kTBN);
    const int total = *a.num_blocks * nbn;
    const int per_xcd = (total + 7) >> 3;
    const int x = (int)(blockIdx.x & 7);
    const int stride = (int)(gridDim.x >> 3);
    for (int t = (int)(blockIdx.x >> 3); t < per_xcd; t += stride) {
        const int L = x * per_xcd + t;
        if (L >= total)
            break;
        tile_body<MODE, PK, FP4>(a, L, smem, s_expert);
        __syncthreads();  // the next tile's loads overwrite LDS the epilogue may still read
    }
}

template <int MODE, bool PK, bool FP4>
__global__ __launch_bounds__(kTThreads) void gemm_tile_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    __shared__ int s_expert;
    if (path_not_taken(a))
        return;
    tile_phase<MODE, PK, FP4>(a, smem, &s_expert);
}

// ---------------------------------------------------------------------------
// The down GEMM as one stream of (tile, group) stages per workgroup.
//
// Per tile the loop above pays an expert lookup, a cold start of its stage
// ring (three groups' loads before the first MFMA) and the fp32 epilogue
// before the next tile's first load (measured: ~2850 cycles per wave and
// group against ~31 us per tile on the EP8 share, ~12 us of it outside the
// main loop).  Here the ring runs on across tiles: while the last groups of
// a tile are computed, the first groups of the workgroup's next tile are
// already loading into the stages freed behind them, and the epilogue's
// stores overlap those loads.  Every tile's expert, weight block and rows
// are found once at the start (block_start and offsets copied into LDS, a
// binary search per tile), so no global load that the compiler would wait on
// sits inside the stream.
// ---------------------------------------------------------------------------
constexpr int kMaxStreamTiles = 256;

template <bool PK, bool FP4>
__device__ __forceinline__ void down_stream(const GemmArgs& a, uint8_t* smem, int4* s_meta, int nt,
                                            int first_L, int stride)
{
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, q = lane >> 4, c16 = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t K = a.K, N = a.N;
    const int G = (int)(K / kGroup);
    const int E = a.num_experts;
    const int nbn = (int)((N + kTBN - 1) / kTBN);
    const int64_t G4 = packed_groups4(G);

    // ---- the tiles' metadata: expert, weight block, first row, rows ----
    {
        int* s_bs = (int*)smem;        // [E + 1] (the stages are not in use yet)
        int* s_off = s_bs + (E + 1);   // [E + 1]
        for (int i = tid; i <= E; i += kTThreads) {
            s_bs[i] = a.block_start[i];
            s_off[i] = a.offsets[i];
        }
        __syncthreads();
        if (tid < nt) {
            const int L = first_L + tid * stride;
            int lo = 0, hi = E;  // the largest e with block_start[e] * nbn <= L owns tile L
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_bs[mid] * nbn <= L)
                    lo = mid;
                else
                    hi = mid;
            }
            const int bs = s_bs[lo], nbe = s_bs[lo + 1] - bs;
            const int local = L - bs * nbn;
            const int nb = local / nbe;
            const int row0 = s_off[lo] + (local - nb * nbe) * kTBM;  // the expert's m-blocks are consecutive
            s_meta[tid] = make_int4(lo, nb, row0, min(kTBM, s_off[lo + 1] - row0));
        }
        __syncthreads();
    }

    // ---- per-tile load addresses (as tile_body) ----
    const v4i ra = sgpr_rsrc(a.act, (uint32_t)(a.act_rows * K));
    const v4i rsd = sgpr_rsrc(a.act_side, (uint32_t)(a.act_rows * G * 8));
    struct Ctx {
        v4i rw, rws;
        uint32_t va[3], vb[2], vx[2];
        int nb, row0, rows;
    };
    auto make_ctx = [&](int k) {
        Ctx c;
        const int4 m = s_meta[k];
        const int e = __builtin_amdgcn_readfirstlane(m.x);
        c.nb = __builtin_amdgcn_readfirstlane(m.y);
        c.row0 = __builtin_amdgcn_readfirstlane(m.z);
        c.rows = __builtin_amdgcn_readfirstlane(m.w);
        c.rw = sgpr_rsrc(a.w + (int64_t)e * a.w_estride, (uint32_t)(N * (K / 2)));
        c.rws = sgpr_rsrc(a.ws + (int64_t)e * a.s_estride, (uint32_t)(PK ? N * G4 * 16 : N * G * 4));
        auto act_row = [&](int i) { return c.row0 + (i < c.rows ? i : 0); };
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int sl = (wave + 8 * j) * 64 + lane;
            const int r = min(sl >> 3, kTBM - 1), ca = (sl & 7) ^ (r & 7);
            c.va[j] = (uint32_t)((int64_t)act_row(r) * K + 16 * ca);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int sl = (wave + 8 * j) * 64 + lane;
            const int wr = sl >> 2, cb = (sl & 3) ^ ((wr >> 1) & 3);
            int64_t n = (int64_t)c.nb * kTBN + wr;
            n = n < N ? n : N - 1;
            c.vb[j] = PK ? (uint32_t)(((n >> 4) * G * 16 + (n & 15)) * 64 + 16 * cb)
                         : (uint32_t)(n * (K / 2) + 16 * cb);
        }
        c.vx[0] = c.vx[1] = 0u;
        if (wave < 4) {
            int64_t n = (int64_t)c.nb * kTBN + wave * 64 + lane;
            n = n < N ? n : N - 1;
            c.vx[0] = PK ? (uint32_t)(((n >> 4) * G4 * 16 + (n & 15)) * 16) : (uint32_t)(n * G * 4);
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int d = min((wave - 4 + 4 * j) * 64 + lane, 2 * kTBM - 1);
                c.vx[j] = (uint32_t)(((int64_t)act_row(d >> 1) * G) * 8 + 4 * (d & 1));
            }
        }
        return c;
    };
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    auto issue = [&](const Ctx& c, int g, int st) {
        const uint32_t base = smem_lds + (uint32_t)(st * kStageBytes);
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (wave + 8 * j < kALoads)
                lds_load16(ra, base + kAOff + (uint32_t)(wave + 8 * j) * 1024u, c.va[j], (uint32_t)g * kGroup);
        const uint32_t gw = (uint32_t)g * (PK ? 1024u : 64u);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            lds_load16(c.rw, base + kBOff + (uint32_t)(wave + 8 * j) * 1024u, c.vb[j], gw);
        if (wave < 4) {
            lds_load4(c.rws, base + kSwOff + wave * 256, c.vx[0],
                      PK ? (uint32_t)(g >> 2) * 256u + (uint32_t)(g & 3) * 4u : (uint32_t)g * 4u);
        } else {
            lds_load4(rsd, base + kSideOff + (wave - 4) * 256, c.vx[0], (uint32_t)g * 8u);
            if (wave == 4)
                lds_load4(rsd, base + kSideOff + 4 * 256, c.vx[1], (uint32_t)g * 8u);
        }
    };
    // this wave's loads per stage: waves 0-4 issue 6, waves 5-7 issue 5
    const bool six_loads = wave <= 4;
    auto wait_behind = [&](int behind) {  // the stage `behind` stages before the newest landed
        if (behind >= 2) {
            if (six_loads)
                wait_vmcnt<12>();
            else
                wait_vmcnt<10>();
        } else if (behind == 1) {
            if (six_loads)
                wait_vmcnt<6>();
            else
                wait_vmcnt<5>();
        } else {
            wait_vmcnt<0>();
        }
    };

    int wrow_f[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
        wrow_f[f] = 64 * wn + 16 * f + c16;
    auto read_b = [&](const uint8_t* base, v4i (&wb)[4], float (&sw)[4]) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            wb[f] = *(const v4i*)(base + kBOff + 16 * b_slot(wrow_f[f], q));
            sw[f] = *(const float*)(base + kSwOff + 4 * wrow_f[f]);
        }
    };
    auto read_a = [&](const uint8_t* base, int m, v4i& a0, v4i& a1) {
        const int trow = kHalf * wm + 16 * m;
        a0 = *(const v4i*)(base + kAOff + 16 * a_slot(trow + c16, q));
        a1 = *(const v4i*)(base + kAOff + 16 * a_slot(trow + c16, 4 + q));
    };
    auto read_side = [&](const uint8_t* base, int m, float4& s01, float4& s23) {
        const float4* sd = (const float4*)(base + kSideOff + 8 * (kHalf * wm + 16 * m + 4 * q));
        s01 = sd[0];
        s23 = sd[1];
    };

    Ctx cur = make_ctx(0);
    bool has_nxt = nt > 1;
    Ctx nxt = make_ctx(has_nxt ? 1 : 0);
    // prologue (G >= 4: positions 0..3 belong to the first tile)
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p)
        issue(cur, p, p);
    wait_behind(2);
    barrier();
    issue(cur, kStages - 1, kStages - 1);

    bool idle = kHalf * wm >= cur.rows;  // this wave's row half of the tile is empty

    int base = 0;  // stream position of the current tile's group 0
    for (int k = 0;;) {
        // the tile's K loop and epilogue for a wave that computes NSL of its
        // half's 16-row slices (as in tile_body: one instance per count,
        // chosen once per tile, the compute behind a run-time test too)
        const int nsl = min(kSlices, max(0, (cur.rows - kHalf * wm + 15) / 16));
        auto pass = [&](auto nsl_c) {
            constexpr int NSL = decltype(nsl_c)::value;
            float acc[NSL > 0 ? NSL : 1][4][4];
#pragma unroll
            for (int m = 0; m < NSL; ++m)
#pragma unroll
                for (int f = 0; f < 4; ++f)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[m][f][r] = 0;
            // group 0's fragments (read here rather than at the end of the
            // previous tile, so that no fragment register lives across the
            // choice of instance)
            v4i wb[4], a0 = {}, a1 = {};
            float sw[4];
            float4 s01 = {}, s23 = {};
            if (NSL > 0 && !idle) {
                const uint8_t* np = smem + (base & 3) * kStageBytes;
                read_b(np, wb, sw);
                read_a(np, 0, a0, a1);
                read_side(np, 0, s01, s23);
            }
            for (int g = 0; g < G; ++g) {
                const uint8_t* sp = smem + ((base + g) & 3) * kStageBytes;
                if (NSL > 0 && !idle) {
                    int eq[4];
                    float swc[4];
                    v8i b8[4];
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        if (FP4) {
                            eq[f] = (int)((__builtin_bit_cast(uint32_t, sw[f]) >> (8 * q)) & 0xFFu);
                        } else {
                            swc[f] = sw[f];
                            b8[f] = unpack_int4_u(wb[f]);
                        }
                    }
#pragma unroll
                    for (int m = 0; m < NSL; ++m) {
                        const v4i ca0 = a0, ca1 = a1;
                        const float4 cs01 = s01, cs23 = s23;
                        if (m + 1 < NSL) {
                            read_a(sp, m + 1, a0, a1);
                            read_side(sp, m + 1, s01, s23);
                        }
                        const v8i av = {ca0[0], ca0[1], ca0[2], ca0[3], ca1[0], ca1[1], ca1[2], ca1[3]};
                        v4f raw[4];
#pragma unroll
                        for (int f = 0; f < 4; ++f)
                            raw[f] = FP4 ? mfma16x16x128_fp4(av, wb[f], eq[f])
                                         : mfma16x16x128(av, b8[f], v4f{0.0f, 0.0f, 0.0f, 0.0f});
                        const float c1[4] = {cs01.x, cs01.z, cs23.x, cs23.z};
                        const float c0[4] = {cs01.y, cs01.w, cs23.y, cs23.w};
#pragma unroll
                        for (int f = 0; f < 4; ++f)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                if (FP4)  // weight scales inside raw: y += sa * raw
                                    acc[m][f][r] = fmaf(raw[f][r], c1[r] * 0x1p-9f, acc[m][f][r]);
                                else
                                    acc[m][f][r] = fmaf(swc[f], fmaf(raw[f][r], c1[r], c0[r]), acc[m][f][r]);
                            }
                    }
                }
                if (g + 1 < G) {
                    // position g + 1 landed for everyone; the stage of group g is
                    // free: refill it with position base + g + 4 (the next tile's
                    // first groups once this tile's are all issued)
                    wait_behind(min(2, G - 2 - g + (has_nxt ? G : 0)));
                    barrier();
                    const int p = g + kStages;
                    if (p < G)
                        issue(cur, p, (base + g) & 3);
                    else if (has_nxt)
                        issue(nxt, p - G, (base + g) & 3);
                    const uint8_t* np = smem + ((base + g + 1) & 3) * kStageBytes;
                    if (NSL > 0 && !idle) {
                        read_b(np, wb, sw);
                        read_a(np, 0, a0, a1);
                        read_side(np, 0, s01, s23);
                    }
                }
            }
            // epilogue: element (tile row 80wm + 16m + 4q + r, fragment f); the
            // next tile's groups 0..2 are in flight meanwhile
            if (NSL > 0 && !idle) {
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const int64_t n = (int64_t)cur.nb * kTBN + wrow_f[f];
                    if (n >= N)
                        continue;
#pragma unroll
                    for (int m = 0; m < NSL; ++m)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int row = kHalf * wm + 16 * m + 4 * q + r;
                            if (row < cur.rows)
                                a.out_f32[(int64_t)(cur.row0 + row) * N + n] = acc[m][f][r];
                        }
                }
            }
        };
        switch (nsl) {
        case 0: pass(std::integral_constant<int, 0>{}); break;
        case 1: pass(std::integral_constant<int, 1>{}); break;
        case 2: pass(std::integral_constant<int, 2>{}); break;
        case 3: pass(std::integral_constant<int, 3>{}); break;
        case 4: pass(std::integral_constant<int, 4>{}); break;
        default: pass(std::integral_constant<int, 5>{}); break;
        }
        if (!has_nxt)
            break;
        // Stores may complete out of order with the loads, so no vmcnt count
        // below zero is exact while they are pending: wait for everything
        // (the stores and the next tile's groups 0..2), then go on with exact
        // counts.  The stage of this tile's last group is free after the
        // barrier: refill it with the next tile's group 3.
        wait_vmcnt<0>();
        barrier();
        issue(nxt, kStages - 1, (base + G - 1) & 3);
        base += G;
        ++k;
        cur = nxt;
        idle = kHalf * wm >= cur.rows;
        has_nxt = k + 1 < nt;
        if (has_nxt)
            nxt = make_ctx(k + 1);
    }
}

template <bool PK, bool FP4>
__device__ __forceinline__ void down_phase(const GemmArgs& a, uint8_t* smem, int4* s_meta, int* s_expert)
{
    const int G = (int)(a.K / kGroup);
    const int nbn = (int)((a.N + kTBN - 1) / kTBN);
    const int total = *a.num_blocks * nbn;
    const int per_xcd = (total + 7) >> 3;
    const int x = (int)(blockIdx.x & 7);
    const int stride = (int)(gridDim.x >> 3);
    const int t0 = (int)(blockIdx.x >> 3);
    // this workgroup's tiles: L = x * per_xcd + t, t = t0, t0 + stride, ...
    const int tend = min(per_xcd, total - x * per_xcd);
    const int nt = tend > t0 ? (tend - t0 + stride - 1) / stride : 0;
    if (nt == 0)
        return;
    if (G >= kStages && nt <= kMaxStreamTiles) {
        down_stream<PK, FP4>(a, smem, s_meta, nt, x * per_xcd + t0, stride);
        return;
    }
    for (int t = t0; t < tend; t += stride) {  // short K or very many tiles: tile by tile
        tile_body<TILE_DOWN, PK, FP4>(a, x * per_xcd + t, smem, s_expert);
        __syncthreads();
    }
}

template <bool PK, bool FP4>
__global__ __launch_bounds__(kTThreads) void gemm_down_stream_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    __shared__ int4 s_meta[kMaxStreamTiles];
    __shared__ int s_expert;
    if (path_not_taken(a))
        return;
    down_phase<PK, FP4>(a, smem, s_meta, &s_expert);
}

// ---------------------------------------------------------------------------
// gate_up, down and the combine in one launch (DeepGEMM PR #53, "Changes":
// one persistent kernel runs L1 GEMM -> SwiGLU -> FP8 requant -> L2 GEMM ->
// combine).  One workgroup per CU, all resident at once (cooperative
// launch), walks the gate_up tiles and the down stream exactly as their
// launches do, then the combine's tokens (one per wave, below); between the
// phases every workgroup passes a grid barrier.  The arithmetic is the
// launches' own, so the output is bit-identical to the block-tiled path's.
// ---------------------------------------------------------------------------

// wall-clock bound of one barrier wait: s_memrealtime counts at 100 MHz
constexpr uint64_t kBarrierTicks = 200000000ull;  // 2 s

// Every workgroup arrives, then waits until `target` arrivals are counted.
// The agent-scope release before the arrival writes this XCD's dirty L2
// lines back, so the phase's outputs are visible to every XCD; the acquire
// after the wait drops stale cached lines.  The other threads are ordered by
// the workgroup barriers around thread 0's wait.  A wait longer than
// kBarrierTicks gives up (false), so that a launch whose workgroups were not
// all resident ends instead of spinning.
__device__ bool grid_barrier(int32_t* counter, int target, int* s_flag)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        int ok = 1;
        while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (__builtin_amdgcn_s_memrealtime() - t0 > kBarrierTicks) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *s_flag = ok;
    }
    __syncthreads();
    return *s_flag != 0;
}

// The combine phase, one token per wave.  The token's slots are read by the
// wave's first topk lanes; the local ones (a ballot) are walked in j order as
// a wave-uniform list; each lane owns 8 columns of every 512-column stripe,
// and the wave takes kCombineStripes stripes at a time, so that a lane has
// 2 * kCombineStripes row loads in flight per local slot, each wave load
// covering 2 KB of one row.  Per token the sum is the combine launch's (local
// slots in j order, one FMA each from +0, one bf16 rounding).  Measured
// against the combine launch: 54 vs 31 us at T = 4096, 322 vs 287 us on the
// EP8 share (at one workgroup per CU; a thread per (token, 8 columns) item
// with the slots listed in LDS reached 64 / 340 us).
constexpr int kCombineStripes = 8;
static_assert(W4A8_MAX_TOPK <= 64, "a token's slots fit one wave");

__device__ __forceinline__ void combine_phase(const TailArgs& t)
{
    const int lane = threadIdx.x & 63;
    const int waves = kTThreads / 64;
    const int64_t k = t.topk, H = t.H;
    const int64_t stride = (int64_t)gridDim.x * waves;
    for (int64_t tok = (int64_t)blockIdx.x * waves + (threadIdx.x >> 6); tok < t.T; tok += stride) {
        const int p_l = lane < k ? t.src2dst[tok * k + lane] : -1;
        const float w_l = lane < k ? t.topk_w[tok * k + lane] : 0.0f;
        const uint64_t local = __ballot(p_l >= 0);  // bit j: slot j is local
        // the column loop is wave-uniform (every lane takes part in the
        // shuffles below; a lane past H loads column 0 and stores nothing)
        for (int64_t cb = 0; cb < H; cb += 512 * kCombineStripes) {
            const int64_t c0 = cb + (int64_t)lane * 8;
            float acc[kCombineStripes][8];
#pragma unroll
            for (int s = 0; s < kCombineStripes; ++s)
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    acc[s][c] = 0.0f;
            for (uint64_t m = local; m != 0; m &= m - 1) {
                const int j = __builtin_ctzll(m);  // ascending j
                const int64_t p = __shfl(p_l, j, 64);
                const float w = __shfl(w_l, j, 64);
                float4 lo[kCombineStripes], hi[kCombineStripes];
#pragma unroll
                for (int s = 0; s < kCombineStripes; ++s) {
                    const int64_t col = c0 + s * 512;
                    const float4* src = (const float4*)(t.y2 + p * H + (col < H ? col : 0));
                    lo[s] = src[0];
                    hi[s] = src[1];
                }
#pragma unroll
                for (int s = 0; s < kCombineStripes; ++s) {
                    acc[s][0] = fmaf(w, lo[s].x, acc[s][0]);
                    acc[s][1] = fmaf(w, lo[s].y, acc[s][1]);
                    acc[s][2] = fmaf(w, lo[s].z, acc[s][2]);
                    acc[s][3] = fmaf(w, lo[s].w, acc[s][3]);
                    acc[s][4] = fmaf(w, hi[s].x, acc[s][4]);
                    acc[s][5] = fmaf(w, hi[s].y, acc[s][5]);
                    acc[s][6] = fmaf(w, hi[s].z, acc[s][6]);
                    acc[s][7] = fmaf(w, hi[s].w, acc[s][7]);
                }
            }
#pragma unroll
            for (int s = 0; s < kCombineStripes; ++s) {
                const int64_t col = c0 + s * 512;
                if (col < H) {
                    uint4 o;
                    o.x = (uint32_t)f32_to_bf16(acc[s][0]) | ((uint32_t)f32_to_bf16(acc[s][1]) << 16);
                    o.y = (uint32_t)f32_to_bf16(acc[s][2]) | ((uint32_t)f32_to_bf16(acc[s][3]) << 16);
                    o.z = (uint32_t)f32_to_bf16(acc[s][4]) | ((uint32_t)f32_to_bf16(acc[s][5]) << 16);
                    o.w = (uint32_t)f32_to_bf16(acc[s][6]) | ((uint32_t)f32_to_bf16(acc[s][7]) << 16);
                    *(uint4*)(t.out + tok * H + col) = o;
                }
            }
        }
    }
}

// The three phases' arguments are read from the kernel-argument segment at
// the start of their phase (through a pointer the compiler cannot see
// through), so that the down GEMM's and the combine's arguments do not sit in
// scalar registers during gate_up: loaded at entry they pushed the kernel's
// scalar-register spills from ~90 to ~180 and slowed both GEMM phases.
struct FusedArgs {
    GemmArgs gu, dn;
    TailArgs t;
};
typedef __attribute__((address_space(4))) const FusedArgs* KernargPtr;

__device__ __forceinline__ const FusedArgs* fused_args()
{
    KernargPtr p = (KernargPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return (const FusedArgs*)p;
}

template <bool PK, bool FP4>
__global__ __launch_bounds__(kTThreads) void fused_tail_kernel(FusedArgs)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    __shared__ int4 s_meta[kMaxStreamTiles];
    __shared__ int s_expert, s_flag;
    const int wgs = (int)gridDim.x;
    {
        const GemmArgs gu = fused_args()->gu;
        tile_phase<TILE_GATEUP, PK, FP4>(gu, smem, &s_expert);
    }
    if (!grid_barrier(fused_args()->t.barrier, wgs, &s_flag))
        return;
    {
        const GemmArgs dn = fused_args()->dn;
        down_phase<PK, FP4>(dn, smem, s_meta, &s_expert);
    }
    if (!grid_barrier(fused_args()->t.barrier, 2 * wgs, &s_flag))
        return;
    const TailArgs t = fused_args()->t;
    combine_phase(t);
}

int64_t tile_launch_workgroups(int64_t tiles)
{
    // one workgroup per CU (the LDS stages allow no more), a multiple of the 8 XCDs
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
        cus = 256;
    const int64_t wgs = tiles < cus ? tiles : cus;
    return (wgs + 7) / 8 * 8;
}

hipError_t launch_fused_tail(const GemmArgs& gu, const GemmArgs& dn, const TailArgs& t, hipStream_t s)
{
    if ((gu.fp4 && !gu.packed) || gu.sub_group != 128 || dn.sub_group != 128)
        return hipErrorInvalidValue;
    const void* fn = gu.fp4      ? reinterpret_cast<const void*>(&fused_tail_kernel<true, true>)
                     : gu.packed ? reinterpret_cast<const void*>(&fused_tail_kernel<true, false>)
                                 : reinterpret_cast<const void*>(&fused_tail_kernel<false, false>);
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kTThreads, 0);
    if (e != hipSuccess)
        return e;
    // one workgroup per CU (the LDS stages allow no more), a multiple of the 8 XCDs
    const int wgs = cus / 8 * 8;
    if (per_cu < 1 || wgs < 8)
        return hipErrorInvalidConfiguration;
    FusedArgs fa = {gu, dn, t};
    void* args[] = {&fa};
    return hipLaunchCooperativeKernel(fn, dim3((unsigned)wgs), dim3(kTThreads), args, 0, s);
}

hipError_t launch_gemm_tile(const GemmArgs& a, int mode, hipStream_t s)
{
    const int64_t nbn = mode == TILE_GATEUP ? a.I / kGroup : (a.N + kTBN - 1) / kTBN;
    const int64_t tiles = nbn * a.max_blocks;
    if (tiles == 0)
        return hipSuccess;
    const dim3 grid((unsigned)tile_launch_workgroups(tiles));
    if ((a.fp4 && !a.packed) || a.sub_group != 128)
        return hipErrorInvalidValue;  // the finer activation recipes run on the skinny kernel
    const dim3 block(kTThreads);
    if (mode == TILE_GATEUP) {
        if (a.fp4)
            hipLaunchKernelGGL((gemm_tile_kernel<TILE_GATEUP, true, true>), grid, block, 0, s, a);
        else if (a.packed)
            hipLaunchKernelGGL((gemm_tile_kernel<TILE_GATEUP, true, false>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((gemm_tile_kernel<TILE_GATEUP, false, false>), grid, block, 0, s, a);
    } else {
        if (a.fp4)
            hipLaunchKernelGGL((gemm_down_stream_kernel<true, true>), grid, block, 0, s, a);
        else if (a.packed)
            hipLaunchKernelGGL((gemm_down_stream_kernel<true, false>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((gemm_down_stream_kernel<false, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace w4a8
