// internal.hpp -- host-side launchers shared between the translation units of
// libw4a8.  Not part of the public ABI (see include/w4a8.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a8 {

// ---- activation quantisation (quant.hip) ----
// mode 0: canonical codes + fp32 scales (the public export)
// mode 1: K-interleaved codes + {c1, c0} side data (the GEMM operand of
//         every path, converted to f16 in registers by the gate_up GEMMs)
// fixed_scale: null for the dynamic rule, else a device pointer to a static
// per-tensor scale
hipError_t launch_quant_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                             float* scales, float2* side, int mode, const float* fixed_scale,
                             hipStream_t s);

// ---- routing permutation (align.hip) ----
// Predicted time (us) of the two GEMMs of one fused call on either path, from
// the per-expert counts the align finds (constants set on the host):
//   skinny: skinny_fixed_us + (m-blocks of both lists) * skinny_block_us
//           (every m-block streams one expert's gate_up and down weights);
//   tiled:  for each of the two tile launches, the slowest workgroup's sum
//           over the tiles it walks (the launchers' static tile order) of
//           groups * (c0 + c1 * rows computed), a tile's rows rounded up to
//           16-row slices in each 80-row half.
struct PathCost {
    float skinny_fixed_us, skinny_block_us;
    float groups_gu, groups_dn;  // 128-K groups per tile
    int32_t nbn_gu, nbn_dn;      // tiles per m-block
    int32_t wgs_gu, wgs_dn;      // workgroups of the two tile launches
    float gu0, gu1, dn0, dn1;    // us per group of one tile: constant + per computed row
};
struct AlignOut {
    int32_t* counts;        // [E]
    int32_t* offsets;       // [E+1]
    int32_t* sorted;        // [F]
    int32_t* src2dst;       // [F]
    int32_t* block_expert;  // [nb_max] or null
    int32_t* block_row;     // [nb_max] or null
    int32_t* num_blocks;    // [1]
    int32_t* block_start;   // [E+1] index of each expert's first m-block, or null
    // Two block lists (block_expert2 != null): experts with at most
    // small_rows pairs get blocks of block_m rows in the first list, the
    // others blocks of block_m2 rows in the second (per-expert block height
    // from the device-side counts)
    int32_t* block_expert2;  // [nb2_max] or null
    int32_t* block_row2;     // [nb2_max]
    int32_t* num_blocks2;    // [1]
    int32_t small_rows;
    int32_t block_m2;
    // Capacity of the per-pair buffers (sorted, the GEMMs' rows), <= 0 for
    // none.  When the local pairs exceed it no expert is computed: offsets,
    // block counts and block_start are written as zero and every src2dst
    // entry as -1, so the GEMMs do nothing and the combine writes +0.
    int32_t max_pairs;
    int32_t* pairs_out;  // [2] receives the number of local pairs and the path, or null
    // Path chosen on the device (path != null): besides the two lists above,
    // a list of kTileRows-row blocks (block_row3, num_blocks3, and
    // block_start for it) is written, and *path receives 1 when the
    // block-tiled GEMMs are predicted faster than the two skinny lists, else
    // 0 (cost model below).  With path == null, static_path is reported.
    int32_t* block_row3;   // [nb3_max]
    int32_t* num_blocks3;  // [1]
    int32_t* path;         // [1]
    int32_t static_path;
    PathCost cost;
    // the single-launch tail's grid-barrier counter, set to 0 here (the
    // launch after the align counts on it), or null
    int32_t* barrier;
};
int64_t align_chunk_count(int64_t F);
size_t align_workspace_bytes(int64_t F, int64_t E);
// The mode-1 quantisation of x [M, K] (row stride ldx) riding along with
// the chunked align: its blocks of 16 x 128 values are split between the
// count and the scatter launch (x == null: none).
struct QuantJob {
    const uint16_t* x;
    int64_t M, K, ldx;
    uint8_t* q;
    float2* side;
    const float* fixed_scale;
};
hipError_t launch_align(const int32_t* ids, int64_t T, int64_t topk, int64_t expert_begin,
                        int64_t E, int64_t block_m, const AlignOut& o, void* ws, hipStream_t s,
                        const QuantJob& qj = QuantJob{});
// align (single chunk: align_chunk_count(T*topk) == 1) and the mode-1
// quantisation of x [T, H] in one launch
hipError_t launch_align_quant(const int32_t* ids, int64_t T, int64_t topk, int64_t expert_begin,
                              int64_t E, int64_t block_m, const AlignOut& o, const uint16_t* x,
                              int64_t H, uint8_t* q, float2* side, const float* fixed_scale,
                              hipStream_t s);

// ---- grouped GEMMs (gemm_skinny.hip) ----
struct GemmArgs {
    // activation operand (fp8 codes, row stride K) + side data [rows, K/128];
    // the K order inside each 8-group depends on the path (see common.hpp)
    const uint8_t* act;
    int f16;
    int64_t act_rows;   // rows of the activation buffer (bounds of its buffer resource)
    const float2* act_side;
    // row map: GEMM row p of an m-block -> activation row.  If sorted != null,
    // act_row = sorted[p] / topk (gather through the permutation), else p.
    const int32_t* sorted;
    int32_t topk;
    // m-blocks
    const int32_t* block_expert;
    const int32_t* block_row;
    const int32_t* num_blocks;
    const int32_t* offsets;  // [E+1] segment ends (rows of expert e: [offsets[e], offsets[e+1]))
    const int32_t* block_start;  // [E+1] first m-block of each expert (tile GEMM)
    int32_t num_experts;
    int32_t dense_rows;      // used when offsets == null: rows [0, dense_rows)
    // weights of expert e: w + e*w_estride, scales ws + e*s_estride; row n at
    // n*K/2, n*K/128, or in the prepacked layout if packed (see common.hpp)
    int packed;
    int fp4;   // prepacked fp4 e2m1 weights; ws then holds UE8M0 dwords
    const uint8_t* w;
    const float* ws;
    int64_t w_estride, s_estride;
    int64_t K;       // reduction length
    int64_t N;       // output features of the weight matrix
    int64_t I;       // SwiGLU epilogue: intermediate size (gate rows [0,I), up rows [I,2I))
    // outputs
    float* out_f32;        // [rows, N]           (store epilogue)
    uint16_t* out_bf16;    // [rows, N]           (bf16 epilogue)
    uint8_t* out_q;        // [rows, I] codes     (SwiGLU+requant epilogue, interleaved)
    float2* out_side;      // [rows, I/128]
    const float* requant_scale;  // static per-tensor scale of the requant, or null (dynamic)
    // K per dynamic activation scale of the down GEMM's input: 128, or 64 / 32
    // (finer recipes; the SwiGLU epilogue emits such blocks, the down GEMM
    // reads them; side data [rows, K/sub_group]); skinny kernel only
    int sub_group;
    int64_t max_blocks;    // grid bound on m-blocks
    // skinny kernel, 16-row m-blocks: blocks of at most this many rows read
    // their activations from a whole-K copy in LDS (set by the launcher)
    int32_t stage_rows;
    // path chosen on the device: the kernel runs only if *path == path_want
    // (path == null: always)
    const int32_t* path;
    int32_t path_want;
};
// a workgroup's early exit when the device chose the other path
__device__ __forceinline__ bool path_not_taken(const GemmArgs& a)
{
    return a.path != nullptr && *a.path != a.path_want;
}
enum Epilogue { EPI_F32 = 0, EPI_SWIGLU_Q = 2 };
hipError_t launch_gemm_skinny(const GemmArgs& a, int epilogue, int block_m, hipStream_t s);
// per-expert block heights: list a1 of 16-row blocks and list a2 of 32-row
// blocks (same operands otherwise) in one launch
hipError_t launch_gemm_skinny_two_lists(const GemmArgs& a1, const GemmArgs& a2, int epilogue,
                                        hipStream_t s);

// ---- dense linear (dense.hip) ----
// canonical codes [M, K] + scales [M, K/128] x packed int4 [N, K/2] + scales
// [N, K/128]; K cut in slices of split_groups 128-groups (at most
// dense_max_split_groups()); one slice: bf16 out, else fp32 partials
// part[slice][M, N]
int dense_max_split_groups();
hipError_t launch_dense_gemm(const uint8_t* a, const float* sa, int64_t M, int64_t K, const uint8_t* w,
                             const float* sw, int64_t N, int32_t split_groups, float* part,
                             uint16_t* out, hipStream_t s);
// out[M, N] bf16 = sum over `splits` fp32 partials part[z][M, N], in z order
hipError_t launch_split_reduce(const float* part, int32_t splits, int64_t M, int64_t N, uint16_t* out,
                               hipStream_t s);

// ---- grouped GEMM for many rows per expert (gemm_tile.hip) ----
// m-blocks of kTileRows rows (two halves of five 16-row slices).
constexpr int kTileRows = 160;
enum TileMode { TILE_DOWN = 0, TILE_GATEUP = 1 };
hipError_t launch_gemm_tile(const GemmArgs& a, int mode, hipStream_t s);
// workgroups launch_gemm_tile starts for `tiles` tiles (at most one per CU,
// a multiple of the 8 XCDs)
int64_t tile_launch_workgroups(int64_t tiles);

// ---- weight prepack (prepack.hip) ----
// [E, N, K/2] int4 + [E, N, K/128] fp32 or bf16 scales (or fp4 + [E, N, K/32]
// UE8M0 bytes) -> the prepacked layouts (common.hpp); 4-byte scale elements
hipError_t launch_prepack(const uint8_t* w, const void* ws, int64_t E, int64_t N, int64_t K,
                          bool shuffle_nibbles, bool bf16_scales, uint8_t* wp, void* sp, hipStream_t s);

// ---- single-launch tail (gemm_tile.hip) ----
// gate_up (gu, block-tiled), down (dn, block-tiled stream) and the combine
// in one cooperative launch of one workgroup per CU, with a grid barrier
// between the phases on the counter `barrier` (0 at entry: the align sets it)
struct TailArgs {
    const float* y2;
    const int32_t* src2dst;
    const float* topk_w;
    int64_t T, topk, H;
    uint16_t* out;
    int32_t* barrier;
};
hipError_t launch_fused_tail(const GemmArgs& gu, const GemmArgs& dn, const TailArgs& t, hipStream_t s);

// ---- combine (combine.hip) ----
hipError_t launch_combine(const float* y2, const int32_t* src2dst, const float* topk_w,
                          int64_t T, int64_t topk, int64_t H, uint16_t* out, hipStream_t s);

} // namespace w4a8
