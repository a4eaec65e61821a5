/*
 * w4a8.h -- C ABI of libw4a8: the W4AFP8 fused-MoE forward on one MI355X
 * (gfx950), as hand-written HIP kernels.
 *
 * The method (page titles; the passage in quotes or in brackets):
 *  - SGLang PR #7762 "feat: support DeepSeek-R1-W4AFP8 model with ep-moe
 *    mode": MoE experts hold INT4 weights and take FP8 activations ["Model
 *    Info"]; the MoE op scales the input hidden states and the intermediate
 *    values, permutes tokens before the w4a8 grouped GEMM and un-permutes
 *    after it, with SiLU-and-Mul between the two GEMMs ["Cutlass W4A8 MoE",
 *    "Kernel"]; the permutation is a stable sort of the local top-k ids with
 *    per-expert segment offsets and a src2dst map [review thread on
 *    run_cutlass_moe_ep_preproess]; global ids become local through the
 *    expert map [review thread on expert_map]; weight groups are 128 wide
 *    along K [review thread on the hard-coded chunk size].
 *  - DeepGEMM PR #53 "SM90 (Hopper) FP4 MegaMoE fused kernel with swapAB
 *    small-batch path": activation scales are plain fp32 per token (no
 *    power-of-two rounding) and amax is clamped before the reciprocal
 *    448/amax [commit note dropping UE8M0]; the fused order is L1 GEMM ->
 *    SwiGLU -> per-token FP8 requant -> L2 GEMM -> combine ["Changes"].
 *  - SGLang PR #37796 "feat(moe_wna16): 2-bit experts, expert streaming,
 *    N-contiguous GEMV": values are saturated to +-448 before the e4m3 cast
 *    [part-1 notes on the fp8 KV write path].
 *
 * Numerical contract (identical in every export):
 *  - fp8 is OCP e4m3 ("fn", max 448).  Quantisation of one 128-wide block of
 *    one row: amax = max|x|; amax_c = max(amax, 1e-10f); inv = 448/amax_c
 *    (IEEE fp32 divide); scale = amax_c/448; code = e4m3(clamp(x*inv, +-448))
 *    with round-to-nearest-even, subnormals kept, sign kept (-0 -> 0x80).
 *  - int4 weights: byte b holds k even in b & 0xF and k odd in b >> 4, two's
 *    complement (-8..7), no zero point; one fp32 scale per 128 K-elements.
 *  - GEMM: y[m,n] = sum_g a_scale[m,g] * w_scale[n,g] * sum_{k in g}
 *    dec(a[m,k]) * w[n,k].  On the GPU each group's sum comes from an MFMA
 *    and is promoted with its two scales into an fp32 accumulator; the
 *    gate_up GEMM of w4a8_fused_moe runs on fp16 MFMA with exactly converted
 *    operands, whose group sums are correctly rounded, because its output is
 *    re-quantised.
 *
 * Conventions:
 *  - Every pointer is a device pointer on the current HIP device unless
 *    noted, 16-byte aligned.  The caller owns all memory; the library never
 *    allocates and never synchronises the host: every launch is asynchronous
 *    on `stream` (0 = the null stream).  The only state between calls is the
 *    per-thread arming of w4a8_fused_moe_stage_events (a profiling hook).
 *  - Return value: W4A8_OK, or an error code.  Arguments are validated on the
 *    host before anything is launched; on error nothing is launched and no
 *    output is touched.  W4A8_ERR_HIP reports a failed launch.
 *  - Workspace: pass workspace == NULL to query; the required size (a pure
 *    function of the shape arguments) is written to *workspace_bytes and
 *    W4A8_OK is returned.  Otherwise *workspace_bytes must hold the size of
 *    the buffer supplied.
 *  - Calls that share a workspace or outputs must be ordered by the caller.
 *  - Size limits (W4A8_ERR_UNSUPPORTED beyond them): the kernels address each
 *    operand through a buffer resource with 32-bit extent and offsets, so the
 *    byte size of every activation matrix a GEMM reads (M*K for w4a8_gemm;
 *    T*H and T*topk*I for the fused forward, every pair counted as local,
 *    or max_local_pairs*I under w4a8_fused_moe_bounded) and of one expert's
 *    weights (N*K/2; I*H for w13) must stay below 2^32.
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A8_OK = 0,
    W4A8_ERR_INVALID_ARG = 1, /* null pointer, negative or zero size, bad leading dim */
    W4A8_ERR_UNSUPPORTED = 2, /* K/H/I not a multiple of 128, topk > 32, misaligned pointer */
    W4A8_ERR_WORKSPACE = 3,   /* workspace smaller than the queried size */
    W4A8_ERR_HIP = 4          /* a kernel launch failed */
} w4a8_status;

#define W4A8_GROUP 128
#define W4A8_MAX_TOPK 32

/* Library version as (major << 16) | minor. */
int w4a8_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* w4a8_status_string(int status);

/*
 * w4a8_quantize_act -- dynamic per-token-per-128 fp8 quantisation
 * (DeepGEMM PR #53, commit note dropping UE8M0; SGLang PR #37796 part-1
 * saturation note).
 *
 *   x_bf16  [M, K] bf16, row stride ldx elements (ldx >= K)
 *   q_e4m3  [M, K] fp8 e4m3 codes, row stride K, canonical K order
 *   scales  [M, K/128] fp32 dequantisation scales (amax_c / 448)
 * M >= 0 (M == 0 launches nothing), K > 0 and K % 128 == 0.
 * Results are bit-exact with the rule above.
 */
int w4a8_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                      uint8_t* q_e4m3, float* scales, hipStream_t stream);

/*
 * w4a8_gemm -- dense W4AFP8 linear: out = bf16(A * W^T) with per-group
 * promotion (SGLang PR #7762, "Model Info" and the chunk-size thread).
 *
 *   a_e4m3    [M, K] codes from w4a8_quantize_act; a_scales [M, K/128] fp32
 *   b_int4    [N, K/2] packed int4;                 b_scales [N, K/128] fp32
 *   out_bf16  [M, N] bf16, round to nearest even from the fp32 accumulator
 *   workspace device scratch of *workspace_bytes bytes (query with NULL):
 *             fp32 partial sums when K is cut into slices that run in
 *             parallel (the query returns 0 when it is not)
 * M >= 0, N > 0, K > 0, K % 128 == 0; M*K < 2^32 and N*K/2 < 2^32 bytes,
 * M <= 8388480 (UNSUPPORTED otherwise).  Reads the codes and scales exactly
 * as w4a8_quantize_act writes them (no re-layout).  fp32 accumulation order
 * is the kernel's (slices are added in K order); the result matches the fp64
 * definition within rounding.
 */
int w4a8_gemm(const uint8_t* a_e4m3, const float* a_scales, int64_t M, int64_t K,
              const uint8_t* b_int4, const float* b_scales, int64_t N,
              void* out_bf16, void* workspace, size_t* workspace_bytes,
              hipStream_t stream);

/*
 * w4a8_moe_align -- routing permutation (SGLang PR #7762, review threads on
 * run_cutlass_moe_ep_preproess and expert_map).
 *
 * Pair f = t*topk + j routes token t to global expert topk_ids[f].  It is
 * local when l = topk_ids[f] - expert_begin is in [0, num_local_experts);
 * every other id (including -1 padding) is skipped.  Outputs:
 *   expert_counts   [E_l]     local pairs per local expert
 *   expert_offsets  [E_l+1]   exclusive prefix sum (offsets[E_l] = P)
 *   sorted_pair_ids [T*topk]  the P local f's, stable-sorted by l (ties keep
 *                             ascending f); entries >= P are left unspecified
 *   src2dst         [T*topk]  position of f in that order, -1 if not local
 *   block_expert, block_row [ceil(T*topk/block_m) + E_l]
 *                             the m-blocks: for l ascending, rows
 *                             offsets[l] + b*block_m for b < ceil(c_l/block_m)
 *   num_blocks      [1]       number of m-blocks written
 *   workspace       device scratch of *workspace_bytes bytes (query with NULL)
 * T >= 0, 1 <= topk <= 32, E_l >= 1, block_m >= 1.  Bit-exact (one
 * correct answer).  block_expert/block_row may be NULL to skip the blocks
 * (num_blocks is then still written).
 */
int w4a8_moe_align(const int32_t* topk_ids, int64_t T, int64_t topk,
                   int64_t expert_begin, int64_t num_local_experts, int64_t block_m,
                   int32_t* expert_counts, int32_t* expert_offsets,
                   int32_t* sorted_pair_ids, int32_t* src2dst,
                   int32_t* block_expert, int32_t* block_row, int32_t* num_blocks,
                   void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * w4a8_fused_moe -- the whole forward on this GPU's experts (SGLang PR
 * #7762 "Cutlass W4A8 MoE" workflow; DeepGEMM PR #53 "Changes"):
 *   align -> quantise hidden -> gate_up grouped GEMM (rows gathered through
 *   the permutation) -> SwiGLU h = silu(y[:, :I]) * y[:, I:] -> fp8 requant
 *   per 128 of I -> down grouped GEMM -> out[t] = bf16(sum over t's local
 *   pairs of topk_weights * y2), +0 for a token with no local pair.
 *
 *   hidden_bf16  [T, H] bf16 (row stride H)
 *   topk_ids     [T, topk] int32 global expert ids; topk_weights [T, topk] fp32
 *   w13_int4     [E_l, 2I, H/2] (gate rows [0, I), up rows [I, 2I))
 *   w13_scales   [E_l, 2I, H/128] fp32
 *   w2_int4      [E_l, H, I/2];   w2_scales [E_l, H, I/128] fp32
 *   out_bf16     [T, H] bf16
 *   workspace    device scratch of *workspace_bytes bytes (query with NULL);
 *                holds the routing permutation, the fp8 activations and the
 *                intermediates between the kernels of one call
 * T >= 0 (T == 0 launches nothing), H, I > 0 and multiples of 128,
 * 1 <= topk <= 32, 1 <= E_l <= 1024, T*topk <= 2^30 - 1, and the byte
 * ranges T*H, T*topk*I and I*H below 2^32 (UNSUPPORTED otherwise).
 */
int w4a8_fused_moe(const void* hidden_bf16, int64_t T, int64_t H,
                   const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                   int64_t expert_begin, int64_t num_local_experts, int64_t I,
                   const uint8_t* w13_int4, const float* w13_scales,
                   const uint8_t* w2_int4, const float* w2_scales,
                   void* out_bf16, void* workspace, size_t* workspace_bytes,
                   hipStream_t stream);

/*
 * w4a8_prepack_weights -- one-time re-layout of int4 weights and their
 * scales for w4a8_fused_moe_prepacked (the load-time weight processing of
 * SGLang PR #7762, "W4AFp8MoEMethod": process_weights_after_loading; the
 * layout is this library's own).  Pure data movement, asynchronous.
 *   w_int4    [E, N, K/2] packed int4 (canonical layout, see above)
 *   w_scales  [E, N, K/128] fp32
 *   w_packed  E*N*K/2 bytes: [E][N/16][K/128][16][64]: the 64 bytes of row n
 *             for K-group g at ((n/16 * (K/128) + g) * 16 + n%16) * 64
 *             within the expert's E-slice of N*K/2 bytes
 *   s_packed  w4a8_prepacked_scale_count(E, N, K) floats:
 *             [E][N/16][G4][16][4], G4 = ceil(K/512): the scale of row n,
 *             group g at ((n/16 * G4 + g/4) * 16 + n%16) * 4 + g%4 within the
 *             expert's slice of N*G4*4 floats; zero past the last group
 * N % 16 == 0, K % 128 == 0; outputs must not alias the inputs.  Errors:
 * INVALID_ARG (null, non-positive sizes, in place), UNSUPPORTED (shape or
 * alignment), HIP.
 */
int w4a8_prepack_weights(const uint8_t* w_int4, const float* w_scales, int64_t E, int64_t N,
                         int64_t K, uint8_t* w_packed, float* s_packed, hipStream_t stream);

/*
 * w4a8_prepack_weights_bf16_scales -- w4a8_prepack_weights for checkpoints
 * that store the int4 weights' per-128 scales as bf16 ([E, N, K/128] bf16,
 * 2-byte aligned).  Each scale is widened to fp32 (exact), so the prepacked
 * output equals w4a8_prepack_weights' on the widened scales, and
 * w4a8_fused_moe_prepacked runs on it unchanged.  Same layout, arguments and
 * errors as w4a8_prepack_weights.
 */
int w4a8_prepack_weights_bf16_scales(const uint8_t* w_int4, const uint16_t* w_scales_bf16, int64_t E,
                                     int64_t N, int64_t K, uint8_t* w_packed, float* s_packed,
                                     hipStream_t stream);

/* 4-byte elements of the prepacked scales of E experts of N x K, for both
 * weight formats (host-only; -1 for a bad shape). */
int64_t w4a8_prepacked_scale_count(int64_t E, int64_t N, int64_t K);

/*
 * w4a8_fused_moe_prepacked -- w4a8_fused_moe on weights prepacked by
 * w4a8_prepack_weights (w13: N = 2I, K = H; w2: N = H, K = I).  Same
 * arguments, results, workspace and errors as w4a8_fused_moe.  Each 16-row x
 * 128-K weight block is one contiguous kilobyte, which the GEMM kernels
 * stream with one load per wave.
 */
int w4a8_fused_moe_prepacked(const void* hidden_bf16, int64_t T, int64_t H,
                             const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                             int64_t expert_begin, int64_t num_local_experts, int64_t I,
                             const uint8_t* w13_packed, const float* w13_scales_packed,
                             const uint8_t* w2_packed, const float* w2_scales_packed,
                             void* out_bf16, void* workspace, size_t* workspace_bytes,
                             hipStream_t stream);

/*
 * w4a8_fused_moe_prepacked_static -- w4a8_fused_moe_prepacked with static
 * per-tensor activation scales, as a checkpoint that ships input scales with
 * its weights provides them (SGLang PR #7762 loads input and weight scales
 * for the W4AFP8 MoE layers).
 *   a1_scale  device pointer to one fp32 scale s for the hidden states, or
 *             NULL for the dynamic per-token-per-128 rule
 *   a2_scale  the same for the requantised SwiGLU output
 * With a static s a 128-block's codes are e4m3(clamp(x * inv, +-448)), inv =
 * 1/s rounded once to fp32, and its dequant scale is s (values beyond
 * 448*s saturate).  The scales are read on the device when the kernels run,
 * so a captured graph follows later updates of them.  Same workspace and
 * errors as w4a8_fused_moe_prepacked, plus UNSUPPORTED for a scale pointer
 * that is not 4-byte aligned.
 */
int w4a8_fused_moe_prepacked_static(const void* hidden_bf16, int64_t T, int64_t H,
                                    const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                                    int64_t expert_begin, int64_t num_local_experts, int64_t I,
                                    const uint8_t* w13_packed, const float* w13_scales_packed,
                                    const uint8_t* w2_packed, const float* w2_scales_packed,
                                    const float* a1_scale, const float* a2_scale, void* out_bf16,
                                    void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * w4a8_fused_moe_recipe -- the fused forward with a finer dynamic activation
 * scale for the down GEMM's input (DeepGEMM PR #53 commit notes: the per-32
 * recipe and the 128/64 recipe): the SwiGLU output is requantised with one
 * scale per down_act_group K (128, 64 or 32) and the down GEMM promotes each
 * such block with its own scale; the gate_up input keeps per-128 scales.
 *   weight_format   W4A8_WEIGHTS_INT4_PACKED (w4a8_prepack_weights output,
 *                   fp32 scales) or W4A8_WEIGHTS_FP4_PACKED
 *                   (w4a8_prepack_weights_fp4 output, UE8M0 dwords)
 *   down_act_group  128, 64 or 32
 * Other arguments, workspace and errors as w4a8_fused_moe_prepacked
 * (INVALID_ARG for an unknown format or group).  With a group below 128 the
 * call runs on the few-rows-per-expert GEMM at every size, and the side data
 * at offsets[10] is [T*topk, I/down_act_group].
 */
#define W4A8_WEIGHTS_INT4 0 /* canonical int4 layout, as w4a8_fused_moe reads it */
#define W4A8_WEIGHTS_INT4_PACKED 1
#define W4A8_WEIGHTS_FP4_PACKED 2
int w4a8_fused_moe_recipe(const void* hidden_bf16, int64_t T, int64_t H, const int32_t* topk_ids,
                          const float* topk_weights, int64_t topk, int64_t expert_begin,
                          int64_t num_local_experts, int64_t I, int weight_format,
                          const uint8_t* w13_packed, const void* w13_scales_packed,
                          const uint8_t* w2_packed, const void* w2_scales_packed, int down_act_group,
                          void* out_bf16, void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * FP4 weights (DeepGEMM PR #53, "Changes": FP8 E4M3 activations x packed FP4
 * E2M1 expert weights with per-32-K UE8M0 weight scales).  Canonical input
 * layout: w_fp4 [E, N, K/2] e2m1 codes, two per byte, k even in the low
 * nibble; w_scales_ue8m0 [E, N, K/32] bytes, the weight at (n, k) being
 * e2m1 * 2^(scale[n, k/32] - 127).  Activations keep their dynamic per-token
 * per-128 fp32 scales.
 *
 * w4a8_prepack_weights_fp4 -- one-time re-layout for
 * w4a8_fused_moe_fp4_prepacked; pure data movement, asynchronous.
 *   role      W4A8_FP4_GATE_UP for w13 (N = 2I, K = H), W4A8_FP4_DOWN for
 *             w2 (N = H, K = I): the gate_up GEMM converts its weights to
 *             f16 in the activation operand's K order, so its nibbles are
 *             reordered; the down GEMM feeds them to the scaled MFMA as they are
 *   w_packed  E*N*K/2 bytes, blocked as w4a8_prepack_weights does; with
 *             W4A8_FP4_GATE_UP each dword's nibbles k0..k7 become
 *             k0,k2,k4,k6,k1,k3,k5,k7
 *   s_packed  w4a8_prepacked_scale_count(E, N, K) dwords, placed as the fp32
 *             scales of w4a8_prepack_weights; the dword of row n, group g
 *             holds the group's four UE8M0 bytes (32-K block b in byte b)
 * N % 16 == 0, K % 128 == 0; w_scales_ue8m0 4-byte aligned, the rest
 * 16-byte aligned; outputs must not alias the inputs.  Errors: INVALID_ARG
 * (null, non-positive sizes, unknown role, in place), UNSUPPORTED (shape or
 * alignment), HIP.
 */
#define W4A8_FP4_GATE_UP 0
#define W4A8_FP4_DOWN 1
int w4a8_prepack_weights_fp4(const uint8_t* w_fp4, const uint8_t* w_scales_ue8m0, int64_t E,
                             int64_t N, int64_t K, int role, uint8_t* w_packed,
                             uint32_t* s_packed, hipStream_t stream);

/*
 * w4a8_fused_moe_fp4_prepacked -- the fused forward on fp4 weights prepacked
 * by w4a8_prepack_weights_fp4 (w13 with W4A8_FP4_GATE_UP, w2 with
 * W4A8_FP4_DOWN).  Same arguments, workspace and errors as
 * w4a8_fused_moe_prepacked; the result follows the same definition with each
 * weight e2m1 * 2^(e - 127).  The gate_up GEMM stays exact (f16 MFMA on
 * exactly converted operands) while the four block exponents of a row's
 * 128-group lie within 23 binades of their maximum; the down GEMM applies the
 * block scales in the MFMA itself.  The requantised intermediate in the
 * workspace (offsets[9]) is stored in natural K order on this path.
 */
int w4a8_fused_moe_fp4_prepacked(const void* hidden_bf16, int64_t T, int64_t H,
                                 const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                                 int64_t expert_begin, int64_t num_local_experts, int64_t I,
                                 const uint8_t* w13_packed, const uint32_t* w13_scales_packed,
                                 const uint8_t* w2_packed, const uint32_t* w2_scales_packed,
                                 void* out_bf16, void* workspace, size_t* workspace_bytes,
                                 hipStream_t stream);

/*
 * w4a8_fused_moe_bounded -- the fused forward with its per-pair buffers sized
 * for a caller's bound on the LOCAL pairs instead of T*topk.  On an
 * expert-parallel rank only the top-k slots that name one of its E_l experts
 * are computed (SGLang PR #7762, review thread on expert_map), about E_l/E of
 * them; a workspace sized for every slot (the other exports: at T = 32768,
 * topk = 8, H = 7168, I = 2048 about 8.4 GB, 7.5 GB of it the fp32 down
 * output) then holds mostly unused rows.  The caller, who knows its share
 * from the dispatch, passes a bound; the workspace query scales with it.
 *   weight_format    W4A8_WEIGHTS_INT4 (canonical, as w4a8_fused_moe),
 *                    W4A8_WEIGHTS_INT4_PACKED (as w4a8_fused_moe_prepacked) or
 *                    W4A8_WEIGHTS_FP4_PACKED (as w4a8_fused_moe_fp4_prepacked)
 *   max_local_pairs  >= 1: the bound on the pairs whose expert is local
 *                    (values above T*topk count as T*topk)
 *   local_pairs      device int32[2], written on the stream: [0] the number
 *                    of local pairs the call found, [1] 1 if the block-tiled
 *                    GEMM kernels ran, 0 if the few-rows ones did (required
 *                    unless T == 0 or workspace == NULL; 8-byte aligned)
 * Within the bound the output equals that of the export of the same weight
 * format (bit for bit when both take the same kernels).  The path follows
 * min(max_local_pairs, T*topk) per local expert: at most 2 rows per expert
 * the few-rows kernel with 16-row m-blocks; above that, while the few-rows
 * kernel's m-block lists stay below 4096 blocks, the align chooses on the
 * device between per-expert 16 / 32-row blocks and the block-tiled kernels
 * from the real per-expert counts (a cost model fitted on MI355X); beyond,
 * the block-tiled kernels.  Beyond the bound nothing is computed
 * out of bounds: every output row is +0 and *local_pairs tells the caller the
 * count, so a caller that cannot guarantee its bound checks *local_pairs
 * after the call.  The byte range max_local_pairs*I (not T*topk*I) must stay
 * below 2^32.  Other arguments and errors as w4a8_fused_moe; INVALID_ARG for
 * an unknown format, a bound below 1 or a missing local_pairs.  T == 0
 * launches nothing and leaves *local_pairs untouched.
 */
int w4a8_fused_moe_bounded(const void* hidden_bf16, int64_t T, int64_t H, const int32_t* topk_ids,
                           const float* topk_weights, int64_t topk, int64_t expert_begin,
                           int64_t num_local_experts, int64_t I, int weight_format,
                           const uint8_t* w13, const void* w13_scales, const uint8_t* w2,
                           const void* w2_scales, int64_t max_local_pairs, int32_t* local_pairs,
                           void* out_bf16, void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * w4a8_fused_moe_persistent -- the fused forward with everything after the
 * align in ONE kernel launch (DeepGEMM PR #53, "Changes": a single persistent
 * kernel runs L1 GEMM -> SwiGLU -> per-token FP8 requant -> L2 GEMM ->
 * combine).  The align with the input quantisation runs first, as in
 * w4a8_fused_moe; then one cooperative launch of one workgroup per CU walks
 * the block-tiled gate_up tiles (160-row m-blocks, at every T), passes a
 * grid barrier, walks the down GEMM's tiles, passes a second barrier and
 * sums the tokens' rows.  Each barrier is an agent-scope release (the XCD's
 * L2 written back), an atomic arrival on a counter in the workspace (set to
 * 0 by the align), a wait bounded to ~2 s of wall-clock time, and an
 * agent-scope acquire.  (The bound only guarantees that the launch ends: all
 * workgroups are resident under the cooperative launch, so no wait comes
 * near it; were one to pass it, the launch would end without writing the
 * rest of the output.)
 *   The output is bit-identical to w4a8_fused_moe's (or the prepacked /
 *   fp4 exports') on the block-tiled path, i.e. whenever T*topk/E_l >= 256;
 *   below that it is the block-tiled path's result for the same inputs
 *   (same arithmetic per element; the multi-launch exports use the skinny
 *   kernel there).
 *   weight_format, w13/w2 and their scales as w4a8_fused_moe_bounded; other
 *   arguments, the workspace query (workspace == NULL) and errors as
 *   w4a8_fused_moe; W4A8_ERR_UNSUPPORTED also for H > 2^24.  W4A8_ERR_HIP
 *   also when the device cannot hold one workgroup per CU at once (the
 *   cooperative launch is refused).
 *   Calls with one workspace must not overlap (the barrier counter lives in
 *   it).  The call records into a HIP graph like the other exports (the
 *   align clears the counter on every replay).
 */
int w4a8_fused_moe_persistent(const void* hidden_bf16, int64_t T, int64_t H, const int32_t* topk_ids,
                              const float* topk_weights, int64_t topk, int64_t expert_begin,
                              int64_t num_local_experts, int64_t I, int weight_format,
                              const uint8_t* w13, const void* w13_scales, const uint8_t* w2,
                              const void* w2_scales, void* out_bf16, void* workspace,
                              size_t* workspace_bytes, hipStream_t stream);

/*
 * w4a8_fused_moe_prepacked_noalloc -- w4a8_fused_moe_prepacked for callers
 * that cannot allocate device memory or pass a workspace: code recorded into
 * a HIP graph, tight serving loops, harnesses that forbid hipMalloc.  The
 * call allocates nothing; its intermediates live in a file-scope device
 * array of W4A8_NOALLOC_SCRATCH_BYTES that every GPU the library runs on
 * holds until the process ends (its address is looked up once per device,
 * on the first call with that device current).
 *   Arguments, results and errors as w4a8_fused_moe_prepacked, without the
 *   workspace pair; the output is bit-identical to that export's.
 *   W4A8_ERR_WORKSPACE if the call needs more than W4A8_NOALLOC_SCRATCH_BYTES
 *   (the size w4a8_fused_moe_prepacked would query for the same shape; at
 *   H = 7168, I = 2048 that is T*topk up to about 2000 pairs); W4A8_ERR_HIP if
 *   the array's address cannot be obtained.
 * Every call on one GPU uses the same array and leaves its contents behind:
 * calls that may overlap on one GPU (other streams, other host threads) race
 * and must be ordered by the caller.
 */
#define W4A8_NOALLOC_SCRATCH_BYTES (64u << 20)
int w4a8_fused_moe_prepacked_noalloc(const void* hidden_bf16, int64_t T, int64_t H,
                                     const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                                     int64_t expert_begin, int64_t num_local_experts, int64_t I,
                                     const uint8_t* w13_packed, const float* w13_scales_packed,
                                     const uint8_t* w2_packed, const float* w2_scales_packed,
                                     void* out_bf16, hipStream_t stream);

/*
 * w4a8_fused_moe_workspace_layout -- where w4a8_fused_moe keeps its
 * intermediates inside the workspace (host-only query, no HIP call), so that
 * tests and tools can read them after a call:
 *   offsets[0]  expert_counts   int32 [E_l]
 *   offsets[1]  expert_offsets  int32 [E_l+1]
 *   offsets[2]  sorted_pair_ids int32 [T*topk]
 *   offsets[3]  src2dst         int32 [T*topk]
 *   offsets[4]  block_expert    int32 [nb]     offsets[5] block_row int32 [nb]
 *   offsets[6]  num_blocks      int32 [1]      (nb <= ceil(T*topk/block_m)+E_l)
 *   offsets[7]  gate_up operand: fp8 codes of the hidden states [T, H];
 *               inside each 128-group, 8-group b (k = 8b..8b+7) sits at byte
 *               16*(4*((b%4)/2) + b/4) + 8*(b%2), in K order
 *               k0,k2,k4,k6,k1,k3,k5,k7
 *   offsets[8]  float2 [T, H/128] {512*scale, -8*scale*sum of the block's
 *               decoded codes}
 *   offsets[9]  requantised intermediate: fp8 codes [T*topk, I] (pair rows
 *               in permuted order); inside each 128-group, 8-group b sits at
 *               byte 16*(4*((b%4)/2) + b/4) + 8*(b%2), in K order
 *               k0,k2,k4,k6,k1,k3,k5,k7
 *   offsets[10] float2 [T*topk, I/128] {512*scale, -8*scale*sum of the block's
 *               decoded codes} ([T*topk, I/g] under w4a8_fused_moe_recipe with
 *               a group g of 64 or 32; the region has room for I/32)
 *   offsets[11] down output fp32 [T*topk, H] (pair rows in permuted order)
 *   offsets[12..14] (n = 15) the second m-block list: block_expert2,
 *               block_row2 int32 [nb2], num_blocks2 int32 [1]; 0 when the
 *               call keeps one list
 * n must be 12, 15 or 18; *block_m receives the height of the m-blocks in the
 * first list.  Calls whose pairs per local expert (T*topk/E_l, every pair
 * counted as local) lie between 16 and 256 choose the height per expert on
 * the device: experts with at most 16 local pairs get 16-row blocks in the
 * first list, the others 32-row blocks in the second; and, while those lists
 * stay below 4096 blocks, the path too: with n = 18,
 *   offsets[15..17] block_row3 int32 [nb3] (160-row blocks), num_blocks3
 *               int32 [1], path int32 [1]: 1 if the call ran the block-tiled
 *               kernels on the third list, 0 if the skinny kernel on the
 *               first two; 0 when the call does not choose on the device
 */
int w4a8_fused_moe_workspace_layout(int64_t T, int64_t H, int64_t topk,
                                    int64_t num_local_experts, int64_t I,
                                    size_t* offsets, int n, int64_t* block_m);

/*
 * w4a8_fused_moe_stage_events -- profiling hook for a per-stage breakdown
 * (the five stages DeepGEMM PR #53 reports with its profile breakdown:
 * dispatch/align, L1 GEMM, act+quant, L2 GEMM, combine).
 *
 * Arms the NEXT w4a8_fused_moe call made on the calling host thread to
 * record events[i] (hipEvent_t handles created by the caller) on its stream:
 *   [0] before align  [1] after align  [2] after the input quantisation
 *   (the quantisation runs inside the align's launches, so [1] and [2] are
 *   both recorded after them)
 *   [3] after gate_up+SwiGLU+requant   [4] after down  [5] after combine
 * A null entry is skipped (so a caller can time one stage with two events).
 * n must be 6 (or 0 to disarm).  The six handles are copied, so the array
 * need not outlive this call; the events must stay valid until the armed
 * call has returned.  The next call of the fused family on this thread
 * consumes the arming whatever it does: a workspace-size query and a
 * rejected call disarm it too (and record nothing).  Never synchronises.
 * Returns W4A8_ERR_INVALID_ARG for a bad n or a null array.
 */
int w4a8_fused_moe_stage_events(void* const* events, int n);

#ifdef __cplusplus
}
#endif
#endif /* W4A8_H */
