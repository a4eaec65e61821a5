/*
 * w4a8_oracle.h -- plain CPU oracle for the W4AFP8 fused-MoE forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this code: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * Every routine is the plain definition of one step of the method, written
 * for readability: single-threaded, fp64 where the method accumulates, and
 * no blocking, fusion or reordering beyond what the definition states.
 *
 * Sources (page title, then the passage):
 *   [P2] SGLang PR #7762 "feat: support DeepSeek-R1-W4AFP8 model with ep-moe
 *        mode" -- "Model Info" (INT4 expert weights, FP8 activations),
 *        "Cutlass W4A8 MoE" / "Kernel" (pre-reorder, w4a8 grouped GEMMs,
 *        SiLU-and-Mul, post-reorder), the review thread on
 *        run_cutlass_moe_ep_preproess (stable sort of the local top-k ids,
 *        seg_indptr, src2dst), the review thread on expert_map, and the
 *        review thread on the hard-coded group size 128.
 *   [P3] SGLang PR #37796 "feat(moe_wna16): 2-bit experts, expert streaming,
 *        N-contiguous GEMV" -- part-1 notes on the fp8 KV write path
 *        (saturate to +-448 before the e4m3 cast).
 *   [P4] DeepGEMM PR #53 "SM90 (Hopper) FP4 MegaMoE fused kernel with swapAB
 *        small-batch path" -- commit note dropping the UE8M0 activation scale
 *        (fp32 per-token activation scales; amax clamped before the
 *        reciprocal 448/amax) and the "Changes" list (L1 GEMM -> SwiGLU ->
 *        per-token FP8 requant -> L2 GEMM -> combine; FP8 E4M3 activations
 *        x packed FP4 E2M1 expert weights with per-32-K UE8M0 weight scales).
 *
 * Readings where the pages are silent (each fixed by the project spec):
 *   - amax clamp constant 1e-10f; dequant scale amax_c/448; codes use the
 *     reciprocal inv = 448/amax_c.
 *   - int4: two's complement nibbles, low nibble = even k, no zero point.
 *   - gate rows [0, I), up rows [I, 2I) of w13; plain SwiGLU (no clamp).
 *   - top-k weights applied in the combine, after the down GEMM.
 *   - non-local top-k ids are skipped; a token with no local pair outputs +0.
 *   - static activation scales (the input scales [P2] loads with the
 *     weights): one per-tensor fp32 s per quantisation point; codes use
 *     inv = 1/s rounded to fp32, then the same multiply, clamp and rounding.
 *   - fp4 weights: e2m1 and E8M0 as the OCP MX formats define them; nibble
 *     order as for int4; one scale byte per 32 consecutive K of a row
 *     (s [E_l, N, K/32]); activations keep their per-128 fp32 scales.
 *
 * Layouts (row-major, K contiguous):
 *   activations bf16 [T, H] (uint16 bit patterns);
 *   w13 [E_l, 2I, H/2] bytes, s13 [E_l, 2I, H/128] fp32;
 *   w2  [E_l, H, I/2] bytes,  s2  [E_l, H, I/128] fp32.
 */
#ifndef W4A8_ORACLE_H
#define W4A8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_GROUP 128
#define ORC_FP4_BLOCK 32

/* ---- codecs ---- */
double   orc_e4m3_decode(uint8_t code);
uint8_t  orc_e4m3_encode(float v);
int      orc_int4_value(uint8_t byte, int odd);
double   orc_e2m1_decode(uint8_t nibble);
double   orc_ue8m0_decode(uint8_t e);
double   orc_bf16_to_double(uint16_t bits);
uint16_t orc_bf16_from_double(double v);

/* ---- step: dynamic per-token-per-128 activation quantisation ---- */
void orc_quantize_block(const float* x, uint8_t* codes, float* scale);
void orc_quantize_block_n(const float* x, int n, uint8_t* codes, float* scale);
void orc_quantize_rows_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* codes, float* scales);
void orc_quantize_rows_f32(const float* x, int64_t M, int64_t K,
                           uint8_t* codes, float* scales);
/* static per-tensor scale s: codes = e4m3(clamp(x * fl32(1/s))), scales = s */
void orc_quantize_block_static(const float* x, float s, uint8_t* codes);
void orc_quantize_block_static_n(const float* x, int n, float s, uint8_t* codes);
void orc_quantize_rows_bf16_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float s,
                                   uint8_t* codes, float* scales);

/* ---- step: routing permutation (align) ---- */
int orc_moe_align(const int32_t* topk_ids, int64_t T, int64_t topk,
                  int64_t expert_begin, int64_t num_local_experts, int64_t block_m,
                  int32_t* expert_counts, int32_t* expert_offsets,
                  int32_t* sorted_pair_ids, int32_t* src2dst,
                  int32_t* block_expert, int32_t* block_row, int32_t* num_blocks);

/* ---- step: W4A8 GEMM with per-group scale promotion ---- */
void orc_gemm_f64(const uint8_t* a, const float* sa, int64_t M, int64_t K,
                  const uint8_t* w, const float* sw, int64_t N, double* y);
void orc_gemm_bf16(const uint8_t* a, const float* sa, int64_t M, int64_t K,
                   const uint8_t* w, const float* sw, int64_t N, uint16_t* out);
/* activation scales sa [M, K/ag] per ag-block (ag in {128, 64, 32}); int4
 * weights with sw [N, K/128] (sb NULL) or fp4 with sb [N, K/32] (sw NULL) */
void orc_gemm_ag_f64(const uint8_t* a, const float* sa, int64_t ag, int64_t M, int64_t K,
                     const uint8_t* w, const float* sw, const uint8_t* sb, int64_t N, double* y);
/* fp4 weights w [N, K/2] (e2m1 nibbles), UE8M0 scales sw [N, K/32] */
void orc_gemm_fp4_f64(const uint8_t* a, const float* sa, int64_t M, int64_t K,
                      const uint8_t* w, const uint8_t* sw, int64_t N, double* y);

/* ---- step: SwiGLU, h = silu(gate) * up in fp64, rounded once to fp32 ---- */
void orc_swiglu(const double* gate, const double* up, int64_t n, float* h);

/* ---- the whole forward: align, quant, GEMM1, SwiGLU, requant, GEMM2, combine ----
 * qh [P, I], sh [P, I/128] and y2 [P, H] (pair order = sorted order) are
 * optional diagnostic outputs; pass NULL to skip.  P <= T*topk. */
int orc_fused_moe(const uint16_t* hidden, int64_t T, int64_t H,
                  const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                  int64_t expert_begin, int64_t num_local_experts, int64_t I,
                  const uint8_t* w13, const float* s13,
                  const uint8_t* w2, const float* s2,
                  uint16_t* out,
                  uint8_t* qh, float* sh, double* y2);
/* the forward with static per-tensor activation scales: a1_scale for the
 * hidden states, a2_scale for the SwiGLU output (host pointers to one fp32;
 * NULL keeps that quantisation dynamic) */
int orc_fused_moe_static(const uint16_t* hidden, int64_t T, int64_t H,
                         const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                         int64_t expert_begin, int64_t num_local_experts, int64_t I,
                         const uint8_t* w13, const float* s13,
                         const uint8_t* w2, const float* s2,
                         const float* a1_scale, const float* a2_scale,
                         uint16_t* out,
                         uint8_t* qh, float* sh, double* y2);
/* the forward with the down GEMM's input quantised per down_act_group
 * (128, 64 or 32) K instead of 128 ([P4]'s 128/64 and per-32 activation
 * recipes); int4 (fp4 = 0, fp32 scales) or fp4 (UE8M0) weights; sh [P,
 * I/down_act_group] */
int orc_fused_moe_recipe(const uint16_t* hidden, int64_t T, int64_t H,
                         const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                         int64_t expert_begin, int64_t num_local_experts, int64_t I,
                         int fp4, const uint8_t* w13, const void* s13,
                         const uint8_t* w2, const void* s2, int down_act_group,
                         uint16_t* out,
                         uint8_t* qh, float* sh, double* y2);
/* the same forward on fp4 weights: s13 [E_l, 2I, H/32], s2 [E_l, H, I/32]
 * UE8M0 bytes; H and I multiples of 128 */
int orc_fused_moe_fp4(const uint16_t* hidden, int64_t T, int64_t H,
                      const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                      int64_t expert_begin, int64_t num_local_experts, int64_t I,
                      const uint8_t* w13, const uint8_t* s13,
                      const uint8_t* w2, const uint8_t* s2,
                      uint16_t* out,
                      uint8_t* qh, float* sh, double* y2);

#ifdef __cplusplus
}
#endif
#endif
