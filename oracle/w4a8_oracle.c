/*
 * w4a8_oracle.c -- plain CPU oracle for the W4AFP8 fused-MoE forward.
 *
 * TEST INFRASTRUCTURE ONLY (see w4a8_oracle.h).  Built with
 * gcc -O2 -ffp-contract=off and without -ffast-math, so every float
 * operation below is one IEEE-754 operation rounded to nearest-even.
 */
#include "w4a8_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Codecs                                                                    */
/* ------------------------------------------------------------------------ */

/* OCP fp8 e4m3 ("fn": no infinities, 0x7F/0xFF are NaN, largest finite
 * magnitude 448 = 0x7E).  Field layout: sign | 4-bit exponent, bias 7 |
 * 3-bit mantissa.  Exponent field 0 encodes subnormals m * 2^-9. */
double orc_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* fp32 -> e4m3 with saturation to +-448 first ([P3]: the cast returns NaN
 * beyond the range, so the value is clamped before it), then round to the
 * nearest representable value, ties to the even code (even mantissa LSB),
 * subnormals kept.  The sign bit follows the input's sign (so -0 -> 0x80).
 *
 * The rounding is done by definition: the finite non-negative codes 0x00 ..
 * 0x7E decode to strictly increasing values, so the two neighbours of |v|
 * are found by bisection over the codes and the nearer one is kept; the
 * midpoint of two neighbours is exact in double, so the comparison is too. */
uint8_t orc_e4m3_encode(float v)
{
    int neg = signbit(v) ? 1 : 0;
    double a = fabs((double)v);
    if (a > 448.0)
        a = 448.0;

    int lo = 0, hi = 0x7E; /* invariant: decode(lo) <= a */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (orc_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo;
    if (c < 0x7E && orc_e4m3_decode((uint8_t)c) != a) {
        double below = orc_e4m3_decode((uint8_t)c);
        double above = orc_e4m3_decode((uint8_t)(c + 1));
        double midpoint = 0.5 * (below + above);
        if (a > midpoint || (a == midpoint && (c & 1)))
            c = c + 1;
    }
    return (uint8_t)(c | (neg << 7));
}

/* Signed int4 in a byte: k even in the low nibble, k odd in the high
 * nibble; two's complement, so a nibble n >= 8 stands for n - 16. */
int orc_int4_value(uint8_t byte, int odd)
{
    int n = odd ? (byte >> 4) : (byte & 0xF);
    return n >= 8 ? n - 16 : n;
}

/* OCP MX fp4 e2m1 ([P4] "Changes": packed FP4 (E2M1) expert weights).
 * Field layout of the nibble: sign | 2-bit exponent, bias 1 | 1-bit
 * mantissa; exponent field 0 encodes the subnormal m * 2^-1 (so 0 and 0.5),
 * otherwise (1 + m/2) * 2^(e-1).  No infinities or NaNs. */
double orc_e2m1_decode(uint8_t nibble)
{
    int sign = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 0x3;
    int m = nibble & 0x1;
    double mag = (e == 0) ? ldexp((double)m, -1) : ldexp(1.0 + (double)m / 2.0, e - 1);
    return sign ? -mag : mag;
}

/* OCP MX E8M0 scale ([P4] "Changes": per-32-K UE8M0 weight scales): an
 * unsigned power-of-two exponent with bias 127, 0xFF = NaN. */
double orc_ue8m0_decode(uint8_t e)
{
    if (e == 0xFF)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

double orc_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> bf16, round to nearest, ties to even, in one rounding (never
 * through fp32).  bf16 keeps 8 significant bits and the fp32 exponent
 * range: the quantum of a normal value v = m * 2^e (m in [0.5, 1)) is
 * 2^(e-8); below 2^-126 the quantum is the fixed subnormal step 2^-133. */
uint16_t orc_bf16_from_double(double v)
{
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int e;
        (void)frexp(a, &e);
        double quantum = (a >= ldexp(1.0, -126)) ? ldexp(1.0, e - 8) : ldexp(1.0, -133);
        r = nearbyint(a / quantum) * quantum; /* default mode: ties to even */
    }
    uint32_t u;
    if (r > (double)FLT_MAX) {
        u = 0x7F800000u; /* overflow rounds to infinity */
    } else {
        float f = (float)r; /* exact: r has at most 8 significant bits */
        memcpy(&u, &f, sizeof u);
    }
    if (neg)
        u |= 0x80000000u;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* Dynamic activation quantisation ([P4] UE8M0 note; [P3] saturation)        */
/* ------------------------------------------------------------------------ */

/* One 128-element block of one row, all in fp32:
 *   amax   = max |x|
 *   amax_c = max(amax, 1e-10f)   -- clamped before the reciprocal
 *   inv    = 448 / amax_c        -- IEEE fp32 divide
 *   scale  = amax_c / 448        -- the stored dequantisation scale
 *   code   = e4m3(fl32(x * inv)) */
void orc_quantize_block(const float* x, uint8_t* codes, float* scale)
{
    orc_quantize_block_n(x, ORC_GROUP, codes, scale);
}

/* the same rule over a block of n elements (the finer activation-scale
 * recipes of [P4]: one scale per 64 or per 32 K) */
void orc_quantize_block_n(const float* x, int n, uint8_t* codes, float* scale)
{
    float amax = 0.0f;
    for (int k = 0; k < n; ++k) {
        float m = fabsf(x[k]);
        if (m > amax)
            amax = m;
    }
    float amax_c = amax > 1e-10f ? amax : 1e-10f;
    float inv = 448.0f / amax_c;
    *scale = amax_c / 448.0f;
    for (int k = 0; k < n; ++k) {
        float p = x[k] * inv;
        codes[k] = orc_e4m3_encode(p);
    }
}

/* The static variant: one per-tensor scale s, fixed ahead of time (the input
 * scales [P2] loads with the weights) instead of each block's amax/448.  The
 * codes follow the same reciprocal-then-multiply rule with inv = 1/s rounded
 * once to fp32, and s is every block's dequant scale. */
void orc_quantize_block_static(const float* x, float s, uint8_t* codes)
{
    orc_quantize_block_static_n(x, ORC_GROUP, s, codes);
}

void orc_quantize_block_static_n(const float* x, int n, float s, uint8_t* codes)
{
    float inv = 1.0f / s;
    for (int k = 0; k < n; ++k) {
        float p = x[k] * inv;
        codes[k] = orc_e4m3_encode(p);
    }
}

/* rows of K in blocks of n (n divides 128), dynamic or with a static scale */
static void quantize_rows_f32_n(const float* x, int64_t M, int64_t K, int n, const float* s,
                                uint8_t* codes, float* scales)
{
    int64_t G = K / n;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < G; ++g) {
            if (s) {
                orc_quantize_block_static_n(x + m * K + g * n, n, *s, codes + m * K + g * n);
                scales[m * G + g] = *s;
            } else {
                orc_quantize_block_n(x + m * K + g * n, n, codes + m * K + g * n, scales + m * G + g);
            }
        }
}

static void quantize_rows_f32_any(const float* x, int64_t M, int64_t K, const float* s,
                                  uint8_t* codes, float* scales)
{
    quantize_rows_f32_n(x, M, K, ORC_GROUP, s, codes, scales);
}

static void quantize_rows_bf16_any(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   const float* s, uint8_t* codes, float* scales)
{
    int64_t G = K / ORC_GROUP;
    float block[ORC_GROUP];
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < G; ++g) {
            for (int k = 0; k < ORC_GROUP; ++k)
                block[k] = (float)orc_bf16_to_double(x[m * ldx + g * ORC_GROUP + k]);
            quantize_rows_f32_any(block, 1, ORC_GROUP, s, codes + m * K + g * ORC_GROUP,
                                  scales + m * G + g);
        }
}

void orc_quantize_rows_bf16_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float s,
                                   uint8_t* codes, float* scales)
{
    quantize_rows_bf16_any(x, M, K, ldx, &s, codes, scales);
}

void orc_quantize_rows_f32(const float* x, int64_t M, int64_t K,
                           uint8_t* codes, float* scales)
{
    int64_t G = K / ORC_GROUP;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < G; ++g)
            orc_quantize_block(x + m * K + g * ORC_GROUP,
                               codes + m * K + g * ORC_GROUP,
                               scales + m * G + g);
}

void orc_quantize_rows_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* codes, float* scales)
{
    int64_t G = K / ORC_GROUP;
    float block[ORC_GROUP];
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < G; ++g) {
            for (int k = 0; k < ORC_GROUP; ++k)
                block[k] = (float)orc_bf16_to_double(x[m * ldx + g * ORC_GROUP + k]);
            orc_quantize_block(block, codes + m * K + g * ORC_GROUP, scales + m * G + g);
        }
}

/* ------------------------------------------------------------------------ */
/* Routing permutation ([P2] review threads on run_cutlass_moe_ep_preproess  */
/* and expert_map)                                                           */
/* ------------------------------------------------------------------------ */

/* Pair f = t*topk + j routes token t to expert topk_ids[f].  It is local when
 * l = topk_ids[f] - expert_begin lies in [0, E_l).  The local pairs are put
 * in the order of a stable sort by l (ties keep ascending f); offsets is the
 * exclusive prefix sum of the per-expert counts (seg_indptr); src2dst[f] is
 * the position of f in that order (-1 when f is not local).  Each expert's
 * segment is then cut into blocks of block_m rows, the last one partial. */
int orc_moe_align(const int32_t* topk_ids, int64_t T, int64_t topk,
                  int64_t expert_begin, int64_t num_local_experts, int64_t block_m,
                  int32_t* expert_counts, int32_t* expert_offsets,
                  int32_t* sorted_pair_ids, int32_t* src2dst,
                  int32_t* block_expert, int32_t* block_row, int32_t* num_blocks)
{
    int64_t E = num_local_experts;
    int64_t F = T * topk;
    if (T < 0 || topk <= 0 || E <= 0 || block_m <= 0)
        return 1;

    for (int64_t e = 0; e < E; ++e)
        expert_counts[e] = 0;
    for (int64_t f = 0; f < F; ++f) {
        int64_t l = (int64_t)topk_ids[f] - expert_begin;
        if (l >= 0 && l < E)
            expert_counts[l] += 1;
    }

    expert_offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e)
        expert_offsets[e + 1] = expert_offsets[e] + expert_counts[e];

    /* counting sort; visiting f in ascending order keeps it stable */
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor)
        return 2;
    for (int64_t e = 0; e < E; ++e)
        cursor[e] = expert_offsets[e];
    for (int64_t f = 0; f < F; ++f) {
        int64_t l = (int64_t)topk_ids[f] - expert_begin;
        if (l >= 0 && l < E) {
            int32_t pos = cursor[l]++;
            sorted_pair_ids[pos] = (int32_t)f;
            src2dst[f] = pos;
        } else {
            src2dst[f] = -1;
        }
    }
    free(cursor);

    int32_t nb = 0;
    for (int64_t e = 0; e < E; ++e)
        for (int32_t r = 0; r < expert_counts[e]; r += (int32_t)block_m) {
            if (block_expert)
                block_expert[nb] = (int32_t)e;
            if (block_row)
                block_row[nb] = expert_offsets[e] + r;
            nb += 1;
        }
    if (num_blocks)
        *num_blocks = nb;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* W4A8 GEMM ([P2] w4a8 grouped GEMM, group size 128)                        */
/* ------------------------------------------------------------------------ */

/* y[m, n] = sum_g sa[m, g] * sw[n, g] * acc_g(m, n),
 * acc_g(m, n) = sum_{k in group g} dec(a[m, k]) * int4(w[n, k]).
 * acc_g is exact in fp64 (each product has at most 8 significant bits and
 * spans 2^-9 .. 2^12, a 128-term sum stays well inside 53 bits); the groups
 * are added in ascending order in fp64. */
void orc_gemm_f64(const uint8_t* a, const float* sa, int64_t M, int64_t K,
                  const uint8_t* w, const float* sw, int64_t N, double* y)
{
    int64_t G = K / ORC_GROUP;
    double* arow = (double*)malloc(sizeof(double) * (size_t)K);
    if (!arow)
        return;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k)
            arow[k] = orc_e4m3_decode(a[m * K + k]);
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* wrow = w + n * (K / 2);
            double total = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double acc = 0.0;
                for (int64_t k = g * ORC_GROUP; k < (g + 1) * ORC_GROUP; ++k)
                    acc += arow[k] * (double)orc_int4_value(wrow[k / 2], (int)(k & 1));
                total += acc * ((double)sa[m * G + g] * (double)sw[n * G + g]);
            }
            y[m * N + n] = total;
        }
    }
    free(arow);
}

void orc_gemm_bf16(const uint8_t* a, const float* sa, int64_t M, int64_t K,
                   const uint8_t* w, const float* sw, int64_t N, uint16_t* out)
{
    double* y = (double*)malloc(sizeof(double) * (size_t)(M * N));
    if (!y)
        return;
    orc_gemm_f64(a, sa, M, K, w, sw, N, y);
    for (int64_t i = 0; i < M * N; ++i)
        out[i] = orc_bf16_from_double(y[i]);
    free(y);
}

/* W4A8 GEMM with fp4 weights: each weight is its e2m1 value times the UE8M0
 * scale of its 32-K block; the activation scale still applies per 128-K
 * group.  y[m,n] = sum_g sa[m,g] * sum_{k in g} a[m,k] * w[n,k] * sw[n,k/32],
 * every group sum exact in fp64 for these operands. */
void orc_gemm_fp4_f64(const uint8_t* a, const float* sa, int64_t M, int64_t K,
                      const uint8_t* w, const uint8_t* sw, int64_t N, double* y)
{
    int64_t G = K / ORC_GROUP;
    int64_t B = K / ORC_FP4_BLOCK;
    /* the codecs tabulated once (16 and 256 entries), for speed only */
    double vtab[16], stab[256];
    for (int c = 0; c < 16; ++c)
        vtab[c] = orc_e2m1_decode((uint8_t)c);
    for (int e = 0; e < 256; ++e)
        stab[e] = orc_ue8m0_decode((uint8_t)e);
    double* arow = (double*)malloc(sizeof(double) * (size_t)K);
    if (!arow)
        return;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k)
            arow[k] = orc_e4m3_decode(a[m * K + k]);
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* wrow = w + n * (K / 2);
            const uint8_t* srow = sw + n * B;
            double total = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double acc = 0.0;
                for (int64_t k = g * ORC_GROUP; k < (g + 1) * ORC_GROUP; ++k) {
                    const uint8_t nib = (k & 1) ? (uint8_t)(wrow[k / 2] >> 4) : (uint8_t)(wrow[k / 2] & 0xF);
                    acc += arow[k] * (vtab[nib] * stab[srow[k / ORC_FP4_BLOCK]]);
                }
                total += acc * (double)sa[m * G + g];
            }
            y[m * N + n] = total;
        }
    }
    free(arow);
}

/* The GEMM with the activation scales per ag-block of K (ag divides 128;
 * [P4]'s 128/64 and per-32 activation recipes): each 128-K weight group's sum
 * splits into its ag-blocks, each block sum promoted with its own activation
 * scale and the group's weight scale.  Weights: int4 with fp32 scales sw
 * [N, K/128] (sb NULL), or fp4 with UE8M0 bytes sb [N, K/32] (sw NULL).
 *   y[m,n] = sum_g sum_{b in g} sa[m,b] * s_w(n,g) * sum_{k in b} a[m,k] * w[n,k] */
void orc_gemm_ag_f64(const uint8_t* a, const float* sa, int64_t ag, int64_t M, int64_t K,
                     const uint8_t* w, const float* sw, const uint8_t* sb, int64_t N, double* y)
{
    int64_t G = K / ORC_GROUP, NB = K / ag;
    /* the fp4 codecs tabulated once, for speed only */
    double vtab[16], stab[256];
    for (int c = 0; c < 16; ++c)
        vtab[c] = orc_e2m1_decode((uint8_t)c);
    for (int e = 0; e < 256; ++e)
        stab[e] = orc_ue8m0_decode((uint8_t)e);
    double* arow = (double*)malloc(sizeof(double) * (size_t)K);
    if (!arow)
        return;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k)
            arow[k] = orc_e4m3_decode(a[m * K + k]);
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* wrow = w + n * (K / 2);
            double total = 0.0;
            for (int64_t g = 0; g < G; ++g)
                for (int64_t b = g * (ORC_GROUP / ag); b < (g + 1) * (ORC_GROUP / ag); ++b) {
                    double acc = 0.0;
                    for (int64_t k = b * ag; k < (b + 1) * ag; ++k) {
                        double wv;
                        if (sb)
                            wv = vtab[(k & 1) ? (wrow[k / 2] >> 4) : (wrow[k / 2] & 0xF)] *
                                 stab[sb[n * (K / ORC_FP4_BLOCK) + k / ORC_FP4_BLOCK]];
                        else
                            wv = (double)orc_int4_value(wrow[k / 2], (int)(k & 1));
                        acc += arow[k] * wv;
                    }
                    total += acc * (sb ? (double)sa[m * NB + b]
                                       : (double)sa[m * NB + b] * (double)sw[n * G + g]);
                }
            y[m * N + n] = total;
        }
    }
    free(arow);
}

/* ------------------------------------------------------------------------ */
/* SwiGLU between the GEMMs ([P2] "Cutlass W4A8 MoE": SiLU and Mul; [P4]    */
/* "Changes": L1 GEMM -> SwiGLU)                                             */
/* ------------------------------------------------------------------------ */

/* h[i] = silu(gate[i]) * up[i] with silu(g) = g * sigmoid(g) = g / (1 + e^-g),
 * evaluated in fp64 (exp from libm), then rounded once to fp32: the value
 * the requantisation step reads.  No clamp of g (plain SwiGLU). */
void orc_swiglu(const double* gate, const double* up, int64_t n, float* h)
{
    for (int64_t i = 0; i < n; ++i) {
        double g = gate[i];
        double silu = g / (1.0 + exp(-g));
        h[i] = (float)(silu * up[i]);
    }
}

/* ------------------------------------------------------------------------ */
/* The fused-MoE forward ([P2] "Cutlass W4A8 MoE" workflow; [P4] "Changes") */
/* ------------------------------------------------------------------------ */

/* fp4: weights e2m1 with UE8M0 scales per 32 K (s13 [E,2I,H/32], s2
 * [E,H,I/32] bytes); otherwise int4 with fp32 scales per 128 K. */
static int fused_moe_impl(const uint16_t* hidden, int64_t T, int64_t H,
                          const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                          int64_t expert_begin, int64_t num_local_experts, int64_t I,
                          const uint8_t* w13, const void* s13,
                          const uint8_t* w2, const void* s2, int fp4,
                          const float* a1_scale, const float* a2_scale, int down_group,
                          uint16_t* out,
                          uint8_t* qh_out, float* sh_out, double* y2_out)
{
    int64_t E = num_local_experts;
    int64_t F = T * topk;
    int64_t GH = H / ORC_GROUP, GI = I / down_group;
    if (down_group != 128 && down_group != 64 && down_group != 32)
        return 1;
    if (T < 0 || H <= 0 || I <= 0 || topk <= 0 || E <= 0 || H % ORC_GROUP || I % ORC_GROUP)
        return 1;

    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* sorted = (int32_t*)malloc(sizeof(int32_t) * (size_t)(F > 0 ? F : 1));
    int32_t* src2dst = (int32_t*)malloc(sizeof(int32_t) * (size_t)(F > 0 ? F : 1));
    uint8_t* qx = (uint8_t*)malloc((size_t)(T * H > 0 ? T * H : 1));
    float* sx = (float*)malloc(sizeof(float) * (size_t)(T * GH > 0 ? T * GH : 1));
    double* y1 = (double*)malloc(sizeof(double) * (size_t)(2 * I));
    float* h32 = (float*)malloc(sizeof(float) * (size_t)I);
    uint8_t* qh = (uint8_t*)malloc((size_t)I);
    float* sh = (float*)malloc(sizeof(float) * (size_t)GI);
    double* y2 = NULL;
    int rc = 2;
    if (!counts || !offsets || !sorted || !src2dst || !qx || !sx || !y1 || !h32 || !qh || !sh)
        goto done;

    /* 1. permutation of the local pairs (stable sort by local expert) */
    rc = orc_moe_align(topk_ids, T, topk, expert_begin, E, 1, counts, offsets, sorted,
                       src2dst, NULL, NULL, NULL);
    if (rc)
        goto done;
    rc = 2;
    y2 = (double*)malloc(sizeof(double) * (size_t)((offsets[E] > 0 ? offsets[E] : 1) * H));
    if (!y2)
        goto done;

    /* 2. dynamic per-token-per-128 quantisation of the hidden states */
    quantize_rows_bf16_any(hidden, T, H, H, a1_scale, qx, sx);

    /* 3.-6. per local pair, in permuted order: gather the token's row,
     * gate_up GEMM, SwiGLU, requantise, down GEMM */
    for (int64_t e = 0; e < E; ++e) {
        const uint8_t* w13e = w13 + e * (2 * I) * (H / 2);
        const uint8_t* w2e = w2 + e * H * (I / 2);
        const float* s13e = fp4 ? NULL : (const float*)s13 + e * (2 * I) * GH;
        const float* s2e = fp4 ? NULL : (const float*)s2 + e * H * (I / ORC_GROUP);
        const uint8_t* b13e = fp4 ? (const uint8_t*)s13 + e * (2 * I) * (H / ORC_FP4_BLOCK) : NULL;
        const uint8_t* b2e = fp4 ? (const uint8_t*)s2 + e * H * (I / ORC_FP4_BLOCK) : NULL;
        for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p) {
            int64_t t = sorted[p] / topk;
            /* 3. GEMM1: y1 = gate_up(x_t), 2I outputs */
            if (fp4)
                orc_gemm_fp4_f64(qx + t * H, sx + t * GH, 1, H, w13e, b13e, 2 * I, y1);
            else
                orc_gemm_f64(qx + t * H, sx + t * GH, 1, H, w13e, s13e, 2 * I, y1);
            /* 4. SwiGLU: gate rows [0, I), up rows [I, 2I) */
            orc_swiglu(y1, y1 + I, I, h32);
            /* 5. requantise with the same per-128 rule as the input */
            quantize_rows_f32_n(h32, 1, I, (int)down_group, a2_scale, qh, sh);
            if (qh_out)
                memcpy(qh_out + p * I, qh, (size_t)I);
            if (sh_out)
                memcpy(sh_out + p * GI, sh, sizeof(float) * (size_t)GI);
            /* 6. GEMM2: y2 = down(h), H outputs */
            if (down_group != ORC_GROUP)
                orc_gemm_ag_f64(qh, sh, down_group, 1, I, w2e, s2e, b2e, H, y2 + p * H);
            else if (fp4)
                orc_gemm_fp4_f64(qh, sh, 1, I, w2e, b2e, H, y2 + p * H);
            else
                orc_gemm_f64(qh, sh, 1, I, w2e, s2e, H, y2 + p * H);
        }
    }
    if (y2_out)
        memcpy(y2_out, y2, sizeof(double) * (size_t)(offsets[E] * H));

    /* 7. combine: un-permute, weight by the routing weight, sum the token's
     * local pairs in ascending j, one rounding to bf16 */
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < H; ++n) {
            double s = 0.0;
            for (int64_t j = 0; j < topk; ++j) {
                int32_t p = src2dst[t * topk + j];
                if (p >= 0)
                    s += (double)topk_weights[t * topk + j] * y2[(int64_t)p * H + n];
            }
            out[t * H + n] = orc_bf16_from_double(s);
        }
    rc = 0;

done:
    free(counts);
    free(offsets);
    free(sorted);
    free(src2dst);
    free(qx);
    free(sx);
    free(y1);
    free(h32);
    free(qh);
    free(sh);
    free(y2);
    return rc;
}

int orc_fused_moe(const uint16_t* hidden, int64_t T, int64_t H,
                  const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                  int64_t expert_begin, int64_t num_local_experts, int64_t I,
                  const uint8_t* w13, const float* s13,
                  const uint8_t* w2, const float* s2,
                  uint16_t* out,
                  uint8_t* qh_out, float* sh_out, double* y2_out)
{
    return fused_moe_impl(hidden, T, H, topk_ids, topk_weights, topk, expert_begin,
                          num_local_experts, I, w13, s13, w2, s2, 0, NULL, NULL, ORC_GROUP, out, qh_out,
                          sh_out, y2_out);
}

int orc_fused_moe_static(const uint16_t* hidden, int64_t T, int64_t H,
                         const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                         int64_t expert_begin, int64_t num_local_experts, int64_t I,
                         const uint8_t* w13, const float* s13,
                         const uint8_t* w2, const float* s2,
                         const float* a1_scale, const float* a2_scale,
                         uint16_t* out,
                         uint8_t* qh_out, float* sh_out, double* y2_out)
{
    return fused_moe_impl(hidden, T, H, topk_ids, topk_weights, topk, expert_begin,
                          num_local_experts, I, w13, s13, w2, s2, 0, a1_scale, a2_scale, ORC_GROUP, out,
                          qh_out, sh_out, y2_out);
}

int orc_fused_moe_fp4(const uint16_t* hidden, int64_t T, int64_t H,
                      const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                      int64_t expert_begin, int64_t num_local_experts, int64_t I,
                      const uint8_t* w13, const uint8_t* s13,
                      const uint8_t* w2, const uint8_t* s2,
                      uint16_t* out,
                      uint8_t* qh_out, float* sh_out, double* y2_out)
{
    if (H % ORC_FP4_BLOCK || I % ORC_FP4_BLOCK)
        return 1;
    return fused_moe_impl(hidden, T, H, topk_ids, topk_weights, topk, expert_begin,
                          num_local_experts, I, w13, s13, w2, s2, 1, NULL, NULL, ORC_GROUP, out, qh_out,
                          sh_out, y2_out);
}

int orc_fused_moe_recipe(const uint16_t* hidden, int64_t T, int64_t H,
                         const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                         int64_t expert_begin, int64_t num_local_experts, int64_t I,
                         int fp4, const uint8_t* w13, const void* s13,
                         const uint8_t* w2, const void* s2, int down_act_group,
                         uint16_t* out,
                         uint8_t* qh_out, float* sh_out, double* y2_out)
{
    if (fp4 && (H % ORC_FP4_BLOCK || I % ORC_FP4_BLOCK))
        return 1;
    return fused_moe_impl(hidden, T, H, topk_ids, topk_weights, topk, expert_begin,
                          num_local_experts, I, w13, s13, w2, s2, fp4 ? 1 : 0, NULL, NULL,
                          down_act_group, out, qh_out, sh_out, y2_out);
}
