// common.hpp -- device helpers shared by the libw4a8 kernels (gfx950 / CDNA4).
//
// Conventions used by every kernel of the library:
//
//  * fp8 is OCP e4m3 (max 448).  Quantising one 128-wide block of a row
//    (DeepGEMM PR #53, commit note dropping UE8M0; SGLang PR #37796, part-1
//    fp8 KV notes): amax -> max(amax, 1e-10f) -> inv = 448/amax_c,
//    scale = amax_c/448 -> code = e4m3(clamp(x*inv, +-448)), round to nearest
//    even.  gfx950's v_cvt_pk_fp8_f32 rounds to nearest even into OCP e4m3
//    and keeps subnormals; the clamp comes first because the conversion does
//    not saturate.
//
//  * int4 -> fp8 without a table.  A weight nibble n (two's complement value
//    v = n - 16*(n >= 8)) is turned into u = n ^ 8 = v + 8 in 0..15, and the
//    byte u is used directly as an e4m3 code: codes 0x00..0x0F are exactly
//    u * 2^-9 (subnormals 0..7, then the first binade 8..15).  So one MFMA
//    over a 128-group returns raw = 2^-9 * sum_k a_k * (v_k + 8) and
//        sum_k a_k * v_k = 512 * raw - 8 * S,   S = sum_k a_k.
//    S is produced with the activation codes by the quantiser, and the
//    promotion of each group folds both constants into one FMA:
//        y += w_scale * fma(raw, c1, c0),  c1 = 512*a_scale, c0 = -8*a_scale*S.
//
//  * Internal fp8 activation layout (down / dense operand).  The unpack of
//    one packed dword x (8 nibbles k0..k7) gives lo = bytes k0,k2,k4,k6 and
//    hi = k1,k3,k5,k7, so activation codes are stored in that order inside
//    every aligned group of 8 K-positions: the bytes an MFMA lane holds for
//    the weights and for the activations always name the same k.  The 16
//    such 8-groups of a 128-group are then placed so that one 16-byte load
//    per lane reads 64 contiguous bytes per row: 8-group b (k = 8b..8b+7) sits
//    at byte 16*(4*((b%4)/2) + b/4) + 8*(b%2) of the group (fp8_group_pos).
//    Per-row-per-group side data is float2 {c1, c0}.
//
//  * The gate_up GEMMs use the same fp8 operand layout and side data, and
//    convert both operands exactly to fp16 in registers (the weight codes
//    u * 2^-9 and every e4m3 value are fp16 numbers) for the fp16 MFMA, whose
//    group sums are correctly rounded.
//
//  * MFMA v_mfma_f32_16x16x128_f8f6f4 (fp8 x fp8): lane l holds row l%16 of
//    A and column l%16 of B, 32 K-bytes each (the lane's quarter q = l/16 of
//    the 128-group); the result D[4*q + r][l%16] sits in register r.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;

// Prepacked weights (w4a8_prepack_weights): 16-row fragments, and inside a
// fragment one 1 KB block per 128-K group, so that the 64 lanes of one load
// read 1 KB contiguous.  Packed bytes of row n, group g at
//   ((n/16 * G + g) * 16 + n%16) * 64.
// Scales: blocks of 4 groups, 16 bytes per row, zero past the last group:
// the scale of row n, group g at float index
//   ((n/16 * G4 + g/4) * 16 + n%16) * 4 + g%4,   G4 = ceil(G/4).
// fp4 weights (w4a8_prepack_weights_fp4) use the same blocks; their scale
// elements are dwords holding the four UE8M0 bytes of a row's group, and for
// the gate_up GEMM the nibbles of every weight dword are reordered to
// k0,k2,k4,k6,k1,k3,k5,k7, the order of the fp8 activation operand.
__host__ __device__ constexpr int64_t packed_groups4(int64_t G)
{
    return (G + 3) / 4;
}

// byte offset of 8-group b (k = 8b..8b+7) inside a 128-byte fp8 activation group
__host__ __device__ constexpr int fp8_group_pos(int b)
{
    return 16 * (4 * ((b % 4) / 2) + b / 4) + 8 * (b % 2);
}

// One 16x16x128 fp8 MFMA (no block scales).
__device__ __forceinline__ v4f mfma16x16x128(const v8i& a, const v8i& b, const v4f& c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// One 16x16x32 f16 MFMA.  Unlike the fp8 forms, whose internal adder keeps
// only ~13 bits below the largest product of a lane's slice, the f16 MFMA
// returns the exactly rounded fp32 sum for these operands (int4 x e4m3
// values), which the gate_up GEMM needs: its output is re-quantised to fp8,
// and a relative error of a few 1e-6 there flips enough codes to move the
// final output by ~1e-3.
__device__ __forceinline__ v4f mfma16x16x32_f16(const v8h& a, const v8h& b, const v4f& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// v_bitop3_b32 computing ((x ^ k) & m) | c for constant k, m, c in one
// instruction: with A = ~m and B = (m & k) | (~m & c), the 3-input function
// F(x, A, B) = A ? B : x ^ B (truth table 0x9A for inputs ordered x, A, B)
// yields x, ~x, 0 or 1 bit by bit as required.
template <uint32_t K, uint32_t M, uint32_t C>
__device__ __forceinline__ uint32_t xor_and_or(uint32_t x)
{
    constexpr uint32_t A = ~M, B = (M & K) | (~M & C);
    return __builtin_amdgcn_bitop3_b32(x, A, B, 0x9A);
}

// 16 bytes of packed int4 (32 nibbles) -> 32 fp8 bytes (u * 2^-9 codes) in
// the K-interleaved order described above.
__device__ __forceinline__ v8i unpack_int4_u(const v4i& w)
{
    v8i r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = (uint32_t)w[i];
        r[2 * i] = (int)xor_and_or<0x08080808u, 0x0F0F0F0Fu, 0u>(x);
        r[2 * i + 1] = (int)xor_and_or<0x08080808u, 0x0F0F0F0Fu, 0u>(x >> 4);
    }
    return r;
}

// two fp8 dwords (4 + 4 codes) -> 8 exact halves, in dword order (e4m3
// values, the u * 2^-9 weight codes included, are all exact in fp16)
__device__ __forceinline__ v8h fp8x8_to_f16(uint32_t d0, uint32_t d1)
{
    const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
    const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
    const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
    const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
    return v8h{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// one dword of 8 fp4 (e2m1) codes, low nibble first, each times a power-of-two
// scale -> 8 halves in nibble order (exact while the scaled values stay in
// f16's range, down to its subnormals)
__device__ __forceinline__ v8h fp4x8_to_f16(uint32_t d, float scale)
{
    const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 0);
    const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 1);
    const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 2);
    const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 3);
    return v8h{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// One fp8 x fp4 MFMA over a 128-K group: A fp8 codes (scale 2^0), B the
// lane's 32 e2m1 codes (low nibble first) times 2^(e - 127) for the lane's
// UE8M0 byte e.  On gfx950 lane quarter q of B holds K [32q, 32q + 32), so a
// per-32-K weight scale is exactly one lane's scale operand; A lane quarter q
// holds K [16q, 16q + 16) and [64 + 16q, 64 + 16q + 16), i.e. an A row in
// its natural K order loaded as the two 16-byte chunks q and 4 + q.
__device__ __forceinline__ v4f mfma16x16x128_fp4(const v8i& a, const v4i& b, int e)
{
    const v8i bb = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 4, 0,
                                                             127, 0, e);
}

// fp4 weight scales of one row and 128-K group: the dword holds the four
// UE8M0 bytes of its 32-K blocks (block b in byte b).  For the exact f16 path
// the lane converts its block (quarter q) with 2^(e_q - e_max), whose values
// stay <= 6, and the group is promoted with 2^(e_max - 127 - 9) (the 2^-9
// matches the activation side data, whose c1 is 512 * scale).
struct Fp4GroupScale {
    float conv;     // 2^(e_q - e_max)
    float promote;  // 2^(e_max - 136)
};
__device__ __forceinline__ Fp4GroupScale fp4_group_scale(uint32_t sd, int q)
{
    const int e0 = (int)(sd & 0xFFu), e1 = (int)((sd >> 8) & 0xFFu);
    const int e2 = (int)((sd >> 16) & 0xFFu), e3 = (int)(sd >> 24);
    const int emax = max(max(e0, e1), max(e2, e3));
    const int eq = (int)((sd >> (8 * q)) & 0xFFu);
    return Fp4GroupScale{__builtin_amdgcn_ldexpf(1.0f, eq - emax), __builtin_amdgcn_ldexpf(1.0f, emax - 136)};
}

// canonical 8 codes (two dwords k0..k3, k4..k7) -> interleaved (k0,k2,k4,k6 | k1,k3,k5,k7)
__device__ __forceinline__ void interleave8(uint32_t d0, uint32_t d1, uint32_t& lo, uint32_t& hi)
{
    lo = __builtin_amdgcn_perm(d1, d0, 0x06040200u);
    hi = __builtin_amdgcn_perm(d1, d0, 0x07050301u);
}

// e4m3 code of clamp(v, -448, 448), round to nearest even; two values at once
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b)
{
    a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
    b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// exact decode of two e4m3 codes in the low half-word
__device__ __forceinline__ float2 dec_e4m3x2(uint32_t codes16)
{
    auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes16, false);
    return make_float2(f[0], f[1]);
}

// 448 / amax_c rounded once to fp32: the fp64 quotient rounded to fp32 equals
// the correctly rounded fp32 quotient (53 >= 2*24 + 2, so double rounding is
// innocuous for division).
__device__ __forceinline__ float recip448(float amax_c)
{
    return (float)(448.0 / (double)amax_c);
}
// 1/s of a static activation scale, rounded once to fp32 (the fp64 quotient
// of two floats rounds to the correctly rounded fp32 quotient)
__device__ __forceinline__ float recip_static(float s)
{
    return (float)(1.0 / (double)s);
}
__device__ __forceinline__ float scale_of(float amax_c)
{
    return (float)((double)amax_c / 448.0);
}
__device__ __forceinline__ float clamp_amax(float amax)
{
    return amax > 1e-10f ? amax : 1e-10f;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}
// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// butterfly reductions over aligned lane groups of width W (power of two <= 64)
template <int W>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

// Raw buffer resource over [base, base + bytes) (bytes < 2^32): loads take a
// 32-bit per-lane offset plus a wave-uniform (scalar) offset, so a streaming
// loop keeps its per-group advance in an SGPR instead of 64-bit VGPR pointers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ v4i bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}
// The same load with the non-temporal cache policy (nt): for streams read
// once, so that they do not push the data that is reused out of the caches.
__device__ __forceinline__ v4i bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2);
}
__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ v4i ldg16(const void* p)
{
    return *(const v4i*)p;
}
__device__ __forceinline__ v4i ldg16_nt(const void* p)
{
    return __builtin_nontemporal_load((const v4i*)p);
}

} // namespace w4a8
