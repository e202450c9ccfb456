// q4_mfma.hpp -- weight dequantization into 16-bit MFMA operands and the
// 16x16x32 matrix-core product, shared by the prefill GEMM and the skinny
// (M <= 16) product.  Every weight value is the one q4_dequantize writes:
// the activation dtype's nearest-even rounding of the binary32 product
// level * scale ("Loading a model in 4-bit", "Where the accuracy goes").
#pragma once

#include "q4_common.hpp"

namespace q4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int ACT>
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    if constexpr (ACT == Q4_F16)
        return pack_h2(a, b);
    else
        return pack_bf2(a, b);
}

template <int ACT>
__device__ __forceinline__ f32x4 mfma(const u32x4 &a, const u32x4 &b, f32x4 c)
{
    if constexpr (ACT == Q4_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(std::bit_cast<bf16x8>(a),
                                                       std::bit_cast<bf16x8>(b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(std::bit_cast<f16x8>(a),
                                                      std::bit_cast<f16x8>(b), c, 0, 0, 0);
}

// The 8 weights of one code dword as binary32 values (element i of the
// dword in v[i]), each the product q4_dequantize rounds.  For NF4 (also with
// double-quantized absmax, s then being the recovered absmax) the level
// pairs lp (one per code byte) come from the LDS table.
template <int FMT>
__device__ __forceinline__ void dequant8_f32(uint32_t w, float s, float bias, const float2 (&lp)[4],
                                             float (&v)[8])
{
    if constexpr (level_fmt(FMT) == Q4_NF4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = keep_f32(lp[i].x * s);
            v[2 * i + 1] = keep_f32(lp[i].y * s);
        }
    } else {
        // (q - z) s as one exact fma per weight on an fp16 operand.  OR-ing
        // a nibble into 0x6400 makes the fp16 1024 + q (low nibble of a
        // byte) or 1024 + 16 q (high nibble), and
        //   fma(1024 + q, s, -(1024 + z) s),  fma(1024 + 16 q, s / 16, -(64 + z) s)
        // have exact terms ((q - z) s needs at most 15 significant bits, the
        // biases at most 22), so each returns the binary32 product itself.
        // v_fma_mix_f32 reads the fp16 from either half of a word: 5
        // instructions unpack 8 weights (with the masks in registers, so
        // that mask and OR fuse into one v_and_or_b32).
        const uint32_t m1 = opaque_word(0x000f000fu), m2 = opaque_word(0x00f000f0u);
        const uint32_t one = opaque_sword(0x64006400u);
        const uint32_t w8 = w >> 8;
        const f16x2 d0 = std::bit_cast<f16x2>((w & m1) | one);   // q0, q4
        const f16x2 d1 = std::bit_cast<f16x2>((w & m2) | one);   // 16 q1, 16 q5
        const f16x2 d2 = std::bit_cast<f16x2>((w8 & m1) | one);  // q2, q6
        const f16x2 d3 = std::bit_cast<f16x2>((w8 & m2) | one);  // 16 q3, 16 q7
        const float b1 = __builtin_fmaf(-1024.0f, s, bias);
        const float s16 = s * 0.0625f;
        const float b16 = __builtin_fmaf(-64.0f, s, bias);
        v[0] = __builtin_fmaf((float)d0[0], s, b1);
        v[1] = __builtin_fmaf((float)d1[0], s16, b16);
        v[2] = __builtin_fmaf((float)d2[0], s, b1);
        v[3] = __builtin_fmaf((float)d3[0], s16, b16);
        v[4] = __builtin_fmaf((float)d0[1], s, b1);
        v[5] = __builtin_fmaf((float)d1[1], s16, b16);
        v[6] = __builtin_fmaf((float)d2[1], s, b1);
        v[7] = __builtin_fmaf((float)d3[1], s16, b16);
    }
}

// The same 8 weights rounded to the activation dtype, as four 16-bit pairs.
template <int FMT, int ACT>
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float s, float bias, const float2 (&lp)[4])
{
    float v[8];
    dequant8_f32<FMT>(w, s, bias, lp, v);
    return u32x4{pack2<ACT>(v[0], v[1]), pack2<ACT>(v[2], v[3]), pack2<ACT>(v[4], v[5]),
                 pack2<ACT>(v[6], v[7])};
}

}  // namespace q4
