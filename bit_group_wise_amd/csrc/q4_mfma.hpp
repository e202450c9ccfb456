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
        const uint32_t lo = opaque_word(w & 0x0f0f0f0fu);
        const uint32_t hi = opaque_word((w >> 4) & 0x0f0f0f0fu);
        v[0] = __builtin_fmaf(ubyte_f32<0>(lo), s, bias);
        v[1] = __builtin_fmaf(ubyte_f32<0>(hi), s, bias);
        v[2] = __builtin_fmaf(ubyte_f32<1>(lo), s, bias);
        v[3] = __builtin_fmaf(ubyte_f32<1>(hi), s, bias);
        v[4] = __builtin_fmaf(ubyte_f32<2>(lo), s, bias);
        v[5] = __builtin_fmaf(ubyte_f32<2>(hi), s, bias);
        v[6] = __builtin_fmaf(ubyte_f32<3>(lo), s, bias);
        v[7] = __builtin_fmaf(ubyte_f32<3>(hi), s, bias);
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
