// q4_common.hpp -- shared device-side definitions of libq4 (gfx950).
//
// The NF4 codebook and every table derived from it are computed here at
// compile time (constexpr), from the 16 decimals printed in "What is 4-bit
// quantization and why does it matter?", section "How 4-bit quantization
// works".  Nothing in this file is generated at run time.
#pragma once

#include <hip/hip_runtime.h>

#include <bit>
#include <cstdint>

#include "q4.h"

namespace q4 {

// --------------------------------------------------------------------------
// Vector types used by the kernels.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// --------------------------------------------------------------------------
// The codebook (each decimal read as the nearest binary32).
inline constexpr float kNF4[16] = {-1.0f,  -0.696f, -0.525f, -0.395f, -0.284f, -0.185f,
                                   -0.091f, 0.0f,   0.079f,  0.161f,  0.246f,  0.338f,
                                   0.441f,  0.562f, 0.720f,  1.0f};

// FP4 ("Loading a model in 4-bit", "Developer", names the fp4 quant type
// beside nf4 without printing its table; a reading): the E2M1 element values
// -- bit 3 the sign, bits 2..1 an exponent e, bit 0 a mantissa bit m; m / 2
// for e = 0, else 2^(e-1) (1 + m / 2) -- divided by 6 so that the largest
// magnitude is 1, each the nearest binary32 of the exact fraction, used as
// NF4's table is (scaled by the binary32 block absmax).  Code 8 is -0.
constexpr float e2m1_over_6(int c)
{
    const int e = (c >> 1) & 3, m = c & 1;
    const double mag = e == 0 ? 0.5 * m : (double)(1 << (e - 1)) * (1.0 + 0.5 * m);
    const float v = (float)(mag / 6.0);
    return (c & 8) ? -v : v;
}
inline constexpr float kFP4[16] = {
    e2m1_over_6(0),  e2m1_over_6(1),  e2m1_over_6(2),  e2m1_over_6(3),
    e2m1_over_6(4),  e2m1_over_6(5),  e2m1_over_6(6),  e2m1_over_6(7),
    e2m1_over_6(8),  e2m1_over_6(9),  e2m1_over_6(10), e2m1_over_6(11),
    e2m1_over_6(12), e2m1_over_6(13), e2m1_over_6(14), e2m1_over_6(15)};
static_assert(kFP4[7] == 1.0f && kFP4[15] == -1.0f && kFP4[5] == 0.5f, "E2M1 / 6");

// The level arithmetic of a format: NF4 with double-quantized absmax decodes
// as NF4 once each block's absmax has been recovered, and FP4 as NF4 with its
// own table (16 binary32 levels times the block absmax).
constexpr int level_fmt(int f) { return (f == Q4_NF4_DQ || f == Q4_FP4) ? Q4_NF4 : f; }
// Formats whose stored scale is the binary32 block absmax itself.
constexpr bool f32_absmax(int f) { return f == Q4_NF4 || f == Q4_FP4; }
// Level i of a table format's codebook.
template <int FMT>
constexpr float level_entry(int i) { return FMT == Q4_FP4 ? kFP4[i] : kNF4[i]; }

// Compile-time IEEE helpers (finite inputs only).
constexpr uint32_t f32_bits(float f) { return std::bit_cast<uint32_t>(f); }
constexpr float bits_f32(uint32_t u) { return std::bit_cast<float>(u); }

// Nearest-even bfloat16 of a finite float, as bits.
constexpr uint16_t bf16_rne_bits(float f)
{
    uint32_t u = f32_bits(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
constexpr float bf16_bits_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

// Nearest-even binary16 of a finite float of magnitude < 65504, as bits
// (gradual underflow: the quantum below 2^-14 is 2^-24).
constexpr uint16_t f16_rne_bits(float f)
{
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    float a = f < 0 ? -f : f;
    if (a == 0.0f)
        return sign;
    // scale so that the fp16 quantum becomes 1, then round half to even
    int e = (int)((f32_bits(a) >> 23) & 0xff) - 127;  // a is a normal float here
    if (e < -14)
        e = -14;
    double q = (double)a;
    for (int i = 0; i < 10 - e; ++i)
        q *= 2.0;
    for (int i = 0; i < e - 10; ++i)
        q *= 0.5;
    uint64_t n = (uint64_t)q;
    double rem = q - (double)n;
    if (rem > 0.5 || (rem == 0.5 && (n & 1)))
        ++n;
    // n * 2^(e-10): encode
    if (e == -14 && n < 1024)
        return (uint16_t)(sign | n);  // subnormal
    if (n >= 2048) {
        n >>= 1;
        ++e;
    }
    return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | (uint32_t)(n - 1024));
}
constexpr float f16_bits_f32(uint16_t h)
{
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v = ex == 0 ? (double)man : (double)(1024 + man);
    int sh = ex == 0 ? -24 : ex - 25;
    for (int i = 0; i < sh; ++i)
        v *= 2.0;
    for (int i = 0; i < -sh; ++i)
        v *= 0.5;
    return (float)((h & 0x8000) ? -v : v);
}

// --------------------------------------------------------------------------
// NF4 coding by thresholds.  The nearest entry to x with ties to the lower
// index is the number of thresholds t_i <= x, where t_i is the smallest
// binary32 strictly above the exact midpoint of Q[i] and Q[i+1] (the midpoint
// of two binary32 values is exact in binary64).
constexpr float next_up(float f)
{
    uint32_t u = f32_bits(f);
    if (f == 0.0f)
        return bits_f32(1u);
    return f > 0 ? bits_f32(u + 1) : bits_f32(u - 1);
}
constexpr float nf4_threshold(int i)
{
    double m = ((double)kNF4[i] + (double)kNF4[i + 1]) * 0.5;
    float f = (float)m;
    // RN(m) is either above m (then it is the smallest binary32 above m) or
    // at/below m (then its successor is)
    if ((double)f <= m)
        f = next_up(f);
    return f;
}

// FP4 coding by the magnitude: the nearest entry to x (ties to the lower
// index) is +-level j, with j the number of thresholds u_j <= |x| (u_j the
// smallest binary32 strictly above the exact midpoint of magnitudes j and
// j + 1, codes 0..7 ascending), and code j + 8 for x < 0 unless j = 0 (the
// tie between +0 and -0 keeps code 0).
constexpr float fp4_threshold(int j)
{
    double m = ((double)kFP4[j] + (double)kFP4[j + 1]) * 0.5;
    float f = (float)m;
    if ((double)f <= m)
        f = next_up(f);
    return f;
}
inline constexpr float kFP4Thr[7] = {fp4_threshold(0), fp4_threshold(1), fp4_threshold(2),
                                     fp4_threshold(3), fp4_threshold(4), fp4_threshold(5),
                                     fp4_threshold(6)};

// Bucket table: x in [-1, 1] falls into bucket b = floor((x + 1) * 16) (b in
// 0..32).  The bucket width 1/16 is below the smallest gap between
// thresholds, so a bucket holds at most one threshold, and the code is
// base_b + (x >= thr_b), where base_b counts the thresholds below the
// bucket and thr_b is the next threshold (+inf after the last one).
struct NF4Bucket {
    float thr;
    uint32_t base;
};
struct NF4BucketTable {
    NF4Bucket e[33];
    float min_edge_distance;  // distance of the nearest threshold to a bucket edge
};
constexpr NF4BucketTable make_bucket_table()
{
    NF4BucketTable t{};
    float thr[16] = {};
    for (int i = 0; i < 15; ++i)
        thr[i] = nf4_threshold(i);
    thr[15] = __builtin_inff();
    t.min_edge_distance = 1.0f;
    for (int i = 0; i < 15; ++i) {
        double pos = ((double)thr[i] + 1.0) * 16.0;
        double d = pos - (double)(int64_t)pos;
        if (d > 0.5)
            d = 1.0 - d;
        if ((float)d < t.min_edge_distance)
            t.min_edge_distance = (float)d;
    }
    for (int b = 0; b <= 32; ++b) {
        double lo = -1.0 + b / 16.0;
        uint32_t base = 0;
        while (base < 15 && (double)thr[base] < lo)
            ++base;
        t.e[b] = NF4Bucket{thr[base], base};
    }
    return t;
}
inline constexpr NF4BucketTable kNF4Buckets = make_bucket_table();
// The rounding of (x + 1) * 16 in binary32 moves a point by at most 2^-20
// bucket units; every threshold is far further than that from an edge.
static_assert(kNF4Buckets.min_edge_distance > 1.0f / 64, "threshold too close to a bucket edge");
static_assert(kNF4Buckets.e[32].base == 15, "x = 1 must code to 15");
static_assert(kNF4Buckets.e[0].base == 0, "x = -1 must code to 0");

// --------------------------------------------------------------------------
// Device helpers.
__device__ __forceinline__ float h2f(uint32_t bits16)
{
    return (float)std::bit_cast<_Float16>((uint16_t)bits16);
}
__device__ __forceinline__ float bf2f(uint32_t bits16) { return std::bit_cast<float>(bits16 << 16); }

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32, denormals kept).
__device__ __forceinline__ uint32_t f2h_bits(float f)
{
    return std::bit_cast<uint16_t>((_Float16)f);
}
// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f2bf_bits(float f)
{
    return std::bit_cast<uint16_t>((__bf16)f);
}
// Pins a binary32 value in a register.  Without it the compiler may fold
// fp16(a * b) into one mixed-precision fma (v_fma_mixlo_f16) that rounds
// the exact product once, instead of rounding to binary32 first and then to
// fp16 as the dequantize rule states.  Emits no instruction.
__device__ __forceinline__ float keep_f32(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Byte I of a dword as a float (v_cvt_f32_ubyte{0..3}).
template <int I>
__device__ __forceinline__ float ubyte_f32(uint32_t v) { return (float)((v >> (8 * I)) & 0xffu); }
// The word itself, opaque to the optimizer (an empty register-only asm).
// Keeps a word of byte-spread nibbles (w & 0x0f0f0f0f) whole: each byte then
// converts with one v_cvt_f32_ubyteN, where the optimizer would otherwise
// fold the mask into a 4-bit field extract (v_bfe) before every convert.
__device__ __forceinline__ uint32_t opaque_word(uint32_t v)
{
    asm("" : "+v"(v));
    return v;
}
// A wave-uniform constant kept in a scalar register (so that an instruction
// that also takes a constant in a vector register can read it).
__device__ __forceinline__ uint32_t opaque_sword(uint32_t v)
{
    asm("" : "+s"(v));
    return v;
}

// Two fp32 -> packed pair (a in the low half).
__device__ __forceinline__ uint32_t pack_h2(float a, float b) { return f2h_bits(a) | (f2h_bits(b) << 16); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b)
{
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return std::bit_cast<uint32_t>(v);
}

}  // namespace q4
