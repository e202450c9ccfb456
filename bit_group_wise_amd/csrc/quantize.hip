// quantize.hip -- fp16 weights -> packed 4-bit codes + per-group metadata.
//
// Method ("Loading a model in 4-bit", "Block-wise quantisation, stated
// exactly"; "What is 4-bit quantization and why does it matter?", "How 4-bit
// quantization works"; "INT4", "How it works" / "Components"): per group of g
// contiguous weights, reduce the absmax (NF4, INT4-sym) or the zero-anchored
// range (INT4-asym), form the stored scale, code each weight to the nearest
// level after an IEEE binary32 division by the stored scale, and pack two
// codes per byte, low nibble first.
//
// gfx950 mapping: the weight matrix is streamed as a flat array.  Each lane
// owns 8 consecutive fp16 (one 16-byte load) and writes their 8 nibbles as
// one dword, so a wave reads 1 KB and writes 256 B per step, fully
// coalesced; both marked non-temporal (each byte is touched once: 7-13 %
// faster on cold 4096 x 4096 .. 14336 x 4096 matrices).  A group spans g/8 adjacent lanes and is reduced with
// cross-lane shuffles.  The quotient w / s is formed from one correctly
// rounded reciprocal per group (rcp_rn) plus Markstein's correction
// (q0 = w*r; e = fma(-q0, s, w); q = fma(e, r, q0)), which equals the
// correctly rounded IEEE quotient for every pair of fp16 operands with s > 0
// (checked exhaustively on all such pairs); NF4 codes come from a 33-bucket table of
// exact decision thresholds held in LDS, FP4 codes from seven exact
// thresholds on the magnitude and the sign.
//
// NF4 with double-quantized absmax (the same page, "Where the accuracy
// goes", and its closing section on NF4: the block constants coded again in
// runs of 256 to 8 bits) runs one workgroup per run, see quantize_dq_kernel.
#include "q4_common.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

constexpr int kBlock = 256;  // 4 waves
constexpr int kUnroll = 4;   // 16-byte loads in flight per lane

__constant__ NF4Bucket c_buckets[33] = {
#define B(i) {kNF4Buckets.e[i].thr, kNF4Buckets.e[i].base}
    B(0),  B(1),  B(2),  B(3),  B(4),  B(5),  B(6),  B(7),  B(8),  B(9),  B(10),
    B(11), B(12), B(13), B(14), B(15), B(16), B(17), B(18), B(19), B(20), B(21),
    B(22), B(23), B(24), B(25), B(26), B(27), B(28), B(29), B(30), B(31), B(32),
#undef B
};

// Correctly rounded a / b given r = RN(1 / b) (Markstein).
__device__ __forceinline__ float div_mk(float a, float b, float r)
{
    float q0 = a * r;
    float e = __builtin_fmaf(-q0, b, a);
    return __builtin_fmaf(e, r, q0);
}

// The scale quotients a / 7 (INT4-sym, a the absmax) and (hi - lo) / 15
// (INT4-asym) with the constant reciprocals RN(1/7) and RN(1/15): three
// instructions instead of a general division.  Equal to the IEEE quotient
// for every operand these can meet (a any non-negative fp16 value; hi - lo
// rounded to binary32 for any non-negative fp16 hi and non-positive fp16 lo),
// checked exhaustively.
constexpr float kInv7 = 1.0f / 7.0f;
constexpr float kInv15 = 1.0f / 15.0f;

// RN(1 / s) for s > 0 an fp16 value (the stored scale, or the absmax): the
// hardware reciprocal (accurate to 1 ulp) and one Newton step,
// r = r0 + r0 * (1 - s * r0) with both steps fused.  The step leaves a
// relative error of order 2^-46, while 1 / s, whose divisor has at most 11
// significant bits, lies at least 2^-35 (relative) away from any rounding
// midpoint, so the result is the correctly rounded reciprocal; checked
// exhaustively for every positive fp16 s and every start within 2 ulps.
__device__ __forceinline__ float rcp_rn(float s)
{
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-r0, s, 1.0f);
    return __builtin_fmaf(e, r0, r0);
}

// INT4 codes q = clamp(rint(x) + z, 0, 15) for any finite x (here x = w / s).
// For |x| < 2^22, adding 1.5 * 2^23 rounds x to an integer exactly as rint
// does (to nearest, ties to even: the sum's unit is 1) and leaves it in the
// low bits of the sum's bit pattern, kRintBias + rint(x); a larger |x| puts
// the sum beyond the clamp below, on the side the clamp of rint(x) + z takes
// too (and |w / s| <= 23 for finite fp16 inputs anyway).  Clamping the sum to
// [1.5 * 2^23 - z, 1.5 * 2^23 + 15 - z] (v_med3; integers there are exact)
// leaves kRintBias - z + q in the bits, so the instructions per weight are
// one add, one clamp and the packing; the offset kRintBias - z comes off
// once per dword (pack8).
constexpr float kRint = 12582912.0f;         // 1.5 * 2^23
constexpr uint32_t kRintBias = 0x4B400000u;  // its bit pattern
__device__ __forceinline__ uint32_t code_bits(float x, float lo, float hi)
{
    return std::bit_cast<uint32_t>(__builtin_amdgcn_fmed3f(x + kRint, lo, hi));
}
// 8 codes as one dword, low nibble first, from code_bits values c = off + q:
// shifted and added (codes below 16 never carry into the next nibble), then
// the offsets' shifted sum, off * 0x11111111 mod 2^32, taken off.
__device__ __forceinline__ uint32_t pack8(const uint32_t (&c)[8], uint32_t off)
{
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        word += c[i] << (4 * i);
    return word - off * 0x11111111u;
}

template <int LPG>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int d = 1; d < LPG; d <<= 1)
        v = fmaxf(v, __shfl_xor(v, d));
    return v;
}
template <int LPG>
__device__ __forceinline__ float group_min(float v)
{
#pragma unroll
    for (int d = 1; d < LPG; d <<= 1)
        v = fminf(v, __shfl_xor(v, d));
    return v;
}

// NF4 codes of 8 weights of a group with absmax c > 0, as one dword (low
// nibble first).
__device__ __forceinline__ uint32_t nf4_word(const float (&v)[8], float c, const NF4Bucket *lut)
{
    const float r = rcp_rn(c);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = div_mk(v[i], c, r);
        // bucket floor((x + 1) * 16), the product formed as one fma (16 (x + 1)
        // rounds as x + 1 does, scaled exactly); |x| <= 1, so b <= 32; the min
        // only guards inputs that break the finite-input precondition
        const uint32_t b = min((uint32_t)__builtin_fmaf(x, 16.0f, 16.0f), 32u);
        const NF4Bucket e = lut[b];
        const uint32_t code = e.base + (x >= e.thr ? 1u : 0u);
        word |= code << (4 * i);
    }
    return word;
}

// FP4 codes of 8 weights of a group with absmax c > 0: the magnitude index
// j = number of thresholds at or below |x| (seven compares), then the sign
// (code j + 8 for x < 0 and j > 0; the tie of +0 and -0 keeps code 0).
__device__ __forceinline__ uint32_t fp4_word(const float (&v)[8], float c)
{
    const float r = rcp_rn(c);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = div_mk(v[i], c, r);
        const float a = fabsf(x);
        uint32_t j = 0;
#pragma unroll
        for (int t = 0; t < 7; ++t)
            j += a >= kFP4Thr[t] ? 1u : 0u;
        const uint32_t code = (x < 0.0f && j != 0) ? j + 8 : j;
        word |= code << (4 * i);
    }
    return word;
}

template <int FMT, int G>
__global__ __launch_bounds__(kBlock) void quantize_kernel(const u32x4 *__restrict__ w,
                                                          uint32_t *__restrict__ codes,
                                                          void *__restrict__ scales,
                                                          uint8_t *__restrict__ zeros,
                                                          int64_t n_slots, int64_t n_groups)
{
    constexpr int LPG = G / 8;  // lanes per group
    __shared__ NF4Bucket lut[33];
    if constexpr (FMT == Q4_NF4) {
        if (threadIdx.x < 33)
            lut[threadIdx.x] = c_buckets[threadIdx.x];
        __syncthreads();
    }
    const int lane = threadIdx.x & 63;
    const int64_t waves_per_block = kBlock / 64;
    const int64_t wave = (int64_t)blockIdx.x * waves_per_block + (threadIdx.x >> 6);
    const int64_t n_waves = (int64_t)gridDim.x * waves_per_block;

    for (int64_t t0 = wave * kUnroll; t0 * 64 < n_slots; t0 += n_waves * kUnroll) {
        u32x4 raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            int64_t slot = (t0 + u) * 64 + lane;
            raw[u] = slot < n_slots ? __builtin_nontemporal_load(&w[slot]) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t slot = (t0 + u) * 64 + lane;
            const bool in = slot < n_slots;
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = h2f(raw[u][i] & 0xffffu);
                v[2 * i + 1] = h2f(raw[u][i] >> 16);
            }
            uint32_t word = 0;
            const int64_t gi = slot / LPG;
            const bool leader = (lane % LPG) == 0;
            if constexpr (FMT == Q4_NF4 || FMT == Q4_FP4) {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    a = fmaxf(a, fabsf(v[i]));
                const float c = group_max<LPG>(a);
                if constexpr (FMT == Q4_NF4)
                    word = c != 0.0f ? nf4_word(v, c, lut) : 0x77777777u;
                else
                    word = c != 0.0f ? fp4_word(v, c) : 0u;
                if (in && leader)
                    ((float *)scales)[gi] = c;
            } else if constexpr (FMT == Q4_INT4_SYM) {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    a = fmaxf(a, fabsf(v[i]));
                a = group_max<LPG>(a);
                // (the quotient rounded to binary32 first, then to fp16: no
                // single-rounding mixed fma)
                const uint32_t s16 = f2h_bits(keep_f32(div_mk(a, 7.0f, kInv7)));
                const float s = h2f(s16);
                if (s != 0.0f) {
                    const float r = rcp_rn(s);
                    // q = clamp(rint(w / s), -8, 7) + 8: z = 8
                    uint32_t c[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        c[i] = code_bits(div_mk(v[i], s, r), kRint - 8.0f, kRint + 7.0f);
                    word = pack8(c, kRintBias - 8u);
                } else {
                    word = 0x88888888u;
                }
                if (in && leader)
                    ((uint16_t *)scales)[gi] = (uint16_t)s16;
            } else {
                float lo = 0.0f, hi = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    lo = fminf(lo, v[i]);
                    hi = fmaxf(hi, v[i]);
                }
                lo = group_min<LPG>(lo);
                hi = group_max<LPG>(hi);
                const uint32_t s16 = f2h_bits(keep_f32(div_mk(hi - lo, 15.0f, kInv15)));
                const float s = h2f(s16);
                int z = 0;
                if (s != 0.0f) {
                    const float r = rcp_rn(s);
                    z = (int)__builtin_rintf(div_mk(-lo, s, r));
                    z = z < 0 ? 0 : (z > 15 ? 15 : z);
                    const float lo_c = kRint - (float)z;
                    uint32_t c[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        c[i] = code_bits(div_mk(v[i], s, r), lo_c, lo_c + 15.0f);
                    word = pack8(c, kRintBias - (uint32_t)z);
                }
                // zero-points: the leader of an even group packs its own and
                // the next group's (LPG lanes further on; both groups lie in
                // the same 64-lane step because 512 / g is even)
                const int z_next = __shfl_down(z, LPG);
                if (in && leader) {
                    ((uint16_t *)scales)[gi] = (uint16_t)s16;
                    if ((gi & 1) == 0) {
                        const uint32_t hi_nib = (gi + 1 < n_groups) ? (uint32_t)z_next : 0u;
                        zeros[gi >> 1] = (uint8_t)((uint32_t)z | (hi_nib << 4));
                    }
                }
            }
            if (in)
                __builtin_nontemporal_store(word, &codes[slot]);
        }
    }
}

// NF4 with double-quantized absmax.  A workgroup owns one run of kDqRun
// groups (flat order): it codes the run's weights as NF4 with each group's
// exact absmax c, keeps the c values in LDS, then forms the run's binary32
// constant s2 = max c / 127 and the 8-bit codes rint(c / s2) clamped to
// 0..127 (one per thread).  The quotient c / s2 is the correctly rounded IEEE
// division (the compiler's default for '/').
template <int G>
__global__ __launch_bounds__(kBlock) void quantize_dq_kernel(const u32x4 *__restrict__ w,
                                                             uint32_t *__restrict__ codes,
                                                             uint8_t *__restrict__ qc,
                                                             float *__restrict__ s2,
                                                             int64_t n_groups, int64_t s2_off)
{
    static_assert(kBlock == kDqRun, "one thread per group of the run");
    constexpr int LPG = G / 8;
    __shared__ NF4Bucket lut[33];
    __shared__ float cs[kDqRun];
    __shared__ float wmax[kBlock / 64];
    if (threadIdx.x < 33)
        lut[threadIdx.x] = c_buckets[threadIdx.x];
    const int tid = threadIdx.x;
    cs[tid] = 0.0f;
    __syncthreads();

    const int64_t gb0 = (int64_t)blockIdx.x * kDqRun;  // the run's first group
    const int ng = n_groups - gb0 < kDqRun ? (int)(n_groups - gb0) : kDqRun;
    const int64_t slot0 = gb0 * LPG;
    const int nsl = ng * LPG;  // 16-byte slots of the run (a multiple of LPG)
    constexpr int kSteps = kDqRun * LPG / kBlock;  // full-run steps (4, 8, 16)
    static_assert(kSteps % kUnroll == 0, "whole unrolled rounds");
    for (int t0 = 0; t0 < kSteps; t0 += kUnroll) {
        u32x4 raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = (t0 + u) * kBlock + tid;
            raw[u] = i < nsl ? __builtin_nontemporal_load(&w[slot0 + i]) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = (t0 + u) * kBlock + tid;
            float v[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[2 * k] = h2f(raw[u][k] & 0xffffu);
                v[2 * k + 1] = h2f(raw[u][k] >> 16);
            }
            float a = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                a = fmaxf(a, fabsf(v[k]));
            const float c = group_max<LPG>(a);
            const uint32_t word = c != 0.0f ? nf4_word(v, c, lut) : 0x77777777u;
            if (i < nsl) {
                __builtin_nontemporal_store(word, &codes[slot0 + i]);
                if (i % LPG == 0)
                    cs[i / LPG] = c;
            }
        }
    }
    __syncthreads();

    // the run's max (absmax values are >= 0; unused slots hold 0)
    const float c = cs[tid];
    float m = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1)
        m = fmaxf(m, __shfl_xor(m, d));
    if ((tid & 63) == 0)
        wmax[tid >> 6] = m;
    __syncthreads();
    float c2 = wmax[0];
#pragma unroll
    for (int i = 1; i < kBlock / 64; ++i)
        c2 = fmaxf(c2, wmax[i]);
    const float sc2 = c2 / 127.0f;
    int q = 0;
    if (sc2 != 0.0f) {
        q = (int)__builtin_rintf(c / sc2);
        q = q < 0 ? 0 : (q > 127 ? 127 : q);
    }
    // codes of the run; a short last run also zero-fills the bytes up to s2
    // (s2_off <= gb0 + kDqRun: both are multiples of 16 and >= n_groups)
    if (gb0 + tid < s2_off)
        qc[gb0 + tid] = (uint8_t)(tid < ng ? q : 0);
    if (tid == 0)
        s2[blockIdx.x] = sc2;
}

template <int G>
hipError_t launch_dq(const void *w, int64_t N, int64_t K, uint8_t *codes, void *scales,
                     hipStream_t s)
{
    const int64_t n_groups = N * K / G;
    const int64_t runs = (n_groups + kDqRun - 1) / kDqRun;
    const int64_t off = dq_s2_offset(n_groups);
    uint8_t *qc = (uint8_t *)scales;
    hipLaunchKernelGGL((quantize_dq_kernel<G>), dim3((unsigned)runs), dim3(kBlock), 0, s,
                       (const u32x4 *)w, (uint32_t *)codes, qc, (float *)(qc + off), n_groups,
                       off);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(int g, const void *w, int64_t N, int64_t K, uint8_t *codes, void *scales,
                      uint8_t *zeros, hipStream_t s)
{
    const int64_t n_slots = N * K / 8;
    const int64_t n_groups = N * K / g;
    const int64_t per_block = (int64_t)kBlock * kUnroll;  // slots per block step
    int64_t blocks = (n_slots + per_block - 1) / per_block;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (blocks > cap)
        blocks = cap;
    dim3 grid((unsigned)blocks), block(kBlock);
    const u32x4 *wp = (const u32x4 *)w;
    uint32_t *cp = (uint32_t *)codes;
    switch (g) {
    case 32:
        hipLaunchKernelGGL((quantize_kernel<FMT, 32>), grid, block, 0, s, wp, cp, scales, zeros,
                           n_slots, n_groups);
        break;
    case 64:
        hipLaunchKernelGGL((quantize_kernel<FMT, 64>), grid, block, 0, s, wp, cp, scales, zeros,
                           n_slots, n_groups);
        break;
    default:
        hipLaunchKernelGGL((quantize_kernel<FMT, 128>), grid, block, 0, s, wp, cp, scales, zeros,
                           n_slots, n_groups);
        break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(q4_format f, int g, const void *w, int64_t N, int64_t K,
                           uint8_t *codes, void *scales, uint8_t *zeros, hipStream_t s)
{
    switch (f) {
    case Q4_NF4_DQ:
        return g == 32 ? launch_dq<32>(w, N, K, codes, scales, s)
                       : (g == 64 ? launch_dq<64>(w, N, K, codes, scales, s)
                                  : launch_dq<128>(w, N, K, codes, scales, s));
    case Q4_NF4:
        return launch_fmt<Q4_NF4>(g, w, N, K, codes, scales, zeros, s);
    case Q4_FP4:
        return launch_fmt<Q4_FP4>(g, w, N, K, codes, scales, zeros, s);
    case Q4_INT4_SYM:
        return launch_fmt<Q4_INT4_SYM>(g, w, N, K, codes, scales, zeros, s);
    default:
        return launch_fmt<Q4_INT4_ASYM>(g, w, N, K, codes, scales, zeros, s);
    }
}

}  // namespace q4
