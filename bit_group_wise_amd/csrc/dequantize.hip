// dequantize.hip -- packed 4-bit codes + metadata -> fp16 / bf16 weights.
//
// Method ("What is 4-bit quantization and why does it matter?", "How 4-bit
// quantization works": unpack the low nibble then the high nibble of each
// byte and multiply the level by the block scale; "Loading a model in 4-bit",
// "Block-wise quantisation, stated exactly": w = c * Q[i]): one binary32
// product per weight, rounded once (nearest-even) to the output dtype.  With
// double-quantized absmax the block's c is first recovered as qc * s2 (one
// binary32 product).
//
// gfx950 mapping: a flat stream.  Each lane decodes one dword of codes (8
// weights, all in one group since groups are >= 32 weights and aligned) and
// writes one 16-byte vector, so loads and stores are fully coalesced.  INT4
// levels are converted with v_cvt_f32_ubyte from a nibble-per-byte spread of
// the dword and scaled by one exact fma ((q - z) * s is exact in binary32);
// NF4 levels come from a 16-entry LDS table (one dword per entry in distinct
// banks, so lookups never conflict).  The stores are non-temporal: with them
// the cold 14336 x 4096 INT4-asym dequantization went from 4.1 to 6.1 TB/s.
#include "q4_common.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 4;

__constant__ float c_nf4[16] = {kNF4[0],  kNF4[1],  kNF4[2],  kNF4[3],  kNF4[4],  kNF4[5],
                                kNF4[6],  kNF4[7],  kNF4[8],  kNF4[9],  kNF4[10], kNF4[11],
                                kNF4[12], kNF4[13], kNF4[14], kNF4[15]};
__constant__ float c_fp4[16] = {kFP4[0],  kFP4[1],  kFP4[2],  kFP4[3],  kFP4[4],  kFP4[5],
                                kFP4[6],  kFP4[7],  kFP4[8],  kFP4[9],  kFP4[10], kFP4[11],
                                kFP4[12], kFP4[13], kFP4[14], kFP4[15]};

template <int OUT>
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    if constexpr (OUT == Q4_F16)
        return pack_h2(a, b);
    else
        return pack_bf2(a, b);
}

template <int FMT, int OUT>
__global__ __launch_bounds__(kBlock) void dequantize_kernel(const uint32_t *__restrict__ codes,
                                                            const void *__restrict__ scales,
                                                            const uint8_t *__restrict__ zeros,
                                                            const float *__restrict__ s2,
                                                            u32x4 *__restrict__ out,
                                                            int64_t n_units, int gshift)
{
    constexpr int LF = level_fmt(FMT);
    __shared__ float tbl[16];
    if constexpr (LF == Q4_NF4) {
        if (threadIdx.x < 16)
            tbl[threadIdx.x] = FMT == Q4_FP4 ? c_fp4[threadIdx.x] : c_nf4[threadIdx.x];
        __syncthreads();
    }
    const int lane = threadIdx.x & 63;
    const int64_t waves_per_block = kBlock / 64;
    const int64_t wave = (int64_t)blockIdx.x * waves_per_block + (threadIdx.x >> 6);
    const int64_t n_waves = (int64_t)gridDim.x * waves_per_block;

    for (int64_t t0 = wave * kUnroll; t0 * 64 < n_units; t0 += n_waves * kUnroll) {
        uint32_t cw[kUnroll];
        float sc[kUnroll];
        int zp[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t unit = (t0 + u) * 64 + lane;
            const int64_t gi = (unit * 8) >> gshift;  // flat group index
            cw[u] = 0;
            sc[u] = 0.0f;
            zp[u] = 0;
            if (unit < n_units) {
                cw[u] = codes[unit];
                if constexpr (f32_absmax(FMT))
                    sc[u] = ((const float *)scales)[gi];
                else if constexpr (FMT == Q4_NF4_DQ)  // c' = qc * s2, one product
                    sc[u] = keep_f32((float)((const uint8_t *)scales)[gi] * s2[gi / kDqRun]);
                else
                    sc[u] = h2f(((const uint16_t *)scales)[gi]);
                if constexpr (FMT == Q4_INT4_ASYM)
                    zp[u] = (zeros[gi >> 1] >> ((gi & 1) * 4)) & 0xf;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t unit = (t0 + u) * 64 + lane;
            float v[8];
            if constexpr (LF == Q4_NF4) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    v[i] = keep_f32(tbl[(cw[u] >> (4 * i)) & 0xf] * sc[u]);
            } else {
                // spread nibbles into bytes: lo holds elements 0,2,4,6 and hi
                // holds elements 1,3,5,7
                const uint32_t lo = cw[u] & 0x0f0f0f0fu;
                const uint32_t hi = (cw[u] >> 4) & 0x0f0f0f0fu;
                const float bias = -(float)(FMT == Q4_INT4_SYM ? 8 : zp[u]) * sc[u];  // exact
                const float s = sc[u];
                v[0] = __builtin_fmaf(ubyte_f32<0>(lo), s, bias);
                v[1] = __builtin_fmaf(ubyte_f32<0>(hi), s, bias);
                v[2] = __builtin_fmaf(ubyte_f32<1>(lo), s, bias);
                v[3] = __builtin_fmaf(ubyte_f32<1>(hi), s, bias);
                v[4] = __builtin_fmaf(ubyte_f32<2>(lo), s, bias);
                v[5] = __builtin_fmaf(ubyte_f32<2>(hi), s, bias);
                v[6] = __builtin_fmaf(ubyte_f32<3>(lo), s, bias);
                v[7] = __builtin_fmaf(ubyte_f32<3>(hi), s, bias);
            }
            if (unit < n_units) {
                u32x4 o = {pack2<OUT>(v[0], v[1]), pack2<OUT>(v[2], v[3]), pack2<OUT>(v[4], v[5]),
                           pack2<OUT>(v[6], v[7])};
                // streamed out (non-temporal: every output byte is written
                // once and not read back here)
                __builtin_nontemporal_store(o, &out[unit]);
            }
        }
    }
}

template <int FMT>
hipError_t launch_fmt(int gshift, const uint8_t *codes, const void *scales, const uint8_t *zeros,
                      int64_t N, int64_t K, q4_dtype out_t, void *out, hipStream_t s)
{
    const int64_t n_units = N * K / 8;
    const int64_t per_block = (int64_t)kBlock * kUnroll;
    int64_t blocks = (n_units + per_block - 1) / per_block;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (blocks > cap)
        blocks = cap;
    dim3 grid((unsigned)blocks), block(kBlock);
    const float *s2 = nullptr;
    if constexpr (FMT == Q4_NF4_DQ)
        s2 = (const float *)((const uint8_t *)scales + dq_s2_offset((N * K) >> gshift));
    if (out_t == Q4_F16)
        hipLaunchKernelGGL((dequantize_kernel<FMT, Q4_F16>), grid, block, 0, s,
                           (const uint32_t *)codes, scales, zeros, s2, (u32x4 *)out, n_units,
                           gshift);
    else
        hipLaunchKernelGGL((dequantize_kernel<FMT, Q4_BF16>), grid, block, 0, s,
                           (const uint32_t *)codes, scales, zeros, s2, (u32x4 *)out, n_units,
                           gshift);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(q4_format f, int g, const uint8_t *codes, const void *scales,
                             const uint8_t *zeros, int64_t N, int64_t K, q4_dtype out_t,
                             void *out, hipStream_t s)
{
    const int gshift = g == 32 ? 5 : (g == 64 ? 6 : 7);
    switch (f) {
    case Q4_NF4:
        return launch_fmt<Q4_NF4>(gshift, codes, scales, zeros, N, K, out_t, out, s);
    case Q4_FP4:
        return launch_fmt<Q4_FP4>(gshift, codes, scales, zeros, N, K, out_t, out, s);
    case Q4_NF4_DQ:
        return launch_fmt<Q4_NF4_DQ>(gshift, codes, scales, zeros, N, K, out_t, out, s);
    case Q4_INT4_SYM:
        return launch_fmt<Q4_INT4_SYM>(gshift, codes, scales, zeros, N, K, out_t, out, s);
    default:
        return launch_fmt<Q4_INT4_ASYM>(gshift, codes, scales, zeros, N, K, out_t, out, s);
    }
}

}  // namespace q4
