// gemm.hip -- prefill-shape fused dequant-GEMM on the matrix cores,
// y[M, N] = x[M, K] . What^T for any M.
//
// Method ("Loading a model in 4-bit", "Where the accuracy goes"; "INT4
// Quantization > Practical Implementation with bitsandbytes"): the weights
// are dequantized to the 16-bit compute dtype and multiplied in a standard
// 16-bit matmul.  Here the dequantized tile never leaves the chip: each
// K-step stages a tile of x and the packed codes of a tile of W, dequantizes
// W into bf16/fp16 in LDS (each value exactly the one q4_dequantize would
// write), and feeds both to v_mfma_f32_16x16x32_{bf16,f16} with fp32
// accumulators; y is rounded once to the activation dtype.
#include "q4_common.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kBlock = 256;       // 4 waves, 2 x 2, each 64 x 64 of y
constexpr int LDS_STRIDE = BK + 8;  // halfs per LDS row (16-byte pad)

__constant__ float c_nf4_gemm[16] = {kNF4[0],  kNF4[1],  kNF4[2],  kNF4[3],  kNF4[4],  kNF4[5],
                                     kNF4[6],  kNF4[7],  kNF4[8],  kNF4[9],  kNF4[10], kNF4[11],
                                     kNF4[12], kNF4[13], kNF4[14], kNF4[15]};

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

// Dequantize 32 consecutive weights of one row (one group) to 16-bit pairs.
template <int FMT, int ACT>
__device__ __forceinline__ void dequant32(const u32x4 &cw, float s, float zf, const float *tbl,
                                          uint32_t out[16])
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = cw[j];
        float v[8];
        if constexpr (FMT == Q4_NF4) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = keep_f32(tbl[(w >> (4 * i)) & 0xf] * s);
        } else {
            const uint32_t lo = w & 0x0f0f0f0fu;
            const uint32_t hi = (w >> 4) & 0x0f0f0f0fu;
            const float bias = -zf * s;  // exact: z and s are short
            v[0] = __builtin_fmaf(ubyte_f32<0>(lo), s, bias);
            v[1] = __builtin_fmaf(ubyte_f32<0>(hi), s, bias);
            v[2] = __builtin_fmaf(ubyte_f32<1>(lo), s, bias);
            v[3] = __builtin_fmaf(ubyte_f32<1>(hi), s, bias);
            v[4] = __builtin_fmaf(ubyte_f32<2>(lo), s, bias);
            v[5] = __builtin_fmaf(ubyte_f32<2>(hi), s, bias);
            v[6] = __builtin_fmaf(ubyte_f32<3>(lo), s, bias);
            v[7] = __builtin_fmaf(ubyte_f32<3>(hi), s, bias);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[4 * j + i] = pack2<ACT>(v[2 * i], v[2 * i + 1]);
    }
}

template <int FMT, int ACT>
__global__ __launch_bounds__(kBlock) void gemm_kernel(const uint16_t *__restrict__ x, int M,
                                                      const uint8_t *__restrict__ codes,
                                                      const void *__restrict__ scales,
                                                      const uint8_t *__restrict__ zeros, int N,
                                                      int K, int gshift, uint16_t *__restrict__ y)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];
    __shared__ float tbl[16];
    if (threadIdx.x < 16)
        tbl[threadIdx.x] = c_nf4_gemm[threadIdx.x];
    __syncthreads();

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int64_t G = (int64_t)(K >> gshift);

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int k0 = 0; k0 < K; k0 += BK) {
        // ---- stage x: 128 rows x 64 halfs = 1024 chunks of 16 B, 4 per thread
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = t + kBlock * i;
            const int r = idx >> 3, cc = idx & 7;
            const int gm = m0 + r, gk = k0 + 8 * cc;
            u32x4 v = {0, 0, 0, 0};
            if (gm < M && gk < K)
                v = *(const u32x4 *)(x + (int64_t)gm * K + gk);
            *(u32x4 *)(As + r * LDS_STRIDE + 8 * cc) = v;
        }
        // ---- stage W: 128 rows x 64 weights; thread -> (row, 32-weight half)
        {
            const int r = t >> 1, hlf = t & 1;
            const int gn = n0 + r, gk = k0 + 32 * hlf;
            uint32_t out[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                out[i] = 0;
            if (gn < N && gk < K) {
                const u32x4 cw = *(const u32x4 *)(codes + (int64_t)gn * (K >> 1) + (gk >> 1));
                const int64_t gi = (int64_t)gn * G + (gk >> gshift);
                float s, zf = 0.0f;
                if constexpr (FMT == Q4_NF4)
                    s = ((const float *)scales)[gi];
                else
                    s = h2f(((const uint16_t *)scales)[gi]);
                if constexpr (FMT == Q4_INT4_SYM)
                    zf = 8.0f;
                if constexpr (FMT == Q4_INT4_ASYM)
                    zf = (float)((zeros[gi >> 1] >> ((gi & 1) * 4)) & 0xf);
                dequant32<FMT, ACT>(cw, s, zf, tbl, out);
            }
            u32x4 *dst = (u32x4 *)(Bs + r * LDS_STRIDE + 32 * hlf);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[i] = u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
        }
        __syncthreads();
        // ---- MFMA over the two 32-deep slices of the tile
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            u32x4 af[4], bf[4];
            const int koff = kk + 8 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *(const u32x4 *)(As + (wm * 64 + 16 * i + (lane & 15)) * LDS_STRIDE + koff);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *(const u32x4 *)(Bs + (wn * 64 + 16 * j + (lane & 15)) * LDS_STRIDE + koff);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = mfma<ACT>(af[i], bf[j], acc[i][j]);
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds column (lane & 15), rows 4 * (lane >> 4) + v
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + 16 * j + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + v;
                if (row < M && col < N)
                    y[(int64_t)row * N + col] =
                        (uint16_t)(ACT == Q4_BF16 ? f2bf_bits(acc[i][j][v]) : f2h_bits(acc[i][j][v]));
            }
        }
}

template <int FMT>
hipError_t launch_fmt(q4_dtype act_t, const void *x, int64_t M, const uint8_t *codes,
                      const void *scales, const uint8_t *zeros, int64_t N, int64_t K, int gshift,
                      void *y, hipStream_t s)
{
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM)), block(kBlock);
    if (act_t == Q4_BF16)
        hipLaunchKernelGGL((gemm_kernel<FMT, Q4_BF16>), grid, block, 0, s, (const uint16_t *)x,
                           (int)M, codes, scales, zeros, (int)N, (int)K, gshift, (uint16_t *)y);
    else
        hipLaunchKernelGGL((gemm_kernel<FMT, Q4_F16>), grid, block, 0, s, (const uint16_t *)x,
                           (int)M, codes, scales, zeros, (int)N, (int)K, gshift, (uint16_t *)y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                       const uint8_t *codes, const void *scales, const uint8_t *zeros, int64_t N,
                       int64_t K, void *y, hipStream_t s)
{
    const int gshift = g == 32 ? 5 : (g == 64 ? 6 : 7);
    switch (f) {
    case Q4_NF4:
        return launch_fmt<Q4_NF4>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
    case Q4_INT4_SYM:
        return launch_fmt<Q4_INT4_SYM>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
    default:
        return launch_fmt<Q4_INT4_ASYM>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
    }
}

}  // namespace q4
