// gemv.hip -- decode-shape fused dequant-GEMV, y[M, N] = x[M, K] . What^T,
// 1 <= M <= 16, with no matrix-core instructions.
//
// Method ("Loading a model in 4-bit", "Where the accuracy goes"; "INT4
// Quantization > Practical Implementation with bitsandbytes"): the layer
// multiplies 16-bit activations by the dequantized weights; "What is 4-bit
// quantization and why does it matter?", "Why it matters for deployment":
// a decode step reads every weight once, so the kernel is bound by the bytes
// of packed codes and scales it streams.
//
// gfx950 mapping:
//  * Each wave owns R rows; lane l streams 16-byte chunks c = l, l+64, ...
//    (32 weights of each row, one dwordx4 load per row) and the matching
//    activations (4 dwordx4 per row of x, shared by the R rows).
//  * The scale is hoisted out of the inner product: a chunk lies inside one
//    group, so p = sum x * level is formed first and then acc += s * p
//    (INT4-asym: acc += s * (p - z * sum x)).
//  * Levels come from a per-workgroup LDS table indexed by a whole code byte:
//    the entry holds the two nibbles' levels as a packed 16-bit pair, so one
//    v_dot2_f32_{bf16,f16} multiplies two weights by two activations with an
//    fp32 accumulator.  NF4 levels are split into hi + lo 16-bit parts (two
//    dot2 per byte, about 17 significant bits); INT4 levels are exact.
//  * The table is replicated for 32 lane slots at a 256-byte entry stride, so
//    every lane reads its own bank (no conflicts), and the LDS address of a
//    byte is formed by one v_perm_b32 (code byte -> address bits 8..15, lane
//    slot -> bits 0..7).
//  * Lane partial sums are reduced across the wave with shuffles; y is
//    rounded once to the activation dtype.
#include "q4_common.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

constexpr int kWaves = 8;
constexpr int kBlock = kWaves * 64;
constexpr int kTableDwords = 256 * 64;  // 256 entries x 256 bytes

__constant__ uint32_t c_parts[4][16] = {
#define ROW(a) {a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8], a[9], a[10], a[11], a[12], a[13], a[14], a[15]}
    ROW(kPairParts.nf4_bf16_hi), ROW(kPairParts.nf4_bf16_lo), ROW(kPairParts.nf4_f16_hi),
    ROW(kPairParts.nf4_f16_lo),
#undef ROW
};

template <int ACT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    if constexpr (ACT == Q4_BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(std::bit_cast<bf16x2>(a), std::bit_cast<bf16x2>(b), c,
                                               false);
    else
        return __builtin_amdgcn_fdot2(std::bit_cast<f16x2>(a), std::bit_cast<f16x2>(b), c, false);
}

template <int ACT>
__device__ __forceinline__ uint32_t level_bits(int v)
{
    return ACT == Q4_BF16 ? f2bf_bits((float)v) : f2h_bits((float)v);
}

// Fill the byte-indexed pair table: entry e, half h (0 = hi, 1 = lo), lane
// slot L at byte offset e*256 + h*128 + 4L.
template <int FMT, int ACT>
__device__ __forceinline__ void fill_table(uint32_t *tbl)
{
    const int e = threadIdx.x >> 1;
    const int h = threadIdx.x & 1;
    const int n0 = e & 15, n1 = e >> 4;
    uint32_t v;
    if constexpr (FMT == Q4_NF4) {
        const int part = (ACT == Q4_BF16 ? 0 : 2) + h;
        v = c_parts[part][n0] | (c_parts[part][n1] << 16);
    } else {
        const int off = FMT == Q4_INT4_SYM ? 8 : 0;
        v = h ? 0u : (level_bits<ACT>(n0 - off) | (level_bits<ACT>(n1 - off) << 16));
    }
    u32x4 *dst = (u32x4 *)(tbl + e * 64 + h * 32);
    const u32x4 vv = {v, v, v, v};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        dst[j] = vv;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        v += __shfl_xor(v, d);
    return v;
}

template <int FMT, int ACT, int MT, int R>
__global__ __launch_bounds__(kBlock) void gemv_kernel(const uint16_t *__restrict__ x, int M,
                                                      const uint8_t *__restrict__ codes,
                                                      const void *__restrict__ scales,
                                                      const uint8_t *__restrict__ zeros, int N,
                                                      int K, int gshift, uint16_t *__restrict__ y)
{
    __shared__ uint32_t tbl[kTableDwords];
    fill_table<FMT, ACT>(tbl);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const uint32_t laneoff = (uint32_t)(lane & 31) << 2;
    const int C = K >> 5;                 // 32-weight chunks per row
    const int64_t G = (int64_t)(K >> gshift);  // groups per row
    const int64_t row_bytes = K >> 1;
    const int n_items = (N + R - 1) / R;
    const int total_waves = gridDim.x * kWaves;
    constexpr uint32_t kSel[4] = {0x0c0c0400u, 0x0c0c0500u, 0x0c0c0600u, 0x0c0c0700u};
    const uint32_t ones = ACT == Q4_BF16 ? 0x3f803f80u : 0x3c003c00u;

    for (int item = blockIdx.x * kWaves + (threadIdx.x >> 6); item < n_items; item += total_waves) {
        const int n0 = item * R;
        float acc[R][MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc[r][m] = 0.0f;

        for (int c = lane; c < C; c += 64) {
            u32x4 cw[R];
            float sc[R];
            float zf[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = n0 + r;
                cw[r] = u32x4{0, 0, 0, 0};
                sc[r] = 0.0f;
                zf[r] = 0.0f;
                if (row < N) {
                    cw[r] = *(const u32x4 *)(codes + (int64_t)row * row_bytes + 16 * (int64_t)c);
                    const int64_t gi = (int64_t)row * G + ((32 * c) >> gshift);
                    if constexpr (FMT == Q4_NF4)
                        sc[r] = ((const float *)scales)[gi];
                    else
                        sc[r] = h2f(((const uint16_t *)scales)[gi]);
                    if constexpr (FMT == Q4_INT4_ASYM)
                        zf[r] = (float)((zeros[gi >> 1] >> ((gi & 1) * 4)) & 0xf);
                }
            }
            float p[R][MT];
            float sx[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                sx[m] = 0.0f;
#pragma unroll
                for (int r = 0; r < R; ++r)
                    p[r][m] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x4 xv[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    xv[m] = u32x4{0, 0, 0, 0};
                    if (m < M)
                        xv[m] = *(const u32x4 *)(x + (int64_t)m * K + 32 * (int64_t)c + 8 * j);
                }
                if constexpr (FMT == Q4_INT4_ASYM) {
#pragma unroll
                    for (int m = 0; m < MT; ++m)
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            sx[m] = dot2<ACT>(xv[m][k], ones, sx[m]);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t addr = __builtin_amdgcn_perm(cw[r][j], laneoff, kSel[k]);
                        const uint32_t hi = *(const uint32_t *)((const char *)tbl + addr);
                        uint32_t lo = 0;
                        if constexpr (FMT == Q4_NF4)
                            lo = *(const uint32_t *)((const char *)tbl + addr + 128);
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            p[r][m] = dot2<ACT>(xv[m][k], hi, p[r][m]);
                            if constexpr (FMT == Q4_NF4)
                                p[r][m] = dot2<ACT>(xv[m][k], lo, p[r][m]);
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float t = p[r][m];
                    if constexpr (FMT == Q4_INT4_ASYM)
                        t = __builtin_fmaf(-zf[r], sx[m], t);
                    acc[r][m] = __builtin_fmaf(t, sc[r], acc[r][m]);
                }
        }

        float out = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float t = wave_sum(acc[r][m]);
                if (lane == r * MT + m)
                    out = t;
            }
        if (lane < R * MT) {
            const int r = lane / MT, m = lane % MT;
            if (m < M && n0 + r < N)
                y[(int64_t)m * N + n0 + r] =
                    (uint16_t)(ACT == Q4_BF16 ? f2bf_bits(out) : f2h_bits(out));
        }
    }
}

template <int FMT, int ACT, int MT, int R>
hipError_t launch_one(const void *x, int M, const uint8_t *codes, const void *scales,
                      const uint8_t *zeros, int64_t N, int64_t K, int gshift, void *y,
                      hipStream_t s)
{
    const int64_t n_items = (N + R - 1) / R;
    int64_t blocks = (n_items + kWaves - 1) / kWaves;
    const int64_t cap = (int64_t)device_cu_count() * 2;  // 64 KB of LDS each: 2 per CU
    if (blocks > cap)
        blocks = cap;
    hipLaunchKernelGGL((gemv_kernel<FMT, ACT, MT, R>), dim3((unsigned)blocks), dim3(kBlock), 0, s,
                       (const uint16_t *)x, M, codes, scales, zeros, (int)N, (int)K, gshift,
                       (uint16_t *)y);
    return hipGetLastError();
}

template <int FMT, int ACT>
hipError_t launch_m(const void *x, int M, const uint8_t *codes, const void *scales,
                    const uint8_t *zeros, int64_t N, int64_t K, int gshift, void *y, hipStream_t s)
{
    if (M <= 1)
        return launch_one<FMT, ACT, 1, 2>(x, M, codes, scales, zeros, N, K, gshift, y, s);
    if (M <= 2)
        return launch_one<FMT, ACT, 2, 2>(x, M, codes, scales, zeros, N, K, gshift, y, s);
    if (M <= 4)
        return launch_one<FMT, ACT, 4, 2>(x, M, codes, scales, zeros, N, K, gshift, y, s);
    if (M <= 8)
        return launch_one<FMT, ACT, 8, 1>(x, M, codes, scales, zeros, N, K, gshift, y, s);
    return launch_one<FMT, ACT, 16, 1>(x, M, codes, scales, zeros, N, K, gshift, y, s);
}

template <int FMT>
hipError_t launch_act(q4_dtype act_t, const void *x, int M, const uint8_t *codes,
                      const void *scales, const uint8_t *zeros, int64_t N, int64_t K, int gshift,
                      void *y, hipStream_t s)
{
    if (act_t == Q4_BF16)
        return launch_m<FMT, Q4_BF16>(x, M, codes, scales, zeros, N, K, gshift, y, s);
    return launch_m<FMT, Q4_F16>(x, M, codes, scales, zeros, N, K, gshift, y, s);
}

}  // namespace

hipError_t launch_gemv(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                       const uint8_t *codes, const void *scales, const uint8_t *zeros, int64_t N,
                       int64_t K, void *y, hipStream_t s)
{
    const int gshift = g == 32 ? 5 : (g == 64 ? 6 : 7);
    switch (f) {
    case Q4_NF4:
        return launch_act<Q4_NF4>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    case Q4_INT4_SYM:
        return launch_act<Q4_INT4_SYM>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    default:
        return launch_act<Q4_INT4_ASYM>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    }
}

}  // namespace q4
